// check_rules.hpp -- the device-resident preconditions that check mode
// verifies, as one grid-stride pass: thread t of nt evaluates its share of
// the entries and returns the MIMO_CHECK_* bits it found violated.
//
// The rules restate the argument contracts of include/mimo_attn.h:
//   cu_seqlens / cu_newlens start at 0, never decrease, hold no sequence
//   longer than max_seqlen and end at the call's token count;
//   0 <= ctx_lens[b] <= max_ctx, and ctx + new positions fit 32 bits;
//   kv_base[b] >= 0; ctx + new <= kv_capacity[b] (GA pool) or
//   <= max_blocks * page_size (paged pool);
//   every block-table entry of a block the call reads or writes lies in
//   [0, num_pages);
//   a sink is finite or -inf; an FP8 scale is positive and finite.
#pragma once
#include <stdint.h>

#include "../../include/mimo_attn.h"
#include "launch.hpp"

namespace mimo {

__host__ __device__ inline bool sink_ok(float s) {
    // Bit tests: the library is built with NaN-unaware float compares.
    uint32_t u;
    __builtin_memcpy(&u, &s, 4);
    const uint32_t mag = u & 0x7fffffffu;
    return mag < 0x7f800000u || u == 0xff800000u;  // finite, or -inf
}

__host__ __device__ inline bool scale_ok(float s) {
    uint32_t u;
    __builtin_memcpy(&u, &s, 4);
    return u != 0 && u < 0x7f800000u;  // sign clear, not zero, finite
}

// Tokens sequence b adds in this call (0 when cu decreases there; that is
// reported by the cu rules).
__host__ __device__ inline long long new_tokens_of(const CheckArgs& a, int b) {
    if (!a.new_from_cu) return a.new_tokens;
    const long long n = (long long)a.cu[b + 1] - a.cu[b];
    return n > 0 ? n : 0;
}

__host__ __device__ inline uint32_t check_rules(const CheckArgs& a, long long t, long long nt) {
    uint32_t f = 0;
    if (a.cu) {
        if (t == 0) {
            if (a.cu[0] != 0) f |= MIMO_CHECK_CU_START;
            if (a.total >= 0 && a.cu[a.n_seqs] != a.total) f |= MIMO_CHECK_CU_TOTAL;
        }
        for (long long i = t; i < a.n_seqs; i += nt) {
            const long long len = (long long)a.cu[i + 1] - a.cu[i];
            if (len < 0) f |= MIMO_CHECK_CU_ORDER;
            else if (a.max_len >= 0 && len > a.max_len) f |= MIMO_CHECK_CU_LENGTH;
        }
    }
    if (a.ctx) {
        const long long pool = a.pages.table ? (long long)a.pages.max_blocks << a.pages.shift : -1;
        for (long long b = t; b < a.batch; b += nt) {
            const long long c = a.ctx[b];
            const long long n = new_tokens_of(a, (int)b);
            if (c < 0 || (a.max_ctx >= 0 && c > a.max_ctx) || c + n > INT32_MAX) f |= MIMO_CHECK_CTX_RANGE;
            if (a.kv_base && a.kv_base[b] < 0) f |= MIMO_CHECK_KV_BASE;
            if (a.kv_capacity && c + n > a.kv_capacity[b]) f |= MIMO_CHECK_CAPACITY;
            if (pool >= 0 && (a.pages_cover_new ? c + n : c) > pool) f |= MIMO_CHECK_CAPACITY;
        }
        if (a.pages.table) {
            const long long entries = (long long)a.batch * a.pages.max_blocks;
            for (long long e = t; e < entries; e += nt) {
                const int b = (int)(e / a.pages.max_blocks);
                const long long blk = e - (long long)b * a.pages.max_blocks;
                const long long c = a.ctx[b];
                if (c < 0) continue;
                const long long lo = a.pages_cover_new ? c : 0;
                const long long hi = a.pages_cover_new ? c + new_tokens_of(a, b) : c;  // positions [lo, hi)
                if (hi <= lo || blk < (lo >> a.pages.shift) || (blk << a.pages.shift) >= hi) continue;
                const int32_t page = a.pages.table[e];
                if (page < 0 || page >= a.pages.num_pages) f |= MIMO_CHECK_BLOCK_TABLE;
            }
        }
    }
    if (a.sink)
        for (long long h = t; h < a.hq; h += nt)
            if (!sink_ok(a.sink[h])) f |= MIMO_CHECK_SINK;
    if (a.scales)
        for (long long g = t; g < a.n_scales; g += nt)
            if (!scale_ok(a.scales[g]) || !scale_ok(a.scales_v[g])) f |= MIMO_CHECK_FP8_SCALE;
    return f;
}

}  // namespace mimo
