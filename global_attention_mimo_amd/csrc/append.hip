// append.hip -- writes new tokens' keys and values into the SWA ring or the GA pool.
//
// Operation (Hugging Face Transformers model doc "MiMo-V2-Flash",
// MiMoV2FlashModel.forward, past_key_values / use_cache): the cache keeps the
// keys and values of processed tokens so later steps pass only new tokens.
// SWA layers need only the last sliding_window-1 = 128 positions (the new
// token is the 129th key), so their cache is a ring of 128 slots per sequence,
// position j in slot j mod 128; GA layers keep every position in a pool row
// kv_base[b] + j, or, in a paged pool, in row j mod P of the page the block
// table gives for block j / P.
//
// One thread moves one 16-byte chunk: a token is Hkv*24 chunks of K and
// Hkv*16 chunks of V, so consecutive threads copy consecutive bytes of a row.
// An FP8 GA pool stores OCP E4M3 codes of the values divided by a per-KV-head
// scale instead (a storage format of the same cache).
#include "device_common.hpp"
#include "launch.hpp"

namespace mimo {
namespace {

constexpr int kDqk = 192;
constexpr int kDv = 128;

// Packed token, chunk (unit) within the token, and owning sequence of this
// thread, for a flat grid of per_tok threads per token (the FP8 append, whose
// per-element division makes per-thread index arithmetic costly).  The 64-bit division
// and the search for the sequence (the last b with cu_newlens[b] <= token) run
// once per wave on the wave's first token, in scalar registers; a thread's
// token lies at most a few tokens past it, reached by stepping over the
// sequences that end before it (empty ones included).
struct TokSeq {
    int64_t tok;
    int c;
    int b;
};
__device__ __forceinline__ TokSeq locate(const int32_t* __restrict__ cu_newlens, int batch, int per_tok) {
    const int w = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
    const int64_t base = (int64_t)blockIdx.x * blockDim.x + (int64_t)w * 64;
    const int64_t tok0 = base / per_tok;
    const int local = (int)(base - tok0 * per_tok) + (int)(threadIdx.x & 63);
    const int dt = local / per_tok;
    TokSeq r;
    r.tok = tok0 + dt;
    r.c = local - dt * per_tok;
    int lo = 0, hi = batch - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (cu_newlens[mid] <= tok0) lo = mid; else hi = mid - 1;
    }
    int b = lo;
    while (b + 1 < batch && cu_newlens[b + 1] <= r.tok) ++b;
    r.b = b;
    return r;
}

__global__ __launch_bounds__(256) void kv_append_kernel(
    const uint16_t* __restrict__ k, const uint16_t* __restrict__ v, const int32_t* __restrict__ cu_newlens,
    const int32_t* __restrict__ ctx_lens, int batch, int total_new, uint16_t* __restrict__ k_cache,
    uint16_t* __restrict__ v_cache, const int64_t* __restrict__ kv_base, const int64_t* __restrict__ kv_capacity,
    int hkv, int ring, int swa, const int32_t* __restrict__ block_table, int max_blocks, int page_shift,
    long long num_pages) {
    // Per-thread lookup: this kernel moves 16 bytes per thread and is bound by
    // its chain of dependent loads, which the once-per-wave scalar search of
    // locate() lengthens (132 -> 180 us per bulk append in the layer stack).
    const int kchunks = hkv * (kDqk / 8), per_tok = hkv * ((kDqk + kDv) / 8);
    const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t tok = idx / per_tok;
    const int c = (int)(idx % per_tok);
    if (tok >= total_new) return;
    // Sequence owning packed token `tok`: the last b with cu_newlens[b] <= tok.
    int lo = 0, hi = batch - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (cu_newlens[mid] <= tok) lo = mid; else hi = mid - 1;
    }
    const int b = lo;
    const int n = cu_newlens[b + 1] - cu_newlens[b];
    const int64_t ctx = ctx_lens[b];
    const int64_t pos = ctx + (tok - cu_newlens[b]);
    int64_t row;
    if (swa) {
        if (pos < ctx + n - ring) return;  // overwritten later in this same append
        row = (int64_t)b * ring + pos % ring;
    } else if (block_table) {
        if (ctx + n > ((int64_t)max_blocks << page_shift)) return;  // the whole sequence is refused
        const int64_t page = block_table[(int64_t)b * max_blocks + (pos >> page_shift)];
        if (page < 0 || page >= num_pages) return;  // unmapped block: not written
        row = (page << page_shift) | (pos & ((1 << page_shift) - 1));
    } else {
        if (ctx + n > kv_capacity[b]) return;  // the whole sequence is refused
        row = kv_base[b] + pos;
    }
    if (c < kchunks) {
        reinterpret_cast<u32x4*>(k_cache + row * hkv * kDqk)[c] = reinterpret_cast<const u32x4*>(k + tok * hkv * kDqk)[c];
    } else {
        const int cv = c - kchunks;
        reinterpret_cast<u32x4*>(v_cache + row * hkv * kDv)[cv] = reinterpret_cast<const u32x4*>(v + tok * hkv * kDv)[cv];
    }
}

// FP8 GA pool (contiguous, or paged as above): one thread turns 8 bf16
// elements (16 bytes) of a new token into 8 E4M3 codes (8 bytes).  A token is Hkv*24 such units of K then Hkv*16 of V;
// unit c of K belongs to KV head c / 24, of V to head c / 16.  Each element is
// divided by its head's scale in fp32, clamped to +-448 (the conversion does
// not saturate by itself) and rounded to nearest-even by the hardware
// conversion.  The codes are those of the IEEE fp32 quotient; the quotient is
// formed from the correctly rounded reciprocal y = 1/b (one division per
// thread) by Markstein's correction: q0 = a*y, r = fma(-b, q0, a) (exact),
// q = fma(r, y, q0), which equals the rounded a/b when nothing underflows or
// overflows (P. Markstein, "Computation of elementary functions on the IBM
// RISC System/6000 processor", 1990).  A q0 that overflows is kept (it clamps
// to +-448 as the true quotient does), as is a zero q0 (its sign then stays).
// Below the normal range q can differ from a/b by an ulp; such quotients are
// far below the smallest E4M3 step and give the same code.
__global__ __launch_bounds__(256) void kv_append_fp8_kernel(
    const uint16_t* __restrict__ k, const uint16_t* __restrict__ v, const int32_t* __restrict__ cu_newlens,
    const int32_t* __restrict__ ctx_lens, int batch, int total_new, uint8_t* __restrict__ k_cache,
    uint8_t* __restrict__ v_cache, const int64_t* __restrict__ kv_base, const int64_t* __restrict__ kv_capacity,
    const float* __restrict__ k_scale, const float* __restrict__ v_scale, int hkv,
    const int32_t* __restrict__ block_table, int max_blocks, int page_shift, long long num_pages) {
    const int kunits = hkv * (kDqk / 8), per_tok = hkv * ((kDqk + kDv) / 8);
    const TokSeq ts = locate(cu_newlens, batch, per_tok);
    const int64_t tok = ts.tok;
    const int c = ts.c;
    if (tok >= total_new) return;
    const int b = ts.b;
    const int n = cu_newlens[b + 1] - cu_newlens[b];
    const int64_t ctx = ctx_lens[b];
    const int64_t pos = ctx + (tok - cu_newlens[b]);
    int64_t row;
    if (block_table) {
        if (ctx + n > ((int64_t)max_blocks << page_shift)) return;  // the whole sequence is refused
        const int64_t page = block_table[(int64_t)b * max_blocks + (pos >> page_shift)];
        if (page < 0 || page >= num_pages) return;  // unmapped block: not written
        row = (page << page_shift) | (pos & ((1 << page_shift) - 1));
    } else {
        if (ctx + n > kv_capacity[b]) return;  // the whole sequence is refused
        row = kv_base[b] + pos;
    }
    const bool is_k = c < kunits;
    const int u = is_k ? c : c - kunits;
    const float scale = is_k ? k_scale[u / (kDqk / 8)] : v_scale[u / (kDv / 8)];
    const uint16_t* src = is_k ? k + tok * hkv * kDqk + u * 8 : v + tok * hkv * kDv + u * 8;
    uint8_t* dst = is_k ? k_cache + row * hkv * kDqk + u * 8 : v_cache + row * hkv * kDv + u * 8;
    const u32x4 w = *reinterpret_cast<const u32x4*>(src);
    float x[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        x[2 * i] = __builtin_bit_cast(float, w[i] << 16);
        x[2 * i + 1] = __builtin_bit_cast(float, w[i] & 0xffff0000u);
    }
    const float y = 1.0f / scale;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const float q0 = x[i] * y;
        const float q = __builtin_fmaf(__builtin_fmaf(-scale, q0, x[i]), y, q0);
        const float qs = (q0 == 0.0f || !__builtin_isfinite(q0)) ? q0 : q;
        x[i] = fminf(fmaxf(qs, -448.0f), 448.0f);
    }
    int lo4 = __builtin_amdgcn_cvt_pk_fp8_f32(x[0], x[1], 0, false);
    lo4 = __builtin_amdgcn_cvt_pk_fp8_f32(x[2], x[3], lo4, true);
    int hi4 = __builtin_amdgcn_cvt_pk_fp8_f32(x[4], x[5], 0, false);
    hi4 = __builtin_amdgcn_cvt_pk_fp8_f32(x[6], x[7], hi4, true);
    *reinterpret_cast<u32x2*>(dst) = u32x2{(uint32_t)lo4, (uint32_t)hi4};
}

}  // namespace

hipError_t launch_kv_append(const AppendArgs& a, hipStream_t stream) {
    if (a.total_new <= 0) return hipSuccess;
    if (a.k_cache8) {
        const int64_t threads = (int64_t)a.total_new * a.hkv * ((kDqk + kDv) / 8);
        hipLaunchKernelGGL(kv_append_fp8_kernel, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, stream, a.k,
                           a.v, a.cu_newlens, a.ctx_lens, a.batch, a.total_new, a.k_cache8, a.v_cache8, a.kv_base,
                           a.kv_capacity, a.k_scale, a.v_scale, a.hkv, a.pages.table, a.pages.max_blocks,
                           a.pages.shift, a.pages.num_pages);
        return hipGetLastError();
    }
    const int64_t threads = (int64_t)a.total_new * a.hkv * ((kDqk + kDv) / 8);
    const int64_t blocks = (threads + 255) / 256;
    hipLaunchKernelGGL(kv_append_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, a.k, a.v, a.cu_newlens,
                       a.ctx_lens, a.batch, a.total_new, a.k_cache, a.v_cache, a.kv_base, a.kv_capacity, a.hkv,
                       a.window - 1, a.swa ? 1 : 0, a.pages.table, a.pages.max_blocks, a.pages.shift,
                       a.pages.num_pages);
    return hipGetLastError();
}

}  // namespace mimo
