// api.cpp -- the C ABI of include/mimo_attn.h: host-side argument validation and dispatch.
//
// Every check here runs on the host before anything is enqueued, so misuse is
// reported by status code without touching the device.
#include <atomic>
#include <cmath>
#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>

#include "../../include/mimo_attn.h"
#include "launch.hpp"

namespace {

thread_local char g_last_error[256] = "";

int fail(int status, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    std::vsnprintf(g_last_error, sizeof g_last_error, fmt, ap);
    va_end(ap);
    return status;
}

int ok() {
    g_last_error[0] = '\0';
    return MIMO_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

constexpr int kMaxGridYZ = 65535;

// Shape checks shared by every entry point.  min_window: 1 for prefill
// (window W keeps keys p-(W-1)..p), 2 where an SWA ring of W-1 slots exists.
int check_dims(const mimo_attn_dims* d, int layer_type, int min_window) {
    if (!d) return fail(MIMO_ERR_INVALID_ARG, "dims is NULL");
    if (layer_type != MIMO_LAYER_SWA && layer_type != MIMO_LAYER_GA)
        return fail(MIMO_ERR_INVALID_ARG, "layer_type %d is neither SWA (0) nor GA (1)", layer_type);
    if (d->num_q_heads <= 0 || d->num_kv_heads <= 0)
        return fail(MIMO_ERR_INVALID_ARG, "head counts must be positive (q %d, kv %d)", d->num_q_heads,
                    d->num_kv_heads);
    if (d->num_q_heads % d->num_kv_heads != 0)
        return fail(MIMO_ERR_UNSUPPORTED, "num_q_heads %d is not a multiple of num_kv_heads %d", d->num_q_heads,
                    d->num_kv_heads);
    if (d->num_q_heads != 16 * d->num_kv_heads)
        return fail(MIMO_ERR_UNSUPPORTED, "kernels need 16 query heads per KV head (got %d/%d)", d->num_q_heads,
                    d->num_kv_heads);
    if (d->head_dim_qk != 192 || d->head_dim_v != 128)
        return fail(MIMO_ERR_UNSUPPORTED, "kernels need head_dim_qk 192 and head_dim_v 128 (got %d/%d)",
                    d->head_dim_qk, d->head_dim_v);
    // Grids carry KV heads on y and the GA combine carries query heads on y.
    if (d->num_q_heads > kMaxGridYZ)
        return fail(MIMO_ERR_UNSUPPORTED, "num_q_heads %d above %d", d->num_q_heads, kMaxGridYZ);
    if (layer_type == MIMO_LAYER_SWA && d->sliding_window < min_window)
        return fail(MIMO_ERR_INVALID_ARG, "sliding_window %d is below %d", d->sliding_window, min_window);
    if (!std::isfinite(d->softmax_scale) || !std::isfinite(d->value_scale))
        return fail(MIMO_ERR_INVALID_ARG, "softmax_scale and value_scale must be finite");
    return MIMO_OK;
}

int hip_status(hipError_t e, const char* what) {
    if (e != hipSuccess) return fail(MIMO_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
    return ok();
}

// Check mode: -1 until first read from MIMO_ATTN_CHECK, then 0 or 1.
std::atomic<int> g_check{-1};

bool check_on() {
    int v = g_check.load(std::memory_order_relaxed);
    if (v < 0) {
        const char* env = std::getenv("MIMO_ATTN_CHECK");
        int expected = -1;
        g_check.compare_exchange_strong(expected, env && std::strcmp(env, "1") == 0 ? 1 : 0);
        v = g_check.load();
    }
    return v == 1;
}

const char* const kCheckNames[] = {
    "cu_seqlens[0] is not 0", "cu_seqlens decreases", "a sequence is longer than the maximum length",
    "cu_seqlens does not end at the token count", "ctx_lens out of range", "kv_base is negative",
    "the context passes the pool capacity", "a block-table entry lies outside the pool", "a sink is NaN or +inf",
    "an FP8 scale is not positive and finite"};

// Check mode's gate in front of a call's kernels: MIMO_OK, or
// MIMO_ERR_PRECONDITION naming the violated rules (nothing else enqueued).
int precheck(const mimo::CheckArgs& c, hipStream_t stream, const char* who) {
    if (!check_on()) return MIMO_OK;
    bool gated = false;
    uint32_t bits = 0;
    if (int st = hip_status(mimo::run_check(c, stream, &gated, &bits), "check-mode pass")) return st;
    if (!gated || !bits) return MIMO_OK;
    char names[200] = "";
    size_t used = 0;
    for (int i = 0; i < (int)(sizeof kCheckNames / sizeof *kCheckNames); ++i) {
        if (!(bits >> i & 1u)) continue;
        const int n = std::snprintf(names + used, sizeof names - used, "%s%s", used ? "; " : "", kCheckNames[i]);
        if (n < 0 || (size_t)n >= sizeof names - used) break;
        used += (size_t)n;
    }
    return fail(MIMO_ERR_PRECONDITION, "%s: check mode found 0x%03x (%s)", who, bits, names);
}

// Paged pool description -> internal page table; MIMO_OK or a failure status.
int check_pages(const mimo_kv_pages* pg, mimo::PageTable* out) {
    if (!pg) return fail(MIMO_ERR_INVALID_ARG, "pages is NULL");
    if (!pg->block_table) return fail(MIMO_ERR_INVALID_ARG, "pages->block_table is NULL");
    if (pg->max_blocks < 1) return fail(MIMO_ERR_INVALID_ARG, "pages->max_blocks %d < 1", pg->max_blocks);
    if (pg->num_pages < 1) return fail(MIMO_ERR_INVALID_ARG, "pages->num_pages %lld < 1", (long long)pg->num_pages);
    if (pg->page_size <= 0) return fail(MIMO_ERR_INVALID_ARG, "pages->page_size %d is not positive", pg->page_size);
    if (pg->page_size < 16 || pg->page_size > 65536 || (pg->page_size & (pg->page_size - 1)))
        return fail(MIMO_ERR_UNSUPPORTED, "page_size %d is not a power of two in [16, 65536]", pg->page_size);
    // Pool rows are addressed as (page << shift) in 64 bits, positions in 32.
    if (pg->num_pages > (INT64_MAX / 65536) / 4096)
        return fail(MIMO_ERR_INVALID_ARG, "num_pages %lld is implausibly large", (long long)pg->num_pages);
    int shift = 0;
    while ((1 << shift) < pg->page_size) ++shift;
    out->table = pg->block_table;
    out->max_blocks = pg->max_blocks;
    out->shift = shift;
    out->num_pages = pg->num_pages;
    return MIMO_OK;
}

// GA decode: the least number of 32-key units per chunk.  split_tokens <= 0
// selects 256 keys; otherwise split_tokens rounded up to a multiple of 32.
int min_units(int32_t split_tokens) {
    if (split_tokens <= 0) return mimo::kDefaultMinUnits;
    const int64_t s = split_tokens > (1 << 30) ? (1 << 30) : split_tokens;
    return (int)((s + mimo::kTileKeys - 1) / mimo::kTileKeys);
}

}  // namespace

extern "C" {

int mimo_attn_prefill(const mimo_attn_dims* dims, int layer_type, const uint16_t* q, const uint16_t* k,
                      const uint16_t* v, const int32_t* cu_seqlens, int32_t num_seqs, int32_t max_seqlen,
                      const float* sink, uint16_t* out, float* lse, hipStream_t stream) {
    if (int st = check_dims(dims, layer_type, 1)) return st;
    if (!q || !k || !v || !cu_seqlens || !out)
        return fail(MIMO_ERR_INVALID_ARG, "q, k, v, cu_seqlens and out must be non-NULL");
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out))
        return fail(MIMO_ERR_INVALID_ARG, "q, k, v and out must be 16-byte aligned");
    if (num_seqs < 1 || num_seqs > kMaxGridYZ)
        return fail(MIMO_ERR_INVALID_ARG, "num_seqs %d outside [1, %d]", num_seqs, kMaxGridYZ);
    if (max_seqlen < 0) return fail(MIMO_ERR_INVALID_ARG, "max_seqlen %d is negative", max_seqlen);
    if (max_seqlen == 0) return ok();
    mimo::PrefillArgs a{q, k, v, cu_seqlens, sink, out, lse, num_seqs, max_seqlen, dims->num_q_heads,
                        dims->num_kv_heads, dims->sliding_window, dims->softmax_scale, dims->value_scale,
                        layer_type == MIMO_LAYER_SWA};
    mimo::CheckArgs c;
    c.cu = cu_seqlens;
    c.n_seqs = num_seqs;
    c.max_len = max_seqlen;
    c.sink = sink;
    c.hq = dims->num_q_heads;
    if (int st = precheck(c, stream, "mimo_attn_prefill")) return st;
    return hip_status(mimo::launch_prefill(a, stream), "prefill launch");
}

}  // extern "C"

namespace {

// FP8 GA pool of a chunk, decode or append call: codes and per-KV-head scales.
struct Fp8Pool {
    const uint8_t* k = nullptr;
    const uint8_t* v = nullptr;
    const float* k_scale = nullptr;
    const float* v_scale = nullptr;
};

int check_fp8(const Fp8Pool& f) {
    if (!f.k || !f.v) return fail(MIMO_ERR_INVALID_ARG, "k_cache and v_cache must be non-NULL");
    if (!aligned16(f.k) || !aligned16(f.v))
        return fail(MIMO_ERR_INVALID_ARG, "k_cache and v_cache must be 16-byte aligned");
    if (!f.k_scale || !f.v_scale) return fail(MIMO_ERR_INVALID_ARG, "k_scale and v_scale must be non-NULL");
    if ((reinterpret_cast<uintptr_t>(f.k_scale) | reinterpret_cast<uintptr_t>(f.v_scale)) & 3u)
        return fail(MIMO_ERR_INVALID_ARG, "k_scale and v_scale must be 4-byte aligned");
    return MIMO_OK;
}

// Fused RoPE of a prefill-style call: the tokens' position ids, the rotation
// and the caller's k_rot and table workspace.
struct RopeReq {
    const int32_t* positions = nullptr;
    int32_t total_tokens = 0;
    float theta = 0.0f;
    int32_t rotary_dim = 0;
    uint16_t* k_rot = nullptr;
    void* workspace = nullptr;
    size_t workspace_bytes = 0;
};

// Host checks of a RopeReq (the non-NULL pointers and the sizes).
int check_rope(const mimo_attn_dims* dims, const RopeReq& r) {
    if (!r.positions || !r.k_rot) return fail(MIMO_ERR_INVALID_ARG, "positions and k_rot must be non-NULL");
    if (!aligned16(r.k_rot)) return fail(MIMO_ERR_INVALID_ARG, "k_rot must be 16-byte aligned");
    if (r.total_tokens < 0) return fail(MIMO_ERR_INVALID_ARG, "total_tokens %d is negative", r.total_tokens);
    if (!std::isfinite(r.theta) || !(r.theta > 1.0f))
        return fail(MIMO_ERR_INVALID_ARG, "rope_theta must be finite and above 1");
    if (r.rotary_dim < 32 || r.rotary_dim > dims->head_dim_qk || r.rotary_dim % 32)
        return fail(MIMO_ERR_UNSUPPORTED, "fused RoPE needs rotary_dim a multiple of 32 in [32, %d] (got %d)",
                    dims->head_dim_qk, r.rotary_dim);
    return MIMO_OK;
}

// The (cos, sin) table workspace of a RopeReq with total_tokens > 0.
int check_rope_workspace(const RopeReq& r) {
    const size_t need = mimo::rope_table_bytes(r.total_tokens, r.rotary_dim);
    if (!r.workspace || r.workspace_bytes < need)
        return fail(MIMO_ERR_WORKSPACE, "fused RoPE needs %zu workspace bytes (got %zu%s)", need, r.workspace_bytes,
                    r.workspace ? "" : ", NULL");
    if (!aligned16(r.workspace)) return fail(MIMO_ERR_INVALID_ARG, "workspace must be 16-byte aligned");
    return MIMO_OK;
}

// Enqueues the K rotation (k -> k_rot) and the (cos, sin) table for a fused
// RoPE call whose attention then reads k_rot and rotates Q from the table.
int rope_prepare(const mimo_attn_dims* dims, const uint16_t* k, const RopeReq& r, hipStream_t stream) {
    mimo::RopePrepArgs pa{k, r.positions, r.k_rot, static_cast<float*>(r.workspace), r.total_tokens,
                          dims->num_kv_heads, r.rotary_dim, (double)r.theta};
    return hip_status(mimo::launch_rope_prep(pa, stream), "RoPE preparation launch");
}

int prefill_chunk_impl(const mimo_attn_dims* dims, int layer_type, const uint16_t* q, const uint16_t* k,
                       const uint16_t* v, const int32_t* cu_newlens, int32_t num_seqs, int32_t max_newlen,
                       const uint16_t* k_cache, const uint16_t* v_cache, const int64_t* kv_base,
                       const mimo_kv_pages* pages, const int32_t* ctx_lens, const float* sink, uint16_t* out,
                       float* lse, hipStream_t stream, const Fp8Pool* fp8 = nullptr, const RopeReq* rope = nullptr) {
    if (int st = check_dims(dims, layer_type, 2)) return st;
    if (rope) {
        if (int st = check_rope(dims, *rope)) return st;
    }
    if (fp8) {
        if (int st = check_fp8(*fp8)) return st;
        // The code pools stand in for the bf16 caches in the checks below.
        k_cache = reinterpret_cast<const uint16_t*>(fp8->k);
        v_cache = reinterpret_cast<const uint16_t*>(fp8->v);
    }
    if (!q || !k || !v || !cu_newlens || !out || !k_cache || !v_cache || !ctx_lens)
        return fail(MIMO_ERR_INVALID_ARG, "q, k, v, cu_newlens, out, k_cache, v_cache and ctx_lens must be non-NULL");
    mimo::PageTable pt;
    if (pages) {
        if (int st = check_pages(pages, &pt)) return st;
    } else if (layer_type == MIMO_LAYER_GA && !kv_base) {
        return fail(MIMO_ERR_INVALID_ARG, "GA needs kv_base");
    }
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out) || !aligned16(k_cache) ||
        !aligned16(v_cache))
        return fail(MIMO_ERR_INVALID_ARG, "q, k, v, out and the caches must be 16-byte aligned");
    if (num_seqs < 1 || num_seqs > kMaxGridYZ)
        return fail(MIMO_ERR_INVALID_ARG, "num_seqs %d outside [1, %d]", num_seqs, kMaxGridYZ);
    if (max_newlen < 0) return fail(MIMO_ERR_INVALID_ARG, "max_newlen %d is negative", max_newlen);
    if (max_newlen == 0 || (rope && rope->total_tokens == 0)) return ok();
    if (rope) {
        if (int st = check_rope_workspace(*rope)) return st;
    }
    mimo::PrefillArgs a{q, rope ? rope->k_rot : k, v, cu_newlens, sink, out, lse, num_seqs, max_newlen,
                        dims->num_q_heads, dims->num_kv_heads, dims->sliding_window, dims->softmax_scale,
                        dims->value_scale, layer_type == MIMO_LAYER_SWA};
    if (rope) {
        a.rope_tab = static_cast<const float*>(rope->workspace);
        a.rope_half = rope->rotary_dim / 2;
    }
    a.k_cache = k_cache;
    a.v_cache = v_cache;
    a.kv_base = kv_base;
    a.ctx_lens = ctx_lens;
    a.pages = pt;
    if (fp8) {
        a.k_cache = a.v_cache = nullptr;
        a.k_cache8 = fp8->k;
        a.v_cache8 = fp8->v;
        a.k_scale = fp8->k_scale;
        a.v_scale = fp8->v_scale;
    }
    mimo::CheckArgs c;
    c.cu = cu_newlens;
    c.n_seqs = num_seqs;
    c.max_len = max_newlen;
    c.ctx = ctx_lens;
    c.batch = num_seqs;
    c.new_from_cu = true;
    if (layer_type == MIMO_LAYER_GA && !pages) c.kv_base = kv_base;
    c.pages = pt;
    c.sink = sink;
    c.hq = dims->num_q_heads;
    if (fp8) {
        c.scales = fp8->k_scale;
        c.scales_v = fp8->v_scale;
        c.n_scales = dims->num_kv_heads;
    }
    if (rope) c.total = rope->total_tokens;
    if (int st = precheck(c, stream, "chunked prefill")) return st;
    if (rope) {
        if (int st = rope_prepare(dims, k, *rope, stream)) return st;
    }
    return hip_status(mimo::launch_prefill_chunk(a, stream), "chunked prefill launch");
}

}  // namespace

extern "C" {

int mimo_attn_prefill_chunk(const mimo_attn_dims* dims, int layer_type, const uint16_t* q, const uint16_t* k,
                            const uint16_t* v, const int32_t* cu_newlens, int32_t num_seqs, int32_t max_newlen,
                            const uint16_t* k_cache, const uint16_t* v_cache, const int64_t* kv_base,
                            const int32_t* ctx_lens, const float* sink, uint16_t* out, float* lse,
                            hipStream_t stream) {
    return prefill_chunk_impl(dims, layer_type, q, k, v, cu_newlens, num_seqs, max_newlen, k_cache, v_cache, kv_base,
                              nullptr, ctx_lens, sink, out, lse, stream);
}

int mimo_attn_prefill_chunk_paged(const mimo_attn_dims* dims, const uint16_t* q, const uint16_t* k,
                                  const uint16_t* v, const int32_t* cu_newlens, int32_t num_seqs, int32_t max_newlen,
                                  const uint16_t* k_cache, const uint16_t* v_cache, const mimo_kv_pages* pages,
                                  const int32_t* ctx_lens, const float* sink, uint16_t* out, float* lse,
                                  hipStream_t stream) {
    if (!pages) return fail(MIMO_ERR_INVALID_ARG, "pages is NULL");
    return prefill_chunk_impl(dims, MIMO_LAYER_GA, q, k, v, cu_newlens, num_seqs, max_newlen, k_cache, v_cache,
                              nullptr, pages, ctx_lens, sink, out, lse, stream);
}

int mimo_attn_prefill_chunk_rope(const mimo_attn_dims* dims, int layer_type, const uint16_t* q, const uint16_t* k,
                                 const uint16_t* v, const int32_t* positions, const int32_t* cu_newlens,
                                 int32_t num_seqs, int32_t max_newlen, int32_t total_new, const uint16_t* k_cache,
                                 const uint16_t* v_cache, const int64_t* kv_base, const mimo_kv_pages* pages,
                                 const int32_t* ctx_lens, float rope_theta, int32_t rotary_dim, const float* sink,
                                 uint16_t* out, float* lse, uint16_t* k_rot, void* workspace, size_t workspace_bytes,
                                 hipStream_t stream) {
    if (pages && layer_type != MIMO_LAYER_GA)
        return fail(MIMO_ERR_INVALID_ARG, "a paged pool holds a GA layer's cache only");
    RopeReq r;
    r.positions = positions;
    r.total_tokens = total_new;
    r.theta = rope_theta;
    r.rotary_dim = rotary_dim;
    r.k_rot = k_rot;
    r.workspace = workspace;
    r.workspace_bytes = workspace_bytes;
    return prefill_chunk_impl(dims, layer_type, q, k, v, cu_newlens, num_seqs, max_newlen, k_cache, v_cache, kv_base,
                              pages, ctx_lens, sink, out, lse, stream, nullptr, &r);
}

int mimo_attn_prefill_chunk_fp8(const mimo_attn_dims* dims, const uint16_t* q, const uint16_t* k, const uint16_t* v,
                                const int32_t* cu_newlens, int32_t num_seqs, int32_t max_newlen, const uint8_t* k_cache,
                                const uint8_t* v_cache, const int64_t* kv_base, const float* k_scale,
                                const float* v_scale, const int32_t* ctx_lens, const float* sink, uint16_t* out,
                                float* lse, hipStream_t stream) {
    const Fp8Pool f{k_cache, v_cache, k_scale, v_scale};
    return prefill_chunk_impl(dims, MIMO_LAYER_GA, q, k, v, cu_newlens, num_seqs, max_newlen, nullptr, nullptr,
                              kv_base, nullptr, ctx_lens, sink, out, lse, stream, &f);
}

int mimo_attn_prefill_chunk_fp8_paged(const mimo_attn_dims* dims, const uint16_t* q, const uint16_t* k,
                                      const uint16_t* v, const int32_t* cu_newlens, int32_t num_seqs,
                                      int32_t max_newlen, const uint8_t* k_cache, const uint8_t* v_cache,
                                      const mimo_kv_pages* pages, const float* k_scale, const float* v_scale,
                                      const int32_t* ctx_lens, const float* sink, uint16_t* out, float* lse,
                                      hipStream_t stream) {
    if (!pages) return fail(MIMO_ERR_INVALID_ARG, "pages is NULL");
    const Fp8Pool f{k_cache, v_cache, k_scale, v_scale};
    return prefill_chunk_impl(dims, MIMO_LAYER_GA, q, k, v, cu_newlens, num_seqs, max_newlen, nullptr, nullptr,
                              nullptr, pages, ctx_lens, sink, out, lse, stream, &f);
}

size_t mimo_attn_decode_workspace_size(const mimo_attn_dims* dims, int layer_type, int32_t batch, int32_t max_ctx,
                                       int32_t split_tokens) {
    if (check_dims(dims, layer_type, 2) != MIMO_OK || batch < 1 || max_ctx < 0 || max_ctx == INT32_MAX) return 0;
    if (layer_type == MIMO_LAYER_SWA || batch > kMaxGridYZ) return 0;
    const int chunks = mimo::ga_grid_chunks(batch, max_ctx, min_units(split_tokens));
    return mimo::ga_workspace_bytes(batch, chunks, dims->num_q_heads);
}

}  // extern "C"

namespace {

int decode_impl(const mimo_attn_dims* dims, int layer_type, const uint16_t* q, const uint16_t* k_new,
                const uint16_t* v_new, const uint16_t* k_cache, const uint16_t* v_cache, const int64_t* kv_base,
                const mimo_kv_pages* pages, const int32_t* ctx_lens, int32_t batch, int32_t max_ctx,
                int32_t split_tokens, const float* sink, uint16_t* out, float* lse, void* workspace,
                size_t workspace_bytes, hipStream_t stream, const Fp8Pool* fp8 = nullptr, bool append = false,
                const int64_t* kv_capacity = nullptr, int max_chunks = mimo::kGaMaxChunks,
                const mimo::DecodeRope* rope = nullptr) {
    if (int st = check_dims(dims, layer_type, 2)) return st;
    if (!q || !k_new || !v_new || !ctx_lens || !out)
        return fail(MIMO_ERR_INVALID_ARG, "q, k_new, v_new, ctx_lens and out must be non-NULL");
    if (!aligned16(q) || !aligned16(k_new) || !aligned16(v_new) || !aligned16(out))
        return fail(MIMO_ERR_INVALID_ARG, "q, k_new, v_new and out must be 16-byte aligned");
    if (batch < 1) return fail(MIMO_ERR_INVALID_ARG, "batch %d < 1", batch);
    if (max_ctx < 0 || max_ctx == INT32_MAX) return fail(MIMO_ERR_INVALID_ARG, "max_ctx %d out of range", max_ctx);
    if (fp8) {
        if (int st = check_fp8(*fp8)) return st;
    } else {
        if (!k_cache || !v_cache) return fail(MIMO_ERR_INVALID_ARG, "k_cache and v_cache must be non-NULL");
        if (!aligned16(k_cache) || !aligned16(v_cache))
            return fail(MIMO_ERR_INVALID_ARG, "k_cache and v_cache must be 16-byte aligned");
    }
    mimo::PageTable pt;
    if (pages) {
        if (int st = check_pages(pages, &pt)) return st;
    } else {
        // The kernels address a sequence's cache rows with 32-bit byte offsets.
        const int64_t row_bytes = (int64_t)dims->num_kv_heads * dims->head_dim_qk * (fp8 ? 1 : 2);
        const int64_t rows = layer_type == MIMO_LAYER_SWA ? (int64_t)dims->sliding_window : (int64_t)max_ctx + 1;
        if (rows * row_bytes > INT32_MAX)
            return fail(MIMO_ERR_UNSUPPORTED, "a sequence's cached keys exceed 2 GiB (%lld rows of %lld bytes)",
                        (long long)rows, (long long)row_bytes);
    }
    mimo::DecodeArgs a{q, k_new, v_new, k_cache, v_cache, kv_base, ctx_lens, sink, out, lse, workspace, batch,
                       max_ctx, min_units(split_tokens), dims->num_q_heads, dims->num_kv_heads, dims->sliding_window,
                       dims->softmax_scale, dims->value_scale};
    a.max_chunks = max_chunks;
    a.pages = pt;
    if (fp8) {
        a.k_cache8 = fp8->k;
        a.v_cache8 = fp8->v;
        a.k_scale = fp8->k_scale;
        a.v_scale = fp8->v_scale;
    }
    if (append) {
        if (fp8 || pages) return fail(MIMO_ERR_UNSUPPORTED, "fused append covers bf16 ring and contiguous pools only");
        if (layer_type == MIMO_LAYER_GA && (!kv_base || !kv_capacity))
            return fail(MIMO_ERR_INVALID_ARG, "GA decode with append needs kv_base and kv_capacity");
        a.append_k = const_cast<uint16_t*>(k_cache);
        a.append_v = const_cast<uint16_t*>(v_cache);
        a.kv_capacity = kv_capacity;
    }
    if (rope) a.rope = *rope;
    mimo::CheckArgs c;
    c.ctx = ctx_lens;
    c.batch = batch;
    c.max_ctx = max_ctx;
    c.new_tokens = 1;
    if (layer_type == MIMO_LAYER_GA && !pages) {
        c.kv_base = kv_base;
        if (append) c.kv_capacity = kv_capacity;
    }
    c.pages = pt;
    c.sink = sink;
    c.hq = dims->num_q_heads;
    if (fp8) {
        c.scales = fp8->k_scale;
        c.scales_v = fp8->v_scale;
        c.n_scales = dims->num_kv_heads;
    }
    if (layer_type == MIMO_LAYER_SWA) {
        if (batch > INT32_MAX / 2) return fail(MIMO_ERR_UNSUPPORTED, "batch too large");
        if (int st = precheck(c, stream, "SWA decode")) return st;
        return hip_status(mimo::launch_decode_swa(a, stream), "SWA decode launch");
    }
    if (!kv_base && !pages) return fail(MIMO_ERR_INVALID_ARG, "GA decode needs kv_base");
    if (batch > kMaxGridYZ) return fail(MIMO_ERR_UNSUPPORTED, "GA decode batch %d above %d", batch, kMaxGridYZ);
    const size_t need = mimo::ga_workspace_bytes(batch, mimo::ga_grid_chunks(batch, max_ctx, a.min_units, max_chunks),
                                                 dims->num_q_heads);
    if (!workspace || workspace_bytes < need)
        return fail(MIMO_ERR_WORKSPACE, "GA decode needs %zu workspace bytes (got %zu%s)", need, workspace_bytes,
                    workspace ? "" : ", NULL");
    if (!aligned16(workspace)) return fail(MIMO_ERR_INVALID_ARG, "workspace must be 16-byte aligned");
    if (int st = precheck(c, stream, "GA decode")) return st;
    return hip_status(mimo::launch_decode_ga(a, stream), "GA decode launch");
}

int kv_append_impl(const mimo_attn_dims* dims, int layer_type, const uint16_t* k, const uint16_t* v,
                   const int32_t* cu_newlens, const int32_t* ctx_lens, int32_t batch, int32_t total_new,
                   uint16_t* k_cache, uint16_t* v_cache, const int64_t* kv_base, const int64_t* kv_capacity,
                   const mimo_kv_pages* pages, hipStream_t stream, const Fp8Pool* fp8 = nullptr) {
    if (int st = check_dims(dims, layer_type, 2)) return st;
    if (!k || !v || !cu_newlens || !ctx_lens)
        return fail(MIMO_ERR_INVALID_ARG, "k, v, cu_newlens and ctx_lens must be non-NULL");
    if (!aligned16(k) || !aligned16(v)) return fail(MIMO_ERR_INVALID_ARG, "k and v must be 16-byte aligned");
    if (fp8) {
        if (int st = check_fp8(*fp8)) return st;
    } else {
        if (!k_cache || !v_cache) return fail(MIMO_ERR_INVALID_ARG, "k_cache and v_cache must be non-NULL");
        if (!aligned16(k_cache) || !aligned16(v_cache))
            return fail(MIMO_ERR_INVALID_ARG, "k_cache and v_cache must be 16-byte aligned");
    }
    if (batch < 1) return fail(MIMO_ERR_INVALID_ARG, "batch %d < 1", batch);
    if (total_new < 0) return fail(MIMO_ERR_INVALID_ARG, "total_new %d is negative", total_new);
    mimo::PageTable pt;
    if (pages) {
        if (int st = check_pages(pages, &pt)) return st;
    } else if (layer_type == MIMO_LAYER_GA && (!kv_base || !kv_capacity)) {
        return fail(MIMO_ERR_INVALID_ARG, "GA append needs kv_base and kv_capacity");
    }
    const int64_t blocks = ((int64_t)total_new * dims->num_kv_heads * 40 + 255) / 256;
    if (blocks > INT32_MAX) return fail(MIMO_ERR_UNSUPPORTED, "append of %d tokens is too large", total_new);
    if (total_new == 0) return ok();
    mimo::AppendArgs a{k, v, cu_newlens, ctx_lens, k_cache, v_cache, kv_base, kv_capacity, batch, total_new,
                       dims->num_kv_heads, dims->sliding_window, layer_type == MIMO_LAYER_SWA};
    a.pages = pt;
    if (fp8) {
        a.k_cache8 = const_cast<uint8_t*>(fp8->k);
        a.v_cache8 = const_cast<uint8_t*>(fp8->v);
        a.k_scale = fp8->k_scale;
        a.v_scale = fp8->v_scale;
    }
    mimo::CheckArgs c;
    c.cu = cu_newlens;
    c.n_seqs = batch;
    c.total = total_new;
    c.ctx = ctx_lens;
    c.batch = batch;
    c.new_from_cu = true;
    if (layer_type == MIMO_LAYER_GA && !pages) {
        c.kv_base = kv_base;
        c.kv_capacity = kv_capacity;
    }
    c.pages = pt;
    c.pages_cover_new = true;
    if (fp8) {
        c.scales = fp8->k_scale;
        c.scales_v = fp8->v_scale;
        c.n_scales = dims->num_kv_heads;
    }
    if (int st = precheck(c, stream, "KV append")) return st;
    return hip_status(mimo::launch_kv_append(a, stream), "KV append launch");
}

}  // namespace

extern "C" {

int mimo_attn_decode(const mimo_attn_dims* dims, int layer_type, const uint16_t* q, const uint16_t* k_new,
                     const uint16_t* v_new, const uint16_t* k_cache, const uint16_t* v_cache, const int64_t* kv_base,
                     const int32_t* ctx_lens, int32_t batch, int32_t max_ctx, int32_t split_tokens, const float* sink,
                     uint16_t* out, float* lse, void* workspace, size_t workspace_bytes, hipStream_t stream) {
    return decode_impl(dims, layer_type, q, k_new, v_new, k_cache, v_cache, kv_base, nullptr, ctx_lens, batch,
                       max_ctx, split_tokens, sink, out, lse, workspace, workspace_bytes, stream);
}

int mimo_attn_decode_noalloc(const mimo_attn_dims* dims, int layer_type, const uint16_t* q, const uint16_t* k_new,
                             const uint16_t* v_new, const uint16_t* k_cache, const uint16_t* v_cache,
                             const int64_t* kv_base, const int32_t* ctx_lens, int32_t batch, int32_t max_ctx,
                             int32_t split_tokens, const float* sink, uint16_t* out, float* lse, hipStream_t stream) {
    if (int st = check_dims(dims, layer_type, 2)) return st;
    if (layer_type == MIMO_LAYER_SWA)  // SWA decode uses no workspace
        return decode_impl(dims, layer_type, q, k_new, v_new, k_cache, v_cache, kv_base, nullptr, ctx_lens, batch,
                           max_ctx, split_tokens, sink, out, lse, nullptr, 0, stream);
    if (batch < 1 || batch > kMaxGridYZ) return fail(MIMO_ERR_INVALID_ARG, "batch %d outside [1, %d]", batch, kMaxGridYZ);
    // The chunk count is capped so that header + (chunks + batch) slots fit the scratch array.
    const size_t slot = (size_t)dims->num_q_heads * (2 + 128) * sizeof(float);
    const size_t header = mimo::ga_header_bytes(batch);
    const size_t room = mimo::kNoAllocScratchBytes > header ? (mimo::kNoAllocScratchBytes - header) / slot : 0;
    const long long chunks = (long long)room - batch;
    if (chunks < 1)
        return fail(MIMO_ERR_UNSUPPORTED,
                    "batch %d with %d query heads needs more than the %zu-byte scratch of the no-allocation decode "
                    "(use mimo_attn_decode with a workspace)",
                    batch, dims->num_q_heads, (size_t)mimo::kNoAllocScratchBytes);
    void* ws = nullptr;
    if (int st = hip_status(mimo::noalloc_scratch(&ws), "no-allocation scratch lookup")) return st;
    return decode_impl(dims, layer_type, q, k_new, v_new, k_cache, v_cache, kv_base, nullptr, ctx_lens, batch,
                       max_ctx, split_tokens, sink, out, lse, ws, mimo::kNoAllocScratchBytes, stream, nullptr, false,
                       nullptr, (int)(chunks < mimo::kGaMaxChunks ? chunks : mimo::kGaMaxChunks));
}

int mimo_attn_decode_append(const mimo_attn_dims* dims, int layer_type, const uint16_t* q, const uint16_t* k_new,
                            const uint16_t* v_new, uint16_t* k_cache, uint16_t* v_cache, const int64_t* kv_base,
                            const int64_t* kv_capacity, const int32_t* ctx_lens, int32_t batch, int32_t max_ctx,
                            int32_t split_tokens, const float* sink, uint16_t* out, float* lse, void* workspace,
                            size_t workspace_bytes, hipStream_t stream) {
    return decode_impl(dims, layer_type, q, k_new, v_new, k_cache, v_cache, kv_base, nullptr, ctx_lens, batch,
                       max_ctx, split_tokens, sink, out, lse, workspace, workspace_bytes, stream, nullptr, true,
                       kv_capacity);
}

int mimo_attn_decode_append_rope(const mimo_attn_dims* dims, int layer_type, const uint16_t* q,
                                 const uint16_t* k_new, const uint16_t* v_new, const int32_t* positions,
                                 uint16_t* k_cache, uint16_t* v_cache, const int64_t* kv_base,
                                 const int64_t* kv_capacity, const int32_t* ctx_lens, int32_t batch, int32_t max_ctx,
                                 int32_t split_tokens, float rope_theta, int32_t rotary_dim, const float* sink,
                                 uint16_t* out, float* lse, void* workspace, size_t workspace_bytes,
                                 hipStream_t stream) {
    if (int st = check_dims(dims, layer_type, 2)) return st;
    if (!positions) return fail(MIMO_ERR_INVALID_ARG, "positions must be non-NULL");
    if (!std::isfinite(rope_theta) || !(rope_theta > 1.0f))
        return fail(MIMO_ERR_INVALID_ARG, "rope_theta must be finite and above 1");
    if (rotary_dim < 64 || rotary_dim > dims->head_dim_qk || rotary_dim % 64)
        return fail(MIMO_ERR_UNSUPPORTED, "fused decode RoPE needs rotary_dim a multiple of 64 in [64, %d] (got %d)",
                    dims->head_dim_qk, rotary_dim);
    mimo::DecodeRope r{positions, rotary_dim / 2, mimo::rope_inv_freq((double)rope_theta, rotary_dim)};
    return decode_impl(dims, layer_type, q, k_new, v_new, k_cache, v_cache, kv_base, nullptr, ctx_lens, batch,
                       max_ctx, split_tokens, sink, out, lse, workspace, workspace_bytes, stream, nullptr, true,
                       kv_capacity, mimo::kGaMaxChunks, &r);
}

int mimo_attn_decode_paged(const mimo_attn_dims* dims, const uint16_t* q, const uint16_t* k_new,
                           const uint16_t* v_new, const uint16_t* k_cache, const uint16_t* v_cache,
                           const mimo_kv_pages* pages, const int32_t* ctx_lens, int32_t batch, int32_t max_ctx,
                           int32_t split_tokens, const float* sink, uint16_t* out, float* lse, void* workspace,
                           size_t workspace_bytes, hipStream_t stream) {
    if (!pages) return fail(MIMO_ERR_INVALID_ARG, "pages is NULL");
    return decode_impl(dims, MIMO_LAYER_GA, q, k_new, v_new, k_cache, v_cache, nullptr, pages, ctx_lens, batch,
                       max_ctx, split_tokens, sink, out, lse, workspace, workspace_bytes, stream);
}

int mimo_kv_append(const mimo_attn_dims* dims, int layer_type, const uint16_t* k, const uint16_t* v,
                   const int32_t* cu_newlens, const int32_t* ctx_lens, int32_t batch, int32_t total_new,
                   uint16_t* k_cache, uint16_t* v_cache, const int64_t* kv_base, const int64_t* kv_capacity,
                   hipStream_t stream) {
    return kv_append_impl(dims, layer_type, k, v, cu_newlens, ctx_lens, batch, total_new, k_cache, v_cache, kv_base,
                          kv_capacity, nullptr, stream);
}

int mimo_kv_append_paged(const mimo_attn_dims* dims, const uint16_t* k, const uint16_t* v,
                         const int32_t* cu_newlens, const int32_t* ctx_lens, int32_t batch, int32_t total_new,
                         uint16_t* k_cache, uint16_t* v_cache, const mimo_kv_pages* pages, hipStream_t stream) {
    if (!pages) return fail(MIMO_ERR_INVALID_ARG, "pages is NULL");
    return kv_append_impl(dims, MIMO_LAYER_GA, k, v, cu_newlens, ctx_lens, batch, total_new, k_cache, v_cache,
                          nullptr, nullptr, pages, stream);
}

int mimo_attn_decode_fp8(const mimo_attn_dims* dims, const uint16_t* q, const uint16_t* k_new,
                         const uint16_t* v_new, const uint8_t* k_cache, const uint8_t* v_cache, const int64_t* kv_base,
                         const float* k_scale, const float* v_scale, const int32_t* ctx_lens, int32_t batch,
                         int32_t max_ctx, int32_t split_tokens, const float* sink, uint16_t* out, float* lse,
                         void* workspace, size_t workspace_bytes, hipStream_t stream) {
    const Fp8Pool f{k_cache, v_cache, k_scale, v_scale};
    return decode_impl(dims, MIMO_LAYER_GA, q, k_new, v_new, nullptr, nullptr, kv_base, nullptr, ctx_lens, batch,
                       max_ctx, split_tokens, sink, out, lse, workspace, workspace_bytes, stream, &f);
}

int mimo_kv_append_fp8(const mimo_attn_dims* dims, const uint16_t* k, const uint16_t* v, const int32_t* cu_newlens,
                       const int32_t* ctx_lens, int32_t batch, int32_t total_new, uint8_t* k_cache, uint8_t* v_cache,
                       const int64_t* kv_base, const int64_t* kv_capacity, const float* k_scale,
                       const float* v_scale, hipStream_t stream) {
    const Fp8Pool f{k_cache, v_cache, k_scale, v_scale};
    return kv_append_impl(dims, MIMO_LAYER_GA, k, v, cu_newlens, ctx_lens, batch, total_new, nullptr, nullptr,
                          kv_base, kv_capacity, nullptr, stream, &f);
}

int mimo_attn_decode_fp8_paged(const mimo_attn_dims* dims, const uint16_t* q, const uint16_t* k_new,
                               const uint16_t* v_new, const uint8_t* k_cache, const uint8_t* v_cache,
                               const mimo_kv_pages* pages, const float* k_scale, const float* v_scale,
                               const int32_t* ctx_lens, int32_t batch, int32_t max_ctx, int32_t split_tokens,
                               const float* sink, uint16_t* out, float* lse, void* workspace, size_t workspace_bytes,
                               hipStream_t stream) {
    if (!pages) return fail(MIMO_ERR_INVALID_ARG, "pages is NULL");
    const Fp8Pool f{k_cache, v_cache, k_scale, v_scale};
    return decode_impl(dims, MIMO_LAYER_GA, q, k_new, v_new, nullptr, nullptr, nullptr, pages, ctx_lens, batch,
                       max_ctx, split_tokens, sink, out, lse, workspace, workspace_bytes, stream, &f);
}

int mimo_kv_append_fp8_paged(const mimo_attn_dims* dims, const uint16_t* k, const uint16_t* v,
                             const int32_t* cu_newlens, const int32_t* ctx_lens, int32_t batch, int32_t total_new,
                             uint8_t* k_cache, uint8_t* v_cache, const mimo_kv_pages* pages, const float* k_scale,
                             const float* v_scale, hipStream_t stream) {
    if (!pages) return fail(MIMO_ERR_INVALID_ARG, "pages is NULL");
    const Fp8Pool f{k_cache, v_cache, k_scale, v_scale};
    return kv_append_impl(dims, MIMO_LAYER_GA, k, v, cu_newlens, ctx_lens, batch, total_new, nullptr, nullptr,
                          nullptr, nullptr, pages, stream, &f);
}

size_t mimo_attn_prefill_backward_workspace_size(const mimo_attn_dims* dims, int32_t total_tokens) {
    if (check_dims(dims, MIMO_LAYER_GA, 1) != MIMO_OK || total_tokens < 0) return 0;
    return mimo::backward_workspace_bytes(total_tokens, dims->num_q_heads);
}

int mimo_attn_prefill_backward(const mimo_attn_dims* dims, int layer_type, const uint16_t* q, const uint16_t* k,
                               const uint16_t* v, const uint16_t* out, const float* lse, const uint16_t* dout,
                               const int32_t* cu_seqlens, int32_t num_seqs, int32_t max_seqlen,
                               int32_t total_tokens, const float* sink, uint16_t* dq, uint16_t* dk, uint16_t* dv,
                               float* dsink, void* workspace, size_t workspace_bytes, hipStream_t stream) {
    if (int st = check_dims(dims, layer_type, 1)) return st;
    if (!q || !k || !v || !out || !lse || !dout || !cu_seqlens || !dq || !dk || !dv)
        return fail(MIMO_ERR_INVALID_ARG, "q, k, v, out, lse, dout, cu_seqlens, dq, dk and dv must be non-NULL");
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out) || !aligned16(dout) || !aligned16(dq) ||
        !aligned16(dk) || !aligned16(dv))
        return fail(MIMO_ERR_INVALID_ARG, "q, k, v, out, dout, dq, dk and dv must be 16-byte aligned");
    if (num_seqs < 1 || num_seqs > kMaxGridYZ)
        return fail(MIMO_ERR_INVALID_ARG, "num_seqs %d outside [1, %d]", num_seqs, kMaxGridYZ);
    if (max_seqlen < 0) return fail(MIMO_ERR_INVALID_ARG, "max_seqlen %d is negative", max_seqlen);
    if (total_tokens < 0) return fail(MIMO_ERR_INVALID_ARG, "total_tokens %d is negative", total_tokens);
    if ((int64_t)total_tokens * dims->num_q_heads > (int64_t)INT32_MAX * 8)
        return fail(MIMO_ERR_UNSUPPORTED, "total_tokens %d is too large", total_tokens);
    const size_t need = mimo::backward_workspace_bytes(total_tokens, dims->num_q_heads);
    mimo::BackwardArgs a{q, k, v, out, lse, dout, cu_seqlens, sink, dq, dk, dv, dsink, workspace, num_seqs,
                         max_seqlen, total_tokens, dims->num_q_heads, dims->num_kv_heads, dims->sliding_window,
                         dims->softmax_scale, dims->value_scale, layer_type == MIMO_LAYER_SWA};
    if (max_seqlen == 0 || total_tokens == 0) {
        // Nothing contributes: no workspace is used, only dsink (if given) is written, as zeros.
        if (!dsink) return ok();
        return hip_status(mimo::launch_prefill_backward(a, stream), "backward launch");
    }
    if (!workspace || workspace_bytes < need)
        return fail(MIMO_ERR_WORKSPACE, "backward needs %zu workspace bytes (got %zu%s)", need, workspace_bytes,
                    workspace ? "" : ", NULL");
    if (!aligned16(workspace)) return fail(MIMO_ERR_INVALID_ARG, "workspace must be 16-byte aligned");
    mimo::CheckArgs c;
    c.cu = cu_seqlens;
    c.n_seqs = num_seqs;
    c.max_len = max_seqlen;
    c.total = total_tokens;
    c.sink = sink;
    c.hq = dims->num_q_heads;
    if (int st = precheck(c, stream, "backward")) return st;
    return hip_status(mimo::launch_prefill_backward(a, stream), "backward launch");
}

size_t mimo_attn_prefill_rope_workspace_size(const mimo_attn_dims* dims, int32_t total_tokens, int32_t rotary_dim) {
    if (check_dims(dims, MIMO_LAYER_GA, 1) != MIMO_OK || total_tokens < 0 || rotary_dim < 32 ||
        rotary_dim > dims->head_dim_qk || rotary_dim % 32)
        return 0;
    return mimo::rope_table_bytes(total_tokens, rotary_dim);
}

int mimo_attn_prefill_rope(const mimo_attn_dims* dims, int layer_type, const uint16_t* q, const uint16_t* k,
                           const uint16_t* v, const int32_t* positions, const int32_t* cu_seqlens, int32_t num_seqs,
                           int32_t max_seqlen, int32_t total_tokens, float rope_theta, int32_t rotary_dim,
                           const float* sink, uint16_t* out, float* lse, uint16_t* k_rot, void* workspace,
                           size_t workspace_bytes, hipStream_t stream) {
    if (int st = check_dims(dims, layer_type, 1)) return st;
    if (!q || !k || !v || !positions || !cu_seqlens || !out || !k_rot)
        return fail(MIMO_ERR_INVALID_ARG, "q, k, v, positions, cu_seqlens, out and k_rot must be non-NULL");
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out) || !aligned16(k_rot))
        return fail(MIMO_ERR_INVALID_ARG, "q, k, v, out and k_rot must be 16-byte aligned");
    if (num_seqs < 1 || num_seqs > kMaxGridYZ)
        return fail(MIMO_ERR_INVALID_ARG, "num_seqs %d outside [1, %d]", num_seqs, kMaxGridYZ);
    if (max_seqlen < 0) return fail(MIMO_ERR_INVALID_ARG, "max_seqlen %d is negative", max_seqlen);
    RopeReq r;
    r.positions = positions;
    r.total_tokens = total_tokens;
    r.theta = rope_theta;
    r.rotary_dim = rotary_dim;
    r.k_rot = k_rot;
    r.workspace = workspace;
    r.workspace_bytes = workspace_bytes;
    if (int st = check_rope(dims, r)) return st;
    if (max_seqlen == 0 || total_tokens == 0) return ok();
    if (int st = check_rope_workspace(r)) return st;
    mimo::CheckArgs c;
    c.cu = cu_seqlens;
    c.n_seqs = num_seqs;
    c.max_len = max_seqlen;
    c.total = total_tokens;
    c.sink = sink;
    c.hq = dims->num_q_heads;
    if (int st = precheck(c, stream, "mimo_attn_prefill_rope")) return st;
    if (int st = rope_prepare(dims, k, r, stream)) return st;
    mimo::PrefillArgs a{q, k_rot, v, cu_seqlens, sink, out, lse, num_seqs, max_seqlen, dims->num_q_heads,
                        dims->num_kv_heads, dims->sliding_window, dims->softmax_scale, dims->value_scale,
                        layer_type == MIMO_LAYER_SWA};
    a.rope_tab = static_cast<const float*>(workspace);
    a.rope_half = rotary_dim / 2;
    return hip_status(mimo::launch_prefill(a, stream), "prefill launch");
}

int mimo_rope_apply(const mimo_attn_dims* dims, uint16_t* q, uint16_t* k, const int32_t* positions,
                    int32_t total_tokens, float rope_theta, int32_t rotary_dim, hipStream_t stream) {
    if (int st = check_dims(dims, MIMO_LAYER_GA, 1)) return st;
    if (!q && !k) return fail(MIMO_ERR_INVALID_ARG, "q and k are both NULL");
    if (!positions) return fail(MIMO_ERR_INVALID_ARG, "positions must be non-NULL");
    if ((q && !aligned16(q)) || (k && !aligned16(k))) return fail(MIMO_ERR_INVALID_ARG, "q and k must be 16-byte aligned");
    if (total_tokens < 0) return fail(MIMO_ERR_INVALID_ARG, "total_tokens %d is negative", total_tokens);
    if (!std::isfinite(rope_theta) || !(rope_theta > 1.0f))
        return fail(MIMO_ERR_INVALID_ARG, "rope_theta must be finite and above 1");
    if (rotary_dim < 0 || rotary_dim > dims->head_dim_qk)
        return fail(MIMO_ERR_INVALID_ARG, "rotary_dim %d outside [0, %d]", rotary_dim, dims->head_dim_qk);
    if (rotary_dim % 16) return fail(MIMO_ERR_UNSUPPORTED, "rotary_dim %d is not a multiple of 16", rotary_dim);
    if (total_tokens == 0 || rotary_dim == 0) return ok();
    mimo::RopeArgs a{q, k, positions, total_tokens, dims->num_q_heads, dims->num_kv_heads, rotary_dim,
                     (double)rope_theta};
    return hip_status(mimo::launch_rope(a, stream), "rope launch");
}

const char* mimo_status_string(int status) {
    switch (status) {
        case MIMO_OK: return "MIMO_OK";
        case MIMO_ERR_INVALID_ARG: return "MIMO_ERR_INVALID_ARG";
        case MIMO_ERR_UNSUPPORTED: return "MIMO_ERR_UNSUPPORTED";
        case MIMO_ERR_WORKSPACE: return "MIMO_ERR_WORKSPACE";
        case MIMO_ERR_HIP: return "MIMO_ERR_HIP";
        case MIMO_ERR_PRECONDITION: return "MIMO_ERR_PRECONDITION";
        default: return "MIMO_ERR_UNKNOWN";
    }
}

int mimo_attn_set_check(int enable) {
    const int before = check_on() ? 1 : 0;
    g_check.store(enable ? 1 : 0);
    return before;
}

int mimo_attn_check_flags(uint32_t* flags, int clear) {
    if (!flags) return fail(MIMO_ERR_INVALID_ARG, "flags is NULL");
    return hip_status(mimo::check_flags(flags, clear != 0), "check word read");
}

const char* mimo_last_error(void) { return g_last_error; }

int mimo_abi_version(void) { return MIMO_ATTN_ABI_VERSION; }

}  // extern "C"
