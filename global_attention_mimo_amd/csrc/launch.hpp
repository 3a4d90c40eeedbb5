// launch.hpp -- host-side launchers of the attention kernels (internal to the library).
// Arguments reach these only after the C-ABI layer has validated them.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mimo {

// A paged GA pool: position j of sequence b lives in row
// table[b * max_blocks + (j >> shift)] << shift | (j & ((1 << shift) - 1)).
// table == nullptr means the contiguous pool addressed through kv_base.
struct PageTable {
    const int32_t* table = nullptr;
    int max_blocks = 0;
    int shift = 0;
    long long num_pages = 0;
};

struct PrefillArgs {
    const uint16_t* q;
    const uint16_t* k;
    const uint16_t* v;
    const int32_t* cu_seqlens;
    const float* sink;
    uint16_t* out;
    float* lse;
    int num_seqs, max_seqlen, hq, hkv, window;
    float softmax_scale, value_scale;
    bool swa;
    // Chunked prefill only: the caches the sequences continue and their lengths.
    const uint16_t* k_cache = nullptr;
    const uint16_t* v_cache = nullptr;
    const int64_t* kv_base = nullptr;
    const int32_t* ctx_lens = nullptr;
    PageTable pages;
};
hipError_t launch_prefill(const PrefillArgs& a, hipStream_t stream);
hipError_t launch_prefill_chunk(const PrefillArgs& a, hipStream_t stream);

struct DecodeArgs {
    const uint16_t* q;
    const uint16_t* k_new;
    const uint16_t* v_new;
    const uint16_t* k_cache;
    const uint16_t* v_cache;
    const int64_t* kv_base;
    const int32_t* ctx_lens;
    const float* sink;
    uint16_t* out;
    float* lse;
    void* workspace;
    int batch, max_ctx, split, hq, hkv, window;
    float softmax_scale, value_scale;
    PageTable pages;
    // FP8 GA pool (E4M3 codes) and its per-KV-head scales; k_cache/v_cache unused then.
    const uint8_t* k_cache8 = nullptr;
    const uint8_t* v_cache8 = nullptr;
    const float* k_scale = nullptr;
    const float* v_scale = nullptr;
    // Fused append (bf16 ring or contiguous pool): the new token is also written
    // to the cache, SWA ring slot p mod (window-1), GA row kv_base[b] + p when
    // p < kv_capacity[b].  Null: attention only.
    uint16_t* append_k = nullptr;
    uint16_t* append_v = nullptr;
    const int64_t* kv_capacity = nullptr;
};
// Pages a GA split kernel preloads per workgroup (two per lane of a wave).
constexpr int kMaxSplitPages = 128;
// Number of GA splits of `split` keys covering positions 0..max_ctx.
inline int ga_num_splits(int max_ctx, int split) { return (int)(((int64_t)max_ctx + split) / split); }
// Bytes of GA workspace: per (sequence, split, head) an (m, l) pair and 128 partial outputs.
inline size_t ga_workspace_bytes(int batch, int max_ctx, int split, int hq) {
    return (size_t)batch * (size_t)ga_num_splits(max_ctx, split) * (size_t)hq * (2 + 128) * sizeof(float);
}
hipError_t launch_decode_swa(const DecodeArgs& a, hipStream_t stream);
hipError_t launch_decode_ga(const DecodeArgs& a, hipStream_t stream);

struct AppendArgs {
    const uint16_t* k;
    const uint16_t* v;
    const int32_t* cu_newlens;
    const int32_t* ctx_lens;
    uint16_t* k_cache;
    uint16_t* v_cache;
    const int64_t* kv_base;
    const int64_t* kv_capacity;
    int batch, total_new, hkv, window;
    bool swa;
    PageTable pages;
    // FP8 GA pool: new tokens are quantised to E4M3 codes under per-KV-head scales.
    uint8_t* k_cache8 = nullptr;
    uint8_t* v_cache8 = nullptr;
    const float* k_scale = nullptr;
    const float* v_scale = nullptr;
};
hipError_t launch_kv_append(const AppendArgs& a, hipStream_t stream);

struct BackwardArgs {
    const uint16_t* q;
    const uint16_t* k;
    const uint16_t* v;
    const uint16_t* out;
    const float* lse;
    const uint16_t* dout;
    const int32_t* cu_seqlens;
    const float* sink;
    uint16_t* dq;
    uint16_t* dk;
    uint16_t* dv;
    float* dsink;
    void* workspace;  // D = dO . o per (token, head), fp32
    int num_seqs, max_seqlen, total_tokens, hq, hkv, window;
    float softmax_scale, value_scale;
    bool swa;
};
// Bytes of backward workspace: one fp32 per (token, query head).
inline size_t backward_workspace_bytes(int total_tokens, int hq) { return (size_t)total_tokens * hq * sizeof(float); }
hipError_t launch_prefill_backward(const BackwardArgs& a, hipStream_t stream);

struct RopeArgs {
    uint16_t* q;
    uint16_t* k;
    const int32_t* positions;
    int total_tokens, hq, hkv, rotary_dim;
    double theta;
};
hipError_t launch_rope(const RopeArgs& a, hipStream_t stream);

}  // namespace mimo
