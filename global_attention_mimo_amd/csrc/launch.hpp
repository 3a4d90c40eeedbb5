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
    // Fused RoPE: Q is rotated as it is loaded, from the (cos, sin) table of
    // each packed token (rope_half pairs per token); null: no rotation.
    const float* rope_tab = nullptr;
    int rope_half = 0;
    // Chunked prefill only: the caches the sequences continue and their lengths.
    const uint16_t* k_cache = nullptr;
    const uint16_t* v_cache = nullptr;
    const int64_t* kv_base = nullptr;
    const int32_t* ctx_lens = nullptr;
    PageTable pages;
    // Chunked prefill over an FP8 GA pool (E4M3 codes, per-KV-head scales);
    // k_cache/v_cache unused then.
    const uint8_t* k_cache8 = nullptr;
    const uint8_t* v_cache8 = nullptr;
    const float* k_scale = nullptr;
    const float* v_scale = nullptr;
};
hipError_t launch_prefill(const PrefillArgs& a, hipStream_t stream);
hipError_t launch_prefill_chunk(const PrefillArgs& a, hipStream_t stream);

// RoPE frequencies f_i = theta^(-2i/rd), i < rd/2 <= 96, formed on the host
// in double (every rotation in the library uses the same values).
struct RopeFreq {
    double f[96];
};
RopeFreq rope_inv_freq(double theta, int rotary_dim);

// Fused RoPE of a decode step: the queries and the new token's keys of
// sequence b rotate at position pos[b] (half = rotary_dim / 2).
struct DecodeRope {
    const int32_t* pos;
    int half;
    RopeFreq freq;
};

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
    int batch, max_ctx, min_units, hq, hkv, window;
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
    // GA: most chunks the split grid may use (sizes the grid and the workspace).
    int max_chunks = 0;
    // Fused RoPE (with the fused append only): rope.pos null means none.
    DecodeRope rope{};
};

// GA decode work plan.  Sequence b's keys form units: ceil(p_b / 32) tiles of
// 32 pool keys and one unit for the new token, p_b = ctx_lens[b] (0 when
// ctx_lens[b] > max_ctx: such a sequence gets NaN outputs and only its new
// token is touched).  The units of all sequences, in order, are one list of K
// units cut into n balanced chunks, chunk i = units [floor(iK/n),
// floor((i+1)K/n)); one split workgroup takes one chunk.  n is kGaRound (one
// workgroup per compute unit, all resident at once: every extra round of
// chunk start-ups measured slower on the layer stack's decode) when the
// chunks then hold at least min_units units, else ceil(K / min_units).  The
// piece of sequence b inside chunk i writes its partial result to slot i + b,
// so a sequence's partials are consecutive slots and at most n + batch - 1
// slots are used.
constexpr int kTileKeys = 32;
constexpr int kGaRound = 256;      // compute units of a gfx950 part (MI350X / MI355X)
constexpr int kGaMaxRounds = 1;
constexpr int kGaMaxChunks = kGaRound * kGaMaxRounds;
constexpr int kDefaultMinUnits = 8;  // 256 keys
// Pages a paged GA workgroup preloads at a time (two per lane of a wave).
constexpr int kMaxSplitPages = 128;

__host__ __device__ inline long long ga_chunk_count(long long units, int min_units, int max_chunks) {
    const long long by_len = (units + min_units - 1) / min_units;
    long long rounds = units / ((long long)kGaRound * min_units);
    rounds = rounds < 1 ? 1 : (rounds > kGaMaxRounds ? kGaMaxRounds : rounds);
    long long n = by_len < rounds * kGaRound ? by_len : rounds * kGaRound;
    if (n > max_chunks) n = max_chunks;
    return n < 1 ? 1 : n;
}
// Units of a sequence whose new token sits at position p.
__host__ __device__ inline long long ga_seq_units(long long p) { return (p + kTileKeys - 1) / kTileKeys + 1; }
// Split grid for a batch whose contexts are at most max_ctx (chunk counts only
// grow with the unit count, so the device's n never exceeds it).
inline int ga_grid_chunks(int batch, int max_ctx, int min_units, int max_chunks = kGaMaxChunks) {
    return (int)ga_chunk_count((long long)batch * ga_seq_units(max_ctx), min_units, max_chunks);
}
// Workspace: a header of batch + 2 int64 (each sequence's first unit, then K
// and n), padded to 256 bytes, then per slot and query head an (m, l) pair and
// 128 partial outputs, fp32.
inline size_t ga_header_bytes(int batch) { return ((size_t)(batch + 2) * 8 + 255) / 256 * 256; }
inline size_t ga_workspace_bytes(int batch, int chunks, int hq) {
    return ga_header_bytes(batch) + (size_t)(chunks + batch) * (size_t)hq * (2 + 128) * sizeof(float);
}
// Bytes of the per-device scratch array of mimo_attn_decode_noalloc.
constexpr size_t kNoAllocScratchBytes = (size_t)32 << 20;
// The calling thread's current device's address of that array (looked up with
// hipGetSymbolAddress on the first call per device, then cached).
hipError_t noalloc_scratch(void** ptr);
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

// Fused-RoPE prefill preparation: K rotated into k_rot and the (cos, sin)
// table [T][rotary_dim/2][2] fp32 for the Q rotation inside the prefill kernels.
struct RopePrepArgs {
    const uint16_t* k;
    const int32_t* positions;
    uint16_t* k_rot;
    float* tab;
    int total_tokens, hkv, rotary_dim;
    double theta;
};
hipError_t launch_rope_prep(const RopePrepArgs& a, hipStream_t stream);
inline size_t rope_table_bytes(int total_tokens, int rotary_dim) {
    return (size_t)total_tokens * (size_t)(rotary_dim / 2) * 2 * sizeof(float);
}

// Check mode: device-resident preconditions of one call, evaluated by a
// one-pass kernel enqueued ahead of the call's own kernels.  Null pointers and
// negative bounds switch a rule off.  The rules are in check_rules.hpp.
struct CheckArgs {
    const int32_t* cu = nullptr;       // [n_seqs + 1] cu_seqlens / cu_newlens
    int n_seqs = 0;
    int max_len = -1;                  // longest sequence the call allows
    long long total = -1;              // required cu[n_seqs]
    const int32_t* ctx = nullptr;      // [batch] ctx_lens
    int batch = 0;
    int max_ctx = -1;                  // largest ctx_lens[b] allowed
    int new_tokens = 0;                // tokens each sequence appends (cu == null)
    bool new_from_cu = false;          // sequence b appends cu[b+1] - cu[b] tokens
    const int64_t* kv_base = nullptr;  // [batch]
    const int64_t* kv_capacity = nullptr;
    PageTable pages;
    bool pages_cover_new = false;      // block entries of the appended positions (else of positions < ctx)
    const float* sink = nullptr;       // [hq]
    int hq = 0;
    const float* scales = nullptr;     // FP8 per-KV-head scales, k then v: [2][n_scales]
    const float* scales_v = nullptr;
    int n_scales = 0;
};
// Enqueues the check kernel on `stream`.  Unless the stream is capturing a
// graph, waits for it and returns this call's violation bits in *bits with
// *gated = true; under capture *gated = false and the bits only reach the
// device's sticky word.
hipError_t run_check(const CheckArgs& a, hipStream_t stream, bool* gated, uint32_t* bits);
// The current device's sticky word (every violation since it was last cleared).
hipError_t check_flags(uint32_t* bits, bool clear);

}  // namespace mimo
