// prefill.hip -- sink-biased GQA attention over packed variable-length sequences, SWA or GA.
//
// Operation (Hugging Face Transformers model doc "MiMo-V2-Flash"): Key features
// (5:1 SWA/GA, 128-token window, learnable attention sink bias) and
// MiMoV2FlashConfig (64 query heads over 4 KV heads, head_dim 192 for q/k,
// v_head_dim 128, sliding_window 129 = keys p-128..p, attention_value_scale).
//
// Two kernels: the tiled kernel below serves GA and SWA windows wider than
// 145 keys; swa_stream_kernel (further down) serves SWA up to 145 keys.
//
// Tiled kernel, work decomposition (one workgroup = WV waves):
//   * a workgroup owns one (sequence, KV group g, block of QT query tokens);
//     its rows are the QT tokens x the 16 query heads of group g, so the 16
//     heads that share K/V head g form the MFMA N dimension together (GQA
//     packing) and K/V tiles are staged once in LDS for all of them;
//   * each wave owns NB blocks of 32 rows (2 tokens x 16 heads per block);
//   * the key loop walks NK-key tiles from the first tile of the band (SWA:
//     key q0-(W-1)) or 0 (GA) to the tile of the last query token, so SWA
//     tiles outside the 129-key band are never touched;
//   * per tile: S^T = K*Q^T on v_mfma_f32_32x32x16_bf16 (K from LDS, Q held in
//     registers for the whole loop), band/causal mask only on tiles that cross
//     a boundary, online softmax in the exp2 domain seeded with the sink
//     (m = sink*log2e, l = 1), P rounded to bf16, O^T += V^T*P^T with V^T read
//     from the row-major LDS tile by ds_read_b64_tr_b16;
//   * epilogue: O = value_scale * O / l to bf16 (RNE), LSE = (m + log2 l) * ln 2.
#include "device_common.hpp"
#include "launch.hpp"

namespace mimo {
namespace {

constexpr int kDqk = 192;
constexpr int kDv = 128;
constexpr int kGroup = 16;         // query heads per KV head
// LDS row strides (bf16 elements).  K: 400 B, so the 16 rows one
// ds_read_b128 cycle serves start 100 dwords apart and cover all 64 banks
// once.  V: 320 B (80 dwords, 16 mod 64), so the four rows x 2 column groups
// that 32 lanes of a ds_read_b64_tr_b16 address land in disjoint bank ranges
// (a 288-byte stride leaves 2-way conflicts on 24 of 32 lanes).
#ifndef MIMO_KSTRIDE_PAD
#define MIMO_KSTRIDE_PAD 8
#endif
#ifndef MIMO_VSTRIDE_PAD
#define MIMO_VSTRIDE_PAD 32
#endif
constexpr int kKStride = kDqk + MIMO_KSTRIDE_PAD;
constexpr int kVStride = kDv + MIMO_VSTRIDE_PAD;

// Tile shape of one workgroup: WV waves, each owning NB blocks of 32 query
// rows (2 tokens x 16 heads), and NK keys per K/V tile.
template <int WV, int NB, int NK>
struct PrefillCfg {
    static constexpr int kWaves = WV;
    static constexpr int kThreads = 64 * WV;
    static constexpr int kTokens = WV * NB * 2;  // query tokens per workgroup
    static constexpr int kKChunks = NK * (kDqk / 8);  // 16-byte chunks per K tile
    static constexpr int kVChunks = NK * (kDv / 8);
    static constexpr int kKPer = (kKChunks + kThreads - 1) / kThreads;
    static constexpr int kVPer = (kVChunks + kThreads - 1) / kThreads;
    static constexpr int kLdsK = NK * kKStride;  // bf16 elements per K buffer
    static constexpr int kLdsV = NK * kVStride;
    static_assert(NK % 32 == 0, "key tile must be a multiple of 32");
};

// LDS reads issued ahead of the first MFMA of the QK^T and PV runs.
#ifndef MIMO_S_AHEAD
#define MIMO_S_AHEAD 4
#endif
#ifndef MIMO_PV_AHEAD
#define MIMO_PV_AHEAD 4
#endif
#ifndef MIMO_STREAM_S_AHEAD
#define MIMO_STREAM_S_AHEAD 4
#endif
#ifndef MIMO_STREAM_PV_AHEAD
#define MIMO_STREAM_PV_AHEAD 4
#endif

// The running max is only raised (and O, l rescaled) when a row's new maximum
// exceeds it by more than this many powers of two, so most tiles skip the
// rescale.  Kept small on purpose: a key that dominates its row by more than
// the threshold then gets p = exp2(0) = 1, exact in bf16, so rounding P to
// bf16 barely moves the output of a sharp softmax (with 2^8 the dominant p
// could be any value up to 256 and carry a 2^-9 relative error into O).
#ifndef MIMO_RESCALE_THRESHOLD
#define MIMO_RESCALE_THRESHOLD 2.0f
#endif
constexpr float kRescaleThreshold = MIMO_RESCALE_THRESHOLD;

// CHUNK: the sequences continue cached ones.  Sequence b has ctx_lens[b]
// positions in the cache (GA pool rows kv_base[b] + j, SWA ring slots j mod
// ring) and its packed tokens sit at positions ctx_lens[b] + i; a key row is
// staged from the cache below that length and from the chunk above it.
// PAGED (GA chunks only): the pool is paged, position j in row j mod P of page
// block_table[b][j / P] (P = 2^page_shift); each staged row looks its page up.
// FP8 (GA chunks only): the pool holds OCP E4M3 codes (k_cache8, v_cache8)
// with one scale per KV head.  A cached row is loaded as 8 codes per 16-byte
// slot and widened exactly to bf16 when the tile is written to LDS, so the
// MFMAs see the codes' values; the K scale joins the score multiplier and the
// V scale the probabilities of the cached keys (for a tile wholly from the
// cache: exp2 of the shifted exponent, its row sum divided back; for the tile
// that straddles ctx_lens[b]: key by key).
template <int WV, int NB, int NK, bool SWA, int WAVES_PER_EU, bool CHUNK, bool PAGED = false, bool FP8 = false>
__global__ __attribute__((amdgpu_flat_work_group_size(64 * WV, 64 * WV),
                          amdgpu_waves_per_eu(WAVES_PER_EU, WAVES_PER_EU)))
void prefill_kernel(const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
                    const uint16_t* __restrict__ v, const int32_t* __restrict__ cu_seqlens,
                    const float* __restrict__ sink, uint16_t* __restrict__ out, float* __restrict__ lse,
                    int hq, int hkv, int window, float c_log2, float value_scale, int num_qblocks,
                    int max_seqlen, const uint16_t* __restrict__ k_cache, const uint16_t* __restrict__ v_cache,
                    const int64_t* __restrict__ kv_base, const int32_t* __restrict__ ctx_lens, int ring,
                    const int32_t* __restrict__ block_table, int max_blocks, int page_shift, long long num_pages,
                    const float* __restrict__ rope_tab, int rope_half, const uint8_t* __restrict__ k_cache8,
                    const uint8_t* __restrict__ v_cache8, const float* __restrict__ k_scale,
                    const float* __restrict__ v_scale) {
    static_assert(!PAGED || (CHUNK && !SWA), "only GA chunks read a paged pool");
    static_assert(!FP8 || (CHUNK && !SWA), "only GA chunks read an FP8 pool");
    using Cfg = PrefillCfg<WV, NB, NK>;
    constexpr int QT = Cfg::kTokens;
    // Two K/V buffers: tile t is computed from buffer t%2 while tile t+1 is staged into the other.
    __shared__ __attribute__((aligned(16))) uint16_t lds_k[2 * Cfg::kLdsK];
    __shared__ __attribute__((aligned(16))) uint16_t lds_v[2 * Cfg::kLdsV];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int r32 = lane & 31;  // row inside a 32-row block
    const int hh = lane >> 5;   // which half of the MFMA K dimension this lane feeds
    const int b = blockIdx.z;
    const int g = blockIdx.y;
    // GA: heaviest (last) query blocks first so the causal tail does not straggle.
    const int qb = SWA ? (int)blockIdx.x : num_qblocks - 1 - (int)blockIdx.x;
    const int s0 = cu_seqlens[b];
    const int L = min(cu_seqlens[b + 1] - s0, max_seqlen);  // tokens past max_seqlen stay unwritten
    const int q0 = qb * QT;
    if (q0 >= L) return;
    // Position of the first token of the sequence (local token t sits at ctx0 + t).
    const int ctx0 = CHUNK ? ctx_lens[b] : 0;

    const int head = g * kGroup + (r32 & 15);
    int tok[NB];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) tok[nb] = q0 + (wave * NB + nb) * 2 + (r32 >> 4);

    // Q^T fragments (MFMA B operand): lane holds q[row r32][16*s + 8*hh .. +7].
    bf16x8 qf[NB][kDqk / 16];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
        if (tok[nb] < L) {
            const u32x4* src = reinterpret_cast<const u32x4*>(q + ((size_t)(s0 + tok[nb]) * hq + head) * kDqk);
#pragma unroll
            for (int s = 0; s < kDqk / 16; ++s) qf[nb][s] = __builtin_bit_cast(bf16x8, src[2 * s + hh]);
            if (rope_tab) rope_frags_rd(qf[nb], rope_tab + (size_t)(s0 + tok[nb]) * rope_half * 2, rope_half, hh);
        } else {
#pragma unroll
            for (int s = 0; s < kDqk / 16; ++s) qf[nb][s] = __builtin_bit_cast(bf16x8, u32x4{0, 0, 0, 0});
        }
    }

    // Online-softmax state per row (log2 domain).  The sink seeds the running
    // max and contributes exp2(sink - m) = 1 to the sum, counted by the lower
    // half only because the two halves' partial sums are added at the end.
    float m_run[NB], l_run[NB];
    {
        float sl = kNoMax;
        bool has = false;
        if (sink) {
            const float sv = sink[head] * kLog2e;
            if (sv > -__builtin_inff()) { sl = sv; has = true; }
        }
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
            m_run[nb] = has ? sl : kNoMax;
            l_run[nb] = (has && hh == 0) ? 1.0f : 0.0f;
        }
    }
    f32x16 oacc[kDv / 32][NB];
#pragma unroll
    for (int db = 0; db < kDv / 32; ++db)
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) oacc[db][nb] = f32x16{};

    const int q_last = min(q0 + QT, L) - 1;
    // Key tiles cover positions; the block's queries sit at ctx0 + q0 .. ctx0 + q_last.
    const int k_lo = SWA ? max(0, ctx0 + q0 - (window - 1)) : 0;
    const int kt_begin = k_lo / NK;
    const int kt_end = (ctx0 + q_last) / NK;

    // Global -> register staging of one K/V tile.  Each thread always moves the
    // same (row, 16-byte column) slots of a tile, so its source pointers are
    // fixed up to the tile's key offset.  Keys past the sequence end are
    // masked (key > every query position), so they only need to be finite:
    // chunk rows are clamped to the last key, contiguous rows read as zeros.
    const uint16_t* kp[Cfg::kKPer];
    const uint16_t* vp[Cfg::kVPer];
    int krow_of[Cfg::kKPer], vrow_of[Cfg::kVPer];
#pragma unroll
    for (int i = 0; i < Cfg::kKPer; ++i) {
        const int c = min(tid + Cfg::kThreads * i, Cfg::kKChunks - 1);
        krow_of[i] = c / (kDqk / 8);
        kp[i] = k + ((size_t)s0 * hkv + g) * kDqk + (c % (kDqk / 8)) * 8;
    }
#pragma unroll
    for (int i = 0; i < Cfg::kVPer; ++i) {
        const int c = min(tid + Cfg::kThreads * i, Cfg::kVChunks - 1);
        vrow_of[i] = c / (kDv / 8);
        vp[i] = v + ((size_t)s0 * hkv + g) * kDv + (c % (kDv / 8)) * 8;
    }
    const size_t kstride = (size_t)hkv * kDqk, vstride = (size_t)hkv * kDv;
    // Byte offsets of this thread's slots inside a tile (contiguous K/V).
    const uint32_t kRowBytesK = (uint32_t)kstride * 2, kRowBytesV = (uint32_t)vstride * 2;
    uint32_t koff[Cfg::kKPer], voff[Cfg::kVPer];
#pragma unroll
    for (int i = 0; i < Cfg::kKPer; ++i) {
        const int c = min(tid + Cfg::kThreads * i, Cfg::kKChunks - 1);
        koff[i] = (uint32_t)krow_of[i] * kRowBytesK + (c % (kDqk / 8)) * 16;
    }
#pragma unroll
    for (int i = 0; i < Cfg::kVPer; ++i) {
        const int c = min(tid + Cfg::kThreads * i, Cfg::kVChunks - 1);
        voff[i] = (uint32_t)vrow_of[i] * kRowBytesV + (c % (kDv / 8)) * 16;
    }
    // Cache sources (CHUNK only): same per-thread columns, rows by position.
    const uint16_t* kcp[Cfg::kKPer];
    const uint16_t* vcp[Cfg::kVPer];
    int kcol8[Cfg::kKPer], vcol8[Cfg::kVPer];  // FP8: byte offsets of the slots inside a pool row
    int64_t cache_row0 = 0;
    if constexpr (CHUNK && !PAGED) cache_row0 = SWA ? (int64_t)b * ring : kv_base[b];
    if constexpr (CHUNK) {
#pragma unroll
        for (int i = 0; i < Cfg::kKPer; ++i) {
            if constexpr (FP8) kcol8[i] = (int)((kp[i] - k) - (size_t)s0 * kstride);  // one byte per element
            else kcp[i] = k_cache + (kp[i] - k) - (size_t)s0 * kstride;
        }
#pragma unroll
        for (int i = 0; i < Cfg::kVPer; ++i) {
            if constexpr (FP8) vcol8[i] = (int)((vp[i] - v) - (size_t)s0 * vstride);
            else vcp[i] = v_cache + (vp[i] - v) - (size_t)s0 * vstride;
        }
    }
    // FP8: the K scale, and the V scale as a log2 shift and a reciprocal (wave-uniform).
    float k_sc = 1.0f, v_sc = 1.0f, v_lg = 0.0f, v_inv = 1.0f;
    if constexpr (FP8) {
        k_sc = k_scale[g];
        v_sc = v_scale[g];
        v_lg = __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, __log2f(v_sc))));
        v_inv = __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, 1.0f / v_sc)));
    }
    u32x4 kreg[Cfg::kKPer], vreg[Cfg::kVPer];
    u32x2 k8lo[Cfg::kKPer], k8hi[Cfg::kKPer], v8lo[Cfg::kVPer], v8hi[Cfg::kVPer];  // FP8 staging halves
    // PAGED: a tile of NK keys (NK a multiple of 16, kbase a multiple of NK)
    // spans max(1, NK / P) whole pages.  Their numbers come one tile ahead:
    // load_tile(kt) reads tile kt's from `pgv` (lane t holds block kt*NK/P + t)
    // and issues the load of tile kt+1's, so no row load waits on the table.
    constexpr int kTilePages = NK / 16;
    const int32_t* tb = PAGED ? block_table + (size_t)b * max_blocks : nullptr;
    auto fetch_pages = [&](int kt) -> int {
        if constexpr (PAGED) {
            const int blk = ((kt * NK) >> page_shift) + (lane & (kTilePages - 1));
            return tb[min(blk, max_blocks - 1)];
        }
        return 0;
    };
    int pgv = fetch_pages(kt_begin);
    auto load_tile = [&](int kt) {
        const int kbase = kt * NK;
        if constexpr (CHUNK) {
            int pg[kTilePages];
            if constexpr (PAGED) {
                const int blk0 = kbase >> page_shift;
#pragma unroll
                for (int t = 0; t < kTilePages; ++t) {
                    // An unmapped block reads page 0: wrong keys, but inside the pool.
                    const int blk = blk0 + t;
                    const int e = __builtin_amdgcn_readlane(pgv, t);
                    const bool ok = blk < max_blocks && ((long long)blk << page_shift) < ctx0 && e >= 0 &&
                                    e < num_pages;
                    pg[t] = ok ? e : 0;
                }
                pgv = fetch_pages(kt + 1);
            }
            // Cache row of position j < ctx0.
            auto cache_row = [&](int j) -> size_t {
                if constexpr (PAGED) {
                    const int t = ((j - kbase) >> page_shift) & (kTilePages - 1);  // 0 when P >= NK
                    int page = pg[0];
#pragma unroll
                    for (int u = 1; u < kTilePages; ++u) page = t == u ? pg[u] : page;
                    return ((size_t)page << page_shift) | (size_t)(j & ((1 << page_shift) - 1));
                }
                return (size_t)(cache_row0 + (SWA ? j % ring : j));
            };
            if constexpr (FP8) {
                // The low 8 bytes of a slot come from the cache (8 codes) or
                // the chunk (4 bf16) through one select of the address, the
                // high 8 bytes always from the chunk row (for a cached row
                // that is the chunk's first row, unused), so every load lands
                // in its own registers and none waits.  Codes are widened in
                // store_tile.
#pragma unroll
                for (int i = 0; i < Cfg::kKPer; ++i) {
                    const int j = kbase + krow_of[i];
                    const uint16_t* crow = kp[i] + (size_t)min(max(j - ctx0, 0), L - 1) * kstride;
                    const void* lo = j < ctx0 ? static_cast<const void*>(k_cache8 + cache_row(j) * kstride + kcol8[i])
                                              : static_cast<const void*>(crow);
                    k8lo[i] = *reinterpret_cast<const u32x2*>(lo);
                    k8hi[i] = *reinterpret_cast<const u32x2*>(crow + 4);
                }
#pragma unroll
                for (int i = 0; i < Cfg::kVPer; ++i) {
                    const int j = kbase + vrow_of[i];
                    const uint16_t* crow = vp[i] + (size_t)min(max(j - ctx0, 0), L - 1) * vstride;
                    const void* lo = j < ctx0 ? static_cast<const void*>(v_cache8 + cache_row(j) * vstride + vcol8[i])
                                              : static_cast<const void*>(crow);
                    v8lo[i] = *reinterpret_cast<const u32x2*>(lo);
                    v8hi[i] = *reinterpret_cast<const u32x2*>(crow + 4);
                }
            } else {
                // Position j: cache row below ctx0, else chunk row j - ctx0 (past
                // the chunk's last token clamped to it: such keys are masked).
                auto src_row = [&](const uint16_t* cache_col, const uint16_t* chunk_col, size_t stride, int j) {
                    if (j < ctx0) return cache_col + cache_row(j) * stride;
                    return chunk_col + (size_t)min(j - ctx0, L - 1) * stride;
                };
                // GA over the contiguous pool: a tile wholly below ctx0 is a
                // run of pool rows and a tile wholly at or past it a run of chunk
                // rows, so both take the descriptor loads of the plain prefill
                // (chunk rows past the chunk's end read as zeros, and are
                // masked); only the tile across ctx0 picks its rows one by one.
                const bool whole = !SWA && !PAGED && (kbase + NK <= ctx0 || kbase >= ctx0);
                if (whole) {
                    const bool cached = kbase + NK <= ctx0;
                    const size_t row0 = cached ? (size_t)(cache_row0 + kbase) : (size_t)s0 + (kbase - ctx0);
                    const uint32_t rows = cached ? (uint32_t)NK : (uint32_t)max(min(L - (kbase - ctx0), NK), 0);
                    const rsrc_t kr = make_rsrc((cached ? k_cache : k) + (row0 * hkv + g) * kDqk, rows * kRowBytesK);
                    const rsrc_t vr = make_rsrc((cached ? v_cache : v) + (row0 * hkv + g) * kDv, rows * kRowBytesV);
#pragma unroll
                    for (int i = 0; i < Cfg::kKPer; ++i) kreg[i] = __builtin_amdgcn_raw_buffer_load_b128(kr, koff[i], 0, 0);
#pragma unroll
                    for (int i = 0; i < Cfg::kVPer; ++i) vreg[i] = __builtin_amdgcn_raw_buffer_load_b128(vr, voff[i], 0, 0);
                } else {
#pragma unroll
                    for (int i = 0; i < Cfg::kKPer; ++i)
                        kreg[i] = *reinterpret_cast<const u32x4*>(src_row(kcp[i], kp[i], kstride, kbase + krow_of[i]));
#pragma unroll
                    for (int i = 0; i < Cfg::kVPer; ++i)
                        vreg[i] = *reinterpret_cast<const u32x4*>(src_row(vcp[i], vp[i], vstride, kbase + vrow_of[i]));
                }
            }
        } else {
            // The tile's rows through the descriptor: its base and record count
            // (the rows up to the sequence end) are wave-uniform scalars, the
            // per-thread byte offsets fixed, so staging costs no vector address
            // arithmetic.  Rows past the end read as zeros: such keys are masked
            // and their zero values meet zero probabilities.
            const uint32_t rows = (uint32_t)min(L - kbase, NK);
            const rsrc_t kr = make_rsrc(k + ((size_t)(s0 + kbase) * hkv + g) * kDqk, rows * kRowBytesK);
            const rsrc_t vr = make_rsrc(v + ((size_t)(s0 + kbase) * hkv + g) * kDv, rows * kRowBytesV);
#pragma unroll
            for (int i = 0; i < Cfg::kKPer; ++i) kreg[i] = __builtin_amdgcn_raw_buffer_load_b128(kr, koff[i], 0, 0);
#pragma unroll
            for (int i = 0; i < Cfg::kVPer; ++i) vreg[i] = __builtin_amdgcn_raw_buffer_load_b128(vr, voff[i], 0, 0);
        }
    };
    // Writes the staged tile kt to LDS buffer buf (FP8: cached rows widened here).
    auto store_tile = [&](int buf, int kt) {
        uint16_t* kb_ = lds_k + buf * Cfg::kLdsK;
        uint16_t* vb_ = lds_v + buf * Cfg::kLdsV;
        if constexpr (FP8) {
#pragma unroll
            for (int i = 0; i < Cfg::kKPer; ++i)
                kreg[i] = kt * NK + krow_of[i] < ctx0 ? fp8x8_to_bf16x8(k8lo[i][0], k8lo[i][1])
                                                      : u32x4{k8lo[i][0], k8lo[i][1], k8hi[i][0], k8hi[i][1]};
#pragma unroll
            for (int i = 0; i < Cfg::kVPer; ++i)
                vreg[i] = kt * NK + vrow_of[i] < ctx0 ? fp8x8_to_bf16x8(v8lo[i][0], v8lo[i][1])
                                                      : u32x4{v8lo[i][0], v8lo[i][1], v8hi[i][0], v8hi[i][1]};
        }
#pragma unroll
        for (int i = 0; i < Cfg::kKPer; ++i) {
            const int c = tid + Cfg::kThreads * i;
            if (c < Cfg::kKChunks)
                *reinterpret_cast<u32x4*>(kb_ + (c / (kDqk / 8)) * kKStride + (c % (kDqk / 8)) * 8) = kreg[i];
        }
#pragma unroll
        for (int i = 0; i < Cfg::kVPer; ++i) {
            const int c = tid + Cfg::kThreads * i;
            if (c < Cfg::kVChunks)
                *reinterpret_cast<u32x4*>(vb_ + (c / (kDv / 8)) * kVStride + (c % (kDv / 8)) * 8) = vreg[i];
        }
    };

    load_tile(kt_begin);
    store_tile(0, kt_begin);
    __syncthreads();
    // Source address of this lane for the transposed V reads: row 4*hh + (lane%16)/4
    // of a K-step, columns 16*((lane/16)%2) + 4*(lane%4) of a 32-column block.
    const int vsrc_off = (4 * hh + ((lane & 15) >> 2)) * kVStride + 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
    const int ksrc_off = r32 * kKStride + 8 * hh;

    for (int kt = kt_begin; kt <= kt_end; ++kt) {
        const int buf = (kt - kt_begin) & 1;
        const bool more = kt < kt_end;
        if (more) load_tile(kt + 1);  // in flight while this tile is computed
        const uint16_t* ktile = lds_k + buf * Cfg::kLdsK;
        const uint16_t* vtile = lds_v + buf * Cfg::kLdsV;
        const int kbase = kt * NK;

        const bool interior =
            (kbase + NK - 1 <= ctx0 + q0) && (!SWA || kbase >= ctx0 + q_last - (window - 1));

        // ---- S^T = K * Q^T ---------------------------------------------------
        f32x16 sacc[NK / 32][NB];
#pragma unroll
        for (int kb = 0; kb < NK / 32; ++kb) {
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) sacc[kb][nb] = f32x16{};
            const uint16_t* krow = ktile + kb * 32 * kKStride + ksrc_off;
#pragma unroll
            for (int s = 0; s < kDqk / 16; ++s) {
                const bf16x8 a = *reinterpret_cast<const bf16x8*>(krow + 16 * s);
#pragma unroll
                for (int nb = 0; nb < NB; ++nb) sacc[kb][nb] = mfma_32x32x16(a, qf[nb][s], sacc[kb][nb]);
            }
        }
        interleave_lds_mfma<(NK / 32) * (kDqk / 16) * NB, (NK / 32) * (kDqk / 16), MIMO_S_AHEAD, 1>();
        // FP8: keys [kbase, kbase + ncached) of this tile come from the cache.
        // A tile wholly from the cache takes the K scale into its score
        // multiplier and the V scale into its exponent shift; the tile across
        // ctx_lens[b] scales key by key (key of element r at offset
        // 32*kb + 8*(r/4) + (r%4) + 4*hh).
        const int ncached = FP8 ? min(max(ctx0 - kbase, 0), NK) : 0;
        const bool all_cached = FP8 && ncached == NK;
        const bool straddles = FP8 && ncached > 0 && ncached < NK;
        const int ncached_lane = ncached - 4 * hh;  // element r is cached when its tile offset is below this
        const float c_t = all_cached ? c_log2 * k_sc : c_log2;
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
            if (straddles) {
#pragma unroll
                for (int kb = 0; kb < NK / 32; ++kb)
#pragma unroll
                    for (int r = 0; r < 16; ++r)
                        if (kb * 32 + 8 * (r >> 2) + (r & 3) < ncached_lane) sacc[kb][nb][r] *= k_sc;
            }
        }
        // ---- mask, online softmax, P^T -> bf16, O^T += V^T * P^T -----------------
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
            // Band/causal mask, only on tiles that cross a boundary: key kk of the
            // tile sits at offset 32*kb + 8*(r/4) + (r%4) + 4*hh; it is kept when
            // tok-(W-1) <= key <= tok (GA: no lower bound).
            if (!interior) {
                const int hi_off = ctx0 + tok[nb] - kbase - 4 * hh;
                const int lo_off = SWA ? hi_off - (window - 1) : -(1 << 30);
#pragma unroll
                for (int kb = 0; kb < NK / 32; ++kb)
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const int off = kb * 32 + 8 * (r >> 2) + (r & 3);
                        const bool ok = off <= hi_off && off >= lo_off;
                        sacc[kb][nb][r] = ok ? sacc[kb][nb][r] : -__builtin_inff();
                    }
            }
            // Row max over raw scores (c_log2 > 0 preserves order).
            float mx = -__builtin_inff();
#pragma unroll
            for (int kb = 0; kb < NK / 32; ++kb)
#pragma unroll
                for (int r = 0; r < 16; r += 2) mx = fmaxf(mx, fmaxf(sacc[kb][nb][r], sacc[kb][nb][r + 1]));
            mx = max_with_partner_half(mx);
            const float m_cand = fmaxf(m_run[nb], mx * c_t);
            if (__builtin_amdgcn_ballot_w64(m_cand > m_run[nb] + kRescaleThreshold)) {
                const float alpha = fast_exp2(m_run[nb] - m_cand);
                l_run[nb] *= alpha;
#pragma unroll
                for (int db = 0; db < kDv / 32; ++db) oacc[db][nb] *= alpha;
                m_run[nb] = m_cand;
            }
            // all_cached: exp2(s - m + log2 vs) = p * vs, whose sum is divided back by vs.
            const float neg_m = all_cached ? v_lg - m_run[nb] : -m_run[nb];
            float rs = 0.0f;
            if constexpr (!FP8 && NK == 64) {
                // Keys 0..31 first: exps, P^T, then their PV MFMAs with the
                // exps of keys 32..63 placed among them.  Transcendental
                // instructions issue in the shadow of independent MFMAs on this
                // part (FMA-class VALU work does not), and the MFMAs of the first
                // half do not wait for them.  Same operations and order per
                // accumulator and per row sum as the plain form below.
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    sacc[0][nb][r] = fast_exp2(__builtin_fmaf(sacc[0][nb][r], c_t, neg_m));
                    rs += sacc[0][nb][r];
                }
                bf16x8 ph[4];
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    const f32x16& sv = sacc[0][nb];
                    ph[h] = pack_bf16x8(sv[8 * h + 0], sv[8 * h + 1], sv[8 * h + 2], sv[8 * h + 3], sv[8 * h + 4],
                                        sv[8 * h + 5], sv[8 * h + 6], sv[8 * h + 7]);
                }
#pragma unroll
                for (int db = 0; db < kDv / 32; ++db) {
#pragma unroll
                    for (int ks = 0; ks < 2; ++ks) {
                        const uint16_t* p = vtile + vsrc_off + ks * 16 * kVStride + db * 32;
                        const bf16x8 a = join_tr(lds_read_tr16(p), lds_read_tr16(p + 8 * kVStride));
                        oacc[db][nb] = mfma_32x32x16(a, ph[ks], oacc[db][nb]);
                    }
                }
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    sacc[1][nb][r] = fast_exp2(__builtin_fmaf(sacc[1][nb][r], c_t, neg_m));
                    rs += sacc[1][nb][r];
                }
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    const f32x16& sv = sacc[1][nb];
                    ph[2 + h] = pack_bf16x8(sv[8 * h + 0], sv[8 * h + 1], sv[8 * h + 2], sv[8 * h + 3], sv[8 * h + 4],
                                            sv[8 * h + 5], sv[8 * h + 6], sv[8 * h + 7]);
                }
                l_run[nb] += rs;
#pragma unroll
                for (int db = 0; db < kDv / 32; ++db) {
#pragma unroll
                    for (int ks = 2; ks < 4; ++ks) {
                        const uint16_t* p = vtile + vsrc_off + ks * 16 * kVStride + db * 32;
                        const bf16x8 a = join_tr(lds_read_tr16(p), lds_read_tr16(p + 8 * kVStride));
                        oacc[db][nb] = mfma_32x32x16(a, ph[ks], oacc[db][nb]);
                    }
                }
                interleave_pv_trans<kDv / 32 * 2, MIMO_PV_AHEAD>();
                continue;
            }
#pragma unroll
            for (int kb = 0; kb < NK / 32; ++kb)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    sacc[kb][nb][r] = fast_exp2(__builtin_fmaf(sacc[kb][nb][r], c_t, neg_m));
                    rs += sacc[kb][nb][r];
                }
            if (all_cached) rs *= v_inv;
            if (straddles) {
#pragma unroll
                for (int kb = 0; kb < NK / 32; ++kb)
#pragma unroll
                    for (int r = 0; r < 16; ++r)
                        if (kb * 32 + 8 * (r >> 2) + (r & 3) < ncached_lane) sacc[kb][nb][r] *= v_sc;
            }
            bf16x8 pf[NK / 16];
#pragma unroll
            for (int ks = 0; ks < NK / 16; ++ks) {
                const f32x16& sv = sacc[ks >> 1][nb];
                const int o = 8 * (ks & 1);
                pf[ks] = pack_bf16x8(sv[o + 0], sv[o + 1], sv[o + 2], sv[o + 3], sv[o + 4], sv[o + 5], sv[o + 6],
                                     sv[o + 7]);
            }
            l_run[nb] += rs;
#pragma unroll
            for (int db = 0; db < kDv / 32; ++db) {
#pragma unroll
                for (int ks = 0; ks < NK / 16; ++ks) {
                    const uint16_t* p = vtile + vsrc_off + ks * 16 * kVStride + db * 32;
                    const bf16x8 a = join_tr(lds_read_tr16(p), lds_read_tr16(p + 8 * kVStride));
                    oacc[db][nb] = mfma_32x32x16(a, pf[ks], oacc[db][nb]);
                }
            }
            interleave_lds_mfma<(kDv / 32) * (NK / 16), 2 * (kDv / 32) * (NK / 16), MIMO_PV_AHEAD, 2>();
        }
        if (more) store_tile(buf ^ 1, kt + 1);
        __syncthreads();
    }

    // ---- epilogue --------------------------------------------------------------
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
        const float l_tot = sum_with_partner_half(l_run[nb]);
        const int t = tok[nb];
        if (t >= L) continue;
        const float inv = value_scale / l_tot;
        uint16_t* orow = out + ((size_t)(s0 + t) * hq + head) * kDv;
#pragma unroll
        for (int db = 0; db < kDv / 32; ++db) {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const f32x16& ov = oacc[db][nb];
                u32x2 w = {pack_bf16x2(ov[4 * j + 0] * inv, ov[4 * j + 1] * inv),
                           pack_bf16x2(ov[4 * j + 2] * inv, ov[4 * j + 3] * inv)};
                *reinterpret_cast<u32x2*>(orow + db * 32 + 8 * j + 4 * hh) = w;
            }
        }
        if (lse && hh == 0) lse[(size_t)(s0 + t) * hq + head] = (m_run[nb] + __log2f(l_tot)) * kLn2;
    }
}

// ---------------------------------------------------------------------------
// SWA prefill, streaming form (windows up to kStreamMaxWindow).  One
// workgroup of 8 waves walks a strip of consecutive 16-token query blocks of
// one (sequence, KV group); wave w owns tokens q0+2w and q0+2w+1 of the block
// at q0 (x 16 heads = one 32-row MFMA block).  The block sees keys
// q0-(W-1) .. q0+15, covered by five 32-key tiles starting at key q0-144.
// K/V live in an LDS ring of 16-key slots: a block's tiles are ten
// consecutive slots, the next block needs nine of them again, so each block
// stages only the 16 keys the next one adds.  While a block is computed, the
// next block's Q (registers) and its 16 new keys are in flight; one barrier
// per block.  Against the tiled kernel above this removes the per-tile wait
// on global loads and the re-staging of every K/V tile by all 17 query
// blocks that see it.
constexpr int kStreamTokens = 16;   // query tokens per block
constexpr int kSlotKeys = 16;       // keys per ring slot
constexpr int kStreamTiles = 5;     // 32-key tiles per block
constexpr int kStreamLead = 144;    // a block's first tile starts at key q0 - kStreamLead
constexpr int kStreamMaxWindow = kStreamLead + 1;
constexpr int kRingSlots = 2 * kStreamTiles + 1;  // ten in use + the one being staged
constexpr int kSlotKChunks = kSlotKeys * kDqk / 8;  // 16-byte chunks per slot: 384 of K
constexpr int kSlotVChunks = kSlotKeys * kDv / 8;   // 256 of V
constexpr int kStreamThreads = 512;
static_assert(kSlotKChunks % 64 == 0 && kSlotKChunks + kSlotVChunks <= 2 * kStreamThreads &&
                  kSlotKChunks + kSlotVChunks > kStreamThreads && kSlotKChunks < kStreamThreads,
              "slot staging assumes chunk 1 of every thread is K (first 384) or V, chunk 2 is V");

__device__ __forceinline__ int ring_slot(int h) { return (h + kRingSlots * 16) % kRingSlots; }  // h >= -176

// CHUNK: the sequences continue cached ones (ctx_lens[b] positions, the last
// W-1 of them in the ring k_cache/v_cache [B][W-1][Hkv][D]).  Keys are counted
// from the chunk's first token; a key at negative index j is cached position
// ctx_lens[b] + j, staged from the ring instead of as zeros.
// ROPE: each block's Q is rotated before its first score tile, from the
// (cos, sin) pairs of its 16 tokens (rope_tab: the packed tokens' fp32 pairs,
// rope_half per token).  The pairs of the next block are loaded with its Q,
// written to one of two LDS tables at the hand-over, and used after the
// block's closing barrier, so no wave waits for them mid-block.
// The streaming kernel rotates up to 64 dims (one table entry per thread;
// wider rotations go to the tiled kernel, whose Q is loaded once per
// workgroup).
constexpr int kStreamRopeHalf = 32;
constexpr int kRopeEntries = kStreamTokens * kStreamRopeHalf;  // pairs per LDS table
constexpr int kRopePerThread = kRopeEntries / 512;
template <bool CHUNK, bool ROPE = false>
__global__ __attribute__((amdgpu_flat_work_group_size(kStreamThreads, kStreamThreads), amdgpu_waves_per_eu(2, 2)))
void swa_stream_kernel(const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
                       const uint16_t* __restrict__ v, const int32_t* __restrict__ cu_seqlens,
                       const float* __restrict__ sink, uint16_t* __restrict__ out, float* __restrict__ lse,
                       int hq, int hkv, int window, float c_log2, float value_scale, int strip_blocks,
                       int max_seqlen, const uint16_t* __restrict__ k_cache, const uint16_t* __restrict__ v_cache,
                       const int32_t* __restrict__ ctx_lens, const float* __restrict__ rope_tab, int rope_half) {
    __shared__ __attribute__((aligned(16))) uint16_t ring_k[kRingSlots * kSlotKeys * kKStride];
    __shared__ __attribute__((aligned(16))) uint16_t ring_v[kRingSlots * kSlotKeys * kVStride];
    // Threads without a second chunk of their own write it here, so that every
    // load is consumed on every path (no load stays in flight across the loop).
    __shared__ __attribute__((aligned(16))) uint16_t discard[(2 * kStreamThreads - kSlotKChunks - kSlotVChunks) * 8];
    __shared__ __attribute__((aligned(16))) f32x2 rope_lds[ROPE ? 2 * kRopeEntries : 1];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int r32 = lane & 31;
    const int hh = lane >> 5;
    const int b = blockIdx.z;
    const int g = blockIdx.y;
    const int s0 = cu_seqlens[b];
    const int L = min(cu_seqlens[b + 1] - s0, max_seqlen);  // tokens past max_seqlen stay unwritten
    const int ctx0 = CHUNK ? ctx_lens[b] : 0;                // keys from -ctx0 exist
    const int ring = window - 1;
    const int blk_begin = blockIdx.x * strip_blocks;
    const int blk_end = min(blk_begin + strip_blocks, (L + kStreamTokens - 1) / kStreamTokens);
    if (blk_begin >= blk_end) return;
    const int head = g * kGroup + (r32 & 15);
    const int tok_in_blk = 2 * wave + (r32 >> 4);

    // Staging of one 16-key slot: chunk A of this thread is K (threads < 384)
    // or V, chunk B (threads < 128) is V; the split is wave-uniform.  Keys
    // below 0 are staged as zeros, keys past the end repeat the last key
    // (masked either way; they only need to be finite).
    const size_t kstride = (size_t)hkv * kDqk, vstride = (size_t)hkv * kDv;
    const uint16_t* ga_src;
    size_t ga_stride;
    int ga_row;
    uint16_t* la_dst;
    int la_slot;
    if (tid < kSlotKChunks) {
        ga_row = tid / (kDqk / 8);
        ga_src = k + ((size_t)s0 * hkv + g) * kDqk + (tid % (kDqk / 8)) * 8;
        ga_stride = kstride;
        la_dst = ring_k + ga_row * kKStride + (tid % (kDqk / 8)) * 8;
        la_slot = kSlotKeys * kKStride;
    } else {
        const int c = tid - kSlotKChunks;
        ga_row = c / (kDv / 8);
        ga_src = v + ((size_t)s0 * hkv + g) * kDv + (c % (kDv / 8)) * 8;
        ga_stride = vstride;
        la_dst = ring_v + ga_row * kVStride + (c % (kDv / 8)) * 8;
        la_slot = kSlotKeys * kVStride;
    }
    constexpr int kNumB = kSlotKChunks + kSlotVChunks - kStreamThreads;  // threads with a chunk B: 128
    const bool has_b = tid < kNumB;
    const int cb = (kStreamThreads - kSlotKChunks) + (tid % kNumB);  // others re-load a valid V chunk
    const int gb_row = cb / (kDv / 8);
    const uint16_t* gb_src = v + ((size_t)s0 * hkv + g) * kDv + (cb % (kDv / 8)) * 8;
    uint16_t* lb_dst = has_b ? ring_v + gb_row * kVStride + (cb % (kDv / 8)) * 8 : discard + (tid - kNumB) * 8;
    const int lb_slot = has_b ? kSlotKeys * kVStride : 0;

    // Keys below 0 are zeroed at the LDS write, where the loaded value is
    // waited for anyway.
    // Cache sources of the same columns (CHUNK): ring rows of sequence b.
    const uint16_t* ga_cache = nullptr;
    const uint16_t* gb_cache = nullptr;
    if constexpr (CHUNK) {
        ga_cache = (tid < kSlotKChunks ? k_cache : v_cache) + (ga_src - (tid < kSlotKChunks ? k : v)) -
                   (size_t)s0 * ga_stride + (size_t)b * ring * ga_stride;
        gb_cache = v_cache + (gb_src - v) - (size_t)s0 * vstride + (size_t)b * ring * vstride;
    }
    // A slot is all negative keys or all non-negative ones (16 | slot start), so
    // the source choice is uniform per slot.
    auto row_ptr = [&](const uint16_t* chunk, const uint16_t* cache, size_t stride, int j) {
        if (CHUNK && j < 0) return cache + (size_t)(max(ctx0 + j, 0) % ring) * stride;
        return chunk + (size_t)min(max(j, 0), L - 1) * stride;
    };
    auto load_slot = [&](int h, u32x4& ra, u32x4& rb) {
        ra = *reinterpret_cast<const u32x4*>(row_ptr(ga_src, ga_cache, ga_stride, h * kSlotKeys + ga_row));
        rb = *reinterpret_cast<const u32x4*>(row_ptr(gb_src, gb_cache, vstride, h * kSlotKeys + gb_row));
    };
    // Keys before the sequence start are staged as zeros (masked, but finite).
    auto store_slot = [&](int h, const u32x4& ra, const u32x4& rb) {
        const int sl = ring_slot(h);
        const u32x4 zero = {0, 0, 0, 0};
        *reinterpret_cast<u32x4*>(la_dst + sl * la_slot) = ctx0 + h * kSlotKeys + ga_row < 0 ? zero : ra;
        *reinterpret_cast<u32x4*>(lb_dst + sl * lb_slot) = ctx0 + h * kSlotKeys + gb_row < 0 ? zero : rb;
    };
    // Q^T fragments of one block (MFMA B operand); rows past the end repeat the last token.
    auto load_q = [&](int blk, bf16x8 (&qv)[kDqk / 16]) {
        const int t = min(blk * kStreamTokens + tok_in_blk, L - 1);
        const u32x4* src = reinterpret_cast<const u32x4*>(q + ((size_t)(s0 + t) * hq + head) * kDqk);
#pragma unroll
        for (int s = 0; s < kDqk / 16; ++s) qv[s] = __builtin_bit_cast(bf16x8, src[2 * s + hh]);
    };
    // RoPE table entries of one block: thread tid holds entries tid + 512 j
    // (token e / rope_half, pair e % rope_half); entries past the block's
    // 16 * rope_half are loaded clamped and written to unused table places,
    // so every load is consumed on every path.
    auto load_tab = [&](int blk, f32x2 (&tv)[kRopePerThread]) {
#pragma unroll
        for (int j = 0; j < kRopePerThread; ++j) {
            const int e = tid + kStreamThreads * j;
            const int t = min(blk * kStreamTokens + min(e / rope_half, kStreamTokens - 1), L - 1);
            tv[j] = reinterpret_cast<const f32x2*>(rope_tab)[(size_t)(s0 + t) * rope_half + e % rope_half];
        }
    };
    auto store_tab = [&](int blk, const f32x2 (&tv)[kRopePerThread]) {
#pragma unroll
        for (int j = 0; j < kRopePerThread; ++j) rope_lds[(blk & 1) * kRopeEntries + tid + kStreamThreads * j] = tv[j];
    };

    // Outputs of the block at q0 through buffer descriptors that cover only
    // its first `rows` rows: stores of rows past the sequence end are dropped
    // by the hardware range check, so every lane takes the same path.
    auto store_outputs = [&](int q0, int rows, const f32x16 (&oacc)[kDv / 32], float inv, float lse_v) {
        const rsrc_t orsrc = make_rsrc(out + (size_t)(s0 + q0) * hq * kDv, (uint32_t)(rows * hq * kDv * 2));
        const rsrc_t lrsrc =
            lse ? make_rsrc(lse + (size_t)(s0 + q0) * hq, (uint32_t)(rows * hq * 4)) : make_rsrc(lse, 0u);
        const int orow = (tok_in_blk * hq + head) * kDv * 2 + 8 * hh;  // byte offset in the block
#pragma unroll
        for (int db = 0; db < kDv / 32; ++db) {
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
                const f32x16& ov = oacc[db];
                const u32x2 w = {pack_bf16x2(ov[4 * jj + 0] * inv, ov[4 * jj + 1] * inv),
                                 pack_bf16x2(ov[4 * jj + 2] * inv, ov[4 * jj + 3] * inv)};
                __builtin_amdgcn_raw_buffer_store_b64(w, orsrc, orow + (db * 32 + 8 * jj) * 2, 0, 0);
            }
        }
        // One LSE per row: the upper half-wave's copy is sent out of range.
        __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, lse_v), lrsrc,
                                              hh ? (int)0x7ffffff0 : (tok_in_blk * hq + head) * 4, 0, 0);
    };

    float sink_l2 = kNoMax;
    bool has_sink = false;
    if (sink) {
        const float sv = sink[head] * kLog2e;
        if (sv > -__builtin_inff()) { sink_l2 = sv; has_sink = true; }
    }

    // Prologue: the first block's Q and its ten slots.
    bf16x8 qf[kDqk / 16], qn[kDqk / 16];
    u32x4 na, nb;
    f32x2 tn[ROPE ? kRopePerThread : 1];
    load_q(blk_begin, qf);
    if constexpr (ROPE) {
        load_tab(blk_begin, tn);
        store_tab(blk_begin, tn);
    }
    {
        const int h0 = blk_begin * (kStreamTokens / kSlotKeys) - 2 * kStreamTiles + 1;
        u32x4 pa[2 * kStreamTiles], pb[2 * kStreamTiles];
#pragma unroll
        for (int i = 0; i < 2 * kStreamTiles; ++i) load_slot(h0 + i, pa[i], pb[i]);
#pragma unroll
        for (int i = 0; i < 2 * kStreamTiles; ++i) store_slot(h0 + i, pa[i], pb[i]);
    }
    __syncthreads();

    const int vsrc_off = (4 * hh + ((lane & 15) >> 2)) * kVStride + 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
    const int ksrc_off = (r32 & 15) * kKStride + 8 * hh;

    for (int blk = blk_begin; blk < blk_end; ++blk) {
        const int q0 = blk * kStreamTokens;
        const int hq0 = q0 / kSlotKeys;  // slot index of the block's own keys
        if constexpr (ROPE) {
            const float* tab = reinterpret_cast<const float*>(rope_lds + (blk & 1) * kRopeEntries + tok_in_blk * rope_half);
            if (rope_half == 32)
                rope_frags<2>(qf, tab, hh);
            else
                rope_frags<1>(qf, tab, hh);
        }
        // In flight while this block computes: the next block's Q and new slot.
        load_q(min(blk + 1, blk_end - 1), qn);
        load_slot(hq0 + 1, na, nb);
        if constexpr (ROPE) load_tab(min(blk + 1, blk_end - 1), tn);
        const int tok = q0 + tok_in_blk;
        float m_run = has_sink ? sink_l2 : kNoMax;
        float l_run = (has_sink && hh == 0) ? 1.0f : 0.0f;
        f32x16 oacc[kDv / 32];
#pragma unroll
        for (int db = 0; db < kDv / 32; ++db) oacc[db] = f32x16{};

        // QK^T of tile j into acc: 12 MFMAs on K fragments read from the ring.
        auto s_tile = [&](int j, f32x16& acc) {
            const int h = hq0 - 2 * kStreamTiles + 1 + 2 * j;
            const uint16_t* klo = ring_k + ring_slot(h) * (kSlotKeys * kKStride);
            const uint16_t* khi = ring_k + ring_slot(h + 1) * (kSlotKeys * kKStride);
            const uint16_t* krow = (r32 < 16 ? klo : khi) + ksrc_off;
            acc = f32x16{};
#pragma unroll
            for (int s = 0; s < kDqk / 16; ++s)
                acc = mfma_32x32x16(*reinterpret_cast<const bf16x8*>(krow + 16 * s), qf[s], acc);
        };
        // Pipelined (the plain kernel): tile j+1's QK^T is issued between the
        // exps of tile j (one MFMA, one K read and five VALU instructions at a
        // time), so the matrix core works while the wave runs tile j's
        // softmax.  The chunked kernel, whose cache addressing leaves no room
        // for the second score tile (it spilled, 4% slower), issues each
        // tile's QK^T at the top of its own step.  Tiles wholly outside the
        // band (only near a sequence's start) are computed and masked: their
        // slots hold zeros or earlier keys, so every score is finite.
        constexpr bool kPipe = !CHUNK;
        f32x16 sa, sb;
        if constexpr (kPipe) {
            s_tile(0, sa);
            interleave_lds_mfma<kDqk / 16, kDqk / 16, MIMO_STREAM_S_AHEAD, 1>();
        }
#pragma unroll
        for (int j = 0; j < kStreamTiles; ++j) {
            f32x16& sacc = (kPipe && (j & 1)) ? sb : sa;
            f32x16& snext = (j & 1) ? sa : sb;
            if constexpr (!kPipe) {
                s_tile(j, sacc);
                interleave_lds_mfma<kDqk / 16, kDqk / 16, MIMO_STREAM_S_AHEAD, 1>();
            }
            const int kbase = q0 - kStreamLead + 32 * j;
            const int h = hq0 - 2 * kStreamTiles + 1 + 2 * j;

            // Mask unless every key of the tile is in every token's band: key
            // offset 8*(r/4) + (r%4) + 4*hh is kept when max(0, tok-(W-1)) <= key <= tok.
            const bool interior =
                kbase >= -ctx0 && kbase + 31 <= q0 && kbase >= q0 + kStreamTokens - 1 - (window - 1);
            if (!interior) {
                const int hi_off = tok - kbase - 4 * hh;
                const int lo_off = max(hi_off - (window - 1), -ctx0 - kbase - 4 * hh);
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int off = 8 * (r >> 2) + (r & 3);
                    const bool ok = off <= hi_off && off >= lo_off;
                    sacc[r] = ok ? sacc[r] : -__builtin_inff();
                }
            }
            float mx = -__builtin_inff();
#pragma unroll
            for (int r = 0; r < 16; r += 2) mx = fmaxf(mx, fmaxf(sacc[r], sacc[r + 1]));
            mx = max_with_partner_half(mx);
            const float m_cand = fmaxf(m_run, mx * c_log2);
            if (__builtin_amdgcn_ballot_w64(m_cand > m_run + kRescaleThreshold)) {
                const float alpha = fast_exp2(m_run - m_cand);
                l_run *= alpha;
#pragma unroll
                for (int db = 0; db < kDv / 32; ++db) oacc[db] *= alpha;
                m_run = m_cand;
            }
            const float neg_m = -m_run;
            if (kPipe && j + 1 < kStreamTiles) s_tile(j + 1, snext);
            float rs = 0.0f;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                sacc[r] = fast_exp2(__builtin_fmaf(sacc[r], c_log2, neg_m));
                rs += sacc[r];
            }
            const bf16x8 p0 = pack_bf16x8(sacc[0], sacc[1], sacc[2], sacc[3], sacc[4], sacc[5], sacc[6], sacc[7]);
            const bf16x8 p1 =
                pack_bf16x8(sacc[8], sacc[9], sacc[10], sacc[11], sacc[12], sacc[13], sacc[14], sacc[15]);
            if (kPipe && j + 1 < kStreamTiles) interleave_mfma_valu<kDqk / 16, kDqk / 16, MIMO_STREAM_S_AHEAD, 5>();
            l_run += rs;
            const uint16_t* vlo = ring_v + ring_slot(h) * (kSlotKeys * kVStride) + vsrc_off;
            const uint16_t* vhi = ring_v + ring_slot(h + 1) * (kSlotKeys * kVStride) + vsrc_off;
#pragma unroll
            for (int db = 0; db < kDv / 32; ++db) {
                const bf16x8 a0 = join_tr(lds_read_tr16(vlo + db * 32), lds_read_tr16(vlo + db * 32 + 8 * kVStride));
                oacc[db] = mfma_32x32x16(a0, p0, oacc[db]);
                const bf16x8 a1 = join_tr(lds_read_tr16(vhi + db * 32), lds_read_tr16(vhi + db * 32 + 8 * kVStride));
                oacc[db] = mfma_32x32x16(a1, p1, oacc[db]);
            }
            interleave_lds_mfma<2 * (kDv / 32), 4 * (kDv / 32), MIMO_STREAM_PV_AHEAD, 2>();
        }

        // Hand-over before this block's output stores (so that waiting for the
        // loads does not also wait for the stores): the next block's slot goes
        // to LDS, replacing key block hq0+1-11, which no block from here on
        // reads, and its Q to qf.
        store_slot(hq0 + 1, na, nb);
        if constexpr (ROPE) store_tab(blk + 1, tn);
#pragma unroll
        for (int s = 0; s < kDqk / 16; ++s) {
            qf[s] = qn[s];
            // Materialise the copy here (an empty asm that claims to modify the
            // register) so that it, and the wait for the Q loads, cannot be
            // deferred past the stores below.
            asm volatile("" : "+v"(qf[s]));
        }

        const float l_tot = sum_with_partner_half(l_run);
        const int rows = min(kStreamTokens, L - q0);
        store_outputs(q0, rows, oacc, value_scale / l_tot, (m_run + __log2f(l_tot)) * kLn2);
        __syncthreads();
    }
}

template <int WV, int NB, int NK, bool SWA, int WPE, bool CHUNK = false, bool PAGED = false, bool FP8 = false>
hipError_t launch(const PrefillArgs& a, hipStream_t stream) {
    using Cfg = PrefillCfg<WV, NB, NK>;
    const int nqb = (a.max_seqlen + Cfg::kTokens - 1) / Cfg::kTokens;
    dim3 grid(nqb, a.hkv, a.num_seqs);
    hipLaunchKernelGGL((prefill_kernel<WV, NB, NK, SWA, WPE, CHUNK, PAGED, FP8>), grid, dim3(Cfg::kThreads), 0,
                       stream, a.q, a.k, a.v, a.cu_seqlens, a.sink, a.out, a.lse, a.hq, a.hkv, a.window,
                       a.softmax_scale * kLog2e, a.value_scale, nqb, a.max_seqlen, a.k_cache, a.v_cache, a.kv_base,
                       a.ctx_lens, a.window - 1, a.pages.table, a.pages.max_blocks, a.pages.shift,
                       a.pages.num_pages, a.rope_tab, a.rope_half, a.k_cache8, a.v_cache8, a.k_scale, a.v_scale);
    return hipGetLastError();
}

// Tile configurations (waves per workgroup, 32-row blocks per wave, keys per
// tile, waves per SIMD), overridable at build time for tuning sweeps.
#ifndef MIMO_GA_CFG
#define MIMO_GA_CFG 8, 1, 64, 2
#endif
#ifndef MIMO_SWA_CFG
#define MIMO_SWA_CFG 4, 1, 32, 2
#endif

template <int WV, int NB, int NK, int WPE>
hipError_t launch_ga(const PrefillArgs& a, hipStream_t s) { return launch<WV, NB, NK, false, WPE>(a, s); }
template <int WV, int NB, int NK, int WPE>
hipError_t launch_swa(const PrefillArgs& a, hipStream_t s) { return launch<WV, NB, NK, true, WPE>(a, s); }
template <int WV, int NB, int NK, int WPE>
hipError_t launch_ga_chunk(const PrefillArgs& a, hipStream_t s) {
    if (a.k_cache8) {
        if (a.pages.table) return launch<WV, NB, NK, false, WPE, true, true, true>(a, s);
        return launch<WV, NB, NK, false, WPE, true, false, true>(a, s);
    }
    if (a.pages.table) return launch<WV, NB, NK, false, WPE, true, true>(a, s);
    return launch<WV, NB, NK, false, WPE, true>(a, s);
}
template <int WV, int NB, int NK, int WPE>
hipError_t launch_swa_chunk(const PrefillArgs& a, hipStream_t s) { return launch<WV, NB, NK, true, WPE, true>(a, s); }

// Streaming SWA grid: strips per compute unit it aims for (one workgroup fits
// a CU), and the longest strip.  The cap keeps ragged batches balanced: the
// host sizes strips from max_seqlen, not from the actual lengths.
#ifndef MIMO_STREAM_ROUNDS
#define MIMO_STREAM_ROUNDS 1
#endif
#ifndef MIMO_STREAM_MAX_STRIP
#define MIMO_STREAM_MAX_STRIP 32
#endif

template <bool CHUNK>
hipError_t launch_swa_stream(const PrefillArgs& a, hipStream_t stream) {
    int dev = 0, cus = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return e;
    // Strip length: spread the (upper bound of the) query blocks over the CUs.
    const long long per_seq = (a.max_seqlen + kStreamTokens - 1) / kStreamTokens;
    const long long total = per_seq * a.hkv * a.num_seqs;
    const long long target = (long long)max(cus, 1) * MIMO_STREAM_ROUNDS;
    const int strip = (int)max(1LL, min(min(per_seq, (long long)MIMO_STREAM_MAX_STRIP), (total + target - 1) / target));
    dim3 grid((unsigned)((per_seq + strip - 1) / strip), a.hkv, a.num_seqs);
    auto kern = a.rope_tab ? swa_stream_kernel<CHUNK, true> : swa_stream_kernel<CHUNK, false>;
    hipLaunchKernelGGL(kern, grid, dim3(kStreamThreads), 0, stream, a.q, a.k, a.v, a.cu_seqlens,
                       a.sink, a.out, a.lse, a.hq, a.hkv, a.window, a.softmax_scale * kLog2e, a.value_scale, strip,
                       a.max_seqlen, a.k_cache, a.v_cache, a.ctx_lens, a.rope_tab, a.rope_half);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_prefill_chunk(const PrefillArgs& a, hipStream_t stream) {
    if (a.max_seqlen <= 0) return hipSuccess;
    if (a.swa && a.window <= kStreamMaxWindow && (!a.rope_tab || a.rope_half <= kStreamRopeHalf))
        return launch_swa_stream<true>(a, stream);
    if (a.swa) return launch_swa_chunk<MIMO_SWA_CFG>(a, stream);
    return launch_ga_chunk<MIMO_GA_CFG>(a, stream);
}

hipError_t launch_prefill(const PrefillArgs& a, hipStream_t stream) {
    if (a.max_seqlen <= 0) return hipSuccess;
    if (a.swa && a.window <= kStreamMaxWindow && (!a.rope_tab || a.rope_half <= kStreamRopeHalf))
        return launch_swa_stream<false>(a, stream);
    if (a.swa) return launch_swa<MIMO_SWA_CFG>(a, stream);
    return launch_ga<MIMO_GA_CFG>(a, stream);
}

}  // namespace mimo
