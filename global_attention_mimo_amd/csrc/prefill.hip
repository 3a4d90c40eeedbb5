// prefill.hip -- sink-biased GQA attention over packed variable-length sequences, SWA or GA.
//
// Operation (Hugging Face Transformers model doc "MiMo-V2-Flash"): Key features
// (5:1 SWA/GA, 128-token window, learnable attention sink bias) and
// MiMoV2FlashConfig (64 query heads over 4 KV heads, head_dim 192 for q/k,
// v_head_dim 128, sliding_window 129 = keys p-128..p, attention_value_scale).
//
// Work decomposition (one workgroup = 4 waves):
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
constexpr int kKStride = kDqk + 8;  // LDS row stride of K tiles (bf16): 400 B, conflict-free b128 reads
constexpr int kVStride = kDv + 16;  // LDS row stride of V tiles (bf16): 288 B, conflict-free tr reads

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

// The running max is only raised when a row's new maximum exceeds it by more
// than this many powers of two; until then exp2(s - m) <= 2^8 stays exact
// enough in fp32 and bf16 and the O/l rescale is skipped.
constexpr float kRescaleThreshold = 8.0f;

template <int WV, int NB, int NK, bool SWA, int WAVES_PER_EU>
__global__ __attribute__((amdgpu_flat_work_group_size(64 * WV, 64 * WV),
                          amdgpu_waves_per_eu(WAVES_PER_EU, WAVES_PER_EU)))
void prefill_kernel(const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
                    const uint16_t* __restrict__ v, const int32_t* __restrict__ cu_seqlens,
                    const float* __restrict__ sink, uint16_t* __restrict__ out, float* __restrict__ lse,
                    int hq, int hkv, int window, float c_log2, float value_scale, int num_qblocks) {
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
    const int L = cu_seqlens[b + 1] - s0;
    const int q0 = qb * QT;
    if (q0 >= L) return;

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
    const int k_lo = SWA ? max(0, q0 - (window - 1)) : 0;
    const int kt_begin = k_lo / NK;
    const int kt_end = q_last / NK;

    // Global -> register staging of one K/V tile.  Each thread always moves the
    // same (row, 16-byte column) slots of a tile, so its source pointers are
    // fixed up to the tile's key offset.  Keys past the sequence end are
    // clamped to its last key: they are masked (key > every query position),
    // so they only need to be finite.
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
    u32x4 kreg[Cfg::kKPer], vreg[Cfg::kVPer];
    auto load_tile = [&](int kt) {
        const int kbase = kt * NK;
        if (kbase + NK <= L) {
#pragma unroll
            for (int i = 0; i < Cfg::kKPer; ++i)
                kreg[i] = *reinterpret_cast<const u32x4*>(kp[i] + (size_t)(kbase + krow_of[i]) * kstride);
#pragma unroll
            for (int i = 0; i < Cfg::kVPer; ++i)
                vreg[i] = *reinterpret_cast<const u32x4*>(vp[i] + (size_t)(kbase + vrow_of[i]) * vstride);
        } else {
#pragma unroll
            for (int i = 0; i < Cfg::kKPer; ++i)
                kreg[i] = *reinterpret_cast<const u32x4*>(kp[i] + (size_t)min(kbase + krow_of[i], L - 1) * kstride);
#pragma unroll
            for (int i = 0; i < Cfg::kVPer; ++i)
                vreg[i] = *reinterpret_cast<const u32x4*>(vp[i] + (size_t)min(kbase + vrow_of[i], L - 1) * vstride);
        }
    };
    auto store_tile = [&](int buf) {
        uint16_t* kb_ = lds_k + buf * Cfg::kLdsK;
        uint16_t* vb_ = lds_v + buf * Cfg::kLdsV;
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
    store_tile(0);
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
        // ---- mask, online softmax, P^T -> bf16, O^T += V^T * P^T -----------------
        const bool interior = (kbase + NK - 1 <= q0) && (!SWA || kbase >= q_last - (window - 1));
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
            // Band/causal mask, only on tiles that cross a boundary: key kk of the
            // tile sits at offset 32*kb + 8*(r/4) + (r%4) + 4*hh; it is kept when
            // tok-(W-1) <= key <= tok (GA: no lower bound).
            if (!interior) {
                const int hi_off = tok[nb] - kbase - 4 * hh;
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
            const float m_cand = fmaxf(m_run[nb], mx * c_log2);
            if (__builtin_amdgcn_ballot_w64(m_cand > m_run[nb] + kRescaleThreshold)) {
                const float alpha = fast_exp2(m_run[nb] - m_cand);
                l_run[nb] *= alpha;
#pragma unroll
                for (int db = 0; db < kDv / 32; ++db) oacc[db][nb] *= alpha;
                m_run[nb] = m_cand;
            }
            const float neg_m = -m_run[nb];
            float rs = 0.0f;
#pragma unroll
            for (int kb = 0; kb < NK / 32; ++kb) {
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const float p = fast_exp2(__builtin_fmaf(sacc[kb][nb][r], c_log2, neg_m));
                    sacc[kb][nb][r] = p;
                    rs += p;
                }
            }
            l_run[nb] += rs;
            bf16x8 pf[NK / 16];
#pragma unroll
            for (int ks = 0; ks < NK / 16; ++ks) {
                const f32x16& sv = sacc[ks >> 1][nb];
                const int o = 8 * (ks & 1);
                pf[ks] = pack_bf16x8(sv[o + 0], sv[o + 1], sv[o + 2], sv[o + 3], sv[o + 4], sv[o + 5], sv[o + 6],
                                     sv[o + 7]);
            }
#pragma unroll
            for (int db = 0; db < kDv / 32; ++db) {
#pragma unroll
                for (int ks = 0; ks < NK / 16; ++ks) {
                    const uint16_t* p = vtile + vsrc_off + ks * 16 * kVStride + db * 32;
                    const bf16x8 a = join_tr(lds_read_tr16(p), lds_read_tr16(p + 8 * kVStride));
                    oacc[db][nb] = mfma_32x32x16(a, pf[ks], oacc[db][nb]);
                }
            }
        }
        if (more) store_tile(buf ^ 1);
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

template <int WV, int NB, int NK, bool SWA, int WPE>
hipError_t launch(const PrefillArgs& a, hipStream_t stream) {
    using Cfg = PrefillCfg<WV, NB, NK>;
    const int nqb = (a.max_seqlen + Cfg::kTokens - 1) / Cfg::kTokens;
    dim3 grid(nqb, a.hkv, a.num_seqs);
    hipLaunchKernelGGL((prefill_kernel<WV, NB, NK, SWA, WPE>), grid, dim3(Cfg::kThreads), 0, stream, a.q, a.k, a.v,
                       a.cu_seqlens, a.sink, a.out, a.lse, a.hq, a.hkv, a.window, a.softmax_scale * kLog2e,
                       a.value_scale, nqb);
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

}  // namespace

hipError_t launch_prefill(const PrefillArgs& a, hipStream_t stream) {
    if (a.max_seqlen <= 0) return hipSuccess;
    if (a.swa) return launch_swa<MIMO_SWA_CFG>(a, stream);
    return launch_ga<MIMO_GA_CFG>(a, stream);
}

}  // namespace mimo
