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

template <int NB, int NK, bool SWA>
struct PrefillCfg {
    static constexpr int kWaves = 4;
    static constexpr int kThreads = 64 * kWaves;
    static constexpr int kRowsPerWave = 32 * NB;
    static constexpr int kTokens = kWaves * kRowsPerWave / kGroup;  // query tokens per workgroup
    static constexpr int kKChunks = NK * (kDqk / 8) / kThreads;      // 16-byte chunks per thread
    static constexpr int kVChunks = NK * (kDv / 8) / kThreads;
    static_assert(NK % 32 == 0, "key tile must be a multiple of 32");
    static_assert(NK * (kDqk / 8) % kThreads == 0 && NK * (kDv / 8) % kThreads == 0, "tile/thread mismatch");
};

template <int NB, int NK, bool SWA, int WAVES_PER_EU>
__global__ __attribute__((amdgpu_flat_work_group_size(256, 256), amdgpu_waves_per_eu(WAVES_PER_EU, WAVES_PER_EU)))
void prefill_kernel(const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
                    const uint16_t* __restrict__ v, const int32_t* __restrict__ cu_seqlens,
                    const float* __restrict__ sink, uint16_t* __restrict__ out, float* __restrict__ lse,
                    int hq, int hkv, int window, float c_log2, float value_scale, int num_qblocks) {
    using Cfg = PrefillCfg<NB, NK, SWA>;
    constexpr int QT = Cfg::kTokens;
    __shared__ __attribute__((aligned(16))) uint16_t lds_k[NK * kKStride];
    __shared__ __attribute__((aligned(16))) uint16_t lds_v[NK * kVStride];

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

    // Global -> register staging of one K/V tile (zero rows past the sequence end).
    u32x4 kreg[Cfg::kKChunks], vreg[Cfg::kVChunks];
    auto load_tile = [&](int kt) {
        const int kbase = kt * NK;
#pragma unroll
        for (int i = 0; i < Cfg::kKChunks; ++i) {
            const int c = tid + Cfg::kThreads * i;
            const int row = c / (kDqk / 8), col = c % (kDqk / 8);
            const int key = kbase + row;
            kreg[i] = key < L ? reinterpret_cast<const u32x4*>(k + ((size_t)(s0 + key) * hkv + g) * kDqk)[col]
                              : u32x4{0, 0, 0, 0};
        }
#pragma unroll
        for (int i = 0; i < Cfg::kVChunks; ++i) {
            const int c = tid + Cfg::kThreads * i;
            const int row = c / (kDv / 8), col = c % (kDv / 8);
            const int key = kbase + row;
            vreg[i] = key < L ? reinterpret_cast<const u32x4*>(v + ((size_t)(s0 + key) * hkv + g) * kDv)[col]
                              : u32x4{0, 0, 0, 0};
        }
    };
    auto store_tile = [&]() {
#pragma unroll
        for (int i = 0; i < Cfg::kKChunks; ++i) {
            const int c = tid + Cfg::kThreads * i;
            const int row = c / (kDqk / 8), col = c % (kDqk / 8);
            *reinterpret_cast<u32x4*>(lds_k + row * kKStride + col * 8) = kreg[i];
        }
#pragma unroll
        for (int i = 0; i < Cfg::kVChunks; ++i) {
            const int c = tid + Cfg::kThreads * i;
            const int row = c / (kDv / 8), col = c % (kDv / 8);
            *reinterpret_cast<u32x4*>(lds_v + row * kVStride + col * 8) = vreg[i];
        }
    };

    load_tile(kt_begin);
    for (int kt = kt_begin; kt <= kt_end; ++kt) {
        __syncthreads();  // every wave is done reading the previous tile
        store_tile();
        __syncthreads();
        if (kt < kt_end) load_tile(kt + 1);  // in flight while this tile is computed

        const int kbase = kt * NK;
        // ---- S^T = K * Q^T ---------------------------------------------------
        f32x16 sacc[NK / 32][NB];
#pragma unroll
        for (int kb = 0; kb < NK / 32; ++kb) {
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) sacc[kb][nb] = f32x16{};
            const uint16_t* krow = lds_k + (kb * 32 + r32) * kKStride + 8 * hh;
#pragma unroll
            for (int s = 0; s < kDqk / 16; ++s) {
                const bf16x8 a = *reinterpret_cast<const bf16x8*>(krow + 16 * s);
#pragma unroll
                for (int nb = 0; nb < NB; ++nb) sacc[kb][nb] = mfma_32x32x16(a, qf[nb][s], sacc[kb][nb]);
            }
        }
        // ---- mask, online softmax --------------------------------------------
        const bool interior = (kbase + NK - 1 <= q0) && (!SWA || kbase >= q_last - (window - 1));
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
            float mx = -__builtin_inff();
#pragma unroll
            for (int kb = 0; kb < NK / 32; ++kb) {
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    float s = sacc[kb][nb][r] * c_log2;
                    if (!interior) {
                        const int key = kbase + kb * 32 + 8 * (r >> 2) + 4 * hh + (r & 3);
                        const bool ok = key <= tok[nb] && (!SWA || key >= tok[nb] - (window - 1));
                        s = ok ? s : -__builtin_inff();
                    }
                    sacc[kb][nb][r] = s;
                    mx = fmaxf(mx, s);
                }
            }
            mx = max_with_partner_half(mx);
            const float m_new = fmaxf(m_run[nb], mx);
            const float alpha = fast_exp2(m_run[nb] - m_new);
            float rs = 0.0f;
#pragma unroll
            for (int kb = 0; kb < NK / 32; ++kb) {
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const float p = fast_exp2(sacc[kb][nb][r] - m_new);
                    sacc[kb][nb][r] = p;
                    rs += p;
                }
            }
            l_run[nb] = l_run[nb] * alpha + rs;
            m_run[nb] = m_new;
#pragma unroll
            for (int db = 0; db < kDv / 32; ++db) oacc[db][nb] *= alpha;
        }
        // ---- O^T += V^T * P^T ------------------------------------------------
        bf16x8 pf[NK / 16][NB];
#pragma unroll
        for (int ks = 0; ks < NK / 16; ++ks)
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) {
                const f32x16& sv = sacc[ks >> 1][nb];
                const int o = 8 * (ks & 1);
                pf[ks][nb] = pack_bf16x8(sv[o + 0], sv[o + 1], sv[o + 2], sv[o + 3], sv[o + 4], sv[o + 5],
                                         sv[o + 6], sv[o + 7]);
            }
        // Source address of this lane for the transposed V reads: row 4*hh + (lane%16)/4
        // of the K-step, columns 16*((lane/16)%2) + 4*(lane%4) of the 32-column block.
        const uint16_t* vsrc = lds_v + (4 * hh + ((lane & 15) >> 2)) * kVStride + 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
#pragma unroll
        for (int db = 0; db < kDv / 32; ++db) {
#pragma unroll
            for (int ks = 0; ks < NK / 16; ++ks) {
                const uint16_t* p = vsrc + ks * 16 * kVStride + db * 32;
                const bf16x8 a = join_tr(lds_read_tr16(p), lds_read_tr16(p + 8 * kVStride));
#pragma unroll
                for (int nb = 0; nb < NB; ++nb) oacc[db][nb] = mfma_32x32x16(a, pf[ks][nb], oacc[db][nb]);
            }
        }
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

template <int NB, int NK, bool SWA, int WPE>
hipError_t launch(const PrefillArgs& a, hipStream_t stream) {
    using Cfg = PrefillCfg<NB, NK, SWA>;
    const int nqb = (a.max_seqlen + Cfg::kTokens - 1) / Cfg::kTokens;
    dim3 grid(nqb, a.hkv, a.num_seqs);
    hipLaunchKernelGGL((prefill_kernel<NB, NK, SWA, WPE>), grid, dim3(Cfg::kThreads), 0, stream, a.q, a.k, a.v,
                       a.cu_seqlens, a.sink, a.out, a.lse, a.hq, a.hkv, a.window, a.softmax_scale * kLog2e,
                       a.value_scale, nqb);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_prefill(const PrefillArgs& a, hipStream_t stream) {
    if (a.max_seqlen <= 0) return hipSuccess;
    if (a.swa) return launch<2, 32, true, 1>(a, stream);
    return launch<2, 32, false, 1>(a, stream);
}

}  // namespace mimo
