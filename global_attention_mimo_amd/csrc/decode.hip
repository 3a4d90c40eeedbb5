// decode.hip -- attention of one new token per sequence over its KV cache, SWA and GA.
//
// Operation (Hugging Face Transformers model doc "MiMo-V2-Flash"): with
// past_key_values only the unprocessed token is passed and earlier keys come
// from the cache (MiMoV2FlashModel.forward); SWA layers see keys p-128..p
// (sliding_window 129), GA layers all keys 0..p; a learnable attention sink
// joins each softmax denominator (Key features); 64 query heads share 4 KV
// heads, head_dim 192 for q/k and 128 for v (MiMoV2FlashConfig).
//
// Shared building block: one wave attends the 16 query heads of one KV group
// (GQA packing into the MFMA N dimension) over a 32-key tile with
// v_mfma_f32_16x16x32_bf16: S^T = K*Q^T with K fragments loaded straight from
// HBM into registers (16 B per lane), then an online softmax whose row
// reductions cross only the four 16-lane groups, then O^T += V^T*P^T where the
// V tile is written row-major to wave-private LDS and read transposed with
// ds_read_b64_tr_b16.  The next tile's loads are issued before the current
// tile is computed.
//
// SWA decode (one workgroup per (sequence, KV group)): the 128 ring slots plus
// the new token are 129 "virtual keys" in 32-key tiles spread over the 4
// waves, so every load of the window is issued at once; the waves' partial
// (m, l, O) are merged in LDS together with the sink.
//
// GA decode: split-K.  Workgroup (split s, sequence b) covers keys
// [s*C, (s+1)*C) of the sequence with one wave per KV group, streaming the
// pool rows (each 384 B of K and 256 B of V) and writing an unnormalised
// partial (m, l, O) without the sink.  A second kernel merges the splits of
// each (sequence, head), adds the sink exactly once, and writes O and LSE.
#include "device_common.hpp"
#include "launch.hpp"

namespace mimo {
namespace {

constexpr int kDqk = 192;
constexpr int kDv = 128;
constexpr int kGroup = 16;
constexpr int kTile = 32;              // keys per wave tile
constexpr int kVStride = kDv + 16;     // LDS row stride (bf16) of a V tile: 288 B
constexpr int kWaveLds = kTile * kVStride;

// Per-wave running state for 16 heads.  Lane l owns head (l % 16); o[db][r]
// is O^T[dv = 16*db + 4*(l/16) + r][head]; m is the same in the 4 lanes of a
// head, l is a per-lane partial sum (the 4 partials add up at the end).
struct WaveAcc {
    f32x4 o[kDv / 16];
    float m, l;
};

struct TileRegs {
    u32x4 k[2 * (kDqk / 32)];  // K rows (16*blk + lane%16), 16 B chunk 4*st + lane/16
    u32x4 v[kTile * (kDv / 8) / 64];  // V rows (lane/16 + 4*i), 16 B chunk lane%16
};

// Loads the K/V rows of tile keys j0..j0+31 into registers.  src.krow(j) and
// src.vrow(j) give row pointers, or nullptr for keys outside the key set
// (their registers are zero).
template <class Src>
__device__ __forceinline__ void load_tile(TileRegs& t, const Src& src, int j0, int lane) {
    const int G = lane >> 4;
#pragma unroll
    for (int blk = 0; blk < 2; ++blk) {
        const uint16_t* kp = src.krow(j0 + 16 * blk + (lane & 15));
#pragma unroll
        for (int st = 0; st < kDqk / 32; ++st)
            t.k[blk * (kDqk / 32) + st] = kp ? reinterpret_cast<const u32x4*>(kp)[4 * st + G] : u32x4{0, 0, 0, 0};
    }
#pragma unroll
    for (int i = 0; i < kTile * (kDv / 8) / 64; ++i) {
        const uint16_t* vp = src.vrow(j0 + G + 4 * i);
        t.v[i] = vp ? reinterpret_cast<const u32x4*>(vp)[lane & 15] : u32x4{0, 0, 0, 0};
    }
}

template <class Src>
__device__ __forceinline__ void attend_tile(WaveAcc& acc, const bf16x8 (&qf)[kDqk / 32], const TileRegs& t,
                                            uint16_t* lds_v, const Src& src, int j0, float c_log2, int lane) {
    const int G = lane >> 4;
    // V rows to wave-private LDS, row-major.
#pragma unroll
    for (int i = 0; i < kTile * (kDv / 8) / 64; ++i)
        *reinterpret_cast<u32x4*>(lds_v + (G + 4 * i) * kVStride + (lane & 15) * 8) = t.v[i];
    wave_lds_fence();

    f32x4 s[2] = {f32x4{}, f32x4{}};
#pragma unroll
    for (int blk = 0; blk < 2; ++blk)
#pragma unroll
        for (int st = 0; st < kDqk / 32; ++st)
            s[blk] = mfma_16x16x32(__builtin_bit_cast(bf16x8, t.k[blk * (kDqk / 32) + st]), qf[st], s[blk]);

    float mx = -__builtin_inff();
#pragma unroll
    for (int blk = 0; blk < 2; ++blk)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const bool ok = src.valid(j0 + 16 * blk + 4 * G + r);
            const float x = ok ? s[blk][r] * c_log2 : -__builtin_inff();
            s[blk][r] = x;
            mx = fmaxf(mx, x);
        }
    mx = fmaxf(mx, __shfl_xor(mx, 16));
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float m_new = fmaxf(acc.m, mx);
    const float alpha = fast_exp2(acc.m - m_new);
    float rs = 0.0f;
#pragma unroll
    for (int blk = 0; blk < 2; ++blk)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const float p = fast_exp2(s[blk][r] - m_new);
            s[blk][r] = p;
            rs += p;
        }
    acc.l = acc.l * alpha + rs;
    acc.m = m_new;
    // P^T as the B operand: position 8*G + t holds key 4*G + t (t < 4) or 16 + 4*G + t - 4.
    const bf16x8 pf = pack_bf16x8(s[0][0], s[0][1], s[0][2], s[0][3], s[1][0], s[1][1], s[1][2], s[1][3]);
    const uint16_t* vsrc = lds_v + (4 * G + ((lane & 15) >> 2)) * kVStride + 4 * (lane & 3);
#pragma unroll
    for (int db = 0; db < kDv / 16; ++db) {
        const uint16_t* p = vsrc + 16 * db;
        const bf16x8 a = join_tr(lds_read_tr16(p), lds_read_tr16(p + 16 * kVStride));
        acc.o[db] = mfma_16x16x32(a, pf, acc.o[db] * alpha);
    }
    wave_lds_fence();  // the next tile's V writes come after these reads
}

// Q^T fragments of the 16 heads of group g for batch row b: lane holds
// q[b][16*g + lane%16][32*st + 8*(lane/16) .. +7].
__device__ __forceinline__ void load_q(bf16x8 (&qf)[kDqk / 32], const uint16_t* q, int b, int g, int hq, int lane) {
    const u32x4* src = reinterpret_cast<const u32x4*>(q + ((size_t)b * hq + g * kGroup + (lane & 15)) * kDqk);
#pragma unroll
    for (int st = 0; st < kDqk / 32; ++st) qf[st] = __builtin_bit_cast(bf16x8, src[4 * st + (lane >> 4)]);
}

__device__ __forceinline__ void acc_init(WaveAcc& acc) {
#pragma unroll
    for (int db = 0; db < kDv / 16; ++db) acc.o[db] = f32x4{};
    acc.m = kNoMax;
    acc.l = 0.0f;
}

// Runs tiles j0 = first, first + stride, ... < end with one tile of loads in flight.
template <class Src>
__device__ __forceinline__ void run_tiles(WaveAcc& acc, const bf16x8 (&qf)[kDqk / 32], uint16_t* lds_v,
                                          const Src& src, int first, int stride, int end, float c_log2,
                                          int lane) {
    if (first >= end) return;
    TileRegs cur, nxt;
    load_tile(cur, src, first, lane);
    for (int j0 = first; j0 < end; j0 += stride) {
        const bool more = j0 + stride < end;
        if (more) load_tile(nxt, src, j0 + stride, lane);
        attend_tile(acc, qf, cur, lds_v, src, j0, c_log2, lane);
        if (more) cur = nxt;
    }
}

// ---------------------------------------------------------------------------
// SWA: virtual key j < R is ring slot j, virtual key R is the new token.
struct SwaSource {
    const uint16_t* ring_k;  // this sequence's ring, group g already applied
    const uint16_t* ring_v;
    const uint16_t* new_k;
    const uint16_t* new_v;
    int R, p, hkv;
    // Slot j holds position p-R+((j-p) mod R); it is in the window unless that
    // position is negative, i.e. unless p < R and j >= p.
    __device__ bool valid(int j) const { return j < R ? (p >= R || j < p) : j == R; }
    __device__ const uint16_t* krow(int j) const {
        if (!valid(j)) return nullptr;
        return j == R ? new_k : ring_k + (size_t)j * hkv * kDqk;
    }
    __device__ const uint16_t* vrow(int j) const {
        if (!valid(j)) return nullptr;
        return j == R ? new_v : ring_v + (size_t)j * hkv * kDv;
    }
};

__global__ __launch_bounds__(256) void swa_decode_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k_new, const uint16_t* __restrict__ v_new,
    const uint16_t* __restrict__ ring_k, const uint16_t* __restrict__ ring_v, const int32_t* __restrict__ ctx_lens,
    const float* __restrict__ sink, uint16_t* __restrict__ out, float* __restrict__ lse, int hq, int hkv, int R,
    float c_log2, float value_scale) {
    // V staging for 4 waves, reused afterwards for the cross-wave merge.
    __shared__ __attribute__((aligned(16))) uint16_t lds[4 * kWaveLds];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int b = blockIdx.x, g = blockIdx.y;
    const int p = ctx_lens[b];

    bf16x8 qf[kDqk / 32];
    load_q(qf, q, b, g, hq, lane);
    SwaSource src{ring_k + ((size_t)b * R * hkv + g) * kDqk, ring_v + ((size_t)b * R * hkv + g) * kDv,
                  k_new + ((size_t)b * hkv + g) * kDqk, v_new + ((size_t)b * hkv + g) * kDv, R, p, hkv};
    WaveAcc acc;
    acc_init(acc);
    run_tiles(acc, qf, lds + wave * kWaveLds, src, wave * kTile, 4 * kTile, R + 1, c_log2, lane);
    acc.l += __shfl_xor(acc.l, 16);
    acc.l += __shfl_xor(acc.l, 32);

    // Merge the 4 waves: per wave 16 x (m, l) and O [16 heads][128 dv] in fp32.
    __syncthreads();
    float* mrg = reinterpret_cast<float*>(lds);
    float* mrg_ml = mrg;                      // [wave][16][2]
    float* mrg_o = mrg + 4 * kGroup * 2;      // [wave][16][128]
    const int G = lane >> 4, h = lane & 15;
    if (G == 0) {
        mrg_ml[(wave * kGroup + h) * 2 + 0] = acc.m;
        mrg_ml[(wave * kGroup + h) * 2 + 1] = acc.l;
    }
#pragma unroll
    for (int db = 0; db < kDv / 16; ++db)
        *reinterpret_cast<f32x4*>(mrg_o + (wave * kGroup + h) * kDv + 16 * db + 4 * G) = acc.o[db];
    __syncthreads();

    const int hl = tid >> 4;          // local head 0..15
    const int e0 = (tid & 15) * 8;    // 8 output columns
    const int head = g * kGroup + hl;
    float sl = kNoMax;
    bool has = false;
    if (sink) {
        const float sv = sink[head] * kLog2e;
        if (sv > -__builtin_inff()) { sl = sv; has = true; }
    }
    float M = has ? sl : kNoMax;
#pragma unroll
    for (int w = 0; w < 4; ++w) M = fmaxf(M, mrg_ml[(w * kGroup + hl) * 2]);
    float Z = has ? fast_exp2(sl - M) : 0.0f;
    float o[8] = {};
#pragma unroll
    for (int w = 0; w < 4; ++w) {
        const float wt = fast_exp2(mrg_ml[(w * kGroup + hl) * 2] - M);
        Z += wt * mrg_ml[(w * kGroup + hl) * 2 + 1];
        const float* src_o = mrg_o + (w * kGroup + hl) * kDv + e0;
#pragma unroll
        for (int e = 0; e < 8; ++e) o[e] += wt * src_o[e];
    }
    const float inv = value_scale / Z;
    u32x4 w4 = {pack_bf16x2(o[0] * inv, o[1] * inv), pack_bf16x2(o[2] * inv, o[3] * inv),
                pack_bf16x2(o[4] * inv, o[5] * inv), pack_bf16x2(o[6] * inv, o[7] * inv)};
    *reinterpret_cast<u32x4*>(out + ((size_t)b * hq + head) * kDv + e0) = w4;
    if (lse && (tid & 15) == 0) lse[(size_t)b * hq + head] = (M + __log2f(Z)) * kLn2;
}

// ---------------------------------------------------------------------------
// GA: keys [k0, k1) of one sequence; position j < p from the pool, j == p new.
struct GaSource {
    const uint16_t* pool_k;  // row kv_base[b] of the pool, group g applied
    const uint16_t* pool_v;
    const uint16_t* new_k;
    const uint16_t* new_v;
    int k1, p, hkv;
    __device__ bool valid(int j) const { return j < k1; }
    __device__ const uint16_t* krow(int j) const {
        if (j >= k1) return nullptr;
        return j == p ? new_k : pool_k + (size_t)j * hkv * kDqk;
    }
    __device__ const uint16_t* vrow(int j) const {
        if (j >= k1) return nullptr;
        return j == p ? new_v : pool_v + (size_t)j * hkv * kDv;
    }
};

__global__ __launch_bounds__(256) void ga_split_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k_new, const uint16_t* __restrict__ v_new,
    const uint16_t* __restrict__ pool_k, const uint16_t* __restrict__ pool_v, const int64_t* __restrict__ kv_base,
    const int32_t* __restrict__ ctx_lens, int hq, int hkv, int split, int nsplit, float c_log2,
    float* __restrict__ ws_ml, float* __restrict__ ws_o) {
    __shared__ __attribute__((aligned(16))) uint16_t lds[4 * kWaveLds];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int s = blockIdx.x, b = blockIdx.y;
    const int g = blockIdx.z * 4 + wave;
    if (g >= hkv) return;
    const int p = ctx_lens[b];
    const int k0 = s * split;
    if (k0 > p) return;
    const int k1 = min(k0 + split, p + 1);

    bf16x8 qf[kDqk / 32];
    load_q(qf, q, b, g, hq, lane);
    const size_t base = (size_t)kv_base[b];
    GaSource src{pool_k + (base * hkv + g) * kDqk, pool_v + (base * hkv + g) * kDv,
                 k_new + ((size_t)b * hkv + g) * kDqk, v_new + ((size_t)b * hkv + g) * kDv, k1, p, hkv};
    WaveAcc acc;
    acc_init(acc);
    run_tiles(acc, qf, lds + wave * kWaveLds, src, k0, kTile, k1, c_log2, lane);
    acc.l += __shfl_xor(acc.l, 16);
    acc.l += __shfl_xor(acc.l, 32);

    const int G = lane >> 4, h = lane & 15;
    const size_t row = ((size_t)b * nsplit + s) * hq + g * kGroup + h;
    if (G == 0) {
        ws_ml[row * 2 + 0] = acc.m;
        ws_ml[row * 2 + 1] = acc.l;
    }
#pragma unroll
    for (int db = 0; db < kDv / 16; ++db) *reinterpret_cast<f32x4*>(ws_o + row * kDv + 16 * db + 4 * G) = acc.o[db];
}

// Merge of the splits of one sequence: block (b, 64-head chunk), thread = (head, 32 columns).
__global__ __launch_bounds__(256) void ga_combine_kernel(const float* __restrict__ ws_ml, const float* __restrict__ ws_o,
                                                         const int32_t* __restrict__ ctx_lens, const float* __restrict__ sink,
                                                         uint16_t* __restrict__ out, float* __restrict__ lse, int hq,
                                                         int split, int nsplit, float value_scale) {
    const int b = blockIdx.x;
    const int head = blockIdx.y * 64 + (threadIdx.x >> 2);
    if (head >= hq) return;
    const int e0 = (threadIdx.x & 3) * 32;
    const int p = ctx_lens[b];
    const int ns = (p + 1 + split - 1) / split;
    uint16_t* orow = out + ((size_t)b * hq + head) * kDv + e0;
    if (ns > nsplit) {  // the grid did not cover this context: refuse loudly
        const uint16_t nan_bf16 = 0x7fc0;
        for (int e = 0; e < 32; ++e) orow[e] = nan_bf16;
        if (lse && e0 == 0) lse[(size_t)b * hq + head] = __builtin_nanf("");
        return;
    }
    float sl = kNoMax;
    bool has = false;
    if (sink) {
        const float sv = sink[head] * kLog2e;
        if (sv > -__builtin_inff()) { sl = sv; has = true; }
    }
    float M = has ? sl : kNoMax;
    for (int s = 0; s < ns; ++s) M = fmaxf(M, ws_ml[(((size_t)b * nsplit + s) * hq + head) * 2]);
    float Z = has ? fast_exp2(sl - M) : 0.0f;
    f32x4 o[8] = {};
    for (int s = 0; s < ns; ++s) {
        const size_t row = ((size_t)b * nsplit + s) * hq + head;
        const float wt = fast_exp2(ws_ml[row * 2] - M);
        Z += wt * ws_ml[row * 2 + 1];
        const f32x4* src = reinterpret_cast<const f32x4*>(ws_o + row * kDv + e0);
#pragma unroll
        for (int i = 0; i < 8; ++i) o[i] += wt * src[i];
    }
    const float inv = value_scale / Z;
#pragma unroll
    for (int i = 0; i < 8; i += 2) {
        u32x4 w = {pack_bf16x2(o[i][0] * inv, o[i][1] * inv), pack_bf16x2(o[i][2] * inv, o[i][3] * inv),
                   pack_bf16x2(o[i + 1][0] * inv, o[i + 1][1] * inv), pack_bf16x2(o[i + 1][2] * inv, o[i + 1][3] * inv)};
        *reinterpret_cast<u32x4*>(orow + 4 * i) = w;
    }
    if (lse && e0 == 0) lse[(size_t)b * hq + head] = (M + __log2f(Z)) * kLn2;
}

}  // namespace

hipError_t launch_decode_swa(const DecodeArgs& a, hipStream_t stream) {
    const int R = a.window - 1;
    hipLaunchKernelGGL(swa_decode_kernel, dim3(a.batch, a.hkv), dim3(256), 0, stream, a.q, a.k_new, a.v_new,
                       a.k_cache, a.v_cache, a.ctx_lens, a.sink, a.out, a.lse, a.hq, a.hkv, R,
                       a.softmax_scale * kLog2e, a.value_scale);
    return hipGetLastError();
}

hipError_t launch_decode_ga(const DecodeArgs& a, hipStream_t stream) {
    const int nsplit = ga_num_splits(a.max_ctx, a.split);
    float* ws_ml = static_cast<float*>(a.workspace);
    float* ws_o = ws_ml + (size_t)a.batch * nsplit * a.hq * 2;
    hipLaunchKernelGGL(ga_split_kernel, dim3(nsplit, a.batch, (a.hkv + 3) / 4), dim3(256), 0, stream, a.q, a.k_new,
                       a.v_new, a.k_cache, a.v_cache, a.kv_base, a.ctx_lens, a.hq, a.hkv, a.split, nsplit,
                       a.softmax_scale * kLog2e, ws_ml, ws_o);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(ga_combine_kernel, dim3(a.batch, (a.hq + 63) / 64), dim3(256), 0, stream, ws_ml, ws_o,
                       a.ctx_lens, a.sink, a.out, a.lse, a.hq, a.split, nsplit, a.value_scale);
    return hipGetLastError();
}

}  // namespace mimo
