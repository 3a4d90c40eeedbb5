// backward.hip -- gradients of prefill attention: dq, dk, dv and the sink's.
//
// Operation (Hugging Face Transformers model doc "MiMo-V2-Flash": Key
// features, SWA/GA with a learnable attention sink; MiMoV2FlashConfig, 64/4
// heads, head_dim 192 / v_head_dim 128, sliding_window 129): the forward is
// o = value_scale * sum_j P_j v_j with P_j = exp(s_j - LSE), s_j = scale q.k_j
// and LSE = log(sum_j exp(s_j) + exp(sink)).  For an upstream dO the gradient
// of sum(dO * o) is, per query row (token t, head h, group g):
//   D     = dO . o                       dP_j = value_scale * dO . v_j
//   dS_j  = P_j (dP_j - D)
//   dq    = scale * sum_j dS_j k_j       dk_j += scale * dS_j q,  dv_j += value_scale * P_j dO
//   dsink[h] = -sum_t exp(sink[h] - LSE_t) D_t
// P is recomputed from the forward's LSE (natural log, sink included) and D
// from its output o, so the sink needs no further term in dq/dk/dv.
//
// Kernels (fp32 accumulate; P and dS are rounded to bf16 as MFMA operands):
//   bwd_rowdot_kernel  D = dO . o per (token, head), into the workspace;
//   bwd_dq_kernel      32x32x16 MFMAs, one wave per 2 tokens x 16 heads of a
//                      KV group (the MFMA N side); Q^T and dO^T stay in
//                      registers, 32-key tiles of K and V are staged in LDS for
//                      16 tokens; S^T = K Q^T and dP^T = V dO^T, then
//                      dQ^T += K^T dS^T with K^T read from the LDS tile by
//                      transposed reads;
//   bwd_dkdv_kernel    16x16x32 MFMAs, one wave per 16 keys (the N side), K and
//                      V rows stay in registers; blocks of 2 tokens x 16 heads
//                      of Q and dO are staged in LDS for 128 keys; S = Q K^T
//                      and dP = dO V^T, then dV^T += dO^T P and dK^T += Q^T dS.
//                      (A 32x32x16 form with 32 keys per wave needs ~390
//                      registers, i.e. one wave per SIMD, and ran 1.4x slower.)
//   bwd_sink_kernel    dsink per head, a fixed-order block reduction.
// LDS tiles are laid out so that neither kernel's reads meet bank conflicts:
// padded rows, and for the dq K tile a permuted row order within 16-row blocks
// (dq_key_row); the dk/dv tiles keep row order at a different pitch.
#include "device_common.hpp"
#include "launch.hpp"

namespace mimo {
namespace {

constexpr int kDqk = 192;
constexpr int kDv = 128;
constexpr int kGroup = 16;
// dk/dv LDS tiles of 32 query rows, in row order, padded to 416 bytes (Q)
// and 288 bytes (dO): a row pitch of 2 mod 4 16-byte chunks is what keeps both
// of this kernel's read patterns free of bank conflicts on gfx950, the 16-byte
// row reads (lanes 16i..16i+15 on 16 consecutive rows, chunk i) and the
// transposed reads below (measured with SQ_LDS_BANK_CONFLICT over pitches of
// 256..528 bytes: odd-chunk pitches halve the row-read rate, multiples of 4
// chunks cost 2-8x).
constexpr int kQRow = kDqk * 2 + 32;  // bytes per staged Q row
constexpr int kVRow = kDv * 2 + 32;   // bytes per staged dO row

// 8 bf16 of tile row r, 16-byte chunk c (a direct MFMA operand).
__device__ __forceinline__ bf16x8 lds_row8(const char* tile, int row_bytes, int r, int c) {
    return *reinterpret_cast<const bf16x8*>(tile + r * row_bytes + c * 16);
}

__device__ __forceinline__ void lds_put16(char* tile, int row_bytes, int r, int c, const u32x4& x) {
    *reinterpret_cast<u32x4*>(tile + r * row_bytes + c * 16) = x;
}

// Transposed A operand over tile rows 0..31, columns 16db .. 16db+15: lane l
// (G = l/16) gets tile[row(8G+t)][16db + l%16] for t = 0..7 with row(8G+t) =
// 4G+t (t < 4) or 16+4G+t-4 (t >= 4): the k order of a B operand packed from
// two 16-row accumulator blocks (rows 4G+r of block 0, then of block 1).
__device__ __forceinline__ bf16x8 lds_tr8(const char* tile, int row_bytes, int db, int lane) {
    const int G = lane >> 4, tq = (lane & 15) >> 2;
    const char* p = tile + (4 * G + tq) * row_bytes + 32 * db + 8 * (lane & 3);
    return join_tr(lds_read_tr16(reinterpret_cast<const uint16_t*>(p)),
                   lds_read_tr16(reinterpret_cast<const uint16_t*>(p + 16 * row_bytes)));
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __builtin_bit_cast(float, w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __builtin_bit_cast(float, w & 0xffff0000u); }

// ---------------------------------------------------------------------------
// D = dO . o, 16 threads (8 elements each) per (token, head) row.
__global__ __launch_bounds__(256) void bwd_rowdot_kernel(const uint16_t* __restrict__ dout,
                                                         const uint16_t* __restrict__ out, float* __restrict__ D,
                                                         int64_t rows) {
    const int64_t row = (int64_t)blockIdx.x * 16 + (threadIdx.x >> 4);
    const int c = threadIdx.x & 15;
    float acc = 0.0f;
    if (row < rows) {
        const u32x4 a = reinterpret_cast<const u32x4*>(dout + row * kDv)[c];
        const u32x4 o = reinterpret_cast<const u32x4*>(out + row * kDv)[c];
#pragma unroll
        for (int i = 0; i < 4; ++i) acc += bf16_lo(a[i]) * bf16_lo(o[i]) + bf16_hi(a[i]) * bf16_hi(o[i]);
    }
    acc += __shfl_xor(acc, 8);
    acc += __shfl_xor(acc, 4);
    acc += __shfl_xor(acc, 2);
    acc += __shfl_xor(acc, 1);
    if (row < rows && c == 0) D[row] = acc;
}

// dsink[h] = -sum over the batch's tokens of exp(sink[h] - lse) * D, one block
// per head; each thread sums a fixed stride of tokens into eight running sums
// (token t + 256u goes to sum u, so the loads of eight tokens are in flight
// together; the last few go to sum 0), then the sums and the threads are
// added in a fixed tree.
constexpr int kSinkUnroll = 8;
__global__ __launch_bounds__(256) void bwd_sink_kernel(const float* __restrict__ sink, const float* __restrict__ lse,
                                                       const float* __restrict__ D, const int32_t* __restrict__ cu,
                                                       int num_seqs, int max_seqlen, int hq,
                                                       float* __restrict__ dsink) {
    __shared__ float part[256];
    const int h = blockIdx.x;
    const float s = sink ? sink[h] : -__builtin_inff();
    float acc[kSinkUnroll] = {};
    if (s > -__builtin_inff()) {
        for (int b = 0; b < num_seqs; ++b) {
            const int s0 = cu[b], L = min(cu[b + 1] - s0, max_seqlen);
            int t = threadIdx.x;
            for (; t + (kSinkUnroll - 1) * 256 < L; t += kSinkUnroll * 256) {
                float l[kSinkUnroll], d[kSinkUnroll];
#pragma unroll
                for (int u = 0; u < kSinkUnroll; ++u) {
                    const size_t row = (size_t)(s0 + t + 256 * u) * hq + h;
                    l[u] = lse[row];
                    d[u] = D[row];
                }
#pragma unroll
                for (int u = 0; u < kSinkUnroll; ++u) acc[u] += fast_exp2((s - l[u]) * kLog2e) * d[u];
            }
            for (; t < L; t += 256) {
                const size_t row = (size_t)(s0 + t) * hq + h;
                acc[0] += fast_exp2((s - lse[row]) * kLog2e) * D[row];
            }
        }
    }
    static_assert(kSinkUnroll == 8, "the tree below adds eight sums");
    part[threadIdx.x] = ((acc[0] + acc[1]) + (acc[2] + acc[3])) + ((acc[4] + acc[5]) + (acc[6] + acc[7]));
    __syncthreads();
    for (int w = 128; w > 0; w >>= 1) {
        if ((int)threadIdx.x < w) part[threadIdx.x] += part[threadIdx.x + w];
        __syncthreads();
    }
    if (threadIdx.x == 0) dsink[h] = 0.0f - part[0];  // +0 for an empty sum (0 - x is exactly -x otherwise)
}

// ---------------------------------------------------------------------------
// dq: the forward's tile shape with v_mfma_f32_32x32x16_bf16 -- each wave owns
// 32 query rows (2 tokens x 16 heads of a KV group, lane row r32 = lane % 32,
// hh = lane / 32 the half of the MFMA K dimension it feeds), so every 16-byte
// operand read from LDS feeds 32 x 32 x 16 MACs.  K and V tiles (32 keys) sit
// in LDS with padded rows, K's in the order dq_key_row().
constexpr int kDqTok = 16;           // tokens per workgroup (8 waves x 2)
constexpr int kDqNK = 32;            // keys per staged tile
constexpr int kKS = kDqk + 8;        // LDS row strides (bf16 elements): 25 and 17 chunks
constexpr int kVS = kDv + 8;
constexpr int kDqLdsK = kDqNK * kKS;
constexpr int kDqLdsV = kDqNK * kVS;

// LDS row of key j of a dq K tile: within each 16-row block, j goes to
// 4(j % 4) + j / 4, so the transposed K^T reads (keys 4hh + t, t = 0..3, in one
// 32-lane phase) take rows 4 apart.  At the 400-byte pitch this order keeps
// both the K^T reads and the direct key-row reads free of bank conflicts on
// gfx950 (SQ_LDS_BANK_CONFLICT zero; in key order, with 320-byte V rows, the
// kernel lost about half its LDS cycles to conflicts).
__device__ __forceinline__ int dq_key_row(int j) { return (j & ~15) | ((j & 3) << 2) | ((j >> 2) & 3); }

template <bool SWA>
__global__ __attribute__((amdgpu_flat_work_group_size(512, 512), amdgpu_waves_per_eu(2, 2))) void bwd_dq_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    const uint16_t* __restrict__ dout, const float* __restrict__ lse, const float* __restrict__ Dws,
    const int32_t* __restrict__ cu_seqlens, uint16_t* __restrict__ dq, int hq, int hkv, int window, float c_log2,
    float scale, float value_scale, int max_seqlen, int nqb) {
    __shared__ __attribute__((aligned(16))) uint16_t lds_k[2 * kDqLdsK];
    __shared__ __attribute__((aligned(16))) uint16_t lds_v[2 * kDqLdsV];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = tid >> 6;
    const int r32 = lane & 31, hh = lane >> 5;
    const int b = blockIdx.z, g = blockIdx.y;
    const int qb = SWA ? (int)blockIdx.x : nqb - 1 - (int)blockIdx.x;  // GA: longest rows first
    const int s0 = cu_seqlens[b];
    const int L = min(cu_seqlens[b + 1] - s0, max_seqlen);
    const int q0 = qb * kDqTok;
    if (q0 >= L) return;
    const int tok = q0 + 2 * wave + (r32 >> 4);
    const bool valid = tok < L;
    const int head = g * kGroup + (r32 & 15);
    const size_t qrow = (size_t)(s0 + min(tok, L - 1)) * hq + head;

    // Q^T and dO^T of the wave's 32 rows as MFMA B operands (d = 16s + 8hh .. +7).
    bf16x8 qf[kDqk / 16], dof[kDv / 16];
#pragma unroll
    for (int st = 0; st < kDqk / 16; ++st)
        qf[st] = __builtin_bit_cast(bf16x8, reinterpret_cast<const u32x4*>(q + qrow * kDqk)[2 * st + hh]);
#pragma unroll
    for (int st = 0; st < kDv / 16; ++st)
        dof[st] = __builtin_bit_cast(bf16x8, reinterpret_cast<const u32x4*>(dout + qrow * kDv)[2 * st + hh]);
    const float lse2 = lse[qrow] * kLog2e;
    const float Drow = Dws[qrow];
    f32x16 dqa[kDqk / 32];
#pragma unroll
    for (int db = 0; db < kDqk / 32; ++db) dqa[db] = f32x16{};

    const int t_last = min(q0 + kDqTok, L) - 1;
    const int k_lo = SWA ? max(0, q0 - (window - 1)) : 0;
    const int kt_begin = k_lo / kDqNK, kt_end = t_last / kDqNK;

    // Staging of a 32-key tile: K rows (768 16-byte chunks), V rows (512).
    // Chunk owners are fixed per thread and uniform per wave: K chunk tid (all
    // waves), K chunk 512 + tid (waves 0-3), V chunk tid - 256 (waves 4-7), V
    // chunk 256 + tid (waves 0-3).  Loads go through descriptors whose base is
    // the tile's first key and whose record count ends at the sequence end
    // (keys past it read as zeros and are masked).
    static_assert(kDqNK * (kDqk / 8) == 768 && kDqNK * (kDv / 8) == 512, "chunk owners assume 32 keys");
    const bool lo_waves = tid < 256;
    const int kc1 = 512 + tid, vc0 = tid - 256, vc1 = 256 + tid;
    const uint32_t krow_b = (uint32_t)hkv * (kDqk * 2), vrow_b = (uint32_t)hkv * (kDv * 2);
    const uint32_t off0 = (uint32_t)(tid / (kDqk / 8)) * krow_b + (tid % (kDqk / 8)) * 16;
    const uint32_t off1 = lo_waves ? (uint32_t)(kc1 / (kDqk / 8)) * krow_b + (kc1 % (kDqk / 8)) * 16
                                   : (uint32_t)(vc0 / (kDv / 8)) * vrow_b + (vc0 % (kDv / 8)) * 16;
    const uint32_t off2 = lo_waves ? (uint32_t)(vc1 / (kDv / 8)) * vrow_b + (vc1 % (kDv / 8)) * 16 : 0u;
    u32x4 reg[3];
    auto load_tile = [&](int kt) {
        const int kb = kt * kDqNK;
        const uint32_t keys = (uint32_t)max(0, min(L - kb, kDqNK));
        const rsrc_t rk = make_rsrc(k + ((size_t)(s0 + kb) * hkv + g) * kDqk, keys * krow_b);
        const rsrc_t rv = make_rsrc(v + ((size_t)(s0 + kb) * hkv + g) * kDv, keys * vrow_b);
        reg[0] = __builtin_amdgcn_raw_buffer_load_b128(rk, off0, 0, 0);
        reg[1] = __builtin_amdgcn_raw_buffer_load_b128(lo_waves ? rk : rv, off1, 0, 0);
        reg[2] = __builtin_amdgcn_raw_buffer_load_b128(rv, off2, 0, 0);  // waves 4-7: unused
    };
    auto put_k = [&](int buf, int c, const u32x4& x) {
        *reinterpret_cast<u32x4*>(lds_k + buf * kDqLdsK + dq_key_row(c / (kDqk / 8)) * kKS + (c % (kDqk / 8)) * 8) = x;
    };
    auto put_v = [&](int buf, int c, const u32x4& x) {
        *reinterpret_cast<u32x4*>(lds_v + buf * kDqLdsV + (c / (kDv / 8)) * kVS + (c % (kDv / 8)) * 8) = x;
    };
    auto store_tile = [&](int buf) {
        put_k(buf, tid, reg[0]);
        if (lo_waves) {
            put_k(buf, kc1, reg[1]);
            put_v(buf, vc1, reg[2]);
        } else {
            put_v(buf, vc0, reg[1]);
        }
    };
    // Direct A operands: key r32, d = 16s + 8hh.  Transposed K^T reads (the
    // forward's V^T pattern): keys 4hh + (lane%16)/4 (+8) of a 16-key step, i.e.
    // LDS rows 4((lane%16)/4) + hh (+2), columns 16((lane/16)%2) + 4(lane%4) of
    // a 32-wide d block.
    const int kdir = dq_key_row(r32) * kKS + 8 * hh, vdir = r32 * kVS + 8 * hh;
    const int ktr = (4 * ((lane & 15) >> 2) + hh) * kKS + 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
    load_tile(kt_begin);
    store_tile(0);
    __syncthreads();
    for (int kt = kt_begin; kt <= kt_end; ++kt) {
        const int buf = (kt - kt_begin) & 1;
        const bool more = kt < kt_end;
        const uint16_t* ktile = lds_k + buf * kDqLdsK;
        const uint16_t* vtile = lds_v + buf * kDqLdsV;
        const int kbase = kt * kDqNK;
        // S^T = K Q^T and dP^T = V dO^T: lane holds key kbase + 8(r/4) + 4hh + r%4, row r32.
        f32x16 s = f32x16{}, dp = f32x16{};
#pragma unroll
        for (int st = 0; st < kDqk / 16; ++st)
            s = mfma_32x32x16(*reinterpret_cast<const bf16x8*>(ktile + kdir + 16 * st), qf[st], s);
#pragma unroll
        for (int st = 0; st < kDv / 16; ++st)
            dp = mfma_32x32x16(*reinterpret_cast<const bf16x8*>(vtile + vdir + 16 * st), dof[st], dp);
        // The next tile's loads go out here rather than at the top: their
        // registers then live only through the dQ MFMAs, not the S/dP ones
        // (at the top: equal time).  Past the last tile they read through an
        // empty descriptor.
        load_tile(kt + 1);
        // Key offset o = 8(r/4) + (r%4) of element r is kept when lo <= o <= hi:
        // the row's causal bound (and window) relative to this lane's keys, with
        // rows past the sequence end given an empty range.
        const int hi = valid ? tok - kbase - 4 * hh : -1;
        const int lo = SWA ? hi - (window - 1) : INT32_MIN;
        float ds[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int o = 8 * (r >> 2) + (r & 3);
            const bool ok = o <= hi && (!SWA || o >= lo);
            const float p = fast_exp2(ok ? __builtin_fmaf(s[r], c_log2, -lse2) : -__builtin_inff());  // masked: 0
            ds[r] = p * (value_scale * dp[r] - Drow);
        }
        // dQ^T += K^T dS^T: B operand of k-step ks holds keys 16ks + {4hh + t, 8 + 4hh + t - 4}.
        const bf16x8 dsf0 = pack_bf16x8(ds[0], ds[1], ds[2], ds[3], ds[4], ds[5], ds[6], ds[7]);
        const bf16x8 dsf1 = pack_bf16x8(ds[8], ds[9], ds[10], ds[11], ds[12], ds[13], ds[14], ds[15]);
#pragma unroll
        for (int db = 0; db < kDqk / 32; ++db) {
            const uint16_t* p0 = ktile + ktr + db * 32;
            const uint16_t* p1 = p0 + 16 * kKS;
            dqa[db] = mfma_32x32x16(join_tr(lds_read_tr16(p0), lds_read_tr16(p0 + 2 * kKS)), dsf0, dqa[db]);
            dqa[db] = mfma_32x32x16(join_tr(lds_read_tr16(p1), lds_read_tr16(p1 + 2 * kKS)), dsf1, dqa[db]);
        }
        if (more) store_tile(buf ^ 1);
        __syncthreads();
    }
    if (!valid) return;
    // lane holds dQ^T[d = 32db + 8j + 4hh + (0..3)][row r32]
    uint16_t* drow = dq + qrow * kDqk;
#pragma unroll
    for (int db = 0; db < kDqk / 32; ++db)
#pragma unroll
        for (int j = 0; j < 4; ++j)
            *reinterpret_cast<u32x2*>(drow + 32 * db + 8 * j + 4 * hh) =
                u32x2{pack_bf16x2(dqa[db][4 * j] * scale, dqa[db][4 * j + 1] * scale),
                      pack_bf16x2(dqa[db][4 * j + 2] * scale, dqa[db][4 * j + 3] * scale)};
}

// ---------------------------------------------------------------------------
constexpr int kKvWaves = 8;                    // 16 keys per wave
constexpr int kKvKeys = 16 * kKvWaves;         // keys per dk/dv workgroup
constexpr int kKvTok = 2;                      // query tokens per staged block (2 x 16 heads = 32 rows)
constexpr int kKvRows = kKvTok * kGroup;
constexpr int kKvTileBytes = kKvRows * (kQRow + kVRow) + kKvRows * 8;  // Q, dO, then lse2 and D per row

template <bool SWA>
__global__ __attribute__((amdgpu_flat_work_group_size(512, 512))) void bwd_dkdv_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    const uint16_t* __restrict__ dout, const float* __restrict__ lse, const float* __restrict__ Dws,
    const int32_t* __restrict__ cu_seqlens, uint16_t* __restrict__ dk, uint16_t* __restrict__ dv, int hq, int hkv,
    int window, float c_log2, float scale, float value_scale, int max_seqlen, int nkb) {
    __shared__ __attribute__((aligned(16))) char lds[2 * kKvTileBytes];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int G = lane >> 4;
    const int b = blockIdx.z;
    const int s0 = cu_seqlens[b];
    const int L = min(cu_seqlens[b + 1] - s0, max_seqlen);
    // SWA: workgroup (key block, group).  GA pairs the key blocks: workgroup
    // (p, g) -- g the fastest index, so that with 4 groups each XCD serves one
    // group -- takes key block p, walking its query blocks from the sequence
    // end down to its diagonal, then key block nkb-1-p, walking up from its
    // diagonal to the end.  At step s of the first walk every workgroup reads
    // query block T-2-2s, at step s of the second 2s-128 (T = 128 nkb): all
    // workgroups of a round read the same block at the same time, and each is
    // fetched about once per L2.  Each workgroup's two walks add up to T+128
    // query tokens.
    int g, kb_a, kb_b;
    if constexpr (SWA) {
        g = blockIdx.y;
        kb_a = blockIdx.x;
        kb_b = -1;
    } else {
        g = (int)blockIdx.x % hkv;
        kb_a = (int)blockIdx.x / hkv;
        kb_b = nkb - 1 - kb_a;
        if (kb_b == kb_a) kb_b = -1;
    }
    auto key_block = [&](const int kb, const bool down) {
        const int k0 = kb * kKvKeys;
        if (k0 >= L) return;
        const int key = k0 + 16 * wave + (lane & 15);
        const int kk = min(key, L - 1);
        const size_t krow = (size_t)(s0 + kk) * hkv + g;

        // K and V rows of this lane's key as MFMA B operands (d = 32st + 8G .. +7).
        bf16x8 kf[kDqk / 32], vf[kDv / 32];
#pragma unroll
        for (int st = 0; st < kDqk / 32; ++st)
            kf[st] = __builtin_bit_cast(bf16x8, reinterpret_cast<const u32x4*>(k + krow * kDqk)[4 * st + G]);
#pragma unroll
        for (int st = 0; st < kDv / 32; ++st)
            vf[st] = __builtin_bit_cast(bf16x8, reinterpret_cast<const u32x4*>(v + krow * kDv)[4 * st + G]);
        f32x4 dka[kDqk / 16], dva[kDv / 16];
#pragma unroll
        for (int db = 0; db < kDqk / 16; ++db) dka[db] = f32x4{};
#pragma unroll
        for (int db = 0; db < kDv / 16; ++db) dva[db] = f32x4{};

        // Queries that see a key of the block: tokens k0 .. q_end-1, in blocks of
        // kKvTok tokens, walked down from the end or up from k0 (see above).
        const int q_end = SWA ? min(L, k0 + kKvKeys - 1 + window) : L;
        const int nblk = (q_end - k0 + kKvTok - 1) / kKvTok;
        auto q0_of = [&](int i) { return k0 + (down ? nblk - 1 - i : i) * kKvTok; };

        // Staging of a block of 2 tokens x 16 heads: 32 Q rows (768 16-byte
        // chunks), 32 dO rows (512 chunks), and the 32 rows' lse2 and D.  Row 16t +
        // h is token q0 + t, head 16g + h.  Chunk owners are fixed per thread and
        // uniform per wave: Q chunk tid (all waves), Q chunk 512 + tid (waves 0-3),
        // dO chunk tid - 256 (waves 4-7), dO chunk 256 + tid (waves 0-3).  Loads go
        // through descriptors whose base is the block's first row and whose record
        // count ends at the sequence end, so rows past it read as zeros (their
        // probabilities are forced to zero) and no per-block address arithmetic is
        // vector work.  Blocks are loaded two ahead, alternating two register sets.
        constexpr int kQChunks = kKvRows * (kDqk / 8);
        const bool lo_waves = wave < 4;
        const int qc1 = 512 + tid, oc0 = tid - 256, oc1 = 256 + tid;
        auto q_off = [&](int qc) {
            const int row = qc / (kDqk / 8);
            return (uint32_t)(((row / kGroup) * hq + row % kGroup) * (kDqk * 2) + (qc % (kDqk / 8)) * 16);
        };
        auto o_off = [&](int oc) {
            const int row = oc / (kDv / 8);
            return (uint32_t)(((row / kGroup) * hq + row % kGroup) * (kDv * 2) + (oc % (kDv / 8)) * 16);
        };
        const uint32_t off0 = q_off(tid);
        const uint32_t off1 = lo_waves ? q_off(qc1) : o_off(oc0);
        const uint32_t off2 = lo_waves ? o_off(oc1) : 0u;
        const uint32_t off_s = (uint32_t)(((tid & 31) / kGroup) * hq + (tid & 31) % kGroup) * 4;
        struct Stage {
            u32x4 r[3];
            float lse2, d;
        };
        auto load_blk = [&](Stage& st, int i) {  // block i of the walk; past the last one nothing is read
            const int q0 = i < nblk ? q0_of(i) : k0;
            const uint32_t toks = i < nblk ? (uint32_t)max(0, min(L - q0, kKvTok)) : 0u;
            const size_t row0 = (size_t)(s0 + q0) * hq + g * kGroup;
            const rsrc_t rq = make_rsrc(q + row0 * kDqk, toks * (uint32_t)hq * (kDqk * 2));
            const rsrc_t ro = make_rsrc(dout + row0 * kDv, toks * (uint32_t)hq * (kDv * 2));
            const rsrc_t rl = make_rsrc(lse + row0, toks * (uint32_t)hq * 4);
            const rsrc_t rd = make_rsrc(Dws + row0, toks * (uint32_t)hq * 4);
            st.r[0] = __builtin_amdgcn_raw_buffer_load_b128(rq, off0, 0, 0);
            st.r[1] = __builtin_amdgcn_raw_buffer_load_b128(lo_waves ? rq : ro, off1, 0, 0);
            st.r[2] = __builtin_amdgcn_raw_buffer_load_b128(ro, off2, 0, 0);  // waves 4-7: unused
            st.lse2 = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rl, off_s, 0, 0)) * kLog2e;
            st.d = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rd, off_s, 0, 0));
        };
        auto store_blk = [&](const Stage& st, int buf) {
            char* qt_ = lds + buf * kKvTileBytes;
            char* ot_ = qt_ + kKvRows * kQRow;
            float* sf = reinterpret_cast<float*>(ot_ + kKvRows * kVRow);
            lds_put16(qt_, kQRow, tid / (kDqk / 8), tid % (kDqk / 8), st.r[0]);
            if (lo_waves) {
                lds_put16(qt_, kQRow, qc1 / (kDqk / 8), qc1 % (kDqk / 8), st.r[1]);
                lds_put16(ot_, kVRow, oc1 / (kDv / 8), oc1 % (kDv / 8), st.r[2]);
            } else {
                lds_put16(ot_, kVRow, oc0 / (kDv / 8), oc0 % (kDv / 8), st.r[1]);
            }
            if (tid < kKvRows) {
                sf[tid] = st.lse2;
                sf[kKvRows + tid] = st.d;
            }
        };
        static_assert(kQChunks == 768 && kKvRows * (kDv / 8) == 512, "chunk owners assume 32 rows of 192 + 128");
        auto compute_blk = [&](int ib, int buf) {
            const int q0 = q0_of(ib);
            const char* Qt = lds + buf * kKvTileBytes;
            const char* Ot = Qt + kKvRows * kQRow;
            const float* sf = reinterpret_cast<const float*>(Ot + kKvRows * kVRow);
            // S = Q K^T and dP = dO V^T: lane holds row 16blk + 4G + r (token
            // q0 + blk, head 4G + r of the group) and key `key`.
            f32x4 s[kKvTok], dp[kKvTok];
#pragma unroll
            for (int blk = 0; blk < kKvTok; ++blk) {
                s[blk] = f32x4{};
                dp[blk] = f32x4{};
#pragma unroll
                for (int st = 0; st < kDqk / 32; ++st)
                    s[blk] = mfma_16x16x32(lds_row8(Qt, kQRow, 16 * blk + (lane & 15), 4 * st + G), kf[st], s[blk]);
#pragma unroll
                for (int st = 0; st < kDv / 32; ++st)
                    dp[blk] = mfma_16x16x32(lds_row8(Ot, kVRow, 16 * blk + (lane & 15), 4 * st + G), vf[st], dp[blk]);
            }
            float p[kKvTok][4], ds[kKvTok][4];
#pragma unroll
            for (int blk = 0; blk < kKvTok; ++blk) {
                const int tok = q0 + blk;
                const bool tok_ok = tok < L && key < L && key <= tok && (!SWA || tok <= key + window - 1);
                // The lane's four rows 16blk + 4G + r are consecutive: one 16-byte read each for lse2 and D.
                const f32x4 l4 = *reinterpret_cast<const f32x4*>(sf + 16 * blk + 4 * G);
                const f32x4 d4 = *reinterpret_cast<const f32x4*>(sf + kKvRows + 16 * blk + 4 * G);
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    // Masked entries take exp2(-inf) = 0 rather than a branch around the exp.
                    const float arg = __builtin_fmaf(s[blk][r], c_log2, -l4[r]);
                    const float pr = fast_exp2(tok_ok ? arg : -__builtin_inff());
                    p[blk][r] = pr;
                    ds[blk][r] = pr * (value_scale * dp[blk][r] - d4[r]);
                }
            }
            const bf16x8 pf = pack_bf16x8(p[0][0], p[0][1], p[0][2], p[0][3], p[1][0], p[1][1], p[1][2], p[1][3]);
            const bf16x8 dsf =
                pack_bf16x8(ds[0][0], ds[0][1], ds[0][2], ds[0][3], ds[1][0], ds[1][1], ds[1][2], ds[1][3]);
#pragma unroll
            for (int db = 0; db < kDv / 16; ++db) dva[db] = mfma_16x16x32(lds_tr8(Ot, kVRow, db, lane), pf, dva[db]);
#pragma unroll
            for (int db = 0; db < kDqk / 16; ++db) dka[db] = mfma_16x16x32(lds_tr8(Qt, kQRow, db, lane), dsf, dka[db]);
        };
        Stage sa, sb;
        load_blk(sa, 0);
        store_blk(sa, 0);
        load_blk(sb, 1);
        __syncthreads();
        int ib = 0;
        for (; ib + 1 < nblk; ib += 2) {
            load_blk(sa, ib + 2);
            compute_blk(ib, 0);
            store_blk(sb, 1);
            __syncthreads();
            load_blk(sb, ib + 3);
            compute_blk(ib + 1, 1);
            if (ib + 2 < nblk) store_blk(sa, 0);
            __syncthreads();
        }
        if (ib < nblk) compute_blk(ib, 0);
        if (key >= L) return;
        // lane holds dK^T[d = 16db + 4G + r][key] and dV^T likewise
        uint16_t* kout = dk + krow * kDqk;
        uint16_t* vout = dv + krow * kDv;
#pragma unroll
        for (int db = 0; db < kDqk / 16; ++db)
            *reinterpret_cast<u32x2*>(kout + 16 * db + 4 * G) =
                u32x2{pack_bf16x2(dka[db][0] * scale, dka[db][1] * scale),
                      pack_bf16x2(dka[db][2] * scale, dka[db][3] * scale)};
#pragma unroll
        for (int db = 0; db < kDv / 16; ++db)
            *reinterpret_cast<u32x2*>(vout + 16 * db + 4 * G) =
                u32x2{pack_bf16x2(dva[db][0] * value_scale, dva[db][1] * value_scale),
                      pack_bf16x2(dva[db][2] * value_scale, dva[db][3] * value_scale)};
    };
    key_block(kb_a, !SWA);
    if (kb_b >= 0) {
        __syncthreads();  // the first walk's last reads of the staging buffers come before the second's writes
        key_block(kb_b, false);
    }
}

}  // namespace

hipError_t launch_prefill_backward(const BackwardArgs& a, hipStream_t stream) {
    if (a.max_seqlen <= 0 || a.total_tokens <= 0) {
        // No token contributes: there are no rows to write, and dsink, a sum
        // over no tokens, is zero (the sink kernel over zero sequences reads
        // nothing and writes it).
        if (!a.dsink) return hipSuccess;
        hipLaunchKernelGGL(bwd_sink_kernel, dim3(a.hq), dim3(256), 0, stream, a.sink, nullptr, nullptr, a.cu_seqlens,
                           0, 0, a.hq, a.dsink);
        return hipGetLastError();
    }
    float* D = static_cast<float*>(a.workspace);
    const int64_t rows = (int64_t)a.total_tokens * a.hq;
    hipLaunchKernelGGL(bwd_rowdot_kernel, dim3((unsigned)((rows + 15) / 16)), dim3(256), 0, stream, a.dout, a.out, D,
                       rows);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const float c_log2 = a.softmax_scale * kLog2e;
    const int nqb = (a.max_seqlen + kDqTok - 1) / kDqTok;
    hipLaunchKernelGGL(a.swa ? bwd_dq_kernel<true> : bwd_dq_kernel<false>, dim3(nqb, a.hkv, a.num_seqs), dim3(512), 0,
                       stream, a.q, a.k, a.v, a.dout, a.lse, D, a.cu_seqlens, a.dq, a.hq, a.hkv, a.window, c_log2,
                       a.softmax_scale, a.value_scale, a.max_seqlen, nqb);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    const int nkb = (a.max_seqlen + kKvKeys - 1) / kKvKeys;
    const dim3 kv_grid = a.swa ? dim3(nkb, a.hkv, a.num_seqs) : dim3((unsigned)((nkb + 1) / 2 * a.hkv), 1, a.num_seqs);
    hipLaunchKernelGGL(a.swa ? bwd_dkdv_kernel<true> : bwd_dkdv_kernel<false>, kv_grid, dim3(512), 0, stream, a.q,
                       a.k, a.v, a.dout, a.lse, D, a.cu_seqlens, a.dk, a.dv, a.hq, a.hkv, a.window, c_log2,
                       a.softmax_scale, a.value_scale, a.max_seqlen, nkb);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    if (a.dsink) {
        hipLaunchKernelGGL(bwd_sink_kernel, dim3(a.hq), dim3(256), 0, stream, a.sink, a.lse, D, a.cu_seqlens,
                           a.num_seqs, a.max_seqlen, a.hq, a.dsink);
        e = hipGetLastError();
    }
    return e;
}

}  // namespace mimo
