// device_common.hpp -- gfx950 (CDNA4) building blocks shared by the attention kernels.
//
// MFMA operand/result lane layouts used throughout (wave64, bf16 inputs, fp32 accumulate):
//
//   v_mfma_f32_32x32x16_bf16   D[32x32] += A[32x16] * B[16x32]
//     lane l supplies A[l%32][8*(l/32) + t] and B[8*(l/32) + t][l%32], t = 0..7
//     lane l holds    D[8*(r/4) + 4*(l/32) + r%4][l%32],            r = 0..15
//
//   v_mfma_f32_16x16x32_bf16   D[16x16] += A[16x32] * B[32x16]
//     lane l supplies A[l%16][8*(l/16) + t] and B[8*(l/16) + t][l%16], t = 0..7
//     lane l holds    D[4*(l/16) + r][l%16],                         r = 0..3
//
//   ds_read_b64_tr_b16 (per 16-lane group, lanes i and j = 0..15 of the group):
//     lane i receives element (i%4) of the 4 x bf16 chunk addressed by lane
//     4*t + i/4, for t = 0..3.  If lane 4*t + c addresses row R(t), column
//     C0 + 4*c of a row-major bf16 tile, lane i receives column C0 + i of rows
//     R(0..3): a 4 x 16 block arrives transposed, one column per lane.
//
// The attention kernels compute S^T = K * Q^T (keys on the MFMA M side, the
// query rows on the N side) so that every lane owns whole query rows: row
// maxima and sums stay inside a lane except for one exchange between the two
// 32-lane halves (v_permlane32_swap).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mimo {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.44269504088896340736f;
constexpr float kLn2 = 0.69314718055994530942f;
// Finite stand-in for a running maximum of -inf: exp2(x - kNoMax) never
// produces NaN, and exp2(kNoMax - finite) is exactly 0.
constexpr float kNoMax = -1.0e30f;

__device__ __forceinline__ f32x16 mfma_32x32x16(const bf16x8& a, const bf16x8& b, const f32x16& c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma_16x16x32(const bf16x8& a, const bf16x8& b, const f32x4& c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// 4 x bf16 transposed LDS read (see the layout note above).
__device__ __forceinline__ i16x4 lds_read_tr16(const uint16_t* p) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)p);
}

__device__ __forceinline__ bf16x8 join_tr(const i16x4& lo, const i16x4& hi) {
    i16x4 x[2] = {lo, hi};
    return __builtin_bit_cast(bf16x8, x);
}

// Value held by lane l^32.  Returned as the pair (own, partner) ordered so that
// max/sum of the two gives the same result in both halves.
__device__ __forceinline__ float max_with_partner_half(float x) {
    uint32_t u = __builtin_bit_cast(uint32_t, x);
    auto p = __builtin_amdgcn_permlane32_swap(u, u, false, false);
    return fmaxf(__builtin_bit_cast(float, (uint32_t)p[0]), __builtin_bit_cast(float, (uint32_t)p[1]));
}
__device__ __forceinline__ float sum_with_partner_half(float x) {
    uint32_t u = __builtin_bit_cast(uint32_t, x);
    auto p = __builtin_amdgcn_permlane32_swap(u, u, false, false);
    return __builtin_bit_cast(float, (uint32_t)p[0]) + __builtin_bit_cast(float, (uint32_t)p[1]);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

// Round-to-nearest-even fp32 -> bf16 pair packed in one dword (one v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
    const f32x2 v = {a, b};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}

__device__ __forceinline__ bf16x8 pack_bf16x8(float a0, float a1, float a2, float a3, float a4, float a5,
                                              float a6, float a7) {
    u32x4 u = {pack_bf16x2(a0, a1), pack_bf16x2(a2, a3), pack_bf16x2(a4, a5), pack_bf16x2(a6, a7)};
    return __builtin_bit_cast(bf16x8, u);
}

// Rotary embedding of one pair of dims (x, y) = (i, i + rd/2) of a head
// vector by the angle whose fp32 cosine and sine are c and s (Transformers'
// rotary convention; model doc, MiMoV2FlashConfig: rope_parameters).  The
// standalone RoPE pass and the rotation of Q fragments in the prefill kernels
// share this arithmetic, so both round to the same bf16 values.
__device__ __forceinline__ void rope_pair(float x, float y, float c, float s, float& xo, float& yo) {
    xo = __builtin_fmaf(x, c, -y * s);
    yo = __builtin_fmaf(y, c, x * s);
}

__device__ __forceinline__ float bf16_word_lo(uint32_t w) { return __builtin_bit_cast(float, w << 16); }
__device__ __forceinline__ float bf16_word_hi(uint32_t w) { return __builtin_bit_cast(float, w & 0xffff0000u); }

// Rotates head-vector fragments in place: frag[s] holds dims STRIDE*s + 8*sub
// .. +7 of one row (the prefill kernels' Q^T fragments: STRIDE 16, sub = hh;
// the decode kernels' Q^T and K fragments: STRIDE 32, sub = lane/16), so with
// rd = 2 * STRIDE * NRS rotated dims the pair of dim i = STRIDE*s + 8*sub + t
// is dim i + rd/2 in frag[s + NRS], same lane and slot.  tab holds the row's
// token's (cos, sin) pairs, fp32, for i = 0 .. rd/2 - 1.
template <int NRS, int STRIDE = 16, class F>
__device__ __forceinline__ void rope_frags(F* frag, const float* tab, int sub) {
#pragma unroll
    for (int s = 0; s < NRS; ++s) {
        const f32x4* cs = reinterpret_cast<const f32x4*>(tab + 2 * (STRIDE * s + 8 * sub));
        const f32x4 c0 = cs[0], c1 = cs[1], c2 = cs[2], c3 = cs[3];  // (cos, sin) of 8 consecutive dims
        const float c[8] = {c0[0], c0[2], c1[0], c1[2], c2[0], c2[2], c3[0], c3[2]};
        const float sn[8] = {c0[1], c0[3], c1[1], c1[3], c2[1], c2[3], c3[1], c3[3]};
        u32x4 x = __builtin_bit_cast(u32x4, frag[s]), y = __builtin_bit_cast(u32x4, frag[s + NRS]);
        u32x4 xo, yo;
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            float a0, a1, b0, b1;
            rope_pair(bf16_word_lo(x[w]), bf16_word_lo(y[w]), c[2 * w], sn[2 * w], a0, b0);
            rope_pair(bf16_word_hi(x[w]), bf16_word_hi(y[w]), c[2 * w + 1], sn[2 * w + 1], a1, b1);
            xo[w] = pack_bf16x2(a0, a1);
            yo[w] = pack_bf16x2(b0, b1);
        }
        frag[s] = __builtin_bit_cast(F, xo);
        frag[s + NRS] = __builtin_bit_cast(F, yo);
    }
}

// rope_frags for the rd (a multiple of 32, at most 192) known at run time.
__device__ __forceinline__ void rope_frags_rd(bf16x8* frag, const float* tab, int rope_half, int hh) {
    switch (rope_half / 16) {
        case 1: rope_frags<1>(frag, tab, hh); break;
        case 2: rope_frags<2>(frag, tab, hh); break;
        case 3: rope_frags<3>(frag, tab, hh); break;
        case 4: rope_frags<4>(frag, tab, hh); break;
        case 5: rope_frags<5>(frag, tab, hh); break;
        case 6: rope_frags<6>(frag, tab, hh); break;
        default: break;
    }
}

// The decode layout (STRIDE 32): rd a multiple of 64, at most 192.
template <class F>
__device__ __forceinline__ void rope_frags32_rd(F* frag, const float* tab, int rope_half, int sub) {
    switch (rope_half / 32) {
        case 1: rope_frags<1, 32>(frag, tab, sub); break;
        case 2: rope_frags<2, 32>(frag, tab, sub); break;
        case 3: rope_frags<3, 32>(frag, tab, sub); break;
        default: break;
    }
}

// Orders this wave's earlier LDS writes before its later LDS reads (the
// compiler must not move accesses across it; the hardware keeps a wave's LDS
// operations in order).
// OCP E4M3 codes -> bf16, exact (an E4M3 value has at most 4 significant bits
// and an exponent inside bf16's range).  4 codes (one dword) -> 4 bf16 (two
// dwords): v_cvt_scalef32_pk_bf16_fp8 with scale 1 turns the two codes of a
// 16-bit word straight into a bf16 pair.  (The route through v_cvt_pk_f32_fp8
// and a byte permute was miscompiled here: the compiler read both floats of
// the pair from the first register.)
__device__ __forceinline__ u32x2 fp8x4_to_bf16x4(uint32_t w) {
    return u32x2{__builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)w, 1.0f, false)),
                 __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)w, 1.0f, true))};
}

// 8 codes (two dwords) -> 8 bf16 (one 16-byte operand).
__device__ __forceinline__ u32x4 fp8x8_to_bf16x8(uint32_t w0, uint32_t w1) {
    const u32x2 a = fp8x4_to_bf16x4(w0), c = fp8x4_to_bf16x4(w1);
    return u32x4{a[0], a[1], c[0], c[1]};
}

__device__ __forceinline__ void wave_lds_fence() { __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront"); }

// Raw buffer resource (gfx9-family descriptor) over `bytes` bytes at `base`:
// the hardware range check turns loads at byte offsets past the record count
// into zeros and drops such stores.
constexpr uint32_t kRsrcWord3 = 0x00020000;
typedef __amdgpu_buffer_rsrc_t rsrc_t;
__device__ __forceinline__ rsrc_t make_rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, (int)kRsrcWord3);
}

// Scheduling hint for a straight-line run of MFMAs fed from LDS: issue
// `ahead` LDS reads first, then alternate one MFMA with `per` reads, so that
// each MFMA's operands were requested several MFMAs earlier instead of right
// before it.  Only orders instructions already in the block; no code.
template <int kMfmas, int kReads, int kAhead, int kPer>
__device__ __forceinline__ void interleave_lds_mfma() {
#ifndef MIMO_NO_INTERLEAVE
    static_assert(kAhead + (kMfmas - 1) * kPer >= kReads, "reads must all be placed");
    __builtin_amdgcn_sched_group_barrier(0x100, kAhead, 0);
#pragma unroll
    for (int i = 0; i < kMfmas; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
#pragma unroll
        for (int j = 0; j < kPer; ++j)
            if (kAhead + i * kPer + j < kReads) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
#endif
}

// As interleave_lds_mfma, with kValu VALU instructions after each MFMA: the
// MFMAs of one tile run on the matrix core while the wave issues another
// tile's independent vector work in their shadow.
template <int kMfmas, int kReads, int kAhead, int kValu>
__device__ __forceinline__ void interleave_mfma_valu() {
#ifndef MIMO_NO_INTERLEAVE
    static_assert(kAhead + kMfmas - 1 >= kReads, "reads must all be placed");
    __builtin_amdgcn_sched_group_barrier(0x100, kAhead, 0);
#pragma unroll
    for (int i = 0; i < kMfmas; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        if (kAhead + i < kReads) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, kValu, 0);
    }
#endif
}

// PV MFMAs of a tile taken in two halves of kHalf MFMAs each (two transposed
// LDS reads per MFMA): the first half's 2*kHalf exps come first, then the
// first half's MFMAs with the second half's exps placed two per MFMA, and the
// reads kAhead ahead.
template <int kHalf, int kAhead>
__device__ __forceinline__ void interleave_pv_trans() {
#ifndef MIMO_NO_INTERLEAVE
    constexpr int kReads = 4 * kHalf;
    __builtin_amdgcn_sched_group_barrier(0x400, 2 * kHalf, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, kAhead, 0);
    int placed = kAhead;
#pragma unroll
    for (int i = 0; i < kHalf; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        if (placed < kReads) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
        placed += 2;
        __builtin_amdgcn_sched_group_barrier(0x400, 2, 0);
    }
#pragma unroll
    for (int i = 0; i < kHalf; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        if (placed < kReads) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
        placed += 2;
    }
#endif
}

}  // namespace mimo
