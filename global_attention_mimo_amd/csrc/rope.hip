// rope.hip -- rotary position embedding of queries and keys, in place.
//
// Operation (Hugging Face Transformers model doc "MiMo-V2-Flash",
// MiMoV2FlashConfig: rope_parameters with rope_theta; the Transformers rotary
// convention): the first rd = rotary_dim dims of each head vector x at
// position p rotate in pairs (i, i + rd/2), i < rd/2, by p * f_i with
// f_i = theta^(-2i/rd):
//   x[i]        <- x[i] cos - x[i + rd/2] sin
//   x[i + rd/2] <- x[i + rd/2] cos + x[i] sin
// and dims rd .. 191 pass through untouched.
//
// One block per token: the token's rd/2 angles p * f_i are formed and reduced
// in fp64 (p up to 2^31 times f_i <= 1 keeps every bit that fp32 would lose at
// long context; the f_i come from the host, in double), their cos/sin rounded
// to fp32 into LDS, and then the token's
// Hq + Hkv head rows are rotated in fp32, 8 pairs (two 16-byte loads) per
// thread, and written back as bf16 (round to nearest even).  Only the rotated
// dims are read and written.
#include <cmath>

#include "device_common.hpp"
#include "launch.hpp"

namespace mimo {
namespace {

constexpr int kD = 192;


using InvFreq = RopeFreq;

__global__ __launch_bounds__(256) void rope_kernel(uint16_t* __restrict__ q, uint16_t* __restrict__ k,
                                                   const int32_t* __restrict__ positions, int hq, int hkv,
                                                   const InvFreq freq, int rd) {
    __shared__ float cs[kD / 2], sn[kD / 2];
    const int64_t t = blockIdx.x;
    const int half = rd / 2;
    const int units = half / 8;  // 8 pairs per thread
    const int rows = (q ? hq : 0) + (k ? hkv : 0);
    const int total = rows * units;
    auto locate = [&](int u, u32x4*& px, u32x4*& py) {
        const int r = u / units, j = u % units;
        uint16_t* row = (q && r < hq) ? q + ((size_t)t * hq + r) * kD
                                      : k + ((size_t)t * hkv + (r - (q ? hq : 0))) * kD;
        px = reinterpret_cast<u32x4*>(row + 8 * j);
        py = reinterpret_cast<u32x4*>(row + 8 * j + half);
    };
    auto rotate = [&](int u, u32x4* px, u32x4* py, const u32x4& x, const u32x4& y) {
        const int j = u % units;
        u32x4 xo, yo;
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            const int i = 8 * j + 2 * w;
            float a0, a1, b0, b1;
            rope_pair(bf16_word_lo(x[w]), bf16_word_lo(y[w]), cs[i], sn[i], a0, b0);
            rope_pair(bf16_word_hi(x[w]), bf16_word_hi(y[w]), cs[i + 1], sn[i + 1], a1, b1);
            xo[w] = pack_bf16x2(a0, a1);
            yo[w] = pack_bf16x2(b0, b1);
        }
        *px = xo;
        *py = yo;
    };
    // This thread's first unit is loaded before the angles are formed, so the
    // memory latency and the fp64 work overlap.
    const int u0 = threadIdx.x;
    u32x4* px0 = nullptr;
    u32x4* py0 = nullptr;
    u32x4 x0 = {}, y0 = {};
    if (u0 < total) {
        locate(u0, px0, py0);
        x0 = *px0;
        y0 = *py0;
    }
    const double p = (double)positions[t];
    for (int i = threadIdx.x; i < half; i += blockDim.x) {
        double s, c;
        sincos(p * freq.f[i], &s, &c);
        cs[i] = (float)c;
        sn[i] = (float)s;
    }
    __syncthreads();
    if (u0 < total) rotate(u0, px0, py0, x0, y0);
    for (int u = u0 + blockDim.x; u < total; u += blockDim.x) {
        u32x4 *px, *py;
        locate(u, px, py);
        rotate(u, px, py, *px, *py);
    }
}

// Preparation for attention with fused RoPE: per token, the (cos, sin) pairs
// of its rd/2 angles (formed exactly as rope_kernel forms them) go to tab
// [T][rd/2][2] fp32, for the prefill kernels to rotate Q with, and the
// token's K rows are written to k_rot rotated (dims rd .. 191 copied).  A block
// serves kPrepTokens consecutive tokens.
constexpr int kPrepTokens = 8;
__global__ __launch_bounds__(256) void rope_prep_kernel(const uint16_t* __restrict__ k,
                                                        const int32_t* __restrict__ positions, int total_tokens,
                                                        int hkv, const InvFreq freq, int rd,
                                                        uint16_t* __restrict__ k_rot, float* __restrict__ tab) {
    __shared__ float cs[kPrepTokens][kD / 2], sn[kPrepTokens][kD / 2];
    const int64_t t0 = (int64_t)blockIdx.x * kPrepTokens;
    const int ntok = (int)min((int64_t)kPrepTokens, total_tokens - t0);
    const int half = rd / 2;
    const int pairs = half / 8;             // 16-byte pair units per head row
    const int per = pairs + (kD - rd) / 8;  // plus the untouched chunks
    for (int e = threadIdx.x; e < ntok * half; e += blockDim.x) {
        const int tt = e / half, i = e % half;
        double s, c;
        sincos((double)positions[t0 + tt] * freq.f[i], &s, &c);
        cs[tt][i] = (float)c;
        sn[tt][i] = (float)s;
        reinterpret_cast<f32x2*>(tab)[(size_t)(t0 + tt) * half + i] = f32x2{(float)c, (float)s};
    }
    __syncthreads();
    for (int u = threadIdx.x; u < ntok * hkv * per; u += blockDim.x) {
        const int tt = u / (hkv * per), h = (u / per) % hkv, j = u % per;
        const size_t row = ((size_t)(t0 + tt) * hkv + h) * kD;
        const u32x4* src = reinterpret_cast<const u32x4*>(k + row);
        u32x4* dst = reinterpret_cast<u32x4*>(k_rot + row);
        if (j < pairs) {
            const u32x4 x = src[j], y = src[j + pairs];
            u32x4 xo, yo;
#pragma unroll
            for (int w = 0; w < 4; ++w) {
                const int i = 8 * j + 2 * w;
                float a0, a1, b0, b1;
                rope_pair(bf16_word_lo(x[w]), bf16_word_lo(y[w]), cs[tt][i], sn[tt][i], a0, b0);
                rope_pair(bf16_word_hi(x[w]), bf16_word_hi(y[w]), cs[tt][i + 1], sn[tt][i + 1], a1, b1);
                xo[w] = pack_bf16x2(a0, a1);
                yo[w] = pack_bf16x2(b0, b1);
            }
            dst[j] = xo;
            dst[j + pairs] = yo;
        } else {
            const int c = rd / 8 + (j - pairs);
            dst[c] = src[c];
        }
    }
}

InvFreq inv_freq(double theta, int rd) { return rope_inv_freq(theta, rd); }

}  // namespace

RopeFreq rope_inv_freq(double theta, int rd) {
    RopeFreq freq{};
    for (int i = 0; i < rd / 2; ++i) freq.f[i] = std::pow(theta, -2.0 * i / rd);
    return freq;
}

hipError_t launch_rope_prep(const RopePrepArgs& a, hipStream_t stream) {
    if (a.total_tokens <= 0) return hipSuccess;
    hipLaunchKernelGGL(rope_prep_kernel, dim3((unsigned)((a.total_tokens + kPrepTokens - 1) / kPrepTokens)), dim3(256), 0,
                       stream, a.k, a.positions, a.total_tokens, a.hkv, inv_freq(a.theta, a.rotary_dim), a.rotary_dim,
                       a.k_rot, a.tab);
    return hipGetLastError();
}

hipError_t launch_rope(const RopeArgs& a, hipStream_t stream) {
    if (a.total_tokens <= 0 || a.rotary_dim == 0) return hipSuccess;
    hipLaunchKernelGGL(rope_kernel, dim3((unsigned)a.total_tokens), dim3(256), 0, stream, a.q, a.k, a.positions, a.hq,
                       a.hkv, inv_freq(a.theta, a.rotary_dim), a.rotary_dim);
    return hipGetLastError();
}

}  // namespace mimo
