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

__device__ __forceinline__ float bf_lo(uint32_t w) { return __builtin_bit_cast(float, w << 16); }
__device__ __forceinline__ float bf_hi(uint32_t w) { return __builtin_bit_cast(float, w & 0xffff0000u); }

// The frequencies f_i = theta^(-2i/rd), formed once on the host in double.
struct InvFreq {
    double f[kD / 2];
};

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
            const float x0 = bf_lo(x[w]), x1 = bf_hi(x[w]), y0 = bf_lo(y[w]), y1 = bf_hi(y[w]);
            xo[w] = pack_bf16x2(__builtin_fmaf(x0, cs[i], -y0 * sn[i]), __builtin_fmaf(x1, cs[i + 1], -y1 * sn[i + 1]));
            yo[w] = pack_bf16x2(__builtin_fmaf(y0, cs[i], x0 * sn[i]), __builtin_fmaf(y1, cs[i + 1], x1 * sn[i + 1]));
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

}  // namespace

hipError_t launch_rope(const RopeArgs& a, hipStream_t stream) {
    if (a.total_tokens <= 0 || a.rotary_dim == 0) return hipSuccess;
    InvFreq freq{};
    for (int i = 0; i < a.rotary_dim / 2; ++i) freq.f[i] = std::pow(a.theta, -2.0 * i / a.rotary_dim);
    hipLaunchKernelGGL(rope_kernel, dim3((unsigned)a.total_tokens), dim3(256), 0, stream, a.q, a.k, a.positions, a.hq,
                       a.hkv, freq, a.rotary_dim);
    return hipGetLastError();
}

}  // namespace mimo
