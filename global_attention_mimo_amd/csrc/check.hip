// check.hip -- check mode: a pass over a call's device-resident arguments
// (check_rules.hpp) enqueued ahead of the call's own kernels.
//
// Each device holds two words: [0] sticky, the OR of every violation found
// since it was last cleared; [1] the bits of the latest check.  A check is a
// one-thread kernel that clears word [1] followed by the rule pass, whose
// workgroups OR their bits into both words.
#include <hip/hip_runtime.h>

#include <mutex>

#include "check_rules.hpp"
#include "launch.hpp"

// In host code this name is a host-side stand-in for the device array; host
// code uses the address check_word_ptr() looks up per device.
static __device__ __attribute__((aligned(16))) uint32_t check_word[4];

namespace mimo {
namespace {

constexpr int kMaxDevices = 64;
constexpr int kThreads = 256;
constexpr long long kMaxBlocks = 1024;
std::mutex g_mu;
uint32_t* g_word[kMaxDevices] = {};

hipError_t check_word_ptr(uint32_t** out) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_mu);
    if (!g_word[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(check_word));
        if (e != hipSuccess) return e;
        if (!p) return hipErrorInvalidSymbol;
        g_word[dev] = static_cast<uint32_t*>(p);
    }
    *out = g_word[dev];
    return hipSuccess;
}

__global__ void check_begin_kernel(uint32_t* word) { word[1] = 0; }

__global__ __launch_bounds__(kThreads) void check_kernel(CheckArgs a, uint32_t* word) {
    __shared__ uint32_t found;
    if (threadIdx.x == 0) found = 0;
    __syncthreads();
    const long long nt = (long long)gridDim.x * kThreads;
    const uint32_t f = check_rules(a, (long long)blockIdx.x * kThreads + threadIdx.x, nt);
    if (f) atomicOr(&found, f);
    __syncthreads();
    if (threadIdx.x == 0 && found) {
        atomicOr(&word[0], found);
        atomicOr(&word[1], found);
    }
}

}  // namespace

hipError_t run_check(const CheckArgs& a, hipStream_t stream, bool* gated, uint32_t* bits) {
    *gated = false;
    *bits = 0;
    uint32_t* word = nullptr;
    hipError_t e = check_word_ptr(&word);
    if (e != hipSuccess) return e;
    long long work = a.n_seqs;
    if (a.batch > work) work = a.batch;
    if (a.pages.table && (long long)a.batch * a.pages.max_blocks > work) work = (long long)a.batch * a.pages.max_blocks;
    if (a.hq > work) work = a.hq;
    long long blocks = (work + kThreads - 1) / kThreads;
    blocks = blocks < 1 ? 1 : (blocks > kMaxBlocks ? kMaxBlocks : blocks);
    hipLaunchKernelGGL(check_begin_kernel, dim3(1), dim3(1), 0, stream, word);
    hipLaunchKernelGGL(check_kernel, dim3((unsigned)blocks), dim3(kThreads), 0, stream, a, word);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
    if ((e = hipStreamIsCapturing(stream, &cap)) != hipSuccess) return e;
    if (cap != hipStreamCaptureStatusNone) return hipSuccess;
    uint32_t got = 0;
    if ((e = hipMemcpyAsync(&got, word + 1, sizeof got, hipMemcpyDeviceToHost, stream)) != hipSuccess) return e;
    if ((e = hipStreamSynchronize(stream)) != hipSuccess) return e;
    *gated = true;
    *bits = got;
    return hipSuccess;
}

hipError_t check_flags(uint32_t* bits, bool clear) {
    uint32_t* word = nullptr;
    hipError_t e = check_word_ptr(&word);
    if (e != hipSuccess) return e;
    if ((e = hipMemcpy(bits, word, sizeof *bits, hipMemcpyDeviceToHost)) != hipSuccess) return e;
    if (clear) {
        const uint32_t zero[2] = {0, 0};
        e = hipMemcpy(word, zero, sizeof zero, hipMemcpyHostToDevice);
    }
    return e;
}

}  // namespace mimo
