// libmnb_probe: the benchmark's achievable-bandwidth control arm (declared in
// include/mnb_probe.h).  Not part of libmnb.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "mnb_probe.h"

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 512;
constexpr int kUnroll = 8;          // 16-byte loads in flight per thread
constexpr uint32_t kMagic = 0x9E3779B9u;

// Grid-stride over 16-byte pieces, kUnroll pieces per thread per iteration
// (consecutive threads read consecutive pieces); the tail is read piecewise.
__global__ __launch_bounds__(kThreads) void stream_read_kernel(const u32x4* __restrict__ buf, int64_t pieces,
                                                               uint32_t* __restrict__ sink) {
    const int64_t stride = (int64_t)gridDim.x * kThreads;
    const int64_t full = pieces / (stride * kUnroll) * (stride * kUnroll);
    uint32_t acc = 0;
    int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    for (; i < full; i += stride * kUnroll) {
        u32x4 v[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; u++) v[u] = __builtin_nontemporal_load(buf + i + u * stride);
#pragma unroll
        for (int u = 0; u < kUnroll; u++) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
    }
    for (int64_t j = full + (int64_t)blockIdx.x * kThreads + threadIdx.x; j < pieces; j += stride) {
        const u32x4 v = __builtin_nontemporal_load(buf + j);
        acc ^= v.x ^ v.y ^ v.z ^ v.w;
    }
    if (acc == kMagic) sink[threadIdx.x & 1023] = acc;
}

}  // namespace

extern "C" int mnb_probe_stream_read(const void* buf, size_t bytes, uint32_t* sink, void* stream) {
    if (!buf || !sink || bytes == 0 || bytes % 16 != 0 || (reinterpret_cast<uintptr_t>(buf) & 15) != 0) return -1;
    int dev = 0, cus = 256;
    if (hipGetDevice(&dev) == hipSuccess) {
        int c = 0;
        if (hipDeviceGetAttribute(&c, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && c > 0) cus = c;
    }
    const int64_t pieces = (int64_t)(bytes / 16);
    int64_t blocks = (int64_t)cus * 4;
    const int64_t need = (pieces + kThreads - 1) / kThreads;
    if (blocks > need) blocks = need;
    hipLaunchKernelGGL(stream_read_kernel, dim3((unsigned)blocks), dim3(kThreads), 0,
                       static_cast<hipStream_t>(stream), static_cast<const u32x4*>(buf), pieces, sink);
    return hipGetLastError() == hipSuccess ? 0 : -5;
}
