// stream.hip -- a read-only HBM stream: the rate at which a kernel can read a
// large buffer it touches once.  It is the measured ceiling the decode
// kernels' byte stream is compared with (they read every cache byte once).
//
// Workgroup b of 256 reads the 8 KB slabs b, b + 256, b + 512, ... of the
// buffer, four slabs in flight per thread (16-byte loads), so at every moment
// the whole grid reads one contiguous stretch of memory.  Each workgroup
// writes the wrapping uint32 sum of the words it read, which lets a caller
// check that every byte was read.
#include "internal.h"

namespace jl {

namespace {
constexpr int kSrThreads = 512;
constexpr int kSrDepth = 4;

__global__ __launch_bounds__(kSrThreads) void stream_read_kernel(const u32x4* __restrict__ src,
                                                                 int64_t n16,
                                                                 uint32_t* __restrict__ out) {
    __shared__ uint32_t part[kSrThreads / 64];
    const int64_t stride = (int64_t)gridDim.x * kSrThreads;
    int64_t i = (int64_t)blockIdx.x * kSrThreads + threadIdx.x;
    uint32_t acc = 0;
    for (; i + (kSrDepth - 1) * stride < n16; i += kSrDepth * stride) {
        u32x4 v[kSrDepth];
#pragma unroll
        for (int d = 0; d < kSrDepth; ++d) v[d] = src[i + d * stride];
#pragma unroll
        for (int d = 0; d < kSrDepth; ++d) acc += v[d][0] + v[d][1] + v[d][2] + v[d][3];
    }
    for (; i < n16; i += stride) {
        const u32x4 t = src[i];
        acc += t[0] + t[1] + t[2] + t[3];
    }
#pragma unroll
    for (int sh = 32; sh > 0; sh >>= 1) acc += __shfl_xor(acc, sh);
    if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = acc;
    __syncthreads();
    if (threadIdx.x == 0) {
        uint32_t t = 0;
#pragma unroll
        for (int w = 0; w < kSrThreads / 64; ++w) t += part[w];
        out[blockIdx.x] = t;
    }
}
}  // namespace

hipError_t launch_stream_read(const void* src, int64_t bytes, uint32_t* out, hipStream_t s) {
    LaunchScope scope("stream_read", s);
    hipLaunchKernelGGL(stream_read_kernel, dim3(kStreamReadWgs), dim3(kSrThreads), 0, s,
                       (const u32x4*)src, bytes / 16, out);
    return hipGetLastError();
}

}  // namespace jl
