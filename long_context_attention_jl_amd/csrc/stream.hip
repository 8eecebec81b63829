// stream.hip -- two measurement aids.
//
// A read-only HBM stream: the rate at which a kernel can read a large buffer
// it touches once.  It is the measured ceiling the decode kernels' byte
// stream is compared with (they read every cache byte once).
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
constexpr int kMsThreads = 512;

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

// A matrix-core stream: 32x32x16 fp16 MFMAs and nothing else, on operands the
// caller provides.  The prefill kernel's matrix work runs on the same
// instruction.  The chip's engine clock is power-limited, and the operands'
// switching activity is part of the power, so the rate this stream sustains
// depends on the data; timing it on operands drawn like the prefill's gives
// the matrix-core rate those data allow.
//
// 256 workgroups of 8 waves (two per SIMD, one workgroup per compute unit).
// Thread t of workgroup b holds the 16 fp16 x 8 vectors at
// operands[(b * 512 + t) * 16 ...] as eight (A, B) pairs and runs four
// independent accumulator chains of 8 MFMAs per iteration; it writes the sum
// of its 64 accumulator elements to out[b * 512 + t].
__global__ __launch_bounds__(kMsThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
void mfma_stream_kernel(const f16x8* __restrict__ ops, int32_t iters, float* __restrict__ out) {
    const int64_t t = (int64_t)blockIdx.x * kMsThreads + threadIdx.x;
    f16x8 a[8], b[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        a[i] = ops[t * 16 + i];
        b[i] = ops[t * 16 + 8 + i];
    }
    f32x16 c0 = {}, c1 = {}, c2 = {}, c3 = {};
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            c0 = __builtin_amdgcn_mfma_f32_32x32x16_f16(a[k], b[k], c0, 0, 0, 0);
            c1 = __builtin_amdgcn_mfma_f32_32x32x16_f16(b[(k + 3) & 7], a[(k + 5) & 7], c1, 0, 0, 0);
            c2 = __builtin_amdgcn_mfma_f32_32x32x16_f16(a[(k + 1) & 7], b[(k + 6) & 7], c2, 0, 0, 0);
            c3 = __builtin_amdgcn_mfma_f32_32x32x16_f16(b[(k + 2) & 7], a[(k + 4) & 7], c3, 0, 0, 0);
        }
    }
    float r = 0.0f;
#pragma unroll
    for (int i = 0; i < 16; ++i) r += (c0[i] + c1[i]) + (c2[i] + c3[i]);
    out[t] = r;
}

hipError_t launch_mfma_stream(const void* operands, int32_t iters, float* out, hipStream_t s) {
    LaunchScope scope("mfma_stream", s);
    hipLaunchKernelGGL(mfma_stream_kernel, dim3(kMfmaStreamWgs), dim3(kMsThreads), 0, s,
                       (const f16x8*)operands, iters, out);
    return hipGetLastError();
}

hipError_t launch_stream_read(const void* src, int64_t bytes, uint32_t* out, hipStream_t s) {
    LaunchScope scope("stream_read", s);
    hipLaunchKernelGGL(stream_read_kernel, dim3(kStreamReadWgs), dim3(kSrThreads), 0, s,
                       (const u32x4*)src, bytes / 16, out);
    return hipGetLastError();
}

}  // namespace jl
