// prefill_f32.hip -- bifocal causal prefill for fp32 inputs (exact fp32 path).
//
// Pages cited (title, section):
//   [BT] "Jet-Long: 具有动态双焦RoPE的高效长上下文扩展" (bittide.aicompass.dev)
//   [TW] "NVIDIA研究团队找到了让AI“看清”超长文本的新方法" (techwalker.com)
//
// One wave per (query row, head).  Scores follow the direct form of the
// pages' merge ([BT] §3.2): key j is scored with standard RoPE when
// i - j < w_local and with remapped RoPE otherwise; keys come pre-rotated
// (fp32) from the pre-pass.  64 keys per step: lane = key for the scores,
// lane = head dimension for the P V accumulation.  Everything stays fp32.
#include "internal.h"

namespace jl {

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) x = fmaxf(x, __shfl_xor(x, o));
    return x;
}
__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o);
    return x;
}

template <int D>
__global__ __launch_bounds__(64) void prefill_f32_kernel(PrefillArgs a) {
    constexpr int HALF = D / 2;
    __shared__ float qs[D], qm[D], pb[64];
    const int lane = threadIdx.x;
    const int64_t tok = blockIdx.x;
    const int head = blockIdx.y;
    const int32_t* plan = (const int32_t*)((const char*)a.ws + a.lay.plan);
    int s = 0;
    while (s + 1 < a.n_seqs && tok >= plan[(s + 1) * kPlanFields + kPlanStart]) ++s;
    const int32_t* e = plan + s * kPlanFields;
    const int32_t start = e[kPlanStart], len = e[kPlanLen], G = e[kPlanG];
    if (tok < start || tok >= (int64_t)start + len) return;
    const int32_t i = (int32_t)(tok - start);
    const bool bif = a.bifocal && G > 1;
    const int g = head / (a.Hq / a.Hkv);
    const float* q = (const float*)a.q + (tok * a.Hq + head) * D;
    if (lane < HALF) {
        const float x0 = q[lane], x1 = q[lane + HALF];
        float c, sn;
        const double rv = rope_rev(a.tab, lane);
        rope_cs(i, rv, c, sn);
        qs[lane] = x0 * c - x1 * sn;
        qs[lane + HALF] = x1 * c + x0 * sn;
        rope_cs(remap(i, G), rv, c, sn);
        qm[lane] = x0 * c - x1 * sn;
        qm[lane + HALF] = x1 * c + x0 * sn;
    }
    __syncthreads();
    const float* KS = (const float*)((const char*)a.ws + a.lay.ks32) + ((int64_t)g * a.T + start) * D;
    const float* KR = (const float*)((const char*)a.ws + a.lay.kr32) + ((int64_t)g * a.T + start) * D;
    const float* V = (const float*)a.v + (int64_t)start * a.Hkv * D + (int64_t)g * D;
    const int64_t vstride = (int64_t)a.Hkv * D;
    float m = -INFINITY, l = 0.0f, acc0 = 0.0f, acc1 = 0.0f;
    for (int32_t j0 = 0; j0 <= i; j0 += 64) {
        const int32_t j = j0 + lane;
        float sc = -INFINITY;
        if (j <= i) {
            const bool local = band(i, j, a.w_local, bif) == 1;
            const float* kr = (local ? KS : KR) + (int64_t)j * D;
            const float* qq = local ? qs : qm;
            float d0 = 0.0f;
            for (int x = 0; x < D; ++x) d0 += qq[x] * kr[x];
            sc = d0 * a.softmax_scale;
        }
        const float mn = fmaxf(m, wave_max(sc));
        const float alpha = expf(m - mn);
        const float p = expf(sc - mn);
        l = l * alpha + wave_sum(p);
        acc0 *= alpha;
        acc1 *= alpha;
        m = mn;
        pb[lane] = p;
        __syncthreads();
        const int32_t nk = min(64, i - j0 + 1);
        for (int jj = 0; jj < nk; ++jj) {
            const float pj = pb[jj];
            const float* vr = V + (int64_t)(j0 + jj) * vstride;
            acc0 += pj * vr[lane];
            if (D == 128) acc1 += pj * vr[lane + 64];
        }
        __syncthreads();
    }
    float* o = (float*)a.o + (tok * a.Hq + head) * D;
    o[lane] = acc0 / l;
    if (D == 128) o[lane + 64] = acc1 / l;
    if (lane == 0) a.lse[(int64_t)head * a.T + tok] = m + logf(l);
}

hipError_t launch_prefill_f32(const PrefillArgs& a, hipStream_t s) {
    LaunchScope scope("prefill_f32", s);
    const dim3 grid((unsigned)a.T, (unsigned)a.Hq);
    if (a.d == 128)
        hipLaunchKernelGGL(prefill_f32_kernel<128>, grid, dim3(64), 0, s, a);
    else
        hipLaunchKernelGGL(prefill_f32_kernel<64>, grid, dim3(64), 0, s, a);
    return hipGetLastError();
}

}  // namespace jl
