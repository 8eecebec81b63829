// prefill_f32.hip -- bifocal causal prefill for fp32 inputs (exact fp32 path).
//
// Pages cited (title, section):
//   [BT] "Jet-Long: 具有动态双焦RoPE的高效长上下文扩展" (bittide.aicompass.dev)
//   [TW] "NVIDIA研究团队找到了让AI“看清”超长文本的新方法" (techwalker.com)
//
// Scores follow the direct form of the pages' merge ([BT] §3.2): key j is
// scored with standard RoPE when i - j < w_local and with remapped RoPE
// otherwise; keys come pre-rotated (fp32) from the pre-pass, queries are
// turned in the kernel.  Everything stays fp32.
#include "internal.h"

namespace jl {

// On the fp32 matrix cores (v_mfma_f32_32x32x2_f32: fp32 products, fp32
// accumulation).  A workgroup of 4 waves takes 128 query rows
// of one head of one sequence; each wave owns 32 rows.  Per 64-key tile the
// pre-rotated keys (fp32) and the values are staged in LDS; per 32-key block
// a wave forms S^T = K Q^T (k-step t pairs the d values t and t + D/2, so
// lane (n, h) keeps the query elements t + h D/2 of row n in registers),
// masks, runs an online softmax in the log2 domain and accumulates
// O^T += V^T P^T, where the probabilities already sit in the B-operand layout
// (lane (n, h), register r holds key 8 (r/4) + 4 h + r%4 of row n).  Like the
// bf16 kernel it runs a remote phase (R(f(i)) q against R(f(j)) k) and a
// local phase (R(i) q against R(j) k); a pair is scored in the phase of its
// band only.
typedef float f32x16_t __attribute__((ext_vector_type(16)));

template <int D>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2))) void prefill_f32_mfma_kernel(PrefillArgs a) {
    constexpr int HALF = D / 2;
    constexpr int ND = D / 32;   // 32-wide d blocks of O^T
    constexpr int RS = D + 4;    // LDS row stride (floats)
    constexpr float kLog2e = 1.4426950408889634f;
    __shared__ __align__(16) float ks[64 * RS];
    __shared__ __align__(16) float vs[64 * RS];
    __shared__ double rvt[HALF];  // theta_t / 2 pi, once per workgroup
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int n = lane & 31, hk = lane >> 5;
    const int sq = blockIdx.z, head = blockIdx.y;
    const int32_t* plan = (const int32_t*)((const char*)a.ws + a.lay.plan);
    const int32_t* e = plan + sq * kPlanFields;
    const int32_t start = e[kPlanStart], len = e[kPlanLen], G = e[kPlanG];
    const int32_t rb0 = (int32_t)blockIdx.x * 128;
    if (rb0 >= len) return;  // uniform per workgroup
    if (threadIdx.x < HALF) rvt[threadIdx.x] = rope_rev(a.tab, threadIdx.x);
    __syncthreads();
    const int32_t rlast = min(rb0 + 127, len - 1);     // last row of the workgroup
    const int32_t w0 = rb0 + 32 * wave;                // first row of this wave
    const int32_t row = w0 + n;                        // this lane's row
    const int32_t rowc = min(row, len - 1);
    const bool bif = a.bifocal && G > 1;
    const int g = head / (a.Hq / a.Hkv);
    const float qscale = a.softmax_scale * kLog2e;
    const float* KSg = (const float*)((const char*)a.ws + a.lay.ks32) + ((int64_t)g * a.T + start) * D;
    const float* KRg = (const float*)((const char*)a.ws + a.lay.kr32) + ((int64_t)g * a.T + start) * D;
    const float* Vg = (const float*)a.v + (int64_t)start * a.Hkv * D + (int64_t)g * D;
    const int64_t vstride = (int64_t)a.Hkv * D;

    // the phase's rotated query: lane (n, hk) turns the elements t + hk D/2
    // of row n in a rolled loop through the tile buffers (32 rows of D
    // floats per wave: waves 0, 1 in ks, waves 2, 3 in vs), then reads them
    // back into registers; the wave reads only what it wrote
    float qv[HALF];
    auto stage_q = [&](bool remapped) __attribute__((always_inline)) {
        __syncthreads();  // no wave still reads the tile buffers
        float* qst = (wave < 2 ? ks : vs) + (wave & 1) * 32 * D + n * D + HALF * hk;
        const float* q = (const float*)a.q + ((int64_t)(start + rowc) * a.Hq + head) * D;
        const int32_t pos = remapped ? remap(rowc, G) : rowc;
        for (int t = 0; t < HALF; ++t) {
            const float x0 = q[t], x1 = q[t + HALF];
            float c, sn;
            rope_cs(pos, rvt[t], c, sn);
            qst[t] = (hk ? (x1 * c + x0 * sn) : (x0 * c - x1 * sn)) * qscale;
        }
#pragma unroll
        for (int t = 0; t < HALF; ++t) qv[t] = qst[t];
    };

    float m_run = -1e30f, l_run = 0.0f;
    f32x16_t O[ND];
#pragma unroll
    for (int db = 0; db < ND; ++db) O[db] = f32x16_t{};

    // rows j0 .. j0 + 63 of the key image and of V into LDS (zeros past len)
    auto load_tile = [&](int32_t j0, const float* K) __attribute__((always_inline)) {
        constexpr int V4 = D / 4;  // float4 per row
        for (int x = threadIdx.x; x < 64 * V4; x += 256) {
            const int r = x / V4, c4 = x % V4;
            const int32_t j = j0 + r;
            float4 kk = make_float4(0.f, 0.f, 0.f, 0.f), vv = kk;
            if (j < len) {
                kk = *reinterpret_cast<const float4*>(K + (int64_t)j * D + 4 * c4);
                vv = *reinterpret_cast<const float4*>(Vg + (int64_t)j * vstride + 4 * c4);
            }
            *reinterpret_cast<float4*>(ks + r * RS + 4 * c4) = kk;
            *reinterpret_cast<float4*>(vs + r * RS + 4 * c4) = vv;
        }
    };

    // one 32-key block of the tile: keys jb .. jb + 31 (tile row offset b32)
    auto do_block = [&](int32_t jb, int b32, bool remote_phase) __attribute__((always_inline)) {
        f32x16_t S = {};
        const float* kr = ks + (b32 + n) * RS + HALF * hk;
#pragma unroll
        for (int t = 0; t < HALF; ++t)
            S = __builtin_amdgcn_mfma_f32_32x32x2f32(kr[t], qv[t], S, 0, 0, 0);
        float mx = -INFINITY;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int32_t j = jb + 8 * (r >> 2) + 4 * hk + (r & 3);
            const int bd = band(row, j, a.w_local, bif);
            const bool keep = row < len && j < len && bd != 0 &&
                              (!bif || (bd == 2) == remote_phase);
            S[r] = keep ? S[r] : -INFINITY;
            mx = fmaxf(mx, S[r]);
        }
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        const float m_new = fmaxf(m_run, mx);
        const float alpha = exp2f(m_run - m_new);
        m_run = m_new;
        float ps = 0.0f;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            S[r] = exp2f(S[r] - m_new);
            ps += S[r];
        }
        l_run = l_run * alpha + ps;
#pragma unroll
        for (int db = 0; db < ND; ++db) {
            O[db] *= alpha;
#pragma unroll
            for (int t = 0; t < 16; ++t) {
                const int key = b32 + 8 * (t >> 2) + 4 * hk + (t & 3);
                O[db] = __builtin_amdgcn_mfma_f32_32x32x2f32(vs[key * RS + 32 * db + n], S[t], O[db],
                                                            0, 0, 0);
            }
        }
    };

    // tiles [t0, t1) of one phase; every wave runs every tile (shared LDS)
    auto run_phase = [&](int32_t t0, int32_t t1, bool remote_phase, const float* K)
        __attribute__((always_inline)) {
        for (int32_t tau = t0; tau < t1; ++tau) {
            const int32_t j0 = 64 * tau;
            __syncthreads();  // the previous tile is no longer read
            load_tile(j0, K);
            __syncthreads();
#pragma unroll
            for (int b = 0; b < 2; ++b) {
                const int32_t jb = j0 + 32 * b;
                // blocks wholly after the wave's last row are causal-masked
                if (jb <= min(w0 + 31, len - 1)) do_block(jb, 32 * b, remote_phase);
            }
        }
    };

    if (bif) {
        const int32_t jr = rlast - a.w_local;  // keys j <= jr are remote for some row
        if (jr >= 0) {
            stage_q(true);
            run_phase(0, jr / 64 + 1, true, KRg);
        }
        const int32_t jl = max(rb0 - a.w_local + 1, 0);  // first key local for some row
        stage_q(false);
        run_phase(jl / 64, rlast / 64 + 1, false, KSg);
    } else {
        stage_q(false);
        run_phase(0, rlast / 64 + 1, false, KSg);
    }

    if (row >= len) return;
    const float l_tot = l_run + __shfl_xor(l_run, 32);
    const float inv = 1.0f / l_tot;
    float* o = (float*)a.o + ((int64_t)(start + row) * a.Hq + head) * D;
#pragma unroll
    for (int db = 0; db < ND; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[32 * db + 8 * (r >> 2) + 4 * hk + (r & 3)] = O[db][r] * inv;
    if (hk == 0)
        a.lse[(int64_t)head * a.T + start + row] = (m_run + log2f(l_tot)) * 0.6931471805599453f;
}

hipError_t launch_prefill_f32(const PrefillArgs& a, hipStream_t s) {
    LaunchScope scope("prefill_f32", s);
    const dim3 grid((unsigned)((a.max_seqlen + 127) / 128), (unsigned)a.Hq, (unsigned)a.n_seqs);
    if (a.d == 128)
        hipLaunchKernelGGL(prefill_f32_mfma_kernel<128>, grid, dim3(256), 0, s, a);
    else
        hipLaunchKernelGGL(prefill_f32_mfma_kernel<64>, grid, dim3(256), 0, s, a);
    return hipGetLastError();
}

}  // namespace jl
