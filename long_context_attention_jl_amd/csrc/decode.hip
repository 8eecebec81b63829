// decode.hip -- bifocal decode: one new query per sequence against a KV cache
// of standard-RoPE keys, split over key chunks, merged in LogSumExp space.
//
// Pages cited (title, section):
//   [BT] "Jet-Long: 具有动态双焦RoPE的高效长上下文扩展" (bittide.aicompass.dev)
//   [TW] "NVIDIA研究团队找到了让AI“看清”超长文本的新方法" (techwalker.com)
//
// The cache holds R(j) k_j and is never rewritten when G changes ([TW] §三).
// At read time the query is rotated to R(p) q (local keys) and R(f(p)) q --
// the pages' correction f(p) - p -- and every key older than the local
// window is turned by the correction f(j) - j in registers before its dot
// product ([BT] §3.3); keys inside the window are used as stored.
//
// Work decomposition: a workgroup owns a chunk of key positions of one
// sequence and up to 8 kv heads (one wave each).  The correction angles
// depend only on (position, pair), so the workgroup computes them once per
// 64 positions into LDS and every head's wave reuses them.  Scores and P V
// run on v_mfma_f32_16x16x4f32 with fp32 operands (decode is bound by the
// cache stream, so the matrix unit has room for fp32 and nothing is rounded
// to bf16): S^T (16 keys x 16 query heads of the GQA group) = K Q^T, then
// O (16 heads x 16 d) += P V with the probabilities used where the score
// product left them.  Each chunk writes (m, l, O) partials; a second kernel
// merges the chunks exactly (max-shifted sums).
#include "internal.h"

namespace jl {

namespace {
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr int kStage = 64;  // key positions per angle-table stage

__device__ __forceinline__ f32x4 mfma16f32(float a, float b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

template <typename TIN, int N>
__device__ __forceinline__ void load_vals(const TIN* p, float* out);

template <>
__device__ __forceinline__ void load_vals<bf16, 8>(const bf16* p, float* out) {
    const bf16x8 x = *reinterpret_cast<const bf16x8*>(p);
#pragma unroll
    for (int u = 0; u < 8; ++u) out[u] = (float)x[u];
}
template <>
__device__ __forceinline__ void load_vals<bf16, 4>(const bf16* p, float* out) {
    const bf16x4 x = *reinterpret_cast<const bf16x4*>(p);
#pragma unroll
    for (int u = 0; u < 4; ++u) out[u] = (float)x[u];
}
template <>
__device__ __forceinline__ void load_vals<float, 8>(const float* p, float* out) {
    const f32x4 x = *reinterpret_cast<const f32x4*>(p);
    const f32x4 y = *reinterpret_cast<const f32x4*>(p + 4);
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        out[u] = x[u];
        out[u + 4] = y[u];
    }
}
template <>
__device__ __forceinline__ void load_vals<float, 4>(const float* p, float* out) {
    const f32x4 x = *reinterpret_cast<const f32x4*>(p);
#pragma unroll
    for (int u = 0; u < 4; ++u) out[u] = x[u];
}

}  // namespace

// BIF = false compiles the same kernel with every bifocal step removed: it is
// plain RoPE attention over the cache, the baseline the overhead is quoted on.
template <int D, typename TIN, bool BIF>
__global__ __launch_bounds__(512) void decode_split_kernel(DecodeArgs a) {
    constexpr int HALF = D / 2;
    constexpr int SEG = HALF / 4;   // pairs per lane group
    constexpr int NST = 2 * SEG;    // k-steps of the QK^T product (d values per lane)
    constexpr int VPL = D / 16;     // d values of V per lane and key
    constexpr int TSTR = HALF + 2;  // LDS row stride of the angle table (float2)
    __shared__ float2 tab[BIF ? kStage * TSTR : 1];

    const int nw = blockDim.x >> 6;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int n = lane & 15, c = lane >> 4;
    const int b = blockIdx.z, split = blockIdx.x;
    const int kvh = blockIdx.y * nw + wave;
    const bool head_ok = kvh < a.Hkv;
    const int grp = a.Hq / a.Hkv;

    int32_t L = a.seqlens[b];
    L = L < 0 ? 0 : (L > a.max_seqlen_k ? a.max_seqlen_k : L);
    const int32_t p = L - 1;
    const int32_t G = (int32_t)group_size(L, a.w_pretrained);
    const bool bif = BIF && G > 1;
    const int32_t rem_last = p - a.w_local;  // keys j <= rem_last are remote (if bif)
    const int32_t kbeg = split * a.lay.chunk;
    const int32_t kend = min(kbeg + a.lay.chunk, L);

    float* pm = (float*)((char*)a.ws + a.lay.part_ml);
    float* po = (float*)((char*)a.ws + a.lay.part_o);
    const int64_t pbase = ((int64_t)b * a.lay.n_splits + split) * a.Hq + (int64_t)kvh * grp;

    if (kbeg >= kend) {  // empty chunk: neutral partial
        if (head_ok) {
            if (c == 0 && n < grp) {
                pm[2 * (pbase + n)] = -INFINITY;
                pm[2 * (pbase + n) + 1] = 0.0f;
            }
            for (int x = lane; x < grp * D; x += 64) po[pbase * D + x] = 0.0f;
        }
        return;
    }

    // ---- query: lane (n, c) holds head n of the group at d(c, s) ----
    // d(c, s) = SEG*c + (s % SEG) + HALF*(s / SEG); the RoPE partner of s is s + SEG.
    float qS[NST], qR[NST];
    {
        const float qscale = a.softmax_scale * kLog2e;
        const bool qok = head_ok && n < grp;
        const TIN* qp = (const TIN*)a.q + ((int64_t)b * a.Hq + kvh * grp + n) * D + SEG * c;
        const int32_t fp = remap(p, G);
#pragma unroll
        for (int s = 0; s < SEG; ++s) {
            const float x0 = qok ? (float)qp[s] : 0.0f;
            const float x1 = qok ? (float)qp[s + HALF] : 0.0f;
            float cs, sn;
            rope_cs(p, a.tab.rev[SEG * c + s], cs, sn);
            qS[s] = (x0 * cs - x1 * sn) * qscale;
            qS[s + SEG] = (x1 * cs + x0 * sn) * qscale;
            if (BIF) {
                rope_cs(fp, a.tab.rev[SEG * c + s], cs, sn);
                qR[s] = (x0 * cs - x1 * sn) * qscale;
                qR[s + SEG] = (x1 * cs + x0 * sn) * qscale;
            }
        }
    }

    const TIN* kc = (const TIN*)a.kc + (int64_t)b * a.S_max * a.Hkv * D + (int64_t)kvh * D;
    const TIN* vc = (const TIN*)a.vc + (int64_t)b * a.S_max * a.Hkv * D + (int64_t)kvh * D;
    const int64_t rstride = (int64_t)a.Hkv * D;

    float m_run = -INFINITY, l_part = 0.0f;
    f32x4 O[VPL];
#pragma unroll
    for (int x = 0; x < VPL; ++x) O[x] = f32x4{};

    for (int32_t js = kbeg; js < kend; js += kStage) {
        const bool need_tab = bif && js <= rem_last;
        if (BIF && need_tab) {
            __syncthreads();
            for (int x = threadIdx.x; x < kStage * HALF; x += blockDim.x) {
                const int r = x / HALF, t = x % HALF;
                const int32_t j = js + r;
                float cs = 1.0f, sn = 0.0f;
                if (j < kend && j <= rem_last) rope_cs((int64_t)remap(j, G) - j, a.tab.rev[t], cs, sn);
                tab[r * TSTR + t] = make_float2(cs, sn);
            }
            __syncthreads();
        }
        if (!head_ok) continue;
#pragma unroll 1
        for (int u = 0; u < kStage / 16; ++u) {
            const int32_t j0 = js + 16 * u;
            if (j0 >= kend) break;
            // keys of this lane as an A-operand row, and as output rows
            const int32_t kj = j0 + n;
            float kv[NST];
            if (kj < kend) {
                const TIN* kp = kc + (int64_t)kj * rstride + SEG * c;
                load_vals<TIN, SEG / 2>(kp, kv);
                load_vals<TIN, SEG / 2>(kp + SEG / 2, kv + SEG / 2);
                load_vals<TIN, SEG / 2>(kp + HALF, kv + SEG);
                load_vals<TIN, SEG / 2>(kp + HALF + SEG / 2, kv + SEG + SEG / 2);
            } else {
#pragma unroll
                for (int s = 0; s < NST; ++s) kv[s] = 0.0f;
            }
            const bool any_remote = bif && j0 <= rem_last;
            const bool any_local = !bif || j0 + 15 > rem_last;
            f32x4 sl = {}, sr = {};
            if (any_local) {
#pragma unroll
                for (int s = 0; s < NST; ++s) sl = mfma16f32(kv[s], qS[s], sl);
            }
            if (BIF && any_remote) {
                float kr[NST];
                const float2* tp = tab + (kj - js) * TSTR + SEG * c;
#pragma unroll
                for (int s = 0; s < SEG; ++s) {
                    const float2 cs = tp[s];
                    kr[s] = kv[s] * cs.x - kv[s + SEG] * cs.y;
                    kr[s + SEG] = kv[s + SEG] * cs.x + kv[s] * cs.y;
                }
#pragma unroll
                for (int s = 0; s < NST; ++s) sr = mfma16f32(kr[s], qR[s], sr);
            }
            float sc[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int32_t key = j0 + 4 * c + i;
                const bool remote = bif && key <= rem_last;
                sc[i] = key < kend ? (remote ? sr[i] : sl[i]) : -INFINITY;
            }
            // online softmax per query head (column n): 4 keys here, 4 lane groups
            float mx = fmaxf(fmaxf(sc[0], sc[1]), fmaxf(sc[2], sc[3]));
            mx = fmaxf(mx, __shfl_xor(mx, 16));
            mx = fmaxf(mx, __shfl_xor(mx, 32));
            const float m_new = fmaxf(m_run, mx);
            const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
            m_run = m_new;
            float pr[4];
            float ps = 0.0f;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                pr[i] = __builtin_amdgcn_exp2f(sc[i] - m_new);
                ps += pr[i];
            }
            l_part = l_part * alpha + ps;
            // O rows are query heads 4c + r: fetch their alpha from lane 4c + r
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const float ar = __shfl(alpha, 4 * c + r);
#pragma unroll
                for (int x = 0; x < VPL; ++x) O[x][r] *= ar;
            }
            // P V: instruction s' uses key 4c + s' of this lane group
#pragma unroll
            for (int sp = 0; sp < 4; ++sp) {
                const int32_t key = j0 + 4 * c + sp;
                float vv[VPL];
                if (key < kend) {
                    load_vals<TIN, VPL>(vc + (int64_t)key * rstride + VPL * n, vv);
                } else {
#pragma unroll
                    for (int x = 0; x < VPL; ++x) vv[x] = 0.0f;
                }
#pragma unroll
                for (int x = 0; x < VPL; ++x) O[x] = mfma16f32(pr[sp], vv[x], O[x]);
            }
        }
    }
    if (!head_ok) return;
    // ---- partial (m, l, unnormalised O) of this chunk ----
    float l_tot = l_part + __shfl_xor(l_part, 16);
    l_tot += __shfl_xor(l_tot, 32);
    if (c == 0 && n < grp) {
        pm[2 * (pbase + n)] = m_run;
        pm[2 * (pbase + n) + 1] = l_tot;
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const int hr = 4 * c + r;
        if (hr < grp) {
#pragma unroll
            for (int x = 0; x < VPL; ++x) po[(pbase + hr) * D + VPL * n + x] = O[x][r];
        }
    }
}

// Merge of the chunk partials: o = sum 2^(m_c - M) O_c / sum 2^(m_c - M) l_c,
// lse = (M + log2 sum ...) ln 2 -- the LogSumExp combination of [TW] §四.
template <typename TOUT>
__global__ void decode_merge_kernel(DecodeArgs a) {
    const int head = blockIdx.x, b = blockIdx.y, x = threadIdx.x;
    const float* pm = (const float*)((const char*)a.ws + a.lay.part_ml);
    const float* po = (const float*)((const char*)a.ws + a.lay.part_o);
    const int64_t base = (int64_t)b * a.lay.n_splits * a.Hq + head;
    float M = -INFINITY;
    for (int sp = 0; sp < a.lay.n_splits; ++sp) M = fmaxf(M, pm[2 * (base + (int64_t)sp * a.Hq)]);
    float Lsum = 0.0f, acc = 0.0f;
    for (int sp = 0; sp < a.lay.n_splits; ++sp) {
        const int64_t idx = base + (int64_t)sp * a.Hq;
        const float w = __builtin_amdgcn_exp2f(pm[2 * idx] - M);
        Lsum += w * pm[2 * idx + 1];
        acc += w * po[idx * a.d + x];
    }
    ((TOUT*)a.o)[((int64_t)b * a.Hq + head) * a.d + x] = (TOUT)(acc / Lsum);
    if (x == 0) a.lse[(int64_t)b * a.Hq + head] = (M + log2f(Lsum)) * kLn2;
}

template <int D, typename TIN>
static hipError_t launch_decode_t(const DecodeArgs& a, hipStream_t s) {
    const int nw = a.Hkv < 8 ? a.Hkv : 8;
    const dim3 grid(a.lay.n_splits, (a.Hkv + nw - 1) / nw, a.B);
    {
        LaunchScope scope(a.bifocal ? "decode_split" : "decode_split_plain", s);
        if (a.bifocal)
            hipLaunchKernelGGL((decode_split_kernel<D, TIN, true>), grid, dim3(64 * nw), 0, s, a);
        else
            hipLaunchKernelGGL((decode_split_kernel<D, TIN, false>), grid, dim3(64 * nw), 0, s, a);
        hipError_t err = hipGetLastError();
        if (err != hipSuccess) return err;
    }
    LaunchScope scope("decode_merge", s);
    hipLaunchKernelGGL(decode_merge_kernel<TIN>, dim3(a.Hq, a.B), dim3(D), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_decode(const DecodeArgs& a, int dtype, hipStream_t s) {
    if (dtype == 1) return a.d == 128 ? launch_decode_t<128, bf16>(a, s) : launch_decode_t<64, bf16>(a, s);
    return a.d == 128 ? launch_decode_t<128, float>(a, s) : launch_decode_t<64, float>(a, s);
}

}  // namespace jl
