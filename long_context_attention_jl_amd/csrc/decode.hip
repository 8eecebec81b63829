// decode.hip -- bifocal decode: one new query per sequence against a KV cache
// of standard-RoPE keys, split over key chunks, merged in LogSumExp space.
//
// Pages cited (title, section):
//   [BT] "Jet-Long: 具有动态双焦RoPE的高效长上下文扩展" (bittide.aicompass.dev)
//   [TW] "NVIDIA研究团队找到了让AI“看清”超长文本的新方法" (techwalker.com)
//
// The cache holds R(j) k_j and is never rewritten when G changes ([TW] §三).
// At read time the query carries the correction f(p) - p, R(f(p)) q, and every
// key older than the local window is turned by the correction f(j) - j in
// registers before its dot product ([BT] §3.3).  Keys inside the window are
// scored against the same R(f(p)) q after the query's correction is undone on
// the key side, R(p - f(p)) inverted, i.e. turned by f(p) - p: <R(p) q, K_j> =
// <R(f(p)) q, R(f(p) - p) K_j>.  One query operand then serves every key.
//
// Work decomposition: a workgroup owns a chunk of key positions of one
// sequence and up to 8 kv heads (one wave each).  The correction angles depend
// only on (position, pair), so the workgroup computes them once per 64
// positions into LDS and every head's wave reuses them.  Per 16-key tile a
// wave forms S^T (16 keys x the GQA group's query heads) = K Q^T on
// v_mfma_f32_16x16x32_bf16 with both operands split into bf16 hi + lo parts
// (hi*hi + hi*lo + lo*hi: about 16 significant bits, so the scores carry no
// visible 16-bit rounding), then accumulates P V in fp32 on the vector ALU.
// Two tiles' K and V loads stay in flight while a tile is processed.
// Each chunk writes (m, l, O) partials; a second kernel merges the chunks
// exactly (max-shifted sums).
#include "internal.h"

namespace jl {

namespace {
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr int kStage = 64;  // key positions per angle-table stage
constexpr int kTile = 16;   // keys per wave step

__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

template <typename TIN>
struct Vec8;
template <>
struct Vec8<bf16> {
    typedef bf16x8 T;
    __device__ static T load(const bf16* p) { return *reinterpret_cast<const bf16x8*>(p); }
    __device__ static float get(const T& x, int i) { return (float)x[i]; }
};
template <>
struct Vec8<float> {
    struct T {
        f32x4 a, b;
    };
    __device__ static T load(const float* p) {
        T t;
        t.a = *reinterpret_cast<const f32x4*>(p);
        t.b = *reinterpret_cast<const f32x4*>(p + 4);
        return t;
    }
    __device__ static float get(const T& x, int i) { return i < 4 ? x.a[i] : x.b[i - 4]; }
};

// DPL consecutive stored values (DPL in {1, 2, 4, 8}) kept in their storage
// type until use.
template <typename TIN, int DPL>
struct VRow {
    TIN x[DPL];
    __device__ void load(const TIN* p) {
#pragma unroll
        for (int u = 0; u < DPL; ++u) x[u] = p[u];
    }
    __device__ void zero() {
#pragma unroll
        for (int u = 0; u < DPL; ++u) x[u] = (TIN)0.0f;
    }
    __device__ float get(int u) const { return (float)x[u]; }
};
template <typename TIN>
struct VRow<TIN, 8> {
    typename Vec8<TIN>::T x;
    __device__ void load(const TIN* p) { x = Vec8<TIN>::load(p); }
    __device__ void zero() { x = typename Vec8<TIN>::T{}; }
    __device__ float get(int u) const { return Vec8<TIN>::get(x, u); }
};

}  // namespace

// BIF = false compiles the kernel with every bifocal step removed: plain RoPE
// attention over the cache, the baseline the decode overhead is quoted on.
// GQ >= Hq / Hkv is the padded GQA group (4, 8 or 16).
template <int D, typename TIN, bool BIF, int GQ>
__global__ __launch_bounds__(512) void decode_split_kernel(DecodeArgs a) {
    constexpr int HALF = D / 2;
    constexpr int NST = D / 32;          // k-steps of the QK^T product
    constexpr int DPL = (32 / GQ) < (D / 8) ? (32 / GQ) : (D / 8);  // d values per lane in PV
    constexpr int DSL = D / DPL;         // lanes per key row in PV
    constexpr int KSUB = 64 / DSL;       // keys processed side by side in PV
    constexpr int TSTR = HALF + 2;       // LDS row stride of the angle table (float2)
    static_assert(KSUB >= 1 && kTile % KSUB == 0, "PV lane split");
    __shared__ float2 tab[BIF ? kStage * TSTR : 1];
    __shared__ float pbuf[8][kTile][16];  // per wave: p[key][query column]
    __shared__ float abuf[8][16];         // per wave: alpha per query column

    const int nw = blockDim.x >> 6;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
    const int n = lane & 15, c = lane >> 4;      // QK^T roles: column n, lane group c
    const int ks = lane / DSL, ds = lane % DSL;  // PV roles: key subset, d slice
    const int b = blockIdx.z, split = blockIdx.x;
    const int kvh = blockIdx.y * nw + wave;
    const bool head_ok = kvh < a.Hkv;
    const int grp = a.Hq / a.Hkv;

    int32_t L = a.seqlens[b];
    L = L < 0 ? 0 : (L > a.max_seqlen_k ? a.max_seqlen_k : L);
    const int32_t p = L - 1;
    const int32_t G = (int32_t)group_size(L, a.w_pretrained);
    const bool bif = BIF && G > 1;
    const int32_t fp = remap(p, G);
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

    // ---- query operand: R(f(p)) q (or R(p) q without bifocal), scaled by
    // softmax_scale * log2(e), split into bf16 hi + lo; lane (n, c) holds
    // head n of the group at d = 32 s + 8 c + u.
    bf16x8 Qh[NST], Ql[NST];
    {
        const float qscale = a.softmax_scale * kLog2e;
        const bool qok = head_ok && n < grp;
        const TIN* qp = (const TIN*)a.q + ((int64_t)b * a.Hq + kvh * grp + n) * D + 8 * c;
        const int32_t qpos = bif ? fp : p;
#pragma unroll
        for (int s = 0; s < NST / 2; ++s) {
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                const float x0 = qok ? (float)qp[32 * s + u] : 0.0f;
                const float x1 = qok ? (float)qp[32 * s + u + HALF] : 0.0f;
                float cs, sn;
                rope_cs(qpos, rope_rev(a.tab, 32 * s + 8 * c + u), cs, sn);
                const float y0 = (x0 * cs - x1 * sn) * qscale;
                const float y1 = (x1 * cs + x0 * sn) * qscale;
                Qh[s][u] = (bf16)y0;
                Ql[s][u] = (bf16)(y0 - (float)Qh[s][u]);
                Qh[s + NST / 2][u] = (bf16)y1;
                Ql[s + NST / 2][u] = (bf16)(y1 - (float)Qh[s + NST / 2][u]);
            }
        }
    }

    const TIN* kc = (const TIN*)a.kc + (int64_t)b * a.S_max * a.Hkv * D + (int64_t)kvh * D;
    const TIN* vc = (const TIN*)a.vc + (int64_t)b * a.S_max * a.Hkv * D + (int64_t)kvh * D;
    const int64_t rstride = (int64_t)a.Hkv * D;

    // register-staged tile loads (zero beyond the chunk)
    typedef typename Vec8<TIN>::T KV8;
    KV8 kbuf[NST];
    VRow<TIN, DPL> vbuf[kTile / KSUB];
    auto load_tile = [&](int32_t j0) {
        const int32_t kj = j0 + n;
        const bool okk = kj < kend;
#pragma unroll
        for (int s = 0; s < NST; ++s) {
            if (okk) kbuf[s] = Vec8<TIN>::load(kc + (int64_t)kj * rstride + 32 * s + 8 * c);
            else kbuf[s] = KV8{};
        }
#pragma unroll
        for (int r = 0; r < kTile / KSUB; ++r) {
            const int32_t key = j0 + KSUB * r + ks;
            if (key < kend) vbuf[r].load(vc + (int64_t)key * rstride + DPL * ds);
            else vbuf[r].zero();
        }
    };

    float m_run = -INFINITY, l_part = 0.0f;
    float O[GQ][DPL];
#pragma unroll
    for (int h = 0; h < GQ; ++h)
#pragma unroll
        for (int u = 0; u < DPL; ++u) O[h][u] = 0.0f;

    // one 16-key tile: scores, online softmax, P V
    auto process = [&](int32_t j0, int32_t js, const KV8* kcur, const VRow<TIN, DPL>* vcur) {
        // ---- S^T = K Q^T with hi/lo operands ----
        f32x4 sacc = {};
        if (BIF && bif) {
            const float2* tp = tab + (j0 + n - js) * TSTR + 8 * c;
#pragma unroll
            for (int s = 0; s < NST / 2; ++s) {
                bf16x8 h0, l0, h1, l1;
#pragma unroll
                for (int x = 0; x < 8; ++x) {
                    const float2 cs = tp[32 * s + x];
                    const float k0 = Vec8<TIN>::get(kcur[s], x);
                    const float k1 = Vec8<TIN>::get(kcur[s + NST / 2], x);
                    const float y0 = k0 * cs.x - k1 * cs.y;
                    const float y1 = k1 * cs.x + k0 * cs.y;
                    h0[x] = (bf16)y0;
                    l0[x] = (bf16)(y0 - (float)h0[x]);
                    h1[x] = (bf16)y1;
                    l1[x] = (bf16)(y1 - (float)h1[x]);
                }
                sacc = mfma16(h0, Qh[s], sacc);
                sacc = mfma16(h0, Ql[s], sacc);
                sacc = mfma16(l0, Qh[s], sacc);
                sacc = mfma16(h1, Qh[s + NST / 2], sacc);
                sacc = mfma16(h1, Ql[s + NST / 2], sacc);
                sacc = mfma16(l1, Qh[s + NST / 2], sacc);
            }
        } else if constexpr (sizeof(TIN) == 2) {
            // stored bf16 keys are exact MFMA operands
#pragma unroll
            for (int s = 0; s < NST; ++s) {
                sacc = mfma16(kcur[s], Qh[s], sacc);
                sacc = mfma16(kcur[s], Ql[s], sacc);
            }
        } else {
#pragma unroll
            for (int s = 0; s < NST; ++s) {
                bf16x8 h0, l0;
#pragma unroll
                for (int x = 0; x < 8; ++x) {
                    const float k0 = Vec8<TIN>::get(kcur[s], x);
                    h0[x] = (bf16)k0;
                    l0[x] = (bf16)(k0 - (float)h0[x]);
                }
                sacc = mfma16(h0, Qh[s], sacc);
                sacc = mfma16(h0, Ql[s], sacc);
                sacc = mfma16(l0, Qh[s], sacc);
            }
        }
        // ---- online softmax per query column n (keys 4c + i here).  The
        // running max is only raised when a score exceeds it by more than
        // 2^8 (log2 units): the partial sums stay exact relative to whatever
        // max they use, and most tiles then skip rescaling O.
        float sc[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) sc[i] = (j0 + 4 * c + i < kend) ? sacc[i] : -INFINITY;
        float mx = fmaxf(fmaxf(sc[0], sc[1]), fmaxf(sc[2], sc[3]));
        mx = fmaxf(mx, __shfl_xor(mx, 16));
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        const bool raise = mx > m_run + 8.0f;
        float alpha = 1.0f;
        if (raise) {
            alpha = __builtin_amdgcn_exp2f(m_run - mx);
            m_run = mx;
        }
        float ps = 0.0f;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float pv = __builtin_amdgcn_exp2f(sc[i] - m_run);
            ps += pv;
            pbuf[wave][4 * c + i][n] = pv;
        }
        l_part = l_part * alpha + ps;
        const bool any_raise = __any(raise);
        if (any_raise && c == 0) abuf[wave][n] = alpha;
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        // ---- O[h][d] = alpha_h O[h][d] + sum_keys p[key][h] V[key][d] ----
        if (any_raise) {
#pragma unroll
            for (int h = 0; h < GQ; ++h) {
                const float ah = abuf[wave][h];
#pragma unroll
                for (int x = 0; x < DPL; ++x) O[h][x] *= ah;
            }
        }
#pragma unroll
        for (int r = 0; r < kTile / KSUB; ++r) {
            const float* prow = &pbuf[wave][KSUB * r + ks][0];
#pragma unroll
            for (int h = 0; h < GQ; ++h) {
                const float ph = prow[h];
#pragma unroll
                for (int x = 0; x < DPL; ++x) O[h][x] += ph * vcur[r].get(x);
            }
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    };

    // two tiles in flight: tile t is staged in buffer t & 1
    KV8 kb1[NST];
    VRow<TIN, DPL> vb1[kTile / KSUB];
    if (head_ok) {
        load_tile(kbeg);
#pragma unroll
        for (int s = 0; s < NST; ++s) kb1[s] = kbuf[s];
#pragma unroll
        for (int r = 0; r < kTile / KSUB; ++r) vb1[r] = vbuf[r];
        // kb1/vb1 now hold tile 0; kbuf/vbuf receive tile 1
        if (kbeg + kTile < kend) load_tile(kbeg + kTile);
    }
    for (int32_t js = kbeg; js < kend; js += kStage) {
        if (BIF && bif) {
            // angle table: remote keys f(j) - j, local keys f(p) - p
            __syncthreads();
            for (int x = threadIdx.x; x < kStage * HALF; x += blockDim.x) {
                const int r = x / HALF, t = x % HALF;
                const int32_t j = js + r;
                float cs = 1.0f, sn = 0.0f;
                if (j < kend) {
                    const int64_t ang = j <= rem_last ? (int64_t)remap(j, G) - j : (int64_t)fp - p;
                    rope_cs_hw(ang, rope_rev(a.tab, t), cs, sn);
                }
                tab[r * TSTR + t] = make_float2(cs, sn);
            }
            __syncthreads();
        }
        if (!head_ok) continue;
#pragma unroll
        for (int u = 0; u < kStage / kTile; ++u) {
            const int32_t j0 = js + kTile * u;
            if (j0 < kend) {
                // even tiles live in kb1/vb1, odd ones in kbuf/vbuf; after use the
                // buffer is refilled with the tile two steps ahead
                KV8 kcur[NST];
                VRow<TIN, DPL> vcur[kTile / KSUB];
                if ((u & 1) == 0) {
#pragma unroll
                    for (int s = 0; s < NST; ++s) kcur[s] = kb1[s];
#pragma unroll
                    for (int r = 0; r < kTile / KSUB; ++r) vcur[r] = vb1[r];
                } else {
#pragma unroll
                    for (int s = 0; s < NST; ++s) kcur[s] = kbuf[s];
#pragma unroll
                    for (int r = 0; r < kTile / KSUB; ++r) vcur[r] = vbuf[r];
                }
                if (j0 + 2 * kTile < kend) {
                    if ((u & 1) == 0) {
                        // load into kbuf/vbuf via a temporary swap
                        KV8 tk[NST];
                        VRow<TIN, DPL> tv[kTile / KSUB];
#pragma unroll
                        for (int s = 0; s < NST; ++s) tk[s] = kbuf[s];
#pragma unroll
                        for (int r = 0; r < kTile / KSUB; ++r) tv[r] = vbuf[r];
                        load_tile(j0 + 2 * kTile);
#pragma unroll
                        for (int s = 0; s < NST; ++s) {
                            kb1[s] = kbuf[s];
                            kbuf[s] = tk[s];
                        }
#pragma unroll
                        for (int r = 0; r < kTile / KSUB; ++r) {
                            vb1[r] = vbuf[r];
                            vbuf[r] = tv[r];
                        }
                    } else {
                        load_tile(j0 + 2 * kTile);
                    }
                }
                process(j0, js, kcur, vcur);
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
    // sum the KSUB key subsets (lanes ds, ds + DSL, ...)
#pragma unroll
    for (int off = DSL; off < 64; off <<= 1)
#pragma unroll
        for (int h = 0; h < GQ; ++h)
#pragma unroll
            for (int x = 0; x < DPL; ++x) O[h][x] += __shfl_xor(O[h][x], off);
    if (ks == 0) {
#pragma unroll
        for (int h = 0; h < GQ; ++h)
            if (h < grp) {
#pragma unroll
                for (int x = 0; x < DPL; ++x) po[(pbase + h) * D + DPL * ds + x] = O[h][x];
            }
    }
}

// Merge of the chunk partials: o = sum 2^(m_c - M) O_c / sum 2^(m_c - M) l_c,
// lse = (M + log2 sum ...) ln 2 -- the LogSumExp combination of [TW] §四.
// Workgroup (head, sequence, 32-wide slice of d) with 256 threads = 32 d
// values x 8 chunk groups; chunk g, g + 8, ... are summed by one thread and
// the 8 groups combined through LDS.
template <typename TOUT>
__global__ __launch_bounds__(256) void decode_merge_kernel(DecodeArgs a) {
    __shared__ float red[256];
    __shared__ float accs[8][33];
    const int head = blockIdx.x, b = blockIdx.y, tid = threadIdx.x;
    const int x = 32 * blockIdx.z + (tid & 31), grp8 = tid >> 5;
    const float* pm = (const float*)((const char*)a.ws + a.lay.part_ml);
    const float* po = (const float*)((const char*)a.ws + a.lay.part_o);
    const int64_t base = (int64_t)b * a.lay.n_splits * a.Hq + head;
    const int ns = a.lay.n_splits;
    float M = -INFINITY;
    for (int sp = tid; sp < ns; sp += 256) M = fmaxf(M, pm[2 * (base + (int64_t)sp * a.Hq)]);
    red[tid] = M;
    __syncthreads();
    for (int o = 128; o > 0; o >>= 1) {
        if (tid < o) red[tid] = fmaxf(red[tid], red[tid + o]);
        __syncthreads();
    }
    M = red[0];
    __syncthreads();
    float ls = 0.0f;
    for (int sp = tid; sp < ns; sp += 256) {
        const int64_t idx = base + (int64_t)sp * a.Hq;
        ls += __builtin_amdgcn_exp2f(pm[2 * idx] - M) * pm[2 * idx + 1];
    }
    red[tid] = ls;
    float acc = 0.0f;
#pragma unroll 4
    for (int sp = grp8; sp < ns; sp += 8) {
        const int64_t idx = base + (int64_t)sp * a.Hq;
        acc += __builtin_amdgcn_exp2f(pm[2 * idx] - M) * po[idx * a.d + x];
    }
    accs[grp8][tid & 31] = acc;
    __syncthreads();
    for (int o = 128; o > 0; o >>= 1) {
        if (tid < o) red[tid] += red[tid + o];
        __syncthreads();
    }
    const float Lsum = red[0];
    if (grp8 == 0) {
        float tot = 0.0f;
#pragma unroll
        for (int q = 0; q < 8; ++q) tot += accs[q][tid & 31];
        ((TOUT*)a.o)[((int64_t)b * a.Hq + head) * a.d + x] = (TOUT)(tot / Lsum);
        if (x == 0) a.lse[(int64_t)b * a.Hq + head] = (M + log2f(Lsum)) * kLn2;
    }
}

template <int D, typename TIN, int GQ>
static hipError_t launch_decode_g(const DecodeArgs& a, hipStream_t s) {
    const int nw = a.Hkv < 8 ? a.Hkv : 8;
    const dim3 grid(a.lay.n_splits, (a.Hkv + nw - 1) / nw, a.B);
    LaunchScope scope(a.bifocal ? "decode_split" : "decode_split_plain", s);
    if (a.bifocal)
        hipLaunchKernelGGL((decode_split_kernel<D, TIN, true, GQ>), grid, dim3(64 * nw), 0, s, a);
    else
        hipLaunchKernelGGL((decode_split_kernel<D, TIN, false, GQ>), grid, dim3(64 * nw), 0, s, a);
    return hipGetLastError();
}

template <int D, typename TIN>
static hipError_t launch_decode_t(const DecodeArgs& a, hipStream_t s) {
    const int grp = a.Hq / a.Hkv;
    hipError_t err;
    if (grp <= 4) err = launch_decode_g<D, TIN, 4>(a, s);
    else if (grp <= 8) err = launch_decode_g<D, TIN, 8>(a, s);
    else err = launch_decode_g<D, TIN, 16>(a, s);
    if (err != hipSuccess) return err;
    LaunchScope scope("decode_merge", s);
    hipLaunchKernelGGL(decode_merge_kernel<TIN>, dim3(a.Hq, a.B, D / 32), dim3(256), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_decode(const DecodeArgs& a, int dtype, hipStream_t s) {
    if (dtype == 1) return a.d == 128 ? launch_decode_t<128, bf16>(a, s) : launch_decode_t<64, bf16>(a, s);
    return a.d == 128 ? launch_decode_t<128, float>(a, s) : launch_decode_t<64, float>(a, s);
}

}  // namespace jl
