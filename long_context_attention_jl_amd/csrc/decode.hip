// decode.hip -- bifocal decode: one new query per sequence against a KV cache
// of standard-RoPE keys, split over key chunks, merged in LogSumExp space.
//
// Pages cited (title, section):
//   [BT] "Jet-Long: 具有动态双焦RoPE的高效长上下文扩展" (bittide.aicompass.dev)
//   [TW] "NVIDIA研究团队找到了让AI“看清”超长文本的新方法" (techwalker.com)
//
// The cache holds R(j) k_j and is never rewritten when G changes ([TW] §三).
// At read time a key older than the local window is scored as
// <R(f(p)) q, R(f(j) - j) K_j>: the query carries the correction f(p) - p and
// the key the correction f(j) - j, applied in registers ([BT] §3.3).  Keys
// inside the window are scored as <R(p) q, K_j> on the stored values.
//
// Work decomposition: a workgroup owns a set of key positions of one
// sequence (a chunk, or for the bf16 kernel on flat caches every n_splits-th
// stage) and a group of kv heads (one wave each); each workgroup writes
// (m, l, O) partials and a second kernel merges them exactly (max-shifted
// sums).  Two split kernels:
//  - fp32 caches (decode_split_kernel, up to 4 kv heads per workgroup): per
//    16-key tile a wave forms S^T = K Q^T on v_mfma_f32_16x16x32_bf16 with the
//    query and the rotated keys split into bf16 hi + lo parts (about 16
//    significant bits), then accumulates P V in fp32 on the vector ALU;
//  - bf16 and fp8 caches (decode_split_bf16_kernel, up to 8 kv heads): QK^T on
//    fp16 MFMA, P V on MFMA through LDS; described above that kernel.
#include "internal.h"

namespace jl {

namespace {
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr int kStage = 64;  // key positions per angle-table stage
constexpr int kTile = 16;   // keys per wave step
constexpr int kDecodeWaves = 4;  // fp32 kernel: waves (kv heads) per workgroup
constexpr int kStageB = kDecodeStageB;  // bf16 kernel: positions per stage (three tiles)
constexpr int kWavesB = 8;       // bf16 kernel: waves (kv heads) per workgroup

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

// O^T-style P V product: A = P^T (16 query columns x 16 keys), B = V (16 keys
// x 16 d), both bf16
__device__ __forceinline__ f32x4 mfma16k16(s16x4 a, s16x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
}


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

// N (1 or 2) consecutive stored values loaded as one vector, kept in their
// storage type until use.
template <typename TIN, int N>
struct VSmall;
template <>
struct VSmall<bf16, 2> {
    bf16x2 x;
    __device__ void load(const bf16* p) { x = *reinterpret_cast<const bf16x2*>(p); }
    __device__ void zero() { x = bf16x2{}; }
    __device__ float get(int u) const { return (float)x[u]; }
};
template <>
struct VSmall<bf16, 1> {
    bf16 x;
    __device__ void load(const bf16* p) { x = *p; }
    __device__ void zero() { x = (bf16)0.0f; }
    __device__ float get(int) const { return (float)x; }
};
template <>
struct VSmall<float, 2> {
    float2 x;
    __device__ void load(const float* p) { x = *reinterpret_cast<const float2*>(p); }
    __device__ void zero() { x = make_float2(0.0f, 0.0f); }
    __device__ float get(int u) const { return u ? x.y : x.x; }
};
template <>
struct VSmall<float, 1> {
    float x;
    __device__ void load(const float* p) { x = *p; }
    __device__ void zero() { x = 0.0f; }
    __device__ float get(int) const { return x; }
};

}  // namespace

// BIF = false compiles the kernel with every bifocal step removed: plain RoPE
// attention over the cache, the baseline the decode overhead is quoted on.
// GQ >= Hq / Hkv is the padded GQA group (4, 8 or 16).
//
// Remote keys.  Within a stage of 64 positions starting at js, the key
// correction angle is f(j) - j = (f(js) - js) - u_j with
// u_j = (j - js) - (f(j) - f(js)) in [0, 64).  The score
//   <R(f(p)) q, R(f(j) - j) K_j> = <R(f(p) - f(js) + js) q, R(-u_j) K_j>
// so each wave turns its query once per stage and every key by a small angle
// -u_j theta_t read from a table built once per workgroup: no per-stage
// table, no workgroup barrier in the key loop.  Local keys are scored against
// R(p) q directly on the stored (exact) cache values.
//
// Lanes.  Scores S^T = K Q^T come from v_mfma_f32_16x16x32_bf16: lane
// (n, c) = (lane % 16, lane / 16) feeds key n of the tile and holds the scores
// of keys 4c..4c+3 for query column n.  With GQ <= 8 the query's bf16 hi part
// sits in columns [0, GQ) and its lo part in [GQ, 2 GQ) of one operand, so one
// product gives both and a lane swap adds them.  For P V each lane owns D/64
// consecutive d of every head and walks all 16 keys of the tile.
template <int D, typename TIN, bool BIF, int GQ>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(sizeof(TIN) == 2 ? 3 : 2)))
void decode_split_kernel(DecodeArgs a) {
    constexpr int HALF = D / 2;
    constexpr int NST = D / 32;          // k-steps of the QK^T product
    constexpr int NH = NST / 2;          // k-steps per RoPE half
    constexpr int DPL = D / 64;          // d values per lane in P V
    constexpr bool PACK = GQ <= 8;       // hi and lo query parts in one operand
    constexpr int TSTR = HALF + 2;       // LDS row stride of the angle table (float2)
    __shared__ float2 tab[BIF ? kStage * TSTR : 1];  // R(-u theta_t): (cos, sin)
    __shared__ double revs[HALF];                    // theta_t / 2 pi
    __shared__ float pbuf[kDecodeWaves][kTile][16];  // per wave: p[key][query column]
    __shared__ float abuf[kDecodeWaves][16];         // per wave: alpha per query column

    const int nw = blockDim.x >> 6;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
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
    const int32_t fp = remap(p, G);
    const int32_t rem_last = p - a.w_local;  // keys j <= rem_last are remote (if bif)
    // Chunks start at z0 + split * chunk with z0 in (-64, 0] chosen so that the
    // first local key rem_last + 1 starts a 64-key stage: every stage is then
    // wholly remote or wholly local.  Positions below 0 are masked.
    int32_t z0 = 0;
    if (bif && rem_last >= 0) {
        const int32_t m = (rem_last + 1) & (kStage - 1);
        z0 = m ? m - kStage : 0;
    }
    const int32_t kbeg = z0 + split * a.lay.chunk;
    const int32_t kend = min(kbeg + a.lay.chunk, L);

    float4* pm = (float4*)((char*)a.ws + a.lay.part_ml);
    float* po = (float*)((char*)a.ws + a.lay.part_o);
    const int64_t pbase = ((int64_t)b * a.lay.n_splits + split) * a.Hq + (int64_t)kvh * grp;

    if (kbeg >= kend) {  // empty chunk: neutral partial
        if (head_ok) {
            if (c == 0 && n < grp) pm[pbase + n] = make_float4(-INFINITY, 0.0f, 0.0f, 0.0f);
            for (int x = lane; x < grp * D; x += 64) po[pbase * D + x] = 0.0f;
        }
        return;
    }

    const TIN* kc = (const TIN*)a.kc + (int64_t)b * a.S_max * a.Hkv * D + (int64_t)kvh * D;
    const TIN* vc = (const TIN*)a.vc + (int64_t)b * a.S_max * a.Hkv * D + (int64_t)kvh * D;
    const int64_t rstride = (int64_t)a.Hkv * D;

    // tile loads into registers (zero beyond the chunk): K as MFMA operands,
    // V as one 64-lane row read per key
    typedef typename Vec8<TIN>::T KV8;
    typedef VSmall<TIN, DPL> VV;
    KV8 kA[NST], kB[NST];
    VV vA[kTile], vB[kTile];
    auto load_tile = [&](int32_t j0, KV8* kd, VV* vd) __attribute__((always_inline)) {
        const int32_t kj = j0 + n;
        const bool okk = kj >= 0 && kj < kend;
#pragma unroll
        for (int s = 0; s < NST; ++s)
            kd[s] = okk ? Vec8<TIN>::load(kc + (int64_t)kj * rstride + 32 * s + 8 * c) : KV8{};
#pragma unroll
        for (int r = 0; r < kTile; ++r) {
            if (j0 + r >= 0 && j0 + r < kend) vd[r].load(vc + (int64_t)(j0 + r) * rstride + DPL * lane);
            else vd[r].zero();
        }
    };
    if (head_ok) load_tile(kbeg, kA, vA);

    // ---- theta_t / 2 pi and the small-angle table, once per workgroup (the
    // only barrier) ----
    {
        const double rv = rope_rev(a.tab, threadIdx.x % HALF);  // blockDim is a multiple of HALF
        if (threadIdx.x < HALF) revs[threadIdx.x] = rv;
        if (BIF && bif) {
            for (int x = threadIdx.x; x < kStage * HALF; x += blockDim.x) {
                float cs, sn;
                rope_cs_hw(-(int64_t)(x / HALF), rv, cs, sn);
                tab[(x / HALF) * TSTR + x % HALF] = make_float2(cs, sn);
            }
        }
        __syncthreads();
    }
    if (!head_ok) return;

    // ---- query.  Lane column n carries head hq; with PACK, columns
    // [GQ, 2 GQ) carry the lo parts.  Raw values at d = 32 s + 8 c + u stay
    // in the input type; Q holds the rotated query the current keys use.
    const float qscale = a.softmax_scale * kLog2e;
    const int hq = PACK ? (n & (GQ - 1)) : n;
    const bool qlo = PACK && n >= GQ;
    KV8 qraw[NST];
    {
        const bool qok = hq < grp && (!PACK || n < 2 * GQ);
        const TIN* qp = (const TIN*)a.q + ((int64_t)b * a.Hq + kvh * grp + hq) * D + 8 * c;
#pragma unroll
        for (int s = 0; s < NST; ++s) qraw[s] = qok ? Vec8<TIN>::load(qp + 32 * s) : KV8{};
    }
    bf16x8 Q[NST];
    bf16x8 Qlo[PACK ? 1 : NST];
    auto rotate_q = [&](int64_t pos) __attribute__((always_inline)) {
#pragma unroll
        for (int s = 0; s < NH; ++s)
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                const int t = 32 * s + 8 * c + u;
                float cs, sn;
                rope_cs_hw(pos, revs[t], cs, sn);
                const float x0 = Vec8<TIN>::get(qraw[s], u), x1 = Vec8<TIN>::get(qraw[s + NH], u);
                const float y0 = (x0 * cs - x1 * sn) * qscale;
                const float y1 = (x1 * cs + x0 * sn) * qscale;
                const bf16 h0 = (bf16)y0, h1 = (bf16)y1;
                const bf16 l0 = (bf16)(y0 - (float)h0), l1 = (bf16)(y1 - (float)h1);
                if constexpr (PACK) {
                    Q[s][u] = qlo ? l0 : h0;
                    Q[s + NH][u] = qlo ? l1 : h1;
                } else {
                    Q[s][u] = h0;
                    Q[s + NH][u] = h1;
                    Qlo[s][u] = l0;
                    Qlo[s + NH][u] = l1;
                }
            }
    };
    // Q is set at every stage start: remote stages turn it to the stage's
    // angle, local stages use R(p) q (kept once set)
    bool q_local = false;

    auto finish = [&](f32x4 acc) __attribute__((always_inline)) -> f32x4 {
        if constexpr (PACK) {
#pragma unroll
            for (int i = 0; i < 4; ++i) acc[i] += __shfl_xor(acc[i], GQ);
        }
        return acc;
    };
    // scores of a tile on the stored keys (Q = R(p) q)
    auto scores_local = [&](const KV8* kcur) __attribute__((always_inline)) -> f32x4 {
        f32x4 acc = {};
#pragma unroll
        for (int s = 0; s < NST; ++s) {
            if constexpr (sizeof(TIN) == 2) {
                // stored bf16 keys are exact MFMA operands
                acc = mfma16(kcur[s], Q[s], acc);
                if constexpr (!PACK) acc = mfma16(kcur[s], Qlo[s], acc);
            } else {
                bf16x8 h0, l0;
#pragma unroll
                for (int x = 0; x < 8; ++x) {
                    const float k0 = Vec8<TIN>::get(kcur[s], x);
                    h0[x] = (bf16)k0;
                    l0[x] = (bf16)(k0 - (float)h0[x]);
                }
                acc = mfma16(h0, Q[s], acc);
                acc = mfma16(l0, Q[s], acc);
                if constexpr (!PACK) acc = mfma16(h0, Qlo[s], acc);
            }
        }
        return finish(acc);
    };
    // scores of a tile of remote keys: key n turned by -u theta (Q = stage query)
    auto scores_remote = [&](const KV8* kcur, int32_t u) __attribute__((always_inline)) -> f32x4 {
        f32x4 acc = {};
        const float2* tp = tab + u * TSTR + 8 * c;
#pragma unroll
        for (int s = 0; s < NH; ++s) {
            bf16x8 h0, l0, h1, l1;
#pragma unroll
            for (int x = 0; x < 8; ++x) {
                const float2 cs = tp[32 * s + x];
                const float k0 = Vec8<TIN>::get(kcur[s], x);
                const float k1 = Vec8<TIN>::get(kcur[s + NH], x);
                const float y0 = k0 * cs.x - k1 * cs.y;
                const float y1 = k1 * cs.x + k0 * cs.y;
                h0[x] = (bf16)y0;
                l0[x] = (bf16)(y0 - (float)h0[x]);
                h1[x] = (bf16)y1;
                l1[x] = (bf16)(y1 - (float)h1[x]);
            }
            acc = mfma16(h0, Q[s], acc);
            acc = mfma16(l0, Q[s], acc);
            acc = mfma16(h1, Q[s + NH], acc);
            acc = mfma16(l1, Q[s + NH], acc);
            if constexpr (!PACK) {
                acc = mfma16(h0, Qlo[s], acc);
                acc = mfma16(h1, Qlo[s + NH], acc);
            }
        }
        return finish(acc);
    };

    float m_run = -INFINITY, l_part = 0.0f;
    float O[GQ][DPL];
#pragma unroll
    for (int h = 0; h < GQ; ++h)
#pragma unroll
        for (int x = 0; x < DPL; ++x) O[h][x] = 0.0f;

    // online softmax and P V of one tile.  The running max is only raised
    // when a score exceeds it by more than 2^8 (log2 units): the partial sums
    // stay exact relative to whatever max they use, and most tiles then skip
    // rescaling O.
    auto process = [&](int32_t j0, const f32x4& sacc, const VV* vcur) __attribute__((always_inline)) {
        const bool col = n < GQ;  // lanes of packed lo parts carry no scores
        float sc[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int32_t kk = j0 + 4 * c + i;
            sc[i] = (col && kk >= 0 && kk < kend) ? sacc[i] : -INFINITY;
        }
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
            // masked keys weigh exactly 0 (also while m_run is still -inf)
            const float pv = sc[i] != -INFINITY ? __builtin_amdgcn_exp2f(sc[i] - m_run) : 0.0f;
            ps += pv;
            pbuf[wave][4 * c + i][n] = pv;
        }
        l_part = l_part * alpha + ps;
        const bool any_raise = __any(raise);
        if (any_raise && c == 0) abuf[wave][n] = alpha;
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        if (any_raise) {
#pragma unroll
            for (int h = 0; h < GQ; ++h) {
                const float ah = abuf[wave][h];
#pragma unroll
                for (int x = 0; x < DPL; ++x) O[h][x] *= ah;
            }
        }
#pragma unroll
        for (int r = 0; r < kTile; ++r) {
#pragma unroll
            for (int h = 0; h < GQ; ++h) {
                const float ph = pbuf[wave][r][h];
#pragma unroll
                for (int x = 0; x < DPL; ++x) O[h][x] += ph * vcur[r].get(x);
            }
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    };

    const float invG = 1.0f / (float)G;
    int32_t jb = 0, r0 = 0;     // angle base of the stage (>= 0) and jb mod G
    bool stage_remote = false;
    auto tile = [&](int32_t j0, const KV8* kcur, const VV* vcur) __attribute__((always_inline)) {
        f32x4 sacc;
        if (BIF && stage_remote) {
            // u of key n: (j - jb) - (f(j) - f(jb)), f(j) - f(jb) = floor((r0 + j - jb) / G)
            const int32_t dl = max(j0 + n - jb, 0);
            int32_t fd = (int32_t)((float)(r0 + dl) * invG);
            if ((fd + 1) * G <= r0 + dl) ++fd;
            if (fd * G > r0 + dl) --fd;
            const int32_t uu = min(max(dl - fd, 0), kStage - 1);
            sacc = scores_remote(kcur, uu);
        } else {
            sacc = scores_local(kcur);
        }
        process(j0, sacc, vcur);
    };

    // stages of 64 positions; within a stage one tile stays in flight while
    // the previous one is processed (even tiles in kA/vA, odd ones in kB/vB)
    for (int32_t js = kbeg; js < kend; js += kStage) {
        stage_remote = BIF && bif && js <= rem_last;
        jb = max(js, 0);
        const int32_t fjb = remap(jb, G);
        r0 = jb - fjb * G;
        if (stage_remote || !q_local) {
            rotate_q(stage_remote ? (int64_t)fp - fjb + jb : (int64_t)p);
            q_local = !stage_remote;
        }
#pragma unroll 1
        for (int u = 0; u < kStage / kTile; u += 2) {
            const int32_t j0 = js + kTile * u;
            if (j0 < kend) {
                const bool more = j0 + kTile < kend;
                if (more) load_tile(j0 + kTile, kB, vB);
                tile(j0, kA, vA);
                if (more) {
                    if (j0 + 2 * kTile < kend) load_tile(j0 + 2 * kTile, kA, vA);
                    tile(j0 + kTile, kB, vB);
                }
            }
        }
    }

    // ---- partial (m, l, unnormalised O) of this chunk ----
    float l_tot = l_part + __shfl_xor(l_part, 16);
    l_tot += __shfl_xor(l_tot, 32);
    if (c == 0 && n < grp) pm[pbase + n] = make_float4(m_run, l_tot, l_tot, 0.0f);
#pragma unroll
    for (int h = 0; h < GQ; ++h)
        if (h < grp) {
#pragma unroll
            for (int x = 0; x < DPL; ++x) po[(pbase + h) * D + DPL * lane + x] = O[h][x];
        }
}

// 8 OCP E4M3 codes (4 per 32-bit word, little-endian) as fp16: an E4M3
// value has 4 significant bits and an exponent in [-9, 8], so fp16 holds it
// exactly.  gfx950's v_cvt_scalef32_pk_f16_fp8 widens two codes straight to
// packed fp16 (times a power-of-two scale, here 1), four instructions for 8
// codes; NaN codes stay NaN.
__device__ __forceinline__ f16x8 e4m3x8_to_f16(uint32_t w0, uint32_t w1) {
    typedef _Float16 h2 __attribute__((ext_vector_type(2)));
    const h2 a = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w0, 1.0f, false);
    const h2 b = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w0, 1.0f, true);
    const h2 c = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w1, 1.0f, false);
    const h2 d = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w1, 1.0f, true);
    return f16x8{a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
}
// 8 bf16 keys as fp16 MFMA operands (exact for magnitudes in [2^-14, 65504])
__device__ __forceinline__ f16x8 bf16x8_to_f16(const bf16x8& x) {
    f16x8 r;
#pragma unroll
    for (int i = 0; i < 8; ++i) r[i] = (f16)(float)x[i];
    return r;
}
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ f32x4 mfma16(f16x8 a, f16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}
// P V product on fp16 operands (bits passed as shorts, as the LDS read gives them)
__device__ __forceinline__ f32x4 mfma16k16h(s16x4 a, s16x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x16f16(__builtin_bit_cast(f16x4, a),
                                                 __builtin_bit_cast(f16x4, b), c, 0, 0, 0);
}

// Buffer resource word 3 for raw (unstructured) buffers on gfx9-family
// chips: 32-bit data format, no swizzle; out-of-range loads return zeros.
constexpr int kBufferRsrcWord3 = 0x00020000;
// 8 or 16 bytes at byte offset off of a raw buffer (zeros past its range)
template <typename T>
__device__ __forceinline__ T buffer_load(__amdgpu_buffer_rsrc_t r, int32_t off) {
    if constexpr (sizeof(T) == 8) {
        return __builtin_bit_cast(T, __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0));
    } else {
        static_assert(sizeof(T) == 16, "8- or 16-byte loads");
        return __builtin_bit_cast(T, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
    }
}

// bf16 decode.  Same scoring as above, with QK^T on fp16 operands: the
// query is an fp16 hi + lo pair, stored keys widen to fp16 (exact), and a
// remote key is turned on packed fp16 by an fp16 (cos, sin) table, a few
// fp16 roundings per element (a key's rounding is independent of the other
// keys' and averages out in the softmax, unlike the query's, hence the
// query's lo part).  P V runs on MFMA.  Each wave stages its V tile in LDS
// and the transposing read ds_read_b64_tr_b16 hands every lane its B operand
// (4 keys x 1 d per 16-d block) directly.  The probabilities are already in
// the A operand layout (lane (n, c) holds keys 4c..4c+3 of query column n),
// rounded to bf16; the row sums use the same rounded values.  K and V tiles
// stay two ahead in registers.  All loads are unconditional (indices clamped
// to the chunk's rows, or flat caches read through buffer resources that
// return zeros outside them), so the memory stream has no branches and the
// compiler's waits stay exact.
// PAGED: the cache is a pool of pages of 2^page_shift rows addressed through
// a per-sequence block table (each workgroup copies its chunk's page numbers
// to LDS, clamped to the pool, so a bad table entry cannot read outside it).
// FP8: the cache holds OCP E4M3 codes with one scale per kv head.  Codes
// widen exactly to fp16 (keys and the V tile in LDS); P is fp16 too.  The
// key scale enters the query's scale and the value scale multiplies the
// partial output.
// PREC (split precision, bf16 caches): remote keys are turned in fp32 against
// an fp32 table and split into fp16 hi + lo operands (two products per
// k-step), so a dominant remote key's score carries no fp16 rounding.
template <int D, bool BIF, int GQ, bool PAGED, bool FP8, bool PREC = false>
__global__ __launch_bounds__(512) void decode_split_bf16_kernel(DecodeArgs a) {
    using TC = typename std::conditional<FP8, uint8_t, bf16>::type;  // cache element
    using KRAW = typename std::conditional<FP8, u32x2, bf16x8>::type;  // 8 key elements
    using VRAW = typename std::conditional<FP8, u32x4, bf16x8>::type;  // 16 bytes of a V row
    using OT = f16;                                                     // QK^T operand element
    using OV = f16x8;                                                   // 8 QK^T operands
    using PT = typename std::conditional<FP8, f16, bf16>::type;         // P V operand element
    constexpr int HALF = D / 2;
    constexpr int NST = D / 32;          // k-steps of the QK^T product
    constexpr int NH = NST / 2;          // k-steps per RoPE half
    constexpr bool PACK = GQ <= 8;       // hi and lo query parts in one operand
    constexpr int ROWB = D * (int)sizeof(TC);  // bytes of one cache row of V
    constexpr int VEL = 16 / (int)sizeof(TC);  // V elements per 16-byte load
    constexpr int CPR = ROWB / 16;       // 16-byte chunks per row
    constexpr int RPI = 64 / CPR;        // rows per 64-lane load
    constexpr int NI = kTile / RPI;      // V loads per lane per tile
    constexpr int VRS = D * 2 + 32;      // LDS row stride of a bf16 V tile (+32 spreads banks)
    constexpr int SLOT = kTile * VRS;    // bytes of one wave's V tile
    constexpr int NDB = D / 16;          // 16-wide d blocks of O
    constexpr int TSTRH = D + 8;         // LDS row stride of the angle table (halves)
    // R(-u theta_t) in fp16: row u holds the HALF cosines, then the HALF sines
    __shared__ __align__(16) f16 tabh[(BIF && !PREC) ? kStageB * TSTRH : 8];
    // the same table in fp32 for split-precision remote keys (row stride D + 4)
    constexpr int TSTRF = D + 4;
    __shared__ __align__(16) float tabf[(BIF && PREC) ? kStageB * TSTRF : 4];
    // query angles: row st < kDecodeMaxStagesB holds R(f(p) - f(jb) + jb) of
    // this workgroup's stage st (remote stages), the last row R(p)
    __shared__ float2 qtab[(kDecodeMaxStagesB + 1) * HALF];
    __shared__ __align__(16) char vs[kWavesB * SLOT];  // per wave: the V tile in use
    // per wave (PACK): the turned query, fp16 hi rows then lo rows
    constexpr int QRS = D + 8;  // row stride (halves)
    __shared__ __align__(16) f16 qs[PACK ? kWavesB * 2 * GQ * QRS : 8];
    __shared__ int32_t ptab[PAGED ? kDecodeMaxPages : 1];  // page numbers of this chunk
    // tiles finished per wave.  Waves w and w + 4 share a SIMD, whose issue
    // arbiter favours the older wave: left alone, waves 0-3 finish their
    // chunks about a fifth earlier and the younger waves then stream alone
    // with half the loads in flight.  A wave that falls behind its partner
    // raises its issue priority until it has caught up.
    __shared__ int done_s[kWavesB];
    volatile int* done = done_s;

    const int nw = blockDim.x >> 6;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
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
    const int32_t fp = remap(p, G);
    const int32_t rem_last = p - a.w_local;  // keys j <= rem_last are remote (if bif)
    // continuous-interpolation variant (bifocal 2): remote positions x / s,
    // s = L / w_pretrained; within a stage the key correction is then
    // -(j - jb)(1 - 1/s) and the table is indexed by j - jb
    const bool interp = BIF && a.bifocal == 2;
    const double rsc = interp ? (double)a.w_pretrained / (double)max(L, 1) : 1.0;
    // stages of kStageB positions start at sbase = z0 (+ kwin), z0 in
    // (-kStageB, 0], so that the first local key starts a stage; positions
    // below 0 are masked.  A single local call of the unfused form sees only
    // keys p - j < w_local (kwin).  NS stages cover [sbase, L).
    int32_t z0 = 0;
    if (bif && rem_last >= 0) {
        const int32_t m = (rem_last + 1) % kStageB;
        z0 = m ? m - kStageB : 0;
    }
    const int32_t kwin = a.window ? max(L - a.w_local, 0) : 0;
    const int32_t sbase = kwin + z0;
    const int32_t NS = L > sbase ? (L - sbase + kStageB - 1) / kStageB : 0;
    // Stages of this workgroup.  ILV (flat caches, up to 8 query heads per
    // kv head, byte offsets within 32 bits; set by the host): stages split,
    // split + n_splits, ..., so that at any moment the workgroups read
    // neighbouring stages, one contiguous front of the cache, which HBM
    // serves faster than one stream per workgroup.  Otherwise chunk /
    // kStageB consecutive stages (the chunk [kbeg, kend)).
    constexpr bool BUF = !PAGED && PACK;
    const bool ilv = BUF && a.ilv;
    const int32_t cps = a.lay.chunk / kStageB;
    const int32_t sfirst = ilv ? split : split * cps;
    const int32_t sstep = ilv ? a.lay.n_splits : 1;
    const int32_t nst = ilv ? (NS > split ? (NS - split + sstep - 1) / sstep : 0)
                            : max(0, min(cps, NS - sfirst));
    auto js_of = [&](int32_t k) __attribute__((always_inline)) -> int32_t {
        return sbase + (sfirst + k * sstep) * kStageB;
    };
    const int32_t kbeg = js_of(0);
    const int32_t kend = ilv ? L : min(kbeg + a.lay.chunk, L);

    float4* pm = (float4*)((char*)a.ws + a.lay.part_ml);
    float* po = (float*)((char*)a.ws + a.lay.part_o);
    const int64_t pbase = ((int64_t)b * a.lay.n_splits + split) * a.Hq + (int64_t)kvh * grp;
    if (nst <= 0) {  // no stage: neutral partial
        if (head_ok) {
            if (c == 0 && n < grp) pm[pbase + n] = make_float4(-INFINITY, 0.0f, 0.0f, 0.0f);
            for (int x = lane; x < grp * D; x += 64) po[pbase * D + x] = 0.0f;
        }
        return;
    }

    // every load below is unconditional (branch-free memory stream, exact
    // waits) and reads only rows of this workgroup's range [klo, kend) (the
    // chunk, or with ILV the whole sequence): the key index is clamped into
    // it, or (BUF: flat caches, up to 8 query heads per kv head, where the
    // registers allow) the loads go through buffer resources whose range ends
    // with row kend - 1, so that other rows read as zeros.  Masked keys weigh
    // 0 either way.
    const int kvh_c = min(kvh, a.Hkv - 1);
    const int64_t boff = PAGED ? 0 : (int64_t)b * a.S_max * a.Hkv * D;
    const int64_t boff_k = PAGED ? 0 : (int64_t)b * (a.S_max_k ? a.S_max_k : a.S_max) * a.Hkv * D;
    const TC* kc = (const TC*)a.kc + boff_k + (int64_t)kvh_c * D;
    const TC* vc = (const TC*)a.vc + boff + (int64_t)kvh_c * D;
    const int64_t rstride = (int64_t)a.Hkv * D;
    char* const slot = vs + wave * SLOT;

    const int32_t klo = max(kbeg, 0), khi = kend - 1;
    // cache row of key j (j in [klo, khi])
    const int32_t pg0 = PAGED ? (klo >> a.page_shift) : 0;
    if constexpr (PAGED) {
        const int32_t npg = (khi >> a.page_shift) - pg0 + 1;
        const int32_t* bt = a.block_table + (int64_t)b * a.bt_stride;
        for (int x = threadIdx.x; x < npg; x += blockDim.x)
            ptab[x] = (int32_t)min(max((int64_t)bt[pg0 + x], (int64_t)0), a.n_pages - 1);
        __syncthreads();
    }
    auto row_of = [&](int32_t j) __attribute__((always_inline)) -> int64_t {
        if constexpr (PAGED) {
            return ((int64_t)ptab[(j >> a.page_shift) - pg0] << a.page_shift) |
                   (j & ((1 << a.page_shift) - 1));
        } else {
            return j;
        }
    };
    // BUF: resources based at row rb (klo, or row 0 with ILV) of this kv
    // head, offsets in bytes from there (32-bit: a chunk spans a few MB; with
    // ILV the host checked the sequence's span), one add per load group and
    // tile in place of clamping and 64-bit row arithmetic
    constexpr int ES = (int)sizeof(TC);
    const int32_t rsb = (int32_t)rstride * ES;  // bytes between rows
    const int32_t rb = ilv ? 0 : klo;
    const int32_t nrec = (kend - rb - 1) * rsb + D * ES;
    const __amdgpu_buffer_rsrc_t rk = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(kc + (int64_t)rb * rstride), (short)0, BUF ? nrec : 0, kBufferRsrcWord3);
    const __amdgpu_buffer_rsrc_t rv = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(vc + (int64_t)rb * rstride), (short)0, BUF ? nrec : 0, kBufferRsrcWord3);
    // K of key j0 + n into registers (keys outside the chunk: masked)
    auto load_k = [&](int32_t j0, KRAW* kd) __attribute__((always_inline)) {
        if constexpr (!BUF) {
            const int32_t kj = min(max(j0 + n, klo), khi);
#pragma unroll
            for (int s = 0; s < NST; ++s)
                kd[s] = *reinterpret_cast<const KRAW*>(kc + row_of(kj) * rstride + 32 * s + 8 * c);
        } else {
            const int32_t off = (j0 - rb + n) * rsb + 8 * c * ES;
#pragma unroll
            for (int s = 0; s < NST; ++s) kd[s] = buffer_load<KRAW>(rk, off + 32 * s * ES);
        }
    };
    // V tiles are staged in registers two tiles ahead (load r of a lane
    // reads 16 bytes of key RPI r + lane / CPR, so one load instruction
    // covers whole rows) and written to the wave's LDS slot, rows VRS bytes
    // apart, right before use
    auto load_vr = [&](int32_t j0, VRAW* vd) __attribute__((always_inline)) {
        const int q = lane / CPR, ch = lane % CPR;
#pragma unroll
        for (int r = 0; r < NI; ++r) {
            if constexpr (!BUF) {
                const int32_t key = min(max(j0 + RPI * r + q, klo), khi);
                vd[r] = *reinterpret_cast<const VRAW*>(vc + row_of(key) * rstride + VEL * ch);
            } else {
                vd[r] = buffer_load<VRAW>(rv, (j0 - rb + RPI * r + q) * rsb + 16 * ch);
            }
        }
    };
    auto store_vr = [&](const VRAW* vsrc, char* dst) __attribute__((always_inline)) {
        const int q = lane / CPR, ch = lane % CPR;
#pragma unroll
        for (int r = 0; r < NI; ++r) {
            char* row = dst + (RPI * r + q) * VRS + 2 * VEL * ch;
            if constexpr (FP8) {
                *reinterpret_cast<f16x8*>(row) = e4m3x8_to_f16(vsrc[r][0], vsrc[r][1]);
                *reinterpret_cast<f16x8*>(row + 16) = e4m3x8_to_f16(vsrc[r][2], vsrc[r][3]);
            } else {
                *reinterpret_cast<bf16x8*>(row) = vsrc[r];
            }
        }
    };
    // the 8 key elements of a k-step as MFMA operands (exact for E4M3 codes)
    auto kop = [&](const KRAW& kr) __attribute__((always_inline)) -> OV {
        if constexpr (FP8) return e4m3x8_to_f16(kr[0], kr[1]);
        else return bf16x8_to_f16(kr);
    };
    VRAW vA[NI], vB[NI], vC[NI];

    KRAW kA[NST], kB[NST], kC[NST];
    // query first (unconditional loads from a clamped head; heads past the
    // group are zeroed).  With PACK each stage's query rotation is done once
    // per element: lane l turns QPL pairs (i, i + HALF) of head qh and writes
    // the fp16 hi and lo parts to its wave's rows of qs (hi rows 0..GQ-1, lo
    // rows GQ..2GQ-1), from which every lane reads its MFMA operand: column
    // n < GQ the hi part of head n, column GQ + h the lo part of head h
    // (columns from 2 GQ on repeat the first ones; their scores are never
    // used).  Without PACK (16 heads) the lanes' operand elements are all
    // distinct and each lane turns its own.
    constexpr int QPL = PACK ? GQ * HALF / 64 : 1;  // pairs per lane
    const int qh = PACK ? lane / (64 / GQ) : n;
    const int qi0 = PACK ? (lane % (64 / GQ)) * QPL : 0;
    float qf[PACK ? 2 * QPL : 1];  // PACK: elements i and i + HALF of the lane's pairs
    bf16x8 qraw[PACK ? 1 : NST];
    {
        const bool qok = qh < grp;
        const int qh_c = min(qh, grp - 1);
        const bf16* qp = (const bf16*)a.q + ((int64_t)b * a.Hq + kvh_c * grp + qh_c) * D;
        if constexpr (PACK) {
#pragma unroll
            for (int k = 0; k < QPL; ++k) {
                const float x0 = (float)qp[qi0 + k], x1 = (float)qp[HALF + qi0 + k];
                qf[k] = qok ? x0 : 0.0f;
                qf[QPL + k] = qok ? x1 : 0.0f;
            }
        } else {
#pragma unroll
            for (int s = 0; s < NST; ++s) {
                const bf16x8 x = *reinterpret_cast<const bf16x8*>(qp + 8 * c + 32 * s);
                qraw[s] = qok ? x : bf16x8{};
            }
        }
    }
    // the first tile's loads go out before the angle tables, the second's
    // after them (the table work then waits less on the load issue queue)
    load_k(kbeg, kA);
    load_vr(kbeg, vA);
    if (threadIdx.x < kWavesB) done_s[threadIdx.x] = 0;

    // ---- angle tables, once per workgroup (the only barrier): the query
    // rows and the small key angles -u theta_t ----
    constexpr int QLOC = kDecodeMaxStagesB;  // row of R(p)
    {
        const double rv = rope_rev(a.tab, threadIdx.x % HALF);  // blockDim is a multiple of HALF
        // (the layout keeps nst <= kDecodeMaxStagesB; the bound keeps LDS safe)
        const int nq = min(nst, (int32_t)kDecodeMaxStagesB);
        for (int x = threadIdx.x; x < (nq + 1) * HALF; x += blockDim.x) {
            const int st = x / HALF;
            float cs, sn;
            if (st < nq) {
                const int32_t jbs = max(js_of(st), 0);
                if (interp)  // R(p / s - jb / s + jb)
                    rope_cs_rev(((double)(p - jbs) * rsc + (double)jbs) * rv, cs, sn);
                else
                    rope_cs_hw((int64_t)fp - remap(jbs, G) + jbs, rv, cs, sn);
            } else {
                rope_cs_hw(a.q_remap ? fp : p, rv, cs, sn);
            }
            qtab[(st < nq ? st : QLOC) * HALF + x % HALF] = make_float2(cs, sn);
        }
        if (BIF && bif) {
            for (int x = threadIdx.x; x < kStageB * HALF; x += blockDim.x) {
                float cs, sn;
                if (interp)  // key delta positions past the stage base: R(-delta (1 - 1/s))
                    rope_cs_rev(-(double)(x / HALF) * (1.0 - rsc) * rv, cs, sn);
                else
                    rope_cs_hw(-(int64_t)(x / HALF), rv, cs, sn);
                if constexpr (PREC) {
                    tabf[(x / HALF) * TSTRF + x % HALF] = cs;
                    tabf[(x / HALF) * TSTRF + HALF + x % HALF] = sn;
                } else {
                    tabh[(x / HALF) * TSTRH + x % HALF] = (f16)cs;
                    tabh[(x / HALF) * TSTRH + HALF + x % HALF] = (f16)sn;
                }
            }
        }
        __syncthreads();
    }
    if (!head_ok) return;
    load_k(kbeg + kTile, kB);
    load_vr(kbeg + kTile, vB);

    // ---- query (as in the generic kernel) ----
    // fp8: the key scale enters the query's scale (a score is linear in k)
    const float kscale = FP8 && a.k_scale ? a.k_scale[kvh_c] : 1.0f;
    const float qscale = a.softmax_scale * kLog2e * kscale;
    OV Q[NST];
    OV Qlo[PACK ? 1 : NST];
    auto rotate_q = [&](int row) __attribute__((always_inline)) {
        if constexpr (PACK) {
            typedef _Float16 QV __attribute__((ext_vector_type(QPL)));
            const float2* qt = qtab + row * HALF + qi0;
            QV h0, h1, l0, l1;
#pragma unroll
            for (int k = 0; k < QPL; ++k) {
                const float2 cs = qt[k];
                const float x0 = qf[k], x1 = qf[QPL + k];
                const float y0 = (x0 * cs.x - x1 * cs.y) * qscale;
                const float y1 = (x1 * cs.x + x0 * cs.y) * qscale;
                h0[k] = (OT)y0;
                h1[k] = (OT)y1;
                l0[k] = (OT)(y0 - (float)h0[k]);
                l1[k] = (OT)(y1 - (float)h1[k]);
            }
            // the wave writes, then reads its own rows: LDS keeps its order
            f16* w = qs + wave * (2 * GQ * QRS);
            *reinterpret_cast<QV*>(w + qh * QRS + qi0) = h0;
            *reinterpret_cast<QV*>(w + qh * QRS + HALF + qi0) = h1;
            *reinterpret_cast<QV*>(w + (GQ + qh) * QRS + qi0) = l0;
            *reinterpret_cast<QV*>(w + (GQ + qh) * QRS + HALF + qi0) = l1;
            const f16* r = w + (n & (2 * GQ - 1)) * QRS + 8 * c;
#pragma unroll
            for (int s = 0; s < NST; ++s) Q[s] = *reinterpret_cast<const f16x8*>(r + 32 * s);
        } else {
            const float2* qt = qtab + row * HALF + 8 * c;
#pragma unroll
            for (int s = 0; s < NH; ++s)
#pragma unroll
                for (int u = 0; u < 8; ++u) {
                    const float2 cs = qt[32 * s + u];
                    const float x0 = (float)qraw[s][u], x1 = (float)qraw[s + NH][u];
                    const float y0 = (x0 * cs.x - x1 * cs.y) * qscale;
                    const float y1 = (x1 * cs.x + x0 * cs.y) * qscale;
                    const OT h0 = (OT)y0, h1 = (OT)y1;
                    Q[s][u] = h0;
                    Q[s + NH][u] = h1;
                    Qlo[s][u] = (OT)(y0 - (float)h0);
                    Qlo[s + NH][u] = (OT)(y1 - (float)h1);
                }
        }
    };
    bool q_local = false;

    auto finish = [&](f32x4 acc) __attribute__((always_inline)) -> f32x4 {
        if constexpr (PACK) {
#pragma unroll
            for (int i = 0; i < 4; ++i) acc[i] += __shfl_xor(acc[i], GQ);
        }
        return acc;
    };
    auto scores_local = [&](const KRAW* kcur) __attribute__((always_inline)) -> f32x4 {
        f32x4 acc = {};
#pragma unroll
        for (int s = 0; s < NST; ++s) {
            const OV kb = kop(kcur[s]);
            acc = mfma16(kb, Q[s], acc);
            if constexpr (!PACK) acc = mfma16(kb, Qlo[s], acc);
        }
        return finish(acc);
    };
    // A remote key turned by -u theta_t: the stored values widen exactly to
    // fp16 and the rotation runs on packed fp16 against the fp16 table (a
    // key's rounding is its own and averages out in the softmax).
    auto scores_remote = [&](const KRAW* kcur, int32_t u) __attribute__((always_inline)) -> f32x4 {
        f32x4 acc = {};
        if constexpr (PREC) {
            const float* tf = tabf + u * TSTRF + 8 * c;
#pragma unroll
            for (int s = 0; s < NH; ++s) {
                const f16x8 k0 = kop(kcur[s]);
                const f16x8 k1 = kop(kcur[s + NH]);
                const f32x4 ca = *reinterpret_cast<const f32x4*>(tf + 32 * s);
                const f32x4 cb = *reinterpret_cast<const f32x4*>(tf + 32 * s + 4);
                const f32x4 sa = *reinterpret_cast<const f32x4*>(tf + HALF + 32 * s);
                const f32x4 sb = *reinterpret_cast<const f32x4*>(tf + HALF + 32 * s + 4);
                f16x8 h0, l0, h1, l1;
#pragma unroll
                for (int x = 0; x < 8; ++x) {
                    const float cs = x < 4 ? ca[x] : cb[x - 4];
                    const float sn = x < 4 ? sa[x] : sb[x - 4];
                    const float a0 = (float)k0[x], a1 = (float)k1[x];
                    const float y0 = a0 * cs - a1 * sn;
                    const float y1 = a1 * cs + a0 * sn;
                    h0[x] = (f16)y0;
                    l0[x] = (f16)(y0 - (float)h0[x]);
                    h1[x] = (f16)y1;
                    l1[x] = (f16)(y1 - (float)h1[x]);
                }
                acc = mfma16(h0, Q[s], acc);
                acc = mfma16(l0, Q[s], acc);
                acc = mfma16(h1, Q[s + NH], acc);
                acc = mfma16(l1, Q[s + NH], acc);
                if constexpr (!PACK) {
                    acc = mfma16(h0, Qlo[s], acc);
                    acc = mfma16(h1, Qlo[s + NH], acc);
                }
            }
            return finish(acc);
        }
        const f16* th = tabh + u * TSTRH + 8 * c;
#pragma unroll
        for (int s = 0; s < NH; ++s) {
            const f16x8 k0 = kop(kcur[s]);
            const f16x8 k1 = kop(kcur[s + NH]);
            const f16x8 cs = *reinterpret_cast<const f16x8*>(th + 32 * s);
            const f16x8 sn = *reinterpret_cast<const f16x8*>(th + HALF + 32 * s);
            const f16x8 h0 = k0 * cs - k1 * sn;
            const f16x8 h1 = k1 * cs + k0 * sn;
            acc = mfma16(h0, Q[s], acc);
            acc = mfma16(h1, Q[s + NH], acc);
            if constexpr (!PACK) {
                acc = mfma16(h0, Qlo[s], acc);
                acc = mfma16(h1, Qlo[s + NH], acc);
            }
        }
        return finish(acc);
    };

    // running softmax state per query column (log2 domain; a finite floor so
    // masked keys give exp2(-inf) = 0, never NaN) and O^T blocks: lane (n, c)
    // of block bd holds O[query 4c + i][d = 16 bd + n]
    // l_part sums the probabilities as rounded for the P V product (it
    // normalises O), l_exact sums them before rounding (it gives the LSE: a
    // dominant probability's rounding would otherwise enter the LSE whole)
    float m_run = -1e30f, l_part = 0.0f, l_exact = 0.0f;
    f32x4 O[NDB];
#pragma unroll
    for (int bd = 0; bd < NDB; ++bd) O[bd] = f32x4{};
    // the lane's transposing-read address in a slot: it supplies the 4 d of
    // key 4c + n/4 starting at d = 4 (n % 4) of each 16-d block
    const int vkey = 4 * c + (n >> 2);
    const int voff = vkey * VRS + (n & 3) * 8;

    int32_t kmask = 0;  // keys from here on are masked (end of the stage in use, or L)
    auto process = [&](int32_t j0, const f32x4& sacc, const char* slot) __attribute__((always_inline)) {
        const bool col = n < GQ;  // lanes of packed lo parts carry no scores
        float sc[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int32_t kk = j0 + 4 * c + i;
            sc[i] = (col && kk >= 0 && kk < kmask) ? sacc[i] : -INFINITY;
        }
        float mx = fmaxf(fmaxf(sc[0], sc[1]), fmaxf(sc[2], sc[3]));
        mx = fmaxf(mx, __shfl_xor(mx, 16));
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        const bool raise = mx > m_run + 8.0f;
        float alpha = 1.0f;
        if (raise) {
            alpha = __builtin_amdgcn_exp2f(m_run - mx);
            m_run = mx;
        }
        s16x4 pa;
        float ps = 0.0f, pe = 0.0f;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float pf = __builtin_amdgcn_exp2f(sc[i] - m_run);
            const PT pb = (PT)pf;
            ps += (float)pb;
            pe += pf;
            pa[i] = __builtin_bit_cast(short, pb);
        }
        l_part = l_part * alpha + ps;
        l_exact = l_exact * alpha + pe;
        if (__any(raise)) {
            // row 4c + i of O belongs to query column 4c + i
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float ai = __shfl(alpha, 4 * c + i);
#pragma unroll
                for (int bd = 0; bd < NDB; ++bd) O[bd][i] *= ai;
            }
        }
#pragma unroll
        for (int bd = 0; bd < NDB; ++bd) {
            const s16x4 vb = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(slot + voff + 32 * bd));
            O[bd] = FP8 ? mfma16k16h(pa, vb, O[bd]) : mfma16k16(pa, vb, O[bd]);
        }
    };

    const float invG = 1.0f / (float)G;
    int32_t jb = 0, r0 = 0;  // angle base of the stage (>= 0) and jb mod G
    bool stage_remote = false;
    int my_done = 0;
    const int partner = wave ^ 4;  // the other wave on this SIMD (if any)
    // one tile: issue the loads two tiles ahead, stage this tile's V in LDS,
    // score, P V, then set this wave's priority from its lead over its partner
    auto step = [&](int32_t j0, const KRAW* kcur, const VRAW* vcur, KRAW* knext, VRAW* vnext,
                    int32_t jpre) __attribute__((always_inline)) {
        load_k(jpre, knext);
        load_vr(jpre, vnext);
        store_vr(vcur, slot);  // the same wave writes then reads: LDS keeps its order
        f32x4 sacc;
        if (BIF && stage_remote) {
            // u of key n: (j - jb) - (f(j) - f(jb)), f(j) - f(jb) = floor((r0 + j - jb) / G)
            const int32_t dl = max(j0 + n - jb, 0);
            int32_t fd = (int32_t)((float)(r0 + dl) * invG);
            if ((fd + 1) * G <= r0 + dl) ++fd;
            if (fd * G > r0 + dl) --fd;
            const int32_t uu = interp ? min(dl, kStageB - 1) : min(max(dl - fd, 0), kStageB - 1);
            sacc = scores_remote(kcur, uu);
        } else {
            sacc = scores_local(kcur);
        }
        process(j0, sacc, slot);
        done[wave] = ++my_done;
        const int other = partner < nw ? done[partner] : 0;
        if (__builtin_amdgcn_readfirstlane(other) > my_done)
            __builtin_amdgcn_s_setprio(3);
        else
            __builtin_amdgcn_s_setprio(0);
    };

    for (int32_t k = 0; k < nst; ++k) {
        const int32_t js = js_of(k), jn = js_of(k + 1);
        kmask = min(js + kStageB, kend);
        stage_remote = BIF && bif && js <= rem_last;
        jb = max(js, 0);
        const int32_t fjb = remap(jb, G);
        r0 = jb - fjb * G;
        if (stage_remote || !q_local) {
            rotate_q(stage_remote ? k : QLOC);
            q_local = !stage_remote;
        }
        // tiles js, js + 16, js + 32 sit in (kA, vA), (kB, vB), (kC, vC); each
        // step loads the tile two ahead (the next stage's first two in the
        // last two steps); tiles past kmask are fully masked
        step(js, kA, vA, kC, vC, js + 2 * kTile);
        step(js + kTile, kB, vB, kA, vA, jn);
        step(js + 2 * kTile, kC, vC, kB, vB, jn + kTile);
    }

    // ---- partial (m, l_o, l_lse, unnormalised O) of this workgroup's stages ----
    float l_tot = l_part + __shfl_xor(l_part, 16);
    l_tot += __shfl_xor(l_tot, 32);
    float l_ex = l_exact + __shfl_xor(l_exact, 16);
    l_ex += __shfl_xor(l_ex, 32);
    if (c == 0 && n < grp) pm[pbase + n] = make_float4(m_run, l_tot, l_ex, 0.0f);
    const float vscale = FP8 && a.v_scale ? a.v_scale[kvh_c] : 1.0f;
#pragma unroll
    for (int i = 0; i < 4; ++i)
        if (4 * c + i < grp) {
#pragma unroll
            for (int bd = 0; bd < NDB; ++bd)
                po[(pbase + 4 * c + i) * D + 16 * bd + n] = FP8 ? O[bd][i] * vscale : O[bd][i];
        }
}

// Merge of the chunk partials ([TW] §四's LogSumExp combination): with m_c
// in log2 units, o = sum 2^(m_c - M) O_c / sum 2^(m_c - M) lo_c and
// lse = (M + log2 sum 2^(m_c - M) ll_c) ln 2, where lo_c sums a chunk's
// probabilities as its P V product used them (so o is a consistent weighted
// mean) and ll_c sums them before any rounding (bf16 caches; the two agree
// for fp32 caches).  Workgroup (head, sequence, 16-wide slice of d), 256
// threads = 64 chunk groups x 4 quads of d.  Each thread folds its chunks
// (loaded together) against their common max; the 16 groups of a wave are
// folded with lane shuffles and the 4 waves through LDS.  A sequence with no
// keys gets o = 0 and lse = -inf.
//
// A merge inside the split kernel (the last workgroup of each group of
// chunks merging them, found with counters) was measured slower: the
// compute units of different XCDs do not share an L2, so handing partials
// across XCDs costs L2 write-back / invalidate or uncached loads on the
// critical path, more than this launch costs.
struct MergeAcc {
    float m, lo, ll;
    f32x4 o;
};
// (m, l, o) of two disjoint key sets -> their union; m = -inf is the empty set
__device__ __forceinline__ MergeAcc merge_acc(const MergeAcc& x, const MergeAcc& y) {
    const float m = fmaxf(x.m, y.m);
    if (m == -INFINITY) return x;
    const float sx = __builtin_amdgcn_exp2f(x.m - m), sy = __builtin_amdgcn_exp2f(y.m - m);
    return MergeAcc{m, sx * x.lo + sy * y.lo, sx * x.ll + sy * y.ll, sx * x.o + sy * y.o};
}

template <typename TOUT>
__global__ __launch_bounds__(256) void decode_merge_kernel(DecodeArgs a) {
    constexpr int NG = 64, NB = 4;  // chunk groups; chunks per group per round
    __shared__ float sm[4][4], slo[4][4], sll[4][4];
    __shared__ f32x4 so[4][4];
    const int head = blockIdx.x, b = blockIdx.y, tid = threadIdx.x;
    const int g = tid >> 2, q4 = tid & 3, wave = tid >> 6;
    const int x0 = 16 * blockIdx.z + 4 * q4;
    const float4* pm = (const float4*)((const char*)a.ws + a.lay.part_ml);
    const float* po = (const float*)((const char*)a.ws + a.lay.part_o);
    const int ns = a.lay.n_splits;
    const int64_t base = (int64_t)b * ns * a.Hq + head;
    MergeAcc acc{-INFINITY, 0.0f, 0.0f, f32x4{}};
    for (int s0 = g; s0 < ns; s0 += NG * NB) {
        float4 ml[NB];
        f32x4 ov[NB];
#pragma unroll
        for (int k = 0; k < NB; ++k) {
            const int sp = min(s0 + NG * k, ns - 1);
            const int64_t idx = base + (int64_t)sp * a.Hq;
            ml[k] = pm[idx];
            ov[k] = *(const f32x4*)(po + idx * a.d + x0);
        }
#pragma unroll
        for (int k = 0; k < NB; ++k)
            if (s0 + NG * k < ns) acc = merge_acc(acc, MergeAcc{ml[k].x, ml[k].y, ml[k].z, ov[k]});
    }
    // groups g of a wave differ in lane bits 2..5
#pragma unroll
    for (int sh = 4; sh < 64; sh <<= 1) {
        MergeAcc y;
        y.m = __shfl_xor(acc.m, sh);
        y.lo = __shfl_xor(acc.lo, sh);
        y.ll = __shfl_xor(acc.ll, sh);
#pragma unroll
        for (int i = 0; i < 4; ++i) y.o[i] = __shfl_xor(acc.o[i], sh);
        acc = merge_acc(acc, y);
    }
    if ((tid & 63) < 4) {
        sm[wave][q4] = acc.m;
        slo[wave][q4] = acc.lo;
        sll[wave][q4] = acc.ll;
        so[wave][q4] = acc.o;
    }
    __syncthreads();
    if (tid < 4) {
#pragma unroll
        for (int w = 1; w < 4; ++w)
            acc = merge_acc(acc, MergeAcc{sm[w][q4], slo[w][q4], sll[w][q4], so[w][q4]});
        const float inv = acc.lo > 0.0f ? 1.0f / acc.lo : 0.0f;
        TOUT* o = (TOUT*)a.o + ((int64_t)b * a.Hq + head) * a.d + x0;
#pragma unroll
        for (int i = 0; i < 4; ++i) o[i] = (TOUT)(acc.o[i] * inv);
        if (blockIdx.z == 0 && q4 == 0)
            a.lse[(int64_t)b * a.Hq + head] =
                acc.ll > 0.0f ? (acc.m + log2f(acc.ll)) * kLn2 : -INFINITY;
    }
}

template <int D, typename TIN, int GQ>
static hipError_t launch_decode_g(const DecodeArgs& a, hipStream_t s) {
    const int wmax = sizeof(TIN) == 2 ? kWavesB : kDecodeWaves;
    const int nw = a.Hkv < wmax ? a.Hkv : wmax;
    const dim3 grid(a.lay.n_splits, (a.Hkv + nw - 1) / nw, a.B);
    LaunchScope scope(a.bifocal ? (a.precise ? "decode_split_precise" : "decode_split")
                                : "decode_split_plain", s);
    if constexpr (sizeof(TIN) == 2) {
        // (bifocal, paged, fp8) -> one instantiation each; split precision
        // for bifocal bf16 caches (plain decode has no remote keys)
        const int sel = (a.bifocal ? 4 : 0) | (a.block_table ? 2 : 0) | (a.fp8 ? 1 : 0);
        const dim3 blk(64 * nw);
        if (a.bifocal && a.precise && !a.fp8) {
            if (a.block_table)
                hipLaunchKernelGGL((decode_split_bf16_kernel<D, true, GQ, true, false, true>), grid, blk, 0, s, a);
            else
                hipLaunchKernelGGL((decode_split_bf16_kernel<D, true, GQ, false, false, true>), grid, blk, 0, s, a);
            return hipGetLastError();
        }
        switch (sel) {
            case 0: hipLaunchKernelGGL((decode_split_bf16_kernel<D, false, GQ, false, false>), grid, blk, 0, s, a); break;
            case 1: hipLaunchKernelGGL((decode_split_bf16_kernel<D, false, GQ, false, true>), grid, blk, 0, s, a); break;
            case 2: hipLaunchKernelGGL((decode_split_bf16_kernel<D, false, GQ, true, false>), grid, blk, 0, s, a); break;
            case 3: hipLaunchKernelGGL((decode_split_bf16_kernel<D, false, GQ, true, true>), grid, blk, 0, s, a); break;
            case 4: hipLaunchKernelGGL((decode_split_bf16_kernel<D, true, GQ, false, false>), grid, blk, 0, s, a); break;
            case 5: hipLaunchKernelGGL((decode_split_bf16_kernel<D, true, GQ, false, true>), grid, blk, 0, s, a); break;
            case 6: hipLaunchKernelGGL((decode_split_bf16_kernel<D, true, GQ, true, false>), grid, blk, 0, s, a); break;
            default: hipLaunchKernelGGL((decode_split_bf16_kernel<D, true, GQ, true, true>), grid, blk, 0, s, a); break;
        }
    } else {
        if (a.bifocal)
            hipLaunchKernelGGL((decode_split_kernel<D, TIN, true, GQ>), grid, dim3(64 * nw), 0, s, a);
        else
            hipLaunchKernelGGL((decode_split_kernel<D, TIN, false, GQ>), grid, dim3(64 * nw), 0, s, a);
    }
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
    if (a.o_f32)  // float32 output (the unfused decode's intermediates)
        hipLaunchKernelGGL(decode_merge_kernel<float>, dim3(a.Hq, a.B, D / 16), dim3(256), 0, s, a);
    else
        hipLaunchKernelGGL(decode_merge_kernel<TIN>, dim3(a.Hq, a.B, D / 16), dim3(256), 0, s, a);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// The pages' unfused generation step ([TW] §四, [BT] §3.2): the cache holds
// standard-RoPE keys, so call B (every key under remapped RoPE) first needs
// the whole cache turned to remapped RoPE: out[b][j] = R(f(j) - j) k[b][j]
// for j < L_b, G = G(L_b) -- the correction rotation of [BT] §3.3 applied
// to every key and stored.  One thread per (sequence, row, 8 pairs), the
// angles shared by all kv heads; rows j >= L_b are not written.
template <int D>
__global__ __launch_bounds__(256) void cache_remap_kernel(bf16* __restrict__ out,
                                                          const bf16* __restrict__ kc,
                                                          const int32_t* __restrict__ seqlens,
                                                          int32_t B, int32_t max_seqlen_k,
                                                          int64_t S_max, int32_t Hkv,
                                                          int32_t w_pretrained, RopeFreq tab) {
    constexpr int HALF = D / 2, NC = HALF / 8;
    const int64_t item = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (item >= (int64_t)B * max_seqlen_k * NC) return;
    const int c = (int)(item % NC);
    const int64_t row = item / NC;
    const int b = (int)(row / max_seqlen_k);
    const int32_t j = (int32_t)(row % max_seqlen_k);
    int32_t L = seqlens[b];
    L = L < 0 ? 0 : (L > max_seqlen_k ? max_seqlen_k : L);
    if (j >= L) return;
    const int32_t G = (int32_t)group_size(L, w_pretrained);
    const int32_t ang = remap(j, G) - j;
    float cs[8], sn[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) rope_cs(ang, rope_rev(tab, 8 * c + u), cs[u], sn[u]);
    for (int g = 0; g < Hkv; ++g) {
        const bf16* src = kc + (((int64_t)b * S_max + j) * Hkv + g) * D + 8 * c;
        bf16* dst = out + (((int64_t)b * max_seqlen_k + j) * Hkv + g) * D + 8 * c;
        const bf16x8 x0 = *reinterpret_cast<const bf16x8*>(src);
        const bf16x8 x1 = *reinterpret_cast<const bf16x8*>(src + HALF);
        bf16x8 y0, y1;
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const float a0 = (float)x0[u], a1 = (float)x1[u];
            y0[u] = (bf16)(a0 * cs[u] - a1 * sn[u]);
            y1[u] = (bf16)(a1 * cs[u] + a0 * sn[u]);
        }
        *reinterpret_cast<bf16x8*>(dst) = y0;
        *reinterpret_cast<bf16x8*>(dst + HALF) = y1;
    }
}

hipError_t launch_cache_remap(void* out, const void* kc, const int32_t* seqlens, int32_t B,
                              int32_t max_seqlen_k, int64_t S_max, int32_t Hkv, int32_t d,
                              int32_t w_pretrained, const RopeFreq& tab, hipStream_t s) {
    const int64_t items = (int64_t)B * max_seqlen_k * (d / 16);
    const dim3 grid((unsigned)((items + 255) / 256));
    LaunchScope scope("cache_remap", s);
    if (d == 128)
        hipLaunchKernelGGL(cache_remap_kernel<128>, grid, dim3(256), 0, s, (bf16*)out,
                           (const bf16*)kc, seqlens, B, max_seqlen_k, S_max, Hkv, w_pretrained, tab);
    else
        hipLaunchKernelGGL(cache_remap_kernel<64>, grid, dim3(256), 0, s, (bf16*)out,
                           (const bf16*)kc, seqlens, B, max_seqlen_k, S_max, Hkv, w_pretrained, tab);
    return hipGetLastError();
}

// LogSumExp combination of the pages' three unfused calls ([TW] §四, [BT]
// §3.2): with B every causal pair under remapped RoPE, A the local pairs
// under standard RoPE and C the local pairs under remapped RoPE,
//   Z = e^lse_B - e^lse_C + e^lse_A,  o = (e^lse_B o_B - e^lse_C o_C + e^lse_A o_A) / Z.
// B and C hold the same local pairs, so the remote mass e^lse_B - e^lse_C is
// taken relative to e^lse_B and clamped at 0 (rows with no remote key give 0
// up to rounding); a clamped remote part contributes nothing.  The three
// calls' outputs are fp32, so the difference e^lse_B o_B - e^lse_C o_C does
// not cancel rounded values.  Row r, head h: o at (r Hq + h) d, lse at
// r * ls_r + h * ls_h (prefill [Hq][T]: ls_r = 1, ls_h = T; decode [B][Hq]:
// ls_r = Hq, ls_h = 1).  One wave per (row, head); lse is the natural log,
// and lse_B is finite for every row that has a key (its own key is in B).
__global__ __launch_bounds__(256) void three_call_merge_kernel(
    const float* __restrict__ oA, const float* __restrict__ oB, const float* __restrict__ oC,
    const float* __restrict__ lA, const float* __restrict__ lB, const float* __restrict__ lC,
    bf16* __restrict__ o, float* __restrict__ lse, int64_t rows, int Hq, int d, int64_t ls_r,
    int64_t ls_h) {
    const int64_t r = blockIdx.x;
    const int head = blockIdx.y * 4 + (int)(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    if (head >= Hq) return;
    const int64_t li = r * ls_r + (int64_t)head * ls_h;
    const float la = lA[li], lb = lB[li], lc = lC[li];
    const int64_t base = (r * Hq + head) * d;
    if (!(lb > -INFINITY)) {  // a row with no key (an empty decode sequence)
        for (int x = lane; x < d; x += 64) o[base + x] = (bf16)0.0f;
        if (lane == 0) lse[li] = -INFINITY;
        return;
    }
    const float ec = expf(lc - lb);
    const float rem = fmaxf(0.0f, 1.0f - ec);  // remote mass / e^lse_B
    const float loc = expf(la - lb);           // local mass / e^lse_B
    const float z = rem + loc;
    const float wB = rem > 0.0f ? 1.0f / z : 0.0f;
    const float wC = rem > 0.0f ? ec / z : 0.0f;
    const float wA = loc / z;
    for (int x = lane; x < d; x += 64)
        o[base + x] = (bf16)(wB * oB[base + x] - wC * oC[base + x] + wA * oA[base + x]);
    if (lane == 0) lse[li] = lb + logf(z);
}

hipError_t launch_three_call_merge(const float* oA, const float* oB, const float* oC,
                                   const float* lA, const float* lB, const float* lC, void* o,
                                   float* lse, int64_t rows, int32_t Hq, int32_t d, int64_t ls_r,
                                   int64_t ls_h, hipStream_t s) {
    LaunchScope scope("three_call_merge", s);
    hipLaunchKernelGGL(three_call_merge_kernel, dim3((unsigned)rows, (unsigned)((Hq + 3) / 4)),
                       dim3(256), 0, s, oA, oB, oC, lA, lB, lC, (bf16*)o, lse, rows, (int)Hq,
                       (int)d, ls_r, ls_h);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// fp8 cache writer: one thread per 8 elements of a row (d / 8 threads per
// (token, head)); the quotient x / scale is a correctly rounded fp32
// division, clamped to +-448 and rounded to nearest even by
// v_cvt_pk_fp8_f32.  NaN stays NaN.
__global__ __launch_bounds__(256) void e4m3_quant_kernel(uint8_t* __restrict__ out,
                                                         const bf16* __restrict__ x,
                                                         const float* __restrict__ scale,
                                                         int64_t n8, int32_t H, int32_t d) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= n8) return;
    const int h = (int)((i * 8 / d) % H);
    const float sc = scale[h];
    const bf16x8 v = *reinterpret_cast<const bf16x8*>(x + 8 * i);
    uint32_t w[2];
#pragma unroll
    for (int half = 0; half < 2; ++half) {
        float q[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const float y = (float)v[4 * half + u] / sc;
            q[u] = y != y ? y : __builtin_amdgcn_fmed3f(y, 448.0f, -448.0f);
        }
        int pk = __builtin_amdgcn_cvt_pk_fp8_f32(q[0], q[1], 0, false);
        pk = __builtin_amdgcn_cvt_pk_fp8_f32(q[2], q[3], pk, true);
        w[half] = (uint32_t)pk;
    }
    *reinterpret_cast<u32x2*>(out + 8 * i) = u32x2{w[0], w[1]};
}

hipError_t launch_e4m3_quant(uint8_t* out, const void* x, const float* scale, int64_t ntok,
                             int32_t H, int32_t d, hipStream_t s) {
    const int64_t n8 = ntok * H * (d / 8);
    LaunchScope scope("e4m3_quant", s);
    hipLaunchKernelGGL(e4m3_quant_kernel, dim3((unsigned)((n8 + 255) / 256)), dim3(256), 0, s,
                       out, (const bf16*)x, scale, n8, H, d);
    return hipGetLastError();
}

hipError_t launch_decode(const DecodeArgs& a, int dtype, hipStream_t s) {
    if (dtype == 1) return a.d == 128 ? launch_decode_t<128, bf16>(a, s) : launch_decode_t<64, bf16>(a, s);
    return a.d == 128 ? launch_decode_t<128, float>(a, s) : launch_decode_t<64, float>(a, s);
}

}  // namespace jl
