// rope.hip -- RoPE rotation kernels, the prefill plan and the key/value
// pre-pass that lays K and V out for the attention kernels.
//
// Pages cited (title, section):
//   [BT] "Jet-Long: 具有动态双焦RoPE的高效长上下文扩展" (bittide.aicompass.dev)
//   [TW] "NVIDIA研究团队找到了让AI“看清”超长文本的新方法" (techwalker.com)
#include "internal.h"

namespace jl {

// ---------------------------------------------------------------------------
// out[t][h] = R(floor(pos[t] / G)) x[t][h]; one thread per (token, pair t),
// the angle computed once and reused for all H heads of the token.
template <typename T>
__global__ __launch_bounds__(256) void rope_apply_kernel(T* __restrict__ out,
                                                         const T* __restrict__ x,
                                                         const int32_t* __restrict__ pos,
                                                         int64_t ntok, int32_t H, int32_t d,
                                                         RopeFreq tab, int32_t G) {
    const int half = d / 2;
    const int64_t item = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (item >= ntok * half) return;
    const int64_t tok = item / half;
    const int t = (int)(item % half);
    const int32_t p = remap(pos[tok], G);
    float c, s;
    rope_cs(p, rope_rev(tab, t), c, s);
    for (int h = 0; h < H; ++h) {
        const int64_t base = (tok * H + h) * (int64_t)d;
        const float x0 = (float)x[base + t];
        const float x1 = (float)x[base + t + half];
        out[base + t] = (T)(x0 * c - x1 * s);
        out[base + t + half] = (T)(x1 * c + x0 * s);
    }
}

hipError_t launch_rope_apply(void* out, const void* x, const int32_t* pos, int64_t T, int32_t H,
                             int32_t d, const RopeFreq& tab, int32_t G, int dtype,
                             hipStream_t s) {
    const int64_t items = T * (d / 2);
    const dim3 grid((unsigned)((items + 255) / 256));
    LaunchScope scope("rope_apply", s);
    if (dtype == 1)
        hipLaunchKernelGGL(rope_apply_kernel<bf16>, grid, dim3(256), 0, s, (bf16*)out,
                           (const bf16*)x, pos, T, H, d, tab, G);
    else
        hipLaunchKernelGGL(rope_apply_kernel<float>, grid, dim3(256), 0, s, (float*)out,
                           (const float*)x, pos, T, H, d, tab, G);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Plan: per-sequence start, length, G ([BT] §3.1: one G per sequence from its
// own length) and the offsets of the padded key layouts.  One thread; the
// number of sequences is small next to the attention work.  If cu_seqlens
// breaks its contract every length is set to 0 (all kernels then do nothing)
// and the "bad" flag is raised, so no kernel leaves its buffers.
__global__ void plan_kernel(int32_t* __restrict__ plan, const int32_t* __restrict__ cu,
                            int32_t n_seqs, int64_t T, int32_t max_seqlen, int32_t w_pretrained,
                            int32_t precise) {
    if (threadIdx.x != 0 || blockIdx.x != 0) return;
    bool bad = false;
    if (cu) {
        if (cu[0] != 0 || (int64_t)cu[n_seqs] != T) bad = true;
        for (int s = 0; s < n_seqs && !bad; ++s) {
            const int64_t len = (int64_t)cu[s + 1] - cu[s];
            if (len < 1 || len > max_seqlen) bad = true;
        }
    }
    int64_t pad = 0, lo = 0;
    for (int s = 0; s < n_seqs; ++s) {
        int32_t* e = plan + s * kPlanFields;
        const int32_t start = cu ? cu[s] : 0;
        const int32_t len = bad ? 0 : (cu ? cu[s + 1] - cu[s] : (int32_t)T);
        e[kPlanStart] = bad ? 0 : start;
        e[kPlanLen] = len;
        e[kPlanG] = (int32_t)group_size(len, w_pretrained);
        e[kPlanPadOff] = (int32_t)pad;
        e[kPlanLoOff] = (int32_t)lo;
        e[kPlanTile0] = (int32_t)(pad / kBN);
        e[kPlanLoTile0] = (int32_t)(lo / kBN);
        e[kPlanBad] = 0;
        e[kPlanQ0] = 0;
        e[kPlanKeep] = 0;
        pad += (len + kBN - 1) / kBN * kBN;
        const int32_t nlo = (precise || len < kPreciseRows) ? len : kPreciseRows;
        lo += (nlo + kBN - 1) / kBN * kBN;
    }
    int32_t* e = plan + n_seqs * kPlanFields;
    e[kPlanStart] = (int32_t)T;
    e[kPlanLen] = 0;
    e[kPlanG] = 1;
    e[kPlanPadOff] = (int32_t)pad;
    e[kPlanLoOff] = (int32_t)lo;
    e[kPlanTile0] = (int32_t)(pad / kBN);
    e[kPlanLoTile0] = (int32_t)(lo / kBN);
    e[kPlanBad] = bad ? 1 : 0;
    e[kPlanQ0] = 0;
    e[kPlanKeep] = 0;
}

hipError_t launch_plan(int32_t* plan, const int32_t* cu, int32_t n_seqs, int64_t T,
                       int32_t max_seqlen, int32_t w_pretrained, int32_t precise, hipStream_t s) {
    LaunchScope scope("plan", s);
    hipLaunchKernelGGL(plan_kernel, dim3(1), dim3(64), 0, s, plan, cu, n_seqs, T, max_seqlen,
                       w_pretrained, precise);
    return hipGetLastError();
}

// Plan of a chunk call ([TW] §三: new rows appended to a cache of
// standard-RoPE keys).  Sequence b has L_b = seqlens_k[b] keys in the cache,
// its own C_b = cu_q[b + 1] - cu_q[b] new rows among them, and one G from L_b
// ([BT] §3.1).  Its key tiles cover [0, L_b); its query rows are positions
// [L_b - C_b, L_b).  A sequence with no new row gets length 0 (no work).  If
// the device arrays break their contract (cu_q not starting at 0 or ending at
// Tq, C_b outside [0, max_seqlen_q], L_b outside [C_b, max_seqlen_k]) every
// length is 0 and the bad flag is raised.
// Every sequence owns a fixed stretch of the image layout (room for
// max_seqlen_k keys), so that its images stay in place from call to call.
// With reuse, the leading whole tiles an earlier call built for this
// sequence are kept (kPlanKeep) when the record in image_state is this
// call's (magic and fingerprint) and the images still hold: the same G for
// bifocal 1 (f depends on G alone), the same L for bifocal 2 (its remote
// positions scale with L), always for plain RoPE.  The record is then
// rewritten for this call: sequences with rows here get their L and G;
// the others keep their entry if the old record was trusted, else none.
__global__ void plan_chunk_kernel(int32_t* __restrict__ plan, void* __restrict__ image_state,
                                  uint64_t fingerprint, int32_t reuse,
                                  const int32_t* __restrict__ cu_q,
                                  const int32_t* __restrict__ seqlens_k, int32_t B, int64_t Tq,
                                  int32_t max_seqlen_q, int32_t max_seqlen_k,
                                  int32_t w_pretrained, int32_t precise, int32_t bifocal) {
    if (threadIdx.x != 0 || blockIdx.x != 0) return;
    bool bad = cu_q && (cu_q[0] != 0 || (int64_t)cu_q[B] != Tq);
    for (int b = 0; b < B && !bad; ++b) {
        const int64_t C = cu_q ? (int64_t)cu_q[b + 1] - cu_q[b] : Tq;
        const int32_t L = seqlens_k[b];
        if (C < 0 || C > max_seqlen_q || L < C || L > max_seqlen_k) bad = true;
    }
    uint64_t* hdr = (uint64_t*)image_state;
    int32_t* built = (int32_t*)(hdr + 2);
    const bool trusted = reuse && hdr[0] == kImageMagic && hdr[1] == fingerprint;
    const int32_t tps = (max_seqlen_k + kBN - 1) / kBN;  // tiles per sequence
    const int32_t nlo = (precise || max_seqlen_k < kPreciseRows) ? max_seqlen_k : kPreciseRows;
    const int32_t ltps = (nlo + kBN - 1) / kBN;          // lo tiles per sequence
    for (int b = 0; b < B; ++b) {
        int32_t* e = plan + b * kPlanFields;
        const int32_t start = cu_q ? cu_q[b] : 0;
        const int32_t C = cu_q ? cu_q[b + 1] - cu_q[b] : (int32_t)Tq;
        const int32_t len = (bad || C == 0) ? 0 : seqlens_k[b];
        const int32_t G = (int32_t)group_size(len, w_pretrained);
        int32_t keep = 0;
        if (trusted && len > 0) {
            const int32_t Lb = built[2 * b], Gb = built[2 * b + 1];
            const bool valid = bifocal == 0 || (bifocal == 1 && Gb == G) || (bifocal == 2 && Lb == len);
            if (valid) keep = (Lb < len ? Lb : len) / kBN;
        }
        e[kPlanStart] = bad ? 0 : start;
        e[kPlanLen] = len;
        e[kPlanG] = G;
        e[kPlanPadOff] = b * tps * kBN;
        e[kPlanLoOff] = b * ltps * kBN;
        e[kPlanTile0] = b * tps;
        e[kPlanLoTile0] = b * ltps;
        e[kPlanBad] = 0;
        e[kPlanQ0] = len - (len ? C : 0);
        e[kPlanKeep] = keep;
    }
    int32_t* e = plan + B * kPlanFields;
    e[kPlanStart] = (int32_t)Tq;
    e[kPlanLen] = 0;
    e[kPlanG] = 1;
    e[kPlanPadOff] = B * tps * kBN;
    e[kPlanLoOff] = B * ltps * kBN;
    e[kPlanTile0] = B * tps;
    e[kPlanLoTile0] = B * ltps;
    e[kPlanBad] = bad ? 1 : 0;
    e[kPlanQ0] = 0;
    e[kPlanKeep] = 0;
    for (int b = 0; b < B; ++b) {
        const int32_t* eb = plan + b * kPlanFields;
        if (eb[kPlanLen] > 0) {
            built[2 * b] = eb[kPlanLen];
            built[2 * b + 1] = eb[kPlanG];
        } else if (!trusted) {
            built[2 * b] = 0;
            built[2 * b + 1] = 0;
        }
    }
    hdr[0] = kImageMagic;
    hdr[1] = fingerprint;
}

hipError_t launch_plan_chunk(int32_t* plan, void* image_state, uint64_t fingerprint, int32_t reuse,
                             const int32_t* cu_q, const int32_t* seqlens_k,
                             int32_t B, int64_t Tq, int32_t max_seqlen_q, int32_t max_seqlen_k,
                             int32_t w_pretrained, int32_t precise, int32_t bifocal, hipStream_t s) {
    LaunchScope scope("plan", s);
    hipLaunchKernelGGL(plan_chunk_kernel, dim3(1), dim3(64), 0, s, plan, image_state, fingerprint,
                       reuse, cu_q, seqlens_k, B, Tq, max_seqlen_q, max_seqlen_k, w_pretrained,
                       precise, bifocal);
    return hipGetLastError();
}

// Sequence owning padded key tile `tile` (plan tile0 is non-decreasing);
// -1 if the tile is beyond the last sequence.
__device__ inline int seq_of_tile(const int32_t* plan, int n_seqs, int tile) {
    if (tile >= plan[n_seqs * kPlanFields + kPlanTile0]) return -1;
    int lo = 0, hi = n_seqs - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) / 2;
        if (plan[mid * kPlanFields + kPlanTile0] <= tile) lo = mid;
        else hi = mid - 1;
    }
    return lo;
}

// Order of keys inside each group of 16 in the transposed V tile.  The
// prefill kernel's P operand holds, in lane half h, the keys
// {4h..4h+3, 8+4h..8+4h+3} of a 16-key step; storing the group as
// [0..3, 8..11, 4..7, 12..15] lets that half read its 8 keys as one 16-byte
// vector.  The permutation is its own inverse.
__host__ __device__ constexpr int vt_perm16(int p) {
    return (p & 4) != ((p >> 1) & 4) ? (p ^ 12) : p;
}

// ---------------------------------------------------------------------------
// Key/value pre-pass of the bf16 prefill (one workgroup per padded key tile,
// looping over kv heads so each (position, pair) angle is computed once):
//   KS[g][row]  = R(n) k_n            (standard RoPE, [TW] §二), fp16
//   KR[g][row]  = R(f(n)) k_n         (remapped RoPE, [BT] §3.1; only if G > 1), fp16
// In a chunk call the source rows are cache rows c_n = R(n) k_n, so
// KS = c_n and KR = R(f(n) - n) c_n (the correction rotation of [BT] §3.3).
//   KS_lo/KR_lo = f16(x - f16(x))     for n < kPreciseRows, or every n when the
//                                     call asks for split precision on all rows
//   VT[g][tile][d][key']              V tile transposed to fp16, keys in vt_perm16 order
// Every tile is written in the piece-major image layout (kt_off, vt_off).
//   k_rot_out[tok][g] = KS row        (optional, the caller's cache layout)
// Pad rows (n >= L) are written as zeros so masked keys never meet NaNs.
template <int D>
__global__ __launch_bounds__(256) void kv_prepass_bf16_kernel(PrefillArgs a) {
    constexpr int HALF = D / 2;
    __shared__ __align__(16) bf16 vs[kBN * (D + 8)];
    __shared__ int64_t vrow[kBN];

    const int32_t* plan = (const int32_t*)((char*)a.ws + a.lay.plan);
    f16* KS = (f16*)((char*)a.ws + a.lay.ks);
    f16* KR = (f16*)((char*)a.ws + a.lay.kr);
    f16* VT = (f16*)((char*)a.ws + a.lay.vt);
    f16* KSlo = (f16*)((char*)a.ws + a.lay.ks_lo);
    f16* KRlo = (f16*)((char*)a.ws + a.lay.kr_lo);
    const bf16* k = (const bf16*)a.k;
    const bf16* v = (const bf16*)a.v;
    bf16* krot = (bf16*)a.k_rot_out;

    const int tile = blockIdx.x;
    const int s = seq_of_tile(plan, a.n_seqs, tile);
    if (s < 0) return;
    const int32_t* e = plan + s * kPlanFields;
    const int32_t start = e[kPlanStart], len = e[kPlanLen], G = e[kPlanG];
    const bool bif = a.bifocal && G > 1;
    const int32_t n0 = (tile - e[kPlanTile0]) * kBN;  // first position of the tile
    // chunk calls: tiles past the sequence's keys (its stretch of the fixed
    // layout) are never read, and kept tiles are already built
    if (n0 >= len || tile - e[kPlanTile0] < e[kPlanKeep]) return;
    const bool cache = a.chunked != 0;
    // source row of position nn < len: the packed input, or the cache
    auto src_row = [&](int32_t nn) -> int64_t {
        if (!cache) return (int64_t)start + nn;
        if (!a.block_table) return (int64_t)s * a.S_max + nn;
        int32_t pg = a.block_table[(int64_t)s * a.bt_stride + (nn >> a.page_shift)];
        pg = pg < 0 ? 0 : (pg >= a.n_pages ? a.n_pages - 1 : pg);
        return ((int64_t)pg << a.page_shift) | (nn & ((1 << a.page_shift) - 1));
    };

    // ---- keys: thread (r, c) rotates pairs [8c, 8c + 8) of row r: one
    // 16-byte vector in each RoPE half, that is tile pieces c and
    // c + D / 16; 256 / (D / 16) rows per pass ----
    constexpr int TPR = D / 16;          // threads per key row
    constexpr int RPP = 256 / TPR;       // rows per pass
    // remote position: f(n) = floor(n / G), or n / s with s = len / w_pretrained
    // for the continuous-interpolation variant (bifocal 2)
    const bool interp = a.bifocal == 2;
    const double rsc = interp ? (double)a.w_pretrained / (double)len : 1.0;
    for (int pass = 0; pass < kBN / RPP; ++pass) {
        const int r = pass * RPP + (int)threadIdx.x / TPR, c = (int)threadIdx.x % TPR;
        const int32_t n = n0 + r;
        const bool valid = n < len;
        const bool lo_row = n < kPreciseRows || a.precise;
        const int64_t krow = valid ? src_row(n) : 0;
        if (c == 0) vrow[r] = krow;  // published by the first barrier of the value loop
        float cs[8], sn[8], cr[8], sr[8];
        if (valid) {
            const int32_t fn = remap(n, G);
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                const double rv = rope_rev(a.tab, 8 * c + u);
                rope_cs(cache ? 0 : n, rv, cs[u], sn[u]);
                if (bif) {
                    if (interp) rope_cs(n, rv * (cache ? rsc - 1.0 : rsc), cr[u], sr[u]);
                    else rope_cs(cache ? fn - n : fn, rv, cr[u], sr[u]);
                }
            }
        } else {
            // pad rows (n >= len): zero angles on zero data give zero tiles
#pragma unroll
            for (int u = 0; u < 8; ++u) cs[u] = sn[u] = cr[u] = sr[u] = 0.0f;
        }
        for (int g = 0; g < a.Hkv; ++g) {
            bf16x8 xa = bf16x8{}, xb = bf16x8{};
            if (valid) {
                const bf16* src = k + (krow * a.Hkv + g) * D + 8 * c;
                xa = *reinterpret_cast<const bf16x8*>(src);
                xb = *reinterpret_cast<const bf16x8*>(src + HALF);
            }
            f16x8 ys0, ys1, yr0, yr1, ls0, ls1, lr0, lr1;
            bf16x8 kb0, kb1;
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                const float x0 = (float)xa[u], x1 = (float)xb[u];
                const float s0 = x0 * cs[u] - x1 * sn[u];
                const float s1 = x1 * cs[u] + x0 * sn[u];
                ys0[u] = (f16)s0;
                ys1[u] = (f16)s1;
                ls0[u] = (f16)(s0 - (float)ys0[u]);
                ls1[u] = (f16)(s1 - (float)ys1[u]);
                kb0[u] = (bf16)s0;
                kb1[u] = (bf16)s1;
                if (bif) {
                    const float r0 = x0 * cr[u] - x1 * sr[u];
                    const float r1 = x1 * cr[u] + x0 * sr[u];
                    yr0[u] = (f16)r0;
                    yr1[u] = (f16)r1;
                    lr0[u] = (f16)(r0 - (float)yr0[u]);
                    lr1[u] = (f16)(r1 - (float)yr1[u]);
                }
            }
            // tile image: pieces c and c + TPR of row r of tile `tile` (the
            // eight lanes of one piece write one whole 128-byte line)
            const int64_t dt = ((int64_t)g * (a.lay.T_pad / kBN) + tile) * ktile_elems(D);
            const int o0 = kt_off(r, c), o1 = kt_off(r, c + TPR);
            *reinterpret_cast<f16x8*>(KS + dt + o0) = ys0;
            *reinterpret_cast<f16x8*>(KS + dt + o1) = ys1;
            if (bif) {
                *reinterpret_cast<f16x8*>(KR + dt + o0) = yr0;
                *reinterpret_cast<f16x8*>(KR + dt + o1) = yr1;
            }
            if (lo_row) {
                const int64_t lt =
                    ((int64_t)g * (a.lay.lo_pad / kBN) + e[kPlanLoTile0] + n / kBN) * ktile_elems(D);
                const int l0 = kt_off(n % kBN, c), l1 = kt_off(n % kBN, c + TPR);
                *reinterpret_cast<f16x8*>(KSlo + lt + l0) = ls0;
                *reinterpret_cast<f16x8*>(KSlo + lt + l1) = ls1;
                if (bif) {
                    *reinterpret_cast<f16x8*>(KRlo + lt + l0) = lr0;
                    *reinterpret_cast<f16x8*>(KRlo + lt + l1) = lr1;
                }
            }
            if (krot && valid) {
                bf16* dst = krot + ((int64_t)(start + n) * a.Hkv + g) * D + 8 * c;
                *reinterpret_cast<bf16x8*>(dst) = kb0;
                *reinterpret_cast<bf16x8*>(dst + HALF) = kb1;
            }
        }
    }

    // ---- values: transpose each head's [kBN][D] tile through LDS ----
    // (source rows of the tile's positions shared through LDS; the first
    // barrier of the loop publishes them).  Rows are read and the transposed
    // tile written in 16-byte vectors: output vector (d, m) holds the keys of
    // positions 8m .. 8m + 7 of row d in vt_perm16 order.
    constexpr int VSS = D + 8;  // LDS row stride (halves), 16-byte aligned rows
    for (int g = 0; g < a.Hkv; ++g) {
        __syncthreads();
        for (int idx = threadIdx.x; idx < kBN * (D / 8); idx += 256) {
            const int rr = idx / (D / 8), ch = idx % (D / 8);
            const int32_t nn = n0 + rr;
            bf16x8 x = bf16x8{};
            if (nn < len) x = *reinterpret_cast<const bf16x8*>(v + (vrow[rr] * a.Hkv + g) * D + 8 * ch);
            *reinterpret_cast<bf16x8*>(vs + rr * VSS + 8 * ch) = x;
        }
        __syncthreads();
        f16* dst = VT + ((int64_t)g * (a.lay.T_pad / kBN) + tile) * vtile_elems(D);
        // consecutive threads take consecutive rows dd of one piece m: a wave
        // writes 1 KB contiguous
        for (int idx = threadIdx.x; idx < D * (kBN / 8); idx += 256) {
            const int dd = idx % D, m = idx / D;
            f16x8 o;
#pragma unroll
            for (int e8 = 0; e8 < 8; ++e8) {
                const int p = 8 * m + e8;
                const int key = (p & ~15) | vt_perm16(p & 15);
                o[e8] = (f16)(float)vs[key * VSS + dd];
            }
            *reinterpret_cast<f16x8*>(dst + vt_off(D, dd, m)) = o;
        }
    }
}

// fp32 path: rotated keys in the caller's token order, [Hkv][T][D] fp32.
__global__ __launch_bounds__(256) void kv_prepass_f32_kernel(PrefillArgs a) {
    const int32_t* plan = (const int32_t*)((char*)a.ws + a.lay.plan);
    float* KS = (float*)((char*)a.ws + a.lay.ks32);
    float* KR = (float*)((char*)a.ws + a.lay.kr32);
    const float* k = (const float*)a.k;
    float* krot = (float*)a.k_rot_out;
    const int half = a.d / 2;
    const int64_t item = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (item >= a.T * half) return;
    const int64_t tok = item / half;
    const int t = (int)(item % half);
    // sequence of this token (linear scan: the fp32 path serves small cases)
    int s = 0;
    while (s + 1 < a.n_seqs && tok >= plan[(s + 1) * kPlanFields + kPlanStart]) ++s;
    const int32_t* e = plan + s * kPlanFields;
    if (tok < e[kPlanStart] || tok >= (int64_t)e[kPlanStart] + e[kPlanLen]) return;
    const int32_t n = (int32_t)(tok - e[kPlanStart]);
    float cs, sn, cr, sr;
    const double rv = rope_rev(a.tab, t);
    rope_cs(n, rv, cs, sn);
    rope_cs(remap(n, e[kPlanG]), rv, cr, sr);
    for (int g = 0; g < a.Hkv; ++g) {
        const float* src = k + (tok * a.Hkv + g) * (int64_t)a.d;
        const float x0 = src[t], x1 = src[t + half];
        const int64_t dst = ((int64_t)g * a.T + tok) * a.d;
        KS[dst + t] = x0 * cs - x1 * sn;
        KS[dst + t + half] = x1 * cs + x0 * sn;
        KR[dst + t] = x0 * cr - x1 * sr;
        KR[dst + t + half] = x1 * cr + x0 * sr;
        if (krot) {
            float* o = krot + (tok * a.Hkv + g) * (int64_t)a.d;
            o[t] = KS[dst + t];
            o[t + half] = KS[dst + t + half];
        }
    }
}

hipError_t launch_kv_prepass(const PrefillArgs& a, int dtype, hipStream_t s) {
    if (dtype == 1) {
        LaunchScope scope("kv_prepass_bf16", s);
        const dim3 grid((unsigned)(a.lay.T_pad / kBN));
        if (a.d == 128)
            hipLaunchKernelGGL(kv_prepass_bf16_kernel<128>, grid, dim3(256), 0, s, a);
        else
            hipLaunchKernelGGL(kv_prepass_bf16_kernel<64>, grid, dim3(256), 0, s, a);
    } else {
        LaunchScope scope("kv_prepass_f32", s);
        const int64_t items = a.T * (a.d / 2);
        hipLaunchKernelGGL(kv_prepass_f32_kernel, dim3((unsigned)((items + 255) / 256)),
                           dim3(256), 0, s, a);
    }
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Test export of the index math the kernels use.
__global__ void debug_index_kernel(int64_t L, int32_t w_pretrained, int32_t w_local,
                                   int32_t bifocal, int32_t bm, int32_t bn, int32_t* G_out,
                                   int32_t* f_out, uint8_t* band_out, uint8_t* tile_out) {
    const int64_t G = group_size(L, w_pretrained);
    const bool bif = bifocal && G > 1;
    const int64_t n = L < 1024 ? L : 1024;
    const int64_t nt_i = (L + bm - 1) / bm, nt_j = (L + bn - 1) / bn;
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    const int64_t id0 = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (id0 == 0) G_out[0] = (int32_t)G;
    for (int64_t x = id0; x < L; x += stride) f_out[x] = remap((int32_t)x, (int32_t)G);
    for (int64_t x = id0; x < n * n; x += stride)
        band_out[x] = (uint8_t)band(x / n, x % n, w_local, bif);
    for (int64_t x = id0; x < nt_i * nt_j; x += stride) {
        const int64_t a = x / nt_j, b = x % nt_j;
        const int64_t i0 = a * bm, i1 = (a + 1) * bm < L ? (a + 1) * bm : L;
        const int64_t j0 = b * bn, j1 = (b + 1) * bn < L ? (b + 1) * bn : L;
        tile_out[x] = (uint8_t)tile_class(i0, i1, j0, j1, w_local, bif);
    }
}

hipError_t launch_debug_index(int64_t L, int32_t w_pretrained, int32_t w_local, int32_t bifocal,
                              int32_t bm, int32_t bn, int32_t* G_out, int32_t* f_out,
                              uint8_t* band_out, uint8_t* tile_out, hipStream_t s) {
    LaunchScope scope("debug_index", s);
    hipLaunchKernelGGL(debug_index_kernel, dim3(256), dim3(256), 0, s, L, w_pretrained, w_local,
                       bifocal, bm, bn, G_out, f_out, band_out, tile_out);
    return hipGetLastError();
}

}  // namespace jl
