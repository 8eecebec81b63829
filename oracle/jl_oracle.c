/*
 * jl_oracle.c -- plain, slow, fp64 CPU oracle for Dynamic Bifocal RoPE attention.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the library calls this file; only the
 * tests, the smoke check and the CPU-baseline leg of the benchmark load it.
 * It shares no code, header, table or constant with the HIP path.
 *
 * Pages this file follows (cited by title and section):
 *   [BT] "Jet-Long: 具有动态双焦RoPE的高效长上下文扩展" (bittide.aicompass.dev,
 *        a rendering of the paper's method sections): §3.1 (group size G and
 *        the remap f), §3.2 (inclusion-exclusion merge), §3.3 (KV-cache
 *        correction rotation).
 *   [TW] "NVIDIA研究团队找到了让AI“看清”超长文本的新方法" (techwalker.com):
 *        §二 (local window of 2048 tokens keeps standard RoPE; remote window
 *        remapped), §三 (cache keeps raw-RoPE keys; correction by the
 *        difference of positions), §四 (three calls B, A, C merged with
 *        LogSumExp weights).
 *
 * Readings taken where the pages are silent (each is also listed in the design
 * notes of the repository):
 *   - RoPE is the half-split form: pair (t, t + d/2), theta_t = base^(-2t/d),
 *     rotation by +angle for both q and k.  The pages give no formula.
 *   - A key j is "local" to query i iff 0 <= i - j < w_local (a window of
 *     exactly w_local keys that includes the diagonal); every older key is
 *     "remote".  [BT] §3.3 writes the remote test as q - k > w0, which differs
 *     at the single distance i - j = w_local; we take that distance as remote.
 *   - One G per sequence, from that sequence's full length L ([BT] §3.1:
 *     "current sequence length").  Positions are 0-based within a sequence.
 *   - Scores are softmax_scale * <q_rot, k_rot>; LSE is the natural log of the
 *     sum of exp(score) (the FlashAttention convention the pages' merge uses).
 *   - GQA: query head h reads kv head h / (Hq / Hkv).
 *
 * Every computation is fp64; inputs (f32, bf16 or f64 bits) are widened
 * exactly before use.  Softmax is two-pass: max, then sum of exp.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define JLO_F32 0
#define JLO_BF16 1
#define JLO_F64 2

/* Exact widening of one stored element to double. */
static double load_elem(const void* p, int dtype, int64_t idx) {
    if (dtype == JLO_F32) return (double)((const float*)p)[idx];
    if (dtype == JLO_BF16) {
        uint32_t bits = (uint32_t)((const uint16_t*)p)[idx] << 16;
        float f;
        memcpy(&f, &bits, sizeof f);
        return (double)f;
    }
    return ((const double*)p)[idx];
}

/* [BT] §3.1: G = max(1, ceil(L / w_pretrained)); integer arithmetic, L >= 0. */
int64_t jlo_group_size(int64_t L, int64_t w_pretrained) {
    int64_t g = (L + w_pretrained - 1) / w_pretrained;
    return g < 1 ? 1 : g;
}

/* [BT] §3.1: f(x) = floor(x / G), for positions x >= 0. */
int64_t jlo_remap(int64_t x, int64_t G) { return x / G; }

/* Band of the pair (query i, key j): 0 = masked (j > i, causal),
 * 1 = local (standard RoPE), 2 = remote (remapped RoPE).
 * [TW] §二 (local window of w_local tokens), [BT] §3.3; boundary reading in
 * the header.  With bifocal == 0 every unmasked pair is local. */
int jlo_band(int64_t i, int64_t j, int64_t w_local, int bifocal) {
    if (j > i) return 0;
    if (!bifocal) return 1;
    return (i - j < w_local) ? 1 : 2;
}

/* theta_t = base^(-2t/d)  (half-split RoPE; reading in the header). */
static double theta(int t, int d, double base) { return pow(base, -2.0 * (double)t / (double)d); }

/* y = R(p) x for one head vector of length d: pair (t, t+d/2) turned by p*theta_t. */
static void rotate(double* y, const double* x, double p, int d, double base) {
    int h = d / 2;
    for (int t = 0; t < h; ++t) {
        double a = p * theta(t, d, base);
        double c = cos(a), s = sin(a);
        double x0 = x[t], x1 = x[t + h];
        y[t] = x0 * c - x1 * s;
        y[t + h] = x1 * c + x0 * s;
    }
}

static void widen(double* y, const void* x, int dtype, int64_t off, int d) {
    for (int e = 0; e < d; ++e) y[e] = load_elem(x, dtype, off + e);
}

static double dot(const double* a, const double* b, int d) {
    double s = 0.0;
    for (int e = 0; e < d; ++e) s += a[e] * b[e];
    return s;
}

/* out[t][h][:] = R(pos[t]) x[t][h][:]   (x is [T][H][d]). */
void jlo_rope(double* out, const void* x, int dtype, const int64_t* pos, int64_t T, int H, int d,
              double base) {
    double* tmp = (double*)malloc(sizeof(double) * (size_t)d);
    for (int64_t t = 0; t < T; ++t)
        for (int h = 0; h < H; ++h) {
            int64_t off = (t * H + h) * (int64_t)d;
            widen(tmp, x, dtype, off, d);
            rotate(out + off, tmp, (double)pos[t], d, base);
        }
    free(tmp);
}

/* Softmax over n scores s[] (two passes) giving o = sum p_j v_j / sum p_j and
 * lse = ln sum exp(s_j).  v rows are fetched by index through vrow(). */
typedef struct {
    const void* v;
    int dtype;
    int64_t row0;   /* token index of key 0 in the value tensor            */
    int64_t stride; /* elements between consecutive tokens                 */
    int64_t col0;   /* element offset of the head inside a token row       */
    const int64_t* idx; /* key j of score n is idx[n] (NULL: j = n)        */
} vsrc;

static void softmax_pv(double* o, double* lse, const double* s, int64_t n, const vsrc* vs, int d) {
    if (n == 0) {
        for (int e = 0; e < d; ++e) o[e] = 0.0;
        *lse = -INFINITY;
        return;
    }
    double m = -INFINITY;
    for (int64_t a = 0; a < n; ++a) m = s[a] > m ? s[a] : m;
    double l = 0.0;
    for (int e = 0; e < d; ++e) o[e] = 0.0;
    for (int64_t a = 0; a < n; ++a) {
        double p = exp(s[a] - m);
        l += p;
        int64_t j = vs->idx ? vs->idx[a] : a;
        int64_t off = (vs->row0 + j) * vs->stride + vs->col0;
        for (int e = 0; e < d; ++e) o[e] += p * load_elem(vs->v, vs->dtype, off + e);
    }
    for (int e = 0; e < d; ++e) o[e] /= l;
    *lse = m + log(l);
}

static int find_seq(const int64_t* cu, int n_seqs, int64_t r) {
    for (int s = 0; s < n_seqs; ++s)
        if (r >= cu[s] && r < cu[s + 1]) return s;
    return -1;
}

/*
 * Remote position of x in a sequence of length L.
 *   bifocal == 1 (the method): f(x) = floor(x / G), G = G(L)  ([BT] §3.1).
 *   bifocal == 2: the continuous-interpolation alternative the pages compare
 *   the integer grouping against ([BT] §4.4, [TW] §八), read as x / s with the
 *   real scale s = max(1, L / w_pretrained), so remote angles may fall between
 *   the integer positions of pretraining.
 */
static double remote_pos(int64_t x, int64_t L, int64_t w, int mode) {
    if (mode == 2) return L > w ? (double)(x * w) / (double)L : (double)x;
    return (double)jlo_remap(x, jlo_group_size(L, w));
}

/* Per-sequence rotated keys: kS[g][n] = R(n) k_n, kR[g][n] = R(remote_pos(n)) k_n. */
static void rotate_keys(double* kS, double* kR, const void* k, int dtype, int64_t start, int64_t L,
                        int Hkv, int d, int64_t w, int mode, double base) {
#pragma omp parallel
    {
        double* tmp = (double*)malloc(sizeof(double) * (size_t)d);
#pragma omp for schedule(static)
        for (int64_t n = 0; n < L; ++n)
            for (int g = 0; g < Hkv; ++g) {
                widen(tmp, k, dtype, ((start + n) * Hkv + g) * (int64_t)d, d);
                int64_t dst = ((int64_t)g * L + n) * d;
                rotate(kS + dst, tmp, (double)n, d, base);
                rotate(kR + dst, tmp, remote_pos(n, L, w, mode), d, base);
            }
        free(tmp);
    }
}

/*
 * Prefill by the plain definition ([BT] §3.2: "equivalent to local keys
 * standard, remote keys remapped"):
 *   for query i (position within its sequence) and every key j <= i:
 *     s_ij = scale * <R(i) q_i, R(j) k_j>        if local,
 *     s_ij = scale * <R(f(i)) q_i, R(f(j)) k_j>  if remote,
 *   then an fp64 softmax over j.
 * q [T][Hq][d], k, v [T][Hkv][d]; cu [n_seqs + 1] token offsets.
 * Only the rows listed in rows[0..n_rows) are computed (rows == NULL: all T);
 * outputs are compact: o_sel[n_rows][Hq][d], lse_sel[n_rows][Hq].
 * Returns 0, or -1 on inconsistent arguments.
 */
int jlo_prefill(double* o_sel, double* lse_sel, const void* q, const void* k, const void* v,
                int dtype, const int64_t* cu, int n_seqs, int64_t T, int Hq, int Hkv, int d,
                int64_t w_pretrained, int64_t w_local, double base, double scale, int bifocal,
                const int64_t* rows, int64_t n_rows, int n_threads) {
    if (Hkv <= 0 || Hq % Hkv != 0 || d <= 0 || d % 2 || w_pretrained < 1 || w_local < 0 ||
        bifocal < 0 || bifocal > 2)
        return -1;
    if (cu[0] != 0 || cu[n_seqs] != T) return -1;
#ifdef _OPENMP
    if (n_threads > 0) omp_set_num_threads(n_threads);
#else
    (void)n_threads;
#endif
    if (!rows) n_rows = T;
    const int grp = Hq / Hkv;
    for (int s = 0; s < n_seqs; ++s) {
        const int64_t start = cu[s], L = cu[s + 1] - cu[s];
        int64_t cnt = 0;
        for (int64_t a = 0; a < n_rows; ++a) {
            int64_t r = rows ? rows[a] : a;
            cnt += (r >= start && r < start + L);
        }
        if (cnt == 0) continue;
        double* kS = (double*)malloc(sizeof(double) * (size_t)(Hkv * L * d));
        double* kR = (double*)malloc(sizeof(double) * (size_t)(Hkv * L * d));
        rotate_keys(kS, kR, k, dtype, start, L, Hkv, d, w_pretrained, bifocal, base);
#pragma omp parallel
        {
            double* qr = (double*)malloc(sizeof(double) * (size_t)d);
            double* qS = (double*)malloc(sizeof(double) * (size_t)d);
            double* qR = (double*)malloc(sizeof(double) * (size_t)d);
            double* sc = (double*)malloc(sizeof(double) * (size_t)L);
#pragma omp for collapse(2) schedule(dynamic, 1)
            for (int64_t a = 0; a < n_rows; ++a)
                for (int h = 0; h < Hq; ++h) {
                    int64_t r = rows ? rows[a] : a;
                    if (r < start || r >= start + L) continue;
                    const int64_t i = r - start;
                    const int g = h / grp;
                    widen(qr, q, dtype, (r * Hq + h) * (int64_t)d, d);
                    rotate(qS, qr, (double)i, d, base);
                    rotate(qR, qr, remote_pos(i, L, w_pretrained, bifocal), d, base);
                    for (int64_t j = 0; j <= i; ++j) {
                        const double* kj;
                        const double* qi;
                        if (jlo_band(i, j, w_local, bifocal) == 1) {
                            kj = kS + ((int64_t)g * L + j) * d;
                            qi = qS;
                        } else {
                            kj = kR + ((int64_t)g * L + j) * d;
                            qi = qR;
                        }
                        sc[j] = scale * dot(qi, kj, d);
                    }
                    vsrc vs = {v, dtype, start, (int64_t)Hkv * d, (int64_t)g * d, NULL};
                    softmax_pv(o_sel + (a * Hq + h) * (int64_t)d, lse_sel + a * Hq + h, sc, i + 1,
                               &vs, d);
                }
            free(qr);
            free(qS);
            free(qR);
            free(sc);
        }
        free(kS);
        free(kR);
    }
    return 0;
}

/*
 * The pages' three-call form of prefill ([TW] §四, [BT] §3.2), used only to
 * check the direct form above:
 *   B: every key j <= i, remapped RoPE;
 *   A: local keys only, standard RoPE;
 *   C: local keys only, remapped RoPE;
 * each gives (O_x, LSE_x) from its own softmax.  The merge works on the
 * unnormalised sums Z_x = exp(LSE_x), N_x = Z_x O_x:
 *   Z = Z_B - Z_C + Z_A,  O = (N_B - N_C + N_A) / Z,  LSE = ln Z,
 * evaluated relative to M = max(LSE_A, LSE_B); the remote mass Z_B - Z_C is
 * clamped at >= 0 (it is exactly 0 when a row has no remote key).
 * Same argument conventions as jlo_prefill; bifocal is implied.
 */
int jlo_prefill_three_call(double* o_sel, double* lse_sel, const void* q, const void* k,
                           const void* v, int dtype, const int64_t* cu, int n_seqs, int64_t T,
                           int Hq, int Hkv, int d, int64_t w_pretrained, int64_t w_local,
                           double base, double scale, const int64_t* rows, int64_t n_rows) {
    if (Hkv <= 0 || Hq % Hkv != 0 || d <= 0 || d % 2 || w_pretrained < 1 || w_local < 0) return -1;
    if (cu[0] != 0 || cu[n_seqs] != T) return -1;
    if (!rows) n_rows = T;
    const int grp = Hq / Hkv;
    for (int64_t a = 0; a < n_rows; ++a) {
        const int64_t r = rows ? rows[a] : a;
        const int s = find_seq(cu, n_seqs, r);
        if (s < 0) return -1;
        const int64_t start = cu[s], L = cu[s + 1] - cu[s], i = r - start;
        const int64_t G = jlo_group_size(L, w_pretrained);
        double* sc = (double*)malloc(sizeof(double) * (size_t)(i + 1));
        int64_t* idx = (int64_t*)malloc(sizeof(int64_t) * (size_t)(i + 1));
        double* qr = (double*)malloc(sizeof(double) * (size_t)d);
        double* qS = (double*)malloc(sizeof(double) * (size_t)d);
        double* qR = (double*)malloc(sizeof(double) * (size_t)d);
        double* kr = (double*)malloc(sizeof(double) * (size_t)d);
        double* kx = (double*)malloc(sizeof(double) * (size_t)d);
        double* oB = (double*)malloc(sizeof(double) * (size_t)d);
        double* oA = (double*)malloc(sizeof(double) * (size_t)d);
        double* oC = (double*)malloc(sizeof(double) * (size_t)d);
        for (int h = 0; h < Hq; ++h) {
            const int g = h / grp;
            widen(qr, q, dtype, (r * Hq + h) * (int64_t)d, d);
            rotate(qS, qr, (double)i, d, base);
            rotate(qR, qr, (double)jlo_remap(i, G), d, base);
            vsrc vs = {v, dtype, start, (int64_t)Hkv * d, (int64_t)g * d, idx};
            double lB, lA, lC;
            /* call B: full causal, remapped */
            for (int64_t j = 0; j <= i; ++j) {
                widen(kr, k, dtype, ((start + j) * Hkv + g) * (int64_t)d, d);
                rotate(kx, kr, (double)jlo_remap(j, G), d, base);
                sc[j] = scale * dot(qR, kx, d);
                idx[j] = j;
            }
            softmax_pv(oB, &lB, sc, i + 1, &vs, d);
            /* calls A and C: the local window only (i - w_local < j <= i) */
            int64_t n = 0;
            for (int64_t j = 0; j <= i; ++j)
                if (i - j < w_local) idx[n++] = j;
            for (int64_t a2 = 0; a2 < n; ++a2) {
                widen(kr, k, dtype, ((start + idx[a2]) * Hkv + g) * (int64_t)d, d);
                rotate(kx, kr, (double)idx[a2], d, base);
                sc[a2] = scale * dot(qS, kx, d);
            }
            softmax_pv(oA, &lA, sc, n, &vs, d);
            for (int64_t a2 = 0; a2 < n; ++a2) {
                widen(kr, k, dtype, ((start + idx[a2]) * Hkv + g) * (int64_t)d, d);
                rotate(kx, kr, (double)jlo_remap(idx[a2], G), d, base);
                sc[a2] = scale * dot(qR, kx, d);
            }
            softmax_pv(oC, &lC, sc, n, &vs, d);
            /* LSE-space merge */
            double M = lA > lB ? lA : lB;
            double zB = exp(lB - M), zC = (n > 0) ? exp(lC - M) : 0.0, zA = (n > 0) ? exp(lA - M) : 0.0;
            double rem = zB - zC;
            if (rem < 0.0) rem = 0.0;
            double Z = rem + zA;
            double* o = o_sel + (a * Hq + h) * (int64_t)d;
            for (int e = 0; e < d; ++e) o[e] = (zB * oB[e] - zC * oC[e] + zA * oA[e]) / Z;
            lse_sel[a * Hq + h] = M + log(Z);
        }
        free(sc);
        free(idx);
        free(qr);
        free(qS);
        free(qR);
        free(kr);
        free(kx);
        free(oB);
        free(oA);
        free(oC);
    }
    return 0;
}

/*
 * Decode as the pages describe it ([TW] §三, [BT] §3.3): one query at position
 * p = L - 1 against a cache whose key rows hold R(j) k_j (standard RoPE at the
 * original index, never rewritten).  G = G(L).  Local keys (p - j < w_local)
 * score against R(p) q; every remote key is turned by the correction
 * R(f(j) - j) and scored against R(f(p)) q.  By R(a) R(b) = R(a + b) this is
 * the prefill definition applied to the raw key R(-j) cache_j.
 * q [B][Hq][d] raw; kc, vc [B][S_max][Hkv][d]; seqlens[B] = L_b (>= 1);
 * o [B][Hq][d], lse [B][Hq].
 */
int jlo_decode(double* o, double* lse, const void* q, const void* kc, const void* vc, int dtype,
               const int64_t* seqlens, int B, int64_t S_max, int Hq, int Hkv, int d,
               int64_t w_pretrained, int64_t w_local, double base, double scale, int bifocal,
               int n_threads) {
    if (Hkv <= 0 || Hq % Hkv != 0 || d <= 0 || d % 2 || w_pretrained < 1 || w_local < 0 ||
        bifocal < 0 || bifocal > 2)
        return -1;
    for (int b = 0; b < B; ++b)
        if (seqlens[b] < 1 || seqlens[b] > S_max) return -1;
#ifdef _OPENMP
    if (n_threads > 0) omp_set_num_threads(n_threads);
#else
    (void)n_threads;
#endif
    const int grp = Hq / Hkv;
#pragma omp parallel for collapse(2) schedule(dynamic, 1)
    for (int b = 0; b < B; ++b)
        for (int h = 0; h < Hq; ++h) {
            const int64_t L = seqlens[b], p = L - 1;
                const int g = h / grp;
            double* qr = (double*)malloc(sizeof(double) * (size_t)d);
            double* qS = (double*)malloc(sizeof(double) * (size_t)d);
            double* qR = (double*)malloc(sizeof(double) * (size_t)d);
            double* kj = (double*)malloc(sizeof(double) * (size_t)d);
            double* kc2 = (double*)malloc(sizeof(double) * (size_t)d);
            double* sc = (double*)malloc(sizeof(double) * (size_t)L);
            widen(qr, q, dtype, ((int64_t)b * Hq + h) * d, d);
            rotate(qS, qr, (double)p, d, base);
            rotate(qR, qr, remote_pos(p, L, w_pretrained, bifocal), d, base);
            for (int64_t j = 0; j < L; ++j) {
                widen(kj, kc, dtype, (((int64_t)b * S_max + j) * Hkv + g) * d, d);
                if (jlo_band(p, j, w_local, bifocal) == 1) {
                    sc[j] = scale * dot(qS, kj, d);
                } else {
                    rotate(kc2, kj, remote_pos(j, L, w_pretrained, bifocal) - (double)j, d, base);
                    sc[j] = scale * dot(qR, kc2, d);
                }
            }
            vsrc vs = {vc, dtype, (int64_t)b * S_max, (int64_t)Hkv * d, (int64_t)g * d, NULL};
            softmax_pv(o + ((int64_t)b * Hq + h) * d, lse + (int64_t)b * Hq + h, sc, L, &vs, d);
            free(qr);
            free(qS);
            free(qR);
            free(kj);
            free(kc2);
            free(sc);
        }
    return 0;
}

/*
 * Chunked prefill against a cache ([TW] §三 and [BT] §3.3 for the cache and
 * its correction rotation, [BT] §3.1 for G).  Sequence b holds L_b =
 * seqlens[b] keys in kc/vc; kc rows hold R(j) k_j (standard RoPE at the
 * original index).  Its newest C_b = cu_q[b + 1] - cu_q[b] positions,
 * L_b - C_b .. L_b - 1, are the queries q[cu_q[b] .. cu_q[b + 1]) (raw).  G is
 * G(L_b), the length the call sees.  A query at position p scores every key
 * j <= p: local keys against R(p) q, remote keys turned by R(f(j) - j) against
 * R(f(p)) q.  Decode is the case C_b = 1.  The turned keys of a sequence do
 * not depend on the query, so they are formed once per sequence.
 * q [Tq][Hq][d]; kc, vc [B][S_max][Hkv][d]; rows as in jlo_prefill (indices
 * into q); returns -1 on inconsistent arguments.
 */
int jlo_prefill_chunk(double* o_sel, double* lse_sel, const void* q, const void* kc,
                      const void* vc, int dtype, const int64_t* cu_q, const int64_t* seqlens,
                      int B, int64_t Tq, int64_t S_max, int Hq, int Hkv, int d,
                      int64_t w_pretrained, int64_t w_local, double base, double scale,
                      int bifocal, const int64_t* rows, int64_t n_rows, int n_threads) {
    if (Hkv <= 0 || Hq % Hkv != 0 || d <= 0 || d % 2 || w_pretrained < 1 || w_local < 0 ||
        bifocal < 0 || bifocal > 2)
        return -1;
    if (cu_q[0] != 0 || cu_q[B] != Tq) return -1;
    for (int b = 0; b < B; ++b) {
        const int64_t C = cu_q[b + 1] - cu_q[b];
        if (C < 0 || C > seqlens[b] || seqlens[b] > S_max) return -1;
    }
#ifdef _OPENMP
    if (n_threads > 0) omp_set_num_threads(n_threads);
#else
    (void)n_threads;
#endif
    if (!rows) n_rows = Tq;
    const int grp = Hq / Hkv;
    for (int b = 0; b < B; ++b) {
        const int64_t L = seqlens[b], C = cu_q[b + 1] - cu_q[b], qstart = cu_q[b];
        int64_t cnt = 0;
        for (int64_t a = 0; a < n_rows; ++a) {
            const int64_t r = rows ? rows[a] : a;
            cnt += (r >= qstart && r < qstart + C);
        }
        if (cnt == 0) continue;
        /* kS[g][j] = cache row j as stored, kR[g][j] = R(f(j) - j) cache row j */
        double* kS = (double*)malloc(sizeof(double) * (size_t)(Hkv * L * d));
        double* kR = (double*)malloc(sizeof(double) * (size_t)(Hkv * L * d));
#pragma omp parallel for schedule(static)
        for (int64_t j = 0; j < L; ++j)
            for (int g = 0; g < Hkv; ++g) {
                double* ks = kS + ((int64_t)g * L + j) * d;
                widen(ks, kc, dtype, (((int64_t)b * S_max + j) * Hkv + g) * d, d);
                rotate(kR + ((int64_t)g * L + j) * d, ks,
                       remote_pos(j, L, w_pretrained, bifocal) - (double)j, d, base);
            }
#pragma omp parallel
        {
            double* qr = (double*)malloc(sizeof(double) * (size_t)d);
            double* qS = (double*)malloc(sizeof(double) * (size_t)d);
            double* qR = (double*)malloc(sizeof(double) * (size_t)d);
            double* sc = (double*)malloc(sizeof(double) * (size_t)L);
#pragma omp for collapse(2) schedule(dynamic, 1)
            for (int64_t a = 0; a < n_rows; ++a)
                for (int h = 0; h < Hq; ++h) {
                    const int64_t r = rows ? rows[a] : a;
                    if (r < qstart || r >= qstart + C) continue;
                    const int64_t p = L - C + (r - qstart);
                    const int g = h / grp;
                    widen(qr, q, dtype, (r * Hq + h) * (int64_t)d, d);
                    rotate(qS, qr, (double)p, d, base);
                    rotate(qR, qr, remote_pos(p, L, w_pretrained, bifocal), d, base);
                    for (int64_t j = 0; j <= p; ++j) {
                        const int local = jlo_band(p, j, w_local, bifocal) == 1;
                        const double* kj = (local ? kS : kR) + ((int64_t)g * L + j) * d;
                        sc[j] = scale * dot(local ? qS : qR, kj, d);
                    }
                    vsrc vs = {vc, dtype, (int64_t)b * S_max, (int64_t)Hkv * d, (int64_t)g * d,
                               NULL};
                    softmax_pv(o_sel + (a * Hq + h) * (int64_t)d, lse_sel + a * Hq + h, sc, p + 1,
                               &vs, d);
                }
            free(qr);
            free(qS);
            free(qR);
            free(sc);
        }
        free(kS);
        free(kR);
    }
    return 0;
}

/*
 * fp8 KV cache (a cache format beside the pages' method: the correction
 * rotation is applied to the dequantized keys, so the method is unchanged).
 * Format: OCP 8-bit floating point (OFP8), E4M3: 1 sign bit, 4 exponent bits
 * with bias 7, 3 mantissa bits; exponent 0 holds subnormals m * 2^-9; there
 * are no infinities; S.1111.111 is NaN, so the largest finite value is
 * S.1111.110 = 448.
 */
double jlo_e4m3_value(uint8_t c) {
    const int s = c >> 7, e = (c >> 3) & 15, m = c & 7;
    if (e == 15 && m == 7) return NAN;
    const double mag = e == 0 ? ldexp((double)m, -9) : ldexp(1.0 + m / 8.0, e - 7);
    return s ? -mag : mag;
}

/* Nearest E4M3 code to x: ties go to the even code (the one whose mantissa
 * ends in 0), magnitudes beyond 448 saturate to +-448, NaN gives S.1111.111.
 * Found by comparing |x| with every finite non-negative code. */
uint8_t jlo_e4m3_encode(double x) {
    const uint8_t sign = signbit(x) ? 0x80 : 0x00;
    if (isnan(x)) return sign | 0x7F;
    const double a = fabs(x);
    if (a >= 448.0) return sign | 0x7E;
    int best = 0;
    double bd = a;  /* distance to code 0 */
    for (int c = 1; c <= 0x7E; ++c) {
        const double dd = fabs(jlo_e4m3_value((uint8_t)c) - a);
        if (dd < bd || (dd == bd && (c & 1) == 0)) {
            best = c;
            bd = dd;
        }
    }
    return sign | (uint8_t)best;
}

/* out[i] = scale[(i / d) % H] * value(code[i]) for a [N][H][d] cache (exact in fp64). */
void jlo_e4m3_dequant(double* out, const uint8_t* code, const float* scale, int64_t N, int H,
                      int d) {
    for (int64_t i = 0; i < N * H * d; ++i)
        out[i] = (double)scale[(i / d) % H] * jlo_e4m3_value(code[i]);
}

/* Quantization of a [N][H][d] cache with one scale per head:
 * code = E4M3(x / scale[h]).  The quotient is formed in fp32 (a correctly
 * rounded float division), the precision the device kernel divides in, so
 * that both sides round the same number to a code. */
void jlo_e4m3_quant(uint8_t* code, const void* x, int dtype, const float* scale, int64_t N, int H,
                    int d) {
    for (int64_t i = 0; i < N * H * d; ++i) {
        const float xi = (float)load_elem(x, dtype, i);
        const float qi = xi / scale[(i / d) % H];
        code[i] = jlo_e4m3_encode((double)qi);
    }
}
