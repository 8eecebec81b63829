// prefill_bf16.hip -- bifocal causal prefill on gfx950 16-bit MFMA.
//
// Pages cited (title, section):
//   [BT] "Jet-Long: 具有动态双焦RoPE的高效长上下文扩展" (bittide.aicompass.dev)
//   [TW] "NVIDIA研究团队找到了让AI“看清”超长文本的新方法" (techwalker.com)
//
// The pages fuse three attention calls -- B: full causal with remapped RoPE,
// A: local window with standard RoPE, C: local window with remapped RoPE --
// into Attn = B + A - C merged in LogSumExp space ([TW] §四, [BT] §3.2).  That
// sum equals one softmax in which local keys are scored under standard RoPE
// and remote keys under remapped RoPE; this kernel evaluates that softmax
// directly, with no L x L mask ([TW] §四).  An online softmax does not depend
// on the order in which keys arrive, so each wave takes its keys in two
// phases: first every remote pair (remapped query R(f(i))q against the
// remapped key tiles), then every local pair (standard query R(i)q against the
// standard key tiles).  Only one query variant and one key tile per buffer
// are live at a time; a block that holds both kinds of pairs, or the causal
// diagonal, is masked per element in each phase.
//
// Work decomposition (one workgroup = 8 waves = 256 query rows of one head):
//   S^T = K Q^T on v_mfma_f32_32x32x16_f16 with K (32 keys x 16 d) from LDS
//   as the A operand and the wave's rotated queries held in registers as B;
//   lane (query r, half h) then holds 16 scores of query r per block, so the
//   row max needs one exchange with lane r + 32 (v_permlane32_swap), and the
//   probabilities feed O^T += V^T P^T directly as its B operand (V^T tiles are
//   laid out by the pre-pass so each lane reads its 8 keys as one 16-byte
//   vector).  Tiles of 64 keys are double-buffered in LDS and filled by
//   global->LDS DMA while the previous tile is processed.
// Queries are rotated at entry (fp64-reduced angles, hardware sin/cos) and
// scaled by softmax_scale * log2(e) so the softmax runs on exp2.  Score
// accumulators start at -m_c (m_c: the running max, or 0 before a row has
// one), so the exponentials need no subtraction unless the max is raised.
//
// Operand precision: rounding a key is a random error per key and averages
// out over the softmax, but rounding a query is a fixed error per row whose
// softmax-weighted mean over the keys does not shrink (the weighted mean key
// points along the query), so it sets the LSE error directly.  QK^T therefore
// uses fp16 operands (11-bit significand, same MFMA rate as bf16 on gfx950):
// rotated q and k must stay below 65504 in magnitude.  PV runs on fp16 too:
// V (bf16 input, exact in fp16 within its range) and the probabilities, whose
// row sum is taken from the same fp16 values with v_dot2_f32_f16.  Rows below
// kPreciseRows, which see few keys, add the fp16 residuals of q and k
// (hi * hi + hi * lo + lo * hi); a call that asks for split precision gets
// that on every row (for concentrated attention, where one key's score
// rounding enters the LSE undiluted).
#include "internal.h"

namespace jl {

namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

template <int D, bool PRECISE>
struct Cfg {
    // tiles in LDS: K [D/8 pieces][kBN keys][8], V^T [kBN/8 pieces][D rows][8]
    static constexpr int KSLOT = ktile_elems(D);  // elements
    static constexpr int VSLOT = vtile_elems(D);
    static constexpr int NK = PRECISE ? 2 : 1; // K of the current phase (+ its lo part)
    static constexpr int BUF = NK * KSLOT + VSLOT;
    static constexpr int NS = D / 16;          // k-steps of a QK^T product
    static constexpr int ND = D / 32;          // 32-row blocks of O^T
    static constexpr int QROWS = 128;          // query rows staged per prologue round
    static_assert(QROWS * D <= BUF, "query staging must fit in one tile buffer");
    static_assert(KSLOT % 512 == 0 && VSLOT % 512 == 0, "tiles are whole 1 KB DMA rounds");
};


__device__ __forceinline__ f32x16 mfma32h(f16x8 a, f16x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}

// max(x, x of lane l ^ 32) through v_permlane32_swap (no LDS round trip)
__device__ __forceinline__ float max_other_half(float x) {
    const unsigned u = __float_as_uint(x);
    const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

}  // namespace

// 8 waves per workgroup, one workgroup per CU: two waves per SIMD, so each
// wave may use the full 256-register budget.
template <int D, bool PRECISE>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2)))
void prefill_bf16_kernel(PrefillArgs a, int rb_first, int n_rb) {
    using C = Cfg<D, PRECISE>;
    // Two distinct LDS objects: a DMA into one buffer and reads of the other
    // then provably do not alias.
    __shared__ __align__(16) bf16 lds0[C::BUF];
    __shared__ __align__(16) bf16 lds1[C::BUF];

    // the wave index is uniform per wave; readfirstlane tells the compiler so,
    // which keeps every per-wave tile-class branch a scalar branch
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int qr = lane & 31, hh = lane >> 5;  // query column, lane half

    // ---- which (head, sequence, row block) ----
    int head = blockIdx.x;
    if ((a.Hq & 7) == 0) head = (blockIdx.x & 7) * (a.Hq >> 3) + (blockIdx.x >> 3);
    const int s = blockIdx.y;
    // key split (main rows of a chunk call): grid z = row block x split
    const int nsp = (!PRECISE && a.ksplit > 1) ? a.ksplit : 1;
    const int rb = rb_first + (n_rb - 1 - (int)blockIdx.z / nsp);  // longest rows first
    const int ks = (int)blockIdx.z % nsp;
    const int32_t* plan = (const int32_t*)((const char*)a.ws + a.lay.plan);
    const int32_t* e = plan + s * kPlanFields;
    const int32_t start = e[kPlanStart], len = e[kPlanLen], G = e[kPlanG];
    // Query rows are positions [q0, len): q0 = 0 for a whole sequence, or the
    // first new row of a chunk appended to a cache.  Row blocks are aligned
    // to multiples of 256 positions, so the split-precision rows (< 2048)
    // never share a block with the others; position `row` is token
    // qbase + row of q, o and lse.
    const int32_t q0 = e[kPlanQ0];
    const int64_t qbase = (int64_t)start - q0;
    const int32_t row0 = (q0 / kBM + rb) * kBM;
    if (row0 >= len) return;
    if (PRECISE != (a.precise || row0 < kPreciseRows)) return;
    const int32_t row_end = min(row0 + kBM, len);
    // Which pairs and which RoPE.  Mode 0 is the bifocal softmax (remote
    // pairs remapped, local pairs standard).  Modes 1-3 are the three
    // separate attention calls of the pages' unfused form ([TW] §四): 1 every
    // causal pair under remapped RoPE (B), 2 the local pairs under standard
    // RoPE (A), 3 the local pairs under remapped RoPE (C).
    const bool have_kr = a.bifocal && G > 1;  // the pre-pass wrote remapped key tiles
    const int mode = a.mode;
    const bool bif = mode == 0 ? have_kr : true;  // the remote/local band split is on
    const int32_t wl = mode == 1 ? 0 : a.w_local;
    const bool do_remote = mode == 0 ? bif : mode == 1;
    const bool do_local = mode != 1;
    const bool local_remapped = mode == 3;
    const int g = head / (a.Hq / a.Hkv);
    // remote queries of the continuous-interpolation variant (bifocal 2) sit at
    // row / s, s = len / w_pretrained
    const bool interp = a.bifocal == 2;
    const double rsc = interp ? (double)a.w_pretrained / (double)len : 1.0;
    const int32_t wr0 = row0 + wave * kWaveRows;
    const int32_t wr_end = min(wr0 + kWaveRows, len);
    const int32_t wlo = max(wr0, q0);  // the wave's first query row
    const bool wave_active = wlo < wr_end;
    const int32_t myrow = wr0 + qr;
    const bool row_valid = myrow >= q0 && myrow < len;

    // ---- the two phases as tile ranges of this workgroup ----
    // remote pairs need key j <= i - w_local; local pairs j > i - w_local.
    const int ntiles = (row_end + kBN - 1) / kBN;
    int r_end = 0, s_begin = 0;
    if (bif) {
        const int32_t jr = row_end - 1 - wl;
        r_end = jr >= 0 ? jr / kBN + 1 : 0;
        s_begin = wl == 0 ? ntiles : max(0, max(row0, q0) - wl + 1) / kBN;
    }
    // this workgroup's share of the phases' tiles (all of them without a key
    // split; with one, an equal slice of the remote tiles followed by the
    // local ones)
    int r_lo = 0, r_hi = do_remote ? r_end : 0, l_lo = s_begin, l_hi = do_local ? ntiles : s_begin;
    if (nsp > 1) {
        const int nrem = r_hi, nloc = max(l_hi - s_begin, 0), ntot = nrem + nloc;
        const int a0 = (int)((int64_t)ntot * ks / nsp), a1 = (int)((int64_t)ntot * (ks + 1) / nsp);
        r_lo = min(a0, nrem);
        r_hi = min(a1, nrem);
        l_lo = s_begin + max(a0 - nrem, 0);
        l_hi = s_begin + max(a1 - nrem, 0);
    }

    // ---- rotated, scaled queries as MFMA B operands ----
    // The workgroup rotates 128 rows at a time into LDS (thread (t, r) does
    // pair t of rows r, r + 512/(D/2), ...), in 16-byte pieces laid out like a
    // K tile ([D/8][QROWS][8]); each wave then reads its operand registers,
    // lane (qr, hh) holding d = 16*st + 8*hh + u, as 16-byte vectors.  Both
    // LDS buffers are idle whenever this runs.
    f16x8 Qc[C::NS], Qcl[C::NS];
    const float qscale = a.softmax_scale * kLog2e;
    auto stage_q = [&](bool remapped)  __attribute__((always_inline)) {
        constexpr int HALF = D / 2;
        f16* qimg = reinterpret_cast<f16*>(lds0);
        const int t = tid % HALF;
        const double rv = rope_rev(a.tab, t);
        const bf16* qg = (const bf16*)a.q + (int64_t)head * D;
        __syncthreads();
        for (int round = 0; round < (PRECISE ? 4 : 2); ++round) {
            const int half_rows = round & 1;
            const bool lo = round >= 2;
#pragma unroll 1
            for (int r = tid / HALF; r < C::QROWS; r += 512 / HALF) {
                const int32_t row = row0 + half_rows * C::QROWS + r;
                float x0 = 0.0f, x1 = 0.0f;
                if (row >= q0 && row < len) {
                    const bf16* qp = qg + (qbase + row) * a.Hq * D;
                    x0 = (float)qp[t];
                    x1 = (float)qp[t + HALF];
                }
                float c, sn;
                if (remapped && interp) rope_cs_hw(row, rv * rsc, c, sn);
                else rope_cs_hw(remapped ? remap(row, G) : row, rv, c, sn);
                const float y0 = (x0 * c - x1 * sn) * qscale, y1 = (x1 * c + x0 * sn) * qscale;
                qimg[((t >> 3) * C::QROWS + r) * 8 + (t & 7)] = lo ? (f16)(y0 - (float)(f16)y0) : (f16)y0;
                qimg[(((t + HALF) >> 3) * C::QROWS + r) * 8 + (t & 7)] =
                    lo ? (f16)(y1 - (float)(f16)y1) : (f16)y1;
            }
            __syncthreads();
            if ((wave * kWaveRows) / C::QROWS == half_rows) {
                const int qoff = (hh * C::QROWS + (wave * kWaveRows) % C::QROWS + qr) * 8;
#pragma unroll
                for (int st = 0; st < C::NS; ++st) {
                    const f16x8 v = *reinterpret_cast<const f16x8*>(qimg + qoff + 16 * C::QROWS * st);
                    if (!lo) Qc[st] = v;
                    if constexpr (PRECISE) {
                        if (lo) Qcl[st] = v;
                    }
                }
            }
            __syncthreads();
        }
    };

    // ---- global tile sources (tiles stored as LDS images) ----
    const int64_t ntp = a.lay.T_pad / kBN, ntl = a.lay.lo_pad / kBN;
    const bf16* KSg = (const bf16*)((const char*)a.ws + a.lay.ks) + ((int64_t)g * ntp + e[kPlanTile0]) * C::KSLOT;
    const bf16* KRg = (const bf16*)((const char*)a.ws + a.lay.kr) + ((int64_t)g * ntp + e[kPlanTile0]) * C::KSLOT;
    const bf16* VTg = (const bf16*)((const char*)a.ws + a.lay.vt) + ((int64_t)g * ntp + e[kPlanTile0]) * C::VSLOT;
    const bf16* KSlg = (const bf16*)((const char*)a.ws + a.lay.ks_lo) + ((int64_t)g * ntl + e[kPlanLoTile0]) * C::KSLOT;
    const bf16* KRlg = (const bf16*)((const char*)a.ws + a.lay.kr_lo) + ((int64_t)g * ntl + e[kPlanLoTile0]) * C::KSLOT;

    // global -> LDS DMA of one tile image: each wave instruction moves 64 x 16
    // contiguous bytes (tile sizes are whole 1 KB rounds).  Only waves 0-3
    // issue copies.  Wave w and wave w + 4 share a SIMD, and the issue arbiter
    // favours the older one, which finishes its blocks first and then idles
    // at the tile barrier; a copy instruction adds latency to the issuing
    // wave's own chain, so it goes where there is slack.
    auto dma = [&](const bf16* src, bf16* dst, int elems)  __attribute__((always_inline)) {
        if (wave < 4)
            for (int c0 = wave * 64; c0 < elems / 8; c0 += 256)
                __builtin_amdgcn_global_load_lds((const void*)(src + (int64_t)(c0 + lane) * 8),
                                                 (void*)(dst + c0 * 8), 16, 0, 0);
    };
    // key tiles of the phase's RoPE (remapped tiles equal the standard ones
    // when G = 1, and the pre-pass then writes only those)
    auto load_tile = [&](int tau, bool remapped, bf16* base)  __attribute__((always_inline)) {
        const bool kr = remapped && have_kr;
        dma((kr ? KRg : KSg) + (int64_t)tau * C::KSLOT, base, C::KSLOT);
        if constexpr (PRECISE)
            dma((kr ? KRlg : KSlg) + (int64_t)tau * C::KSLOT, base + C::KSLOT, C::KSLOT);
        dma(VTg + (int64_t)tau * C::VSLOT, base + C::NK * C::KSLOT, C::VSLOT);
    };

    // ---- running softmax state (log2 domain) and O^T accumulators ----
    // m starts at a finite floor so rows that have not met a key of the
    // current phase yet give exp2(-inf - m) = 0, never NaN.
    float m_run = -1e30f, l_run = 0.0f;
    float m_c = 0.0f;  // what the score accumulators start from (negated)
    float thr_c = m_run + 8.0f - m_c;  // raise threshold on s - m_c
    f32x16 negm = {};  // -m_c in every element: the C operand of a block's first MFMA
    f32x16 O[C::ND];
#pragma unroll
    for (int db = 0; db < C::ND; ++db) O[db] = f32x16{};
    const f16x2 ones = {(f16)1.0f, (f16)1.0f};

    // One 32-key block: scores, optional per-element mask, online softmax
    // (the running max is raised only when a score exceeds it by more than 8
    // in log2 units: sums stay exact relative to the max they use, p stays
    // below 2^8, and most blocks skip rescaling O), then O^T += V^T P^T.
    auto do_block = [&](const bf16* base, int b, bool masked, bool remote_phase, int32_t jb)  __attribute__((always_inline)) {
        // piece 2 st + hh of key row 32 b + qr
        const bf16* kp = base + kt_off(32 * b + qr, hh);
        f16x8 kv[C::NS];
#pragma unroll
        for (int st = 0; st < C::NS; ++st) kv[st] = *reinterpret_cast<const f16x8*>(kp + kt_off(0, 2 * st));
        // the K operands are in flight before the score chain starts
        __builtin_amdgcn_sched_barrier(0);
        f32x16 Sb = negm;
#pragma unroll
        for (int st = 0; st < C::NS; ++st) {
            Sb = mfma32h(kv[st], Qc[st], Sb);
            if constexpr (PRECISE) {
                Sb = mfma32h(kv[st], Qcl[st], Sb);
                const f16x8 kl = *reinterpret_cast<const f16x8*>(kp + C::KSLOT + kt_off(0, 2 * st));
                Sb = mfma32h(kl, Qc[st], Sb);
            }
        }
        // the V operands are read while the score chain and the softmax run
        // piece 4 b + hh + 2 u (keys 32 b + 8 hh + 16 u ..) of row qr + 32 db
        const bf16* vb = base + C::NK * C::KSLOT + vt_off(D, qr, 4 * b + hh);
        f16x8 vv[2][C::ND];
#pragma unroll
        for (int u = 0; u < 2; ++u)
#pragma unroll
            for (int db = 0; db < C::ND; ++db)
                vv[u][db] = *reinterpret_cast<const f16x8*>(vb + vt_off(D, 32 * db, 2 * u));
        __builtin_amdgcn_sched_barrier(0);
        if (masked) {
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int32_t key = jb + (i >> 2) * 8 + 4 * hh + (i & 3);
                const int32_t dist = myrow - key;
                const bool keep = dist >= 0 && (!bif || ((dist >= wl) == remote_phase));
                if (!keep) Sb[i] = -INFINITY;
            }
        }
        // Sb holds s - m_c; while m_c == m_run (always, once a row has a
        // finite max) p = exp2(Sb) directly
        float mx = -INFINITY;
#pragma unroll
        for (int i = 0; i < 16; ++i) mx = fmaxf(mx, Sb[i]);
        // A row's max is raised when its max score exceeds m_run + 8.  The
        // lane half that holds that score sees the test on its own 16 scores
        // (against the threshold kept relative to m_c), so the wave enters
        // the branch when some row must raise, up to the rounding of the two
        // forms of the test (a row that skips a raise by rounding keeps
        // probabilities a rounding step above 2^8, which fp16 holds); the row
        // max over both halves is formed only there.  A lane that enters
        // without raising keeps its state exactly (alpha = 1, d = 0).
        if (__any(mx > thr_c)) {
            mx = max_other_half(mx) + m_c;
            const bool raise = mx > m_run + 8.0f;
            const float m_new = raise ? mx : m_run;
            const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
            const float d = m_new - m_c;
#pragma unroll
            for (int i = 0; i < 16; ++i) Sb[i] -= d;
            m_run = m_new;
            m_c = m_new > -1e29f ? m_new : 0.0f;
            thr_c = m_run + 8.0f - m_c;
#pragma unroll
            for (int i = 0; i < 16; ++i) negm[i] = -m_c;
            l_run *= alpha;
#pragma unroll
            for (int db = 0; db < C::ND; ++db)
#pragma unroll
                for (int i = 0; i < 16; ++i) O[db][i] *= alpha;
        }
        f16x8 Pb[2];
#pragma unroll
        for (int i = 0; i < 16; ++i) Pb[i >> 3][i & 7] = (f16)__builtin_amdgcn_exp2f(Sb[i]);
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
            for (int i = 0; i < 8; i += 2) {
                const f16x2 pp = {Pb[h2][i], Pb[h2][i + 1]};
                l_run = __builtin_amdgcn_fdot2(pp, ones, l_run, false);
            }
#pragma unroll
        for (int u = 0; u < 2; ++u)
#pragma unroll
            for (int db = 0; db < C::ND; ++db) O[db] = mfma32h(vv[u][db], Pb[u], O[db]);
    };

    auto compute = [&](int tau, const bf16* base, bool remote_phase)  __attribute__((always_inline)) {
        const uint32_t want = (bif && remote_phase) ? kHasRemote : kHasLocal;
        // most tiles hold only pairs of the phase for every row of the wave
        // (no band edge, no diagonal): skip the per-block classification
        const int32_t jl = tau * kBN + kBN - 1;  // the tile's last key
        const bool pure = (bif && remote_phase)
                              ? jl <= wlo - wl
                              : (jl <= wlo && (!bif || (wr_end - 1) - tau * kBN < wl));
#pragma unroll
        for (int b = 0; b < 2; ++b) {
            const int32_t jb = tau * kBN + 32 * b;
            // uniform per wave: readfirstlane keeps it (and the branches on
            // it) in scalar registers
            const uint32_t cls = __builtin_amdgcn_readfirstlane(
                pure ? want : tile_class32(wlo, wr_end, jb, jb + 32, wl, bif));
            if (cls & want) do_block(base, b, cls != want, remote_phase, jb);
        }
    };

    // ---- one phase: tiles [t0, t1), unrolled by two so each step names its
    // LDS buffers statically ----
    auto step = [&](int tau, int t1, bool remote_phase, bool remapped, const bf16* cur, bf16* nxt)
        __attribute__((always_inline)) {
        const bool more = tau + 1 < t1;
        // the other buffer was last read in the previous step, which every
        // wave finished before the barrier that ended it
        if (more) load_tile(tau + 1, remapped, nxt);
        if (wave_active) compute(tau, cur, remote_phase);
        if (more) {
            __builtin_amdgcn_s_waitcnt(0);  // this wave's DMA writes have landed
            __syncthreads();
        }
    };
    // remote_phase selects the band (pairs with i - j >= wl, or < wl);
    // remapped selects the RoPE of the key tiles
    auto run_phase = [&](int t0, int t1, bool remote_phase, bool remapped) __attribute__((always_inline)) {
        load_tile(t0, remapped, lds0);
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
        for (int tau = t0; tau < t1; tau += 2) {
            step(tau, t1, remote_phase, remapped, lds0, lds1);
            if (tau + 1 < t1) step(tau + 1, t1, remote_phase, remapped, lds1, lds0);
        }
    };

    if (r_hi > r_lo) {
        stage_q(true);
        run_phase(r_lo, r_hi, true, true);
    }
    if (l_hi > l_lo) {
        stage_q(local_remapped);  // begins with a barrier: no wave still reads a buffer
        run_phase(l_lo, l_hi, false, local_remapped);
    }

    if (nsp > 1) {
        // partial of this key share: unnormalised O^T and (m, l), relative to m
        if (!wave_active || !row_valid) return;
        const float l_tot = l_run + __shfl_xor(l_run, 32);
        const int64_t tok = qbase + myrow;
        float* po = a.part_o + (((int64_t)ks * a.T + tok) * a.Hq + head) * D;
#pragma unroll
        for (int db = 0; db < C::ND; ++db)
#pragma unroll
            for (int g4 = 0; g4 < 4; ++g4) {
                const f32x4 w = {O[db][4 * g4], O[db][4 * g4 + 1], O[db][4 * g4 + 2], O[db][4 * g4 + 3]};
                *reinterpret_cast<f32x4*>(po + 32 * db + 8 * g4 + 4 * hh) = w;
            }
        if (hh == 0)
            a.part_ml[((int64_t)ks * a.Hq + head) * a.T + tok] =
                make_float2(l_tot > 0.0f ? m_run : -INFINITY, l_tot);
        return;
    }

    // ---- epilogue: O = O^T / l, LSE = ln(sum exp(score)) ----
    if (!wave_active || !row_valid) return;
    l_run += __shfl_xor(l_run, 32);
    // a row with no key of the call (the local calls with w_local = 0): o = 0, lse = -inf
    const bool none = !(l_run > 0.0f);
    const float inv = none ? 0.0f : 1.0f / l_run;
    const int64_t oofs = ((qbase + myrow) * a.Hq + head) * D;
    if (a.o_f32) {  // the unfused form's separate calls keep fp32 outputs
        float* op = (float*)a.o + oofs;
#pragma unroll
        for (int db = 0; db < C::ND; ++db)
#pragma unroll
            for (int g4 = 0; g4 < 4; ++g4) {
                const f32x4 w = {O[db][4 * g4] * inv, O[db][4 * g4 + 1] * inv,
                                 O[db][4 * g4 + 2] * inv, O[db][4 * g4 + 3] * inv};
                *reinterpret_cast<f32x4*>(op + 32 * db + 8 * g4 + 4 * hh) = w;
            }
    } else {
        bf16* op = (bf16*)a.o + oofs;
#pragma unroll
        for (int db = 0; db < C::ND; ++db)
#pragma unroll
            for (int g4 = 0; g4 < 4; ++g4) {
                bf16x4 w;
#pragma unroll
                for (int r = 0; r < 4; ++r) w[r] = (bf16)(O[db][4 * g4 + r] * inv);
                *reinterpret_cast<bf16x4*>(op + 32 * db + 8 * g4 + 4 * hh) = w;
            }
    }
    if (hh == 0) a.lse[(int64_t)head * a.T + qbase + myrow] = none ? -INFINITY : (m_run + log2f(l_run)) * kLn2;
}

template <int D, bool PRECISE>
static hipError_t launch_one(const PrefillArgs& a, int rb_first, int n_rb, hipStream_t s,
                             const char* name) {
    if (n_rb <= 0) return hipSuccess;
    LaunchScope scope(name, s);
    const int nsp = (!PRECISE && a.ksplit > 1) ? a.ksplit : 1;
    hipLaunchKernelGGL((prefill_bf16_kernel<D, PRECISE>), dim3(a.Hq, a.n_seqs, n_rb * nsp),
                       dim3(512), 0, s, a, rb_first, n_rb);
    return hipGetLastError();
}

hipError_t launch_prefill_bf16(const PrefillArgs& a, hipStream_t s) {
    const int precise_rb = kPreciseRows / kBM;
    int total_rb, main_first;
    if (a.chunked) {
        // row blocks counted from the block holding a chunk's first row: a
        // chunk of at most max_seqlen rows touches at most this many
        total_rb = (a.max_seqlen + kBM - 1) / kBM + 1;
        const int key_rb = (a.max_seqlen_k + kBM - 1) / kBM;
        total_rb = total_rb < key_rb ? total_rb : key_rb;
        main_first = 0;
    } else {
        total_rb = (a.max_seqlen + kBM - 1) / kBM;
        main_first = precise_rb;
    }
    // split precision on every row: the split-precision kernel takes all row blocks
    const int n_prec = a.precise ? total_rb : (total_rb < precise_rb ? total_rb : precise_rb);
    if (a.precise) main_first = total_rb;
    hipError_t err;
    if (a.d == 128) {
        err = launch_one<128, true>(a, 0, n_prec, s, "prefill_bf16_precise");
        if (err != hipSuccess) return err;
        return launch_one<128, false>(a, main_first, total_rb - main_first, s, "prefill_bf16");
    }
    err = launch_one<64, true>(a, 0, n_prec, s, "prefill_bf16_precise");
    if (err != hipSuccess) return err;
    return launch_one<64, false>(a, main_first, total_rb - main_first, s, "prefill_bf16");
}

// Key-split partials of a chunk call, combined in LogSumExp space
// ([TW] §四's merge of partial attentions): with m_k in log2 units,
//   Z = sum_k 2^(m_k - M) l_k,  o = sum_k 2^(m_k - M) O_k / Z,
//   lse = (M + log2 Z) ln 2,  M = max_k m_k.
// One wave per (token, head); lane l holds elements [D/64 * l, D/64 * (l + 1))
// of the row, read from each share as one vector.  A token is looked up in
// the plan (its sequence and position); rows of a block below the
// split-precision bound were written directly by that kernel and are
// skipped, as are tokens of no sequence (a broken plan has every length 0).
template <int D>
__global__ __launch_bounds__(256) void chunk_merge_kernel(PrefillArgs a) {
    constexpr int E = D / 64;
    using vecE = float __attribute__((ext_vector_type(E)));
    const int64_t tok = blockIdx.x;
    const int head = blockIdx.y * 4 + (int)(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    if (head >= a.Hq) return;
    const int32_t* plan = (const int32_t*)((const char*)a.ws + a.lay.plan);
    int lo = 0, hi = a.n_seqs - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) / 2;
        if (plan[mid * kPlanFields + kPlanStart] <= tok) lo = mid;
        else hi = mid - 1;
    }
    const int32_t* e = plan + lo * kPlanFields;
    const int32_t len = e[kPlanLen], q0 = e[kPlanQ0];
    if (len <= 0 || tok < e[kPlanStart] || tok >= (int64_t)e[kPlanStart] + (len - q0)) return;
    const int32_t pos = q0 + (int32_t)(tok - e[kPlanStart]);
    if (pos - pos % kBM < kPreciseRows) return;
    const int K = a.ksplit;
    // every share's row vector is in flight before the weights are known
    vecE ov[kChunkMaxSplit];
    float2 ml[kChunkMaxSplit];
#pragma unroll
    for (int k = 0; k < kChunkMaxSplit; ++k) {
        if (k < K) {
            ml[k] = a.part_ml[((int64_t)k * a.Hq + head) * a.T + tok];
            ov[k] = *reinterpret_cast<const vecE*>(a.part_o + (((int64_t)k * a.T + tok) * a.Hq + head) * D + E * lane);
        }
    }
    float M = -INFINITY;
#pragma unroll
    for (int k = 0; k < kChunkMaxSplit; ++k)
        if (k < K) M = fmaxf(M, ml[k].x);
    // a share with no key of the row (l = 0) carries no weight
    float Z = 0.0f;
#pragma unroll
    for (int k = 0; k < kChunkMaxSplit; ++k) {
        if (k < K) {
            const float w = (M == -INFINITY || ml[k].x == -INFINITY) ? 0.0f
                                                                     : __builtin_amdgcn_exp2f(ml[k].x - M) * ml[k].y;
            Z += ml[k].y > 0.0f ? w : 0.0f;
        }
    }
    const bool none = !(Z > 0.0f);
    vecE acc = {};
#pragma unroll
    for (int k = 0; k < kChunkMaxSplit; ++k) {
        if (k < K) {
            const float wk = (none || ml[k].y <= 0.0f) ? 0.0f : __builtin_amdgcn_exp2f(ml[k].x - M);
            acc += wk * ov[k];
        }
    }
    bf16* o = (bf16*)a.o + (tok * a.Hq + head) * (int64_t)D + E * lane;
#pragma unroll
    for (int i = 0; i < E; ++i) o[i] = (bf16)(none ? 0.0f : acc[i] / Z);
    if (lane == 0) a.lse[(int64_t)head * a.T + tok] = none ? -INFINITY : (M + log2f(Z)) * kLn2;
}

hipError_t launch_chunk_merge(const PrefillArgs& a, hipStream_t s) {
    LaunchScope scope("chunk_merge", s);
    if (a.ksplit > kChunkMaxSplit) return hipErrorInvalidValue;
    const dim3 grid((unsigned)a.T, (unsigned)((a.Hq + 3) / 4));
    if (a.d == 128) hipLaunchKernelGGL(chunk_merge_kernel<128>, grid, dim3(256), 0, s, a);
    else hipLaunchKernelGGL(chunk_merge_kernel<64>, grid, dim3(256), 0, s, a);
    return hipGetLastError();
}

}  // namespace jl
