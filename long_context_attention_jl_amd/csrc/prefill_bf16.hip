// prefill_bf16.hip -- bifocal causal prefill on gfx950 bf16 MFMA.
//
// Pages cited (title, section):
//   [BT] "Jet-Long: 具有动态双焦RoPE的高效长上下文扩展" (bittide.aicompass.dev)
//   [TW] "NVIDIA研究团队找到了让AI“看清”超长文本的新方法" (techwalker.com)
//
// The pages fuse three attention calls -- B: full causal with remapped RoPE,
// A: local window with standard RoPE, C: local window with remapped RoPE --
// into Attn = B + A - C merged in LogSumExp space ([TW] §四, [BT] §3.2).  That
// sum equals one softmax in which local keys are scored under standard RoPE
// and remote keys under remapped RoPE, so this kernel evaluates that single
// softmax directly: each 32x32 score block is classified from its extreme
// distances (all local, all remote, straddling the band edge, or masked),
// fully local/remote blocks cost one QK^T product and only straddling blocks
// compute both and select per element.  No L x L mask exists ([TW] §四).
//
// Work decomposition (one workgroup = 8 waves = 256 query rows of one head):
//   S^T = K Q^T on v_mfma_f32_32x32x16_f16 with K (32 keys x 16 d) from LDS
//   as the A operand and the wave's rotated queries held in registers as B;
//   lane (query r, half h) then holds 16 scores of query r per block, so the
//   row max needs one exchange with lane r + 32, and the probabilities feed the
//   PV product O^T += V^T P^T directly as its B operand (V^T tiles are laid
//   out by the pre-pass so each lane reads its 8 keys as one 16-byte vector).
//   K/V^T tiles of 64 keys are double-buffered in LDS; the next tile's global
//   loads are issued before the current tile's math.
// Queries are rotated in registers at entry (fp64-reduced angles) and scaled
// by softmax_scale * log2(e) so the softmax runs on exp2.
//
// Operand precision: the rotated queries and keys are 16-bit MFMA operands.
// Rounding a key is a random error per key and averages out over the
// softmax, but rounding a query is a fixed error per row whose weighted mean
// over the keys does not shrink (the softmax-weighted mean key points along
// the query), so its size sets the LSE error directly.  The QK^T product
// therefore uses fp16 operands (11-bit significand, same MFMA rate as bf16 on
// gfx950): rotated q and k must stay below 65504 in magnitude.  PV runs on
// fp16 too: V (bf16 input, exact in fp16 within its range) and the
// probabilities, whose row sum is taken from the same fp16 values with
// v_dot2_f32_f16 so numerator and denominator agree.  Rows below kPreciseRows, which see few keys, add
// the fp16 residuals of q and k (hi * hi + hi * lo + lo * hi).
#include "internal.h"

namespace jl {

namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

template <int D, bool PRECISE>
struct Cfg {
    static constexpr int KSTR = D + 8;         // LDS row stride of a K tile (bf16)
    static constexpr int VSTR = kBN + 8;       // LDS row stride of a V^T tile
    static constexpr int KSLOT = kBN * KSTR;   // elements
    static constexpr int VSLOT = D * VSTR;
    static constexpr int NK = PRECISE ? 4 : 2; // KS, KR (+ KS_lo, KR_lo)
    static constexpr int NBUF = PRECISE ? 1 : 2;
    static constexpr int BUF = NK * KSLOT + VSLOT;
    static constexpr int QIMG = 2 * kBM * KSTR * 2;    // rotated-query images (prologue)
    static constexpr int LDS_BYTES = (NBUF * BUF * 2) > QIMG ? (NBUF * BUF * 2) : QIMG;
    static constexpr int CH = D * kBN * 2 / 16 / 512;  // 16-byte chunks per thread per slot
    static constexpr int NS = D / 16;                   // k-steps of a QK^T product
    static constexpr int ND = D / 32;                   // 32-row blocks of O^T
};

template <bool B>
struct BoolC {
    static constexpr bool value = B;
};

__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x16 mfma32h(f16x8 a, f16x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}

}  // namespace

template <int D, bool PRECISE>
__global__ __launch_bounds__(512) void prefill_bf16_kernel(PrefillArgs a, int rb_first,
                                                           int n_rb) {
    using C = Cfg<D, PRECISE>;
    extern __shared__ __align__(16) char smem_raw[];
    bf16* lds = reinterpret_cast<bf16*>(smem_raw);

    // the wave index is uniform per wave; readfirstlane tells the compiler so,
    // which keeps every per-wave tile-class branch a scalar branch (otherwise
    // all score paths would run under lane masks, MFMAs included)
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int qr = lane & 31, hh = lane >> 5;  // query column, lane half

    // ---- which (head, sequence, row block) ----
    int head = blockIdx.x;
    if ((a.Hq & 7) == 0) head = (blockIdx.x & 7) * (a.Hq >> 3) + (blockIdx.x >> 3);
    const int s = blockIdx.y;
    const int rb = rb_first + (n_rb - 1 - (int)blockIdx.z);  // longest rows first
    const int32_t* plan = (const int32_t*)((const char*)a.ws + a.lay.plan);
    const int32_t* e = plan + s * kPlanFields;
    const int32_t start = e[kPlanStart], len = e[kPlanLen], G = e[kPlanG];
    const int32_t row0 = rb * kBM;
    if (row0 >= len) return;
    if (!PRECISE && row0 < kPreciseRows) return;
    const int32_t row_end = min(row0 + kBM, len);
    const bool bif = a.bifocal && G > 1;
    const int g = head / (a.Hq / a.Hkv);
    const int32_t wr0 = row0 + wave * kWaveRows;
    const int32_t wr_end = min(wr0 + kWaveRows, len);
    const bool wave_active = wr0 < wr_end;
    const int32_t myrow = wr0 + qr;
    const bool row_valid = myrow < len;

    // ---- rotated, scaled queries as MFMA B operands ----
    // The workgroup rotates its 256 query rows cooperatively into LDS (the
    // K/V buffers are not in use yet): thread (t, r) handles pair t of rows
    // r, r + 512/(D/2), ...; then lane (qr, hh) of each wave reads its
    // operand registers, d = 16*st + 8*hh + u, as 16-byte vectors.
    f16x8 QS[C::NS], QR[C::NS], QSl[C::NS], QRl[C::NS];
    {
        const float qscale = a.softmax_scale * kLog2e;
        constexpr int HALF = D / 2;
        f16* qs_l = reinterpret_cast<f16*>(smem_raw);
        f16* qr_l = qs_l + kBM * C::KSTR;
        const int t = tid % HALF;
        const double rv = rope_rev(a.tab, t);
        const bf16* qg = (const bf16*)a.q + (int64_t)head * D;
        for (int round = 0; round < (PRECISE ? 2 : 1); ++round) {
#pragma unroll 1
            for (int r = tid / HALF; r < kBM; r += 512 / HALF) {
                const int32_t row = row0 + r;
                float x0 = 0.0f, x1 = 0.0f;
                if (row < len) {
                    const bf16* qp = qg + (int64_t)(start + row) * a.Hq * D;
                    x0 = (float)qp[t];
                    x1 = (float)qp[t + HALF];
                }
                float c, sn;
                rope_cs(row, rv, c, sn);
                float y0 = (x0 * c - x1 * sn) * qscale, y1 = (x1 * c + x0 * sn) * qscale;
                if (round == 0) {
                    qs_l[r * C::KSTR + t] = (f16)y0;
                    qs_l[r * C::KSTR + t + HALF] = (f16)y1;
                } else {
                    qs_l[r * C::KSTR + t] = (f16)(y0 - (float)(f16)y0);
                    qs_l[r * C::KSTR + t + HALF] = (f16)(y1 - (float)(f16)y1);
                }
                if (bif) {
                    rope_cs(remap(row, G), rv, c, sn);
                    y0 = (x0 * c - x1 * sn) * qscale;
                    y1 = (x1 * c + x0 * sn) * qscale;
                }
                if (round == 0) {
                    qr_l[r * C::KSTR + t] = (f16)y0;
                    qr_l[r * C::KSTR + t + HALF] = (f16)y1;
                } else {
                    qr_l[r * C::KSTR + t] = (f16)(y0 - (float)(f16)y0);
                    qr_l[r * C::KSTR + t + HALF] = (f16)(y1 - (float)(f16)y1);
                }
            }
            __syncthreads();
            const int qoff = (wave * kWaveRows + qr) * C::KSTR + 8 * hh;
#pragma unroll
            for (int st = 0; st < C::NS; ++st) {
                const f16x8 vs = *reinterpret_cast<const f16x8*>(qs_l + qoff + 16 * st);
                const f16x8 vr = *reinterpret_cast<const f16x8*>(qr_l + qoff + 16 * st);
                if (round == 0) {
                    QS[st] = vs;
                    QR[st] = vr;
                } else {
                    QSl[st] = vs;
                    QRl[st] = vr;
                }
            }
            __syncthreads();
        }
    }

    const int64_t ntp = a.lay.T_pad / kBN, ntl = a.lay.lo_pad / kBN;
    const bf16* KSg = (const bf16*)((const char*)a.ws + a.lay.ks) + ((int64_t)g * ntp + e[kPlanTile0]) * C::KSLOT;
    const bf16* KRg = (const bf16*)((const char*)a.ws + a.lay.kr) + ((int64_t)g * ntp + e[kPlanTile0]) * C::KSLOT;
    const bf16* VTg = (const bf16*)((const char*)a.ws + a.lay.vt) + ((int64_t)g * ntp + e[kPlanTile0]) * C::VSLOT;
    const bf16* KSlg = (const bf16*)((const char*)a.ws + a.lay.ks_lo) + ((int64_t)g * ntl + e[kPlanLoTile0]) * C::KSLOT;
    const bf16* KRlg = (const bf16*)((const char*)a.ws + a.lay.kr_lo) + ((int64_t)g * ntl + e[kPlanLoTile0]) * C::KSLOT;

    const int ntiles = (row_end + kBN - 1) / kBN;

    auto tile_need = [&](int tau) -> uint32_t {
        return tile_class32(row0, row_end, tau * kBN, tau * kBN + kBN, a.w_local, bif);
    };
    // global -> LDS DMA of one tile image: each wave instruction moves 64 x 16
    // contiguous bytes; the workspace holds the tiles in their LDS layout.
    auto dma = [&](const bf16* src, bf16* dst, int elems) {
        const int nchunk = elems / 8;
        for (int c0 = wave * 64; c0 < nchunk; c0 += 512) {
            if (c0 + lane < nchunk)
                __builtin_amdgcn_global_load_lds((const void*)(src + (int64_t)(c0 + lane) * 8),
                                                 (void*)(dst + c0 * 8), 16, 0, 0);
        }
    };
    auto load_tile = [&](int tau, int buf, uint32_t cls) {
        bf16* base = lds + buf * C::BUF;
        if (cls & kHasLocal) {
            dma(KSg + (int64_t)tau * C::KSLOT, base, C::KSLOT);
            if constexpr (PRECISE) dma(KSlg + (int64_t)tau * C::KSLOT, base + 2 * C::KSLOT, C::KSLOT);
        }
        if (cls & kHasRemote) {
            dma(KRg + (int64_t)tau * C::KSLOT, base + C::KSLOT, C::KSLOT);
            if constexpr (PRECISE) dma(KRlg + (int64_t)tau * C::KSLOT, base + 3 * C::KSLOT, C::KSLOT);
        }
        dma(VTg + (int64_t)tau * C::VSLOT, base + C::NK * C::KSLOT, C::VSLOT);
    };

    // ---- running softmax state (log2 domain) and O^T accumulators ----
    float m_run = -INFINITY, l_run = 0.0f;
    f32x16 O[C::ND];
#pragma unroll
    for (int db = 0; db < C::ND; ++db) O[db] = f32x16{};

    auto qk = [&](const bf16* kslot, const bf16* kslot_lo, const f16x8* Q, const f16x8* Ql,
                  int b) -> f32x16 {
        f32x16 acc = {};
        const bf16* kp = kslot + (32 * b + qr) * C::KSTR + 8 * hh;
#pragma unroll
        for (int st = 0; st < C::NS; ++st) {
            const f16x8 kv = *reinterpret_cast<const f16x8*>(kp + 16 * st);
            acc = mfma32h(kv, Q[st], acc);
            if constexpr (PRECISE) {
                acc = mfma32h(kv, Ql[st], acc);
                const f16x8 kl = *reinterpret_cast<const f16x8*>(kslot_lo + (32 * b + qr) * C::KSTR + 8 * hh + 16 * st);
                acc = mfma32h(kl, Q[st], acc);
            }
        }
        return acc;
    };

    // Raises the running max when a score exceeds it by more than 8 (log2
    // units).  Sums stay exact relative to whatever max they use, p stays
    // below 2^8, and most tiles skip rescaling O entirely.
    auto maybe_raise = [&](float mx) {
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        const bool raise = mx > m_run + 8.0f;
        if (__any(raise)) {
            const float m_new = raise ? mx : m_run;
            const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
            m_run = m_new;
            l_run *= alpha;
#pragma unroll
            for (int db = 0; db < C::ND; ++db)
#pragma unroll
                for (int i = 0; i < 16; ++i) O[db][i] *= alpha;
        }
    };
    const f16x2 ones = {(f16)1.0f, (f16)1.0f};
    // p = exp2(s - m) as fp16 B operands, and their row sum
    auto probs = [&](const f32x16& Sb, f16x8* Pb) {
#pragma unroll
        for (int i = 0; i < 16; ++i) Pb[i >> 3][i & 7] = (f16)__builtin_amdgcn_exp2f(Sb[i] - m_run);
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
            for (int i = 0; i < 8; i += 2) {
                const f16x2 pp = {Pb[h2][i], Pb[h2][i + 1]};
                l_run = __builtin_amdgcn_fdot2(pp, ones, l_run, false);
            }
    };
    // O^T += V^T P^T for one 32-key block (two 16-key steps)
    auto pv = [&](const bf16* vb, int b, const f16x8* Pb) {
#pragma unroll
        for (int u = 0; u < 2; ++u)
#pragma unroll
            for (int db = 0; db < C::ND; ++db) {
                const f16x8 vv = *reinterpret_cast<const f16x8*>(
                    vb + (32 * db + qr) * C::VSTR + 32 * b + 16 * u + 8 * hh);
                O[db] = mfma32h(vv, Pb[u], O[db]);
            }
    };

    // Fast path: the wave's whole tile is local or remote and unmasked.  Both
    // score blocks are issued first; then block 0's probabilities; then the
    // block-0 PV products are interleaved with block 1's exponentials so the
    // matrix unit and the vector ALU work at the same time.
    auto fast_tile = [&](const bf16* base, auto remote_c) {
        constexpr bool REMOTE = decltype(remote_c)::value;
        const f16x8* Q = REMOTE ? QR : QS;
        const bf16* kp = base + (REMOTE ? C::KSLOT : 0) + qr * C::KSTR + 8 * hh;
        f32x16 S0 = {}, S1 = {};
#pragma unroll
        for (int st = 0; st < C::NS; ++st)
            S0 = mfma32h(*reinterpret_cast<const f16x8*>(kp + 16 * st), Q[st], S0);
#pragma unroll
        for (int st = 0; st < C::NS; ++st)
            S1 = mfma32h(*reinterpret_cast<const f16x8*>(kp + 32 * C::KSTR + 16 * st), Q[st], S1);
        float mx = -INFINITY;
#pragma unroll
        for (int i = 0; i < 16; ++i) mx = fmaxf(mx, fmaxf(S0[i], S1[i]));
        maybe_raise(mx);
        const bf16* vb = base + C::NK * C::KSLOT;
        f16x8 P0[2], P1[2];
        probs(S0, P0);
        pv(vb, 0, P0);
        probs(S1, P1);
        // PV(block 0): 8 x (1 LDS read + 1 MFMA) interleaved with the 48
        // vector instructions of block 1's probabilities
#pragma unroll
        for (int g = 0; g < 8; ++g) {
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // DS read
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
            __builtin_amdgcn_sched_group_barrier(0x002, 6, 0);  // VALU
        }
        pv(vb, 1, P1);
    };

    auto compute = [&](int tau, int buf) {
        const bf16* base = lds + buf * C::BUF;
        const int32_t j0 = tau * kBN;
        const uint32_t tc = tile_class32(wr0, wr_end, j0, j0 + kBN, a.w_local, bif);
        if (tc == 0) return;
        if constexpr (!PRECISE) {
            if (tc == kHasLocal) {
                fast_tile(base, BoolC<false>{});
                return;
            }
            if (tc == kHasRemote) {
                fast_tile(base, BoolC<true>{});
                return;
            }
        }
        f32x16 S[2];
        uint32_t bcls[2];
#pragma unroll
        for (int b = 0; b < 2; ++b) {
            const int32_t jb = j0 + 32 * b;
            bcls[b] = tile_class32(wr0, wr_end, jb, jb + 32, a.w_local, bif);
            if (bcls[b] == 0) {
#pragma unroll
                for (int i = 0; i < 16; ++i) S[b][i] = -INFINITY;
                continue;
            }
            const uint32_t both = kHasLocal | kHasRemote;
            if ((bcls[b] & both) == kHasLocal) {
                S[b] = qk(base + 0 * C::KSLOT, base + 2 * C::KSLOT, QS, QSl, b);
            } else if ((bcls[b] & both) == kHasRemote) {
                S[b] = qk(base + 1 * C::KSLOT, base + 3 * C::KSLOT, QR, QRl, b);
            } else {
                const f32x16 sl = qk(base + 0 * C::KSLOT, base + 2 * C::KSLOT, QS, QSl, b);
                const f32x16 sr = qk(base + 1 * C::KSLOT, base + 3 * C::KSLOT, QR, QRl, b);
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const int32_t key = jb + (i >> 2) * 8 + 4 * hh + (i & 3);
                    S[b][i] = (myrow - key < a.w_local) ? sl[i] : sr[i];
                }
            }
            if (bcls[b] & kHasMasked) {
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const int32_t key = jb + (i >> 2) * 8 + 4 * hh + (i & 3);
                    if (key > myrow) S[b][i] = -INFINITY;
                }
            }
        }
        float mx = -INFINITY;
#pragma unroll
        for (int i = 0; i < 16; ++i) mx = fmaxf(mx, fmaxf(S[0][i], S[1][i]));
        maybe_raise(mx);
        f16x8 P[2][2];
        probs(S[0], P[0]);
        probs(S[1], P[1]);
        const bf16* vb = base + C::NK * C::KSLOT;
        if (bcls[0] != 0) pv(vb, 0, P[0]);
        if (bcls[1] != 0) pv(vb, 1, P[1]);
    };

    // ---- main loop over key tiles ----
    load_tile(0, 0, tile_need(0));
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    for (int tau = 0; tau < ntiles; ++tau) {
        const int cur = (C::NBUF == 2) ? (tau & 1) : 0;
        const bool more = tau + 1 < ntiles;
        const uint32_t cn = more ? tile_need(tau + 1) : 0u;
        // the other buffer was last read in iteration tau - 1, which every
        // wave finished before the barrier that ended it
        if (C::NBUF == 2 && more) load_tile(tau + 1, cur ^ 1, cn);
        if (wave_active) compute(tau, cur);
        if (more) {
            if (C::NBUF == 1) {
                __syncthreads();
                load_tile(tau + 1, 0, cn);
            }
            __builtin_amdgcn_s_waitcnt(0);  // this wave's DMA writes have landed
            __syncthreads();
        }
    }

    // ---- epilogue: O = O^T / l, LSE = ln(sum exp(score)) ----
    if (!wave_active || !row_valid) return;
    const float l_tot = l_run + __shfl_xor(l_run, 32);
    const float inv = 1.0f / l_tot;
    bf16* op = (bf16*)a.o + ((int64_t)(start + myrow) * a.Hq + head) * D;
#pragma unroll
    for (int db = 0; db < C::ND; ++db)
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
            bf16x4 w;
#pragma unroll
            for (int r = 0; r < 4; ++r) w[r] = (bf16)(O[db][4 * g4 + r] * inv);
            *reinterpret_cast<bf16x4*>(op + 32 * db + 8 * g4 + 4 * hh) = w;
        }
    if (hh == 0) a.lse[(int64_t)head * a.T + start + myrow] = (m_run + log2f(l_tot)) * kLn2;
}

template <int D, bool PRECISE>
static hipError_t launch_one(const PrefillArgs& a, int rb_first, int n_rb, hipStream_t s,
                             const char* name) {
    using C = Cfg<D, PRECISE>;
    if (n_rb <= 0) return hipSuccess;
    static bool attr_set = false;
    if (!attr_set) {
        hipError_t err = hipFuncSetAttribute((const void*)prefill_bf16_kernel<D, PRECISE>,
                                             hipFuncAttributeMaxDynamicSharedMemorySize,
                                             C::LDS_BYTES);
        if (err != hipSuccess) return err;
        attr_set = true;
    }
    LaunchScope scope(name, s);
    hipLaunchKernelGGL((prefill_bf16_kernel<D, PRECISE>), dim3(a.Hq, a.n_seqs, n_rb), dim3(512),
                       C::LDS_BYTES, s, a, rb_first, n_rb);
    return hipGetLastError();
}

hipError_t launch_prefill_bf16(const PrefillArgs& a, hipStream_t s) {
    const int total_rb = (a.max_seqlen + kBM - 1) / kBM;
    const int precise_rb = kPreciseRows / kBM;
    const int n_prec = total_rb < precise_rb ? total_rb : precise_rb;
    hipError_t err;
    if (a.d == 128) {
        err = launch_one<128, true>(a, 0, n_prec, s, "prefill_bf16_precise");
        if (err != hipSuccess) return err;
        return launch_one<128, false>(a, precise_rb, total_rb - precise_rb, s, "prefill_bf16");
    }
    err = launch_one<64, true>(a, 0, n_prec, s, "prefill_bf16_precise");
    if (err != hipSuccess) return err;
    return launch_one<64, false>(a, precise_rb, total_rb - precise_rb, s, "prefill_bf16");
}

}  // namespace jl
