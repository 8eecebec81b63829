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
// gfx950): rotated q and k must stay below 65504 in magnitude.  P and V stay
// bf16 for the PV product.  Rows below kPreciseRows, which see few keys, add
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
    static constexpr int LDS_BYTES = NBUF * BUF * 2;
    static constexpr int CH = D * kBN * 2 / 16 / 512;  // 16-byte chunks per thread per slot
    static constexpr int NS = D / 16;                   // k-steps of a QK^T product
    static constexpr int ND = D / 32;                   // 32-row blocks of O^T
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

    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
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

    // ---- rotate this lane's query values into B-operand registers ----
    // lane (qr, hh) holds d = 16*st + 8*hh + u for st < NS, u < 8; the RoPE
    // partner of step st is step st + NS/2.
    f16x8 QS[C::NS], QR[C::NS], QSl[C::NS], QRl[C::NS];
    {
        const float qscale = a.softmax_scale * kLog2e;
        float xq[C::NS][8];
        const bf16* qp = (const bf16*)a.q + ((int64_t)(start + myrow) * a.Hq + head) * D + 8 * hh;
#pragma unroll
        for (int st = 0; st < C::NS; ++st) {
            bf16x8 raw = {};
            if (row_valid) raw = *reinterpret_cast<const bf16x8*>(qp + 16 * st);
#pragma unroll
            for (int u = 0; u < 8; ++u) xq[st][u] = (float)raw[u];
        }
        const int32_t fpos = remap(myrow, G);
#pragma unroll
        for (int st = 0; st < C::NS / 2; ++st) {
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                const int t = 16 * st + 8 * hh + u;
                const float x0 = xq[st][u], x1 = xq[st + C::NS / 2][u];
                float c, sn;
                rope_cs(myrow, a.tab.rev[t], c, sn);
                float y0 = (x0 * c - x1 * sn) * qscale, y1 = (x1 * c + x0 * sn) * qscale;
                QS[st][u] = (f16)y0;
                QS[st + C::NS / 2][u] = (f16)y1;
                if constexpr (PRECISE) {
                    QSl[st][u] = (f16)(y0 - (float)QS[st][u]);
                    QSl[st + C::NS / 2][u] = (f16)(y1 - (float)QS[st + C::NS / 2][u]);
                }
                if (bif) {
                    rope_cs(fpos, a.tab.rev[t], c, sn);
                    y0 = (x0 * c - x1 * sn) * qscale;
                    y1 = (x1 * c + x0 * sn) * qscale;
                }
                QR[st][u] = (f16)y0;
                QR[st + C::NS / 2][u] = (f16)y1;
                if constexpr (PRECISE) {
                    QRl[st][u] = (f16)(y0 - (float)QR[st][u]);
                    QRl[st + C::NS / 2][u] = (f16)(y1 - (float)QR[st + C::NS / 2][u]);
                }
            }
        }
    }

    // ---- global tile sources ----
    const int64_t pad_off = e[kPlanPadOff];
    const bf16* KSg = (const bf16*)((const char*)a.ws + a.lay.ks) + ((int64_t)g * a.lay.T_pad + pad_off) * D;
    const bf16* KRg = (const bf16*)((const char*)a.ws + a.lay.kr) + ((int64_t)g * a.lay.T_pad + pad_off) * D;
    const bf16* VTg = (const bf16*)((const char*)a.ws + a.lay.vt) + ((int64_t)g * a.lay.T_pad + pad_off) * D;
    const bf16* KSlg = (const bf16*)((const char*)a.ws + a.lay.ks_lo) + ((int64_t)g * a.lay.lo_pad + e[kPlanLoOff]) * D;
    const bf16* KRlg = (const bf16*)((const char*)a.ws + a.lay.kr_lo) + ((int64_t)g * a.lay.lo_pad + e[kPlanLoOff]) * D;

    const int ntiles = (row_end + kBN - 1) / kBN;
    u32x4 rk[C::NK][C::CH];
    u32x4 rv[C::CH];

    auto tile_need = [&](int tau) -> uint32_t {
        return tile_class(row0, row_end, (int64_t)tau * kBN, (int64_t)tau * kBN + kBN, a.w_local, bif);
    };
    auto gload = [&](int tau, uint32_t cls) {
        const int64_t off = (int64_t)tau * kBN * D;
#pragma unroll
        for (int c = 0; c < C::CH; ++c) {
            const int64_t ch = (int64_t)(tid + 512 * c) * 8;
            if (cls & kHasLocal) {
                rk[0][c] = *reinterpret_cast<const u32x4*>(KSg + off + ch);
                if constexpr (PRECISE) rk[2][c] = *reinterpret_cast<const u32x4*>(KSlg + off + ch);
            }
            if (cls & kHasRemote) {
                rk[1][c] = *reinterpret_cast<const u32x4*>(KRg + off + ch);
                if constexpr (PRECISE) rk[3][c] = *reinterpret_cast<const u32x4*>(KRlg + off + ch);
            }
            rv[c] = *reinterpret_cast<const u32x4*>(VTg + off + ch);
        }
    };
    auto lstore = [&](int buf, uint32_t cls) {
        bf16* base = lds + buf * C::BUF;
#pragma unroll
        for (int c = 0; c < C::CH; ++c) {
            const int ch = tid + 512 * c;
            const int kr = ch / (D / 8), kc = (ch % (D / 8)) * 8;
            const int vr = ch / (kBN / 8), vc = (ch % (kBN / 8)) * 8;
            if (cls & kHasLocal) {
                *reinterpret_cast<u32x4*>(base + 0 * C::KSLOT + kr * C::KSTR + kc) = rk[0][c];
                if constexpr (PRECISE) *reinterpret_cast<u32x4*>(base + 2 * C::KSLOT + kr * C::KSTR + kc) = rk[2][c];
            }
            if (cls & kHasRemote) {
                *reinterpret_cast<u32x4*>(base + 1 * C::KSLOT + kr * C::KSTR + kc) = rk[1][c];
                if constexpr (PRECISE) *reinterpret_cast<u32x4*>(base + 3 * C::KSLOT + kr * C::KSTR + kc) = rk[3][c];
            }
            *reinterpret_cast<u32x4*>(base + C::NK * C::KSLOT + vr * C::VSTR + vc) = rv[c];
        }
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

    auto compute = [&](int tau, int buf) {
        const bf16* base = lds + buf * C::BUF;
        const int32_t j0 = tau * kBN;
        if (tile_class(wr0, wr_end, j0, j0 + kBN, a.w_local, bif) == 0) return;
        f32x16 S[2];
        uint32_t bcls[2];
#pragma unroll
        for (int b = 0; b < 2; ++b) {
            const int32_t jb = j0 + 32 * b;
            bcls[b] = tile_class(wr0, wr_end, jb, jb + 32, a.w_local, bif);
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
        // online softmax over this tile's 32 scores per lane (+ partner lane)
        float mx = -INFINITY;
#pragma unroll
        for (int b = 0; b < 2; ++b)
#pragma unroll
            for (int i = 0; i < 16; ++i) mx = fmaxf(mx, S[b][i]);
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        const float m_new = fmaxf(m_run, mx);
        const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
        m_run = m_new;
        float ls = 0.0f;
        bf16x8 P[2][2];
#pragma unroll
        for (int b = 0; b < 2; ++b)
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const float p = __builtin_amdgcn_exp2f(S[b][i] - m_new);
                ls += p;
                P[b][i >> 3][i & 7] = (bf16)p;
            }
        l_run = l_run * alpha + ls;
#pragma unroll
        for (int db = 0; db < C::ND; ++db)
#pragma unroll
            for (int i = 0; i < 16; ++i) O[db][i] *= alpha;
        // O^T += V^T P^T over the tile's four 16-key steps
        const bf16* vb = base + C::NK * C::KSLOT;
#pragma unroll
        for (int b = 0; b < 2; ++b) {
            if (bcls[b] == 0) continue;
#pragma unroll
            for (int u = 0; u < 2; ++u) {
#pragma unroll
                for (int db = 0; db < C::ND; ++db) {
                    const bf16x8 vv = *reinterpret_cast<const bf16x8*>(
                        vb + (32 * db + qr) * C::VSTR + 32 * b + 16 * u + 8 * hh);
                    O[db] = mfma32(vv, P[b][u], O[db]);
                }
            }
        }
    };

    // ---- main loop over key tiles ----
    {
        const uint32_t c0 = tile_need(0);
        gload(0, c0);
        lstore(0, c0);
        __syncthreads();
    }
    for (int tau = 0; tau < ntiles; ++tau) {
        const int cur = (C::NBUF == 2) ? (tau & 1) : 0;
        const bool more = tau + 1 < ntiles;
        uint32_t cn = 0;
        if (more) cn = tile_need(tau + 1);
        if (C::NBUF == 2 && more) gload(tau + 1, cn);
        if (wave_active) compute(tau, cur);
        if (more) {
            if (C::NBUF == 2) {
                lstore(cur ^ 1, cn);
            } else {
                __syncthreads();
                gload(tau + 1, cn);
                lstore(0, cn);
            }
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
