// api.hip -- the C ABI of libjetlong: argument validation, workspace layout,
// dispatch to the gfx950 kernels, error reporting and kernel timing.
//
// Pages cited (title, section):
//   [BT] "Jet-Long: 具有动态双焦RoPE的高效长上下文扩展" (bittide.aicompass.dev)
//   [TW] "NVIDIA研究团队找到了让AI“看清”超长文本的新方法" (techwalker.com)
#include <math.h>
#include <stdlib.h>
#include <string.h>

#include <initializer_list>
#include <mutex>
#include <string>
#include <vector>

#include "jetlong.h"
#include "internal.h"

namespace jl {

// ---------------------------------------------------------------------------
// errors

static thread_local std::string g_err;

static jl_status fail(jl_status st, const std::string& msg) {
    g_err = msg;
    if (getenv("JL_LOG")) fprintf(stderr, "libjetlong: %s\n", msg.c_str());
    return st;
}

static jl_status hip_fail(hipError_t e, const char* where) {
    return fail(JL_ERR_HIP, std::string(where) + ": " + hipGetErrorString(e));
}

static jl_status finish(hipStream_t s, const char* where) {
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return hip_fail(e, where);
    if (getenv("JL_DEBUG_SYNC")) {
        e = hipStreamSynchronize(s);
        if (e == hipSuccess) e = hipGetLastError();
        if (e != hipSuccess) return hip_fail(e, where);
    }
    g_err.clear();
    return JL_OK;
}

// ---------------------------------------------------------------------------
// kernel timing

namespace {
struct Rec {
    const char* name;
    hipEvent_t start, stop;
};
std::mutex g_prof_mu;
bool g_prof_on = false;
std::vector<Rec> g_recs;
std::vector<hipEvent_t> g_pool;

hipEvent_t take_event() {
    if (!g_pool.empty()) {
        hipEvent_t e = g_pool.back();
        g_pool.pop_back();
        return e;
    }
    hipEvent_t e = nullptr;
    if (hipEventCreate(&e) != hipSuccess) return nullptr;
    return e;
}

void clear_records() {
    for (auto& r : g_recs) {
        g_pool.push_back(r.start);
        g_pool.push_back(r.stop);
    }
    g_recs.clear();
}
}  // namespace

LaunchScope::LaunchScope(const char* name, hipStream_t s) : name_(name), stream_(s), slot_(-1) {
    std::lock_guard<std::mutex> lk(g_prof_mu);
    if (!g_prof_on) return;
    Rec r{name, take_event(), take_event()};
    if (!r.start || !r.stop) return;
    if (hipEventRecord(r.start, s) != hipSuccess) return;
    slot_ = (int)g_recs.size();
    g_recs.push_back(r);
}

LaunchScope::~LaunchScope() {
    if (slot_ < 0) return;
    std::lock_guard<std::mutex> lk(g_prof_mu);
    if (slot_ < (int)g_recs.size()) (void)hipEventRecord(g_recs[slot_].stop, stream_);
}

// ---------------------------------------------------------------------------
// layouts

static size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

PrefillLayout prefill_layout(int64_t T, int32_t n_seqs, int32_t Hkv, int32_t d, int dtype,
                             int precise) {
    PrefillLayout L{};
    L.T_pad = (T + (int64_t)n_seqs * (kBN - 1) + kBN - 1) / kBN * kBN;
    int64_t lo = precise ? T : (int64_t)n_seqs * kPreciseRows;
    if (lo > T) lo = T;
    L.lo_pad = (lo + (int64_t)n_seqs * (kBN - 1) + kBN - 1) / kBN * kBN;
    size_t off = 0;
    L.plan = off;
    off = align256(off + (size_t)(n_seqs + 1) * kPlanFields * sizeof(int32_t));
    if (dtype == JL_DTYPE_BF16) {
        const size_t kb = (size_t)Hkv * (L.T_pad / kBN) * ktile_elems(d) * 2;
        const size_t vb = (size_t)Hkv * (L.T_pad / kBN) * vtile_elems(d) * 2;
        const size_t lb = (size_t)Hkv * (L.lo_pad / kBN) * ktile_elems(d) * 2;
        L.ks = off; off = align256(off + kb);
        L.kr = off; off = align256(off + kb);
        L.vt = off; off = align256(off + vb);
        L.ks_lo = off; off = align256(off + lb);
        L.kr_lo = off; off = align256(off + lb);
    } else {
        const size_t kb = (size_t)Hkv * T * d * 4;
        L.ks32 = off; off = align256(off + kb);
        L.kr32 = off; off = align256(off + kb);
    }
    L.total = off;
    return L;
}

DecodeLayout decode_layout(int32_t B, int32_t max_seqlen_k, int32_t Hq, int32_t Hkv, int32_t d,
                           int dtype, int target_wg) {
    DecodeLayout L{};
    // bf16: 8-wave workgroups (one per compute unit), 48-position stages;
    // fp32: 4-wave workgroups (two per compute unit), 64-position stages
    const bool b16 = dtype == JL_DTYPE_BF16;
    const int wmax = b16 ? 8 : 4;
    const int stage = b16 ? kDecodeStageB : 64;
    const int nw = Hkv < wmax ? Hkv : wmax;  // waves (kv heads) per decode workgroup
    const int64_t groups = (Hkv + nw - 1) / nw;
    // workgroups per call (one 8-wave bf16 workgroup per compute unit)
    const int64_t target = target_wg > 0 ? target_wg : (b16 ? 256 : 512);
    const int64_t span = (int64_t)max_seqlen_k + stage - 1;
    int64_t want = (target + (int64_t)B * groups - 1) / ((int64_t)B * groups);
    if (want < 1) want = 1;
    int64_t chunk = (span + want - 1) / want;
    chunk = (chunk + stage - 1) / stage * stage;
    if (b16 && chunk > (int64_t)kDecodeMaxStagesB * stage) chunk = (int64_t)kDecodeMaxStagesB * stage;
    if (b16) {  // the kernel's byte offsets within a chunk (plus loads ahead) stay 32-bit
        const int64_t rowb = (int64_t)Hkv * d * 2;
        int64_t cap = ((int64_t)INT32_MAX / rowb - 64) / stage * stage;
        if (cap < stage) cap = stage;
        if (chunk > cap) chunk = cap;
    }
    L.chunk = (int32_t)chunk;
    L.n_splits = (int32_t)((span + chunk - 1) / chunk);
    size_t off = 0;
    L.part_ml = off;
    off = align256(off + (size_t)B * L.n_splits * Hq * 4 * sizeof(float));
    L.part_o = off;
    off = align256(off + (size_t)B * L.n_splits * Hq * d * sizeof(float));
    L.total = off;
    return L;
}

bool decode_interleave(bool paged, int32_t Hq, int32_t Hkv, int32_t d, int32_t max_seqlen_k,
                       int32_t elem_bytes) {
    if (paged || Hq / Hkv > 8) return false;
    // loads reach past L by up to a stride of n_splits stages (at most the
    // sequence's span plus a chunk) and two tiles; negative offsets (stages
    // starting below 0) stay above -2^31 as well
    const int64_t rows = 2 * ((int64_t)max_seqlen_k + (int64_t)(kDecodeMaxStagesB + 4) * kDecodeStageB);
    return rows * Hkv * d * elem_bytes < (int64_t)INT32_MAX;
}

RopeFreq make_rope_freq(double base, int d) {
    RopeFreq f;
    f.c = -2.0 * log2(base) / (double)d;
    return f;
}

}  // namespace jl

using namespace jl;

// ---------------------------------------------------------------------------
// shared checks (pure host code: no HIP call happens before they pass)

static jl_status check_dtype_d(jl_dtype dtype, int32_t d) {
    if (dtype != JL_DTYPE_F32 && dtype != JL_DTYPE_BF16)
        return fail(JL_ERR_UNSUPPORTED, "dtype must be JL_DTYPE_F32 or JL_DTYPE_BF16");
    if (d <= 0 || (d & 1)) return fail(JL_ERR_INVALID_ARGUMENT, "d must be a positive even number");
    if (d != 64 && d != 128) return fail(JL_ERR_UNSUPPORTED, "d must be 64 or 128");
    return JL_OK;
}

static jl_status check_params(const jl_params* p) {
    if (!p) return fail(JL_ERR_INVALID_ARGUMENT, "params is NULL");
    if (p->w_pretrained < 1) return fail(JL_ERR_INVALID_ARGUMENT, "w_pretrained must be >= 1");
    if (p->w_local < 0) return fail(JL_ERR_INVALID_ARGUMENT, "w_local must be >= 0");
    if (!(p->rope_base > 0.0) || !isfinite(p->rope_base))
        return fail(JL_ERR_INVALID_ARGUMENT, "rope_base must be finite and > 0");
    if (!(p->softmax_scale > 0.0f) || !isfinite(p->softmax_scale))
        return fail(JL_ERR_INVALID_ARGUMENT, "softmax_scale must be finite and > 0");
    if (p->bifocal < 0 || p->bifocal > 2)
        return fail(JL_ERR_INVALID_ARGUMENT, "bifocal must be 0, 1 or 2");
    if (p->precise != 0 && p->precise != 1)
        return fail(JL_ERR_INVALID_ARGUMENT, "precise must be 0 or 1");
    if (p->reuse_images != 0 && p->reuse_images != 1)
        return fail(JL_ERR_INVALID_ARGUMENT, "reuse_images must be 0 or 1");
    return JL_OK;
}

// precise flag of an optional params pointer (workspace queries)
static int precise_of(const jl_params* p) { return p && p->precise ? 1 : 0; }

// The kernels move tensors in 16-byte vectors.
static bool al16(const void* p) { return ((uintptr_t)p & 15) == 0; }
static jl_status check_aligned(std::initializer_list<const void*> ps) {
    for (const void* p : ps)
        if (p && !al16(p)) return fail(JL_ERR_INVALID_ARGUMENT, "tensors must be 16-byte aligned");
    return JL_OK;
}

static jl_status check_heads(int32_t Hq, int32_t Hkv) {
    if (Hq < 1 || Hkv < 1) return fail(JL_ERR_INVALID_ARGUMENT, "Hq and Hkv must be >= 1");
    if (Hq % Hkv) return fail(JL_ERR_INVALID_ARGUMENT, "Hq must be a multiple of Hkv");
    if (Hq > 65535) return fail(JL_ERR_UNSUPPORTED, "Hq above 65535");
    return JL_OK;
}

extern "C" {

int jl_abi_version(void) { return JL_ABI_VERSION; }

const char* jl_status_string(int status) {
    switch (status) {
        case JL_OK: return "JL_OK";
        case JL_ERR_INVALID_ARGUMENT: return "JL_ERR_INVALID_ARGUMENT";
        case JL_ERR_UNSUPPORTED: return "JL_ERR_UNSUPPORTED";
        case JL_ERR_WORKSPACE_TOO_SMALL: return "JL_ERR_WORKSPACE_TOO_SMALL";
        case JL_ERR_HIP: return "JL_ERR_HIP";
        default: return "JL_UNKNOWN_STATUS";
    }
}

const char* jl_last_error(void) { return g_err.c_str(); }

jl_status jl_group_size(int64_t L, int32_t w_pretrained, int32_t* G_out) {
    if (!G_out) return fail(JL_ERR_INVALID_ARGUMENT, "G_out is NULL");
    if (L < 1) return fail(JL_ERR_INVALID_ARGUMENT, "L must be >= 1");
    if (w_pretrained < 1) return fail(JL_ERR_INVALID_ARGUMENT, "w_pretrained must be >= 1");
    const int64_t G = group_size(L, w_pretrained);
    if (G > 2147483647LL) return fail(JL_ERR_INVALID_ARGUMENT, "G does not fit in int32");
    *G_out = (int32_t)G;
    g_err.clear();
    return JL_OK;
}

jl_status jl_rope_apply(void* out, const void* x, const int32_t* positions, int64_t T, int32_t H,
                        int32_t d, double rope_base, int32_t G, jl_dtype dtype, void* stream) {
    if (!out || !x || !positions) return fail(JL_ERR_INVALID_ARGUMENT, "null pointer argument");
    if (T < 1 || H < 1) return fail(JL_ERR_INVALID_ARGUMENT, "T and H must be >= 1");
    jl_status st = check_dtype_d(dtype, d);
    if (st != JL_OK) return st;
    if (!(rope_base > 0.0) || !isfinite(rope_base))
        return fail(JL_ERR_INVALID_ARGUMENT, "rope_base must be finite and > 0");
    if (G < 1) return fail(JL_ERR_INVALID_ARGUMENT, "G must be >= 1");
    if (T > (1LL << 40) / ((int64_t)H * d)) return fail(JL_ERR_INVALID_ARGUMENT, "T*H*d too large");
    hipStream_t s = (hipStream_t)stream;
    hipError_t e = launch_rope_apply(out, x, positions, T, H, d, make_rope_freq(rope_base, d), G,
                                     dtype, s);
    if (e != hipSuccess) return hip_fail(e, "jl_rope_apply launch");
    return finish(s, "jl_rope_apply");
}

jl_status jl_bifocal_prefill_workspace(int64_t T, int32_t n_seqs, int32_t Hq, int32_t Hkv,
                                       int32_t d, jl_dtype dtype, const jl_params* params,
                                       size_t* bytes) {
    if (!bytes) return fail(JL_ERR_INVALID_ARGUMENT, "bytes is NULL");
    if (T < 1 || n_seqs < 1) return fail(JL_ERR_INVALID_ARGUMENT, "T and n_seqs must be >= 1");
    jl_status st = check_heads(Hq, Hkv);
    if (st != JL_OK) return st;
    st = check_dtype_d(dtype, d);
    if (st != JL_OK) return st;
    if (T + (int64_t)n_seqs * kBN >= 2147483647LL)
        return fail(JL_ERR_UNSUPPORTED, "T + 64 * n_seqs must stay below 2^31");
    if (params) {
        const jl_status pst = check_params(params);
        if (pst != JL_OK) return pst;
    }
    *bytes = prefill_layout(T, n_seqs, Hkv, d, dtype, precise_of(params)).total;
    g_err.clear();
    return JL_OK;
}

jl_status jl_bifocal_prefill(void* o, float* lse, const void* q, const void* k, const void* v,
                             const int32_t* cu_seqlens, int32_t n_seqs, int64_t T,
                             int32_t max_seqlen, int32_t Hq, int32_t Hkv, int32_t d,
                             const jl_params* params, jl_dtype dtype, void* k_rot_out,
                             void* workspace, size_t workspace_bytes, void* stream) {
    if (!o || !lse || !q || !k || !v || !workspace)
        return fail(JL_ERR_INVALID_ARGUMENT, "null pointer argument");
    jl_status st = check_params(params);
    if (st != JL_OK) return st;
    if (T < 1) return fail(JL_ERR_INVALID_ARGUMENT, "T must be >= 1");
    if (n_seqs < 1) return fail(JL_ERR_INVALID_ARGUMENT, "n_seqs must be >= 1");
    if (!cu_seqlens && n_seqs != 1)
        return fail(JL_ERR_INVALID_ARGUMENT, "cu_seqlens == NULL requires n_seqs == 1");
    if (max_seqlen < 1 || max_seqlen > T)
        return fail(JL_ERR_INVALID_ARGUMENT, "max_seqlen must be in [1, T]");
    if (!cu_seqlens && max_seqlen != T)
        return fail(JL_ERR_INVALID_ARGUMENT, "a single sequence needs max_seqlen == T");
    if ((int64_t)n_seqs > T) return fail(JL_ERR_INVALID_ARGUMENT, "n_seqs > T");
    if (n_seqs > 65535) return fail(JL_ERR_UNSUPPORTED, "n_seqs above 65535");
    if ((int64_t)max_seqlen > 65535LL * kBM)
        return fail(JL_ERR_UNSUPPORTED, "max_seqlen above 65535 * 256");
    st = check_heads(Hq, Hkv);
    if (st != JL_OK) return st;
    st = check_dtype_d(dtype, d);
    if (st != JL_OK) return st;
    if (T + (int64_t)n_seqs * kBN >= 2147483647LL)
        return fail(JL_ERR_UNSUPPORTED, "T + 64 * n_seqs must stay below 2^31");
    if (o == q || o == k || o == v || (void*)lse == q || (k_rot_out && (k_rot_out == k || k_rot_out == q || k_rot_out == v || k_rot_out == o)))
        return fail(JL_ERR_INVALID_ARGUMENT, "outputs must not alias inputs");
    if ((uintptr_t)workspace & 255) return fail(JL_ERR_INVALID_ARGUMENT, "workspace must be 256-byte aligned");
    st = check_aligned({o, q, k, v, k_rot_out});
    if (st != JL_OK) return st;
    const int precise = dtype == JL_DTYPE_BF16 ? params->precise : 0;
    const PrefillLayout lay = prefill_layout(T, n_seqs, Hkv, d, dtype, precise);
    if (workspace_bytes < lay.total)
        return fail(JL_ERR_WORKSPACE_TOO_SMALL,
                    "workspace needs " + std::to_string(lay.total) + " bytes");

    PrefillArgs a{};
    a.q = q; a.k = k; a.v = v; a.o = o; a.lse = lse; a.k_rot_out = k_rot_out; a.ws = workspace;
    a.lay = lay;
    a.n_seqs = n_seqs; a.Hq = Hq; a.Hkv = Hkv; a.d = d; a.max_seqlen = max_seqlen; a.T = T;
    a.w_local = params->w_local; a.bifocal = params->bifocal;
    a.softmax_scale = params->softmax_scale;
    a.tab = make_rope_freq(params->rope_base, d);
    a.w_pretrained = params->w_pretrained;
    a.precise = precise;
    if (params->bifocal == 2 && dtype != JL_DTYPE_BF16)
        return fail(JL_ERR_UNSUPPORTED, "continuous interpolation (bifocal = 2) is bf16 only");

    hipStream_t s = (hipStream_t)stream;
    hipError_t e = launch_plan((int32_t*)((char*)workspace + lay.plan), cu_seqlens, n_seqs, T,
                               max_seqlen, params->w_pretrained, precise, s);
    if (e != hipSuccess) return hip_fail(e, "plan launch");
    e = launch_kv_prepass(a, dtype, s);
    if (e != hipSuccess) return hip_fail(e, "key/value pre-pass launch");
    e = dtype == JL_DTYPE_BF16 ? launch_prefill_bf16(a, s) : launch_prefill_f32(a, s);
    if (e != hipSuccess) return hip_fail(e, "prefill launch");
    return finish(s, "jl_bifocal_prefill");
}

// Unfused form: scratch for the three calls' outputs after the prefill workspace.
struct ThreeCallLayout {
    size_t oA, oB, oC, lA, lB, lC, total;
};
static ThreeCallLayout three_call_layout(const PrefillLayout& pl, int64_t T, int32_t Hq, int32_t d) {
    ThreeCallLayout L{};
    // fp32 outputs of the three calls
    const size_t ob = align256((size_t)T * Hq * d * 4), lb = align256((size_t)Hq * T * 4);
    size_t off = align256(pl.total);
    L.oA = off; off += ob;
    L.oB = off; off += ob;
    L.oC = off; off += ob;
    L.lA = off; off += lb;
    L.lB = off; off += lb;
    L.lC = off; off += lb;
    L.total = off;
    return L;
}

jl_status jl_bifocal_prefill_three_call_workspace(int64_t T, int32_t n_seqs, int32_t Hq, int32_t Hkv,
                                                  int32_t d, jl_dtype dtype, const jl_params* params,
                                                  size_t* bytes) {
    if (!bytes) return fail(JL_ERR_INVALID_ARGUMENT, "bytes is NULL");
    if (T < 1 || n_seqs < 1) return fail(JL_ERR_INVALID_ARGUMENT, "T and n_seqs must be >= 1");
    jl_status st = check_heads(Hq, Hkv);
    if (st != JL_OK) return st;
    st = check_dtype_d(dtype, d);
    if (st != JL_OK) return st;
    if (dtype != JL_DTYPE_BF16) return fail(JL_ERR_UNSUPPORTED, "the unfused form is bf16 only");
    if (params) {
        const jl_status pst = check_params(params);
        if (pst != JL_OK) return pst;
    }
    *bytes = three_call_layout(prefill_layout(T, n_seqs, Hkv, d, dtype, precise_of(params)), T, Hq,
                               d).total;
    g_err.clear();
    return JL_OK;
}

jl_status jl_bifocal_prefill_three_call(void* o, float* lse, const void* q, const void* k,
                                        const void* v, const int32_t* cu_seqlens, int32_t n_seqs,
                                        int64_t T, int32_t max_seqlen, int32_t Hq, int32_t Hkv,
                                        int32_t d, const jl_params* params, jl_dtype dtype,
                                        void* workspace, size_t workspace_bytes, void* stream) {
    if (!o || !lse || !q || !k || !v || !workspace)
        return fail(JL_ERR_INVALID_ARGUMENT, "null pointer argument");
    jl_status st = check_params(params);
    if (st != JL_OK) return st;
    if (params->bifocal != 1) return fail(JL_ERR_INVALID_ARGUMENT, "the unfused form needs bifocal = 1");
    if (T < 1) return fail(JL_ERR_INVALID_ARGUMENT, "T must be >= 1");
    if (n_seqs < 1) return fail(JL_ERR_INVALID_ARGUMENT, "n_seqs must be >= 1");
    if (!cu_seqlens && n_seqs != 1)
        return fail(JL_ERR_INVALID_ARGUMENT, "cu_seqlens == NULL requires n_seqs == 1");
    if (max_seqlen < 1 || max_seqlen > T)
        return fail(JL_ERR_INVALID_ARGUMENT, "max_seqlen must be in [1, T]");
    if (!cu_seqlens && max_seqlen != T)
        return fail(JL_ERR_INVALID_ARGUMENT, "a single sequence needs max_seqlen == T");
    if ((int64_t)n_seqs > T) return fail(JL_ERR_INVALID_ARGUMENT, "n_seqs > T");
    if (n_seqs > 65535) return fail(JL_ERR_UNSUPPORTED, "n_seqs above 65535");
    if ((int64_t)max_seqlen > 65535LL * kBM)
        return fail(JL_ERR_UNSUPPORTED, "max_seqlen above 65535 * 256");
    st = check_heads(Hq, Hkv);
    if (st != JL_OK) return st;
    st = check_dtype_d(dtype, d);
    if (st != JL_OK) return st;
    if (dtype != JL_DTYPE_BF16) return fail(JL_ERR_UNSUPPORTED, "the unfused form is bf16 only");
    if (T + (int64_t)n_seqs * kBN >= 2147483647LL)
        return fail(JL_ERR_UNSUPPORTED, "T + 64 * n_seqs must stay below 2^31");
    if ((unsigned long long)T > 2147483647ULL) return fail(JL_ERR_UNSUPPORTED, "T above 2^31 - 1");
    if (o == q || o == k || o == v || (void*)lse == q)
        return fail(JL_ERR_INVALID_ARGUMENT, "outputs must not alias inputs");
    if ((uintptr_t)workspace & 255) return fail(JL_ERR_INVALID_ARGUMENT, "workspace must be 256-byte aligned");
    st = check_aligned({o, q, k, v});
    if (st != JL_OK) return st;
    const PrefillLayout lay = prefill_layout(T, n_seqs, Hkv, d, dtype, params->precise);
    const ThreeCallLayout tl = three_call_layout(lay, T, Hq, d);
    if (workspace_bytes < tl.total)
        return fail(JL_ERR_WORKSPACE_TOO_SMALL,
                    "workspace needs " + std::to_string(tl.total) + " bytes");

    char* ws = (char*)workspace;
    PrefillArgs a{};
    a.q = q; a.k = k; a.v = v; a.k_rot_out = nullptr; a.ws = workspace; a.lay = lay;
    a.n_seqs = n_seqs; a.Hq = Hq; a.Hkv = Hkv; a.d = d; a.max_seqlen = max_seqlen; a.T = T;
    a.w_local = params->w_local; a.bifocal = 1;
    a.softmax_scale = params->softmax_scale;
    a.tab = make_rope_freq(params->rope_base, d);
    a.precise = params->precise;

    hipStream_t s = (hipStream_t)stream;
    hipError_t e = launch_plan((int32_t*)(ws + lay.plan), cu_seqlens, n_seqs, T, max_seqlen,
                               params->w_pretrained, params->precise, s);
    if (e != hipSuccess) return hip_fail(e, "plan launch");
    e = launch_kv_prepass(a, dtype, s);
    if (e != hipSuccess) return hip_fail(e, "key/value pre-pass launch");
    const size_t oofs[3] = {tl.oB, tl.oA, tl.oC}, lofs[3] = {tl.lB, tl.lA, tl.lC};
    a.o_f32 = 1;
    for (int c = 0; c < 3; ++c) {  // modes 1 (B), 2 (A), 3 (C)
        a.mode = c + 1;
        a.o = ws + oofs[c];
        a.lse = (float*)(ws + lofs[c]);
        e = launch_prefill_bf16(a, s);
        if (e != hipSuccess) return hip_fail(e, "prefill launch");
    }
    e = launch_three_call_merge((const float*)(ws + tl.oA), (const float*)(ws + tl.oB),
                                (const float*)(ws + tl.oC), (const float*)(ws + tl.lA),
                                (const float*)(ws + tl.lB), (const float*)(ws + tl.lC), o, lse, T,
                                Hq, d, 1, T, s);
    if (e != hipSuccess) return hip_fail(e, "merge launch");
    return finish(s, "jl_bifocal_prefill_three_call");
}

jl_status jl_bifocal_decode_workspace(int32_t batch, int32_t max_seqlen_k, int32_t Hq,
                                      int32_t Hkv, int32_t d, jl_dtype dtype, size_t* bytes) {
    if (!bytes) return fail(JL_ERR_INVALID_ARGUMENT, "bytes is NULL");
    if (batch < 1 || max_seqlen_k < 1)
        return fail(JL_ERR_INVALID_ARGUMENT, "batch and max_seqlen_k must be >= 1");
    jl_status st = check_heads(Hq, Hkv);
    if (st != JL_OK) return st;
    st = check_dtype_d(dtype, d);
    if (st != JL_OK) return st;
    *bytes = decode_layout(batch, max_seqlen_k, Hq, Hkv, d, dtype).total;
    g_err.clear();
    return JL_OK;
}

// Shared body of the four decode entry points: flat or paged cache, bf16
// (or f32) or fp8 codes.  Every check runs on the host before any launch.
struct DecodeCall {
    void* o;
    float* lse;
    const void* q;
    const void* kc;
    const void* vc;
    const int32_t* seqlens_k;
    int32_t batch, max_seqlen_k;
    int64_t S_max;  // flat cache
    const int32_t* block_table;  // paged cache (else nullptr)
    int32_t page_size;
    int64_t n_pages;
    int32_t bt_stride;
    int32_t fp8;
    const float* k_scale;
    const float* v_scale;
    int32_t Hq, Hkv, d;
};

static jl_status scratch_of_device(void* stream, void** out);

// static_scratch: `workspace` is a placeholder; once every check has passed
// (the size against workspace_bytes included) the library's own scratch
// array of the current device takes its place.
static jl_status decode_impl(const DecodeCall& c, const jl_params* params, jl_dtype dtype,
                             void* workspace, size_t workspace_bytes, void* stream,
                             const char* where, bool static_scratch = false) {
    if (!c.o || !c.lse || !c.q || !c.kc || !c.vc || !c.seqlens_k || !workspace)
        return fail(JL_ERR_INVALID_ARGUMENT, "null pointer argument");
    jl_status st = check_params(params);
    if (st != JL_OK) return st;
    if (c.batch < 1 || c.max_seqlen_k < 1)
        return fail(JL_ERR_INVALID_ARGUMENT, "batch and max_seqlen_k must be >= 1");
    if (c.batch > 65535) return fail(JL_ERR_UNSUPPORTED, "batch above 65535");
    const bool paged = c.block_table != nullptr;
    if (paged) {
        if (c.page_size < 16 || c.page_size > 65536 || (c.page_size & (c.page_size - 1)))
            return fail(JL_ERR_INVALID_ARGUMENT, "page_size must be a power of two in [16, 65536]");
        if (c.n_pages < 1) return fail(JL_ERR_INVALID_ARGUMENT, "n_pages must be >= 1");
        if ((int64_t)c.bt_stride * c.page_size < c.max_seqlen_k)
            return fail(JL_ERR_INVALID_ARGUMENT, "bt_stride * page_size < max_seqlen_k");
    } else if (c.S_max < c.max_seqlen_k) {
        return fail(JL_ERR_INVALID_ARGUMENT, "S_max < max_seqlen_k");
    }
    st = check_heads(c.Hq, c.Hkv);
    if (st != JL_OK) return st;
    if (c.Hq / c.Hkv > 16) return fail(JL_ERR_UNSUPPORTED, "decode supports Hq / Hkv <= 16");
    st = check_dtype_d(dtype, c.d);
    if (st != JL_OK) return st;
    if ((paged || c.fp8 || params->bifocal == 2) && dtype != JL_DTYPE_BF16)
        return fail(JL_ERR_UNSUPPORTED,
                    "paged, fp8 and continuous-interpolation decode take bf16 queries");
    if (paged) {
        if (c.n_pages > (1LL << 40) / ((int64_t)c.page_size * c.Hkv * c.d))
            return fail(JL_ERR_INVALID_ARGUMENT, "page pool too large");
    } else if (c.S_max > (1LL << 40) / ((int64_t)c.batch * c.Hkv * c.d)) {
        return fail(JL_ERR_INVALID_ARGUMENT, "cache too large");
    }
    if (c.o == c.q || c.o == c.kc || c.o == c.vc)
        return fail(JL_ERR_INVALID_ARGUMENT, "outputs must not alias inputs");
    if ((uintptr_t)workspace & 255) return fail(JL_ERR_INVALID_ARGUMENT, "workspace must be 256-byte aligned");
    {
        const jl_status ast = check_aligned({c.o, c.q, c.kc, c.vc});
        if (ast != JL_OK) return ast;
    }
    const DecodeLayout lay = decode_layout(c.batch, c.max_seqlen_k, c.Hq, c.Hkv, c.d, dtype);
    if (workspace_bytes < lay.total)
        return fail(JL_ERR_WORKSPACE_TOO_SMALL,
                    static_scratch
                        ? "these sizes need " + std::to_string(lay.total) +
                              " bytes of scratch; the library's static scratch holds " +
                              std::to_string(workspace_bytes) + " (use jl_bifocal_decode)"
                        : "workspace needs " + std::to_string(lay.total) + " bytes");
    DecodeArgs a{};
    a.q = c.q; a.kc = c.kc; a.vc = c.vc; a.o = c.o; a.lse = c.lse; a.seqlens = c.seqlens_k;
    a.ws = workspace; a.lay = lay;
    a.B = c.batch; a.max_seqlen_k = c.max_seqlen_k; a.Hq = c.Hq; a.Hkv = c.Hkv; a.d = c.d;
    a.S_max = paged ? 0 : c.S_max;
    a.w_pretrained = params->w_pretrained; a.w_local = params->w_local;
    a.bifocal = params->bifocal; a.softmax_scale = params->softmax_scale;
    a.tab = make_rope_freq(params->rope_base, c.d);
    if (paged) {
        a.block_table = c.block_table;
        int shift = 0;
        while ((1 << shift) < c.page_size) ++shift;
        a.page_shift = shift; a.bt_stride = c.bt_stride; a.n_pages = c.n_pages;
    }
    a.fp8 = c.fp8; a.k_scale = c.k_scale; a.v_scale = c.v_scale;
    // split-precision remote keys: bf16 caches (fp32 caches are scored in
    // split bf16 anyway; an fp8 cache's own rounding is far coarser)
    if (params->precise && c.fp8)
        return fail(JL_ERR_UNSUPPORTED, "split precision (precise = 1) is not offered for fp8 caches");
    a.precise = dtype == JL_DTYPE_BF16 ? params->precise : 0;
    a.ilv = dtype == JL_DTYPE_BF16 &&
            decode_interleave(paged, c.Hq, c.Hkv, c.d, c.max_seqlen_k, c.fp8 ? 1 : 2);
    // Flat bf16 caches of 64K keys and more run faster on fewer, longer
    // workgroups (192 against 256 at L = 131072: fewer partials to write and
    // merge, fewer table prologues per byte); shorter caches and fp8 caches
    // keep 256.  Fewer splits need less workspace than the size checked above.
    if (a.ilv && !c.fp8 && c.max_seqlen_k >= 65536)
        a.lay = decode_layout(c.batch, c.max_seqlen_k, c.Hq, c.Hkv, c.d, dtype, kDecodeLongTargetWG);
    if (static_scratch) {
        const jl_status sst = scratch_of_device(stream, &a.ws);
        if (sst != JL_OK) return sst;
    }
    hipStream_t s = (hipStream_t)stream;
    hipError_t e = launch_decode(a, dtype, s);
    if (e != hipSuccess) return hip_fail(e, "decode launch");
    return finish(s, where);
}

// The unfused decode: the cache turned to remapped RoPE, the three calls'
// fp32 outputs and LSEs, and one decode workspace the calls take in turn.
struct DecodeThreeLayout {
    DecodeLayout full, win;  // call B (all keys); calls A and C (the local window)
    size_t kr, oA, oB, oC, lA, lB, lC, dec, total;
};
static DecodeThreeLayout decode_three_layout(int32_t B, int32_t max_seqlen_k, int32_t Hq,
                                             int32_t Hkv, int32_t d, int32_t w_local) {
    DecodeThreeLayout L{};
    L.full = decode_layout(B, max_seqlen_k, Hq, Hkv, d, JL_DTYPE_BF16);
    const int32_t wk = w_local < 1 ? 1 : (w_local < max_seqlen_k ? w_local : max_seqlen_k);
    L.win = decode_layout(B, wk, Hq, Hkv, d, JL_DTYPE_BF16);
    const size_t ob = align256((size_t)B * Hq * d * 4), lb = align256((size_t)B * Hq * 4);
    size_t off = 0;
    L.kr = off; off = align256(off + (size_t)B * max_seqlen_k * Hkv * d * 2);
    L.oA = off; off += ob;
    L.oB = off; off += ob;
    L.oC = off; off += ob;
    L.lA = off; off += lb;
    L.lB = off; off += lb;
    L.lC = off; off += lb;
    L.dec = off;
    off += L.full.total > L.win.total ? L.full.total : L.win.total;
    L.total = align256(off);
    return L;
}

jl_status jl_bifocal_decode_three_call_workspace(int32_t batch, int32_t max_seqlen_k, int32_t Hq,
                                                 int32_t Hkv, int32_t d, jl_dtype dtype,
                                                 const jl_params* params, size_t* bytes) {
    if (!bytes) return fail(JL_ERR_INVALID_ARGUMENT, "bytes is NULL");
    jl_status st = check_params(params);
    if (st != JL_OK) return st;
    if (batch < 1 || max_seqlen_k < 1)
        return fail(JL_ERR_INVALID_ARGUMENT, "batch and max_seqlen_k must be >= 1");
    st = check_heads(Hq, Hkv);
    if (st != JL_OK) return st;
    st = check_dtype_d(dtype, d);
    if (st != JL_OK) return st;
    if (dtype != JL_DTYPE_BF16) return fail(JL_ERR_UNSUPPORTED, "the unfused decode is bf16 only");
    *bytes = decode_three_layout(batch, max_seqlen_k, Hq, Hkv, d, params->w_local).total;
    g_err.clear();
    return JL_OK;
}

jl_status jl_bifocal_decode_three_call(void* o, float* lse, const void* q, const void* k_cache,
                                       const void* v_cache, const int32_t* seqlens_k,
                                       int32_t batch, int32_t max_seqlen_k, int64_t S_max,
                                       int32_t Hq, int32_t Hkv, int32_t d,
                                       const jl_params* params, jl_dtype dtype, void* workspace,
                                       size_t workspace_bytes, void* stream) {
    if (!o || !lse || !q || !k_cache || !v_cache || !seqlens_k || !workspace)
        return fail(JL_ERR_INVALID_ARGUMENT, "null pointer argument");
    jl_status st = check_params(params);
    if (st != JL_OK) return st;
    if (params->bifocal != 1) return fail(JL_ERR_INVALID_ARGUMENT, "the unfused form needs bifocal = 1");
    if (params->precise) return fail(JL_ERR_UNSUPPORTED, "the unfused decode has no split-precision mode");
    if (batch < 1 || max_seqlen_k < 1)
        return fail(JL_ERR_INVALID_ARGUMENT, "batch and max_seqlen_k must be >= 1");
    if (batch > 65535) return fail(JL_ERR_UNSUPPORTED, "batch above 65535");
    if (S_max < max_seqlen_k) return fail(JL_ERR_INVALID_ARGUMENT, "S_max < max_seqlen_k");
    st = check_heads(Hq, Hkv);
    if (st != JL_OK) return st;
    if (Hq / Hkv > 16) return fail(JL_ERR_UNSUPPORTED, "decode supports Hq / Hkv <= 16");
    st = check_dtype_d(dtype, d);
    if (st != JL_OK) return st;
    if (dtype != JL_DTYPE_BF16) return fail(JL_ERR_UNSUPPORTED, "the unfused decode is bf16 only");
    if (S_max > (1LL << 40) / ((int64_t)batch * Hkv * d))
        return fail(JL_ERR_INVALID_ARGUMENT, "cache too large");
    if (o == q || o == k_cache || o == v_cache)
        return fail(JL_ERR_INVALID_ARGUMENT, "outputs must not alias inputs");
    if ((uintptr_t)workspace & 255) return fail(JL_ERR_INVALID_ARGUMENT, "workspace must be 256-byte aligned");
    st = check_aligned({o, q, k_cache, v_cache});
    if (st != JL_OK) return st;
    const DecodeThreeLayout tl = decode_three_layout(batch, max_seqlen_k, Hq, Hkv, d, params->w_local);
    if (workspace_bytes < tl.total)
        return fail(JL_ERR_WORKSPACE_TOO_SMALL, "workspace needs " + std::to_string(tl.total) + " bytes");
    char* ws = (char*)workspace;
    DecodeArgs a{};
    a.q = q; a.seqlens = seqlens_k; a.B = batch; a.max_seqlen_k = max_seqlen_k;
    a.Hq = Hq; a.Hkv = Hkv; a.d = d;
    a.w_pretrained = params->w_pretrained; a.w_local = params->w_local;
    a.bifocal = 0;  // each call is a plain attention call over its keys
    a.softmax_scale = params->softmax_scale;
    a.tab = make_rope_freq(params->rope_base, d);
    a.ws = ws + tl.dec;
    a.o_f32 = 1;
    a.ilv = decode_interleave(false, Hq, Hkv, d, max_seqlen_k, 2);
    hipStream_t s = (hipStream_t)stream;
    hipError_t e = launch_cache_remap(ws + tl.kr, k_cache, seqlens_k, batch, max_seqlen_k, S_max,
                                      Hkv, d, params->w_pretrained, a.tab, s);
    if (e != hipSuccess) return hip_fail(e, "cache remap launch");
    struct Call {
        const void* kc;
        int64_t S_max;
        int32_t q_remap, window;
        size_t o, l;
    };
    const Call calls[3] = {
        {ws + tl.kr, max_seqlen_k, 1, 0, tl.oB, tl.lB},  // B: every key, remapped RoPE
        {k_cache, S_max, 0, 1, tl.oA, tl.lA},           // A: the local window, standard RoPE
        {ws + tl.kr, max_seqlen_k, 1, 1, tl.oC, tl.lC},  // C: the local window, remapped RoPE
    };
    for (const Call& c : calls) {
        // keys from the caller's cache or the remapped copy, values always
        // from the caller's cache (rows per sequence S_max)
        a.kc = c.kc; a.vc = v_cache; a.S_max = S_max; a.S_max_k = c.S_max;
        a.q_remap = c.q_remap; a.window = c.window;
        a.lay = c.window ? tl.win : tl.full;
        a.o = ws + c.o; a.lse = (float*)(ws + c.l);
        e = launch_decode(a, JL_DTYPE_BF16, s);
        if (e != hipSuccess) return hip_fail(e, "decode launch");
    }
    e = launch_three_call_merge((const float*)(ws + tl.oA), (const float*)(ws + tl.oB),
                                (const float*)(ws + tl.oC), (const float*)(ws + tl.lA),
                                (const float*)(ws + tl.lB), (const float*)(ws + tl.lC), o, lse,
                                batch, Hq, d, Hq, 1, s);
    if (e != hipSuccess) return hip_fail(e, "merge launch");
    return finish(s, "jl_bifocal_decode_three_call");
}

jl_status jl_bifocal_decode(void* o, float* lse, const void* q, const void* k_cache,
                            const void* v_cache, const int32_t* seqlens_k, int32_t batch,
                            int32_t max_seqlen_k, int64_t S_max, int32_t Hq, int32_t Hkv,
                            int32_t d, const jl_params* params, jl_dtype dtype, void* workspace,
                            size_t workspace_bytes, void* stream) {
    DecodeCall c{o, lse, q, k_cache, v_cache, seqlens_k, batch, max_seqlen_k, S_max,
                 nullptr, 0, 0, 0, 0, nullptr, nullptr, Hq, Hkv, d};
    return decode_impl(c, params, dtype, workspace, workspace_bytes, stream, "jl_bifocal_decode");
}

// ---------------------------------------------------------------------------
// Decode with library-owned scratch, for callers that cannot allocate.  The
// split partials live in a file-scope device array; each device holds its
// own copy, whose address is looked up once per device.  Every call writes
// each partial it later reads, so nothing in the array needs clearing.
constexpr size_t kDecodeScratchBytes = (size_t)32 << 20;
static __device__ __align__(256) char scratch[kDecodeScratchBytes];
static std::mutex g_scratch_mu;
constexpr int kMaxDevices = 64;
static void* g_scratch_ptr[kMaxDevices];

static jl_status scratch_of_device(void* stream, void** out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
    if (stream) {
        hipDevice_t sdev = 0;
        e = hipStreamGetDevice((hipStream_t)stream, &sdev);
        if (e != hipSuccess) return hip_fail(e, "hipStreamGetDevice");
        if ((int)sdev != dev)
            return fail(JL_ERR_INVALID_ARGUMENT, "the stream belongs to another device than the current one");
    }
    if (dev < 0 || dev >= kMaxDevices) return fail(JL_ERR_UNSUPPORTED, "device index above 63");
    std::lock_guard<std::mutex> lk(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress(scratch)");
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return JL_OK;
}

jl_status jl_bifocal_decode_noalloc(void* o, float* lse, const void* q, const void* k_cache,
                                    const void* v_cache, const int32_t* seqlens_k, int32_t batch,
                                    int32_t max_seqlen_k, int64_t S_max, int32_t Hq, int32_t Hkv,
                                    int32_t d, const jl_params* params, jl_dtype dtype,
                                    void* stream) {
    DecodeCall c{o, lse, q, k_cache, v_cache, seqlens_k, batch, max_seqlen_k, S_max,
                 nullptr, 0, 0, 0, 0, nullptr, nullptr, Hq, Hkv, d};
    // a placeholder that passes the null and alignment checks; replaced by
    // the device's scratch once the sizes are known to fit
    return decode_impl(c, params, dtype, (void*)(uintptr_t)256, kDecodeScratchBytes, stream,
                       "jl_bifocal_decode_noalloc", true);
}

jl_status jl_bifocal_decode_paged(void* o, float* lse, const void* q, const void* k_pages,
                                  const void* v_pages, const int32_t* block_table,
                                  const int32_t* seqlens_k, int32_t batch, int32_t max_seqlen_k,
                                  int32_t page_size, int64_t n_pages, int32_t bt_stride, int32_t Hq,
                                  int32_t Hkv, int32_t d, const jl_params* params, jl_dtype dtype,
                                  void* workspace, size_t workspace_bytes, void* stream) {
    if (!block_table) return fail(JL_ERR_INVALID_ARGUMENT, "null pointer argument");
    DecodeCall c{o, lse, q, k_pages, v_pages, seqlens_k, batch, max_seqlen_k, 0,
                 block_table, page_size, n_pages, bt_stride, 0, nullptr, nullptr, Hq, Hkv, d};
    return decode_impl(c, params, dtype, workspace, workspace_bytes, stream,
                       "jl_bifocal_decode_paged");
}

jl_status jl_bifocal_decode_fp8(void* o, float* lse, const void* q, const void* k_cache,
                                const void* v_cache, const float* k_scale, const float* v_scale,
                                const int32_t* seqlens_k, int32_t batch, int32_t max_seqlen_k,
                                int64_t S_max, int32_t Hq, int32_t Hkv, int32_t d,
                                const jl_params* params, void* workspace, size_t workspace_bytes,
                                void* stream) {
    if (!k_scale || !v_scale) return fail(JL_ERR_INVALID_ARGUMENT, "null pointer argument");
    DecodeCall c{o, lse, q, k_cache, v_cache, seqlens_k, batch, max_seqlen_k, S_max,
                 nullptr, 0, 0, 0, 1, k_scale, v_scale, Hq, Hkv, d};
    return decode_impl(c, params, JL_DTYPE_BF16, workspace, workspace_bytes, stream,
                       "jl_bifocal_decode_fp8");
}

jl_status jl_bifocal_decode_fp8_paged(void* o, float* lse, const void* q, const void* k_pages,
                                      const void* v_pages, const float* k_scale,
                                      const float* v_scale, const int32_t* block_table,
                                      const int32_t* seqlens_k, int32_t batch,
                                      int32_t max_seqlen_k, int32_t page_size, int64_t n_pages,
                                      int32_t bt_stride, int32_t Hq, int32_t Hkv, int32_t d,
                                      const jl_params* params, void* workspace,
                                      size_t workspace_bytes, void* stream) {
    if (!k_scale || !v_scale || !block_table)
        return fail(JL_ERR_INVALID_ARGUMENT, "null pointer argument");
    DecodeCall c{o, lse, q, k_pages, v_pages, seqlens_k, batch, max_seqlen_k, 0,
                 block_table, page_size, n_pages, bt_stride, 1, k_scale, v_scale, Hq, Hkv, d};
    return decode_impl(c, params, JL_DTYPE_BF16, workspace, workspace_bytes, stream,
                       "jl_bifocal_decode_fp8_paged");
}

jl_status jl_kv_quantize_fp8(void* out, const void* x, const float* scale, int64_t ntok,
                             int32_t H, int32_t d, void* stream) {
    if (!out || !x || !scale) return fail(JL_ERR_INVALID_ARGUMENT, "null pointer argument");
    if (ntok < 1 || H < 1) return fail(JL_ERR_INVALID_ARGUMENT, "ntok and H must be >= 1");
    if (d < 8 || d % 8) return fail(JL_ERR_INVALID_ARGUMENT, "d must be a positive multiple of 8");
    if (ntok > (1LL << 40) / ((int64_t)H * d)) return fail(JL_ERR_INVALID_ARGUMENT, "too many elements");
    if (((uintptr_t)out & 7) || ((uintptr_t)x & 15))
        return fail(JL_ERR_INVALID_ARGUMENT, "out must be 8-byte and x 16-byte aligned");
    if (out == x) return fail(JL_ERR_INVALID_ARGUMENT, "outputs must not alias inputs");
    hipStream_t s = (hipStream_t)stream;
    hipError_t e = launch_e4m3_quant((uint8_t*)out, x, scale, ntok, H, d, s);
    if (e != hipSuccess) return hip_fail(e, "quantize launch");
    return finish(s, "jl_kv_quantize_fp8");
}

// ---------------------------------------------------------------------------
// Chunked prefill against a cache: the prefill workspace for batch sequences
// of up to max_seqlen_k keys each.
static jl_status chunk_sizes_ok(int32_t batch, int32_t max_seqlen_k) {
    if (batch < 1 || max_seqlen_k < 1)
        return fail(JL_ERR_INVALID_ARGUMENT, "batch and max_seqlen_k must be >= 1");
    if (batch > 65535) return fail(JL_ERR_UNSUPPORTED, "batch above 65535");
    if ((int64_t)batch * max_seqlen_k + (int64_t)batch * kBN >= 2147483647LL)
        return fail(JL_ERR_UNSUPPORTED, "batch * (max_seqlen_k + 64) must stay below 2^31");
    return JL_OK;
}

// Workspace of a chunk call: the prefill layout for the cache keys (each
// sequence a fixed stretch of max_seqlen_k keys), the record of the images it
// holds, then the key-split partials.  The images and the record sit at
// offsets that depend on batch, max_seqlen_k, Hkv, d and the precise flag
// only, so that calls with other chunk sizes find them.  A call whose
// main-rows grid holds fewer than kChunkTargetWgs workgroups (one per compute
// unit) splits each row block's key tiles in up to kChunkMaxSplit shares; the
// partials are sized for the most shares Tq query rows can need (every row
// block holds at most 256 of them).
constexpr int kChunkTargetWgs = 256;  // one workgroup per compute unit
static int chunk_split_bound(int64_t wgs) {
    if (wgs < 1) wgs = 1;
    const int64_t k = (kChunkTargetWgs + wgs - 1) / wgs;
    return (int)(k < 1 ? 1 : (k > kChunkMaxSplit ? kChunkMaxSplit : k));
}
struct ChunkLayout {
    PrefillLayout pl;
    int kmax;
    size_t state, part_o, part_ml, total;
};
static ChunkLayout chunk_layout(int64_t Tq, int32_t batch, int32_t max_seqlen_k, int32_t Hq,
                                int32_t Hkv, int32_t d, int precise) {
    ChunkLayout L{};
    L.pl = prefill_layout((int64_t)batch * max_seqlen_k, batch, Hkv, d, JL_DTYPE_BF16, precise);
    // split-precision calls run every row in one kernel without key shares
    L.kmax = precise ? 1 : chunk_split_bound((int64_t)Hq * ((Tq + kBM - 1) / kBM));
    size_t off = align256(L.pl.total);
    L.state = off;
    off = align256(off + image_state_bytes(batch));
    if (L.kmax > 1) {
        L.part_o = off;
        off = align256(off + (size_t)L.kmax * Tq * Hq * d * sizeof(float));
        L.part_ml = off;
        off = align256(off + (size_t)L.kmax * Hq * Tq * 2 * sizeof(float));
    }
    L.total = off;
    return L;
}

jl_status jl_bifocal_prefill_chunk_workspace(int64_t Tq, int32_t batch, int32_t max_seqlen_k,
                                             int32_t Hq, int32_t Hkv, int32_t d, jl_dtype dtype,
                                             const jl_params* params, size_t* bytes) {
    if (!bytes) return fail(JL_ERR_INVALID_ARGUMENT, "bytes is NULL");
    if (Tq < 1 || Tq >= 2147483647LL) return fail(JL_ERR_INVALID_ARGUMENT, "Tq must be in [1, 2^31)");
    jl_status st = chunk_sizes_ok(batch, max_seqlen_k);
    if (st != JL_OK) return st;
    st = check_heads(Hq, Hkv);
    if (st != JL_OK) return st;
    st = check_dtype_d(dtype, d);
    if (st != JL_OK) return st;
    if (dtype != JL_DTYPE_BF16) return fail(JL_ERR_UNSUPPORTED, "chunked prefill is bf16 only");
    if (params) {
        const jl_status pst = check_params(params);
        if (pst != JL_OK) return pst;
    }
    *bytes = chunk_layout(Tq, batch, max_seqlen_k, Hq, Hkv, d, precise_of(params)).total;
    g_err.clear();
    return JL_OK;
}

// FNV-1a over everything a chunk call's key/value images depend on besides
// the cache rows and the lengths: the caches (and block table) by address,
// their geometry, the layout's sizes and the parameters the rotations use.
static uint64_t image_fingerprint(const PrefillArgs& a, const jl_params* p) {
    uint64_t h = 0xcbf29ce484222325ULL;
    auto mix = [&](const void* x, size_t n) {
        const unsigned char* c = (const unsigned char*)x;
        for (size_t i = 0; i < n; ++i) h = (h ^ c[i]) * 0x100000001b3ULL;
    };
    const uintptr_t ptrs[3] = {(uintptr_t)a.k, (uintptr_t)a.v, (uintptr_t)a.block_table};
    const int64_t ints[10] = {a.S_max, a.page_shift, a.n_pages, a.bt_stride, a.Hkv, a.d,
                              a.n_seqs, a.max_seqlen_k, p->bifocal, p->precise};
    mix(ptrs, sizeof(ptrs));
    mix(ints, sizeof(ints));
    mix(&p->rope_base, sizeof(p->rope_base));
    mix(&p->w_pretrained, sizeof(p->w_pretrained));
    return h;
}

// Shared checks and launches of the flat and paged chunk calls.
static jl_status chunk_call(PrefillArgs& a, const int32_t* cu_seqlens_q,
                            const int32_t* seqlens_k, const jl_params* params, jl_dtype dtype,
                            void* workspace, size_t workspace_bytes, void* stream,
                            const char* where) {
    if (!a.o || !a.lse || !a.q || !a.k || !a.v || !seqlens_k || !workspace)
        return fail(JL_ERR_INVALID_ARGUMENT, "null pointer argument");
    jl_status st = check_params(params);
    if (st != JL_OK) return st;
    st = chunk_sizes_ok(a.n_seqs, a.max_seqlen_k);
    if (st != JL_OK) return st;
    if (a.T < 1) return fail(JL_ERR_INVALID_ARGUMENT, "Tq must be >= 1");
    if (!cu_seqlens_q && a.n_seqs != 1)
        return fail(JL_ERR_INVALID_ARGUMENT, "cu_seqlens_q == NULL requires batch == 1");
    if (a.max_seqlen < 1 || a.max_seqlen > a.T || a.max_seqlen > a.max_seqlen_k)
        return fail(JL_ERR_INVALID_ARGUMENT, "max_seqlen_q must be in [1, min(Tq, max_seqlen_k)]");
    if (!cu_seqlens_q && a.max_seqlen != a.T)
        return fail(JL_ERR_INVALID_ARGUMENT, "a single chunk needs max_seqlen_q == Tq");
    if (a.T >= 2147483647LL) return fail(JL_ERR_UNSUPPORTED, "Tq must stay below 2^31");
    st = check_heads(a.Hq, a.Hkv);
    if (st != JL_OK) return st;
    st = check_dtype_d(dtype, a.d);
    if (st != JL_OK) return st;
    if (dtype != JL_DTYPE_BF16) return fail(JL_ERR_UNSUPPORTED, "chunked prefill is bf16 only");
    if (a.o == a.q || a.o == a.k || a.o == a.v || (const void*)a.lse == a.q)
        return fail(JL_ERR_INVALID_ARGUMENT, "outputs must not alias inputs");
    if ((uintptr_t)workspace & 255) return fail(JL_ERR_INVALID_ARGUMENT, "workspace must be 256-byte aligned");
    st = check_aligned({a.o, a.q, a.k, a.v});
    if (st != JL_OK) return st;
    const ChunkLayout cl = chunk_layout(a.T, a.n_seqs, a.max_seqlen_k, a.Hq, a.Hkv, a.d,
                                        params->precise);
    const PrefillLayout& lay = cl.pl;
    if (workspace_bytes < cl.total)
        return fail(JL_ERR_WORKSPACE_TOO_SMALL,
                    "workspace needs " + std::to_string(cl.total) + " bytes");
    a.ws = workspace;
    a.lay = lay;
    a.chunked = 1;
    // key split of the main rows: the launcher's row-block count per sequence
    {
        int64_t rb = (a.max_seqlen + kBM - 1) / kBM + 1;
        const int64_t key_rb = (a.max_seqlen_k + kBM - 1) / kBM;
        rb = rb < key_rb ? rb : key_rb;
        int k = chunk_split_bound((int64_t)a.Hq * a.n_seqs * rb);
        a.ksplit = k < cl.kmax ? k : cl.kmax;
        if (a.ksplit > 1) {
            a.part_o = (float*)((char*)workspace + cl.part_o);
            a.part_ml = (float2*)((char*)workspace + cl.part_ml);
        }
    }
    a.w_local = params->w_local; a.bifocal = params->bifocal;
    a.softmax_scale = params->softmax_scale;
    a.tab = make_rope_freq(params->rope_base, a.d);
    a.w_pretrained = params->w_pretrained;
    a.precise = params->precise;
    hipStream_t s = (hipStream_t)stream;
    // the plan also rewrites the image record; the pre-pass launched next
    // builds what the record then claims
    hipError_t e = launch_plan_chunk((int32_t*)((char*)workspace + lay.plan),
                                     (char*)workspace + cl.state, image_fingerprint(a, params),
                                     params->reuse_images, cu_seqlens_q, seqlens_k, a.n_seqs, a.T,
                                     a.max_seqlen, a.max_seqlen_k, params->w_pretrained,
                                     params->precise, params->bifocal, s);
    if (e != hipSuccess) return hip_fail(e, "plan launch");
    e = launch_kv_prepass(a, dtype, s);
    if (e != hipSuccess) return hip_fail(e, "key/value pre-pass launch");
    e = launch_prefill_bf16(a, s);
    if (e != hipSuccess) return hip_fail(e, "prefill launch");
    if (a.ksplit > 1) {
        e = launch_chunk_merge(a, s);
        if (e != hipSuccess) return hip_fail(e, "chunk merge launch");
    }
    return finish(s, where);
}

jl_status jl_bifocal_prefill_chunk(void* o, float* lse, const void* q,
                                   const int32_t* cu_seqlens_q, int64_t Tq, int32_t max_seqlen_q,
                                   const void* k_cache, const void* v_cache,
                                   const int32_t* seqlens_k, int32_t batch,
                                   int32_t max_seqlen_k, int64_t S_max, int32_t Hq, int32_t Hkv,
                                   int32_t d, const jl_params* params, jl_dtype dtype,
                                   void* workspace, size_t workspace_bytes, void* stream) {
    if (S_max < max_seqlen_k || S_max < 1)
        return fail(JL_ERR_INVALID_ARGUMENT, "S_max must be >= max_seqlen_k");
    PrefillArgs a{};
    a.q = q; a.k = k_cache; a.v = v_cache; a.o = o; a.lse = lse;
    a.n_seqs = batch; a.Hq = Hq; a.Hkv = Hkv; a.d = d; a.max_seqlen = max_seqlen_q; a.T = Tq;
    a.max_seqlen_k = max_seqlen_k; a.S_max = S_max;
    return chunk_call(a, cu_seqlens_q, seqlens_k, params, dtype, workspace, workspace_bytes,
                      stream, "jl_bifocal_prefill_chunk");
}

jl_status jl_bifocal_prefill_chunk_paged(void* o, float* lse, const void* q,
                                         const int32_t* cu_seqlens_q, int64_t Tq,
                                         int32_t max_seqlen_q, const void* k_pages,
                                         const void* v_pages, const int32_t* block_table,
                                         const int32_t* seqlens_k, int32_t batch,
                                         int32_t max_seqlen_k, int32_t page_size,
                                         int64_t n_pages, int32_t bt_stride, int32_t Hq,
                                         int32_t Hkv, int32_t d, const jl_params* params,
                                         jl_dtype dtype, void* workspace,
                                         size_t workspace_bytes, void* stream) {
    if (!block_table) return fail(JL_ERR_INVALID_ARGUMENT, "null pointer argument");
    if (page_size < 16 || page_size > 65536 || (page_size & (page_size - 1)))
        return fail(JL_ERR_INVALID_ARGUMENT, "page_size must be a power of two in [16, 65536]");
    if (n_pages < 1) return fail(JL_ERR_INVALID_ARGUMENT, "n_pages must be >= 1");
    if ((int64_t)bt_stride * page_size < max_seqlen_k)
        return fail(JL_ERR_INVALID_ARGUMENT, "bt_stride * page_size < max_seqlen_k");
    if (Hkv >= 1 && d >= 1 && n_pages > (1LL << 40) / ((int64_t)page_size * Hkv * d))
        return fail(JL_ERR_INVALID_ARGUMENT, "page pool too large");
    PrefillArgs a{};
    a.q = q; a.k = k_pages; a.v = v_pages; a.o = o; a.lse = lse;
    a.n_seqs = batch; a.Hq = Hq; a.Hkv = Hkv; a.d = d; a.max_seqlen = max_seqlen_q; a.T = Tq;
    a.max_seqlen_k = max_seqlen_k; a.S_max = 0;
    a.block_table = block_table;
    int shift = 0;
    while ((1 << shift) < page_size) ++shift;
    a.page_shift = shift; a.bt_stride = bt_stride; a.n_pages = (int32_t)n_pages;
    return chunk_call(a, cu_seqlens_q, seqlens_k, params, dtype, workspace, workspace_bytes,
                      stream, "jl_bifocal_prefill_chunk_paged");
}

jl_status jl_debug_index_math(int64_t L, int32_t w_pretrained, int32_t w_local, int32_t bifocal,
                              int32_t bm, int32_t bn, int32_t* G_out, int32_t* f_out,
                              uint8_t* band_out, uint8_t* tile_out, void* stream) {
    if (!G_out || !f_out || !band_out || !tile_out)
        return fail(JL_ERR_INVALID_ARGUMENT, "null pointer argument");
    if (L < 1 || L > 2147483647LL) return fail(JL_ERR_INVALID_ARGUMENT, "L must be in [1, 2^31)");
    if (w_pretrained < 1 || w_local < 0)
        return fail(JL_ERR_INVALID_ARGUMENT, "w_pretrained >= 1 and w_local >= 0 required");
    if (bifocal != 0 && bifocal != 1) return fail(JL_ERR_INVALID_ARGUMENT, "bifocal must be 0 or 1");
    if (bm < 1 || bm > 4096 || bn < 1 || bn > 4096)
        return fail(JL_ERR_INVALID_ARGUMENT, "bm and bn must be in [1, 4096]");
    hipStream_t s = (hipStream_t)stream;
    hipError_t e = launch_debug_index(L, w_pretrained, w_local, bifocal, bm, bn, G_out, f_out,
                                      band_out, tile_out, s);
    if (e != hipSuccess) return hip_fail(e, "debug index launch");
    return finish(s, "jl_debug_index_math");
}

jl_status jl_debug_stream_read(const void* src, size_t bytes, uint32_t* partial_sums,
                               void* stream) {
    if (!src || !partial_sums) return fail(JL_ERR_INVALID_ARGUMENT, "null pointer argument");
    if (bytes < 16 || bytes % 16) return fail(JL_ERR_INVALID_ARGUMENT, "bytes must be a positive multiple of 16");
    if (bytes > (1ULL << 40)) return fail(JL_ERR_INVALID_ARGUMENT, "bytes above 2^40");
    if (!al16(src) || ((uintptr_t)partial_sums & 3))
        return fail(JL_ERR_INVALID_ARGUMENT, "src must be 16-byte and partial_sums 4-byte aligned");
    hipStream_t s = (hipStream_t)stream;
    hipError_t e = launch_stream_read(src, (int64_t)bytes, partial_sums, s);
    if (e != hipSuccess) return hip_fail(e, "stream read launch");
    return finish(s, "jl_debug_stream_read");
}

jl_status jl_debug_mfma_stream(const void* operands, size_t operand_bytes, int32_t iters,
                               float* out, void* stream) {
    if (!operands || !out) return fail(JL_ERR_INVALID_ARGUMENT, "null pointer argument");
    if (operand_bytes < kMfmaStreamOperandBytes)
        return fail(JL_ERR_INVALID_ARGUMENT,
                    "operand_bytes must be at least " + std::to_string(kMfmaStreamOperandBytes));
    if (iters < 1 || iters > (1 << 24)) return fail(JL_ERR_INVALID_ARGUMENT, "iters must be in [1, 2^24]");
    if (!al16(operands) || ((uintptr_t)out & 3))
        return fail(JL_ERR_INVALID_ARGUMENT, "operands must be 16-byte and out 4-byte aligned");
    hipStream_t s = (hipStream_t)stream;
    hipError_t e = launch_mfma_stream(operands, iters, out, s);
    if (e != hipSuccess) return hip_fail(e, "mfma stream launch");
    return finish(s, "jl_debug_mfma_stream");
}

jl_status jl_profile_enable(int32_t on) {
    std::lock_guard<std::mutex> lk(g_prof_mu);
    clear_records();
    g_prof_on = on != 0;
    g_err.clear();
    return JL_OK;
}

jl_status jl_profile_read(const char** names, int32_t* counts, double* total_ms, int32_t capacity,
                          int32_t* n_out) {
    if (!n_out || (capacity > 0 && (!names || !counts || !total_ms)))
        return fail(JL_ERR_INVALID_ARGUMENT, "null pointer argument");
    std::lock_guard<std::mutex> lk(g_prof_mu);
    std::vector<const char*> nm;
    std::vector<int32_t> cnt;
    std::vector<double> tot;
    for (auto& r : g_recs) {
        hipError_t e = hipEventSynchronize(r.stop);
        if (e != hipSuccess) return hip_fail(e, "jl_profile_read");
        float ms = 0.0f;
        e = hipEventElapsedTime(&ms, r.start, r.stop);
        if (e != hipSuccess) return hip_fail(e, "jl_profile_read");
        size_t i = 0;
        while (i < nm.size() && strcmp(nm[i], r.name) != 0) ++i;
        if (i == nm.size()) {
            nm.push_back(r.name);
            cnt.push_back(0);
            tot.push_back(0.0);
        }
        cnt[i] += 1;
        tot[i] += ms;
    }
    clear_records();
    *n_out = (int32_t)nm.size();
    for (int32_t i = 0; i < capacity && i < (int32_t)nm.size(); ++i) {
        names[i] = nm[i];
        counts[i] = cnt[i];
        total_ms[i] = tot[i];
    }
    g_err.clear();
    return JL_OK;
}

}  // extern "C"
