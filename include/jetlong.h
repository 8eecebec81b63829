/*
 * jetlong.h -- C ABI of libjetlong: Dynamic Bifocal RoPE attention (Jet-Long)
 * on AMD Instinct MI355X (gfx950).
 *
 * The method (pages cited by title and section):
 *   [BT] "Jet-Long: 具有动态双焦RoPE的高效长上下文扩展" (bittide.aicompass.dev):
 *        §3.1 group size G = max(1, ceil(L / w_pretrained)) and remap
 *        f(x) = floor(x / G); §3.2 inclusion-exclusion merge; §3.3 KV-cache
 *        correction rotation; §3.4 one fused kernel for prefill and generation.
 *   [TW] "NVIDIA研究团队找到了让AI“看清”超长文本的新方法" (techwalker.com):
 *        §二 local window (standard RoPE) and remote window (remapped RoPE);
 *        §三 cache keeps raw-RoPE keys, correction rotations at read time;
 *        §四 three attention calls B, A, C merged with LogSumExp weights.
 *
 * Conventions shared by every entry point:
 *   - Tensors are row-major and contiguous.  q, o: [T][Hq][d]; k, v: [T][Hkv][d]
 *     (packed "varlen" layout); lse: float32.  d is 64 or 128; Hq % Hkv == 0 and
 *     query head h reads kv head h / (Hq / Hkv).
 *   - RoPE is the half-split form: pair (t, t + d/2) is turned by p * theta_t,
 *     theta_t = rope_base^(-2t/d).
 *   - Positions are 0-based within each sequence.  A key j is local to query i
 *     iff 0 <= i - j < w_local and remote iff i - j >= w_local; keys j > i are
 *     masked (causal).
 *   - Scores are softmax_scale * <q_rot, k_rot>; lse is the natural log of the
 *     sum of exp(score) over the keys of a row.
 *   - All pointers except those marked "host" are device pointers owned by the
 *     caller.  The library allocates no device memory and never synchronizes:
 *     work is enqueued on `stream` (a hipStream_t; NULL is the default stream)
 *     and is complete when the caller synchronizes that stream.  A call
 *     enqueues kernels only (no memset, copy or allocation), so it can be
 *     captured in a HIP graph and replayed; a replay reads the buffers the
 *     call was given.  State the library keeps: a thread-local error string;
 *     the kernel-timing record while jl_profile_enable(1) is in force
 *     (process-wide, see there); the static scratch of
 *     jl_bifocal_decode_noalloc (one array per device).  Workspace sizes and
 *     launch shapes depend only on the arguments.  Two environment variables
 *     are read for debugging only: JL_LOG (print failures to stderr) and
 *     JL_DEBUG_SYNC (synchronize the stream after each call and report its
 *     errors); neither changes results or sizes.
 *   - Every argument is validated on the host before any HIP call.  A failing
 *     entry point launches nothing and returns a status; jl_last_error() then
 *     holds a description.  Values that live in device memory (cu_seqlens,
 *     seqlens_k, positions) cannot be checked on the host: if they break the
 *     documented contract the outputs are unspecified, but no kernel reads or
 *     writes outside the buffers whose sizes the host arguments describe.
 *   - Outputs must not alias inputs (except in jl_rope_apply).
 *   - The attention entry points move tensors in 16-byte vectors: q, k, v, o,
 *     k_rot_out and the caches or page pools must start on a 16-byte boundary
 *     (JL_ERR_INVALID_ARGUMENT otherwise).  Workspaces start on a 256-byte
 *     boundary.
 */
#ifndef JETLONG_H
#define JETLONG_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define JL_ABI_VERSION 3

typedef enum {
    JL_OK = 0,
    JL_ERR_INVALID_ARGUMENT = 1, /* null pointer, bad size, inconsistent shapes        */
    JL_ERR_UNSUPPORTED = 2,      /* legal request this build does not implement       */
    JL_ERR_WORKSPACE_TOO_SMALL = 3,
    JL_ERR_HIP = 4               /* a HIP runtime call or kernel launch failed        */
} jl_status;

typedef enum { JL_DTYPE_F32 = 0, JL_DTYPE_BF16 = 1 } jl_dtype;

typedef struct {
    int32_t w_pretrained;  /* >= 1: the model's pretraining window ([BT] §3.1)            */
    int32_t w_local;       /* >= 0: local window size in tokens ([TW] §二; 2048 there)     */
    double rope_base;      /* > 0: theta_t = rope_base^(-2t/d)                             */
    float softmax_scale;   /* > 0 and finite                                               */
    int32_t bifocal;       /* 1: Jet-Long; 0: plain RoPE causal attention (same kernels);  */
                           /* 2: the remote-window variant the pages compare against     */
                           /*    ([BT] §4.4, [TW] §八): continuous interpolation, remote  */
                           /*    position x / s with the real s = max(1, L / w_pretrained) */
                           /*    in place of floor(x / G).  bf16 prefill, chunked prefill */
                           /*    and decode only (JL_ERR_UNSUPPORTED elsewhere)           */
    int32_t precise;       /* 0: fast scores (below); 1: split-precision scores for       */
                           /*    concentrated attention (a few keys carry the softmax, so */
                           /*    one key's score rounding reaches the LSE undiluted).     */
                           /*    bf16 prefill: q and k as fp16 hi + lo on every row       */
                           /*    (3 products instead of 1; rows below 2048 always do so); */
                           /*    bf16 decode: remote keys turned in fp32 and split hi + lo */
                           /*    (the stored keys and the query already are exact / split).*/
                           /*    Ignored by the fp32 paths (already split); fp8 decode:   */
                           /*    JL_ERR_UNSUPPORTED.  Must be 0 or 1.                     */
    int32_t reuse_images;  /* chunk calls only (ignored elsewhere); 0 or 1.  1: the      */
                           /*    caller keeps the workspace from one chunk call to the    */
                           /*    next on the same caches and changes no cache row below   */
                           /*    the lengths an earlier call saw; key/value images that   */
                           /*    call built are then reused while they still hold (same   */
                           /*    caches, sizes and parameters, same G, for bifocal 2 the  */
                           /*    same L), and only the new rows are turned.  0: rebuild   */
                           /*    (the first call of every prefill: a workspace may hold   */
                           /*    images of other caches that sat at the same addresses).  */
} jl_params;

/* JL_ABI_VERSION of the built library. */
int jl_abi_version(void);

/* Static, never-null text for a status value. */
const char* jl_status_string(int status);

/* Thread-local description of the last failure on this thread ("" if none). */
const char* jl_last_error(void);

/*
 * [BT] §3.1: *G_out = max(1, ceil(L / w_pretrained)) computed in exact integer
 * arithmetic on the host.  L >= 1, w_pretrained >= 1; G_out is a host pointer.
 */
jl_status jl_group_size(int64_t L, int32_t w_pretrained, int32_t* G_out);

/*
 * RoPE rotation: out[t][h][:] = R(floor(positions[t] / G)) x[t][h][:].
 * G = 1 gives standard RoPE (what a KV cache stores, [TW] §三); G > 1 gives the
 * remapped rotation of the remote window ([BT] §3.1).
 *   x, out     [T][H][d] of `dtype`; out may equal x (in place).
 *   positions  device int32 [T], each >= 0.
 *   T >= 1, H >= 1, d in {64, 128}, rope_base > 0, G >= 1.
 * Angles are reduced in fp64 before sin/cos, so positions up to 2^31 - 1 keep
 * full fp32 accuracy; bf16 outputs are rounded to nearest even.
 */
jl_status jl_rope_apply(void* out, const void* x, const int32_t* positions, int64_t T, int32_t H,
                        int32_t d, double rope_base, int32_t G, jl_dtype dtype, void* stream);

/*
 * Bytes of device workspace jl_bifocal_prefill needs for these sizes
 * (host pointer `bytes`).  Depends only on the arguments, never on data.
 * `params` (host, may be NULL for the defaults) matters only through
 * params->precise: split precision on every row needs low-part key tiles for
 * every key.
 */
jl_status jl_bifocal_prefill_workspace(int64_t T, int32_t n_seqs, int32_t Hq, int32_t Hkv,
                                       int32_t d, jl_dtype dtype, const jl_params* params,
                                       size_t* bytes);

/*
 * Causal bifocal prefill ([BT] §3.2, [TW] §四).  For query i of a sequence of
 * length L (G = G(L), f(x) = floor(x/G)) and every key j <= i:
 *     local  (i - j <  w_local): s = scale * <R(i) q_i,    R(j) k_j>
 *     remote (i - j >= w_local): s = scale * <R(f(i)) q_i, R(f(j)) k_j>
 * then o_i = softmax(s) v and lse_i = ln sum_j exp(s_ij).  This is exactly the
 * pages' merge of full remote attention plus local-standard minus
 * local-remapped; the kernel evaluates it tile by tile without a mask.
 *   o          [T][Hq][d] of dtype (written).
 *   lse        float32 [Hq][T] (written).
 *   q, k, v    raw, un-rotated inputs, [T][Hq][d] and [T][Hkv][d].
 *   cu_seqlens device int32 [n_seqs + 1]: 0 = cu[0] < cu[1] < ... < cu[n_seqs] = T
 *              (each sequence non-empty, each length <= max_seqlen), or NULL
 *              for a single sequence of T tokens (then n_seqs must be 1).
 *   max_seqlen >= every sequence length (sizes the launch grid).
 *   k_rot_out  optional (NULL to skip): [T][Hkv][d] of dtype receives R(j) k_j,
 *              the standard-RoPE keys a KV cache stores for later decode.
 *   workspace  device buffer of at least jl_bifocal_prefill_workspace() bytes,
 *              256-byte aligned; contents need no initialisation and are
 *              scratch after the call.
 * Supported: dtype bf16 (MFMA path) or f32 (fp32 path), d in {64, 128}.
 * The bf16 path forms q k^T and P v on fp16 MFMA operands (fp32 accumulate):
 * inputs must be finite and the rotated q (times softmax_scale * log2 e), the
 * rotated k and v must stay below 65504 in magnitude.  Device data is not
 * range-checked and operands are not clamped: a row that scores an operand
 * beyond that range gets a non-finite o or lse (rows that never see it are
 * unaffected), so such input shows rather than giving a quietly wrong value.
 */
jl_status jl_bifocal_prefill(void* o, float* lse, const void* q, const void* k, const void* v,
                             const int32_t* cu_seqlens, int32_t n_seqs, int64_t T,
                             int32_t max_seqlen, int32_t Hq, int32_t Hkv, int32_t d,
                             const jl_params* params, jl_dtype dtype, void* k_rot_out,
                             void* workspace, size_t workspace_bytes, void* stream);

/* Bytes of device workspace jl_bifocal_prefill_three_call needs (bf16 only);
 * params as for jl_bifocal_prefill_workspace. */
jl_status jl_bifocal_prefill_three_call_workspace(int64_t T, int32_t n_seqs, int32_t Hq,
                                                  int32_t Hkv, int32_t d, jl_dtype dtype,
                                                  const jl_params* params, size_t* bytes);

/*
 * The pages' unfused form of the same prefill ([TW] §四, [BT] §3.2): three
 * separate attention calls,
 *     B: every causal pair under remapped RoPE,
 *     A: the local pairs (i - j < w_local) under standard RoPE,
 *     C: the local pairs under remapped RoPE,
 * combined as Z = e^lse_B - e^lse_C + e^lse_A and
 * o = (e^lse_B o_B - e^lse_C o_C + e^lse_A o_A) / Z (the remote mass
 * e^lse_B - e^lse_C clamped at 0), from the calls' fp32 outputs.  Up to
 * rounding this equals jl_bifocal_prefill; it exists to compare the two
 * forms on the device.
 * Arguments as for jl_bifocal_prefill (no k_rot_out); params->bifocal must
 * be 1; dtype must be JL_DTYPE_BF16 (else JL_ERR_UNSUPPORTED).  The three
 * calls' outputs live in the workspace.
 */
jl_status jl_bifocal_prefill_three_call(void* o, float* lse, const void* q, const void* k,
                                        const void* v, const int32_t* cu_seqlens, int32_t n_seqs,
                                        int64_t T, int32_t max_seqlen, int32_t Hq, int32_t Hkv,
                                        int32_t d, const jl_params* params, jl_dtype dtype,
                                        void* workspace, size_t workspace_bytes, void* stream);

/* Bytes of device workspace jl_bifocal_decode (and the paged and fp8 decode
 * calls) need for these sizes: the split partials of the key chunks. */
jl_status jl_bifocal_decode_workspace(int32_t batch, int32_t max_seqlen_k, int32_t Hq,
                                      int32_t Hkv, int32_t d, jl_dtype dtype, size_t* bytes);

/*
 * Bifocal decode ([TW] §三, [BT] §3.3): one new query per sequence against a
 * KV cache that stores keys under standard RoPE at their original positions
 * (k_cache[b][j] = R(j) k_j, e.g. written by jl_rope_apply with G = 1 or by
 * jl_bifocal_prefill's k_rot_out).  The cache is read-only: it is never
 * rewritten when G changes.  With L = seqlens_k[b] (the current token is
 * already appended), p = L - 1, G = G(L):
 *     local  (p - j <  w_local): s = scale * <R(p) q, k_cache[j]>
 *     remote (p - j >= w_local): s = scale * <R(f(p)) q, R(f(j) - j) k_cache[j]>
 * i.e. the query carries the correction f(p) - p and every remote key the
 * correction f(j) - j, applied in registers.
 *   o          [B][Hq][d] of dtype (written); lse float32 [B][Hq] (written).
 *   q          raw (un-rotated) query [B][Hq][d].
 *   k_cache, v_cache  [B][S_max][Hkv][d] of dtype, read-only.
 *   seqlens_k  device int32 [B], 1 <= L_b <= max_seqlen_k <= S_max.
 *   workspace  at least jl_bifocal_decode_workspace() bytes (scratch).
 * Supported: dtype bf16 or f32 (bf16 only for params->bifocal == 2), d in {64, 128},
 * Hq / Hkv <= 16.  The bf16 path forms q k^T on fp16 MFMA operands and P v on
 * bf16 ones (fp32 accumulate): the rotated query (times softmax_scale *
 * log2 e) and the cached keys must stay below 65504 in magnitude; device
 * data is not range-checked.
 */
jl_status jl_bifocal_decode(void* o, float* lse, const void* q, const void* k_cache,
                            const void* v_cache, const int32_t* seqlens_k, int32_t batch,
                            int32_t max_seqlen_k, int64_t S_max, int32_t Hq, int32_t Hkv,
                            int32_t d, const jl_params* params, jl_dtype dtype, void* workspace,
                            size_t workspace_bytes, void* stream);

/*
 * jl_bifocal_decode without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation).  Same arguments, results and kernels as
 * jl_bifocal_decode; the split partials live in a static device array of
 * the library (32 MiB per device, held until the
 * process ends).  Sizes whose decode workspace (jl_bifocal_decode_workspace)
 * exceeds 32 MiB return JL_ERR_WORKSPACE_TOO_SMALL before any HIP call (at
 * 128K keys with 32 query heads a batch of 1 needs about 4.3 MB).  The first
 * call on a device looks up that device's copy of the array; `stream` must
 * belong to the current device (JL_ERR_INVALID_ARGUMENT otherwise).  Every
 * call on a device shares its array: calls that overlap on one device (on
 * different streams, or from several threads) race and must be serialized
 * by the caller.  The array keeps the last call's partials, which need no
 * clearing (every call writes each partial it reads).  Allocates nothing.
 */
jl_status jl_bifocal_decode_noalloc(void* o, float* lse, const void* q, const void* k_cache,
                                    const void* v_cache, const int32_t* seqlens_k, int32_t batch,
                                    int32_t max_seqlen_k, int64_t S_max, int32_t Hq, int32_t Hkv,
                                    int32_t d, const jl_params* params, jl_dtype dtype,
                                    void* stream);

/* Bytes of device workspace jl_bifocal_decode_three_call needs (bf16 only):
 * a remapped copy of the cache's keys [batch][max_seqlen_k][Hkv][d], the three
 * calls' fp32 outputs and the split partials.  params->w_local sizes the
 * local calls' partials. */
jl_status jl_bifocal_decode_three_call_workspace(int32_t batch, int32_t max_seqlen_k, int32_t Hq,
                                                 int32_t Hkv, int32_t d, jl_dtype dtype,
                                                 const jl_params* params, size_t* bytes);

/*
 * The pages' unfused form of a generation step ([TW] §四, [BT] §3.2), the
 * counterpart of jl_bifocal_prefill_three_call: three separate attention
 * calls over the cache and a LogSumExp merge.  Because the cache holds
 * standard-RoPE keys ([TW] §三), call B first needs every key turned to
 * remapped RoPE: the call writes R(f(j) - j) k_cache[b][j] for all j < L_b
 * into the workspace ([BT] §3.3's correction, applied to the whole cache and
 * stored), then runs
 *     B: the query R(f(p)) q against every remapped key,
 *     A: R(p) q against the stored keys with p - j < w_local,
 *     C: R(f(p)) q against the remapped keys with p - j < w_local,
 * each a plain decode with fp32 output, and merges
 * o = (e^lse_B o_B - e^lse_C o_C + e^lse_A o_A) / Z, Z = e^lse_B - e^lse_C +
 * e^lse_A (the remote mass clamped at 0).  Up to rounding this equals
 * jl_bifocal_decode; it exists to measure the two forms on the device.
 * Arguments as for jl_bifocal_decode (flat bf16 caches, read-only);
 * params->bifocal must be 1 and params->precise 0 (JL_ERR_INVALID_ARGUMENT
 * / JL_ERR_UNSUPPORTED otherwise).
 */
jl_status jl_bifocal_decode_three_call(void* o, float* lse, const void* q, const void* k_cache,
                                       const void* v_cache, const int32_t* seqlens_k,
                                       int32_t batch, int32_t max_seqlen_k, int64_t S_max,
                                       int32_t Hq, int32_t Hkv, int32_t d,
                                       const jl_params* params, jl_dtype dtype, void* workspace,
                                       size_t workspace_bytes, void* stream);

/*
 * jl_bifocal_decode on a paged KV cache (the layout serving systems keep):
 * k_pages, v_pages are pools of n_pages pages, each [page_size][Hkv][d] bf16
 * holding standard-RoPE keys (values) at their original positions; key j of
 * sequence b sits in page block_table[b * bt_stride + j / page_size], row
 * j % page_size.  Same scores, outputs and workspace size
 * (jl_bifocal_decode_workspace) as jl_bifocal_decode; the pool is read-only.
 *   block_table  device int32 [batch][bt_stride]; bt_stride * page_size >= max_seqlen_k.
 *   page_size    a power of two in [16, 65536].
 * Page numbers outside [0, n_pages) are clamped into the pool (the result is
 * then unspecified, but nothing is read outside it).  bf16 only.
 */
jl_status jl_bifocal_decode_paged(void* o, float* lse, const void* q, const void* k_pages,
                                  const void* v_pages, const int32_t* block_table,
                                  const int32_t* seqlens_k, int32_t batch, int32_t max_seqlen_k,
                                  int32_t page_size, int64_t n_pages, int32_t bt_stride, int32_t Hq,
                                  int32_t Hkv, int32_t d, const jl_params* params, jl_dtype dtype,
                                  void* workspace, size_t workspace_bytes, void* stream);

/*
 * jl_bifocal_decode on an fp8 KV cache, for decode bandwidth: k_cache and
 * v_cache hold OCP E4M3 codes (1 byte per element, the OCP 8-bit floating
 * point format: bias 7, subnormals, no infinities), and element (b, j, h, x)
 * stands for k_scale[h] * E4M3(code) (v_scale[h] for values).  The scores,
 * the correction rotation ([TW] §三, [BT] §3.3) and the outputs are those
 * of jl_bifocal_decode on these dequantized values: the rotation is applied
 * after dequantization, so the cache format leaves the method unchanged.
 * Codes widen exactly to fp16 (the MFMA operands); the key scale multiplies
 * the finished scores, so the query's fp16 parts keep their range, and the
 * value scale multiplies the output.
 *   q, o          bf16 [B][Hq][d]; lse float32 [B][Hq].
 *   k_cache, v_cache  uint8 [B][S_max][Hkv][d] E4M3 codes, read-only.
 *   k_scale, v_scale  device float32 [Hkv].
 *   workspace     jl_bifocal_decode_workspace(..., JL_DTYPE_BF16) bytes.
 * NaN codes (S.1111.111) are the caller's to avoid (jl_kv_quantize_fp8
 * writes them only for NaN input).  d in {64, 128}, Hq / Hkv <= 16.
 */
jl_status jl_bifocal_decode_fp8(void* o, float* lse, const void* q, const void* k_cache,
                                const void* v_cache, const float* k_scale, const float* v_scale,
                                const int32_t* seqlens_k, int32_t batch, int32_t max_seqlen_k,
                                int64_t S_max, int32_t Hq, int32_t Hkv, int32_t d,
                                const jl_params* params, void* workspace, size_t workspace_bytes,
                                void* stream);

/* jl_bifocal_decode_fp8 on a paged pool of E4M3 pages [n_pages][page_size][Hkv][d],
 * addressed as in jl_bifocal_decode_paged. */
jl_status jl_bifocal_decode_fp8_paged(void* o, float* lse, const void* q, const void* k_pages,
                                      const void* v_pages, const float* k_scale,
                                      const float* v_scale, const int32_t* block_table,
                                      const int32_t* seqlens_k, int32_t batch,
                                      int32_t max_seqlen_k, int32_t page_size, int64_t n_pages,
                                      int32_t bt_stride, int32_t Hq, int32_t Hkv, int32_t d,
                                      const jl_params* params, void* workspace,
                                      size_t workspace_bytes, void* stream);

/*
 * Writes fp8 cache rows: out[t][h][x] = E4M3(x[t][h][x] / scale[h]) with the
 * quotient a correctly rounded fp32 division, rounded to the nearest code
 * (ties to the even code) and saturated to +-448; NaN input gives a NaN code.
 *   x      bf16 [ntok][H][d], 16-byte aligned;  out uint8 [ntok][H][d], 8-byte aligned.
 *   scale  device float32 [H] (> 0).  d a multiple of 8.
 */
jl_status jl_kv_quantize_fp8(void* out, const void* x, const float* scale, int64_t ntok,
                             int32_t H, int32_t d, void* stream);

/* Bytes of device workspace the chunk calls below need for Tq query rows in
 * batch sequences of at most max_seqlen_k keys (bf16 only).  It holds the
 * fp16 images of the cache's key and value tiles (each sequence a fixed
 * stretch of max_seqlen_k keys), a small record of what they were built for
 * (see jl_params.reuse_images), and fp32 partials for calls whose grid is
 * small (fewer 256-row workgroups than compute units, e.g. a 1024-row chunk
 * of 32 heads): those split each row block's keys in up to four shares
 * and merge the shares in LogSumExp space.  The images and the record sit at
 * the same offsets for every Tq, so a workspace sized for the largest chunk
 * serves every chunk size.  params as for jl_bifocal_prefill_workspace
 * (split-precision calls take no key shares). */
jl_status jl_bifocal_prefill_chunk_workspace(int64_t Tq, int32_t batch, int32_t max_seqlen_k,
                                             int32_t Hq, int32_t Hkv, int32_t d, jl_dtype dtype,
                                             const jl_params* params, size_t* bytes);

/*
 * Chunked prefill ([TW] §三 and [BT] §3.3 for the cache, [BT] §3.1 for G): a
 * chunk of new tokens per sequence attends causally to every key of its
 * sequence held in a KV cache of standard-RoPE keys (the chunk's own keys,
 * appended by the caller, included).  Sequence b has L_b = seqlens_k[b] keys
 * and C_b = cu_seqlens_q[b + 1] - cu_seqlens_q[b] new query rows at positions
 * L_b - C_b .. L_b - 1, with G = G(L_b), the length the call sees: each row
 * gets exactly what jl_bifocal_prefill gives that row of the whole sequence
 * of length L_b.  A query at position p scores key j <= p as
 *     local  (p - j <  w_local): s = scale * <R(p) q, k_cache[j]>
 *     remote (p - j >= w_local): s = scale * <R(f(p)) q, R(f(j) - j) k_cache[j]>
 * and the cache is never rewritten (jl_bifocal_decode is the case C_b = 1).
 *   o             [Tq][Hq][d] bf16 (written); lse float32 [Hq][Tq] (written).
 *   q             raw (un-rotated) queries [Tq][Hq][d], the chunks packed.
 *   cu_seqlens_q  device int32 [batch + 1], 0 = cu[0] <= ... <= cu[batch] = Tq;
 *                 NULL for one chunk (batch == 1, max_seqlen_q == Tq).
 *                 A sequence may have C_b = 0 (nothing is computed for it).
 *   max_seqlen_q  host int, >= every C_b.
 *   k_cache, v_cache  [batch][S_max][Hkv][d] bf16, read-only.
 *   seqlens_k     device int32 [batch], C_b <= L_b <= max_seqlen_k <= S_max.
 *   workspace     at least jl_bifocal_prefill_chunk_workspace() bytes.
 *                 Each call turns the cache rows [0, L_b) into fp16 images
 *                 (remote keys to remapped RoPE) in the workspace; with
 *                 params->reuse_images = 1 it turns only the rows past the
 *                 whole 64-key tiles an earlier call on this workspace built
 *                 and that still hold (a chunked prefill then turns each
 *                 row about once).  The first call of a prefill passes 0.
 *                 Calls that share a workspace must not overlap.
 * If the device arrays break their contract nothing is read or written
 * outside the buffers and o, lse are left unwritten.  bf16 only; d in
 * {64, 128}; rotated q and k must stay below 65504 in magnitude (fp16 MFMA
 * operands).
 */
jl_status jl_bifocal_prefill_chunk(void* o, float* lse, const void* q,
                                   const int32_t* cu_seqlens_q, int64_t Tq, int32_t max_seqlen_q,
                                   const void* k_cache, const void* v_cache,
                                   const int32_t* seqlens_k, int32_t batch,
                                   int32_t max_seqlen_k, int64_t S_max, int32_t Hq, int32_t Hkv,
                                   int32_t d, const jl_params* params, jl_dtype dtype,
                                   void* workspace, size_t workspace_bytes, void* stream);

/*
 * jl_bifocal_prefill_chunk on a paged KV cache: pools k_pages, v_pages of
 * n_pages pages [page_size][Hkv][d] bf16; key j of sequence b sits in page
 * block_table[b * bt_stride + j / page_size], row j % page_size (page_size a
 * power of two in [16, 65536], bt_stride * page_size >= max_seqlen_k).  Page
 * numbers outside [0, n_pages) are clamped into the pool.  Same results and
 * workspace as the flat form.
 */
jl_status jl_bifocal_prefill_chunk_paged(void* o, float* lse, const void* q,
                                         const int32_t* cu_seqlens_q, int64_t Tq,
                                         int32_t max_seqlen_q, const void* k_pages,
                                         const void* v_pages, const int32_t* block_table,
                                         const int32_t* seqlens_k, int32_t batch,
                                         int32_t max_seqlen_k, int32_t page_size,
                                         int64_t n_pages, int32_t bt_stride, int32_t Hq,
                                         int32_t Hkv, int32_t d, const jl_params* params,
                                         jl_dtype dtype, void* workspace,
                                         size_t workspace_bytes, void* stream);

/*
 * Test export: runs the kernels' own device index functions for a sequence of
 * length L (1 <= L) and writes
 *   G_out     device int32 [1]    G(L)
 *   f_out     device int32 [L]    f(x) for x = 0..L-1
 *   band_out  device uint8 [n*n], n = min(L, 1024): band of (i, j) for
 *             i, j < n: 0 masked (j > i), 1 local, 2 remote
 *   tile_out  device uint8 [ceil(L/bm) * ceil(L/bn)]: class of the tile
 *             rows [a*bm, min((a+1)*bm, L)) x keys [b*bn, min((b+1)*bn, L)):
 *             bit 0 = holds a local pair, bit 1 = holds a remote pair,
 *             bit 2 = holds a masked (j > i) pair; 0 = skipped (all masked).
 * bm, bn in [1, 4096]; bifocal as in jl_params.
 */
jl_status jl_debug_index_math(int64_t L, int32_t w_pretrained, int32_t w_local, int32_t bifocal,
                              int32_t bm, int32_t bn, int32_t* G_out, int32_t* f_out,
                              uint8_t* band_out, uint8_t* tile_out, void* stream);

/*
 * Measurement aid: reads `bytes` of device memory at `src` once, as a
 * read-only stream (256 workgroups, 16-byte loads, four in flight per thread),
 * and writes the wrapping uint32 sum of the words each workgroup read to
 * partial_sums (device uint32 [256]); their wrapping sum is the sum of every
 * uint32 word of the buffer.  Timing it gives the HBM read rate the decode
 * kernels, which read each cache byte once, are compared with.  src 16-byte
 * aligned, bytes a positive multiple of 16 (JL_ERR_INVALID_ARGUMENT otherwise).
 */
jl_status jl_debug_stream_read(const void* src, size_t bytes, uint32_t* partial_sums, void* stream);

/*
 * Measurement aid: a stream of 32 x 32 x 16 fp16 MFMAs (the instruction the
 * bf16 prefill's QK^T and P V run on) and nothing else, on operands the caller
 * provides.  256 workgroups of 512 threads (two waves per SIMD); thread t of
 * workgroup b reads 16 fp16 x 8 vectors at byte offset (b * 512 + t) * 256 of
 * `operands` as eight (A, B) operand pairs, runs `iters` iterations of 32
 * MFMAs (four independent accumulator chains of 8) and writes the sum of its
 * 64 fp32 accumulator elements to out[b * 512 + t] (device float [131072]).
 * One call performs 256 * 8 * iters * 32 MFMAs of 32768 flops each.  The
 * engine clock is power-limited and the operands' switching activity is part
 * of the power, so timing this on operands drawn like a workload's gives the
 * matrix-core rate those data allow.  operands 16-byte aligned, operand_bytes
 * >= 33554432, iters in [1, 2^24] (JL_ERR_INVALID_ARGUMENT otherwise).
 */
jl_status jl_debug_mfma_stream(const void* operands, size_t operand_bytes, int32_t iters,
                               float* out, void* stream);

/*
 * Kernel timing (profiling aid, off by default).  While enabled, every kernel
 * the library launches is bracketed by HIP events recorded on its stream;
 * jl_profile_read() synchronizes those events and reports, per kernel name,
 * the launch count and the summed duration in milliseconds, then clears the
 * record.  Enabling or disabling clears it too.  The record is one
 * process-wide list guarded by a mutex (calls from several threads are
 * safe, their launches share it); the events come from a pool that grows on
 * demand (hipEventCreate, host-side only) and is reused.  While enabled,
 * entry points are no longer free of state and should not be captured in a
 * HIP graph.  Host pointers; `names` receives static strings.
 */
jl_status jl_profile_enable(int32_t on);
jl_status jl_profile_read(const char** names, int32_t* counts, double* total_ms, int32_t capacity,
                          int32_t* n_out);

#ifdef __cplusplus
}
#endif

#endif /* JETLONG_H */
