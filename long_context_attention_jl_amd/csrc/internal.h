// internal.h -- launchers shared between libjetlong's entry points and kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "common.h"

namespace jl {

// Records start/stop events around one launch when profiling is on.
struct LaunchScope {
    LaunchScope(const char* name, hipStream_t s);
    ~LaunchScope();
    const char* name_;
    hipStream_t stream_;
    int slot_;
};

// most key shares a chunk call splits a row block's tiles into
constexpr int kChunkMaxSplit = 4;

// Byte layout of the prefill workspace; every region starts 256-byte aligned.
struct PrefillLayout {
    int64_t T_pad;    // padded key rows (multiple of kBN)
    int64_t lo_pad;   // padded rows of the split-precision ("lo") key copies
    size_t plan, ks, kr, vt, ks_lo, kr_lo;  // offsets (bf16 path)
    size_t ks32, kr32;                      // offsets (f32 path)
    size_t total;
};
// precise: the split-precision ("lo") key tiles cover every key, not only the
// first kPreciseRows of each sequence
PrefillLayout prefill_layout(int64_t T, int32_t n_seqs, int32_t Hkv, int32_t d, int dtype,
                             int precise);

// bf16 decode: positions per stage and the most stages one chunk may hold
// (the kernel keeps one query-angle row per stage in LDS)
constexpr int kDecodeStageB = 48;
constexpr int kDecodeMaxStagesB = 32;
// a chunk spans at most 32 * 48 + 47 positions: with pages of >= 16 rows, at
// most this many pages
constexpr int kDecodeMaxPages = (kDecodeMaxStagesB * kDecodeStageB + kDecodeStageB - 1) / 16 + 2;

// Decode workspace: per (sequence, key chunk, query head) a partial
// (m, l_o, l_lse) and the unnormalised O, merged by a second kernel.
struct DecodeLayout {
    int32_t n_splits;
    int32_t chunk;
    size_t part_ml;  // float4 (m, l_o, l_lse, 0) [B][n_splits][Hq]
    size_t part_o;   // float [B][n_splits][Hq][d]
    size_t total;
};
// target_wg: workgroups per call to aim at (0: the default, 256 for bf16);
// a smaller target never needs more workspace than the default.
DecodeLayout decode_layout(int32_t batch, int32_t max_seqlen_k, int32_t Hq, int32_t Hkv, int32_t d,
                           int dtype, int target_wg = 0);
// workgroup target of flat bf16 decode at max_seqlen_k >= 65536
constexpr int kDecodeLongTargetWG = 192;

RopeFreq make_rope_freq(double base, int d);

constexpr int kStreamReadWgs = 256;  // workgroups (and partial sums) of the read stream
hipError_t launch_stream_read(const void* src, int64_t bytes, uint32_t* out, hipStream_t s);
// matrix-core stream: 256 workgroups x 512 threads, each thread 16 fp16 x 8 operand vectors
constexpr int kMfmaStreamWgs = 256;
constexpr size_t kMfmaStreamOperandBytes = (size_t)kMfmaStreamWgs * 512 * 16 * 16;
hipError_t launch_mfma_stream(const void* operands, int32_t iters, float* out, hipStream_t s);
hipError_t launch_rope_apply(void* out, const void* x, const int32_t* pos, int64_t T, int32_t H,
                             int32_t d, const RopeFreq& tab, int32_t G, int dtype,
                             hipStream_t s);

hipError_t launch_plan(int32_t* plan, const int32_t* cu, int32_t n_seqs, int64_t T,
                       int32_t max_seqlen, int32_t w_pretrained, int32_t precise, hipStream_t s);

struct PrefillArgs {
    const void* q;
    const void* k;
    const void* v;
    void* o;
    float* lse;
    void* k_rot_out;
    void* ws;
    PrefillLayout lay;
    int32_t n_seqs, Hq, Hkv, d, max_seqlen;
    int64_t T;
    int32_t w_local, bifocal;  // bifocal: 0 plain, 1 integer grouping, 2 continuous interpolation
    float softmax_scale;
    RopeFreq tab;
    int32_t mode;
    int32_t w_pretrained;  // for the continuous scale s = L / w_pretrained (bifocal 2)
    // Key split of a chunk call (ksplit > 1): the main-rows kernel runs each
    // row block as ksplit workgroups over equal shares of its key tiles and
    // writes partials (unnormalised O in fp32 [ksplit][T][Hq][D], and
    // (m in log2 units, l) [ksplit][Hq][T]) that a merge kernel combines.
    int32_t ksplit;
    float* part_o;
    float2* part_ml;  // 0 bifocal; unfused calls: 1 all pairs remapped, 2 local standard, 3 local remapped
    // A chunk against a cache (chunked != 0): the queries are each sequence's
    // newest rows, keys and values are read from the cache, whose keys already
    // carry standard RoPE.  Flat cache: sequence s owns rows [s * S_max, ...);
    // paged cache (block_table != nullptr): key j of sequence s sits in row
    // block_table[s * bt_stride + j / 2^page_shift] * 2^page_shift + j % 2^page_shift.
    int32_t chunked, max_seqlen_k;
    int64_t S_max;
    const int32_t* block_table;
    int32_t page_shift, bt_stride, n_pages;
    // split-precision (hi + lo) scores on every row, not only the first
    // kPreciseRows of each sequence
    int32_t precise;
    // o is written as float32 (the unfused form's separate calls)
    int32_t o_f32;
};

// Plan of a chunk call: per sequence b, C_b = cu_q[b + 1] - cu_q[b] query rows
// at positions seqlens_k[b] - C_b .. seqlens_k[b] - 1.
hipError_t launch_plan_chunk(int32_t* plan, void* image_state, uint64_t fingerprint, int32_t reuse,
                             const int32_t* cu_q, const int32_t* seqlens_k,
                             int32_t B, int64_t Tq, int32_t max_seqlen_q, int32_t max_seqlen_k,
                             int32_t w_pretrained, int32_t precise, int32_t bifocal, hipStream_t s);
// out[t][h][:] = E4M3(x[t][h][:] / scale[h]) (fp32 quotient, round to nearest
// even, saturating at +-448); x bf16 [ntok][H][d]
hipError_t launch_e4m3_quant(uint8_t* out, const void* x, const float* scale, int64_t ntok,
                             int32_t H, int32_t d, hipStream_t s);
hipError_t launch_kv_prepass(const PrefillArgs& a, int dtype, hipStream_t s);
// O = the LogSumExp combination of the three unfused calls B + A - C (fp32
// outputs of the calls, bf16 o); lse of row r, head h at r * ls_r + h * ls_h
hipError_t launch_three_call_merge(const float* oA, const float* oB, const float* oC,
                                   const float* lA, const float* lB, const float* lC, void* o,
                                   float* lse, int64_t rows, int32_t Hq, int32_t d, int64_t ls_r,
                                   int64_t ls_h, hipStream_t s);
// out[b][j] = R(f(j) - j) k_cache[b][j] for j < L_b (bf16 [B][max_seqlen_k][Hkv][d])
hipError_t launch_cache_remap(void* out, const void* kc, const int32_t* seqlens, int32_t B,
                              int32_t max_seqlen_k, int64_t S_max, int32_t Hkv, int32_t d,
                              int32_t w_pretrained, const RopeFreq& tab, hipStream_t s);
hipError_t launch_prefill_bf16(const PrefillArgs& a, hipStream_t s);
// combines the key-split partials of the main rows (positions >= 2048) of a
// chunk call into o and lse
hipError_t launch_chunk_merge(const PrefillArgs& a, hipStream_t s);
hipError_t launch_prefill_f32(const PrefillArgs& a, hipStream_t s);

struct DecodeArgs {
    const void* q;
    const void* kc;
    const void* vc;
    void* o;
    float* lse;
    const int32_t* seqlens;
    void* ws;
    DecodeLayout lay;
    int32_t B, max_seqlen_k, Hq, Hkv, d;
    int64_t S_max;
    int32_t w_pretrained, w_local, bifocal;
    float softmax_scale;
    RopeFreq tab;
    // paged cache (block_table != nullptr): key j of sequence b sits in row
    // block_table[b * bt_stride + j / 2^page_shift] * 2^page_shift + j % 2^page_shift
    const int32_t* block_table;
    int32_t page_shift, bt_stride;
    int64_t n_pages;
    // fp8 cache (fp8 != 0): OCP E4M3 codes, element = scale[kv head] * code
    // (k_scale / v_scale device float32 [Hkv], or nullptr for 1)
    int32_t fp8;
    const float* k_scale;
    const float* v_scale;
    // Single-call pieces of the unfused form (bf16, bifocal off): q_remap
    // turns the query by R(f(p)) instead of R(p); window keeps only the keys
    // p - j < w_local; o_f32 writes o as float32.
    int32_t q_remap, window, o_f32;
    // rows per sequence of the key cache when they differ from the value
    // cache's S_max (the unfused form's remapped copy of the keys); 0: S_max
    int64_t S_max_k;
    // remote keys turned in fp32 and split into fp16 hi + lo operands
    int32_t precise;
    // workgroup `split` takes the stages split, split + n_splits, ... of its
    // sequence (flat caches whose rows, plus three tiles, span less than
    // 2^31 bytes per sequence; see decode_interleave) instead of one chunk
    int32_t ilv;
};
// Whether the bf16 decode kernels may interleave stages across workgroups:
// flat caches, up to 8 query heads per kv head, and byte offsets of a
// sequence's rows within 32 bits.
bool decode_interleave(bool paged, int32_t Hq, int32_t Hkv, int32_t d, int32_t max_seqlen_k,
                       int32_t elem_bytes);
hipError_t launch_decode(const DecodeArgs& a, int dtype, hipStream_t s);

hipError_t launch_debug_index(int64_t L, int32_t w_pretrained, int32_t w_local, int32_t bifocal,
                              int32_t bm, int32_t bn, int32_t* G_out, int32_t* f_out,
                              uint8_t* band_out, uint8_t* tile_out, hipStream_t s);

}  // namespace jl
