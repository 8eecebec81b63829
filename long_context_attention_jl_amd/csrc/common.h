// common.h -- definitions shared by libjetlong's host code and gfx950 kernels.
//
// Pages cited (title, section):
//   [BT] "Jet-Long: 具有动态双焦RoPE的高效长上下文扩展" (bittide.aicompass.dev)
//   [TW] "NVIDIA研究团队找到了让AI“看清”超长文本的新方法" (techwalker.com)
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace jl {

typedef __bf16 bf16;
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16;
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float float2v __attribute__((ext_vector_type(2)));

// ---------------------------------------------------------------------------
// Tiling constants of the bf16 prefill path (also size its workspace).
constexpr int kBN = 64;             // keys per K/V tile
constexpr int kWaveRows = 32;       // query rows per wave (one 32x32 MFMA block)
constexpr int kWaves = 8;           // waves per prefill workgroup
constexpr int kBM = kWaveRows * kWaves;  // 256 query rows per workgroup
// Rows [0, kPreciseRows) of every sequence take the split-fp16 (hi + lo) score
// path: those rows see few keys, so the LSE inherits the rounding of a single
// score almost undiluted.  Keys they read are < kPreciseRows as well.
constexpr int kPreciseRows = 2048;
constexpr int kPlanFields = 10;     // int32 fields per sequence in the plan

// Key and value tiles are stored in the workspace exactly as they sit in LDS,
// so the prefill kernel fills LDS with flat global->LDS DMA copies.  A tile is
// stored in 16-byte pieces (8 halves), piece-major: piece c of every row, the
// rows in order, then piece c + 1.  An MFMA operand read (lane = one row's
// piece, 32 rows x 2 pieces) then covers 16 consecutive rows of one piece as
// one contiguous 256-byte stretch, which meets every LDS bank once: no
// padding, and every piece a lane reads sits at a compile-time offset from
// its first one.
//   K tile   [d / 8 pieces][kBN keys][8]   (piece c: elements 8c .. 8c + 7)
//   V^T tile [kBN / 8 pieces][d rows][8]   (piece c: keys 8c .. 8c + 7)
__host__ __device__ constexpr int ktile_elems(int d) { return kBN * d; }
__host__ __device__ constexpr int vtile_elems(int d) { return d * kBN; }
// element offset of piece c of key row r in a K tile
__host__ __device__ constexpr int kt_off(int r, int c) { return (c * kBN + r) * 8; }
// element offset of piece c (keys 8c ..) of row dd in a V^T tile of head size d
__host__ __device__ constexpr int vt_off(int d, int dd, int c) { return (c * d + dd) * 8; }

// Plan fields (per sequence s, written by the plan kernel).
enum PlanField {
    kPlanStart = 0,   // token of the sequence's first query row (cu_seqlens[s])
    kPlanLen = 1,     // L_s: keys of the sequence
    kPlanG = 2,       // G(L_s)
    kPlanPadOff = 3,  // first row of the sequence in the padded key layout (multiple of kBN)
    kPlanLoOff = 4,   // first row in the padded "lo" layout (multiple of kBN)
    kPlanTile0 = 5,   // kPlanPadOff / kBN
    kPlanLoTile0 = 6, // kPlanLoOff / kBN
    kPlanBad = 7,     // nonzero in entry n_seqs if cu_seqlens broke its contract
    kPlanQ0 = 8,      // position of the first query row: 0, or L_s - C_s for a chunk of
                      // C_s new rows appended to a cache
    kPlanKeep = 9     // chunk calls: leading key tiles whose workspace images an earlier
                      // call built and that are still valid (the pre-pass skips them)
};

// Record of the key/value images a chunk call leaves in its workspace (read
// by the next call that opts into reusing them): uint64 magic word, uint64
// fingerprint of everything the images depend on besides the cache rows and
// the lengths, then int32 [batch][2]: the key count L and group size G each
// sequence's images were built for (L = 0: none).  Every image row below L
// was built from the cache rows that call saw.
constexpr uint64_t kImageMagic = 0x4a4c494d47535431ULL;
__host__ __device__ constexpr size_t image_state_bytes(int32_t batch) {
    return 16 + 8 * (size_t)batch;
}

// ---------------------------------------------------------------------------
// Index math ([BT] §3.1, [TW] §二).  Integer only, so host and device agree
// bit for bit.

// G = max(1, ceil(L / w_pretrained)), L >= 0, w_pretrained >= 1.
__host__ __device__ inline int64_t group_size(int64_t L, int64_t w_pretrained) {
    int64_t g = (L + w_pretrained - 1) / w_pretrained;
    return g < 1 ? 1 : g;
}

// f(x) = floor(x / G) for x >= 0.
__host__ __device__ inline int32_t remap(int32_t x, int32_t G) { return x / G; }

// Band of (query i, key j): 0 masked (j > i), 1 local (0 <= i - j < w_local),
// 2 remote.  `bif` is false when the bifocal logic is off or G == 1 (then
// remapped and standard RoPE coincide and every unmasked pair is local).
__host__ __device__ inline int band(int64_t i, int64_t j, int64_t w_local, bool bif) {
    if (j > i) return 0;
    if (!bif) return 1;
    return (i - j < w_local) ? 1 : 2;
}

// Class bits of the block rows [i0, i1) x keys [j0, j1) (both non-empty):
// bit 0: holds a local pair, bit 1: a remote pair, bit 2: a masked pair.
// 0 means every pair is masked.  Derived from the extreme distances: the
// unmasked distances i - j span [max(0, i0 - (j1 - 1)), (i1 - 1) - j0].
enum { kHasLocal = 1, kHasRemote = 2, kHasMasked = 4 };
__host__ __device__ inline uint32_t tile_class(int64_t i0, int64_t i1, int64_t j0, int64_t j1,
                                               int64_t w_local, bool bif) {
    if (j0 > i1 - 1) return 0;
    uint32_t c = (j1 - 1 > i0) ? kHasMasked : 0u;
    const int64_t dmax = (i1 - 1) - j0;
    const int64_t dmin = (i0 - (j1 - 1)) > 0 ? (i0 - (j1 - 1)) : 0;
    if (!bif) return c | kHasLocal;
    if (dmin < w_local) c |= kHasLocal;
    if (dmax >= w_local) c |= kHasRemote;
    return c;
}

__host__ __device__ inline uint32_t tile_class32(int32_t i0, int32_t i1, int32_t j0, int32_t j1,
                                                 int32_t w_local, bool bif) {
    if (j0 > i1 - 1) return 0;
    uint32_t c = (j1 - 1 > i0) ? kHasMasked : 0u;
    const int32_t dmax = (i1 - 1) - j0;
    const int32_t dmin = (i0 - (j1 - 1)) > 0 ? (i0 - (j1 - 1)) : 0;
    if (!bif) return c | kHasLocal;
    if (dmin < w_local) c |= kHasLocal;
    if (dmax >= w_local) c |= kHasRemote;
    return c;
}

// ---------------------------------------------------------------------------
// RoPE angles.  theta_t = base^(-2t/d) is formed on the device as
// exp2(t * c), c = -2 log2(base) / d (fp64), and used in revolutions
// (theta_t / 2pi).  The angle p * theta_t is reduced modulo one revolution in
// fp64, so sin/cos see |arg| <= pi and keep fp32 accuracy for any position
// below 2^31.
struct RopeFreq {
    double c;  // -2 log2(base) / d
};

__device__ __forceinline__ double rope_rev(const RopeFreq& f, int t) {
    return exp2(f.c * (double)t) * 0.15915494309189533576888376337251;
}

__device__ __forceinline__ void rope_cs(int64_t p, double rev_t, float& c, float& s) {
    double x = (double)p * rev_t;
    x -= rint(x);
    const float a = (float)(x * 6.283185307179586476925286766559);
    sincosf(a, &s, &c);
}

// Angle given directly in revolutions (any real position times theta_t / 2pi),
// reduced in fp64, through the hardware sine and cosine.
__device__ __forceinline__ void rope_cs_rev(double x, float& c, float& s) {
    x -= rint(x);
    const float r = (float)x;
    s = __builtin_amdgcn_sinf(r);
    c = __builtin_amdgcn_cosf(r);
}

// Same angle through the hardware sine and cosine (v_sin_f32 / v_cos_f32 take
// their argument in revolutions); used where many angles are needed per key.
__device__ __forceinline__ void rope_cs_hw(int64_t p, double rev_t, float& c, float& s) {
    double x = (double)p * rev_t;
    x -= rint(x);
    const float r = (float)x;
    s = __builtin_amdgcn_sinf(r);
    c = __builtin_amdgcn_cosf(r);
}

}  // namespace jl
