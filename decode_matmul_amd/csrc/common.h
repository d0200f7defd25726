// Device helpers and internal launcher declarations of the packed-code
// matmul library (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "decode_matmul.h"

namespace dmm {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x3 __attribute__((ext_vector_type(3)));
// 16-byte vectors loaded from 4-byte aligned addresses.
typedef uint32_t u32x4a __attribute__((ext_vector_type(4), aligned(4)));
typedef uint32_t u32x3a __attribute__((ext_vector_type(3), aligned(4)));
// 16-byte vectors of activations at any element offset (2-byte aligned): the
// hardware serves unaligned global loads, so this is still one dwordx4 load.
typedef uint32_t u32x4h __attribute__((ext_vector_type(4), aligned(2)));

// ------------------------------------------------------------ conversions

__device__ __forceinline__ float f16_bits_to_f32(uint16_t h) {
    return (float)__builtin_bit_cast(_Float16, h);   // exact
}

__device__ __forceinline__ float bf16_bits_to_f32(uint16_t h) {
    return __builtin_bit_cast(float, (uint32_t)h << 16);
}

// fp32 -> bf16, nearest-even (NaN stays a quiet NaN).
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
    uint32_t u = __builtin_bit_cast(uint32_t, f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);
    u += 0x7fffu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

// float64 -> fp16 bits, nearest-even, one rounding straight from the
// float64 value (integer arithmetic on the bit pattern).
__device__ __forceinline__ uint16_t f64_to_f16_rne(double x) {
    uint64_t b = __builtin_bit_cast(uint64_t, x);
    uint32_t sign = (uint32_t)(b >> 48) & 0x8000u;
    uint64_t a = b & 0x7fffffffffffffffull;
    if (a >= 0x7ff0000000000000ull)                       // inf or nan
        return (uint16_t)(sign | (a > 0x7ff0000000000000ull ? 0x7e00u : 0x7c00u));
    int e = (int)(a >> 52) - 1023;                         // binade of |x|
    if (e > 15) return (uint16_t)(sign | 0x7c00u);         // >= 2^16
    if (e < -25) return (uint16_t)sign;                    // < 2^-25 -> 0
    uint64_t m = (a & 0x000fffffffffffffull) | 0x0010000000000000ull;
    // spacing of fp16 at this binade: 2^(e-10) for normals, 2^-24 below 2^-14
    int s = (e >= -14) ? 42 : (28 - e);                    // 42..53
    uint64_t q = m >> s;
    uint64_t rem = m & ((1ull << s) - 1ull);
    uint64_t half = 1ull << (s - 1);
    if (rem > half || (rem == half && (q & 1ull))) q += 1ull;
    uint32_t bits = (e >= -14) ? (((uint32_t)(e + 15) << 10) + (uint32_t)(q - 1024ull))
                               : (uint32_t)q;              // carries roll into exponent
    return (uint16_t)(sign | bits);
}

// ------------------------------------------------------------ small ops

__device__ __forceinline__ uint32_t perm_b32(uint32_t hi, uint32_t lo, uint32_t sel) {
    return __builtin_amdgcn_perm(hi, lo, sel);
}

// A code-book entry as two bf16 terms packed in one dword: hi = bf16(v) in
// the low half, lo = bf16(v - hi) in the high half (v - hi is exact, and
// |v - hi - lo| <= 2^-17 |v|).
__device__ __forceinline__ uint32_t split_bf16_pair(float v) {
    const uint16_t hi = f32_to_bf16_rne(v);
    const float r = v - bf16_bits_to_f32(hi);
    const uint16_t lo = f32_to_bf16_rne(r);
    return (uint32_t)hi | ((uint32_t)lo << 16);
}

// Bytes [sh, sh+4) of the 8-byte little-endian value {hi:lo}, sh in 0..3.
__device__ __forceinline__ uint32_t align_bytes(uint32_t hi, uint32_t lo, uint32_t sh) {
    return __builtin_amdgcn_alignbyte(hi, lo, sh);
}

__device__ __forceinline__ void atomic_or_status(int32_t* st, int32_t flag) {
    if (st) atomicOr(st, flag);
}

// ------------------------------------------------- bf16 -> fp16 activations
// (used by the MFMA prefill kernels, which multiply in fp16)

typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));

// Running range of the activations of one chunk (bf16 bits with the sign
// cleared, two halves per word): the largest value, and the smallest
// nonzero value minus one (a zero wraps to 0xffff and drops out).
struct Range {
    u16x2 hi = {0, 0};
    u16x2 lo = {0xffff, 0xffff};
};

// Two bf16 activations -> two fp16 (exact inside the range that R checks).
__device__ __forceinline__ uint32_t bf16x2_to_f16x2(uint32_t d, Range& R) {
    const u16x2 t = __builtin_bit_cast(u16x2, d & 0x7fff7fffu);
    R.hi = __builtin_elementwise_max(R.hi, t);
    R.lo = __builtin_elementwise_min(R.lo, (u16x2)(t - (u16x2){1, 1}));
    const float a = __builtin_bit_cast(float, d << 16);
    const float b = __builtin_bit_cast(float, d & 0xffff0000u);
    return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(a, b));
}

// True when every activation seen is 0 or has 2^-17 <= |x| <= 65280
// (bf16 bits 0x3700 .. 0x477f), i.e. is exact in fp16.
__device__ __forceinline__ bool range_ok(const Range& R) {
    return max(R.hi.x, R.hi.y) <= 0x477f && min(R.lo.x, R.lo.y) >= 0x36ff;
}

// Prefill replays: the 32-row MFMA tiles (bit i) holding a chunk flagged by
// any of 8 converting waves, wave v's flag in byte v of f.  Converting wave v
// covers rows 16 v .. 16 v + 15 of each 128-row half, tile v / 2 of that half.
__device__ __forceinline__ uint32_t flag_tiles(uint64_t f) {
    uint32_t t = 0u;
#pragma unroll
    for (int v = 0; v < 8; ++v) t |= (((f >> (8 * v)) & 0xffull) != 0ull ? 1u : 0u) << (v >> 1);
    return t;
}

// Row block of workgroup bx in a grid of nb: consecutive workgroups go to
// the 8 XCDs in turn, so when nb is a multiple of 8 each XCD is given one
// contiguous range of blocks (its L2 and TLB then see an eighth of the
// matrix); other grids keep the plain order.
__device__ __forceinline__ int64_t xcd_block(int64_t bx, int64_t nb) {
    return (nb % 8 == 0) ? (bx % 8) * (nb / 8) + bx / 8 : bx;
}

// Wave-uniform read of an SGPR-able value.
__device__ __forceinline__ int readfirstlane(int v) {
    return __builtin_amdgcn_readfirstlane(v);
}

}  // namespace dmm

// ------------------------------------------------------------ launchers
// Each returns hipSuccess or the launch error; arguments were validated by
// the C entry points.

namespace dmm {

hipError_t launch_status_clear(int32_t* d_status, hipStream_t s);

hipError_t launch_pack(const float* W, int64_t rows, int64_t K, int G, int planes,
                       uint8_t* c1, uint16_t* s1, uint8_t* c2, uint16_t* s2,
                       int32_t* d_status, hipStream_t s);

hipError_t launch_unpack(const uint8_t* codes, const uint16_t* scales, int64_t rows,
                         int64_t K, int G, void* out, int out_dtype, int32_t* d_status,
                         hipStream_t s);

struct TqMatmulArgs {
    const uint16_t* x;
    int64_t M, K, N;
    const uint8_t* codes[2];
    const uint16_t* scales[2];
    int planes;
    int G;
    int n_experts;          // 0 = dense
    int e_begin, e_end;     // grouped: the experts this launch computes
    bool nan_rows;          // grouped: this launch writes the rows of invalid ids
    const int32_t* ids;     // [M, top_k] when grouped
    int top_k;
    void* y;
    int y_dtype;
    void* workspace;        // NULL, or tq_prefill_ws_bytes(M, K) bytes for the dense
                            // prefill's pre-converted activations
};

// Workspace of a ternary prefill with pre-converted activations: fp16 x
// [M][K], then at a 256-byte boundary one flag word per (128-row block,
// group of 64 columns).
inline int64_t tq_prefill_ws_flags_offset(int64_t M, int64_t K) { return (M * K * 2 + 255) / 256 * 256; }
inline int64_t tq_prefill_ws_bytes(int64_t M, int64_t K) {
    return tq_prefill_ws_flags_offset(M, K) + (M + 127) / 128 * ((K + 63) / 64) * 4;
}

// Compute units of the current device (256 when the query fails), read once;
// kernels that place one workgroup per compute unit size their grids by it.
inline int compute_unit_count() {
    static const int cus = [] {
        int dev = 0, v = 0;
        if (hipGetDevice(&dev) == hipSuccess &&
            hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && v > 0)
            return v;
        return 256;
    }();
    return cus;
}

hipError_t launch_tq_matmul(const TqMatmulArgs& a, hipStream_t s);
// Streaming form for a few tokens (dense M <= 4, or <= 16 when the codes stay
// in LDS; grouped experts); false when the call is outside its domain.
bool launch_tq_rows(const TqMatmulArgs& a, hipStream_t s, hipError_t* err);
// Wave-local form for dense calls of 1..4 tokens and grouped calls of at
// most 256 (token, slot) pairs (G = 64, K = 1024..4096 in steps of 1024);
// false when the call is outside its domain.
bool launch_tq_wave(const TqMatmulArgs& a, hipStream_t s, hipError_t* err);
// Dense calls of 5..16 tokens on full-width MFMAs (one plane, G = 64,
// K = 256, 512, 1024, 2048 or 4096; x, codes and scales 4-byte aligned);
// false when the call is outside its domain.
bool launch_tq_batch(const TqMatmulArgs& a, hipStream_t s, hipError_t* err);
// A hot-prefix call (two-plane hot launch, one-plane cold launch that writes
// the invalid-id rows) as one wave-local launch; false outside its domain.
bool launch_tq_wave_hot(const TqMatmulArgs& hot, const TqMatmulArgs& cold, hipStream_t s,
                        hipError_t* err);
// A hot-prefix call (two-plane hot launch, one-plane cold launch that writes
// the invalid-id rows) as one streaming launch; false outside its domain.
bool launch_tq_rows_hot(const TqMatmulArgs& hot, const TqMatmulArgs& cold, hipStream_t s,
                        hipError_t* err);
// MFMA prefill form for many tokens (dense, one plane, G = 64, M >= 128).
bool launch_tq_prefill(const TqMatmulArgs& a, hipStream_t s, hipError_t* err);
int tq_max_grouped_pairs();  // largest M * top_k of a grouped call

struct RbMatmulArgs {
    const uint16_t* x;
    int64_t M, K, N;
    const uint8_t* codes;   // one byte per weight, or 7-bit indices when `used` is set
    const uint8_t* used;    // 7-bit form: index -> code, [128]; NULL for code bytes
    const float* table;     // [243], or [ceil(N / table_rows)][243]
    int64_t table_rows;     // 0: one code book; else rows per code book (a multiple of 32)
    float alpha;
    const uint16_t* row_scale;
    int64_t rho_rows;       // rows sharing one row_scale entry (>= 1)
    const float* bias;
    void* y;
    int y_dtype;
    void* workspace;        // NULL, or rb_prefill_ws_bytes(M, K) bytes for the prefill's
                            // pre-converted activations
};

// Workspace of a prefill with pre-converted activations: fp16 x [M][K], then
// at a 256-byte boundary one flag word per (256-row block, 32-wide K-slice).
inline int64_t rb_prefill_ws_flags_offset(int64_t M, int64_t K) { return (M * K * 2 + 255) / 256 * 256; }
inline int64_t rb_prefill_ws_bytes(int64_t M, int64_t K) {
    return rb_prefill_ws_flags_offset(M, K) + (M + 255) / 256 * ((K + 31) / 32) * 4;
}

// Library-owned scratch of rb_matmul_noalloc: one array per device, as large
// as the prefill workspace of M = 2048 tokens at K = 8192 plus room to spare.
constexpr int64_t kScratchBytes = DMM_SCRATCH_BYTES;
// Device address of the scratch array on the current device (looked up once
// per device, then cached).
hipError_t scratch_of_current_device(void** out);

// Bytes of one row of 7-bit indices.
inline int64_t rb7_row_bytes(int64_t K) { return (7 * K + 7) / 8; }

// Code book of the rows starting at row0 (table_rows is a multiple of 32, so
// a 16- or 32-row block of rows shares one).
__host__ __device__ inline const float* rb_table_of(const float* table, int64_t table_rows,
                                                    int64_t row0) {
    return table + (table_rows > 0 ? row0 / table_rows : 0) * 243;
}

hipError_t launch_rb_gemv(const RbMatmulArgs& a, hipStream_t s);
hipError_t launch_rb7_gemv(const RbMatmulArgs& a, hipStream_t s);
hipError_t launch_rb_prefill(const RbMatmulArgs& a, hipStream_t s);
hipError_t launch_rb_truncate(const uint8_t* codes, int64_t N, int64_t K, uint8_t* used,
                              int32_t* n_used, uint8_t* codes7, int32_t* status, hipStream_t s);
hipError_t launch_rb_encode(const float* W, int64_t N, int64_t K, const float* ladder, float zeta,
                            int64_t rho_rows, uint8_t* codes, float* alpha, uint16_t* row_scale,
                            int32_t* status, hipStream_t s);

}  // namespace dmm
