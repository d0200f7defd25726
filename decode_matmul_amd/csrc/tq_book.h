// Code book and trit arithmetic shared by the ternary GEMV kernels.
//
// Format: pack-unpack-run, "Five trits in a byte": a byte b = d0 + 3 d1 +
// 9 d2 + 27 d3 + 81 d4 holds five base-3 digits, least significant first,
// and trit t = d - 1.  The kernels multiply by 2t (exact in bf16 and fp16)
// and halve the sum at the end.
#pragma once

#include "common.h"

namespace dmm {

typedef unsigned short u16x2v __attribute__((ext_vector_type(2)));

// Trit 4 (floor(b / 81)) of two code bytes held in the low bytes of the two
// 16-bit halves, as a bf16 pair of 2 t4: with v = 203 b + 0xC000 (mod 2^16)
// bits 14..15 hold the digit + 3 (mod 4), since floor(203 b / 2^14) =
// floor(b / 81) for b <= 242, so the masked value is 0xC000 (-2), 0 or 0x4000.
__device__ __forceinline__ uint32_t t4pair(uint32_t bytes16) {
    u16x2v v = __builtin_bit_cast(u16x2v, bytes16);
    v = v * (u16x2v){203, 203} + (u16x2v){0xC000, 0xC000};
    return __builtin_bit_cast(uint32_t, v) & 0xC000C000u;
}

// bf16 high byte of 2t for a base-3 digit d (t = d - 1)
__device__ __forceinline__ uint32_t trit_hb(uint32_t d) { return d == 2u ? 0x40u : (d == 0u ? 0xC0u : 0u); }

// Code book: entry e (a byte) holds its trits 0..3 as bf16 pairs of 2t; 32
// copies, entry e copy c at (e << 8) | (c << 3) (64 KB).  A 1024-thread
// workgroup fills it: thread tid fills copies 8 (tid & 3) .. + 7 of entry
// tid / 4 with four 16-byte stores, rotated by tid / 4 so that the lanes of
// a store spread over the banks.
__device__ __forceinline__ void fill_book(unsigned char* lut, int tid) {
    const uint32_t e = (uint32_t)(tid >> 2);
    // digits by exact division: floor(v / 3) = (171 v) >> 9 for v < 256
    const uint32_t q1 = (e * 171u) >> 9, q2 = (q1 * 171u) >> 9, q3 = (q2 * 171u) >> 9;
    const uint32_t d0 = e - 3u * q1, d1 = q1 - 3u * q2, d2 = q2 - 3u * q3;
    const uint32_t d3 = q3 - 3u * ((q3 * 171u) >> 9);
    const bool valid = e < 243u;                   // bytes 243..255 decode to zero
    const uint32_t e0 = valid ? (trit_hb(d0) << 8) | (trit_hb(d1) << 24) : 0u;
    const uint32_t e1 = valid ? (trit_hb(d2) << 8) | (trit_hb(d3) << 24) : 0u;
    const u32x4 v = {e0, e1, e0, e1};
    unsigned char* d = lut + ((e << 8) | (64u * (tid & 3)));
#pragma unroll
    for (int c = 0; c < 4; ++c) *(u32x4*)(d + 16 * ((c + (tid >> 2)) & 3)) = v;
}

}  // namespace dmm
