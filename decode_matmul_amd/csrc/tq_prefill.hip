// Ternary prefill (dense, G = 64, one or two planes, many tokens):
// y = x (s1 T1 + s2 T2)^T as an MFMA GEMM whose weight tiles are decoded from
// the packed trits into LDS.
//
// Format: "Does your weight format deserve a kernel?" (pack-unpack-run),
// "Five trits in a byte" (trit 5i + q of a group is digit q of byte i, least
// significant first, t = d - 1) and "Three values and a shared scale" (w =
// s t with one fp16 s per group of 64); the second plane follows the FUCINA
// README ("The method": W ~ d1 T1 + d2 T2), each plane its own K-slice.
//
// Numerics.  The products run on fp16 MFMAs with fp32 accumulation:
//  * A weight s t (t in {-1, 0, +1}, s an fp16 scale) is an fp16 value, so
//    the decoded tile holds the exact weights and the group scale needs no
//    separate multiply (one K-slice is one group).
//  * bf16 activations are converted to fp16 exactly when 2^-17 <= |x| <=
//    65280 or x = 0.  An 8-value chunk outside that range enters the fp16
//    pass as zeros and is added afterwards on bf16 MFMAs in two passes, against
//    hi = bf16(s t) and lo = bf16(s t - hi) (together exact: an fp16 value has
//    11 significant bits).  So every input meets the bound.
//
// Mapping onto gfx950:
//  * A 512-thread workgroup (8 waves in a 2 x 4 grid, two per SIMD) owns a
//    128 x 256 tile of y (tokens x rows); each wave owns 64 x 64 = 2 x 2 MFMA
//    32x32x16 tiles.
//  * K-slices of 64 (one group of one plane; with two planes, slice 2g + q is
//    plane q of group g over the same activations) in two LDS buffers: while the MFMAs of slice s
//    run, slice s + 1 (loaded from global memory an iteration earlier) is
//    decoded into the other buffer and slice s + 2 is loaded.  One barrier per
//    slice.
//  * Decode: thread t owns row t % 256 and half t / 256 of the group (a
//    wave-uniform half, so the trit-to-byte mapping is a compile-time pattern):
//    7 code bytes (bytes 0..6 or 6..12), each looked up in a 16-copy table of
//    the five trits' fp16 high bytes, v_perm pairs of fp16 t, and one packed
//    fp16 multiply by (s, s) per pair.
//  * Tile rows are 144 bytes apart, so 16 lanes reading 16 bytes of 16
//    consecutive rows cover all 64 banks.
#include "common.h"

namespace dmm {

namespace {

constexpr int BM = 128, BN = 256, BK = 64;     // BK = G: one group per K-slice
constexpr int kThreads = 512;
constexpr int kWN = 4;                         // waves along N (2 along M)
constexpr int MT = 2, NT = 2;                  // 32x32 MFMA tiles per wave along M and N
constexpr int kNB = 13;                        // code bytes per group
constexpr int kPitch = 2 * BK + 16;            // bytes per LDS tile row
constexpr int kXTile = BM * kPitch;
constexpr int kWTile = BN * kPitch;
constexpr int kBuf = kXTile + kWTile;          // one buffer: activations, then weights
constexpr int kLutBytes = 256 * 128;           // entry b, copy c at (b << 7) | (c << 3)
constexpr int kMapSlices = 1024;               // slices tracked one by one (K <= 65536)
constexpr int kSmemBytes = kLutBytes + 2 * kBuf + 64 + 8 * (kMapSlices + 1);
static_assert(kSmemBytes <= 160 * 1024, "LDS");
static_assert(kMapSlices * 2 <= kXTile, "the slice list fits buffer 1's activation tile");

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

struct Params {
    const uint16_t* x;
    int64_t M, K, N;
    int ng;                        // groups per row (K / 64)
    int planes;                    // 1 or 2
    const uint8_t* codes;          // plane 1 [N][ng][13]
    const uint16_t* scales;        // plane 1 [N][ng] fp16 bits
    const uint8_t* codes2;         // plane 2 (planes == 2)
    const uint16_t* scales2;
    void* y;
    int y_dtype;
    // pre-converted activations (tq_matmul_ws): fp16 x with the chunks fp16
    // cannot hold zeroed, and per (128-row block, group) a flag that the group
    // holds such a chunk; NULL when the kernel converts x itself
    const uint16_t* xf;
    const uint32_t* xflags;        // [ceil(M / 128)][ng]
};

// Per-thread loads of one K-slice: 2 chunks of 8 activations; 7 code bytes
// of one (row, group half) as three aligned words and a byte shift; the scale.
struct Slice {
    u32x4 xa[2];
    uint32_t cw[3];
    uint32_t sh;
    uint32_t sc;
};

// fp16 high byte of the trit of base-3 digit d (t = d - 1).
__device__ __forceinline__ uint32_t trit_f16_hi(int d) {
    return d == 2 ? 0x3Cu : (d == 0 ? 0xBCu : 0x00u);
}

// Pairs (trits 32h + 2p, 32h + 2p + 1) of fp16 t from the looked-up bytes:
// El[i] holds the high bytes of digits 0..3 of byte i of the half, Eh[i] of
// digit 4; the half's byte 0 is group byte 6h.
template <int H>
__device__ __forceinline__ void trit_pairs(const uint32_t* El, const uint32_t* Eh, uint32_t* P) {
#pragma unroll
    for (int p = 0; p < 16; ++p) {
        const int ja = 32 * H + 2 * p, jb = ja + 1;
        const int ia = ja / 5 - 6 * H, qa = ja % 5, ib = jb / 5 - 6 * H, qb = jb % 5;
        const uint32_t ra = qa < 4 ? El[ia] : Eh[ia];
        const uint32_t rb = qb < 4 ? El[ib] : Eh[ib];
        const uint32_t ba = qa < 4 ? (uint32_t)qa : 0u, bb = qb < 4 ? (uint32_t)qb : 0u;
        const bool same = (ia == ib) && ((qa < 4) == (qb < 4));
        // bytes: 0, hi(a), 0, hi(b)
        P[p] = same ? perm_b32(ra, ra, 0x0cu | (ba << 8) | (0x0cu << 16) | (bb << 24))
                    : perm_b32(rb, ra, 0x0cu | (ba << 8) | (0x0cu << 16) | ((4u + bb) << 24));
    }
}

template <bool XF>
__global__ void __launch_bounds__(kThreads, 1) tq_prefill_kernel(Params p) {
    __shared__ __attribute__((aligned(16))) unsigned char smem[kSmemBytes];
    unsigned char* const lut = smem;
    unsigned char* const bufs = smem + kLutBytes;               // [2][x tile, w tile]
    unsigned char* const words = bufs + 2 * kBuf;
    int& redo_n = *(int*)(words);
    uint64_t* const bad_map = (uint64_t*)(words + 64);
    uint16_t* const redo = (uint16_t*)(bufs + kBuf);            // buffer 1's activation tile

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = readfirstlane(tid >> 6);
    const int wm = wave / kWN, wn = wave % kWN;
    const int H = wave >> 2;                                    // group half this wave decodes

    // ---- trit table: 16 copies; entries 243..255 decode to zero
    for (int i = tid; i < 256 * 16; i += kThreads) {
        const int b = i >> 4, c = i & 15;
        uint32_t lo = 0, hi = 0;
        if (b < 243) {
            const int d0 = b % 3, d1 = (b / 3) % 3, d2 = (b / 9) % 3, d3 = (b / 27) % 3, d4 = b / 81;
            lo = trit_f16_hi(d0) | (trit_f16_hi(d1) << 8) | (trit_f16_hi(d2) << 16) |
                 (trit_f16_hi(d3) << 24);
            hi = trit_f16_hi(d4);
        }
        *(uint2*)(lut + ((b << 7) | (c << 3))) = make_uint2(lo, hi);
    }
    if (tid == 0) redo_n = 0;
    for (int i = tid; i <= kMapSlices; i += kThreads) bad_map[i] = 0ull;

    const int64_t m0 = (int64_t)blockIdx.y * BM;
    const int64_t n0 = (int64_t)blockIdx.x * BN;
    const int nslices = p.ng * p.planes;
    const uint32_t cofs = (uint32_t)(lane & 15) << 4;           // >> 1 below: copy lane % 16

    // this thread's activation chunks (rows xr_i, 8 values at column xc) and
    // weight row / half
    const int xr0 = tid >> 3, xc = (tid & 7) * 8;               // chunk i: row xr0 + 64 i
    const int wr = tid & 255;
    const int64_t wrow = min(n0 + wr, p.N - 1);
    const int64_t row_bytes = (int64_t)p.ng * kNB;

    // from_xf: the fp16 pass of a call with pre-converted activations
    auto gload = [&](int s, Slice& S, bool from_xf) {
        const int sc = min(s, nslices - 1);
        const int g = p.planes == 2 ? sc >> 1 : sc;
        const bool second = p.planes == 2 && (sc & 1);
        const uint8_t* codes = second ? p.codes2 : p.codes;
        const uint16_t* scales = second ? p.scales2 : p.scales;
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int64_t m = min(m0 + xr0 + 64 * i, p.M - 1);
            S.xa[i] = *(const u32x4*)(((XF && from_xf) ? p.xf : p.x) + m * p.K + (int64_t)g * BK + xc);
        }
        const int64_t off = wrow * row_bytes + (int64_t)g * kNB + 6 * H;   // 7 bytes
        const int64_t a0 = off & ~(int64_t)3;
        const int64_t a2 = (off + 6) & ~(int64_t)3;                        // word of the last byte
        S.cw[0] = *(const uint32_t*)(codes + a0);
        S.cw[1] = *(const uint32_t*)(codes + a0 + 4);
        S.cw[2] = *(const uint32_t*)(codes + a2);
        S.sh = (uint32_t)(off & 3);
        S.sc = scales[wrow * p.ng + g];
    };

    // fp16 pairs of t for this thread's 32 trits
    auto decode_pairs = [&](const Slice& S, uint32_t* P) {
        const uint32_t w2 = S.cw[2];
        const uint32_t D0 = align_bytes(S.cw[1], S.cw[0], S.sh);
        const uint32_t D1 = align_bytes(w2, S.cw[1], S.sh);
        uint32_t El[7], Eh[7];
#pragma unroll
        for (int i = 0; i < 7; ++i) {
            const uint32_t a =
                perm_b32(i < 4 ? D0 : D1, cofs, 0x0c0c0400u + ((uint32_t)(i & 3) << 8)) >> 1;
            const uint2 e = *(const uint2*)(lut + a);
            El[i] = e.x;
            Eh[i] = e.y;
        }
        if (H == 0) trit_pairs<0>(El, Eh, P);
        else trit_pairs<1>(El, Eh, P);
    };

    // fp16 activations and weights of a slice into buffer buf.  A chunk of 8
    // activations outside the exact range is written as zeros and counted
    // for the bf16 pass.
    auto store_f16 = [&](int s, int buf, const Slice& S) {
        unsigned char* X = bufs + buf * kBuf;
        unsigned char* Wt = X + kXTile;
        if constexpr (XF) {
            // converted and flagged by the pre-pass (the replay list reads its flags)
#pragma unroll
            for (int i = 0; i < 2; ++i) *(u32x4*)(X + (xr0 + 64 * i) * kPitch + 2 * xc) = S.xa[i];
        } else {
            int nbad = 0;
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                Range R;
                u32x4 v;
#pragma unroll
                for (int w = 0; w < 4; ++w) v[w] = bf16x2_to_f16x2(S.xa[i][w], R);
                const bool bad = !range_ok(R);
                nbad += bad;
#pragma unroll
                for (int w = 0; w < 4; ++w) v[w] = bad ? 0u : v[w];
                *(u32x4*)(X + (xr0 + 64 * i) * kPitch + 2 * xc) = v;
            }
            const bool wbad = __builtin_amdgcn_ballot_w64(nbad != 0) != 0;
            unsigned char* fb = (unsigned char*)&bad_map[min(s, kMapSlices)] + wave;
            *fb = (unsigned char)((s >= kMapSlices ? *fb : 0) | (wbad ? 1 : 0));
        }
        uint32_t P[16];
        decode_pairs(S, P);
        const f16x2 s2 = {__builtin_bit_cast(_Float16, (uint16_t)S.sc),
                          __builtin_bit_cast(_Float16, (uint16_t)S.sc)};
        u32x4 o[4];
#pragma unroll
        for (int q = 0; q < 16; ++q)
            o[q >> 2][q & 3] = __builtin_bit_cast(uint32_t, __builtin_bit_cast(f16x2, P[q]) * s2);
        unsigned char* dst = Wt + wr * kPitch + 64 * H;
#pragma unroll
        for (int q = 0; q < 4; ++q) *(u32x4*)(dst + 16 * q) = o[q];
    };

    // the bf16 pass: raw bf16 activations of the chunks the fp16 pass left
    // out (zeros elsewhere) and the bf16 hi (part 0) or lo (part 1) weights
    auto store_bf16 = [&](const Slice& S) {
        unsigned char* X = bufs;
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            Range R;
#pragma unroll
            for (int w = 0; w < 4; ++w) (void)bf16x2_to_f16x2(S.xa[i][w], R);
            const bool bad = !range_ok(R);
            u32x4 v;
#pragma unroll
            for (int w = 0; w < 4; ++w) v[w] = bad ? S.xa[i][w] : 0u;
            *(u32x4*)(X + (xr0 + 64 * i) * kPitch + 2 * xc) = v;
        }
        uint32_t P[16];
        decode_pairs(S, P);
        const float sf = f16_bits_to_f32((uint16_t)S.sc);
        const uint32_t hb = f32_to_bf16_rne(sf);
        const uint32_t lb = f32_to_bf16_rne(sf - bf16_bits_to_f32((uint16_t)hb));
        const uint32_t hb2 = hb * 0x10001u, lb2 = lb * 0x10001u;
        u32x4 oh[4], ol[4];
#pragma unroll
        for (int q = 0; q < 16; ++q) {
            // t halves are 0x3C00 (+1), 0xBC00 (-1) or 0: a full mask where t != 0
            const uint32_t mask = ((P[q] >> 10) & 0x000F000Fu) * 0x1111u;
            const uint32_t sign = P[q] & 0x80008000u;
            oh[q >> 2][q & 3] = (mask & hb2) ^ (sign & (mask & 0x80008000u));
            ol[q >> 2][q & 3] = (mask & lb2) ^ (sign & (mask & 0x80008000u));
        }
        unsigned char* dh = bufs + kXTile + wr * kPitch + 64 * H;            // buffer 0 weights
        unsigned char* dl = bufs + kBuf + kXTile + wr * kPitch + 64 * H;     // buffer 1 weights
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            *(u32x4*)(dh + 16 * q) = oh[q];
            *(u32x4*)(dl + 16 * q) = ol[q];
        }
    };

    // accumulators start life in the accumulation registers
    f32x16 acc[MT][NT];
#pragma unroll
    for (int i = 0; i < MT; ++i)
#pragma unroll
        for (int jn = 0; jn < NT; ++jn) {
            f32x16 z;
#pragma unroll
            for (int r = 0; r < 16; ++r) z[r] = 0.f;
            asm volatile("" : "+a"(z));
            acc[i][jn] = z;
        }

    // A fragment: lane l holds A[l % 32][8 (l / 32) .. +7] of a 16-wide
    // K-step; B alike with the rows of the weight tile.
    const int frow = lane & 31;
    const int fk = 16 * (lane >> 5);
    struct Frag {
        u32x4 a[MT];
        u32x4 b[NT];
    };
    auto load_frag = [&](int xbuf, int wbuf, int ks, Frag& F) {
        const unsigned char* A = bufs + xbuf * kBuf + (wm * 32 * MT + frow) * kPitch + fk + 32 * ks;
        const unsigned char* B =
            bufs + wbuf * kBuf + kXTile + (wn * 32 * NT + frow) * kPitch + fk + 32 * ks;
#pragma unroll
        for (int i = 0; i < MT; ++i) F.a[i] = *(const u32x4*)(A + i * 32 * kPitch);
#pragma unroll
        for (int jn = 0; jn < NT; ++jn) F.b[jn] = *(const u32x4*)(B + jn * 32 * kPitch);
    };
    auto mfma_frag = [&](const Frag& F, bool f16) {
#pragma unroll
        for (int i = 0; i < MT; ++i)
#pragma unroll
            for (int jn = 0; jn < NT; ++jn) {
                if (f16)
                    acc[i][jn] = __builtin_amdgcn_mfma_f32_32x32x16_f16(
                        __builtin_bit_cast(f16x8, F.a[i]), __builtin_bit_cast(f16x8, F.b[jn]),
                        acc[i][jn], 0, 0, 0);
                else
                    acc[i][jn] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                        __builtin_bit_cast(bf16x8, F.a[i]), __builtin_bit_cast(bf16x8, F.b[jn]),
                        acc[i][jn], 0, 0, 0);
            }
    };

    __syncthreads();                       // table and flags written

    // ---- fp16 pass: slice s is computed from buffer s & 1 while slice s + 1
    // is decoded into the other buffer and slice s + 2 is loaded
    Slice S;
    if (nslices > 0) {
        gload(0, S, true);
        store_f16(0, 0, S);
        gload(1, S, true);
    }
    __syncthreads();
#pragma unroll 1
    for (int s = 0; s < nslices; ++s) {
        const int buf = s & 1;
        if (s + 1 < nslices) store_f16(s + 1, buf ^ 1, S);
        gload(s + 2, S, true);             // clamped; unused past the end
        Frag F0, F1;
        load_frag(buf, buf, 0, F0);
        load_frag(buf, buf, 1, F1);
        mfma_frag(F0, true);
        load_frag(buf, buf, 2, F0);
        mfma_frag(F1, true);
        load_frag(buf, buf, 3, F1);
        mfma_frag(F0, true);
        mfma_frag(F1, true);
        __syncthreads();
    }

    // ---- bf16 pass over the chunks left out: flagged slices below
    // kMapSlices one by one, then every slice from kMapSlices on if any there
    // was flagged.  Activations and hi weights in buffer 0, lo weights in
    // buffer 1's weight tile.
    if (tid == 0) {
        int n = 0;
        const int mapped = min(nslices, kMapSlices);
        if constexpr (XF) {
            // the pre-pass flags of this 128-row block (one per group: both
            // planes of a group share its activations); later slices as one flag
            const uint32_t* fr = p.xflags + (int64_t)blockIdx.y * p.ng;
            for (int w = 0; w < mapped; ++w)
                if (fr[p.planes == 2 ? w >> 1 : w]) redo[n++] = (uint16_t)w;
            bool late = false;
            for (int w = kMapSlices; w < nslices; ++w) late = late || fr[p.planes == 2 ? w >> 1 : w] != 0u;
            bad_map[kMapSlices] = late ? 1ull : 0ull;
        } else
        for (int w = 0; w < mapped; ++w)
            if (bad_map[w]) redo[n++] = (uint16_t)w;
        redo_n = n;
    }
    __syncthreads();
    const int nlist = readfirstlane(redo_n);
    const int late_end = readfirstlane(bad_map[kMapSlices] != 0ull ? 1 : 0) ? nslices : kMapSlices;
    const int nreplay = nlist + max(late_end - kMapSlices, 0);
    auto replay_slice = [&](int r) {
        return r < nlist ? (int)readfirstlane(redo[r]) : kMapSlices + (r - nlist);
    };
    if (nreplay > 0) gload(replay_slice(0), S, false);
#pragma unroll 1
    for (int r = 0; r < nreplay; ++r) {
        store_bf16(S);
        __syncthreads();
        gload(replay_slice(min(r + 1, nreplay - 1)), S, false);
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            Frag F0, F1;
            load_frag(0, 0, ks, F0);
            mfma_frag(F0, false);
            load_frag(0, 1, ks, F1);
            mfma_frag(F1, false);
        }
        __syncthreads();
    }

    // ---- epilogue: C[m][n] of tile (i, jn) in register r of lane l is
    // m = 8 (r / 4) + 4 (l / 32) + r % 4, n = l % 32
#pragma unroll
    for (int jn = 0; jn < NT; ++jn) {
        const int64_t n = n0 + wn * 32 * NT + jn * 32 + (lane & 31);
        if (n >= p.N) continue;
#pragma unroll
        for (int i = 0; i < MT; ++i) {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int64_t m = m0 + wm * 32 * MT + i * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
                if (m >= p.M) continue;
                const float v = acc[i][jn][r];
                const int64_t idx = m * p.N + n;
                if (p.y_dtype == TQ_F32) ((float*)p.y)[idx] = v;
                else ((uint16_t*)p.y)[idx] = f32_to_bf16_rne(v);
            }
        }
    }
}

// Pre-pass of tq_matmul_ws: bf16 x -> fp16, once per call instead of once per
// N-tile workgroup (and per plane).  A workgroup converts rows 128 by,
// columns 128 bx (two groups); a chunk of 8 activations that fp16 cannot hold
// exactly becomes zeros, and a group's flag says whether any of its chunks
// in this row block did (the prefill replays that group in bf16).  Every
// flag word is written by exactly one workgroup.
constexpr int kXcCols = 128;
static_assert(kXcCols % BK == 0 && BM == 128, "flags per prefill row block and group");
__global__ void __launch_bounds__(256) tq_xconv_kernel(const uint16_t* __restrict__ x, int64_t M,
                                                      int64_t K, int ng, uint16_t* __restrict__ xf,
                                                      uint32_t* __restrict__ flags) {
    __shared__ uint32_t fl[kXcCols / BK];
    const int tid = threadIdx.x;
    if (tid < kXcCols / BK) fl[tid] = 0u;
    __syncthreads();
    const int64_t m0 = (int64_t)blockIdx.y * BM;
    const int cc = tid & 15;                              // chunk of 8 columns
    const int64_t col = (int64_t)blockIdx.x * kXcCols + 8 * cc;
    bool bad_any = false;
    if (col < K) {                                        // K % 64 == 0: chunks are whole
#pragma unroll 4
        for (int i = 0; i < BM / 16; ++i) {
            const int64_t m = m0 + (tid >> 4) + 16 * i;
            if (m < M) {
                const u32x4 v = *(const u32x4*)(x + m * K + col);
                Range R;
                u32x4 o;
#pragma unroll
                for (int w = 0; w < 4; ++w) o[w] = bf16x2_to_f16x2(v[w], R);
                const bool bad = !range_ok(R);
#pragma unroll
                for (int w = 0; w < 4; ++w) o[w] = bad ? 0u : o[w];
                *(u32x4*)(xf + m * K + col) = o;
                bad_any = bad_any || bad;
            }
        }
    }
    if (bad_any) atomicOr(&fl[cc >> 3], 1u);              // group (col mod 128) / 64
    __syncthreads();
    if (tid < kXcCols / BK) {
        const int64_t g = (int64_t)blockIdx.x * (kXcCols / BK) + tid;
        if (g < ng) flags[(int64_t)blockIdx.y * ng + g] = fl[tid];
    }
}

}  // namespace

// Dense ternary matmul for many tokens; false (nothing launched) outside its
// domain: G = 64, M >= 128, x 16-byte and codes 4-byte aligned, K / 64 * planes
// slices within the LDS flag map's index range, a grid within the launch limits.
bool launch_tq_prefill(const TqMatmulArgs& a, hipStream_t s, hipError_t* err) {
    if (a.n_experts != 0 || a.G != 64 || a.M < BM || a.K < BK || a.K % BK != 0 ||
        ((uintptr_t)a.x & 15) != 0 || ((uintptr_t)a.codes[0] & 3) != 0 ||
        ((uintptr_t)a.scales[0] & 1) != 0)
        return false;
    if (a.planes == 2 && (((uintptr_t)a.codes[1] & 3) != 0 || ((uintptr_t)a.scales[1] & 1) != 0))
        return false;
    if ((a.K / BK) * a.planes >= (1ll << 30)) return false;
    const int64_t gx = (a.N + BN - 1) / BN, gy = (a.M + BM - 1) / BM;
    if (gx == 0 || gx >= (1ll << 31) || gy >= 65536) return false;
    Params p;
    p.x = a.x;
    p.M = a.M;
    p.K = a.K;
    p.N = a.N;
    p.ng = (int)(a.K / BK);
    p.planes = a.planes;
    p.codes = a.codes[0];
    p.scales = a.scales[0];
    p.codes2 = a.planes == 2 ? a.codes[1] : a.codes[0];
    p.scales2 = a.planes == 2 ? a.scales[1] : a.scales[0];
    p.y = a.y;
    p.y_dtype = a.y_dtype;
    p.xf = nullptr;
    p.xflags = nullptr;
    if (a.workspace) {
        // activations converted once for the whole call
        uint16_t* xf = (uint16_t*)a.workspace;
        uint32_t* fl = (uint32_t*)((char*)a.workspace + tq_prefill_ws_flags_offset(a.M, a.K));
        hipLaunchKernelGGL(tq_xconv_kernel, dim3((unsigned)((a.K + kXcCols - 1) / kXcCols), (unsigned)gy),
                           dim3(256), 0, s, a.x, a.M, a.K, p.ng, xf, fl);
        *err = hipGetLastError();
        if (*err != hipSuccess) return true;
        p.xf = xf;
        p.xflags = fl;
        hipLaunchKernelGGL(tq_prefill_kernel<true>, dim3((unsigned)gx, (unsigned)gy), dim3(kThreads), 0, s, p);
    } else {
        hipLaunchKernelGGL(tq_prefill_kernel<false>, dim3((unsigned)gx, (unsigned)gy), dim3(kThreads), 0, s, p);
    }
    *err = hipGetLastError();
    return true;
}

}  // namespace dmm
