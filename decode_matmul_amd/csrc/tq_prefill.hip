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
//    separate multiply (a K-slice lies within one group).
//  * bf16 activations are converted to fp16 exactly when 2^-17 <= |x| <=
//    65280 or x = 0.  An 8-value chunk outside that range enters the fp16
//    pass as zeros and is added afterwards on bf16 MFMAs in two passes, against
//    hi = bf16(s t) and lo = bf16(s t - hi) (together exact: an fp16 value has
//    11 significant bits).  So every input meets the bound.
//
// Mapping onto gfx950:
//  * A 512-thread workgroup (8 waves in a 2 x 4 grid, two per SIMD) owns a
//    256 x 256 tile of y (tokens x rows); each wave owns 128 x 64 = 4 x 2 MFMA
//    32x32x16 tiles (128 fp32 accumulators per lane).
//  * K-slices of 32, half a group each: slice s is half s & 1 of group g of
//    plane q (one plane: g = s / 2; two planes: q = (s / 2) & 1, g = s / 4).
//    Two LDS buffers: while the MFMAs of slice s run from registers, the next
//    K-step's fragments are read and slice s + 2 (loaded from global memory
//    an iteration earlier) is decoded into the buffer slice s has just
//    vacated.  One barrier per slice.
//  * Decode: lanes 2 r and 2 r + 1 of wave w own tile row 32 w + r (so one
//    load instruction touches 32 rows' lines, not 64) and the 16 trits
//    16 u .. 16 u + 15 of the group, u = 2 h + (lane & 1) (h the slice's
//    half).  They are base-3 digits u .. u + 15 of the four code bytes
//    3 u .. 3 u + 3 read as one digit stream (byte i, digit d at position
//    5 i + d).  Each byte is looked up in a 32-copy table of its five digits'
//    fp16 high bytes; the 20 stream bytes are packed into five words and each
//    fp16 pair of t is one v_perm, so every (half, u) takes the same
//    instructions.  One packed fp16 multiply by (s, s) per pair gives the
//    weights.
//  * Tile rows are 80 bytes apart, so the 8 lanes of a 16-byte column read
//    cover distinct banks.
#include <type_traits>

#include "common.h"

namespace dmm {

namespace {

constexpr int BM = 256, BN = 256, BK = 32;     // BK: half a group of G = 64
constexpr int G = 64;
constexpr int kThreads = 512;
constexpr int kWN = 4;                         // waves along N (2 along M)
constexpr int MT = 4, NT = 2;                  // 32x32 MFMA tiles per wave along M and N
constexpr int kNB = 13;                        // code bytes per group
constexpr int kPitch = 2 * BK + 16;            // bytes per LDS tile row
constexpr int kTileBytes = BM * kPitch;        // one operand tile (BM == BN)
constexpr int kLutBytes = 256 * 256;           // entry b, copy c at (b << 8) | (c << 3)
constexpr int kMapSlices = 1536;               // slices tracked one by one
constexpr int kFlagRows = 128;                 // rows per pre-pass flag block
constexpr int kSmemBytes = kLutBytes + 4 * kTileBytes + 64 + 8 * (kMapSlices + 2);
static_assert(kSmemBytes <= 160 * 1024, "LDS");
static_assert(kMapSlices * 2 <= kTileBytes,
              "the slice list fits the activation tile of LDS buffer 1 (its weight tile takes the lo weights of a replay)");
static_assert(BM == BN && BM == 2 * kFlagRows, "square tiles; two flag blocks per row tile");

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
    // cannot hold zeroed, and per (128-row block, group) a flag word whose
    // bit 2 t + h marks such a chunk in rows 32 t .. 32 t + 31, half h; NULL
    // when the kernel converts x itself
    const uint16_t* xf;
    const uint32_t* xflags;        // [ceil(M / 128)][ng]
};

typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x2a __attribute__((ext_vector_type(2), aligned(4)));

// Per-thread loads of one K-slice: 2 chunks of 8 activations; the 4 code
// bytes of the thread's trits inside an aligned 8-byte piece, at byte sh of
// it (sh = 4: the piece was moved back one word at the end of the codes);
// the group scale (loaded with the first half of a group, kept for the
// second).
struct Slice {
    u32x4 xa[2];
    u32x2 cp;
    uint32_t sh;
    uint32_t sc;
};

// fp16 high byte of the trit of base-3 digit d (t = d - 1).
__device__ __forceinline__ uint32_t trit_f16_hi(int d) {
    return d == 2 ? 0x3Cu : (d == 0 ? 0xBCu : 0x00u);
}

template <bool XF>
__global__ void __launch_bounds__(kThreads, 1) tq_prefill_kernel(Params p) {
    __shared__ __attribute__((aligned(16))) unsigned char smem[kSmemBytes];
    unsigned char* const lut = smem;
    typedef unsigned char Tile[kTileBytes];
    Tile* const tiles2 = (Tile*)(smem + kLutBytes);            // [buf * 2 + (0: A, 1: B)]
    unsigned char* const words = smem + kLutBytes + 4 * kTileBytes;
    int& redo_n = *(int*)(words);
    uint64_t* const bad_map = (uint64_t*)(words + 64);
    uint16_t* const redo = (uint16_t*)tiles2[2];               // buffer 1, idle during the replays

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = readfirstlane(tid >> 6);
    const int wm = wave / kWN, wn = wave % kWN;
    const int jpart = lane & 1;                                 // which 16 trits of a half

    // ---- trit table: 32 copies; entries 243..255 decode to zero
    for (int i = tid; i < 256 * 32; i += kThreads) {
        const int b = i >> 5, c = i & 31;
        uint32_t lo = 0, hi = 0;
        if (b < 243) {
            const int d0 = b % 3, d1 = (b / 3) % 3, d2 = (b / 9) % 3, d3 = (b / 27) % 3, d4 = b / 81;
            lo = trit_f16_hi(d0) | (trit_f16_hi(d1) << 8) | (trit_f16_hi(d2) << 16) |
                 (trit_f16_hi(d3) << 24);
            hi = trit_f16_hi(d4);
        }
        *(uint2*)(lut + ((b << 8) | (c << 3))) = make_uint2(lo, hi);
    }
    if (tid == 0) redo_n = 0;
    for (int i = tid; i <= kMapSlices + 1; i += kThreads) bad_map[i] = 0ull;

    const int64_t m0 = (int64_t)blockIdx.y * BM;
    const int64_t n0 = (int64_t)blockIdx.x * BN;
    const int nslices = 2 * p.ng * p.planes;
    const int psh = p.planes == 2 ? 2 : 1;                      // slice -> group shift
    const uint32_t cofs = (uint32_t)(lane & 31) << 3;           // copy lane % 32

    // this thread's activation chunks (rows xr + 128 i, 8 values at column
    // 8 xc) and weight row
    const int xc = tid & 3, xr = tid >> 2;
    const int wr = 32 * wave + (lane >> 1);                     // the two lanes of a row share its lines
    const int64_t wrow = min(n0 + wr, p.N - 1);
    const int64_t row_bytes = (int64_t)p.ng * kNB;

    // 32-bit offsets from uniform per-tile bases: activations (rows of this
    // tile), codes and scales (rows of this tile, per plane)
    uint32_t xo[2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
        xo[i] = (uint32_t)((min(m0 + xr + 128 * i, p.M - 1) - m0) * p.K + 8 * xc);
    const uint16_t* const xt = p.x + m0 * p.K;
    const uint16_t* const xft = XF ? p.xf + m0 * p.K : xt;
    const uint8_t* const ct0 = p.codes + n0 * row_bytes;
    const uint8_t* const ct1 = p.codes2 + n0 * row_bytes;
    const uint16_t* const st0 = p.scales + n0 * p.ng;
    const uint16_t* const st1 = p.scales2 + n0 * p.ng;
    const uint32_t co = (uint32_t)((wrow - n0) * row_bytes + 3 * jpart);    // group byte 3 jpart
    const uint32_t so = (uint32_t)((wrow - n0) * p.ng);
    // last code word of the buffer, relative to this tile (at least 12)
    const uint32_t clast = (uint32_t)min((((int64_t)p.N * row_bytes - 1) & ~(int64_t)3) - n0 * row_bytes,
                                         (int64_t)0x7fffffff);

    // loads of slice s (clamped to the last).  HL: the slice's half when
    // known at compile time (0 or 1), -1 when not.  A first half loads the
    // group scale, a second half keeps the one loaded with the first.
    // from_xf: the fp16 pass of a call with pre-converted activations.
    auto gload = [&](auto HLc, int s, Slice& S, bool from_xf) {
        constexpr int HL = decltype(HLc)::value;
        const int sc = min(s, nslices - 1);
        const int h = HL >= 0 ? HL : (sc & 1);
        const bool second = p.planes == 2 && ((sc >> 1) & 1);
        const int g = sc >> psh;
        const uint32_t k0 = (uint32_t)(g * G + BK * h);
        const uint16_t* xs = (XF && from_xf) ? xft : xt;
#pragma unroll
        for (int i = 0; i < 2; ++i) S.xa[i] = *(const u32x4*)(xs + xo[i] + k0);
        // bytes 3 u .. 3 u + 3 of the group, u = 2 h + jpart: the aligned
        // 8-byte piece holding them; at the end of the codes the piece of a
        // second half may start one word earlier, so that both its words
        // hold code bytes
        const uint32_t o = co + (uint32_t)(g * kNB + 6 * h);
        uint32_t b = o & ~3u;
        if (HL != 0) b = min(b, clast - 4);
        S.cp = *(const u32x2a*)((second ? ct1 : ct0) + b);
        S.sh = o - b;
        if (HL != 1) S.sc = (second ? st1 : st0)[so + (uint32_t)g];
    };

    // fp16 pairs of t for this thread's 16 trits (h: the slice's half)
    auto decode_pairs = [&](const Slice& S, int h, uint32_t* P) {
        const uint32_t al = align_bytes(S.cp[1], S.cp[0], S.sh);
        const uint32_t D = (S.sh & 4u) ? S.cp[1] : al;
        uint32_t x[4], y[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const uint32_t a = perm_b32(D, cofs, 0x0c0c0400u + ((uint32_t)i << 8));
            const uint2 e = *(const uint2*)(lut + a);
            x[i] = e.x;
            y[i] = e.y;
        }
        // digit stream: word w holds positions 4 w .. 4 w + 3
        uint32_t W[5];
        W[0] = x[0];
        W[1] = perm_b32(x[1], y[0], 0x06050400u);
        W[2] = align_bytes(y[1], x[1], 3) | (x[2] << 16);
        W[3] = align_bytes(y[2], x[2], 2) | (x[3] << 24);
        W[4] = align_bytes(y[3], x[3], 1);
        // pair e of word m: positions 4 m + u + 2 e and + 1 -> bytes (0, t, 0, t)
        const uint32_t u = (uint32_t)(2 * h + jpart);
        const uint32_t sel0 = 0x000c000cu | (u << 8) | ((u + 1) << 24);
        const uint32_t sel1 = 0x000c000cu | ((u + 2) << 8) | ((u + 3) << 24);
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            P[2 * m] = perm_b32(W[m + 1], W[m], sel0);
            P[2 * m + 1] = perm_b32(W[m + 1], W[m], sel1);
        }
    };

    // fp16 activations and weights of a slice into buffer buf.  A chunk of 8
    // activations outside the exact range is written as zeros and counted
    // for the bf16 pass.
    auto store_f16 = [&](int s, int h, int buf, const Slice& S) {
        unsigned char* A = tiles2[2 * buf];
        unsigned char* Wt = tiles2[2 * buf + 1];
        if constexpr (XF) {
            // converted and flagged by the pre-pass (the replay list reads its flags)
#pragma unroll
            for (int i = 0; i < 2; ++i) *(u32x4*)(A + (xr + 128 * i) * kPitch + 16 * xc) = S.xa[i];
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
                *(u32x4*)(A + (xr + 128 * i) * kPitch + 16 * xc) = v;
            }
            // the wave's flag for this slice; the word past the map keeps an
            // OR of every later slice, the one after it takes the decodes
            // past the last slice
            const bool wbad = __builtin_amdgcn_ballot_w64(nbad != 0) != 0;
            const int slot = s >= nslices ? kMapSlices + 1 : min(s, kMapSlices);
            unsigned char* fb = (unsigned char*)&bad_map[slot] + wave;
            *fb = (unsigned char)((slot >= kMapSlices ? *fb : 0) | (wbad ? 1 : 0));
        }
        uint32_t P[8];
        decode_pairs(S, h, P);
        const f16x2 s2 = {__builtin_bit_cast(_Float16, (uint16_t)S.sc),
                          __builtin_bit_cast(_Float16, (uint16_t)S.sc)};
        u32x4 o[2];
#pragma unroll
        for (int q = 0; q < 8; ++q)
            o[q >> 2][q & 3] = __builtin_bit_cast(uint32_t, __builtin_bit_cast(f16x2, P[q]) * s2);
        unsigned char* dst = Wt + wr * kPitch + 32 * jpart;
        *(u32x4*)dst = o[0];
        *(u32x4*)(dst + 16) = o[1];
    };

    // the bf16 pass: raw bf16 activations of the chunks the fp16 pass left
    // out (zeros elsewhere) into buffer 0, and the bf16 hi weights into
    // buffer 0, the lo weights into buffer 1
    auto store_bf16 = [&](const Slice& S, int h) {
        unsigned char* A = tiles2[0];
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            Range R;
#pragma unroll
            for (int w = 0; w < 4; ++w) (void)bf16x2_to_f16x2(S.xa[i][w], R);
            const bool bad = !range_ok(R);
            u32x4 v;
#pragma unroll
            for (int w = 0; w < 4; ++w) v[w] = bad ? S.xa[i][w] : 0u;
            *(u32x4*)(A + (xr + 128 * i) * kPitch + 16 * xc) = v;
        }
        uint32_t P[8];
        decode_pairs(S, h, P);
        const float sf = f16_bits_to_f32((uint16_t)S.sc);
        const uint32_t hb = f32_to_bf16_rne(sf);
        const uint32_t lb = f32_to_bf16_rne(sf - bf16_bits_to_f32((uint16_t)hb));
        const uint32_t hb2 = hb * 0x10001u, lb2 = lb * 0x10001u;
        u32x4 oh[2], ol[2];
#pragma unroll
        for (int q = 0; q < 8; ++q) {
            // t halves are 0x3C00 (+1), 0xBC00 (-1) or 0: a full mask where t != 0
            const uint32_t mask = ((P[q] >> 10) & 0x000F000Fu) * 0x1111u;
            const uint32_t sign = P[q] & 0x80008000u;
            oh[q >> 2][q & 3] = (mask & hb2) ^ (sign & (mask & 0x80008000u));
            ol[q >> 2][q & 3] = (mask & lb2) ^ (sign & (mask & 0x80008000u));
        }
        unsigned char* dh = tiles2[1] + wr * kPitch + 32 * jpart;
        unsigned char* dl = tiles2[3] + wr * kPitch + 32 * jpart;
        *(u32x4*)dh = oh[0];
        *(u32x4*)(dh + 16) = oh[1];
        *(u32x4*)dl = ol[0];
        *(u32x4*)(dl + 16) = ol[1];
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
    auto load_frag = [&](int abuf, int bbuf, int ks, Frag& F) {
        const unsigned char* A = tiles2[2 * abuf] + (wm * 32 * MT + frow) * kPitch + fk + 32 * ks;
        const unsigned char* B = tiles2[2 * bbuf + 1] + (wn * 32 * NT + frow) * kPitch + fk + 32 * ks;
#pragma unroll
        for (int i = 0; i < MT; ++i) F.a[i] = *(const u32x4*)(A + i * 32 * kPitch);
#pragma unroll
        for (int jn = 0; jn < NT; ++jn) F.b[jn] = *(const u32x4*)(B + jn * 32 * kPitch);
    };
    // tiles: bit i set = this wave's 32-row tile i takes part (uniform)
    auto mfma_frag = [&](const Frag& F, bool f16, uint32_t tiles) {
#pragma unroll
        for (int i = 0; i < MT; ++i) {
            if (!((tiles >> i) & 1u)) continue;
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
        }
    };
    static_assert(BK == 32, "two K-steps of 16 per slice");

    __syncthreads();                       // table and flags written

    // ---- fp16 pass over every slice (out-of-range chunks enter as zeros).
    // Slice t sits in buffer t & 1.  Step s runs the MFMAs of slice s from
    // registers while reading the next fragments; between its two K-steps
    // one barrier marks buffer s & 1 as read by every wave, and slice s + 2
    // is decoded into it.  The loop takes two steps (both halves of a
    // group), so each step's half is a compile-time constant.
    Slice S;
    Frag F0, F1;
    const std::integral_constant<int, 0> H0;
    const std::integral_constant<int, 1> H1;
    if (nslices > 0) {                     // nslices is even
        gload(H0, 0, S, true);
        store_f16(0, 0, 0, S);
        gload(H1, 1, S, true);
        store_f16(1, 1, 1, S);
        gload(H0, 2, S, true);
    }
    __syncthreads();
    load_frag(0, 0, 0, F0);
    auto step = [&](auto Hc, int s) {
        constexpr int H = decltype(Hc)::value;
        // the scheduler interleaves the MFMAs with the LDS traffic around
        // them (strategy 0); the arithmetic and its order are unchanged
        __builtin_amdgcn_iglp_opt(0);
        load_frag(H, H, 1, F1);            // slice s, second K-step
        mfma_frag(F0, true, 0xFu);
        __syncthreads();                   // every wave is done reading buffer H
        // decode slice s + 2 into buffer H (past the end: into a buffer
        // nobody reads; no branch, so the decode interleaves with the MFMAs)
        store_f16(s + 2, H, H, S);
        load_frag(H ^ 1, H ^ 1, 0, F0);    // slice s + 1, first K-step
        mfma_frag(F1, true, 0xFu);
        gload(std::integral_constant<int, H ^ 1>(), s + 3, S, true);   // clamped; unused past the end
    };
#pragma unroll 1
    for (int s = 0; s < nslices; s += 2) {
        step(H0, s);
        step(H1, s + 1);
    }

    // ---- bf16 pass over the chunks left out: flagged slices below
    // kMapSlices one by one, then every slice from kMapSlices on if any there
    // was flagged.  Activations and hi weights in buffer 0, lo weights in
    // buffer 1's weight tile.
    __syncthreads();
    const int64_t nfb = (p.M + kFlagRows - 1) / kFlagRows;     // pre-pass flag blocks
    const int64_t fb0 = 2 * (int64_t)blockIdx.y;               // this tile's two blocks
    // pre-pass flag word of block b and the group of slice w (zero past M)
    auto flag_word = [&](int64_t b, int w) -> uint32_t {
        return b < nfb ? p.xflags[b * p.ng + (w >> psh)] : 0u;
    };
    if (tid == 0) {
        int n = 0;
        const int mapped = min(nslices, kMapSlices);
        if constexpr (XF) {
            // the pre-pass flags of this tile's two 128-row blocks: bit
            // 2 t + h of a group's word marks rows 32 t .. 32 t + 31 of the
            // block in half h (both planes of a group share its activations);
            // later slices as one flag
            auto flagged = [&](int w) {
                const uint32_t m = 0x55u << (w & 1);
                return ((flag_word(fb0, w) | flag_word(fb0 + 1, w)) & m) != 0u;
            };
            for (int w = 0; w < mapped; ++w)
                if (flagged(w)) redo[n++] = (uint16_t)w;
            bool late = false;
            for (int w = kMapSlices; w < nslices; ++w) late = late || flagged(w);
            bad_map[kMapSlices] = late ? 1ull : 0ull;
        } else {
            for (int w = 0; w < mapped; ++w)
                if (bad_map[w]) redo[n++] = (uint16_t)w;
        }
        redo_n = n;
    }
    __syncthreads();
    const int nlist = readfirstlane(redo_n);
    const int late_end = readfirstlane(bad_map[kMapSlices] != 0ull ? 1 : 0) ? nslices : kMapSlices;
    const int nreplay = nlist + max(late_end - kMapSlices, 0);
    auto replay_slice = [&](int r) {
        return r < nlist ? (int)readfirstlane(redo[r]) : kMapSlices + (r - nlist);
    };
    const std::integral_constant<int, -1> HR;
    if (nreplay > 0) gload(HR, replay_slice(0), S, false);
#pragma unroll 1
    for (int r = 0; r < nreplay; ++r) {
        const int w = replay_slice(r);
        // with pre-pass flags, only this wave's 32-row tiles holding a chunk
        // fp16 cannot hold take part (the others would add zeros)
        uint32_t tmask = 0xFu;
        if constexpr (XF) {
            const uint32_t f = flag_word(fb0 + wm, w) >> (w & 1);
            tmask = (uint32_t)readfirstlane((int)((f & 1u) | ((f >> 1) & 2u) | ((f >> 2) & 4u) | ((f >> 3) & 8u)));
        } else if (w < kMapSlices) {
            // wave v's flag byte covers its converted rows 16 v .. 16 v + 15
            // and 128 + 16 v .., in 32-row tile v / 2 of either half
            tmask = (uint32_t)readfirstlane((int)flag_tiles(bad_map[w]));
        }
        store_bf16(S, w & 1);
        __syncthreads();
        gload(HR, replay_slice(min(r + 1, nreplay - 1)), S, false);
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
            load_frag(0, 0, ks, F0);
            mfma_frag(F0, false, tmask);
            load_frag(0, 1, ks, F1);
            mfma_frag(F1, false, tmask);
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
// exactly becomes zeros, and bit 2 t + h of its group's flag word marks that
// rows 32 t .. 32 t + 31 of this row block hold such a chunk in half h of the
// group (the prefill replays that half in bf16, for those rows).  Every flag
// word is written by exactly one workgroup.
constexpr int kXcCols = 128;
static_assert(kXcCols % G == 0, "whole groups per pre-pass workgroup");
__global__ void __launch_bounds__(256) tq_xconv_kernel(const uint16_t* __restrict__ x, int64_t M,
                                                      int64_t K, int ng, uint16_t* __restrict__ xf,
                                                      uint32_t* __restrict__ flags) {
    __shared__ uint32_t fl[kXcCols / G];
    const int tid = threadIdx.x;
    if (tid < kXcCols / G) fl[tid] = 0u;
    __syncthreads();
    const int64_t m0 = (int64_t)blockIdx.y * kFlagRows;
    const int cc = tid & 15;                              // chunk of 8 columns
    const int64_t col = (int64_t)blockIdx.x * kXcCols + 8 * cc;
    uint32_t bits = 0u;
    if (col < K) {                                        // K % 64 == 0: chunks are whole
#pragma unroll 4
        for (int i = 0; i < kFlagRows / 16; ++i) {
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
                const int t = ((tid >> 4) + 16 * i) >> 5;             // 32-row part of the block
                bits |= bad ? 1u << (2 * t + ((cc >> 2) & 1)) : 0u;
            }
        }
    }
    if (bits) atomicOr(&fl[cc >> 3], bits);               // group (col mod 128) / 64
    __syncthreads();
    if (tid < kXcCols / G) {
        const int64_t g = (int64_t)blockIdx.x * (kXcCols / G) + tid;
        if (g < ng) flags[(int64_t)blockIdx.y * ng + g] = fl[tid];
    }
}

}  // namespace

// Dense ternary matmul for many tokens; false (nothing launched) outside its
// domain: G = 64, M >= 128, K < 2^23, x 16-byte and codes 4-byte aligned, a
// grid within the launch limits.
bool launch_tq_prefill(const TqMatmulArgs& a, hipStream_t s, hipError_t* err) {
    if (a.n_experts != 0 || a.G != G || a.M < kFlagRows || a.K < G || a.K % G != 0 ||
        ((uintptr_t)a.x & 15) != 0 || ((uintptr_t)a.codes[0] & 3) != 0 ||
        ((uintptr_t)a.scales[0] & 1) != 0)
        return false;
    if (a.planes == 2 && (((uintptr_t)a.codes[1] & 3) != 0 || ((uintptr_t)a.scales[1] & 1) != 0))
        return false;
    if (2 * (a.K / G) * a.planes >= (1ll << 30)) return false;        // slice count in an int
    if (a.K >= (1ll << 23)) return false;             // 32-bit element offsets inside a 256-row tile
    const int64_t gx = (a.N + BN - 1) / BN, gy = (a.M + BM - 1) / BM;
    const int64_t gyf = (a.M + kFlagRows - 1) / kFlagRows;            // pre-pass row blocks
    if (gx == 0 || gx >= (1ll << 31) || gyf >= 65536) return false;
    Params p;
    p.x = a.x;
    p.M = a.M;
    p.K = a.K;
    p.N = a.N;
    p.ng = (int)(a.K / G);
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
        hipLaunchKernelGGL(tq_xconv_kernel, dim3((unsigned)((a.K + kXcCols - 1) / kXcCols), (unsigned)gyf),
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
