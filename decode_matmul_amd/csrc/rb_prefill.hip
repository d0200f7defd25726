// Route B prefill (M > 16): y[m, n] = alpha * rho_n * sum_k x[m, k] T[codes[n, k]] + bias_n
// as an MFMA GEMM whose weight tiles are decoded from code bytes into LDS.
//
// Semantics: "A Discrete Weight Language for Large Language Models" (Route
// B), section 4.2: the code book is loaded on chip once per block and a
// K-sliced GEMM dereferences every code byte through it; y = alpha rho_n acc
// + bias_n, so rho multiplies the finished sum (sections 3.3 and 4.2).
//
// Numerics.  The products run on fp16 MFMAs with fp32 accumulation:
//  * The code book is scaled by sigma = 2^j so that max |sigma T| lies in
//    [2^14, 2^15) and each entry is rounded to fp16 once (relative error at
//    most 2^-11, against the 2e-3 acceptance bound).  The output is scaled
//    back by 1/sigma exactly.
//  * bf16 activations are converted to fp16 exactly when 2^-17 <= |x| <=
//    65280 or x = 0 (fp16 holds every such bf16 value).
//  * An 8-value activation chunk outside that range (every chunk, when a
//    nonzero code-book entry falls below the fp16 normal range after
//    scaling) enters the fp16 pass as zeros and is added afterwards on bf16
//    MFMAs in two passes: the bf16 activations against hi = bf16(sigma T),
//    then against lo = bf16(sigma T - hi) (together within 2^-17 of
//    sigma T), with every other chunk zero.  So every input meets the bound;
//    typical activations take only the fp16 pass.
//
// Mapping onto gfx950:
//  * A 512-thread workgroup (8 waves in a 2 x 4 grid, two per SIMD so one
//    wave's decode overlaps the other's MFMAs) owns a 256 x 256 tile of y
//    (tokens x rows); each wave owns 128 x 64 = 4 x 2 MFMA 32x32x16 tiles
//    (128 fp32 accumulators per lane).
//  * K-slices of 32 in two LDS buffers: slice t's activation tile (256 x 32,
//    converted to fp16) and weight tile (256 rows x 32 codes, decoded
//    through the LDS code book) sit in buffer t & 1.  While the MFMAs of
//    slice s run from registers, the next K-step's fragments are read and
//    slice s + 2 (loaded from global memory an iteration earlier) is decoded
//    into the buffer slice s has just vacated.  One barrier per slice.
//  * The code book sits in LDS in 8 slots of 4 copies: slot h serves tile
//    rows 32 h .. 32 h + 31 (with one book per block of 32 rows, section
//    8.3, each slot holds its block's book; with one book, all eight hold
//    it).  Entry b of slot h, copy c, at byte (b << 8) | (h << 4) | (c << 2)
//    holds the fp16 value, and 128 bytes further the (hi, lo) bf16 pair; a
//    slot's book has its own power-of-two scale sigma_h.  One v_perm of the
//    code word and the lane offset forms the address.
//  * A thread decodes 16 codes of tile row 32 (q % 8) + q / 8 (q = thread /
//    2), so the lanes of a phase spread over the 8 slots and, with the copy
//    index, over distinct banks.  The decoded row goes to LDS row
//    32 h + (j ^ s_h) (row j of slot h, s_h = 0, 1, 4, 5, 8, 9, 12, 13): the
//    16-byte stores of a phase then cover distinct banks, and the fragment
//    reads (32 consecutive rows of one slot) stay conflict-free.
//  * Tile rows are 80 bytes apart, so the 8 lanes of a 16-byte column read
//    cover all 32 banks.
//  * 7-bit indices (section 8.1): a K-slice of a row is 28 bytes; the two
//    threads of a row load 16 bytes at byte 0 and 12, funnel-shift the
//    second by 16 bits, and index i is then bit 7 i of the four dwords; one
//    shift and one and-or give its address in the book, whose entry j is
//    T[used[j]].
#include "common.h"

namespace dmm {

namespace {

constexpr int BM = 256, BN = 256, BK = 32;
constexpr int kThreads = 512;
constexpr int kWN = 4;                         // waves along N (2 along M)
constexpr int MT = 4, NT = 2;                  // 32x32 MFMA tiles per wave along M and N
constexpr int kPitch = 2 * BK + 16;            // bytes per LDS tile row
constexpr int kTileBytes = BM * kPitch;        // one operand tile (BM == BN)
constexpr int kLutBytes = 256 * 256;
constexpr int kSlots = 8;                      // code-book slots (32 tile rows each)
constexpr int kMapSlices = 1536;                // slices tracked one by one (K <= 49152)
constexpr int kWords = 64 + 4 * 4 * kThreads / 64 + 32;   // flags, maxima, slot exponents
constexpr int kSmemBytes = kLutBytes + 4 * kTileBytes + kWords + 8 * (kMapSlices + 1);
static_assert(kSlots * 32 == BN, "one slot per 32 tile rows");
static_assert(kSmemBytes <= 160 * 1024, "fits the LDS of a CU");
static_assert(kThreads / 64 <= 8, "one flag byte per wave");
static_assert(kMapSlices * 2 <= kTileBytes,
              "the slice list fits the activation tile of LDS buffer 1 (its weight tile takes the lo weights of a replay)");
static_assert(BM == BN, "square tiles share one pitch");

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

struct Params {
    const uint16_t* x;
    int64_t M, K, N;
    const uint8_t* codes;                    // code bytes, or 7-bit rows
    int64_t row_bytes;                       // bytes per row of codes
    const uint8_t* used;                     // 7-bit form: index -> code [128]
    const float* table;
    int64_t table_rows;                      // 0: one code book; else rows per book
    float alpha;
    const uint16_t* row_scale;
    int64_t rho_rows;                        // rows sharing one row_scale entry
    const float* bias;
    void* y;
    int y_dtype;
    // pre-converted activations (rb_matmul_ws): fp16 x with the chunks fp16
    // cannot hold zeroed, and per (256-row block, K-slice) a flag that the
    // slice holds such a chunk; NULL when the kernel converts x itself
    const uint16_t* xf;
    const uint32_t* xflags;                  // [ceil(M / 256)][ceil(K / 32)]: bit t = rows 32 t .. 32 t + 31
};

// Row j of slot h sits in LDS row 32 h + (j ^ row_swizzle(h)).
__device__ __forceinline__ int row_swizzle(int h) { return (h & 1) | ((h & 6) << 1); }

// Index k of a 7-bit row (byte-granular reads).
__device__ __forceinline__ uint32_t load_index7(const uint8_t* row, int64_t row_bytes, int64_t k) {
    const int64_t bit = 7 * k;
    const int64_t b = bit >> 3;
    uint32_t v = row[b];
    if (b + 1 < row_bytes) v |= (uint32_t)row[b + 1] << 8;
    return (v >> (bit & 7)) & 0x7fu;
}

// Book address (index << 8) | off of index i (constant after unrolling) of
// 16 indices held at bits 7 i of F[0..3].
__device__ __forceinline__ uint32_t index7_addr(const uint32_t* F, int i, uint32_t off) {
    const int bit = 7 * i, d = bit >> 5, o = bit & 31;
    uint32_t v;
    if (o + 7 <= 32) v = o >= 8 ? F[d] >> (o - 8) : F[d] << (8 - o);
    else v = __builtin_amdgcn_alignbit(F[d + 1], F[d], (uint32_t)(o - 8));
    return (v & 0x7f00u) | off;
}

// Per-thread loads of one K-slice: 2 chunks of 8 activations, 1 chunk of 16 codes.
constexpr int XCH = BM * BK / 8 / kThreads, CCH = BN * BK / 16 / kThreads;
struct Slice {
    u32x4 xa[XCH];
    u32x4 cd[CCH];
};

// AL: 16-byte aligned activations and codes, K % 32 == 0.  C7: 7-bit indices.
template <bool AL, bool C7, bool XF>
__global__ void __launch_bounds__(kThreads, 1) rb_prefill_kernel(Params p) {
    // one LDS block: the code book at address 0 (so a v_perm result is its
    // own address), two buffers of (activation, weight) tiles, a few words
    __shared__ __attribute__((aligned(16))) unsigned char smem[kSmemBytes];
    unsigned char* const lut = smem;
    typedef unsigned char Tile[kTileBytes];
    Tile* const tiles2 = (Tile*)(smem + kLutBytes);            // [buf * 2 + (0: A, 1: B)]
    unsigned char* const words = smem + kLutBytes + 4 * kTileBytes;
    int& table_bad = *(int*)(words);
    int& redo_n = *(int*)(words + 8);
    float* const red_max = (float*)(words + 64);                 // [wave][4]
    int* const slot_exp = (int*)(words + kWords - 32);           // [kSlots]
    // one flag word per slice s < kMapSlices, one byte per wave (written by
    // the whole wave, so no atomics); word kMapSlices collects later slices
    uint64_t* const bad_map = (uint64_t*)(words + kWords);
    uint16_t* const redo = (uint16_t*)tiles2[2];        // list of flagged slices (buffer 1, idle then)

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = readfirstlane(tid >> 6);
    const int wm = wave / kWN, wn = wave % kWN;

    const int64_t m0 = (int64_t)blockIdx.y * BM;
    const int64_t n0 = (int64_t)blockIdx.x * BN;

    // ---- code books: thread tid fills entry b = tid % 256 of slots
    // tid / 256 + 2 i (i < 4).  Slot h scales its book by sigma_h = 2^j_h
    // with max |sigma_h T| in [2^14, 2^15).
    const int eb = tid & 255;
    float tv[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int h = (tid >> 8) + 2 * i;
        const float* table = rb_table_of(p.table, p.table_rows, min(n0 + 32 * h, p.N - 1));
        if constexpr (C7) {
            const uint32_t c = p.used[eb & 127];
            const float v = table[c < 243 ? c : 0];
            tv[i] = (eb < 128 && c < 243) ? v : 0.f;
        } else {
            const float v = table[eb < 243 ? eb : 0];
            tv[i] = eb < 243 ? v : 0.f;
        }
    }
    {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            float a = fabsf(tv[i]);
            for (int o = 32; o > 0; o >>= 1) a = fmaxf(a, __shfl_xor(a, o));
            if (lane == 0) red_max[wave * 4 + i] = a;
        }
        if (tid == 0) { table_bad = 0; redo_n = 0; }
        for (int i = tid; i <= kMapSlices; i += kThreads) bad_map[i] = 0ull;
    }
    __syncthreads();
    if (tid < kSlots) {                 // slot tid: waves 4 (tid & 1) .. + 3, column tid / 2
        float tmax = 0.f;
#pragma unroll
        for (int w = 0; w < 4; ++w) tmax = fmaxf(tmax, red_max[(4 * (tid & 1) + w) * 4 + (tid >> 1)]);
        int e2 = 0;
        if (tmax > 0.f && tmax <= 3.0e38f) (void)frexpf(tmax, &e2);     // tmax < 2^e2
        slot_exp[tid] = min(max(15 - e2, -120), 120);
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        // entry eb of slot h (zero for padding codes): fp16 of sigma_h T and
        // the bf16 hi/lo pair, in the slot's 4 copies
        const int h = (tid >> 8) + 2 * i;
        const float s = tv[i] * ldexpf(1.f, slot_exp[h]);              // exact power-of-two scaling
        const _Float16 hf = (_Float16)s;                                // nearest-even
        const uint32_t hb = __builtin_bit_cast(uint16_t, hf);
        const bool ok = (s == 0.f) || (fabsf(s) >= 0x1p-14f && fabsf(s) <= 65504.f);
        if (!ok) table_bad = 1;
        const uint16_t hi = f32_to_bf16_rne(s);
        const uint16_t lo = f32_to_bf16_rne(s - bf16_bits_to_f32(hi));
        const uint32_t fb = (uint32_t)hi | ((uint32_t)lo << 16);
        unsigned char* e = lut + ((eb << 8) | (h << 4));
        *(u32x4*)e = u32x4{hb, hb, hb, hb};
        *(u32x4*)(e + 128) = u32x4{fb, fb, fb, fb};
    }

    const int nslices = (int)((p.K + BK - 1) / BK);

    // this thread's chunks: activations (rows xr + 128 i, 8 values at column
    // 8 xc), codes (tile row cr = 32 ch + cj, 16 codes at column 16 cc),
    // decoded through slot ch, copy 2 (cj & 1) + cc, into LDS row crs
    const int xc = tid & 3, xr = tid >> 2;
    const int cc = tid & 1, cq = tid >> 1;
    const int ch = cq & 7, cj = cq >> 3;
    const int cr = 32 * ch + cj;
    const int crs = 32 * ch + (cj ^ row_swizzle(ch));
    const uint32_t cofs = (uint32_t)((ch << 4) | ((((cj & 1) << 1) | cc) << 2));
    static_assert(XCH == 2 && CCH == 1, "chunk mapping");

    // from_xf: the fp16 pass of a call with pre-converted activations
    auto gload = [&](int s, Slice& S, bool from_xf) {
        const int64_t k0 = (int64_t)min(s, nslices - 1) * BK;
        if constexpr (AL) {
            const uint16_t* xs = (XF && from_xf) ? p.xf : p.x;
#pragma unroll
            for (int i = 0; i < XCH; ++i) {
                const int64_t m = min(m0 + xr + 128 * i, p.M - 1);
                S.xa[i] = *(const u32x4*)(xs + m * p.K + k0 + 8 * xc);
            }
            const int64_t n = min(n0 + cr, p.N - 1);
            if constexpr (C7)      // 28 bytes per slice: dwords 0..3 or 3..6
                S.cd[0] = *(const u32x4a*)(p.codes + n * p.row_bytes + (k0 / BK) * 28 + 12 * cc);
            else
                S.cd[0] = *(const u32x4*)(p.codes + n * p.row_bytes + k0 + 16 * cc);
        } else {
            // element loads: activations past M or K are 0, codes past N or K
            // are 255 (a zero entry of the padded table)
#pragma unroll
            for (int i = 0; i < XCH; ++i) {
                const int64_t m = m0 + xr + 128 * i;
#pragma unroll
                for (int w = 0; w < 4; ++w) {
                    const int64_t k = k0 + 8 * xc + 2 * w;
                    uint32_t lo = 0, hi = 0;
                    if (m < p.M) {
                        if (k < p.K) lo = p.x[m * p.K + k];
                        if (k + 1 < p.K) hi = p.x[m * p.K + k + 1];
                    }
                    S.xa[i][w] = lo | (hi << 16);
                }
            }
            // (7-bit indices arrive one per byte, as code bytes do)
            const int64_t n = n0 + cr;
            const uint8_t* row = p.codes + (n < p.N ? n : 0) * p.row_bytes;
#pragma unroll
            for (int w = 0; w < 4; ++w) {
                uint32_t v = 0;
#pragma unroll
                for (int b = 0; b < 4; ++b) {
                    const int64_t k = k0 + 16 * cc + 4 * w + b;
                    uint32_t c = 0xffu;
                    if (n < p.N && k < p.K) c = C7 ? load_index7(row, p.row_bytes, k) : row[k];
                    v |= c << (8 * b);
                }
                S.cd[0][w] = v;
            }
        }
    };

    // weight tile of a slice from the code book: fp16 (word 0) or bf16 hi / lo
    // (word at + 128, part 0 / 1)
    auto store_weights = [&](int buf, const Slice& S, uint32_t lut_off, uint32_t sel) {
        unsigned char* B = tiles2[2 * buf + 1];
        uint32_t F[4];
        if constexpr (C7 && AL) {
            // the second thread of a row loaded from dword 3: drop 16 bits so
            // that index i of either thread sits at bit 7 i
            const uint32_t sh = 16u * (uint32_t)cc;
            F[0] = __builtin_amdgcn_alignbit(S.cd[0][1], S.cd[0][0], sh);
            F[1] = __builtin_amdgcn_alignbit(S.cd[0][2], S.cd[0][1], sh);
            F[2] = __builtin_amdgcn_alignbit(S.cd[0][3], S.cd[0][2], sh);
            F[3] = S.cd[0][3] >> sh;
        }
        u32x4 o0, o1;
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            uint32_t e[4];
#pragma unroll
            for (int b = 0; b < 4; ++b) {
                uint32_t a;
                if constexpr (C7 && AL) a = index7_addr(F, 4 * w + b, cofs | lut_off);
                else a = perm_b32(S.cd[0][w], cofs | lut_off, 0x0c0c0400u + ((uint32_t)b << 8));
                e[b] = *(const uint32_t*)(lut + a);
            }
            const uint32_t p01 = perm_b32(e[1], e[0], sel);
            const uint32_t p23 = perm_b32(e[3], e[2], sel);
            if (w < 2) { o0[2 * w] = p01; o0[2 * w + 1] = p23; }
            else { o1[2 * w - 4] = p01; o1[2 * w - 3] = p23; }
        }
        unsigned char* dst = B + crs * kPitch + 32 * cc;
        *(u32x4*)dst = o0;
        *(u32x4*)(dst + 16) = o1;
    };

    // fp16 activations and weights of a slice into buffer buf.  A chunk of 8
    // activations outside the exact range (or every chunk, when the code book
    // does not fit fp16) is written as zeros and counted for the bf16 pass.
    auto store_f16 = [&](int s, int buf, const Slice& S, bool force_bad) {
        unsigned char* A = tiles2[2 * buf];
        if constexpr (XF) {
            // converted and flagged by the pre-pass (the replay list reads its flags)
#pragma unroll
            for (int i = 0; i < XCH; ++i) {
                u32x4 v = S.xa[i];
#pragma unroll
                for (int w = 0; w < 4; ++w) v[w] = force_bad ? 0u : v[w];
                *(u32x4*)(A + (xr + 128 * i) * kPitch + 16 * xc) = v;
            }
            store_weights(buf, S, 0u, 0x05040100u);
            return;
        }
        int nbad = 0;
#pragma unroll
        for (int i = 0; i < XCH; ++i) {
            Range R;
            u32x4 v;
#pragma unroll
            for (int w = 0; w < 4; ++w) v[w] = bf16x2_to_f16x2(S.xa[i][w], R);
            const bool bad = force_bad | !range_ok(R);     // no short circuit: no branch
            nbad += bad;
#pragma unroll
            for (int w = 0; w < 4; ++w) v[w] = bad ? 0u : v[w];
            *(u32x4*)(A + (xr + 128 * i) * kPitch + 16 * xc) = v;
        }
        // the wave's flag for this slice, stored by every lane (same value);
        // the word past the map keeps an OR of every later slice
        const bool wbad = __builtin_amdgcn_ballot_w64(nbad != 0) != 0;
        unsigned char* fb = (unsigned char*)&bad_map[min(s, kMapSlices)] + wave;
        *fb = (unsigned char)((s >= kMapSlices ? *fb : 0) | (wbad ? 1 : 0));
        store_weights(buf, S, 0u, 0x05040100u);
    };

    // the bf16 pass's weights in one lookup per code: the book's (hi, lo)
    // word gives the hi tile (buffer 0) and the lo tile (buffer 1)
    auto store_weights_hilo = [&](const Slice& S) {
        uint32_t F[4];
        if constexpr (C7 && AL) {
            const uint32_t sh = 16u * (uint32_t)cc;
            F[0] = __builtin_amdgcn_alignbit(S.cd[0][1], S.cd[0][0], sh);
            F[1] = __builtin_amdgcn_alignbit(S.cd[0][2], S.cd[0][1], sh);
            F[2] = __builtin_amdgcn_alignbit(S.cd[0][3], S.cd[0][2], sh);
            F[3] = S.cd[0][3] >> sh;
        }
        u32x4 h0, h1, l0, l1;
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            uint32_t e[4];
#pragma unroll
            for (int b = 0; b < 4; ++b) {
                uint32_t a;
                if constexpr (C7 && AL) a = index7_addr(F, 4 * w + b, cofs | 128u);
                else a = perm_b32(S.cd[0][w], cofs | 128u, 0x0c0c0400u + ((uint32_t)b << 8));
                e[b] = *(const uint32_t*)(lut + a);
            }
            const uint32_t h01 = perm_b32(e[1], e[0], 0x05040100u), h23 = perm_b32(e[3], e[2], 0x05040100u);
            const uint32_t l01 = perm_b32(e[1], e[0], 0x07060302u), l23 = perm_b32(e[3], e[2], 0x07060302u);
            if (w < 2) { h0[2 * w] = h01; h0[2 * w + 1] = h23; l0[2 * w] = l01; l0[2 * w + 1] = l23; }
            else { h1[2 * w - 4] = h01; h1[2 * w - 3] = h23; l1[2 * w - 4] = l01; l1[2 * w - 3] = l23; }
        }
        unsigned char* dh = tiles2[1] + crs * kPitch + 32 * cc;
        unsigned char* dl = tiles2[3] + crs * kPitch + 32 * cc;
        *(u32x4*)dh = h0;
        *(u32x4*)(dh + 16) = h1;
        *(u32x4*)dl = l0;
        *(u32x4*)(dl + 16) = l1;
    };

    // the bf16 pass: bf16 activations of the chunks the fp16 pass left out
    // (zeros elsewhere) and the hi (part 0) or lo (part 1) bf16 weights
    // (part -1: the activations alone)
    auto store_bf16 = [&](int buf, const Slice& S, bool force_bad, int part) {
        unsigned char* A = tiles2[2 * buf];
        if (part <= 0) {
#pragma unroll
            for (int i = 0; i < XCH; ++i) {
                Range R;
#pragma unroll
                for (int w = 0; w < 4; ++w) (void)bf16x2_to_f16x2(S.xa[i][w], R);
                const bool bad = force_bad | !range_ok(R);     // no short circuit: no branch
                u32x4 v;
#pragma unroll
                for (int w = 0; w < 4; ++w) v[w] = bad ? S.xa[i][w] : 0u;
                *(u32x4*)(A + (xr + 128 * i) * kPitch + 16 * xc) = v;
            }
        }
        if (part >= 0) store_weights(buf, S, 128u, part == 0 ? 0x05040100u : 0x07060302u);
    };

    // accumulators start life in the accumulation registers (the empty asm
    // pins the register class), so the loop never copies them through VGPRs
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

    // A fragment: lane l holds A[l % 32][8 (l / 32) .. +7]; B alike with the
    // rows of the weight tile (tile rows 32 h + l % 32 of slot h = NT wn + jn,
    // at their swizzled LDS rows).  One K-step (16) of a slice per Frag.
    const int frow = lane & 31;
    const int fk = 16 * (lane >> 5);
    static_assert(NT * 32 * kWN == BN, "a wave's B tiles are whole slots");
    int brow[NT];
#pragma unroll
    for (int jn = 0; jn < NT; ++jn) {
        const int h = wn * NT + jn;
        brow[jn] = (32 * h + (frow ^ row_swizzle(h))) * kPitch;
    }
    struct Frag {
        u32x4 a[MT];
        u32x4 b[NT];
    };
    auto load_frag = [&](int abuf, int bbuf, int ks, Frag& F) {
        const unsigned char* A = tiles2[2 * abuf] + (wm * 32 * MT + frow) * kPitch + fk + 32 * ks;
        const unsigned char* B = tiles2[2 * bbuf + 1] + fk + 32 * ks;
#pragma unroll
        for (int i = 0; i < MT; ++i) F.a[i] = *(const u32x4*)(A + i * 32 * kPitch);
#pragma unroll
        for (int jn = 0; jn < NT; ++jn) F.b[jn] = *(const u32x4*)(B + brow[jn]);
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
    const bool all_bf16 = readfirstlane(table_bad) != 0;   // uniform: LDS values are not known to be

    // ---- fp16 pass over every slice (out-of-range chunks enter as zeros).
    // Slice t sits in buffer t & 1.  Iteration s runs the MFMAs of slice s
    // from registers while reading the next fragments; between its two
    // K-steps one barrier marks buffer s & 1 as read by every wave, and
    // slice s + 2 is decoded into it.
    Slice S;
    Frag F0, F1;
    if (nslices > 0) {                     // K = 0 reads nothing (x may be null)
        gload(0, S, true);
        store_f16(0, 0, S, all_bf16);
        gload(1, S, true);
        store_f16(min(1, nslices - 1), 1, S, all_bf16);
        gload(2, S, true);
    }
    __syncthreads();
    load_frag(0, 0, 0, F0);
#pragma unroll 1
    for (int s = 0; s < nslices; ++s) {
        // ask the scheduler to interleave the MFMAs with the LDS reads and
        // writes around them (strategy 0); the order of the arithmetic is
        // unchanged, and so is every output bit
        __builtin_amdgcn_iglp_opt(0);
        const int buf = s & 1;
        load_frag(buf, buf, 1, F1);        // slice s, second K-step
        mfma_frag(F0, true, 0xFu);
        __syncthreads();                   // every wave is done reading buffer buf
        // decode slice s + 2 into buffer buf (past the end: the last slice
        // again, into a buffer nobody reads; no branch, so the decode
        // interleaves with the MFMAs)
        store_f16(min(s + 2, nslices - 1), buf, S, all_bf16);
        load_frag(buf ^ 1, buf ^ 1, 0, F0); // slice s + 1, first K-step
        mfma_frag(F1, true, 0xFu);
        gload(s + 3, S, true);             // clamped; unused past the end
    }

    // ---- bf16 pass over the chunks left out: the flagged slices below
    // kMapSlices one by one, every slice from kMapSlices on if any there was
    // flagged (a slice without flagged chunks adds zero, so extra ones are
    // harmless).  The activations and hi weights go to buffer 0, the lo
    // weights to the weight tile of buffer 1.
    __syncthreads();
    if (tid == 0) {
        int n = 0;
        const int mapped = min(nslices, kMapSlices);
        if constexpr (XF) {
            // the pre-pass flags of this 256-row block; later slices as one flag
            const uint32_t* fr = p.xflags + (int64_t)blockIdx.y * nslices;
            for (int w = 0; w < mapped; ++w)
                if (all_bf16 || fr[w]) redo[n++] = (uint16_t)w;
            bool late = false;
            for (int w = kMapSlices; w < nslices; ++w) late = late || all_bf16 || fr[w] != 0u;
            bad_map[kMapSlices] = late ? 1ull : 0ull;
        } else {
            for (int w = 0; w < mapped; ++w)
                if (bad_map[w]) redo[n++] = (uint16_t)w;
        }
        redo_n = n;
    }
    __syncthreads();
    // slice of the r-th replay: the listed ones, then (if flagged) every
    // slice from kMapSlices on; the next replay's loads are issued before
    // the current one's MFMAs
    const int nlist = readfirstlane(redo_n);
    const int late_end = readfirstlane(bad_map[kMapSlices] != 0ull ? 1 : 0) ? nslices : kMapSlices;
    const int nreplay = nlist + max(late_end - kMapSlices, 0);
    auto replay_slice = [&](int r) {
        return r < nlist ? (int)readfirstlane(redo[r]) : kMapSlices + (r - nlist);
    };
    if (nreplay > 0) gload(replay_slice(0), S, false);
#pragma unroll 1
    for (int r = 0; r < nreplay; ++r) {
        // with pre-pass flags, only this wave's 32-row tiles holding a chunk
        // fp16 cannot hold take part (the others add zeros)
        uint32_t tmask = 0xFu;
        if constexpr (XF) {
            if (!all_bf16) {
                const uint32_t f = p.xflags[(int64_t)blockIdx.y * nslices + replay_slice(r)];
                tmask = readfirstlane((f >> (wm * MT)) & 0xFu);
            }
        } else {
            // a mapped slice: wave v's flag byte covers its converted rows
            // 16 v .. 16 v + 15 and 128 + 16 v .., in 32-row tile v / 2 of
            // either half
            const int w = replay_slice(r);
            if (w < kMapSlices) tmask = (uint32_t)readfirstlane((int)flag_tiles(bad_map[w]));
        }
        store_bf16(0, S, all_bf16, -1);                 // activations only
        store_weights_hilo(S);
        __syncthreads();
        gload(replay_slice(min(r + 1, nreplay - 1)), S, false);
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
        const float inv_sigma = ldexpf(1.f, -slot_exp[wn * NT + jn]);
        const float rho = p.row_scale ? f16_bits_to_f32(p.row_scale[n / p.rho_rows]) : 1.f;
        const float bias = p.bias ? p.bias[n] : 0.f;
#pragma unroll
        for (int i = 0; i < MT; ++i) {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int64_t m = m0 + wm * 32 * MT + i * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
                if (m >= p.M) continue;
                float v = acc[i][jn][r] * inv_sigma;      // exact
                v = v * rho;
                v = v * p.alpha;
                v = v + bias;
                const int64_t idx = m * p.N + n;
                if (p.y_dtype == TQ_F32) ((float*)p.y)[idx] = v;
                else ((uint16_t*)p.y)[idx] = f32_to_bf16_rne(v);
            }
        }
    }
}

// Pre-pass of rb_matmul_ws: bf16 x -> fp16, once per call instead of once per
// N-tile workgroup.  A workgroup converts rows 256 by, columns 128 bx (four
// K-slices); a chunk of 8 activations that fp16 cannot hold exactly becomes
// zeros, and bit t of a slice's flag word says that rows 32 t .. 32 t + 31
// of this row block hold such a chunk (the prefill replays those slices in
// bf16, with the MFMAs of the flagged 32-row tiles only).  Every flag word
// is written by exactly one workgroup, so nothing needs clearing first.
constexpr int kXcRows = 256, kXcCols = 128;
static_assert(kXcRows == BM && kXcCols % BK == 0, "flags per prefill row block and K-slice");
__global__ void __launch_bounds__(256) xconv_kernel(const uint16_t* __restrict__ x, int64_t M,
                                                   int64_t K, int64_t nsl,
                                                   uint16_t* __restrict__ xf,
                                                   uint32_t* __restrict__ flags) {
    __shared__ uint32_t fl[kXcCols / BK];
    const int tid = threadIdx.x;
    if (tid < kXcCols / BK) fl[tid] = 0u;
    __syncthreads();
    const int64_t m0 = (int64_t)blockIdx.y * kXcRows;
    const int cc = tid & 15;                              // chunk of 8 columns
    const int64_t col = (int64_t)blockIdx.x * kXcCols + 8 * cc;
    uint32_t tiles = 0u;                                  // 32-row tiles with a bad chunk
    if (col < K) {                                        // K % 32 == 0: chunks are whole
#pragma unroll 4
        for (int i = 0; i < kXcRows / 16; ++i) {
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
                tiles |= (bad ? 1u : 0u) << (((tid >> 4) + 16 * i) >> 5);
            }
        }
    }
    if (tiles) atomicOr(&fl[cc >> 2], tiles);              // slice (col mod 128) / 32
    __syncthreads();
    if (tid < kXcCols / BK) {
        const int64_t sl = (int64_t)blockIdx.x * (kXcCols / BK) + tid;
        if (sl < nsl) flags[(int64_t)blockIdx.y * nsl + sl] = fl[tid];
    }
}

}  // namespace

hipError_t launch_rb_prefill(const RbMatmulArgs& a, hipStream_t s) {
    Params p;
    p.x = a.x;
    p.M = a.M;
    p.K = a.K;
    p.N = a.N;
    p.codes = a.codes;
    p.used = a.used;
    p.row_bytes = a.used ? rb7_row_bytes(a.K) : a.K;
    p.table = a.table;
    p.table_rows = a.table_rows;
    p.alpha = a.alpha;
    p.row_scale = a.row_scale;
    p.rho_rows = a.rho_rows;
    p.bias = a.bias;
    p.y = a.y;
    p.y_dtype = a.y_dtype;
    // vector loads: 16-byte activation rows; code rows of 16 bytes a slice
    // (bytes) or 28-byte slices on 4-byte boundaries (7-bit indices)
    const bool aligned = (((uintptr_t)a.x & 15) == 0) && (a.K % BK == 0) &&
                         (((uintptr_t)a.codes & (a.used ? 3 : 15)) == 0);
    const int64_t gx = (a.N + BN - 1) / BN, gy = (a.M + BM - 1) / BM;
    if (gx == 0 || gy == 0) return hipSuccess;
    const dim3 grid((unsigned)gx, (unsigned)gy), block(kThreads);
    p.xf = nullptr;
    p.xflags = nullptr;
    if (a.workspace && aligned && a.K > 0) {
        // activations converted once for the whole call
        uint16_t* xf = (uint16_t*)a.workspace;
        uint32_t* fl = (uint32_t*)((char*)a.workspace + rb_prefill_ws_flags_offset(a.M, a.K));
        const int64_t nsl = (a.K + BK - 1) / BK;
        hipLaunchKernelGGL(xconv_kernel, dim3((unsigned)((a.K + kXcCols - 1) / kXcCols), (unsigned)gy),
                           dim3(256), 0, s, a.x, a.M, a.K, nsl, xf, fl);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        p.xf = xf;
        p.xflags = fl;
        if (a.used) hipLaunchKernelGGL((rb_prefill_kernel<true, true, true>), grid, block, 0, s, p);
        else hipLaunchKernelGGL((rb_prefill_kernel<true, false, true>), grid, block, 0, s, p);
        return hipGetLastError();
    }
    if (a.used) {
        if (aligned) hipLaunchKernelGGL((rb_prefill_kernel<true, true, false>), grid, block, 0, s, p);
        else hipLaunchKernelGGL((rb_prefill_kernel<false, true, false>), grid, block, 0, s, p);
    } else {
        if (aligned) hipLaunchKernelGGL((rb_prefill_kernel<true, false, false>), grid, block, 0, s, p);
        else hipLaunchKernelGGL((rb_prefill_kernel<false, false, false>), grid, block, 0, s, p);
    }
    return hipGetLastError();
}

}  // namespace dmm
