// Ternary GEMV for 5 to 16 dense tokens: y = x (s T)^T with G = 64 and one
// plane, decoded inside the kernel.
//
// Format: pack-unpack-run, "Five trits in a byte" (five base-3 digits per
// byte, least significant first) and "Three values and a shared scale"
// (W_hat = s t per group of 64).
//
// A wave owns a slice of four groups of K and walks the 16-row blocks of its
// workgroup's rows; its activations for the slice stay in registers.  The
// multiply is the 16x16x32 bf16 MFMA at full width (16 tokens x 16 rows),
// with one accumulator per group so that the group's fp16 scale is applied
// in fp32:
//  * lane (c, r) = (lane / 16, lane % 16) supplies row r (B) or token r (A)
//    and K-chunk c of each MFMA.  Within a group it owns trits 16c .. 16c+15,
//    which all lie in the four bytes 3c .. 3c+3: one unaligned dword.
//  * its B operands hold every digit of those four bytes in a fixed order:
//    digits 0..3 of bytes 0, 1 (first 16x16x32 MFMA) and of bytes 2, 3
//    (second) from an LDS code book of ready bf16 pairs, then digit 4 of
//    bytes 0, 2, 1, 3 (a 16x16x16 MFMA) from packed 16-bit arithmetic;
//  * its A operands hold the activations of the same K positions, and zero
//    where a digit belongs to the neighbouring lane (bytes 3c and 3c+3 are
//    shared) or to the padding, so every trit is counted once;
//  * the group's sum is scaled by its fp16 scale in fp32 and added to the
//    lane's 4 tokens of row r.
// The partial sums of the K slices meet in LDS and are added in a fixed
// order, so results are bit-reproducible.
#include "common.h"
#include "tq_book.h"

namespace dmm {

namespace {

constexpr int kW = 16;
constexpr int kT = 64 * kW;
constexpr int kNB = 13;                  // code bytes per group of 64 trits
// floats of one wave's partial sums, stored value-major ([4][64]: value v of
// lane l at 64 v + l); the 16 padding floats put the slices that a lane
// group adds 16 banks apart, so a wave's 64 reads hit 64 distinct banks
constexpr int kPart = 64 * 4 + 16;
constexpr int kTileBytes = 17920;        // code + scale tile of a super-block, largest K
constexpr int kBookBytes = 256 * 256;    // code book: 256 entries x 32 copies x 8 bytes
constexpr int kRedBytes = kW * kPart * 4;  // partial sums of a super-block
constexpr int kXPieces = 8;              // staged x: 16-byte pieces per thread (16 tokens x 4096)
constexpr int kXStageMinM = 9;           // activations staged in LDS from this many tokens

typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x2a __attribute__((ext_vector_type(2), aligned(4)));

struct BatchParams {
    const uint16_t* x;
    int64_t K, N;
    int ng, M;
    const uint8_t* codes;
    const uint16_t* scales;
    int pitch, spitch;           // LDS bytes of a code / scale row of a tile
    int lnks;                    // log2 of the 4-group slices of K
    int lT;                      // log2 of the lanes that add up one output
    int lxpr;                    // staged x: log2 of the 16-byte pieces of a row
    int rows_per_wg;
    void* y;
    int y_dtype;
};

// Operands of one group on one lane: A0, A1 (16x16x32) and A2 (16x16x16).
struct GroupA {
    u32x4 a0, a1;
    u32x2 a2;
};

// Activations of lane (c, t) for group g: elements 64 g + 15 c .. + 18 of
// token t's row, as the ten dwords from the even element at or below the
// first (all inside the group), from the row in memory ...
__device__ __forceinline__ void load_group_x(const uint16_t* xrow, int g, int c, uint32_t (&X)[10]) {
    const uint16_t* p = xrow + ((64 * g + 15 * c) & ~1);
    const u32x4 v0 = *(const u32x4a*)(p), v1 = *(const u32x4a*)(p + 8);
    const u32x2 v2 = *(const u32x2a*)(p + 16);
    X[0] = v0.x; X[1] = v0.y; X[2] = v0.z; X[3] = v0.w;
    X[4] = v1.x; X[5] = v1.y; X[6] = v1.z; X[7] = v1.w;
    X[8] = v2.x; X[9] = v2.y;
}

// ... or from the row staged in LDS at xs.
__device__ __forceinline__ void lds_group_x(const unsigned char* xs, int g, int c, uint32_t (&X)[10]) {
    const unsigned char* p = xs + 2 * ((64 * g + 15 * c) & ~1);
#pragma unroll
    for (int q = 0; q < 10; q += 2) {
        const u32x2 v = *(const u32x2a*)(p + 4 * q);
        X[q] = v.x;
        X[q + 1] = v.y;
    }
}

// Masks of the lane's A operands: digits of the first byte below c and of
// the last byte above c are the neighbours'.  (Rows of A past M need no
// mask: they only reach rows of the product that are never written.)
struct AMask {
    uint32_t m0, m1, m6, m7;
};

__device__ __forceinline__ AMask a_masks(int c) {
    AMask k;
    k.m0 = (c <= 0 ? 0x0000FFFFu : 0u) | (c <= 1 ? 0xFFFF0000u : 0u);
    k.m1 = (c <= 2 ? 0x0000FFFFu : 0u) | 0xFFFF0000u;
    k.m6 = 0x0000FFFFu | (c >= 1 ? 0xFFFF0000u : 0u);
    k.m7 = (c >= 2 ? 0x0000FFFFu : 0u) | (c >= 3 ? 0xFFFF0000u : 0u);
    return k;
}

// The lane's A operands for one group, in the K order of its B operands:
// element 15 c + 5 j + d of the group for digit d of byte j, zero where the
// trit is not the lane's (the first byte's digits below c, the last byte's
// digits above c, the last byte's digit 4).
__device__ __forceinline__ GroupA build_group_a(const uint32_t (&X)[10], uint32_t sh, const AMask& k) {
    uint32_t Y[10];                                    // Y[q]: elements 2q, 2q + 1 of the lane's run
#pragma unroll
    for (int q = 0; q < 10; ++q) Y[q] = align_bytes(q + 1 < 10 ? X[q + 1] : 0u, X[q], sh);
    GroupA A;
    // digits 0..3 of bytes 0, 1: elements 0..3, 5..8
    A.a0 = u32x4{Y[0] & k.m0, Y[1] & k.m1, align_bytes(Y[3], Y[2], 2), align_bytes(Y[4], Y[3], 2)};
    // digits 0..3 of bytes 2, 3: elements 10..13, 15..18
    A.a1 = u32x4{Y[5], Y[6], align_bytes(Y[8], Y[7], 2) & k.m6, align_bytes(Y[9], Y[8], 2) & k.m7};
    // digit 4 of bytes 0, 2 | 1, 3: elements 4, 14 | 9 (byte 3's is not the lane's)
    A.a2 = u32x2{perm_b32(Y[7], Y[2], 0x05040100u), Y[4] >> 16};
    return A;
}

// Workgroup w owns rows [w rows_per_wg, ...), taken in super-blocks of
// 16 nrs rows (13 KB of codes and 2 KB of scales at every K).  A super-block
// is loaded with coalesced 16-byte pieces, two super-blocks ahead, and stored
// to an LDS tile; after one barrier wave (ks, rs) multiplies 16-row block rs
// of it by the 4-group slice ks of K.  The slices' partial sums of a
// super-block are added up after the next barrier, by all waves.
// XS: the activations go through LDS (more than 8 tokens: every workgroup
// reads all of x, and coalesced pieces cost less than per-lane windows of 16
// token rows); otherwise each lane reads its windows directly, and the code
// book is filled while they are in flight.
template <bool XS>
__global__ void __launch_bounds__(kT, 1) tq_batch_kernel(BatchParams p) {
    // code book at LDS address 0 (a lookup address is one v_perm), then two
    // tiles and two sets of partial sums
    __shared__ __attribute__((aligned(16))) unsigned char smem[kBookBytes + 2 * kTileBytes + 2 * kRedBytes];
    unsigned char* const lut = smem;
    unsigned char* const tiles = smem + kBookBytes;
    float* const red = (float*)(smem + kBookBytes + 2 * kTileBytes);

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = readfirstlane(tid >> 6);
    // read here, before the first branch, so that their argument loads go out
    // with the others (one trip to memory before the first load, not two)
    const int rows_per_wg = p.rows_per_wg;
    const uint8_t* const codes = p.codes;
    const uint16_t* const scales = p.scales;
    asm volatile("" ::"s"(rows_per_wg), "s"(codes), "s"(scales));
    const int64_t r0 = (int64_t)blockIdx.x * rows_per_wg;
    const int nrows = (int)(min(r0 + (int64_t)rows_per_wg, p.N) - r0);
    const int lnks = p.lnks;                          // log2 of the 4-group slices of K (2, 3, 4)
    const int nks = 1 << lnks;
    const int ks = wave & (nks - 1), rs = wave >> lnks;
    const int lsbr = 8 - lnks;                        // super-block rows 16 nrs = 256 / nks
    const int sbr = 1 << lsbr;
    const int nsb = (nrows + sbr - 1) >> lsbr;
    const int c = lane >> 4, r = lane & 15;
    const uint32_t rb = (uint32_t)p.ng * kNB;         // code bytes of a row
    const uint32_t sbb = rb << lsbr;                  // code bytes of a super-block (13312)
    const uint32_t sbs = (uint32_t)p.ng << (lsbr + 1);   // scale bytes (2048)

    // ---- thread tid moves piece tid of a super-block: code pieces first
    // (sbb / 16 of them), then scale pieces.  Rows past the workgroup's last
    // row (and super-blocks past its last one) read its last row again, a
    // cache hit, so that no launch fetches a neighbour's rows from HBM.
    const int ncp = (int)(sbb >> 4);
    const bool is_code = tid < ncp;
    const int sp = tid - ncp;                         // scale piece when >= 0
    const bool stores = is_code || sp < (int)(sbs >> 4);
    const uint8_t* src = is_code ? codes : (const uint8_t*)scales;
    int prow, pcol;                                   // row and byte of the piece in the super-block
    {
        const int ppr = is_code ? (int)(rb >> 4) : (p.ng >> 3);   // 16-byte pieces of a row
        const int piece = is_code ? tid : (stores ? sp : 0);
        prow = piece / ppr;
        pcol = 16 * (piece - prow * ppr);
    }
    const uint32_t rowb = is_code ? rb : 2u * (uint32_t)p.ng;   // bytes of a row
    auto load_sb = [&](int k) {
        const int row = min((k << lsbr) + prow, nrows - 1);
        const uint32_t o = (uint32_t)(r0 + row) * rowb + (uint32_t)pcol;
        return __builtin_nontemporal_load((const u32x4a*)(src + o));
    };
    // LDS destination of the piece in a tile: row-padded code rows, then
    // row-padded scale rows (conflict-free reads)
    const uint32_t dst = is_code ? (uint32_t)(prow * p.pitch + pcol)
                                 : (uint32_t)(sbr * p.pitch + prow * p.spitch + pcol);
    // ---- activations first and the first two super-blocks right behind them
    // (memory counters retire in order, so waiting for x does not wait for
    // the code stream).  Rows of A past M read token 0 and feed unwritten
    // outputs.
    u32x4 R0, R1;
    GroupA A[4];
    const AMask mk = a_masks(c);
    const uint32_t xsh = 2u * (uint32_t)(c & 1);      // the lane's first element is odd when c is
    if constexpr (XS) {
        // x through LDS as coalesced 16-byte pieces, one half of K at a time
        // in the tiles' space, so that the code book is filled while the
        // pieces are in flight.  Token rows are padded by 16 bytes so that
        // the 16 tokens fall in distinct banks.
        const int lpr = p.lxpr;
        const int xp = p.M << lpr;
        u32x4 XP[kXPieces];
#pragma unroll
        for (int j = 0; j < kXPieces; ++j) {
            const int q = min(tid + kT * j, xp - 1);
            XP[j] = *(const u32x4a*)(p.x + 8 * (int64_t)q);
        }
        R0 = load_sb(0);
        R1 = load_sb(1);
        fill_book(lut, tid);
        // every piece of this thread lies in K half (tid >> (lpr - 1)) & 1
        // (kT is a multiple of the pieces of a row); the waves of slices
        // ks < nks / 2 read half 0
        const int hb = lpr - 1;
        const int half = (tid >> hb) & 1;
        const int xhp = (int)p.K + 16;                // LDS bytes of a half row
        const unsigned char* xs = tiles + (r < p.M ? r : 0) * xhp;
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
            if (half == hh) {
#pragma unroll
                for (int j = 0; j < kXPieces; ++j) {
                    const int q = tid + kT * j;
                    if (q < xp) {
                        const int t = q >> lpr;
                        *(u32x4*)(tiles + t * xhp + 16 * (q - (t << lpr) - (hh << hb))) = XP[j];
                    }
                }
            }
            __syncthreads();
            if ((ks >= (nks >> 1)) == (hh == 1)) {
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    uint32_t X[10];
                    lds_group_x(xs, 4 * ks + i - hh * (p.ng >> 1), c, X);
                    A[i] = build_group_a(X, xsh, mk);
                }
            }
            __syncthreads();                          // the staged half is read
        }
    } else {
        uint32_t XR[4][10];
        const uint16_t* xrow = p.x + (int64_t)(r < p.M ? r : 0) * p.K;
#pragma unroll
        for (int i = 0; i < 4; ++i) load_group_x(xrow, 4 * ks + i, c, XR[i]);
        R0 = load_sb(0);
        R1 = load_sb(1);
        __builtin_amdgcn_sched_barrier(0);
        fill_book(lut, tid);
#pragma unroll
        for (int i = 0; i < 4; ++i) A[i] = build_group_a(XR[i], xsh, mk);
    }

    const uint32_t cofs = (uint32_t)(lane & 31) << 3;    // code-book copy lane % 32

    // ---- reduction of super-block k by every thread: output (m, n) of the
    // super-block takes lanes q = tid & (T - 1) of a group of T, which add
    // slices q, q + T, ... (at most four a lane: nks / T <= 4 for every K
    // and M) and then sum across the group in a fixed order.  T is chosen so
    // that one pass covers the super-block, so every index is set up once.
    const int lT = p.lT, T = 1 << lT;
    const int rq = tid & (T - 1);
    const int ro = tid >> lT;                         // output of this lane group
    const int rn = ro & (sbr - 1), rm = ro >> lsbr;
    const bool rvalid = rm < p.M && rq == 0;
    const int rsrc = ((rn >> 4) << lnks) * kPart + 64 * (rm & 3) + 16 * ((rm & 15) >> 2) + (rn & 15);
    const uint32_t ry = (uint32_t)min(rm, p.M - 1) * (uint32_t)p.N + (uint32_t)rn;   // y index less r0 and the super-block
    auto reduce = [&](int k) {
        const float* src_p = red + (k & 1) * kW * kPart + rsrc;
        float v[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int w = rq + (j << lT);             // (read clamped into the slices)
            const float r = src_p[min(w, nks - 1) * kPart];
            v[j] = w < nks ? r : 0.f;
        }
        float sum = (v[0] + v[1]) + (v[2] + v[3]);
        // groups of T consecutive lanes: pairwise in a fixed order
        if (T >= 2) sum += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, sum), 0xB1, 0xF, 0xF, true));
        if (T >= 4) sum += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, sum), 0x4E, 0xF, 0xF, true));
        if (rvalid && rn < nrows - (k << lsbr)) {
            const float r = 0.5f * sum;               // the code book holds 2t
            const uint32_t yi = ry + (uint32_t)(r0 + (k << lsbr));
            if (p.y_dtype == TQ_F32) ((float*)p.y)[yi] = r;
            else ((uint16_t*)p.y)[yi] = f32_to_bf16_rne(r);
        }
    };

    // super-block k: store the pieces loaded two steps ago, load k + 2 into
    // the same registers, one barrier, then the previous super-block's sums
    // and this one's products
    auto step = [&](int k, u32x4& R) {
        unsigned char* tile = tiles + (k & 1) * kTileBytes;
        const bool live = k < nsb;                    // uniform
        if (live && stores) {
            *(u32x2*)(tile + dst) = u32x2{R.x, R.y};
            *(u32x2*)(tile + dst + 8) = u32x2{R.z, R.w};
        }
        R = load_sb(k + 2);
        if (!live) return;
        __syncthreads();
        if (k > 0) reduce(k - 1);
        if ((rs << 4) < nrows - (k << lsbr)) {
            const unsigned char* trow = tile + ((rs << 4) + r) * p.pitch;
            const unsigned char* srow = tile + (sbr * p.pitch) + ((rs << 4) + r) * p.spitch;
            const u32x2 S = *(const u32x2*)(srow + 8 * ks);
            // the four groups in phases (code words, lookups, then the three
            // MFMAs of every group in turn), so that the groups' MFMA chains
            // interleave instead of waiting on each other
            uint32_t W[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const uint32_t byte = (uint32_t)(kNB * (4 * ks + i) + 3 * c);
                const u32x2 d = *(const u32x2a*)(trow + (byte & ~3u));
                W[i] = align_bytes(d.y, d.x, byte & 3u);
            }
            uint2 e[4][4];
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    e[i][j] = *(const uint2*)(lut + perm_b32(W[i], cofs, 0x0c0c0400u + ((uint32_t)j << 8)));
            f32x4 acc[4];
#pragma unroll
            for (int i = 0; i < 4; ++i)
                acc[i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                    __builtin_bit_cast(bf16x8, A[i].a0),
                    __builtin_bit_cast(bf16x8, u32x4{e[i][0].x, e[i][0].y, e[i][1].x, e[i][1].y}),
                    f32x4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
#pragma unroll
            for (int i = 0; i < 4; ++i)
                acc[i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                    __builtin_bit_cast(bf16x8, A[i].a1),
                    __builtin_bit_cast(bf16x8, u32x4{e[i][2].x, e[i][2].y, e[i][3].x, e[i][3].y}),
                    acc[i], 0, 0, 0);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                // digit 4 of bytes (0, 2) and (1, 3)
                const u32x2 q = {t4pair(W[i] & 0x00FF00FFu), t4pair(perm_b32(W[i], W[i], 0x0c030c01u))};
                acc[i] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(bf16x4, A[i].a2),
                                                                   __builtin_bit_cast(bf16x4, q), acc[i], 0, 0, 0);
            }
            f32x4 tot = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const uint32_t sw = (i < 2 ? S.x : S.y) >> (16 * (i & 1));
                const float sc = (float)__builtin_bit_cast(_Float16, (uint16_t)sw);
#pragma unroll
                for (int v = 0; v < 4; ++v) tot[v] = __builtin_fmaf(sc, acc[i][v], tot[v]);
            }
            // D[4 c + v][r]: token 4c + v of row r of the block, value-major
            float* dst_p = red + ((k & 1) * kW + wave) * kPart + lane;
#pragma unroll
            for (int v = 0; v < 4; ++v) dst_p[64 * v] = tot[v];
        }
    };
    // two steps a trip, so that super-blocks k and k + 1 stay in their own
    // registers; every load is issued (past the end they are not used), so
    // that each wait is for the older super-block only
    for (int k = 0; k < nsb; k += 2) {
        step(k, R0);
        step(k + 1, R1);
    }
    __syncthreads();
    reduce(nsb - 1);
}

}  // namespace

bool launch_tq_batch(const TqMatmulArgs& a, hipStream_t s, hipError_t* err) {
    if (a.G != 64 || a.n_experts != 0 || a.planes != 1 || a.M < 5 || a.M > 16 || a.N < 1) return false;
    const int64_t ng = a.K / 64;
    // 4-group slices of K: 4, 8 or 16 (code rows of a multiple of 16 bytes)
    if (a.K != 1024 && a.K != 2048 && a.K != 4096) return false;
    if (((uintptr_t)a.x & 3) != 0 || ((uintptr_t)a.codes[0] & 3) != 0 ||
        ((uintptr_t)a.scales[0] & 3) != 0)
        return false;
    if (a.N * ng * kNB >= (1ll << 31)) return false;   // 32-bit byte offsets
    BatchParams p;
    p.x = a.x;
    p.K = a.K;
    p.N = a.N;
    p.ng = (int)ng;
    p.M = (int)a.M;
    p.codes = a.codes[0];
    p.scales = a.scales[0];
    // code rows: a multiple of 16 bytes, at least 4 past the row, and
    // pitch / 4 == 4 (mod 8) so that 16 rows start in distinct bank quads;
    // scale rows: pitch / 4 == 2 (mod 4) for 8-byte reads of 16 rows
    const int rb = (int)ng * kNB;
    int pd = (rb + 4 + 3) / 4;
    while (pd % 8 != 4) ++pd;
    p.pitch = 4 * pd;
    p.spitch = 4 * ((int)ng / 2 + 2);
    p.lnks = ng == 16 ? 2 : ng == 32 ? 3 : 4;
    p.lxpr = p.lnks + 5;                         // K / 8 = 32 * 4-group slices
    const bool xs = a.M >= kXStageMinM;
    // staged x: half rows of K + 16 bytes in the space of the tiles and sums
    if (xs && a.M * (a.K + 16) > 2 * kTileBytes + 2 * kRedBytes) return false;
    const int nrs = kW >> p.lnks;
    if (16 * nrs * (p.pitch + p.spitch) > kTileBytes) return false;
    // lanes per output: the outputs of a super-block (M x 16 nrs) times the
    // lanes fit the workgroup, at most 4 and at most the slices
    const int outs = (int)a.M * 16 * nrs;
    p.lT = outs * 4 <= kT ? 2 : outs * 2 <= kT ? 1 : 0;
    const int cus = compute_unit_count();
    const int64_t rpw = (a.N + cus - 1) / cus;
    p.rows_per_wg = (int)rpw;
    p.y = a.y;
    p.y_dtype = a.y_dtype;
    const int64_t wgs = (a.N + rpw - 1) / rpw;
    if (xs) hipLaunchKernelGGL(tq_batch_kernel<true>, dim3((unsigned)wgs), dim3(kT), 0, s, p);
    else hipLaunchKernelGGL(tq_batch_kernel<false>, dim3((unsigned)wgs), dim3(kT), 0, s, p);
    *err = hipGetLastError();
    return true;
}

}  // namespace dmm
