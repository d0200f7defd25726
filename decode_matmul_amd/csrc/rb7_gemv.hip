// Route B GEMV over 7-bit indices (M <= 16):
//
//     y[m, n] = alpha * rho_n * sum_k x[m, k] T[used[index[n, k]]] + bias_n
//
// Semantics: "A Discrete Weight Language for Large Language Models" (Route
// B), section 8.1 (the 7-bit truncated alphabet: a layer that uses at most
// 128 of the 243 codes stores each weight as a 7-bit index into the list of
// codes it uses), with the code book, row scale and epilogue of sections
// 3.2, 3.3 and 4.2, and one code book per block of rows (section 8.3).
// Row n of the index matrix holds ceil(7 K / 8) bytes; index k is bits
// 7 k .. 7 k + 6 of the row read as a little-endian bit string.
//
// Mapping onto gfx950 (tiled path: K % 512 == 0, indices 16-byte and
// activations 4-byte aligned):
//  * The workgroup (8 waves) owns 16 rows and walks K in tiles of 16 rows x
//    512 indices (448 bytes a row), as the byte-code kernel does: each wave
//    fetches its two rows as 56 aligned 16-byte pieces, two tiles ahead, and
//    stores them in LDS rows 464 bytes apart (the 16 rows a lane group reads
//    at once fall in distinct banks); after the tile's one barrier each lane
//    reads back its 16 indices (112 bits from bit 112 c of the row, c its
//    K-slice) as four dwords and funnel-shifts them to start at bit 0, so
//    that index i is at bit 7 i for every lane: one shift (a funnel shift
//    when the index straddles two dwords) and one and-or give its LDS address.
//  * The LDS code book is composed once per workgroup: entry j is
//    T[used[j]] of the block's code book, stored as the bf16 pair
//    (hi, lo) = (bf16(v), bf16(v - hi)) in 16 copies (entry j, copy c at
//    byte 64 j + 4 c; lane l reads copy l % 16).
//  * bf16 MFMA 16x16x32 with each weight's (hi, lo) pair in two K-slots
//    against the activation twice, as in the byte-code kernel: 4 MFMAs per
//    lane and tile.
// Other shapes take a plain kernel: one wave per row at a time, lanes
// striding over K, fp32 products and sums, a wave reduction.
#include "common.h"

namespace dmm {

namespace {

constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;
constexpr int kTileK = 512;                       // indices per row and tile
constexpr int kTileRowBytes = kTileK * 7 / 8;     // 448
constexpr int kPieces = kTileRowBytes / 16;       // 28
constexpr int kPitch = kTileRowBytes + 16;        // LDS bytes per tile row
constexpr int kTileBytes = 16 * kPitch;
static_assert(2 * kTileBytes >= kWaves * 64 * 4 * 4, "a block's reduction fits two tile buffers");

constexpr int kPlainThreads = 256;                // plain kernel: 4 waves, 16 rows

struct Params {
    const uint16_t* x;
    int64_t M, K, N;
    const uint8_t* codes;      // 7-bit rows
    int64_t row_bytes;         // ceil(7 K / 8)
    const uint8_t* used;       // [128]: index -> code
    const float* table;
    int64_t table_rows;
    float alpha;
    const uint16_t* row_scale;
    int64_t rho_rows;
    const float* bias;
    void* y;
    int y_dtype;
};

// Code-book value of index j (codes 243..255 in the list read zero).
__device__ __forceinline__ float index_value(const Params& p, const float* table, int j) {
    const uint32_t c = p.used[j];
    const float v = table[c < 243 ? c : 0];
    return c < 243 ? v : 0.f;
}

// LDS byte address (index << SH) + lane_off of index i (constant after
// unrolling) of indices held at bits 7 i of F; SH = log2 of an entry's bytes.
template <int SH>
__device__ __forceinline__ uint32_t index_addr(const uint32_t* F, int i, uint32_t lane_off) {
    const int bit = 7 * i, d = bit >> 5, o = bit & 31;
    uint32_t v;
    if (o + 7 <= 32) v = o >= SH ? F[d] >> (o - SH) : F[d] << (SH - o);
    else v = __builtin_amdgcn_alignbit(F[d + 1], F[d], (uint32_t)(o - SH));
    return (v & (0x7fu << SH)) | lane_off;
}

__device__ __forceinline__ void epilogue(const Params& p, int64_t n, int m, float v) {
    const float rho = p.row_scale ? f16_bits_to_f32(p.row_scale[n / p.rho_rows]) : 1.f;
    const float bias = p.bias ? p.bias[n] : 0.f;
    v = v * rho;
    v = v * p.alpha;
    v = v + bias;
    const int64_t idx = (int64_t)m * p.N + n;
    if (p.y_dtype == TQ_F32) ((float*)p.y)[idx] = v;
    else ((uint16_t*)p.y)[idx] = f32_to_bf16_rne(v);
}

// NB = 2: a workgroup of 16 waves owns two adjacent 16-row blocks (8 waves
// each, one code book, one barrier per tile for all 16), as in the byte-code
// kernel: two 8-wave workgroups on one compute unit drift apart, one keeps
// both blocks in step.  Its code book has 64 copies (every lane its own
// bank); the 8-wave form keeps 16.
template <int NB>
__global__ void __launch_bounds__(kThreads * NB, 2 / NB)
rb7_gemv_tiled_kernel(Params p) {
    constexpr int kCopies = NB == 2 ? 64 : 16;
    constexpr int kEntryShift = NB == 2 ? 8 : 6;           // log2(4 kCopies)
    constexpr int kPerEntry = kThreads * NB / 128;         // threads filling one entry
    __shared__ __attribute__((aligned(16))) unsigned char lut[128 * 4 * kCopies];
    // tile t of block b in tiles[NB (t & 1) + b]; after the loop block b's
    // partial sums take tiles[2 b] and tiles[2 b + 1]
    __shared__ __attribute__((aligned(16))) unsigned char tiles[2 * NB][kTileBytes];

    const int tid = threadIdx.x;
    const int wave_all = readfirstlane(tid >> 6);   // wave-uniform: scalar loop bounds
    const int blk = wave_all / kWaves;              // row block of this wave
    const int wave = wave_all % kWaves;             // its role in the block
    const int lane = tid & 63;
    const int64_t row0 = (xcd_block(blockIdx.x, gridDim.x) * NB + blk) * 16;
    const int64_t ntiles = p.K / kTileK;          // >= 1: the launcher requires K >= kTileK

    // fetch: piece (lane % 28) of tile row 2 wave + lane / 28 (lanes 56..63
    // load a piece again and store nothing)
    const int lrow = min(2 * wave + lane / kPieces, 15);
    const int lpiece = lane % kPieces;
    const bool writer = lane < 2 * kPieces;
    const uint8_t* grow = p.codes + min(row0 + lrow, p.N - 1) * p.row_bytes + 16 * lpiece;
    // what this lane multiplies: row (lane & 15), K-slice 4 wave + (lane >> 4)
    // of 16 indices, against 16 activations of token (lane & 15)
    const int col = lane & 15;
    const int rchunk = 4 * wave + (lane >> 4);                  // 16 indices: bit 112 rchunk
    const int rd0 = (112 * rchunk) >> 5;
    const uint32_t rsh = (uint32_t)((112 * rchunk) & 31);
    const bool a_ok = col < p.M;
    const uint16_t* xrow = p.x + (a_ok ? col : 0) * p.K + 16 * rchunk;

    struct Stage {
        u32x4 c;
        uint32_t X[8];
    };
    auto fetch = [&](int64_t t, Stage& S) {
        const int64_t tc = min(t, ntiles - 1);
        S.c = __builtin_nontemporal_load((const u32x4*)(grow + tc * kTileRowBytes));   // read once: streaming
        const u32x4a* xp = (const u32x4a*)(xrow + tc * kTileK);
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const u32x4a a = xp[i];
            S.X[4 * i] = a.x; S.X[4 * i + 1] = a.y; S.X[4 * i + 2] = a.z; S.X[4 * i + 3] = a.w;
        }
    };

    // the list entry is read ahead of the tiles; the book entry it names is
    // read behind them (waiting for it waits for the first two tiles too)
    const int lj = tid / kPerEntry;                            // code-book entry 0..127
    const uint32_t uc = p.used[lj];
    Stage s0, s1;
    fetch(0, s0);
    fetch(1, s1);
    {   // entry lj, copies (kCopies / kPerEntry) (tid % kPerEntry) .. (the book
        // of the workgroup's first row: both blocks share it)
        const float* table = rb_table_of(p.table, p.table_rows, row0 - 16 * blk);
        const float tv = table[uc < 243 ? uc : 0];
        const uint32_t e = split_bf16_pair(uc < 243 ? tv : 0.f);
        unsigned char* base = lut + lj * 4 * kCopies + (tid % kPerEntry) * 4 * (kCopies / kPerEntry);
#pragma unroll
        for (int i = 0; i < kCopies / kPerEntry / 4; ++i) *(u32x4*)(base + 16 * i) = u32x4{e, e, e, e};
    }

    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    // copy (lane % kCopies); the empty asm hides its known bits, so that each
    // address stays one and-or rather than an and plus an add
    uint32_t lane_off = (uint32_t)(lane & (kCopies - 1)) << 2;
    asm volatile("" : "+v"(lane_off));

    // tile t goes to LDS buffer t & 1: the barrier after writing tile t also
    // orders every read of tile t - 2 (same buffer) before its overwrite
    auto step = [&](const Stage& S, int buf) {
        // keep the next stage's work (it waits on younger loads) out of this step
        __builtin_amdgcn_sched_barrier(0);
        unsigned char* tile = tiles[NB * buf + blk];
        if (writer) *(u32x4*)(tile + lrow * kPitch + 16 * lpiece) = S.c;
        __syncthreads();
        const uint32_t* r = (const uint32_t*)(tile + col * kPitch) + rd0;
        const uint32_t D0 = r[0], D1 = r[1], D2 = r[2], D3 = r[3];
        const uint32_t F[4] = {__builtin_amdgcn_alignbit(D1, D0, rsh),
                               __builtin_amdgcn_alignbit(D2, D1, rsh),
                               __builtin_amdgcn_alignbit(D3, D2, rsh), D3 >> rsh};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            u32x4 aq, bq;
            // lanes of tokens >= M hold token 0's activations: they only feed
            // rows of C that are never stored
            const uint32_t x01 = S.X[2 * j], x23 = S.X[2 * j + 1];
            aq[0] = perm_b32(x01, x01, 0x01000100u);
            aq[1] = perm_b32(x01, x01, 0x03020302u);
            aq[2] = perm_b32(x23, x23, 0x01000100u);
            aq[3] = perm_b32(x23, x23, 0x03020302u);
#pragma unroll
            for (int i = 0; i < 4; ++i)
                bq[i] = *(const uint32_t*)(lut + index_addr<kEntryShift>(F, 4 * j + i, lane_off));
            acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, aq),
                                                          __builtin_bit_cast(bf16x8, bq), acc,
                                                          0, 0, 0);
        }
    };

    int64_t t = 0;
    for (; t + 1 < ntiles; t += 2) {
        step(s0, 0);
        fetch(t + 2, s0);
        step(s1, 1);
        fetch(t + 3, s1);
    }
    if (t < ntiles) step(s0, 0);

    // partials of a block's 8 waves meet in two (now idle) tile buffers;
    // C[4 (lane >> 4) + i][lane & 15] is token 4 (lane >> 4) + i, row lane & 15
    __syncthreads();
    float* red = (float*)tiles[2 * blk];                          // [kWaves][64][4]
#pragma unroll
    for (int i = 0; i < 4; ++i) red[(wave * 64 + lane) * 4 + i] = acc[i];
    __syncthreads();
    if (wave == 0) {
        const int64_t n = row0 + col;
        if (n < p.N) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int m = 4 * (lane >> 4) + i;
                if (m >= p.M) continue;
                float v = red[lane * 4 + i];
                for (int w = 1; w < kWaves; ++w) v += red[(w * 64 + lane) * 4 + i];
                epilogue(p, n, m, v);
            }
        }
    }
}

// Index k of a 7-bit row of `row_bytes` bytes (byte-granular reads).
__device__ __forceinline__ uint32_t load_index(const uint8_t* row, int64_t row_bytes, int64_t k) {
    const int64_t bit = 7 * k;
    const int64_t b = bit >> 3;
    uint32_t v = row[b];
    if (b + 1 < row_bytes) v |= (uint32_t)row[b + 1] << 8;
    return (v >> (bit & 7)) & 0x7fu;
}

// Any shape and alignment: 16 rows per workgroup, each wave takes four of
// them in turn.
__global__ void __launch_bounds__(kPlainThreads)
rb7_gemv_plain_kernel(Params p) {
    __shared__ float lut[128];
    const int tid = threadIdx.x;
    const int wave = tid >> 6, lane = tid & 63;
    const int64_t row0 = (int64_t)blockIdx.x * 16;
    if (tid < 128) lut[tid] = index_value(p, rb_table_of(p.table, p.table_rows, row0), tid);
    __syncthreads();
    for (int r = 0; r < 4; ++r) {
        const int64_t n = row0 + 4 * wave + r;
        if (n >= p.N) break;
        const uint8_t* row = p.codes + n * p.row_bytes;
        float acc[16];
#pragma unroll
        for (int m = 0; m < 16; ++m) acc[m] = 0.f;
        for (int64_t k = lane; k < p.K; k += 64) {
            const float w = lut[load_index(row, p.row_bytes, k)];
#pragma unroll
            for (int m = 0; m < 16; ++m)
                if (m < p.M) acc[m] += w * bf16_bits_to_f32(p.x[(int64_t)m * p.K + k]);
        }
#pragma unroll
        for (int m = 0; m < 16; ++m) {
            float v = acc[m];
            for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
            if (lane == 0 && m < p.M) epilogue(p, n, m, v);
        }
    }
}

}  // namespace

hipError_t launch_rb7_gemv(const RbMatmulArgs& a, hipStream_t s) {
    Params p;
    p.x = a.x;
    p.M = a.M;
    p.K = a.K;
    p.N = a.N;
    p.codes = a.codes;
    p.row_bytes = rb7_row_bytes(a.K);
    p.used = a.used;
    p.table = a.table;
    p.table_rows = a.table_rows;
    p.alpha = a.alpha;
    p.row_scale = a.row_scale;
    p.rho_rows = a.rho_rows;
    p.bias = a.bias;
    p.y = a.y;
    p.y_dtype = a.y_dtype;
    const int64_t blocks = (a.N + 15) / 16;
    if (blocks == 0 || a.M == 0) return hipSuccess;
    // whole tiles and 16-byte aligned rows (7 K / 8 is then a multiple of 448)
    const bool tiled = a.K >= kTileK && (a.K % kTileK == 0) &&
                       (((uintptr_t)a.codes & 15) == 0) && (((uintptr_t)a.x & 3) == 0);
    if (tiled) {
        // two row blocks a workgroup when that still gives every compute unit
        // one, and both blocks use one code book
        const bool pair = blocks >= 2 * (int64_t)compute_unit_count() &&
                          (a.table_rows == 0 || a.table_rows % 32 == 0);
        if (pair)
            hipLaunchKernelGGL(rb7_gemv_tiled_kernel<2>, dim3((unsigned)((blocks + 1) / 2)),
                               dim3(2 * kThreads), 0, s, p);
        else
            hipLaunchKernelGGL(rb7_gemv_tiled_kernel<1>, dim3((unsigned)blocks), dim3(kThreads), 0, s, p);
    } else
        hipLaunchKernelGGL(rb7_gemv_plain_kernel, dim3((unsigned)blocks), dim3(kPlainThreads), 0,
                           s, p);
    return hipGetLastError();
}

}  // namespace dmm
