// Route B GEMV (M <= 16): y[m, n] = alpha * rho_n * sum_k x[m, k] T[codes[n, k]] + bias_n.
//
// Semantics: "A Discrete Weight Language for Large Language Models" (Route
// B), section 3.2 (codes index a 243-entry code book), section 3.3 (per-row
// scale rho_n) and section 4.2 (the code book sits in on-chip memory, every
// code byte is dereferenced through it inside a K-sliced GEMM; rho_n
// multiplies the finished sum and the bias comes after it).  With per-block code books
// (section 8.3: one ladder per block of 32 rows) T is the book of the row's
// block; a workgroup's rows lie in one block, so it stages that one.
//
// Mapping onto gfx950:
//  * General path: the workgroup (16 waves, one per CU: the replicated table
//    fills LDS) owns 32 output rows; its waves split K into contiguous
//    ranges, each wave streams both 16-row blocks with loads two steps ahead
//    of the MFMAs, and the partials meet in LDS at the end (fixed summation
//    order).  Tiled path (K % 512 == 0): see rb_gemv_tiled_kernel.
//  * Each code byte is looked up in an LDS copy of the code book.  Every
//    fp32 entry v is stored as two bf16 terms, hi = bf16(v) and
//    lo = bf16(v - hi) (|v - hi - lo| <= 2^-17 |v|), packed as one dword.
//    The table is replicated (64 copies in the general path, entry b of copy
//    c at byte 256 b + 4 c; 32 in the tiled path, 16 when the activations
//    are staged in LDS too) so that the lanes reading
//    at once mostly hit distinct banks, and the address is a single v_perm
//    of the code dword with the lane offset.
//  * bf16 MFMA 16x16x32: B takes the looked-up (hi, lo) dword as two K-slots
//    of one weight, A holds the activation twice in the same two slots, so
//    one MFMA accumulates x*hi + x*lo = x*v for four weights per lane.
//    A rows are the M <= 16 tokens; C columns are the 16 rows.
//  * Tiled path: every workgroup walks K from the same end, so at any time
//    the chip reads one column window of all rows (measured faster than
//    staggered starts or free-running waves), and the row blocks are dealt
//    out so that each XCD streams one contiguous eighth of the matrix.
#include "common.h"

namespace dmm {

namespace {

constexpr int kWaves = 16;                // K split over the waves of a workgroup
constexpr int kThreads = 64 * kWaves;
constexpr int kRB = 2;                    // 16-row blocks per workgroup, all streamed by each wave
// tiled path: 8 waves on 16 rows; a tile is 16 rows x 512 code bytes, each
// wave fetches two of its rows and reads back a 64-column slice of all 16
constexpr int kTWaves = 8;
constexpr int kTThreads = 64 * kTWaves;
constexpr int kTileK = 64 * kTWaves;        // K bytes per tile
constexpr int kTilePitch = kTileK + 16;     // padded LDS row pitch: column reads hit distinct banks
constexpr int kTileBytes = 16 * kTilePitch;
static_assert(2 * kTileBytes >= kTWaves * 64 * 4 * 4, "reduction fits the tile buffers");
constexpr int kLutBytes = 256 * 256;       // 256 entries x 64 copies x 4 B

struct Params {
    const uint16_t* x;
    int64_t M, K, N;
    const uint8_t* codes;
    const float* table;
    int64_t table_rows;                      // 0: one code book; else rows per code book
    float alpha;
    const uint16_t* row_scale;
    int64_t rho_rows;                        // rows sharing one row_scale entry
    const float* bias;
    void* y;
    int y_dtype;
    int64_t steps;                           // ceil(K / 64)
    int64_t full_steps;                      // steps entirely inside K
};

// Raw words holding the 16 code bytes of row `row` at column k (k + 16 <= K).
// ALIGNED: row + k is 4-byte aligned, the four words are the bytes.
// Otherwise five aligned words are read (the fifth only when the bytes spill
// into it) and realigned later by realign16(), so the loads stay in flight.
template <bool ALIGNED>
__device__ __forceinline__ void load_codes_raw(const uint8_t* row, int64_t k, uint32_t* R,
                                               uint32_t& sh) {
    if constexpr (ALIGNED) {
        u32x4a v = *(const u32x4a*)(row + k);
        R[0] = v.x; R[1] = v.y; R[2] = v.z; R[3] = v.w; R[4] = 0u;
        sh = 0;
    } else {
        const uint8_t* q = row + k;
        sh = (uint32_t)((uintptr_t)q & 3);
        const uint32_t* aw = (const uint32_t*)(q - sh);
        u32x4a v = *(const u32x4a*)aw;
        R[0] = v.x; R[1] = v.y; R[2] = v.z; R[3] = v.w;
        R[4] = sh ? aw[4] : 0u;
    }
}

template <bool ALIGNED>
__device__ __forceinline__ void realign16(const uint32_t* R, uint32_t sh, uint32_t* D) {
    if constexpr (ALIGNED) {
        D[0] = R[0]; D[1] = R[1]; D[2] = R[2]; D[3] = R[3];
    } else {
        D[0] = align_bytes(R[1], R[0], sh);
        D[1] = align_bytes(R[2], R[1], sh);
        D[2] = align_bytes(R[3], R[2], sh);
        D[3] = align_bytes(R[4], R[3], sh);
    }
}

// Tail step: bytes at k + j >= K read as code 255 (a zero table entry).
__device__ __forceinline__ void load_codes16_tail(const uint8_t* row, int64_t k, int64_t K,
                                                  uint32_t* D) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        uint32_t w = 0;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            int64_t kk = k + 4 * i + j;
            uint32_t b = kk < K ? (uint32_t)row[kk] : 0xffu;
            w |= b << (8 * j);
        }
        D[i] = w;
    }
}

// 16 activations x[m][k .. k+15] as 8 bf16 pairs; zero past K.
__device__ __forceinline__ void load_x16(const uint16_t* xrow, int64_t k, int64_t K, bool tail,
                                         uint32_t* X) {
    if (!tail) {
        const u32x4a* p = (const u32x4a*)(xrow + k);
        u32x4a a = p[0], b = p[1];
        X[0] = a.x; X[1] = a.y; X[2] = a.z; X[3] = a.w;
        X[4] = b.x; X[5] = b.y; X[6] = b.z; X[7] = b.w;
    } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            int64_t k0 = k + 2 * i;
            uint32_t lo = k0 < K ? xrow[k0] : 0u;
            uint32_t hi = k0 + 1 < K ? xrow[k0 + 1] : 0u;
            X[i] = lo | (hi << 16);
        }
    }
}

template <bool ALIGNED>
__global__ void __launch_bounds__(kThreads)
rb_gemv_kernel(Params p) {
    __shared__ __attribute__((aligned(16))) unsigned char lut[kLutBytes];
    __shared__ float red[kWaves * kRB * 64 * 4];

    const int tid = threadIdx.x;
    const int wave = readfirstlane(tid >> 6);   // wave-uniform: scalar loop bounds
    const int lane = tid & 63;

    {   // entry b, copies 16 (tid & 3) .. + 15: one global read per thread
        const int b = tid >> 2;
        const float* table = rb_table_of(p.table, p.table_rows, (int64_t)blockIdx.x * 16 * kRB);
        const uint32_t e = split_bf16_pair(b < 243 ? table[b] : 0.f);
        const u32x4 q = {e, e, e, e};
        unsigned char* base = lut + b * 256 + (tid & 3) * 64;
#pragma unroll
        for (int i = 0; i < 4; ++i) *(u32x4*)(base + 16 * i) = q;
    }

    const int col = lane & 15;
    const int kb = lane >> 4;
    int64_t n[kRB];
    bool row_ok[kRB];
    const uint8_t* crow[kRB];
#pragma unroll
    for (int r = 0; r < kRB; ++r) {
        n[r] = ((int64_t)blockIdx.x * kRB + r) * 16 + col;
        row_ok[r] = n[r] < p.N;
        crow[r] = p.codes + (row_ok[r] ? n[r] : 0) * p.K;
    }
    const int am = lane & 15;                                     // A row = token
    const bool a_ok = am < p.M;
    const uint16_t* xrow = p.x + (a_ok ? am : 0) * p.K;
    const uint32_t lane_off = (uint32_t)lane << 2;

    // contiguous K range of this wave, in 64-column steps
    const int64_t per = (p.steps + kWaves - 1) / kWaves;
    const int64_t s_begin = min(p.steps, per * wave);
    const int64_t s_end = min(p.steps, s_begin + per);

    __syncthreads();

    f32x4 acc[kRB];
#pragma unroll
    for (int r = 0; r < kRB; ++r) acc[r] = f32x4{0.f, 0.f, 0.f, 0.f};

    struct Slot {
        uint32_t R[kRB][5];
        uint32_t sh[kRB];
        uint32_t X[8];
    };

    // codes of all kRB rows and 16 activations for one step.  Loads are issued
    // unconditionally (rows past N read row 0, idle A lanes read token 0) and
    // masked when consumed, so no branch separates a load from its wait.
    auto stage = [&](int64_t st, Slot& S) {
        const int64_t k = st * 64 + 16 * kb;
#pragma unroll
        for (int r = 0; r < kRB; ++r) load_codes_raw<ALIGNED>(crow[r], k, S.R[r], S.sh[r]);
        load_x16(xrow, k, p.K, false, S.X);
    };

    auto compute = [&](const uint32_t (*D)[4], const uint32_t* X) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            u32x4 aq;
            const uint32_t x01 = X[2 * j], x23 = X[2 * j + 1];
            aq[0] = perm_b32(x01, x01, 0x01000100u);
            aq[1] = perm_b32(x01, x01, 0x03020302u);
            aq[2] = perm_b32(x23, x23, 0x01000100u);
            aq[3] = perm_b32(x23, x23, 0x03020302u);
#pragma unroll
            for (int r = 0; r < kRB; ++r) {
                u32x4 bq;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const uint32_t addr =
                        perm_b32(D[r][j], lane_off, 0x0c0c0400u + ((uint32_t)i << 8));
                    bq[i] = *(const uint32_t*)(lut + addr);
                }
                acc[r] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                    __builtin_bit_cast(bf16x8, aq), __builtin_bit_cast(bf16x8, bq), acc[r], 0,
                    0, 0);
            }
        }
    };

    auto compute_slot = [&](const Slot& S) {
        uint32_t D[kRB][4], X[8];
#pragma unroll
        for (int r = 0; r < kRB; ++r) {
            realign16<ALIGNED>(S.R[r], S.sh[r], D[r]);
#pragma unroll
            for (int i = 0; i < 4; ++i) D[r][i] = row_ok[r] ? D[r][i] : 0xffffffffu;
        }
#pragma unroll
        for (int i = 0; i < 8; ++i) X[i] = a_ok ? S.X[i] : 0u;
        compute(D, X);
    };

    // steps entirely inside K: loads run two steps ahead of the MFMAs
    const int64_t s_full_end = max(s_begin, min(s_end, p.full_steps));
    int64_t st = s_begin;
    if (st < s_full_end) {
        // three register slots in rotation, no copies: while one step's MFMAs
        // run, the next two steps' loads are in flight.  Prefetches past the
        // end re-read the last full step and are never consumed.
        const int64_t last = s_full_end - 1;
        Slot s0, s1, s2;
        stage(st, s0);
        stage(min(st + 1, last), s1);
        stage(min(st + 2, last), s2);
        for (; st + 2 < s_full_end; st += 3) {
            compute_slot(s0);
            stage(min(st + 3, last), s0);
            compute_slot(s1);
            stage(min(st + 4, last), s1);
            compute_slot(s2);
            stage(min(st + 5, last), s2);
        }
        if (st < s_full_end) {
            compute_slot(s0);
            ++st;
        }
        if (st < s_full_end) {
            compute_slot(s1);
            ++st;
        }
    }
    // the ragged tail of K (and every step when rows are not 4-byte aligned)
    for (; st < s_end; ++st) {
        const int64_t k = st * 64 + 16 * kb;
        uint32_t D[kRB][4], X[8];
#pragma unroll
        for (int r = 0; r < kRB; ++r) {
            if (row_ok[r]) load_codes16_tail(crow[r], k, p.K, D[r]);
            else D[r][0] = D[r][1] = D[r][2] = D[r][3] = 0xffffffffu;
        }
        if (a_ok) load_x16(xrow, k, p.K, true, X);
        else {
#pragma unroll
            for (int i = 0; i < 8; ++i) X[i] = 0u;
        }
        compute(D, X);
    }

    // C[4*(lane>>4) + i][lane & 15]: token 4*(lane>>4)+i, row col of block r
#pragma unroll
    for (int r = 0; r < kRB; ++r)
#pragma unroll
        for (int i = 0; i < 4; ++i) red[((wave * kRB + r) * 64 + lane) * 4 + i] = acc[r][i];
    __syncthreads();
    if (wave < kRB) {
        const int r = wave;
        if (row_ok[r]) {
            const float rho = p.row_scale ? f16_bits_to_f32(p.row_scale[n[r] / p.rho_rows]) : 1.f;
            const float bias = p.bias ? p.bias[n[r]] : 0.f;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int m = 4 * kb + i;
                if (m >= p.M) continue;
                float v = red[(r * 64 + lane) * 4 + i];
                for (int w = 1; w < kWaves; ++w) v += red[((w * kRB + r) * 64 + lane) * 4 + i];
                v = v * rho;
                v = v * p.alpha;
                v = v + bias;
                const int64_t idx = (int64_t)m * p.N + n[r];
                if (p.y_dtype == TQ_F32) ((float*)p.y)[idx] = v;
                else ((uint16_t*)p.y)[idx] = f32_to_bf16_rne(v);
            }
        }
    }
}

// Fast path: codes 16-byte aligned, K % 512 == 0, x 4-byte aligned.
//
// The workgroup (8 waves, up to four per CU) owns 16 rows.  K is walked in
// tiles of 16 rows x 512 bytes: each wave fetches two rows of the tile (32
// lanes x 16 B per row), two tiles ahead in registers; the tile goes to one of
// two LDS buffers and each wave then reads its 64-column slice of all 16 rows
// in the MFMA layout, one barrier per tile.  Small workgroups with a small
// code-book copy (16 copies, 16 KB) let several workgroups share a CU, so one
// waiting at its barrier leaves the others streaming.
// XS (13 to 16 tokens): the tile's activations of all 16 token slots are
// staged in LDS by coalesced loads (thread t loads 32 bytes of token t / 32,
// so a wave instruction reads whole token rows of the tile) and each lane
// then reads its MFMA operand from there.  The direct per-lane loads gather
// 16 rows per instruction: 24.6 against 21.5 us at M = 16, N = K = 8192.
// Staging costs a fixed 16 rows of loads and LDS traffic, so below 13 tokens
// the direct loads are faster (M = 12: equal; M = 8: 19.4 against 22.0 us).
constexpr int kXPitch = 2 * kTileK + 16;     // bytes per staged token row (8 lanes of a read phase hit distinct banks)
constexpr int kXStageMinM = 13;
// NB = 2: a workgroup of 16 waves owns two adjacent 16-row blocks (8 waves
// each, one code book, one barrier per tile for all 16).  Two 8-wave
// workgroups on one compute unit drift apart (the older one's waves win the
// issue slots and it finishes about a fifth of the run earlier, leaving the
// other alone on the compute unit); one workgroup keeps both blocks in step.
template <bool XS, int NB>
__global__ void __launch_bounds__(kTThreads * NB, 2 / NB)
rb_gemv_tiled_kernel(Params p) {
    // code-book copies: 64 for one workgroup a compute unit (NB = 2; the
    // v_perm result is the address, every lane its own bank); for two, 32,
    // or 16 when the staged activations share LDS
    constexpr int kTCopies = NB == 2 ? 64 : (XS ? 16 : 32);
    __shared__ __attribute__((aligned(16))) unsigned char lut[256 * 4 * kTCopies];
    __shared__ __attribute__((aligned(16))) unsigned char tiles[2][NB][kTileBytes];
    __shared__ __attribute__((aligned(16))) unsigned char xtiles[XS ? 2 : 1][XS ? 16 * kXPitch : 16];

    const int tid = threadIdx.x;
    const int wave_all = readfirstlane(tid >> 6);   // wave-uniform: scalar loop bounds
    const int blk = wave_all / kTWaves;             // row block of this wave
    const int wave = wave_all % kTWaves;            // its role in the block
    const int lane = tid & 63;
    const int64_t row0 = (xcd_block(blockIdx.x, gridDim.x) * NB + blk) * 16;
    const int64_t ntiles = p.K / kTileK;          // >= 1: the launcher requires K >= kTileK

    // tile row this lane fetches (clamped into range), 16 bytes at 16 (lane & 31)
    const int lrow = 2 * wave + (lane >> 5);
    const uint8_t* grow = p.codes + min(row0 + lrow, p.N - 1) * p.K + 16 * (lane & 31);
    // activations of this wave's slice: token (lane & 15), 16 columns
    const int am = lane & 15;
    const bool a_ok = am < p.M;
    const int col = lane & 15;
    const int kb = lane >> 4;
    const uint16_t* xrow = p.x + (a_ok ? am : 0) * p.K + 64 * wave + 16 * kb;
    // staged activations: thread tid (< 512) loads token tid / 32 (clamped
    // to M - 1), columns 16 (tid % 32) .. + 15 of the tile; both blocks read
    // the copy that block 0's threads store
    const int xt = (tid >> 5) & 15, xc = tid & 31;
    const uint16_t* xsrc = p.x + min((int64_t)xt, p.M - 1) * p.K + 16 * xc;

    struct Stage {
        u32x4a c;
        uint32_t X[8];
    };
    auto fetch = [&](int64_t t, Stage& S) {
        const int64_t tc = min(t, ntiles - 1);
        // the codes are read once: a streaming (nontemporal) load
        S.c = __builtin_nontemporal_load((const u32x4a*)(grow + tc * kTileK));
        const u32x4a* xp = (const u32x4a*)((XS ? xsrc : xrow) + tc * kTileK);
        u32x4a a = xp[0], b = xp[1];
        S.X[0] = a.x; S.X[1] = a.y; S.X[2] = a.z; S.X[3] = a.w;
        S.X[4] = b.x; S.X[5] = b.y; S.X[6] = b.z; S.X[7] = b.w;
    };

    // the code-book read goes first so that waiting for it leaves the tile
    // loads in flight (memory counters complete in order)
    const int lb = tid / (2 * NB);
    const float tv = rb_table_of(p.table, p.table_rows, row0)[lb < 243 ? lb : 0];
    Stage s0, s1;
    fetch(0, s0);
    fetch(1, s1);

    {   // entry b, copies kTCopies / (2 NB) (tid % 2 NB) .. ; entries 243..255 read zero
        const uint32_t e = split_bf16_pair(lb < 243 ? tv : 0.f);
        const u32x4 q = {e, e, e, e};
        unsigned char* base = lut + lb * 4 * kTCopies + (tid % (2 * NB)) * 2 * kTCopies / NB;
#pragma unroll
        for (int i = 0; i < kTCopies / (8 * NB); ++i) *(u32x4*)(base + 16 * i) = q;
    }

    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    // entry b, copy c at byte 4 kTCopies b + 4 c; lane l reads copy
    // l % kTCopies: the v_perm below forms 256 b + (256 / kTCopies) (l % kTCopies),
    // shifted right by 6 - log2(kTCopies)
    constexpr uint32_t kCopyShift = kTCopies == 64 ? 0u : (kTCopies == 32 ? 1u : 2u);  // 6 - log2(kTCopies)
    const uint32_t lane_off = (uint32_t)(lane & (kTCopies - 1)) << (2 + kCopyShift);

    // tile t goes to LDS buffer t & 1: the barrier after writing tile t also
    // orders every read of tile t - 2 (same buffer) before its overwrite
    auto step = [&](const Stage& S, int buf) {
        // keep the next stage's work (it waits on younger loads) out of this step
        __builtin_amdgcn_sched_barrier(0);
        unsigned char* tile = tiles[buf][blk];
        *(u32x4*)(tile + lrow * kTilePitch + 16 * (lane & 31)) = u32x4{S.c.x, S.c.y, S.c.z, S.c.w};
        uint32_t XV[8];
        if constexpr (XS) {
            if (blk == 0) {
                unsigned char* xb = xtiles[buf] + xt * kXPitch + 32 * xc;
                *(u32x4*)xb = u32x4{S.X[0], S.X[1], S.X[2], S.X[3]};
                *(u32x4*)(xb + 16) = u32x4{S.X[4], S.X[5], S.X[6], S.X[7]};
            }
        }
        __syncthreads();
        const u32x4 v = *(const u32x4*)(tile + col * kTilePitch + 64 * wave + 16 * kb);
        const uint32_t D[4] = {v.x, v.y, v.z, v.w};
        if constexpr (XS) {
            const unsigned char* xa = xtiles[buf] + (a_ok ? am : 0) * kXPitch + 2 * (64 * wave + 16 * kb);
            const u32x4 a = *(const u32x4*)xa, b = *(const u32x4*)(xa + 16);
            XV[0] = a.x; XV[1] = a.y; XV[2] = a.z; XV[3] = a.w;
            XV[4] = b.x; XV[5] = b.y; XV[6] = b.z; XV[7] = b.w;
        } else {
#pragma unroll
            for (int q = 0; q < 8; ++q) XV[q] = S.X[q];
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            u32x4 aq, bq;
            // lanes of tokens >= M hold token 0's activations: they only feed
            // rows of C that are never stored
            const uint32_t x01 = XV[2 * j], x23 = XV[2 * j + 1];
            aq[0] = perm_b32(x01, x01, 0x01000100u);
            aq[1] = perm_b32(x01, x01, 0x03020302u);
            aq[2] = perm_b32(x23, x23, 0x01000100u);
            aq[3] = perm_b32(x23, x23, 0x03020302u);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const uint32_t addr =
                    perm_b32(D[j], lane_off, 0x0c0c0400u + ((uint32_t)i << 8)) >> kCopyShift;
                bq[i] = *(const uint32_t*)(lut + addr);
            }
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

    // partials of a block's 8 waves meet in its (now idle) tile buffer
    __syncthreads();
    float* red = (float*)tiles[0][blk];                           // [kTWaves][64][4]
#pragma unroll
    for (int i = 0; i < 4; ++i) red[(wave * 64 + lane) * 4 + i] = acc[i];
    __syncthreads();
    if (wave == 0) {
        const int64_t n = row0 + col;
        if (n < p.N) {
            const float rho = p.row_scale ? f16_bits_to_f32(p.row_scale[n / p.rho_rows]) : 1.f;
            const float bias = p.bias ? p.bias[n] : 0.f;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int m = 4 * kb + i;
                if (m >= p.M) continue;
                float v = red[lane * 4 + i];
                for (int w = 1; w < kTWaves; ++w) v += red[(w * 64 + lane) * 4 + i];
                v = v * rho;
                v = v * p.alpha;
                v = v + bias;
                const int64_t idx = (int64_t)m * p.N + n;
                if (p.y_dtype == TQ_F32) ((float*)p.y)[idx] = v;
                else ((uint16_t*)p.y)[idx] = f32_to_bf16_rne(v);
            }
        }
    }
}

}  // namespace

hipError_t launch_rb_gemv(const RbMatmulArgs& a, hipStream_t s) {
    Params p;
    p.x = a.x;
    p.M = a.M;
    p.K = a.K;
    p.N = a.N;
    p.codes = a.codes;
    p.table = a.table;
    p.table_rows = a.table_rows;
    p.alpha = a.alpha;
    p.row_scale = a.row_scale;
    p.rho_rows = a.rho_rows;
    p.bias = a.bias;
    p.y = a.y;
    p.y_dtype = a.y_dtype;
    p.steps = (a.K + 63) / 64;
    // a step is "full" when every lane's 16 bytes lie inside K
    p.full_steps = a.K / 64;
    // vector activation loads need 4-byte aligned rows; otherwise every step
    // takes the element-wise path
    if ((a.K & 1) || ((uintptr_t)a.x & 3)) p.full_steps = 0;
    const int64_t blocks = (a.N + 16 * kRB - 1) / (16 * kRB);
    if (blocks == 0 || a.M == 0) return hipSuccess;
    // tiles need at least one full tile: K = 0 (null operands) takes the
    // general path, which issues no loads at all
    const bool tiled = a.K >= kTileK && (a.K % kTileK == 0) &&
                       (((uintptr_t)a.codes & 15) == 0) && (((uintptr_t)a.x & 3) == 0);
    if (tiled) {
        // two row blocks a workgroup when that still gives every compute unit
        // one, and both blocks use one code book
        const int64_t nblk = (a.N + 15) / 16;
        const bool pair = nblk >= 2 * (int64_t)compute_unit_count() &&
                          (a.table_rows == 0 || a.table_rows % 32 == 0);
        const dim3 g1((unsigned)nblk), g2((unsigned)((nblk + 1) / 2));
        if (a.M >= kXStageMinM) {
            if (pair) hipLaunchKernelGGL((rb_gemv_tiled_kernel<true, 2>), g2, dim3(2 * kTThreads), 0, s, p);
            else hipLaunchKernelGGL((rb_gemv_tiled_kernel<true, 1>), g1, dim3(kTThreads), 0, s, p);
        } else {
            if (pair) hipLaunchKernelGGL((rb_gemv_tiled_kernel<false, 2>), g2, dim3(2 * kTThreads), 0, s, p);
            else hipLaunchKernelGGL((rb_gemv_tiled_kernel<false, 1>), g1, dim3(kTThreads), 0, s, p);
        }
        return hipGetLastError();
    }
    const bool aligned4 = (((uintptr_t)a.codes & 3) == 0) && (a.K % 4 == 0);
    if (aligned4)
        hipLaunchKernelGGL(rb_gemv_kernel<true>, dim3((unsigned)blocks), dim3(kThreads), 0, s, p);
    else
        hipLaunchKernelGGL(rb_gemv_kernel<false>, dim3((unsigned)blocks), dim3(kThreads), 0, s, p);
    return hipGetLastError();
}

}  // namespace dmm
