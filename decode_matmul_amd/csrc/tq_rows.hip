// Ternary GEMV for a few tokens over dense weights: y = x (s1 T1 + s2 T2)^T
// with G = 64, decoded inside the kernel.
//
// Format: "Does your weight format deserve a kernel?" (pack-unpack-run),
// "Five trits in a byte" and "Three values and a shared scale"; the second
// plane follows the FUCINA README ("The method").
//
// This is the streaming form for a few tokens, where the time is the HBM read
// of the package: dense calls with M <= 4, or up to 16 in passes of four when
// every block of a workgroup's range stays in its LDS tile across the passes,
// and grouped expert calls with any number of tokens per expert.  A row's codes (ng * 13 bytes) and scales (ng * 2 bytes)
// are contiguous and consecutive rows follow each other, so a range of rows
// is one contiguous byte range per array.
//
//  * One 1024-thread workgroup per compute unit owns rows_per_wg consecutive
//    rows and walks them in blocks of 16 (one MFMA column block).  A block's
//    bytes (codes and scales, every plane) are fetched as 16-byte chunks by
//    the whole workgroup, so each load instruction reads 1 KiB of one
//    contiguous range.  Four blocks are in flight in registers.  When the
//    whole range is in flight (dense calls whose range has at most four
//    blocks, 56 rows at N = 14336) every block is written to a tile of its
//    own and one barrier precedes the decode of all of them, so each wave
//    runs its quad of every block back to back; otherwise a block is written
//    to one of two LDS tiles and decoded while the next blocks arrive.
//  * Wave w owns the K-groups 4w .. 4w+3 (a quad) of every block, so its
//    activations are loaded into registers once and reused for all blocks.
//  * Decode and MFMA mapping as in the general kernel: lane l decodes group
//    4w + (l >> 4) of row (l & 15) into bf16 pairs of 2t through a table of
//    the five trits' bf16 high bytes, and the MFMA A operand is block
//    diagonal (A row 4m + g' carries token m's activations for group g' in
//    the K-slots of lane block g'), so C[4m + g', row] is one group's partial
//    sum and the fp16 group scale is applied in fp32 afterwards.
//  * The trit table has 16 copies in LDS, entry b of copy c at byte
//    (b << 8) | (c << 3), so one v_perm of the code byte and the copy offset
//    forms the address and the 16 lanes of a phase hit distinct banks.  Its
//    256 entries are a compile-time constant; each thread reads one, ahead
//    of every other load (memory counters retire in order, so a later read
//    would wait for the whole code stream), and stores four copies.
//  * Tile rows are padded to 8 mod 16 bytes so the 16 rows of a block start
//    in distinct bank pairs.
//  * Wave partials are kept per block in LDS and summed in a fixed order at
//    the end, so results do not depend on timing.
#include <algorithm>

#include "common.h"

namespace dmm {

namespace {

constexpr int kW = 16;                  // waves per workgroup
constexpr int kT = 64 * kW;             // threads per workgroup
constexpr int kNB = 13;                 // code bytes per group of 64 trits
constexpr int kNSB = 4;                 // blocks in flight (one block per thread slot)
constexpr int kLutBytes = 256 * 256;    // entry b, copy c at (b << 8) | (c << 3)
static_assert(kT == 4 * 256, "one thread per (trit-table entry, four copies)");

struct RowsParams {
    const uint16_t* x;
    int64_t K, N;
    int ng;                  // groups per row, a multiple of 16
    int M;                   // dense: tokens, 1..16 (passes of four); grouped: 0
    const uint8_t* base;     // plane-1 codes; the other arrays sit at byte offsets from it
    int64_t off_codes2, off_scales1, off_scales2;
    uint32_t mul_cc, mul_cpr, mul_sc, mul_spr;   // 2^32 / d + 1 for the chunk divisions
    int rows_per_wg;         // multiple of 8, <= 16 * kMaxBlocks
    int pitch;               // LDS bytes per tile code row (row bytes + 8)
    int spitch;              // LDS bytes per tile scale row (2 ng + 8)
    int tile_bytes;          // one LDS tile: planes * 16 * (pitch + spitch)
    int all_tiles;           // every block of the range has its own tile (no ring)
    void* y;
    int y_dtype;
    // grouped experts: workgroup w owns rows [c * rows_per_wg, ...) of expert
    // w / chunks (c = w % chunks) for the token slots routed to it
    const int32_t* ids;      // [T * top_k] expert of each (token, slot)
    int total;               // T * top_k
    int top_k;
    int chunks;              // workgroups per expert
    int n_experts;           // ids outside [0, n_experts) are invalid
    int e_begin;             // first expert of this launch
    int n_items;             // workgroups of expert rows (n_launched * chunks); one
                             // more, when present, writes the NaN rows of invalid ids
    int64_t e_codes, e_scales;   // bytes per expert in a code / scale plane
};

// Code book of byte b: trits 0..3 (digit q of b in base 3, least significant
// first, t = digit - 1) as two ready bf16 pairs (2t0, 2t1) and (2t2, 2t3),
// each value 2t stored as its high byte (0x40, 0x00 or 0xC0) over a zero low
// byte.  Trit 4 is computed arithmetically (t4pair).  Bytes 243..255 decode
// to zero.  Built at compile time.
constexpr uint32_t trit_hb(int d) { return d == 2 ? 0x40u : (d == 0 ? 0xC0u : 0x00u); }
struct TritPairs {
    uint2 e[256];
};
constexpr TritPairs make_trit_pairs() {
    TritPairs t{};
    for (int b = 0; b < 243; ++b) {
        const int d0 = b % 3, d1 = (b / 3) % 3, d2 = (b / 9) % 3, d3 = (b / 27) % 3;
        t.e[b].x = (trit_hb(d0) << 8) | (trit_hb(d1) << 24);
        t.e[b].y = (trit_hb(d2) << 8) | (trit_hb(d3) << 24);
    }
    return t;
}
__constant__ TritPairs kTritPairs = make_trit_pairs();

typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));

// Trit 4 (the most significant digit, floor(b / 81)) of two code bytes held
// in the low bytes of the two 16-bit halves, as a bf16 pair of 2 t4: with
// v = 203 b + 0xC000 (mod 2^16) bits 14..15 are digit + 3 (mod 4), since
// floor(203 b / 2^14) = floor(b / 81) for b <= 242, which the masked value
// reads as 0xC000 (-2), 0 or 0x4000 (+2).
__device__ __forceinline__ uint32_t t4pair(uint32_t bytes16) {
    u16x2 v = __builtin_bit_cast(u16x2, bytes16);
    v = v * (u16x2){203, 203} + (u16x2){0xC000, 0xC000};
    return __builtin_bit_cast(uint32_t, v) & 0xC000C000u;
}

// K order of a group inside the MFMA operands.  The 32 B-operand dwords of a
// lane (four per MFMA, eight MFMAs) are: for bytes i = 0..12 the two code-book
// pairs (t_5i, t_5i+1), (t_5i+2, t_5i+3) as dwords 2i, 2i+1; then, for the
// code dwords k = 0..2 (bytes 4k..4k+3), trit 4 of bytes (4k, 4k+2) and of
// bytes (4k+1, 4k+3) as dwords 26 + 2k and 27 + 2k.  Byte 12's trit 4 is
// padding and is not used.  The activations are placed in the same order.
__device__ __forceinline__ void permute_group_x(const uint32_t (&xw)[32], u32x4 (&A)[8]) {
    uint32_t a[32];
#pragma unroll
    for (int d = 0; d < 26; ++d) {
        const int i = d >> 1, h = d & 1, t = 5 * i + 2 * h;          // first trit of the pair
        a[d] = (t & 1) ? align_bytes(xw[(t + 1) >> 1], xw[(t - 1) >> 1], 2) : xw[t >> 1];
    }
#pragma unroll
    for (int j = 0; j < 6; ++j) {
        const int k = j >> 1;
        const int ta = (j & 1) ? 20 * k + 9 : 20 * k + 4;               // trit 4 of byte 4k (+1)
        const int tb = (j & 1) ? 20 * k + 19 : 20 * k + 14;             // trit 4 of byte 4k+2 (+3)
        const uint32_t sa = (ta & 1) ? 0x0302u : 0x0100u;
        const uint32_t sb = (tb & 1) ? 0x0706u : 0x0504u;
        a[26 + j] = perm_b32(xw[tb >> 1], xw[ta >> 1], sa | (sb << 16));
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) A[j] = u32x4{a[4 * j], a[4 * j + 1], a[4 * j + 2], a[4 * j + 3]};
}

// 16-byte chunk j of a block: where it comes from and where it goes.
struct Chunk {
    bool scale;              // a scale chunk (else codes)
    int64_t base;            // array offset from the plane-1 codes (codes or scales of one plane)
    int64_t row_bytes;       // bytes per row in that array
    int row;                 // row within the block
    int col_bytes;           // byte offset within the row
    int dst;                 // LDS byte offset within a tile
    bool valid;
};

template <int PL>
__device__ __forceinline__ Chunk chunk_of(const RowsParams& p, int j) {
    const int rb = p.ng * kNB;            // code bytes per row
    const int cpr = rb >> 4;              // code chunks per row
    const int cc = 16 * cpr;              // code chunks per plane and block
    const int spr = p.ng >> 3;            // scale chunks per row
    const int sc = 16 * spr;              // scale chunks per plane and block
    // q = umulhi(j, 2^32 / d + 1) is exact for j, d < 2^16
    auto div = [](int j, uint32_t mul) { return (int)__umulhi((uint32_t)j, mul); };
    Chunk c;
    if (j < PL * cc) {
        const int pl = div(j, p.mul_cc), jj = j - pl * cc;
        const int r = div(jj, p.mul_cpr), k = jj - r * cpr;
        c.scale = false;
        c.base = pl == 0 ? 0 : p.off_codes2;
        c.row_bytes = rb;
        c.row = r;
        c.col_bytes = 16 * k;
        c.dst = pl * 16 * p.pitch + r * p.pitch + 16 * k;
        c.valid = true;
    } else if (j < PL * (cc + sc)) {
        const int jj = j - PL * cc;
        const int pl = div(jj, p.mul_sc), js = jj - pl * sc;
        const int r = div(js, p.mul_spr), k = js - r * spr;
        c.scale = true;
        c.base = pl == 0 ? p.off_scales1 : p.off_scales2;
        c.row_bytes = 2 * p.ng;
        c.row = r;
        c.col_bytes = 16 * k;
        c.dst = PL * 16 * p.pitch + pl * 16 * p.spitch + r * p.spitch + 16 * k;
        c.valid = true;
    } else {
        c.scale = false;
        c.base = 0;
        c.row_bytes = rb;
        c.row = 0;
        c.col_bytes = 0;
        c.dst = 0;
        c.valid = false;
    }
    return c;
}

// RU: a dense call of more than four tokens whose blocks all have tiles of
// their own (passes after the first read no codes).
template <int PL, int SPB, bool GR, bool RU>
__device__ __forceinline__ void tq_rows_body(const RowsParams& p, const int bid,
                                             unsigned char* lut, unsigned char* dyn) {
    unsigned char* tiles = dyn;                              // 2 tiles
    constexpr int NSB = SPB == 1 ? kNSB : kNSB - 1;          // blocks in flight
    float* red = (float*)(dyn + (p.all_tiles ? NSB : 2) * p.tile_bytes);   // [blocks][kW][64]

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = readfirstlane(tid >> 6);
    if constexpr (GR) {
        if (bid == p.n_items) {
            // slots whose expert id is out of range: NaN rows
            for (int i = 0; i < p.total; ++i) {
                const int ei = p.ids[i];
                if (ei >= 0 && ei < p.n_experts) continue;
                for (int64_t n = tid; n < p.N; n += kT) {
                    const int64_t o = (int64_t)i * p.N + n;
                    if (p.y_dtype == TQ_F32) ((float*)p.y)[o] = __builtin_nanf("");
                    else ((uint16_t*)p.y)[o] = 0x7fc0u;
                }
            }
            return;
        }
    }
    // Work item: the row range and (grouped) the expert.  Grouped launches of
    // at most 64 experts and 256 (token, slot) ids take their experts
    // heaviest first (most passes of four tokens, then lowest index), so that
    // an expert needing several passes starts in the first round instead of
    // lengthening the last.  Every wave holds the ids in registers; wave 0
    // counts the tokens of each expert in the partial buffer (idle until the
    // first tile barrier) and ranks them, one ballot per pass count.
    int el = GR ? bid / p.chunks : 0;                        // expert within the launch
    int vid[4] = {-1, -1, -1, -1};
    const bool ids_in_regs = GR && p.total <= 256;
    if constexpr (GR) {
        if (ids_in_regs) {
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int i = 64 * u + lane;
                vid[u] = i < p.total ? p.ids[i] : -1;
            }
            const int nl = p.n_items / p.chunks;
            if (nl > 1 && nl <= 64) {
                int* cnt = (int*)red;
                int* order = cnt + 64;
                if (wave == 0) {
                    // one wave counts, ranks and writes the order: its LDS
                    // operations complete in issue order, so no barrier between
                    cnt[lane] = 0;
                    __builtin_amdgcn_wave_barrier();      // keep the three steps in this order
#pragma unroll
                    for (int u = 0; u < 4; ++u) {
                        const int d = vid[u] - p.e_begin;
                        if (d >= 0 && d < nl) atomicAdd(&cnt[d], 1);
                    }
                    __builtin_amdgcn_wave_barrier();
                    const int key = lane < nl ? (cnt[lane] + 3) >> 2 : -1;
                    int kmax = key;
#pragma unroll
                    for (int o = 32; o > 0; o >>= 1) kmax = max(kmax, __shfl_xor(kmax, o));
                    kmax = readfirstlane(kmax);
                    int base = 0, rank = 0;
                    for (int k = kmax; k >= 0; --k) {
                        const uint64_t m = __builtin_amdgcn_ballot_w64(key == k);
                        if (key == k) rank = base + __builtin_popcountll(m & ((1ull << lane) - 1ull));
                        base += __builtin_popcountll(m);
                    }
                    if (lane < nl) order[rank] = lane;
                }
                __syncthreads();
                el = order[el];
            }
        }
    }
    const int e = GR ? p.e_begin + el : 0;
    const int64_t r0 = (int64_t)(GR ? bid % p.chunks : bid) * p.rows_per_wg;
    const int64_t r1 = min(r0 + (int64_t)p.rows_per_wg, p.N);
    const int64_t rlast = r1 - 1;
    const int nb = (int)((r1 - r0 + 15) >> 4);

    // tokens: dense, rows 0 .. M-1 of x; grouped, the (token, slot) pairs
    // routed to expert e, found by a wave-uniform scan of the ids
    // Each wave scans the ids itself (64 per vector load, a ballot of the
    // matches), so every wave holds the same uniform answer without a barrier.
    // The k-th match is found from the ballot masks with scalar bit scans.
    auto match_mask = [&](int i0) -> uint64_t {
        const int i = i0 + lane;
        const int v = i < p.total ? p.ids[i] : -1;
        return __builtin_amdgcn_ballot_w64(v == e);
    };
    // One scan counts the expert's tokens and records its first four (token,
    // slot) pairs, the first pass's rows; four chunks of ids are matched at a
    // time (from the registers when they hold every id).
    int ntok = p.M;
    int f0 = 0, f1 = 1, f2 = 2, f3 = 3;
    if constexpr (GR) {
        ntok = 0;
        for (int i0 = 0; i0 < p.total; i0 += 256) {
            int v[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int i = i0 + 64 * u + lane;
                v[u] = ids_in_regs ? vid[u] : (i < p.total ? p.ids[i] : -1);
            }
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                uint64_t m = __builtin_amdgcn_ballot_w64(v[u] == e);
                while (m != 0ull && ntok < 4) {
                    const int i = i0 + 64 * u + (int)__builtin_ctzll(m);
                    if (ntok == 0) f0 = i;
                    else if (ntok == 1) f1 = i;
                    else if (ntok == 2) f2 = i;
                    else f3 = i;
                    ++ntok;
                    m &= m - 1ull;
                }
                ntok += __builtin_popcountll(m);
            }
        }
        if (ntok == 0) return;                   // whole workgroup: nothing routed here
    }
    const int npass = (ntok + 3) >> 2;
    // the code-book entry of this thread, read ahead of every other load
    const uint2 tt = kTritPairs.e[tid >> 2];
    __builtin_amdgcn_sched_barrier(0);

    const int col = lane & 15;
    const int kb = lane >> 4;
    const int nquads = p.ng >> 2;
    const bool quad_ok = wave < nquads;
    const int g = 4 * wave + kb;
    const int ar = lane & 15;
    const uint32_t cofs = (uint32_t)(lane & 31) << 3;    // code-book copy lane % 32

    // this thread's chunks of every block: byte offset (from p.base) in block
    // 0, the offset of the same chunk in the last row of the range (rows past
    // it are clamped onto it), the per-block step and the LDS destination
    int64_t c_first[SPB], c_last[SPB];
    int c_dst[SPB];
    bool c_scale[SPB], c_valid[SPB];
#pragma unroll
    for (int s = 0; s < SPB; ++s) {
        const Chunk c = chunk_of<PL>(p, s * kT + tid);
        int64_t base = c.base;
        if constexpr (GR) base += c.scale ? (int64_t)e * p.e_scales : (int64_t)e * p.e_codes;
        c_first[s] = base + min(r0 + c.row, rlast) * c.row_bytes + c.col_bytes;
        c_last[s] = base + rlast * c.row_bytes + c.col_bytes;
        c_dst[s] = c.dst;
        c_scale[s] = c.scale;
        c_valid[s] = c.valid;
    }
    const int64_t step_codes = 16 * (int64_t)p.ng * kNB, step_scales = 32 * (int64_t)p.ng;
    auto load = [&](int blk, u32x4 (&R)[SPB]) {
        const int bc = min(blk, nb - 1);
#pragma unroll
        for (int s = 0; s < SPB; ++s) {
            const int64_t off = min(c_first[s] + bc * (c_scale[s] ? step_scales : step_codes), c_last[s]);
            R[s] = __builtin_nontemporal_load((const u32x4*)(p.base + off));
        }
    };

  for (int pass = 0; pass < npass; ++pass) {
    // the pass's tokens m < mt: activation row xr_m and output row or slot or_m
    const int mt = min(4, ntok - 4 * pass);
    int o0 = 4 * pass, o1 = 4 * pass + 1, o2 = 4 * pass + 2, o3 = 4 * pass + 3;
    if constexpr (GR) {
        if (pass == 0) { o0 = f0; o1 = f1; o2 = f2; o3 = f3; }
    }
    if (GR && pass > 0) {
        int k = 0;                         // matches before the current 64 ids
        for (int i0 = 0; i0 < p.total && k < 4 * pass + 4; i0 += 64) {
            uint64_t m = match_mask(i0);
            while (m != 0ull) {
                const int q = k - 4 * pass;
                const int i = i0 + (int)__builtin_ctzll(m);
                if (q == 0) o0 = i;
                else if (q == 1) o1 = i;
                else if (q == 2) o2 = i;
                else if (q == 3) o3 = i;
                ++k;
                m &= m - 1ull;
            }
        }
    }
    auto out_row = [&](int m) { return m == 0 ? o0 : (m == 1 ? o1 : (m == 2 ? o2 : o3)); };
    auto x_row = [&](int m) { return GR ? out_row(m) / p.top_k : out_row(m); };

    // ---- activations of this wave's quad, block diagonal, zero elsewhere
    // (loaded first so that masking them below waits for these loads only)
    const bool a_ok = (ar & 3) == kb && (ar >> 2) < mt && quad_ok;
    uint32_t xw[32];
    {
        const int mc = x_row(min(ar >> 2, mt - 1));
        const int gc = quad_ok ? g : 0;
        const uint16_t* xp = p.x + (int64_t)mc * p.K + (int64_t)gc * 64;
#pragma unroll
        for (int q = 0; q < 8; ++q) {
            const u32x4 v = *(const u32x4*)(xp + 8 * q);
            xw[4 * q] = v.x; xw[4 * q + 1] = v.y; xw[4 * q + 2] = v.z; xw[4 * q + 3] = v.w;
        }
    }
    __builtin_amdgcn_sched_barrier(0);     // activations are issued before the code stream

    // ---- the first NSB blocks (fewer in flight when a block takes two slots)
    // (dense passes after the first find every block still in its tile)
    const bool reuse = RU && pass > 0;
    u32x4 R[NSB][SPB];
    if (!reuse)
#pragma unroll
        for (int d = 0; d < NSB; ++d) load(d, R[d]);

    // ---- code book, 32 copies (first pass; read only after the first barrier)
    if (pass == 0) {
        // entry tid / 4, copies 8 (tid & 3) .. + 7; the four 16-byte stores are
        // rotated by tid / 4 so that the lanes of each store spread over the banks
        const u32x4 e = {tt.x, tt.y, tt.x, tt.y};
        unsigned char* d = lut + (((tid >> 2) << 8) | (64 * (tid & 3)));
#pragma unroll
        for (int c = 0; c < 4; ++c) *(u32x4*)(d + 16 * ((c + (tid >> 2)) & 3)) = e;
    }

    u32x4 A[8];
#pragma unroll
    for (int q = 0; q < 32; ++q) xw[q] = a_ok ? xw[q] : 0u;
    permute_group_x(xw, A);

    auto store = [&](int buf, const u32x4 (&R)[SPB]) {
        unsigned char* t = tiles + buf * p.tile_bytes;
#pragma unroll
        for (int s = 0; s < SPB; ++s) {
            if (c_valid[s]) {
                uint2* d = (uint2*)(t + c_dst[s]);
                d[0] = make_uint2(R[s].x, R[s].y);
                d[1] = make_uint2(R[s].z, R[s].w);
            }
        }
    };

    // decode + MFMA of block blk from tile buf; the partial goes to red
    auto compute = [&](int blk, int buf) {
        float part = 0.f;
        if (quad_ok) {
            const unsigned char* t = tiles + buf * p.tile_bytes;
#pragma unroll
            for (int pl = 0; pl < PL; ++pl) {
                // 13 code bytes of group g, row col: byte offset == kb (mod 4)
                const int off = pl * 16 * p.pitch + col * p.pitch + kNB * g;
                const uint32_t* wp = (const uint32_t*)(t + (off & ~3));
                const uint32_t W0 = wp[0], W1 = wp[1], W2 = wp[2], W3 = wp[3];
                const uint32_t sh = (uint32_t)kb;
                uint32_t D[4];
                D[0] = align_bytes(W1, W0, sh);
                D[1] = align_bytes(W2, W1, sh);
                D[2] = align_bytes(W3, W2, sh);
                D[3] = align_bytes(0u, W3, sh);
                // B operands in the group's K order (see permute_group_x)
                u32x4 Bq[8];
#pragma unroll
                for (int i = 0; i < kNB; ++i) {
                    const uint32_t a = perm_b32(D[i >> 2], cofs, 0x0c0c0400u + ((uint32_t)(i & 3) << 8));
                    const uint2 e2 = *(const uint2*)(lut + a);
                    Bq[i >> 1][2 * (i & 1)] = e2.x;
                    Bq[i >> 1][2 * (i & 1) + 1] = e2.y;
                }
#pragma unroll
                for (int k = 0; k < 3; ++k) {
                    const int d = 26 + 2 * k;
                    Bq[d >> 2][d & 3] = t4pair(D[k] & 0x00FF00FFu);
                    Bq[(d + 1) >> 2][(d + 1) & 3] = t4pair(perm_b32(D[k], D[k], 0x0c030c01u));
                }
                f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int j = 0; j < 8; ++j)
                    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                        __builtin_bit_cast(bf16x8, A[j]), __builtin_bit_cast(bf16x8, Bq[j]), acc, 0, 0, 0);
                // scales of groups 4w .. 4w+3 of row col (C rows 4m + i); the
                // factor 1/2 of the code book's 2t is applied after the sum
                const uint2 sw = *(const uint2*)(t + PL * 16 * p.pitch + pl * 16 * p.spitch +
                                                 col * p.spitch + 8 * wave);
                const _Float16 h0 = __builtin_bit_cast(_Float16, (uint16_t)(sw.x & 0xffffu));
                const _Float16 h1 = __builtin_bit_cast(_Float16, (uint16_t)(sw.x >> 16));
                const _Float16 h2 = __builtin_bit_cast(_Float16, (uint16_t)(sw.y & 0xffffu));
                const _Float16 h3 = __builtin_bit_cast(_Float16, (uint16_t)(sw.y >> 16));
                part = __builtin_fmaf((float)h0, acc[0], part);
                part = __builtin_fmaf((float)h1, acc[1], part);
                part = __builtin_fmaf((float)h2, acc[2], part);
                part = __builtin_fmaf((float)h3, acc[3], part);
            }
        }
        red[(blk * kW + wave) * 64 + lane] = part;
    };

    // blocks b0 .. b0+NSB-1 sit in R[0..NSB-1]; tile parity equals block parity
    auto body = [&](int blk, u32x4 (&Rb)[SPB]) {
        store(blk & 1, Rb);
        __syncthreads();
        load(blk + NSB, Rb);
        if (blk < nb) compute(blk, blk & 1);
    };
    if (p.all_tiles) {
        // the range fits in flight: every block to its own tile, one barrier,
        // then each wave decodes its quad of all blocks back to back
        if (!reuse)
#pragma unroll
            for (int d = 0; d < NSB; ++d)
                if (d < nb) store(d, R[d]);
        __syncthreads();
#pragma unroll
        for (int d = 0; d < NSB; ++d)
            if (d < nb) compute(d, d);
    } else {
        for (int b0 = 0; b0 < nb; b0 += NSB) {
#pragma unroll
            for (int d = 0; d < NSB; ++d) body(b0 + d, R[d]);
        }
    }
    __syncthreads();

    // ---- fixed-order sum of the wave partials, then y (grouped: row slot of y)
    for (int o = tid; o < nb * 64; o += kT) {
        const int blk = o >> 6, l = o & 63;
        const int m = l >> 4;
        const int64_t n = r0 + 16 * blk + (l & 15);
        float v = 0.f;
#pragma unroll
        for (int w = 0; w < kW; ++w) v += red[(blk * kW + w) * 64 + l];
        v *= 0.5f;                             // the code book holds 2t
        if (m < mt && n < r1) {
            const int64_t idx = (int64_t)out_row(m) * p.N + n;
            if (p.y_dtype == TQ_F32) ((float*)p.y)[idx] = v;
            else ((uint16_t*)p.y)[idx] = f32_to_bf16_rne(v);
        }
    }
    __syncthreads();                       // the next pass reuses the tiles and partials
  }
}

template <int PL, int SPB, bool GR, bool RU>
__global__ void __launch_bounds__(kT, 1) tq_rows_kernel(RowsParams p) {
    __shared__ __attribute__((aligned(16))) unsigned char lut[kLutBytes];
    extern __shared__ __attribute__((aligned(16))) unsigned char dyn[];
    tq_rows_body<PL, SPB, GR, RU>(p, (int)blockIdx.x, lut, dyn);
}

// A hot-prefix call in one launch: workgroups below ph.n_items take the hot
// experts' two-plane items (heaviest first within them), the rest the cold
// experts' one-plane items and, last, the rows of invalid ids.  The hardware
// hands the cold items to CUs as the hot ones finish, so neither part ends
// in a round of its own.
template <int SPBH, int SPBC>
__global__ void __launch_bounds__(kT, 1) tq_rows_hot_kernel(RowsParams ph, RowsParams pc) {
    __shared__ __attribute__((aligned(16))) unsigned char lut[kLutBytes];
    extern __shared__ __attribute__((aligned(16))) unsigned char dyn[];
    const int b = (int)blockIdx.x;
    if (b < ph.n_items) tq_rows_body<2, SPBH, true, false>(ph, b, lut, dyn);
    else tq_rows_body<1, SPBC, true, false>(pc, b - ph.n_items, lut, dyn);
}

constexpr int kMaxBlocks = 8;
constexpr int kLdsLimit = 160 * 1024;

}  // namespace

// Streaming ternary GEMV; returns false (launching nothing) when the call is
// outside its domain: G = 64, groups per row 16, 32, 48 or 64, 16-byte
// aligned operands, LDS within the limit; dense calls with 1 <= M <= 4 (up to
// 16 when the range's blocks all have tiles of their own, so passes after the
// first re-read no codes), or grouped expert calls (any number of tokens per
// expert, in passes of four). rows_setup fills the parameters, LDS bytes,
// slots per block and grid, and is false outside that domain.
static bool rows_setup(const TqMatmulArgs& a, RowsParams& p, size_t& smem_out, int& spb_out,
                       int64_t& wgs_out) {
    const bool grouped = a.n_experts > 0;
    if (a.G != 64 || a.M < 1 || a.N < 1) return false;
    const int64_t ng = a.K / 64;
    if (a.K % 64 != 0 || ng < 16 || ng % 16 != 0 || ng > 64) return false;
    auto al16 = [](const void* q) { return ((uintptr_t)q & 15) == 0; };
    if (!al16(a.x) || !al16(a.codes[0]) || !al16(a.scales[0])) return false;
    if (a.planes == 2 && (!al16(a.codes[1]) || !al16(a.scales[1]))) return false;
    p.x = a.x;
    p.K = a.K;
    p.N = a.N;
    p.ng = (int)ng;
    p.M = grouped ? 0 : (int)a.M;
    // byte distances between the operand arrays, so the kernel addresses all
    // four from one base without selecting pointers per lane
    auto dist = [&](const void* q) { return (int64_t)((intptr_t)q - (intptr_t)a.codes[0]); };
    p.base = a.codes[0];
    p.off_codes2 = a.planes == 2 ? dist(a.codes[1]) : 0;
    p.off_scales1 = dist(a.scales[0]);
    p.off_scales2 = a.planes == 2 ? dist(a.scales[1]) : dist(a.scales[0]);
    auto magic = [](int64_t d) { return (uint32_t)((1ull << 32) / (uint64_t)d + 1ull); };
    p.mul_cc = magic(ng * kNB);          // code chunks per plane and block = 16 * row bytes / 16
    p.mul_cpr = magic(ng * kNB / 16);
    p.mul_sc = magic(2 * ng);
    p.mul_spr = magic(ng / 8);
    p.pitch = (int)ng * kNB + 8;
    p.spitch = 2 * (int)ng + 8;
    p.tile_bytes = a.planes * 16 * (p.pitch + p.spitch);
    int64_t rpw;
    if (grouped) {
        rpw = std::min<int64_t>(16 * kMaxBlocks, (a.N + 7) & ~(int64_t)7);
    } else {
        const int cus = compute_unit_count();
        rpw = (a.N + cus - 1) / cus;
        rpw = (rpw + 7) & ~(int64_t)7;
        if (rpw > 16 * kMaxBlocks) rpw = 16 * kMaxBlocks;
    }
    p.rows_per_wg = (int)rpw;
    const int blocks = (int)((rpw + 15) / 16);
    const int chunks = a.planes * ((int)ng * kNB + 2 * (int)ng);
    const int spb = (chunks + kT - 1) / kT;
    if (spb > 2) return false;
    const int nsb = spb == 1 ? kNSB : kNSB - 1;
    const size_t red_bytes = (size_t)blocks * kW * 64 * sizeof(float);
    p.all_tiles = !grouped && blocks <= nsb &&
                  nsb * (size_t)p.tile_bytes + red_bytes + kLutBytes <= (size_t)kLdsLimit;
    const size_t smem = (p.all_tiles ? nsb : 2) * (size_t)p.tile_bytes + red_bytes;
    if (smem + kLutBytes > (size_t)kLdsLimit) return false;
    if (!grouped && (a.M > 16 || (a.M > 4 && !p.all_tiles))) return false;
    p.y = a.y;
    p.y_dtype = a.y_dtype;
    p.ids = a.ids;
    p.total = grouped ? (int)(a.M * a.top_k) : 0;
    p.top_k = a.top_k;
    p.chunks = (int)((a.N + rpw - 1) / rpw);
    p.n_experts = grouped ? a.n_experts : 0;
    p.e_begin = grouped ? a.e_begin : 0;
    p.e_codes = a.N * ng * kNB;
    p.e_scales = a.N * ng * 2;
    // grouped: the launch's experts, and one more workgroup for the slots
    // routed to no valid expert when this launch writes them
    const int64_t items = grouped ? (int64_t)(a.e_end - a.e_begin) * p.chunks : p.chunks;
    const int64_t wgs = items + ((grouped && a.nan_rows) ? 1 : 0);
    if (wgs >= (1ll << 31)) return false;
    p.n_items = (int)items;
    smem_out = smem;
    spb_out = spb;
    wgs_out = wgs;
    return true;
}

bool launch_tq_rows(const TqMatmulArgs& a, hipStream_t s, hipError_t* err) {
    RowsParams p;
    size_t smem;
    int spb;
    int64_t wgs;
    if (!rows_setup(a, p, smem, spb, wgs)) return false;
    if (wgs == 0) {
        *err = hipSuccess;
        return true;
    }
    const bool grouped = a.n_experts > 0;
    const dim3 grid((unsigned)wgs), block(kT);
#define DMM_ROWS(PL_, SPB_)                                                                \
    do {                                                                                   \
        if (grouped) hipLaunchKernelGGL((tq_rows_kernel<PL_, SPB_, true, false>), grid, block, smem, s, p); \
        else if (a.M > 4) hipLaunchKernelGGL((tq_rows_kernel<PL_, SPB_, false, true>), grid, block, smem, s, p); \
        else hipLaunchKernelGGL((tq_rows_kernel<PL_, SPB_, false, false>), grid, block, smem, s, p); \
    } while (0)
    if (a.planes == 1) {
        if (spb == 1) DMM_ROWS(1, 1);
        else DMM_ROWS(1, 2);
    } else {
        if (spb == 1) DMM_ROWS(2, 1);
        else DMM_ROWS(2, 2);
    }
#undef DMM_ROWS
    *err = hipGetLastError();
    return true;
}

bool launch_tq_rows_hot(const TqMatmulArgs& hot, const TqMatmulArgs& cold, hipStream_t s,
                        hipError_t* err) {
    if (hot.n_experts < 1 || cold.n_experts < 1) return false;
    if (hot.planes != 2 || cold.planes != 1 || hot.nan_rows || !cold.nan_rows) return false;
    RowsParams ph, pc;
    size_t smh, smc;
    int spbh, spbc;
    int64_t wgh, wgc;
    if (!rows_setup(hot, ph, smh, spbh, wgh) || !rows_setup(cold, pc, smc, spbc, wgc)) return false;
    if (spbc != 1 || wgh + wgc >= (1ll << 31)) return false;
    const size_t smem = smh > smc ? smh : smc;
    const dim3 grid((unsigned)(wgh + wgc)), block(kT);
    if (spbh == 1) hipLaunchKernelGGL((tq_rows_hot_kernel<1, 1>), grid, block, smem, s, ph, pc);
    else hipLaunchKernelGGL((tq_rows_hot_kernel<2, 1>), grid, block, smem, s, ph, pc);
    *err = hipGetLastError();
    return true;
}

}  // namespace dmm
