// Ternary GEMV for a few tokens over dense weights: y = x (s1 T1 + s2 T2)^T
// with G = 64, decoded inside the kernel.
//
// Format: "Does your weight format deserve a kernel?" (pack-unpack-run),
// "Five trits in a byte" and "Three values and a shared scale"; the second
// plane follows the FUCINA README ("The method").
//
// This is the streaming form for M <= 4 tokens, where the time is the HBM read
// of the package.  A row's codes (ng * 13 bytes) and scales (ng * 2 bytes)
// are contiguous and consecutive rows follow each other, so a range of rows
// is one contiguous byte range per array.
//
//  * One 1024-thread workgroup per compute unit owns rows_per_wg consecutive
//    rows and walks them in blocks of 16 (one MFMA column block).  A block's
//    bytes (codes and scales, every plane) are fetched as 16-byte chunks by
//    the whole workgroup, so each load instruction reads 1 KiB of one
//    contiguous range.  Four blocks are in flight in registers; a block is
//    written to one of two LDS tiles, then decoded while the next blocks
//    arrive.
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
//    forms the address and the 16 lanes of a phase hit distinct banks.
//  * Tile rows are padded to 8 mod 16 bytes so the 16 rows of a block start
//    in distinct bank pairs.
//  * Wave partials are kept per block in LDS and summed in a fixed order at
//    the end, so results do not depend on timing.
#include "common.h"

namespace dmm {

namespace {

constexpr int kW = 16;                  // waves per workgroup
constexpr int kT = 64 * kW;             // threads per workgroup
constexpr int kNB = 13;                 // code bytes per group of 64 trits
constexpr int kNSB = 4;                 // blocks in flight
constexpr int kLutBytes = 256 * 256;    // entry b, copy c at (b << 8) | (c << 3)

struct RowsParams {
    const uint16_t* x;
    int64_t K, N;
    int ng;                  // groups per row, a multiple of 16
    int M;                   // tokens, 1..4
    const uint8_t* base;     // plane-1 codes; the other arrays sit at byte offsets from it
    int64_t off_codes2, off_scales1, off_scales2;
    uint32_t mul_cc, mul_cpr, mul_sc, mul_spr;   // 2^32 / d + 1 for the chunk divisions
    int rows_per_wg;         // multiple of 8, <= 16 * kMaxBlocks
    int pitch;               // LDS bytes per tile code row (row bytes + 8)
    int spitch;              // LDS bytes per tile scale row (2 ng + 8)
    int tile_bytes;          // one LDS tile: planes * 16 * (pitch + spitch)
    void* y;
    int y_dtype;
};

__device__ __forceinline__ uint32_t trit_hi(int d) {     // bf16 high byte of 2t, d = t + 1
    return d == 2 ? 0x40u : (d == 0 ? 0xC0u : 0x00u);
}

// 16-byte chunk j of a block: where it comes from and where it goes.
struct Chunk {
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
        c.base = pl == 0 ? p.off_scales1 : p.off_scales2;
        c.row_bytes = 2 * p.ng;
        c.row = r;
        c.col_bytes = 16 * k;
        c.dst = PL * 16 * p.pitch + pl * 16 * p.spitch + r * p.spitch + 16 * k;
        c.valid = true;
    } else {
        c.base = 0;
        c.row_bytes = rb;
        c.row = 0;
        c.col_bytes = 0;
        c.dst = 0;
        c.valid = false;
    }
    return c;
}

template <int PL, int SPB>
__global__ void __launch_bounds__(kT, 1) tq_rows_kernel(RowsParams p) {
    __shared__ __attribute__((aligned(16))) unsigned char lut[kLutBytes];
    extern __shared__ __attribute__((aligned(16))) unsigned char dyn[];
    unsigned char* tiles = dyn;                              // 2 tiles
    float* red = (float*)(dyn + 2 * p.tile_bytes);           // [blocks][kW][64]

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = readfirstlane(tid >> 6);
    const int64_t r0 = (int64_t)blockIdx.x * p.rows_per_wg;
    const int64_t r1 = min(r0 + (int64_t)p.rows_per_wg, p.N);
    const int64_t rlast = r1 - 1;
    const int nb = (int)((r1 - r0 + 15) >> 4);

    // ---- activations of this wave's quad, block diagonal, zero elsewhere
    const int col = lane & 15;
    const int kb = lane >> 4;
    const int nquads = p.ng >> 2;
    const bool quad_ok = wave < nquads;
    const int g = 4 * wave + kb;
    // (loaded first so that masking them below waits for these loads only)
    const int ar = lane & 15;
    const bool a_ok = (ar & 3) == kb && (ar >> 2) < p.M && quad_ok;
    u32x4 A[8];
    {
        const int mc = min(ar >> 2, p.M - 1);
        const int gc = quad_ok ? g : 0;
        const uint16_t* xp = p.x + (int64_t)mc * p.K + (int64_t)gc * 64;
#pragma unroll
        for (int q = 0; q < 8; ++q) A[q] = *(const u32x4*)(xp + 8 * q);
    }
    __builtin_amdgcn_sched_barrier(0);     // activations are issued before the code stream

    // ---- this thread's chunks of every block, and the first kNSB blocks
    Chunk ch[SPB];
#pragma unroll
    for (int s = 0; s < SPB; ++s) ch[s] = chunk_of<PL>(p, s * kT + tid);
    auto load = [&](int blk, u32x4 (&R)[SPB]) {
        const int bc = min(blk, nb - 1);
#pragma unroll
        for (int s = 0; s < SPB; ++s) {
            const int64_t row = min(r0 + 16 * bc + ch[s].row, rlast);
            R[s] = __builtin_nontemporal_load(
                (const u32x4*)(p.base + ch[s].base + row * ch[s].row_bytes + ch[s].col_bytes));
        }
    };
    u32x4 R0[SPB], R1[SPB], R2[SPB], R3[SPB];
    load(0, R0);
    load(1, R1);
    load(2, R2);
    load(3, R3);

    // ---- trit table, 16 copies
    for (int i = tid; i < 256 * 16; i += kT) {
        const int b = i >> 4, c = i & 15;
        uint32_t lo = 0, hi = 0;
        if (b < 243) {
            int v = b;
            uint32_t h[5];
#pragma unroll
            for (int q = 0; q < 5; ++q) { h[q] = trit_hi(v % 3); v /= 3; }
            lo = h[0] | (h[1] << 8) | (h[2] << 16) | (h[3] << 24);
            hi = h[4];
        }
        *(uint2*)(lut + ((b << 8) | (c << 3))) = make_uint2(lo, hi);
    }

#pragma unroll
    for (int q = 0; q < 8; ++q) A[q] = a_ok ? A[q] : u32x4{0u, 0u, 0u, 0u};
    const uint32_t cofs = (uint32_t)col << 3;

    auto store = [&](int buf, const u32x4 (&R)[SPB]) {
        unsigned char* t = tiles + buf * p.tile_bytes;
#pragma unroll
        for (int s = 0; s < SPB; ++s) {
            if (ch[s].valid) {
                uint2* d = (uint2*)(t + ch[s].dst);
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
                uint32_t Elo[kNB], Ehi[kNB];
#pragma unroll
                for (int i = 0; i < kNB; ++i) {
                    const uint32_t a = perm_b32(D[i >> 2], cofs, 0x0c0c0400u + ((uint32_t)(i & 3) << 8));
                    const uint2 e = *(const uint2*)(lut + a);
                    Elo[i] = e.x;
                    Ehi[i] = e.y;
                }
                uint32_t B[32];
#pragma unroll
                for (int p2 = 0; p2 < 32; ++p2) {
                    const int ja = 2 * p2, jb = 2 * p2 + 1;
                    const int ia = ja / 5, qa = ja % 5, ib = jb / 5, qb = jb % 5;
                    const uint32_t ra = qa < 4 ? Elo[ia] : Ehi[ia];
                    const uint32_t rbv = qb < 4 ? Elo[ib] : Ehi[ib];
                    const uint32_t ba = qa < 4 ? qa : 0, bb = qb < 4 ? qb : 0;
                    const bool same = (ia == ib) && ((qa < 4) == (qb < 4));
                    B[p2] = same ? perm_b32(ra, ra, 0x0cu | (ba << 8) | (0x0cu << 16) | (bb << 24))
                                 : perm_b32(rbv, ra, 0x0cu | (ba << 8) | (0x0cu << 16) | ((4u + bb) << 24));
                }
                f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int q = 0; q < 8; ++q) {
                    const u32x4 bq = {B[4 * q], B[4 * q + 1], B[4 * q + 2], B[4 * q + 3]};
                    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                        __builtin_bit_cast(bf16x8, A[q]), __builtin_bit_cast(bf16x8, bq), acc, 0, 0, 0);
                }
                // scales of groups 4w .. 4w+3 of row col (C rows 4m + i)
                const uint2 sw = *(const uint2*)(t + PL * 16 * p.pitch + pl * 16 * p.spitch +
                                                 col * p.spitch + 8 * wave);
                const float s0 = f16_bits_to_f32((uint16_t)(sw.x & 0xffffu));
                const float s1 = f16_bits_to_f32((uint16_t)(sw.x >> 16));
                const float s2 = f16_bits_to_f32((uint16_t)(sw.y & 0xffffu));
                const float s3 = f16_bits_to_f32((uint16_t)(sw.y >> 16));
                // the table holds 2t: halve once
                part += 0.5f * (s0 * acc[0] + s1 * acc[1] + s2 * acc[2] + s3 * acc[3]);
            }
        }
        red[(blk * kW + wave) * 64 + lane] = part;
    };

    // blocks b0 .. b0+3 sit in R0..R3; tile parity equals block parity
    auto body = [&](int blk, u32x4 (&R)[SPB]) {
        store(blk & 1, R);
        __syncthreads();
        load(blk + kNSB, R);
        if (blk < nb) compute(blk, blk & 1);
    };
    for (int b0 = 0; b0 < nb; b0 += kNSB) {
        body(b0, R0);
        body(b0 + 1, R1);
        body(b0 + 2, R2);
        body(b0 + 3, R3);
    }
    __syncthreads();

    // ---- fixed-order sum of the wave partials, then y
    for (int o = tid; o < nb * 64; o += kT) {
        const int blk = o >> 6, l = o & 63;
        const int m = l >> 4;
        const int64_t n = r0 + 16 * blk + (l & 15);
        float v = 0.f;
#pragma unroll
        for (int w = 0; w < kW; ++w) v += red[(blk * kW + w) * 64 + l];
        if (m < p.M && n < r1) {
            const int64_t idx = (int64_t)m * p.N + n;
            if (p.y_dtype == TQ_F32) ((float*)p.y)[idx] = v;
            else ((uint16_t*)p.y)[idx] = f32_to_bf16_rne(v);
        }
    }
}

constexpr int kMaxBlocks = 8;
constexpr int kLdsLimit = 160 * 1024;

int compute_units() {
    static int cus = 0;
    if (cus == 0) {
        int dev = 0, v = 0;
        if (hipGetDevice(&dev) == hipSuccess &&
            hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess &&
            v > 0)
            cus = v;
        else
            cus = 256;
    }
    return cus;
}

}  // namespace

// Streaming ternary GEMV; returns false (launching nothing) when the call is
// outside its domain: dense, G = 64, 1 <= M <= 4, groups per row 16, 32, 48
// or 64, 16-byte aligned operands, LDS within the limit.
bool launch_tq_rows(const TqMatmulArgs& a, hipStream_t s, hipError_t* err) {
    if (a.n_experts != 0 || a.G != 64 || a.M < 1 || a.M > 4 || a.N < 1) return false;
    const int64_t ng = a.K / 64;
    if (a.K % 64 != 0 || ng < 16 || ng % 16 != 0 || ng > 64) return false;
    auto al16 = [](const void* q) { return ((uintptr_t)q & 15) == 0; };
    if (!al16(a.x) || !al16(a.codes[0]) || !al16(a.scales[0])) return false;
    if (a.planes == 2 && (!al16(a.codes[1]) || !al16(a.scales[1]))) return false;
    RowsParams p;
    p.x = a.x;
    p.K = a.K;
    p.N = a.N;
    p.ng = (int)ng;
    p.M = (int)a.M;
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
    const int cus = compute_units();
    int64_t rpw = (a.N + cus - 1) / cus;
    rpw = (rpw + 7) & ~(int64_t)7;
    if (rpw > 16 * kMaxBlocks) rpw = 16 * kMaxBlocks;
    p.rows_per_wg = (int)rpw;
    const int blocks = (int)((rpw + 15) / 16);
    const size_t smem = 2 * (size_t)p.tile_bytes + (size_t)blocks * kW * 64 * sizeof(float);
    if (smem + kLutBytes > (size_t)kLdsLimit) return false;
    const int chunks = a.planes * ((int)ng * kNB + 2 * (int)ng);
    const int spb = (chunks + kT - 1) / kT;
    if (spb > 2) return false;
    p.y = a.y;
    p.y_dtype = a.y_dtype;
    const dim3 grid((unsigned)((a.N + rpw - 1) / rpw)), block(kT);
    if (a.planes == 1) {
        if (spb == 1) hipLaunchKernelGGL((tq_rows_kernel<1, 1>), grid, block, smem, s, p);
        else hipLaunchKernelGGL((tq_rows_kernel<1, 2>), grid, block, smem, s, p);
    } else {
        if (spb == 1) hipLaunchKernelGGL((tq_rows_kernel<2, 1>), grid, block, smem, s, p);
        else hipLaunchKernelGGL((tq_rows_kernel<2, 2>), grid, block, smem, s, p);
    }
    *err = hipGetLastError();
    return true;
}

}  // namespace dmm
