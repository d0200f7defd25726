// Ternary GEMV for up to four tokens over dense weights, wave by wave:
// y = x (s1 T1 + s2 T2)^T with G = 64, decoded inside the kernel.
//
// Format: pack-unpack-run, "Five trits in a byte" (five base-3 digits per
// byte, least significant first) and "Three values and a shared scale"
// (W_hat = s t per group of 64); the second plane follows the FUCINA README
// ("The method").
//
// Each wave owns tasks of 4 rows x 16 groups and loads its own bytes, so a
// wave decodes a task as soon as that task's bytes have arrived, without
// waiting for the rest of the workgroup:
//  * a task's load instruction reads 208 contiguous code bytes of each of 4
//    rows (lane 4 b + j: row j, group b of the 16), which streams almost as
//    fast as a flat read, and the next task's load is issued before the
//    current task is decoded;
//  * the multiply is the 4x4x4 bf16 MFMA with 16 blocks: block b is group b,
//    its B operand is 4 trits of each of the 4 rows and its A operand 4
//    activations of each of the 4 tokens, so no operand is wasted at M = 4;
//  * a code byte's trits 0..3 come from one LDS lookup into a code book of
//    ready bf16 pairs (the B operand of one MFMA, 32 copies, entry b copy c
//    at (b << 8) | (c << 3), the address one v_perm of the code byte); trit 4
//    of four bytes is computed with packed 16-bit arithmetic and feeds a
//    fourteenth to sixteenth MFMA;
//  * the activations are staged in LDS once per workgroup with coalesced
//    loads issued ahead of the code stream, and each lane takes its 64 in the
//    K order of the MFMA operands;
//  * a group's sum is scaled by its fp16 scale in fp32; the 16 group slices
//    of a row are summed across lanes and waves in a fixed order.
#include "common.h"

namespace dmm {

namespace {

constexpr int kW = 16;
constexpr int kT = 64 * kW;
constexpr int kNB = 13;                  // code bytes per group of 64 trits
constexpr int kMaxTasks = 4;             // tasks per wave
constexpr int kXsPitch = 144;            // LDS bytes per staged group of 64 activations
constexpr int kXsTok = 64 * kXsPitch;    // per token (at most 64 groups)
constexpr int kTaskStride = 68;          // floats per task: [4 lane rows][4 rows][4 tokens] + pad

typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef unsigned short u16x2v __attribute__((ext_vector_type(2)));

struct WaveParams {
    const uint16_t* x;
    int64_t K, N;
    int ng, M;
    const uint8_t* codes[2];
    const uint16_t* scales[2];
    int rows_per_wg;
    void* y;
    int y_dtype;
};

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

// K order of a group (one lane's A and B operands over the 16 MFMAs of a
// group): MFMA i < 13 takes trits 5i .. 5i+3 of code byte i; MFMA 13 + k takes
// trit 4 of bytes 4k, 4k+2 (first dword) and 4k+1, 4k+3 (second dword).  Byte
// 12's trit 4 is padding.  a_dword gives the activation pair of MFMA t, dword h.
__device__ __forceinline__ uint32_t a_dword(const uint32_t (&xw)[32], int t, int h) {
    if (t < 13) {
        const int s = 5 * t + 2 * h;                       // first trit of the pair
        return (s & 1) ? align_bytes(xw[(s + 1) >> 1], xw[(s - 1) >> 1], 2) : xw[s >> 1];
    }
    const int k = t - 13;
    const int ta = h ? 20 * k + 9 : 20 * k + 4;
    const int tb = h ? 20 * k + 19 : 20 * k + 14;
    const uint32_t sa = (ta & 1) ? 0x0302u : 0x0100u;
    const uint32_t sb = (tb & 1) ? 0x0706u : 0x0504u;
    return perm_b32(xw[tb >> 1], xw[ta >> 1], sa | (sb << 16));
}

template <int PL>
__global__ void __launch_bounds__(kT, 1) tq_wave_kernel(WaveParams p) {
    __shared__ __attribute__((aligned(16))) unsigned char lut[256 * 256];
    __shared__ __attribute__((aligned(16))) unsigned char xs[4 * kXsTok];
    extern __shared__ __attribute__((aligned(16))) float red[];   // [row quad][slice][kTaskStride]

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = readfirstlane(tid >> 6);
    const int64_t r0 = (int64_t)blockIdx.x * p.rows_per_wg;
    const int nrows = (int)(min(r0 + (int64_t)p.rows_per_wg, p.N) - r0);
    const int nrq = (nrows + 3) >> 2;                 // row quads of the workgroup
    const int nkq = p.ng >> 4;                        // 16-group slices of K
    const int kq = wave % nkq, rr = wave / nkq, nrr = kW / nkq;
    const int b = lane >> 2, j = lane & 3;
    const int g = 16 * kq + b;
    const uint32_t sh = (uint32_t)(b & 3);            // 13 g == g (mod 4)
    const int64_t rb = (int64_t)p.ng * kNB;

    // ---- activations: 16-byte pieces of the M x K rows, issued first
    uint32_t xr[2][4];
    const int per_tok = (int)(p.K >> 3);
    const int xchunks = p.M * per_tok;
#pragma unroll
    for (int u = 0; u < 2; ++u) {
        const int c = tid + u * kT;
        if (c < xchunks) {
            const u32x4 v = *(const u32x4*)(p.x + 8 * (int64_t)c);
            xr[u][0] = v.x; xr[u][1] = v.y; xr[u][2] = v.z; xr[u][3] = v.w;
        }
    }
    // ---- task t is row quad rr + t nrr: lane (b, j) reads row j's group b
    // (16 aligned bytes at 13 g - sh; the last group of a row ends exactly at
    // the row's end) and its scale.  Task 0 goes out right behind the
    // activations: memory counters retire in order, so waiting for x does
    // not wait for it.
    u32x4 C[PL][kMaxTasks];
    uint16_t S[PL][kMaxTasks];
    auto issue = [&](int t) {
        const int rq = min(rr + t * nrr, nrq - 1);
        const int64_t row = r0 + min(4 * rq + j, nrows - 1);
        const int64_t co = row * rb + kNB * g - (int64_t)sh;
#pragma unroll
        for (int pl = 0; pl < PL; ++pl) {
            C[pl][t] = __builtin_nontemporal_load((const u32x4a*)(p.codes[pl] + co));
            S[pl][t] = p.scales[pl][row * p.ng + g];
        }
    };
    issue(0);
    __builtin_amdgcn_sched_barrier(0);

    // ---- stage x: token m's group q at m kXsTok + q kXsPitch
#pragma unroll
    for (int u = 0; u < 2; ++u) {
        const int c = tid + u * kT;
        if (c < xchunks) {
            const int m = c / per_tok, cc = c - m * per_tok;
            *(u32x4*)(xs + m * kXsTok + (cc >> 3) * kXsPitch + 16 * (cc & 7)) =
                u32x4{xr[u][0], xr[u][1], xr[u][2], xr[u][3]};
        }
    }
    // ---- code book: entry e (a byte) holds its trits 0..3 as bf16 pairs of
    // 2t; 32 copies, entry e copy c at (e << 8) | (c << 3).  Thread tid fills
    // copies 8 (tid & 3) .. + 7 of entry tid / 4 with four 16-byte stores,
    // rotated by tid / 4 so that the lanes of a store spread over the banks.
    {
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
    __syncthreads();

    // ---- A operands: token j's group g in the K order above (zero for j >= M)
    u32x2 A[16];
    {
        uint32_t xw[32];
        const bool ok = j < p.M;
        const unsigned char* xp = xs + (ok ? j : 0) * kXsTok + g * kXsPitch;
#pragma unroll
        for (int q = 0; q < 8; ++q) {
            const u32x4 v = *(const u32x4*)(xp + 16 * q);
            xw[4 * q] = ok ? v.x : 0u;
            xw[4 * q + 1] = ok ? v.y : 0u;
            xw[4 * q + 2] = ok ? v.z : 0u;
            xw[4 * q + 3] = ok ? v.w : 0u;
        }
#pragma unroll
        for (int t = 0; t < 16; ++t) A[t] = u32x2{a_dword(xw, t, 0), a_dword(xw, t, 1)};
    }

    const uint32_t cofs = (uint32_t)(lane & 31) << 3;    // code-book copy lane % 32
#pragma unroll
    for (int t = 0; t < kMaxTasks; ++t) {
        if (t + 1 < kMaxTasks) issue(t + 1);
        const int rq = rr + t * nrr;
        if (rq < nrq) {
            // D[t][r] for block b: token r, row j of the task, summed over
            // both planes with their group scales
            f32x4 tot = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int pl = 0; pl < PL; ++pl) {
                uint32_t D[4];
                D[0] = align_bytes(C[pl][t].y, C[pl][t].x, sh);
                D[1] = align_bytes(C[pl][t].z, C[pl][t].y, sh);
                D[2] = align_bytes(C[pl][t].w, C[pl][t].z, sh);
                D[3] = align_bytes(0u, C[pl][t].w, sh);
                f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int i = 0; i < kNB; ++i) {
                    const uint32_t a = perm_b32(D[i >> 2], cofs, 0x0c0c0400u + ((uint32_t)(i & 3) << 8));
                    const uint2 e = *(const uint2*)(lut + a);
                    acc = __builtin_amdgcn_mfma_f32_4x4x4bf16_1k(__builtin_bit_cast(bf16x4, A[i]),
                                                                 __builtin_bit_cast(bf16x4, u32x2{e.x, e.y}),
                                                                 acc, 0, 0, 0);
                }
#pragma unroll
                for (int k = 0; k < 3; ++k) {
                    const u32x2 q = {t4pair(D[k] & 0x00FF00FFu), t4pair(perm_b32(D[k], D[k], 0x0c030c01u))};
                    acc = __builtin_amdgcn_mfma_f32_4x4x4bf16_1k(__builtin_bit_cast(bf16x4, A[13 + k]),
                                                                 __builtin_bit_cast(bf16x4, q), acc, 0, 0, 0);
                }
                const float s = (float)__builtin_bit_cast(_Float16, S[pl][t]);
#pragma unroll
                for (int r = 0; r < 4; ++r) tot[r] = __builtin_fmaf(s, acc[r], tot[r]);
            }
            // sum over the four blocks of each 16-lane row (lanes 4 b' + j)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                float v = tot[r];
                v += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0x124, 0xF, 0xF, false));
                v += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0x128, 0xF, 0xF, false));
                tot[r] = v;
            }
            if ((lane & 12) == 0)
                *(f32x4*)(red + (rq * nkq + kq) * kTaskStride + (lane >> 4) * 16 + 4 * j) = tot;
        }
    }
    __syncthreads();

    // ---- y[m, n] = 1/2 (the code book holds 2t) of the sum over the slices
    // and the four lane rows, in a fixed order
    for (int o = tid; o < nrows * p.M; o += kT) {
        const int m = o / nrows, rloc = o - m * nrows;
        const int rq = rloc >> 2, c = rloc & 3;
        float v = 0.f;
        for (int q = 0; q < nkq; ++q)
#pragma unroll
            for (int r = 0; r < 4; ++r) v += red[(rq * nkq + q) * kTaskStride + r * 16 + 4 * c + m];
        v *= 0.5f;
        const int64_t idx = (int64_t)m * p.N + r0 + rloc;
        if (p.y_dtype == TQ_F32) ((float*)p.y)[idx] = v;
        else ((uint16_t*)p.y)[idx] = f32_to_bf16_rne(v);
    }
}

int wave_compute_units() {
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

// Dense calls with 1 <= M <= 4, G = 64, K a multiple of 1024 up to 4096, x
// 16-byte and codes 4-byte aligned; false (nothing launched) otherwise.
bool launch_tq_wave(const TqMatmulArgs& a, hipStream_t s, hipError_t* err) {
    if (a.n_experts != 0 || a.G != 64 || a.M < 1 || a.M > 4 || a.N < 1) return false;
    if (a.K < 1024 || a.K > 4096 || a.K % 1024 != 0) return false;
    if (((uintptr_t)a.x & 15) != 0) return false;
    for (int pl = 0; pl < a.planes; ++pl)
        if (((uintptr_t)a.codes[pl] & 3) != 0 || ((uintptr_t)a.scales[pl] & 1) != 0) return false;
    const int ng = (int)(a.K / 64);
    const int nkq = ng / 16, nrr = kW / nkq;
    int64_t rpw = (a.N + wave_compute_units() - 1) / wave_compute_units();
    rpw = (rpw + 3) & ~(int64_t)3;
    if (rpw > 4 * kMaxTasks * nrr) rpw = 4 * kMaxTasks * nrr;
    const int64_t wgs = (a.N + rpw - 1) / rpw;
    if (wgs >= (1ll << 31)) return false;
    WaveParams p;
    p.x = a.x;
    p.K = a.K;
    p.N = a.N;
    p.ng = ng;
    p.M = (int)a.M;
    p.codes[0] = a.codes[0];
    p.codes[1] = a.planes == 2 ? a.codes[1] : a.codes[0];
    p.scales[0] = a.scales[0];
    p.scales[1] = a.planes == 2 ? a.scales[1] : a.scales[0];
    p.rows_per_wg = (int)rpw;
    p.y = a.y;
    p.y_dtype = a.y_dtype;
    const size_t smem = (size_t)((rpw + 3) / 4) * nkq * kTaskStride * sizeof(float);
    if (a.planes == 2)
        hipLaunchKernelGGL(tq_wave_kernel<2>, dim3((unsigned)wgs), dim3(kT), smem, s, p);
    else
        hipLaunchKernelGGL(tq_wave_kernel<1>, dim3((unsigned)wgs), dim3(kT), smem, s, p);
    *err = hipGetLastError();
    return true;
}

}  // namespace dmm
