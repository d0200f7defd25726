// Route B GEMV (M <= 16): y[m, n] = alpha * rho_n * sum_k x[m, k] T[codes[n, k]] + bias_n.
//
// Semantics: "A Discrete Weight Language for Large Language Models" (Route
// B), section 3.2 (codes index a 243-entry code book), section 3.3 (per-row
// scale rho_n) and section 4.2 (the code book sits in on-chip memory, every
// code byte is dereferenced through it inside a K-sliced GEMM, rho_n is
// applied to the accumulator before the bias).
//
// Mapping onto gfx950:
//  * The workgroup owns 16 output rows; its 8 waves split K into contiguous
//    ranges and meet in LDS at the end (fixed summation order).
//  * Each code byte is looked up in an LDS copy of the code book.  Every
//    fp32 entry v is stored as two bf16 terms, hi = bf16(v) and
//    lo = bf16(v - hi) (|v - hi - lo| <= 2^-17 |v|), packed as one dword.
//    The table is replicated 64 times with entry b of copy c at byte
//    256 b + 4 c, so lane c always hits its own bank and the address is a
//    single v_perm of the code dword with the lane offset.
//  * bf16 MFMA 16x16x32: B takes the looked-up (hi, lo) dword as two K-slots
//    of one weight, A holds the activation twice in the same two slots, so
//    one MFMA accumulates x*hi + x*lo = x*v for four weights per lane.
//    A rows are the M <= 16 tokens; C columns are the 16 rows.
//  * Each lane streams 16 consecutive code bytes of one row per step
//    (16 B loads; 4 lanes cover 64 contiguous bytes of a row).
#include "common.h"

namespace dmm {

namespace {

constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;
constexpr int kLutBytes = 256 * 256;       // 256 entries x 64 copies x 4 B

struct Params {
    const uint16_t* x;
    int64_t M, K, N;
    const uint8_t* codes;
    const float* table;
    float alpha;
    const uint16_t* row_scale;
    const float* bias;
    void* y;
    int y_dtype;
    int64_t steps;                           // ceil(K / 64)
    int64_t full_steps;                      // steps entirely inside K
};

__device__ __forceinline__ uint32_t split_entry(float v) {
    uint16_t hi = f32_to_bf16_rne(v);
    float r = v - bf16_bits_to_f32(hi);      // exact
    uint16_t lo = f32_to_bf16_rne(r);
    return (uint32_t)hi | ((uint32_t)lo << 16);
}

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
    __shared__ float red[kWaves * 64 * 4];

    const int tid = threadIdx.x;
    const int wave = tid >> 6;
    const int lane = tid & 63;

    for (int i = tid; i < 256 * 64; i += kThreads) {
        const int b = i >> 6;
        const float v = b < 243 ? p.table[b] : 0.f;
        *(uint32_t*)(lut + 4 * i) = split_entry(v);
    }

    const int64_t rb = blockIdx.x;
    const int col = lane & 15;
    const int kb = lane >> 4;
    const int64_t n = rb * 16 + col;
    const bool row_ok = n < p.N;
    const uint8_t* crow = p.codes + (row_ok ? n : 0) * p.K;
    const int am = lane & 15;                                     // A row = token
    const bool a_ok = am < p.M;
    const uint16_t* xrow = p.x + (a_ok ? am : 0) * p.K;
    const uint32_t lane_off = (uint32_t)lane << 2;

    // contiguous K range of this wave, in 64-column steps
    const int64_t per = (p.steps + kWaves - 1) / kWaves;
    const int64_t s_begin = min(p.steps, per * wave);
    const int64_t s_end = min(p.steps, s_begin + per);

    __syncthreads();

    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    auto compute = [&](const uint32_t* D, const uint32_t* X) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            u32x4 bq, aq;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const uint32_t addr = perm_b32(D[j], lane_off, 0x0c0c0400u + ((uint32_t)i << 8));
                bq[i] = *(const uint32_t*)(lut + addr);
            }
            const uint32_t x01 = X[2 * j], x23 = X[2 * j + 1];
            aq[0] = perm_b32(x01, x01, 0x01000100u);
            aq[1] = perm_b32(x01, x01, 0x03020302u);
            aq[2] = perm_b32(x23, x23, 0x01000100u);
            aq[3] = perm_b32(x23, x23, 0x03020302u);
            acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, aq),
                                                          __builtin_bit_cast(bf16x8, bq), acc,
                                                          0, 0, 0);
        }
    };
    auto load_full = [&](int64_t st, uint32_t* R, uint32_t& sh, uint32_t* X) {
        const int64_t k = st * 64 + 16 * kb;
        if (row_ok) load_codes_raw<ALIGNED>(crow, k, R, sh);
        else { R[0] = R[1] = R[2] = R[3] = R[4] = 0xffffffffu; sh = 0; }
        if (a_ok) load_x16(xrow, k, p.K, false, X);
        else {
#pragma unroll
            for (int i = 0; i < 8; ++i) X[i] = 0u;
        }
    };

    // steps entirely inside K, with the next step's loads in flight
    const int64_t s_full_end = max(s_begin, min(s_end, p.full_steps));
    int64_t st = s_begin;
    if (st < s_full_end) {
        uint32_t Rn[5], Xn[8], shn;
        load_full(st, Rn, shn, Xn);
        for (; st < s_full_end; ++st) {
            uint32_t R[5], X[8], sh = shn;
#pragma unroll
            for (int i = 0; i < 5; ++i) R[i] = Rn[i];
#pragma unroll
            for (int i = 0; i < 8; ++i) X[i] = Xn[i];
            if (st + 1 < s_full_end) load_full(st + 1, Rn, shn, Xn);
            uint32_t D[4];
            realign16<ALIGNED>(R, sh, D);
            compute(D, X);
        }
    }
    // the ragged tail of K (and every step when rows are not 4-byte aligned)
    for (; st < s_end; ++st) {
        const int64_t k = st * 64 + 16 * kb;
        uint32_t D[4], X[8];
        if (row_ok) load_codes16_tail(crow, k, p.K, D);
        else D[0] = D[1] = D[2] = D[3] = 0xffffffffu;
        if (a_ok) load_x16(xrow, k, p.K, true, X);
        else {
#pragma unroll
            for (int i = 0; i < 8; ++i) X[i] = 0u;
        }
        compute(D, X);
    }

    // C[4*(lane>>4) + i][lane & 15]: token 4*(lane>>4)+i, row col
#pragma unroll
    for (int i = 0; i < 4; ++i) red[(wave * 64 + lane) * 4 + i] = acc[i];
    __syncthreads();
    if (wave == 0 && row_ok) {
        const float rho = p.row_scale ? f16_bits_to_f32(p.row_scale[n]) : 1.f;
        const float bias = p.bias ? p.bias[n] : 0.f;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int m = 4 * kb + i;
            if (m >= p.M) continue;
            float v = red[lane * 4 + i];
#pragma unroll
            for (int w = 1; w < kWaves; ++w) v += red[(w * 64 + lane) * 4 + i];
            v = v * rho;
            v = v * p.alpha;
            v = v + bias;
            const int64_t idx = (int64_t)m * p.N + n;
            if (p.y_dtype == TQ_F32) ((float*)p.y)[idx] = v;
            else ((uint16_t*)p.y)[idx] = f32_to_bf16_rne(v);
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
    p.alpha = a.alpha;
    p.row_scale = a.row_scale;
    p.bias = a.bias;
    p.y = a.y;
    p.y_dtype = a.y_dtype;
    p.steps = (a.K + 63) / 64;
    // a step is "full" when every lane's 16 bytes lie inside K
    p.full_steps = a.K / 64;
    // vector activation loads need 4-byte aligned rows; otherwise every step
    // takes the element-wise path
    if ((a.K & 1) || ((uintptr_t)a.x & 3)) p.full_steps = 0;
    const int64_t blocks = (a.N + 15) / 16;
    if (blocks == 0 || a.M == 0) return hipSuccess;
    const bool aligned4 = (((uintptr_t)a.codes & 3) == 0) && (a.K % 4 == 0);
    if (aligned4)
        hipLaunchKernelGGL(rb_gemv_kernel<true>, dim3((unsigned)blocks), dim3(kThreads), 0, s, p);
    else
        hipLaunchKernelGGL(rb_gemv_kernel<false>, dim3((unsigned)blocks), dim3(kThreads), 0, s, p);
    return hipGetLastError();
}

}  // namespace dmm
