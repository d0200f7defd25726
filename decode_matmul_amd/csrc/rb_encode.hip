// Route B encoder: fp32 W -> code bytes, the global scale alpha and the
// optional fp16 per-row scales.
//
// Semantics: "A Discrete Weight Language for Large Language Models" (Route
// B), section 3.1 (the greedy 5-step word: each step takes the c in
// {-1, 0, +1} nearest to the residual and subtracts c s_i; r_0 = x / alpha
// with alpha = max |W|; a zero-bias zeta forces c_i = 0 while
// |r_{i-1}| < zeta s_i), section 3.2 (the code is the base-3 encoding of
// c_1..c_5) and section 3.3 (per-row scale: r_0 = W[n, k] / alpha_n with
// alpha_n = max_k |W[n, k]|, rho_n = alpha_n / alpha in fp16).
//
// Every decision is taken on IEEE float64 values: r_0 is one float64
// division, each residual one float64 subtraction (c s_i is exact), the
// distances |r - s_i|, |r|, |r + s_i| and zeta s_i are float64, ties go to
// c = 0, and rho_n is one float64 division rounded once to fp16 (on the bit
// pattern).  So the codes do not depend on the order of operations or on the
// hardware.  A zero scale gives r_0 = 0 (the all-zero word, code 121) and
// rho_n = 0.
//
// Two launches after the clear: a grid-stride max |W| (atomic max on the
// bits of the non-negative float, which order like integers; non-finite
// weights raise TQ_DATA_RANGE), then one workgroup per row that finds the
// row maximum when per-row scales are asked for and encodes the row.  Not on
// the timed path of a matmul; it reads W twice (three times with per-row
// scales) and writes one byte per weight.
#include "common.h"

namespace dmm {

namespace {

constexpr int kEncThreads = 256;

struct EncParams {
    const float* W;
    int64_t N, K;
    double s[5];             // the ladder as float64 (each >= 0)
    double zs[5];            // zeta * s_i, float64 products
    int per_row;
    uint8_t* codes;
    float* alpha;            // device fp32: max |W| (written by the first pass)
    uint16_t* row_scale;     // device fp16 [N] when per_row
    int32_t* status;
};

__global__ void enc_clear_kernel(float* alpha, int32_t* status) {
    if (threadIdx.x == 0 && blockIdx.x == 0) {
        *alpha = 0.f;
        *status = 0;
    }
}

// Largest |W| over the matrix.
__global__ void __launch_bounds__(kEncThreads) enc_absmax_kernel(const float* W, int64_t n,
                                                                 float* alpha, int32_t* status) {
    float m = 0.f;
    bool finite = true;
    const int64_t stride = (int64_t)gridDim.x * kEncThreads;
    for (int64_t i = (int64_t)blockIdx.x * kEncThreads + threadIdx.x; i < n; i += stride) {
        const float a = fabsf(W[i]);
        finite = finite && (a <= 3.402823466e38f);
        m = fmaxf(m, a);
    }
    for (int o = 32; o > 0; o >>= 1) m = fmaxf(m, __shfl_xor(m, o));
    const bool bad = __builtin_amdgcn_ballot_w64(!finite) != 0;
    if ((threadIdx.x & 63) == 0) {
        atomicMax((unsigned int*)alpha, __builtin_bit_cast(unsigned int, m));
        if (bad) atomicOr(status, (int32_t)TQ_DATA_RANGE);
    }
}

// The code of r_0 (section 3.1 steps, c_1 most significant).  With s >= 0
// the candidate on the far side of zero is never nearer: for r >= 0,
// fl(r + s) >= r (rounding is monotone), so only +1 can beat 0, and it does
// when |r - s| < r; for r < 0 only -1, when |r + s| < -r.  This is the
// three-way argmin with ties to 0, decided on the same float64 values.
__device__ __forceinline__ uint32_t encode_word(double r, const EncParams& p) {
    uint32_t code = 0;
#pragma unroll
    for (int i = 0; i < 5; ++i) {
        const double s = p.s[i];
        const double a = fabs(r);
        const double t = r >= 0.0 ? r - s : r + s;        // the nearer nonzero candidate
        int c = fabs(t) < a ? (r >= 0.0 ? 1 : -1) : 0;
        c = a < p.zs[i] ? 0 : c;                          // zero-bias
        r = c != 0 ? t : r;
        code = code * 3u + (uint32_t)(c + 1);
    }
    return code;
}

__device__ __forceinline__ float block_max(float m, float* red) {
    for (int o = 32; o > 0; o >>= 1) m = fmaxf(m, __shfl_xor(m, o));
    const int wave = threadIdx.x >> 6;
    if ((threadIdx.x & 63) == 0) red[wave] = m;
    __syncthreads();
    float r = red[0];
#pragma unroll
    for (int w = 1; w < kEncThreads / 64; ++w) r = fmaxf(r, red[w]);
    return r;
}

__global__ void __launch_bounds__(kEncThreads) enc_rows_kernel(EncParams p) {
    __shared__ float red[kEncThreads / 64];
    const int64_t n = blockIdx.x;
    const float* row = p.W + n * p.K;
    float scale = *p.alpha;
    if (p.per_row) {
        float m = 0.f;
        for (int64_t k = threadIdx.x; k < p.K; k += kEncThreads) m = fmaxf(m, fabsf(row[k]));
        const float an = block_max(m, red);
        if (threadIdx.x == 0) {
            const double q = scale > 0.f ? (double)an / (double)scale : 0.0;
            p.row_scale[n] = f64_to_f16_rne(q);
        }
        scale = an;
    }
    const double ds = (double)scale;
    const bool pos = scale > 0.f;
    uint8_t* out = p.codes + n * p.K;
    for (int64_t k = threadIdx.x; k < p.K; k += kEncThreads) {
        const double r0 = pos ? (double)row[k] / ds : 0.0;
        out[k] = (uint8_t)encode_word(r0, p);
    }
}

}  // namespace

hipError_t launch_rb_encode(const float* W, int64_t N, int64_t K, const float* ladder, float zeta,
                            int per_row, uint8_t* codes, float* alpha, uint16_t* row_scale,
                            int32_t* status, hipStream_t s) {
    hipLaunchKernelGGL(enc_clear_kernel, dim3(1), dim3(64), 0, s, alpha, status);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int64_t total = N * K;
    if (total > 0) {
        const int64_t want = (total + kEncThreads * 16 - 1) / (kEncThreads * 16);
        const unsigned blocks = (unsigned)(want < 4096 ? want : 4096);
        hipLaunchKernelGGL(enc_absmax_kernel, dim3(blocks), dim3(kEncThreads), 0, s, W, total, alpha,
                           status);
        e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    if (N == 0) return hipSuccess;
    EncParams p;
    p.W = W;
    p.N = N;
    p.K = K;
    for (int i = 0; i < 5; ++i) {
        p.s[i] = (double)ladder[i];
        p.zs[i] = (double)zeta * p.s[i];
    }
    p.per_row = per_row;
    p.codes = codes;
    p.alpha = alpha;
    p.row_scale = row_scale;
    p.status = status;
    hipLaunchKernelGGL(enc_rows_kernel, dim3((unsigned)N), dim3(kEncThreads), 0, s, p);
    return hipGetLastError();
}

}  // namespace dmm
