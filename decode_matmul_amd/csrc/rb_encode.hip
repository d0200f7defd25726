// Route B encoder: fp32 W -> code bytes, the global scale alpha and the
// optional fp16 row or head scales.
//
// Semantics: "A Discrete Weight Language for Large Language Models" (Route
// B), section 3.1 (the greedy 5-step word: each step takes the c in
// {-1, 0, +1} nearest to the residual and subtracts c s_i; r_0 = x / alpha
// with alpha = max |W|; a zero-bias zeta forces c_i = 0 while
// |r_{i-1}| < zeta s_i), section 3.2 (the code is the base-3 encoding of
// c_1..c_5) and section 3.3 (per-row scale: r_0 = W[n, k] / alpha_n with
// alpha_n = max_k |W[n, k]|, rho_n = alpha_n / alpha in fp16).  Per-head
// prosody (section 8.2: one rho per attention head, the rows of a head
// sharing the scale) is the same rule over blocks of rho_rows consecutive
// rows: alpha_h is the block's largest |W| and rho_h = fp16(alpha_h / alpha);
// rho_rows = 1 is section 3.3, rho_rows = 0 the global scale alone.
//
// Every decision is taken on IEEE float64 values: r_0 is one float64
// division, each residual one float64 subtraction (c s_i is exact), the
// distances |r - s_i|, |r|, |r + s_i| and zeta s_i are float64, ties go to
// c = 0, and rho_h is one float64 division rounded once to fp16 (on the bit
// pattern).  So the codes do not depend on the order of operations or on the
// hardware.  A zero scale gives r_0 = 0 (the all-zero word, code 121) and
// rho_h = 0.
//
// Three launches: a clear of alpha and the block scales; one workgroup per
// row taking the row's max |W| into alpha and into its block's scale (atomic
// max on the bits of the non-negative float, which order like integers;
// non-finite weights raise TQ_DATA_RANGE); one workgroup per row that
// encodes it (the block's first row also writes rho_h).  W is read twice.
// With one scale per row (rho_rows = 1, K <= 16384) a row needs only its own
// maximum: one workgroup stages the row in LDS, takes its maximum and encodes
// it (W read once), and a last small launch writes rho_n once the global
// maximum is complete.  The arithmetic is the same, so are the codes.
#include "common.h"

namespace dmm {

namespace {

constexpr int kEncThreads = 256;

struct EncParams {
    const float* W;
    int64_t N, K;
    double s[5];             // the ladder as float64 (each >= 0)
    double zs[5];            // zeta * s_i, float64 products
    int64_t rho_rows;        // 0: global scale; b: one scale per b rows
    uint8_t* codes;
    float* alpha;            // device fp32 [1 + blocks]: max |W|, then alpha_h
    uint16_t* row_scale;     // device fp16 [blocks] when rho_rows > 0
    int32_t* status;
};

__global__ void enc_clear_kernel(float* alpha, int64_t n, int32_t* status) {
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride)
        alpha[i] = 0.f;
    if (threadIdx.x == 0 && blockIdx.x == 0) *status = 0;
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

// Largest |W| of row blockIdx.x into alpha[0] and (blocks) alpha[1 + n / b].
__global__ void __launch_bounds__(kEncThreads) enc_rowmax_kernel(EncParams p) {
    __shared__ float red[kEncThreads / 64];
    const int64_t n = blockIdx.x;
    const float* row = p.W + n * p.K;
    float m = 0.f;
    bool finite = true;
    for (int64_t k = threadIdx.x; k < p.K; k += kEncThreads) {
        const float a = fabsf(row[k]);
        finite = finite && (a <= 3.402823466e38f);
        m = fmaxf(m, a);
    }
    const bool bad = __syncthreads_or(!finite) != 0;
    const float rm = block_max(m, red);
    if (threadIdx.x == 0) {
        atomicMax((unsigned int*)p.alpha, __builtin_bit_cast(unsigned int, rm));
        if (p.rho_rows > 0)
            atomicMax((unsigned int*)(p.alpha + 1 + n / p.rho_rows),
                      __builtin_bit_cast(unsigned int, rm));
        if (bad) atomicOr(p.status, (int32_t)TQ_DATA_RANGE);
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

__global__ void __launch_bounds__(kEncThreads) enc_rows_kernel(EncParams p) {
    const int64_t n = blockIdx.x;
    const float* row = p.W + n * p.K;
    const float alpha = p.alpha[0];
    float scale = alpha;
    if (p.rho_rows > 0) {
        const int64_t h = n / p.rho_rows;
        scale = p.alpha[1 + h];
        if (threadIdx.x == 0 && n == h * p.rho_rows) {
            const double q = alpha > 0.f ? (double)scale / (double)alpha : 0.0;
            p.row_scale[h] = f64_to_f16_rne(q);
        }
    }
    const double ds = (double)scale;
    const bool pos = scale > 0.f;
    uint8_t* out = p.codes + n * p.K;
    for (int64_t k = threadIdx.x; k < p.K; k += kEncThreads) {
        const double r0 = pos ? (double)row[k] / ds : 0.0;
        out[k] = (uint8_t)encode_word(r0, p);
    }
}

constexpr int64_t kFusedMaxK = 16384;          // floats of a row staged in LDS

// rho_rows = 1: row blockIdx.x staged in LDS, its maximum, then its codes.
__global__ void __launch_bounds__(kEncThreads) enc_fused_row_kernel(EncParams p) {
    extern __shared__ float wrow[];
    __shared__ float red[kEncThreads / 64];
    const int64_t n = blockIdx.x;
    const float* row = p.W + n * p.K;
    float m = 0.f;
    bool finite = true;
    for (int64_t k = threadIdx.x; k < p.K; k += kEncThreads) {
        const float v = row[k];
        wrow[k] = v;
        const float a = fabsf(v);
        finite = finite && (a <= 3.402823466e38f);
        m = fmaxf(m, a);
    }
    const bool bad = __syncthreads_or(!finite) != 0;
    const float rm = block_max(m, red);                 // its barrier also publishes wrow
    if (threadIdx.x == 0) {
        atomicMax((unsigned int*)p.alpha, __builtin_bit_cast(unsigned int, rm));
        p.alpha[1 + n] = rm;                            // the row is its own block
        if (bad) atomicOr(p.status, (int32_t)TQ_DATA_RANGE);
    }
    const double ds = (double)rm;
    const bool pos = rm > 0.f;
    uint8_t* out = p.codes + n * p.K;
    for (int64_t k = threadIdx.x; k < p.K; k += kEncThreads) {
        const double r0 = pos ? (double)wrow[k] / ds : 0.0;
        out[k] = (uint8_t)encode_word(r0, p);
    }
}

// rho_n = fp16(alpha_n / alpha) after every row's maximum is in.
__global__ void enc_rho_kernel(EncParams p) {
    const float alpha = p.alpha[0];
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t h = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; h < p.N; h += stride) {
        const double q = alpha > 0.f ? (double)p.alpha[1 + h] / (double)alpha : 0.0;
        p.row_scale[h] = f64_to_f16_rne(q);
    }
}

}  // namespace

hipError_t launch_rb_encode(const float* W, int64_t N, int64_t K, const float* ladder, float zeta,
                            int64_t rho_rows, uint8_t* codes, float* alpha, uint16_t* row_scale,
                            int32_t* status, hipStream_t s) {
    const int64_t blocks = rho_rows > 0 ? (N + rho_rows - 1) / rho_rows : 0;
    const int64_t nclear = 1 + blocks;
    const int64_t cg = (nclear + 255) / 256;
    hipLaunchKernelGGL(enc_clear_kernel, dim3((unsigned)(cg < 1024 ? cg : 1024)), dim3(256), 0, s,
                       alpha, nclear, status);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || N == 0) return e;
    EncParams p;
    p.W = W;
    p.N = N;
    p.K = K;
    for (int i = 0; i < 5; ++i) {
        p.s[i] = (double)ladder[i];
        p.zs[i] = (double)zeta * p.s[i];
    }
    p.rho_rows = rho_rows;
    p.codes = codes;
    p.alpha = alpha;
    p.row_scale = row_scale;
    p.status = status;
    if (rho_rows == 1 && K <= kFusedMaxK) {
        hipLaunchKernelGGL(enc_fused_row_kernel, dim3((unsigned)N), dim3(kEncThreads),
                           (size_t)K * sizeof(float), s, p);
        e = hipGetLastError();
        if (e != hipSuccess) return e;
        const int64_t rg = (N + 255) / 256;
        hipLaunchKernelGGL(enc_rho_kernel, dim3((unsigned)(rg < 1024 ? rg : 1024)), dim3(256), 0, s, p);
        return hipGetLastError();
    }
    hipLaunchKernelGGL(enc_rowmax_kernel, dim3((unsigned)N), dim3(kEncThreads), 0, s, p);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(enc_rows_kernel, dim3((unsigned)N), dim3(kEncThreads), 0, s, p);
    return hipGetLastError();
}

}  // namespace dmm
