// Mean-abs ternary pack and unpack kernels.
//
// Format: "Does your weight format deserve a kernel?" (pack-unpack-run),
// sections "Three values and a shared scale" (s = fp16(mean |W|),
// t = clip(round(W/s), -1, 1), ties to even, zero scale -> all-zero group),
// "Five trits in a byte" (b = d0 + 3 d1 + 9 d2 + 27 d3 + 81 d4, d = t + 1,
// first digit least significant; bytes 243..255 rejected; padding decodes to
// zero) and "Count the bytes you actually wrote" (each group starts on a
// byte boundary: ceil(G/5) code bytes + one fp16 scale).  Two planes: FUCINA
// README, "The method" (W ~ d1 T1 + d2 T2; plane 2 packs the residual of
// plane 1).
//
// One thread owns one (row, group).  Packing is not on the timed path; the
// kernel is written for bit-exactness: a sequential float64 sum, one
// float64 division, one float64 -> fp16 rounding, and the exact threshold
// |W| > s/2 in place of round(W/s).
#include "common.h"

namespace dmm {

namespace {

constexpr int kPackThreads = 256;

__global__ void status_clear_kernel(int32_t* st) {
    if (threadIdx.x == 0 && blockIdx.x == 0) *st = 0;
}

// Trit of w against scale s (s >= 0 finite): sign(w) * [|w| > s/2].
__device__ __forceinline__ int trit_of(float w, float s_half, bool s_pos) {
    if (!s_pos) return 0;
    float a = fabsf(w);
    if (!(a > s_half)) return 0;
    return w > 0.f ? 1 : -1;
}

// Quantize one group of values produced by `val(j)`, write its bytes and
// scale, return the fp32 scale used (0 on error).  Returns false through
// `ok` when the group has a non-finite value or the scale overflows.
template <typename ValFn>
__device__ float quantize_group(ValFn val, int n, int nb, uint8_t* out_codes,
                                uint16_t* out_scale, bool& ok) {
    double S = 0.0;
    bool finite = true;
    for (int j = 0; j < n; ++j) {
        float v = val(j);
        finite = finite && (fabsf(v) <= 3.402823466e38f);
        S += (double)fabsf(v);
    }
    uint16_t sb = 0;
    if (finite) sb = f64_to_f16_rne(S / (double)n);
    ok = finite && ((sb & 0x7fffu) < 0x7c00u);
    if (!ok) sb = 0;
    float s = f16_bits_to_f32(sb);
    float s_half = 0.5f * s;                 // exact
    bool s_pos = s > 0.f;
    for (int i = 0; i < nb; ++i) {
        int b = 0;
        int p3 = 1;
        for (int q = 0; q < 5; ++q) {
            int j = 5 * i + q;
            int d = 1;                       // padding digit (trit 0)
            if (j < n && ok) d = trit_of(val(j), s_half, s_pos) + 1;
            b += d * p3;
            p3 *= 3;
        }
        out_codes[i] = (uint8_t)b;
    }
    *out_scale = sb;
    return s;
}

__global__ void __launch_bounds__(kPackThreads)
pack_kernel(const float* __restrict__ W, int64_t rows, int64_t K, int G, int ng, int nb,
            int planes, uint8_t* __restrict__ c1, uint16_t* __restrict__ s1,
            uint8_t* __restrict__ c2, uint16_t* __restrict__ s2, int32_t* st) {
    int64_t gid = (int64_t)blockIdx.x * kPackThreads + threadIdx.x;
    if (gid >= rows * (int64_t)ng) return;
    int64_t r = gid / ng;
    int g = (int)(gid - r * ng);
    int64_t k0 = (int64_t)g * G;
    int n = (int)((K - k0) < (int64_t)G ? (K - k0) : (int64_t)G);
    const float* w = W + r * K + k0;

    bool ok1 = true;
    float sc1 = quantize_group([&](int j) { return w[j]; }, n, nb, c1 + gid * nb, s1 + gid, ok1);
    if (!ok1) atomic_or_status(st, TQ_DATA_RANGE);
    if (planes == 2) {
        float sh1 = 0.5f * sc1;
        bool sp1 = sc1 > 0.f && ok1;
        // residual R = fl32(W - s1 t1): s1 t1 is exact, one fp32 rounding
        auto res = [&](int j) {
            float v = w[j];
            int t = trit_of(v, sh1, sp1);
            float st1 = t > 0 ? sc1 : (t < 0 ? -sc1 : 0.f);
            return v - st1;
        };
        bool ok2 = true;
        quantize_group(res, n, nb, c2 + gid * nb, s2 + gid, ok2);
        if (!ok2) atomic_or_status(st, TQ_DATA_RANGE);
    }
}

__global__ void __launch_bounds__(kPackThreads)
unpack_kernel(const uint8_t* __restrict__ codes, const uint16_t* __restrict__ scales,
              int64_t rows, int64_t K, int G, int ng, int nb, void* __restrict__ out,
              int out_dtype, int32_t* st) {
    int64_t gid = (int64_t)blockIdx.x * kPackThreads + threadIdx.x;
    if (gid >= rows * (int64_t)ng) return;
    int64_t r = gid / ng;
    int g = (int)(gid - r * ng);
    int64_t k0 = (int64_t)g * G;
    int n = (int)((K - k0) < (int64_t)G ? (K - k0) : (int64_t)G);
    const uint8_t* cb = codes + gid * nb;
    float s = f16_bits_to_f32(scales[gid]);
    int flags = 0;
    for (int i = 0; i < nb; ++i) {
        int b = cb[i];
        if (b > 242) { flags |= TQ_DATA_CODE; b = 121; }
        for (int q = 0; q < 5; ++q) {
            int d = b % 3;
            b /= 3;
            int j = 5 * i + q;
            if (j >= n) {
                if (d != 1) flags |= TQ_DATA_PADDING;
                continue;
            }
            float v = d == 2 ? s : (d == 0 ? -s : 0.f);     // exact s * t
            int64_t idx = r * K + k0 + j;
            if (out_dtype == 0) ((float*)out)[idx] = v;
            else ((uint16_t*)out)[idx] = f32_to_bf16_rne(v);
        }
    }
    if (flags) atomic_or_status(st, flags);
}

}  // namespace

hipError_t launch_status_clear(int32_t* d_status, hipStream_t s) {
    hipLaunchKernelGGL(status_clear_kernel, dim3(1), dim3(64), 0, s, d_status);
    return hipGetLastError();
}

hipError_t launch_pack(const float* W, int64_t rows, int64_t K, int G, int planes,
                       uint8_t* c1, uint16_t* s1, uint8_t* c2, uint16_t* s2,
                       int32_t* d_status, hipStream_t s) {
    int ng = (int)((K + G - 1) / G);
    int nb = (G + 4) / 5;
    int64_t groups = rows * (int64_t)ng;
    if (groups == 0) return hipSuccess;
    int64_t blocks = (groups + kPackThreads - 1) / kPackThreads;
    hipLaunchKernelGGL(pack_kernel, dim3((unsigned)blocks), dim3(kPackThreads), 0, s, W, rows,
                       K, G, ng, nb, planes, c1, s1, c2, s2, d_status);
    return hipGetLastError();
}

hipError_t launch_unpack(const uint8_t* codes, const uint16_t* scales, int64_t rows,
                         int64_t K, int G, void* out, int out_dtype, int32_t* d_status,
                         hipStream_t s) {
    int ng = (int)((K + G - 1) / G);
    int nb = (G + 4) / 5;
    int64_t groups = rows * (int64_t)ng;
    if (groups == 0) return hipSuccess;
    int64_t blocks = (groups + kPackThreads - 1) / kPackThreads;
    hipLaunchKernelGGL(unpack_kernel, dim3((unsigned)blocks), dim3(kPackThreads), 0, s, codes,
                       scales, rows, K, G, ng, nb, out, out_dtype, d_status);
    return hipGetLastError();
}

}  // namespace dmm
