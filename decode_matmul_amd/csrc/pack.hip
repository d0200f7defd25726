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
// One thread owns one (row, group); it is written for bit-exactness: a
// sequential float64 sum, one float64 division, one float64 -> fp16
// rounding, and the exact threshold |W| > s/2 in place of round(W/s).
// A workgroup owns consecutive groups, whose weights are one contiguous
// span of W (rows are contiguous): the span is moved between HBM and LDS
// with coalesced accesses, and each thread works on its group in LDS (one
// pad word per 64 floats, so the lanes' sequential walks hit distinct
// banks).  The code bytes are staged in LDS as well and stored coalesced.
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

constexpr int kStageFloats = 16384;                  // floats of W staged per workgroup
constexpr int kStageBytes = 256 * 13;                 // code bytes per plane and workgroup

// Groups per workgroup at group size G (64 or 128): 256 or 128.
inline int groups_per_wg(int G) { return kStageFloats / G < kPackThreads ? kStageFloats / G : kPackThreads; }

__device__ __forceinline__ int stage_idx(int64_t i) { return (int)(i + (i >> 6)); }

// First element (in W's row-major order) of group gid, and its size.
__device__ __forceinline__ int64_t group_start(int64_t gid, int64_t K, int G, int ng, int* n) {
    const int64_t r = gid / ng;
    const int64_t k0 = (gid - r * ng) * (int64_t)G;
    *n = (int)((K - k0) < (int64_t)G ? (K - k0) : (int64_t)G);
    return r * K + k0;
}

__global__ void __launch_bounds__(kPackThreads)
pack_kernel(const float* __restrict__ W, int64_t rows, int64_t K, int G, int ng, int nb,
            int gpw, int planes, uint8_t* __restrict__ c1, uint16_t* __restrict__ s1,
            uint8_t* __restrict__ c2, uint16_t* __restrict__ s2, int32_t* st) {
    __shared__ float wl[kStageFloats + kStageFloats / 64];
    __shared__ uint8_t cl[2][kStageBytes];
    const int tid = threadIdx.x;
    const int64_t total = rows * (int64_t)ng;
    const int64_t g0 = (int64_t)blockIdx.x * gpw;
    const int64_t g1 = g0 + gpw < total ? g0 + gpw : total;
    int n_last;
    const int64_t start = group_start(g0, K, G, ng, &n_last);
    const int64_t len = group_start(g1 - 1, K, G, ng, &n_last) + n_last - start;   // <= gpw * G
    if (((start | len) & 3) == 0 && ((uintptr_t)W & 15) == 0) {
        // 16-byte loads; four consecutive floats never straddle a pad word
        const float4* w4 = (const float4*)(W + start);
        const int len4 = (int)(len >> 2);
#pragma unroll 4
        for (int i = tid; i < len4; i += kPackThreads) {
            const float4 v = w4[i];
            float* d = wl + stage_idx(4 * (int64_t)i);
            d[0] = v.x; d[1] = v.y; d[2] = v.z; d[3] = v.w;
        }
    } else {
#pragma unroll 4
        for (int64_t i = tid; i < len; i += kPackThreads) wl[stage_idx(i)] = W[start + i];
    }
    __syncthreads();

    const int64_t gid = g0 + tid;
    if (tid < gpw && gid < g1) {
        int n;
        const int64_t o = group_start(gid, K, G, ng, &n) - start;
        auto w = [&](int j) { return wl[stage_idx(o + j)]; };
        bool ok1 = true;
        const float sc1 = quantize_group(w, n, nb, cl[0] + tid * nb, s1 + gid, ok1);
        if (!ok1) atomic_or_status(st, TQ_DATA_RANGE);
        if (planes == 2) {
            const float sh1 = 0.5f * sc1;
            const bool sp1 = sc1 > 0.f && ok1;
            // residual R = fl32(W - s1 t1): s1 t1 is exact, one fp32 rounding
            auto res = [&](int j) {
                const float v = w(j);
                const int t = trit_of(v, sh1, sp1);
                const float st1 = t > 0 ? sc1 : (t < 0 ? -sc1 : 0.f);
                return v - st1;
            };
            bool ok2 = true;
            quantize_group(res, n, nb, cl[1] + tid * nb, s2 + gid, ok2);
            if (!ok2) atomic_or_status(st, TQ_DATA_RANGE);
        }
    }
    __syncthreads();
    const int64_t nbytes = (g1 - g0) * nb;
    for (int64_t i = tid; i < nbytes; i += kPackThreads) c1[g0 * nb + i] = cl[0][i];
    if (planes == 2)
        for (int64_t i = tid; i < nbytes; i += kPackThreads) c2[g0 * nb + i] = cl[1][i];
}

__global__ void __launch_bounds__(kPackThreads)
unpack_kernel(const uint8_t* __restrict__ codes, const uint16_t* __restrict__ scales,
              int64_t rows, int64_t K, int G, int ng, int nb, int gpw, void* __restrict__ out,
              int out_dtype, int32_t* st) {
    __shared__ float wl[kStageFloats + kStageFloats / 64];
    const int tid = threadIdx.x;
    const int64_t total = rows * (int64_t)ng;
    const int64_t g0 = (int64_t)blockIdx.x * gpw;
    const int64_t g1 = g0 + gpw < total ? g0 + gpw : total;
    int n_last;
    const int64_t start = group_start(g0, K, G, ng, &n_last);
    const int64_t len = group_start(g1 - 1, K, G, ng, &n_last) + n_last - start;

    const int64_t gid = g0 + tid;
    if (tid < gpw && gid < g1) {
        int n;
        const int64_t o = group_start(gid, K, G, ng, &n) - start;
        const uint8_t* cb = codes + gid * nb;
        const float s = f16_bits_to_f32(scales[gid]);
        int flags = 0;
        for (int i = 0; i < nb; ++i) {
            int b = cb[i];
            if (b > 242) { flags |= TQ_DATA_CODE; b = 121; }
            for (int q = 0; q < 5; ++q) {
                const int d = b % 3;
                b /= 3;
                const int j = 5 * i + q;
                if (j >= n) {
                    if (d != 1) flags |= TQ_DATA_PADDING;
                    continue;
                }
                wl[stage_idx(o + j)] = d == 2 ? s : (d == 0 ? -s : 0.f);     // exact s * t
            }
        }
        if (flags) atomic_or_status(st, flags);
    }
    __syncthreads();
    if (((start | len) & 3) == 0 && ((uintptr_t)out & (out_dtype == 0 ? 15 : 7)) == 0) {
        // four values per store
        const int len4 = (int)(len >> 2);
#pragma unroll 4
        for (int i = tid; i < len4; i += kPackThreads) {
            const float* v = wl + stage_idx(4 * (int64_t)i);
            if (out_dtype == 0) {
                ((float4*)((float*)out + start))[i] = make_float4(v[0], v[1], v[2], v[3]);
            } else {
                const uint32_t lo = (uint32_t)f32_to_bf16_rne(v[0]) | ((uint32_t)f32_to_bf16_rne(v[1]) << 16);
                const uint32_t hi = (uint32_t)f32_to_bf16_rne(v[2]) | ((uint32_t)f32_to_bf16_rne(v[3]) << 16);
                ((uint2*)((uint16_t*)out + start))[i] = make_uint2(lo, hi);
            }
        }
    } else {
        for (int64_t i = tid; i < len; i += kPackThreads) {
            const float v = wl[stage_idx(i)];
            if (out_dtype == 0) ((float*)out)[start + i] = v;
            else ((uint16_t*)out)[start + i] = f32_to_bf16_rne(v);
        }
    }
}

// Unpack at G = 64 with whole groups (K % 64 == 0), so that group g's 64
// values are elements 64 g .. 64 g + 63 of the output.  A wave takes 8
// groups (104 code bytes, 512 values) at a time; lane (g, q) writes values
// 8 q .. 8 q + 7 of its group as one 16-byte piece (two for fp32).  Those are
// digits o .. o + 7 of the 15 held by code bytes f, f + 1, f + 2 of the group
// (f = floor(8 q / 5), o = 8 q - 5 f; the third byte, needed when o >= 3,
// is clamped into the group).  Each byte's five digits come from a
// 256-entry table (2 bits a digit; bytes 243..255 decode as 121, all
// zeros).  A digit d gives the value bits (s ^ sign) & mask: mask clears
// d = 1 (t = 0), sign flips d = 0 (t = -1), so each value is exactly
// s * t rounded as the general kernel rounds it.  Every code byte of a
// group lies in some lane's window, and lane q = 7's window holds the
// padding digit (digit 4 of byte 12), so the status flags match too.  The
// output is written with streaming (nontemporal) stores: nothing reads it
// back in this kernel, and the write stream then runs about a third faster.
constexpr int kUn64Threads = 256;
typedef unsigned short u16x2un __attribute__((ext_vector_type(2)));

__global__ void __launch_bounds__(kUn64Threads)
unpack64_kernel(const uint8_t* __restrict__ codes, const uint16_t* __restrict__ scales,
                int64_t groups, void* __restrict__ out, int out_dtype, int32_t* st) {
    __shared__ uint32_t dig[256];
    const int tid = threadIdx.x;
    {
        uint32_t v = tid > 242 ? 121u : (uint32_t)tid, e = 0;
#pragma unroll
        for (int i = 0; i < 5; ++i) {
            e |= (v % 3u) << (2 * i);
            v /= 3u;
        }
        dig[tid] = e;
    }
    __syncthreads();
    const int lane = tid & 63;
    const uint32_t q = (uint32_t)(lane & 7);
    const uint32_t f = (8u * q) / 5u, o = 8u * q - 5u * f;
    const uint32_t f3 = f + 2u < 12u ? f + 2u : 12u;
    int flags = 0;
    const int64_t tasks = (groups + 7) >> 3;
    const int64_t stride = (int64_t)gridDim.x * (kUn64Threads / 64);
    for (int64_t t = (int64_t)blockIdx.x * (kUn64Threads / 64) + (tid >> 6); t < tasks; t += stride) {
        const int64_t g = 8 * t + (lane >> 3);
        if (g >= groups) continue;
        const uint8_t* cb = codes + 13 * g;
        const uint32_t b0 = cb[f], b1 = cb[f + 1], b2 = cb[f3];
        if (b0 > 242u || b1 > 242u || b2 > 242u) flags |= TQ_DATA_CODE;
        const uint32_t w = (dig[b0] | (dig[b1] << 10) | (dig[b2] << 20)) >> (2u * o);
        if (q == 7u && ((w >> 16) & 3u) != 1u) flags |= TQ_DATA_PADDING;
        const float sf = f16_bits_to_f32(scales[g]);
        if (out_dtype == TQ_BF16) {
            const uint32_t sb = f32_to_bf16_rne(sf);
            const uint32_t s2 = sb | (sb << 16);
            u32x4 v;
#pragma unroll
            for (int p = 0; p < 4; ++p) {
                // digits 2p (low half) and 2p + 1 (high half)
                const uint32_t x = w >> (4 * p);
                const uint32_t d = (x & 3u) | ((x << 14) & 0x30000u);
                // per 16-bit half: (d & 1) - 1 is 0 where d == 1, else 0xFFFF
                const uint32_t mask = __builtin_bit_cast(
                    uint32_t, __builtin_bit_cast(u16x2un, d & 0x00010001u) - (u16x2un){1, 1});
                const uint32_t sign = ((d ^ 0x00020002u) & 0x00020002u) << 14;
                v[p] = (s2 ^ sign) & mask;
            }
            __builtin_nontemporal_store(v, (u32x4*)((uint16_t*)out + 64 * g + 8 * q));
        } else {
            const uint32_t s32 = __builtin_bit_cast(uint32_t, sf);
            u32x4 v[2];
#pragma unroll
            for (int k = 0; k < 8; ++k) {
                const uint32_t d = (w >> (2 * k)) & 3u;
                const uint32_t mask = (d & 1u) - 1u;                     // 0 where d == 1
                const uint32_t sign = ((d ^ 2u) & 2u) << 30;
                v[k >> 2][k & 3] = (s32 ^ sign) & mask;
            }
            __builtin_nontemporal_store(v[0], (u32x4*)((float*)out + 64 * g + 8 * q));
            __builtin_nontemporal_store(v[1], (u32x4*)((float*)out + 64 * g + 8 * q + 4));
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
    const int gpw = groups_per_wg(G);
    int64_t blocks = (groups + gpw - 1) / gpw;
    hipLaunchKernelGGL(pack_kernel, dim3((unsigned)blocks), dim3(kPackThreads), 0, s, W, rows,
                       K, G, ng, nb, gpw, planes, c1, s1, c2, s2, d_status);
    return hipGetLastError();
}

hipError_t launch_unpack(const uint8_t* codes, const uint16_t* scales, int64_t rows,
                         int64_t K, int G, void* out, int out_dtype, int32_t* d_status,
                         hipStream_t s) {
    int ng = (int)((K + G - 1) / G);
    int nb = (G + 4) / 5;
    int64_t groups = rows * (int64_t)ng;
    if (groups == 0) return hipSuccess;
    if (G == 64 && K % 64 == 0 && ((uintptr_t)out & 15) == 0) {
        // whole groups of 64: the wave-per-8-groups kernel, a grid of a few
        // workgroups per compute unit striding over the groups
        const int64_t wgs = (groups + 8 * (kUn64Threads / 64) - 1) / (8 * (kUn64Threads / 64));
        const int64_t cap = 8 * (int64_t)compute_unit_count();
        hipLaunchKernelGGL(unpack64_kernel, dim3((unsigned)(wgs < cap ? wgs : cap)),
                           dim3(kUn64Threads), 0, s, codes, scales, groups, out, out_dtype, d_status);
        return hipGetLastError();
    }
    const int gpw = groups_per_wg(G);
    int64_t blocks = (groups + gpw - 1) / gpw;
    hipLaunchKernelGGL(unpack_kernel, dim3((unsigned)blocks), dim3(kPackThreads), 0, s, codes,
                       scales, rows, K, G, ng, nb, gpw, out, out_dtype, d_status);
    return hipGetLastError();
}

}  // namespace dmm
