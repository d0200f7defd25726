// Route B 7-bit truncated alphabet: code bytes -> the list of used codes and
// 7-bit indices into it.
//
// Semantics: "A Discrete Weight Language for Large Language Models" (Route
// B), section 8.1: a layer whose weights use at most 128 of the 243 codes
// can store each weight in 7 bits plus a table from the 7-bit index to the
// code.  The used codes are listed in increasing order (index j is the j-th
// smallest code present) and the list is padded to 128 with code 121, the
// all-zero word.  Row n of the output holds ceil(7 K / 8) bytes: bit q of
// index k is bit 7 k + q of the row read as a little-endian bit string; the
// bits past 7 K are zero.
//
// Four launches, no scratch memory of its own (the first 32 bytes of the
// caller's 128-byte list hold a 256-bit presence set until the list is
// written):
//  1. clear the presence set, the count and the status;
//  2. presence: each workgroup marks the codes it sees in LDS and ORs its
//     set into the global one (a byte 243..255 raises TQ_DATA_CODE);
//  3. one workgroup turns the set into the ascending list and the count
//     (more than 128 codes raise TQ_DATA_ALPHABET);
//  4. one workgroup per row writes the row's bytes, mapping codes to
//     indices through an LDS table built from the list.
#include "common.h"

namespace dmm {

namespace {

constexpr int kThreads = 256;

__global__ void tr_clear_kernel(uint32_t* set, int32_t* n_used, int32_t* status) {
    if (threadIdx.x < 8) set[threadIdx.x] = 0u;
    if (threadIdx.x == 0) {
        *n_used = 0;
        *status = 0;
    }
}

__global__ void __launch_bounds__(kThreads)
tr_presence_kernel(const uint8_t* codes, int64_t total, uint32_t* set, int32_t* status) {
    __shared__ uint32_t seen[256];
    __shared__ uint32_t words[8];
    const int tid = threadIdx.x;
    seen[tid] = 0u;
    __syncthreads();
    const int64_t stride = (int64_t)gridDim.x * kThreads;
    const int64_t first = (int64_t)blockIdx.x * kThreads + tid;
    if (((uintptr_t)codes & 15) == 0) {
        const int64_t nvec = total / 16;
        for (int64_t v = first; v < nvec; v += stride) {
            const u32x4 q = *(const u32x4*)(codes + 16 * v);
#pragma unroll
            for (int w = 0; w < 4; ++w)
#pragma unroll
                for (int b = 0; b < 4; ++b) seen[(q[w] >> (8 * b)) & 0xffu] = 1u;
        }
        for (int64_t i = 16 * nvec + first; i < total; i += stride) seen[codes[i]] = 1u;
    } else {
        for (int64_t i = first; i < total; i += stride) seen[codes[i]] = 1u;
    }
    __syncthreads();
    if (tid < 8) {
        uint32_t word = 0u;
        for (int b = 0; b < 32; ++b) word |= (seen[32 * tid + b] != 0u ? 1u : 0u) << b;
        words[tid] = word;
        if (word) atomicOr(set + tid, word);
    }
    __syncthreads();
    // codes 243..255 live in bits 19..31 of word 7
    if (tid == 0 && (words[7] >> 19) != 0u) atomicOr(status, (int32_t)TQ_DATA_CODE);
}

__global__ void __launch_bounds__(kThreads)
tr_list_kernel(uint8_t* used, int32_t* n_used, int32_t* status) {
    const uint32_t* set = (const uint32_t*)used;
    const int t = threadIdx.x;                           // candidate code t
    uint32_t w[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) w[i] = set[i];
    w[7] &= (1u << 19) - 1u;                             // codes 0..242 only
    int below = 0, total = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int c = __builtin_popcount(w[i]);
        total += c;
        if (i < (t >> 5)) below += c;
    }
    below += __builtin_popcount(w[t >> 5] & ((1u << (t & 31)) - 1u));
    const bool present = (w[t >> 5] >> (t & 31)) & 1u;
    __syncthreads();                                     // every thread has read the set
    if (present && below < 128) used[below] = (uint8_t)t;
    if (t < 128 && t >= total) used[t] = 121;
    if (t == 0) {
        *n_used = total;
        if (total > 128) atomicOr(status, (int32_t)TQ_DATA_ALPHABET);
    }
}

__global__ void __launch_bounds__(kThreads)
tr_pack_kernel(const uint8_t* codes, int64_t K, int64_t row_bytes, const uint8_t* used,
               const int32_t* n_used, uint8_t* out) {
    __shared__ uint8_t index_of[256];
    const int tid = threadIdx.x;
    index_of[tid] = 0;
    __syncthreads();
    const int n = min(*n_used, 128);
    if (tid < n) index_of[used[tid]] = (uint8_t)tid;
    __syncthreads();
    const int64_t row = blockIdx.x;
    const uint8_t* src = codes + row * K;
    uint8_t* dst = out + row * row_bytes;
    for (int64_t j = tid; j < row_bytes; j += kThreads) {
        // byte j holds stream bits 8 j .. 8 j + 7: index k0 from bit o on,
        // then index k0 + 1
        const uint64_t bit = 8 * (uint64_t)j;
        const int64_t k0 = (int64_t)(bit / 7);
        const uint32_t o = (uint32_t)(bit - 7 * (uint64_t)k0);
        uint32_t v = k0 < K ? index_of[src[k0]] : 0u;
        if (k0 + 1 < K) v |= (uint32_t)index_of[src[k0 + 1]] << 7;
        dst[j] = (uint8_t)(v >> o);
    }
}

}  // namespace

hipError_t launch_rb_truncate(const uint8_t* codes, int64_t N, int64_t K, uint8_t* used,
                              int32_t* n_used, uint8_t* codes7, int32_t* status, hipStream_t s) {
    uint32_t* set = (uint32_t*)used;
    hipLaunchKernelGGL(tr_clear_kernel, dim3(1), dim3(64), 0, s, set, n_used, status);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int64_t total = N * K;
    if (total > 0) {
        int64_t g = (total + 16 * kThreads * 8 - 1) / (16 * kThreads * 8);
        g = g < 1 ? 1 : (g > 2048 ? 2048 : g);
        hipLaunchKernelGGL(tr_presence_kernel, dim3((unsigned)g), dim3(kThreads), 0, s, codes,
                           total, set, status);
        e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL(tr_list_kernel, dim3(1), dim3(kThreads), 0, s, used, n_used, status);
    e = hipGetLastError();
    if (e != hipSuccess || N == 0 || K == 0) return e;
    hipLaunchKernelGGL(tr_pack_kernel, dim3((unsigned)N), dim3(kThreads), 0, s, codes, K,
                       rb7_row_bytes(K), used, n_used, codes7);
    return hipGetLastError();
}

}  // namespace dmm
