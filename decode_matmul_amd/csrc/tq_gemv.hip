// Ternary GEMV: y = x (s1 T1 + s2 T2)^T over the mean-abs ternary package,
// decoded inside the kernel.
//
// Format: "Does your weight format deserve a kernel?" (pack-unpack-run),
// "Five trits in a byte" and "Three values and a shared scale"; the second
// plane and the expert selection follow the FUCINA README ("The method",
// "Runtime requirements").
//
// Mapping onto gfx950 (wave64, bf16 MFMA 16x16x32, fp32 accumulate):
//
//  * A workgroup owns 16 output rows (one MFMA column block) of one expert
//    and splits the K groups over its waves; wave partials meet in LDS.
//  * Each lane of a wave decodes one whole group of one row: lane l handles
//    row (l & 15) and group 4*quad + (l >> 4).  The group's ceil(G/5) code
//    bytes are fetched with aligned dword loads and realigned with
//    v_alignbyte; each byte indexes a 256-entry LDS table that holds the
//    five trits as the high bytes of bf16 values 2t (0x40 / 0x00 / 0xC0), and
//    v_perm assembles bf16 pairs (2t_j, 2t_{j+1}) in natural trit order.
//    Trits are exact in bf16; the factor 2 is folded into the group scale.
//  * The MFMA A operand is block diagonal: A row r = 4 m + g' holds token m's
//    activations for group g' in the K-slots of lane block g' and zeros
//    elsewhere.  C[4 m + g', col] is then the partial sum of exactly one
//    group, so the fp16 group scale is applied in fp32 after the MFMA (per
//    group, as the format requires) at no extra MFMA cost for M <= 4.  More
//    tokens run further token quads over the same decoded operands.
//  * Activations are read straight from global memory (they are tiny and
//    stay in L1/L2) at any element offset; codes stream from HBM once per
//    token chunk of 16.
#include "common.h"

namespace dmm {

namespace {

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kChunk = 16;          // tokens per pass over the codes
constexpr int kMaxList = 4096;      // grouped mode: M * top_k limit

struct Params {
    const uint16_t* x;
    int64_t K, N;
    int ng;                          // groups per row
    const uint8_t* codes0;
    const uint8_t* codes1;
    const uint16_t* scales0;
    const uint16_t* scales1;
    int planes;
    int64_t code_stride;             // bytes per expert
    int64_t scale_stride;            // scales per expert
    int grouped;
    int e_begin;                     // grouped: first expert of this launch
    const int32_t* ids;
    int top_k;
    int M;                           // tokens
    int row_blocks;
    void* y;
    int y_dtype;
    int list_bytes;                  // dynamic LDS for the grouped token list
};

// bf16 high byte of 2t for digit d = t + 1.
__device__ __forceinline__ uint32_t trit_hi_byte(int d) {
    return d == 2 ? 0x40u : (d == 0 ? 0xC0u : 0x00u);
}

// Raw aligned words holding the NB code bytes of one group at byte address
// p: W[0..NW-1] plus the byte shift sh = p & 3.  Every word read holds at
// least one byte of the group (so no read leaves the package).
template <int NB>
struct RawGroup {
    static constexpr int NW = (NB == 13) ? 4 : 8;
    uint32_t W[NW];
    uint32_t sh;
};

template <int NB>
__device__ __forceinline__ void load_group_raw(const uint8_t* p, RawGroup<NB>& R) {
    R.sh = (uint32_t)((uintptr_t)p & 3);
    const uint32_t* aw = (const uint32_t*)(p - R.sh);    // keeps the global address space
    if constexpr (NB == 13) {
        // 13 bytes at offset sh <= 3 always fit the 16 aligned bytes
        u32x4a v = *(const u32x4a*)aw;
        R.W[0] = v.x; R.W[1] = v.y; R.W[2] = v.z; R.W[3] = v.w;
    } else {
        static_assert(NB == 26, "G = 64 or 128");
        u32x4a v = *(const u32x4a*)aw;
        u32x3a u = *(const u32x3a*)(aw + 4);
        R.W[0] = v.x; R.W[1] = v.y; R.W[2] = v.z; R.W[3] = v.w;
        R.W[4] = u.x; R.W[5] = u.y; R.W[6] = u.z;
        R.W[7] = aw[R.sh == 3 ? 7 : 6];     // byte 25 sits in word 7 only if sh == 3
    }
}

// Decode one group (G trits) into G/2 bf16 pair registers, natural order.
template <int G>
__device__ __forceinline__ void decode_group(const RawGroup<(G + 4) / 5>& R, const uint2* lut,
                                             uint32_t* B) {
    constexpr int NB = (G + 4) / 5;
    constexpr int ND = (NB + 3) / 4;
    uint32_t D[ND];
#pragma unroll
    for (int i = 0; i < ND; ++i) {
        const uint32_t hi = (i + 1 < RawGroup<NB>::NW) ? R.W[i + 1] : 0u;
        D[i] = align_bytes(hi, R.W[i], R.sh);
    }
    uint32_t Elo[NB], Ehi[NB];
#pragma unroll
    for (int i = 0; i < NB; ++i) {
        uint32_t b = (D[i >> 2] >> (8 * (i & 3))) & 0xffu;
        uint2 e = lut[b];
        Elo[i] = e.x;
        Ehi[i] = e.y;
    }
#pragma unroll
    for (int p2 = 0; p2 < G / 2; ++p2) {
        const int ja = 2 * p2, jb = 2 * p2 + 1;
        const int ia = ja / 5, qa = ja % 5, ib = jb / 5, qb = jb % 5;
        const uint32_t ra = qa < 4 ? Elo[ia] : Ehi[ia];
        const uint32_t rb = qb < 4 ? Elo[ib] : Ehi[ib];
        const uint32_t ba = qa < 4 ? qa : 0, bb = qb < 4 ? qb : 0;
        const bool same = (ia == ib) && ((qa < 4) == (qb < 4));
        if (same) {
            B[p2] = perm_b32(ra, ra, 0x0cu | (ba << 8) | (0x0cu << 16) | (bb << 24));
        } else {
            B[p2] = perm_b32(rb, ra, 0x0cu | (ba << 8) | (0x0cu << 16) | ((4u + bb) << 24));
        }
    }
}

// G: group size.  PL: planes (1 or 2).  XLDS: the chunk's activations (<= 4
// tokens) are staged in LDS; otherwise A operands are read from global memory
// in chunks of 16 tokens.  SV: the four scales of a quad are one 8-byte load.
template <int G, int PL, bool XLDS, bool SV>
__global__ void __launch_bounds__(kThreads, (PL == 2 || G == 128) ? 2 : 3)
tq_gemv_kernel(Params p) {
    constexpr int NB = (G + 4) / 5;
    constexpr int NQ = G / 8;             // MFMAs per group (8 trits per lane each)
    constexpr int kTokChunk = XLDS ? 4 : kChunk;
    __shared__ uint2 lut[256];
    __shared__ int list_n;
    __shared__ float red[kWaves][4][64];
    extern __shared__ __attribute__((aligned(16))) unsigned char dyn[];
    int* list = (int*)dyn;                                       // grouped: M * top_k
    uint16_t* xs = (uint16_t*)(dyn + p.list_bytes);              // XLDS: [4][K]

    const int tid = threadIdx.x;
    const int wave = readfirstlane(tid >> 6);   // wave-uniform: scalar loop bounds
    const int lane = tid & 63;

    {   // byte -> five trits, as bf16 high bytes of 2t
        int b = tid;
        uint32_t lo = 0, hi = 0;
        if (b < 243) {
            int v = b;
            uint32_t h[5];
#pragma unroll
            for (int q = 0; q < 5; ++q) { h[q] = trit_hi_byte(v % 3); v /= 3; }
            lo = h[0] | (h[1] << 8) | (h[2] << 16) | (h[3] << 24);
            hi = h[4];
        }
        lut[b] = make_uint2(lo, hi);
    }

    const int item = blockIdx.x;
    const int rb = item % p.row_blocks;
    const int e = p.e_begin + item / p.row_blocks;

    if (p.grouped && wave == 0) {
        int count = 0;
        const int total = p.M * p.top_k;
        for (int base = 0; base < total; base += 64) {
            int idx = base + lane;
            bool pred = idx < total && p.ids[idx] == e;
            uint64_t mask = __ballot(pred);
            int pos = count + __popcll(mask & ((1ull << lane) - 1ull));
            if (pred) list[pos] = idx;
            count += __popcll(mask);
        }
        if (lane == 0) list_n = count;
    }
    __syncthreads();
    const int n_list = p.grouped ? list_n : p.M;
    if (n_list == 0) return;

    const uint8_t* Cp[2];
    const uint16_t* Sp[2];
    Cp[0] = p.codes0 + (int64_t)e * p.code_stride;
    Sp[0] = p.scales0 + (int64_t)e * p.scale_stride;
    Cp[1] = PL == 2 ? p.codes1 + (int64_t)e * p.code_stride : Cp[0];
    Sp[1] = PL == 2 ? p.scales1 + (int64_t)e * p.scale_stride : Sp[0];

    const int col = lane & 15;
    const int kb = lane >> 4;                 // group within a quad (B side)
    const int64_t n = (int64_t)rb * 16 + col;
    const bool row_ok = n < p.N;
    const int64_t nc = row_ok ? n : 0;        // clamped row for branch-free loads
    const int ar = lane & 15;                 // A row: 4 * token + group
    const int am = ar >> 2;
    const bool a_diag = (ar & 3) == kb;
    const int nquads = (p.ng + 3) >> 2;
    // this wave's quads: wave, wave + kWaves, ...
    const int nmy = wave < nquads ? (nquads - wave + kWaves - 1) / kWaves : 0;

    struct Slot {
        RawGroup<NB> raw[PL];
        uint32_t scw[PL][2];
    };
    // loads of the j-th quad of this wave, clamped so they never branch
    auto stage = [&](int j, Slot& S) {
        const int qd = wave + kWaves * min(j, nmy - 1);
        const int g = 4 * qd + kb;
        const int64_t gi = nc * p.ng + (g < p.ng ? g : 0);
#pragma unroll
        for (int pl = 0; pl < PL; ++pl) {
            load_group_raw<NB>(Cp[pl] + gi * NB, S.raw[pl]);
            if constexpr (SV) {
                const uint32_t* sp = (const uint32_t*)(Sp[pl] + nc * p.ng + 4 * qd);
                S.scw[pl][0] = sp[0];
                S.scw[pl][1] = sp[1];
            } else {
                uint32_t h[4];
#pragma unroll
                for (int j2 = 0; j2 < 4; ++j2) {
                    const int gj = 4 * qd + j2;
                    h[j2] = Sp[pl][nc * p.ng + (gj < p.ng ? gj : 0)];
                }
                S.scw[pl][0] = h[0] | (h[1] << 16);
                S.scw[pl][1] = h[2] | (h[3] << 16);
            }
        }
    };

    for (int tok0 = 0; tok0 < n_list; tok0 += kTokChunk) {
        const int ntok = min(kTokChunk, n_list - tok0);
        const int ntq = (ntok + 3) >> 2;

        if constexpr (XLDS) {
            // stage x rows of this chunk: xs[t][0:K], zero rows past ntok
            const int per_row = (int)(p.K >> 3);               // 16-byte pieces per row
            for (int i = tid; i < 4 * per_row; i += kThreads) {
                const int t = i / per_row, c = i - t * per_row;
                u32x4 v = {0u, 0u, 0u, 0u};
                if (t < ntok) {
                    const int sl = p.grouped ? list[tok0 + t] : (tok0 + t);
                    const int64_t row = p.grouped ? (int64_t)(sl / p.top_k) : (int64_t)sl;
                    u32x4h w = *(const u32x4h*)(p.x + row * p.K + 8 * c);
                    v = u32x4{w.x, w.y, w.z, w.w};
                }
                *(u32x4*)(xs + t * p.K + 8 * c) = v;
            }
            __syncthreads();
        }

        float yacc[4] = {0.f, 0.f, 0.f, 0.f};

        // decode + MFMA of the j-th quad of this wave from its loaded slot
        auto proc = [&](int j, const Slot& S) {
            const int qd = wave + kWaves * j;
            const int g = 4 * qd + kb;
            const bool g_ok = row_ok && g < p.ng;
#pragma unroll
            for (int pl = 0; pl < PL; ++pl) {
                float sc[4];
#pragma unroll
                for (int j2 = 0; j2 < 4; ++j2) {
                    const uint32_t w = S.scw[pl][j2 >> 1];
                    const uint16_t h = (uint16_t)((j2 & 1) ? (w >> 16) : (w & 0xffffu));
                    sc[j2] = (row_ok && 4 * qd + j2 < p.ng) ? 0.5f * f16_bits_to_f32(h) : 0.f;
                }
                uint32_t B[G / 2];
                decode_group<G>(S.raw[pl], lut, B);
                const int ntq_eff = XLDS ? 1 : ntq;
                for (int tq = 0; tq < ntq_eff; ++tq) {
                    const int tl = 4 * tq + am;
                    const bool a_ok = a_diag && tl < ntok && g < p.ng;
                    int64_t xrow = 0;
                    if (!XLDS && a_ok) {
                        const int sl = p.grouped ? list[tok0 + tl] : (tok0 + tl);
                        xrow = p.grouped ? (int64_t)(sl / p.top_k) : (int64_t)sl;
                    }
                    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int q = 0; q < NQ; ++q) {
                        u32x4 A = {0u, 0u, 0u, 0u};
                        if (a_ok) {
                            if constexpr (XLDS) {
                                A = *(const u32x4*)(xs + tl * p.K + (int64_t)g * G + 8 * q);
                            } else {
                                u32x4h v = *(const u32x4h*)(p.x + xrow * p.K + (int64_t)g * G +
                                                            8 * q);
                                A = u32x4{v.x, v.y, v.z, v.w};
                            }
                        }
                        u32x4 bq = {B[4 * q], B[4 * q + 1], B[4 * q + 2], B[4 * q + 3]};
#pragma unroll
                        for (int i = 0; i < 4; ++i) bq[i] = g_ok ? bq[i] : 0u;
                        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                            __builtin_bit_cast(bf16x8, A), __builtin_bit_cast(bf16x8, bq), acc,
                            0, 0, 0);
                    }
                    const float contrib =
                        sc[0] * acc[0] + sc[1] * acc[1] + sc[2] * acc[2] + sc[3] * acc[3];
                    if (tq == 0) yacc[0] += contrib;
                    else if (tq == 1) yacc[1] += contrib;
                    else if (tq == 2) yacc[2] += contrib;
                    else yacc[3] += contrib;
                }
            }
        };

        if (nmy > 0) {
            // three slots in rotation: two quads' loads stay in flight while
            // one quad is decoded and multiplied
            Slot s0, s1, s2;
            stage(0, s0);
            stage(1, s1);
            stage(2, s2);
            int j = 0;
            for (; j + 2 < nmy; j += 3) {
                proc(j, s0);
                stage(j + 3, s0);
                proc(j + 1, s1);
                stage(j + 4, s1);
                proc(j + 2, s2);
                stage(j + 5, s2);
            }
            if (j < nmy) proc(j, s0);
            if (j + 1 < nmy) proc(j + 1, s1);
        }

        // wave partials -> LDS -> fixed-order sum in wave 0
#pragma unroll
        for (int tq = 0; tq < 4; ++tq) red[wave][tq][lane] = yacc[tq];
        __syncthreads();
        if (wave == 0) {
            for (int tq = 0; tq < ntq; ++tq) {
                float v = red[0][tq][lane];
#pragma unroll
                for (int w = 1; w < kWaves; ++w) v += red[w][tq][lane];
                const int tl = 4 * tq + (lane >> 4);
                if (tl < ntok && row_ok) {
                    const int sl = p.grouped ? list[tok0 + tl] : (tok0 + tl);
                    const int64_t idx = (int64_t)sl * p.N + n;
                    if (p.y_dtype == TQ_F32) ((float*)p.y)[idx] = v;
                    else ((uint16_t*)p.y)[idx] = f32_to_bf16_rne(v);
                }
            }
        }
        __syncthreads();
    }
}

// Rows of y whose expert id is out of range become NaN.
__global__ void bad_ids_kernel(const int32_t* ids, int total, int n_experts, int64_t N, void* y,
                               int y_dtype) {
    const int idx = blockIdx.x;
    if (idx >= total) return;
    const int e = ids[idx];
    if (e >= 0 && e < n_experts) return;
    for (int64_t n = threadIdx.x; n < N; n += blockDim.x) {
        const int64_t o = (int64_t)idx * N + n;
        if (y_dtype == TQ_F32) ((float*)y)[o] = __builtin_nanf("");
        else ((uint16_t*)y)[o] = 0x7fc0u;
    }
}

}  // namespace

hipError_t launch_tq_matmul(const TqMatmulArgs& a, hipStream_t s) {
    Params p;
    p.x = a.x;
    p.K = a.K;
    p.N = a.N;
    p.ng = (int)(a.K / a.G);
    p.codes0 = a.codes[0];
    p.codes1 = a.planes == 2 ? a.codes[1] : nullptr;
    p.scales0 = a.scales[0];
    p.scales1 = a.planes == 2 ? a.scales[1] : nullptr;
    p.planes = a.planes;
    const int nb = (a.G + 4) / 5;
    p.code_stride = a.N * (int64_t)p.ng * nb;
    p.scale_stride = a.N * (int64_t)p.ng;
    p.grouped = a.n_experts > 0;
    p.ids = a.ids;
    p.top_k = a.top_k;
    p.M = (int)a.M;
    p.row_blocks = (int)((a.N + 15) / 16);
    p.y = a.y;
    p.y_dtype = a.y_dtype;
    p.e_begin = p.grouped ? a.e_begin : 0;
    const int experts = p.grouped ? a.e_end - a.e_begin : 1;
    const int64_t items = (int64_t)p.row_blocks * experts;
    if (items == 0) return hipSuccess;
    {
        // the streaming form writes the rows of out-of-range expert ids itself
        hipError_t e;
        if (launch_tq_wave(a, s, &e)) return e;
        if (launch_tq_batch(a, s, &e)) return e;
        if (launch_tq_rows(a, s, &e)) return e;
        if (launch_tq_prefill(a, s, &e)) return e;
    }
    if (p.grouped && a.nan_rows) {
        // slots routed to no valid expert: NaN rows (no expert kernel writes them)
        const int total = (int)(a.M * a.top_k);
        hipLaunchKernelGGL(bad_ids_kernel, dim3(total), dim3(256), 0, s, a.ids, total,
                           a.n_experts, a.N, a.y, a.y_dtype);
    }
    // activations staged in LDS when a chunk of <= 4 tokens fits comfortably
    const int64_t xlds_bytes = 4 * a.K * 2;
    // dense: M tokens per workgroup; grouped: on average M * top_k / experts
    const int64_t tok_per_item =
        p.grouped ? ((int64_t)a.M * a.top_k + a.n_experts - 1) / a.n_experts : a.M;
    const bool xlds = tok_per_item <= 4 && xlds_bytes <= 64 * 1024;
    p.list_bytes = p.grouped ? (int)(((int64_t)a.M * a.top_k * 4 + 15) & ~15) : 0;
    const size_t smem = (size_t)p.list_bytes + (xlds ? (size_t)xlds_bytes : 0);
    const bool sv = (p.ng % 4 == 0) && (((uintptr_t)a.scales[0] & 7) == 0) &&
                    (a.planes < 2 || (((uintptr_t)a.scales[1] & 7) == 0));
    const dim3 grid((unsigned)items), block(kThreads);
#define DMM_TQ_LAUNCH(G_, P_, X_, S_) \
    hipLaunchKernelGGL((tq_gemv_kernel<G_, P_, X_, S_>), grid, block, smem, s, p)
#define DMM_TQ_XS(G_, P_, S_) \
    do { if (xlds) DMM_TQ_LAUNCH(G_, P_, true, S_); else DMM_TQ_LAUNCH(G_, P_, false, S_); } while (0)
    if (a.G == 64) {
        if (a.planes == 2) { if (sv) DMM_TQ_XS(64, 2, true); else DMM_TQ_XS(64, 2, false); }
        else { if (sv) DMM_TQ_XS(64, 1, true); else DMM_TQ_XS(64, 1, false); }
    } else {
        if (a.planes == 2) DMM_TQ_XS(128, 2, false);
        else DMM_TQ_XS(128, 1, false);
    }
#undef DMM_TQ_XS
#undef DMM_TQ_LAUNCH
    return hipGetLastError();
}

int tq_max_grouped_pairs() { return kMaxList; }

}  // namespace dmm
