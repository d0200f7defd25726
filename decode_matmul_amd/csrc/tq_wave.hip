// Ternary GEMV for a few tokens over dense weights, and the grouped expert
// form of it, wave by wave: y = x (s1 T1 + s2 T2)^T with G = 64, decoded
// inside the kernel.
//
// Format: pack-unpack-run, "Five trits in a byte" (five base-3 digits per
// byte, least significant first) and "Three values and a shared scale"
// (W_hat = s t per group of 64); the second plane, the experts and the hot
// prefix follow the FUCINA README ("The method", "Runtime requirements").
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
//  * the activations are staged in LDS with coalesced loads issued ahead of
//    the code stream, and each lane takes its 64 in the K order of the MFMA
//    operands;
//  * a group's sum is scaled by its fp16 scale in fp32; the 16 group slices
//    of a row are summed across lanes and waves in a fixed order.
// Dense calls take one range of rows per workgroup.  Grouped calls run one
// persistent workgroup per compute unit over the routed work (expert, pass
// of up to four of its (token, slot) pairs, row quad), in rounds whose next
// load goes out before the round's closing barrier.
#include <algorithm>

#include "common.h"
#include "tq_book.h"

namespace dmm {

namespace {

constexpr int kW = 16;
constexpr int kT = 64 * kW;
constexpr int kNB = 13;                  // code bytes per group of 64 trits
constexpr int kMaxTasks = 4;             // tasks per wave
constexpr int kXsPitch = 144;            // LDS bytes per staged group of 64 activations
// per token (at most 64 groups), padded by 64 bytes: the 16 lanes of an
// operand read (groups 4p .. 4p + 3 of tokens 0 .. 3) then hit 16 distinct
// 16-byte bank units (64 banks) instead of one unit per token
constexpr int kXsTok = 64 * kXsPitch + 64;
constexpr int kTaskStride = 68;          // floats per task: [4 lane rows][4 rows][4 tokens] + pad

typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

struct WaveParams {
    const uint16_t* x;
    int64_t K, N;
    int ng, M;                   // dense: M tokens (rows of x and of y)
    const uint8_t* codes[2];
    const uint16_t* scales[2];
    int rows_per_wg;             // dense: rows of a workgroup
    int nrq;                     // grouped: row quads of one expert, ceil(N / 4)
    int nwg;                     // grouped: workgroups that share the work
    void* y;
    int y_dtype;
    // grouped experts: the (token, slot) pairs routed to expert e_begin + el,
    // el < nl, in passes of up to four
    const int32_t* ids;          // [M * top_k]
    int total, top_k, n_experts, e_begin, nl;
    int nan_rows;                // workgroup 0 writes the rows of out-of-range ids
    int64_t e_codes, e_scales;   // bytes / scales of one expert in a plane
};

// grouped bookkeeping in LDS: per local expert its pair count, first list
// slot and first work index (row quads over all passes), then the pair list
constexpr int kMaxLocal = 256;
constexpr int kCnt = 0, kPst = kMaxLocal, kQst = 2 * kMaxLocal, kList = 3 * kMaxLocal + 4;
constexpr int kMetaInts = kList + 256;

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

// One launch's work (a dense call, or the experts of one grouped call) on a
// workgroup: lut is the code book (filled here when book is set), xs the
// staged activations, meta the grouped bookkeeping, red the per-round slices.
// Issue priority after a wave's task t of a round (3 at the round's start):
// a wave that is ahead yields to those behind.
__device__ __forceinline__ void yield_after(int t) {
    if (t == 0) __builtin_amdgcn_s_setprio(2);
    else if (t == 1) __builtin_amdgcn_s_setprio(1);
    else if (t == 2) __builtin_amdgcn_s_setprio(0);
}

// A operands of lane (b, j): token j's group g from the staged activations,
// in the K order above (zero for j >= nt).
__device__ __forceinline__ void build_a(const unsigned char* xs, int j, int g, int nt, u32x2 (&A)[16]) {
    uint32_t xw[32];
    const bool ok = j < nt;
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

// One task on lane (b, j): D[r] of block b is token r, row j of the task,
// summed over the planes with their group scales (codes c[pl], aligned down
// by sh bytes, scale s[pl]); the four blocks of each 16-lane row are summed
// and lanes 16 i + j (i = lane row) store their 4 tokens at dst + 16 i + 4 j.
template <int PL>
__device__ __forceinline__ void decode_task(const u32x4 (&c)[PL], const uint16_t (&s)[PL],
                                            const u32x2 (&A)[16], const unsigned char* lut,
                                            uint32_t cofs, uint32_t sh, int lane, float* dst) {
    f32x4 tot = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int pl = 0; pl < PL; ++pl) {
        uint32_t D[4];
        D[0] = align_bytes(c[pl].y, c[pl].x, sh);
        D[1] = align_bytes(c[pl].z, c[pl].y, sh);
        D[2] = align_bytes(c[pl].w, c[pl].z, sh);
        D[3] = align_bytes(0u, c[pl].w, sh);
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
        const float sc = (float)__builtin_bit_cast(_Float16, s[pl]);
#pragma unroll
        for (int r = 0; r < 4; ++r) tot[r] = __builtin_fmaf(sc, acc[r], tot[r]);
    }
    // sum over the four blocks of each 16-lane row (lanes 4 b' + j)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        float v = tot[r];
        // (a rotation inside the row reads valid lanes only; bound_ctrl lets
        // the move fold into the add)
        v += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0x124, 0xF, 0xF, true));
        v += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0x128, 0xF, 0xF, true));
        tot[r] = v;
    }
    if ((lane & 12) == 0) *(f32x4*)(dst + (lane >> 4) * 16 + 4 * (lane & 3)) = tot;
}

// y[m, n] = 1/2 (the code book holds 2t) of the sum over the slices and the
// four lane rows of row n, in a fixed order: the slices of row quad rq sit at
// red + (rq nkq + q) kTaskStride; nrows rows from row n0, y row yrow(m).
// Thread (rq, c, q) sums slice q of row 4 rq + c over the lane rows (one
// float4 per lane row: the four tokens), the four threads of a row add their
// sums pairwise, and thread q writes token q.
template <typename YRow>
__device__ __forceinline__ void write_rows(const float* red, int nkq, int nrows, int nt, int64_t n0,
                                           int64_t N, void* y, int y_dtype, YRow yrow) {
    const int tid = threadIdx.x;
    const int q = tid & 3, c = (tid >> 2) & 3, rq = tid >> 4;
    const int row = 4 * rq + c;
    f32x4 v = {0.f, 0.f, 0.f, 0.f};
    if (row < nrows && q < nkq) {
        const float* src = red + (rq * nkq + q) * kTaskStride + 4 * c;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const f32x4 w = *(const f32x4*)(src + 16 * r);
            v[0] += w[0]; v[1] += w[1]; v[2] += w[2]; v[3] += w[3];
        }
    }
    // (q0 + q1) + (q2 + q3) on every lane of the quad (addition commutes)
#pragma unroll
    for (int m = 0; m < 4; ++m) {
        float t = v[m];
        t += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, t), 0xB1, 0xF, 0xF, true));
        t += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, t), 0x4E, 0xF, 0xF, true));
        v[m] = t;
    }
    if (row < nrows && q < nt) {
        const float o = 0.5f * (q == 0 ? v[0] : q == 1 ? v[1] : q == 2 ? v[2] : v[3]);
        const int64_t idx = yrow(q) * N + n0 + row;
        if (y_dtype == TQ_F32) ((float*)y)[idx] = o;
        else ((uint16_t*)y)[idx] = f32_to_bf16_rne(o);
    }
}

// ---- dense: workgroup w owns rows [w rows_per_wg, ...), row quad rr + t nrr
// of them for task t of the wave (kq, rr); one pass.
template <int PL>
__global__ void __launch_bounds__(kT, 1) tq_wave_dense_kernel(WaveParams p) {
    __shared__ __attribute__((aligned(16))) unsigned char lut[256 * 256];
    __shared__ __attribute__((aligned(16))) unsigned char xs[4 * kXsTok];
    extern __shared__ __attribute__((aligned(16))) float red[];   // [row quad][slice][kTaskStride]

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = readfirstlane(tid >> 6);
    // read here, before the first branch, so that its argument load goes out
    // with the others instead of after the activation loads (a second trip)
    const int rows_per_wg = p.rows_per_wg;
    asm volatile("" ::"s"(rows_per_wg));
    const int64_t r0 = (int64_t)blockIdx.x * rows_per_wg;
    const int nrows = (int)(min(r0 + (int64_t)rows_per_wg, p.N) - r0);
    const int nrq = (nrows + 3) >> 2;                 // row quads of the workgroup
    const int nkq = p.ng >> 4;                        // 16-group slices of K
    const int kq = wave % nkq, rr = wave / nkq, nrr = kW / nkq;
    const bool active = rr < nrr;                     // K = 3072 leaves one wave out
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
    // not wait for it.  Every task is loaded (past the end: the last row
    // quad again, a cache hit), so that no load sits under a branch.
    // The row quad's first row is uniform (a scalar base address); a lane
    // adds its own 32-bit offset.
    u32x4 C[kMaxTasks][PL];
    uint16_t S[kMaxTasks][PL];
    const uint32_t lane_co = (uint32_t)(kNB * g) - sh, lane_so = 2u * (uint32_t)g;
    auto issue = [&](int t) {
        const int rq = min(rr + t * nrr, nrq - 1);
        const uint32_t jj = (uint32_t)min(j, nrows - 1 - 4 * rq);
        const int64_t row0 = r0 + 4 * rq;
        const uint32_t co = jj * (uint32_t)rb + lane_co, so = jj * (uint32_t)(2 * p.ng) + lane_so;
#pragma unroll
        for (int pl = 0; pl < PL; ++pl) {
            const uint8_t* cb = p.codes[pl] + row0 * rb;
            const uint8_t* sb = (const uint8_t*)p.scales[pl] + row0 * 2 * p.ng;
            C[t][pl] = __builtin_nontemporal_load((const u32x4a*)(cb + co));
            S[t][pl] = __builtin_nontemporal_load((const uint16_t*)(sb + so));   // read once
        }
    };
    issue(0);
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_setprio(3);

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
    fill_book(lut, tid);
    __syncthreads();

    u32x2 A[16];
    build_a(xs, j, g, p.M, A);
    const uint32_t cofs = (uint32_t)(lane & 31) << 3;    // code-book copy lane % 32
#pragma unroll
    for (int t = 0; t < kMaxTasks; ++t) {
        if (t + 1 < kMaxTasks) issue(t + 1);
        const int rq = rr + t * nrr;
        if (active && rq < nrq)
            decode_task<PL>(C[t], S[t], A, lut, cofs, sh, lane, red + (rq * nkq + kq) * kTaskStride);
        // a wave that is ahead yields issue priority to those behind, so
        // that the waves reach the barrier together
        yield_after(t);
    }
    __builtin_amdgcn_s_setprio(0);
    __syncthreads();
    write_rows(red, nkq, nrows, p.M, r0, p.N, p.y, p.y_dtype, [](int m) { return (int64_t)m; });
}

// Where a grouped workgroup's work stands: local expert el, pass of four
// tokens, first row quad rq and number of row quads len of a round, its first
// work index q, and the first work index of its (expert, pass) segment, which
// names the tokens of the round.
struct Round {
    int el, pass, rq, len, q, seg;
};

// ---- grouped: work item q is a row quad of one (expert, pass) segment:
// segments in expert order, passes in order, row quads in order.  Workgroup
// w takes items [w Q / nwg, (w + 1) Q / nwg) in rounds of at most 4 nrr row
// quads that stay inside a segment; a round ends with the slices of K summed
// across waves.  lut is the code book (filled here when book is set), xs the
// staged activations, meta the bookkeeping, red the per-round slices.
template <int PL>
__device__ __forceinline__ void grouped_work(const WaveParams& p, unsigned char* lut, unsigned char* xs,
                                             int* meta, float* red, bool book) {
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = readfirstlane(tid >> 6);
    const int bid = (int)blockIdx.x;
    const int nkq = p.ng >> 4;                        // 16-group slices of K
    const int kq = wave % nkq, rr = wave / nkq, nrr = kW / nkq;
    const bool active = rr < nrr;                     // K = 3072 leaves one wave out
    const int L = 4 * nrr;                            // row quads of a full round
    const int b = lane >> 2, j = lane & 3;
    const int g = 16 * kq + b;
    const uint32_t sh = (uint32_t)(b & 3);            // 13 g == g (mod 4)
    const int64_t rb = (int64_t)p.ng * kNB;
    const int per_tok = (int)(p.K >> 3);              // 16-byte pieces of a row of x

    // ---- per local expert the pairs routed to it (counted by one wave), the
    // exclusive scans of counts and of work items, and the pair list in
    // increasing pair order (one wave per expert, from ballots)
    int vid[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        const int i = 64 * u + lane;
        vid[u] = i < p.total ? p.ids[i] : -1;
    }
    if (book) fill_book(lut, tid);
    // every wave consumes the ids here, so that no later reuse of their
    // registers has to wait on the memory counter
    uint64_t bad[4];                                  // pairs 64 u + lane routed outside [0, n_experts)
#pragma unroll
    for (int u = 0; u < 4; ++u)
        bad[u] = __builtin_amdgcn_ballot_w64(64 * u + lane < p.total && (vid[u] < 0 || vid[u] >= p.n_experts));
    if (wave == 0) {
        *(int4*)(meta + kCnt + 4 * lane) = int4{0, 0, 0, 0};
        __builtin_amdgcn_wave_barrier();
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int d = vid[u] - p.e_begin;
            if (d >= 0 && d < p.nl) atomicAdd(&meta[kCnt + d], 1);
        }
        __builtin_amdgcn_wave_barrier();
        const int4 c = *(const int4*)(meta + kCnt + 4 * lane);
        const int w0 = ((c.x + 3) >> 2) * p.nrq, w1 = ((c.y + 3) >> 2) * p.nrq;
        const int w2 = ((c.z + 3) >> 2) * p.nrq, w3 = ((c.w + 3) >> 2) * p.nrq;
        const int sc = c.x + c.y + c.z + c.w, sq = w0 + w1 + w2 + w3;
        int ic = sc, iq = sq;
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
            const int tc = __shfl_up(ic, o), tq = __shfl_up(iq, o);
            if (lane >= o) {
                ic += tc;
                iq += tq;
            }
        }
        const int pc = ic - sc, pq = iq - sq;
        *(int4*)(meta + kPst + 4 * lane) = int4{pc, pc + c.x, pc + c.x + c.y, pc + c.x + c.y + c.z};
        *(int4*)(meta + kQst + 4 * lane) = int4{pq, pq + w0, pq + w0 + w1, pq + w0 + w1 + w2};
        if (lane == 63) meta[kQst + kMaxLocal] = iq;
    }
    __syncthreads();
    for (int el = wave; el < p.nl; el += kW) {
        if (readfirstlane(meta[kCnt + el]) == 0) continue;
        const int e = p.e_begin + el;
        int base = readfirstlane(meta[kPst + el]);
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const uint64_t m = __builtin_amdgcn_ballot_w64(vid[u] == e);
            if (vid[u] == e) meta[kList + base + __builtin_popcountll(m & ((1ull << lane) - 1ull))] = 64 * u + lane;
            base += __builtin_popcountll(m);
        }
    }
    const int Q = readfirstlane(meta[kQst + kMaxLocal]);   // work items of the launch
    __syncthreads();                                  // the pair list
    const int q0 = (int)((int64_t)bid * Q / p.nwg), q1 = (int)((int64_t)(bid + 1) * Q / p.nwg);

    // round starting at work item q: the last expert whose first item is
    // <= q holds q (an empty expert shares its first item with the next one)
    auto locate = [&](int q) {
        Round r;
        r.q = q;
        const int4 qs = *(const int4*)(meta + kQst + 4 * lane);
        const int n = __builtin_popcountll(__builtin_amdgcn_ballot_w64(qs.x <= q)) +
                      __builtin_popcountll(__builtin_amdgcn_ballot_w64(qs.y <= q)) +
                      __builtin_popcountll(__builtin_amdgcn_ballot_w64(qs.z <= q)) +
                      __builtin_popcountll(__builtin_amdgcn_ballot_w64(qs.w <= q));
        r.el = readfirstlane(n - 1);
        const int off = q - readfirstlane(meta[kQst + r.el]);
        r.pass = off / p.nrq;
        r.rq = off - r.pass * p.nrq;
        r.seg = q - r.rq;
        r.len = min(min(L, p.nrq - r.rq), q1 - q);
        return r;
    };
    // tokens of a round: how many (at most 4) and where their pairs start in the list
    auto tokens = [&](const Round& r, int& nt, int& pbase) {
        nt = min(4, readfirstlane(meta[kCnt + r.el]) - 4 * r.pass);
        pbase = readfirstlane(meta[kPst + r.el]) + 4 * r.pass;
    };
    // activations of a round's tokens: 16-byte pieces into registers, then LDS
    // (token m's group q at m kXsTok + q kXsPitch)
    uint32_t xr[2][4];
    auto load_x = [&](int nt, int pbase) {
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const int c = tid + u * kT;
            if (c < nt * per_tok) {
                const int m = c / per_tok, cc = c - m * per_tok;
                const int64_t xrow = meta[kList + pbase + m] / p.top_k;
                const u32x4 v = *(const u32x4*)(p.x + xrow * p.K + 8 * cc);
                xr[u][0] = v.x; xr[u][1] = v.y; xr[u][2] = v.z; xr[u][3] = v.w;
            }
        }
    };
    auto store_x = [&](int nt) {
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const int c = tid + u * kT;
            if (c < nt * per_tok) {
                const int m = c / per_tok, cc = c - m * per_tok;
                *(u32x4*)(xs + m * kXsTok + (cc >> 3) * kXsPitch + 16 * (cc & 7)) =
                    u32x4{xr[u][0], xr[u][1], xr[u][2], xr[u][3]};
            }
        }
    };
    // ---- task slot t: row quad tq of round r; lane (b, j) reads row j's
    // group b of the round's expert and its scale (16 aligned bytes at
    // 13 g - sh, as in the dense kernel).  Every slot is loaded, a
    // slot past the round's end with the round's last row quad (a cache
    // hit): a load under a branch would leave the wait counts unknown after
    // it, and the decode of a task would then wait for the next task's bytes.
    // The row quad's first row is uniform (a scalar base address); a lane
    // adds its own 32-bit offset.
    u32x4 C[4][PL];
    uint16_t S[4][PL];
    const uint32_t lane_co = (uint32_t)(kNB * g) - sh, lane_so = 2u * (uint32_t)g;
    auto issue = [&](int t, const Round& r, int tq) {
        const int row0 = 4 * (r.rq + min(tq, r.len - 1));
        const uint32_t jj = (uint32_t)min(j, (int)(p.N - 1 - row0));
        const int64_t e = p.e_begin + r.el;
        const uint32_t co = jj * (uint32_t)rb + lane_co, so = jj * (uint32_t)(2 * p.ng) + lane_so;
#pragma unroll
        for (int pl = 0; pl < PL; ++pl) {
            const uint8_t* cb = p.codes[pl] + (e * p.e_codes + (int64_t)row0 * rb);
            const uint8_t* sb = (const uint8_t*)p.scales[pl] + 2 * (e * p.e_scales + (int64_t)row0 * p.ng);
            C[t][pl] = __builtin_nontemporal_load((const u32x4a*)(cb + co));
            S[t][pl] = *(const uint16_t*)(sb + so);
        }
    };

    if (q0 < q1) {
        Round cur = locate(q0);
        int nt, pbase;
        tokens(cur, nt, pbase);
        // activations first, the first task right behind them: memory
        // counters retire in order, so waiting for x does not wait for it
        load_x(nt, pbase);
        issue(0, cur, rr);
        issue(1, cur, rr + nrr);
        __builtin_amdgcn_sched_barrier(0);
        store_x(nt);
        __syncthreads();

        const uint32_t cofs = (uint32_t)(lane & 31) << 3;    // code-book copy lane % 32
        u32x2 A[16];
        int a_seg = -1;
        for (;;) {
            if (cur.seg != a_seg) {
                a_seg = cur.seg;
                build_a(xs, j, g, nt, A);
            }
            __builtin_amdgcn_s_setprio(3);
            const int qn = cur.q + cur.len;
            const bool more = qn < q1;
            Round nx = cur;
            int nnt = nt, npb = pbase;
            bool restage = false;
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                // the load two tasks ahead goes out before this task is
                // decoded (the next round's first two from t = 2 on; nx is
                // cur after the last round)
                if (t < 2) issue(t + 2, cur, rr + (t + 2) * nrr);
                else issue(t - 2, nx, rr + (t - 2) * nrr);
                const int tq = rr + t * nrr;
                if (active && tq < cur.len)
                    decode_task<PL>(C[t], S[t], A, lut, cofs, sh, lane, red + (tq * nkq + kq) * kTaskStride);
                if (t == 0 && more) {
                    // the next round; its activations go out now when its
                    // tokens differ
                    nx = locate(qn);
                    if (nx.seg != cur.seg) {
                        restage = true;
                        tokens(nx, nnt, npb);
                        load_x(nnt, npb);
                    }
                }
                // a wave that is ahead yields issue priority to those behind,
                // so that the waves reach the barrier together
                yield_after(t);
            }
            __builtin_amdgcn_s_setprio(0);
            __syncthreads();
            if (restage) store_x(nnt);
            const int nrows = (int)min((int64_t)4 * cur.len, p.N - 4 * (int64_t)cur.rq);
            write_rows(red, nkq, nrows, nt, 4 * (int64_t)cur.rq, p.N, p.y, p.y_dtype,
                       [&](int m) { return (int64_t)meta[kList + pbase + m]; });
            if (!more) break;
            __syncthreads();                          // red read, next activations staged
            cur = nx;
            nt = nnt;
            pbase = npb;
        }
    }
    // pairs routed to an id outside [0, n_experts): NaN rows
    if (p.nan_rows && bid == 0) {
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            uint64_t m = bad[u];
            while (m) {
                const int pair = 64 * u + __builtin_ctzll(m);
                m &= m - 1;
                for (int64_t n = tid; n < p.N; n += kT) {
                    const int64_t o = (int64_t)pair * p.N + n;
                    if (p.y_dtype == TQ_F32) ((float*)p.y)[o] = __builtin_nanf("");
                    else ((uint16_t*)p.y)[o] = 0x7fc0u;
                }
            }
        }
    }
}

template <int PL>
__global__ void __launch_bounds__(kT, 1) tq_wave_grouped_kernel(WaveParams p) {
    __shared__ __attribute__((aligned(16))) unsigned char lut[256 * 256];
    __shared__ __attribute__((aligned(16))) unsigned char xs[4 * kXsTok];
    __shared__ __attribute__((aligned(16))) int meta[kMetaInts];
    extern __shared__ __attribute__((aligned(16))) float red[];   // [row quad][slice][kTaskStride]
    grouped_work<PL>(p, lut, xs, meta, red, true);
}

// A hot prefix in one launch: every workgroup takes its share of the hot
// experts (both planes), then of the cold ones (plane 1, and the rows of
// out-of-range ids); the per-row arithmetic is that of the plain grouped
// launches of the same planes.
__global__ void __launch_bounds__(kT, 1) tq_wave_hot_kernel(WaveParams hot, WaveParams cold) {
    __shared__ __attribute__((aligned(16))) unsigned char lut[256 * 256];
    __shared__ __attribute__((aligned(16))) unsigned char xs[4 * kXsTok];
    __shared__ __attribute__((aligned(16))) int meta[kMetaInts];
    extern __shared__ __attribute__((aligned(16))) float red[];
    grouped_work<2>(hot, lut, xs, meta, red, true);
    __syncthreads();                                  // bookkeeping, activations and slices reused
    grouped_work<1>(cold, lut, xs, meta, red, false);
}

}  // namespace

// Parameters of a call in the wave form's domain: dense calls with
// 1 <= M <= 4, grouped calls with at most 256 (token, slot) pairs and 256
// experts in the launch; G = 64, K a multiple of 1024 up to 4096, x 16-byte,
// codes 4-byte and scales 2-byte aligned.  False outside that domain.
static bool wave_setup(const TqMatmulArgs& a, WaveParams& p, size_t& smem) {
    const bool grouped = a.n_experts > 0;
    if (a.G != 64 || a.M < 1 || a.N < 1) return false;
    if (a.K < 1024 || a.K > 4096 || a.K % 1024 != 0) return false;
    if (((uintptr_t)a.x & 15) != 0) return false;
    for (int pl = 0; pl < a.planes; ++pl)
        if (((uintptr_t)a.codes[pl] & 3) != 0 || ((uintptr_t)a.scales[pl] & 1) != 0) return false;
    const int64_t nrq = (a.N + 3) / 4;
    const int64_t total = grouped ? a.M * a.top_k : 0;
    const int nl = grouped ? a.e_end - a.e_begin : 1;
    if (grouped) {
        if (total > 256 || nl < 0 || nl > kMaxLocal || ((uintptr_t)a.ids & 3) != 0) return false;
        // work items: row quads over every pass, sum of ceil(count / 4) <= total / 4 + nl
        if (nrq * (total / 4 + nl + 1) >= (1ll << 31)) return false;
    } else {
        if (a.M > 4 || nrq >= (1ll << 31)) return false;
    }
    const int ng = (int)(a.K / 64);
    const int nkq = ng / 16, nrr = kW / nkq;
    const int cus = compute_unit_count();
    p.x = a.x;
    p.K = a.K;
    p.N = a.N;
    p.ng = ng;
    p.M = (int)a.M;
    p.codes[0] = a.codes[0];
    p.codes[1] = a.planes == 2 ? a.codes[1] : a.codes[0];
    p.scales[0] = a.scales[0];
    p.scales[1] = a.planes == 2 ? a.scales[1] : a.scales[0];
    p.nrq = (int)nrq;
    p.nwg = cus;
    // dense: ceil(N / compute units) rows a workgroup (whole row quads), at
    // most four tasks a wave
    int64_t rpw = (a.N + cus - 1) / cus;
    rpw = (rpw + 3) & ~(int64_t)3;
    if (rpw > 4 * kMaxTasks * nrr) rpw = 4 * kMaxTasks * nrr;
    p.rows_per_wg = (int)rpw;
    if (!grouped && (a.N + rpw - 1) / rpw >= (1ll << 31)) return false;
    p.y = a.y;
    p.y_dtype = a.y_dtype;
    p.ids = a.ids;
    p.total = (int)total;
    p.top_k = a.top_k;
    p.n_experts = a.n_experts;
    p.e_begin = grouped ? a.e_begin : 0;
    p.nl = nl;
    p.nan_rows = grouped && a.nan_rows ? 1 : 0;
    p.e_codes = a.N * ng * kNB;
    p.e_scales = a.N * ng;
    smem = (size_t)4 * nrr * nkq * kTaskStride * sizeof(float);
    return true;
}

bool launch_tq_wave(const TqMatmulArgs& a, hipStream_t s, hipError_t* err) {
    WaveParams p;
    size_t smem;
    if (!wave_setup(a, p, smem)) return false;
    const dim3 block(kT);
    if (a.n_experts > 0) {
        const dim3 grid((unsigned)p.nwg);
        if (a.planes == 2) hipLaunchKernelGGL(tq_wave_grouped_kernel<2>, grid, block, smem, s, p);
        else hipLaunchKernelGGL(tq_wave_grouped_kernel<1>, grid, block, smem, s, p);
    } else {
        const dim3 grid((unsigned)((a.N + p.rows_per_wg - 1) / p.rows_per_wg));
        if (a.planes == 2) hipLaunchKernelGGL(tq_wave_dense_kernel<2>, grid, block, smem, s, p);
        else hipLaunchKernelGGL(tq_wave_dense_kernel<1>, grid, block, smem, s, p);
    }
    *err = hipGetLastError();
    return true;
}

bool launch_tq_wave_hot(const TqMatmulArgs& hot, const TqMatmulArgs& cold, hipStream_t s,
                        hipError_t* err) {
    if (hot.n_experts < 1 || cold.n_experts < 1) return false;
    if (hot.planes != 2 || cold.planes != 1 || hot.nan_rows || !cold.nan_rows) return false;
    WaveParams ph, pc;
    size_t smh, smc;
    if (!wave_setup(hot, ph, smh) || !wave_setup(cold, pc, smc)) return false;
    hipLaunchKernelGGL(tq_wave_hot_kernel, dim3((unsigned)ph.nwg), dim3(kT), smh > smc ? smh : smc, s,
                       ph, pc);
    *err = hipGetLastError();
    return true;
}

}  // namespace dmm
