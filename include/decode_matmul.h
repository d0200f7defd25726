/*
 * decode_matmul.h -- C ABI of the packed ternary-code matmul library for
 * AMD MI355X (gfx950).
 *
 * Two weight formats, both decoded inside the matmul kernels (no bf16 copy of
 * the weight matrix is ever written):
 *
 *  1. Mean-abs ternary ("Does your weight format deserve a kernel?",
 *     pack-unpack-run, sections "Three values and a shared scale", "Five
 *     trits in a byte", "Count the bytes you actually wrote"): a group of G
 *     consecutive weights of a row shares s = fp16(mean |W|); each weight is
 *     t = clip(round(W/s), -1, 1); five trits per byte, b = sum_q (t_q+1) 3^q,
 *     first trit least significant; ceil(G/5) code bytes per group.
 *     Optionally a second plane quantizes the residual of the first
 *     (FUCINA README, "The method": W ~ d1 T1 + d2 T2).
 *
 *  2. Route B code book ("A Discrete Weight Language for Large Language
 *     Models", sections 3.2, 3.3, 4.1, 4.2): one byte per weight indexes a
 *     243-entry table of 5-step ternary ladder values, times one fp32 scale
 *     per layer and an optional fp16 scale per output row.
 *
 * Conventions for every entry point:
 *  - Pointers named d_* or documented "device" are device pointers owned by
 *    the caller; the library keeps no global state and allocates no memory.
 *  - `stream` is a hipStream_t (NULL = the legacy default stream).  Work is
 *    enqueued asynchronously on it; the return value is a host-side
 *    tq_status, decided before anything is enqueued (argument errors never
 *    launch a kernel).  TQ_ERR_HIP means a launch was rejected by the runtime.
 *  - Data errors that only the device can see are OR-ed into the caller's
 *    int32 *d_status as TQ_DATA_* flags.  The call first sets *d_status to 0
 *    (with a kernel on `stream`, not a memset); read it after synchronizing.
 *  - Matrices are dense and row-major.  The packed layout of a [rows, K]
 *    matrix at group size G is planar:
 *        codes  uint8  [rows][ceil(K/G)][ceil(G/5)]
 *        scales fp16   [rows][ceil(K/G)]        (IEEE binary16 bit patterns)
 *    A ragged final group (K % G != 0) has K - (ceil(K/G)-1) G members and
 *    still occupies ceil(G/5) bytes; its unused trit slots are padding.
 *  - bf16 values are passed as uint16 bit patterns.
 *  - Calls that overlap on one stream are ordered; calls on different
 *    streams that write the same buffers race, as usual.
 */
#ifndef DECODE_MATMUL_H
#define DECODE_MATMUL_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Host-side status codes (return values). */
enum tq_status {
    TQ_OK = 0,
    TQ_ERR_NULL = 1,         /* a required pointer is NULL                     */
    TQ_ERR_SHAPE = 2,        /* a size is negative, inconsistent or too large  */
    TQ_ERR_UNSUPPORTED = 3,  /* G not in {64, 128}, planes not in {1, 2}, ...   */
    TQ_ERR_DTYPE = 4,        /* unknown output dtype                           */
    TQ_ERR_ALIGN = 5,        /* a pointer is not aligned as documented         */
    TQ_ERR_HIP = 6,          /* the HIP runtime rejected a launch              */
    TQ_ERR_SCRATCH = 7       /* the call needs more than the library's static
                                scratch (DMM_SCRATCH_BYTES) holds               */
};

/* Bytes of the device scratch array that rb_matmul_noalloc uses in place of a
   workspace; each GPU the library runs on holds one until the process ends. */
#define DMM_SCRATCH_BYTES ((int64_t)34 << 20)

/* Device-side data-error flags, OR-ed into *d_status. */
enum tq_data_flag {
    TQ_DATA_RANGE = 1,       /* non-finite weight, or group scale overflows fp16 */
    TQ_DATA_CODE = 2,        /* byte value 243..255 in a ternary package or as a
                                Route B code                                     */
    TQ_DATA_PADDING = 4,     /* a padding trit slot does not decode to zero      */
    TQ_DATA_ALPHABET = 8     /* more than 128 distinct Route B codes (rb_truncate) */
};

/* Element types of outputs. */
enum tq_dtype { TQ_F32 = 0, TQ_BF16 = 1 };

/*
 * tq_pack -- quantize and pack W (pack-unpack-run, "Three values and a
 * shared scale" and "Five trits in a byte").
 *
 *  W        device fp32 [rows, K], row-major, 4-byte aligned.
 *  G        group size, 64 or 128.
 *  planes   1 or 2.  Plane 2 quantizes R = fl32(W - s1 t1) with the same
 *           rule (FUCINA README, "The method").
 *  codes1, scales1   device outputs of plane 1 (layout above); scales 2-byte
 *           aligned; codes any alignment.
 *  codes2, scales2   outputs of plane 2; must be NULL when planes == 1.
 *  d_status device int32; receives TQ_DATA_RANGE if a weight is not finite or
 *           a group mean rounds to fp16 infinity.  Such a group is written as
 *           scale 0 and all-zero trits.
 *
 * Per group of n members: S = sum |W_j| in float64, j ascending; mean =
 * S / n in float64; s = fp16 nearest-even of mean (one rounding);
 * t_j = sign(W_j) if s > 0 and |W_j| > s/2, else 0 (the exact form of
 * clip(round(W_j/s), -1, 1) with ties to even).  Bit-exact and
 * deterministic.
 */
int tq_pack(const float* W, int64_t rows, int64_t K, int32_t G, int32_t planes,
            uint8_t* codes1, uint16_t* scales1, uint8_t* codes2, uint16_t* scales2,
            int32_t* d_status, void* stream);

/*
 * tq_unpack -- decode a package to weights (pack-unpack-run, "Five trits in
 * a byte": the format rejects bytes 243..255 and padding must decode to 0).
 *
 *  codes, scales  device package of a [rows, K] matrix at group size G.
 *  W_out          device [rows, K] of out_dtype: TQ_F32 gives s*t exactly,
 *                 TQ_BF16 gives bf16 nearest-even of s*t.  4-byte aligned
 *                 for fp32, 2-byte for bf16.
 *  d_status       device int32; TQ_DATA_CODE / TQ_DATA_PADDING flags.  An
 *                 invalid byte decodes as five zero trits.
 */
int tq_unpack(const uint8_t* codes, const uint16_t* scales, int64_t rows, int64_t K,
              int32_t G, void* W_out, int32_t out_dtype, int32_t* d_status, void* stream);

/*
 * tq_matmul -- y = x W_hat^T over a ternary package, decoded in-kernel
 * (pack-unpack-run, "What survives the round trip?": the runtime decodes
 * small pieces inside the matrix multiplication; FUCINA README, "Runtime
 * requirements": second-plane outputs are summed with the first, and the
 * expert matmul selects each token's experts).
 *
 *  x          device bf16 [M, K] (M tokens), 2-byte aligned: any element
 *             offset is accepted (the fastest forms need 16-byte aligned rows).
 *  codes1, scales1   plane 1.  Dense: one [N, K] package.  Grouped:
 *             n_experts packages back to back, [n_experts][N][K/G][...].
 *  codes2, scales2   optional plane 2 with the same layout (NULL = 1 plane);
 *             W_hat = s1 T1 + s2 T2.
 *  G          64 or 128; K % G must be 0.
 *  n_experts  0 = dense: y is [M, N].  > 0 = grouped: expert_ids is device
 *             int32 [M, top_k] and y is [M, top_k, N] with
 *             y[t, j] = x[t] W_hat_{expert_ids[t, j]}^T.  A (t, j) whose id
 *             is outside [0, n_experts) gets a row of NaN.
 *  y          device output of y_dtype (fp32, or bf16 nearest-even of the
 *             fp32 result).
 *
 * Accuracy: fp32 accumulation of exact trit-times-activation products, one
 * fp32 multiply by the group scale per group; |y - y_ref| <= 2e-3 sum_k
 * |x_k w_hat_k| against a float64 reference.  Bytes are not validated here
 * (an invalid byte contributes an unspecified but finite value; memory
 * accesses stay in bounds).  M = 0 or N = 0 is a no-op; with K = 0, x and
 * the package may be NULL and y is written with zeros.
 */
int tq_matmul(const uint16_t* x, int64_t M, int64_t K,
              const uint8_t* codes1, const uint16_t* scales1,
              const uint8_t* codes2, const uint16_t* scales2,
              int64_t N, int32_t G, int32_t n_experts, const int32_t* expert_ids,
              int32_t top_k, void* y, int32_t y_dtype, void* stream);

/*
 * tq_prefill_workspace_bytes -- bytes of the workspace tq_matmul_ws uses for
 * an [M, K] activation matrix: an fp16 copy of x, then one flag word per
 * 128-row block and group of 64 columns.  -1 for negative or too large sizes.
 */
int64_t tq_prefill_workspace_bytes(int64_t M, int64_t K);

/*
 * tq_matmul_ws -- dense tq_matmul (n_experts = 0) with a caller-provided
 * workspace that lets the prefill (M >= 128, G = 64) convert the activations
 * once per call.
 *
 * The computation and the accuracy are those of tq_matmul (pack-unpack-run,
 * "Three values and a shared scale": W_hat = s * t per group; FUCINA README,
 * "The method", for two planes).  The prefill multiplies in fp16, and
 * activations are exact in fp16 unless they fall outside [2^-17, 65280] in
 * magnitude; such chunks are replayed in bf16.  Without a workspace, every
 * N-tile workgroup converts its activation tile itself, once per plane.
 * With one, a first kernel converts x once and flags the groups holding
 * chunks fp16 cannot hold.  The output is bit for bit that of tq_matmul.
 *
 *  workspace        device memory of at least tq_prefill_workspace_bytes(M,
 *                   K) bytes, 256-byte aligned (TQ_ERR_ALIGN), owned by the
 *                   caller.  Its contents on entry do not matter, and it is
 *                   overwritten.  NULL makes the call tq_matmul.
 *  workspace_bytes  its size; smaller than required gives TQ_ERR_SHAPE.
 *
 * The workspace is used only when the call takes the prefill kernel; otherwise
 * it is ignored.  Calls that share a workspace must not overlap in time.
 * Every other argument and error is that of tq_matmul.
 */
int tq_matmul_ws(const uint16_t* x, int64_t M, int64_t K, const uint8_t* codes1,
                 const uint16_t* scales1, const uint8_t* codes2, const uint16_t* scales2,
                 int64_t N, int32_t G, void* y, int32_t y_dtype, void* workspace,
                 int64_t workspace_bytes, void* stream);

/*
 * tq_matmul_hot -- grouped two-plane experts with a hot prefix (FUCINA
 * README, "The method": hot experts get both planes and cold experts one,
 * and experts are stored hot-first so that the second plane covers the
 * expert prefix 0 .. n_hot - 1; "Runtime requirements": the second-plane
 * tensors hold their own expert count):
 *
 *     y[t, j, :] = x[t] (s1 T1_e + [e < n_hot] s2 T2_e)^T,  e = expert_ids[t, j]
 *
 *  codes1, scales1  plane 1 of all n_experts experts, as in tq_matmul.
 *  codes2, scales2  plane 2 of experts 0 .. n_hot - 1 only (same per-expert
 *                   layout), NULL when n_hot = 0.
 *  n_hot            0 <= n_hot <= n_experts; the count is an argument, never
 *                   inferred from the buffers.
 *
 * Grouped calls only (n_experts >= 1, else TQ_ERR_UNSUPPORTED); every other
 * argument, the invalid-id NaN rows and the accuracy are those of tq_matmul
 * (n_hot = n_experts is its two-plane call, n_hot = 0 its one-plane call).
 */
int tq_matmul_hot(const uint16_t* x, int64_t M, int64_t K,
                  const uint8_t* codes1, const uint16_t* scales1,
                  const uint8_t* codes2, const uint16_t* scales2, int32_t n_hot,
                  int64_t N, int32_t G, int32_t n_experts, const int32_t* expert_ids,
                  int32_t top_k, void* y, int32_t y_dtype, void* stream);

/*
 * rb_table -- build the 243-entry Route B code book on the host (Route B
 * paper, section 3.2: the 3^5 words of a 5-step ternary ladder are
 * enumerated once per layer).
 *
 *  ladder     host fp32 [5], a_1..a_5.
 *  table_out  host fp32 [243]; entry b is sum_i c_i a_i for the word
 *             (c_1..c_5) whose base-3 encoding sum_i (c_i+1) 3^(5-i) is b
 *             (c_1 most significant), summed in float64 for i = 1..5 and
 *             rounded once to fp32.
 *
 * The per-layer scale alpha is not folded in; rb_matmul takes it separately.
 */
int rb_table(const float* ladder, float* table_out);

/*
 * rb_encode -- the Route B encoder on the device (Route B paper, section 3.1:
 * the greedy 5-step ternary word of r_0 = x / scale, each step taking the c
 * in {-1, 0, +1} nearest to the residual, with a zero-bias zeta that keeps
 * c_i = 0 while |r_{i-1}| < zeta * s_i; section 3.2: codes are the base-3
 * encoding of c_1..c_5; section 3.3: the per-row scale; section 8.2: one
 * scale per attention head, i.e. per block of consecutive rows).
 *
 *  W          device fp32 [N, K] row-major, 4-byte aligned.
 *  ladder     host fp32 [5], s_1..s_5 (finite, >= 0; the pages' ladders are
 *             positive).
 *  zeta       zero-bias in [0, 1] (0: the plain greedy word).
 *  rho_rows   0: r_0 = W / alpha with alpha = max |W| over the matrix;
 *             b >= 1: rows are taken in blocks h of b consecutive rows (the
 *             last one may be shorter), r_0 = W[n, k] / alpha_h with
 *             alpha_h the block's largest |W| (b = 1: per row; b = head_dim:
 *             per attention head).
 *  codes      device uint8 [N, K]: sum_i (c_i + 1) 3^(5-i) (c_1 most
 *             significant, the order rb_table enumerates).
 *  alpha_out  device fp32 [1] when rho_rows = 0, else [1 + ceil(N / b)]:
 *             alpha = max |W| (0 for an empty or all-zero W), then alpha_h.
 *  row_scale  device fp16 [ceil(N / b)] when rho_rows > 0 (rho_h =
 *             fp16(alpha_h / alpha), 0 when alpha = 0), else NULL.
 *  d_status   device int32; set to 0, then TQ_DATA_RANGE if a weight is not
 *             finite (the outputs are then unspecified, memory stays in bounds).
 *
 * Decisions are taken on IEEE float64 values: r_0 is one float64 division of
 * the fp32 weight by the fp32 scale, each residual one float64 subtraction,
 * ties of the argmin go to c = 0, and rho_h is the float64 quotient rounded
 * once to fp16.  A zero scale gives the all-zero word (code 121).  Then
 * rb_matmul_rho_block(x, codes, rb_table(ladder), alpha, row_scale, b)
 * applies W_hat[n, k] = rho_{n / b} * alpha * sum_i c_i s_i.  One call reads
 * W twice and allocates nothing.
 */
int rb_encode(const float* W, int64_t N, int64_t K, const float* ladder, float zeta,
              int32_t rho_rows, uint8_t* codes, float* alpha_out, uint16_t* row_scale,
              int32_t* d_status, void* stream);

/*
 * rb_matmul -- Route B matmul (Route B paper, sections 3.3 and 4.2: each code
 * byte is looked up in the code book inside the GEMM, and the row's scale
 * multiplies the finished sum, with the bias added last):
 *
 *     y[m, n] = alpha * rho_n * sum_k x[m, k] * table[codes[n, k]]  (+ bias[n])
 *
 *  x          device bf16 [M, K] (fastest when 4-byte aligned with K even).
 *  codes      device uint8 [N, K] (one code per weight), any alignment.
 *  table      device fp32 [243] (e.g. from rb_table), 4-byte aligned.
 *  alpha      per-layer fp32 scale.
 *  row_scale  device fp16 [N] (rho_n) or NULL (rho = 1).
 *  bias       device fp32 [N] or NULL.
 *  y          device [M, N] of y_dtype.
 *
 * M <= 16 runs a GEMV kernel that keeps each weight as an exact split of the
 * table value into two bf16 terms (error < 2^-16 per term); M > 16 runs an
 * MFMA kernel that multiplies in fp16 against the code book scaled by a power
 * of two (error <= 2^-11 per term), with activations converted to fp16
 * exactly and any 8-value chunk fp16 cannot hold replayed on bf16 MFMAs
 * against the two-term bf16 split.  Both accumulate in fp32.  Codes 243..255 read a zero
 * table entry.  M = 0 or N = 0 is a no-op; with K = 0, x and codes may be
 * NULL and y = bias (or 0).
 */
int rb_matmul(const uint16_t* x, int64_t M, int64_t K, const uint8_t* codes, int64_t N,
              const float* table, float alpha, const uint16_t* row_scale,
              const float* bias, void* y, int32_t y_dtype, void* stream);

/*
 * rb_matmul_rho_block -- rb_matmul with one row scale per block of rho_rows
 * consecutive rows (Route B paper, section 8.2: per-head prosody, one rho
 * per attention head whose rows share it; section 3.3's per-row scale is
 * rho_rows = 1):
 *
 *     y[m, n] = alpha * rho_{n / rho_rows} * sum_k x[m, k] * table[codes[n, k]]  (+ bias[n])
 *
 *  row_scale  device fp16 [ceil(N / rho_rows)] or NULL (rho = 1).
 *  rho_rows   >= 1 (TQ_ERR_SHAPE otherwise).
 *
 * Every other argument, the kernels and the accuracy are those of rb_matmul
 * (which is this call with rho_rows = 1).
 */
int rb_matmul_rho_block(const uint16_t* x, int64_t M, int64_t K, const uint8_t* codes, int64_t N,
                        const float* table, float alpha, const uint16_t* row_scale,
                        int32_t rho_rows, const float* bias, void* y, int32_t y_dtype,
                        void* stream);

/*
 * rb_matmul_blocks -- Route B matmul with one code book per block of rows
 * (Route B paper, section 8.3, adaptive alphabets: one ladder per group of 32
 * rows instead of one per layer family):
 *
 *     y[m, n] = alpha * rho_{n / rho_rows} * sum_k x[m, k] * tables[n / table_rows][codes[n, k]]
 *               (+ bias[n])
 *
 *  tables      device fp32 [ceil(N / table_rows)][243], 4-byte aligned; book
 *              h serves rows h * table_rows .. (h + 1) * table_rows - 1 (e.g.
 *              rb_table of block h's ladder).
 *  table_rows  a positive multiple of 32, or 0 for one book of 243 entries
 *              (TQ_ERR_UNSUPPORTED for other values, TQ_ERR_SHAPE if
 *              negative).
 *
 * Every other argument, the kernels and the accuracy are those of
 * rb_matmul_rho_block (which is this call with table_rows = 0).
 */
int rb_matmul_blocks(const uint16_t* x, int64_t M, int64_t K, const uint8_t* codes, int64_t N,
                     const float* tables, int32_t table_rows, float alpha,
                     const uint16_t* row_scale, int32_t rho_rows, const float* bias, void* y,
                     int32_t y_dtype, void* stream);

/*
 * rb_prefill_workspace_bytes -- bytes of the workspace rb_matmul_ws uses for
 * an [M, K] activation matrix: an fp16 copy of x, then one flag word per
 * 256-row block and 32-wide K-slice.  -1 for negative or too large sizes.
 */
int64_t rb_prefill_workspace_bytes(int64_t M, int64_t K);

/*
 * rb_matmul_ws -- rb_matmul_blocks with a caller-provided workspace that lets
 * the prefill (M > 16) convert the activations once per call.
 *
 * The computation and the accuracy are those of rb_matmul_blocks (Route B
 * paper, sections 3.2 and 3.3: y = alpha * rho_n * sum_k x[m, k] T[codes[n, k]]
 * + bias_n; section 8.3 for several code books).  The prefill multiplies in
 * fp16, and activations are exact in fp16 unless they fall outside
 * [2^-17, 65280] in magnitude; such chunks are replayed in bf16.  Without a
 * workspace, every N-tile workgroup converts its activation tile itself.
 * With one, a first kernel converts x once and flags the K-slices holding
 * chunks fp16 cannot hold, and the matmul reads the fp16 copy.
 *
 *  workspace        device memory of at least rb_prefill_workspace_bytes(M,
 *                   K) bytes, 256-byte aligned (TQ_ERR_ALIGN), owned by the
 *                   caller.  Its contents on entry do not matter, and it is
 *                   overwritten.  NULL makes the call rb_matmul_blocks.
 *  workspace_bytes  its size; smaller than required gives TQ_ERR_SHAPE.
 *
 * The workspace is used only by the prefill with 16-byte aligned x, 16-byte
 * aligned codes and K % 32 == 0; otherwise it is ignored.  Calls that share a
 * workspace must not overlap in time.  Every other argument and error is
 * that of rb_matmul_blocks.
 */
int rb_matmul_ws(const uint16_t* x, int64_t M, int64_t K, const uint8_t* codes, int64_t N,
                 const float* tables, int32_t table_rows, float alpha, const uint16_t* row_scale,
                 int32_t rho_rows, const float* bias, void* y, int32_t y_dtype, void* workspace,
                 int64_t workspace_bytes, void* stream);

/*
 * rb_matmul_noalloc -- rb_matmul_ws for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc): the workspace is the library's own static device array
 * of DMM_SCRATCH_BYTES, one per GPU, instead of caller memory.
 *
 * Arguments, computation, accuracy and output are those of rb_matmul_ws
 * without its workspace arguments; the output is bit for bit that of
 * rb_matmul_ws.  The call allocates nothing (no hipMalloc, no allocating
 * library routine).
 *
 *  - M > 16 with rb_prefill_workspace_bytes(M, K) > DMM_SCRATCH_BYTES gives
 *    TQ_ERR_SCRATCH before any launch (M = 2048 at K = 8192 fits).
 *  - The scratch of the calling thread's current device is used: `stream`
 *    must belong to that device.
 *  - Every call on a GPU shares that GPU's array and overwrites it; calls
 *    that overlap in time on one GPU (two streams, two threads) race.
 *    The array's contents on entry do not matter.
 *  - The array's device address is looked up on the first call on each
 *    device; TQ_ERR_HIP if the lookup fails.
 */
int rb_matmul_noalloc(const uint16_t* x, int64_t M, int64_t K, const uint8_t* codes, int64_t N,
                      const float* tables, int32_t table_rows, float alpha,
                      const uint16_t* row_scale, int32_t rho_rows, const float* bias, void* y,
                      int32_t y_dtype, void* stream);

/*
 * rb_truncate -- the 7-bit truncated alphabet (Route B paper, section 8.1: a
 * layer that uses at most 128 of the 243 codes stores each weight in 7 bits,
 * plus a table from the 7-bit index to the code).
 *
 *  codes       device uint8 [N, K] Route B code bytes, any alignment.
 *  used_out    device uint8 [128], 4-byte aligned: the codes present, in
 *              increasing order, then code 121 (the all-zero word) up to 128
 *              entries.  Index j stands for used_out[j].
 *  n_used_out  device int32: the number of distinct codes 0..242 present.
 *  codes7      device uint8 [N][ceil(7 K / 8)]: bit q of the index of weight
 *              (n, k) is bit 7 k + q of row n read as a little-endian bit
 *              string (bit p in byte p / 8, position p % 8); the bits past
 *              7 K are zero.
 *  d_status    device int32; set to 0, then TQ_DATA_CODE for a byte
 *              243..255 and TQ_DATA_ALPHABET for more than 128 distinct codes
 *              (codes7 is then unspecified; memory stays in bounds).
 *
 * Four launches on `stream`: the first 32 bytes of used_out serve as a
 * presence set until the list is written.  codes is read twice.
 */
int rb_truncate(const uint8_t* codes, int64_t N, int64_t K, uint8_t* used_out,
                int32_t* n_used_out, uint8_t* codes7, int32_t* d_status, void* stream);

/*
 * rb_matmul7 -- Route B matmul over 7-bit indices (Route B paper, section
 * 8.1, with the per-block books of section 8.3):
 *
 *     y[m, n] = alpha * rho_{n / rho_rows} * sum_k x[m, k] *
 *               tables[n / table_rows][used[index(n, k)]]  (+ bias[n])
 *
 *  codes7      device uint8 [N][ceil(7 K / 8)] in rb_truncate's layout
 *              (fastest with K % 512 == 0 and a 16-byte aligned pointer at
 *              M <= 16, K % 32 == 0 and a 4-byte aligned pointer above).
 *  used        device uint8 [128]: index -> code; codes 243..255 read zero.
 *  tables, table_rows, alpha, row_scale, rho_rows, bias, y, y_dtype, stream
 *              as in rb_matmul_blocks.
 *
 * M <= 16 runs a GEMV kernel with the two-term bf16 split of each book entry
 * (K % 512 == 0 with 16-byte aligned indices and 4-byte aligned activations;
 * a plain fp32 kernel otherwise); M > 16 runs the fp16 MFMA kernel of rb_matmul with its
 * bf16 replay.  The accuracy is that of rb_matmul.
 */
int rb_matmul7(const uint16_t* x, int64_t M, int64_t K, const uint8_t* codes7, int64_t N,
               const uint8_t* used, const float* tables, int32_t table_rows, float alpha,
               const uint16_t* row_scale, int32_t rho_rows, const float* bias, void* y,
               int32_t y_dtype, void* stream);

/* Human-readable name of a tq_status value. */
const char* tq_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* DECODE_MATMUL_H */
