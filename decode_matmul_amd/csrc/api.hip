// extern "C" entry points: argument validation on the host, then launches on
// the caller's stream.  No memory is allocated and no state is kept.
#include <stddef.h>

#include "common.h"

namespace {

constexpr int64_t kMaxDim = (int64_t)1 << 31;

bool aligned(const void* p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) == 0; }

bool group_ok(int G) { return G == 64 || G == 128; }

int hip_status(hipError_t e) { return e == hipSuccess ? TQ_OK : TQ_ERR_HIP; }

}  // namespace

extern "C" {

const char* tq_status_string(int status) {
    switch (status) {
        case TQ_OK: return "ok";
        case TQ_ERR_NULL: return "a required pointer is NULL";
        case TQ_ERR_SHAPE: return "a size is negative, inconsistent or too large";
        case TQ_ERR_UNSUPPORTED: return "unsupported group size, plane count or mode";
        case TQ_ERR_DTYPE: return "unknown dtype";
        case TQ_ERR_ALIGN: return "a pointer is not aligned as documented";
        case TQ_ERR_HIP: return "the HIP runtime rejected a launch";
        case TQ_ERR_SCRATCH:
            return "the call needs more device scratch than DMM_SCRATCH_BYTES (34 MiB)";
        default: return "unknown status";
    }
}

int tq_pack(const float* W, int64_t rows, int64_t K, int32_t G, int32_t planes,
            uint8_t* codes1, uint16_t* scales1, uint8_t* codes2, uint16_t* scales2,
            int32_t* d_status, void* stream) {
    if (!W || !codes1 || !scales1 || !d_status) return TQ_ERR_NULL;
    if (rows < 0 || K < 0 || rows >= kMaxDim || K >= kMaxDim) return TQ_ERR_SHAPE;
    if (!group_ok(G) || (planes != 1 && planes != 2)) return TQ_ERR_UNSUPPORTED;
    if (planes == 2 && (!codes2 || !scales2)) return TQ_ERR_NULL;
    if (planes == 1 && (codes2 || scales2)) return TQ_ERR_SHAPE;
    if (!aligned(W, 4) || !aligned(scales1, 2) || (scales2 && !aligned(scales2, 2)) ||
        !aligned(d_status, 4))
        return TQ_ERR_ALIGN;
    const int64_t groups = rows * ((K + G - 1) / G);
    if (groups / 128 >= kMaxDim) return TQ_ERR_SHAPE;   // grid: 128 or 256 groups a workgroup
    hipStream_t s = (hipStream_t)stream;
    hipError_t e = dmm::launch_status_clear(d_status, s);
    if (e != hipSuccess) return TQ_ERR_HIP;
    return hip_status(dmm::launch_pack(W, rows, K, G, planes, codes1, scales1, codes2, scales2,
                                       d_status, s));
}

int rb_encode(const float* W, int64_t N, int64_t K, const float* ladder, float zeta,
              int32_t rho_rows, uint8_t* codes, float* alpha_out, uint16_t* row_scale,
              int32_t* d_status, void* stream) {
    if (!ladder || !alpha_out || !d_status) return TQ_ERR_NULL;
    if (N < 0 || K < 0 || N >= kMaxDim || K >= kMaxDim) return TQ_ERR_SHAPE;
    if (rho_rows < 0) return TQ_ERR_SHAPE;
    if (!(zeta >= 0.f && zeta <= 1.f)) return TQ_ERR_UNSUPPORTED;
    for (int i = 0; i < 5; ++i)                       // finite, nonnegative steps
        if (!(ladder[i] >= 0.f && ladder[i] <= 3.402823466e38f)) return TQ_ERR_UNSUPPORTED;
    if (N > 0 && K > 0 && (!W || !codes)) return TQ_ERR_NULL;
    if (rho_rows > 0 && N > 0 && !row_scale) return TQ_ERR_NULL;
    if (rho_rows == 0 && row_scale) return TQ_ERR_SHAPE;
    if ((W && !aligned(W, 4)) || !aligned(alpha_out, 4) || (row_scale && !aligned(row_scale, 2)) ||
        !aligned(d_status, 4))
        return TQ_ERR_ALIGN;
    return hip_status(dmm::launch_rb_encode(W, N, K, ladder, zeta, rho_rows, codes, alpha_out,
                                            row_scale, d_status, (hipStream_t)stream));
}

int tq_unpack(const uint8_t* codes, const uint16_t* scales, int64_t rows, int64_t K,
              int32_t G, void* W_out, int32_t out_dtype, int32_t* d_status, void* stream) {
    if (!codes || !scales || !W_out || !d_status) return TQ_ERR_NULL;
    if (rows < 0 || K < 0 || rows >= kMaxDim || K >= kMaxDim) return TQ_ERR_SHAPE;
    if (!group_ok(G)) return TQ_ERR_UNSUPPORTED;
    if (out_dtype != TQ_F32 && out_dtype != TQ_BF16) return TQ_ERR_DTYPE;
    if (!aligned(scales, 2) || !aligned(W_out, out_dtype == TQ_F32 ? 4 : 2) ||
        !aligned(d_status, 4))
        return TQ_ERR_ALIGN;
    const int64_t groups = rows * ((K + G - 1) / G);
    if (groups / 128 >= kMaxDim) return TQ_ERR_SHAPE;   // grid: 128 or 256 groups a workgroup
    hipStream_t s = (hipStream_t)stream;
    hipError_t e = dmm::launch_status_clear(d_status, s);
    if (e != hipSuccess) return TQ_ERR_HIP;
    return hip_status(dmm::launch_unpack(codes, scales, rows, K, G, W_out, out_dtype, d_status, s));
}

// tq_matmul and tq_matmul_hot: n_hot < 0 gives every expert the planes
// passed; 0 <= n_hot <= n_experts gives plane 2 to experts 0 .. n_hot - 1.
static int tq_matmul_common(const uint16_t* x, int64_t M, int64_t K, const uint8_t* codes1,
                            const uint16_t* scales1, const uint8_t* codes2,
                            const uint16_t* scales2, int32_t n_hot, int64_t N, int32_t G,
                            int32_t n_experts, const int32_t* expert_ids, int32_t top_k, void* y,
                            int32_t y_dtype, void* stream, void* workspace = nullptr,
                            int64_t workspace_bytes = 0) {
    if (M < 0 || K < 0 || N < 0 || M >= kMaxDim || K >= kMaxDim || N >= kMaxDim)
        return TQ_ERR_SHAPE;
    if (!group_ok(G)) return TQ_ERR_UNSUPPORTED;
    if (K % G != 0) return TQ_ERR_SHAPE;
    if (y_dtype != TQ_F32 && y_dtype != TQ_BF16) return TQ_ERR_DTYPE;
    if (n_experts < 0) return TQ_ERR_SHAPE;
    if ((codes2 == nullptr) != (scales2 == nullptr)) return TQ_ERR_NULL;
    if (n_experts > 0) {
        if (top_k < 1) return TQ_ERR_SHAPE;
        if (M * (int64_t)top_k > dmm::tq_max_grouped_pairs()) return TQ_ERR_SHAPE;
    }
    if (M == 0 || N == 0) return TQ_OK;
    if (!y || (K > 0 && (!x || !codes1 || !scales1))) return TQ_ERR_NULL;
    if (n_experts > 0 && !expert_ids) return TQ_ERR_NULL;
    if (!aligned(x, 2) || !aligned(scales1, 2) || (scales2 && !aligned(scales2, 2)) ||
        !aligned(y, y_dtype == TQ_F32 ? 4 : 2) || (expert_ids && !aligned(expert_ids, 4)))
        return TQ_ERR_ALIGN;
    const int64_t row_blocks = (N + 15) / 16;
    if (row_blocks * (n_experts > 0 ? n_experts : 1) >= kMaxDim) return TQ_ERR_SHAPE;
    dmm::TqMatmulArgs a;
    a.x = x;
    a.M = M;
    a.K = K;
    a.N = N;
    a.codes[0] = codes1;
    a.codes[1] = codes2;
    a.scales[0] = scales1;
    a.scales[1] = scales2;
    a.planes = codes2 ? 2 : 1;
    a.G = G;
    a.n_experts = n_experts;
    a.ids = n_experts > 0 ? expert_ids : nullptr;
    a.top_k = n_experts > 0 ? top_k : 1;
    a.y = y;
    a.y_dtype = y_dtype;
    a.e_begin = 0;
    a.e_end = n_experts;
    a.nan_rows = true;
    a.workspace = nullptr;
    if (workspace) {
        if (!aligned(workspace, 256)) return TQ_ERR_ALIGN;
        if (workspace_bytes < dmm::tq_prefill_ws_bytes(M, K)) return TQ_ERR_SHAPE;
        a.workspace = workspace;
    }
    hipStream_t s = (hipStream_t)stream;
    if (n_hot < 0 || n_hot == n_experts) return hip_status(dmm::launch_tq_matmul(a, s));
    if (n_hot == 0) {
        a.planes = 1;
        a.codes[1] = nullptr;
        a.scales[1] = nullptr;
        return hip_status(dmm::launch_tq_matmul(a, s));
    }
    // hot prefix: experts 0 .. n_hot - 1 with both planes, the rest with one
    // (disjoint output slots; the cold launch writes the rows of invalid ids)
    dmm::TqMatmulArgs hot = a;
    hot.e_end = n_hot;
    hot.nan_rows = false;
    dmm::TqMatmulArgs cold = a;
    cold.planes = 1;
    cold.codes[1] = nullptr;
    cold.scales[1] = nullptr;
    cold.e_begin = n_hot;
    hipError_t e = hipSuccess;
    if (dmm::launch_tq_wave_hot(hot, cold, s, &e)) return hip_status(e);   // one launch
    if (dmm::launch_tq_rows_hot(hot, cold, s, &e)) return hip_status(e);
    e = dmm::launch_tq_matmul(hot, s);
    if (e != hipSuccess) return TQ_ERR_HIP;
    return hip_status(dmm::launch_tq_matmul(cold, s));
}

int tq_matmul(const uint16_t* x, int64_t M, int64_t K, const uint8_t* codes1,
              const uint16_t* scales1, const uint8_t* codes2, const uint16_t* scales2,
              int64_t N, int32_t G, int32_t n_experts, const int32_t* expert_ids,
              int32_t top_k, void* y, int32_t y_dtype, void* stream) {
    return tq_matmul_common(x, M, K, codes1, scales1, codes2, scales2, -1, N, G, n_experts,
                            expert_ids, top_k, y, y_dtype, stream);
}

int64_t tq_prefill_workspace_bytes(int64_t M, int64_t K) {
    if (M < 0 || K < 0 || M >= kMaxDim || K >= kMaxDim) return -1;
    return dmm::tq_prefill_ws_bytes(M, K);
}

int tq_matmul_ws(const uint16_t* x, int64_t M, int64_t K, const uint8_t* codes1,
                 const uint16_t* scales1, const uint8_t* codes2, const uint16_t* scales2,
                 int64_t N, int32_t G, void* y, int32_t y_dtype, void* workspace,
                 int64_t workspace_bytes, void* stream) {
    return tq_matmul_common(x, M, K, codes1, scales1, codes2, scales2, -1, N, G, 0, nullptr, 1, y,
                            y_dtype, stream, workspace, workspace_bytes);
}

int tq_matmul_hot(const uint16_t* x, int64_t M, int64_t K, const uint8_t* codes1,
                  const uint16_t* scales1, const uint8_t* codes2, const uint16_t* scales2,
                  int32_t n_hot, int64_t N, int32_t G, int32_t n_experts,
                  const int32_t* expert_ids, int32_t top_k, void* y, int32_t y_dtype,
                  void* stream) {
    if (n_experts < 1) return TQ_ERR_UNSUPPORTED;     // grouped calls only
    if (n_hot < 0 || n_hot > n_experts) return TQ_ERR_SHAPE;
    if (n_hot > 0 && (!codes2 || !scales2)) return TQ_ERR_NULL;
    if (n_hot == 0 && (codes2 || scales2)) return TQ_ERR_SHAPE;
    return tq_matmul_common(x, M, K, codes1, scales1, codes2, scales2, n_hot, N, G, n_experts,
                            expert_ids, top_k, y, y_dtype, stream);
}

int rb_table(const float* ladder, float* table_out) {
    if (!ladder || !table_out) return TQ_ERR_NULL;
    for (int b = 0; b < 243; ++b) {
        double acc = 0.0;
        int p3 = 81;                               // 3^(5-i) for i = 1
        for (int i = 0; i < 5; ++i) {
            const int c = (b / p3) % 3 - 1;        // c_1 is the most significant digit
            acc += (double)c * (double)ladder[i];
            p3 /= 3;
        }
        table_out[b] = (float)acc;                 // one nearest-even rounding
    }
    return TQ_OK;
}

int rb_matmul(const uint16_t* x, int64_t M, int64_t K, const uint8_t* codes, int64_t N,
              const float* table, float alpha, const uint16_t* row_scale, const float* bias,
              void* y, int32_t y_dtype, void* stream) {
    return rb_matmul_rho_block(x, M, K, codes, N, table, alpha, row_scale, 1, bias, y, y_dtype,
                               stream);
}

// Every Route B matmul: code bytes (used == NULL) or 7-bit indices, one code
// book (table_rows == 0) or one per block of table_rows rows.
static int rb_matmul_common(const uint16_t* x, int64_t M, int64_t K, const uint8_t* codes,
                            const uint8_t* used, int64_t N, const float* table,
                            int32_t table_rows, float alpha, const uint16_t* row_scale,
                            int32_t rho_rows, const float* bias, void* y, int32_t y_dtype,
                            void* stream, void* workspace = nullptr, int64_t workspace_bytes = 0,
                            bool static_scratch = false) {
    if (M < 0 || K < 0 || N < 0 || M >= kMaxDim || K >= kMaxDim || N >= kMaxDim)
        return TQ_ERR_SHAPE;
    if (rho_rows < 1 || table_rows < 0) return TQ_ERR_SHAPE;
    if (table_rows % 32 != 0) return TQ_ERR_UNSUPPORTED;
    if (y_dtype != TQ_F32 && y_dtype != TQ_BF16) return TQ_ERR_DTYPE;
    if (M == 0 || N == 0) return TQ_OK;
    if (!table || !y || (K > 0 && (!x || !codes))) return TQ_ERR_NULL;
    if (!aligned(x, 2) || !aligned(table, 4) || (row_scale && !aligned(row_scale, 2)) ||
        (bias && !aligned(bias, 4)) || !aligned(y, y_dtype == TQ_F32 ? 4 : 2))
        return TQ_ERR_ALIGN;
    dmm::RbMatmulArgs a;
    a.x = x;
    a.M = M;
    a.K = K;
    a.N = N;
    a.codes = codes;
    a.used = used;
    a.table = table;
    a.table_rows = table_rows;
    a.alpha = alpha;
    a.row_scale = row_scale;
    a.rho_rows = rho_rows;
    a.bias = bias;
    a.y = y;
    a.y_dtype = y_dtype;
    a.workspace = nullptr;
    hipStream_t s = (hipStream_t)stream;
    if (M <= 16) {
        if ((N + 15) / 16 >= kMaxDim) return TQ_ERR_SHAPE;
        return hip_status(used ? dmm::launch_rb7_gemv(a, s) : dmm::launch_rb_gemv(a, s));
    }
    if ((M + 255) / 256 >= 65536) return TQ_ERR_SHAPE;
    if (static_scratch) {
        // the library's own per-device array stands in for the workspace
        if (dmm::rb_prefill_ws_bytes(M, K) > dmm::kScratchBytes) return TQ_ERR_SCRATCH;
        if (dmm::scratch_of_current_device(&workspace) != hipSuccess) return TQ_ERR_HIP;
        workspace_bytes = dmm::kScratchBytes;
    }
    if (workspace) {
        if (!aligned(workspace, 256)) return TQ_ERR_ALIGN;
        if (workspace_bytes < dmm::rb_prefill_ws_bytes(M, K)) return TQ_ERR_SHAPE;
        a.workspace = workspace;
    }
    return hip_status(dmm::launch_rb_prefill(a, s));
}

int64_t rb_prefill_workspace_bytes(int64_t M, int64_t K) {
    if (M < 0 || K < 0 || M >= kMaxDim || K >= kMaxDim) return -1;
    return dmm::rb_prefill_ws_bytes(M, K);
}

int rb_matmul_ws(const uint16_t* x, int64_t M, int64_t K, const uint8_t* codes, int64_t N,
                 const float* tables, int32_t table_rows, float alpha, const uint16_t* row_scale,
                 int32_t rho_rows, const float* bias, void* y, int32_t y_dtype, void* workspace,
                 int64_t workspace_bytes, void* stream) {
    return rb_matmul_common(x, M, K, codes, nullptr, N, tables, table_rows, alpha, row_scale,
                            rho_rows, bias, y, y_dtype, stream, workspace, workspace_bytes);
}

int rb_matmul_noalloc(const uint16_t* x, int64_t M, int64_t K, const uint8_t* codes, int64_t N,
                      const float* tables, int32_t table_rows, float alpha,
                      const uint16_t* row_scale, int32_t rho_rows, const float* bias, void* y,
                      int32_t y_dtype, void* stream) {
    return rb_matmul_common(x, M, K, codes, nullptr, N, tables, table_rows, alpha, row_scale,
                            rho_rows, bias, y, y_dtype, stream, nullptr, 0, true);
}

int rb_matmul_rho_block(const uint16_t* x, int64_t M, int64_t K, const uint8_t* codes, int64_t N,
                        const float* table, float alpha, const uint16_t* row_scale,
                        int32_t rho_rows, const float* bias, void* y, int32_t y_dtype,
                        void* stream) {
    return rb_matmul_common(x, M, K, codes, nullptr, N, table, 0, alpha, row_scale, rho_rows,
                            bias, y, y_dtype, stream);
}

int rb_matmul_blocks(const uint16_t* x, int64_t M, int64_t K, const uint8_t* codes, int64_t N,
                     const float* tables, int32_t table_rows, float alpha,
                     const uint16_t* row_scale, int32_t rho_rows, const float* bias, void* y,
                     int32_t y_dtype, void* stream) {
    return rb_matmul_common(x, M, K, codes, nullptr, N, tables, table_rows, alpha, row_scale,
                            rho_rows, bias, y, y_dtype, stream);
}

int rb_truncate(const uint8_t* codes, int64_t N, int64_t K, uint8_t* used_out,
                int32_t* n_used_out, uint8_t* codes7, int32_t* d_status, void* stream) {
    if (!used_out || !n_used_out || !d_status) return TQ_ERR_NULL;
    if (N < 0 || K < 0 || N >= kMaxDim || K >= kMaxDim) return TQ_ERR_SHAPE;
    if (N > 0 && K > 0 && (!codes || !codes7)) return TQ_ERR_NULL;
    if (!aligned(used_out, 4) || !aligned(n_used_out, 4) || !aligned(d_status, 4))
        return TQ_ERR_ALIGN;
    return hip_status(dmm::launch_rb_truncate(codes, N, K, used_out, n_used_out, codes7, d_status,
                                              (hipStream_t)stream));
}

int rb_matmul7(const uint16_t* x, int64_t M, int64_t K, const uint8_t* codes7, int64_t N,
               const uint8_t* used, const float* tables, int32_t table_rows, float alpha,
               const uint16_t* row_scale, int32_t rho_rows, const float* bias, void* y,
               int32_t y_dtype, void* stream) {
    if (!used) return TQ_ERR_NULL;
    return rb_matmul_common(x, M, K, codes7, used, N, tables, table_rows, alpha, row_scale,
                            rho_rows, bias, y, y_dtype, stream);
}

}  // extern "C"
