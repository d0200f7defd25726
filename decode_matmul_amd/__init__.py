"""Python binding of libdecode_matmul.so (packed ternary-code matmul, gfx950).

Argument marshalling only: each function below has the name of a C entry
point of include/decode_matmul.h, checks that the torch tensors it is handed
have the dtype, device, contiguity and size the C call will touch, passes raw
device pointers and the current HIP stream, and raises RuntimeError on a
non-zero status.  All arithmetic runs in the HIP kernels.  PyTorch supplies
device memory and streams.

If the shared library has not been built, importing this package raises
ImportError: there is no fallback path.
"""

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libdecode_matmul.so")

TQ_OK = 0
TQ_F32 = 0
TQ_BF16 = 1
TQ_DATA_RANGE = 1
TQ_DATA_CODE = 2
TQ_DATA_PADDING = 4
TQ_DATA_ALPHABET = 8

EXPORTS = ("tq_pack", "tq_unpack", "tq_matmul", "tq_matmul_hot", "rb_table", "rb_encode",
           "rb_matmul", "rb_matmul_rho_block", "rb_matmul_blocks", "rb_truncate",
           "rb_matmul7", "rb_matmul_ws", "rb_prefill_workspace_bytes", "tq_matmul_ws",
           "tq_prefill_workspace_bytes", "rb_matmul_noalloc", "tq_status_string")

if not os.path.exists(LIB_PATH):
    raise ImportError(
        f"{LIB_PATH} is missing: build it with `python decode_matmul_amd/build.py` "
        "(there is no CPU fallback)")

_lib = ctypes.CDLL(LIB_PATH)

_p = ctypes.c_void_p
_i64 = ctypes.c_int64
_i32 = ctypes.c_int32

_lib.tq_pack.argtypes = [_p, _i64, _i64, _i32, _i32, _p, _p, _p, _p, _p, _p]
_lib.tq_unpack.argtypes = [_p, _p, _i64, _i64, _i32, _p, _i32, _p, _p]
_lib.tq_matmul.argtypes = [_p, _i64, _i64, _p, _p, _p, _p, _i64, _i32, _i32, _p, _i32, _p,
                           _i32, _p]
_lib.tq_matmul_hot.argtypes = [_p, _i64, _i64, _p, _p, _p, _p, _i32, _i64, _i32, _i32, _p,
                               _i32, _p, _i32, _p]
_lib.rb_table.argtypes = [_p, _p]
_lib.rb_encode.argtypes = [_p, _i64, _i64, _p, ctypes.c_float, _i32, _p, _p, _p, _p, _p]
_lib.rb_matmul.argtypes = [_p, _i64, _i64, _p, _i64, _p, ctypes.c_float, _p, _p, _p, _i32, _p]
_lib.rb_matmul_rho_block.argtypes = [_p, _i64, _i64, _p, _i64, _p, ctypes.c_float, _p, _i32, _p,
                                     _p, _i32, _p]
_lib.rb_matmul_blocks.argtypes = [_p, _i64, _i64, _p, _i64, _p, _i32, ctypes.c_float, _p, _i32,
                                  _p, _p, _i32, _p]
_lib.rb_truncate.argtypes = [_p, _i64, _i64, _p, _p, _p, _p, _p]
_lib.rb_matmul7.argtypes = [_p, _i64, _i64, _p, _i64, _p, _p, _i32, ctypes.c_float, _p, _i32,
                            _p, _p, _i32, _p]
_lib.rb_matmul_ws.argtypes = [_p, _i64, _i64, _p, _i64, _p, _i32, ctypes.c_float, _p, _i32,
                              _p, _p, _i32, _p, _i64, _p]
_lib.rb_prefill_workspace_bytes.argtypes = [_i64, _i64]
_lib.tq_matmul_ws.argtypes = [_p, _i64, _i64, _p, _p, _p, _p, _i64, _i32, _p, _i32, _p, _i64, _p]
_lib.rb_matmul_noalloc.argtypes = [_p, _i64, _i64, _p, _i64, _p, _i32, ctypes.c_float, _p, _i32,
                                   _p, _p, _i32, _p]
_lib.tq_prefill_workspace_bytes.argtypes = [_i64, _i64]
_lib.tq_status_string.argtypes = [_i32]
_lib.tq_status_string.restype = ctypes.c_char_p
for _name in EXPORTS[:-1]:
    getattr(_lib, _name).restype = _i32
_lib.rb_prefill_workspace_bytes.restype = _i64
_lib.tq_prefill_workspace_bytes.restype = _i64


def tq_status_string(status):
    return _lib.tq_status_string(int(status)).decode()


def _raise(rc, what):
    if rc != TQ_OK:
        raise RuntimeError(f"{what}: {tq_status_string(rc)} (status {rc})")


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _need(t, name, dtypes, numel, device):
    if t is None:
        raise ValueError(f"{name} is required")
    if t.dtype not in dtypes:
        raise TypeError(f"{name}: dtype {t.dtype} not in {dtypes}")
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if t.numel() != numel:
        raise ValueError(f"{name} has {t.numel()} elements, expected {numel}")


_U8 = (torch.uint8,)
_H16 = (torch.float16, torch.int16, torch.uint16)
_BF16 = (torch.bfloat16, torch.int16, torch.uint16)
_F32 = (torch.float32,)
_I32 = (torch.int32,)


def packed_shape(rows, K, G):
    """(codes shape, scales shape) of the package of a [rows, K] matrix."""
    ng = -(-K // G)
    return (rows, ng, -(-G // 5)), (rows, ng)


def _ydtype(y):
    if y.dtype == torch.float32:
        return TQ_F32
    if y.dtype in _BF16:
        return TQ_BF16
    raise TypeError(f"y dtype {y.dtype} must be float32 or bfloat16")


def tq_pack(W, G, planes, codes1, scales1, codes2=None, scales2=None, status=None):
    """Quantize and pack fp32 W [rows, K] into caller-allocated packages."""
    dev = W.device
    rows, K = W.shape
    cs, ss = packed_shape(rows, K, G)
    _need(W, "W", _F32, rows * K, dev)
    _need(codes1, "codes1", _U8, cs[0] * cs[1] * cs[2], dev)
    _need(scales1, "scales1", _H16, ss[0] * ss[1], dev)
    if planes == 2:
        _need(codes2, "codes2", _U8, cs[0] * cs[1] * cs[2], dev)
        _need(scales2, "scales2", _H16, ss[0] * ss[1], dev)
    if status is None:
        status = torch.zeros(1, dtype=torch.int32, device=dev)
    _need(status, "status", _I32, 1, dev)
    rc = _lib.tq_pack(_ptr(W), rows, K, G, planes, _ptr(codes1), _ptr(scales1), _ptr(codes2),
                      _ptr(scales2), _ptr(status), _stream(dev))
    _raise(rc, "tq_pack")
    return status


def tq_unpack(codes, scales, rows, K, G, W_out, status=None):
    """Decode a package into W_out [rows, K] (float32 exact, or bfloat16)."""
    dev = codes.device
    cs, ss = packed_shape(rows, K, G)
    _need(codes, "codes", _U8, cs[0] * cs[1] * cs[2], dev)
    _need(scales, "scales", _H16, ss[0] * ss[1], dev)
    if W_out.dtype == torch.float32:
        odt = TQ_F32
    elif W_out.dtype in _BF16:
        odt = TQ_BF16
    else:
        raise TypeError("W_out must be float32 or bfloat16")
    _need(W_out, "W_out", (W_out.dtype,), rows * K, dev)
    if status is None:
        status = torch.zeros(1, dtype=torch.int32, device=dev)
    _need(status, "status", _I32, 1, dev)
    rc = _lib.tq_unpack(_ptr(codes), _ptr(scales), rows, K, G, _ptr(W_out), odt, _ptr(status),
                        _stream(dev))
    _raise(rc, "tq_unpack")
    return status


def tq_matmul(x, codes1, scales1, N, G, y, codes2=None, scales2=None, n_experts=0,
              expert_ids=None, top_k=1):
    """y = x W_hat^T; dense (n_experts=0) or grouped by expert_ids [M, top_k]."""
    dev = x.device
    M, K = x.shape
    E = max(n_experts, 1)
    cs, ss = packed_shape(N, K, G)
    _need(x, "x", _BF16, M * K, dev)
    _need(codes1, "codes1", _U8, E * cs[0] * cs[1] * cs[2], dev)
    _need(scales1, "scales1", _H16, E * ss[0] * ss[1], dev)
    if codes2 is not None or scales2 is not None:
        _need(codes2, "codes2", _U8, E * cs[0] * cs[1] * cs[2], dev)
        _need(scales2, "scales2", _H16, E * ss[0] * ss[1], dev)
    if n_experts > 0:
        _need(expert_ids, "expert_ids", _I32, M * top_k, dev)
        _need(y, "y", (y.dtype,), M * top_k * N, dev)
    else:
        _need(y, "y", (y.dtype,), M * N, dev)
    rc = _lib.tq_matmul(_ptr(x), M, K, _ptr(codes1), _ptr(scales1), _ptr(codes2), _ptr(scales2),
                        N, G, n_experts, _ptr(expert_ids), top_k, _ptr(y), _ydtype(y),
                        _stream(dev))
    _raise(rc, "tq_matmul")


def tq_prefill_workspace_bytes(M, K):
    """Bytes of the workspace tq_matmul_ws takes for [M, K] activations."""
    n = int(_lib.tq_prefill_workspace_bytes(int(M), int(K)))
    if n < 0:
        raise ValueError(f"tq_prefill_workspace_bytes: bad shape {M} x {K}")
    return n


def tq_matmul_ws(x, codes1, scales1, N, G, y, workspace, codes2=None, scales2=None):
    """Dense tq_matmul with a workspace (uint8 device tensor of at least
    tq_prefill_workspace_bytes(M, K) bytes, or None) in which the prefill
    converts the activations once per call."""
    dev = x.device
    M, K = x.shape
    cs, ss = packed_shape(N, K, G)
    _need(x, "x", _BF16, M * K, dev)
    _need(codes1, "codes1", _U8, cs[0] * cs[1] * cs[2], dev)
    _need(scales1, "scales1", _H16, ss[0] * ss[1], dev)
    if codes2 is not None or scales2 is not None:
        _need(codes2, "codes2", _U8, cs[0] * cs[1] * cs[2], dev)
        _need(scales2, "scales2", _H16, ss[0] * ss[1], dev)
    _need(y, "y", (y.dtype,), M * N, dev)
    nbytes = 0
    if workspace is not None:
        nbytes = workspace.numel()
        _need(workspace, "workspace", _U8, nbytes, dev)
    rc = _lib.tq_matmul_ws(_ptr(x), M, K, _ptr(codes1), _ptr(scales1), _ptr(codes2),
                           _ptr(scales2), N, G, _ptr(y), _ydtype(y), _ptr(workspace), nbytes,
                           _stream(dev))
    _raise(rc, "tq_matmul_ws")


def tq_matmul_hot(x, codes1, scales1, N, G, y, n_hot, n_experts, expert_ids, top_k,
                  codes2=None, scales2=None):
    """Grouped experts whose plane 2 covers only the hot prefix 0 .. n_hot - 1:
    codes2 / scales2 hold n_hot experts' second planes."""
    dev = x.device
    M, K = x.shape
    cs, ss = packed_shape(N, K, G)
    _need(x, "x", _BF16, M * K, dev)
    _need(codes1, "codes1", _U8, n_experts * cs[0] * cs[1] * cs[2], dev)
    _need(scales1, "scales1", _H16, n_experts * ss[0] * ss[1], dev)
    if n_hot > 0:
        _need(codes2, "codes2", _U8, n_hot * cs[0] * cs[1] * cs[2], dev)
        _need(scales2, "scales2", _H16, n_hot * ss[0] * ss[1], dev)
    _need(expert_ids, "expert_ids", _I32, M * top_k, dev)
    _need(y, "y", (y.dtype,), M * top_k * N, dev)
    rc = _lib.tq_matmul_hot(_ptr(x), M, K, _ptr(codes1), _ptr(scales1), _ptr(codes2),
                            _ptr(scales2), n_hot, N, G, n_experts, _ptr(expert_ids), top_k,
                            _ptr(y), _ydtype(y), _stream(dev))
    _raise(rc, "tq_matmul_hot")


def rb_table(ladder):
    """Host: 243-entry fp32 code book of a 5-step ladder (numpy float32 arrays)."""
    import numpy as np
    a = np.ascontiguousarray(ladder, dtype=np.float32)
    if a.shape != (5,):
        raise ValueError("the ladder has five steps")
    out = np.zeros(243, dtype=np.float32)
    rc = _lib.rb_table(a.ctypes.data_as(_p), out.ctypes.data_as(_p))
    _raise(rc, "rb_table")
    return out


def rb_encode(W, ladder, codes, alpha_out, zeta=0.0, row_scale=None, rho_rows=None,
              status=None):
    """Route B encoder: fp32 W [N, K] -> codes uint8 [N, K] and alpha_out fp32.
    Without row_scale: one global scale, alpha_out [1].  With row_scale (fp16
    [ceil(N / rho_rows)], rho_rows 1 by default): one scale per block of
    rho_rows rows, alpha_out [1 + ceil(N / rho_rows)]."""
    import numpy as np
    dev = W.device
    N, K = W.shape
    b = 0 if row_scale is None else (1 if rho_rows is None else int(rho_rows))
    nb = -(-N // b) if b > 0 else 0
    _need(W, "W", _F32, N * K, dev)
    _need(codes, "codes", _U8, N * K, dev)
    _need(alpha_out, "alpha_out", _F32, 1 + nb, dev)
    if row_scale is not None:
        _need(row_scale, "row_scale", _H16, nb, dev)
    if status is None:
        status = torch.zeros(1, dtype=torch.int32, device=dev)
    _need(status, "status", _I32, 1, dev)
    a = np.ascontiguousarray(np.asarray(ladder, dtype=np.float32).reshape(5))
    rc = _lib.rb_encode(_ptr(W), N, K, a.ctypes.data_as(_p), float(zeta), b, _ptr(codes),
                        _ptr(alpha_out), _ptr(row_scale), _ptr(status), _stream(dev))
    _raise(rc, "rb_encode")
    return status


def rb_matmul(x, codes, table, alpha, y, row_scale=None, bias=None, rho_rows=1):
    """y = alpha * rho * (x T[codes]^T) + bias for uint8 codes [N, K]; rho of
    row n is row_scale[n // rho_rows]."""
    dev = x.device
    M, K = x.shape
    N = codes.shape[0]
    _need(x, "x", _BF16, M * K, dev)
    _need(codes, "codes", _U8, N * K, dev)
    _need(table, "table", _F32, 243, dev)
    if row_scale is not None:
        _need(row_scale, "row_scale", _H16, -(-N // int(rho_rows)) if rho_rows > 0 else N, dev)
    if bias is not None:
        _need(bias, "bias", _F32, N, dev)
    _need(y, "y", (y.dtype,), M * N, dev)
    if rho_rows == 1:
        rc = _lib.rb_matmul(_ptr(x), M, K, _ptr(codes), N, _ptr(table), float(alpha),
                            _ptr(row_scale), _ptr(bias), _ptr(y), _ydtype(y), _stream(dev))
    else:
        rc = _lib.rb_matmul_rho_block(_ptr(x), M, K, _ptr(codes), N, _ptr(table), float(alpha),
                                      _ptr(row_scale), int(rho_rows), _ptr(bias), _ptr(y),
                                      _ydtype(y), _stream(dev))
    _raise(rc, "rb_matmul")


def _tables(tables, N, table_rows, dev):
    nb = -(-N // int(table_rows)) if table_rows > 0 else 1
    _need(tables, "tables", _F32, nb * 243, dev)


def rb_matmul_blocks(x, codes, tables, table_rows, alpha, y, row_scale=None, bias=None,
                     rho_rows=1):
    """rb_matmul with code book tables[n // table_rows] for row n (fp32
    [ceil(N / table_rows), 243]; table_rows a multiple of 32, or 0 for one
    book)."""
    dev = x.device
    M, K = x.shape
    N = codes.shape[0]
    _need(x, "x", _BF16, M * K, dev)
    _need(codes, "codes", _U8, N * K, dev)
    _tables(tables, N, table_rows, dev)
    if row_scale is not None:
        _need(row_scale, "row_scale", _H16, -(-N // int(rho_rows)) if rho_rows > 0 else N, dev)
    if bias is not None:
        _need(bias, "bias", _F32, N, dev)
    _need(y, "y", (y.dtype,), M * N, dev)
    rc = _lib.rb_matmul_blocks(_ptr(x), M, K, _ptr(codes), N, _ptr(tables), int(table_rows),
                               float(alpha), _ptr(row_scale), int(rho_rows), _ptr(bias), _ptr(y),
                               _ydtype(y), _stream(dev))
    _raise(rc, "rb_matmul_blocks")


def rb_prefill_workspace_bytes(M, K):
    """Bytes of the workspace rb_matmul_ws takes for [M, K] activations."""
    n = int(_lib.rb_prefill_workspace_bytes(int(M), int(K)))
    if n < 0:
        raise ValueError(f"rb_prefill_workspace_bytes: bad shape {M} x {K}")
    return n


def rb_matmul_ws(x, codes, tables, table_rows, alpha, y, workspace, row_scale=None, bias=None,
                 rho_rows=1):
    """rb_matmul_blocks with a workspace (uint8 device tensor of at least
    rb_prefill_workspace_bytes(M, K) bytes, or None) in which the prefill
    converts the activations once per call."""
    dev = x.device
    M, K = x.shape
    N = codes.shape[0]
    _need(x, "x", _BF16, M * K, dev)
    _need(codes, "codes", _U8, N * K, dev)
    _tables(tables, N, table_rows, dev)
    if row_scale is not None:
        _need(row_scale, "row_scale", _H16, -(-N // int(rho_rows)) if rho_rows > 0 else N, dev)
    if bias is not None:
        _need(bias, "bias", _F32, N, dev)
    _need(y, "y", (y.dtype,), M * N, dev)
    nbytes = 0
    if workspace is not None:
        nbytes = workspace.numel()
        _need(workspace, "workspace", _U8, nbytes, dev)
    rc = _lib.rb_matmul_ws(_ptr(x), M, K, _ptr(codes), N, _ptr(tables), int(table_rows),
                           float(alpha), _ptr(row_scale), int(rho_rows), _ptr(bias), _ptr(y),
                           _ydtype(y), _ptr(workspace), nbytes, _stream(dev))
    _raise(rc, "rb_matmul_ws")


def rb_matmul_noalloc(x, codes, tables, table_rows, alpha, y, row_scale=None, bias=None,
                      rho_rows=1):
    """rb_matmul_ws whose workspace is the library's own per-device scratch
    array (DMM_SCRATCH_BYTES): the call allocates nothing."""
    dev = x.device
    M, K = x.shape
    N = codes.shape[0]
    _need(x, "x", _BF16, M * K, dev)
    _need(codes, "codes", _U8, N * K, dev)
    _tables(tables, N, table_rows, dev)
    if row_scale is not None:
        _need(row_scale, "row_scale", _H16, -(-N // int(rho_rows)) if rho_rows > 0 else N, dev)
    if bias is not None:
        _need(bias, "bias", _F32, N, dev)
    _need(y, "y", (y.dtype,), M * N, dev)
    with torch.cuda.device(dev):
        rc = _lib.rb_matmul_noalloc(_ptr(x), M, K, _ptr(codes), N, _ptr(tables), int(table_rows),
                                    float(alpha), _ptr(row_scale), int(rho_rows), _ptr(bias),
                                    _ptr(y), _ydtype(y), _stream(dev))
    _raise(rc, "rb_matmul_noalloc")


def rb7_row_bytes(K):
    """Bytes per row of 7-bit indices."""
    return -(-7 * int(K) // 8)


def rb_truncate(codes, used, n_used, codes7, status=None):
    """uint8 codes [N, K] -> used uint8 [128] (increasing used codes, padded
    with 121), n_used int32 [1] and codes7 uint8 [N, ceil(7 K / 8)]."""
    dev = codes.device
    N, K = codes.shape
    _need(codes, "codes", _U8, N * K, dev)
    _need(used, "used", _U8, 128, dev)
    _need(n_used, "n_used", _I32, 1, dev)
    _need(codes7, "codes7", _U8, N * rb7_row_bytes(K), dev)
    if status is None:
        status = torch.zeros(1, dtype=torch.int32, device=dev)
    _need(status, "status", _I32, 1, dev)
    rc = _lib.rb_truncate(_ptr(codes), N, K, _ptr(used), _ptr(n_used), _ptr(codes7),
                          _ptr(status), _stream(dev))
    _raise(rc, "rb_truncate")
    return status


def rb_matmul7(x, codes7, N, used, tables, table_rows, alpha, y, row_scale=None, bias=None,
               rho_rows=1):
    """Route B matmul over 7-bit indices codes7 [N, ceil(7 K / 8)]: weight
    (n, k) is tables[n // table_rows][used[index]] (table_rows 0: one book)."""
    dev = x.device
    M, K = x.shape
    _need(x, "x", _BF16, M * K, dev)
    _need(codes7, "codes7", _U8, N * rb7_row_bytes(K), dev)
    _need(used, "used", _U8, 128, dev)
    _tables(tables, N, table_rows, dev)
    if row_scale is not None:
        _need(row_scale, "row_scale", _H16, -(-N // int(rho_rows)) if rho_rows > 0 else N, dev)
    if bias is not None:
        _need(bias, "bias", _F32, N, dev)
    _need(y, "y", (y.dtype,), M * N, dev)
    rc = _lib.rb_matmul7(_ptr(x), M, K, _ptr(codes7), N, _ptr(used), _ptr(tables),
                         int(table_rows), float(alpha), _ptr(row_scale), int(rho_rows),
                         _ptr(bias), _ptr(y), _ydtype(y), _stream(dev))
    _raise(rc, "rb_matmul7")


def raw():
    """The ctypes handle, for callers that marshal pointers themselves."""
    return _lib
