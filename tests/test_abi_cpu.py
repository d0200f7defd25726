"""The C ABI without a GPU: the library loads, exports every entry point of
include/decode_matmul.h, rejects bad arguments before touching the device,
and its host-side code-book builder matches the oracle bit for bit."""

import ctypes
import os
import re

import numpy as np
import pytest

import oracle
import workloads

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "decode_matmul.h")

dmm = pytest.importorskip("decode_matmul_amd")
lib = dmm.raw()

TQ_ERR_NULL, TQ_ERR_SHAPE, TQ_ERR_UNSUPPORTED, TQ_ERR_DTYPE, TQ_ERR_ALIGN = 1, 2, 3, 4, 5
TQ_ERR_SCRATCH = 7
FAKE = ctypes.c_void_p(0x10000)          # never dereferenced: every call below fails first
FAKE_ODD = ctypes.c_void_p(0x10001)


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^(?:int|int64_t|const char\*)\s+(\w+)\s*\(", text, re.M)))


def test_every_declared_symbol_is_exported():
    names = declared_functions()
    assert set(names) == set(dmm.EXPORTS)
    for n in names:
        assert hasattr(lib, n), n


def test_status_strings():
    for s in range(8):
        assert lib.tq_status_string(s) and lib.tq_status_string(s) != b"unknown status"
    assert lib.tq_status_string(99) == b"unknown status"


def test_rb_table_matches_oracle():
    """Host code book vs the oracle on the workload ladders, the integer
    ladder (exact b - 121) and the balanced ladder S0."""
    ladders = [workloads.routeb_gemv(seed=s, N=1, K=1, M=1)["ladder"] for s in range(6)]
    ladders.append(np.array([81, 27, 9, 3, 1], np.float32))
    ladders.append(np.array([1, 1 / 3, 1 / 9, 1 / 27, 1 / 81], np.float32))
    ladders.append(np.array([1.0, 0.33, 0.115, 0.037, 0.012], np.float32))
    for a in ladders:
        got = dmm.rb_table(a)
        ref = oracle.rb_table(a)
        assert np.array_equal(got.view(np.uint32), ref.view(np.uint32))


def test_rb_table_null():
    assert lib.rb_table(None, FAKE) == TQ_ERR_NULL


def test_pack_argument_errors():
    f = lib.tq_pack
    assert f(None, 4, 64, 64, 1, FAKE, FAKE, None, None, FAKE, None) == TQ_ERR_NULL
    assert f(FAKE, 4, 64, 64, 1, FAKE, FAKE, None, None, None, None) == TQ_ERR_NULL
    assert f(FAKE, -1, 64, 64, 1, FAKE, FAKE, None, None, FAKE, None) == TQ_ERR_SHAPE
    assert f(FAKE, 4, 64, 32, 1, FAKE, FAKE, None, None, FAKE, None) == TQ_ERR_UNSUPPORTED
    assert f(FAKE, 4, 64, 64, 3, FAKE, FAKE, None, None, FAKE, None) == TQ_ERR_UNSUPPORTED
    assert f(FAKE, 4, 64, 64, 2, FAKE, FAKE, None, None, FAKE, None) == TQ_ERR_NULL
    assert f(FAKE, 4, 64, 64, 1, FAKE, FAKE, FAKE, FAKE, FAKE, None) == TQ_ERR_SHAPE
    assert f(FAKE_ODD, 4, 64, 64, 1, FAKE, FAKE, None, None, FAKE, None) == TQ_ERR_ALIGN
    assert f(FAKE, 4, 64, 64, 1, FAKE, FAKE_ODD, None, None, FAKE, None) == TQ_ERR_ALIGN


def test_unpack_argument_errors():
    f = lib.tq_unpack
    assert f(None, FAKE, 4, 64, 64, FAKE, 0, FAKE, None) == TQ_ERR_NULL
    assert f(FAKE, FAKE, 4, 64, 100, FAKE, 0, FAKE, None) == TQ_ERR_UNSUPPORTED
    assert f(FAKE, FAKE, 4, 64, 64, FAKE, 7, FAKE, None) == TQ_ERR_DTYPE
    assert f(FAKE, FAKE, 4, -64, 64, FAKE, 0, FAKE, None) == TQ_ERR_SHAPE
    assert f(FAKE, FAKE, 4, 64, 64, FAKE_ODD, 0, FAKE, None) == TQ_ERR_ALIGN


def test_matmul_argument_errors():
    f = lib.tq_matmul
    ok = (FAKE, 1, 128, FAKE, FAKE, None, None, 16, 64, 0, None, 1, FAKE, 0, None)
    bad = list(ok); bad[8] = 96
    assert f(*bad) == TQ_ERR_UNSUPPORTED
    bad = list(ok); bad[2] = 100                       # K % G != 0
    assert f(*bad) == TQ_ERR_SHAPE
    bad = list(ok); bad[13] = 5
    assert f(*bad) == TQ_ERR_DTYPE
    bad = list(ok); bad[5] = FAKE                      # codes2 without scales2
    assert f(*bad) == TQ_ERR_NULL
    bad = list(ok); bad[0] = None
    assert f(*bad) == TQ_ERR_NULL
    bad = list(ok); bad[9] = 4                         # grouped without ids
    assert f(*bad) == TQ_ERR_NULL
    bad = list(ok); bad[9] = 4; bad[10] = FAKE; bad[11] = 0
    assert f(*bad) == TQ_ERR_SHAPE
    bad = list(ok); bad[9] = 4; bad[10] = FAKE; bad[1] = 1000; bad[11] = 8
    assert f(*bad) == TQ_ERR_SHAPE                     # M * top_k above the list limit
    bad = list(ok); bad[0] = FAKE_ODD
    assert f(*bad) == TQ_ERR_ALIGN
    bad = list(ok); bad[1] = 0                         # M = 0: no-op
    assert f(*bad) == 0
    bad = list(ok); bad[7] = 0                         # N = 0: no-op
    assert f(*bad) == 0


def test_rb_matmul_noalloc_argument_errors():
    """The allocation-free prefill entry point checks its arguments like
    rb_matmul_ws, and refuses a prefill whose workspace would exceed the
    library's static scratch before touching a device."""
    f = lib.rb_matmul_noalloc
    ok = [FAKE, 2048, 8192, FAKE, 8, FAKE, 0, ctypes.c_float(0.02), None, 1, None, FAKE, 0, None]
    bad = list(ok); bad[3] = None
    assert f(*bad) == TQ_ERR_NULL
    bad = list(ok); bad[12] = 2
    assert f(*bad) == TQ_ERR_DTYPE
    bad = list(ok); bad[0] = FAKE_ODD
    assert f(*bad) == TQ_ERR_ALIGN
    bad = list(ok); bad[1] = 4096                      # 64 MiB of fp16 activations
    assert f(*bad) == TQ_ERR_SCRATCH
    assert dmm.rb_prefill_workspace_bytes(2048, 8192) <= 34 << 20
    assert dmm.rb_prefill_workspace_bytes(4096, 8192) > 34 << 20
    bad = list(ok); bad[1] = 0                         # M = 0: no-op
    assert f(*bad) == 0


def test_rb_matmul_argument_errors():
    f = lib.rb_matmul
    ok = [FAKE, 4, 64, FAKE, 8, FAKE, ctypes.c_float(0.02), None, None, FAKE, 0, None]
    bad = list(ok); bad[3] = None
    assert f(*bad) == TQ_ERR_NULL
    bad = list(ok); bad[5] = None
    assert f(*bad) == TQ_ERR_NULL
    bad = list(ok); bad[10] = 2
    assert f(*bad) == TQ_ERR_DTYPE
    bad = list(ok); bad[2] = -1
    assert f(*bad) == TQ_ERR_SHAPE
    bad = list(ok); bad[5] = FAKE_ODD
    assert f(*bad) == TQ_ERR_ALIGN
    bad = list(ok); bad[1] = 0
    assert f(*bad) == 0


def test_rb_encode_argument_errors():
    f = lib.rb_encode
    lad = np.array([1, 1 / 3, 1 / 9, 1 / 27, 1 / 81], np.float32)
    lp = lad.ctypes.data_as(ctypes.c_void_p)
    bad_lad = lad.copy()
    bad_lad[2] = np.nan
    bp = bad_lad.ctypes.data_as(ctypes.c_void_p)
    z = ctypes.c_float
    ok = [FAKE, 4, 64, lp, z(0.0), 0, FAKE, FAKE, None, FAKE, None]

    def call(i, v):
        a = list(ok)
        a[i] = v
        return f(*a)

    assert call(3, None) == TQ_ERR_NULL                # ladder
    assert call(7, None) == TQ_ERR_NULL                # alpha_out
    assert call(9, None) == TQ_ERR_NULL                # d_status
    assert call(0, None) == TQ_ERR_NULL                # W with N, K > 0
    assert call(6, None) == TQ_ERR_NULL                # codes
    assert call(1, -1) == TQ_ERR_SHAPE
    assert call(2, -5) == TQ_ERR_SHAPE
    assert call(5, -1) == TQ_ERR_SHAPE                 # rho_rows
    assert call(4, z(1.5)) == TQ_ERR_UNSUPPORTED       # zeta outside [0, 1]
    assert call(4, z(-0.1)) == TQ_ERR_UNSUPPORTED
    assert call(4, z(float("nan"))) == TQ_ERR_UNSUPPORTED
    assert call(3, bp) == TQ_ERR_UNSUPPORTED           # non-finite ladder step
    assert call(5, 1) == TQ_ERR_NULL                   # row scales without row_scale
    assert call(5, 256) == TQ_ERR_NULL                 # head scales without row_scale
    assert call(8, FAKE) == TQ_ERR_SHAPE               # row_scale with the global scale
    assert call(0, FAKE_ODD) == TQ_ERR_ALIGN
    assert call(7, FAKE_ODD) == TQ_ERR_ALIGN


def test_tq_matmul_hot_argument_errors():
    f = lib.tq_matmul_hot
    ok = [FAKE, 2, 128, FAKE, FAKE, FAKE, FAKE, 2, 16, 64, 4, FAKE, 2, FAKE, 0, None]
    bad = list(ok); bad[10] = 0
    assert f(*bad) == TQ_ERR_UNSUPPORTED               # dense: not a grouped call
    bad = list(ok); bad[7] = 5
    assert f(*bad) == TQ_ERR_SHAPE                     # n_hot > n_experts
    bad = list(ok); bad[7] = -1
    assert f(*bad) == TQ_ERR_SHAPE
    bad = list(ok); bad[5] = None
    assert f(*bad) == TQ_ERR_NULL                      # hot experts without plane 2
    bad = list(ok); bad[7] = 0
    assert f(*bad) == TQ_ERR_SHAPE                     # plane 2 given for no hot expert
    bad = list(ok); bad[9] = 96
    assert f(*bad) == TQ_ERR_UNSUPPORTED               # group size
    bad = list(ok); bad[11] = None
    assert f(*bad) == TQ_ERR_NULL                      # ids
    bad = list(ok); bad[1] = 0
    assert f(*bad) == 0                                # M = 0: no-op


def test_rb_matmul_rho_block_argument_errors():
    f = lib.rb_matmul_rho_block
    ok = [FAKE, 4, 64, FAKE, 8, FAKE, ctypes.c_float(0.02), FAKE, 2, None, FAKE, 0, None]
    bad = list(ok); bad[8] = 0
    assert f(*bad) == TQ_ERR_SHAPE                     # rho_rows < 1
    bad = list(ok); bad[8] = -3
    assert f(*bad) == TQ_ERR_SHAPE
    bad = list(ok); bad[7] = FAKE_ODD
    assert f(*bad) == TQ_ERR_ALIGN
    bad = list(ok); bad[5] = None
    assert f(*bad) == TQ_ERR_NULL
    bad = list(ok); bad[1] = 0
    assert f(*bad) == 0                                # M = 0: no-op


def test_binding_refuses_wrong_tensors():
    import torch
    x = torch.zeros(1, 64, dtype=torch.float32)
    with pytest.raises(TypeError):
        dmm.tq_matmul(x, torch.zeros(16 * 13, dtype=torch.uint8),
                      torch.zeros(16, dtype=torch.float16), 16, 64,
                      torch.zeros(1, 16, dtype=torch.float32))
    xb = torch.zeros(1, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        dmm.tq_matmul(xb, torch.zeros(15 * 13, dtype=torch.uint8),
                      torch.zeros(16, dtype=torch.float16), 16, 64,
                      torch.zeros(1, 16, dtype=torch.float32))


def test_rb_matmul_blocks_argument_errors():
    f = lib.rb_matmul_blocks
    # x, M, K, codes, N, tables, table_rows, alpha, row_scale, rho_rows, bias, y, y_dtype, stream
    ok = [FAKE, 4, 64, FAKE, 64, FAKE, 32, ctypes.c_float(0.02), None, 1, None, FAKE, 0, None]
    for tr in (16, 33, 48, 1):
        bad = list(ok); bad[6] = tr
        assert f(*bad) == TQ_ERR_UNSUPPORTED            # not a multiple of 32
    bad = list(ok); bad[6] = -32
    assert f(*bad) == TQ_ERR_SHAPE
    bad = list(ok); bad[9] = 0
    assert f(*bad) == TQ_ERR_SHAPE                      # rho_rows < 1
    bad = list(ok); bad[5] = None
    assert f(*bad) == TQ_ERR_NULL
    bad = list(ok); bad[5] = FAKE_ODD
    assert f(*bad) == TQ_ERR_ALIGN
    bad = list(ok); bad[12] = 7
    assert f(*bad) == TQ_ERR_DTYPE
    bad = list(ok); bad[4] = 0
    assert f(*bad) == 0                                 # N = 0: no-op


def test_rb_truncate_argument_errors():
    f = lib.rb_truncate
    # codes, N, K, used_out, n_used_out, codes7, d_status, stream
    ok = [FAKE, 8, 64, FAKE, FAKE, FAKE, FAKE, None]
    for i in (3, 4, 6):
        bad = list(ok); bad[i] = None
        assert f(*bad) == TQ_ERR_NULL
    bad = list(ok); bad[0] = None
    assert f(*bad) == TQ_ERR_NULL
    bad = list(ok); bad[5] = None
    assert f(*bad) == TQ_ERR_NULL
    bad = list(ok); bad[1] = -1
    assert f(*bad) == TQ_ERR_SHAPE
    bad = list(ok); bad[2] = 1 << 31
    assert f(*bad) == TQ_ERR_SHAPE
    for i in (3, 4, 6):
        bad = list(ok); bad[i] = ctypes.c_void_p(0x10002)
        assert f(*bad) == TQ_ERR_ALIGN                  # used_out, n_used_out, d_status


def test_rb_matmul7_argument_errors():
    f = lib.rb_matmul7
    # x, M, K, codes7, N, used, tables, table_rows, alpha, row_scale, rho_rows, bias, y, dtype, stream
    ok = [FAKE, 4, 64, FAKE, 64, FAKE, FAKE, 0, ctypes.c_float(0.02), None, 1, None, FAKE, 0, None]
    bad = list(ok); bad[5] = None
    assert f(*bad) == TQ_ERR_NULL                       # the used-code list
    bad = list(ok); bad[7] = 20
    assert f(*bad) == TQ_ERR_UNSUPPORTED
    bad = list(ok); bad[6] = None
    assert f(*bad) == TQ_ERR_NULL
    bad = list(ok); bad[3] = None
    assert f(*bad) == TQ_ERR_NULL
    bad = list(ok); bad[1] = 0
    assert f(*bad) == 0


def test_status_string_new_flags():
    assert dmm.TQ_DATA_ALPHABET == 8
    text = open(HEADER).read()
    assert re.search(r"TQ_DATA_ALPHABET\s*=\s*8", text)


def test_rb_matmul_ws_workspace_checks():
    """The prefill workspace: its size formula, and a misaligned or short
    workspace rejected before any launch (M > 16 takes the prefill path)."""
    M, K, N = 300, 1024, 64
    nbytes = lib.rb_prefill_workspace_bytes(M, K)
    want = (M * K * 2 + 255) // 256 * 256 + (-(-M // 256)) * (-(-K // 32)) * 4
    assert nbytes == want
    assert lib.rb_prefill_workspace_bytes(-1, K) == -1
    ws_args = lambda ws, nb: (FAKE, M, K, FAKE, N, FAKE, 0, ctypes.c_float(1.0), None, 1, None,
                              FAKE, 0, ws, nb, None)
    assert lib.rb_matmul_ws(*ws_args(FAKE_ODD, nbytes)) == TQ_ERR_ALIGN
    assert lib.rb_matmul_ws(*ws_args(FAKE, nbytes - 1)) == TQ_ERR_SHAPE


def test_tq_matmul_ws_workspace_checks():
    """The ternary prefill workspace: its size formula, and a misaligned or
    short workspace rejected before any launch."""
    M, K, N = 300, 1024, 64
    nbytes = lib.tq_prefill_workspace_bytes(M, K)
    want = (M * K * 2 + 255) // 256 * 256 + (-(-M // 128)) * (-(-K // 64)) * 4
    assert nbytes == want
    assert lib.tq_prefill_workspace_bytes(M, -1) == -1
    args = lambda ws, nb: (FAKE, M, K, FAKE, FAKE, None, None, N, 64, FAKE, 0, ws, nb, None)
    assert lib.tq_matmul_ws(*args(FAKE_ODD, nbytes)) == TQ_ERR_ALIGN
    assert lib.tq_matmul_ws(*args(FAKE, nbytes - 1)) == TQ_ERR_SHAPE
