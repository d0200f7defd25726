"""rb_matmul_noalloc through the C ABI: the allocation-free prefill entry
point, whose workspace is the library's own per-device scratch array, against
rb_matmul_ws with a caller workspace (bit for bit) and the oracle (the
acceptance bound), on two calls in a row, the second smaller, so that it
runs over the first call's leftovers in the shared array."""

import ctypes

import numpy as np
import pytest

import oracle
import workloads

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

DEV = "cuda:0"
TQ_F32, TQ_ERR_SCRATCH = 0, 7


def say(msg):
    print(f"[case] {msg}", flush=True)


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def bits16(a):
    return np.ascontiguousarray(a).view(np.int16)


def p(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def case(dmm, lib, M, N, K, seed, special):
    rng = np.random.default_rng(seed)
    codes = rng.integers(0, 243, (N, K), dtype=np.uint8)
    ladder = np.array([1.0, 0.33, 0.115, 0.037, 0.012], np.float32) * np.float32(rng.uniform(0.8, 1.2))
    table = oracle.rb_table(ladder.astype(np.float32))
    xf = rng.standard_normal((M, K)).astype(np.float32)
    if special:
        # activations fp16 cannot hold: the pre-pass flags their slices for replay
        xf[rng.integers(0, M, 8), rng.integers(0, K, 8)] = 3.0e-7
        xf[rng.integers(0, M, 8), rng.integers(0, K, 8)] = -7.0e4
    xb = workloads.bf16_bits(xf)
    rs = rng.uniform(0.5, 1.5, N).astype(np.float16).view(np.uint16)
    alpha = np.float32(0.02)
    xd, cd, td, rsd = dev(bits16(xb)), dev(codes), dev(table), dev(bits16(rs))
    y_na = torch.empty((M, N), dtype=torch.float32, device=DEV)
    y_ws = torch.empty((M, N), dtype=torch.float32, device=DEV)
    ws = torch.empty(dmm.rb_prefill_workspace_bytes(M, K), dtype=torch.uint8, device=DEV)
    ws.fill_(0xA5)
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    say(f"rb_matmul_noalloc M={M} N={N} K={K} special={special}")
    rc = lib.rb_matmul_noalloc(p(xd), M, K, p(cd), N, p(td), 0, ctypes.c_float(alpha), p(rsd), 1,
                               None, p(y_na), TQ_F32, stream)
    assert rc == 0, dmm.tq_status_string(rc)
    dmm.rb_matmul_ws(xd, cd, td, 0, float(alpha), y_ws, ws, rsd)
    torch.cuda.synchronize()
    a, b = y_na.cpu().numpy(), y_ws.cpu().numpy()
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32)), "differs from rb_matmul_ws"
    y_ref, B = oracle.matmul_ref(xb, oracle.rb_weights(codes, table, alpha, rs))
    r = oracle.check_bound(a, y_ref, B, stored="f32")
    assert r["ok"], r


def test_rb_matmul_noalloc_two_calls():
    import decode_matmul_amd as dmm
    lib = dmm.raw()
    case(dmm, lib, 600, 520, 8192, seed=1, special=True)
    case(dmm, lib, 40, 130, 512, seed=2, special=False)
    # beyond the scratch: refused on the host before any launch
    say("rb_matmul_noalloc over the limit")
    rc = lib.rb_matmul_noalloc(ctypes.c_void_p(0x10000), 4096, 8192, ctypes.c_void_p(0x10000), 8,
                               ctypes.c_void_p(0x10000), 0, ctypes.c_float(1.0), None, 1, None,
                               ctypes.c_void_p(0x10000), TQ_F32, None)
    assert rc == TQ_ERR_SCRATCH
