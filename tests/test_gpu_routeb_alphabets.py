"""Route B section 8.1 (7-bit truncated alphabet) and section 8.3 (one code
book per block of rows) on the HIP path, against the CPU oracle through the
C ABI: rb_truncate bit for bit, rb_matmul_blocks and rb_matmul7 within the
matmul bound |y - y_ref| <= 2e-3 * sum_k |x_k w_hat_k|.  Each GPU step prints
its case first."""

import numpy as np
import pytest

import oracle
import workloads

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def say(msg):
    print(f"[case] {msg}", flush=True)


@pytest.fixture(scope="module")
def dmm():
    import decode_matmul_amd
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return decode_matmul_amd


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def host(t):
    torch.cuda.synchronize()
    return t.cpu().numpy()


def bits16(a):
    return np.ascontiguousarray(a).view(np.int16)


def y_host(y):
    if y.dtype == torch.bfloat16:
        return oracle.bf16_bits_to_f64(host(y.view(torch.int16)).view(np.uint16))
    return host(y).astype(np.float64)


def assert_bound(y, y_ref, B, what, ydt):
    r = oracle.check_bound(y, y_ref, B, stored="bf16" if ydt == torch.bfloat16 else "f32")
    assert r["ok"], f"{what}: {r}"
    return r


def offset_dev(a, off):
    """Device copy of a uint8 array starting `off` bytes into its allocation."""
    flat = np.concatenate([np.zeros(off, np.uint8), np.ascontiguousarray(a).reshape(-1)])
    return dev(flat)[off:].view(*a.shape)


def block_ladders(rng, nb, spread):
    """One ladder per block, as the workloads draw them; with spread, block
    h is also scaled by 2^(4 (h % 5) - 8) so that the books' magnitudes
    differ by up to 2^16."""
    lad = np.stack([(rng.uniform(0.8, 1.2, 5) * 0.5 ** np.arange(5)).astype(np.float32)
                    for _ in range(max(nb, 1))])
    if spread:
        lad = (lad * (2.0 ** (4 * (np.arange(len(lad)) % 5) - 8))[:, None]).astype(np.float32)
    return lad[:nb] if nb else lad[:1]


def tables_pair(dmm, ladders):
    """(device-side input from the library's rb_table, oracle's tables)."""
    lib = np.stack([dmm.rb_table(a) for a in ladders]).astype(np.float32)
    ref = np.stack([oracle.rb_table(a) for a in ladders]).astype(np.float32)
    return lib, ref


# ------------------------------------------------------------ per-block books

def blocks_case(dmm, M, N, K, table_rows, seed, ydt=torch.float32, rho_rows=0, bias=False,
                spread=True, code_off=0, rows=None):
    rng = np.random.default_rng(seed)
    codes = rng.integers(0, 243, (N, K), dtype=np.uint8)
    nb = -(-N // table_rows) if table_rows else 1
    lib_t, ref_t = tables_pair(dmm, block_ladders(rng, nb, spread))
    xb = workloads.bf16_bits(rng.standard_normal((M, K)).astype(np.float32))
    rs = None
    if rho_rows:
        rs = rng.uniform(0.5, 1.5, -(-N // rho_rows)).astype(np.float16).view(np.uint16)
    bs = rng.standard_normal(N).astype(np.float32) if bias else None
    alpha = np.float32(0.02)
    y = torch.empty((M, N), dtype=ydt, device=DEV)
    say(f"rb_matmul_blocks M={M} N={N} K={K} table_rows={table_rows} y={ydt} "
        f"rho_rows={rho_rows} bias={bias} off={code_off}")
    dmm.rb_matmul_blocks(dev(bits16(xb)), offset_dev(codes, code_off), dev(lib_t), table_rows,
                         alpha, y, None if rs is None else dev(bits16(rs)),
                         None if bs is None else dev(bs), max(rho_rows, 1))
    got = y_host(y)
    sel = slice(None) if rows is None else rows
    w = oracle.rb_weights(codes, ref_t if table_rows else ref_t[0], alpha, rs, max(rho_rows, 1),
                          table_rows)
    y_ref, B = oracle.matmul_ref(xb[sel], w, bs)
    return assert_bound(got[sel], y_ref, B, f"blocks M={M} N={N} K={K}", ydt)


# GEMV tiled (K % 512 == 0), GEMV general, prefill aligned and not; books of
# 32, 64 and 96 rows; ragged last blocks
BLOCK_CASES = [
    (1, 100, 1024, 32), (16, 4100, 1024, 64), (4, 33, 512, 32), (3, 70, 300, 32),
    (1, 1, 1, 32), (40, 300, 320, 32), (300, 257, 333, 32), (256, 520, 512, 96),
    (130, 64, 64, 32), (17, 1000, 256, 32),
]


@pytest.mark.parametrize("M,N,K,table_rows", BLOCK_CASES)
def test_rb_matmul_blocks_shapes(dmm, M, N, K, table_rows):
    blocks_case(dmm, M, N, K, table_rows, seed=M * 13 + N + K)
    blocks_case(dmm, M, N, K, table_rows, seed=M + 3 * N + K, ydt=torch.bfloat16,
                rho_rows=1, bias=True)


def test_rb_matmul_blocks_offsets_and_heads(dmm):
    """Unaligned code pointers (general kernels) and head-block row scales."""
    blocks_case(dmm, 4, 96, 512, 32, 41, code_off=3)
    blocks_case(dmm, 60, 96, 512, 32, 42, code_off=1, rho_rows=32)
    blocks_case(dmm, 2, 200, 1024, 64, 43, rho_rows=50)


def test_rb_matmul_blocks_one_book_is_rb_matmul(dmm):
    """table_rows = 0 (one book) gives rb_matmul's bits, on the GEMV and the
    prefill kernels; equal books for every block give them too."""
    rng = np.random.default_rng(44)
    N, K = 300, 1024
    codes = dev(rng.integers(0, 243, (N, K), dtype=np.uint8))
    table = dmm.rb_table(block_ladders(rng, 1, False)[0])
    for M in (4, 40):
        xb = dev(bits16(workloads.bf16_bits(rng.standard_normal((M, K)).astype(np.float32))))
        say(f"rb_matmul_blocks one book M={M}")
        y0 = torch.empty((M, N), dtype=torch.float32, device=DEV)
        dmm.rb_matmul(xb, codes, dev(table), 0.02, y0)
        y1 = torch.empty_like(y0)
        dmm.rb_matmul_blocks(xb, codes, dev(table), 0, 0.02, y1)
        y2 = torch.empty_like(y0)
        dmm.rb_matmul_blocks(xb, codes, dev(np.tile(table, (-(-N // 32), 1))), 32, 0.02, y2)
        a = host(y0).view(np.uint32)
        assert np.array_equal(a, host(y1).view(np.uint32))
        assert np.array_equal(a, host(y2).view(np.uint32))


def test_rb_matmul_blocks_routeb_blocks_full(dmm):
    """routeb_blocks: N = K = 8192, one ladder per 32 rows, M = 1 and 4, and
    the M = 2048 prefill; every output against the oracle."""
    d = workloads.routeb_blocks(M=2048)
    lib_t, ref_t = tables_pair(dmm, d["ladders"])
    w = oracle.rb_weights(d["codes"], ref_t, d["alpha"], table_rows=32)
    cd, td = dev(d["codes"]), dev(lib_t)
    for M in (1, 4):
        y = torch.empty((M, 8192), dtype=torch.bfloat16, device=DEV)
        say(f"rb_matmul_blocks routeb_blocks M={M}")
        dmm.rb_matmul_blocks(dev(bits16(d["x"][:M])), cd, td, 32, d["alpha"], y)
        y_ref, B = oracle.matmul_ref(d["x"][:M], w)
        assert_bound(y_host(y), y_ref, B, f"routeb_blocks M={M}", torch.bfloat16)
    y = torch.empty((2048, 8192), dtype=torch.bfloat16, device=DEV)
    say("rb_matmul_blocks routeb_blocks M=2048")
    dmm.rb_matmul_blocks(dev(bits16(d["x"])), cd, td, 32, d["alpha"], y)
    y_ref, B = oracle.matmul_ref(d["x"], w)
    assert_bound(y_host(y), y_ref, B, "routeb_blocks M=2048", torch.bfloat16)


# ------------------------------------------------------------ rb_truncate

def alphabet_codes(rng, N, K, n_codes):
    alphabet = rng.choice(243, n_codes, replace=False).astype(np.uint8)
    return alphabet[rng.integers(0, n_codes, (N, K))]


def gpu_truncate(dmm, codes, code_off=0):
    N, K = codes.shape
    used = torch.empty(128, dtype=torch.uint8, device=DEV)
    n_used = torch.empty(1, dtype=torch.int32, device=DEV)
    c7 = torch.empty((N, dmm.rb7_row_bytes(K)), dtype=torch.uint8, device=DEV)
    st = dmm.rb_truncate(offset_dev(codes, code_off), used, n_used, c7)
    return host(used), int(host(n_used)[0]), host(c7), int(host(st)[0])


TRUNC_CASES = [(40, 70, 45, 0), (5, 1, 1, 0), (3, 3, 2, 0), (17, 1000, 128, 1), (300, 1024, 60, 0),
               (64, 8192, 100, 3), (1, 5, 5, 2)]


@pytest.mark.parametrize("N,K,n_codes,code_off", TRUNC_CASES)
def test_rb_truncate_bit_exact(dmm, N, K, n_codes, code_off):
    rng = np.random.default_rng(N * 7 + K + n_codes)
    codes = alphabet_codes(rng, N, K, n_codes)
    say(f"rb_truncate N={N} K={K} codes={n_codes} off={code_off}")
    used, n_used, c7, st = gpu_truncate(dmm, codes, code_off)
    r_used, r_n, r_index = oracle.rb_truncate(codes)
    assert st == 0
    assert n_used == r_n
    assert np.array_equal(used, r_used)
    assert np.array_equal(c7, oracle.pack7(r_index))


def test_rb_truncate_errors_and_empty(dmm):
    rng = np.random.default_rng(71)
    say("rb_truncate too many codes")
    codes = rng.integers(0, 243, (50, 400), dtype=np.uint8)        # all 243 codes
    _, n_used, _, st = gpu_truncate(dmm, codes)
    assert n_used == len(np.unique(codes)) and st == dmm.TQ_DATA_ALPHABET
    say("rb_truncate non-code byte")
    codes = alphabet_codes(rng, 8, 64, 10)
    codes[3, 7] = 250
    _, n_used, _, st = gpu_truncate(dmm, codes)
    assert st & dmm.TQ_DATA_CODE and n_used == 10
    say("rb_truncate empty")
    used, n_used, c7, st = gpu_truncate(dmm, np.zeros((0, 16), np.uint8))
    assert st == 0 and n_used == 0 and (used == 121).all() and c7.size == 0
    used, n_used, _, st = gpu_truncate(dmm, np.zeros((4, 0), np.uint8))
    assert st == 0 and n_used == 0 and (used == 121).all()


def test_rb_truncate_routeb_alphabet_full(dmm):
    """routeb_alphabet (8192 x 8192, 60 codes): list and count exact, 64
    sampled rows of indices bit for bit (the first and last included)."""
    d = workloads.routeb_alphabet()
    say("rb_truncate routeb_alphabet")
    used, n_used, c7, st = gpu_truncate(dmm, d["codes"])
    r_used, r_n, r_index = oracle.rb_truncate(d["codes"])
    assert st == 0 and n_used == r_n == 60 and np.array_equal(used, r_used)
    rows = np.sort(np.random.default_rng(2).choice(8192, 64, replace=False))
    rows[0], rows[-1] = 0, 8191
    assert np.array_equal(c7[rows], oracle.pack7(r_index[rows]))


# ------------------------------------------------------------ rb_matmul7

def m7_case(dmm, M, N, K, seed, table_rows=0, ydt=torch.float32, rho_rows=0, bias=False,
            code_off=0, x_off=0, n_codes=60, garbage_used=False, rows=None):
    rng = np.random.default_rng(seed)
    codes = alphabet_codes(rng, N, K, n_codes)
    used, n_used, index = oracle.rb_truncate(codes)
    if garbage_used:
        used = used.copy()
        used[n_used:] = rng.integers(0, 256, 128 - n_used)          # read through, never used
        used[0] = 250                                                 # a non-code: reads zero
    packed = oracle.pack7(index)
    nb = -(-N // table_rows) if table_rows else 1
    lib_t, ref_t = tables_pair(dmm, block_ladders(rng, nb, table_rows > 0))
    xb = workloads.bf16_bits(rng.standard_normal((M, K)).astype(np.float32))
    rs = None
    if rho_rows:
        rs = rng.uniform(0.5, 1.5, -(-N // rho_rows)).astype(np.float16).view(np.uint16)
    bs = rng.standard_normal(N).astype(np.float32) if bias else None
    alpha = np.float32(0.02)
    xs = np.concatenate([np.zeros(x_off, np.uint16), xb.reshape(-1)])
    xd = dev(bits16(xs))[x_off:].view(M, K)
    y = torch.empty((M, N), dtype=ydt, device=DEV)
    say(f"rb_matmul7 M={M} N={N} K={K} table_rows={table_rows} y={ydt} rho_rows={rho_rows} "
        f"bias={bias} off={code_off},{x_off}")
    dmm.rb_matmul7(xd, offset_dev(packed, code_off), N, dev(used), dev(lib_t), table_rows,
                   alpha, y, None if rs is None else dev(bits16(rs)),
                   None if bs is None else dev(bs), max(rho_rows, 1))
    got = y_host(y)
    sel = slice(None) if rows is None else rows
    w = oracle.rb_weights7(packed, K, used, ref_t if table_rows else ref_t[0], alpha, rs,
                           max(rho_rows, 1), table_rows)
    y_ref, B = oracle.matmul_ref(xb[sel], w, bs)
    return assert_bound(got[sel], y_ref, B, f"m7 M={M} N={N} K={K}", ydt)


# tiled GEMV (K % 512 == 0, one or an odd number of tiles), plain GEMV,
# prefill with 28-byte slices (K % 32 == 0) and element-wise prefill
M7_CASES = [
    (1, 16, 512), (2, 40, 1536), (16, 17, 2048), (3, 1000, 3072), (7, 33, 1024), (4, 4100, 1024),
    (1, 3, 5120), (1, 64, 64), (2, 37, 999), (16, 17, 63), (5, 100, 1000), (1, 1, 1),
    (17, 130, 256), (64, 128, 128), (256, 520, 1024), (300, 257, 320), (40, 50, 333),
    (100, 256, 500),
]


@pytest.mark.parametrize("M,N,K", M7_CASES)
def test_rb_matmul7_shapes(dmm, M, N, K):
    m7_case(dmm, M, N, K, seed=M * 5 + N + 3 * K)
    m7_case(dmm, M, N, K, seed=M + N + K, table_rows=32, ydt=torch.bfloat16, rho_rows=1,
            bias=True, n_codes=128)


# the two-block form (16 waves on two 16-row blocks, taken when the row
# blocks are at least twice the compute units): an odd block count (the last
# workgroup's second block lies past N), N ending inside a block, one book,
# 32- and 64-row books (both blocks share one), and a row count just below
# the two-block form
M7_PAIR_CASES = [(1, 8208, 512, 0), (3, 8208, 1024, 32), (16, 8200, 512, 0), (4, 8192, 1024, 64),
                 (2, 8000, 512, 64)]


@pytest.mark.parametrize("M,N,K,table_rows", M7_PAIR_CASES)
def test_rb_matmul7_two_blocks(dmm, M, N, K, table_rows):
    m7_case(dmm, M, N, K, seed=M + N + 7 * K + table_rows, table_rows=table_rows)
    m7_case(dmm, M, N, K, seed=2 * M + N + K, table_rows=table_rows, ydt=torch.bfloat16,
            rho_rows=1, bias=True, n_codes=128)


def test_rb_matmul7_offsets_heads_and_list_entries(dmm):
    """Unaligned index rows and activations, head-block scales, and a list
    whose unused entries hold arbitrary bytes (index 0 names code 250)."""
    m7_case(dmm, 4, 64, 1024, 51, code_off=1)
    m7_case(dmm, 4, 64, 1024, 52, x_off=1, table_rows=64)
    m7_case(dmm, 40, 64, 1024, 53, code_off=2, rho_rows=32)
    m7_case(dmm, 4, 64, 1024, 56, code_off=4)        # 4-byte aligned: plain GEMV
    m7_case(dmm, 40, 64, 1024, 57, code_off=4)       # 4-byte aligned: sliced prefill
    m7_case(dmm, 2, 300, 2048, 54, garbage_used=True, n_codes=20)
    m7_case(dmm, 100, 300, 256, 55, garbage_used=True, n_codes=20, table_rows=32)


def test_rb_truncate_then_matmul7(dmm):
    """The device chain rb_truncate -> rb_matmul7 (no host round trip) on the
    GEMV and prefill kernels, against the oracle's weights of the code bytes."""
    rng = np.random.default_rng(61)
    N, K = 200, 2048
    codes_h = alphabet_codes(rng, N, K, 60)
    lad = block_ladders(rng, 1, False)[0]
    table = dev(dmm.rb_table(lad))
    used = torch.empty(128, dtype=torch.uint8, device=DEV)
    n_used = torch.empty(1, dtype=torch.int32, device=DEV)
    c7 = torch.empty((N, dmm.rb7_row_bytes(K)), dtype=torch.uint8, device=DEV)
    say("rb_truncate then rb_matmul7")
    st = dmm.rb_truncate(dev(codes_h), used, n_used, c7)
    assert int(host(st)[0]) == 0
    w = oracle.rb_weights(codes_h, oracle.rb_table(lad), np.float32(0.02))
    for M in (1, 16, 64):
        xb = workloads.bf16_bits(rng.standard_normal((M, K)).astype(np.float32))
        y = torch.empty((M, N), dtype=torch.float32, device=DEV)
        dmm.rb_matmul7(dev(bits16(xb)), c7, N, used, table, 0, 0.02, y)
        y_ref, B = oracle.matmul_ref(xb, w)
        assert_bound(y_host(y), y_ref, B, f"chain M={M}", torch.float32)


def test_rb_matmul7_zero_k(dmm):
    say("rb_matmul7 K = 0")
    bias = torch.tensor([1.0, -2.0, 3.0], device=DEV)
    tbl = torch.zeros(243, dtype=torch.float32, device=DEV)
    used = torch.full((128,), 121, dtype=torch.uint8, device=DEV)
    for M in (2, 40):
        y = torch.full((M, 3), 7.0, dtype=torch.float32, device=DEV)
        dmm.rb_matmul7(torch.zeros((M, 0), dtype=torch.bfloat16, device=DEV),
                       torch.zeros((3, 0), dtype=torch.uint8, device=DEV), 3, used, tbl, 0, 0.5,
                       y, None, bias)
        assert np.array_equal(host(y), np.array([[1.0, -2.0, 3.0]] * M, np.float32))


def test_rb_matmul7_routeb_alphabet_full(dmm):
    """routeb_alphabet: N = K = 8192 over 60 codes, M = 1 and 4, and the
    M = 2048 prefill; every output against the oracle."""
    d = workloads.routeb_alphabet(M=2048)
    used, n_used, index = oracle.rb_truncate(d["codes"])
    packed = oracle.pack7(index)
    table = dmm.rb_table(d["ladder"])
    w = oracle.rb_weights7(packed, 8192, used, oracle.rb_table(d["ladder"]), d["alpha"])
    cd, ud, td = dev(packed), dev(used), dev(table)
    for M in (1, 4):
        y = torch.empty((M, 8192), dtype=torch.bfloat16, device=DEV)
        say(f"rb_matmul7 routeb_alphabet M={M}")
        dmm.rb_matmul7(dev(bits16(d["x"][:M])), cd, 8192, ud, td, 0, d["alpha"], y)
        y_ref, B = oracle.matmul_ref(d["x"][:M], w)
        assert_bound(y_host(y), y_ref, B, f"routeb_alphabet M={M}", torch.bfloat16)
    y = torch.empty((2048, 8192), dtype=torch.bfloat16, device=DEV)
    say("rb_matmul7 routeb_alphabet M=2048")
    dmm.rb_matmul7(dev(bits16(d["x"])), cd, 8192, ud, td, 0, d["alpha"], y)
    y_ref, B = oracle.matmul_ref(d["x"], w)
    assert_bound(y_host(y), y_ref, B, "routeb_alphabet M=2048", torch.bfloat16)
