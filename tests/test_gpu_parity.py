"""HIP path against the CPU oracle, element by element, through the C ABI.

Pack and unpack must match bit for bit; matmuls must satisfy
|y - y_ref| <= 2e-3 * sum_k |x_k w_hat_k| for every element (the acceptance
bound of the packed-matmul workloads), with y_ref and the sum in float64.
Inputs are the seeded synthetic workloads of workloads.py and small ragged
shapes around them.  Each GPU step prints its case first.
"""

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


def gpu_pack(dmm, W, G, planes):
    rows, K = W.shape
    cs, ss = dmm.packed_shape(rows, K, G)
    c1 = torch.empty(cs, dtype=torch.uint8, device=DEV)
    s1 = torch.empty(ss, dtype=torch.int16, device=DEV)
    c2 = s2 = None
    if planes == 2:
        c2 = torch.empty(cs, dtype=torch.uint8, device=DEV)
        s2 = torch.empty(ss, dtype=torch.int16, device=DEV)
    st = dmm.tq_pack(dev(W), G, planes, c1, s1, c2, s2)
    out = [host(c1), host(s1).view(np.uint16)]
    if planes == 2:
        out += [host(c2), host(s2).view(np.uint16)]
    return out, int(host(st)[0])


def y_host(y):
    if y.dtype == torch.bfloat16:
        return oracle.bf16_bits_to_f64(host(y.view(torch.int16)).view(np.uint16))
    return host(y).astype(np.float64)


def stored_of(y):
    return "bf16" if y.dtype == torch.bfloat16 else "f32"


def assert_bound(y, y_ref, B, what, stored="f32"):
    r = oracle.check_bound(y, y_ref, B, stored=stored)
    assert r["ok"], f"{what}: {r}"
    return r


# ------------------------------------------------------------------ pack

PACK_CASES = [
    ("ternary_small 256x256", lambda: workloads.ternary_small()["W"], 64, 1),
    ("ragged 37x70 G64", lambda: (np.random.default_rng(1).standard_normal((37, 70)) * 0.02).astype(np.float32), 64, 1),
    ("ragged 5x300 G128", lambda: (np.random.default_rng(2).standard_normal((5, 300)) * 0.02).astype(np.float32), 128, 1),
    ("single group 3x64", lambda: (np.random.default_rng(3).standard_normal((3, 64))).astype(np.float32), 64, 1),
    ("two-plane 64x320", lambda: (np.random.default_rng(4).standard_normal((64, 320)) * 0.02).astype(np.float32), 64, 2),
    ("two-plane ragged 9x200 G128", lambda: (np.random.default_rng(5).standard_normal((9, 200)) * 3).astype(np.float32), 128, 2),
    # many workgroups of 256 (G = 64) or 128 (G = 128) groups: boundaries
    # inside rows and next to ragged last groups
    ("multi-workgroup ragged 300x700 G64", lambda: (np.random.default_rng(6).standard_normal((300, 700)) * 0.02).astype(np.float32), 64, 1),
    ("multi-workgroup ragged 200x1000 G128 two-plane", lambda: (np.random.default_rng(7).standard_normal((200, 1000)) * 0.02).astype(np.float32), 128, 2),
    ("multi-workgroup ragged 129x333 G64 two-plane", lambda: (np.random.default_rng(8).standard_normal((129, 333))).astype(np.float32), 64, 2),
]


@pytest.mark.parametrize("name,make,G,planes", PACK_CASES, ids=[c[0] for c in PACK_CASES])
def test_pack_bit_exact(dmm, name, make, G, planes):
    W = make()
    say(f"tq_pack {name} G={G} planes={planes}")
    got, st = gpu_pack(dmm, W, G, planes)
    assert st == 0
    if planes == 1:
        c, s = oracle.quantize_pack(W, G)
        ref = [c, s]
    else:
        (c1, s1), (c2, s2) = oracle.two_plane(W, G)
        ref = [c1, s1, c2, s2]
    for g, r in zip(got, ref):
        assert np.array_equal(g, r)


def test_pack_special_groups(dmm):
    """Ties, zeros, tiny means, the largest finite scale; then non-finite
    weights and fp16 overflow raise TQ_DATA_RANGE on their group only."""
    W = np.zeros((8, 128), np.float32)
    W[0, :64] = [0.75] * 32 + [-0.25] * 32
    W[1, :64] = 2.0 ** -26
    W[2, :64] = 65519.0
    W[3, 64:] = np.linspace(-1, 1, 64)
    W[4, :] = 1e-30
    W[5, 5] = -0.64
    say("tq_pack special groups")
    got, st = gpu_pack(dmm, W, 64, 2)
    (c1, s1), (c2, s2) = oracle.two_plane(W, 64)
    assert st == 0
    for g, r in zip(got, [c1, s1, c2, s2]):
        assert np.array_equal(g, r)
    for bad, val in (("nan", np.nan), ("inf", np.inf), ("overflow", 65520.0)):
        W2 = W.copy()
        if bad == "overflow":
            W2[6, 64:] = val
        else:
            W2[6, 70] = val
        say(f"tq_pack range error {bad}")
        got, st = gpu_pack(dmm, W2, 64, 1)
        assert st == dmm.TQ_DATA_RANGE
        c, s = oracle.quantize_pack(np.where(np.arange(8)[:, None] == 6, 0, W2).astype(np.float32), 64)
        keep = np.ones((8, 2), bool)
        keep[6, 1] = False
        assert np.array_equal(got[0][keep], c[keep]) and np.array_equal(got[1][keep], s[keep])
        assert np.all(got[0][6, 1] == 121) and got[1][6, 1] == 0


def test_pack_full_ternary_gemv(dmm):
    """14336 x 4096 at G=64, bit-exact over every group."""
    W = workloads.ternary_gemv()["W"]
    say("tq_pack ternary_gemv 14336x4096")
    got, st = gpu_pack(dmm, W, 64, 1)
    c, s = oracle.quantize_pack(W, 64)
    assert st == 0 and np.array_equal(got[0], c) and np.array_equal(got[1], s)


# ------------------------------------------------------------------ unpack

@pytest.mark.parametrize("rows,K,G", [(256, 256, 64), (11, 70, 64), (7, 300, 128), (1, 64, 64),
                                      (300, 700, 64), (200, 1000, 128)])
def test_unpack_bit_exact(dmm, rows, K, G):
    W = (np.random.default_rng(rows + K).standard_normal((rows, K)) * 0.02).astype(np.float32)
    c, s = oracle.quantize_pack(W, G)
    ref = oracle.unpack(c, s, K, G)
    for odt in (torch.float32, torch.bfloat16):
        say(f"tq_unpack {rows}x{K} G={G} {odt}")
        out = torch.empty((rows, K), dtype=odt, device=DEV)
        st = dmm.tq_unpack(dev(c), dev(bits16(s)), rows, K, G, out)
        assert int(host(st)[0]) == 0
        if odt == torch.float32:
            assert np.array_equal(host(out).view(np.uint32), ref.astype(np.float32).view(np.uint32))
        else:
            got = host(out.view(torch.int16)).view(np.uint16)
            assert np.array_equal(got, oracle.f64_to_bf16_bits(ref))


def test_unpack_rejects_bad_bytes(dmm):
    W = (np.random.default_rng(9).standard_normal((4, 128)) * 0.02).astype(np.float32)
    c, s = oracle.quantize_pack(W, 64)
    ref = oracle.unpack(c, s, 128, 64)
    for bad, flag in ((243, 2), (255, 2)):
        c2 = c.copy()
        c2[2, 1, 4] = bad
        out = torch.empty((4, 128), dtype=torch.float32, device=DEV)
        say(f"tq_unpack invalid byte {bad}")
        st = dmm.tq_unpack(dev(c2), dev(bits16(s)), 4, 128, 64, out)
        assert int(host(st)[0]) == flag
        got = host(out)
        mask = np.ones((4, 128), bool)
        mask[2, 64 + 20: 64 + 25] = False
        assert np.array_equal(got[mask], ref[mask].astype(np.float32))
        assert np.all(got[2, 84:89] == 0)
    c3 = c.copy()
    c3[1, 0, 12] += 81                   # padding digit of byte 12 -> 2
    out = torch.empty((4, 128), dtype=torch.float32, device=DEV)
    say("tq_unpack bad padding")
    st = dmm.tq_unpack(dev(c3), dev(bits16(s)), 4, 128, 64, out)
    assert int(host(st)[0]) == 4


@pytest.mark.parametrize("rows,K", [(1, 64), (37, 320), (3, 4096), (129, 1024), (1000, 128)])
def test_unpack_whole_groups(dmm, rows, K):
    """G = 64 with K % 64 == 0 (the wave-per-8-groups kernel): group counts
    that end inside a wave's 8 groups, one group, many workgroups; fp32 and
    bf16 bit-exact against the oracle, and an output view offset by one
    element (not 16-byte aligned) through the general kernel."""
    W = (np.random.default_rng(rows * 7 + K).standard_normal((rows, K)) * 0.02).astype(np.float32)
    W[0, :64] = 0.0                                     # a zero-scale group
    c, s = oracle.quantize_pack(W, 64)
    ref = oracle.unpack(c, s, K, 64)
    for odt in (torch.float32, torch.bfloat16):
        for off in (0, 1):
            say(f"tq_unpack whole groups {rows}x{K} {odt} offset {off}")
            buf = torch.empty(rows * K + off, dtype=odt, device=DEV)
            out = buf[off:]
            st = dmm.tq_unpack(dev(c), dev(bits16(s)), rows, K, 64, out)
            assert int(host(st)[0]) == 0
            if odt == torch.float32:
                got = host(out).reshape(rows, K).view(np.uint32)
                assert np.array_equal(got, ref.astype(np.float32).view(np.uint32))
            else:
                got = host(out.view(torch.int16)).reshape(rows, K).view(np.uint16)
                assert np.array_equal(got, oracle.f64_to_bf16_bits(ref))


def test_unpack_whole_groups_flags_every_byte(dmm):
    """Every code byte position of a G = 64 group, set to an invalid value in
    turn, is reported and decodes to zeros, with the rest of the package
    unchanged; a padding digit is reported in any group of a wave."""
    rows, K = 5, 192                                    # 15 groups: two waves' worth
    W = (np.random.default_rng(17).standard_normal((rows, K)) * 0.02).astype(np.float32)
    c, s = oracle.quantize_pack(W, 64)
    ref = oracle.unpack(c, s, K, 64).astype(np.float32)
    for r, g in ((0, 0), (2, 1), (4, 2)):
        for i in range(13):
            c2 = c.copy()
            c2[r, g, i] = 243 + (i % 13)
            out = torch.empty((rows, K), dtype=torch.float32, device=DEV)
            say(f"tq_unpack whole groups invalid byte {i} of group ({r}, {g})")
            st = dmm.tq_unpack(dev(c2), dev(bits16(s)), rows, K, 64, out)
            assert int(host(st)[0]) == 2
            got = host(out)
            lo, hi = 64 * g + 5 * i, min(64 * g + 5 * i + 5, 64 * (g + 1))
            mask = np.ones((rows, K), bool)
            mask[r, lo:hi] = False
            assert np.array_equal(got[mask], ref[mask])
            assert np.all(got[r, lo:hi] == 0)
    for r, g in ((0, 2), (3, 0), (4, 2)):
        c3 = c.copy()
        c3[r, g, 12] = (c3[r, g, 12] % 81) + 162            # padding digit -> 2
        out = torch.empty((rows, K), dtype=torch.bfloat16, device=DEV)
        say(f"tq_unpack whole groups bad padding in group ({r}, {g})")
        st = dmm.tq_unpack(dev(c3), dev(bits16(s)), rows, K, 64, out)
        assert int(host(st)[0]) == 4


def test_unpack_full_ternary_gemv(dmm):
    """The 14336 x 4096 package of the GEMV workload, bf16 and fp32, bit-exact
    over every element."""
    W = workloads.ternary_gemv()["W"]
    c, s = oracle.quantize_pack(W, 64)
    ref = oracle.unpack(c, s, 4096, 64)
    for odt in (torch.bfloat16, torch.float32):
        say(f"tq_unpack ternary_gemv 14336x4096 {odt}")
        out = torch.empty((14336, 4096), dtype=odt, device=DEV)
        st = dmm.tq_unpack(dev(c), dev(bits16(s)), 14336, 4096, 64, out)
        assert int(host(st)[0]) == 0
        if odt == torch.float32:
            assert np.array_equal(host(out).view(np.uint32), ref.astype(np.float32).view(np.uint32))
        else:
            assert np.array_equal(host(out.view(torch.int16)).view(np.uint16), oracle.f64_to_bf16_bits(ref))


# ------------------------------------------------------------------ tq_matmul

def tq_case(dmm, M, N, K, G, planes, ydt, seed, code_off=0, x_off=0, x_special=False):
    rng = np.random.default_rng(seed)
    W = (rng.standard_normal((N, K)) * 0.02).astype(np.float32)
    xf = rng.standard_normal((M, K)).astype(np.float32)
    if x_special:
        # activations fp16 cannot hold (tiny, huge) in a few chunks, zeros
        # elsewhere, and one row entirely below 2^-17 (its products are the
        # row's whole output, so a chunk left out of the replay would break
        # the bound)
        xf[rng.integers(0, M, 6), rng.integers(0, K, 6)] = 3.0e-7
        xf[rng.integers(0, M, 6), rng.integers(0, K, 6)] = -7.0e4
        xf[rng.integers(0, M, 20), rng.integers(0, K, 20)] = 0.0
        xf[(2 * M) // 3] *= np.float32(1e-7)
    xb = workloads.bf16_bits(xf)
    if planes == 1:
        c1, s1 = oracle.quantize_pack(W, G)
        c2 = s2 = None
    else:
        (c1, s1), (c2, s2) = oracle.two_plane(W, G)
    y_ref, B = oracle.matmul_ref(xb, oracle.ternary_weights(K, G, c1, s1, c2, s2))

    def put_codes(c):
        if c is None:
            return None
        flat = np.concatenate([np.zeros(code_off, np.uint8), c.reshape(-1)])
        return dev(flat)[code_off:]

    xs = np.concatenate([np.zeros(x_off, np.uint16), xb.reshape(-1)])
    xd = dev(bits16(xs))[x_off:].view(M, K)
    y = torch.empty((M, N), dtype=ydt, device=DEV)
    say(f"tq_matmul M={M} N={N} K={K} G={G} planes={planes} y={ydt} off={code_off},{x_off}")
    dmm.tq_matmul(xd, put_codes(c1), dev(bits16(s1)), N, G, y,
                  put_codes(c2), None if s2 is None else dev(bits16(s2)))
    return assert_bound(y_host(y), y_ref, B, f"tq M={M} N={N} K={K}", stored_of(y))


# Shapes of the MFMA prefill form (dense, one or two planes, G = 64, M >= 128):
# one group, ragged M and N tiles, N below one tile, several tiles each way.
TQ_PREFILL_CASES = [
    (128, 256, 64), (130, 300, 128), (300, 257, 320), (256, 1000, 1024), (129, 17, 192),
    (512, 600, 512),
]


@pytest.mark.parametrize("M,N,K", TQ_PREFILL_CASES)
def test_tq_matmul_prefill_shapes(dmm, M, N, K):
    tq_case(dmm, M, N, K, 64, 1, torch.float32, seed=M + 3 * N + K)
    tq_case(dmm, M, N, K, 64, 1, torch.bfloat16, seed=M + 5 * N + K, x_special=True)
    tq_case(dmm, M, N, K, 64, 2, torch.float32, seed=M + 7 * N + K)
    tq_case(dmm, M, N, K, 64, 2, torch.bfloat16, seed=M + 9 * N + K, x_special=True)


def test_tq_matmul_prefill_full(dmm):
    """ternary_gemv weights (14336 x 4096, the oracle's package) at M = 2048
    tokens: every output against the oracle, fp32 output (the bound alone)
    and bf16 output, with and without a workspace."""
    d = workloads.ternary_gemv(M=1)
    c, s = oracle.quantize_pack(d["W"], 64)
    rng = np.random.default_rng(60)
    xb = workloads.bf16_bits(rng.standard_normal((2048, 4096)).astype(np.float32))
    w = oracle.ternary_weights(4096, 64, c, s)
    y_ref, B = oracle.matmul_ref(xb, w)
    xd, cd, sd = dev(bits16(xb)), dev(c), dev(bits16(s))
    for ydt in (torch.float32, torch.bfloat16):
        y = torch.empty((2048, 14336), dtype=ydt, device=DEV)
        say(f"tq_matmul prefill M=2048 N=14336 K=4096 {ydt}")
        dmm.tq_matmul(xd, cd, sd, 14336, 64, y)
        assert_bound(y_host(y), y_ref, B, f"ternary prefill {ydt}", stored_of(y))
    ws = torch.empty(dmm.tq_prefill_workspace_bytes(2048, 4096), dtype=torch.uint8, device=DEV)
    y = torch.empty((2048, 14336), dtype=torch.float32, device=DEV)
    say("tq_matmul_ws prefill M=2048 fp32")
    dmm.tq_matmul_ws(xd, cd, sd, 14336, 64, y, ws)
    assert_bound(y_host(y), y_ref, B, "ternary prefill ws fp32", "f32")


TQ_CASES = [
    (1, 256, 256, 64, 1), (2, 100, 320, 64, 1), (3, 100, 320, 64, 1), (4, 100, 320, 64, 1),
    (5, 100, 320, 64, 1), (8, 33, 192, 64, 1), (16, 64, 512, 64, 1), (17, 40, 256, 64, 1),
    (33, 20, 128, 64, 1), (3, 48, 384, 128, 1), (4, 64, 256, 64, 2), (7, 30, 640, 128, 2),
    (1, 1, 64, 64, 1), (1, 17, 64, 64, 2),
]


@pytest.mark.parametrize("M,N,K,G,planes", TQ_CASES)
def test_tq_matmul_small(dmm, M, N, K, G, planes):
    for ydt in (torch.float32, torch.bfloat16):
        tq_case(dmm, M, N, K, G, planes, ydt, seed=M * 1000 + N + K)


# Shapes of the streaming form (dense, M <= 4, K = 1024 .. 4096): every
# groups-per-row it takes, one and two planes, row counts that leave partial
# 16-row blocks and partial workgroup ranges, and row ranges of 5 to 8 blocks
# (more than the four blocks in flight).
TQ_STREAM_CASES = [
    (1, 1000, 1024, 1), (2, 777, 2048, 2), (3, 300, 3072, 1), (4, 2050, 4096, 2),
    (1, 5, 4096, 1), (4, 4100, 4096, 1), (1, 20000, 1024, 1), (2, 33000, 1024, 1),
    (3, 1, 2048, 2), (2, 20000, 4096, 1), (1, 16400, 4096, 2), (4, 3, 3072, 1),
    # more than four tokens: passes over codes kept in LDS, or the general kernel
    (5, 1000, 1024, 1), (8, 2050, 4096, 2), (12, 4100, 4096, 1), (16, 300, 3072, 1),
    (13, 14336, 4096, 1), (8, 14336, 4096, 1), (16, 20000, 1024, 1), (7, 33000, 1024, 2),
]


@pytest.mark.parametrize("M,N,K,planes", TQ_STREAM_CASES)
def test_tq_matmul_streaming_shapes(dmm, M, N, K, planes):
    for ydt in (torch.float32, torch.bfloat16):
        tq_case(dmm, M, N, K, 64, planes, ydt, seed=7 * M + N + K)


# Shapes of the full-width form (dense, one plane, 5 to 16 tokens, K = 1024,
# 2048 or 4096, super-blocks of 64, 32 or 16 rows): one row, rows that end
# inside a 16-row block and inside a super-block, workgroups of one to many
# super-blocks, and the last row's last group (the last code piece of the
# array is read clamped).
TQ_BATCH_CASES = [
    (5, 1, 1024), (16, 17, 2048), (6, 1000, 1024), (9, 777, 2048), (12, 4100, 4096),
    (16, 70000, 1024), (16, 40000, 4096), (5, 3, 4096), (13, 300, 1024), (7, 16, 2048),
    (16, 14336, 4096), (11, 257, 4096), (16, 65, 1024), (8, 33000, 2048),
]


@pytest.mark.parametrize("M,N,K", TQ_BATCH_CASES)
def test_tq_matmul_batch_shapes(dmm, M, N, K):
    for ydt in (torch.float32, torch.bfloat16):
        tq_case(dmm, M, N, K, 64, 1, ydt, seed=3 * M + N + K)


def test_tq_matmul_batch_extreme_activations(dmm):
    """Activations far outside fp16's range (tiny and huge) and zeros: the
    full-width form multiplies in bf16 against exact 2t, so every value is
    used as it is."""
    for M, N, K in ((16, 300, 1024), (5, 64, 4096)):
        tq_case(dmm, M, N, K, 64, 1, torch.float32, seed=M + K, x_special=True)


@pytest.mark.parametrize("code_off,x_off", [(1, 0), (2, 2), (3, 4), (5, 6), (0, 1), (7, 3)])
def test_tq_matmul_offset_views(dmm, code_off, x_off):
    """Non-zero view offsets of codes (any byte) and x (any element, odd ones
    included: a 2-byte aligned x is accepted)."""
    tq_case(dmm, 3, 50, 320, 64, 2, torch.float32, seed=77, code_off=code_off, x_off=x_off)
    tq_case(dmm, 1, 50, 256, 128, 1, torch.float32, seed=78, code_off=code_off, x_off=x_off)
    tq_case(dmm, 4, 64, 1024, 64, 1, torch.bfloat16, seed=79, code_off=code_off, x_off=x_off)
    tq_case(dmm, 130, 40, 192, 64, 1, torch.float32, seed=80, code_off=code_off, x_off=x_off)


def test_tq_matmul_ternary_gemv_full(dmm):
    """ternary_gemv: 14336 x 4096 at M = 1, 4, 16 on the oracle's package
    (the device pack of the same W is checked bit for bit by the pack tests)."""
    d = workloads.ternary_gemv()
    W, x = d["W"], d["x"]
    c, s = oracle.quantize_pack(W, 64)
    w_hat = oracle.ternary_weights(4096, 64, c, s)
    cd, sd = dev(c), dev(bits16(s))
    for M in (1, 4, 16):
        y_ref, B = oracle.matmul_ref(x[:M], w_hat)
        for ydt in (torch.float32, torch.bfloat16):
            y = torch.empty((M, 14336), dtype=ydt, device=DEV)
            say(f"tq_matmul ternary_gemv M={M} {ydt}")
            dmm.tq_matmul(dev(bits16(x[:M])), cd, sd, 14336, 64, y)
            assert_bound(y_host(y), y_ref, B, f"ternary_gemv M={M}", stored_of(y))


def test_tq_matmul_ternary_small_full(dmm):
    d = workloads.ternary_small()
    c, s = oracle.quantize_pack(d["W"], 64)
    y_ref, B = oracle.matmul_ref(d["x"], oracle.ternary_weights(256, 64, c, s))
    y = torch.empty((1, 256), dtype=torch.float32, device=DEV)
    say("tq_matmul ternary_small")
    dmm.tq_matmul(dev(bits16(d["x"])), dev(c), dev(bits16(s)), 256, 64, y)
    assert_bound(y_host(y), y_ref, B, "ternary_small")


def grouped_case(dmm, E, N, K, T, top_k, planes, seed, bad_ids=False, ydt=torch.float32):
    rng = np.random.default_rng(seed)
    W = (rng.standard_normal((E, N, K)) * 0.02).astype(np.float32)
    xb = workloads.bf16_bits(rng.standard_normal((T, K)).astype(np.float32))
    ids = np.stack([rng.choice(E, top_k, replace=False) for _ in range(T)]).astype(np.int32)
    if bad_ids == "all":
        ids[:] = np.where(np.arange(ids.size).reshape(ids.shape) % 2 == 0, -7, E + 3)
    elif bad_ids:
        ids[1, 0] = E
        ids[2, top_k - 1] = -1
    if planes == 2:
        (c1, s1), (c2, s2) = oracle.two_plane(W.reshape(-1, K), 64)
    else:
        c1, s1 = oracle.quantize_pack(W.reshape(-1, K), 64)
        c2 = s2 = None
    y = torch.empty((T, top_k, N), dtype=ydt, device=DEV)
    say(f"tq_matmul grouped E={E} N={N} K={K} T={T} top_k={top_k} planes={planes} bad={bad_ids} y={ydt}")
    dmm.tq_matmul(dev(bits16(xb)), dev(c1), dev(bits16(s1)), N, 64, y,
                  None if c2 is None else dev(c2), None if s2 is None else dev(bits16(s2)),
                  n_experts=E, expert_ids=dev(ids), top_k=top_k)
    got = y_host(y)

    def w_of(e):
        r = slice(e * N, (e + 1) * N)
        return oracle.ternary_weights(K, 64, c1[r], s1[r],
                                      None if c2 is None else c2[r], None if s2 is None else s2[r])
    valid = (ids >= 0) & (ids < E)
    ids_ok = np.where(valid, ids, 0)
    y_ref, B = oracle.grouped_ref(xb, ids_ok, w_of)
    if valid.any():
        assert_bound(got[valid], y_ref[valid], B[valid], "grouped", stored_of(y))
    assert np.all(np.isnan(got[~valid]))


def test_tq_matmul_grouped_small(dmm):
    grouped_case(dmm, 8, 40, 256, 6, 3, 2, seed=5)
    grouped_case(dmm, 5, 33, 128, 9, 2, 1, seed=6)
    grouped_case(dmm, 8, 40, 256, 6, 3, 2, seed=7, bad_ids=True)
    grouped_case(dmm, 5, 33, 128, 4, 2, 1, seed=8, bad_ids="all", ydt=torch.bfloat16)


def test_tq_matmul_grouped_streaming(dmm):
    """Grouped shapes of the streaming form (K = 1024 .. 4096): experts with
    more than four routed slots (several passes), partial row ranges, tiny N,
    out-of-range expert ids."""
    grouped_case(dmm, 6, 100, 1024, 9, 3, 1, seed=21)
    grouped_case(dmm, 4, 300, 2048, 16, 2, 2, seed=22)
    grouped_case(dmm, 8, 64, 4096, 6, 3, 2, seed=23, bad_ids=True)
    grouped_case(dmm, 3, 17, 3072, 2, 1, 1, seed=24)
    grouped_case(dmm, 4, 40, 1024, 5, 2, 2, seed=25, bad_ids=True, ydt=torch.bfloat16)
    grouped_case(dmm, 4, 40, 1024, 3, 2, 1, seed=26, bad_ids="all")
    # several hundred (token, slot) ids: the routing scan takes them in steps of
    # 256, an expert's first four matches can sit in different 64-id chunks,
    # and every expert needs many passes of four
    grouped_case(dmm, 6, 50, 1024, 100, 4, 1, seed=27, bad_ids=True)
    grouped_case(dmm, 12, 24, 2048, 333, 3, 2, seed=28)


def test_tq_matmul_grouped_heavy_first(dmm):
    """Launches of at most 64 experts and 256 ids take their experts in order
    of passes (heaviest first): idle experts, experts of one to several passes
    and equal pass counts in one launch; 65 experts keep the launch order."""
    grouped_case(dmm, 64, 40, 1024, 30, 8, 1, seed=31)          # 240 ids, 0..9 tokens each
    grouped_case(dmm, 8, 36, 2048, 40, 4, 2, seed=32, bad_ids=True)
    grouped_case(dmm, 64, 24, 1024, 32, 8, 2, seed=33)          # exactly 256 ids
    grouped_case(dmm, 65, 24, 1024, 20, 6, 1, seed=34)


def hot_case(dmm, E, N, K, T, top_k, n_hot, seed, bad_ids=False, ydt=torch.float32):
    """tq_matmul_hot: plane 2 only for experts 0 .. n_hot - 1."""
    rng = np.random.default_rng(seed)
    W = (rng.standard_normal((E * N, K)) * 0.02).astype(np.float32)
    xb = workloads.bf16_bits(rng.standard_normal((T, K)).astype(np.float32))
    ids = np.stack([rng.choice(E, top_k, replace=False) for _ in range(T)]).astype(np.int32)
    if bad_ids:
        ids[0, 0] = -2
        ids[T - 1, top_k - 1] = E
    (c1, s1), (c2, s2) = oracle.two_plane(W, 64)
    c2h, s2h = c2[:n_hot * N], s2[:n_hot * N]
    y = torch.empty((T, top_k, N), dtype=ydt, device=DEV)
    say(f"tq_matmul_hot E={E} N={N} K={K} T={T} top_k={top_k} n_hot={n_hot} bad={bad_ids} y={ydt}")
    dmm.tq_matmul_hot(dev(bits16(xb)), dev(c1), dev(bits16(s1)), N, 64, y, n_hot, E, dev(ids),
                      top_k, None if n_hot == 0 else dev(c2h),
                      None if n_hot == 0 else dev(bits16(s2h)))
    got = y_host(y)
    valid = (ids >= 0) & (ids < E)
    w_of = oracle.hot_prefix_weights(K, 64, N, n_hot, c1, s1, c2h, s2h)
    y_ref, B = oracle.grouped_ref(xb, np.where(valid, ids, 0), w_of)
    assert_bound(got[valid], y_ref[valid], B[valid], f"hot n_hot={n_hot}", stored_of(y))
    assert np.all(np.isnan(got[~valid]))


@pytest.mark.parametrize("K", [256, 1024, 4096])
def test_tq_matmul_hot_prefix(dmm, K):
    """Hot prefixes of every size on the general (K = 256) and streaming
    (K = 1024, 4096) forms, with invalid ids and bf16 output."""
    E, N, T, top_k = 6, 40, 7, 3
    for n_hot in (0, 1, 4, E):
        hot_case(dmm, E, N, K, T, top_k, n_hot, seed=K + n_hot)
    hot_case(dmm, E, N, K, T, top_k, 2, seed=K + 9, bad_ids=True, ydt=torch.bfloat16)


@pytest.mark.parametrize("K", [256, 1024, 4096])
def test_tq_matmul_hot_equals_plain_grouped(dmm, K):
    """tq_matmul_hot against the plain grouped calls on the same ids, bit for
    bit: a (token, slot) of a hot expert equals the two-plane call over all
    experts, one of a cold expert the one-plane call (same per-row
    arithmetic; the hot call only changes which workgroups run which
    experts), and invalid ids are NaN in all three."""
    rng = np.random.default_rng(70 + K)
    E, N, T, top_k, n_hot = 6, 40, 9, 3, 2
    W = (rng.standard_normal((E * N, K)) * 0.02).astype(np.float32)
    xb = dev(bits16(workloads.bf16_bits(rng.standard_normal((T, K)).astype(np.float32))))
    ids = np.stack([rng.choice(E, top_k, replace=False) for _ in range(T)]).astype(np.int32)
    ids[1, 2] = -1
    ids[T - 1, 0] = E + 3
    (c1, s1), (c2, s2) = oracle.two_plane(W, 64)
    c1d, s1d, idd = dev(c1), dev(bits16(s1)), dev(ids)
    yh, y2, y1 = (torch.empty((T, top_k, N), dtype=torch.float32, device=DEV) for _ in range(3))
    say(f"tq_matmul_hot vs plain grouped K={K}")
    dmm.tq_matmul_hot(xb, c1d, s1d, N, 64, yh, n_hot, E, idd, top_k,
                      dev(c2[:n_hot * N]), dev(bits16(s2[:n_hot * N])))
    dmm.tq_matmul(xb, c1d, s1d, N, 64, y2, dev(c2), dev(bits16(s2)), n_experts=E,
                  expert_ids=idd, top_k=top_k)
    dmm.tq_matmul(xb, c1d, s1d, N, 64, y1, n_experts=E, expert_ids=idd, top_k=top_k)
    h, a2, a1 = host(yh), host(y2), host(y1)
    valid = (ids >= 0) & (ids < E)
    hot = valid & (ids < n_hot)
    cold = valid & (ids >= n_hot)
    assert hot.any() and cold.any()
    assert np.array_equal(h[hot], a2[hot])
    assert np.array_equal(h[cold], a1[cold])
    assert np.all(np.isnan(h[~valid])) and np.all(np.isnan(a2[~valid]))


def test_tq_grouped_equals_dense_when_one_expert(dmm):
    """Every (token, slot) routed to expert 2 gives, slot by slot, exactly the
    dense result of expert 2's package (same kernel arithmetic)."""
    rng = np.random.default_rng(12)
    E, N, K, T = 4, 48, 256, 5
    W = (rng.standard_normal((E * N, K)) * 0.02).astype(np.float32)
    xb = workloads.bf16_bits(rng.standard_normal((T, K)).astype(np.float32))
    c, s = oracle.quantize_pack(W, 64)
    ids = np.full((T, 2), 2, np.int32)
    yg = torch.empty((T, 2, N), dtype=torch.float32, device=DEV)
    yd = torch.empty((T, N), dtype=torch.float32, device=DEV)
    say("tq_matmul grouped-vs-dense")
    dmm.tq_matmul(dev(bits16(xb)), dev(c), dev(bits16(s)), N, 64, yg, n_experts=E,
                  expert_ids=dev(ids), top_k=2)
    r = slice(2 * N, 3 * N)
    dmm.tq_matmul(dev(bits16(xb)), dev(c[r]), dev(bits16(s[r])), N, 64, yd)
    g, d = host(yg), host(yd)
    assert np.array_equal(g[:, 0], d) and np.array_equal(g[:, 1], d)


@pytest.fixture(scope="module")
def moe_workload():
    """moe_two_plane (64 experts of 2048 x 4096, 16 tokens, top-8) with the
    oracle's own two planes of every touched expert and the float64
    reference of every (token, slot): two planes, and plane 1 alone (the
    cold experts of a hot prefix).  Experts are independent, so the oracle
    runs them in a thread pool."""
    from concurrent.futures import ThreadPoolExecutor
    d = workloads.moe_two_plane()
    W, x, ids = d["W"], d["x"], d["ids"]
    experts = sorted(set(ids.reshape(-1).tolist()))

    def one(e):
        (c1, s1), (c2, s2) = oracle.two_plane(W[e], 64)
        if e not in experts:
            return e, (c1, s1, c2, s2), None, None, None
        tt, jj = np.nonzero(ids == e)
        ref2 = oracle.matmul_ref(x[tt], oracle.ternary_weights(4096, 64, c1, s1, c2, s2))
        ref1 = oracle.matmul_ref(x[tt], oracle.ternary_weights(4096, 64, c1, s1))
        return e, (c1, s1, c2, s2), (tt, jj), ref2, ref1

    with ThreadPoolExecutor(8) as ex:
        per = {r[0]: r[1:] for r in ex.map(one, range(64))}
    return d, experts, per


def moe_check(got, ids, per, which, what, stored):
    """Every (token, slot) of every touched expert against its reference
    (which: 'two' for two planes, or a set of hot experts)."""
    seen = np.zeros(ids.shape, bool)
    for e, (_, where, ref2, ref1) in per.items():
        if where is None:
            continue
        tt, jj = where
        y_ref, B = ref2 if (which == "two" or e in which) else ref1
        assert_bound(got[tt, jj], y_ref, B, f"{what} expert {e}", stored)
        seen[tt, jj] = True
    assert seen.all()


def test_tq_matmul_moe_every_expert(dmm, moe_workload):
    """moe_two_plane at full size: the device pack of all 64 experts (2 GiB of
    fp32 in one call) matches the oracle's planes bit for bit, and the
    grouped two-plane matmul and
    the hot-prefix call (16 hot experts) are checked against the oracle on
    every (token, slot) of every touched expert, the multi-pass experts
    (more than four tokens) included, with fp32 and bf16 outputs."""
    d, experts, per = moe_workload
    W, x, ids = d["W"], d["x"], d["ids"]
    counts = np.bincount(ids.reshape(-1), minlength=64)
    assert len(experts) == 54 and int(counts.max()) > 4
    (c1, s1, c2, s2), st = gpu_pack(dmm, W.reshape(-1, 4096), 64, 2)
    assert st == 0
    for e, (planes, _, _, _) in per.items():
        rows = slice(e * 2048, (e + 1) * 2048)
        for g, r in zip((c1, s1, c2, s2), planes):
            assert np.array_equal(g[rows], r), f"pack differs on expert {e}"
    xd, idd = dev(bits16(x)), dev(ids)
    c1d, s1d, c2d, s2d = dev(c1), dev(bits16(s1)), dev(c2), dev(bits16(s2))
    for ydt in (torch.float32, torch.bfloat16):
        y = torch.empty((16, 8, 2048), dtype=ydt, device=DEV)
        say(f"tq_matmul moe_two_plane every expert {ydt}")
        dmm.tq_matmul(xd, c1d, s1d, 2048, 64, y, c2d, s2d, n_experts=64, expert_ids=idd, top_k=8)
        moe_check(y_host(y), ids, per, "two", "moe", stored_of(y))
    n_hot = 16
    y = torch.empty((16, 8, 2048), dtype=torch.float32, device=DEV)
    say("tq_matmul_hot moe_two_plane n_hot=16 every expert")
    dmm.tq_matmul_hot(xd, c1d, s1d, 2048, 64, y, n_hot, 64, idd, 8,
                      c2d[:n_hot * 2048], s2d[:n_hot * 2048])
    moe_check(y_host(y), ids, per, set(range(n_hot)), "moe hot", "f32")


# ------------------------------------------------------------------ rb_matmul

def rb_case(dmm, M, N, K, seed, ydt=torch.float32, rho=False, bias=False, code_off=0,
            x_off=0, bad_codes=False, rows=None):
    rng = np.random.default_rng(seed)
    codes = rng.integers(0, 243, (N, K), dtype=np.uint8)
    if bad_codes:
        codes[rng.integers(0, N, 20), rng.integers(0, K, 20)] = 250
    ladder = np.array([1.0, 0.33, 0.115, 0.037, 0.012], np.float32) * rng.uniform(0.8, 1.2)
    table = oracle.rb_table(ladder.astype(np.float32))
    xb = workloads.bf16_bits(rng.standard_normal((M, K)).astype(np.float32))
    rs = rng.uniform(0.5, 1.5, N).astype(np.float16).view(np.uint16) if rho else None
    bs = rng.standard_normal(N).astype(np.float32) if bias else None
    alpha = np.float32(0.02)
    cflat = np.concatenate([np.zeros(code_off, np.uint8), codes.reshape(-1)])
    cd = dev(cflat)[code_off:].view(N, K)
    xs = np.concatenate([np.zeros(x_off, np.uint16), xb.reshape(-1)])
    xd = dev(bits16(xs))[x_off:].view(M, K)
    y = torch.empty((M, N), dtype=ydt, device=DEV)
    say(f"rb_matmul M={M} N={N} K={K} y={ydt} rho={rho} bias={bias} off={code_off},{x_off}")
    dmm.rb_matmul(xd, cd, dev(table), alpha, y, None if rs is None else dev(bits16(rs)),
                  None if bs is None else dev(bs))
    got = y_host(y)
    sel = slice(None) if rows is None else rows
    w = oracle.rb_weights(codes, table, alpha, rs)
    y_ref, B = oracle.matmul_ref(xb[sel], w, bs)
    return assert_bound(got[sel], y_ref, B, f"rb M={M} N={N} K={K}", stored_of(y))


RB_CASES = [
    (1, 64, 64), (1, 100, 1000), (2, 37, 999), (3, 16, 128), (4, 256, 1024), (5, 100, 4096),
    (8, 48, 200), (16, 80, 640), (1, 1, 1), (16, 17, 63),
    (17, 130, 200), (64, 128, 128), (100, 256, 512), (300, 257, 333),
]


@pytest.mark.parametrize("M,N,K", RB_CASES)
def test_rb_matmul_small(dmm, M, N, K):
    rb_case(dmm, M, N, K, seed=M * 7 + N * 3 + K)
    rb_case(dmm, M, N, K, seed=M + N + K, ydt=torch.bfloat16, rho=True, bias=True)


# Shapes of the tiled GEMV form (K % 512 == 0, aligned operands): a single
# tile, an odd number of tiles, ragged N (partial last 16-row block), N < 16,
# every M up to 16, and code 250 (a zero entry) mixed in.
RB_TILED_CASES = [
    (1, 16, 512), (16, 17, 512), (3, 1000, 1536), (7, 33, 2560), (16, 4100, 1024),
    (2, 1, 3584), (12, 250, 5120), (1, 3, 512),
    # 13 to 16 tokens stage the activations in LDS
    (13, 333, 1536), (14, 48, 512), (15, 1000, 2048), (13, 16, 3584),
]


@pytest.mark.parametrize("M,N,K", RB_TILED_CASES)
def test_rb_matmul_tiled_shapes(dmm, M, N, K):
    rb_case(dmm, M, N, K, seed=M * 11 + N + K, bad_codes=True)
    rb_case(dmm, M, N, K, seed=M + 5 * N + K, ydt=torch.bfloat16, rho=True, bias=True)


# Shapes of the wave-local GEMV form (1 to 4 tokens, K % 256 == 0, aligned
# operands): one row quad split over 16 waves (N = 4), 1000 rows (one row
# quad a workgroup), 5000 rows (5 row quads, K split 3 ways unevenly), a
# ragged last workgroup (8190), several row quads a wave (70000 rows), a
# partial last row quad (257) and a single K step (K = 256).
RB_WAVE_CASES = [
    (1, 4, 4096), (2, 1000, 256), (3, 5000, 1792), (4, 8190, 2048), (1, 70000, 256),
    (4, 257, 768), (2, 3, 256),
]


@pytest.mark.parametrize("M,N,K", RB_WAVE_CASES)
def test_rb_matmul_wave_shapes(dmm, M, N, K):
    rb_case(dmm, M, N, K, seed=M * 13 + N + K, bad_codes=True)
    rb_case(dmm, M, N, K, seed=M + 3 * N + K, ydt=torch.bfloat16, rho=True, bias=True)


def test_rb_matmul_wave_per_block_books(dmm):
    """One code book per 32 rows on the wave-local form (a workgroup's rows
    lie in one book): N = 8192 (32 rows a workgroup) and N = 1000 (4)."""
    rng = np.random.default_rng(77)
    for N, K, M in ((8192, 512, 2), (1000, 1024, 4)):
        codes = rng.integers(0, 243, (N, K), dtype=np.uint8)
        nb = -(-N // 32)
        tables = np.stack([oracle.rb_table((S_LADDER * rng.uniform(0.5, 2.0)).astype(np.float32))
                           for _ in range(nb)])
        xb = workloads.bf16_bits(rng.standard_normal((M, K)).astype(np.float32))
        y = torch.empty((M, N), dtype=torch.float32, device=DEV)
        say(f"rb_matmul_blocks wave N={N} K={K} M={M}")
        dmm.rb_matmul_blocks(dev(bits16(xb)), dev(codes), dev(tables.reshape(-1)), 32, 0.02, y)
        w = np.concatenate([oracle.rb_weights(codes[h * 32:(h + 1) * 32], tables[h], np.float32(0.02))
                            for h in range(nb)])
        y_ref, B = oracle.matmul_ref(xb, w)
        assert_bound(y_host(y), y_ref, B, f"blocks wave N={N}")


@pytest.mark.parametrize("code_off,x_off", [(1, 1), (2, 0), (3, 3)])
def test_rb_matmul_offsets_and_bad_codes(dmm, code_off, x_off):
    rb_case(dmm, 4, 50, 256, 31, code_off=code_off, x_off=x_off, bad_codes=True)
    rb_case(dmm, 40, 50, 256, 32, code_off=code_off, x_off=x_off, rho=True)


def rb_custom(dmm, xb, codes, table, alpha, what, ydt=torch.float32):
    """rb_matmul on given bf16 bits, codes and a 243-entry table, against the oracle."""
    M, K = xb.shape
    N = codes.shape[0]
    y = torch.empty((M, N), dtype=ydt, device=DEV)
    say(f"rb_matmul {what} M={M} N={N} K={K} y={ydt}")
    dmm.rb_matmul(dev(bits16(xb)), dev(codes), dev(np.asarray(table, np.float32)),
                  np.float32(alpha), y)
    y_ref, B = oracle.matmul_ref(xb, oracle.rb_weights(codes, table, alpha))
    return assert_bound(y_host(y), y_ref, B, what, stored_of(y))


BOUND_SHAPES = [(4, 64, 512), (40, 64, 512), (300, 130, 320)]   # GEMV and prefill


@pytest.mark.parametrize("M,N,K", BOUND_SHAPES)
def test_rb_matmul_constant_worst_code(dmm, M, N, K):
    """Every weight is the code-book entry whose bf16 rounding is worst
    (relative error 0.0036 > 2e-3 for this ladder) and every activation is
    positive, so no error cancels: the bound must hold by construction."""
    table = oracle.rb_table(np.array([1.0, 0.33, 0.115, 0.037, 0.012], np.float32))
    tb = oracle.bf16_bits_to_f64(oracle.f64_to_bf16_bits(table.astype(np.float64)))
    with np.errstate(divide="ignore", invalid="ignore"):
        rel = np.where(table != 0, np.abs(tb - table) / np.abs(table), 0.0)
    worst = int(np.argmax(rel))
    assert rel[worst] > 2e-3
    rng = np.random.default_rng(M + N + K)
    xb = workloads.bf16_bits(np.abs(rng.standard_normal((M, K))).astype(np.float32))
    codes = np.full((N, K), worst, np.uint8)
    r = rb_custom(dmm, xb, codes, table, 0.02, f"constant code {worst}")
    assert r["max_err_over_B"] < 1e-3


@pytest.mark.parametrize("M,N,K", BOUND_SHAPES)
def test_rb_matmul_activations_outside_fp16(dmm, M, N, K):
    """Activations fp16 cannot hold exactly (above 65280, below 2^-17, far
    below, exact zeros) scattered through x, one row entirely huge and one
    entirely below 2^-17."""
    rng = np.random.default_rng(3 * M + K)
    x = rng.standard_normal((M, K)).astype(np.float32)
    specials = np.array([1e5, -7e4, 3e-6, -1e-30, 0.0, 65536.0, 2.0 ** -17, 1e30],
                        np.float32)
    idx = rng.integers(0, M * K, 40)
    x.reshape(-1)[idx] = specials[rng.integers(0, len(specials), 40)]
    x[M // 2] *= np.float32(1e6)
    if M // 3 != M // 2:
        x[M // 3] *= np.float32(1e-7)
    xb = workloads.bf16_bits(x)
    codes = rng.integers(0, 243, (N, K), dtype=np.uint8)
    table = oracle.rb_table(np.array([1.0, 0.33, 0.115, 0.037, 0.012], np.float32))
    rb_custom(dmm, xb, codes, table, 0.02, "activations outside fp16")
    rb_custom(dmm, xb, codes, table, 0.02, "activations outside fp16", torch.bfloat16)


@pytest.mark.parametrize("M,N,K", BOUND_SHAPES)
def test_rb_matmul_wide_code_book(dmm, M, N, K):
    """A code book spanning more than fp16's range (1e30 next to 1e-30)."""
    rng = np.random.default_rng(5 * M + N)
    table = oracle.rb_table(np.array([1.0, 0.33, 0.115, 0.037, 0.012], np.float32)).copy()
    table[0], table[1], table[2] = 1e30, -1e-30, 3e-9
    xb = workloads.bf16_bits(rng.standard_normal((M, K)).astype(np.float32))
    codes = rng.integers(0, 243, (N, K), dtype=np.uint8)
    rb_custom(dmm, xb, codes, table, 0.5, "wide code book")


def test_rb_matmul_routeb_gemv_full(dmm):
    """routeb_gemv: N = K = 8192 at M = 1, 4 and 16 (direct and LDS-staged
    activations), fp32 and bf16 outputs."""
    d = workloads.routeb_gemv(M=16)
    table = dmm.rb_table(d["ladder"])
    w = oracle.rb_weights(d["codes"], oracle.rb_table(d["ladder"]), d["alpha"])
    cd, td = dev(d["codes"]), dev(table)
    for M in (1, 4, 16):
        y_ref, B = oracle.matmul_ref(d["x"][:M], w)
        for ydt in (torch.float32, torch.bfloat16):
            y = torch.empty((M, 8192), dtype=ydt, device=DEV)
            say(f"rb_matmul routeb_gemv M={M} {ydt}")
            dmm.rb_matmul(dev(bits16(d["x"][:M])), cd, td, d["alpha"], y)
            assert_bound(y_host(y), y_ref, B, f"routeb_gemv M={M}", stored_of(y))


def test_rb_matmul_routeb_prefill_full(dmm):
    """routeb_prefill: M = 2048, K = N = 8192 with row scales; every output
    against the oracle, fp32 output (the bound alone) and bf16 output, with
    and without a workspace."""
    d = workloads.routeb_prefill()
    table = dmm.rb_table(d["ladder"])
    w = oracle.rb_weights(d["codes"], oracle.rb_table(d["ladder"]), d["alpha"], d["row_scale"])
    y_ref, B = oracle.matmul_ref(d["x"], w)
    xd, cd, td, rsd = dev(bits16(d["x"])), dev(d["codes"]), dev(table), dev(bits16(d["row_scale"]))
    for ydt in (torch.float32, torch.bfloat16):
        y = torch.empty((2048, 8192), dtype=ydt, device=DEV)
        say(f"rb_matmul routeb_prefill M=2048 {ydt}")
        dmm.rb_matmul(xd, cd, td, d["alpha"], y, rsd)
        assert_bound(y_host(y), y_ref, B, f"routeb_prefill {ydt}", stored_of(y))
    ws = torch.empty(dmm.rb_prefill_workspace_bytes(2048, 8192), dtype=torch.uint8, device=DEV)
    y = torch.empty((2048, 8192), dtype=torch.float32, device=DEV)
    say("rb_matmul_ws routeb_prefill M=2048 fp32")
    dmm.rb_matmul_ws(xd, cd, td, 0, float(d["alpha"]), y, ws, rsd)
    assert_bound(y_host(y), y_ref, B, "routeb_prefill ws fp32", "f32")


# ------------------------------------------------------------------ misc

def test_zero_sizes_and_empty_k(dmm):
    say("zero sizes")
    y = torch.full((2, 3), 7.0, dtype=torch.float32, device=DEV)
    x = torch.zeros((0, 64), dtype=torch.bfloat16, device=DEV)
    dmm.tq_matmul(x, torch.zeros(3 * 13, dtype=torch.uint8, device=DEV),
                  torch.zeros(3, dtype=torch.int16, device=DEV), 3, 64,
                  torch.empty((0, 3), dtype=torch.float32, device=DEV))
    # K = 0: y = 0 (ternary) and y = bias (Route B)
    x0 = torch.zeros((2, 0), dtype=torch.bfloat16, device=DEV)
    dmm.tq_matmul(x0, torch.zeros(0, dtype=torch.uint8, device=DEV),
                  torch.zeros(0, dtype=torch.int16, device=DEV), 3, 64, y)
    assert np.all(host(y) == 0)
    bias = torch.tensor([1.0, -2.0, 3.0], device=DEV)
    tbl = torch.zeros(243, dtype=torch.float32, device=DEV)
    dmm.rb_matmul(x0, torch.zeros((3, 0), dtype=torch.uint8, device=DEV), tbl, 0.5, y, None, bias)
    assert np.array_equal(host(y), np.array([[1.0, -2.0, 3.0]] * 2, np.float32))
    # K = 0 at a prefill size (M > 16)
    say("prefill K = 0")
    y40 = torch.full((40, 3), 7.0, dtype=torch.float32, device=DEV)
    dmm.rb_matmul(torch.zeros((40, 0), dtype=torch.bfloat16, device=DEV),
                  torch.zeros((3, 0), dtype=torch.uint8, device=DEV), tbl, 0.5, y40, None, bias)
    assert np.array_equal(host(y40), np.array([[1.0, -2.0, 3.0]] * 40, np.float32))


def test_bit_determinism(dmm):
    """Two runs of every kernel family give identical bits (fixed-order
    reductions, no atomics on the accumulation path): dense ternary GEMV
    (wave-local form at 4 tokens, full-width form at 9), grouped two-plane
    experts, the hot
    prefix, the ternary prefill (with and without a workspace), the Route B
    GEMV and prefill, per-block code books, 7-bit indices, the packer and
    the encoder."""
    rng = np.random.default_rng(99)
    W = (rng.standard_normal((300, 1024)) * 0.02).astype(np.float32)
    c, s = oracle.quantize_pack(W, 64)
    E, NE = 6, 64
    WE = (rng.standard_normal((E * NE, 1024)) * 0.02).astype(np.float32)
    (e1, f1), (e2, f2) = oracle.two_plane(WE, 64)
    ids = np.stack([rng.choice(E, 3, replace=False) for _ in range(9)]).astype(np.int32)
    xb = dev(bits16(workloads.bf16_bits(rng.standard_normal((200, 1024)).astype(np.float32))))
    codes_np = rng.integers(0, 243, (300, 1024), dtype=np.uint8)
    codes = dev(codes_np)
    tbl = dev(oracle.rb_table(np.array([1, .3, .1, .03, .01], np.float32)))
    tables = dev(np.stack([oracle.rb_table(np.array([1, .3, .1, .03, .01], np.float32) * (1 + i / 10))
                           for i in range(10)]))
    used_np = np.zeros(128, np.uint8)
    used_np[:100] = np.arange(100, dtype=np.uint8) * 2
    used_np[100:] = 121
    small = rng.integers(0, 128, (300, 1024)).astype(np.uint8)
    c7 = dev(oracle.pack7(small))
    used = dev(used_np)
    Wd = dev(W)
    say("determinism")
    outs = []
    for _ in range(2):
        got = []

        def f32(*shape):
            t = torch.empty(shape, dtype=torch.float32, device=DEV)
            got.append(t)
            return t
        dmm.tq_matmul(xb[:4], dev(c), dev(bits16(s)), 300, 64, f32(4, 300))
        dmm.tq_matmul(xb[:9], dev(c), dev(bits16(s)), 300, 64, f32(9, 300))
        dmm.tq_matmul(xb[:9], dev(e1), dev(bits16(f1)), NE, 64, f32(9, 3, NE), dev(e2),
                      dev(bits16(f2)), n_experts=E, expert_ids=dev(ids), top_k=3)
        dmm.tq_matmul_hot(xb[:9], dev(e1), dev(bits16(f1)), NE, 64, f32(9, 3, NE), 2, E,
                          dev(ids), 3, dev(e2[:2 * NE]), dev(bits16(f2[:2 * NE])))
        dmm.tq_matmul(xb[:200], dev(c), dev(bits16(s)), 300, 64, f32(200, 300))
        ws = torch.empty(dmm.tq_prefill_workspace_bytes(200, 1024), dtype=torch.uint8, device=DEV)
        dmm.tq_matmul_ws(xb[:200], dev(c), dev(bits16(s)), 300, 64, f32(200, 300), ws)
        dmm.rb_matmul(xb[:4], codes, tbl, 0.02, f32(4, 300))
        dmm.rb_matmul(xb[:40], codes, tbl, 0.02, f32(40, 300))
        dmm.rb_matmul_blocks(xb[:4], codes, tables, 32, 0.02, f32(4, 300))
        dmm.rb_matmul_blocks(xb[:40], codes, tables, 32, 0.02, f32(40, 300))
        dmm.rb_matmul7(xb[:4], c7, 300, used, tbl, 0, 0.02, f32(4, 300))
        dmm.rb_matmul7(xb[:40], c7, 300, used, tbl, 0, 0.02, f32(40, 300))
        cs, ss = dmm.packed_shape(300, 1024, 64)
        pc = torch.empty(cs, dtype=torch.uint8, device=DEV)
        ps = torch.empty(ss, dtype=torch.int16, device=DEV)
        dmm.tq_pack(Wd, 64, 1, pc, ps)
        got += [pc, ps]
        ec = torch.empty((300, 1024), dtype=torch.uint8, device=DEV)
        ea = torch.empty(301, dtype=torch.float32, device=DEV)
        er = torch.empty(300, dtype=torch.float16, device=DEV)
        dmm.rb_encode(Wd, np.array([1, .3, .1, .03, .01], np.float32), ec, ea, row_scale=er)
        got += [ec, ea, er]
        outs.append([host(t).view(np.uint8) for t in got])
    for i, (a, b) in enumerate(zip(*outs)):
        assert np.array_equal(a, b), f"output {i} differs between two runs"


# ------------------------------------------------------------------ rb_encode

S0_LADDER = np.array([1, 1 / 3, 1 / 9, 1 / 27, 1 / 81], np.float32)
S_LADDER = np.array([1.0, 0.33, 0.115, 0.037, 0.012], np.float32)


def encode_case(dmm, W, ladder, zeta=0.0, per_row=False, rho_rows=None):
    """rb_encode on the device, bit for bit against the oracle's encoder
    (codes, alpha, block scales, rho)."""
    N, K = W.shape
    b = (1 if per_row else 0) if rho_rows is None else rho_rows
    nb = -(-N // b) if b > 0 else 0
    say(f"rb_encode N={N} K={K} zeta={zeta} rho_rows={b}")
    codes = torch.empty((N, K), dtype=torch.uint8, device=DEV)
    alpha = torch.empty(1 + nb, dtype=torch.float32, device=DEV)
    rs = torch.empty(nb, dtype=torch.float16, device=DEV) if b > 0 else None
    st = dmm.rb_encode(dev(W), ladder, codes, alpha, zeta=zeta, row_scale=rs,
                       rho_rows=b if b > 0 else None)
    assert int(host(st)[0]) == 0
    c_ref, a_ref, r_ref = oracle.rb_encode(W, ladder, zeta=zeta, rho_rows=b)
    got = host(codes)
    assert np.array_equal(got, c_ref), f"{int(np.count_nonzero(got != c_ref))} codes differ"
    a_got = host(alpha).view(np.uint32)
    assert a_got[0] == np.float32(a_ref).view(np.uint32)
    if b > 0:
        assert np.array_equal(a_got[1:], oracle.rb_block_scales(W, b).view(np.uint32))
        assert np.array_equal(host(rs.view(torch.int16)).view(np.uint16), r_ref)
    return codes, alpha, rs


def encode_inputs(N, K, seed):
    """Gaussian weights with per-row magnitudes spread over two decades, plus
    exact ladder points and half-way points of the first step (ties)."""
    rng = np.random.default_rng(seed)
    W = (rng.standard_normal((N, K)) * 0.02 * rng.uniform(0.1, 10.0, (N, 1))).astype(np.float32)
    if N * K >= 8:
        a = float(np.abs(W).max())
        flat = W.reshape(-1)
        idx = rng.choice(flat.size, min(flat.size // 4, 64), replace=False)
        flat[idx[0::2]] = np.float32(a / 2) * rng.choice([-1, 1], idx[0::2].size)
        flat[idx[1::2]] = np.float32(a / 3) * rng.choice([-1, 1], idx[1::2].size)
    return W


# (3, 16384) is the longest row encoded in one pass with per-row scales;
# (2, 16400) takes the two-pass form
ENCODE_SHAPES = [(1, 1), (3, 70), (17, 1000), (64, 4096), (300, 257), (3, 16384), (2, 16400)]


@pytest.mark.parametrize("N,K", ENCODE_SHAPES)
def test_rb_encode_shapes(dmm, N, K):
    W = encode_inputs(N, K, seed=N + K)
    for lad in (S0_LADDER, S_LADDER):
        for per_row in (False, True):
            encode_case(dmm, W, lad, zeta=0.0, per_row=per_row)
    encode_case(dmm, W, S_LADDER, zeta=0.8, per_row=True)
    encode_case(dmm, W, S0_LADDER, zeta=1.0, per_row=False)
    for b in (2, 16, N + 3):                         # head blocks, one ragged, one oversized
        encode_case(dmm, W, S_LADDER, rho_rows=b)


def test_rb_encode_worked_examples_and_ties(dmm):
    """The hand-worked words (tie at |r| = s_1 / 2 goes to 0), and a matrix
    made only of ladder points and midpoints."""
    W = np.array([[0.9, -0.5, 1.0, 0.0]], np.float32)
    for zeta in (0.0, 1.0):
        codes, _, _ = encode_case(dmm, W, S0_LADDER, zeta=zeta)
        want = [194, 81, 202, 121] if zeta == 0 else [161, 81, 202, 121]
        assert list(host(codes)[0]) == want
    pts = np.array([0.5, -0.5, 1 / 6, -1 / 6, 1 / 3, 2 / 3, 1.0, -1.0, 1 / 162, 0.0], np.float32)
    encode_case(dmm, np.tile(pts, (5, 3)), S0_LADDER)


def test_rb_encode_zero_rows_empty_and_bad_values(dmm):
    W = np.zeros((6, 40), np.float32)
    W[2] = np.linspace(-1, 1, 40, dtype=np.float32)
    encode_case(dmm, W, S_LADDER, per_row=True)
    encode_case(dmm, np.zeros((3, 5), np.float32), S_LADDER, per_row=True)
    # K = 0: alpha = 0, rho = 0 for every row; N = 0: only alpha
    alpha = torch.full((5,), 7.0, dtype=torch.float32, device=DEV)
    rs = torch.full((4,), 1.0, dtype=torch.float16, device=DEV)
    say("rb_encode K=0")
    dmm.rb_encode(torch.empty((4, 0), dtype=torch.float32, device=DEV), S_LADDER,
                  torch.empty((4, 0), dtype=torch.uint8, device=DEV), alpha, row_scale=rs)
    assert np.all(host(alpha) == 0.0) and np.all(host(rs.view(torch.int16)) == 0)
    say("rb_encode N=0")
    alpha = torch.full((1,), 7.0, dtype=torch.float32, device=DEV)
    dmm.rb_encode(torch.empty((0, 8), dtype=torch.float32, device=DEV), S_LADDER,
                  torch.empty((0, 8), dtype=torch.uint8, device=DEV), alpha)
    assert float(host(alpha)[0]) == 0.0
    for bad in (np.nan, np.inf):
        W2 = encode_inputs(5, 33, seed=9)
        W2[3, 7] = bad
        codes = torch.empty((5, 33), dtype=torch.uint8, device=DEV)
        alpha = torch.empty(1, dtype=torch.float32, device=DEV)
        say(f"rb_encode non-finite {bad}")
        st = dmm.rb_encode(dev(W2), S_LADDER, codes, alpha)
        assert int(host(st)[0]) & 1
        alpha = torch.empty(6, dtype=torch.float32, device=DEV)
        rs = torch.empty(5, dtype=torch.float16, device=DEV)
        say(f"rb_encode non-finite {bad}, per-row scales")
        st = dmm.rb_encode(dev(W2), S_LADDER, codes, alpha, row_scale=rs)
        assert int(host(st)[0]) & 1


def test_rb_encode_then_matmul(dmm):
    """Section 3.3 end to end: encode W on the device, then rb_matmul with
    the device's codes, alpha and rho against the oracle's W_hat."""
    N, K, M = 200, 768, 5
    W = encode_inputs(N, K, seed=31)
    rng = np.random.default_rng(32)
    xb = workloads.bf16_bits(rng.standard_normal((M, K)).astype(np.float32))
    codes, alpha, rs = encode_case(dmm, W, S_LADDER, per_row=True)
    table = oracle.rb_table(S_LADDER)
    a = float(host(alpha)[0])
    y = torch.empty((M, N), dtype=torch.float32, device=DEV)
    dmm.rb_matmul(dev(bits16(xb)), codes, dev(table), np.float32(a), y, rs)
    c_ref, a_ref, r_ref = oracle.rb_encode(W, S_LADDER, per_row=True)
    w = oracle.rb_weights(c_ref, table, a_ref, r_ref)
    y_ref, B = oracle.matmul_ref(xb, w)
    assert_bound(y_host(y), y_ref, B, "encode then matmul")


@pytest.mark.parametrize("M", [3, 40])
def test_rb_encode_heads_then_matmul(dmm, M):
    """Section 8.2 per-head prosody end to end: encode with one scale per
    block of 64 rows (a ragged last head), then rb_matmul with rho_rows = 64
    on the GEMV (M = 3) and prefill (M = 40) paths, against the oracle's
    W_hat with rho_{n // 64}."""
    N, K, b = 300, 512, 64
    W = encode_inputs(N, K, seed=50 + M)
    rng = np.random.default_rng(51)
    xb = workloads.bf16_bits(rng.standard_normal((M, K)).astype(np.float32))
    codes, alpha, rs = encode_case(dmm, W, S_LADDER, rho_rows=b)
    table = oracle.rb_table(S_LADDER)
    a = float(host(alpha)[0])
    bs = rng.standard_normal(N).astype(np.float32)
    for ydt in (torch.float32, torch.bfloat16):
        y = torch.empty((M, N), dtype=ydt, device=DEV)
        say(f"rb_matmul rho_rows={b} M={M} y={ydt}")
        dmm.rb_matmul(dev(bits16(xb)), codes, dev(table), np.float32(a), y, rs, dev(bs),
                      rho_rows=b)
        c_ref, a_ref, r_ref = oracle.rb_encode(W, S_LADDER, rho_rows=b)
        w = oracle.rb_weights(c_ref, table, a_ref, r_ref, rho_rows=b)
        y_ref, B = oracle.matmul_ref(xb, w, bs)
        assert_bound(y_host(y), y_ref, B, f"heads M={M}", stored_of(y))


def test_rb_matmul_rho_block_tiled_gemv(dmm):
    """Block scales on the tiled GEMV path (K % 512 == 0, aligned): random
    fp16 head scales for blocks of 256 rows, N = 1000 (ragged last head)."""
    N, K, M, b = 1000, 1024, 2, 256
    rng = np.random.default_rng(52)
    codes = rng.integers(0, 243, (N, K), dtype=np.uint8)
    table = oracle.rb_table(S_LADDER)
    rho = rng.uniform(0.05, 1.0, -(-N // b)).astype(np.float16).view(np.uint16)
    xb = workloads.bf16_bits(rng.standard_normal((M, K)).astype(np.float32))
    y = torch.empty((M, N), dtype=torch.float32, device=DEV)
    say("rb_matmul tiled rho_rows=256")
    dmm.rb_matmul(dev(bits16(xb)), dev(codes), dev(table), np.float32(0.02), y,
                  dev(bits16(rho)), rho_rows=b)
    w = oracle.rb_weights(codes, table, np.float32(0.02), rho, rho_rows=b)
    y_ref, B = oracle.matmul_ref(xb, w)
    assert_bound(y_host(y), y_ref, B, "tiled rho_rows")


def test_rb_encode_large(dmm):
    """4096 x 4096 Gaussian weights, per-row and global scales."""
    W = encode_inputs(4096, 4096, seed=41)
    encode_case(dmm, W, S_LADDER, per_row=True)
    encode_case(dmm, W, S0_LADDER, per_row=False)


def test_rb_encode_routeb_encode_full(dmm):
    """routeb_encode at full size (8192 x 8192 with per-row scales, the timed
    encoder workload): codes, alpha, the row maxima and rho bit for bit."""
    d = workloads.routeb_encode()
    encode_case(dmm, d["W"], d["ladder"], per_row=True)


# ----------------------------------------------- prefill with a workspace

def ws_case(dmm, xb, codes, tables, table_rows, what, rs=None, rho_rows=1, ydt=torch.float32):
    """rb_matmul_ws against the oracle, and bit for bit against the same call
    without a workspace (the pre-pass converts and flags exactly what the
    kernel would)."""
    M, K = xb.shape
    N = codes.shape[0]
    xd, cd, td = dev(bits16(xb)), dev(codes), dev(tables.reshape(-1))
    rsd = None if rs is None else dev(bits16(rs))
    ws = torch.empty(dmm.rb_prefill_workspace_bytes(M, K), dtype=torch.uint8, device=DEV)
    ws.fill_(0xA5)                                   # contents on entry do not matter
    y_ws = torch.empty((M, N), dtype=ydt, device=DEV)
    y_no = torch.empty((M, N), dtype=ydt, device=DEV)
    say(f"rb_matmul_ws {what} M={M} N={N} K={K} table_rows={table_rows} y={ydt}")
    dmm.rb_matmul_ws(xd, cd, td, table_rows, 0.02, y_ws, ws, rsd, None, rho_rows)
    dmm.rb_matmul_blocks(xd, cd, td, table_rows, 0.02, y_no, rsd, None, rho_rows)
    a, b = host(y_ws.view(torch.int16) if ydt == torch.bfloat16 else y_ws), \
        host(y_no.view(torch.int16) if ydt == torch.bfloat16 else y_no)
    assert np.array_equal(a, b), f"{what}: workspace and in-kernel conversion differ"
    if table_rows:
        blocks = [oracle.rb_weights(codes[h * table_rows:(h + 1) * table_rows], tables[h], np.float32(0.02),
                                    None if rs is None else rs[h * table_rows // rho_rows:])
                  for h in range(-(-N // table_rows))] if rho_rows == 1 or rs is None else None
        w = np.concatenate(blocks) if blocks is not None else None
    else:
        w = oracle.rb_weights(codes, tables.reshape(243), np.float32(0.02),
                              None if rs is None else np.repeat(rs, rho_rows)[:N])
    if w is not None:
        y_ref, B = oracle.matmul_ref(xb, w)
        assert_bound(y_host(y_ws), y_ref, B, f"ws {what}", stored_of(y_ws))


WS_SHAPES = [(17, 64, 64), (40, 50, 320), (300, 130, 512), (256, 520, 1024), (513, 96, 4128)]


@pytest.mark.parametrize("M,N,K", WS_SHAPES)
def test_rb_matmul_ws_shapes(dmm, M, N, K):
    """Ragged M (partial 256-row blocks), K not a multiple of the pre-pass's
    128 columns, fp32 and bf16 outputs, row scales."""
    rng = np.random.default_rng(M + 7 * K)
    xb = workloads.bf16_bits(rng.standard_normal((M, K)).astype(np.float32))
    codes = rng.integers(0, 243, (N, K), dtype=np.uint8)
    table = oracle.rb_table(np.array([1.0, 0.33, 0.115, 0.037, 0.012], np.float32))
    rs = rng.uniform(0.5, 1.5, N).astype(np.float16).view(np.uint16)
    ws_case(dmm, xb, codes, table, 0, "gaussian")
    ws_case(dmm, xb, codes, table, 0, "gaussian, row scales", rs=rs, ydt=torch.bfloat16)


@pytest.mark.parametrize("M,N,K", [(300, 64, 512), (40, 96, 1024)])
def test_rb_matmul_ws_activations_outside_fp16(dmm, M, N, K):
    """Chunks fp16 cannot hold (huge, tiny, a whole huge row, a whole tiny
    row) are flagged by the pre-pass and replayed in bf16, as the in-kernel
    conversion does."""
    rng = np.random.default_rng(5 * M + K)
    x = rng.standard_normal((M, K)).astype(np.float32)
    specials = np.array([1e5, -7e4, 3e-6, -1e-30, 0.0, 65536.0, 2.0 ** -17, 1e30], np.float32)
    idx = rng.integers(0, M * K, 40)
    x.reshape(-1)[idx] = specials[rng.integers(0, len(specials), 40)]
    x[M // 2] *= np.float32(1e6)
    x[M // 3] *= np.float32(1e-7)
    xb = workloads.bf16_bits(x)
    codes = rng.integers(0, 243, (N, K), dtype=np.uint8)
    table = oracle.rb_table(np.array([1.0, 0.33, 0.115, 0.037, 0.012], np.float32))
    ws_case(dmm, xb, codes, table, 0, "outside fp16")
    ws_case(dmm, xb, codes, table, 0, "outside fp16", ydt=torch.bfloat16)


def test_rb_matmul_ws_blocks_small_m_and_errors(dmm):
    """Per-block code books with a workspace; M <= 16 ignores it; a short
    workspace is refused."""
    rng = np.random.default_rng(91)
    M, N, K = 100, 96, 512
    xb = workloads.bf16_bits(rng.standard_normal((M, K)).astype(np.float32))
    codes = rng.integers(0, 243, (N, K), dtype=np.uint8)
    tables = np.stack([oracle.rb_table((np.array([1.0, 0.33, 0.115, 0.037, 0.012]) *
                                        rng.uniform(0.8, 1.2)).astype(np.float32)) for _ in range(3)])
    ws_case(dmm, xb, codes, tables, 32, "per-block books")
    xs = dev(bits16(xb[:4]))
    ws = torch.empty(dmm.rb_prefill_workspace_bytes(4, K), dtype=torch.uint8, device=DEV)
    y1 = torch.empty((4, N), dtype=torch.float32, device=DEV)
    y2 = torch.empty((4, N), dtype=torch.float32, device=DEV)
    say("rb_matmul_ws M=4 (GEMV)")
    dmm.rb_matmul_ws(xs, dev(codes), dev(tables.reshape(-1)), 32, 0.02, y1, ws)
    dmm.rb_matmul_blocks(xs, dev(codes), dev(tables.reshape(-1)), 32, 0.02, y2)
    assert torch.equal(y1, y2)
    short = torch.empty(dmm.rb_prefill_workspace_bytes(M, K) - 4, dtype=torch.uint8, device=DEV)
    with pytest.raises(Exception):
        dmm.rb_matmul_ws(dev(bits16(xb)), dev(codes), dev(tables.reshape(-1)), 32, 0.02,
                         torch.empty((M, N), dtype=torch.float32, device=DEV), short)


def test_rb_matmul_ws_routeb_prefill_full(dmm):
    """routeb_prefill (M = 2048, N = K = 8192, row scales) with a workspace:
    bit for bit the in-kernel conversion's result."""
    d = workloads.routeb_prefill()
    M, K = d["x"].shape
    N = d["codes"].shape[0]
    xd, cd, td = dev(bits16(d["x"])), dev(d["codes"]), dev(dmm.rb_table(d["ladder"]))
    rsd = dev(bits16(d["row_scale"]))
    ws = torch.empty(dmm.rb_prefill_workspace_bytes(M, K), dtype=torch.uint8, device=DEV)
    y_ws = torch.empty((M, N), dtype=torch.bfloat16, device=DEV)
    y_no = torch.empty((M, N), dtype=torch.bfloat16, device=DEV)
    say("rb_matmul_ws routeb_prefill M=2048")
    dmm.rb_matmul_ws(xd, cd, td, 0, float(d["alpha"]), y_ws, ws, rsd)
    dmm.rb_matmul(xd, cd, td, float(d["alpha"]), y_no, rsd)
    assert torch.equal(y_ws.view(torch.int16), y_no.view(torch.int16))


def tq_ws_case(dmm, M, N, K, planes, ydt, seed, x_special=False):
    """tq_matmul_ws against the oracle, and bit for bit against tq_matmul."""
    rng = np.random.default_rng(seed)
    W = (rng.standard_normal((N, K)) * 0.02).astype(np.float32)
    xf = rng.standard_normal((M, K)).astype(np.float32)
    if x_special:
        xf[rng.integers(0, M, 6), rng.integers(0, K, 6)] = 3.0e-7
        xf[rng.integers(0, M, 6), rng.integers(0, K, 6)] = -7.0e4
        xf[rng.integers(0, M, 20), rng.integers(0, K, 20)] = 0.0
        xf[M // 2] *= np.float32(1e6)
        xf[M // 3] *= np.float32(1e-7)
    xb = workloads.bf16_bits(xf)
    if planes == 1:
        c1, s1 = oracle.quantize_pack(W, 64)
        c2 = s2 = None
    else:
        (c1, s1), (c2, s2) = oracle.two_plane(W, 64)
    xd = dev(bits16(xb))
    args = (dev(c1), dev(bits16(s1)), N, 64)
    extra = (None if c2 is None else dev(c2), None if s2 is None else dev(bits16(s2)))
    ws = torch.empty(dmm.tq_prefill_workspace_bytes(M, K), dtype=torch.uint8, device=DEV)
    ws.fill_(0x5A)                                   # contents on entry do not matter
    y_ws = torch.empty((M, N), dtype=ydt, device=DEV)
    y_no = torch.empty((M, N), dtype=ydt, device=DEV)
    say(f"tq_matmul_ws M={M} N={N} K={K} planes={planes} y={ydt} special={x_special}")
    dmm.tq_matmul_ws(xd, *args, y_ws, ws, *extra)
    dmm.tq_matmul(xd, *args, y_no, *extra)
    v = (lambda t: t.view(torch.int16)) if ydt == torch.bfloat16 else (lambda t: t)
    assert torch.equal(v(y_ws), v(y_no)), "workspace and in-kernel conversion differ"
    y_ref, B = oracle.matmul_ref(xb, oracle.ternary_weights(K, 64, c1, s1, c2, s2))
    assert_bound(y_host(y_ws), y_ref, B, f"tq ws M={M} N={N} K={K}", stored_of(y_ws))


@pytest.mark.parametrize("M,N,K", TQ_PREFILL_CASES + [(1000, 96, 4160)])
def test_tq_matmul_ws_shapes(dmm, M, N, K):
    """The prefill shapes with a workspace, one and two planes, activations
    fp16 cannot hold (one whole row among them)."""
    tq_ws_case(dmm, M, N, K, 1, torch.float32, seed=M + 11 * N + K)
    tq_ws_case(dmm, M, N, K, 2, torch.bfloat16, seed=M + 13 * N + K, x_special=True)


def test_tq_matmul_ws_small_m_and_errors(dmm):
    """M below the prefill ignores the workspace; a short one is refused."""
    rng = np.random.default_rng(77)
    M, N, K = 8, 40, 256
    W = (rng.standard_normal((N, K)) * 0.02).astype(np.float32)
    c, s = oracle.quantize_pack(W, 64)
    xd = dev(bits16(workloads.bf16_bits(rng.standard_normal((M, K)).astype(np.float32))))
    ws = torch.empty(dmm.tq_prefill_workspace_bytes(M, K), dtype=torch.uint8, device=DEV)
    y1 = torch.empty((M, N), dtype=torch.float32, device=DEV)
    y2 = torch.empty((M, N), dtype=torch.float32, device=DEV)
    say("tq_matmul_ws M=8")
    dmm.tq_matmul_ws(xd, dev(c), dev(bits16(s)), N, 64, y1, ws)
    dmm.tq_matmul(xd, dev(c), dev(bits16(s)), N, 64, y2)
    assert torch.equal(y1, y2)
    short = torch.empty(dmm.tq_prefill_workspace_bytes(M, K) - 8, dtype=torch.uint8, device=DEV)
    with pytest.raises(Exception):
        dmm.tq_matmul_ws(xd, dev(c), dev(bits16(s)), N, 64, y1, short)


def test_tq_matmul_ws_prefill_full(dmm):
    """ternary_gemv weights at M = 2048 with a workspace: bit for bit the
    in-kernel conversion's result."""
    d = workloads.ternary_gemv(M=1)
    c, s = oracle.quantize_pack(d["W"], 64)
    rng = np.random.default_rng(60)
    xd = dev(bits16(workloads.bf16_bits(rng.standard_normal((2048, 4096)).astype(np.float32))))
    ws = torch.empty(dmm.tq_prefill_workspace_bytes(2048, 4096), dtype=torch.uint8, device=DEV)
    y_ws = torch.empty((2048, 14336), dtype=torch.bfloat16, device=DEV)
    y_no = torch.empty((2048, 14336), dtype=torch.bfloat16, device=DEV)
    say("tq_matmul_ws prefill M=2048 N=14336 K=4096")
    dmm.tq_matmul_ws(xd, dev(c), dev(bits16(s)), 14336, 64, y_ws, ws)
    dmm.tq_matmul(xd, dev(c), dev(bits16(s)), 14336, 64, y_no)
    assert torch.equal(y_ws.view(torch.int16), y_no.view(torch.int16))
