"""Seeded synthetic inputs shaped like the pages' workloads.

This module only draws random numbers and rounds the drawn activations to
the input dtype (bf16, nearest-even).  It holds none of the method's
arithmetic: quantization, packing, code-book construction and matmul live in
the HIP library and, independently, in the CPU oracle.  Both consume the
exact bytes produced here.

Every configuration draws from numpy.random.default_rng(seed) with the
configuration's index as the seed, in the order written below.

  ternary_small  Ternary G=64: W fp32 256x256 ~ N(0, 0.02^2); x bf16 1x256.
  routeb_gemv    Route B GEMV: codes uint8 8192x8192 uniform in 0..242;
                 ladder a_i = 0.5^(i-1) u_i, u_i ~ U(0.8, 1.2); alpha 0.02;
                 x bf16 [M, 8192], M in {1, 4}.
  ternary_gemv   Ternary G=64 GEMV: W fp32 14336x4096 ~ N(0, 0.02^2);
                 x bf16 [M, 4096], M in {1, 4, 16}.
  moe_two_plane  Two-plane ternary MoE: 64 experts of W fp32 2048x4096 ~
                 N(0, 0.02^2); 16 tokens x bf16 [16, 4096]; top-8 routing,
                 8 distinct experts per token drawn uniformly.
  routeb_prefill Route B prefill: codes uint8 8192x8192 as routeb_gemv,
                 ladder as routeb_gemv, alpha 0.02, row scales fp16 of
                 U(0.5, 1.5), x bf16 [2048, 8192].

Variants of the Route B layer (their own seeds):

  routeb_encode   fp32 weights for the encoder (seed 5).
  routeb_blocks   codes as routeb_gemv, one ladder per block of 32 rows
                  (each drawn as routeb_gemv's), alpha 0.02 (seed 6).
  routeb_alphabet codes over an alphabet of 60 distinct codes drawn without
                  replacement, letter j (j = 1..60) taken with probability
                  proportional to 1/j: about 75 % of the weights use the 18
                  commonest codes and 94 % the 45 commonest, near the code
                  histogram the Route B page reports (section 8.1); ladder
                  and alpha as routeb_gemv (seed 7).
"""

import numpy as np

CONFIG_NAMES = ("ternary_small", "routeb_gemv", "ternary_gemv",
                "moe_two_plane", "routeb_prefill")


def bf16_bits(a):
    """Nearest-even bf16 bit patterns of finite float32 values."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    return ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)


def _gauss_f32(rng, shape, sigma):
    z = rng.standard_normal(size=shape, dtype=np.float32)
    z *= np.float32(sigma)
    return z


def _x(rng, M, K):
    return bf16_bits(rng.standard_normal(size=(M, K), dtype=np.float32))


def _ladder(rng):
    u = rng.uniform(0.8, 1.2, size=5).astype(np.float32)
    return (u * (np.float32(0.5) ** np.arange(5, dtype=np.float32))).astype(np.float32)


def ternary_small(seed=0, rows=256, K=256, M=1):
    rng = np.random.default_rng(seed)
    W = _gauss_f32(rng, (rows, K), 0.02)
    x = _x(rng, M, K)
    return {"W": W, "x": x, "G": 64}


def routeb_gemv(seed=1, N=8192, K=8192, M=4):
    rng = np.random.default_rng(seed)
    codes = rng.integers(0, 243, size=(N, K), dtype=np.uint8)
    ladder = _ladder(rng)
    x = _x(rng, M, K)
    return {"codes": codes, "ladder": ladder, "alpha": np.float32(0.02), "x": x}


def ternary_gemv(seed=2, N=14336, K=4096, M=16):
    rng = np.random.default_rng(seed)
    W = _gauss_f32(rng, (N, K), 0.02)
    x = _x(rng, M, K)
    return {"W": W, "x": x, "G": 64}


def moe_two_plane(seed=3, E=64, N=2048, K=4096, T=16, top_k=8):
    rng = np.random.default_rng(seed)
    W = _gauss_f32(rng, (E, N, K), 0.02)
    x = _x(rng, T, K)
    ids = np.stack([rng.choice(E, size=top_k, replace=False) for _ in range(T)])
    return {"W": W, "x": x, "ids": ids.astype(np.int32), "G": 64}


def routeb_encode(seed=5, N=8192, K=8192):
    """fp32 weights for the Route B encoder: Gaussian rows whose scales
    spread over two decades (so per-row scales matter), and a ladder."""
    rng = np.random.default_rng(seed)
    row_mag = rng.uniform(0.1, 10.0, size=(N, 1))
    W = (rng.standard_normal((N, K)) * 0.02 * row_mag).astype(np.float32)
    return {"W": W, "ladder": _ladder(rng)}


def routeb_prefill(seed=4, N=8192, K=8192, M=2048):
    rng = np.random.default_rng(seed)
    codes = rng.integers(0, 243, size=(N, K), dtype=np.uint8)
    ladder = _ladder(rng)
    rho = rng.uniform(0.5, 1.5, size=N).astype(np.float16).view(np.uint16)
    x = _x(rng, M, K)
    return {"codes": codes, "ladder": ladder, "alpha": np.float32(0.02),
            "row_scale": rho, "x": x}


def routeb_blocks(seed=6, N=8192, K=8192, M=1, table_rows=32):
    rng = np.random.default_rng(seed)
    codes = rng.integers(0, 243, size=(N, K), dtype=np.uint8)
    nb = -(-N // table_rows)
    ladders = np.stack([_ladder(rng) for _ in range(nb)]) if nb else np.zeros((0, 5), np.float32)
    x = _x(rng, M, K)
    return {"codes": codes, "ladders": ladders, "table_rows": table_rows,
            "alpha": np.float32(0.02), "x": x}


def routeb_alphabet(seed=7, N=8192, K=8192, M=1, n_codes=60):
    rng = np.random.default_rng(seed)
    alphabet = rng.choice(243, size=n_codes, replace=False).astype(np.uint8)
    p = 1.0 / np.arange(1, n_codes + 1)
    p /= p.sum()
    codes = alphabet[rng.choice(n_codes, size=(N, K), p=p)]
    ladder = _ladder(rng)
    x = _x(rng, M, K)
    return {"codes": codes, "ladder": ladder, "alpha": np.float32(0.02), "x": x}
