"""Mean-abs ternary quantizer and five-trits-per-byte package.

Follows "Does your weight format deserve a kernel?" (precisit.com,
pack-unpack-run):

* "Three values and a shared scale": a group of G consecutive weights shares
  s = fp16(mean |W_j|); each weight becomes t_j = clip(round(W_j / s), -1, 1)
  with nearest-even ties; a zero scale gives an all-zero group without
  dividing; the reconstruction is s * t_j (bf16 of it in the page's screen).
* "Five trits in a byte": digits d = t + 1, byte b = d0 + 3 d1 + 9 d2 + 27 d3
  + 81 d4, first digit least significant; bytes 243..255 are rejected and
  padding positions must decode to zero.
* "Count the bytes you actually wrote": every group starts on a byte
  boundary, ceil(G/5) code bytes plus a 2-byte fp16 scale.

Readings taken where the page is silent:

* Groups run along K, inside one row of a row-major [rows, K] matrix.
* A ragged final group (K % G != 0) has n_g < G members: its mean is over the
  n_g members, and its unused trit slots are padding (digit 1, trit 0).  Every
  group, ragged or not, occupies ceil(G/5) bytes.
* The mean is a sequential float64 sum over the group (ascending j) divided by
  n_g in float64, then rounded once to fp16 (never through fp32).
* round() acts on the exact quotient W_j / s.  In float64 the quotient of an
  fp32 weight by an fp16 scale never lands on the 0.5 tie unless it is
  exactly 0.5, so rint of the float64 quotient is that exact rounding.
* Non-finite weights, and a mean that rounds to fp16 infinity (>= 65520),
  are errors ("range"); nothing is clamped.
* Package layout is planar: codes [rows, ng, ceil(G/5)] uint8 and scales
  [rows, ng] fp16 bits.
* Two planes (the FUCINA README, "The method", W ~ d1 T1 + d2 T2): plane 1
  is this quantizer on W, plane 2 is the same quantizer on the residual
  R = fl32(W - s1 t1), one fp32 rounding.
"""

import numpy as np

from .fpround import f64_to_f16_bits, f16_bits_to_f64


class OracleDataError(ValueError):
    """A data error the format defines: kind is "range", "code" or "padding"."""

    def __init__(self, kind, message):
        super().__init__(message)
        self.kind = kind


def bytes_per_group(G):
    """ceil(G/5) code bytes per group ("Count the bytes you actually wrote")."""
    return -(-G // 5)


def bits_per_weight(G):
    """8 (ceil(G/5) + 2) / G: code bytes plus the 2-byte fp16 scale."""
    return 8.0 * (bytes_per_group(G) + 2) / G


def _n_groups(K, G):
    return -(-K // G)


def _members(K, G):
    """n_g for every group of a K-long row."""
    ng = _n_groups(K, G)
    n = np.full(ng, G, dtype=np.int64)
    n[-1] = K - (ng - 1) * G
    return n


def quantize(W, G):
    """W float32 [rows, K] -> (scale fp16 bits [rows, ng], trits int8 [rows, K])."""
    W = np.asarray(W, dtype=np.float32)
    rows, K = W.shape
    if not np.all(np.isfinite(W)):
        raise OracleDataError("range", "non-finite weight")
    ng = _n_groups(K, G)
    n_g = _members(K, G)

    # |W| laid out [rows, ng, G]; the missing slots of a ragged group are 0,
    # and adding 0.0 leaves a float64 sum unchanged.
    A = np.zeros((rows, ng * G), dtype=np.float64)
    A[:, :K] = np.abs(W.astype(np.float64))
    A = A.reshape(rows, ng, G)
    S = np.zeros((rows, ng), dtype=np.float64)
    for j in range(G):                       # sequential sum, j ascending
        S = S + A[:, :, j]
    mean = S / n_g

    s_bits = f64_to_f16_bits(mean)
    s = f16_bits_to_f64(s_bits)
    if np.any(np.isinf(s)):
        raise OracleDataError("range", "group scale overflows fp16")

    s_k = np.repeat(s, G, axis=1)[:, :K]     # the scale of each weight's group
    t = np.zeros((rows, K), dtype=np.int8)
    nz = s_k > 0                             # zero scale: all-zero group
    q = np.rint(W.astype(np.float64)[nz] / s_k[nz])
    t[nz] = np.clip(q, -1, 1).astype(np.int8)
    return s_bits, t


def pack(t, G):
    """trits int8 [rows, K] -> codes uint8 [rows, ng, ceil(G/5)]."""
    t = np.asarray(t, dtype=np.int64)
    rows, K = t.shape
    ng = _n_groups(K, G)
    nb = bytes_per_group(G)
    d = np.ones((rows, ng, nb * 5), dtype=np.int64)       # padding digit 1
    for g, n in enumerate(_members(K, G)):
        d[:, g, :n] = t[:, g * G: g * G + n] + 1
    d = d.reshape(rows, ng, nb, 5)
    b = d[..., 0] + 3 * d[..., 1] + 9 * d[..., 2] + 27 * d[..., 3] + 81 * d[..., 4]
    return b.astype(np.uint8)


def quantize_pack(W, G):
    """W float32 [rows, K] -> (codes uint8 [rows, ng, nb], scales fp16 bits [rows, ng])."""
    s_bits, t = quantize(W, G)
    return pack(t, G), s_bits


def unpack_trits(codes, K, G):
    """codes [rows, ng, nb] -> trits int8 [rows, K]; validates every byte."""
    codes = np.asarray(codes, dtype=np.uint8)
    rows, ng, nb = codes.shape
    if ng != _n_groups(K, G) or nb != bytes_per_group(G):
        raise ValueError("codes shape does not match K and G")
    if np.any(codes > 242):
        raise OracleDataError("code", "byte value 243..255")
    b = codes.astype(np.int64)
    d = np.stack([(b // 3 ** q) % 3 for q in range(5)], axis=-1)
    d = d.reshape(rows, ng, nb * 5)
    t = np.zeros((rows, K), dtype=np.int8)
    for g, n in enumerate(_members(K, G)):
        if np.any(d[:, g, n:] != 1):
            raise OracleDataError("padding", "padding position does not decode to zero")
        t[:, g * G: g * G + n] = d[:, g, :n] - 1
    return t


def unpack(codes, s_bits, K, G):
    """Package -> reconstruction s * t as float64 [rows, K].

    The value is exactly representable in fp32 (an fp16 scale times -1, 0 or
    1); its bf16 form is f64_to_bf16_bits of it.
    """
    t = unpack_trits(codes, K, G)
    s = f16_bits_to_f64(s_bits)
    s_k = np.repeat(s, G, axis=1)[:, :K]
    return s_k * t


def two_plane(W, G):
    """W float32 [rows, K] -> ((codes1, scales1), (codes2, scales2))."""
    W = np.asarray(W, dtype=np.float32)
    s1_bits, t1 = quantize(W, G)
    K = W.shape[1]
    s1_k = np.repeat(f16_bits_to_f64(s1_bits), G, axis=1)[:, :K]
    recon1 = (s1_k * t1).astype(np.float32)              # exact: +-s1 or 0
    R = W - recon1                                        # one fp32 rounding
    s2_bits, t2 = quantize(R, G)
    return (pack(t1, G), s1_bits), (pack(t2, G), s2_bits)
