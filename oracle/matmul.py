"""float64 matmul over decoded weights, and the acceptance bound.

y = x W_hat^T (+ bias) is what every packed matmul computes: the fused LUT
matmul of the Route B paper (section 4.2, "Fused Triton matmul": rho_n on the
accumulator, then the bias), the plain reconstruction matmul of the
pack-unpack-run page, and the expert matmul of the FUCINA README ("Runtime
requirements": the second plane's output is summed with the first inside the
expert FFN, i.e. y = x (d1 T1 + d2 T2)^T).

The acceptance rule compares a result against the float64 reference element
by element:  |y - y_ref| <= 2e-3 * B,  B = sum_k |x_k w_hat_k| (+ |bias|).
The bound is on the matmul's value.  A result stored as bf16 additionally
carries the rounding to that format, at most half a bf16 spacing of the
value (2^-8 |y| in the worst case, more than 2e-3 B whenever |y| is close to
B), so for bf16 outputs that half spacing is added to the allowance.
"""

import numpy as np

from .fpround import bf16_bits_to_f64
from .ternary import unpack

REL_BOUND = 2e-3


def matmul_ref(x_bits, w_hat, bias=None):
    """x bf16 bits [M, K], W_hat float64 [N, K] -> (y_ref, B), both float64 [M, N]."""
    x = bf16_bits_to_f64(x_bits)
    w = np.asarray(w_hat, dtype=np.float64)
    y = x @ w.T
    B = np.abs(x) @ np.abs(w).T
    if bias is not None:
        b = np.asarray(bias, dtype=np.float32).astype(np.float64)
        y = y + b[None, :]
        B = B + np.abs(b)[None, :]
    return y, B


def ternary_weights(K, G, codes1, scales1, codes2=None, scales2=None):
    """W_hat = s1 T1 (+ s2 T2) as float64 [N, K]."""
    w = unpack(codes1, scales1, K, G)
    if codes2 is not None:
        w = w + unpack(codes2, scales2, K, G)
    return w


def grouped_ref(x_bits, expert_ids, weights_of):
    """Grouped expert matmul.

    x bf16 bits [T, K]; expert_ids int [T, top_k]; weights_of(e) -> W_hat_e
    float64 [N, K].  Returns (y_ref, B) float64 [T, top_k, N] with
    y_ref[t, j] = x[t] W_hat_{ids[t, j]}^T.
    """
    ids = np.asarray(expert_ids)
    T, top_k = ids.shape
    y = None
    B = None
    for e in np.unique(ids):
        tt, jj = np.nonzero(ids == e)
        w = weights_of(int(e))
        ye, Be = matmul_ref(np.asarray(x_bits)[tt], w)
        if y is None:
            y = np.zeros((T, top_k, w.shape[0]))
            B = np.zeros((T, top_k, w.shape[0]))
        y[tt, jj] = ye
        B[tt, jj] = Be
    return y, B


def hot_prefix_weights(K, G, N, n_hot, codes1, scales1, codes2=None, scales2=None):
    """weights_of(e) for experts stored hot-first (FUCINA README, "The
    method": hot experts get both planes, cold experts one, and the second
    plane covers the expert prefix 0 .. n_hot - 1).  codes1 / scales1 hold
    every expert's plane 1 ([n_experts * N] rows), codes2 / scales2 the first
    n_hot experts' plane 2 ([n_hot * N] rows)."""
    def weights_of(e):
        r = slice(e * N, (e + 1) * N)
        if e < n_hot:
            return ternary_weights(K, G, codes1[r], scales1[r], codes2[r], scales2[r])
        return ternary_weights(K, G, codes1[r], scales1[r])
    return weights_of


def bf16_half_spacing(v):
    """Half the distance between neighbouring bf16 values around |v|:
    2^(e-8) for 2^e <= |v| < 2^(e+1) (8 significant bits), 2^-134 below the
    normal range."""
    a = np.abs(np.asarray(v, dtype=np.float64))
    _, e2 = np.frexp(a)
    e = np.maximum(e2 - 1, -126)
    return np.ldexp(1.0, e - 8)


def check_bound(y, y_ref, B, rel=REL_BOUND, stored="f32"):
    """Element-wise |y - y_ref| <= rel * B (+ half a bf16 spacing of y_ref when
    the result is stored as bf16), and no NaN or Inf in y."""
    y = np.asarray(y, dtype=np.float64)
    err = np.abs(y - y_ref)
    finite = np.isfinite(y)
    allow = rel * B
    if stored == "bf16":
        # the value rounded was the kernel's fp32 result, within rel*B of y_ref;
        # the wider of the two spacings covers a power-of-two boundary between them
        allow = allow + bf16_half_spacing(np.maximum(np.abs(y_ref), np.abs(y)))
    elif stored != "f32":
        raise ValueError("stored is 'f32' or 'bf16'")
    viol = (~finite) | (err > allow)
    with np.errstate(divide="ignore", invalid="ignore"):
        ratio = np.where(B > 0, err / B, np.where(err > 0, np.inf, 0.0))
    return {
        "ok": not bool(np.any(viol)),
        "violations": int(np.count_nonzero(viol)),
        "nonfinite": int(np.count_nonzero(~finite)),
        "max_err_over_B": float(np.max(ratio)) if ratio.size else 0.0,
    }
