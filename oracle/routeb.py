"""Route B: 5-step ternary words, the 243-entry code book and decoding.

Follows "A Discrete Weight Language for Large Language Models: Compressing
Gemma 4 31B with a 5-Step Ternary Route":

* section 3.2: a weight is W_hat[n, k] = alpha * sum_{i=1..5} c_i s_i with a
  word c in {-1, 0, +1}^5; the 3^5 = 243 words are enumerated once per layer
  into a look-up table and the weight is stored as the word's index
  codes[n, k] in {0..242}, the base-3 encoding of c_1..c_5;
* section 3.3: with a per-row scale, W_hat[n, k] = rho_n * alpha * LUT entry,
  rho_n stored in fp16;
* section 4.1: one code per byte (uint8), one fp32 alpha per layer.

Readings taken where the page is silent:

* c_1 is the most significant base-3 digit: codes = sum_i (c_i + 1) 3^(5-i).
  Under the balanced ladder S0 = (1, 1/3, 1/9, 1/27, 1/81) this makes the
  table increasing in the code.
* Table entry T[b] = sum_i c_i a_i is evaluated as a float64 sum in the order
  i = 1..5 and rounded once to fp32.  For ladders whose entries span less
  than 2**29 in magnitude (every ladder on the pages) that float64 sum is
  exact, so T[b] is the nearest fp32 of the exact sum.
* alpha (fp32) and rho_n (fp16) are separate inputs; the weight is the
  float64 product alpha * T[b] * rho_n.
* Bytes 243..255 are not code words: the table is padded with zeros to 256.
"""

import numpy as np

from .fpround import f16_bits_to_f64, f64_to_f32


def code_words():
    """int8 [243, 5]: row b is (c_1, ..., c_5) of code b, c_1 most significant."""
    b = np.arange(243, dtype=np.int64)
    cols = [(b // 3 ** (5 - i)) % 3 - 1 for i in range(1, 6)]
    return np.stack(cols, axis=1).astype(np.int8)


def rb_table(ladder):
    """ladder a_1..a_5 (float32) -> code book T float32 [243]."""
    a = np.asarray(ladder, dtype=np.float32).astype(np.float64)
    if a.shape != (5,):
        raise ValueError("the ladder has five steps")
    c = code_words().astype(np.float64)
    acc = np.zeros(243, dtype=np.float64)
    for i in range(5):                       # float64 sum, i = 1..5
        acc = acc + c[:, i] * a[i]
    return f64_to_f32(acc)


def rb_weights(codes, table, alpha, row_scale_bits=None):
    """codes uint8 [N, K] -> W_hat float64 [N, K] = alpha * T[code] * rho_n."""
    codes = np.asarray(codes, dtype=np.uint8)
    t256 = np.zeros(256, dtype=np.float64)
    t256[:243] = np.asarray(table, dtype=np.float32).astype(np.float64)
    w = float(np.float32(alpha)) * t256[codes]
    if row_scale_bits is not None:
        rho = f16_bits_to_f64(row_scale_bits)
        w = w * rho[:, None]
    return w
