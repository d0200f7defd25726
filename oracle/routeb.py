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

The encoder (rb_encode) follows section 3.1 (the greedy 5-step word: each
step picks the c in {-1, 0, +1} closest to the residual, then subtracts
c * s_i; r_0 = x / alpha with alpha the largest |W| of the matrix; a zero-bias
zeta forces c_i = 0 while |r_{i-1}| < zeta * s_i) and section 3.3 (per-row
scale: r_0 = W[n, k] / alpha_n with alpha_n the row's largest |W|, and
rho_n = alpha_n / alpha stored in fp16).  Readings where the page is silent:

* The steps run in float64: r_0 is the float64 quotient of the fp32 weight
  by the fp32 scale (one rounding), each residual r - c * s_i is rounded once
  (c * s_i is exact), and the distances |r - s_i|, |r|, |r + s_i| and
  zeta * s_i are float64 values.  A quantized code therefore depends only on
  IEEE float64 operations, which any implementation reproduces bit for bit.
* Ties in the argmin go to c = 0 (the value the zero-bias favours); a tie
  between -1 and +1 cannot occur unless r = 0 or s_i = 0, where 0 wins too.
* The zero-bias test is strict (|r| < zeta * s_i), zeta defaults to 0, and
  with zeta <= 1/2 it never changes a word (the argmin already picks 0 there).
* A zero scale (an all-zero row, or an all-zero matrix) gives r_0 = 0, hence
  the all-zero word (code 121) for every weight, and rho_n = 0.
* rho_n is the float64 quotient alpha_n / alpha rounded once to fp16
  (nearest-even); alpha itself is returned as the fp32 value max |W|.
* Non-finite weights are an error (the scale would not be defined).

Per-head prosody (section 8.2: one rho per attention head, the rows of a
head sharing a scale) is the same rule over blocks of consecutive rows:
with rho_rows = b, block h = rows [h b, (h + 1) b) is normalised by its
largest |W| (alpha_h) and rho_h = fp16(alpha_h / alpha); rho_rows = 1 is the
per-row scale of section 3.3, and the decoded weight of row n uses
rho_{n // b}.

Adaptive alphabets (section 8.3: a ladder per block of 32 rows instead of
one per family) decode row n through the code book of its block: with
table_rows = b, rows [h b, (h + 1) b) read tables[h], each table built from
its block's ladder by rb_table.  Readings: the stored form is the block's
ladder (five fp32 steps, the size of ten fp16 numbers); alpha stays one
per-layer scale, and the block scales rho are unchanged.

The 7-bit truncated alphabet (section 8.1: when a layer uses at most 128 of
the 243 codes, each weight is stored in 7 bits plus a table from the 7-bit
index to the code) is rb_truncate, pack7 and unpack7.  Readings:

* The used codes are listed in increasing order; index j stands for the
  j-th smallest code that occurs in the matrix.  The list is padded to 128
  entries with code 121 (the all-zero word, a zero weight for any ladder).
* Row n of the packed matrix is a little-endian bit string of ceil(7 K / 8)
  bytes: bit q of index k is bit 7 k + q of the string, and bit p of the
  string is bit p % 8 of byte p // 8.  The bits past 7 K are zero.
* More than 128 distinct codes, or a byte 243..255, is an error.
"""

import numpy as np

from .fpround import f16_bits_to_f64, f64_to_f16_bits, f64_to_f32


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


def rb_weights(codes, table, alpha, row_scale_bits=None, rho_rows=1, table_rows=0):
    """codes uint8 [N, K] -> W_hat float64 [N, K] = alpha * T[code] * rho,
    rho of row n being row_scale[n // rho_rows].  table_rows = 0: one code
    book T float32 [243]; table_rows = b: tables float32 [ceil(N / b), 243]
    and row n reads tables[n // b] (section 8.3)."""
    codes = np.asarray(codes, dtype=np.uint8)
    N = codes.shape[0]
    tab = np.asarray(table, dtype=np.float32).astype(np.float64).reshape(-1, 243)
    if table_rows == 0:
        if tab.shape[0] != 1:
            raise ValueError("one code book without table_rows")
        block = np.zeros(N, dtype=np.int64)
    else:
        if tab.shape[0] != -(-N // table_rows):
            raise ValueError("one code book per block of table_rows rows")
        block = np.arange(N) // table_rows
    t256 = np.zeros((tab.shape[0], 256), dtype=np.float64)
    t256[:, :243] = tab
    w = float(np.float32(alpha)) * t256[block[:, None], codes]
    if row_scale_bits is not None:
        rho = f16_bits_to_f64(row_scale_bits)
        w = w * rho[np.arange(codes.shape[0]) // rho_rows][:, None]
    return w


def rb_block_scales(W, rho_rows):
    """alpha_h float32 [ceil(N / rho_rows)]: the largest |W| of each block of
    rho_rows consecutive rows (0 for an empty block)."""
    a = np.abs(np.asarray(W, dtype=np.float32))
    N = a.shape[0]
    nb = -(-N // rho_rows)
    out = np.zeros(nb, dtype=np.float32)
    for h in range(nb):
        blk = a[h * rho_rows:(h + 1) * rho_rows]
        out[h] = blk.max() if blk.size else 0.0
    return out


def rb_encode(W, ladder, zeta=0.0, per_row=False, rho_rows=None):
    """Route B encoder: W float32 [N, K] -> (codes uint8 [N, K], alpha float32,
    rho fp16 bits uint16 [ceil(N / rho_rows)] or None).  Section 3.1 steps,
    section 3.3 scales (per_row, i.e. rho_rows = 1) or section 8.2 per-head
    blocks (rho_rows = head rows); rho_rows = 0 (the default without per_row)
    is the global scale alone."""
    if rho_rows is None:
        rho_rows = 1 if per_row else 0
    W = np.asarray(W, dtype=np.float32)
    if W.ndim != 2:
        raise ValueError("W is a matrix")
    if not np.all(np.isfinite(W)):
        raise ValueError("non-finite weight")
    s = np.asarray(ladder, dtype=np.float32).astype(np.float64)
    if s.shape != (5,):
        raise ValueError("the ladder has five steps")
    a = np.abs(W.astype(np.float64))
    alpha = float(a.max()) if W.size else 0.0            # max |W|: an fp32 value
    N, K = W.shape
    if rho_rows > 0:
        blocks = rb_block_scales(W, rho_rows).astype(np.float64)   # alpha_h
        scale = blocks[np.arange(N) // rho_rows]
    else:
        scale = np.full(N, alpha)
    r = np.zeros((N, K), dtype=np.float64)
    pos = scale > 0
    r[pos] = W[pos].astype(np.float64) / scale[pos][:, None]
    z = np.float64(np.float32(zeta))
    codes = np.zeros((N, K), dtype=np.int64)
    for i in range(5):                                     # c_1 .. c_5
        d_zero = np.abs(r)
        d_plus = np.abs(r - s[i])
        d_minus = np.abs(r + s[i])
        c = np.zeros((N, K), dtype=np.int64)
        c[(d_plus < d_zero) & (d_plus < d_minus)] = 1
        c[(d_minus < d_zero) & (d_minus < d_plus)] = -1
        c[d_zero < z * s[i]] = 0                           # zero-bias
        r = r - c * s[i]
        codes = codes * 3 + (c + 1)                        # c_1 most significant
    rho = None
    if rho_rows > 0:
        q = np.zeros(blocks.size, dtype=np.float64)
        if alpha > 0:
            q = blocks / alpha
        rho = f64_to_f16_bits(q)
    return codes.astype(np.uint8), np.float32(alpha), rho


def rb_truncate(codes):
    """Section 8.1 truncated alphabet: codes uint8 [N, K] -> (used uint8 [128],
    n_used, index uint8 [N, K]) with used[index[n, k]] == codes[n, k]."""
    codes = np.asarray(codes, dtype=np.uint8)
    if codes.size and int(codes.max()) > 242:
        raise ValueError("byte 243..255 is not a code")
    present = np.zeros(243, dtype=bool)
    present[codes.ravel()] = True
    used_codes = np.flatnonzero(present)                  # increasing
    n_used = int(used_codes.size)
    if n_used > 128:
        raise ValueError("more than 128 codes in use")
    index_of = np.zeros(256, dtype=np.uint8)
    index_of[used_codes] = np.arange(n_used)
    used = np.full(128, 121, dtype=np.uint8)
    used[:n_used] = used_codes
    return used, n_used, index_of[codes]


def pack7(index):
    """index uint8 [N, K], each < 128 -> uint8 [N, ceil(7 K / 8)]: bit q of
    index k is bit 7 k + q of the row's little-endian bit string."""
    index = np.asarray(index, dtype=np.uint8)
    if index.size and int(index.max()) > 127:
        raise ValueError("a 7-bit index is below 128")
    N, K = index.shape
    L = -(-7 * K // 8)
    bits = (index[:, :, None] >> np.arange(7, dtype=np.uint8)) & 1     # [N, K, 7]
    stream = np.zeros((N, 8 * L), dtype=np.uint8)
    stream[:, :7 * K] = bits.reshape(N, 7 * K)
    return np.packbits(stream, axis=1, bitorder="little")


def unpack7(packed, K):
    """Inverse of pack7: uint8 [N, ceil(7 K / 8)] -> index uint8 [N, K]."""
    packed = np.asarray(packed, dtype=np.uint8)
    N = packed.shape[0]
    if packed.shape[1] != -(-7 * K // 8):
        raise ValueError("ceil(7 K / 8) bytes per row")
    bits = np.unpackbits(packed, axis=1, bitorder="little")[:, :7 * K].reshape(N, K, 7)
    return (bits.astype(np.uint32) << np.arange(7, dtype=np.uint32)).sum(axis=2).astype(np.uint8)


def rb_weights7(packed, K, used, table, alpha, row_scale_bits=None, rho_rows=1, table_rows=0):
    """W_hat of a 7-bit packed matrix: the code of weight (n, k) is
    used[index[n, k]], then rb_weights."""
    codes = np.asarray(used, dtype=np.uint8)[unpack7(packed, K)]
    return rb_weights(codes, table, alpha, row_scale_bits, rho_rows, table_rows)
