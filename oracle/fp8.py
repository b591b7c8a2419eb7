"""CPU oracle for the block-scaled fp8 mode: the E4M3 number format, block quantisation,
and attention on the dequantised tensors.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import this module.  It shares no code with the
HIP path and the HIP path never calls it.

What the pages fix and what is read into them:

  * [P1] section 9.1 keeps K and V in 8 bits with a scale, dequantises each tile when it is
    loaded and computes the scores in 16-bit; [P2] (FlashAttention-3 summary) names native
    FP8 with block-wise scale factors.  Neither page fixes the format, the block or the
    scale rule, so this module takes one reading and the GPU path follows it:
  * format: OCP 8-bit E4M3 ("E4M3FN"): 1 sign bit, 4 exponent bits with bias 7, 3 mantissa
    bits; exponent field 0 holds subnormals m/8 * 2^-6; S.1111.111 is NaN; no infinities;
    largest finite value 448.  Encoding rounds to nearest, ties to the even code.
  * blocks: 64 consecutive rows (tokens) of one (batch, head), all d columns, one scale
    per block -- for Q, K and V alike.
  * scale: the smallest power of two 2^e with amax <= 448 * 2^e, so x / 2^e is exact and
    the largest element of the block lands in (224, 448].  An all-zero block takes
    e = -126 (the smallest normal fp32 exponent); e is clamped to [-126, 127].
  * attention in fp8 mode is the plain attention definition (``oracle.attention``) on the
    dequantised tensors code * 2^e: quantisation is an input transformation, after which
    the method is the same exact attention.

Everything is float64 numpy.
"""

from __future__ import annotations

import numpy as np

from .attention import attention_forward, attention_rows

E4M3_MAX = 448.0
E4M3_MIN_NORMAL = 2.0 ** -6
E4M3_SUBNORMAL_STEP = 2.0 ** -9
BLOCK_ROWS = 64
_E_MIN, _E_MAX = -126, 127


def e4m3_decode(codes):
    """Value of each E4M3 code (uint8 array) as float64; NaN for the two NaN codes."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 7).astype(np.float64)
    normal = sign * np.ldexp(1.0 + m / 8.0, (e - 7).astype(np.int64))
    sub = sign * (m / 8.0) * E4M3_MIN_NORMAL
    v = np.where(e == 0, sub, normal)
    return np.where((e == 15) & (m == 7), np.nan, v)


def e4m3_encode(x):
    """Round float64 values with |x| <= 448 to E4M3 codes, nearest with ties to even.

    Subnormal range (|x| < 2^-6): the code is the nearest multiple of 2^-9 (an integer
    0..8; 8 is the smallest normal, code 0x08).  Normal range: with |x| = 2^e * f,
    f in [1, 2), the mantissa field is round(8 (f - 1)); a carry to 8 moves to the next
    binade.  The sign bit is set for negative values and for -0.
    """
    x = np.asarray(x, dtype=np.float64)
    if np.isnan(x).any() or (np.abs(x) > E4M3_MAX).any():
        raise ValueError("e4m3_encode: input outside [-448, 448]")
    a = np.abs(x)
    sub_code = np.round(a / E4M3_SUBNORMAL_STEP)                # np.round: half to even
    frac, exp = np.frexp(np.where(a > 0, a, 1.0))               # a = frac * 2^exp, frac in [0.5, 1)
    e = exp - 1                                                 # a = (2 frac) * 2^e
    m = np.round((2.0 * frac - 1.0) * 8.0)
    carry = m == 8.0
    e = np.where(carry, e + 1, e)
    m = np.where(carry, 0.0, m)
    norm_code = ((e + 7) << 3) + m.astype(np.int64)
    code = np.where(a < E4M3_MIN_NORMAL, sub_code.astype(np.int64), norm_code)
    code = code | np.where(np.signbit(x), 0x80, 0)
    return code.astype(np.uint8)


def block_exponent(amax):
    """The e of the block scale 2^e: the smallest integer with amax <= 448 * 2^e."""
    amax = float(amax)
    if amax == 0.0:
        return _E_MIN
    frac, exp = np.frexp(amax)          # amax in [2^(exp-1), 2^exp)
    e = int(exp) - 9                    # amax / 2^e in [256, 512)
    if amax > E4M3_MAX * 2.0 ** e:
        e += 1
    return int(min(max(e, _E_MIN), _E_MAX))


def quantize_blocks(X, block=BLOCK_ROWS):
    """Block quantisation of X [..., N, d]: returns (codes uint8 [..., N, d],
    scales float64 [..., ceil(N / block)]) with X ~= e4m3_decode(codes) * scale of the
    row's block."""
    X = np.asarray(X, dtype=np.float64)
    N = X.shape[-2]
    nb = -(-N // block)
    codes = np.empty(X.shape, dtype=np.uint8)
    scales = np.empty(X.shape[:-2] + (nb,), dtype=np.float64)
    for idx in np.ndindex(*X.shape[:-2]):
        for b in range(nb):
            rows = slice(b * block, min(N, (b + 1) * block))
            blk = X[idx][rows]
            e = block_exponent(np.abs(blk).max())
            scales[idx + (b,)] = 2.0 ** e
            codes[idx][rows] = e4m3_encode(blk / 2.0 ** e)
    return codes, scales


def dequantize_blocks(codes, scales, block=BLOCK_ROWS):
    """code * 2^e with each row's block scale; the inverse map of ``quantize_blocks``."""
    v = e4m3_decode(codes)
    N = v.shape[-2]
    row_scale = np.repeat(np.asarray(scales, dtype=np.float64), block, axis=-1)[..., :N]
    return v * row_scale[..., None]


def attention_fp8(Qc, Qs, Kc, Ks, Vc, Vs, scale, block=BLOCK_ROWS, return_p=False, causal=False):
    """Attention of the dequantised tensors, per head ([N, d] codes, [nb] scales); with
    ``causal`` the mask of ``attention_forward`` (keys after the query row dropped)."""
    Q = dequantize_blocks(Qc, Qs, block)
    K = dequantize_blocks(Kc, Ks, block)
    V = dequantize_blocks(Vc, Vs, block)
    return attention_forward(Q, K, V, scale, causal=causal, return_p=return_p)


def attention_fp8_rows(Qc, Qs, Kc, Ks, Vc, Vs, scale, rows, block=BLOCK_ROWS, causal=False):
    """``attention_fp8`` for query rows ``rows`` of one head only."""
    Q = dequantize_blocks(Qc, Qs, block)
    K = dequantize_blocks(Kc, Ks, block)
    V = dequantize_blocks(Vc, Vs, block)
    return attention_rows(Q, K, V, scale, rows, causal=causal)
