"""Pins of the fp8 oracle (``oracle.fp8``) against facts of the OCP E4M3 format, brute-force
rounding over the code table, the definition of the block scale, and a rounding-error bound.
A mutation test at the end plants plausible mistakes and checks that a pin rejects each."""

import inspect
import types

import numpy as np
import pytest

import oracle.fp8 as fp8
from oracle import attention_forward

ALL = np.arange(256, dtype=np.uint8)


# ------------------------------------------------------------------ the format itself ---

def _pins_decode(m):
    v = m.e4m3_decode(ALL)
    # values the OCP 8-bit floating point specification lists for E4M3
    assert v[0x38] == 1.0 and v[0xB8] == -1.0
    assert v[0x7E] == 448.0 and v[0xFE] == -448.0          # largest finite magnitude
    assert v[0x08] == 2.0 ** -6                            # smallest normal
    assert v[0x01] == 2.0 ** -9 and v[0x07] == 7 * 2.0 ** -9   # subnormals m/8 * 2^-6
    assert v[0x00] == 0.0 and v[0x80] == 0.0 and np.signbit(v[0x80])
    assert v[0x40] == 2.0 and v[0x30] == 0.5 and v[0x3C] == 1.5 and v[0x44] == 3.0
    # S.1111.111 is NaN and nothing else is; no infinities
    assert set(np.flatnonzero(np.isnan(v))) == {0x7F, 0xFF}
    assert not np.isinf(v).any()
    pos = v[:0x7F]
    assert (np.diff(pos) > 0).all()                        # positive codes are ordered
    np.testing.assert_array_equal(v[0x80:0xFF], -pos)      # sign bit mirrors
    # 8 values per binade, evenly spaced, in every normal binade
    for e in range(-6, 9):
        binade = pos[(pos >= 2.0 ** e) & (pos < 2.0 ** (e + 1))]
        assert len(binade) == (7 if e == 8 else 8)          # 448 = 1.75 * 2^8 ends the last
        np.testing.assert_allclose(np.diff(binade), 2.0 ** (e - 3))


def test_decode_table_matches_the_format():
    _pins_decode(fp8)


def _nearest_even(x, table):
    """Brute force: the finite code nearest to x, ties to the even code; -0 for x <= -0."""
    best, best_d = [], np.inf
    for c in range(256):
        if np.isnan(table[c]) or c == 0x80:
            continue
        d = abs(table[c] - x)
        if d < best_d:
            best, best_d = [c], d
        elif d == best_d:
            best.append(c)
    c = best[0] if len(best) == 1 else [b for b in best if b % 2 == 0][0]
    if table[c] == 0.0 and np.signbit(x):
        c = 0x80
    return c


def _pins_encode(m):
    table = fp8.e4m3_decode(ALL)
    # every finite code round-trips
    finite = [c for c in range(256) if not np.isnan(table[c])]
    np.testing.assert_array_equal(m.e4m3_encode(table[finite]), np.array(finite, np.uint8))
    # every midpoint between neighbouring values, and points just either side of it
    pos = np.sort(table[:0x7F])
    mids = (pos[:-1] + pos[1:]) / 2
    xs = np.concatenate([mids, np.nextafter(mids, 0), np.nextafter(mids, 1e9), -mids])
    rng = np.random.default_rng(11)
    xs = np.concatenate([xs, rng.uniform(-448, 448, 300),
                         rng.choice([-1, 1], 300) * 2.0 ** rng.uniform(-12, 8.8, 300)])
    xs = np.clip(xs, -448, 448)
    got = m.e4m3_encode(xs)
    want = np.array([_nearest_even(x, table) for x in xs], np.uint8)
    np.testing.assert_array_equal(got, want)
    assert m.e4m3_encode(np.array([-0.0]))[0] == 0x80
    with pytest.raises(ValueError):
        m.e4m3_encode(np.array([449.0]))


def test_encode_is_nearest_ties_to_even():
    _pins_encode(fp8)


# ------------------------------------------------------------------ block scales ---

def _pins_scale(m):
    rng = np.random.default_rng(3)
    amaxes = list(2.0 ** rng.uniform(-40, 40, 400)) + [448.0, 448.0 * 2 ** 5, 448.0 * 2 ** -7,
                                                       np.nextafter(448.0, 1e9), 224.0, 1.0, 2.0 ** -130]
    for a in amaxes:
        e = m.block_exponent(a)
        # the definition: the smallest integer e with amax <= 448 * 2^e
        assert a <= 448.0 * 2.0 ** e or e == 127
        assert a > 448.0 * 2.0 ** (e - 1) or e == -126
    assert m.block_exponent(0.0) == -126


def test_block_exponent_is_the_smallest_fitting_power_of_two():
    _pins_scale(fp8)


def _pins_quantize(m):
    rng = np.random.default_rng(5)
    for N, sigma in ((200, 1.0), (64, 30.0), (1, 1e-3), (130, 1e4)):
        X = rng.standard_normal((2, N, 8)) * sigma
        X[0, :3] *= 50.0                         # an outlier block
        codes, scales = m.quantize_blocks(X, 64)
        assert scales.shape == (2, -(-N // 64))
        Xh = m.dequantize_blocks(codes, scales, 64)
        for b in range(scales.shape[1]):
            rows = slice(64 * b, min(N, 64 * b + 64))
            s = scales[:, b][:, None, None]
            blk = X[:, rows]
            # the largest element lands in (224, 448] of the code range
            top = np.abs(blk).max(axis=(1, 2)) / s[:, 0, 0]
            assert ((top > 224) & (top <= 448)).all()
            # rounding error: half a step, 2^-4 relative (normal) or 2^-10 * s (subnormal)
            err = np.abs(Xh[:, rows] - blk)
            assert (err <= np.maximum(2.0 ** -4 * np.abs(blk), 2.0 ** -10 * s) * (1 + 1e-12)).all()
    # an all-zero block: codes 0, scale 2^-126
    c, s = m.quantize_blocks(np.zeros((70, 4)), 64)
    assert (c == 0).all() and (s == 2.0 ** -126).all()


def test_quantize_round_trip_error_bound():
    _pins_quantize(fp8)


def test_attention_fp8_is_attention_of_the_dequantised_tensors():
    rng = np.random.default_rng(9)
    Q, K, V = (rng.standard_normal((100, 16)) for _ in range(3))
    qc, qs = fp8.quantize_blocks(Q)
    kc, ks = fp8.quantize_blocks(K)
    vc, vs = fp8.quantize_blocks(V)
    O, L = fp8.attention_fp8(qc, qs, kc, ks, vc, vs, 0.25)
    # inputs already on the fp8 grid with unit scales quantise to themselves
    Qg = fp8.e4m3_decode(fp8.e4m3_encode(np.clip(Q, -448, 448)))
    c2, s2 = fp8.quantize_blocks(Qg * 1.0)
    np.testing.assert_allclose(fp8.dequantize_blocks(c2, s2), Qg, rtol=0, atol=0)
    Qd, Kd, Vd = (fp8.dequantize_blocks(c, s) for c, s in ((qc, qs), (kc, ks), (vc, vs)))
    O2, L2 = attention_forward(Qd, Kd, Vd, 0.25)
    np.testing.assert_array_equal(O, O2)
    np.testing.assert_array_equal(L, L2)
    # and it stays close to full-precision attention (quantisation only perturbs inputs)
    O3, _ = attention_forward(Q, K, V, 0.25)
    assert np.abs(O - O3).max() < 0.1
    rows = np.array([0, 63, 64, 99])
    Or, Lr = fp8.attention_fp8_rows(qc, qs, kc, ks, vc, vs, 0.25, rows)
    np.testing.assert_allclose(Or, O[rows], atol=1e-13)
    np.testing.assert_allclose(Lr, L[rows], atol=1e-13)


def test_attention_fp8_causal_closed_forms():
    """Causal fp8 attention: row 0 sees only key 0 (O = V^_0, LSE = its one score), the
    last row sees every key (the non-causal row), and row i matches attention over the
    first i + 1 dequantised keys alone."""
    rng = np.random.default_rng(10)
    Q, K, V = (rng.standard_normal((130, 16)) for _ in range(3))
    (qc, qs), (kc, ks), (vc, vs) = (fp8.quantize_blocks(x) for x in (Q, K, V))
    Qd, Kd, Vd = (fp8.dequantize_blocks(c, s) for c, s in ((qc, qs), (kc, ks), (vc, vs)))
    O, L = fp8.attention_fp8(qc, qs, kc, ks, vc, vs, 0.3, causal=True)
    np.testing.assert_array_equal(O[0], Vd[0])
    assert abs(L[0] - 0.3 * float(Qd[0] @ Kd[0])) < 1e-14
    Of, Lf = fp8.attention_fp8(qc, qs, kc, ks, vc, vs, 0.3)
    np.testing.assert_allclose(O[-1], Of[-1], rtol=0, atol=1e-14)
    np.testing.assert_allclose(L[-1], Lf[-1], rtol=0, atol=1e-14)
    for i in (1, 63, 64, 100):
        S = 0.3 * (Kd[: i + 1] @ Qd[i])
        w = np.exp(S - S.max())
        np.testing.assert_allclose(O[i], (w / w.sum()) @ Vd[: i + 1], rtol=0, atol=1e-13)
        np.testing.assert_allclose(L[i], S.max() + np.log(w.sum()), rtol=0, atol=1e-13)
    rows = np.array([0, 5, 64, 129])
    Or, Lr = fp8.attention_fp8_rows(qc, qs, kc, ks, vc, vs, 0.3, rows, causal=True)
    np.testing.assert_allclose(Or, O[rows], atol=1e-13)
    np.testing.assert_allclose(Lr, L[rows], atol=1e-13)


# ------------------------------------------------------------------ mutations ---

def _mutant(old, new):
    src = inspect.getsource(fp8)
    assert src.count(old) >= 1, f"mutation anchor not found: {old!r}"
    src = src.replace("from .attention import", "from oracle.attention import")
    mod = types.ModuleType("fp8_mutant")
    exec(compile(src.replace(old, new, 1), "fp8_mutant", "exec"), mod.__dict__)
    return mod


MUTANTS = [
    ("normal = sign * np.ldexp(1.0 + m / 8.0, (e - 7)", "normal = sign * np.ldexp(1.0 + m / 8.0, (e - 8)"),
    ("sub = sign * (m / 8.0) * E4M3_MIN_NORMAL", "sub = sign * (m / 16.0) * E4M3_MIN_NORMAL"),
    ("return np.where((e == 15) & (m == 7), np.nan, v)", "return v"),
    ("m = np.round((2.0 * frac - 1.0) * 8.0)", "m = np.floor((2.0 * frac - 1.0) * 8.0)"),
    ("sub_code = np.round(a / E4M3_SUBNORMAL_STEP)", "sub_code = np.floor(a / E4M3_SUBNORMAL_STEP + 0.5)"),
    ("norm_code = ((e + 7) << 3)", "norm_code = ((e + 6) << 3)"),
    ("e = int(exp) - 9", "e = int(exp) - 8"),
    ("if amax > E4M3_MAX * 2.0 ** e:", "if amax >= E4M3_MAX * 2.0 ** e:"),
    ("rows = slice(b * block, min(N, (b + 1) * block))", "rows = slice(b * block, min(N, (b + 1) * block - 1))"),
    ("codes[idx][rows] = e4m3_encode(blk / 2.0 ** e)", "codes[idx][rows] = e4m3_encode(blk / 2.0 ** (e + 1))"),
]


@pytest.mark.parametrize("old,new", MUTANTS)
def test_every_fp8_mutant_is_rejected(old, new):
    m = _mutant(old, new)
    failed = False
    for pin in (_pins_decode, _pins_encode, _pins_scale, _pins_quantize):
        try:
            pin(m)
        except (AssertionError, ValueError, IndexError):
            failed = True
            break
    assert failed, f"no pin rejects the mutant {new!r}"
