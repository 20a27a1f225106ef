"""Pins of the W8A8 projection oracle (CPU only): the E4M3 encoder against a
brute-force nearest-code search, the quantisation rules against closed forms,
and the product and its layout against integer arithmetic."""
import numpy as np

from oracle import proj as P
from oracle.rola import e4m3fn_decode

CODES = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], dtype=np.uint8)  # no NaN codes
VALUES = e4m3fn_decode(CODES)


def brute_encode(y):
    """Nearest E4M3 value by exhaustive search; ties to the even mantissa; zero keeps its sign."""
    out = np.empty(len(y), dtype=np.uint8)
    for i, v in enumerate(np.asarray(y, np.float64)):
        if v == 0.0:
            out[i] = 0x80 if np.signbit(v) else 0x00
            continue
        same_sign = CODES[(CODES >> 7) == (1 if v < 0 else 0)]
        vals = e4m3fn_decode(same_sign)
        err = np.abs(vals - v)
        best = np.flatnonzero(err == err.min())
        if len(best) > 1:  # a midpoint: the code with an even mantissa
            best = [b for b in best if (same_sign[b] & 1) == 0]
        out[i] = same_sign[best[0]]
    return out


def test_encoder_matches_brute_force_nearest_code():
    rng = np.random.default_rng(5)
    mags = np.exp(rng.uniform(np.log(2.0 ** -12), np.log(448.0), 3000))
    y = (mags * rng.choice([-1.0, 1.0], 3000)).astype(np.float32)
    mids = ((VALUES[:-1] + VALUES[1:]) / 2)[(CODES[:-1] >> 7) == (CODES[1:] >> 7)]  # exact midpoints
    y = np.concatenate([y, mids.astype(np.float32), np.float32([0.0, -0.0, 448.0, -448.0, 2.0 ** -9])])
    np.testing.assert_array_equal(P.e4m3_encode(y), brute_encode(y))


def test_row_quantisation_rules():
    rng = np.random.default_rng(6)
    x = rng.standard_normal((5, 300)).astype(np.float32)
    x[2] = 0.0
    codes, s = P.quantize_rows(x)
    assert s[2] == 1.0 and np.all(codes[2] == 0)
    for r in (0, 1, 3, 4):
        amax = np.abs(x[r]).max()
        assert s[r] == np.float32(amax / np.float32(448.0))
        j = np.argmax(np.abs(x[r]))
        assert codes[r, j] in (0x7E, 0xFE)  # the largest magnitude lands on +-448
        back = e4m3fn_decode(codes[r]) * np.float64(s[r])
        # round to nearest: within half a step (2^-4 relative for normals, 2^-10 s absolute below)
        assert np.all(np.abs(back - x[r]) <= np.maximum(np.abs(x[r]) * 2.0 ** -4, 2.0 ** -10 * s[r]) * 1.0000001)


def test_product_equals_integer_matmul():
    rng = np.random.default_rng(7)
    ints = np.arange(-8, 9)
    code_of = {int(v): int(c) for c, v in zip(CODES, VALUES) if float(v).is_integer() and abs(v) <= 8}
    xi = rng.choice(ints, (24, 256))
    wi = rng.choice(ints, (48, 256))
    xq = np.vectorize(code_of.get)(xi).astype(np.uint8)
    wq = np.vectorize(code_of.get)(wi).astype(np.uint8)
    sx = (2.0 ** rng.integers(-3, 4, 24)).astype(np.float32)
    sw = (2.0 ** rng.integers(-3, 4, 48)).astype(np.float32)
    y = P.project(xq, sx, wq, sw)
    exact = (xi.astype(np.int64) @ wi.T.astype(np.int64)) * sx[:, None].astype(np.float64) * sw[None, :]
    np.testing.assert_array_equal(y, exact)


def test_layout_of_the_three_tensors():
    B, n_pad, H, d = 2, 128, 3, 8
    y = np.arange(B * n_pad * 3 * H * d, dtype=np.float64).reshape(B * n_pad, 3 * H * d)
    q, k, v = P.split_heads(y, B, n_pad, H, d)
    # token n of batch b, head h, dim e of tensor t sits at row b * n_pad + n, column (t * H + h) * d + e
    assert q[1, 2, 5, 7] == y[1 * n_pad + 5, (0 * H + 2) * d + 7]
    assert k[0, 0, 127, 0] == y[127, (1 * H + 0) * d + 0]
    assert v[1, 1, 64, 3] == y[n_pad + 64, (2 * H + 1) * d + 3]


def test_tile_quantisation_rules():
    rng = np.random.default_rng(8)
    y = rng.standard_normal((1, 2, 128, 16))
    codes, s = P.quantize_tiles(y)
    assert s.shape == (1, 2, 2)
    for h in range(2):
        for a in range(2):
            blk = y[0, h, 64 * a: 64 * a + 64].astype(np.float32)
            assert s[0, h, a] == np.float32(np.abs(blk).max() / np.float32(448.0))
            c = codes[0, h, 64 * a: 64 * a + 64]
            assert np.sum((c & 0x7F) == 0x7E) >= 1
