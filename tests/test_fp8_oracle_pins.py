"""Pins of the FP8 oracle (oracle/fp8.py) against facts outside it.

* The E4M3 decoder and encoder agree with PyTorch's own float8_e4m3fn
  conversion (an independent implementation of the same OCP format) on all
  256 codes, on random values over the whole range, on every representable
  value, on every tie between neighbours and on the float32 values next to
  each tie.
* The encoder agrees with a brute-force nearest-value search over the code
  table (ties to the even code) written here.
* The scale exponent is the smallest e with amax <= 448 * 2^e (checked
  against a brute-force search over e); the quantizer maps each row's
  largest magnitude into (224, 448], gives zero codes to a zero row, is
  invariant under power-of-two scaling of a row (codes unchanged, scale
  scaled), and its round trip stays within the format's half-step bound.
* On inputs that lie on the E4M3 grid times a power of two per row and per
  column (so the quantization is lossless), the FP8 layer must equal the
  plain fp64 layer of the bf16 oracle -- base product and low-rank term --
  for a non-square W, which fails on a transposed operand, a scale applied
  the wrong way, a dropped scale or a wrong row.
"""
import numpy as np
import pytest
import torch

from oracle import BF16, bf16_bits_from_f32, f32_from_bf16_bits, lora_scale, oracle_rows
from oracle.fp8 import (E4M3_MAX, e4m3_decode, e4m3_encode, oracle_fp8_base, oracle_fp8_rows,
                        quantize_rows_e4m3, quantize_weight_e4m3, scale_exponent)

ALL = np.arange(256, dtype=np.uint8)


def torch_codes(v32):
    return torch.from_numpy(np.ascontiguousarray(v32, np.float32)).to(torch.float8_e4m3fn).view(
        torch.uint8).numpy()


def finite_values():
    """All finite non-negative E4M3 values, ascending, with their codes."""
    c = np.arange(0, 0x7F, dtype=np.uint8)
    return e4m3_decode(c), c


def test_decode_matches_torch_on_all_codes():
    ref = torch.from_numpy(ALL.copy()).view(torch.float8_e4m3fn).float().numpy().astype(np.float64)
    got = e4m3_decode(ALL)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert nan.sum() == 2 and np.isnan(got[0x7F]) and np.isnan(got[0xFF])
    assert np.array_equal(got[~nan], ref[~nan])
    assert got[0x7E] == E4M3_MAX and got[0x38] == 1.0 and got[0x01] == 2.0 ** -9 and got[0x08] == 2.0 ** -6
    assert np.all(np.diff(got[:0x7F]) > 0)             # codes 0..0x7e ascend


def test_encode_matches_torch_random_and_ties():
    rng = np.random.default_rng(0)
    mags = np.exp2(rng.uniform(-14, np.log2(E4M3_MAX), size=200_000)).astype(np.float32)
    mags = np.minimum(mags, np.float32(E4M3_MAX))
    vals = np.where(rng.random(mags.size) < 0.5, -mags, mags).astype(np.float32)
    grid, _ = finite_values()
    ties = ((grid[1:] + grid[:-1]) / 2).astype(np.float32)
    assert np.array_equal(ties.astype(np.float64), (grid[1:] + grid[:-1]) / 2)   # ties are exact in fp32
    near = np.concatenate([np.nextafter(ties, np.float32(0)), np.nextafter(ties, np.float32(1e9))])
    near = near[np.abs(near) <= E4M3_MAX]
    pts = np.concatenate([vals, grid.astype(np.float32), ties, near, [0.0, -0.0, 1e-30, -1e-30]]).astype(np.float32)
    pts = np.concatenate([pts, -pts])
    got = e4m3_encode(pts.astype(np.float64))
    ref = torch_codes(pts)
    bad = np.nonzero(got != ref)[0]
    assert bad.size == 0, "first mismatch %r: oracle %#x torch %#x" % (pts[bad[0]], got[bad[0]], ref[bad[0]])


def test_encode_matches_brute_force_nearest():
    grid, codes = finite_values()
    rng = np.random.default_rng(1)
    v = np.concatenate([rng.uniform(-E4M3_MAX, E4M3_MAX, 3000), rng.normal(0, 0.01, 3000),
                        (grid[1:] + grid[:-1]) / 2])
    v = np.clip(v, -E4M3_MAX, E4M3_MAX)

    def brute(x):
        d = np.abs(grid - abs(x))
        best = np.nonzero(d == d.min())[0]
        c = int(codes[best[0]]) if best.size == 1 else int([codes[i] for i in best if codes[i] % 2 == 0][0])
        return c | (0x80 if np.signbit(x) else 0)

    got = e4m3_encode(v)
    ref = np.array([brute(x) for x in v], np.uint8)
    assert np.array_equal(got, ref)


def test_encode_rejects_out_of_range():
    with pytest.raises(ValueError):
        e4m3_encode(np.array([449.0]))
    with pytest.raises(ValueError):
        e4m3_encode(np.array([np.nan]))


def test_scale_exponent_is_the_smallest_power():
    rng = np.random.default_rng(5)
    amax = np.concatenate([np.exp2(rng.uniform(-140, 120, 5000)), [448.0, 449.0, 224.0, 224.0001, 447.9999,
                           1.75, 1.7500001, 2.0 ** -130, 3.0e38, 1.0]]).astype(np.float32).astype(np.float64)
    e = scale_exponent(amax)
    for a, k in zip(amax, e):
        if a < 448.0 * 2.0 ** -127:
            assert k == -127
            continue
        assert a <= 448.0 * 2.0 ** k and (k == -127 or a > 448.0 * 2.0 ** (k - 1)), (a, k)
    assert scale_exponent(np.array([0.0]))[0] == -127
    assert list(scale_exponent(np.array([448.0, 449.0, 224.0, 1.0]))) == [0, 1, -1, -8]


def test_quantize_rows_properties():
    rng = np.random.default_rng(2)
    a = (rng.normal(size=(64, 300)) * np.exp2(rng.integers(-20, 20, size=(64, 1)))).astype(np.float32)
    a[5] = 0.0
    a[6] = -0.0
    codes, scale = quantize_rows_e4m3(a)
    assert codes.shape == a.shape and scale.dtype == np.float32
    assert not codes[5].any() and np.all(codes[6] == 0x80)
    live = np.abs(a).max(axis=1) > 0
    # scales are powers of two; the largest magnitude of a row lands in (224, 448]
    m, _ = np.frexp(scale.astype(np.float64))
    assert np.all(m == 0.5)
    am = np.argmax(np.abs(a), axis=1)
    top = np.abs(a[np.arange(64), am].astype(np.float64)) / scale
    assert np.all(((top > 224) & (top <= 448))[live])
    # power-of-two invariance (no overflow or underflow at these magnitudes)
    c2, s2 = quantize_rows_e4m3(a * np.float32(2.0 ** 7))
    assert np.array_equal(c2, codes) and np.array_equal(s2[live], scale[live] * np.float32(2.0 ** 7))
    assert s2[5] == scale[5] == np.float32(2.0 ** -127)       # zero rows keep the smallest scale
    # round trip: within half a step of the format (relative 2^-4 for normals,
    # 2^-10 of the scale in the subnormal range)
    back = e4m3_decode(codes) * scale[:, None].astype(np.float64)
    err = np.abs(back - a)
    bound = np.maximum(2.0 ** -4 * np.abs(a), 2.0 ** -10 * scale[:, None])
    assert np.all((err <= bound)[live])


def grid_matrix(rng, rows, cols, exps):
    """Rows of E4M3 grid values times 2^exps[row], each row holding +-448 * 2^e
    at least once, so per-row quantization reproduces it exactly."""
    grid, _ = finite_values()
    v = rng.choice(grid, size=(rows, cols)) * np.where(rng.random((rows, cols)) < 0.5, -1.0, 1.0)
    v[np.arange(rows), rng.integers(0, cols, rows)] = E4M3_MAX
    return (v * np.exp2(np.asarray(exps, np.float64))[:, None]).astype(np.float32)


def test_grid_inputs_reduce_to_the_plain_layer():
    rng = np.random.default_rng(3)
    T, d_in, d_out = 24, 96, 40
    x = grid_matrix(rng, T, d_in, rng.integers(-12, 0, T))             # [T, d_in]
    Wt = grid_matrix(rng, d_out, d_in, rng.integers(-16, -8, d_out))    # column n of W = row n
    W = np.ascontiguousarray(Wt.T)
    xb, Wb = bf16_bits_from_f32(x), bf16_bits_from_f32(W)
    assert np.array_equal(f32_from_bf16_bits(xb), x) and np.array_equal(f32_from_bf16_bits(Wb), W)
    xq, xs = quantize_rows_e4m3(x)
    wq, ws = quantize_weight_e4m3(W)
    assert np.array_equal(e4m3_decode(xq) * xs[:, None], x)          # lossless here
    assert np.array_equal(e4m3_decode(wq) * ws[:, None], Wt)
    base = oracle_fp8_base(xq, xs, wq, ws)
    plain = x.astype(np.float64) @ W.astype(np.float64)
    assert np.allclose(base, plain, rtol=1e-13, atol=0)
    # whole layer with adapters against the bf16 oracle (same fp64 arithmetic)
    ranks = [8, 0, 5]
    A = [bf16_bits_from_f32(rng.normal(size=(d_in, max(r, 1))).astype(np.float32) * 0.1) if r else None
         for r in ranks]
    B = [bf16_bits_from_f32(rng.normal(size=(max(r, 1), d_out)).astype(np.float32) * 0.1) if r else None
         for r in ranks]
    sc = [lora_scale(2.0 * r + 1, r) if r else 0.0 for r in ranks]
    ids = rng.integers(-1, 3, size=T).astype(np.int32)
    ids[:4] = [0, 1, 2, -1]
    got = oracle_fp8_rows(xb, Wb, ids, A, B, ranks, sc, n_threads=2)
    ref = oracle_rows(BF16, xb, Wb, ids, A, B, ranks, sc, n_threads=2)["y"]
    assert np.allclose(got["y"], ref, rtol=1e-12, atol=1e-12 * np.abs(ref).max())
    # a subset of rows gives the same rows
    sub = oracle_fp8_rows(xb, Wb, ids, A, B, ranks, sc, rows=[7, 2, 19], n_threads=2)
    assert np.array_equal(sub["y"], got["y"][[7, 2, 19]])
