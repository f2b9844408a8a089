"""fp64 oracle of the FP8 base product with a bf16 low-rank term (test infrastructure).

TEST INFRASTRUCTURE ONLY: only the tests, ``__graft_entry__.smoke()`` and the
benchmark's CPU-baseline leg may import this module.  It shares no code with
the HIP library under ``rank_adapter_gemm_amd/`` and never imports it.

What it follows
---------------
"Multi-LoRA Serving 与 Adapter 隔离", the section on numerics and mixed
precision: a quantized base weight (INT4 or FP8) with a half-precision
adapter is a common mix, and the low-rank term must be added to the base
product's result in the kernel's accumulator, never folded into the packed
quantized weights.  The pages fix no quantization scheme; the reading used
here (and by the library) is the plainest FP8 one:

  * format: OCP 8-bit E4M3 ("e4m3fn": 1 sign, 4 exponent bits with bias 7,
    3 mantissa bits, subnormals, no infinities, codes 0x7f / 0xff are NaN,
    largest finite 448), rounding to nearest with ties to even;
  * one power-of-two scale per token row of x and per output column of W
    (codes of W stored K-contiguous: row n of Wq holds column n of W):
    s = 2^e with e the smallest integer such that amax <= 448 * 2^e, where
    amax is the row's (column's) largest magnitude, clamped to
    [-127, 127] (the range of the matrix cores' E8M0 block scales, which
    apply these scales inside the product); an all-zero row or column gets
    e = -127 and zero codes;
  * a code is E4M3(v * 2^-e): the scaled value is exact (a power-of-two
    product that stays within +-448), so the codes depend on no rounding
    but the one to E4M3;
  * output: y[t,n] = s_x[t] s_w[n] sum_k dq(xq[t,k]) dq(wq[n,k])
                     + s_a * ((x[t] A_a) B_a)[n]   (adapter rows),
    where the low-rank term uses the unquantized bf16 x.

The base sum is exact in fp64: every product of two decoded E4M3 values is an
integer multiple of 2^-18 and below 2^17.6 in magnitude, so for K <= 2^17 all
partial sums are integers times 2^-18 below 2^53.
"""
from __future__ import annotations

from typing import Sequence

import numpy as np

from .oracle import BF16, f32_from_bf16_bits, oracle_rows

E4M3_MAX = 448.0


def e4m3_decode(codes: np.ndarray) -> np.ndarray:
    """Value of each E4M3 code as float64 (NaN for 0x7f and 0xff).

    Exponent field e, mantissa m: e = 0 gives the subnormal m * 2^-9,
    otherwise (1 + m / 8) * 2^(e - 7)."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 7).astype(np.float64)
    mag = np.where(e == 0, m * 2.0 ** -9, (1.0 + m / 8.0) * np.exp2(e.astype(np.float64) - 7.0))
    out = sign * mag
    return np.where((c & 0x7F) == 0x7F, np.nan, out)


def _round_half_even(q: np.ndarray) -> np.ndarray:
    """Nearest integer, ties to the even one (exact for the doubles used here)."""
    f = np.floor(q)
    d = q - f
    up = (d > 0.5) | ((d == 0.5) & (np.fmod(f, 2.0) != 0.0))
    return f + up


def e4m3_encode(v: np.ndarray) -> np.ndarray:
    """E4M3 code of each value, rounded to nearest with ties to even.

    Values must be finite with |v| <= 448 (callers clamp first).  The sign of
    zero is kept (a negative value that rounds to zero gives 0x80)."""
    v = np.asarray(v, dtype=np.float64)
    if not np.all(np.isfinite(v)) or np.any(np.abs(v) > E4M3_MAX):
        raise ValueError("e4m3_encode takes finite values within [-448, 448]")
    a = np.abs(v)
    sign = np.signbit(v).astype(np.int64) << 7
    code = np.zeros(v.shape, dtype=np.int64)
    # subnormal range |v| < 2^-6: steps of 2^-9 (rounding to 8 steps gives 2^-6, code 0x08)
    sub = a < 2.0 ** -6
    code[sub] = _round_half_even(a[sub] * 2.0 ** 9).astype(np.int64)
    # normal range: exponent from the binade, mantissa in steps of 2^(e-3)
    nrm = ~sub
    if np.any(nrm):
        an = a[nrm]
        e = np.floor(np.log2(an))
        # guard the binade against log2 rounding at exact powers of two
        e = np.where(np.exp2(e) > an, e - 1, e)
        e = np.where(np.exp2(e + 1) <= an, e + 1, e)
        mq = _round_half_even((an / np.exp2(e) - 1.0) * 8.0)
        carry = mq >= 8.0
        e = np.where(carry, e + 1, e)
        mq = np.where(carry, 0.0, mq)
        code[nrm] = ((e + 7).astype(np.int64) << 3) | mq.astype(np.int64)
    return (code | sign).astype(np.uint8)


def scale_exponent(amax: np.ndarray) -> np.ndarray:
    """Smallest integer e with amax <= 448 * 2^e, clamped to [-127, 127]
    (-127 for amax = 0).  Exact: with amax = m * 2^E, 1 <= m < 2, and
    448 = 1.75 * 2^8, e = E - 8 when m <= 1.75, else E - 7."""
    amax = np.asarray(amax, dtype=np.float64)
    f, E = np.frexp(amax)                   # amax = f * 2^E, 0.5 <= f < 1
    m = 2.0 * f                             # amax = m * 2^(E - 1)
    e = np.where(m <= 1.75, (E - 1) - 8, (E - 1) - 7)
    e = np.where(amax > 0, e, -127)
    return np.clip(e, -127, 127).astype(np.int64)


def quantize_rows_e4m3(a: np.ndarray):
    """Per-row E4M3 quantization of a float32 matrix [R, K].

    Returns (codes uint8 [R, K], scale float32 [R]) with scale = 2^e, e from
    ``scale_exponent`` of the row's largest magnitude, and
    codes = E4M3(a * 2^-e) (an exact scaling)."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    if a.ndim != 2:
        raise ValueError("quantize_rows_e4m3 takes a 2-D array")
    amax = np.abs(a).max(axis=1) if a.shape[1] else np.zeros(a.shape[0], np.float32)
    e = scale_exponent(amax)
    scaled = np.ldexp(a.astype(np.float64), -e[:, None])
    codes = e4m3_encode(scaled)
    scale = np.ldexp(1.0, e).astype(np.float32)      # 2^-127 is an fp32 subnormal, still exact
    return codes, scale


def quantize_weight_e4m3(W: np.ndarray):
    """Per-output-column quantization of W [K, N] (float32 values): returns
    (codes uint8 [N, K], scale float32 [N]), row n of the codes being column
    n of W."""
    W = np.asarray(W, dtype=np.float32)
    return quantize_rows_e4m3(np.ascontiguousarray(W.T))


def oracle_fp8_base(xq: np.ndarray, xs: np.ndarray, wq: np.ndarray, ws: np.ndarray) -> np.ndarray:
    """y0[t, n] = xs[t] * ws[n] * sum_k dq(xq[t, k]) dq(wq[n, k]) in fp64.

    xq [T, K] and wq [N, K] are E4M3 codes, xs [T] and ws [N] float32."""
    xq = np.asarray(xq, dtype=np.uint8)
    wq = np.asarray(wq, dtype=np.uint8)
    if xq.ndim != 2 or wq.ndim != 2 or xq.shape[1] != wq.shape[1]:
        raise ValueError("xq [T, K] and wq [N, K] must agree on K")
    if xq.shape[1] > 2 ** 17:
        raise ValueError("the exact-sum argument holds for K <= 2^17")
    acc = e4m3_decode(xq) @ e4m3_decode(wq).T
    return acc * np.asarray(xs, np.float64)[:, None] * np.asarray(ws, np.float64)[None, :]


def oracle_fp8_rows(x_bits: np.ndarray, W_bits: np.ndarray, ids: np.ndarray, A: Sequence, B: Sequence,
                    ranks: Sequence[int], scales: Sequence[float], rows: Sequence[int] | None = None,
                    wq: np.ndarray | None = None, ws: np.ndarray | None = None,
                    n_threads: int | None = None) -> dict:
    """fp64 output rows of the FP8-base layer.

    x_bits [T, d_in] and W_bits [d_in, d_out] are bf16 bit patterns (uint16);
    A, B, ranks, scales describe the slots as for ``oracle_rows`` (bf16).  The
    weight codes are taken from (wq, ws) when given, else quantized here.
    Returns {"y": [n, d_out], "xq": [n, d_in], "xs": [n], "wq", "ws"} for the
    listed rows (all rows when ``rows`` is None)."""
    x_bits = np.ascontiguousarray(x_bits, dtype=np.uint16)
    W_bits = np.ascontiguousarray(W_bits, dtype=np.uint16)
    T, d_in = x_bits.shape
    d_out = W_bits.shape[1]
    rows = np.arange(T, dtype=np.int64) if rows is None else np.asarray(rows, dtype=np.int64)
    if wq is None or ws is None:
        wq, ws = quantize_weight_e4m3(f32_from_bf16_bits(W_bits))
    xq, xs = quantize_rows_e4m3(f32_from_bf16_bits(x_bits[rows]))
    y = oracle_fp8_base(xq, xs, wq, ws)
    # low-rank term from the bf16 x, through the fp64 row oracle with a zero
    # base weight (its y is then exactly s_a * delta, or 0 for base rows)
    zero_w = np.zeros((d_in, d_out), dtype=np.uint16)
    y += oracle_rows(BF16, x_bits, zero_w, ids, A, B, ranks, scales, rows=rows, n_threads=n_threads)["y"]
    return {"y": y, "xq": xq, "xs": xs, "wq": wq, "ws": ws}
