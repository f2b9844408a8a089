"""Pins for the fp64 CPU oracle: checks against what the pages and the
mathematics fix, never against the oracle's own formula retyped.

Each test names the passage or the mathematical fact it relies on.  Chosen so
that a dropped term, a wrong sign, a wrong index or a transposed operand in
the oracle fails at least one of them (non-square shapes throughout, so a
transposed operand cannot pass silently).
"""
import itertools
import json
import os
from fractions import Fraction

import numpy as np
import pytest
from hypothesis import given, settings
from hypothesis import strategies as st

from oracle import (BF16, F32, adapter_param_count, bf16_bits_from_f32, f32_from_bf16_bits,
                    lora_scale, oracle_rows, oracle_segmented, oracle_segments)


def _rand_case(rng, T, d_in, d_out, ranks, alphas, base_frac=0.2, bad_frac=0.0):
    x = rng.standard_normal((T, d_in)).astype(np.float32)
    W = (rng.standard_normal((d_in, d_out)) / np.sqrt(d_in)).astype(np.float32)
    A, B = [], []
    for r in ranks:
        if r == 0:
            A.append(None)
            B.append(None)
        else:
            A.append((rng.standard_normal((d_in, r)) / np.sqrt(d_in)).astype(np.float32))
            B.append((rng.standard_normal((r, d_out)) / np.sqrt(r)).astype(np.float32))
    n = len(ranks)
    ids = rng.integers(0, n, size=T).astype(np.int32)
    ids[rng.random(T) < base_frac] = -1
    if bad_frac:
        bad = rng.random(T) < bad_frac
        ids[bad] = rng.choice(np.array([-7, -2, n, n + 3], dtype=np.int32), size=int(bad.sum()))
    scales = [lora_scale(a, r) for a, r in zip(alphas, ranks)]
    return x, W, A, B, ids, scales


# ---------------------------------------------------------------------------
# Row formula
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("seed", [0, 1, 2])
def test_merged_weight_identity(seed):
    """A row with adapter a equals x (W + s A B) -- the merged-weight form
    ("Serving multiple LoRAs ...", 'Self-test' answer 1 and 'Not merging the
    weights'; the merged assertion of the grouped-batch experiment in
    "Multi-LoRA Serving 与 Adapter 隔离").  The merged weight is formed with
    numpy float64 matrix products, a different route and summation order."""
    rng = np.random.default_rng(seed)
    T, d_in, d_out = 23, 37, 29
    ranks = [3, 5, 1, 7]
    alphas = [6.0, 2.5, 1.0, 14.0]
    x, W, A, B, ids, scales = _rand_case(rng, T, d_in, d_out, ranks, alphas)
    y = oracle_rows(F32, x, W, ids, A, B, ranks, scales)["y"]
    xd, Wd = x.astype(np.float64), W.astype(np.float64)
    for t in range(T):
        a = ids[t]
        Weff = Wd if a < 0 else Wd + scales[a] * (A[a].astype(np.float64) @ B[a].astype(np.float64))
        ref = xd[t] @ Weff
        np.testing.assert_allclose(y[t], ref, rtol=1e-12, atol=1e-12)


def _int_case(rng, T, d_in, d_out, ranks):
    x = rng.integers(-3, 4, size=(T, d_in))
    W = rng.integers(-3, 4, size=(d_in, d_out))
    A = [rng.integers(-3, 4, size=(d_in, r)) for r in ranks]
    B = [rng.integers(-3, 4, size=(r, d_out)) for r in ranks]
    return x, W, A, B


@pytest.mark.parametrize("dtype", [F32, BF16])
def test_exact_integer_inputs(dtype):
    """Small integers are exact in fp32 and bf16 and scales are powers of two,
    so fp64 must reproduce exact rational arithmetic bit for bit.  The
    reference is pure-Python integer/Fraction arithmetic of the definition
    y = xW + s (xA) B."""
    rng = np.random.default_rng(7)
    T, d_in, d_out = 9, 11, 6
    ranks = [2, 3, 4]
    alphas = [4.0, 1.5, 2.0]          # s = 2, 0.5, 0.5
    x, W, A, B = _int_case(rng, T, d_in, d_out, ranks)
    ids = np.array([0, -1, 1, 2, 2, 0, -1, 1, 0], dtype=np.int32)
    scales = [lora_scale(a, r) for a, r in zip(alphas, ranks)]
    assert scales == [2.0, 0.5, 0.5]

    def store(a):
        f = np.asarray(a, dtype=np.float32)
        return f if dtype == F32 else bf16_bits_from_f32(f)

    y = oracle_rows(dtype, store(x), store(W), ids, [store(a) for a in A], [store(b) for b in B],
                    ranks, scales)["y"]
    for t in range(T):
        for n in range(d_out):
            ref = Fraction(sum(int(x[t, i]) * int(W[i, n]) for i in range(d_in)))
            a = int(ids[t])
            if a >= 0:
                u = [sum(int(x[t, i]) * int(A[a][i, j]) for i in range(d_in)) for j in range(ranks[a])]
                ref += Fraction(scales[a]) * sum(u[j] * int(B[a][j, n]) for j in range(ranks[a]))
            assert Fraction(y[t, n]) == ref, (t, n)


def test_unit_rows_gather_the_right_row():
    """x = e_i gives y = W[i,:] + s A[i,:] B (closed form): checks that the
    right row of W and of A is used for each token and the right adapter."""
    rng = np.random.default_rng(3)
    d_in, d_out = 13, 8
    ranks, alphas = [2, 4], [4.0, 4.0]
    _, W, A, B, _, scales = _rand_case(rng, 1, d_in, d_out, ranks, alphas)
    rows, ids = [], []
    for i in range(d_in):
        for a in (-1, 0, 1):
            e = np.zeros(d_in, dtype=np.float32)
            e[i] = 1.0
            rows.append(e)
            ids.append(a)
    x = np.stack(rows)
    y = oracle_rows(F32, x, W, np.array(ids, dtype=np.int32), A, B, ranks, scales)["y"]
    k = 0
    for i in range(d_in):
        for a in (-1, 0, 1):
            ref = W[i].astype(np.float64)
            if a >= 0:
                ref = ref + scales[a] * (A[a][i].astype(np.float64) @ B[a].astype(np.float64))
            np.testing.assert_allclose(y[k], ref, rtol=1e-14, atol=1e-15)
            k += 1


def test_base_only_rows_equal_xW():
    """Rows without an adapter equal x W (the 'base' group of the grouped-batch
    experiment): exactly on integer inputs, and to 1e-13 against numpy's
    float64 product on random inputs."""
    rng = np.random.default_rng(11)
    T, d_in, d_out = 17, 31, 12
    ranks, alphas = [3, 2], [3.0, 8.0]
    x, W, A, B, ids, scales = _rand_case(rng, T, d_in, d_out, ranks, alphas, base_frac=0.5)
    y = oracle_rows(F32, x, W, ids, A, B, ranks, scales)["y"]
    ref = x.astype(np.float64) @ W.astype(np.float64)
    base = ids < 0
    assert base.any()
    np.testing.assert_allclose(y[base], ref[base], rtol=1e-13, atol=1e-13)
    # a row's value does not depend on the other rows' adapters
    y_none = oracle_rows(F32, x, W, np.full(T, -1, np.int32), A, B, ranks, scales)["y"]
    assert np.array_equal(y[base], y_none[base])
    # integer inputs: exact
    xi, Wi, _, _ = _int_case(rng, 5, 7, 4, [1])
    yi = oracle_rows(F32, xi.astype(np.float32), Wi.astype(np.float32), np.full(5, -1, np.int32),
                     [], [], [], [])["y"]
    assert np.array_equal(yi, (xi @ Wi).astype(np.float64))


def test_zero_scale_or_zero_B_reduces_to_gemm():
    """s = 0 or B = 0 leaves the plain product x W (special case of the
    definition); cross-checked against numpy float64 matmul."""
    rng = np.random.default_rng(5)
    T, d_in, d_out = 12, 19, 10
    ranks = [4, 4]
    x, W, A, B, ids, _ = _rand_case(rng, T, d_in, d_out, ranks, [1.0, 1.0], base_frac=0.0)
    ref = x.astype(np.float64) @ W.astype(np.float64)
    y0 = oracle_rows(F32, x, W, ids, A, B, ranks, [0.0, 0.0])["y"]
    np.testing.assert_allclose(y0, ref, rtol=1e-13, atol=1e-13)
    Bz = [np.zeros_like(b) for b in B]
    yb = oracle_rows(F32, x, W, ids, A, Bz, ranks, [2.0, 2.0])["y"]
    np.testing.assert_allclose(yb, ref, rtol=1e-13, atol=1e-13)


def test_shrink_and_delta_outputs():
    """u = x A and delta = (x A) B for rows with an adapter (the shrink then
    expand split of "Serving multiple LoRAs ...", and of the wrapped-layer
    step in "Serving LoRA adapters: from the model name to the wrapped
    layer"), zero otherwise; checked against numpy float64 products."""
    rng = np.random.default_rng(9)
    T, d_in, d_out = 15, 21, 9
    ranks, alphas = [2, 5, 3], [2.0, 5.0, 6.0]
    x, W, A, B, ids, scales = _rand_case(rng, T, d_in, d_out, ranks, alphas)
    out = oracle_rows(F32, x, W, ids, A, B, ranks, scales, want_u=True, u_stride=8, want_delta=True)
    for t in range(T):
        a = ids[t]
        if a < 0:
            assert not out["u"][t].any() and not out["delta"][t].any()
            continue
        u = x[t].astype(np.float64) @ A[a].astype(np.float64)
        np.testing.assert_allclose(out["u"][t, :ranks[a]], u, rtol=1e-13, atol=1e-13)
        assert not out["u"][t, ranks[a]:].any()
        np.testing.assert_allclose(out["delta"][t], u @ B[a].astype(np.float64), rtol=1e-12, atol=1e-13)


def test_bad_ids_and_empty_slots_are_base_only():
    """Ids outside [-1, n_slots) and slots of rank 0 contribute nothing."""
    rng = np.random.default_rng(13)
    T, d_in, d_out = 40, 16, 8
    ranks, alphas = [2, 0, 3], [2.0, 1.0, 3.0]
    x, W, A, B, ids, scales = _rand_case(rng, T, d_in, d_out, ranks, alphas, bad_frac=0.3)
    ids[:3] = 1  # the empty slot
    y = oracle_rows(F32, x, W, ids, A, B, ranks, scales)["y"]
    y_none = oracle_rows(F32, x, W, np.full(T, -1, np.int32), A, B, ranks, scales)["y"]
    usable = (ids >= 0) & (ids < 3) & (ids != 1)
    assert np.array_equal(y[~usable], y_none[~usable])
    assert (~usable).sum() > 3 and usable.sum() > 3


@pytest.mark.parametrize("seed", [0, 1])
def test_segmented_route_equals_per_row(seed):
    """The segment-by-segment route (base block, then each adapter segment,
    scattered back through perm; the structure of lora_mixed_batch in
    "LoRAX, in depth") equals the per-row route exactly, as the printed
    True/True of the BGMV/SGMV example and the grouped experiment assert."""
    rng = np.random.default_rng(100 + seed)
    T, d_in, d_out = 61, 24, 14
    ranks = [4, 0, 2, 6, 1]
    alphas = [8.0, 1.0, 2.0, 3.0, 1.0]
    x, W, A, B, ids, scales = _rand_case(rng, T, d_in, d_out, ranks, alphas, bad_frac=0.1)
    y = oracle_rows(F32, x, W, ids, A, B, ranks, scales, n_threads=3)["y"]
    ys = oracle_segmented(F32, x, W, ids, A, B, ranks, scales, n_threads=2)
    assert np.array_equal(y, ys)


def test_zero_padding_to_max_rank_is_exact():
    """A rank-r adapter padded with zero columns of A and zero rows of B (the
    'allocate by the maximum rank' layout of "Serving multiple LoRAs ...",
    exercise 2) gives exactly the same rows, with s kept at alpha / r."""
    rng = np.random.default_rng(17)
    T, d_in, d_out, R = 20, 18, 11, 8
    ranks, alphas = [2, 5], [4.0, 10.0]
    x, W, A, B, ids, scales = _rand_case(rng, T, d_in, d_out, ranks, alphas)
    y = oracle_rows(F32, x, W, ids, A, B, ranks, scales)["y"]
    Ap = [np.concatenate([a, np.zeros((d_in, R - a.shape[1]), np.float32)], 1) for a in A]
    Bp = [np.concatenate([b, np.zeros((R - b.shape[0], d_out), np.float32)], 0) for b in B]
    yp = oracle_rows(F32, x, W, ids, Ap, Bp, [R, R], scales)["y"]
    assert np.array_equal(y, yp)


def test_row_permutation_permutes_output():
    """Rows are independent: permuting rows (with their ids) permutes y."""
    rng = np.random.default_rng(19)
    T, d_in, d_out = 33, 10, 7
    ranks, alphas = [3, 2], [3.0, 2.0]
    x, W, A, B, ids, scales = _rand_case(rng, T, d_in, d_out, ranks, alphas)
    p = rng.permutation(T)
    y = oracle_rows(F32, x, W, ids, A, B, ranks, scales)["y"]
    yp = oracle_rows(F32, np.ascontiguousarray(x[p]), W, ids[p], A, B, ranks, scales)["y"]
    assert np.array_equal(y[p], yp)


def test_bf16_inputs_widen_exactly():
    """bf16 storage is widened exactly: bf16 inputs give the same fp64 rows as
    fp32 inputs holding the same (bf16-representable) values."""
    rng = np.random.default_rng(23)
    T, d_in, d_out = 14, 20, 9
    ranks, alphas = [4, 3], [8.0, 6.0]
    x, W, A, B, ids, scales = _rand_case(rng, T, d_in, d_out, ranks, alphas)
    q = lambda a: bf16_bits_from_f32(a)
    w = lambda a: f32_from_bf16_bits(q(a))
    yb = oracle_rows(BF16, q(x), q(W), ids, [q(a) for a in A], [q(b) for b in B], ranks, scales)["y"]
    yf = oracle_rows(F32, w(x), w(W), ids, [w(a) for a in A], [w(b) for b in B], ranks, scales)["y"]
    assert np.array_equal(yb, yf)
    # the rounding itself: ties go to even, and values round to nearest
    v = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, 1.0 + 2 ** -9, -2.5, 3.0e-3], np.float32)
    got = f32_from_bf16_bits(bf16_bits_from_f32(v))
    assert got[0] == 1.0 and got[1] == 1.0 and got[2] == 1.0 + 4 * 2 ** -8
    assert got[3] == 1.0 and got[4] == -2.5
    assert abs(got[5] - 3.0e-3) <= 3.0e-3 * 2 ** -8


def test_thread_count_does_not_change_results():
    rng = np.random.default_rng(29)
    x, W, A, B, ids, scales = _rand_case(rng, 50, 16, 12, [3, 4], [3.0, 8.0])
    y1 = oracle_rows(F32, x, W, ids, A, B, [3, 4], scales, n_threads=1)["y"]
    y5 = oracle_rows(F32, x, W, ids, A, B, [3, 4], scales, n_threads=5)["y"]
    assert np.array_equal(y1, y5)


# ---------------------------------------------------------------------------
# The pages' worked examples
# ---------------------------------------------------------------------------
def test_p2_example_counts_and_routes(golden_dir):
    """The mixed batch of the BGMV/SGMV example: 53 rows, 6 per-request
    calls, 4 segments (printed); and the three routes agree (printed True).
    Our values are seeded here; the page's RNG stream is not reproduced."""
    g = json.load(open(os.path.join(golden_dir, "p2_mixed_batch_example.json")))
    inp, printed = g["inputs"], g["printed"]
    lengths, adapters = inp["request_lengths"], inp["request_adapters"]
    ids = np.array([a for a, n in zip(adapters, lengths) for _ in range(n)], dtype=np.int32)
    seg = oracle_segments(ids, inp["n_adapters"])
    assert len(ids) == printed["base_gemm_rows"]
    assert len(lengths) == printed["per_request_calls"]
    assert seg["n_seg"] == printed["sgmv_segments"]
    # the same metadata worked out by hand from the example's definition
    assert seg["seg_id"].tolist() == [0, 3, 5, 7]
    assert seg["seg_start"].tolist() == [0, 1, 39, 41, 53]
    assert seg["offsets"].tolist() == [0, 0, 1, 1, 1, 39, 39, 41, 41, 53]

    rng = np.random.default_rng(0)
    d_in, d_out, r, n = inp["d_in"], inp["d_out"], inp["rank"], inp["n_adapters"]
    dv = inp["weight_divisors"]
    W = (rng.standard_normal((d_in, d_out)) / dv["W"]).astype(np.float32)
    A = [(rng.standard_normal((d_in, r)) / dv["A"]).astype(np.float32) for _ in range(n)]
    B = [(rng.standard_normal((r, d_out)) / dv["B"]).astype(np.float32) for _ in range(n)]
    x = rng.standard_normal((len(ids), d_in)).astype(np.float32)
    scales = [inp["scale"]] * n
    y = oracle_rows(F32, x, W, ids, A, B, [r] * n, scales)["y"]
    # per-request route (one product per request) in numpy float64
    xd, Wd = x.astype(np.float64), W.astype(np.float64)
    s0 = 0
    for a, m in zip(adapters, lengths):
        xi = xd[s0:s0 + m]
        ref = xi @ Wd + inp["scale"] * ((xi @ A[a].astype(np.float64)) @ B[a].astype(np.float64))
        np.testing.assert_allclose(y[s0:s0 + m], ref, rtol=1e-12, atol=1e-12)
        s0 += m
    # per-token gather route (BGMV) via einsum in float64
    Ag = np.stack([A[a] for a in ids]).astype(np.float64)
    Bg = np.stack([B[a] for a in ids]).astype(np.float64)
    sh = np.einsum("ti,tir->tr", xd, Ag)
    ref_b = xd @ Wd + inp["scale"] * np.einsum("tr,tro->to", sh, Bg)
    assert np.allclose(y, ref_b, atol=printed["allclose_atol"] * 1e-6)
    assert np.array_equal(y, oracle_segmented(F32, x, W, ids, A, B, [r] * n, scales))


def test_p5_experiment(golden_dir):
    """The grouped-batch experiment: groups of 2 rows each, grouped == per-row
    == merged, 26 delta elements vs 40 full-weight elements."""
    g = json.load(open(os.path.join(golden_dir, "p5_grouped_experiment.json")))
    inp, printed = g["inputs"], g["printed"]
    names = sorted(inp["alpha"])                 # slots in sorted-name order: code=0, finance=1
    slot = {nm: k for k, nm in enumerate(names)}
    ids = np.array([slot.get(nm, -1) for nm in inp["adapter_ids"]], dtype=np.int32)
    assert ids.tolist() == [1, -1, 0, 1, 0, -1]
    seg = oracle_segments(ids, len(names))
    counts = np.diff(seg["offsets"]).tolist()    # base, code, finance
    assert counts == [printed["grouped_batch_sizes"]["base"], printed["grouped_batch_sizes"]["code"],
                      printed["grouped_batch_sizes"]["finance"]]
    assert seg["perm"].tolist() == [1, 5, 2, 4, 0, 3]
    assert seg["seg_id"].tolist() == [0, 1] and seg["seg_start"].tolist() == [2, 4, 6]

    hid, out, r = inp["hidden"], inp["output"], inp["rank"]
    assert adapter_param_count(hid, out, r) == printed["per_adapter_delta_elements"]
    assert hid * out == printed["full_weight_elements"]

    rng = np.random.default_rng(241)
    W = rng.standard_normal((hid, out)).astype(np.float32)
    A = [rng.standard_normal((hid, r)).astype(np.float32) for _ in names]
    B = [rng.standard_normal((r, out)).astype(np.float32) for _ in names]
    x = rng.standard_normal((inp["tokens"], hid)).astype(np.float32)
    scales = [lora_scale(inp["alpha"][nm], r) for nm in names]
    assert scales == [1.0, 2.0]
    y = oracle_rows(F32, x, W, ids, A, B, [r, r], scales)["y"]
    ys = oracle_segmented(F32, x, W, ids, A, B, [r, r], scales)
    # the page's fp32 grouped-vs-row difference is at most 1.907e-06; the
    # fp64 routes here agree exactly
    assert np.abs(y - ys).max() <= printed["grouped_vs_row_reference_max_abs_diff_fp32"]
    assert np.array_equal(y, ys)
    for t in range(len(ids)):
        a = ids[t]
        Wm = W.astype(np.float64)
        if a >= 0:
            Wm = Wm + scales[a] * (A[a].astype(np.float64) @ B[a].astype(np.float64))
        np.testing.assert_allclose(y[t], x[t].astype(np.float64) @ Wm, rtol=1e-12, atol=1e-12)


def test_parameter_counts_match_printed_sizing(golden_dir):
    """r (d_in + d_out) per adapted matrix against every sizing figure the
    pages print (exact where the page is exact, else within its rounding)."""
    g = json.load(open(os.path.join(golden_dir, "sizing_figures.json")))
    e = g["entries"]
    assert adapter_param_count(4096, 4096, 16) == e[0]["printed"]["per_projection_params"]

    def total(entry, r=None):
        r = entry["rank"] if r is None else r
        return entry["layers"] * sum(adapter_param_count(a, b, r) for a, b in entry["projections"])

    p1 = e[0]
    assert 4 * adapter_param_count(4096, 4096, 16) == p1["printed"]["per_layer_params"]
    assert total(p1) == p1["printed"]["total_params"]
    # 33,554,432 bytes: the page states 33.5 MB (truncated, not rounded)
    assert abs(total(p1) * 2 / 1e6 - p1["printed"]["total_megabytes"]) < 0.06

    p3a, p3b, p2, p5 = e[1], e[2], e[3], e[4]
    size_a = total(p3a) * 2
    lo, hi = p3a["reservation_gb"][0] * 1e9 / size_a, p3a["reservation_gb"][1] * 1e9 / size_a
    tol = p3a["relative_tolerance"]
    assert abs(lo - p3a["printed"]["adapters_fitting_low"]) <= tol * p3a["printed"]["adapters_fitting_low"]
    assert abs(hi - p3a["printed"]["adapters_fitting_high"]) <= tol * p3a["printed"]["adapters_fitting_high"]

    size_b = total(p3b) * 2
    assert total(p3b) == 167_772_160
    assert abs(total(p3b) / 1e6 - p3b["printed"]["total_params_millions"]) <= 0.01 * 168
    assert abs(size_b / 1e6 - p3b["printed"]["total_megabytes"]) <= 0.01 * 335
    lo_b, hi_b = 6e9 / size_b, 8e9 / size_b
    assert lo_b <= p3b["printed"]["adapters_fitting"] <= hi_b
    ratio = size_b / size_a
    assert abs(ratio - p3b["printed"]["capacity_ratio_vs_rank16_attention"]) <= 0.05 * 12

    size2 = total(p2) * 2
    assert total(p2) == 41_943_040
    assert abs(size2 / 2 ** 20 - p2["printed"]["megabytes_each"]) < 1e-9       # 80 MiB exactly
    assert abs(8e9 / size2 - p2["printed"]["adapters_resident"]) <= p2["relative_tolerance"] * 100

    assert total(p5) == p5["printed"]["total_params"]


def test_scale_values():
    """s = alpha / r: 2.0 at r = 16 in the BGMV/SGMV example (alpha 32); the
    grouped experiment's alpha 4 and 2 at rank 2 give 2 and 1."""
    assert lora_scale(32, 16) == 2.0
    assert lora_scale(16, 8) == 2.0
    assert lora_scale(4.0, 2) == 2.0 and lora_scale(2.0, 2) == 1.0
    assert lora_scale(2 * 64, 64) == 2.0
    assert lora_scale(5.0, 0) == 0.0
    # one fp32 value per adapter: 1/3 is the fp32 number 0x3eaaaaab = 11184811 * 2^-25
    assert lora_scale(1.0, 3) == 11184811 / 2 ** 25
    assert lora_scale(1.0, 3) != 1.0 / 3.0


# ---------------------------------------------------------------------------
# Segment metadata
# ---------------------------------------------------------------------------
def _argsort_reference(ids, n_slots):
    ids = np.asarray(ids, dtype=np.int64)
    keys = np.where((ids >= -1) & (ids < n_slots), ids + 1, 0)
    perm = np.argsort(keys, kind="stable")
    uniq, counts = np.unique(keys[perm], return_counts=True)   # consecutive after sorting
    offsets = np.zeros(n_slots + 2, dtype=np.int64)
    for u, c in zip(uniq, counts):
        offsets[u + 1] = c
    offsets = np.cumsum(offsets)
    nz = [(u - 1, offsets[u]) for u in uniq if u >= 1]
    seg_id = [a for a, _ in nz]
    seg_start = [s for _, s in nz] + [len(ids)]
    return perm, offsets, seg_id, seg_start


def test_segments_brute_force_small():
    """Every id vector of length <= 6 over {-1, 0, 1, 2} (and one invalid
    value) against numpy's stable argsort + unique counts, the library
    routines the SGMV example uses."""
    vals = [-1, 0, 1, 2]
    checked = 0
    for L in range(0, 7):
        for combo in itertools.product(vals, repeat=L):
            seg = oracle_segments(list(combo), 3)
            perm, offsets, seg_id, seg_start = _argsort_reference(combo, 3)
            assert seg["perm"].tolist() == perm.tolist()
            assert seg["offsets"].tolist() == offsets.tolist()
            assert seg["seg_id"].tolist() == seg_id
            assert seg["seg_start"].tolist() == seg_start
            checked += 1
    assert checked == sum(4 ** L for L in range(7))
    seg = oracle_segments([5, -4, 0, 3], 3)      # invalid ids go with the base block
    assert seg["offsets"].tolist() == [0, 3, 4, 4, 4] and seg["perm"].tolist() == [0, 1, 3, 2]


@settings(max_examples=60, deadline=None)
@given(st.integers(1, 40), st.lists(st.integers(-2, 45), min_size=0, max_size=300))
def test_segments_random_against_argsort(n_slots, ids):
    seg = oracle_segments(ids, n_slots)
    perm, offsets, seg_id, seg_start = _argsort_reference(ids, n_slots)
    assert seg["perm"].tolist() == perm.tolist()
    assert seg["offsets"].tolist() == offsets.tolist()
    assert seg["seg_id"].tolist() == seg_id and seg["seg_start"].tolist() == seg_start
    assert seg["n_seg"] == len(seg_id)
