"""FP8-base test plumbing: a bf16 batch with its FP8 base weight, the fp64
oracle reference rows with their element-wise tolerance (derived in the
FP8 parity tests' docstring), and the check against that tolerance."""
import numpy as np
import torch

from oracle import BF16, lora_scale, oracle_rows
from oracle.fp8 import e4m3_decode, oracle_fp8_base, quantize_rows_e4m3, quantize_weight_e4m3
from rank_adapter_gemm_amd import lora as L

from helpers import TOL, to_oracle


def f32(t):
    return t.float().cpu().numpy()


def fp8_bound(xq, xs, wq, ws):
    """2^-11 * s_x s_w sum_k |dq(xq)| |dq(wq)|: the FP8 accumulation term."""
    S = np.abs(e4m3_decode(xq)) @ np.abs(e4m3_decode(wq)).T
    return 2.0 ** -11 * S * xs.astype(np.float64)[:, None] * ws.astype(np.float64)[None, :]


def assert_within(y, ref, tol, what):
    y = y.float().cpu().double().numpy() if torch.is_tensor(y) else y
    err = np.abs(y - ref)
    ratio = err / tol
    i = np.unravel_index(np.argmax(ratio), ratio.shape)
    assert ratio.max() <= 1.0, "%s: |y-ref| %.3e > tol %.3e at %s (ref %.4e)" % (what, err[i], tol[i], i, ref[i])
    # the plain bf16 bar holds as well
    assert np.max(err / (1 + np.abs(ref))) <= TOL[torch.bfloat16], what


class Fp8Case:
    """A bf16 batch with explicit slot ranks, its FP8 base weight, and the
    oracle pieces (codes from the bf16 values; nothing from the GPU)."""

    def __init__(self, T, d_in, d_out, ranks, R, seed=0, ids=None, base_frac=0.2, sd=(1.0, None)):
        g = torch.Generator(device="cuda")
        g.manual_seed(seed)
        rng = np.random.default_rng(seed)
        sx, sw = sd[0], sd[1] if sd[1] is not None else d_in ** -0.5
        self.T, self.d_in, self.d_out, self.R, self.ranks = T, d_in, d_out, R, list(ranks)
        self.n_slots = len(ranks)
        self.alphas = [2.0 * r + 1 for r in ranks]
        self.x = (torch.randn(max(T, 1), d_in, generator=g, device="cuda") * sx).to(torch.bfloat16)
        self.W = (torch.randn(d_in, d_out, generator=g, device="cuda") * sw).to(torch.bfloat16)
        self.A = [(torch.randn(d_in, max(r, 1), generator=g, device="cuda") / d_in ** 0.5).to(torch.bfloat16)
                  for r in ranks]
        self.B = [(torch.randn(max(r, 1), d_out, generator=g, device="cuda") / max(r, 1) ** 0.5).to(torch.bfloat16)
                  for r in ranks]
        if ids is None:
            ids = rng.integers(0, self.n_slots, size=max(T, 1)).astype(np.int32)
            ids[rng.random(ids.size) < base_frac] = -1
        self.ids = np.asarray(ids, np.int32)
        self.ids_dev = torch.as_tensor(self.ids, device="cuda")
        self.pool = L.AdapterPool(self.n_slots, d_in, d_out, R, torch.bfloat16)
        for s, r in enumerate(ranks):
            if r > 0:
                self.pool.upload(s, self.A[s], self.B[s], r, self.alphas[s])
        self.wt = L.Fp8Weight(self.W)
        self._wq = None

    def weight_codes(self):
        if self._wq is None:
            self._wq = quantize_weight_e4m3(f32(self.W))
        return self._wq

    def reference(self, rows=None):
        """fp64 y rows and their element-wise tolerance."""
        rows = np.arange(self.T) if rows is None else np.asarray(rows)
        xb = to_oracle(self.x)
        xq, xs = quantize_rows_e4m3(f32(self.x)[rows])
        wq, ws = self.weight_codes()
        base = oracle_fp8_base(xq, xs, wq, ws)
        A = [to_oracle(a) if r > 0 else None for a, r in zip(self.A, self.ranks)]
        B = [to_oracle(b) if r > 0 else None for b, r in zip(self.B, self.ranks)]
        sc = [lora_scale(a, r) if r > 0 else 0.0 for a, r in zip(self.alphas, self.ranks)]
        zero_w = np.zeros((self.d_in, self.d_out), np.uint16)
        lo = oracle_rows(BF16, xb, zero_w, self.ids[:max(self.T, 1)], A, B, self.ranks, sc, rows=rows,
                         want_u=True, u_stride=self.R)
        ref = base + lo["y"]
        # magnitude of the low-rank terms: |s| sum_j |u_j| |B_jn|
        lmag = np.zeros_like(ref)
        for i, t in enumerate(rows):
            a = int(self.ids[t])
            if 0 <= a < self.n_slots and self.ranks[a] > 0:
                r = self.ranks[a]
                Bf = np.abs(f32(self.B[a]).astype(np.float64))
                lmag[i] = abs(sc[a]) * (np.abs(lo["u"][i, :r]) @ Bf)
        tol = 2.0 ** -8 * (np.abs(ref) + np.abs(base)) + 2.0 ** -10 * lmag + fp8_bound(xq, xs, wq, ws) + 1e-30
        return ref, tol

    def run(self, mode=L.LORA_MODE_AUTO, flags=0, T=None):
        T = self.T if T is None else T
        ws = L.Workspace(max(T, 1), self.n_slots, self.R, self.d_out, fp8_d_in=self.d_in)
        y = torch.full((max(T, 1), self.d_out), 7.0, dtype=torch.bfloat16, device="cuda")
        L.lora_linear_forward_fp8(self.x, self.wt.codes, self.wt.scale, y, T, self.pool.pool, self.ids_dev,
                                  mode, flags, ws.buf)
        torch.cuda.synchronize()
        return y, ws
