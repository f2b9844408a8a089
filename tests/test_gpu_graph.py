"""The layer captured into a HIP graph replays bit-identically to eager
execution, on every replay, with eager work and synchronisation between
replays (the benchmark times graph replays)."""
import numpy as np
import pytest
import torch

from rank_adapter_gemm_amd import lora as L

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _lib():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    L.load()


# (256, 4096 columns): the decode-sized path with the shrink fused into the
# split GEMM and the expand in its reduction.
@pytest.mark.parametrize("T,mode,d_out", [(256, L.LORA_MODE_AUTO, 768), (1500, L.LORA_MODE_AUTO, 768),
                                          (700, L.LORA_MODE_SGMV, 768), (256, L.LORA_MODE_AUTO, 4096)])
def test_graph_replay_matches_eager(T, mode, d_out):
    d_in, R, n_slots = 1024, 16, 5
    g = torch.Generator(device="cuda")
    g.manual_seed(T)
    x = torch.randn(T, d_in, generator=g, device="cuda").to(torch.bfloat16)
    W = (torch.randn(d_in, d_out, generator=g, device="cuda") / 32).to(torch.bfloat16)
    pool = L.AdapterPool(n_slots, d_in, d_out, R, torch.bfloat16)
    for s in range(n_slots):
        r = [16, 8, 12, 16, 4][s]
        A = (torch.randn(d_in, r, generator=g, device="cuda") / 32).to(torch.bfloat16)
        B = (torch.randn(r, d_out, generator=g, device="cuda") / 4).to(torch.bfloat16)
        pool.upload(s, A, B, r, 2.0 * r)
    ids = torch.as_tensor(np.random.default_rng(T).integers(-1, n_slots, size=T).astype(np.int32),
                          device="cuda")
    ws = L.Workspace(T, n_slots, R, d_out)
    y_eager = torch.empty(T, d_out, dtype=torch.bfloat16, device="cuda")
    L.lora_linear_forward(x, W, y_eager, T, pool.pool, ids, mode, 0, ws.buf)
    torch.cuda.synchronize()

    ws_g = L.Workspace(T, n_slots, R, d_out)
    y_graph = torch.zeros(T, d_out, dtype=torch.bfloat16, device="cuda")
    L.lora_linear_forward(x, W, y_graph, T, pool.pool, ids, mode, 0, ws_g.buf)   # warm-up
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        L.lora_linear_forward(x, W, y_graph, T, pool.pool, ids, mode, 0, ws_g.buf)
    scratch = torch.empty_like(y_eager)
    for rep in range(4):
        y_graph.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(y_graph, y_eager), "replay %d" % rep
        # eager work between replays on the same workspace layout
        L.lora_linear_forward(x, W, scratch, T, pool.pool, ids, mode, 0, ws.buf)
        torch.cuda.synchronize()
        assert torch.equal(scratch, y_eager)
    assert L.lora_get_device_error(ws_g.buf) == -1


def test_graph_of_several_calls_sharing_a_workspace():
    """As the benchmark runs it: one graph holding several decode-sized
    forwards (shrink fused into the split GEMM) over different inputs, all
    through one workspace; every replay matches each call's eager result."""
    T, d_in, d_out, R, n_slots, n_sets = 256, 1024, 4096, 16, 6, 3
    g = torch.Generator(device="cuda")
    g.manual_seed(11)
    ids = torch.as_tensor(np.random.default_rng(11).integers(-1, n_slots, size=T).astype(np.int32),
                          device="cuda")
    sets = []
    for i in range(n_sets):
        x = torch.randn(T, d_in, generator=g, device="cuda").to(torch.bfloat16)
        W = (torch.randn(d_in, d_out, generator=g, device="cuda") / 32).to(torch.bfloat16)
        pool = L.AdapterPool(n_slots, d_in, d_out, R, torch.bfloat16)
        for s in range(n_slots):
            r = [16, 8, 12, 16, 4, 16][s]
            A = (torch.randn(d_in, r, generator=g, device="cuda") / 32).to(torch.bfloat16)
            B = (torch.randn(r, d_out, generator=g, device="cuda") / 4).to(torch.bfloat16)
            pool.upload(s, A, B, r, 2.0 * r)
        sets.append((x, W, pool, torch.zeros(T, d_out, dtype=torch.bfloat16, device="cuda")))
    ws = L.Workspace(T, n_slots, R, d_out)
    eager = []
    for x, W, pool, _ in sets:
        y = torch.empty(T, d_out, dtype=torch.bfloat16, device="cuda")
        L.lora_linear_forward(x, W, y, T, pool.pool, ids, L.LORA_MODE_AUTO, 0, ws.buf)
        eager.append(y)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for x, W, pool, y in sets:
            L.lora_linear_forward(x, W, y, T, pool.pool, ids, L.LORA_MODE_AUTO, 0, ws.buf)
    for rep in range(3):
        for *_, y in sets:
            y.zero_()
        torch.cuda.synchronize()
        graph.replay()
        graph.replay()
        torch.cuda.synchronize()
        for i, (*_, y) in enumerate(sets):
            assert torch.equal(y, eager[i]), "replay %d, call %d" % (rep, i)
    assert L.lora_get_device_error(ws.buf) == -1
