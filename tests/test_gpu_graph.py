"""The library's calls under HIP graph capture: they enqueue kernels only (no
allocation, no memset, no host synchronisation), so a captured forward +
backward replays to the eager result. Each replay follows eager work of the
program's own and a synchronisation, and is checked bit for bit."""

from __future__ import annotations

import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():  # pragma: no cover - CPU container
    pytest.skip("needs a GPU", allow_module_level=True)

import memory_bound_normalization_rmsnorm_amd as rn  # noqa: E402


def _bits(t):
    return t.view(torch.int32) if t.dtype == torch.float32 else t.view(torch.int16)


@pytest.mark.parametrize("M,N,residual", [(4096, 4096, False), (1, 4096, False), (1000, 128, False),
                                          (777, 5120, True), (333, 4100, False), (129, 4095, True),
                                          (300, 65536, False),   # split rows (fill kernel + exchange)
                                          (64, 262144, False),   # two-pass forward, 16 split members
                                          (100, 98304, True)])   # residual two-pass forward and split rows
def test_graph_replay_matches_eager(M, N, residual):
    print(f"graph M={M} N={N} residual={residual}", flush=True)
    g = torch.Generator(device="cuda")
    g.manual_seed(M + N)
    x = torch.randn((M, N), generator=g, device="cuda").to(torch.bfloat16)
    res = torch.randn((M, N), generator=g, device="cuda").to(torch.bfloat16)
    dy = (torch.randn((M, N), generator=g, device="cuda") * 1e-2).to(torch.bfloat16)
    dh = (torch.randn((M, N), generator=g, device="cuda") * 1e-2).to(torch.bfloat16)
    w = (1 + 0.1 * torch.randn(N, generator=g, device="cuda")).to(torch.bfloat16)
    h, y, dx = (torch.empty_like(x) for _ in range(3))
    rstd = torch.empty(M, device="cuda")
    dw = torch.empty(N, device="cuda")
    nbytes = rn.rmsnorm_bwd_workspace_bytes(M, N, rn.BF16)
    ws = torch.empty(max(nbytes, 256) // 4, device="cuda")

    def step():
        if residual:
            rn.rmsnorm_fwd_residual(x, res, w, 1e-6, M, N, rn.BF16, h, y, rstd)
            rn.rmsnorm_bwd_residual(h, w, dy, dh, rstd, M, N, rn.BF16, dx, dw, ws, nbytes)
        else:
            rn.rmsnorm_fwd(x, w, 1e-6, M, N, rn.BF16, y, rstd)
            rn.rmsnorm_bwd(x, w, dy, rstd, M, N, rn.BF16, dx, dw, ws, nbytes)

    step()
    torch.cuda.synchronize()
    outs = (h, y, rstd, dx, dw) if residual else (y, rstd, dx, dw)
    ref = [o.clone() for o in outs]
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    for rep in range(3):
        for o in outs:
            o.fill_(float("nan"))
        _ = (x.float() * 2).sum()  # unrelated eager work between replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for o, r in zip(outs, ref):
            assert torch.equal(_bits(o), _bits(r)), f"replay {rep} differs"
