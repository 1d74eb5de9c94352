"""A whole forward+backward step captured as a HIP graph and replayed.

The library only launches kernels on the caller's stream (no allocation, no
synchronisation, zero fills by kernel), so a step can be captured. Each
replay runs after unrelated eager work and a synchronisation, and must equal
the eager step bit for bit (every kernel sums in a fixed order).
"""
import sys

import numpy as np
import pytest

import oracle as O
from monarch_block_diagonal_amd import synthetic as S

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def lib():
    if not torch.cuda.is_available():
        pytest.fail("a GPU is required for the gpu-marked tests")
    import monarch_block_diagonal_amd as M
    return M


# in, out, b1, b2, batch, dtype, relu: one case per path (fused 32x32,
# square 128x128, generic)
CASES = [(1024, 1024, 32, 32, 300, "bf16", True),
         (4096, 4096, 32, 32, 100, "bf16", False),
         (96, 160, 4, 8, 77, "f32", True)]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "x".join(map(str, c[:5])) + "_" + c[5])
def test_graph_replays_equal_eager(lib, case):
    M = lib
    fi, fo, b1, b2, B, dt, relu = case
    say(f"graph case {case}")
    tdt = torch.float32 if dt == "f32" else torch.bfloat16
    code = M.F32 if dt == "f32" else M.BF16
    act = M.ACT_RELU if relu else M.ACT_NONE
    s = O.derive_sizes(fi, fo, b1, b2)
    seed = 4242 + fi + B
    x = S.draw(seed, (B, fi), "normal", 1.0, dt)
    w1 = S.draw(seed + 1, (b1, s["q1o"], s["q1i"]), "normal", 1.0 / s["q1i"], dt)
    w2 = S.draw(seed + 2, (b2, s["q2o"], s["q2i"]), "normal", 1.0 / s["q2i"], dt)
    dy = S.draw(seed + 3, (B, fo), "normal", 1.0, dt)
    d = lambda a: torch.from_numpy(np.ascontiguousarray(a, np.float32)).to("cuda:0").to(tdt)  # noqa: E731
    X, W1, W2, DY = d(x), d(w1), d(w2), d(dy)
    Y = torch.empty(B, fo, dtype=tdt, device="cuda:0")
    Z = torch.empty(B, fo, dtype=tdt, device="cuda:0")
    DX, DW1, DW2 = torch.empty_like(X), torch.empty_like(W1), torch.empty_like(W2)
    need = M.monarch_bwd_workspace_bytes(fi, fo, b1, b2, B, code)
    ws = torch.empty(need, dtype=torch.uint8, device="cuda:0")

    def step():
        M.monarch_fwd(X, W1, W2, Y, Z, fi, fo, b1, b2, B, code, act)
        M.monarch_bwd(DY, X, W1, W2, Z, Y if relu else None, DX, DW1, DW2, ws, need, fi, fo,
                      b1, b2, B, code, act)

    outs = [Y, Z, DX, DW1, DW2]
    step()
    torch.cuda.synchronize()
    ref = [t.clone() for t in outs]

    # the eager step's values are checked against the oracle by the parity
    # tests (same paths and shapes); here they only have to be finite
    for t in ref:
        assert torch.isfinite(t.float()).all()

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    other = torch.randn(1 << 20, device="cuda:0")
    for rep in range(3):
        # unrelated eager work, then clear the outputs and replay
        other.mul_(1.5).add_(float(rep))
        torch.cuda.synchronize()
        for t in outs:
            t.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for name, got, want in zip(("y", "z", "dx", "dw1", "dw2"), outs, ref):
            assert torch.equal(got, want), f"replay {rep}: {name} differs from the eager step"
    say(f"graph case {case}: 3 replays equal the eager step")


def replay_equals_eager(step, outs, label):
    """Eager step, then capture and three replays (after unrelated eager work
    and with the outputs cleared), each equal to the eager step bit for bit."""
    step()
    torch.cuda.synchronize()
    ref = [t.clone() for t in outs]
    for t in ref:
        assert torch.isfinite(t.float()).all()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    other = torch.randn(1 << 20, device="cuda:0")
    for rep in range(3):
        other.mul_(1.5).add_(float(rep))
        torch.cuda.synchronize()
        for t in outs:
            t.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for i, (got, want) in enumerate(zip(outs, ref)):
            assert torch.equal(got, want), f"{label} replay {rep}: output {i} differs from eager"
    say(f"{label}: 3 replays equal the eager step")


def test_graph_hypercube(lib):
    """bf16 16 x 24 x 32 lattice: fiber rounds, the fused round-and-swap
    steps (one of them in place), fiber weight gradients and the swaps."""
    M = lib
    dims, B = (16, 24, 32), 100
    N = 16 * 24 * 32
    gen = torch.Generator(device="cuda:0")
    gen.manual_seed(77)
    x = torch.randn((B, N), generator=gen, device="cuda:0").to(torch.bfloat16)
    dy = torch.randn((B, N), generator=gen, device="cuda:0").to(torch.bfloat16)
    ws = [torch.randn((N // d, d, d), generator=gen, device="cuda:0").mul_(d ** -0.5)
          .to(torch.bfloat16) for d in dims]
    y, dx = torch.empty_like(x), torch.empty_like(x)
    dws = [torch.empty_like(w) for w in ws]
    saved = torch.empty((M.monarch_hyper_saved_elems(dims, B),), dtype=torch.bfloat16,
                        device="cuda:0")
    need = M.monarch_hyper_bwd_workspace_bytes(dims, B, M.BF16)
    wsb = torch.empty((need,), dtype=torch.uint8, device="cuda:0")
    assert "hyper_round_bwd_data_swap" in M.monarch_hyper_describe(1, dims, B, M.BF16)

    def step():
        M.monarch_hyper_fwd(x, ws, y, saved, dims, B, M.BF16)
        M.monarch_hyper_bwd(dy, x, ws, saved, dx, dws, wsb, need, dims, B, M.BF16)

    replay_equals_eager(step, [y, saved, dx] + dws, "hypercube 16x24x32")


@pytest.mark.parametrize("n,nb", [(512, 8), (1024, 4)])
def test_graph_dyad(lib, n, nb):
    """bf16 DYAD layer (blocks of 64, then of 256): gathers, both terms and the
    weight-gradient reduction."""
    M = lib
    B = 77
    q = n // nb
    gen = torch.Generator(device="cuda:0")
    gen.manual_seed(78)
    bf = torch.bfloat16
    x = torch.randn((B, n), generator=gen, device="cuda:0").to(bf)
    dy = torch.randn((B, n), generator=gen, device="cuda:0").to(bf)
    wa = torch.randn((nb, q, q), generator=gen, device="cuda:0").mul_(q ** -0.5).to(bf)
    wb = torch.randn((nb, q, q), generator=gen, device="cuda:0").mul_(q ** -0.5).to(bf)
    y, dx = torch.empty_like(x), torch.empty_like(x)
    dwa, dwb = torch.empty_like(wa), torch.empty_like(wb)
    need = M.monarch_dyad_bwd_workspace_bytes(n, n, nb, B, M.BF16)
    need_f = M.monarch_dyad_fwd_workspace_bytes(n, n, nb, B, M.BF16)
    ws = torch.empty((max(need, need_f),), dtype=torch.uint8, device="cuda:0")

    def step():
        M.monarch_dyad_fwd(x, wa, wb, y, ws, need_f, n, n, nb, B, M.BF16)
        M.monarch_dyad_bwd(dy, x, wa, wb, dx, dwa, dwb, ws, need, n, n, nb, B, M.BF16)

    replay_equals_eager(step, [y, dx, dwa, dwb], f"dyad {n}/{nb}")
