"""monarch_bwd_noalloc (the backward with the library's static scratch in
place of a caller workspace) against monarch_bwd, through the C ABI.

Both run the same kernels on the same inputs, so the results must agree bit
for bit. Each case makes two calls in a row, the second with fewer rows, so
the second call runs on scratch that still holds the first call's
intermediates; a kernel that read scratch before writing it would differ
from monarch_bwd's freshly allocated workspace.
"""
import numpy as np
import pytest
import torch

import oracle as O
from monarch_block_diagonal_amd import binding as B
from monarch_block_diagonal_amd import torch_api as T

pytestmark = pytest.mark.gpu

# (in, out, nb1, nb2, dtype, act, (batch of call 1, batch of call 2), path)
CASES = [
    (4096, 4096, 32, 32, torch.bfloat16, B.ACT_NONE, (2048, 700), "sq128"),
    (4096, 4096, 32, 32, torch.bfloat16, B.ACT_RELU, (1024, 333), "sq128"),
    (1024, 1024, 32, 32, torch.bfloat16, B.ACT_NONE, (4096, 1000), "sm32"),
    (1024, 512, 16, 16, torch.float32, B.ACT_RELU, (3000, 777), "generic"),
    (768, 3072, 4, 4, torch.bfloat16, B.ACT_NONE, (4096, 1500), "generic"),
]


def _inputs(fi, fo, nb1, nb2, dt, act, batch, seed):
    g = torch.Generator().manual_seed(seed)
    dev = lambda *s, scale=1.0: (torch.randn(*s, generator=g) * scale).to("cuda").to(dt)  # noqa: E731
    x = dev(batch, fi)
    w1 = dev(nb1, fo // nb1, fi // nb1, scale=(nb1 / fi) ** 0.5)
    w2 = dev(nb2, fo // nb2, fo // nb2, scale=(nb2 / fo) ** 0.5)
    dy = dev(batch, fo)
    y, z = T.monarch_forward(x, w1, w2, act)
    return x, w1, w2, dy, y, z


def _noalloc(dy, x, w1, w2, z, y, fi, fo, nb1, nb2, act):
    dx, dw1, dw2 = torch.empty_like(x), torch.empty_like(w1), torch.empty_like(w2)
    code = T.dtype_code(x)
    B.monarch_bwd_noalloc(dy, x, w1, w2, z, y if act == B.ACT_RELU else None, dx, dw1, dw2, fi,
                          fo, nb1, nb2, x.shape[0], code, act)
    return dx, dw1, dw2


@pytest.mark.parametrize("fi,fo,nb1,nb2,dt,act,batches,path", CASES)
def test_noalloc_matches_monarch_bwd(fi, fo, nb1, nb2, dt, act, batches, path):
    code = T.dtype_code(torch.empty(0, dtype=dt))
    desc = B.monarch_describe(1, fi, fo, nb1, nb2, batches[0], code, act)
    assert desc[0].startswith(path), desc
    for i, batch in enumerate(batches):
        need = B.monarch_bwd_workspace_bytes(fi, fo, nb1, nb2, batch, code)
        assert 0 < need <= B.NOALLOC_SCRATCH_BYTES
        print(f"noalloc {path} {fi}x{fo} nb {nb1}/{nb2} {dt} act {act} batch {batch}", flush=True)
        x, w1, w2, dy, y, z = _inputs(fi, fo, nb1, nb2, dt, act, batch, seed=1000 + 10 * i)
        ref = T.monarch_backward(dy, x, w1, w2, z, y if act == B.ACT_RELU else None, act)
        got = _noalloc(dy, x, w1, w2, z, y, fi, fo, nb1, nb2, act)
        torch.cuda.synchronize()
        for name, a, r in zip(("dx", "dw1", "dw2"), got, ref):
            assert torch.equal(a.view(torch.int16 if dt == torch.bfloat16 else torch.int32),
                               r.view(torch.int16 if dt == torch.bfloat16 else torch.int32)), \
                (path, batch, name)


def test_noalloc_matches_oracle():
    # the same call checked against the fp64 oracle at the bf16 bound (2e-2)
    fi, fo, nb, batch = 1024, 1024, 32, 600
    x, w1, w2, dy, y, z = _inputs(fi, fo, nb, nb, torch.bfloat16, B.ACT_NONE, batch, seed=77)
    got = _noalloc(dy, x, w1, w2, z, None, fi, fo, nb, nb, B.ACT_NONE)
    torch.cuda.synchronize()
    h = lambda t: t.float().cpu().numpy().astype(np.float64)  # noqa: E731
    ref = O.backward(h(dy), h(x), h(w1), h(w2), fi, fo)
    for a, r in zip(got, ref):
        assert O.rel_frobenius(h(a), r) <= 2e-2


def test_noalloc_rejects_oversized_problem():
    x = torch.empty(16, 16, device="cuda", dtype=torch.bfloat16)
    with pytest.raises(B.MonarchError) as e:
        B.monarch_bwd_noalloc(x, x, x, x, x, None, x, x, x, 16384, 16384, 128, 128, 65536,
                              B.BF16)
    assert e.value.status == B.MONARCH_ERR_SCRATCH
