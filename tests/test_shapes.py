"""Shape validation of the tensor-level helpers (CPU, no kernel launched).

The kernels take every extent from the sizes passed through the C ABI, so a
tensor of another shape would be read or written past its end. The helpers
in torch_api check every tensor's exact shape before anything else (before
the device check, so these run on host tensors and prove that the call stops
before the library is reached); a correctly shaped host tensor gets as far as
the device check.
"""
import pytest
import torch

from monarch_block_diagonal_amd import binding as B
from monarch_block_diagonal_amd import torch_api as T


def _t(*shape, dtype=torch.float32):
    return torch.zeros(shape, dtype=dtype)


def _shape_error(fn, *a, **k):
    with pytest.raises(ValueError) as e:
        fn(*a, **k)
    assert "GPU" not in str(e.value), str(e.value)


def _reaches_device_check(fn, *a, **k):
    with pytest.raises(ValueError, match="GPU"):
        fn(*a, **k)


def test_square_forward_rejects_expanding_layer_weights():
    # MonarchLinear's expanding-layer shapes (768 -> 3072, 4 blocks: mid = in)
    # are not the mid = out layout of monarch_forward
    x = _t(8, 768)
    w1, w2 = _t(4, 192, 192), _t(4, 768, 192)
    _shape_error(T.monarch_forward, x, w1, w2)
    _shape_error(T.MonarchLinearFunction.apply, x, w1, w2)
    # the mid = out layout of the same layer is accepted up to the device check
    _reaches_device_check(T.monarch_forward, x, _t(4, 768, 192), _t(4, 768, 768))


@pytest.mark.parametrize("bad", [
    dict(w1=(4, 16, 8)),            # q1i != in/b1
    dict(w1=(4, 8, 16)),            # q1o != out/b1
    dict(w2=(4, 16, 8)),            # q2i != out/b2
    dict(x=(5, 48)),                # in not a multiple of b1 * q1i
])
def test_square_forward_shapes(bad):
    shapes = dict(x=(5, 64), w1=(4, 16, 16), w2=(4, 16, 16))
    shapes.update(bad)
    _shape_error(T.monarch_forward, _t(*shapes["x"]), _t(*shapes["w1"]), _t(*shapes["w2"]))


@pytest.mark.parametrize("name,shape", [("dy", (5, 32)), ("dy", (4, 64)), ("z", (5, 65)),
                                        ("y", (6, 64))])
def test_square_backward_shapes(name, shape):
    args = dict(dy=_t(5, 64), x=_t(5, 64), w1=_t(4, 16, 16), w2=_t(4, 16, 16), z=_t(5, 64),
                y=_t(5, 64))
    args[name] = _t(*shape)
    _shape_error(T.monarch_backward, args["dy"], args["x"], args["w1"], args["w2"], args["z"],
                 args["y"], B.ACT_RELU)


def test_square_backward_relu_needs_y():
    _shape_error(T.monarch_backward, _t(5, 64), _t(5, 64), _t(4, 16, 16), _t(4, 16, 16),
                 _t(5, 64), None, B.ACT_RELU)
    _reaches_device_check(T.monarch_backward, _t(5, 64), _t(5, 64), _t(4, 16, 16),
                          _t(4, 16, 16), _t(5, 64))


def test_general_layer_shapes():
    # in = 100, out = 70, 4 blocks, mid = 96: w1 [4, 24, 25], w2 [4, 18, 24]
    x = _t(3, 100)
    w1, w2, bias = _t(4, 24, 25), _t(4, 18, 24), _t(70)
    _reaches_device_check(T.monarch_forward_ex, x, w1, w2, 70, bias)
    _shape_error(T.monarch_forward_ex, x, _t(4, 24, 26), w2, 70, bias)   # w1[2] != ceil(in/b1)
    _shape_error(T.monarch_forward_ex, x, w1, _t(4, 17, 24), 70, bias)   # w2[1] != ceil(out/b2)
    _shape_error(T.monarch_forward_ex, x, w1, _t(4, 18, 20), 70, bias)   # mid disagrees
    _shape_error(T.monarch_forward_ex, x, w1, w2, 70, _t(71))            # bias length
    _shape_error(T.monarch_forward_ex, x, w1, w2, 70, _t(7, 10))         # bias rank
    z = _t(3, 96)
    _reaches_device_check(T.monarch_backward_ex, _t(3, 70), x, w1, w2, z)
    _shape_error(T.monarch_backward_ex, _t(3, 70), x, w1, w2, _t(3, 100))   # z != [batch, mid]
    _shape_error(T.monarch_backward_ex, _t(3, 70), x, w1, w2, z, _t(3, 71), False, B.ACT_RELU)
    _shape_error(T.monarch_backward_ex, _t(2, 70), x, w1, w2, z)           # dy batch


def test_hypercube_shapes():
    dims = (4, 6, 8)
    x = _t(3, 192)
    ws = [_t(48, 4, 4), _t(32, 6, 6), _t(24, 8, 8)]
    _reaches_device_check(T.hyper_forward, x, ws, dims)
    _shape_error(T.hyper_forward, x, [ws[0], _t(24, 8, 8), ws[2]], dims)
    _shape_error(T.hyper_forward, _t(3, 191), ws, dims)
    _shape_error(T.hyper_forward, x, ws[:2], dims)
    saved = _t(B.monarch_hyper_saved_elems(dims, 3))
    _shape_error(T.hyper_backward, _t(3, 190), x, ws, saved, dims)
    _shape_error(T.hyper_backward, _t(3, 192), x, ws, _t(10), dims)
    _reaches_device_check(T.hyper_backward, _t(3, 192), x, ws, saved, dims)


def test_dyad_shapes():
    x, wa = _t(3, 64), _t(4, 8, 16)
    _reaches_device_check(T.dyad_forward, x, wa, _t(4, 8, 16))
    _shape_error(T.dyad_forward, x, wa, _t(4, 16, 8))
    _shape_error(T.dyad_forward, _t(3, 60), wa, _t(4, 8, 16))
    _shape_error(T.dyad_backward, _t(3, 33), x, wa, _t(4, 8, 16))
    _reaches_device_check(T.dyad_backward, _t(3, 32), x, wa, _t(4, 8, 16))
