"""Host-side checks of the C ABI: the library loads, exports every symbol the
header declares, and rejects bad arguments before any HIP call (these run
without a GPU; no call here reaches a kernel launch)."""
import ctypes
import os
import re

import pytest

import monarch_block_diagonal_amd as M
from monarch_block_diagonal_amd import binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "monarch.h")

A = 0x10000      # fake 16-byte-aligned device addresses (never dereferenced)
A2 = 0x20000
MIS = 0x10008    # 8-byte but not 16-byte aligned


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(monarch_[a-z_0-9]+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    lib = M.load_library()
    declared = header_functions()
    assert declared, "no declarations parsed"
    for name in declared:
        assert hasattr(lib, name), name
    assert set(declared) == set(B.EXPORTED)


def test_abi_version_matches_header():
    text = open(HEADER).read()
    ver = int(re.search(r"#define MONARCH_ABI_VERSION (\d+)", text).group(1))
    assert M.monarch_abi_version() == ver


def test_status_strings():
    for st in (0, -1, -2, -3, -4, -5, -6, -7, 7):
        s = M.monarch_status_string(st)
        assert isinstance(s, str) and s
    assert "aligned" in M.monarch_status_string(B.MONARCH_ERR_ALIGN)


def fwd(x=A, w1=A, w2=A, y=A2, z=A2, fi=16, fo=16, nb1=4, nb2=4, b=8, dt=B.F32, act=B.ACT_NONE):
    lib = M.load_library()
    return lib.monarch_fwd(x, w1, w2, y, z, fi, fo, nb1, nb2, b, dt, act, None)


def bwd(dy=A, x=A, w1=A, w2=A, z=A, y=A, dx=A2, dw1=A2, dw2=A2, ws=A2, wsb=1 << 40, fi=16,
        fo=16, nb1=4, nb2=4, b=8, dt=B.F32, act=B.ACT_NONE):
    lib = M.load_library()
    return lib.monarch_bwd(dy, x, w1, w2, z, y, dx, dw1, dw2, ws, wsb, fi, fo, nb1, nb2, b, dt,
                           act, None)


@pytest.mark.parametrize("kw", [dict(dt=2), dict(dt=-1), dict(act=2), dict(act=-1)])
def test_bad_dtype_or_act(kw):
    assert fwd(**kw) == B.MONARCH_ERR_DTYPE
    assert bwd(**kw) == B.MONARCH_ERR_DTYPE


@pytest.mark.parametrize("kw", [
    dict(fi=0), dict(fo=0), dict(nb1=0), dict(nb2=0), dict(b=-1), dict(fi=-16),
    dict(fi=18),                 # in % nb1
    dict(fo=18, nb2=2),          # mid % nb1
    dict(fo=20, nb1=4, nb2=8),   # mid % nb2
    dict(fi=1 << 31, nb1=1),     # per-dimension limit
])
def test_bad_shapes(kw):
    assert fwd(**kw) == B.MONARCH_ERR_SHAPE
    assert bwd(**kw) == B.MONARCH_ERR_SHAPE
    args = {k: kw.get(k, d) for k, d in dict(fi=16, fo=16, nb1=4, nb2=4, b=8).items()}
    assert M.monarch_bwd_workspace_bytes(args["fi"], args["fo"], args["nb1"], args["nb2"],
                                         args["b"], 0) == 0


@pytest.mark.parametrize("name", ["x", "w1", "w2", "y", "z"])
def test_fwd_null_pointers(name):
    assert fwd(**{name: None}) == B.MONARCH_ERR_NULL


@pytest.mark.parametrize("name", ["dy", "x", "w1", "w2", "z", "dx", "dw1", "dw2", "ws"])
def test_bwd_null_pointers(name):
    assert bwd(**{name: None}) == B.MONARCH_ERR_NULL


def test_bwd_relu_needs_y():
    assert bwd(y=None, act=B.ACT_RELU) == B.MONARCH_ERR_NULL


@pytest.mark.parametrize("name", ["x", "w1", "w2", "y", "z"])
def test_fwd_misaligned(name):
    assert fwd(**{name: MIS}) == B.MONARCH_ERR_ALIGN


@pytest.mark.parametrize("name", ["dy", "x", "w1", "w2", "z", "y", "dx", "dw1", "dw2", "ws"])
def test_bwd_misaligned(name):
    assert bwd(**{name: MIS}) == B.MONARCH_ERR_ALIGN


def test_bwd_workspace_too_small():
    need = M.monarch_bwd_workspace_bytes(16, 16, 4, 4, 8, 0)
    assert need > 0
    assert bwd(wsb=need - 1) == B.MONARCH_ERR_WORKSPACE
    assert bwd(wsb=0) == B.MONARCH_ERR_WORKSPACE


def test_batch_zero_forward_is_a_no_op():
    # no launch: null activations are accepted and nothing touches the GPU
    assert fwd(x=None, y=None, z=None, b=0) == B.MONARCH_OK
    assert M.monarch_bwd_workspace_bytes(16, 16, 4, 4, 0, 0) == 0
    assert M.monarch_describe(0, 16, 16, 4, 4, 0, 0) == []
    assert M.monarch_describe(1, 16, 16, 4, 4, 0, 0) == ["zero_dw"]


def test_workspace_grows_with_batch_and_dtype():
    a = M.monarch_bwd_workspace_bytes(1024, 1024, 32, 32, 4096, B.BF16)
    b = M.monarch_bwd_workspace_bytes(1024, 1024, 32, 32, 8192, B.BF16)
    c = M.monarch_bwd_workspace_bytes(1024, 1024, 32, 32, 4096, B.F32)
    assert 0 < a < b and a < c
    big = M.monarch_bwd_workspace_bytes(16384, 16384, 128, 128, 65536, B.BF16)
    assert big >= 65536 * 16384 * 2


def test_describe_lists_kernels():
    f = M.monarch_describe(0, 1024, 1024, 32, 32, 4096, B.BF16)
    b = M.monarch_describe(1, 1024, 1024, 32, 32, 4096, B.BF16)
    assert len(f) >= 1 and len(b) >= 1
    assert all(isinstance(n, str) and n for n in f + b)
    with pytest.raises(M.MonarchError):
        M.monarch_describe(0, 18, 16, 4, 4, 8, 0)


def test_binding_raises_on_error():
    with pytest.raises(M.MonarchError) as e:
        M.monarch_fwd(None, A, A, A, A, 16, 16, 4, 4, 8, B.F32, B.ACT_NONE, stream=0)
    assert e.value.status == B.MONARCH_ERR_NULL


def test_path_selection():
    # 128x128 bf16 blocks, 32, 64 or 128 of them, take the square fast path
    for n, nb in [(16384, 128), (8192, 64), (4096, 32)]:
        assert all(k.startswith("sq128") for k in M.monarch_describe(0, n, n, nb, nb, 64, B.BF16))
        assert M.monarch_describe(1, n, n, nb, nb, 64, B.BF16)[0].startswith("sq128")
    # 32x32 bf16 blocks, 8, 16 or 32 of them, take the fused small-block path
    for n, nb in [(1024, 32), (512, 16), (256, 8)]:
        assert M.monarch_describe(0, n, n, nb, nb, 64, B.BF16) == ["sm32_fwd"]
        assert M.monarch_describe(1, n, n, nb, nb, 64, B.BF16, B.ACT_RELU) == [
            "sm32_bwd_data", "sm32_bwd_weight", "reduce_dw"]
    # everything else takes the generic path
    for args in [(16384, 16384, 128, 128, 64, B.F32), (1024, 1024, 32, 32, 64, B.F32),
                 (2048, 2048, 64, 64, 64, B.BF16), (1024, 1024, 8, 8, 64, B.BF16), (2048, 2048, 16, 16, 64, B.BF16),
                 (768, 3072, 4, 4, 64, B.BF16), (512, 512, 4, 4, 64, B.BF16),
                 (12288, 12288, 96, 96, 64, B.BF16)]:
        assert M.monarch_describe(0, *args)[0].startswith("generic")


def proj(m=A, w1=A2, w2=A2, fi=16, fo=16, nb1=4, nb2=4, dt=B.F32, steps=8, conv=None):
    lib = M.load_library()
    return lib.monarch_project(m, w1, w2, fi, fo, nb1, nb2, dt, steps, conv, None)


@pytest.mark.parametrize("kw", [
    dict(fo=32),                      # out != nb1 * nb2
    dict(fi=18),                      # in % nb1
    dict(nb1=0), dict(fi=0),
    dict(steps=0), dict(steps=5000),
    dict(fi=256 * 512, fo=16, nb1=4, nb2=4),   # slice 4 x 32768: a side beyond 128
    dict(fi=4 * 129, fo=16, nb1=4, nb2=4),     # 4 x 129
    dict(fi=516, fo=516, nb1=129, nb2=4),      # slices 129 x 4
])
def test_project_bad_shapes(kw):
    assert proj(**kw) == B.MONARCH_ERR_SHAPE


def test_project_bad_dtype_null_align():
    assert proj(dt=3) == B.MONARCH_ERR_DTYPE
    for name in ("m", "w1", "w2"):
        assert proj(**{name: None}) == B.MONARCH_ERR_NULL
        assert proj(**{name: MIS}) == B.MONARCH_ERR_ALIGN
    assert proj(conv=A2 + 2) == B.MONARCH_ERR_ALIGN   # int32 status array


# ---------------------------------------------------------------------------
# general layer (*_ex): explicit mid, zero padding, truncation, bias

def fwd_ex(x=A, w1=A, w2=A, bias=None, y=A2, z=A2, fi=10, fo=7, mid=8, nb1=4, nb2=4, b=5,
           dt=B.F32, act=B.ACT_NONE):
    lib = M.load_library()
    return lib.monarch_fwd_ex(x, w1, w2, bias, y, z, fi, fo, mid, nb1, nb2, b, dt, act, None,
                              None, 0)


def bwd_ex(dy=A, x=A, w1=A, w2=A, z=A, y=A, dx=A2, dw1=A2, dw2=A2, db=None, ws=A2, wsb=1 << 40,
           fi=10, fo=7, mid=8, nb1=4, nb2=4, b=5, dt=B.F32, act=B.ACT_NONE):
    lib = M.load_library()
    return lib.monarch_bwd_ex(dy, x, w1, w2, z, y, dx, dw1, dw2, db, ws, wsb, fi, fo, mid, nb1,
                              nb2, b, dt, act, None, None, 0)


def test_linear_mid_follows_the_constructor_rule():
    # ceil block sizes; mid = in_ext when in_ext < out_ext, else out_ext
    assert M.monarch_linear_mid(768, 3072, 4) == 768
    assert M.monarch_linear_mid(3072, 768, 4) == 768
    assert M.monarch_linear_mid(10, 7, 4) == 8
    assert M.monarch_linear_mid(5, 13, 4) == 8
    assert M.monarch_linear_mid(10000, 1024, 16) == 1024
    with pytest.raises(M.MonarchError):
        M.monarch_linear_mid(0, 8, 4)


@pytest.mark.parametrize("kw", [
    dict(mid=10),                 # mid % nb1
    dict(mid=12, nb2=8),          # mid % nb2
    dict(mid=0), dict(fi=0), dict(fo=0), dict(b=-1), dict(nb1=0),
    dict(fi=1 << 31, nb1=1),
])
def test_ex_bad_shapes(kw):
    assert fwd_ex(**kw) == B.MONARCH_ERR_SHAPE
    assert bwd_ex(**kw) == B.MONARCH_ERR_SHAPE


def test_ex_accepts_padded_sizes_and_checks_pointers():
    # padded in/out are valid shapes: the pointer checks decide
    assert fwd_ex(x=0) == B.MONARCH_ERR_NULL
    assert fwd_ex(bias=MIS) == B.MONARCH_ERR_ALIGN
    assert bwd_ex(db=MIS) == B.MONARCH_ERR_ALIGN
    assert bwd_ex(wsb=0) == B.MONARCH_ERR_WORKSPACE
    assert bwd_ex(act=B.ACT_RELU, y=None) == B.MONARCH_ERR_NULL
    assert fwd_ex(b=0, x=None, y=None, z=None) == B.MONARCH_OK


def test_ex_workspace_and_plan():
    need = M.monarch_bwd_ex_workspace_bytes(10, 7, 8, 4, 4, 5, B.F32, True)
    need_nb = M.monarch_bwd_ex_workspace_bytes(10, 7, 8, 4, 4, 5, B.F32, False)
    assert need > need_nb > 0
    names = M.monarch_describe_ex(1, 10, 7, 8, 4, 4, 5, B.F32, B.ACT_NONE, True)
    assert "generic_bias_partials" in names and names[-1] == "reduce_dw"
    # whole blocks, mid = out, no bias: the same plan as monarch_describe
    for d in (0, 1):
        assert (M.monarch_describe_ex(d, 16384, 16384, 16384, 128, 128, 4096, B.BF16)
                == M.monarch_describe(d, 16384, 16384, 128, 128, 4096, B.BF16))
    # a bias moves even the square shape to the generic path
    names = M.monarch_describe_ex(0, 16384, 16384, 16384, 128, 128, 4096, B.BF16, B.ACT_NONE, True)
    assert all(n.startswith("generic_") for n in names)
    assert M.monarch_bwd_ex_workspace_bytes(16, 16, 16, 4, 4, 8, B.F32) == \
        M.monarch_bwd_workspace_bytes(16, 16, 4, 4, 8, B.F32)


# ---------------------------------------------------------------------------
# k-factor (hypercube) layer

def test_hyper_sizes_and_plan():
    dims = (16, 24, 32)
    assert M.monarch_hyper_saved_elems(dims, 10) == 3 * 10 * 12288
    assert M.monarch_hyper_saved_elems((64,), 10) == 0
    assert M.monarch_hyper_describe(0, dims, 10, B.F32) == (
        ["hyper_transpose"] + ["hyper_round_fwd", "hyper_permute"] * 2 + ["hyper_round_fwd"])
    # bf16: round 0 reads x in its natural layout (joined with the transpose),
    # round 1's swap arrays ([32][24], 768 elements) are small enough for the
    # fused round-and-swap kernel, round 0's (12288) are not
    assert M.monarch_hyper_describe(0, dims, 10, B.BF16) == (
        ["hyper_transpose_round_fwd", "hyper_permute", "hyper_round_fwd_swap", "hyper_round_fwd"])
    assert M.monarch_hyper_describe(0, (64,), 10, B.BF16) == ["hyper_round_fwd"]
    names = M.monarch_hyper_describe(1, dims, 10, B.F32)
    assert names == (["hyper_round_bwd_weight", "hyper_round_bwd_data", "hyper_permute"] * 2
                     + ["hyper_round_bwd_weight", "hyper_round_bwd_data", "hyper_transpose"]
                     + ["reduce_dw"])
    # bf16 fibers of 16, 24 or 32 units take the fiber kernel, whose data
    # products use per-fiber transposed weights
    names = M.monarch_hyper_describe(1, dims, 10, B.BF16)
    step = ["hyper_round_bwd_weight", "hyper_weight_transpose", "hyper_round_bwd_data"]
    assert names == (step[:2] + ["hyper_round_bwd_data_swap"] + step + ["hyper_permute"]
                     + step[:2] + ["hyper_round_bwd_data_transpose", "reduce_dw"])
    assert M.monarch_hyper_describe(1, (64,), 10, B.BF16) == [
        "hyper_round_bwd_weight", "hyper_round_bwd_data", "reduce_dw"]
    assert len(M.monarch_hyper_describe(1, (2, 3, 4, 5), 10, B.BF16)) == 14
    assert M.monarch_hyper_describe(1, (2, 2, 2, 2), 10, B.F32)[-2:] == ["reduce_dw", "reduce_dw"]
    assert M.monarch_hyper_describe(1, dims, 0, B.BF16) == ["zero_dw"] * 3
    assert M.monarch_hyper_bwd_workspace_bytes(dims, 1000, B.BF16) > 0


@pytest.mark.parametrize("dims", [(), (2, 2, 2, 2, 2), (0, 4), (4, -1), (1 << 16, 1 << 16)])
def test_hyper_bad_lattice(dims):
    lib = M.load_library()
    d = (ctypes.c_int64 * max(len(dims), 1))(*dims)
    w = (ctypes.c_void_p * 5)(*([A] * 5))
    assert lib.monarch_hyper_fwd(A, w, A2, A2, len(dims), d, 4, B.F32, None, None, 0) == \
        B.MONARCH_ERR_SHAPE


def test_hyper_pointer_checks():
    lib = M.load_library()
    d = (ctypes.c_int64 * 2)(4, 8)
    w = (ctypes.c_void_p * 2)(A, A)
    wnull = (ctypes.c_void_p * 2)(A, None)
    wmis = (ctypes.c_void_p * 2)(A, MIS)
    assert lib.monarch_hyper_fwd(A, wnull, A2, A2, 2, d, 4, B.F32, None, None, 0) == B.MONARCH_ERR_NULL
    assert lib.monarch_hyper_fwd(A, wmis, A2, A2, 2, d, 4, B.F32, None, None, 0) == B.MONARCH_ERR_ALIGN
    assert lib.monarch_hyper_fwd(A, w, A2, None, 2, d, 4, B.F32, None, None, 0) == B.MONARCH_ERR_NULL
    assert lib.monarch_hyper_fwd(A, w, A2, A2, 2, d, 4, 7, None, None, 0) == B.MONARCH_ERR_DTYPE
    dw = (ctypes.c_void_p * 2)(A2, A2)
    assert lib.monarch_hyper_bwd(A, A, w, A, A2, dw, A2, 0, 2, d, 4, B.F32, None, None, 0) == \
        B.MONARCH_ERR_WORKSPACE


# ---------------------------------------------------------------------------
# DYAD-style layer

def test_dyad_plan_and_checks():
    # term B goes through block-major rows, added in by an accumulating swap
    assert M.monarch_dyad_describe(0, 64, 32, 4, 10, B.BF16) == [
        "dyad_gather_x", "dyad_term_b_fwd", "dyad_term_a_fwd", "dyad_add_term_b"]
    assert M.monarch_dyad_describe(1, 64, 32, 4, 10, B.BF16) == [
        "dyad_gather_x", "dyad_gather_dy", "dyad_term_a_bwd_weight", "dyad_term_b_bwd_weight",
        "dyad_term_b_bwd_data", "dyad_term_a_bwd_data", "dyad_add_term_b", "reduce_dw"]
    # the forward workspace holds block-major x and term B's rows
    assert M.monarch_dyad_fwd_workspace_bytes(64, 32, 4, 1000, B.F32) >= 1000 * (64 + 32) * 4
    assert M.monarch_dyad_describe(1, 64, 32, 4, 0, B.BF16) == ["zero_dw", "zero_dw"]
    assert M.monarch_dyad_bwd_workspace_bytes(64, 32, 4, 1000, B.F32) > 0
    assert M.monarch_dyad_bwd_workspace_bytes(63, 32, 4, 1000, B.F32) == 0
    # the forward's workspace holds x in block-major order
    assert M.monarch_dyad_fwd_workspace_bytes(64, 32, 4, 1000, B.F32) >= 1000 * 64 * 4
    assert M.monarch_dyad_fwd_workspace_bytes(64, 32, 4, 0, B.F32) == 0
    lib = M.load_library()
    big = 1 << 20
    assert lib.monarch_dyad_fwd(A, A, A, A2, A2, big, 63, 32, 4, 8, B.F32, None, None,
                                0) == B.MONARCH_ERR_SHAPE
    assert lib.monarch_dyad_fwd(A, A, A, A2, A2, big, 64, 32, 0, 8, B.F32, None, None,
                                0) == B.MONARCH_ERR_SHAPE
    assert lib.monarch_dyad_fwd(A, None, A, A2, A2, big, 64, 32, 4, 8, B.F32, None, None,
                                0) == B.MONARCH_ERR_NULL
    assert lib.monarch_dyad_fwd(A, A, A, A2, None, big, 64, 32, 4, 8, B.F32, None, None,
                                0) == B.MONARCH_ERR_NULL
    assert lib.monarch_dyad_fwd(MIS, A, A, A2, A2, big, 64, 32, 4, 8, B.F32, None, None,
                                0) == B.MONARCH_ERR_ALIGN
    assert lib.monarch_dyad_fwd(A, A, A, A2, A2, 16, 64, 32, 4, 8, B.F32, None, None,
                                0) == B.MONARCH_ERR_WORKSPACE
    assert lib.monarch_dyad_fwd(A, A, A, A2, A2, big, 64, 32, 4, 8, 5, None, None,
                                0) == B.MONARCH_ERR_DTYPE
    assert lib.monarch_dyad_bwd(A, A, A, A, A2, A2, A2, A2, 0, 64, 32, 4, 8, B.F32, None, None,
                                0) == B.MONARCH_ERR_WORKSPACE


def bwd_noalloc(dy=A, x=A, w1=A, w2=A, z=A, y=A, dx=A2, dw1=A2, dw2=A2, fi=16, fo=16, nb1=4,
                nb2=4, b=8, dt=B.F32, act=B.ACT_NONE):
    lib = M.load_library()
    return lib.monarch_bwd_noalloc(dy, x, w1, w2, z, y, dx, dw1, dw2, fi, fo, nb1, nb2, b, dt,
                                   act, None)


def test_noalloc_checks_before_any_hip_call():
    # every rejection below happens before the library touches the device
    assert bwd_noalloc(dt=2) == B.MONARCH_ERR_DTYPE
    assert bwd_noalloc(fi=18) == B.MONARCH_ERR_SHAPE
    assert bwd_noalloc(dx=0) == B.MONARCH_ERR_NULL
    assert bwd_noalloc(y=0, act=B.ACT_RELU) == B.MONARCH_ERR_NULL
    assert bwd_noalloc(w2=MIS) == B.MONARCH_ERR_ALIGN
    # the largest square layer at full batch needs 4 GiB of workspace
    big = dict(fi=16384, fo=16384, nb1=128, nb2=128, b=65536, dt=B.BF16)
    need = M.monarch_bwd_workspace_bytes(16384, 16384, 128, 128, 65536, B.BF16)
    assert need > B.NOALLOC_SCRATCH_BYTES
    assert bwd_noalloc(**big) == B.MONARCH_ERR_SCRATCH
    assert "scratch" in M.monarch_status_string(B.MONARCH_ERR_SCRATCH)


def test_noalloc_scratch_size_matches_header():
    text = open(HEADER).read()
    m = re.search(r"#define MONARCH_NOALLOC_SCRATCH_BYTES \((\d+)ull << (\d+)\)", text)
    assert m and (int(m.group(1)) << int(m.group(2))) == B.NOALLOC_SCRATCH_BYTES
    # the workloads it is sized for fit: the 1024-feature square layer at 4096
    # rows and both recommender layers at 10000 rows
    for args in ((1024, 1024, 32, 32, 4096, B.BF16), (10000, 1024, 4, 4, 10000, B.F32),
                 (1024, 512, 16, 16, 10000, B.F32)):
        assert M.monarch_bwd_workspace_bytes(*args) <= B.NOALLOC_SCRATCH_BYTES


def test_stream_copy_checks():
    lib = M.load_library()
    assert lib.monarch_stream_copy(A, A2, 0, None) == B.MONARCH_OK      # nothing to do
    assert lib.monarch_stream_copy(None, A2, 64, None) == B.MONARCH_ERR_NULL
    assert lib.monarch_stream_copy(A, None, 64, None) == B.MONARCH_ERR_NULL
    assert lib.monarch_stream_copy(MIS, A2, 64, None) == B.MONARCH_ERR_ALIGN
