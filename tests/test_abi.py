"""The C ABI library loads, exports every function include/*.h declares, sizes its
workspace and rejects bad arguments before launching anything (CPU only: no call here
reaches the GPU)."""
import ctypes
import glob
import os
import re

import pytest

from local_sparse_attention_amd import dsa3d

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADERS = sorted(glob.glob(os.path.join(ROOT, "include", "*.h")))

OK, ERR_NULL, ERR_DTYPE, ERR_HEAD_DIM, ERR_GRID, ERR_WINDOW, ERR_ALIGN, ERR_WORKSPACE, ERR_LAUNCH, ERR_SCALE = (
    0, -1, -2, -3, -4, -5, -6, -7, -8, -9)
ERR_FLAGS, ERR_SCRATCH = -10, -11


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(dsa3d.LIBPATH):
        from local_sparse_attention_amd import _build
        _build.build_lib()
    return dsa3d.load()


def declared_functions():
    names = set()
    for h in HEADERS:
        text = re.sub(r"/\*.*?\*/", "", open(h).read(), flags=re.S)
        names |= set(re.findall(r"\b(dsa3d_\w+)\s*\(", text))
    return sorted(names)


def test_exports_every_declared_function(lib):
    names = declared_functions()
    assert set(names) >= {"dsa3d_forward", "dsa3d_backward", "dsa3d_window_starts", "dsa3d_workspace_bytes",
                          "dsa3d_status_string", "dsa3d_forward_heads", "dsa3d_sampled_forward",
                          "dsa3d_sampled_backward", "dsa3d_peak_mfma_bf16"}
    for n in names:
        assert hasattr(lib, n), n


def test_status_strings(lib):
    for code in (OK, ERR_NULL, ERR_DTYPE, ERR_HEAD_DIM, ERR_GRID, ERR_WINDOW, ERR_ALIGN, ERR_WORKSPACE, ERR_LAUNCH,
                 ERR_SCALE, ERR_FLAGS, ERR_SCRATCH):
        s = dsa3d.status_string(code)
        assert s and s != "unknown status"
    assert dsa3d.status_string(-100) == "unknown status"


def test_workspace_bytes(lib):
    fwd = lib.dsa3d_workspace_bytes(256, 68, 120, 16, 5, 9, 9, 0)
    bwd = lib.dsa3d_workspace_bytes(256, 68, 120, 16, 5, 9, 9, 1)
    N = 256 * 68 * 120
    assert fwd > 16 * N and bwd >= fwd + 4 * 16 * N  # starts + fp32 Delta [H][N]
    # key-centric dK/dV item lists: every query listed for at most 3 x 3 key block
    # columns, 12 bytes each (token, window start y / x)
    assert bwd >= fwd + 4 * 16 * N + 9 * 12 * N
    assert bwd < 400 * N  # modest: a tenth of one [N][16][128] bf16 tensor
    assert lib.dsa3d_workspace_bytes(4, 8, 8, 2, 3, 3, 3, 1) > 0
    # invalid geometry -> 0
    assert lib.dsa3d_workspace_bytes(4, 8, 8, 2, 2, 3, 3, 0) == 0
    assert lib.dsa3d_workspace_bytes(4, 8, 8, 2, 5, 3, 3, 0) == 0
    assert lib.dsa3d_workspace_bytes(0, 8, 8, 2, 1, 3, 3, 0) == 0
    assert lib.dsa3d_workspace_bytes(4, 8, 8, 0, 3, 3, 3, 0) == 0


P = 1 << 20  # a fake, aligned, non-null "device" address: validation fails before any use


def fwd(lib, flags=None, **kw):
    a = dict(q=P, k=P, v=P, off=P, F=4, Hp=8, Wp=8, H=2, D=64, kt=3, ky=3, kx=3, scale=0.125, dtype=1, out=P, lse=P,
             ws=P, wsb=1 << 40)
    a.update(kw)
    args = (a["q"], a["k"], a["v"], a["off"], a["F"], a["Hp"], a["Wp"], a["H"], a["D"], a["kt"], a["ky"], a["kx"],
            a["scale"], a["dtype"], a["out"], a["lse"], a["ws"], a["wsb"], None)
    if flags is None:
        return lib.dsa3d_forward(*args)
    return lib.dsa3d_forward_ex(*args, flags, None)


def bwd(lib, flags=None, **kw):
    a = dict(q=P, k=P, v=P, off=P, o=P, lse=P, do=P, F=4, Hp=8, Wp=8, H=2, D=64, kt=3, ky=3, kx=3, scale=0.125,
             dtype=0, dq=P, dk=P, dv=P, ws=P, wsb=1 << 40)
    a.update(kw)
    args = (a["q"], a["k"], a["v"], a["off"], a["o"], a["lse"], a["do"], a["F"], a["Hp"], a["Wp"], a["H"], a["D"],
            a["kt"], a["ky"], a["kx"], a["scale"], a["dtype"], a["dq"], a["dk"], a["dv"], a["ws"], a["wsb"], None)
    if flags is None:
        return lib.dsa3d_backward(*args)
    return lib.dsa3d_backward_ex(*args, flags, None)


@pytest.mark.parametrize("call", [fwd, bwd])
def test_argument_validation(lib, call):
    assert call(lib, q=None) == ERR_NULL
    assert call(lib, ws=None) == ERR_NULL
    assert call(lib, dtype=2) == ERR_DTYPE
    assert call(lib, D=96) == ERR_HEAD_DIM
    assert call(lib, D=256) == ERR_HEAD_DIM
    assert call(lib, F=0) == ERR_GRID
    assert call(lib, H=0) == ERR_GRID
    assert call(lib, H=70000) == ERR_GRID
    assert call(lib, F=1024, Hp=1024, Wp=1024) == ERR_GRID
    assert call(lib, kt=2) == ERR_WINDOW
    assert call(lib, kx=9) == ERR_WINDOW
    assert call(lib, ky=0) == ERR_WINDOW
    assert call(lib, scale=float("inf")) == ERR_SCALE
    assert call(lib, scale=float("nan")) == ERR_SCALE
    assert call(lib, q=P + 8) == ERR_ALIGN
    assert call(lib, ws=P + 4) == ERR_ALIGN
    assert call(lib, wsb=1000) == ERR_WORKSPACE
    assert call(lib, flags=2) == ERR_FLAGS
    assert call(lib, flags=0x80000000) == ERR_FLAGS
    # thin grids: N < 2^30 but 2^28 blobs of start cells (32-bit sort keys of 16 cells each)
    assert call(lib, F=1 << 28, Hp=1, Wp=1, kt=1, ky=1, kx=1) == ERR_GRID
    assert call(lib, F=(1 << 27) - 1, Hp=1, Wp=1, kt=1, ky=1, kx=1, wsb=1000) == ERR_WORKSPACE


def test_start_cell_bound(lib):
    assert lib.dsa3d_workspace_bytes(1 << 28, 1, 1, 1, 1, 1, 1, 0) == 0
    assert lib.dsa3d_workspace_bytes((1 << 27) - 1, 1, 1, 1, 1, 1, 1, 0) > 0
    assert lib.dsa3d_window_starts(P, 1 << 28, 1, 1, 1, 1, 1, P, None) == ERR_GRID


def test_window_starts_validation(lib):
    f = lib.dsa3d_window_starts
    assert f(None, 4, 8, 8, 3, 3, 3, P, None) == ERR_NULL
    assert f(P, 4, 8, 8, 3, 4, 3, P, None) == ERR_WINDOW
    assert f(P, 4, 8, 8, 5, 3, 3, P, None) == ERR_WINDOW
    assert f(P, -1, 8, 8, 3, 3, 3, P, None) == ERR_GRID
    assert f(P + 2, 4, 8, 8, 3, 3, 3, P, None) == ERR_ALIGN


def test_binding_refuses_cpu_tensors(lib):
    import torch

    q = torch.zeros(256, 2, 64)
    off = torch.zeros(256, 3, dtype=torch.int32)
    with pytest.raises(dsa3d.DSA3DError, match="GPU"):
        dsa3d.forward(q, q, q, off, (4, 8, 8), (3, 3, 3), ws=torch.zeros(1 << 20, dtype=torch.uint8))


def test_binding_checks_shapes_and_dtypes(lib):
    """Every tensor argument is checked for shape and dtype before any pointer reaches the
    library (int64 offsets, a wrongly shaped lse or an undersized output would otherwise be
    read or written as raw memory)."""
    import torch

    grid, window = (4, 8, 8), (3, 3, 3)
    q = torch.zeros(256, 2, 64)
    off = torch.zeros(256, 3, dtype=torch.int32)
    lse = torch.zeros(2, 256)
    E = dsa3d.DSA3DError
    with pytest.raises(E, match="offsets has dtype"):
        dsa3d.forward(q, q, q, off.long(), grid, window)
    with pytest.raises(E, match="offsets has shape"):
        dsa3d.forward(q, q, q, off[:, :2].contiguous(), grid, window)
    with pytest.raises(E, match="k has shape"):
        dsa3d.forward(q, q[:128], q, off, grid, window)
    with pytest.raises(E, match="v has dtype"):
        dsa3d.forward(q, q, q.bfloat16(), off, grid, window)
    with pytest.raises(E, match="out has shape"):
        dsa3d.forward(q, q, q, off, grid, window, out=q[:100])
    with pytest.raises(E, match="lse has shape"):
        dsa3d.forward(q, q, q, off, grid, window, lse=lse.T.contiguous())
    with pytest.raises(E, match="lse has dtype"):
        dsa3d.forward(q, q, q, off, grid, window, lse=lse.double())
    with pytest.raises(E, match="tokens"):
        dsa3d.forward(q, q, q, off, (4, 8, 9), window)
    with pytest.raises(E, match="unsupported dtype"):
        dsa3d.forward(q.half(), q.half(), q.half(), off, grid, window)
    with pytest.raises(E, match="lse has shape"):
        dsa3d.backward(q, q, q, off, q, lse[:1], q, grid, window)
    with pytest.raises(E, match="lse has dtype"):
        dsa3d.backward(q, q, q, off, q, lse.bfloat16(), q, grid, window)
    with pytest.raises(E, match="offsets has dtype"):
        dsa3d.backward(q, q, q, off.long(), q, lse, q, grid, window)
    with pytest.raises(E, match="dout has shape"):
        dsa3d.backward(q, q, q, off, q, lse, q[:, :1], grid, window)
    with pytest.raises(E, match="dk has dtype"):
        dsa3d.backward(q, q, q, off, q, lse, q, grid, window, dk=q.bfloat16())
    with pytest.raises(E, match="dv has shape"):
        dsa3d.backward(q, q, q, off, q, lse, q, grid, window, dv=q[:10])
    with pytest.raises(E, match="offsets has dtype"):
        dsa3d.window_starts(off.long(), grid, window)
