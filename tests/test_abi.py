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
    # columns, 8 bytes each (token, mask of the block's keys in its window)
    assert bwd >= fwd + 4 * 16 * N + 9 * 8 * N
    assert bwd < 400 * N  # modest: a tenth of one [N][16][128] bf16 tensor
    assert lib.dsa3d_workspace_bytes(4, 8, 8, 2, 3, 3, 3, 1) > 0
    # invalid geometry -> 0
    assert lib.dsa3d_workspace_bytes(4, 8, 8, 2, 2, 3, 3, 0) == 0
    assert lib.dsa3d_workspace_bytes(4, 8, 8, 2, 5, 3, 3, 0) == 0
    assert lib.dsa3d_workspace_bytes(0, 8, 8, 2, 1, 3, 3, 0) == 0
    assert lib.dsa3d_workspace_bytes(4, 8, 8, 0, 3, 3, 3, 0) == 0


P = 1 << 20  # a fake, aligned, non-null "device" address: every call below fails validation
# before any launch (calls meant to be valid stop at a deliberately null output)


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
    # DSA3D_FLAG_REUSE_PREP (2) is a backward flag
    assert call(lib, flags=2 if call is fwd else 4) == ERR_FLAGS
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


ERR_MODE, ERR_LAYOUT = -12, -13


def test_status_strings_of_the_wider_forms(lib):
    for code in (ERR_MODE, ERR_LAYOUT):
        assert dsa3d.status_string(code) != "unknown status"


def sampled_fwd(lib, **kw):
    a = dict(q=P, k=P, v=P, off=P, sn=3, sh=0, ss=0, mode=0, F=4, Hp=8, Wp=8, H=2, D=64, kt=3, ky=3, kx=3,
             scale=0.125, dtype=1, out=P, lse=P)
    a.update(kw)
    return lib.dsa3d_sampled_forward(a["q"], a["k"], a["v"], a["off"], a["sn"], a["sh"], a["ss"], a["mode"], a["F"],
                                     a["Hp"], a["Wp"], a["H"], a["D"], a["kt"], a["ky"], a["kx"], a["scale"],
                                     a["dtype"], a["out"], a["lse"], None)


def test_sampled_validation(lib):
    f = sampled_fwd
    assert f(lib, q=None) == ERR_NULL
    assert f(lib, off=None) == ERR_NULL
    assert f(lib, mode=2) == ERR_MODE
    assert f(lib, dtype=3) == ERR_DTYPE
    assert f(lib, D=32) == ERR_HEAD_DIM
    assert f(lib, kt=2) == ERR_WINDOW
    assert f(lib, kt=5) == ERR_WINDOW                      # box windows must fit the grid
    # free positions may leave the grid (a valid call: out=None stops it before any launch)
    assert f(lib, kt=5, mode=1, ss=3, sh=135, sn=270, out=None) == ERR_NULL
    assert f(lib, kt=17, ky=17, kx=17, mode=1, ss=3, sh=3 * 4913, sn=6 * 4913) == ERR_WINDOW  # > 4096 samples
    assert f(lib, scale=float("nan")) == ERR_SCALE
    assert f(lib, ss=3) == ERR_LAYOUT                      # box mode takes one offset per (query, head)
    assert f(lib, sn=2) == ERR_LAYOUT                      # entries of 3 floats overlap
    assert f(lib, sh=1) == ERR_LAYOUT                      # heads overlap the tokens' entries
    assert f(lib, sh=-3) == ERR_LAYOUT
    # valid layouts get as far as the output check (out=None): [N][H][3] and [H][N][3]
    assert f(lib, sn=6, sh=3, out=None) == ERR_NULL
    assert f(lib, sn=3, sh=3 * 256, out=None) == ERR_NULL
    assert f(lib, q=P + 4) == ERR_ALIGN
    assert f(lib, off=P + 2) == ERR_ALIGN
    assert f(lib, out=None) == ERR_NULL
    free = dict(mode=1, sn=3 * 2 * 27, sh=3 * 27, ss=3)
    assert f(lib, **{**free, "sh": 3 * 26}) == ERR_LAYOUT  # samples of two heads overlap
    assert f(lib, **free, out=None) == ERR_NULL
    # workspace sizes: 0 for invalid geometry, the forward needs none
    ws = lib.dsa3d_sampled_workspace_bytes
    assert ws(4, 8, 8, 2, 3, 3, 3, 0, 0) == 256
    assert ws(4, 8, 8, 2, 3, 3, 3, 1, 1) > 4 * 8 * 8 * 2 * 27 * 36
    assert ws(4, 8, 8, 2, 2, 3, 3, 1, 1) == 0
    assert ws(4, 8, 8, 2, 3, 3, 3, 5, 1) == 0
    # box windows whose lattice of corner rows, (kt+1)(ky+1)(kx+1), fits the kernels' LDS
    # work per lattice point (~41 bytes each); past it (5 x 15 x 15: 1536 points) per
    # sample like free windows (~49 bytes a sample in box mode)
    NHL = 16 * 32 * 32 * 8 * 4 * 8 * 8
    assert 40 * NHL <= ws(16, 32, 32, 8, 3, 7, 7, 0, 1) <= 42 * NHL
    NHK = 6 * 16 * 17 * 225 * 5
    assert 48 * NHK <= ws(6, 16, 17, 1, 5, 15, 15, 0, 1) <= 50 * NHK


def test_sampled_backward_validation(lib):
    f = lib.dsa3d_sampled_backward
    base = [P, P, P, P, 3, 0, 0, 0, P, P, P, 4, 8, 8, 2, 64, 3, 3, 3, 0.125, 1, P, P, P, P, P]
    args = list(base)
    args[25] = None  # workspace
    assert f(*args, 1 << 40, None) == ERR_NULL
    assert f(*base, 100, None) == ERR_WORKSPACE
    args = list(base)
    args[24] = P + 2  # doffsets misaligned
    assert f(*args, 1 << 40, None) == ERR_ALIGN


def test_heads_validation(lib):
    f = lib.dsa3d_forward_heads
    ok = [P, P, P, P, 4, 8, 8, 2, 64, 3, 3, 3, 0.125, 1, P, P, P, 1 << 40, None]
    assert f(*ok, 4) == ERR_FLAGS
    bad = list(ok)
    bad[16] = None
    assert f(*bad, 0) == ERR_NULL
    bad = list(ok)
    bad[17] = 100
    assert f(*bad, 0) == ERR_WORKSPACE
    b = lib.dsa3d_backward_heads
    okb = [P] * 7 + [4, 8, 8, 2, 64, 3, 3, 3, 0.125, 0, P, P, P, P, 1 << 40, None]
    assert b(*okb, 4) == ERR_FLAGS
    assert f(*ok, 2) == ERR_FLAGS  # DSA3D_FLAG_REUSE_PREP is a backward flag
    bad = list(okb)
    bad[11] = 96  # head_dim
    assert b(*bad, 0) == ERR_HEAD_DIM


def test_dwconv_and_linear_validation(lib):
    fw = lib.dsa3d_dwconv3d_forward
    ok = [P, P, P, 4, 8, 8, 64, 3, 3, 3, 1, P, 0, None]
    assert fw(*[None] + ok[1:]) == ERR_NULL
    bad = list(ok); bad[6] = 12  # C not a multiple of 8
    assert fw(*bad) == ERR_GRID
    bad = list(ok); bad[7] = 2
    assert fw(*bad) == ERR_WINDOW
    bad = list(ok); bad[7], bad[8], bad[9] = 9, 9, 9  # 729 taps > 512
    assert fw(*bad) == ERR_WINDOW
    bad = list(ok); bad[10] = 2
    assert fw(*bad) == ERR_DTYPE
    bad = list(ok); bad[11] = P + 8
    assert fw(*bad) == ERR_ALIGN
    assert lib.dsa3d_dwconv3d_workspace_bytes(4, 8, 8, 64, 3, 3, 3) > 0
    assert lib.dsa3d_dwconv3d_workspace_bytes(4, 8, 8, 63, 3, 3, 3) == 0
    bw = lib.dsa3d_dwconv3d_backward
    okb = [P, P, P, 4, 8, 8, 64, 3, 3, 3, 1, P, P, P, P, 1 << 40, None]
    bad = list(okb); bad[15] = 10
    assert bw(*bad) == ERR_WORKSPACE
    lf = lib.dsa3d_linear_forward
    okl = [P, P, P, 100, 64, 81, 1, P, None]
    bad = list(okl); bad[3] = 0
    assert lf(*bad) == ERR_GRID
    bad = list(okl); bad[6] = 5
    assert lf(*bad) == ERR_DTYPE
    bad = list(okl); bad[1] = P + 4
    assert lf(*bad) == ERR_ALIGN
    assert lib.dsa3d_linear_workspace_bytes(100, 64, 81, 1) > 0
    assert lib.dsa3d_linear_workspace_bytes(1 << 20, 1 << 12, 81, 1) == 0  # M K >= 2^31
    lb = lib.dsa3d_linear_backward
    okb = [P, P, P, 100, 64, 81, 1, P, P, P, P, 1 << 40, None]
    bad = list(okb); bad[11] = 1
    assert lb(*bad) == ERR_WORKSPACE


def test_dwconv_and_linear_binding_checks_shapes(lib):
    """The binding checks the token count, channel count and dtypes of the convolution and
    linear calls before any pointer reaches the library: the C calls take sizes, not
    tensors, so a mismatch would otherwise be read or written as raw memory."""
    import torch

    E = dsa3d.DSA3DError
    grid = (4, 8, 8)
    x = torch.zeros(256, 64)
    w = torch.zeros(64, 3, 3, 3)
    with pytest.raises(E, match="tokens"):
        dsa3d.dwconv3d_backward(x, w, x, (4, 8, 9))
    with pytest.raises(E, match="weight must be"):
        dsa3d.dwconv3d_backward(x, w[:32], x, grid)
    with pytest.raises(E, match="weight must be"):
        dsa3d.dwconv3d_backward(x, w[:, 0], x, grid)
    with pytest.raises(E, match="weight has dtype"):
        dsa3d.dwconv3d_backward(x, w.double(), x, grid)
    with pytest.raises(E, match="x must be"):
        dsa3d.dwconv3d_backward(x[None], w, x, grid)
    with pytest.raises(E, match="dy has shape"):
        dsa3d.dwconv3d_backward(x, w, x[:100], grid)
    with pytest.raises(E, match="tokens"):
        dsa3d.dwconv3d_forward(x[:100], w, None, grid)
    with pytest.raises(E, match="x must be"):
        dsa3d.linear_backward(x[None], torch.zeros(81, 64), torch.zeros(256, 81))
    with pytest.raises(E, match="weight has shape"):
        dsa3d.linear_backward(x, torch.zeros(81, 32), torch.zeros(256, 81))
    with pytest.raises(E, match="dy has shape"):
        dsa3d.linear_backward(x, torch.zeros(81, 64), torch.zeros(256, 80))

