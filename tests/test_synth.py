"""The seeded input generator: deterministic, thread-count independent, right shapes and
distributions for every workload recipe (CPU only)."""
import os
import subprocess
import sys

import numpy as np
import pytest
import torch

from local_sparse_attention_amd import configs, synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_values_do_not_depend_on_thread_count(tmp_path):
    a = synth.normal(7, 2, (4096, 3), "f32")
    code = ("import sys; sys.path.insert(0, %r); import numpy as np; from local_sparse_attention_amd import synth;"
            "np.save(sys.argv[1], synth.normal(7, 2, (4096, 3), 'f32'))" % ROOT)
    path = str(tmp_path / "synth_1thread.npy")
    subprocess.run([sys.executable, "-c", code, path], check=True, env={**os.environ, "OMP_NUM_THREADS": "1"})
    assert np.array_equal(np.load(path), a)


def test_normal_distribution_and_streams():
    from scipy import stats

    a = synth.normal(3, 0, (200000,), "f32").astype(np.float64)
    assert abs(a.mean()) < 0.01 and abs(a.std() - 1) < 0.01
    assert stats.kstest(a, "norm").pvalue > 1e-3
    b = synth.normal(3, 1, (200000,), "f32")
    c = synth.normal(4, 0, (200000,), "f32")
    assert abs(np.corrcoef(a, b)[0, 1]) < 0.01 and abs(np.corrcoef(a, c)[0, 1]) < 0.01
    # counter based: a window of words starting at `first` equals the same slice
    assert np.array_equal(synth.normal(3, 0, (1000,), "f32", first=500), a[500:1500].astype(np.float32))


def test_bf16_is_round_to_nearest_even_of_the_fp32_value():
    f = synth.normal(5, 1, (100000,), "f32", scale=0.125)
    b = synth.normal(5, 1, (100000,), "bf16", scale=0.125)
    ref = torch.as_tensor(f).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(b, ref)


def test_offset_recipes():
    off = synth.make_offsets(configs.C1)
    assert set(np.unique(off)) == {-2, -1, 0, 1, 2}
    off = synth.make_offsets(configs.C2)
    assert off.min() == -4 and off.max() == 4 and abs(off.std() - 2) < 0.1
    wl = configs.C3
    off = synth.make_offsets(wl).reshape(wl.F, wl.Hp, wl.Wp, 3)
    # block value + jitter in {-1, 0, 1}: inside an 8x8 block a component spans at most 2
    for by in range(0, wl.Hp, 8):
        for bx in range(0, wl.Wp, 8):
            blk = off[:, by:by + 8, bx:bx + 8]
            assert (blk.max((0, 1, 2)) - blk.min((0, 1, 2)) <= 2).all()
    assert off.std() > 2  # the block values move
    wl5 = configs.C5.with_frames(40)
    off5 = synth.make_offsets(wl5).reshape(wl5.F, wl5.Hp, wl5.Wp, 3)
    assert np.abs(off5).max() <= 9
    # drift: the same block moves between frames
    assert (off5[0, :8, :8] != off5[39, :8, :8]).any()


def test_first_frames_match_the_full_grid():
    wl = configs.C5.with_frames(6)
    sub = configs.C5.with_frames(2)
    a, b = synth.make_inputs(wl), synth.make_inputs(sub)
    for key in ("q", "k", "v", "dout", "offsets"):
        assert np.array_equal(a[key][: sub.N], b[key]), key


@pytest.mark.parametrize("name", list(configs.ALL))
def test_workload_sizes(name):
    wl = configs.ALL[name]
    assert wl.kt % 2 == 1 and wl.ky % 2 == 1 and wl.kx % 2 == 1
    assert wl.kt <= wl.F and wl.ky <= wl.Hp and wl.kx <= wl.Wp
    if name == "C5":
        assert wl.N == 2088960 and wl.K == 405
        assert abs(wl.flops() - 24.26e12) < 0.01e12
        assert abs(wl.bytes() - 102.99e9) < 0.01e9
