"""3D Deformable Slide Attention (3D-DSA) on AMD MI355X (gfx950).

The compute path is the C-ABI library ``libdsa3d.so`` (HIP kernels, declared in
``include/dsa3d.h``); :mod:`local_sparse_attention_amd.dsa3d` is its thin Python binding.
"""
