"""Workload table for 3D Deformable Slide Attention (3D-DSA).

Each workload is a synthetic video-token grid F x Hp x Wp (token n = (t*Hp + y)*Wp + x,
the T x H' x W' reshape of the paper's method section), a head count and head size,
a window kt x ky x kx (the neighbourhood of the method section; the paper trains with
3 x 7 x 7) and a recipe for the per-query integer motion offsets (dt, dy, dx).

The five rows are the tiny fp32 parity case, the bf16 forward case, the 720p-like case,
one DiT layer's full width (d = 8192) and the pages' video length (N ~ 2.09M tokens,
the 256-frame sequence of the paper's memory section, a 16-head slice).
"""
from dataclasses import dataclass, replace


@dataclass(frozen=True)
class Workload:
    name: str
    F: int
    Hp: int
    Wp: int
    heads: int
    head_dim: int
    kt: int
    ky: int
    kx: int
    dtype: str  # "f32" or "bf16"
    backward: bool
    seed: int
    qkv_scale: float  # Q/K/V are N(0,1) * qkv_scale
    offsets: tuple  # recipe, see synth.make_offsets

    @property
    def N(self) -> int:
        return self.F * self.Hp * self.Wp

    @property
    def K(self) -> int:
        return self.kt * self.ky * self.kx

    @property
    def scale(self) -> float:
        return self.head_dim ** -0.5

    @property
    def elem_bytes(self) -> int:
        return 4 if self.dtype == "f32" else 2

    def with_frames(self, F: int) -> "Workload":
        """Same workload on the first F frames (same generator words for those frames)."""
        return replace(self, F=F, name=f"{self.name}[F={F}]")

    # Algorithmic work per (query token, head): forward 4*K*D flops (QK^T and PV),
    # backward 10*K*D (S recompute, dP, dV, dQ, dK).
    def flops(self, fwd=True, bwd=True) -> float:
        per = (4 if fwd else 0) + (10 if bwd else 0)
        return float(per) * self.K * self.head_dim * self.N * self.heads

    # Algorithmic HBM bytes: forward reads Q, K, V and writes O (4 rows) plus LSE;
    # backward reads Q, K, V, O, dO and LSE and writes dQ, dK, dV (8 rows); each pass
    # also reads the int32 offsets (12 bytes per token).
    def bytes(self, fwd=True, bwd=True) -> float:
        s, D, NH = self.elem_bytes, self.head_dim, self.N * self.heads
        b = 0.0
        if fwd:
            b += (4 * D * s + 4) * NH + 12 * self.N
        if bwd:
            b += (8 * D * s + 4) * NH + 12 * self.N
        return b


C1 = Workload("C1-tiny-f32", 4, 8, 8, 2, 64, 3, 3, 3, "f32", True, 0, 1.0, ("uniform", -2, 2))
C2 = Workload("C2-bf16-fwd", 16, 32, 32, 8, 64, 3, 7, 7, "bf16", False, 1, 0.125, ("round_normal", 2.0, 4))
C3 = Workload("C3-720p", 32, 45, 80, 16, 128, 3, 9, 9, "bf16", True, 2, 1.0, ("blocks", 8, 3.0, False, 0.0))
C4 = Workload("C4-full-width", 64, 68, 120, 64, 128, 3, 9, 9, "bf16", True, 3, 1.0, ("blocks", 8, 3.0, False, 0.0))
C5 = Workload("C5-256f", 256, 68, 120, 16, 128, 5, 9, 9, "bf16", True, 4, 1.0, ("blocks", 8, 3.0, True, 8.0))

ALL = {"C1": C1, "C2": C2, "C3": C3, "C4": C4, "C5": C5}

# Sampled windows (real offsets, trilinear sampling): the pages' 3 x 7 x 7 window on a
# 16-frame 32 x 32 grid, 8 heads x 128, bf16, a drifting block motion field plus real
# jitter (synth.make_real_offsets): one offset per query (box windows) or one per
# sample (free positions).
S_BOX = Workload("S-box-real-offsets", 16, 32, 32, 8, 128, 3, 7, 7, "bf16", True, 5, 1.0,
                 ("blocks", 8, 3.0, True, 8.0))
S_FREE = Workload("S-free-per-sample-offsets", 16, 32, 32, 8, 128, 3, 7, 7, "bf16", True, 6, 1.0,
                  ("blocks", 8, 3.0, True, 8.0))
