"""Seeded synthetic workloads for routed block-sparse attention.

This module only draws random numbers and rounds them to bf16; it holds none
of the attention method's arithmetic.  Both the HIP path (via the Python
binding) and the CPU oracle consume what it produces, so it is the one piece
of code the two sides share.

Tensors are returned as ``numpy.uint16`` arrays holding bf16 bit patterns in
the BTHD layout ``[B, N, H, D]`` (D contiguous), the layout the MiniMax-H3
attention calls use (aikraft.ru "ComfyUI Sol-Attn" news, section
"Производительность на RTX 5090": BTHD, H=56; thakicloud "MiniMax-H3 ComfyUI
accel stack", kernel table: B=1, H=56, D=128, bf16).

Workload recipes (random-number draw order is part of the recipe):

* ``iid``: Q, K, V independent N(0, 1) in that order, float32 then bf16 RNE.
* ``clustered``: per head h and dimension d a smooth random signal
  ``s_hd(t) = (1/sqrt 2) * sum_{j<4} sin(2 pi t / P_hdj + phi_hdj)`` with the
  periods P log-uniform in [256, 4096] tokens and phi ~ U[0, 2 pi), so that s
  has unit variance.  Draws: periods [H, D, 4], phases [H, D, 4], then the
  noise of Q, then V.  ``Q = K = bf16(1.5 s + N(0,1))`` (one tensor) and
  ``V = bf16(N(0,1))``.  Neighbouring 64-row blocks have similar means, so
  the per-block routing picks a content-dependent sparse set.
* ``h3``: a packed joint sequence.  The first ``prefix_len`` rows stand for
  the text/audio conditioning rows that H3 packs ahead of the video rows
  (keys-SM121 MiniMax-H3 README; Star7 README, section "Sol"); they are i.i.d.
  N(0, 1) for Q, K and V (three draws, in that order).  The remaining rows lie
  row-major on a frames x 24 x 42 latent grid (1344 x 768 at 32x spatial
  compression, thakicloud post, sequence-length table); the signal is
  ``s_hd(f,y,x) = (1/sqrt 2) sum_j sin(2 pi (f/Pf + y/Py + x/Px)_hdj + phi_hdj)``
  with every period log-uniform in [2, 32] (draw order Pf, Py, Px, phi), then
  the Q noise, then V.  Q = K = bf16(1.5 s + N(0,1)), V = bf16(N(0,1)).
* ``clustered_soft`` and ``h3_joint(..., amp=0.5, shared_qk=False)``: test
  inputs with the same signals, a weaker amplitude and independent key noise
  (drawn after the query noise), so that no key copies its query and the
  centroid terms carry much of each row's softmax mass.
"""

from __future__ import annotations

import dataclasses
import math
from typing import Optional

import numpy as np

__all__ = [
    "Workload",
    "CONFIGS",
    "make_workload",
    "iid",
    "clustered",
    "clustered_soft",
    "h3_joint",
    "f32_to_bf16_bits",
    "bf16_bits_to_f32",
    "to_torch_bf16",
]

_GRID_H = 24  # 768 / 32 latent rows per frame
_GRID_W = 42  # 1344 / 32 latent columns per frame


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (round to nearest, ties to even).

    Returns the 16-bit patterns as ``uint16``.  Inputs are finite here.
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    bias = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((u + bias) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns to float32 (exact)."""
    bits = np.ascontiguousarray(bits, dtype=np.uint16)
    return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32)


def to_torch_bf16(bits: np.ndarray, device="cpu"):
    """Wrap bf16 bit patterns as a ``torch.bfloat16`` tensor (no rounding)."""
    import torch

    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16)
    return t.to(device) if str(device) != "cpu" else t


@dataclasses.dataclass
class Workload:
    """One seeded problem: bf16 bit arrays plus the routing parameters."""

    name: str
    q: np.ndarray  # uint16 [B, N, H, D]
    k: np.ndarray
    v: np.ndarray
    tau: Optional[float] = 1.0
    topk_ratio: Optional[float] = None
    prefix_len: int = 0
    centroid: bool = True
    logmass: bool = True

    @property
    def shape(self):
        return self.q.shape

    def params(self) -> dict:
        return dict(
            tau=self.tau,
            topk_ratio=self.topk_ratio,
            prefix_len=self.prefix_len,
            centroid=self.centroid,
            logmass=self.logmass,
        )


def _bf16(x) -> np.ndarray:
    """float32 (numpy or torch) -> bf16 bit patterns, round to nearest even.

    torch's float32 -> bfloat16 cast rounds to nearest even (checked against
    ``f32_to_bf16_bits`` in the tests) and runs on all host threads."""
    import torch

    t = x if isinstance(x, torch.Tensor) else torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def iid(B: int, N: int, H: int, D: int, seed: int):
    """Q, K, V i.i.d. N(0,1), drawn in that order, rounded to bf16."""
    rng = np.random.Generator(np.random.PCG64(seed))
    out = []
    for _ in range(3):
        out.append(_bf16(rng.standard_normal((B, N, H, D), dtype=np.float32)))
    return tuple(out)


def _sum_of_sines(ang_fn, rows, H, D, chunk=1024):
    """(1/sqrt 2) * sum_j sin(angle[t, h, d, j]) for t < rows, float32 [rows, H, D].

    The elementwise math runs in torch (float64, all host threads); the
    random draws stay with numpy's PCG64 generator."""
    import torch

    s = np.empty((rows, H, D), dtype=np.float32)
    for t0 in range(0, rows, chunk):
        t1 = min(rows, t0 + chunk)
        ang = ang_fn(torch.arange(t0, t1, dtype=torch.int64))
        s[t0:t1] = (torch.sin(ang).sum(dim=-1) / math.sqrt(2.0)).to(torch.float32).numpy()
    return s


def _smooth_1d(rng, B, N, H, D):
    import torch

    periods = np.exp(rng.uniform(math.log(256.0), math.log(4096.0), size=(H, D, 4)))
    phases = torch.from_numpy(rng.uniform(0.0, 2.0 * math.pi, size=(H, D, 4)))
    omega = torch.from_numpy(2.0 * math.pi / periods)  # [H, D, 4]

    def ang(t):
        return t.to(torch.float64)[:, None, None, None] * omega[None] + phases[None]

    return _sum_of_sines(ang, N, H, D)


def _signal_plus_noise(rng, s, B, amp=1.5):
    """bf16(amp s + N(0,1)) with s [rows, H, D] shared by every batch entry."""
    import torch

    rows, H, D = s.shape
    noise = torch.from_numpy(rng.standard_normal((B, rows, H, D), dtype=np.float32))
    return _bf16(noise.add_(torch.from_numpy(s)[None], alpha=amp))


def clustered(B: int, N: int, H: int, D: int, seed: int):
    """Q = K = 1.5 s(t) + N(0,1), V = N(0,1); s is a smooth per-head signal."""
    rng = np.random.Generator(np.random.PCG64(seed))
    s = _smooth_1d(rng, B, N, H, D)
    q = _signal_plus_noise(rng, s, B)
    v = _bf16(rng.standard_normal((B, N, H, D), dtype=np.float32))
    return q, q, v


def clustered_soft(B: int, N: int, H: int, D: int, seed: int, amp: float = 0.5):
    """The clustered signal with independent query and key noise and a
    weaker signal: Q = bf16(amp s + N(0,1)), K = bf16(amp s + N'(0,1)),
    V = bf16(N(0,1)).  Draws: periods, phases, Q noise, K noise, V.  Routing
    still follows the smooth signal, but no key copies its query, so each
    row's softmax mass spreads over many blocks and the unselected blocks'
    centroid terms carry a large share of it (test inputs for the centroid
    path; the benchmarked workloads use ``clustered``)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    s = _smooth_1d(rng, B, N, H, D)
    q = _signal_plus_noise(rng, s, B, amp)
    k = _signal_plus_noise(rng, s, B, amp)
    v = _bf16(rng.standard_normal((B, N, H, D), dtype=np.float32))
    return q, k, v


def h3_joint(B: int, N: int, H: int, D: int, prefix_len: int, seed: int, amp: float = 1.5,
             shared_qk: bool = True):
    """Packed joint sequence: an i.i.d. prefix, then a frames x 24 x 42 video
    grid.  With ``shared_qk=False`` the video keys get their own noise
    (drawn after the query noise) instead of equalling the queries."""
    rng = np.random.Generator(np.random.PCG64(seed))
    P = prefix_len
    pre = [rng.standard_normal((B, P, H, D), dtype=np.float32) for _ in range(3)]
    nvid = N - P
    per = [np.exp(rng.uniform(math.log(2.0), math.log(32.0), size=(H, D, 4))) for _ in range(3)]
    phases = rng.uniform(0.0, 2.0 * math.pi, size=(H, D, 4))
    import torch

    inv = [torch.from_numpy(1.0 / p) for p in per]
    ph = torch.from_numpy(phases)
    frame = _GRID_H * _GRID_W

    def ang(t):
        f = (t // frame).to(torch.float64)[:, None, None, None]
        y = ((t % frame) // _GRID_W).to(torch.float64)[:, None, None, None]
        x = (t % _GRID_W).to(torch.float64)[:, None, None, None]
        return 2.0 * math.pi * (f * inv[0][None] + y * inv[1][None] + x * inv[2][None]) + ph[None]

    s = _sum_of_sines(ang, nvid, H, D)
    qk_vid = _signal_plus_noise(rng, s, B, amp)
    k_vid = qk_vid if shared_qk else _signal_plus_noise(rng, s, B, amp)
    v_vid = _bf16(rng.standard_normal((B, nvid, H, D), dtype=np.float32))
    q = np.concatenate([_bf16(pre[0]), qk_vid], axis=1)
    k = np.concatenate([_bf16(pre[1]), k_vid], axis=1)
    v = np.concatenate([_bf16(pre[2]), v_vid], axis=1)
    return q, k, v


# The five named problems.  Sizes and routing follow the workload table this
# package is measured on: a tiny i.i.d. case, three clustered video-like
# cases at N = 4096 / 16384 / 32768 with H = 56 and D = 128, and one packed
# H3-shaped joint sequence of 38,247 rows with a 1024-row prefix.
CONFIGS = {
    "tiny": dict(kind="iid", B=1, H=2, N=1024, D=64, seed=0, tau=1.0),
    "n4k": dict(kind="clustered", B=1, H=56, N=4096, D=128, seed=1, tau=1.0),
    "n16k": dict(kind="clustered", B=1, H=56, N=16384, D=128, seed=2, tau=1.0),
    "n32k": dict(kind="clustered", B=1, H=56, N=32768, D=128, seed=3, tau=1.0),
    "h3": dict(kind="h3", B=1, H=56, N=38247, D=128, seed=4, prefix_len=1024, topk_ratio=0.1),
}


def make_workload(name: str, **overrides) -> Workload:
    """Build one of the named problems; ``overrides`` replace recipe fields
    (e.g. ``H=4`` for a head subset or ``tau=float('-inf')`` for the dense path)."""
    cfg = dict(CONFIGS[name])
    cfg.update(overrides)
    kind = cfg["kind"]
    B, H, N, D, seed = cfg["B"], cfg["H"], cfg["N"], cfg["D"], cfg["seed"]
    if kind == "iid":
        q, k, v = iid(B, N, H, D, seed)
    elif kind == "clustered":
        q, k, v = clustered(B, N, H, D, seed)
    elif kind == "h3":
        q, k, v = h3_joint(B, N, H, D, cfg["prefix_len"], seed)
    else:
        raise ValueError(f"unknown workload kind {kind!r}")
    return Workload(
        name=name,
        q=q,
        k=k,
        v=v,
        tau=cfg.get("tau") if cfg.get("topk_ratio") is None else None,
        topk_ratio=cfg.get("topk_ratio"),
        prefix_len=cfg.get("prefix_len", 0),
        centroid=cfg.get("centroid", True),
        logmass=cfg.get("logmass", True),
    )
