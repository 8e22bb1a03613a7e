"""Seeded synthetic inputs for the H3 per-rank attention path.

This module holds no arithmetic of the method itself.  It only draws random
numbers, rounds those draws to bfloat16 bit patterns (through PyTorch's own
fp32 -> bf16 conversion, round-to-nearest-even), lays out the packed
video+audio position list, and picks the query rows a sampled check looks at.
The oracle-side tests and the GPU-side harness both take their inputs from
here, so the two paths see the same bits.

Workloads (one Ulysses rank's share of MiniMax-H3's 56 heads, head_dim 128,
over the whole packed sequence; "buqi-minimax-h3-multigpu", How it works;
"Tensor parallelism for MiniMax-H3", whn09's Neuron FYI on the packed, unmasked
self-attention):

  tiny         H=2,  L=512,    positions 0..511
  ws8          H=7,  L=32768,  31744 video tokens (0..31743) + 1024 audio (0..1023)
  ws2          H=28, L=32768,  same layout
  ws1          H=56, L=32768,  same layout
  canvas128k   H=7,  L=131072, 126976 video + 4096 audio; q and k drawn x3
  odd37726     H=7,  L=37726,  a real-length sequence that is not a multiple of
               any tile (the 768p canvas with a short prompt, whn09's Neuron
               FYI); split read as 32256 video (32 latent frames of 42x24
               patches) + 5470 audio

Draw order from numpy.random.Generator(PCG64(seed)): q, k, v (standard normal,
fp32, times the workload's qk_scale for q and k), then gamma_q and gamma_k
(1 + 0.1 * standard normal, fp32).

Projection workloads (the rank's row-sliced qkv_proj over the gathered hidden
state, H3's hidden size 5376; "buqi-minimax-h3-multigpu", How it works):

  proj_tiny    H=2,  L=300,   hidden=512   (256 video + 44 audio)
  proj_ws8     H=7,  L=32768, hidden=5376  (31744 video + 1024 audio)
  proj_ws2     H=28, L=32768, hidden=5376  (the all_gather form's world_size 2)

  proj8_ws8    the fp8 form of proj_ws8;   proj8_ws2  the fp8 form of proj_ws2

Draw order from Generator(PCG64(seed)): x (standard normal), then wq, wk, wv
(standard normal / sqrt(hidden), so each projected feature is about N(0,1)),
each rounded to bf16; then gamma_q and gamma_k (1 + 0.1 * standard normal).
The fp8 forms draw the same fp32 values and quantise them instead: x with
x_scale = max|x| / 448, the three weight slices with one w_scale = max over
all three / 448 (one scale per tensor), each value / scale rounded to e4m3 by
PyTorch's float8_e4m3fn conversion (data preparation, not the method).
"""
from __future__ import annotations

import math
from dataclasses import dataclass

import numpy as np

HEAD_DIM = 128
ROPE_THETA = 10000.0
RMS_EPS = 1e-6


@dataclass(frozen=True)
class Workload:
    name: str
    H: int
    L: int
    n_video: int
    n_audio: int
    qk_scale: float = 1.0
    D: int = HEAD_DIM

    @property
    def attn_scale(self) -> float:
        return 1.0 / math.sqrt(self.D)

    @property
    def flops(self) -> float:
        """Attention work counted as 4*H*L^2*D (two L x L x D contractions)."""
        return 4.0 * self.H * float(self.L) ** 2 * self.D


WORKLOADS = {
    "tiny": Workload("tiny", H=2, L=512, n_video=512, n_audio=0),
    "ws8": Workload("ws8", H=7, L=32768, n_video=31744, n_audio=1024),
    "ws2": Workload("ws2", H=28, L=32768, n_video=31744, n_audio=1024),
    "ws1": Workload("ws1", H=56, L=32768, n_video=31744, n_audio=1024),
    "canvas128k": Workload("canvas128k", H=7, L=131072, n_video=126976,
                           n_audio=4096, qk_scale=3.0),
    "odd37726": Workload("odd37726", H=7, L=37726, n_video=32256, n_audio=5470),
}


@dataclass(frozen=True)
class ProjWorkload:
    name: str
    H: int
    L: int
    n_video: int
    n_audio: int
    hidden: int
    fp8: bool = False
    D: int = HEAD_DIM

    @property
    def flops(self) -> float:
        """2 * L * (3 H D) * hidden: one multiply-add per token, feature and
        hidden element."""
        return 2.0 * self.L * 3 * self.H * self.D * self.hidden


PROJ_WORKLOADS = {
    "proj_tiny": ProjWorkload("proj_tiny", H=2, L=300, n_video=256, n_audio=44, hidden=512),
    "proj_ws8": ProjWorkload("proj_ws8", H=7, L=32768, n_video=31744, n_audio=1024, hidden=5376),
    "proj_ws2": ProjWorkload("proj_ws2", H=28, L=32768, n_video=31744, n_audio=1024, hidden=5376),
    "proj8_ws8": ProjWorkload("proj8_ws8", H=7, L=32768, n_video=31744, n_audio=1024, hidden=5376, fp8=True),
    "proj8_ws2": ProjWorkload("proj8_ws2", H=28, L=32768, n_video=31744, n_audio=1024, hidden=5376, fp8=True),
}


def _to_e4m3_bits(x: np.ndarray, scale: float) -> np.ndarray:
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x / np.float32(scale), dtype=np.float32))
    return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def make_proj_inputs(w: ProjWorkload, seed: int = 0) -> dict:
    """Hidden state, weight slices, gammas and positions of a projection
    workload.  x: uint16 bf16 bits [L, hidden]; wq, wk, wv: bits [H*D, hidden]
    (fp8 forms: uint8 e4m3 codes, plus fp32 x_scale and w_scale);
    gamma_q, gamma_k fp32 [D]; positions int32 [L]; eps and theta."""
    rng = np.random.Generator(np.random.PCG64(seed))
    xf = rng.standard_normal((w.L, w.hidden), dtype=np.float32)
    wscale = np.float32(1.0 / math.sqrt(w.hidden))
    wf = {n: rng.standard_normal((w.H * w.D, w.hidden), dtype=np.float32) * wscale for n in ("wq", "wk", "wv")}
    out = {}
    if w.fp8:
        out["x_scale"] = np.float32(np.abs(xf).max() / 448.0)
        out["w_scale"] = np.float32(max(float(np.abs(a).max()) for a in wf.values()) / 448.0)
        out["x"] = _to_e4m3_bits(xf, out["x_scale"])
        for name, a in wf.items():
            out[name] = _to_e4m3_bits(a, out["w_scale"])
    else:
        out["x"] = f32_to_bf16_bits(xf)
        for name, a in wf.items():
            out[name] = f32_to_bf16_bits(a)
    del xf, wf
    out["gamma_q"] = (1.0 + 0.1 * rng.standard_normal(w.D, dtype=np.float32)).astype(np.float32)
    out["gamma_k"] = (1.0 + 0.1 * rng.standard_normal(w.D, dtype=np.float32)).astype(np.float32)
    out["positions"] = packed_positions(w.n_video, w.n_audio)
    out["eps"] = RMS_EPS
    out["theta"] = ROPE_THETA
    return out


def custom_workload(H: int, L: int, n_audio: int = 0, qk_scale: float = 1.0,
                    D: int = HEAD_DIM) -> Workload:
    """A workload of any shape; the last n_audio tokens restart at position 0."""
    if not (0 <= n_audio <= L):
        raise ValueError("n_audio must lie in [0, L]")
    return Workload(f"H{H}_L{L}", H=H, L=L, n_video=L - n_audio,
                    n_audio=n_audio, qk_scale=qk_scale, D=D)


def packed_positions(n_video: int, n_audio: int) -> np.ndarray:
    """Rotary position of every packed token: video 0..n_video-1, then audio
    restarting at 0 (int32, length n_video + n_audio)."""
    return np.concatenate([np.arange(n_video, dtype=np.int32),
                           np.arange(n_audio, dtype=np.int32)])


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp32 draws to bf16 (PyTorch's RNE conversion); returns uint16 bits."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def make_inputs(w: Workload, seed: int = 0) -> dict:
    """All inputs of one workload, as host arrays.

    q, k, v: uint16 bf16 bit patterns [H, L, D]; gamma_q, gamma_k: fp32 [D];
    positions: int32 [L]; plus eps, attention scale and rotary theta.
    """
    rng = np.random.Generator(np.random.PCG64(seed))
    shape = (w.H, w.L, w.D)
    out = {}
    for name, mult in (("q", w.qk_scale), ("k", w.qk_scale), ("v", 1.0)):
        x = rng.standard_normal(shape, dtype=np.float32)
        if mult != 1.0:
            x *= np.float32(mult)
        out[name] = f32_to_bf16_bits(x)
        del x
    out["gamma_q"] = (1.0 + 0.1 * rng.standard_normal(w.D, dtype=np.float32)).astype(np.float32)
    out["gamma_k"] = (1.0 + 0.1 * rng.standard_normal(w.D, dtype=np.float32)).astype(np.float32)
    out["positions"] = packed_positions(w.n_video, w.n_audio)
    out["eps"] = RMS_EPS
    out["scale"] = w.attn_scale
    out["theta"] = ROPE_THETA
    return out


def sample_rows(w, head: int, n: int = 4096, seed: int = 0) -> np.ndarray:
    """Sorted query rows a sampled check compares for one head.

    n distinct rows drawn by Generator(PCG64(seed + 1000 + head)), always
    including the segment boundaries 0, n_video-1, n_video and L-1.  Returns all
    rows when n >= L.
    """
    if n >= w.L:
        return np.arange(w.L, dtype=np.int64)
    rng = np.random.Generator(np.random.PCG64(seed + 1000 + head))
    rows = set(rng.choice(w.L, size=n, replace=False).tolist())
    for b in (0, w.n_video - 1, w.n_video, w.L - 1):
        if 0 <= b < w.L:
            rows.add(b)
    return np.array(sorted(rows), dtype=np.int64)
