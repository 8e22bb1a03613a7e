"""Oracle for the H3 per-rank path: a plain, slow fp64 CPU definition.

TEST INFRASTRUCTURE ONLY.  Only the tests, the package's smoke check and the
benchmark's CPU-baseline leg may import or call this module.  The GPU path
never does, and this module imports nothing from it: the two share no code,
tables or constants.  Inputs come as plain host arrays.

What it computes (sources are the three pages the build follows):

* QK-RMSNorm: a head_dim-shaped RMSNorm applied to q and to k after the head
  split, one weight vector for q and one for k ("Tensor parallelism for
  MiniMax-H3", PR description, the paragraph on replicated norms and QK-norms).
  Reading: r = 1/sqrt(mean_d x_d^2 + eps), y = x * r * gamma.
* RoPE with real cos/sin tables that broadcast over the head axis (same page,
  PR description, "No RoPE change was needed"), the angle being position times
  inv_freq (same page, whn09's "Bug: non-persistent buffers" comment, where
  inv_freq is a non-persistent buffer).  Readings: inv_freq_j = theta^(-2j/D),
  j = 0..D/2-1, theta = 10000; pairs are adjacent (2j, 2j+1) and rotate by the
  2x2 matrix [[c, -s], [s, c]]; tables are computed in fp64 and stored fp32;
  RMSNorm and RoPE are one fused step with a single round to bf16.
* Exact full attention per head, no mask, no causality, over the whole packed
  sequence: out = softmax(scale * q k^T) v ("buqi-minimax-h3-multigpu",
  On accuracy and How it works; "Tensor parallelism for MiniMax-H3", whn09's
  Neuron FYI: packed full self-attention with no mask).  The oracle writes the
  plain definition; the GPU's tiled online softmax reaches the same value up to
  rounding.

* Partial attention over a key range with its log-sum-exp, and the merge of
  such partials.  The pages' next scaling axis past the 56-head Ulysses cap is
  context/ring parallelism over K/V blocks ("Tensor parallelism for
  MiniMax-H3", whn09's comments on the ceiling and on TP x CP meshes); its
  building block is exact: lse = log sum_j exp(scale * q.k_j) over the range,
  and parts combine as out = sum_p exp(lse_p - lse) out_p with
  lse = log sum_p exp(lse_p).

* The row-sliced qkv projection with the prologue behind it.  A rank that
  receives the whole modulated hidden state projects it through only its own
  heads' rows of qkv_proj; slicing rows is exact because the weight's scale is
  per-tensor ("buqi-minimax-h3-multigpu", How it works, the all_gather form
  used at world_size <= 4; H3 has hidden 5376 and inner 7168 = 56 x 128).
  Readings: no bias; within each of the q, k and v slices, row h*D + d is
  head h, dim d; the projection is exact (fp64) and q and k go straight into
  RMSNorm and RoPE with no rounding in between, then one round to bf16.
  The fp8 form (the checkpoint the page recommends stores fp8 weights with
  one scale per tensor): hidden state and weight rows are OCP e4m3 codes
  with one fp32 scale each, and the projection is
  x_scale * w_scale * sum_c x8[t, c] * w8[f, c], exact in fp64.  Reading:
  both operands are fp8 (the pages' transformer GEMMs run in fp8) and the
  scales multiply the exact dot product before the norm.

Every pin of these functions lives in tests/test_oracle.py.  One part is
parity unpinned: whether the adjacent-pair RoPE convention and the fp64 tables
match the real MiniMax-H3 checkpoint (no page states it; the GPU kernel takes
the tables as inputs, so a different convention changes data, not code).
"""
from __future__ import annotations

import numpy as np

# --------------------------------------------------------------------------
# bfloat16 codec (IEEE binary32 truncated to its top 16 bits)
# --------------------------------------------------------------------------


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """Decode bf16 bit patterns exactly: the pattern is the top half of a
    binary32, so shifting it up 16 bits gives that binary32 exactly."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def f64_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp64 values to the nearest bf16, ties to even, in one step.

    bf16 keeps 8 significant bits and binary32's exponent range.  Writing a
    nonzero finite x as m * 2^e with 0.5 <= |m| < 1 (frexp), the spacing of
    bf16 values around x is 2^(e-8) in the normal range and 2^-133 below
    2^-126 (subnormals).  x / spacing is exact in fp64 (a power-of-two
    scale), so rint() on it is the round-half-even of the definition, done
    once -- no double rounding through fp32.  Results at or past 2^128 are inf.
    """
    x = np.asarray(x, dtype=np.float64)
    m, e = np.frexp(x)
    spacing_exp = np.maximum(e.astype(np.int64) - 8, -133)
    q = np.rint(np.ldexp(x, -spacing_exp))          # exact scaling, then RNE
    y = np.ldexp(q, spacing_exp)                     # a bf16 value (or 2^128)
    with np.errstate(over="ignore"):
        y32 = y.astype(np.float32)                   # exact; 2^128 -> inf
    y32 = np.where(np.isnan(x), np.float32(np.nan), y32)
    bits = (y32.view(np.uint32) >> np.uint32(16)).astype(np.uint16)
    bits = np.where(np.isnan(x), np.uint16(0x7FC0), bits)
    return bits.astype(np.uint16)


# --------------------------------------------------------------------------
# Rotary tables
# --------------------------------------------------------------------------


def rope_tables(positions: np.ndarray, D: int = 128, theta: float = 10000.0):
    """cos and sin of position * inv_freq_j for j = 0..D/2-1, as fp32 [L, D/2].

    inv_freq_j = theta^(-2j/D); angles, cos and sin in fp64, one round to fp32.
    """
    pos = np.asarray(positions, dtype=np.float64)
    j = np.arange(D // 2, dtype=np.float64)
    inv_freq = np.power(float(theta), -2.0 * j / D)
    angle = pos[:, None] * inv_freq[None, :]
    return np.cos(angle).astype(np.float32), np.sin(angle).astype(np.float32)


# --------------------------------------------------------------------------
# QK-RMSNorm + RoPE
# --------------------------------------------------------------------------


def rms_norm(x: np.ndarray, gamma: np.ndarray, eps: float) -> np.ndarray:
    """y = x / sqrt(mean(x^2 over the last axis) + eps) * gamma, in fp64."""
    x = np.asarray(x, dtype=np.float64)
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return x / np.sqrt(ms + float(eps)) * np.asarray(gamma, dtype=np.float64)


def rope_rotate(y: np.ndarray, cos: np.ndarray, sin: np.ndarray) -> np.ndarray:
    """Rotate adjacent pairs (y[2j], y[2j+1]) by the angle whose cos/sin are
    cos[..., j], sin[..., j]; cos/sin broadcast against y's leading axes."""
    y = np.asarray(y, dtype=np.float64)
    c = np.asarray(cos, dtype=np.float64)
    s = np.asarray(sin, dtype=np.float64)
    even, odd = y[..., 0::2], y[..., 1::2]
    out = np.empty_like(y)
    out[..., 0::2] = even * c - odd * s
    out[..., 1::2] = even * s + odd * c
    return out


def qknorm_rope(x_bits: np.ndarray, gamma: np.ndarray, cos: np.ndarray,
                sin: np.ndarray, eps: float):
    """The prologue for one of q or k.

    x_bits: bf16 bits [H, L, D]; gamma fp32 [D]; cos, sin fp32 [L, D/2].
    Returns (y, y_bits): the exact fp64 result and its bf16 RNE bits [H, L, D].
    """
    x = bf16_to_f64(x_bits)
    y = rope_rotate(rms_norm(x, gamma, eps), cos[None], sin[None])
    return y, f64_to_bf16_bits(y)


# --------------------------------------------------------------------------
# Attention
# --------------------------------------------------------------------------


def attention_head(q: np.ndarray, k: np.ndarray, v: np.ndarray, scale: float,
                   block: int = 256) -> np.ndarray:
    """softmax(scale * q k^T) v for one head, in fp64.

    q [R, D] (the query rows to evaluate), k [L, D], v [L, D] as fp64 arrays.
    Each query row is independent, so rows are taken `block` at a time only to
    bound memory.  Uses PyTorch CPU fp64 matmul/exp as library primitives.
    """
    import torch
    kt = torch.from_numpy(np.ascontiguousarray(k, dtype=np.float64))
    vt = torch.from_numpy(np.ascontiguousarray(v, dtype=np.float64))
    qt = torch.from_numpy(np.ascontiguousarray(q, dtype=np.float64))
    out = torch.empty((qt.shape[0], vt.shape[1]), dtype=torch.float64)
    for r0 in range(0, qt.shape[0], block):
        s = float(scale) * (qt[r0:r0 + block] @ kt.T)
        m = s.max(dim=1, keepdim=True).values
        e = torch.exp(s - m)
        p = e / e.sum(dim=1, keepdim=True)
        out[r0:r0 + block] = p @ vt
    return out.numpy()


def attention(q_bits: np.ndarray, k_bits: np.ndarray, v_bits: np.ndarray,
              scale: float, rows=None) -> np.ndarray:
    """Per-head attention over bf16 inputs [H, L, D].

    rows: None for every query row, else a list with one index array per head.
    Returns an fp64 array [H, R, D] (R = L, or the length of each head's rows,
    which must then be equal across heads).
    """
    H = q_bits.shape[0]
    outs = []
    for h in range(H):
        r = np.arange(q_bits.shape[1]) if rows is None else np.asarray(rows[h])
        q = bf16_to_f64(q_bits[h, r])
        k = bf16_to_f64(k_bits[h])
        v = bf16_to_f64(v_bits[h])
        outs.append(attention_head(q, k, v, scale))
    return np.stack(outs)


# --------------------------------------------------------------------------
# Partial attention with log-sum-exp, and the merge of partials
# --------------------------------------------------------------------------


def attention_lse_head(q: np.ndarray, k: np.ndarray, v: np.ndarray, scale: float, block: int = 256):
    """(out, lse) for one head over the given keys, in fp64.

    out = softmax(scale * q k^T) v as in attention_head; lse[r] is the natural
    log of sum_j exp(scale * <q_r, k_j>), computed as m + log(sum exp(s - m)).
    """
    import torch
    kt = torch.from_numpy(np.ascontiguousarray(k, dtype=np.float64))
    vt = torch.from_numpy(np.ascontiguousarray(v, dtype=np.float64))
    qt = torch.from_numpy(np.ascontiguousarray(q, dtype=np.float64))
    out = torch.empty((qt.shape[0], vt.shape[1]), dtype=torch.float64)
    lse = torch.empty(qt.shape[0], dtype=torch.float64)
    for r0 in range(0, qt.shape[0], block):
        s = float(scale) * (qt[r0:r0 + block] @ kt.T)
        m = s.max(dim=1, keepdim=True).values
        e = torch.exp(s - m)
        z = e.sum(dim=1, keepdim=True)
        out[r0:r0 + block] = (e / z) @ vt
        lse[r0:r0 + block] = (m + torch.log(z))[:, 0]
    return out.numpy(), lse.numpy()


def merge_partials(outs: np.ndarray, lses: np.ndarray):
    """Combine P partial results over disjoint key ranges.

    outs [P, ..., D], lses [P, ...]: lse = log sum_p exp(lse_p) (max-shifted),
    out = sum_p exp(lse_p - lse) * out_p.  Returns (out, lse) in fp64.
    """
    outs = np.asarray(outs, dtype=np.float64)
    lses = np.asarray(lses, dtype=np.float64)
    m = lses.max(axis=0)
    w = np.exp(lses - m[None])
    z = w.sum(axis=0)
    lse = m + np.log(z)
    out = (w[..., None] * outs).sum(axis=0) / z[..., None]
    return out, lse


# --------------------------------------------------------------------------
# Row-sliced qkv projection followed by the prologue
# --------------------------------------------------------------------------


def qkv_project(x_bits: np.ndarray, w_bits: np.ndarray) -> np.ndarray:
    """y[t, f] = sum_c x[t, c] * w[f, c] in fp64.

    x_bits: bf16 bits [L, C] (tokens x hidden); w_bits: bf16 bits [N, C] (the
    output features' weight rows, nn.Linear layout).  Returns fp64 [L, N].
    """
    return bf16_to_f64(x_bits) @ bf16_to_f64(w_bits).T


def split_heads(y: np.ndarray, H: int, D: int = 128) -> np.ndarray:
    """[L, H*D] -> [H, L, D]: feature h*D + d is head h, dim d."""
    L = y.shape[0]
    return np.ascontiguousarray(y.reshape(L, H, D).transpose(1, 0, 2))


def qkv_proj_qknorm_rope(x_bits, wq_bits, wk_bits, wv_bits, gamma_q, gamma_k, cos, sin,
                         eps: float, H: int, D: int = 128) -> dict:
    """q, k and v of H heads from the hidden state.

    x_bits [L, C]; wq/wk/wv bits [H*D, C]; gamma fp32 [D]; cos, sin fp32
    [L, D/2].  q = RoPE(RMSNorm(x Wq^T)), k likewise with gamma_k, v = x Wv^T,
    each split into heads and rounded once to bf16.  Returns
    {"q": (fp64 [H, L, D], bits), "k": ..., "v": ...}.
    """
    out = {}
    for name, w, gamma in (("q", wq_bits, gamma_q), ("k", wk_bits, gamma_k), ("v", wv_bits, None)):
        y = split_heads(qkv_project(x_bits, w), H, D)
        if gamma is not None:
            y = rope_rotate(rms_norm(y, gamma, eps), cos[None], sin[None])
        out[name] = (y, f64_to_bf16_bits(y))
    return out


# --------------------------------------------------------------------------
# fp8 (OCP e4m3: 1 sign, 4 exponent bits with bias 7, 3 mantissa bits; no
# infinities; exponent and mantissa all ones is NaN)
# --------------------------------------------------------------------------


def e4m3_to_f64(bits: np.ndarray) -> np.ndarray:
    """Decode e4m3 codes exactly: normal (1 + m/8) 2^(e-7) for e >= 1,
    subnormal (m/8) 2^-6 for e = 0, NaN for the two all-ones codes."""
    b = np.asarray(bits, dtype=np.uint8).astype(np.int64)
    sign = np.where(b & 0x80, -1.0, 1.0)
    e = (b >> 3) & 0xF
    m = (b & 0x7).astype(np.float64)
    mag = np.where(e == 0, m / 8.0 * 2.0 ** -6, (1.0 + m / 8.0) * np.exp2(e.astype(np.float64) - 7.0))
    out = sign * mag
    return np.where((e == 15) & ((b & 7) == 7), np.nan, out)


def qkv_proj_fp8_qknorm_rope(x8, x_scale, wq8, wk8, wv8, w_scale, gamma_q, gamma_k, cos, sin,
                             eps: float, H: int, D: int = 128) -> dict:
    """The fp8 form of qkv_proj_qknorm_rope: x8 e4m3 codes [L, C] with scale
    x_scale, weight rows e4m3 [H*D, C] with the per-tensor scale w_scale;
    y = x_scale * w_scale * (x8 w8^T) exactly, then the same head split,
    RMSNorm + RoPE for q and k, and one round to bf16."""
    xf = e4m3_to_f64(x8)
    out = {}
    for name, w, gamma in (("q", wq8, gamma_q), ("k", wk8, gamma_k), ("v", wv8, None)):
        y = float(x_scale) * float(w_scale) * (xf @ e4m3_to_f64(w).T)
        y = split_heads(y, H, D)
        if gamma is not None:
            y = rope_rotate(rms_norm(y, gamma, eps), cos[None], sin[None])
        out[name] = (y, f64_to_bf16_bits(y))
    return out
