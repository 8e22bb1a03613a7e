"""Shared plumbing of the GPU tests: upload seeded inputs, read bf16 back, and
the comparison metrics of the parity checks."""
import functools

import numpy as np

from exact_head_attention_amd import inputs as I

# Parity bar for attention: per query row, ||gpu - ref||_2 / ||ref||_2 <= 4e-3.
ATTN_TOL = 4e-3


def to_dev(a, dtype):
    import torch
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(a).view(dtype).to("cuda:0")


def bits(t):
    import torch
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


@functools.lru_cache(maxsize=2)
def host_inputs(name: str, seed: int = 0):
    return I.make_inputs(I.WORKLOADS[name], seed)


def device_inputs(x):
    import torch
    return dict(q=to_dev(x["q"], torch.bfloat16), k=to_dev(x["k"], torch.bfloat16),
                v=to_dev(x["v"], torch.bfloat16), gamma_q=to_dev(x["gamma_q"], torch.float32),
                gamma_k=to_dev(x["gamma_k"], torch.float32), positions=to_dev(x["positions"], torch.int32))


def row_rel_err(got_bits_rows, ref_rows):
    """Per-row 2-norm relative error of bf16 GPU rows against fp64 oracle rows."""
    import oracle
    got = oracle.bf16_to_f64(got_bits_rows)
    return np.linalg.norm(got - ref_rows, axis=-1) / np.linalg.norm(ref_rows, axis=-1)


def bf16_ulp_distance(a_bits, b_bits):
    """|a - b| in units of the bf16 spacing at max(|a|, |b|) (elementwise)."""
    import oracle
    a, b = oracle.bf16_to_f64(a_bits), oracle.bf16_to_f64(b_bits)
    mag = np.maximum(np.abs(a), np.abs(b))
    e = np.floor(np.log2(np.where(mag > 0, mag, 1.0)))
    spacing = np.exp2(np.maximum(e - 7, -133))
    return np.abs(a - b) / spacing
