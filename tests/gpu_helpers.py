"""Shared plumbing of the GPU tests: upload seeded inputs, read bf16 back, and
the comparison metrics of the parity checks."""
import functools

import numpy as np

from exact_head_attention_amd import inputs as I

# Parity bars for attention, both gated:
#   per query row:  ||gpu - ref||_2 / ||ref||_2 <= 4e-3 (the stated tolerance);
#   per element:    |gpu - ref| <= spacing_bf16(ref) + ATTN_ELEM_C * max_row|ref|.
# The element bar: the output's final RNE can move an element by up to half a
# bf16 spacing of a nearby fp32 value (one spacing covers it); before that the
# only lossy step is rounding each attention weight to bf16.  Those roundings
# are independent, with relative standard deviation at most 2^-8/sqrt(3)
# (~2.3e-3; ~1.6e-3 for weights spread over their binade), so they move an
# element by a zero-mean sum whose standard deviation is about 1.6e-3 of the
# row's RMS.  The largest of ~3e7 checked elements (56 heads x 4096 rows x 128)
# sits near 6 standard deviations, about 1e-2 of the RMS, and max_row|ref| is
# 2.2-3.3 times the RMS of a 128-element row, so 2^-7 * max_row|ref| (2-3e-2 of
# the RMS) leaves about a factor two.  The fp32 accumulation (2^-24 per add)
# and the exp2 approximation (~2^-23 relative) are three orders smaller.
ATTN_TOL = 4e-3
ATTN_ELEM_C = 2.0 ** -7


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


def bf16_spacing(x):
    """Spacing of the bf16 grid at |x| (elementwise, fp64)."""
    mag = np.abs(x)
    return np.exp2(np.maximum(np.floor(np.log2(np.where(mag > 0, mag, 1.0))) - 7, -133))


def attention_errors(got, ref, rounded=True):
    """Error metrics of GPU attention rows got (fp64 values, [..., 128]) against
    oracle rows ref.  rounded: got was rounded to bf16 (the spacing term of the
    element bar applies); False for the fp32 partial outputs.

    Returns a dict: row (max per-row 2-norm relative error, gated), elem (max
    element error over its bar, gated <= 1), inf (max over rows of
    max|d| / max|ref|), fro (whole-tensor Frobenius relative error), p999 (the
    99.9th percentile of |d| / max_row|ref|)."""
    got = np.asarray(got, dtype=np.float64).reshape(-1, 128)
    ref = np.asarray(ref, dtype=np.float64).reshape(-1, 128)
    d = np.abs(got - ref)
    rmax = np.abs(ref).max(axis=-1, keepdims=True)
    bar = ATTN_ELEM_C * rmax + (bf16_spacing(ref) if rounded else 0.0)
    return {
        "row": float((np.linalg.norm(got - ref, axis=-1) / np.linalg.norm(ref, axis=-1)).max()),
        "elem": float((d / bar).max()),
        "inf": float((d.max(axis=-1, keepdims=True) / rmax).max()),
        "fro": float(np.linalg.norm(got - ref) / np.linalg.norm(ref)),
        "p999": float(np.quantile(d / rmax, 0.999)),
        "n": int(ref.shape[0]),
    }


def merge_errors(parts):
    """Combine attention_errors dicts of disjoint row sets (fro weighted by rows)."""
    out = {k: max(p[k] for p in parts) for k in ("row", "elem", "inf", "p999")}
    n = sum(p["n"] for p in parts)
    out["fro"] = float(np.sqrt(sum(p["fro"] ** 2 * p["n"] for p in parts) / n))
    out["n"] = n
    return out


def check_attention_errors(label, m):
    """Print and record the metrics, then gate the row and element bars."""
    import json
    import os
    print(f"{label}: max row rel {m['row']:.3e}, max elem err/bar {m['elem']:.3f}, inf-norm rel {m['inf']:.3e}, "
          f"frobenius rel {m['fro']:.3e}, p99.9 elem/max_row {m['p999']:.3e} ({m['n']} rows)", flush=True)
    path = os.environ.get("H3_PARITY_LOG")
    if path:
        with open(path, "a") as f:
            f.write(json.dumps({"case": label, **m}) + "\n")
    assert m["row"] <= ATTN_TOL, f"{label}: row error {m['row']:.3e} over {ATTN_TOL}"
    assert m["elem"] <= 1.0, f"{label}: element error {m['elem']:.3f} of its bar"
