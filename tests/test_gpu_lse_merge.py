"""GPU parity of h3_attention_lse and h3_attention_merge against the oracle.

Partial outputs are fp32 (the only rounding is the bf16 of the attention
weights, as in h3_attention), so they share the 4e-3 per-row bar.  The
log-sum-exp is compared absolutely: it is ln(l) + m with l a sum of bf16
weights, so its error is about the relative error of that sum (<< 1e-3).
"""
import math

import numpy as np
import pytest

import oracle
from exact_head_attention_amd import inputs as I
from tests.gpu_helpers import attention_errors, bits, check_attention_errors, host_inputs, merge_errors, to_dev

pytestmark = pytest.mark.gpu
LSE_TOL = 2e-3


def _raw(H, L, seed, mult=1.0):
    import torch
    rng = np.random.Generator(np.random.PCG64(seed))
    return [to_dev(I.f32_to_bf16_bits(mult * rng.standard_normal((H, L, 128), dtype=np.float32)), torch.bfloat16)
            for _ in range(3)]


def _lse_vs_oracle(gpu_lib, q, k, v, s, label):
    """h3_attention_lse on device tensors: out (fp32, no output rounding) on
    the row and element bars, lse absolutely, every row."""
    import torch
    out, lse = gpu_lib.attention_lse(q, k, v, scale=s)
    torch.cuda.synchronize()
    qb, kb, vb = bits(q), bits(k), bits(v)
    parts, lerr = [], 0.0
    for h in range(qb.shape[0]):
        ref, ref_lse = oracle.attention_lse_head(oracle.bf16_to_f64(qb[h]), oracle.bf16_to_f64(kb[h]),
                                                 oracle.bf16_to_f64(vb[h]), s)
        parts.append(attention_errors(out[h].double().cpu().numpy(), ref, rounded=False))
        lerr = max(lerr, float(np.abs(lse[h].double().cpu().numpy() - ref_lse).max()))
    print(f"{label}: max |dlse| {lerr:.2e}")
    check_attention_errors(label, merge_errors(parts))
    assert lerr <= LSE_TOL


@pytest.mark.parametrize("Lq,j0,j1", [(300, 0, 300), (257, 100, 1000), (64, 999, 1000), (1000, 0, 1)])
def test_attention_lse_range_vs_oracle(gpu_lib, Lq, j0, j1):
    """Queries against a key range given as a pointer offset into a larger
    tensor; out (fp32) and lse against the oracle on every row."""
    q, _, _ = _raw(2, Lq, seed=31 + Lq)
    _, kf, vf = _raw(2, 1000, seed=32)
    _lse_vs_oracle(gpu_lib, q, kf[:, j0:j1], vf[:, j0:j1], 1 / math.sqrt(128), f"Lq={Lq} keys [{j0},{j1})")


@pytest.mark.parametrize("scale", [0.03, 0.3])
@pytest.mark.parametrize("H,L", [(10, 4900), (3, 1000)])
def test_attention_lse_nondefault_scale(gpu_lib, scale, H, L):
    """The partial form at two scales other than 1/sqrt(128), through the
    main launch (200 units) and the tail launch (12 units); lse carries the
    scale directly (ln sum exp(scale q.k))."""
    q, k, v = _raw(H, L, seed=800 + L)
    _lse_vs_oracle(gpu_lib, q, k, v, scale, f"lse scale={scale} H={H} L={L}")


@pytest.mark.parametrize("cuts", [[0, 500, 1000], [0, 1, 333, 334, 1000], [0, 64, 128, 1000],
                                  [0, 100, 200, 300, 400, 700, 1000]])
def test_split_merge_equals_full(gpu_lib, cuts):
    """Keys split into uneven ranges, partials merged on the GPU: the bf16
    output and merged lse match the oracle's unsplit attention.  2, 3 and 4
    parts take the merge's unrolled forms, 6 parts its run-time loop."""
    import torch
    q, k, v = _raw(3, 1000, seed=40, mult=2.0)
    s = 1 / math.sqrt(128)
    parts = [gpu_lib.attention_lse(q, k[:, a:b], v[:, a:b], scale=s) for a, b in zip(cuts, cuts[1:])]
    outs = torch.stack([p[0] for p in parts])
    lses = torch.stack([p[1] for p in parts])
    out, lse = gpu_lib.attention_merge(outs, lses, want_lse=True)
    torch.cuda.synchronize()
    qb, kb, vb, ob = bits(q), bits(k), bits(v), bits(out)
    parts = []
    for h in range(3):
        ref, ref_lse = oracle.attention_lse_head(oracle.bf16_to_f64(qb[h]), oracle.bf16_to_f64(kb[h]),
                                                 oracle.bf16_to_f64(vb[h]), s)
        parts.append(attention_errors(oracle.bf16_to_f64(ob[h]), ref))
        assert np.abs(lse[h].double().cpu().numpy() - ref_lse).max() <= LSE_TOL
    check_attention_errors(f"cuts {cuts} merged", merge_errors(parts))


@pytest.mark.parametrize("Lq", [4900, 4000])
def test_attention_lse_tail_workgroups_bit_identical(gpu_lib, Lq):
    """The partial form through both kernels: ten heads in one launch (200 or
    160 units: all in the main launch) against one launch per head (20 units:
    128-row tail workgroups; 16 units: 64-row tail workgroups), over a key
    range given as a pointer offset.  out and lse bit-identical per head."""
    import torch
    q, k, v = _raw(10, Lq, seed=44)
    a, b = 100, 4037
    out_all, lse_all = gpu_lib.attention_lse(q, k[:, a:b], v[:, a:b])
    for h in range(10):
        out_h, lse_h = gpu_lib.attention_lse(q[h:h + 1], k[h:h + 1, a:b], v[h:h + 1, a:b])
        torch.cuda.synchronize()
        assert torch.equal(out_all[h], out_h[0]), f"head {h}: out differs between the launches"
        assert torch.equal(lse_all[h], lse_h[0]), f"head {h}: lse differs between the launches"
    assert bool(torch.isfinite(out_all).all()) and bool(torch.isfinite(lse_all).all())


def test_merge_single_part_is_rounding_of_it(gpu_lib):
    """Special case: merging one part returns its bf16 rounding (RNE) exactly."""
    import torch
    q, k, v = _raw(2, 700, seed=41)
    o32, l32 = gpu_lib.attention_lse(q, k, v)
    out = gpu_lib.attention_merge(o32[None], l32[None])
    torch.cuda.synchronize()
    assert torch.equal(out, o32.to(torch.bfloat16))


def test_ws8_two_halves_sampled(gpu_lib):
    """One rank's workload with its keys split in two halves and merged; 4096
    sampled rows per head against the oracle."""
    import torch
    x = host_inputs("ws8")
    w = I.WORKLOADS["ws8"]
    q, k, v = (to_dev(x[n], torch.bfloat16) for n in ("q", "k", "v"))
    half = w.L // 2 + 77
    parts = [gpu_lib.attention_lse(q, k[:, a:b], v[:, a:b], scale=x["scale"]) for a, b in ((0, half), (half, w.L))]
    out = gpu_lib.attention_merge(torch.stack([p[0] for p in parts]), torch.stack([p[1] for p in parts]))
    torch.cuda.synchronize()
    qb, kb, vb, ob = bits(q), bits(k), bits(v), bits(out)
    parts = []
    for h in range(w.H):
        rows = I.sample_rows(w, h, 4096)
        ref = oracle.attention_head(oracle.bf16_to_f64(qb[h, rows]), oracle.bf16_to_f64(kb[h]),
                                    oracle.bf16_to_f64(vb[h]), x["scale"])
        parts.append(attention_errors(oracle.bf16_to_f64(ob[h, rows]), ref))
    check_attention_errors("ws8 split in two and merged", merge_errors(parts))


def test_attention_lse_head_splits_bit_identical(gpu_lib):
    """Per-head determinism of the partial kernel: 4 heads at once vs 2 x 2."""
    import torch
    q, k, v = _raw(4, 900, seed=42)
    o_all, l_all = gpu_lib.attention_lse(q, k[:, 100:800], v[:, 100:800])
    for h0 in (0, 2):
        o, l = gpu_lib.attention_lse(q[h0:h0 + 2], k[h0:h0 + 2, 100:800], v[h0:h0 + 2, 100:800])
        torch.cuda.synchronize()
        assert torch.equal(o, o_all[h0:h0 + 2]) and torch.equal(l, l_all[h0:h0 + 2])
