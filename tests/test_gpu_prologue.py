"""GPU parity of the rotary tables and the QK-RMSNorm + RoPE prologue against
the oracle, element by element over every row."""
import numpy as np
import pytest

import oracle
from exact_head_attention_amd import inputs as I
from tests.gpu_helpers import bf16_ulp_distance, bits, device_inputs, host_inputs, row_rel_err, to_dev

pytestmark = pytest.mark.gpu


def _table_close(got, ref):
    """Both sides build the tables in fp64 and round once to fp32, but their
    fp64 pow and cos may differ in the last bit.  At angles up to 1.3e5 rad
    (position 126975) a last-bit difference is about 2^-35 absolute in the
    angle, so an entry may differ by that much absolutely, or by one fp32 ulp
    from the final rounding."""
    spacing = np.spacing(np.abs(ref).astype(np.float32)).astype(np.float64)
    diff = np.abs(got.astype(np.float64) - ref.astype(np.float64))
    return diff <= np.maximum(spacing, 2.0 ** -30)


@pytest.mark.parametrize("name", ["tiny", "ws8", "canvas128k"])
def test_rope_tables_match_oracle(gpu_lib, name):
    import torch
    w = I.WORKLOADS[name]
    pos = I.packed_positions(w.n_video, w.n_audio)
    c, s = gpu_lib.rope_tables(to_dev(pos, torch.int32), 128, I.ROPE_THETA)
    c_ref, s_ref = oracle.rope_tables(pos, 128, I.ROPE_THETA)
    c, s = c.cpu().numpy(), s.cpu().numpy()
    for got, ref in ((c, c_ref), (s, s_ref)):
        assert np.all(_table_close(got, ref))
        assert np.mean(got != ref) < 1e-2
    print(f"{name}: tables identical in {np.mean(c == c_ref) * 100:.4f}% / {np.mean(s == s_ref) * 100:.4f}%")


def _prologue_check(gpu_lib, x, label):
    """Every element against the exact fp64 value y of the oracle.

    The GPU computes in fp32 and rounds once to bf16 (the ABI's definition), so
    an element may differ from y by one bf16 spacing (rounding of a slightly
    different fp32 value) plus the fp32 arithmetic error.  That error scales
    with the terms being combined, not with the result: where the rotation
    cancels (y2j*c - y2j+1*s << its terms) it can exceed one spacing of the
    small result.  A few fp32 roundings of terms bounded by the row's largest
    |y| give the 2^-18 * max_row|y| slack."""
    import torch
    d = device_inputs(x)
    cos, sin = gpu_lib.rope_tables(d["positions"], 128, x["theta"])
    gpu_lib.qknorm_rope(d["q"], d["k"], d["gamma_q"], d["gamma_k"], cos, sin, x["eps"])
    torch.cuda.synchronize()
    c_ref, s_ref = oracle.rope_tables(x["positions"], 128, x["theta"])
    for nm, gname in (("q", "gamma_q"), ("k", "gamma_k")):
        got = bits(d[nm])
        y, yb = oracle.qknorm_rope(x[nm], x[gname], c_ref, s_ref, x["eps"])
        g64 = oracle.bf16_to_f64(got)
        mag = np.abs(y)
        spacing = np.exp2(np.maximum(np.floor(np.log2(np.where(mag > 0, mag, 1.0))) - 7, -133))
        slack = spacing + 2.0 ** -18 * mag.max(axis=-1, keepdims=True)
        err = np.abs(g64 - y)
        ulps = bf16_ulp_distance(got, yb)
        frac = float(np.mean(got != yb))
        rel = row_rel_err(got.reshape(-1, 128), y.reshape(-1, 128))
        print(f"{label} {nm}: max ulp vs RNE(ref) {ulps.max():.0f} (elements > 1 ulp: {int((ulps > 1).sum())}), "
              f"mismatching {frac:.2e}, max err/slack {float((err / slack).max()):.3f}, max row rel {rel.max():.2e}")
        assert np.all(err <= slack)
        assert frac < 2e-3
        assert rel.max() <= 4e-3


@pytest.mark.parametrize("name", ["tiny", "ws8", "odd37726"])
def test_prologue_parity(gpu_lib, name):
    _prologue_check(gpu_lib, host_inputs(name), name)


def test_prologue_parity_canvas_x3(gpu_lib):
    """q and k drawn x3: RMSNorm removes the scale, the rows must still match."""
    _prologue_check(gpu_lib, host_inputs("canvas128k"), "canvas128k")


@pytest.mark.parametrize("L", [1, 5, 17, 300, 32768 + 45])
def test_prologue_ragged_lengths(gpu_lib, L):
    """Lengths that end inside a 16-token workgroup, and (32768 + 45) one
    that ends 45 tokens into a second 32768-token chunk."""
    w = I.custom_workload(H=3, L=L, n_audio=L // 3)
    _prologue_check(gpu_lib, I.make_inputs(w, seed=L), f"L={L}")
