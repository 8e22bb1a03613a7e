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
    fp64 pow and sincos may each be off by an ulp.  inv_freq = theta^(-2j/D)
    may then differ by 2^-52 relative, and the angle pos * inv_freq by
    2^-51 relative after its own rounding on each side; at the largest
    position checked (126975 < 2^17, inv_freq <= 1) that is under 2^-34
    absolute, and sincos adds 2^-52.  Rounding both fp64 values to fp32 can
    then add one fp32 spacing.  Bound: spacing_fp32(ref) + 2^-33 (a factor
    two over the analysis)."""
    spacing = np.spacing(np.abs(ref).astype(np.float32)).astype(np.float64)
    diff = np.abs(got.astype(np.float64) - ref.astype(np.float64))
    return diff <= spacing + 2.0 ** -33


def _tables_vs_oracle(gpu_lib, pos, theta, label):
    import torch
    c, s = gpu_lib.rope_tables(to_dev(pos, torch.int32), 128, theta)
    c_ref, s_ref = oracle.rope_tables(pos, 128, theta)
    c, s = c.cpu().numpy(), s.cpu().numpy()
    for got, ref in ((c, c_ref), (s, s_ref)):
        worst = float(np.abs(got.astype(np.float64) - ref.astype(np.float64)).max())
        print(f"{label}: max |gpu - oracle| {worst:.3e} (2^{np.log2(max(worst, 2.0 ** -80)):.1f})")
        assert np.all(_table_close(got, ref))
        assert np.mean(got != ref) < 1e-2
    print(f"{label}: tables identical in {np.mean(c == c_ref) * 100:.4f}% / {np.mean(s == s_ref) * 100:.4f}%")


@pytest.mark.parametrize("name", ["tiny", "ws8", "canvas128k"])
def test_rope_tables_match_oracle(gpu_lib, name):
    w = I.WORKLOADS[name]
    _tables_vs_oracle(gpu_lib, I.packed_positions(w.n_video, w.n_audio), I.ROPE_THETA, name)


@pytest.mark.parametrize("theta", [500.0, 1e6])
def test_rope_tables_nondefault_theta(gpu_lib, theta):
    """theta reaches the kernel as a run-time argument: two bases other than
    10000 on the ws8 positions."""
    w = I.WORKLOADS["ws8"]
    _tables_vs_oracle(gpu_lib, I.packed_positions(w.n_video, w.n_audio), theta, f"theta={theta:g}")


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
        # Rows whose exact value is zero have no relative error; the element
        # check above covers them.
        nz = np.linalg.norm(y.reshape(-1, 128), axis=-1) > 0
        rel = row_rel_err(got.reshape(-1, 128)[nz], y.reshape(-1, 128)[nz])
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


@pytest.mark.parametrize("eps,rms", [(1e-3, 0.03), (1e-9, 3e-5)])
def test_prologue_nondefault_eps(gpu_lib, eps, rms):
    """eps reaches the kernel as a run-time argument: inputs drawn with an RMS
    near sqrt(eps) (their mean square about eps), so that eps moves every
    output by tens of per cent and a kernel that used another eps fails."""
    w = I.custom_workload(H=3, L=1000, n_audio=200)
    x = dict(I.make_inputs(w, seed=17))
    for n in ("q", "k"):
        x[n] = I.f32_to_bf16_bits((rms * oracle.bf16_to_f64(x[n])).astype(np.float32))
    x["eps"] = eps
    _prologue_check(gpu_lib, x, f"eps={eps:g}")


@pytest.mark.parametrize("L", [1, 5, 17, 300, 32768 + 45])
def test_prologue_ragged_lengths(gpu_lib, L):
    """Lengths that end inside a 16-token workgroup, and (32768 + 45) one
    that ends 45 tokens into a second 32768-token chunk."""
    w = I.custom_workload(H=3, L=L, n_audio=L // 3)
    _prologue_check(gpu_lib, I.make_inputs(w, seed=L), f"L={L}")


def test_prologue_one_norm_per_token(gpu_lib):
    """All 16 lanes of a token must normalise by the same r.  With gamma = 1,
    cos = 1 and sin = 0 an output element is RNE(fl(x * r)), so when one lane
    holds exactly twice another lane's values (a power of two commutes with
    both roundings) its outputs must be exactly twice the other's.  Elements
    32..63 (lanes 4-7) are set to 2x elements 0..31 (lanes 0-3), and 96..127
    to 2x 64..95: partners in different quads of the 16-lane row, where a
    reduction that summed in a different order per quad would give r values
    one fp32 ulp apart on some tokens.  A build with such a reduction (quad
    sums combined by row rotations) failed this check on 17 elements of q
    and 24 of k; the butterfly passes with none."""
    import torch
    H, L = 7, 32768
    g = torch.Generator(device="cuda:0").manual_seed(5)
    xs = []
    for _ in range(2):
        x = torch.randn((H, L, 128), generator=g, device="cuda:0").to(torch.bfloat16)
        x[:, :, 32:64] = x[:, :, 0:32] * 2
        x[:, :, 96:128] = x[:, :, 64:96] * 2
        xs.append(x)
    q, k = xs
    ones = torch.ones(128, dtype=torch.float32, device="cuda:0")
    cos = torch.ones((L, 64), dtype=torch.float32, device="cuda:0")
    sin = torch.zeros((L, 64), dtype=torch.float32, device="cuda:0")
    gpu_lib.qknorm_rope(q, k, ones, ones, cos, sin, 1e-6)
    torch.cuda.synchronize()
    for name, t in (("q", q), ("k", k)):
        f = t.float()
        bad = int((f[:, :, 32:64] != 2 * f[:, :, 0:32]).sum()) + int((f[:, :, 96:128] != 2 * f[:, :, 64:96]).sum())
        print(f"{name}: {bad} elements not exactly twice their partner")
        assert bad == 0


def test_prologue_zero_tokens(gpu_lib):
    """Tokens whose q or k row is all zero: r = 1/sqrt(eps) multiplies
    zeros, so the row stays exactly zero (+0 or -0: the rotation's products
    with a negative cos or sin carry the sign); the other tokens are
    unaffected (checked against the oracle as usual)."""
    import torch
    w = I.custom_workload(H=3, L=1000, n_audio=200)
    x = dict(I.make_inputs(w, seed=23))
    for n in ("q", "k"):
        a = x[n].copy()
        a[:, ::7] = 0
        x[n] = a
    _prologue_check(gpu_lib, x, "zero tokens")
    d = device_inputs(x)
    cos, sin = gpu_lib.rope_tables(d["positions"], 128, x["theta"])
    gpu_lib.qknorm_rope(d["q"], d["k"], d["gamma_q"], d["gamma_k"], cos, sin, x["eps"])
    torch.cuda.synchronize()
    assert np.all(bits(d["q"])[:, ::7] & 0x7FFF == 0) and np.all(bits(d["k"])[:, ::7] & 0x7FFF == 0)
