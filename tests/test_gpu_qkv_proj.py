"""GPU parity of h3_qkv_proj_qknorm_rope (row-sliced qkv projection with
QK-RMSNorm + RoPE fused behind it) against the oracle, through the C ABI.

Bar, per element z of q, k and v against the exact fp64 value:
    |gpu - z| <= spacing_bf16(z) + 2^-16 * max_row |z|
The spacing term is the final round to bf16 of a slightly different fp32
value.  The second term covers the fp32 work before it: the accumulation of
hidden/16 matrix-core block sums (a random walk of ~2^-24-relative roundings,
~1e-6 of |z| at hidden = 5376), and for q and k the norm and rotation, whose
fp32 roundings scale with the row's largest term (as for h3_qknorm_rope).
2^-16 leaves 10x room over those and stays 500x under one bf16 spacing at the
row's largest element, so a wrong weight row, token, head or pairing fails.
Elements that differ from RNE(z) at all must be rarer than 1e-3 (near-ties).
"""
import math

import numpy as np
import pytest

import oracle
from exact_head_attention_amd import inputs as I
from tests.gpu_helpers import ATTN_TOL, bits, row_rel_err, to_dev

pytestmark = pytest.mark.gpu


def _upload(x):
    import torch
    d = {n: to_dev(x[n], torch.bfloat16) for n in ("x", "wq", "wk", "wv")}
    d.update(gamma_q=to_dev(x["gamma_q"], torch.float32), gamma_k=to_dev(x["gamma_k"], torch.float32),
             positions=to_dev(x["positions"], torch.int32))
    return d


def _check(label, got_bits, ref, ref_bits):
    mag = np.abs(ref)
    spacing = np.exp2(np.maximum(np.floor(np.log2(np.where(mag > 0, mag, 1.0))) - 7, -133))
    slack = spacing + 2.0 ** -16 * mag.max(axis=-1, keepdims=True)
    err = np.abs(oracle.bf16_to_f64(got_bits) - ref)
    ratio = float((err / slack).max())
    mism = float(np.mean(got_bits != ref_bits))
    rel = float(row_rel_err(got_bits.reshape(-1, 128), ref.reshape(-1, 128)).max())
    print(f"{label}: max err/bound {ratio:.3f}, mismatch vs RNE(exact) {mism:.2e}, max row rel {rel:.2e}")
    assert ratio <= 1.0
    assert mism < 1e-3
    assert rel <= ATTN_TOL


def _run(gpu_lib, x, H, rows=None, label=""):
    """Project on the GPU; compare all heads of q, k, v on the given tokens
    (all tokens if rows is None) with the oracle."""
    import torch
    d = _upload(x)
    cos, sin = gpu_lib.rope_tables(d["positions"], 128, x["theta"])
    q, k, v = gpu_lib.qkv_proj_qknorm_rope(d["x"], d["wq"], d["wk"], d["wv"], d["gamma_q"], d["gamma_k"],
                                           cos, sin, x["eps"])
    torch.cuda.synchronize()
    c_ref, s_ref = oracle.rope_tables(x["positions"], 128, x["theta"])
    xs = x["x"] if rows is None else x["x"][rows]
    cr, sr = (c_ref, s_ref) if rows is None else (c_ref[rows], s_ref[rows])
    ref = oracle.qkv_proj_qknorm_rope(xs, x["wq"], x["wk"], x["wv"], x["gamma_q"], x["gamma_k"], cr, sr,
                                      x["eps"], H)
    for name, t in (("q", q), ("k", k), ("v", v)):
        got = bits(t)
        if rows is not None:
            got = got[:, rows]
        _check(f"{label} {name}", got, *ref[name])
    return q, k, v


def _custom(H, L, hidden, n_audio, seed):
    w = I.ProjWorkload(f"H{H}_L{L}_C{hidden}", H=H, L=L, n_video=L - n_audio, n_audio=n_audio, hidden=hidden)
    return w, I.make_proj_inputs(w, seed)


def test_qkv_proj_tiny_all_elements(gpu_lib):
    w = I.PROJ_WORKLOADS["proj_tiny"]
    _run(gpu_lib, I.make_proj_inputs(w, 0), w.H, label="proj_tiny")


@pytest.mark.parametrize("H,L,hidden", [(1, 1, 32), (1, 7, 64), (3, 257, 96), (2, 513, 160)])
def test_qkv_proj_ragged_shapes_all_elements(gpu_lib, H, L, hidden):
    """One token, a single hidden step, token counts one past a tile, hidden
    sizes that are odd multiples of the 32-element step."""
    w, x = _custom(H, L, hidden, n_audio=L // 3, seed=100 + L)
    _run(gpu_lib, x, H, label=f"H={H} L={L} hidden={hidden}")


def test_qkv_proj_ws8_sampled(gpu_lib):
    """H = 7, L = 32768, hidden 5376: 1024 sampled tokens (segment boundaries
    included), every head and feature of q, k and v."""
    w = I.PROJ_WORKLOADS["proj_ws8"]
    x = I.make_proj_inputs(w, 0)
    _run(gpu_lib, x, w.H, rows=I.sample_rows(w, 0, 1024), label="proj_ws8")


@pytest.mark.timeout(600)
def test_qkv_proj_ws2_sampled(gpu_lib):
    """H = 28 (the all_gather form at world_size 2), 512 sampled tokens."""
    w = I.PROJ_WORKLOADS["proj_ws2"]
    x = I.make_proj_inputs(w, 0)
    _run(gpu_lib, x, w.H, rows=I.sample_rows(w, 0, 512), label="proj_ws2")


def test_qkv_proj_head_slices_bit_identical(gpu_lib):
    """Four heads in one launch against two launches of two heads each, fed
    row slices of the same weights (pointer offsets): every head of q, k and
    v bit-identical."""
    import torch
    w, x = _custom(4, 1000, 512, n_audio=100, seed=7)
    d = _upload(x)
    cos, sin = gpu_lib.rope_tables(d["positions"], 128, x["theta"])
    args = (d["gamma_q"], d["gamma_k"], cos, sin, x["eps"])
    full = gpu_lib.qkv_proj_qknorm_rope(d["x"], d["wq"], d["wk"], d["wv"], *args)
    parts = [gpu_lib.qkv_proj_qknorm_rope(d["x"], d["wq"][r:r + 256], d["wk"][r:r + 256], d["wv"][r:r + 256],
                                          *args) for r in (0, 256)]
    torch.cuda.synchronize()
    for i in range(3):
        assert torch.equal(full[i][:2], parts[0][i]) and torch.equal(full[i][2:], parts[1][i])


def test_qkv_proj_then_attention_chain(gpu_lib):
    """Projection (with the fused prologue) then attention on the GPU, against
    the all-oracle chain: per-row relative error within the attention bar."""
    import torch
    w = I.PROJ_WORKLOADS["proj_tiny"]
    x = I.make_proj_inputs(w, 1)
    d = _upload(x)
    cos, sin = gpu_lib.rope_tables(d["positions"], 128, x["theta"])
    q, k, v = gpu_lib.qkv_proj_qknorm_rope(d["x"], d["wq"], d["wk"], d["wv"], d["gamma_q"], d["gamma_k"],
                                           cos, sin, x["eps"])
    out = gpu_lib.attention(q, k, v, scale=1 / math.sqrt(128))
    torch.cuda.synchronize()
    c_ref, s_ref = oracle.rope_tables(x["positions"], 128, x["theta"])
    ref = oracle.qkv_proj_qknorm_rope(x["x"], x["wq"], x["wk"], x["wv"], x["gamma_q"], x["gamma_k"], c_ref,
                                      s_ref, x["eps"], w.H)
    o_ref = oracle.attention(ref["q"][1], ref["k"][1], ref["v"][1], 1 / math.sqrt(128))
    err = row_rel_err(bits(out).reshape(-1, 128), o_ref.reshape(-1, 128))
    print(f"projection -> attention chain: max row rel err {err.max():.3e}")
    assert err.max() <= ATTN_TOL


# ------------------------------------------------------------- fp8 form
#
# The fp8 matrix instruction does not sum its 64 products exactly in fp32.
# Measured on MI355X with in-bounds probes of one instruction: the products
# are summed in groups of 8 (8 consecutive bytes of one lane's operand), each
# product truncated toward zero on a grid 13 bits below the group's largest
# product (2^-13 of it is kept, 2^-14 is lost), and group sums then add in
# fp32.  A group of 8 therefore loses less than 7 * 2^-13 of its largest
# product, so for the pre-norm value y = s * sum_c x_c w_c:
#     |y_gpu - y| <= s * (7 * 2^-13 + 2^-20) * sum_c |x_c w_c| = dy
# (the 2^-20 covers the fp32 adds).  For q and k the norm and rotation carry
# it on: a pair rotates two errors of size dy scaled by r * gamma, and r
# itself moves by at most sqrt(D) * max dy / ||y|| relative.  Each element is
# held to spacing(z) + 2^-16 max_row|z| plus that propagated dy, and every
# row to the 4e-3 relative bar.


def _check8(label, got_bits, ref, ref_bits, dy, y_pre, gamma):
    """dy, y_pre: [H, T, D] error bound and exact pre-norm value; gamma None for v."""
    mag = np.abs(ref)
    spacing = np.exp2(np.maximum(np.floor(np.log2(np.where(mag > 0, mag, 1.0))) - 7, -133))
    slack = spacing + 2.0 ** -16 * mag.max(axis=-1, keepdims=True)
    if gamma is None:
        slack = slack + dy
    else:
        D = y_pre.shape[-1]
        norm = np.linalg.norm(y_pre, axis=-1, keepdims=True)
        r = np.sqrt(D) / np.maximum(norm, 1e-300)
        dmax = dy.max(axis=-1, keepdims=True)
        slack = (slack + 2.0 * r * float(np.abs(gamma).max()) * dmax
                 + mag.max(axis=-1, keepdims=True) * 1.1 * np.sqrt(D) * dmax / np.maximum(norm, 1e-300))
    err = np.abs(oracle.bf16_to_f64(got_bits) - ref)
    ratio = float((err / slack).max())
    mism = float(np.mean(got_bits != ref_bits))
    rel = float(row_rel_err(got_bits.reshape(-1, 128), ref.reshape(-1, 128)).max())
    print(f"{label}: max err/bound {ratio:.3f}, mismatch vs RNE(exact) {mism:.2e}, max row rel {rel:.2e}")
    assert ratio <= 1.0
    assert rel <= ATTN_TOL
    # The instruction's truncation moves every element whose exact value lies
    # within about dy of a bf16 rounding boundary: ~1.2% of elements were
    # measured to differ from RNE(exact) at H3's hidden size (1.6-3.9% on a
    # single 128-element token); a wrong operand, scale or pairing would move
    # most of them.  Gate: a binomial bound at a 2% rate, four standard
    # deviations plus three elements of slack for small counts.
    n = got_bits.size
    assert int(np.sum(got_bits != ref_bits)) <= 0.02 * n + 4 * np.sqrt(0.02 * n) + 3


def _run8(gpu_lib, x, H, rows=None, label=""):
    import torch
    d = {n: to_dev(x[n], torch.uint8).view(torch.float8_e4m3fn) for n in ("x", "wq", "wk", "wv")}
    xs = to_dev(np.array([x["x_scale"]], np.float32), torch.float32)
    ws = to_dev(np.array([x["w_scale"]], np.float32), torch.float32)
    gq, gk = to_dev(x["gamma_q"], torch.float32), to_dev(x["gamma_k"], torch.float32)
    cos, sin = gpu_lib.rope_tables(to_dev(x["positions"], torch.int32), 128, x["theta"])
    q, k, v = gpu_lib.qkv_proj_fp8_qknorm_rope(d["x"], xs, d["wq"], d["wk"], d["wv"], ws, gq, gk, cos, sin,
                                               x["eps"])
    torch.cuda.synchronize()
    c_ref, s_ref = oracle.rope_tables(x["positions"], 128, x["theta"])
    xr = x["x"] if rows is None else x["x"][rows]
    cr, sr = (c_ref, s_ref) if rows is None else (c_ref[rows], s_ref[rows])
    ref = oracle.qkv_proj_fp8_qknorm_rope(xr, x["x_scale"], x["wq"], x["wk"], x["wv"], x["w_scale"],
                                          x["gamma_q"], x["gamma_k"], cr, sr, x["eps"], H)
    xf = np.abs(oracle.e4m3_to_f64(xr))
    sc = float(x["x_scale"]) * float(x["w_scale"])
    for name, t, gname in (("q", q, "gamma_q"), ("k", k, "gamma_k"), ("v", v, None)):
        got = bits(t)
        if rows is not None:
            got = got[:, rows]
        wf = oracle.e4m3_to_f64(x["w" + name])
        dy = oracle.split_heads(sc * (7 * 2.0 ** -13 + 2.0 ** -20) * (xf @ np.abs(wf).T), H)
        y_pre = oracle.split_heads(sc * (oracle.e4m3_to_f64(xr) @ wf.T), H)
        _check8(f"{label} fp8 {name}", got, *ref[name], dy, y_pre, None if gname is None else x[gname])
    return q, k, v


@pytest.mark.parametrize("H,L,hidden", [(2, 300, 512), (1, 1, 64), (3, 257, 192), (1, 1000, 5376)])
def test_qkv_proj_fp8_all_elements(gpu_lib, H, L, hidden):
    """e4m3 operands with per-tensor scales: every element of q, k and v, on
    one token, a single hidden step, ragged token tiles and H3's hidden size."""
    w = I.ProjWorkload(f"f8_H{H}_L{L}", H=H, L=L, n_video=L - L // 5, n_audio=L // 5, hidden=hidden, fp8=True)
    _run8(gpu_lib, I.make_proj_inputs(w, 200 + L), H, label=f"H={H} L={L} hidden={hidden}")


def test_qkv_proj_fp8_ws2_sampled(gpu_lib):
    """H = 28, L = 32768, hidden 5376 in fp8: 512 sampled tokens."""
    w = I.PROJ_WORKLOADS["proj8_ws2"]
    x = I.make_proj_inputs(w, 0)
    _run8(gpu_lib, x, w.H, rows=I.sample_rows(w, 0, 512), label="proj8_ws2")


# eps reaches the kernel as a run-time argument.  The q and k weight slices
# are scaled by an exact power of two so that the pre-norm values have a mean
# square near eps, and eps then moves every q and k output substantially.
@pytest.mark.parametrize("eps,shift", [(1e-3, 5), (1e-9, 15)])
def test_qkv_proj_nondefault_eps(gpu_lib, eps, shift):
    w = I.ProjWorkload("eps_bf16", H=2, L=300, n_video=256, n_audio=44, hidden=512)
    x = dict(I.make_proj_inputs(w, 31))
    for n in ("wq", "wk"):
        x[n] = I.f32_to_bf16_bits((oracle.bf16_to_f64(x[n]) * 2.0 ** -shift).astype(np.float32))
    x["eps"] = eps
    _run(gpu_lib, x, w.H, label=f"bf16 eps={eps:g}")


@pytest.mark.parametrize("eps,shift", [(1e-3, 5), (1e-9, 15)])
def test_qkv_proj_fp8_nondefault_eps(gpu_lib, eps, shift):
    """The fp8 form: the weight tensor's scale carries the power of two (the
    same factor for the v slice, which the norm does not touch)."""
    w = I.ProjWorkload("eps_fp8", H=2, L=300, n_video=256, n_audio=44, hidden=512, fp8=True)
    x = dict(I.make_proj_inputs(w, 32))
    x["w_scale"] = np.float32(float(x["w_scale"]) * 2.0 ** -shift)
    x["eps"] = eps
    _run8(gpu_lib, x, w.H, label=f"fp8 eps={eps:g}")


@pytest.mark.parametrize("shared", [True, False])
def test_qkv_proj_fp8_group_truncation(gpu_lib, shared):
    """The fp8 element bound rests on how the matrix instruction sums its
    products: in groups of 8 consecutive hidden elements of a lane's operand,
    each product truncated toward zero 2^-13 below the group's largest.  This
    case makes that visible through the ABI.  674 groups hold a product of 1
    (1.0 x 1.0) and seven products of 0.875 * 2^-13 (0.875 * 2^-6 x 2^-7), so
    the exact sum is 674 * (1 + 6.125 * 2^-13) = 674.504, which rounds to
    bf16 676.  With the small products in the same groups as the 1s
    (shared) they are truncated away: the sum is exactly 674, a tie between
    672 and 676 that rounds to even, 672.  In groups of their own they are
    each their group's largest, survive, and the result is 676.  Both results
    must lie within the bound the other fp8 checks use: one bf16 spacing plus
    2^-16 of the row's largest value plus (7 * 2^-13 + 2^-20) * sum |x w|."""
    import torch
    n_big = 674
    C = 5440 if shared else 10816            # multiples of 64
    one, small_x, small_w = 0x38, 0x07, 0x04   # e4m3 codes of 1.0, 0.875 * 2^-6, 2^-7
    assert oracle.e4m3_to_f64(np.array([one, small_x, small_w], np.uint8)).tolist() == [1.0, 0.875 / 64, 1 / 128]
    x8 = np.zeros((1, C), np.uint8)
    w8 = np.zeros((128, C), np.uint8)
    for m in range(n_big):
        x8[0, 8 * m] = one
        w8[:, 8 * m] = one
        base = 8 * m if shared else 8 * (n_big + m)
        x8[0, base + 1:base + 8] = small_x
        w8[:, base + 1:base + 8] = small_w
    zeros = np.zeros_like(w8)
    dev8 = lambda a: to_dev(a, torch.uint8).view(torch.float8_e4m3fn)
    unit = to_dev(np.array([1.0], np.float32), torch.float32)
    g = to_dev(np.ones(128, np.float32), torch.float32)
    cos, sin = gpu_lib.rope_tables(to_dev(np.zeros(1, np.int32), torch.int32), 128, 10000.0)
    q, k, v = gpu_lib.qkv_proj_fp8_qknorm_rope(dev8(x8), unit, dev8(zeros), dev8(zeros), dev8(w8), unit, g, g,
                                               cos, sin, 1e-6)
    torch.cuda.synchronize()
    got = oracle.bf16_to_f64(bits(v)).reshape(-1)
    y = 1.0 * (oracle.e4m3_to_f64(x8) @ oracle.e4m3_to_f64(w8).T).reshape(-1)
    assert np.allclose(y, n_big * (1 + 6.125 * 2.0 ** -13), rtol=0, atol=1e-9)
    assert np.all(oracle.bf16_to_f64(oracle.f64_to_bf16_bits(y)) == 676.0)
    dy = (7 * 2.0 ** -13 + 2.0 ** -20) * (np.abs(oracle.e4m3_to_f64(x8)) @ np.abs(oracle.e4m3_to_f64(w8)).T).reshape(-1)
    slack = 4.0 + 2.0 ** -16 * np.abs(y).max() + dy    # one bf16 spacing in [512, 1024) is 4
    ratio = float((np.abs(got - y) / slack).max())
    print(f"shared={shared}: v = {sorted(set(got.tolist()))}, exact {y[0]:.4f}, err/bound {ratio:.3f}")
    assert ratio <= 1.0
    assert np.all(got == (672.0 if shared else 676.0))
    assert np.all(bits(q) == 0) and np.all(bits(k) == 0)
