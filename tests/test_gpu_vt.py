"""GPU checks of the transposed-V forms, through the C ABI.

h3_attention_vt must give h3_attention's result bit for bit on the same values
(it performs the same products in the same order; only the LDS layout of V
differs), and is also compared with the oracle directly.  The padding columns
it may read (from L up to the next multiple of 8) hold arbitrary finite values
and every later column holds NaN: neither may reach the output.  The
projection's _vt forms must write q and k exactly as the [H][L][D] forms do,
v transposed bit for bit, zeros in the padding columns and nothing past them.
"""
import math

import numpy as np
import pytest

import oracle
from exact_head_attention_amd import inputs as I
from tests.gpu_helpers import attention_errors, bits, check_attention_errors, merge_errors, to_dev

pytestmark = pytest.mark.gpu


def _raw(H, L, seed):
    import torch
    rng = np.random.Generator(np.random.PCG64(seed))
    return [to_dev(I.f32_to_bf16_bits(rng.standard_normal((H, L, 128), dtype=np.float32)), torch.bfloat16)
            for _ in range(3)]


def _transposed(v, ldv, seed):
    """vt [H, 128, ldv] holding v's values; finite noise (|x| up to ~400) in
    the columns from L to the next multiple of 8, NaN in every later column."""
    import torch
    H, L, D = v.shape
    l8 = (L + 7) // 8 * 8
    vt = torch.full((H, D, ldv), float("nan"), dtype=torch.bfloat16, device=v.device)
    vt[:, :, :L] = v.transpose(1, 2)
    if l8 > L:
        rng = np.random.Generator(np.random.PCG64(seed))
        noise = I.f32_to_bf16_bits(100 * rng.standard_normal((H, D, l8 - L), dtype=np.float32))
        vt[:, :, L:l8] = to_dev(noise, torch.bfloat16)
    return vt


def _same_bits(a, b, label):
    import torch
    torch.cuda.synchronize()
    ab, bb = bits(a), bits(b)
    n = int(np.sum(ab != bb))
    print(f"{label}: {n} differing elements of {ab.size}")
    assert n == 0


# Ragged tails in every position of the last key tile, a length with no
# padding column (a multiple of 8) and one past a whole tile.
@pytest.mark.parametrize("L", [1, 7, 8, 63, 64, 65, 129, 255, 257, 513, 1000])
def test_attention_vt_equals_attention(gpu_lib, L):
    q, k, v = _raw(2, L, seed=300 + L)
    ldv = (L + 7) // 8 * 8 + 16
    vt = _transposed(v, ldv, seed=L)
    _same_bits(gpu_lib.attention_vt(q, k, vt), gpu_lib.attention(q, k, v), f"vt L={L} ldv={ldv}")


def _vt_vs_oracle(gpu_lib, H, L, seed, scale):
    import torch
    q, k, v = _raw(H, L, seed=seed)
    out = gpu_lib.attention_vt(q, k, _transposed(v, (L + 7) // 8 * 8 + 8, seed=5), scale=scale)
    torch.cuda.synchronize()
    qb, kb, vb, ob = bits(q), bits(k), bits(v), bits(out)
    parts = []
    for h in range(H):
        ref = oracle.attention_head(oracle.bf16_to_f64(qb[h]), oracle.bf16_to_f64(kb[h]),
                                    oracle.bf16_to_f64(vb[h]), scale)
        parts.append(attention_errors(oracle.bf16_to_f64(ob[h]), ref))
    check_attention_errors(f"vt H={H} L={L} scale={scale:.4g}", merge_errors(parts))


def test_attention_vt_vs_oracle(gpu_lib):
    """Every row of a ragged 3-head case against the oracle directly."""
    _vt_vs_oracle(gpu_lib, 3, 777, 41, 1 / math.sqrt(128))


@pytest.mark.parametrize("scale", [0.03, 0.3])
@pytest.mark.parametrize("H,L", [(10, 4900), (3, 1000)])
def test_attention_vt_nondefault_scale(gpu_lib, scale, H, L):
    """Two scales other than 1/sqrt(128), through the main launch (200 units)
    and the tail launch (12 units), every row against the oracle."""
    _vt_vs_oracle(gpu_lib, H, L, 900 + L, scale)


# On a 256-CU part: (1, 4096) runs every unit in the tail launch; (7, 32768),
# one rank's share at world size 8, three full rounds plus a tail launch;
# (10, 6000) one partial round in the main launch only; (56, 4096) all 56
# heads at once, again three rounds plus a tail.
@pytest.mark.parametrize("H,L", [(1, 4096), (7, 32768), (10, 6000), (56, 4096)])
def test_attention_vt_launch_shapes_bit_identical(gpu_lib, H, L):
    q, k, v = _raw(H, L, seed=H * 100003 + L)
    vt = _transposed(v, L, seed=1)
    _same_bits(gpu_lib.attention_vt(q, k, vt), gpu_lib.attention(q, k, v), f"vt H={H} L={L}")


def test_attention_vt_longest_rows(gpu_lib):
    """ldv at its maximum (2^23): one head's V^T spans exactly 2^31 bytes, the
    largest buffer range and row offsets the loads use."""
    import torch
    L, ldv = 1000, 1 << 23
    q, k, v = _raw(1, L, seed=77)
    vt = torch.zeros((1, 128, ldv), dtype=torch.bfloat16, device=v.device)
    vt[:, :, :L] = v.transpose(1, 2)
    vt[:, :, 1008:] = float("nan")
    _same_bits(gpu_lib.attention_vt(q, k, vt), gpu_lib.attention(q, k, v), f"vt L={L} ldv=2^23")
    del vt
    torch.cuda.empty_cache()


def test_attention_vt_head_splits_bit_identical(gpu_lib):
    """Heads launched together or one at a time (vt offset by h*128*ldv)."""
    import torch
    H, L, ldv = 5, 1500, 1512
    q, k, v = _raw(H, L, seed=9)
    vt = _transposed(v, ldv, seed=2)
    full = gpu_lib.attention_vt(q, k, vt)
    parts = torch.cat([gpu_lib.attention_vt(q[h:h + 1], k[h:h + 1], vt[h:h + 1]) for h in range(H)])
    _same_bits(parts, full, "vt head splits")


# ------------------------------------------------------------ projection


def _proj_pair(gpu_lib, w, x, ldv):
    """(q, k, v) of the [H][L][D] form and (q, k, vt) of the _vt form, vt
    pre-filled with a sentinel so untouched columns can be recognised."""
    import torch
    cos, sin = gpu_lib.rope_tables(to_dev(x["positions"], torch.int32), 128, x["theta"])
    gq, gk = to_dev(x["gamma_q"], torch.float32), to_dev(x["gamma_k"], torch.float32)
    vt = torch.full((w.H, 128, ldv), 12345.0, dtype=torch.bfloat16, device="cuda:0")
    q0 = torch.empty((w.H, w.L, 128), dtype=torch.bfloat16, device="cuda:0")
    out_vt = (q0, torch.empty_like(q0), vt)
    if w.fp8:
        d = {n: to_dev(x[n], torch.uint8).view(torch.float8_e4m3fn) for n in ("x", "wq", "wk", "wv")}
        xs = to_dev(np.array([x["x_scale"]], np.float32), torch.float32)
        ws = to_dev(np.array([x["w_scale"]], np.float32), torch.float32)
        ref = gpu_lib.qkv_proj_fp8_qknorm_rope(d["x"], xs, d["wq"], d["wk"], d["wv"], ws, gq, gk, cos, sin, x["eps"])
        got = gpu_lib.qkv_proj_fp8_qknorm_rope(d["x"], xs, d["wq"], d["wk"], d["wv"], ws, gq, gk, cos, sin, x["eps"],
                                               out=out_vt, ldv=ldv)
    else:
        d = {n: to_dev(x[n], torch.bfloat16) for n in ("x", "wq", "wk", "wv")}
        ref = gpu_lib.qkv_proj_qknorm_rope(d["x"], d["wq"], d["wk"], d["wv"], gq, gk, cos, sin, x["eps"])
        got = gpu_lib.qkv_proj_qknorm_rope(d["x"], d["wq"], d["wk"], d["wv"], gq, gk, cos, sin, x["eps"],
                                           out=out_vt, ldv=ldv)
    torch.cuda.synchronize()
    return ref, got


@pytest.mark.parametrize("H,L,hidden,fp8", [(1, 1, 32, False), (3, 257, 96, False), (2, 513, 160, False),
                                            (2, 300, 512, True), (1, 1, 64, True), (3, 1003, 192, True)])
def test_qkv_proj_vt_matches_row_major(gpu_lib, H, L, hidden, fp8):
    w = I.ProjWorkload(f"vt_H{H}_L{L}", H=H, L=L, n_video=L - L // 5, n_audio=L // 5, hidden=hidden, fp8=fp8)
    x = I.make_proj_inputs(w, 3)
    l8 = (L + 7) // 8 * 8
    ldv = l8 + 8
    (q, k, v), (qt, kt, vt) = _proj_pair(gpu_lib, w, x, ldv)
    assert np.array_equal(bits(qt), bits(q)) and np.array_equal(bits(kt), bits(k))
    vtb, vb = bits(vt), bits(v)
    assert np.array_equal(vtb[:, :, :L], vb.transpose(0, 2, 1)), "v transposed"
    assert np.all(vtb[:, :, L:l8] == 0), "padding columns are +0"
    sentinel = I.f32_to_bf16_bits(np.float32(12345.0))
    assert np.all(vtb[:, :, l8:] == sentinel), "columns past the padding untouched"


def test_qkv_proj_vt_then_attention_vt(gpu_lib):
    """The transposed chain equals the row-major chain bit for bit."""
    w = I.PROJ_WORKLOADS["proj_tiny"]
    x = I.make_proj_inputs(w, 1)
    (q, k, v), (qt, kt, vt) = _proj_pair(gpu_lib, w, x, (w.L + 7) // 8 * 8)
    _same_bits(gpu_lib.attention_vt(qt, kt, vt), gpu_lib.attention(q, k, v), "proj_tiny vt chain")
