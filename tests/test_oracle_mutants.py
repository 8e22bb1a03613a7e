"""The pins catch plausible oracle mistakes.

Each case plants one mistake in a copy of an oracle function (on the CPU only),
runs the pin tests of tests/test_oracle.py against it, and requires at least
one of them to fail.
"""
import numpy as np
import pytest

import oracle
import oracle.h3_oracle as H
from tests import test_oracle as T


def _rms_no_eps(x, gamma, eps):
    x = np.asarray(x, np.float64)
    return x / np.sqrt(np.mean(x * x, axis=-1, keepdims=True)) * gamma


def _rms_sum(x, gamma, eps):
    x = np.asarray(x, np.float64)
    return x / np.sqrt(np.sum(x * x, axis=-1, keepdims=True) + eps) * gamma


def _rms_no_gamma(x, gamma, eps):
    x = np.asarray(x, np.float64)
    return x / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps)


def _rope_sign(y, cos, sin):
    y = np.asarray(y, np.float64)
    out = np.empty_like(y)
    out[..., 0::2] = y[..., 0::2] * cos + y[..., 1::2] * sin
    out[..., 1::2] = -y[..., 0::2] * sin + y[..., 1::2] * cos
    return out


def _rope_half_split(y, cos, sin):
    y = np.asarray(y, np.float64)
    h = y.shape[-1] // 2
    a, b = y[..., :h], y[..., h:]
    return np.concatenate([a * cos - b * sin, a * sin + b * cos], axis=-1)


def _tables_wrong_exponent(positions, D=128, theta=10000.0):
    pos = np.asarray(positions, np.float64)
    inv = np.power(float(theta), -np.arange(D // 2) / D)
    ang = pos[:, None] * inv[None, :]
    return np.cos(ang).astype(np.float32), np.sin(ang).astype(np.float32)


def _bf16_double_rounding(x):
    x32 = np.asarray(x, np.float64).astype(np.float32)
    import torch
    return torch.from_numpy(x32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def _bf16_truncate(x):
    x32 = np.asarray(x, np.float64).astype(np.float32)
    return (x32.view(np.uint32) >> np.uint32(16)).astype(np.uint16)


def _attn_no_scale(q, k, v, scale, block=256):
    return H.__dict__["_orig_attention_head"](q, k, v, 1.0, block)


def _attn_transposed(q, k, v, scale, block=256):
    s = scale * (np.asarray(k) @ np.asarray(q).T).T if q.shape[0] == k.shape[0] else scale * (k @ q.T)
    s = s - s.max(axis=1, keepdims=True)
    e = np.exp(s)
    return (e / e.sum(axis=1, keepdims=True)) @ v


def _attn_unnormalised(q, k, v, scale, block=256):
    s = scale * (np.asarray(q) @ np.asarray(k).T)
    e = np.exp(s - s.max(axis=1, keepdims=True))
    return e @ v


def _attn_no_max(q, k, v, scale, block=256):
    s = scale * (np.asarray(q) @ np.asarray(k).T)
    with np.errstate(all="ignore"):
        e = np.exp(s)
        return (e / e.sum(axis=1, keepdims=True)) @ v


def _attn_softmax_over_queries(q, k, v, scale, block=256):
    s = scale * (np.asarray(q) @ np.asarray(k).T)
    e = np.exp(s - s.max(axis=0, keepdims=True))
    return (e / e.sum(axis=0, keepdims=True)) @ v


def _merge_linear_weights(outs, lses):
    outs, lses = np.asarray(outs, np.float64), np.asarray(lses, np.float64)
    w = lses - lses.min(axis=0)[None] + 1.0
    return (w[..., None] * outs).sum(axis=0) / w.sum(axis=0)[..., None], np.log(np.exp(lses).sum(axis=0))


def _lse_missing_log(q, k, v, scale, block=256):
    out, lse = H.__dict__["_orig_attention_lse_head"](q, k, v, scale, block)
    s = scale * (np.asarray(q) @ np.asarray(k).T)
    return out, s.max(axis=1) + np.exp(lse - s.max(axis=1))


def _split_heads_dim_major(y, H, D=128):
    L = y.shape[0]
    return np.ascontiguousarray(y.reshape(L, D, H).transpose(2, 0, 1))


def _project_no_transpose_rows(x_bits, w_bits):
    # uses the weight's columns in reverse order (a transposed/reversed operand)
    return H.bf16_to_f64(x_bits) @ H.bf16_to_f64(w_bits)[:, ::-1].T


def _qkv_norms_v_too(x_bits, wq_bits, wk_bits, wv_bits, gamma_q, gamma_k, cos, sin, eps, Hh, D=128):
    out = H.__dict__["_orig_qkv"](x_bits, wq_bits, wk_bits, wv_bits, gamma_q, gamma_k, cos, sin, eps, Hh, D)
    y = H.rope_rotate(H.rms_norm(out["v"][0], gamma_k, eps), cos[None], sin[None])
    out["v"] = (y, H.f64_to_bf16_bits(y))
    return out


def _qkv_swapped_gammas(x_bits, wq_bits, wk_bits, wv_bits, gamma_q, gamma_k, cos, sin, eps, Hh, D=128):
    return H.__dict__["_orig_qkv"](x_bits, wq_bits, wk_bits, wv_bits, gamma_k, gamma_q, cos, sin, eps, Hh, D)


def _e4m3_bias8(bits):
    return H.__dict__["_orig_e4m3"](bits) / 2.0


def _fp8_scale_dropped_for_qk(x8, x_scale, wq8, wk8, wv8, w_scale, gamma_q, gamma_k, cos, sin, eps, Hh, D=128):
    out = H.__dict__["_orig_qkv8"](x8, 1.0, wq8, wk8, wv8, 1.0, gamma_q, gamma_k, cos, sin, eps, Hh, D)
    ref = H.__dict__["_orig_qkv8"](x8, x_scale, wq8, wk8, wv8, w_scale, gamma_q, gamma_k, cos, sin, eps, Hh, D)
    out["v"] = ref["v"]
    return out


PIN_TESTS = [getattr(T, n) for n in dir(T) if n.startswith("test_")]

MUTANTS = {
    "rms_no_eps": ("rms_norm", _rms_no_eps),
    "rms_sum_not_mean": ("rms_norm", _rms_sum),
    "rms_no_gamma": ("rms_norm", _rms_no_gamma),
    "rope_sign": ("rope_rotate", _rope_sign),
    "rope_half_split": ("rope_rotate", _rope_half_split),
    "tables_exponent": ("rope_tables", _tables_wrong_exponent),
    "bf16_double_rounding": ("f64_to_bf16_bits", _bf16_double_rounding),
    "bf16_truncate": ("f64_to_bf16_bits", _bf16_truncate),
    "attn_no_scale": ("attention_head", _attn_no_scale),
    "attn_transposed": ("attention_head", _attn_transposed),
    "attn_unnormalised": ("attention_head", _attn_unnormalised),
    "attn_no_max_shift": ("attention_head", _attn_no_max),
    "attn_softmax_wrong_axis": ("attention_head", _attn_softmax_over_queries),
    "merge_linear_weights": ("merge_partials", _merge_linear_weights),
    "lse_missing_log": ("attention_lse_head", _lse_missing_log),
    "split_heads_dim_major": ("split_heads", _split_heads_dim_major),
    "project_reversed_operand": ("qkv_project", _project_no_transpose_rows),
    "qkv_norms_v": ("qkv_proj_qknorm_rope", _qkv_norms_v_too),
    "qkv_swapped_gammas": ("qkv_proj_qknorm_rope", _qkv_swapped_gammas),
    "e4m3_bias8": ("e4m3_to_f64", _e4m3_bias8),
    "fp8_scale_dropped_for_qk": ("qkv_proj_fp8_qknorm_rope", _fp8_scale_dropped_for_qk),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_mutant(name, monkeypatch):
    fn_name, mutant = MUTANTS[name]
    monkeypatch.setitem(H.__dict__, "_orig_attention_head", H.attention_head)
    monkeypatch.setitem(H.__dict__, "_orig_attention_lse_head", H.attention_lse_head)
    monkeypatch.setitem(H.__dict__, "_orig_qkv", H.qkv_proj_qknorm_rope)
    monkeypatch.setitem(H.__dict__, "_orig_e4m3", H.e4m3_to_f64)
    monkeypatch.setitem(H.__dict__, "_orig_qkv8", H.qkv_proj_fp8_qknorm_rope)
    monkeypatch.setattr(H, fn_name, mutant)
    monkeypatch.setattr(oracle, fn_name, mutant)
    failed = []
    for t in PIN_TESTS:
        try:
            t()
        except Exception:  # an assertion or an error: either way the pin caught it
            failed.append(t.__name__)
    assert failed, f"mutant {name} passed every pin"
