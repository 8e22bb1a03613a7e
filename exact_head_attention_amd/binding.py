"""Python binding of libh3attn.so (ctypes).  Argument marshalling only.

Tensors are PyTorch device tensors on the current HIP device; every call is
enqueued on torch's current stream.  The binding checks dtypes, shapes and
contiguity, passes raw pointers, and raises H3Error on a nonzero status.  There
is no fallback: if the library is missing, importing this module fails.
"""
from __future__ import annotations

import ctypes
import math
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libh3attn.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is not built; run `python -m exact_head_attention_amd.build` "
                      "(or __graft_entry__.build()) first")

lib = ctypes.CDLL(LIB_PATH)

_vp, _i, _f, _d = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_double
lib.h3_qknorm_rope.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _f, _vp]
lib.h3_qknorm_rope.restype = _i
lib.h3_attention.argtypes = [_vp, _vp, _vp, _vp, _i, _i, _i, _f, _vp]
lib.h3_attention.restype = _i
lib.h3_rope_tables.argtypes = [_vp, _i, _i, _d, _vp, _vp, _vp]
lib.h3_rope_tables.restype = _i
_ll = ctypes.c_longlong
lib.h3_attention_vt.argtypes = [_vp, _vp, _vp, _vp, _i, _i, _i, _i, _f, _vp]
lib.h3_attention_vt.restype = _i
lib.h3_attention_lse.argtypes = [_vp, _vp, _vp, _vp, _vp, _i, _i, _i, _ll, _i, _f, _vp]
lib.h3_attention_lse.restype = _i
lib.h3_attention_merge.argtypes = [_vp, _vp, _i, _vp, _vp, _i, _i, _i, _vp]
lib.h3_attention_merge.restype = _i
lib.h3_qkv_proj_qknorm_rope.argtypes = [_vp] * 11 + [_i, _i, _i, _i, _f, _vp]
lib.h3_qkv_proj_qknorm_rope.restype = _i
lib.h3_qkv_proj_fp8_qknorm_rope.argtypes = [_vp] * 13 + [_i, _i, _i, _i, _f, _vp]
lib.h3_qkv_proj_fp8_qknorm_rope.restype = _i
lib.h3_qkv_proj_qknorm_rope_vt.argtypes = [_vp] * 11 + [_i, _i, _i, _i, _i, _f, _vp]
lib.h3_qkv_proj_qknorm_rope_vt.restype = _i
lib.h3_qkv_proj_fp8_qknorm_rope_vt.argtypes = [_vp] * 13 + [_i, _i, _i, _i, _i, _f, _vp]
lib.h3_qkv_proj_fp8_qknorm_rope_vt.restype = _i
lib.h3_status_string.argtypes = [_i]
lib.h3_status_string.restype = ctypes.c_char_p
lib.h3_abi_version.argtypes = []
lib.h3_abi_version.restype = _i

HEAD_DIM = 128
EXPORTED = ("h3_qknorm_rope", "h3_attention", "h3_attention_vt", "h3_rope_tables", "h3_attention_lse", "h3_attention_merge",
            "h3_qkv_proj_qknorm_rope", "h3_qkv_proj_fp8_qknorm_rope", "h3_qkv_proj_qknorm_rope_vt",
            "h3_qkv_proj_fp8_qknorm_rope_vt", "h3_status_string", "h3_abi_version")


class H3Error(RuntimeError):
    def __init__(self, fn: str, status: int):
        self.status = status
        super().__init__(f"{fn}: {lib.h3_status_string(status).decode()} (status {status})")


def _check(fn: str, status: int) -> None:
    if status != 0:
        raise H3Error(fn, status)


def _stream():
    import torch
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _dev(t, dtype, name):
    import torch
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError(f"{name} must be a GPU tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _hld(t, name):
    if t.dim() != 3 or t.shape[2] != HEAD_DIM:
        raise ValueError(f"{name} must be [H, L, {HEAD_DIM}], got {tuple(t.shape)}")
    return t.shape[0], t.shape[1], t.shape[2]


def rope_tables(positions, D: int = HEAD_DIM, theta: float = 10000.0):
    """cos, sin fp32 [L, D/2] of positions (int32 [L], on the GPU)."""
    import torch
    L = positions.shape[0]
    cos = torch.empty((L, D // 2), dtype=torch.float32, device=positions.device)
    sin = torch.empty_like(cos)
    _check("h3_rope_tables", lib.h3_rope_tables(_dev(positions, torch.int32, "positions"), L, D,
                                                float(theta), _dev(cos, torch.float32, "cos"),
                                                _dev(sin, torch.float32, "sin"), _stream()))
    return cos, sin


def qknorm_rope(q, k, gamma_q, gamma_k, cos, sin, eps: float = 1e-6) -> None:
    """In place: q, k (bf16 [H, L, 128]) <- RoPE(RMSNorm(x) * gamma)."""
    import torch
    H, L, D = _hld(q, "q")
    if tuple(k.shape) != (H, L, D):
        raise ValueError("k must have q's shape")
    if tuple(cos.shape) != (L, D // 2) or tuple(sin.shape) != (L, D // 2):
        raise ValueError(f"cos/sin must be [{L}, {D // 2}]")
    if gamma_q.numel() != D or gamma_k.numel() != D:
        raise ValueError(f"gamma_q/gamma_k must have {D} elements")
    _check("h3_qknorm_rope", lib.h3_qknorm_rope(
        _dev(q, torch.bfloat16, "q"), _dev(k, torch.bfloat16, "k"),
        _dev(gamma_q, torch.float32, "gamma_q"), _dev(gamma_k, torch.float32, "gamma_k"),
        _dev(cos, torch.float32, "cos"), _dev(sin, torch.float32, "sin"),
        H, L, D, float(eps), _stream()))


def attention(q, k, v, out=None, scale: float | None = None):
    """out = softmax(scale q k^T) v per head; bf16 [H, L, 128].  Returns out."""
    import torch
    H, L, D = _hld(q, "q")
    if tuple(k.shape) != (H, L, D) or tuple(v.shape) != (H, L, D):
        raise ValueError("k and v must have q's shape")
    if out is None:
        out = torch.empty_like(q)
    elif tuple(out.shape) != (H, L, D):
        raise ValueError("out must have q's shape")
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    _check("h3_attention", lib.h3_attention(
        _dev(q, torch.bfloat16, "q"), _dev(k, torch.bfloat16, "k"), _dev(v, torch.bfloat16, "v"),
        _dev(out, torch.bfloat16, "out"), H, L, D, float(scale), _stream()))
    return out


def attention_vt(q, k, vt, out=None, scale: float | None = None):
    """attention() with V transposed: vt bf16 [H, 128, ldv], row (h, d) holding
    v[h, :, d] in its first L columns (L <= ldv, ldv a multiple of 8; columns
    L .. up to the next multiple of 8 finite).  Returns out bf16 [H, L, 128]."""
    import torch
    H, L, D = _hld(q, "q")
    if tuple(k.shape) != (H, L, D):
        raise ValueError("k must have q's shape")
    if vt.dim() != 3 or vt.shape[0] != H or vt.shape[1] != D or vt.shape[2] < L:
        raise ValueError(f"vt must be [{H}, {D}, ldv >= {L}], got {tuple(vt.shape)}")
    if out is None:
        out = torch.empty_like(q)
    elif tuple(out.shape) != (H, L, D):
        raise ValueError("out must have q's shape")
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    _check("h3_attention_vt", lib.h3_attention_vt(
        _dev(q, torch.bfloat16, "q"), _dev(k, torch.bfloat16, "k"), _dev(vt, torch.bfloat16, "vt"),
        _dev(out, torch.bfloat16, "out"), H, L, vt.shape[2], D, float(scale), _stream()))
    return out


def _kv_view(t, name):
    """Pointer and head stride of a key/value tensor [H, Lk, D] whose rows are
    contiguous (e.g. a key-range slice t_full[:, j0:j1] of a [H, L, D] tensor)."""
    import torch
    if not isinstance(t, torch.Tensor) or not t.is_cuda or t.dtype != torch.bfloat16:
        raise TypeError(f"{name} must be a bf16 GPU tensor")
    if t.dim() != 3 or t.shape[2] != HEAD_DIM or t.stride(2) != 1 or t.stride(1) != HEAD_DIM:
        raise ValueError(f"{name} must be [H, Lk, {HEAD_DIM}] with contiguous rows")
    return ctypes.c_void_p(t.data_ptr()), int(t.stride(0)) if t.shape[0] > 1 else t.shape[1] * HEAD_DIM


def attention_lse(q, k, v, scale: float | None = None, out=None, lse=None):
    """Partial attention of q over the keys in k, v (which may be a key-range
    slice of a larger tensor).  Returns (out fp32 [H, Lq, 128], lse fp32 [H, Lq])."""
    import torch
    H, Lq, D = _hld(q, "q")
    pk, sk = _kv_view(k, "k")
    pv, sv = _kv_view(v, "v")
    if k.shape != v.shape or k.shape[0] != H or sk != sv:
        raise ValueError("k and v must have the same shape and head stride, with q's head count")
    Lk = k.shape[1]
    if out is None:
        out = torch.empty((H, Lq, D), dtype=torch.float32, device=q.device)
    if lse is None:
        lse = torch.empty((H, Lq), dtype=torch.float32, device=q.device)
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    _check("h3_attention_lse", lib.h3_attention_lse(
        _dev(q, torch.bfloat16, "q"), pk, pv, _dev(out, torch.float32, "out"), _dev(lse, torch.float32, "lse"),
        H, Lq, Lk, sk, D, float(scale), _stream()))
    return out, lse


def attention_merge(outs, lses, out=None, want_lse: bool = False):
    """Merge stacked partials outs fp32 [P, H, L, 128], lses fp32 [P, H, L]
    into bf16 [H, L, 128] (and the merged lse when want_lse)."""
    import torch
    if outs.dim() != 4 or outs.shape[3] != HEAD_DIM or tuple(lses.shape) != tuple(outs.shape[:3]):
        raise ValueError("outs must be [P, H, L, 128] and lses [P, H, L]")
    P, H, L, D = outs.shape
    if out is None:
        out = torch.empty((H, L, D), dtype=torch.bfloat16, device=outs.device)
    lse_out = torch.empty((H, L), dtype=torch.float32, device=outs.device) if want_lse else None
    _check("h3_attention_merge", lib.h3_attention_merge(
        _dev(outs, torch.float32, "outs"), _dev(lses, torch.float32, "lses"), P, _dev(out, torch.bfloat16, "out"),
        _dev(lse_out, torch.float32, "lse_out") if want_lse else None, H, L, D, _stream()))
    return (out, lse_out) if want_lse else out


def _proj_shapes(x, wq, wk, wv, gamma_q, gamma_k, cos, sin, out, ldv):
    """Checks the projection's shapes; returns (H, L, C, out) with out
    allocated when None (v as [H, 128, ldv] when ldv is not None)."""
    import torch
    if x.dim() != 2:
        raise ValueError(f"x must be [L, hidden], got {tuple(x.shape)}")
    L, C = x.shape
    if wq.dim() != 2 or wq.shape[1] != C or wq.shape[0] % HEAD_DIM:
        raise ValueError(f"wq must be [H*{HEAD_DIM}, {C}], got {tuple(wq.shape)}")
    if tuple(wk.shape) != tuple(wq.shape) or tuple(wv.shape) != tuple(wq.shape):
        raise ValueError("wq, wk and wv must have the same shape")
    H = wq.shape[0] // HEAD_DIM
    if tuple(cos.shape) != (L, HEAD_DIM // 2) or tuple(sin.shape) != (L, HEAD_DIM // 2):
        raise ValueError(f"cos/sin must be [{L}, {HEAD_DIM // 2}]")
    if gamma_q.numel() != HEAD_DIM or gamma_k.numel() != HEAD_DIM:
        raise ValueError(f"gamma_q/gamma_k must have {HEAD_DIM} elements")
    v_shape = (H, L, HEAD_DIM) if ldv is None else (H, HEAD_DIM, ldv)
    if out is None:
        out = tuple(torch.empty(s, dtype=torch.bfloat16, device=x.device)
                    for s in ((H, L, HEAD_DIM), (H, L, HEAD_DIM), v_shape))
    for t, n, s in zip(out, "qkv", ((H, L, HEAD_DIM), (H, L, HEAD_DIM), v_shape)):
        if tuple(t.shape) != s:
            raise ValueError(f"out {n} must be {list(s)}")
    return H, L, C, out


def qkv_proj_qknorm_rope(x, wq, wk, wv, gamma_q, gamma_k, cos, sin, eps: float = 1e-6, out=None,
                         ldv: int | None = None):
    """The rank's qkv projection with QK-RMSNorm + RoPE fused behind it.

    x: bf16 [L, hidden]; wq, wk, wv: bf16 [H*128, hidden] (a contiguous row
    slice of the full weight is fine); gamma fp32 [128]; cos, sin fp32
    [L, 64].  Returns (q, k, v), bf16 [H, L, 128] each (or fills `out`, a
    (q, k, v) tuple of such tensors).  With ldv (a multiple of 8, >= L), v is
    written transposed as [H, 128, ldv] for attention_vt.
    """
    import torch
    H, L, C, out = _proj_shapes(x, wq, wk, wv, gamma_q, gamma_k, cos, sin, out, ldv)
    args = [_dev(x, torch.bfloat16, "x"), _dev(wq, torch.bfloat16, "wq"), _dev(wk, torch.bfloat16, "wk"),
            _dev(wv, torch.bfloat16, "wv"), _dev(gamma_q, torch.float32, "gamma_q"),
            _dev(gamma_k, torch.float32, "gamma_k"), _dev(cos, torch.float32, "cos"),
            _dev(sin, torch.float32, "sin"), _dev(out[0], torch.bfloat16, "q"), _dev(out[1], torch.bfloat16, "k"),
            _dev(out[2], torch.bfloat16, "v")]
    if ldv is None:
        _check("h3_qkv_proj_qknorm_rope", lib.h3_qkv_proj_qknorm_rope(
            *args, H, L, C, HEAD_DIM, float(eps), _stream()))
    else:
        _check("h3_qkv_proj_qknorm_rope_vt", lib.h3_qkv_proj_qknorm_rope_vt(
            *args, H, L, int(ldv), C, HEAD_DIM, float(eps), _stream()))
    return out


def qkv_proj_fp8_qknorm_rope(x, x_scale, wq, wk, wv, w_scale, gamma_q, gamma_k, cos, sin, eps: float = 1e-6,
                             out=None, ldv: int | None = None):
    """The fp8 form: x float8_e4m3fn [L, hidden] with x_scale (fp32 tensor of
    one element), wq/wk/wv float8_e4m3fn [H*128, hidden] with the weight's
    per-tensor w_scale.  Returns (q, k, v), bf16 [H, L, 128] each (v as
    [H, 128, ldv] when ldv is given)."""
    import torch
    f8 = torch.float8_e4m3fn
    if x_scale.numel() != 1 or w_scale.numel() != 1:
        raise ValueError("x_scale and w_scale must hold one element each")
    H, L, C, out = _proj_shapes(x, wq, wk, wv, gamma_q, gamma_k, cos, sin, out, ldv)
    args = [_dev(x, f8, "x"), _dev(x_scale, torch.float32, "x_scale"), _dev(wq, f8, "wq"), _dev(wk, f8, "wk"),
            _dev(wv, f8, "wv"), _dev(w_scale, torch.float32, "w_scale"), _dev(gamma_q, torch.float32, "gamma_q"),
            _dev(gamma_k, torch.float32, "gamma_k"), _dev(cos, torch.float32, "cos"),
            _dev(sin, torch.float32, "sin"), _dev(out[0], torch.bfloat16, "q"), _dev(out[1], torch.bfloat16, "k"),
            _dev(out[2], torch.bfloat16, "v")]
    if ldv is None:
        _check("h3_qkv_proj_fp8_qknorm_rope", lib.h3_qkv_proj_fp8_qknorm_rope(
            *args, H, L, C, HEAD_DIM, float(eps), _stream()))
    else:
        _check("h3_qkv_proj_fp8_qknorm_rope_vt", lib.h3_qkv_proj_fp8_qknorm_rope_vt(
            *args, H, L, int(ldv), C, HEAD_DIM, float(eps), _stream()))
    return out
