"""The C ABI library loads, exports what include/h3attn.h declares, and rejects
invalid arguments before touching the GPU (no compute call needs a device)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "h3attn.h")


@pytest.fixture(scope="module")
def B():
    from exact_head_attention_amd import binding
    return binding


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(h3_[a-z_0-9]+)\s*\(", text)))


def test_header_declares_the_boundary():
    names = _declared_functions()
    for n in ("h3_qknorm_rope", "h3_attention", "h3_attention_vt", "h3_rope_tables", "h3_attention_lse",
              "h3_attention_merge", "h3_qkv_proj_qknorm_rope", "h3_qkv_proj_fp8_qknorm_rope",
              "h3_qkv_proj_qknorm_rope_vt", "h3_qkv_proj_fp8_qknorm_rope_vt", "h3_status_string",
              "h3_abi_version"):
        assert n in names


def test_library_exports_every_declared_symbol(B):
    for name in _declared_functions():
        assert hasattr(B.lib, name), name
    assert B.lib.h3_abi_version() == 1


def test_status_strings(B):
    for code in range(0, -8, -1):
        s = B.lib.h3_status_string(code)
        assert s and len(s) >= 2
    assert b"unknown" in B.lib.h3_status_string(42)


# Fake, never-dereferenced device addresses: validation rejects these calls
# before any HIP call is made.
A = 0x7F0000000000
MB = 1 << 20


def _attn(B, q=A, k=A + 64 * MB, v=A + 128 * MB, o=A + 192 * MB, H=2, L=512, D=128, scale=0.088):
    return B.lib.h3_attention(q, k, v, o, H, L, D, scale, None)


def _pro(B, q=A, k=A + 64 * MB, gq=A + 128 * MB, gk=A + 129 * MB, c=A + 130 * MB, s=A + 140 * MB,
         H=2, L=512, D=128, eps=1e-6):
    return B.lib.h3_qknorm_rope(q, k, gq, gk, c, s, H, L, D, eps, None)


def _tab(B, p=A, L=512, D=128, theta=10000.0, c=A + 1 * MB, s=A + 2 * MB):
    return B.lib.h3_rope_tables(p, L, D, theta, c, s, None)


def test_attention_argument_errors(B):
    assert _attn(B, q=None) == -1 and _attn(B, o=None) == -1
    assert _attn(B, H=0) == -2 and _attn(B, L=0) == -2 and _attn(B, L=-5) == -2
    assert _attn(B, H=1 << 16, L=1 << 16) == -2
    assert _attn(B, H=1, L=(1 << 23) + 1) == -2
    assert _attn(B, D=64) == -3 and _attn(B, D=129) == -3
    assert _attn(B, q=A + 8) == -4 and _attn(B, o=A + 192 * MB + 2) == -4
    assert _attn(B, o=A + 64 * MB + 16) == -5              # out overlaps k
    assert _attn(B, o=A) == -5                             # out is q
    assert _attn(B, scale=0.0) == -6 and _attn(B, scale=-1.0) == -6
    assert _attn(B, scale=float("inf")) == -6 and _attn(B, scale=float("nan")) == -6
    # scale * log2(e) must stay finite in fp32: 3e38 is a finite float whose
    # product with log2(e) is not; 2e38 still is.
    assert _attn(B, scale=3e38) == -6
    assert _attn(B, scale=2e38, o=A) == -5                 # passes the value check, fails later


def test_scale_range_is_shared_by_every_attention_call(B):
    assert _attn_vt(B, scale=3e38) == -6
    assert _lse(B, scale=3e38) == -6


def _attn_vt(B, q=A, k=A + 64 * MB, vt=A + 128 * MB, o=A + 192 * MB, H=2, L=512, ldv=512, D=128, scale=0.088):
    return B.lib.h3_attention_vt(q, k, vt, o, H, L, ldv, D, scale, None)


def test_attention_vt_argument_errors(B):
    assert _attn_vt(B, vt=None) == -1 and _attn_vt(B, k=None) == -1
    assert _attn_vt(B, H=0) == -2 and _attn_vt(B, L=0) == -2
    assert _attn_vt(B, ldv=504) == -2                      # ldv < L
    assert _attn_vt(B, ldv=(1 << 23) + 8) == -2            # a head's V^T past 2 GiB
    assert _attn_vt(B, D=64) == -3
    assert _attn_vt(B, ldv=516) == -4                      # rows not 16-byte aligned
    assert _attn_vt(B, vt=A + 128 * MB + 8) == -4
    assert _attn_vt(B, o=A + 128 * MB + 1024) == -5        # out inside vt
    assert _attn_vt(B, ldv=(1 << 17) + 8) == -5            # the longer vt rows reach out
    assert _attn_vt(B, scale=0.0) == -6 and _attn_vt(B, scale=float("nan")) == -6


def test_prologue_argument_errors(B):
    assert _pro(B, q=None) == -1 and _pro(B, s=None) == -1 and _pro(B, gk=None) == -1
    assert _pro(B, H=0) == -2 and _pro(B, L=0) == -2
    assert _pro(B, D=256) == -3
    assert _pro(B, c=A + 130 * MB + 4) == -4 and _pro(B, k=A + 64 * MB + 2) == -4
    assert _pro(B, k=A) == -5                               # q and k are one buffer
    assert _pro(B, c=A + 16) == -5                          # cos inside q
    assert _pro(B, eps=0.0) == -6 and _pro(B, eps=float("nan")) == -6 and _pro(B, eps=-1e-6) == -6


def test_rope_table_argument_errors(B):
    assert _tab(B, p=None) == -1 and _tab(B, c=None) == -1
    assert _tab(B, L=0) == -2
    assert _tab(B, D=96) == -3
    assert _tab(B, p=A + 2) == -4 and _tab(B, s=A + 2 * MB + 4) == -4
    assert _tab(B, s=A + 1 * MB + 64) == -5
    assert _tab(B, theta=1.0) == -6 and _tab(B, theta=float("inf")) == -6


def test_binding_rejects_cpu_tensors(B):
    import torch
    q = torch.zeros(1, 4, 128, dtype=torch.bfloat16)
    with pytest.raises(TypeError):
        B.attention(q, q, q)
    with pytest.raises(ValueError):
        B.attention(torch.zeros(1, 4, 64, dtype=torch.bfloat16), q, q)
    vt = torch.zeros(1, 128, 8, dtype=torch.bfloat16)
    with pytest.raises(TypeError):
        B.attention_vt(q, q, vt)
    with pytest.raises(ValueError):
        B.attention_vt(q, q, torch.zeros(1, 128, 2, dtype=torch.bfloat16))   # ldv < L
    with pytest.raises(ValueError):
        B.attention_vt(q, q, torch.zeros(2, 128, 8, dtype=torch.bfloat16))   # head count


def _lse(B, q=A, k=A + 64 * MB, v=A + 128 * MB, o=A + 192 * MB, lse=A + 320 * MB, H=2, Lq=512, Lk=256,
         stride=512 * 128, D=128, scale=0.088):
    return B.lib.h3_attention_lse(q, k, v, o, lse, H, Lq, Lk, stride, D, scale, None)


def _merge(B, outs=A, lses=A + 64 * MB, P=3, out=A + 128 * MB, lse_out=A + 192 * MB, H=2, L=512, D=128):
    return B.lib.h3_attention_merge(outs, lses, P, out, lse_out, H, L, D, None)


def test_attention_lse_argument_errors(B):
    assert _lse(B, q=None) == -1 and _lse(B, lse=None) == -1 and _lse(B, o=None) == -1
    assert _lse(B, H=0) == -2 and _lse(B, Lq=0) == -2 and _lse(B, Lk=0) == -2
    assert _lse(B, Lk=(1 << 23) + 1, stride=((1 << 23) + 1) * 128) == -2
    assert _lse(B, stride=255 * 128) == -2                 # head stride shorter than Lk rows
    assert _lse(B, D=64) == -3
    assert _lse(B, k=A + 64 * MB + 8) == -4 and _lse(B, lse=A + 320 * MB + 2) == -4
    assert _lse(B, stride=512 * 128 + 4) == -4             # head bases lose 16-byte alignment
    assert _lse(B, scale=0.0) == -6 and _lse(B, scale=float("nan")) == -6
    assert _lse(B, o=A + 64 * MB) == -5                    # out over k
    assert _lse(B, lse=A + 192 * MB + 16) == -5            # lse inside out


def test_attention_merge_argument_errors(B):
    assert _merge(B, outs=None) == -1 and _merge(B, out=None) == -1
    assert _merge(B, P=0) == -2 and _merge(B, H=0) == -2 and _merge(B, L=0) == -2
    assert _merge(B, D=256) == -3
    assert _merge(B, outs=A + 4) == -4 and _merge(B, lse_out=A + 192 * MB + 1) == -4
    assert _merge(B, out=A + 16) == -5                     # out inside outs
    assert _merge(B, lse_out=A + 128 * MB) == -5           # lse_out over out


def _qkv(B, x=A, wq=A + 1 * MB, wk=A + 2 * MB, wv=A + 3 * MB, gq=A + 4 * MB, gk=A + 5 * MB, c=A + 6 * MB,
         s=A + 7 * MB, q=A + 8 * MB, k=A + 9 * MB, v=A + 10 * MB, H=2, L=512, C=256, D=128, eps=1e-6):
    return B.lib.h3_qkv_proj_qknorm_rope(x, wq, wk, wv, gq, gk, c, s, q, k, v, H, L, C, D, eps, None)


def test_qkv_proj_argument_errors(B):
    assert _qkv(B, x=None) == -1 and _qkv(B, wv=None) == -1 and _qkv(B, v=None) == -1 and _qkv(B, s=None) == -1
    assert _qkv(B, H=0) == -2 and _qkv(B, L=0) == -2
    assert _qkv(B, C=0) == -2 and _qkv(B, C=48) == -2 and _qkv(B, C=(1 << 20) + 32) == -2
    assert _qkv(B, H=1 << 16, L=1 << 16) == -2
    assert _qkv(B, D=64) == -3
    assert _qkv(B, x=A + 8) == -4 and _qkv(B, gk=A + 5 * MB + 4) == -4 and _qkv(B, k=A + 9 * MB + 2) == -4
    assert _qkv(B, q=A + 16) == -5                         # q over x
    assert _qkv(B, v=A + 3 * MB) == -5                     # v over wv
    assert _qkv(B, k=A + 8 * MB + 64) == -5                # k inside q
    assert _qkv(B, q=A + 6 * MB) == -5                     # q over cos
    assert _qkv(B, eps=0.0) == -6 and _qkv(B, eps=float("inf")) == -6


def _qkv8(B, x=A, xs=A + 11 * MB, wq=A + 1 * MB, wk=A + 2 * MB, wv=A + 3 * MB, ws=A + 11 * MB + 64,
          gq=A + 4 * MB, gk=A + 5 * MB, c=A + 6 * MB, s=A + 7 * MB, q=A + 8 * MB, k=A + 9 * MB, v=A + 10 * MB,
          H=2, L=512, C=256, D=128, eps=1e-6):
    return B.lib.h3_qkv_proj_fp8_qknorm_rope(x, xs, wq, wk, wv, ws, gq, gk, c, s, q, k, v, H, L, C, D, eps, None)


def test_qkv_proj_fp8_argument_errors(B):
    assert _qkv8(B, xs=None) == -1 and _qkv8(B, ws=None) == -1 and _qkv8(B, x=None) == -1
    assert _qkv8(B, C=32) == -2 and _qkv8(B, C=96) == -2 and _qkv8(B, L=0) == -2
    assert _qkv8(B, D=256) == -3
    assert _qkv8(B, xs=A + 11 * MB + 2) == -4 and _qkv8(B, wq=A + 1 * MB + 8) == -4
    assert _qkv8(B, q=A + 11 * MB - 16) == -5               # q's end covers x_scale
    assert _qkv8(B, v=A + 10 * MB, k=A + 10 * MB + 4096) == -5
    assert _qkv8(B, eps=-1.0) == -6


def _qkv_vt(B, x=A, wq=A + 1 * MB, wk=A + 2 * MB, wv=A + 3 * MB, gq=A + 4 * MB, gk=A + 5 * MB, c=A + 6 * MB,
            s=A + 7 * MB, q=A + 8 * MB, k=A + 9 * MB, v=A + 10 * MB, H=2, L=512, ldv=512, C=256, D=128, eps=1e-6):
    return B.lib.h3_qkv_proj_qknorm_rope_vt(x, wq, wk, wv, gq, gk, c, s, q, k, v, H, L, ldv, C, D, eps, None)


def _qkv8_vt(B, x=A, xs=A + 11 * MB, wq=A + 1 * MB, wk=A + 2 * MB, wv=A + 3 * MB, ws=A + 11 * MB + 64,
             gq=A + 4 * MB, gk=A + 5 * MB, c=A + 6 * MB, s=A + 7 * MB, q=A + 8 * MB, k=A + 9 * MB, v=A + 10 * MB,
             H=2, L=512, ldv=512, C=256, D=128, eps=1e-6):
    return B.lib.h3_qkv_proj_fp8_qknorm_rope_vt(x, xs, wq, wk, wv, ws, gq, gk, c, s, q, k, v, H, L, ldv, C, D, eps,
                                                None)


def test_qkv_proj_vt_argument_errors(B):
    assert _qkv_vt(B, v=None) == -1 and _qkv_vt(B, x=None) == -1
    assert _qkv_vt(B, ldv=0) == -2 and _qkv_vt(B, ldv=504) == -2 and _qkv_vt(B, ldv=(1 << 23) + 8) == -2
    assert _qkv_vt(B, C=48) == -2
    assert _qkv_vt(B, ldv=524) == -4                       # rows not 16-byte aligned
    assert _qkv_vt(B, ldv=4096, q=A + 11 * MB) == -5       # 2 MB of vt rows reach q
    assert _qkv_vt(B, eps=0.0) == -6
    assert _qkv8_vt(B, xs=None) == -1 and _qkv8_vt(B, v=None) == -1
    assert _qkv8_vt(B, ldv=8) == -2 and _qkv8_vt(B, C=96) == -2
    assert _qkv8_vt(B, ldv=514) == -4
    assert _qkv8_vt(B, ldv=8192) == -5                     # 4 MB of vt rows reach x_scale
    assert _qkv8_vt(B, eps=float("nan")) == -6
