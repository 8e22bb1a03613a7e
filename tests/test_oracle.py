"""Pins of the fp64 oracle against facts that do not come from the oracle.

Each test names the kind of pin: an exhaustive check, a hand-derived fixture
(tests/golden), a closed form, an invariant, a special case that reduces to a
textbook value, brute force with pure-Python loops, or a library routine.
"""
import math
import os

import numpy as np
import pytest
import torch

import oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
RTOL = 1e-12


def _bits_of(vals64):
    return O.f64_to_bf16_bits(np.asarray(vals64, dtype=np.float64))


# ---------------------------------------------------------------- bf16 codec


def test_bf16_roundtrip_exhaustive():
    """Exhaustive: every finite bf16 pattern decodes and re-encodes to itself;
    every NaN pattern encodes to a NaN."""
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    with np.errstate(invalid="ignore"):   # casting the signalling-NaN patterns
        x = O.bf16_to_f64(bits)
        back = O.f64_to_bf16_bits(x)
        finite = np.isfinite(x) | np.isinf(x)
        assert np.array_equal(back[finite], bits[finite])
        nan_back = O.bf16_to_f64(back[~finite])
    assert np.all(np.isnan(nan_back))


def test_bf16_decode_known_values():
    """Closed form: decoding follows the binary32 layout."""
    assert O.bf16_to_f64(np.array([0x3F80], np.uint16))[0] == 1.0
    assert O.bf16_to_f64(np.array([0xC040], np.uint16))[0] == -3.0
    assert O.bf16_to_f64(np.array([0x0001], np.uint16))[0] == 2.0 ** -133
    assert O.bf16_to_f64(np.array([0x7F7F], np.uint16))[0] == 255 * 2.0 ** 120


def test_bf16_rne_golden_cases():
    """Hand-derived fixture: halfway cases, overflow, subnormals, and a value
    where rounding through fp32 first would give a different answer."""
    path = os.path.join(GOLDEN, "bf16_rne_cases.txt")
    n = 0
    with open(path) as f:
        for line in f:
            if not line.strip() or line.startswith("#"):
                continue
            expr, hexbits, _why = [p.strip() for p in line.split(";", 2)]
            val = eval(expr, {"__builtins__": {}})  # fixture holds arithmetic literals only
            got = int(_bits_of([val])[0])
            assert got == int(hexbits, 16), (expr, hex(got), hexbits)
            n += 1
    assert n >= 10


def test_bf16_rne_matches_torch_on_fp32_values():
    """Library: fp32 -> fp64 is exact, so for fp32 inputs the one-step RNE must
    equal PyTorch's fp32 -> bf16 conversion (also RNE)."""
    rng = np.random.default_rng(7)
    x32 = np.concatenate([
        rng.standard_normal(200000).astype(np.float32) * np.float32(50.0),
        rng.integers(0, 1 << 32, size=200000, dtype=np.uint64).astype(np.uint32).view(np.float32),
    ])
    x32 = x32[np.isfinite(x32)]
    ours = O.f64_to_bf16_bits(x32.astype(np.float64))
    theirs = torch.from_numpy(x32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, theirs)


# ------------------------------------------------------------ rotary tables


def test_rope_table_special_columns():
    """Closed form: with theta=10000 and D=128, inv_freq for pairs 0, 16, 32, 48
    is exactly 1, 1/10, 1/100, 1/1000 (10000^(-2j/128) at j = 0, 16, 32, 48),
    so those columns hold cos/sin of p, p/10, p/100, p/1000."""
    pos = np.array([0, 1, 7, 100, 31743, 126975], dtype=np.int32)
    c, s = O.rope_tables(pos, 128, 10000.0)
    assert c.shape == (6, 64) and c.dtype == np.float32
    for col, div in ((0, 1.0), (16, 10.0), (32, 100.0), (48, 1000.0)):
        for r, p in enumerate(pos):
            a = float(p) / div
            assert abs(float(c[r, col]) - math.cos(a)) <= 2e-7 * max(1.0, abs(math.cos(a))) + 1e-9
            assert abs(float(s[r, col]) - math.sin(a)) <= 2e-7 * max(1.0, abs(math.sin(a))) + 1e-9


def test_rope_table_position_zero_and_monotone_frequencies():
    """Closed form: position 0 gives cos 1, sin 0 exactly in every column; at
    position 1 the angles theta^(-2j/D) fall strictly with j from 1 to 10^-4 * 10^(4/64)."""
    c, s = O.rope_tables(np.array([0, 1], np.int32), 128, 10000.0)
    assert np.all(c[0] == 1.0) and np.all(s[0] == 0.0)
    ang = np.arcsin(s[1].astype(np.float64))       # angles < pi/2 at p = 1
    assert np.all(np.diff(ang) < 0)
    assert abs(ang[63] - 10000.0 ** (-126 / 128)) < 1e-7


# -------------------------------------------------------------- QK-RMSNorm


def test_rmsnorm_constant_vector():
    """Closed form: x = c*1 gives y = gamma * c / sqrt(c^2 + eps)."""
    g = 1.0 + 0.1 * np.random.default_rng(1).standard_normal(128)
    for c, eps in ((0.75, 1e-6), (-3.0, 0.5), (1e-3, 1e-6)):
        y = O.rms_norm(np.full(128, c), g, eps)
        np.testing.assert_allclose(y, g * c / math.sqrt(c * c + eps), rtol=RTOL)


def test_rmsnorm_one_hot():
    """Closed form: x = a*e_d gives y_d = a*gamma_d / sqrt(a^2/128 + eps), 0 elsewhere."""
    g = np.linspace(0.5, 1.5, 128)
    a, eps, d = 2.5, 1e-3, 37
    x = np.zeros(128)
    x[d] = a
    y = O.rms_norm(x, g, eps)
    expect = np.zeros(128)
    expect[d] = a * g[d] / math.sqrt(a * a / 128 + eps)
    np.testing.assert_allclose(y, expect, rtol=RTOL, atol=0)


def test_rmsnorm_zero_and_scale_invariance():
    """Invariants: x = 0 gives 0; with eps = 0 RMSNorm(alpha x) = RMSNorm(x) for
    alpha > 0, and the output's RMS over gamma = 1 is exactly 1."""
    assert np.all(O.rms_norm(np.zeros((3, 128)), np.ones(128), 1e-6) == 0.0)
    x = np.random.default_rng(2).standard_normal((5, 128))
    g = np.ones(128)
    y1 = O.rms_norm(x, g, 0.0)
    np.testing.assert_allclose(O.rms_norm(7.5 * x, g, 0.0), y1, rtol=RTOL)
    np.testing.assert_allclose(np.sqrt(np.mean(y1 * y1, axis=-1)), 1.0, rtol=RTOL)


# ------------------------------------------------------------------- RoPE


def _rot_tables(angles):
    a = np.asarray(angles, dtype=np.float64)
    return np.cos(a), np.sin(a)


def test_rope_one_hot_closed_form():
    """Closed form: e_0 rotates into (cos t, sin t) on dims (0, 1); e_1 into
    (-sin t, cos t).  Pins the adjacent-pair convention and the sign."""
    t = np.linspace(0.1, 1.0, 64)
    c, s = _rot_tables(t)
    e0 = np.zeros(128)
    e0[0] = 1.0
    y = O.rope_rotate(e0, c, s)
    assert y[0] == pytest.approx(math.cos(t[0]), rel=RTOL)
    assert y[1] == pytest.approx(math.sin(t[0]), rel=RTOL)
    assert np.all(y[2:] == 0.0)
    e1 = np.zeros(128)
    e1[1] = 1.0
    y = O.rope_rotate(e1, c, s)
    assert y[0] == pytest.approx(-math.sin(t[0]), rel=RTOL)
    assert y[1] == pytest.approx(math.cos(t[0]), rel=RTOL)
    e126 = np.zeros(128)
    e126[126] = 1.0
    y = O.rope_rotate(e126, c, s)
    assert y[126] == pytest.approx(math.cos(t[63]), rel=RTOL)
    assert y[127] == pytest.approx(math.sin(t[63]), rel=RTOL)


def test_rope_position_zero_identity_and_norm():
    """Invariants: the position-0 table is the identity (exactly); each pair's
    2-norm is preserved at any position."""
    x = np.random.default_rng(3).standard_normal((4, 128))
    c0, s0 = O.rope_tables(np.zeros(4, np.int32))
    assert np.array_equal(O.rope_rotate(x, c0, s0), x)
    c, s = O.rope_tables(np.array([5, 999, 31000, 77], np.int32))
    y = O.rope_rotate(x, c, s)
    n_in = x[:, 0::2] ** 2 + x[:, 1::2] ** 2
    n_out = y[:, 0::2] ** 2 + y[:, 1::2] ** 2
    np.testing.assert_allclose(n_out, n_in, rtol=1e-6)  # fp32 tables: cos^2+sin^2 = 1 +- 1e-7


def test_rope_relative_position_and_composition():
    """Invariants: <R_m q, R_n k> depends only on m - n, and R_a R_b = R_{a+b}
    (with fp64 angle tables, so only fp64 rounding remains)."""
    rng = np.random.default_rng(4)
    q, k = rng.standard_normal(128), rng.standard_normal(128)
    inv = 10000.0 ** (-2.0 * np.arange(64) / 128)

    def R(p, x):
        c, s = _rot_tables(p * inv)
        return O.rope_rotate(x, c, s)

    base = float(R(40, q) @ R(13, k))
    for t in (1, 250, 9000):
        assert float(R(40 + t, q) @ R(13 + t, k)) == pytest.approx(base, rel=1e-9, abs=1e-9)
    np.testing.assert_allclose(R(17, R(25, q)), R(42, q), rtol=1e-9, atol=1e-12)


def test_qknorm_rope_fused_order_and_single_rounding():
    """Special case: a one-hot bf16 input at position p with eps = 0 gives
    RMSNorm value a*gamma_0/sqrt(a^2/128) = sqrt(128)*gamma_0 on dim 0, which
    RoPE at pair 0 (angle p) sends to (sqrt(128) g0 cos p, sqrt(128) g0 sin p);
    the stored bits are the single RNE of those fp64 values."""
    H, L, D = 1, 3, 128
    x = np.zeros((H, L, D), np.float64)
    x[0, :, 0] = 3.0
    xb = O.f64_to_bf16_bits(x)
    g = np.full(D, 1.25, np.float32)
    pos = np.array([0, 1, 2], np.int32)
    c, s = O.rope_tables(pos)
    y, yb = O.qknorm_rope(xb, g, c, s, 0.0)
    for i, p in enumerate(pos):
        a = math.sqrt(128) * 1.25
        assert y[0, i, 0] == pytest.approx(a * float(c[i, 0]), rel=RTOL)
        assert y[0, i, 1] == pytest.approx(a * float(s[i, 0]), rel=RTOL)
        assert abs(float(c[i, 0]) - math.cos(p)) < 1e-7
    assert np.array_equal(yb, O.f64_to_bf16_bits(y))


def test_packed_restart_gives_identical_prologue():
    """Invariant: an audio token whose content equals a video token's at the
    same position index gets the identical prologue output (positions restart
    for the audio segment)."""
    from exact_head_attention_amd.inputs import packed_positions
    pos = packed_positions(6, 3)                  # 0..5 then 0..2
    rng = np.random.default_rng(5)
    x = O.f64_to_bf16_bits(rng.standard_normal((2, 9, 128)))
    x[:, 6:9] = x[:, 0:3]
    g = (1 + 0.1 * rng.standard_normal(128)).astype(np.float32)
    c, s = O.rope_tables(pos)
    _, yb = O.qknorm_rope(x, g, c, s, 1e-6)
    assert np.array_equal(yb[:, 6:9], yb[:, 0:3])
    assert not np.array_equal(yb[:, 3:6], yb[:, 0:3])


# -------------------------------------------------------------- attention


def _brute_attention(q, k, v, scale):
    """Pure-Python loops with the math module."""
    out = []
    for qi in q:
        logits = [scale * sum(a * b for a, b in zip(qi, kj)) for kj in k]
        m = max(logits)
        w = [math.exp(s - m) for s in logits]
        z = sum(w)
        out.append([sum(wj * vj[d] for wj, vj in zip(w, v)) / z for d in range(len(v[0]))])
    return np.array(out)


def test_attention_brute_force_small():
    """Brute force: H=1, L<=8, D=4 against pure-Python loops (R != L query rows
    catch a transposed q k^T)."""
    rng = np.random.default_rng(6)
    for L in (1, 2, 5, 8):
        q = rng.standard_normal((3, 4))
        k = rng.standard_normal((L, 4))
        v = rng.standard_normal((L, 4))
        got = O.attention_head(q, k, v, 0.7)
        np.testing.assert_allclose(got, _brute_attention(q.tolist(), k.tolist(), v.tolist(), 0.7),
                                   rtol=1e-12, atol=1e-14)


def test_attention_vs_torch_sdpa():
    """Library: torch's CPU fp64 scaled_dot_product_attention."""
    rng = np.random.default_rng(8)
    q = rng.standard_normal((2, 64, 128))
    k = rng.standard_normal((2, 200, 128))
    v = rng.standard_normal((2, 200, 128))
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q)[None], torch.from_numpy(k)[None], torch.from_numpy(v)[None],
        scale=1 / math.sqrt(128)).numpy()[0]
    for h in range(2):
        np.testing.assert_allclose(O.attention_head(q[h], k[h], v[h], 1 / math.sqrt(128)), ref[h],
                                   rtol=1e-10, atol=1e-12)


def test_attention_golden_two_keys():
    """Hand-derived fixture: two keys, the softmax is the logistic function."""
    with open(os.path.join(GOLDEN, "attention_two_keys.txt")) as f:
        rows = [ln for ln in f if ln.strip() and not ln.startswith("#")]
    for ln in rows:
        qs, ks, vs, sc, outs = [np.array(p.split(), dtype=np.float64) for p in ln.split(";")]
        got = O.attention_head(qs.reshape(1, 2), ks.reshape(2, 2), vs.reshape(2, 2), float(sc[0]))
        np.testing.assert_allclose(got[0], outs, rtol=1e-15)


def _bf16_tensor(rng, shape, mult=1.0):
    return O.f64_to_bf16_bits(mult * rng.standard_normal(shape))


def test_attention_weights_sum_to_one_and_convexity():
    """Invariant: rows of P are nonnegative and sum to 1, so V rows all equal c
    give O = c, and every output lies inside the V columns' [min, max]."""
    rng = np.random.default_rng(9)
    q, k = rng.standard_normal((16, 128)), rng.standard_normal((300, 128))
    v = np.tile(rng.standard_normal(128), (300, 1))
    np.testing.assert_allclose(O.attention_head(q, k, v, 0.3), v[:16], rtol=1e-13)
    v = rng.standard_normal((300, 128))
    o = O.attention_head(q, k, v, 0.3)
    assert np.all(o <= v.max(axis=0) + 1e-12) and np.all(o >= v.min(axis=0) - 1e-12)
    ones = O.attention_head(q, k, np.ones((300, 1)), 0.3)
    np.testing.assert_allclose(ones, 1.0, rtol=1e-13)


def test_attention_single_key_returns_its_value():
    """Special case: L = 1 returns that V row exactly, for any q."""
    rng = np.random.default_rng(10)
    k, v = rng.standard_normal((1, 128)), rng.standard_normal((1, 128))
    o = O.attention_head(rng.standard_normal((5, 128)) * 30, k, v, 1 / math.sqrt(128))
    assert np.array_equal(o, np.tile(v, (5, 1)))


def test_attention_identical_keys_and_zero_scale_give_mean():
    """Special cases: all keys identical, or scale = 0, give the mean of V."""
    rng = np.random.default_rng(11)
    q = rng.standard_normal((4, 128))
    v = rng.standard_normal((77, 128))
    k_same = np.tile(rng.standard_normal(128), (77, 1))
    np.testing.assert_allclose(O.attention_head(q, k_same, v, 1.0), np.tile(v.mean(0), (4, 1)), rtol=1e-12, atol=1e-14)
    k = rng.standard_normal((77, 128))
    np.testing.assert_allclose(O.attention_head(q, k, v, 0.0), np.tile(v.mean(0), (4, 1)), rtol=1e-12, atol=1e-14)


def test_attention_dominant_key():
    """Special case: one key whose logit exceeds every other by > 800 returns its
    V row exactly (every other exp underflows to 0 in fp64)."""
    rng = np.random.default_rng(12)
    k = rng.standard_normal((50, 128)) * 0.01
    q = np.zeros((1, 128))
    q[0, 0] = 1.0
    k[17, 0] = 1000.0
    v = rng.standard_normal((50, 128))
    o = O.attention_head(q, k, v, 1.0)
    assert np.array_equal(o[0], v[17])


def test_attention_permutation_invariance():
    """Invariant: permuting keys and values together leaves O unchanged;
    permuting query rows permutes O's rows."""
    rng = np.random.default_rng(13)
    qb, kb, vb = (_bf16_tensor(rng, (1, 96, 128)) for _ in range(3))
    o = O.attention(qb, kb, vb, 1 / math.sqrt(128))
    perm = rng.permutation(96)
    o2 = O.attention(qb, kb[:, perm], vb[:, perm], 1 / math.sqrt(128))
    np.testing.assert_allclose(o2, o, rtol=1e-12, atol=1e-14)
    o3 = O.attention(qb[:, perm], kb, vb, 1 / math.sqrt(128))
    np.testing.assert_allclose(o3, o[:, perm], rtol=1e-12, atol=1e-14)


def test_attention_heads_independent_and_rows_subset():
    """Invariant: heads are independent (perturbing head 1 leaves head 0 bit-
    identical; one call over 3 heads equals three calls over one), and a row
    subset equals those rows of the full result."""
    rng = np.random.default_rng(14)
    qb, kb, vb = (_bf16_tensor(rng, (3, 80, 128)) for _ in range(3))
    s = 1 / math.sqrt(128)
    o = O.attention(qb, kb, vb, s)
    for h in range(3):
        assert np.array_equal(O.attention(qb[h:h + 1], kb[h:h + 1], vb[h:h + 1], s)[0], o[h])
    kb2 = kb.copy()
    kb2[1] ^= np.uint16(0x0001)
    o2 = O.attention(qb, kb2, vb, s)
    assert np.array_equal(o2[0], o[0]) and np.array_equal(o2[2], o[2])
    assert not np.array_equal(o2[1], o[1])
    rows = [np.array([0, 5, 79]), np.array([1, 2, 3]), np.array([79, 40, 0])]
    osub = O.attention(qb, kb, vb, s, rows=rows)
    for h in range(3):
        assert np.array_equal(osub[h], o[h][rows[h]])


def test_attention_block_size_does_not_change_rows():
    """Invariant: the row blocking is only a memory bound (rows are independent)."""
    rng = np.random.default_rng(15)
    q, k, v = rng.standard_normal((70, 128)), rng.standard_normal((90, 128)), rng.standard_normal((90, 128))
    a = O.attention_head(q, k, v, 0.1, block=256)
    b = O.attention_head(q, k, v, 0.1, block=7)
    np.testing.assert_allclose(a, b, rtol=1e-13, atol=1e-15)


# ------------------------------------------------ log-sum-exp and merging


def test_lse_closed_forms():
    """Closed forms: one key gives lse = scale*<q,k>; L identical keys give
    scale*<q,k> + ln L; the output part equals attention_head's."""
    rng = np.random.default_rng(20)
    q, k1 = rng.standard_normal((3, 128)), rng.standard_normal((1, 128))
    v1 = rng.standard_normal((1, 128))
    out, lse = O.attention_lse_head(q, k1, v1, 0.3)
    np.testing.assert_allclose(lse, 0.3 * (q @ k1[0]), rtol=1e-13)
    assert np.array_equal(out, np.tile(v1, (3, 1)))
    kk = np.tile(k1, (50, 1))
    _, lse50 = O.attention_lse_head(q, kk, rng.standard_normal((50, 128)), 0.3)
    np.testing.assert_allclose(lse50, 0.3 * (q @ k1[0]) + math.log(50), rtol=1e-13)
    k, v = rng.standard_normal((77, 128)), rng.standard_normal((77, 128))
    out, _ = O.attention_lse_head(q, k, v, 0.1)
    np.testing.assert_allclose(out, O.attention_head(q, k, v, 0.1), rtol=1e-13, atol=1e-15)


def test_lse_vs_scipy_logsumexp():
    """Library: scipy.special.logsumexp of the scaled scores, including logits
    large enough that an unshifted exp would overflow."""
    from scipy.special import logsumexp
    rng = np.random.default_rng(21)
    q, k = rng.standard_normal((9, 128)) * 40, rng.standard_normal((300, 128)) * 40
    _, lse = O.attention_lse_head(q, k, rng.standard_normal((300, 128)), 1 / math.sqrt(128))
    np.testing.assert_allclose(lse, logsumexp(q @ k.T / math.sqrt(128), axis=1), rtol=1e-12)


def test_merge_of_split_equals_unsplit():
    """Invariant: attention over keys split into ranges, merged, equals the
    attention over all keys (outputs and lse), for uneven splits."""
    rng = np.random.default_rng(22)
    q, k, v = rng.standard_normal((40, 128)), rng.standard_normal((500, 128)), rng.standard_normal((500, 128))
    s = 1 / math.sqrt(128)
    full, lse_full = O.attention_lse_head(q, k, v, s)
    cuts = [0, 7, 200, 201, 500]
    parts = [O.attention_lse_head(q, k[a:b], v[a:b], s) for a, b in zip(cuts, cuts[1:])]
    out, lse = O.merge_partials(np.stack([p[0] for p in parts]), np.stack([p[1] for p in parts]))
    np.testing.assert_allclose(out, full, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(lse, lse_full, rtol=1e-13)


def test_merge_single_part_and_empty_part():
    """Special cases: one part is returned unchanged; a part with lse = -inf
    (no keys) contributes nothing."""
    rng = np.random.default_rng(23)
    o1, l1 = rng.standard_normal((2, 5, 128)), rng.standard_normal((2, 5))
    out, lse = O.merge_partials(o1[None], l1[None])
    np.testing.assert_allclose(out, o1, rtol=1e-15)
    np.testing.assert_allclose(lse, l1, rtol=1e-15)
    out2, lse2 = O.merge_partials(np.stack([o1, rng.standard_normal((2, 5, 128))]),
                                  np.stack([l1, np.full((2, 5), -np.inf)]))
    np.testing.assert_allclose(out2, o1, rtol=1e-15)
    np.testing.assert_allclose(lse2, l1, rtol=1e-15)


# ------------------------------------------- qkv projection + fused prologue


def _rand_bits(rng, shape, std=1.0):
    return _bits_of(std * rng.standard_normal(shape))


def test_qkv_project_brute_force():
    """Brute force with pure-Python loops: y[t, f] = sum_c x[t, c] w[f, c]."""
    rng = np.random.default_rng(11)
    x, w = _rand_bits(rng, (3, 7)), _rand_bits(rng, (5, 7))
    xf, wf = O.bf16_to_f64(x), O.bf16_to_f64(w)
    y = O.qkv_project(x, w)
    assert y.shape == (3, 5)
    for t in range(3):
        for f in range(5):
            ref = 0.0
            for c in range(7):
                ref += float(xf[t, c]) * float(wf[f, c])
            assert abs(y[t, f] - ref) <= 1e-14 * (1 + abs(ref))


def test_qkv_split_heads_element_definition():
    """Brute force on a few elements: head h, dim d of v is feature h*D + d of
    the projection, for token t (the head split's reading)."""
    rng = np.random.default_rng(12)
    H, D, L, C = 2, 128, 5, 40
    x, wv = _rand_bits(rng, (L, C)), _rand_bits(rng, (H * D, C), 0.2)
    wq = wk = _rand_bits(rng, (H * D, C), 0.2)
    cos, sin = O.rope_tables(np.arange(L), D)
    v = O.qkv_proj_qknorm_rope(x, wq, wk, wv, np.ones(D, np.float32), np.ones(D, np.float32),
                               cos, sin, 1e-6, H)["v"][0]
    xf, wf = O.bf16_to_f64(x), O.bf16_to_f64(wv)
    for h, t, d in ((0, 0, 0), (1, 4, 127), (1, 2, 5), (0, 3, 64)):
        ref = sum(float(xf[t, c]) * float(wf[h * D + d, c]) for c in range(C))
        assert abs(v[h, t, d] - ref) <= 1e-14 * (1 + abs(ref))


def test_qkv_one_hot_weights_reduce_to_the_prologue():
    """Special case: one-hot weight rows select hidden columns exactly, so the
    fused chain must equal the (separately pinned) prologue applied to those
    columns, bit for bit, and v must be the selected columns themselves."""
    rng = np.random.default_rng(13)
    H, D, L, C = 2, 128, 37, 3 * 2 * 128 + 20
    x = _rand_bits(rng, (L, C))
    perm = rng.permutation(C)
    sel = {n: perm[i * H * D:(i + 1) * H * D] for i, n in enumerate("qkv")}
    one = O.f64_to_bf16_bits(np.array([1.0]))[0]

    def onehot(cols):
        w = np.zeros((len(cols), C), np.uint16)
        w[np.arange(len(cols)), cols] = one
        return w

    gq = (1 + 0.1 * rng.standard_normal(D)).astype(np.float32)
    gk = (1 + 0.1 * rng.standard_normal(D)).astype(np.float32)
    cos, sin = O.rope_tables(np.arange(L), D)
    res = O.qkv_proj_qknorm_rope(x, onehot(sel["q"]), onehot(sel["k"]), onehot(sel["v"]), gq, gk,
                                 cos, sin, 1e-6, H)
    for n, g in (("q", gq), ("k", gk)):
        cols = x[:, sel[n]].reshape(L, H, D).transpose(1, 0, 2)
        y_ref, b_ref = O.qknorm_rope(cols, g, cos, sin, 1e-6)
        assert np.array_equal(res[n][1], b_ref)
        np.testing.assert_allclose(res[n][0], y_ref, rtol=1e-13, atol=1e-13)
    assert np.array_equal(res["v"][1], x[:, sel["v"]].reshape(L, H, D).transpose(1, 0, 2))


def test_qkv_norm_removes_weight_scale_but_v_keeps_it():
    """Invariant: RMSNorm(2y) = RMSNorm(y) up to eps, so doubling the weights
    (exact in bf16) leaves q and k unchanged and doubles v exactly."""
    rng = np.random.default_rng(14)
    H, D, L, C = 1, 128, 9, 64
    x = _rand_bits(rng, (L, C))
    w = {n: _rand_bits(rng, (H * D, C), 0.3) for n in "qkv"}
    w2 = {n: O.f64_to_bf16_bits(2 * O.bf16_to_f64(b)) for n, b in w.items()}
    g = (1 + 0.1 * rng.standard_normal(D)).astype(np.float32)
    cos, sin = O.rope_tables(np.arange(L), D)
    a = O.qkv_proj_qknorm_rope(x, w["q"], w["k"], w["v"], g, g, cos, sin, 1e-12, H)
    b = O.qkv_proj_qknorm_rope(x, w2["q"], w2["k"], w2["v"], g, g, cos, sin, 1e-12, H)
    for n in "qk":
        np.testing.assert_allclose(b[n][0], a[n][0], rtol=1e-9, atol=1e-12)
    assert np.array_equal(b["v"][0], 2 * a["v"][0])


def test_qkv_head_permutation_equivariance():
    """Invariant: swapping the two heads' weight row blocks swaps the output
    heads (norm and rotation act per head with shared gamma and tables)."""
    rng = np.random.default_rng(15)
    H, D, L, C = 2, 128, 6, 48
    x = _rand_bits(rng, (L, C))
    w = {n: _rand_bits(rng, (H * D, C), 0.3) for n in "qkv"}
    sw = {n: np.concatenate([b[D:], b[:D]]) for n, b in w.items()}
    g = (1 + 0.1 * rng.standard_normal(D)).astype(np.float32)
    cos, sin = O.rope_tables(np.arange(L) * 7, D)
    a = O.qkv_proj_qknorm_rope(x, w["q"], w["k"], w["v"], g, g, cos, sin, 1e-6, H)
    b = O.qkv_proj_qknorm_rope(x, sw["q"], sw["k"], sw["v"], g, g, cos, sin, 1e-6, H)
    for n in "qkv":
        assert np.array_equal(b[n][1], a[n][1][::-1])


# ---------------------------------------------------------------- fp8 e4m3


def test_e4m3_known_codes():
    """Closed form: the OCP e4m3 encoding's landmark codes."""
    vals = O.e4m3_to_f64(np.array([0x00, 0x80, 0x38, 0xB8, 0x7E, 0x08, 0x07, 0x01, 0x40, 0x3C], np.uint8))
    assert vals[0] == 0.0 and vals[1] == 0.0 and math.copysign(1, vals[1]) == -1
    assert vals[2] == 1.0 and vals[3] == -1.0
    assert vals[4] == 448.0                        # largest finite
    assert vals[5] == 2.0 ** -6                    # smallest normal
    assert vals[6] == 7 / 8 * 2.0 ** -6 and vals[7] == 2.0 ** -9   # subnormals
    assert vals[8] == 2.0 and vals[9] == 1.5
    assert np.isnan(O.e4m3_to_f64(np.array([0x7F, 0xFF], np.uint8))).all()


def test_e4m3_matches_torch_exhaustive():
    """Library routine, all 256 codes: torch's float8_e4m3fn decoding."""
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = O.e4m3_to_f64(codes)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])


def test_fp8_projection_brute_force_and_scales():
    """Brute force with loops on a tiny case: v = x_scale * w_scale *
    sum_c x[t, c] w[f, c]; q and k equal the bf16 form's prologue applied to
    the same (exactly representable) projection."""
    rng = np.random.default_rng(21)
    H, D, L, C = 1, 128, 3, 8
    x8 = rng.integers(0, 256, (L, C), dtype=np.uint8)
    x8[(x8 & 0x7F) == 0x7F] = 0x38                 # no NaN codes
    w8 = {n: rng.integers(0, 256, (H * D, C), dtype=np.uint8) for n in "qkv"}
    for n in w8:
        w8[n][(w8[n] & 0x7F) == 0x7F] = 0x30
    sx, sw = 0.375, 1.0 / 64
    g = (1 + 0.1 * rng.standard_normal(D)).astype(np.float32)
    cos, sin = O.rope_tables(np.arange(L), D)
    res = O.qkv_proj_fp8_qknorm_rope(x8, sx, w8["q"], w8["k"], w8["v"], sw, g, g, cos, sin, 1e-6, H)
    xf, wf = O.e4m3_to_f64(x8), O.e4m3_to_f64(w8["v"])
    for t in range(L):
        for f in (0, 5, 127):
            ref = 0.0
            for c in range(C):
                ref += float(xf[t, c]) * float(wf[f, c])
            assert abs(res["v"][0][0, t, f] - sx * sw * ref) <= 1e-12 * (1 + abs(sx * sw * ref))
    yq = sx * sw * (xf @ O.e4m3_to_f64(w8["q"]).T)
    ref_q = O.rope_rotate(O.rms_norm(yq.reshape(L, H, D).transpose(1, 0, 2), g, 1e-6), cos[None], sin[None])
    np.testing.assert_allclose(res["q"][0], ref_q, rtol=1e-12, atol=1e-12)
