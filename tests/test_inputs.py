"""The seeded input generators: determinism, layout, shapes."""
import numpy as np

from exact_head_attention_amd import inputs as I


def test_positions_packed_layout():
    pos = I.packed_positions(31744, 1024)
    assert pos.dtype == np.int32 and pos.shape == (32768,)
    assert np.array_equal(pos[:31744], np.arange(31744))
    assert np.array_equal(pos[31744:], np.arange(1024))


def test_workload_shapes_match_the_rank_shares():
    assert I.WORKLOADS["ws8"].H * 8 == 56 and I.WORKLOADS["ws2"].H * 2 == 56
    assert I.WORKLOADS["ws1"].H == 56
    for w in I.WORKLOADS.values():
        assert w.n_video + w.n_audio == w.L and w.D == 128
    assert I.WORKLOADS["canvas128k"].qk_scale == 3.0
    assert I.WORKLOADS["odd37726"].L == 37726 and 37726 % 64 != 0


def test_make_inputs_deterministic_and_distributed():
    w = I.WORKLOADS["tiny"]
    a, b = I.make_inputs(w, seed=0), I.make_inputs(w, seed=0)
    c = I.make_inputs(w, seed=1)
    for key in ("q", "k", "v", "gamma_q", "gamma_k", "positions"):
        assert np.array_equal(a[key], b[key])
    assert not np.array_equal(a["q"], c["q"])
    assert a["q"].dtype == np.uint16 and a["q"].shape == (2, 512, 128)
    x = (a["v"].astype(np.uint32) << 16).view(np.float32)
    assert abs(float(x.mean())) < 0.02 and abs(float(x.std()) - 1.0) < 0.02
    assert abs(float(a["gamma_q"].mean()) - 1.0) < 0.05


def test_canvas_qk_scale():
    w = I.custom_workload(H=1, L=4096, n_audio=96, qk_scale=3.0)
    a = I.make_inputs(w, seed=0)
    x = (a["q"].astype(np.uint32) << 16).view(np.float32)
    assert abs(float(x.std()) - 3.0) < 0.1


def test_sample_rows_contains_boundaries():
    w = I.WORKLOADS["ws8"]
    r = I.sample_rows(w, head=3, n=4096)
    assert len(r) >= 4096 and np.all(np.diff(r) > 0)
    for b in (0, 31743, 31744, 32767):
        assert b in r
    assert np.array_equal(r, I.sample_rows(w, head=3, n=4096))
    assert not np.array_equal(r, I.sample_rows(w, head=4, n=4096))
    assert np.array_equal(I.sample_rows(I.WORKLOADS["tiny"], 0, 4096), np.arange(512))


def test_projection_inputs():
    w = I.PROJ_WORKLOADS["proj_tiny"]
    a, b = I.make_proj_inputs(w, seed=0), I.make_proj_inputs(w, seed=0)
    for key in ("x", "wq", "wk", "wv", "gamma_q", "gamma_k", "positions"):
        assert np.array_equal(a[key], b[key])
    assert a["x"].shape == (300, 512) and a["wq"].shape == (256, 512) and a["x"].dtype == np.uint16
    wf = (a["wv"].astype(np.uint32) << 16).view(np.float32)
    assert abs(float(wf.std()) * np.sqrt(512) - 1.0) < 0.05
    assert not np.array_equal(a["wq"], a["wk"])
    assert I.PROJ_WORKLOADS["proj_ws2"].hidden == 5376 and I.PROJ_WORKLOADS["proj_ws2"].H == 28
    assert I.PROJ_WORKLOADS["proj_ws2"].flops == 2.0 * 32768 * 3 * 28 * 128 * 5376


def test_projection_fp8_inputs():
    w = I.ProjWorkload("t8", H=1, L=64, n_video=64, n_audio=0, hidden=128, fp8=True)
    a = I.make_proj_inputs(w, seed=3)
    assert a["x"].dtype == np.uint8 and a["wq"].shape == (128, 128)
    import torch
    x = torch.from_numpy(a["x"]).view(torch.float8_e4m3fn).float().numpy() * a["x_scale"]
    assert abs(float(np.abs(x).max()) - 448.0 * float(a["x_scale"])) < 1e-6 * 448.0 * float(a["x_scale"]) * 4
    assert abs(float(x.std()) - 1.0) < 0.1
    b = I.make_proj_inputs(I.ProjWorkload("t16", H=1, L=64, n_video=64, n_audio=0, hidden=128), seed=3)
    xb = (b["x"].astype(np.uint32) << 16).view(np.float32)
    assert np.corrcoef(xb.ravel(), x.ravel())[0, 1] > 0.99   # same draws, two encodings
