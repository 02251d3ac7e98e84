"""GPU parity: the HIP path (through the C ABI) against the CPU oracle.

Bars:
  * Q_W, s_W, Q_X, s_X, A and the W8A8 output Y: bit-exact.  The library
    computes the rotations exactly and takes every rounding decision in the
    same fp32 operations as the oracle, so no allowance at rounding ties is
    needed.
  * W8A16 and the fp16 baseline accumulate in fp32 on the MFMA, so Y is
    compared per element against the oracle's float64 result with
      |dY| <= ulp16(Y_ref) + c(K) * S_main + 2^-9 * S_lora,
      c(K) = max(2^-14, (K + 2) 2^-24)
    (S_* = the sums of |terms|; (K + 2) 2^-24 bounds K - 1 fp32 additions in
    any order plus the scale multiplication, so the bound holds at every K),
    plus relative Frobenius error <= 1e-3.
Inputs come from workload/ (seeded) and are handed to both sides unchanged.
"""

import math

import numpy as np
import pytest
import torch

import rotation_quantized_int8_amd as cr
import workload as wl
from oracle import convrot_oracle as O

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    cr.lib()  # raises if the library is missing: the GPU path must be native
    torch.cuda.set_device(0)


DEV = "cuda:0"


def _np(t):
    return t.detach().cpu().numpy()


def _say(*a):
    print(*a, flush=True)


def _qw_oracle_and_gpu(w_cpu):
    qo, so = O.quantize_weights(w_cpu.numpy())
    qg, sg = cr.quantize_weights(w_cpu.to(DEV))
    torch.cuda.synchronize()
    return qo, so, _np(qg), _np(sg)


# --------------------------------------------------------------- weights (a0)

@pytest.mark.parametrize("N,K", [(256, 256), (80, 512), (37, 768), (3, 2048), (5, 8192)])
def test_weight_quant_bitexact(N, K):
    _say(f"weight quant N={N} K={K}")
    w = wl.make_weights(N, K, seed=N + K)
    qo, so, qg, sg = _qw_oracle_and_gpu(w)
    assert np.array_equal(sg.view(np.uint32), so.view(np.uint32))
    assert np.array_equal(qg, qo)


def test_weight_quant_extreme_values_bitexact():
    _say("weight quant extremes")
    rng = np.random.default_rng(5)
    w = (rng.normal(0, 1, (12, 512)) * np.exp2(rng.integers(-140, 120, (12, 512)))).astype(np.float32)
    w[0] = 0.0                                           # zero row
    w[1, :3] = [1.0, 2.0 ** -24, 2.0 ** -80]             # double-rounding trap
    w[1, 3:] = 0.0
    w[2] = np.float32(2.0 ** -149) * rng.integers(-5, 6, 512)   # subnormals only
    w[3, 0], w[3, 1] = np.float32(3e38), np.float32(-3e38)      # near fp32 max
    wt = torch.from_numpy(w)
    qo, so, qg, sg = _qw_oracle_and_gpu(wt)
    assert np.array_equal(sg.view(np.uint32), so.view(np.uint32))
    assert np.array_equal(qg, qo)
    assert so[0] == 0 and not qg[0].any()


@pytest.mark.parametrize("N,K", [(n, k) for (n, k, _) in wl.LAYER_SHAPES])
def test_weight_quant_bitexact_full_shapes(N, K):
    _say(f"weight quant full N={N} K={K}")
    w = wl.make_weights(N, K, seed=1)
    qo, so, qg, sg = _qw_oracle_and_gpu(w)
    assert np.array_equal(sg.view(np.uint32), so.view(np.uint32))
    assert int((qg != qo).sum()) == 0


# ----------------------------------------------------------- prologue (a1-a3)

def _act_compare(x_cpu):
    qo, so = O.quantize_activations(x_cpu.numpy())
    qg, sg = cr.act_quant(x_cpu.to(DEV))
    qg, sg = _np(qg), _np(sg)
    s_mis = int((sg.view(np.uint32) != so.view(np.uint32)).sum())
    q_mis = int((qg != qo).sum())
    return q_mis, s_mis


@pytest.mark.parametrize("M,K,dist", [(64, 256, "normal"), (37, 768, "normal"), (300, 2048, "normal"),
                                      (33, 4096, "t3"), (5, 8192, "normal"), (3, 12288, "t3"),
                                      (3, 20480, "normal"), (2, 131072, "t3"), (1, 256, "normal"),
                                      # more row blocks than the device holds at once: workgroups of
                                      # the persistent prologue walk two or more blocks, the last
                                      # one ragged
                                      (16389, 256, "normal"), (2051, 2048, "t3"), (1001, 8192, "normal")])
def test_act_quant_bitexact(M, K, dist):
    _say(f"act quant M={M} K={K} {dist}")
    x = wl.make_activations(M, K, seed=M * 7 + K, dist=dist)
    q_mis, s_mis = _act_compare(x)
    _say(f"  Q_X mismatches {q_mis} / {M * K}, s_X mismatches {s_mis}")
    assert s_mis == 0 and q_mis == 0


def test_act_quant_special_rows():
    _say("act quant special rows")
    import json
    import os
    g = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "hand_cases.json")))
    rows = []
    for r in g["tie_rows"]["rows"]:
        x = np.empty(512)
        x[0:256:2] = r["x_even_num"] / r["den"]
        x[1:256:2] = r["x_odd_num"] / r["den"]
        x[256:] = 0.0
        rows.append(x)
    rows.append(np.zeros(512))                                   # zero row
    rows.append(np.full(512, 65504.0))                           # fp16 max
    rows.append(np.full(512, -65504.0))
    rows.append(np.where(np.arange(512) % 3 == 0, 2.0 ** -24, -(2.0 ** -24)))  # subnormals
    rows.append(np.concatenate([np.full(256, 0.5), np.zeros(256)]))           # constant group
    x = torch.from_numpy(np.array(rows).astype(np.float16))
    qo, so = O.quantize_activations(x.numpy())
    qg, sg = cr.act_quant(x.to(DEV))
    qg, sg = _np(qg), _np(sg)
    assert np.array_equal(sg.view(np.uint32), so.view(np.uint32))
    assert np.array_equal(qg, qo)
    assert list(qg[:4, 1]) == [r["Q_X_1"] for r in g["tie_rows"]["rows"]]
    assert sg[4] == 0 and not qg[4].any()


def test_act_quant_sampled_rows_large_m():
    # rows are independent: the oracle runs on a sample of the rows
    M, K = 16384, 8192
    _say(f"act quant sampled M={M} K={K}")
    x = wl.make_activations(M, K, seed=3, dist="t3")
    qg, sg = cr.act_quant(x.to(DEV))
    rows = np.random.default_rng(0).choice(M, 48, replace=False)
    rows = np.concatenate([rows, [0, M - 1]])
    qo, so = O.quantize_activations(x.numpy()[rows])
    assert np.array_equal(_np(sg)[rows].view(np.uint32), so.view(np.uint32))
    assert np.array_equal(_np(qg)[rows], qo)


# ------------------------------------------------------- integer GEMM (a4)

@pytest.mark.parametrize("M,N,K", [(37, 80, 256), (1, 8, 256), (300, 200, 768), (129, 130, 512),
                                   (64, 256, 256), (17, 3, 1024), (256, 256, 131072)])
def test_gemm_i8_i32_bitexact(M, N, K):
    _say(f"gemm i8->i32 M={M} N={N} K={K}")
    rng = np.random.default_rng(M + N + K)
    qx = rng.integers(-127, 128, (M, K), dtype=np.int8)
    qw = rng.integers(-127, 128, (N, K), dtype=np.int8)
    if K == 131072:
        qx[0] = 127
        qw[0] = 127
        qw[1] = -127
    ao = O.int8_gemm(qx, qw)
    ag = _np(cr.gemm_i8_i32(torch.from_numpy(qx).to(DEV), torch.from_numpy(qw).to(DEV)))
    assert int((ag.astype(np.int64) != ao).sum()) == 0


@pytest.mark.parametrize("N,K", [(n, k) for (n, k, _) in wl.LAYER_SHAPES])
def test_gemm_i8_i32_bitexact_full_shapes(N, K):
    M = wl.M_FIXED
    _say(f"gemm i8->i32 full M={M} N={N} K={K}")
    rng = np.random.default_rng(N * 3 + K)
    qx = rng.integers(-127, 128, (M, K), dtype=np.int8)
    qw = rng.integers(-127, 128, (N, K), dtype=np.int8)
    ao = O.int8_gemm(qx, qw)
    ag = _np(cr.gemm_i8_i32(torch.from_numpy(qx).to(DEV), torch.from_numpy(qw).to(DEV)))
    assert int((ag.astype(np.int64) != ao).sum()) == 0


# ------------------------------------------------------ scale epilogue (a5)

@pytest.mark.parametrize("M,N,K,with_bias", [(37, 80, 256, False), (300, 203, 768, True),
                                             (1024, 2048, 2048, True)])
def test_gemm_i8_f16_bitexact_given_same_inputs(M, N, K, with_bias):
    _say(f"gemm i8->f16 M={M} N={N} K={K} bias={with_bias}")
    x = wl.make_activations(M, K, seed=11)
    w = wl.make_weights(N, K, seed=12)
    qx, sx = O.quantize_activations(x.numpy())
    qw, sw = O.quantize_weights(w.numpy())
    bias = wl.make_bias(N, seed=13).numpy() if with_bias else None
    yo = O.epilogue_w8a8(O.int8_gemm(qx, qw), sx, sw, bias)
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(DEV)
    yg = _np(cr.gemm_i8_f16(t(qx), t(sx), t(qw), t(sw), None if bias is None else t(bias)))
    assert np.array_equal(yg.view(np.uint16), yo.view(np.uint16))


def test_gemm_i8_f16_repeated_launches_every_tile():
    """Back-to-back launches over shapes that select each int8 tile
    configuration (128x128 on two stages, 256x128, 128x64, 64x64 and 32x32
    tiles), interleaved so
    that the timing of one launch differs from the next; every output must
    equal the oracle bit for bit.  Guards the ordering of the LDS writes of
    the staged output tile before the barrier that publishes them."""
    shapes = [(1024, 6144, 256), (1024, 2048, 2048), (512, 1024, 4096), (128, 6144, 2048), (1024, 256, 2048)]
    rng = np.random.default_rng(2024)
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(DEV)
    cases = []
    for (M, N, K) in shapes:
        qx = rng.integers(-127, 128, (M, K), dtype=np.int8)
        qw = rng.integers(-127, 128, (N, K), dtype=np.int8)
        sx = (rng.random(M, dtype=np.float32) * np.float32(0.01) + np.float32(1e-4)).astype(np.float32)
        sw = (rng.random(N, dtype=np.float32) * np.float32(0.001) + np.float32(1e-5)).astype(np.float32)
        ao = O.int8_gemm(qx, qw)
        yo = O.epilogue_w8a8(ao, sx, sw, None)
        cases.append(((M, N, K), t(qx), t(sx), t(qw), t(sw), t(yo.view(np.int16)), t(ao.astype(np.int32))))
    for rep in range(12):
        for (shape, qx, sx, qw, sw, yo, ao) in cases:
            yg = cr.gemm_i8_f16(qx, sx, qw, sw, None)
            ag = cr.gemm_i8_i32(qx, qw) if rep % 3 == 0 else None   # the int32 tile staging too
            torch.cuda.synchronize()
            bad = int((yg.view(torch.int16) != yo).sum())
            assert bad == 0, f"launch {rep} of M, N, K = {shape}: {bad} fp16 elements differ"
            if ag is not None:
                bad = int((ag != ao).sum())
                assert bad == 0, f"launch {rep} of M, N, K = {shape}: {bad} int32 elements differ"


@pytest.mark.parametrize("M,N,K", [(4, 8192, 2048), (64, 8192, 2048), (1024, 6144, 256)])
def test_linear_repeats_are_bit_identical(M, N, K):
    """The fused few-row, K-split and tiled W8A8 paths, alone and with LoRA
    and a residual, give the same bits on every repeat while other layers'
    launches run in between (no result may depend on launch timing)."""
    _say(f"repeat determinism M={M} N={N} K={K}")
    x = wl.make_activations(M, K, seed=5).to(DEV)
    w = wl.make_weights(N, K, seed=6).to(DEV)
    qw, sw = cr.quantize_weights(w)
    b = wl.make_bias(N, seed=7).to(DEV)
    g = torch.Generator().manual_seed(8)
    r = (torch.randn(M, N, generator=g) * 0.1).half().to(DEV)
    down = (torch.randn(32, K, generator=g) * 0.02).to(DEV)
    up = (torch.randn(N, 32, generator=g) * 0.02).to(DEV)
    xo = wl.make_activations(256, 2048, seed=9).to(DEV)
    qo, so = cr.quantize_weights(wl.make_weights(2048, 2048, seed=10).to(DEV))
    paths = [lambda: cr.linear_w8a8(x, qw, sw, b),
             lambda: cr.linear_w8a8_ex(x, qw, sw, b, lora=(down, up, 0.5), residual=r)]
    for f in paths:
        ref = f().view(torch.int16).clone()
        for rep in range(8):
            cr.linear_w8a8(xo, qo, so)
            y = f()
            torch.cuda.synchronize()
            assert torch.equal(y.view(torch.int16), ref), f"repeat {rep} differs"


# ------------------------------------------------- end-to-end W8A8 (a1-a5)

def _e_max(yg, yo, sx, sw, K):
    d = np.abs(yg.astype(np.float64) - yo.astype(np.float64))
    return float((d / (np.outer(sx, sw).astype(np.float64) * K + 1e-300)).max())


def _w8a8_case(M, N, K, seed=0, dist="normal", bias=False, rows=None):
    x = wl.make_activations(M, K, seed=seed, dist=dist)
    w = wl.make_weights(N, K, seed=seed)
    b = wl.make_bias(N, seed=seed) if bias else None
    qw_g, sw_g = cr.quantize_weights(w.to(DEV))
    yg = _np(cr.linear_w8a8(x.to(DEV), qw_g, sw_g, None if b is None else b.to(DEV)))
    qw, sw = O.quantize_weights(w.numpy())
    assert np.array_equal(_np(qw_g), qw) and np.array_equal(_np(sw_g).view(np.uint32), sw.view(np.uint32))
    xs = x.numpy() if rows is None else x.numpy()[rows]
    yo, qx, sx, a = O.linear_w8a8(xs, qw, sw, None if b is None else b.numpy())
    ygs = yg if rows is None else yg[rows]
    mism = int((ygs.view(np.uint16) != yo.view(np.uint16)).sum())
    emax = _e_max(ygs, yo, sx, sw, K)
    truth = O.linear_true(xs.astype(np.float64), w.numpy())
    if b is not None:
        truth = truth + b.numpy()[None, :]
    rel = float(np.linalg.norm(ygs.astype(np.float64) - truth) / np.linalg.norm(truth))
    _say(f"  Y mismatches {mism} / {ygs.size}, e_max {emax:.3g}, rel. error vs unquantised {rel:.4f}")
    return mism, emax, rel


@pytest.mark.parametrize("M,N,K,bias", [(64, 256, 256, False), (64, 256, 256, True),
                                        (300, 203, 768, True), (1, 1, 256, False), (5, 4, 512, True)])
def test_linear_w8a8_end_to_end_bitexact(M, N, K, bias):
    _say(f"linear w8a8 M={M} N={N} K={K} bias={bias}")
    mism, emax, rel = _w8a8_case(M, N, K, seed=M + N, bias=bias)
    assert mism == 0 and emax == 0.0


@pytest.mark.parametrize("N,K", [(n, k) for (n, k, _) in wl.LAYER_SHAPES])
def test_linear_w8a8_end_to_end_full_shapes(N, K):
    _say(f"linear w8a8 full M=1024 N={N} K={K}")
    mism, emax, rel = _w8a8_case(wl.M_FIXED, N, K, seed=0)
    assert mism == 0 and emax == 0.0
    assert rel < 0.05


@pytest.mark.parametrize("M", [1, 16, 128, 4096, 16384])
@pytest.mark.parametrize("N,K", [(8192, 2048), (2048, 8192)])
@pytest.mark.parametrize("dist", ["normal", "t3"])
def test_linear_w8a8_m_sweep(M, N, K, dist):
    _say(f"linear w8a8 m-sweep M={M} N={N} K={K} {dist}")
    rows = None
    if M > 1024:
        rows = np.unique(np.concatenate([np.random.default_rng(M).choice(M, 64, replace=False), [0, M - 1]]))
    mism, emax, rel = _w8a8_case(M, N, K, seed=2, dist=dist, rows=rows)
    assert mism == 0 and emax == 0.0


@pytest.mark.parametrize("M,N,K,bias", [(32, 2048, 2048, False), (5, 200, 4096, True),
                                        (16, 2048, 8192, True), (64, 1000, 2048, False)])
def test_linear_w8a8_split_k_bitexact(M, N, K, bias):
    # few rows: K is split over workgroups and the int32 partials are summed
    # in a separate epilogue; the result must equal the unsplit definition
    _say(f"linear w8a8 split-K M={M} N={N} K={K} bias={bias}")
    mism, emax, rel = _w8a8_case(M, N, K, seed=M * 7 + N, bias=bias)
    assert mism == 0 and emax == 0.0


def test_linear_w8a8_empty_1d_and_leading_dims():
    _say("linear w8a8 empty / 1-D / 3-D")
    K, N = 512, 40
    w = wl.make_weights(N, K, seed=3)
    qw, sw = cr.quantize_weights(w.to(DEV))
    y0 = cr.linear_w8a8(torch.empty((0, K), dtype=torch.float16, device=DEV), qw, sw)
    assert tuple(y0.shape) == (0, N)
    x = wl.make_activations(6, K, seed=4)
    y_full = _np(cr.linear_w8a8(x.to(DEV), qw, sw))
    y1 = _np(cr.linear_w8a8(x[2].to(DEV), qw, sw))
    assert y1.shape == (N,) and np.array_equal(y1.view(np.uint16), y_full[2].view(np.uint16))
    y3 = _np(cr.linear_w8a8(x.reshape(2, 3, K).to(DEV), qw, sw))
    assert np.array_equal(y3.reshape(6, N).view(np.uint16), y_full.view(np.uint16))
    # strided input / storage offset
    xs = torch.zeros((6, 2 * K), dtype=torch.float16)
    xs[:, K:] = x
    y_str = _np(cr.linear_w8a8(xs[:, K:].to(DEV), qw, sw))
    assert np.array_equal(y_str.view(np.uint16), y_full.view(np.uint16))


def test_linear_w8a8_deterministic():
    _say("linear w8a8 determinism")
    x = wl.make_activations(256, 2048, seed=9).to(DEV)
    qw, sw = cr.quantize_weights(wl.make_weights(512, 2048, seed=9).to(DEV))
    a = cr.linear_w8a8(x, qw, sw)
    b = cr.linear_w8a8(x, qw, sw)
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


@pytest.mark.parametrize("M,N,K", [(40, 64, 16384), (7, 48, 65536), (3, 16, 131072)])
def test_linear_w8a8_long_rows_bitexact(M, N, K):
    # rows longer than one prologue pass: the transform is recomputed per chunk
    _say(f"linear w8a8 long rows M={M} N={N} K={K}")
    mism, emax, rel = _w8a8_case(M, N, K, seed=K % 97)
    assert mism == 0 and emax == 0.0


# Assorted sizes around the tile plans: both large tiles (256x128 on 8
# waves, 128x64), ragged M and N, K of 1 to 32 rotation groups.
@pytest.mark.parametrize("M,N,K,bias", [(1024, 6144, 256, False), (1000, 2000, 1024, True),
                                        (777, 300, 512, False), (129, 72, 256, True),
                                        (600, 4100, 768, False), (1024, 256, 8192, False),
                                        (520, 8200, 2048, True)])
def test_linear_w8a8_assorted_shapes_bitexact(M, N, K, bias):
    _say(f"linear w8a8 assorted M={M} N={N} K={K} bias={bias}")
    mism, emax, rel = _w8a8_case(M, N, K, seed=M + K, bias=bias)
    assert mism == 0 and emax == 0.0


def test_linear_w8a8_workspace_reuse():
    # one workspace (filled with garbage first) for calls of different sizes,
    # back to back: every result bit-exact
    _say("linear w8a8 workspace reuse")
    shapes = [(1024, 2048, 2048), (16, 256, 8192), (300, 203, 768), (2048, 8192, 2048), (1, 8, 256)]
    need = max(cr.workspace_bytes(cr.PATH_W8A8, M, N, K) for (M, N, K) in shapes)
    ws = torch.full((need,), 0xA5, dtype=torch.uint8, device=DEV)
    for i, (M, N, K) in enumerate(shapes):
        x = wl.make_activations(M, K, seed=20 + i)
        w = wl.make_weights(N, K, seed=20 + i)
        qw, sw = O.quantize_weights(w.numpy())
        t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(DEV)
        yg = _np(cr.linear_w8a8(x.to(DEV), t(qw), t(sw), workspace=ws))
        torch.cuda.synchronize()
        yo = O.linear_w8a8(x.numpy(), qw, sw)[0]
        mism = int((yg.view(np.uint16) != yo.view(np.uint16)).sum())
        _say(f"  M={M} N={N} K={K}: mismatches {mism}")
        assert mism == 0


def test_linear_w8a8_graph_replays_match_eager():
    # a captured graph of W8A8 calls, replayed with eager work in between
    _say("linear w8a8 graph replay vs eager")
    M, N, K = 512, 2048, 2048
    x = wl.make_activations(M, K, seed=31).to(DEV)
    qw, sw = cr.quantize_weights(wl.make_weights(N, K, seed=31).to(DEV))
    ws = torch.empty(cr.workspace_bytes(cr.PATH_W8A8, M, N, K), dtype=torch.uint8, device=DEV)
    ref = cr.linear_w8a8(x, qw, sw, workspace=ws).clone()
    ys = [torch.empty((M, N), dtype=torch.float16, device=DEV) for _ in range(3)]
    stream = torch.cuda.Stream()
    L = cr.lib()
    def calls():
        h = torch.cuda.current_stream().cuda_stream
        for y in ys:
            st = L.convrot_linear_w8a8(x.data_ptr(), M, K, qw.data_ptr(), sw.data_ptr(), N, None,
                                       y.data_ptr(), ws.data_ptr(), ws.numel(), h)
            assert st == 0
    torch.cuda.synchronize()
    with torch.cuda.stream(stream):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=stream):
            calls()
    torch.cuda.synchronize()
    for rep in range(4):
        for y in ys:
            y.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for y in ys:
            assert torch.equal(y.view(torch.int16), ref.view(torch.int16)), f"replay {rep}"
        e = cr.linear_w8a8(x, qw, sw, workspace=ws)   # eager call between replays
        torch.cuda.synchronize()
        assert torch.equal(e.view(torch.int16), ref.view(torch.int16))
    _say("  4 replays x 3 calls equal to the eager result")


# ------------------------------ W8A8 with bias, unmerged LoRA and residual

def _ulp16(y):
    a = np.abs(y.astype(np.float64))
    e = np.floor(np.log2(np.maximum(a, 2.0 ** -14)))
    return np.exp2(e - 10)


def _w8a8_ex_case(M, N, K, seed, bias=False, rank=0, residual=True, in_place=False, up_zero=False):
    """Runs the GPU and the oracle on one seeded case; returns (Y_gpu, Y_oracle, tolerance)."""
    x = wl.make_activations(M, K, seed=seed)
    w = wl.make_weights(N, K, seed=seed)
    qw, sw = O.quantize_weights(w.numpy())
    b = wl.make_bias(N, seed=seed) if bias else None
    r = wl.make_residual(M, N, seed=seed) if residual else None
    lora = None
    if rank:
        d, u = wl.make_lora(N, K, rank=rank, seed=seed)
        if up_zero:
            u = torch.zeros_like(u)
        lora = (d, u, 0.5)
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(DEV)
    dlora = None if lora is None else (lora[0].to(DEV), lora[1].to(DEV), lora[2])
    db = None if b is None else b.to(DEV)
    if in_place:
        buf = r.to(DEV).clone()
        yt = cr.linear_w8a8_ex(x.to(DEV), t(qw), t(sw), bias=db, lora=dlora, residual=buf, out=buf)
        assert yt.data_ptr() == buf.data_ptr()
    else:
        yt = cr.linear_w8a8_ex(x.to(DEV), t(qw), t(sw), bias=db, lora=dlora,
                               residual=None if r is None else r.to(DEV))
    yg = _np(yt)
    olora = None if lora is None else (lora[0].numpy(), lora[1].numpy(), lora[2])
    ob = None if b is None else b.numpy()
    yo = O.linear_w8a8_ex(x.numpy(), qw, sw, bias=ob, lora=olora, residual=None if r is None else r.numpy())
    tol = np.zeros(yo.shape)
    if lora is not None:
        # the LoRA term is fp16 MFMA work (down, T and scale * up rounded to
        # fp16, fp32 sums): bounded by 2^-9 of the sum of its magnitudes; one
        # fp16 ulp before the residual step and one after it cover the roundings
        pre = O.linear_w8a8_ex(x.numpy(), qw, sw, bias=ob, lora=olora)
        tt = np.abs(x.numpy().astype(np.float64) @ olora[0].astype(np.float64).T)
        s_lora = abs(olora[2]) * (tt @ np.abs(olora[1].astype(np.float64)).T)
        tol = _ulp16(pre) + (_ulp16(yo) if r is not None else 0.0) + 2.0 ** -9 * s_lora
    return yg, yo, tol


@pytest.mark.parametrize("M,N,K,bias", [(64, 256, 256, False), (300, 203, 768, True),
                                        (1024, 2048, 2048, True), (16, 2048, 8192, True),
                                        (5, 200, 4096, False), (1024, 6144, 256, True),
                                        (129, 72, 256, True)])
def test_linear_w8a8_ex_bias_residual_bitexact(M, N, K, bias):
    # no LoRA: the residual step is one correctly rounded fp16 addition, so
    # the whole result is exact (few-row shapes take the K-split path)
    _say(f"linear w8a8_ex bias+residual M={M} N={N} K={K} bias={bias}")
    yg, yo, _ = _w8a8_ex_case(M, N, K, seed=M + 3 * N, bias=bias)
    mism = int((yg.view(np.uint16) != yo.view(np.uint16)).sum())
    _say(f"  mismatches {mism} / {yo.size}")
    assert mism == 0


@pytest.mark.parametrize("M,N,K,rank", [(300, 203, 768, 0), (16, 2048, 8192, 0), (1024, 2048, 2048, 0),
                                        (64, 256, 256, 32), (16, 2048, 8192, 32)])
def test_linear_w8a8_ex_in_place_residual(M, N, K, rank):
    _say(f"linear w8a8_ex in-place residual M={M} N={N} K={K} rank={rank}")
    yg, yo, tol = _w8a8_ex_case(M, N, K, seed=M + N + rank, bias=True, rank=rank, in_place=True)
    if rank == 0:
        assert np.array_equal(yg.view(np.uint16), yo.view(np.uint16))
    else:
        d = np.abs(yg.astype(np.float64) - yo.astype(np.float64))
        assert int((d > tol).sum()) == 0


@pytest.mark.parametrize("M,N,K,rank,bias,residual", [(64, 256, 256, 32, True, True),
                                                      (300, 203, 768, 17, True, True),
                                                      (1, 8, 512, 64, False, True),
                                                      (1024, 2048, 2048, 32, True, True),
                                                      (1024, 6144, 256, 32, False, False),
                                                      (16, 2048, 8192, 32, True, True),
                                                      (5, 200, 4096, 3, False, False)])
def test_linear_w8a8_ex_lora_within_tolerance(M, N, K, rank, bias, residual):
    _say(f"linear w8a8_ex LoRA M={M} N={N} K={K} rank={rank} bias={bias} residual={residual}")
    yg, yo, tol = _w8a8_ex_case(M, N, K, seed=M + rank, bias=bias, rank=rank, residual=residual)
    d = np.abs(yg.astype(np.float64) - yo.astype(np.float64))
    viol = int((d > tol).sum())
    rel = float(np.linalg.norm(d) / np.linalg.norm(yo.astype(np.float64)))
    exact = int((yg.view(np.uint16) == yo.view(np.uint16)).sum())
    _say(f"  violations {viol}, max |dY|/tol {float((d / tol).max()):.3f}, bit-equal {exact}/{yo.size}, "
         f"rel. Frobenius {rel:.2e}")
    assert viol == 0 and rel <= 1e-3


@pytest.mark.parametrize("M,N,K", [(64, 256, 256), (16, 2048, 8192), (300, 203, 768)])
def test_linear_w8a8_ex_zero_up_is_exact(M, N, K):
    # a LoRA whose up weight is zero adds exact zeros: the result is the exact
    # bias + residual layer, bit for bit, on both the GEMM and K-split paths
    _say(f"linear w8a8_ex zero-up LoRA M={M} N={N} K={K}")
    yg, _, _ = _w8a8_ex_case(M, N, K, seed=7 * M, bias=True, rank=32, up_zero=True)
    _, yo, _ = _w8a8_ex_case(M, N, K, seed=7 * M, bias=True)
    assert np.array_equal(yg.view(np.uint16), yo.view(np.uint16))


def test_linear_w8a8_ex_without_extras_equals_linear_w8a8():
    _say("linear w8a8_ex without extras == linear w8a8")
    for (M, N, K) in ((300, 203, 768), (16, 2048, 8192)):
        x = wl.make_activations(M, K, seed=41).to(DEV)
        qw, sw = cr.quantize_weights(wl.make_weights(N, K, seed=41).to(DEV))
        b = wl.make_bias(N, seed=41).to(DEV)
        a = cr.linear_w8a8(x, qw, sw, b)
        e = cr.linear_w8a8_ex(x, qw, sw, bias=b)
        assert torch.equal(a.view(torch.int16), e.view(torch.int16))


# ------------------------------------------------ weight-only W8A16 (a6, a7)

def _acc_c(K):
    """Per-element accumulation allowance of the fp32-accumulated paths."""
    return max(2.0 ** -14, (K + 2) * 2.0 ** -24)


def _sample_rows(M, n=96, tile=256):
    """Rows for oracle comparison at large M: both rows of every tile edge,
    the first and last rows, and a seeded spread in between."""
    edges = [r for t in range(0, M, tile) for r in (t, min(t + tile, M) - 1)]
    rng = np.random.default_rng(M)
    pick = rng.choice(M, min(M, n), replace=False)
    return np.unique(np.concatenate([edges, pick, [0, M - 1]])).astype(np.int64)


def _w8a16_case(M, N, K, rank=0, bias=False, seed=0, rows=None):
    x = wl.make_activations(M, K, seed=seed)
    w = wl.make_weights(N, K, seed=seed)
    qw, sw = O.quantize_weights(w.numpy())
    b = wl.make_bias(N, seed=seed) if bias else None
    lora = None
    if rank:
        d, u = wl.make_lora(N, K, rank=rank, seed=seed)
        lora = (d, u, 1.0)
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(DEV)
    yg = _np(cr.linear_w8a16(x.to(DEV), t(qw), t(sw), None if b is None else b.to(DEV),
                             None if lora is None else (lora[0].to(DEV), lora[1].to(DEV), lora[2])))
    xs = x.numpy() if rows is None else x.numpy()[rows]
    if rows is not None:
        yg = yg[rows]
    yo = O.linear_w8a16(xs, qw, sw, None if b is None else b.numpy(),
                        None if lora is None else (lora[0].numpy(), lora[1].numpy(), lora[2]))
    x16r = O.rotate_activations_f16(xs).astype(np.float64)
    s_main = (np.abs(x16r) @ np.abs(qw.astype(np.float64)).T) * sw.astype(np.float64)[None, :]
    s_lora = 0.0
    if rank:
        tt = np.abs(xs.astype(np.float64) @ lora[0].numpy().astype(np.float64).T)
        s_lora = tt @ np.abs(lora[1].numpy().astype(np.float64)).T
    bound = _ulp16(yo) + _acc_c(K) * s_main + 2.0 ** -9 * s_lora
    d = np.abs(yg.astype(np.float64) - yo.astype(np.float64))
    viol = int((d > bound).sum())
    rel = float(np.linalg.norm(yg.astype(np.float64) - yo.astype(np.float64)) / np.linalg.norm(yo.astype(np.float64)))
    _say(f"  violations {viol}, max |dY|/bound {float((d / bound).max()):.3f}, rel. Frobenius {rel:.2e}")
    return viol, rel


def test_act_rotate_f16_bitexact():
    for M, K in ((64, 256), (37, 768), (3, 20480)):
        _say(f"rotate f16 M={M} K={K}")
        x = wl.make_activations(M, K, seed=K)
        yo = O.rotate_activations_f16(x.numpy())
        yg = _np(cr.act_rotate_f16(x.to(DEV)))
        assert np.array_equal(yg.view(np.uint16), yo.view(np.uint16))


@pytest.mark.parametrize("M,N,K,rank,bias", [(64, 256, 256, 0, False), (64, 256, 256, 32, True),
                                             (300, 203, 768, 17, True), (1, 8, 512, 64, False),
                                             (1024, 2048, 2048, 32, False), (1024, 256, 2048, 32, True)])
def test_linear_w8a16_within_tolerance(M, N, K, rank, bias):
    _say(f"linear w8a16 M={M} N={N} K={K} rank={rank} bias={bias}")
    viol, rel = _w8a16_case(M, N, K, rank=rank, bias=bias, seed=M + rank)
    assert viol == 0 and rel <= 1e-3


# Shapes that select the remaining tile instances of the fp16-MFMA kernels:
# 1024x6144x256 and 1024x8192x2048 the 256x128 tile (8 waves), 300x2048x8192
# the 64x64 tile.  The GPU computes every row; the oracle the sampled rows,
# which cover both edges of every 256-row tile and every column.
TILE_SHAPES = [(1024, 6144, 256), (1024, 8192, 2048), (300, 2048, 8192)]


@pytest.mark.parametrize("M,N,K", TILE_SHAPES)
@pytest.mark.parametrize("rank,bias", [(0, False), (32, True)])
def test_linear_w8a16_tile_instances(M, N, K, rank, bias):
    _say(f"linear w8a16 tile instance M={M} N={N} K={K} rank={rank} bias={bias}")
    viol, rel = _w8a16_case(M, N, K, rank=rank, bias=bias, seed=M + N + rank, rows=_sample_rows(M))
    assert viol == 0 and rel <= 1e-3


# ----------------------------------------------------------- fp16 baseline (a8)

@pytest.mark.parametrize("M,N,K", [(64, 256, 256), (300, 203, 768), (1024, 2048, 2048)] + TILE_SHAPES)
def test_gemm_f16_within_tolerance(M, N, K):
    _say(f"gemm f16 M={M} N={N} K={K}")
    x = wl.make_activations(M, K, seed=5)
    w16 = wl.make_weights(N, K, seed=5).to(torch.float16)
    yg = _np(cr.gemm_f16(x.to(DEV), w16.to(DEV)))
    rows = _sample_rows(M) if M * N * K > 2 ** 32 else np.arange(M)
    xs = x.numpy()[rows]
    yo = O.linear_f16(xs, w16.numpy())
    yg = yg[rows]
    s = np.abs(xs.astype(np.float64)) @ np.abs(w16.numpy().astype(np.float64)).T
    bound = _ulp16(yo) + _acc_c(K) * s
    d = np.abs(yg.astype(np.float64) - yo.astype(np.float64))
    rel = float(np.linalg.norm(d) / np.linalg.norm(yo.astype(np.float64)))
    _say(f"  violations {int((d > bound).sum())}, max |dY|/bound {float((d / bound).max()):.3f}, "
         f"rel. Frobenius {rel:.2e}")
    assert int((d > bound).sum()) == 0 and rel <= 1e-3


# --------------------------------- dequantise-every-call baseline (next-4)

@pytest.mark.parametrize("N,K", [(256, 256), (80, 512), (37, 768), (3, 8192)])
def test_dequantize_weights_bitexact(N, K):
    _say(f"dequantize weights N={N} K={K}")
    qw, sw = O.quantize_weights(wl.make_weights(N, K, seed=N + K).numpy())
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(DEV)
    wg = _np(cr.dequantize_weights(t(qw), t(sw)))
    wo = O.dequantize_weights(qw, sw)
    assert np.array_equal(wg.view(np.uint16), wo.view(np.uint16))


@pytest.mark.parametrize("N,K", [(n, k) for (n, k, _) in wl.LAYER_SHAPES])
def test_dequantize_weights_bitexact_full_shapes(N, K):
    # every element on the GPU; the oracle on 64 sampled rows plus the first and last
    _say(f"dequantize weights full N={N} K={K}")
    qw, sw = O.quantize_weights(wl.make_weights(N, K, seed=1).numpy())
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(DEV)
    wg = _np(cr.dequantize_weights(t(qw), t(sw)))
    rows = np.unique(np.concatenate([np.random.default_rng(N).choice(N, min(N, 64), replace=False), [0, N - 1]]))
    wo = O.dequantize_weights(qw[rows], sw[rows])
    assert np.array_equal(wg[rows].view(np.uint16), wo.view(np.uint16))


@pytest.mark.parametrize("M,N,K,bias", [(64, 256, 256, False), (300, 203, 768, True), (1024, 2048, 2048, True),
                                        (5, 200, 4096, False)] + [(m, n, k, True) for (m, n, k) in TILE_SHAPES])
def test_linear_dequant_within_tolerance(M, N, K, bias):
    _say(f"linear dequant M={M} N={N} K={K} bias={bias}")
    x = wl.make_activations(M, K, seed=M + 5)
    qw, sw = O.quantize_weights(wl.make_weights(N, K, seed=M + 5).numpy())
    b = wl.make_bias(N, seed=M + 5) if bias else None
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(DEV)
    yg = _np(cr.linear_dequant(x.to(DEV), t(qw), t(sw), None if b is None else b.to(DEV)))
    rows = _sample_rows(M) if M * N * K > 2 ** 32 else np.arange(M)
    xs = x.numpy()[rows]
    yg = yg[rows]
    yo = O.linear_dequant(xs, qw, sw, None if b is None else b.numpy())
    wd = O.dequantize_weights(qw, sw).astype(np.float64)
    s_main = np.abs(xs.astype(np.float64)) @ np.abs(wd).T
    bound = _ulp16(yo) + _acc_c(K) * s_main
    d = np.abs(yg.astype(np.float64) - yo.astype(np.float64))
    viol = int((d > bound).sum())
    rel = float(np.linalg.norm(d) / np.linalg.norm(yo.astype(np.float64)))
    _say(f"  violations {viol}, max |dY|/bound {float((d / bound).max()):.3f}, rel. Frobenius {rel:.2e}")
    assert viol == 0 and rel <= 1e-3


# ------------------------------------- one-launch layer for K = 256 (next-1)
# With K = 256 each row is a single rotation group, so for 16 < M <= 2048 and
# N a multiple of 4 the layer runs as one launch in which every workgroup
# quantises its band of 32 rows itself.  Cases cover a single ragged band,
# ragged 64-column chunks, rows that are not 16-byte aligned (N % 8 = 4),
# fewer chunks than wavefronts, and the wide column groups whose wavefronts
# loop over several chunks (M = 1500, 2048 and N = 12288 at M = 1024).

@pytest.mark.parametrize("M,N,bias,dist", [(17, 4, False, "normal"), (31, 60, True, "t3"),
                                           (32, 64, False, "normal"), (33, 100, True, "normal"),
                                           (100, 252, False, "t3"), (513, 2048, True, "normal"),
                                           (1000, 6148, False, "t3"), (1500, 6144, True, "normal"),
                                           (2048, 4096, False, "normal"), (1024, 12288, True, "t3")])
def test_linear_w8a8_band_bitexact(M, N, bias, dist):
    _say(f"linear w8a8 one launch K=256 M={M} N={N} bias={bias} {dist}")
    rows = None
    if M * N > (1 << 21):
        rows = np.unique(np.concatenate([np.random.default_rng(M + N).choice(M, 96, replace=False),
                                         [0, 31, 32, M - 1]]))
    mism, emax, rel = _w8a8_case(M, N, 256, seed=M * 3 + N, dist=dist, bias=bias, rows=rows)
    assert mism == 0 and emax == 0.0


@pytest.mark.parametrize("M", [40, 200])
def test_linear_w8a8_band_special_rows(M):
    # rounding-tie rows (their first group, whose maximum decides the row
    # scale), a zero row, fp16 extremes, subnormals and a constant row, then
    # ordinary rows into a ragged last band (16-row bands at M = 40, 32-row
    # bands at M = 200)
    _say(f"linear w8a8 one launch K=256 special rows M={M}")
    import json
    import os
    g = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "hand_cases.json")))
    rows = []
    for r in g["tie_rows"]["rows"]:
        x = np.empty(256)
        x[0:256:2] = r["x_even_num"] / r["den"]
        x[1:256:2] = r["x_odd_num"] / r["den"]
        rows.append(x)
    rows.append(np.zeros(256))
    rows.append(np.full(256, 65504.0))
    rows.append(np.full(256, -65504.0))
    rows.append(np.where(np.arange(256) % 3 == 0, 2.0 ** -24, -(2.0 ** -24)))
    rows.append(np.full(256, 0.5))
    rest = wl.make_activations(M - len(rows), 256, seed=77).numpy().astype(np.float64)
    x = np.concatenate([np.array(rows), rest]).astype(np.float16)
    w = wl.make_weights(72, 256, seed=78)
    qw, sw = O.quantize_weights(w.numpy())
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(DEV)
    yg = _np(cr.linear_w8a8(t(x), t(qw), t(sw)))
    with np.errstate(over="ignore"):   # the fp16-max rows overflow Y to +-inf on both sides
        yo, qx, sx, a = O.linear_w8a8(x, qw, sw, None)
    assert list(qx[:4, 1]) == [r["Q_X_1"] for r in g["tie_rows"]["rows"]]
    assert np.array_equal(yg.view(np.uint16), yo.view(np.uint16))
    assert not yg[4].any()


@pytest.mark.parametrize("M,N", [(33, 100), (100, 252), (1024, 6144), (1500, 6144)])
def test_linear_w8a8_band_residual_in_place(M, N):
    # bias and an fp16 residual that is the output buffer itself
    _say(f"linear w8a8_ex one launch K=256 in place M={M} N={N}")
    yg, yo, tol = _w8a8_ex_case(M, N, 256, seed=M + N, bias=True, in_place=True)
    assert np.array_equal(yg.view(np.uint16), yo.view(np.uint16))


# ------------------------------------- seeded random shapes, every plan
# Shapes drawn (fixed seed) from the size ranges that select each way the
# W8A8 layer runs: one fused launch (few short rows), the K = 256 band kernel
# (16- and 32-row bands), the narrow-layer kernel, the few-row kernel, the
# tiled GEMM with few rows (K split) and with many, including N that is not a
# multiple of 4 (no one-launch path).  Every case is bit-exact.

def _random_w8a8_shapes():
    rng = np.random.default_rng(20241)
    out = []
    for _ in range(3):
        out.append((int(rng.integers(1, 9)), int(rng.integers(1, 300)), 256 * int(rng.integers(1, 3))))      # fused / few-row
        out.append((int(rng.integers(17, 129)), 4 * int(rng.integers(1, 700)), 256))                         # band, 16 rows
        out.append((int(rng.integers(129, 2049)), 4 * int(rng.integers(1, 400)), 256))                       # band, 32 rows
        out.append((int(rng.integers(17, 1025)), 4 * int(rng.integers(1, 65)), 256 * int(rng.choice([2, 4]))))  # narrow
        out.append((int(rng.integers(1, 9)), int(rng.integers(300, 2000)), 256 * int(rng.integers(8, 33))))   # few-row kernel
        out.append((int(rng.integers(9, 129)), int(rng.integers(64, 1500)), 256 * int(rng.integers(16, 33))))  # K split
        out.append((int(rng.integers(129, 1500)), 4 * int(rng.integers(1, 300)) + 2, 256 * int(rng.integers(1, 9))))  # tiled, N % 4 = 2
    return out


@pytest.mark.parametrize("M,N,K", _random_w8a8_shapes())
def test_linear_w8a8_random_shapes_bitexact(M, N, K):
    _say(f"linear w8a8 random shape M={M} N={N} K={K}")
    mism, emax, rel = _w8a8_case(M, N, K, seed=M * 7 + N * 3 + K, dist="t3" if (M + N) % 2 else "normal",
                                 bias=(M + K) % 2 == 1)
    assert mism == 0 and emax == 0.0


# ------------------------- one-launch layer for narrow layers (next-1)
# With K = 512 or 1024 and N <= 256, while ceil(M / 8) ceil(N / 128) <= 256,
# the layer runs as one launch in which every workgroup quantises its band
# of 8 rows itself (twice per band when N > 128).  Cases cover a single
# ragged band, ragged 128-column groups, rows that are not 16-byte aligned
# (N % 8 = 4), both K, bias, heavy-tailed rows, and the largest grid
# (2048 x 128) next to a size just past it (2048 x 256, two launches).

@pytest.mark.parametrize("M,N,K,bias,dist", [(17, 4, 512, False, "normal"), (33, 100, 1024, True, "t3"),
                                             (64, 128, 512, False, "normal"), (100, 252, 1024, False, "t3"),
                                             (513, 256, 512, True, "normal"), (777, 132, 512, True, "normal"),
                                             (1000, 200, 1024, False, "normal"), (1024, 256, 1024, True, "t3"),
                                             (2048, 128, 1024, False, "normal"), (2048, 256, 1024, True, "normal")])
def test_linear_w8a8_narrow_bitexact(M, N, K, bias, dist):
    _say(f"linear w8a8 one launch narrow M={M} N={N} K={K} bias={bias} {dist}")
    mism, emax, rel = _w8a8_case(M, N, K, seed=M * 5 + N + K, dist=dist, bias=bias)
    assert mism == 0 and emax == 0.0


@pytest.mark.parametrize("K", [512, 1024])
def test_linear_w8a8_narrow_special_rows(K):
    # rounding-tie rows (their first group decides the row scale; the rest of
    # the row is zero), a zero row, fp16 extremes, subnormals and a constant
    # row, in the first band and into a ragged second one
    _say(f"linear w8a8 one launch narrow K={K} special rows")
    import json
    import os
    g = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "hand_cases.json")))
    rows = []
    for r in g["tie_rows"]["rows"]:
        x = np.zeros(K)
        x[0:256:2] = r["x_even_num"] / r["den"]
        x[1:256:2] = r["x_odd_num"] / r["den"]
        rows.append(x)
    rows.append(np.zeros(K))
    rows.append(np.full(K, 65504.0))
    rows.append(np.full(K, -65504.0))
    rows.append(np.where(np.arange(K) % 3 == 0, 2.0 ** -24, -(2.0 ** -24)))
    rows.append(np.full(K, 0.5))
    rest = wl.make_activations(21 - len(rows), K, seed=79).numpy().astype(np.float64)
    x = np.concatenate([np.array(rows), rest]).astype(np.float16)
    w = wl.make_weights(136, K, seed=80)
    qw, sw = O.quantize_weights(w.numpy())
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(DEV)
    yg = _np(cr.linear_w8a8(t(x), t(qw), t(sw)))
    with np.errstate(over="ignore"):   # the fp16-max rows overflow Y to +-inf on both sides
        yo, qx, sx, a = O.linear_w8a8(x, qw, sw, None)
    assert list(qx[:4, 1]) == [r["Q_X_1"] for r in g["tie_rows"]["rows"]]
    assert np.array_equal(yg.view(np.uint16), yo.view(np.uint16))
    assert not yg[4].any()


@pytest.mark.parametrize("M,N,K", [(33, 100, 1024), (300, 252, 512), (1024, 256, 1024)])
def test_linear_w8a8_narrow_residual_in_place(M, N, K):
    # bias and an fp16 residual that is the output buffer itself
    _say(f"linear w8a8_ex one launch narrow in place M={M} N={N} K={K}")
    yg, yo, tol = _w8a8_ex_case(M, N, K, seed=M + N + K, bias=True, in_place=True)
    assert np.array_equal(yg.view(np.uint16), yo.view(np.uint16))


# ------------------------------------------ few activation rows (next-1)
# M <= 16 with M K <= 8192 runs as one fused launch; M <= 16 with N <= 4096
# otherwise runs the prologue and the few-row kernel (K split into int32
# partials when N is small); larger M the tiled GEMM with narrow tiles (K
# split when even those give few workgroups).  All bit-exact.

@pytest.mark.parametrize("M,N,K,bias", [(1, 8192, 2048, False), (1, 2048, 8192, True), (4, 2048, 2048, True),
                                        (16, 6144, 256, False), (3, 203, 768, True), (2, 8, 4096, False),
                                        (16, 2048, 8192, True), (32, 8192, 2048, False), (17, 300, 4096, True),
                                        (8, 256, 8192, False), (24, 1000, 1024, True), (1, 256, 131072, False),
                                        (24, 64, 65536, True), (100, 128, 16384, False), (128, 8192, 2048, True),
                                        (64, 6144, 256, False), (8, 4096, 4096, True), (9, 4096, 4096, False),
                                        (12, 1024, 8192, True), (300, 256, 2048, False)])
def test_linear_w8a8_few_rows_bitexact(M, N, K, bias):
    _say(f"linear w8a8 few rows M={M} N={N} K={K} bias={bias}")
    mism, emax, rel = _w8a8_case(M, N, K, seed=3 * M + K, bias=bias)
    assert mism == 0 and emax == 0.0


@pytest.mark.parametrize("M,N,K,rank", [(1, 2048, 2048, 0), (4, 8192, 2048, 0), (16, 2048, 8192, 0),
                                        (8, 256, 8192, 0), (1, 2048, 2048, 32), (16, 2048, 8192, 32),
                                        (24, 64, 16384, 0), (24, 64, 16384, 32), (32, 8192, 2048, 32)])
def test_linear_w8a8_ex_few_rows(M, N, K, rank):
    _say(f"linear w8a8_ex few rows M={M} N={N} K={K} rank={rank}")
    yg, yo, tol = _w8a8_ex_case(M, N, K, seed=M + K + rank, bias=True, rank=rank, in_place=(M == 4))
    if rank == 0:
        assert np.array_equal(yg.view(np.uint16), yo.view(np.uint16))
    else:
        d = np.abs(yg.astype(np.float64) - yo.astype(np.float64))
        assert int((d > tol).sum()) == 0


# ------------------------------------ range-safe weight-only path (next-3)

def _rs_input(M, K, dtype, kind, seed):
    """float32 values representable in the 16-bit input type, and that tensor."""
    g = torch.Generator().manual_seed(seed)
    if kind == "normal":
        v = wl.make_activations(M, K, seed=seed).float()
    elif kind == "huge":
        v = torch.randn((M, K), generator=g) * 1e30
    elif kind == "nearmax":
        v = torch.sign(torch.randn((M, K), generator=g)) * 65504.0
        v[1::2] = torch.randn((M // 2, K), generator=g) * 3.0
    else:   # zero row, a row of tiny values, a normal row
        v = torch.randn((M, K), generator=g)
        v[0] = 0
        v[1] = torch.randint(-3, 4, (K,), generator=g).float() * 2.0 ** -24
    t = v.to(torch.float16 if dtype == "f16" else torch.bfloat16)
    return t.float().numpy(), t


@pytest.mark.parametrize("M,K,dtype,kind", [(64, 256, "f16", "normal"), (37, 768, "bf16", "huge"),
                                            (6, 20480, "f16", "nearmax"), (300, 2048, "bf16", "normal"),
                                            (3, 512, "f16", "zero_tiny"), (4, 1024, "bf16", "nearmax")])
def test_act_rotate_scaled_bitexact(M, K, dtype, kind):
    _say(f"range-safe prologue M={M} K={K} {dtype} {kind}")
    x32, xt = _rs_input(M, K, dtype, kind, seed=M + K)
    x16g, eg = cr.act_rotate_scaled(xt.to(DEV))
    x16o, eo = O.rotate_rowscaled_f16(x32)
    assert np.array_equal(_np(eg).astype(np.int64), eo)
    assert np.array_equal(_np(x16g).view(np.uint16), x16o.view(np.uint16))


def _ulp_out(y, out):
    a = np.abs(np.asarray(y, np.float64))
    if out == "f16":
        return np.exp2(np.floor(np.log2(np.maximum(a, 2.0 ** -14))) - 10)
    return np.exp2(np.floor(np.log2(np.maximum(a, 2.0 ** -126))) - 7)


@pytest.mark.parametrize("M,N,K,xd,yd,bias,res,kind", [(64, 256, 256, "f16", "f16", False, False, "normal"),
                                                       (300, 203, 768, "bf16", "bf16", True, True, "normal"),
                                                       (1024, 2048, 2048, "bf16", "bf16", True, False, "normal"),
                                                       (37, 80, 512, "f16", "bf16", False, True, "nearmax"),
                                                       (16, 256, 4096, "f16", "f16", True, True, "normal"),
                                                       (8, 128, 1024, "bf16", "bf16", False, False, "huge"),
                                                       # K beyond fp16's largest finite value (65504)
                                                       (4, 64, 65792, "f16", "f16", True, False, "normal"),
                                                       (4, 64, 65792, "bf16", "bf16", False, True, "nearmax"),
                                                       # the 256x128 and 64x64 tile instances
                                                       (1024, 6144, 256, "f16", "f16", True, True, "normal"),
                                                       (1024, 8192, 2048, "bf16", "bf16", False, False, "normal"),
                                                       (1024, 8192, 2048, "f16", "bf16", True, False, "nearmax"),
                                                       (300, 2048, 8192, "bf16", "f16", True, True, "normal")])
def test_linear_w8a16_rs_within_tolerance(M, N, K, xd, yd, bias, res, kind):
    _say(f"range-safe w8a16 M={M} N={N} K={K} {xd}->{yd} bias={bias} residual={res} {kind}")
    x32, xt = _rs_input(M, K, xd, kind, seed=M + N)
    qw, sw = O.quantize_weights(wl.make_weights(N, K, seed=M + N).numpy())
    b = wl.make_bias(N, seed=M) if bias else None
    ydt = torch.float16 if yd == "f16" else torch.bfloat16
    r = wl.make_residual(M, N, seed=M).float().to(ydt) if res else None
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(DEV)
    yg = cr.linear_w8a16_rs(xt.to(DEV), t(qw), t(sw), None if b is None else b.to(DEV),
                            None if r is None else r.to(DEV), out_dtype=ydt)
    yg = yg.float().cpu().numpy().astype(np.float64)
    rows = _sample_rows(M, n=48) if M * N * K > 2 ** 32 else np.arange(M)
    xs, yg = x32[rows], yg[rows]
    rs = None if r is None else r.float().numpy()[rows]
    yo = O.linear_w8a16_rs(xs, qw, sw, None if b is None else b.numpy(), rs, out=yd).astype(np.float64)
    pre = O.linear_w8a16_rs(xs, qw, sw, None if b is None else b.numpy(), None, out=yd).astype(np.float64)
    x16s, e = O.rotate_rowscaled_f16(xs)
    s_main = (np.abs(x16s.astype(np.float64)) @ np.abs(qw.astype(np.float64)).T) * \
        sw.astype(np.float64)[None, :] * np.exp2(e.astype(np.float64))[:, None]
    tol = _ulp_out(pre, yd) + (_ulp_out(yo, yd) if res else 0.0) + _acc_c(K) * s_main
    assert np.isfinite(yg).all() and np.isfinite(yo).all()
    d = np.abs(yg - yo)
    viol = int((d > tol).sum())
    rel = float(np.linalg.norm(d) / np.linalg.norm(yo))
    _say(f"  violations {viol}, max |dY|/tol {float((d / tol).max()):.3f}, rel. Frobenius {rel:.2e}")
    # Both sides round the same nearly equal value once to the output type, so
    # they differ only where the fp32 accumulation moves it across a rounding
    # boundary of that type: rare, whether the type is fp16 or bf16.
    assert viol == 0 and rel <= 1e-3


def test_graph_replays_of_every_path_match_eager():
    # every entry point captured once in a HIP graph (with its workspace) and
    # replayed with eager calls in between: each replay equals the eager bits
    _say("graph replays: fused few-row, LoRA, residual, range-safe, dequantise-every-call")
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(DEV)
    K, N = 2048, 2048
    qw, sw = O.quantize_weights(wl.make_weights(N, K, seed=51).numpy())
    qw, sw = t(qw), t(sw)
    d, u = wl.make_lora(N, K, seed=51)
    lora = (d.to(DEV), u.to(DEV), 0.5)
    b = wl.make_bias(N, seed=51).to(DEV)
    xs = {M: wl.make_activations(M, K, seed=M).to(DEV) for M in (1, 16, 300)}
    res = wl.make_residual(300, N, seed=51).to(DEV)
    xb = xs[300].to(torch.bfloat16)
    wss = {
        "fused": torch.empty(cr.workspace_bytes(cr.PATH_W8A8, 1, N, K), dtype=torch.uint8, device=DEV),
        "lora16": torch.empty(cr.workspace_bytes(cr.PATH_W8A8, 16, N, K, 32), dtype=torch.uint8, device=DEV),
        "lora300": torch.empty(cr.workspace_bytes(cr.PATH_W8A8, 300, N, K, 32), dtype=torch.uint8, device=DEV),
        "rs": torch.empty(cr.workspace_bytes(cr.PATH_W8A16_RS, 300, N, K), dtype=torch.uint8, device=DEV),
        "dq": torch.empty(cr.workspace_bytes(cr.PATH_DEQUANT, 300, N, K), dtype=torch.uint8, device=DEV),
    }
    outs = {
        "fused": torch.empty((1, N), dtype=torch.float16, device=DEV),
        "lora16": torch.empty((16, N), dtype=torch.float16, device=DEV),
        "lora300": torch.empty((300, N), dtype=torch.float16, device=DEV),
        "rs": torch.empty((300, N), dtype=torch.bfloat16, device=DEV),
    }

    def calls():
        cr.linear_w8a8_ex(xs[1], qw, sw, bias=b, out=outs["fused"], workspace=wss["fused"])
        cr.linear_w8a8_ex(xs[16], qw, sw, bias=b, lora=lora, out=outs["lora16"], workspace=wss["lora16"])
        cr.linear_w8a8_ex(xs[300], qw, sw, bias=b, lora=lora, residual=res, out=outs["lora300"],
                          workspace=wss["lora300"])
        cr.linear_w8a16_rs(xb, qw, sw, bias=b, out=outs["rs"], workspace=wss["rs"])
        return cr.linear_dequant(xs[300], qw, sw, b, workspace=wss["dq"])

    ref_dq = calls().clone()
    torch.cuda.synchronize()
    ref = {k: v.clone() for k, v in outs.items()}
    stream = torch.cuda.Stream()
    with torch.cuda.stream(stream):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=stream):
            dq = calls()
    torch.cuda.synchronize()
    for rep in range(3):
        for v in outs.values():
            v.zero_()
        dq.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for k, v in outs.items():
            assert torch.equal(v.view(torch.int16), ref[k].view(torch.int16)), f"{k}, replay {rep}"
        assert torch.equal(dq.view(torch.int16), ref_dq.view(torch.int16)), f"dequant, replay {rep}"
        calls()                       # eager work between replays
        torch.cuda.synchronize()
    _say("  3 replays of 5 entry points equal to eager")


def test_empty_contraction_every_entry_point():
    # K = 0: every sum over k is empty (the oracle's reading of empty
    # contractions); outputs are pre-filled with NaN so that every element
    # must be written
    _say("K = 0 (empty contraction) on every entry point")
    M, N, R = 5, 24, 4
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(DEV)
    g = np.random.default_rng(0)
    bias_np = g.normal(size=N).astype(np.float32)
    bias_np[1] = -0.0
    bias_np[2] = 7e4     # rounds to fp16 inf
    bias = t(bias_np)
    res_np = g.normal(size=(M, N)).astype(np.float16)
    up_np = g.normal(size=(N, R)).astype(np.float32)
    x0 = torch.empty((M, 0), dtype=torch.float16, device=DEV)
    qw0, sw0 = cr.quantize_weights(torch.empty((N, 0), dtype=torch.float32, device=DEV))
    torch.cuda.synchronize()
    assert qw0.shape == (N, 0) and torch.equal(sw0.cpu(), torch.zeros(N))
    sw = t(g.random(N).astype(np.float32) * 0.01)   # any scale: K = 0 does not read it
    down0 = torch.empty((R, 0), dtype=torch.float32, device=DEV)
    lora = (down0, t(up_np), 0.5)
    x0n = np.zeros((M, 0), np.float16)
    qw0n = np.zeros((N, 0), np.int8)
    lora_n = (np.zeros((R, 0), np.float32), up_np, 0.5)

    def bits(a):
        a = np.asarray(a)
        return a.view(np.uint16) if a.dtype in (np.float16,) else a.view(np.uint8)

    def nan_out(dtype):
        return torch.full((M, N), float("nan"), dtype=dtype, device=DEV)

    y = cr.linear_w8a8(x0, qw0, sw, bias)
    exp = O.linear_w8a8(x0n, qw0n, sw.cpu().numpy(), bias_np)[0]
    assert np.array_equal(bits(_np(y)), bits(exp))
    y = cr.linear_w8a8_ex(x0, qw0, sw, bias=bias, lora=lora, residual=t(res_np), out=nan_out(torch.float16))
    exp = O.linear_w8a8_ex(x0n, qw0n, sw.cpu().numpy(), bias_np, lora_n, res_np)
    assert np.array_equal(bits(_np(y)), bits(exp))
    r = t(res_np)
    cr.linear_w8a8_ex(x0, qw0, sw, bias=bias, residual=r, out=r)       # in place
    assert np.array_equal(bits(_np(r)), bits(O.linear_w8a8_ex(x0n, qw0n, sw.cpu().numpy(), bias_np, None, res_np)))
    y = cr.linear_w8a16(x0, qw0, sw, bias, lora=lora)
    exp = O.linear_w8a16(x0n, qw0n, sw.cpu().numpy(), bias_np, lora_n)
    assert np.array_equal(bits(_np(y)), bits(exp))
    y = cr.linear_dequant(x0, qw0, sw, bias)
    assert np.array_equal(bits(_np(y)), bits(O.linear_dequant(x0n, qw0n, sw.cpu().numpy(), bias_np)))
    for dt, name in ((torch.float16, "f16"), (torch.bfloat16, "bf16")):
        res_t = t(res_np).to(dt)
        res_ref = res_t.float().cpu().numpy()
        y = cr.linear_w8a16_rs(x0.to(dt), qw0, sw, bias, residual=res_t, out=torch.full((M, N), float("nan"),
                               dtype=dt, device=DEV))
        exp = O.linear_w8a16_rs(x0n, qw0n, sw.cpu().numpy(), bias_np, res_ref, out=name)
        assert np.array_equal(y.float().cpu().numpy().view(np.uint32), np.asarray(exp, np.float32).view(np.uint32)), name
    q, s = cr.act_quant(x0)
    assert q.shape == (M, 0) and torch.equal(s.cpu(), torch.zeros(M))
    assert cr.act_rotate_f16(x0).shape == (M, 0)
    x16, e = cr.act_rotate_scaled(x0)
    assert x16.shape == (M, 0) and torch.equal(e.cpu(), torch.zeros(M, dtype=torch.int32))
    a = cr.gemm_i8_i32(q, qw0)
    assert torch.equal(a.cpu(), torch.zeros((M, N), dtype=torch.int32))
    y = cr.gemm_i8_f16(q, s, qw0, sw, bias)
    assert np.array_equal(bits(_np(y)), bits(O.epilogue_w8a8(np.zeros((M, N), np.int64), np.zeros(M, np.float32),
                                                             sw.cpu().numpy(), bias_np)))
    y = cr.gemm_f16(x0, torch.empty((N, 0), dtype=torch.float16, device=DEV))
    assert torch.equal(y.cpu().view(torch.int16), torch.zeros((M, N), dtype=torch.int16))
    assert cr.dequantize_weights(qw0, sw).shape == (N, 0)
    torch.cuda.synchronize()
    _say("  every entry point bit-exact at K = 0")


def test_concurrent_host_threads_on_separate_streams():
    # the library is documented thread-safe: four host threads issue W8A8 and
    # weight-only calls on their own streams (own workspaces and outputs);
    # every result equals the single-threaded one bit for bit
    import threading
    _say("concurrent host threads, one stream each")
    shapes = [(300, 2048, 8192), (64, 6144, 256), (1024, 256, 2048), (5, 2048, 4096)]
    cases = []
    for i, (M, N, K) in enumerate(shapes):
        x = wl.make_activations(M, K, seed=40 + i).to(DEV)
        qw, sw = cr.quantize_weights(wl.make_weights(N, K, seed=40 + i).to(DEV))
        cases.append((x, qw, sw))
    torch.cuda.synchronize()
    ref = [(cr.linear_w8a8(x, qw, sw), cr.linear_w8a16(x, qw, sw)) for (x, qw, sw) in cases]
    torch.cuda.synchronize()
    results, errors = [None] * len(cases), []

    def work(i):
        try:
            x, qw, sw = cases[i]
            s = torch.cuda.Stream()
            with torch.cuda.stream(s):
                outs = []
                for _ in range(5):
                    outs = [cr.linear_w8a8(x, qw, sw), cr.linear_w8a16(x, qw, sw)]
            s.synchronize()
            results[i] = outs
        except Exception as e:   # reported below, on the main thread
            errors.append(repr(e))

    threads = [threading.Thread(target=work, args=(i,)) for i in range(len(cases))]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    torch.cuda.synchronize()
    assert not errors, errors
    for (r8, r16), (g8, g16) in zip(ref, results):
        assert torch.equal(r8.view(torch.int16), g8.view(torch.int16))
        assert torch.equal(r16.view(torch.int16), g16.view(torch.int16))
    _say("  4 threads x 5 calls equal to the single-threaded results")


@pytest.mark.parametrize("M,K", [(2051, 2048), (1001, 8192)])
def test_weight_only_prologues_many_blocks(M, K):
    # the weight-only and range-safe prologues with more row blocks than
    # resident workgroups (each workgroup walks several blocks)
    _say(f"weight-only prologues, many blocks M={M} K={K}")
    x = wl.make_activations(M, K, seed=M + K)
    x16 = _np(cr.act_rotate_f16(x.to(DEV)))
    assert np.array_equal(x16.view(np.uint16), O.rotate_activations_f16(x.numpy()).view(np.uint16))
    xs, e = cr.act_rotate_scaled(x.to(DEV))
    xo, eo = O.rotate_rowscaled_f16(x.numpy().astype(np.float32))
    assert np.array_equal(_np(xs).view(np.uint16), xo.view(np.uint16))
    assert np.array_equal(_np(e).astype(np.int64), eo)


# ------------------------- activation rows written in XCD row bands
# Where the prologue's grid holds every row block once, the linear calls
# write Q_X (or X16) in 8 row bands, band x by the workgroups on XCD x, and
# the GEMM's tile order gives each XCD those rows.  Only the assignment of
# blocks and tiles to workgroups changes, so the result must equal the
# stand-alone prologue + GEMM (interleaved rows, default order) bit for bit,
# and every row must equal the same row computed in a call whose M does not
# split into bands.  Shapes: the three banded sweep layers, the 256-row tile
# (fewer than 8 row tiles), more tiles than CUs (M = 2048), K = 4096, and
# row counts that do not band.

@pytest.mark.gpu
@pytest.mark.parametrize("M,N,K", [(1024, 2048, 2048), (1024, 256, 2048), (1024, 2048, 1024), (1024, 8192, 2048),
                                   (2048, 2048, 2048), (512, 1024, 4096), (1000, 2048, 2048)])
def test_linear_w8a8_xcd_bands_equal_staged_calls(M, N, K):
    _say(f"linear w8a8 XCD row bands M={M} N={N} K={K}")
    x = wl.make_activations(M, K, seed=M + N + K).to(DEV)
    qw, sw = cr.quantize_weights(wl.make_weights(N, K, seed=N + K).to(DEV))
    b = wl.make_bias(N, seed=K).to(DEV)
    y = cr.linear_w8a8(x, qw, sw, bias=b)
    qx, sx = cr.act_quant(x)
    ys = cr.gemm_i8_f16(qx, sx, qw, sw, bias=b)
    torch.cuda.synchronize()
    assert torch.equal(y.view(torch.int16), ys.view(torch.int16))


@pytest.mark.gpu
@pytest.mark.parametrize("path", ["w8a8", "w8a16", "w8a16_rs"])
def test_linear_xcd_bands_rows_independent_of_m(path):
    # M = 1024 bands (K = 2048: 16 rows per band unit); M = 1032 does not.
    # The first 1024 rows of both calls must be identical.
    _say(f"linear {path} rows under XCD bands equal the unbanded call's")
    N, K = 2048, 2048
    x = wl.make_activations(1032, K, seed=11).to(DEV)
    qw, sw = cr.quantize_weights(wl.make_weights(N, K, seed=12).to(DEV))
    if path == "w8a8":
        f = lambda t: cr.linear_w8a8(t, qw, sw)
    elif path == "w8a16":
        f = lambda t: cr.linear_w8a16(t, qw, sw)
    else:
        f = lambda t: cr.linear_w8a16_rs(t, qw, sw)
    y_band = f(x[:1024].contiguous())
    y_all = f(x)
    torch.cuda.synchronize()
    assert torch.equal(y_band.view(torch.int16), y_all[:1024].view(torch.int16))
