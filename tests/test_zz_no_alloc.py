"""The allocation-free W8A8 entry point against the workspace one.

convrot_linear_w8a8_noalloc keeps Q_X, s_X and any K-split partials in the
library's fixed per-GPU scratch; its output must equal convrot_linear_w8a8's
bit for bit (the W8A8 output is exact under the library's arithmetic
contract).  Calls follow each other on one stream with a smaller problem
second, so the second reads a scratch that still holds the first call's data.
"""

import numpy as np
import pytest
import torch

import rotation_quantized_int8_amd as cr
import workload as wl

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
TOO_LARGE = 7


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    cr.lib()
    torch.cuda.set_device(0)


def _problem(M, N, K, seed):
    x = wl.make_activations(M, K, seed=seed).to(DEV)
    qw, sw = cr.quantize_weights(wl.make_weights(N, K, seed=seed).to(DEV))
    b = wl.make_bias(N, seed=seed).to(DEV)
    return x, qw, sw, b


def _with_workspace(L, x, qw, sw, b, h):
    M, K = x.shape
    N = qw.shape[0]
    y = torch.empty((M, N), dtype=torch.float16, device=DEV)
    ws = torch.empty(max(cr.workspace_bytes(cr.PATH_W8A8, M, N, K), 16), dtype=torch.uint8, device=DEV)
    st = L.convrot_linear_w8a8(x.data_ptr(), M, K, qw.data_ptr(), sw.data_ptr(), N, b.data_ptr(),
                               y.data_ptr(), ws.data_ptr(), ws.numel(), h)
    assert st == 0, L.convrot_status_string(st)
    return y


def _noalloc(L, x, qw, sw, b, y, h):
    M, K = x.shape
    N = qw.shape[0]
    return L.convrot_linear_w8a8_noalloc(x.data_ptr(), M, K, qw.data_ptr(), sw.data_ptr(), N, b.data_ptr(),
                                         y.data_ptr(), h)


# (first, second): the second call is smaller.  Paths: the tiled GEMM
# (1024 rows), the few-row GEMM with int32 K-split partials in the scratch
# (16 x 2048 x 8192: 4 K ranges), the few-row kernel, the one-launch path for
# few short rows, and the one-launch paths for K = 256 and for narrow
# layers (each workgroup quantises its own band of rows; no scratch), each
# followed by a ragged one.
PAIRS = [((1024, 2048, 2048), (300, 203, 768)),
         ((1024, 8192, 2048), (16, 2048, 8192)),
         ((16, 2048, 8192), (4, 256, 8192)),
         ((4094, 2048, 8192), (1, 8192, 2048)),
         ((1024, 6144, 256), (100, 252, 256)),
         ((1024, 256, 1024), (100, 132, 512))]


@pytest.mark.parametrize("first,second", PAIRS)
def test_noalloc_matches_workspace_entry_point(first, second):
    L = cr.lib()
    print(f"no-alloc pair {first} then {second}", flush=True)
    h = torch.cuda.current_stream().cuda_stream
    probs = [_problem(*first, seed=1), _problem(*second, seed=2)]
    outs = []
    for (x, qw, sw, b) in probs:
        y = torch.full((x.shape[0], qw.shape[0]), float("nan"), dtype=torch.float16, device=DEV)
        st = _noalloc(L, x, qw, sw, b, y, h)
        assert st == 0, L.convrot_status_string(st)
        outs.append(y)
    refs = [_with_workspace(L, *p, h) for p in probs]
    torch.cuda.synchronize()
    for y, r in zip(outs, refs):
        assert torch.equal(y.view(torch.int16), r.view(torch.int16))


def test_noalloc_repeated_on_one_stream_and_too_large():
    L = cr.lib()
    print("no-alloc repeated calls; too-large problem refused", flush=True)
    h = torch.cuda.current_stream().cuda_stream
    big, small = _problem(1024, 2048, 8192, seed=3), _problem(64, 256, 256, seed=4)
    rb, rs = _with_workspace(L, *big, h), _with_workspace(L, *small, h)
    yb = torch.empty_like(rb)
    ys = torch.empty_like(rs)
    for _ in range(3):
        assert _noalloc(L, *big, yb, h) == 0
        assert _noalloc(L, *small, ys, h) == 0
    torch.cuda.synchronize()
    assert torch.equal(yb.view(torch.int16), rb.view(torch.int16))
    assert torch.equal(ys.view(torch.int16), rs.view(torch.int16))
    # 4095 rows of 8192 need more than the 32 MiB scratch: refused, nothing written
    x = torch.zeros((4095, 8192), dtype=torch.float16, device=DEV)
    qw = torch.zeros((8, 8192), dtype=torch.int8, device=DEV)
    sw = torch.zeros(8, dtype=torch.float32, device=DEV)
    b = torch.zeros(8, dtype=torch.float32, device=DEV)
    y = torch.full((4095, 8), 7.0, dtype=torch.float16, device=DEV)
    assert _noalloc(L, x, qw, sw, b, y, h) == TOO_LARGE
    torch.cuda.synchronize()
    assert bool((y == 7.0).all())
