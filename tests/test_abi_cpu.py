"""Host-side checks of the C ABI: the library loads, exports every function
that include/convrot.h declares, and rejects bad arguments before touching a
GPU (every call here returns from the host-side checks; no kernel runs)."""

import ctypes
import os

import pytest

import rotation_quantized_int8_amd as cr
from rotation_quantized_int8_amd import build as crbuild

OK, INVALID, SHAPE, ALIGN, DEVICE, LAUNCH, WORKSPACE, TOO_LARGE = range(8)


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(cr.LIB_PATH):
        crbuild.build()
    return cr.lib()


def test_exports_every_declared_symbol(L):
    declared = cr.header_functions()
    assert len(declared) == 17
    for name in declared:
        assert hasattr(L, name), name
    assert set(declared) == set(cr._SIGNATURES)


def test_version_and_status_strings(L):
    assert L.convrot_abi_version() == 1
    for s in range(8):
        assert L.convrot_status_string(s)
    assert b"unknown" in L.convrot_status_string(99)


def test_workspace_bytes(L):
    assert L.convrot_workspace_bytes(0, 1024, 2048, 2048, 0) == 1024 * 2048 + 4096
    assert L.convrot_workspace_bytes(0, 3, 5, 256, 0) == 768 + 256
    assert L.convrot_workspace_bytes(1, 4, 8, 256, 0) == 2048
    # W8A16 with LoRA: X16, T fp16 [M, 32], U' fp16 [N, 32] (256-byte pieces)
    assert L.convrot_workspace_bytes(1, 4, 8, 256, 32) == 2048 + 256 + 512
    assert L.convrot_workspace_bytes(0, 0, 5, 256, 0) == 0
    # few rows: with 16 rows the 32x32-tile GEMM streams 512 KiB per tile at
    # K = 8192 over only 64 tiles, so K is split 4 ways into int32 partials ...
    assert L.convrot_workspace_bytes(0, 16, 2048, 8192, 0) == 16 * 8192 + 256 + 4 * 16 * 2048 * 4
    # ... and 8 ways for 256 outputs (8 tiles; ranges of at least 1024)
    assert L.convrot_workspace_bytes(0, 16, 256, 8192, 0) == 16 * 8192 + 256 + 8 * 16 * 256 * 4
    # up to 8 rows the few-row kernel: 2048 outputs need no K split ...
    assert L.convrot_workspace_bytes(0, 4, 2048, 8192, 0) == 4 * 8192 + 256
    # ... 256 outputs get 2 K ranges (a workgroup would stream > 64 KiB)
    assert L.convrot_workspace_bytes(0, 4, 256, 8192, 0) == 4 * 8192 + 256 + 2 * 4 * 256 * 4
    # with a LoRA the few-row kernel always goes through int32 partials
    assert L.convrot_workspace_bytes(0, 4, 2048, 8192, 32) == \
        4 * 8192 + 256 + 4 * 2048 * 4 + 4 * 32 * 2 + 2048 * 32 * 2 + 32 * 4 * 32 * 4
    # the K-split GEMM with a LoRA
    assert L.convrot_workspace_bytes(0, 16, 2048, 8192, 32) == \
        16 * 8192 + 256 + 4 * 16 * 2048 * 4 + 16 * 32 * 2 + 2048 * 32 * 2 + 32 * 16 * 32 * 4
    # a LoRA adds its fp16 low-rank activation [M, t_ld], the fp16 scaled up
    # weight [N, t_ld] (t_ld = rank rounded up to 32) and, when K spans
    # several 256-column chunks, fp32 partial sums per K range
    # (M = 3 with a LoRA: also the int32 product of the few-row kernel)
    assert L.convrot_workspace_bytes(0, 3, 5, 256, 17) == 768 + 256 + 256 + 256 + 512
    assert L.convrot_workspace_bytes(0, 1024, 2048, 2048, 64) == \
        1024 * 2048 + 4096 + 1024 * 64 * 2 + 2048 * 64 * 2 + 8 * 1024 * 64 * 4
    bad = ctypes.c_size_t(-1).value
    assert L.convrot_workspace_bytes(0, 4, 4, 255, 0) == bad
    assert L.convrot_workspace_bytes(0, 4, 4, 131072 + 256, 0) == bad
    assert L.convrot_workspace_bytes(0, -1, 4, 256, 0) == bad
    assert L.convrot_workspace_bytes(1, 4, 4, 256, 65) == bad
    assert L.convrot_workspace_bytes(7, 4, 4, 256, 0) == bad
    # dequantise-every-call: the fp16 weight [N, K]
    assert L.convrot_workspace_bytes(2, 4, 8, 256, 0) == 8 * 256 * 2
    assert L.convrot_workspace_bytes(2, 4, 8, 256, 4) == bad
    # range-safe weight-only: fp16 activation [M, K] and the row exponents [M]
    assert L.convrot_workspace_bytes(3, 4, 8, 256, 0) == 2048 + 256
    assert L.convrot_workspace_bytes(3, 4, 8, 256, 1) == bad
    # K = 0 (an empty contraction) needs no workspace on any path
    for path in (0, 1, 2, 3):
        assert L.convrot_workspace_bytes(path, 4, 8, 0, 0) == 0
    assert L.convrot_workspace_bytes(0, 4, 8, 0, 32) == 0
    assert L.convrot_workspace_bytes(1, 4, 8, 0, 32) == 0
    assert L.convrot_workspace_bytes(2, 4, 8, 0, 1) == bad
    assert L.convrot_workspace_bytes(3, 4, 8, 0, 1) == bad
    assert L.convrot_workspace_bytes(0, 4, 8, -256, 0) == bad


P = 1 << 20          # a fake, 16-byte aligned "device" address: never dereferenced
Q = 1 << 24
R = 1 << 28
S = 1 << 30


def test_linear_w8a8_argument_errors(L):
    f = L.convrot_linear_w8a8
    ws = L.convrot_workspace_bytes(0, 4, 8, 256, 0)
    # empty problems succeed without touching anything
    assert f(None, 0, 256, None, None, 8, None, None, None, 0, None) == OK
    assert f(None, 4, 256, None, None, 0, None, None, None, 0, None) == OK
    # shapes
    assert f(P, 4, 255, Q, R, 8, None, S, S + 4096, ws, None) == SHAPE
    assert f(P, -1, 256, Q, R, 8, None, S, S + 4096, ws, None) == SHAPE
    assert f(P, 4, 131072 + 256, Q, R, 8, None, S, S + 4096, ws, None) == SHAPE
    # null pointers
    assert f(None, 4, 256, Q, R, 8, None, S, S + 4096, ws, None) == INVALID
    assert f(P, 4, 256, Q, R, 8, None, None, S + 4096, ws, None) == INVALID
    # alignment
    assert f(P + 2, 4, 256, Q, R, 8, None, S, S + 4096, ws, None) == ALIGN
    assert f(P, 4, 256, Q, R, 8, R + 4096 + 4, S, S + 4096, ws, None) == ALIGN
    # workspace
    assert f(P, 4, 256, Q, R, 8, None, S, None, ws, None) == WORKSPACE
    assert f(P, 4, 256, Q, R, 8, None, S, S + 4096, ws - 1, None) == WORKSPACE
    # output overlapping an input or the workspace
    assert f(P, 4, 256, Q, R, 8, None, P + 16, S + 4096, ws, None) == INVALID
    assert f(P, 4, 256, Q, R, 8, None, S, S, ws, None) == INVALID
    assert f(P, 4, 256, Q, R, 8, None, S, P, ws, None) == INVALID


def test_linear_w8a8_noalloc_argument_errors(L):
    f = L.convrot_linear_w8a8_noalloc
    assert f(None, 0, 256, None, None, 8, None, None, None) == OK
    assert f(None, 4, 256, None, None, 0, None, None, None) == OK
    assert f(P, 4, 255, Q, R, 8, None, S, None) == SHAPE
    assert f(P, -1, 256, Q, R, 8, None, S, None) == SHAPE
    assert f(P, 4, 131072 + 256, Q, R, 8, None, S, None) == SHAPE
    assert f(None, 4, 256, Q, R, 8, None, S, None) == INVALID
    assert f(P, 4, 256, Q, R, 8, None, None, None) == INVALID
    assert f(P + 2, 4, 256, Q, R, 8, None, S, None) == ALIGN
    assert f(P, 4, 256, Q, R, 8, R + 4096 + 4, S, None) == ALIGN
    assert f(P, 4, 256, Q, R, 8, None, P + 16, None) == INVALID
    # the fixed scratch holds Q_X and s_X (256-byte pieces) of at most 32 MiB:
    # 4094 rows of 8192 fill it exactly, 4095 rows do not fit
    cap = 32 << 20
    assert L.convrot_workspace_bytes(0, 4094, 8, 8192, 0) == cap
    assert L.convrot_workspace_bytes(0, 4095, 8, 8192, 0) > cap
    assert f(P, 4095, 8192, Q, R, 8, None, S, None) == TOO_LARGE
    assert f(P, 8192, 8192, Q, R, 8, None, S, None) == TOO_LARGE
    assert f(None, 4095, 8192, None, None, 8, None, None, None) == TOO_LARGE
    # a size that fits passes every host check and stops at the device check
    # (no GPU in the CPU suite)
    assert f(P, 4094, 8192, Q, R, 8, None, S, None) in (DEVICE, OK)


def test_linear_w8a8_ex_argument_errors(L):
    f = L.convrot_linear_w8a8_ex
    ws = L.convrot_workspace_bytes(0, 4, 8, 256, 0)
    Y, W = S, S + 4096
    # (no call here may pass every host check: with a GPU present it would
    # launch kernels on these fake addresses)
    assert f(None, 0, 256, None, None, 8, None, None, None, None, None, 0, None) == OK
    # residual: alignment, partial overlap with Y, overlap with the workspace
    assert f(P, 4, 256, Q, R, 8, None, None, Y + 8, Y, W, ws, None) == ALIGN
    assert f(P, 4, 256, Q, R, 8, None, None, Y + 16, Y, W, ws, None) == INVALID
    assert f(P, 4, 256, Q, R, 8, None, None, W + 256, Y, W, ws, None) == INVALID
    # LoRA: rank, null factors, alignment, workspace sized for the rank
    lora = cr._Lora(P + 65536, Q + 65536, 0, 1.0)
    assert f(P, 4, 256, Q, R, 8, None, ctypes.byref(lora), None, Y, W, ws, None) == SHAPE
    lora.rank = 65
    assert f(P, 4, 256, Q, R, 8, None, ctypes.byref(lora), None, Y, W, ws, None) == SHAPE
    lora.rank, lora.up = 4, None
    assert f(P, 4, 256, Q, R, 8, None, ctypes.byref(lora), None, Y, W, ws, None) == INVALID
    lora.up = Q + 65536 + 4
    wsl = L.convrot_workspace_bytes(0, 4, 8, 256, 4)
    assert f(P, 4, 256, Q, R, 8, None, ctypes.byref(lora), None, Y, W, wsl, None) == ALIGN
    lora.up = Q + 65536
    assert wsl > ws
    assert f(P, 4, 256, Q, R, 8, None, ctypes.byref(lora), None, Y, W, ws, None) == WORKSPACE
    # output overlapping a LoRA factor
    lora.down = Y + 256
    assert f(P, 4, 256, Q, R, 8, None, ctypes.byref(lora), None, Y, W, wsl, None) == INVALID


def test_linear_w8a16_argument_errors(L):
    f = L.convrot_linear_w8a16
    lora = cr._Lora(P, Q, 0, 1.0)
    ws = L.convrot_workspace_bytes(1, 4, 8, 256, 0)
    assert f(P, 4, 256, Q, R, 8, None, ctypes.byref(lora), S, S + 4096, ws, None) == SHAPE
    lora.rank = 65
    assert f(P, 4, 256, Q, R, 8, None, ctypes.byref(lora), S, S + 4096, ws, None) == SHAPE
    lora.rank, lora.down = 4, None
    assert f(P, 4, 256, Q, R, 8, None, ctypes.byref(lora), S, S + 4096, ws, None) == INVALID
    lora.down = P + 65536 + 8
    wsl = L.convrot_workspace_bytes(1, 4, 8, 256, 4)
    assert f(P, 4, 256, Q, R, 8, None, ctypes.byref(lora), S, S + 4096, wsl, None) == ALIGN
    assert f(P, 4, 256, Q, R, 8, None, None, S, S + 4096, ws - 16, None) == WORKSPACE
    assert f(None, 0, 256, None, None, 8, None, None, None, None, 0, None) == OK


def test_dequant_argument_errors(L):
    f = L.convrot_linear_dequant
    ws = L.convrot_workspace_bytes(2, 4, 8, 256, 0)
    assert f(None, 0, 256, None, None, 8, None, None, None, 0, None) == OK
    assert f(P, 4, 300, Q, R, 8, None, S, S + 8192, ws, None) == SHAPE
    assert f(P, 4, 256, Q, R, 8, None, None, S + 8192, ws, None) == INVALID
    assert f(P, 4, 256, Q, R, 8, R + 4096 + 8, S, S + 8192, ws, None) == ALIGN
    assert f(P, 4, 256, Q, R, 8, None, S, S + 8192, ws - 1, None) == WORKSPACE
    assert f(P, 4, 256, Q, R, 8, None, S, S, ws, None) == INVALID        # Y inside the workspace
    assert f(P, 4, 256, Q, R, 8, None, S, Q, ws, None) == INVALID        # workspace over Q_W
    d = L.convrot_dequantize_weights
    assert d(None, None, 0, 256, None, None) == OK
    assert d(P, Q, 8, 255, R, None) == SHAPE
    assert d(P, Q, 8, 256, None, None) == INVALID
    assert d(P, Q, 8, 256, P + 16, None) == INVALID
    assert d(P, Q + 4, 8, 256, R, None) == ALIGN


def test_w8a16_rs_argument_errors(L):
    f = L.convrot_linear_w8a16_rs
    ws = L.convrot_workspace_bytes(3, 4, 8, 256, 0)
    Y, W = S, S + 4096
    assert f(None, 0, 0, 256, None, None, 8, None, None, None, 0, None, 0, None) == OK
    assert f(P, 2, 4, 256, Q, R, 8, None, None, Y, 0, W, ws, None) == INVALID        # bad x dtype
    assert f(P, 0, 4, 256, Q, R, 8, None, None, Y, 5, W, ws, None) == INVALID        # bad y dtype
    assert f(P, 1, 4, 300, Q, R, 8, None, None, Y, 1, W, ws, None) == SHAPE
    assert f(P, 1, 4, 256, Q, R, 8, None, Y + 8, Y, 1, W, ws, None) == ALIGN         # residual alignment
    assert f(P, 1, 4, 256, Q, R, 8, None, Y + 16, Y, 1, W, ws, None) == INVALID      # residual overlaps Y
    assert f(P, 1, 4, 256, Q, R, 8, None, None, Y, 1, W, ws - 1, None) == WORKSPACE
    assert f(P, 1, 4, 256, Q, R, 8, None, None, W, 1, W, ws, None) == INVALID        # Y in the workspace
    a = L.convrot_act_rotate_scaled
    assert a(P, 3, 4, 256, Q, R, None) == INVALID
    assert a(P, 1, 4, 255, Q, R, None) == SHAPE
    assert a(P, 1, 4, 256, Q, R + 4, None) == ALIGN
    assert a(P, 1, 4, 256, P + 512, R, None) == INVALID


def test_stage_argument_errors(L):
    assert L.convrot_act_quant(P, 4, 300, Q, R, None) == SHAPE
    assert L.convrot_act_quant(P, 4, 256, None, R, None) == INVALID
    assert L.convrot_act_quant(P, 4, 256, Q + 1, R, None) == ALIGN
    assert L.convrot_act_quant(P, 4, 256, P + 256, R, None) == INVALID
    assert L.convrot_act_quant(None, 0, 256, None, None, None) == OK
    assert L.convrot_act_rotate_f16(P, 4, 256, P, None) == INVALID
    assert L.convrot_gemm_i8_i32(P, Q, 4, 8, 257, R, None) == SHAPE
    assert L.convrot_gemm_i8_i32(P, Q, 4, 8, 256, P, None) == INVALID
    assert L.convrot_gemm_i8_f16(P, Q, R, S, None, 4, 8, 256, None, None) == INVALID
    assert L.convrot_gemm_f16(P, Q, 4, 8, 256, R + 8, None) == ALIGN
    assert L.convrot_quantize_weights(P, 8, 256, Q, Q + 16, None) == INVALID
    assert L.convrot_quantize_weights(P, -8, 256, Q, R, None) == SHAPE
    assert L.convrot_quantize_weights(None, 0, 256, None, None, None) == OK


def test_empty_contraction_argument_errors(L):
    # K = 0: X, Q_X, Q_W and lora.down have no elements and may be NULL, but
    # the scales, the output and the other operands with elements are checked
    # as usual (every call here fails before the device check)
    f = L.convrot_linear_w8a8
    assert f(None, 4, 0, None, None, 8, None, S, None, 0, None) == INVALID       # s_W
    assert f(None, 4, 0, None, R, 8, None, None, None, 0, None) == INVALID       # Y
    assert f(None, 4, 0, None, R, 8, None, S + 2, None, 0, None) == ALIGN
    assert f(None, 4, 0, None, R, 8, R + 4, S, None, 0, None) == ALIGN         # bias
    assert f(None, 4, 0, None, R, 8, S + 16, S, None, 0, None) == INVALID      # bias inside Y
    assert f(None, 4, 0, None, S + 32, 8, None, S, None, 0, None) == INVALID   # s_W inside Y
    fx = L.convrot_linear_w8a8_ex
    Y = S
    lora = cr._Lora(None, None, 4, 1.0)
    assert fx(None, 4, 0, None, R, 8, None, ctypes.byref(lora), None, Y, None, 0, None) == INVALID  # up
    lora = cr._Lora(None, Q, 0, 1.0)
    assert fx(None, 4, 0, None, R, 8, None, ctypes.byref(lora), None, Y, None, 0, None) == SHAPE
    lora = cr._Lora(None, Y + 16, 4, 1.0)
    assert fx(None, 4, 0, None, R, 8, None, ctypes.byref(lora), None, Y, None, 0, None) == INVALID
    assert fx(None, 4, 0, None, R, 8, None, None, Y + 2, Y, None, 0, None) == ALIGN   # residual
    assert fx(None, 4, 0, None, R, 8, None, None, Y + 16, Y, None, 0, None) == INVALID
    assert L.convrot_linear_w8a16(None, 4, 0, None, None, 8, None, None, Y, None, 0, None) == INVALID
    assert L.convrot_linear_dequant(None, 4, 0, None, R, 8, None, None, None, 0, None) == INVALID
    assert L.convrot_linear_w8a16_rs(None, 0, 4, 0, None, R, 8, None, None, None, 1, None, 0, None) == INVALID
    assert L.convrot_linear_w8a16_rs(None, 2, 4, 0, None, R, 8, None, None, Y, 1, None, 0, None) == INVALID
    assert L.convrot_quantize_weights(None, 8, 0, None, None, None) == INVALID  # s_W
    assert L.convrot_quantize_weights(None, 8, 0, None, R + 4, None) == ALIGN
    assert L.convrot_act_quant(None, 4, 0, None, None, None) == INVALID          # s_X
    assert L.convrot_act_rotate_scaled(None, 0, 4, 0, None, None, None) == INVALID  # e
    assert L.convrot_gemm_i8_i32(None, None, 4, 8, 0, None, None) == INVALID     # A
    assert L.convrot_gemm_i8_f16(None, None, None, R, None, 4, 8, 0, S, None) == INVALID   # s_X
    assert L.convrot_gemm_i8_f16(None, P, None, None, None, 4, 8, 0, S, None) == INVALID   # s_W
    assert L.convrot_gemm_f16(None, None, 4, 8, 0, None, None) == INVALID        # Y
    assert L.convrot_gemm_f16(None, None, 4, 8, 0, S + 8, None) == ALIGN
    assert L.convrot_quantize_weights(None, 8, -256, None, R, None) == SHAPE


def test_python_wrapper_refuses_cpu_tensors():
    import torch
    with pytest.raises((ValueError, TypeError)):
        cr.linear_w8a8(torch.zeros(4, 256, dtype=torch.float16),
                       torch.zeros(8, 256, dtype=torch.int8), torch.zeros(8))
