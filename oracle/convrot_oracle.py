"""CPU oracle for the INT8ConvRot linear layer -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import or call this module.  The product (the HIP library and
its Python binding) never does, and this module imports nothing from it.

It is a plain, slow, obviously correct restatement of what the layer computes,
written from the pages, in float64 / exact integer arithmetic with one stated
rounding per step.  Citations name a page by tag:

  [P1] "INT8ConvRot GEMM vs fp16 on M1 Max with Metal, MPSMatrix, and MLX
       (fp16 Wins)" (lilting.ch, English article).
  [P4] "[PR #249] Add an mps backend: weight-only INT8 and W4A8/W6A8 linears
       for Apple GPUs" (comfy-kitchen pull request mirror).

[P1] section "What changed in the computation" fixes the method:
  * H: Kronecker products of 4x4 Hadamard matrices up to 256x256, divided by
    sqrt(256) = 16; symmetric with HH = I; applied to the last dimension in
    groups of 256 elements.
  * weights, once at model creation: W_rot = W H^T, s_W[n] = max_k|W_rot[n,k]|/127,
    Q_W = round(W_rot / s_W), clamped to [-128, 127], one scale per output channel.
  * activations, every call: X_rot = X H, s_X[m] = max_k|X_rot[m,k]|/127,
    Q_X = round(X_rot / s_X), clamped to [-128, 127].
  * A = Q_X Q_W^T in int32, Y = A (.) s_X s_W^T (outer product of the scales).
The same section gives the weight-only (W8A16) variant: the activations are
rotated and kept in fp16 and multiplied by the int8 weights and their
per-channel scale.  [P4] section "Design" adds the unmerged LoRA
(lora_down [R, K], lora_up [N, R], lora_scale) to that linear.

Readings where the pages leave a step open:
  R1  the 4x4 Hadamard is Sylvester's [[1,1],[1,-1]] (x) [[1,1],[1,-1]];
  R2  "round" is round-half-to-even, and every division is an IEEE fp32 division;
  R3  W_rot and X_rot are the exact products rounded once to fp32; s and Q are
      then computed from those fp32 values in fp32 arithmetic;
  R4  s is per row over the whole row (all K/256 groups); an all-zero row has
      s = 0 and Q = 0;
  R5  Y = fp16( fp32(A) * fp32(s_X[m] * s_W[n]) [+ bias[n]] ), each operation an
      fp32 operation with round-to-nearest-even, the scale product formed first;
  R6  W8A16: X16 = fp16(exact X H); Y = fp16(exact s_W[n] * sum_k X16 Q_W
      + lora_scale * (X D^T) U^T + bias), the LoRA term on the unrotated X and D;
  R7  K must be a multiple of 256 and at most 131072 (so |A| < 2^31);
  R8  the W8A8 layer with its extras ([P4] "Design": bias and residual added
      in eager's order; [P4] "What": the unmerged LoRA of the int8 linear):
      the linear's own output is formed first -- R5's fp32 value with the bias,
      plus, when a LoRA is given, the exact term scale * (X D^T) U^T, rounded
      once to fp16 -- and the residual is then added as one fp16 tensor
      addition (the exact sum of the two fp16 values, rounded once to fp16);
  R10 the dequantise-every-call baseline ([P1] "What changed in the
      computation": the earlier patch turned Q_W (.) s_W back into fp16,
      un-rotated it and ran the plain X W^T): W_deq = fp16(exact (Q_W (.) s_W) H),
      one rounding (H is its own inverse), then Y = fp16(exact X W_deq^T + bias);
  R11 the range-safe weight-only path ([P4] "Design", range safety by
      construction): each activation row (fp16 or bf16) is rotated exactly and
      divided by 2^e_m, e_m the smallest integer with max|X_rot[m,:]| <= 2^e_m
      (0 for a zero row), before the one rounding to fp16; the epilogue
      multiplies by 2^e_m again, so Y = out(exact 2^e_m s_W[n] sum_k X16s Q_W
      + bias) with one rounding to the output type (fp16 or bf16), and a
      residual is one addition in that type.  The fp32 accumulation of the
      MFMA path has no K limit (the pages' fp16 accumulation needs fp32 for
      K > 65504).
  R12 an empty contraction ([P4], the commit that returns empty contractions
      early): with K = 0 every sum over k is empty, so A = 0, a row maximum is
      0 (a zero row in R4's sense: s = 0, e = 0) and the LoRA term is 0; each
      path's formula then gives Y = out(+0 + bias), or +0 without a bias, with
      a residual added as usual.  K = 0 is therefore a valid size.
"""

from __future__ import annotations

import math

import numpy as np

GROUP = 256
K_MAX = 131072
QMAX = 127.0

# ---------------------------------------------------------------------------
# exact rounding to a binary floating-point format
# ---------------------------------------------------------------------------

F32 = (24, -126, 127)     # (significand bits p, emin, emax)
F16 = (11, -14, 15)
BF16 = (8, -126, 127)


def round_scaled_int(t: int, shift: int, fmt=F32) -> float:
    """Nearest value of format ``fmt`` (round half to even) to ``t * 2**-shift``.

    ``t`` is a Python integer, so the input is exact.  The result is returned
    as a Python float (both fp32 and fp16 embed exactly in float64); values at
    or beyond the rounding boundary above the largest finite number give +-inf
    as IEEE 754 round-to-nearest does.
    """
    p, emin, emax = fmt
    if t == 0:
        return 0.0
    sign = -1.0 if t < 0 else 1.0
    a = -t if t < 0 else t
    e = a.bit_length() - 1 - shift          # exponent of the leading bit
    qexp = max(e, emin) - (p - 1)           # exponent of one unit in the last place
    s = -shift - qexp                       # value / ulp = a * 2**s
    if s >= 0:
        q = a << s
    else:
        d = -s
        q, r = divmod(a, 1 << d)
        half = 1 << (d - 1)
        if r > half or (r == half and (q & 1)):
            q += 1
    if q.bit_length() + qexp > emax + 1:    # q * 2**qexp >= 2**(emax + 1)
        return sign * math.inf
    return sign * math.ldexp(q, qexp)


def exact_int_of_f32(w: np.ndarray) -> np.ndarray:
    """Object array of Python ints t with w == t * 2**-149 exactly (w fp32)."""
    w = np.asarray(w, dtype=np.float32)
    m, ex = np.frexp(w.astype(np.float64))  # w = m * 2**ex, 0.5 <= |m| < 1
    out = np.empty(w.shape, dtype=object)
    flat_m, flat_e, flat_o = m.ravel(), ex.ravel(), out.reshape(-1)
    for i in range(flat_m.size):
        mi = int(flat_m[i] * (1 << 24))     # exact: fp32 has 24 significand bits
        sh = int(flat_e[i]) - 24 + 149
        if sh >= 0:
            flat_o[i] = mi << sh
        else:
            assert mi % (1 << -sh) == 0
            flat_o[i] = mi >> -sh
    return out


# ---------------------------------------------------------------------------
# the Hadamard matrix  ([P1] "What changed in the computation")
# ---------------------------------------------------------------------------

def hadamard4() -> np.ndarray:
    """Sylvester 4x4 Hadamard (reading R1), integer entries +-1."""
    h2 = np.array([[1, 1], [1, -1]], dtype=np.int64)
    return np.kron(h2, h2)


def hadamard256_pm1() -> np.ndarray:
    """H4 (x) H4 (x) H4 (x) H4: the 256x256 matrix before normalisation (+-1)."""
    h4 = hadamard4()
    h = h4
    for _ in range(3):
        h = np.kron(h, h4)
    return h


def hadamard256() -> np.ndarray:
    """H = (H4 (x) H4 (x) H4 (x) H4) / 16 in float64 (entries exactly +-1/16)."""
    return hadamard256_pm1().astype(np.float64) / 16.0


def _check_k(K: int) -> None:
    if K % GROUP != 0 or K < 0 or K > K_MAX:
        raise ValueError(f"K={K} must be a multiple of {GROUP} in 0 .. {K_MAX} (R7, R12)")


# ---------------------------------------------------------------------------
# rotation
# ---------------------------------------------------------------------------

def rotate_f64(x: np.ndarray) -> np.ndarray:
    """X H (equivalently X H^T) group-wise in float64, no final rounding."""
    x = np.asarray(x, dtype=np.float64)
    R, K = x.shape
    _check_k(K)
    return (x.reshape(R, K // GROUP, GROUP) @ hadamard256()).reshape(R, K)


def rotate_activations_exact(x16: np.ndarray) -> np.ndarray:
    """Exact X_rot = X H for fp16 X, as float64.

    Exactness: every fp16 value is an integer multiple of 2^-24 with magnitude
    at most 65504 < 2^16, so each term x*(+-1/16) is a multiple of 2^-28 below
    2^12 and any partial sum of at most 256 of them is a multiple of 2^-28 below
    2^20.  Such numbers need at most 48 significand bits, so every addition (or
    fused multiply-add) inside the float64 matrix product is exact, whatever
    order the library uses.
    """
    x16 = np.asarray(x16)
    if x16.dtype != np.float16:
        raise TypeError("activations must be fp16")
    return rotate_f64(x16.astype(np.float64))


def rotate_activations_f32(x16: np.ndarray) -> np.ndarray:
    """X_rot rounded once to fp32 (reading R3)."""
    return rotate_activations_exact(x16).astype(np.float32)


def _exact_group_rounding(w_group: np.ndarray, fmt=F32) -> np.ndarray:
    """Exact (w_group @ H) for fp32 rows of 256, rounded once to ``fmt``."""
    t = exact_int_of_f32(w_group).dot(hadamard256_pm1().astype(object))
    out = np.empty(t.shape, dtype=np.float64)
    for idx, v in np.ndenumerate(t):
        out[idx] = round_scaled_int(v, 149 + 4, fmt)   # /16 = 2^-4
    return out


def rotate_weights_f32(w32: np.ndarray, force_exact: bool = False) -> np.ndarray:
    """W_rot = W H^T per 256-group: the exact product rounded once to fp32 (R3).

    A group's float64 product is already exact when its values span few enough
    binades: all terms are multiples of 2^lo (lo = lowest significand-bit
    exponent in the group) and every partial sum is below 2^(hi+8) with
    2^hi > max|w|, so hi + 8 - lo <= 52 bits means no float64 addition rounds.
    Groups that fail this test (or all groups with ``force_exact``) are summed
    with Python integers instead.  Either way the value handed to the fp32
    rounding is the exact one.
    """
    w = np.asarray(w32, dtype=np.float32)
    N, K = w.shape
    _check_k(K)
    out = rotate_f64(w.astype(np.float64)).astype(np.float32)
    g = w.reshape(N, K // GROUP, GROUP).astype(np.float64)
    nz = g != 0
    _, ex = np.frexp(g)                               # |w| = f * 2^ex, f in [0.5, 1)
    lo = np.where(nz, np.maximum(ex - 24, -149), 10_000).min(axis=2)
    hi = np.where(nz, ex, -10_000).max(axis=2)
    inexact = (hi + 8 - lo > 52) & nz.any(axis=2)
    if force_exact:
        inexact = nz.any(axis=2)
    for n, gi in zip(*np.nonzero(inexact)):
        sl = slice(gi * GROUP, (gi + 1) * GROUP)
        out[n, sl] = _exact_group_rounding(w[n:n + 1, sl])[0].astype(np.float32)
    return out


# ---------------------------------------------------------------------------
# row-wise quantisation  ([P1] "What changed in the computation")
# ---------------------------------------------------------------------------

def quantize_rows(v32: np.ndarray):
    """s[r] = max_k |v[r,k]| / 127 and Q = clamp(round(v / s), -128, 127).

    All arithmetic is fp32 (reading R3): the maximum is exact, the two
    divisions are IEEE fp32 divisions and round is half-to-even (R2).  A zero
    row gets s = 0 and Q = 0 (R4).  Returns (Q int8 [R, K], s fp32 [R]).
    """
    v = np.asarray(v32, dtype=np.float32)
    amax = np.max(np.abs(v), axis=1, initial=np.float32(0))   # an empty row (K = 0) has maximum 0 (R12)
    s = (amax / np.float32(QMAX)).astype(np.float32)
    safe = np.where(s == 0, np.float32(1), s).astype(np.float32)
    r = (v / safe[:, None]).astype(np.float32)
    q = np.rint(r)
    q = np.where((s == 0)[:, None], 0.0, q)
    q = np.clip(q, -128, 127).astype(np.int8)
    return q, s


def quantize_weights(w32: np.ndarray, force_exact: bool = False):
    """Offline weight preparation: (Q_W int8 [N, K], s_W fp32 [N])."""
    return quantize_rows(rotate_weights_f32(w32, force_exact=force_exact))


def quantize_activations(x16: np.ndarray):
    """Per-call activation prologue: (Q_X int8 [M, K], s_X fp32 [M])."""
    return quantize_rows(rotate_activations_f32(x16))


# ---------------------------------------------------------------------------
# integer product and scale restore
# ---------------------------------------------------------------------------

def int8_gemm(qx: np.ndarray, qw: np.ndarray) -> np.ndarray:
    """A = Q_X Q_W^T exactly (int64 result).

    The float64 product is exact here: each term is an integer of magnitude at
    most 128^2 = 2^14 and K <= 2^17, so every partial sum is an integer below
    2^31 < 2^53.
    """
    qx = np.asarray(qx, dtype=np.int8)
    qw = np.asarray(qw, dtype=np.int8)
    if qx.shape[1] != qw.shape[1] or qx.shape[1] > K_MAX:
        raise ValueError("bad K")
    a = qx.astype(np.float64) @ qw.astype(np.float64).T
    return a.astype(np.int64)


def epilogue_w8a8_f32(a: np.ndarray, sx: np.ndarray, sw: np.ndarray, bias=None) -> np.ndarray:
    """fp32( fp32(A) * fp32(s_X[m] * s_W[n]) [+ bias[n]] ): R5 before its fp16 cast."""
    af = np.asarray(a).astype(np.float32)
    scale = np.asarray(sx, np.float32)[:, None] * np.asarray(sw, np.float32)[None, :]
    y = af * scale
    if bias is not None:
        y = y + np.asarray(bias, np.float32)[None, :]
    return y.astype(np.float32)


def epilogue_w8a8(a: np.ndarray, sx: np.ndarray, sw: np.ndarray, bias=None) -> np.ndarray:
    """Y = fp16( fp32(A) * fp32(s_X[m] * s_W[n]) [+ bias[n]] ) (reading R5)."""
    return epilogue_w8a8_f32(a, sx, sw, bias).astype(np.float16)


def linear_w8a8(x16, qw, sw, bias=None):
    """The W8A8 linear: returns (Y fp16 [M, N], Q_X, s_X, A)."""
    qx, sx = quantize_activations(x16)
    a = int8_gemm(qx, qw)
    return epilogue_w8a8(a, sx, sw, bias), qx, sx, a


def lora_term(x16, lora) -> np.ndarray:
    """scale * (X down^T) up^T in float64 on the unrotated X and down ([P4] "Design").

    ``lora`` is (down fp32 [R, K], up fp32 [N, R], scale).  H is symmetric and
    orthogonal, so this equals the product of the rotated X and rotated down.
    """
    down, up, scale = lora
    t = np.asarray(x16, np.float16).astype(np.float64) @ np.asarray(down, np.float32).astype(np.float64).T
    return float(scale) * (t @ np.asarray(up, np.float32).astype(np.float64).T)


def add_f16(a16, b16) -> np.ndarray:
    """fp16 tensor addition: the exact sum of two fp16 values rounded once.

    Two fp16 values are multiples of 2^-24 below 2^16, so their sum needs at
    most 41 significand bits and is exact in float64; the cast to fp16 is the
    single rounding.
    """
    s = np.asarray(a16, np.float16).astype(np.float64) + np.asarray(b16, np.float16).astype(np.float64)
    return s.astype(np.float16)


def linear_w8a8_ex(x16, qw, sw, bias=None, lora=None, residual=None) -> np.ndarray:
    """The W8A8 linear with bias, unmerged LoRA and residual (reading R8).

    Without ``lora`` and ``residual`` this is ``linear_w8a8``'s Y.  ``lora`` is
    (down fp32 [R, K], up fp32 [N, R], scale); ``residual`` is fp16 [M, N].
    """
    qx, sx = quantize_activations(x16)
    y32 = epilogue_w8a8_f32(int8_gemm(qx, qw), sx, sw, bias)
    if lora is None:
        y = y32.astype(np.float16)
    else:
        y = (y32.astype(np.float64) + lora_term(x16, lora)).astype(np.float16)
    if residual is not None:
        y = add_f16(y, residual)
    return y


# ---------------------------------------------------------------------------
# weight-only (W8A16) path, fp16 baseline, float truth
# ---------------------------------------------------------------------------

def rotate_activations_f16(x16: np.ndarray) -> np.ndarray:
    """X16 = fp16(exact X H): one rounding from the exact value (R6)."""
    ex = rotate_activations_exact(x16)
    return ex.astype(np.float16)


def linear_w8a16(x16, qw, sw, bias=None, lora=None):
    """Weight-only linear with optional unmerged LoRA (reading R6).

    ``lora`` is (down fp32 [R, K], up fp32 [N, R], scale).  Everything after the
    fp16 rotation is float64; the single rounding is the final cast to fp16.
    """
    x16r = rotate_activations_f16(x16).astype(np.float64)
    acc = x16r @ np.asarray(qw, np.int8).astype(np.float64).T
    y = acc * np.asarray(sw, np.float32).astype(np.float64)[None, :]
    if lora is not None:
        y = y + lora_term(x16, lora)
    if bias is not None:
        y = y + np.asarray(bias, np.float32).astype(np.float64)[None, :]
    return y.astype(np.float16)


def dequantize_weights(qw, sw) -> np.ndarray:
    """W_deq = fp16( (Q_W (.) s_W) H ) per 256-group, rounded once (reading R10).

    Exactness: the group sum is s_W[n] / 16 times an integer of magnitude at
    most 256 * 128 = 2^15, so the float64 product of that integer with the
    fp32 scale has at most 15 + 24 bits and is exact; the cast to fp16 is the
    single rounding.
    """
    q = np.asarray(qw, np.int8).astype(np.int64)
    N, K = q.shape
    _check_k(K)
    t = (q.reshape(N, K // GROUP, GROUP) @ hadamard256_pm1()).reshape(N, K)   # exact integers
    w = t.astype(np.float64) * (np.asarray(sw, np.float32).astype(np.float64)[:, None] / 16.0)
    return w.astype(np.float16)


def linear_dequant(x16, qw, sw, bias=None) -> np.ndarray:
    """Dequantise-every-call baseline: fp16( X W_deq^T [+ bias] ), the sum in float64."""
    y = np.asarray(x16, np.float16).astype(np.float64) @ dequantize_weights(qw, sw).astype(np.float64).T
    if bias is not None:
        y = y + np.asarray(bias, np.float32).astype(np.float64)[None, :]
    return y.astype(np.float16)


# ---------------------------------------------------------------------------
# range-safe weight-only path  ([P4] "Design", reading R11)
# ---------------------------------------------------------------------------

def to_bf16(a) -> np.ndarray:
    """Round float64 values to bfloat16 (round half to even), returned as float32.

    Normal range: keep 8 significand bits of the float64 value; below 2^-126
    the grid is 2^-133; at or beyond the overflow boundary (2 - 2^-8) 2^127
    the result is +-inf, as IEEE round-to-nearest gives.
    """
    a = np.asarray(a, np.float64)
    out = np.empty(a.shape, np.float64)
    flat, res = a.ravel(), out.reshape(-1)
    for i, v in enumerate(flat):
        if v == 0 or not math.isfinite(v):
            res[i] = v
            continue
        f, e = math.frexp(abs(v))                 # |v| = f 2^e, f in [0.5, 1)
        q = max(e - 8, -133)                      # exponent of one unit in the last place
        m = abs(v) / 2.0 ** q                     # exact (power-of-two scaling)
        r = np.round(m)                           # half to even
        val = math.copysign(r * 2.0 ** q, v)
        res[i] = val if abs(val) < 2.0 ** 128 else math.copysign(math.inf, v)
    return out.astype(np.float32)


def _row_rotation_exact(x32_row) -> list:
    """Exact X_rot values of one row (fp32-representable inputs) as Fractions."""
    t = exact_int_of_f32(np.asarray(x32_row, np.float32).reshape(-1, GROUP))
    t = t.dot(hadamard256_pm1().astype(object)).reshape(-1)
    from fractions import Fraction
    return [Fraction(int(v), 1 << (149 + 4)) for v in t]


def rotate_rowscaled_f16(x):
    """Range-safe prologue (reading R11): (X16s fp16 [M, K], e int64 [M]).

    X16s = fp16(X_rot 2^-e_m) rounded once from the exact rotation, e_m the
    smallest integer with max|X_rot[m, :]| <= 2^e_m (0 for a zero row).  The
    input holds fp16 or bf16 values (any fp32 values work).  Rows whose
    float64 rotation is exact (every group spanning at most 45 binades, which
    keeps each partial sum within 53 bits) take the float64 route; others are
    rotated with Python integers.
    """
    x = np.asarray(x, np.float32)
    M, K = x.shape
    _check_k(K)
    xr = rotate_f64(x.astype(np.float64))
    g = x.reshape(M, K // GROUP, GROUP).astype(np.float64)
    nz = g != 0
    _, ex = np.frexp(g)
    lo = np.where(nz, np.maximum(ex - 24, -149), 10_000).min(axis=2)
    hi = np.where(nz, ex, -10_000).max(axis=2)
    exact_row = ~(((hi + 8 - lo) > 52) & nz.any(axis=2)).any(axis=1)
    x16 = np.empty((M, K), np.float16)
    e = np.zeros(M, np.int64)
    for m in range(M):
        if exact_row[m]:
            amax = float(np.max(np.abs(xr[m]), initial=0.0))   # K = 0: maximum 0, e = 0 (R12)
            if amax > 0:
                f, ex2 = math.frexp(amax)
                e[m] = ex2 - 1 if f == 0.5 else ex2
            x16[m] = (xr[m] * 2.0 ** -int(e[m])).astype(np.float16)
        else:
            vals = _row_rotation_exact(x[m])
            amax = max(abs(v) for v in vals)
            em = 0
            if amax > 0:
                em = math.ceil(math.log2(amax))
                while amax > 2 ** em:                   # guard the float log
                    em += 1
                while em > -10_000 and amax <= 2 ** (em - 1):
                    em -= 1
            e[m] = em
            for k, v in enumerate(vals):
                sv = v / (2 ** em) if em >= 0 else v * (2 ** -em)
                sh = sv.denominator.bit_length() - 1
                x16[m, k] = round_scaled_int(sv.numerator, sh, F16)
    return x16, e


def linear_w8a16_rs(x, qw, sw, bias=None, residual=None, out="f16") -> np.ndarray:
    """Range-safe weight-only linear (reading R11), output fp16 or bf16 (as float32).

    The product of the scaled fp16 activations and the int8 codes is exact in
    float64 (multiples of 2^-24 below 2^24); the scale, the exponent restore
    and the bias are applied in float64 and rounded once to the output type;
    a residual (same type) is then one addition rounded once.
    """
    x16s, e = rotate_rowscaled_f16(x)
    acc = x16s.astype(np.float64) @ np.asarray(qw, np.int8).astype(np.float64).T
    y = acc * np.asarray(sw, np.float32).astype(np.float64)[None, :] * np.exp2(e.astype(np.float64))[:, None]
    if bias is not None:
        y = y + np.asarray(bias, np.float32).astype(np.float64)[None, :]
    rnd = (lambda a: np.asarray(a, np.float64).astype(np.float16)) if out == "f16" else to_bf16
    y = rnd(y)
    if residual is not None:
        y = rnd(np.asarray(y, np.float64) + np.asarray(residual, np.float32).astype(np.float64))
    return y


def linear_f16(x16, w16) -> np.ndarray:
    """fp16 baseline: fp16( sum_k X W16 ) with the sum in float64."""
    y = np.asarray(x16, np.float16).astype(np.float64) @ np.asarray(w16, np.float16).astype(np.float64).T
    return y.astype(np.float16)


def linear_true(x, w) -> np.ndarray:
    """Unquantised Y = X W^T in float64."""
    return np.asarray(x, np.float64) @ np.asarray(w, np.float64).T
