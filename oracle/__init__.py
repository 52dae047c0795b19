"""CPU oracle for the W4A16 NVFP4 matrix multiply.

TEST INFRASTRUCTURE ONLY.  Only the tests, ``__graft_entry__.smoke()`` and the
benchmark's ``cpu_baseline`` leg may import this package.  The product path
(the HIP library and its Python binding) never imports, links or calls it, and
the two share no code.

Two independent implementations of the same plain definition live here:

* the C oracle (``nvfp4_oracle.c``, fp64, OpenMP over output columns), used
  for parity and for the CPU baseline timing;
* a numpy twin (``*_np`` functions below), fp64 with ``np.matmul`` as its only
  library step, used to pin the C oracle.

The definition (see the header of ``nvfp4_oracle.c`` for the passages of the
pages each step follows):

    T[n,k]  = e2m1(code(n,k)) * e4m3(S[n, k//16])
    g       = fp32(1/stored) if the global scale is stored as a divisor else stored
    X'[m,k] = RNE_bf16(X[m,k] * s[k]) if a pre-quant scale s is given else X[m,k]
    Y[m,n]  = g * sum_k X'[m,k] * T[n,k]          (fp64, never rounded)

Grouped (MoE) form: rows offsets[e]..offsets[e+1]-1 use expert e's weights and
global scale; the pre-quant scale is shared by all experts.

MXFP4 weight-only (``fmt="mxfp4"``; SGLang compressed-tensors NVFP4
weight-only page, Modifications, the paragraph on MXFP4: group_blocks == 2,
E8M0 scales, no global_scale):

    T[n,k]  = e2m1(code(n,k)) * e8m0(S[n, k//32]),   e8m0(e) = 2^(e-127), 0xFF NaN
    Y[m,n]  = sum_k X'[m,k] * T[n,k]                 (no global scale)

MoE glue (numpy, fp64; the steps either side of the grouped GEMM in a
mixture-of-experts layer: "Support Nemotron-H nvfp4 ckpt on Hopper", Changes
table, MoE W4A16 execution path; the gate and up projections held together in
FC1: SGLang compressed-tensors NVFP4 weight-only page, review discussion):

    moe_route   : the (token, slot) pairs p = t*k + j sorted by expert, ties in
                  pair order; offsets, row -> token and pair -> row
    silu_mul    : a = silu(gate) * up with gate = h[:, :I], up = h[:, I:],
                  silu(v) = v / (1 + exp(-v))                    (fp64, not rounded)
    relu2       : a = max(h, 0)^2 (non-gated experts)            (fp64, not rounded)
    combine     : out[t] = sum_j w[t, j] * y[row of (t, j)]      (fp64, not rounded)

FP16 activations (numpy, fp64; the same operation with X, the pre-quant scale
and Y in IEEE binary16, which weight-only FP4 serves as well as bf16: "Support
nvfp4 w4a16 on sm120", Summary; SGLang compressed-tensors NVFP4 weight-only
page, Motivation):

    X'[m,k] = RNE_fp16(X[m,k] * s[k]) if a pre-quant scale s is given else X[m,k]
    Y[m,n]  = g * sum_k X'[m,k] * T[n,k]          (fp64, never rounded)

with T from the C oracle's dequant and the sum as one fp64 np.matmul
(``gemm_f16``, ``grouped_gemm_f16``).

Acceptance of a GPU result against the oracle (``accept``): relative Frobenius
error <= 2e-3, every element within 1e-2 * (|ref| + rms(ref)), and every
element finite; outputs of fewer than 1024 elements may meet the Frobenius
bound through the fp32 rounding interval instead (``accumulation_slack``).
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "nvfp4_oracle.c")
_LIB_PATH = os.path.join(_HERE, "_liboracle.so")
_lock = threading.Lock()
_lib = None

REL_FRO_TOL = 2e-3
ELEM_TOL = 1e-2
SMALL_OUTPUT = 1024

# E2M1 magnitudes by 3-bit code, from the OCP MX specification's FP4 (E2M1)
# encoding table: exponent bits 2..1 (bias 1), mantissa bit 0, code 1 subnormal.
_E2M1_MAG = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0], dtype=np.float64)


def build(force: bool = False) -> str:
    """Compile the C oracle into ``oracle/_liboracle.so`` (gcc, fp64, OpenMP)."""
    if force or not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
        tmp = _LIB_PATH + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-fopenmp", "-ffp-contract=off", "-shared", "-fPIC",
                               "-Wall", "-Wextra", _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def lib() -> ctypes.CDLL:
    global _lib
    with _lock:
        if _lib is None:
            build()
            L = ctypes.CDLL(_LIB_PATH)
            P, I64, I, F, D = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_float, ctypes.c_double
            L.oracle_e2m1.argtypes, L.oracle_e2m1.restype = [I], D
            L.oracle_e4m3.argtypes, L.oracle_e4m3.restype = [I], D
            L.oracle_e8m0.argtypes, L.oracle_e8m0.restype = [I], D
            L.oracle_dequant_fmt.argtypes, L.oracle_dequant_fmt.restype = [P, I64, P, I64, I64, I64, I, P], None
            L.oracle_gemm_fmt.argtypes = [P, I64, P, P, I64, P, I64, F, I, I, I64, I64, I64, P, P, I, P]
            L.oracle_gemm_fmt.restype = None
            L.oracle_gemm_sampled_fmt.argtypes = [P, I64, P, P, I64, P, I64, F, I, I, I64, P, P, I64, P]
            L.oracle_gemm_sampled_fmt.restype = None
            L.oracle_grouped_gemm_fmt.argtypes = [P, I64, P, P, P, I64, P, I64, P, I, I, I64, I64, I64, I64, P]
            L.oracle_grouped_gemm_fmt.restype = None
            L.oracle_round_bf16.argtypes, L.oracle_round_bf16.restype = [D], D
            L.oracle_global_scale.argtypes, L.oracle_global_scale.restype = [F, I], D
            L.oracle_dequant.argtypes, L.oracle_dequant.restype = [P, I64, P, I64, I64, I64, P], None
            L.oracle_activation.argtypes, L.oracle_activation.restype = [P, I64, P, I64, I64, P], None
            L.oracle_gemm.argtypes = [P, I64, P, P, I64, P, I64, F, I, I64, I64, I64, P, P, I, P]
            L.oracle_gemm.restype = None
            L.oracle_gemm_sampled.argtypes = [P, I64, P, P, I64, P, I64, F, I, I64, P, P, I64, P]
            L.oracle_gemm_sampled.restype = None
            L.oracle_grouped_gemm.argtypes = [P, I64, P, P, P, I64, P, I64, P, I, I64, I64, I64, I64, P]
            L.oracle_grouped_gemm.restype = None
            L.oracle_grouped_gemm_sampled.argtypes = [P, I64, P, P, P, I64, P, I64, P, I, I64, I64, I64,
                                                      P, P, I64, P]
            L.oracle_grouped_gemm_sampled.restype = None
            L.oracle_max_threads.argtypes, L.oracle_max_threads.restype = [], I
            _lib = L
    return _lib


def _ptr(a):
    return None if a is None else ctypes.c_void_p(a.ctypes.data)


def _c(a, dtype):
    return None if a is None else np.ascontiguousarray(a, dtype=dtype)


# ---------------------------------------------------------------- C oracle ---

def e2m1(code: int) -> float:
    return lib().oracle_e2m1(int(code))


def e4m3(byte: int) -> float:
    return lib().oracle_e4m3(int(byte))


def e8m0(byte: int) -> float:
    return lib().oracle_e8m0(int(byte))


_FMT = {"nvfp4": 0, "mxfp4": 1}


def _fmt(fmt: str) -> int:
    if fmt not in _FMT:
        raise ValueError(f"weight format {fmt!r} (nvfp4 or mxfp4)")
    return _FMT[fmt]


def scale_group(fmt: str) -> int:
    """K elements per block scale: 16 for NVFP4 (E4M3), 32 for MXFP4 (E8M0)."""
    return 32 if _fmt(fmt) == 1 else 16


def round_bf16(v: float) -> float:
    return lib().oracle_round_bf16(float(v))


def global_scale(stored: float, is_divisor: bool) -> float:
    return lib().oracle_global_scale(float(stored), int(bool(is_divisor)))


def dequant(w_packed: np.ndarray, w_scale: np.ndarray, fmt: str = "nvfp4") -> np.ndarray:
    """Weight tile T [N, K] (fp64) from canonical u8 [N, K/2] codes and u8 block scales: [N, K/16] E4M3 (NVFP4)
    or [N, K/32] E8M0 (MXFP4)."""
    w, s = _c(w_packed, np.uint8), _c(w_scale, np.uint8)
    N, K = w.shape[0], w.shape[1] * 2
    assert s.shape == (N, K // scale_group(fmt)), (s.shape, N, K, fmt)
    out = np.empty((N, K), dtype=np.float64)
    lib().oracle_dequant_fmt(_ptr(w), w.shape[1], _ptr(s), s.shape[1], N, K, _fmt(fmt), _ptr(out))
    return out


def activation(x_bits: np.ndarray, pre_bits: np.ndarray | None) -> np.ndarray:
    x, p = _c(x_bits, np.uint16), _c(pre_bits, np.uint16)
    out = np.empty(x.shape, dtype=np.float64)
    lib().oracle_activation(_ptr(x), x.shape[1], _ptr(p), x.shape[0], x.shape[1], _ptr(out))
    return out


def gemm(x_bits, w_packed, w_scale, g_stored, g_is_divisor=False, pre_bits=None, threads=None,
         fmt: str = "nvfp4") -> np.ndarray:
    """Dense Y [M, N] in fp64.  x_bits: bf16 bit patterns (uint16) [M, K].  MXFP4 (fmt="mxfp4") has no global
    scale: g_stored and g_is_divisor are ignored."""
    x, w, s, p = _c(x_bits, np.uint16), _c(w_packed, np.uint8), _c(w_scale, np.uint8), _c(pre_bits, np.uint16)
    M, K = x.shape
    N = w.shape[0]
    assert w.shape[1] * 2 == K and s.shape == (N, K // scale_group(fmt))
    L = lib()
    threads = int(threads or L.oracle_max_threads())
    out = np.empty((M, N), dtype=np.float64)
    xbuf = np.empty((max(M, 1), K), dtype=np.float64)
    tbuf = np.empty((threads, max(K, 1)), dtype=np.float64)
    L.oracle_gemm_fmt(_ptr(x), K, _ptr(p), _ptr(w), w.shape[1], _ptr(s), s.shape[1], float(np.float32(g_stored)),
                      int(bool(g_is_divisor)), _fmt(fmt), M, N, K, _ptr(xbuf), _ptr(tbuf), threads, _ptr(out))
    return out


def gemm_sampled(x_bits, w_packed, w_scale, g_stored, g_is_divisor, pre_bits, rows, cols,
                 fmt: str = "nvfp4") -> np.ndarray:
    """Y[rows[i], cols[i]] for each i, each output computed on its own."""
    x, w, s, p = _c(x_bits, np.uint16), _c(w_packed, np.uint8), _c(w_scale, np.uint8), _c(pre_bits, np.uint16)
    r, c = _c(rows, np.int64), _c(cols, np.int64)
    out = np.empty(r.shape[0], dtype=np.float64)
    lib().oracle_gemm_sampled_fmt(_ptr(x), x.shape[1], _ptr(p), _ptr(w), w.shape[1], _ptr(s), s.shape[1],
                                  float(np.float32(g_stored)), int(bool(g_is_divisor)), _fmt(fmt), x.shape[1],
                                  _ptr(r), _ptr(c), r.shape[0], _ptr(out))
    return out


def grouped_gemm(x_bits, offsets, w_packed, w_scale, g_stored, g_is_divisor=False, pre_bits=None,
                 fmt: str = "nvfp4") -> np.ndarray:
    """Grouped Y [R, N] in fp64.  w_packed [E, N, K/2], w_scale [E, N, K/16] (NVFP4) or [E, N, K/32] (MXFP4),
    g_stored [E] (ignored for MXFP4)."""
    x, o = _c(x_bits, np.uint16), _c(offsets, np.int32)
    w, s, p = _c(w_packed, np.uint8), _c(w_scale, np.uint8), _c(pre_bits, np.uint16)
    R, K = x.shape
    E, N = w.shape[0], w.shape[1]
    g = _c(np.ones(E, np.float32) if g_stored is None else g_stored, np.float32)
    out = np.full((R, N), np.nan, dtype=np.float64)
    lib().oracle_grouped_gemm_fmt(_ptr(x), K, _ptr(o), _ptr(p), _ptr(w), w.shape[2], _ptr(s), s.shape[2], _ptr(g),
                                  int(bool(g_is_divisor)), _fmt(fmt), R, E, N, K, _ptr(out))
    return out


def grouped_gemm_sampled(x_bits, offsets, w_packed, w_scale, g_stored, g_is_divisor, pre_bits, rows, cols):
    x, o = _c(x_bits, np.uint16), _c(offsets, np.int32)
    w, s, g, p = _c(w_packed, np.uint8), _c(w_scale, np.uint8), _c(g_stored, np.float32), _c(pre_bits, np.uint16)
    r, c = _c(rows, np.int64), _c(cols, np.int64)
    E, N, K = w.shape[0], w.shape[1], x.shape[1]
    out = np.empty(r.shape[0], dtype=np.float64)
    lib().oracle_grouped_gemm_sampled(_ptr(x), K, _ptr(o), _ptr(p), _ptr(w), w.shape[2], _ptr(s), s.shape[2],
                                      _ptr(g), int(bool(g_is_divisor)), E, N, K, _ptr(r), _ptr(c), r.shape[0],
                                      _ptr(out))
    return out


def max_threads() -> int:
    return int(lib().oracle_max_threads())


# ------------------------------------------------------------ numpy twin ----
# Independent of the C code: table lookup instead of bit arithmetic for E2M1,
# vectorised E4M3 decode, an integer-bit bf16 rounding, and np.matmul.

def e2m1_np(codes: np.ndarray) -> np.ndarray:
    c = np.asarray(codes).astype(np.int64)
    return np.where(c & 8, -1.0, 1.0) * _E2M1_MAG[c & 7]


def e8m0_np(b: np.ndarray) -> np.ndarray:
    """E8M0 bytes -> 2^(e - 127) (exact in fp64), NaN for 0xFF."""
    e = np.asarray(b).astype(np.int64) & 255
    return np.where(e == 255, np.nan, np.exp2((e - 127).astype(np.float64)))


def e4m3_np(b: np.ndarray) -> np.ndarray:
    b = np.asarray(b).astype(np.int64)
    e, m = (b >> 3) & 15, b & 7
    mag = np.where(e == 0, m * 2.0 ** -9, (8 + m) * np.exp2(e.astype(np.float64) - 10))
    mag = np.where((e == 15) & (m == 7), np.nan, mag)
    return np.where(b & 128, -mag, mag)


def bf16_np(bits: np.ndarray) -> np.ndarray:
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def rne_bf16_np(v: np.ndarray) -> np.ndarray:
    """RNE to bf16 for values that are exact in fp32 (true for a bf16 x bf16 product)."""
    f = np.asarray(v, dtype=np.float64).astype(np.float32)
    assert np.array_equal(f.astype(np.float64), np.asarray(v, dtype=np.float64), equal_nan=True), \
        "rne_bf16_np needs values exact in fp32"
    u = f.view(np.uint32).astype(np.uint64)
    r = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16) & 0xFFFF
    nan = np.isnan(f)
    r = np.where(nan, 0x7FC0, r)
    return bf16_np(r.astype(np.uint16))


def dequant_np(w_packed: np.ndarray, w_scale: np.ndarray, fmt: str = "nvfp4") -> np.ndarray:
    w = np.asarray(w_packed, dtype=np.uint8)
    codes = np.stack([w & 15, w >> 4], axis=-1).reshape(w.shape[0], -1)   # even k = low nibble
    if fmt == "mxfp4":
        scale = np.repeat(e8m0_np(w_scale), 32, axis=1)
    else:
        scale = np.repeat(e4m3_np(w_scale), 16, axis=1)
    return e2m1_np(codes) * scale


def activation_np(x_bits, pre_bits=None) -> np.ndarray:
    x = bf16_np(x_bits)
    if pre_bits is not None:
        x = rne_bf16_np(x * bf16_np(pre_bits)[None, :])
    return x


def global_scale_np(stored, is_divisor) -> float:
    st = np.float32(stored)
    return float(np.float32(1.0) / st) if is_divisor else float(st)


def gemm_np(x_bits, w_packed, w_scale, g_stored, g_is_divisor=False, pre_bits=None, fmt: str = "nvfp4") -> np.ndarray:
    g = 1.0 if fmt == "mxfp4" else global_scale_np(g_stored, g_is_divisor)
    return g * np.matmul(activation_np(x_bits, pre_bits), dequant_np(w_packed, w_scale, fmt).T)


def grouped_gemm_np(x_bits, offsets, w_packed, w_scale, g_stored, g_is_divisor=False, pre_bits=None,
                    fmt: str = "nvfp4"):
    x = activation_np(x_bits, pre_bits)
    E, N = w_packed.shape[0], w_packed.shape[1]
    out = np.full((x.shape[0], N), np.nan)
    for e in range(E):
        a, b = int(offsets[e]), int(offsets[e + 1])
        if b > a:
            g = 1.0 if fmt == "mxfp4" else global_scale_np(g_stored[e], g_is_divisor)
            out[a:b] = g * (x[a:b] @ dequant_np(w_packed[e], w_scale[e], fmt).T)
    return out


# ------------------------------------------------------------ acceptance ----

def round_bf16_np(v: np.ndarray) -> np.ndarray:
    """RNE of fp64 values to bf16 values (8 significant bits, binary32 exponent range)."""
    v = np.asarray(v, dtype=np.float64)
    out = v.copy()
    fin = np.isfinite(v) & (v != 0)
    _, e = np.frexp(v[fin])
    q = np.maximum(e - 8, -133)
    r = np.ldexp(np.rint(np.ldexp(v[fin], -q)), q)
    r = np.where(np.abs(r) > np.ldexp(255.0, 120), np.copysign(np.inf, r), r)
    out[fin] = r
    return out


# ----------------------------------------------------------- fp16 (numpy) ---

def f16_np(bits: np.ndarray) -> np.ndarray:
    """IEEE binary16 bit patterns (uint16) -> fp64 values (exact)."""
    return np.asarray(bits, dtype=np.uint16).view(np.float16).astype(np.float64)


def rne_f16_np(v: np.ndarray) -> np.ndarray:
    """fp64 -> nearest binary16 value, ties to even, overflow to +-inf (numpy's conversion), back in fp64."""
    with np.errstate(over="ignore"):
        return np.asarray(v, dtype=np.float64).astype(np.float16).astype(np.float64)


def activation_f16(x_bits: np.ndarray, pre_bits: np.ndarray | None = None) -> np.ndarray:
    """X' [M, K] (fp64): X, or RNE_fp16(X * s) with the pre-quant scale s (the product of two binary16 values
    is exact in fp64, so this is one correct rounding)."""
    x = f16_np(x_bits)
    return x if pre_bits is None else rne_f16_np(x * f16_np(pre_bits)[None, :])


def gemm_f16(x_bits, w_packed, w_scale, g_stored, g_is_divisor=False, pre_bits=None, fmt: str = "nvfp4") -> np.ndarray:
    """Dense Y [M, N] in fp64 for fp16 activations (x_bits: binary16 bit patterns [M, K])."""
    t = dequant(w_packed, w_scale, fmt)
    g = 1.0 if fmt == "mxfp4" else global_scale(g_stored, g_is_divisor)
    return g * np.matmul(activation_f16(x_bits, pre_bits), t.T)


def grouped_gemm_f16(x_bits, offsets, w_packed, w_scale, g_stored, g_is_divisor=False, pre_bits=None,
                     fmt: str = "nvfp4") -> np.ndarray:
    """Grouped Y [R, N] in fp64 for fp16 activations; rows owned by no expert are NaN."""
    o = np.asarray(offsets, dtype=np.int64)
    xa = activation_f16(x_bits, pre_bits)
    E, N = np.asarray(w_packed).shape[0], np.asarray(w_packed).shape[1]
    out = np.full((xa.shape[0], N), np.nan)
    for e in range(E):
        a, b = o[e], o[e + 1]
        if b > a:
            g = 1.0 if fmt == "mxfp4" else global_scale(float(np.asarray(g_stored, dtype=np.float32)[e]),
                                                        g_is_divisor)
            out[a:b] = g * np.matmul(xa[a:b], dequant(w_packed[e], w_scale[e], fmt).T)
    return out


def accumulation_slack(x_bits, w_packed, w_scale, g_stored, g_is_divisor=False, pre_bits=None, act="bf16",
                       fmt: str = "nvfp4"):
    """Per-output bound d on how far a correct fp32 computation can be from the exact value before its one
    rounding to the output type (numpy, fp64; for small shapes).

    Every product X'[m,k] * T[n,k] is exact in fp32 (a 16-bit activation times a value of at most 6 significant
    bits), so the only fp32 errors are the K - 1 additions, in any order, and the multiply by g.  For recursive
    summation in any order |fl(sum p) - sum p| <= (K - 1) u sum |p| (u = 2^-24; Higham, Accuracy and Stability of
    Numerical Algorithms, section 4.2), and the multiply adds u |g acc|.  d takes twice both terms (margin for
    second-order terms and for accumulators that round internally in another order):
        d[m,n] = 2 K u |g| sum_k |X'[m,k] T[n,k]| + 2 u |Y_ref[m,n]|.
    """
    xa = activation_np(x_bits, pre_bits) if act == "bf16" else activation_f16(x_bits, pre_bits)
    t = dequant_np(w_packed, w_scale, fmt)
    g = 1.0 if fmt == "mxfp4" else abs(global_scale_np(g_stored, g_is_divisor))
    K = xa.shape[1]
    u = 2.0 ** -24
    terms = np.abs(xa) @ np.abs(t).T
    return 2.0 * K * u * g * terms + 2.0 * u * g * np.abs(xa @ t.T)


def accept(y, ref, rel_fro_tol: float = REL_FRO_TOL, elem_tol: float = ELEM_TOL, slack=None, out: str = "bf16"):
    """Return (ok, info) for a result y against the fp64 oracle ref (same shape).

    ok requires: every y finite; |y-ref| <= elem_tol * (|ref| + rms(ref)) element-wise (rms over the set); and
    ||y-ref||_F / ||ref||_F <= rel_fro_tol.  For outputs of fewer than SMALL_OUTPUT elements, where rounding one
    dominant element to bf16 (unit roundoff 2^-8) can exceed 2e-3 by itself so that no 16-bit result could meet
    the Frobenius bound, that bound may instead be met by the rounding interval: with `slack` d from
    accumulation_slack, every element must lie in [RNE(ref - d), RNE(ref + d)] (RNE to the output type `out`,
    which is monotone), i.e. be a rounding of a value within the fp32 error bound of the exact result.
    """
    y = np.asarray(y, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert y.shape == ref.shape, (y.shape, ref.shape)
    info = {"n": int(y.size)}
    if y.size == 0:
        return True, info
    finite = bool(np.all(np.isfinite(y)))
    err = np.abs(y - ref)
    nref = float(np.linalg.norm(ref))
    rel = float(np.linalg.norm(y - ref) / nref) if nref > 0 else float(np.linalg.norm(y - ref))
    rms = float(np.sqrt(np.mean(ref * ref)))
    bound = elem_tol * (np.abs(ref) + rms)
    with np.errstate(invalid="ignore"):
        bad = int(np.count_nonzero(~(err <= bound)))
    fro_ok = rel <= rel_fro_tol
    info.update(finite=finite, rel_fro=rel, rel_fro_bound=rel_fro_tol, bad_elems=bad,
                max_abs_err=float(np.nanmax(err)) if err.size else 0.0)
    if not fro_ok and y.size < SMALL_OUTPUT and slack is not None:
        d = np.broadcast_to(np.asarray(slack, dtype=np.float64), ref.shape)
        rnd = round_bf16_np if out == "bf16" else rne_f16_np
        lo, hi = rnd(ref - d), rnd(ref + d)
        outside = int(np.count_nonzero(~((y >= lo) & (y <= hi))))
        info.update(rounding_interval_misses=outside)
        fro_ok = outside == 0
    ok = finite and fro_ok and bad == 0
    return ok, info


# ------------------------------------------------------------ MoE glue ------
# Plain definitions of the steps around the grouped GEMM.

def moe_route(topk_ids: np.ndarray, E: int):
    """(offsets [E+1], row_token [T*k], token_row [T*k]) of the pairs p = t*k + j sorted by expert, ties in pair
    order (numpy's stable sort is the definition written out)."""
    ids = np.asarray(topk_ids, dtype=np.int64)
    T, k = ids.shape
    flat = ids.reshape(-1)
    order = np.argsort(flat, kind="stable")             # grouped row r holds pair order[r]
    offsets = np.zeros(E + 1, dtype=np.int64)
    offsets[1:] = np.cumsum(np.bincount(flat, minlength=E))
    token_row = np.empty(T * k, dtype=np.int64)
    token_row[order] = np.arange(T * k)
    return offsets, order // k, token_row


def _act_np(bits: np.ndarray, act: str) -> np.ndarray:
    if act == "bf16":
        return bf16_np(bits)
    if act == "f16":
        return f16_np(bits)
    raise ValueError(f"activation type {act!r}")


def silu_mul(h_bits: np.ndarray, act: str = "bf16") -> np.ndarray:
    """h bits [R, 2I] (gate | up; bf16, or fp16 with act='f16') -> silu(gate) * up in fp64, not rounded."""
    h = _act_np(h_bits, act)
    I = h.shape[1] // 2
    g, u = h[:, :I], h[:, I:]
    return g / (1.0 + np.exp(-g)) * u


def relu2(h_bits: np.ndarray, act: str = "bf16") -> np.ndarray:
    """h bits [R, I] (bf16, or fp16 with act='f16') -> max(h, 0)^2 in fp64, not rounded."""
    h = _act_np(h_bits, act)
    return np.where(h > 0, h, 0.0) ** 2


def combine(y_bits: np.ndarray, token_row: np.ndarray, weights: np.ndarray, act: str = "bf16") -> np.ndarray:
    """y bits [R, H] (bf16, or fp16 with act='f16') in grouped row order, token_row [T*k], weights fp32 [T, k]
    -> [T, H] fp64, not rounded."""
    y = _act_np(y_bits, act)
    w = np.asarray(weights, dtype=np.float32).astype(np.float64)
    T, k = w.shape
    rows = np.asarray(token_row, dtype=np.int64).reshape(T, k)
    out = np.zeros((T, y.shape[1]), dtype=np.float64)
    for j in range(k):
        out += w[:, j:j + 1] * y[rows[:, j]]
    return out
