"""Python binding of the MI355X W4A16 NVFP4 GEMM library (``libnvfp4_w4a16.so``).

Argument marshalling only: every step of the computation runs in the HIP
kernels behind the C ABI declared in ``include/nvfp4_w4a16.h``.  torch is
used for device memory and the current stream.  There is no fallback: if the
built library is missing, or a tensor is not on the GPU, the call raises.

    blob = repack(w_packed, w_scale)                       # once per weight
    y = gemm(x, blob, N, K, global_scale, divisor=False, pre_scale=None)
    y = grouped_gemm(x_sorted, expert_offsets, blob, E, N, K, global_scales)

Formats: w_packed uint8 [(E,) N, K/2], two E2M1 codes per byte, even k in the
low nibble; w_scale uint8 or float8_e4m3fn [(E,) N, K/16]; x bf16 [M, K];
global scale(s) fp32 on the device ([1] or [E]); pre_scale bf16 [K].
"""
from __future__ import annotations

import ctypes
import os

import torch

__all__ = ["repack", "repack_bytes", "gemm", "gemm_variant", "grouped_gemm", "dequant", "lib", "Nvfp4Error",
           "workspace", "gemm_workspace_bytes", "grouped_gemm_gather", "moe_route", "moe_silu_mul", "moe_relu2",
           "moe_combine",
           "gemm_plan", "gemm_variants", "gemm_noalloc", "stream_read", "repack_mxfp4", "dequant_mxfp4",
           "gemm_mxfp4", "gemm_variant_mxfp4", "grouped_gemm_mxfp4", "VARIANT_AUTO", "VARIANT_SMALL_M", "VARIANT_LARGE_M", "VARIANT_MFMA", "VARIANT_RESIDENT",
           "VARIANT_MFMA_QUARTER", "VARIANT_KERNELS", "LIB_PATH"]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libnvfp4_w4a16.so")
VARIANT_AUTO, VARIANT_SMALL_M, VARIANT_LARGE_M, VARIANT_MFMA, VARIANT_RESIDENT = 0, 1, 2, 3, 4
VARIANT_MFMA_QUARTER = 5   # MFMA-bound kernel with 64-row workgroups (several per compute unit)
# kernel symbol run by each variant (nvfp4_w4a16_gemm_plan names the variant the automatic choice takes)
VARIANT_KERNELS = {VARIANT_SMALL_M: "k_gemm_small_m", VARIANT_LARGE_M: "k_gemm_tile", VARIANT_MFMA: "k_gemm_mfma",
                   VARIANT_RESIDENT: "k_gemm_xres", VARIANT_MFMA_QUARTER: "k_gemm_mfma"}
_STATUS = {0: "OK", 1: "INVALID_ARG", 2: "ALIGNMENT", 3: "BUFFER_TOO_SMALL", 4: "HIP"}
_lib = None


class Nvfp4Error(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"{_STATUS.get(status, status)}: {msg}")
        self.status = status


def lib() -> ctypes.CDLL:
    """Load the built library (never builds; see weight_only_fp4_amd.build)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m weight_only_fp4_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        P, I64, I = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
        L.nvfp4_last_error.argtypes, L.nvfp4_last_error.restype = [], ctypes.c_char_p
        L.nvfp4_repack_bytes.argtypes, L.nvfp4_repack_bytes.restype = [I64, I64, I64], I64
        L.nvfp4_repack.argtypes, L.nvfp4_repack.restype = [P, I64, P, I64, I64, I64, I64, P, I64, P], I
        L.nvfp4_dequant_bf16.argtypes, L.nvfp4_dequant_bf16.restype = [P, I64, I64, I64, P, I64, P], I
        L.nvfp4_w4a16_gemm_workspace_bytes.argtypes = [I64, I64, I64]
        L.nvfp4_w4a16_gemm_workspace_bytes.restype = I64
        L.nvfp4_w4a16_gemm.argtypes = [P, I64, P, P, P, I, P, I64, I64, I64, I64, P, I64, P]
        L.nvfp4_w4a16_gemm.restype = I
        L.nvfp4_w4a16_gemm_variant.argtypes = [P, I64, P, P, P, I, P, I64, I64, I64, I64, P, I64, I, P]
        L.nvfp4_w4a16_gemm_variant.restype = I
        L.nvfp4_w4a16_gemm_plan.argtypes, L.nvfp4_w4a16_gemm_plan.restype = [I64, I64, I64], I
        L.nvfp4_bench_stream_read.argtypes, L.nvfp4_bench_stream_read.restype = [P, I64, P, I64, I, P], I
        L.mxfp4_repack_bytes.argtypes, L.mxfp4_repack_bytes.restype = [I64, I64, I64], I64
        L.mxfp4_repack.argtypes, L.mxfp4_repack.restype = [P, I64, P, I64, I64, I64, I64, P, I64, P], I
        L.mxfp4_dequant_bf16.argtypes, L.mxfp4_dequant_bf16.restype = [P, I64, I64, I64, P, I64, P], I
        for f in (L.mxfp4_w4a16_gemm, L.mxfp4_w4a16_gemm_f16):
            f.argtypes, f.restype = [P, I64, P, P, P, I64, I64, I64, I64, P, I64, P], I
        L.mxfp4_w4a16_gemm_variant.argtypes = [P, I64, P, P, P, I64, I64, I64, I64, P, I64, I, I, P]
        L.mxfp4_w4a16_gemm_variant.restype = I
        for f in (L.mxfp4_w4a16_grouped_gemm, L.mxfp4_w4a16_grouped_gemm_f16):
            f.argtypes, f.restype = [P, I64, P, P, P, P, I64, I64, I64, I64, I64, P, I64, P], I
        L.nvfp4_w4a16_gemm_noalloc.argtypes = [P, I64, P, P, P, I, P, I64, I64, I64, I64, P]
        L.nvfp4_w4a16_gemm_noalloc.restype = I
        L.nvfp4_w4a16_gemm_noalloc_max_scratch_bytes.argtypes = []
        L.nvfp4_w4a16_gemm_noalloc_max_scratch_bytes.restype = I64
        L.nvfp4_w4a16_gemm_variant_takes.argtypes = [I64, I64, I64, I]
        L.nvfp4_w4a16_gemm_variant_takes.restype = I
        L.nvfp4_w4a16_gemm_f16.argtypes = [P, I64, P, P, P, I, P, I64, I64, I64, I64, P, I64, P]
        L.nvfp4_w4a16_gemm_f16.restype = I
        L.nvfp4_w4a16_gemm_variant_f16.argtypes = [P, I64, P, P, P, I, P, I64, I64, I64, I64, P, I64, I, P]
        L.nvfp4_w4a16_gemm_variant_f16.restype = I
        L.nvfp4_w4a16_grouped_gemm_workspace_bytes.argtypes = [I64, I64, I64, I64]
        L.nvfp4_w4a16_grouped_gemm_workspace_bytes.restype = I64
        L.nvfp4_w4a16_grouped_gemm.argtypes = [P, I64, P, P, P, P, I, P, I64, I64, I64, I64, I64, P, I64, P]
        L.nvfp4_w4a16_grouped_gemm.restype = I
        L.nvfp4_w4a16_grouped_gemm_f16.argtypes = [P, I64, P, P, P, P, I, P, I64, I64, I64, I64, I64, P, I64, P]
        L.nvfp4_w4a16_grouped_gemm_f16.restype = I
        L.nvfp4_w4a16_grouped_gemm_gather_workspace_bytes.argtypes = [I64, I64, I64, I64, I64]
        L.nvfp4_w4a16_grouped_gemm_gather_workspace_bytes.restype = I64
        L.nvfp4_w4a16_grouped_gemm_gather.argtypes = [P, I64, I64, P, P, P, P, P, I, P, I64, I64, I64, I64, I64, P,
                                                      I64, P]
        L.nvfp4_w4a16_grouped_gemm_gather.restype = I
        L.nvfp4_moe_route_workspace_bytes.argtypes = [I64, I64, I64]
        L.nvfp4_moe_route_workspace_bytes.restype = I64
        L.nvfp4_moe_route.argtypes, L.nvfp4_moe_route.restype = [P, I64, I64, I64, P, P, P, P, I64, P], I
        L.nvfp4_moe_silu_mul.argtypes, L.nvfp4_moe_silu_mul.restype = [P, I64, I64, I64, P, I64, P], I
        L.nvfp4_moe_combine.argtypes, L.nvfp4_moe_combine.restype = [P, I64, P, P, I64, I64, I64, P, I64, P], I
        L.nvfp4_moe_relu2.argtypes, L.nvfp4_moe_relu2.restype = [P, I64, I64, I64, P, I64, P], I
        L.nvfp4_moe_silu_mul_f16.argtypes, L.nvfp4_moe_silu_mul_f16.restype = [P, I64, I64, I64, P, I64, P], I
        L.nvfp4_moe_relu2_f16.argtypes, L.nvfp4_moe_relu2_f16.restype = [P, I64, I64, I64, P, I64, P], I
        L.nvfp4_moe_combine_f16.argtypes = [P, I64, P, P, I64, I64, I64, P, I64, P]
        L.nvfp4_moe_combine_f16.restype = I
        L.nvfp4_w4a16_grouped_gemm_gather_f16.argtypes = L.nvfp4_w4a16_grouped_gemm_gather.argtypes
        L.nvfp4_w4a16_grouped_gemm_gather_f16.restype = I
        L.nvfp4_repack_gated_bytes.argtypes, L.nvfp4_repack_gated_bytes.restype = [I64, I64, I64], I64
        L.nvfp4_repack_gated.argtypes = [P, I64, P, I64, I64, I64, I64, I, P, I64, P]
        L.nvfp4_repack_gated.restype = I
        for f in (L.nvfp4_moe_fc1, L.nvfp4_moe_fc1_f16):
            f.argtypes, f.restype = [P, I64, I64, P, P, P, P, P, I, I, P, I64, I64, I64, I64, I64, P], I
        L.mxfp4_repack_gated_bytes.argtypes, L.mxfp4_repack_gated_bytes.restype = [I64, I64, I64], I64
        L.mxfp4_repack_gated.argtypes = L.nvfp4_repack_gated.argtypes
        L.mxfp4_repack_gated.restype = I
        for f in (L.mxfp4_moe_fc1, L.mxfp4_moe_fc1_f16):
            f.argtypes, f.restype = [P, I64, I64, P, P, P, P, I, P, I64, I64, I64, I64, I64, P], I
        L.nvfp4_w4a16_grouped_gemm_variant.argtypes = [P, I64, I64, P, P, P, P, P, I, I, P, I64, I64, I64, I64, I64,
                                                       I, I, I, P]
        L.nvfp4_w4a16_grouped_gemm_variant.restype = I
        _lib = L
    return _lib


def _check(status: int):
    if status != 0:
        raise Nvfp4Error(status, lib().nvfp4_last_error().decode())


def _stream(device: torch.device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _dev(name, t, dtype=None, ndim=None):
    if not isinstance(t, torch.Tensor):
        raise ValueError(f"{name} must be a torch tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be on the GPU")
    if dtype is not None and t.dtype not in (dtype if isinstance(dtype, tuple) else (dtype,)):
        raise ValueError(f"{name} must have dtype {dtype}, got {t.dtype}")
    if ndim is not None and t.dim() not in (ndim if isinstance(ndim, tuple) else (ndim,)):
        raise ValueError(f"{name} must have {ndim} dims, got shape {tuple(t.shape)}")
    if t.dim() and t.stride(-1) != 1:
        raise ValueError(f"{name} must have unit stride in its last dim")
    return t


def repack_bytes(E: int, N: int, K: int) -> int:
    n = lib().nvfp4_repack_bytes(E, N, K)
    if n < 0:
        raise ValueError(f"invalid weight shape E={E} N={N} K={K} (K must be a positive multiple of 16)")
    return n


def repack(w_packed: torch.Tensor, w_scale: torch.Tensor) -> torch.Tensor:
    """Canonical uint8 [(E,) N, K/2] codes + E4M3 [(E,) N, K/16] scales -> repacked uint8 blob."""
    _dev("w_packed", w_packed, torch.uint8, (2, 3))
    _dev("w_scale", w_scale, (torch.uint8, torch.float8_e4m3fn), w_packed.dim())
    if w_scale.dtype != torch.uint8:
        w_scale = w_scale.view(torch.uint8)
    E = w_packed.shape[0] if w_packed.dim() == 3 else 1
    N, K = w_packed.shape[-2], w_packed.shape[-1] * 2
    if tuple(w_scale.shape[-2:]) != (N, K // 16) or (w_packed.dim() == 3 and w_scale.shape[0] != E):
        raise ValueError(f"w_scale shape {tuple(w_scale.shape)} does not match w_packed {tuple(w_packed.shape)}")
    for name, t in (("w_packed", w_packed), ("w_scale", w_scale)):
        if w_packed.dim() == 3 and t.stride(0) != t.shape[1] * t.stride(1):
            raise ValueError(f"{name}: experts must be stored back to back (stride(0) == N * stride(1))")
    nbytes = repack_bytes(E, N, K)
    out = torch.empty(nbytes, dtype=torch.uint8, device=w_packed.device)
    _check(lib().nvfp4_repack(_ptr(w_packed), w_packed.stride(-2), _ptr(w_scale), w_scale.stride(-2), E, N, K,
                              _ptr(out), nbytes, _stream(w_packed.device)))
    return out


def repack_gated(w_packed: torch.Tensor, w_scale: torch.Tensor, up_first: bool = False,
                 mxfp4: bool = False) -> torch.Tensor:
    """Gated FC1 weights, canonical uint8 [E, 2I, K/2] codes + E4M3 [E, 2I, K/16] scales (mxfp4: E8M0 [E, 2I, K/32])
    with the gate projection in rows [0, I) and the up projection in [I, 2I) (up_first: the other way round) -> blob
    for moe_fc1 (its 16-row units alternate gate / up)."""
    _dev("w_packed", w_packed, torch.uint8, 3)
    _dev("w_scale", w_scale, (torch.uint8, torch.float8_e8m0fnu if mxfp4 else torch.float8_e4m3fn), 3)
    if w_scale.dtype != torch.uint8:
        w_scale = w_scale.view(torch.uint8)
    E, N2, K = w_packed.shape[0], w_packed.shape[1], w_packed.shape[2] * 2
    blk = 32 if mxfp4 else 16
    if tuple(w_scale.shape) != (E, N2, K // blk) or N2 % 32:
        raise ValueError(f"w_scale {tuple(w_scale.shape)} must match w_packed {tuple(w_packed.shape)} (one scale per "
                         f"{blk} K), 2I a multiple of 32")
    for name, t in (("w_packed", w_packed), ("w_scale", w_scale)):
        if t.stride(0) != t.shape[1] * t.stride(1):
            raise ValueError(f"{name}: experts must be stored back to back (stride(0) == N * stride(1))")
    pre = "mxfp4" if mxfp4 else "nvfp4"
    nbytes = int(getattr(lib(), pre + "_repack_gated_bytes")(E, N2 // 2, K))
    if nbytes < 0:
        raise ValueError(f"invalid gated weight shape E={E} 2I={N2} K={K} (K a positive multiple of {blk})")
    out = torch.empty(nbytes, dtype=torch.uint8, device=w_packed.device)
    _check(getattr(lib(), pre + "_repack_gated")(_ptr(w_packed), w_packed.stride(1), _ptr(w_scale), w_scale.stride(1),
                                                 E, N2 // 2, K, int(bool(up_first)), _ptr(out), nbytes,
                                                 _stream(w_packed.device)))
    return out


def dequant(blob: torch.Tensor, E: int, N: int, K: int) -> torch.Tensor:
    """Repacked blob -> bf16 [E, N, K] (exact e2m1 * e4m3, no global scale)."""
    _dev("blob", blob, torch.uint8, 1)
    out = torch.empty((E, N, K), dtype=torch.bfloat16, device=blob.device)
    _check(lib().nvfp4_dequant_bf16(_ptr(blob), E, N, K, _ptr(out), K, _stream(blob.device)))
    return out


_ACT_DTYPES = (torch.bfloat16, torch.float16)


def _act_dtype(name, t):
    """The activation type of tensor t (bf16 or fp16); anything else is an error."""
    if not isinstance(t, torch.Tensor) or t.dtype not in _ACT_DTYPES:
        raise ValueError(f"{name} must be a bf16 or fp16 tensor")
    return t.dtype


def _gemm_args(x, blob, N, K, global_scale, pre_scale, out, rows_name="M"):
    """Checks shared by the GEMM calls.  x is bf16 or fp16; pre_scale and out must have x's dtype; global_scale
    None for the formats without one (MXFP4)."""
    if not isinstance(x, torch.Tensor) or x.dtype not in _ACT_DTYPES:
        raise ValueError("x must be a bf16 or fp16 tensor")
    dt = x.dtype
    _dev("x", x, dt, 2)
    _dev("blob", blob, torch.uint8, 1)
    if global_scale is not None:
        _dev("global_scale", global_scale, torch.float32)
        if not global_scale.is_contiguous():
            raise ValueError("global_scale must be contiguous")
    if x.shape[1] != K:
        raise ValueError(f"x has {x.shape[1]} columns, K = {K}")
    if pre_scale is not None:
        _dev("pre_scale", pre_scale, dt, 1)
        if pre_scale.shape[0] != K or not pre_scale.is_contiguous():
            raise ValueError(f"pre_scale must be a contiguous {dt} [{K}]")
    M = x.shape[0]
    if out is None:
        out = torch.empty((M, N), dtype=dt, device=x.device)
    else:
        _dev("out", out, dt, 2)
        if out.shape[0] != M or out.shape[1] != N:
            raise ValueError(f"out must be [{M}, {N}]")
    return M, out


def gemm(x, blob, N, K, global_scale, divisor=False, pre_scale=None, out=None, workspace_buf=None):
    """Y[M, N] = g * (x (.) pre_scale) . dequant(W)^T in x's dtype, bf16 or fp16 (dense linear / LM head).
    workspace_buf: an optional
    buffer from ``workspace(gemm_workspace_bytes(M, N, K), device)``, reusable across calls on one stream."""
    return gemm_variant(x, blob, N, K, global_scale, divisor, pre_scale, out, workspace_buf, VARIANT_AUTO)


def workspace(nbytes: int, device) -> torch.Tensor:
    """A workspace for the GEMM calls: zero-filled once (the split-K counters in it must start at zero; every call
    leaves them zero again, so the buffer can be reused by later calls on the same stream)."""
    return torch.zeros(max(int(nbytes), 1), dtype=torch.uint8, device=device)


def gemm_workspace_bytes(M: int, N: int, K: int) -> int:
    return int(lib().nvfp4_w4a16_gemm_workspace_bytes(M, N, K))


def gemm_variants(M: int, N: int, K: int) -> list:
    """Every forced variant (VARIANT_*) that takes an M x N x K call, automatic first."""
    L = lib()
    return [v for v in (VARIANT_AUTO, VARIANT_SMALL_M, VARIANT_LARGE_M, VARIANT_MFMA, VARIANT_RESIDENT)
            if L.nvfp4_w4a16_gemm_variant_takes(M, N, K, v) == 1]


def gemm_plan(M: int, N: int, K: int) -> int:
    """The variant (VARIANT_*) the automatic choice runs for an M x N x K call; 0 when it launches nothing."""
    v = int(lib().nvfp4_w4a16_gemm_plan(M, N, K))
    if v < 0:
        raise ValueError(f"invalid GEMM shape M={M} N={N} K={K}")
    return v


def gemm_variant(x, blob, N, K, global_scale, divisor=False, pre_scale=None, out=None, workspace_buf=None,
                 variant=VARIANT_AUTO):
    M, out = _gemm_args(x, blob, N, K, global_scale, pre_scale, out)
    need = gemm_workspace_bytes(M, N, K)
    if need < 0:
        raise ValueError(f"invalid GEMM shape M={M} N={N} K={K}")
    if workspace_buf is None:
        workspace_buf = workspace(need, x.device)
    fn = lib().nvfp4_w4a16_gemm_variant_f16 if x.dtype == torch.float16 else lib().nvfp4_w4a16_gemm_variant
    _check(fn(_ptr(x), x.stride(0), _ptr(pre_scale), _ptr(blob), _ptr(global_scale), int(bool(divisor)), _ptr(out),
              out.stride(0), M, N, K, _ptr(workspace_buf), workspace_buf.numel(), int(variant), _stream(x.device)))
    return out


def gemm_noalloc(x, blob, N, K, global_scale, divisor=False, pre_scale=None, out=None):
    """The dense bf16 GEMM through the entry point that allocates nothing (split-K scratch in the library's static
    device array; calls on one GPU must not overlap in time).  ``out`` is allocated here only if not given."""
    if x.dtype != torch.bfloat16:
        raise ValueError("gemm_noalloc takes bf16 activations")
    M, out = _gemm_args(x, blob, N, K, global_scale, pre_scale, out)
    _check(lib().nvfp4_w4a16_gemm_noalloc(_ptr(x), x.stride(0), _ptr(pre_scale), _ptr(blob), _ptr(global_scale),
                                          int(bool(divisor)), _ptr(out), out.stride(0), M, N, K, _stream(x.device)))
    return out


# -------------------------------------------------------------------- MXFP4 --

def repack_mxfp4(w_packed: torch.Tensor, w_scale: torch.Tensor) -> torch.Tensor:
    """MXFP4 weights: codes uint8 [(E,) N, K/2] + E8M0 scales uint8 or float8_e8m0fnu [(E,) N, K/32] -> repacked
    blob (for the *_mxfp4 calls only)."""
    _dev("w_packed", w_packed, torch.uint8, (2, 3))
    _dev("w_scale", w_scale, (torch.uint8, torch.float8_e8m0fnu), w_packed.dim())
    if w_scale.dtype != torch.uint8:
        w_scale = w_scale.view(torch.uint8)
    E = w_packed.shape[0] if w_packed.dim() == 3 else 1
    N, K = w_packed.shape[-2], w_packed.shape[-1] * 2
    if tuple(w_scale.shape[-2:]) != (N, K // 32) or (w_packed.dim() == 3 and w_scale.shape[0] != E):
        raise ValueError(f"w_scale shape {tuple(w_scale.shape)} does not match w_packed {tuple(w_packed.shape)} "
                         "(one E8M0 scale per 32 K)")
    for name, t in (("w_packed", w_packed), ("w_scale", w_scale)):
        if w_packed.dim() == 3 and t.stride(0) != t.shape[1] * t.stride(1):
            raise ValueError(f"{name}: experts must be stored back to back (stride(0) == N * stride(1))")
    nbytes = int(lib().mxfp4_repack_bytes(E, N, K))
    if nbytes < 0:
        raise ValueError(f"invalid MXFP4 weight shape E={E} N={N} K={K} (K must be a positive multiple of 32)")
    out = torch.empty(nbytes, dtype=torch.uint8, device=w_packed.device)
    _check(lib().mxfp4_repack(_ptr(w_packed), w_packed.stride(-2), _ptr(w_scale), w_scale.stride(-2), E, N, K,
                              _ptr(out), nbytes, _stream(w_packed.device)))
    return out


def dequant_mxfp4(blob: torch.Tensor, E: int, N: int, K: int) -> torch.Tensor:
    """Repacked MXFP4 blob -> bf16 [E, N, K] (e2m1 * e8m0)."""
    _dev("blob", blob, torch.uint8, 1)
    out = torch.empty((E, N, K), dtype=torch.bfloat16, device=blob.device)
    _check(lib().mxfp4_dequant_bf16(_ptr(blob), E, N, K, _ptr(out), K, _stream(blob.device)))
    return out


def gemm_variant_mxfp4(x, blob, N, K, pre_scale=None, out=None, workspace_buf=None, variant=VARIANT_AUTO):
    """Y[M, N] = (x (.) pre_scale) . dequant_mxfp4(W)^T in x's dtype (bf16 or fp16), no global scale."""
    M, out = _gemm_args(x, blob, N, K, None, pre_scale, out)
    need = gemm_workspace_bytes(M, N, K)
    if need < 0:
        raise ValueError(f"invalid GEMM shape M={M} N={N} K={K}")
    if workspace_buf is None:
        workspace_buf = workspace(need, x.device)
    _check(lib().mxfp4_w4a16_gemm_variant(_ptr(x), x.stride(0), _ptr(pre_scale), _ptr(blob), _ptr(out), out.stride(0),
                                          M, N, K, _ptr(workspace_buf), workspace_buf.numel(), int(variant),
                                          int(x.dtype == torch.float16), _stream(x.device)))
    return out


def gemm_mxfp4(x, blob, N, K, pre_scale=None, out=None, workspace_buf=None):
    return gemm_variant_mxfp4(x, blob, N, K, pre_scale, out, workspace_buf, VARIANT_AUTO)


def grouped_gemm_mxfp4(x, expert_offsets, blob, E, N, K, pre_scale=None, out=None):
    """Grouped MXFP4 form: rows [offsets[e], offsets[e+1]) of x use expert e (no global scales)."""
    _dev("expert_offsets", expert_offsets, torch.int32, 1)
    if expert_offsets.shape[0] != E + 1 or not expert_offsets.is_contiguous():
        raise ValueError(f"expert_offsets must be a contiguous int32 [{E + 1}]")
    if out is None and isinstance(x, torch.Tensor) and x.dtype in _ACT_DTYPES:
        out = torch.zeros((x.shape[0], N), dtype=x.dtype, device=x.device)
    R, out = _gemm_args(x, blob, N, K, None, pre_scale, out)
    fn = lib().mxfp4_w4a16_grouped_gemm_f16 if x.dtype == torch.float16 else lib().mxfp4_w4a16_grouped_gemm
    _check(fn(_ptr(x), x.stride(0), _ptr(expert_offsets), _ptr(pre_scale), _ptr(blob), _ptr(out), out.stride(0), R, E,
              N, K, None, 0, _stream(x.device)))
    return out


def stream_read(buf: torch.Tensor, out: torch.Tensor, workgroups: int, unroll: int = 4):
    """Measurement: a plain read of the uint8 device buffer ``buf`` (its size a multiple of 16); ``out`` an int32
    device tensor of at least ``workgroups`` elements."""
    _dev("buf", buf, torch.uint8, 1)
    _dev("out", out, torch.int32, 1)
    if out.numel() < workgroups:
        raise ValueError("out needs one element per workgroup")
    _check(lib().nvfp4_bench_stream_read(_ptr(buf), buf.numel(), _ptr(out), workgroups, unroll, _stream(buf.device)))


def grouped_gemm(x, expert_offsets, blob, E, N, K, global_scales, divisor=False, pre_scale=None, out=None,
                 workspace_buf=None):
    """Grouped (MoE) form: rows [offsets[e], offsets[e+1]) of x use expert e.  Rows owned by no expert are left
    untouched in ``out`` (a fresh ``out`` is zero-filled)."""
    _dev("expert_offsets", expert_offsets, torch.int32, 1)
    if expert_offsets.shape[0] != E + 1 or not expert_offsets.is_contiguous():
        raise ValueError(f"expert_offsets must be a contiguous int32 [{E + 1}]")
    if global_scales.numel() != E:
        raise ValueError(f"global_scales must hold {E} values")
    if out is None and isinstance(x, torch.Tensor) and x.dtype in _ACT_DTYPES:
        out = torch.zeros((x.shape[0], N), dtype=x.dtype, device=x.device)
    R, out = _gemm_args(x, blob, N, K, global_scales, pre_scale, out)
    need = int(lib().nvfp4_w4a16_grouped_gemm_workspace_bytes(R, E, N, K))
    if need < 0:
        raise ValueError(f"invalid grouped GEMM shape R={R} E={E} N={N} K={K}")
    if workspace_buf is None:
        workspace_buf = workspace(need, x.device)
    fn = lib().nvfp4_w4a16_grouped_gemm_f16 if x.dtype == torch.float16 else lib().nvfp4_w4a16_grouped_gemm
    _check(fn(_ptr(x), x.stride(0), _ptr(expert_offsets), _ptr(pre_scale), _ptr(blob), _ptr(global_scales),
              int(bool(divisor)), _ptr(out), out.stride(0), R, E, N, K, _ptr(workspace_buf), workspace_buf.numel(),
              _stream(x.device)))
    return out


# ------------------------------------------------------------------ MoE glue --

def moe_route(topk_ids, E):
    """topk_ids int32 [T, k] -> (expert_offsets [E+1], row_token [T*k], token_row [T*k]), all int32 on the device:
    the (token, slot) pairs sorted by expert, ties in pair order."""
    _dev("topk_ids", topk_ids, torch.int32, 2)
    if not topk_ids.is_contiguous():
        raise ValueError("topk_ids must be contiguous")
    T, k = topk_ids.shape
    dev = topk_ids.device
    offsets = torch.zeros(E + 1, dtype=torch.int32, device=dev)
    row_token = torch.empty(T * k, dtype=torch.int32, device=dev)
    token_row = torch.empty(T * k, dtype=torch.int32, device=dev)
    need = int(lib().nvfp4_moe_route_workspace_bytes(T, k, E))
    if need < 0:
        raise ValueError(f"invalid routing shape T={T} k={k} E={E}")
    ws = torch.empty(max(need, 4), dtype=torch.uint8, device=dev)
    _check(lib().nvfp4_moe_route(_ptr(topk_ids), T, k, E, _ptr(offsets), _ptr(row_token), _ptr(token_row),
                                 _ptr(ws), ws.numel(), _stream(dev)))
    return offsets, row_token, token_row


def grouped_gemm_gather(x, row_token, expert_offsets, blob, E, N, K, global_scales, divisor=False, pre_scale=None,
                        out=None, workspace_buf=None):
    """Grouped GEMM whose row r reads token row row_token[r] of x [T, K] (no gathered copy of x is made); x bf16 or
    fp16, the output of x's type."""
    dt = _act_dtype("x", x)
    _dev("x", x, dt, 2)
    _dev("row_token", row_token, torch.int32, 1)
    _dev("expert_offsets", expert_offsets, torch.int32, 1)
    if expert_offsets.shape[0] != E + 1 or not expert_offsets.is_contiguous() or not row_token.is_contiguous():
        raise ValueError(f"expert_offsets must be a contiguous int32 [{E + 1}], row_token contiguous")
    if global_scales.numel() != E:
        raise ValueError(f"global_scales must hold {E} values")
    T, R = x.shape[0], row_token.shape[0]
    if x.shape[1] != K:
        raise ValueError(f"x must be [T, {K}]")
    if pre_scale is not None:
        _dev("pre_scale", pre_scale, dt, 1)
    if out is None:
        out = torch.zeros((R, N), dtype=dt, device=x.device)
    else:
        _dev("out", out, dt, 2)
        if tuple(out.shape) != (R, N):
            raise ValueError(f"out must be [{R}, {N}]")
    need = int(lib().nvfp4_w4a16_grouped_gemm_gather_workspace_bytes(T, R, E, N, K))
    if need < 0:
        raise ValueError(f"invalid grouped GEMM shape T={T} R={R} E={E} N={N} K={K}")
    if workspace_buf is None:
        workspace_buf = workspace(need, x.device)
    fn = lib().nvfp4_w4a16_grouped_gemm_gather_f16 if dt == torch.float16 else lib().nvfp4_w4a16_grouped_gemm_gather
    _check(fn(_ptr(x), x.stride(0), T, _ptr(row_token), _ptr(expert_offsets), _ptr(pre_scale), _ptr(blob),
              _ptr(global_scales), int(bool(divisor)), _ptr(out), out.stride(0), R, E, N, K, _ptr(workspace_buf),
              workspace_buf.numel(), _stream(x.device)))
    return out


MOE_SILU_GLU, MOE_RELU2 = 1, 2
GROUPED_AUTO, GROUPED_SMALL_M, GROUPED_TILE, GROUPED_MFMA = 0, 1, 2, 3


def grouped_gemm_variant(x, row_token, expert_offsets, blob, E, N, K, global_scales, variant, activation=0,
                         divisor=False, pre_scale=None, out=None, mxfp4=False):
    """Test export: the grouped GEMM (activation 0) or fused FC1 (MOE_SILU_GLU on a gated blob of N = 2I rows,
    MOE_RELU2) on a chosen kernel (GROUPED_SMALL_M, GROUPED_TILE, GROUPED_MFMA or GROUPED_AUTO).  row_token None:
    x holds the grouped rows.  mxfp4: an MXFP4 blob (global_scales not read; may be None)."""
    dt = _act_dtype("x", x)
    _dev("x", x, dt, 2)
    _dev("expert_offsets", expert_offsets, torch.int32, 1)
    T = x.shape[0]
    R = row_token.shape[0] if row_token is not None else T
    cols = N // 2 if activation == MOE_SILU_GLU else N
    if out is None:
        out = torch.zeros((R, cols), dtype=dt, device=x.device)
    _check(lib().nvfp4_w4a16_grouped_gemm_variant(
        _ptr(x), x.stride(0), T, _ptr(row_token), _ptr(expert_offsets), _ptr(pre_scale), _ptr(blob),
        _ptr(global_scales), int(bool(divisor)), int(activation), _ptr(out), out.stride(0), R, E, N, K, int(variant),
        int(dt == torch.float16), int(bool(mxfp4)), _stream(x.device)))
    return out


def moe_fc1(x, row_token, expert_offsets, blob, E, I, K, global_scales, activation=MOE_SILU_GLU, divisor=False,
            pre_scale=None, out=None, mxfp4=False):
    """FC1 of a MoE layer with its activation in the GEMM epilogue -> a [R, I] (x's type).  activation MOE_SILU_GLU:
    blob from repack_gated; MOE_RELU2: blob from repack (N = I).  row_token None: x holds the R grouped rows.
    mxfp4: a blob from repack_gated(..., mxfp4=True) or repack_mxfp4, with no global scales (global_scales None)."""
    dt = _act_dtype("x", x)
    _dev("x", x, dt, 2)
    _dev("expert_offsets", expert_offsets, torch.int32, 1)
    if expert_offsets.shape[0] != E + 1 or not expert_offsets.is_contiguous():
        raise ValueError(f"expert_offsets must be a contiguous int32 [{E + 1}]")
    if mxfp4 and global_scales is not None:
        raise ValueError("MXFP4 weights take no global scales (pass None)")
    if not mxfp4 and (global_scales is None or global_scales.numel() != E):
        raise ValueError(f"global_scales must hold {E} values")
    if x.shape[1] != K:
        raise ValueError(f"x must be [T, {K}]")
    T = x.shape[0]
    if row_token is not None:
        _dev("row_token", row_token, torch.int32, 1)
        if not row_token.is_contiguous():
            raise ValueError("row_token must be contiguous")
        R = row_token.shape[0]
    else:
        R = T
    if pre_scale is not None:
        _dev("pre_scale", pre_scale, dt, 1)
    if out is None:
        out = torch.empty((R, I), dtype=dt, device=x.device)
    else:
        _dev("out", out, dt, 2)
        if tuple(out.shape) != (R, I):
            raise ValueError(f"out must be [{R}, {I}]")
    if mxfp4:
        fn = lib().mxfp4_moe_fc1_f16 if dt == torch.float16 else lib().mxfp4_moe_fc1
        _check(fn(_ptr(x), x.stride(0), T, _ptr(row_token), _ptr(expert_offsets), _ptr(pre_scale), _ptr(blob),
                  int(activation), _ptr(out), out.stride(0), R, E, I, K, _stream(x.device)))
        return out
    fn = lib().nvfp4_moe_fc1_f16 if dt == torch.float16 else lib().nvfp4_moe_fc1
    _check(fn(_ptr(x), x.stride(0), T, _ptr(row_token), _ptr(expert_offsets), _ptr(pre_scale), _ptr(blob),
              _ptr(global_scales), int(bool(divisor)), int(activation), _ptr(out), out.stride(0), R, E, I, K,
              _stream(x.device)))
    return out


def moe_silu_mul(h, out=None):
    """h [R, 2I] (gate | up) -> silu(gate) * up [R, I], bf16 or fp16 (h's type)."""
    dt = _act_dtype("h", h)
    _dev("h", h, dt, 2)
    R, I2 = h.shape
    if I2 % 2:
        raise ValueError("h must have an even number of columns (gate | up)")
    I = I2 // 2
    if out is None:
        out = torch.empty((R, I), dtype=dt, device=h.device)
    else:
        _dev("out", out, dt, 2)
    fn = lib().nvfp4_moe_silu_mul_f16 if dt == torch.float16 else lib().nvfp4_moe_silu_mul
    _check(fn(_ptr(h), h.stride(0), R, I, _ptr(out), out.stride(0), _stream(h.device)))
    return out


def moe_relu2(h, out=None):
    """h [R, I] -> max(h, 0)^2 [R, I] (non-gated experts), bf16 or fp16 (h's type)."""
    dt = _act_dtype("h", h)
    _dev("h", h, dt, 2)
    R, I = h.shape
    if out is None:
        out = torch.empty((R, I), dtype=dt, device=h.device)
    else:
        _dev("out", out, dt, 2)
    fn = lib().nvfp4_moe_relu2_f16 if dt == torch.float16 else lib().nvfp4_moe_relu2
    _check(fn(_ptr(h), h.stride(0), R, I, _ptr(out), out.stride(0), _stream(h.device)))
    return out


def moe_combine(y, token_row, topk_weights, out=None):
    """y [R, H] in grouped row order, token_row int32 [T*k], topk_weights fp32 [T, k] -> [T, H]; y and the output
    bf16 or fp16 (y's type)."""
    dt = _act_dtype("y", y)
    _dev("y", y, dt, 2)
    _dev("token_row", token_row, torch.int32, 1)
    _dev("topk_weights", topk_weights, torch.float32, 2)
    if not topk_weights.is_contiguous() or not token_row.is_contiguous():
        raise ValueError("topk_weights and token_row must be contiguous")
    T, k = topk_weights.shape
    H = y.shape[1]
    if out is None:
        out = torch.empty((T, H), dtype=dt, device=y.device)
    else:
        _dev("out", out, dt, 2)
    fn = lib().nvfp4_moe_combine_f16 if dt == torch.float16 else lib().nvfp4_moe_combine
    _check(fn(_ptr(y), y.stride(0), _ptr(token_row), _ptr(topk_weights), T, k, H, _ptr(out), out.stride(0),
              _stream(y.device)))
    return out
