"""Seeded synthetic inputs for the W4A16 NVFP4 GEMM workloads.

Shared by the tests, the smoke check and the benchmark, and by both sides of
every parity check (the GPU library and the CPU oracle).  This module holds
none of the method's arithmetic: it only draws random numbers and writes them
in the canonical input formats (bf16 or fp16 bit patterns, packed 4-bit codes with the
even k in the low nibble, E4M3 scale bytes, fp32 global scales, expert
offsets).  Decoding any of these is the oracle's and the library's business.

Every array comes from ``numpy.random.Generator(PCG64(seed))`` drawn in a fixed
order: X, codes, scales, global scale(s), pre-quant scale, routing.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np
import torch

E4M3_MAX = 448.0
E2M1_MAX = 6.0


def rng(seed: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(seed))


def bf16_bits_from_f32(a: np.ndarray) -> np.ndarray:
    """float32 values -> bf16 bit patterns (uint16), round to nearest even (torch cast)."""
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16).copy()


def e4m3_bytes_from_f32(a: np.ndarray) -> np.ndarray:
    """float32 values -> OCP E4M3FN bytes, round to nearest even (torch cast)."""
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(torch.float8_e4m3fn)
    return t.view(torch.uint8).numpy().copy()


def pack_codes(codes: np.ndarray) -> np.ndarray:
    """4-bit codes [..., K] -> bytes [..., K/2]; code of even k in the low nibble."""
    c = np.asarray(codes, dtype=np.uint8)
    return (c[..., 0::2] & 15) | ((c[..., 1::2] & 15) << 4)


def random_codes(g: np.random.Generator, shape) -> np.ndarray:
    """Uniform over all 16 E2M1 codes, packed along the last axis."""
    return pack_codes(g.integers(0, 16, size=shape, dtype=np.uint8))


def scales_pow2_mant(g: np.random.Generator, shape, umin=-4, umax=2) -> np.ndarray:
    """E4M3 bytes of 2^u * (1 + m/8), u uniform in [umin, umax], m uniform in 0..7."""
    u = g.integers(umin, umax + 1, size=shape)
    m = g.integers(0, 8, size=shape)
    return (((u + 7) << 3) | m).astype(np.uint8)


def scales_log_uniform(g: np.random.Generator, shape, lo=-6.0, hi=3.0) -> np.ndarray:
    """E4M3 bytes nearest to 2^u with u uniform in [lo, hi]."""
    u = g.uniform(lo, hi, size=shape)
    return e4m3_bytes_from_f32(np.exp2(u).astype(np.float32))


def scales_e8m0(g: np.random.Generator, shape, umin=-9, umax=2) -> np.ndarray:
    """E8M0 bytes (MXFP4 group scales) of 2^u, u uniform in [umin, umax]: byte = u + 127."""
    return (g.integers(umin, umax + 1, size=shape) + 127).astype(np.uint8)


def f16_bits_from_f32(a: np.ndarray) -> np.ndarray:
    """float32 values -> IEEE binary16 bit patterns (uint16), round to nearest even (numpy cast)."""
    return np.ascontiguousarray(a, dtype=np.float32).astype(np.float16).view(np.uint16).copy()


def _act_bits(a: np.ndarray, act: str) -> np.ndarray:
    if act == "bf16":
        return bf16_bits_from_f32(a)
    if act == "f16":
        return f16_bits_from_f32(a)
    raise ValueError(f"activation type {act!r}")


def normal_bf16(g: np.random.Generator, shape) -> np.ndarray:
    return bf16_bits_from_f32(g.standard_normal(size=shape, dtype=np.float32))


def normal_act(g: np.random.Generator, shape, act: str = "bf16") -> np.ndarray:
    """N(0, 1) activations as bf16 or fp16 bits (the same draws either way)."""
    return _act_bits(g.standard_normal(size=shape, dtype=np.float32), act)


def awq_prescale(g: np.random.Generator, K: int, act: str = "bf16") -> np.ndarray:
    """Per-channel pre-quant scale, uniform in [1/e, e], as bf16 (or fp16) bits."""
    return _act_bits(g.uniform(1.0 / math.e, math.e, size=K).astype(np.float32), act)


@dataclass
class DenseCase:
    name: str
    M: int
    N: int
    K: int
    x: np.ndarray             # uint16 bf16 (or fp16, act == "f16") bits [M, K]
    w: np.ndarray             # uint8 [N, K/2]
    s: np.ndarray             # uint8 E4M3 [N, K/16] (NVFP4) or E8M0 [N, K/32] (MXFP4)
    g_stored: float           # fp32 value as stored (MXFP4: no global scale, 1.0)
    g_is_divisor: bool
    pre: np.ndarray | None    # uint16 bits [K] (the type of x) or None
    meta: dict = field(default_factory=dict)
    act: str = "bf16"         # activation / output type
    fmt: str = "nvfp4"        # weight format: nvfp4 or mxfp4


def dense_case(M: int, N: int, K: int, seed: int, *, scales: str = "pow2_mant", g_stored: float = 1.0 / 448.0,
               g_is_divisor: bool = False, prescale: bool = False, name: str = "", act: str = "bf16",
               fmt: str = "nvfp4") -> DenseCase:
    """One dense workload.  scales: 'pow2_mant' (2^u (1+m/8), u in [-4,2]) or 'log_uniform' ([2^-6, 2^3]).
    act: activation type, 'bf16' or 'f16' (the same random draws, rounded to that type).  fmt 'mxfp4': E8M0
    scales 2^u, u in [-9, 2], one per 32 K, and no global scale (g_stored 1.0, not a divisor)."""
    assert K % (32 if fmt == "mxfp4" else 16) == 0
    g = rng(seed)
    x = normal_act(g, (M, K), act)
    w = random_codes(g, (N, K))
    if fmt == "mxfp4":
        s = scales_e8m0(g, (N, K // 32))
        g_stored, g_is_divisor, scales = 1.0, False, "e8m0"
    else:
        s = scales_pow2_mant(g, (N, K // 16)) if scales == "pow2_mant" else scales_log_uniform(g, (N, K // 16))
    pre = awq_prescale(g, K, act) if prescale else None
    return DenseCase(name or f"dense_M{M}_N{N}_K{K}", M, N, K, x, w, s, float(np.float32(g_stored)),
                     bool(g_is_divisor), pre, {"seed": seed, "scales": scales}, act, fmt)


def zipf_routing(g: np.random.Generator, T: int, E: int, topk: int, s: float = 1.1) -> np.ndarray:
    """[T, topk] distinct experts per token; P(rank r) ~ r^-s, ranks mapped to experts by a seeded permutation."""
    perm = g.permutation(E)
    p = np.arange(1, E + 1, dtype=np.float64) ** (-s)
    p /= p.sum()
    pe = np.empty(E)
    pe[perm] = p
    return np.stack([g.choice(E, size=topk, replace=False, p=pe) for _ in range(T)])


@dataclass
class GroupedCase:
    name: str
    E: int
    N: int
    K: int
    R: int
    x: np.ndarray             # uint16 bf16 (or fp16) bits [R, K], rows grouped by expert
    offsets: np.ndarray       # int32 [E+1]
    w: np.ndarray             # uint8 [E, N, K/2]
    s: np.ndarray             # uint8 [E, N, K/16] (E8M0 [E, N, K/32] for MXFP4)
    g_stored: np.ndarray      # float32 [E] (MXFP4: ones)
    g_is_divisor: bool
    pre: np.ndarray | None
    meta: dict = field(default_factory=dict)
    act: str = "bf16"
    fmt: str = "nvfp4"

    @property
    def active(self) -> np.ndarray:
        return np.nonzero(np.diff(self.offsets) > 0)[0]


def routing_seed(seed: int) -> int:
    return seed + 500


def grouped_case(T: int, E: int, topk: int, N: int, K: int, seed: int, *, x_source: str = "gather",
                 prescale: bool = False, g_base: float = 1.0 / 2688.0, name: str = "",
                 routing: np.ndarray | None = None, seed0: int | None = None, act: str = "bf16",
                 fmt: str = "nvfp4") -> GroupedCase:
    """Grouped MoE workload.  x_source 'gather': rows are tokens X[T, K] gathered per (token, expert) pair in
    expert order; 'fresh': a new N(0,1) [R, K] input (the FC2 side, whose real input is FC1's activation).
    The routing comes from its own stream, seeded by ``routing_seed(seed0 or seed)``, so FC1 and FC2 cases
    built with the same seed0 share it."""
    g = rng(seed)
    xt = normal_act(g, (T, K), act)
    w = random_codes(g, (E, N, K))
    s = scales_e8m0(g, (E, N, K // 32)) if fmt == "mxfp4" else scales_pow2_mant(g, (E, N, K // 16))
    v = g.integers(-2, 3, size=E)
    gs = (np.exp2(v.astype(np.float64)) * g_base).astype(np.float32) if fmt != "mxfp4" else np.ones(E, np.float32)
    pre = awq_prescale(g, K, act) if prescale else None
    route = zipf_routing(rng(routing_seed(seed0 if seed0 is not None else seed)), T, E, topk) \
        if routing is None else routing
    tok = np.repeat(np.arange(T), route.shape[1])
    exp_ = route.reshape(-1)
    order = np.argsort(exp_, kind="stable")
    counts = np.bincount(exp_, minlength=E)
    offsets = np.zeros(E + 1, dtype=np.int32)
    offsets[1:] = np.cumsum(counts)
    R = int(offsets[-1])
    x = xt[tok[order]] if x_source == "gather" else normal_act(g, (R, K), act)
    return GroupedCase(name or f"grouped_T{T}_E{E}_N{N}_K{K}", E, N, K, R, np.ascontiguousarray(x), offsets,
                       w, s, gs, False, pre, {"seed": seed, "T": T, "topk": topk, "token_of_row": tok[order],
                                              "routing": route}, act, fmt)


# ------------------------------------------------------------- workloads ---
# The five workload families the path is measured and checked on.

def tiny_case(seed: int = 1000) -> DenseCase:
    """M=4, N=256, K=512, pow2-mantissa scales, g = 1/448."""
    return dense_case(4, 256, 512, seed, g_stored=1.0 / 448.0, name="tiny_4x256x512")


def decode_case(M: int, N: int = 14336, K: int = 4096, seed: int = 1001) -> DenseCase:
    """Decode-shaped dense linear, g = 1/(448*6)."""
    return dense_case(M, N, K, seed, g_stored=1.0 / (448.0 * 6.0), name=f"decode_M{M}_N{N}_K{K}")


def prefill_case(M: int = 4096, N: int = 14336, K: int = 4096, seed: int = 1002) -> DenseCase:
    """Prefill-shaped dense linear, log-uniform scales in [2^-6, 2^3], g = 1/2688."""
    return dense_case(M, N, K, seed, scales="log_uniform", g_stored=1.0 / 2688.0, name=f"prefill_M{M}_N{N}_K{K}")


def lmhead_case(M: int, N: int = 131072, K: int = 4096, seed: int = 1003, divisor: bool = True,
                prescale: bool = True) -> DenseCase:
    """LM-head / padding shapes: divisor-stored global scale (2688) and AWQ pre-scale by default."""
    return dense_case(M, N, K, seed, g_stored=2688.0 if divisor else 1.0 / 2688.0, g_is_divisor=divisor,
                      prescale=prescale, name=f"lmhead_M{M}_N{N}_K{K}")


def ragged_case(seed: int = 1003) -> DenseCase:
    """M=33, K=1040 (multiple of 16, not 64), N=1000 (not a multiple of 128), divisor g, AWQ pre-scale."""
    return dense_case(33, 1000, 1040, seed, g_stored=2688.0, g_is_divisor=True, prescale=True,
                      name="ragged_33x1000x1040")


def moe_fc1_case(T: int, seed: int = 1004, E: int = 128, topk: int = 8, prescale: bool = False) -> GroupedCase:
    """Grouped FC1 (gate+up fused): K=2048 -> N=2*768 per expert."""
    return grouped_case(T, E, topk, 2 * 768, 2048, seed, x_source="gather", prescale=prescale,
                        name=f"moe_fc1_T{T}")


def moe_fc2_case(T: int, seed: int = 1004, E: int = 128, topk: int = 8) -> GroupedCase:
    """Grouped FC2: K=768 -> N=2048 per expert, fresh N(0,1) input rows, same routing as FC1 of this seed."""
    return grouped_case(T, E, topk, 2048, 768, seed + 100, x_source="fresh", seed0=seed, name=f"moe_fc2_T{T}")


# ------------------------------------------------------- device generators ---
# Same distributions as above, drawn on the GPU with a seeded torch generator,
# for benchmark workloads too large to draw quickly on the host.  (A different
# random stream than the numpy recipes: used only where no oracle comparison
# is made on the exact values.)

def _tgen(seed: int, device):
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def device_codes(shape, seed: int, device="cuda") -> torch.Tensor:
    """Packed codes [..., K/2]: uniform bytes = two independent uniform 4-bit codes."""
    return torch.randint(0, 256, shape, dtype=torch.uint8, device=device, generator=_tgen(seed, device))


def device_scales(shape, seed: int, kind: str = "pow2_mant", device="cuda") -> torch.Tensor:
    """Scale bytes on the device: 'pow2_mant' and 'log_uniform' E4M3 as on the host; 'e8m0' MXFP4 scales
    2^u, u uniform in [-9, 2] (byte u + 127)."""
    g = _tgen(seed, device)
    if kind == "e8m0":
        return (torch.randint(-9, 3, shape, device=device, generator=g) + 127).to(torch.uint8)
    if kind == "pow2_mant":
        u = torch.randint(-4, 3, shape, device=device, generator=g)
        m = torch.randint(0, 8, shape, device=device, generator=g)
        return (((u + 7) << 3) | m).to(torch.uint8)
    u = torch.rand(shape, device=device, generator=g, dtype=torch.float32) * 9.0 - 6.0
    return torch.exp2(u).to(torch.float8_e4m3fn).view(torch.uint8)


def device_normal_bf16(shape, seed: int, device="cuda") -> torch.Tensor:
    return torch.randn(shape, device=device, generator=_tgen(seed, device), dtype=torch.float32).to(torch.bfloat16)


def device_prescale(K: int, seed: int, device="cuda") -> torch.Tensor:
    g = _tgen(seed, device)
    return (torch.rand(K, device=device, generator=g) * (math.e - 1.0 / math.e) + 1.0 / math.e).to(torch.bfloat16)
