"""Helpers shared by the GPU tests: move synthetic cases to the device and run
the library on them.  Test-side only."""
import numpy as np
import torch

import weight_only_fp4_amd as nv

DEV = "cuda:0"


def bf16_dev(bits: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(DEV)


def f16_dev(bits: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.float16).to(DEV)


def act_dev(bits: np.ndarray, act: str) -> torch.Tensor:
    """Activation bit patterns -> a device tensor of the case's type (bf16 or fp16)."""
    return f16_dev(bits) if act == "f16" else bf16_dev(bits)


def u8_dev(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.uint8)).to(DEV)


def f32_dev(a) -> torch.Tensor:
    return torch.tensor(np.atleast_1d(np.asarray(a, dtype=np.float32)), device=DEV)


def to_f64(y: torch.Tensor) -> np.ndarray:
    return y.float().cpu().numpy().astype(np.float64)


def bits16(y: torch.Tensor) -> np.ndarray:
    """The 16-bit patterns of a bf16 or fp16 tensor."""
    return y.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def bf16_bits(y: torch.Tensor) -> np.ndarray:
    return y.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


class DenseDev:
    """A DenseCase on the device, repacked once."""

    def __init__(self, c):
        self.c = c
        act = getattr(c, "act", "bf16")
        self.x = act_dev(c.x, act)
        self.w = u8_dev(c.w)
        self.s = u8_dev(c.s)
        self.g = f32_dev(c.g_stored)
        self.pre = None if c.pre is None else act_dev(c.pre, act)
        self.blob = nv.repack(self.w, self.s)

    def run(self, variant=nv.VARIANT_AUTO, x=None, g=None, divisor=None, pre="case", out=None):
        c = self.c
        return nv.gemm_variant(self.x if x is None else x, self.blob, c.N, c.K, self.g if g is None else g,
                               c.g_is_divisor if divisor is None else divisor,
                               self.pre if pre == "case" else pre, out=out, variant=variant)


class GroupedDev:
    def __init__(self, gc):
        self.c = gc
        act = getattr(gc, "act", "bf16")
        self.x = act_dev(gc.x, act)
        self.off = torch.from_numpy(gc.offsets.astype(np.int32)).to(DEV)
        self.w = u8_dev(gc.w)
        self.s = u8_dev(gc.s)
        self.g = f32_dev(gc.g_stored)
        self.pre = None if gc.pre is None else act_dev(gc.pre, act)
        self.blob = nv.repack(self.w, self.s)

    def run(self, out=None):
        c = self.c
        return nv.grouped_gemm(self.x, self.off, self.blob, c.E, c.N, c.K, self.g, c.g_is_divisor, self.pre, out=out)
