"""The MoE FC1 with its activation in the GEMM epilogue (nvfp4_moe_fc1) on the GPU.

The fused call rounds FC1's outputs to the activation type and applies the same fp32 activation as the standalone
glue kernels, so it must equal, bitwise, the unfused chain (grouped GEMM with the gather, then nvfp4_moe_silu_mul or
nvfp4_moe_relu2) on the canonical weights; the unfused chain is in turn checked against the oracle.  The gated blob
is built from either gate / up order of the canonical FC1 weight (gate first, as SGLang's w13; up first, as
TensorRT-LLM's w3_w1), which must give the same bytes.  At the benchmark's sizes the oracle is evaluated on
sampled outputs."""
import numpy as np
import pytest
import torch

import oracle
import synth
import weight_only_fp4_amd as nv
from gpu_util import DEV, act_dev, bits16, f32_dev, to_f64, u8_dev

pytestmark = pytest.mark.gpu


def say(msg):
    print(f"[gpu-case] {msg}", flush=True)


def i32_dev(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(DEV)


class Fc1Case:
    """Tokens X[T, K], routing, and one gated FC1 weight (E experts, 2I rows: gate rows then up rows)."""

    def __init__(self, T, E, topk, I, K, seed, pre=False, act="bf16"):
        g = synth.rng(seed)
        self.T, self.E, self.topk, self.I, self.K, self.act = T, E, topk, I, K, act
        self.xt = synth.normal_act(g, (T, K), act)
        self.w = synth.random_codes(g, (E, 2 * I, K))
        self.s = synth.scales_pow2_mant(g, (E, 2 * I, K // 16))
        self.g = (np.exp2(g.integers(-2, 3, E).astype(np.float64)) / 2688).astype(np.float32)
        self.pre = synth.awq_prescale(g, K, act) if pre else None
        self.ids = synth.zipf_routing(synth.rng(seed + 1), T, E, topk)
        self.r_off, self.r_rt, self.r_tr = oracle.moe_route(self.ids, E)

    def dev(self):
        off, row_token, token_row = nv.moe_route(i32_dev(self.ids), self.E)
        x = act_dev(self.xt, self.act)
        p = None if self.pre is None else act_dev(self.pre, self.act)
        return off, row_token, x, p


def _up_first(a):
    """The same weight with the up rows first (the w3_w1 order)."""
    I = a.shape[1] // 2
    return np.ascontiguousarray(np.concatenate([a[:, I:], a[:, :I]], axis=1))


CASES = [   # (T, E, topk, I, K, pre): R <= 16 E runs the small-M grouped kernel, above it the tile kernel
    (16, 16, 4, 192, 256, False),
    (16, 32, 4, 96, 272, True),       # ragged K (not a multiple of 128)
    (256, 16, 4, 192, 256, True),     # tile grouped kernel
    (300, 8, 2, 48, 128, False),      # tile, I = 48: three 16-column pairs
    (1, 4, 1, 16, 64, False),         # one row
]


@pytest.mark.parametrize("act", ["bf16", "f16"])
@pytest.mark.parametrize("T,E,topk,I,K,pre", CASES)
def test_fused_silu_equals_unfused_chain_and_oracle(T, E, topk, I, K, pre, act):
    c = Fc1Case(T, E, topk, I, K, seed=T * 3 + I + K, pre=pre, act=act)
    say(f"fused FC1 SiLU T={T} E={E} k={topk} I={I} K={K} pre={pre} act={act}")
    off, row_token, x, p = c.dev()
    g = f32_dev(c.g)
    w, s = u8_dev(c.w), u8_dev(c.s)
    blob = nv.repack(w, s)
    gated = nv.repack_gated(w, s)
    gated_uf = nv.repack_gated(u8_dev(_up_first(c.w)), u8_dev(_up_first(c.s)), up_first=True)
    h = nv.grouped_gemm_gather(x, row_token, off, blob, E, 2 * I, K, g, False, p)
    a_ref = nv.moe_silu_mul(h)
    a = nv.moe_fc1(x, row_token, off, gated, E, I, K, g, nv.MOE_SILU_GLU, pre_scale=p)
    a_uf = nv.moe_fc1(x, row_token, off, gated_uf, E, I, K, g, nv.MOE_SILU_GLU, pre_scale=p)
    # x pre-gathered (no row index)
    xg = x[row_token.long()].contiguous()
    a_pg = nv.moe_fc1(xg, None, off, gated, E, I, K, g, nv.MOE_SILU_GLU, pre_scale=p)
    torch.cuda.synchronize()
    assert torch.equal(gated, gated_uf)
    assert a.dtype == a_ref.dtype == x.dtype
    assert torch.equal(a, a_ref)
    assert torch.equal(a_uf, a_ref)
    assert torch.equal(a_pg, a_ref)
    # the unfused chain against the oracle: FC1, then the activation on the GPU's own FC1 output
    xr = c.xt[c.r_rt]
    ref_h = (oracle.grouped_gemm if act == "bf16" else oracle.grouped_gemm_f16)(xr, c.r_off, c.w, c.s, c.g, False,
                                                                              c.pre)
    ok, info = oracle.accept(to_f64(h), ref_h, out=act)
    assert ok, ("fc1", info)
    ok, info = oracle.accept(to_f64(a), oracle.silu_mul(bits16(h), act), out=act)
    assert ok, ("silu", info)


@pytest.mark.parametrize("act", ["bf16", "f16"])
@pytest.mark.parametrize("T,E,topk,I,K", [(16, 16, 4, 192, 256), (256, 16, 4, 200, 256)])
def test_fused_relu2_equals_unfused_chain(T, E, topk, I, K, act):
    c = Fc1Case(T, E, topk, I, K, seed=T + I * 5, act=act)
    say(f"fused FC1 relu2 T={T} E={E} I={I} K={K} act={act}")
    off, row_token, x, _ = c.dev()
    g = f32_dev(c.g)
    w, s = u8_dev(c.w[:, :I]), u8_dev(c.s[:, :I])      # a non-gated expert: one projection of I rows
    blob = nv.repack(w, s)
    h = nv.grouped_gemm_gather(x, row_token, off, blob, E, I, K, g)
    a_ref = nv.moe_relu2(h)
    a = nv.moe_fc1(x, row_token, off, blob, E, I, K, g, nv.MOE_RELU2)
    torch.cuda.synchronize()
    assert torch.equal(a, a_ref)
    ok, info = oracle.accept(to_f64(a), oracle.relu2(bits16(h), act), out=act)
    assert ok, info


MX_CASES = [   # (T, E, topk, I, K, pre): the 4-row small-M form, the dynamic small-M form, the tile kernel
    (3, 16, 4, 96, 256, False),
    (16, 16, 4, 192, 288, True),      # K = 288: a K tail of one 32-wide MXFP4 group past 256
    (256, 16, 4, 192, 256, True),
]


@pytest.mark.parametrize("act", ["bf16", "f16"])
@pytest.mark.parametrize("T,E,topk,I,K,pre", MX_CASES)
def test_fused_silu_mxfp4_equals_unfused_chain_and_oracle(T, E, topk, I, K, pre, act):
    """MXFP4 weights (E8M0 scale per 32 K, no global scale): mxfp4_moe_fc1 on either gate / up order equals the
    MXFP4 grouped GEMM with the gather followed by the standalone SiLU, bitwise; that FC1 output matches the
    oracle.  Scales stay at or below 2^-3 (with no global scale, larger ones take silu(gate) * up past fp16's
    range)."""
    g = synth.rng(T * 7 + I + K)
    xt = synth.normal_act(g, (T, K), act)
    w = synth.random_codes(g, (E, 2 * I, K))
    s = synth.scales_e8m0(g, (E, 2 * I, K // 32), umin=-9, umax=-3)
    pre_bits = synth.awq_prescale(g, K, act) if pre else None
    ids = synth.zipf_routing(synth.rng(T * 7 + 1), T, E, topk)
    r_off, r_rt, _ = oracle.moe_route(ids, E)
    say(f"fused FC1 SiLU MXFP4 T={T} E={E} k={topk} I={I} K={K} pre={pre} act={act}")
    off, row_token, _ = nv.moe_route(i32_dev(ids), E)
    x = act_dev(xt, act)
    p = None if pre_bits is None else act_dev(pre_bits, act)
    blob = nv.repack_mxfp4(u8_dev(w), u8_dev(s))
    gated = nv.repack_gated(u8_dev(w), u8_dev(s), mxfp4=True)
    gated_uf = nv.repack_gated(u8_dev(_up_first(w)), u8_dev(_up_first(s)), up_first=True, mxfp4=True)
    h = nv.grouped_gemm_variant(x, row_token, off, blob, E, 2 * I, K, None, nv.GROUPED_AUTO, pre_scale=p,
                                mxfp4=True)
    a_ref = nv.moe_silu_mul(h)
    a = nv.moe_fc1(x, row_token, off, gated, E, I, K, None, nv.MOE_SILU_GLU, pre_scale=p, mxfp4=True)
    a_uf = nv.moe_fc1(x, row_token, off, gated_uf, E, I, K, None, nv.MOE_SILU_GLU, pre_scale=p, mxfp4=True)
    torch.cuda.synchronize()
    assert torch.equal(gated, gated_uf)
    assert torch.equal(a, a_ref)
    assert torch.equal(a_uf, a_ref)
    ref_h = (oracle.grouped_gemm if act == "bf16" else oracle.grouped_gemm_f16)(
        xt[r_rt], r_off, w, s, np.ones(E, np.float32), False, pre_bits, fmt="mxfp4")
    ok, info = oracle.accept(to_f64(h), ref_h, out=act)
    assert ok, ("fc1", info)
    ok, info = oracle.accept(to_f64(a), oracle.silu_mul(bits16(h), act), out=act)
    assert ok, ("silu", info)


@pytest.mark.parametrize("T", [3, 256])
def test_fused_relu2_mxfp4_equals_unfused_chain(T):
    E, topk, I, K = 8, 2, 80, 320
    g = synth.rng(T + 5)
    xt = synth.normal_act(g, (T, K), "bf16")
    w = synth.random_codes(g, (E, I, K))
    s = synth.scales_e8m0(g, (E, I, K // 32))
    ids = synth.zipf_routing(synth.rng(T + 6), T, E, topk)
    say(f"fused FC1 relu2 MXFP4 T={T} E={E} I={I} K={K}")
    off, row_token, _ = nv.moe_route(i32_dev(ids), E)
    x = act_dev(xt, "bf16")
    blob = nv.repack_mxfp4(u8_dev(w), u8_dev(s))
    h = nv.grouped_gemm_variant(x, row_token, off, blob, E, I, K, None, nv.GROUPED_AUTO, mxfp4=True)
    a = nv.moe_fc1(x, row_token, off, blob, E, I, K, None, nv.MOE_RELU2, mxfp4=True)
    ref = nv.moe_relu2(h)
    torch.cuda.synchronize()
    assert torch.equal(a, ref)


@pytest.mark.parametrize("act", ["bf16", "f16"])
def test_fused_fc1_outputs_any_alignment(act):
    """The tile kernel's epilogue (16-byte row pieces through LDS for aligned outputs, single values otherwise):
    the fused SiLU into an output with an odd row stride equals the contiguous output bitwise and leaves its
    padding alone; the squared ReLU with I = 196 (not a multiple of 8) equals the unfused chain."""
    T, E, topk, I, K = 256, 16, 4, 192, 256
    c = Fc1Case(T, E, topk, I, K, seed=77, act=act)
    say(f"fused FC1 output alignment act={act}")
    off, row_token, x, _ = c.dev()
    g = f32_dev(c.g)
    w, s = u8_dev(c.w), u8_dev(c.s)
    gated = nv.repack_gated(w, s)
    a = nv.moe_fc1(x, row_token, off, gated, E, I, K, g, nv.MOE_SILU_GLU)
    big = torch.full((T * topk, I + 3), 7.0, dtype=x.dtype, device=DEV)
    nv.moe_fc1(x, row_token, off, gated, E, I, K, g, nv.MOE_SILU_GLU, out=big[:, :I])
    I2 = 196
    blob2 = nv.repack(u8_dev(c.w[:, :I2]), u8_dev(c.s[:, :I2]))
    h2 = nv.grouped_gemm_gather(x, row_token, off, blob2, E, I2, K, g)
    r2 = nv.moe_fc1(x, row_token, off, blob2, E, I2, K, g, nv.MOE_RELU2)
    ref2 = nv.moe_relu2(h2)
    torch.cuda.synchronize()
    assert torch.equal(big[:, :I], a)
    assert torch.all(big[:, I:] == 7.0)
    assert torch.equal(r2, ref2)


@pytest.mark.parametrize("T", [16, 2048])
def test_fused_silu_at_benchmark_size(T):
    """E = 128, top-8, hidden 2048, I = 768 (the benchmark's MoE layer): bitwise against the unfused chain, and
    sampled outputs against the oracle (each sample's gate and up outputs computed on their own, rounded to bf16,
    then the activation)."""
    E, topk, I, K = 128, 8, 768, 2048
    c = Fc1Case(T, E, topk, I, K, seed=1004 + T)
    say(f"fused FC1 SiLU benchmark size T={T} R={T * topk}")
    off, row_token, x, _ = c.dev()
    g = f32_dev(c.g)
    w, s = u8_dev(c.w), u8_dev(c.s)
    h = nv.grouped_gemm_gather(x, row_token, off, nv.repack(w, s), E, 2 * I, K, g)
    a_ref = nv.moe_silu_mul(h)
    a = nv.moe_fc1(x, row_token, off, nv.repack_gated(w, s), E, I, K, g, nv.MOE_SILU_GLU)
    torch.cuda.synchronize()
    assert torch.equal(a, a_ref)
    R = T * topk
    rg = synth.rng(T + 99)
    rows, cols = rg.integers(0, R, 256), rg.integers(0, I, 256)
    xr = c.xt[c.r_rt]
    hg = oracle.grouped_gemm_sampled(xr, c.r_off, c.w, c.s, c.g, False, None, rows, cols)
    hu = oracle.grouped_gemm_sampled(xr, c.r_off, c.w, c.s, c.g, False, None, rows, cols + I)
    # [samples, 2]: gate | up, each rounded once (RNE) from the exact value (bf16 values convert exactly)
    hb = np.stack([synth.bf16_bits_from_f32(oracle.round_bf16_np(v).astype(np.float32)) for v in (hg, hu)], axis=1)
    ref = oracle.silu_mul(hb)[:, 0]
    ok, info = oracle.accept(to_f64(a)[rows, cols], ref)
    assert ok, info


@pytest.mark.parametrize("T", [16, 256])
def test_moe_layer_with_fused_fc1(T):
    """route -> fused FC1 (gathered) -> FC2 -> combine equals the unfused layer bitwise."""
    E, topk, Hd, I = 16, 4, 256, 192
    c = Fc1Case(T, E, topk, I, Hd, seed=T + 11)
    g = synth.rng(T + 12)
    w2, s2 = synth.random_codes(g, (E, Hd, I)), synth.scales_pow2_mant(g, (E, Hd, I // 16))
    g2 = (np.exp2(g.integers(-2, 3, E).astype(np.float64)) / 2688).astype(np.float32)
    wts = torch.from_numpy(g.random((T, topk)).astype(np.float32)).to(DEV)
    say(f"moe layer with fused FC1 T={T}")
    off, row_token, x, _ = c.dev()
    _, _, token_row = nv.moe_route(i32_dev(c.ids), E)
    w, s = u8_dev(c.w), u8_dev(c.s)
    b2 = nv.repack(u8_dev(w2), u8_dev(s2))
    g1 = f32_dev(c.g)
    a0 = nv.moe_silu_mul(nv.grouped_gemm_gather(x, row_token, off, nv.repack(w, s), E, 2 * I, Hd, g1))
    out0 = nv.moe_combine(nv.grouped_gemm(a0, off, b2, E, Hd, I, f32_dev(g2)), token_row, wts)
    a1 = nv.moe_fc1(x, row_token, off, nv.repack_gated(w, s), E, I, Hd, g1, nv.MOE_SILU_GLU)
    out1 = nv.moe_combine(nv.grouped_gemm(a1, off, b2, E, Hd, I, f32_dev(g2)), token_row, wts)
    torch.cuda.synchronize()
    assert torch.equal(out1, out0)
