"""The grouped GEMM's three kernels on the same inputs: small-M (passes of 16 rows), tile (64-row tiles) and the
MFMA-bound kernel in 256-row tiles per expert (whose row blocks past an expert's last row skip their MFMAs), each
against the oracle.  Experts take row counts around the tile edges (0, 1, 255, 256, 257, ...), N and K tails, the
pre-scale, the gather, fp16, MXFP4 and the gated SiLU epilogue; the gated epilogue of the MFMA-bound kernel must
equal, bitwise, its plain output followed by the standalone SiLU.  At the benchmark's MoE sizes the oracle is
evaluated on sampled outputs."""
import numpy as np
import pytest
import torch

import oracle
import synth
import weight_only_fp4_amd as nv
from gpu_util import DEV, act_dev, bits16, f32_dev, to_f64, u8_dev

pytestmark = pytest.mark.gpu

KERNELS = [nv.GROUPED_SMALL_M, nv.GROUPED_TILE, nv.GROUPED_MFMA]


def say(msg):
    print(f"[gpu-case] {msg}", flush=True)


class Experts:
    """E experts with the given row counts: grouped rows X[R, K], weights [E, N, K], per-expert global scales."""

    def __init__(self, rows, N, K, seed, act="bf16", fmt="nvfp4", pre=False):
        g = synth.rng(seed)
        self.E, self.N, self.K, self.act, self.fmt = len(rows), N, K, act, fmt
        self.offsets = np.zeros(self.E + 1, dtype=np.int32)
        self.offsets[1:] = np.cumsum(rows)
        self.R = int(self.offsets[-1])
        self.x = synth.normal_act(g, (self.R, K), act)
        self.w = synth.random_codes(g, (self.E, N, K))
        if fmt == "mxfp4":
            self.s = synth.scales_e8m0(g, (self.E, N, K // 32))
            self.g = np.ones(self.E, np.float32)
        else:
            self.s = synth.scales_pow2_mant(g, (self.E, N, K // 16))
            self.g = (np.exp2(g.integers(-2, 3, self.E).astype(np.float64)) / 2688).astype(np.float32)
        self.pre = synth.awq_prescale(g, K, act) if pre else None

    def blob(self, gated=False):
        w, s = u8_dev(self.w), u8_dev(self.s)
        if self.fmt == "mxfp4":
            return nv.repack_mxfp4(w, s)
        return nv.repack_gated(w, s) if gated else nv.repack(w, s)

    def run(self, blob, variant, activation=0):
        p = None if self.pre is None else act_dev(self.pre, self.act)
        return nv.grouped_gemm_variant(act_dev(self.x, self.act), None, i32_dev(self.offsets), blob, self.E, self.N,
                                       self.K, f32_dev(self.g), variant, activation, pre_scale=p,
                                       mxfp4=self.fmt == "mxfp4")

    def ref(self):
        f = oracle.grouped_gemm if self.act == "bf16" else oracle.grouped_gemm_f16
        return f(self.x, self.offsets, self.w, self.s, self.g, False, self.pre, fmt=self.fmt)


def i32_dev(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(DEV)


CASES = [   # (rows per expert, N, K, pre)
    ([0, 1, 255, 256, 257, 600, 0, 33], 272, 384, False),   # tile edges, an N tail (17 units), K a multiple of 128
    ([300, 5, 0, 512], 256, 272, True),                     # K tail (272), pre-scale
    ([64], 48, 128, False),                                 # one expert, three units
]


@pytest.mark.parametrize("act", ["bf16", "f16"])
@pytest.mark.parametrize("rows,N,K,pre", CASES)
def test_grouped_kernels_agree_with_oracle(rows, N, K, pre, act):
    c = Experts(rows, N, K, seed=sum(rows) + N + K, act=act, pre=pre)
    say(f"grouped kernels rows={rows} N={N} K={K} pre={pre} act={act}")
    blob = c.blob()
    ys = [c.run(blob, v) for v in KERNELS]
    again = c.run(blob, nv.GROUPED_MFMA)
    torch.cuda.synchronize()
    assert torch.equal(again, ys[2])                         # run to run
    ref = c.ref()
    for v, y in zip(KERNELS, ys):
        ok, info = oracle.accept(to_f64(y), ref, out=act)
        assert ok, (v, info)


def test_grouped_mfma_mxfp4():
    c = Experts([256, 100, 3, 0, 300], 512, 256, seed=5, fmt="mxfp4")
    say("grouped MFMA-bound kernel, MXFP4")
    blob = c.blob()
    ref = c.ref()
    for v in KERNELS:
        ok, info = oracle.accept(to_f64(c.run(blob, v)), ref)
        assert ok, (v, info)


@pytest.mark.parametrize("rows", [[0, 1, 255, 256, 257, 600, 0, 33], [40, 700, 2]])
def test_grouped_mfma_gated_silu_epilogue(rows):
    """The gated epilogue equals the plain output of the same kernel followed by the SiLU kernel, bitwise, and
    the tile kernel's gated epilogue within the bound."""
    I, K = 96, 256
    c = Experts(rows, 2 * I, K, seed=len(rows) * 13 + I)
    say(f"grouped MFMA-bound gated SiLU rows={rows}")
    plain = c.run(c.blob(), nv.GROUPED_MFMA)
    gated = c.blob(gated=True)
    fused = c.run(gated, nv.GROUPED_MFMA, nv.MOE_SILU_GLU)
    fused_tile = c.run(gated, nv.GROUPED_TILE, nv.MOE_SILU_GLU)
    ref = nv.moe_silu_mul(plain)
    torch.cuda.synchronize()
    assert torch.equal(fused, ref)
    ok, info = oracle.accept(to_f64(fused_tile), oracle.silu_mul(bits16(plain)))
    assert ok, info


def test_grouped_mfma_gather_and_prescale():
    """Rows read through the token gather (row index) on the MFMA-bound kernel equal the pre-gathered rows."""
    gc = synth.grouped_case(T=256, E=4, topk=2, N=300, K=272, seed=41, prescale=True)
    say(f"grouped MFMA-bound gather R={gc.R}")
    T = gc.meta["T"]
    xt = np.empty((T, gc.K), dtype=np.uint16)
    xt[gc.meta["token_of_row"]] = gc.x
    off = i32_dev(gc.offsets)
    blob = nv.repack(u8_dev(gc.w), u8_dev(gc.s))
    g, p = f32_dev(gc.g_stored), act_dev(gc.pre, "bf16")
    row_token = i32_dev(gc.meta["token_of_row"])
    y_gather = nv.grouped_gemm_variant(act_dev(xt, "bf16"), row_token, off, blob, gc.E, gc.N, gc.K, g,
                                       nv.GROUPED_MFMA, pre_scale=p)
    y_plain = nv.grouped_gemm_variant(act_dev(gc.x, "bf16"), None, off, blob, gc.E, gc.N, gc.K, g, nv.GROUPED_MFMA,
                                      pre_scale=p)
    torch.cuda.synchronize()
    assert torch.equal(y_gather, y_plain)
    ref = oracle.grouped_gemm(gc.x, gc.offsets, gc.w, gc.s, gc.g_stored, False, gc.pre)
    ok, info = oracle.accept(to_f64(y_gather), ref)
    assert ok, info


@pytest.mark.parametrize("fc", ["fc1", "fc2"])
def test_grouped_mfma_at_benchmark_size(fc):
    """E = 128, top-8, T = 2048 (R = 16384 rows, Zipf routing: 128 rows per expert on average, so the automatic
    choice takes the tile kernel): the tile and MFMA-bound kernels against the oracle on stratified samples (every
    expert)."""
    K, N = (2048, 1536) if fc == "fc1" else (768, 2048)
    gc = synth.grouped_case(T=2048, E=128, topk=8, N=N, K=K, seed=1004, x_source="fresh")
    say(f"grouped benchmark size {fc} R={gc.R}")
    off, blob, g = i32_dev(gc.offsets), nv.repack(u8_dev(gc.w), u8_dev(gc.s)), f32_dev(gc.g_stored)
    x = act_dev(gc.x, "bf16")
    y = nv.grouped_gemm_variant(x, None, off, blob, gc.E, N, K, g, nv.GROUPED_AUTO)
    y_mfma = nv.grouped_gemm_variant(x, None, off, blob, gc.E, N, K, g, nv.GROUPED_MFMA)
    y_tile = nv.grouped_gemm_variant(x, None, off, blob, gc.E, N, K, g, nv.GROUPED_TILE)
    torch.cuda.synchronize()
    assert torch.equal(y, y_tile)
    rg = synth.rng(7)
    rows = np.concatenate([gc.offsets[e] + rg.integers(0, c, 2) for e, c in enumerate(np.diff(gc.offsets)) if c > 0])
    cols = rg.integers(0, N, rows.shape[0])
    ref = oracle.grouped_gemm_sampled(gc.x, gc.offsets, gc.w, gc.s, gc.g_stored, False, None, rows, cols)
    ok, info = oracle.accept(to_f64(y_mfma)[rows, cols], ref)
    assert ok, info
    ok, info = oracle.accept(to_f64(y_tile)[rows, cols], ref)
    assert ok, info


def test_grouped_auto_takes_mfma_for_many_rows_per_expert():
    """256 rows per expert on average: the automatic choice is the MFMA-bound kernel (bitwise its output)."""
    c = Experts([300, 212, 256, 256], 256, 256, seed=77)
    say("grouped auto choice at 256 rows per expert")
    blob = c.blob()
    torch.cuda.synchronize()
    assert torch.equal(c.run(blob, nv.GROUPED_AUTO), c.run(blob, nv.GROUPED_MFMA))


@pytest.mark.parametrize("act", ["bf16", "f16"])
@pytest.mark.parametrize("K,pre", [(256, False), (272, True)])
def test_grouped_small_m_four_row_passes(K, pre, act):
    """At most one row per expert on average (R <= E) the small-M kernel runs its 4-row form, taking an expert's
    rows in passes of 4: experts of 9, 5 and 4 rows (three, two and one passes) against the oracle, and the gated
    SiLU epilogue bitwise against the plain output followed by the standalone SiLU."""
    rows = [9, 5, 4, 3, 2, 1, 1, 1] + [0] * 24            # R = 26 <= E = 32
    I = 48
    c = Experts(rows, 2 * I, K, seed=K + 9 * pre, act=act, pre=pre)
    say(f"grouped small-M 4-row passes K={K} pre={pre} act={act}")
    plain = c.run(c.blob(), nv.GROUPED_SMALL_M)
    auto = c.run(c.blob(), nv.GROUPED_AUTO)
    fused = c.run(c.blob(gated=True), nv.GROUPED_SMALL_M, nv.MOE_SILU_GLU)
    ref_silu = nv.moe_silu_mul(plain)
    torch.cuda.synchronize()
    assert torch.equal(auto, plain)
    assert torch.equal(fused, ref_silu)
    ok, info = oracle.accept(to_f64(plain), c.ref(), out=act)
    assert ok, info


@pytest.mark.parametrize("fmt", ["nvfp4", "mxfp4"])
def test_grouped_small_m_four_row_passes_relu2_and_formats(fmt):
    """The 4-row form (R <= E) with MXFP4 weights and the squared-ReLU epilogue: the plain output against the
    oracle, and the fused squared ReLU bitwise against the plain output followed by the standalone kernel."""
    rows = [0, 7, 1, 0, 4, 2, 0, 3] + [0] * 12             # R = 17 <= E = 20
    c = Experts(rows, 80, 320, seed=3 + len(fmt), fmt=fmt)
    say(f"grouped small-M 4-row passes, squared ReLU, {fmt}")
    blob = c.blob()
    plain = c.run(blob, nv.GROUPED_SMALL_M)
    fused = c.run(blob, nv.GROUPED_SMALL_M, nv.MOE_RELU2)
    ref_relu2 = nv.moe_relu2(plain)
    torch.cuda.synchronize()
    assert torch.equal(fused, ref_relu2)
    ok, info = oracle.accept(to_f64(plain), c.ref())
    assert ok, info


@pytest.mark.parametrize("rows", [[3, 0, 9, 1, 2, 0, 1] + [0] * 9,    # R = 16 <= E: the 4-row small-M form
                                  [40, 0, 300, 17]])
def test_grouped_nan_scale_codes_propagate(rows):
    """E4M3 NaN scale bytes (0x7F, 0xFF) in one expert's weight rows make exactly those output columns NaN for that
    expert's rows, in every grouped kernel (4-row or dynamic small-M, tile, MFMA-bound); every other output matches
    the oracle."""
    N, K = 96, 256
    c = Experts(rows, N, K, seed=len(rows) + sum(rows))
    bad = [(0, 5, 2, 0x7F), (2, 40, 7, 0xFF), (2, 41, 0, 0x7F)]    # (expert, row n, scale block, byte)
    for e, n, b, v in bad:
        c.s[e, n, b] = v
    say(f"grouped NaN scale codes rows={rows}")
    blob = c.blob()
    ref = c.ref()
    nan = np.zeros(ref.shape, dtype=bool)
    for e, n, _, _ in bad:
        nan[c.offsets[e]:c.offsets[e + 1], n] = True
    assert np.all(np.isnan(ref[nan]))
    for v in KERNELS:
        y = to_f64(c.run(blob, v))
        assert np.array_equal(np.isnan(y), nan), v
        ok, info = oracle.accept(np.where(nan, 0.0, y), np.where(nan, 0.0, ref))
        assert ok, (v, info)
