"""Parity of the fp16 activation / output form (X, pre-quant scale and Y in IEEE binary16) with the CPU oracle's
fp16 definition, on the GPU, through the *_f16 entry points: every kernel variant on decode, ragged, prefill-like
and grouped shapes within the acceptance bound of ``oracle.accept``; the identity product bit-exact (decoded
weights are exact in fp16); the divisor and pre-scale invariants bit-exact; outputs past the fp16 range become
infinities exactly where the oracle's value rounds past 65504."""
import numpy as np
import pytest
import torch

import oracle
import synth
import weight_only_fp4_amd as nv
from gpu_util import DEV, DenseDev, GroupedDev, bits16, f16_dev, f32_dev, to_f64, u8_dev

pytestmark = pytest.mark.gpu


def say(msg):
    print(f"[gpu-case] {msg}", flush=True)


def accept_or_fail(y, ref, what):
    ok, info = oracle.accept(y, ref)
    assert ok, (what, info)


def variants(M, K, N):
    """Every kernel variant that takes this shape, as the library reports it."""
    return nv.gemm_variants(M, N, K)


F16_DENSE = [
    ("tiny_4x256x512", dict(M=4, N=256, K=512, seed=2000)),
    ("ragged_33x1000x1040_pre_div", dict(M=33, N=1000, K=1040, seed=2001, prescale=True, g_stored=2688.0,
                                         g_is_divisor=True)),
    ("decode_M1", dict(M=1, N=2064, K=4096, seed=2002, g_stored=1 / 2688.0)),
    ("decode_M9_ragged", dict(M=9, N=2000, K=3968, seed=2003, g_stored=1 / 2688.0, prescale=True)),
    ("decode_M16", dict(M=16, N=14336, K=4096, seed=2004, g_stored=1 / 2688.0)),
    ("mid_300x700x2048", dict(M=300, N=700, K=2048, seed=2005, scales="log_uniform", g_stored=1 / 2688.0)),
    ("split_M24_N2000_K4096", dict(M=24, N=2000, K=4096, seed=2006)),
]


@pytest.mark.parametrize("name,kw", F16_DENSE, ids=[d[0] for d in F16_DENSE])
def test_f16_dense_parity_every_variant(name, kw):
    c = synth.dense_case(act="f16", **kw)
    say(f"f16 dense {name}")
    d = DenseDev(c)
    assert d.x.dtype == torch.float16
    ref = oracle.gemm_f16(c.x, c.w, c.s, c.g_stored, c.g_is_divisor, c.pre)
    for v in variants(c.M, c.K, c.N):
        y = d.run(v)
        assert y.dtype == torch.float16
        accept_or_fail(to_f64(y), ref, (name, v))


def test_f16_prefill_sampled():
    c = synth.dense_case(4096, 14336, 4096, 2007, act="f16", scales="log_uniform", g_stored=1 / 2688.0)
    say("f16 prefill sampled")
    d = DenseDev(c)
    y = to_f64(d.run())
    assert np.all(np.isfinite(y))
    g = synth.rng(2008)
    rows, cols = g.integers(0, c.M, 512), g.integers(0, c.N, 512)
    rows[:2], cols[:2] = [0, c.M - 1], [c.N - 1, 0]
    # each sampled output on its own: g * <X'[r], T[n]> with T's rows decoded by the oracle
    t = oracle.dequant(c.w[cols], c.s[cols])
    xa = oracle.activation_f16(c.x[rows])
    ref = oracle.global_scale(c.g_stored, False) * np.einsum("ik,ik->i", xa, t)
    accept_or_fail(y[rows, cols], ref, "f16 prefill")


@pytest.mark.parametrize("variant,M,N", [(nv.VARIANT_SMALL_M, 16, 40), (nv.VARIANT_RESIDENT, 16, 40),
                                         (nv.VARIANT_LARGE_M, 256, 300), (nv.VARIANT_MFMA, 256, 300)])
def test_f16_identity_activation_gives_tile_bit_exact(variant, M, N):
    """X = I, g = 1: each output is one exact product, so Y = T^T bit for bit in fp16."""
    K = M
    say(f"f16 identity variant {variant}")
    c = synth.dense_case(1, N, K, seed=9)
    eye = np.eye(K, dtype=np.float16).view(np.uint16)
    blob = nv.repack(u8_dev(c.w), u8_dev(c.s))
    y = to_f64(nv.gemm_variant(f16_dev(eye), blob, N, K, f32_dev(1.0), False, None, variant=variant))
    assert np.array_equal(y, oracle.dequant(c.w, c.s).T)


@pytest.mark.parametrize("variant", [nv.VARIANT_SMALL_M, nv.VARIANT_LARGE_M, nv.VARIANT_MFMA, nv.VARIANT_RESIDENT])
def test_f16_scale_invariants_bit_exact(variant):
    c = synth.dense_case(16, 520, 1040, seed=41, g_stored=2688.0, g_is_divisor=True, prescale=True, act="f16")
    say(f"f16 invariants variant {variant}")
    d = DenseDev(c)
    y = bits16(d.run(variant))
    ginv = np.float32(1.0) / np.float32(c.g_stored)
    assert np.array_equal(bits16(d.run(variant, g=f32_dev(ginv), divisor=False)), y)
    xs = oracle.activation_f16(c.x, c.pre).astype(np.float16).view(np.uint16)
    assert np.array_equal(bits16(d.run(variant, x=f16_dev(xs), pre=None)), y)


def test_f16_outputs_overflow_to_infinity_where_the_oracle_does():
    """fp16 has a narrow range: with a large global scale the outputs whose exact value rounds past 65504 are
    infinities of the right sign, the others finite and within the acceptance bound."""
    c = synth.dense_case(8, 512, 1024, seed=43, act="f16", g_stored=2000.0)
    say("f16 overflow")
    d = DenseDev(c)
    ref = oracle.gemm_f16(c.x, c.w, c.s, c.g_stored)
    big = np.abs(ref) >= 65520.0
    small = np.abs(ref) < 65000.0           # clear of the rounding boundary
    assert big.any() and small.any()
    for v in variants(c.M, c.K, c.N):
        y = to_f64(d.run(v))
        assert np.array_equal(y[big], np.sign(ref[big]) * np.inf), v
        ok, info = oracle.accept(y[small], ref[small])
        assert ok, (v, info)


@pytest.mark.parametrize("T,E,topk,N,K", [(16, 32, 4, 96, 256), (256, 4, 2, 300, 272)])
def test_f16_grouped_parity(T, E, topk, N, K):
    """Small-M grouped path (few rows per expert) and the tile grouped path (R > 16 E), with a pre-scale."""
    gc = synth.grouped_case(T=T, E=E, topk=topk, N=N, K=K, seed=T + N, prescale=True, act="f16")
    say(f"f16 grouped T={T} R={gc.R} E={E}")
    gd = GroupedDev(gc)
    y = gd.run()
    assert y.dtype == torch.float16
    ref = oracle.grouped_gemm_f16(gc.x, gc.offsets, gc.w, gc.s, gc.g_stored, False, gc.pre)
    accept_or_fail(to_f64(y), ref, ("f16 grouped", T, E))


def test_f16_rejects_mixed_dtypes():
    c = synth.dense_case(4, 32, 64, seed=44, act="f16")
    d = DenseDev(c)
    with pytest.raises(ValueError):
        nv.gemm(d.x, d.blob, c.N, c.K, d.g, pre_scale=torch.ones(c.K, dtype=torch.bfloat16, device=DEV))
    with pytest.raises(ValueError):
        nv.gemm(d.x, d.blob, c.N, c.K, d.g, out=torch.empty((c.M, c.N), dtype=torch.bfloat16, device=DEV))
