"""MXFP4 weight-only (E2M1 codes, one E8M0 scale per 32 K, no global scale; SGLang compressed-tensors NVFP4
weight-only page, Modifications, the paragraph on MXFP4) on the GPU, through the mxfp4_* entry points.

The decoded tile is bit-exact for every one of the 256 E8M0 codes under every E2M1 code (RNE to bf16 of the exact
product: exact where it lies in bf16's range, infinite beyond, NaN for the NaN code); one-hot activations push
every code under every E8M0 scale whose products stay in the activation type's normal range through every
kernel bit-exactly; GEMM outputs meet the oracle's acceptance bound on every variant, dense and grouped, bf16 and
fp16, with and without a pre-quant scale; the pre-scale invariant holds bit for bit."""
import numpy as np
import pytest
import torch

import oracle
import synth
import weight_only_fp4_amd as nv
from gpu_util import DEV, act_dev, bits16, to_f64, u8_dev

pytestmark = pytest.mark.gpu

ONE = {"bf16": 0x3F80, "f16": 0x3C00}
# E8M0 bytes whose products with every E2M1 code lie in the normal range of the activation type
EXACT = {"bf16": np.arange(2, 253), "f16": np.arange(114, 141)}


def say(msg):
    print(f"[gpu-case] {msg}", flush=True)


def accept_or_fail(y, ref, what):
    ok, info = oracle.accept(y, ref)
    assert ok, (what, info)


def enumeration_weight(scales):
    """len(scales) rows x K = 256: row n has E8M0 byte scales[n] on all 8 of its 32-groups and code (n + k) % 16 at
    k, so every 32-group holds every code twice."""
    N, K = len(scales), 256
    codes = (np.arange(K)[None, :] + np.arange(N)[:, None]) % 16
    w = synth.pack_codes(codes.astype(np.uint8))
    s = np.repeat(np.asarray(scales, dtype=np.uint8)[:, None], K // 32, axis=1)
    return w, s


def test_dequant_tile_bit_exact_for_every_e8m0_code():
    w, s = enumeration_weight(np.arange(256))
    N, K = s.shape[0], 256
    say("mxfp4 dequant all 256 E8M0 codes")
    blob = nv.repack_mxfp4(u8_dev(w), u8_dev(s))
    got = to_f64(nv.dequant_mxfp4(blob, 1, N, K))[0]
    exp = oracle.round_bf16_np(oracle.dequant(w, s, "mxfp4"))      # exact, or +-inf past bf16's range, NaN for 0xFF
    assert np.array_equal(got, exp, equal_nan=True), np.argwhere(~((got == exp) | (np.isnan(got) & np.isnan(exp))))[:5]
    assert np.isnan(got[255]).all() and np.isinf(got[254]).any()


FORMS = [
    ("small_m_4rows", nv.VARIANT_SMALL_M, 4),
    ("small_m_8rows", nv.VARIANT_SMALL_M, 8),
    ("small_m_16rows", nv.VARIANT_SMALL_M, 16),
    ("resident_16rows", nv.VARIANT_RESIDENT, 16),
    ("resident_5rows", nv.VARIANT_RESIDENT, 5),
    ("tile_256rows", nv.VARIANT_LARGE_M, 256),
    ("mfma_2304rows", nv.VARIANT_MFMA, 2304),
    ("mfma_quarter_2304rows", nv.VARIANT_MFMA_QUARTER, 2304),
]


@pytest.mark.parametrize("act", ["bf16", "f16"])
@pytest.mark.parametrize("name,variant,rows", FORMS, ids=[f[0] for f in FORMS])
def test_every_kernel_decodes_every_code_under_every_scale(name, variant, rows, act):
    w, s = enumeration_weight(EXACT[act])
    N, K = s.shape[0], 256
    T = oracle.dequant(w, s, "mxfp4")
    say(f"mxfp4 decode enumeration {name} {act} N={N}")
    blob = nv.repack_mxfp4(u8_dev(w), u8_dev(s))
    for k0 in range(0, K, rows):
        r = min(rows, K - k0) if rows <= K else rows
        x = np.zeros((r, K), dtype=np.uint16)
        ks = (k0 + np.arange(r)) % K
        x[np.arange(r), ks] = ONE[act]
        y = to_f64(nv.gemm_variant_mxfp4(act_dev(x, act), blob, N, K, variant=variant))
        assert np.array_equal(y, T[:, ks].T), (name, act, k0, np.argwhere(y != T[:, ks].T)[:5])


@pytest.mark.parametrize("act", ["bf16", "f16"])
@pytest.mark.parametrize("rows", [4, 16, 256], ids=["small_m_4rows", "small_m_16rows", "tile_256rows"])
def test_grouped_kernels_decode_every_code_under_every_scale(rows, act):
    """The enumeration weight is expert 1 of 3 (experts 0 and 2 random, with no rows)."""
    w1, s1 = enumeration_weight(EXACT[act])
    N, K = s1.shape[0], 256
    g = synth.rng(81)
    w = np.stack([synth.random_codes(g, (N, K)), w1, synth.random_codes(g, (N, K))])
    s = np.stack([synth.scales_e8m0(g, (N, K // 32)), s1, synth.scales_e8m0(g, (N, K // 32))])
    T = oracle.dequant(w1, s1, "mxfp4")
    say(f"mxfp4 grouped decode enumeration rows={rows} {act}")
    blob = nv.repack_mxfp4(u8_dev(w), u8_dev(s))
    for k0 in range(0, K, rows):
        r = min(rows, K - k0)
        x = np.zeros((r, K), dtype=np.uint16)
        x[np.arange(r), k0 + np.arange(r)] = ONE[act]
        off = torch.tensor([0, 0, r, r], dtype=torch.int32, device=DEV)
        y = to_f64(nv.grouped_gemm_mxfp4(act_dev(x, act), off, blob, 3, N, K))
        assert np.array_equal(y, T[:, k0:k0 + r].T), (rows, act, k0)


DENSE = [
    ("tiny_4x256x512", dict(M=4, N=256, K=512, seed=3101)),
    ("ragged_33x1000x1056_pre", dict(M=33, N=1000, K=1056, seed=3102, prescale=True)),
    ("decode_16x4096x4096", dict(M=16, N=4096, K=4096, seed=3103)),
    ("decode_8x2000x8192_pre", dict(M=8, N=2000, K=8192, seed=3104, prescale=True)),
    ("mid_300x700x2048", dict(M=300, N=700, K=2048, seed=3105)),
    ("prefill_pre_512x2048x1056", dict(M=512, N=2048, K=1056, seed=3106, prescale=True)),
]


@pytest.mark.parametrize("act", ["bf16", "f16"])
@pytest.mark.parametrize("name,kw", DENSE, ids=[d[0] for d in DENSE])
def test_dense_parity_every_variant(name, kw, act):
    c = synth.dense_case(fmt="mxfp4", act=act, **kw)
    say(f"mxfp4 dense {name} {act}")
    x = act_dev(c.x, act)
    pre = None if c.pre is None else act_dev(c.pre, act)
    blob = nv.repack_mxfp4(u8_dev(c.w), u8_dev(c.s))
    ref = (oracle.gemm_f16 if act == "f16" else oracle.gemm)(c.x, c.w, c.s, 1.0, False, c.pre, fmt="mxfp4")
    for v in nv.gemm_variants(c.M, c.N, c.K) + [nv.VARIANT_MFMA_QUARTER]:
        y = nv.gemm_variant_mxfp4(x, blob, c.N, c.K, pre, variant=v)
        assert y.dtype == x.dtype
        accept_or_fail(to_f64(y), ref, (name, act, v))
    # pre-scale invariant, bit for bit
    if pre is not None:
        xs = (oracle.activation(c.x, c.pre).astype(np.float32) if act == "bf16" else
              oracle.activation_f16(c.x, c.pre))
        xs = synth.bf16_bits_from_f32(xs) if act == "bf16" else xs.astype(np.float16).view(np.uint16)
        for v in nv.gemm_variants(c.M, c.N, c.K):
            assert np.array_equal(bits16(nv.gemm_variant_mxfp4(act_dev(xs, act), blob, c.N, c.K, None, variant=v)),
                                  bits16(nv.gemm_variant_mxfp4(x, blob, c.N, c.K, pre, variant=v))), (name, v)


@pytest.mark.parametrize("act", ["bf16", "f16"])
@pytest.mark.parametrize("T,E,topk,N,K", [(16, 32, 4, 96, 256), (256, 4, 2, 300, 288)])
def test_grouped_parity(T, E, topk, N, K, act):
    """Grouped small-M path (few rows per expert) and grouped tile path (R > 16 E), with a pre-scale."""
    gc = synth.grouped_case(T=T, E=E, topk=topk, N=N, K=K, seed=T + N + 7, prescale=True, act=act, fmt="mxfp4")
    say(f"mxfp4 grouped T={T} R={gc.R} E={E} {act}")
    x = act_dev(gc.x, act)
    off = torch.from_numpy(gc.offsets.astype(np.int32)).to(DEV)
    blob = nv.repack_mxfp4(u8_dev(gc.w), u8_dev(gc.s))
    y = nv.grouped_gemm_mxfp4(x, off, blob, E, N, K, act_dev(gc.pre, act))
    f = oracle.grouped_gemm_f16 if act == "f16" else oracle.grouped_gemm
    ref = f(gc.x, gc.offsets, gc.w, gc.s, None, False, gc.pre, fmt="mxfp4")
    accept_or_fail(to_f64(y), ref, ("mxfp4 grouped", T, E, act))


@pytest.mark.parametrize("act", ["bf16", "f16"])
def test_nan_scale_code_propagates_in_every_kernel(act):
    """The E8M0 NaN code (0xFF) on a 32-wide K group makes exactly its output column NaN in every dense variant
    (M = 4, 16 and 300 reach the small-M, activation-resident, tile and MFMA-bound kernels) and in the grouped
    kernels (small-M and tile), for that expert's rows only; every other output matches the oracle.  The kernels
    apply E8M0 scales inside the E2M1 conversion, so this pins that the NaN code still gives NaN there."""
    bad = [(3, 0), (17, 5), (40, 7)]                     # (row n, 32-wide K group)
    for M in (4, 16, 300):
        c = synth.dense_case(M, 64, 256, seed=91 + M, act=act, fmt="mxfp4")
        s = c.s.copy()
        for n, b in bad:
            s[n, b] = 0xFF
        c.s = s
        say(f"mxfp4 nan scale code dense M={M} {act}")
        x = act_dev(c.x, act)
        blob = nv.repack_mxfp4(u8_dev(c.w), u8_dev(c.s))
        ref = (oracle.gemm_f16 if act == "f16" else oracle.gemm)(c.x, c.w, c.s, 1.0, False, None, fmt="mxfp4")
        nan_cols = sorted({n for n, _ in bad})
        assert np.all(np.isnan(ref[:, nan_cols]))
        keep = [n for n in range(c.N) if n not in nan_cols]
        for v in nv.gemm_variants(M, c.N, c.K):
            y = to_f64(nv.gemm_variant_mxfp4(x, blob, c.N, c.K, variant=v))
            assert np.array_equal(np.isnan(y), np.isnan(ref)), (M, v)
            accept_or_fail(y[:, keep], ref[:, keep], ("mxfp4 nan code", M, act, v))
    for T in (16, 256):                                  # grouped small-M and tile paths
        gc = synth.grouped_case(T=T, E=4, topk=2, N=64, K=256, seed=T + 5, act=act, fmt="mxfp4")
        w_s = gc.s.copy()
        for n, b in bad:
            w_s[1, n, b] = 0xFF                          # expert 1 only
        say(f"mxfp4 nan scale code grouped T={T} {act}")
        x = act_dev(gc.x, act)
        off = torch.from_numpy(gc.offsets.astype(np.int32)).to(DEV)
        blob = nv.repack_mxfp4(u8_dev(gc.w), u8_dev(w_s))
        y = to_f64(nv.grouped_gemm_mxfp4(x, off, blob, 4, 64, 256))
        f = oracle.grouped_gemm_f16 if act == "f16" else oracle.grouped_gemm
        ref = f(gc.x, gc.offsets, gc.w, w_s, None, False, None, fmt="mxfp4")
        nan = np.zeros(ref.shape, dtype=bool)
        for n, _ in bad:
            nan[gc.offsets[1]:gc.offsets[2], n] = True
        assert np.array_equal(np.isnan(ref), nan)
        assert np.array_equal(np.isnan(y), nan), T
        accept_or_fail(np.where(nan, 0.0, y), np.where(nan, 0.0, ref), ("mxfp4 nan code grouped", T, act))
