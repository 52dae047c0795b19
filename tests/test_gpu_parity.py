"""Parity of the HIP path (through the C ABI) with the CPU oracle, on the GPU.

Bars: decoded weight tiles bit-exact; GEMM outputs within the acceptance
bound of ``oracle.accept`` (relative Frobenius error <= 2e-3, every element
within 1e-2 * (|ref| + rms(ref)), all finite); hand cases, the identity
product and the scale invariants bit-exact.  Small sizes use the full oracle;
the full-size workloads use outputs the oracle computes one by one.
"""
import math
import os

import numpy as np
import pytest
import torch

import oracle
import synth
import weight_only_fp4_amd as nv
from gpu_util import DEV, DenseDev, GroupedDev, bf16_bits, bf16_dev, f32_dev, to_f64, u8_dev

pytestmark = pytest.mark.gpu

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def say(msg):
    print(f"[gpu-case] {msg}", flush=True)


def accept_or_fail(y, ref, what, slack=None):
    ok, info = oracle.accept(y, ref, slack=slack)
    assert ok, (what, info)
    return info


def dense_variants(M: int, K: int, N: int):
    """Every kernel variant that takes this shape, as the library reports it (automatic, small-M, tile,
    MFMA-bound, activation-resident)."""
    return nv.gemm_variants(M, N, K)


def oracle_bf16_bits(t64: np.ndarray) -> np.ndarray:
    """fp64 values exactly representable in bf16 -> bf16 bit patterns (sign of zero kept)."""
    f = t64.astype(np.float32)
    assert np.array_equal(f.astype(np.float64), t64, equal_nan=True)
    return (f.view(np.uint32) >> 16).astype(np.uint16)


# ------------------------------------------------------------ decode tiles --

def _enumeration_weight():
    """254 rows (one per finite E4M3 code) x 256 k; each 16-wide block holds all 16 codes, rotated per row."""
    finite = [b for b in range(256) if b not in (0x7F, 0xFF)]
    N, K = len(finite), 256
    codes = (np.arange(K)[None, :] + np.arange(N)[:, None]) % 16
    w = synth.pack_codes(codes.astype(np.uint8))
    s = np.repeat(np.array(finite, dtype=np.uint8)[:, None], K // 16, axis=1)
    return w, s


@pytest.mark.parametrize("case", ["enumeration", "ragged", "grouped"])
def test_dequant_tiles_bit_exact(case):
    say(f"dequant {case}")
    if case == "enumeration":
        w, s = _enumeration_weight()
        w, s = w[None], s[None]
    elif case == "ragged":
        c = synth.ragged_case()
        w, s = c.w[None], c.s[None]
    else:
        gc = synth.grouped_case(T=8, E=3, topk=2, N=40, K=272, seed=5)
        w, s = gc.w, gc.s
    E, N, K = w.shape[0], w.shape[1], w.shape[2] * 2
    blob = nv.repack(u8_dev(w if E > 1 else w[0]), u8_dev(s if E > 1 else s[0]))
    got = bf16_bits(nv.dequant(blob, E, N, K))
    for e in range(E):
        ref = oracle_bf16_bits(oracle.dequant(w[e], s[e]))
        assert np.array_equal(got[e], ref), (case, e, np.argwhere(got[e] != ref)[:5])


def test_repack_is_deterministic_and_pure():
    say("repack twice")
    c = synth.ragged_case()
    w, s = u8_dev(c.w), u8_dev(c.s)
    w0, s0 = w.clone(), s.clone()
    b1, b2 = nv.repack(w, s), nv.repack(w, s)
    torch.cuda.synchronize()
    assert torch.equal(b1, b2)
    assert torch.equal(w, w0) and torch.equal(s, s0)


# -------------------------------------------------------------- hand cases --

def _read_hand():
    rows = {}
    for line in open(os.path.join(GOLDEN, "hand_cases.txt")):
        line = line.strip()
        if line and not line.startswith("#"):
            p = line.split()
            rows[p[0]] = [float(v) for v in p[1:]]
    return rows


@pytest.mark.parametrize("variant", [nv.VARIANT_SMALL_M, nv.VARIANT_LARGE_M, nv.VARIANT_MFMA,
                                     nv.VARIANT_RESIDENT])
@pytest.mark.parametrize("case", ["H1", "H2", "H3", "H4"])
def test_hand_cases_exact(case, variant):
    from test_oracle_pins import _hand_inputs
    say(f"hand case {case} variant {variant}")
    x, w, s, g, div, pre = _hand_inputs(case)
    blob = nv.repack(u8_dev(w), u8_dev(s))
    y = nv.gemm_variant(bf16_dev(x), blob, 16, 16, f32_dev(g), div, None if pre is None else bf16_dev(pre),
                        variant=variant)
    got = to_f64(y)[0]
    exp = _read_hand()[case]
    for n in range(16):
        assert got[n] == exp[n], (case, variant, n, got[n], exp[n])


@pytest.mark.parametrize("variant,M,N", [(nv.VARIANT_SMALL_M, 16, 40), (nv.VARIANT_LARGE_M, 256, 300),
                                         (nv.VARIANT_RESIDENT, 16, 40)])
def test_identity_activation_gives_tile_bit_exact(variant, M, N):
    """X = I_K, g = 1: every output is one exact product, so Y = T^T bit for bit (signed zeros compare equal)."""
    K = M
    say(f"identity variant {variant} K={K} N={N}")
    c = synth.dense_case(1, N, K, seed=9)
    eye = synth.bf16_bits_from_f32(np.eye(K, dtype=np.float32))
    blob = nv.repack(u8_dev(c.w), u8_dev(c.s))
    y = to_f64(nv.gemm_variant(bf16_dev(eye), blob, N, K, f32_dev(1.0), False, None, variant=variant))
    assert np.array_equal(y, oracle.dequant(c.w, c.s).T)


# ------------------------------------------------------------ dense parity --

DENSE_FULL = [
    ("tiny", lambda: synth.tiny_case()),
    ("ragged_33x1000x1040", lambda: synth.ragged_case()),
    ("ragged_M13", lambda: synth.dense_case(13, 1000, 1040, 1003, g_stored=2688.0, g_is_divisor=True, prescale=True)),
    ("mid_300x700x2048", lambda: synth.dense_case(300, 700, 2048, 77, scales="log_uniform", g_stored=1 / 2688)),
    # split-K across workgroups with a ragged N tail / 2-tile rows / ragged last K chunk
    ("split_M24_N2000_K4096", lambda: synth.dense_case(24, 2000, 4096, 1005)),
    ("split_M48_N1000_K2176_pre", lambda: synth.dense_case(48, 1000, 2176, 1006, prescale=True)),
    ("split_M16_N4000_K2064", lambda: synth.dense_case(16, 4000, 2064, 1007, scales="log_uniform")),
    ("decode_M1", lambda: synth.decode_case(1)),
    ("decode_M8", lambda: synth.decode_case(8)),
    ("decode_M16", lambda: synth.decode_case(16)),
    ("decode_T_M1", lambda: synth.decode_case(1, N=4096, K=14336)),
    ("decode_T_M16", lambda: synth.decode_case(16, N=4096, K=14336)),
    ("lmhead_M1", lambda: synth.lmhead_case(1)),
    # the MFMA-bound kernel's pre-scale form (forced among the variants) with a divisor-stored global scale
    ("prefill_pre_512x2048x4096", lambda: synth.dense_case(512, 2048, 4096, 1009, prescale=True, g_stored=2688.0,
                                                           g_is_divisor=True)),
]


@pytest.mark.parametrize("name,make", DENSE_FULL, ids=[d[0] for d in DENSE_FULL])
def test_dense_parity_full_oracle(name, make):
    c = make()
    say(f"dense {name} M={c.M} N={c.N} K={c.K} pre={c.pre is not None} div={c.g_is_divisor}")
    d = DenseDev(c)
    ref = oracle.gemm(c.x, c.w, c.s, c.g_stored, c.g_is_divisor, c.pre)
    for v in dense_variants(c.M, c.K, c.N):
        accept_or_fail(to_f64(d.run(v)), ref, (name, v))


DENSE_SAMPLED = [
    ("prefill_4096x14336x4096", lambda: synth.prefill_case()),
    ("prefill_8192x17408x5120", lambda: synth.prefill_case(8192, 17408, 5120)),
    ("lmhead_M64", lambda: synth.lmhead_case(64)),
]


def stratified_samples(M, N, seed, tile_rows=128, tile_cols=256, per=2):
    """`per` random outputs in every tile_rows x tile_cols block of the output (every 256 x 256 tile of the
    MFMA-bound kernel and each of its 128-row halves, which the last partial wave of tiles runs as separate
    workgroups), plus the four corners."""
    g = synth.rng(seed)
    r0 = np.arange(0, M, tile_rows)
    c0 = np.arange(0, N, tile_cols)
    rr, cc = np.meshgrid(r0, c0, indexing="ij")
    rr, cc = np.repeat(rr.ravel(), per), np.repeat(cc.ravel(), per)
    rows = rr + (g.random(rr.size) * np.minimum(tile_rows, M - rr)).astype(np.int64)
    cols = cc + (g.random(cc.size) * np.minimum(tile_cols, N - cc)).astype(np.int64)
    return (np.concatenate([rows, [0, 0, M - 1, M - 1]]), np.concatenate([cols, [0, N - 1, 0, N - 1]]))


@pytest.mark.parametrize("name,make", DENSE_SAMPLED, ids=[d[0] for d in DENSE_SAMPLED])
def test_dense_parity_full_size_sampled(name, make):
    c = make()
    say(f"dense sampled {name}")
    d = DenseDev(c)
    y = to_f64(d.run())
    assert np.all(np.isfinite(y))
    rows, cols = stratified_samples(c.M, c.N, 123, tile_rows=min(128, c.M))
    ref = oracle.gemm_sampled(c.x, c.w, c.s, c.g_stored, c.g_is_divisor, c.pre, rows, cols)
    accept_or_fail(y[rows, cols], ref, name)


def test_wide_n_tile_ragged_sampled():
    """The wide-N 64-row tile shape (512 columns per workgroup) with N one unit past a multiple of 512 columns,
    K not a multiple of 128 and a pre-quant scale; every row and the last columns are sampled."""
    c = synth.dense_case(40, 65552, 1040, 1008, prescale=True, g_stored=2688.0, g_is_divisor=True)
    say(f"wide-N tile M={c.M} N={c.N} K={c.K}")
    d = DenseDev(c)
    y = to_f64(d.run(nv.VARIANT_LARGE_M))
    assert np.all(np.isfinite(y))
    g = synth.rng(321)
    rows = np.concatenate([np.arange(c.M).repeat(8), g.integers(0, c.M, 512)])
    cols = np.concatenate([np.tile(np.arange(c.N - 8, c.N), c.M), g.integers(0, c.N, 512)])
    ref = oracle.gemm_sampled(c.x, c.w, c.s, c.g_stored, c.g_is_divisor, c.pre, rows, cols)
    accept_or_fail(y[rows, cols], ref, "wide-N tile")


def test_small_and_large_variants_agree():
    c = synth.decode_case(8, N=2048, K=4096, seed=31)
    say("variants agree M=8")
    d = DenseDev(c)
    a, b = to_f64(d.run(nv.VARIANT_SMALL_M)), to_f64(d.run(nv.VARIANT_LARGE_M))
    ok, info = oracle.accept(a, b)
    assert ok, info


# ---------------------------------------------------------- grouped parity --

@pytest.mark.parametrize("fc", ["fc1", "fc2"])
def test_grouped_parity_T16_full_oracle(fc):
    gc = synth.moe_fc1_case(16) if fc == "fc1" else synth.moe_fc2_case(16)
    say(f"grouped {fc} T=16 R={gc.R} active={len(gc.active)}")
    assert len(gc.active) < gc.E      # some experts receive no rows
    d = GroupedDev(gc)
    y = to_f64(d.run())
    ref = oracle.grouped_gemm(gc.x, gc.offsets, gc.w, gc.s, gc.g_stored, gc.g_is_divisor, gc.pre)
    accept_or_fail(y, ref, fc)


@pytest.mark.parametrize("fc", ["fc1", "fc2"])
def test_grouped_parity_T2048_sampled(fc):
    gc = synth.moe_fc1_case(2048) if fc == "fc1" else synth.moe_fc2_case(2048)
    say(f"grouped {fc} T=2048 R={gc.R} active={len(gc.active)}")
    d = GroupedDev(gc)
    y = to_f64(d.run())
    assert np.all(np.isfinite(y))
    g = synth.rng(7)
    rows, cols = [], []
    for e in gc.active:
        a, b = int(gc.offsets[e]), int(gc.offsets[e + 1])
        rr = np.unique(np.concatenate([[a, b - 1], g.integers(a, b, 2)]))
        for r in rr:
            rows.extend([r] * 16)
            cols.extend(g.integers(0, gc.N, 16).tolist())
    rows, cols = np.array(rows), np.array(cols)
    ref = oracle.grouped_gemm_sampled(gc.x, gc.offsets, gc.w, gc.s, gc.g_stored, gc.g_is_divisor, gc.pre, rows, cols)
    accept_or_fail(y[rows, cols], ref, fc)


def test_grouped_tile_path_ragged_experts():
    """Enough rows per expert for the grouped tile kernel (64-row tiles): experts of 300, 0, 129, 1 and 70
    rows (an empty expert, whole tiles plus one row, a single row), N and K not multiples of 256 and 128,
    per-expert global scales stored as divisors, and a pre-quant scale."""
    counts = [300, 0, 129, 1, 70]
    route = np.repeat(np.arange(len(counts)), counts)
    synth.rng(17).shuffle(route)
    gc = synth.grouped_case(T=len(route), E=len(counts), topk=1, N=300, K=272, seed=12, prescale=True,
                            routing=route[:, None])
    gc.g_is_divisor = True
    gc.g_stored = (1.0 / gc.g_stored).astype(np.float32)
    assert list(np.diff(gc.offsets)) == counts
    say(f"grouped tile path R={gc.R} E={gc.E}")
    d = GroupedDev(gc)
    ref = oracle.grouped_gemm(gc.x, gc.offsets, gc.w, gc.s, gc.g_stored, True, gc.pre)
    accept_or_fail(to_f64(d.run()), ref, "grouped ragged experts")


def test_grouped_prescale_and_divisor_small_experts():
    gc = synth.grouped_case(T=40, E=6, topk=2, N=72, K=160, seed=3, prescale=True)
    gc.g_is_divisor = True
    gc.g_stored = (1.0 / gc.g_stored).astype(np.float32)
    say("grouped prescale+divisor")
    d = GroupedDev(gc)
    ref = oracle.grouped_gemm(gc.x, gc.offsets, gc.w, gc.s, gc.g_stored, True, gc.pre)
    accept_or_fail(to_f64(d.run()), ref, "grouped prescale")


def test_grouped_matches_per_expert_dense_calls():
    gc = synth.grouped_case(T=64, E=8, topk=2, N=96, K=256, seed=8)
    say("grouped vs per-expert dense")
    d = GroupedDev(gc)
    y = d.run()
    for e in gc.active:
        a, b = int(gc.offsets[e]), int(gc.offsets[e + 1])
        blob = nv.repack(d.w[e], d.s[e])
        ye = nv.gemm(d.x[a:b], blob, gc.N, gc.K, d.g[e:e + 1], False)
        ok, info = oracle.accept(to_f64(y[a:b]), to_f64(ye))
        assert ok, (e, info)


# -------------------------------------------------------------- invariants --

@pytest.mark.parametrize("variant", [nv.VARIANT_SMALL_M, nv.VARIANT_LARGE_M, nv.VARIANT_MFMA,
                                     nv.VARIANT_RESIDENT])
def test_scale_invariants_bit_exact(variant):
    c = synth.dense_case(16, 520, 1040, seed=41, g_stored=2688.0, g_is_divisor=True, prescale=True)
    say(f"invariants variant {variant}")
    d = DenseDev(c)
    y = bf16_bits(d.run(variant))
    # divisor flag == multiplier RN(1/v)
    ginv = np.float32(1.0) / np.float32(c.g_stored)
    assert np.array_equal(bf16_bits(d.run(variant, g=f32_dev(ginv), divisor=False)), y)
    # pre-scale == activation rounded on the host by the oracle's own rule, no pre-scale
    xs = synth.bf16_bits_from_f32(oracle.activation(c.x, c.pre).astype(np.float32))
    assert np.array_equal(bf16_bits(d.run(variant, x=bf16_dev(xs), pre=None)), y)
    # power-of-two scaling of X scales Y exactly
    x4 = synth.bf16_bits_from_f32(oracle.bf16_np(xs).astype(np.float32) * 4)
    y4 = to_f64(d.run(variant, x=bf16_dev(x4), pre=None))
    assert np.array_equal(y4, 4 * to_f64(d.run(variant)))


def test_divisor_inversion_restores_finite_outputs():
    c = synth.tiny_case()
    say("divisor inversion finite")
    d = DenseDev(c)
    big = f32_dev(2.0 ** 120)
    assert torch.isfinite(d.run(g=big, divisor=True)).all()
    assert not torch.isfinite(d.run(g=big, divisor=False)).all()   # used as a multiplier it overflows


# ------------------------------------------------------------------- edges --

def test_zero_sizes_return_ok_and_write_nothing():
    """M == 0, R == 0 or N == 0 through the C ABI with real device buffers: status OK, and a sentinel-filled
    output buffer handed to the call (as y, with the leading dimension of a real output) is untouched."""
    c = synth.tiny_case()
    say("zero sizes")
    d = DenseDev(c)
    L = nv.lib()
    st = nv._stream(torch.device(DEV))
    sentinel = torch.full((c.M, c.N), 7.0, dtype=torch.bfloat16, device=DEV)
    P = lambda t: None if t is None else nv._ptr(t)
    for fn in (L.nvfp4_w4a16_gemm, L.nvfp4_w4a16_gemm_f16):
        for M, N in ((0, c.N), (c.M, 0)):
            assert fn(P(d.x), c.K, None, P(d.blob), P(d.g), 0, P(sentinel), c.N, M, N, c.K, None, 0, st) == 0
    for v in (nv.VARIANT_SMALL_M, nv.VARIANT_LARGE_M, nv.VARIANT_MFMA, nv.VARIANT_RESIDENT, nv.VARIANT_MFMA_QUARTER):
        assert L.nvfp4_w4a16_gemm_variant(P(d.x), c.K, None, P(d.blob), P(d.g), 0, P(sentinel), c.N, c.M, 0, c.K,
                                          None, 0, v, st) == 0
    gc = synth.grouped_case(T=4, E=3, topk=1, N=32, K=64, seed=2)
    gd = GroupedDev(gc)
    gs = torch.full((gc.R, gc.N), 7.0, dtype=torch.bfloat16, device=DEV)
    off0 = torch.zeros(gc.E + 1, dtype=torch.int32, device=DEV)
    assert L.nvfp4_w4a16_grouped_gemm(P(gd.x), gc.K, P(off0), None, P(gd.blob), P(gd.g), 0, P(gs), gc.N, 0, gc.E,
                                      gc.N, gc.K, None, 0, st) == 0
    assert L.nvfp4_w4a16_grouped_gemm(P(gd.x), gc.K, P(gd.off), None, P(gd.blob), P(gd.g), 0, P(gs), gc.N, gc.R,
                                      gc.E, 0, gc.K, None, 0, st) == 0
    torch.cuda.synchronize()
    assert torch.all(sentinel == 7.0) and torch.all(gs == 7.0)
    # the binding: an empty result of the right shape
    assert tuple(nv.gemm(d.x, d.blob, 0, c.K, d.g).shape) == (c.M, 0)
    assert tuple(nv.gemm(d.x[:0], d.blob, c.N, c.K, d.g).shape) == (0, c.N)


def test_one_workspace_serves_calls_of_any_shape():
    """One workspace, zero-filled once, shared by split-K calls of different shapes in a row (the later calls with
    more split tiles, whose counters would sit where earlier calls left partial sums if the counters did not have
    their own fixed prefix): every result is bitwise that of the call with a fresh workspace."""
    say("workspace reuse across shapes")
    shapes = [(16, 4096, 14336, nv.VARIANT_AUTO), (16, 16384, 8192, nv.VARIANT_AUTO), (1, 2048, 4096, nv.VARIANT_AUTO),
              (24, 2000, 4096, nv.VARIANT_LARGE_M), (16, 4096, 14336, nv.VARIANT_LARGE_M), (8, 2064, 8192, nv.VARIANT_AUTO)]
    ws = nv.workspace(max(nv.gemm_workspace_bytes(M, N, K) for M, N, K, _ in shapes), DEV)
    for rnd in range(2):
        for i, (M, N, K, v) in enumerate(shapes):
            d = DenseDev(synth.dense_case(M, N, K, seed=4000 + i))
            fresh = d.run(v)
            shared = nv.gemm_variant(d.x, d.blob, N, K, d.g, False, None, workspace_buf=ws, variant=v)
            assert torch.equal(shared, fresh), (rnd, M, N, K, v)


@pytest.mark.parametrize("M,N,K", [(5, 14336, 4096), (8, 14336, 4096), (16, 14336, 4096), (16, 4096, 14336),
                                   (12, 2000, 3968)])
def test_automatic_choice_runs_the_resident_kernel_for_5_to_16_rows(M, N, K):
    """The automatic choice for 5..16 rows is the activation-resident kernel where it takes the shape: the plan
    says so and the automatic result is bitwise that of the forced resident variant (which is itself
    reproducible run to run)."""
    c = synth.dense_case(M, N, K, seed=M + K)
    say(f"auto = resident M={M} N={N} K={K}")
    assert nv.gemm_plan(M, N, K) == nv.VARIANT_RESIDENT
    d = DenseDev(c)
    r = d.run(nv.VARIANT_RESIDENT)
    assert torch.equal(d.run(nv.VARIANT_AUTO), r)
    assert torch.equal(d.run(nv.VARIANT_RESIDENT), r)


@pytest.mark.parametrize("pre", [False, True])
def test_mfma_kernel_shares_compute_units_safely(pre):
    """The MFMA-bound kernel with 64-row workgroups (LDS for several per compute unit; 1152 workgroups here, so
    several share each compute unit at once and more start where others ended) gives bitwise the outputs of
    its whole- and half-tile forms (one workgroup per compute unit; the same sums in the same order per output).
    With a pre-quant scale the outputs are also bitwise those of the pre-scaled activation without one."""
    c = synth.dense_case(2304, 8192, 1040, seed=1010, prescale=pre, g_stored=2688.0, g_is_divisor=True)
    say(f"MFMA co-resident workgroups pre={pre} M={c.M} N={c.N} K={c.K}")
    d = DenseDev(c)
    whole = d.run(nv.VARIANT_MFMA)
    quarter = d.run(nv.VARIANT_MFMA_QUARTER)
    assert torch.equal(quarter, whole)
    assert torch.equal(d.run(nv.VARIANT_MFMA_QUARTER), quarter)
    if pre:
        xs = synth.bf16_bits_from_f32(oracle.activation(c.x, c.pre).astype(np.float32))
        assert torch.equal(d.run(nv.VARIANT_MFMA, x=bf16_dev(xs), pre=None), whole)
    rows, cols = stratified_samples(c.M, c.N, 124)
    ref = oracle.gemm_sampled(c.x, c.w, c.s, c.g_stored, c.g_is_divisor, c.pre, rows, cols)
    accept_or_fail(to_f64(whole)[rows, cols], ref, ("mfma co-resident", pre))


@pytest.mark.parametrize("variant", [nv.VARIANT_SMALL_M, nv.VARIANT_LARGE_M, nv.VARIANT_MFMA,
                                     nv.VARIANT_RESIDENT])
def test_strided_io_and_untouched_padding(variant):
    c = synth.dense_case(5, 40, 96, seed=13)
    say(f"strided io variant {variant}")
    d = DenseDev(c)
    xbig = torch.zeros((c.M, 200), dtype=torch.bfloat16, device=DEV)
    xbig[:, 96:] = float("nan")            # beyond K: must never be read
    xbig[:, :96] = d.x
    ybig = torch.full((c.M, 48), 5.0, dtype=torch.bfloat16, device=DEV)
    nv.gemm_variant(xbig[:, :96], d.blob, c.N, c.K, d.g, False, None, out=ybig[:, :40], variant=variant)
    ref = oracle.gemm(c.x, c.w, c.s, c.g_stored, False, None)
    accept_or_fail(to_f64(ybig[:, :40]), ref, "strided", slack=oracle.accumulation_slack(c.x, c.w, c.s, c.g_stored))
    assert torch.all(ybig[:, 40:] == 5.0)


@pytest.mark.parametrize("act", ["bf16", "f16"])
@pytest.mark.parametrize("M", [10, 20, 70, 200])
def test_tile_outputs_any_alignment(M, act):
    """The tile kernel stages its outputs through LDS and writes 16-byte row pieces when the output is 16-byte
    aligned with a row stride and a width that are multiples of 8, and one value at a time otherwise.  Each row
    count takes another tile shape.  An output with an odd row stride gives the same bits as a contiguous one and
    leaves its padding alone; a width that is not a multiple of 8 (N = 1004) matches the oracle."""
    dt = torch.bfloat16 if act == "bf16" else torch.float16
    c = synth.dense_case(M, 1000, 384, seed=31 + M, act=act)
    say(f"tile outputs any alignment M={M} act={act}")
    d = DenseDev(c)
    y = d.run(nv.VARIANT_LARGE_M)
    ybig = torch.full((M, 1003), 7.0, dtype=dt, device=DEV)
    d.run(nv.VARIANT_LARGE_M, out=ybig[:, :1000])
    c2 = synth.dense_case(M, 1004, 384, seed=37 + M, act=act)
    y2 = DenseDev(c2).run(nv.VARIANT_LARGE_M)
    torch.cuda.synchronize()
    assert torch.equal(ybig[:, :1000], y)
    assert torch.all(ybig[:, 1000:] == 7.0)
    ref = (oracle.gemm if act == "bf16" else oracle.gemm_f16)(c2.x, c2.w, c2.s, c2.g_stored, False, None)
    ok, info = oracle.accept(to_f64(y2), ref, out=act)
    assert ok, info


def test_nan_scale_codes_propagate():
    """E4M3 NaN scale bytes (0x7F, 0xFF) decode to NaN (read literally): the decoded tile holds NaN exactly on
    their blocks, every output column whose weights hold one is NaN in every variant, and the other columns are
    unaffected."""
    c = synth.dense_case(16, 64, 256, seed=77)
    s = c.s.copy()
    bad = [(3, 0, 0x7F), (17, 5, 0xFF), (40, 15, 0x7F)]       # (row n, block, byte)
    for n, b, v in bad:
        s[n, b] = v
    c.s = s
    say("nan scale codes")
    d = DenseDev(c)
    tile = bf16_bits(nv.dequant(d.blob, 1, c.N, c.K))[0].astype(np.uint32)
    is_nan = ((tile & 0x7F80) == 0x7F80) & ((tile & 0x7F) != 0)
    exp = np.zeros((c.N, c.K), dtype=bool)
    for n, b, _ in bad:
        exp[n, 16 * b:16 * b + 16] = True
    assert np.array_equal(is_nan, exp)
    ref = oracle.gemm(c.x, c.w, c.s, c.g_stored, False, None)
    nan_cols = sorted({n for n, _, _ in bad})
    assert np.all(np.isnan(ref[:, nan_cols]))
    keep = [n for n in range(c.N) if n not in nan_cols]
    for v in dense_variants(c.M, c.K, c.N):
        y = to_f64(d.run(v))
        assert np.all(np.isnan(y[:, nan_cols])), v
        accept_or_fail(y[:, keep], ref[:, keep], ("nan scales", v))


def test_largest_activation_stride():
    """ld_x at its limit (2^23 elements): the kernels address a tile's rows with 32-bit offsets from the tile's
    first row, which must not wrap at this stride (up to 255 rows x 2^24 bytes)."""
    c = synth.dense_case(300, 272, 256, seed=78)
    say("ld_x = 2^23")
    d = DenseDev(c)
    big = torch.empty((c.M, 1 << 23), dtype=torch.bfloat16, device=DEV)
    big[:, :c.K] = d.x
    ref = oracle.gemm(c.x, c.w, c.s, c.g_stored, False, None)
    for v in (nv.VARIANT_AUTO, nv.VARIANT_LARGE_M, nv.VARIANT_MFMA):
        y = to_f64(d.run(v, x=big[:, :c.K]))
        accept_or_fail(y, ref, ("ld_x max", v))
    del big
    torch.cuda.empty_cache()


@pytest.mark.parametrize("variant", [nv.VARIANT_SMALL_M, nv.VARIANT_RESIDENT])
def test_largest_activation_stride_small_rows(variant):
    """ld_x at its limit (2^23 elements) for the kernels of up to 16 rows."""
    c = synth.dense_case(16, 272, 256, seed=79)
    say(f"ld_x = 2^23 small rows variant {variant}")
    d = DenseDev(c)
    big = torch.empty((c.M, 1 << 23), dtype=torch.bfloat16, device=DEV)
    big[:, :c.K] = d.x
    accept_or_fail(to_f64(d.run(variant, x=big[:, :c.K])), oracle.gemm(c.x, c.w, c.s, c.g_stored, False, None),
                   ("ld_x max", variant))
    del big
    torch.cuda.empty_cache()


def test_smallest_shapes():
    for M, N, K in [(1, 1, 16), (1, 17, 16), (17, 1, 32), (16, 16, 16)]:
        say(f"shape {M}x{N}x{K}")
        c = synth.dense_case(M, N, K, seed=M * 100 + N)
        d = DenseDev(c)
        ref = oracle.gemm(c.x, c.w, c.s, c.g_stored, False, None)
        slack = oracle.accumulation_slack(c.x, c.w, c.s, c.g_stored)
        for v in dense_variants(M, K, N):
            accept_or_fail(to_f64(d.run(v)), ref, (M, N, K, v), slack=slack)


def test_run_to_run_bitwise_determinism():
    for make in (lambda: synth.decode_case(16, N=2048, K=4096, seed=3), lambda: synth.dense_case(200, 512, 1024, 4),
                 lambda: synth.dense_case(16, 2048, 4096, 5, act="f16")):
        c = make()
        say(f"determinism M={c.M}")
        d = DenseDev(c)
        assert torch.equal(d.run(), d.run())
        # the MFMA kernel splits this shape's tiles over K: the order of the split sums is fixed
        assert torch.equal(d.run(nv.VARIANT_MFMA), d.run(nv.VARIANT_MFMA))


# ------------------------------------------------------------ graph replay --

def test_graph_replays_match_eager():
    """Calls captured in a HIP graph give the eager results on every replay, with eager work on the outputs
    between replays.  The split-K counters live in workspaces zeroed once before capture: the kernels themselves
    must leave them zero after every call, since nothing clears them between replays."""
    say("graph replays")
    cases = [(synth.decode_case(16, N=4096, K=14336, seed=3), nv.VARIANT_AUTO),    # activation-resident, K split 4 ways
             (synth.decode_case(16, N=4096, K=14336, seed=3), nv.VARIANT_LARGE_M),  # tile, K split 2 ways
             (synth.decode_case(1, N=2048, K=4096, seed=4), nv.VARIANT_AUTO),      # small-M, K split
             (synth.dense_case(300, 700, 2048, 5, prescale=True), nv.VARIANT_MFMA),  # two MFMA launches + pre-scale
             (synth.dense_case(24, 2000, 4096, 1005), nv.VARIANT_LARGE_M),          # tile, split with N tail
             (synth.decode_case(8, N=2064, K=3968, seed=6), nv.VARIANT_AUTO),       # activation-resident, ragged
             (synth.dense_case(12, 1000, 2048, 8, act="f16", prescale=True), nv.VARIANT_AUTO)]   # fp16 + pre-scale
    devs = [DenseDev(c) for c, _ in cases]
    wss = [nv.workspace(nv.gemm_workspace_bytes(c.M, c.N, c.K), DEV) for c, _ in cases]
    ys = [torch.empty((c.M, c.N), dtype=d.x.dtype, device=DEV) for (c, _), d in zip(cases, devs)]
    gc = synth.grouped_case(T=16, E=8, topk=2, N=96, K=256, seed=6)
    gd = GroupedDev(gc)
    gws = nv.workspace(nv.lib().nvfp4_w4a16_grouped_gemm_workspace_bytes(gc.R, gc.E, gc.N, gc.K), DEV)
    gy = torch.zeros((gc.R, gc.N), dtype=torch.bfloat16, device=DEV)

    def run_all():
        for (c, v), d, ws, y in zip(cases, devs, wss, ys):
            nv.gemm_variant(d.x, d.blob, c.N, c.K, d.g, c.g_is_divisor, d.pre, out=y, workspace_buf=ws, variant=v)
        nv.grouped_gemm(gd.x, gd.off, gd.blob, gc.E, gc.N, gc.K, gd.g, False, gd.pre, out=gy, workspace_buf=gws)

    run_all()
    torch.cuda.synchronize()
    ref = [y.clone() for y in ys] + [gy.clone()]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        run_all()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        run_all()
    for rep in range(3):
        for y in ys + [gy]:
            y.fill_(float("nan"))
        graph.replay()
        torch.cuda.synchronize()
        for i, (y, r) in enumerate(zip(ys + [gy], ref)):
            assert torch.equal(y, r), (rep, i)
        run_all()      # eager calls between replays share the workspaces
        torch.cuda.synchronize()


# ---------------------------------------------------- activation-resident --

XRES_SHAPES = [
    (16, 14336, 4096),   # two chunks per wave, four units per workgroup (the decode workload's launch)
    (9, 2064, 2048),     # one chunk per wave, N one unit past a multiple of 256 units
    (16, 1000, 4000),    # K ragged in its last chunk, N ragged in its last unit
    (5, 48, 272),        # most waves own no chunk (K = 2 chunks + 16)
    (16, 32752, 1024),   # the widest N it takes (eight units per workgroup), last unit ragged
    (16, 4096, 14336),   # K split 4 ways across workgroups (the last split a half), published partials
    (7, 1000, 8320),     # K split 3 ways, ragged K and N
]


@pytest.mark.parametrize("M,N,K", XRES_SHAPES, ids=[f"{m}x{n}x{k}" for m, n, k in XRES_SHAPES])
def test_resident_variant_parity(M, N, K):
    """The activation-resident kernel against the oracle over its launch shapes: chunks per wave (1, 2),
    units per workgroup (1..8), waves without chunks, K split across workgroups, ragged K and N; with a
    pre-quant scale and a divisor-stored global scale on the odd shapes."""
    ragged = K % 128 != 0
    c = synth.dense_case(M, N, K, seed=M + N + K, prescale=ragged, g_stored=2688.0 if ragged else 1 / 2688,
                         g_is_divisor=ragged)
    say(f"resident M={M} N={N} K={K}")
    d = DenseDev(c)
    y = to_f64(d.run(nv.VARIANT_RESIDENT))
    accept_or_fail(y, oracle.gemm(c.x, c.w, c.s, c.g_stored, c.g_is_divisor, c.pre), ("resident", M, N, K))
    assert torch.equal(d.run(nv.VARIANT_RESIDENT), d.run(nv.VARIANT_RESIDENT))   # split order fixed
