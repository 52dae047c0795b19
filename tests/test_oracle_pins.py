"""Pins of the CPU oracle to facts outside itself (runs on CPU, no GPU).

Each test ties the oracle to something it cannot have copied from itself: the
format tables (OCP MX / OFP8), a library decoder (torch's float8_e4m3fn),
closed-form hand cases, exact rational arithmetic on tiny inputs, an
independent numpy twin, and invariants of the definition.  The negative
controls plant a mistake in a copy of the numpy twin and check that the
acceptance check catches it.
"""
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _read_table(name):
    rows = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                rows.append(line.split())
    return rows


def _same(a, b):
    """Equal as numbers, NaN == NaN, and the sign of zero must agree."""
    if math.isnan(a) or math.isnan(b):
        return math.isnan(a) and math.isnan(b)
    return a == b and math.copysign(1.0, a) == math.copysign(1.0, b)


# ------------------------------------------------------------ formats ------

def test_e2m1_all_codes_match_format_table():
    table = {int(c): float(v) for c, v in _read_table("e2m1_codes.txt")}
    assert sorted(table) == list(range(16))
    for c in range(16):
        assert _same(oracle.e2m1(c), table[c]), c
        assert _same(float(oracle.e2m1_np(np.array([c]))[0]), table[c]), c


def test_e4m3_named_codes_match_format_table():
    for b, v in _read_table("e4m3_special.txt"):
        assert _same(oracle.e4m3(int(b, 16)), float(v)), b


def test_e4m3_all_256_codes_match_torch_float8_e4m3fn():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    lib = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    mine = np.array([oracle.e4m3(b) for b in range(256)])
    twin = oracle.e4m3_np(np.arange(256))
    for b in range(256):
        assert _same(mine[b], float(lib[b])), hex(b)
        assert _same(twin[b], float(lib[b])), hex(b)
    finite = np.isfinite(mine)
    assert finite.sum() == 254 and np.nanmax(mine) == 448.0 and np.min(np.abs(mine[finite & (mine != 0)])) == 2.0 ** -9


def test_all_code_scale_products_are_exact_in_bf16():
    """Every e2m1 x finite-e4m3 product is a bf16 value: the decoded tile can be bit-exact."""
    vals = np.array([oracle.e2m1(c) * oracle.e4m3(b) for c in range(16) for b in range(256)
                     if math.isfinite(oracle.e4m3(b))])
    assert vals.size == 16 * 254
    t = torch.from_numpy(vals)
    assert torch.equal(t.to(torch.bfloat16).to(torch.float64), t)


# ------------------------------------------------------------ hand cases ---

def _hand_inputs(case):
    N, K = 16, 16
    codes = np.zeros((N, K), dtype=np.uint8)
    x = np.full((1, K), 1.0, dtype=np.float32)
    s = np.full((N, 1), 0x38, dtype=np.uint8)
    g, div, pre = 1.0, False, None
    if case == "H1":
        codes[:] = np.arange(N, dtype=np.uint8)[:, None]
    elif case == "H2":
        x[:] = 0.0
        x[0, 1] = 1.0
        codes[:] = (np.arange(N)[:, None] + np.arange(K)[None, :]) % 16
    elif case == "H3":
        codes[:] = 2
        s[:, 0] = np.arange(1, N + 1)
        g = 2.0 ** -4
    elif case == "H4":
        codes[:] = 2
        x[:] = 1.0234375
        pre = synth.bf16_bits_from_f32(np.full(K, 1.5, dtype=np.float32))
        g, div = 0.25, True
    return synth.bf16_bits_from_f32(x), synth.pack_codes(codes), s, g, div, pre


@pytest.mark.parametrize("case", ["H1", "H2", "H3", "H4"])
def test_hand_cases_closed_form(case):
    expected = {r[0]: [float(v) for v in r[1:]] for r in _read_table("hand_cases.txt")}[case]
    x, w, s, g, div, pre = _hand_inputs(case)
    y = oracle.gemm(x, w, s, g, div, pre)
    yn = oracle.gemm_np(x, w, s, g, div, pre)
    for n in range(16):
        assert y[0, n] == expected[n], (case, n, y[0, n], expected[n])
        assert yn[0, n] == expected[n], (case, n)


def test_hand_case_h2_detects_swapped_nibbles():
    x, w, s, g, div, pre = _hand_inputs("H2")
    swapped = ((w & 15) << 4) | (w >> 4)
    y = oracle.gemm(x, swapped, s, g, div, pre)
    expected = [float(v) for v in _read_table("hand_cases.txt")[1][1:]]
    assert any(y[0, n] != expected[n] for n in range(16))


# ------------------------------------------------------ exact arithmetic ---

def _exact_gemm(x_bits, w, s, g_stored, div, pre_bits):
    """Exact rational evaluation of the definition, pure Python loops (tiny inputs only)."""
    def bfv(b):
        return Fraction(float(oracle.bf16_np(np.array([b]))[0]))

    def e2m1(c):
        mag = [Fraction(0), Fraction(1, 2), Fraction(1), Fraction(3, 2), Fraction(2), Fraction(3), Fraction(4),
               Fraction(6)][c & 7]
        return -mag if c & 8 else mag

    def e4m3(b):
        e, m = (b >> 3) & 15, b & 7
        mag = Fraction(m, 512) if e == 0 else Fraction(8 + m, 8) * Fraction(2) ** (e - 7)
        return -mag if b & 128 else mag

    M, K = x_bits.shape
    N = w.shape[0]
    gv = Fraction(float(np.float32(1.0) / np.float32(g_stored))) if div else Fraction(float(np.float32(g_stored)))
    out = [[None] * N for _ in range(M)]
    for m in range(M):
        xs = []
        for k in range(K):
            v = bfv(x_bits[m, k])
            if pre_bits is not None:
                v = Fraction(float(torch.tensor(float(v * bfv(pre_bits[k])), dtype=torch.float64)
                                   .to(torch.bfloat16).to(torch.float64)))
            xs.append(v)
        for n in range(N):
            acc = Fraction(0)
            for k in range(K):
                code = (int(w[n, k >> 1]) >> (4 * (k & 1))) & 15
                acc += xs[k] * e2m1(code) * e4m3(int(s[n, k >> 4]))
            out[m][n] = gv * acc
    return out


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_oracle_matches_exact_rational_arithmetic(seed):
    g = synth.rng(seed)
    M, N, K = 2, 3, 48
    x = synth.normal_bf16(g, (M, K))
    w = synth.random_codes(g, (N, K))
    s = synth.scales_pow2_mant(g, (N, K // 16), umin=-9, umax=8)
    pre = synth.awq_prescale(g, K)
    for div, gst in ((False, 1.0 / 448.0), (True, 2688.0)):
        for p in (None, pre):
            y = oracle.gemm(x, w, s, gst, div, p)
            ex = _exact_gemm(x, w, s, gst, div, p)
            for m in range(M):
                for n in range(N):
                    # fp64 summation of K exact products: error <= K * 2^-52 * sum|terms|
                    bound = 1e-13 * max(1.0, float(abs(ex[m][n])) * 10)
                    assert abs(y[m, n] - float(ex[m][n])) <= bound, (m, n, y[m, n], float(ex[m][n]))


# ------------------------------------------------------------- rounding ----

def test_round_bf16_matches_torch_on_bf16_products():
    """X' = RNE_bf16(x*s): for bf16 x bf16 products (exact in fp32) torch's fp32->bf16 cast is RNE."""
    g = synth.rng(7)
    a = synth.normal_bf16(g, 4096)
    b = synth.awq_prescale(g, 4096)
    prod = oracle.bf16_np(a) * oracle.bf16_np(b)
    lib = torch.from_numpy(prod.astype(np.float32)).to(torch.bfloat16).to(torch.float64).numpy()
    mine = np.array([oracle.round_bf16(v) for v in prod])
    assert np.array_equal(mine, lib)
    assert np.array_equal(oracle.rne_bf16_np(prod), lib)


def test_round_bf16_ties_and_limits():
    # 1 + 2^-8 is a tie between 1 and 1 + 2^-7: to even -> 1.0; 1 + 3*2^-8 -> 1 + 2^-6
    assert oracle.round_bf16(1.0 + 2.0 ** -8) == 1.0
    assert oracle.round_bf16(1.0 + 3 * 2.0 ** -8) == 1.0 + 2.0 ** -6
    assert oracle.round_bf16(-(1.0 + 2.0 ** -8)) == -1.0
    assert oracle.round_bf16(1.0 + 2.0 ** -8 + 2.0 ** -40) == 1.0 + 2.0 ** -7
    maxbf = (2 - 2.0 ** -7) * 2.0 ** 127
    assert oracle.round_bf16(maxbf) == maxbf
    assert oracle.round_bf16(2.0 ** 128 * (1 - 2.0 ** -9)) == math.inf   # halfway above max: to even = 2^128
    assert oracle.round_bf16(2.0 ** -133) == 2.0 ** -133                  # min subnormal
    assert oracle.round_bf16(2.0 ** -135) == 0.0


def test_global_scale_inversion_is_fp32_reciprocal():
    for v in [2688.0, 448.0 * 6, 3.0, 0.1, 7.0, 2.0 ** 120]:
        st = np.float32(v)
        assert oracle.global_scale(st, True) == float(np.float32(1.0) / st)
        assert oracle.global_scale(st, False) == float(st)


# ---------------------------------------------------------------- twin ----

@pytest.mark.parametrize("case", ["tiny", "ragged"])
def test_c_oracle_matches_numpy_twin(case):
    c = synth.tiny_case() if case == "tiny" else synth.ragged_case()
    y = oracle.gemm(c.x, c.w, c.s, c.g_stored, c.g_is_divisor, c.pre)
    yn = oracle.gemm_np(c.x, c.w, c.s, c.g_stored, c.g_is_divisor, c.pre)
    rel = np.linalg.norm(y - yn) / np.linalg.norm(yn)
    assert rel <= 1e-12
    assert np.array_equal(oracle.dequant(c.w, c.s), oracle.dequant_np(c.w, c.s))


def test_sampled_and_grouped_agree_with_dense():
    c = synth.ragged_case()
    y = oracle.gemm(c.x, c.w, c.s, c.g_stored, c.g_is_divisor, c.pre)
    g = synth.rng(3)
    rows, cols = g.integers(0, c.M, 200), g.integers(0, c.N, 200)
    ys = oracle.gemm_sampled(c.x, c.w, c.s, c.g_stored, c.g_is_divisor, c.pre, rows, cols)
    assert np.allclose(ys, y[rows, cols], rtol=1e-13, atol=1e-13)
    # grouped with one expert owning every row == dense
    off = np.array([0, c.M], dtype=np.int32)
    yg = oracle.grouped_gemm(c.x, off, c.w[None], c.s[None], np.array([c.g_stored], np.float32), c.g_is_divisor,
                             c.pre)
    assert np.allclose(yg, y, rtol=1e-13, atol=1e-13)


def test_grouped_oracle_matches_twin_and_skips_empty_experts():
    gc = synth.grouped_case(T=6, E=8, topk=2, N=48, K=64, seed=11)
    assert len(gc.active) < gc.E or True
    y = oracle.grouped_gemm(gc.x, gc.offsets, gc.w, gc.s, gc.g_stored, False, None)
    yn = oracle.grouped_gemm_np(gc.x, gc.offsets, gc.w, gc.s, gc.g_stored, False, None)
    assert np.allclose(y, yn, rtol=1e-12, atol=1e-12)
    rows = np.arange(gc.R)
    cols = np.arange(gc.R) % gc.N
    ys = oracle.grouped_gemm_sampled(gc.x, gc.offsets, gc.w, gc.s, gc.g_stored, False, None, rows, cols)
    assert np.allclose(ys, y[rows, cols], rtol=1e-13, atol=1e-13)


# ----------------------------------------------------------- invariants ---

def test_identity_activation_gives_transposed_tile():
    c = synth.dense_case(1, 40, 64, seed=5)
    eye = synth.bf16_bits_from_f32(np.eye(64, dtype=np.float32))
    y = oracle.gemm(eye, c.w, c.s, 1.0, False, None)
    assert np.array_equal(y, oracle.dequant(c.w, c.s).T)


def test_power_of_two_scaling_and_prescale_equivalence():
    c = synth.ragged_case()
    y = oracle.gemm(c.x, c.w, c.s, c.g_stored, c.g_is_divisor, c.pre)
    x2 = synth.bf16_bits_from_f32(oracle.bf16_np(c.x).astype(np.float32) * 4)
    assert np.array_equal(oracle.gemm(x2, c.w, c.s, c.g_stored, c.g_is_divisor, c.pre), 4 * y)
    xs = synth.bf16_bits_from_f32(oracle.activation(c.x, c.pre).astype(np.float32))
    assert np.array_equal(oracle.gemm(xs, c.w, c.s, c.g_stored, c.g_is_divisor, None), y)
    ginv = float(np.float32(1.0) / np.float32(c.g_stored))
    assert np.array_equal(oracle.gemm(c.x, c.w, c.s, ginv, False, c.pre), y)


def test_divisor_inversion_restores_finite_outputs():
    """A huge divisor-stored scale is harmless once inverted and overflows bf16 if used as a multiplier."""
    c = synth.tiny_case()
    big = 2.0 ** 120
    y = oracle.gemm(c.x, c.w, c.s, big, True, None)
    assert np.all(np.isfinite(y))
    assert np.all(np.isfinite([oracle.round_bf16(v) for v in y.ravel()[:512]]))
    y_bad = oracle.gemm(c.x, c.w, c.s, big, False, None)
    assert np.any(~np.isfinite([oracle.round_bf16(v) for v in y_bad.ravel()]))


# ----------------------------------------------------- negative controls ---

def _planted(kind, c):
    x = oracle.activation_np(c.x, c.pre)
    T = oracle.dequant_np(c.w, c.s)
    g = oracle.global_scale_np(c.g_stored, c.g_is_divisor)
    if kind == "drop_prescale":
        x = oracle.activation_np(c.x, None)
    elif kind == "drop_inversion":
        g = float(np.float32(c.g_stored))
    elif kind == "swap_nibbles":
        T = oracle.dequant_np(((c.w & 15) << 4) | (c.w >> 4), c.s)
    elif kind == "block_k_over_8":
        codes = np.stack([c.w & 15, c.w >> 4], axis=-1).reshape(c.w.shape[0], -1)
        idx = np.minimum(np.arange(c.K) >> 3, c.s.shape[1] - 1)
        T = oracle.e2m1_np(codes) * oracle.e4m3_np(c.s[:, idx])
    elif kind == "no_prescale_rounding":
        x = oracle.bf16_np(c.x) * oracle.bf16_np(c.pre)[None, :]
    elif kind == "truncate_output":
        y = (g * (x @ T.T)).astype(np.float32)
        return (y.view(np.uint32) & 0xFFFF0000).view(np.float32).astype(np.float64)
    elif kind == "fold_g_into_bf16_tile":
        T = torch.from_numpy(T * g).to(torch.bfloat16).to(torch.float64).numpy()
        g = 1.0
    y = (g * (x @ T.T)).astype(np.float32)
    return torch.from_numpy(y).to(torch.bfloat16).to(torch.float64).numpy()


def test_bf16_rounded_result_passes_acceptance():
    """The correct result rounded once to bf16 (what the kernels store) is inside the bound."""
    for c in (synth.tiny_case(), synth.ragged_case()):
        ref = oracle.gemm(c.x, c.w, c.s, c.g_stored, c.g_is_divisor, c.pre)
        ok, info = oracle.accept(_planted("none", c), ref)
        assert ok, info


@pytest.mark.parametrize("kind", ["drop_prescale", "drop_inversion", "swap_nibbles", "block_k_over_8",
                                  "no_prescale_rounding", "truncate_output", "fold_g_into_bf16_tile"])
def test_planted_mistakes_fail_acceptance(kind):
    c = synth.dense_case(64, 512, 1024, seed=21, g_stored=2688.0, g_is_divisor=True, prescale=True)
    ref = oracle.gemm(c.x, c.w, c.s, c.g_stored, c.g_is_divisor, c.pre)
    ok, info = oracle.accept(_planted(kind, c), ref)
    assert not ok, (kind, info)


def test_round_bf16_np_matches_c_oracle():
    g = synth.rng(17)
    v = np.concatenate([g.standard_normal(2000) * 10.0 ** g.integers(-30, 30, 2000),
                        [1 + 2.0 ** -8, 1 + 3 * 2.0 ** -8, 2.0 ** -133, 2.0 ** -135, 0.0, -0.0]])
    assert np.array_equal(oracle.round_bf16_np(v), np.array([oracle.round_bf16(a) for a in v]))


def test_acceptance_rounding_interval_only_for_tiny_outputs():
    """From 1024 outputs up only the 2e-3 Frobenius bound applies; the correctly rounded result meets it there."""
    c = synth.tiny_case()                       # 4 x 256 = 1024 outputs
    ref = oracle.gemm(c.x, c.w, c.s, c.g_stored, False, None)
    ok, info = oracle.accept(oracle.round_bf16_np(ref), ref, slack=np.zeros_like(ref))
    assert ok and "rounding_interval_misses" not in info


# a 17-output column dominated by one element: rounding alone exceeds 2e-3
_R17 = np.array([0.0272096, 0.0712413, 0.0512778, 0.0185412, 0.0525297, -0.0131747, -0.0721159, 0.0510564,
                 -0.12936933, -0.0099833, 0.01, 0.02, -0.03, 0.004, 0.005, -0.006, 0.007])


def test_acceptance_rounding_interval_accepts_the_correct_rounding_only():
    """Tiny outputs: the correctly rounded result passes through the rounding interval although its relative
    Frobenius error is above 2e-3; the same result with the dominant element one bf16 ulp off fails, and so does
    the correct rounding when no slack is given (the interval is the only route past the Frobenius bound)."""
    r = _R17
    y = oracle.round_bf16_np(r)
    assert oracle.accept(y, r)[1]["rel_fro"] > 2e-3
    assert not oracle.accept(y, r)[0]
    ok, info = oracle.accept(y, r, slack=np.zeros_like(r))
    assert ok and info["rounding_interval_misses"] == 0, info
    bump = y.copy()
    i = int(np.argmax(np.abs(r)))
    bump[i] += np.sign(y[i]) * 2.0 ** (np.frexp(abs(y[i]))[1] - 8)      # one bf16 ulp away from zero
    assert oracle.round_bf16_np(bump)[i] == bump[i] != y[i]
    ok, info = oracle.accept(bump, r, slack=np.zeros_like(r))
    assert not ok and info["rounding_interval_misses"] == 1, info


def test_accumulation_slack_bounds_fp32_summation_error():
    """The slack covers fp32 sums in any order: ascending, descending, sorted and pairwise fp32 sums of the exact
    products, times g, stay within d of the fp64 oracle."""
    c = synth.dense_case(3, 5, 2048, seed=61)
    ref = oracle.gemm(c.x, c.w, c.s, c.g_stored, False, None)
    d = oracle.accumulation_slack(c.x, c.w, c.s, c.g_stored)
    xa, t = oracle.activation_np(c.x), oracle.dequant_np(c.w, c.s)
    g = np.float32(c.g_stored)
    for m in range(c.M):
        for n in range(c.N):
            p = (xa[m] * t[n]).astype(np.float32)                 # exact products
            assert np.array_equal(p.astype(np.float64), xa[m] * t[n])
            for order in (p, p[::-1], np.sort(p), np.sort(p)[::-1]):
                acc = np.float32(0)
                for v in order:
                    acc = np.float32(acc + v)
                assert abs(float(np.float32(g * acc)) - ref[m, n]) <= d[m, n]
            while p.size > 1:                                      # pairwise
                p = (p[0::2] + p[1::2]).astype(np.float32) if p.size % 2 == 0 else np.append(p[:-1], np.float32(0))
            assert abs(float(np.float32(g * p[0])) - ref[m, n]) <= d[m, n]
    # the bound is worst-case (linear in K); at the sizes it serves, tiny outputs with short K, it is far below
    # half a bf16 ulp (2^-9 relative)
    c = synth.dense_case(17, 1, 32, seed=62)
    d = oracle.accumulation_slack(c.x, c.w, c.s, c.g_stored)
    ref = oracle.gemm(c.x, c.w, c.s, c.g_stored, False, None)
    assert np.median(d / np.abs(ref)) < 2.0 ** -12


# ------------------------------------------------------------ MoE glue -------

def test_moe_route_hand_case():
    """Tokens 0..2 with top-2 experts (2,0), (0,1), (2,3) over E = 4.  Pairs p = 2t + j choose experts
    2,0,0,1,2,3; sorted by expert with ties in pair order the rows hold pairs 1,2 | 3 | 0,4 | 5."""
    off, row_token, token_row = oracle.moe_route(np.array([[2, 0], [0, 1], [2, 3]]), 4)
    assert off.tolist() == [0, 2, 3, 5, 6]
    assert row_token.tolist() == [0, 1, 1, 0, 2, 2]
    assert token_row.tolist() == [3, 0, 1, 2, 4, 5]


@pytest.mark.parametrize("T,k,E", [(16, 8, 128), (200, 3, 7), (5, 1, 1), (9, 4, 4)])
def test_moe_route_matches_brute_force(T, k, E):
    """Every expert's rows hold exactly its pairs in increasing pair order (an O(P E) scan), and token_row is the
    inverse of the row order."""
    g = synth.rng(T * 31 + E)
    ids = np.stack([g.choice(E, size=k, replace=False) for _ in range(T)])
    off, row_token, token_row = oracle.moe_route(ids, E)
    r = 0
    for e in range(E):
        assert off[e] == r
        for p in range(T * k):
            if ids.reshape(-1)[p] == e:
                assert row_token[r] == p // k and token_row[p] == r
                r += 1
    assert off[E] == r == T * k


def test_silu_mul_closed_forms():
    """silu(v) = v * sigmoid(v) at a few points (math.exp), silu(v) - silu(-v) = v, and up scales the result."""
    vals = np.array([0.0, 0.5, -0.5, 1.0, -3.0, 4.0, -8.0, 10.0], dtype=np.float32)
    gate = synth.bf16_bits_from_f32(vals)

    def run(gate_bits, up):
        up_bits = synth.bf16_bits_from_f32(np.full_like(vals, up))
        return oracle.silu_mul(np.concatenate([gate_bits[None], up_bits[None]], axis=1))[0]

    v = oracle.bf16_np(gate)
    s = run(gate, 1.0)
    for a, x in zip(s, v):
        assert a == pytest.approx(x / (1.0 + math.exp(-x)), rel=1e-15, abs=0)
    assert np.allclose(s - run(synth.bf16_bits_from_f32(-vals), 1.0), v, rtol=0, atol=1e-12)
    assert np.array_equal(run(gate, 2.0), 2 * s)


def test_combine_matches_loops_and_one_hot_gather():
    g = synth.rng(5)
    T, k, H, E = 6, 3, 40, 5
    ids = np.stack([g.choice(E, size=k, replace=False) for _ in range(T)])
    _, _, token_row = oracle.moe_route(ids, E)
    y = synth.normal_bf16(g, (T * k, H))
    w = g.random((T, k)).astype(np.float32)
    out = oracle.combine(y, token_row, w)
    yv = oracle.bf16_np(y)
    for t in range(T):
        for c in range(H):
            ref = sum(float(w[t, j]) * float(yv[token_row[t * k + j], c]) for j in range(k))
            assert out[t, c] == pytest.approx(ref, rel=1e-13, abs=1e-300)
    onehot = np.zeros((T, k), dtype=np.float32)
    onehot[:, 1] = 1.0
    assert np.array_equal(oracle.combine(y, token_row, onehot), yv[token_row.reshape(T, k)[:, 1]])


def test_relu2_closed_forms():
    """relu2 is 0 for v <= 0 (signed zero and negatives) and v*v above; a bf16 v has at most 8 significant bits,
    so v*v is exact in fp64."""
    vals = np.array([-2.0, -0.0, 0.0, 0.5, 1.5, 3.0, -1e-3, 255.0], dtype=np.float32)
    bits = synth.bf16_bits_from_f32(vals)[None]
    v = oracle.bf16_np(bits)[0]
    out = oracle.relu2(bits)[0]
    assert np.array_equal(out, np.array([x * x if x > 0 else 0.0 for x in v]))
    assert np.all(out[v <= 0] == 0)


# ------------------------------------------------------------ fp16 oracle ---

def test_f16_decode_matches_struct_for_every_pattern():
    """All 65536 binary16 patterns decode as Python's own IEEE half unpacking (struct 'e') does."""
    import struct
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    got = oracle.f16_np(bits)
    ref = np.array([struct.unpack("<e", int(b).to_bytes(2, "little"))[0] for b in bits], dtype=np.float64)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(ref[~nan]))   # signed zeros


def test_rne_f16_ties_subnormals_and_overflow():
    """Round to nearest even into binary16: exact ties go to the even significand, in the normal and the subnormal
    range; 65504 is the largest finite value and everything from 65520 (the tie with 2^16) up overflows."""
    ulp1 = 2.0 ** -10
    cases = [
        (1.0 + ulp1 / 2, 1.0),                     # tie, even is 1.0
        (1.0 + 3 * ulp1 / 2, 1.0 + 2 * ulp1),      # tie, even is 1 + 2 ulp
        (1.0 + ulp1 / 2 + 2.0 ** -30, 1.0 + ulp1),  # just above the tie
        (2.0 ** -25, 0.0),                          # half the smallest subnormal: tie, even is 0
        (3 * 2.0 ** -25, 2.0 ** -23),               # tie between 1 and 2 subnormal steps: even is 2
        (2.0 ** -24, 2.0 ** -24),                   # smallest subnormal, exact
        (65504.0, 65504.0),
        (65519.99, 65504.0),
        (65520.0, math.inf),
        (-65520.0, -math.inf),
        (1e300, math.inf),
    ]
    v = np.array([a for a, _ in cases])
    assert np.array_equal(oracle.rne_f16_np(v), np.array([b for _, b in cases]))
    # and random finite values agree with Python's half packing (round-half-even)
    import struct
    g = synth.rng(5)
    r = g.standard_normal(2000) * np.exp2(g.integers(-26, 16, 2000))
    r = r[np.abs(r) < 65504.0]   # struct refuses values that overflow (covered by the cases above)
    ref = [struct.unpack("<e", struct.pack("<e", float(a)))[0] for a in r]
    assert np.array_equal(oracle.rne_f16_np(r), np.array(ref))


def test_activation_f16_prescale_rounds_each_exact_product_once():
    import struct
    g = synth.rng(6)
    x = synth.f16_bits_from_f32(g.standard_normal((3, 64)).astype(np.float32) * 8)
    pre = synth.f16_bits_from_f32(g.uniform(1 / math.e, math.e, 64).astype(np.float32))
    got = oracle.activation_f16(x, pre)
    dec = lambda b: struct.unpack("<e", int(b).to_bytes(2, "little"))[0]
    for m in range(3):
        for k in range(64):
            p = dec(x[m, k]) * dec(pre[k])    # exact in binary64
            assert got[m, k] == struct.unpack("<e", struct.pack("<e", p))[0]
    assert np.array_equal(oracle.activation_f16(x, None), oracle.f16_np(x))


def test_gemm_f16_brute_force_loops():
    """A tiny fp16 GEMM against plain loops over exact rationals (codes, scales and halves decoded here)."""
    import struct
    c = synth.dense_case(2, 3, 32, 11, act="f16", prescale=True, g_stored=3.0, g_is_divisor=True)
    dec = lambda b: Fraction(struct.unpack("<e", int(b).to_bytes(2, "little"))[0])
    e2m1 = [Fraction(0), Fraction(1, 2), Fraction(1), Fraction(3, 2), Fraction(2), Fraction(3), Fraction(4),
            Fraction(6)]

    def e4m3(b):
        e, m = (b >> 3) & 15, b & 7
        v = Fraction(m, 8) * Fraction(2) ** -6 if e == 0 else (1 + Fraction(m, 8)) * Fraction(2) ** (e - 7)
        return -v if b & 0x80 else v

    def code(n, k):
        byte = int(c.w[n, k // 2])
        q = byte & 15 if k % 2 == 0 else byte >> 4
        return -e2m1[q & 7] if q & 8 else e2m1[q & 7]

    g = Fraction(float(np.float32(1) / np.float32(3.0)))
    ref = np.zeros((2, 3))
    for m in range(2):
        for n in range(3):
            acc = Fraction(0)
            for k in range(32):
                xs = float(dec(c.x[m, k]) * dec(c.pre[k]))
                xp = Fraction(struct.unpack("<e", struct.pack("<e", xs))[0])
                acc += xp * code(n, k) * e4m3(int(c.s[n, k // 16]))
            ref[m, n] = float(g * acc)
    got = oracle.gemm_f16(c.x, c.w, c.s, c.g_stored, True, c.pre)
    assert np.allclose(got, ref, rtol=1e-13, atol=0)


def test_gemm_f16_equals_bf16_oracle_on_values_both_types_hold():
    """Activations exactly representable in bf16 and in fp16 (at most 8 significant bits, in fp16's normal range):
    the fp16 oracle and the C oracle's bf16 path define the same Y."""
    g = synth.rng(12)
    M, N, K = 3, 20, 96
    mant = g.integers(-255, 256, (M, K)).astype(np.float64)
    vals = mant * np.exp2(g.integers(-12, -2, (M, K)).astype(np.float64))
    x16 = vals.astype(np.float16).view(np.uint16)
    xbf = synth.bf16_bits_from_f32(vals.astype(np.float32))
    assert np.array_equal(oracle.f16_np(x16), oracle.bf16_np(xbf))
    c = synth.dense_case(M, N, K, 13)
    a = oracle.gemm_f16(x16, c.w, c.s, 1 / 2688.0)
    b = oracle.gemm(xbf, c.w, c.s, 1 / 2688.0)
    assert np.allclose(a, b, rtol=1e-12, atol=0)


def test_grouped_gemm_f16_rows_follow_their_expert():
    gc = synth.grouped_case(T=12, E=5, topk=2, N=24, K=64, seed=14, act="f16", prescale=True)
    got = oracle.grouped_gemm_f16(gc.x, gc.offsets, gc.w, gc.s, gc.g_stored, False, gc.pre)
    for e in range(gc.E):
        a, b = gc.offsets[e], gc.offsets[e + 1]
        if b > a:
            ref = oracle.gemm_f16(gc.x[a:b], gc.w[e], gc.s[e], float(gc.g_stored[e]), False, gc.pre)
            assert np.array_equal(got[a:b], ref)


def test_moe_glue_f16_decodes_inputs_as_binary16():
    """The fp16 forms of the MoE elementwise steps: the same definitions on binary16-decoded inputs; closed forms
    (silu(0) = 0, relu2 of a negative = 0, one-hot combine = the row) checked on fp16 bit patterns."""
    import struct
    h = np.array([[0x0000, 0x3C00, 0x4000, 0xBC00]], dtype=np.uint16)   # gate (0, 1) | up (2, -1) in fp16
    a = oracle.silu_mul(h, "f16")
    assert a[0, 0] == 0.0 and np.isclose(a[0, 1], (1 / (1 + math.exp(-1))) * -1.0, rtol=1e-15)
    r = oracle.relu2(np.array([[0xC000, 0x4200]], dtype=np.uint16), "f16")    # -2, 3
    assert r[0, 0] == 0.0 and r[0, 1] == 9.0
    y = synth.f16_bits_from_f32(synth.rng(15).standard_normal((4, 8)).astype(np.float32))
    out = oracle.combine(y, np.array([2, 0], dtype=np.int32), np.array([[1.0, 0.0]], dtype=np.float32), "f16")
    dec = np.array([struct.unpack("<e", int(b).to_bytes(2, "little"))[0] for b in y[2]])
    assert np.array_equal(out[0], dec)



# ------------------------------------------------------- MXFP4 weight-only ---
# E2M1 codes with one E8M0 scale per 32 K and no global scale (SGLang compressed-tensors NVFP4 weight-only page,
# Modifications, the paragraph on MXFP4: group_blocks == 2, E8M0 scales, no global_scale).  E8M0 per the OCP MX
# specification: 2^(e - 127), 0xFF NaN.

def test_e8m0_all_256_codes_match_closed_form_and_torch():
    """Every E8M0 byte: 2^(e - 127) for e < 255 (a closed form) and NaN for 255; and torch's float8_e8m0fnu
    decoder (a library routine) agrees on all 256 codes; the numpy twin too."""
    codes = np.arange(256)
    c = np.array([oracle.e8m0(int(b)) for b in codes])
    closed = np.where(codes == 255, np.nan, np.ldexp(1.0, codes - 127))
    assert np.array_equal(c, closed, equal_nan=True)
    t = torch.arange(256, dtype=torch.uint8).view(torch.float8_e8m0fnu).to(torch.float64).numpy()
    assert np.array_equal(c, t, equal_nan=True)
    assert np.array_equal(oracle.e8m0_np(codes), c, equal_nan=True)
    assert oracle.e8m0(0) == 2.0 ** -127 and oracle.e8m0(254) == 2.0 ** 127 and oracle.e8m0(127) == 1.0


def test_mxfp4_tile_is_code_times_power_of_two_over_groups_of_32():
    """Every code under every E8M0 scale: T = e2m1(code) * 2^(e-127) exactly (fp64); the scale index is k // 32
    (a row whose 32-groups carry different scales: k = 31 and k = 32 take different scales, k = 0 and 31 the
    same), and the numpy twin agrees."""
    K = 256
    N = 256                                   # row n: scale byte n on its first group, n ^ 0x55 on the others
    codes = (np.arange(K)[None, :] + np.arange(N)[:, None]) % 16
    w = synth.pack_codes(codes.astype(np.uint8))
    s = np.empty((N, K // 32), dtype=np.uint8)
    s[:, 0] = np.arange(N)
    s[:, 1:] = (np.arange(N) ^ 0x55)[:, None]
    t = oracle.dequant(w, s, "mxfp4")
    exp = oracle.e2m1_np(codes) * np.repeat(np.where(s == 255, np.nan, np.ldexp(1.0, s.astype(np.int64) - 127)),
                                            32, axis=1)
    assert np.array_equal(t, exp, equal_nan=True)
    assert np.array_equal(oracle.dequant_np(w, s, "mxfp4"), t, equal_nan=True)
    n = 130
    assert t[n, 31] / oracle.e2m1((31 + n) % 16) == 2.0 ** (130 - 127)
    assert t[n, 32] / oracle.e2m1((32 + n) % 16) == 2.0 ** ((130 ^ 0x55) - 127)


def test_mxfp4_hand_case_closed_form():
    """1 x 64 x 4: X = 1 on k = 0..63; row n holds code 2 (1.0) on the first 32-group and code 4 (2.0) on the
    second, scales 2^(n-1) and 2^-n: Y[0, n] = 32 * 2^(n-1) + 32 * 2 * 2^-n, exactly, with no global scale (the
    stored value passed in is ignored)."""
    N, K = 4, 64
    codes = np.zeros((N, K), dtype=np.uint8)
    codes[:, :32], codes[:, 32:] = 2, 4
    w = synth.pack_codes(codes)
    s = np.stack([np.arange(N) - 1 + 127, -np.arange(N) + 127], axis=1).astype(np.uint8)
    x = np.full((1, K), 0x3F80, dtype=np.uint16)
    y = oracle.gemm(x, w, s, 123.0, True, None, fmt="mxfp4")
    exp = [32 * 2.0 ** (n - 1) + 64 * 2.0 ** -n for n in range(N)]
    assert list(y[0]) == exp


def test_mxfp4_gemm_matches_twin_sampled_grouped_and_exact_arithmetic():
    c = synth.dense_case(17, 96, 320, 71, fmt="mxfp4", prescale=True)
    assert c.s.shape == (96, 10) and c.g_stored == 1.0
    ref = oracle.gemm(c.x, c.w, c.s, c.g_stored, False, c.pre, fmt="mxfp4")
    tw = oracle.gemm_np(c.x, c.w, c.s, c.g_stored, False, c.pre, fmt="mxfp4")
    assert np.max(np.abs(ref - tw)) <= 1e-12 * np.max(np.abs(ref))
    rows, cols = np.array([0, 16, 5]), np.array([95, 0, 33])
    assert np.array_equal(oracle.gemm_sampled(c.x, c.w, c.s, 1.0, False, c.pre, rows, cols, fmt="mxfp4"),
                          ref[rows, cols])
    # exact rational arithmetic on one output: every term is a dyadic rational
    xa = oracle.activation_np(c.x, c.pre)
    t = oracle.dequant(c.w, c.s, "mxfp4")
    exact = sum(Fraction(float(a)) * Fraction(float(b)) for a, b in zip(xa[3], t[7]))
    assert abs(Fraction(ref[3, 7]) - exact) <= abs(exact) * Fraction(1, 2 ** 45)
    gc = synth.grouped_case(T=12, E=4, topk=2, N=40, K=128, seed=72, fmt="mxfp4")
    assert gc.s.shape == (4, 40, 4)
    g = oracle.grouped_gemm(gc.x, gc.offsets, gc.w, gc.s, None, False, None, fmt="mxfp4")
    gt = oracle.grouped_gemm_np(gc.x, gc.offsets, gc.w, gc.s, None, False, None, fmt="mxfp4")
    assert np.allclose(g, gt, rtol=1e-12, atol=0, equal_nan=True)


def _planted_mx(kind, c):
    codes = np.stack([c.w & 15, c.w >> 4], axis=-1).reshape(c.w.shape[0], -1)
    x = oracle.activation_np(c.x, c.pre)
    if kind == "group_16":        # scale index k // 16 (the NVFP4 grouping) instead of k // 32
        idx = np.minimum(np.arange(c.K) >> 4, c.s.shape[1] - 1)
        T = oracle.e2m1_np(codes) * oracle.e8m0_np(c.s[:, idx])
    elif kind == "bias_128":      # E8M0 bias off by one
        T = oracle.e2m1_np(codes) * np.repeat(np.exp2(c.s.astype(np.float64) - 128), 32, axis=1)
    elif kind == "as_e4m3":       # scale bytes read as E4M3
        T = oracle.e2m1_np(codes) * np.repeat(oracle.e4m3_np(c.s), 32, axis=1)
    else:
        T = oracle.dequant_np(c.w, c.s, "mxfp4")
    y = (x @ T.T).astype(np.float32)
    return torch.from_numpy(y).to(torch.bfloat16).to(torch.float64).numpy()


@pytest.mark.parametrize("kind", ["group_16", "bias_128", "as_e4m3"])
def test_mxfp4_planted_mistakes_fail_acceptance(kind):
    c = synth.dense_case(64, 512, 1024, seed=73, fmt="mxfp4", prescale=True)
    ref = oracle.gemm(c.x, c.w, c.s, c.g_stored, False, c.pre, fmt="mxfp4")
    assert oracle.accept(_planted_mx("none", c), ref)[0]
    ok, info = oracle.accept(_planted_mx(kind, c), ref)
    assert not ok, (kind, info)
