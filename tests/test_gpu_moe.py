"""Parity of the MoE glue around the grouped GEMM (routing, the gathering grouped GEMM, the gated SiLU, the
non-gated squared ReLU and the top-k combine) with the CPU oracle, on the GPU.  Routing is integer work:
bit-exact.  The gathering GEMM runs the same kernels as the grouped GEMM on pre-gathered rows: bit-exact against
it, and within the acceptance bound of ``oracle.accept`` against the oracle, as are the activations and the
combine."""
import numpy as np
import pytest
import torch

import oracle
import synth
import weight_only_fp4_amd as nv
from gpu_util import DEV, bf16_bits, bf16_dev, bits16, f16_dev, f32_dev, to_f64, u8_dev

pytestmark = pytest.mark.gpu


def say(msg):
    print(f"[gpu-case] {msg}", flush=True)


def accept_or_fail(y, ref, what):
    ok, info = oracle.accept(y, ref)
    assert ok, (what, info)


def i32_dev(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(DEV)


def routing(T, k, E, seed):
    if E == 1:
        return np.zeros((T, 1), dtype=np.int64)
    return synth.zipf_routing(synth.rng(seed), T, E, k)


@pytest.mark.parametrize("T,k,E", [(16, 8, 128), (2048, 8, 128), (1, 1, 1), (300, 4, 4), (1500, 2, 1000),
                                   (7, 5, 5), (5000, 8, 128), (4096, 8, 64)])
def test_route_bit_exact(T, k, E):
    """One workgroup (up to 1024 pairs), count + place with the scan folded into place (up to 32 blocks of 1024
    pairs: T = 2048 and 4096 at k = 8), and count + scan + place (T = 5000 at k = 8: 40 blocks)."""
    say(f"route T={T} k={k} E={E}")
    ids = routing(T, k, E, seed=T + E)
    off, row_token, token_row = nv.moe_route(i32_dev(ids), E)
    r_off, r_rt, r_tr = oracle.moe_route(ids, E)
    assert np.array_equal(off.cpu().numpy(), r_off)
    assert np.array_equal(row_token.cpu().numpy(), r_rt)
    assert np.array_equal(token_row.cpu().numpy(), r_tr)


def _tokens_of(gc):
    """The token rows X[T, K] of a grouped case (its x holds them gathered in expert order)."""
    T = gc.meta["T"]
    xt = np.empty((T, gc.K), dtype=np.uint16)
    xt[gc.meta["token_of_row"]] = gc.x
    return xt


@pytest.mark.parametrize("T,E,topk,N,K,pre", [(16, 32, 4, 96, 256, False),      # small-M grouped path
                                              (256, 4, 2, 300, 272, True),      # tile grouped path, ragged N, K
                                              (64, 8, 8, 64, 128, False)])      # every expert active
def test_gather_gemm_matches_pre_gathered_and_oracle(T, E, topk, N, K, pre):
    gc = synth.grouped_case(T=T, E=E, topk=topk, N=N, K=K, seed=T + N, prescale=pre)
    say(f"gather gemm T={T} R={gc.R} E={E} N={N} K={K} pre={pre}")
    ids = gc.meta["routing"]
    off, row_token, _ = nv.moe_route(i32_dev(ids), E)
    assert np.array_equal(off.cpu().numpy(), gc.offsets)
    assert np.array_equal(row_token.cpu().numpy(), gc.meta["token_of_row"])
    xt = bf16_dev(_tokens_of(gc))
    blob = nv.repack(u8_dev(gc.w), u8_dev(gc.s))
    g = f32_dev(gc.g_stored)
    p = None if gc.pre is None else bf16_dev(gc.pre)
    y_gather = nv.grouped_gemm_gather(xt, row_token, off, blob, E, N, K, g, False, p)
    y_plain = nv.grouped_gemm(bf16_dev(gc.x), off, blob, E, N, K, g, False, p)
    torch.cuda.synchronize()
    assert torch.equal(y_gather, y_plain)
    ref = oracle.grouped_gemm(gc.x, gc.offsets, gc.w, gc.s, gc.g_stored, False, gc.pre)
    accept_or_fail(to_f64(y_gather), ref, "gather")


@pytest.mark.parametrize("R,I", [(128, 768), (37, 100), (1, 8)])
def test_silu_mul(R, I):
    say(f"silu_mul R={R} I={I}")
    g = synth.rng(R * 7 + I)
    h = synth.bf16_bits_from_f32((g.standard_normal((R, 2 * I)) * 3).astype(np.float32))
    hbig = torch.zeros((R, 2 * I + 16), dtype=torch.bfloat16, device=DEV)   # strided rows
    hbig[:, :2 * I] = bf16_dev(h)
    abig = torch.full((R, I + 8), 7.0, dtype=torch.bfloat16, device=DEV)
    nv.moe_silu_mul(hbig[:, :2 * I], out=abig[:, :I])
    accept_or_fail(to_f64(abig[:, :I]), oracle.silu_mul(h), "silu")
    assert torch.all(abig[:, I:] == 7.0)


@pytest.mark.parametrize("R,I", [(128, 768), (37, 100)])
def test_relu2(R, I):
    say(f"relu2 R={R} I={I}")
    g = synth.rng(R * 11 + I)
    h = synth.bf16_bits_from_f32((g.standard_normal((R, I)) * 4).astype(np.float32))
    a = nv.moe_relu2(bf16_dev(h))
    ref = oracle.relu2(h)
    y = to_f64(a)
    assert np.all(y[ref == 0] == 0)               # exact zeros where the input is not positive
    accept_or_fail(y, ref, "relu2")


@pytest.mark.parametrize("T,k,E,H", [(16, 8, 128, 2048), (300, 2, 8, 100), (1, 1, 1, 8)])
def test_combine(T, k, E, H):
    say(f"combine T={T} k={k} H={H}")
    ids = routing(T, k, E, seed=3 * T + H)
    _, _, token_row = oracle.moe_route(ids, E)
    g = synth.rng(T + H)
    y = synth.normal_bf16(g, (T * k, H))
    w = g.random((T, k)).astype(np.float32)
    out = nv.moe_combine(bf16_dev(y), i32_dev(token_row), torch.from_numpy(w).to(DEV))
    accept_or_fail(to_f64(out), oracle.combine(y, token_row, w), "combine")


@pytest.mark.parametrize("T", [16, 256])
def test_moe_layer_chain(T):
    """route -> FC1 (gathered) -> SiLU -> FC2 -> combine on the GPU; every stage checked against the oracle
    applied to the GPU's own input of that stage."""
    E, topk, Hd, I = 16, 4, 256, 192
    g = synth.rng(T)
    ids = synth.zipf_routing(synth.rng(T + 1), T, E, topk)
    say(f"moe layer T={T} E={E} top-{topk} hidden={Hd} I={I}")
    xt = synth.normal_bf16(g, (T, Hd))
    w1, s1 = synth.random_codes(g, (E, 2 * I, Hd)), synth.scales_pow2_mant(g, (E, 2 * I, Hd // 16))
    w2, s2 = synth.random_codes(g, (E, Hd, I)), synth.scales_pow2_mant(g, (E, Hd, I // 16))
    g1 = (np.exp2(g.integers(-2, 3, E).astype(np.float64)) / 2688).astype(np.float32)
    g2 = (np.exp2(g.integers(-2, 3, E).astype(np.float64)) / 2688).astype(np.float32)
    wts = g.random((T, topk)).astype(np.float32)
    b1, b2 = nv.repack(u8_dev(w1), u8_dev(s1)), nv.repack(u8_dev(w2), u8_dev(s2))

    off, row_token, token_row = nv.moe_route(i32_dev(ids), E)
    h = nv.grouped_gemm_gather(bf16_dev(xt), row_token, off, b1, E, 2 * I, Hd, f32_dev(g1))
    a = nv.moe_silu_mul(h)
    y2 = nv.grouped_gemm(a, off, b2, E, Hd, I, f32_dev(g2))
    out = nv.moe_combine(y2, token_row, torch.from_numpy(wts).to(DEV))
    torch.cuda.synchronize()

    r_off, r_rt, r_tr = oracle.moe_route(ids, E)
    assert np.array_equal(off.cpu().numpy(), r_off) and np.array_equal(token_row.cpu().numpy(), r_tr)
    accept_or_fail(to_f64(h), oracle.grouped_gemm(xt[r_rt], r_off, w1, s1, g1), "fc1")
    accept_or_fail(to_f64(a), oracle.silu_mul(bf16_bits(h)), "silu")
    accept_or_fail(to_f64(y2), oracle.grouped_gemm(bf16_bits(a), r_off, w2, s2, g2), "fc2")
    accept_or_fail(to_f64(out), oracle.combine(bf16_bits(y2), r_tr, wts), "combine")


@pytest.mark.parametrize("T", [16, 256])
def test_moe_layer_chain_f16(T):
    """The fp16 form of the layer: route -> FC1 (gathered, fp16) -> SiLU -> FC2 -> combine, and the squared ReLU,
    every stage checked against the oracle's fp16 definition applied to the GPU's own input of that stage."""
    E, topk, Hd, I = 16, 4, 256, 192
    g = synth.rng(T + 7)
    ids = synth.zipf_routing(synth.rng(T + 8), T, E, topk)
    say(f"moe layer fp16 T={T}")
    xt = synth.normal_act(g, (T, Hd), "f16")
    w1, s1 = synth.random_codes(g, (E, 2 * I, Hd)), synth.scales_pow2_mant(g, (E, 2 * I, Hd // 16))
    w2, s2 = synth.random_codes(g, (E, Hd, I)), synth.scales_pow2_mant(g, (E, Hd, I // 16))
    g1 = (np.exp2(g.integers(-2, 3, E).astype(np.float64)) / 2688).astype(np.float32)
    g2 = (np.exp2(g.integers(-2, 3, E).astype(np.float64)) / 2688).astype(np.float32)
    wts = g.random((T, topk)).astype(np.float32)
    b1, b2 = nv.repack(u8_dev(w1), u8_dev(s1)), nv.repack(u8_dev(w2), u8_dev(s2))

    off, row_token, token_row = nv.moe_route(i32_dev(ids), E)
    h = nv.grouped_gemm_gather(f16_dev(xt), row_token, off, b1, E, 2 * I, Hd, f32_dev(g1))
    a = nv.moe_silu_mul(h)
    r2 = nv.moe_relu2(h[:, :I])
    y2 = nv.grouped_gemm(a, off, b2, E, Hd, I, f32_dev(g2))
    out = nv.moe_combine(y2, token_row, torch.from_numpy(wts).to(DEV))
    torch.cuda.synchronize()
    assert h.dtype == a.dtype == r2.dtype == y2.dtype == out.dtype == torch.float16

    r_off, r_rt, r_tr = oracle.moe_route(ids, E)
    accept_or_fail(to_f64(h), oracle.grouped_gemm_f16(xt[r_rt], r_off, w1, s1, g1), "fc1 f16")
    accept_or_fail(to_f64(a), oracle.silu_mul(bits16(h), "f16"), "silu f16")
    accept_or_fail(to_f64(r2), oracle.relu2(bits16(h[:, :I]), "f16"), "relu2 f16")
    accept_or_fail(to_f64(y2), oracle.grouped_gemm_f16(bits16(a), r_off, w2, s2, g2), "fc2 f16")
    accept_or_fail(to_f64(out), oracle.combine(bits16(y2), r_tr, wts, "f16"), "combine f16")

