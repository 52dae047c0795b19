"""The weight decode of every production GEMM kernel, pinned bit-exactly over the whole format, on the GPU.

A weight whose 16-wide K blocks hold all 16 E2M1 codes and whose scale bytes run through every ordered pair of
the 254 finite E4M3 codes (NaN codes excluded; negative, zero and subnormal codes included) as the two blocks of
a 32-wide K group is pushed through each kernel with one-hot activation rows and g = 1: every output is then a
single exact product, Y[m, n] = T[n, k_m] (all 16 x 254 code-scale products are exact in bf16 and fp16), so the
kernels' own scale and code decoding is compared bit for bit (signed zeros compare equal) with the oracle's
decode (the E2M1 codebook times the E4M3 scale: "Support Nemotron-H nvfp4 ckpt on Hopper", Walkthrough; OCP
E4M3FN).  Forms: the small-M kernel's one- and two-row-group 4x4x4 passes (4 and 8 rows) and its 16x16x32 pass
(16 rows), the activation-resident kernel, the tile kernel, the MFMA-bound kernel in whole, half and 64-row
tiles, and both grouped paths with the weight as the only active expert among empty ones."""
import numpy as np
import pytest
import torch

import oracle
import synth
import weight_only_fp4_amd as nv
from gpu_util import DEV, act_dev, f32_dev, to_f64, u8_dev

pytestmark = pytest.mark.gpu

FINITE_E4M3 = np.array([b for b in range(256) if b not in (0x7F, 0xFF)], dtype=np.uint8)
ONE = {"bf16": 0x3F80, "f16": 0x3C00}


def say(msg):
    print(f"[gpu-case] {msg}", flush=True)


def pair_enumeration_weight():
    """N = 8065 rows x K = 256: pair p = 8 n + j (mod 254^2) puts scale bytes (finite[p % 254], finite[p // 254])
    on blocks 2 j and 2 j + 1 of row n; code(n, k) = (n + k) mod 16, so every block holds all 16 codes."""
    nf = len(FINITE_E4M3)
    N, K = -(-nf * nf // 8), 256
    p = np.arange(N * 8) % (nf * nf)
    s = np.stack([FINITE_E4M3[p % nf], FINITE_E4M3[p // nf]], axis=1).reshape(N, 16)
    codes = (np.arange(K)[None, :] + np.arange(N)[:, None]) % 16
    return synth.pack_codes(codes.astype(np.uint8)), s


_W = {}


def weight():
    if not _W:
        w, s = pair_enumeration_weight()
        _W.update(w=w, s=s, T=oracle.dequant(w, s))
        # the enumeration is complete: every finite byte pair, and every code under every finite scale
        pairs = {(int(a), int(b)) for a, b in s.reshape(-1, 2)}
        assert len(pairs) == len(FINITE_E4M3) ** 2
    return _W


def one_hot(rows, K, k0, act):
    """rows x K activation bits with row m one-hot at (k0 + m) mod K."""
    x = np.zeros((rows, K), dtype=np.uint16)
    x[np.arange(rows), (k0 + np.arange(rows)) % K] = ONE[act]
    return x


DENSE_FORMS = [
    ("small_m_4rows", nv.VARIANT_SMALL_M, 4),      # 4x4x4, one row group
    ("small_m_8rows", nv.VARIANT_SMALL_M, 8),      # 4x4x4, two row groups
    ("small_m_16rows", nv.VARIANT_SMALL_M, 16),    # 16x16x32
    ("resident_16rows", nv.VARIANT_RESIDENT, 16),
    ("resident_5rows", nv.VARIANT_RESIDENT, 5),
    ("tile_256rows", nv.VARIANT_LARGE_M, 256),
    ("tile_16rows", nv.VARIANT_LARGE_M, 16),
    # 2304 rows = 9 x 256 one-hot blocks: 288 output tiles, 256 run whole and the last 32 as half tiles
    ("mfma_2304rows", nv.VARIANT_MFMA, 2304),
    ("mfma_quarter_2304rows", nv.VARIANT_MFMA_QUARTER, 2304),
]


@pytest.mark.parametrize("act", ["bf16", "f16"])
@pytest.mark.parametrize("name,variant,rows", DENSE_FORMS, ids=[f[0] for f in DENSE_FORMS])
def test_dense_kernels_decode_every_code_and_scale_pair(name, variant, rows, act):
    W = weight()
    N, K = W["T"].shape
    say(f"decode enumeration {name} {act} N={N} K={K}")
    blob = nv.repack(u8_dev(W["w"]), u8_dev(W["s"]))
    g = f32_dev(1.0)
    for k0 in range(0, K, rows):
        r = min(rows, K - k0) if rows <= K else rows
        x = act_dev(one_hot(r, K, k0, act), act)
        y = to_f64(nv.gemm_variant(x, blob, N, K, g, False, None, variant=variant))
        ks = (k0 + np.arange(r)) % K
        exp = W["T"][:, ks].T
        if not np.array_equal(y, exp):
            bad = np.argwhere(y != exp)[:5]
            raise AssertionError((name, act, k0, [(int(m), int(n), y[m, n], exp[m, n],
                                                   hex(W["s"][n, ks[m] // 16])) for m, n in bad]))


@pytest.mark.parametrize("act", ["bf16", "f16"])
@pytest.mark.parametrize("rows", [4, 16, 256], ids=["small_m_4rows", "small_m_16rows", "tile_256rows"])
def test_grouped_kernels_decode_every_code_and_scale_pair(rows, act):
    """The enumeration weight is expert 1 of 3; experts 0 and 2 get no rows (their weights are random and must
    not be read into any output).  R <= 16 E takes the grouped small-M path, R > 16 E the grouped tile path."""
    W = weight()
    N, K = W["T"].shape
    say(f"grouped decode enumeration rows={rows} {act}")
    other = synth.rng(71)
    w = np.stack([synth.random_codes(other, (N, K)), W["w"], synth.random_codes(other, (N, K))])
    s = np.stack([synth.scales_pow2_mant(other, (N, K // 16)), W["s"], synth.scales_pow2_mant(other, (N, K // 16))])
    blob = nv.repack(u8_dev(w), u8_dev(s))
    g = f32_dev([1.0, 1.0, 1.0])
    for k0 in range(0, K, rows):
        r = min(rows, K - k0)
        off = torch.tensor([0, 0, r, r], dtype=torch.int32, device=DEV)
        x = act_dev(one_hot(r, K, k0, act), act)
        y = to_f64(nv.grouped_gemm(x, off, blob, 3, N, K, g))
        assert np.array_equal(y, W["T"][:, k0:k0 + r].T), (rows, act, k0)
