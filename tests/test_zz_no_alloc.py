"""The entry point that allocates nothing (nvfp4_w4a16_gemm_noalloc), on the GPU, through the C ABI: its outputs
are bitwise those of nvfp4_w4a16_gemm with a caller's workspace, on calls in a row that use the library's static
split-K scratch (the second with a smaller input, whose partials and counters overlap the first call's), a call
that needs no scratch, and a pre-quant scale; a call needing more scratch than the array holds is rejected
before anything runs."""
import pytest
import torch

import synth
import weight_only_fp4_amd as nv
from gpu_util import DEV, DenseDev

pytestmark = pytest.mark.gpu


def say(msg):
    print(f"[gpu-case] {msg}", flush=True)


CASES = [
    # (M, N, K, seed, pre): the activation-resident kernel split 4 ways, then 2 ways on a smaller input
    (16, 4096, 14336, 3001, False),
    (8, 2064, 8192, 3002, True),
    (1, 2048, 512, 3003, False),     # no K split: no scratch touched
    (24, 2000, 4096, 3004, False),   # the tile kernel split across workgroups, N tail
]


def test_noalloc_matches_workspace_entry_point_on_calls_in_a_row():
    L = nv.lib()
    assert L.nvfp4_w4a16_gemm_noalloc_max_scratch_bytes() == 4 << 20
    devs = []
    for M, N, K, seed, pre in CASES:
        c = synth.dense_case(M, N, K, seed, prescale=pre, g_stored=2688.0 if pre else 1 / 2688,
                             g_is_divisor=pre)
        devs.append(DenseDev(c))
    for rnd in range(2):
        for d in devs:
            c = d.c
            need = nv.gemm_workspace_bytes(c.M, c.N, c.K)
            say(f"noalloc round {rnd} M={c.M} N={c.N} K={c.K} scratch={need}")
            assert need <= 4 << 20
            ref = nv.gemm(d.x, d.blob, c.N, c.K, d.g, c.g_is_divisor, d.pre)
            y = torch.full((c.M, c.N), float("nan"), dtype=torch.bfloat16, device=DEV)
            st = L.nvfp4_w4a16_gemm_noalloc(nv._ptr(d.x), c.K, nv._ptr(d.pre), nv._ptr(d.blob), nv._ptr(d.g),
                                            int(c.g_is_divisor), nv._ptr(y), c.N, c.M, c.N, c.K,
                                            nv._stream(torch.device(DEV)))
            assert st == 0, L.nvfp4_last_error().decode()
            torch.cuda.synchronize()
            assert torch.equal(y, ref), (rnd, c.M, c.N, c.K)
            assert torch.equal(nv.gemm_noalloc(d.x, d.blob, c.N, c.K, d.g, c.g_is_divisor, d.pre), ref)


def test_noalloc_rejects_calls_beyond_its_scratch():
    """M = 256, N = 512, K = 65536: the tile kernel splits K 16 ways over 4 tiles of 128 x 256 (8 MiB of
    partials), more than the 4 MiB array: BUFFER_TOO_SMALL, and the output is untouched."""
    M, N, K = 256, 512, 65536
    L = nv.lib()
    assert nv.gemm_workspace_bytes(M, N, K) > 4 << 20
    x = torch.zeros((M, K), dtype=torch.bfloat16, device=DEV)
    blob = torch.zeros(nv.repack_bytes(1, N, K), dtype=torch.uint8, device=DEV)
    g = torch.ones(1, dtype=torch.float32, device=DEV)
    y = torch.full((M, N), 3.0, dtype=torch.bfloat16, device=DEV)
    st = L.nvfp4_w4a16_gemm_noalloc(nv._ptr(x), K, None, nv._ptr(blob), nv._ptr(g), 0, nv._ptr(y), N, M, N, K,
                                    nv._stream(torch.device(DEV)))
    assert st == 3 and "scratch" in L.nvfp4_last_error().decode()
    torch.cuda.synchronize()
    assert torch.all(y == 3.0)
