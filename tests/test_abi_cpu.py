"""The C ABI on the CPU: the library loads, exports every function the header
declares, and rejects invalid arguments on the host before any launch (no
GPU is touched: every call here returns before reaching the HIP runtime)."""
import ctypes
import os
import re

import pytest

import weight_only_fp4_amd as nv

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "nvfp4_w4a16.h")

OK, INVALID, ALIGN, SMALL = 0, 1, 2, 3


def _declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(nvfp4_[a-z0-9_]+)\s*\(", src)))


def test_library_exports_every_declared_function():
    names = _declared()
    assert len(names) >= 9
    L = nv.lib()
    for n in names:
        assert hasattr(L, n), n


def test_library_links_no_oracle_code():
    with open(nv.LIB_PATH, "rb") as f:
        blob = f.read()
    assert b"oracle_" not in blob


def test_repack_bytes_layout_size():
    # 16-row units x 128-wide K chunks, 1024 code bytes + 128 scale bytes each
    assert nv.repack_bytes(1, 16, 128) == 1152
    assert nv.repack_bytes(1, 1000, 1040) == 63 * 9 * 1152
    assert nv.repack_bytes(128, 1536, 2048) == 128 * 96 * 16 * 1152
    assert nv.lib().nvfp4_repack_bytes(1, 16, 8) < 0
    assert nv.lib().nvfp4_repack_bytes(0, 16, 16) < 0
    assert nv.lib().nvfp4_repack_bytes(1, 0, 16) == 0      # no rows: nothing to repack
    assert nv.lib().nvfp4_repack_bytes(1, -1, 16) < 0


def _p(v):
    return ctypes.c_void_p(v)


A = 1 << 20   # a fake, 16-byte-aligned address; never dereferenced (calls fail on the host first)


@pytest.mark.parametrize("args,status,needle", [
    (dict(K=24), INVALID, "multiple of 16"),
    (dict(K=0), INVALID, "multiple of 16"),
    (dict(N=-1), INVALID, "N ="),
    (dict(M=-1), INVALID, "negative"),
    (dict(ld_x=100), INVALID, "ld_x"),
    (dict(ld_y=10), INVALID, "ld_y"),
    (dict(w=None), INVALID, "w_repacked"),
    (dict(g=None), INVALID, "global scale"),
    (dict(x=A + 2), ALIGN, "16-byte"),
    (dict(ld_x=132), ALIGN, "ld_x"),
    (dict(y=A + 1), ALIGN, "y must be"),
    (dict(M=16, N=4096, K=14336, ld_x=14336, ld_y=4096, variant=2, pre=A, ws=A, wsb=10), SMALL, "workspace"),
    (dict(M=16, N=4096, K=14336, ld_x=14336, ld_y=4096, variant=2, ws=A + 16, wsb=1 << 30), ALIGN, "workspace"),
    (dict(ld_x=(1 << 23) + 8), INVALID, "exceeds"),
    (dict(variant=1, M=17), INVALID, "small-M"),
    (dict(variant=4, M=17), INVALID, "activation-resident"),
    (dict(variant=4, K=32896, ld_x=32896), INVALID, "activation-resident"),
    (dict(variant=4, N=32784, ld_y=32784), INVALID, "activation-resident"),
    # ceil(N / 16) * ceil(K / 4096) = 2048 * 2 > 2048: beyond the resident kernel although N, K <= 32768
    (dict(variant=4, M=16, N=32768, K=8192, ld_x=8192, ld_y=32768), INVALID, "ceil(N / 16) * ceil(K / 4096) <= 2048"),
    (dict(variant=4, M=16, N=14336, K=16384, ld_x=16384, ld_y=14336), INVALID, "activation-resident"),
    (dict(variant=5, K=24), INVALID, "multiple of 16"),
    (dict(variant=7), INVALID, "variant"),
])
def test_gemm_argument_errors(args, status, needle):
    a = dict(x=A, ld_x=128, pre=None, w=A, g=A, div=0, y=A, ld_y=32, M=4, N=32, K=128, ws=None, wsb=0, variant=0)
    a.update(args)
    L = nv.lib()
    st = L.nvfp4_w4a16_gemm_variant(_p(a["x"]), a["ld_x"], _p(a["pre"]), _p(a["w"]), _p(a["g"]), a["div"],
                                    _p(a["y"]), a["ld_y"], a["M"], a["N"], a["K"], _p(a["ws"]), a["wsb"],
                                    a["variant"], None)
    assert st == status
    assert needle in L.nvfp4_last_error().decode()


def test_zero_sizes_launch_nothing_and_succeed():
    """M == 0, R == 0 or N == 0: the call checks its arguments, returns OK and launches nothing (every pointer
    here is fake; a launch would fail on this host, which has no GPU, and report NVFP4_ERR_HIP)."""
    L = nv.lib()
    assert L.nvfp4_w4a16_gemm(None, 128, None, _p(A), _p(A), 0, None, 32, 0, 32, 128, None, 0, None) == OK
    assert L.nvfp4_last_error().decode() == ""
    assert L.nvfp4_w4a16_grouped_gemm(None, 128, _p(A), None, _p(A), _p(A), 0, None, 32, 0, 4, 32, 128,
                                      None, 0, None) == OK
    # no output columns: weights and output hold no bytes and may be NULL
    assert L.nvfp4_w4a16_gemm(_p(A), 128, None, None, _p(A), 0, None, 0, 4, 0, 128, None, 0, None) == OK
    assert L.nvfp4_w4a16_gemm_variant(_p(A), 128, None, None, _p(A), 0, None, 0, 4, 0, 128, None, 0, 4, None) == OK
    assert L.nvfp4_w4a16_gemm_f16(_p(A), 128, _p(A), None, _p(A), 1, None, 0, 300, 0, 128, None, 0, None) == OK
    assert L.nvfp4_w4a16_grouped_gemm(_p(A), 128, _p(A), None, None, _p(A), 0, None, 0, 8, 4, 0, 128,
                                      None, 0, None) == OK
    assert L.nvfp4_repack(None, 64, None, 8, 1, 0, 128, None, 0, None) == OK
    assert L.nvfp4_repack_bytes(3, 0, 128) == 0
    assert L.nvfp4_dequant_bf16(None, 1, 0, 128, None, 128, None) == OK
    assert L.nvfp4_w4a16_gemm_workspace_bytes(16, 0, 4096) == 0
    assert L.nvfp4_w4a16_gemm_plan(16, 0, 4096) == 0 and L.nvfp4_w4a16_gemm_plan(0, 4096, 4096) == 0
    # the other arguments are still checked
    assert L.nvfp4_w4a16_gemm(_p(A), 128, None, None, _p(A), 0, None, 0, 4, 0, 24, None, 0, None) == INVALID


def test_noalloc_entry_point_rejects_calls_beyond_its_scratch_before_any_launch():
    """The no-allocation entry point checks its arguments and its scratch need on the host first (fake pointers:
    nothing here reaches the GPU)."""
    L = nv.lib()
    cap = L.nvfp4_w4a16_gemm_noalloc_max_scratch_bytes()
    assert cap == 4 << 20
    assert L.nvfp4_w4a16_gemm_workspace_bytes(256, 512, 65536) > cap
    st = L.nvfp4_w4a16_gemm_noalloc(_p(A), 65536, None, _p(A), _p(A), 0, _p(A), 512, 256, 512, 65536, None)
    assert st == SMALL and "scratch" in L.nvfp4_last_error().decode()
    st = L.nvfp4_w4a16_gemm_noalloc(_p(A), 128, None, _p(A), _p(A), 0, _p(A), 32, 4, 32, 24, None)
    assert st == INVALID and "multiple of 16" in L.nvfp4_last_error().decode()
    assert L.nvfp4_w4a16_gemm_noalloc(None, 128, None, _p(A), _p(A), 0, None, 32, 0, 32, 128, None) == OK


def test_gemm_plan_names_the_automatic_kernel():
    """The automatic choice: small-M up to 4 rows, the activation-resident kernel for 5..16 rows where it takes the
    shape, the MFMA-bound kernel from 256 rows when the call has at least 48 of its 256 x 256 tiles, the tile kernel
    otherwise."""
    plan = nv.gemm_plan
    assert plan(1, 14336, 4096) == nv.VARIANT_SMALL_M and plan(4, 131072, 4096) == nv.VARIANT_SMALL_M
    for M in (5, 8, 16):
        assert plan(M, 14336, 4096) == nv.VARIANT_RESIDENT
        assert plan(M, 4096, 14336) == nv.VARIANT_RESIDENT
    assert plan(16, 16384, 8192) == nv.VARIANT_RESIDENT          # ceil(N/16) * ceil(K/4096) = 2048: the limit
    assert plan(16, 32768, 8192) == nv.VARIANT_LARGE_M           # 4096 > 2048
    assert plan(16, 131072, 4096) == nv.VARIANT_LARGE_M
    assert plan(16, 4096, 40960) == nv.VARIANT_LARGE_M           # K above 32768
    assert plan(17, 14336, 4096) == nv.VARIANT_LARGE_M
    assert plan(4096, 14336, 4096) == nv.VARIANT_MFMA and plan(8192, 17408, 5120) == nv.VARIANT_MFMA
    assert plan(256, 2048, 4096) == nv.VARIANT_LARGE_M           # 8 tiles: too few for the MFMA-bound kernel
    assert plan(64, 131072, 4096) == nv.VARIANT_LARGE_M
    with pytest.raises(ValueError):
        plan(4, 32, 24)


def test_grouped_and_repack_argument_errors():
    L = nv.lib()
    st = L.nvfp4_w4a16_grouped_gemm(_p(A), 128, None, None, _p(A), _p(A), 0, _p(A), 32, 8, 4, 32, 128, None, 0, None)
    assert st == INVALID and "expert_offsets" in L.nvfp4_last_error().decode()
    st = L.nvfp4_w4a16_grouped_gemm(_p(A), 128, _p(A), None, _p(A), _p(A), 0, _p(A), 32, 8, 0, 32, 128, None, 0, None)
    assert st == INVALID and "E =" in L.nvfp4_last_error().decode()
    n = nv.repack_bytes(1, 32, 128)
    assert L.nvfp4_repack(_p(A), 32, _p(A), 8, 1, 32, 128, _p(A), n, None) == INVALID      # ld_w < K/2
    assert L.nvfp4_repack(_p(A), 64, _p(A), 4, 1, 32, 128, _p(A), n, None) == INVALID      # ld_s < K/16
    assert L.nvfp4_repack(_p(A), 64, _p(A), 8, 1, 32, 128, _p(A + 8), n, None) == ALIGN
    assert L.nvfp4_repack(_p(A), 64, _p(A), 8, 1, 32, 128, _p(A), n - 1, None) == SMALL
    assert L.nvfp4_repack(None, 64, _p(A), 8, 1, 32, 128, _p(A), n, None) == INVALID
    assert L.nvfp4_dequant_bf16(_p(A), 1, 32, 128, _p(A), 64, None) == INVALID             # ld_out < K


def test_workspace_queries():
    """The workspace holds split-K partials and counters only: the pre-quant scale is applied in the kernels'
    activation loads, and calls whose kernels do not split K need none."""
    L = nv.lib()
    assert L.nvfp4_w4a16_gemm_workspace_bytes(0, 1000, 1040) == 0
    # M=16, N=4096, K=14336: K split across workgroups -> fp32 partials of 16 x 4096 per split, plus counters
    assert L.nvfp4_w4a16_gemm_workspace_bytes(16, 4096, 14336) > 2 * 16 * 4096 * 4
    # the MFMA-bound prefill call never splits K
    assert L.nvfp4_w4a16_gemm_workspace_bytes(4096, 14336, 4096) == 0
    # shapes the activation-resident kernel does not take size for the kernels that do (no split at these
    # widths): nothing, where the resident kernel's split area was counted before (16.8 MB, 134 MB, 2.16 GB)
    assert L.nvfp4_w4a16_gemm_workspace_bytes(1, 131072, 8192) == 0
    assert L.nvfp4_w4a16_gemm_workspace_bytes(1, 131072, 65536) == 0
    assert L.nvfp4_w4a16_gemm_workspace_bytes(4, 131072, 1 << 20) == 0
    assert L.nvfp4_w4a16_gemm_workspace_bytes(16, 32768, 8192) == 0
    assert L.nvfp4_w4a16_grouped_gemm_workspace_bytes(128, 128, 1536, 2048) == 0
    assert L.nvfp4_w4a16_gemm_workspace_bytes(-1, 10, 16) < 0


def test_moe_glue_argument_errors_and_empty_calls():
    L = nv.lib()
    route = lambda ids, T, k, E, off, rt, tr, ws=_p(A), wsb=1 << 20: L.nvfp4_moe_route(ids, T, k, E, off, rt, tr,
                                                                                       ws, wsb, None)
    assert route(_p(A), 4, 2, 0, _p(A), _p(A), _p(A)) == INVALID and "E =" in L.nvfp4_last_error().decode()
    assert route(_p(A), 4, 2, 2000, _p(A), _p(A), _p(A)) == INVALID
    assert route(_p(A), 4, 0, 8, _p(A), _p(A), _p(A)) == INVALID and "k =" in L.nvfp4_last_error().decode()
    assert route(_p(A), 4, 9, 8, _p(A), _p(A), _p(A)) == INVALID
    assert route(_p(A), -1, 2, 8, _p(A), _p(A), _p(A)) == INVALID
    assert route(_p(A), 4, 2, 8, None, _p(A), _p(A)) == INVALID
    assert route(_p(A + 2), 4, 2, 8, _p(A), _p(A), _p(A)) == ALIGN
    assert route(_p(A), 4, 2, 8, _p(A), _p(A), _p(A), wsb=8) == SMALL and "workspace" in L.nvfp4_last_error().decode()
    assert route(None, 0, 2, 8, _p(A), None, None, None, 0) == OK                    # zero tokens: no launch
    assert L.nvfp4_moe_route_workspace_bytes(2048, 8, 128) == 16 * 128 * 4            # one count per block, expert
    silu = L.nvfp4_moe_silu_mul
    assert silu(_p(A), 100, 4, 64, _p(A), 64, None) == INVALID and "ld_h" in L.nvfp4_last_error().decode()
    assert silu(_p(A), 128, 4, 64, _p(A), 32, None) == INVALID and "ld_a" in L.nvfp4_last_error().decode()
    assert silu(_p(A + 1), 128, 4, 64, _p(A), 64, None) == ALIGN
    assert silu(None, 128, 0, 64, None, 64, None) == OK
    comb = L.nvfp4_moe_combine
    assert comb(_p(A), 64, _p(A), _p(A), 4, 2, 0, _p(A), 64, None) == INVALID
    assert comb(_p(A), 32, _p(A), _p(A), 4, 2, 64, _p(A), 64, None) == INVALID
    assert comb(_p(A), 64, _p(A + 2), _p(A), 4, 2, 64, _p(A), 64, None) == ALIGN
    assert comb(None, 64, None, None, 0, 2, 64, None, 64, None) == OK
    gg = L.nvfp4_w4a16_grouped_gemm_gather
    args = lambda **kw: [kw.get(n, d) for n, d in [
        ("x", _p(A)), ("ld_x", 128), ("T", 16), ("rt", _p(A)), ("off", _p(A)), ("pre", None), ("w", _p(A)),
        ("g", _p(A)), ("div", 0), ("y", _p(A)), ("ld_y", 32), ("R", 32), ("E", 4), ("N", 32), ("K", 128),
        ("ws", None), ("wsb", 0), ("st", None)]]
    assert gg(*args(rt=None)) == INVALID and "row_token" in L.nvfp4_last_error().decode()
    assert gg(*args(rt=_p(A + 2))) == ALIGN
    assert gg(*args(T=0)) == INVALID
    assert gg(*args(T=1 << 20, ld_x=1 << 12)) == INVALID and "2^31" in L.nvfp4_last_error().decode()
    assert gg(*args(R=0)) == OK                                                      # zero rows: no launch
    assert L.nvfp4_w4a16_grouped_gemm_gather_workspace_bytes(16, 32, 4, 32, 128) == 0   # no copy of the tokens
    assert L.nvfp4_w4a16_grouped_gemm_gather_workspace_bytes(-1, 32, 4, 32, 128) == -1


def test_f16_entry_points_check_arguments_and_name_themselves():
    """The fp16 forms share the bf16 argument checks; their errors name the fp16 entry point."""
    L = nv.lib()
    st = L.nvfp4_w4a16_gemm_f16(_p(A), 128, None, _p(A), _p(A), 0, _p(A), 32, 4, 32, 24, None, 0, None)
    assert st == INVALID and "nvfp4_w4a16_gemm_f16" in L.nvfp4_last_error().decode()
    st = L.nvfp4_w4a16_gemm_variant_f16(_p(A), 128, None, _p(A), _p(A), 0, _p(A), 32, 17, 32, 128, None, 0, 1, None)
    assert st == INVALID and "small-M" in L.nvfp4_last_error().decode()
    st = L.nvfp4_w4a16_grouped_gemm_f16(_p(A), 100, _p(A), None, _p(A), _p(A), 0, _p(A), 32, 4, 2, 32, 128, None, 0,
                                        None)
    assert st == INVALID and "nvfp4_w4a16_grouped_gemm_f16" in L.nvfp4_last_error().decode()
    st = L.nvfp4_moe_silu_mul_f16(_p(A), 10, 4, 8, _p(A), 8, None)
    assert st == INVALID and "nvfp4_moe_silu_mul_f16" in L.nvfp4_last_error().decode()



def test_gated_repack_and_fused_fc1_argument_errors():
    """nvfp4_repack_gated and nvfp4_moe_fc1 reject bad arguments on the host; empty calls succeed."""
    L = nv.lib()
    assert L.nvfp4_repack_gated_bytes(4, 768, 2048) == L.nvfp4_repack_bytes(4, 1536, 2048)
    assert L.nvfp4_repack_gated_bytes(4, 100, 2048) == -1                              # I not a multiple of 16
    rg = lambda I=32, up=0, out=_p(A), nb=1 << 30: L.nvfp4_repack_gated(_p(A), 64, _p(A), 8, 2, I, 128, up, out, nb,
                                                                        None)
    assert rg(I=24) == INVALID and "multiple of 16" in L.nvfp4_last_error().decode()
    assert rg(up=2) == INVALID and "up_first" in L.nvfp4_last_error().decode()
    assert rg(nb=16) == SMALL
    assert rg(out=_p(A + 8)) == ALIGN
    assert rg(I=0) == OK                                                              # no rows: nothing to do
    fc1 = L.nvfp4_moe_fc1
    args = lambda **kw: [kw.get(n, d) for n, d in [
        ("x", _p(A)), ("ld_x", 128), ("T", 16), ("rt", _p(A)), ("off", _p(A)), ("pre", None), ("w", _p(A)),
        ("g", _p(A)), ("div", 0), ("act", 1), ("a", _p(A)), ("ld_a", 48), ("R", 32), ("E", 4), ("I", 48),
        ("K", 128), ("st", None)]]
    assert fc1(*args(act=0)) == INVALID and "activation" in L.nvfp4_last_error().decode()
    assert fc1(*args(act=3)) == INVALID
    assert fc1(*args(I=40, ld_a=40)) == INVALID and "multiple of 16" in L.nvfp4_last_error().decode()
    assert fc1(*args(act=2, I=40, ld_a=40, R=0)) == OK                                # relu2: any I; no rows
    assert fc1(*args(ld_a=40)) == INVALID and "ld_a" in L.nvfp4_last_error().decode()
    assert fc1(*args(rt=None)) == INVALID and "T = R" in L.nvfp4_last_error().decode()
    assert fc1(*args(rt=None, T=32, R=0)) == INVALID                                  # T != R without row_token
    assert fc1(*args(rt=None, T=0, R=0)) == OK
    assert fc1(*args(rt=_p(A + 2))) == ALIGN
    assert fc1(*args(K=120)) == INVALID                                               # K % 16
    assert fc1(*args(R=0)) == OK                                                      # zero rows: no launch
    st = L.nvfp4_moe_fc1_f16(*args(act=0))
    assert st == INVALID and "nvfp4_moe_fc1_f16" in L.nvfp4_last_error().decode()


def test_mxfp4_gated_repack_and_fused_fc1_argument_errors():
    """mxfp4_repack_gated and mxfp4_moe_fc1 (no global scales) reject bad arguments on the host: K a multiple of 32,
    I of 16, E8M0 scale rows of at least K/32 bytes; empty calls succeed."""
    L = nv.lib()
    assert L.mxfp4_repack_gated_bytes(4, 768, 2048) == L.mxfp4_repack_bytes(4, 1536, 2048)
    assert L.mxfp4_repack_gated_bytes(4, 100, 2048) == -1                              # I not a multiple of 16
    assert L.mxfp4_repack_gated_bytes(4, 32, 48) == -1                                 # K not a multiple of 32
    rg = lambda I=32, K=128, ld_s=4, up=0, out=_p(A), nb=1 << 30: L.mxfp4_repack_gated(
        _p(A), 64, _p(A), ld_s, 2, I, K, up, out, nb, None)
    assert rg(I=24) == INVALID and "multiple of 16" in L.nvfp4_last_error().decode()
    assert rg(up=2) == INVALID and "up_first" in L.nvfp4_last_error().decode()
    assert rg(K=80) == INVALID and "mxfp4_repack_gated" in L.nvfp4_last_error().decode()
    assert rg(ld_s=3) == INVALID and "K/32" in L.nvfp4_last_error().decode()
    assert rg(nb=16) == SMALL
    assert rg(out=_p(A + 8)) == ALIGN
    assert rg(I=0) == OK
    args = lambda **kw: [kw.get(n, d) for n, d in [
        ("x", _p(A)), ("ld_x", 128), ("T", 16), ("rt", _p(A)), ("off", _p(A)), ("pre", None), ("w", _p(A)),
        ("act", 1), ("a", _p(A)), ("ld_a", 48), ("R", 32), ("E", 4), ("I", 48), ("K", 128), ("st", None)]]
    for fc1, name in ((L.mxfp4_moe_fc1, "mxfp4_moe_fc1"), (L.mxfp4_moe_fc1_f16, "mxfp4_moe_fc1_f16")):
        assert fc1(*args(act=0)) == INVALID and name in L.nvfp4_last_error().decode()
        assert fc1(*args(I=40, ld_a=40)) == INVALID and "multiple of 16" in L.nvfp4_last_error().decode()
        assert fc1(*args(K=80, ld_x=80)) == INVALID                                   # K % 32
        assert fc1(*args(ld_a=40)) == INVALID and "ld_a" in L.nvfp4_last_error().decode()
        assert fc1(*args(rt=None)) == INVALID and "T = R" in L.nvfp4_last_error().decode()
        assert fc1(*args(rt=_p(A + 2))) == ALIGN
        assert fc1(*args(act=2, I=40, ld_a=40, R=0)) == OK                            # relu2: any I; no rows
        assert fc1(*args(R=0)) == OK
