"""Host-only checks of the C-ABI library (no GPU needed): it loads, exports
every function include/ocg.h declares, rejects bad arguments with status
codes, and its closed-form ticket schedule equals the oracle's enumerated
re-derivation ticket by ticket."""
import ctypes as C
import os
import re
import subprocess
import sys

import pytest

import communication_overlapped_gemm_amd as ocg
from communication_overlapped_gemm_amd import _lib
from oracle import schedule as sch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ocg.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(ocg_[a-z_]+)\s*\(", text)))


def test_header_declares_the_binding_exports():
    assert declared_functions() == sorted(ocg.EXPORTS)


def test_library_exports_every_declared_symbol():
    out = subprocess.run(["nm", "-D", "--defined-only", ocg.LIB_PATH], capture_output=True, text=True, check=True)
    exported = set(re.findall(r"\bT (ocg_\w+)", out.stdout))
    missing = [f for f in declared_functions() if f not in exported]
    assert not missing, f"not exported: {missing}"
    for f in declared_functions():
        assert hasattr(ocg.lib, f)


def test_builder_loads_without_the_library(tmp_path):
    """A fresh checkout has no libocg.so: the builder must load without
    importing the package (whose import loads the library), as the build
    entry point does."""
    import shutil
    pkg = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "communication_overlapped_gemm_amd")
    dst = tmp_path / "communication_overlapped_gemm_amd"
    shutil.copytree(pkg, dst, ignore=shutil.ignore_patterns("*.so", "__pycache__"))
    code = ("import importlib.util, sys; "
            f"spec = importlib.util.spec_from_file_location('b', {str(dst / 'build.py')!r}); "
            "m = importlib.util.module_from_spec(spec); spec.loader.exec_module(m); "
            "assert callable(m.build) and 'communication_overlapped_gemm_amd' not in sys.modules")
    subprocess.run([sys.executable, "-c", code], check=True, cwd=str(tmp_path))
    res = subprocess.run([sys.executable, "-c", "import communication_overlapped_gemm_amd"], cwd=str(tmp_path),
                         capture_output=True, text=True)
    assert res.returncode != 0 and "no fallback" in res.stderr   # the product path fails loudly


def test_status_strings_and_defaults():
    assert ocg.status_string(ocg.OK) == "ok"
    assert "timed out" in ocg.status_string(ocg.ERR_TIMEOUT)
    c = ocg.default_config()
    assert c.tile == -1 and c.swizzle == 1 and c.mode == 0 and c.fault_skip_slab == -1 and not c.trace


def test_workspace_bytes_validation():
    lib = ocg.lib
    assert lib.ocg_workspace_bytes(None, 0, 8, 1024, 8192, 3584, 0, 0) > 256
    assert lib.ocg_workspace_bytes(None, 0, 8, 1024, 8190, 3584, 0, 0) == 0      # K % 64
    assert lib.ocg_workspace_bytes(None, 0, 8, 1024, 8192, 3583, 0, 0) == 0      # N % 8
    assert lib.ocg_workspace_bytes(None, 0, 17, 1024, 8192, 3584, 0, 0) == 0     # R > 16
    assert lib.ocg_workspace_bytes(None, 1, 8, 4095, 1792, 4096, 0, 0) == 0      # M % R
    assert lib.ocg_workspace_bytes(None, 2, 8, 512, 4096, 1792, 32, 2) > 0
    assert lib.ocg_workspace_bytes(None, 2, 8, 512, 4096, 1792, 65, 2) == 0      # E > 64
    assert lib.ocg_workspace_bytes(None, 2, 8, 512, 4096, 1792, 32, 5) == 0      # topk > 4
    assert lib.ocg_workspace_bytes(None, 3, 8, 512, 4096, 1792, 0, 0) == 0       # bad op


def test_entry_points_reject_null_arguments_without_a_device():
    lib = ocg.lib
    cfg = ocg.default_config()
    ptrs = (C.c_void_p * 2)()
    assert lib.ocg_ag_gemm(None, ptrs, 2, 0, 64, 64, None, 64, None, None, None, 0, C.byref(cfg), None) \
        == ocg.ERR_INVALID_ARG
    assert lib.ocg_gemm_rs(None, None, None, 64, 64, 64, 2, 0, ptrs, None, None, None, 0, C.byref(cfg), None) \
        == ocg.ERR_INVALID_ARG
    assert lib.ocg_signal(None, 4, 1, None) == ocg.ERR_INVALID_ARG
    assert lib.ocg_create(0, None) == ocg.ERR_INVALID_ARG


def test_plan_info_tile_choice():
    # 70B share: 256x224 tiles (exactly 512 = two rounds of 256 CUs)
    p = ocg.plan_info(ocg.OP_AG_GEMM, 8, 0, 1024, 8192, 3584)
    assert (p["BM"], p["BN"], p["n_tiles"]) == (256, 224, 512)
    assert ocg.plan_ag(8, 0, 1024, 8192, 3584)["split_k"] == 1
    # 8B share: 128x224 (256 tiles, one per CU), whole tiles (K halves of
    # 256x224 tiles and 224 tiles of 128x256 measured slower)
    p = ocg.plan_info(ocg.OP_AG_GEMM, 8, 0, 512, 4096, 1792)
    assert (p["BM"], p["BN"], p["n_tiles"]) == (128, 224, 256)
    assert ocg.plan_ag(8, 0, 512, 4096, 1792)["split_k"] == 1
    # a 1024-row share with K 8192: 112 tiles of 128x128 fill under half the
    # CUs, so they run as 224 K halves
    p = ocg.plan_info(ocg.OP_AG_GEMM, 8, 0, 128, 8192, 1792)
    assert (p["BM"], p["BN"], p["n_tiles"]) == (128, 128, 112)
    assert ocg.plan_ag(8, 0, 128, 8192, 1792)["split_k"] == 2
    # GEMM-RS 4096 x 4096: 256x256 (256 tiles, one round)
    p = ocg.plan_info(ocg.OP_GEMM_RS, 8, 0, 4096, 1792, 4096)
    assert (p["BM"], p["BN"], p["n_tiles"]) == (256, 256, 256)
    # tiny AllGather share (4 x [128, 256] x [256, 256]): 128x128, 8 tiles
    p = ocg.plan_info(ocg.OP_AG_GEMM, 4, 0, 128, 256, 256)
    assert (p["BM"], p["BN"], p["n_tiles"]) == (128, 128, 8)
    assert ocg.plan_ag(4, 0, 128, 256, 256)["split_k"] == 1


def test_plan_info_moe_tile_choice():
    # 4096 tokens x top-2 over 32 experts: 256 rows per expert on average,
    # standard deviation 15.5: one 288-row tile per expert
    p = ocg.plan_info(ocg.OP_AG_GROUPED_GEMM, 8, 0, 512, 4096, 1792, E=32, topk=2)
    assert (p["BM"], p["BN"]) == (288, 224)
    # 2048 tokens x top-2 over 16: mean 256, deviation 15.5 -> 288 as well;
    # 1536 tokens x top-3 over 16: mean 288, deviation 16.4 -> 320
    p = ocg.plan_info(ocg.OP_AG_GROUPED_GEMM, 8, 0, 192, 128, 448, E=16, topk=3)
    assert (p["BM"], p["BN"]) == (320, 224)
    p = ocg.plan_info(ocg.OP_AG_GROUPED_GEMM, 2, 0, 64, 128, 96, E=6, topk=2)
    assert (p["BM"], p["BN"]) == (128, 224)
    p = ocg.plan_info(ocg.OP_AG_GROUPED_GEMM, 8, 0, 1024, 128, 96, E=8, topk=2)
    assert (p["BM"], p["BN"]) == (256, 224)   # ~2048 rows per expert: many 256-row tiles
    # the 288- and 320-row presets are the grouped GEMM's only
    for op, m in ((ocg.OP_AG_GEMM, 512), (ocg.OP_GEMM_RS, 4096)):
        for t in (ocg.TILE_320x224, ocg.TILE_288x224):
            with pytest.raises(ocg.OcgError):
                ocg.plan_info(op, 8, 0, m, 1792, 4096, ocg.default_config(tile=t))


AG_CASES = [
    # R, m, K, N, local, tile
    (4, 128, 256, 256, 0, -1),
    (8, 512, 4096, 1792, 0, -1),
    (8, 1024, 8192, 3584, 0, -1),
    (8, 1024, 8192, 3584, 3, -1),
    (3, 100, 64, 72, 1, ocg.TILE_128x128),
    (5, 37, 128, 40, 4, ocg.TILE_128x128),
    (3, 300, 192, 520, 2, ocg.TILE_256x224),
    (3, 300, 256, 600, 1, ocg.TILE_256x256),
]


def ag_grid_tiles(info, R, m, N):
    """Tiles per round of the persistent GEMM grid on a 256-CU MI355X: one
    workgroup per CU (two for the 128x128 tile, by LDS and registers)."""
    return 256 * (2 if (info["BM"], info["BN"]) == (128, 128) else 1)


@pytest.mark.parametrize("case", AG_CASES)
@pytest.mark.parametrize("swizzle", [1, 0])
@pytest.mark.parametrize("mode", ["fused", "gemm_only", "copy_only"])
@pytest.mark.parametrize("transfer,kslab", [(ocg.TRANSFER_INLINE, 0), (ocg.TRANSFER_SIDE, 0),
                                            (ocg.TRANSFER_INLINE, 256)])
def test_ag_plan_matches_oracle_schedule(case, swizzle, mode, transfer, kslab):
    R, m, K, N, local, tile = case
    modes = {"fused": 0, "gemm_only": 1, "copy_only": 2}
    cfg = ocg.default_config(tile=tile, swizzle=swizzle, mode=modes[mode], transfer=transfer, kslab_cols=kslab)
    info = ocg.plan_info(ocg.OP_AG_GEMM, R, local, m, K, N, cfg)
    ag = ocg.plan_ag(R, local, m, K, N, cfg)
    # K-slab width: the whole K unless asked for, 512 by default for the side producer
    side = transfer == ocg.TRANSFER_SIDE and mode != "gemm_only"
    want_ks = min(K, kslab or (512 if side else K))
    assert ag["kslab_cols"] == want_ks and ag["nks"] == -(-K // want_ks)
    # rows per round: the persistent grid's tiles per round over the column blocks
    n_cb = -(-N // info["BN"])
    assert ag["rows_per_round"] == max(1, ag_grid_tiles(info, R, m, N) // (n_cb * ag["split_k"])) * info["BM"]
    want = sch.ag_gemm_plan(R, m, K, N, local, info["BM"], info["BN"], info["slab_rows"], info["copy_rows"],
                            bool(swizzle), mode, KS=ag["kslab_cols"], rpr=ag["rows_per_round"], sk=ag["split_k"])
    if side and mode != "gemm_only":
        # the GEMM kernel copies the first K-slab of the first phase itself
        first = sch.copy_phases(R, m, local, bool(swizzle), ag["rows_per_round"])[0]
        n_inline = len(first) * -(-m // info["copy_rows"]) if ag["nks"] > 1 or len(first) < R else len(want)
        assert ag["n_inline"] == min(n_inline, info["n_copy_or_strips"])
    assert len(want) == info["n_copy_or_strips"] + info["n_tiles"] * ag["split_k"]
    n_flags = R * -(-m // info["slab_rows"]) * ag["nks"]
    assert info["n_slabs_or_strip_rows"] == n_flags
    for t in want + [None]:
        ticket = len(want) if t is None else t.ticket
        d = ocg.plan_task(ocg.OP_AG_GEMM, R, local, m, K, N, ticket, cfg)
        if t is None:
            assert d[0] == 0
        elif isinstance(t, sch.CopyTask):
            assert d[:7] == [1, t.chunk, t.piece, t.row0, t.row1, t.slab, t.kslab]
            assert 0 <= t.flag < n_flags
        else:
            deps = list(t.deps)
            assert d[:4] == [2, t.rb, t.cb, len(deps)]
            assert d[4:4 + min(3, len(deps))] == deps[:3]
            assert d[7] == t.part


def test_split_k_rules_and_workspace():
    lib = ocg.lib
    ws = lambda R, m, K, N, cfg=None: lib.ocg_workspace_bytes_for(None, ocg.OP_AG_GEMM, R, m, K, N, 0, 0,
                                                                  C.byref(cfg) if cfg is not None else None)
    # a 1024-row share with K 8192 splits by default: room for 112 tiles of
    # 128x128 fp32 sums
    base = ws(8, 128, 8192, 1792, ocg.default_config(split_k=1))
    assert ws(8, 128, 8192, 1792) == lib.ocg_workspace_bytes(None, ocg.OP_AG_GEMM, 8, 128, 8192, 1792, 0, 0)
    assert ws(8, 128, 8192, 1792) >= base + 112 * 128 * 128 * 4
    # the 8B share keeps whole tiles: flags only
    assert lib.ocg_workspace_bytes(None, ocg.OP_AG_GEMM, 8, 512, 4096, 1792, 0, 0) < (1 << 20)
    # the 70B share does not, unless asked
    base70 = lib.ocg_workspace_bytes(None, ocg.OP_AG_GEMM, 8, 1024, 8192, 3584, 0, 0)
    assert base70 < (1 << 20)
    forced = ocg.default_config(split_k=2)
    assert ocg.plan_ag(8, 0, 1024, 8192, 3584, forced)["split_k"] == 2
    p = ocg.plan_info(ocg.OP_AG_GEMM, 8, 0, 1024, 8192, 3584, forced)
    assert ws(8, 1024, 8192, 3584, forced) >= base70 + p["n_tiles"] * p["BM"] * p["BN"] * 4
    # split off, explicitly
    assert ocg.plan_ag(8, 0, 512, 4096, 1792, ocg.default_config(split_k=1))["split_k"] == 1
    # split needs inline copies, one K-slab and K % 128 == 0; the knob is 0..2
    for cfg, K in ((ocg.default_config(split_k=2, transfer=ocg.TRANSFER_SIDE), 4096),
                   (ocg.default_config(split_k=2, kslab_cols=1024), 4096),
                   (ocg.default_config(split_k=2), 4160),
                   (ocg.default_config(split_k=2, mode=ocg.MODE_COPY_ONLY), 4096),
                   (ocg.default_config(split_k=3), 4096), (ocg.default_config(split_k=-1), 4096)):
        with pytest.raises(ocg.OcgError):
            ocg.plan_ag(8, 0, 512, K, 1792, cfg)
        assert ws(8, 512, K, 1792, cfg) == 0
    # the automatic choice only splits where it can: SIDE and K-slabs keep whole tiles
    assert ocg.plan_ag(8, 0, 128, 8192, 1792, ocg.default_config(transfer=ocg.TRANSFER_SIDE))["split_k"] == 1
    assert ocg.plan_ag(8, 0, 128, 8192, 1792, ocg.default_config(kslab_cols=1024))["split_k"] == 1
    assert ocg.plan_ag(8, 0, 128, 8128, 1792)["split_k"] == 1


@pytest.mark.parametrize("case", [(8, 512, 4096, 1792, 0, -1), (8, 512, 4096, 1792, 5, -1),
                                  (3, 300, 256, 600, 1, ocg.TILE_256x224), (5, 37, 128, 40, 4, ocg.TILE_128x128),
                                  (2, 200, 384, 296, 1, ocg.TILE_256x256)])
@pytest.mark.parametrize("mode", ["fused", "gemm_only"])
def test_split_plan_matches_oracle_schedule(case, mode):
    R, m, K, N, local, tile = case
    modes = {"fused": 0, "gemm_only": 1}
    cfg = ocg.default_config(tile=tile, mode=modes[mode], split_k=2)
    info = ocg.plan_info(ocg.OP_AG_GEMM, R, local, m, K, N, cfg)
    ag = ocg.plan_ag(R, local, m, K, N, cfg)
    assert ag["split_k"] == 2 and ag["nks"] == 1
    n_cb = -(-N // info["BN"])
    assert ag["rows_per_round"] == max(1, ag_grid_tiles(info, R, m, N) // (n_cb * 2)) * info["BM"]
    want = sch.ag_gemm_plan(R, m, K, N, local, info["BM"], info["BN"], info["slab_rows"], info["copy_rows"],
                            True, mode, KS=K, rpr=ag["rows_per_round"], sk=2)
    assert len(want) == info["n_copy_or_strips"] + 2 * info["n_tiles"]
    units = [t for t in want if isinstance(t, sch.Tile)]
    assert [t.part for t in units] == [0, 1] * info["n_tiles"]
    for t in want + [None]:
        ticket = len(want) if t is None else t.ticket
        d = ocg.plan_task(ocg.OP_AG_GEMM, R, local, m, K, N, ticket, cfg)
        if t is None:
            assert d[0] == 0
        elif isinstance(t, sch.CopyTask):
            assert d[:7] == [1, t.chunk, t.piece, t.row0, t.row1, t.slab, t.kslab]
        else:
            deps = list(t.deps)
            assert d[:4] == [2, t.rb, t.cb, len(deps)] and d[7] == t.part
            assert d[4:4 + min(3, len(deps))] == deps[:3]


@pytest.mark.parametrize("R,M,K,N,local,tile", [(8, 4096, 1792, 4096, 0, -1), (8, 4096, 1792, 4096, 5, -1),
                                                (4, 96, 64, 40, 2, ocg.TILE_128x128),
                                                (3, 600, 128, 264, 1, ocg.TILE_256x224)])
def test_rs_plan_matches_oracle_schedule(R, M, K, N, local, tile):
    cfg = ocg.default_config(tile=tile)
    info = ocg.plan_info(ocg.OP_GEMM_RS, R, local, M, K, N, cfg)
    want = sch.gemm_rs_plan(R, M, N, local, info["BM"], info["BN"], info["n_slabs_or_strip_rows"])
    for t in want:
        d = ocg.plan_task(ocg.OP_GEMM_RS, R, local, M, K, N, t[1], cfg)
        if t[0] == "tile":
            assert d[:6] == [3, t[2], t[3], int(t[4]), t[5], t[6]]
        else:
            assert d[:3] == [5, t[2], t[3]]
    assert ocg.plan_task(ocg.OP_GEMM_RS, R, local, M, K, N, len(want), cfg)[0] == 0


ATTN_CASES = [
    # R, m, Hq, Hkv, local, slab_rows, copy_rows
    (8, 2048, 32, 8, 0, 0, 0),
    (8, 2048, 32, 8, 5, 256, 0),
    (3, 200, 8, 2, 2, 64, 16),
    (4, 70, 6, 2, 1, 0, 0),
    (2, 1, 4, 4, 1, 0, 0),
]


@pytest.mark.parametrize("case", ATTN_CASES)
@pytest.mark.parametrize("swizzle", [1, 0])
@pytest.mark.parametrize("mode", ["fused", "gemm_only", "copy_only"])
def test_attention_plan_matches_oracle_schedule(case, swizzle, mode):
    R, m, Hq, Hkv, local, S, CT = case
    modes = {"fused": 0, "gemm_only": 1, "copy_only": 2}
    cfg = ocg.default_config(swizzle=swizzle, mode=modes[mode], slab_rows=S, copy_rows=CT)
    info = ocg.plan_info(ocg.OP_AG_ATTENTION, R, local, m, Hq, Hkv, cfg)
    assert (info["BM"], info["BN"]) == (256, 64)
    want = sch.attention_plan(R, m, Hq, Hkv, local, info["slab_rows"], info["copy_rows"], bool(swizzle), mode)
    assert len(want) == info["n_copy_or_strips"] + info["n_tiles"]
    assert info["n_slabs_or_strip_rows"] == R * (-(-m // info["slab_rows"]))
    for t in want:
        d = ocg.plan_task(ocg.OP_AG_ATTENTION, R, local, m, Hq, Hkv, t[1], cfg)
        if t[0] == "copy":
            c = t[2]
            assert d[:7] == [1, c.chunk, c.piece, c.row0, c.row1, c.slab, t[3]]
        else:
            assert d[:6] == [7, t[2], t[3], len(t[5]), t[6], t[7]]
    assert ocg.plan_task(ocg.OP_AG_ATTENTION, R, local, m, Hq, Hkv, len(want), cfg)[0] == 0


def test_attention_plan_defaults_and_validation():
    # the 16K-context GQA share: one flag per chunk, 256-token (512 KiB) copy
    # tasks, 256 tiles (one per CU), 128 copy tickets
    p = ocg.plan_info(ocg.OP_AG_ATTENTION, 8, 0, 2048, 32, 8)
    assert (p["slab_rows"], p["copy_rows"], p["n_tiles"], p["n_copy_or_strips"]) == (2048, 256, 256, 128)
    lib = ocg.lib
    assert lib.ocg_workspace_bytes(None, ocg.OP_AG_ATTENTION, 8, 2048, 32, 8, 0, 0) > 256
    assert lib.ocg_workspace_bytes(None, ocg.OP_AG_ATTENTION, 8, 2048, 30, 8, 0, 0) == 0   # Hq % Hkv
    assert lib.ocg_workspace_bytes(None, ocg.OP_AG_ATTENTION, 17, 2048, 32, 8, 0, 0) == 0  # R > 16
    assert lib.ocg_workspace_bytes(None, ocg.OP_AG_ATTENTION, 8, 0, 32, 8, 0, 0) == 0      # m < 1
    with pytest.raises(ocg.OcgError):
        ocg.plan_info(ocg.OP_AG_ATTENTION, 8, 0, 2048, 32, 8, ocg.default_config(slab_rows=8))
    cfg = ocg.default_config()
    ptrs = (C.c_void_p * 2)()
    assert lib.ocg_ag_attention(None, None, ptrs, ptrs, 2, 0, 64, 4, 1, 128, None, None, None, None, 0,
                                C.byref(cfg), None) == ocg.ERR_INVALID_ARG
