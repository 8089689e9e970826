"""The C ABI on a host without a GPU: the library loads, exports every symbol the header
declares, and rejects bad arguments before touching the HIP runtime."""
import ctypes
import os
import re

import pytest

import fp32_gemm_f32_amd as g
import workloads as wl

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "sgemm_f32.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(sgemm_f32\w*)\s*\(", text)))


def test_exports_every_declared_symbol():
    names = declared_functions()
    assert "sgemm_f32" in names and "sgemm_f32_naive" in names and len(names) >= 8
    lib = ctypes.CDLL(g.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), f"{n} declared in sgemm_f32.h but not exported"


def test_abi_version_and_status_strings():
    assert g.abi_version() == 2
    lib = g.library()
    for code in range(-8, 1):
        s = lib.sgemm_f32_status_string(code).decode()
        assert s and s != "unknown status"
    assert lib.sgemm_f32_status_string(-99).decode() == "unknown status"


def test_variant_table():
    names = g.variant_names()
    assert len(names) == g.library().sgemm_f32_variant_count() >= 2
    assert g.library().sgemm_f32_variant_name(len(names)) is None
    assert g.library().sgemm_f32_variant_name(-1) is None


P = 1 << 20   # a fake, 16-byte aligned "device" address: never dereferenced on these paths


def call(fn, *args):
    return getattr(g.library(), fn)(*args)


@pytest.mark.parametrize("fn", ["sgemm_f32", "sgemm_f32_naive"])
def test_validation_codes(fn):
    ok = (4, 4, 4, P, 4, P + 4096, 4, P + 8192, 4, None)
    def with_(**kw):
        a = list(ok)
        for k, v in kw.items():
            a["M N K A lda B ldb C ldc".split().index(k)] = v
        return call(fn, *a)
    assert with_(M=-1) == -1 and with_(N=-3) == -1 and with_(K=-2) == -1
    assert with_(lda=3) == -2 and with_(ldb=3) == -2 and with_(ldc=3) == -2
    assert with_(lda=0, K=0) == -2            # ld >= max(1, K)
    assert with_(A=None) == -3 and with_(B=None) == -3 and with_(C=None) == -3
    assert with_(A=P + 2) == -3               # not 4-byte aligned
    assert with_(C=P + 4) == -4               # C overlaps A
    assert with_(C=P + 4096 + 60) == -4       # C overlaps the tail of B
    # M == 0 or N == 0: nothing to do, no launch, no pointer needed for empty regions
    assert with_(M=0, A=None, C=None) == 0
    assert with_(N=0, B=None, C=None) == 0


def test_tiled_option_validation():
    args = (4, 4, 4, P, 4, P + 4096, 4, P + 8192, 4)
    assert call("sgemm_f32_tiled", *args, 8, 0, None) == -6
    assert call("sgemm_f32_tiled", *args, 16, 2, None) == -6
    assert call("sgemm_f32_tiled", 0, 4, 4, P, 4, P + 4096, 4, P + 8192, 4, 32, 1, None) == 0


def test_variant_option_validation():
    n = g.library().sgemm_f32_variant_count()
    args = (8, 8, 8, P, 8, P + 4096, 8, P + 8192, 8, None)
    assert call("sgemm_f32_variant", n, *args) == -6
    # validation comes first, for forced variants too
    assert call("sgemm_f32_variant", 0, 8, 8, 8, P + 2, 8, P + 4096, 8, P + 8192, 8, None) == -3
    assert call("sgemm_f32_variant", 0, 8, 8, 8, P, 7, P + 4096, 8, P + 8192, 8, None) == -2
    # a leading dimension too large for 31-bit buffer offsets inside one workgroup's rows
    huge = 1 << 22
    assert call("sgemm_f32_variant", 0, 8, 8, 8, P, huge, P + (1 << 40), 8, P + (1 << 41), 8,
                None) == -7


@pytest.mark.parametrize("shape,expect_tile", [
    ((8192, 8192, 8192), 256),
    ((16384, 16384, 64), None),
    ((1024, 1024, 1024), None),
    ((1023, 1025, 1027), None),
    ((6, 6, 9), None),
])
def test_plan(shape, expect_tile):
    M, N, K = shape
    plan = g.sgemm_f32_plan_describe(M, N, K, P, None, P + (1 << 30), None, P + (1 << 31), None,
                                     num_cus=256)
    tiles = plan["tiles"][0] * plan["tiles"][1]
    info = g.sgemm_f32_variant_info(plan["variant"])
    # one workgroup per tile, or one per CU walking the tiles
    assert plan["grid"] == (min(tiles, 256) if info["persistent"] else tiles)
    assert plan["direct_loads"] == plan["name"].endswith("_dl")
    # the tiles cover C but for the strip's columns, which lie past whole tile columns
    assert plan["tiles"][0] * plan["BM"] >= M
    assert plan["tiles"][1] * plan["BN"] == N - plan["strip_cols"] or (
        plan["strip_cols"] == 0 and plan["tiles"][1] * plan["BN"] >= N)
    if plan["strip_cols"]:
        assert info["strip"] and 1 <= plan["strip_cols"] <= 4
        rows = plan["strip_rows"]
        if rows:
            # spread: every tile column holding some of the strip's rows computes them,
            # each tile a share that one K-group's threads cover
            assert rows * plan["tiles"][1] >= plan["BM"] > (rows - 1) * plan["tiles"][1]
            assert rows * plan["BK"] // 4 <= 64 * plan["waves"][0] * plan["waves"][1]
            assert plan["strip_tiles"] == plan["tiles"][0] * min(
                plan["tiles"][1], -(-plan["BM"] // rows))
        else:
            assert plan["strip_tiles"] == plan["tiles"][0]
    if shape == (1023, 1025, 1027):
        # the ragged workload: 256 whole 64 x 64 tiles and a one-column strip, instead of
        # a 17th column of nearly empty tiles; its rows spread four to a tile
        assert plan["strip_cols"] == 1 and tiles == 256
        assert plan["strip_rows"] == 4 and plan["strip_tiles"] == 256
    if expect_tile:
        assert plan["BM"] == plan["BN"] == expect_tile
    elif M * N >= 1 << 20:
        assert plan["grid"] >= 64   # 1024-class shapes still spread over the chip
    if shape == (16384, 16384, 64):
        assert plan["name"] == "mfma_128x256x32_w2x4_ps"   # C's stores among the MFMAs
    # the request-bytes model: each A panel once per tile column, each B panel per tile row
    tm, tn = plan["tiles"]
    assert plan["tile_request_bytes"] == 4 * (M * K * tn + K * N * tm)


def test_plan_buffer_too_small():
    buf = ctypes.create_string_buffer(8)
    assert g.library().sgemm_f32_plan_describe(64, 64, 64, P, 64, P, 64, P, 64, 256, buf, 8) == -6


def test_regtiled_validation():
    args = (8, 8, 8, P, 8, P + 4096, 8, P + 8192, 8)
    for tm, tn in [(2, 2), (4, 2), (8, 4), (1, 4), (0, 0)]:
        assert call("sgemm_f32_regtiled", *args, tm, tn, None) == -6
    assert call("sgemm_f32_regtiled", -1, 8, 8, P, 8, P + 4096, 8, P + 8192, 8, 4, 4, None) == -1
    assert call("sgemm_f32_regtiled", 8, 8, 8, P, 8, P + 4096, 8, P + 16, 8, 4, 1, None) == -4
    assert call("sgemm_f32_regtiled", 0, 8, 8, P, 8, P + 4096, 8, P + 8192, 8, 8, 8, None) == 0


def test_lds_transpose_validation():
    t = lambda *a: call("sgemm_f32_lds_transpose", *a)
    assert t(-1, 4, P, 4, P + 4096, 4, 32, 0, None) == -1
    assert t(4, 5, P, 4, P + 4096, 4, 32, 0, None) == -2     # ldi < cols
    assert t(5, 4, P, 4, P + 4096, 4, 32, 0, None) == -2     # ldo < rows
    assert t(4, 4, None, 4, P + 4096, 4, 32, 0, None) == -3
    assert t(4, 4, P, 4, P + 8, 4, 32, 0, None) == -4        # out overlaps in
    assert t(4, 4, P, 4, P + 4096, 4, 16, 0, None) == -6
    assert t(4, 4, P, 4, P + 4096, 4, 64, 2, None) == -6
    assert t(0, 4, P, 4, P + 4096, 1, 64, 1, None) == 0


def test_splitk_validation_and_workspace_size():
    lib = g.library()
    args = (64, 48, 4096, P, 4096, P + (1 << 26), 48, P + (1 << 27), 48)
    ws = P + (1 << 28)
    assert lib.sgemm_f32_splitk_workspace_size(64, 48, 4096, 1) == 0
    assert lib.sgemm_f32_splitk_workspace_size(64, 48, 4096, 4) == 4 * 64 * 48 * 4
    assert lib.sgemm_f32_splitk_workspace_size(64, 48, 4096, 33) == 0
    assert lib.sgemm_f32_splitk_workspace_size(0, 48, 4096, 4) == 0
    need = 4 * 64 * 48 * 4
    assert lib.sgemm_f32_splitk(*args, 33, ws, need, None) == -6
    assert lib.sgemm_f32_splitk(*args, -1, ws, need, None) == -6
    assert lib.sgemm_f32_splitk(*args, 4, None, need, None) == -3
    assert lib.sgemm_f32_splitk(*args, 4, ws + 2, need, None) == -3
    assert lib.sgemm_f32_splitk(*args, 4, ws, need - 4, None) == -6
    assert lib.sgemm_f32_splitk(*args, 4, P + 64, need, None) == -4     # overlaps A
    assert lib.sgemm_f32_splitk(*args, 4, P + (1 << 27) - 64, need, None) == -4   # overlaps C
    assert lib.sgemm_f32_splitk(-1, 48, 4096, P, 4096, P + 4096, 48, P + 8192, 48, 4, ws, need,
                                None) == -1
    assert lib.sgemm_f32_splitk(0, 48, 4096, P, 4096, P + 4096, 48, P + 8192, 48, 4, ws, need,
                                None) == 0



def test_streamk_validation():
    lib = g.library()
    n = lib.sgemm_f32_variant_count()
    args = (64, 48, 4096, P, 4096, P + (1 << 26), 48, P + (1 << 27), 48)
    ws = P + (1 << 28)
    assert lib.sgemm_f32_streamk(*args, n, ws, 1 << 20, None) == -6          # no such variant
    without = [i for i in range(n) if i not in g.streamk_variants()]
    assert without
    for i in without:                                                       # no stream-K form
        assert lib.sgemm_f32_streamk(*args, i, ws, 1 << 20, None) == -6
    assert lib.sgemm_f32_streamk(*args, -1, None, 1 << 20, None) == -3
    assert lib.sgemm_f32_streamk(*args, -1, ws + 4, 1 << 20, None) == -3    # not 16-byte aligned
    assert lib.sgemm_f32_streamk(*args, -1, P + 64, 1 << 20, None) == -4    # overlaps A
    sk0 = g.streamk_variants()[0]
    assert lib.sgemm_f32_streamk(*args, sk0, P + (1 << 27) - 64, 1 << 20, None) == -4  # overlaps C
    assert lib.sgemm_f32_streamk(-1, 48, 64, P, 64, P + 4096, 48, P + 8192, 48, -1, ws, 64,
                                 None) == -1
    assert lib.sgemm_f32_streamk(64, 48, 64, P, 63, P + 4096, 48, P + 8192, 48, -1, ws, 64,
                                 None) == -2
    # empty output: nothing to do, before any device query
    assert lib.sgemm_f32_streamk(0, 48, 64, P, 64, P + 4096, 48, P + 8192, 48, -1, ws, 64,
                                 None) == 0


def test_streamk_noalloc_validation():
    """The no-allocation stream-K entry point validates like sgemm_f32_streamk, before any
    HIP call, and reports its fixed scratch size."""
    lib = g.library()
    assert lib.sgemm_f32_streamk_noalloc_scratch_bytes() == 64 << 20
    n = lib.sgemm_f32_variant_count()
    args = (64, 48, 4096, P, 4096, P + (1 << 26), 48, P + (1 << 27), 48)
    assert lib.sgemm_f32_streamk_noalloc(*args, n, None) == -6              # no such variant
    for i in [i for i in range(n) if i not in g.streamk_variants()]:      # no stream-K form
        assert lib.sgemm_f32_streamk_noalloc(*args, i, None) == -6
    assert lib.sgemm_f32_streamk_noalloc(-1, 48, 64, P, 64, P + 4096, 48, P + 8192, 48, -1,
                                         None) == -1
    assert lib.sgemm_f32_streamk_noalloc(64, 48, 64, P, 63, P + 4096, 48, P + 8192, 48, -1,
                                         None) == -2
    assert lib.sgemm_f32_streamk_noalloc(64, 48, 64, 0, 64, P + 4096, 48, P + 8192, 48, -1,
                                         None) == -3
    assert lib.sgemm_f32_streamk_noalloc(64, 48, 64, P, 64, P + 4096, 48, P + 64, 48, -1,
                                         None) == -4                        # C overlaps A
    assert lib.sgemm_f32_streamk_noalloc(0, 48, 64, P, 64, P + 4096, 48, P + 8192, 48, -1,
                                         None) == 0
    assert lib.sgemm_f32_status_string(-8).decode().startswith("the plan's partial tiles")


def test_workspace_queries_validate_leading_dimensions():
    lib = g.library()
    # invalid dimensions or leading dimensions need no workspace (and make no device query)
    assert lib.sgemm_f32_streamk_workspace_size(64, 48, 64, 63, 48, 48, -1) == 0
    assert lib.sgemm_f32_streamk_workspace_size(64, 48, 64, 64, 47, 48, -1) == 0
    assert lib.sgemm_f32_streamk_workspace_size(64, 48, 64, 64, 48, 47, -1) == 0
    assert lib.sgemm_f32_streamk_workspace_size(-1, 48, 64, 64, 48, 48, -1) == 0


def test_plan_describe_validates_leading_dimensions():
    lib = g.library()
    buf = ctypes.create_string_buffer(1024)
    assert lib.sgemm_f32_plan_describe(64, 48, 64, P, 63, P, 48, P, 48, 256, buf, 1024) == -2
    assert lib.sgemm_f32_plan_describe(64, 48, 64, P, 64, P, 47, P, 48, 256, buf, 1024) == -2
    assert lib.sgemm_f32_plan_describe(64, 48, 64, P, 64, P, 48, P, 40, 256, buf, 1024) == -2
    assert lib.sgemm_f32_plan_describe(-1, 48, 64, P, 64, P, 48, P, 48, 256, buf, 1024) == -1
    assert lib.sgemm_f32_plan_describe(64, 48, 64, P, 64, P, 48, P, 48, 256, buf, 1024) >= 0


def _shapes(n, seed):
    import random
    rnd = random.Random(seed)
    out = [(1023, 1025, 1027), (256, 256, 32768), (1, 1, 1), (64, 64, 32), (65, 65, 33),
           (5000, 5000, 1000), (3000, 3000, 3000), (2107, 2107, 100), (1, 4000, 7)]
    out += [(rnd.randint(1, 3000), rnd.randint(1, 3000), rnd.randint(1, 5000)) for _ in range(n)]
    return out


def test_streamk_partition_self_check():
    """The library walks every stream-K range with the kernels' own partition functions:
    each K-panel unit belongs to exactly one range, each range holds at least one unit,
    and every partial slot the fixup reads for a shared tile was written for that tile by
    exactly one segment. Checked over random shapes, every variant and several CU counts."""
    planned = g.streamk_variants()
    seen_sk = seen_dp_and_sk = seen_tiny = 0
    for M, N, K in _shapes(60, 7):
        for v in [-1] + planned:
            for cus in (256, 80, 7, 1):
                d = g.sgemm_f32_streamk_describe(M, N, K, v, cus)
                assert d["partition_ok"], (M, N, K, v, cus, d)
                assert d["G"] >= 1 and d["max_segments"] <= 3, d
                if not d["streamk"]:
                    assert d["workspace_bytes"] == 0 and d["tiles_sk"] == 0
                    continue
                seen_sk += 1
                tiles = d["tiles"]
                assert d["tiles_dp"] + d["tiles_sk"] == tiles
                # plain tiles come in whole rounds of the resident workgroups (G may be
                # lowered afterwards to the shared unit count)
                assert d["tiles_sk"] > 0 and d["tiles_dp"] % cus == 0
                assert d["units"] == d["tiles_sk"] * d["panels"] >= d["G"]
                assert d["panels"] == -(-K // d["BK"])
                assert d["workspace_bytes"] == 2 * d["G"] * d["BM"] * d["BN"] * 4
                assert d["shared_tiles"] <= d["tiles_sk"]
                seen_dp_and_sk += d["tiles_dp"] > 0
                seen_tiny += d["units"] < cus
    assert seen_sk and seen_dp_and_sk and seen_tiny


def test_streamk_plan_choices():
    """The automatic choice shares tiles where the plain grid would leave most CUs idle (a
    few tiles with a long K) and never plans a partly filled second round of plain tiles
    on the ragged shape; it keeps the plain grid where tiles divide evenly."""
    deep = g.sgemm_f32_streamk_describe(256, 256, 32768, -1, 256)
    assert deep["streamk"] and deep["shared_tiles"] > 0
    c3 = g.sgemm_f32_streamk_describe(1023, 1025, 1027, -1, 256)
    assert c3["streamk"] or c3["tiles"] <= c3["G"], c3
    for shape in [(8192, 8192, 8192), (1024, 1024, 1024), (16384, 16384, 64)]:
        d = g.sgemm_f32_streamk_describe(*shape, -1, 256)
        assert not d["streamk"], d
        assert d["name"] == g.sgemm_f32_plan_describe(*shape, num_cus=256)["name"]
    # forced stream-K with a variant whose tiles divide evenly is the plain grid
    rp = g.variant_names().index("mfma_256x256x32_w2x2_rp")
    d = g.sgemm_f32_streamk_describe(8192, 8192, 8192, rp, 256)
    assert not d["streamk"] and d["tiles"] == 1024


def test_variant_info():
    names = g.variant_names()
    planned = g.planned_variants()
    assert names.index("mfma_256x256x32_w2x2_rp") in planned and len(planned) >= 5
    for i, name in enumerate(names):
        info = g.sgemm_f32_variant_info(i)
        assert info["name"] == name and info["variant"] == i
        assert info["mfma"] in ("32x32x2", "16x16x4")
        assert name.startswith("mfma16_") == (info["mfma"] == "16x16x4")
        w0, w1 = info["waves"]
        assert info["threads"] == 64 * w0 * w1 * info["k_groups"]
        assert info["kernel"] in ("mfma", "regpanel", "persist")
        # planned variants have a stream-K form, except the persistent one (one workgroup
        # per CU already balances its tiles)
        assert info["persistent"] == (info["kernel"] == "persist")
        assert info["whole_tiles"] == info["persistent"]
        if info["persistent"]:
            assert not info["streamk"] and not info["splitk"]
        else:
            assert info["streamk"] == info["planned"]
        assert info["direct_loads"] == name.endswith("_dl")
        assert f"{info['BM']}x{info['BN']}x{info['BK']}" in name
        # three LDS stages only in the template kernel with direct loads, named _s3
        assert info["lds_stages"] == (3 if "_s3_" in name else 2)
        if info["lds_stages"] == 3:
            assert info["kernel"] == "mfma" and info["direct_loads"]
    with pytest.raises(g.SgemmError):
        g.sgemm_f32_variant_info(len(names))
    buf = ctypes.create_string_buffer(8)
    assert g.library().sgemm_f32_variant_info(0, buf, 8) == -6


def test_one_hip_runtime_in_the_process():
    """Loading the library first must not leave two HIP runtimes in the process: torch
    carries its own under the system one's soname, and a second runtime sees no device.
    In a fresh interpreter: load the library, then import torch, and count the distinct
    libamdhip64 files mapped."""
    import subprocess, sys
    code = (
        "import fp32_gemm_f32_amd as g; g.library(); import torch;"
        "paths = {l.split()[-1] for l in open('/proc/self/maps') if 'libamdhip64' in l};"
        "print(len(paths), sorted(paths))")
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True,
                       cwd=ROOT, timeout=300)
    assert r.returncode == 0, r.stderr[-2000:]
    n = int(r.stdout.split()[0])
    assert n == 1, r.stdout



# The plan's choices for the named workloads on 256 compute units (the kernels each
# committed profile under profiles/ was taken on). A change to the cost model that moves
# one of them needs new measurements.
WORKLOAD_PLANS = {
    "c1": ("mfma_32x32x16_w1x1_kg8_s3_dl", 0),
    "c2": ("mfma_64x64x32_w2x1_kg2_dl", 0),
    "c3": ("mfma16_64x64x64_w2x2_kg2_dl", 1),
    "c4": ("mfma_256x256x32_w2x2_rp", 0),
    "c5": ("mfma_128x256x32_w2x4_ps", 0),
    "sk": ("mfma_32x32x16_w1x1_kg8_s3_dl", 0),
    "rk": ("mfma16_80x64x32_w1x2_kg2_dl", 0),
}


@pytest.mark.parametrize("name", sorted(WORKLOAD_PLANS))
def test_workload_plans(name):
    w = wl.WORKLOADS[name]
    plan = g.sgemm_f32_plan_describe(w.M, w.N, w.K, num_cus=256)
    assert (plan["name"], plan["strip_cols"]) == WORKLOAD_PLANS[name], plan


def test_workload_streamk_plans():
    """Stream-K shares tiles where it pays (the under-filled 256 x 256 x 32768) and keeps
    the plain grid on the ragged shapes, where the strip or the plain 80 x 64 grid wins."""
    sk = wl.WORKLOADS["sk"]
    d = g.sgemm_f32_streamk_describe(sk.M, sk.N, sk.K, num_cus=256)
    assert d["streamk"] and d["name"] == "mfma16_64x64x64_w2x2_kg2_dl", d
    assert d["streamk_cost_us"] < d["plain_cost_us"]
    for name in ("c3", "rk"):
        w = wl.WORKLOADS[name]
        d = g.sgemm_f32_streamk_describe(w.M, w.N, w.K, num_cus=256)
        assert not d["streamk"], d


def test_variant_describe_wide_strips():
    """Two to four strip columns: every strip-capable variant takes up to its
    strip_cols_max of them, always in the spread form (the last-column form computes one
    column only), where that form's rows fit a K-group; wider remainders, and remainders
    past the variant's width, mask a last tile column instead. The plan gives the
    1024-class products with N = 1026..1028 a spread strip."""
    cus = 256
    widths = set()
    for v in range(len(g.variant_names())):
        info = g.sgemm_f32_variant_info(v)
        if not info["strip"]:
            assert info["strip_cols_max"] == 0, info
            continue
        bm, bn, bk = info["BM"], info["BN"], info["BK"]
        nt = 64 * info["waves"][0] * info["waves"][1]
        scm = info["strip_cols_max"]
        assert scm in (1, 2, 4), info
        widths.add(scm)
        rows = -(-bm // 16)
        for sc in range(2, 6):
            M, N, K = 16 * bm - 3, 16 * bn + sc, 33
            d = g.sgemm_f32_variant_describe(v, M, N, K, K + 1, N + 3, N + 2, num_cus=cus)
            if sc <= scm and rows * bk // 4 <= nt:
                assert d["strip_cols"] == sc and d["strip_rows"] == rows, (info["name"], sc, d)
                assert d["tiles"][1] == 16, d
            else:
                assert d["strip_cols"] == 0 and d["tiles"][1] == 17, (info["name"], sc, d)
    assert widths >= {2, 4}, widths
    for (M, N, K) in [(1024, 1026, 1024), (1024, 1027, 1024), (1024, 1028, 1024),
                      (1023, 1027, 1027)]:
        d = g.sgemm_f32_plan_describe(M, N, K, num_cus=cus)
        assert d["strip_cols"] == N % d["BN"] and d["strip_rows"] > 0, d
        assert d["tiles"][1] == N // d["BN"], d


def test_variant_describe_row_strips():
    """One to four rows of M past the last whole tile row: every strip-capable variant takes
    up to its strip_cols_max of them as a row strip (each tile row computing a share of its
    tile column's columns) where that share's threads fit a K-group and the strip saves a
    round of tiles; never together with a column strip. The plan gives 1025..1028 x 1024 x
    1024 a row strip and keeps 1029 off it."""
    cus = 256
    for v in range(len(g.variant_names())):
        info = g.sgemm_f32_variant_info(v)
        if not info["strip"]:
            continue
        bm, bn, bk = info["BM"], info["BN"], info["BK"]
        nt = 64 * info["waves"][0] * info["waves"][1]
        cols = -(-bn // 16)
        for rr in range(1, 6):
            M, N, K = 16 * bm + rr, 16 * bn - 3, 33
            d = g.sgemm_f32_variant_describe(v, M, N, K, K + 3, N + 1, N + 2, num_cus=cus)
            if rr <= info["strip_cols_max"] and cols * bk // 4 <= nt:
                assert d["row_strip"] == rr and d["row_strip_cols"] == cols, (info["name"], d)
                assert d["tiles"] == [16, 16] and d["strip_cols"] == 0, d
            else:
                assert d["row_strip"] == 0 and d["tiles"][0] == 17, (info["name"], rr, d)
    for M in (1025, 1026, 1027, 1028):
        d = g.sgemm_f32_plan_describe(M, 1024, 1024, num_cus=cus)
        assert d["row_strip"] == M - 1024 and d["tiles"][0] == 16 and d["strip_cols"] == 0, d
    d = g.sgemm_f32_plan_describe(1029, 1024, 1024, num_cus=cus)
    assert d["row_strip"] == 0, d


def test_variant_describe_strip_forms():
    """A forced variant's plan, as sgemm_f32_variant runs it: the column strip spread over
    the tiles of each row where one K-group's threads cover a tile's share of the rows,
    else computed by the last tile column; no strip where the masked tile column costs no
    extra round. variant -1 describes the plan's own choice."""
    cus = 256
    for v in range(len(g.variant_names())):
        info = g.sgemm_f32_variant_info(v)
        if not info["strip"]:
            continue
        bm, bn, bk = info["BM"], info["BN"], info["BK"]
        nt = 64 * info["waves"][0] * info["waves"][1]
        for (M, N, K, tn) in [(16 * bm - 3, 16 * bn + 1, 33, 16), (15 * bm, 17 * bn + 1, 72, 17),
                              (cus * bm - 5, bn + 1, 40, 1)]:
            d = g.sgemm_f32_variant_describe(v, M, N, K, K + 1, N + 3, N + 2, num_cus=cus)
            assert d["variant"] == v and d["strip_cols"] == 1, (info["name"], d)
            rows = -(-bm // tn)
            if rows * bk // 4 <= nt:
                assert d["strip_rows"] == rows, (info["name"], d)
                assert d["strip_tiles"] == d["tiles"][0] * min(tn, -(-bm // rows))
            else:
                assert d["strip_rows"] == 0 and d["strip_tiles"] == d["tiles"][0], d
        # a handful of tiles: the masked column costs no extra round, so no strip
        d = g.sgemm_f32_variant_describe(v, 63, 5 * bn + 1, 33, num_cus=cus)
        assert d["strip_cols"] == 0 and d["tiles"][1] == 6, d
    for (M, N, K) in [(1023, 1025, 1027), (8192, 8192, 8192), (6, 6, 9)]:
        assert (g.sgemm_f32_variant_describe(-1, M, N, K, num_cus=cus) ==
                g.sgemm_f32_plan_describe(M, N, K, num_cus=cus))
    with pytest.raises(g.SgemmError):
        g.sgemm_f32_variant_describe(len(g.variant_names()), 64, 64, 64, num_cus=cus)
    with pytest.raises(g.SgemmError):
        g.sgemm_f32_variant_describe(0, 64, 64, 64, 63, 64, 64, num_cus=cus)


def test_persistent_plan_edges():
    """The plan runs the persistent variant on the whole tiles of a ragged product and its
    right and bottom edges as launches of their own, where that prices lowest; it keeps the
    variant off rows of C that do not start on 32-byte boundaries and prices its panels
    whole."""
    ps = "mfma_128x256x32_w2x4_ps"
    d = g.sgemm_f32_plan_describe(16383, 16384, 64, num_cus=256)
    assert (d["name"], d["edge_launches"], d["tiles"], d["grid"]) == (ps, 1, [127, 64], 256), d
    d = g.sgemm_f32_plan_describe(8200, 8200, 128, num_cus=256)
    assert (d["name"], d["edge_launches"], d["tiles"]) == (ps, 2, [64, 32]), d
    d = g.sgemm_f32_plan_describe(16384, 16384, 64, num_cus=256)
    assert (d["name"], d["edge_launches"]) == (ps, 0), d
    for ldc in (16385, 16388):
        assert g.sgemm_f32_plan_describe(16384, 16384, 64, ldc=ldc, num_cus=256)["name"] != ps
    assert g.sgemm_f32_plan_describe(16384, 16384, 64, ldc=16392, num_cus=256)["name"] == ps
    assert g.sgemm_f32_plan_describe(16384, 16385, 64, num_cus=256)["name"] != ps
    # K = 65 would run three whole 32-deep panels
    assert g.sgemm_f32_plan_describe(16384, 16384, 65, num_cus=256)["name"] != ps
    # forced on a product without a whole tile the variant leaves it all to the plan
    v = g.variant_names().index(ps)
    d = g.sgemm_f32_variant_describe(v, 100, 200, 64, num_cus=256)
    assert d["name"] != ps and d["edge_launches"] == 0, d
    d = g.sgemm_f32_variant_describe(v, 300, 600, 64, num_cus=256)
    assert (d["name"], d["edge_launches"], d["tiles"]) == (ps, 2, [2, 2]), d
