"""The C ABI on a machine without a GPU: the library loads, exports every declared
symbol, validates arguments before any HIP call, and its host-side planning logic
(configuration table, LDS budget, heuristic) behaves as documented.  No kernel runs."""

import ctypes
import glob
import os
import re

import pytest

import software_pipelined_tiled_gemm_amd as spg

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADERS = [os.path.join(ROOT, "include", h) for h in ("spgemm.h", "spgelu.h")]
GOLDEN = os.path.join(ROOT, "tests", "golden")


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(spg.LIB_PATH):
        pytest.fail("libspgemm.so is not built; run __graft_entry__.build()")
    return spg.lib()


def declared_functions():
    names = set()
    for h in HEADERS:
        src = re.sub(r"/\*.*?\*/", "", open(h).read(), flags=re.S)
        names.update(re.findall(r"\b((?:gemm|gelu)_[a-z_]+)\s*\(", src))
    return sorted(names)


def test_every_header_is_listed():
    assert sorted(glob.glob(os.path.join(ROOT, "include", "*.h"))) == sorted(HEADERS)


def test_every_declared_symbol_is_exported(L):
    names = declared_functions()
    assert set(names) == set(spg.EXPORTED)
    for n in names:
        assert hasattr(L, n), n


def test_poison_library_exports_the_same_abi():
    # the race-detecting test build: same entry points, a subset of the configurations,
    # every one of which the production library also holds
    if not os.path.exists(spg.POISON_LIB_PATH):
        pytest.fail("libspgemm_poison.so is not built; run __graft_entry__.build()")
    P = spg.poison_lib()
    for n in declared_functions():
        assert hasattr(P, n), n
    def cfgs(lib):
        out = []
        for i in range(lib.gemm_num_configs()):
            c = spg.TileConfig()
            assert lib.gemm_list_config(i, ctypes.byref(c)) == 0
            out.append(tuple(sorted(c.as_dict().items())))
        return out
    poison, prod = cfgs(P), set(cfgs(spg.lib()))
    assert 0 < len(poison) < len(prod) and set(poison) <= prod


def _plan(lib, M, N, K, dt, lay):
    h = ctypes.c_void_p()
    st = lib.gemm_create(ctypes.byref(h), M, N, K, spg.DTYPES[dt], spg.DTYPES[dt],
                         spg.B_LAYOUTS[lay], spg.EPILOGUES["none"], None)
    assert st == 0, (M, N, K, dt, lay, st)
    c = spg.TileConfig()
    assert lib.gemm_get_config(h, ctypes.byref(c)) == 0
    twin = spg.TileConfig()
    # a pointer that is not 16-byte aligned: the plan's misaligned-operand twin
    assert lib.gemm_launch_config(h, ctypes.c_void_p(2), ctypes.c_void_p(0), ctypes.c_void_p(0),
                                  ctypes.byref(twin)) == 0
    lib.gemm_destroy(h)
    return c.as_dict(), twin.as_dict()


def test_poison_library_plans_what_the_production_library_plans():
    # The poison build compiles a subset of the configurations; the heuristic considers
    # only the ones a library holds, so the poison build tests the production plans only
    # if it holds every configuration the heuristic picks (and every misaligned twin).
    if not os.path.exists(spg.POISON_LIB_PATH):
        pytest.fail("libspgemm_poison.so is not built; run __graft_entry__.build()")
    P, Q = spg.poison_lib(), spg.lib()
    shapes = [(8192, 8192, 8192), (6144, 6144, 6144), (4096, 4096, 4096), (4096, 4096, 1024),
              (3072, 4096, 4096), (3000, 5000, 1000), (3000, 5000, 1001), (1024, 8192, 8192),
              (2048, 2048, 2048), (2048, 2048, 1024), (1024, 2048, 4096), (1024, 1024, 1024),
              (256, 256, 256), (300, 263, 200), (16384, 1024, 1024), (512, 512, 8192), (129, 8, 64)]
    for (M, N, K) in shapes:
        for dt in ("f16", "bf16"):
            for lay in ("kn", "nk"):
                assert _plan(P, M, N, K, dt, lay) == _plan(Q, M, N, K, dt, lay), (M, N, K, dt, lay)


def test_status_strings(L):
    for code, text in spg.STATUS.items():
        assert spg.gemm_status_string(code) == text


def test_invalid_arguments_rejected_without_gpu(L):
    h = ctypes.c_void_p()
    ok = lambda *a: L.gemm_create(ctypes.byref(h), *a, None)
    assert L.gemm_create(None, 8, 8, 8, 0, 0, 0, 0, None) == 1
    assert ok(-1, 8, 8, 0, 0, 0, 0) == 1
    assert ok(8, -1, 8, 0, 0, 0, 0) == 1
    assert ok(8, 8, -1, 0, 0, 0, 0) == 1
    assert ok(8, 8, 8, 2, 0, 0, 0) == 1    # fp32 input is not supported
    assert ok(8, 8, 8, 7, 0, 0, 0) == 1    # unknown input dtype
    assert ok(8, 8, 8, 0, 9, 0, 0) == 1    # unknown output dtype
    assert ok(8, 8, 8, 0, 0, 2, 0) == 1    # unknown layout
    assert ok(8, 8, 8, 0, 0, 0, 5) == 1    # unknown epilogue
    assert ok(1 << 40, 8, 8, 0, 0, 0, 0) == 2
    # the standalone GELU: n < 0, unknown dtype, NULL with n > 0; n == 0 is a no-op
    assert L.gelu_run(None, None, -1, 1, None) == 1
    assert L.gelu_run(None, None, 8, 5, None) == 1
    assert L.gelu_run(None, None, 8, 1, None) == 1
    assert L.gelu_run(None, None, 0, 1, None) == 0
    assert L.gelu_run(None, None, 1 << 40, 1, None) == 1
    assert L.gelu_run(16, 32, 1 << 40, 1, None) == 2    # over the grid limit: no launch
    # NULL handle / pointers
    assert L.gemm_run(None, None, None, None, None) == 1
    assert L.gemm_get_config(None, None) == 1
    assert L.gemm_autotune(None, None, None, None, None, 1, None) == 1
    assert L.gemm_destroy(None) == 0
    assert L.gemm_wait_timeouts(None, 0) == 1


def test_wait_timeouts_without_a_device(L):
    # the device word cannot be read without a GPU: a HIP error, and the count is zeroed
    n = ctypes.c_uint32(7)
    assert L.gemm_wait_timeouts(ctypes.byref(n), 0) == 4
    assert n.value == 0


def test_largest_k_plans_the_simple_kernel(L):
    # K up to INT32_MAX is accepted (the simple kernel walks K with 64-bit indices); one
    # more is unsupported
    h = spg.gemm_create(8, 8, (1 << 31) - 1, "bf16", "f32", "nk")
    assert spg.gemm_get_config(h).block_k == 0
    spg.gemm_destroy(h)
    hh = ctypes.c_void_p()
    assert L.gemm_create(ctypes.byref(hh), 8, 8, 1 << 31, 1, 2, 1, 0, None) == 2


def test_plan_lifecycle_and_pointer_checks(L):
    h = spg.gemm_create(64, 64, 64, "f16", "f16", "nk")
    try:
        cfg = spg.gemm_get_config(h)
        assert cfg.block_k == 64 and cfg.stages >= 2
        # non-empty problem with NULL operands: rejected before any launch
        assert L.gemm_run(h, None, None, None, None) == 1
        assert L.gemm_run(h, None, None, 4096, None) == 1
    finally:
        spg.gemm_destroy(h)
    # an empty problem is a successful no-op even with NULL pointers
    h = spg.gemm_create(0, 64, 64, "f16", "f16", "nk")
    assert L.gemm_run(h, None, None, None, None) == 0
    spg.gemm_destroy(h)


def test_forced_configs(L):
    n = spg.gemm_num_configs()
    assert n >= 8
    for i in range(n):
        c = spg.gemm_list_config(i)
        assert spg.gemm_lds_bytes(c) <= 160 * 1024
        h = spg.gemm_create(1000, 1000, 1000, "bf16", "bf16", "kn", "none", c)
        got = spg.gemm_get_config(h)
        assert got.as_dict()["block_m"] == c.block_m and got.stages == c.stages
        spg.gemm_destroy(h)
    bad = spg.TileConfig(block_m=256, block_n=256, block_k=64, stages=3, wave_m=128,
                         wave_n=128, swizzle=1, group_m=4, xcd_remap=1)
    with pytest.raises(spg.GemmError) as e:   # 192 KiB of LDS: over the 160 KiB budget
        spg.gemm_create(512, 512, 512, force=bad)
    assert e.value.status == 2
    odd = spg.TileConfig(block_m=96, block_n=128, block_k=64, stages=2, wave_m=32, wave_n=64,
                         swizzle=1, group_m=4, xcd_remap=1)
    with pytest.raises(spg.GemmError) as e:
        spg.gemm_create(512, 512, 512, force=odd)
    assert e.value.status == 2
    neg = spg.TileConfig(block_m=128, block_n=128, block_k=64, stages=2, wave_m=64, wave_n=64,
                         swizzle=3, group_m=4, xcd_remap=1)
    with pytest.raises(spg.GemmError) as e:
        spg.gemm_create(512, 512, 512, force=neg)
    assert e.value.status == 1
    sch = spg.TileConfig(block_m=256, block_n=256, block_k=64, stages=2, wave_m=128,
                         wave_n=64, swizzle=1, group_m=4, xcd_remap=1, schedule=3)
    with pytest.raises(spg.GemmError) as e:
        spg.gemm_create(512, 512, 512, force=sch)
    assert e.value.status == 1
    # the ping-pong schedule is compiled for the B-deep ring only
    sch.schedule = 2
    with pytest.raises(spg.GemmError) as e:
        spg.gemm_create(512, 512, 512, force=sch)
    assert e.value.status == 2
    sch.staging, sch.mfma = 6, 16
    h = spg.gemm_create(512, 512, 512, force=sch)
    assert spg.gemm_get_config(h).schedule == 2
    spg.gemm_destroy(h)
    per = spg.TileConfig(block_m=256, block_n=256, block_k=64, stages=2, wave_m=128,
                         wave_n=64, swizzle=1, group_m=4, xcd_remap=1, persistent=2)
    with pytest.raises(spg.GemmError) as e:
        spg.gemm_create(512, 512, 512, force=per)
    assert e.value.status == 1
    assert any(spg.gemm_list_config(i).persistent for i in range(n))
    sto = spg.TileConfig(block_m=256, block_n=256, block_k=64, stages=2, wave_m=128,
                         wave_n=64, swizzle=1, group_m=4, xcd_remap=1, store=2)
    with pytest.raises(spg.GemmError) as e:
        spg.gemm_create(512, 512, 512, force=sto)
    assert e.value.status == 1
    # release delay 1 (staging 5) needs a ring of three slots; the A-deep ring (staging 4)
    # holds one more k-tile of A than the TileLang budget formula counts, the B-deep ring
    # (staging 6) one more of B
    deep = set()
    for i in range(n):
        c = spg.gemm_list_config(i)
        assert c.staging != 5 or c.stages >= 3
        if c.staging == 4:
            assert spg.gemm_lds_bytes(c) == (c.stages * (c.block_m + c.block_n) + c.block_m) * c.block_k * 2
        if c.staging == 6:
            assert spg.gemm_lds_bytes(c) == (c.stages * (c.block_m + c.block_n) + c.block_n) * c.block_k * 2
        if c.staging in (4, 6):
            deep.add(c.staging)
            assert c.stages == 2 and spg.gemm_lds_bytes(c) <= 160 * 1024
    assert deep == {4, 6}
    bad_staging = spg.TileConfig(block_m=256, block_n=256, block_k=64, stages=2, wave_m=128,
                                 wave_n=64, swizzle=1, group_m=4, xcd_remap=1, staging=8)
    with pytest.raises(spg.GemmError) as e:
        spg.gemm_create(512, 512, 512, force=bad_staging)
    assert e.value.status == 1
    for look in (0, 3):
        far = spg.TileConfig(block_m=256, block_n=256, block_k=64, stages=2, wave_m=128,
                             wave_n=128, swizzle=1, group_m=4, xcd_remap=1, lookahead=look)
        with pytest.raises(spg.GemmError) as e:
            spg.gemm_create(512, 512, 512, force=far)
        assert e.value.status == 1


def test_lds_budget_is_the_tilelang_formula(L):
    # stages * (block_M*block_K + block_N*block_K) * elem_bytes, evaluated at the
    # TileLang tutorial's defaults (golden file)
    for line in open(os.path.join(GOLDEN, "tilelang_smem_budget.txt")):
        if line.startswith("#") or not line.strip():
            continue
        bm, bn, bk, eb, st, want = map(int, line.split())
        assert eb == 2
        c = spg.TileConfig(block_m=bm, block_n=bn, block_k=bk, stages=st, wave_m=32, wave_n=32)
        assert spg.gemm_lds_bytes(c) == want


def test_misaligned_rows_plan_the_register_staged_mfma_path(L):
    # K % 8 != 0 (or B stored [K,N] with N % 8 != 0): rows are not 16 bytes apart, so the
    # plan is copy mode 7 (register-staged loads at any 2-byte alignment), block_k 64
    for (M, N, K, layout) in ((100, 100, 77, "nk"), (100, 101, 64, "kn"), (3000, 5000, 1001, "nk"),
                              (100, 100, 9, "kn"), (8, 8, 8, "kn")):
        h = spg.gemm_create(M, N, K, "f16", "f16", layout)
        c = spg.gemm_get_config(h)
        spg.gemm_destroy(h)
        aligned = K % 8 == 0 and (layout == "nk" or N % 8 == 0)
        assert c.block_k == 64 and (c.staging == 7) != aligned, (M, N, K, layout, c)
        # mode 7 runs 32x32x16 MFMAs; the aligned plans are the 8-wave 16x16x32 tiles
        assert c.mfma == (32 if c.staging == 7 else 16)
    h = spg.gemm_create(100, 101, 64, "bf16", "bf16", "nk")   # [N,K] rows are 16-B
    assert spg.gemm_get_config(h).block_k == 64 and spg.gemm_get_config(h).staging != 7
    spg.gemm_destroy(h)
    # K < 8, or N < 8 with B stored [K,N]: no 8-element window fits a row: simple kernel
    for (M, N, K, layout) in ((100, 100, 7, "nk"), (100, 5, 64, "kn"), (3, 3, 1, "kn")):
        h = spg.gemm_create(M, N, K, "f16", "f16", layout)
        assert spg.gemm_get_config(h).block_k == 0, (M, N, K, layout)
        spg.gemm_destroy(h)
    h = spg.gemm_create(100, 5, 64, "f16", "f16", "nk")       # a [N,K] B may have N < 8
    assert spg.gemm_get_config(h).block_k == 64
    spg.gemm_destroy(h)


def test_misaligned_pointers_select_the_twin(L):
    # the launch configuration follows the alignment of A and B (host logic, no launch):
    # 16-byte aligned -> the plan's direct-copy configuration; otherwise its mode-7 twin
    h = spg.gemm_create(4096, 4096, 4096, "bf16", "bf16", "kn")
    base = spg.gemm_get_config(h)
    assert base.staging != 7
    assert spg.gemm_launch_config(h, 1 << 20, 2 << 20, 3 << 20).as_dict() == base.as_dict()
    for a, b in ((2 + (1 << 20), 2 << 20), (1 << 20, 8 + (2 << 20))):
        u = spg.gemm_launch_config(h, a, b, 3 << 20)
        assert u.staging == 7 and u.block_k == 64 and u.group_m == base.group_m
    # C's alignment does not change the configuration (element stores in the epilogue)
    assert spg.gemm_launch_config(h, 1 << 20, 2 << 20, 2 + (3 << 20)).staging == base.staging
    spg.gemm_destroy(h)
    # a plan on the simple kernel reports block_k = 0 whatever the pointers
    h = spg.gemm_create(10, 10, 3, "bf16", "bf16", "kn")
    assert spg.gemm_launch_config(h, 1 << 20, 2 << 20, 3 << 20).block_k == 0
    spg.gemm_destroy(h)
    # forcing a direct-copy configuration onto rows that are not 16 bytes apart is refused
    c = [spg.gemm_list_config(i) for i in range(spg.gemm_num_configs())]
    direct = [x for x in c if x.staging == 0][0]
    with pytest.raises(spg.GemmError) as e:
        spg.gemm_create(512, 512, 500, force=direct)
    assert e.value.status == 2


def test_size_limits_of_the_pipelined_kernel(L):
    # a copy resource (256 rows of A or of a [N,K] B, all of a [K,N] B, plus up to 63 k of
    # the leading partial k-tile) must stay within 2^31 bytes: just inside runs pipelined,
    # just outside plans the simple kernel (block_k = 0)
    def bk(M, N, K, layout):
        h = spg.gemm_create(M, N, K, "bf16", "bf16", layout)
        c = spg.gemm_get_config(h).block_k
        spg.gemm_destroy(h)
        return c
    kmax = (1 << 31) // (256 * 2) - 64          # 4,194,240
    assert bk(40, 40, kmax, "nk") == 64
    assert bk(40, 40, kmax + 8, "nk") == 0
    K = 16376
    nmax = ((1 << 31) // ((K + 64) * 2)) // 8 * 8   # 65,312
    assert bk(48, nmax, K, "kn") == 64
    assert bk(48, nmax + 8, K, "kn") == 0
    assert bk(48, nmax + 8, K, "nk") == 64     # [N,K] B is bounded per 256-row panel


def test_heuristic_tiles(L):
    def cfg(M, N, K):
        h = spg.gemm_create(M, N, K, "bf16", "bf16", "kn")
        c = spg.gemm_get_config(h)
        spg.gemm_destroy(h)
        return c
    big = cfg(8192, 8192, 8192)
    assert (big.block_m, big.block_n, big.wave_m, big.wave_n) == (256, 256, 128, 64)
    # 16x16x32 MFMAs on the 8-wave tiles; B stored [K,N] on a grid of several rounds:
    # the B-deep ring under the compiler's schedule
    assert (big.mfma, big.staging, big.schedule) == (16, 6, 1)
    h = spg.gemm_create(8192, 8192, 8192, "bf16", "bf16", "nk")
    tn = spg.gemm_get_config(h)
    spg.gemm_destroy(h)
    # B stored [N,K] on a grid of several rounds: the same ring under the ping-pong schedule
    assert (tn.block_m, tn.block_n, tn.mfma, tn.staging, tn.schedule) == (256, 256, 16, 6, 2)
    # one round of 256x256 tiles: the two-slot ring, compiler-placed with more than 16
    # k-tiles, hand-placed with fewer
    one_round = cfg(4096, 4096, 4096)
    assert (one_round.staging, one_round.schedule) == (0, 1)
    assert cfg(4096, 4096, 1024).schedule == 0
    assert cfg(1024, 8192, 8192).mfma == 16
    # small problems: 128x128, 8 waves of 32x64, 16x16x32; three slots on grids under
    # two rounds with more than 16 k-tiles or at least half a round of tiles, else two
    small = cfg(256, 256, 256)
    assert (small.block_m, small.block_n, small.wave_m, small.wave_n, small.mfma, small.stages) == \
        (128, 128, 32, 64, 16, 2)
    assert cfg(2048, 2048, 2048).stages == 3      # 256 tiles, 32 k-tiles
    assert cfg(2048, 2048, 1024).stages == 3      # 16 k-tiles, but a full round of tiles
    assert cfg(1024, 1024, 1024).stages == 2      # 64 tiles, 16 k-tiles
    assert cfg(1024, 2048, 4096).stages == 3      # 128 tiles, 64 k-tiles
    # the cost model: rounds of 256 CUs x tile area / per-tile throughput
    shard = cfg(1024, 8192, 8192)           # 128 tiles of 256x256, 256 of 256x128
    assert (shard.block_m, shard.block_n, shard.schedule) == (256, 128, 1)
    gelu = cfg(3072, 4096, 4096)            # 192 tiles of 256x256, 256 of 192x256: one round
    assert (gelu.block_m, gelu.block_n, gelu.wave_m, gelu.mfma) == (192, 256, 96, 16)
    tall = cfg(6144, 8192, 8192)            # 3 rounds of 256x256 against 4 of 192x256
    assert (tall.block_m, tall.block_n) == (256, 256)
    ragged = cfg(3000, 5000, 1000)          # 12 x 20 = 240 tiles of 256x256
    assert (ragged.block_m, ragged.block_n) == (256, 256)
    assert cfg(4096, 4096, 4096).group_m == 4 and big.group_m == 4


def test_every_ablation_row_names_a_compiled_configuration(L):
    import sys
    sys.path.insert(0, ROOT)
    import bench
    for name in ["nn_bf16_8192", *bench.ABLATIONS_BY_WORKLOAD]:
        specs = [s for _, s in bench.ablations_for(name)]
        assert len(set(specs)) == len(specs), name
        for spec in specs:
            bench.parse_tile(spec)   # SystemExit if no compiled configuration matches
