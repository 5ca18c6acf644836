"""GPU parity: the HIP path through the C ABI against the CPU oracle.

Tolerance (the accepted reading of the bound): with s = sqrt(K) max|A| max|B|,
fp32 output: max|C - C_ref| / s <= 1e-4; fp16/bf16 output: the error in excess
of half an output ulp of C_ref, divided by s, <= 4e-3 (the literal err_lit is
reported too).  Every test compares every element of C with the oracle, the
benchmark workloads at full size included (the oracle's OpenMP triple loop does
8192^3 in about 15 s on 16 host cores).
"""

import numpy as np
import pytest

import software_pipelined_tiled_gemm_amd as spg
import workloads as W
from tests import gpu_util as G

pytestmark = pytest.mark.gpu


def _log(msg):
    print(msg, flush=True)


def _variants():
    return [spg.gemm_list_config(i) for i in range(spg.gemm_num_configs())]


# ---------------------------------------------------------------------------
# every compiled configuration, both layouts, both input dtypes, ragged shape
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("in_dtype", [W.F16, W.BF16])
@pytest.mark.parametrize("b_layout", [W.B_KN, W.B_NK])
def test_all_variants_ragged(in_dtype, b_layout):
    # spans several 256-tiles in M and N with ragged edges, and a K tail (K % 64 = 40)
    w = W.custom(520, 648, 616, in_dtype, in_dtype, b_layout, "none", ("uniform", -1.0, 1.0))
    a, b = W.make_inputs(w)
    results = {}
    for cfg in _variants():
        _log(f"variant {cfg} {w.describe()}")
        C, used = G.run(w, a, b, force=cfg)
        got = G.c_values(C, w)
        G.check(w, a, b, got)
        results.setdefault(cfg.mfma, []).append(got)
    # every pipelined configuration with the same MFMA shape keeps the same per-element
    # k order (k-tiles ascending, MFMA steps of 16 or 32 k ascending), so their results
    # must be bitwise identical: a slot reused too early would break this
    assert set(results) == {16, 32}
    for vals in results.values():
        for v in vals[1:]:
            assert np.array_equal(v, vals[0])
    # the wave-specialized ring ran among them: none of its bounded waits gave up
    assert spg.gemm_wait_timeouts(reset=True) == 0


@pytest.mark.parametrize("out_dtype", [W.BF16, W.F32])
def test_relu_every_wave_tile(out_dtype):
    # the epilogue is instantiated per (output type, epilogue, wave tile, MFMA shape): run
    # ReLU on one configuration of every distinct block, wave tile and MFMA shape, ragged
    # in M, N and K
    w = W.custom(520, 648, 616, W.F16, out_dtype, W.B_KN, "relu", ("uniform", -1.0, 1.0))
    a, b = W.make_inputs(w)
    seen = set()
    for cfg in _variants():
        key = (cfg.block_m, cfg.block_n, cfg.wave_m, cfg.wave_n, cfg.mfma)
        if key in seen:
            continue
        seen.add(key)
        _log(f"relu {cfg} {w.describe()}")
        C, _ = G.run(w, a, b, force=cfg)
        got = G.c_values(C, w)
        G.check(w, a, b, got)
        assert np.all(got >= 0) and np.any(got == 0) and np.any(got > 0)


@pytest.mark.parametrize("out_dtype", [W.F16, W.BF16, W.F32])
@pytest.mark.parametrize("epilogue", ["none", "gelu_tanh", "relu"])
def test_output_dtypes_and_epilogue(out_dtype, epilogue):
    for b_layout in (W.B_KN, W.B_NK):
        w = W.custom(384, 392, 320, W.BF16, out_dtype, b_layout, epilogue, ("normal", 0.3))
        a, b = W.make_inputs(w)
        _log(w.describe())
        C, _ = G.run(w, a, b)
        G.check(w, a, b, G.c_values(C, w))


# ---------------------------------------------------------------------------
# small shapes: masks on M, N and K; rows that are not 16 bytes apart run the
# register-staged copy mode 7 of the same MFMA kernel
# ---------------------------------------------------------------------------

SIZES = [1, 2, 3, 7, 8, 15, 16, 17, 31, 33, 63, 64, 65, 127, 129]


def _small_cases():
    r = np.random.Generator(np.random.PCG64(2024))
    cases = set()
    for M in SIZES:
        cases.add((M, int(r.choice(SIZES)), int(r.choice(SIZES))))
    for N in SIZES:
        cases.add((int(r.choice(SIZES)), N, int(r.choice(SIZES))))
    for K in SIZES:
        cases.add((int(r.choice(SIZES)), int(r.choice(SIZES)), K))
    cases.update({(1, 1, 1), (129, 129, 129), (64, 64, 64), (8, 8, 8), (65, 65, 72)})
    return sorted(cases)


@pytest.mark.parametrize("b_layout", [W.B_KN, W.B_NK])
@pytest.mark.parametrize("in_dtype", [W.F16, W.BF16])
def test_small_shapes(b_layout, in_dtype):
    for (M, N, K) in _small_cases():
        for out_dtype, epi in ((in_dtype, "none"), (W.F32, "gelu_tanh"), (in_dtype, "relu")):
            w = W.custom(M, N, K, in_dtype, out_dtype, b_layout, epi)
            a, b = W.make_inputs(w)
            C, cfg = G.run(w, a, b)
            # every shape whose rows hold an 8-element copy window runs the MFMA kernel
            mfma_path = K >= 8 and (b_layout == W.B_NK or N >= 8)
            assert (cfg.block_k == 64) == mfma_path, (M, N, K, cfg)
            aligned_rows = K % 8 == 0 and (b_layout == W.B_NK or N % 8 == 0)
            if mfma_path:
                assert (cfg.staging == 7) != aligned_rows, (M, N, K, cfg)
            G.check(w, a, b, G.c_values(C, w))


def test_empty_and_k_zero():
    import torch
    # M == 0 / N == 0: no-op
    for (M, N) in ((0, 16), (16, 0)):
        w = W.custom(M, N, 32, W.F16, W.F16, W.B_NK)
        a, b = W.make_inputs(w)
        G.run(w, a, b)
    # K == 0: C = epi(0) = 0 everywhere, written over a non-zero fill
    for epi in ("none", "gelu_tanh", "relu"):
        w = W.custom(40, 24, 0, W.BF16, W.F32, W.B_KN, epi)
        a, b = W.make_inputs(w)
        C = G.alloc_c(w, fill=7)
        G.run(w, a, b, C=C)
        assert torch.all(C == 0)


def _offset_copy(bits, elems):
    """A device copy of bits that starts `elems` 2-byte elements into its buffer."""
    import torch
    buf = torch.zeros(bits.size + elems + 8, dtype=torch.int16, device=G.torch_dev())
    buf[elems:elems + bits.size] = G.to_dev(bits).reshape(-1)
    return buf, buf[elems:elems + bits.size]


@pytest.mark.parametrize("b_layout", [W.B_KN, W.B_NK])
@pytest.mark.parametrize("which", ["A", "B", "AB"])
def test_misaligned_pointers_run_the_mfma_path(b_layout, which):
    """A or B starting 2 (or 6) bytes past a 16-byte boundary: gemm_run switches to the
    plan's copy-mode-7 twin (16-byte loads at any 2-byte alignment), same MFMA kernel."""
    import torch
    w = W.custom(300, 520, 200, W.F16, W.F16, b_layout, "gelu_tanh", ("uniform", -1.0, 1.0))
    a, b = W.make_inputs(w)
    _, A = _offset_copy(a, 1 if "A" in which else 0)
    _, B = _offset_copy(b, 3 if "B" in which else 0)
    C = G.alloc_c(w)
    with spg.Gemm(w.M, w.N, w.K, w.in_dtype, w.out_dtype, w.b_layout, w.epilogue) as g:
        used = g.launch_config(A.data_ptr(), B.data_ptr(), C.data_ptr())
        assert used.staging == 7 and used.block_k == 64, used
        assert g.config().staging != 7
        g(A.data_ptr(), B.data_ptr(), C)
    torch.cuda.synchronize()
    G.check(w, a, b, G.c_values(C, w))


@pytest.mark.parametrize("out_dtype", [W.BF16, W.F32])
def test_mfma16_gelu_and_direct_store(out_dtype):
    # the 16x16x32 accumulator layout through the staged epilogue with GELU (all output
    # types) and through the direct store, against the oracle, ragged in M, N and K
    m16 = [c for c in _variants() if c.mfma == 16 and c.staging == 0]
    assert m16
    for c in m16:
        for layout in (W.B_KN, W.B_NK):
            w = W.custom(300, 520, 200, W.BF16, out_dtype, layout, "gelu_tanh", ("uniform", -1.0, 1.0))
            a, b = W.make_inputs(w)
            _log(f"mfma16 {c} {w.describe()}")
            C, _ = G.run(w, a, b, force=c)
            got = G.c_values(C, w)
            G.check(w, a, b, got)
            d = spg.TileConfig.from_dict(dict(c.as_dict(), store=1))
            C2, _ = G.run(w, a, b, force=d)
            assert np.array_equal(G.c_values(C2, w), got)


@pytest.mark.parametrize("out_dtype", [W.BF16, W.F32])
def test_misaligned_output_keeps_the_configuration(out_dtype):
    """C starting 2 (bf16) or 4 (fp32) bytes past a 16-byte boundary: the same
    configuration runs, its epilogue writes elements instead of 16-byte vectors, and
    nothing outside C is touched."""
    import torch
    w = W.custom(100, 72, 64, W.BF16, out_dtype, W.B_KN)
    a, b = W.make_inputs(w)
    A, B = G.to_dev(a), G.to_dev(b)
    if out_dtype == W.F32:
        big = torch.zeros(w.M * w.N + 2, dtype=torch.float32, device=G.torch_dev())
    else:
        big = torch.zeros(w.M * w.N + 2, dtype=torch.int16, device=G.torch_dev())
    C = big[1:1 + w.M * w.N].view(w.M, w.N)
    with spg.Gemm(w.M, w.N, w.K, w.in_dtype, w.out_dtype, w.b_layout) as g:
        assert g.launch_config(A, B, C).as_dict() == g.config().as_dict()
        assert g.config().block_k == 64
        g(A, B, C)
    torch.cuda.synchronize()
    assert float(big[0]) == 0 and float(big[-1]) == 0
    G.check(w, a, b, G.c_values(C, w))


@pytest.mark.parametrize("out_dtype", [W.F16, W.BF16, W.F32])
def test_direct_store_epilogue(out_dtype):
    # the epilogue stored from registers (the ablation of LDS staging): same values as the
    # staged one, masked edges, N % 4 != 0 element stores; fp32 output keeps the staging
    picks = [c for c in _variants() if c.staging == 0 and c.persistent == 0 and c.schedule == 0
             and c.lookahead == 1 and c.swizzle == 1 and c.stages >= 2 and c.mfma == 32
             and (c.block_m, c.block_n, c.wave_m, c.wave_n) in ((256, 256, 128, 64), (128, 128, 64, 64))]
    one_per_tile = {}
    for c in picks:
        one_per_tile.setdefault((c.block_m, c.block_n), c)
    assert len(one_per_tile) == 2
    for base in one_per_tile.values():
        for (M, N, K, epi) in ((300, 520, 200, "gelu_tanh"), (257, 262, 64, "relu"), (512, 512, 128, "none")):
            w = W.custom(M, N, K, W.F16, out_dtype, W.B_NK, epi, ("uniform", -1.0, 1.0))
            a, b = W.make_inputs(w)
            d = spg.TileConfig.from_dict(dict(base.as_dict(), store=1))
            _log(f"direct store {d} {w.describe()}")
            C, used = G.run(w, a, b, force=d)
            assert used.store == 1
            got = G.c_values(C, w)
            G.check(w, a, b, got)
            C2, _ = G.run(w, a, b, force=base)
            assert np.array_equal(G.c_values(C2, w), got)


def test_deterministic_and_untouched_outside():
    import torch
    w = W.custom(300, 200, 256, W.BF16, W.BF16, W.B_KN)
    a, b = W.make_inputs(w)
    A, B = G.to_dev(a), G.to_dev(b)
    big = torch.full((w.M + 2, w.N), 0x5A5A, dtype=torch.int16, device=G.torch_dev())
    C = big[1:-1]
    with spg.Gemm(w.M, w.N, w.K, w.in_dtype, w.out_dtype, w.b_layout) as g:
        g(A, B, C)
        first = C.clone()
        g(A, B, C)
    torch.cuda.synchronize()
    assert torch.equal(first, C)
    assert torch.all(big[0] == 0x5A5A) and torch.all(big[-1] == 0x5A5A)


@pytest.mark.parametrize("case", ["max_k_nk", "max_kn_bytes"])
def test_largest_pipelined_operands(case):
    # the largest operands the pipelined kernel takes (copy resources just inside 2^31
    # bytes), with a leading partial k-tile (K % 64 = 56) and, for [K,N], a ragged N
    # whose columns past N must read as zero
    if case == "max_k_nk":
        w = W.custom(40, 40, (1 << 31) // 512 - 72, W.BF16, W.BF16, W.B_NK)   # K = 4,194,232
    else:
        K = 16376
        N = ((1 << 31) // ((K + 64) * 2)) // 8 * 8                           # 65,312
        w = W.custom(48, N, K, W.BF16, W.BF16, W.B_KN)
    _log(f"{case}: {w.describe()}")
    a, b = W.make_inputs(w)
    C, cfg = G.run(w, a, b)
    assert cfg.block_k == 64, cfg
    res = G.check(w, a, b, G.c_values(C, w))
    _log(f"  err_q={res['err_q']:.3e}")


def _persistent_pair():
    """The persistent configuration and the same tile with one workgroup per tile."""
    pers = [c for c in _variants() if c.persistent]
    assert pers, "no persistent configuration compiled"
    p = pers[0]
    for c in _variants():
        d, e = c.as_dict(), p.as_dict()
        d.pop("persistent"), e.pop("persistent")
        if d == e and not c.persistent:
            return p, c
    raise AssertionError("the persistent tile has no one-tile-per-workgroup twin")


# (M, N, K, layout): more tiles than CUs (some workgroups take two or three tiles),
# ragged M (and N for [N,K]), k-tile counts that are odd, one, and not a multiple of
# the ring depth, and a grid smaller than the CU count
PERSISTENT_SHAPES = [(4100, 4352, 192, W.B_KN), (4100, 4200, 128, W.B_NK),
                     (2056, 8192, 64, W.B_KN), (520, 768, 320, W.B_NK), (300, 256, 64, W.B_KN),
                     (8200, 8192, 64, W.B_NK)]


@pytest.mark.parametrize("shape", PERSISTENT_SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_persistent_matches_oracle_and_twin(shape):
    M, N, K, layout = shape
    pers, twin = _persistent_pair()
    for in_dtype, out_dtype, epi in ((W.BF16, W.BF16, "none"), (W.F16, W.F16, "gelu_tanh"),
                                     (W.BF16, W.F16, "relu")):
        w = W.custom(M, N, K, in_dtype, out_dtype, layout, epi, ("uniform", -1.0, 1.0))
        a, b = W.make_inputs(w)
        _log(f"persistent {pers} {w.describe()}")
        C, used = G.run(w, a, b, force=pers)
        assert used.persistent == 1
        got = G.c_values(C, w)
        G.check(w, a, b, got)
        # the same tile, one workgroup per tile: the same k order, so the same bits
        C2, _ = G.run(w, a, b, force=twin)
        assert np.array_equal(G.c_values(C2, w), got)


def test_persistent_falls_back_where_it_does_not_apply():
    # fp32 output, K % 64 != 0, [K,N] with N % 256 != 0: the persistent tile runs one
    # workgroup per tile, with the same result as its twin
    pers, twin = _persistent_pair()
    for (M, N, K, layout, out) in ((600, 512, 256, W.B_KN, W.F32), (600, 512, 200, W.B_NK, W.BF16),
                                   (600, 520, 256, W.B_KN, W.F16)):
        w = W.custom(M, N, K, W.BF16, out, layout, "gelu_tanh", ("uniform", -1.0, 1.0))
        a, b = W.make_inputs(w)
        _log(f"persistent fallback {w.describe()}")
        C, _ = G.run(w, a, b, force=pers)
        got = G.c_values(C, w)
        G.check(w, a, b, got)
        C2, _ = G.run(w, a, b, force=twin)
        assert np.array_equal(G.c_values(C2, w), got)


@pytest.mark.parametrize("staging", [4, 6], ids=["a_deep", "b_deep"])
def test_deep_ring_every_tail(staging):
    # the A-deep (B-deep) ring runs six k-tiles per iteration and then the rest one by
    # one: every remainder 0..5, fewer k-tiles than one iteration, a leading partial
    # k-tile, both layouts; bitwise equal to the two-deep ring of the same tile, MFMA
    # shape and schedule (same k order) and within tolerance
    deep = [c for c in _variants() if c.staging == staging and c.schedule != 2]
    assert deep, f"no staging-{staging} configuration compiled"
    d = deep[0]
    twin = [c for c in _variants() if c.staging == 0 and (c.block_m, c.block_n, c.block_k, c.stages,
            c.wave_m, c.wave_n, c.lookahead, c.schedule, c.persistent, c.mfma) ==
            (d.block_m, d.block_n, d.block_k, d.stages, d.wave_m, d.wave_n, d.lookahead, d.schedule,
             d.persistent, d.mfma)][0]
    for K in (40, 64, 128, 192, 256, 320, 384, 448, 760, 1024):
        for layout in (W.B_KN, W.B_NK):
            w = W.custom(300, 520, K, W.BF16, W.BF16, layout, "none", ("uniform", -1.0, 1.0))
            a, b = W.make_inputs(w)
            _log(f"staging {staging} K={K} {w.describe()}")
            C, used = G.run(w, a, b, force=d)
            assert used.staging == staging
            got = G.c_values(C, w)
            G.check(w, a, b, got)
            C2, _ = G.run(w, a, b, force=twin)
            assert np.array_equal(G.c_values(C2, w), got)


def test_b_deep_ring_epilogues_and_outputs():
    # the default kernel for B stored [K,N] on large grids: every output type and
    # epilogue on a ragged shape, against the oracle and bitwise against its two-slot twin
    deep = [c for c in _variants() if c.staging == 6 and c.schedule != 2][0]
    twin = [c for c in _variants() if c.staging == 0 and (c.block_m, c.block_n, c.block_k, c.stages,
            c.wave_m, c.wave_n, c.lookahead, c.schedule, c.mfma) ==
            (deep.block_m, deep.block_n, deep.block_k, deep.stages, deep.wave_m, deep.wave_n,
             deep.lookahead, deep.schedule, deep.mfma)][0]
    for in_dtype, out_dtype, epi, K in ((W.BF16, W.F32, "gelu_tanh", 760), (W.F16, W.F16, "relu", 448),
                                        (W.BF16, W.BF16, "gelu_tanh", 1000)):
        w = W.custom(600, 776, K, in_dtype, out_dtype, W.B_KN, epi, ("uniform", -1.0, 1.0))
        a, b = W.make_inputs(w)
        _log(f"b-deep {w.describe()}")
        C, used = G.run(w, a, b, force=deep)
        assert used.staging == 6
        got = G.c_values(C, w)
        G.check(w, a, b, got)
        C2, _ = G.run(w, a, b, force=twin)
        assert np.array_equal(G.c_values(C2, w), got)


def _mode7():
    return [c for c in _variants() if c.staging == 7]


# K residues mod 8 and mod 64, K just above 8 and one partial k-tile; N with residues
# mod 8 (B stored [K,N]); M and N ragged against every tile; last column tiles with
# fewer than 8 columns (263 = 2 x 128 + 7, 517 = 2 x 256 + 5), whose straddling chunk
# is loaded from a window that starts before the tile
MISALIGNED = [(300, 520, 9), (257, 264, 63), (130, 300, 65), (520, 648, 1001), (64, 136, 15),
              (300, 131, 200), (33, 257, 127), (600, 523, 760), (96, 9, 64), (129, 129, 129),
              (300, 263, 200), (300, 517, 100)]


@pytest.mark.parametrize("b_layout", [W.B_KN, W.B_NK])
def test_misaligned_rows_every_mode7_configuration(b_layout):
    """Rows that are not 16 bytes apart, through every compiled copy-mode-7
    configuration, fp16 and bf16, every output type and epilogue, against the oracle."""
    cfgs = _mode7()
    assert len(cfgs) >= 3
    for i, (M, N, K) in enumerate(MISALIGNED):
        in_dtype = (W.F16, W.BF16)[i % 2]
        out_dtype = (W.F16, W.BF16, W.F32)[i % 3]
        epi = ("none", "gelu_tanh", "relu")[i % 3]
        w = W.custom(M, N, K, in_dtype, out_dtype, b_layout, epi, ("uniform", -1.0, 1.0))
        a, b = W.make_inputs(w)
        for c in cfgs:
            _log(f"mode 7 {c} {w.describe()}")
            C, used = G.run(w, a, b, force=c)
            assert used.staging == 7
            G.check(w, a, b, G.c_values(C, w))


def test_mode7_bitwise_equals_its_register_staged_twin():
    """On 16-byte aligned operands copy mode 7 computes exactly what copy mode 1 (the same
    register staging without realignment) does with the same tile: the same k order, so
    the same bits, with and without a partial k-tile, both layouts."""
    for c in _mode7():
        twin = [t for t in _variants() if t.staging == 1 and (t.block_m, t.block_n, t.block_k,
                t.stages, t.wave_m, t.wave_n, t.mfma, t.schedule, t.lookahead) ==
                (c.block_m, c.block_n, c.block_k, c.stages, c.wave_m, c.wave_n, c.mfma,
                 c.schedule, c.lookahead)]
        assert twin, f"no register-staged twin of {c}"
        for layout in (W.B_KN, W.B_NK):
            for K in (200, 512):
                w = W.custom(520, 648, K, W.BF16, W.BF16, layout, "none", ("uniform", -1.0, 1.0))
                a, b = W.make_inputs(w)
                C1, _ = G.run(w, a, b, force=c)
                C2, _ = G.run(w, a, b, force=twin[0])
                assert np.array_equal(G.c_values(C1, w), G.c_values(C2, w)), (c, layout, K)


@pytest.mark.parametrize("shape", [(3000, 5000, 1001, W.F16, W.F32, W.B_NK),
                                   (3000, 3001, 1000, W.BF16, W.BF16, W.B_KN),
                                   (4096, 4096, 4095, W.F16, W.F16, W.B_NK)],
                         ids=["K1001_tn", "N3001_nn", "K4095_tn"])
def test_misaligned_rows_full_size(shape):
    """The K % 8 != 0 neighbour of the masked-tail workload, a [K,N] B with N % 8 != 0,
    and a 4096^2 problem with K = 4095, in the configuration the library picks, every
    element against the oracle."""
    M, N, K, dt, od, layout = shape
    w = W.custom(M, N, K, dt, od, layout, "none", ("uniform", -1.0, 1.0))
    _log(f"full size misaligned rows: {w.describe()}")
    a, b = W.make_inputs(w)
    C, cfg = G.run(w, a, b)
    assert cfg.staging == 7 and cfg.block_k == 64, cfg
    got = G.c_values(C, w)
    del C
    res = G.check(w, a, b, got)
    _log(f"  err_lit={res['err_lit']:.3e} err_q={res['err_q']:.3e}")


def test_autotune_keeps_parity():
    w = W.custom(1024, 768, 512, W.F16, W.F16, W.B_NK)
    a, b = W.make_inputs(w)
    C, cfg = G.run(w, a, b, autotune=True)
    _log(f"autotuned {cfg}")
    assert cfg.block_k == 64 and cfg.stages >= 2
    G.check(w, a, b, G.c_values(C, w))


# ---------------------------------------------------------------------------
# the benchmark workloads at full size, in the configuration the benchmark times
# ---------------------------------------------------------------------------

FULL = ["tn_f16_256", "tn_f16_3000x5000x1000_f32out", "pallas_hopper_example",
        "nn_f16_2048x2048x1024_relu_f32out",
        "tn_f16_4096", "nn_bf16_3072x4096x4096_gelu", "nn_bf16_8192", "nn_f16_8192", "tn_f16_8192"]


@pytest.mark.parametrize("name", FULL)
def test_workload_full_size(name):
    """Every benchmark workload in the configuration the benchmark times, every element of
    C against the oracle."""
    w = W.WORKLOADS[name]
    _log(f"workload {name}: {w.describe()}")
    a, b = W.make_inputs(w)
    C, cfg = G.run(w, a, b)
    _log(f"  config {cfg}")
    got = G.c_values(C, w)
    del C
    res = G.check(w, a, b, got)
    _log(f"  all {w.M * w.N} elements: err_lit={res['err_lit']:.3e} floor={res['floor']:.3e} "
         f"err_q={res['err_q']:.3e}")


@pytest.mark.parametrize("b_layout", [W.B_KN, W.B_NK])
def test_full_size_fp32_output_isolates_the_accumulation(b_layout):
    """bf16 8192^3 (B stored [K,N] or [N,K]) in the tile configuration the benchmark times,
    with an fp32 output: nothing is rounded to 16 bits, so the literal bound (1e-4 for an
    fp32 output) applies to the fp32 accumulation itself, on every element against the
    oracle."""
    w = W.custom(8192, 8192, 8192, W.BF16, W.F32, b_layout, "none", ("uniform", -1.0, 1.0),
                 name=f"{'nn' if b_layout == W.B_KN else 'tn'}_bf16_8192_f32out")
    _log(f"workload {w.name}: {w.describe()}")
    a, b = W.make_inputs(w)
    C, cfg = G.run(w, a, b)
    _log(f"  config {cfg}")
    assert (cfg.block_m, cfg.block_n, cfg.mfma) == (256, 256, 16)
    got = G.c_values(C, w)
    del C
    res = G.check(w, a, b, got)
    _log(f"  all elements: err_lit={res['err_lit']:.3e} err_q={res['err_q']:.3e}")
    assert res["err_lit"] <= 1e-4


@pytest.mark.parametrize("in_dtype", [W.BF16, W.F16])
def test_b_deep_ring_bitwise_at_full_size(in_dtype):
    """The B-deep ring (staging 6), the default for B stored [K,N] on grids of several
    rounds, at 8192^3 in the benchmark's configuration, against its two-slot twin (same
    tile, MFMA shape and schedule, staging 0): the same k order, so C must be bitwise
    equal over all 67M elements.  At this size copies land late and slots turn over 128
    times per tile, which is where a slot refilled too early would show."""
    import torch
    w = W.custom(8192, 8192, 8192, in_dtype, in_dtype, W.B_KN, "none", ("uniform", -1.0, 1.0),
                 name=f"nn_{in_dtype}_8192")
    a, b = W.make_inputs(w)
    with spg.Gemm(w.M, w.N, w.K, w.in_dtype, w.out_dtype, w.b_layout) as g:
        deep = g.config()
    assert deep.staging == 6, deep
    twin = [c for c in _variants() if c.staging == 0 and (c.block_m, c.block_n, c.block_k,
            c.stages, c.wave_m, c.wave_n, c.lookahead, c.schedule, c.mfma) ==
            (deep.block_m, deep.block_n, deep.block_k, deep.stages, deep.wave_m, deep.wave_n,
             deep.lookahead, deep.schedule, deep.mfma)][0]
    twin.group_m, twin.xcd_remap = deep.group_m, deep.xcd_remap
    _log(f"b-deep {deep} against {twin}: {w.describe()}")
    C1, _ = G.run(w, a, b)
    C2, used = G.run(w, a, b, force=twin)
    assert used.staging == 0
    assert torch.equal(C1, C2)


def _ping_pong_and_twin():
    """The ping-pong configuration and its twin: the same B-deep ring, tile and MFMA shape
    under the compiler-placed schedule.  Both give each accumulator its k-steps in the same
    order, so their results are bitwise equal."""
    pp = [c for c in _variants() if c.schedule == 2]
    assert len(pp) == 1 and pp[0].staging == 6 and pp[0].mfma == 16, pp
    pp = pp[0]
    twin = [c for c in _variants() if c.schedule == 1 and c.staging == 6 and
            (c.block_m, c.block_n, c.block_k, c.stages, c.wave_m, c.wave_n, c.mfma) ==
            (pp.block_m, pp.block_n, pp.block_k, pp.stages, pp.wave_m, pp.wave_n, pp.mfma)]
    assert twin, "no compiler-scheduled B-deep twin"
    return pp, twin[0]


def test_ping_pong_every_tail_and_epilogue():
    """The ping-pong schedule (the two waves of each SIMD take turns at a workgroup barrier,
    waves 4..7 one phase behind waves 0..3): fewer k-tiles than the six of one unrolled
    iteration, every remainder, a leading partial k-tile, every output type and epilogue,
    both layouts; within tolerance of the oracle and bitwise equal to its twin."""
    pp, twin = _ping_pong_and_twin()
    cases = [(K, W.BF16, W.BF16, "none") for K in (40, 64, 128, 192, 256, 320, 384, 448, 760, 1024)]
    cases += [(1000, W.F16, W.F32, "gelu_tanh"), (448, W.F16, W.F16, "relu"), (520, W.BF16, W.BF16, "gelu_tanh")]
    for K, in_dtype, out_dtype, epi in cases:
        for layout in (W.B_KN, W.B_NK):
            w = W.custom(300, 520, K, in_dtype, out_dtype, layout, epi, ("uniform", -1.0, 1.0))
            a, b = W.make_inputs(w)
            _log(f"ping-pong K={K} {w.describe()}")
            C, used = G.run(w, a, b, force=pp)
            assert used.schedule == 2
            got = G.c_values(C, w)
            G.check(w, a, b, got)
            C2, _ = G.run(w, a, b, force=twin)
            assert np.array_equal(G.c_values(C2, w), got)


@pytest.mark.parametrize("in_dtype", [W.BF16, W.F16])
def test_ping_pong_bitwise_at_full_size(in_dtype):
    """B stored [N,K] at 8192^3: the heuristic's configuration is the ping-pong schedule;
    its C equals its twin's bit for bit over all 67M elements (128 k-tiles per tile, four
    rounds of tiles, where a turn taken out of order would show)."""
    import torch
    w = W.custom(8192, 8192, 8192, in_dtype, in_dtype, W.B_NK, "none", ("uniform", -1.0, 1.0),
                 name=f"tn_{in_dtype}_8192")
    a, b = W.make_inputs(w)
    pp, twin = _ping_pong_and_twin()
    with spg.Gemm(w.M, w.N, w.K, w.in_dtype, w.out_dtype, w.b_layout) as g:
        planned = g.config()
    assert planned.schedule == 2 and planned.staging == 6, planned
    twin.group_m, twin.xcd_remap = planned.group_m, planned.xcd_remap
    _log(f"ping-pong {planned} against {twin}: {w.describe()}")
    C1, _ = G.run(w, a, b)
    C2, used = G.run(w, a, b, force=twin)
    assert used.schedule == 1
    assert torch.equal(C1, C2)


def test_wave_specialized_ring_reports_no_timeouts():
    """The wave-specialized ring (staging 3) on a ragged multi-tile shape: within
    tolerance of the oracle, and none of its bounded waits gave up (the device word
    that gemm_wait_timeouts reads stays 0)."""
    ws = [c for c in _variants() if c.staging == 3]
    assert ws
    spg.gemm_wait_timeouts(reset=True)
    for layout in (W.B_KN, W.B_NK):
        w = W.custom(1000, 1096, 1000, W.F16, W.F16, layout, "gelu_tanh", ("uniform", -1.0, 1.0))
        a, b = W.make_inputs(w)
        _log(f"wave-specialized {ws[0]} {w.describe()}")
        C, used = G.run(w, a, b, force=ws[0])
        assert used.staging == 3
        G.check(w, a, b, G.c_values(C, w))
    assert spg.gemm_wait_timeouts(reset=True) == 0


@pytest.mark.parametrize("shape", [(1000, 1100, 700), (3072, 4096, 4096)], ids=["ragged", "gelu_workload"])
def test_gemm_run_replays_in_a_hip_graph(shape):
    """gemm_run neither allocates nor synchronizes, so a caller can capture it in a HIP
    graph.  Captured once (torch.cuda.graph) and replayed several times, with eager work
    and synchronizations between the replays, every replay gives the eager result bitwise
    (and the eager result is within tolerance of the oracle on every element)."""
    import torch
    M, N, K = shape
    w = W.custom(M, N, K, W.BF16, W.BF16, W.B_KN, "gelu_tanh", ("uniform", -1.0, 1.0),
                 name="graph_replay")
    _log(f"graph replay: {w.describe()}")
    a, b = W.make_inputs(w)
    A, B = G.to_dev(a), G.to_dev(b)
    C_eager, C_graph = G.alloc_c(w), G.alloc_c(w)
    with spg.Gemm(M, N, K, w.in_dtype, w.out_dtype, w.b_layout, w.epilogue) as g:
        _log(f"  config {g.config()}")
        g(A, B, C_eager)
        torch.cuda.synchronize()
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            g(A, B, C_graph)                 # warm-up launch on a side stream
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            g(A, B, C_graph)                 # gemm_run on the capture stream
        for i in range(4):
            C_graph.fill_(-1)                # eager work between the replays
            torch.cuda.synchronize()
            graph.replay()
            torch.cuda.synchronize()
            assert torch.equal(C_graph, C_eager), f"replay {i}"
        del graph
    G.check(w, a, b, G.c_values(C_eager, w))


def test_one_plan_on_two_streams():
    """A plan is read-only after gemm_create, so one handle may run on several streams at
    once.  Two streams (default priority) run the same plan back to back without any
    synchronization between them: one on 16-byte aligned operands, the other on an A whose
    base address is 2 bytes past a 16-byte boundary (the plan's register-staged twin).
    Every launch gives its problem's single-stream result bitwise, and those results are
    within tolerance of the oracle."""
    import torch
    M, N, K = 1000, 1096, 704
    w = W.custom(M, N, K, W.F16, W.F16, W.B_NK, "none", ("uniform", -1.0, 1.0), name="two_streams")
    a, b = W.make_inputs(w)
    a2, b2 = W.make_inputs(w, seed_a=7, seed_b=8)
    A1, B1 = G.to_dev(a), G.to_dev(b)
    buf = torch.zeros(M * K + 8, dtype=torch.int16, device=G.torch_dev())
    A2 = buf[1:1 + M * K].view(M, K)          # 2-byte aligned only
    A2.copy_(G.to_dev(a2))
    B2 = G.to_dev(b2)
    with spg.Gemm(M, N, K, w.in_dtype, w.out_dtype, w.b_layout, w.epilogue) as g:
        R1, R2 = G.alloc_c(w), G.alloc_c(w)
        assert g.launch_config(A1, B1, R1).staging != 7
        assert g.launch_config(A2, B2, R2).staging == 7
        _log(f"two streams: {g.launch_config(A1, B1, R1)} and {g.launch_config(A2, B2, R2)}")
        g(A1, B1, R1)
        g(A2, B2, R2)
        torch.cuda.synchronize()
        s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
        s1.wait_stream(torch.cuda.current_stream())
        s2.wait_stream(torch.cuda.current_stream())
        C1 = [G.alloc_c(w, -1) for _ in range(4)]
        C2 = [G.alloc_c(w, -1) for _ in range(4)]
        torch.cuda.synchronize()
        for i in range(4):
            g(A1, B1, C1[i], s1)
            g(A2, B2, C2[i], s2)
        torch.cuda.synchronize()
        for i in range(4):
            assert torch.equal(C1[i], R1), f"stream 1, launch {i}"
            assert torch.equal(C2[i], R2), f"stream 2, launch {i}"
    G.check(w, a, b, G.c_values(R1, w))
    G.check(w, a2, b2, G.c_values(R2, w))
