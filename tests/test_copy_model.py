"""CPU model of how the pipelined kernel copies k-tiles into LDS (no GPU).

The model restates, in numpy, the index arithmetic of the copy path in
csrc/gemm_kernels.hpp: which row and 16-byte chunk each lane of each copy instruction
fetches, the XOR swizzle that places it, the buffer resource (start and size) of every
k-tile, the leading partial k-tile, and the misaligned-operand mode (staging 7) with its
shifted windows.  It then runs every copy of every workgroup and k-tile against an
emulated operand and checks:

  * no dword that a copy fetches lies outside the operand (the buffer resource returns
    zero past its size, dword by dword; a fetched dword must not touch memory before or
    after the matrix, which may be unmapped);
  * every lane that carries a valid element has its whole 16 bytes inside the resource
    (so no valid element is lost whether the hardware range-checks per dword or per
    access);
  * after the realignment of staging 7, every valid element lands at its logical
    position, and every element at k < 0 (the partial k-tile) is exactly zero in both
    operands, so out-of-range products are 0 * x = 0 (the masked loads of the Triton
    lecture notes' matmul, other = 0).

It also checks the swizzles: each is a permutation of a row's chunks, and the operand
fragment reads of both MFMA shapes hit every LDS bank once per group of lanes that the
LDS serves together (64 banks of 4 bytes: 16 lanes of a 16-byte read, 32 lanes of an
8-byte transposing read).
"""

import numpy as np
import pytest

BK = 64
OOB = 0x80000000


# ---------------------------------------------------------------------------
# the swizzles (restated)
# ---------------------------------------------------------------------------

def kswz(r):
    return (r >> 1) & 7


def kswz32(r):
    return ((r >> 1) ^ (r >> 2)) & 3


def nswz(k):
    return ((0xAC60 >> ((k & 3) * 4)) & 15) ^ ((k >> 2) & 2)


def test_swizzles_are_permutations():
    r = np.arange(512)
    for row in range(512):
        assert sorted(c ^ kswz(row) for c in range(8)) == list(range(8))
        assert sorted(c ^ kswz32(row) for c in range(4)) == list(range(4))
        for cpr in (16, 32):
            assert sorted(c ^ nswz(row) for c in range(cpr)) == list(range(cpr))
    assert max(nswz(k) for k in range(64)) < 16 and min(kswz(x) for x in r) == 0


def _banks_once(addrs_by_lane, nbytes, group):
    """Each group of `group` lanes touches each of the 64 4-byte banks at most once."""
    for g0 in range(0, 64, group):
        seen = {}
        for lane in range(g0, g0 + group):
            for b in range(0, nbytes, 4):
                a = addrs_by_lane[lane] + b
                bank = (a // 4) % 64
                if bank in seen and seen[bank] != a:
                    return False
                seen[bank] = a
    return True


@pytest.mark.parametrize("mi", [32, 16])
def test_k_contiguous_fragment_reads_are_conflict_free(mi):
    # A (and B stored [N,K]): lane l reads row l % MI of the fragment and the 16-byte
    # chunk of its 8 k values, 2 kk + l / 32 (32x32x16) or 4 kk + l / 16 (16x16x32),
    # physical chunk = logical ^ kswz(row); rows are 128 bytes
    ksteps = BK // (16 if mi == 32 else 32)
    for base_row in (0, 32, 64, 96):
        for kk in range(ksteps):
            addrs = []
            for lane in range(64):
                c = kk * 2 + lane // 32 if mi == 32 else kk * 4 + lane // 16
                r = lane % mi
                addrs.append((base_row + r) * 128 + (c ^ kswz(r)) * 16)
            assert _banks_once(addrs, 16, 16), (mi, base_row, kk)
            # without the swizzle the same reads collide
            plain = [(base_row + lane % mi) * 128 + (kk * 2 + lane // 32 if mi == 32 else
                     kk * 4 + lane // 16) * 16 for lane in range(64)]
            assert not _banks_once(plain, 16, 16)


@pytest.mark.parametrize("mi", [32, 16])
@pytest.mark.parametrize("bn", [128, 256])
def test_kn_transposing_reads_are_conflict_free(mi, bn):
    # B stored [K,N]: ds_read_b64_tr_b16, lane i of a 16-lane group supplies 8 bytes of
    # row kl = (group offset) + (i & 15) / 4 at columns 4 (i % 4) .. +3 of its chunk;
    # physical chunk = logical ^ nswz(kl); rows are 2 BN bytes
    rb = bn * 2
    for wn_col in range(0, bn, 64):
        for kstep in range(BK // (16 if mi == 32 else 32)):
            for h in range(2):
                addrs = []
                for lane in range(64):
                    if mi == 32:
                        kl = (lane >> 5) * 8 + ((lane & 15) >> 2)
                        chunk = wn_col // 8 + ((lane >> 4) & 1) * 2 + ((lane >> 1) & 1)
                    else:
                        kl = (lane >> 4) * 8 + ((lane & 15) >> 2)
                        chunk = wn_col // 8 + ((lane >> 1) & 1)
                    row = kl + kstep * (16 if mi == 32 else 32) + h * 4
                    addrs.append(row * rb + (chunk ^ nswz(kl)) * 16 + (lane & 1) * 8)
                assert _banks_once(addrs, 8, 32), (mi, bn, wn_col, kstep, h)


# ---------------------------------------------------------------------------
# the copies of one workgroup (restated)
# ---------------------------------------------------------------------------

class Tile:
    def __init__(self, bm, bn, nw):
        self.bm, self.bn, self.nw = bm, bn, nw
        self.a_dma = bm * BK * 2 // 1024 // nw
        self.b_dma = bn * BK * 2 // 1024 // nw


def lane_layout_k(d, lane):
    """K-contiguous copy op d: row and logical chunk each lane fetches."""
    cpr = BK // 8
    r = d * (64 // cpr) + lane // cpr
    p = lane % cpr
    return r, p ^ kswz(r)


def lane_layout_n(d, lane, bn):
    """[K,N] copy op d: k row and logical column chunk each lane fetches."""
    cpr = bn // 8
    r = d * (64 // cpr) + lane // cpr
    p = lane % cpr
    return r, p ^ nswz(r)


def shl(vals, s):
    """Elements move up by s (zeros come in), as shl128 by 16 s bits."""
    out = np.zeros(8, dtype=np.int64)
    if s < 8:
        out[s:] = vals[:8 - s]
    return out


def shr(vals, s):
    out = np.zeros(8, dtype=np.int64)
    if s < 8:
        out[:8 - s] = vals[s:]
    return out


def fetch(mem, base, nr, off):
    """The 8 elements a buffer_load_dwordx4 returns at byte `off` (an unsigned 32-bit
    offset: a negative one wraps far past the end) of a resource starting at byte `base`
    with size nr (per-dword range check, zero past nr); also checks that every fetched
    dword lies inside the operand (bytes [0, 2 * mem.size))."""
    out = np.zeros(8, dtype=np.int64)
    off &= 0xFFFFFFFF             # the offset is an unsigned 32-bit VGPR value
    if off >= nr:
        return out, True
    for i in range(4):
        o = off + 4 * i
        if o >= nr:
            continue
        a = base + o
        if a < 0 or a + 4 > 2 * mem.size or a % 2:
            return out, False
        out[2 * i] = mem[a // 2]
        out[2 * i + 1] = mem[a // 2 + 1]
    return out, True


def run_copies(M, N, K, b_nk, tile, mode):
    """Every copy of every workgroup and k-tile; returns the number of lanes checked.
    Elements are emulated as their flat index + 1 (zero means 'read as zero')."""
    unal = mode == 7
    A = np.arange(1, M * K + 1, dtype=np.int64)
    B = np.arange(1, K * N + 1, dtype=np.int64) + 10 ** 9
    nk = (K + BK - 1) // BK
    pad = (BK - K % BK) % BK
    checked = 0
    for m0 in range(0, M, tile.bm):
        for n0 in range(0, N, tile.bn):
            a_rows = min(M - m0, tile.bm)
            a_base, a_bytes = m0 * K * 2, a_rows * K * 2
            if b_nk:
                b_rows = min(N - n0, tile.bn)
                b_base, b_bytes, b_kb = n0 * K * 2, b_rows * K * 2, 2
            else:
                b_base, b_bytes, b_kb = n0 * 2, (K * N - n0) * 2, 2 * N
            for kt in range(nk):
                first = kt == 0
                k0 = kt * BK - pad
                for w in range(tile.nw):
                    # --- A ---
                    for j in range(tile.a_dma):
                        d = w * tile.a_dma + j
                        for lane in range(64):
                            r, c = lane_layout_k(d, lane)
                            kin = c * 8
                            off = r * K * 2 + c * 16
                            if first and kin < pad:
                                off = off + 2 * (pad - kin) if unal and kin + 8 > pad else OOB
                            base = a_base + k0 * 2
                            nr = a_bytes - k0 * 2
                            vals, safe = fetch(A, base, nr, off)
                            assert safe, ("A read outside", M, N, K, m0, kt, d, lane)
                            if unal and first and kin < pad < kin + 8:
                                vals = shl(vals, pad - kin)
                            checked += _check_k_contig(vals, A, M, K, m0 + r, k0 + kin,
                                                       off, nr, "A")
                    # --- B ---
                    for j in range(tile.b_dma):
                        d = w * tile.b_dma + j
                        for lane in range(64):
                            if b_nk:
                                r, c = lane_layout_k(d, lane)
                                kin = c * 8
                                off = r * K * 2 + c * 16
                                if first and kin < pad:
                                    off = off + 2 * (pad - kin) if unal and kin + 8 > pad else OOB
                                vals, safe = fetch(B, b_base + k0 * 2, b_bytes - k0 * 2, off)
                                assert safe, ("B read outside", M, N, K, n0, kt, d, lane)
                                if unal and first and kin < pad < kin + 8:
                                    vals = shl(vals, pad - kin)
                                checked += _check_k_contig(vals, B - 10 ** 9 * 0, N, K, n0 + r,
                                                           k0 + kin, off, b_bytes - k0 * 2, "B")
                            else:
                                r, c = lane_layout_n(d, lane, tile.bn)
                                over = n0 + c * 8 + 8 - N
                                # mode 7: the resource starts 16 bytes early, so that a
                                # window starting up to 7 columns before n0 has an offset >= 0
                                lead = 16 if unal else 0
                                if unal:
                                    off = OOB if over >= 8 else lead + r * N * 2 + c * 16 - 2 * max(over, 0)
                                else:
                                    off = OOB if over > 0 else r * N * 2 + c * 16
                                if first and r < pad:
                                    off = OOB
                                base = b_base - lead + k0 * b_kb
                                nr = b_bytes + lead - k0 * b_kb
                                vals, safe = fetch(B, base, nr, off)
                                assert safe, ("B[K,N] read outside", M, N, K, n0, kt, d, lane)
                                if unal and 0 < over < 8:
                                    vals = shr(vals, over)
                                k = k0 + r
                                valid = [n0 + c * 8 + e < N for e in range(8)]
                                if k < 0:
                                    assert not vals.any(), ("k < 0 not zero", kt, d, lane)
                                    continue
                                if any(valid):
                                    assert off + 16 <= nr, ("valid B[K,N] chunk cut", kt, d, lane)
                                for e in range(8):
                                    if valid[e]:
                                        want = B[k * N + n0 + c * 8 + e]
                                        assert vals[e] == want, ("B[K,N] element", k, n0 + c * 8 + e)
                                checked += 1
    return checked


def _check_k_contig(vals, X, rows, K, row, kstart, off, nr, what):
    """A lane of a K-contiguous operand: its 8 elements are X[row, kstart + e] where
    0 <= k < K and row < rows, zero where k < 0; rows past the end are unconstrained."""
    if row >= rows:
        return 0
    ks = [kstart + e for e in range(8)]
    for e, k in enumerate(ks):
        if k < 0:
            assert vals[e] == 0, (what, "k < 0 not zero", row, k)
    if any(0 <= k < K for k in ks):
        assert off + 16 <= nr, (what, "valid chunk cut by the resource", row, kstart)
    for e, k in enumerate(ks):
        if 0 <= k < K:
            assert vals[e] == X[row * K + k], (what, "element", row, k, vals[e], X[row * K + k])
    return 1


# (M, N, K) shapes: ragged M/N, K with every residue mod 8 and mod 64, K just above 8,
# a single partial k-tile, and N with every residue mod 8
SHAPES_UNAL = [(40, 40, 8), (33, 17, 9), (70, 264, 23), (300, 136, 63), (65, 130, 65),
               (17, 9, 127), (129, 257, 130), (8, 8, 1001), (20, 300, 77), (129, 129, 129),
               (40, 263, 70)]
SHAPES_ALIGNED = [(40, 40, 8), (70, 264, 24), (300, 136, 64), (65, 136, 72), (17, 16, 136)]


@pytest.mark.parametrize("b_nk", [False, True], ids=["kn", "nk"])
@pytest.mark.parametrize("tile", [(256, 256, 8), (256, 128, 4), (128, 128, 4)],
                         ids=["256x256w8", "256x128w4", "128x128w4"])
def test_misaligned_mode_copies(b_nk, tile):
    t = Tile(*tile)
    n = 0
    for (M, N, K) in SHAPES_UNAL:
        if not b_nk and N < 8:
            continue
        n += run_copies(M, N, K, b_nk, t, 7)
    assert n > 0


@pytest.mark.parametrize("b_nk", [False, True], ids=["kn", "nk"])
@pytest.mark.parametrize("tile", [(256, 256, 8), (192, 256, 8), (128, 128, 4), (128, 128, 8)],
                         ids=["256x256w8", "192x256w8", "128x128w4", "128x128w8"])
def test_direct_mode_copies(b_nk, tile):
    # the direct-to-LDS modes: rows 16 bytes apart (K % 8 == 0; N % 8 == 0 for [K,N])
    t = Tile(*tile)
    n = 0
    for (M, N, K) in SHAPES_ALIGNED:
        n += run_copies(M, N, K, b_nk, t, 0)
    assert n > 0


def test_model_catches_a_wrong_window():
    # the model is not vacuous: without the shifted window of staging 7, K = 9 reads
    # before the start of A (k < 0 of row 0) or loses elements
    t = Tile(128, 128, 4)
    with pytest.raises(AssertionError):
        run_copies(33, 17, 9, True, t, 0)


@pytest.mark.parametrize("bn", [128, 256])
def test_copy_placement_matches_the_fragment_reads(bn):
    # a copy op d writes its lanes at LDS bytes d*1024 + 16 lane of the operand's part;
    # the fragment reads look for row r, logical chunk c at r * rowbytes + (c ^ swz(r)) * 16
    for d in range(32):
        for lane in range(64):
            r, c = lane_layout_k(d, lane)
            assert d * 1024 + 16 * lane == r * 128 + (c ^ kswz(r)) * 16
            r, c = lane_layout_n(d, lane, bn)
            assert d * 1024 + 16 * lane == r * (2 * bn) + (c ^ nswz(r)) * 16
