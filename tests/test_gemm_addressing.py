"""Host-side replay of the per-tile FP8 GEMM's buffer addressing (CPU).

gemm_fp8_kernel (csrc/gemm_fp8.hip) loads its operands and scales with raw
buffer loads: a VGPR offset that the hardware range-checks against the
resource's size (per dword for multi-dword loads) and a scalar offset that it
does not check.  A partial last K stage ("Why grind FP8 GEMM on CDNA4",
section 5.3: edge tiles must not read past the matrix) is where an unchecked
scalar stage offset could reach past the end of an operand or a scale array.

These tests replay, in Python, the offsets the kernel computes for every
load of the edge tiles, apply the range check, and assert that no byte past
the caller's buffers (A: M x K, B: N x K, scales: ceil(rows / 128) x K / 32
floats) is touched, for ragged K.  The replay follows the kernel's launch
order: the prologue loads stages 0 and 1 (checked), full stage s loads the
scales of stage s + 1 and the codes of stage s + 2 (both clamped to the last
stage), and only the last two full stages use the checked forms when a
partial stage exists.  A second run with the checked forms switched off (the
kernel's earlier addressing) must find the overrun, which shows the replay
can see one.
"""
import pytest

OOB = 0x80000000


def _stages(K):
    nkb = K // 32
    nst = (nkb + 3) // 4
    nfull = nkb // 4
    nfast = max(0, nfull - 2) if nfull < nst else nfull
    return nkb, nst, nfull, nfast


def _load_schedule(K, fixed=True):
    """(stage, checked) of every code-load group and every scale load, in order."""
    nkb, nst, nfull, nfast = _stages(K)
    codes = [(0, True), (1, True)]
    scales = [(0, True)]
    for s in range(nfull):
        checked = fixed and s >= nfast
        scales.append((s + 1, checked))
        codes.append((s + 2, checked))
    if not fixed:
        codes = [(st, False) for st, _ in codes]
        scales = [(st, False) for st, _ in scales]
    return codes, scales


def _touch(voff, soff, nbytes, records):
    """Bytes touched by a raw buffer load of nbytes (range check per dword on
    the VGPR offset), relative to the resource base; empty when checked out."""
    out = []
    for j in range(0, nbytes, 4):
        v = (voff + j) & 0xFFFFFFFF
        if v < records:
            out.append(v + soff + 3)
    return out


def max_code_byte(rows, K, fixed=True):
    """Largest byte offset of an operand (rows x K codes) that the direct loads touch."""
    nkb, nst, nfull, nfast = _stages(K)
    last = nst - 1
    codes, _ = _load_schedule(K, fixed)
    tiles = (rows + 127) // 128
    worst = -1
    for t in {0, tiles - 1}:
        r0 = t * 128
        rows_here = min(128, rows - r0)
        records = rows_here * K
        for wave in range(4):
            for lane in range(64):
                drow = 8 * wave + (lane >> 3)
                dchunk = (lane & 7) ^ ((drow >> 1) & 7)
                dma = drow * K + dchunk * 16
                kend = K - dchunk * 16
                for stage, checked in codes:
                    so = min(stage, last) * 128
                    for i in range(4):
                        vo = dma + i * 32 * K
                        if checked and not so < kend:
                            vo = OOB
                        for b in _touch(vo, so, 16, records):
                            worst = max(worst, r0 * K + b)
    return worst


def max_scale_byte(rows, K, fixed=True, tensor=False):
    """Largest byte offset of a scale array that the scale loads touch."""
    nkb, nst, nfull, nfast = _stages(K)
    last = nst - 1
    _, scales = _load_schedule(K, fixed)
    tiles = (rows + 127) // 128
    records = 4 if tensor else tiles * nkb * 4
    worst = -1
    for t in {0, tiles - 1}:
        base_v = 0 if tensor else t * nkb * 4
        for stage, checked in scales:
            so = 0 if tensor else min(stage, last) * 16
            if checked:
                touched = _touch(base_v + so, 0, 16, records)
            else:
                touched = _touch(base_v, so, 16, records)
            worst = max([worst, *touched])
    return worst


RAGGED_K = [32, 64, 96, 128, 160, 288, 4000, 4096]
ROWS = [128, 1000, 4096, 4100]


@pytest.mark.parametrize("K", RAGGED_K)
@pytest.mark.parametrize("rows", ROWS)
def test_code_loads_stay_inside_operand(rows, K):
    assert max_code_byte(rows, K) < rows * K


@pytest.mark.parametrize("K", RAGGED_K)
@pytest.mark.parametrize("rows", ROWS)
def test_scale_loads_stay_inside_scale_array(rows, K):
    nscale_bytes = ((rows + 127) // 128) * (K // 32) * 4
    assert max_scale_byte(rows, K) < nscale_bytes
    assert max_scale_byte(rows, K, tensor=True) < 4


@pytest.mark.parametrize("K", [160, 288, 4000])
def test_replay_finds_the_unchecked_overrun(K):
    # the earlier addressing (stage offset unchecked in every stage) reads past
    # the last row of the operand and past the scale array when K is ragged
    # and the partial stage is not the first (with one stage, K = 96, the
    # stage offset is zero and the range check alone keeps the loads inside)
    rows = 1000
    assert max_code_byte(rows, K, fixed=False) >= rows * K
    if (K // 32) % 4:
        assert max_scale_byte(rows, K, fixed=False) >= ((rows + 127) // 128) * (K // 32) * 4


# ---------------------------------------------------------------- large tiles
# gemm_fp8_big_kernel (csrc/gemm_fp8_big.hip): 256-row operand bands, 8 waves;
# load j (0..7) of wave w covers rows 64 (j / 2) + 8 w + lane / 8 of A (even j)
# or B (odd j).  Stage 0 is loaded (checked) before the loop; full stage s loads
# the codes and scales of stage s + 1 (clamped to the last stage), checked in
# the last full stage when a partial stage follows.
def _big_schedule(K, fixed=True):
    nkb, nst, nfull, _ = _stages(K)
    nfast = nfull - 1 if nfull < nst else nfull
    loads = [(0, True)] + [(s + 1, fixed and s >= nfast) for s in range(nfull)]
    if not fixed:
        loads = [(st, False) for st, _ in loads]
    return loads


def max_code_byte_big(rows, K, fixed=True):
    nkb, nst, _, _ = _stages(K)
    last = nst - 1
    tiles = (rows + 255) // 256
    worst = -1
    for t in {0, tiles - 1}:
        r0 = t * 256
        records = min(256, rows - r0) * K
        for wave in range(8):
            for lane in range(64):
                drow = 8 * wave + (lane >> 3)
                dchunk = (lane & 7) ^ ((drow >> 1) & 7)
                dma = drow * K + dchunk * 16
                kend = K - dchunk * 16
                for stage, checked in _big_schedule(K, fixed):
                    so = min(stage, last) * 128
                    for i in range(4):
                        vo = dma + i * 64 * K
                        if checked and not so < kend:
                            vo |= OOB
                        for b in _touch(vo, so, 16, records):
                            worst = max(worst, r0 * K + b)
    return worst


def max_scale_byte_big(rows, K, fixed=True):
    nkb, nst, _, _ = _stages(K)
    last = nst - 1
    st_rows = (rows + 127) // 128
    records = st_rows * nkb * 4
    worst = -1
    for t in {0, (rows + 255) // 256 - 1}:
        for half in (0, 1):
            so_a = (2 * t + half) * nkb * 4
            for stage, checked in _big_schedule(K, fixed):
                so = min(stage, last) * 16
                if checked:
                    touched = _touch(so_a + so, 0, 16, records)
                else:
                    touched = _touch(so_a, so, 16, records)
                worst = max([worst, *touched])
    return worst


@pytest.mark.parametrize("K", RAGGED_K)
@pytest.mark.parametrize("rows", ROWS)
def test_big_tile_code_loads_stay_inside_operand(rows, K):
    assert max_code_byte_big(rows, K) < rows * K


@pytest.mark.parametrize("K", RAGGED_K)
@pytest.mark.parametrize("rows", ROWS)
def test_big_tile_scale_loads_stay_inside_scale_array(rows, K):
    assert max_scale_byte_big(rows, K) < ((rows + 127) // 128) * (K // 32) * 4


@pytest.mark.parametrize("K", [160, 288, 4000])
def test_big_tile_replay_finds_the_unchecked_overrun(K):
    rows = 1000
    assert max_code_byte_big(rows, K, fixed=False) >= rows * K


# ------------------------------------------------- MXFP4 large tiles: scales
# gemm_mxfp4_big_kernel (csrc/gemm_mxfp4.hip) stages the E8M0 scales through
# LDS.  SUB scale blocks per 32 K values (1: MXFP4, 2: blocks of 16); a stage
# is 256 K values, 8 SUB scale bytes per row, and a period of 4 / SUB stages
# is 32 bytes of each of the tile's 256 A rows and 256 B rows.  Wave w (0..3)
# issues load q (0..3) of a period as one 16-byte-per-lane direct load: lane
# l brings bytes 16 (l / 32) .. + 15 of the period's 32 bytes of row
# 128 (w % 2) + 32 q + l % 32 of A (w < 2) or B, range-checked against the
# scale array (rows * K SUB / 32 bytes), into LDS buffer (period % 2) at
# (period % 2) * 16384 + (4 w + q) * 1024 + 16 l.  A lane (frag_row r) of
# wave (wm, wn) reads the 8 SUB bytes of stage s of A tile t at
# stage_off(s) + (4 wm + t) * 1024 + 16 r, and of B tile t at the same place
# with load index 8 + 4 wn + t, where stage_off(s) is
# (s / 4 % 2) * 16384 + (s / 2 % 2) * 512 + (s % 2) * 8 (SUB 1) or
# (s / 2 % 2) * 16384 + (s % 2) * 512 (SUB 2).  With SUB 4 (blocks of 8) a
# stage is a period and each K step ks reads only the 4 bytes of the lane's
# half h (blocks 8 ks + 4 h .. + 3): at
# (s % 2) * 16384 + (ks / 2) * 512 + (ks % 2) * 8 + 4 h + tile offset + 16 r.
def _mx_stage_off(s, sub):
    if sub == 1:
        return ((s >> 2) & 1) * 16384 + ((s >> 1) & 1) * 512 + (s & 1) * 8
    return ((s >> 1) & 1) * 16384 + (s & 1) * 512


def _mx_step_off(s, ks, h):
    return (s & 1) * 16384 + (ks >> 1) * 512 + (ks & 1) * 8 + 4 * h


def _mx_scale_dma(scales, rows, nsb, r0, wave, q, period, lastp):
    """The 1 KB one direct load writes: {lds offset: byte}."""
    records = rows * nsb
    out = {}
    for lane in range(64):
        row = r0 + 128 * (wave & 1) + 32 * q + (lane & 31)
        vo = row * nsb + (lane >> 5) * 16 + min(period, lastp) * 32
        for j in range(16):
            v = vo + j
            # per-dword range check: a dword wholly inside reads, else zero
            d0 = v - (v % 4)
            out[(period & 1) * 16384 + (4 * wave + q) * 1024 + 16 * lane + j] = \
                scales[v] if d0 + 4 <= records else 0
    return out


def _mx_scale_replay(M, N, K, tm, tn, sub=1, read_off=_mx_stage_off, step_off=_mx_step_off):
    """Replay the staging and the reads of tile (tm, tn); return the number of
    (lane, stage, tile) reads (SUB 4: lane, K step, tile) whose bytes differ
    from the rows' scales."""
    import numpy as np
    rng = np.random.default_rng(M * 7 + N + K)
    nsb = K // 32 * sub
    nst = K // 256
    per = 4 // sub
    lastp = (nst - 1) // per
    sa = rng.integers(0, 256, size=M * nsb, dtype=np.int64)
    sb = rng.integers(0, 256, size=N * nsb, dtype=np.int64)
    m0, n0 = 256 * tm, 256 * tn
    bad = 0
    lds = {}
    for period in range(lastp + 1):
        # a period's loads land in its buffer before its first stage reads
        # them; the next period's go to the other buffer
        for wave in range(4):
            for q in range(4):
                if wave < 2:
                    lds.update(_mx_scale_dma(sa, M, nsb, m0, wave, q, period, lastp))
                else:
                    lds.update(_mx_scale_dma(sb, N, nsb, n0, wave, q, period, lastp))
        for s in range(per * period, min(per * period + per, nst)):
            for wm_or_wn, base_j, arr, rows, r_base in ((0, 0, sa, M, m0), (1, 0, sa, M, m0),
                                                        (0, 8, sb, N, n0), (1, 8, sb, N, n0)):
                for t in range(4):
                    for r in range(32):
                        row = r_base + 128 * wm_or_wn + 32 * t + r
                        if sub == 4:
                            for ks in range(4):
                                for h in range(2):
                                    off = step_off(s, ks, h) + (base_j + 4 * wm_or_wn + t) * 1024 + 16 * r
                                    got = [lds.get(off + i) for i in range(4)]
                                    want = [int(arr[row * nsb + 32 * s + 8 * ks + 4 * h + i])
                                            if row < rows else 0 for i in range(4)]
                                    bad += got != want
                            continue
                        off = read_off(s, sub) + (base_j + 4 * wm_or_wn + t) * 1024 + 16 * r
                        got = [lds.get(off + i) for i in range(8 * sub)]   # None: never written
                        want = [int(arr[row * nsb + 8 * sub * s + i]) if row < rows else 0
                                for i in range(8 * sub)]
                        bad += got != want
    return bad


@pytest.mark.parametrize("sub", [1, 2, 4])
@pytest.mark.parametrize("M,N,K,tm,tn", [
    (512, 512, 1024, 1, 1),      # one full period (two with blocks of 16)
    (2088, 2072, 768, 8, 8),     # partial period, edge tile: rows past M and N read as zero
    (600, 520, 1280, 2, 2),      # a last period of one stage
    (512, 520, 2304, 0, 2),      # several periods and one stage
])
def test_mxfp4_big_scale_staging_delivers_each_rows_bytes(M, N, K, tm, tn, sub):
    assert _mx_scale_replay(M, N, K, tm, tn, sub) == 0


def test_mxfp4_big_scale_replay_finds_a_wrong_read_offset():
    # reading the other 8-byte word of the 16-byte piece must be caught
    assert _mx_scale_replay(512, 512, 1024, 0, 0, 1,
                            lambda s, sub: _mx_stage_off(s, 1) ^ 8) > 0
    # blocks of 16: the other stage's half of the period, or the other buffer
    assert _mx_scale_replay(512, 512, 1024, 0, 0, 2,
                            lambda s, sub: _mx_stage_off(s, 2) ^ 512) > 0
    assert _mx_scale_replay(512, 512, 1024, 0, 0, 2,
                            lambda s, sub: _mx_stage_off(s, 2) ^ 16384) > 0
    # blocks of 8: the other half's dword, or the other buffer
    assert _mx_scale_replay(512, 512, 1024, 0, 0, 4,
                            step_off=lambda s, ks, h: _mx_step_off(s, ks, 1 - h)) > 0
    assert _mx_scale_replay(512, 512, 1024, 0, 0, 4,
                            step_off=lambda s, ks, h: _mx_step_off(s, ks, h) ^ 16384) > 0
