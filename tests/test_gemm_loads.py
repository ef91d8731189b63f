"""Coverage of the grouped GEMM's per-super-block loads into LDS (CPU only).

Every wave of a grouped-GEMM workgroup issues the same global->LDS loads, so
that "chunk c has landed" is a fixed count of outstanding loads. This test
restates, for every tile shape the library instantiates, how gemm.hpp
(GemmShape and the load offsets of gemm_mainloop) maps lanes to bytes:

* headers (d, dmin, scales and mins: 256 bytes per weight group and
  super-block, after the group's 2 KB of quants), moved as 16-byte loads where
  they split evenly over the waves, else as 4-byte loads (16 x 128 tiles);
* the k-step sums of the tile rows (32 bytes per row), as 4-byte pieces
  (8 waves, or 16-row tiles) or 16-byte halves (4-wave 64-row tiles);

and checks that the LDS image is the one the readers assume (group g's header
at g*256, row r's sums at r*32), each byte written from the right source byte,
every header byte and every tile row covered, nothing written past the buffer,
and that the LDS budget gives the workgroups per CU the kernels are sized for.
"""
import pytest

KQ4_BYTES = 144
ROW_GROUP = 16
GROUP_SB_BYTES = ROW_GROUP * KQ4_BYTES   # 2304: one row group x one super-block
GROUP_QS_BYTES = 2048                    # its quants; the 256 header bytes follow
CHUNK_BYTES = 256
RING = 4
LDS_PER_CU = 160 * 1024


def shape(RB, CW, NW, Q8=False):
    """GemmShape<RB, CW, NW, Q8> restated."""
    M, groups = 16 * RB, NW * CW
    abuf, bqbuf, hdrbuf = M * CHUNK_BYTES, groups * 1024, groups * 256
    hdr_b = 16 if hdrbuf % (NW * 1024) == 0 else 4
    hdr_loads = hdrbuf // (NW * 64 * hdr_b)
    xs_narrow = NW == 8 or RB == 1
    xsbuf = 2048 if NW == 8 else (1024 if RB == 1 else 4096)
    dxbuf = NW * 256 if Q8 else 0
    dx_off = RING * abuf + 2 * bqbuf + 2 * hdrbuf + 2 * xsbuf
    sv_off = dx_off + 2 * dxbuf
    lds = sv_off + NW * 64 * 4
    return dict(M=M, groups=groups, NW=NW, CW=CW, RB=RB, hdrbuf=hdrbuf, hdr_b=hdr_b, hdr_loads=hdr_loads,
                xs_narrow=xs_narrow, xsbuf=xsbuf, lds=lds, abuf=abuf, out_ld=16 * groups + 4, sv_off=sv_off)


# (RB, CW, NW, Q8, workgroups per CU the kernel is sized for): the big tiles
# (64 x 512 and 64 x 256, 8 waves) run one per CU, the 16 x 128 small tiles
# four (three with the Q8 row scales); the 4-wave 64 x 256 shape (no launch
# uses it; the template still supports it) is checked too
SHAPES = [(4, 4, 8, False, 1), (4, 2, 8, False, 1), (1, 2, 4, False, 4), (4, 4, 4, False, 1),
          (4, 4, 8, True, 1), (4, 2, 8, True, 1), (1, 2, 4, True, 3), (4, 4, 4, True, 1)]


@pytest.mark.parametrize("RB,CW,NW,Q8,per_cu", SHAPES)
def test_header_loads(RB, CW, NW, Q8, per_cu):
    sh = shape(RB, CW, NW, Q8)
    b, per = sh["hdr_b"], 256 // sh["hdr_b"]
    assert sh["hdr_loads"] >= 1 and sh["hdrbuf"] % (NW * 64 * b) == 0
    nsb = 8
    image = {}
    for wave in range(NW):
        for i in range(sh["hdr_loads"]):
            for lane in range(64):
                f = (wave * sh["hdr_loads"] + i) * 64 + lane         # flat b-byte slot
                src = (f // per) * nsb * GROUP_SB_BYTES + GROUP_QS_BYTES + (f % per) * b   # hoff
                # destination: the wave's base + load i's 64 lanes of b bytes (global->LDS puts lane l at +l*b)
                dst = wave * sh["hdr_loads"] * 64 * b + i * 64 * b + lane * b
                for j in range(b):
                    assert dst + j not in image, "an LDS header byte written twice"
                    image[dst + j] = src + j
    assert sorted(image) == list(range(sh["hdrbuf"])), "headers must fill the buffer exactly"
    for g in range(sh["groups"]):
        for j in range(256):
            # the reader takes group g's header (row n: bytes n*16 .. n*16+15) at g*256 + n*16
            assert image[g * 256 + j] == g * nsb * GROUP_SB_BYTES + GROUP_QS_BYTES + j


@pytest.mark.parametrize("RB,CW,NW,Q8,per_cu", SHAPES)
def test_kstep_sum_loads(RB, CW, NW, Q8, per_cu):
    sh = shape(RB, CW, NW, Q8)
    M, rows_loaded = sh["M"], {}
    for wave in range(NW):
        for lane in range(64):
            if sh["xs_narrow"]:
                r, piece, size = 8 * wave + lane // 8, lane % 8, 4
                dst = wave * 256 + lane * 4
            else:
                r, piece, size = 32 * (wave % 2) + lane // 2, lane % 2, 16
                dst = wave * 1024 + lane * 16
            assert dst + size <= sh["xsbuf"], "k-step sums written past their buffer"
            if dst < 64 * 32:   # the reader's image: row r at r*32 (waves past the first copy write duplicates)
                assert dst == r * 32 + piece * size
                rows_loaded.setdefault(r, 0)
                rows_loaded[r] += size
    for r in range(M):
        assert rows_loaded.get(r) == 32, f"row {r}'s 32 bytes of sums not loaded exactly once"


@pytest.mark.parametrize("RB,CW,NW,Q8,per_cu", SHAPES)
def test_lds_budget(RB, CW, NW, Q8, per_cu):
    sh = shape(RB, CW, NW, Q8)
    assert sh["lds"] * per_cu <= LDS_PER_CU, "the workgroups per CU the kernel is sized for must fit the LDS"
    if per_cu > 1:
        assert sh["lds"] * (per_cu + 1) > LDS_PER_CU, "exactly that many fit (the register budget assumes it)"
    assert sh["abuf"] % (NW * 1024) == 0
    assert sh["M"] * sh["out_ld"] * 4 <= sh["sv_off"], "output staging must fit below the 1/s copies"


def load_schedule(RB, CW, NW, Q8, nld):
    """gemm_mainloop's interleave restated: global->LDS loads placed after each
    MFMA slot of a half (the MFMAs left after the LDS-read group)."""
    k_m = (1 if Q8 else 2) * RB * CW
    k_ds0 = ((1 if Q8 else 2) * RB + CW + 1) // 2
    k_ds = k_ds0 if k_ds0 < k_m else k_m - 1
    slots = k_m - k_ds
    every = 1 if nld > slots else (slots // nld if nld > 0 else slots)
    per = (nld + slots - 1) // slots if nld > slots else 1
    assert slots >= 1 and every >= 1 and per <= 16
    placed = []
    for i in range(slots):
        n = 0
        if nld > 0 and i % every == every - 1:
            first = (i // every) * per
            n = sum(1 for c in range(16) if c < per and first + c < nld)
        placed.append(n)
    return placed


@pytest.mark.parametrize("RB,CW,NW,Q8,per_cu", SHAPES)
def test_load_schedule(RB, CW, NW, Q8, per_cu):
    # the load counts of the main loop's issue groups: HX + A (q == 0), A
    # (q == 2), Bq + A (odd q), none (the last super-block's iterations)
    sh = shape(RB, CW, NW, Q8)
    a_loads = sh["abuf"] // (NW * 1024)
    hx_loads = sh["hdr_loads"] + 1 + (1 if Q8 else 0)
    for nld in (0, hx_loads + a_loads, a_loads, CW + a_loads):
        placed = load_schedule(RB, CW, NW, Q8, nld)
        assert sum(placed) == nld, "every load of the group must be placed once"
        assert max(placed) <= -(-nld // len(placed)), "loads spread evenly over the slots"
