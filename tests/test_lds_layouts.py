"""Host-side checks of the 128-token e4m3fn tile's LDS layout and stage
ring (mixture_experts_moe_amd/csrc/ffn_gemm_mid.hip), replayed in Python:

- every byte the direct-to-LDS loads write (weight load i of wave w: 16
  rows x 64 bytes, lane l -> row l/4, physical slot l%4 holding logical slot
  (l%4) ^ ((row >> 1) & 3); token load i: 8 rows x 128 bytes, lane l -> row
  l/8, slot l%8 holding (l%8) ^ ((row >> 1) & 7)) is the byte the fragment
  reads of the two 32-K steps expect (lane (r16, g): weight bytes
  32j + 8g .. +7 of row r16 of a 16-row tile, token K 32j + 8g .. +7);
- the four-buffer ring consumes every stage once, in order, from the buffer
  it was issued into, never overwrites a stage before it is read, and waits
  at each stage for exactly the loads of the stages issued before it.

A mistake in either (a swizzle that ignores a load's row offset, a wait one
stage short) gives in-bounds but wrong reads on the GPU, which only a
parity test with the right shapes would catch.

Further sections replay the register-token tile's layouts and rings
(ffn_gemm_wide.hip), the XCD raster over the realised row blocks, and the
LDS-staged router's stage layout and K quarters (router.hip).
"""

import pytest

ROWS, TOKENS, WAVES = 256, 128, 8
A_ROW, B_ROW = 64, 128           # bytes per row and stage: 64 e4m3fn, 64 bf16
A_BYTES = ROWS * A_ROW           # 16 KB
LOADS_A = A_BYTES // 1024 // WAVES
LOADS_B = TOKENS * B_ROW // 1024 // WAVES


def a_row(wave, i, lane):
    return 32 * wave + 16 * i + lane // 4


def a_slot(lane):
    return (lane % 4) ^ (((lane // 4) >> 1) & 3)


def b_row(wave, i, lane):
    return 16 * wave + 8 * i + lane // 8


def b_slot(i, lane):
    return (lane % 8) ^ (((8 * i + lane // 8) >> 1) & 7)


def _written():
    """LDS byte -> (operand, row, k) as the loaders fill one stage."""
    lds = {}
    for w in range(WAVES):
        for i in range(LOADS_A):
            for lane in range(64):
                base = (w * LOADS_A + i) * 1024 + lane * 16
                row = a_row(w, i, lane)
                assert base // A_ROW == row  # the load writes 16 whole rows
                for byte in range(16):
                    lds[base + byte] = ("A", row, 16 * a_slot(lane) + byte)
        for i in range(LOADS_B):
            for lane in range(64):
                base = A_BYTES + (w * LOADS_B + i) * 1024 + lane * 16
                row = b_row(w, i, lane)
                assert (base - A_BYTES) // B_ROW == row
                for byte in range(0, 16, 2):  # bf16: two bytes per k
                    lds[base + byte] = ("B", row, (16 * b_slot(i, lane) + byte) // 2)
    return lds


def test_every_fragment_read_finds_its_operand():
    lds = _written()
    assert len(lds) == A_BYTES + TOKENS * B_ROW // 2
    for lane in range(64):
        r16, g = lane % 16, lane // 16
        swa, swb = (r16 >> 1) & 3, (r16 >> 1) & 7
        for j in range(2):
            a_off = r16 * A_ROW + (((2 * j + (g >> 1)) ^ swa) << 4) + 8 * (g & 1)
            b_off = A_BYTES + r16 * B_ROW + (((4 * j + g) ^ swb) << 4)
            for tile in range(0, ROWS, 16):
                for e in range(8):
                    assert lds[a_off + tile * A_ROW + e] == ("A", tile + r16, 32 * j + 8 * g + e)
            for tile in range(0, TOKENS, 16):
                for e in range(8):
                    assert lds[b_off + tile * B_ROW + 2 * e] == ("B", tile + r16, 32 * j + 8 * g + e)


def test_a_swizzle_that_ignores_the_load_offset_is_caught():
    """The planted mistake the first version made (token slots swizzled
    with load 0's rows for every load) must fail the check above."""
    def bad_slot(i, lane):
        return (lane % 8) ^ (((lane // 8) >> 1) & 7)
    mismatches = 0
    for i in range(LOADS_B):
        for lane in range(64):
            mismatches += bad_slot(i, lane) != b_slot(i, lane)
    assert mismatches > 0


def _ring(nst):
    """The ring of MidRing::run (four buffers): returns the consumed order,
    asserting the waits and the buffer reuse."""
    S = 4
    issued, consumed, held = [], [], {}

    def issue(buf, s):
        assert s < nst and buf == s % S and buf not in held
        held[buf] = s
        issued.append(s)

    def step(p, W, k_issue, s):
        later = [x for x in issued if x > s]
        assert s in issued and len(later) == W, (nst, s, W, later)
        assert held.get(p) == s
        if k_issue:
            issue((p + 3) % S, s + 3)
        consumed.append(s)
        del held[p]

    issue(0, 0), issue(1, 1), issue(2, 2)
    s = 0
    while s + 4 < nst:
        for p in range(4):
            step(p, 2, True, s + p)
        s += 4
    step(0, 2, True, s)
    step(1, 2, False, s + 1)
    step(2, 1, False, s + 2)
    step(3, 0, False, s + 3)
    return consumed


@pytest.mark.parametrize("nst", [4, 8, 12, 16, 32, 56, 112, 224])
def test_ring_consumes_every_stage_in_order(nst):
    assert _ring(nst) == list(range(nst))


def test_ring_needs_a_multiple_of_four_stages():
    with pytest.raises(AssertionError):
        _ring(6)


# ---------------------------------------------------------------- the 128-token register-token tile
# (mixture_experts_moe_amd/csrc/ffn_gemm_wide.hip): weights only through
# LDS, 256 rows x 128 bytes per stage in eight-row loads; the token
# fragments of a stage in one of D register sets; a ring of depth D (3 for
# e4m3fn, 4 for bf16).


def test_wide_weight_fragments_find_their_rows():
    """Weight load q covers rows 8q .. 8q+7, lane l -> row 8q + l/8, physical
    slot (l%8) holding logical slot (l%8) ^ ((row >> 1) & 7); the fragment
    reads of each k-step find k = 32j + 8g .. +7 of row r16 of every tile."""
    for wsize in (1, 2):
        lds = {}
        for q in range(32):
            for lane in range(64):
                row = 8 * q + lane // 8
                slot = (lane % 8) ^ ((row >> 1) & 7)
                for byte in range(16):
                    lds[q * 1024 + lane * 16 + byte] = (row, (16 * slot + byte) // wsize)
        for lane in range(64):
            r16, g = lane % 16, lane // 16
            sw = (r16 >> 1) & 7
            for j in range(128 // wsize // 32):
                if wsize == 1:
                    off = r16 * 128 + (((2 * j + (g >> 1)) ^ sw) << 4) + 8 * (g & 1)
                    elems = [off + e for e in range(8)]
                else:
                    off = r16 * 128 + (((4 * j + g) ^ sw) << 4)
                    elems = [off + 2 * e for e in range(8)]
                for tile in range(0, 256, 16):
                    for e in range(8):
                        assert lds[elems[e] + tile * 128] == (tile + r16, 32 * j + 8 * g + e)


def _wide_ring(nst, D):
    """WidRing::run: stages 0 .. D-2 issued up front; the loop runs D issuing
    stages at a time while s + 2D - 1 <= nst; the tail of N stages (N = D-1
    when nst % D == D-1, else nst % D + D) waits with min(D-2, N-1-i) later
    stages issued and issues while i < N - (D-1)."""
    issued, consumed, held = [], [], {}

    def issue(buf, s):
        assert s < nst and buf == s % D and buf not in held
        held[buf] = s
        issued.append(s)

    def step(p, W, k_issue, s):
        later = [x for x in issued if x > s]
        assert s in issued and len(later) == W, (nst, D, s, W, later)
        assert held.get(p) == s
        del held[p]
        if k_issue:
            issue((p + D - 1) % D, s + D - 1)
        consumed.append(s)

    for i in range(D - 1):
        issue(i, i)
    s = 0
    while s + 2 * D - 1 <= nst:
        for p in range(D):
            step(p, D - 2, True, s + p)
        s += D
    R = nst % D
    N = D - 1 if R == D - 1 else R + D
    assert s + N == nst
    for i in range(N):
        step(i % D, min(D - 2, N - 1 - i), i < N - (D - 1), s + i)
    return consumed


@pytest.mark.parametrize("D", [3, 4])
@pytest.mark.parametrize("nst", list(range(4, 40)) + [45, 56, 112, 224])
def test_wide_ring_consumes_every_stage_in_order(D, nst):
    assert _wide_ring(nst, D) == list(range(nst))


def test_wide_ring_shortest_k():
    # the launcher asks for at least D stages; D - 1 would do, D - 2 would not
    assert _wide_ring(3, 3) == [0, 1, 2]
    assert _wide_ring(3, 4) == [0, 1, 2]
    with pytest.raises(AssertionError):
        _wide_ring(2, 4)


def _big_tile_of(p, gx, gy, cols, xcds=8):
    """big_tile_of (ffn_big_common.h): workgroup p -> (live, b, y)."""
    total = gx * gy
    per_xcd = -(-total // xcds)
    l = (p % xcds) * per_xcd + p // xcds
    if not (p // xcds < per_xcd and l < total):
        return None
    band = cols * gx
    sr, rem = divmod(l, band)
    c = min(cols, gy - sr * cols)
    return rem // c, sr * cols + rem % c


@pytest.mark.parametrize("gx_grid,gx_live,gy,cols", [
    (384, 256, 16, 2), (384, 256, 28, 4), (384, 256, 4, 2), (384, 256, 7, 4),
    (48, 36, 23, 1), (48, 36, 12, 2), (40, 40, 112, 4), (10, 0, 8, 2), (5, 3, 1, 4)])
def test_raster_over_realised_blocks_covers_each_tile_once(gx_grid, gx_live, gy, cols):
    """The grid is sized for the capacity's blocks (gx_grid, rounded up to
    whole XCD rounds) while the raster runs over the realised ones: every
    tile (b < gx_live, y) goes to exactly one workgroup, the same number of
    tiles to each XCD but the last (which takes what is left, fewer than
    eight less), and the workgroups left over have none."""
    grid = -(-gx_grid * gy // 8) * 8
    seen = {}
    per = [0] * 8
    for p in range(grid):
        t = _big_tile_of(p, gx_live, gy, cols)
        if t is None:
            continue
        assert t not in seen, (t, p, seen.get(t))
        seen[t] = p
        per[p % 8] += 1
    assert set(seen) == {(b, y) for b in range(gx_live) for y in range(gy)}
    assert max(per) - min(per) < 8
    assert all(n == max(per) for n in per[:7]) or gx_live * gy < 8


def test_wide_half_block_token_rows_find_their_fragments():
    """Half-full blocks of the register-token tile (e4m3fn weights): 64 token
    rows of 256 bytes per stage after the 32 KB of weights, four rows per
    1 KB load (wave w, load i: rows 4 (2w + i) + l / 16, physical slot l % 16
    holding logical slot (l % 16) ^ (row & 15)); the k-step j fragment of
    lane (r16, g) in token tile u reads k = 32j + 8g .. +7 of row 16u + r16."""
    base_b = 256 * 128
    lds = {}
    rows_of_wave = {}
    for w in range(8):
        for i in range(2):
            for lane in range(64):
                row = 4 * (2 * w + i) + lane // 16
                rows_of_wave.setdefault(w, set()).add(row)
                slot = (lane % 16) ^ (row & 15)
                base = base_b + (2 * w + i) * 1024 + lane * 16
                assert (base - base_b) // 256 == row
                for byte in range(0, 16, 2):
                    lds[base + byte] = (row, (16 * slot + byte) // 2)
    assert all(rows_of_wave[w] == set(range(8 * w, 8 * w + 8)) for w in range(8))
    assert len(lds) == 64 * 128
    for lane in range(64):
        r16, g = lane % 16, lane // 16
        for j in range(4):
            off = base_b + r16 * 256 + (((4 * j + g) ^ r16) << 4)
            for tile in range(0, 64, 16):
                for e in range(8):
                    assert lds[off + tile * 256 + 2 * e] == (tile + r16, 32 * j + 8 * g + e)


def test_wide_full_block_token_rows_find_their_fragments():
    """Full blocks of the register-token tile (e4m3fn weights, more than 64
    tokens): 128 token rows of 256 bytes per stage in two 16 KB arrays (rows
    0-63 and 64-127); wave w, load i fills rows 16w + 4i + l / 16 at
    physical slot l % 16 holding logical slot (l % 16) ^ (row & 15); the
    k-step j fragment of lane (r16, g) in token tile u reads k = 32j + 8g ..
    +7 of row 16u + r16."""
    lds = {}
    for w in range(8):
        region = "a" if w < 4 else "b"
        for i in range(4):
            base = (w & 3) * 16 * 256 + i * 1024
            for lane in range(64):
                row = 16 * w + 4 * i + lane // 16
                slot = (lane % 16) ^ (row & 15)
                off = base + lane * 16
                assert off // 256 == row % 64 and off + 16 <= 16384
                for byte in range(0, 16, 2):
                    assert (region, off + byte) not in lds
                    lds[(region, off + byte)] = (row, (16 * slot + byte) // 2)
    assert len(lds) == 128 * 128
    for lane in range(64):
        r16, g = lane % 16, lane // 16
        for j in range(4):
            lb = r16 * 256 + (((4 * j + g) ^ r16) << 4)
            for u in range(8):
                region = "a" if u < 4 else "b"
                for e in range(8):
                    got = lds[(region, lb + 16 * (u & 3) * 256 + 2 * e)]
                    assert got == (16 * u + r16, 32 * j + 8 * g + e)


def _full_rings(total):
    """FullRing::run: weights W(0), tokens T(0), weights W(1) up front; stage s
    waits until only the weights of s + 1 (when issued) may be in flight,
    then issues T(s + 1) into token buffer (s + 1) % 2 and W(s + 2) into
    weight buffer (s + 2) % 3.  Checks that each stage's operands have
    landed, in the buffers it reads, and that no buffer is reloaded before
    the stage that read it is over."""
    issued = []  # (kind, stage, buffer) in issue order
    wbuf, xbuf = {}, {}

    def issue(kind, st):
        nb = 3 if kind == "W" else 2
        held = wbuf if kind == "W" else xbuf
        b = st % nb
        assert b not in held, (kind, st, held)  # the stage that used it is over
        held[b] = st
        issued.append((kind, st))

    issue("W", 0)
    issue("T", 0)
    issue("W", 1)
    done = []
    for s in range(total):
        allowed = 1 if s + 1 < total else 0   # loads (of four) still in flight
        landed = issued[:len(issued) - allowed]
        assert ("W", s) in landed and ("T", s) in landed
        if allowed:
            assert issued[-1] == ("W", s + 1)
        # the barrier: stage s - 1 is over everywhere
        for held, nb in ((wbuf, 3), (xbuf, 2)):
            for b in [b for b, st in held.items() if st == s - 1]:
                del held[b]
        if s + 1 < total:
            issue("T", s + 1)
        if s + 2 < total:
            issue("W", s + 2)
        assert wbuf.get(s % 3) == s and xbuf.get(s % 2) == s
        done.append(s)
    return done


@pytest.mark.parametrize("total", list(range(3, 20)) + [56, 112])
def test_wide_full_block_rings(total):
    assert _full_rings(total) == list(range(total))


# ---------------------------------------------------------------- router logits through LDS
# (mixture_experts_moe_amd/csrc/router.hip, router_logits_lds_kernel): one
# stage is 128 x rows x 64 bf16 (128 bytes, eight 16-byte slots, slot s of
# row r at s ^ ((r >> 1) & 7)) and 64 W_gate rows x 64 fp32 (256 bytes,
# sixteen slots, slot s of row r at s ^ (r & 15)); thread t of 512 stores x
# slot u = t + 512 i (row u >> 3, slot u & 7) and W_gate slot u (row u >> 4,
# slot u & 15) for i = 0, 1, from global element k = 8 (u & 7) of its x row
# and k = 4 (u & 15) of its W_gate row.

RL_THREADS = 512


def _router_lds_written():
    xs, ws = {}, {}
    for t in range(RL_THREADS):
        for i in range(2):
            u = t + RL_THREADS * i
            xr, xsl = u >> 3, u & 7
            off = xr * 128 + ((xsl ^ ((xr >> 1) & 7)) << 4)
            for b in range(0, 16, 2):
                assert off + b not in xs
                xs[off + b] = (xr, 8 * xsl + b // 2)  # (token row, k)
            wr, wsl = u >> 4, u & 15
            off = wr * 256 + ((wsl ^ (wr & 15)) << 4)
            for b in range(0, 16, 4):
                assert off + b not in ws
                ws[off + b] = (wr, 4 * wsl + b // 4)  # (expert row, k)
    return xs, ws


def test_router_lds_fragments_find_their_operands():
    """Every fragment the eight waves read (lane (r16, g) of wave w, step h:
    W_gate row 16 (w % 4) + r16, k = 32 h + 8 g .. +8 in two 16-byte slots;
    x row 64 (w / 4) + 16 u + r16, k = 32 h + 8 g .. +8) holds exactly those
    values, both buffers are filled whole, and the 16 rows one 16-lane group
    reads at one k fall in 16 different 16-byte bank groups."""
    xs, ws = _router_lds_written()
    assert len(xs) == 128 * 64 and len(ws) == 64 * 64
    for w in range(8):
        for lane in range(64):
            r16, g = lane & 15, lane >> 4
            er = 16 * (w & 3) + r16
            for h in range(2):
                sl = 8 * h + 2 * g
                for half, slot in enumerate((sl, sl + 1)):
                    off = er * 256 + ((slot ^ r16) << 4)
                    for q in range(4):
                        assert ws[off + 4 * q] == (er, 32 * h + 8 * g + 4 * half + q)
                for u in range(4):
                    tr = 64 * (w >> 2) + 16 * u + r16
                    off = tr * 128 + (((4 * h + g) ^ ((tr >> 1) & 7)) << 4)
                    for q in range(8):
                        assert xs[off + 2 * q] == (tr, 32 * h + 8 * g + q)
    # bank groups of one 16-lane group's reads (16-byte groups mod 256 bytes)
    for w in range(8):
        for g in range(4):
            for h in range(2):
                wb = {((16 * (w & 3) + r) * 256 + (((8 * h + 2 * g) ^ r) << 4)) % 256 // 16
                      for r in range(16)}
                assert len(wb) == 16
                for u in range(4):
                    xb = set()
                    for r in range(16):
                        tr = 64 * (w >> 2) + 16 * u + r
                        xb.add((tr * 128 + (((4 * h + g) ^ ((tr >> 1) & 7)) << 4)) % 256 // 16)
                    assert len(xb) == 16


def test_router_lds_quarters_are_the_wide_waves_ranges():
    """The LDS tile's K quarter z covers the 32-wide steps [z S/4, (z+1) S/4)
    of the wide tiles' wave z, in whole 64-wide stages, for every d the
    layer sends it (d % 256 == 0)."""
    for d in range(256, 16385, 256):
        steps = d // 32
        covered = []
        for z in range(4):
            k_begin = (z * steps // 4) * 32
            nst = ((z + 1) * steps // 4 - z * steps // 4) // 2
            assert ((z + 1) * steps // 4 - z * steps // 4) % 2 == 0
            covered += list(range(k_begin // 32, k_begin // 32 + 2 * nst))
            assert covered[-1] + 1 == (z + 1) * steps // 4
        assert covered == list(range(steps))
