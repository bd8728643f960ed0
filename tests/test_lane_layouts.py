"""CPU models of two lane-to-data mappings in the HIP kernels.

Both move weight data between the layout it is loaded in and the layout the
products need; a wrong index would silently mix rows or blocks, which the GPU
parity tests would catch only as a numerical mismatch.  These models restate the
index arithmetic of the kernels and check it against its intent exhaustively.

* Decode GEMV scales (ffn_gemv.hip, gemv_scale_byte): a group's 8 rows x 64 E8M0
  blocks of one slice are loaded as two dwords per lane -- lane L, dword m holds
  rows 4m + L/16, blocks 4 (L % 16) .. +3 -- and lane L takes the byte of block L
  of row j from lane 16 (j % 4) + L/4, byte L % 4 of dword j/4.
* Tiled kernel, 80-row tiles (ffn_tile.hip, put_pair / compute): the same stores,
  two chunks of 128 elements per 128-byte row visit; for chunk j of the pair lane l
  reads row l % 16, block 4j + l / 16 (the FP4 operand: lane group g holds
  elements 32g .. 32g + 31 of the chunk).
* Streaming kernel, 32-row tiles (ffn_stream.hip, transit): load instruction h of a
  16-row fragment gives lane l row 8h + l/8, 16-byte block l % 8 of a 128-byte
  chunk; the wavefront stores it to LDS and reads back, for the MFMA layout, row
  l % 16, blocks 2 (l / 16) + j (j = 0, 1).  Row r's block b sits in 256-byte line
  r/2 at quad 8 (r % 2) + (b ^ r/2).  LDS serves a 16-byte access of 8 lanes
  (stores) or 16 lanes (loads) at once; no two of them may share a quad (bank
  group of 16 bytes in a 256-byte window).
"""
import itertools


def test_gemv_scale_byte_holder():
    # scale block b of row r (r < 8, b < 64) as the byte the loads deliver
    def loaded(lane, m):
        row = 4 * m + lane // 16
        return [(row, 4 * (lane % 16) + i) for i in range(4)]

    for j, lane in itertools.product(range(8), range(64)):
        holder = 16 * (j % 4) + lane // 4
        got = loaded(holder, j // 4)[lane % 4]
        assert got == (j, lane), (j, lane, got)


def _store_addr(h, lane):
    r, b = 8 * h + lane // 8, lane % 8
    return (r // 2) * 256 + ((r % 2) * 8 + (b ^ (r // 2))) * 16


def _load_addr(j, lane):
    r16, g = lane % 16, lane // 16
    bj = 2 * g + j
    return (r16 // 2) * 256 + ((r16 % 2) * 8 + (bj ^ (r16 // 2))) * 16


def _place(r, b):
    return (r // 2) * 256 + ((r % 2) * 8 + (b ^ (r // 2))) * 16


def _tile_load_addr(j, lane):
    r16, g = lane % 16, lane // 16
    bj = 4 * j + g
    return (r16 // 2) * 256 + ((r16 % 2) * 8 + (bj ^ (r16 // 2))) * 16


def test_tile_transit_round_trip_gives_the_fp4_operand_layout():
    lds = {}
    for h, lane in itertools.product(range(2), range(64)):
        lds[_store_addr(h, lane)] = (8 * h + lane // 8, lane % 8)
    for j, lane in itertools.product(range(2), range(64)):
        assert lds[_tile_load_addr(j, lane)] == (lane % 16, 4 * j + lane // 16)


def test_tile_transit_reads_are_free_of_bank_conflicts():
    quad = lambda a: (a // 16) % 16
    for j in range(2):
        for first in range(0, 64, 16):
            qs = [quad(_tile_load_addr(j, lane)) for lane in range(first, first + 16)]
            assert len(set(qs)) == 16, (j, first, qs)


def test_tile_scale_slots():
    # lane l stores the four scale dwords of row (fragment l // 16, row l % 16) for
    # chunks c = 0..3 of two pairs at dword (16 c + row) * 4 + fragment; lane (r16, g)
    # reads four consecutive dwords at (16 (kc % 4) + r16) * 4: fragment f's dword
    slots = {}
    for lane, c in itertools.product(range(64), range(4)):
        slots[(16 * c + lane % 16) * 4 + lane // 16] = (lane // 16, lane % 16, c)
    assert sorted(slots) == list(range(256))
    for kc, lane in itertools.product(range(8), range(64)):
        r16 = lane % 16
        for f in range(4):
            assert slots[(16 * (kc % 4) + r16) * 4 + f] == (f, r16, kc % 4)


def test_transit_layout_is_a_bijection_onto_2kb():
    addrs = {_place(r, b) for r in range(16) for b in range(8)}
    assert len(addrs) == 128
    assert addrs == set(range(0, 2048, 16))


def test_transit_round_trip_gives_the_mfma_layout():
    lds = {}
    for h, lane in itertools.product(range(2), range(64)):
        lds[_store_addr(h, lane)] = (8 * h + lane // 8, lane % 8)   # (row, block) loaded
    assert len(lds) == 128
    for j, lane in itertools.product(range(2), range(64)):
        assert lds[_load_addr(j, lane)] == (lane % 16, 2 * (lane // 16) + j)


def test_transit_accesses_are_free_of_bank_conflicts():
    quad = lambda a: (a // 16) % 16
    for h in range(2):
        for first in range(0, 64, 8):   # stores: 8 lanes at a time
            qs = [quad(_store_addr(h, lane)) for lane in range(first, first + 8)]
            assert len(set(qs)) == 8, (h, first, qs)
    for j in range(2):
        for first in range(0, 64, 16):   # loads: 16 lanes at a time
            qs = [quad(_load_addr(j, lane)) for lane in range(first, first + 16)]
            assert len(set(qs)) == 16, (j, first, qs)


def test_models_match_the_kernel_sources():
    # the index expressions modelled above, as they stand in the kernels
    import os
    csrc = os.path.join(os.path.dirname(__file__), "..", "mxfp4_routed_expert_route_amd", "csrc")
    stream = open(os.path.join(csrc, "ffn_stream.hip")).read()
    assert "(r >> 1) * 256 + ((r & 1) * 8 + (b ^ (r >> 1))) * 16" in stream
    assert "(r16 >> 1) * 256 + ((r16 & 1) * 8 + (bj ^ (r16 >> 1))) * 16" in stream
    assert "const int r = 8 * h + (lane >> 3), b = lane & 7;" in stream
    assert "const int bj = 2 * g + h;" in stream
    tile = open(os.path.join(csrc, "ffn_tile.hip")).read()
    assert "const int r = 8 * h + (lane >> 3), b = lane & 7;" in tile
    assert "(r >> 1) * 256 + ((r & 1) * 8 + (b ^ (r >> 1))) * 16" in tile
    assert "const int j = kc & 1, bj = 4 * j + g;" in tile
    assert "(r16 >> 1) * 256 + ((r16 & 1) * 8 + (bj ^ (r16 >> 1))) * 16" in tile
    assert "wts[(32 + r16) * kFrag + (lane >> 4)] = sr.z;" in tile
    assert "wts + (16 * (kc & 3) + r16) * kFrag" in tile
    gemv = open(os.path.join(csrc, "ffn_gemv.hip")).read()
    assert "const int holder = 16 * (j & 3) + (lane >> 2);" in gemv
    assert "return (d >> (8 * (lane & 3))) & 0xFFu;" in gemv
    assert "const int lane_s = (lane >> 4) * (K / 32) + 4 * (lane & 15);" in gemv
