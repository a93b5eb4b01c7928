"""The swizzled LDS tile layout of the direct-to-LDS kernels (host-side check).

The bf16/fp16 kernels that load their tiles HBM -> LDS with the LDS bit of
the buffer loads (forward d = 128; backward dK/dV and dQ at d = 64 and 128)
store a tile of 32 rows x d columns unpadded, with the 16-byte chunks of row
r XOR-permuted by a swizzle of r: chunk_swz (fa_lds_dma.hpp) for 256-byte
rows and row_swz<64> (fa_bwd_h16.hip) for 128-byte rows.  The swizzle
expressions are read from those sources and evaluated here (C's and Python's
integer bit operators agree on non-negative values), and the load mapping and
the read addresses the kernels compute are restated from the kernel code:

  * load: wave w's 16-byte load i writes LDS bytes [16 l, 16 l + 16) of the
    block of rows R = (64 / chunks) (4 i + w); lane l fetches row
    R + l / chunks, chunk (l % chunks) ^ swz(row);
  * row reads (the A operands of S and dP): lane (col, grp) reads row col,
    chunk 2 kc + grp, at (col * rowbytes + 16 (grp ^ swz(col))) ^ 32 kc;
  * transpose reads (ds_read_b64_tr_b16, the transposed operands): lane reads
    8 bytes of rows trow = 4 grp + (lane % 16) / 4 and trow + 8 of each
    16-row chunk, logical byte 64 db + 32 ((lane / 16) % 2) + 8 (lane % 4),
    at (row * rowbytes + 16 (tx ^ swz(row)) + 8 (lane % 2)) ^ 64 db.

The checks: the load writes every (row, chunk) of the tile exactly once and
stays inside the stage; every read returns the logical element the MFMA
operand layout needs; and the reads are free of LDS bank conflicts with 64
banks (and with 32) of 4 bytes.  "FlashAttention dissected", section "The
physical bottleneck: GPU memory hierarchy dissected" (on-chip shared memory
as the staging level); "CUDA Flash Attention: Online Softmax with Shared
Memory Tiling", section "Design decisions" (shared rows laid out against
bank conflicts).
"""
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "exact_attention_13_amd", "csrc")
ROWS = 32   # rows of a streamed tile
WAVES = 4   # waves that share the tile's loads


def _expr(path, pattern):
    text = open(os.path.join(CSRC, path)).read()
    m = re.search(pattern, text, re.S)
    assert m, f"swizzle expression not found in {path}"
    return " ".join(m.group(1).split())


def _swizzles():
    e128 = _expr("fa_lds_dma.hpp", r"int chunk_swz\(int r\) \{\s*return (.*?);")
    e64 = _expr("fa_bwd_h16.hip", r"int row_swz\(int r\) \{.*?else\s*return (.*?);")
    f128 = eval("lambda r: " + e128)
    f64 = eval("lambda r: " + e64)
    return {128: f128, 64: f64}


SWZ = _swizzles()


@pytest.mark.parametrize("d", [64, 128])
def test_swizzle_is_a_permutation_per_row_group(d):
    chunks = d // 8
    swz = SWZ[d]
    for r in range(64):
        assert 0 <= swz(r) < chunks
        assert swz(r) == swz(r % 16), "the swizzle must depend on the row within 16 only"
    # rows 2j and 2j + 1 share a 256-byte bank line at d = 64: (r & 1, swz(r))
    # must then be distinct over 16 rows, i.e. swz a bijection per row parity
    if d == 64:
        assert len({(r & 1, swz(r)) for r in range(16)}) == 16
    else:
        assert len({swz(r) for r in range(16)}) == 16


def _load_map(d):
    rowbytes, chunks = 2 * d, d // 8
    load_rows = 64 // chunks
    per = ROWS * d * 2 // (WAVES * 64 * 16)
    lds = {}
    for i in range(per):
        for w in range(WAVES):
            block = load_rows * (i * WAVES + w)
            for lane in range(64):
                dma_row = load_rows * w + lane // chunks
                row = block + lane // chunks
                assert SWZ[d](row) == SWZ[d](dma_row)
                chunk = (lane % chunks) ^ SWZ[d](dma_row)
                addr = block * rowbytes + 16 * lane
                assert addr not in lds and 0 <= addr < ROWS * rowbytes
                lds[addr] = (row, chunk)
    return lds


@pytest.mark.parametrize("d", [64, 128])
def test_load_writes_each_chunk_once(d):
    lds = _load_map(d)
    assert sorted(lds.values()) == sorted((r, c) for r in range(ROWS) for c in range(d // 8))


@pytest.mark.parametrize("d", [64, 128])
def test_row_reads_fetch_their_operand(d):
    lds, swz, rowbytes = _load_map(d), SWZ[d], 2 * d
    for lane in range(64):
        col, grp = lane & 31, lane >> 5
        base = col * rowbytes + 16 * (grp ^ swz(col))
        for kc in range(d // 16):
            assert lds[base ^ (32 * kc)] == (col, 2 * kc + grp)


def _tr_addr(d, lane, second, db, ch):
    swz, rowbytes = SWZ[d], 2 * d
    grp = lane >> 5
    trow = 4 * grp + ((lane & 15) >> 2) + (8 if second else 0)
    tx = 2 * ((lane >> 4) & 1) + ((lane & 3) >> 1)
    off = trow * rowbytes + 16 * (tx ^ swz(trow)) + 8 * (lane & 1)
    return (off ^ (64 * db)) + ch * 16 * rowbytes, ch * 16 + trow


@pytest.mark.parametrize("d", [64, 128])
def test_transpose_reads_fetch_their_operand(d):
    lds = _load_map(d)
    for lane in range(64):
        for second in (False, True):
            for db in range(d // 32):
                for ch in range(2):
                    a, row = _tr_addr(d, lane, second, db, ch)
                    r, c = lds[a & ~15]
                    assert r == row
                    assert 16 * c + (a & 15) == 64 * db + 32 * ((lane >> 4) & 1) + 8 * (lane & 3)


@pytest.mark.parametrize("banks", [64, 32])
@pytest.mark.parametrize("d", [64, 128])
def test_reads_are_bank_conflict_free(d, banks):
    swz, rowbytes = SWZ[d], 2 * d
    line = 4 * banks
    # 16-byte row reads: line / 16 lanes per cycle, each on its own 16 bytes
    per = line // 16
    for kc in range(d // 16):
        for g in range(64 // per):
            lanes = range(per * g, per * g + per)
            slots = {(((l & 31) * rowbytes + 16 * ((l >> 5) ^ swz(l & 31))) ^ (32 * kc)) % line // 16
                     for l in lanes}
            assert len(slots) == per, (d, banks, kc, g)
    # 8-byte transpose reads: line / 8 lanes per cycle, two banks each
    per = line // 8
    for db in range(d // 32):
        for second in (False, True):
            for g in range(64 // per):
                used = set()
                for lane in range(per * g, per * g + per):
                    a, _ = _tr_addr(d, lane, second, db, 0)
                    used |= {(a % line) // 4, (a % line) // 4 + 1}
                assert len(used) == 2 * per, (d, banks, db, second, g)
