"""CPU check of the fp8 forward kernel's V operand path (no GPU).

The kernel DMAs fp8 V rows into LDS with their 32-byte bands XOR-swizzled by
the row, then reads each P V operand with ds_read_b64_tr_b8.  A probe on
gfx950 fixed that load's lane layout: in each 16-lane group G, output lane
16 G + 8 h + c receives byte c of the 8-byte reads of lanes 16 G + h, + 2, ...,
+ 14.  This test repeats the kernel's index formulas (DMA lane offsets,
per-lane read offsets, swizzle) in Python, applies that layout, and checks,
element by element, that every lane ends up with the V values its MFMA
operand slot needs: column 32 cb + lane % 32 at the keys of P^T's order
4 g + {0..3, 8..11} (g = lane / 32), for every column block and key step.
It also checks that every DMA destination and LDS read stays inside the tile.
"""
import numpy as np
import pytest

BN = 64  # keys per tile


def swzw(d, row):
    return (((row >> 1) & 3) << 1) if d == 128 else (((row >> 2) & 1) << 1)


def dma_tile(v_tile, d):
    """LDS bytes after the kernel's DMA of one fp8 V tile (4 waves)."""
    ch8 = d // 16
    rpw8 = 64 // ch8
    rounds = BN // (4 * rpw8)
    round8 = 4 * rpw8 * d
    src = v_tile.reshape(-1)
    lds = np.full(BN * d, -1, dtype=np.int64)
    for w in range(4):
        for r in range(rounds):
            for lane in range(64):
                ld_row = w * rpw8 + lane // ch8
                ld_slot = lane % ch8
                voff = ld_row * d + ((ld_slot ^ swzw(d, ld_row)) * 16)
                dst = (r * 4 + w) * rpw8 * d + lane * 16
                at = voff + r * round8
                assert 0 <= dst and dst + 16 <= BN * d and at + 16 <= BN * d
                lds[dst:dst + 16] = src[at:at + 16]
    assert (lds >= 0).all(), "the DMA leaves part of the tile unwritten"
    return lds


def read_offsets(d):
    """The kernel's per-lane byte offsets v_off[lane][cb]."""
    cbs = d // 32
    off = np.zeros((64, cbs), dtype=np.int64)
    for lane in range(64):
        grp, i = lane >> 4, lane & 15
        e, hb = i >> 1, i & 1
        rl = 4 * (grp >> 1) + (e if e < 4 else e + 4)
        for cb in range(cbs):
            off[lane, cb] = rl * d + (((2 * cb + (grp & 1)) ^ swzw(d, rl)) * 16) + 8 * hb
    return off


def tr8_load(lds, addrs):
    """ds_read_b64_tr_b8 as probed: each lane supplies an 8-byte-aligned
    address; output lane 16 G + 8 h + c, element e = byte c of lane
    16 G + 2 e + h."""
    rd = np.stack([lds[a:a + 8] for a in addrs])
    out = np.zeros((64, 8), dtype=np.int64)
    for lane in range(64):
        grp, h, c = lane >> 4, (lane >> 3) & 1, lane & 7
        for e in range(8):
            out[lane, e] = rd[16 * grp + 2 * e + h, c]
    return out


@pytest.mark.parametrize("d", [128, 64])
def test_fp8_v_operands(d):
    rng = np.random.default_rng(d)
    v = rng.integers(0, 256, size=(BN, d))
    lds = dma_tile(v, d)
    off = read_offsets(d)
    for cb in range(d // 32):
        for kt in range(2):
            for hh in range(2):
                base = (kt * 32 + 16 * hh) * d
                addrs = [base + int(off[lane, cb]) for lane in range(64)]
                assert all(a % 8 == 0 and a + 8 <= BN * d for a in addrs)
                got = tr8_load(lds, addrs)
                for lane in range(64):
                    m, g = lane % 32, lane // 32
                    for e in range(8):
                        key = 32 * kt + 16 * hh + 4 * g + (e if e < 4 else e + 4)
                        assert got[lane, e] == v[key, 32 * cb + m], (d, cb, kt, hh, lane, e)


@pytest.mark.parametrize("d", [128, 64])
def test_fp8_v_reads_conflict_free(d):
    """Each 16-lane group of one read touches 16 rows x one 32-byte band;
    with the swizzle, the 64 lanes' 8-byte pieces cover every 4-byte bank of
    a 256-byte bank line exactly twice (512 bytes, two passes), the minimum."""
    off = read_offsets(d)
    for cb in range(d // 32):
        addrs = [int(off[lane, cb]) for lane in range(64)]
        banks = np.zeros(64, dtype=int)
        for a in addrs:
            for b in range(2):
                banks[((a // 4) + b) % 64] += 1
        assert (banks == 2).all(), (d, cb, banks)
