"""Pins of the oracle's staged scale order (oracle_stage_scales), the storage
order the library's grouped GEMM reads one K stage of 256 elements in
(include/mx.h, MX_SCALES_STAGED).  The order is the library's, not the
pages'; it permutes bytes and does no arithmetic.

- two examples worked out by hand (tests/golden/staged_scales.txt): a
  row-wise grid with a ragged last stage, and a grouped grid with an empty
  group, a group of two stages and a one-block group;
- on random grids the order equals sequential packing (each group's blocks
  appended to fresh stages of 8, stage after stage), computed here by a
  different route: walking the blocks one by one with a running cursor;
- every input byte lands exactly once and no two blocks share a slot.

Also the column-wise layout with groups padded to 256 tokens: RTNE blocks
equal those of the 32-token padding at the new starts with zero-filled
padding blocks, and SR draws at the padded position (rebuilt element by
element from the generator and the SR magnitude rule).
"""
import os

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "staged_scales.txt")


def _cases():
    cases, cur = [], None
    for line in open(GOLDEN):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        if line.startswith("case"):
            f = dict(kv.split("=") for kv in line.split()[2:])
            cur = {"name": line.split()[1], "rows": int(f["rows"]), "nblk": int(f["nblk"]),
                   "groups": None if f["groups"] == "none" else [int(v) for v in f["groups"].split(",")],
                   "lines": []}
            cases.append(cur)
        else:
            head, vals = line.split(":")
            s, r = (int(v) for v in head.split())
            cur["lines"].append((s, r, [255 if v == "." else int(v) for v in vals.split()]))
    return cases


@pytest.mark.parametrize("case", _cases(), ids=lambda c: c["name"])
def test_hand_worked_examples(case):
    rows, nblk = case["rows"], case["nblk"]
    mult = 10 if case["groups"] is None else 100
    sc = np.array([[mult * r + b for b in range(nblk)] for r in range(rows)], dtype=np.uint8)
    off = None if case["groups"] is None else np.concatenate([[0], np.cumsum(case["groups"])])
    got = oracle.stage_scales(sc, off, fill=255)
    want = np.full_like(got, 255)
    for s, r, vals in case["lines"]:
        want[s, r] = vals
    assert got.shape[0] == 1 + max(s for s, _, _ in case["lines"])
    assert np.array_equal(got, want)


def _sequential_pack(sc, counts):
    """Walk the blocks group by group with a cursor (stage, slot) that moves
    to a fresh stage at every group start and every 8 blocks."""
    rows, nblk = sc.shape
    pos = {}
    stage, b = -1, 0
    for n in counts:
        nb = (n + 31) // 32
        for i in range(nb):
            if i % 8 == 0:
                stage += 1
            pos[b] = (stage, i % 8)
            b += 1
    out = {}
    for r in range(rows):
        for blk, (s, j) in pos.items():
            out[(s, r, j)] = sc[r, blk]
    return out, stage + 1


@pytest.mark.parametrize("seed", [0, 1, 2, 3])
def test_random_groupings_match_sequential_packing(seed):
    rng = np.random.default_rng(seed)
    G = int(rng.integers(1, 7))
    counts = rng.integers(0, 700, G)
    counts[rng.integers(0, G)] = 0                     # at least one empty group
    nblk = int(np.sum((counts + 31) // 32))
    rows = int(rng.integers(1, 5))
    sc = rng.integers(0, 256, (rows, nblk), dtype=np.uint8)
    got = oracle.stage_scales(sc, np.concatenate([[0], np.cumsum(counts)]), fill=0)
    want, nst = _sequential_pack(sc, counts)
    assert got.shape == (nst, rows, 8)
    seen = np.zeros(got.shape, dtype=bool)
    for (s, r, j), v in want.items():
        assert got[s, r, j] == v
        assert not seen[s, r, j]
        seen[s, r, j] = True
    assert seen.sum() == rows * nblk                  # every byte once
    assert np.all(got[~seen] == 0)                    # the rest untouched


def test_row_wise_is_one_group_per_row_and_extra_stages_stay_filled():
    rng = np.random.default_rng(9)
    sc = rng.integers(0, 256, (3, 19), dtype=np.uint8)
    a = oracle.stage_scales(sc, fill=7)
    b = oracle.stage_scales(sc, np.array([0, 19 * 32]), stages=5, fill=7)
    assert a.shape == (3, 3, 8) and b.shape == (5, 3, 8)
    assert np.array_equal(a, b[:3]) and np.all(b[3:] == 7)
    for r in range(3):
        assert np.array_equal(a[:, r, :].reshape(-1)[:19], sc[r])


def test_group_pad_256_places_blocks_and_zero_fills():
    """Groups padded to 256 tokens (the layout whose weight-gradient K stages
    start on whole code lines): with RTNE, which does not depend on position,
    each group's blocks equal those of the 32-token padding at the group's
    new start, and the blocks between a group's 32-padded and 256-padded ends
    are all-zero codes with scale byte 0 (amax 0)."""
    rng = np.random.default_rng(11)
    counts = [100, 0, 257, 31]
    off = np.concatenate([[0], np.cumsum(counts)])
    x = rng.standard_normal((int(off[-1]), 40)).astype(np.float32)
    c32, s32 = oracle.quantize_1d(x, block_axis=0, group_offsets=off)
    c256, s256 = oracle.quantize_1d(x, block_axis=0, group_offsets=off, group_pad=256)
    assert s256.shape == (40, (256 + 0 + 512 + 256) // 32)
    p32 = p256 = 0
    for n in counts:
        b32, b256 = (n + 31) // 32, (n + 255) // 256 * 8
        assert np.array_equal(s256[:, p256:p256 + b32], s32[:, p32:p32 + b32])
        assert np.array_equal(c256[:, 16 * p256:16 * (p256 + b32)], c32[:, 16 * p32:16 * (p32 + b32)])
        assert np.all(s256[:, p256 + b32:p256 + b256] == 0)
        assert np.all(c256[:, 16 * (p256 + b32):16 * (p256 + b256)] == 0)
        p32 += b32
        p256 += b256


def test_group_pad_256_sr_uses_the_padded_position():
    """With SR each element draws its 16 bits at index c * kp + its padded
    position: rebuilt here for a few elements from the generator and the SR
    magnitude rule, for the third group (which starts at 512 when groups are
    padded to 256, at 160 when padded to 32)."""
    rng = np.random.default_rng(12)
    counts = [100, 60, 300]
    off = np.concatenate([[0], np.cumsum(counts)])
    x = rng.standard_normal((int(off[-1]), 8)).astype(np.float32)
    c, s = oracle.quantize_1d(x, block_axis=0, group_offsets=off, group_pad=256, rnd=oracle.SR, seed=7, stream=3)
    kp = c.shape[1] * 2
    assert kp == 256 + 256 + 512
    for col, r in ((0, 0), (5, 37), (7, 299)):
        pos = 512 + r
        v = float(x[off[2] + r, col])
        byte = int(s[col, pos // 32])
        a = abs(v) / 2.0 ** (byte - 127)
        mag = oracle.sr_mag(a, oracle.sr_bits(7, 3, col * kp + pos))
        code = (c[col, pos // 2] >> (4 * (pos % 2))) & 0xF
        assert code & 7 == mag
        assert (code >> 3) == (1 if v < 0 else 0) or mag == 0
