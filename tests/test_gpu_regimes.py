"""GPU parity of launch regimes the small tests do not reach, and the
kernels' guards against malformed device arguments.

- The row-wise quantizer grid-strides: a launch covers at most 8192
  workgroups x 256 blocks = 2,097,152 blocks per trip.  The expert step's
  65536 x 2880 and 65536 x 5760 operands take 3 and 6 trips, through the
  contiguous kernel or, with code rows padded to whole 128-byte lines, the
  wave-uniform padded-row kernel (rows of >= 64 blocks).  Narrow padded rows
  take the per-lane row-split kernel.  Each regime is compared with the
  oracle on the whole matrix.
- Stochastic rounding through the hardware SR conversion: blocks of one
  magnitude placed at, and one fp32 step below, the points where
  D = floor(2^16 d) changes, with over 2^20 elements per value so every
  16-bit random draw occurs; bit-exact against the oracle's rule r16 < D.
- Device-side guards: group offsets are device data the host cannot check.
  Outputs and inputs are views into larger, sentinel-filled allocations, so
  a stray access stays inside memory the test owns and is detected.
"""
import numpy as np
import pytest

import oracle
from mxfp4_precision_numerics_amd import mx, synth
from tests.gpu_util import dev, dev_bf16, first_mismatch, host, rel_fro

pytestmark = pytest.mark.gpu


def _assert_same(got, want, what):
    mm = first_mismatch(np.asarray(got), np.asarray(want))
    assert mm is None, "%s: first mismatch at %s got %s want %s (%d total)" % ((what,) + mm)


def _padded_codes(torch, rows, row_bytes, ld, fill=0xA5):
    """A code output whose rows are `ld` bytes apart: a row-slice view of a
    sentinel-filled buffer."""
    buf = torch.full((rows, ld), fill, dtype=torch.uint8, device="cuda")
    return buf, buf[:, :row_bytes]


# ---------------------------------------------------------------------------
# Row-wise quantizer: several grid-stride trips, padded rows
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("rows,cols,ld,rnd", [
    (65536, 2880, 0, 0),        # 5.9M blocks: 3 trips, contiguous kernel, RTNE
    (65536, 2880, 0, 1),        #   the same, SR
    (65536, 2880, 1536, 0),     # 3 trips, padded rows (wave-uniform split), RTNE
    (65536, 2880, 1536, 1),     #   the same, SR (the expert step's dY2 launch)
    (65536, 5760, 2944, 1),     # 11.8M blocks: 6 trips, padded rows, SR (dY1)
])
def test_rowwise_multi_trip_full_size_vs_oracle(rows, cols, ld, rnd):
    import torch
    print("rowwise multi-trip", rows, cols, ld, rnd, flush=True)
    x = synth.normal_bf16((rows, cols), 1e-3 if rnd else 1.0, seed=21 + cols + rnd)
    xd = dev_bf16(x)
    if ld:
        buf, codes = _padded_codes(torch, rows, cols // 2, ld)
        c, s = mx.quantize_1d(xd, rnd=rnd, seed=5, stream_id=1, codes=codes)
    else:
        c, s = mx.quantize_1d(xd, rnd=rnd, seed=5, stream_id=1)
    oc, os_ = oracle.quantize_1d(x, rnd=rnd, seed=5, stream=1)
    _assert_same(host(s), os_, "scales")
    _assert_same(host(c.contiguous()), oc, "codes")
    if ld:
        assert bool((buf[:, cols // 2:] == 0xA5).all()), "row padding was written"


def test_rowwise_narrow_padded_rows_multi_trip_vs_oracle():
    """Rows of 3 blocks at a 64-byte pitch (the per-lane row split and carry),
    750,000 rows = 2.25M blocks: two grid-stride trips, RHT + SR."""
    import torch
    rows, cols, ld = 750000, 96, 64
    x = synth.normal_bf16((rows, cols), 1.0, seed=33)
    mask = mx.rht_sign_mask(1)
    buf, codes = _padded_codes(torch, rows, cols // 2, ld)
    c, s = mx.quantize_1d(dev_bf16(x), use_rht=True, sign_mask=mask, rnd=1, seed=9, stream_id=2,
                          codes=codes)
    oc, os_ = oracle.quantize_1d(x, use_rht=True, sign_mask=mask, rnd=1, seed=9, stream=2)
    _assert_same(host(s), os_, "scales")
    _assert_same(host(c.contiguous()), oc, "codes")
    assert bool((buf[:, cols // 2:] == 0xA5).all()), "row padding was written"


# ---------------------------------------------------------------------------
# The hardware SR conversion at the decision boundaries
# ---------------------------------------------------------------------------
def _sr_boundary_matrix(rows_per_value=34, cols=32768):
    """fp32 rows: every 32-block holds 7.0 at position 0 (so the block scale
    is 2^0 and 7 saturates) and one magnitude v elsewhere, with alternating
    signs.  v runs over the grid intervals [0, 0.5), [1, 1.5), [2, 3) and
    [4, 6), at d = D / 2^16 exactly (floor(2^16 d) = D) and at the fp32 value
    just below it (floor = D - 1), for D in {1, 32767, 32768, 65535}, plus d = 0
    exactly.  rows_per_value rows per v: over 2^20 elements each."""
    vals = []
    for lo, step in ((0.0, 0.5), (1.0, 0.5), (2.0, 1.0), (4.0, 2.0)):
        vals.append(np.float32(lo) if lo > 0 else np.float32(2.0 ** -20))   # d = 0 (or tiny)
        for D in (1, 32767, 32768, 65535):
            v = np.float32(lo + step * D / 65536.0)
            assert float(v) == lo + step * D / 65536.0                      # exact in fp32
            vals += [v, np.nextafter(v, np.float32(0))]
    x = np.empty((len(vals) * rows_per_value, cols), dtype=np.float32)
    sign = np.where(np.arange(cols) % 2 == 0, 1.0, -1.0).astype(np.float32)
    for k, v in enumerate(vals):
        x[k * rows_per_value:(k + 1) * rows_per_value] = v * sign
    x[:, ::32] = 7.0
    return x, vals


def test_sr_conversion_at_decision_boundaries():
    x, vals = _sr_boundary_matrix()
    rows, cols = x.shape
    per_value = (x.shape[0] // len(vals)) * cols * 31 // 32
    assert per_value > 2 ** 20
    c, s = mx.quantize_1d(dev(x), rnd=1, seed=12345, stream_id=7)
    oc, os_ = oracle.quantize_1d(x, rnd=1, seed=12345, stream=7)
    _assert_same(host(s), os_, "scales")
    _assert_same(host(c), oc, "codes")
    # the draws behind one value's elements cover all 2^16 values of r16
    seen = np.zeros(65536, dtype=bool)
    L = oracle.lib()
    for i in range(0, 34 * cols):
        if i % 32:
            seen[L.oracle_sr_bits(12345, 7, i)] = True
    assert seen.all(), int((~seen).sum())
    # and each value rounds up in a share D / 2^16 of its elements, within 5
    # sigma (a check that the data sit where intended: the bit-exact
    # comparison above is the test)
    from fractions import Fraction
    grid = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
    nib = np.stack([oc & 0xF, oc >> 4], axis=2).reshape(rows, cols) & 7
    keep = np.arange(cols) % 32 != 0
    per = rows // len(vals)
    for k, v in enumerate(vals):
        a = Fraction(float(v))
        m0 = max(i for i in range(7) if Fraction(grid[i]) <= a)
        D = int((a - Fraction(grid[m0])) / (Fraction(grid[m0 + 1]) - Fraction(grid[m0])) * 65536)
        sel = nib[k * per:(k + 1) * per][:, keep]
        assert set(np.unique(sel)) <= {m0, m0 + 1}, (float(v), np.unique(sel))
        n, up, p = sel.size, int((sel == m0 + 1).sum()), D / 65536.0
        assert abs(up - p * n) <= 5 * np.sqrt(p * (1 - p) * n) + 1, (float(v), D, up, p * n)


# ---------------------------------------------------------------------------
# Guards against malformed device arguments
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("use_rht,rnd", [(False, 0), (True, 1)])
def test_colwise_capacity_below_padded_total_stays_in_bounds(use_rht, rnd):
    """kp smaller than the padded total (a caller error the host cannot see:
    the offsets live on the device).  The kernel writes blocks below kp only,
    identical to the oracle's, and nothing past the outputs."""
    import torch
    counts = [300, 17, 0, 500, 90]
    off = synth.offsets_from_counts(counts)
    rows, cols = int(off[-1]), 160
    x = synth.normal_bf16((rows, cols), 1.0, seed=44)
    total = oracle.padded_total(off)
    kp = 512                                     # < total = 992
    assert kp < total
    mask = mx.rht_sign_mask(5)
    cbuf = torch.full((cols * kp // 2 + 4096,), 0x5A, dtype=torch.uint8, device="cuda")
    sbuf = torch.full((cols * kp // 32 + 4096,), 0x5A, dtype=torch.uint8, device="cuda")
    codes = cbuf[:cols * kp // 2].view(cols, kp // 2)
    scales = sbuf[:cols * kp // 32].view(cols, kp // 32)
    mx.quantize_1d(dev_bf16(x), block_axis=0, group_offsets=dev(off), kp=kp, use_rht=use_rht,
                   sign_mask=mask, rnd=rnd, seed=5, stream_id=3, codes=codes, scales=scales)
    oc, os_ = oracle.quantize_1d(x, block_axis=0, group_offsets=off, kp=kp, use_rht=use_rht,
                                 sign_mask=mask, rnd=rnd, seed=5, stream=3)
    _assert_same(host(scales), os_, "scales")
    _assert_same(host(codes), oc, "codes")
    assert bool((cbuf[cols * kp // 2:] == 0x5A).all()), "codes written past the output"
    assert bool((sbuf[cols * kp // 32:] == 0x5A).all()), "scales written past the output"


@pytest.mark.parametrize("gather", [False, True])
def test_colwise_offsets_past_the_rows_read_as_padding(gather):
    """The last offset exceeds the number of token rows.  Positions past the
    rows are quantized as padding (zeros): the result equals the oracle on x
    extended with zero rows.  x (and the row index) are views into larger
    allocations whose extra rows hold large values, so a read past the rows
    would change the codes instead of faulting."""
    import torch
    rows, cols, extra = 200, 96, 150
    off = np.array([0, 120, rows + extra], dtype=np.int32)
    xall = synth.normal_bf16((rows + extra + 64, cols), 1.0, seed=45)
    xall[rows:] = synth.f32_to_bf16_bits(np.full((extra + 64, cols), 1000.0, np.float32))
    xd = dev_bf16(xall)
    mask = mx.rht_sign_mask(5)
    kp = mx.padded_capacity(rows + extra, 2)
    if gather:
        idx_all = np.arange(rows + extra + 64, dtype=np.int32) % rows
        idx_all[rows:] = rows + 3                     # past-the-end entries point at the 1000s
        idx = np.random.default_rng(3).permutation(rows).astype(np.int32)
        idx_all[:rows] = idx
        ridx = dev(idx_all)[:rows]
        c, s = mx.quantize_1d(xd[:rows], block_axis=0, group_offsets=dev(off), kp=kp, use_rht=True,
                              sign_mask=mask, rnd=1, seed=5, stream_id=2, row_index=ridx)
        src = xall[idx]
    else:
        c, s = mx.quantize_1d(xd[:rows], block_axis=0, group_offsets=dev(off), kp=kp, use_rht=True,
                              sign_mask=mask, rnd=1, seed=5, stream_id=2)
        src = xall[:rows]
    ext = np.concatenate([src, np.zeros((extra, cols), np.uint16)])
    oc, os_ = oracle.quantize_1d(ext, block_axis=0, group_offsets=off, kp=kp, use_rht=True,
                                 sign_mask=mask, rnd=1, seed=5, stream=2)
    total = oracle.padded_total(off)
    _assert_same(host(s)[:, :total // 32], os_[:, :total // 32], "scales")
    _assert_same(host(c)[:, :total // 2], oc[:, :total // 2], "codes")


@pytest.mark.parametrize("gather", [False, True])
def test_gemm_offsets_past_m_are_clamped(gather):
    """Groups along M whose last offset exceeds M: rows past M are neither
    read nor stored.  A, the row index and C are views into larger
    sentinel-filled allocations."""
    import torch
    rng = np.random.default_rng(60)
    M, N, K, extra = 300, 96, 256, 200
    off = np.array([0, 100, M + extra], dtype=np.int32)
    a_rows = 128 if gather else M
    ac = rng.integers(0, 256, (a_rows + extra, K // 2), dtype=np.uint8)
    asc = rng.integers(124, 130, (a_rows + extra, K // 32), dtype=np.uint8)
    bc = rng.integers(0, 256, (2, N, K // 2), dtype=np.uint8)
    bs = rng.integers(124, 130, (2, N, K // 32), dtype=np.uint8)
    idx_all = rng.integers(0, a_rows, M + extra).astype(np.int32)
    idx_all[M:] = a_rows + 5                             # would read the extra A rows
    cbuf = torch.full((M + extra, N), 12345.0, dtype=torch.float32, device="cuda")
    ad, asd = dev(ac), dev(asc)
    c = mx.grouped_gemm(ad[:a_rows], asd[:a_rows], dev(bc), dev(bs), dev(off), M, N, K,
                        a_row_index=dev(idx_all)[:M] if gather else None, out=cbuf[:M])
    torch.cuda.synchronize()
    assert bool((cbuf[M:] == 12345.0).all()), "C written past row M"
    offc = np.array([0, 100, M], dtype=np.int32)
    rows, want = oracle.grouped_gemm(ac[:a_rows], asc[:a_rows], bc, bs, offc, M, N, K,
                                     a_row_index=idx_all[:M] if gather else None)
    got = host(c).astype(np.float64)[rows[:, 1]]
    assert rel_fro(got, want) <= 1e-5


def test_wgrad_offsets_past_k_are_clamped():
    """Groups along K whose last offset exceeds K: no chunk past K is read.
    The operands' code rows are padded (pitch > K/2) with nonzero codes and
    their scales are views into larger buffers, so a read past K would change
    the result instead of faulting."""
    import torch
    rng = np.random.default_rng(61)
    M, N, K = 96, 64, 512
    off = np.array([0, 192, K + 256], dtype=np.int32)
    pitch = K // 2 + 128

    def operand(rows):
        codes = rng.integers(0, 256, (rows, pitch), dtype=np.uint8)
        scales = rng.integers(124, 130, (rows + 4, K // 32), dtype=np.uint8)
        return codes, scales

    ac, asc = operand(M)
    bc, bs = operand(N)
    acd, bcd = dev(ac), dev(bc)
    c = mx.grouped_gemm(acd[:, :K // 2], dev(asc)[:M], bcd[:, :K // 2], dev(bs)[:N], dev(off), M, N, K,
                        group_dim_k=True, out_dtype=torch.float32)
    offc = np.array([0, 192, K], dtype=np.int32)
    rows, want = oracle.grouped_gemm(np.ascontiguousarray(ac[:, :K // 2]), np.ascontiguousarray(asc[:M]),
                                     np.ascontiguousarray(bc[:, :K // 2]), np.ascontiguousarray(bs[:N]),
                                     offc, M, N, K, group_dim_k=True)
    got = host(c)
    for g in range(2):
        sel = rows[:, 0] == g
        assert rel_fro(got[g][rows[sel, 1]].astype(np.float64), want[sel]) <= 1e-5, g


# ---------------------------------------------------------------------------
# One read, both 1x32 layouts (mx_quantize_1d_dual)
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("dt,cols", [("bf16", 96), ("bf16", 160), ("f32", 96), ("bf16", 70 * 32)])
@pytest.mark.parametrize("use_rht,col_rnd,row_rnd", [(True, 1, 1), (True, 1, 0), (False, 0, 1)])
def test_dual_matches_oracle(dt, cols, use_rht, col_rnd, row_rnd):
    """Both outputs of the dual call against the oracle's two quantizations
    (row-wise without the RHT, column-wise with it), ragged groups."""
    import torch
    counts = [45, 0, 32, 7, 300, 1]
    off = synth.offsets_from_counts(counts)
    rows = int(off[-1])
    rng = np.random.default_rng(cols + 3 * use_rht + col_rnd + 7 * row_rnd)
    xf = (rng.standard_normal((rows, cols)) * np.exp2(rng.integers(-6, 6, (1, cols)))).astype(np.float32)
    x = xf if dt == "f32" else synth.f32_to_bf16_bits(xf)
    xd = dev(x) if dt == "f32" else dev_bf16(x)
    mask = mx.rht_sign_mask(5)
    kp = mx.padded_capacity(rows, len(counts))
    buf, rcodes = _padded_codes(torch, rows, cols // 2, (cols // 2 + 127) // 128 * 128 + 16)
    cc, cs, rc, rs = mx.quantize_1d_dual(xd, dev(off), kp=kp, use_rht=use_rht, sign_mask=mask, col_rnd=col_rnd,
                                         col_stream_id=3, row_rnd=row_rnd, row_stream_id=0, seed=5,
                                         row_index_base=64, row_codes=rcodes)
    oc, os_ = oracle.quantize_1d(x, block_axis=0, group_offsets=off, kp=kp, use_rht=use_rht, sign_mask=mask,
                                 rnd=col_rnd, seed=5, stream=3)
    total = oracle.padded_total(off)
    _assert_same(host(cs)[:, :total // 32], os_[:, :total // 32], "column scales")
    _assert_same(host(cc)[:, :total // 2], oc[:, :total // 2], "column codes")
    orc, ors = oracle.quantize_1d(x, rnd=row_rnd, seed=5, stream=0, index_base=64)
    _assert_same(host(rs), ors, "row scales")
    _assert_same(host(rc.contiguous()), orc, "row codes")
    assert bool((buf[:, cols // 2:] == 0xA5).all()), "row padding was written"


@pytest.mark.parametrize("cols,row_rnd", [(2880, 0), (2880, 1), (5760, 1)])
def test_dual_full_size_equals_two_calls(cols, row_rnd):
    """The expert step's h (row RTNE), dY2 and dY1 (row SR) at 65,536 routed
    rows, 32 Zipf groups, padded code rows: the dual call equals the two
    separate calls everywhere (compared on the device)."""
    import torch
    counts = synth.zipf_counts()
    off = dev(synth.offsets_from_counts(counts))
    rows = 65536
    g = torch.Generator(device="cuda").manual_seed(cols + row_rnd)
    x = (torch.randn(rows, cols, device="cuda", generator=g) * 1e-3).to(torch.bfloat16)
    kp = mx.padded_capacity(rows, 32)
    mask = mx.rht_sign_mask(5)
    ldp = (cols // 2 + 127) // 128 * 128
    rbuf = torch.zeros(rows, ldp, dtype=torch.uint8, device="cuda")
    cc, cs, rc, rs = mx.quantize_1d_dual(x, off, kp=kp, use_rht=True, sign_mask=mask, col_rnd=1, col_stream_id=5,
                                         row_rnd=row_rnd, row_stream_id=1, seed=5, row_codes=rbuf[:, :cols // 2])
    cc2, cs2 = mx.quantize_1d(x, block_axis=0, group_offsets=off, kp=kp, use_rht=True, sign_mask=mask, rnd=1,
                              seed=5, stream_id=5)
    rc2, rs2 = mx.quantize_1d(x, rnd=row_rnd, seed=5, stream_id=1)
    total = int(sum((int(n) + 31) // 32 * 32 for n in counts))
    assert torch.equal(cc[:, :total // 2], cc2[:, :total // 2]) and torch.equal(cs[:, :total // 32], cs2[:, :total // 32])
    assert torch.equal(rc.contiguous(), rc2) and torch.equal(rs, rs2)


JUNK = 0xA7


@pytest.mark.parametrize("dt,cols,row_rnd", [("bf16", 96, 1), ("bf16", 352, 0), ("f32", 160, 1)])
def test_dual_staged_pad256_matches_oracle(dt, cols, row_rnd):
    """The dual call with both outputs' scales in the staged order and the
    column-wise groups padded to 256 tokens (the layouts the expert step's
    GEMMs read), against the oracle: codes bit for bit, every staged scale
    slot the oracle maps equal to its byte, the others untouched."""
    import torch
    counts = [300, 0, 17, 700, 256, 1]
    off = synth.offsets_from_counts(counts)
    rows, G = int(off[-1]), len(counts)
    rng = np.random.default_rng(cols + 11 * row_rnd)
    xf = (rng.standard_normal((rows, cols)) * np.exp2(rng.integers(-6, 6, (1, cols)))).astype(np.float32)
    x = xf if dt == "f32" else synth.f32_to_bf16_bits(xf)
    xd = dev(x) if dt == "f32" else dev_bf16(x)
    mask = mx.rht_sign_mask(6)
    kp = mx.padded_capacity(rows, G, 256)
    Sc, Sr = kp // 256 + G, (cols + 255) // 256
    csb = torch.full((Sc, cols, 8), JUNK, dtype=torch.uint8, device="cuda")
    rsb = torch.full((Sr, rows, 8), JUNK, dtype=torch.uint8, device="cuda")
    buf, rcodes = _padded_codes(torch, rows, cols // 2, (cols // 2 + 127) // 128 * 128 + 16)
    cc, cs, rc, rs = mx.quantize_1d_dual(xd, dev(off), kp=kp, use_rht=True, sign_mask=mask, col_rnd=1,
                                         col_stream_id=2, row_rnd=row_rnd, row_stream_id=1, seed=9,
                                         row_codes=rcodes, col_scales=csb, row_scales=rsb, staged=True,
                                         group_pad=256)
    oc, os_ = oracle.quantize_1d(x, block_axis=0, group_offsets=off, kp=kp, use_rht=True, sign_mask=mask, rnd=1,
                                 seed=9, stream=2, group_pad=256)
    tot = oracle.padded_total(off, 256)
    _assert_same(host(cc)[:, :tot // 2], oc[:, :tot // 2], "column codes")
    want = oracle.stage_scales(os_, off, stages=Sc, fill=JUNK, group_pad=256)
    m = oracle.stage_scales(np.ones_like(os_), off, stages=Sc, fill=0, group_pad=256).astype(bool)
    got = host(cs)
    assert np.array_equal(got[m], want[m]) and np.all(got[~m] == JUNK), "column scales"
    orc, ors = oracle.quantize_1d(x, rnd=row_rnd, seed=9, stream=1)
    _assert_same(host(rc.contiguous()), orc, "row codes")
    want = oracle.stage_scales(ors, stages=Sr, fill=JUNK)
    m = oracle.stage_scales(np.ones_like(ors), stages=Sr, fill=0).astype(bool)
    got = host(rs)
    assert np.array_equal(got[m], want[m]) and np.all(got[~m] == JUNK), "row scales"
    assert bool((buf[:, cols // 2:] == 0xA5).all()), "row padding was written"


@pytest.mark.parametrize("cols,row_rnd", [(2880, 0), (5760, 1)])
def test_dual_full_size_staged_pad256_equals_two_calls(cols, row_rnd):
    """The expert step's layouts at full size (65,536 routed rows, 32 Zipf
    groups padded to 256 tokens, staged scales, padded code rows): the dual
    call equals the two separate calls the step would otherwise make."""
    import torch
    counts = synth.zipf_counts()
    off = dev(synth.offsets_from_counts(counts))
    rows = 65536
    g = torch.Generator(device="cuda").manual_seed(cols + 7 * row_rnd)
    x = (torch.randn(rows, cols, device="cuda", generator=g) * 1e-3).to(torch.bfloat16)
    kp = mx.padded_capacity(rows, 32, 256)
    mask = mx.rht_sign_mask(5)
    ldp = (cols // 2 + 127) // 128 * 128
    rbuf = torch.zeros(rows, ldp, dtype=torch.uint8, device="cuda")
    # staged row scales: the slots past a row's last block are never written
    Sr = (cols + 255) // 256
    rsb = torch.full((Sr, rows, 8), JUNK, dtype=torch.uint8, device="cuda")
    rsb2 = torch.full((Sr, rows, 8), JUNK, dtype=torch.uint8, device="cuda")
    cc, cs, rc, rs = mx.quantize_1d_dual(x, off, kp=kp, use_rht=True, sign_mask=mask, col_rnd=1, col_stream_id=5,
                                         row_rnd=row_rnd, row_stream_id=1, seed=5, row_codes=rbuf[:, :cols // 2],
                                         row_scales=rsb, staged=True, group_pad=256)
    cc2, cs2 = mx.quantize_1d(x, block_axis=0, group_offsets=off, kp=kp, use_rht=True, sign_mask=mask, rnd=1,
                              seed=5, stream_id=5, staged=True, group_pad=256)
    rbuf2 = torch.zeros(rows, ldp, dtype=torch.uint8, device="cuda")
    rc2, rs2 = mx.quantize_1d(x, rnd=row_rnd, seed=5, stream_id=1, staged=True, codes=rbuf2[:, :cols // 2],
                              scales=rsb2)
    pad = (np.asarray(counts) + 255) // 256 * 256
    total = int(pad.sum())
    assert torch.equal(cc[:, :total // 2], cc2[:, :total // 2])
    # staged column scales: compare the slots the groups' blocks occupy
    S = kp // 256 + 32
    m = torch.from_numpy(oracle.stage_scales(np.ones((cols, total // 32), np.uint8),
                                             synth.offsets_from_counts(counts), stages=S, fill=0,
                                             group_pad=256).astype(bool)).cuda()
    assert torch.equal(cs[m], cs2[m])
    assert torch.equal(rbuf, rbuf2) and torch.equal(rs, rs2)


@pytest.mark.parametrize("dt,row_rnd", [("f32", 0), ("bf16", 1)])
def test_dual_nonfinite_blocks_match_oracle(dt, row_rnd):
    """Blocks holding Inf, -Inf or NaN (and finite values whose RHT sums
    overflow) in the dual call: both outputs take scale 0xFF and zero codes
    exactly where the oracle does.  The row pass undoes the RHT's signs on
    its codes, so this checks that a non-finite block's codes are zeroed
    after that flip."""
    rng = np.random.default_rng(21)
    counts = [64, 40, 96]
    off = synth.offsets_from_counts(counts)
    rows, cols = int(off[-1]), 96
    x = rng.standard_normal((rows, cols)).astype(np.float32)
    x[3, 0] = np.inf
    x[40, 5] = -np.inf
    x[70, 33] = np.nan
    x[100:104, 64] = 3.0e38
    x = synth.f32_to_bf16_bits(x) if dt == "bf16" else x
    xd = dev_bf16(x) if dt == "bf16" else dev(x)
    kp = mx.padded_capacity(rows, len(counts))
    mask = 0xFFFFFFFF          # every sign flipped: every row-wise code goes through the flip
    cc, cs, rc, rs = mx.quantize_1d_dual(xd, dev(off), kp=kp, use_rht=True, sign_mask=mask, col_rnd=1,
                                         col_stream_id=2, row_rnd=row_rnd, row_stream_id=0, seed=4)
    oc, os_ = oracle.quantize_1d(x, block_axis=0, group_offsets=off, kp=kp, use_rht=True, sign_mask=mask, rnd=1,
                                 seed=4, stream=2)
    total = oracle.padded_total(off)
    _assert_same(host(cs)[:, :total // 32], os_[:, :total // 32], "column scales")
    _assert_same(host(cc)[:, :total // 2], oc[:, :total // 2], "column codes")
    orc, ors = oracle.quantize_1d(x, rnd=row_rnd, seed=4, stream=0)
    assert np.count_nonzero(ors == 0xFF) >= 3
    _assert_same(host(rs), ors, "row scales")
    _assert_same(host(rc), orc, "row codes")
