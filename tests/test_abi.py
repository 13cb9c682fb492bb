"""C-ABI checks that need no GPU: the library loads, exports every declared
symbol, and rejects bad arguments on the host before any launch."""
import ctypes

import pytest

import oracle
from mxfp4_precision_numerics_amd import mx


@pytest.fixture(scope="module")
def L():
    return mx.lib()


def test_every_declared_symbol_is_exported(L):
    names = mx.declared_functions()
    assert set(names) >= {"mx_rht", "mx_quantize_1d", "mx_quantize_2d", "mx_quantize_2d_deosc", "mx_quantize_1d_ex",
                          "mx_dequantize_1d_ex", "mx_quantize_1d_dual", "mx_dequantize",
                          "mx_grouped_gemm", "mx_grouped_gemm_q", "mx_rht_sign_mask", "mx_status_str",
                          "mx_version"}
    for n in names:
        assert hasattr(L, n), n


def test_status_strings(L):
    for code, name in mx.STATUS.items():
        assert L.mx_status_str(code).decode() == name
    assert L.mx_version() >= 1


def test_sign_mask_matches_oracle(L):
    for seed in (0, 1, 2, 5, 123456789, 2**63 + 11):
        assert L.mx_rht_sign_mask(seed) == oracle.rht_sign_mask(seed)


FAKE = 0x1000  # a 16-byte aligned non-null address; never dereferenced (validation fails first)


def test_quantize_1d_validation(L):
    q = L.mx_quantize_1d
    # cols not a multiple of 32
    assert q(FAKE, mx.MX_BF16, 4, 33, 1, None, 0, 0, None, 0, 0, 0, 0, 0, 0, FAKE, 0, FAKE, None) == 2
    # bad dtype, bad rounding mode
    assert q(FAKE, 7, 4, 32, 1, None, 0, 0, None, 0, 0, 0, 0, 0, 0, FAKE, 0, FAKE, None) == 4
    assert q(FAKE, mx.MX_BF16, 4, 32, 1, None, 0, 0, None, 0, 0, 3, 0, 0, 0, FAKE, 0, FAKE, None) == 5
    # null pointers
    assert q(None, mx.MX_BF16, 4, 32, 1, None, 0, 0, None, 0, 0, 0, 0, 0, 0, FAKE, 0, FAKE, None) == 1
    assert q(FAKE, mx.MX_BF16, 4, 32, 1, None, 0, 0, None, 0, 0, 0, 0, 0, 0, None, 0, FAKE, None) == 1
    # misaligned input
    assert q(FAKE + 2, mx.MX_BF16, 4, 32, 1, None, 0, 0, None, 0, 0, 0, 0, 0, 0, FAKE, 0, FAKE, None) == 3
    # index base not a multiple of 32
    assert q(FAKE, mx.MX_BF16, 4, 32, 1, None, 0, 0, None, 0, 0, 1, 7, 0, 8, FAKE, 0, FAKE, None) == 2
    # row-wise with groups given
    assert q(FAKE, mx.MX_BF16, 4, 32, 1, FAKE, 2, 0, None, 0, 0, 0, 0, 0, 0, FAKE, 0, FAKE, None) == 2
    # column-wise: missing offsets, bad kp, bad group count
    assert q(FAKE, mx.MX_BF16, 4, 32, 0, None, 2, 64, None, 0, 0, 0, 0, 0, 0, FAKE, 0, FAKE, None) == 1
    assert q(FAKE, mx.MX_BF16, 4, 32, 0, FAKE, 2, 40, None, 0, 0, 0, 0, 0, 0, FAKE, 0, FAKE, None) == 2
    assert q(FAKE, mx.MX_BF16, 4, 32, 0, FAKE, 0, 64, None, 0, 0, 0, 0, 0, 0, FAKE, 0, FAKE, None) == 2
    # column-wise: one row of x over 4 GiB (2^31 bf16 columns)
    assert q(FAKE, mx.MX_BF16, 4, 2 ** 31, 0, FAKE, 2, 64, None, 0, 0, 0, 0, 0, 0, FAKE, 0, FAKE, None) == 2
    # a row gather is column-wise only
    assert q(FAKE, mx.MX_BF16, 4, 32, 1, None, 0, 0, FAKE, 0, 0, 0, 0, 0, 0, FAKE, 0, FAKE, None) == 5
    # code row pitch: below cols / 2, not a multiple of 16; column-wise other than kp / 2
    assert q(FAKE, mx.MX_BF16, 4, 64, 1, None, 0, 0, None, 0, 0, 0, 0, 0, 0, FAKE, 16, FAKE, None) == 2
    assert q(FAKE, mx.MX_BF16, 4, 64, 1, None, 0, 0, None, 0, 0, 0, 0, 0, 0, FAKE, 40, FAKE, None) == 2
    assert q(FAKE, mx.MX_BF16, 4, 32, 0, FAKE, 2, 64, None, 0, 0, 0, 0, 0, 0, FAKE, 48, FAKE, None) == 2
    # staged scales keep the axis checks; an unknown axis value stays a shape error
    assert q(FAKE, mx.MX_BF16, 4, 32, 1 | mx.SCALES_STAGED, FAKE, 2, 0, None, 0, 0, 0, 0, 0, 0, FAKE, 0, FAKE,
             None) == 2
    assert q(FAKE, mx.MX_BF16, 4, 33, 1 | mx.SCALES_STAGED, None, 0, 0, None, 0, 0, 0, 0, 0, 0, FAKE, 0, FAKE,
             None) == 2
    assert q(FAKE, mx.MX_BF16, 4, 32, 8, None, 0, 0, None, 0, 0, 0, 0, 0, 0, FAKE, 0, FAKE, None) == 2
    # groups padded to 256 tokens: column-wise only
    assert q(FAKE, mx.MX_BF16, 4, 32, 1 | mx.GROUPS_PAD256, None, 0, 0, None, 0, 0, 0, 0, 0, 0, FAKE, 0, FAKE,
             None) == 2
    assert q(FAKE, mx.MX_BF16, 4, 32, 0 | mx.SCALES_STAGED, FAKE, 2, 40, None, 0, 0, 0, 0, 0, 0, FAKE, 0, FAKE,
             None) == 2
    # empty input is a no-op that launches nothing
    assert q(None, mx.MX_BF16, 0, 32, 1, None, 0, 0, None, 0, 0, 0, 0, 0, 0, None, 0, None, None) == 0


def test_quantize_2d_validation(L):
    q = L.mx_quantize_2d
    assert q(FAKE, mx.MX_BF16, 1, 48, 32, FAKE, 0, FAKE, None, 0, None, None) == 2
    assert q(FAKE, mx.MX_BF16, 1, 32, 32, None, 0, None, None, 0, None, None) == 1
    assert q(FAKE, mx.MX_BF16, 1, 32, 32, FAKE, 0, None, None, 0, None, None) == 1
    assert q(FAKE, 9, 1, 32, 32, FAKE, 0, FAKE, None, 0, None, None) == 4
    assert q(FAKE + 8, mx.MX_BF16, 1, 32, 32, FAKE, 0, FAKE, None, 0, None, None) == 3
    # code row pitches: W rows below cols / 2, W^T rows not a multiple of 16
    assert q(FAKE, mx.MX_BF16, 1, 64, 64, FAKE, 16, FAKE, None, 0, None, None) == 2
    assert q(FAKE, mx.MX_BF16, 1, 64, 64, None, 0, None, FAKE, 40, FAKE, None) == 2
    assert q(FAKE, mx.MX_BF16, 0, 32, 32, FAKE, 0, FAKE, None, 0, None, None) == 0
    # empty: no pointer is looked at (zero-size tensors may have null pointers)
    assert q(None, mx.MX_BF16, 0, 32, 32, None, 0, None, None, 0, None, None) == 0


def test_quantize_2d_deosc_validation(L):
    q = L.mx_quantize_2d_deosc
    ok = dict(w=FAKE, wt=mx.MX_F32, b=1, r=64, c=64, pc=FAKE, pld=0, ps=FAKE, m=8, cd=FAKE, ld=0,
              sc=FAKE, ct=None, ldt=0, st=None, fl=FAKE, s=None)

    def call(**kw):
        a = dict(ok, **kw)
        return q(a["w"], a["wt"], a["b"], a["r"], a["c"], a["pc"], a["pld"], a["ps"], a["m"], a["cd"], a["ld"],
                 a["sc"], a["ct"], a["ldt"], a["st"], a["fl"], a["s"])

    assert call(r=48) == 2                       # rows not a multiple of 32
    assert call(m=32) == 2 and call(m=-1) == 2   # margin outside [0, 31]
    assert call(wt=3) == 4
    assert call(pc=None) == 1 and call(ps=None) == 1 and call(cd=None) == 1 and call(sc=None) == 1
    assert call(ct=FAKE) == 1                    # transposed codes without their scales
    assert call(w=FAKE + 4) == 3 and call(pc=FAKE + 8) == 3 and call(fl=FAKE + 1) == 3
    assert call(pld=16) == 2 and call(ld=40) == 2
    assert call(pc=FAKE, cd=FAKE, pld=64, ld=0) == 2    # in place with another pitch
    assert call(b=0, w=None, pc=None, ps=None, cd=None, sc=None) == 0


def test_study_variant_validation(L):
    q = L.mx_quantize_1d_ex
    args = [FAKE, mx.MX_F32, 4, 256, 0, 0, 0, 0, 0, 0, 1.0, 128, FAKE, FAKE, FAKE, None]

    def call(i_vals):
        a = list(args)
        for i, v in i_vals:
            a[i] = v
        return q(*a)

    assert call([(10, -0.5)]) == 2 and call([(10, 1.5)]) == 2 and call([(10, float("nan"))]) == 2
    assert call([(11, 96)]) == 2 and call([(11, 48)]) == 2 and call([(11, -32)]) == 2
    assert call([(14, None)]) == 1 and call([(12, None)]) == 1
    assert call([(14, FAKE + 2)]) == 3 and call([(0, FAKE + 4)]) == 3
    assert call([(1, 5)]) == 4 and call([(6, 2)]) == 5 and call([(3, 48)]) == 2
    assert call([(2, 0), (0, None), (12, None), (13, None), (14, None)]) == 0
    d = L.mx_dequantize_1d_ex
    assert d(FAKE, FAKE, None, 4, 256, 128, FAKE, None) == 1
    assert d(FAKE, FAKE, FAKE, 4, 256, 96, FAKE, None) == 2
    assert d(FAKE + 4, FAKE, None, 4, 256, 0, FAKE, None) == 3


def test_quantize_1d_dual_validation(L):
    q = L.mx_quantize_1d_dual
    args = [FAKE, mx.MX_BF16, 64, 96, FAKE, 2, 128, 1, 0, 1, 0, 0, FAKE, FAKE, 1, 0, 0, FAKE, 0, FAKE, 0, 0, None]

    def call(i_vals):
        a = list(args)
        for i, v in i_vals:
            a[i] = v
        return q(*a)

    assert call([(3, 48)]) == 2                     # cols not a multiple of 32
    assert call([(6, 40)]) == 2 and call([(5, 0)]) == 2
    assert call([(11, 16)]) == 2 and call([(16, 8)]) == 2     # index bases
    assert call([(18, 16)]) == 2 and call([(18, 40)]) == 2    # row pitch
    assert call([(9, 3)]) == 5 and call([(14, 3)]) == 5       # rounding modes
    assert call([(1, 2)]) == 4
    assert call([(4, None)]) == 1 and call([(17, None)]) == 1 and call([(19, None)]) == 1
    assert call([(0, FAKE + 2)]) == 3 and call([(17, FAKE + 8)]) == 3
    assert call([(2, 0), (0, None), (12, None), (13, None), (17, None), (19, None)]) == 0
    assert call([(21, 8)]) == 5 and call([(21, 1)]) == 5      # layout flags: staged and pad256 only
    assert call([(21, mx.SCALES_STAGED | mx.GROUPS_PAD256), (2, 0), (0, None), (12, None), (13, None),
                 (17, None), (19, None)]) == 0
    # staged: the row-wise order's 32-bit offsets (ceil(cols / 256) * rows * 8 bytes)
    assert call([(21, mx.SCALES_STAGED), (2, 2 ** 31), (3, 256)]) == 2


def test_dequantize_validation(L):
    d = L.mx_dequantize
    assert d(FAKE, 0, FAKE, 1, 4, 48, 1, FAKE, mx.MX_F32, None) == 2
    assert d(FAKE, 0, FAKE, 1, 4, 32, 16, FAKE, mx.MX_F32, None) == 2
    assert d(FAKE, 0, FAKE, 1, 40, 32, 32, FAKE, mx.MX_F32, None) == 2
    assert d(FAKE, 0, None, 1, 4, 32, 1, FAKE, mx.MX_F32, None) == 1
    assert d(FAKE, 0, FAKE, 1, 4, 32, 1, FAKE, 5, None) == 4
    # code row pitch below cols / 2
    assert d(FAKE, 16, FAKE, 1, 4, 64, 1, FAKE, mx.MX_F32, None) == 2


def test_rht_validation(L):
    r = L.mx_rht
    assert r(FAKE, mx.MX_F32, FAKE, 4, 48, 0, 0, None) == 2
    assert r(None, mx.MX_F32, FAKE, 4, 32, 0, 0, None) == 1
    assert r(FAKE, mx.MX_F32, FAKE + 4, 4, 32, 0, 0, None) == 3
    assert r(FAKE, mx.MX_F32, FAKE, 0, 32, 0, 0, None) == 0


def test_gemm_validation(L):
    g = L.mx_grouped_gemm
    args = dict(M=64, N=64, K=64)

    def call(**kw):
        a = dict(a_codes=FAKE, a_ld=0, a_scales=FAKE, a_row_index=None, b_codes=FAKE, b_ld=0, b_scales=FAKE,
                 b_scale_2d=0, off=FAKE, G=1, gk=0, M=64, N=64, K=64, alpha=1.0, c=FAKE,
                 ct=mx.MX_BF16)
        a.update(kw)
        return g(a["a_codes"], a["a_ld"], a["a_scales"], a["a_row_index"], a["b_codes"], a["b_ld"],
                 a["b_scales"], a["b_scale_2d"], a["off"], a["G"], a["gk"], a["M"], a["N"], a["K"],
                 ctypes.c_float(a["alpha"]), a["c"], a["ct"], None)

    assert call(K=48) == 2
    assert call(N=48) == 2
    assert call(G=0) == 2
    assert call(gk=2) == 2
    assert call(off=None) == 1
    assert call(c=None) == 1
    assert call(ct=3) == 4
    assert call(a_codes=FAKE + 1) == 3
    assert call(gk=1, b_scale_2d=1) == 5
    assert call(gk=1, a_row_index=FAKE) == 5
    # code row pitches: below K / 2, not a multiple of 16
    assert call(a_ld=16) == 2
    assert call(b_ld=40) == 2
    # B group of N rows at the pitch beyond 4 GiB - 1
    assert call(N=2**20, K=64, b_ld=2**13) == 2
    # scale flags: unknown bits; staged scales with groups along K need
    # fewer than 64 groups and 4-byte aligned scales; along M they need 2D
    # B scales and no row index
    S, B2 = mx.SCALES_STAGED, mx.SCALES_B_2D
    assert call(b_scale_2d=4) == 5
    assert call(gk=1, b_scale_2d=S, G=64) == 5
    assert call(gk=1, b_scale_2d=S, a_scales=FAKE + 2) == 3
    assert call(gk=1, b_scale_2d=S, b_scales=FAKE + 1) == 3
    assert call(b_scale_2d=S) == 5
    assert call(b_scale_2d=S | B2, a_row_index=FAKE) == 5
    assert call(b_scale_2d=S | B2, a_scales=FAKE + 2) == 3
    # staged scales addressed past 4 GiB: (K/256 + G + 1) * 8 * rows
    assert call(gk=1, b_scale_2d=S, M=64, N=2**23, K=64, G=63) == 2
    assert call(M=0) == 0


def test_gemm_q_validation(L):
    g = L.mx_grouped_gemm_q

    def call(**kw):
        a = dict(a_codes=FAKE, a_ld=0, a_scales=FAKE, a_row_index=None, b_codes=FAKE, b_ld=0, b_scales=FAKE,
                 b_scale_2d=0, off=FAKE, G=1, M=64, N=64, K=64, alpha=1.0, c=FAKE, qc=FAKE, qc_ld=0, qs=FAKE)
        a.update(kw)
        return g(a["a_codes"], a["a_ld"], a["a_scales"], a["a_row_index"], a["b_codes"], a["b_ld"],
                 a["b_scales"], a["b_scale_2d"], a["off"], a["G"], a["M"], a["N"], a["K"],
                 ctypes.c_float(a["alpha"]), a["c"], a["qc"], a["qc_ld"], a["qs"], None)

    assert call(K=48) == 2
    assert call(N=48) == 2
    assert call(G=0) == 2
    assert call(off=None) == 1
    assert call(qc=None) == 1
    assert call(qs=None) == 1
    assert call(a_codes=FAKE + 1) == 3
    assert call(qc=FAKE + 8) == 3
    assert call(c=FAKE + 2) == 3
    # codes of M x N / 2 bytes beyond 4 GiB - 1
    assert call(M=2**20, N=2**13, K=64) == 2
    # output code pitch: below N / 2, not a multiple of 16, M rows of it beyond 4 GiB - 1
    assert call(qc_ld=16) == 2
    assert call(qc_ld=40) == 3
    assert call(M=2**20, N=64, qc_ld=2**12) == 2
    # staged A scales need 2D B scales; unknown flag bits
    assert call(b_scale_2d=mx.SCALES_STAGED) == 5
    assert call(b_scale_2d=8) == 5
    assert call(M=0) == 0


def test_output_buffer_checks():
    """Caller-provided outputs are checked against the shape and dtype the
    library writes before any call (the shape and dtype checks come before
    the device check, so they run on the CPU)."""
    import torch
    u8 = torch.uint8
    with pytest.raises(ValueError, match="expected shape"):
        mx._shaped(torch.empty(3, 4, dtype=u8), (3, 5), u8, "codes", pitched=True)
    with pytest.raises(ValueError, match="expected shape"):
        mx._shaped(torch.empty(2, 3, 4, dtype=u8), (1, 3, 4), u8, "codes")
    with pytest.raises(TypeError, match="expected"):
        mx._shaped(torch.empty(3, 4, dtype=torch.float32), (3, 4), torch.bfloat16, "out")
    # right shape (a leading batch of 1 may be left out) and dtype: only the
    # device check remains
    with pytest.raises(ValueError, match="device"):
        mx._shaped(torch.empty(3, 4, dtype=u8), (1, 3, 4), u8, "codes", pitched=True)


def test_index_vectors_are_checked():
    """Group offsets and row indices must be 1-D int32 (an int64 tensor would
    be read as pairs of int32 words); offsets need at least two entries.
    These checks come before the device check, so they run on the CPU."""
    import torch
    with pytest.raises(ValueError, match="int32"):
        mx._index_vector(torch.zeros(3, dtype=torch.int64), "group_offsets", min_numel=2)
    with pytest.raises(ValueError, match="int32"):
        mx._index_vector(torch.zeros(1, dtype=torch.int32), "group_offsets", min_numel=2)
    with pytest.raises(ValueError, match="int32"):
        mx._index_vector(torch.zeros(2, 2, dtype=torch.int32), "row_index")
    with pytest.raises(ValueError, match="device"):
        mx._index_vector(torch.zeros(2, dtype=torch.int32), "row_index")
    # rht: a caller-provided output must be fp32 of x's shape
    with pytest.raises(TypeError, match="float32"):
        mx._shaped(torch.empty(4, 32, dtype=torch.bfloat16), (4, 32), torch.float32, "out")
