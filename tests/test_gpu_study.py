"""GPU parity of the study variants of the row quantizer (outlier clipping
and macro-block scaling, mx_quantize_1d_ex / mx_dequantize_1d_ex) against
the oracle: codes, scales, macro multipliers and the fp32 decode, bit for
bit."""
import numpy as np
import pytest

import oracle
from mxfp4_precision_numerics_amd import mx, synth
from tests.gpu_util import dev, dev_bf16, first_mismatch, host

pytestmark = pytest.mark.gpu


def _assert_same(got, want, what):
    mm = first_mismatch(np.asarray(got), np.asarray(want))
    assert mm is None, "%s: first mismatch at %s got %s want %s (%d total)" % ((what,) + mm)


def _data(rows, cols, seed, dt):
    x = synth.channel_scaled_activations(rows=rows, cols=cols, seed=seed)
    xf = synth.bf16_bits_to_f32(x)
    flat = xf.reshape(-1)
    rng = np.random.default_rng(seed)
    pos = rng.choice(flat.size, max(1, flat.size // 1000), replace=False)
    flat[pos] *= 50.0                                   # outliers
    if dt == "bf16":
        b = synth.f32_to_bf16_bits(xf)
        return b, dev_bf16(b)
    return xf, dev(xf)


@pytest.mark.parametrize("dt", ["bf16", "f32"])
@pytest.mark.parametrize("use_rht,rnd", [(False, 0), (True, 1)])
@pytest.mark.parametrize("clip,bm", [(1.0, 0), (0.75, 0), (0.5, 0), (0.0, 0), (1.0, 160), (0.875, 320),
                                     (1.0, 2880), (0.0, 320)])
def test_study_variants_parity(dt, use_rht, rnd, clip, bm):
    rows, cols = 37, 2880
    xh, xd = _data(rows, cols, 7, dt)
    mask = mx.rht_sign_mask(1)
    c, s, mr = mx.quantize_1d_ex(xd, use_rht=use_rht, sign_mask=mask, rnd=rnd, seed=3, stream_id=1,
                                 clip_ratio=clip, macro_block=bm)
    oc, os_, omr = oracle.quantize_1d_ex(xh, use_rht=use_rht, sign_mask=mask, rnd=rnd, seed=3, stream=1,
                                         clip_ratio=clip, macro_block=bm)
    if bm:
        _assert_same(host(mr), omr, "macro_r")
    _assert_same(host(s), os_, "scales")
    _assert_same(host(c), oc, "codes")
    y = mx.dequantize_1d_ex(c, s, mr, macro_block=bm)
    _assert_same(host(y), oracle.dequantize_1d_ex(oc, os_, omr, macro_block=bm), "decoded")


def test_search_on_clippable_blocks():
    """Blocks built so that clipping a binade pays (a lone maximum just above
    a power of two) mixed with Gaussian ones: the search takes X - 1 on
    some, bit for bit as the oracle."""
    rng = np.random.default_rng(4)
    x = (rng.standard_normal((256, 512)) * np.exp2(rng.integers(-8, 8, (256, 1)))).astype(np.float32)
    blocks = x.reshape(-1, 32)
    for b in range(0, blocks.shape[0], 2):
        k = float(np.exp2(rng.integers(-6, 6)))
        blocks[b] = rng.uniform(0.2, 0.35, 32).astype(np.float32) * k * rng.choice([-1, 1], 32)
        blocks[b, rng.integers(0, 32)] = (4.0 + float(rng.uniform(0, 0.5))) * k
    for rnd in (0, 1):
        c, s, _ = mx.quantize_1d_ex(dev(x), rnd=rnd, seed=6, clip_ratio=0.0)
        oc, os_, _ = oracle.quantize_1d_ex(x, rnd=rnd, seed=6, clip_ratio=0.0)
        _assert_same(host(s), os_, "scales")
        _assert_same(host(c), oc, "codes")
    plain = oracle.quantize_1d_ex(x)[1]
    assert np.any(os_ != plain)


def test_study_plain_case_equals_the_row_quantizer():
    xh, xd = _data(64, 512, 9, "bf16")
    c, s, _ = mx.quantize_1d_ex(xd, rnd=1, seed=2)
    c2, s2 = mx.quantize_1d(xd, rnd=1, seed=2)
    _assert_same(host(c), host(c2), "codes")
    _assert_same(host(s), host(s2), "scales")


def test_study_full_size_activations():
    """16384 x 2880 bf16 activations with 0.1% outliers, RHT + SR, rho 0.75,
    macro-blocks of 320: the whole matrix against the oracle."""
    xh, xd = _data(16384, 2880, 1, "bf16")
    mask = mx.rht_sign_mask(1)
    c, s, mr = mx.quantize_1d_ex(xd, use_rht=True, sign_mask=mask, rnd=1, seed=2, clip_ratio=0.75,
                                 macro_block=320)
    oc, os_, omr = oracle.quantize_1d_ex(xh, use_rht=True, sign_mask=mask, rnd=1, seed=2, clip_ratio=0.75,
                                         macro_block=320)
    _assert_same(host(mr), omr, "macro_r")
    _assert_same(host(s), os_, "scales")
    _assert_same(host(c), oc, "codes")
