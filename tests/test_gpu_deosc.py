"""GPU parity of the weight de-oscillation quantizer (mx_quantize_2d_deosc)
against the oracle: codes and scales of both layouts and the per-tile flip
counts, bit for bit.  The previous state comes from the oracle's own
quantization of a nearby weight tensor, or from the kernel's previous call
along a master-weight trajectory (the state carried on the device, checked
against the oracle carrying its own)."""
import numpy as np
import pytest

import oracle
from mxfp4_precision_numerics_amd import mx, synth
from tests.gpu_util import dev, dev_bf16, first_mismatch, host

pytestmark = pytest.mark.gpu


def _assert_same(got, want, what):
    mm = first_mismatch(np.asarray(got), np.asarray(want))
    assert mm is None, "%s: first mismatch at %s got %s want %s (%d total)" % ((what,) + mm)


def _flips(t):
    return host(t).view(np.uint16)


def _check(got, want, tag=""):
    names = ("codes", "scales", "codes_t", "scales_t")
    for g, w, n in zip(got[:4], want[:4], names):
        _assert_same(host(g), w, tag + n)
    _assert_same(_flips(got[4]), want[4], tag + "flips")


def _case(seed, batch, rows, cols, step):
    rng = np.random.default_rng(seed)
    w0 = (rng.standard_normal((batch, rows, cols)) * 0.02).astype(np.float32)
    w1 = w0 + (rng.standard_normal(w0.shape) * step).astype(np.float32)
    w1[0, :32, :32] *= 2.5            # a tile whose scale changes
    if rows * cols >= 64 * 64:
        w1[-1, -32:, -32:] = np.inf   # a tile that becomes non-finite
    return w0, w1


@pytest.mark.parametrize("batch,rows,cols", [(1, 32, 32), (2, 64, 288), (3, 96, 544), (1, 320, 96)])
@pytest.mark.parametrize("margin", [0, 8, 31])
@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_deosc_parity(batch, rows, cols, margin, dt):
    w0, w1 = _case(rows + cols + margin, batch, rows, cols, 2e-3)
    if dt == "bf16":
        w0, w1 = synth.f32_to_bf16_bits(w0), synth.f32_to_bf16_bits(np.nan_to_num(w1, posinf=np.inf))
        w1d = dev_bf16(w1)
    else:
        w1d = dev(w1)
    pc, ps, _, _ = oracle.quantize_2d(w0)
    got = mx.quantize_2d_deosc(w1d, dev(pc), dev(ps), margin)
    _check(got, oracle.quantize_2d_deosc(w1, pc, ps, margin))


def test_deosc_in_place_and_pitched():
    """The state updated in place, with padded code rows, equals the
    out-of-place result; the padding is untouched."""
    import torch
    w0, w1 = _case(3, 2, 96, 320, 2e-3)
    pc, ps, _, _ = oracle.quantize_2d(w0)
    want = oracle.quantize_2d_deosc(w1, pc, ps, 12)
    buf = torch.full((2, 96, 192), 0xA5, dtype=torch.uint8, device="cuda")
    buf[..., :160] = dev(pc)
    state_c, state_s = buf[..., :160], dev(ps)
    got = mx.quantize_2d_deosc(dev(w1), state_c, state_s, 12, codes=state_c, scales=state_s)
    assert got[0].data_ptr() == state_c.data_ptr()
    _assert_same(host(state_c.contiguous()), want[0], "in-place codes")
    _assert_same(host(state_s), want[1], "in-place scales")
    _assert_same(host(got[2]), want[2], "codes_t")
    _assert_same(_flips(got[4]), want[4], "flips")
    assert bool((buf[..., 160:] == 0xA5).all())


def test_deosc_trajectory_state_on_device():
    """20 steps of a random-walk master-weight trajectory: the kernel carries
    its own state on the device (updated in place), the oracle carries its
    own; every step's codes, scales and flips agree."""
    rng = np.random.default_rng(17)
    w = (rng.standard_normal((2, 128, 256)) * 0.02).astype(np.float32)
    c, s, _, _ = oracle.quantize_2d(w)
    dc, ds = dev(c), dev(s)
    total = 0
    for k in range(20):
        w = w + (rng.standard_normal(w.shape) * 1e-4).astype(np.float32)
        want = oracle.quantize_2d_deosc(w, c, s, 10)
        got = mx.quantize_2d_deosc(dev(w), dc, ds, 10, codes=dc, scales=ds)
        _check(got, want, "step %d " % k)
        c, s = want[0], want[1]
        total += int(want[4].sum())
    assert total > 0


def test_deosc_full_size_expert_weights():
    """32 experts x fp32 master weights 2880 x 5760 N(0, 0.02), against the
    quantization of a nearby tensor, margin 8/64: every expert in full."""
    import torch
    E, R, C = 32, 2880, 5760
    rng = np.random.default_rng(31)
    w0 = (rng.standard_normal((E, R, C), dtype=np.float32) * np.float32(0.02))
    pc, ps, _, _ = oracle.quantize_2d(w0)
    w1 = w0 + rng.standard_normal((E, R, C), dtype=np.float32) * np.float32(2e-4)
    del w0
    got = [host(t) if t.dtype != torch.int16 else _flips(t)
           for t in mx.quantize_2d_deosc(dev(w1), dev(pc), dev(ps), 8)]
    for e in range(E):
        want = oracle.quantize_2d_deosc(w1[e], pc[e], ps[e], 8)
        for g, wnt, n in zip(got, want, ("codes", "scales", "codes_t", "scales_t", "flips")):
            _assert_same(g[e], wnt, "%s e%d" % (n, e))


def test_deosc_scale_band_hovering_tiles():
    """Tiles whose largest weight alternates just above and below a power of
    two (the previous scale kept on the way down) on many tiles at once,
    against the oracle carrying its own state; with margin 8 the flips stop
    after the first step."""
    rng = np.random.default_rng(19)
    base = (rng.standard_normal((2, 256, 512)) * 0.02).astype(np.float32)
    tiles = base.reshape(2, 8, 32, 16, 32)
    tiles[:, :, 3, :, 9] = 4.01 * 2.0 ** -5            # one element per tile sets the amax
    c, s, _, _ = oracle.quantize_2d(base)
    dc, ds = dev(c), dev(s)
    flips = []
    for k in range(6):
        w = base.copy()
        w.reshape(2, 8, 32, 16, 32)[:, :, 3, :, 9] = (3.99 if k % 2 == 0 else 4.01) * 2.0 ** -5
        want = oracle.quantize_2d_deosc(w, c, s, 8)
        got = mx.quantize_2d_deosc(dev(w), dc, ds, 8, codes=dc, scales=ds)
        _check(got, want, "step %d " % k)
        c, s = want[0], want[1]
        flips.append(int(want[4].sum()))
    assert flips[1:] == [0] * 5, flips
