"""The grouped gate's selection sigmoid on the GPU (moe_sigmoid, the code the
route kernel runs) against the oracle's own fp32 sigmoid, bit for bit.  Both
evaluate exp by Cody-Waite reduction and a degree-7 Taylor polynomial in
fused multiply-adds, written separately on each side; the sigmoid gate's
top-k compares these values, so selection parity needs them identical, not
merely close."""
import ctypes

import numpy as np
import pytest

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu

CHUNK = 1 << 25


def _oracle_sigmoid(olib, x32):
    key = np.empty_like(x32)
    sig = np.empty_like(x32)
    olib.oracle_sigmoid_keys(1, x32.size, x32.ctypes.data, None, key.ctypes.data, sig.ctypes.data)
    return sig


def _check(olib, m, bits):
    x = bits.view(np.float32)
    xd = torch.from_numpy(x).to("cuda")
    yd = torch.empty_like(xd)
    m.moe_sigmoid(xd, yd)
    torch.cuda.synchronize()
    got = yd.cpu().numpy()
    ref = _oracle_sigmoid(olib, x)
    bad = got.view(np.uint32) != ref.view(np.uint32)
    if bad.any():
        i = int(np.flatnonzero(bad)[0])
        raise AssertionError("sigmoid(%r): GPU %r, oracle %r (%d of %d differ)"
                             % (float(x[i]), float(got[i]), float(ref[i]), int(bad.sum()), x.size))
    return x.size


def test_sigmoid_bit_identical_dense(olib):
    from token_routing_shuffle_amd import moe as m
    # every 7th fp32 bit pattern of each sign up to |x| = 96 (past both ends
    # of exp's range), in chunks
    top = int(np.float32(96.0).view(np.uint32))
    n = 0
    for sign in (0, 0x80000000):
        for lo in range(0, top + 1, CHUNK * 7):
            bits = np.arange(lo, min(top + 1, lo + CHUNK * 7), 7, dtype=np.uint64)
            n += _check(olib, m, (bits + sign).astype(np.uint32))
    print("[sigmoid] %d values bit-identical" % n, flush=True)


def test_sigmoid_bit_identical_every_value_of_two_binades(olib):
    from token_routing_shuffle_amd import moe as m
    # all fp32 values in [2, 4) and (-4, -2]: where the key gaps between
    # strong experts fall
    lo = int(np.float32(2.0).view(np.uint32))
    hi = int(np.float32(4.0).view(np.uint32))
    bits = np.arange(lo, hi, dtype=np.uint32)
    assert _check(olib, m, bits) == 1 << 23
    assert _check(olib, m, bits | np.uint32(0x80000000)) == 1 << 23


def test_sigmoid_special_values(olib):
    from token_routing_shuffle_amd import moe as m
    x = np.array([0.0, -0.0, 1e-45, -1e-45, 87.0, -87.0, 88.0, -88.0, 87.5, -87.5, 88.5, -88.5,
                  1e30, -1e30, np.inf, -np.inf], dtype=np.float32)
    _check(olib, m, x.view(np.uint32))
    xd = torch.tensor([np.nan], dtype=torch.float32, device="cuda")
    yd = torch.empty_like(xd)
    m.moe_sigmoid(xd, yd)
    torch.cuda.synchronize()
    assert torch.isnan(yd).all()
