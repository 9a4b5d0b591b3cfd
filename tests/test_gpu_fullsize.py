"""GPU parity at the full layer sizes, in the launch configuration bench.py
times (moe_forward with the bench's gather setting and, for bf16 layers, its
tile-blocked weights).  The determinism re-run uses the row-major weights, so
it also checks the two weight layouts against each other bit for bit.

The oracle computes routing for every token (its fp32 selection on the
GPU's exported logits must equal the GPU's exactly; against its own fp64
logits the near-tie rule applies), the dispatch metadata of the GPU's own
routing for the whole layer (bit-exact, unconditionally), and the layer
output for a sample of tokens one by one.
"""
import os

import numpy as np
import pytest
import torch

from tests import harness as hn
from tests.test_gpu_parity import run_forward

pytestmark = pytest.mark.gpu

BENCH_FUSE = int(os.environ.get("MOE_BENCH_FUSE_GATHER", "1"))
FULL = ["tiny", "dsv2lite", "qwen3", "prism"]
DSV3 = ["dsv3_decode", "dsv3_prefill"]


def sample_rows(T, n=96):
    rng = np.random.default_rng(7)
    head = np.arange(min(T, 8))
    tail = np.arange(max(0, T - 8), T)
    mid = rng.choice(T, size=min(T, n), replace=False)
    return np.unique(np.concatenate([head, tail, mid]))


def _full_case(name):
    print("[fullsize] building", name, flush=True)
    return hn.make_case(name, profile_tokens=65536)


def _blocked_dev(c):
    """The layer's device weights with the expert FFN weights packed into the
    tile-blocked layout (as bench.py does once before timing)."""
    from token_routing_shuffle_amd import moe
    cfg = moe.make_cfg(c.cfg, weights_blocked=1)
    dev = dict(c.dev)
    for which, k13, k2 in ((moe.MOE_FFN_ROUTED, "W13", "W2"), (moe.MOE_FFN_SHARED, "Wsh13", "Wsh2")):
        if dev.get(k13) is None:
            continue
        b13, b2 = torch.empty_like(dev[k13]), torch.empty_like(dev[k2])
        moe.moe_pack_weights(cfg, which, dev[k13], dev[k2], b13, b2)
        dev[k13], dev[k2] = b13, b2
    torch.cuda.synchronize()
    return dev


def _check(c, fuse=BENCH_FUSE):
    cfg = c.cfg
    T = cfg.T
    kw = dict(dev=_blocked_dev(c), weights_blocked=1) if cfg.dtype == "bf16" else {}
    r = run_forward(c, fuse=fuse, **kw)
    print("[fullsize] %s: forward done" % cfg.name, flush=True)
    # strict routing and dispatch parity on every token; near-tie rule
    # against the oracle's own logits; outputs on a sample of tokens
    hn.check_forward(c, r, "fullsize %s T=%d" % (cfg.name, T), rows=sample_rows(T))
    # run-to-run determinism at full size (row-major weights, the other
    # gather setting: the same bits)
    kw.clear()
    r2 = run_forward(c, fuse=1 - fuse, exports=False)
    assert torch.equal(r["out"], r2["out"])


@pytest.mark.parametrize("name", FULL)
def test_full_size(name):
    _check(_full_case(name))


@pytest.mark.slow
@pytest.mark.parametrize("name", DSV3)
def test_full_size_dsv3(name):
    _check(_full_case(name))


def test_max_tokens():
    """A layer whose sorted rows lie far beyond 2 GiB: the DeepSeek-V2-Lite
    shape at T = 262144 tokens, A = 1 572 864 rows, x_sorted and y_sorted
    [A, 2048] bf16 = 6.4 GB each and the intermediate 4.4 GB; the grouped
    GEMMs address those rows per tile.  Materialised gather (GEMM1 reads
    x_sorted), then the fused gather for the determinism re-run; same checks
    as the full-size layers."""
    from token_routing_shuffle_amd import moe
    T = 262144
    c = hn.make_case("dsv2lite", T=T, profile_tokens=65536)
    assert T * c.cfg.k * c.cfg.H * 2 > 2 ** 32
    assert moe.moe_validate(moe.make_cfg(c.cfg)) == moe.MOE_OK
    _check(c, fuse=0)
