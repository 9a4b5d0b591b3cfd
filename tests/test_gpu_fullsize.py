"""GPU parity at the full layer sizes, in the launch configuration bench.py
times (moe_forward with the bench's gather setting and, for bf16 layers, its
tile-blocked weights).  The determinism re-run uses the row-major weights, so
it also checks the two weight layouts against each other bit for bit.

The oracle computes routing for every token (selection compared with the
near-tie rule, CSR offsets exactly), the dispatch metadata for the whole
layer (bit-exact), and the layer output for a sample of tokens one by one.
"""
import os

import numpy as np
import pytest
import torch

from oracle import moe_oracle as mo
from tests import harness as hn
from tests.test_gpu_parity import csr_to_sel, k_tok_of, oracle_routing, run_forward

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


def _check(c):
    cfg = c.cfg
    T, E, P = cfg.T, cfg.E, cfg.P
    kw = dict(dev=_blocked_dev(c), weights_blocked=1) if cfg.dtype == "bf16" else {}
    r = run_forward(c, fuse=BENCH_FUSE, **kw)
    print("[fullsize] %s: forward done" % cfg.name, flush=True)
    l64, sel_or, w_or, rp_or, slot_or, _ = oracle_routing(c)
    np.testing.assert_array_equal(r["row_ptr"][:T + 1], rp_or)
    A = int(rp_or[-1])
    l_gpu = np.empty((T, E))
    l_gpu[:, c.tables.slot_to_orig] = r["logits"][:T * E].reshape(T, E)
    sel_gpu, _ = csr_to_sel(c, r["row_ptr"], r["topk_slot"][:A])
    ndiff = hn.check_selection(c, sel_gpu, l64, l_gpu, k_tok_of(c))
    # the whole layer's dispatch metadata, bit-exact, from the oracle's routing
    ref = mo.shuffle(rp_or, slot_or, c.tok, c.lut, E, P)
    if ndiff == 0:
        for n in ("expert_count", "expert_off", "group_count", "group_off", "pair_count",
                  "tok_perm", "tok_off"):
            np.testing.assert_array_equal(r[n][:ref[n].size], ref[n].reshape(-1), err_msg=n)
        np.testing.assert_array_equal(r["sorted_to_assign"][:A], ref["sorted_to_assign"])
        np.testing.assert_array_equal(r["assign_to_sorted"][:A], ref["assign_to_sorted"])
    else:
        s2a = r["sorted_to_assign"][:A]
        assert (np.sort(s2a) == np.arange(A)).all()
        assert (r["assign_to_sorted"][:A][s2a] == np.arange(A)).all()
        assert r["expert_count"][:E].sum() == A == r["pair_count"][:P * P].sum()
    # sampled outputs
    rows = sample_rows(T)
    rows = rows[(sel_gpu[rows] == sel_or[rows]).all(axis=1)]
    outr = mo.moe_output(c.h["x"][rows], sel_or[rows], w_or[rows], c.h["W13"], c.h["W2"], cfg.I,
                         c.h.get("Wsh13"), c.h.get("Wsh2"), cfg.n_shared, cfg.I_shared)
    got = hn.f64_of(hn.host(r["out"]))[rows]
    err = hn.rel_err(got, outr)
    print("[fullsize] %s: T=%d A=%d near-tie tokens=%d LAR=%.3f sampled rel err=%.3g over %d tokens"
          % (cfg.name, T, A, ndiff, ref["lar"], err, len(rows)), flush=True)
    assert err <= hn.tol_out(cfg)
    # run-to-run determinism at full size (row-major weights: the same bits)
    kw.clear()
    r2 = run_forward(c, fuse=BENCH_FUSE, exports=False)
    assert torch.equal(r["out"], r2["out"])


@pytest.mark.parametrize("name", FULL)
def test_full_size(name):
    _check(_full_case(name))


@pytest.mark.slow
@pytest.mark.parametrize("name", DSV3)
def test_full_size_dsv3(name):
    _check(_full_case(name))


def test_max_tokens():
    """The largest layer moe_validate accepts for the DeepSeek-V2-Lite shape:
    T = 87381 tokens, whose A*H*2 = 2 147 469 312 bytes of sorted rows sit
    just below the grouped GEMM's 2 GiB buffer-offset limit; same checks as
    the full-size layers."""
    from token_routing_shuffle_amd import moe
    T = (2 ** 31 - 1) // (6 * 2048 * 2)
    c = hn.make_case("dsv2lite", T=T, profile_tokens=65536)
    assert moe.moe_validate(moe.make_cfg(c.cfg)) == moe.MOE_OK
    assert moe.moe_validate(moe.make_cfg(c.cfg.replace(T=T + 1))) == moe.MOE_ESHAPE
    _check(c)

