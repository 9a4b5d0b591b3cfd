"""The entry point that allocates nothing (moe_shuffle_noalloc: scratch in
the library's static device array) against moe_shuffle with a caller
workspace, through the C ABI: every dispatch table and the gathered rows
bit for bit, on two calls in a row on the same device, the second with a
smaller layer (the array keeps the first call's contents), and a layer
whose scratch exceeds the array is rejected before anything is enqueued."""
import numpy as np
import pytest
import torch

from oracle import moe_oracle as mo
from tests import harness as hn

pytestmark = pytest.mark.gpu

TABLES = ("expert_count", "expert_off", "group_count", "group_off", "pair_count", "tok_perm",
          "tok_off", "sorted_to_assign", "assign_to_sorted")


def _routing(c):
    """The oracle's routing of the layer (CSR), as device tensors."""
    l64 = hn.oracle_logits(c)
    k_tok = hn.k_tok_of(c)
    sel, _ = hn.oracle_route(c, l64, k_tok)
    kt = np.full(c.cfg.T, c.cfg.k) if k_tok is None else k_tok
    rp = mo.row_ptr_of(kt)
    slot = np.concatenate([c.tables.perm[sel[t, :kt[t]]] for t in range(c.cfg.T)]).astype(np.int32)
    return hn.to_dev(rp), hn.to_dev(np.concatenate([slot, np.zeros(1, np.int32)])), int(rp[-1])


def _outs(c):
    T, E, P, A_max = c.cfg.T, c.cfg.E, c.cfg.P, c.cfg.T * c.cfg.k
    sizes = dict(expert_count=E, expert_off=E + 1, group_count=P, group_off=P + 1, pair_count=P * P,
                 tok_perm=T, tok_off=P + 1, sorted_to_assign=A_max, assign_to_sorted=A_max)
    o = {n: torch.full((sizes[n],), -3, dtype=torch.int32, device=hn.DEV) for n in TABLES}
    xs = torch.zeros((A_max, c.cfg.H), dtype=hn.act_dtype(c.cfg), device=hn.DEV)
    return o, xs


def _run_both(c):
    from token_routing_shuffle_amd import moe
    cfg = moe.make_cfg(c.cfg)
    rp, slot, A = _routing(c)
    tok = torch.as_tensor(c.tok, device=hn.DEV)
    ref, xs_ref = _outs(c)
    moe.moe_shuffle(cfg, rp, slot, tok, c.dev["lut"], c.x, *[ref[n] for n in TABLES], xs_ref,
                    moe.workspace(cfg))
    got, xs = _outs(c)
    moe.moe_shuffle_noalloc(cfg, rp, slot, tok, c.dev["lut"], c.x, *[got[n] for n in TABLES], xs)
    torch.cuda.synchronize()
    for n in TABLES:
        lim = A if n in ("sorted_to_assign", "assign_to_sorted") else ref[n].numel()
        assert torch.equal(got[n][:lim], ref[n][:lim]), n
    assert torch.equal(xs[:A], xs_ref[:A])
    return A


def test_noalloc_matches_workspace_call_twice_second_smaller():
    big = hn.make_case("prism", 1024, profile_tokens=1024)
    small = hn.make_case("qwen3", 200, profile_tokens=1024)
    print("[noalloc] prism T=1024 then qwen3 T=200", flush=True)
    a1 = _run_both(big)
    a2 = _run_both(small)
    assert a2 < a1


def test_noalloc_rejects_layers_beyond_the_array():
    from token_routing_shuffle_amd import moe
    from token_routing_shuffle_amd import workload as wl
    cfg = moe.make_cfg(wl.CONFIGS["prism"].replace(T=520000))
    assert moe.moe_validate(cfg) == moe.MOE_OK
    d = torch.zeros(16, dtype=torch.int32, device=hn.DEV)
    with pytest.raises(moe.MoeError) as ei:
        moe.moe_shuffle_noalloc(cfg, d, d, d, d, None, d, d, d, d, d, d, d, d, d)
    assert ei.value.code == moe.MOE_EWORKSPACE
    assert "scratch" in moe.moe_last_error()
