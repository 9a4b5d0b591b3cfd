"""The empty layer (T = 0 tokens) through the C ABI on the GPU.

Every call returns MOE_OK.  The dispatch tables come out as the empty
layer's own: row_ptr = [0], every per-slot and per-group count and offset
zero, and the would-be all-to-all matrix zero.  Nothing else is written:
sentinel values in the per-token and per-row exports, and in the output,
survive the call.
"""
import pytest
import torch

from tests import harness as hn

pytestmark = pytest.mark.gpu

SENT = -7


def _moe():
    from token_routing_shuffle_amd import moe
    return moe


def _i32(n):
    return torch.full((n,), SENT, dtype=torch.int32, device=hn.DEV)


def _f32(n):
    return torch.full((n,), float(SENT), dtype=torch.float32, device=hn.DEV)


def _tables(E, P):
    """Count and offset tables (checked to be written) and per-token or
    per-row exports (checked to stay untouched), all sentinel-filled."""
    written = dict(row_ptr=_i32(1), expert_count=_i32(E), expert_off=_i32(E + 1),
                   group_count=_i32(P), group_off=_i32(P + 1), pair_count=_i32(P * P),
                   tok_off=_i32(P + 1))
    untouched = dict(topk_slot=_i32(4), topk_w=_f32(4), logits=_f32(4), tok_perm=_i32(4),
                     sorted_to_assign=_i32(4), assign_to_sorted=_i32(4))
    return written, untouched


def _check_tables(written, untouched):
    torch.cuda.synchronize()
    for k, v in written.items():
        assert (v == 0).all(), (k, v.cpu().numpy())
    for k, v in untouched.items():
        assert (v == SENT).all(), (k, v.cpu().numpy())


@pytest.mark.parametrize("name,over", [("tiny", {}), ("dsv2lite", {}), ("dsv2lite", {"weights_blocked": 1}),
                                       ("prism", {}), ("qwen3", {})])
def test_forward_empty(name, over):
    m = _moe()
    c = hn.make_case(name, 8, profile_tokens=256)
    cfg = m.make_cfg(c.cfg, T=0, **over)
    assert m.moe_validate(cfg) == m.MOE_OK
    E, P, H = c.cfg.E, c.cfg.P, c.cfg.H
    written, untouched = _tables(E, P)
    out = torch.full((4, H), 3.0, dtype=hn.act_dtype(c.cfg), device=hn.DEV)
    k_tok = hn.k_tok_of(c)
    k_tok = None if k_tok is None else torch.as_tensor(k_tok, device=hn.DEV)[:0]
    tok = torch.as_tensor(c.tok, device=hn.DEV)
    ws = m.workspace(cfg)
    # zero-length views of real tensors: valid pointers, nothing to read
    m.moe_forward(cfg, m.weights_struct(c.dev), m.inputs_struct(c.x[:0], tok[:0], k_tok),
                  out, m.exports_struct(dict(written, **untouched)), ws)
    _check_tables(written, untouched)
    assert (out == 3.0).all()


@pytest.mark.parametrize("noalloc", [False, True])
def test_stages_empty(noalloc):
    """moe_route, moe_shuffle (or moe_shuffle_noalloc), moe_expert_ffn and
    moe_combine on the empty layer, one by one."""
    m = _moe()
    c = hn.make_case("dsv2lite", 8, profile_tokens=256)
    cfg = m.make_cfg(c.cfg, T=0)
    E, P, H = c.cfg.E, c.cfg.P, c.cfg.H
    written, untouched = _tables(E, P)
    ws = m.workspace(cfg)
    d = c.dev
    tok = torch.as_tensor(c.tok, device=hn.DEV)[:0]
    x = c.x[:0]
    m.moe_route(cfg, x, d["Wg"], d.get("ebias"), d["slot_to_orig"], tok, d.get("pref"), None,
                written["row_ptr"], untouched["topk_slot"], untouched["topk_w"], untouched["logits"], ws)
    shuffle = m.moe_shuffle_noalloc if noalloc else m.moe_shuffle
    kw = {} if noalloc else dict(ws=ws)
    shuffle(cfg, written["row_ptr"], untouched["topk_slot"], tok, d["lut"], x,
            written["expert_count"], written["expert_off"], written["group_count"], written["group_off"],
            written["pair_count"], untouched["tok_perm"], written["tok_off"],
            untouched["sorted_to_assign"], untouched["assign_to_sorted"], **kw)
    y = torch.full((4, H), 3.0, dtype=hn.act_dtype(c.cfg), device=hn.DEV)
    m.moe_expert_ffn(cfg, m.MOE_FFN_ROUTED, None, x, written["row_ptr"], untouched["sorted_to_assign"],
                     written["expert_off"], d["W13"], d["W2"], 0, E, y, ws)
    m.moe_expert_ffn(cfg, m.MOE_FFN_SHARED, None, x, None, None, None, d["Wsh13"], d["Wsh2"], 0, 0, y, ws)
    out = torch.full((4, H), 3.0, dtype=hn.act_dtype(c.cfg), device=hn.DEV)
    m.moe_combine(cfg, y, untouched["assign_to_sorted"], written["row_ptr"], untouched["topk_w"], None, out)
    _check_tables(written, untouched)
    assert (y == 3.0).all() and (out == 3.0).all()
