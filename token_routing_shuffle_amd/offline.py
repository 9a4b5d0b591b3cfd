"""Offline tables of a layer: placement-ordered weights and the token->group
lookup table.

Sem-MoE prepares both before serving (Japanese summary, technical overview
§2.2A and §2.3; German summary, technical summary §2A):
  * the expert placement is applied by shuffling the gate matrix's columns
    (and moving each expert's weights with it) — ``place`` reorders every
    per-expert tensor into slot order, slot = placement position;
  * a lightweight table maps each token ID to the placement group that its
    experts most often live in, learned by profiling — ``profile_lut`` routes
    a profiling draw through the library's own moe_route on the GPU and keeps,
    for each token ID, the group that received most of its assignments (ties
    to the lower group; IDs never seen map to v mod P).
Neither runs on the per-layer hot path.
"""
from __future__ import annotations

import numpy as np
import torch

from . import moe


def place(w: dict, slot_to_orig: np.ndarray, device) -> dict:
    """Per-expert tensors in slot order: out[s] = in[slot_to_orig[s]]."""
    idx = torch.as_tensor(np.asarray(slot_to_orig, np.int64), device=device)
    out = {}
    for name in ("Wg", "W13", "W2"):
        out[name] = w[name].to(device).index_select(0, idx).contiguous()
    for name in ("Wsh13", "Wsh2"):
        out[name] = None if w.get(name) is None else w[name].to(device).contiguous()
    return out


def device_layer(cfg, tables, w: dict, lut: np.ndarray, device="cuda") -> dict:
    """Every device tensor moe_forward needs, keyed like moe_weights."""
    d = place(w, tables.slot_to_orig, device)
    d["slot_to_orig"] = torch.as_tensor(tables.slot_to_orig, device=device)
    d["ebias"] = None
    if tables.ebias is not None:
        d["ebias"] = torch.as_tensor(tables.ebias[tables.slot_to_orig], device=device)
    d["lut"] = torch.as_tensor(np.asarray(lut, np.int32), device=device)
    d["pref"] = None if tables.pref is None else torch.as_tensor(tables.pref, device=device)
    return d


def route_chunk(cfg, chunk: int = 16384) -> int:
    """Largest token count <= chunk whose layer configuration passes
    moe_validate's bf16 limit on the activations (x [T,H] below 2 GiB: the
    gate kernel addresses its rows through 32-bit buffer offsets)."""
    if cfg.dtype != "bf16":
        return chunk
    cap = (2 ** 31 - 1) // (2 * cfg.H)
    return max(1, min(chunk, cap))


def profile_routing(cfg, dev: dict, prof_x: torch.Tensor, prof_tok: np.ndarray,
                    chunk: int = 16384):
    """Route a profiling draw with moe_route (chunks of at most `chunk`
    tokens, fewer where the layer's operand limit requires) and return the
    whole draw's routing as device CSR (row_ptr [n+1], slots [A]) plus its
    token IDs (device int32)."""
    device = prof_x.device
    n = prof_x.shape[0]
    chunk = route_chunk(cfg, chunk)
    tok_all = torch.as_tensor(np.asarray(prof_tok, np.int32), device=device)
    rps, sls, base = [torch.zeros(1, dtype=torch.int32, device=device)], [], 0
    for s in range(0, n, chunk):
        m = min(chunk, n - s)
        c = moe.make_cfg(cfg, T=m)
        k_tok = None
        if cfg.ragged:
            k_tok = torch.full((m,), cfg.k, dtype=torch.int32, device=device)
        row_ptr = torch.empty(m + 1, dtype=torch.int32, device=device)
        slots = torch.empty(m * cfg.k, dtype=torch.int32, device=device)
        wts = torch.empty(m * cfg.k, dtype=torch.float32, device=device)
        moe.moe_route(c, prof_x[s:s + m], dev["Wg"], dev.get("ebias"), dev["slot_to_orig"],
                      tok_all[s:s + m], dev.get("pref"), k_tok, row_ptr, slots, wts,
                      ws=moe.route_workspace(c, device))
        a = int(row_ptr[m].item())
        rps.append(row_ptr[1:] + base)
        sls.append(slots[:a])
        base += a
    return torch.cat(rps), torch.cat(sls), tok_all


def lut_of_grouping(cfg, row_ptr, slots, tok, group: np.ndarray) -> torch.Tensor:
    """Token step of the co-scheduling (moe_token_group_counts and
    moe_lut_from_counts): the group that receives most of each token ID's
    profiled assignments; group[s] = placement group of slot s."""
    device = row_ptr.device
    c = moe.make_cfg(cfg)
    counts = torch.empty(cfg.V * cfg.P, dtype=torch.int32, device=device)
    lut = torch.empty(cfg.V, dtype=torch.int32, device=device)
    moe.moe_token_group_counts(c, tok.numel(), row_ptr, slots, tok,
                               torch.as_tensor(np.asarray(group, np.int32), device=device), counts)
    moe.moe_lut_from_counts(c, counts, lut)
    return lut


def profile_lut(cfg, dev: dict, prof_x: torch.Tensor, prof_tok: np.ndarray,
                chunk: int = 16384) -> np.ndarray:
    """Token->group table from routing a profiling draw with moe_route, for
    the layer's current placement (slot s is in group s // (E/P))."""
    rp, sl, tok = profile_routing(cfg, dev, prof_x, prof_tok, chunk)
    group = np.arange(cfg.E, dtype=np.int32) // (cfg.E // cfg.P)
    return lut_of_grouping(cfg, rp, sl, tok, group).cpu().numpy()
