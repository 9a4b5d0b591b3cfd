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


# ----------------------------------------------------------------------------
# persisted offline tables
#
# Placement, token->group table and the preferred-expert (affinity) table of a
# layer are offline artefacts (the pages fix placement and the token table
# before serving, ja technical overview §2.2A and §2.3).  They are saved as one
# .npz per layer configuration, keyed by a hash of the configuration and of
# how the token table was profiled, and read back with numpy's non-pickle
# loader.

TABLE_FORMAT = 1


def config_key(cfg, profile_tokens: int, placement: str = "random") -> str:
    """Hex key of a layer configuration (every LayerConfig field), the
    profiling-draw size and the placement rule."""
    import dataclasses
    import hashlib
    import json
    d = dataclasses.asdict(cfg)
    d["k_choices"] = list(d["k_choices"])
    blob = json.dumps({"cfg": d, "profile_tokens": int(profile_tokens), "placement": placement,
                       "format": TABLE_FORMAT}, sort_keys=True)
    return hashlib.sha256(blob.encode()).hexdigest()[:24]


def table_path(directory: str, cfg, profile_tokens: int, placement: str = "random") -> str:
    import os
    return os.path.join(directory, "%s_%s.npz" % (cfg.name, config_key(cfg, profile_tokens, placement)))


def save_tables(directory: str, cfg, tables, lut, profile_tokens: int, placement: str = "random") -> str:
    """Write slot_to_orig, perm, lut and (when present) the preferred-expert
    table and the expert selection bias of a layer; returns the file path."""
    import os
    os.makedirs(directory, exist_ok=True)
    path = table_path(directory, cfg, profile_tokens, placement)
    arrays = dict(slot_to_orig=np.asarray(tables.slot_to_orig, np.int32),
                  perm=np.asarray(tables.perm, np.int32), lut=np.asarray(lut, np.int32),
                  key=np.frombuffer(config_key(cfg, profile_tokens, placement).encode(), np.uint8))
    if tables.pref is not None:
        arrays["pref"] = np.asarray(tables.pref, np.int32)
    if tables.ebias is not None:
        arrays["ebias"] = np.asarray(tables.ebias, np.float32)
    tmp = path + ".tmp.npz"
    np.savez(tmp, **arrays)
    os.replace(tmp, path)
    return path


def load_tables(directory: str, cfg, profile_tokens: int, placement: str = "random"):
    """The saved tables of this exact configuration as a dict of arrays, or
    None when there is no file for it.  A file whose stored key does not
    match (renamed or corrupted) raises ValueError."""
    import os
    path = table_path(directory, cfg, profile_tokens, placement)
    if not os.path.exists(path):
        return None
    with np.load(path, allow_pickle=False) as z:
        out = {k: z[k] for k in z.files}
    key = bytes(out.pop("key")).decode()
    if key != config_key(cfg, profile_tokens, placement):
        raise ValueError("%s: stored key %s does not match the configuration" % (path, key))
    E, P, V = cfg.E, cfg.P, cfg.V
    if out["slot_to_orig"].shape != (E,) or out["perm"].shape != (E,) or out["lut"].shape != (V,):
        raise ValueError("%s: table shapes do not match the configuration" % path)
    if not (np.sort(out["slot_to_orig"]) == np.arange(E)).all() or (out["lut"] < 0).any() or (out["lut"] >= P).any():
        raise ValueError("%s: placement is not a permutation or the token table is out of range" % path)
    return out
