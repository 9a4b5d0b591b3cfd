"""Test harness: seeded layers on the GPU, their host copies for the oracle,
and the oracle-side reference pieces (routing with the near-tie rule, LUT).

Inputs come only from token_routing_shuffle_amd.workload (the seeded
generators) and from the oracle; nothing the HIP library computes is fed to
the oracle.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional

import numpy as np
import torch

from oracle import moe_oracle as mo
from token_routing_shuffle_amd import workload as wl

DEV = "cuda"


def host(t: Optional[torch.Tensor]) -> Optional[np.ndarray]:
    """Device tensor -> numpy; bf16 as uint16 bit patterns (exact)."""
    if t is None:
        return None
    t = t.detach()
    if t.dtype == torch.bfloat16:
        return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


def to_dev(a: np.ndarray, dtype=None, device=DEV) -> torch.Tensor:
    """numpy -> device tensor; uint16 arrays become bf16 (bit copy)."""
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).to(device).view(torch.bfloat16)
    t = torch.from_numpy(a).to(device)
    return t if dtype is None else t.to(dtype)


def bf16_bits(a64: np.ndarray) -> np.ndarray:
    """Round fp64 values to bf16 (RNE) bit patterns, through torch's cast."""
    return torch.from_numpy(np.asarray(a64, np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


@dataclasses.dataclass
class Case:
    cfg: wl.LayerConfig
    tables: wl.Tables
    w: dict            # device tensors, original order
    x: torch.Tensor    # device [T, H]
    h: dict            # host copies (numpy) of x and weights, original order
    lut: np.ndarray
    dev: dict = None   # device tensors in slot order (moe_weights keys)

    @property
    def tok(self):
        return self.tables.tok


def make_case(name_or_cfg, T: Optional[int] = None, profile_tokens: int = 4096,
              identity_placement: bool = False, device=DEV, **over) -> Case:
    from token_routing_shuffle_amd import offline
    cfg = wl.CONFIGS[name_or_cfg] if isinstance(name_or_cfg, str) else name_or_cfg
    if T is not None:
        over["T"] = T
    if over:
        cfg = cfg.replace(**over)
    tables = wl.make_tables(cfg, profile_tokens=profile_tokens)
    if identity_placement:
        tables.slot_to_orig = np.arange(cfg.E, dtype=np.int32)
        tables.perm = np.arange(cfg.E, dtype=np.int32)
    w = wl.make_weights(cfg, device)
    x = wl.make_x(cfg, device)
    h = {k: host(v) for k, v in w.items()}
    h["x"] = host(x)
    case = Case(cfg, tables, w, x, h, None)
    case.lut = oracle_lut(case, profile_tokens, device)
    case.dev = offline.device_layer(cfg, tables, w, case.lut, device)
    return case


# ---------------------------------------------------------------- oracle pieces

def oracle_logits(case: Case, rows=None, x_h=None, tok=None) -> np.ndarray:
    cfg = case.cfg
    x_h = case.h["x"] if x_h is None else x_h
    tok = case.tok if tok is None else tok
    if rows is not None:
        x_h, tok = x_h[rows], tok[rows]
    pref = case.tables.pref
    return mo.logits(x_h, case.h["Wg"], tok, pref, cfg.aff_bias if pref is not None else 0.0)


def oracle_route(case: Case, l64: np.ndarray, k_tok=None):
    cfg = case.cfg
    return mo.route(l64, cfg, k_tok, case.tables.ebias)


def oracle_lut(case: Case, n: int, device=DEV) -> np.ndarray:
    cfg = case.cfg
    px = host(wl.make_prof_x(cfg, device, n))
    ptok = case.tables.prof_tok[:n]
    sels = []
    for s in range(0, n, 4096):
        l64 = oracle_logits(case, None, px[s:s + 4096], ptok[s:s + 4096])
        k_tok = np.full(l64.shape[0], cfg.k, np.int32) if cfg.ragged else None
        sel, _ = oracle_route(case, l64, k_tok)
        sels.append(sel)
    sel = np.concatenate(sels)
    return mo.build_lut(ptok, sel, case.tables.perm, cfg.E, cfg.P, cfg.V)


def key_tolerance(cfg, dl):
    """Bound on |key_gpu - key_oracle| given the logit difference dl."""
    if cfg.gate == "softmax":
        return dl
    # sigmoid' <= 1/4, plus a few fp32 roundings of values near 1
    return dl / 4 + 4e-7


def logit_bound(case: Case, rows=None) -> np.ndarray:
    """A priori bound on fp32-accumulated gate dot products in any order:
    gamma_H * sum_h |x_h w_h| (Higham, Accuracy and Stability of Numerical
    Algorithms, 2nd ed., §3.1), plus roundings of the result and bias add."""
    xh = mo.f64(case.h["x"] if rows is None else case.h["x"][rows])
    wg = mo.f64(case.h["Wg"])
    H = xh.shape[1]
    u = 2.0 ** -24
    gamma = H * u / (1 - H * u)
    s = np.abs(xh) @ np.abs(wg).T
    return gamma * s + 4 * u * (s + abs(case.cfg.aff_bias))


def _oracle_keys(case: Case, l64):
    if case.cfg.gate == "softmax":
        return l64.astype(np.float32).astype(np.float64)
    key32, _ = mo.sigmoid_keys(l64.astype(np.float32), case.tables.ebias)
    return key32.astype(np.float64)


def _valid_under_tolerance(cfg, keys_t, picks, kt, tol):
    """Is `picks` the top-kt of some key vector within +-tol of keys_t?"""
    E = len(keys_t)
    if cfg.gate == "softmax" or cfg.n_rgroups <= 1 or cfg.topk_rgroups >= cfg.n_rgroups:
        kth = np.sort(keys_t)[::-1][kt - 1]
        return bool((keys_t[picks] >= kth - 2 * tol).all())
    import itertools
    G, keep, n = cfg.n_rgroups, cfg.topk_rgroups, cfg.rgroup_topn
    gs = E // G
    score = np.array([np.sort(keys_t[g * gs:(g + 1) * gs])[::-1][:n].sum() for g in range(G)])
    need = set((np.asarray(picks) // gs).tolist())
    for S in itertools.combinations(range(G), keep):
        if not need <= set(S):
            continue
        out = [g for g in range(G) if g not in S]
        if out and score[list(S)].min() < score[out].max() - 2 * n * tol:
            continue
        allowed = np.concatenate([np.arange(g * gs, (g + 1) * gs) for g in S])
        kth = np.sort(keys_t[allowed])[::-1][kt - 1]
        if (keys_t[picks] >= kth - 2 * tol).all():
            return True
    return False


def check_selection(case: Case, sel_gpu_orig: np.ndarray, l64: np.ndarray, l_gpu: np.ndarray,
                    k_tok=None, max_frac=0.01):
    """GPU selections (original ids) against the oracle's on its own logits.

    delta_t = max_e |l_gpu - l_oracle| must stay within the a priori bound.
    A token may route differently only if the oracle's keys near-tie at the
    selection boundary within 2*delta (in key space): its GPU picks must be
    the top-k of some key vector within that distance of the oracle's.
    Returns the number of differing tokens."""
    cfg = case.cfg
    sel_or, _ = oracle_route(case, l64, k_tok)
    dl = np.abs(l_gpu.astype(np.float64) - l64).max(axis=1) if len(l64) else np.zeros(0)
    diff_rows = np.nonzero((sel_or != sel_gpu_orig).any(axis=1))[0]
    if len(diff_rows) == 0:
        return 0
    keys = _oracle_keys(case, l64)
    for t in diff_rows:
        kt = cfg.k if k_tok is None else int(k_tok[t])
        g = sel_gpu_orig[t, :kt]
        assert (sel_gpu_orig[t, kt:] == -1).all()
        assert len(set(g.tolist())) == kt, "duplicate expert in GPU selection"
        tol = key_tolerance(cfg, float(dl[t])) + 1e-12
        assert _valid_under_tolerance(cfg, keys[t], g, kt, tol), (t, g, sel_or[t], dl[t])
    assert len(diff_rows) <= max(1, max_frac * len(l64)), \
        "%d of %d tokens route differently" % (len(diff_rows), len(l64))
    return len(diff_rows)


def rel_err(y, ref) -> float:
    return mo.relative_error(np.asarray(y, np.float64), np.asarray(ref, np.float64))


def tol_out(cfg) -> float:
    return 1e-5 if cfg.dtype == "f32" else 2e-2


def dev_i32(n, device=DEV):
    return torch.empty(max(n, 1), dtype=torch.int32, device=device)


def dev_f32(n, device=DEV):
    return torch.empty(max(n, 1), dtype=torch.float32, device=device)


def act_dtype(cfg):
    return torch.bfloat16 if cfg.dtype == "bf16" else torch.float32


def f64_of(a) -> np.ndarray:
    return mo.f64(a)


def ceil_div(a, b):
    return -(-a // b)


__all__ = [n for n in dir() if not n.startswith("_")] + ["math"]
