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
              identity_placement: bool = False, device=DEV, mutate=None, **over) -> Case:
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
    if mutate is not None:
        # test-specific structure (duplicated gate rows, zero activations,
        # zero selection bias) applied to the drawn inputs before anything
        # is derived from them
        mutate(cfg, tables, w, x)
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


# ---------------------------------------------------------------- parity checks

# Lines kept for the end-of-run summary (tests/conftest.py prints them even
# under -q): per-case counts of exact ties and near-tie tokens.
REPORT = []


def report(line: str) -> None:
    REPORT.append(line)
    print(line, flush=True)


def csr_to_sel(case: Case, rp, slot_flat, vals=None, fill=-1):
    """CSR (slot ids) -> [T, k] original ids (and values), padded."""
    T, k = case.cfg.T, case.cfg.k
    rp = np.asarray(rp, np.int64)
    cnt = np.diff(rp)
    sel = np.full((T, k), fill, np.int64)
    out = np.zeros((T, k)) if vals is not None else None
    t_of_a = np.repeat(np.arange(T), cnt)
    j_of_a = np.arange(int(rp[-1])) - np.repeat(rp[:-1], cnt)
    s2o = np.asarray(case.tables.slot_to_orig, np.int64)
    sel[t_of_a, j_of_a] = s2o[np.asarray(slot_flat, np.int64)[:int(rp[-1])]]
    if vals is not None:
        out[t_of_a, j_of_a] = np.asarray(vals)[:int(rp[-1])]
    return sel, out


def logits_orig(case: Case, logits_slot) -> np.ndarray:
    """Exported GPU logits (slot order, fp32 [T*E]) in original expert order."""
    T, E = case.cfg.T, case.cfg.E
    l = np.asarray(logits_slot, np.float32)[:T * E].reshape(T, E)
    out = np.empty_like(l)
    out[:, case.tables.slot_to_orig] = l
    return out


def k_tok_of(case: Case):
    return case.tables.k_tok if case.cfg.ragged else None


def selection_keys32(case: Case, l32) -> np.ndarray:
    """The fp32 selection keys of the oracle for fp32 logits l32 [T,E]."""
    if case.cfg.gate == "softmax":
        return np.asarray(l32, np.float32)
    key, _ = mo.sigmoid_keys(np.asarray(l32, np.float32), case.tables.ebias)
    return key


def exact_tie_tokens(case: Case, key32, sel_orig, k_tok=None) -> int:
    """Tokens whose selection depends on the tie-break: an unselected expert
    has exactly the key of the last selected one, or two selected experts
    have equal keys (then the selection order is the tie-break's)."""
    T, E = key32.shape
    n = 0
    for t in range(T):
        kt = case.cfg.k if k_tok is None else int(k_tok[t])
        if kt == 0:
            continue
        s = sel_orig[t, :kt]
        ks = key32[t, s]
        if len(np.unique(ks)) < kt:
            n += 1
            continue
        if kt < E:
            rest = np.setdiff1d(np.arange(E), s)
            if (key32[t, rest] == ks.min()).any():
                n += 1
    return n


def strict_route_parity(case: Case, rp_gpu, slot_gpu, w_gpu, l_gpu32, label: str) -> dict:
    """Tier (i) of the parity rule: the oracle's fp32 selection and its
    weights, run on the GPU's own exported logits, against the GPU's routing.
    row_ptr and every token's selected experts (original ids, in selection
    order) must be identical; the weights agree to fp32 rounding of the same
    logits.  Returns the oracle's routing on those logits and the tie count."""
    cfg = case.cfg
    T, E = cfg.T, cfg.E
    k_tok = k_tok_of(case)
    kt = np.full(T, cfg.k) if k_tok is None else np.asarray(k_tok)
    np.testing.assert_array_equal(np.asarray(rp_gpu)[:T + 1], mo.row_ptr_of(kt), err_msg="row_ptr")
    sel_ref, w_ref = mo.route(l_gpu32, cfg, k_tok, case.tables.ebias)
    sel_gpu, w_gpu_tk = csr_to_sel(case, rp_gpu, slot_gpu, w_gpu)
    bad = np.nonzero((sel_gpu != sel_ref).any(axis=1))[0]
    assert len(bad) == 0, "%s: %d tokens select differently from the oracle on the GPU's logits, " \
        "first %s: gpu %s oracle %s" % (label, len(bad), bad[:3], sel_gpu[bad[:3]], sel_ref[bad[:3]])
    # weights: the same fp32 logits through fp32 exp / sigmoid, a sum of at
    # most E terms and one division on the GPU; fp64 in the oracle
    u = 2.0 ** -24
    tol = (E + 16) * u * np.abs(w_ref) + 1e-30
    werr = np.abs(w_gpu_tk - w_ref)
    assert (werr <= tol).all(), "%s: weights differ by up to %.3g (tolerance %.3g)" % (
        label, werr.max(), tol[np.unravel_index(np.argmax(werr - tol), tol.shape)])
    ties = exact_tie_tokens(case, selection_keys32(case, l_gpu32), sel_ref, k_tok)
    return dict(sel=sel_ref, w=w_ref, ties=ties)


SHUFFLE_TABLES = ("expert_count", "expert_off", "group_count", "group_off", "pair_count",
                  "tok_perm", "tok_off")


def strict_shuffle_parity(case: Case, rp_gpu, slot_gpu, tables: dict, label: str) -> dict:
    """Tier (i) for the dispatch metadata: the oracle's shuffle run on the
    GPU's own routing (row_ptr, topk_slot) must reproduce every count,
    offset and permutation bit for bit."""
    cfg = case.cfg
    T = cfg.T
    A = int(np.asarray(rp_gpu)[T])
    ref = mo.shuffle(np.asarray(rp_gpu)[:T + 1], np.asarray(slot_gpu)[:A], case.tok, case.lut,
                     cfg.E, cfg.P)
    for n in SHUFFLE_TABLES:
        if n in tables:
            want = ref[n].reshape(-1)
            np.testing.assert_array_equal(np.asarray(tables[n])[:want.size], want,
                                          err_msg="%s: %s" % (label, n))
    for n in ("sorted_to_assign", "assign_to_sorted"):
        if n in tables:
            np.testing.assert_array_equal(np.asarray(tables[n])[:A], ref[n], err_msg="%s: %s" % (label, n))
    return ref


def check_forward(case: Case, r: dict, label: str, rows=None) -> dict:
    """Every check of a moe_forward result with exports (harness.run_forward
    in the tests): strict routing and shuffle parity on the GPU's own
    logits and routing; the GPU's selection against the oracle's own fp64
    logits under the near-tie rule; the layer output against the dense
    oracle -- with the oracle's routing where the selections agree, with the
    oracle's routing of the GPU logits where a near tie made them differ --
    on every token or on `rows`."""
    cfg = case.cfg
    T, E = cfg.T, cfg.E
    A = int(r["row_ptr"][T])
    l_gpu32 = logits_orig(case, r["logits"])
    st = strict_route_parity(case, r["row_ptr"], r["topk_slot"][:A], r["topk_w"][:A], l_gpu32, label)
    sh = strict_shuffle_parity(case, r["row_ptr"], r["topk_slot"][:A], r, label)
    k_tok = k_tok_of(case)
    l64 = oracle_logits(case)
    sel_or, w_or = oracle_route(case, l64, k_tok)
    sel_gpu = st["sel"]
    ndiff = check_selection(case, sel_gpu, l64, l_gpu32.astype(np.float64), k_tok)
    rows = np.arange(T) if rows is None else np.asarray(rows)
    same = (sel_gpu[rows] == sel_or[rows]).all(axis=1)
    got = f64_of(host(r["out"]))[rows]
    ref = np.zeros((len(rows), cfg.H))
    for m, sel, w in ((same, sel_or, w_or), (~same, sel_gpu, st["w"])):
        if m.any():
            rr = rows[m]
            ref[m] = mo.moe_output(case.h["x"][rr], sel[rr], w[rr], case.h["W13"], case.h["W2"], cfg.I,
                                   case.h.get("Wsh13"), case.h.get("Wsh2"), cfg.n_shared, cfg.I_shared)
    err = rel_err(got, ref) if len(rows) else 0.0
    report("[parity] %s: T=%d A=%d selection bit-exact on the GPU logits (%d exact-tie tokens), "
           "dispatch tables bit-exact; vs oracle logits %d near-tie tokens, max|dl|=%.3g; "
           "output rel err %.3g over %d tokens (tol %g); LAR=%.3f"
           % (label, T, A, st["ties"], ndiff, float(np.abs(l_gpu32 - l64).max()) if T else 0.0,
              err, len(rows), tol_out(cfg), sh["lar"]))
    assert err <= tol_out(cfg), "%s: output rel err %.3g" % (label, err)
    return dict(strict=st, shuffle=sh, ndiff=ndiff, err=err, sel_or=sel_or, w_or=w_or, l64=l64)


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
