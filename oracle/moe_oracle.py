"""CPU oracle for one MoE layer with affinity-aware token dispatch.

TEST INFRASTRUCTURE ONLY.  Only tests/, __graft_entry__.smoke() and
bench.py's cpu_baseline leg may import this module.  It shares no code with
the HIP library or its binding and imports nothing from the product package.

It is a plain, slow, dense per-token MoE in fp64 (numpy), computed in
ORIGINAL expert labels: no placement permutation, no lookup table, no sort.
A separate plain reference (``shuffle``) defines the dispatch metadata.  Where
floating point decides an integer (which experts are selected) the decision
is taken in fp32, the kernel's precision, by the C part in oracle.c.

Passages followed (pages: "Semantic Parallelism: Redefining Efficient MoE
Inference via Model-Data Co-Scheduling", summaries in Korean (ko), German (de)
and Japanese (ja); "MoE-Prism: Disentangling Monolithic Experts for Elastic MoE
Services via Model-System Co-Designs", Korean summary):

* each token activates only a few experts chosen by the gate and has to
  reach the device that holds them (ko/de technical summary §1);
* experts are placed by shuffling the gate matrix's columns, which changes
  the physical placement without changing the model's logic (ja technical
  overview §2.2A) -> the oracle works in original labels and is therefore
  placement-invariant by construction;
* before the MoE layer, tokens are shuffled to the device of their predicted
  experts and, after the experts, results are gathered and put back into the
  original order (de technical summary §2B, ja §2.2B) -> ``shuffle`` and the
  token-order combine in ``forward``;
* a lightweight table maps a token to its expert group (ja §2.3) -> ``lut``;
* the local activation rate is the share of work processed locally
  (de §4) -> ``shuffle`` reports LAR per assignment;
* MoE-Prism splits each monolithic expert into N finer sub-experts made of
  neuron subsets (MoE-Prism technical summary §2A) and treats top-k as a
  per-request knob (§1, §5) -> sub-experts are neuron slices; k may be ragged.

Everything the pages leave open (gate function, top-k rule and tie-break,
SwiGLU expert form, shared experts, weight normalisation) follows the layer
configurations' own description (the named models' published layer forms);
each function's docstring states the choice it makes.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None


def lib():
    """Load the fp32 decision library (build with oracle/build.py)."""
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            from . import build as _b
            _b.build()
        L = ctypes.CDLL(_LIB_PATH)
        L.oracle_expf.restype = ctypes.c_float
        L.oracle_expf.argtypes = [ctypes.c_float]
        L.oracle_sigmoidf.restype = ctypes.c_float
        L.oracle_sigmoidf.argtypes = [ctypes.c_float]
        L.oracle_expf_array.argtypes = [ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p]
        L.oracle_sigmoid_keys.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_void_p,
                                          ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
        L.oracle_select.restype = ctypes.c_int
        L.oracle_select.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p,
                                    ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                    ctypes.c_void_p]
        _lib = L
    return _lib


def _ptr(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


# ----------------------------------------------------------------------------
# input decoding
# ----------------------------------------------------------------------------

def f64(a) -> np.ndarray:
    """Exact widening to fp64.  uint16 arrays are bf16 bit patterns."""
    a = np.asarray(a)
    if a.dtype == np.uint16:
        return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return a.astype(np.float64)


# ----------------------------------------------------------------------------
# O1: gate logits (+ synthetic affinity bias)
# ----------------------------------------------------------------------------

def logits(x, Wg, tok=None, pref=None, aff_bias: float = 0.0) -> np.ndarray:
    """l[t,e] = sum_h x[t,h] * Wg[e,h] in fp64, original expert order.

    If ``pref`` is given, ``aff_bias`` is added to the logits of the n_pref
    preferred (original) experts of token ID tok[t]: a single add after the
    dot product.  This is synthetic scaffolding for the context-independent
    token-expert affinity the pages observe (ko technical summary §2.1).
    """
    l = f64(x) @ f64(Wg).T
    if pref is not None and aff_bias != 0.0:
        rows = np.repeat(np.arange(l.shape[0]), pref.shape[1])
        cols = np.asarray(pref)[np.asarray(tok)].reshape(-1)
        l[rows, cols] += aff_bias
    return l


# ----------------------------------------------------------------------------
# O2-O4: routing
# ----------------------------------------------------------------------------

def sigmoid_keys(l32: np.ndarray, ebias: Optional[np.ndarray]):
    """fp32 selection keys sigmoid(l) + b and sigmoid(l), via the C part."""
    l32 = np.ascontiguousarray(l32, dtype=np.float32)
    T, E = l32.shape
    key = np.empty_like(l32)
    sig = np.empty_like(l32)
    b = None if ebias is None else np.ascontiguousarray(ebias, dtype=np.float32)
    lib().oracle_sigmoid_keys(T, E, _ptr(l32), _ptr(b), _ptr(key), _ptr(sig))
    return key, sig


def select(key32: np.ndarray, k_max: int, k_tok=None, n_rgroups=1, topk_rgroups=1,
           rgroup_topn=0) -> np.ndarray:
    """Top-k by (key desc, original id asc); returns sel[T, k_max], -1 padded."""
    key32 = np.ascontiguousarray(key32, dtype=np.float32)
    T, E = key32.shape
    sel = np.empty((T, k_max), np.int32)
    kt = None if k_tok is None else np.ascontiguousarray(k_tok, dtype=np.int32)
    rc = lib().oracle_select(T, E, _ptr(key32), _ptr(kt), k_max, n_rgroups, topk_rgroups,
                             rgroup_topn, _ptr(sel))
    if rc != 0:
        raise ValueError("oracle_select: bad arguments")
    return sel


def route(l, cfg, k_tok=None, ebias=None):
    """Selection and weights from logits ``l`` [T,E] (original order).

    ``l`` may be fp64 (the oracle's own logits) or fp32 (e.g. exported GPU
    logits); selection keys are always fp32, weights fp64.

    Softmax gate: p = softmax over all E; weights are p_j, or p_j / sum over
    the selected p when renormalised.  Sigmoid gate: selection on
    sigmoid(l) + b (grouped), weights route_scale * sigmoid(l_j) / sum_j
    sigmoid(l_j) without the bias.
    Returns (sel [T,k] int32 original ids, -1 padded; w [T,k] fp64, 0 padded).
    """
    l = np.asarray(l)
    l32 = l.astype(np.float32)
    l64 = l.astype(np.float64)
    T, E = l.shape
    k = cfg.k
    if cfg.gate == "softmax":
        sel = select(l32, k, k_tok)
        m = l64.max(axis=1, keepdims=True)
        ex = np.exp(l64 - m)
        p = ex / ex.sum(axis=1, keepdims=True)
        valid = sel >= 0
        ps = np.where(valid, np.take_along_axis(p, np.maximum(sel, 0), axis=1), 0.0)
        if cfg.renorm:
            # a token with routing budget k_t = 0 selects nothing: no weights
            tot = ps.sum(axis=1, keepdims=True)
            w = np.divide(ps, tot, out=np.zeros_like(ps), where=tot > 0)
        else:
            w = ps
    elif cfg.gate == "sigmoid_grouped":
        key, _ = sigmoid_keys(l32, ebias)
        sel = select(key, k, k_tok, cfg.n_rgroups, cfg.topk_rgroups, cfg.rgroup_topn)
        s64 = 1.0 / (1.0 + np.exp(-l64))
        valid = sel >= 0
        ss = np.where(valid, np.take_along_axis(s64, np.maximum(sel, 0), axis=1), 0.0)
        tot = ss.sum(axis=1, keepdims=True)
        w = cfg.route_scale * np.divide(ss, tot, out=np.zeros_like(ss), where=tot > 0)
    else:
        raise ValueError(cfg.gate)
    return sel, w


# ----------------------------------------------------------------------------
# O5: expert FFN
# ----------------------------------------------------------------------------

def silu(g):
    return g / (1.0 + np.exp(-g))


def ffn(x64: np.ndarray, W1, W3, W2) -> np.ndarray:
    """SwiGLU expert: W2 (silu(W1 x) * (W3 x)), fp64, rows of x are tokens."""
    g = x64 @ f64(W1).T
    u = x64 @ f64(W3).T
    return (silu(g) * u) @ f64(W2).T


def expert_ffn(x64, W13, W2, e: int, I: int):
    """FFN of original expert e with W13[e] = [W1; W3] ([2I, H]) and W2[e] [H, I]."""
    w13 = W13[e]
    return ffn(x64, w13[:I], w13[I:], W2[e])


def shared_ffn(x64, Wsh13, Wsh2, n_shared: int, I_shared: int):
    """Sum of the n_shared shared SwiGLU experts, each evaluated separately.

    Wsh13 stacks the shared experts' W1 rows ([ns*Is, H]) then their W3 rows;
    Wsh2 [H, ns*Is] holds their W2 blocks side by side.
    """
    nI = n_shared * I_shared
    y = np.zeros((x64.shape[0], Wsh2.shape[0]))
    for s in range(n_shared):
        r = slice(s * I_shared, (s + 1) * I_shared)
        W1 = Wsh13[:nI][r]
        W3 = Wsh13[nI:][r]
        y += ffn(x64, W1, W3, Wsh2[:, r])
    return y


# ----------------------------------------------------------------------------
# O6: dense per-token MoE output
# ----------------------------------------------------------------------------

def moe_output(x, sel, w, W13, W2, I, Wsh13=None, Wsh2=None, n_shared=0, I_shared=0):
    """out[t] = sum_j w[t,j] * FFN_{sel[t,j]}(x[t]) + sum_s FFN^sh_s(x[t]), fp64.

    Loops expert-major over the experts that are used (the per-(token, expert)
    arithmetic is the same in any loop order), then sums each token's terms
    in j order.  Returns out [T, H] fp64 in the ORIGINAL token order.
    """
    x64 = f64(x)
    T, k = sel.shape
    H = x64.shape[1]
    Y = np.zeros((T, k, H))
    for e in np.unique(sel[sel >= 0]):
        ts, js = np.nonzero(sel == e)
        Y[ts, js] = expert_ffn(x64[ts], W13, W2, int(e), I)
    out = np.zeros((T, H))
    for j in range(k):
        out += w[:, j:j + 1] * Y[:, j]
    if n_shared > 0:
        out += shared_ffn(x64, Wsh13, Wsh2, n_shared, I_shared)
    return out


# ----------------------------------------------------------------------------
# O7: dispatch metadata ("shuffle"), integer, exact
# ----------------------------------------------------------------------------

def row_ptr_of(k_tok) -> np.ndarray:
    """CSR offsets: exclusive scan of the per-token k, T+1 entries."""
    return np.concatenate([[0], np.cumsum(np.asarray(k_tok, np.int64))]).astype(np.int32)


def shuffle(row_ptr, slot, tok, lut, E: int, P: int) -> dict:
    """Dispatch metadata for assignments a = row_ptr[t] + j with expert slot[a].

    The expert group of a slot is slot // (E/P) (the placement puts E/P
    consecutive slots on each device); a token's predicted group is
    lut[tok[t]].  Assignments are ordered by (slot, predicted group, token):
    expert-contiguous, hence device-contiguous, and inside an expert in the
    order a device receives rows after the predicted-group token shuffle.
    Tokens alone are ordered by (predicted group, token).
    """
    row_ptr = np.asarray(row_ptr, np.int64)
    T = len(row_ptr) - 1
    A = int(row_ptr[-1])
    slot = np.asarray(slot, np.int64)[:A]
    epg = E // P
    t_of_a = np.repeat(np.arange(T), np.diff(row_ptr))
    g_pred = np.asarray(lut, np.int64)[np.asarray(tok, np.int64)]
    ga = g_pred[t_of_a]
    grp = slot // epg
    order = np.lexsort((t_of_a, ga, slot))           # primary key last
    s2a = order.astype(np.int32)
    a2s = np.empty(A, np.int32)
    a2s[order] = np.arange(A, dtype=np.int32)
    expert_count = np.bincount(slot, minlength=E).astype(np.int32)
    expert_off = np.concatenate([[0], np.cumsum(expert_count)]).astype(np.int32)
    group_count = expert_count.reshape(P, epg).sum(axis=1).astype(np.int32)
    group_off = np.concatenate([[0], np.cumsum(group_count)]).astype(np.int32)
    pair = np.zeros((P, P), np.int64)
    np.add.at(pair, (ga, grp), 1)
    tok_perm = np.lexsort((np.arange(T), g_pred)).astype(np.int32)
    tok_count = np.bincount(g_pred, minlength=P)
    tok_off = np.concatenate([[0], np.cumsum(tok_count)]).astype(np.int32)
    lar = float(np.trace(pair)) / A if A else 0.0
    return dict(expert_count=expert_count, expert_off=expert_off, group_count=group_count,
                group_off=group_off, pair_count=pair.astype(np.int32), tok_perm=tok_perm,
                tok_off=tok_off, sorted_to_assign=s2a, assign_to_sorted=a2s,
                g_pred=g_pred.astype(np.int32), lar=lar)


def gather(x, sorted_to_assign, row_ptr):
    """x_sorted[s] = x[token of assignment sorted_to_assign[s]] (bit copy)."""
    row_ptr = np.asarray(row_ptr, np.int64)
    T = len(row_ptr) - 1
    t_of_a = np.repeat(np.arange(T), np.diff(row_ptr))
    return np.asarray(x)[t_of_a[np.asarray(sorted_to_assign, np.int64)]]


def combine(y_sorted, assign_to_sorted, row_ptr, w_flat, y_sh=None):
    """out[t] = sum_j w[a] * y_sorted[assign_to_sorted[a]], a = row_ptr[t]+j, + y_sh[t].

    fp64, summed in j order; puts the expert outputs back in token order.
    """
    row_ptr = np.asarray(row_ptr, np.int64)
    T = len(row_ptr) - 1
    y = f64(y_sorted)
    out = np.zeros((T, y.shape[1]))
    for t in range(T):
        for a in range(row_ptr[t], row_ptr[t + 1]):
            out[t] += w_flat[a] * y[assign_to_sorted[a]]
    if y_sh is not None:
        out += f64(y_sh)
    return out


# ----------------------------------------------------------------------------
# one-GPU forms of the shuffled collectives around the MoE layer
# ----------------------------------------------------------------------------

def srs(x_part, tok_perm):
    """Shuffled reduce-scatter, one-GPU form.

    Under attention tensor parallelism every rank holds a partial sum of the
    attention output for all T tokens; the reduce-scatter that follows is
    reordered so that each rank receives the reduced rows of the tokens
    predicted to need its experts (de technical summary §2B, ja technical
    overview §2.2B: SRS).  With all P ranks' partials on one device the
    result is the reduced [T, H] rows laid out in tok_perm order, rank g's
    share being rows [tok_off[g], tok_off[g+1]):
        y[i] = sum_p x_part[p, tok_perm[i]]            (fp64)
    """
    x = f64(x_part)
    return x.sum(axis=0)[np.asarray(tok_perm, np.int64)]


def sag(y, tok_perm):
    """Shuffled all-gather, one-GPU form: the rows that the ranks hold in
    tok_perm order are gathered and put back into token order (de §2B, ja
    §2.2B: SAG):  out[tok_perm[i]] = y[i]  (bit copy)."""
    y = np.asarray(y)
    out = np.empty_like(y)
    out[np.asarray(tok_perm, np.int64)] = y
    return out


# ----------------------------------------------------------------------------
# offline table: token -> predicted expert group
# ----------------------------------------------------------------------------

def build_lut(prof_tok, prof_sel_orig, perm, E: int, P: int, V: int) -> np.ndarray:
    """lut[v] = the group that received most of token ID v's profiled
    assignments (ties to the lower group); IDs never seen map to v mod P.

    The pages build a token->expert probability table by offline profiling
    (de technical summary §2A) and keep a lightweight token->group table for
    the online shuffle (ja technical overview §2.3).
    """
    epg = E // P
    sel = np.asarray(prof_sel_orig)
    t_idx, _ = np.nonzero(sel >= 0)
    e = sel[sel >= 0]
    g = np.asarray(perm)[e] // epg
    v = np.asarray(prof_tok)[t_idx]
    cnt = np.zeros((V, P), np.int64)
    np.add.at(cnt, (v, g), 1)
    return lut_from_counts(cnt)


# ----------------------------------------------------------------------------
# offline co-scheduling: expert placement and request placement
# ----------------------------------------------------------------------------
#
# The pages pose expert placement and token/request scheduling as one 0-1
# co-clustering problem (experts and tokens into P device groups, maximising
# the work that stays local under balanced groups) solved by alternating
# optimisation (de technical summary §2B and key contribution 4; ko technical
# summary §2.2.1; ja technical overview §2.2A).  Reading taken: the objective
# is the number of profiled assignments whose token is predicted for the
# group holding its expert, sum_a [lut[tok_a] == group[expert_a]]; the two
# alternating steps each maximise it exactly with the other side fixed:
#   token step   lut[v] = argmax_g (assignments of token ID v on group g's
#                experts), ties to the lower group, unseen IDs v mod P;
#   expert step  group[] = the assignment of experts to groups, E/P experts
#                per group, maximising sum_e count[group[e]][e], where
#                count[g][e] = assignments at expert e of tokens with lut = g.
# Experts are original ids here (profiling runs with the identity placement).

def _assignment_token_ids(row_ptr, tok):
    row_ptr = np.asarray(row_ptr, np.int64)
    T = len(row_ptr) - 1
    return np.asarray(tok, np.int64)[np.repeat(np.arange(T), np.diff(row_ptr))]


def token_group_counts(row_ptr, expert, tok, group, V: int, P: int) -> np.ndarray:
    """D[v][g] = profiled assignments of token ID v to experts of group g."""
    A = int(np.asarray(row_ptr)[-1])
    v = _assignment_token_ids(row_ptr, tok)
    g = np.asarray(group, np.int64)[np.asarray(expert, np.int64)[:A]]
    D = np.zeros((V, P), np.int64)
    np.add.at(D, (v, g), 1)
    return D


def lut_from_counts(D: np.ndarray) -> np.ndarray:
    """Token step: lut[v] = argmax_g D[v][g] (lowest g on ties), unseen -> v mod P."""
    V, P = D.shape
    lut = np.argmax(D, axis=1).astype(np.int32)      # first maximum = lowest g
    unseen = D.sum(axis=1) == 0
    lut[unseen] = (np.arange(V)[unseen] % P).astype(np.int32)
    return lut


def expert_group_counts(row_ptr, expert, tok, lut, E: int, P: int) -> np.ndarray:
    """count[g][e] = profiled assignments at expert e of tokens with lut[tok] = g."""
    A = int(np.asarray(row_ptr)[-1])
    g = np.asarray(lut, np.int64)[_assignment_token_ids(row_ptr, tok)]
    cnt = np.zeros((P, E), np.int64)
    np.add.at(cnt, (g, np.asarray(expert, np.int64)[:A]), 1)
    return cnt


def balanced_assign(score: np.ndarray) -> np.ndarray:
    """Items to groups, n/P items per group, maximising sum_i score[i, group[i]].

    score is [n, P] with P dividing n.  Each group is given n/P identical
    slots and the n x n assignment problem is solved exactly (a library
    linear-assignment routine).  Returns group[i]."""
    from scipy.optimize import linear_sum_assignment
    n, P = score.shape
    cap = n // P
    cost = -np.repeat(np.asarray(score, np.float64), cap, axis=1)
    rows, cols = linear_sum_assignment(cost)
    group = np.empty(n, np.int32)
    group[rows] = (cols // cap).astype(np.int32)
    return group


def local_count(row_ptr, expert, tok, group, lut) -> int:
    """Objective: assignments whose token is predicted for its expert's group."""
    A = int(np.asarray(row_ptr)[-1])
    gt = np.asarray(lut, np.int64)[_assignment_token_ids(row_ptr, tok)]
    ge = np.asarray(group, np.int64)[np.asarray(expert, np.int64)[:A]]
    return int((gt == ge).sum())


def optimize_placement(row_ptr, expert, tok, group0, V: int, E: int, P: int, max_iters: int = 20):
    """Alternate token and expert steps from the expert grouping group0 until
    the grouping repeats.  Returns (group, lut, objective after each step)."""
    group = np.asarray(group0, np.int32).copy()
    trace = []
    lut = None
    for _ in range(max_iters):
        lut = lut_from_counts(token_group_counts(row_ptr, expert, tok, group, V, P))
        trace.append(local_count(row_ptr, expert, tok, group, lut))
        new = balanced_assign(expert_group_counts(row_ptr, expert, tok, lut, E, P).T)
        trace.append(local_count(row_ptr, expert, tok, new, lut))
        if trace[-1] <= trace[-2]:
            break                    # no strict gain: keep the previous grouping
        group = new
    lut = lut_from_counts(token_group_counts(row_ptr, expert, tok, group, V, P))
    return group, lut, trace


def placement_of_groups(group, P: int) -> np.ndarray:
    """perm[orig] = slot: group g's experts take slots [g*E/P, (g+1)*E/P) in
    ascending original id."""
    group = np.asarray(group, np.int64)
    order = np.lexsort((np.arange(len(group)), group))
    perm = np.empty(len(group), np.int32)
    perm[order] = np.arange(len(group), dtype=np.int32)
    return perm


def request_group_hist(req_ptr, tok, lut, P: int) -> np.ndarray:
    """Inter-request scheduling under attention data parallelism: H[r][g] =
    tokens of request r (tokens [req_ptr[r], req_ptr[r+1])) predicted for
    group g (de technical summary §2B; ko technical summary §2.2.2)."""
    req_ptr = np.asarray(req_ptr, np.int64)
    R = len(req_ptr) - 1
    r_of_t = np.repeat(np.arange(R), np.diff(req_ptr))
    g = np.asarray(lut, np.int64)[np.asarray(tok, np.int64)[:req_ptr[-1]]]
    H = np.zeros((R, P), np.int64)
    np.add.at(H, (r_of_t, g), 1)
    return H


def assign_requests(H: np.ndarray) -> np.ndarray:
    """Requests to data-parallel ranks, R/P per rank, maximising the tokens
    whose predicted group is their rank's: balanced_assign on H."""
    return balanced_assign(H)


def relative_error(y, ref) -> float:
    """max over tokens of ||y_t - r_t||_inf / ||r_t||_inf."""
    y = np.asarray(y, np.float64)
    ref = np.asarray(ref, np.float64)
    num = np.abs(y - ref).max(axis=1)
    den = np.abs(ref).max(axis=1)
    den = np.where(den == 0, 1.0, den)
    return float((num / den).max()) if len(num) else 0.0
