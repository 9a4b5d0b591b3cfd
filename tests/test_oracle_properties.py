"""Property tests of the CPU oracle over generated shapes (hypothesis): the
top-k selection and the dispatch metadata against brute force written here,
on random sizes including the degenerate ones (one token, k = E, P = 1,
P = E, empty experts, ragged budgets with zeros) and keys with many exact
ties.  CPU only."""
import numpy as np
import pytest

hyp = pytest.importorskip("hypothesis")
from hypothesis import given, settings, strategies as st  # noqa: E402

from oracle import moe_oracle as mo  # noqa: E402

SETTINGS = settings(max_examples=60, deadline=None, derandomize=True)


def _brute_topk(row, k, allowed=None):
    ids = [e for e in range(len(row)) if allowed is None or allowed[e]]
    return sorted(ids, key=lambda e: (-float(row[e]), e))[:k]


@st.composite
def selection_case(draw):
    T = draw(st.integers(1, 12))
    E = draw(st.integers(1, 16))
    k_max = draw(st.integers(1, E))
    ragged = draw(st.booleans())
    seed = draw(st.integers(0, 2**31 - 1))
    rng = np.random.default_rng(seed)
    # keys on a coarse grid: exact ties are common
    key = (rng.integers(-3, 4, (T, E)) * 0.5).astype(np.float32)
    k_tok = rng.integers(0, k_max + 1, T).astype(np.int32) if ragged else None
    return key, k_max, k_tok


@SETTINGS
@given(selection_case())
def test_select_matches_brute_force(case):
    key, k_max, k_tok = case
    sel = mo.select(key, k_max, k_tok)
    assert sel.shape == (key.shape[0], k_max)
    for t in range(key.shape[0]):
        kt = k_max if k_tok is None else int(k_tok[t])
        assert sel[t, :kt].tolist() == _brute_topk(key[t], kt)
        assert (sel[t, kt:] == -1).all()


@st.composite
def grouped_case(draw):
    G = draw(st.sampled_from([1, 2, 3, 4]))
    gs = draw(st.integers(2, 6))
    E = G * gs
    keep = draw(st.integers(1, G))
    topn = draw(st.integers(1, min(3, gs)))
    k = draw(st.integers(1, keep * gs))
    T = draw(st.integers(1, 8))
    rng = np.random.default_rng(draw(st.integers(0, 2**31 - 1)))
    key = (rng.integers(-4, 5, (T, E)) * 0.25).astype(np.float32)
    return key, k, G, keep, topn


@SETTINGS
@given(grouped_case())
def test_grouped_select_matches_brute_force(case):
    key, k, G, keep, topn = case
    T, E = key.shape
    gs = E // G
    sel = mo.select(key, k, None, G, keep, topn)
    for t in range(T):
        score = []
        for g in range(G):
            v = sorted(key[t, g * gs:(g + 1) * gs].tolist(), reverse=True)[:topn]
            s = np.float32(v[0])
            for x in v[1:]:
                s = np.float32(s + np.float32(x))
            score.append(s)
        kept = sorted(range(G), key=lambda g: (-score[g], g))[:keep]
        allowed = [(e // gs) in kept for e in range(E)]
        assert sel[t].tolist() == _brute_topk(key[t], k, allowed)


@st.composite
def shuffle_case(draw):
    log_epg = draw(st.integers(0, 3))
    P = draw(st.integers(1, 4))
    E = P << log_epg
    T = draw(st.integers(0, 20))
    k_max = draw(st.integers(1, E))
    ragged = draw(st.booleans())
    V = draw(st.integers(1, 9))
    rng = np.random.default_rng(draw(st.integers(0, 2**31 - 1)))
    k_tok = rng.integers(0, k_max + 1, T) if ragged else np.full(T, k_max)
    row_ptr = mo.row_ptr_of(k_tok)
    # a skewed expert draw (weights 1/(e+1)^2) leaves some experts empty
    pw = 1.0 / (np.arange(E) + 1.0) ** 2
    pw /= pw.sum()
    slot = np.concatenate([rng.choice(E, size=int(k), replace=False, p=pw) for k in k_tok]).astype(np.int32) \
        if row_ptr[-1] else np.zeros(0, np.int32)
    tok = rng.integers(0, V, T).astype(np.int32)
    lut = rng.integers(0, P, V).astype(np.int32)
    return row_ptr, slot, tok, lut, E, P


@SETTINGS
@given(shuffle_case())
def test_shuffle_matches_brute_force(case):
    row_ptr, slot, tok, lut, E, P = case
    T = len(row_ptr) - 1
    A = int(row_ptr[-1])
    r = mo.shuffle(row_ptr, slot, tok, lut, E, P)
    items = sorted(((int(slot[a]), int(lut[tok[t]]), t), a)
                   for t in range(T) for a in range(row_ptr[t], row_ptr[t + 1]))
    assert r["sorted_to_assign"].tolist() == [a for _, a in items]
    assert r["tok_perm"].tolist() == sorted(range(T), key=lambda t: (int(lut[tok[t]]), t))
    inv = np.empty(A, np.int64)
    inv[[a for _, a in items]] = np.arange(A)
    np.testing.assert_array_equal(r["assign_to_sorted"], inv)
    cnt = [sum(1 for a in range(A) if slot[a] == e) for e in range(E)]
    assert r["expert_count"].tolist() == cnt
    assert r["expert_off"].tolist() == [sum(cnt[:e]) for e in range(E + 1)]
    epg = E // P
    gcnt = [sum(cnt[g * epg:(g + 1) * epg]) for g in range(P)]
    assert r["group_count"].tolist() == gcnt
    assert r["group_off"].tolist() == [sum(gcnt[:g]) for g in range(P + 1)]
    pc = np.zeros((P, P), int)
    for t in range(T):
        for a in range(row_ptr[t], row_ptr[t + 1]):
            pc[lut[tok[t]], slot[a] // epg] += 1
    np.testing.assert_array_equal(np.asarray(r["pair_count"]).reshape(P, P), pc)
    tcnt = [sum(1 for t in range(T) if lut[tok[t]] == g) for g in range(P)]
    assert r["tok_off"].tolist() == [sum(tcnt[:g]) for g in range(P + 1)]
