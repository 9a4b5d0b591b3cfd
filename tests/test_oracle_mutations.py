"""Mutation check of the oracle's pins.

Each case copies the oracle (and its pin tests) to a temporary directory,
plants one plausible mistake in the copy (a dropped term, a flipped sign or
comparison, swapped operands or keys), rebuilds it and runs the pins there.
The pins must fail for every mutant; the real oracle is never modified.
"""
import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

C_MUTANTS = {
    "tie_break_flipped": ("(ka == kb && ia < ib)", "(ka == kb && ia > ib)"),
    "taylor_term_wrong": ("(float)(1.0 / 6.0)", "(float)(1.0 / 7.0)"),
    "ln2_low_part_dropped": ("r = fmaf(-n, ln2_lo, r);", "r = r;"),
    "group_score_top1_only": ("s = (j == 0) ? kr[g * gsize + best] : s + kr[g * gsize + best];",
                              "s = (j == 0) ? kr[g * gsize + best] : s;"),
    "sigmoid_sign": ("float e = oracle_expf(-l);", "float e = oracle_expf(l);"),
    "group_tie_to_higher_id": ("if (best < 0 || better(score[g], g, score[best], best)) best = g;",
                               "if (best < 0 || score[g] >= score[best]) best = g;"),
    "bias_dropped": ("key[(int64_t)t * E + e] = bias ? s + bias[e] : s;",
                     "key[(int64_t)t * E + e] = s;"),
}

PY_MUTANTS = {
    "logits_operand_transposed": ("l = f64(x) @ f64(Wg).T", "l = (f64(Wg) @ f64(x).T).T[:, ::-1]"),
    "affinity_bias_wrong_rows": ("rows = np.repeat(np.arange(l.shape[0]), pref.shape[1])",
                                 "rows = np.tile(np.arange(l.shape[0]), pref.shape[1])"),
    "renorm_dropped": ("            w = np.divide(ps, tot, out=np.zeros_like(ps), where=tot > 0)",
                       "            w = ps"),
    "route_scale_dropped": ("w = cfg.route_scale * np.divide(ss, tot, out=np.zeros_like(ss), where=tot > 0)",
                            "w = np.divide(ss, tot, out=np.zeros_like(ss), where=tot > 0)"),
    "zero_budget_weights_nan": ("w = np.divide(ps, tot, out=np.zeros_like(ps), where=tot > 0)",
                                "w = ps / tot"),
    "silu_sign": ("return g / (1.0 + np.exp(-g))", "return g / (1.0 + np.exp(g))"),
    "gate_up_swapped": ("return ffn(x64, w13[:I], w13[I:], W2[e])",
                        "return ffn(x64, w13[I:], w13[:I], W2[e])"),
    "up_proj_dropped": ("return (silu(g) * u) @ f64(W2).T", "return (silu(g) * g) @ f64(W2).T"),
    "weights_index_j_ignored": ("out += w[:, j:j + 1] * Y[:, j]", "out += w[:, 0:1] * Y[:, j]"),
    "shuffle_keys_reordered": ("order = np.lexsort((t_of_a, ga, slot))", "order = np.lexsort((ga, t_of_a, slot))"),
    "pair_count_transposed": ("np.add.at(pair, (ga, grp), 1)", "np.add.at(pair, (grp, ga), 1)"),
    "expert_off_off_by_one": ("expert_off = np.concatenate([[0], np.cumsum(expert_count)]).astype(np.int32)",
                              "expert_off = np.concatenate([[0], np.cumsum(expert_count) - 1]).astype(np.int32)"),
    "tok_perm_ignores_group": ("tok_perm = np.lexsort((np.arange(T), g_pred)).astype(np.int32)",
                               "tok_perm = np.arange(T).astype(np.int32)"),
    "combine_shared_dropped": ("        out += f64(y_sh)", "        pass"),
    "shared_w3_from_w1": ("        W3 = Wsh13[nI:][r]", "        W3 = Wsh13[:nI][r]"),
    "lut_unseen_fallback": ("lut[unseen] = (np.arange(V)[unseen] % P).astype(np.int32)", "pass"),
    "srs_inverse_permutation": ("return x.sum(axis=0)[np.asarray(tok_perm, np.int64)]",
                                "return x.sum(axis=0)[np.argsort(np.asarray(tok_perm, np.int64))]"),
    "srs_one_partial_only": ("return x.sum(axis=0)[np.asarray(tok_perm, np.int64)]",
                             "return x[0][np.asarray(tok_perm, np.int64)]"),
    "sag_gathers_instead_of_scattering": ("out[np.asarray(tok_perm, np.int64)] = y",
                                          "out[:] = y[np.asarray(tok_perm, np.int64)]"),
    "balanced_assign_minimises": ("cost = -np.repeat(np.asarray(score, np.float64), cap, axis=1)",
                                  "cost = np.repeat(np.asarray(score, np.float64), cap, axis=1)"),
    "lut_ties_to_higher_group": ("lut = np.argmax(D, axis=1).astype(np.int32)",
                                 "lut = (P - 1 - np.argmax(D[:, ::-1], axis=1)).astype(np.int32)"),
    "expert_counts_use_expert_group": ("g = np.asarray(lut, np.int64)[_assignment_token_ids(row_ptr, tok)]\n    cnt",
                                       "g = np.asarray(lut, np.int64)[np.asarray(expert, np.int64)[:A] % len(lut)]\n    cnt"),
    "slots_descending_ids": ("order = np.lexsort((np.arange(len(group)), group))",
                             "order = np.lexsort((-np.arange(len(group)), group))"),
    "request_hist_by_token_index": ("g = np.asarray(lut, np.int64)[np.asarray(tok, np.int64)[:req_ptr[-1]]]",
                                    "g = np.asarray(lut, np.int64)[np.arange(req_ptr[-1]) % len(lut)]"),
}


def _make_copy(tmp, name, target, old, new):
    d = os.path.join(tmp, name)
    shutil.copytree(os.path.join(ROOT, "oracle"), os.path.join(d, "oracle"),
                    ignore=shutil.ignore_patterns("*.so", "__pycache__"))
    os.makedirs(os.path.join(d, "tests"))
    for f in ("conftest.py", "test_oracle_pins.py"):
        shutil.copy(os.path.join(ROOT, "tests", f), os.path.join(d, "tests", f))
    shutil.copytree(os.path.join(ROOT, "tests", "golden"), os.path.join(d, "tests", "golden"))
    os.makedirs(os.path.join(d, "token_routing_shuffle_amd"))
    for f in ("__init__.py", "workload.py"):
        shutil.copy(os.path.join(ROOT, "token_routing_shuffle_amd", f),
                    os.path.join(d, "token_routing_shuffle_amd", f))
    shutil.copy(os.path.join(ROOT, "pytest.ini"), os.path.join(d, "pytest.ini"))
    path = os.path.join(d, "oracle", target)
    src = open(path).read()
    assert src.count(old) == 1, (name, old)
    open(path, "w").write(src.replace(old, new))
    subprocess.run([sys.executable, os.path.join(d, "oracle", "build.py")], check=True,
                   capture_output=True)
    return d


def _run_pins(d, fast):
    cmd = [sys.executable, "-m", "pytest", "-x", "-q", "tests/test_oracle_pins.py"]
    if fast:
        cmd += ["-k", "not dense_sample"]
    env = dict(os.environ, PYTHONDONTWRITEBYTECODE="1")
    return subprocess.run(cmd, cwd=d, capture_output=True, text=True, env=env, timeout=600)


def test_every_mutant_is_caught(tmp_path):
    jobs = [(n, "oracle.c", o, w, False) for n, (o, w) in C_MUTANTS.items()]
    jobs += [(n, "moe_oracle.py", o, w, True) for n, (o, w) in PY_MUTANTS.items()]

    def one(job):
        name, target, old, new, fast = job
        d = _make_copy(str(tmp_path), name, target, old, new)
        r = _run_pins(d, fast)
        return name, r.returncode, r.stdout[-400:]

    with ThreadPoolExecutor(max_workers=4) as ex:
        results = list(ex.map(one, jobs))
    survivors = [(n, out) for n, rc, out in results if rc == 0]
    assert not survivors, survivors
