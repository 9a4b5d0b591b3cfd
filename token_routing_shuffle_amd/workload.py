"""Seeded synthetic MoE-layer workloads.

This module only draws inputs: token IDs, the expert placement, the
token->preferred-expert affinity table, per-request routing budgets and the
dense tensors (activations and weights).  It holds none of the layer's
arithmetic (no routing, no sorting by expert, no FFN), so both the HIP path
and the CPU oracle can be fed from it.

Shapes follow the five layer configurations of the Sem-MoE / MoE-Prism
workloads (DeepSeek-V2-Lite-, Qwen3-30B-A3B- and DeepSeek-V3-shaped layers and
a MoE-Prism sub-expert variant).  The pages never print tensor shapes, so the
shapes are those of the named models; the distributions are:

* token IDs: uniform (tiny case) or bounded Zipf, P(id = r-1) ~ r^-s for
  r = 1..V, drawn by inverse CDF over the explicit pmf;
* x ~ N(0, 1), weights ~ N(0, 1/fan_in), rounded to bf16 (RNE) except in the
  fp32 case;
* placement: a uniformly random permutation of experts into P equal groups
  (the "shuffled gate columns" of the Sem-MoE summary, technical overview
  §2.2A);
* affinity: each token ID prefers n_pref distinct experts drawn without
  replacement; the gate adds a fixed logit bias to them.  This stands in for
  the context-independent token-expert affinity the pages report (technical
  overview §2.1); it is synthetic scaffolding, not a trained gate.
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np

# Order of the child seed streams spawned from SeedSequence([2026, c]).
STREAMS = ("placement", "tokens", "pref", "prof_tokens", "prof_x", "x", "Wg",
           "ebias", "W13", "W2", "shared", "k_req", "partials")

PROFILE_TOKENS = 65536


@dataclasses.dataclass(frozen=True)
class LayerConfig:
    name: str
    seed_id: int
    T: int
    H: int
    E: int
    k: int               # top-k (maximum k when ragged)
    I: int
    P: int
    V: int
    dtype: str           # "f32" or "bf16"
    gate: str            # "softmax" or "sigmoid_grouped"
    renorm: bool
    route_scale: float = 1.0
    n_shared: int = 0
    I_shared: int = 0
    n_rgroups: int = 1
    topk_rgroups: int = 1
    rgroup_topn: int = 0
    aff_bias: float = 0.0
    n_pref: int = 0
    zipf_s: Optional[float] = None     # None: uniform token IDs
    ragged: bool = False               # per-request k (MoE-Prism)
    req_tokens: int = 0                # tokens per request when ragged
    k_choices: tuple = ()              # k values drawn per request
    sub_split: int = 1                 # sub-experts per parent (MoE-Prism)
    ebias_range: float = 0.0           # per-expert selection bias U(-r, r)

    @property
    def A_max(self) -> int:
        return self.T * self.k

    @property
    def parents(self) -> int:
        return self.E // self.sub_split

    def replace(self, **kw) -> "LayerConfig":
        return dataclasses.replace(self, **kw)


CONFIGS = {
    # tiny fp32 parity case
    "tiny": LayerConfig("tiny", 1, T=64, H=128, E=8, k=2, I=256, P=2, V=512,
                        dtype="f32", gate="softmax", renorm=True),
    # DeepSeek-V2-Lite-shaped
    "dsv2lite": LayerConfig("dsv2lite", 2, T=4096, H=2048, E=64, k=6, I=1408, P=8,
                            V=102400, dtype="bf16", gate="softmax", renorm=False,
                            n_shared=2, I_shared=1408, aff_bias=3.0, n_pref=6,
                            zipf_s=1.1),
    # Qwen3-30B-A3B-shaped prefill
    "qwen3": LayerConfig("qwen3", 3, T=16384, H=2048, E=128, k=8, I=768, P=8,
                         V=151936, dtype="bf16", gate="softmax", renorm=True,
                         aff_bias=2.5, n_pref=8, zipf_s=1.05),
    # DeepSeek-V3-shaped, decode and prefill batches of one layer
    "dsv3_decode": LayerConfig("dsv3_decode", 4, T=256, H=7168, E=256, k=8, I=2048,
                               P=8, V=129280, dtype="bf16", gate="sigmoid_grouped",
                               renorm=True, route_scale=2.5, n_shared=1,
                               I_shared=2048, n_rgroups=8, topk_rgroups=4,
                               rgroup_topn=2, aff_bias=3.0, n_pref=8, zipf_s=1.1,
                               ebias_range=0.1),
    "dsv3_prefill": LayerConfig("dsv3_prefill", 4, T=8192, H=7168, E=256, k=8,
                                I=2048, P=8, V=129280, dtype="bf16",
                                gate="sigmoid_grouped", renorm=True,
                                route_scale=2.5, n_shared=1, I_shared=2048,
                                n_rgroups=8, topk_rgroups=4, rgroup_topn=2,
                                aff_bias=3.0, n_pref=8, zipf_s=1.1,
                                ebias_range=0.1),
    # MoE-Prism: Qwen3-shaped experts split into 4 neuron slices each
    "prism": LayerConfig("prism", 5, T=8192, H=2048, E=512, k=32, I=192, P=8,
                         V=151936, dtype="bf16", gate="softmax", renorm=True,
                         aff_bias=2.5, n_pref=32, zipf_s=1.05, ragged=True,
                         req_tokens=128, k_choices=(8, 12, 16, 20, 24, 28, 32),
                         sub_split=4),
}

# The DeepSeek-V3 decode batch is the first 256 tokens of the prefill draw.
_DRAW_T = {"dsv3_decode": 8192}


def _streams(cfg: LayerConfig):
    root = np.random.SeedSequence([2026, cfg.seed_id])
    return dict(zip(STREAMS, root.spawn(len(STREAMS))))


def _rng(ss) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(ss))


def _torch_seed(ss) -> int:
    return int(ss.generate_state(1, dtype=np.uint64)[0] & np.uint64(2**63 - 1))


def bounded_zipf(rng: np.random.Generator, s: float, V: int, n: int) -> np.ndarray:
    """IDs in [0, V) with P(id = r-1) proportional to r^-s (r = 1..V)."""
    r = np.arange(1, V + 1, dtype=np.float64)
    pmf = r ** (-s)
    cdf = np.cumsum(pmf)
    cdf /= cdf[-1]
    u = rng.random(n)
    ids = np.searchsorted(cdf, u, side="right")
    return np.minimum(ids, V - 1).astype(np.int32)


def draw_tokens(cfg: LayerConfig, rng: np.random.Generator, n: int) -> np.ndarray:
    if cfg.zipf_s is None:
        return rng.integers(0, cfg.V, size=n, dtype=np.int32)
    return bounded_zipf(rng, cfg.zipf_s, cfg.V, n)


@dataclasses.dataclass
class Tables:
    """Small host-side integer/float structures of one layer."""
    slot_to_orig: np.ndarray   # [E] int32: expert held by each slot
    perm: np.ndarray           # [E] int32: slot of each original expert
    tok: np.ndarray            # [T] int32 token IDs
    pref: Optional[np.ndarray]  # [V, n_pref] int32 original expert IDs, or None
    k_tok: Optional[np.ndarray]  # [T] int32 per-token k when ragged, else None
    ebias: Optional[np.ndarray]  # [E] float32 per-expert selection bias (orig order)
    prof_tok: np.ndarray       # [PROFILE_TOKENS] int32 profiling-draw token IDs


def make_tables(cfg: LayerConfig, profile_tokens: int = PROFILE_TOKENS) -> Tables:
    st = _streams(cfg)
    E, P = cfg.E, cfg.P
    # placement: random permutation; slot s belongs to group s // (E/P)
    slot_to_orig = _rng(st["placement"]).permutation(E).astype(np.int32)
    perm = np.empty(E, np.int32)
    perm[slot_to_orig] = np.arange(E, dtype=np.int32)

    T_draw = _DRAW_T.get(cfg.name, cfg.T)
    tok = draw_tokens(cfg, _rng(st["tokens"]), T_draw)[: cfg.T].copy()

    pref = None
    if cfg.n_pref > 0:
        rng = _rng(st["pref"])
        n_par = cfg.n_pref // cfg.sub_split
        # n_par distinct parents per token ID: first n_par columns of a random
        # permutation per row (argsort of uniform keys)
        keys = rng.random((cfg.V, cfg.parents), dtype=np.float32)
        par = np.argsort(keys, axis=1, kind="stable")[:, :n_par].astype(np.int32)
        if cfg.sub_split > 1:
            sub = np.arange(cfg.sub_split, dtype=np.int32)
            pref = (par[:, :, None] * cfg.sub_split + sub[None, None, :]).reshape(cfg.V, -1)
        else:
            pref = par
        pref = np.ascontiguousarray(pref, dtype=np.int32)

    k_tok = None
    if cfg.ragged:
        rng = _rng(st["k_req"])
        n_req = -(-cfg.T // cfg.req_tokens)
        k_req = rng.choice(np.asarray(cfg.k_choices, np.int32), size=n_req)
        k_tok = np.repeat(k_req, cfg.req_tokens)[: cfg.T].astype(np.int32)

    ebias = None
    if cfg.ebias_range > 0:
        r = cfg.ebias_range
        ebias = _rng(st["ebias"]).uniform(-r, r, size=E).astype(np.float32)

    prof_tok = draw_tokens(cfg, _rng(st["prof_tokens"]), profile_tokens)
    return Tables(slot_to_orig, perm, tok, pref, k_tok, ebias, prof_tok)


def _randn(shape, std, gen, device, dtype):
    import torch
    t = torch.randn(shape, generator=gen, device=device, dtype=torch.float32)
    if std != 1.0:
        t.mul_(std)
    return t if dtype == "f32" else t.to(torch.bfloat16)


def _gen(ss, device):
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(_torch_seed(ss))
    return g


def make_x(cfg: LayerConfig, device="cpu", n: Optional[int] = None, stream="x"):
    """Activations x[n, H] ~ N(0,1) (bf16-rounded unless fp32)."""
    st = _streams(cfg)
    n = cfg.T if n is None else n
    T_draw = _DRAW_T.get(cfg.name, n) if stream == "x" else n
    x = _randn((max(T_draw, n), cfg.H), 1.0, _gen(st[stream], device), device, cfg.dtype)
    return x[:n].contiguous() if x.shape[0] != n else x


def make_gate(cfg: LayerConfig, device="cpu"):
    """The gate rows Wg[E, H] alone, as make_weights draws them on `device`
    (the draw depends on the device's generator)."""
    st = _streams(cfg)
    return _randn((cfg.E, cfg.H), cfg.H ** -0.5, _gen(st["Wg"], device), device, cfg.dtype)


def make_partials(cfg: LayerConfig, n_part: int, device="cpu", n: Optional[int] = None):
    """Tensor-parallel partial sums x_part[n_part, n, H] of an attention
    output, each ~ N(0, 1/n_part) so that their sum is ~ N(0, 1)
    (bf16-rounded unless fp32)."""
    st = _streams(cfg)
    n = cfg.T if n is None else n
    return _randn((n_part, n, cfg.H), n_part ** -0.5, _gen(st["partials"], device), device,
                  cfg.dtype)


def make_weights(cfg: LayerConfig, device="cpu"):
    """Dense weights in ORIGINAL expert order.

    Returns dict with
      Wg   [E, H]        gate rows
      W13  [E, 2I, H]    rows [0, I) gate projection W1, rows [I, 2I) up projection W3
      W2   [E, H, I]     down projection
      Wsh13 [2*ns*Is, H] shared experts' W1 rows stacked, then their W3 rows
      Wsh2  [H, ns*Is]   shared experts' W2 concatenated along the intermediate axis
    (the ns shared experts stacked along the intermediate axis form one SwiGLU
    FFN whose output is exactly the sum of theirs).
    For a sub-expert layer (sub_split > 1) the parents are drawn with the
    parent intermediate I*sub_split and sliced into contiguous neuron slices:
    sub-expert 4e+s of parent e owns neurons [s*I, (s+1)*I).
    """
    import torch
    st = _streams(cfg)
    E, H, I = cfg.E, cfg.H, cfg.I
    out = {}
    out["Wg"] = _randn((E, H), H ** -0.5, _gen(st["Wg"], device), device, cfg.dtype)
    if cfg.sub_split == 1:
        out["W13"] = _randn((E, 2 * I, H), H ** -0.5, _gen(st["W13"], device), device, cfg.dtype)
        out["W2"] = _randn((E, H, I), I ** -0.5, _gen(st["W2"], device), device, cfg.dtype)
    else:
        S, Ip, Ep = cfg.sub_split, I * cfg.sub_split, cfg.parents
        w13p = _randn((Ep, 2 * Ip, H), H ** -0.5, _gen(st["W13"], device), device, cfg.dtype)
        w2p = _randn((Ep, H, Ip), Ip ** -0.5, _gen(st["W2"], device), device, cfg.dtype)
        # W1 slice rows then W3 slice rows for each sub-expert
        w1 = w13p[:, :Ip].reshape(Ep, S, I, H)
        w3 = w13p[:, Ip:].reshape(Ep, S, I, H)
        out["W13"] = torch.cat([w1, w3], dim=2).reshape(E, 2 * I, H).contiguous()
        out["W2"] = w2p.reshape(Ep, H, S, I).permute(0, 2, 1, 3).reshape(E, H, I).contiguous()
        del w13p, w2p, w1, w3
    if cfg.n_shared > 0:
        ns, Is = cfg.n_shared, cfg.I_shared
        g = _gen(st["shared"], device)
        w13s = _randn((ns, 2 * Is, H), H ** -0.5, g, device, cfg.dtype)
        w2s = _randn((ns, H, Is), Is ** -0.5, g, device, cfg.dtype)
        w1 = w13s[:, :Is].reshape(ns * Is, H)
        w3 = w13s[:, Is:].reshape(ns * Is, H)
        out["Wsh13"] = torch.cat([w1, w3], dim=0).contiguous()
        out["Wsh2"] = w2s.permute(1, 0, 2).reshape(H, ns * Is).contiguous()
    else:
        out["Wsh13"] = None
        out["Wsh2"] = None
    return out


def make_prof_x(cfg: LayerConfig, device="cpu", n: int = PROFILE_TOKENS):
    return make_x(cfg, device, n=n, stream="prof_x")
