"""ctypes binding of libmoe (include/moe.h): argument marshalling only.

Every step of the layer runs in the HIP library; this module converts torch
tensors to device pointers and the current HIP stream, and raises MoeError on
a non-zero status.  There is no fallback: if libmoe.so is missing or cannot
be loaded, importing the library raises.
"""
from __future__ import annotations

import contextlib
import ctypes
import os
from typing import Optional

import torch  # noqa: F401  (loads the HIP runtime libmoe then binds to)

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmoe.so")
# the same library built with device data checks (moe_debug_errors)
DEBUG_LIB_PATH = os.path.join(_HERE, "libmoe_debug.so")

MOE_OK, MOE_EINVAL, MOE_ESHAPE, MOE_EDTYPE, MOE_EWORKSPACE, MOE_EHIP = 0, -1, -2, -3, -4, -5
MOE_F32, MOE_BF16 = 0, 1
MOE_GATE_SOFTMAX, MOE_GATE_SIGMOID_GROUPED = 0, 1
MOE_FFN_ROUTED, MOE_FFN_SHARED = 0, 1
MOE_DATA_TOKEN_ID, MOE_DATA_LUT, MOE_DATA_SLOT, MOE_DATA_K, MOE_DATA_PLACEMENT, MOE_DATA_PREF = 1, 2, 4, 8, 16, 32
STAGES = ("route", "shuffle", "gather", "ffn_up", "ffn_down", "combine")
MOE_NSTAGES = len(STAGES)


class MoeError(RuntimeError):
    def __init__(self, code, msg):
        super().__init__("libmoe error %d: %s" % (code, msg))
        self.code = code


class moe_cfg(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in
                ("T", "H", "E", "P", "I", "k_max", "ragged", "n_shared", "I_shared", "V",
                 "n_pref", "dtype", "gate", "renorm")] + [
        ("route_scale", ctypes.c_float),
        ("n_rgroups", ctypes.c_int32), ("topk_rgroups", ctypes.c_int32),
        ("rgroup_topn", ctypes.c_int32), ("aff_bias", ctypes.c_float),
        ("fuse_gather", ctypes.c_int32),
        ("weights_blocked", ctypes.c_int32)]


_vp = ctypes.c_void_p


class moe_weights(ctypes.Structure):
    _fields_ = [(n, _vp) for n in ("Wg", "ebias", "slot_to_orig", "W13", "W2", "Wsh13", "Wsh2",
                                   "lut", "pref")]


class moe_inputs(ctypes.Structure):
    _fields_ = [(n, _vp) for n in ("x", "tok", "k_tok")]


class moe_exports(ctypes.Structure):
    _fields_ = [(n, _vp) for n in ("logits", "row_ptr", "topk_slot", "topk_w", "expert_count",
                                   "expert_off", "group_count", "group_off", "pair_count",
                                   "tok_perm", "tok_off", "sorted_to_assign", "assign_to_sorted",
                                   "x_sorted", "y_sorted", "y_shared", "events")]


def _load(path=None):
    path = LIB_PATH if path is None else path
    if not os.path.exists(path):
        raise OSError("%s is not built; run: python -m token_routing_shuffle_amd.build" % path)
    lib = ctypes.CDLL(path)
    # libmoe must bind to the HIP runtime torch already loaded (same SONAME);
    # two runtimes in one process would not share streams or allocations.
    with open("/proc/self/maps") as f:
        hips = {ln.split()[-1] for ln in f if "libamdhip64" in ln}
    if len(hips) > 1:
        raise OSError("two HIP runtimes mapped: %s" % sorted(hips))
    i32, sz, vp = ctypes.c_int32, ctypes.c_size_t, ctypes.c_void_p
    P = ctypes.POINTER
    lib.moe_validate.restype = i32
    lib.moe_validate.argtypes = [P(moe_cfg)]
    lib.moe_workspace_bytes.restype = sz
    lib.moe_workspace_bytes.argtypes = [P(moe_cfg)]
    lib.moe_route_workspace_bytes.restype = sz
    lib.moe_route_workspace_bytes.argtypes = [P(moe_cfg)]
    lib.moe_last_error.restype = ctypes.c_char_p
    lib.moe_last_error.argtypes = []
    lib.moe_debug_checks.restype = i32
    lib.moe_debug_checks.argtypes = []
    lib.moe_debug_errors.restype = i32
    lib.moe_debug_errors.argtypes = [vp, vp, i32, vp]
    lib.moe_route.restype = i32
    lib.moe_route.argtypes = [P(moe_cfg)] + [vp] * 11 + [vp, sz, vp]
    lib.moe_shuffle.restype = i32
    lib.moe_shuffle.argtypes = [P(moe_cfg)] + [vp] * 15 + [vp, sz, vp]
    lib.moe_shuffle_noalloc.restype = i32
    lib.moe_shuffle_noalloc.argtypes = [P(moe_cfg)] + [vp] * 15 + [vp]
    lib.moe_expert_ffn.restype = i32
    lib.moe_expert_ffn.argtypes = [P(moe_cfg), i32] + [vp] * 7 + [i32, i32, vp, vp, sz, vp]
    lib.moe_combine.restype = i32
    lib.moe_combine.argtypes = [P(moe_cfg)] + [vp] * 7
    lib.moe_srs.restype = i32
    lib.moe_srs.argtypes = [P(moe_cfg), i32, vp, vp, vp, vp]
    lib.moe_sag.restype = i32
    lib.moe_sag.argtypes = [P(moe_cfg), vp, vp, vp, vp]
    lib.moe_token_group_counts.restype = i32
    lib.moe_token_group_counts.argtypes = [P(moe_cfg), i32, vp, vp, vp, vp, vp, vp]
    lib.moe_lut_from_counts.restype = i32
    lib.moe_lut_from_counts.argtypes = [P(moe_cfg), vp, vp, vp]
    lib.moe_expert_group_counts.restype = i32
    lib.moe_expert_group_counts.argtypes = [P(moe_cfg), i32, vp, vp, vp, vp, vp, vp]
    lib.moe_balanced_assign.restype = ctypes.c_int64
    lib.moe_balanced_assign.argtypes = [i32, i32, vp, vp]
    lib.moe_optimize_placement.restype = i32
    lib.moe_optimize_placement.argtypes = [P(moe_cfg), i32, vp, vp, vp, i32, vp, vp, vp, vp, vp, vp,
                                           vp, vp]
    lib.moe_request_group_hist.restype = i32
    lib.moe_request_group_hist.argtypes = [P(moe_cfg), i32, vp, vp, vp, vp, vp]
    lib.moe_forward.restype = i32
    lib.moe_forward.argtypes = [P(moe_cfg), P(moe_weights), P(moe_inputs), vp, P(moe_exports),
                                vp, sz, vp]
    lib.moe_sigmoid.restype = i32
    lib.moe_sigmoid.argtypes = [vp, vp, ctypes.c_int64, vp]
    lib.moe_pack_weights.restype = i32
    lib.moe_pack_weights.argtypes = [P(moe_cfg), i32, vp, vp, vp, vp, vp]
    return lib


_lib = None
_variants = {}


def lib():
    global _lib
    if _lib is None:
        _lib = _load()
    return _lib


@contextlib.contextmanager
def use_library(path):
    """Route every wrapper below to another build of the library (e.g. the
    device-data-check build at DEBUG_LIB_PATH) inside the block."""
    global _lib
    if path not in _variants:
        _variants[path] = _load(path)
    prev = lib()
    _lib = _variants[path]
    try:
        yield _lib
    finally:
        _lib = prev


EXPORTED = ("moe_validate", "moe_workspace_bytes", "moe_route_workspace_bytes", "moe_last_error",
            "moe_route", "moe_shuffle", "moe_shuffle_noalloc",
            "moe_expert_ffn", "moe_combine", "moe_forward", "moe_srs", "moe_sag",
            "moe_token_group_counts", "moe_lut_from_counts", "moe_expert_group_counts",
            "moe_balanced_assign", "moe_optimize_placement", "moe_request_group_hist",
            "moe_sigmoid", "moe_pack_weights", "moe_debug_checks", "moe_debug_errors")


def _p(t) -> Optional[int]:
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream):
    if stream is not None:
        return stream if isinstance(stream, int) else stream.cuda_stream
    return torch.cuda.current_stream().cuda_stream


def _check(rc, name):
    if rc != MOE_OK:
        raise MoeError(rc, "%s: %s" % (name, lib().moe_last_error().decode()))


def make_cfg(layer, **over) -> moe_cfg:
    """moe_cfg from a workload.LayerConfig (or any object with the same fields)."""
    c = moe_cfg()
    c.T, c.H, c.E, c.P, c.I = layer.T, layer.H, layer.E, layer.P, layer.I
    c.k_max = layer.k
    c.ragged = int(layer.ragged)
    c.n_shared, c.I_shared = layer.n_shared, layer.I_shared
    c.V, c.n_pref = layer.V, layer.n_pref
    c.dtype = MOE_BF16 if layer.dtype == "bf16" else MOE_F32
    c.gate = MOE_GATE_SIGMOID_GROUPED if layer.gate == "sigmoid_grouped" else MOE_GATE_SOFTMAX
    c.renorm = int(layer.renorm)
    c.route_scale = layer.route_scale
    c.n_rgroups, c.topk_rgroups, c.rgroup_topn = layer.n_rgroups, layer.topk_rgroups, layer.rgroup_topn
    c.aff_bias = layer.aff_bias
    c.fuse_gather = 0
    c.weights_blocked = 0
    for k, v in over.items():
        setattr(c, k, v)
    return c


def moe_validate(cfg: moe_cfg) -> int:
    return lib().moe_validate(ctypes.byref(cfg))


def moe_workspace_bytes(cfg: moe_cfg) -> int:
    return lib().moe_workspace_bytes(ctypes.byref(cfg))


def moe_last_error() -> str:
    return lib().moe_last_error().decode()


def moe_route_workspace_bytes(cfg: moe_cfg) -> int:
    return lib().moe_route_workspace_bytes(ctypes.byref(cfg))


def route_workspace(cfg: moe_cfg, device="cuda"):
    """Device workspace for moe_route alone (None when the layer needs none);
    its data-error word (first bytes) is cleared."""
    n = moe_route_workspace_bytes(cfg)
    if n == 0:
        return None
    ws = torch.empty(n, dtype=torch.uint8, device=device)
    ws[:256].zero_()
    return ws


def workspace(cfg: moe_cfg, device="cuda"):
    """Device workspace for every call of this layer; its data-error word
    (first bytes) is cleared."""
    n = moe_workspace_bytes(cfg)
    if n == 0 and moe_validate(cfg) != MOE_OK:
        raise MoeError(moe_validate(cfg), moe_last_error())
    ws = torch.empty(max(n, 256), dtype=torch.uint8, device=device)
    ws[:256].zero_()
    return ws


def moe_debug_checks() -> int:
    return lib().moe_debug_checks()


def moe_debug_errors(ws=None, clear=True, stream=None) -> int:
    """moe_data_error bits recorded in workspace ws (None: the static scratch
    of moe_shuffle_noalloc); synchronous; debug builds only."""
    flags = ctypes.c_uint32(0)
    rc = lib().moe_debug_errors(_p(ws), ctypes.byref(flags), int(bool(clear)), _stream(stream))
    _check(rc, "moe_debug_errors")
    return flags.value


def _ws(ws):
    return (None, 0) if ws is None else (ws.data_ptr(), ws.numel() * ws.element_size())


def moe_route(cfg, x, Wg, ebias, slot_to_orig, tok, pref, k_tok, row_ptr, topk_slot, topk_w,
              logits=None, ws=None, stream=None):
    wp, wb = _ws(ws)
    rc = lib().moe_route(ctypes.byref(cfg), _p(x), _p(Wg), _p(ebias), _p(slot_to_orig), _p(tok),
                         _p(pref), _p(k_tok), _p(row_ptr), _p(topk_slot), _p(topk_w), _p(logits),
                         wp, wb, _stream(stream))
    _check(rc, "moe_route")


def moe_shuffle(cfg, row_ptr, topk_slot, tok, lut, x, expert_count, expert_off, group_count,
                group_off, pair_count, tok_perm, tok_off, sorted_to_assign, assign_to_sorted,
                x_sorted=None, ws=None, stream=None):
    wp, wb = _ws(ws)
    rc = lib().moe_shuffle(ctypes.byref(cfg), _p(row_ptr), _p(topk_slot), _p(tok), _p(lut), _p(x),
                           _p(expert_count), _p(expert_off), _p(group_count), _p(group_off),
                           _p(pair_count), _p(tok_perm), _p(tok_off), _p(sorted_to_assign),
                           _p(assign_to_sorted), _p(x_sorted), wp, wb, _stream(stream))
    _check(rc, "moe_shuffle")


def moe_shuffle_noalloc(cfg, row_ptr, topk_slot, tok, lut, x, expert_count, expert_off, group_count,
                        group_off, pair_count, tok_perm, tok_off, sorted_to_assign, assign_to_sorted,
                        x_sorted=None, stream=None):
    """moe_shuffle with its scratch in the library's static device array
    (no workspace; nothing allocated)."""
    rc = lib().moe_shuffle_noalloc(ctypes.byref(cfg), _p(row_ptr), _p(topk_slot), _p(tok), _p(lut), _p(x),
                                   _p(expert_count), _p(expert_off), _p(group_count), _p(group_off),
                                   _p(pair_count), _p(tok_perm), _p(tok_off), _p(sorted_to_assign),
                                   _p(assign_to_sorted), _p(x_sorted), _stream(stream))
    _check(rc, "moe_shuffle_noalloc")


def moe_expert_ffn(cfg, which, x_sorted, x, row_ptr, sorted_to_assign, expert_off, W13, W2,
                   e_begin, e_end, y, ws=None, stream=None):
    wp, wb = _ws(ws)
    rc = lib().moe_expert_ffn(ctypes.byref(cfg), which, _p(x_sorted), _p(x), _p(row_ptr),
                              _p(sorted_to_assign), _p(expert_off), _p(W13), _p(W2), e_begin,
                              e_end, _p(y), wp, wb, _stream(stream))
    _check(rc, "moe_expert_ffn")


def moe_combine(cfg, y_sorted, assign_to_sorted, row_ptr, topk_w, y_sh, out, stream=None):
    rc = lib().moe_combine(ctypes.byref(cfg), _p(y_sorted), _p(assign_to_sorted), _p(row_ptr),
                           _p(topk_w), _p(y_sh), _p(out), _stream(stream))
    _check(rc, "moe_combine")


def moe_srs(cfg, n_part, x_part, tok_perm, y, stream=None):
    rc = lib().moe_srs(ctypes.byref(cfg), int(n_part), _p(x_part), _p(tok_perm), _p(y),
                       _stream(stream))
    _check(rc, "moe_srs")


def moe_sag(cfg, y, tok_perm, out, stream=None):
    rc = lib().moe_sag(ctypes.byref(cfg), _p(y), _p(tok_perm), _p(out), _stream(stream))
    _check(rc, "moe_sag")


def _host_ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def moe_token_group_counts(cfg, n_tok, row_ptr, expert, tok, group, counts, stream=None):
    rc = lib().moe_token_group_counts(ctypes.byref(cfg), int(n_tok), _p(row_ptr), _p(expert), _p(tok),
                                      _p(group), _p(counts), _stream(stream))
    _check(rc, "moe_token_group_counts")


def moe_lut_from_counts(cfg, counts, lut, stream=None):
    rc = lib().moe_lut_from_counts(ctypes.byref(cfg), _p(counts), _p(lut), _stream(stream))
    _check(rc, "moe_lut_from_counts")


def moe_expert_group_counts(cfg, n_tok, row_ptr, expert, tok, lut, counts, stream=None):
    rc = lib().moe_expert_group_counts(ctypes.byref(cfg), int(n_tok), _p(row_ptr), _p(expert),
                                       _p(tok), _p(lut), _p(counts), _stream(stream))
    _check(rc, "moe_expert_group_counts")


def moe_balanced_assign(score):
    """score: host int64 array [n, P]; returns (group int32 [n], optimum)."""
    import numpy as np
    score = np.ascontiguousarray(score, dtype=np.int64)
    n, P = score.shape
    group = np.zeros(n, np.int32)
    best = lib().moe_balanced_assign(n, P, _host_ptr(score), _host_ptr(group))
    if best < 0:
        _check(int(best), "moe_balanced_assign")
    return group, int(best)


def moe_optimize_placement(cfg, n_tok, row_ptr, expert, tok, group0, lut, counts_vp, counts_pe,
                           max_iters=20, stream=None):
    """Returns (group, perm, objective trace) as host arrays; lut (device) is
    filled with the final token table."""
    import numpy as np
    group = np.ascontiguousarray(group0, dtype=np.int32).copy()
    perm = np.zeros_like(group)
    obj = np.zeros(2 * max_iters, np.int64)
    n_steps = ctypes.c_int32(0)
    rc = lib().moe_optimize_placement(ctypes.byref(cfg), int(n_tok), _p(row_ptr), _p(expert), _p(tok),
                                      int(max_iters), _host_ptr(group), _host_ptr(perm), _p(lut),
                                      _p(counts_vp), _p(counts_pe), _host_ptr(obj),
                                      ctypes.byref(n_steps), _stream(stream))
    _check(rc, "moe_optimize_placement")
    return group, perm, obj[:n_steps.value]


def moe_request_group_hist(cfg, n_req, req_ptr, tok, lut, hist, stream=None):
    rc = lib().moe_request_group_hist(ctypes.byref(cfg), int(n_req), _p(req_ptr), _p(tok), _p(lut),
                                      _p(hist), _stream(stream))
    _check(rc, "moe_request_group_hist")


def moe_pack_weights(cfg, which, W13, W2, W13_blk, W2_blk, stream=None):
    """W13/W2 (routed or shared) into the tile-blocked layout of cfg."""
    rc = lib().moe_pack_weights(ctypes.byref(cfg), int(which), _p(W13), _p(W2), _p(W13_blk), _p(W2_blk),
                                _stream(stream))
    _check(rc, "moe_pack_weights")


def moe_sigmoid(x, y, n=None, stream=None):
    """y[:n] = the selection sigmoid of x[:n] (fp32 device tensors)."""
    n = x.numel() if n is None else int(n)
    rc = lib().moe_sigmoid(_p(x), _p(y), n, _stream(stream))
    _check(rc, "moe_sigmoid")


def moe_forward(cfg, weights: moe_weights, inputs: moe_inputs, out, exports=None, ws=None,
                stream=None):
    wp, wb = _ws(ws)
    ex = ctypes.byref(exports) if exports is not None else None
    rc = lib().moe_forward(ctypes.byref(cfg), ctypes.byref(weights), ctypes.byref(inputs), _p(out),
                           ex, wp, wb, _stream(stream))
    _check(rc, "moe_forward")


def weights_struct(d) -> moe_weights:
    """moe_weights from a dict of device tensors (missing / None entries -> NULL)."""
    w = moe_weights()
    for name, _ in moe_weights._fields_:
        setattr(w, name, _p(d.get(name)))
    return w


def inputs_struct(x, tok, k_tok=None) -> moe_inputs:
    i = moe_inputs()
    i.x, i.tok, i.k_tok = _p(x), _p(tok), _p(k_tok)
    return i


def exports_struct(d=None, events=None):
    """moe_exports from a dict of device tensors; ``events`` is a list of
    2*MOE_NSTAGES torch.cuda.Event (already recorded once) or None."""
    e = moe_exports()
    d = d or {}
    for name, _ in moe_exports._fields_:
        if name != "events":
            setattr(e, name, _p(d.get(name)))
    keep = None
    if events is not None:
        arr = (ctypes.c_void_p * (2 * MOE_NSTAGES))()
        for i, ev in enumerate(events):
            arr[i] = None if ev is None else ev.cuda_event
        e.events = ctypes.cast(arr, ctypes.c_void_p)
        keep = arr
    e._keep = keep  # keep the handle array alive with the struct
    return e
