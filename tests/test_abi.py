"""C-ABI boundary checks that need no GPU: the library loads, exports every
entry point include/moe.h declares, validates descriptions on the host and
rejects bad arguments before anything is enqueued."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def m():
    from token_routing_shuffle_amd import moe
    if not os.path.exists(moe.LIB_PATH):
        from token_routing_shuffle_amd import build
        build.build()
    moe.lib()
    return moe


def declared_functions():
    src = open(os.path.join(ROOT, "include", "moe.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:int32_t|int64_t|size_t|const char\*)\s+(moe_\w+)\s*\(", src, re.M)))


def test_header_declares_the_boundary():
    assert declared_functions() == sorted([
        "moe_combine", "moe_expert_ffn", "moe_forward", "moe_last_error", "moe_route",
        "moe_sag", "moe_shuffle", "moe_srs", "moe_validate", "moe_workspace_bytes",
        "moe_route_workspace_bytes",
        "moe_token_group_counts", "moe_lut_from_counts", "moe_expert_group_counts",
        "moe_balanced_assign", "moe_optimize_placement", "moe_request_group_hist",
        "moe_sigmoid", "moe_pack_weights", "moe_shuffle_noalloc", "moe_debug_checks",
        "moe_debug_errors"])


def test_library_exports_every_declared_symbol(m):
    lib = m.lib()
    for name in declared_functions():
        assert hasattr(lib, name), name
    assert sorted(m.EXPORTED) == declared_functions()


def test_struct_layouts_match_header(m):
    # moe_cfg: 21 int32/float fields, no padding; moe_exports: 17 pointers
    assert ctypes.sizeof(m.moe_cfg) == 21 * 4
    assert ctypes.sizeof(m.moe_weights) == 9 * 8
    assert ctypes.sizeof(m.moe_inputs) == 3 * 8
    assert ctypes.sizeof(m.moe_exports) == 17 * 8
    hdr = open(os.path.join(ROOT, "include", "moe.h")).read()
    body = hdr[hdr.index("typedef struct moe_cfg"):hdr.index("} moe_cfg;")]
    names = re.findall(r"^\s*(?:int32_t|float)\s+(\w+);", body, re.M)
    assert names == [f for f, _ in m.moe_cfg._fields_]


def _cfgs(m):
    from token_routing_shuffle_amd import workload as wl
    return {n: m.make_cfg(c) for n, c in wl.CONFIGS.items()}


def test_every_workload_config_validates(m):
    for name, c in _cfgs(m).items():
        assert m.moe_validate(c) == m.MOE_OK, (name, m.moe_last_error())
        assert m.moe_workspace_bytes(c) > 0


def test_profiling_chunks_validate(m):
    """The offline profile routes its 65536-token draw in chunks; every
    chunk's layer configuration must pass validation."""
    from token_routing_shuffle_amd import offline
    from token_routing_shuffle_amd import workload as wl
    for name, cfg in wl.CONFIGS.items():
        n = offline.route_chunk(cfg)
        assert 1 <= n <= 16384
        assert m.moe_validate(m.make_cfg(cfg, T=n)) == m.MOE_OK, (name, n, m.moe_last_error())
    assert offline.route_chunk(wl.CONFIGS["dsv3_prefill"].replace(H=131072)) == 8191


@pytest.mark.parametrize("field,value,code", [
    ("E", 12, "MOE_ESHAPE"),            # E/P = 1.5
    ("P", 3, "MOE_ESHAPE"),             # E % P != 0
    ("k_max", 0, "MOE_ESHAPE"),
    ("k_max", 65, "MOE_ESHAPE"),
    ("H", 100, "MOE_ESHAPE"),           # bf16 needs H % 128
    ("I", 1400, "MOE_ESHAPE"),          # bf16 needs I % 64
    ("dtype", 7, "MOE_EDTYPE"),
    ("gate", 5, "MOE_EDTYPE"),
    ("T", -1, "MOE_ESHAPE"),
    ("V", 0, "MOE_ESHAPE"),
    ("n_pref", 65, "MOE_ESHAPE"),
    ("ragged", 2, "MOE_EINVAL"),
    ("weights_blocked", 2, "MOE_EINVAL"),
    ("weights_blocked", -1, "MOE_EINVAL"),
    ("E", 1024, "MOE_ESHAPE"),
    ("T", 524288, "MOE_ESHAPE"),        # bf16 x [T,H] = 524288*2048*2 B = 2 GiB
])
def test_validate_rejects(m, field, value, code):
    c = _cfgs(m)["dsv2lite"]
    setattr(c, field, value)
    assert m.moe_validate(c) == getattr(m, code)
    assert m.moe_last_error()
    assert m.moe_workspace_bytes(c) == 0


def test_validate_accepts_rows_just_below_the_offset_limit(m):
    """The sorted-row operands of the grouped GEMMs are addressed per tile:
    T * k * H * 2 may exceed 2 GiB; the activations x [T,H] may not."""
    c = _cfgs(m)["dsv2lite"]
    c.T = (2 ** 31 - 1) // (c.H * 2)               # 524287 tokens, 6.4 GB of sorted rows
    assert c.T * c.k_max * c.H * 2 > 2 ** 32
    assert m.moe_validate(c) == m.MOE_OK, m.moe_last_error()
    c.T += 1
    assert m.moe_validate(c) == m.MOE_ESHAPE


def test_validate_rejects_weights_beyond_the_offset_limit(m):
    """One expert's W13 [2I,H] (and the stacked shared experts', and the gate
    [E,H]) are addressed through 32-bit buffer offsets: each must stay below
    2 GiB."""
    c = _cfgs(m)["dsv2lite"]
    c.H, c.I, c.n_shared, c.I_shared = 32768, 16384 - 64, 0, 0
    assert m.moe_validate(c) == m.MOE_OK, m.moe_last_error()   # 2*I*H*2 just below 2 GiB
    c.I = 16384
    assert m.moe_validate(c) == m.MOE_ESHAPE                     # exactly 2 GiB
    c = _cfgs(m)["dsv2lite"]
    c.H, c.n_shared, c.I_shared = 32768, 1, 16384
    assert m.moe_validate(c) == m.MOE_ESHAPE                     # shared [2*Is,H] = 2 GiB
    c = _cfgs(m)["dsv2lite"]
    c.E, c.H, c.P, c.n_shared, c.I_shared = 512, 2 ** 21, 8, 0, 0
    c.I, c.T = 64, 16
    assert m.moe_validate(c) == m.MOE_ESHAPE                     # gate [E,H] = 2 GiB


def test_validate_sigmoid_group_rules(m):
    base = _cfgs(m)["dsv3_prefill"]
    assert m.moe_validate(base) == m.MOE_OK
    for field, value in [("n_rgroups", 7), ("topk_rgroups", 9), ("topk_rgroups", 0),
                         ("rgroup_topn", 0), ("rgroup_topn", 33)]:
        c = _cfgs(m)["dsv3_prefill"]
        setattr(c, field, value)
        assert m.moe_validate(c) == m.MOE_ESHAPE, (field, value)
    c = _cfgs(m)["dsv3_prefill"]
    c.k_max, c.topk_rgroups = 64, 1          # one kept group of 32 experts < k
    assert m.moe_validate(c) == m.MOE_ESHAPE


def test_validate_null_cfg(m):
    assert m.lib().moe_validate(None) == m.MOE_EINVAL


def test_calls_reject_null_pointers_before_launching(m):
    c = _cfgs(m)["dsv2lite"]
    L = m.lib()
    ref = ctypes.byref(c)
    assert L.moe_route(ref, *([None] * 11), None, 0, None) == m.MOE_EINVAL
    assert "NULL" in m.moe_last_error()
    assert L.moe_shuffle(ref, *([None] * 15), None, 0, None) == m.MOE_EINVAL
    assert L.moe_expert_ffn(ref, 0, *([None] * 7), 0, 64, None, None, 0, None) == m.MOE_EINVAL
    assert L.moe_expert_ffn(ref, 9, *([None] * 7), 0, 64, None, None, 0, None) == m.MOE_EINVAL
    assert L.moe_combine(ref, *([None] * 7)) == m.MOE_EINVAL
    w, i = m.moe_weights(), m.moe_inputs()
    assert L.moe_forward(ref, ctypes.byref(w), ctypes.byref(i), None, None, None, 0, None) == m.MOE_EINVAL
    assert L.moe_sigmoid(None, None, 10, None) == m.MOE_EINVAL
    assert L.moe_sigmoid(None, None, -1, None) == m.MOE_EINVAL
    assert L.moe_sigmoid(None, None, 0, None) == m.MOE_OK


def test_blocked_weights_rules(m):
    """The tile-blocked weight layout exists for bf16 layers only, and
    moe_pack_weights rejects bad arguments before it launches anything."""
    c = _cfgs(m)["dsv2lite"]
    c.weights_blocked = 1
    assert m.moe_validate(c) == m.MOE_OK, m.moe_last_error()
    c.dtype = m.MOE_F32
    assert m.moe_validate(c) == m.MOE_EDTYPE
    c.dtype = m.MOE_BF16
    L = m.lib()
    ref = ctypes.byref(c)
    fake = 1 << 40   # never dereferenced: the checks fail first
    assert L.moe_pack_weights(ref, 5, fake, fake, fake + 4096, fake + 8192, None) == m.MOE_EINVAL
    assert L.moe_pack_weights(ref, m.MOE_FFN_ROUTED, None, fake, fake, fake, None) == m.MOE_EINVAL
    assert L.moe_pack_weights(ref, m.MOE_FFN_ROUTED, fake, fake, fake, fake + 8192, None) == m.MOE_EINVAL
    assert "alias" in m.moe_last_error()
    assert L.moe_pack_weights(ref, m.MOE_FFN_ROUTED, fake + 2, fake, fake + 4096, fake + 8192,
                              None) == m.MOE_EINVAL
    assert "aligned" in m.moe_last_error()
    c.n_shared = 0
    assert L.moe_pack_weights(ref, m.MOE_FFN_SHARED, fake, fake, fake + 4096, fake + 8192,
                              None) == m.MOE_EINVAL
    assert "shared" in m.moe_last_error()
    c.n_shared = 2
    c.dtype = m.MOE_F32
    c.weights_blocked = 0
    assert L.moe_pack_weights(ref, m.MOE_FFN_ROUTED, fake, fake, fake + 4096, fake + 8192,
                              None) == m.MOE_EDTYPE


def test_calls_reject_small_or_misaligned_workspace(m):
    c = _cfgs(m)["tiny"]
    L = m.lib()
    need = m.moe_workspace_bytes(c)
    fake = 1 << 40   # never dereferenced: the checks fail first
    ptrs = [fake] * 15
    rc = L.moe_shuffle(ctypes.byref(c), *ptrs, None, 0, None)
    assert rc == m.MOE_EWORKSPACE
    rc = L.moe_shuffle(ctypes.byref(c), *ptrs, fake + 8, need, None)
    assert rc == m.MOE_EWORKSPACE and "aligned" in m.moe_last_error()
    rc = L.moe_shuffle(ctypes.byref(c), *ptrs, fake, 256, None)
    assert rc == m.MOE_EWORKSPACE
    w = m.moe_weights(Wg=fake, slot_to_orig=fake, W13=fake, W2=fake, lut=fake)
    i = m.moe_inputs(x=fake, tok=fake)
    rc = L.moe_forward(ctypes.byref(c), ctypes.byref(w), ctypes.byref(i), fake, None, fake, need - 1, None)
    assert rc == m.MOE_EWORKSPACE


def test_calls_reject_misaligned_tensors(m):
    c = _cfgs(m)["dsv2lite"]
    L = m.lib()
    fake = 1 << 40
    rc = L.moe_route(ctypes.byref(c), fake + 2, fake, None, fake, fake, None, None, fake, fake,
                     fake, None, None, 0, None)
    assert rc == m.MOE_EINVAL and "aligned" in m.moe_last_error()


def test_route_workspace(m):
    """bf16 layers with E >= 128 need a route workspace (the tiled gate GEMM's
    partial logits, within the layer workspace); moe_route rejects a missing
    one before launching anything; E = 64 and fp32 layers need none."""
    cf = _cfgs(m)
    for name in ("tiny", "dsv2lite"):
        assert m.moe_route_workspace_bytes(cf[name]) == 0, name
    for name in ("qwen3", "prism", "dsv3_decode", "dsv3_prefill"):
        c = cf[name]
        n = m.moe_route_workspace_bytes(c)
        assert n >= c.T * c.E * 4, name
        assert n <= m.moe_workspace_bytes(c), name
    c = cf["qwen3"]
    fake = 1 << 40
    rc = m.lib().moe_route(ctypes.byref(c), fake, fake, None, fake, fake, None, None, fake, fake,
                           fake, None, None, 0, None)
    assert rc == m.MOE_EWORKSPACE
    bad = _cfgs(m)["qwen3"]
    bad.E = 12
    assert m.moe_route_workspace_bytes(bad) == 0


def test_route_workspace_gate_slices(m):
    """The route workspace holds the tiled gate GEMM's K slices of partial
    logits, S * T * E fp32 after the dispatch tables.  Layers with at least
    32 tiles of 128 tokens x 256 experts (128 when E < 256) take those wide
    tiles, others 64 x 128 tiles; S doubles while the blocks number under
    256 and each slice keeps at least four 64-wide chunks."""
    from token_routing_shuffle_amd import workload as wl
    for name, T, over, S in [("dsv3_prefill", 8192, {}, 4),      # 64 wide tiles
                             ("dsv3_prefill", 4097, {}, 8),      # 33 wide tiles
                             ("dsv3_prefill", 3969, {}, 8),      # 32 wide tiles: the smallest wide layer
                             ("dsv3_prefill", 3968, {}, 4),      # 31: 62 x 2 narrow tiles
                             ("qwen3", 16384, {}, 2),            # 128 wide tiles of 128 experts
                             ("qwen3", 4100, dict(E=192, P=3), 4),  # 33 x 2, partial expert tile
                             ("prism", 8192, {}, 2),             # 64 x 2
                             ("prism", 4160, {}, 4),             # 33 x 2
                             ("dsv3_decode", 256, {}, 16),       # 2 wide tiles: 4 x 2 narrow ones
                             ("qwen3", 300, dict(E=192, P=3), 8)]:  # 5 x 2 narrow ones
        c = m.make_cfg(wl.CONFIGS[name], T=T, **over)
        n = m.moe_route_workspace_bytes(c)
        assert n // (T * c.E * 4) == S, (name, T, over, n)


def test_workspace_grows_with_tokens_and_shrinks_with_fused_gather(m):
    from token_routing_shuffle_amd import workload as wl
    c1 = m.make_cfg(wl.CONFIGS["qwen3"], T=1024)
    c2 = m.make_cfg(wl.CONFIGS["qwen3"], T=2048)
    c3 = m.make_cfg(wl.CONFIGS["qwen3"], T=2048, fuse_gather=1)
    assert m.moe_workspace_bytes(c1) < m.moe_workspace_bytes(c2)
    assert m.moe_workspace_bytes(c3) < m.moe_workspace_bytes(c2)
    # the x_sorted buffer (A_max rows of H bf16) is what fusing the gather saves
    assert m.moe_workspace_bytes(c2) - m.moe_workspace_bytes(c3) == 2048 * 8 * 2048 * 2


def test_expert_ffn_empty_layer_reads_no_rows(m):
    """T = 0 (or an empty slot range): moe_expert_ffn returns MOE_OK with the
    row arguments NULL, after checking the rest; nothing is launched."""
    from token_routing_shuffle_amd import workload as wl
    L = m.lib()
    fake = ctypes.c_void_p(0x1000)       # never dereferenced
    c = m.make_cfg(wl.CONFIGS["dsv2lite"], T=0)
    ws_bytes = max(m.moe_workspace_bytes(c), 256)
    for which in (m.MOE_FFN_ROUTED, m.MOE_FFN_SHARED):
        assert L.moe_expert_ffn(ctypes.byref(c), which, None, None, None, None, None, fake, fake, 0, c.E,
                                fake, fake, ws_bytes, None) == m.MOE_OK
    # the weights are still checked
    assert L.moe_expert_ffn(ctypes.byref(c), m.MOE_FFN_ROUTED, None, None, None, None, None, None, fake, 0,
                            c.E, fake, fake, ws_bytes, None) == m.MOE_EINVAL
    # an empty slot range of a non-empty layer
    c1 = m.make_cfg(wl.CONFIGS["dsv2lite"])
    ws1 = m.moe_workspace_bytes(c1)
    assert L.moe_expert_ffn(ctypes.byref(c1), m.MOE_FFN_ROUTED, None, None, None, None, None, fake, fake, 5, 5,
                            fake, fake, ws1, None) == m.MOE_OK
    assert L.moe_expert_ffn(ctypes.byref(c1), m.MOE_FFN_ROUTED, None, None, None, None, None, fake, fake, 0, 5,
                            fake, fake, ws1, None) == m.MOE_EINVAL


def test_empty_layer_validates(m):
    from token_routing_shuffle_amd import workload as wl
    c = m.make_cfg(wl.CONFIGS["tiny"], T=0)
    assert m.moe_validate(c) == m.MOE_OK


def test_srs_sag_reject_bad_arguments_before_launching(m):
    c = _cfgs(m)["dsv2lite"]
    fake = ctypes.c_void_p(0x1000)      # never dereferenced: checks come first
    odd = ctypes.c_void_p(0x1008)
    assert m.lib().moe_srs(ctypes.byref(c), 0, fake, fake, fake, None) == m.MOE_EINVAL
    assert m.lib().moe_srs(ctypes.byref(c), 65, fake, fake, fake, None) == m.MOE_EINVAL
    assert m.lib().moe_srs(ctypes.byref(c), 8, None, fake, fake, None) == m.MOE_EINVAL
    assert m.lib().moe_srs(ctypes.byref(c), 8, odd, fake, fake, None) == m.MOE_EINVAL
    assert m.lib().moe_sag(ctypes.byref(c), fake, None, fake, None) == m.MOE_EINVAL
    assert m.lib().moe_sag(ctypes.byref(c), fake, fake, fake, None) == m.MOE_EINVAL   # y == out
    bad = _cfgs(m)["dsv2lite"]
    bad.P = 3
    assert m.lib().moe_sag(ctypes.byref(bad), fake, fake, fake, None) == m.MOE_ESHAPE
    empty = _cfgs(m)["dsv2lite"]
    empty.T = 0                          # nothing to do, nothing touched
    assert m.lib().moe_srs(ctypes.byref(empty), 8, None, None, None, None) == m.MOE_OK


def test_balanced_assign_host_only(m):
    """The host-only solver runs without a GPU; checked against brute force
    (the same rule the oracle's pin uses, independently of the oracle)."""
    import itertools
    import numpy as np
    rng = np.random.default_rng(4)
    for n, P in [(6, 2), (6, 3), (8, 4), (4, 1), (0, 2)]:
        score = rng.integers(0, 50, size=(n, P))
        g, best = m.moe_balanced_assign(score)
        assert (np.bincount(g, minlength=P) == n // P).all()
        assert best == sum(score[i, g[i]] for i in range(n))
        brute = max([sum(score[i, lab[i]] for i in range(n))
                     for lab in itertools.product(range(P), repeat=n)
                     if all(lab.count(q) == n // P for q in range(P))] or [0])
        assert best == brute
    assert m.lib().moe_balanced_assign(5, 2, None, None) == m.MOE_ESHAPE


def test_coscheduling_calls_reject_bad_arguments(m):
    c = _cfgs(m)["dsv2lite"]
    fake = ctypes.c_void_p(0x1000)
    lib = m.lib()
    assert lib.moe_token_group_counts(ctypes.byref(c), -1, fake, fake, fake, fake, fake, None) == m.MOE_EINVAL
    assert lib.moe_token_group_counts(ctypes.byref(c), 4, None, fake, fake, fake, fake, None) == m.MOE_EINVAL
    assert lib.moe_expert_group_counts(ctypes.byref(c), 4, fake, fake, fake, None, fake, None) == m.MOE_EINVAL
    assert lib.moe_lut_from_counts(ctypes.byref(c), None, fake, None) == m.MOE_EINVAL
    assert lib.moe_request_group_hist(ctypes.byref(c), 3, fake, fake, fake, None, None) == m.MOE_EINVAL
    import numpy as np
    group = np.zeros(c.E, np.int32)             # not balanced: every expert in group 0
    rc = lib.moe_optimize_placement(ctypes.byref(c), 4, fake, fake, fake, 5,
                                    group.ctypes.data_as(ctypes.c_void_p), None, fake, fake, fake,
                                    None, None, None)
    assert rc == m.MOE_EINVAL


def test_debug_library_exports_every_declared_symbol_and_reports_its_build(m):
    """libmoe_debug.so (device data checks) has the same ABI; only it records
    data errors, and its route workspace always holds the error word."""
    from token_routing_shuffle_amd import workload as wl
    with m.use_library(m.DEBUG_LIB_PATH) as dbg:
        for name in declared_functions():
            assert hasattr(dbg, name), name
        assert m.moe_debug_checks() == 1
        for name, cfg in wl.CONFIGS.items():
            c = m.make_cfg(cfg)
            assert m.moe_route_workspace_bytes(c) >= 256, name
            assert m.moe_workspace_bytes(c) == m.lib().moe_workspace_bytes(ctypes.byref(c))
        assert dbg.moe_debug_errors(None, None, 0, None) == m.MOE_EINVAL
    assert m.moe_debug_checks() == 0
    flags = ctypes.c_uint32(7)
    assert m.lib().moe_debug_errors(None, ctypes.byref(flags), 0, None) == m.MOE_EINVAL
    assert flags.value == 0
    assert "release build" in m.moe_last_error()
    assert m.lib().moe_debug_errors(None, None, 0, None) == m.MOE_EINVAL
