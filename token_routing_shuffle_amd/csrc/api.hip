// C ABI of libmoe: argument checks, workspace layout and the launch sequence.
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <algorithm>
#include <vector>

#include "internal.h"

namespace moe {
namespace {

thread_local char g_err[512] = "";

int32_t fail(int32_t code, const char* fmt, ...)
{
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof(g_err), fmt, ap);
    va_end(ap);
    return code;
}

int32_t hip_fail(hipError_t e, const char* where)
{
    return fail(MOE_EHIP, "%s: %s", where, hipGetErrorString(e));
}

bool is_pow2(int v) { return v > 0 && (v & (v - 1)) == 0; }
bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

int esize(const moe_cfg& c) { return c.dtype == MOE_BF16 ? 2 : 4; }

int32_t check_cfg(const moe_cfg* cp)
{
    if (cp == nullptr) return fail(MOE_EINVAL, "cfg is NULL");
    const moe_cfg& c = *cp;
    if (c.dtype != MOE_F32 && c.dtype != MOE_BF16) return fail(MOE_EDTYPE, "dtype %d unsupported", c.dtype);
    if (c.gate != MOE_GATE_SOFTMAX && c.gate != MOE_GATE_SIGMOID_GROUPED)
        return fail(MOE_EDTYPE, "gate %d unsupported", c.gate);
    if (c.T < 0 || c.H <= 0 || c.E <= 0 || c.P <= 0 || c.I <= 0 || c.V <= 0)
        return fail(MOE_ESHAPE, "T must be >= 0 and H, E, P, I, V > 0");
    if (c.k_max < 1 || c.k_max > c.E || c.k_max > 64) return fail(MOE_ESHAPE, "k_max must be in [1, min(E, 64)]");
    if (c.E > 512) return fail(MOE_ESHAPE, "E must be <= 512");
    if (c.E % c.P != 0 || !is_pow2(c.E / c.P)) return fail(MOE_ESHAPE, "E/P must be a power-of-two integer");
    if (c.P > 64 || c.E * c.P > 4096) return fail(MOE_ESHAPE, "P <= 64 and E*P <= 4096 required");
    if (c.n_pref < 0 || c.n_pref > c.E) return fail(MOE_ESHAPE, "n_pref must be in [0, E]");
    if (c.ragged != 0 && c.ragged != 1) return fail(MOE_EINVAL, "ragged must be 0 or 1");
    if (c.n_shared < 0 || c.I_shared < 0 || (c.n_shared > 0 && c.I_shared == 0))
        return fail(MOE_ESHAPE, "bad shared-expert sizes");
    if (c.H % 8 != 0) return fail(MOE_ESHAPE, "H must be a multiple of 8");
    if (c.dtype == MOE_BF16) {
        if (c.H % 128 != 0) return fail(MOE_ESHAPE, "bf16 needs H %% 128 == 0");
        if (c.I % 64 != 0) return fail(MOE_ESHAPE, "bf16 needs I %% 64 == 0");
        if ((long long)c.n_shared * c.I_shared % 64 != 0)
            return fail(MOE_ESHAPE, "bf16 needs n_shared*I_shared %% 64 == 0");
    }
    if ((long long)c.T * c.k_max >= (1LL << 31) || (long long)c.T * c.k_max * c.H >= (1LL << 40))
        return fail(MOE_ESHAPE, "T*k_max too large");
    if (c.dtype == MOE_BF16) {
        // 32-bit buffer offsets: the activations x [T,H] (rows gathered by the
        // grouped GEMM and read by the gate kernel), the gate [E,H] and one
        // expert's (or the stacked shared experts') weight matrices must each
        // stay below 2 GiB.  Sorted-row operands are addressed per tile.
        const long long Ish = (long long)c.n_shared * c.I_shared;
        if ((long long)c.T * c.H * 2 >= (1LL << 31)) return fail(MOE_ESHAPE, "bf16 x [T,H] must stay below 2 GiB");
        if ((long long)c.E * c.H * 2 >= (1LL << 31)) return fail(MOE_ESHAPE, "bf16 gate [E,H] must stay below 2 GiB");
        if (2LL * c.I * c.H * 2 >= (1LL << 31) || 2LL * Ish * c.H * 2 >= (1LL << 31))
            return fail(MOE_ESHAPE, "bf16 per-expert weights [2I,H] must stay below 2 GiB");
    }
    if (c.gate == MOE_GATE_SIGMOID_GROUPED) {
        if (c.n_rgroups < 1 || c.n_rgroups > 64 || c.E % c.n_rgroups != 0)
            return fail(MOE_ESHAPE, "n_rgroups must divide E and be in [1, 64]");
        if (c.topk_rgroups < 1 || c.topk_rgroups > c.n_rgroups)
            return fail(MOE_ESHAPE, "topk_rgroups must be in [1, n_rgroups]");
        const int gs = c.E / c.n_rgroups;
        if (c.rgroup_topn < 1 || c.rgroup_topn > 8 || c.rgroup_topn > gs)
            return fail(MOE_ESHAPE, "rgroup_topn must be in [1, min(8, E/n_rgroups)]");
        if (c.n_rgroups > 1 && c.topk_rgroups < c.n_rgroups && c.topk_rgroups * gs < c.k_max)
            return fail(MOE_ESHAPE, "kept routing groups hold fewer than k_max experts");
        if (!(c.route_scale == c.route_scale) || c.route_scale > 3.0e38f || c.route_scale < -3.0e38f)
            return fail(MOE_EINVAL, "route_scale must be finite");
    }
    if (!(c.aff_bias == c.aff_bias)) return fail(MOE_EINVAL, "aff_bias is NaN");
    if (c.weights_blocked != 0 && c.weights_blocked != 1) return fail(MOE_EINVAL, "weights_blocked must be 0 or 1");
    if (c.weights_blocked && c.dtype != MOE_BF16) return fail(MOE_EDTYPE, "blocked weights need bf16");
    return MOE_OK;
}

hipError_t record(const moe_exports* ex, int stage, int end, hipStream_t s)
{
    if (ex == nullptr || ex->events == nullptr) return hipSuccess;
    void* e = ex->events[2 * stage + end];
    if (e == nullptr) return hipSuccess;
    return hipEventRecord((hipEvent_t)e, s);
}

}  // namespace

WsLayout ws_layout(const moe_cfg& c)
{
    WsLayout L;
    memset(&L, 0, sizeof(L));
    size_t off = 0;
    auto take = [&](size_t bytes) {
        const size_t o = off;
        off += (bytes + 255) & ~(size_t)255;
        return o;
    };
    const size_t T = (size_t)c.T, A = (size_t)c.T * c.k_max, E = c.E, P = c.P;
    const size_t es = (size_t)esize(c);
    const size_t Ish = (size_t)c.n_shared * c.I_shared;
    L.tpb = shuffle_tpb(c.T, c.E, c.P);
    L.nb = std::max(1, ceil_div(c.T, L.tpb));
    L.err = take(4);
    L.row_ptr = take((T + 1) * 4);
    L.topk_slot = take(A * 4);
    L.topk_w = take(A * 4);
    L.g_pred = take(T * 4);
    L.hist = take(E * P * L.nb * 4);
    L.thist = take(P * L.nb * 4);
    L.rowtot = take((E * P + P) * 4);
    L.bstart = take((E * P + 1) * 4);
    L.tstart = take((P + 1) * 4);
    L.expert_count = take(E * 4);
    L.expert_off = take((E + 1) * 4);
    L.group_count = take(P * 4);
    L.group_off = take((P + 1) * 4);
    L.pair_count = take(P * P * 4);
    L.tok_perm = take(T * 4);
    L.tok_off = take((P + 1) * 4);
    L.s2a = take(A * 4);
    L.a2s = take(A * 4);
    L.row_tok = take(A * 4);
    L.shuffle_need = off;
    L.h = take(A * c.I * es);
    L.h_sh = take(T * Ish * es);
    L.gemm_ctr = take(16 * 4);
    L.ffn_need = off;
    L.x_sorted = c.fuse_gather ? off : take(A * c.H * es);
    L.y_sorted = take(A * c.H * es);
    L.y_sh = take(c.n_shared > 0 ? T * c.H * es : 0);
    L.total = off;
    // The tiled gate GEMM's partial logits live at the start of the expert
    // FFN buffers: the route is done before the FFN writes them.
    L.glog = L.h;
    L.route_need = MOE_DEBUG_CHECKS ? L.err + 256 : 0;
    if (gate_tiled(c) && c.T > 0) {
        L.route_need = L.glog + (((size_t)gate_split(c) * T * E * 4 + 255) & ~(size_t)255);
        L.total = std::max(L.total, L.route_need);
    }
    return L;
}

}  // namespace moe

using namespace moe;

#define MOE_API extern "C" __attribute__((visibility("default")))

#define REQUIRE(ptr)                                                     \
    do {                                                                 \
        if ((ptr) == nullptr) return fail(MOE_EINVAL, "%s is NULL", #ptr); \
    } while (0)

#define REQUIRE16(ptr)                                                          \
    do {                                                                        \
        if (!aligned16(ptr)) return fail(MOE_EINVAL, "%s not 16-byte aligned", #ptr); \
    } while (0)

// The data-error word of a workspace (debug builds), else nullptr.
static uint32_t* err_word(void* ws, const WsLayout& L)
{
    if (!MOE_DEBUG_CHECKS || ws == nullptr) return nullptr;
    return (uint32_t*)((char*)ws + L.err);
}

static int32_t check_ws(const void* ws, size_t ws_bytes, size_t need)
{
    if (need == 0) return MOE_OK;
    if (ws == nullptr) return fail(MOE_EWORKSPACE, "workspace is NULL (need %zu bytes)", need);
    if (((uintptr_t)ws & 255u) != 0) return fail(MOE_EWORKSPACE, "workspace not 256-byte aligned");
    if (ws_bytes < need) return fail(MOE_EWORKSPACE, "workspace %zu bytes < %zu needed", ws_bytes, need);
    return MOE_OK;
}

template <typename T>
static T* at(void* ws, size_t off) { return (T*)((char*)ws + off); }

MOE_API int32_t moe_validate(const moe_cfg* cfg)
{
    return check_cfg(cfg);
}

MOE_API size_t moe_workspace_bytes(const moe_cfg* cfg)
{
    if (check_cfg(cfg) != MOE_OK) return 0;
    return ws_layout(*cfg).total;
}

MOE_API const char* moe_last_error(void) { return g_err; }

MOE_API int32_t moe_debug_checks(void) { return MOE_DEBUG_CHECKS ? 1 : 0; }

MOE_API int32_t moe_debug_errors(const void* ws, uint32_t* flags, int32_t clear, void* stream)
{
    REQUIRE(flags);
    *flags = 0;
    if (!MOE_DEBUG_CHECKS) return fail(MOE_EINVAL, "release build: no device data checks recorded");
    void* word = const_cast<void*>(ws);
    hipError_t e = hipSuccess;
    if (word == nullptr) {
        e = noalloc_scratch(&word);   // the error word starts the static scratch
        if (e != hipSuccess) return hip_fail(e, "moe_debug_errors");
    }
    hipStream_t s = (hipStream_t)stream;
    e = hipMemcpyAsync(flags, word, sizeof(uint32_t), hipMemcpyDeviceToHost, s);
    if (e == hipSuccess && clear) e = hipMemsetAsync(word, 0, sizeof(uint32_t), s);
    if (e == hipSuccess) e = hipStreamSynchronize(s);
    return e == hipSuccess ? MOE_OK : hip_fail(e, "moe_debug_errors");
}

MOE_API size_t moe_route_workspace_bytes(const moe_cfg* cfg)
{
    if (check_cfg(cfg) != MOE_OK) return 0;
    return ws_layout(*cfg).route_need;
}

MOE_API int32_t moe_route(const moe_cfg* cfg, const void* x, const void* Wg, const float* ebias,
                          const int32_t* slot_to_orig, const int32_t* tok, const int32_t* pref,
                          const int32_t* k_tok, int32_t* row_ptr, int32_t* topk_slot,
                          float* topk_w, float* logits, void* ws, size_t ws_bytes, void* stream)
{
    int32_t rc = check_cfg(cfg);
    if (rc != MOE_OK) return rc;
    const moe_cfg& c = *cfg;
    const WsLayout L = ws_layout(c);
    float* glog = nullptr;
    if (L.route_need > 0) {
        rc = check_ws(ws, ws_bytes, L.route_need);
        if (rc != MOE_OK) return rc;
        if (gate_tiled(c) && c.T > 0) glog = at<float>(ws, L.glog);
    }
    uint32_t* err = L.route_need > 0 ? err_word(ws, L) : nullptr;
    REQUIRE(row_ptr);
    if (c.T > 0) {
        REQUIRE(x);
        REQUIRE(Wg);
        REQUIRE(slot_to_orig);
        REQUIRE(tok);
        REQUIRE(topk_slot);
        REQUIRE(topk_w);
        REQUIRE16(x);
        REQUIRE16(Wg);
        if (c.ragged) REQUIRE(k_tok);
    }
    hipStream_t s = (hipStream_t)stream;
    hipError_t e = launch_row_ptr(c, k_tok, row_ptr, err, s);
    if (e == hipSuccess)
        e = launch_route(c, x, Wg, ebias, slot_to_orig, tok, pref, k_tok, row_ptr, topk_slot, topk_w,
                         logits, glog, err, s);
    return e == hipSuccess ? MOE_OK : hip_fail(e, "moe_route");
}

// Argument checks shared by moe_shuffle and moe_shuffle_noalloc.
static int32_t check_shuffle_args(const moe_cfg& c, const int32_t* row_ptr, const int32_t* topk_slot,
                                  const int32_t* tok, const int32_t* lut, const void* x,
                                  int32_t* expert_count, int32_t* expert_off, int32_t* group_count,
                                  int32_t* group_off, int32_t* pair_count, int32_t* tok_perm,
                                  int32_t* tok_off, int32_t* sorted_to_assign, int32_t* assign_to_sorted,
                                  void* x_sorted)
{
    REQUIRE(row_ptr);
    REQUIRE(expert_count);
    REQUIRE(expert_off);
    REQUIRE(group_count);
    REQUIRE(group_off);
    REQUIRE(pair_count);
    REQUIRE(tok_off);
    if (c.T > 0) {
        REQUIRE(topk_slot);
        REQUIRE(tok);
        REQUIRE(lut);
        REQUIRE(tok_perm);
        REQUIRE(sorted_to_assign);
        REQUIRE(assign_to_sorted);
    }
    if (x_sorted != nullptr) {
        REQUIRE(x);
        REQUIRE16(x);
        REQUIRE16(x_sorted);
    }
    return MOE_OK;
}

static ShuffleOut shuffle_outputs(int32_t* expert_count, int32_t* expert_off, int32_t* group_count,
                                  int32_t* group_off, int32_t* pair_count, int32_t* tok_perm,
                                  int32_t* tok_off, int32_t* sorted_to_assign, int32_t* assign_to_sorted)
{
    ShuffleOut o;
    memset(&o, 0, sizeof(o));
    o.expert_count = expert_count;
    o.expert_off = expert_off;
    o.group_count = group_count;
    o.group_off = group_off;
    o.pair_count = pair_count;
    o.tok_perm = tok_perm;
    o.tok_off = tok_off;
    o.s2a = sorted_to_assign;
    o.a2s = assign_to_sorted;
    o.row_tok = nullptr;
    o.gemm_ctr = nullptr;
    return o;
}

MOE_API int32_t moe_shuffle(const moe_cfg* cfg, const int32_t* row_ptr, const int32_t* topk_slot,
                            const int32_t* tok, const int32_t* lut, const void* x,
                            int32_t* expert_count, int32_t* expert_off, int32_t* group_count,
                            int32_t* group_off, int32_t* pair_count, int32_t* tok_perm,
                            int32_t* tok_off, int32_t* sorted_to_assign, int32_t* assign_to_sorted,
                            void* x_sorted, void* ws, size_t ws_bytes, void* stream)
{
    int32_t rc = check_cfg(cfg);
    if (rc != MOE_OK) return rc;
    const moe_cfg& c = *cfg;
    rc = check_shuffle_args(c, row_ptr, topk_slot, tok, lut, x, expert_count, expert_off, group_count,
                            group_off, pair_count, tok_perm, tok_off, sorted_to_assign, assign_to_sorted,
                            x_sorted);
    if (rc != MOE_OK) return rc;
    const WsLayout L = ws_layout(c);
    rc = check_ws(ws, ws_bytes, L.shuffle_need);
    if (rc != MOE_OK) return rc;
    ShuffleOut o = shuffle_outputs(expert_count, expert_off, group_count, group_off, pair_count, tok_perm,
                                   tok_off, sorted_to_assign, assign_to_sorted);
    o.g_pred = at<int32_t>(ws, L.g_pred);
    o.hist = at<int32_t>(ws, L.hist);
    o.thist = at<int32_t>(ws, L.thist);
    o.rowtot = at<int32_t>(ws, L.rowtot);
    o.bstart = at<int32_t>(ws, L.bstart);
    o.tstart = at<int32_t>(ws, L.tstart);
    o.err = err_word(ws, L);
    hipStream_t s = (hipStream_t)stream;
    hipError_t e = launch_shuffle(c, L.nb, L.tpb, row_ptr, topk_slot, tok, lut, o, s);
    if (e == hipSuccess && x_sorted != nullptr) e = launch_gather(c, x, row_ptr, assign_to_sorted, x_sorted, s);
    return e == hipSuccess ? MOE_OK : hip_fail(e, "moe_shuffle");
}

// Scratch of the shuffle alone, packed from offset 0: the data-error word,
// g_pred [T], the per-block histograms hist [nb][E*P] and thist [nb][P], row
// totals, bucket and group starts (256-byte aligned sections) at `base` (0:
// sizes only).  Returns the bytes needed.
static size_t shuffle_scratch(const moe_cfg& c, ShuffleOut& o, uintptr_t base, int* nb, int* tpb)
{
    *tpb = shuffle_tpb(c.T, c.E, c.P);
    *nb = std::max(1, ceil_div(c.T, *tpb));
    const size_t E = c.E, P = c.P, NB = (size_t)*nb;
    size_t off = 0;
    auto take = [&](size_t bytes) {
        int32_t* p = (int32_t*)(base + off);
        off += (bytes + 255) & ~(size_t)255;
        return p;
    };
    uint32_t* err = (uint32_t*)take(4);
    o.err = MOE_DEBUG_CHECKS && base != 0 ? err : nullptr;
    o.g_pred = take((size_t)c.T * 4);
    o.hist = take(E * P * NB * 4);
    o.thist = take(P * NB * 4);
    o.rowtot = take((E * P + P) * 4);
    o.bstart = take((E * P + 1) * 4);
    o.tstart = take((P + 1) * 4);
    return off;
}

MOE_API int32_t moe_shuffle_noalloc(const moe_cfg* cfg, const int32_t* row_ptr, const int32_t* topk_slot,
                                    const int32_t* tok, const int32_t* lut, const void* x,
                                    int32_t* expert_count, int32_t* expert_off, int32_t* group_count,
                                    int32_t* group_off, int32_t* pair_count, int32_t* tok_perm,
                                    int32_t* tok_off, int32_t* sorted_to_assign, int32_t* assign_to_sorted,
                                    void* x_sorted, void* stream)
{
    int32_t rc = check_cfg(cfg);
    if (rc != MOE_OK) return rc;
    const moe_cfg& c = *cfg;
    rc = check_shuffle_args(c, row_ptr, topk_slot, tok, lut, x, expert_count, expert_off, group_count,
                            group_off, pair_count, tok_perm, tok_off, sorted_to_assign, assign_to_sorted,
                            x_sorted);
    if (rc != MOE_OK) return rc;
    ShuffleOut o = shuffle_outputs(expert_count, expert_off, group_count, group_off, pair_count, tok_perm,
                                   tok_off, sorted_to_assign, assign_to_sorted);
    int nb = 0, tpb = 0;
    const size_t need = shuffle_scratch(c, o, 0, &nb, &tpb);
    if (need > (size_t)MOE_NOALLOC_SCRATCH_BYTES)
        return fail(MOE_EWORKSPACE, "moe_shuffle_noalloc: layer needs %zu bytes of scratch, the static "
                    "array holds %zu", need, (size_t)MOE_NOALLOC_SCRATCH_BYTES);
    void* base = nullptr;
    hipError_t e = noalloc_scratch(&base);
    if (e != hipSuccess) return hip_fail(e, "moe_shuffle_noalloc (scratch address)");
    shuffle_scratch(c, o, (uintptr_t)base, &nb, &tpb);
    hipStream_t s = (hipStream_t)stream;
    e = launch_shuffle(c, nb, tpb, row_ptr, topk_slot, tok, lut, o, s);
    if (e == hipSuccess && x_sorted != nullptr) e = launch_gather(c, x, row_ptr, assign_to_sorted, x_sorted, s);
    return e == hipSuccess ? MOE_OK : hip_fail(e, "moe_shuffle_noalloc");
}

MOE_API int32_t moe_expert_ffn(const moe_cfg* cfg, int32_t which, const void* x_sorted,
                               const void* x, const int32_t* row_ptr,
                               const int32_t* sorted_to_assign, const int32_t* expert_off,
                               const void* W13, const void* W2, int32_t e_begin, int32_t e_end,
                               void* y, void* ws, size_t ws_bytes, void* stream)
{
    int32_t rc = check_cfg(cfg);
    if (rc != MOE_OK) return rc;
    const moe_cfg& c = *cfg;
    if (which != MOE_FFN_ROUTED && which != MOE_FFN_SHARED) return fail(MOE_EINVAL, "bad `which`");
    REQUIRE(W13);
    REQUIRE(W2);
    REQUIRE(y);
    REQUIRE16(W13);
    REQUIRE16(W2);
    REQUIRE16(y);
    const WsLayout L = ws_layout(c);
    rc = check_ws(ws, ws_bytes, L.ffn_need);
    if (rc != MOE_OK) return rc;
    hipStream_t s = (hipStream_t)stream;
    FfnArgs a;
    memset(&a, 0, sizeof(a));
    a.A_max = c.T * c.k_max;
    a.ctr = at<int32_t>(ws, L.gemm_ctr);
    if (which == MOE_FFN_SHARED) {
        if (c.n_shared == 0) return fail(MOE_ESHAPE, "no shared experts in cfg");
        if (c.T == 0) return MOE_OK;  // nothing to read or write
        REQUIRE(x);
        REQUIRE16(x);
        a.n_routed = 0;
        a.sh_x = x;
        a.sh_W13 = W13;
        a.sh_W2 = W2;
        a.sh_h = at<void>(ws, L.h_sh);
        a.sh_y = y;
        a.Ish = c.n_shared * c.I_shared;
    } else {
        if (e_begin < 0 || e_end > c.E || e_begin > e_end) return fail(MOE_EINVAL, "bad expert range");
        if (c.T == 0 || e_begin == e_end) return MOE_OK;  // nothing to read or write
        REQUIRE(expert_off);
        if (x_sorted == nullptr) {
            REQUIRE(x);
            REQUIRE(row_ptr);
            REQUIRE(sorted_to_assign);
            REQUIRE16(x);
        } else {
            REQUIRE16(x_sorted);
        }
        a.n_routed = e_end - e_begin;
        a.e_begin = e_begin;
        a.expert_off = expert_off;
        a.xs = x_sorted;
        a.x = x;
        a.W13 = W13;
        a.W2 = W2;
        a.h = at<void>(ws, L.h);
        a.y = y;
        if (x_sorted == nullptr) {
            a.row_tok = at<int32_t>(ws, L.row_tok);
            hipError_t e = launch_row_tok(c, row_ptr, sorted_to_assign, at<int32_t>(ws, L.row_tok), s);
            if (e != hipSuccess) return hip_fail(e, "moe_expert_ffn");
        }
    }
    hipError_t e = launch_ffn_up(c, a, s);
    if (e == hipSuccess) e = launch_ffn_down(c, a, s);
    return e == hipSuccess ? MOE_OK : hip_fail(e, "moe_expert_ffn");
}

MOE_API int32_t moe_combine(const moe_cfg* cfg, const void* y_sorted,
                            const int32_t* assign_to_sorted, const int32_t* row_ptr,
                            const float* topk_w, const void* y_sh, void* out, void* stream)
{
    int32_t rc = check_cfg(cfg);
    if (rc != MOE_OK) return rc;
    const moe_cfg& c = *cfg;
    if (c.T == 0) return MOE_OK;
    REQUIRE(y_sorted);
    REQUIRE(assign_to_sorted);
    REQUIRE(row_ptr);
    REQUIRE(topk_w);
    REQUIRE(out);
    REQUIRE16(y_sorted);
    REQUIRE16(out);
    if (y_sh != nullptr) REQUIRE16(y_sh);
    hipError_t e = launch_combine(c, y_sorted, assign_to_sorted, row_ptr, topk_w, y_sh, out,
                                  (hipStream_t)stream);
    return e == hipSuccess ? MOE_OK : hip_fail(e, "moe_combine");
}

MOE_API int32_t moe_srs(const moe_cfg* cfg, int32_t n_part, const void* x_part,
                        const int32_t* tok_perm, void* y, void* stream)
{
    int32_t rc = check_cfg(cfg);
    if (rc != MOE_OK) return rc;
    const moe_cfg& c = *cfg;
    if (n_part < 1 || n_part > 64) return fail(MOE_EINVAL, "n_part must be in [1, 64]");
    if (c.T == 0) return MOE_OK;
    REQUIRE(x_part);
    REQUIRE(tok_perm);
    REQUIRE(y);
    REQUIRE16(x_part);
    REQUIRE16(y);
    hipError_t e = launch_srs(c, n_part, x_part, tok_perm, y, (hipStream_t)stream);
    return e == hipSuccess ? MOE_OK : hip_fail(e, "moe_srs");
}

MOE_API int32_t moe_sag(const moe_cfg* cfg, const void* y, const int32_t* tok_perm, void* out,
                        void* stream)
{
    int32_t rc = check_cfg(cfg);
    if (rc != MOE_OK) return rc;
    const moe_cfg& c = *cfg;
    if (c.T == 0) return MOE_OK;
    REQUIRE(y);
    REQUIRE(tok_perm);
    REQUIRE(out);
    REQUIRE16(y);
    REQUIRE16(out);
    if (y == out) return fail(MOE_EINVAL, "y and out must not overlap");
    hipError_t e = launch_sag(c, y, tok_perm, out, (hipStream_t)stream);
    return e == hipSuccess ? MOE_OK : hip_fail(e, "moe_sag");
}

// ---------------------------------------------------------------- co-scheduling

MOE_API int32_t moe_token_group_counts(const moe_cfg* cfg, int32_t n_tok, const int32_t* row_ptr,
                                       const int32_t* expert, const int32_t* tok,
                                       const int32_t* group, int32_t* counts, void* stream)
{
    int32_t rc = check_cfg(cfg);
    if (rc != MOE_OK) return rc;
    const moe_cfg& c = *cfg;
    if (n_tok < 0) return fail(MOE_EINVAL, "n_tok < 0");
    if ((long long)c.V * c.P >= (1LL << 31)) return fail(MOE_ESHAPE, "V*P must stay below 2^31 (token table)");
    REQUIRE(counts);
    if (n_tok > 0) {
        REQUIRE(row_ptr);
        REQUIRE(expert);
        REQUIRE(tok);
        REQUIRE(group);
    }
    hipError_t e = launch_token_group_counts(n_tok, c.V, c.E, c.P, row_ptr, expert, tok, group, counts,
                                             (hipStream_t)stream);
    return e == hipSuccess ? MOE_OK : hip_fail(e, "moe_token_group_counts");
}

MOE_API int32_t moe_lut_from_counts(const moe_cfg* cfg, const int32_t* counts, int32_t* lut,
                                    void* stream)
{
    int32_t rc = check_cfg(cfg);
    if (rc != MOE_OK) return rc;
    REQUIRE(counts);
    REQUIRE(lut);
    hipError_t e = launch_lut_from_counts(cfg->V, cfg->P, counts, lut, (hipStream_t)stream);
    return e == hipSuccess ? MOE_OK : hip_fail(e, "moe_lut_from_counts");
}

MOE_API int32_t moe_expert_group_counts(const moe_cfg* cfg, int32_t n_tok, const int32_t* row_ptr,
                                        const int32_t* expert, const int32_t* tok,
                                        const int32_t* lut, int32_t* counts, void* stream)
{
    int32_t rc = check_cfg(cfg);
    if (rc != MOE_OK) return rc;
    const moe_cfg& c = *cfg;
    if (n_tok < 0) return fail(MOE_EINVAL, "n_tok < 0");
    REQUIRE(counts);
    if (n_tok > 0) {
        REQUIRE(row_ptr);
        REQUIRE(expert);
        REQUIRE(tok);
        REQUIRE(lut);
    }
    hipError_t e = launch_expert_group_counts(n_tok, c.V, c.E, c.P, row_ptr, expert, tok, lut, counts,
                                              (hipStream_t)stream);
    return e == hipSuccess ? MOE_OK : hip_fail(e, "moe_expert_group_counts");
}

MOE_API int64_t moe_balanced_assign(int32_t n, int32_t P, const int64_t* score, int32_t* group)
{
    if (n < 0 || P < 1 || n % P != 0) return fail(MOE_ESHAPE, "need n >= 0, P >= 1, P | n");
    if (n > 4096) return fail(MOE_ESHAPE, "n > 4096");
    if (n > 0) {
        REQUIRE(score);
        REQUIRE(group);
    }
    return balanced_assign_host(n, P, (const long long*)score, group);
}

MOE_API int32_t moe_optimize_placement(const moe_cfg* cfg, int32_t n_tok, const int32_t* row_ptr,
                                       const int32_t* expert, const int32_t* tok, int32_t max_iters,
                                       int32_t* group, int32_t* perm, int32_t* lut,
                                       int32_t* counts_vp, int32_t* counts_pe, int64_t* objective,
                                       int32_t* n_steps, void* stream)
{
    int32_t rc = check_cfg(cfg);
    if (rc != MOE_OK) return rc;
    const moe_cfg& c = *cfg;
    const int E = c.E, P = c.P, epg = c.E / c.P;
    if (n_tok < 0 || max_iters < 1) return fail(MOE_EINVAL, "n_tok < 0 or max_iters < 1");
    if ((long long)c.V * c.P >= (1LL << 31)) return fail(MOE_ESHAPE, "V*P must stay below 2^31 (token table)");
    REQUIRE(group);
    REQUIRE(lut);
    REQUIRE(counts_vp);
    REQUIRE(counts_pe);
    if (n_tok > 0) {
        REQUIRE(row_ptr);
        REQUIRE(expert);
        REQUIRE(tok);
    }
    std::vector<int> cnt(P, 0);
    for (int e = 0; e < E; ++e) {
        if (group[e] < 0 || group[e] >= P) return fail(MOE_EINVAL, "group[%d] out of range", e);
        ++cnt[group[e]];
    }
    for (int g = 0; g < P; ++g)
        if (cnt[g] != epg) return fail(MOE_EINVAL, "initial grouping is not balanced");
    hipStream_t s = (hipStream_t)stream;
    int32_t* dgroup = counts_pe;   // the expert grouping rides in the first E ints of counts_pe
    std::vector<int32_t> hC((size_t)P * E), cur(group, group + E), nxt(E);
    std::vector<long long> score((size_t)E * P);
    int steps = 0;
    hipError_t e = hipSuccess;
#define HIPCHK(x)                                           \
    do {                                                    \
        e = (x);                                            \
        if (e != hipSuccess) return hip_fail(e, "moe_optimize_placement"); \
    } while (0)
    // token step for the grouping `cur`: lut on the device
    auto token_step = [&]() -> hipError_t {
        hipError_t r = hipMemcpyAsync(dgroup, cur.data(), E * sizeof(int32_t), hipMemcpyHostToDevice, s);
        if (r != hipSuccess) return r;
        r = launch_token_group_counts(n_tok, c.V, E, P, row_ptr, expert, tok, dgroup, counts_vp, s);
        if (r != hipSuccess) return r;
        return launch_lut_from_counts(c.V, P, counts_vp, lut, s);
    };
    for (int it = 0; it < max_iters; ++it) {
        HIPCHK(token_step());
        HIPCHK(launch_expert_group_counts(n_tok, c.V, E, P, row_ptr, expert, tok, lut, counts_pe, s));
        HIPCHK(hipMemcpyAsync(hC.data(), counts_pe, hC.size() * sizeof(int32_t), hipMemcpyDeviceToHost, s));
        HIPCHK(hipStreamSynchronize(s));
        long long before = 0;
        for (int x = 0; x < E; ++x) {
            before += hC[(size_t)cur[x] * E + x];
            for (int g = 0; g < P; ++g) score[(size_t)x * P + g] = hC[(size_t)g * E + x];
        }
        const long long after = balanced_assign_host(E, P, score.data(), nxt.data());
        if (objective) {
            objective[2 * it] = before;
            objective[2 * it + 1] = after;
        }
        steps = 2 * it + 2;
        if (after <= before) break;   // no strict gain: keep the current grouping
        cur = nxt;
    }
    HIPCHK(token_step());             // final table for the kept grouping
    HIPCHK(hipStreamSynchronize(s));
#undef HIPCHK
    std::copy(cur.begin(), cur.end(), group);
    if (perm) {
        // group g's experts take slots [g*E/P, (g+1)*E/P) in ascending id
        std::vector<int> next_slot(P);
        for (int g = 0; g < P; ++g) next_slot[g] = g * epg;
        for (int x = 0; x < E; ++x) perm[x] = next_slot[cur[x]]++;
    }
    if (n_steps) *n_steps = steps;
    return MOE_OK;
}

MOE_API int32_t moe_request_group_hist(const moe_cfg* cfg, int32_t n_req, const int32_t* req_ptr,
                                       const int32_t* tok, const int32_t* lut, int32_t* hist,
                                       void* stream)
{
    int32_t rc = check_cfg(cfg);
    if (rc != MOE_OK) return rc;
    if (n_req < 0) return fail(MOE_EINVAL, "n_req < 0");
    if (n_req == 0) return MOE_OK;
    REQUIRE(req_ptr);
    REQUIRE(tok);
    REQUIRE(lut);
    REQUIRE(hist);
    hipError_t e = launch_request_group_hist(n_req, cfg->V, cfg->P, req_ptr, tok, lut, hist,
                                             (hipStream_t)stream);
    return e == hipSuccess ? MOE_OK : hip_fail(e, "moe_request_group_hist");
}

MOE_API int32_t moe_pack_weights(const moe_cfg* cfg, int32_t which, const void* W13, const void* W2,
                                 void* W13_blk, void* W2_blk, void* stream)
{
    int32_t rc = check_cfg(cfg);
    if (rc != MOE_OK) return rc;
    const moe_cfg& c = *cfg;
    if (c.dtype != MOE_BF16) return fail(MOE_EDTYPE, "blocked weights need bf16");
    if (which != MOE_FFN_ROUTED && which != MOE_FFN_SHARED) return fail(MOE_EINVAL, "which must be ROUTED or SHARED");
    const bool shared = which == MOE_FFN_SHARED;
    if (shared && c.n_shared == 0) return fail(MOE_EINVAL, "no shared experts");
    REQUIRE(W13);
    REQUIRE(W2);
    REQUIRE(W13_blk);
    REQUIRE(W2_blk);
    REQUIRE16(W13);
    REQUIRE16(W2);
    REQUIRE16(W13_blk);
    REQUIRE16(W2_blk);
    if (W13 == W13_blk || W2 == W2_blk) return fail(MOE_EINVAL, "blocked weights must not alias their source");
    hipError_t e = launch_pack_weights(c, shared, W13, W2, W13_blk, W2_blk, (hipStream_t)stream);
    return e == hipSuccess ? MOE_OK : hip_fail(e, "moe_pack_weights");
}

MOE_API int32_t moe_sigmoid(const float* x, float* y, int64_t n, void* stream)
{
    if (n < 0) return fail(MOE_EINVAL, "n < 0");
    if (n == 0) return MOE_OK;
    REQUIRE(x);
    REQUIRE(y);
    hipError_t e = launch_sigmoid(x, y, n, (hipStream_t)stream);
    return e == hipSuccess ? MOE_OK : hip_fail(e, "moe_sigmoid");
}

MOE_API int32_t moe_forward(const moe_cfg* cfg, const moe_weights* w, const moe_inputs* in,
                            void* out, const moe_exports* ex, void* ws, size_t ws_bytes,
                            void* stream)
{
    int32_t rc = check_cfg(cfg);
    if (rc != MOE_OK) return rc;
    const moe_cfg& c = *cfg;
    REQUIRE(w);
    REQUIRE(in);
    REQUIRE(out);
    REQUIRE16(out);
    if (c.T > 0) {
        REQUIRE(in->x);
        REQUIRE(in->tok);
        REQUIRE(w->Wg);
        REQUIRE(w->slot_to_orig);
        REQUIRE(w->W13);
        REQUIRE(w->W2);
        REQUIRE(w->lut);
        REQUIRE16(in->x);
        REQUIRE16(w->Wg);
        REQUIRE16(w->W13);
        REQUIRE16(w->W2);
        if (c.ragged) REQUIRE(in->k_tok);
        if (c.n_shared > 0) {
            REQUIRE(w->Wsh13);
            REQUIRE(w->Wsh2);
            REQUIRE16(w->Wsh13);
            REQUIRE16(w->Wsh2);
        }
    }
    const WsLayout L = ws_layout(c);
    rc = check_ws(ws, ws_bytes, L.total);
    if (rc != MOE_OK) return rc;
    static const moe_exports kNone = {};
    const moe_exports* X = ex ? ex : &kNone;
    auto pick = [&](auto* p, size_t off) { return p ? p : at<std::remove_pointer_t<decltype(p)>>(ws, off); };
    int32_t* row_ptr = pick(X->row_ptr, L.row_ptr);
    int32_t* topk_slot = pick(X->topk_slot, L.topk_slot);
    float* topk_w = pick(X->topk_w, L.topk_w);
    ShuffleOut o;
    o.expert_count = pick(X->expert_count, L.expert_count);
    o.expert_off = pick(X->expert_off, L.expert_off);
    o.group_count = pick(X->group_count, L.group_count);
    o.group_off = pick(X->group_off, L.group_off);
    o.pair_count = pick(X->pair_count, L.pair_count);
    o.tok_perm = pick(X->tok_perm, L.tok_perm);
    o.tok_off = pick(X->tok_off, L.tok_off);
    o.s2a = pick(X->sorted_to_assign, L.s2a);
    o.a2s = pick(X->assign_to_sorted, L.a2s);
    o.row_tok = at<int32_t>(ws, L.row_tok);
    o.g_pred = at<int32_t>(ws, L.g_pred);
    o.hist = at<int32_t>(ws, L.hist);
    o.thist = at<int32_t>(ws, L.thist);
    o.rowtot = at<int32_t>(ws, L.rowtot);
    o.bstart = at<int32_t>(ws, L.bstart);
    o.tstart = at<int32_t>(ws, L.tstart);
    o.gemm_ctr = at<int32_t>(ws, L.gemm_ctr);   // zeroed by the shuffle for the FFN below
    o.err = err_word(ws, L);
    void* x_sorted = c.fuse_gather ? nullptr : (X->x_sorted ? X->x_sorted : at<void>(ws, L.x_sorted));
    void* y_sorted = X->y_sorted ? X->y_sorted : at<void>(ws, L.y_sorted);
    void* y_sh = c.n_shared > 0 ? (X->y_shared ? X->y_shared : at<void>(ws, L.y_sh)) : nullptr;
    if (x_sorted) REQUIRE16(x_sorted);
    REQUIRE16(y_sorted);
    if (y_sh) REQUIRE16(y_sh);

    hipStream_t s = (hipStream_t)stream;
    hipError_t e = hipSuccess;
#define STEP(expr)                          \
    do {                                    \
        if (e == hipSuccess) e = (expr);    \
    } while (0)
    STEP(record(X, MOE_STAGE_ROUTE, 0, s));
    STEP(launch_row_ptr(c, in->k_tok, row_ptr, o.err, s));
    STEP(launch_route(c, in->x, w->Wg, w->ebias, w->slot_to_orig, in->tok, w->pref, in->k_tok,
                      row_ptr, topk_slot, topk_w, X->logits,
                      gate_tiled(c) && c.T > 0 ? at<float>(ws, L.glog) : nullptr, o.err, s));
    STEP(record(X, MOE_STAGE_ROUTE, 1, s));
    STEP(record(X, MOE_STAGE_SHUFFLE, 0, s));
    STEP(launch_shuffle(c, L.nb, L.tpb, row_ptr, topk_slot, in->tok, w->lut, o, s));
    STEP(record(X, MOE_STAGE_SHUFFLE, 1, s));
    STEP(record(X, MOE_STAGE_GATHER, 0, s));
    if (x_sorted) STEP(launch_gather(c, in->x, row_ptr, o.a2s, x_sorted, s));
    STEP(record(X, MOE_STAGE_GATHER, 1, s));

    FfnArgs a;
    memset(&a, 0, sizeof(a));
    a.A_max = c.T * c.k_max;
    a.ctr = at<int32_t>(ws, L.gemm_ctr);
    a.ctr_zeroed = true;
    a.n_routed = c.T > 0 ? c.E : 0;
    a.e_begin = 0;
    a.expert_off = o.expert_off;
    a.xs = x_sorted;
    a.x = in->x;
    a.row_tok = o.row_tok;
    a.W13 = w->W13;
    a.W2 = w->W2;
    a.h = at<void>(ws, L.h);
    a.y = y_sorted;
    if (c.n_shared > 0 && c.T > 0) {
        a.sh_x = in->x;
        a.sh_W13 = w->Wsh13;
        a.sh_W2 = w->Wsh2;
        a.sh_h = at<void>(ws, L.h_sh);
        a.sh_y = y_sh;
        a.Ish = c.n_shared * c.I_shared;
    }
    STEP(record(X, MOE_STAGE_FFN_UP, 0, s));
    STEP(launch_ffn_up(c, a, s));
    STEP(record(X, MOE_STAGE_FFN_UP, 1, s));
    STEP(record(X, MOE_STAGE_FFN_DOWN, 0, s));
    STEP(launch_ffn_down(c, a, s));
    STEP(record(X, MOE_STAGE_FFN_DOWN, 1, s));
    STEP(record(X, MOE_STAGE_COMBINE, 0, s));
    STEP(launch_combine(c, y_sorted, o.a2s, row_ptr, topk_w, y_sh, out, s));
    STEP(record(X, MOE_STAGE_COMBINE, 1, s));
#undef STEP
    return e == hipSuccess ? MOE_OK : hip_fail(e, "moe_forward");
}
