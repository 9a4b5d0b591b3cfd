// Internal declarations shared by the libmoe translation units (host side).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/moe.h"

#ifndef MOE_DEBUG_CHECKS
#define MOE_DEBUG_CHECKS 0   // 1: kernels record clamped input data (libmoe_debug.so)
#endif

namespace moe {

// Tokens per block of the histogram / scatter kernels of the shuffle: 256,
// halved (down to 64) while the layer would get fewer than 128 blocks, so
// that mid-sized layers still spread the histogram and scatter over many CUs.
// (While the per-block counts were scanned by a single block, 64-token blocks
// at T = 4096 were slower, the larger count table costing that scan more than
// the shorter blocks gained; with one wave per bucket row they are faster.)
constexpr int kShuffleMaxTPB = 256;
inline int shuffle_tpb(int T, int, int)
{
    int tpb = kShuffleMaxTPB;
    while (tpb > 64 && (T + tpb - 1) / tpb < 128) tpb /= 2;
    return tpb;
}

inline int ceil_div(int a, int b) { return (a + b - 1) / b; }
inline int ilog2(int v) { int r = 0; while ((1 << r) < v) ++r; return r; }

// Workspace layout (byte offsets, 256-byte aligned sections).
struct WsLayout {
    size_t err;                                   // data-error word (first 256 bytes)
    size_t row_ptr, topk_slot, topk_w;            // route outputs (moe_forward)
    size_t g_pred, hist, thist, rowtot, bstart, tstart;  // shuffle scratch
    size_t expert_count, expert_off, group_count, group_off, pair_count;
    size_t tok_perm, tok_off, s2a, a2s, row_tok;  // shuffle outputs / scratch
    size_t x_sorted, h, h_sh, y_sorted, y_sh;     // expert FFN buffers
    size_t gemm_ctr;                              // grouped-GEMM tile counters
    size_t glog, route_need;                      // gate partial logits (aliases h..), route's need
    size_t shuffle_need, ffn_need, total;
    int nb, tpb;                                  // shuffle blocks, tokens per block
};

WsLayout ws_layout(const moe_cfg& c);

// Route of large-E bf16 layers: the gate GEMM runs as its own tiled kernel
// into gate_split(c) slices of partial logits (fp32 [S][T][E], workspace).
bool gate_tiled(const moe_cfg& c);
int gate_split(const moe_cfg& c);

// --- launchers (no argument checks; callers validate) ---------------------
// err: the data-error word (debug builds; nullptr in the release build)
hipError_t launch_row_ptr(const moe_cfg& c, const int32_t* k_tok, int32_t* row_ptr, uint32_t* err,
                          hipStream_t s);
hipError_t launch_route(const moe_cfg& c, const void* x, const void* Wg, const float* ebias,
                        const int32_t* slot_to_orig, const int32_t* tok, const int32_t* pref,
                        const int32_t* k_tok, int32_t* row_ptr, int32_t* topk_slot,
                        float* topk_w, float* logits, float* glog, uint32_t* err, hipStream_t s);

struct ShuffleOut {
    int32_t *expert_count, *expert_off, *group_count, *group_off, *pair_count;
    int32_t *tok_perm, *tok_off, *s2a, *a2s, *row_tok;
    int32_t *g_pred, *hist, *thist;
    int32_t *rowtot, *bstart, *tstart;  // row totals, bucket and group starts (scratch)
    int32_t* gemm_ctr;  // [16] grouped-GEMM tile counters to zero, or nullptr
    uint32_t* err;      // data-error word (debug builds), or nullptr
};
hipError_t launch_sigmoid(const float* x, float* y, int64_t n, hipStream_t s);

// This device's copy of the static scratch array of moe_shuffle_noalloc
// (MOE_NOALLOC_SCRATCH_BYTES, 256-byte aligned); its address is looked up
// once per device.
hipError_t noalloc_scratch(void** out);
hipError_t launch_shuffle(const moe_cfg& c, int nb, int tpb, const int32_t* row_ptr,
                          const int32_t* topk_slot, const int32_t* tok, const int32_t* lut,
                          const ShuffleOut& o, hipStream_t s);
hipError_t launch_gather(const moe_cfg& c, const void* x, const int32_t* row_ptr,
                         const int32_t* a2s, void* x_sorted, hipStream_t s);
hipError_t launch_row_tok(const moe_cfg& c, const int32_t* row_ptr, const int32_t* s2a,
                          int32_t* row_tok, hipStream_t s);

// One grouped-FFN launch pair covers the routed slots [e_begin, e_end)
// (rows expert_off[e]..expert_off[e+1] of the sorted row space) and, when
// sh_x != nullptr, the shared experts over all T rows.
struct FfnArgs {
    // routed part
    int n_routed;                // e_end - e_begin (0: none)
    const int32_t* expert_off;   // [E+1]; segment e uses [off[e_begin+i], off[e_begin+i+1])
    int e_begin;
    const void* xs;              // rows in sorted order, or nullptr -> x via row_tok
    const void* x;               // [T,H]
    const int32_t* row_tok;      // token of each sorted row (used when xs == nullptr)
    const void* W13;             // [E,2I,H]
    const void* W2;              // [E,H,I]
    void* h;                     // [A_max, I] intermediate
    void* y;                     // [A_max, H] output rows
    int A_max;
    // shared part (all T rows of x)
    const void* sh_x;            // [T,H] or nullptr
    const void* sh_W13;          // [2*Ish, H]
    const void* sh_W2;           // [H, Ish]
    void* sh_h;                  // [T, Ish]
    void* sh_y;                  // [T, H]
    int Ish;                     // n_shared * I_shared
    int32_t* ctr;                // [16] workspace tile counters (up: 0..7, down: 8..15)
    bool ctr_zeroed;             // ctr already zero on the stream (else the up GEMM zeroes it)
};
hipError_t launch_ffn_up(const moe_cfg& c, const FfnArgs& a, hipStream_t s);
hipError_t launch_ffn_down(const moe_cfg& c, const FfnArgs& a, hipStream_t s);
hipError_t launch_pack_weights(const moe_cfg& c, bool shared, const void* W13, const void* W2, void* W13b,
                               void* W2b, hipStream_t s);

hipError_t launch_combine(const moe_cfg& c, const void* y_sorted, const int32_t* a2s,
                          const int32_t* row_ptr, const float* topk_w, const void* y_sh,
                          void* out, hipStream_t s);

hipError_t launch_srs(const moe_cfg& c, int n_part, const void* x_part, const int32_t* tok_perm,
                      void* y, hipStream_t s);
hipError_t launch_sag(const moe_cfg& c, const void* y, const int32_t* tok_perm, void* out,
                      hipStream_t s);

// offline co-scheduling (cosched.hip)
hipError_t launch_fill_i32(int32_t* p, long long n, int32_t v, hipStream_t s);
hipError_t launch_token_group_counts(int n_tok, int V, int E, int P, const int32_t* row_ptr,
                                     const int32_t* expert, const int32_t* tok, const int32_t* group,
                                     int32_t* D, hipStream_t s);
hipError_t launch_lut_from_counts(int V, int P, const int32_t* D, int32_t* lut, hipStream_t s);
hipError_t launch_expert_group_counts(int n_tok, int V, int E, int P, const int32_t* row_ptr,
                                      const int32_t* expert, const int32_t* tok, const int32_t* lut,
                                      int32_t* C, hipStream_t s);
hipError_t launch_request_group_hist(int n_req, int V, int P, const int32_t* req_ptr,
                                     const int32_t* tok, const int32_t* lut, int32_t* H,
                                     hipStream_t s);
long long balanced_assign_host(int n, int P, const long long* score, int32_t* group);

}  // namespace moe
