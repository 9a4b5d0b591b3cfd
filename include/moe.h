/*
 * moe.h — C ABI of libmoe: one Mixture-of-Experts layer forward pass with
 * affinity-aware token dispatch, on one AMD Instinct MI355X (gfx950).
 *
 * The method (Sem-MoE "semantic parallelism"; pages: "Semantic Parallelism:
 * Redefining Efficient MoE Inference via Model-Data Co-Scheduling", Korean,
 * German and Japanese summaries, and "MoE-Prism: Disentangling Monolithic
 * Experts for Elastic MoE Services via Model-System Co-Designs"):
 *   - each token activates only a few experts picked by the gate, and under
 *     expert parallelism its row has to travel to the device holding them
 *     (ko/de technical summary §1, ja technical overview §1);
 *   - experts are placed on devices by shuffling the gate matrix's columns,
 *     which moves experts physically without changing what the model computes
 *     (ja technical overview §2.2A) — here: every per-expert tensor is stored
 *     in "slot" order, slot = placement position, and the P placement groups
 *     are the E/P consecutive slots [g*E/P, (g+1)*E/P);
 *   - a lightweight table maps a token ID to the expert group it is predicted
 *     to need (ja technical overview §2.3);
 *   - before the MoE layer tokens are shuffled to the device of their predicted
 *     experts, and after the experts the results are gathered back into the
 *     original token order (de technical summary §2B, ja technical overview
 *     §2.2B);
 *   - MoE-Prism's sub-experts are neuron slices of a monolithic expert and the
 *     routing budget k is a per-request knob (MoE-Prism technical summary §2A,
 *     §1, §5) — here: ragged per-token k in CSR form.
 * On one GPU there is no communication: the shuffle is a stable counting sort
 * by (slot, predicted group, token) and the would-be all-to-all traffic is the
 * P x P matrix pair_count.
 *
 * Conventions for every call
 *   - All pointers are DEVICE pointers unless marked "host".  Row-major
 *     layouts; per-expert tensors in slot order.  dtype MOE_BF16: activations
 *     and weights are bf16 (uint16 bit patterns), accumulation fp32;
 *     dtype MOE_F32: everything fp32.
 *   - The caller owns every buffer.  The library allocates no device memory
 *     and is re-entrant when concurrent calls use distinct workspaces.  Its
 *     only mutable global state: a per-device cache of the compute-unit
 *     count and of the address of moe_shuffle_noalloc's static scratch (both
 *     set once, thread-safe), and that scratch itself.
 *     moe_workspace_bytes(cfg) bytes of workspace (256-byte aligned) are
 *     enough for every call.
 *   - Calls enqueue kernels on `stream` (a hipStream_t; NULL = the null
 *     stream) and return without synchronising.  Device-side sizes that the
 *     host cannot know (the number of assignments A = row_ptr[T] when k is
 *     ragged) stay on the device; buffers sized by A are allocated for
 *     A_max = T * k_max.
 *   - Return value: MOE_OK (0) or a negative moe_status.  Argument checks
 *     happen before anything is enqueued; MOE_EHIP reports a launch error
 *     (hipGetLastError) and moe_last_error() gives its text.
 */
#ifndef MOE_H
#define MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum moe_status {
    MOE_OK = 0,
    MOE_EINVAL = -1,     /* null pointer or invalid argument value */
    MOE_ESHAPE = -2,     /* unsupported or inconsistent sizes */
    MOE_EDTYPE = -3,     /* unsupported dtype / gate combination */
    MOE_EWORKSPACE = -4, /* workspace missing, too small or misaligned */
    MOE_EHIP = -5        /* HIP runtime / launch error, see moe_last_error() */
};

enum moe_dtype { MOE_F32 = 0, MOE_BF16 = 1 };

enum moe_gate {
    MOE_GATE_SOFTMAX = 0,         /* softmax over all E logits */
    MOE_GATE_SIGMOID_GROUPED = 1  /* sigmoid + per-expert bias, group-limited */
};

enum moe_ffn_which { MOE_FFN_ROUTED = 0, MOE_FFN_SHARED = 1 };

/* Stages timed by moe_forward when moe_exports.events is set. */
enum moe_stage {
    MOE_STAGE_ROUTE = 0,    /* gate GEMM + top-k + weights */
    MOE_STAGE_SHUFFLE = 1,  /* LUT lookup + counting sort metadata */
    MOE_STAGE_GATHER = 2,   /* x -> x_sorted (skipped when fuse_gather) */
    MOE_STAGE_FFN_UP = 3,   /* grouped GEMM1 + SwiGLU, routed and shared */
    MOE_STAGE_FFN_DOWN = 4, /* grouped GEMM2, routed and shared */
    MOE_STAGE_COMBINE = 5,  /* weighted combine back to token order */
    MOE_NSTAGES = 6
};

/* Bits of the device data-error word that libraries built with device data
 * checks (libmoe_debug.so) set when a kernel meets an out-of-range input
 * value.  Every library clamps such values (or skips the entry) so that no
 * access leaves its buffer; only the debug build records them. */
enum moe_data_error {
    MOE_DATA_TOKEN_ID = 1,   /* tok[t] outside [0, V) */
    MOE_DATA_LUT = 2,        /* lut[v] outside [0, P) */
    MOE_DATA_SLOT = 4,       /* topk_slot[a] outside [0, E) */
    MOE_DATA_K = 8,          /* k_tok[t] outside [0, k_max] */
    MOE_DATA_PLACEMENT = 16, /* slot_to_orig[s] outside [0, E) */
    MOE_DATA_PREF = 32       /* pref entry outside [0, E) (skipped) */
};

/* Layer description (host struct). */
typedef struct moe_cfg {
    int32_t T;            /* tokens */
    int32_t H;            /* hidden size */
    int32_t E;            /* routed experts (or sub-experts) */
    int32_t P;            /* placement groups; E % P == 0, E/P a power of 2 */
    int32_t I;            /* routed expert intermediate size */
    int32_t k_max;        /* top-k; with ragged, the largest per-token k */
    int32_t ragged;       /* 1: per-token k from k_tok[] */
    int32_t n_shared;     /* always-on shared experts (weight 1) */
    int32_t I_shared;     /* intermediate size of each shared expert */
    int32_t V;            /* vocabulary size (token IDs in [0, V)) */
    int32_t n_pref;       /* preferred experts per token ID (affinity table width) */
    int32_t dtype;        /* moe_dtype */
    int32_t gate;         /* moe_gate */
    int32_t renorm;       /* softmax: 1 = renormalise weights over the selected */
    float route_scale;    /* sigmoid gate: weights scaled to sum to route_scale */
    int32_t n_rgroups;    /* sigmoid gate: routing groups (contiguous original ids) */
    int32_t topk_rgroups; /* sigmoid gate: routing groups kept */
    int32_t rgroup_topn;  /* sigmoid gate: a group's score sums its top-n keys */
    float aff_bias;       /* logit bias on a token's preferred experts */
    int32_t fuse_gather;  /* moe_forward: 1 = GEMM1 reads x rows through the
                             permutation instead of materialising x_sorted */
    int32_t weights_blocked; /* bf16: 1 = the W13/W2 arrays (routed and shared)
                                passed to moe_expert_ffn / moe_forward are in the
                                tile-blocked layout moe_pack_weights writes */
} moe_cfg;

/*
 * Host only; needs no GPU.  Checks the description: T >= 0 (an empty layer
 * is valid: the calls then enqueue nothing that reads a row); positive H, E,
 * P, I, V; k_max in [1, min(E, 64)]; T * k_max < 2^31 and T * k_max * H
 * < 2^40; for bf16 (32-bit buffer offsets) also x [T,H], the gate [E,H] and
 * one expert's [2I,H] (and the stacked shared experts' [2*n_shared*I_shared,
 * H]) below 2^31 bytes each -- the sorted-row operands of the grouped GEMMs
 * ([T*k_max, H] and [T*k_max, I]) are addressed per tile and have no such
 * limit; E <= 512; E % P == 0 and E/P a power of two; P <= 64 and
 * E*P <= 4096; n_pref in [0, E]; H % 8 == 0; for bf16 H % 128 == 0,
 * I % 64 == 0 and (n_shared*I_shared) % 64 == 0; sigmoid gate only with
 * n_rgroups in [1, 64] dividing E, 1 <= topk_rgroups <= n_rgroups,
 * 1 <= rgroup_topn <= min(8, E/n_rgroups), at least k_max experts in the
 * kept groups and a finite route_scale; aff_bias not NaN; weights_blocked
 * 0 or 1, and 1 only with bf16.  Returns MOE_OK or the error code
 * (MOE_ESHAPE, MOE_EDTYPE, MOE_EINVAL).
 */
int32_t moe_validate(const moe_cfg* cfg);

/* Host only.  Workspace bytes enough for every call with this cfg (0 if the
 * cfg is invalid). */
size_t moe_workspace_bytes(const moe_cfg* cfg);

/* Workspace bytes moe_route needs for this layer (0: none; also 0 when cfg
 * is invalid, see moe_validate).  Host only.  moe_workspace_bytes covers it. */
size_t moe_route_workspace_bytes(const moe_cfg* cfg);

/* Text of the last error on the calling thread (never NULL). */
const char* moe_last_error(void);

/* 1 when this library was built with device data checks (libmoe_debug.so),
 * 0 for the release build.  Host only. */
int32_t moe_debug_checks(void);

/*
 * Device data errors (debug builds only; not on the hot path): reads into *flags (host) the moe_data_error bits recorded in
 * the error word at the start of workspace ws -- every workspace that
 * moe_workspace_bytes or moe_route_workspace_bytes sizes begins with it -- or,
 * with ws == NULL, in the static scratch of moe_shuffle_noalloc on the
 * current device; clear != 0 zeroes the word afterwards.  The word
 * accumulates until cleared: a fresh workspace must be cleared once before
 * its first call (or its initial contents read as errors).  SYNCHRONOUS:
 * waits on `stream`.  The release build returns MOE_EINVAL (it records
 * nothing).  MOE_EINVAL also for flags == NULL.
 */
int32_t moe_debug_errors(const void* ws, uint32_t* flags, int32_t clear, void* stream);

/*
 * Route: gate GEMM (MFMA), affinity bias, top-k selection and weights.
 * Passages: each token activates the few experts its gate picks, which is
 * what makes its row travel under expert parallelism (Semantic Parallelism,
 * ko/de technical summary §1); the gate's columns are shuffled to place the
 * experts, so the chosen column index is already the placement slot and the
 * model's function is unchanged (ja technical overview §2.2A) -- the
 * selection therefore breaks ties by ORIGINAL id; top-k as a per-request
 * knob (MoE-Prism technical summary §1, §5) gives the ragged k_tok.
 *   x[T,H]          activations
 *   Wg[E,H]         gate rows in slot order (the shuffled gate columns)
 *   ebias[E]        fp32 per-expert selection bias in slot order, or NULL
 *                   (sigmoid gate only; enters selection, not the weights)
 *   slot_to_orig[E] original expert id of each slot (tie-break and routing
 *                   groups use original ids)
 *   tok[T]          token IDs in [0, V)
 *   pref[V,n_pref]  preferred ORIGINAL expert ids per token ID, or NULL; the
 *                   gate adds aff_bias to those logits (synthetic affinity)
 *   k_tok[T]        per-token k in [0, k_max] when ragged, else ignored
 * Outputs:
 *   row_ptr[T+1]    CSR offsets, exclusive scan of k_t (A = row_ptr[T])
 *   topk_slot[A_max] selected slots, token-major, in selection order:
 *                   key descending, ties to the lower ORIGINAL id.  Keys:
 *                   softmax gate — the fp32 logit; sigmoid gate —
 *                   sigmoid(l) + ebias, with sigmoid on an exp evaluated as
 *                   Cody-Waite reduction + degree-7 Taylor polynomial in fp32
 *                   fused multiply-adds (bit-reproducible).
 *   topk_w[A_max]   fp32 weights: softmax p_j (renorm: p_j / sum of selected
 *                   p); sigmoid: route_scale * s_j / sum_j s_j, s = sigmoid(l)
 *   logits[T,E]     optional fp32 export of the biased logits, slot order
 * Workspace: moe_route_workspace_bytes(cfg) bytes (device, 256-byte
 * aligned), or NULL when that is 0.  bf16 layers with E > 64 run the gate
 * GEMM as its own tiled kernel and keep its fp32 partial logits there; every
 * other layer computes the gate inside the route kernel.  In debug builds the
 * workspace also holds the data-error word, so it is never 0 there.
 * MOE_EWORKSPACE if it is missing or too small.
 */
int32_t moe_route(const moe_cfg* cfg, const void* x, const void* Wg, const float* ebias,
                  const int32_t* slot_to_orig, const int32_t* tok, const int32_t* pref,
                  const int32_t* k_tok, int32_t* row_ptr, int32_t* topk_slot, float* topk_w,
                  float* logits, void* ws, size_t ws_bytes, void* stream);

/*
 * Shuffle: token->group lookup and the dispatch metadata (Sem-MoE's token
 * shuffle by predicted device, done on one GPU as a stable counting sort).
 * Passages: before the MoE layer tokens are shuffled to the device that
 * holds their predicted experts (Semantic Parallelism, de technical summary
 * §2B, ja technical overview §2.2B), the prediction coming from a
 * lightweight token->group table (ja technical overview §2.3); the local
 * activation rate is the share of work that stays on its device (de §4):
 * here trace(pair_count) / A.
 *   row_ptr, topk_slot  as produced by moe_route
 *   tok[T], lut[V]      lut[v] in [0, P): predicted placement group of token ID v
 *   x[T,H]              activations (read only if x_sorted != NULL)
 * Outputs (int32):
 *   expert_count[E], expert_off[E+1]   rows per slot and their offsets
 *   group_count[P], group_off[P+1]     rows per placement group
 *   pair_count[P*P]     [p*P + g] = assignments of tokens predicted for group
 *                       p whose expert is in group g (the all-to-all matrix;
 *                       trace / A is the local activation rate)
 *   tok_perm[T], tok_off[P+1]  tokens ordered by (predicted group, token)
 *   sorted_to_assign[A_max]    assignment index of each sorted row; rows are
 *                       ordered by (slot, predicted group, token), so each
 *                       slot's rows are contiguous and each group's slots are
 *   assign_to_sorted[A_max]    inverse permutation
 *   x_sorted[A_max,H]   optional: x_sorted[s] = x[token of row s]; NULL skips
 * Workspace: required.
 */
int32_t moe_shuffle(const moe_cfg* cfg, const int32_t* row_ptr, const int32_t* topk_slot,
                    const int32_t* tok, const int32_t* lut, const void* x,
                    int32_t* expert_count, int32_t* expert_off, int32_t* group_count,
                    int32_t* group_off, int32_t* pair_count, int32_t* tok_perm, int32_t* tok_off,
                    int32_t* sorted_to_assign, int32_t* assign_to_sorted, void* x_sorted,
                    void* ws, size_t ws_bytes, void* stream);

/*
 * moe_shuffle without a workspace, for callers that cannot allocate device
 * memory: code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc.  Arguments, results and errors as moe_shuffle without
 * ws / ws_bytes.  Its scratch -- the predicted groups g_pred [T], the
 * per-block histograms [E*P][nb] and [P][nb] (nb = ceil(T / tpb) blocks of
 * tpb = 64..256 tokens), the row totals and the bucket and group starts --
 * lives in a static device array of MOE_NOALLOC_SCRATCH_BYTES that every GPU
 * the library runs on holds until the process ends; a layer that needs more
 * is rejected with MOE_EWORKSPACE before anything is enqueued.  Every kernel
 * overwrites the scratch it reads, so nothing needs clearing between calls,
 * but all calls on one GPU share the array: calls that overlap on one GPU
 * (other streams, other host threads) race.  Allocates nothing: no hipMalloc,
 * no hipFree, no allocating library routine.
 */
#define MOE_NOALLOC_SCRATCH_BYTES (32u << 20)
int32_t moe_shuffle_noalloc(const moe_cfg* cfg, const int32_t* row_ptr, const int32_t* topk_slot,
                            const int32_t* tok, const int32_t* lut, const void* x,
                            int32_t* expert_count, int32_t* expert_off, int32_t* group_count,
                            int32_t* group_off, int32_t* pair_count, int32_t* tok_perm,
                            int32_t* tok_off, int32_t* sorted_to_assign, int32_t* assign_to_sorted,
                            void* x_sorted, void* stream);

/*
 * Expert FFN (grouped SwiGLU GEMMs on MFMA).  Passages: each device runs the
 * experts placed on it over the rows shuffled to it (Semantic Parallelism,
 * ja technical overview §2.2A-B) -- one placement group's slot range is one
 * device's share; MoE-Prism's sub-experts are neuron slices of a monolithic
 * expert (MoE-Prism technical summary §2A), which is why each slot is a
 * plain SwiGLU over its own rows.  The SwiGLU form itself is the evaluated
 * models' (the pages name DeepSeek-V2-Lite and Qwen3-30B-A3B).  For each row
 * r of an expert e,
 *   y[r] = W2_e (silu(W1_e x_r) * (W3_e x_r)), fp32 accumulation; with bf16
 *   the intermediate is rounded to bf16 before the down projection.
 * which == MOE_FFN_ROUTED:
 *   rows [expert_off[e], expert_off[e+1]) of slots e in [e_begin, e_end)
 *   (one placement group's range is one device's share);
 *   x_sorted[A_max,H] holds the rows, or is NULL: then row s is read from
 *   x[t] with t the token of assignment sorted_to_assign[s] (CSR row_ptr);
 *   W13[E,2I,H]: rows [0,I) = W1_e, rows [I,2I) = W3_e;  W2[E,H,I];
 *   y[A_max,H]: rows written at their sorted positions.
 * which == MOE_FFN_SHARED: all T rows of x[T,H] through the n_shared shared
 *   experts stacked along the intermediate axis (their sum):
 *   W13 = Wsh13[2*ns*Is, H] (all W1 rows, then all W3 rows), W2 = Wsh2[H, ns*Is];
 *   y[T,H].  x_sorted, sorted_to_assign, row_ptr, expert_off, e_begin, e_end
 *   are ignored.
 * Nothing to compute (T = 0, or an empty slot range): returns MOE_OK after
 * checking cfg, which, the weights, y and the workspace, without reading
 * the row arguments (x, x_sorted, row_ptr, sorted_to_assign, expert_off),
 * which may then be NULL.
 * Workspace: required.
 */
int32_t moe_expert_ffn(const moe_cfg* cfg, int32_t which, const void* x_sorted, const void* x,
                       const int32_t* row_ptr, const int32_t* sorted_to_assign,
                       const int32_t* expert_off, const void* W13, const void* W2,
                       int32_t e_begin, int32_t e_end, void* y, void* ws, size_t ws_bytes,
                       void* stream);

/*
 * Combine (restore token order).  Passage: after the experts, the results
 * are gathered back and put into the original token order (Semantic
 * Parallelism, de technical summary §2B, ja technical overview §2.2B).
 * out[t] = sum_{j<k_t} topk_w[a] *
 * y_sorted[assign_to_sorted[a]] + y_sh[t], a = row_ptr[t] + j, summed in fp32
 * in j order then rounded to the dtype.  Deterministic, no atomics.
 *   y_sh[T,H] shared-expert output or NULL.
 */
int32_t moe_combine(const moe_cfg* cfg, const void* y_sorted, const int32_t* assign_to_sorted,
                    const int32_t* row_ptr, const float* topk_w, const void* y_sh, void* out,
                    void* stream);

/*
 * Shuffled reduce-scatter (SRS), one-GPU form.  Semantic Parallelism (de
 * technical summary §2B, ja technical overview §2.2B): under attention tensor
 * parallelism each of the P ranks holds a partial sum of the attention output
 * for all T tokens; the reduce-scatter is reordered so that every rank
 * receives the reduced rows of the tokens predicted to need its experts.
 * With all partials on one device:
 *     y[i] = sum_{p < n_part} x_part[p][tok_perm[i]]
 * summed in fp32 in p order and rounded once to the dtype (bf16: RNE); rank
 * g's share is rows [tok_off[g], tok_off[g+1]) (tok_perm, tok_off as
 * produced by moe_shuffle).  Rows whose tok_perm entry lies outside [0, T)
 * are written as zeros.
 *   n_part           number of partials, 1..64;
 *   x_part[n_part,T,H] partials (16-byte aligned);
 *   tok_perm[T]      int32 token of each output row;
 *   y[T,H]           output rows in tok_perm order (16-byte aligned).
 * Errors: MOE_EINVAL (null or misaligned pointer, n_part out of range),
 * configuration errors as moe_validate; MOE_EHIP on a launch failure.
 */
int32_t moe_srs(const moe_cfg* cfg, int32_t n_part, const void* x_part, const int32_t* tok_perm,
                void* y, void* stream);

/*
 * Shuffled all-gather (SAG), one-GPU form (same passages): the rows the ranks
 * hold in tok_perm order are gathered and restored to token order:
 *     out[tok_perm[i]] = y[i]          (bit copy)
 * Entries of tok_perm outside [0, T) are skipped; a tok_perm that is not a
 * permutation leaves rows of out unwritten.
 *   y[T,H] rows in tok_perm order; tok_perm[T]; out[T,H] token order (y and
 *   out 16-byte aligned, not overlapping).
 * Errors as moe_srs.
 */
int32_t moe_sag(const moe_cfg* cfg, const void* y, const int32_t* tok_perm, void* out,
                void* stream);

/*
 * Offline co-scheduling of experts, tokens and requests (Semantic
 * Parallelism: expert placement and token/request scheduling co-clustered
 * as a 0-1 program solved by alternating optimisation, de technical summary
 * §2B and key contribution 4, ko technical summary §2.2; placement fixed
 * before deployment, ja technical overview §2.2A).  Objective: profiled
 * assignments whose token is predicted for the group holding its expert.
 * Experts are ORIGINAL ids (profile with the identity placement).  Profiled
 * routing is CSR: row_ptr[n_tok+1], expert[row_ptr[n_tok]], tok[n_tok];
 * entries out of range are ignored.  All calls: MOE_EINVAL on null
 * pointers / bad sizes, configuration errors as moe_validate, MOE_EHIP on
 * launch failures.
 */

/* Token step counts: counts[v*P + g] = assignments of token ID v on experts
 * e with group[e] = g (counts [V*P] int32, device, overwritten; V*P < 2^31,
 * else MOE_ESHAPE). */
int32_t moe_token_group_counts(const moe_cfg* cfg, int32_t n_tok, const int32_t* row_ptr,
                               const int32_t* expert, const int32_t* tok, const int32_t* group,
                               int32_t* counts, void* stream);

/* Token step: lut[v] = argmax_g counts[v*P + g], ties to the lower group,
 * IDs with no count map to v mod P (lut [V] int32, device). */
int32_t moe_lut_from_counts(const moe_cfg* cfg, const int32_t* counts, int32_t* lut, void* stream);

/* Expert step counts: counts[g*E + e] = assignments at expert e of tokens
 * with lut[tok] = g (counts [P*E] int32, device, overwritten). */
int32_t moe_expert_group_counts(const moe_cfg* cfg, int32_t n_tok, const int32_t* row_ptr,
                                const int32_t* expert, const int32_t* tok, const int32_t* lut,
                                int32_t* counts, void* stream);

/* Host only.  Assigns n items to P groups, n/P per group, maximising
 * sum_i score[i*P + group[i]] exactly (Hungarian method, O(n^3), n <= 4096).
 * score [n*P] and group [n] are host arrays.  Returns the optimum, or a
 * negative moe_status (MOE_ESHAPE unless P divides n, MOE_EINVAL on NULL). */
int64_t moe_balanced_assign(int32_t n, int32_t P, const int64_t* score, int32_t* group);

/* Alternating optimisation of the expert grouping, starting from the
 * balanced grouping group[E] (host, in/out): token step (lut), then expert
 * step (moe_balanced_assign on the expert counts); stops after max_iters
 * rounds or when the expert step gains nothing (the grouping is then kept).
 * Outputs: group (host), perm[E] (host, slot of each original expert: group
 * g's experts take slots [g*E/P, (g+1)*E/P) in ascending id; or NULL),
 * lut[V] (device, the token step of the final grouping), objective
 * [2*max_iters] (host or NULL: the objective before and after each expert
 * step), n_steps (host or NULL: entries written).  counts_vp [V*P] and
 * counts_pe [P*E] are device scratch.  SYNCHRONOUS: waits on `stream`. */
int32_t moe_optimize_placement(const moe_cfg* cfg, int32_t n_tok, const int32_t* row_ptr,
                               const int32_t* expert, const int32_t* tok, int32_t max_iters,
                               int32_t* group, int32_t* perm, int32_t* lut, int32_t* counts_vp,
                               int32_t* counts_pe, int64_t* objective, int32_t* n_steps,
                               void* stream);

/* Inter-request scheduling under attention data parallelism (de technical
 * summary §2B; ko technical summary §2.2): hist[r*P + g] = tokens of request
 * r (tokens [req_ptr[r], req_ptr[r+1]) of tok) with lut[tok] = g (device,
 * int32, P <= 64).  Requests then go to ranks with moe_balanced_assign on
 * hist. */
int32_t moe_request_group_hist(const moe_cfg* cfg, int32_t n_req, const int32_t* req_ptr,
                               const int32_t* tok, const int32_t* lut, int32_t* hist, void* stream);

/* The sigmoid of the grouped gate's selection keys, on its own: y[i] =
 * 1 / (1 + exp(-x[i])) in fp32 with exp evaluated as in moe_route (Cody-Waite
 * reduction, degree-7 Taylor polynomial in fused multiply-adds, exact
 * scaling; 0 below -87, +inf above 88), each step one IEEE-rounded fp32
 * operation, so any other implementation of the same steps reproduces it bit
 * for bit.  The selection of the sigmoid gate compares these values, which is
 * why they are exported for checking.  (The pages do not describe this gate:
 * they name DeepSeek-V3 only as an example of a large MoE model in their
 * problem statements, de technical summary §1 and ja §1, and evaluate on
 * DeepSeek-V2-Lite and Qwen3-30B-A3B; the sigmoid gate with per-expert bias
 * and group-limited selection is the DeepSeek-V3-shaped layer's own form.)
 *   x[n], y[n]  device fp32 arrays (y may equal x); n >= 0.
 * MOE_EINVAL for n < 0 or a NULL pointer with n > 0. */
int32_t moe_sigmoid(const float* x, float* y, int64_t n, void* stream);

/* Weights in the tile-blocked layout (bf16 layers; for callers that set
 * cfg->weights_blocked).  The grouped GEMMs read a weight tile's 64-wide
 * k-step as one contiguous block instead of a 128-byte piece of each of its
 * rows, which lie a whole row apart in the row-major layout: per expert,
 * for each n-tile j and k-step kt, the block [BN rows][64 elements] at
 * ((j * K/64 + kt) * BN) * 64 elements; for W13 a block's rows are the
 * tile's BN/2 W1 rows followed by the matching BN/2 W3 rows, for W2 the
 * tile's BN rows of W2.  BN = 256 when 2*I, 2*n_shared*I_shared and H are
 * multiples of 256, else 128 (the GEMMs' own tile width).
 *   which = MOE_FFN_ROUTED: W13 [E,2I,H], W2 [E,H,I];
 *   which = MOE_FFN_SHARED: W13 = Wsh13 [2*ns*Is,H], W2 = Wsh2 [H,ns*Is].
 * The outputs W13_blk, W2_blk have the inputs' sizes (device, distinct
 * from the inputs).  A one-time step, like the slot permutation. */
int32_t moe_pack_weights(const moe_cfg* cfg, int32_t which, const void* W13, const void* W2,
                         void* W13_blk, void* W2_blk, void* stream);

/* Device tensors of one layer for moe_forward (host struct of device pointers). */
typedef struct moe_weights {
    const void* Wg;              /* [E,H] slot order */
    const float* ebias;          /* [E] slot order, or NULL */
    const int32_t* slot_to_orig; /* [E] */
    const void* W13;             /* [E,2I,H] slot order */
    const void* W2;              /* [E,H,I] slot order */
    const void* Wsh13;           /* [2*ns*Is,H] or NULL when n_shared == 0 */
    const void* Wsh2;            /* [H,ns*Is] or NULL */
    const int32_t* lut;          /* [V] */
    const int32_t* pref;         /* [V,n_pref] original ids, or NULL */
} moe_weights;

typedef struct moe_inputs {
    const void* x;        /* [T,H] */
    const int32_t* tok;   /* [T] */
    const int32_t* k_tok; /* [T] when ragged, else NULL */
} moe_inputs;

/* Optional outputs of moe_forward; every NULL member is kept in the
 * workspace instead.  events: 2*MOE_NSTAGES hipEvent_t handles (or NULL);
 * events[2*s] and events[2*s+1] are recorded on the stream before and after
 * stage s. */
typedef struct moe_exports {
    float* logits;
    int32_t* row_ptr;
    int32_t* topk_slot;
    float* topk_w;
    int32_t* expert_count;
    int32_t* expert_off;
    int32_t* group_count;
    int32_t* group_off;
    int32_t* pair_count;
    int32_t* tok_perm;
    int32_t* tok_off;
    int32_t* sorted_to_assign;
    int32_t* assign_to_sorted;
    void* x_sorted; /* ignored when fuse_gather */
    void* y_sorted;
    void* y_shared;
    void* const* events;
} moe_exports;

/*
 * The whole layer: route -> shuffle -> gather -> expert FFN (routed and
 * shared) -> combine, enqueued on one stream.  out[T,H] in token order.
 * Passages: the Sem-MoE layer step on one device -- routing through the
 * shuffled gate (Semantic Parallelism, ja technical overview §2.2A), token
 * shuffle by predicted group (de technical summary §2B, ja §2.2B-§2.3),
 * the experts, and the restore to the original order (de §2B, ja §2.2B);
 * the all-to-all that expert parallelism would need (ko/de §1) is replaced
 * by the counting sort and a gather fused into the first GEMM's row loads.
 * ex may be NULL.  Workspace: moe_workspace_bytes(cfg).
 */
int32_t moe_forward(const moe_cfg* cfg, const moe_weights* w, const moe_inputs* in, void* out,
                    const moe_exports* ex, void* ws, size_t ws_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MOE_H */
