// Offline co-scheduling of experts, tokens and requests into P device groups
// (Semantic Parallelism: experts and tokens are co-clustered as a 0-1
// program solved by alternating optimisation, German summary, technical
// summary §2B and key contribution 4; Korean summary, technical summary §2.2;
// expert placement before deployment, Japanese summary, technical overview
// §2.2A; requests placed on data-parallel ranks by affinity, German summary
// §2B).
//
// Objective: the profiled assignments whose token is predicted for the group
// holding its expert.  The alternating steps each maximise it exactly:
//   token step   lut[v] = argmax_g D[v][g], D[v][g] = assignments of token
//                ID v on experts of group g (ties to the lower group; IDs
//                never seen map to v mod P);
//   expert step  an exact balanced assignment of experts to groups (E/P per
//                group) maximising sum_e C[group[e]][e], C[g][e] = assignments
//                at expert e of tokens with lut = g.
// The counts are GPU histograms over the profiled assignments; the balanced
// assignment is solved on the host (Hungarian method with potentials on the
// n x n matrix that gives each group n/P identical columns).
#include "common.h"
#include "internal.h"

#include <algorithm>
#include <limits>
#include <vector>

namespace moe {
namespace {

constexpr int kThreads = 256;

__global__ __launch_bounds__(kThreads) void k_fill_i32(int32_t* p, long long n, int32_t v)
{
    for (long long i = blockIdx.x * (long long)kThreads + threadIdx.x; i < n;
         i += (long long)gridDim.x * kThreads)
        p[i] = v;
}

// D[v][g] += 1 for every assignment (token t, expert e): v = tok[t], g = group[e].
// Thread per token; the wave's lanes take their j-th assignments together and
// lanes with the same (v, g) key add their count with one atomic (the lowest
// of them): frequent token ids would otherwise serialise thousands of
// atomics on a few counters.
__global__ __launch_bounds__(kThreads) void k_token_group_counts(int n_tok, int V, int E, int P, int key_bits,
                                                                 const int32_t* __restrict__ row_ptr,
                                                                 const int32_t* __restrict__ expert,
                                                                 const int32_t* __restrict__ tok,
                                                                 const int32_t* __restrict__ group,
                                                                 int32_t* __restrict__ D)
{
    const int t = blockIdx.x * kThreads + threadIdx.x;
    int v = t < n_tok ? tok[t] : -1;
    const bool ok = t < n_tok && (unsigned)v < (unsigned)V;
    const int a0 = ok ? row_ptr[t] : 0;
    const int n = ok ? row_ptr[t + 1] - a0 : 0;
    int nmax = n;  // wave-uniform loop bound: every lane takes part in the ballots
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) nmax = max(nmax, __shfl_xor(nmax, o));
    for (int j = 0; j < nmax; ++j) {
        bool valid = j < n;
        uint32_t key = 0;
        if (valid) {
            const int e = expert[a0 + j];
            valid = (unsigned)e < (unsigned)E;
            if (valid) {
                const int g = group[e];
                valid = (unsigned)g < (unsigned)P;
                key = (uint32_t)(v * P + g);
            }
        }
        const uint64_t act = __ballot(valid);
        if (act == 0) continue;
        const uint64_t peers = match_key(key, key_bits, act);
        if (valid && (peers & lanemask_lt()) == 0) atomicAdd(&D[key], (int)__popcll(peers));
    }
}

__global__ __launch_bounds__(kThreads) void k_lut_from_counts(int V, int P, const int32_t* __restrict__ D,
                                                              int32_t* __restrict__ lut)
{
    const int v = blockIdx.x * kThreads + threadIdx.x;
    if (v >= V) return;
    int best = 0, bc = D[(size_t)v * P];
    for (int g = 1; g < P; ++g) {
        const int c = D[(size_t)v * P + g];
        if (c > bc) {
            bc = c;
            best = g;
        }
    }
    lut[v] = bc > 0 ? best : v % P;
}

// C[g][e] += 1 for every assignment: g = lut[tok[t]].  Per-block histogram in
// LDS (P*E <= 4096 counters), added to the global one at the end.
__global__ __launch_bounds__(kThreads) void k_expert_group_counts(int n_tok, int V, int E, int P,
                                                                  const int32_t* __restrict__ row_ptr,
                                                                  const int32_t* __restrict__ expert,
                                                                  const int32_t* __restrict__ tok,
                                                                  const int32_t* __restrict__ lut,
                                                                  int32_t* __restrict__ C)
{
    __shared__ int h[4096];
    const int n = P * E;
    for (int i = threadIdx.x; i < n; i += kThreads) h[i] = 0;
    __syncthreads();
    const int per_block = 4 * kThreads;
    const int t0 = blockIdx.x * per_block, t1 = min(n_tok, t0 + per_block);
    for (int t = t0 + threadIdx.x; t < t1; t += kThreads) {
        const int v = tok[t];
        if ((unsigned)v >= (unsigned)V) continue;
        const int g = lut[v];
        if ((unsigned)g >= (unsigned)P) continue;
        for (int a = row_ptr[t]; a < row_ptr[t + 1]; ++a) {
            const int e = expert[a];
            if ((unsigned)e < (unsigned)E) atomicAdd(&h[g * E + e], 1);
        }
    }
    __syncthreads();
    for (int i = threadIdx.x; i < n; i += kThreads)
        if (h[i]) atomicAdd(&C[i], h[i]);
}

// H[r][g] = tokens of request r predicted for group g: one block per request
__global__ __launch_bounds__(kThreads) void k_request_group_hist(int n_req, int V, int P,
                                                                 const int32_t* __restrict__ req_ptr,
                                                                 const int32_t* __restrict__ tok,
                                                                 const int32_t* __restrict__ lut,
                                                                 int32_t* __restrict__ H)
{
    __shared__ int h[64];
    const int r = blockIdx.x;
    if (threadIdx.x < 64) h[threadIdx.x] = 0;
    __syncthreads();
    for (int t = req_ptr[r] + threadIdx.x; t < req_ptr[r + 1]; t += kThreads) {
        const int v = tok[t];
        if ((unsigned)v >= (unsigned)V) continue;
        const int g = lut[v];
        if ((unsigned)g < (unsigned)P) atomicAdd(&h[g], 1);
    }
    __syncthreads();
    if (threadIdx.x < P) H[(size_t)r * P + threadIdx.x] = h[threadIdx.x];
}

}  // namespace

hipError_t launch_fill_i32(int32_t* p, long long n, int32_t v, hipStream_t s)
{
    if (n <= 0) return hipSuccess;
    const long long blocks = std::min<long long>((n + kThreads - 1) / kThreads, 4096);
    hipLaunchKernelGGL(k_fill_i32, dim3((unsigned)blocks), dim3(kThreads), 0, s, p, n, v);
    return hipGetLastError();
}

hipError_t launch_token_group_counts(int n_tok, int V, int E, int P, const int32_t* row_ptr,
                                     const int32_t* expert, const int32_t* tok, const int32_t* group,
                                     int32_t* D, hipStream_t s)
{
    hipError_t e = launch_fill_i32(D, (long long)V * P, 0, s);
    if (e != hipSuccess || n_tok == 0) return e;
    hipLaunchKernelGGL(k_token_group_counts, dim3((unsigned)ceil_div(n_tok, kThreads)), dim3(kThreads),
                       0, s, n_tok, V, E, P, ilog2(V * P), row_ptr, expert, tok, group, D);
    return hipGetLastError();
}

hipError_t launch_lut_from_counts(int V, int P, const int32_t* D, int32_t* lut, hipStream_t s)
{
    hipLaunchKernelGGL(k_lut_from_counts, dim3((unsigned)ceil_div(V, kThreads)), dim3(kThreads), 0, s,
                       V, P, D, lut);
    return hipGetLastError();
}

hipError_t launch_expert_group_counts(int n_tok, int V, int E, int P, const int32_t* row_ptr,
                                      const int32_t* expert, const int32_t* tok, const int32_t* lut,
                                      int32_t* C, hipStream_t s)
{
    hipError_t e = launch_fill_i32(C, (long long)P * E, 0, s);
    if (e != hipSuccess || n_tok == 0) return e;
    hipLaunchKernelGGL(k_expert_group_counts, dim3((unsigned)ceil_div(n_tok, 4 * kThreads)),
                       dim3(kThreads), 0, s, n_tok, V, E, P, row_ptr, expert, tok, lut, C);
    return hipGetLastError();
}

hipError_t launch_request_group_hist(int n_req, int V, int P, const int32_t* req_ptr,
                                     const int32_t* tok, const int32_t* lut, int32_t* H,
                                     hipStream_t s)
{
    if (n_req == 0) return hipSuccess;
    hipLaunchKernelGGL(k_request_group_hist, dim3((unsigned)n_req), dim3(kThreads), 0, s, n_req, V, P,
                       req_ptr, tok, lut, H);
    return hipGetLastError();
}

// Items to groups, n/P per group, maximising sum_i score[i][group[i]]
// (score row-major [n][P]).  Hungarian method with potentials (shortest
// augmenting paths, O(n^3)) on the n x n cost matrix -score[i][j / (n/P)].
// Returns the optimum.
long long balanced_assign_host(int n, int P, const long long* score, int32_t* group)
{
    if (n == 0) return 0;
    const int cap = n / P;
    const long long INF = std::numeric_limits<long long>::max() / 4;
    auto cost = [&](int i, int j) { return -score[(size_t)i * P + j / cap]; };  // 0-based
    // 1-based arrays: u rows, v columns, p[j] = row matched to column j
    std::vector<long long> u(n + 1, 0), v(n + 1, 0), minv(n + 1);
    std::vector<int> p(n + 1, 0), way(n + 1, 0);
    std::vector<char> used(n + 1);
    for (int i = 1; i <= n; ++i) {
        p[0] = i;
        int j0 = 0;
        std::fill(minv.begin(), minv.end(), INF);
        std::fill(used.begin(), used.end(), 0);
        do {
            used[j0] = 1;
            const int i0 = p[j0];
            long long delta = INF;
            int j1 = 0;
            for (int j = 1; j <= n; ++j) {
                if (used[j]) continue;
                const long long cur = cost(i0 - 1, j - 1) - u[i0] - v[j];
                if (cur < minv[j]) {
                    minv[j] = cur;
                    way[j] = j0;
                }
                if (minv[j] < delta) {
                    delta = minv[j];
                    j1 = j;
                }
            }
            for (int j = 0; j <= n; ++j) {
                if (used[j]) {
                    u[p[j]] += delta;
                    v[j] -= delta;
                } else {
                    minv[j] -= delta;
                }
            }
            j0 = j1;
        } while (p[j0] != 0);
        do {
            const int j1 = way[j0];
            p[j0] = p[j1];
            j0 = j1;
        } while (j0);
    }
    long long total = 0;
    for (int j = 1; j <= n; ++j) {
        const int i = p[j] - 1;
        group[i] = (j - 1) / cap;
        total += score[(size_t)i * P + group[i]];
    }
    return total;
}

}  // namespace moe
