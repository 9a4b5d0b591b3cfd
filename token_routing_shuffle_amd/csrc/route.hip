// Route: gate GEMM on MFMA, synthetic affinity bias, top-k selection and
// routing weights, fused in one kernel per 16-token tile.
//
// The gate matrix rows are stored in slot order (the Sem-MoE placement is a
// shuffle of the gate's columns: Japanese summary, technical overview
// §2.2A), so the selected indices come out as slots directly; the tie-break
// and the DeepSeek-V3-style routing groups use the original expert id through
// slot_to_orig, which keeps the layer's result independent of the placement.
#include "common.h"
#include "internal.h"

namespace moe {
namespace {

constexpr int kBM = 16;        // tokens per block
constexpr int kThreads = 512;  // 8 waves
constexpr int kWaves = kThreads / 64;

struct RouteParams {
    int T, H, E, V, n_pref, k_max, ragged, gate, renorm;
    float route_scale, aff_bias;
    int n_rgroups, topk_rgroups, rgroup_topn;
    const void* x;
    const void* Wg;
    const float* ebias;
    const int32_t* s2o;
    const int32_t* tok;
    const int32_t* pref;
    const int32_t* k_tok;
    int32_t* row_ptr;   // read when ragged (k_row_ptr wrote it), else written here
    int32_t* topk_slot;
    float* topk_w;
    float* logits;
};

// CSR offsets: row_ptr[t] = sum of k over tokens < t (k_tok clamped to
// [0, k_max] so that A never exceeds T*k_max).
__global__ __launch_bounds__(1024) void k_row_ptr(int T, int k_max, int ragged,
                                                   const int32_t* __restrict__ k_tok,
                                                   int32_t* __restrict__ row_ptr)
{
    __shared__ int smem[17];
    if (!ragged) {
        for (int t = threadIdx.x; t <= T; t += blockDim.x) row_ptr[t] = t * k_max;
        return;
    }
    int carry = 0;
    for (int base = 0; base < T; base += 4 * 1024) {
        int v[4];
        int sum = 0;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int t = base + threadIdx.x * 4 + q;
            v[q] = t < T ? clampi(k_tok[t], 0, k_max) : 0;
            sum += v[q];
        }
        int total;
        int run = carry + block_excl_scan(sum, smem, &total);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int t = base + threadIdx.x * 4 + q;
            if (t < T) row_ptr[t] = run;
            run += v[q];
        }
        carry += total;
    }
    if (threadIdx.x == 0) row_ptr[T] = carry;
}

// Winner of (ordered key desc, original id asc); sentinel uk = 0 loses to any key.
MOE_DEV void better_take(uint32_t& uk, uint32_t& id, uint32_t& s, uint32_t ouk, uint32_t oid,
                         uint32_t os)
{
    if (ouk > uk || (ouk == uk && oid < id)) {
        uk = ouk;
        id = oid;
        s = os;
    }
}

template <int NTW, bool BF16>
__global__ __launch_bounds__(kThreads) void k_route(RouteParams p)
{
    constexpr int EP = NTW * 64;  // experts padded to a multiple of 64
    __shared__ float s_log[kBM][EP + 4];
    __shared__ int s_s2o[EP];
    __shared__ int s_o2s[EP];
    __shared__ float s_key[kWaves][EP];
    __shared__ float s_gs[kWaves][64];
    constexpr int kSK = NTW >= kWaves ? 1 : kWaves / NTW;
    __shared__ float s_part[kSK > 1 ? kSK : 1][kBM][kSK > 1 ? EP : 1];

    const int tid = threadIdx.x;
    const int w = tid >> 6;
    const int l = tid & 63;
    const int t0 = blockIdx.x * kBM;
    const int T = p.T, H = p.H, E = p.E;

    __shared__ int s_rp[kBM], s_kt[kBM];
    for (int s = tid; s < EP; s += kThreads) s_s2o[s] = s < E ? clampi(p.s2o[s], 0, E - 1) : s;
    if (tid < kBM) {
        const int t = t0 + tid;
        if (p.ragged) {
            s_rp[tid] = t < T ? p.row_ptr[t] : 0;
        } else {  // fixed k: the CSR offsets are t * k, written by the token's block
            s_rp[tid] = t * p.k_max;
            if (t < T) p.row_ptr[t] = t * p.k_max;
            if (t == T - 1) p.row_ptr[T] = T * p.k_max;
        }
        s_kt[tid] = t >= T ? 0 : (p.ragged ? clampi(p.k_tok[t], 0, p.k_max) : p.k_max);
    }
    // the affinity table is read before the GEMM so its latency overlaps it
    const bool do_bias = p.pref != nullptr && p.aff_bias != 0.0f && p.n_pref > 0;
    const int np = p.n_pref;
    int pre_o[4], pre_row[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        pre_o[q] = -1;
        pre_row[q] = 0;
        const int idx = tid + q * kThreads;
        if (do_bias && idx < kBM * np) {
            const int row = idx / np, j = idx % np;
            const int t = t0 + row;
            if (t < T) {
                const int v = clampi(p.tok[t], 0, p.V - 1);
                pre_o[q] = p.pref[(size_t)v * np + j];
                pre_row[q] = row;
            }
        }
    }
    __syncthreads();
    for (int s = tid; s < E; s += kThreads) s_o2s[s_s2o[s]] = s;

    // ---------------- gate GEMM: logits[16 tokens][E] ----------------
    if constexpr (BF16) {
        // MFMA 16x16x32 bf16.  Lane l feeds token row (l & 15) and expert
        // column (l & 15) of its tile; its 4-lane group kg = l >> 4 owns the
        // contiguous k-range [16kg, 16kg+16) of every 64-wide chunk, split over
        // two MFMAs (A and B use the same k assignment, so the contraction is
        // complete; only the summation order is the hardware's).
        // Waves split the chunks (SK ways, interleaved) and the column tiles
        // (SN ways); partial sums over the K split are added in wave order.
        constexpr int SK = kSK;
        constexpr int SN = kWaves / SK;
        constexpr int TPW = NTW * 4 / SN;   // 16-column tiles per wave
        constexpr int U = TPW <= 4 ? 4 : 1; // chunks in flight per iteration
        const int wk = w % SK, wn = w / SK;
        const int r = l & 15, kg = l >> 4;
        const int tA = min(t0 + r, T - 1);
        const uint16_t* xa = (const uint16_t*)p.x + (size_t)tA * H + kg * 16;
        const uint16_t* wb[TPW];
        f32x4_t acc[TPW];
#pragma unroll
        for (int i = 0; i < TPW; ++i) {
            const int col = min((wn * TPW + i) * 16 + r, E - 1);
            wb[i] = (const uint16_t*)p.Wg + (size_t)col * H + kg * 16;
            acc[i] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        }
        const int nch = H / 64;
        for (int c = wk; c < nch; c += U * SK) {
            bf16x8_t a[U][2], b[U][TPW][2];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int k0 = min(c + u * SK, nch - 1) * 64;
                a[u][0] = *(const bf16x8_t*)(xa + k0);
                a[u][1] = *(const bf16x8_t*)(xa + k0 + 8);
#pragma unroll
                for (int i = 0; i < TPW; ++i) {
                    b[u][i][0] = *(const bf16x8_t*)(wb[i] + k0);
                    b[u][i][1] = *(const bf16x8_t*)(wb[i] + k0 + 8);
                }
            }
#pragma unroll
            for (int u = 0; u < U; ++u) {
                if (c + u * SK < nch) {
#pragma unroll
                    for (int i = 0; i < TPW; ++i) {
                        acc[i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[u][0], b[u][i][0], acc[i], 0, 0, 0);
                        acc[i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[u][1], b[u][i][1], acc[i], 0, 0, 0);
                    }
                }
            }
        }
        // D layout: lane l holds column (l & 15), rows 4*(l >> 4) + v
        if constexpr (SK == 1) {
#pragma unroll
            for (int i = 0; i < TPW; ++i)
#pragma unroll
                for (int v = 0; v < 4; ++v) s_log[kg * 4 + v][(wn * TPW + i) * 16 + r] = acc[i][v];
        } else {
#pragma unroll
            for (int i = 0; i < TPW; ++i)
#pragma unroll
                for (int v = 0; v < 4; ++v)
                    s_part[wk][kg * 4 + v][(wn * TPW + i) * 16 + r] = acc[i][v];
            __syncthreads();
            for (int idx = tid; idx < kBM * EP; idx += kThreads) {
                const int row = idx / EP, col = idx % EP;
                float sum = s_part[0][row][col];
#pragma unroll
                for (int q = 1; q < SK; ++q) sum += s_part[q][row][col];
                s_log[row][col] = sum;
            }
        }
    } else {
        const float* x = (const float*)p.x;
        const float* Wg = (const float*)p.Wg;
        for (int idx = tid; idx < kBM * EP; idx += kThreads) {
            const int row = idx / EP, col = idx % EP;
            const int t = t0 + row;
            float s = 0.0f;
            if (t < T && col < E) {
                const float* xr = x + (size_t)t * H;
                const float* wr = Wg + (size_t)col * H;
                for (int h = 0; h < H; ++h) s = fmaf(xr[h], wr[h], s);
            }
            s_log[row][col] = s;
        }
    }
    __syncthreads();

    // ---------------- synthetic affinity bias ----------------
    if (do_bias) {
#pragma unroll
        for (int q = 0; q < 4; ++q)
            if (pre_o[q] >= 0 && pre_o[q] < E) s_log[pre_row[q]][s_o2s[pre_o[q]]] += p.aff_bias;
        for (int idx = tid + 4 * kThreads; idx < kBM * np; idx += kThreads) {
            const int row = idx / np, j = idx % np;
            const int t = t0 + row;
            if (t < T) {
                const int v = clampi(p.tok[t], 0, p.V - 1);
                const int o = p.pref[(size_t)v * np + j];
                if (o >= 0 && o < E) s_log[row][s_o2s[o]] += p.aff_bias;
            }
        }
        __syncthreads();
    }
    if (p.logits != nullptr) {
        for (int idx = tid; idx < kBM * E; idx += kThreads) {
            const int row = idx / E, col = idx % E;
            if (t0 + row < T) p.logits[(size_t)(t0 + row) * E + col] = s_log[row][col];
        }
    }

    // ---------------- selection + weights: one wave per token ----------------
    const bool sigm = p.gate == MOE_GATE_SIGMOID_GROUPED;
    const bool grouped = sigm && p.n_rgroups > 1 && p.topk_rgroups < p.n_rgroups;
    const int gsize = grouped ? E / p.n_rgroups : E;
    for (int it = 0; it < kBM / kWaves; ++it) {
        const int row = w + kWaves * it;
        const int t = t0 + row;
        const bool active = t < T;  // wave-uniform
        const int kt = s_kt[row];
        (void)active;

        float lg[NTW], key[NTW];
        uint32_t oid[NTW];
        bool ok[NTW];
#pragma unroll
        for (int i = 0; i < NTW; ++i) {
            const int s = l + 64 * i;
            ok[i] = s < E;
            lg[i] = ok[i] ? s_log[row][s] : 0.0f;
            oid[i] = (uint32_t)s_s2o[s];
            if (sigm) {
                key[i] = cw_sigmoidf(lg[i]);
                if (p.ebias != nullptr && ok[i]) key[i] = key[i] + p.ebias[s];
            } else {
                key[i] = lg[i];
            }
        }
        if (grouped) {
#pragma unroll
            for (int i = 0; i < NTW; ++i)
                if (ok[i]) s_key[w][oid[i]] = key[i];
            __syncthreads();
            if (l < p.n_rgroups) {
                // sum of the rgroup_topn largest keys, largest first
                float top[8];
                const int n = p.rgroup_topn;
                for (int q = 0; q < 8; ++q) top[q] = -__builtin_inff();
                for (int e = 0; e < gsize; ++e) {
                    float v = s_key[w][l * gsize + e];
                    for (int q = 0; q < 8; ++q) {
                        if (q < n && v > top[q]) {
                            const float tmp = top[q];
                            top[q] = v;
                            v = tmp;
                        }
                    }
                }
                float sc = top[0];
                for (int q = 1; q < 8; ++q)
                    if (q < n) sc = sc + top[q];
                s_gs[w][l] = sc;
            }
            __syncthreads();
            uint64_t kept = 0;
            for (int j = 0; j < p.topk_rgroups; ++j) {
                int best = -1;
                float bs = 0.0f;
                for (int g = 0; g < p.n_rgroups; ++g) {
                    if ((kept >> g) & 1ull) continue;
                    const float sc = s_gs[w][g];
                    if (best < 0 || sc > bs) {
                        best = g;
                        bs = sc;
                    }
                }
                kept |= 1ull << best;
            }
#pragma unroll
            for (int i = 0; i < NTW; ++i) ok[i] = ok[i] && ((kept >> (oid[i] / gsize)) & 1ull);
        }

        bool taken[NTW];
#pragma unroll
        for (int i = 0; i < NTW; ++i) taken[i] = false;
        uint32_t myslot = 0;
        for (int j = 0; j < kt; ++j) {
            uint32_t buk = 0, bid = 0xffffffffu, bs = 0;
#pragma unroll
            for (int i = 0; i < NTW; ++i)
                if (ok[i] && !taken[i]) better_take(buk, bid, bs, ordered_key(key[i]), oid[i], l + 64 * i);
            wave_argbest(buk, bid, bs);
#pragma unroll
            for (int i = 0; i < NTW; ++i)
                if (bs == (uint32_t)(l + 64 * i)) taken[i] = true;
            if (l == j) myslot = bs;
        }
        if (kt == 0) continue;

        const int base = s_rp[row];
        const float mylog = s_log[row][l < kt ? myslot : 0];
        float wt;
        if (!sigm) {
            float m = -__builtin_inff();
#pragma unroll
            for (int i = 0; i < NTW; ++i)
                if (l + 64 * i < E) m = fmaxf(m, lg[i]);
            m = wave_max(m);
            const float ej = l < kt ? expf(mylog - m) : 0.0f;
            float denom;
            if (p.renorm) {
                denom = wave_sum(ej);
            } else {
                // sum over all experts in ORIGINAL id order (lane l adds ids
                // l, l+64, ...), so the rounding does not depend on placement
#pragma unroll
                for (int i = 0; i < NTW; ++i)
                    if (ok[i]) s_key[w][oid[i]] = expf(lg[i] - m);
                __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
                __builtin_amdgcn_wave_barrier();
                float sa = 0.0f;
#pragma unroll
                for (int i = 0; i < NTW; ++i)
                    if (l + 64 * i < E) sa += s_key[w][l + 64 * i];
                denom = wave_sum(sa);
                __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
                __builtin_amdgcn_wave_barrier();
            }
            wt = ej / denom;
        } else {
            const float sj = l < kt ? cw_sigmoidf(mylog) : 0.0f;
            const float denom = wave_sum(sj);
            wt = p.route_scale * sj / denom;
        }
        if (l < kt) {
            p.topk_slot[base + l] = (int32_t)myslot;
            p.topk_w[base + l] = wt;
        }
    }
}

template <bool BF16>
hipError_t launch_route_t(const RouteParams& p, hipStream_t s)
{
    const dim3 grid(ceil_div(p.T, kBM)), block(kThreads);
    const int ntw = ceil_div(p.E, 64);
    if (ntw <= 1)
        hipLaunchKernelGGL((k_route<1, BF16>), grid, block, 0, s, p);
    else if (ntw <= 2)
        hipLaunchKernelGGL((k_route<2, BF16>), grid, block, 0, s, p);
    else if (ntw <= 4)
        hipLaunchKernelGGL((k_route<4, BF16>), grid, block, 0, s, p);
    else
        hipLaunchKernelGGL((k_route<8, BF16>), grid, block, 0, s, p);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_row_ptr(const moe_cfg& c, const int32_t* k_tok, int32_t* row_ptr, hipStream_t s)
{
    // with a fixed k and T > 0 the route kernel writes row_ptr itself
    if (!c.ragged && c.T > 0) return hipSuccess;
    hipLaunchKernelGGL(k_row_ptr, dim3(1), dim3(1024), 0, s, c.T, c.k_max, c.ragged, k_tok, row_ptr);
    return hipGetLastError();
}

hipError_t launch_route(const moe_cfg& c, const void* x, const void* Wg, const float* ebias,
                        const int32_t* slot_to_orig, const int32_t* tok, const int32_t* pref,
                        const int32_t* k_tok, int32_t* row_ptr, int32_t* topk_slot,
                        float* topk_w, float* logits, hipStream_t s)
{
    if (c.T == 0) return hipSuccess;
    RouteParams p;
    p.T = c.T;
    p.H = c.H;
    p.E = c.E;
    p.V = c.V;
    p.n_pref = c.n_pref;
    p.k_max = c.k_max;
    p.ragged = c.ragged;
    p.gate = c.gate;
    p.renorm = c.renorm;
    p.route_scale = c.route_scale;
    p.aff_bias = c.aff_bias;
    p.n_rgroups = c.n_rgroups;
    p.topk_rgroups = c.topk_rgroups;
    p.rgroup_topn = c.rgroup_topn;
    p.x = x;
    p.Wg = Wg;
    p.ebias = c.gate == MOE_GATE_SIGMOID_GROUPED ? ebias : nullptr;
    p.s2o = slot_to_orig;
    p.tok = tok;
    p.pref = pref;
    p.k_tok = k_tok;
    p.row_ptr = row_ptr;
    p.topk_slot = topk_slot;
    p.topk_w = topk_w;
    p.logits = logits;
    return c.dtype == MOE_BF16 ? launch_route_t<true>(p, s) : launch_route_t<false>(p, s);
}

}  // namespace moe
