// Shuffle: token->group lookup table and the dispatch metadata, as a stable
// counting sort of the (token, expert) assignments by the key
// (slot, predicted group, token), plus the token-level order by
// (predicted group, token).
//
// The pages shuffle each token, before the MoE layer, to the device hosting
// its predicted experts and put results back in the original order afterwards
// (German summary, technical summary §2B; Japanese summary, technical overview
// §2.2B), with the prediction read from a lightweight token->group table
// (Japanese summary, §2.3).  On one GPU the "devices" are the P placement
// groups of consecutive slots and no data moves between GPUs: the sort yields
// expert-contiguous rows (each group's slots adjacent), per-slot / per-group
// counts and offsets, the P x P would-be all-to-all matrix and the token
// permutation.
//
// Three kernels: per-block LDS histograms, stored block-major (one
// contiguous row of bucket counts per block); a column scan that turns each
// bucket's per-block counts into offsets within the bucket (and the bucket's
// total); a scatter whose blocks each scan the bucket totals (E*P of them)
// into bucket starts in LDS (one extra block writes the per-slot / per-group
// results from the same scan; an empty layer runs that scan as a kernel of
// its own) and rank equal buckets inside a wave with ballots (stable: blocks,
// waves, chunks and lanes all follow assignment order).  The global offset of
// (bucket k, block b) is bucket_start[k] + (counts of k in blocks before b).
#include "common.h"
#include "internal.h"

namespace moe {
namespace {

constexpr int kThreads = 256;
constexpr int kMaxTPB = kShuffleMaxTPB; // tokens per block (at most)
constexpr int kMaxBuckets = 4096;      // E * P

struct ShParams {
    int T, E, P, V, nb, tpb, nbk, log2_epg, bucket_bits, group_bits, k_max;
    const int32_t* row_ptr;
    const int32_t* slot;
    const int32_t* tok;
    const int32_t* lut;
    ShuffleOut o;
};

__global__ __launch_bounds__(kThreads) void k_hist(ShParams p)
{
    __shared__ int cnt[kMaxBuckets];
    __shared__ int tcnt[64];
    const int b = blockIdx.x;
    const int t0 = b * p.tpb, t1 = min(p.T, t0 + p.tpb);
    for (int i = threadIdx.x; i < p.nbk; i += kThreads) cnt[i] = 0;
    if (threadIdx.x < 64) tcnt[threadIdx.x] = 0;
    __syncthreads();
    for (int t = t0 + threadIdx.x; t < t1; t += kThreads) {
        const int v = checked_clamp(p.tok[t], 0, p.V - 1, p.o.err, MOE_DATA_TOKEN_ID);
        const int g = checked_clamp(p.lut[v], 0, p.P - 1, p.o.err, MOE_DATA_LUT);
        p.o.g_pred[t] = g;
        atomicAdd(&tcnt[g], 1);
        const int a0 = p.row_ptr[t], a1 = p.row_ptr[t + 1];
        // eight slot loads in flight before their counts are added (one
        // dependent load per atomic would serialise k_t memory latencies)
        for (int a = a0; a < a1; a += 8) {
            int s[8];
#pragma unroll
            for (int q = 0; q < 8; ++q) s[q] = a + q < a1 ? p.slot[a + q] : -1;
#pragma unroll
            for (int q = 0; q < 8; ++q)
                if (a + q < a1) atomicAdd(&cnt[checked_clamp(s[q], 0, p.E - 1, p.o.err, MOE_DATA_SLOT) * p.P + g], 1);
        }
    }
    __syncthreads();
    // block-major tables: block b's counts are one contiguous row
    for (int i = threadIdx.x; i < p.nbk; i += kThreads) p.o.hist[(size_t)b * p.nbk + i] = cnt[i];
    if (threadIdx.x < p.P) p.o.thist[(size_t)b * p.P + threadIdx.x] = tcnt[threadIdx.x];
}

// Columns of the count tables (buckets, then predicted groups) turned into
// exclusive offsets in place, with the column totals.  A block takes 64
// columns (one per lane: neighbouring lanes read neighbouring columns, so
// every access to a block row is coalesced) and splits the nb block rows
// between its sixteen waves: each wave sums its rows, the waves' sums are
// scanned through LDS, and each wave rewrites its rows as running offsets.
// Up to 256 block rows a wave's rows (at most 16) are read in one batch and
// kept in registers for the rewrite.
constexpr int kScanWaves = 16;
__global__ __launch_bounds__(64 * kScanWaves) void k_rowscan(ShParams p)
{
    __shared__ int s_part[kScanWaves][64];
    const int w = threadIdx.x >> 6, l = threadIdx.x & 63;
    const int col = blockIdx.x * 64 + l;
    const bool valid = col < p.nbk + p.P;
    const bool bucket = col < p.nbk;
    int32_t* a = bucket ? p.o.hist + col : p.o.thist + (col - p.nbk);
    const size_t stride = bucket ? (size_t)p.nbk : (size_t)p.P;
    const int per = (p.nb + kScanWaves - 1) / kScanWaves;
    const int r0 = min(p.nb, w * per), r1 = min(p.nb, r0 + per);
    constexpr int kHeld = 16;   // rows a wave keeps in registers between the passes
    int held[kHeld];
    int sum = 0;
    if (valid) {
        if (per <= kHeld) {
            // one batch of loads; the rewrite below reuses the values
#pragma unroll
            for (int q = 0; q < kHeld; ++q) held[q] = r0 + q < r1 ? a[(size_t)(r0 + q) * stride] : 0;
#pragma unroll
            for (int q = 0; q < kHeld; ++q) sum += held[q];
        } else {
            int r = r0;
            for (; r + 8 <= r1; r += 8) {
                int v[8];
#pragma unroll
                for (int q = 0; q < 8; ++q) v[q] = a[(size_t)(r + q) * stride];
#pragma unroll
                for (int q = 0; q < 8; ++q) sum += v[q];
            }
            for (; r < r1; ++r) sum += a[(size_t)r * stride];
        }
    }
    s_part[w][l] = sum;
    __syncthreads();
    int run = 0;
    for (int q = 0; q < w; ++q) run += s_part[q][l];
    if (valid) {
        if (per <= kHeld) {
#pragma unroll
            for (int q = 0; q < kHeld; ++q) {
                if (r0 + q < r1) a[(size_t)(r0 + q) * stride] = run;
                run += held[q];
            }
        } else {
            int r = r0;
            for (; r + 8 <= r1; r += 8) {
                int v[8];
#pragma unroll
                for (int q = 0; q < 8; ++q) v[q] = a[(size_t)(r + q) * stride];
#pragma unroll
                for (int q = 0; q < 8; ++q) {
                    a[(size_t)(r + q) * stride] = run;
                    run += v[q];
                }
            }
            for (; r < r1; ++r) {
                const int v = a[(size_t)r * stride];
                a[(size_t)r * stride] = run;
                run += v;
            }
        }
        if (w == kScanWaves - 1) p.o.rowtot[col] = run;
    }
}

// Bucket totals -> bucket starts in LDS (s_start[0..nbk], the last entry A)
// and predicted-group starts (s_tstart[0..P]); any block size, NT threads.
template <int NT>
MOE_DEV void bucket_starts(const ShParams& p, int* smem, int* s_start, int* s_tstart)
{
    constexpr int kPer = (kMaxBuckets + NT - 1) / NT;  // buckets per thread
    const int nbk = p.nbk, P = p.P;
    // the P group totals, one per lane of the first wave, loaded with the
    // bucket totals and scanned in a wave
    const int gv = threadIdx.x < P ? p.o.rowtot[nbk + threadIdx.x] : 0;
    int v[kPer], sum = 0;
#pragma unroll
    for (int q = 0; q < kPer; ++q) {
        const int k = threadIdx.x * kPer + q;
        v[q] = k < nbk ? p.o.rowtot[k] : 0;
        sum += v[q];
    }
    int A;
    int run = block_excl_scan(sum, smem, &A);
#pragma unroll
    for (int q = 0; q < kPer; ++q) {
        const int k = threadIdx.x * kPer + q;
        if (k < nbk) s_start[k] = run;
        run += v[q];
    }
    if (threadIdx.x < 64) {
        const int gi = wave_incl_scan(gv);
        if (threadIdx.x < P) s_tstart[threadIdx.x] = gi - gv;
        if (threadIdx.x == P - 1) s_tstart[P] = gi;
        if (threadIdx.x == 0) s_start[nbk] = A;
    }
    __syncthreads();
}

// The per-slot / per-group results, the pair matrix and the token offsets
// from the LDS starts; zeroes the grouped GEMMs' tile counters.  Called by
// every thread of one block; s_pair is LDS scratch of P*P ints.
template <int NT>
MOE_DEV void write_offsets(const ShParams& p, const int* s_start, const int* s_tstart, int* s_pair)
{
    if (p.o.gemm_ctr != nullptr && threadIdx.x < 16) p.o.gemm_ctr[threadIdx.x] = 0;
    const int E = p.E, P = p.P, epg = E / P;
    for (int i = threadIdx.x; i < P * P; i += NT) s_pair[i] = 0;
    for (int s = threadIdx.x; s <= E; s += NT) {
        const int off = s_start[s * P];
        p.o.expert_off[s] = off;
        if (s < E) p.o.expert_count[s] = s_start[(s + 1) * P] - off;
    }
    for (int g = threadIdx.x; g <= P; g += NT) {
        const int off = s_start[g * epg * P];
        p.o.group_off[g] = off;
        if (g < P) p.o.group_count[g] = s_start[(g + 1) * epg * P] - off;
        p.o.tok_off[g] = s_tstart[g];
    }
    __syncthreads();
    // pair_count[pg * P + g]: predicted group pg, expert group g.  Each
    // (pg, g) sums its epg bucket counts in `parts` interleaved pieces, one
    // thread per piece, four bucket reads in flight; the pieces are added
    // into LDS (at most `parts` adds per entry).
    const int parts = P * P >= NT ? 1 : NT / (P * P);
    for (int i = threadIdx.x; i < P * P * parts; i += NT) {
        const int pc = i / (P * P), pq = i % (P * P), pg = pq / P, g = pq % P;
        int sum = 0;
        int s = g * epg + pc;
        for (; s + 3 * parts < (g + 1) * epg; s += 4 * parts) {
            int c[4];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int b = (s + q * parts) * P + pg;
                c[q] = s_start[b + 1] - s_start[b];
            }
            sum += (c[0] + c[1]) + (c[2] + c[3]);
        }
        for (; s < (g + 1) * epg; s += parts) sum += s_start[s * P + pg + 1] - s_start[s * P + pg];
        atomicAdd(&s_pair[pq], sum);
    }
    __syncthreads();
    for (int i = threadIdx.x; i < P * P; i += NT) p.o.pair_count[i] = s_pair[i];
}

// Empty layers only (no scatter runs): the offsets of zero assignments.
__global__ __launch_bounds__(1024) void k_scan(ShParams p)
{
    __shared__ int smem[17];
    __shared__ int s_start[kMaxBuckets + 1];
    __shared__ int s_tstart[65];
    __shared__ int s_pair[64 * 64];
    bucket_starts<1024>(p, smem, s_start, s_tstart);
    write_offsets<1024>(p, s_start, s_tstart, s_pair);
}

__global__ __launch_bounds__(kThreads) void k_scatter(ShParams p)
{
    __shared__ int base[4][kMaxBuckets];
    __shared__ int tbase[4][64];
    __shared__ int s_rp[kMaxTPB + 1];
    const int b = blockIdx.x;
    const int w = threadIdx.x >> 6, l = threadIdx.x & 63;
    const int t0 = b * p.tpb, t1 = min(p.T, t0 + p.tpb);
    const int nt = t1 - t0;
    const int tpw = p.tpb / 4;   // tokens per wave
    const int tw0 = min(t1, t0 + w * tpw), tw1 = min(t1, t0 + (w + 1) * tpw);
    const int nbk = p.nbk, P = p.P;

    // bucket and predicted-group starts: every block scans the bucket totals
    // itself (E*P of them); the extra last block writes the offset tables
    __shared__ int s_smem[17];
    __shared__ int s_start[kMaxBuckets + 1];
    __shared__ int s_tstart[65];
    __shared__ int s_gp[kMaxTPB];   // predicted group of each of the block's tokens
    bucket_starts<kThreads>(p, s_smem, s_start, s_tstart);
    if (b == p.nb) {
        // the extra last block: the offset tables only (off the token
        // blocks' critical path)
        write_offsets<kThreads>(p, s_start, s_tstart, &base[0][0]);
        return;
    }
    for (int i = threadIdx.x; i < nbk; i += kThreads) {
#pragma unroll
        for (int q = 0; q < 4; ++q) base[q][i] = 0;
    }
    if (threadIdx.x < 64) {
#pragma unroll
        for (int q = 0; q < 4; ++q) tbase[q][threadIdx.x] = 0;
    }
    for (int i = threadIdx.x; i <= nt; i += kThreads) s_rp[i] = p.row_ptr[t0 + i];
    for (int i = threadIdx.x; i < nt; i += kThreads) s_gp[i] = p.o.g_pred[t0 + i];
    __syncthreads();
    // per-wave counts
    for (int t = tw0 + l; t < tw1; t += 64) {
        const int g = s_gp[t - t0];
        atomicAdd(&tbase[w][g], 1);
        const int a1 = s_rp[t - t0 + 1];
        for (int a = s_rp[t - t0]; a < a1; a += 8) {
            int s[8];
#pragma unroll
            for (int q = 0; q < 8; ++q) s[q] = a + q < a1 ? p.slot[a + q] : -1;
#pragma unroll
            for (int q = 0; q < 8; ++q)
                if (a + q < a1) atomicAdd(&base[w][clampi(s[q], 0, p.E - 1) * P + g], 1);
        }
    }
    __syncthreads();
    // counts -> starting positions: block offset + earlier waves' counts
    {
        // this block's row of the offset table, loaded before it is used
        constexpr int kPerB = (kMaxBuckets + kThreads - 1) / kThreads;
        int hv[kPerB];
#pragma unroll
        for (int q = 0; q < kPerB; ++q) {
            const int i = threadIdx.x + q * kThreads;
            hv[q] = i < nbk ? p.o.hist[(size_t)b * nbk + i] : 0;
        }
#pragma unroll
        for (int q = 0; q < kPerB; ++q) {
            const int i = threadIdx.x + q * kThreads;
            if (i < nbk) {
                int run = s_start[i] + hv[q];
#pragma unroll
                for (int wq = 0; wq < 4; ++wq) {
                    const int c = base[wq][i];
                    base[wq][i] = run;
                    run += c;
                }
            }
        }
    }
    if (threadIdx.x < P) {
        int run = s_tstart[threadIdx.x] + p.o.thist[(size_t)b * P + threadIdx.x];
        for (int q = 0; q < 4; ++q) {
            const int c = tbase[q][threadIdx.x];
            tbase[q][threadIdx.x] = run;
            run += c;
        }
    }
    __syncthreads();

    // assignments of this wave's tokens, 64 at a time, in assignment order
    const int a_begin = s_rp[tw0 - t0], a_end = s_rp[tw1 - t0];
    int nslot = a_begin + l < a_end ? p.slot[a_begin + l] : 0;   // next chunk's slot, loaded ahead
    for (int c0 = a_begin; c0 < a_end; c0 += 64) {
        const int a = c0 + l;
        const bool valid = a < a_end;
        const int myslot = nslot;
        if (c0 + 64 + l < a_end) nslot = p.slot[c0 + 64 + l];
        uint32_t bucket = 0;
        int t = 0;
        if (valid) {
            // token of assignment a: last i with s_rp[i] <= a, within this wave's tokens
            int lo = tw0 - t0, hi = tw1 - t0 - 1;
            while (lo < hi) {
                const int mid = (lo + hi + 1) >> 1;
                if (s_rp[mid] <= a) lo = mid; else hi = mid - 1;
            }
            t = t0 + lo;
            bucket = (uint32_t)(clampi(myslot, 0, p.E - 1) * P + s_gp[lo]);
        }
        const uint64_t act = __ballot(valid);
        const uint64_t peers = match_key(bucket, p.bucket_bits, act);
        if (valid) {
            const int rank = __popcll(peers & lanemask_lt());
            const int dest = base[w][bucket] + rank;
            p.o.s2a[dest] = a;
            p.o.a2s[a] = dest;
            if (p.o.row_tok) p.o.row_tok[dest] = t;
            // the highest lane of each bucket advances its running position
            if ((peers >> l) == 1ull) base[w][bucket] = dest + 1;
        }
    }
    // tokens of this wave in token order -> tok_perm
    for (int c0 = tw0; c0 < tw1; c0 += 64) {
        const int t = c0 + l;
        const bool valid = t < tw1;
        const uint32_t g = valid ? (uint32_t)s_gp[t - t0] : 0u;
        const uint64_t act = __ballot(valid);
        const uint64_t peers = match_key(g, p.group_bits, act);
        if (valid) {
            const int dest = tbase[w][g] + __popcll(peers & lanemask_lt());
            p.o.tok_perm[dest] = t;
            if ((peers >> l) == 1ull) tbase[w][g] = dest + 1;
        }
    }
}

// x_sorted[assign_to_sorted[a]] = x[t] for every assignment a of token t:
// each x row is read once and written k_t times.  One wave per token, 16-byte
// chunks.  The token's k_t destinations are read once, one per lane, and
// handed to the stores with readlane (an index load between two stores would
// wait for the earlier store: vector memory counters retire in order).
__global__ __launch_bounds__(kThreads) void k_gather(int T, int row_bytes,
                                                     const char* __restrict__ x,
                                                     const int32_t* __restrict__ row_ptr,
                                                     const int32_t* __restrict__ a2s,
                                                     char* __restrict__ xs)
{
    const int t = __builtin_amdgcn_readfirstlane(blockIdx.x * 4 + (threadIdx.x >> 6));
    const int l = threadIdx.x & 63;
    if (t >= T) return;
    const int nch = row_bytes >> 4;
    const int a0 = row_ptr[t], a1 = row_ptr[t + 1];
    const int kt = a1 - a0;
    const int my_s = l < kt ? a2s[a0 + l] : 0;
    const u32x4_t* src = (const u32x4_t*)(x + (size_t)t * row_bytes);
    for (int c = l; c < nch; c += 4 * 64) {
        u32x4_t v[4];
#pragma unroll
        for (int q = 0; q < 4; ++q)
            if (c + q * 64 < nch) v[q] = src[c + q * 64];
        for (int j = 0; j < kt; ++j) {
            const int s = __builtin_amdgcn_readlane(my_s, j);
            u32x4_t* dst = (u32x4_t*)(xs + (size_t)s * row_bytes);
#pragma unroll
            for (int q = 0; q < 4; ++q)
                if (c + q * 64 < nch) __builtin_nontemporal_store(v[q], &dst[c + q * 64]);
        }
    }
}

// row_tok[s] = token of assignment s2a[s] (binary search in row_ptr).
__global__ __launch_bounds__(kThreads) void k_row_tok(int T, int A_max,
                                                      const int32_t* __restrict__ row_ptr,
                                                      const int32_t* __restrict__ s2a,
                                                      int32_t* __restrict__ row_tok)
{
    const int s = blockIdx.x * kThreads + threadIdx.x;
    const int A = row_ptr[T];
    if (s >= A || s >= A_max) return;
    const int a = s2a[s];
    int lo = 0, hi = T - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (row_ptr[mid] <= a) lo = mid; else hi = mid - 1;
    }
    row_tok[s] = lo;
}

}  // namespace

hipError_t launch_shuffle(const moe_cfg& c, int nb, int tpb, const int32_t* row_ptr,
                          const int32_t* topk_slot, const int32_t* tok, const int32_t* lut,
                          const ShuffleOut& o, hipStream_t s)
{
    ShParams p;
    p.T = c.T;
    p.E = c.E;
    p.P = c.P;
    p.V = c.V;
    p.nb = nb;
    p.tpb = tpb;
    p.nbk = c.E * c.P;
    p.log2_epg = ilog2(c.E / c.P);
    p.bucket_bits = ilog2(p.nbk);
    p.group_bits = ilog2(c.P);
    p.k_max = c.k_max;
    p.row_ptr = row_ptr;
    p.slot = topk_slot;
    p.tok = tok;
    p.lut = lut;
    p.o = o;
    // the histogram kernel also runs for T == 0 so the table it writes is zero
    hipLaunchKernelGGL(k_hist, dim3(nb), dim3(kThreads), 0, s, p);
    hipLaunchKernelGGL(k_rowscan, dim3(ceil_div(p.nbk + c.P, 64)), dim3(64 * kScanWaves), 0, s, p);
    // one block per token block, plus one for the offset tables
    if (c.T > 0)
        hipLaunchKernelGGL(k_scatter, dim3(nb + 1), dim3(kThreads), 0, s, p);
    else
        hipLaunchKernelGGL(k_scan, dim3(1), dim3(1024), 0, s, p);
    return hipGetLastError();
}

hipError_t launch_gather(const moe_cfg& c, const void* x, const int32_t* row_ptr,
                         const int32_t* a2s, void* x_sorted, hipStream_t s)
{
    if (c.T == 0) return hipSuccess;
    const int esz = c.dtype == MOE_BF16 ? 2 : 4;
    hipLaunchKernelGGL(k_gather, dim3(ceil_div(c.T, 4)), dim3(kThreads), 0, s, c.T, c.H * esz,
                       (const char*)x, row_ptr, a2s, (char*)x_sorted);
    return hipGetLastError();
}

hipError_t launch_row_tok(const moe_cfg& c, const int32_t* row_ptr, const int32_t* s2a,
                          int32_t* row_tok, hipStream_t s)
{
    const int A_max = c.T * c.k_max;
    if (A_max == 0) return hipSuccess;
    hipLaunchKernelGGL(k_row_tok, dim3(ceil_div(A_max, kThreads)), dim3(kThreads), 0, s, c.T,
                       A_max, row_ptr, s2a, row_tok);
    return hipGetLastError();
}

}  // namespace moe
