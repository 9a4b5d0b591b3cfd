// One-GPU forms of the shuffled collectives around the MoE layer
// (Semantic Parallelism, German summary, technical summary §2B; Japanese
// summary, technical overview §2.2B):
//
//   SRS  shuffled reduce-scatter: the attention partials of the P
//        tensor-parallel ranks are summed and each rank receives the rows of
//        the tokens predicted to need its experts.  All partials on one
//        device: y[i] = sum_p x_part[p][tok_perm[i]], rank g's share being
//        rows [tok_off[g], tok_off[g+1]).
//   SAG  shuffled all-gather: the rows the ranks hold in tok_perm order are
//        gathered and restored to token order: out[tok_perm[i]] = y[i].
//
// Both are HBM-bound row moves: one wave per row, 16-byte lane accesses,
// the partial rows of a chunk (eight at a time, streaming loads and stores)
// loaded before they are summed (in p order, in fp32, rounded once to the
// output type).
#include "common.h"
#include "internal.h"

namespace moe {
namespace {

constexpr int kThreads = 256;   // 4 rows per block
constexpr int kBatch = 8;       // partial rows in flight per chunk

template <bool BF16>
__global__ __launch_bounds__(kThreads) void k_srs(int T, int H, int n_part,
                                                  const u32x4_t* __restrict__ x,
                                                  const int32_t* __restrict__ tok_perm,
                                                  u32x4_t* __restrict__ y)
{
    const int i = blockIdx.x * 4 + (threadIdx.x >> 6);
    const int l = threadIdx.x & 63;
    if (i >= T) return;
    constexpr int EPC = BF16 ? 8 : 4;  // elements per 16-byte chunk
    const int nch = H / EPC;
    const int t = tok_perm[i];
    const bool ok = (unsigned)t < (unsigned)T;
    const size_t part_stride = (size_t)T * nch;
    for (int c = l; c < nch; c += 64) {
        float acc[8];
#pragma unroll
        for (int q = 0; q < 8; ++q) acc[q] = 0.0f;
        for (int p0 = 0; ok && p0 < n_part; p0 += kBatch) {
            u32x4_t v[kBatch];
#pragma unroll
            for (int j = 0; j < kBatch; ++j)
                if (p0 + j < n_part) v[j] = __builtin_nontemporal_load(&x[(size_t)(p0 + j) * part_stride + (size_t)t * nch + c]);
#pragma unroll
            for (int j = 0; j < kBatch; ++j) {
                if (p0 + j < n_part) {
                    // the first partial initialises the sum, so one partial
                    // is an exact row permutation (signed zeros included)
                    const bool first = p0 + j == 0;
                    if constexpr (BF16) {
#pragma unroll
                        for (int q = 0; q < 4; ++q) {
                            const float lo = bf2f(v[j][q] & 0xffffu), hi = bf2f(v[j][q] >> 16);
                            acc[2 * q] = first ? lo : acc[2 * q] + lo;
                            acc[2 * q + 1] = first ? hi : acc[2 * q + 1] + hi;
                        }
                    } else {
#pragma unroll
                        for (int q = 0; q < 4; ++q) {
                            const float f = __uint_as_float(v[j][q]);
                            acc[q] = first ? f : acc[q] + f;
                        }
                    }
                }
            }
        }
        u32x4_t o;
        if constexpr (BF16) {
#pragma unroll
            for (int q = 0; q < 4; ++q) o[q] = pack_bf2(acc[2 * q], acc[2 * q + 1]);
        } else {
#pragma unroll
            for (int q = 0; q < 4; ++q) o[q] = __float_as_uint(acc[q]);
        }
        __builtin_nontemporal_store(o, &y[(size_t)i * nch + c]);
    }
}

__global__ __launch_bounds__(kThreads) void k_sag(int T, int nch, const u32x4_t* __restrict__ y,
                                                  const int32_t* __restrict__ tok_perm,
                                                  u32x4_t* __restrict__ out)
{
    const int i = blockIdx.x * 4 + (threadIdx.x >> 6);
    const int l = threadIdx.x & 63;
    if (i >= T) return;
    const int t = tok_perm[i];
    if ((unsigned)t >= (unsigned)T) return;
    const u32x4_t* src = y + (size_t)i * nch;
    u32x4_t* dst = out + (size_t)t * nch;
    int c = l;
    // four chunks in flight per lane
    for (; c + 192 < nch; c += 256) {
        const u32x4_t a = src[c], b = src[c + 64], d = src[c + 128], e = src[c + 192];
        dst[c] = a;
        dst[c + 64] = b;
        dst[c + 128] = d;
        dst[c + 192] = e;
    }
    for (; c < nch; c += 64) dst[c] = src[c];
}

}  // namespace

hipError_t launch_srs(const moe_cfg& c, int n_part, const void* x_part, const int32_t* tok_perm,
                      void* y, hipStream_t s)
{
    if (c.T == 0) return hipSuccess;
    const dim3 grid((unsigned)ceil_div(c.T, 4));
    if (c.dtype == MOE_BF16)
        hipLaunchKernelGGL(k_srs<true>, grid, dim3(kThreads), 0, s, c.T, c.H, n_part,
                           (const u32x4_t*)x_part, tok_perm, (u32x4_t*)y);
    else
        hipLaunchKernelGGL(k_srs<false>, grid, dim3(kThreads), 0, s, c.T, c.H, n_part,
                           (const u32x4_t*)x_part, tok_perm, (u32x4_t*)y);
    return hipGetLastError();
}

hipError_t launch_sag(const moe_cfg& c, const void* y, const int32_t* tok_perm, void* out,
                      hipStream_t s)
{
    if (c.T == 0) return hipSuccess;
    const int nch = c.H * (c.dtype == MOE_BF16 ? 2 : 4) / 16;
    hipLaunchKernelGGL(k_sag, dim3((unsigned)ceil_div(c.T, 4)), dim3(kThreads), 0, s, c.T, nch,
                       (const u32x4_t*)y, tok_perm, (u32x4_t*)out);
    return hipGetLastError();
}

}  // namespace moe
