// Combine: weighted sum of each token's expert outputs back in the original
// token order (the Shuffled-Allgather's "restore the original order" step,
// German summary, technical summary §2B; Japanese summary, technical overview
// §2.2B), plus the shared-expert output.
//
// Gather-style and deterministic: each wave takes 64 16-byte chunks (1 KB)
// of one token's row, reads them from the token's k_t rows of y_sorted
// through assign_to_sorted, accumulates w * y in fp32 in j order, adds y_sh
// and writes them once.  No atomics.  A token's row is split over
// ceil(H / 512) waves (bf16) so that many small, independent waves keep the
// HBM busy.  The token's k_t indices and weights are read once, one per
// lane, and handed to the row loads with readlane: an index load between
// two row loads would make the second wait for the first (vector memory
// counters retire in order).
#include "common.h"
#include "internal.h"

namespace moe {
namespace {

constexpr int kThreads = 256;

template <bool BF16>
__global__ __launch_bounds__(kThreads) void k_combine(int T, int H, const void* __restrict__ ys,
                                                      const int32_t* __restrict__ a2s,
                                                      const int32_t* __restrict__ row_ptr,
                                                      const float* __restrict__ topk_w,
                                                      const void* __restrict__ ysh,
                                                      void* __restrict__ out)
{
    constexpr int EPC = BF16 ? 8 : 4;  // elements per 16-byte chunk
    const int nch = H / EPC;
    const int nq = (nch + 63) / 64;    // waves per token
    const int wid = __builtin_amdgcn_readfirstlane(blockIdx.x * 4 + (threadIdx.x >> 6));
    const int t = wid / nq;
    const int l = threadIdx.x & 63;
    if (t >= T) return;
    const int a0 = row_ptr[t], a1 = row_ptr[t + 1];
    const int c = (wid % nq) * 64 + l;
    // The token's sorted positions and weights, lane j holding assignment
    // a0 + j (k_t <= 64), loaded once: the row loads below then go out back
    // to back instead of each waiting for its own index load.
    const int kt = a1 - a0;
    int my_s = 0;
    float my_w = 0.0f;
    if (l < kt) {
        my_s = a2s[a0 + l];
        my_w = topk_w[a0 + l];
    }
    if (c >= nch) return;
    float acc[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) acc[q] = 0.0f;
    // rows of up to 16 assignments are loaded before they are summed, so
    // their memory latencies overlap; the sum stays in j order
    for (int j8 = 0; j8 < kt; j8 += 16) {
        u32x4_t v[16];
#pragma unroll
        for (int j = 0; j < 16; ++j) {
            if (j8 + j < kt) {
                const int s = __builtin_amdgcn_readlane(my_s, j8 + j);
                v[j] = __builtin_nontemporal_load(&((const u32x4_t*)ys)[(size_t)s * nch + c]);
            }
        }
#pragma unroll
        for (int j = 0; j < 16; ++j) {
            if (j8 + j < kt) {
                const float wt = __uint_as_float((uint32_t)__builtin_amdgcn_readlane((int)__float_as_uint(my_w), j8 + j));
                if constexpr (BF16) {
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        acc[2 * q] = fmaf(wt, bf2f(v[j][q] & 0xffffu), acc[2 * q]);
                        acc[2 * q + 1] = fmaf(wt, bf2f(v[j][q] >> 16), acc[2 * q + 1]);
                    }
                } else {
#pragma unroll
                    for (int q = 0; q < 4; ++q) acc[q] = fmaf(wt, __uint_as_float(v[j][q]), acc[q]);
                }
            }
        }
    }
    if (ysh != nullptr) {
        const u32x4_t v = __builtin_nontemporal_load(&((const u32x4_t*)ysh)[(size_t)t * nch + c]);
        if constexpr (BF16) {
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                acc[2 * q] += bf2f(v[q] & 0xffffu);
                acc[2 * q + 1] += bf2f(v[q] >> 16);
            }
        } else {
#pragma unroll
            for (int q = 0; q < 4; ++q) acc[q] += __uint_as_float(v[q]);
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
    __builtin_nontemporal_store(o, &((u32x4_t*)out)[(size_t)t * nch + c]);
}

}  // namespace

hipError_t launch_combine(const moe_cfg& c, const void* y_sorted, const int32_t* a2s,
                          const int32_t* row_ptr, const float* topk_w, const void* y_sh,
                          void* out, hipStream_t s)
{
    if (c.T == 0) return hipSuccess;
    const int nq = ceil_div(c.H / (c.dtype == MOE_BF16 ? 8 : 4), 64);
    const dim3 grid((unsigned)ceil_div(c.T * nq, 4)), block(kThreads);
    if (c.dtype == MOE_BF16)
        hipLaunchKernelGGL(k_combine<true>, grid, block, 0, s, c.T, c.H, y_sorted, a2s, row_ptr,
                           topk_w, y_sh, out);
    else
        hipLaunchKernelGGL(k_combine<false>, grid, block, 0, s, c.T, c.H, y_sorted, a2s, row_ptr,
                           topk_w, y_sh, out);
    return hipGetLastError();
}

}  // namespace moe
