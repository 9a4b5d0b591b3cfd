// Route: gate GEMM on MFMA, synthetic affinity bias, top-k selection and
// routing weights.  Up to 64 experts (and in fp32) one kernel does it all
// per 16-token tile; bf16 layers with more experts compute the gate in a
// tiled GEMM kernel (64 x 128 or 128 x 256 / 128 x 128 output tiles, K
// split into slices of partial logits) and the route kernel adds the slices
// and selects, 8 tokens per block.
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

// Maximum of a 32-bit value over the wave, returned to every lane (all 64
// lanes active): quad swaps and the half-row and row mirrors leave each
// row's maximum in all its lanes, then the four rows' are combined.
MOE_DEV uint32_t wave_max_u32(uint32_t v)
{
    v = max(v, dpp_u32<0xB1>(v));
    v = max(v, dpp_u32<0x4E>(v));
    v = max(v, dpp_u32<0x141>(v));
    v = max(v, dpp_u32<0x140>(v));
    return max(max(readlane_u32(v, 0), readlane_u32(v, 16)), max(readlane_u32(v, 32), readlane_u32(v, 48)));
}

// Tokens per route block: 16 (one MFMA row tile) when the kernel computes
// the gate itself (E <= 64), 8 when it only sums the tiled gate kernel's
// partial logits and selects (E > 64): one token per wave, twice the blocks.
constexpr int route_tokens(int ntw) { return ntw >= 2 ? 8 : 16; }
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
    const float* glog;  // [gS][T][E] partial logits of the tiled gate GEMM, or nullptr
    int gS;
    uint32_t* err;      // data-error word (debug builds), or nullptr
};

// CSR offsets: row_ptr[t] = sum of k over tokens < t (k_tok clamped to
// [0, k_max] so that A never exceeds T*k_max).
__global__ __launch_bounds__(1024) void k_row_ptr(int T, int k_max, int ragged,
                                                   const int32_t* __restrict__ k_tok,
                                                   int32_t* __restrict__ row_ptr, uint32_t* err)
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
            v[q] = t < T ? checked_clamp(k_tok[t], 0, k_max, err, MOE_DATA_K) : 0;
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

// ---------------------------------------------------------------------------
// Gate GEMM for large E (bf16): partial logits glog[s][t][e] = sum over the
// K slice s of x[t,k] * Wg[e,k], a 64-token x 128-expert tile per block.
// The fused route kernel reads all of Wg once per 16 tokens, which for E of
// 128 and more makes its L2 traffic T/16 * E*H*2 bytes; this tiling reads Wg
// once per 64 tokens and x once per 128 experts.  Both operands go to LDS by
// DMA (64-wide k-chunks, 128-byte rows XOR-swizzled c ^ (row & 7), three
// buffers: the chunk being read and the next two in flight, 72 KB, two
// blocks per CU); four waves
// take 16 tokens each against all 128 experts (8 MFMA 16x16x32 column tiles).
constexpr int kGT = 64, kGE = 128, kGNB = 3;
constexpr int kGRows = kGT + kGE;           // LDS rows per chunk
constexpr int kGChunkE = kGRows * 64;       // bf16 elements per chunk buffer
constexpr int kGNI = kGRows / 8 / 4;        // DMA instructions per wave per chunk

__global__ __launch_bounds__(256) void k_gate_logits(int T, int H, int E, int Kc, const uint16_t* x,
                                                      const uint16_t* Wg, float* __restrict__ glog)
{
    __shared__ __attribute__((aligned(16))) uint16_t s_g[kGNB * kGChunkE];
    const int tid = threadIdx.x;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6), l = tid & 63;
    const int t0 = blockIdx.x * kGT, e0 = blockIdx.y * kGE, ks = blockIdx.z;
    const int nch = Kc / 64;
    const __amdgpu_buffer_rsrc_t rx = __builtin_amdgcn_make_buffer_rsrc((void*)x, (short)0, T * H * 2, 0x00020000);
    const __amdgpu_buffer_rsrc_t rw = __builtin_amdgcn_make_buffer_rsrc((void*)Wg, (short)0, E * H * 2, 0x00020000);
    // DMA instruction q = w * kGNI + j covers LDS rows 8q..8q+7 (x rows first,
    // then Wg rows); lane l fills row 8q + (l >> 3) at slot l & 7, which
    // holds the row's global chunk (l & 7) ^ (row & 7).  Rows past T or E
    // repeat the last one.
    int doff[kGNI];
#pragma unroll
    for (int j = 0; j < kGNI; ++j) {
        const int q = w * kGNI + j;
        const int row = q * 8 + (l >> 3);
        const int chunk = (l & 7) ^ (row & 7);
        const int src = row < kGT ? min(t0 + row, T - 1) : min(e0 + row - kGT, E - 1);
        doff[j] = src * H * 2 + chunk * 16;
    }
    auto dma = [&](int c) {
        const int ko = (ks * Kc + c * 64) * 2;
        uint16_t* buf = s_g + (c % kGNB) * kGChunkE;
#pragma unroll
        for (int j = 0; j < kGNI; ++j) {
            const int q = w * kGNI + j;
            uint16_t* dst = buf + q * 8 * 64;
#if defined(__HIP_DEVICE_COMPILE__)  // the host pass cannot form LDS pointers
            if (q * 8 < kGT)
                __builtin_amdgcn_raw_ptr_buffer_load_lds(rx, MOE_LDS_PTR(dst), 16, doff[j], ko, 0, 0);
            else
                __builtin_amdgcn_raw_ptr_buffer_load_lds(rw, MOE_LDS_PTR(dst), 16, doff[j], ko, 0, 0);
#else
            (void)dst;
            (void)ko;
#endif
        }
    };
    // Fragments: lane (r = l & 15, kg = l >> 4) reads row r of its 16-row
    // block at chunks kg (first 32-wide half) and kg + 4 (second half).
    const int r = l & 15, kg = l >> 4;
    const uint32_t sbase = lds_addr(s_g);
    const uint32_t a_row = sbase + (w * 16 + r) * 128, b_row = sbase + (kGT + r) * 128;
    const uint32_t c0 = (uint32_t)((kg ^ (r & 7)) << 4), c1 = (uint32_t)(((kg + 4) ^ (r & 7)) << 4);
    f32x4_t acc[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    dma(0);
    if (nch > 1) dma(1);
    for (int c = 0; c < nch; ++c) {
        // this wave's DMA of chunk c has landed (chunk c+1's may be in flight;
        // a partial count is sound because only LDS DMA loads, which retire in
        // order among themselves, are issued in this loop)
        if (c + 1 < nch) wait_vmcnt<kGNI>(); else wait_vmcnt<0>();
        __builtin_amdgcn_s_barrier();  // chunk c visible; chunk c-1's buffer free
        if (c + 2 < nch) dma(c + 2);
        const uint32_t so = (uint32_t)((c % kGNB) * kGChunkE * 2);
        bf16x8_t a[2], b[16];
        a[0] = lds_read_b128<0>(a_row + so + c0);
        a[1] = lds_read_b128<0>(a_row + so + c1);
        static_for<0, 8>([&](auto it) {
            constexpr int i = it.value;
            b[2 * i] = lds_read_b128<i * 16 * 128>(b_row + so + c0);
            b[2 * i + 1] = lds_read_b128<i * 16 * 128>(b_row + so + c1);
        });
        frag_wait(a, b);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            acc[i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[0], b[2 * i], acc[i], 0, 0, 0);
            acc[i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[1], b[2 * i + 1], acc[i], 0, 0, 0);
        }
    }
    // D layout: lane l holds expert column (l & 15) of tile i, tokens 4*kg + v
    float* out = glog + (size_t)ks * T * E;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int e = e0 + i * 16 + r;
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            const int t = t0 + w * 16 + kg * 4 + v;
            if (t < T && e < E) out[(size_t)t * E + e] = acc[i][v];
        }
    }
}

// The same gate GEMM in 128-token x TE-expert tiles (TE = 128 or 256) for
// layers with enough tiles to fill the chip: per 64-wide k-chunk a block
// loads (128 + TE) rows for 128 * TE outputs, against 192 rows for 64 * 128
// above, which halves the bytes through the LDS DMA path (the bound of
// both) at TE = 256.  Eight waves as 2 (tokens) x 4 (experts), each owning
// a 64 x TE/4 block of 16x16 MFMA tiles; three chunk buffers (144 KB at
// TE = 256, one block per CU), the same row swizzle and DMA ordering.
constexpr int kBT = 128;

template <int TE>
__global__ __launch_bounds__(512) void k_gate_logits_wide(int T, int H, int E, int Kc, const uint16_t* x,
                                                          const uint16_t* Wg, float* __restrict__ glog)
{
    constexpr int kRows = kBT + TE;          // LDS rows per chunk
    constexpr int kChunkE = kRows * 64;      // bf16 elements per chunk buffer
    constexpr int kNI = kRows / 8 / 8;       // DMA instructions per wave per chunk
    constexpr int RM = 4, RN = TE / 64;      // 16x16 tiles per wave: 64 tokens x TE/4 experts
    __shared__ __attribute__((aligned(16))) uint16_t s_g[kGNB * kChunkE];
    const int tid = threadIdx.x;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6), l = tid & 63;
    const int wm = w >> 2, wn = w & 3;
    const int t0 = blockIdx.x * kBT, e0 = blockIdx.y * TE, ks = blockIdx.z;
    const int nch = Kc / 64;
    const __amdgpu_buffer_rsrc_t rx = __builtin_amdgcn_make_buffer_rsrc((void*)x, (short)0, T * H * 2, 0x00020000);
    const __amdgpu_buffer_rsrc_t rw = __builtin_amdgcn_make_buffer_rsrc((void*)Wg, (short)0, E * H * 2, 0x00020000);
    // DMA instruction q = w * kNI + j covers LDS rows 8q..8q+7 (x rows
    // first, then Wg rows); lane l fills row 8q + (l >> 3) at slot l & 7,
    // which holds the row's global chunk (l & 7) ^ (row & 7).  Rows past T
    // or E repeat the last one.
    int doff[kNI];
#pragma unroll
    for (int j = 0; j < kNI; ++j) {
        const int q = w * kNI + j;
        const int row = q * 8 + (l >> 3);
        const int chunk = (l & 7) ^ (row & 7);
        const int src = row < kBT ? min(t0 + row, T - 1) : min(e0 + row - kBT, E - 1);
        doff[j] = src * H * 2 + chunk * 16;
    }
    auto dma = [&](int c) {
        const int ko = (ks * Kc + c * 64) * 2;
        uint16_t* buf = s_g + (c % kGNB) * kChunkE;
#pragma unroll
        for (int j = 0; j < kNI; ++j) {
            const int q = w * kNI + j;
            uint16_t* dst = buf + q * 8 * 64;
#if defined(__HIP_DEVICE_COMPILE__)  // the host pass cannot form LDS pointers
            if (q * 8 < kBT)
                __builtin_amdgcn_raw_ptr_buffer_load_lds(rx, MOE_LDS_PTR(dst), 16, doff[j], ko, 0, 0);
            else
                __builtin_amdgcn_raw_ptr_buffer_load_lds(rw, MOE_LDS_PTR(dst), 16, doff[j], ko, 0, 0);
#else
            (void)dst;
            (void)ko;
#endif
        }
    };
    // Fragments: lane (r = l & 15, kg = l >> 4) reads row r of each 16-row
    // block at chunks kg (first 32-wide half) and kg + 4 (second half).
    const int r = l & 15, kg = l >> 4;
    const uint32_t sbase = lds_addr(s_g);
    const uint32_t a_row = sbase + (wm * 64 + r) * 128, b_row = sbase + (kBT + wn * (TE / 4) + r) * 128;
    const uint32_t c0 = (uint32_t)((kg ^ (r & 7)) << 4), c1 = (uint32_t)(((kg + 4) ^ (r & 7)) << 4);
    f32x4_t acc[RM][RN];
#pragma unroll
    for (int i = 0; i < RM; ++i)
#pragma unroll
        for (int j = 0; j < RN; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    dma(0);
    if (nch > 1) dma(1);
    for (int c = 0; c < nch; ++c) {
        // this wave's DMA of chunk c has landed (chunk c+1's may be in
        // flight; only LDS DMA loads are issued in this loop, and they retire
        // in order among themselves)
        if (c + 1 < nch) wait_vmcnt<kNI>(); else wait_vmcnt<0>();
        __builtin_amdgcn_s_barrier();  // chunk c visible; chunk c-1's buffer free
        if (c + 2 < nch) dma(c + 2);
        const uint32_t so = (uint32_t)((c % kGNB) * kChunkE * 2);
        bf16x8_t a[2 * RM], b[2 * RN];
        static_for<0, RM>([&](auto it) {
            constexpr int i = it.value;
            a[2 * i] = lds_read_b128<i * 16 * 128>(a_row + so + c0);
            a[2 * i + 1] = lds_read_b128<i * 16 * 128>(a_row + so + c1);
        });
        static_for<0, RN>([&](auto it) {
            constexpr int j = it.value;
            b[2 * j] = lds_read_b128<j * 16 * 128>(b_row + so + c0);
            b[2 * j + 1] = lds_read_b128<j * 16 * 128>(b_row + so + c1);
        });
        frag_wait(a, b);
#pragma unroll
        for (int i = 0; i < RM; ++i)
#pragma unroll
            for (int j = 0; j < RN; ++j) {
                acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[2 * i], b[2 * j], acc[i][j], 0, 0, 0);
                acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[2 * i + 1], b[2 * j + 1], acc[i][j], 0, 0, 0);
            }
    }
    // D layout: lane l holds expert column (l & 15) of tile (i, j), tokens 4*kg + v
    float* out = glog + (size_t)ks * T * E;
#pragma unroll
    for (int i = 0; i < RM; ++i)
#pragma unroll
        for (int j = 0; j < RN; ++j) {
            const int e = e0 + wn * (TE / 4) + j * 16 + r;
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int t = t0 + wm * 64 + i * 16 + kg * 4 + v;
                if (t < T && e < E) out[(size_t)t * E + e] = acc[i][j][v];
            }
        }
}

template <int NTW, bool BF16>
__global__ __launch_bounds__(kThreads) void k_route(RouteParams p)
{
    constexpr int EP = NTW * 64;  // experts padded to a multiple of 64
    constexpr int kBM = route_tokens(NTW);
    static_assert(kBM % kWaves == 0, "whole tokens per wave");
    __shared__ float s_log[kBM][EP + 4];
    __shared__ int s_s2o[EP];
    __shared__ int s_o2s[EP];
    __shared__ float s_key[kWaves][EP];
    constexpr int kSK = NTW >= kWaves ? 1 : kWaves / NTW;
    __shared__ float s_part[kSK > 1 ? kSK : 1][kBM][kSK > 1 ? EP : 1];

    const int tid = threadIdx.x;
    const int w = tid >> 6;
    const int l = tid & 63;
    const int t0 = blockIdx.x * kBM;
    const int T = p.T, H = p.H, E = p.E;

    __shared__ int s_rp[kBM], s_kt[kBM];
    // s_o2s starts at slot 0 everywhere, so that a slot_to_orig that is not
    // a permutation (clamped entries, duplicates) leaves no entry unset
    for (int s = tid; s < EP; s += kThreads) {
        s_s2o[s] = s < E ? checked_clamp(p.s2o[s], 0, E - 1, p.err, MOE_DATA_PLACEMENT) : s;
        s_o2s[s] = 0;
    }
    if (tid < kBM) {
        const int t = t0 + tid;
        if (p.ragged) {
            s_rp[tid] = t < T ? p.row_ptr[t] : 0;
        } else {  // fixed k: the CSR offsets are t * k, written by the token's block
            s_rp[tid] = t * p.k_max;
            if (t < T) p.row_ptr[t] = t * p.k_max;
            if (t == T - 1) p.row_ptr[T] = T * p.k_max;
        }
        s_kt[tid] = t >= T ? 0 : (p.ragged ? checked_clamp(p.k_tok[t], 0, p.k_max, p.err, MOE_DATA_K) : p.k_max);
    }
    // the affinity table is read before the GEMM so its latency overlaps it
    const bool do_bias = p.pref != nullptr && p.aff_bias != 0.0f && p.n_pref > 0;
    const int np = p.n_pref;
    int pre_o[4], pre_row[4];   // pre_row -1: no entry
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        pre_o[q] = 0;
        pre_row[q] = -1;
        const int idx = tid + q * kThreads;
        if (do_bias && idx < kBM * np) {
            const int row = idx / np, j = idx % np;
            const int t = t0 + row;
            if (t < T) {
                const int v = checked_clamp(p.tok[t], 0, p.V - 1, p.err, MOE_DATA_TOKEN_ID);
                pre_o[q] = p.pref[(size_t)v * np + j];
                pre_row[q] = row;
            }
        }
    }
    __syncthreads();
    for (int s = tid; s < E; s += kThreads) s_o2s[s_s2o[s]] = s;

    // ---------------- gate GEMM: logits[16 tokens][E] ----------------
    if (p.glog != nullptr) {
        // from the tiled gate GEMM: partial sums added in slice order, eight
        // loads in flight per lane (kPer elements, kQ slices of each)
        static_assert(kBM * EP % kThreads == 0, "whole elements per thread");
        constexpr int kPer = kBM * EP / kThreads;
        constexpr int kQ = kPer >= 8 ? 1 : 8 / kPer;
        const size_t sstride = (size_t)T * E;
        float sum[kPer];
        size_t off[kPer];
        bool in[kPer];
#pragma unroll
        for (int u = 0; u < kPer; ++u) {
            const int idx = tid + u * kThreads;
            const int row = idx / EP, col = idx % EP;
            const int t = t0 + row;
            in[u] = t < T && col < E;
            off[u] = in[u] ? (size_t)t * E + col : 0;
            sum[u] = in[u] ? p.glog[off[u]] : 0.0f;
        }
        for (int q0 = 1; q0 < p.gS; q0 += kQ) {
            float v[kPer][kQ];
#pragma unroll
            for (int u = 0; u < kPer; ++u)
#pragma unroll
                for (int q = 0; q < kQ; ++q)
                    v[u][q] = (in[u] && q0 + q < p.gS) ? p.glog[(size_t)(q0 + q) * sstride + off[u]] : 0.0f;
#pragma unroll
            for (int u = 0; u < kPer; ++u)
#pragma unroll
                for (int q = 0; q < kQ; ++q)
                    if (q0 + q < p.gS) sum[u] += v[u][q];
        }
#pragma unroll
        for (int u = 0; u < kPer; ++u) {
            const int idx = tid + u * kThreads;
            s_log[idx / EP][idx % EP] = sum[u];
        }
    } else if constexpr (BF16 && kBM == 16) {
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
        for (int q = 0; q < 4; ++q) {
            if (pre_row[q] >= 0) {
                if (pre_o[q] >= 0 && pre_o[q] < E) s_log[pre_row[q]][s_o2s[pre_o[q]]] += p.aff_bias;
                else data_error(p.err, MOE_DATA_PREF);
            }
        }
        for (int idx = tid + 4 * kThreads; idx < kBM * np; idx += kThreads) {
            const int row = idx / np, j = idx % np;
            const int t = t0 + row;
            if (t < T) {
                const int v = checked_clamp(p.tok[t], 0, p.V - 1, p.err, MOE_DATA_TOKEN_ID);
                const int o = p.pref[(size_t)v * np + j];
                if (o >= 0 && o < E) s_log[row][s_o2s[o]] += p.aff_bias;
                else data_error(p.err, MOE_DATA_PREF);
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
        const int kt = __builtin_amdgcn_readfirstlane(s_kt[row]);  // one token per wave
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
            // keys in original-id order, so that a routing group (a block of
            // gsize consecutive original ids) is a contiguous range
#pragma unroll
            for (int i = 0; i < NTW; ++i)
                if (ok[i]) s_key[w][oid[i]] = key[i];
            __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
            __builtin_amdgcn_wave_barrier();
            // Group scores: L lanes per group (L * n_rgroups <= 64, L a power
            // of two), each scanning m of its group's keys as (key, original
            // id) candidates.  Round j takes the group maximum over the
            // segment and its owner marks it taken: the rgroup_topn largest
            // keys in descending order, added in that order.
            const int G = p.n_rgroups;
            int G2 = 1;
            while (G2 < G) G2 <<= 1;
            const int L = 64 / G2;
            const int m = (gsize + L - 1) / L;
            const int g = l / L, sub = l % L;
            const int first = g * gsize + sub * m;
            const int mine = g < G ? max(0, min(m, gsize - sub * m)) : 0;  // keys this lane scans
            uint32_t taken = 0;
            float sc = 0.0f;
            for (int j = 0; j < p.rgroup_topn; ++j) {
                uint64_t b = 0ull;
                int be = 0;
#pragma unroll 4
                for (int e = 0; e < mine; ++e) {
                    if (!((taken >> e) & 1u)) {
                        const uint64_t c = ((uint64_t)ordered_key(s_key[w][first + e]) << 32) |
                                           (0xFFFFFFFFu - (uint32_t)(first + e));
                        if (c > b) {
                            b = c;
                            be = e;
                        }
                    }
                }
                const uint64_t gb = seg_max_u64(b, L);
                if (b == gb && b != 0ull) taken |= 1u << be;
                const float v = unordered_key((uint32_t)(gb >> 32));
                sc = j == 0 ? v : sc + v;
            }
            // topk_rgroups rounds of the wave maximum over the groups' ordered
            // scores, one candidate per group (its segment's first lane, so
            // lane order is group order): of equal scores the lowest lane,
            // the lower group id, wins; the winner drops out
            uint32_t gh = (g < G && sub == 0) ? ordered_key(sc) : 0u;
            uint64_t kept = 0;
            for (int j = 0; j < p.topk_rgroups; ++j) {
                const uint32_t mh = wave_max_u32(gh);
                const int win = __builtin_ctzll(__ballot(gh == mh));
                if (l == win) gh = 0u;
                kept |= 1ull << (win / L);
            }
#pragma unroll
            for (int i = 0; i < NTW; ++i) ok[i] = ok[i] && ((kept >> (oid[i] / gsize)) & 1ull);
        }

        // Candidates as one 64-bit key each: the ordered selection key above
        // the complement of the original id, so a plain maximum is the
        // (key desc, original id asc) winner; 0 marks no candidate (every
        // real key's upper half is nonzero).  Each lane sorts its NTW keys
        // descending; a round takes the wave maximum of the lanes' heads and
        // the lane holding it drops its head.  The maximum is found on the
        // upper (key) halves; the lower (id) halves are compared only when
        // several heads share the largest key.
        uint64_t pk[NTW];
#pragma unroll
        for (int i = 0; i < NTW; ++i)
            pk[i] = ok[i] ? ((uint64_t)ordered_key(key[i]) << 32) | (0xFFFFFFFFu - oid[i]) : 0ull;
#pragma unroll
        for (int a = 0; a < NTW; ++a)
#pragma unroll
            for (int b = NTW - 1; b > a; --b)
                if (pk[b] > pk[b - 1]) {
                    const uint64_t t = pk[b];
                    pk[b] = pk[b - 1];
                    pk[b - 1] = t;
                }
        uint64_t mine = 0;
        for (int j = 0; j < kt; ++j) {
            const uint32_t hh = (uint32_t)(pk[0] >> 32), hl = (uint32_t)pk[0];
            const uint32_t mh = wave_max_u32(hh);
            const uint64_t tied = __ballot(hh == mh);
            uint32_t ml;
            int win;
            if (__builtin_popcountll(tied) == 1) {
                win = __builtin_ctzll(tied);
                ml = readlane_u32(hl, win);
            } else {
                ml = wave_max_u32(hh == mh ? hl : 0u);
                win = __builtin_ctzll(__ballot(hh == mh && hl == ml));
            }
            if (l == win) {
#pragma unroll
                for (int i = 0; i + 1 < NTW; ++i) pk[i] = pk[i + 1];
                pk[NTW - 1] = 0ull;
            }
            if (l == j) mine = ((uint64_t)mh << 32) | ml;
        }
        if (kt == 0) continue;
        // (a round with no candidate left — k above the candidates, which
        // validation excludes — would yield 0: slot 0, as a guard)
        const uint32_t mo = 0xFFFFFFFFu - (uint32_t)mine;
        const uint32_t myslot = (l < kt && mine != 0ull && mo < (uint32_t)E) ? (uint32_t)s_o2s[mo] : 0u;

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
    const dim3 block(kThreads);
    const int ntw = ceil_div(p.E, 64);
    // bf16 layers with E > 64 take their logits from the tiled gate kernel
    if (BF16 && ntw >= 2 && p.glog == nullptr) return hipErrorInvalidValue;
    const dim3 grid(ceil_div(p.T, route_tokens(ntw)));
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

namespace {
// y[i] = the selection sigmoid of x[i] (cw_sigmoidf, the same code the route
// kernel runs), grid-stride.
__global__ __launch_bounds__(256) void k_sigmoid(const float* __restrict__ x, float* __restrict__ y, int64_t n)
{
    const int64_t stride = (int64_t)gridDim.x * 256;
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += stride) y[i] = cw_sigmoidf(x[i]);
}
}  // namespace

hipError_t launch_sigmoid(const float* x, float* y, int64_t n, hipStream_t s)
{
    if (n <= 0) return hipSuccess;
    const int64_t blocks = std::min<int64_t>((n + 255) / 256, 4096);
    hipLaunchKernelGGL(k_sigmoid, dim3((unsigned)blocks), dim3(256), 0, s, x, y, n);
    return hipGetLastError();
}

hipError_t launch_row_ptr(const moe_cfg& c, const int32_t* k_tok, int32_t* row_ptr, uint32_t* err,
                          hipStream_t s)
{
    // with a fixed k and T > 0 the route kernel writes row_ptr itself
    if (!c.ragged && c.T > 0) return hipSuccess;
    hipLaunchKernelGGL(k_row_ptr, dim3(1), dim3(1024), 0, s, c.T, c.k_max, c.ragged, k_tok, row_ptr, err);
    return hipGetLastError();
}

// bf16 layers with more than 64 experts: the route kernel's own MFMA gate is
// compiled for one 64-wide expert tile per lane set only (E <= 64); the tiled
// kernel clamps a partial 128-expert tile and writes only e < E.
bool gate_tiled(const moe_cfg& c) { return c.dtype == MOE_BF16 && c.E > 64; }

namespace {
// Expert width of the wide gate tiles (0: the 64 x 128 tiles), chosen when
// the layer has at least 32 wide tiles, so that a K split of at most eight
// fills the chip.
int gate_wide(const moe_cfg& c)
{
    const int te = c.E >= 256 ? 256 : 128;
    const long long tiles = (long long)ceil_div(c.T, kBT) * ceil_div(c.E, te);
    return tiles >= 32 ? te : 0;
}
}  // namespace

int gate_split(const moe_cfg& c)
{
    // K slices: enough blocks for the chip (256 CUs), each slice at least
    // four 64-wide chunks; the partial sums are added in slice order.
    const int te = gate_wide(c);
    const long long tiles = te ? (long long)ceil_div(c.T, kBT) * ceil_div(c.E, te)
                               : (long long)ceil_div(c.T, kGT) * ceil_div(c.E, kGE);
    const int nch = c.H / 64;
    int S = 1;
    while (tiles * S < 256 && nch % (2 * S) == 0 && nch / (2 * S) >= 4) S *= 2;
    return S;
}

hipError_t launch_route(const moe_cfg& c, const void* x, const void* Wg, const float* ebias,
                        const int32_t* slot_to_orig, const int32_t* tok, const int32_t* pref,
                        const int32_t* k_tok, int32_t* row_ptr, int32_t* topk_slot,
                        float* topk_w, float* logits, float* glog, uint32_t* err, hipStream_t s)
{
    if (c.T == 0) return hipSuccess;
    RouteParams p;
    p.err = err;
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
    p.glog = nullptr;
    p.gS = 1;
    if (gate_tiled(c)) {
        const int S = gate_split(c);
        const int te = gate_wide(c);
        if (te == 256)
            hipLaunchKernelGGL(k_gate_logits_wide<256>, dim3(ceil_div(c.T, kBT), ceil_div(c.E, 256), S), dim3(512),
                               0, s, c.T, c.H, c.E, c.H / S, (const uint16_t*)x, (const uint16_t*)Wg, glog);
        else if (te == 128)
            hipLaunchKernelGGL(k_gate_logits_wide<128>, dim3(ceil_div(c.T, kBT), ceil_div(c.E, 128), S), dim3(512),
                               0, s, c.T, c.H, c.E, c.H / S, (const uint16_t*)x, (const uint16_t*)Wg, glog);
        else
            hipLaunchKernelGGL(k_gate_logits, dim3(ceil_div(c.T, kGT), ceil_div(c.E, kGE), S), dim3(256), 0, s,
                               c.T, c.H, c.E, c.H / S, (const uint16_t*)x, (const uint16_t*)Wg, glog);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        p.glog = glog;
        p.gS = S;
    }
    return c.dtype == MOE_BF16 ? launch_route_t<true>(p, s) : launch_route_t<false>(p, s);
}

}  // namespace moe
