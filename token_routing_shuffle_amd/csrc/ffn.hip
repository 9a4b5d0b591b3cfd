// Expert FFN: grouped SwiGLU GEMMs on MFMA (bf16 in, fp32 accumulate).
//
// The experts are the usual SwiGLU FFNs of the named models (the pages do not
// give the expert form).  Rows of one slot are contiguous after the shuffle,
// so every expert is a plain GEMM over its row segment:
//   up:   h[r, n]  = silu(x_r . W1[n]) * (x_r . W3[n])        (GEMM1 + SwiGLU)
//   down: y[r, :]  = h_r . W2^T                               (GEMM2)
// Both are "NT" products: A rows and B rows are contiguous along K.
//
// One persistent kernel per GEMM walks a tile list covering the routed
// segments [e_begin, e_end) and (optionally) the shared experts over all T
// rows.  Tiles are ordered (segment, n-tile, m-tile) so the m-tiles that
// share a weight tile are adjacent, and the list is cut into 8 contiguous
// chunks, one per XCD (workgroup i runs on XCD i % 8), so weight tiles are
// reused from that XCD's L2.
//
// Tile 128 x 128 x 64, 256 threads (2 x 2 waves of 64 x 64), MFMA
// 16x16x32 bf16, LDS double buffer.  LDS rows are 64 bf16 (128 bytes, eight
// 16-byte chunks) stored with an XOR swizzle: chunk c of row r sits at chunk
// position c ^ (r & 7).  Measured on gfx950, both the loader's row-wise
// ds_write_b128 and the MFMA fragment ds_read_b128 (16 rows x one chunk) are
// then free of bank conflicts, unlike a padded row stride.
#include "common.h"
#include "internal.h"

namespace moe {
namespace {

constexpr int BM = 128, BN = 128, BK = 64;
constexpr int LDSK = BK;   // no padding: XOR-swizzled chunks
constexpr int kThreads = 256;
constexpr int kMaxSeg = 516;

struct GemmParams {
    int up;           // 1: GEMM1 + SwiGLU epilogue, 0: GEMM2
    int n_routed, e_begin, has_shared, T;
    const int32_t* expert_off;
    // routed operands
    const uint16_t* A;       // rows in sorted order (ld = K), or nullptr: gather x rows
    const uint16_t* X;       // [T, K] source of gathered rows (up only)
    const int32_t* row_tok;  // token of each sorted row (gather)
    const uint16_t* B;       // up: W13 [E, 2N, K]; down: W2 [E, N, K]
    uint16_t* C;             // up: h [A_max, N]; down: y [A_max, N]
    int K, N;                // up: K=H, N=I (neurons); down: K=I, N=H
    // shared operands (all T rows)
    const uint16_t* shA;     // up: x [T, H]; down: h_sh [T, Ish]
    const uint16_t* shB;     // up: Wsh13 [2*Ish, H]; down: Wsh2 [H, Ish]
    uint16_t* shC;           // up: h_sh [T, Ish]; down: y_sh [T, H]
    int shK, shN;
};

MOE_DEV float silu(float g) { return g / (1.0f + expf(-g)); }

template <bool UP>
__global__ __launch_bounds__(kThreads, 2) void k_grouped_gemm(GemmParams p)
{
    // LDS: two stages of [A tile | B tile] (XOR-swizzled 128-byte rows);
    // reused after the K loop to stage the output tile for 16-byte stores.
    constexpr int kStage = (BM + BN) * LDSK;
    __shared__ __attribute__((aligned(16))) uint16_t smem[2 * kStage];
    __shared__ int s_pref[kMaxSeg + 1];
    __shared__ int s_row0[kMaxSeg];
    __shared__ int s_cnt[kMaxSeg];
    __shared__ int s_smem[17];

    const int tid = threadIdx.x;
    const int w = tid >> 6, l = tid & 63;
    const int wm = w >> 1, wn = w & 1;
    const int nseg = p.n_routed + p.has_shared;

    // ---- tile list prefix over segments (3 segments per thread at most)
    {
        int tiles[3], sum = 0;
#pragma unroll
        for (int q = 0; q < 3; ++q) {
            const int i = tid * 3 + q;
            tiles[q] = 0;
            if (i < nseg) {
                int row0, cnt, nt;
                if (i < p.n_routed) {
                    const int e = p.e_begin + i;
                    row0 = p.expert_off[e];
                    cnt = p.expert_off[e + 1] - row0;
                    nt = UP ? p.N / 64 : p.N / BN;
                } else {
                    row0 = 0;
                    cnt = p.T;
                    nt = UP ? p.shN / 64 : p.shN / BN;
                }
                s_row0[i] = row0;
                s_cnt[i] = cnt;
                tiles[q] = ((cnt + BM - 1) / BM) * nt;
            }
            sum += tiles[q];
        }
        int total;
        int run = block_excl_scan(sum, s_smem, &total);
#pragma unroll
        for (int q = 0; q < 3; ++q) {
            const int i = tid * 3 + q;
            if (i < nseg) s_pref[i] = run;
            run += tiles[q];
        }
        if (tid == 0) s_pref[nseg] = total;
        __syncthreads();
    }
    const int total = s_pref[nseg];
    const int xcd = blockIdx.x & 7, G8 = gridDim.x >> 3, j = blockIdx.x >> 3;
    const int L0 = (int)(((long long)total * xcd) >> 3);
    const int L1 = (int)(((long long)total * (xcd + 1)) >> 3);

    const int lr = tid >> 3;        // loader row 0..31 (+32 q)
    const int lc = (tid & 7) * 8;   // loader k offset (elements)

    for (int L = L0 + j; L < L1; L += G8) {
        // ---- locate the tile
        int lo = 0, hi = nseg - 1;
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (s_pref[mid] <= L) lo = mid; else hi = mid - 1;
        }
        const int seg = lo;
        const bool shared = seg >= p.n_routed;
        const int row0 = s_row0[seg], cnt = s_cnt[seg];
        const int mt = (cnt + BM - 1) / BM;
        const int local = L - s_pref[seg];
        const int ntile = local / mt, m0 = (local % mt) * BM;
        const int K = shared ? p.shK : p.K;
        const int N = shared ? p.shN : p.N;
        const int rows = min(BM, cnt - m0);

        // ---- operand row pointers (rows past the segment end repeat its last row)
        const uint16_t* ap[4];
        const uint16_t* bp[4];
        const uint16_t* Bseg = shared ? p.shB : p.B + (size_t)(p.e_begin + seg) * (UP ? 2 * (size_t)N : (size_t)N) * K;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int r = lr + 32 * q;
            const int gr = row0 + m0 + min(r, rows - 1);
            const uint16_t* arow;
            if (shared)
                arow = p.shA + (size_t)gr * K;
            else if (p.A != nullptr)
                arow = p.A + (size_t)gr * K;
            else
                arow = p.X + (size_t)p.row_tok[gr] * K;
            ap[q] = arow + lc;
            int brow;
            if (UP) {
                const int n0 = ntile * 64;
                brow = r < 64 ? n0 + r : N + n0 + (r - 64);
            } else {
                brow = ntile * BN + r;
            }
            bp[q] = Bseg + (size_t)brow * K + lc;
        }

        f32x4_t acc[4][4];
#pragma unroll
        for (int a = 0; a < 4; ++a)
#pragma unroll
            for (int b = 0; b < 4; ++b) acc[a][b] = f32x4_t{0.f, 0.f, 0.f, 0.f};

        // global -> register stages, two k-tiles ahead of the MFMAs
        u32x4_t r0a[4], r0b[4], r1a[4], r1b[4];
        auto gload = [&](u32x4_t* ra, u32x4_t* rb, int kt) {
            const int ko = kt * BK;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                ra[q] = *(const u32x4_t*)(ap[q] + ko);
                rb[q] = *(const u32x4_t*)(bp[q] + ko);
            }
        };
        auto lstore = [&](const u32x4_t* ra, const u32x4_t* rb, int buf) {
            uint16_t* As = smem + buf * kStage;
            uint16_t* Bs = As + BM * LDSK;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int row = lr + 32 * q;
                const int pos = (((lc >> 3) ^ (row & 7)) << 3);
                *(u32x4_t*)&As[row * LDSK + pos] = ra[q];
                *(u32x4_t*)&Bs[row * LDSK + pos] = rb[q];
            }
        };
        auto compute = [&](int buf) {
            const uint16_t* As = smem + buf * kStage;
            const uint16_t* Bs = As + BM * LDSK;
#pragma unroll
            for (int kk = 0; kk < BK; kk += 32) {
                bf16x8_t af[4], bfr[4];
#pragma unroll
                for (int rt = 0; rt < 4; ++rt) {
                    const int row = wm * 64 + rt * 16 + (l & 15);
                    const int pos = ((((kk >> 3) + (l >> 4)) ^ (row & 7)) << 3);
                    af[rt] = *(const bf16x8_t*)&As[row * LDSK + pos];
                }
#pragma unroll
                for (int ct = 0; ct < 4; ++ct) {
                    const int cb = UP ? ((ct < 2) ? wn * 32 + ct * 16 : 64 + wn * 32 + (ct - 2) * 16)
                                      : wn * 64 + ct * 16;
                    const int row = cb + (l & 15);
                    const int pos = ((((kk >> 3) + (l >> 4)) ^ (row & 7)) << 3);
                    bfr[ct] = *(const bf16x8_t*)&Bs[row * LDSK + pos];
                }
#pragma unroll
                for (int rt = 0; rt < 4; ++rt)
#pragma unroll
                    for (int ct = 0; ct < 4; ++ct)
                        acc[rt][ct] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[rt], bfr[ct], acc[rt][ct], 0, 0, 0);
            }
        };

        const int KT = K / BK;
        gload(r0a, r0b, 0);
        lstore(r0a, r0b, 0);
        if (KT > 1) gload(r1a, r1b, 1);
        if (KT > 2) gload(r0a, r0b, 2);
        __syncthreads();
        // invariant at even kt: LDS buf 0 holds tile kt, r1 holds kt+1, r0 holds kt+2
        for (int kt = 0; kt < KT; kt += 2) {
            compute(0);
            if (kt + 1 < KT) lstore(r1a, r1b, 1);
            if (kt + 3 < KT) gload(r1a, r1b, kt + 3);
            __syncthreads();
            if (kt + 1 < KT) {
                compute(1);
                if (kt + 2 < KT) lstore(r0a, r0b, 0);
                if (kt + 4 < KT) gload(r0a, r0b, kt + 4);
                __syncthreads();
            }
        }

        // ---- epilogue: D lane layout: column (l & 15), rows 4*(l >> 4) + v.
        // Stage the bf16 tile in LDS, then write 16-byte row chunks.
        uint16_t* Cseg = shared ? p.shC : p.C;
        constexpr int CW = UP ? 64 : BN;   // output columns of the tile
        constexpr int CS = CW + 8;         // padded LDS row stride
        uint16_t* Cs = smem;
        if (UP) {
#pragma unroll
            for (int rt = 0; rt < 4; ++rt)
#pragma unroll
                for (int c = 0; c < 2; ++c)
#pragma unroll
                    for (int v = 0; v < 4; ++v) {
                        const int row = wm * 64 + rt * 16 + (l >> 4) * 4 + v;
                        const float g = acc[rt][c][v], u = acc[rt][c + 2][v];
                        Cs[row * CS + wn * 32 + c * 16 + (l & 15)] = (uint16_t)f2bf(silu(g) * u);
                    }
        } else {
#pragma unroll
            for (int rt = 0; rt < 4; ++rt)
#pragma unroll
                for (int ct = 0; ct < 4; ++ct)
#pragma unroll
                    for (int v = 0; v < 4; ++v) {
                        const int row = wm * 64 + rt * 16 + (l >> 4) * 4 + v;
                        Cs[row * CS + wn * 64 + ct * 16 + (l & 15)] = (uint16_t)f2bf(acc[rt][ct][v]);
                    }
        }
        __syncthreads();
        constexpr int CPR = CW / 8;        // 16-byte chunks per row
        const int n_out = UP ? ntile * 64 : ntile * BN;
#pragma unroll
        for (int q = 0; q < (BM * CPR) / kThreads; ++q) {
            const int idx = tid + q * kThreads;
            const int row = idx / CPR, ch = idx % CPR;
            if (row < rows)
                *(u32x4_t*)&Cseg[(size_t)(row0 + m0 + row) * N + n_out + ch * 8] =
                    *(const u32x4_t*)&Cs[row * CS + ch * 8];
        }
        __syncthreads();
    }
}

// ---------------------------------------------------------------------------
// fp32 path (small parity layers): one thread per output element, plain fma
// loops.  Routed rows r in [expert_off[e_begin], expert_off[e_end]) find
// their slot by binary search over expert_off.
struct F32Params {
    int up, shared, e_begin, e_end, rows_max;
    const int32_t* expert_off;
    const float* A;          // rows (ld = K) or nullptr: gather from X via row_tok
    const float* X;
    const int32_t* row_tok;
    const float* B;          // up: [E or 1, 2N, K]; down: [E or 1, N, K]
    float* C;                // [rows, N]
    int K, N;
};

__global__ __launch_bounds__(256) void k_ffn_f32(F32Params p)
{
    const long long gid = (long long)blockIdx.x * 256 + threadIdx.x;
    const int r = (int)(gid / p.N), n = (int)(gid % p.N);
    if (r >= p.rows_max) return;
    int e = 0;
    if (!p.shared) {
        const int lo_row = p.expert_off[p.e_begin], hi_row = p.expert_off[p.e_end];
        if (r < lo_row || r >= hi_row) return;
        int lo = p.e_begin, hi = p.e_end - 1;
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (p.expert_off[mid] <= r) lo = mid; else hi = mid - 1;
        }
        e = lo;
    }
    const float* a = p.A != nullptr ? p.A + (size_t)r * p.K : p.X + (size_t)p.row_tok[r] * p.K;
    if (p.up) {
        const float* w1 = p.B + ((size_t)e * 2 * p.N + n) * p.K;
        const float* w3 = p.B + ((size_t)e * 2 * p.N + p.N + n) * p.K;
        float g = 0.f, u = 0.f;
        for (int k = 0; k < p.K; ++k) {
            g = fmaf(a[k], w1[k], g);
            u = fmaf(a[k], w3[k], u);
        }
        p.C[(size_t)r * p.N + n] = silu(g) * u;
    } else {
        const float* w2 = p.B + ((size_t)e * p.N + n) * p.K;
        float y = 0.f;
        for (int k = 0; k < p.K; ++k) y = fmaf(a[k], w2[k], y);
        p.C[(size_t)r * p.N + n] = y;
    }
}

int num_cus()
{
    static int cached[64] = {0};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    if (cached[dev] == 0) {
        int v = 0;
        if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || v <= 0)
            v = 256;
        cached[dev] = v;
    }
    return cached[dev];
}

hipError_t launch_gemm(const moe_cfg& c, const FfnArgs& a, bool up, hipStream_t s)
{
    GemmParams p;
    p.up = up;
    p.n_routed = a.n_routed;
    p.e_begin = a.e_begin;
    p.has_shared = a.sh_x != nullptr;
    p.T = c.T;
    p.expert_off = a.expert_off;
    if (up) {
        p.A = (const uint16_t*)a.xs;
        p.X = (const uint16_t*)a.x;
        p.row_tok = a.row_tok;
        p.B = (const uint16_t*)a.W13;
        p.C = (uint16_t*)a.h;
        p.K = c.H;
        p.N = c.I;
        p.shA = (const uint16_t*)a.sh_x;
        p.shB = (const uint16_t*)a.sh_W13;
        p.shC = (uint16_t*)a.sh_h;
        p.shK = c.H;
        p.shN = a.Ish;
    } else {
        p.A = (const uint16_t*)a.h;
        p.X = nullptr;
        p.row_tok = nullptr;
        p.B = (const uint16_t*)a.W2;
        p.C = (uint16_t*)a.y;
        p.K = c.I;
        p.N = c.H;
        p.shA = (const uint16_t*)a.sh_h;
        p.shB = (const uint16_t*)a.sh_W2;
        p.shC = (uint16_t*)a.sh_y;
        p.shK = a.Ish;
        p.shN = c.H;
    }
    // host upper bound on the tile count (A is only known on the device)
    long long ub = 0;
    if (a.n_routed > 0) {
        const int nt = up ? c.I / 64 : c.H / BN;
        ub += ((long long)ceil_div(a.A_max, BM) + a.n_routed) * nt;
    }
    if (p.has_shared) {
        const int nt = up ? a.Ish / 64 : c.H / BN;
        ub += (long long)ceil_div(c.T, BM) * nt;
    }
    if (ub == 0) return hipSuccess;
    long long grid = std::min<long long>(ub, 2LL * num_cus());
    grid = (grid + 7) / 8 * 8;
    if (up)
        hipLaunchKernelGGL(k_grouped_gemm<true>, dim3((unsigned)grid), dim3(kThreads), 0, s, p);
    else
        hipLaunchKernelGGL(k_grouped_gemm<false>, dim3((unsigned)grid), dim3(kThreads), 0, s, p);
    return hipGetLastError();
}

hipError_t launch_f32(const moe_cfg& c, const FfnArgs& a, bool up, hipStream_t s)
{
    auto run = [&](const F32Params& p) {
        const long long n = (long long)p.rows_max * p.N;
        if (n == 0) return;
        hipLaunchKernelGGL(k_ffn_f32, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, p);
    };
    if (a.n_routed > 0) {
        F32Params p;
        p.up = up;
        p.shared = 0;
        p.e_begin = a.e_begin;
        p.e_end = a.e_begin + a.n_routed;
        p.rows_max = a.A_max;
        p.expert_off = a.expert_off;
        p.A = (const float*)(up ? a.xs : a.h);
        p.X = (const float*)a.x;
        p.row_tok = a.row_tok;
        p.B = (const float*)(up ? a.W13 : a.W2);
        p.C = (float*)(up ? a.h : a.y);
        p.K = up ? c.H : c.I;
        p.N = up ? c.I : c.H;
        run(p);
    }
    if (a.sh_x != nullptr) {
        F32Params p;
        p.up = up;
        p.shared = 1;
        p.e_begin = p.e_end = 0;
        p.rows_max = c.T;
        p.expert_off = nullptr;
        p.A = (const float*)(up ? a.sh_x : a.sh_h);
        p.X = nullptr;
        p.row_tok = nullptr;
        p.B = (const float*)(up ? a.sh_W13 : a.sh_W2);
        p.C = (float*)(up ? a.sh_h : a.sh_y);
        p.K = up ? c.H : a.Ish;
        p.N = up ? a.Ish : c.H;
        run(p);
    }
    return hipGetLastError();
}

}  // namespace

hipError_t launch_ffn_up(const moe_cfg& c, const FfnArgs& a, hipStream_t s)
{
    return c.dtype == MOE_BF16 ? launch_gemm(c, a, true, s) : launch_f32(c, a, true, s);
}

hipError_t launch_ffn_down(const moe_cfg& c, const FfnArgs& a, hipStream_t s)
{
    return c.dtype == MOE_BF16 ? launch_gemm(c, a, false, s) : launch_f32(c, a, false, s);
}

}  // namespace moe
