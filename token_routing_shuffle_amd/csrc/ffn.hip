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

constexpr int BM = 128, BK = 64;
constexpr int LDSK = BK;   // no padding: XOR-swizzled chunks
constexpr int kMaxSeg = 516;

struct GemmParams {
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
    int A_max;               // rows of the sorted row space (bounds of A, C)
};

MOE_DEV float silu(float g) { return g / (1.0f + expf(-g)); }

// SiLU for the bf16 path, whose result is rounded to bf16 right after:
// hardware exp2 and reciprocal (about 1 ulp each) are far inside that rounding.
MOE_DEV float silu_fast(float g)
{
    return g * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(g * -1.4426950408889634f));
}

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

// Two floats -> packed bf16 pair (v_cvt_pk_bf16_f32, round to nearest even).
MOE_DEV uint32_t pack2_bf16(float lo, float hi)
{
    const f32x2_t f = {lo, hi};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2_t));
}

#define MOE_LDS_PTR(p) ((void __attribute__((address_space(3)))*)(p))

// s_waitcnt vmcnt(N) (gfx9 encoding; expcnt and lgkmcnt left alone)
template <int N>
MOE_DEV void wait_vmcnt()
{
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

// LDS fragment read issued as inline asm: the compiler's wait-count pass then
// does not treat it as a read of the in-flight LDS DMA (it would drain all
// outstanding loads before it); completion is waited for explicitly with
// frag_wait, whose operands tie the fragments so no use moves above it.
// (The asm exists only in the device pass; the host pass never runs these.)
MOE_DEV bf16x8_t lds_read_b128(const uint16_t* p)
{
#if defined(__HIP_DEVICE_COMPILE__)
    const uint32_t a = (uint32_t)(uintptr_t)((__attribute__((address_space(3))) const uint16_t*)p);
    bf16x8_t v;
    asm volatile("ds_read_b128 %0, %1" : "=v"(v) : "v"(a));
    return v;
#else
    return *(const bf16x8_t*)p;
#endif
}

MOE_DEV void frag_wait(bf16x8_t (&a)[4], bf16x8_t (&b)[4])
{
#if defined(__HIP_DEVICE_COMPILE__)
    asm volatile("s_waitcnt lgkmcnt(0)"
                 : "+v"(a[0]), "+v"(a[1]), "+v"(a[2]), "+v"(a[3]), "+v"(b[0]), "+v"(b[1]),
                   "+v"(b[2]), "+v"(b[3]));
#else
    (void)a;
    (void)b;
#endif
}

// Tile BM x BN x BK, BN/32 waves in a 2 x (BN/64) grid, each wave owning a
// 64 x 64 block of the output (4 x 4 MFMA 16x16x32 tiles).  For the up
// projection the BN columns are BN/2 gate neurons followed by the same BN/2
// up neurons, and every wave holds matching gate and up columns so the SwiGLU
// product is formed in registers.
//
// Operands go HBM/L2 -> LDS directly (buffer_load_dwordx4 ... lds): no
// staging registers and no ds_write instructions.  LDS holds a ring of three
// stages of [A tile | B tile]; rows are 128 bytes (eight 16-byte chunks),
// XOR-swizzled (chunk c of row r at position c ^ (r & 7)), which keeps the
// MFMA fragment reads free of bank conflicts; the swizzle is applied on the
// global side, since each wave-wide LDS DMA writes 64 consecutive 16-byte
// slots.  Each k-step: wait for this wave's DMA of tile kt, barrier, issue
// the DMA of tile kt+2 into the stage read at step kt-1, compute tile kt.
template <bool UP, int BN>
__global__ __launch_bounds__(BN * 2, 1) void k_grouped_gemm(GemmParams p)
{
    constexpr int kThreads = BN * 2;        // BN/32 waves
    constexpr int NW = kThreads / 64;
    constexpr int WN = BN / 64;             // waves along N
    constexpr int NPT = BN / 2;             // up: neurons per tile
    constexpr int kRows = BM + BN;          // 128-byte rows per stage
    constexpr int kStageE = kRows * 64;     // bf16 elements per stage
    constexpr int NS = 3;                   // LDS stages
    constexpr int NI = kRows * 8 / 64 / NW; // DMA instructions per wave per stage
    static_assert(kRows * 8 == NI * 64 * NW, "stage split");
    static_assert(BM % 8 == 0, "a DMA instruction covers 8 rows of one operand");
    __shared__ __attribute__((aligned(16))) uint16_t smem[NS * kStageE];
    __shared__ int s_pref[kMaxSeg + 1];
    __shared__ int s_row0[kMaxSeg];
    __shared__ int s_cnt[kMaxSeg];
    __shared__ int s_smem[17];

    const int tid = threadIdx.x;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6), l = tid & 63;
    const int wm = w / WN, wn = w % WN;
    const int nseg = p.n_routed + p.has_shared;

    // ---- tile list prefix over segments
    {
        constexpr int SPT = (kMaxSeg + kThreads - 1) / kThreads;
        int tiles[SPT], sum = 0;
#pragma unroll
        for (int q = 0; q < SPT; ++q) {
            const int i = tid * SPT + q;
            tiles[q] = 0;
            if (i < nseg) {
                int row0, cnt, nt;
                if (i < p.n_routed) {
                    const int e = p.e_begin + i;
                    row0 = p.expert_off[e];
                    cnt = p.expert_off[e + 1] - row0;
                    nt = UP ? p.N / NPT : p.N / BN;
                } else {
                    row0 = 0;
                    cnt = p.T;
                    nt = UP ? p.shN / NPT : p.shN / BN;
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
        for (int q = 0; q < SPT; ++q) {
            const int i = tid * SPT + q;
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

    for (int L = L0 + j; L < L1; L += G8) {
        // ---- locate the tile
        int lo = 0, hi = nseg - 1;
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (s_pref[mid] <= L) lo = mid; else hi = mid - 1;
        }
        // tile values are wave-uniform: keep them in scalar registers
        const int seg = __builtin_amdgcn_readfirstlane(lo);
        const bool shared = seg >= p.n_routed;
        const int row0 = __builtin_amdgcn_readfirstlane(s_row0[seg]);
        const int cnt = __builtin_amdgcn_readfirstlane(s_cnt[seg]);
        const int mt = (cnt + BM - 1) / BM;
        const int local = L - __builtin_amdgcn_readfirstlane(s_pref[seg]);
        const int ntile = local / mt, m0 = (local % mt) * BM;
        const int K = shared ? p.shK : p.K;
        const int N = shared ? p.shN : p.N;
        const int rows = min(BM, cnt - m0);

        // ---- operands as buffer resources (base + bounds); per-lane 32-bit
        // row offsets; the k-step goes in the scalar offset.  Rows past the
        // segment end repeat its last row.
        const uint16_t* Abase;
        int a_bytes;
        if (shared) {
            Abase = p.shA;
            a_bytes = p.T * K * 2;
        } else if (p.A != nullptr) {
            Abase = p.A;
            a_bytes = p.A_max * K * 2;
        } else {
            Abase = p.X;
            a_bytes = p.T * K * 2;
        }
        const uint16_t* Bseg = shared ? p.shB : p.B + (size_t)(p.e_begin + seg) * (UP ? 2 * (size_t)N : (size_t)N) * K;
        const int b_bytes = (UP ? 2 * N : N) * K * 2;
        const __amdgpu_buffer_rsrc_t rsA = __builtin_amdgcn_make_buffer_rsrc((void*)Abase, (short)0, a_bytes, 0x00020000);
        const __amdgpu_buffer_rsrc_t rsB = __builtin_amdgcn_make_buffer_rsrc((void*)Bseg, (short)0, b_bytes, 0x00020000);
        // DMA instruction jj of this wave covers stage rows [8(w*NI+jj), +8);
        // lane l fills slot l: row 8(w*NI+jj) + l/8, position l%8, which holds
        // the row's global chunk (l%8) ^ (row & 7).
        int doff[NI];
#pragma unroll
        for (int jj = 0; jj < NI; ++jj) {
            const int row = (w * NI + jj) * 8 + (l >> 3);
            const int chunk = (l & 7) ^ (row & 7);
            if (row < BM) {
                const int gr = row0 + m0 + min(row, rows - 1);
                const int src_row = (!shared && p.A == nullptr) ? p.row_tok[gr] : gr;
                doff[jj] = src_row * K * 2 + chunk * 16;
            } else {
                const int r = row - BM;
                int brow;
                if (UP) {
                    const int n0 = ntile * NPT;
                    brow = r < NPT ? n0 + r : N + n0 + (r - NPT);
                } else {
                    brow = ntile * BN + r;
                }
                doff[jj] = brow * K * 2 + chunk * 16;
            }
        }
        auto dma = [&](int kt, int st) {
            const int ko = kt * BK * 2;
#pragma unroll
            for (int jj = 0; jj < NI; ++jj) {
                uint16_t* dst = smem + st * kStageE + (w * NI + jj) * 512;
#if defined(__HIP_DEVICE_COMPILE__)  // the host pass cannot form LDS pointers
                if ((w * NI + jj) * 8 < BM)
                    __builtin_amdgcn_raw_ptr_buffer_load_lds(rsA, MOE_LDS_PTR(dst), 16, doff[jj], ko, 0, 0);
                else
                    __builtin_amdgcn_raw_ptr_buffer_load_lds(rsB, MOE_LDS_PTR(dst), 16, doff[jj], ko, 0, 0);
#else
                (void)dst;
                (void)ko;
#endif
            }
        };

        f32x4_t acc[4][4];
#pragma unroll
        for (int a = 0; a < 4; ++a)
#pragma unroll
            for (int b = 0; b < 4; ++b) acc[a][b] = f32x4_t{0.f, 0.f, 0.f, 0.f};

        auto compute = [&](int st) {
            const uint16_t* As = smem + st * kStageE;
            const uint16_t* Bs = As + BM * BK;
            bf16x8_t af[2][4], bfr[2][4];
            auto read = [&](int kk) {
#pragma unroll
                for (int rt = 0; rt < 4; ++rt) {
                    const int row = wm * 64 + rt * 16 + (l & 15);
                    af[kk][rt] = lds_read_b128(&As[row * BK + ((((kk << 2) + (l >> 4)) ^ (row & 7)) << 3)]);
                }
#pragma unroll
                for (int ct = 0; ct < 4; ++ct) {
                    const int cb = UP ? ((ct < 2) ? wn * 32 + ct * 16 : NPT + wn * 32 + (ct - 2) * 16)
                                      : wn * 64 + ct * 16;
                    const int row = cb + (l & 15);
                    bfr[kk][ct] = lds_read_b128(&Bs[row * BK + ((((kk << 2) + (l >> 4)) ^ (row & 7)) << 3)]);
                }
            };
            auto mfma = [&](int kk) {
#pragma unroll
                for (int rt = 0; rt < 4; ++rt)
#pragma unroll
                    for (int ct = 0; ct < 4; ++ct)
                        acc[rt][ct] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bfr[kk][ct], af[kk][rt], acc[rt][ct], 0, 0, 0);
            };
            read(0);
            frag_wait(af[0], bfr[0]);
            read(1);             // overlaps the first half's MFMAs
            mfma(0);
            frag_wait(af[1], bfr[1]);
            mfma(1);
        };

        const int KT = K / BK;
        dma(0, 0);
        if (KT > 1) dma(1, 1);
        int st = 0;
        for (int kt = 0; kt < KT; ++kt) {
            // this wave's DMA of tile kt is done once at most the NI loads of
            // tile kt+1 are still outstanding
            if (kt + 1 < KT) wait_vmcnt<NI>(); else wait_vmcnt<0>();
            __builtin_amdgcn_s_barrier();
            if (kt + 2 < KT) dma(kt + 2, st == 0 ? 2 : st - 1);
            compute(st);
            st = st == 2 ? 0 : st + 1;
        }
        __syncthreads();

        // ---- epilogue.  The MFMAs compute the transposed tile (B rows as
        // the first operand), so lane l holds output row (l & 15) and four
        // consecutive output columns 4*(l >> 4) + v: packed into one 8-byte
        // LDS store, then written out as 16-byte row chunks.
        uint16_t* Cseg = shared ? p.shC : p.C;
        constexpr int CW = UP ? NPT : BN;  // output columns of the tile
        constexpr int CS = CW + 8;         // padded LDS row stride
        uint16_t* Cs = smem;
        if (UP) {
#pragma unroll
            for (int rt = 0; rt < 4; ++rt)
#pragma unroll
                for (int c = 0; c < 2; ++c) {
                    const int row = wm * 64 + rt * 16 + (l & 15);
                    const f32x4_t g = acc[rt][c], u = acc[rt][c + 2];
                    uint2 v;
                    v.x = pack2_bf16(silu_fast(g[0]) * u[0], silu_fast(g[1]) * u[1]);
                    v.y = pack2_bf16(silu_fast(g[2]) * u[2], silu_fast(g[3]) * u[3]);
                    *(uint2*)&Cs[row * CS + wn * 32 + c * 16 + (l >> 4) * 4] = v;
                }
        } else {
#pragma unroll
            for (int rt = 0; rt < 4; ++rt)
#pragma unroll
                for (int ct = 0; ct < 4; ++ct) {
                    const int row = wm * 64 + rt * 16 + (l & 15);
                    const f32x4_t a = acc[rt][ct];
                    uint2 v;
                    v.x = pack2_bf16(a[0], a[1]);
                    v.y = pack2_bf16(a[2], a[3]);
                    *(uint2*)&Cs[row * CS + wn * 64 + ct * 16 + (l >> 4) * 4] = v;
                }
        }
        __syncthreads();
        constexpr int CPR = CW / 8;        // 16-byte chunks per row
        const int n_out = UP ? ntile * NPT : ntile * BN;
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

template <bool UP, int BN>
hipError_t launch_gemm_t(const GemmParams& p, long long ub, hipStream_t s)
{
    // one resident block per CU (three LDS stages: 96 or 144 KB)
    long long grid = std::min<long long>(ub, (long long)num_cus());
    grid = (grid + 7) / 8 * 8;
    hipLaunchKernelGGL((k_grouped_gemm<UP, BN>), dim3((unsigned)grid), dim3(BN * 2), 0, s, p);
    return hipGetLastError();
}

hipError_t launch_gemm(const moe_cfg& c, const FfnArgs& a, bool up, hipStream_t s)
{
    GemmParams p;
    p.n_routed = a.n_routed;
    p.e_begin = a.e_begin;
    p.has_shared = a.sh_x != nullptr;
    p.T = c.T;
    p.A_max = a.A_max;
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
    // wide tiles (BN = 256) when every segment's N splits into them
    const int nw_r = up ? 2 * c.I : c.H;
    const int nw_s = up ? 2 * a.Ish : c.H;
    const bool wide = (a.n_routed == 0 || nw_r % 256 == 0) && (!p.has_shared || nw_s % 256 == 0);
    const int BN = wide ? 256 : 128;
    // host upper bound on the tile count (A is only known on the device)
    long long ub = 0;
    if (a.n_routed > 0) ub += ((long long)ceil_div(a.A_max, BM) + a.n_routed) * (nw_r / BN);
    if (p.has_shared) ub += (long long)ceil_div(c.T, BM) * (nw_s / BN);
    if (ub == 0) return hipSuccess;
    if (up)
        return wide ? launch_gemm_t<true, 256>(p, ub, s) : launch_gemm_t<true, 128>(p, ub, s);
    return wide ? launch_gemm_t<false, 256>(p, ub, s) : launch_gemm_t<false, 128>(p, ub, s);
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
