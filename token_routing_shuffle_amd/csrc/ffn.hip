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
// rows.  Segments are grouped by the height of their m-tiles, tallest first,
// and inside a segment tiles are ordered (n-tile, m-tile), so the m-tiles that
// share a weight tile are adjacent.  Each height class is cut into 8 slices of
// equal work, one per XCD (workgroup i runs on XCD i % 8), so weight tiles are
// reused from that XCD's L2.  An XCD's workgroups claim the tiles of its
// slices from a counter, tallest class first, so the tiles left at the end are
// the shortest; once its slices are exhausted they claim from the other XCDs'.
//
// Tiles are 256 x 256, or 384 x 128 when N does not split into 256-wide
// tiles; a segment's m-tiles all have the height (a multiple of 32 rows, or
// of 64 for the 384-row tiles) that covers its rows in the fewest tiles, so
// little MFMA work is padding.  Eight waves: at 256 x 256 a 2 x 4 grid of
// 128 x 64 blocks per wave, 8 x 4 MFMA 16x16x32 bf16 blocks with 128 fp32
// accumulators per lane; at 384 x 128 a 4 x 2 grid of 96 x 64 blocks (96
// accumulators); two waves per SIMD.  The 256 x 256
// tile fetches 2/3 of the L2 bytes per flop of a 128 x 256 tile.
//
// Operands go HBM/L2 -> LDS directly (buffer_load_dwordx4 ... lds): no
// staging registers and no ds_write instructions.  LDS holds two stages of
// [A rows | B rows] with BK = 64: 128-byte rows (whole cache lines: with
// 64-byte row pieces the L2 delivers half the bytes per cycle, measured),
// eight 16-byte chunks per row, XOR-swizzled (see swz) so the fragment reads
// are free of bank conflicts.  The swizzle is applied on the global side, since
// each wave-wide LDS DMA writes 64 consecutive 16-byte slots.
//
// Pipeline per k-step (two MFMA k-halves of 32):
//   wait for this wave's DMA of step kt, barrier
//   read half 0's fragments, wait; read half 1's; MFMAs of half 0; wait
//   barrier (every wave has read stage kt & 1); DMA step kt+2 into it
//   MFMAs of half 1
// so a DMA has about one and a half k-steps to land and up to two stages
// (128 KB per CU) are in flight.  The partial wait (vmcnt(NI): the DMA of
// step kt+1 may still be in flight) relies on the LDS DMA loads retiring in
// order among themselves.  Loads into registers do not retire in order
// relative to them (measured: with such loads counted in the allowance, LDS
// reads ran ahead of the DMA now and then), so none is issued between a DMA
// and the wait that counts it; a gathered tile's row-index loads all come
// before its first DMA.
#include <atomic>

#include "common.h"
#include "internal.h"

namespace moe {
namespace {

constexpr int BM = 256, BK = 64, NS = 2;
// waves along N of the 256 x 256 tiles (the wave grid is 2 x kWavesN)
constexpr int kWavesN = 4;
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
    int blocked;             // B in the tile-blocked layout (moe_pack_weights)
    int* ctr;                // [8] tile counters, one per XCD, zero at launch
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

// Keeps two accumulator blocks in AGPRs up to this point of the program
// order.  Without it the compiler hoists the epilogue's reads of all 256
// accumulators into VGPRs at once and spills.
MOE_DEV void acc_fence(f32x4_t& a, f32x4_t& b)
{
#if defined(__HIP_DEVICE_COMPILE__)
    asm volatile("" : "+a"(a), "+a"(b)::"memory");
#else
    (void)a;
    (void)b;
#endif
}

// Position of 16-byte chunk c of LDS row r (128-byte rows, eight chunks):
// c ^ (r & 7).  Measured on gfx950, MFMA fragment reads (16 rows at one
// chunk, for either 32-wide k-half) are then free of bank conflicts.
MOE_DEV int swz(int r, int c) { return c ^ (r & 7); }

// SO: the layer's weights far exceed the caches, so weight tiles read once per
// call are streamed (see run_tile); without it the kernel is the same code
// with the default cache policy everywhere.
template <bool UP, int BN, int BMT, bool SO>
__global__ __launch_bounds__(512, 1) void k_grouped_gemm(GemmParams p)
{
    // tile rows at most: 256 (waves 2 x 4), or 384 with BN = 128 (waves 4 x 2)
    constexpr int BM = BMT;
    constexpr int kWN = BMT == 384 ? 2 : kWavesN;   // waves along N
    constexpr int kWM = 8 / kWN;                    // waves along M
    constexpr int kHq = kWM * 16;                   // tile height granularity
    constexpr int NW = kWM * kWN;            // waves
    constexpr int kThreads = 64 * NW;
    constexpr int WC = BN / (16 * kWN);      // 16-column blocks per wave
    constexpr int NPT = BN / 2;              // up: neurons per tile
    constexpr int kStageE = (BM + BN) * BK;  // bf16 elements per stage
    __shared__ __attribute__((aligned(16))) uint16_t smem[NS * kStageE];
    // segment lists in class-major order (position j holds segment s_seg[j])
    __shared__ int s_seg[kMaxSeg];
    __shared__ int s_pref[kMaxSeg + 1];   // tile index of each position's first tile
    __shared__ int s_wpref[kMaxSeg + 1];  // work before each position
    __shared__ int s_row0[kMaxSeg];
    __shared__ int s_cnt[kMaxSeg];
    __shared__ int s_smem[17];
    __shared__ int s_cls[5];         // first position of each class, then nseg
    __shared__ int s_bound[4 * 9];   // per class: slice start of each XCD, then its end
    __shared__ int s_tile;

    const int tid = threadIdx.x;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6), l = tid & 63;
    const int wm = w / kWN, wn = w % kWN;
    const int nseg = p.n_routed + p.has_shared;
    const int xcd = blockIdx.x & 7;

    // ---- tile list over segments.  A tile's work is its k-steps times a
    // weight of its height (tile_w).
    auto seg_geom = [&](int i, int& row0, int& cnt, int& nt, int& kt) {
        if (i < p.n_routed) {
            const int e = p.e_begin + i;
            row0 = p.expert_off[e];
            cnt = p.expert_off[e + 1] - row0;
            nt = UP ? p.N / NPT : p.N / BN;
            kt = p.K / BK;
        } else {
            row0 = 0;
            cnt = p.T;
            nt = UP ? p.shN / NPT : p.shN / BN;
            kt = p.shK / BK;
        }
    };
    // A segment of cnt rows is cut into mt = ceil(cnt / BM) m-tiles of
    // equal height (a multiple of kHq rows: 32, or 64 for the 384-row tiles):
    // the tiles that share a weight tile then run at the same speed, so the
    // second reader finds it in L2.
    auto mtile_h = [&](int cnt) {
        const int mt = (cnt + BM - 1) / BM;
        return ((cnt + mt - 1) / mt + kHq - 1) / kHq * kHq;
    };
    // Work of one k-step of an m-tile of height h, in units fitted to the
    // measured k-step times of 192- and 256-row tiles (about 0.8 : 1): the
    // MFMA work grows with h, the fixed part (barriers, B fragment reads,
    // DMA of the B rows) does not.
    auto tile_w = [&](int h) { return h / 16 + 6; };
    auto ntile_work = [&](int cnt, int kt) {
        const int mt = (cnt + BM - 1) / BM;
        return mt * tile_w(mtile_h(cnt)) * kt;
    };
    {
        constexpr int SPT = (kMaxSeg + kThreads - 1) / kThreads;
        // Segments in class-major order: class c holds the segments whose
        // m-tiles are BM - BM/4 * c high or a little less (256-row tiles:
        // 256 - 64c or 224 - 64c; empty segments go last), in segment order
        // inside a class.  Ranks inside a class come from two scans of 16-bit
        // counters packed in pairs.
        int cls[SPT], pk01 = 0, pk23 = 0;
#pragma unroll
        for (int q = 0; q < SPT; ++q) {
            const int i = tid * SPT + q;
            cls[q] = 3;
            if (i < nseg) {
                int row0, cnt, nt, kt;
                seg_geom(i, row0, cnt, nt, kt);
                if (cnt > 0) cls[q] = min(3, (BM - mtile_h(cnt)) / (BM / 4));
                if (cls[q] < 2) pk01 += 1 << (16 * cls[q]);
                else pk23 += 1 << (16 * (cls[q] - 2));
            }
        }
        int t01, t23;
        const int r01 = block_excl_scan(pk01, s_smem, &t01);
        const int r23 = block_excl_scan(pk23, s_smem, &t23);
        const int n0 = t01 & 0xFFFF, n1 = t01 >> 16, n2 = t23 & 0xFFFF;
        int rk0 = r01 & 0xFFFF, rk1 = r01 >> 16, rk2 = (r23 & 0xFFFF) + n0 + n1, rk3 = (r23 >> 16) + n0 + n1 + n2;
        rk1 += n0;
#pragma unroll
        for (int q = 0; q < SPT; ++q) {
            const int i = tid * SPT + q;
            if (i < nseg) {
                const int c = cls[q];
                s_seg[c == 0 ? rk0 : c == 1 ? rk1 : c == 2 ? rk2 : rk3] = i;
                rk0 += c == 0;
                rk1 += c == 1;
                rk2 += c == 2;
                rk3 += c == 3;
            }
        }
        if (tid == 0) {
            s_cls[0] = 0;
            s_cls[1] = n0;
            s_cls[2] = n0 + n1;
            s_cls[3] = n0 + n1 + n2;
            s_cls[4] = nseg;
        }
        __syncthreads();
        // tile and work prefix sums over that order (position j holds
        // segment s_seg[j])
        int tiles[SPT], work[SPT], tsum = 0, wsum = 0;
#pragma unroll
        for (int q = 0; q < SPT; ++q) {
            const int j = tid * SPT + q;
            tiles[q] = 0;
            work[q] = 0;
            if (j < nseg) {
                int row0, cnt, nt, kt;
                seg_geom(s_seg[j], row0, cnt, nt, kt);
                s_row0[j] = row0;
                s_cnt[j] = cnt;
                tiles[q] = ((cnt + BM - 1) / BM) * nt;
                work[q] = cnt > 0 ? nt * ntile_work(cnt, kt) : 0;
            }
            tsum += tiles[q];
            wsum += work[q];
        }
        int ttot, wtot;
        int trun = block_excl_scan(tsum, s_smem, &ttot);
        int wrun = block_excl_scan(wsum, s_smem, &wtot);
#pragma unroll
        for (int q = 0; q < SPT; ++q) {
            const int j = tid * SPT + q;
            if (j < nseg) {
                s_pref[j] = trun;
                s_wpref[j] = wrun;
            }
            trun += tiles[q];
            wrun += work[q];
        }
        if (tid == 0) {
            s_pref[nseg] = ttot;
            s_wpref[nseg] = wtot;
        }
        __syncthreads();
        // Each class's tiles are cut into eight slices of equal work, one per
        // XCD: XCD x owns the class-c tiles whose work starts in
        // [W * x / 8, W * (x + 1) / 8) of that class's work W.  Workgroup i
        // runs on XCD i % 8; the XCD's workgroups take tiles from its counter,
        // through its slices of classes 0, 1, 2, 3 in turn (tiles differ in
        // length, so a static split would leave some workgroups idle at the
        // end, and with the tallest tiles first the last ones claimed are the
        // shortest).  A workgroup whose XCD has run out continues on the
        // next XCDs' counters.
        if (tid < 36) {
            const int c = tid / 9, x = tid % 9;
            const int ps = s_cls[c], pe = s_cls[c + 1];
            const int w0 = s_wpref[ps], w1 = s_wpref[pe];
            const long long target = w0 + (((long long)(w1 - w0) * x) >> 3);
            int b = s_pref[pe];
            if (target < w1) {
                int lo = ps, hi = pe - 1;
                while (lo < hi) {
                    const int mid = (lo + hi + 1) >> 1;
                    if (s_wpref[mid] <= target) lo = mid; else hi = mid - 1;
                }
                int row0, cnt, nt, kt;
                seg_geom(s_seg[lo], row0, cnt, nt, kt);
                const int mt = (cnt + BM - 1) / BM;
                const int wn_ = ntile_work(cnt, kt);
                const int rem = (int)(target - s_wpref[lo]);
                const int n = rem / wn_;
                const int m = min((rem % wn_) / (tile_w(mtile_h(cnt)) * kt), mt - 1);
                b = s_pref[lo] + n * mt + m;
            }
            s_bound[tid] = b;
        }
        __syncthreads();
    }
    // tile claims (thread 0): the tile for counter value v of XCD
    // (xcd + src) & 7, through its four class slices; else the next XCDs';
    // -1 when all are done
    int src = 0;
    auto claim = [&]() -> int {
        for (;;) {
            const int y = (xcd + src) & 7;
            int v = atomicAdd(&p.ctr[y], 1);
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                const int b0 = s_bound[c * 9 + y], len = s_bound[c * 9 + y + 1] - b0;
                if (v < len) return b0 + v;
                v -= len;
            }
            if (++src == 8) return -1;
        }
    };

    for (;;) {
        if (tid == 0) s_tile = claim();
        __syncthreads();
        const int L = __builtin_amdgcn_readfirstlane(s_tile);
        if (L < 0) break;
        // ---- locate the tile
        int lo = 0, hi = nseg - 1;
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (s_pref[mid] <= L) lo = mid; else hi = mid - 1;
        }
        // tile values are wave-uniform: keep them in scalar registers
        const int pos = __builtin_amdgcn_readfirstlane(lo);
        const int seg = __builtin_amdgcn_readfirstlane(s_seg[pos]);
        const bool shared = seg >= p.n_routed;
        const int row0 = __builtin_amdgcn_readfirstlane(s_row0[pos]);
        const int cnt = __builtin_amdgcn_readfirstlane(s_cnt[pos]);
        const int mt = (cnt + BM - 1) / BM;
        const int local = L - __builtin_amdgcn_readfirstlane(s_pref[pos]);
        const int hgt = mtile_h(cnt);
        const int ntile = local / mt, m0 = (local % mt) * hgt;
        const int K = shared ? p.shK : p.K;
        const int N = shared ? p.shN : p.N;
        const int rows = min(hgt, cnt - m0);

        // ---- operands as buffer resources (base + bounds); per-lane 32-bit
        // row offsets; the k-step goes in the scalar offset.  Rows past the
        // segment end repeat its last row.  A rows held in sorted order are
        // addressed from the tile's first row (64-bit base), so only a tile's
        // rows, not the whole sorted row space, must fit the 32-bit offsets;
        // gathered rows are addressed from the start of x [T, K].
        const bool gath = !shared && p.A == nullptr;
        const uint16_t* Abase;
        long long a_bytes;
        if (gath) {
            Abase = p.X;
            a_bytes = (long long)p.T * K * 2;
        } else {
            Abase = (shared ? p.shA : p.A) + (size_t)(row0 + m0) * K;
            a_bytes = (long long)rows * K * 2;
        }
        const uint16_t* Bseg = shared ? p.shB : p.B + (size_t)(p.e_begin + seg) * (UP ? 2 * (size_t)N : (size_t)N) * K;
        const long long b_bytes = (long long)(UP ? 2 * N : N) * K * 2;
        const __amdgpu_buffer_rsrc_t rsA = __builtin_amdgcn_make_buffer_rsrc((void*)Abase, (short)0, (int)a_bytes, 0x00020000);
        const __amdgpu_buffer_rsrc_t rsB = __builtin_amdgcn_make_buffer_rsrc((void*)Bseg, (short)0, (int)b_bytes, 0x00020000);
        const int KT = K / BK;

        // RT = 16-row blocks per wave: the tile has 32 * RT rows (RT = 1..8),
        // split between the two wave rows.  The DMA loads the A rows in
        // groups of 64 (kAload), so for odd RT the last 32 rows loaded are
        // not used by the MFMAs.
        // STB: the weight tiles are streamed (non-temporal loads).  Chosen for
        // a segment of one m-tile, which reads each of its weight tiles once,
        // when the layer's weights far exceed the caches (SO): such a tile is
        // gone from the Infinity Cache by the next call, and caching it only
        // evicts the activation rows and intermediates that are reused.
        auto run_tile = [&](auto rt_tag, auto stb_tag) {
            constexpr bool STB = decltype(stb_tag)::value != 0;
            constexpr int RT = decltype(rt_tag)::value;
            constexpr int kArows = RT * kHq;                 // A rows of the tile
            constexpr int kAload = (kArows + 63) / 64 * 64;  // A rows loaded
            constexpr int NA = kAload / 8;                   // A DMA instructions
            constexpr int NI = (kAload + BN) / 8 / NW;       // DMA instructions per wave
            static_assert((kAload + BN) % 64 == 0, "stage split");
            // DMA instruction q = w*NI + jj covers 8 LDS rows; lane l fills
            // row (l >> 3) of them at position l & 7, which holds the row's
            // global chunk swz(row, l & 7) (the swizzle is an involution).
            // The lane id is laundered through an empty asm so that the
            // per-lane address arithmetic below stays inside the tile loop:
            // hoisted out of it, its tile-invariant parts would occupy
            // registers across the whole k-loop.
            int lane = l;
            asm volatile("" : "+v"(lane));
            int doff[NI];
#pragma unroll
            for (int jj = 0; jj < NI; ++jj) {
                const int q = w * NI + jj;
                const int rin = lane >> 3;
                const int chunk = swz(rin, lane & 7);
                if (q < NA) {
                    const int row = q * 8 + rin;
                    const int tr = min(row, rows - 1);
                    const int src_row = gath ? p.row_tok[row0 + m0 + tr] : tr;
                    doff[jj] = src_row * K * 2 + chunk * 16;
                } else {
                    const int r = (q - NA) * 8 + rin;
                    int brow;
                    if (UP) {
                        const int n0 = ntile * NPT;
                        brow = r < NPT ? n0 + r : N + n0 + (r - NPT);
                    } else {
                        brow = ntile * BN + r;
                    }
                    // blocked: row r of the n-tile's contiguous [BN][64] block
                    doff[jj] = p.blocked ? (ntile * KT * BN + r) * 128 + chunk * 16 : brow * K * 2 + chunk * 16;
                }
            }
            auto dma = [&](int kt, int st) {
                const int ko = kt * BK * 2;
                const int kob = p.blocked ? kt * BN * 128 : ko;  // B: next block, or next 128 bytes of each row
#pragma unroll
                for (int jj = 0; jj < NI; ++jj) {
                    const int q = w * NI + jj;
                    uint16_t* dst = smem + st * kStageE + (q < NA ? q * 8 : BM + (q - NA) * 8) * BK;
#if defined(__HIP_DEVICE_COMPILE__)  // the host pass cannot form LDS pointers
                    if (q < NA)
                        __builtin_amdgcn_raw_ptr_buffer_load_lds(rsA, MOE_LDS_PTR(dst), 16, doff[jj], ko, 0, 0);
                    else
                        __builtin_amdgcn_raw_ptr_buffer_load_lds(rsB, MOE_LDS_PTR(dst), 16, doff[jj], kob, 0,
                                                                 STB ? 2 : 0);  // 2: non-temporal
#else
                    (void)dst;
                    (void)ko;
                    (void)kob;
#endif
                }
            };

            f32x4_t acc[RT][WC];
#pragma unroll
            for (int a = 0; a < RT; ++a)
#pragma unroll
                for (int b = 0; b < WC; ++b) acc[a][b] = f32x4_t{0.f, 0.f, 0.f, 0.f};

            // Fragments of the two 32-wide k-halves of a stage.  Fragment rows
            // are 16-row aligned, so the swizzled position depends on the lane
            // only: one lane base per operand and k-half plus immediates.
            bf16x8_t af0[RT], bf0[WC], af1[RT], bf1[WC];
            const int lrow = lane & 15;
            const uint32_t a_row = lds_addr(smem) + (wm * (RT * 16) + lrow) * (BK * 2);
            const uint32_t b_row = lds_addr(smem) + (BM + wn * (UP ? NPT / kWN : BN / kWN) + lrow) * (BK * 2);
            const uint32_t c0 = swz(lrow, lane >> 4) << 4, c1 = swz(lrow, 4 + (lane >> 4)) << 4;
            const uint32_t a_base[2] = {a_row + c0, a_row + c1};
            const uint32_t b_base[2] = {b_row + c0, b_row + c1};
            auto read = [&](int st, auto half, bf16x8_t (&af)[RT], bf16x8_t (&bfr)[WC]) {
                constexpr int h = decltype(half)::value;
                const uint32_t so = st * (kStageE * 2);
                const uint32_t ab = a_base[h] + so, bb = b_base[h] + so;
                static_for<0, RT>([&](auto rt) {
                    af[rt.value] = lds_read_b128<rt.value * 16 * (BK * 2)>(ab);
                });
                static_for<0, WC>([&](auto ct) {
                    constexpr int c = ct.value;
                    constexpr int cb = UP ? (c < WC / 2 ? c * 16 : NPT + (c - WC / 2) * 16) : c * 16;
                    bfr[c] = lds_read_b128<cb * (BK * 2)>(bb);
                });
            };
            auto mfma = [&](bf16x8_t (&af)[RT], bf16x8_t (&bfr)[WC]) {
#pragma unroll
                for (int rt = 0; rt < RT; ++rt)
#pragma unroll
                    for (int ct = 0; ct < WC; ++ct)
                        acc[rt][ct] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bfr[ct], af[rt], acc[rt][ct], 0, 0, 0);
            };

            // Two LDS stages of BK = 64.  Step kt: wait for this wave's DMA of
            // step kt (at most the DMA of step kt+1 still in flight), barrier;
            // read the first k-half's fragments, wait, read the second half's
            // while the first half's MFMAs run, wait; barrier (every wave has
            // read stage kt & 1); DMA step kt+2 into it; second half's MFMAs.
            // A DMA thus has about one and a half k-steps to land, and up to
            // two stages are in flight.
            dma(0, 0);
            if (KT > 1) dma(1, 1);
            for (int kt = 0; kt < KT; ++kt) {
                const int st = kt & 1;
                if (kt + 1 < KT) wait_vmcnt<NI>(); else wait_vmcnt<0>();
                __builtin_amdgcn_s_barrier();
                read(st, IntC<0>{}, af0, bf0);
                frag_wait(af0, bf0);
                read(st, IntC<1>{}, af1, bf1);
                mfma(af0, bf0);
                frag_wait(af1, bf1);
                __builtin_amdgcn_s_barrier();
                if (kt + 2 < KT) dma(kt + 2, st);
                mfma(af1, bf1);
            }
            __syncthreads();

            // ---- epilogue.  The MFMAs compute the transposed tile (B rows as
            // the first operand), so lane l holds output row (l & 15) and four
            // consecutive output columns 4*(l >> 4) + v: packed into one
            // 8-byte LDS store, then written out as 16-byte row chunks.
            uint16_t* Cseg = shared ? p.shC : p.C;
            constexpr int CW = UP ? NPT : BN / 2;  // output columns staged per pass
            constexpr int CS = CW + 8;             // padded LDS row stride
            constexpr int CPR = CW / 8;            // 16-byte chunks per staged row
            constexpr int NPASS = UP ? 1 : 2;
            uint16_t* Cs = smem;
#pragma unroll
            for (int pass = 0; pass < NPASS; ++pass) {
                if (UP) {
#pragma unroll
                    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
                        for (int c = 0; c < WC / 2; ++c) {
                            acc_fence(acc[rt][c], acc[rt][c + WC / 2]);
                            const int row = wm * (RT * 16) + rt * 16 + (l & 15);
                            const f32x4_t g = acc[rt][c], u = acc[rt][c + WC / 2];
                            uint2 v;
                            v.x = pack2_bf16(silu_fast(g[0]) * u[0], silu_fast(g[1]) * u[1]);
                            v.y = pack2_bf16(silu_fast(g[2]) * u[2], silu_fast(g[3]) * u[3]);
                            *(uint2*)&Cs[row * CS + wn * (NPT / kWN) + c * 16 + (l >> 4) * 4] = v;
                        }
                } else {
#pragma unroll
                    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
                        for (int c = 0; c < WC / 2; ++c) {
                            acc_fence(acc[rt][pass * (WC / 2) + c], acc[rt][pass * (WC / 2) + c]);
                            const int row = wm * (RT * 16) + rt * 16 + (l & 15);
                            const f32x4_t a = acc[rt][pass * (WC / 2) + c];
                            uint2 v;
                            v.x = pack2_bf16(a[0], a[1]);
                            v.y = pack2_bf16(a[2], a[3]);
                            *(uint2*)&Cs[row * CS + wn * (BN / (2 * kWN)) + c * 16 + (l >> 4) * 4] = v;
                        }
                }
                __syncthreads();
#pragma unroll
                for (int qq = 0; qq < (kArows * CPR + kThreads - 1) / kThreads; ++qq) {
                    const int idx = tid + qq * kThreads;
                    const int row = idx / CPR, ch = idx % CPR;
                    int col;
                    if (UP) {
                        col = ntile * NPT + ch * 8;
                    } else {
                        constexpr int WPP = BN / (2 * kWN);  // columns per wave per pass
                        const int lc = ch * 8, wv = lc / WPP;
                        col = ntile * BN + wv * (BN / kWN) + pass * WPP + lc % WPP;
                    }
                    if (row < rows)
                        *(u32x4_t*)&Cseg[(size_t)(row0 + m0 + row) * N + col] =
                            *(const u32x4_t*)&Cs[row * CS + ch * 8];
                }
                __syncthreads();
            }
        };
        auto go = [&](auto rt_tag) {
            if constexpr (SO) {
                if (mt == 1) run_tile(rt_tag, IntC<1>{});
                else run_tile(rt_tag, IntC<0>{});
            } else {
                run_tile(rt_tag, IntC<0>{});
            }
        };
        if constexpr (BM == 384) {
            const int rt = hgt / 64;
            if (rt >= 6) go(IntC<6>{});
            else if (rt == 5) go(IntC<5>{});
            else if (rt == 4) go(IntC<4>{});
            else if (rt == 3) go(IntC<3>{});
            else if (rt == 2) go(IntC<2>{});
            else go(IntC<1>{});
        } else {
            if (hgt > 224) go(IntC<8>{});
            else if (hgt > 192) go(IntC<7>{});
            else if (hgt > 160) go(IntC<6>{});
            else if (hgt > 128) go(IntC<5>{});
            else if (hgt > 96) go(IntC<4>{});
            else if (hgt > 64) go(IntC<3>{});
            else if (hgt > 32) go(IntC<2>{});
            else go(IntC<1>{});
        }
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

// Compute units of the current device, queried once per device.  The cache
// is written with relaxed atomics: concurrent first calls from several host
// threads may all query, and they store the same value.
int num_cus()
{
    static std::atomic<int> cached[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    int v = cached[dev].load(std::memory_order_relaxed);
    if (v <= 0) {
        if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || v <= 0)
            v = 256;
        cached[dev].store(v, std::memory_order_relaxed);
    }
    return v;
}

__global__ __launch_bounds__(64) void k_zero_ctr(int* ctr)
{
    if (threadIdx.x < 16) ctr[threadIdx.x] = 0;
}

template <bool UP, int BN, int BMT, bool SO>
hipError_t launch_gemm_t(const GemmParams& p, long long ub, hipStream_t s)
{
    // one resident block per CU (four LDS stages: 96 or 128 KB)
    long long grid = std::min<long long>(ub, (long long)num_cus());
    grid = (grid + 7) / 8 * 8;
    hipLaunchKernelGGL((k_grouped_gemm<UP, BN, BMT, SO>), dim3((unsigned)grid), dim3(512), 0, s, p);
    return hipGetLastError();
}

// 256-wide tiles when every segment's N of this layer splits into them (the
// rule for blocked weights, whose layout is fixed per layer).
bool gemm_wide(const moe_cfg& c, bool up)
{
    const long long Ish = (long long)c.n_shared * c.I_shared;
    const long long nw_r = up ? 2LL * c.I : c.H, nw_s = up ? 2 * Ish : c.H;
    return nw_r % 256 == 0 && (Ish == 0 || nw_s % 256 == 0);
}

// dst = src (one operand of nexp experts, rows x K) in the tile-blocked
// layout: chunk d of 8 elements is chunk c8 of row r of block (e, j, kt).
__global__ __launch_bounds__(256) void k_pack(const uint16_t* __restrict__ src, uint16_t* __restrict__ dst,
                                              long long nchunks, int rows, int half_rows, int K, int BN, int up)
{
    const int KT = K / 64, nt = rows / BN, npt = BN / 2;
    for (long long d = (long long)blockIdx.x * 256 + threadIdx.x; d < nchunks; d += (long long)gridDim.x * 256) {
        const int c8 = (int)(d & 7);
        long long rem = d >> 3;
        const int r = (int)(rem % BN);
        rem /= BN;
        const int kt = (int)(rem % KT);
        rem /= KT;
        const int j = (int)(rem % nt);
        const long long e = rem / nt;
        const int srow = up ? (r < npt ? j * npt + r : half_rows + j * npt + (r - npt)) : j * BN + r;
        ((u32x4_t*)dst)[d] = *(const u32x4_t*)(src + ((size_t)e * rows + srow) * K + kt * 64 + c8 * 8);
    }
}

hipError_t launch_pack_one(const uint16_t* src, uint16_t* dst, long long nexp, int rows, int half_rows, int K,
                           int BN, bool up, hipStream_t s)
{
    const long long n = nexp * rows * (long long)(K / 8);
    if (n == 0) return hipSuccess;
    const long long blocks = std::min<long long>((n + 255) / 256, 8192);
    hipLaunchKernelGGL(k_pack, dim3((unsigned)blocks), dim3(256), 0, s, src, dst, n, rows, half_rows, K, BN,
                       up ? 1 : 0);
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
    p.ctr = a.ctr + (up ? 0 : 8);
    p.blocked = c.weights_blocked;
    // both GEMMs' counters are zeroed once, before the up projection
    if (up && !a.ctr_zeroed) hipLaunchKernelGGL(k_zero_ctr, dim3(1), dim3(64), 0, s, a.ctr);
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
    // the k-loop runs whole pairs of 32-wide k-steps
    if (c.H % 64 != 0 || c.I % 64 != 0 || a.Ish % 64 != 0) return hipErrorInvalidValue;
    // wide tiles (BN = 256) when every segment's N splits into them
    const int nw_r = up ? 2 * c.I : c.H;
    const int nw_s = up ? 2 * a.Ish : c.H;
    const bool wide = c.weights_blocked ? gemm_wide(c, up)
                                        : (a.n_routed == 0 || nw_r % 256 == 0) && (!p.has_shared || nw_s % 256 == 0);
    // otherwise (N a multiple of 128 only) 384 x 128 tiles, waves 4 x 2: a
    // third fewer LDS fragment bytes per output than 256 x 128 with waves
    // 2 x 4, and a segment of up to 384 rows reads its weight tile once
    const int BN = wide ? 256 : 128;
    const int TBM = wide ? BM : 384;
    // host upper bound on the tile count (A is only known on the device)
    long long ub = 0;
    if (a.n_routed > 0) ub += ((long long)ceil_div(a.A_max, TBM) + a.n_routed) * (nw_r / BN);
    if (p.has_shared) ub += (long long)ceil_div(c.T, TBM) * (nw_s / BN);
    if (ub == 0) return hipSuccess;
    // the routed experts' weights (3 I x H each) more than 8x the 256 MB
    // Infinity Cache: a weight tile read once is not found in it again
    const bool so = 3.0 * c.E * c.I * c.H * 2 > 8.0 * (256 << 20);
    if (!wide) {
        if (so) return up ? launch_gemm_t<true, 128, 384, true>(p, ub, s) : launch_gemm_t<false, 128, 384, true>(p, ub, s);
        return up ? launch_gemm_t<true, 128, 384, false>(p, ub, s) : launch_gemm_t<false, 128, 384, false>(p, ub, s);
    }
    if (so) return up ? launch_gemm_t<true, 256, 256, true>(p, ub, s) : launch_gemm_t<false, 256, 256, true>(p, ub, s);
    return up ? launch_gemm_t<true, 256, 256, false>(p, ub, s) : launch_gemm_t<false, 256, 256, false>(p, ub, s);
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

hipError_t launch_pack_weights(const moe_cfg& c, bool shared, const void* W13, const void* W2, void* W13b,
                               void* W2b, hipStream_t s)
{
    const int nexp = shared ? 1 : c.E;
    const int N = shared ? c.n_shared * c.I_shared : c.I;  // intermediate width
    const int BNu = gemm_wide(c, true) ? 256 : 128, BNd = gemm_wide(c, false) ? 256 : 128;
    hipError_t e = launch_pack_one((const uint16_t*)W13, (uint16_t*)W13b, nexp, 2 * N, N, c.H, BNu, true, s);
    if (e == hipSuccess) e = launch_pack_one((const uint16_t*)W2, (uint16_t*)W2b, nexp, c.H, 0, N, BNd, false, s);
    return e;
}

}  // namespace moe
