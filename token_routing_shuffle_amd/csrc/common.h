// Device helpers shared by the libmoe kernels (gfx950 / CDNA4, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#define MOE_DEV __device__ __forceinline__

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;

// bf16 <-> fp32 (bf16 kept as raw uint16 bit patterns in memory)
MOE_DEV float bf2f(uint32_t b) { return __uint_as_float(b << 16); }

MOE_DEV uint32_t f2bf(float f)  // round to nearest even
{
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return (u >> 16) | 0x40u;  // quiet NaN
    u += 0x7fffu + ((u >> 16) & 1u);
    return u >> 16;
}

MOE_DEV uint32_t pack_bf2(float lo, float hi) { return f2bf(lo) | (f2bf(hi) << 16); }

MOE_DEV int lane_id() { return (int)__lane_id(); }

MOE_DEV uint64_t lanemask_lt() { return (1ull << lane_id()) - 1ull; }

// Lanes (among `active`) whose `key` equals this lane's key; key < 2^nbits.
// Multi-split by per-bit ballots: gfx950 has no match instruction.
MOE_DEV uint64_t match_key(uint32_t key, int nbits, uint64_t active)
{
    uint64_t m = active;
    for (int b = 0; b < nbits; ++b) {
        const bool bit = (key >> b) & 1u;
        const uint64_t ones = __ballot(bit);
        m &= bit ? ones : ~ones;
    }
    return m;
}

// Cross-lane moves through DPP (no LDS round trip).  Control codes:
// quad_perm [1,0,3,2] = 0xB1 (lane ^ 1), quad_perm [2,3,0,1] = 0x4E (lane ^ 2),
// row_half_mirror = 0x141 (i <-> 7-i in 8 lanes), row_mirror = 0x140
// (i <-> 15-i in 16 lanes).  After the four steps every lane of a 16-lane
// row holds the row's result; the four rows are then combined through
// readlane in a fixed order, so every lane gets the same, deterministic
// value.  All 64 lanes must be active.
template <int CTRL>
MOE_DEV uint32_t dpp_u32(uint32_t v)
{
    return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, CTRL, 0xF, 0xF, false);
}

template <int CTRL>
MOE_DEV float dpp_f32(float v)
{
    return __uint_as_float(dpp_u32<CTRL>(__float_as_uint(v)));
}

MOE_DEV float readlane_f32(float v, int lane)
{
    return __uint_as_float((uint32_t)__builtin_amdgcn_readlane((int)__float_as_uint(v), lane));
}

MOE_DEV uint32_t readlane_u32(uint32_t v, int lane)
{
    return (uint32_t)__builtin_amdgcn_readlane((int)v, lane);
}

MOE_DEV float wave_sum(float v)
{
    v += dpp_f32<0xB1>(v);
    v += dpp_f32<0x4E>(v);
    v += dpp_f32<0x141>(v);
    v += dpp_f32<0x140>(v);
    return ((readlane_f32(v, 0) + readlane_f32(v, 16)) + readlane_f32(v, 32)) + readlane_f32(v, 48);
}

MOE_DEV float wave_max(float v)
{
    v = fmaxf(v, dpp_f32<0xB1>(v));
    v = fmaxf(v, dpp_f32<0x4E>(v));
    v = fmaxf(v, dpp_f32<0x141>(v));
    v = fmaxf(v, dpp_f32<0x140>(v));
    return fmaxf(fmaxf(readlane_f32(v, 0), readlane_f32(v, 16)),
                 fmaxf(readlane_f32(v, 32), readlane_f32(v, 48)));
}

// One DPP step of a 64-bit maximum: lanes the control gives no source keep
// their value.  Row shifts 1, 2, 4, 8 leave each 16-lane row's maximum in its
// lane 15; row_bcast:15 (rows 1 and 3) and row_bcast:31 (rows 2 and 3) carry
// it to lane 63.
template <int CTRL, int ROWMASK>
MOE_DEV uint64_t dpp_max_u64(uint64_t v)
{
    const int lo = (int)(uint32_t)v, hi = (int)(uint32_t)(v >> 32);
    const uint32_t olo = (uint32_t)__builtin_amdgcn_update_dpp(lo, lo, CTRL, ROWMASK, 0xF, false);
    const uint32_t ohi = (uint32_t)__builtin_amdgcn_update_dpp(hi, hi, CTRL, ROWMASK, 0xF, false);
    const uint64_t o = ((uint64_t)ohi << 32) | olo;
    return o > v ? o : v;
}

// Maximum of a 64-bit value over the wave, returned to every lane.  All 64
// lanes must be active.
MOE_DEV uint64_t wave_max_u64(uint64_t v)
{
    v = dpp_max_u64<0x111, 0xF>(v);  // row_shr:1
    v = dpp_max_u64<0x112, 0xF>(v);  // row_shr:2
    v = dpp_max_u64<0x114, 0xF>(v);  // row_shr:4
    v = dpp_max_u64<0x118, 0xF>(v);  // row_shr:8
    v = dpp_max_u64<0x142, 0xA>(v);  // row_bcast:15
    v = dpp_max_u64<0x143, 0xC>(v);  // row_bcast:31
    const uint32_t lo = readlane_u32((uint32_t)v, 63), hi = readlane_u32((uint32_t)(v >> 32), 63);
    return ((uint64_t)hi << 32) | lo;
}

// Maximum of a 64-bit value over aligned segments of L lanes (L a power of
// two from 1 to 64), returned to every lane of its segment.  All 64 lanes
// must be active.  Within a row: quad swaps (lane ^ 1, lane ^ 2), then the
// half-row and row mirrors, which pair each quad (half-row) with the other
// of its half-row (row); across rows, lane ^ 16 and lane ^ 32 by permute.
MOE_DEV uint64_t seg_max_u64(uint64_t v, int L)
{
    if (L >= 2) v = dpp_max_u64<0xB1, 0xF>(v);
    if (L >= 4) v = dpp_max_u64<0x4E, 0xF>(v);
    if (L >= 8) v = dpp_max_u64<0x141, 0xF>(v);
    if (L >= 16) v = dpp_max_u64<0x140, 0xF>(v);
#pragma unroll
    for (int o = 16; o <= 32; o <<= 1) {
        if (L > o) {
            const uint32_t lo = (uint32_t)__shfl_xor((int)(uint32_t)v, o);
            const uint32_t hi = (uint32_t)__shfl_xor((int)(uint32_t)(v >> 32), o);
            const uint64_t w = ((uint64_t)hi << 32) | lo;
            v = w > v ? w : v;
        }
    }
    return v;
}

MOE_DEV int wave_incl_scan(int v)
{
    const int l = lane_id();
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        int t = __shfl_up(v, o);
        if (l >= o) v += t;
    }
    return v;
}

// Block-wide exclusive scan of one int per thread (blockDim.x <= 1024).
// `smem` must hold 17 ints (16 wave prefixes + the total).  Returns the
// exclusive prefix; *total = block sum.
MOE_DEV int block_excl_scan(int v, int* smem, int* total)
{
    const int l = lane_id();
    const int w = threadIdx.x >> 6;
    const int nw = (blockDim.x + 63) >> 6;
    int incl = wave_incl_scan(v);
    if (l == 63) smem[w] = incl;
    __syncthreads();
    if (w == 0) {
        int s = (l < nw) ? smem[l] : 0;
        int si = wave_incl_scan(s);
        if (l < nw) smem[l] = si - s;
        if (l == nw - 1) smem[16] = si;
    }
    __syncthreads();
    int r = incl - v + smem[w];
    *total = smem[16];
    __syncthreads();
    return r;
}

// Workgroup barrier that waits only for this wave's LDS operations.
// __syncthreads() also fences global memory, which makes every barrier wait
// for all outstanding global loads (vmcnt(0)) and so defeats prefetching
// across barriers; LDS data written before this barrier is visible after it.
MOE_DEV void lds_barrier()
{
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0); vmcnt, expcnt untouched
    __builtin_amdgcn_s_barrier();
}

MOE_DEV int clampi(int v, int lo, int hi) { return v < lo ? lo : (v > hi ? hi : v); }

// Device data checks.  Kernels clamp input values they index with (token
// ids, table entries, slots, budgets) so that bad data cannot send a load out
// of bounds.  A library built with MOE_DEBUG_CHECKS=1 also records every
// clamp or skip in a workspace error word (bits moe_data_error of moe.h);
// the release build compiles the check away.
#ifndef MOE_DEBUG_CHECKS
#define MOE_DEBUG_CHECKS 0
#endif

MOE_DEV void data_error(uint32_t* err, uint32_t bit)
{
    if constexpr (MOE_DEBUG_CHECKS) {
        if (err != nullptr) atomicOr(err, bit);
    } else {
        (void)err;
        (void)bit;
    }
}

MOE_DEV int checked_clamp(int v, int lo, int hi, uint32_t* err, uint32_t bit)
{
    if (v < lo || v > hi) data_error(err, bit);
    return clampi(v, lo, hi);
}

// Own fp32 exp: Cody-Waite additive range reduction n = rint(x*log2 e),
// r = x - n*ln2 with ln2 split into an fp32 high part and the fp32 rounding
// of the remainder (one fused multiply-add each), exp(r) by the degree-7
// Taylor polynomial in Horner form with fused multiply-adds, exact scaling
// by 2^n.  Defined on [-87, 88] (normal results): 0 below, +inf above.
// Bit-reproducible: every step is a single IEEE-rounded fp32 operation.
MOE_DEV float cw_expf(float x)
{
#pragma clang fp contract(off)
    constexpr double kLn2 = 0.69314718055994530942;
    constexpr float ln2_hi = (float)kLn2;
    constexpr float ln2_lo = (float)(kLn2 - (double)(float)kLn2);
    constexpr float log2e = (float)1.44269504088896340736;
    if (x != x) return x;
    if (x < -87.0f) return 0.0f;
    if (x > 88.0f) return __builtin_inff();
    const float n = __builtin_rintf(x * log2e);
    float r = __builtin_fmaf(-n, ln2_hi, x);
    r = __builtin_fmaf(-n, ln2_lo, r);
    float p = (float)(1.0 / 5040.0);
    p = __builtin_fmaf(p, r, (float)(1.0 / 720.0));
    p = __builtin_fmaf(p, r, (float)(1.0 / 120.0));
    p = __builtin_fmaf(p, r, (float)(1.0 / 24.0));
    p = __builtin_fmaf(p, r, (float)(1.0 / 6.0));
    p = __builtin_fmaf(p, r, 0.5f);
    p = __builtin_fmaf(p, r, 1.0f);
    p = __builtin_fmaf(p, r, 1.0f);
    const float scale = __uint_as_float((uint32_t)((int)n + 127) << 23);
    return p * scale;
}

MOE_DEV float cw_sigmoidf(float l)
{
#pragma clang fp contract(off)
    const float e = cw_expf(-l);
    const float d = 1.0f + e;
    return 1.0f / d;
}

// Order-preserving map of a (non-NaN) float to uint32, -0 folded onto +0.
MOE_DEV uint32_t ordered_key(float f)
{
    const float g = f + 0.0f;  // -0 + 0 = +0 under round-to-nearest
    const uint32_t u = __float_as_uint(g);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Inverse of ordered_key (a key of -0 comes back as +0).
MOE_DEV float unordered_key(uint32_t k)
{
    return __uint_as_float((k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k);
}

// ---------------------------------------------------------------------------
// LDS staging helpers of the MFMA kernels (operands DMA'd HBM/L2 -> LDS with
// buffer_load ... lds, fragments read back with ds_read_b128).

#define MOE_LDS_PTR(p) ((void __attribute__((address_space(3)))*)(p))

// s_waitcnt vmcnt(N) (gfx9 encoding; expcnt and lgkmcnt left alone)
template <int N>
MOE_DEV void wait_vmcnt()
{
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

template <int V>
struct IntC {
    static constexpr int value = V;
};

// LDS fragment read issued as inline asm: the compiler's wait-count pass then
// does not treat it as a read of the in-flight LDS DMA (it would drain all
// outstanding loads before it); completion is waited for explicitly with
// frag_wait, whose operands tie the fragments so no use moves above it.  The
// fragment's position inside the stage is the instruction's immediate byte
// offset, so one address register serves all fragments of an operand.
// (The asm exists only in the device pass; the host pass never runs these.)
template <int OFF>
MOE_DEV bf16x8_t lds_read_b128(uint32_t addr)
{
    static_assert(OFF >= 0 && OFF < 65536, "ds_read offset range");
    bf16x8_t v;
#if defined(__HIP_DEVICE_COMPILE__)
    asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(v) : "v"(addr), "i"(OFF));
#else
    (void)addr;
    v = bf16x8_t{};
#endif
    return v;
}

MOE_DEV uint32_t lds_addr(const void* p)
{
#if defined(__HIP_DEVICE_COMPILE__)
    return (uint32_t)(uintptr_t)((__attribute__((address_space(3))) const void*)p);
#else
    return (uint32_t)(uintptr_t)p;
#endif
}

template <int I, int N, typename F>
MOE_DEV void static_for(F&& f)
{
    if constexpr (I < N) {
        f(IntC<I>{});
        static_for<I + 1, N>(f);
    }
}

template <int NA, int NB>
MOE_DEV void frag_wait(bf16x8_t (&a)[NA], bf16x8_t (&b)[NB])
{
#if defined(__HIP_DEVICE_COMPILE__)
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
    for (int i = 0; i < NA; ++i) asm volatile("" : "+v"(a[i]));
#pragma unroll
    for (int i = 0; i < NB; ++i) asm volatile("" : "+v"(b[i]));
#else
    (void)a;
    (void)b;
#endif
}
