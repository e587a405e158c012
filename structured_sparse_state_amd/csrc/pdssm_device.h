// pdssm_device.h -- device helpers for the PD recurrence scan on gfx950.
//
// Everything here runs on one 64-lane wavefront at a time.  The state of a
// sequence lives "lane = state": lane i of a group of NP lanes holds x[i].
// A step x' = P (d * x) + b is a scatter-add (column j of P sends x[j] to row
// pi[j]); it goes through a 64-slot LDS scratch owned by the wave.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pdssm.h"

namespace pdssm {

// Complex fp32 value; in real mode the imaginary part is a constant zero
// that the compiler folds away.
struct cf {
    float r, i;
};

__device__ __forceinline__ cf cmul(cf a, cf b)
{
    return {a.r * b.r - a.i * b.i, a.r * b.i + a.i * b.r};
}

// Compiler-level memory barrier.  LDS instructions of one wavefront execute
// in issue order, so a write by one lane followed by a read by another lane
// of the same wave needs no hardware wait -- only that the compiler keeps
// the order.
__device__ __forceinline__ void lds_order() { asm volatile("" ::: "memory"); }

// Materialise two values here: the compiler may neither sink their
// computation towards a distant use (which would keep every input of it
// alive instead of the result) nor recompute them later.
__device__ __forceinline__ void keep_here(float &a, float &b) { asm volatile("" : "+v"(a), "+v"(b)); }

// A copy of v that the compiler cannot see through: everything derived from
// it is computed after this point.  Inside a loop this keeps lane-derived
// constants from being hoisted out and held in registers across the loop.
__device__ __forceinline__ int opaque(int v)
{
    asm volatile("" : "+v"(v));
    return v;
}

// The same for a wave-uniform value (kept in a scalar register).
__device__ __forceinline__ int opaque_s(int v)
{
    asm volatile("" : "+s"(v));
    return v;
}
__device__ __forceinline__ uint32_t opaque_s(uint32_t v)
{
    asm volatile("" : "+s"(v));
    return v;
}

// bf16 <-> fp32.  bf16 is the upper half of an fp32 bit pattern.
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// fp32 -> bf16, rounded to nearest even: one v_cvt_pk_bf16_f32 (a NaN
// stays a quiet NaN).  The pair form converts (lo, hi) into one word.
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f)
{
    const __bf16 h = (__bf16)f;
    uint16_t u;
    __builtin_memcpy(&u, &h, 2);
    return u;
}

__device__ __forceinline__ uint32_t f32x2_to_bf16x2_rne(float lo, float hi)
{
    typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
    typedef float f32x2_t __attribute__((ext_vector_type(2)));
    const f32x2_t v = {lo, hi};
    const bf16x2_t h = __builtin_convertvector(v, bf16x2_t);
    uint32_t u;
    __builtin_memcpy(&u, &h, 4);
    return u;
}

// ---------------------------------------------------------------------------
// Per-element loads of the step inputs.  `e` is the flat element index
// ((b*H + h)*L + t)*N + i; complex arrays hold (re, im) pairs.
// ---------------------------------------------------------------------------
template <bool CPLX>
__device__ __forceinline__ cf load_diag(const float *__restrict__ p, int64_t e)
{
    if constexpr (CPLX) {
        const float2 v = reinterpret_cast<const float2 *>(p)[e];
        return {v.x, v.y};
    } else {
        return {p[e], 0.f};
    }
}

template <bool CPLX, bool BF16>
__device__ __forceinline__ cf load_vec(const void *__restrict__ p, int64_t e)
{
    if constexpr (BF16) {
        if constexpr (CPLX) {
            const uint32_t w = reinterpret_cast<const uint32_t *>(p)[e];
            return {bf16_lo(w), bf16_hi(w)};
        } else {
            const uint16_t w = reinterpret_cast<const uint16_t *>(p)[e];
            return {bf16_lo(w), 0.f};
        }
    } else {
        return load_diag<CPLX>(reinterpret_cast<const float *>(p), e);
    }
}

// ---------------------------------------------------------------------------
// Hard selection of one step (argmax over K scores, first maximum wins, a
// NaN is above every number and the first NaN wins; index modes read the
// index).  The result is clamped into [0, K).
// ---------------------------------------------------------------------------
__device__ __forceinline__ void argmax_take(float v, int k, float &best_v, int &best)
{
    // v replaces the current best when the best is a number and v is either
    // a NaN or strictly larger.
    const bool take = (best_v == best_v) && ((v != v) || (v > best_v));
    best_v = take ? v : best_v;
    best = take ? k : best;
}

__device__ __forceinline__ int select_step(const void *__restrict__ src, uint32_t mode,
                                           int64_t step, int K)
{
    int k;
    if (mode == PDSSM_SEL_I32) {
        k = reinterpret_cast<const int32_t *>(src)[step];
    } else if (mode == PDSSM_SEL_I16) {
        k = reinterpret_cast<const int16_t *>(src)[step];
    } else if (mode == PDSSM_LOGITS_F32) {
        const float *row = reinterpret_cast<const float *>(src) + step * (int64_t)K;
        float bv = row[0];
        k = 0;
        if ((K & 3) == 0) {
            for (int q = 0; q < K; q += 4) {
                const float4 v = *reinterpret_cast<const float4 *>(row + q);
                argmax_take(v.x, q, bv, k);
                argmax_take(v.y, q + 1, bv, k);
                argmax_take(v.z, q + 2, bv, k);
                argmax_take(v.w, q + 3, bv, k);
            }
        } else {
            for (int q = 1; q < K; ++q)
                argmax_take(row[q], q, bv, k);
        }
    } else {
        const uint16_t *row = reinterpret_cast<const uint16_t *>(src) + step * (int64_t)K;
        float bv = bf16_lo(row[0]);
        k = 0;
        if ((K & 7) == 0) {
            for (int q = 0; q < K; q += 8) {
                const uint4 v = *reinterpret_cast<const uint4 *>(row + q);
                argmax_take(bf16_lo(v.x), q, bv, k);
                argmax_take(bf16_hi(v.x), q + 1, bv, k);
                argmax_take(bf16_lo(v.y), q + 2, bv, k);
                argmax_take(bf16_hi(v.y), q + 3, bv, k);
                argmax_take(bf16_lo(v.z), q + 4, bv, k);
                argmax_take(bf16_hi(v.z), q + 5, bv, k);
                argmax_take(bf16_lo(v.w), q + 6, bv, k);
                argmax_take(bf16_hi(v.w), q + 7, bv, k);
            }
        } else {
            for (int q = 1; q < K; ++q)
                argmax_take(bf16_lo(row[q]), q, bv, k);
        }
    }
    return (int)min((unsigned)k, (unsigned)(K - 1));
}

// ---------------------------------------------------------------------------
// Cross-lane moves inside a wavefront.
// ---------------------------------------------------------------------------
__device__ __forceinline__ float bperm(float v, int src_lane)
{
    return __int_as_float(__builtin_amdgcn_ds_bpermute(src_lane << 2, __float_as_int(v)));
}
__device__ __forceinline__ int bperm(int v, int src_lane)
{
    return __builtin_amdgcn_ds_bpermute(src_lane << 2, v);
}
__device__ __forceinline__ uint32_t bperm(uint32_t v, int src_lane)
{
    return (uint32_t)__builtin_amdgcn_ds_bpermute(src_lane << 2, (int)v);
}

// DPP lane moves inside rows of 16 lanes.
constexpr int kDppXor1 = 0xB1;        // quad_perm [1,0,3,2]
constexpr int kDppXor2 = 0x4E;        // quad_perm [2,3,0,1]
constexpr int kDppHalfMirror = 0x141; // lane i <-> 7-i within each 8
constexpr int kDppRowRor8 = 0x128;    // lane i <- (i+8) mod 16 within each row

template <int CTRL>
__device__ __forceinline__ float dpp(float v)
{
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}

// The partner value across lane bit b (used only as a summation partner:
// for b = 2 the partner is the mirror lane 7-i, which differs in bit 2 and
// keeps bits >= 3, enough for a reduction that later sums bits 1 and 0).
template <int BIT>
__device__ __forceinline__ float across_bit(float v)
{
    if constexpr (BIT == 3)
        return dpp<kDppRowRor8>(v);
    else if constexpr (BIT == 2)
        return dpp<kDppHalfMirror>(v);
    else if constexpr (BIT == 1)
        return dpp<kDppXor2>(v);
    else
        return dpp<kDppXor1>(v);
}

// Sum of the two values held across lane bit BIT (5: lanes l and l^32,
// 4: l and l^16): the permlane swaps of gfx950 exchange half-waves / odd
// and even rows between two registers in one instruction.
template <int BIT>
__device__ __forceinline__ void swap_halves(float &lo_keep, float &hi_keep)
{
    // After the swap, lanes with BIT clear hold (lo[l], lo[partner]) in the
    // two registers and lanes with BIT set hold (hi[partner], hi[l]).
    if constexpr (BIT == 5) {
        auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(lo_keep), __float_as_uint(hi_keep),
                                                  false, false);
        lo_keep = __uint_as_float(r[0]);
        hi_keep = __uint_as_float(r[1]);
    } else {
        auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(lo_keep), __float_as_uint(hi_keep),
                                                  false, false);
        lo_keep = __uint_as_float(r[0]);
        hi_keep = __uint_as_float(r[1]);
    }
}

// Transposed butterfly sum inside groups of NP lanes.  On entry every lane
// holds v[t] for T steps; on exit register r of lane i (group-local index)
// holds the group sum of step  r + RF * (i >> NPLAIN), with RF and NPLAIN
// below, and every lane whose low NPLAIN bits are zero owns its steps.
template <int NP, int T>
struct Butterfly {
    static constexpr int LOG = NP == 8 ? 3 : NP == 16 ? 4 : NP == 32 ? 5 : 6;
    static constexpr int LT = T == 1 ? 0 : T == 2 ? 1 : T == 4 ? 2 : T == 8 ? 3 : T == 16 ? 4 : T == 32 ? 5 : 6;
    static constexpr int NH = LT < LOG ? LT : LOG;   // halving levels
    static constexpr int NPLAIN = LOG - NH;          // plain levels
    static constexpr int RF = T >> NH;               // registers left
};

template <int BIT, int R>
__device__ __forceinline__ void butterfly_level(float *v, int i)
{
    if constexpr (R > 1) {
        constexpr int H = R / 2;
        const bool hi = (i >> BIT) & 1;
#pragma unroll
        for (int r = 0; r < H; ++r) {
            if constexpr (BIT >= 4) {
                float a = v[r], b = v[r + H];
                swap_halves<BIT>(a, b);
                v[r] = a + b;
            } else {
                const float send = hi ? v[r] : v[r + H];
                const float keep = hi ? v[r + H] : v[r];
                v[r] = keep + across_bit<BIT>(send);
            }
        }
    } else {
        if constexpr (BIT >= 4) {
            float a = v[0], b = v[0];
            swap_halves<BIT>(a, b);
            v[0] = a + b;
        } else {
            v[0] = v[0] + across_bit<BIT>(v[0]);
        }
    }
}

template <int BIT, int R>
__device__ __forceinline__ void butterfly_from(float *v, int i)
{
    butterfly_level<BIT, R>(v, i);
    if constexpr (BIT > 0)
        butterfly_from<BIT - 1, (R > 1 ? R / 2 : 1)>(v, i);
}

template <int NP, int T>
__device__ __forceinline__ void group_transpose_sum(float (&v)[T], int i)
{
    butterfly_from<Butterfly<NP, T>::LOG - 1, T>(v, i);
}

// The same sum taken in two stages, so that only four per-step registers
// are live at a time: every four consecutive steps first fold over the two
// top lane bits of the group (group_fold4, one register out), and the T/4
// folded registers then finish over the remaining bits (group_finish).
// Afterwards register r of lane i holds the group sum of step
//   4 * (r + RF * ((i >> NPLAIN) & (2^NH - 1))) + ((i >> (LOG - 2)) & 3)
// and every lane whose low NPLAIN bits are zero owns its RF steps.
template <int NP, int T>
struct GroupedButterfly {
    static_assert(T % 4 == 0 && T >= 4, "steps come in groups of four");
    static constexpr int LOG = Butterfly<NP, T>::LOG;
    static constexpr int LT4 = Butterfly<NP, T / 4>::LT;
    static constexpr int NH = LT4 < LOG - 2 ? LT4 : LOG - 2;
    static constexpr int NPLAIN = LOG - 2 - NH;
    static constexpr int RF = (T / 4) >> NH;

    __device__ static int step_of(int r, int i)
    {
        return 4 * (r + RF * ((i >> NPLAIN) & ((1 << NH) - 1))) + ((i >> (LOG - 2)) & 3);
    }
};

template <int NP>
__device__ __forceinline__ float group_fold4(float (&v)[4], int i)
{
    constexpr int LOG = Butterfly<NP, 4>::LOG;
    butterfly_level<LOG - 1, 4>(v, i);
    butterfly_level<LOG - 2, 2>(v, i);
    return v[0];
}

template <int NP, int R>
__device__ __forceinline__ void group_finish(float (&w)[R], int i)
{
    constexpr int LOG = Butterfly<NP, 4>::LOG;
    if constexpr (LOG >= 3)
        butterfly_from<LOG - 3, R>(w, i);
}

// ds_bpermute with the source given as a byte address (4 * lane).
__device__ __forceinline__ float bperm_a(float v, int addr)
{
    return __int_as_float(__builtin_amdgcn_ds_bpermute(addr, __float_as_int(v)));
}
__device__ __forceinline__ uint32_t bperm_a(uint32_t v, int addr)
{
    return (uint32_t)__builtin_amdgcn_ds_bpermute(addr, (int)v);
}

// Raw buffer access: a wave-uniform base in scalar registers, a per-lane
// byte offset and a wave-uniform byte offset, so stepping through rows costs
// no vector arithmetic.  Callers keep every access inside `bytes`.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *p, uint64_t bytes)
{
    const uint32_t n = bytes > 0xFFFFFFFFull ? 0xFFFFFFFFu : (uint32_t)bytes;
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(p), (short)0, (int)n, 0x00020000);
}

template <typename V>
__device__ __forceinline__ V bload(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff)
{
    V out;
    if constexpr (sizeof(V) == 8) {
        const auto v = __builtin_amdgcn_raw_buffer_load_b64(r, voff, soff, 0);
        __builtin_memcpy(&out, &v, 8);
    } else if constexpr (sizeof(V) == 4) {
        const uint32_t v = __builtin_amdgcn_raw_buffer_load_b32(r, voff, soff, 0);
        __builtin_memcpy(&out, &v, 4);
    } else {
        static_assert(sizeof(V) == 2, "2, 4 or 8 bytes");
        const uint16_t v = __builtin_amdgcn_raw_buffer_load_b16(r, voff, soff, 0);
        __builtin_memcpy(&out, &v, 2);
    }
    return out;
}

// ---------------------------------------------------------------------------
// Cooperative hard selection for SPW consecutive steps of one sequence by
// one wave.  With SPW <= 64, 64/SPW lanes share a step: each takes a slice of
// the K scores (coalesced, 16-byte loads when aligned), then the slices
// combine across lanes.  Writes k to out[q] for q < SPW (0 past the end).
// ---------------------------------------------------------------------------
// (v2, k2) beats (v1, k1): the higher score, then the lower index; a NaN is
// above every number and the first NaN wins.  One boolean expression, so
// that callers select instead of branching per comparison.
__device__ __forceinline__ bool better(float v2, int k2, float v1, int k1)
{
    const bool n1 = v1 != v1, n2 = v2 != v2;
    const bool klt = k2 < k1;
    return (n2 & (!n1 | klt)) | (!n2 & !n1 & ((v2 > v1) | ((v2 == v1) & klt)));
}

// Keep the better of (bv, bk) and (v, k); `ok` false leaves them as they are.
__device__ __forceinline__ void take_better(float v, int k, bool ok, float &bv, int &bk)
{
    const bool t = ok & better(v, k, bv, bk);
    bv = t ? v : bv;
    bk = t ? k : bk;
}

__device__ __forceinline__ void slice_argmax(const void *__restrict__ src, uint32_t mode,
                                             int64_t step, int K, int k0, int k1, float &bv, int &bk)
{
    if (mode == PDSSM_LOGITS_F32) {
        const float *row = reinterpret_cast<const float *>(src) + step * (int64_t)K;
        if (((K | k0 | k1) & 3) == 0) {
            for (int q = k0; q < k1; q += 4) {
                const float4 v = *reinterpret_cast<const float4 *>(row + q);
                take_better(v.x, q, true, bv, bk);
                take_better(v.y, q + 1, true, bv, bk);
                take_better(v.z, q + 2, true, bv, bk);
                take_better(v.w, q + 3, true, bv, bk);
            }
        } else {
            for (int q = k0; q < k1; ++q) {
                const float v = row[q];
                take_better(v, q, true, bv, bk);
            }
        }
    } else {
        const uint16_t *row = reinterpret_cast<const uint16_t *>(src) + step * (int64_t)K;
        if (((K | k0 | k1) & 7) == 0) {
            for (int q = k0; q < k1; q += 8) {
                const uint4 w = *reinterpret_cast<const uint4 *>(row + q);
                const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
                for (int m = 0; m < 4; ++m) {
                    const float lo = bf16_lo(ws[m]), hi = bf16_hi(ws[m]);
                    take_better(lo, q + 2 * m, true, bv, bk);
                    take_better(hi, q + 2 * m + 1, true, bv, bk);
                }
            }
        } else {
            for (int q = k0; q < k1; ++q) {
                const float v = bf16_lo(row[q]);
                take_better(v, q, true, bv, bk);
            }
        }
    }
}

template <int SPW>
__device__ __forceinline__ void wave_select(const void *__restrict__ src, uint32_t mode, int K,
                                            int64_t L, int64_t seq_row, int64_t t_first,
                                            int16_t *out, int lane)
{
    constexpr int LPS = SPW >= 64 ? 1 : 64 / SPW;   // lanes per step
    constexpr int SPL = SPW >= 64 ? SPW / 64 : 1;   // steps per lane
    const bool index_mode = (mode == PDSSM_SEL_I32 || mode == PDSSM_SEL_I16);
#pragma unroll
    for (int s = 0; s < SPL; ++s) {
        const int q = SPW >= 64 ? s * 64 + lane : lane / LPS;
        const int part = SPW >= 64 ? 0 : lane % LPS;
        const int64_t t = t_first + q;
        const bool live = t < L;
        int k = 0;
        if (index_mode) {
            if (live && part == 0)
                k = (mode == PDSSM_SEL_I32) ? reinterpret_cast<const int32_t *>(src)[seq_row + t]
                                            : reinterpret_cast<const int16_t *>(src)[seq_row + t];
        } else {
            // Slice of the K scores for this lane, a multiple of 8 wide when
            // K is, so every slice stays 16-byte aligned.
            int seg = (K + LPS - 1) / LPS;
            if ((K & 7) == 0)
                seg = (seg + 7) & ~7;
            const int k0 = min(part * seg, K), k1 = min(k0 + seg, K);
            float bv = __int_as_float(opaque((int)0xFF800000u));   // -inf, made here
            int bk = K;
            if (live && k0 < k1)
                slice_argmax(src, mode, seq_row + t, K, k0, k1, bv, bk);
#pragma unroll
            for (int m = 1; m < LPS; m <<= 1) {
                const int from = (lane ^ m) << 2;
                const float ov = bperm_a(bv, from);
                const int ok = (int)bperm_a((uint32_t)bk, from);
                take_better(ov, ok, true, bv, bk);
            }
            k = bk;
        }
        k = (int)min((unsigned)k, (unsigned)(K - 1));
        if (part == 0)
            out[q] = (int16_t)(live ? k : 0);
    }
}

// ---------------------------------------------------------------------------
// Split form of the cooperative selection for the common case: one step per
// lane group of LPS = 64/SPW lanes, K a multiple of 8 (bf16) or 4 (fp32), and
// a slice of at most NV 16-byte vectors per lane.  select_issue() starts the loads (all
// addresses clamped in range, so they are unconditional); select_finish()
// reduces them once they have arrived.
// ---------------------------------------------------------------------------
template <int NV>
struct ScoreSlice {
    uint4 v[NV];
};

template <int SPW>
__host__ __device__ constexpr int lanes_per_step() { return SPW >= 64 ? 1 : 64 / SPW; }

// The cooperative path needs every lane's slice of a step's K scores to fit
// NV 16-byte vectors (and K a multiple of the vector width).
__host__ __device__ inline bool select_fast_ok(uint32_t mode, int K, int LPS, int SPW, int NV)
{
    if (SPW > 64)
        return false;
    if (mode == PDSSM_LOGITS_BF16)
        return (K & 7) == 0 && (((K + LPS - 1) / LPS + 7) & ~7) <= 8 * NV;
    if (mode == PDSSM_LOGITS_F32)
        return (K & 3) == 0 && (((K + LPS - 1) / LPS + 3) & ~3) <= 4 * NV;
    return true;   // index modes
}

template <int SPW>
__device__ __forceinline__ void select_slice(uint32_t mode, int K, int lane, int &k0, int &k1)
{
    constexpr int LPS = lanes_per_step<SPW>();
    const int part = lane % LPS;
    int seg = (K + LPS - 1) / LPS;
    seg = (mode == PDSSM_LOGITS_BF16) ? ((seg + 7) & ~7) : ((seg + 3) & ~3);
    k0 = min(part * seg, K);
    k1 = min(k0 + seg, K);
}

template <int SPW, int NV>
__device__ __forceinline__ ScoreSlice<NV> select_issue(const void *__restrict__ src, uint32_t mode, int K,
                                                       int64_t L, int64_t seq_row, int64_t t_first, int lane)
{
    constexpr int LPS = lanes_per_step<SPW>();
    ScoreSlice<NV> s = {};
    const int q = lane / LPS;
    const int64_t t = min(t_first + q, L - 1);
    if (mode == PDSSM_SEL_I32 || mode == PDSSM_SEL_I16) {
        const int v = (mode == PDSSM_SEL_I32) ? reinterpret_cast<const int32_t *>(src)[seq_row + t]
                                              : reinterpret_cast<const int16_t *>(src)[seq_row + t];
        s.v[0].x = (uint32_t)v;
        return s;
    }
    int k0, k1;
    select_slice<SPW>(mode, K, lane, k0, k1);
    const int esz = (mode == PDSSM_LOGITS_BF16) ? 2 : 4;
    const int per = 16 / esz;   // elements per 16-byte vector
    const char *row = reinterpret_cast<const char *>(src) + (seq_row + t) * (int64_t)K * esz;
#pragma unroll
    for (int v = 0; v < NV; ++v) {
        const int e = min(k0 + v * per, K - per);
        s.v[v] = *reinterpret_cast<const uint4 *>(row + (int64_t)e * esz);
    }
    return s;
}

// Score i of a lane's slice (bf16 pairs or fp32 words, in index order).
template <bool BF, int NV>
__device__ __forceinline__ float slice_score(const ScoreSlice<NV> &s, int i)
{
    constexpr int PER = BF ? 8 : 4;
    const uint4 &v = s.v[i / PER];
    const int m = i % PER;
    const int wi = BF ? m >> 1 : m;   // the 32-bit word of the vector
    const uint32_t w = wi == 0 ? v.x : wi == 1 ? v.y : wi == 2 ? v.z : v.w;
    if constexpr (BF)
        return (m & 1) ? bf16_hi(w) : bf16_lo(w);
    else
        return __uint_as_float(w);
}

// Argmax of the first n scores of a lane's slice, scanned in index order.
// Without NaN a strict comparison is the whole rule: among equal scores
// (+0 and -0 included) the first one stays.  Returns the position in the
// slice (0 for an empty one) and flags a slice whose scores may hold a NaN
// (their sum is NaN), for which the caller takes the exact comparison.
// MASKED: positions n and on are read as -inf.
template <bool BF, bool MASKED, int NV>
__device__ __forceinline__ int slice_argmax(const ScoreSlice<NV> &s, int n, float &bv, bool &nan)
{
    constexpr int CNT = (BF ? 8 : 4) * NV;
    const float ninf = __int_as_float((int)0xFF800000u);
    float acc = 0.f;
    int bi = 0;
#pragma unroll
    for (int i = 0; i < CNT; ++i) {
        float v = slice_score<BF, NV>(s, i);
        if constexpr (MASKED)
            v = (i < n) ? v : ninf;
        acc += v;
        if (i == 0) {
            bv = v;
        } else {
            const bool t = v > bv;
            bv = t ? v : bv;
            bi = t ? i : bi;
        }
    }
    nan = acc != acc;
    return bi;
}

template <int SPW, int NV>
__device__ __forceinline__ void select_finish(const ScoreSlice<NV> &s, uint32_t mode, int K, int64_t L,
                                              int64_t t_first, int16_t *out, int lane)
{
    constexpr int LPS = lanes_per_step<SPW>();
    const int q = lane / LPS, part = lane % LPS;
    const bool live = t_first + q < L;
    int k;
    if (mode == PDSSM_SEL_I32 || mode == PDSSM_SEL_I16) {
        k = (int)s.v[0].x;
    } else {
        int k0, k1;
        select_slice<SPW>(mode, K, lane, k0, k1);
        const bool bf = (mode == PDSSM_LOGITS_BF16);
        const int n = k1 - k0;
        float bv = __int_as_float((int)0xFF800000u);
        bool nan = true;
        int bk = K;
        // Slices of up to two vectors (one chunk per wave): one wave-uniform
        // branch picks the unpacking and whether any lane's slice is short
        // (its tail then reads as -inf).  Longer slices go the exact way.
        if constexpr (NV <= 2) {
            int bi;
            if (bf)
                bi = __all(n >= 8 * NV) ? slice_argmax<true, false, NV>(s, n, bv, nan)
                                        : slice_argmax<true, true, NV>(s, n, bv, nan);
            else
                bi = __all(n >= 4 * NV) ? slice_argmax<false, false, NV>(s, n, bv, nan)
                                        : slice_argmax<false, true, NV>(s, n, bv, nan);
            bk = (n > 0) ? k0 + bi : K;   // an empty slice offers K, below every index
        }
        if (__any(nan)) {
            // A NaN (or +inf and -inf) in the slice: the exact rule, NaN
            // above every number and the first NaN winning.
            if (nan) {
                bv = __int_as_float((int)0xFF800000u);
                bk = K;
#pragma unroll
                for (int v = 0; v < NV; ++v) {
                    const uint32_t w[4] = {s.v[v].x, s.v[v].y, s.v[v].z, s.v[v].w};
#pragma unroll
                    for (int m = 0; m < 8; ++m) {
                        const int kk = bf ? k0 + v * 8 + m : k0 + v * 4 + (m & 3);
                        if (!bf && m >= 4)
                            continue;
                        const float val = bf ? ((m & 1) ? bf16_hi(w[m >> 1]) : bf16_lo(w[m >> 1]))
                                             : __uint_as_float(w[m]);
                        take_better(val, kk, kk < k1, bv, bk);
                    }
                }
            }
        }
#pragma unroll
        for (int m = 1; m < LPS; m <<= 1) {
            float ov;
            int ok;
            if (m == 1) {
                ov = dpp<kDppXor1>(bv);
                ok = __float_as_int(dpp<kDppXor1>(__int_as_float(bk)));
            } else if (m == 2) {
                ov = dpp<kDppXor2>(bv);
                ok = __float_as_int(dpp<kDppXor2>(__int_as_float(bk)));
            } else {
                const int src = (lane ^ m) << 2;
                ov = bperm_a(bv, src);
                ok = (int)bperm_a((uint32_t)bk, src);
            }
            take_better(ov, ok, true, bv, bk);
        }
        k = bk;
    }
    k = (int)min((unsigned)k, (unsigned)(K - 1));
    if (part == 0)
        out[q] = (int16_t)(live ? k : 0);
}

// ---------------------------------------------------------------------------
// Scatter-add through the wave's LDS scratch:  out[i] = add[i] +
// sum_{j : pi[j] = i} v[j], over the NP lanes of one group.  `base` is the
// group's first slot.  Every lane of the wave must call it (convergent).
// ---------------------------------------------------------------------------
// Float add into LDS (no ordering wider than the workgroup is needed).
__device__ __forceinline__ void lds_add(float *p, float v)
{
    (void)__hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}

// Byte offset of an LDS object (the low half of its generic address).
template <typename P>
__device__ __forceinline__ uint32_t lds_addr(P *p)
{
    return (uint32_t)(uintptr_t)p;
}

// The adds and the read-back form one asm block that waits for its own LDS
// operations.  Written as C++, the compiler makes LDS atomics wait for every
// global-to-LDS copy still in flight, since it cannot tell that they touch
// other bytes; the wave that stages the entry table must not stall on it.
template <bool CPLX>
__device__ __forceinline__ cf scatter_add(cf *scr, int lane, int base, int pi, cf v, cf add)
{
    scr[lane] = add;
    const uint32_t to = lds_addr(&scr[base + pi]);
    const uint32_t from = lds_addr(&scr[lane]);
    float2 out;
    if constexpr (CPLX)
        asm volatile("ds_add_f32 %1, %3\n\tds_add_f32 %1, %4 offset:4\n\tds_read_b64 %0, %2\n\ts_waitcnt lgkmcnt(0)"
                     : "=v"(out)
                     : "v"(to), "v"(from), "v"(v.r), "v"(v.i)
                     : "memory");
    else
        asm volatile("ds_add_f32 %1, %3\n\tds_read_b64 %0, %2\n\ts_waitcnt lgkmcnt(0)"
                     : "=v"(out)
                     : "v"(to), "v"(from), "v"(v.r)
                     : "memory");
    return {out.x, out.y};
}

// ---------------------------------------------------------------------------
// The collision-free scatter of one step.  A chunk wave's scatter area has
// 2R + 2 blocks of 64 complex slots: blocks 0 .. R-1 hold regions R-1 .. 0
// (region r at block R-1-r), R .. 2R-1 stay zero, 2R is the spare region and
// 2R+1 a trash block.  Source j stores into row pi(j) of the region of its
// rank (rank = number of sources j' < j with the same destination), so a
// region never has two sources on one row; row i reads the R blocks from
// block R - min(deg(i), R) on: its deg(i) regions, then zero blocks.  The
// source of rank R stores into row pi(j) of the spare region, and a row of
// in-degree above R also reads its spare slot (a read under its own lane
// mask).  Sources of rank above R (rare: a row with five or more sources)
// store into the trash block and then add atomically into the spare slot.
// ---------------------------------------------------------------------------
// The forward scan can keep the state before every chunk of kCarryStride
// steps; the backward scan works on chunks of the same length.
constexpr int kCarryStride = 16;

#ifndef PDSSM_SCAN_REGIONS
#define PDSSM_SCAN_REGIONS 3
#endif
constexpr int kRegions = PDSSM_SCAN_REGIONS;   // collision-free regions (ranks 0..kRegions-1)
constexpr int kRegionBytes = 64 * 8;           // one block: 64 complex slots
constexpr int kBlocks = 2 * kRegions + 2;
constexpr uint32_t kSpareOff = 2 * kRegions * kRegionBytes;         // the spare region
constexpr uint32_t kTrashOff = (2 * kRegions + 1) * kRegionBytes;   // stores of sources of rank > R
constexpr int kBlockBits = kBlocks <= 8 ? 3 : 4;   // bits of the scatter block field
constexpr int kDegOvfBit = 6 + kBlockBits + 3;     // the row has more than R sources (top bit)
static_assert(kRegions >= 1 && kRegions <= 4, "the entry's read-block field holds 0..kRegions in 3 bits");
static_assert(kDegOvfBit < 16, "entries are 16 bits");

// Byte offset of a source's scatter slot (block * 512 + pi * 8) and of the
// first block its row reads, from its entry.
__device__ __forceinline__ uint32_t entry_slot(uint32_t ent) { return (ent & ((1u << (6 + kBlockBits)) - 1u)) << 3; }
__device__ __forceinline__ uint32_t entry_row(uint32_t ent)
{
    return ((ent >> (6 + kBlockBits)) & 7u) * (uint32_t)kRegionBytes;
}
// The row has more than R sources: it also reads its spare slot.
__device__ __forceinline__ bool entry_deg_ovf(uint32_t ent) { return ent >= (1u << kDegOvfBit); }
// The source has rank above R: it adds into the spare slot of its row.
__device__ __forceinline__ bool slot_rank_ovf(uint32_t slot) { return slot >= kTrashOff; }

// The 16-bit entry of source `lane` for the index map row[0..N):
//   pi | scatter block << 6 | read block << (6 + kBlockBits) | (deg > R) << kDegOvfBit.
// Called by a wave whose lanes [0, N) are all active (lanes >= N are padding
// sources that map to themselves with rank 0 and in-degree 1); entries
// outside [0,N) clamp.  The rank is the number of lower sources with the same
// destination, the in-degree the number of sources whose destination is this
// lane.  Both come from six ballots, one per bit of a destination: the lanes
// that agree with a value on every bit are the AND, over the bits, of the
// ballot or its complement.
__device__ __forceinline__ uint16_t dict_entry(const int32_t *row, int N, int lane)
{
    const int pi = lane < N ? (int)min((unsigned)row[lane], (unsigned)(N - 1)) : lane;
    const uint64_t real = N >= 64 ? ~0ull : ((1ull << N) - 1ull);
    uint64_t same = real, into = real;
#pragma unroll
    for (int bit = 0; bit < 6; ++bit) {
        const uint64_t m = __ballot((pi >> bit) & 1);
        same &= ((pi >> bit) & 1) ? m : ~m;
        into &= ((lane >> bit) & 1) ? m : ~m;
    }
    const int rank = __popcll(same & ((1ull << lane) - 1ull));
    int deg = __popcll(into);
    if (lane >= N)
        deg = 1;   // padding rows hold their own (zero) state
    const int block = rank < kRegions ? kRegions - 1 - rank : rank == kRegions ? 2 * kRegions : 2 * kRegions + 1;
    const int rblock = kRegions - min(deg, kRegions);
    return (uint16_t)(pi | (block << 6) | (rblock << (6 + kBlockBits)) | ((deg > kRegions ? 1 : 0) << kDegOvfBit));
}

// ---------------------------------------------------------------------------
// Carry records in the workspace.  Each 64-bit word holds a 32-bit payload
// and, in its upper half, the epoch of the call that wrote it, so a reader
// knows a word is from this call without any fence between words.
// ---------------------------------------------------------------------------
__device__ __forceinline__ void put_word(uint64_t *p, uint32_t payload, uint32_t epoch)
{
    __hip_atomic_store(p, ((uint64_t)epoch << 32) | payload, __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ bool get_word(const uint64_t *p, uint32_t epoch, uint32_t &payload)
{
    const uint64_t w = __hip_atomic_load(const_cast<uint64_t *>(p), __ATOMIC_RELAXED,
                                         __HIP_MEMORY_SCOPE_AGENT);
    payload = (uint32_t)w;
    return (uint32_t)(w >> 32) == epoch;
}

// Workspace header (first 256 bytes).  The ticket counter has a 128-byte
// line to itself: every workgroup reads the epoch, and sharing a line with
// those reads would slow each ticket increment several-fold.
struct Header {
    uint64_t magic;
    uint32_t epoch;
    uint32_t reserved0[29];
    uint32_t ticket;
    uint32_t reserved1[31];
};
static_assert(sizeof(Header) == 256, "workspace header is 256 bytes");
// The upper half is an epoch value the library never uses (epochs restart
// below 0xFFFFFFF0), so no record word can look like the magic.
constexpr uint64_t kMagic = 0xFFFFFFFF5D55A7B1ull;
constexpr uint32_t kEpochLimit = 0xFFFFFFF0u;

}  // namespace pdssm
