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

// bf16 <-> fp32.  bf16 is the upper half of an fp32 bit pattern.
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f)
{
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7FFFFFFFu) > 0x7F800000u)   // NaN: keep it a (quiet) NaN
        return (uint16_t)((u >> 16) | 0x40u);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
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
// Scatter-add through the wave's LDS scratch:  out[i] = add[i] +
// sum_{j : pi[j] = i} v[j], over the NP lanes of one group.  `base` is the
// group's first slot.  Every lane of the wave must call it (convergent).
// ---------------------------------------------------------------------------
template <bool CPLX>
__device__ __forceinline__ cf scatter_add(cf *scr, int lane, int base, int pi, cf v, cf add)
{
    scr[lane] = add;
    lds_order();
    atomicAdd(&scr[base + pi].r, v.r);
    if constexpr (CPLX)
        atomicAdd(&scr[base + pi].i, v.i);
    lds_order();
    const cf out = scr[lane];
    lds_order();
    return out;
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

// Workspace header (first 256 bytes).
struct Header {
    uint64_t magic;
    uint32_t epoch;
    uint32_t ticket;
    uint32_t reserved[60];
};
// The upper half is an epoch value the library never uses (epochs restart
// below 0xFFFFFFF0), so no record word can look like the magic.
constexpr uint64_t kMagic = 0xFFFFFFFF5D55A7B1ull;
constexpr uint32_t kEpochLimit = 0xFFFFFFF0u;

}  // namespace pdssm
