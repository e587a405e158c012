// Two small kernels beside the scan, on the same boundary:
//
//  * pdssm_dict_hardmax -- the dictionary pre-compute.  "Flash PD-SSM:
//    Memory-Optimized Structured Sparse State-Space Models" (Technical
//    Summary, Methodology, "1. Novel Selection Mechanism (Hard Selection)"):
//    the structured matrices come from dense N x N matrices by a column-wise
//    hardmax, leaving one non-zero per column -- the index map dict_idx.
//  * pdssm_decode_step -- one new token per sequence: x <- P (d * x) + b,
//    y = Re(c . x), O(N) work and constant memory per step (the recurrent
//    inference mode the same summary names for state-space models, Problem
//    Statement).
//
// Both are bound by launch latency and HBM streaming, not by arithmetic.
#include <hip/hip_runtime.h>

#include "pdssm.h"
#include "pdssm_device.h"
#include "pdssm_host.h"

namespace pdssm {
namespace {

// ---------------------------------------------------------------------------
// Column-wise hardmax.  One wave per matrix, lane j = column j: rows are read
// in order (a row of N values is contiguous, so each read is one coalesced
// row), every lane keeping its column's running argmax under the selection's
// rule (first maximum, NaN above every number).  Rows are fetched kHmRows at
// a time so that several loads are in flight per wave.
// ---------------------------------------------------------------------------
constexpr int kHmWaves = 4;
#ifndef PDSSM_HM_ROWS
#define PDSSM_HM_ROWS 16
#endif
constexpr int kHmRows = PDSSM_HM_ROWS;

template <bool BF16>
__global__ void __launch_bounds__(kHmWaves * 64) hardmax_kernel(const void *__restrict__ m,
                                                               int32_t *__restrict__ out, int64_t mats,
                                                               int N)
{
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int64_t mat = (int64_t)blockIdx.x * kHmWaves + wave;
    if (mat >= mats)
        return;
    const int col = min(lane, N - 1);
    const int64_t base = mat * (int64_t)N * N + col;
    auto value = [&](int r) -> float {
        const int64_t e = base + (int64_t)r * N;
        if constexpr (BF16)
            return bf16_lo(reinterpret_cast<const uint16_t *>(m)[e]);
        else
            return reinterpret_cast<const float *>(m)[e];
    };
    float bv = value(0);
    int bk = 0;
    for (int r0 = 1; r0 < N; r0 += kHmRows) {
        float v[kHmRows];
#pragma unroll
        for (int u = 0; u < kHmRows; ++u)
            v[u] = value(min(r0 + u, N - 1));
#pragma unroll
        for (int u = 0; u < kHmRows; ++u)
            if (r0 + u < N)
                argmax_take(v[u], r0 + u, bv, bk);
    }
    if (lane < N)
        out[mat * N + lane] = bk;
}

// ---------------------------------------------------------------------------
// Decode step.  One wave per sequence, lane = state.  The step's entry is
// chosen like a scan step (argmax of its K scores over the wave's lanes, or
// the stored index); source j adds d[j] x[j] into row pi[j] of a per-wave
// LDS vector with float atomics (collisions sum in any order), then row i
// adds b[i], writes the new state over the old one and the rows' readout
// terms are summed across the wave.  Every read of the old state precedes
// the wave's first LDS atomic, so updating x in place is safe.
// ---------------------------------------------------------------------------
constexpr int kDecWaves = 4;

struct DecodeArgs {
    const void *sel;
    const int32_t *dict;
    const float *diag;
    const void *b, *c;
    void *y;
    float *x;
    int64_t S, H;
    int N, K;
    uint32_t sel_mode;
    int y_bf16;
};

__device__ __forceinline__ float wave_sum(float v)
{
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1)
        v += __shfl_xor(v, m, 64);
    return v;
}

template <bool CPLX, bool BCBF>
__global__ void __launch_bounds__(kDecWaves * 64) decode_kernel(DecodeArgs a)
{
    __shared__ int16_t s_sel[kDecWaves][2];
    __shared__ float s_acc[kDecWaves][64][2];
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
    const int64_t seq = (int64_t)blockIdx.x * kDecWaves + wave;
    if (seq >= a.S)
        return;
    const int N = a.N;
    const bool act = lane < N;
    const int64_t e = seq * N + (act ? lane : 0);
    // the old state and this step's rows; padding lanes hold zero
    cf x = {0.f, 0.f}, d = {0.f, 0.f}, bb = {0.f, 0.f}, cc = {0.f, 0.f};
    if (act) {
        x = load_diag<CPLX>(a.x, e);
        d = load_diag<CPLX>(a.diag, e);
        bb = load_vec<CPLX, BCBF>(a.b, e);
        cc = load_vec<CPLX, BCBF>(a.c, e);
    }
    wave_select<1>(a.sel, a.sel_mode, a.K, 1, seq, 0, s_sel[wave], lane);
    const int k = __builtin_amdgcn_readfirstlane((int)s_sel[wave][0]);
    const int64_t h = seq % a.H;
    const int pi = act ? (int)min((unsigned)a.dict[(h * a.K + k) * N + lane], (unsigned)(N - 1)) : lane;
    const cf v = cmul(d, x);
    s_acc[wave][lane][0] = 0.f;
    s_acc[wave][lane][1] = 0.f;
    if (act) {
        atomicAdd(&s_acc[wave][pi][0], v.r);
        if constexpr (CPLX)
            atomicAdd(&s_acc[wave][pi][1], v.i);
    }
    cf xn = {s_acc[wave][lane][0] + bb.r, CPLX ? s_acc[wave][lane][1] + bb.i : 0.f};
    if (!act)
        xn = {0.f, 0.f};
    if (act) {
        if constexpr (CPLX)
            reinterpret_cast<float2 *>(a.x)[e] = make_float2(xn.r, xn.i);
        else
            a.x[e] = xn.r;
    }
    const float yv = wave_sum(cc.r * xn.r - cc.i * xn.i);
    if (lane == 0) {
        if (a.y_bf16)
            reinterpret_cast<uint16_t *>(a.y)[seq] = f32_to_bf16_rne(yv);
        else
            reinterpret_cast<float *>(a.y)[seq] = yv;
    }
}

}  // namespace
}  // namespace pdssm

using namespace pdssm;

extern "C" int pdssm_dict_hardmax(const void *m, int32_t *dict_idx, int64_t H, int32_t K, int32_t N,
                                  uint32_t flags, hipStream_t stream)
{
    const int rc = check_dims(1, H, 1, N, K);
    if (rc != PDSSM_OK)
        return rc;
    const uint32_t mode = flags & PDSSM_SEL_MASK;
    if ((flags & ~PDSSM_SEL_MASK) || (mode != PDSSM_LOGITS_F32 && mode != PDSSM_LOGITS_BF16))
        return PDSSM_ERR_FLAGS;
    if (H == 0)
        return PDSSM_OK;
    if (!m || !dict_idx)
        return PDSSM_ERR_NULL;
    if (!aligned16(m) || !aligned16(dict_idx))
        return PDSSM_ERR_ALIGN;
    const int64_t mats = H * (int64_t)K;
    const dim3 grid((unsigned)((mats + kHmWaves - 1) / kHmWaves)), block(kHmWaves * 64);
    if (mode == PDSSM_LOGITS_BF16)
        hipLaunchKernelGGL(hardmax_kernel<true>, grid, block, 0, stream, m, dict_idx, mats, (int)N);
    else
        hipLaunchKernelGGL(hardmax_kernel<false>, grid, block, 0, stream, m, dict_idx, mats, (int)N);
    return hip_status(hipGetLastError());
}

extern "C" int pdssm_decode_step(const void *sel_or_logits, const int32_t *dict_idx, const void *diag,
                                 const void *b, const void *c, void *y, void *x, int64_t B, int64_t H,
                                 int32_t N, int32_t K, uint32_t flags, hipStream_t stream)
{
    const int rc = check_dims(B, H, 1, N, K);
    if (rc != PDSSM_OK)
        return rc;
    if (flags & ~PDSSM_FLAGS_ALL)
        return PDSSM_ERR_FLAGS;
    if (B == 0 || H == 0)
        return PDSSM_OK;
    if (!sel_or_logits || !dict_idx || !diag || !b || !c || !y || !x)
        return PDSSM_ERR_NULL;
    const void *ptrs[] = {sel_or_logits, dict_idx, diag, b, c, y, x};
    for (const void *p : ptrs)
        if (!aligned16(p))
            return PDSSM_ERR_ALIGN;
    DecodeArgs a;
    a.sel = sel_or_logits;
    a.dict = dict_idx;
    a.diag = static_cast<const float *>(diag);
    a.b = b;
    a.c = c;
    a.y = y;
    a.x = static_cast<float *>(x);
    a.S = B * H;
    a.H = H;
    a.N = N;
    a.K = K;
    a.sel_mode = flags & PDSSM_SEL_MASK;
    a.y_bf16 = (flags & PDSSM_Y_BF16) ? 1 : 0;
    const dim3 grid((unsigned)((a.S + kDecWaves - 1) / kDecWaves)), block(kDecWaves * 64);
    const bool cplx = flags & PDSSM_COMPLEX, bcbf = flags & PDSSM_BC_BF16;
    if (cplx && bcbf)
        hipLaunchKernelGGL((decode_kernel<true, true>), grid, block, 0, stream, a);
    else if (cplx)
        hipLaunchKernelGGL((decode_kernel<true, false>), grid, block, 0, stream, a);
    else if (bcbf)
        hipLaunchKernelGGL((decode_kernel<false, true>), grid, block, 0, stream, a);
    else
        hipLaunchKernelGGL((decode_kernel<false, false>), grid, block, 0, stream, a);
    return hip_status(hipGetLastError());
}
