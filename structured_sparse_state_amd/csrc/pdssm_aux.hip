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
// Column-wise hardmax.  One workgroup per matrix, lane j = column j; the
// kHmWaves waves take consecutive blocks of at most kHmRows rows (a row of N
// values is contiguous, so each read is one coalesced row) and issue all of
// their rows' loads at once.  Each wave keeps its columns' running argmax
// over its rows in order under the selection's rule (first maximum, NaN
// above every number); the first wave then merges the waves' results in
// row order under the same rule, which keeps the first maximum over the
// whole column.
// ---------------------------------------------------------------------------
constexpr int kHmWaves = 4;
constexpr int kHmRows = 16;   // rows per wave: N <= 64
static_assert(kHmWaves * kHmRows >= 64, "the waves cover every row");

template <bool BF16>
__global__ void __launch_bounds__(kHmWaves * 64) hardmax_kernel(const void *__restrict__ m,
                                                               int32_t *__restrict__ out, int64_t mats,
                                                               int N)
{
    __shared__ float s_v[kHmWaves][64];
    __shared__ int s_k[kHmWaves][64];
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int col = min(lane, N - 1);
    const int rows = (N + kHmWaves - 1) / kHmWaves;   // <= kHmRows
    const int r0 = wave * rows, r1 = min(N, r0 + rows);
    // Matrices blockIdx.x, + gridDim.x, ... (the whole workgroup loops).
    for (int64_t mat = blockIdx.x; mat < mats; mat += gridDim.x) {
        const int64_t base = mat * (int64_t)N * N + col;
        auto value = [&](int r) -> float {
            const int64_t e = base + (int64_t)r * N;
            if constexpr (BF16)
                return bf16_lo(reinterpret_cast<const uint16_t *>(m)[e]);
            else
                return reinterpret_cast<const float *>(m)[e];
        };
        float bv = 0.f;
        int bk = -1;   // no rows in this wave's block
        if (r0 < r1) {
            float v[kHmRows];
#pragma unroll
            for (int u = 0; u < kHmRows; ++u)
                v[u] = value(min(r0 + u, r1 - 1));
            bv = v[0];
            bk = r0;
#pragma unroll
            for (int u = 1; u < kHmRows; ++u)
                if (r0 + u < r1)
                    argmax_take(v[u], r0 + u, bv, bk);
        }
        s_v[wave][lane] = bv;
        s_k[wave][lane] = bk;
        __syncthreads();
        if (wave == 0) {
#pragma unroll
            for (int w = 1; w < kHmWaves; ++w)
                if (s_k[w][lane] >= 0)
                    argmax_take(s_v[w][lane], s_k[w][lane], bv, bk);
            if (lane < N)
                out[mat * N + lane] = bk;
        }
        __syncthreads();   // the merge has read s_v, s_k before the next matrix
    }
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
    // One workgroup per matrix (at most 2^20 workgroups, each then taking
    // several matrices).
    const dim3 grid((unsigned)(mats < (1 << 20) ? mats : (1 << 20))), block(kHmWaves * 64);
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
