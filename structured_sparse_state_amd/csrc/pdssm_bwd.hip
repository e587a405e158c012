// pdssm_bwd.hip -- gradients of the Flash PD-SSM scan (the backward pass) for
// MI355X (gfx950).
//
// The forward recurrence ("Flash PD-SSM: Memory-Optimized Structured Sparse
// State-Space Models", gist.science explainer, Technical Summary,
// Methodology sections 1 and 3) is
//     x_t = A_t x_{t-1} + b_t,   A_t = P_t D_t,   y_t = Re(sum_i c_t[i] x_t[i]).
// Training runs it backwards.  The selection is a hard argmax and gets no
// gradient here (the pages train the scores through a straight-through
// estimator whose formula they do not print).  For a real loss with dL/dy_t =
// gy_t and dL/dx_final = gxf, and complex gradients written dL/dRe + i dL/dIm:
//     lambda_{L-1} = gy_{L-1} conj(c_{L-1}) + gxf
//     lambda_t     = gy_t conj(c_t) + A_{t+1}^H lambda_{t+1}
//     gb_t = lambda_t,  gc_t = gy_t conj(x_t),
//     gd_t[j] = conj(x_{t-1}[j]) lambda_t[pi_t[j]],  gx0 = A_0^H lambda_0.
// A^H is a gather, (A^H l)[j] = conj(d[j]) l[pi[j]] -- the transpose of the
// forward's one-hot column scatter -- so the adjoint needs no collision
// handling at all.
//
// Chunks of 16 steps.  With K_c the adjoint carried into chunk c's last step
// (K = gxf after the last chunk, and A_0^H lambda_0 = gx0 before the first):
//     K_{c-1} = M_c K_c + v_c,   M_c = (A_e ... A_s)^H,
// and M_c is the conjugate transpose of the chunk's forward operator: in
// gather form (M K)[j] = conj(dacc[j]) K[pacc[j]], with (pacc, dacc) the
// forward path of source j through the chunk.  Its affine part is
//     v_c[j] = sum_t gy_t conj(c_t[pacc_t[j]] dacc_t[j]),
// a sum of the forward's own readout weights.  Three kernels:
//   bwd_ops    per chunk, in parallel: (pacc, conj(dacc), v_c), by gathers.
//   bwd_carry  per sequence: K_c for every chunk, right to left.
//   bwd_grad   per chunk, in parallel: x over the chunk from the forward's
//              saved carry-in (the forward's scatter step), then lambda back
//              over it from K_c, writing gb, gc and gd.
#include <hip/hip_runtime.h>

#include "pdssm.h"
#include "pdssm_device.h"
#include "pdssm_host.h"

namespace pdssm {

constexpr int kBT = kCarryStride;   // steps per chunk (the forward saves one carry per chunk)
constexpr int kBW = 4;              // chunk waves per workgroup
constexpr int kCarryRing = 8;       // chunk records in flight in bwd_carry

struct BwdArgs {
    const void *sel;
    const int32_t *dict;
    const float *diag;
    const void *b;
    const void *c;
    const float *xch;   // [S][nch][N(,2)] state before each chunk (from the forward)
    const void *gy;     // [S][L], the y storage type
    const float *gxf;   // [S][N(,2)] or null
    void *gb;           // storage of b
    void *gc;           // storage of c
    float *gd;          // storage of diag
    float *gx0;         // [S][N(,2)] or null
    const uint16_t *tab;   // [H][K][64] scatter entries (dict_entry)
    int32_t *sig;       // [S*nch][64] composed map of each chunk
    float4 *mv;         // [S*nch][64] (conj dacc, v)
    float2 *kc;         // [S*nch][64] adjoint carried into each chunk's last step
    int64_t H, L, S, nch;
    int N, K;
    uint32_t sel_mode;
    int y_bf16;
};

template <bool CPLX>
__device__ __forceinline__ void store_grad(float *p, int64_t e, cf v)
{
    if constexpr (CPLX)
        reinterpret_cast<float2 *>(p)[e] = make_float2(v.r, v.i);
    else
        p[e] = v.r;
}

// A gradient in the storage of b or c (bf16, rounded to nearest even, or fp32).
template <bool CPLX, bool BF16>
__device__ __forceinline__ void store_vec(void *p, int64_t e, cf v)
{
    if constexpr (BF16) {
        if constexpr (CPLX)
            reinterpret_cast<uint32_t *>(p)[e] =
                (uint32_t)f32_to_bf16_rne(v.r) | ((uint32_t)f32_to_bf16_rne(v.i) << 16);
        else
            reinterpret_cast<uint16_t *>(p)[e] = f32_to_bf16_rne(v.r);
    } else {
        store_grad<CPLX>(reinterpret_cast<float *>(p), e, v);
    }
}

__device__ __forceinline__ float load_gy(const BwdArgs &a, int64_t step)
{
    if (a.y_bf16)
        return bf16_lo(reinterpret_cast<const uint16_t *>(a.gy)[step]);
    return reinterpret_cast<const float *>(a.gy)[step];
}

// ---------------------------------------------------------------------------
// The scatter entries for 64 lanes (one wave per dictionary entry).
// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(256) bwd_tab_kernel(const int32_t *dict, uint16_t *tab, int64_t entries, int N)
{
    const int64_t e = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (e >= entries)
        return;
    const int lane = threadIdx.x & 63;
    tab[e * 64 + lane] = dict_entry(dict + e * N, N, lane);
}

// ---------------------------------------------------------------------------
// bwd_ops: per chunk, lane j follows its forward path (pacc, dacc) through
// the chunk and sums the adjoint's affine part v[j].
// ---------------------------------------------------------------------------
template <bool CPLX, bool BCBF>
__global__ void __launch_bounds__(kBW * 64) bwd_ops_kernel(BwdArgs a)
{
    __shared__ int16_t s_sel[kBW][kBT];
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
    const int64_t ch = (int64_t)blockIdx.x * kBW + wave;
    if (ch >= a.S * a.nch)
        return;
    const int64_t seq = ch / a.nch;
    const int64_t t0 = (ch - seq * a.nch) * kBT;
    const int nv = (int)min((int64_t)kBT, a.L - t0);
    const int64_t h = seq % a.H;
    const int N = a.N, K = a.K;
    wave_select<kBT>(a.sel, a.sel_mode, K, a.L, seq * a.L, t0, s_sel[wave], lane);
    const bool act = lane < N;
    int pacc4 = lane * 4;
    cf dacc = {1.f, 0.f}, v = {0.f, 0.f};
    for (int tt = 0; tt < nv; ++tt) {
        const int64_t step = seq * a.L + t0 + tt;
        const int k = s_sel[wave][tt];
        const int pi = act ? (int)min((unsigned)a.dict[(h * K + k) * N + lane], (unsigned)(N - 1)) : lane;
        const cf d = act ? load_diag<CPLX>(a.diag, step * N + lane) : cf{1.f, 0.f};
        const cf cv = act ? load_vec<CPLX, BCBF>(a.c, step * N + lane) : cf{0.f, 0.f};
        const float g = load_gy(a, step);
        // pacc_t = pi_t[pacc_{t-1}], dacc_t = d_t[pacc_{t-1}] * dacc_{t-1}
        const int np = (int)bperm_a((uint32_t)pi, pacc4);
        cf dd;
        dd.r = bperm_a(d.r, pacc4);
        dd.i = CPLX ? bperm_a(d.i, pacc4) : 0.f;
        dacc = cmul(dd, dacc);
        pacc4 = np * 4;
        // readout weight g_t[j] = c_t[pacc_t[j]] dacc_t[j]; v += gy_t conj(g_t)
        cf cg;
        cg.r = bperm_a(cv.r, pacc4);
        cg.i = CPLX ? bperm_a(cv.i, pacc4) : 0.f;
        const cf w = cmul(cg, dacc);
        v.r += g * w.r;
        v.i -= g * w.i;
    }
    a.sig[ch * 64 + lane] = pacc4 >> 2;
    a.mv[ch * 64 + lane] = make_float4(dacc.r, -dacc.i, v.r, v.i);
}

// ---------------------------------------------------------------------------
// bwd_carry: per sequence (one wave, lane = state), right to left over the
// chunks: record K_c, then K_{c-1} = conj(dacc) K_c[pacc] + v_c.  The chunk
// records do not depend on K, so a ring of them is in flight ahead.
// ---------------------------------------------------------------------------
template <bool CPLX>
__global__ void __launch_bounds__(kBW * 64) bwd_carry_kernel(BwdArgs a)
{
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
    const int64_t seq = (int64_t)blockIdx.x * kBW + wave;
    if (seq >= a.S)
        return;
    const bool act = lane < a.N;
    cf kk = {0.f, 0.f};
    if (a.gxf && act)
        kk = load_diag<CPLX>(a.gxf, seq * a.N + lane);
    const int64_t nch = a.nch, base = seq * nch;
    int32_t sg[kCarryRing];
    float4 mv[kCarryRing];
#pragma unroll
    for (int r = 0; r < kCarryRing; ++r) {
        const int64_t c = max(nch - 1 - r, (int64_t)0);
        sg[r] = a.sig[(base + c) * 64 + lane];
        mv[r] = a.mv[(base + c) * 64 + lane];
    }
    for (int64_t c0 = nch - 1; c0 >= 0; c0 -= kCarryRing) {
#pragma unroll
        for (int r = 0; r < kCarryRing; ++r) {
            const int64_t c = c0 - r;
            if (c < 0)
                break;
            a.kc[(base + c) * 64 + lane] = make_float2(kk.r, kk.i);
            const int src = sg[r];
            const float4 m = mv[r];
            // the record kCarryRing chunks further left, into this slot
            const int64_t cn = max(c - kCarryRing, (int64_t)0);
            sg[r] = a.sig[(base + cn) * 64 + lane];
            mv[r] = a.mv[(base + cn) * 64 + lane];
            cf kg;
            kg.r = bperm(kk.r, src);
            kg.i = CPLX ? bperm(kk.i, src) : 0.f;
            kk = {m.x * kg.r - m.y * kg.i + m.z, CPLX ? m.x * kg.i + m.y * kg.r + m.w : 0.f};
        }
    }
    if (a.gx0 && act)
        store_grad<CPLX>(a.gx0, seq * a.N + lane, kk);
}

// ---------------------------------------------------------------------------
// bwd_grad: per chunk (one wave, lane = state).  The states x_t of the chunk
// by the forward's collision-free scatter from the saved carry-in (kept in
// registers), then lambda backwards from K_c by gathers.
// ---------------------------------------------------------------------------
template <bool CPLX, bool BCBF>
__global__ void __launch_bounds__(kBW * 64) bwd_grad_kernel(BwdArgs a)
{
    __shared__ int16_t s_sel[kBW][kBT];
    __shared__ __attribute__((aligned(16))) cf s_reg[kBW][kBlocks][64];
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
    const int64_t ch = (int64_t)blockIdx.x * kBW + wave;
    if (ch >= a.S * a.nch)
        return;
    const int64_t seq = ch / a.nch;
    const int64_t t0 = (ch - seq * a.nch) * kBT;
    const int nv = (int)min((int64_t)kBT, a.L - t0);
    const int64_t h = seq % a.H;
    const int N = a.N, K = a.K;
    const bool act = lane < N;
#pragma unroll
    for (int r = kRegions; r < 2 * kRegions; ++r)
        s_reg[wave][r][lane] = cf{0.f, 0.f};
    wave_select<kBT>(a.sel, a.sel_mode, K, a.L, seq * a.L, t0, s_sel[wave], lane);
    char *const regp = reinterpret_cast<char *>(&s_reg[wave][0][0]);
    const char *const rowbase = regp + lane * (int)sizeof(cf);
    const uint16_t *const tab_h = a.tab + h * (int64_t)K * 64 + lane;

    // The inputs of step tt of the chunk (clamped to its last step, so every
    // load is in range), two steps ahead of their use.
    struct In {
        cf d, bb, cv;
        float g;
        uint32_t ent;
    };
    auto load_in = [&](int tt, bool with_b) -> In {
        const int ts = max(0, min(tt, nv - 1));
        const int64_t step = seq * a.L + t0 + ts;
        const int64_t e = step * N + (act ? lane : N - 1);
        In r;
        r.ent = tab_h[(int)s_sel[wave][ts] * 64];
        r.d = load_diag<CPLX>(a.diag, e);
        r.bb = with_b ? load_vec<CPLX, BCBF>(a.b, e) : cf{0.f, 0.f};
        r.cv = load_vec<CPLX, BCBF>(a.c, e);
        r.g = load_gy(a, step);
        return r;
    };

    // ---- x over the chunk: x_t = P_t (d_t * x_{t-1}) + b_t
    cf xin = {0.f, 0.f};
    if (act)
        xin = load_diag<CPLX>(a.xch, ch * N + lane);
    cf xs[kBT];
    cf x = xin;
    In ring[2] = {load_in(0, true), load_in(1, true)};
#pragma unroll
    for (int tt = 0; tt < kBT; ++tt) {
        if (tt < nv) {
            const In in = ring[tt & 1];
            ring[tt & 1] = load_in(tt + 2, true);
            const int64_t step = seq * a.L + t0 + tt;
            const cf v = cmul(in.d, x);
            const uint32_t slot = (in.ent & 0x1FFu) << 3;
            *static_cast<float2 *>(__builtin_assume_aligned(regp + slot, 8)) = make_float2(v.r, v.i);
            lds_order();
            if (__any(slot >= kSpareOff)) {
                if (slot >= kSpareOff) {
                    cf *o = reinterpret_cast<cf *>(regp + (slot - kSpareOff));
                    lds_add(&o->r, v.r);
                    if constexpr (CPLX)
                        lds_add(&o->i, v.i);
                }
                lds_order();
            }
            const char *rowp = rowbase + (in.ent & 0x600u);
            cf sum = in.bb;
#pragma unroll
            for (int r = 0; r < kRegions; ++r) {
                const float2 u = *static_cast<const float2 *>(__builtin_assume_aligned(rowp + r * kRegionBytes, 8));
                sum.r += u.x;
                sum.i += u.y;
            }
            lds_order();
            x = sum;
            xs[tt] = x;
            if (act)
                store_vec<CPLX, BCBF>(a.gc, step * N + lane, cf{in.g * x.r, -in.g * x.i});
        }
    }

    // ---- lambda back over the chunk
    const float2 k0 = a.kc[ch * 64 + lane];
    cf lc = {k0.x, k0.y};   // A_{t+1}^H lambda_{t+1}, the part carried into step t
    ring[0] = load_in(nv - 1, false);
    ring[1] = load_in(nv - 2, false);
#pragma unroll
    for (int tt = kBT - 1; tt >= 0; --tt) {
        if (tt < nv) {
            const int q = (nv - 1 - tt) & 1;   // ring slot of step tt
            const In in = ring[q];
            ring[q] = load_in(tt - 2, false);
            const int64_t step = seq * a.L + t0 + tt;
            const cf lam = {lc.r + in.g * in.cv.r, lc.i - in.g * in.cv.i};
            const int pi = (int)(in.ent & 63u);
            cf lg;
            lg.r = bperm(lam.r, pi);
            lg.i = CPLX ? bperm(lam.i, pi) : 0.f;
            const cf xp = (tt > 0) ? xs[tt > 0 ? tt - 1 : 0] : xin;
            if (act) {
                store_vec<CPLX, BCBF>(a.gb, step * N + lane, lam);
                store_grad<CPLX>(a.gd, step * N + lane, cf{xp.r * lg.r + xp.i * lg.i, xp.r * lg.i - xp.i * lg.r});
            }
            lc = {in.d.r * lg.r + in.d.i * lg.i, in.d.r * lg.i - in.d.i * lg.r};
        }
    }
}

// ---------------------------------------------------------------------------
// Host side.
// ---------------------------------------------------------------------------
struct BwdLayout {
    int64_t nch, S, tab_bytes, sig_bytes, mv_bytes, kc_bytes, total;
};

static BwdLayout bwd_layout(int64_t B, int64_t H, int64_t L, int32_t K)
{
    BwdLayout lo;
    lo.S = B * H;
    lo.nch = (L + kBT - 1) / kBT;
    const int64_t chunks = lo.S * lo.nch;
    auto up = [](int64_t n) { return (n + 255) / 256 * 256; };
    lo.tab_bytes = up(H * (int64_t)K * 64 * 2);
    lo.sig_bytes = up(chunks * 64 * 4);
    lo.mv_bytes = up(chunks * 64 * 16);
    lo.kc_bytes = up(chunks * 64 * 8);
    lo.total = lo.tab_bytes + lo.sig_bytes + lo.mv_bytes + lo.kc_bytes;
    return lo;
}

template <bool CPLX, bool BCBF>
static void launch_bwd(const BwdArgs &a, hipStream_t st)
{
    const int64_t chunks = a.S * a.nch;
    const dim3 blk(kBW * 64);
    hipLaunchKernelGGL((bwd_ops_kernel<CPLX, BCBF>), dim3((unsigned)((chunks + kBW - 1) / kBW)), blk, 0, st, a);
    hipLaunchKernelGGL((bwd_carry_kernel<CPLX>), dim3((unsigned)((a.S + kBW - 1) / kBW)), blk, 0, st, a);
    hipLaunchKernelGGL((bwd_grad_kernel<CPLX, BCBF>), dim3((unsigned)((chunks + kBW - 1) / kBW)), blk, 0, st, a);
}

}  // namespace pdssm

using namespace pdssm;

extern "C" size_t pdssm_scan_bwd_workspace_bytes(int64_t B, int64_t H, int64_t L, int32_t N,
                                                 int32_t K, uint32_t flags)
{
    if (check_dims(B, H, L, N, K) != PDSSM_OK || (flags & ~PDSSM_FLAGS_ALL))
        return 0;
    return (size_t)bwd_layout(B, H, L, K).total;
}

extern "C" int pdssm_scan_bwd(const void *sel_or_logits, const int32_t *dict_idx, const void *diag,
                              const void *b, const void *c, const void *x_chunks, const void *gy,
                              const void *gx_final, void *gb, void *gc, void *gd, void *gx0,
                              int64_t B, int64_t H, int64_t L, int32_t N, int32_t K, uint32_t flags,
                              void *workspace, size_t workspace_bytes, hipStream_t stream)
{
    if (!sel_or_logits || !dict_idx || !diag || !b || !c || !x_chunks || !gy || !gb || !gc || !gd ||
        !workspace)
        return PDSSM_ERR_NULL;
    int rc = check_dims(B, H, L, N, K);
    if (rc != PDSSM_OK)
        return rc;
    if (flags & ~PDSSM_FLAGS_ALL)
        return PDSSM_ERR_FLAGS;
    const void *ptrs[] = {sel_or_logits, dict_idx, diag, b, c, x_chunks, gy, gx_final, gb, gc, gd, gx0,
                          workspace};
    for (const void *p : ptrs)
        if (p && !aligned16(p))
            return PDSSM_ERR_ALIGN;
    const BwdLayout lo = bwd_layout(B, H, L, K);
    if (workspace_bytes < (size_t)lo.total)
        return PDSSM_ERR_WORKSPACE;

    BwdArgs a;
    a.sel = sel_or_logits;
    a.dict = dict_idx;
    a.diag = static_cast<const float *>(diag);
    a.b = b;
    a.c = c;
    a.xch = static_cast<const float *>(x_chunks);
    a.gy = gy;
    a.gxf = static_cast<const float *>(gx_final);
    a.gb = gb;
    a.gc = gc;
    a.gd = static_cast<float *>(gd);
    a.gx0 = static_cast<float *>(gx0);
    char *w = static_cast<char *>(workspace);
    a.tab = reinterpret_cast<uint16_t *>(w);
    a.sig = reinterpret_cast<int32_t *>(w + lo.tab_bytes);
    a.mv = reinterpret_cast<float4 *>(w + lo.tab_bytes + lo.sig_bytes);
    a.kc = reinterpret_cast<float2 *>(w + lo.tab_bytes + lo.sig_bytes + lo.mv_bytes);
    a.H = H;
    a.L = L;
    a.S = lo.S;
    a.nch = lo.nch;
    a.N = N;
    a.K = K;
    a.sel_mode = flags & PDSSM_SEL_MASK;
    a.y_bf16 = (flags & PDSSM_Y_BF16) ? 1 : 0;

    const int64_t entries = H * (int64_t)K;
    hipLaunchKernelGGL(bwd_tab_kernel, dim3((unsigned)((entries + 3) / 4)), dim3(256), 0, stream, dict_idx,
                       const_cast<uint16_t *>(a.tab), entries, N);
    const bool cplx = flags & PDSSM_COMPLEX, bcbf = flags & PDSSM_BC_BF16;
    if (cplx)
        bcbf ? launch_bwd<true, true>(a, stream) : launch_bwd<true, false>(a, stream);
    else
        bcbf ? launch_bwd<false, true>(a, stream) : launch_bwd<false, false>(a, stream);
    return hip_status(hipGetLastError());
}
