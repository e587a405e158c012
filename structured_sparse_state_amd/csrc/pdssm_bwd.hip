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

#include <type_traits>

#include "pdssm.h"
#include "pdssm_device.h"
#include "pdssm_host.h"

namespace pdssm {

constexpr int kBT = kCarryStride;   // steps per chunk (the forward saves one carry per chunk)
constexpr int kBW = 4;              // chunk waves per workgroup
#ifndef PDSSM_BWD_GRAD_D
#define PDSSM_BWD_GRAD_D 4   // steps of input in flight per wave (gradient kernel)
#endif

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
    int32_t *gsig;      // [S*ng][64] group operators (ng = ceil(nch / kGroup))
    float4 *gmv;
    float2 *gk;         // [S*ng][64] adjoint carried into each group's last chunk
    int16_t *ksel;      // [S*L] selections picked by bwd_ops from logits (logits modes only)
    int64_t H, L, S, nch;
    int N, K;
    uint32_t sel_mode;
    int y_bf16;
    int idx32;          // chunk and sequence counts fit 31 bits: 32-bit index arithmetic
};

// Sequence and first step of chunk ch, and the sequence's head.  The
// divisions are 32-bit when the counts allow (a 64-bit one costs a few
// hundred instructions before the chunk's first load can go out).
struct ChunkPos {
    int64_t seq, t0, h;
};
__device__ __forceinline__ ChunkPos chunk_of(const BwdArgs &a, int64_t ch)
{
    ChunkPos p;
    if (a.idx32) {
        const uint32_t c = (uint32_t)ch, n = (uint32_t)a.nch;
        const uint32_t sq = c / n;
        p.seq = sq;
        p.t0 = (int64_t)(c - sq * n) * kBT;
        p.h = sq % (uint32_t)a.H;
    } else {
        p.seq = ch / a.nch;
        p.t0 = (ch - p.seq * a.nch) * kBT;
        p.h = p.seq % a.H;
    }
    return p;
}

template <bool CPLX>
__device__ __forceinline__ void store_grad(float *p, int64_t e, cf v)
{
    if constexpr (CPLX)
        reinterpret_cast<float2 *>(p)[e] = make_float2(v.r, v.i);
    else
        p[e] = v.r;
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
// Loads and stores of one chunk's rows through buffer resources: the rows of
// the chunk start at the resource base, the row offset of a step is
// wave-uniform (scalar), the lane offset is fixed.  Padding lanes (>= N) get
// an offset past every resource, so their loads read 0 and their stores are
// dropped by the hardware -- no branches.
// ---------------------------------------------------------------------------
constexpr uint32_t kOffLane = 0x80000000u;

// b and c as loaded: bf16 words stay packed (a pair when complex).
template <bool CPLX, bool BCBF>
struct RawOf {
    using type = typename std::conditional<BCBF, uint32_t, typename std::conditional<CPLX, float2, float>::type>::type;
};

template <bool CPLX, bool BCBF>
__device__ __forceinline__ cf unpack_c(typename RawOf<CPLX, BCBF>::type v)
{
    if constexpr (BCBF)
        return {bf16_lo(v), CPLX ? bf16_hi(v) : 0.f};
    else if constexpr (CPLX)
        return {v.x, v.y};
    else
        return {v, 0.f};
}

// The raw value of the lane at byte address addr (4 * lane).
template <bool CPLX, bool BCBF>
__device__ __forceinline__ typename RawOf<CPLX, BCBF>::type bperm_raw(typename RawOf<CPLX, BCBF>::type v, int addr)
{
    if constexpr (BCBF)
        return bperm_a((uint32_t)v, addr);
    else if constexpr (CPLX)
        return make_float2(bperm_a(v.x, addr), bperm_a(v.y, addr));
    else
        return bperm_a(v, addr);
}

template <bool CPLX, bool BCBF>
struct ChunkIO {
    using DRaw = typename std::conditional<CPLX, float2, float>::type;
    using Stored = typename std::conditional<BCBF, typename std::conditional<CPLX, uint32_t, uint16_t>::type,
                                             DRaw>::type;
    __amdgpu_buffer_rsrc_t rd, rb, rc, rt;
    uint32_t vd, vs, vt;   // lane offsets (bytes) into diag-like, b/c-like rows and the entry table
    int N;

    __device__ void init(const BwdArgs &a, int64_t seq, int64_t t0, int nv, int64_t h, int lane)
    {
        N = a.N;
        const int64_t e0 = (seq * a.L + t0) * a.N;   // first element of the chunk
        const uint64_t rows = (uint64_t)nv * (uint64_t)a.N;
        rd = make_rsrc(reinterpret_cast<const DRaw *>(a.diag) + e0, rows * sizeof(DRaw));
        rb = make_rsrc(reinterpret_cast<const Stored *>(a.b) + e0, rows * sizeof(Stored));
        rc = make_rsrc(reinterpret_cast<const Stored *>(a.c) + e0, rows * sizeof(Stored));
        rt = make_rsrc(a.tab + h * (int64_t)a.K * 64, (uint64_t)a.K * 64 * 2);
        const bool act = lane < a.N;
        vd = act ? (uint32_t)(lane * sizeof(DRaw)) : kOffLane;
        vs = act ? (uint32_t)(lane * sizeof(Stored)) : kOffLane;
        vt = (uint32_t)(lane * 2);   // the table has all 64 lanes (padding maps to itself)
    }
    __device__ cf d(int tt) const
    {
        const DRaw v = bload<DRaw>(rd, vd, (uint32_t)(tt * N * (int)sizeof(DRaw)));
        if constexpr (CPLX)
            return {v.x, v.y};
        else
            return {v, 0.f};
    }
    __device__ typename RawOf<CPLX, BCBF>::type raw_b(int tt) const
    {
        return (typename RawOf<CPLX, BCBF>::type)bload<Stored>(rb, vs, (uint32_t)(tt * N * (int)sizeof(Stored)));
    }
    __device__ typename RawOf<CPLX, BCBF>::type raw_c(int tt) const
    {
        return (typename RawOf<CPLX, BCBF>::type)bload<Stored>(rc, vs, (uint32_t)(tt * N * (int)sizeof(Stored)));
    }
    __device__ uint32_t ent(int k) const { return bload<uint16_t>(rt, vt, (uint32_t)(k * 128)); }
};

// The chunk's 16 upstream gradients gy as stored (fp32 bits, or bf16 bits in
// the low half), one per lane (lanes 0..nv-1).  They are converted where a
// step uses them, so that the load stays in flight meanwhile.
__device__ __forceinline__ uint32_t chunk_gy_raw(const BwdArgs &a, int64_t step0, int nv, int lane)
{
    const int l = min(lane, nv - 1);
    if (a.y_bf16)
        return reinterpret_cast<const uint16_t *>(a.gy)[step0 + l];
    return reinterpret_cast<const uint32_t *>(a.gy)[step0 + l];
}

__device__ __forceinline__ float gy_step(const BwdArgs &a, uint32_t raw, int tt)
{
    const uint32_t r = (uint32_t)__builtin_amdgcn_readlane((int)raw, tt);
    return __uint_as_float(a.y_bf16 ? r << 16 : r);
}

// Index-mode selections of a chunk in two halves: sel_raw issues the load
// (lane l < nv reads step l of the chunk), sel_put stores the clamped index
// for the step's entry lookups once the chunk's row loads are also in flight.
__device__ __forceinline__ bool index_mode(uint32_t mode)
{
    return mode == PDSSM_SEL_I32 || mode == PDSSM_SEL_I16;
}

__device__ __forceinline__ int sel_raw(const void *src, uint32_t mode, int64_t row, int nv, int lane)
{
    if (lane >= nv)
        return 0;
    return mode == PDSSM_SEL_I32 ? reinterpret_cast<const int32_t *>(src)[row + lane]
                                 : reinterpret_cast<const int16_t *>(src)[row + lane];
}

__device__ __forceinline__ void sel_put(int k, int K, int nv, int16_t *out, int lane)
{
    if (lane < kBT)
        out[lane] = (int16_t)(lane < nv ? (int)min((unsigned)k, (unsigned)(K - 1)) : 0);
}

template <typename V>
__device__ __forceinline__ void bstore(__amdgpu_buffer_rsrc_t r, V v, uint32_t voff, uint32_t soff)
{
    if constexpr (sizeof(V) == 8) {
        typedef unsigned int u2 __attribute__((ext_vector_type(2)));
        u2 w;
        __builtin_memcpy(&w, &v, 8);
        __builtin_amdgcn_raw_buffer_store_b64(w, r, voff, soff, 0);
    } else if constexpr (sizeof(V) == 4) {
        uint32_t w;
        __builtin_memcpy(&w, &v, 4);
        __builtin_amdgcn_raw_buffer_store_b32(w, r, voff, soff, 0);
    } else {
        static_assert(sizeof(V) == 2, "2, 4 or 8 bytes");
        uint16_t w;
        __builtin_memcpy(&w, &v, 2);
        __builtin_amdgcn_raw_buffer_store_b16(w, r, voff, soff, 0);
    }
}

// A gradient in the raw storage of b or c (bf16 rounded to nearest even, or fp32).
template <bool CPLX, bool BCBF>
__device__ __forceinline__ typename ChunkIO<CPLX, BCBF>::Stored pack_vec(cf v)
{
    if constexpr (BCBF) {
        if constexpr (CPLX)
            return f32x2_to_bf16x2_rne(v.r, v.i);
        else
            return f32_to_bf16_rne(v.r);
    } else if constexpr (CPLX) {
        return make_float2(v.r, v.i);
    } else {
        return v.r;
    }
}

template <bool CPLX>
__device__ __forceinline__ typename std::conditional<CPLX, float2, float>::type pack_d(cf v)
{
    if constexpr (CPLX)
        return make_float2(v.r, v.i);
    else
        return v.r;
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
    const ChunkPos cp = chunk_of(a, ch);
    const int64_t seq = cp.seq, t0 = cp.t0, h = cp.h;
    const int nv = (int)min((int64_t)kBT, a.L - t0);
    // The chunk's d and c rows do not depend on the selection: all of them
    // are in flight before the selections are used.
    const bool idx = index_mode(a.sel_mode);
    int kraw = 0;
    if (idx)
        kraw = sel_raw(a.sel, a.sel_mode, seq * a.L + t0, nv, lane);
    const uint32_t gyr = chunk_gy_raw(a, seq * a.L + t0, nv, lane);
    ChunkIO<CPLX, BCBF> io;
    io.init(a, seq, t0, nv, h, lane);
    using Raw = typename RawOf<CPLX, BCBF>::type;
    cf rd[kBT];
    Raw rc[kBT];
#pragma unroll
    for (int tt = 0; tt < kBT; ++tt) {
        const int ts = min(tt, nv - 1);
        rd[tt] = io.d(ts);
        rc[tt] = io.raw_c(ts);
    }
    if (idx) {
        sel_put(kraw, a.K, nv, s_sel[wave], lane);
    } else {
        wave_select<kBT>(a.sel, a.sel_mode, a.K, a.L, seq * a.L, t0, s_sel[wave], lane);
        if (a.ksel && lane < nv)   // the gradient pass reads these instead of the K scores
            a.ksel[seq * a.L + t0 + lane] = s_sel[wave][lane];
    }
    uint32_t re[kBT];
#pragma unroll
    for (int tt = 0; tt < kBT; ++tt)
        re[tt] = io.ent(__builtin_amdgcn_readfirstlane((int)s_sel[wave][min(tt, nv - 1)]));
    int pacc4 = lane * 4;
    cf dacc = {1.f, 0.f}, v = {0.f, 0.f};
#pragma unroll
    for (int tt = 0; tt < kBT; ++tt) {
        const cf d = rd[tt];
        const Raw craw = rc[tt];
        const uint32_t ent = re[tt];
        if (tt < nv) {
            const float g = gy_step(a, gyr, tt);
            // pacc_t = pi_t[pacc_{t-1}], dacc_t = d_t[pacc_{t-1}] * dacc_{t-1}
            const uint32_t np = bperm_a(ent & 63u, pacc4);
            cf dd;
            dd.r = bperm_a(d.r, pacc4);
            dd.i = CPLX ? bperm_a(d.i, pacc4) : 0.f;
            dacc = cmul(dd, dacc);
            pacc4 = (int)(np << 2);
            // readout weight g_t[j] = c_t[pacc_t[j]] dacc_t[j]; v += gy_t conj(g_t)
            const cf cg = unpack_c<CPLX, BCBF>(bperm_raw<CPLX, BCBF>(craw, pacc4));
            const cf w = cmul(cg, dacc);
            v.r += g * w.r;
            v.i -= g * w.i;
        }
    }
    a.sig[ch * 64 + lane] = pacc4 >> 2;
    a.mv[ch * 64 + lane] = make_float4(dacc.r, -dacc.i, v.r, v.i);
}

// ---------------------------------------------------------------------------
// The carries K_c, right to left, in three shallow passes instead of one
// chain over all chunks: compose each group of kGroup chunk operators (in
// parallel), chain the group operators per sequence, then expand each group
// from its carry.  An operator (sig, m, v) maps K to m[j] K[sig[j]] + v[j];
// applying (sig1, m1, v1) after (sig2, m2, v2) -- the chunk on the left
// after the one on its right -- gives
//     sig = sig2[sig1],  m = m1 * m2[sig1],  v = m1 * v2[sig1] + v1.
// ---------------------------------------------------------------------------
constexpr int kGroup = 32;   // chunks per group

struct GOp {
    int sig;
    cf m, v;
};

template <bool CPLX>
__device__ __forceinline__ GOp load_op(const BwdArgs &a, const int32_t *sig, const float4 *mv, int64_t rec, int lane)
{
    const float4 q = mv[rec * 64 + lane];
    return {sig[rec * 64 + lane], {q.x, CPLX ? q.y : 0.f}, {q.z, CPLX ? q.w : 0.f}};
}

// apply `left` after `right` (right = the operator of the chunks on the right)
template <bool CPLX>
__device__ __forceinline__ GOp compose_left(GOp left, GOp right)
{
    const int src = left.sig * 4;
    GOp r;
    r.sig = (int)bperm_a((uint32_t)right.sig, src);
    cf m2, v2;
    m2.r = bperm_a(right.m.r, src);
    m2.i = CPLX ? bperm_a(right.m.i, src) : 0.f;
    v2.r = bperm_a(right.v.r, src);
    v2.i = CPLX ? bperm_a(right.v.i, src) : 0.f;
    r.m = cmul(left.m, m2);
    const cf t = cmul(left.m, v2);
    r.v = {t.r + left.v.r, t.i + left.v.i};
    return r;
}

template <bool CPLX>
__device__ __forceinline__ cf apply_op(GOp op, cf k)
{
    cf kg;
    kg.r = bperm(k.r, op.sig);
    kg.i = CPLX ? bperm(k.i, op.sig) : 0.f;
    const cf t = cmul(op.m, kg);
    return {t.r + op.v.r, t.i + op.v.i};
}

// One wave per group: the group's operator, its chunks composed right to left.
template <bool CPLX>
__global__ void __launch_bounds__(kBW * 64) bwd_group_kernel(BwdArgs a)
{
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
    const int64_t ng = (a.nch + kGroup - 1) / kGroup;
    const int64_t gi = (int64_t)blockIdx.x * kBW + wave;
    if (gi >= a.S * ng)
        return;
    const int64_t seq = gi / ng, g = gi - seq * ng;
    const int64_t c0 = g * kGroup, c1 = min(c0 + kGroup, a.nch) - 1;
    // ring slot r holds the chunk i = r (mod 4) from the right end of the group
    GOp ring[4];
#pragma unroll
    for (int r = 0; r < 4; ++r)
        ring[r] = load_op<CPLX>(a, a.sig, a.mv, seq * a.nch + max(c1 - r, c0), lane);
    GOp acc = ring[0];
    for (int64_t i0 = 0; i0 <= c1 - c0; i0 += 4) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int64_t c = c1 - (i0 + r);
            if (c >= c0) {
                const GOp op = ring[r];
                ring[r] = load_op<CPLX>(a, a.sig, a.mv, seq * a.nch + max(c - 4, c0), lane);
                acc = (i0 + r == 0) ? op : compose_left<CPLX>(op, acc);
            }
        }
    }
    a.gsig[gi * 64 + lane] = acc.sig;
    a.gmv[gi * 64 + lane] = make_float4(acc.m.r, acc.m.i, acc.v.r, acc.v.i);
}

// One wave per sequence: the carry into each group's last chunk, right to
// left over the groups; then gx0.
template <bool CPLX>
__global__ void __launch_bounds__(kBW * 64) bwd_chain_kernel(BwdArgs a)
{
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
    const int64_t seq = (int64_t)blockIdx.x * kBW + wave;
    if (seq >= a.S)
        return;
    const int64_t ng = (a.nch + kGroup - 1) / kGroup;
    const bool act = lane < a.N;
    cf kk = {0.f, 0.f};
    if (a.gxf && act)
        kk = load_diag<CPLX>(a.gxf, seq * a.N + lane);
    for (int64_t g = ng - 1; g >= 0; --g) {
        a.gk[(seq * ng + g) * 64 + lane] = make_float2(kk.r, kk.i);
        kk = apply_op<CPLX>(load_op<CPLX>(a, a.gsig, a.gmv, seq * ng + g, lane), kk);
    }
    if (a.gx0 && act)
        store_grad<CPLX>(a.gx0, seq * a.N + lane, kk);
}

// One wave per group: the carry into every chunk of the group.
template <bool CPLX>
__global__ void __launch_bounds__(kBW * 64) bwd_expand_kernel(BwdArgs a)
{
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
    const int64_t ng = (a.nch + kGroup - 1) / kGroup;
    const int64_t gi = (int64_t)blockIdx.x * kBW + wave;
    if (gi >= a.S * ng)
        return;
    const int64_t seq = gi / ng, g = gi - seq * ng;
    const int64_t c0 = g * kGroup, c1 = min(c0 + kGroup, a.nch) - 1;
    const float2 k0 = a.gk[gi * 64 + lane];
    cf kk = {k0.x, k0.y};
    GOp ring[4];
#pragma unroll
    for (int r = 0; r < 4; ++r)
        ring[r] = load_op<CPLX>(a, a.sig, a.mv, seq * a.nch + max(c1 - r, c0), lane);
    for (int64_t i0 = 0; i0 <= c1 - c0; i0 += 4) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int64_t c = c1 - (i0 + r);
            if (c >= c0) {
                a.kc[(seq * a.nch + c) * 64 + lane] = make_float2(kk.r, kk.i);
                const GOp op = ring[r];
                ring[r] = load_op<CPLX>(a, a.sig, a.mv, seq * a.nch + max(c - 4, c0), lane);
                kk = apply_op<CPLX>(op, kk);
            }
        }
    }
}

// ---------------------------------------------------------------------------
// bwd_grad: per chunk (one wave, lane = state).  The states x_t of the chunk
// by the forward's collision-free scatter from the saved carry-in (kept in
// registers), then lambda backwards from K_c by gathers, writing gb, gc and
// gd.  Inputs stream through rings of D steps; the loads of both passes are
// issued before any store of the chunk waits on them.
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
    const ChunkPos cp = chunk_of(a, ch);
    const int64_t seq = cp.seq, t0 = cp.t0, h = cp.h;
    const int nv = (int)min((int64_t)kBT, a.L - t0);
    const int N = a.N;
#pragma unroll
    for (int r = kRegions; r < 2 * kRegions; ++r)
        s_reg[wave][r][lane] = cf{0.f, 0.f};
    char *const regp = reinterpret_cast<char *>(&s_reg[wave][0][0]);
    const char *const rowbase = regp + lane * (int)sizeof(cf);

    using IO = ChunkIO<CPLX, BCBF>;
    using Raw = typename RawOf<CPLX, BCBF>::type;
    using DRaw = typename IO::DRaw;
    using Stored = typename IO::Stored;
    IO io;
    io.init(a, seq, t0, nv, h, lane);
    // selections: the forward's (index modes) or the ones the operator pass
    // picked from the scores
    const void *ssrc = a.ksel ? static_cast<const void *>(a.ksel) : a.sel;
    const uint32_t smode = a.ksel ? PDSSM_SEL_I16 : a.sel_mode;
    const int kraw = sel_raw(ssrc, smode, seq * a.L + t0, nv, lane);
    const uint32_t gyr = chunk_gy_raw(a, seq * a.L + t0, nv, lane);
    auto gy_at = [&](int tt) { return gy_step(a, gyr, tt); };
    auto sel_at = [&](int ts) { return __builtin_amdgcn_readfirstlane((int)s_sel[wave][ts]); };
    const int64_t e0 = (seq * a.L + t0) * N;
    const uint64_t rows = (uint64_t)nv * (uint64_t)N;
    const __amdgpu_buffer_rsrc_t ogb = make_rsrc(reinterpret_cast<Stored *>(a.gb) + e0, rows * sizeof(Stored));
    const __amdgpu_buffer_rsrc_t ogc = make_rsrc(reinterpret_cast<Stored *>(a.gc) + e0, rows * sizeof(Stored));
    const __amdgpu_buffer_rsrc_t ogd = make_rsrc(reinterpret_cast<DRaw *>(a.gd) + e0, rows * sizeof(DRaw));
    const __amdgpu_buffer_rsrc_t rx = make_rsrc(reinterpret_cast<const DRaw *>(a.xch) + ch * N, (uint64_t)N * sizeof(DRaw));

    constexpr int D = PDSSM_BWD_GRAD_D;
    cf rd[D];
    Raw rv[D];   // b in the forward pass, c in the backward pass
    uint32_t re[D];

    // ---- x over the chunk: x_t = P_t (d_t * x_{t-1}) + b_t.  The first
    // rows of d and b are in flight before the selections are read.
    auto fetch_db = [&](int tt) {
        const int ts = min(tt, nv - 1);
        rd[tt % D] = io.d(ts);
        rv[tt % D] = io.raw_b(ts);
    };
    auto fetch_f = [&](int tt) {
        fetch_db(tt);
        re[tt % D] = io.ent(sel_at(min(tt, nv - 1)));
    };
#pragma unroll
    for (int tt = 0; tt < D; ++tt)
        fetch_db(tt);
    sel_put(kraw, a.K, nv, s_sel[wave], lane);
#pragma unroll
    for (int tt = 0; tt < D; ++tt)
        re[tt % D] = io.ent(sel_at(min(tt, nv - 1)));
    cf xin;
    {
        const DRaw v = bload<DRaw>(rx, io.vd, 0);
        if constexpr (CPLX)
            xin = {v.x, v.y};
        else
            xin = {v, 0.f};
    }
    cf xs[kBT];   // x_t, and d_t and pi_t (four 6-bit maps a word) for the reverse pass
    cf ds[kBT];
    uint32_t pis[kBT / 4] = {};
    cf x = xin;
#pragma unroll
    for (int tt = 0; tt < kBT; ++tt) {
        const cf d = rd[tt % D];
        const cf bb = unpack_c<CPLX, BCBF>(rv[tt % D]);
        const uint32_t ent = re[tt % D];
        if (tt + D < kBT)
            fetch_f(tt + D);
        ds[tt] = d;
        pis[tt / 4] |= (ent & 63u) << (8 * (tt % 4));
        if (tt < nv) {
            const cf v = cmul(d, x);
            const uint32_t slot = entry_slot(ent);
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
            const char *rowp = rowbase + entry_row(ent);
            cf sum = bb;
#pragma unroll
            for (int r = 0; r < kRegions; ++r) {
                const float2 u = *static_cast<const float2 *>(__builtin_assume_aligned(rowp + r * kRegionBytes, 8));
                sum.r += u.x;
                sum.i += u.y;
            }
            lds_order();
            x = sum;
        }
        xs[tt] = x;
    }

    // ---- lambda back over the chunk, from the carried part K_c
    auto fetch_b = [&](int u) {   // u-th step from the end: step 15 - u, clamped into the chunk
        const int ts = min(kBT - 1 - u, nv - 1);
        rv[u % D] = io.raw_c(max(ts, 0));
    };
#pragma unroll
    for (int u = 0; u < D; ++u)
        fetch_b(u);
    const float2 k0 = a.kc[ch * 64 + lane];
    cf lc = {k0.x, k0.y};   // A_{t+1}^H lambda_{t+1}, the part carried into step t
#pragma unroll
    for (int u = 0; u < kBT; ++u) {
        const int tt = kBT - 1 - u;
        const cf d = ds[tt];
        const cf cv = unpack_c<CPLX, BCBF>(rv[u % D]);
        const uint32_t ent = pis[tt / 4] >> (8 * (tt % 4));
        if (u + D < kBT)
            fetch_b(u + D);
        if (tt < nv) {
            const float g = gy_at(tt);
            const cf lam = {lc.r + g * cv.r, lc.i - g * cv.i};
            const int pi4 = (int)((ent & 63u) << 2);
            cf lg;
            lg.r = bperm_a(lam.r, pi4);
            lg.i = CPLX ? bperm_a(lam.i, pi4) : 0.f;
            const cf xt = xs[tt];
            const cf xp = (tt > 0) ? xs[tt > 0 ? tt - 1 : 0] : xin;
            const uint32_t rs = (uint32_t)(tt * N * (int)sizeof(Stored));
            bstore<Stored>(ogb, pack_vec<CPLX, BCBF>(lam), io.vs, rs);
            bstore<Stored>(ogc, pack_vec<CPLX, BCBF>(cf{g * xt.r, -g * xt.i}), io.vs, rs);
            bstore<DRaw>(ogd, pack_d<CPLX>(cf{xp.r * lg.r + xp.i * lg.i, xp.r * lg.i - xp.i * lg.r}), io.vd,
                         (uint32_t)(tt * N * (int)sizeof(DRaw)));
            lc = {d.r * lg.r + d.i * lg.i, d.r * lg.i - d.i * lg.r};
        }
    }
}

// ---------------------------------------------------------------------------
// Host side.
// ---------------------------------------------------------------------------
struct BwdLayout {
    int64_t nch, S, tab_bytes, sig_bytes, mv_bytes, kc_bytes, grp_bytes, ksel_bytes, total;
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
    const int64_t groups = lo.S * ((lo.nch + kGroup - 1) / kGroup);
    lo.grp_bytes = up(groups * 64 * 4) + up(groups * 64 * 16) + up(groups * 64 * 8);
    lo.ksel_bytes = up(lo.S * L * 2);
    lo.total = lo.tab_bytes + lo.sig_bytes + lo.mv_bytes + lo.kc_bytes + lo.grp_bytes + lo.ksel_bytes;
    return lo;
}

template <bool CPLX, bool BCBF>
static void launch_bwd(const BwdArgs &a, hipStream_t st)
{
    const int64_t chunks = a.S * a.nch;
    const dim3 blk(kBW * 64);
    hipLaunchKernelGGL((bwd_ops_kernel<CPLX, BCBF>), dim3((unsigned)((chunks + kBW - 1) / kBW)), blk, 0, st, a);
    const int64_t groups = a.S * ((a.nch + kGroup - 1) / kGroup);
    hipLaunchKernelGGL((bwd_group_kernel<CPLX>), dim3((unsigned)((groups + kBW - 1) / kBW)), blk, 0, st, a);
    hipLaunchKernelGGL((bwd_chain_kernel<CPLX>), dim3((unsigned)((a.S + kBW - 1) / kBW)), blk, 0, st, a);
    hipLaunchKernelGGL((bwd_expand_kernel<CPLX>), dim3((unsigned)((groups + kBW - 1) / kBW)), blk, 0, st, a);
    hipLaunchKernelGGL((bwd_grad_kernel<CPLX, BCBF>), dim3((unsigned)((chunks + kBW - 1) / kBW)), blk, 0, st, a);
}

}  // namespace pdssm

using namespace pdssm;

extern "C" size_t pdssm_scan_bwd_workspace_bytes(int64_t B, int64_t H, int64_t L, int32_t N,
                                                 int32_t K, uint32_t flags)
{
    if (check_dims(B, H, L, N, K) != PDSSM_OK || (flags & ~PDSSM_FLAGS_ALL))
        return 0;
    // Never 0 (which means invalid arguments), also for empty shapes.
    const int64_t total = bwd_layout(B, H, L, K).total;
    return (size_t)(total > 256 ? total : 256);
}

extern "C" int pdssm_scan_bwd(const void *sel_or_logits, const int32_t *dict_idx, const void *diag,
                              const void *b, const void *c, const void *x_chunks, const void *gy,
                              const void *gx_final, void *gb, void *gc, void *gd, void *gx0,
                              int64_t B, int64_t H, int64_t L, int32_t N, int32_t K, uint32_t flags,
                              void *workspace, size_t workspace_bytes, hipStream_t stream)
{
    int rc = check_dims(B, H, L, N, K);
    if (rc != PDSSM_OK)
        return rc;
    if (flags & ~PDSSM_FLAGS_ALL)
        return PDSSM_ERR_FLAGS;
    if (B == 0 || H == 0)
        return PDSSM_OK;   // no sequences: nothing to read or write
    if (L == 0) {
        // No steps: x_final = x0, so gx0 = gx_final (or zero).
        if (!gx0)
            return PDSSM_OK;
        if (!aligned16(gx0) || (gx_final && !aligned16(gx_final)))
            return PDSSM_ERR_ALIGN;
        return launch_state_fill(gx_final, gx0, B * H * N * ((flags & PDSSM_COMPLEX) ? 2 : 1), stream);
    }
    if (!sel_or_logits || !dict_idx || !diag || !b || !c || !x_chunks || !gy || !gb || !gc || !gd ||
        !workspace)
        return PDSSM_ERR_NULL;
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
    {
        char *gw = w + lo.tab_bytes + lo.sig_bytes + lo.mv_bytes + lo.kc_bytes;
        const int64_t groups = lo.S * ((lo.nch + kGroup - 1) / kGroup);
        auto up = [](int64_t n) { return (n + 255) / 256 * 256; };
        a.gsig = reinterpret_cast<int32_t *>(gw);
        a.gmv = reinterpret_cast<float4 *>(gw + up(groups * 64 * 4));
        a.gk = reinterpret_cast<float2 *>(gw + up(groups * 64 * 4) + up(groups * 64 * 16));
    }
    const bool logits = (flags & PDSSM_SEL_MASK) == PDSSM_LOGITS_F32 || (flags & PDSSM_SEL_MASK) == PDSSM_LOGITS_BF16;
    a.ksel = logits ? reinterpret_cast<int16_t *>(w + lo.total - lo.ksel_bytes) : nullptr;
    a.H = H;
    a.L = L;
    a.S = lo.S;
    a.nch = lo.nch;
    a.N = N;
    a.K = K;
    a.sel_mode = flags & PDSSM_SEL_MASK;
    a.y_bf16 = (flags & PDSSM_Y_BF16) ? 1 : 0;
    a.idx32 = (lo.S * lo.nch < ((int64_t)1 << 31) && H < ((int64_t)1 << 31)) ? 1 : 0;

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
