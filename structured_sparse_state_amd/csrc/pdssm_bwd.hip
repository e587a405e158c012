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
// a sum of the forward's own readout weights.  One kernel, bwd_fused, does
// it all in one pass over the inputs: per chunk, (pacc, conj(dacc), v_c) and
// x over the chunk (from the forward's saved carry-in), K_c by a decoupled
// look-back over the chunks on its right, then lambda back over the chunk,
// writing gb, gc and gd.
#include <hip/hip_runtime.h>

#include <type_traits>

#include "pdssm.h"
#include "pdssm_device.h"
#include "pdssm_host.h"

namespace pdssm {

constexpr int kBT = kCarryStride;   // steps per chunk (the forward saves one carry per chunk)
#ifndef PDSSM_BWD_W
#define PDSSM_BWD_W 4   // chunk waves per workgroup (one tile)
#endif
constexpr int kBW = PDSSM_BWD_W;
#ifndef PDSSM_BWD_GRAD_D
#define PDSSM_BWD_GRAD_D 4   // steps of b and c in flight per wave
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
    Header *hdr;        // epoch and ticket counter
    uint64_t *agg;      // [S*tiles][AW][64] each tile's adjoint operator, epoch-tagged words
    uint64_t *incl;     // [S*tiles][NC][64] the adjoint each tile carries out of its first step
    uint32_t total;     // tickets: S * tiles
    int64_t tiles;      // tiles per sequence (kBW * 64 / NP chunks each)
    int64_t H, L, S, nch;
    int N, K;
    uint32_t sel_mode;
    int y_bf16;
    int strict;         // the carry only from the tile just after (no aggregate records)
};

template <bool CPLX>
__device__ __forceinline__ void store_grad(float *p, int64_t e, cf v)
{
    if constexpr (CPLX)
        reinterpret_cast<float2 *>(p)[e] = make_float2(v.r, v.i);
    else
        p[e] = v.r;
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

// A wave holds G = 64 / NP chunks (lane group g = lane / NP runs the g-th,
// lane i = lane % NP its state i).  The resources start at the wave's first
// row; a lane's rows lie at its chunk's offset from there.  Steps are
// clamped into the sequence: with one chunk per wave by the wave-uniform
// row offset, with several by the lane's own offset.
template <int NP, bool CPLX, bool BCBF>
struct ChunkIO {
    static constexpr int G = 64 / NP;
    using DRaw = typename std::conditional<CPLX, float2, float>::type;
    using Stored = typename std::conditional<BCBF, typename std::conditional<CPLX, uint32_t, uint16_t>::type,
                                             DRaw>::type;
    __amdgpu_buffer_rsrc_t rd, rb, rc, rt;
    uint32_t vd, vs, vt;   // lane offsets (bytes) into diag-like, b/c-like rows and the entry table
    int N, last;           // last: the lane's last valid row, counted from the wave's first
    int rel;               // the lane's first row, counted from the wave's first
    bool act;

    __device__ void init(const BwdArgs &a, int64_t seq, int64_t tw, int64_t t0, int64_t h, int i)
    {
        N = a.N;
        const int64_t e0 = (seq * a.L + tw) * a.N;   // first element of the wave's rows
        // The wave's rows only (at most 64 steps): padding lanes' offsets
        // (kOffLane, 2 GiB) must stay beyond the range.
        const int64_t wrows = (a.L - tw < (int64_t)(G * kBT)) ? a.L - tw : (int64_t)(G * kBT);
        const uint64_t rows = (uint64_t)wrows * (uint64_t)a.N;
        rd = make_rsrc(reinterpret_cast<const DRaw *>(a.diag) + e0, rows * sizeof(DRaw));
        rb = make_rsrc(reinterpret_cast<const Stored *>(a.b) + e0, rows * sizeof(Stored));
        rc = make_rsrc(reinterpret_cast<const Stored *>(a.c) + e0, rows * sizeof(Stored));
        rt = make_rsrc(a.tab + h * (int64_t)a.K * NP, (uint64_t)a.K * NP * 2);
        act = i < a.N;
        rel = (int)(t0 - tw);
        last = (int)(a.L - 1 - tw);
        vd = act ? (uint32_t)(i * sizeof(DRaw)) : kOffLane;
        vs = act ? (uint32_t)(i * sizeof(Stored)) : kOffLane;
        vt = (uint32_t)(i * 2);   // the table has all NP lanes (padding maps to itself)
    }
    // byte offsets of step tt of the lane's chunk (ts: the same step clamped
    // into the chunk, used with one chunk per wave)
    template <typename V>
    __device__ void offs(int tt, int ts, uint32_t base, uint32_t &voff, uint32_t &soff) const
    {
        if constexpr (G == 1) {
            voff = base;
            soff = (uint32_t)(ts * N * (int)sizeof(V));
        } else {
            voff = act ? base + (uint32_t)(min(rel + tt, last) * N * (int)sizeof(V)) : kOffLane;
            soff = 0;
        }
    }
    __device__ cf d(int tt, int ts) const
    {
        uint32_t vo, so;
        offs<DRaw>(tt, ts, vd, vo, so);
        const DRaw v = bload<DRaw>(rd, vo, so);
        if constexpr (CPLX)
            return {v.x, v.y};
        else
            return {v, 0.f};
    }
    __device__ typename RawOf<CPLX, BCBF>::type raw_b(int tt, int ts) const
    {
        uint32_t vo, so;
        offs<Stored>(tt, ts, vs, vo, so);
        return (typename RawOf<CPLX, BCBF>::type)bload<Stored>(rb, vo, so);
    }
    __device__ typename RawOf<CPLX, BCBF>::type raw_c(int tt, int ts) const
    {
        uint32_t vo, so;
        offs<Stored>(tt, ts, vs, vo, so);
        return (typename RawOf<CPLX, BCBF>::type)bload<Stored>(rc, vo, so);
    }
    // the entry of dictionary entry k for this lane (k wave-uniform when G == 1)
    __device__ uint32_t ent(int k) const
    {
        if constexpr (G == 1)
            return bload<uint16_t>(rt, vt, (uint32_t)(k * NP * 2));
        else
            return bload<uint16_t>(rt, vt + (uint32_t)(k * NP * 2), 0);
    }
    // the store offsets of step tt (inside the sequence) of the lane's chunk
    template <typename V>
    __device__ void store_offs(int tt, uint32_t base, uint32_t &voff, uint32_t &soff) const
    {
        if constexpr (G == 1) {
            voff = base;
            soff = (uint32_t)(tt * N * (int)sizeof(V));
        } else {
            voff = act ? base + (uint32_t)((rel + tt) * N * (int)sizeof(V)) : kOffLane;
            soff = 0;
        }
    }
};

// The wave's upstream gradients gy as stored (fp32 bits, or bf16 bits in
// the low half), one step per lane (lanes 0..nv-1 of the wave's steps).
// They are converted where a step uses them, so that the load stays in
// flight meanwhile.
__device__ __forceinline__ uint32_t chunk_gy_raw(const BwdArgs &a, int64_t step0, int nv, int lane)
{
    const int l = min(lane, nv - 1);
    if (a.y_bf16)
        return reinterpret_cast<const uint16_t *>(a.gy)[step0 + l];
    return reinterpret_cast<const uint32_t *>(a.gy)[step0 + l];
}

// gy of step s of the wave's steps (s wave-uniform with one chunk per wave,
// else per lane)
template <int G>
__device__ __forceinline__ float gy_step(const BwdArgs &a, uint32_t raw, int s)
{
    uint32_t r;
    if constexpr (G == 1)
        r = (uint32_t)__builtin_amdgcn_readlane((int)raw, s);
    else
        r = bperm_a(raw, s * 4);
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

template <int WS>
__device__ __forceinline__ void sel_put(int k, int K, int nv, int16_t *out, int lane)
{
    if (lane < WS)
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
__device__ __forceinline__ typename ChunkIO<64, CPLX, BCBF>::Stored pack_vec(cf v)
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
// Adjoint chunk operators.  An operator (sig, m, v) maps K to
// m[j] K[sig[j]] + v[j]; applying (sig1, m1, v1) after (sig2, m2, v2) -- the
// chunk on the left after the one on its right -- gives
//     sig = sig2[sig1],  m = m1 * m2[sig1],  v = m1 * v2[sig1] + v1.
// ---------------------------------------------------------------------------
struct GOp {
    int sig;
    cf m, v;
};

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

// ---------------------------------------------------------------------------
// bwd_fused: the whole backward in one pass over the inputs.  A lane group
// of NP lanes owns one chunk of kBT steps (64 / NP chunks per wave), a
// workgroup a tile of kBW * 64 / NP consecutive chunks.
// Workgroups take tickets in reverse time order (the last tiles of every
// sequence first), so every tile to the right of a workgroup's tile belongs
// to a workgroup that has started, and a workgroup only ever waits for
// those.  Each lane group
//  1. loads its chunk's rows and selections (picking them from the scores in
//     the logits modes),
//  2. runs forward through the chunk: the states x_t from the saved carry-in
//     by the forward scan's collision-free scatter and, alongside, the
//     chunk's adjoint operator (sig, m, v), which maps the adjoint carried
//     into its last step to the one it carries out of its first:
//     K_out[j] = m[j] K_in[sig[j]] + v[j],
//  3. hands its operator to wave 0, which composes the tile's operator,
//     publishes it and looks back to the right (decoupled look-back,
//     Merrill & Garland) for the tile's K_in: it composes the operators of
//     the tiles on its right until it meets one whose K_out is published
//     (the sequence's last tile publishes no operator: its K_in is
//     gx_final, so its K_out follows at once),
//  4. (wave 0) derives every chunk's K_in from the tile's and publishes the
//     tile's K_out (gx0 for the first tile of a sequence),
//  5. runs backward through its chunk from K_in, writing gb, gc and gd.
// Records are 64-bit words with the call's epoch in the upper half, as in
// the forward scan, so a reader needs no fence; word k of every lane is
// contiguous (word-major records).
// ---------------------------------------------------------------------------
template <bool CPLX>
struct BwdRec {
    static constexpr int NC = CPLX ? 2 : 1;
    static constexpr int AW = 1 + 2 * NC;   // operator words per lane: sig, m.r, v.r (, m.i, v.i)
};

template <int NP, bool CPLX, bool BCBF>
__global__ void __launch_bounds__(kBW * 64) bwd_fused_kernel(BwdArgs a)
{
    using Rec = BwdRec<CPLX>;
    constexpr int NC = Rec::NC, AW = Rec::AW;
    constexpr int G = 64 / NP, TC = kBW * G, WS = G * kBT;   // chunks per wave, per tile; steps per wave
    static_assert(G >= 1 && WS <= 64, "one step of the wave per lane");
    __shared__ int16_t s_sel[kBW][WS];
    __shared__ __attribute__((aligned(16))) cf s_reg[kBW][kBlocks][64];
    __shared__ uint32_t s_ticket;
    __shared__ int s_osig[kBW][64];   // each chunk's operator (group g of wave w at [w][g*NP..]), then its carry
    __shared__ cf s_om[kBW][64];
    __shared__ cf s_ov[kBW][64];
    __shared__ cf s_k[kBW][64];
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
    const int g = (G == 1) ? 0 : lane / NP, i = (G == 1) ? lane : lane % NP, gbase = g * NP;
    if (threadIdx.x == 0)
        s_ticket = atomicAdd(&a.hdr->ticket, 1u);
#pragma unroll
    for (int r = kRegions; r < 2 * kRegions; ++r)
        s_reg[wave][r][lane] = cf{0.f, 0.f};
    __syncthreads();
    // Ticket u -> (tile from the right, sequence), tile-major over sequences.
    const uint32_t u = __builtin_amdgcn_readfirstlane(s_ticket);
    const uint32_t S32 = (uint32_t)a.S;
#ifdef PDSSM_TEST_TICKET_REMAP
    // Test build: the sequences of a tile row are handed out in reverse.
    const uint32_t tile = u / S32, seq32 = S32 - 1u - (u - tile * S32);
#else
    const uint32_t tile = u / S32, seq32 = u - tile * S32;
#endif
    if (u >= a.total)
        return;
    // The tile's chunks from the right: wave w holds the G chunks from
    // c_w on (group g the g-th, in time order).  The sequence's first tile
    // may have fewer than TC chunks: a lane group without one runs chunk 0's
    // loads and arithmetic to no effect (its operator is the identity and it
    // stores nothing), so that its wave meets the barriers.
    const int64_t c_w = a.nch - 1 - (int64_t)tile * TC - (int64_t)wave * G - (G - 1);
    const int64_t c_own = c_w + g;
    const bool has = c_own >= 0;
    const int64_t c = has ? c_own : 0;
    const int64_t tw = (c_w > 0 ? c_w : 0) * kBT;   // the wave's first step
    const uint32_t epoch = a.hdr->epoch;
    const int64_t seq = seq32, t0 = c * kBT, h = seq32 % (uint32_t)a.H;
    const int nv = (int)min((int64_t)kBT, a.L - t0);             // steps of the lane's chunk
    const int nvw = (int)min((int64_t)WS, a.L - tw);             // steps of the wave
    const int sofs = (int)(t0 - tw);                             // the chunk's first step in the wave's
    const int N = a.N;
    char *const regp = reinterpret_cast<char *>(&s_reg[wave][0][0]) + gbase * (int)sizeof(cf);
    const char *const rowbase = regp + i * (int)sizeof(cf);

    using IO = ChunkIO<NP, CPLX, BCBF>;
    using Raw = typename RawOf<CPLX, BCBF>::type;
    using DRaw = typename IO::DRaw;
    using Stored = typename IO::Stored;
    IO io;
    io.init(a, seq, tw, t0, h, i);
    const bool idx = index_mode(a.sel_mode);
    const int kraw = idx ? sel_raw(a.sel, a.sel_mode, seq * a.L + tw, nvw, lane) : 0;
    const uint32_t gyr = chunk_gy_raw(a, seq * a.L + tw, nvw, lane);
    // the selection of step ts of the lane's chunk
    auto sel_at = [&](int ts) {
        if constexpr (G == 1)
            return __builtin_amdgcn_readfirstlane((int)s_sel[wave][ts]);
        else
            return (int)s_sel[wave][sofs + ts];
    };

    // ---- 1. loads: every d row of the chunk (kept for both passes) and
    // every c row (kept for the operator and the backward pass), the first D
    // rows of b, the carry-in state; then the selections.
    constexpr int D = PDSSM_BWD_GRAD_D;
    cf ds[kBT];
    Raw cs[kBT];
#pragma unroll
    for (int tt = 0; tt < kBT; ++tt) {
        ds[tt] = io.d(tt, min(tt, nv - 1));
        cs[tt] = io.raw_c(tt, min(tt, nv - 1));
    }
    Raw rb[D];
    uint32_t re[D];
#pragma unroll
    for (int tt = 0; tt < D; ++tt)
        rb[tt] = io.raw_b(tt, min(tt, nv - 1));
    cf xin = {0.f, 0.f};
    if (i < N) {
        const int64_t xe = (seq * a.nch + c) * N + i;
        if constexpr (CPLX) {
            const float2 v = reinterpret_cast<const float2 *>(a.xch)[xe];
            xin = {v.x, v.y};
        } else {
            xin = {a.xch[xe], 0.f};
        }
    }
    if (idx)
        sel_put<WS>(kraw, a.K, nvw, s_sel[wave], lane);
    else
        wave_select<WS>(a.sel, a.sel_mode, a.K, a.L, seq * a.L, tw, s_sel[wave], lane);
#pragma unroll
    for (int tt = 0; tt < D; ++tt)
        re[tt] = io.ent(sel_at(min(tt, nv - 1)));

    // ---- 2. forward through the chunk: x_t, and the adjoint operator.
    // Lane j follows the chunk-start source j: pacc (byte address) is where
    // it sits after step t, dacc its factor; the readout weight of step t is
    // g_t[j] = c_t[pacc_t[j]] dacc_t[j] and v = sum_t gy_t conj(g_t).
    cf xs[kBT];
    uint32_t pis[kBT / 4] = {};
    cf x = xin;
    int pacc4 = lane * 4;
    cf dacc = {1.f, 0.f}, v = {0.f, 0.f};
#pragma unroll
    for (int tt = 0; tt < kBT; ++tt) {
        const cf d = ds[tt];
        const Raw braw = rb[tt % D], craw = cs[tt];
        const uint32_t ent = re[tt % D];
        if (tt + D < kBT) {
            const int ts = min(tt + D, nv - 1);
            rb[tt % D] = io.raw_b(tt + D, ts);
            re[tt % D] = io.ent(sel_at(ts));
        }
        pis[tt / 4] |= (ent & 63u) << (8 * (tt % 4));
        if (tt < nv) {
            // the operator: gathers at the previous position (no dependence on x)
            const uint32_t np = bperm_a(ent & 63u, pacc4);
            cf dd;
            dd.r = bperm_a(d.r, pacc4);
            dd.i = CPLX ? bperm_a(d.i, pacc4) : 0.f;
            // x_t = P_t (d_t * x_{t-1}) + b_t by the rank-region scatter
            const cf vv = cmul(d, x);
            const uint32_t slot = entry_slot(ent);
            *static_cast<float2 *>(__builtin_assume_aligned(regp + slot, 8)) = make_float2(vv.r, vv.i);
            lds_order();
            if (__any(slot_rank_ovf(slot))) {
                if (slot_rank_ovf(slot)) {
                    cf *o = reinterpret_cast<cf *>(regp + (slot - kRegionBytes));
                    lds_add(&o->r, vv.r);
                    if constexpr (CPLX)
                        lds_add(&o->i, vv.i);
                }
                lds_order();
            }
            const char *rowp = rowbase + entry_row(ent);
            cf sum = unpack_c<CPLX, BCBF>(braw);
#pragma unroll
            for (int r = 0; r < kRegions; ++r) {
                const float2 q = *static_cast<const float2 *>(__builtin_assume_aligned(rowp + r * kRegionBytes, 8));
                sum.r += q.x;
                sum.i += q.y;
            }
            if (__any(entry_deg_ovf(ent))) {
                if (entry_deg_ovf(ent)) {
                    const float2 q = *static_cast<const float2 *>(__builtin_assume_aligned(rowbase + kSpareOff, 8));
                    sum.r += q.x;
                    sum.i += q.y;
                }
            }
            lds_order();
            x = sum;
            dacc = cmul(dd, dacc);
            pacc4 = (int)((np + gbase) << 2);
            const float gq = gy_step<G>(a, gyr, (G == 1) ? tt : sofs + tt);
            const cf cg = unpack_c<CPLX, BCBF>(bperm_raw<CPLX, BCBF>(craw, pacc4));
            const cf w = cmul(cg, dacc);
            v.r += gq * w.r;
            v.i -= gq * w.i;
        }
        xs[tt] = x;
    }

    // ---- 3. the tile's carries.  The chunks' operators meet in LDS; wave 0
    // composes the tile's operator (the leftmost chunk's applied last), looks
    // back over the tiles on the right for the adjoint carried into the tile,
    // and hands every chunk the adjoint carried into it.  Chunk k of the tile
    // (from the right) is group G-1-(k mod G) of wave k / G; wave 0 works on
    // NP-lane operators, its lane groups all holding the same copy.
    s_osig[wave][lane] = has ? ((pacc4 >> 2) - gbase) : i;
    s_om[wave][lane] = has ? cf{dacc.r, -dacc.i} : cf{1.f, 0.f};
    s_ov[wave][lane] = has ? v : cf{0.f, 0.f};
    __syncthreads();
    if (wave == 0) {
        auto op_of = [&](int k) {
            const int w = k / G, at = (G - 1 - k % G) * NP + i;
            return GOp{s_osig[w][at], s_om[w][at], s_ov[w][at]};
        };
        const int64_t seq_rec = seq * a.tiles, trec = seq_rec + tile;
        cf K = {0.f, 0.f};
        if (tile == 0) {
            if (a.gxf && i < N)
                K = load_diag<CPLX>(a.gxf, seq * N + i);   // the adjoint after the last step
        } else {
            GOp tagg = op_of(0);
#pragma unroll
            for (int k = 1; k < TC; ++k)
                tagg = compose_left<CPLX>(op_of(k), tagg);
            // words: sig, m.r, v.r (, m.i, v.i); with PDSSM_DETERMINISTIC no
            // tile reads them (each takes only the carry of the tile just
            // after it), so none are written.
            if (!a.strict) {
                uint64_t *const aw_own = a.agg + trec * (AW * 64);
                put_word(aw_own + lane, (uint32_t)tagg.sig, epoch);
                put_word(aw_own + 64 + lane, __float_as_uint(tagg.m.r), epoch);
                put_word(aw_own + 128 + lane, __float_as_uint(tagg.v.r), epoch);
                if constexpr (CPLX) {
                    put_word(aw_own + 192 + lane, __float_as_uint(tagg.m.i), epoch);
                    put_word(aw_own + 256 + lane, __float_as_uint(tagg.v.i), epoch);
                }
            }
            GOp acc = {i, {1.f, 0.f}, {0.f, 0.f}};   // the tiles tile-1 .. j+1, composed
            int64_t j = tile - 1;
            // The look-back waits without a bound, as the forward's does: a
            // workgroup takes its ticket when it starts, so every record it
            // waits for belongs to a workgroup that has started and will
            // publish it.
            while (true) {
                const uint64_t *iw = a.incl + (seq_rec + j) * (NC * 64);
                const uint64_t *aw = a.agg + (seq_rec + j) * (AW * 64);
                // Probe one word of tile j's carry-out (lane 0) and of its
                // operator (lane 1; the sequence's last tile publishes none);
                // read a whole record only once its probe word has landed.
                uint32_t pw = 0;
                bool pr = false;
                if (lane == 0)
                    pr = get_word(iw, epoch, pw);
                else if (lane == 1 && j > 0 && !a.strict)
                    pr = get_word(aw, epoch, pw);
                const uint64_t ready = __ballot(pr);
                if (ready & 1) {
                    uint32_t p0 = 0, p1 = 0;
                    bool ok = get_word(iw + lane, epoch, p0);
                    if constexpr (CPLX)
                        ok = get_word(iw + 64 + lane, epoch, p1) && ok;
                    if (__all(ok)) {
                        K = apply_op<CPLX>(acc, cf{__uint_as_float(p0), CPLX ? __uint_as_float(p1) : 0.f});
                        break;
                    }
                } else if (ready & 2) {
                    uint32_t q[5] = {0u, 0u, 0u, 0u, 0u};
                    bool okb = true;
#pragma unroll
                    for (int k = 0; k < AW; ++k)
                        okb = get_word(aw + k * 64 + lane, epoch, q[k]) && okb;
                    if (__all(okb)) {
                        GOp opj;
                        opj.sig = (int)min(q[0], (uint32_t)(NP - 1));
                        opj.m = {__uint_as_float(q[1]), CPLX ? __uint_as_float(q[3]) : 0.f};
                        opj.v = {__uint_as_float(q[2]), CPLX ? __uint_as_float(q[4]) : 0.f};
                        acc = compose_left<CPLX>(acc, opj);
                        --j;
                        continue;
                    }
                }
                __builtin_amdgcn_s_sleep(8);
            }
        }
        // ---- 4. every chunk's carry, then the tile's carry-out (gx0 for
        // the sequence's first tile)
#pragma unroll
        for (int k = 0; k < TC; ++k) {
            const GOp ok = op_of(k);
            if (lane < NP)
                s_k[k / G][(G - 1 - k % G) * NP + lane] = K;
            K = apply_op<CPLX>(ok, K);
        }
        if (tile + 1 < a.tiles) {
            uint64_t *const iw_own = a.incl + trec * (NC * 64);
            put_word(iw_own + lane, __float_as_uint(K.r), epoch);
            if constexpr (CPLX)
                put_word(iw_own + 64 + lane, __float_as_uint(K.i), epoch);
        } else if (a.gx0 && lane < N) {
            store_grad<CPLX>(a.gx0, seq * N + lane, K);
        }
    }
    __syncthreads();
    if (G == 1 && !has)
        return;   // the whole wave is idle
    // With several chunks per wave an idle lane group stays to the end: the
    // other groups gather their upstream gradients from its lanes.  Its
    // stores are dropped.
    io.act = io.act && has;
    const cf K = s_k[wave][lane];

    // ---- 5. backward through the chunk from K, writing the gradients
    const int64_t e0 = (seq * a.L + tw) * N;
    const uint64_t rows = (uint64_t)nvw * (uint64_t)N;
    const __amdgpu_buffer_rsrc_t ogb = make_rsrc(reinterpret_cast<Stored *>(a.gb) + e0, rows * sizeof(Stored));
    const __amdgpu_buffer_rsrc_t ogc = make_rsrc(reinterpret_cast<Stored *>(a.gc) + e0, rows * sizeof(Stored));
    const __amdgpu_buffer_rsrc_t ogd = make_rsrc(reinterpret_cast<DRaw *>(a.gd) + e0, rows * sizeof(DRaw));
    cf lc = K;   // A_{t+1}^H lambda_{t+1}, the part carried into step t
#pragma unroll
    for (int q = 0; q < kBT; ++q) {
        const int tt = kBT - 1 - q;
        const cf d = ds[tt];
        const cf cv = unpack_c<CPLX, BCBF>(cs[tt]);
        const uint32_t ent = pis[tt / 4] >> (8 * (tt % 4));
        if (tt < nv) {
            const float gq = gy_step<G>(a, gyr, (G == 1) ? tt : sofs + tt);
            const cf lam = {lc.r + gq * cv.r, lc.i - gq * cv.i};
            const int pi4 = (int)(((ent & 63u) + gbase) << 2);
            cf lg;
            lg.r = bperm_a(lam.r, pi4);
            lg.i = CPLX ? bperm_a(lam.i, pi4) : 0.f;
            const cf xt = xs[tt];
            const cf xp = (tt > 0) ? xs[tt > 0 ? tt - 1 : 0] : xin;
            uint32_t vo, so;
            io.template store_offs<Stored>(tt, io.vs, vo, so);
            bstore<Stored>(ogb, pack_vec<CPLX, BCBF>(lam), vo, so);
            bstore<Stored>(ogc, pack_vec<CPLX, BCBF>(cf{gq * xt.r, -gq * xt.i}), vo, so);
            io.template store_offs<DRaw>(tt, io.vd, vo, so);
            bstore<DRaw>(ogd, pack_d<CPLX>(cf{xp.r * lg.r + xp.i * lg.i, xp.r * lg.i - xp.i * lg.r}), vo, so);
            lc = {d.r * lg.r + d.i * lg.i, d.r * lg.i - d.i * lg.r};
        }
    }
}

// ---------------------------------------------------------------------------
// Host side.
// ---------------------------------------------------------------------------
struct BwdLayout {
    int NP;
    int64_t nch, S, tiles, tab_bytes, agg_bytes, incl_bytes, total;
};

// Lanes per chunk: N padded to 16, 32 or 64 (a wave runs 64 / NP chunks).
static int bwd_lanes(int N) { return N <= 16 ? 16 : N <= 32 ? 32 : 64; }

// Workspace: header | entry table [H][K][NP] | operator records | carry records.
static BwdLayout bwd_layout(int64_t B, int64_t H, int64_t L, int32_t N, int32_t K, uint32_t flags)
{
    BwdLayout lo;
    const int nc = (flags & PDSSM_COMPLEX) ? 2 : 1;
    lo.NP = bwd_lanes(N);
    lo.S = B * H;
    lo.nch = (L + kBT - 1) / kBT;
    const int64_t tc = (int64_t)kBW * (64 / lo.NP);   // chunks per tile
    lo.tiles = (lo.nch + tc - 1) / tc;
    const int64_t recs = lo.S * lo.tiles;
    auto up = [](int64_t n) { return (n + 255) / 256 * 256; };
    lo.tab_bytes = up(H * (int64_t)K * lo.NP * 2);
    lo.agg_bytes = up(recs * 64 * (1 + 2 * nc) * 8);
    lo.incl_bytes = up(recs * 64 * nc * 8);
    lo.total = (int64_t)sizeof(Header) + lo.tab_bytes + lo.agg_bytes + lo.incl_bytes;
    return lo;
}

// Aggregate records let a tile's carry skip ahead of unfinished tiles, at the
// cost of writing and polling them.  When the device holds up to this many
// workgroups per sequence, the plain chain (each tile waits for the tile just
// after it) keeps up with the tiles being worked on, and is used.  A link of
// the backward's chain is slower than the forward's (its look-back composes
// and publishes more words per lane), hence a lower bound than the forward's.
#ifndef PDSSM_BWD_STRICT_WGS_PER_SEQ
#define PDSSM_BWD_STRICT_WGS_PER_SEQ 4
#endif
constexpr int64_t kStrictWgsPerSeq = PDSSM_BWD_STRICT_WGS_PER_SEQ;

template <int NP, bool CPLX, bool BCBF>
static hipError_t launch_fused_t(BwdArgs a, hipStream_t st)
{
    // Resident workgroups per device, cached per device.
    static thread_local int c_dev = -1, c_wgs = 0;
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess)
        return e;
    if (dev != c_dev) {
        int per_cu = 0, cus = 0;
        e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, bwd_fused_kernel<NP, CPLX, BCBF>, kBW * 64, 0);
        if (e != hipSuccess)
            return e;
        e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
        if (e != hipSuccess)
            return e;
        c_wgs = (per_cu > 0 ? per_cu : 1) * (cus > 0 ? cus : 1);
        c_dev = dev;
    }
    const int64_t in_flight = (int64_t)a.total < c_wgs ? (int64_t)a.total : c_wgs;
    if (in_flight <= kStrictWgsPerSeq * a.S)
        a.strict = 1;
    hipLaunchKernelGGL((bwd_fused_kernel<NP, CPLX, BCBF>), dim3(a.total), dim3(kBW * 64), 0, st, a);
    return hipSuccess;
}

template <int NP>
static hipError_t launch_fused(const BwdArgs &a, bool cplx, bool bcbf, hipStream_t st)
{
    if (cplx)
        return bcbf ? launch_fused_t<NP, true, true>(a, st) : launch_fused_t<NP, true, false>(a, st);
    return bcbf ? launch_fused_t<NP, false, true>(a, st) : launch_fused_t<NP, false, false>(a, st);
}

}  // namespace pdssm

using namespace pdssm;

extern "C" size_t pdssm_scan_bwd_workspace_bytes(int64_t B, int64_t H, int64_t L, int32_t N,
                                                 int32_t K, uint32_t flags)
{
    if (check_dims(B, H, L, N, K) != PDSSM_OK || (flags & ~PDSSM_FLAGS_ALL))
        return 0;
    return (size_t)bwd_layout(B, H, L, N, K, flags).total;
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
    const BwdLayout lo = bwd_layout(B, H, L, N, K, flags);
    if (workspace_bytes < (size_t)lo.total)
        return PDSSM_ERR_WORKSPACE;
    if ((double)lo.S * (double)lo.tiles > 4.0e9)
        return PDSSM_ERR_DIM;   // tickets are 32-bit

    BwdArgs a = {};
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
    a.hdr = reinterpret_cast<Header *>(w);
    uint16_t *tab = reinterpret_cast<uint16_t *>(w + sizeof(Header));
    a.tab = tab;
    a.agg = reinterpret_cast<uint64_t *>(w + sizeof(Header) + lo.tab_bytes);
    a.incl = reinterpret_cast<uint64_t *>(w + sizeof(Header) + lo.tab_bytes + lo.agg_bytes);
    a.H = H;
    a.L = L;
    a.S = lo.S;
    a.nch = lo.nch;
    a.total = (uint32_t)(lo.S * lo.tiles);
    a.tiles = lo.tiles;
    a.N = N;
    a.K = K;
    a.sel_mode = flags & PDSSM_SEL_MASK;
    a.strict = (flags & PDSSM_DETERMINISTIC) ? 1 : 0;   // launch_fused may set it too
    a.y_bf16 = (flags & PDSSM_Y_BF16) ? 1 : 0;

    // New epoch and ticket, the entry table; on first use every record is cleared.
    rc = launch_prep(a.hdr, a.agg, (lo.agg_bytes + lo.incl_bytes) / 16, dict_idx, tab, H * (int64_t)K, N, lo.NP,
                     stream);
    if (rc != PDSSM_OK)
        return rc;
    const bool cplx = flags & PDSSM_COMPLEX, bcbf = flags & PDSSM_BC_BF16;
    hipError_t e;
    switch (lo.NP) {
    case 16: e = launch_fused<16>(a, cplx, bcbf, stream); break;
    case 32: e = launch_fused<32>(a, cplx, bcbf, stream); break;
    default: e = launch_fused<64>(a, cplx, bcbf, stream); break;
    }
    if (e != hipSuccess)
        return hip_status(e);
    return hip_status(hipGetLastError());
}
