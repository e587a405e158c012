// pdssm_scan.hip -- Flash PD-SSM forward recurrence scan for MI355X (gfx950).
//
// The path ("Flash PD-SSM: Memory-Optimized Structured Sparse State-Space
// Models", gist.science explainer, Technical Summary, Methodology sections 1
// and 3), as one kernel launch over tiles of the sequence:
//
//   a1  selection      argmax of the K router scores (or a stored index), then
//                      the dictionary row: the index map pi of P.
//   a2  P D step       x' = P (d * x) + b as an LDS scatter-add, lane = state.
//   a3  composition    each chunk's operator (pi, d, e) = A_last ... A_first
//                      applied to zero state, composed in O(N) by a gather and
//                      a multiply; chunks of a tile combine in log2 levels
//                      (Hillis-Steele over LDS).
//   a4  carry          tiles of one sequence chain through a carry record in
//                      the workspace: decoupled look-back over tile aggregates
//                      (Merrill & Garland's single-pass scan), with an atomic
//                      ticket so every tile only waits on tiles already running.
//   a5  readout        y_t = Re(c_t . x_t) with x_t = x_loc_t + (prefix operator)
//                      applied to the chunk's carry-in, in gather form, so the
//                      chunk's inputs are read from HBM exactly once.
//
// Per wave: G = 64/NP chunks of T steps (one per group of NP lanes).
// Per workgroup (tile): W waves, C = W*G chunks, TILE = C*T steps.
#include <hip/hip_runtime.h>

#include <cstdio>
#include <cstring>
#include <string>
#include <type_traits>

#include "pdssm.h"
#include "pdssm_device.h"

namespace pdssm {

struct ScanArgs {
    const void *sel;
    const int32_t *dict;
    const float *diag;
    const void *b;
    const void *c;
    void *y;
    float *xfinal;
    const float *x0;
    Header *hdr;
    uint64_t *agg;
    uint64_t *incl;
    int64_t H, L, S, n_tiles;
    int N, K;
    uint32_t sel_mode;
    int y_bf16;
    int dict_lds;   // the head's entry table fits in LDS
    const uint32_t *tab;   // [H][K][NP]: pi | rank << 8 | indegree << 16 (see prep_kernel)
};

// Scan tiling: a chunk is kScanT steps of one group of NP lanes; a wave holds
// 64/NP chunks; a workgroup (tile) holds kScanW waves.
#ifndef PDSSM_SCAN_T
#define PDSSM_SCAN_T 16
#endif
#ifndef PDSSM_SCAN_W
#define PDSSM_SCAN_W 7
#endif
#ifndef PDSSM_SCAN_D
#define PDSSM_SCAN_D 8
#endif
#ifndef PDSSM_SCAN_WAVES_PER_EU
#define PDSSM_SCAN_WAVES_PER_EU 1
#endif
constexpr int kScanT = PDSSM_SCAN_T;
constexpr int kScanW = PDSSM_SCAN_W;
constexpr int kScanD = PDSSM_SCAN_D;   // steps of inputs in flight per lane (register ring)
constexpr int kDictLdsMax = 32768;   // bytes of the head's entry table kept in LDS
constexpr int kRegions = 4;          // collision-free scatter regions (ranks 0..3)

__host__ __device__ constexpr int scan_tile_steps(int NP) { return kScanW * (64 / NP) * kScanT; }

template <int NP, bool CPLX>
__host__ __device__ constexpr int agg_words() { return NP * (1 + 2 * (CPLX ? 2 : 1)); }
template <int NP, bool CPLX>
__host__ __device__ constexpr int incl_words() { return NP * (CPLX ? 2 : 1); }

// Raw per-step storage of b and c in registers (bf16 pairs stay packed).
template <bool CPLX, bool BCBF>
struct RawVec {
    using type = typename std::conditional<BCBF, uint32_t, typename std::conditional<CPLX, float2, float>::type>::type;
};

template <bool CPLX, bool BCBF>
__device__ __forceinline__ typename RawVec<CPLX, BCBF>::type load_raw(const void *__restrict__ p, int64_t e)
{
    if constexpr (BCBF) {
        if constexpr (CPLX)
            return reinterpret_cast<const uint32_t *>(p)[e];
        else
            return (uint32_t)reinterpret_cast<const uint16_t *>(p)[e];
    } else if constexpr (CPLX) {
        return reinterpret_cast<const float2 *>(p)[e];
    } else {
        return reinterpret_cast<const float *>(p)[e];
    }
}

template <bool CPLX, bool BCBF>
__device__ __forceinline__ cf unpack_raw(typename RawVec<CPLX, BCBF>::type v)
{
    if constexpr (BCBF)
        return {bf16_lo(v), CPLX ? bf16_hi(v) : 0.f};
    else if constexpr (CPLX)
        return {v.x, v.y};
    else
        return {v, 0.f};
}

template <bool CPLX, bool BCBF>
__device__ __forceinline__ typename RawVec<CPLX, BCBF>::type zero_raw()
{
    if constexpr (BCBF)
        return 0u;
    else if constexpr (CPLX)
        return make_float2(0.f, 0.f);
    else
        return 0.f;
}

template <bool CPLX, bool BCBF>
__device__ __forceinline__ typename RawVec<CPLX, BCBF>::type bperm_raw(typename RawVec<CPLX, BCBF>::type v, int src)
{
    if constexpr (BCBF)
        return bperm(v, src);
    else if constexpr (CPLX)
        return make_float2(bperm(v.x, src), bperm(v.y, src));
    else
        return bperm(v, src);
}

// ---------------------------------------------------------------------------
// a4: the carry of one tile, run by wave 0 with lane = state (lanes >= NP
// idle but convergent).  (api, ad, ae) is the tile's inclusive operator;
// returns the carry into the tile and publishes the carry out of it.
// ---------------------------------------------------------------------------
template <int NP, bool CPLX>
__device__ cf tile_carry(const ScanArgs &a, int64_t tile, int64_t seq, uint32_t epoch, int api,
                         cf ad, cf ae, cf *scr)
{
    constexpr int NC = CPLX ? 2 : 1;
    constexpr int AW = agg_words<NP, CPLX>(), IW = incl_words<NP, CPLX>();
    const int lane = threadIdx.x & 63;
    const bool act = lane < NP;
    cf xin = {0.f, 0.f};

    if (tile == 0) {
        if (a.x0 && lane < a.N) {
            const int64_t e = seq * a.N + lane;
            xin = load_diag<CPLX>(a.x0, e);
        }
    } else {
        // Publish this tile's aggregate so later tiles need not wait for the carry.
        uint64_t *aw = a.agg + (tile * a.S + seq) * AW;
        if (act) {
            put_word(aw + lane, (uint32_t)api, epoch);
            put_word(aw + NP + lane * NC, __float_as_uint(ad.r), epoch);
            put_word(aw + NP + NP * NC + lane * NC, __float_as_uint(ae.r), epoch);
            if constexpr (CPLX) {
                put_word(aw + NP + lane * NC + 1, __float_as_uint(ad.i), epoch);
                put_word(aw + NP + NP * NC + lane * NC + 1, __float_as_uint(ae.i), epoch);
            }
        }
        // Look back: (bpi, bd, be) = tiles j+1 .. tile-1 composed, latest last.
        int bpi = lane;
        cf bd = {1.f, 0.f}, be = {0.f, 0.f};
        int64_t j = tile - 1;
        while (true) {
            const int64_t rj = j * a.S + seq;
            bool ok = true;
            cf X = {0.f, 0.f};
            if (act) {
                const uint64_t *iw = a.incl + rj * IW;
                uint32_t u0 = 0, u1 = 0;
                ok = get_word(iw + lane * NC, epoch, u0);
                if constexpr (CPLX)
                    ok = get_word(iw + lane * NC + 1, epoch, u1) && ok;
                X = {__uint_as_float(u0), __uint_as_float(u1)};
            }
            if (__all(ok)) {
                xin = scatter_add<CPLX>(scr, lane, 0, bpi, cmul(bd, X), be);
                break;
            }
            if (j > 0) {
                ok = true;
                int p = lane;
                cf d = {1.f, 0.f}, e = {0.f, 0.f};
                if (act) {
                    const uint64_t *w = a.agg + rj * AW;
                    uint32_t up = 0, dr = 0, di = 0, er = 0, ei = 0;
                    ok = get_word(w + lane, epoch, up);
                    ok = get_word(w + NP + lane * NC, epoch, dr) && ok;
                    ok = get_word(w + NP + NP * NC + lane * NC, epoch, er) && ok;
                    if constexpr (CPLX) {
                        ok = get_word(w + NP + lane * NC + 1, epoch, di) && ok;
                        ok = get_word(w + NP + NP * NC + lane * NC + 1, epoch, ei) && ok;
                    }
                    p = (int)min(up, (uint32_t)(NP - 1));
                    d = {__uint_as_float(dr), __uint_as_float(di)};
                    e = {__uint_as_float(er), __uint_as_float(ei)};
                }
                if (__all(ok)) {
                    // acc <- acc o agg_j  (acc is later in time)
                    const int npi = bperm(bpi, p);
                    cf gd;
                    gd.r = bperm(bd.r, p);
                    gd.i = CPLX ? bperm(bd.i, p) : 0.f;
                    const cf ne = scatter_add<CPLX>(scr, lane, 0, bpi, cmul(bd, e), be);
                    bpi = npi;
                    bd = cmul(gd, d);
                    be = ne;
                    --j;
                    continue;
                }
            }
            __builtin_amdgcn_s_sleep(2);
        }
    }

    const cf xout = scatter_add<CPLX>(scr, lane, 0, api, cmul(ad, xin), ae);
    if (act) {
        uint64_t *iw = a.incl + (tile * a.S + seq) * IW;
        put_word(iw + lane * NC, __float_as_uint(xout.r), epoch);
        if constexpr (CPLX)
            put_word(iw + lane * NC + 1, __float_as_uint(xout.i), epoch);
    }
    if (tile == a.n_tiles - 1 && a.xfinal && lane < a.N) {
        const int64_t e = (seq * a.N + lane) * NC;
        a.xfinal[e] = xout.r;
        if constexpr (CPLX)
            a.xfinal[e + 1] = xout.i;
    }
    return xin;
}

// ---------------------------------------------------------------------------
// The fused scan kernel: one workgroup per tile.  Workgroups take tiles from
// an atomic ticket in tile-major order (index u = tile * S + seq), so every
// tile waits only on tiles that hold a smaller ticket -- tiles that are
// already running or done -- and the look-back cannot deadlock.
//
// Waves 0..W-1 ("chunk waves") each own G chunks of T steps.  Wave W (the
// "carry wave") stages the dictionary table, chains the chunk operators of
// the tile and runs the look-back.  The two roles run on separate
// wave-uniform paths that meet only at barriers, so the chunk waves'
// per-step readout state never has to share registers with the carry code.
// ---------------------------------------------------------------------------
template <int NP, bool CPLX, bool BCBF>
__global__ void __launch_bounds__((kScanW + 1) * 64) __attribute__((amdgpu_waves_per_eu(PDSSM_SCAN_WAVES_PER_EU))) scan_kernel(ScanArgs a)
{
    constexpr int W = kScanW, T = kScanT, G = 64 / NP, C = W * G, TILE = C * T, SLOTS = W * 64;
    using Raw = typename RawVec<CPLX, BCBF>::type;
    using DRaw = typename std::conditional<CPLX, float2, float>::type;
    using Stored = typename std::conditional<BCBF, typename std::conditional<CPLX, uint32_t, uint16_t>::type, Raw>::type;
    // Entry table: the head's [K][NP] (pi | rank << 8 | indegree << 16) when
    // it fits, else this tile's entries per (wave, step, lane).
    extern __shared__ __attribute__((aligned(16))) uint32_t s_tab[];
    __shared__ int16_t s_sel[W][G * T];
    __shared__ cf s_reg[W][kRegions + 1][64];   // scatter regions; the last one takes ranks >= kRegions
    __shared__ cf s_scr[W + 1][64];
    __shared__ int s_pi[SLOTS];   // chunk operators, then their inclusive prefixes
    __shared__ cf s_d[SLOTS];
    __shared__ cf s_e[SLOTS];
    __shared__ cf s_xin[64];
    __shared__ uint32_t s_ticket;

    // Tile indices, sequences and heads fit 32 bits (the host checks).
    const uint32_t S32 = (uint32_t)a.S, H32 = (uint32_t)a.H;
    const int N = a.N, K = a.K;
    const int tid = threadIdx.x;
    const int wave = tid >> 6, lane = tid & 63;
    if (tid == 0)
        s_ticket = atomicAdd(&a.hdr->ticket, 1u);
    __syncthreads();
    const uint32_t u = s_ticket;
    const uint32_t tile = u / S32, seq = u - tile * S32;
    const uint32_t h = seq % H32;
    const int64_t tile_t0 = (int64_t)tile * TILE;
    const int64_t seq_row = (int64_t)seq * a.L;
    const uint32_t *tab_h = a.tab + h * (int64_t)K * NP;

    if (wave == W) {
        // ================= carry wave =================
        // The head's entry table straight to LDS (16 bytes per lane per
        // instruction, no registers involved).
        if (a.dict_lds) {
            const int tab_vecs = (K * NP) >> 2;   // 4 entries per 16 bytes
            const uint4 *src = reinterpret_cast<const uint4 *>(tab_h);
            for (int w0 = 0; w0 < tab_vecs; w0 += 64) {
                const int w = min(w0 + lane, tab_vecs - 1);
                __builtin_amdgcn_global_load_lds(
                    src + w, (__attribute__((address_space(3))) void *)(reinterpret_cast<uint8_t *>(s_tab) + w0 * 16),
                    16, 0, 0);
            }
        }
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // the copy has landed
        const uint32_t epoch = a.hdr->epoch;
        __syncthreads();   // (1) table ready
        __syncthreads();   // (2) chunk operators ready

        // ---- a3: chain the C chunk operators in time order; slot c then
        // holds the operator of chunks 0..c of the tile.  Lane = state;
        // lanes >= NP carry an identity that touches only their own slot.
        const bool act = lane < NP;
        const int l = act ? lane : 0;
        int ppi = act ? lane : 0;
        cf pd = {1.f, 0.f}, pe = {0.f, 0.f};
        cf *scr = s_scr[W];
        for (int c = 0; c < C; ++c) {
            const int base = c * NP;
            const int cpi = act ? s_pi[base + l] : lane;
            const cf cd = act ? s_d[base + l] : cf{1.f, 0.f};
            const cf ce = act ? s_e[base + l] : cf{0.f, 0.f};
            // (op_c o prefix): pi[j] = cpi[ppi[j]], d[j] = cd[ppi[j]] * pd[j],
            // e = P_c D_c pe + ce.
            const int npi = s_pi[base + ppi];
            const cf gd = s_d[base + ppi];
            const cf ne = scatter_add<CPLX>(scr, lane, 0, cpi, act ? cmul(cd, pe) : cf{0.f, 0.f}, ce);
            if (act) {
                ppi = npi;
                pd = cmul(gd, pd);
                pe = ne;
                s_pi[base + lane] = ppi;
                s_d[base + lane] = pd;
                s_e[base + lane] = pe;
            }
            lds_order();
        }
        // ---- a4: carry into / out of the tile.
        s_xin[lane] = tile_carry<NP, CPLX>(a, (int64_t)tile, (int64_t)seq, epoch, act ? ppi : lane,
                                           act ? pd : cf{1.f, 0.f}, act ? pe : cf{0.f, 0.f}, scr);
        __syncthreads();   // (3) carry ready
        return;
    }

    // ================= chunk waves =================
    const int g = lane / NP, i = lane % NP, chunk = wave * G + g, gbase = g * NP;
    const int icl = min(i, N - 1);
    const bool sel_fast = select_fast_ok(a.sel_mode, K, lanes_per_step<G * T>(), G * T);

    // ---- Router-score slice of this wave's steps first (the selection
    // needs it before any step can run) ...
    ScoreSlice sc;
    if (sel_fast)
        sc = select_issue<G * T>(a.sel, a.sel_mode, K, a.L, seq_row, tile_t0 + (int64_t)wave * G * T, lane);
    // ... then the chunk's step inputs, streamed through a ring of D
    // register slots: the first D steps now, step t + D once step t is used.
    // Addresses are clamped in range (steps past the end reload the last
    // row), so every load is unconditional.
    constexpr int D = kScanD < T ? kScanD : T;
    const int64_t tc0 = tile_t0 + (int64_t)chunk * T;
    const int64_t row0 = seq_row + (tc0 < a.L ? tc0 : a.L - 1);
    const int last = tc0 < a.L ? (int)min((int64_t)(T - 1), a.L - 1 - tc0) : 0;
    const DRaw *dbase = reinterpret_cast<const DRaw *>(a.diag) + row0 * N;
    const Stored *bbase = reinterpret_cast<const Stored *>(a.b) + row0 * N;
    const Stored *cbase = reinterpret_cast<const Stored *>(a.c) + row0 * N;
    DRaw dv[D];
    Raw bv[D], cv[D];
    auto fetch = [&](int tt) {
        const int off = min(tt, last) * N + icl;
        dv[tt % D] = dbase[off];
        bv[tt % D] = (Raw)bbase[off];
        cv[tt % D] = (Raw)cbase[off];
    };
#pragma unroll
    for (int tt = 0; tt < D; ++tt)
        fetch(tt);
    const int64_t tw0 = tile_t0 + (int64_t)wave * G * T;   // first step of the wave

    // ---- a1: selection of this wave's G*T consecutive steps.
    if (sel_fast)
        select_finish<G * T>(sc, a.sel_mode, K, a.L, tw0, s_sel[wave], lane);
    else
        wave_select<G * T>(a.sel, a.sel_mode, K, a.L, seq_row, tw0, s_sel[wave], lane);

    // ---- When the head's entry table does not fit in LDS, this wave's
    // entries straight from the table in memory.
    if (!a.dict_lds) {
        lds_order();
        for (int tt = 0; tt < T; ++tt) {
            const int k = s_sel[wave][g * T + tt];
            s_tab[(wave * T + tt) * 64 + lane] = tab_h[(int64_t)k * NP + i];
        }
    }
    __syncthreads();   // (1) table ready

    // ---- a2 + chunk-local a3: recurrence from zero state, and the prefix
    // operator of the chunk (source j sits at pacc[j] with factor dacc[j]).
    cf *scr = s_scr[wave];
    cf x = {0.f, 0.f};
    int pacc = i;
    cf dacc = {1.f, 0.f};
    float q[T], gr[T], gi[T];
    Raw craw_prev = zero_raw<CPLX, BCBF>();
    // With one chunk per wave the step's selection is wave-uniform: keep
    // the chunk's selections in one register and broadcast them per step.
    int selv = 0;
    if constexpr (G == 1)
        selv = s_sel[wave][lane % T];
    auto entry = [&](int tt) {
        if (!a.dict_lds)
            return s_tab[(wave * T + tt) * 64 + lane];
        const int k = (G == 1) ? __builtin_amdgcn_readlane(selv, tt) : (int)s_sel[wave][g * T + tt];
        return s_tab[k * NP + i];
    };
    uint32_t ent_next = entry(0);
#pragma unroll
    for (int tt = 0; tt < T; ++tt) {
        const bool valid = (tc0 + tt < a.L) && (i < N);
        const uint32_t ent = ent_next;
        if (tt + 1 < T)
            ent_next = entry(tt + 1);
        const int p = valid ? (int)(ent & 0xFF) : i;
        const int rank = valid ? (int)((ent >> 8) & 0xFF) : 0;
        const int deg = valid ? (int)((ent >> 16) & 0xFF) : 1;
        const int sl = tt % D;
        cf d;
        if constexpr (CPLX)
            d = valid ? cf{dv[sl].x, dv[sl].y} : cf{1.f, 0.f};
        else
            d = valid ? cf{dv[sl], 0.f} : cf{1.f, 0.f};
        const cf b = valid ? unpack_raw<CPLX, BCBF>(bv[sl]) : cf{0.f, 0.f};
        const Raw craw = valid ? cv[sl] : zero_raw<CPLX, BCBF>();
        const cf c = unpack_raw<CPLX, BCBF>(craw);
        if (tt + D < T)
            fetch(tt + D);
        // x_t = P_t (d_t * x_{t-1}) + b_t.  Source j goes to region rank(j)
        // at row pi(j): within a region every row has at most one source, so
        // plain stores suffice.  Row i then reads the regions below its
        // in-degree -- exactly the slots written in this step, so stale
        // slots are never read and nothing needs clearing.  Sources of rank
        // >= kRegions (rare) add atomically into the last region.
        {
            const cf v = cmul(d, x);
            const int ri = rank < kRegions ? rank : kRegions;
            s_reg[wave][ri][gbase + p] = v;
            lds_order();
            if (__any(rank >= kRegions)) {
                if (rank >= kRegions) {
                    atomicAdd(&s_reg[wave][kRegions - 1][gbase + p].r, v.r);
                    if constexpr (CPLX)
                        atomicAdd(&s_reg[wave][kRegions - 1][gbase + p].i, v.i);
                }
                lds_order();
            }
            // All regions are read back to back (one LDS round trip); rows
            // keep only the regions below their in-degree.
            cf uu[kRegions];
#pragma unroll
            for (int r = 0; r < kRegions; ++r)
                uu[r] = s_reg[wave][r][lane];
            lds_order();
            cf sum = b;
#pragma unroll
            for (int r = 0; r < kRegions; ++r) {
                sum.r += deg > r ? uu[r].r : 0.f;
                sum.i += deg > r ? uu[r].i : 0.f;
            }
            x = sum;
        }
        q[tt] = c.r * x.r - c.i * x.i;
        // Extend the prefix operator by step t (source j sits at pacc[j]
        // with factor dacc[j]); the same gather also brings the readout
        // weight of step t-1:  Re(c_{t-1} . P D X) = Re(sum_j g_{t-1}[j] X[j])
        // with g_{t-1}[j] = c_{t-1}[pacc_{t-1}[j]] * dacc_{t-1}[j].
        const int src = gbase + pacc;
        const int npacc = bperm(p, src);
        cf dd;
        dd.r = bperm(d.r, src);
        dd.i = CPLX ? bperm(d.i, src) : 0.f;
        if (tt > 0) {
            const cf gg = cmul(unpack_raw<CPLX, BCBF>(bperm_raw<CPLX, BCBF>(craw_prev, src)), dacc);
            gr[tt - 1] = gg.r;
            gi[tt - 1] = gg.i;
        }
        dacc = cmul(dd, dacc);
        pacc = npacc;
        craw_prev = craw;
    }
    {
        const cf gg = cmul(unpack_raw<CPLX, BCBF>(bperm_raw<CPLX, BCBF>(craw_prev, gbase + pacc)), dacc);
        gr[T - 1] = gg.r;
        gi[T - 1] = gg.i;
    }

    // ---- The chunk's operator (pi, d, e) = (pacc, dacc, x) for the carry wave.
    s_pi[tid] = pacc;
    s_d[tid] = dacc;
    s_e[tid] = x;
    __syncthreads();   // (2) chunk operators ready
    __syncthreads();   // (3) carry ready

    // ---- a5: carry into this chunk, then the readout
    //   y_t = sum_j ( Re(c_t[j] x_loc_t[j]) + Re(g_t[j] X_chunk[j]) ).
    const cf xt = s_xin[i];
    int ppi = i;
    cf pd = {1.f, 0.f}, pe = {0.f, 0.f};
    if (chunk > 0) {
        ppi = s_pi[tid - NP];
        pd = s_d[tid - NP];
        pe = s_e[tid - NP];
    }
    const cf xc = scatter_add<CPLX>(scr, lane, gbase, ppi, cmul(pd, xt), pe);
#pragma unroll
    for (int tt = 0; tt < T; ++tt) {
        q[tt] += gr[tt] * xc.r;
        if constexpr (CPLX)
            q[tt] -= gi[tt] * xc.i;
    }
    group_transpose_sum<NP, T>(q, i);
    using BF = Butterfly<NP, T>;
    if ((i & ((1 << BF::NPLAIN) - 1)) == 0) {
#pragma unroll
        for (int r = 0; r < BF::RF; ++r) {
            const int tt = r + BF::RF * (i >> BF::NPLAIN);
            const int64_t t = tc0 + tt;
            if (t < a.L) {
                if (a.y_bf16)
                    reinterpret_cast<uint16_t *>(a.y)[seq_row + t] = f32_to_bf16_rne(q[r]);
                else
                    reinterpret_cast<float *>(a.y)[seq_row + t] = q[r];
            }
        }
    }
}

// ---------------------------------------------------------------------------
// Per-call preparation.
//  * Blocks >= 1, one wave per dictionary entry (h, k): the entry table
//    tab[h][k][j] = pi(j) | rank(j) << 8 | deg(j) << 16, where rank(j)
//    counts the sources j' < j with the same destination and deg(j) is the
//    number of sources whose destination is j.  Padding sources j >= N map
//    to themselves with rank 0 and in-degree 1.
//  * Block 0: new epoch and ticket reset; on first use (or after the epoch
//    wraps) clear every carry record.
// ---------------------------------------------------------------------------
constexpr int kPrepThreads = 1024;

__global__ void __launch_bounds__(kPrepThreads) prep_kernel(Header *hdr, uint4 *recs, int64_t n16,
                                                            const int32_t *dict, uint32_t *tab,
                                                            int64_t entries, int N, int NP)
{
    if (blockIdx.x > 0) {
        const int lane = threadIdx.x & 63;
        const int64_t e = (int64_t)(blockIdx.x - 1) * (kPrepThreads / 64) + (threadIdx.x >> 6);
        if (e >= entries || lane >= NP)
            return;
        const int pi = lane < N ? (int)min((unsigned)dict[e * N + lane], (unsigned)(N - 1)) : lane;
        int rank = 0, deg = 0;
        for (int jj = 0; jj < N; ++jj) {
            const int pj = __builtin_amdgcn_readlane(pi, jj);
            rank += (jj < lane && pj == pi) ? 1 : 0;
            deg += (pj == lane) ? 1 : 0;
        }
        if (lane >= N)
            deg = 1;   // padding rows hold their own (zero) state
        tab[e * NP + lane] = (uint32_t)pi | ((uint32_t)min(rank, 255) << 8) | ((uint32_t)deg << 16);
        return;
    }
    __shared__ int s_fresh;
    if (threadIdx.x == 0)
        s_fresh = (hdr->magic != kMagic) || (hdr->epoch >= kEpochLimit) || (hdr->epoch == 0);
    __syncthreads();
    if (s_fresh) {
        const uint4 z = {0u, 0u, 0u, 0u};
        for (int64_t w = threadIdx.x; w < n16; w += blockDim.x)
            recs[w] = z;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        if (s_fresh) {
            hdr->magic = kMagic;
            hdr->epoch = 1;
        } else {
            hdr->epoch = hdr->epoch + 1;
        }
        hdr->ticket = 0;
    }
}

// ---------------------------------------------------------------------------
// pdssm_select: one thread per step.
// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(256) select_kernel(const void *src, uint32_t mode, int32_t *out,
                                                     int64_t steps, int K)
{
    for (int64_t s = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; s < steps;
         s += (int64_t)gridDim.x * blockDim.x)
        out[s] = select_step(src, mode, s, K);
}

// ---------------------------------------------------------------------------
// pdssm_compose: per tile, the chunk operators (pi, d) and their in-tile
// combination; then per sequence, the tile operators in time order.
// ---------------------------------------------------------------------------
struct ComposeArgs {
    const void *sel;
    const int32_t *dict;
    const float *diag;
    int32_t *pi_out;
    float *d_out;
    int32_t *tile_pi;   // [S * n_tiles][NP]
    float *tile_d;      // [S * n_tiles][NP][NC]
    int64_t H, L, S, n_tiles;
    int N, K;
    uint32_t sel_mode;
};

// Compose tiling (independent of the scan's): chunks of kCompT steps, kCompW waves.
constexpr int kCompT = 32;
constexpr int kCompW = 4;
__host__ __device__ constexpr int compose_tile_steps(int NP) { return kCompW * (64 / NP) * kCompT; }

template <int NP, bool CPLX>
__global__ void __launch_bounds__(kCompW * 64) compose_tiles_kernel(ComposeArgs a)
{
    constexpr int G = 64 / NP, C = kCompW * G, T = kCompT, TILE = C * T, SLOTS = kCompW * 64;
    constexpr int NC = CPLX ? 2 : 1;
    __shared__ int16_t s_sel[kCompW][G * T];
    __shared__ int s_pi[2][SLOTS];
    __shared__ cf s_d[2][SLOTS];

    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int g = lane / NP, i = lane % NP, chunk = wave * G + g, gbase = g * NP;
    const int64_t rec = blockIdx.x;                    // = seq * n_tiles + tile
    const int64_t seq = rec / a.n_tiles, tile = rec - seq * a.n_tiles;
    const int64_t h = seq % a.H;
    const int64_t tile_t0 = tile * TILE, seq_row = seq * a.L;

    for (int q = lane; q < G * T; q += 64) {
        const int64_t t = tile_t0 + (int64_t)(wave * G) * T + q;
        int k = 0;
        if (t < a.L)
            k = select_step(a.sel, a.sel_mode, seq_row + t, a.K);
        s_sel[wave][q] = (int16_t)k;
    }
    lds_order();

    const int64_t tc0 = tile_t0 + (int64_t)chunk * T;
    const int32_t *dict_h = a.dict + h * (int64_t)a.K * a.N;
    int pacc = i;
    cf dacc = {1.f, 0.f};
#pragma unroll 8
    for (int tt = 0; tt < T; ++tt) {
        const int64_t t = tc0 + tt;
        const bool valid = (t < a.L) && (i < a.N);
        int pit = i;
        cf d = {1.f, 0.f};
        if (valid) {
            const int k = s_sel[wave][g * T + tt];
            pit = (int)min((unsigned)dict_h[(int64_t)k * a.N + i], (unsigned)(a.N - 1));
            d = load_diag<CPLX>(a.diag, (seq_row + t) * a.N + i);
        }
        const int src = gbase + pacc;
        const int npacc = __shfl(pit, src);
        cf dd;
        dd.r = __shfl(d.r, src);
        dd.i = CPLX ? __shfl(d.i, src) : 0.f;
        dacc = cmul(dd, dacc);
        pacc = npacc;
    }

    int opi = pacc;
    cf opd = dacc;
    s_pi[0][tid] = opi;
    s_d[0][tid] = opd;
    __syncthreads();
    int buf = 0;
#pragma unroll
    for (int s = 1; s < C; s <<= 1) {
        const int nb = buf ^ 1;
        if (chunk >= s) {
            const int es = tid - s * NP;
            const int p1 = s_pi[buf][es];
            const cf d1 = s_d[buf][es];
            const int ls = tid - i + p1;
            opi = s_pi[buf][ls];
            opd = cmul(s_d[buf][ls], d1);
        }
        s_pi[nb][tid] = opi;
        s_d[nb][tid] = opd;
        __syncthreads();
        buf = nb;
    }
    if (chunk == C - 1) {
        a.tile_pi[rec * NP + i] = opi;
        a.tile_d[(rec * NP + i) * NC] = opd.r;
        if constexpr (CPLX)
            a.tile_d[(rec * NP + i) * NC + 1] = opd.i;
    }
}

template <int NP, bool CPLX>
__global__ void __launch_bounds__(64) compose_final_kernel(ComposeArgs a)
{
    constexpr int NC = CPLX ? 2 : 1;
    const int lane = threadIdx.x;
    const int64_t seq = blockIdx.x;
    int pacc = lane < NP ? lane : 0;
    cf dacc = {1.f, 0.f};
    for (int64_t r = 0; r < a.n_tiles; ++r) {
        const int64_t rec = seq * a.n_tiles + r;
        // later tile r after the accumulated earlier ones
        const int tp = lane < NP ? a.tile_pi[rec * NP + lane] : 0;
        cf td = {1.f, 0.f};
        if (lane < NP) {
            td.r = a.tile_d[(rec * NP + lane) * NC];
            if constexpr (CPLX)
                td.i = a.tile_d[(rec * NP + lane) * NC + 1];
        }
        const int npacc = __shfl(tp, pacc);
        cf dd;
        dd.r = __shfl(td.r, pacc);
        dd.i = CPLX ? __shfl(td.i, pacc) : 0.f;
        dacc = cmul(dd, dacc);
        pacc = npacc;
    }
    if (lane < a.N) {
        a.pi_out[seq * a.N + lane] = pacc;
        a.d_out[(seq * a.N + lane) * NC] = dacc.r;
        if constexpr (CPLX)
            a.d_out[(seq * a.N + lane) * NC + 1] = dacc.i;
    }
}

// ---------------------------------------------------------------------------
// Host side.
// ---------------------------------------------------------------------------
static thread_local std::string g_err;

static int pad_states(int N) { return N <= 8 ? 8 : N <= 16 ? 16 : N <= 32 ? 32 : 64; }

static bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

static int check_dims(int64_t B, int64_t H, int64_t L, int32_t N, int32_t K)
{
    if (B < 1 || H < 1 || L < 1 || N < 1 || N > 64 || K < 1 || K > 32767)
        return PDSSM_ERR_DIM;
    // Element counts must fit int64 and tile tickets a uint32.
    const double steps = (double)B * (double)H * (double)L;
    if (steps * 64.0 * 8.0 > 9.0e18)
        return PDSSM_ERR_DIM;
    const int NP = pad_states(N);
    const int64_t n_tiles = (L + scan_tile_steps(NP) - 1) / scan_tile_steps(NP);
    const int64_t n_ctiles = (L + compose_tile_steps(NP) - 1) / compose_tile_steps(NP);
    if ((double)B * (double)H * (double)(n_tiles > n_ctiles ? n_tiles : n_ctiles) > 2.0e9)
        return PDSSM_ERR_DIM;
    return PDSSM_OK;
}

struct Layout {
    int NP;
    int64_t n_tiles, n_ctiles, S, tab_bytes, agg_bytes, incl_bytes, compose_bytes, total;
};

static Layout layout_of(int64_t B, int64_t H, int64_t L, int32_t N, int32_t K, uint32_t flags)
{
    Layout lo;
    lo.NP = pad_states(N);
    const int nc = (flags & PDSSM_COMPLEX) ? 2 : 1;
    lo.n_tiles = (L + scan_tile_steps(lo.NP) - 1) / scan_tile_steps(lo.NP);
    lo.n_ctiles = (L + compose_tile_steps(lo.NP) - 1) / compose_tile_steps(lo.NP);
    lo.S = B * H;
    const int64_t recs = lo.n_tiles * lo.S;
    lo.agg_bytes = recs * lo.NP * (1 + 2 * nc) * 8;
    lo.incl_bytes = recs * lo.NP * nc * 8;
    lo.compose_bytes = lo.n_ctiles * lo.S * lo.NP * (1 + nc) * 4;
    lo.tab_bytes = (H * (int64_t)K * lo.NP * 4 + 255) / 256 * 256;
    const int64_t scan = lo.tab_bytes + lo.agg_bytes + lo.incl_bytes;
    lo.total = (int64_t)sizeof(Header) + ((scan > lo.compose_bytes ? scan : lo.compose_bytes) + 15) / 16 * 16;
    return lo;
}

static int hip_status(hipError_t e)
{
    if (e == hipSuccess)
        return PDSSM_OK;
    g_err = std::string("HIP error: ") + hipGetErrorString(e);
    return PDSSM_ERR_HIP;
}

template <int NP, bool CPLX, bool BCBF>
static hipError_t launch_scan(const ScanArgs &a, hipStream_t st)
{
    const size_t dyn = a.dict_lds ? (((size_t)a.K * NP * 4 + 15) & ~(size_t)15)
                                  : (size_t)kScanW * kScanT * 64 * 4;
    hipLaunchKernelGGL((scan_kernel<NP, CPLX, BCBF>), dim3((unsigned)(a.n_tiles * a.S)),
                       dim3((kScanW + 1) * 64), dyn, st, a);
    return hipSuccess;
}

template <int NP>
static hipError_t dispatch_scan(const ScanArgs &a, bool cplx, bool bcbf, hipStream_t st)
{
    if (cplx)
        return bcbf ? launch_scan<NP, true, true>(a, st) : launch_scan<NP, true, false>(a, st);
    return bcbf ? launch_scan<NP, false, true>(a, st) : launch_scan<NP, false, false>(a, st);
}

template <int NP>
static void dispatch_compose(const ComposeArgs &a, bool cplx, hipStream_t st)
{
    const dim3 tiles((unsigned)(a.n_tiles * a.S)), seqs((unsigned)a.S);   // n_tiles = compose tiles
    if (cplx) {
        hipLaunchKernelGGL((compose_tiles_kernel<NP, true>), tiles, dim3(kCompW * 64), 0, st, a);
        hipLaunchKernelGGL((compose_final_kernel<NP, true>), seqs, dim3(64), 0, st, a);
    } else {
        hipLaunchKernelGGL((compose_tiles_kernel<NP, false>), tiles, dim3(kCompW * 64), 0, st, a);
        hipLaunchKernelGGL((compose_final_kernel<NP, false>), seqs, dim3(64), 0, st, a);
    }
}

}  // namespace pdssm

using namespace pdssm;

extern "C" size_t pdssm_scan_workspace_bytes(int64_t B, int64_t H, int64_t L, int32_t N,
                                             int32_t K, uint32_t flags)
{
    if (check_dims(B, H, L, N, K) != PDSSM_OK || (flags & ~PDSSM_FLAGS_ALL))
        return 0;
    return (size_t)layout_of(B, H, L, N, K, flags).total;
}

extern "C" int pdssm_scan_fwd(const void *sel_or_logits, const int32_t *dict_idx, const void *diag,
                              const void *b, const void *c, void *y, void *x_final, int64_t B,
                              int64_t H, int64_t L, int32_t N, int32_t K, uint32_t flags,
                              const void *x0, void *workspace, size_t workspace_bytes,
                              hipStream_t stream)
{
    if (!sel_or_logits || !dict_idx || !diag || !b || !c || !y || !workspace)
        return PDSSM_ERR_NULL;
    int rc = check_dims(B, H, L, N, K);
    if (rc != PDSSM_OK)
        return rc;
    if (flags & ~PDSSM_FLAGS_ALL)
        return PDSSM_ERR_FLAGS;
    const void *ptrs[] = {sel_or_logits, dict_idx, diag, b, c, y, x_final, x0, workspace};
    for (const void *p : ptrs)
        if (p && !aligned16(p))
            return PDSSM_ERR_ALIGN;
    const Layout lo = layout_of(B, H, L, N, K, flags);
    if (workspace_bytes < (size_t)lo.total)
        return PDSSM_ERR_WORKSPACE;

    ScanArgs a;
    a.sel = sel_or_logits;
    a.dict = dict_idx;
    a.diag = static_cast<const float *>(diag);
    a.b = b;
    a.c = c;
    a.y = y;
    a.xfinal = static_cast<float *>(x_final);
    a.x0 = static_cast<const float *>(x0);
    a.hdr = static_cast<Header *>(workspace);
    uint32_t *tab = reinterpret_cast<uint32_t *>(static_cast<char *>(workspace) + sizeof(Header));
    a.tab = tab;
    a.agg = reinterpret_cast<uint64_t *>(reinterpret_cast<char *>(tab) + lo.tab_bytes);
    a.incl = reinterpret_cast<uint64_t *>(reinterpret_cast<char *>(a.agg) + lo.agg_bytes);
    a.H = H;
    a.L = L;
    a.S = lo.S;
    a.n_tiles = lo.n_tiles;
    a.N = N;
    a.K = K;
    a.sel_mode = flags & PDSSM_SEL_MASK;
    a.y_bf16 = (flags & PDSSM_Y_BF16) ? 1 : 0;
    a.dict_lds = ((int64_t)K * lo.NP * 4 <= kDictLdsMax) ? 1 : 0;

    const int64_t rec_bytes = lo.agg_bytes + lo.incl_bytes;
    const int64_t entries = H * (int64_t)K;
    const int64_t prep_blocks = 1 + (entries + kPrepThreads / 64 - 1) / (kPrepThreads / 64);
    hipLaunchKernelGGL(prep_kernel, dim3((unsigned)prep_blocks), dim3(kPrepThreads), 0, stream, a.hdr,
                       reinterpret_cast<uint4 *>(a.agg), (int64_t)(rec_bytes / 16), dict_idx, tab,
                       entries, N, lo.NP);
    rc = hip_status(hipGetLastError());
    if (rc != PDSSM_OK)
        return rc;
    const bool cplx = flags & PDSSM_COMPLEX, bcbf = flags & PDSSM_BC_BF16;
    hipError_t e;
    switch (lo.NP) {
    case 8: e = dispatch_scan<8>(a, cplx, bcbf, stream); break;
    case 16: e = dispatch_scan<16>(a, cplx, bcbf, stream); break;
    case 32: e = dispatch_scan<32>(a, cplx, bcbf, stream); break;
    default: e = dispatch_scan<64>(a, cplx, bcbf, stream); break;
    }
    if (e == hipSuccess)
        e = hipGetLastError();
    return hip_status(e);
}

extern "C" int pdssm_select(const void *sel_or_logits, int32_t *sel_out, int64_t B, int64_t H,
                            int64_t L, int32_t K, uint32_t flags, hipStream_t stream)
{
    if (!sel_or_logits || !sel_out)
        return PDSSM_ERR_NULL;
    int rc = check_dims(B, H, L, 1, K);
    if (rc != PDSSM_OK)
        return rc;
    if (flags & ~PDSSM_SEL_MASK)
        return PDSSM_ERR_FLAGS;
    if (!aligned16(sel_or_logits) || !aligned16(sel_out))
        return PDSSM_ERR_ALIGN;
    const int64_t steps = B * H * L;
    int64_t blocks = (steps + 255) / 256;
    if (blocks > 65536)
        blocks = 65536;
    hipLaunchKernelGGL(select_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, sel_or_logits,
                       flags & PDSSM_SEL_MASK, sel_out, steps, K);
    return hip_status(hipGetLastError());
}

extern "C" int pdssm_compose(const void *sel_or_logits, const int32_t *dict_idx, const void *diag,
                             int32_t *pi_out, void *d_out, int64_t B, int64_t H, int64_t L,
                             int32_t N, int32_t K, uint32_t flags, void *workspace,
                             size_t workspace_bytes, hipStream_t stream)
{
    if (!sel_or_logits || !dict_idx || !diag || !pi_out || !d_out || !workspace)
        return PDSSM_ERR_NULL;
    int rc = check_dims(B, H, L, N, K);
    if (rc != PDSSM_OK)
        return rc;
    if (flags & ~(PDSSM_SEL_MASK | PDSSM_COMPLEX))
        return PDSSM_ERR_FLAGS;
    const void *ptrs[] = {sel_or_logits, dict_idx, diag, pi_out, d_out, workspace};
    for (const void *p : ptrs)
        if (!aligned16(p))
            return PDSSM_ERR_ALIGN;
    const Layout lo = layout_of(B, H, L, N, K, flags);
    if (workspace_bytes < (size_t)lo.total)
        return PDSSM_ERR_WORKSPACE;
    ComposeArgs a;
    a.sel = sel_or_logits;
    a.dict = dict_idx;
    a.diag = static_cast<const float *>(diag);
    a.pi_out = pi_out;
    a.d_out = static_cast<float *>(d_out);
    char *base = static_cast<char *>(workspace) + sizeof(Header);
    a.tile_pi = reinterpret_cast<int32_t *>(base);
    a.tile_d = reinterpret_cast<float *>(base + lo.n_ctiles * lo.S * lo.NP * 4);
    a.H = H;
    a.L = L;
    a.S = lo.S;
    a.n_tiles = lo.n_ctiles;
    a.N = N;
    a.K = K;
    a.sel_mode = flags & PDSSM_SEL_MASK;
    const bool cplx = flags & PDSSM_COMPLEX;
    switch (lo.NP) {
    case 8: dispatch_compose<8>(a, cplx, stream); break;
    case 16: dispatch_compose<16>(a, cplx, stream); break;
    case 32: dispatch_compose<32>(a, cplx, stream); break;
    default: dispatch_compose<64>(a, cplx, stream); break;
    }
    return hip_status(hipGetLastError());
}

extern "C" const char *pdssm_strerror(int status)
{
    switch (status) {
    case PDSSM_OK: return "success";
    case PDSSM_ERR_NULL: return "a required pointer is NULL";
    case PDSSM_ERR_DIM: return "invalid sizes (B,H,L >= 1, N in [1,64], K in [1,32767])";
    case PDSSM_ERR_FLAGS: return "invalid flags";
    case PDSSM_ERR_ALIGN: return "a pointer is not 16-byte aligned";
    case PDSSM_ERR_WORKSPACE: return "workspace too small";
    case PDSSM_ERR_HIP: return g_err.empty() ? "HIP error" : g_err.c_str();
    default: return "unknown status";
    }
}
