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
};

// Tiling constants, shared by the host sizing code and the kernels.
constexpr int kT = 32;   // steps per chunk
constexpr int kW = 4;    // waves per workgroup

__host__ __device__ constexpr int tile_steps(int NP) { return kW * (64 / NP) * kT; }

template <int NP, bool CPLX>
__host__ __device__ constexpr int agg_words() { return NP * (1 + 2 * (CPLX ? 2 : 1)); }
template <int NP, bool CPLX>
__host__ __device__ constexpr int incl_words() { return NP * (CPLX ? 2 : 1); }

// ---------------------------------------------------------------------------
// a4: the carry of one tile, run by wave 0 with lane = state (lanes >= NP
// idle but convergent).  `agg` is the tile's inclusive operator (pi, d, e);
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
        // Look back: acc = (tiles j+1 .. tile-1) composed, latest last.
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
                    const int npi = __shfl(bpi, p);
                    cf gd;
                    gd.r = __shfl(bd.r, p);
                    gd.i = CPLX ? __shfl(bd.i, p) : 0.f;
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
// The fused scan kernel: one workgroup per tile, tiles taken in ticket order.
// ---------------------------------------------------------------------------
template <int NP, bool CPLX, bool BCBF>
__global__ void __launch_bounds__(kW * 64) scan_kernel(ScanArgs a)
{
    constexpr int G = 64 / NP, C = kW * G, T = kT, TILE = C * T, SLOTS = kW * 64;
    __shared__ uint32_t s_ticket;
    __shared__ int16_t s_sel[kW][G * T];
    __shared__ cf s_scr[kW][64];
    __shared__ int s_pi[2][SLOTS];
    __shared__ cf s_d[2][SLOTS];
    __shared__ cf s_e[2][SLOTS];
    __shared__ cf s_xin[64];

    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int g = lane / NP, i = lane % NP, chunk = wave * G + g, gbase = g * NP;

    if (tid == 0)
        s_ticket = atomicAdd(&a.hdr->ticket, 1u);
    __syncthreads();
    const int64_t ticket = s_ticket;
    const int64_t tile = ticket / a.S, seq = ticket - tile * a.S;
    const int64_t h = seq % a.H;
    const uint32_t epoch = a.hdr->epoch;
    const int64_t tile_t0 = tile * TILE;
    const int64_t seq_row = seq * a.L;

    // ---- a1: selection of this wave's G*T steps (lane = step).
    for (int q = lane; q < G * T; q += 64) {
        const int64_t t = tile_t0 + (int64_t)(wave * G) * T + q;
        int k = 0;
        if (t < a.L)
            k = select_step(a.sel, a.sel_mode, seq_row + t, a.K);
        s_sel[wave][q] = (int16_t)k;
    }
    lds_order();

    // ---- a2 + chunk-local a3: recurrence from zero and prefix operators.
    const int64_t tc0 = tile_t0 + (int64_t)chunk * T;
    const int32_t *dict_h = a.dict + h * (int64_t)a.K * a.N;
    cf *scr = s_scr[wave];
    cf x = {0.f, 0.f};
    int pacc = i;
    cf dacc = {1.f, 0.f};
    float pr[T], gr[T], gi[T];

#pragma unroll
    for (int tt = 0; tt < T; ++tt) {
        const int64_t t = tc0 + tt;
        const bool valid = (t < a.L) && (i < a.N);
        int pit = i;
        cf d = {1.f, 0.f}, bv = {0.f, 0.f}, cv = {0.f, 0.f};
        if (valid) {
            const int k = s_sel[wave][g * T + tt];
            const int64_t e = (seq_row + t) * a.N + i;
            pit = (int)min((unsigned)dict_h[(int64_t)k * a.N + i], (unsigned)(a.N - 1));
            d = load_diag<CPLX>(a.diag, e);
            bv = load_vec<CPLX, BCBF>(a.b, e);
            cv = load_vec<CPLX, BCBF>(a.c, e);
        }
        // x_t = P_t (d_t * x_{t-1}) + b_t
        x = scatter_add<CPLX>(scr, lane, gbase, pit, cmul(d, x), bv);
        pr[tt] = cv.r * x.r - cv.i * x.i;
        // Prefix operator of the chunk up to step t: source j now sits at
        // pacc[j] with factor dacc[j].
        const int src = gbase + pacc;
        const int npacc = __shfl(pit, src);
        cf dd;
        dd.r = __shfl(d.r, src);
        dd.i = CPLX ? __shfl(d.i, src) : 0.f;
        dacc = cmul(dd, dacc);
        pacc = npacc;
        // Readout coefficient of the carry-in: Re(c_t . P D X) = Re(sum_j g_t[j] X[j]).
        const int src2 = gbase + pacc;
        cf cc;
        cc.r = __shfl(cv.r, src2);
        cc.i = CPLX ? __shfl(cv.i, src2) : 0.f;
        const cf gg = cmul(cc, dacc);
        gr[tt] = gg.r;
        gi[tt] = gg.i;
    }

    // ---- a3: combine the C chunk operators of the tile (inclusive scan).
    int opi = pacc;
    cf opd = dacc, ope = x;
    s_pi[0][tid] = opi;
    s_d[0][tid] = opd;
    s_e[0][tid] = ope;
    __syncthreads();
    int buf = 0;
#pragma unroll
    for (int s = 1; s < C; s <<= 1) {
        const int nb = buf ^ 1;
        if (chunk >= s) {
            const int es = tid - s * NP;          // earlier operator, state i
            const int p1 = s_pi[buf][es];
            const cf d1 = s_d[buf][es], e1 = s_e[buf][es];
            const int ls = tid - i + p1;          // this chunk's operator at state p1
            const int npi = s_pi[buf][ls];
            const cf nd = cmul(s_d[buf][ls], d1);
            ope = scatter_add<CPLX>(s_e[nb] + (tid - lane), lane, gbase, opi, cmul(opd, e1), ope);
            opi = npi;
            opd = nd;
        } else {
            s_e[nb][tid] = ope;
        }
        s_pi[nb][tid] = opi;
        s_d[nb][tid] = opd;
        __syncthreads();
        buf = nb;
    }

    // ---- a4: carry into / out of the tile.
    if (wave == 0) {
        const int ls = (C - 1) * NP + (lane < NP ? lane : 0);
        const int api = lane < NP ? s_pi[buf][ls] : lane;
        const cf ad = lane < NP ? s_d[buf][ls] : cf{1.f, 0.f};
        const cf ae = lane < NP ? s_e[buf][ls] : cf{0.f, 0.f};
        s_xin[lane] = tile_carry<NP, CPLX>(a, tile, seq, epoch, api, ad, ae, s_scr[0]);
    }
    __syncthreads();

    // ---- a5: carry into this chunk, then the readout.
    const cf xt = s_xin[i];
    int ppi = i;
    cf pd = {1.f, 0.f}, pe = {0.f, 0.f};
    if (chunk > 0) {
        ppi = s_pi[buf][tid - NP];
        pd = s_d[buf][tid - NP];
        pe = s_e[buf][tid - NP];
    }
    const cf xc = scatter_add<CPLX>(scr, lane, gbase, ppi, cmul(pd, xt), pe);

    constexpr int R = (T + NP - 1) / NP;
    float yv[R];
#pragma unroll
    for (int r = 0; r < R; ++r)
        yv[r] = 0.f;
#pragma unroll
    for (int tt = 0; tt < T; ++tt) {
        float q = pr[tt] + gr[tt] * xc.r;
        if constexpr (CPLX)
            q -= gi[tt] * xc.i;
#pragma unroll
        for (int m = 1; m < NP; m <<= 1)
            q += __shfl_xor(q, m);
        if (i == tt % NP)
            yv[tt / NP] = q;
    }
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const int tt = r * NP + i;
        const int64_t t = tc0 + tt;
        if (tt < T && t < a.L) {
            if (a.y_bf16)
                reinterpret_cast<uint16_t *>(a.y)[seq_row + t] = f32_to_bf16_rne(yv[r]);
            else
                reinterpret_cast<float *>(a.y)[seq_row + t] = yv[r];
        }
    }
}

// ---------------------------------------------------------------------------
// Workspace preparation: new epoch, ticket reset; on first use (or after the
// epoch wraps) clear every carry record.  One workgroup.
// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(1024) prep_kernel(Header *hdr, uint4 *recs, int64_t n16)
{
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

template <int NP, bool CPLX>
__global__ void __launch_bounds__(kW * 64) compose_tiles_kernel(ComposeArgs a)
{
    constexpr int G = 64 / NP, C = kW * G, T = kT, TILE = C * T, SLOTS = kW * 64;
    constexpr int NC = CPLX ? 2 : 1;
    __shared__ int16_t s_sel[kW][G * T];
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
    const int64_t n_tiles = (L + tile_steps(pad_states(N)) - 1) / tile_steps(pad_states(N));
    if ((double)B * (double)H * (double)n_tiles > 2.0e9)
        return PDSSM_ERR_DIM;
    return PDSSM_OK;
}

struct Layout {
    int NP;
    int64_t n_tiles, S, agg_bytes, incl_bytes, compose_bytes, total;
};

static Layout layout_of(int64_t B, int64_t H, int64_t L, int32_t N, uint32_t flags)
{
    Layout lo;
    lo.NP = pad_states(N);
    const int nc = (flags & PDSSM_COMPLEX) ? 2 : 1;
    const int64_t tile = tile_steps(lo.NP);
    lo.n_tiles = (L + tile - 1) / tile;
    lo.S = B * H;
    const int64_t recs = lo.n_tiles * lo.S;
    lo.agg_bytes = recs * lo.NP * (1 + 2 * nc) * 8;
    lo.incl_bytes = recs * lo.NP * nc * 8;
    lo.compose_bytes = recs * lo.NP * (1 + nc) * 4;
    const int64_t scan = lo.agg_bytes + lo.incl_bytes;
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
static void launch_scan(const ScanArgs &a, hipStream_t st)
{
    hipLaunchKernelGGL((scan_kernel<NP, CPLX, BCBF>), dim3((unsigned)(a.n_tiles * a.S)),
                       dim3(kW * 64), 0, st, a);
}

template <int NP>
static void dispatch_scan(const ScanArgs &a, bool cplx, bool bcbf, hipStream_t st)
{
    if (cplx) {
        if (bcbf) launch_scan<NP, true, true>(a, st);
        else launch_scan<NP, true, false>(a, st);
    } else {
        if (bcbf) launch_scan<NP, false, true>(a, st);
        else launch_scan<NP, false, false>(a, st);
    }
}

template <int NP>
static void dispatch_compose(const ComposeArgs &a, bool cplx, hipStream_t st)
{
    const dim3 tiles((unsigned)(a.n_tiles * a.S)), seqs((unsigned)a.S);
    if (cplx) {
        hipLaunchKernelGGL((compose_tiles_kernel<NP, true>), tiles, dim3(kW * 64), 0, st, a);
        hipLaunchKernelGGL((compose_final_kernel<NP, true>), seqs, dim3(64), 0, st, a);
    } else {
        hipLaunchKernelGGL((compose_tiles_kernel<NP, false>), tiles, dim3(kW * 64), 0, st, a);
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
    return (size_t)layout_of(B, H, L, N, flags).total;
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
    const Layout lo = layout_of(B, H, L, N, flags);
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
    a.agg = reinterpret_cast<uint64_t *>(static_cast<char *>(workspace) + sizeof(Header));
    a.incl = reinterpret_cast<uint64_t *>(reinterpret_cast<char *>(a.agg) + lo.agg_bytes);
    a.H = H;
    a.L = L;
    a.S = lo.S;
    a.n_tiles = lo.n_tiles;
    a.N = N;
    a.K = K;
    a.sel_mode = flags & PDSSM_SEL_MASK;
    a.y_bf16 = (flags & PDSSM_Y_BF16) ? 1 : 0;

    const int64_t rec_bytes = lo.agg_bytes + lo.incl_bytes;
    hipLaunchKernelGGL(prep_kernel, dim3(1), dim3(1024), 0, stream, a.hdr,
                       reinterpret_cast<uint4 *>(a.agg), (int64_t)(rec_bytes / 16));
    rc = hip_status(hipGetLastError());
    if (rc != PDSSM_OK)
        return rc;
    const bool cplx = flags & PDSSM_COMPLEX, bcbf = flags & PDSSM_BC_BF16;
    switch (lo.NP) {
    case 8: dispatch_scan<8>(a, cplx, bcbf, stream); break;
    case 16: dispatch_scan<16>(a, cplx, bcbf, stream); break;
    case 32: dispatch_scan<32>(a, cplx, bcbf, stream); break;
    default: dispatch_scan<64>(a, cplx, bcbf, stream); break;
    }
    return hip_status(hipGetLastError());
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
    const Layout lo = layout_of(B, H, L, N, flags);
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
    a.tile_d = reinterpret_cast<float *>(base + lo.n_tiles * lo.S * lo.NP * 4);
    a.H = H;
    a.L = L;
    a.S = lo.S;
    a.n_tiles = lo.n_tiles;
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
