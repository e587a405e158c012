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
//                      a multiply; the chunk waves of a tile chain their
//                      operators into inclusive prefixes, in time order,
//                      through LDS.
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
#include <mutex>
#include <string>
#include <type_traits>

#include "pdssm.h"
#include "pdssm_device.h"
#include "pdssm_host.h"

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
    uint32_t total;   // tiles in the call: n_tiles * S
    // Per-head tickets (null: one shared stream): workgroup w serves head
    // w % H and takes its tiles from ctr[32 * h], total_head = n_tiles * B.
    uint32_t *ctr;
    uint32_t total_head;
    // Optional: the state before each chunk of kScanT steps, [S][nch][N(,2)],
    // and every step's selected entry, [S][L].
    float *xsave;
    int16_t *selsave;
    int64_t nch;
    int N, K;
    uint32_t sel_mode;
    int y_bf16;
    int strict;     // the carry only from the tile just before (no aggregate records)
    int dict_lds;   // the head's entry table fits in LDS
    const uint16_t *tab;   // [H][K][NP]: dict_entry() of every source (see prep_kernel)
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
#define PDSSM_SCAN_D 4
#endif
constexpr int kScanT = PDSSM_SCAN_T;
constexpr int kScanW = PDSSM_SCAN_W;
constexpr int kScanD = PDSSM_SCAN_D;   // steps of inputs in flight per lane (register ring)
static_assert(kScanW >= 1 && kScanW <= 32, "chunk waves post into a 32-bit mask");
static_assert(kScanT == kCarryStride, "the saved carries are one per chunk of the backward scan");
constexpr int kDictLdsMax = 32768;   // bytes of the head's entry table kept in LDS
// The carry wave's nap between polls (s_sleep units of 64 clocks): it shares
// its SIMD with chunk waves, so it should not spin.
#ifndef PDSSM_CARRY_NAP
#define PDSSM_CARRY_NAP 4
#endif
#ifndef PDSSM_CARRY_PRIO
#define PDSSM_CARRY_PRIO 2   // s_setprio level of the carry wave and of the chunk waves' chain
#endif
// The chunk waves' s_setprio level during their local pass (0 in the other
// phases): the waves of a CU's workgroups are in different phases at any
// time, and those in the local pass, which saturates the LDS, go first.
#ifndef PDSSM_LOCAL_PRIO
#define PDSSM_LOCAL_PRIO 1
#endif

__host__ __device__ constexpr int scan_tile_steps(int NP) { return kScanW * (64 / NP) * kScanT; }

// Which chunk wave runs the tile's p-th group of chunks.  The carry wave
// chains the groups in time order as their waves finish, so the order
// follows the order in which the waves of a workgroup tend to finish their
// local pass (measured for seven chunk waves: the waves sharing a SIMD with
// an older wave of the workgroup finish last).  Any order is correct.
__host__ __device__ constexpr int wave_at(int p)
{
    constexpr int order7[7] = {1, 2, 3, 0, 5, 6, 4};
    return (kScanW == 7) ? order7[p] : p;
}
__host__ __device__ constexpr int chunk_pos(int w)
{
    constexpr int pos7[7] = {3, 0, 1, 2, 6, 4, 5};
    return (kScanW == 7) ? pos7[w] : w;
}
constexpr bool chunk_order_ok()
{
    for (int p = 0; p < kScanW; ++p)
        if (wave_at(p) < 0 || wave_at(p) >= kScanW || chunk_pos(wave_at(p)) != p)
            return false;
    return true;
}
static_assert(chunk_order_ok(), "wave_at and chunk_pos must be inverse permutations");

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
__device__ __forceinline__ typename RawVec<CPLX, BCBF>::type bperm_raw_a(typename RawVec<CPLX, BCBF>::type v, int addr)
{
    if constexpr (BCBF)
        return bperm_a((uint32_t)v, addr);
    else if constexpr (CPLX)
        return make_float2(bperm_a(v.x, addr), bperm_a(v.y, addr));
    else
        return bperm_a(v, addr);
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
// a4: the carry between tiles, run by the carry wave with lane = state
// (lanes >= NP idle but convergent).  Tile records (decoupled look-back,
// Merrill & Garland's single-pass scan): AGG = the tile's operator (pi, d,
// e), INCL = the state after the tile.
//
// LookBack gathers the carry into a tile: (bpi, bd, be) = tiles j+1 ..
// tile-1 composed (latest last); it ends at the first INCL found.  One
// attempt reads tile j's INCL and AGG records whole, in one round trip (two
// and five words per lane), and takes the INCL if every word of it is from
// this call, else the AGG if every word of that is; otherwise it tries the
// same tile again.  The carry wave issues no store while an attempt is in
// flight: on this GPU one counter tracks loads and stores alike, so waiting
// for the attempt's loads would also wait for the stores to complete.
// ---------------------------------------------------------------------------
template <int NP, bool CPLX>
struct LookBack {
    static constexpr int NC = CPLX ? 2 : 1;
    static constexpr int AW = agg_words<NP, CPLX>(), IW = incl_words<NP, CPLX>();
    int64_t j = 0, seq = 0;
    int bpi = 0;
    cf bd = {1.f, 0.f}, be = {0.f, 0.f}, xin = {0.f, 0.f};
    bool done = false;

    __device__ void start(const ScanArgs &a, int64_t tile, int64_t sq, int lane)
    {
        seq = sq;
        bpi = lane;
        bd = {1.f, 0.f};
        be = {0.f, 0.f};
        xin = {0.f, 0.f};
        j = tile - 1;
        done = tile == 0;
        if (done && a.x0 && lane < a.N)
            xin = load_diag<CPLX>(a.x0, sq * a.N + lane);
    }

    __device__ static uint64_t load(const uint64_t *p)
    {
        return __hip_atomic_load(const_cast<uint64_t *>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    __device__ static bool from(uint64_t word, uint32_t epoch) { return (uint32_t)(word >> 32) == epoch; }
    __device__ static float val(uint64_t word) { return __uint_as_float((uint32_t)word); }

    // One attempt; true when it made progress (found the INCL or took an AGG).
    __device__ bool attempt(const ScanArgs &a, uint32_t epoch, int lane, cf *scr)
    {
        if (done)
            return false;
        const bool act = lane < NP;
        const bool has_agg = j > 0 && !a.strict;   // tile 0 publishes no AGG (it knows its carry)
        const int64_t rj = j * a.S + seq;
        const uint64_t *iw = a.incl + rj * IW;
        const uint64_t *aw = a.agg + rj * AW;
        // Words of other calls never match the epoch, so lanes that load
        // nothing start from a word that cannot pass for a loaded one.
        uint64_t i0 = 0, i1 = 0, a0 = 0, a1 = 0, a2 = 0, a3 = 0, a4 = 0;
        if (act) {
            i0 = load(iw + lane * NC);
            if constexpr (CPLX)
                i1 = load(iw + lane * NC + 1);
            if (has_agg) {
                a0 = load(aw + lane);
                a1 = load(aw + NP + lane * NC);
                a2 = load(aw + NP + NP * NC + lane * NC);
                if constexpr (CPLX) {
                    a3 = load(aw + NP + lane * NC + 1);
                    a4 = load(aw + NP + NP * NC + lane * NC + 1);
                }
            }
        }
        const bool iok = !act || (from(i0, epoch) && (!CPLX || from(i1, epoch)));
        if (__all(iok)) {
            const cf X = {act ? val(i0) : 0.f, (CPLX && act) ? val(i1) : 0.f};
            xin = scatter_add<CPLX>(scr, lane, 0, bpi, cmul(bd, X), be);
            done = true;
            return true;
        }
        const bool aok = !act || (from(a0, epoch) && from(a1, epoch) && from(a2, epoch) &&
                                  (!CPLX || (from(a3, epoch) && from(a4, epoch))));
        // With PDSSM_DETERMINISTIC only the INCL of the tile just before is
        // taken, so the carry is formed the same way on every call.
        if (has_agg && __all(aok)) {
            int p = lane;
            cf d = {1.f, 0.f}, e = {0.f, 0.f};
            if (act) {
                p = (int)min((uint32_t)a0, (uint32_t)(NP - 1));
                d = {val(a1), CPLX ? val(a3) : 0.f};
                e = {val(a2), CPLX ? val(a4) : 0.f};
            }
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
            return true;
        }
        return false;
    }
};

// Publish a tile's AGG record (tile > 0 only; tile 0 knows its carry); `i`
// is the state the calling lane holds, and only lanes with `act` store.
template <int NP, bool CPLX>
__device__ void publish_agg(const ScanArgs &a, int64_t tile, int64_t seq, uint32_t epoch, int lane, bool act,
                            int api, cf ad, cf ae)
{
    constexpr int NC = CPLX ? 2 : 1;
    uint64_t *aw = a.agg + (tile * a.S + seq) * agg_words<NP, CPLX>();
    if (act) {
        put_word(aw + lane, (uint32_t)api, epoch);
        put_word(aw + NP + lane * NC, __float_as_uint(ad.r), epoch);
        put_word(aw + NP + NP * NC + lane * NC, __float_as_uint(ae.r), epoch);
        if constexpr (CPLX) {
            put_word(aw + NP + lane * NC + 1, __float_as_uint(ad.i), epoch);
            put_word(aw + NP + NP * NC + lane * NC + 1, __float_as_uint(ae.i), epoch);
        }
    }
}

// The state after the tile from its carry-in: publish INCL, and x_final
// after the last tile.
template <int NP, bool CPLX>
__device__ void publish_incl(const ScanArgs &a, int64_t tile, int64_t seq, uint32_t epoch, int lane, int api,
                             cf ad, cf ae, cf xin, cf *scr)
{
    constexpr int NC = CPLX ? 2 : 1;
    const cf xout = scatter_add<CPLX>(scr, lane, 0, api, cmul(ad, xin), ae);
    if (lane < NP) {
        uint64_t *iw = a.incl + (tile * a.S + seq) * incl_words<NP, CPLX>();
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
}

// ---------------------------------------------------------------------------
// The fused scan kernel.  Persistent workgroups take tiles from an atomic
// ticket in tile-major order (u = tile * S + seq, or, with one ticket stream
// per head, u = tile * B + b) and run them one after another.  A workgroup
// holds at most two tickets, its current tile and the next one, and starts
// the next only once the current tile's carry is out.  So the smallest
// unfinished ticket of a stream always belongs to a current tile, whose
// look-back waits only on smaller tickets of the same stream -- all
// finished: no deadlock.
//
// Waves 0..W-1 ("chunk waves") each own G chunks of T steps of the tile.
// Wave W (the "carry wave") takes the tickets, stages the dictionary table
// and runs the look-back while the chunk waves are busy (the carry into a
// tile depends only on earlier tiles).  Per tile:
//
//   chunk waves:  local pass, chain prefixes      (B) next tile's scores     (C) prefixes (D) readout, next inputs, selection
//   carry wave:   next ticket, look-back          (B) next table, carry,
//                                                     publish                (C)          (D) previous y
//
// so the next tile's router scores and first input steps are in flight
// while the carry of the current one is worked out.  The two roles run on
// separate wave-uniform paths that meet only at barriers.
// ---------------------------------------------------------------------------
// Waves per SIMD the scan kernel is compiled for: six (three 8-wave
// workgroups per CU) where the register allocator fits that without
// spilling, else no constraint.
template <int NP, bool CPLX, bool BCBF>
constexpr int scan_waves_per_eu()
{
#ifdef PDSSM_SCAN_WAVES_PER_EU
    return (!CPLX || (BCBF && NP == 64)) ? PDSSM_SCAN_WAVES_PER_EU : 1;
#else
    return (!CPLX || (BCBF && NP == 64)) ? 6 : 1;
#endif
}

template <int NP, bool CPLX, bool BCBF>
__global__ void __launch_bounds__((kScanW + 1) * 64)
__attribute__((amdgpu_waves_per_eu(scan_waves_per_eu<NP, CPLX, BCBF>()))) scan_kernel(ScanArgs a)
{
    constexpr int W = kScanW, T = kScanT, G = 64 / NP, C = W * G, TILE = C * T, SLOTS = W * 64;
    constexpr int NV = (G == 1) ? 2 : 4;   // 16-byte score vectors per lane in the fast selection
    using Raw = typename RawVec<CPLX, BCBF>::type;
    using DRaw = typename std::conditional<CPLX, float2, float>::type;
    using Stored = typename std::conditional<BCBF, typename std::conditional<CPLX, uint32_t, uint16_t>::type, Raw>::type;
    // Entry table: the head's [K][NP] 16-bit entries when they fit, else the
    // tile's entries, one row of NP 16-bit entries per (wave, step).
    extern __shared__ __attribute__((aligned(16))) uint32_t s_tab[];
    __shared__ int16_t s_sel[W][G * T];
    // Scatter regions, zero blocks, spare region and trash block per chunk
    // wave.  The trash block only takes stores during the wave's local pass;
    // between local passes it holds the d part of the wave's chunk operators
    // (slot wave * 64 + lane), which is written after the local pass and last
    // read before (D).
    __shared__ __attribute__((aligned(16))) cf s_reg[W][kBlocks][64];
    __shared__ cf s_cscr[64];   // the carry wave's scatter scratch
    __shared__ int s_pi[SLOTS];   // chunk operators, then their inclusive prefixes
    auto s_d = [&](int slot) -> cf & { return s_reg[slot >> 6][kBlocks - 1][slot & 63]; };
    __shared__ cf s_e[SLOTS];
    __shared__ cf s_xin[64];
    __shared__ float s_y[2][TILE];   // finished tiles' outputs by iteration parity, stored by the carry wave
    __shared__ float s_q[TILE];   // per step: sum_j Re(c_t[j] x_loc_t[j]), until the correction
    __shared__ uint32_t s_next;   // ticket published by the carry wave
    __shared__ uint32_t s_ready;  // bit w: chunk wave w has posted its inclusive prefixes
    __shared__ uint32_t s_known;  // 1 + index (in this workgroup) of the last tile whose carry is known

    // Tile indices, sequences and heads fit 32 bits (the host checks).
    const uint32_t S32 = (uint32_t)a.S, H32 = (uint32_t)a.H;
    // Ticket u -> (tile, sequence): tile-major over all sequences, or, with
    // per-head tickets, over the sequences b * H + hp of this workgroup's head.
    // PDSSM_TEST_TICKET_REMAP (a test build) reverses the order in which
    // the sequences of a tile row are handed out and the heads workgroups
    // serve; every tile still follows the tiles before it in its sequence.
    const bool pinned = a.ctr != nullptr;
    const uint32_t per = pinned ? S32 / H32 : S32;
    const uint32_t total = pinned ? a.total_head : a.total;
#ifdef PDSSM_TEST_TICKET_REMAP
    const uint32_t hp = pinned ? H32 - 1u - (uint32_t)blockIdx.x % H32 : 0u;
    auto decode = [&](uint32_t u, uint32_t &tile, uint32_t &seq) {
        tile = __builtin_amdgcn_readfirstlane(u / per);
        const uint32_t r = per - 1u - (u - tile * per);
        seq = pinned ? r * H32 + hp : r;
    };
#else
    const uint32_t hp = pinned ? (uint32_t)blockIdx.x % H32 : 0u;
    auto decode = [&](uint32_t u, uint32_t &tile, uint32_t &seq) {
        tile = __builtin_amdgcn_readfirstlane(u / per);
        const uint32_t r = u - tile * per;
        seq = pinned ? r * H32 + hp : r;
    };
#endif
    const int N = a.N, K = a.K;
    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;

    if (wave == W) {
        // ================= carry wave =================
        // Its work is on every tile's critical path: issue it first.
        __builtin_amdgcn_s_setprio(PDSSM_CARRY_PRIO);
        auto take_ticket = [&]() -> uint32_t {
            uint32_t t = 0;
            if (lane == 0)
                t = atomicAdd(pinned ? a.ctr + 32 * hp : &a.hdr->ticket, 1u);
            return __builtin_amdgcn_readfirstlane(t);
        };
        // The head's entry table straight to LDS (16 bytes per lane per
        // instruction, no registers involved); waited for before (C).
        auto stage_table = [&](uint32_t u) {
            if (!a.dict_lds)
                return;
            uint32_t tile, seq;
            decode(u, tile, seq);
            const uint32_t h = __builtin_amdgcn_readfirstlane(seq % H32);
            const uint4 *src = reinterpret_cast<const uint4 *>(a.tab + h * (int64_t)K * NP);
            const int tab_vecs = (K * NP) >> 3;   // 8 entries per 16 bytes
            for (int w0 = 0; w0 < tab_vecs; w0 += 64) {
                const int w = min(w0 + lane, tab_vecs - 1);
                __builtin_amdgcn_global_load_lds(
                    src + w, (__attribute__((address_space(3))) void *)(reinterpret_cast<uint8_t *>(s_tab) + w0 * 16),
                    16, 0, 0);
            }
        };
        uint32_t cur = take_ticket();
        if (lane == 0) {
            s_next = cur;
            s_ready = 0;
            s_known = 0;
        }
        const uint32_t epoch = a.hdr->epoch;
        __syncthreads();   // (P) first ticket published
        if (cur >= total)
            return;
        stage_table(cur);
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();   // (Q) first table and selections ready

        // Store output v of the previous tile, which chunk wave w staged in
        // s_y (step j * 64 + lane of the wave's chunks: a wave holds G * T
        // steps, 16 to 128, so up to two per lane).
        constexpr int YR = (G * T + 63) / 64;
        int64_t py0 = 0, pt0 = 0;   // the previous tile: y index and step of its first output
        auto store_y = [&](int w, int j, float v) {
            const int k = chunk_pos(w) * G * T + j * 64 + lane;   // step within the tile
            if (j * 64 + lane < G * T && pt0 + k < a.L) {
                if (a.y_bf16)
                    reinterpret_cast<uint16_t *>(a.y)[py0 + k] = f32_to_bf16_rne(v);
                else
                    reinterpret_cast<float *>(a.y)[py0 + k] = v;
            }
        };
        const bool act = lane < NP;
        cf *scr = s_cscr;
        bool have_prev = false;
        LookBack<NP, CPLX> lb;
        for (uint32_t iter = 1;; ++iter) {
            // The next ticket; its value is needed only at (B).
            uint32_t tk = 0;
            if (lane == 0)
                tk = atomicAdd(pinned ? a.ctr + 32 * hp : &a.hdr->ticket, 1u);
            uint32_t tile, seq;
            decode(cur, tile, seq);
            lb.start(a, tile, seq, lane);

            // ---- a4 while the chunk waves run their local pass and chain
            // their prefixes: look back for the carry into this tile, which
            // depends only on earlier tiles, until every chunk wave has
            // posted (then the aggregate is known).  Once the carry is known
            // the tile needs no AGG record: the last chunk wave of the chain
            // publishes one only while s_known is behind.
            while (!lb.done) {
                const uint32_t posted = __builtin_amdgcn_readfirstlane(*reinterpret_cast<volatile uint32_t *>(&s_ready));
                if (posted == (1u << W) - 1u)
                    break;
                if (!lb.attempt(a, epoch, lane, scr))
                    __builtin_amdgcn_s_sleep(PDSSM_CARRY_NAP);
            }
            if (lb.done && lane == 0)
                *reinterpret_cast<volatile uint32_t *>(&s_known) = iter;
            const uint32_t nxt = __builtin_amdgcn_readfirstlane(tk);
            if (lane == 0)
                s_next = nxt;
            __syncthreads();   // (B) all chunk operators taken, next ticket published
            if (lane == 0)
                s_ready = 0;
            const bool more = nxt < total;
            // The tile's aggregate: the inclusive prefix of its last chunk,
            // read before the table copy starts (the compiler would make LDS
            // reads wait for it).
            int ppi = lane;
            cf pd = {1.f, 0.f}, pe = {0.f, 0.f};
            if (act) {
                const int as = wave_at(W - 1) * 64 + (G - 1) * NP + lane;
                ppi = s_pi[as];
                pd = s_d(as);
                pe = s_e[as];
            }
            // Every chunk wave is past its local pass, the only reader of the
            // entry table: stage the next tile's (a workgroup serving one
            // head keeps its table).
            if (more && !pinned)
                stage_table(nxt);
            // ---- a4, second part: the carry if it is still unknown (the
            // tile's AGG record is out), then the state after the tile.
            while (!lb.done)
                if (!lb.attempt(a, epoch, lane, scr))
                    __builtin_amdgcn_s_sleep(PDSSM_CARRY_NAP);
            // The next table has landed (it was staged before (B)), then the
            // state after the tile goes out at once: the next tile of the
            // sequence may be waiting for it.
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
            publish_incl<NP, CPLX>(a, tile, seq, epoch, lane, ppi, pd, pe, lb.xin, scr);
            s_xin[lane] = lb.xin;
            __syncthreads();   // (C) carry ready, next table staged
            __syncthreads();   // (D) chunk waves have read the prefixes and the carry
            // While the chunk waves run the readout: the previous tile's
            // outputs, from the other s_y buffer (the chunk waves rewrite it
            // only in the next iteration, after the next (D)); the stores
            // need not complete here.
            if (have_prev)
                for (int w = 0; w < W; ++w)
#pragma unroll
                    for (int j = 0; j < YR; ++j)
                        if (j * 64 + lane < G * T)
                            store_y(w, j, s_y[(iter - 1) & 1][w * G * T + j * 64 + lane]);
            if (!more)
                return;
            pt0 = (int64_t)tile * TILE;
            py0 = (int64_t)seq * a.L + pt0;
            have_prev = true;
            cur = nxt;
        }
    }

    // ================= chunk waves =================
    // Lane roles: group g of NP lanes runs chunk chunk_pos(wave) * G + g of
    // the tile (its operator slot is wave * 64 + g * NP); lane i of the
    // group holds state i.  Every phase below derives them from its own
    // opaque copy of the lane index, so that per-lane constants are made
    // where they are used instead of being held across the whole loop.
    struct Lanes {
        int ln, g, i, gbase, icl;
        bool row_ok;   // padding rows (i >= N) hold no state
    };
    auto lanes = [&]() {
        Lanes q;
        q.ln = opaque(lane);
        q.g = (G == 1) ? 0 : q.ln / NP;
        q.i = (G == 1) ? q.ln : q.ln % NP;
        q.gbase = q.g * NP;
        q.icl = min(q.i, N - 1);
        q.row_ok = q.i < N;
        return q;
    };
    const bool sel_fast = select_fast_ok(a.sel_mode, K, lanes_per_step<G * T>(), G * T, NV);
    constexpr int D = kScanD < T ? kScanD : T;

    // ---- Streaming state of the tile whose loads are in flight: the
    // router-score slice of the wave's steps (the selection needs it first)
    // and the chunk's step inputs, streamed through a ring of D register
    // slots: the first D steps at issue, step t + D once step t is used.
    // Buffer resources start at the wave's first row.  Rows past the end of
    // the sequence are clamped to the last one, so every load is in range;
    // with one chunk per wave the row offset is wave-uniform (scalar), and in
    // a whole wave a lane's offset is fixed while the row offset steps.
    ScoreSlice<NV> sc;
    __amdgpu_buffer_rsrc_t rsd, rsb, rsc;
    const int L = (int)a.L;   // steps fit 31 bits (the host checks)
    int64_t row0 = 0;         // index of the sequence's first step
    uint32_t cseq = 0;        // the sequence
    uint32_t ctile = 0;       // the tile
    int tw0 = 0, wrow = 0;    // the wave's first step; the first buffer row
    bool full = false;        // every chunk of the wave lies inside the sequence
    uint32_t h = 0;
    DRaw dv[D];
    Raw bv[D], cv[D];
    auto fetch = [&](const Lanes &q, int tt) {
        uint32_t el, row_el;
        if (G == 1 || full) {
            el = (uint32_t)(q.g * T * N + q.icl);
            row_el = (uint32_t)((min(tw0 + tt, L - 1) - wrow) * N);   // == tt * N in a whole wave
        } else {
            el = (uint32_t)((min(tw0 + q.g * T + tt, L - 1) - wrow) * N + q.icl);
            row_el = 0;
        }
        dv[tt % D] = bload<DRaw>(rsd, el * (uint32_t)sizeof(DRaw), row_el * (uint32_t)sizeof(DRaw));
        bv[tt % D] = (Raw)bload<Stored>(rsb, el * (uint32_t)sizeof(Stored), row_el * (uint32_t)sizeof(Stored));
        cv[tt % D] = (Raw)bload<Stored>(rsc, el * (uint32_t)sizeof(Stored), row_el * (uint32_t)sizeof(Stored));
    };
    // Two parts: the router scores (and the tile's geometry), then the
    // first D input steps.
    auto issue_scores = [&](uint32_t u) {
        const Lanes q = lanes();
        uint32_t tile, seq;
        decode(u, tile, seq);
        h = __builtin_amdgcn_readfirstlane(seq % H32);
        cseq = seq;
        ctile = tile;
        row0 = (int64_t)seq * a.L;
        tw0 = (int)tile * TILE + chunk_pos(wave) * G * T;
        full = tw0 + G * T <= L;
        // Assigned on every path, so no older value is kept around the loop.
        sc = sel_fast ? select_issue<G * T, NV>(a.sel, opaque_s(a.sel_mode), opaque_s(K), a.L, row0, tw0, q.ln)
                      : ScoreSlice<NV>{};
    };
    auto issue_inputs = [&]() {
        const Lanes q = lanes();
        wrow = min(tw0, L - 1);
        const uint64_t rem = (uint64_t)(L - wrow) * (uint64_t)N;   // elements to the end of the sequence
        const int64_t e0 = (row0 + wrow) * N;
        rsd = make_rsrc(reinterpret_cast<const DRaw *>(a.diag) + e0, rem * sizeof(DRaw));
        rsb = make_rsrc(reinterpret_cast<const Stored *>(a.b) + e0, rem * sizeof(Stored));
        rsc = make_rsrc(reinterpret_cast<const Stored *>(a.c) + e0, rem * sizeof(Stored));
#pragma unroll
        for (int tt = 0; tt < D; ++tt)
            fetch(q, tt);
    };
    // ---- a1: selection of the wave's G*T consecutive steps of the tile
    // whose loads are in flight (and, when the head's entry table does not
    // fit in LDS, the wave's entries straight from the table in memory).
    auto select = [&]() {
        const Lanes q = lanes();
        const int Kq = opaque_s(K);
        const uint32_t mode = opaque_s(a.sel_mode);
        if (sel_fast)
            select_finish<G * T, NV>(sc, mode, Kq, a.L, tw0, s_sel[wave], q.ln);
        else
            wave_select<G * T>(a.sel, mode, Kq, a.L, row0, tw0, s_sel[wave], q.ln);
        if (!a.dict_lds) {
            // The entries of the wave's steps, one NP-wide row per step.
            lds_order();
            const uint16_t *tab_h = a.tab + h * (int64_t)K * NP;
            uint16_t *tb = reinterpret_cast<uint16_t *>(s_tab) + (wave * G * T + q.g * T) * NP + q.i;
            for (int tt = 0; tt < T; ++tt) {
                const int k = s_sel[wave][q.g * T + tt];
                tb[tt * NP] = tab_h[k * NP + q.i];
            }
        }
        lds_order();
        if (a.selsave) {
            for (int st = q.ln; st < G * T; st += 64)
                if (tw0 + st < a.L)
                    a.selsave[row0 + tw0 + st] = s_sel[wave][st];
        }
    };

    // The zero blocks of this wave's scatter area (never written again).
#pragma unroll
    for (int r = kRegions; r < 2 * kRegions; ++r)
        s_reg[wave][r][lane] = cf{0.f, 0.f};
    __syncthreads();   // (P) first ticket published
    uint32_t cur = __builtin_amdgcn_readfirstlane(s_next);
    if (cur >= total)
        return;
    const uint32_t epoch = __builtin_amdgcn_readfirstlane(a.hdr->epoch);
    issue_scores(cur);
    issue_inputs();
    select();
    __syncthreads();   // (Q) first table and selections ready

    for (uint32_t iter = 1;; ++iter) {
        const Lanes q = lanes();
        // ---- a2 + chunk-local a3: recurrence from zero state, and the
        // prefix operator of the chunk: source j of the chunk start sits at
        // lane pa4 / 4 (a byte address, as ds_bpermute takes it) with factor
        // dacc[j].  Steps past the end of the sequence are skipped (the
        // identity).  Padding rows only ever exchange values among
        // themselves; they are kept out of the two sums over rows (the
        // readout and its correction).
        // (issue() moves tw0 and row0 on to the next tile before the readout.)
        const int cw0 = tw0;                // the wave's first step
        const int tc0 = cw0 + q.g * T;      // first step of the chunk
        const int64_t y0 = row0 + cw0;      // y index of the wave's first step
        const uint32_t seq0 = cseq, tile0 = ctile;
        const int nvalid = max(0, min(T, L - tc0));
        // The same bound, re-derived where it is tested again, so that the
        // compiler does not keep one test's outcome alive across blocks.
        auto nvalid_again = [&]() {
            if constexpr (G == 1)
                return opaque_s(__builtin_amdgcn_readfirstlane(nvalid));   // wave-uniform: one chunk per wave
            else
                return opaque(nvalid);
        };
        char *const regp = reinterpret_cast<char *>(&s_reg[wave][0][0]) + q.gbase * (int)sizeof(cf);
        // The entries of this lane: column i of the head's table, or its own
        // word per step of the wave's entries (both as byte addresses).
        // Both are rows of NP 16-bit entries: the head's table, row = the
        // step's selection, or the wave's staged entries, row = the step.
        const char *const tbp = reinterpret_cast<const char *>(s_tab) +
                                (a.dict_lds ? q.i * 2 : ((wave * G * T + q.g * T) * NP + q.i) * 2);
        const char *const rowbase = regp + q.i * (int)sizeof(cf);   // row i of block 0
        cf x = {0.f, 0.f};
        int pa4 = q.ln * 4;
        cf dacc = {1.f, 0.f};
        float qg[4], w[T / 4], gr[T], gi[T];
        Raw craw_prev = zero_raw<CPLX, BCBF>();
        // With one chunk per wave the step's selection is wave-uniform: keep
        // the chunk's selections in one register and broadcast them per step.
        int selv = 0;
        if constexpr (G == 1)
            selv = a.dict_lds ? (int)s_sel[wave][q.ln % T] : q.ln % T;
        auto entry = [&](int tt) -> uint32_t {
            if constexpr (G == 1)
                return *reinterpret_cast<const uint16_t *>(tbp + __builtin_amdgcn_readlane(selv, tt) * NP * 2);
            if (a.dict_lds)
                return *reinterpret_cast<const uint16_t *>(tbp + (int)s_sel[wave][q.g * T + tt] * NP * 2);
            return *reinterpret_cast<const uint16_t *>(tbp + tt * NP * 2);
        };
        uint32_t ent_next = entry(0);
        __builtin_amdgcn_s_setprio(PDSSM_LOCAL_PRIO);
#pragma unroll
        for (int tt = 0; tt < T; ++tt) {
            const uint32_t ent = ent_next;
            const int sl = tt % D;
            cf d;
            if constexpr (CPLX)
                d = {dv[sl].x, dv[sl].y};
            else
                d = {dv[sl], 0.f};
            const cf b = unpack_raw<CPLX, BCBF>(bv[sl]);
            const Raw craw = cv[sl];
            const cf c = unpack_raw<CPLX, BCBF>(craw);
            // The gathers at pacc before step t (byte address pa4): c_{t-1}
            // for the readout weight of step t-1, and pi_t, d_t to extend
            // the prefix operator.  They do not depend on x, so they are
            // issued first and their LDS round trip overlaps the scatter's.
            Raw cgat = zero_raw<CPLX, BCBF>();
            if (tt > 0)
                cgat = bperm_raw_a<CPLX, BCBF>(craw_prev, pa4);
            uint32_t pe;   // set, and used, only on steps inside the sequence
            cf dd;
            if (tt < nvalid) {
                pe = bperm_a(ent, pa4);
                dd.r = bperm_a(d.r, pa4);
                dd.i = CPLX ? bperm_a(d.i, pa4) : 0.f;
            }
            cf uu[kRegions];
            if (tt < nvalid_again()) {
                // x_t = P_t (d_t * x_{t-1}) + b_t.  Source j stores into the
                // slot its entry names: region rank(j) at row pi(j), so within
                // a region every row has at most one source and plain stores
                // suffice (rank kRegions: the spare region).  Sources of
                // higher rank (rare) store into the trash block and then add
                // atomically into the spare slot of their row.  Row i reads
                // kRegions blocks from the offset its entry names: the
                // in-degree(i) regions written in this step, then zero
                // blocks; a row with more sources also reads its spare slot.
                const cf v = cmul(d, x);
                const uint32_t slot = entry_slot(ent);   // block * 512 + pi * 8
                *static_cast<float2 *>(__builtin_assume_aligned(regp + slot, 8)) = make_float2(v.r, v.i);
                lds_order();
                if (__any(slot_rank_ovf(slot))) {
                    if (slot_rank_ovf(slot)) {
                        cf *o = reinterpret_cast<cf *>(regp + (slot - kRegionBytes));
                        lds_add(&o->r, v.r);
                        if constexpr (CPLX)
                            lds_add(&o->i, v.i);
                    }
                    lds_order();
                }
                const char *rowp = rowbase + entry_row(ent);   // read block * 512
#pragma unroll
                for (int r = 0; r < kRegions; ++r) {
                    const float2 u = *static_cast<const float2 *>(__builtin_assume_aligned(rowp + r * kRegionBytes, 8));
                    uu[r] = {u.x, u.y};
                }
                if (__any(entry_deg_ovf(ent))) {
                    if (entry_deg_ovf(ent)) {
                        const float2 u = *static_cast<const float2 *>(__builtin_assume_aligned(rowbase + kSpareOff, 8));
                        uu[0].r += u.x;
                        uu[0].i += u.y;
                    }
                }
                lds_order();
            }
            if (tt + 1 < T)
                ent_next = entry(tt + 1);
            if (tt + D < T)
                fetch(q, tt + D);
            // Readout weight of step t-1, through the prefix operator before
            // step t:  Re(c_{t-1} . P D X) = Re(sum_j g_{t-1}[j] X[j]) with
            // g_{t-1}[j] = c_{t-1}[pacc_{t-1}[j]] * dacc_{t-1}[j].
            if (tt > 0) {
                const cf gg = cmul(unpack_raw<CPLX, BCBF>(cgat), dacc);
                gr[tt - 1] = gg.r;
                gi[tt - 1] = gg.i;
                keep_here(gr[tt - 1], gi[tt - 1]);
            }
            if (tt < nvalid_again()) {
                // Extend the prefix operator by step t.
                dacc = cmul(dd, dacc);
                pa4 = (int)((pe & 63u) << 2) + q.gbase * 4;
                cf sum = b;
#pragma unroll
                for (int r = 0; r < kRegions; ++r) {
                    sum.r += uu[r].r;
                    sum.i += uu[r].i;
                }
                x = sum;
                const float qv = c.r * x.r - c.i * x.i;
                qg[tt & 3] = q.row_ok ? qv : 0.f;
            }
            craw_prev = craw;
            if ((tt & 3) == 3)
                w[tt >> 2] = group_fold4<NP>(qg, q.i);
        }
        {
            const cf gg = cmul(unpack_raw<CPLX, BCBF>(bperm_raw_a<CPLX, BCBF>(craw_prev, pa4)), dacc);
            gr[T - 1] = gg.r;
            gi[T - 1] = gg.i;
            keep_here(gr[T - 1], gi[T - 1]);
        }

        __builtin_amdgcn_s_setprio(0);
        // ---- The chunk's operator (pi, d, e) = (pacc, dacc, x) for the carry wave.
        // The local part of the readout, summed over the group's rows now
        // (the sum is linear, so the carry's part is summed on its own).
        using GB = GroupedButterfly<NP, T>;
        group_finish<NP, T / 4>(w, q.i);
        if ((q.i & ((1 << GB::NPLAIN) - 1)) == 0) {
#pragma unroll
            for (int rr = 0; rr < GB::RF; ++rr)
                s_q[wave * G * T + q.g * T + GB::step_of(rr, q.i)] = w[rr];
        }
        // ---- a3: the prefix operators of the tile's chunks, in time order.
        // A wave's G chunks first combine among themselves by an inclusive
        // scan over its lane groups in log2(G) rounds (group g composes its
        // value onto that of group g - s), which needs nothing from the
        // other waves.  Then the wave waits for the prefix of the chunks
        // before its own, composes it under all of its groups at once, and
        // posts the inclusive prefixes (slot wave * 64 + g * NP + i) for the
        // next wave: one composition per wave on the chain across the
        // waves.  The chain is on the tile's critical path, so it runs at
        // raised priority, and its hand-offs rely on the LDS executing each
        // wave's operations in order: a prefix is written before its flag,
        // and read after it.
        //   (later o earlier): pi[j] = pi_l[pi_e[j]], d[j] = d_l[pi_e[j]] * d_e[j],
        //                      e = scatter(pi_l, d_l * e_e) + e_l.
        {
            const int pos = chunk_pos(wave);
            const int slot = wave * 64 + q.ln;
            cf *scr = &s_reg[wave][0][0];   // scatter scratch: a region the next local pass rewrites
            __builtin_amdgcn_s_setprio(PDSSM_CARRY_PRIO);
            int api = (pa4 >> 2) - q.gbase;   // this lane's prefix: first the chunk's own operator
            cf ad = dacc, ae = x;
#pragma unroll
            for (int s = 1; s < G; s <<= 1) {
                // Group g - s's value, from the lane s groups down (lanes of
                // groups g < s fetch another group's value and discard the
                // result; every index stays inside the group).
                const int from = (q.ln - s * NP) & 63;
                const int epi = (int)bperm((uint32_t)api, from);
                cf ed, ee;
                ed.r = bperm(ad.r, from);
                ed.i = CPLX ? bperm(ad.i, from) : 0.f;
                ee.r = bperm(ae.r, from);
                ee.i = CPLX ? bperm(ae.i, from) : 0.f;
                const int src = (q.gbase + epi) * 4;
                const int npi = (int)bperm_a((uint32_t)api, src);
                cf gd;
                gd.r = bperm_a(ad.r, src);
                gd.i = CPLX ? bperm_a(ad.i, src) : 0.f;
                const cf ne = scatter_add<CPLX>(scr, q.ln, q.gbase, api, cmul(ad, ee), ae);
                if (q.g >= s) {
                    api = npi;
                    ad = cmul(gd, ed);
                    ae = ne;
                }
            }
            if (pos > 0) {
                const uint32_t need = 1u << wave_at(pos - 1);
                const int ps = wave_at(pos - 1) * 64 + (G - 1) * NP + q.i;
                int ppi;
                cf pd, pe;
                while (true) {
                    const uint32_t f = *reinterpret_cast<volatile uint32_t *>(&s_ready);
                    lds_order();
                    ppi = s_pi[ps];
                    pd = s_d(ps);
                    pe = s_e[ps];
                    lds_order();
                    if (__builtin_amdgcn_readfirstlane(f) & need)
                        break;
                    __builtin_amdgcn_s_sleep(1);
                }
                const int src = (q.gbase + ppi) * 4;
                const int rpi = (int)bperm_a((uint32_t)api, src);
                cf gd;
                gd.r = bperm_a(ad.r, src);
                gd.i = CPLX ? bperm_a(ad.i, src) : 0.f;
                ae = scatter_add<CPLX>(scr, q.ln, q.gbase, api, cmul(ad, pe), ae);
                api = rpi;
                ad = cmul(gd, pd);
            }
            s_pi[slot] = api;
            s_d(slot) = ad;
            s_e[slot] = ae;
            lds_order();
            if (q.ln == 0)
                __hip_atomic_fetch_or(&s_ready, 1u << wave, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
            __builtin_amdgcn_s_setprio(0);
            // The last prefix of the tile is its aggregate.  While the
            // tile's carry is unknown, later tiles may need it: publish the
            // AGG record (its stores complete while this wave has nothing to
            // wait for).
            if (pos == W - 1 && tile0 > 0 && tile0 + 1 < a.n_tiles && !a.strict) {
                const uint32_t known = __builtin_amdgcn_readfirstlane(*reinterpret_cast<volatile uint32_t *>(&s_known));
                if (known != iter)
                    publish_agg<NP, CPLX>(a, tile0, seq0, epoch, q.i, q.g == G - 1, api, ad, ae);
            }
        }
        __syncthreads();   // (B) all chunk operators taken, next ticket published
        const uint32_t nxt = __builtin_amdgcn_readfirstlane(s_next);
        const bool more = nxt < total;
        // Issued unconditionally (the workgroup's last tile reloads its own
        // rows, which are in range): a load under a condition would keep its
        // registers live around the whole loop.
        issue_scores(more ? nxt : cur);
        __syncthreads();   // (C) carry ready, next table staged

        // ---- a5: carry into this chunk, then the readout
        //   y_t = sum_j ( Re(c_t[j] x_loc_t[j]) + Re(g_t[j] X_chunk[j]) ).
        {
            const Lanes r = lanes();
            const int chunk = chunk_pos(wave) * G + r.g, slot = wave * 64 + r.ln;
            // The slot of the chunk before: this wave's previous group, or
            // the last group of the wave that runs the chunks before.
            const int pslot = (r.g > 0) ? slot - NP : wave_at(max(chunk_pos(wave) - 1, 0)) * 64 + (G - 1) * NP + r.i;
            // Scratch for the scatter: the wave's first scatter region, which
            // the local pass rewrites before it reads it.
            cf *scr = &s_reg[wave][0][0];
            const cf xt = s_xin[r.i];
            int ppi = r.i;
            cf pd = {1.f, 0.f}, pe = {0.f, 0.f};
            if (chunk > 0) {
                ppi = s_pi[pslot];
                pd = s_d(pslot);
                pe = s_e[pslot];
            }
            // The previous wave's slots are rewritten with its next operator
            // once it has left this barrier.
            __syncthreads();   // (D) prefixes and carry read
            const cf xc = scatter_add<CPLX>(scr, r.ln, r.gbase, ppi, cmul(pd, xt), pe);
            // The state before the chunk's first step, kept for the backward scan.
            if (a.xsave) {
                const int tcs = cw0 + r.g * T;
                if (tcs < L && r.row_ok) {
                    constexpr int NC = CPLX ? 2 : 1;
                    float *o = a.xsave + (((int64_t)seq0 * a.nch + tcs / T) * N + r.i) * NC;
                    o[0] = xc.r;
                    if constexpr (CPLX)
                        o[1] = xc.i;
                }
            }
            float wc[T / 4];
#pragma unroll
            for (int m = 0; m < T / 4; ++m) {
                float c4[4];
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    float v = gr[4 * m + k] * xc.r;
                    if constexpr (CPLX)
                        v -= gi[4 * m + k] * xc.i;
                    c4[k] = r.row_ok ? v : 0.f;
                }
                wc[m] = group_fold4<NP>(c4, r.i);
            }
            group_finish<NP, T / 4>(wc, r.i);
            // Outputs go through s_y to the carry wave, which stores them
            // after the next (B), so no store stands between this wave and
            // its next loads; the workgroup's last tile stores them here.
            if ((r.i & ((1 << GB::NPLAIN) - 1)) == 0) {
#pragma unroll
                for (int rr = 0; rr < GB::RF; ++rr) {
                    const int tt = r.g * T + GB::step_of(rr, r.i);   // step within the wave
                    const float yv = s_q[wave * G * T + tt] + wc[rr];
                    if (more) {
                        s_y[iter & 1][wave * G * T + tt] = yv;
                    } else if (cw0 + tt < L) {
                        if (a.y_bf16)
                            (reinterpret_cast<uint16_t *>(a.y) + y0)[tt] = f32_to_bf16_rne(yv);
                        else
                            (reinterpret_cast<float *>(a.y) + y0)[tt] = yv;
                    }
                }
            }
        }
        if (!more)
            return;
        // The next tile's first input steps, then its selection (its scores
        // have been in flight since (B)).  Issued only after the readout, the
        // input loads keep their registers free through it; issued before
        // the selection, their latency overlaps the selection's work (its
        // wait for the scores, loaded earlier, does not wait for them).
        issue_inputs();
        select();
        cur = nxt;
    }
}

// ---------------------------------------------------------------------------
// Per-call preparation.
//  * Blocks >= 1, one wave per dictionary entry (h, k): the entry table
//    tab[h][k][j] = dict_entry(): the 16-bit scatter entry of source j.
//  * Block 0: new epoch and ticket resets; on first use (or after the epoch
//    wraps) clear every carry record.
// ---------------------------------------------------------------------------
constexpr int kPrepThreads = 1024;

__global__ void __launch_bounds__(kPrepThreads) prep_kernel(Header *hdr, uint32_t *ctr, int64_t nctr,
                                                            uint4 *recs, int64_t n16,
                                                            const int32_t *dict, uint16_t *tab,
                                                            int64_t entries, int N, int NP)
{
    if (blockIdx.x > 0) {
        const int lane = threadIdx.x & 63;
        const int64_t e = (int64_t)(blockIdx.x - 1) * (kPrepThreads / 64) + (threadIdx.x >> 6);
        if (e >= entries || lane >= NP)
            return;
        tab[e * NP + lane] = dict_entry(dict + e * N, N, lane);
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
    for (int64_t h = threadIdx.x; h < nctr; h += blockDim.x)
        ctr[32 * h] = 0;
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
// Sequences of no steps.  The state after zero steps is the initial one, and
// the product of no step operators is the identity (pi[j] = j, d[j] = 1).
// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(256) state_fill_kernel(const float *src, float *dst, int64_t n)
{
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256)
        dst[i] = src ? src[i] : 0.f;
}

__global__ void __launch_bounds__(256) identity_op_kernel(int32_t *pi, float *d, int64_t n, int N, int nc)
{
    for (int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x; e < n; e += (int64_t)gridDim.x * 256) {
        pi[e] = (int32_t)(e % N);
        d[e * nc] = 1.f;
        if (nc == 2)
            d[e * nc + 1] = 0.f;
    }
}

static unsigned fill_blocks(int64_t n) { return (unsigned)((n + 255) / 256 < 4096 ? (n + 255) / 256 : 4096); }

int launch_prep(Header *hdr, void *recs, int64_t n16, const int32_t *dict, uint16_t *tab, int64_t entries,
                int N, int NP, hipStream_t stream)
{
    const int64_t blocks = 1 + (entries + kPrepThreads / 64 - 1) / (kPrepThreads / 64);
    hipLaunchKernelGGL(prep_kernel, dim3((unsigned)blocks), dim3(kPrepThreads), 0, stream, hdr, nullptr,
                       (int64_t)0, static_cast<uint4 *>(recs), n16, dict, tab, entries, N, NP);
    return hip_status(hipGetLastError());
}

int launch_state_fill(const void *src, void *dst, int64_t n, hipStream_t stream)
{
    if (n <= 0)
        return PDSSM_OK;
    hipLaunchKernelGGL(state_fill_kernel, dim3(fill_blocks(n)), dim3(256), 0, stream,
                       static_cast<const float *>(src), static_cast<float *>(dst), n);
    return hip_status(hipGetLastError());
}

// ---------------------------------------------------------------------------
// Host side.
// ---------------------------------------------------------------------------
static thread_local std::string g_err;

// Step indices inside a sequence are 32-bit on the device (with room for a
// tile past the end).
constexpr int64_t kMaxL = (int64_t)1 << 30;

static int pad_states(int N) { return N <= 8 ? 8 : N <= 16 ? 16 : N <= 32 ? 32 : 64; }

bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

int check_dims(int64_t B, int64_t H, int64_t L, int32_t N, int32_t K)
{
    if (B < 0 || H < 0 || L < 0 || L > kMaxL || N < 1 || N > 64 || K < 1 || K > 32767)
        return PDSSM_ERR_DIM;
    // Element counts must fit int64 and tile tickets a uint32.
    const double steps = (double)B * (double)H * (double)L;
    if (steps * 64.0 * 8.0 > 9.0e18 || (double)B * (double)H * 64.0 * 8.0 > 9.0e18)
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
    int64_t n_tiles, n_ctiles, S, ctr_bytes, tab_bytes, agg_bytes, incl_bytes, compose_bytes, total;
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
    lo.ctr_bytes = H * 128;   // one ticket counter per head, each on its own 128-byte line
    lo.tab_bytes = (H * (int64_t)K * lo.NP * 2 + 255) / 256 * 256;
    const int64_t scan = lo.ctr_bytes + lo.tab_bytes + lo.agg_bytes + lo.incl_bytes;
    lo.total = (int64_t)sizeof(Header) + ((scan > lo.compose_bytes ? scan : lo.compose_bytes) + 15) / 16 * 16;
    return lo;
}

int hip_status(hipError_t e)
{
    if (e == hipSuccess)
        return PDSSM_OK;
    g_err = std::string("HIP error: ") + hipGetErrorString(e);
    return PDSSM_ERR_HIP;
}

// Persistent grid: as many workgroups as the device holds at once (they
// loop over the tiles), never more than there are tiles.
#ifndef PDSSM_STRICT_WGS_PER_SEQ
#define PDSSM_STRICT_WGS_PER_SEQ 12
#endif
constexpr int64_t kStrictWgsPerSeq = PDSSM_STRICT_WGS_PER_SEQ;

template <int NP, bool CPLX, bool BCBF>
static hipError_t launch_scan(const ScanArgs &a, hipStream_t st)
{
    // The table is staged in rows of 64 lanes x 16 bytes: whole rows fit.
    const size_t dyn = a.dict_lds ? (((size_t)a.K * NP * 2 + 1023) & ~(size_t)1023)
                                  : (size_t)kScanW * kScanT * 64 * 2;
    const int block = (kScanW + 1) * 64;
    // Resident workgroups per device, cached per (device, LDS size).
    static thread_local int c_dev = -1, c_wgs = 0;
    static thread_local size_t c_dyn = 0;
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess)
        return e;
    if (dev != c_dev || dyn != c_dyn) {
        int per_cu = 0, cus = 0;
        e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, scan_kernel<NP, CPLX, BCBF>, block, dyn);
        if (e != hipSuccess)
            return e;
        e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
        if (e != hipSuccess)
            return e;
        c_wgs = (per_cu > 0 ? per_cu : 1) * (cus > 0 ? cus : 1);
        c_dev = dev;
        c_dyn = dyn;
    }
    // When the head's table lives in LDS and every head gets at least one
    // resident workgroup, workgroup w serves head w % H only: its table is
    // staged once.  Otherwise one ticket stream covers all sequences.
    ScanArgs b = a;
    unsigned grid;
    if (a.dict_lds && a.ctr && (int64_t)c_wgs >= a.H) {
        const int64_t per_head = ((int64_t)c_wgs / a.H < (int64_t)a.total_head) ? (int64_t)c_wgs / a.H
                                                                              : (int64_t)a.total_head;
        grid = (unsigned)(per_head * a.H);
    } else {
        b.ctr = nullptr;
        grid = (unsigned)((int64_t)a.total < c_wgs ? (int64_t)a.total : c_wgs);
    }
    // Aggregate records let a tile's carry skip ahead of unfinished tiles;
    // writing and polling them costs a few per cent of the call.  A tile
    // whose predecessor has its carry gets its own about 1.1 us later, so
    // with up to kStrictWgsPerSeq workgroups per sequence the plain chain
    // keeps up with the tiles being worked on, and is used.
    if ((int64_t)grid <= kStrictWgsPerSeq * a.S)
        b.strict = 1;
    hipLaunchKernelGGL((scan_kernel<NP, CPLX, BCBF>), dim3(grid), dim3(block), dyn, st, b);
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

// ---------------------------------------------------------------------------
// Scratch of the allocation-free forward scan: one file-scope device array
// that every GPU the library runs on holds (its own copy) until the process
// ends.  Host code uses the array's device address, found once per device
// with hipGetSymbolAddress: the array's name on the host is only a stand-in.
// ---------------------------------------------------------------------------
constexpr size_t kScratchBytes = (size_t)64 << 20;
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
static std::mutex g_scratch_mu;
static void *g_scratch[kMaxDevices];

static int scratch_address(void **out)
{
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess)
        return hip_status(e);
    if (dev < 0 || dev >= kMaxDevices) {
        g_err = "device index beyond the allocation-free scratch table";
        return PDSSM_ERR_HIP;
    }
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch[dev]) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess)
            return hip_status(e);
        if (!p) {
            g_err = "hipGetSymbolAddress gave no address for the scratch array";
            return PDSSM_ERR_HIP;
        }
        g_scratch[dev] = p;
    }
    *out = g_scratch[dev];
    return PDSSM_OK;
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

static int scan_fwd(const void *sel_or_logits, const int32_t *dict_idx, const void *diag,
                    const void *b, const void *c, void *y, void *x_final, int64_t B, int64_t H,
                    int64_t L, int32_t N, int32_t K, uint32_t flags, const void *x0,
                    void *workspace, size_t workspace_bytes, bool save, void *x_chunks,
                    int16_t *sel_save, hipStream_t stream)
{
    int rc = check_dims(B, H, L, N, K);
    if (rc != PDSSM_OK)
        return rc;
    if (flags & ~PDSSM_FLAGS_ALL)
        return PDSSM_ERR_FLAGS;
    if (B == 0 || H == 0)
        return PDSSM_OK;   // no sequences: nothing to read or write
    if (L == 0) {
        // No steps: x_final = x0 (or zero); every other buffer is empty.
        if (!x_final)
            return PDSSM_OK;
        if (!aligned16(x_final) || (x0 && !aligned16(x0)))
            return PDSSM_ERR_ALIGN;
        return launch_state_fill(x0, x_final, B * H * N * ((flags & PDSSM_COMPLEX) ? 2 : 1), stream);
    }
    if (!sel_or_logits || !dict_idx || !diag || !b || !c || !y || !workspace || (save && !x_chunks))
        return PDSSM_ERR_NULL;
    if ((x_chunks && !aligned16(x_chunks)) || (sel_save && !aligned16(sel_save)))
        return PDSSM_ERR_ALIGN;
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
    a.xsave = static_cast<float *>(x_chunks);
    a.selsave = sel_save;
    a.nch = (L + kScanT - 1) / kScanT;
    a.hdr = static_cast<Header *>(workspace);
    uint32_t *ctr = reinterpret_cast<uint32_t *>(static_cast<char *>(workspace) + sizeof(Header));
    uint16_t *tab = reinterpret_cast<uint16_t *>(reinterpret_cast<char *>(ctr) + lo.ctr_bytes);
    a.tab = tab;
    a.ctr = ctr;   // launch_scan decides whether the tickets run per head
    a.total_head = (uint32_t)(lo.n_tiles * B);
    a.agg = reinterpret_cast<uint64_t *>(reinterpret_cast<char *>(tab) + lo.tab_bytes);
    a.incl = reinterpret_cast<uint64_t *>(reinterpret_cast<char *>(a.agg) + lo.agg_bytes);
    a.H = H;
    a.L = L;
    a.S = lo.S;
    a.n_tiles = lo.n_tiles;
    a.total = (uint32_t)(lo.n_tiles * lo.S);
    a.N = N;
    a.K = K;
    a.sel_mode = flags & PDSSM_SEL_MASK;
    a.y_bf16 = (flags & PDSSM_Y_BF16) ? 1 : 0;
    a.strict = (flags & PDSSM_DETERMINISTIC) ? 1 : 0;   // launch_scan may set it too
    a.dict_lds = ((int64_t)K * lo.NP * 2 <= kDictLdsMax) ? 1 : 0;

    const int64_t rec_bytes = lo.agg_bytes + lo.incl_bytes;
    const int64_t entries = H * (int64_t)K;
    const int64_t prep_blocks = 1 + (entries + kPrepThreads / 64 - 1) / (kPrepThreads / 64);
    hipLaunchKernelGGL(prep_kernel, dim3((unsigned)prep_blocks), dim3(kPrepThreads), 0, stream, a.hdr, ctr,
                       (int64_t)H, reinterpret_cast<uint4 *>(a.agg), (int64_t)(rec_bytes / 16), dict_idx, tab,
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

extern "C" int pdssm_scan_fwd(const void *sel_or_logits, const int32_t *dict_idx, const void *diag,
                              const void *b, const void *c, void *y, void *x_final, int64_t B,
                              int64_t H, int64_t L, int32_t N, int32_t K, uint32_t flags,
                              const void *x0, void *workspace, size_t workspace_bytes,
                              hipStream_t stream)
{
    return scan_fwd(sel_or_logits, dict_idx, diag, b, c, y, x_final, B, H, L, N, K, flags, x0,
                    workspace, workspace_bytes, false, nullptr, nullptr, stream);
}

extern "C" int pdssm_scan_fwd_noalloc(const void *sel_or_logits, const int32_t *dict_idx,
                                      const void *diag, const void *b, const void *c, void *y,
                                      void *x_final, int64_t B, int64_t H, int64_t L, int32_t N,
                                      int32_t K, uint32_t flags, const void *x0, hipStream_t stream)
{
    int rc = check_dims(B, H, L, N, K);
    if (rc != PDSSM_OK)
        return rc;
    if (flags & ~PDSSM_FLAGS_ALL)
        return PDSSM_ERR_FLAGS;
    if (B == 0 || H == 0 || L == 0)   // touches no workspace
        return scan_fwd(sel_or_logits, dict_idx, diag, b, c, y, x_final, B, H, L, N, K, flags, x0,
                        nullptr, 0, false, nullptr, nullptr, stream);
    if ((size_t)layout_of(B, H, L, N, K, flags).total > kScratchBytes)
        return PDSSM_ERR_SCRATCH;
    void *ws = nullptr;
    rc = scratch_address(&ws);
    if (rc != PDSSM_OK)
        return rc;
    return scan_fwd(sel_or_logits, dict_idx, diag, b, c, y, x_final, B, H, L, N, K, flags, x0, ws,
                    kScratchBytes, false, nullptr, nullptr, stream);
}

extern "C" int pdssm_scan_fwd_save(const void *sel_or_logits, const int32_t *dict_idx,
                                   const void *diag, const void *b, const void *c, void *y,
                                   void *x_final, void *x_chunks, int16_t *sel_out, int64_t B,
                                   int64_t H, int64_t L, int32_t N, int32_t K, uint32_t flags,
                                   const void *x0, void *workspace, size_t workspace_bytes,
                                   hipStream_t stream)
{
    return scan_fwd(sel_or_logits, dict_idx, diag, b, c, y, x_final, B, H, L, N, K, flags, x0,
                    workspace, workspace_bytes, true, x_chunks, sel_out, stream);
}

extern "C" int pdssm_select(const void *sel_or_logits, int32_t *sel_out, int64_t B, int64_t H,
                            int64_t L, int32_t K, uint32_t flags, hipStream_t stream)
{
    int rc = check_dims(B, H, L, 1, K);
    if (rc != PDSSM_OK)
        return rc;
    if (flags & ~PDSSM_SEL_MASK)
        return PDSSM_ERR_FLAGS;
    if (B == 0 || H == 0 || L == 0)
        return PDSSM_OK;
    if (!sel_or_logits || !sel_out)
        return PDSSM_ERR_NULL;
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
    int rc = check_dims(B, H, L, N, K);
    if (rc != PDSSM_OK)
        return rc;
    if (flags & ~(PDSSM_SEL_MASK | PDSSM_COMPLEX))
        return PDSSM_ERR_FLAGS;
    if (B == 0 || H == 0)
        return PDSSM_OK;
    if (L == 0) {
        // The product of no steps: the identity.
        if (!pi_out || !d_out)
            return PDSSM_ERR_NULL;
        if (!aligned16(pi_out) || !aligned16(d_out))
            return PDSSM_ERR_ALIGN;
        const int64_t n = B * H * N;
        hipLaunchKernelGGL(identity_op_kernel, dim3(fill_blocks(n)), dim3(256), 0, stream, pi_out,
                           static_cast<float *>(d_out), n, (int)N, (flags & PDSSM_COMPLEX) ? 2 : 1);
        return hip_status(hipGetLastError());
    }
    if (!sel_or_logits || !dict_idx || !diag || !pi_out || !d_out || !workspace)
        return PDSSM_ERR_NULL;
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
    case PDSSM_ERR_DIM:
        return "invalid sizes (B, H, L >= 0; N in [1,64]; K in [1,32767], at most 128 for the router; "
               "router D a positive multiple of 32; or a size too large)";
    case PDSSM_ERR_FLAGS: return "invalid flags";
    case PDSSM_ERR_ALIGN: return "a pointer is not 16-byte aligned";
    case PDSSM_ERR_WORKSPACE: return "workspace too small";
    case PDSSM_ERR_SCRATCH:
        return "the sizes need more workspace than the allocation-free entry point's 64 MiB scratch";
    case PDSSM_ERR_HIP: return g_err.empty() ? "HIP error" : g_err.c_str();
    default: return "unknown status";
    }
}
