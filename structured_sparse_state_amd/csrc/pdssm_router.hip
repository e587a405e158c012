// Router selection fused with its GEMM: the step's K scores per head come
// from the step input by a linear transformation, and only their argmax -- the
// selected dictionary entry -- leaves the chip.  "Flash PD-SSM:
// Memory-Optimized Structured Sparse State-Space Models" (Technical Summary,
// Methodology, "1. Novel Selection Mechanism (Hard Selection)").
//
//     scores[b,h,t,k] = sum_d u[b,t,d] * w[h,k,d]        (no bias)
//     sel[b,h,t]      = argmax_k scores[b,h,t,k]         (first maximum wins)
//
// As a matrix product: C[M, H*64] = U[M, D] * W^T with M = B*L tokens and each
// head's K <= 64 weight rows padded to 64 columns.  It is a dense
// contraction, so it runs on the matrix cores: v_mfma_f32_32x32x16_bf16,
// fp32 accumulation.  A workgroup computes a 256-token x 2-head tile; each of
// its four waves owns 128 tokens x one head (4 x 2 MFMA tiles), so the argmax
// over a head's scores stays inside one wave.  U and W tiles of 32 features
// go straight from global memory into a three-stage LDS ring
// (global_load_lds, 16 bytes per lane, chunks swizzled within each row so
// fragment reads do not conflict); two stages are in flight while the third
// is consumed.
#include <hip/hip_runtime.h>

#include "pdssm.h"
#include "pdssm_device.h"
#include "pdssm_host.h"

namespace pdssm {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

#ifndef PDSSM_ROUTER_HEADS
#define PDSSM_ROUTER_HEADS 2
#endif
constexpr int kRM = 256;                  // tokens per workgroup tile
constexpr int kRH = PDSSM_ROUTER_HEADS;   // heads per workgroup tile (2 or 4)
constexpr int kWH = kRH / 2;              // heads per wave (waves are 2 x 2)
constexpr int kNT = 2 * kWH;              // 32-column MFMA tiles per wave
constexpr int kRN = kRH * 64;             // padded score columns per tile
#ifndef PDSSM_ROUTER_BK
#define PDSSM_ROUTER_BK 32
#endif
#ifndef PDSSM_ROUTER_STAGES
#define PDSSM_ROUTER_STAGES 2
#endif
constexpr int kRK = PDSSM_ROUTER_BK;      // features per LDS stage (32 or 64)
constexpr int kRStages = PDSSM_ROUTER_STAGES;
constexpr int kRowBytes = kRK * 2;        // bytes of one row of a stage
constexpr int kChunks = kRK / 8;          // 16-byte chunks per row
constexpr int kRowsPerLoad = 64 / kChunks;   // rows one 64-lane 16-byte load fills
constexpr int kABytes = kRM * kRowBytes;  // token rows per stage
constexpr int kBBytes = kRN * kRowBytes;  // weight rows per stage
constexpr int kStageBytes = kABytes + kBBytes;
constexpr int kRThreads = 256;
constexpr int kALoads = kRM / kRowsPerLoad / 4;   // direct-to-LDS loads per wave per stage
constexpr int kBLoads = kRN / kRowsPerLoad / 4;
constexpr int kLoadsPerStage = kALoads + kBLoads;
// Workgroups per CU that the LDS allows (one wave of each per SIMD), at most
// three with one head per wave (about 168 VGPRs, 128 of them accumulators)
// and one with two (256 accumulators).
constexpr int kRWaveCap = kWH == 1 ? 3 : 1;
constexpr int kRWavesPerEU = (160 * 1024) / (kRStages * kStageBytes) < kRWaveCap
                                 ? (160 * 1024) / (kRStages * kStageBytes) : kRWaveCap;
static_assert(kRH == 2 || kRH == 4, "heads per tile");
static_assert(kRK == 16 || kRK == 32 || kRK == 64, "stage depth");
static_assert(kRStages >= 2 && kRStages * kStageBytes <= 160 * 1024, "stages fit in LDS");

struct RouterArgs {
    const uint16_t *u;   // [M][D] bf16
    const uint16_t *w;   // [H][K][D] bf16
    int16_t *sel;        // [B][H][L]
    int64_t M, L, H;
    int K, D;
    uint32_t m_tiles, h_tiles;
};

// Position of 16-byte chunk c of row r inside the row.  A fragment read
// (ds_read_b128) has lane l read row l % 32 of a 32-row block; the chunks are
// rotated from row to row so that both the 8 lanes of every 128-byte group
// and the 16 lanes of every 256-byte group of the read land on distinct
// 16-byte bank groups.  The rotation depends on r % 32 only: fragments
// start at multiples of 32 rows.
__device__ __forceinline__ int chunk_pos(int r, int c)
{
    if constexpr (kChunks == 2)
        return c ^ (((r >> 2) ^ (r >> 3)) & 1);
    else if constexpr (kChunks == 4)
        return c ^ (((r >> 1) ^ (r >> 3)) & 3);
    else
        return c ^ ((r ^ ((r >> 3) & 3)) & 7);
}

// better() of the selection (the score, then the lower index; a NaN above
// every number, the first NaN winning) as one boolean expression, so that the
// compiler selects instead of branching per comparison.
__device__ __forceinline__ bool beats(float v2, int k2, float v1, int k1)
{
    const bool n1 = v1 != v1, n2 = v2 != v2;
    const bool klt = k2 < k1;
    return (n2 & (!n1 | klt)) | (!n2 & !n1 & ((v2 > v1) | ((v2 == v1) & klt)));
}

// s_waitcnt with only the vector-memory count constrained (gfx9 encoding).
template <int N>
__device__ __forceinline__ void wait_vm()
{
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

__global__ void __launch_bounds__(kRThreads, kRWavesPerEU) router_kernel(RouterArgs a)
{
    __shared__ __attribute__((aligned(1024))) char smem[kRStages * kStageBytes];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);

    // Tile of this workgroup.  Consecutive workgroups go to different XCDs;
    // the mapping gives each XCD a contiguous run of tiles, so the head tiles
    // of one token tile (which read the same U rows) share that XCD's L2.
    const uint32_t total = a.m_tiles * a.h_tiles, per = total / 8;
    const uint32_t bx = blockIdx.x;
    const uint32_t tile = (bx < per * 8) ? (bx % 8) * per + bx / 8 : bx;
    const uint32_t mt = tile / a.h_tiles, ht = tile % a.h_tiles;
    const int64_t m0 = (int64_t)mt * kRM;
    const int64_t h0 = (int64_t)ht * kRH;
    const int D = a.D, K = a.K;

    // Direct-to-LDS loads: load j of this wave fills the kRowsPerLoad rows
    // from R g on (g = wave * loads + j, R = kRowsPerLoad), lane i writing
    // the 16-byte slot i, i.e. row R g + i / kChunks at position
    // i % kChunks, which holds the chunk chunk_pos(row, i % kChunks) (the
    // swizzle is its own inverse).  Rows past the token count or padding
    // score columns read row 0 instead: their results are never used.
    const uint16_t *asrc[kALoads];
#pragma unroll
    for (int j = 0; j < kALoads; ++j) {
        const int r = kRowsPerLoad * (wave * kALoads + j) + lane / kChunks;
        const int64_t m = m0 + r;
        asrc[j] = a.u + (m < a.M ? m : 0) * (int64_t)D + chunk_pos(r, lane % kChunks) * 8;
    }
    const uint16_t *bsrc[kBLoads];
#pragma unroll
    for (int j = 0; j < kBLoads; ++j) {
        const int col = kRowsPerLoad * (wave * kBLoads + j) + lane / kChunks;
        const int64_t h = h0 + col / 64;
        const int k = col % 64;
        bsrc[j] = a.w + ((h < a.H && k < K) ? (h * K + k) : 0) * (int64_t)D + chunk_pos(col, lane % kChunks) * 8;
    }
    // The loads are written in asm so that the compiler does not see them
    // as stores to LDS: it would otherwise make every fragment read wait
    // for all of them (it cannot tell the stages apart).  They write no
    // registers; the stage waits below are explicit.
    auto dma = [](const uint16_t *src, uint32_t lds) {
        asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off"
                     :
                     : "v"(src), "s"(lds)
                     : "memory", "m0");
    };
    auto issue = [&](char *buf, int k0) {
        const uint32_t base = __builtin_amdgcn_readfirstlane(lds_addr(buf));
#pragma unroll
        for (int j = 0; j < kALoads; ++j)
            dma(asrc[j] + k0, base + (uint32_t)((wave * kALoads + j) * 1024));
#pragma unroll
        for (int j = 0; j < kBLoads; ++j)
            dma(bsrc[j] + k0, base + (uint32_t)(kABytes + (wave * kBLoads + j) * 1024));
    };

    // This wave: tokens wm*128 .. +128 of the tile, heads wn*kWH .. +kWH.
    const int wm = wave >> 1, wn = wave & 1;
    f32x16 acc[4][kNT];
#pragma unroll
    for (int mi = 0; mi < 4; ++mi)
#pragma unroll
        for (int ni = 0; ni < kNT; ++ni)
#pragma unroll
            for (int e = 0; e < 16; ++e)
                acc[mi][ni][e] = 0.f;

    // Fragments: row (lane % 32) of a 32-row block, features 16 ks + 8 (lane
    // / 32).  Blocks start at multiples of 32 rows, so the swizzled offset of
    // the lane inside a block depends on the lane and ks only.
    uint32_t lane_off[kRK / 16];
#pragma unroll
    for (int ks = 0; ks < kRK / 16; ++ks)
        lane_off[ks] = (uint32_t)((lane & 31) * kRowBytes + chunk_pos(lane & 31, ks * 2 + (lane >> 5)) * 16);
    auto compute = [&](const char *base) {
        const char *ab = base + wm * 128 * kRowBytes;
        const char *bb = base + kABytes + wn * kWH * 64 * kRowBytes;
#pragma unroll
        for (int ks = 0; ks < kRK / 16; ++ks) {
            bf16x8 af[4], bf[kNT];
#pragma unroll
            for (int mi = 0; mi < 4; ++mi)
                af[mi] = *reinterpret_cast<const bf16x8 *>(ab + mi * 32 * kRowBytes + lane_off[ks]);
#pragma unroll
            for (int ni = 0; ni < kNT; ++ni)
                bf[ni] = *reinterpret_cast<const bf16x8 *>(bb + ni * 32 * kRowBytes + lane_off[ks]);
#pragma unroll
            for (int mi = 0; mi < 4; ++mi)
#pragma unroll
                for (int ni = 0; ni < kNT; ++ni)
                    acc[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[mi], bf[ni], acc[mi][ni], 0, 0, 0);
        }
    };

    // Ring of kRStages stages: stage s is consumed while the next
    // kRStages - 1 load.  Before consuming s each wave waits for its own
    // loads of s (those of the younger stages may stay in flight), then the
    // barrier makes every wave's rows of s visible and frees the buffer of
    // s - 1, which the loads of s + kRStages - 1 then refill.
    const int stages = D / kRK;
#pragma unroll
    for (int p = 0; p < kRStages - 1; ++p)
        if (p < stages)
            issue(smem + p * kStageBytes, p * kRK);
    for (int s = 0; s < stages; ++s) {
        const int ahead = min(stages - 1 - s, kRStages - 2);   // younger stages already issued
        if (ahead >= kRStages - 2)
            wait_vm<kLoadsPerStage * (kRStages - 2)>();
        else if (kRStages > 3 && ahead == 1)
            wait_vm<kLoadsPerStage>();
        else
            wait_vm<0>();
        __builtin_amdgcn_s_barrier();
        lds_order();   // no LDS access moves across the barrier
        if (s + kRStages - 1 < stages)
            issue(smem + ((s + kRStages - 1) % kRStages) * kStageBytes, (s + kRStages - 1) * kRK);
        compute(smem + (s % kRStages) * kStageBytes);
    }

    // Argmax per token over the head's K scores.  acc[mi][ni][e] is the
    // score of token wm*128 + mi*32 + 8*(e/4) + 4*(lane/32) + e%4 and entry
    // k = ni*32 + lane%32.  Each lane first keeps the better of its two
    // entries for each of its 64 tokens (c = mi*16 + e); then the 32 lanes
    // of each half-wave reduce by recursive halving: at the exchange with the
    // lane 2^s apart, a lane keeps half of its tokens and hands the other
    // half to its partner, so after five exchanges lane l holds the result of
    // tokens c = 2 (l % 32) and 2 (l % 32) + 1 (62 values sent per lane
    // instead of 5 per token).  better() orders by score, then by lower
    // index, so the merge order does not matter.
#pragma unroll
    for (int hn = 0; hn < kWH; ++hn) {
        const int64_t h = h0 + wn * kWH + hn;
        float bv[64];
        int bk[64];
#pragma unroll
        for (int mi = 0; mi < 4; ++mi) {
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const int c = mi * 16 + e;
                const int k0 = lane & 31, k1 = 32 + (lane & 31);
                bv[c] = (k0 < K) ? acc[mi][2 * hn][e] : __uint_as_float(0xFF800000u);   // -inf: beaten by any score
                bk[c] = (k0 < K) ? k0 : 64;
                const bool take = (k1 < K) & beats(acc[mi][2 * hn + 1][e], k1, bv[c], bk[c]);
                bv[c] = take ? acc[mi][2 * hn + 1][e] : bv[c];
                bk[c] = take ? k1 : bk[c];
            }
        }
#pragma unroll
        for (int st = 0; st < 5; ++st) {
            const int m = 16 >> st;          // partner distance
            const int n = 32 >> st;          // tokens kept after this exchange
            const bool upper = (lane & m) != 0;
#pragma unroll
            for (int i = 0; i < n; ++i) {
                // keep i (lower lane) or n + i (upper lane); send the other
                const float sv = upper ? bv[i] : bv[n + i];
                const int sk = upper ? bk[i] : bk[n + i];
                float kv = upper ? bv[n + i] : bv[i];
                int kk = upper ? bk[n + i] : bk[i];
                const float ov = __shfl_xor(sv, m, 64);
                const int ok = __shfl_xor(sk, m, 64);
                const bool take = beats(ov, ok, kv, kk);
                bv[i] = take ? ov : kv;
                bk[i] = take ? ok : kk;
            }
        }
        if (h < a.H) {
#pragma unroll
            for (int r = 0; r < 2; ++r) {
                const int c = 2 * (lane & 31) + r, mi = c >> 4, e = c & 15;
                const int64_t m = m0 + wm * 128 + mi * 32 + 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3);
                if (m < a.M) {
                    const int64_t b = m / a.L, t = m - b * a.L;
                    a.sel[(b * a.H + h) * a.L + t] = (int16_t)bk[r];
                }
            }
        }
    }
}

}  // namespace
}  // namespace pdssm

using namespace pdssm;

extern "C" int pdssm_router_select(const void *u, const void *w, int16_t *sel_out, int64_t B, int64_t L,
                                   int64_t H, int32_t K, int32_t D, uint32_t flags, hipStream_t stream)
{
    if (B < 0 || L < 0 || H < 0 || K < 1 || K > 64 || D < kRK || (D % kRK) != 0)
        return PDSSM_ERR_DIM;
    const double tokens = (double)B * (double)L;
    const double m_tiles = (tokens + kRM - 1) / kRM, h_tiles = (double)((H + kRH - 1) / kRH);
    if (tokens > 2.0e9 || m_tiles * h_tiles > 2.0e9 || (double)H * K * D > 4.0e18)
        return PDSSM_ERR_DIM;
    if (flags != 0)
        return PDSSM_ERR_FLAGS;
    if (B == 0 || L == 0 || H == 0)
        return PDSSM_OK;   // no tokens or no heads: nothing to write
    if (!u || !w || !sel_out)
        return PDSSM_ERR_NULL;
    if (!aligned16(u) || !aligned16(w) || !aligned16(sel_out))
        return PDSSM_ERR_ALIGN;
    RouterArgs a;
    a.u = static_cast<const uint16_t *>(u);
    a.w = static_cast<const uint16_t *>(w);
    a.sel = sel_out;
    a.M = B * L;
    a.L = L;
    a.H = H;
    a.K = K;
    a.D = D;
    a.m_tiles = (uint32_t)((a.M + kRM - 1) / kRM);
    a.h_tiles = (uint32_t)((H + kRH - 1) / kRH);
    hipLaunchKernelGGL(router_kernel, dim3(a.m_tiles * a.h_tiles), dim3(kRThreads), 0, stream, a);
    return hip_status(hipGetLastError());
}
