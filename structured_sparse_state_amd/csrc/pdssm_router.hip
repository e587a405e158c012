// Router selection fused with its GEMM: the step's K scores per head come
// from the step input by a linear transformation, and only their argmax -- the
// selected dictionary entry -- leaves the chip.  "Flash PD-SSM:
// Memory-Optimized Structured Sparse State-Space Models" (Technical Summary,
// Methodology, "1. Novel Selection Mechanism (Hard Selection)").
//
//     scores[b,h,t,k] = sum_d u[b,t,d] * w[h,k,d]        (no bias)
//     sel[b,h,t]      = argmax_k scores[b,h,t,k]         (first maximum wins)
//
// As a matrix product: C[M, H*P] = U[M, D] * W^T with M = B*L tokens and each
// head's K weight rows padded to P = 64 or 128 columns.  It is a dense
// contraction, so it runs on the matrix cores: v_mfma_f32_32x32x16_bf16,
// fp32 accumulation.  Each of a workgroup's four waves owns 128 tokens x 128
// columns (4 x 4 MFMA tiles, 256 accumulators, one wave per SIMD), so every
// head's scores stay inside one wave and each fragment feeds four MFMAs.
// With one wave per SIMD nothing else hides latency, so the loops are
// software-pipelined: the fragments of the next 16 features are read while
// the MFMAs of the current ones run.
//
// Two kernels, by the layout of the weights:
//   * [H][K][D] (router_lds_kernel): a workgroup tile of 256 tokens x 256
//     columns, waves 2 x 2.  Token rows and weight rows both go straight
//     from global memory into a ring of LDS stages (global_load_lds, 16
//     bytes per lane, whole 128-byte lines per load).  Per 16 features a CU
//     then writes 16 KB and reads 32 KB of LDS, more than the LDS delivers
//     in the MFMAs' time, which bounds this kernel.
//   * packed, [H][D/8][P][8] (router_wreg_kernel; pdssm_router_pack_weights
//     writes it): a workgroup tile of 128 tokens x 512 columns, so the four
//     waves share one set of token rows, which go through LDS as above, and
//     each loads its own weight fragments straight into a ring of
//     registers.  In this layout the 32 columns of a fragment are 512
//     contiguous bytes per 8 features, so a fragment load touches whole
//     lines (in [H][K][D] it would touch 32 rows).  Per 16 features a CU
//     then writes 4 KB and reads 16 KB of LDS and loads 16 KB of weights.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <type_traits>

#include "pdssm.h"
#include "pdssm_device.h"
#include "pdssm_host.h"

namespace pdssm {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kRM = 256;     // router_lds_kernel: tokens per workgroup tile
constexpr int kRN = 256;     // and score columns (waves 2 x 2)
constexpr int kWM = 128;     // router_wreg_kernel: tokens per workgroup tile
constexpr int kWN = 512;     // and score columns (waves 1 x 4)
constexpr int kRThreads = 256;
constexpr int kRingBytes = 128 * 1024;   // LDS ring of every stage depth

// router_lds_kernel's LDS stage of BK features of token and weight rows: 64
// (two stages in the ring) when the feature count allows it, else 32 (four
// stages).  Deeper stages mean fewer stage hand-overs (barriers) per MFMA.
template <int BK>
struct PairStage {
    static constexpr int kRK = BK;                      // features per LDS stage
    static constexpr int kRowBytes = BK * 2;            // bytes of one row of a stage
    static constexpr int kChunks = BK / 8;              // 16-byte chunks per row
    static constexpr int kRowsPerLoad = 64 / kChunks;   // rows one 64-lane 16-byte load fills
    static constexpr int kABytes = kRM * kRowBytes;     // token rows per stage
    static constexpr int kBBytes = kRN * kRowBytes;     // weight rows per stage
    static constexpr int kStageBytes = kABytes + kBBytes;
    static constexpr int kRStages = kRingBytes / kStageBytes;
    static constexpr int kALoads = kRM / kRowsPerLoad / 4;   // direct-to-LDS loads per wave per stage
    static constexpr int kBLoads = kRN / kRowsPerLoad / 4;
    static constexpr int kLoadsPerStage = kALoads + kBLoads;
    static_assert(BK == 32 || BK == 64, "stage depth");
    static_assert(kRStages >= 2 && kRStages <= 4, "stage waits cover up to three younger stages");
    static_assert((BK / 16) % 2 == 0, "the fragment double buffer alternates by step parity");
    static_assert(kLoadsPerStage * 3 < 64, "vmcnt range");
};

// router_wreg_kernel's LDS stage of BK features of its 128 token rows: 64
// when the feature count allows it, else 32.  The weight rows do not pass
// through LDS (each wave loads its own fragments into registers), so the
// ring holds token rows only: two groups of 128 features, four 64-feature
// stages or eight 32-feature ones (64 KB).
template <int BK>
struct TokenStage {
    static constexpr int kRK = BK;                      // features per LDS stage
    static constexpr int kRowBytes = BK * 2;            // bytes of one row of a stage
    static constexpr int kChunks = BK / 8;              // 16-byte chunks per row
    static constexpr int kRowsPerLoad = 64 / kChunks;   // rows one 64-lane 16-byte load fills
    static constexpr int kStageBytes = kWM * kRowBytes;   // token rows per stage
    static constexpr int kRStages = 2 * (128 / BK);      // two groups of 128 features
    static constexpr int kALoads = kWM / kRowsPerLoad / 4;   // direct-to-LDS loads per wave per stage
    static_assert(BK == 32 || BK == 64, "stage depth");
    static constexpr int kGroupStages = 128 / BK;   // stages of 128 features (one hand-over each)
    static_assert(kRStages == 2 * kGroupStages, "the ring holds two groups of 128 features");
};

struct RouterArgs {
    const uint16_t *u;   // [M][D] bf16
    const uint16_t *w;   // [H][K][D] bf16, or packed [H][D/8][P][8] (P = 64 or 128)
    int16_t *sel;        // [B][H][L]
    int64_t M, L, H;
    int K, D;
    uint32_t m_tiles, n_tiles;
};

// Position of 16-byte chunk c of row r inside the row.  A fragment read
// (ds_read_b128) has lane l read row l % 32 of a 32-row block; the chunks are
// rotated from row to row so that the reads do not conflict in the LDS banks
// (for four chunks per row the rotation was chosen by measuring fragment-read
// throughput: three of eight candidate rotations run 1.5 times faster than
// the others and match the conflict-free eight-chunk rotation's rate).  The
// rotation depends on r % 32 only: fragments start at multiples of 32 rows.
template <int kChunks>
__device__ __forceinline__ int chunk_pos(int r, int c)
{
    if constexpr (kChunks == 4)
        return c ^ ((r ^ (r >> 2)) & 3);
    else
        return c ^ ((r ^ ((r >> 3) & 3)) & 7);
}

// The selection's order on values (-0 equal to +0; a NaN above every number)
// in integers: value_key maps the score's bits to an int32 that orders like
// the value (negative values have their magnitude bits flipped, -0 is made
// +0 first, every NaN becomes INT32_MAX).  A strict comparison of keys in
// index order then keeps the first maximum, and the first NaN.
__device__ __forceinline__ int32_t value_key(float v)
{
    const float f = v + 0.0f;   // -0 + 0 = +0 (round to nearest); NaN stays NaN
    const int32_t i = __float_as_int(f);
    const int32_t key = i ^ ((i >> 31) & 0x7fffffff);
    return (f != f) ? 0x7fffffff : key;
}
// Below the key of every score (-inf's is INT32_MIN + 0x7fffff).
constexpr int32_t kNoValue = INT32_MIN;

// s_waitcnt with only the vector-memory count constrained (gfx9 encoding).
template <int N>
__device__ __forceinline__ void wait_vm()
{
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// The epilogue's LDS: per wave, 64 score columns of its 128 tokens, each
// column 512 bytes plus 16 of padding (so that the 32 columns a store
// instruction writes fall in different banks).
constexpr int kEpiColBytes = 128 * 4 + 16;
constexpr int kEpiWaveBytes = 64 * kEpiColBytes;
constexpr int kSmemBytes = kRingBytes > 4 * kEpiWaveBytes ? kRingBytes : 4 * kEpiWaveBytes;

// The selection of every token of a wave's 128 x 128 score tile, stored to
// sel.  acc[mi][ni][e] is the score of token wm*128 + mi*32 + 8*(e/4) +
// 4*(lane/32) + e%4 and column ni*32 + lane%32 of the wave, i.e. entry k =
// (ni % NI)*32 + lane%32 of head ni / NI (NI = P / 32).  Blocks of 64
// columns of a head go through the wave's LDS area transposed, so that lane
// l holds tokens 2l and 2l+1 and scans their scores in index order: a later
// score replaces the best only when it is larger (the first maximum stays;
// -0 and +0 compare equal).  A token whose block holds a NaN (its sum is
// then NaN, as it is with +inf beside -inf) has the block scanned again by
// value keys, which put a NaN above every number (the first NaN winning);
// later blocks win over earlier ones only with a larger key.  The caller
// has finished every other use of smem.
template <int P>
__device__ __forceinline__ void select_store(const f32x16 (&acc)[4][4], const RouterArgs &a, int64_t m0,
                                             int64_t h0, int wm, int wn, int wave, int lane, char *smem)
{
    constexpr int HW = 128 / P;   // heads per wave
    constexpr int NI = P / 32;    // 32-column MFMA tiles per head
    const int K = a.K;
    char *const wb = smem + wave * kEpiWaveBytes;
    const int wr = (lane & 31) * kEpiColBytes + 16 * (lane >> 5);   // column lane%32, tokens 4 (lane/32) + ...
    const int rd = 8 * lane;                                        // tokens 2 lane, 2 lane + 1
#pragma unroll
    for (int hn = 0; hn < HW; ++hn) {
        const int64_t h = h0 + wn * HW + hn;
        int32_t best_key[2] = {0, 0};
        int best_k[2] = {0, 0};
#pragma unroll
        for (int ps = 0; ps < P / 64; ++ps) {
            // columns (2 ps + t2) * 32 + lane % 32 of the head, t2 = 0, 1
#pragma unroll
            for (int t2 = 0; t2 < 2; ++t2) {
                const int ni = hn * NI + 2 * ps + t2;
#pragma unroll
                for (int mi = 0; mi < 4; ++mi)
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        const float4 v = make_float4(acc[mi][ni][4 * q], acc[mi][ni][4 * q + 1], acc[mi][ni][4 * q + 2],
                                                     acc[mi][ni][4 * q + 3]);
                        *reinterpret_cast<float4 *>(wb + t2 * 32 * kEpiColBytes + wr + (mi * 32 + 8 * q) * 4) = v;
                    }
            }
            const int k0 = ps * 64;
            const int nk = min(K - k0, 64);   // >= 1: P = 128 only when K > 64
            float bv0 = -__builtin_inff(), bv1 = -__builtin_inff(), s0 = 0.f, s1 = 0.f;
            int bk0 = k0, bk1 = k0;
#pragma unroll 8
            for (int c = 0; c < nk; ++c) {
                const float2 v = *reinterpret_cast<const float2 *>(wb + c * kEpiColBytes + rd);
                const bool t0 = v.x > bv0, t1 = v.y > bv1;
                bv0 = t0 ? v.x : bv0;
                bk0 = t0 ? k0 + c : bk0;
                bv1 = t1 ? v.y : bv1;
                bk1 = t1 ? k0 + c : bk1;
                s0 += v.x;
                s1 += v.y;
            }
            int32_t key0 = value_key(bv0), key1 = value_key(bv1);
            if (__builtin_amdgcn_ballot_w64(s0 != s0 || s1 != s1) != 0) {
                int32_t q0 = kNoValue, q1 = kNoValue;
                for (int c = 0; c < nk; ++c) {
                    const float2 v = *reinterpret_cast<const float2 *>(wb + c * kEpiColBytes + rd);
                    const int32_t v0 = value_key(v.x), v1 = value_key(v.y);
                    bk0 = v0 > q0 ? k0 + c : bk0;
                    q0 = v0 > q0 ? v0 : q0;
                    bk1 = v1 > q1 ? k0 + c : bk1;
                    q1 = v1 > q1 ? v1 : q1;
                }
                key0 = q0;
                key1 = q1;
            }
            if (ps == 0 || key0 > best_key[0]) {
                best_key[0] = key0;
                best_k[0] = bk0;
            }
            if (ps == 0 || key1 > best_key[1]) {
                best_key[1] = key1;
                best_k[1] = bk1;
            }
        }
        if (h < a.H) {
#pragma unroll
            for (int r = 0; r < 2; ++r) {
                const int64_t m = m0 + wm * 128 + 2 * lane + r;
                if (m < a.M) {
                    const int64_t b = m / a.L, t = m - b * a.L;
                    a.sel[(b * a.H + h) * a.L + t] = (int16_t)best_k[r];
                }
            }
        }
    }
}

// Weights [H][K][D].  P: padded score columns per head (64 or 128); a
// wave's 128 columns hold 128 / P heads.
template <int P, int BK>
__global__ void __launch_bounds__(kRThreads, 1) router_lds_kernel(RouterArgs a)
{
    using SG = PairStage<BK>;
    constexpr int kRK = SG::kRK, kRowBytes = SG::kRowBytes, kChunks = SG::kChunks,
                  kRowsPerLoad = SG::kRowsPerLoad, kABytes = SG::kABytes, kStageBytes = SG::kStageBytes,
                  kRStages = SG::kRStages, kALoads = SG::kALoads, kBLoads = SG::kBLoads,
                  kLoadsPerStage = SG::kLoadsPerStage;
    __shared__ __attribute__((aligned(1024))) char smem[kSmemBytes];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);

    // Tile of this workgroup.  Consecutive workgroups go to different XCDs;
    // the mapping gives each XCD a contiguous run of tiles, so the column
    // tiles of one token tile (which read the same U rows) share that XCD's
    // L2.
    const uint32_t total = a.m_tiles * a.n_tiles, per = total / 8;
    const uint32_t bx = blockIdx.x;
    const uint32_t tile = (bx < per * 8) ? (bx % 8) * per + bx / 8 : bx;
    const uint32_t mt = tile / a.n_tiles, nt = tile % a.n_tiles;
    const int64_t m0 = (int64_t)mt * kRM;
    const int64_t h0 = (int64_t)nt * (kRN / P);
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
        asrc[j] = a.u + (m < a.M ? m : 0) * (int64_t)D + chunk_pos<kChunks>(r, lane % kChunks) * 8;
    }
    const uint16_t *bsrc[kBLoads];
#pragma unroll
    for (int j = 0; j < kBLoads; ++j) {
        const int col = kRowsPerLoad * (wave * kBLoads + j) + lane / kChunks;
        const int64_t h = h0 + col / P;
        const int k = col % P;
        bsrc[j] = a.w + ((h < a.H && k < K) ? (h * K + k) : 0) * (int64_t)D + chunk_pos<kChunks>(col, lane % kChunks) * 8;
    }
    // The loads are written in asm so that the compiler does not see them
    // as stores to LDS: it would otherwise make every fragment read wait
    // for all of them (it cannot tell the stages apart).  They write no
    // registers; the stage waits below are explicit.  M0 carries the LDS
    // address as an input operand.
    auto dma = [](const uint16_t *src, uint32_t lds) {
        asm volatile("global_load_lds_dwordx4 %0, off" : : "v"(src), "{m0}"(lds) : "memory");
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

    // This wave: tokens wm*128 .. +128 of the tile, columns wn*128 .. +128.
    const int wm = wave >> 1, wn = wave & 1;
    f32x16 acc[4][4];
#pragma unroll
    for (int mi = 0; mi < 4; ++mi)
#pragma unroll
        for (int ni = 0; ni < 4; ++ni)
#pragma unroll
            for (int e = 0; e < 16; ++e)
                acc[mi][ni][e] = 0.f;

    // Fragments: row (lane % 32) of a 32-row block, features 16 ks + 8 (lane
    // / 32).  Blocks start at multiples of 32 rows, so the swizzled offset of
    // the lane inside a block depends on the lane and ks only.
    constexpr int KS = kRK / 16;   // 16-feature MFMA steps per stage
    uint32_t lane_off[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
        lane_off[ks] = (uint32_t)((lane & 31) * kRowBytes + chunk_pos<kChunks>(lane & 31, ks * 2 + (lane >> 5)) * 16);
    bf16x8 af[2][4], bf[2][4];
    auto read_frags = [&](int buf, const char *base, int ks) {
        const char *ab = base + wm * 128 * kRowBytes + lane_off[ks];
        const char *bb = base + kABytes + wn * 128 * kRowBytes + lane_off[ks];
#pragma unroll
        for (int mi = 0; mi < 4; ++mi)
            af[buf][mi] = *reinterpret_cast<const bf16x8 *>(ab + mi * 32 * kRowBytes);
#pragma unroll
        for (int ni = 0; ni < 4; ++ni)
            bf[buf][ni] = *reinterpret_cast<const bf16x8 *>(bb + ni * 32 * kRowBytes);
    };
    auto mfmas = [&](int buf) {
#pragma unroll
        for (int mi = 0; mi < 4; ++mi)
#pragma unroll
            for (int ni = 0; ni < 4; ++ni)
                acc[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[buf][mi], bf[buf][ni], acc[mi][ni], 0, 0, 0);
    };
    // One MFMA, then one LDS read, eight times, then the other eight MFMAs.
    auto interleave_reads = []() {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // MFMA
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);   // LDS read
        }
        __builtin_amdgcn_sched_group_barrier(0x008, 8, 0);
        __builtin_amdgcn_sched_barrier(0);
    };
    // The own loads of stage s have landed once at most `ahead` younger
    // stages' loads are still in flight.
    auto wait_stage = [&](int ahead) {
        if (ahead >= 3)
            wait_vm<kLoadsPerStage * 3>();
        else if (ahead == 2)
            wait_vm<kLoadsPerStage * 2>();
        else if (ahead == 1)
            wait_vm<kLoadsPerStage>();
        else
            wait_vm<0>();
    };

    // Software pipeline over 16-feature steps g = s * KS + ks: the fragments
    // of step g + 1 are read from LDS while the MFMAs of step g run.  Ring of
    // kRStages stages, all in flight: in the last step of stage s each wave
    // has finished its reads of stage s (its fragments are in registers),
    // waits for its own loads of stage s + 1, and the barrier makes every
    // wave's rows of s + 1 visible and frees the buffer of stage s, which the
    // loads of stage s + kRStages then refill.
    const int stages = D / kRK;
    char *const ring = smem;
#pragma unroll
    for (int p = 0; p < kRStages; ++p)
        if (p < stages)
            issue(ring + p * kStageBytes, p * kRK);
    wait_stage(min(stages - 1, kRStages - 1));
    __builtin_amdgcn_s_barrier();
    lds_order();
    read_frags(0, ring, 0);
    // Every stage but the last hands over to the next one in its last step;
    // the last stage is peeled off, so the loop body has one count of LDS
    // operations in flight on every path (the compiler's waits then let the
    // next fragments stay in flight under the MFMAs).
    for (int s = 0; s + 1 < stages; ++s) {
        const char *cur = ring + (s % kRStages) * kStageBytes;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            const int buf = ks & 1;   // KS is even: step parity
            if (ks + 1 < KS) {
                read_frags(buf ^ 1, cur, ks + 1);
            } else {
                // this wave's reads of stage s are done (its fragments of
                // this step are waited for here), then stage s + 1
                __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0)
                wait_stage(min(stages - 2 - s, kRStages - 2));   // issued so far: stages up to s + kRStages - 1
                __builtin_amdgcn_s_barrier();
                lds_order();   // no LDS access moves across the barrier
                if (s + kRStages < stages)
                    issue(ring + (s % kRStages) * kStageBytes, (s + kRStages) * kRK);
                read_frags(buf ^ 1, ring + ((s + 1) % kRStages) * kStageBytes, 0);
            }
            // The next fragments' reads go out between this step's MFMAs
            // (clustered, they would leave the matrix core idle while they
            // issue).
            mfmas(buf);
            interleave_reads();
        }
    }
    {
        const char *cur = ring + ((stages - 1) % kRStages) * kStageBytes;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            if (ks + 1 < KS)
                read_frags((ks & 1) ^ 1, cur, ks + 1);
            mfmas(ks & 1);
            interleave_reads();
        }
    }
    // Every wave is past its last fragment read before the epilogue reuses
    // the ring.
    __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0)
    __builtin_amdgcn_s_barrier();
    lds_order();
    select_store<P>(acc, a, m0, h0, wm, wn, wave, lane, smem);
}

// Packed weights [H][D/8][P][8].  P: score columns per head (64 or 128); a
// wave's 128 columns hold 128 / P heads.
template <int P, int BK>
__global__ void __launch_bounds__(kRThreads, 1) router_wreg_kernel(RouterArgs a)
{
    using SG = TokenStage<BK>;
    constexpr int kRK = SG::kRK, kRowBytes = SG::kRowBytes, kChunks = SG::kChunks,
                  kRowsPerLoad = SG::kRowsPerLoad, kStageBytes = SG::kStageBytes, kRStages = SG::kRStages,
                  kALoads = SG::kALoads;
    __shared__ __attribute__((aligned(1024))) char smem[kSmemBytes];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);

    // Tile of this workgroup.  Consecutive workgroups go to different XCDs;
    // the mapping gives each XCD a contiguous run of tiles, so the column
    // tiles of one token tile (which read the same U rows) share that XCD's
    // L2.
    const uint32_t total = a.m_tiles * a.n_tiles, per = total / 8;
    const uint32_t bx = blockIdx.x;
    const uint32_t tile = (bx < per * 8) ? (bx % 8) * per + bx / 8 : bx;
    const uint32_t mt = tile / a.n_tiles, nt = tile % a.n_tiles;
    const int64_t m0 = (int64_t)mt * kWM;
    const int64_t h0 = (int64_t)nt * (kWN / P);
    const int D = a.D;

    // Token rows go straight from global memory into LDS (global_load_lds):
    // load j of this wave fills the kRowsPerLoad rows from R g on (g = wave
    // * loads + j, R = kRowsPerLoad), lane i writing the 16-byte slot i, i.e.
    // row R g + i / kChunks at position i % kChunks, which holds the chunk
    // chunk_pos(row, i % kChunks) (the swizzle is its own inverse).  Rows
    // past the token count read row 0 instead: their results are never used.
    const uint16_t *asrc[kALoads];
#pragma unroll
    for (int j = 0; j < kALoads; ++j) {
        const int r = kRowsPerLoad * (wave * kALoads + j) + lane / kChunks;
        const int64_t m = m0 + r;
        asrc[j] = a.u + (m < a.M ? m : 0) * (int64_t)D + chunk_pos<kChunks>(r, lane % kChunks) * 8;
    }
    // The loads are written in asm so that the compiler does not see them
    // as stores to LDS: it would otherwise make every fragment read wait
    // for all of them (it cannot tell the stages apart).  They write no
    // registers; the stage waits below are explicit.  M0 carries the LDS
    // address as an input operand.
    auto dma = [](const uint16_t *src, uint32_t lds) {
        asm volatile("global_load_lds_dwordx4 %0, off" : : "v"(src), "{m0}"(lds) : "memory");
    };
    // Stage s of the token rows into ring slot s % kRStages.  Stages past
    // the last one reload the last one into a slot nobody reads any more, so
    // every hand-over sees the same count of loads in flight.
    const int stages = D / kRK;
    auto issue_a = [&](int s) {
        char *buf = smem + (s % kRStages) * kStageBytes;
        const int k0 = min(s, stages - 1) * kRK;
        const uint32_t base = __builtin_amdgcn_readfirstlane(lds_addr(buf));
#pragma unroll
        for (int j = 0; j < kALoads; ++j)
            dma(asrc[j] + k0, base + (uint32_t)((wave * kALoads + j) * 1024));
    };

    // This wave: the tile's 128 tokens (all four waves), columns wn*128 ..
    // +128.
    const int wm = 0, wn = wave;
    f32x16 acc[4][4];
#pragma unroll
    for (int mi = 0; mi < 4; ++mi)
#pragma unroll
        for (int ni = 0; ni < 4; ++ni)
#pragma unroll
            for (int e = 0; e < 16; ++e)
                acc[mi][ni][e] = 0.f;

    // Fragments of 16-feature step g: row (lane % 32) of a 32-row block,
    // features 16 g + 8 (lane / 32) .. + 8.  Token fragments come from the
    // LDS stage; blocks start at multiples of 32 rows, so the swizzled
    // offset of the lane inside a block depends on the lane and the step
    // within the stage only.
    constexpr int KS = kRK / 16;   // 16-feature steps per stage
    uint32_t lane_off[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
        lane_off[ks] = (uint32_t)((lane & 31) * kRowBytes + chunk_pos<kChunks>(lane & 31, ks * 2 + (lane >> 5)) * 16);
    bf16x8 af[2][4];
    auto read_a = [&](int buf, int g) {
        const char *ab = smem + ((g / KS) % kRStages) * kStageBytes + wm * 128 * kRowBytes + lane_off[g % KS];
#pragma unroll
        for (int mi = 0; mi < 4; ++mi)
            af[buf][mi] = *reinterpret_cast<const bf16x8 *>(ab + mi * 32 * kRowBytes);
    };
    // Weight fragments go from global memory straight into a ring of kNB
    // register slots, kNB - 1 steps ahead of their MFMAs: 4 x 16 bytes per
    // lane per step, one 16-byte load per 32-column block; the four waves
    // load disjoint columns.  Padding columns and heads past H read row 0
    // (their scores are never used); steps past the last one reload the last
    // one, so the loads issued never depend on the step count.
    constexpr int kNB = 8;
    const int G = D / 16;
    // One buffer resource over the weights; lane offsets per 32-column
    // block (column k of head h at ((h * D/8 + lane / 32) * P + k) * 16
    // bytes), the step's offset in a scalar register (no address arithmetic
    // per load).  The host keeps the weights below 4 GB.
    uint32_t boff[4];
    const __amdgpu_buffer_rsrc_t wr = make_rsrc(a.w, (uint64_t)a.H * (uint64_t)P * (uint64_t)D * 2u);
#pragma unroll
    for (int ni = 0; ni < 4; ++ni) {
        const int col = wn * 128 + ni * 32 + (lane & 31);
        const int64_t h = h0 + col / P;
        const int k = col % P;
        boff[ni] = (uint32_t)((((h < a.H ? h : 0) * (int64_t)(D / 8) + (lane >> 5)) * P + k) * 16);
    }
    constexpr uint32_t kStepBytes = 2u * P * 16u;
    bf16x8 bq[kNB][4];
    auto issue_b = [&](int slot, int g) {
        const uint32_t soff = (uint32_t)min(g, G - 1) * kStepBytes;
#pragma unroll
        for (int ni = 0; ni < 4; ++ni) {
            const auto v = __builtin_amdgcn_raw_buffer_load_b128(wr, boff[ni], soff, 0);
            __builtin_memcpy(&bq[slot][ni], &v, 16);
        }
    };
    auto mfmas = [&](int buf, int slot) {
#pragma unroll
        for (int mi = 0; mi < 4; ++mi)
#pragma unroll
            for (int ni = 0; ni < 4; ++ni)
                acc[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[buf][mi], bq[slot][ni], acc[mi][ni], 0, 0, 0);
    };

    // The token ring holds two groups of 128 features (kNB steps, HS =
    // kGroupStages stages each); the waves hand over once per group.
    // Vector-memory loads of this wave, in issue order: groups 0 and 1 of
    // the token stages, weight steps 0 .. kNB - 2, then per step g: in the
    // last step of group q (the hand-over) the token stages of group q + 2,
    // then the weights of step g + kNB - 1.  At the hand-over of group q,
    // group q + 1 has landed once at most 4 kNB loads are in flight: the
    // weights of kNB steps were issued after it (q >= 1; for q = 0, 2 kNB - 2
    // steps' weights).  The compiler's own waits before each step's MFMAs
    // count the weight loads only, which makes them stricter than needed,
    // never laxer.
    constexpr int HS = SG::kGroupStages;
    static_assert(HS * KS == kNB, "a group of stages is a group of weight slots");
    constexpr int kHandWait = 4 * kNB;
    constexpr int kFirstWait = HS * kALoads + 4 * (kNB - 1);   // group 0 landed
    static_assert(kFirstWait < 64 && kHandWait < 64, "vmcnt range");
    // (The scheduling barriers keep the loads in this order: the loop's
    // waits hold on every path into it only if each slot's loads are as old
    // on entry as in the steady state.)
#pragma unroll
    for (int s = 0; s < kRStages; ++s)
        issue_a(s);
#pragma unroll
    for (int g = 0; g + 1 < kNB; ++g) {
        __builtin_amdgcn_sched_barrier(0);
        issue_b(g, g);
    }
    __builtin_amdgcn_sched_barrier(0);
    wait_vm<kFirstWait>();
    __builtin_amdgcn_s_barrier();
    lds_order();
    read_a(0, 0);

    // Steps g0 .. g0 + kNB - 1 per group, so that every weight slot has a
    // fixed register home.  Per step: the weights of step g + kNB - 1 go out,
    // the token fragments of step g + 1 are read from LDS (after the
    // hand-over when g + 1 starts a group), then the MFMAs of step g run.
    // Only the MFMAs of steps past the last one are skipped (in the one
    // partial group at the end): every load, read and hand-over is issued on
    // every path, at clamped addresses, so the compiler's waits count the
    // loads exactly and never fall back to waiting for all of them.
    auto group = [&](int g0, auto tailc) {
        constexpr bool TAIL = decltype(tailc)::value;
#pragma unroll
        for (int j = 0; j < kNB; ++j) {
            const int g = g0 + j;
            if (j == kNB - 1) {
                // Hand-over from group q = g0 / kNB to group q + 1: this
                // wave's reads of group q are done, group q + 1 has landed
                // (every wave's rows of it, after the barrier), and the
                // slots of group q are refilled with group q + 2.
                __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0)
                wait_vm<kHandWait>();
                __builtin_amdgcn_s_barrier();
                lds_order();   // no LDS access moves across the barrier
#pragma unroll
                for (int t = 0; t < HS; ++t)
                    issue_a(g0 / KS + t + kRStages);
            }
            issue_b((j + kNB - 1) % kNB, g + kNB - 1);
            read_a((j + 1) & 1, g + 1);
            if (!TAIL || g < G)
                mfmas(j & 1, j);
            // The loads and fragment reads go out between the MFMAs (one
            // wave per SIMD issues everything: clustered, they would leave
            // the matrix core idle while they issue).
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // MFMA
                __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);   // vector memory read
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);   // LDS read
            }
            __builtin_amdgcn_sched_group_barrier(0x008, 8, 0);
            __builtin_amdgcn_sched_barrier(0);
        }
    };
    const int g_full = G & ~(kNB - 1);
    for (int g0 = 0; g0 < g_full; g0 += kNB)
        group(g0, std::false_type{});
    if (g_full < G)
        group(g_full, std::true_type{});
    // Every load has landed before the epilogue: the weight slots loaded
    // past the last step are consumed here (so no load is dropped or moved,
    // and the counts above hold), and the token stages past the last one
    // finish writing LDS before the workgroup ends.
#pragma unroll
    for (int j = 0; j < kNB; ++j)
#pragma unroll
        for (int ni = 0; ni < 4; ++ni)
            asm volatile("" : : "v"(bq[j][ni]));
    wait_vm<0>();
    // Every wave's loads into the ring have landed and every wave is past
    // its last fragment read before the epilogue reuses the ring.
    __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0)
    __builtin_amdgcn_s_barrier();
    lds_order();
    select_store<P>(acc, a, m0, h0, wm, wn, wave, lane, smem);
}

// The packed weight layout: wp[h][d/8][k][d%8] = w[h][k][d] for k < K, zero
// for K <= k < P.  One thread per 16-byte chunk of the output.
__global__ void __launch_bounds__(256) pack_kernel(const uint4 *__restrict__ w, uint4 *__restrict__ wp, int64_t H,
                                                   int K, int D, int P)
{
    const int64_t n = H * (int64_t)(D / 8) * P;
    for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x) {
        const int k = (int)(i % P);
        const int64_t r = i / P;
        const int d8 = (int)(r % (D / 8));
        const int64_t h = r / (D / 8);
        wp[i] = k < K ? w[(h * K + k) * (D / 8) + d8] : make_uint4(0u, 0u, 0u, 0u);
    }
}

}  // namespace
}  // namespace pdssm

using namespace pdssm;

extern "C" int pdssm_router_select(const void *u, const void *w, int16_t *sel_out, int64_t B, int64_t L,
                                   int64_t H, int32_t K, int32_t D, uint32_t flags, hipStream_t stream)
{
    if (B < 0 || L < 0 || H < 0 || K < 1 || K > 128 || D < 32 || (D % 32) != 0)
        return PDSSM_ERR_DIM;
    const int P = K <= 64 ? 64 : 128;
    const double tokens = (double)B * (double)L;
    const double m_tiles = (tokens + kRM - 1) / kRM, n_tiles = (double)((H * P + kRN - 1) / kRN);
    if (tokens > 2.0e9 || m_tiles * n_tiles > 2.0e9 || (double)H * K * D > 4.0e18)
        return PDSSM_ERR_DIM;
    if ((flags & ~PDSSM_ROUTER_W_PACKED) != 0)
        return PDSSM_ERR_FLAGS;
    const bool packed = (flags & PDSSM_ROUTER_W_PACKED) != 0;
    // Packed weights are addressed by 32-bit byte offsets.
    if (packed && (double)H * P * D * 2.0 > 4294967295.0)
        return PDSSM_ERR_DIM;
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
    a.n_tiles = (uint32_t)((H * P + kRN - 1) / kRN);
    dim3 grid(a.m_tiles * a.n_tiles), block(kRThreads);
    const bool deep = (D % 64) == 0;
    if (packed) {
        // tiles of 128 tokens x 512 columns
        a.m_tiles = (uint32_t)((a.M + kWM - 1) / kWM);
        a.n_tiles = (uint32_t)((H * P + kWN - 1) / kWN);
        grid = dim3(a.m_tiles * a.n_tiles);
        if (P == 64 && deep)
            router_wreg_kernel<64, 64><<<grid, block, 0, stream>>>(a);
        else if (P == 64)
            router_wreg_kernel<64, 32><<<grid, block, 0, stream>>>(a);
        else if (deep)
            router_wreg_kernel<128, 64><<<grid, block, 0, stream>>>(a);
        else
            router_wreg_kernel<128, 32><<<grid, block, 0, stream>>>(a);
    } else {
        if (P == 64 && deep)
            router_lds_kernel<64, 64><<<grid, block, 0, stream>>>(a);
        else if (P == 64)
            router_lds_kernel<64, 32><<<grid, block, 0, stream>>>(a);
        else if (deep)
            router_lds_kernel<128, 64><<<grid, block, 0, stream>>>(a);
        else
            router_lds_kernel<128, 32><<<grid, block, 0, stream>>>(a);
    }
    return hip_status(hipGetLastError());
}

extern "C" int pdssm_router_pack_weights(const void *w, void *w_packed, int64_t H, int32_t K, int32_t D,
                                         hipStream_t stream)
{
    if (H < 0 || K < 1 || K > 128 || D < 32 || (D % 32) != 0)
        return PDSSM_ERR_DIM;
    const int P = K <= 64 ? 64 : 128;
    if ((double)H * P * D * 2.0 > 4294967295.0)
        return PDSSM_ERR_DIM;
    if (H == 0)
        return PDSSM_OK;
    if (!w || !w_packed)
        return PDSSM_ERR_NULL;
    if (!aligned16(w) || !aligned16(w_packed))
        return PDSSM_ERR_ALIGN;
    const int64_t n = H * (int64_t)(D / 8) * P;
    const unsigned blocks = (unsigned)((n + 255) / 256 < 8192 ? (n + 255) / 256 : 8192);
    pack_kernel<<<blocks, 256, 0, stream>>>(static_cast<const uint4 *>(w), static_cast<uint4 *>(w_packed), H, K, D, P);
    return hip_status(hipGetLastError());
}
