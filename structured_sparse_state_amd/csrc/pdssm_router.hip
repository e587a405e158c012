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

constexpr int kRM = 256;                  // tokens per workgroup tile
constexpr int kRH = 2;                    // heads per workgroup tile
constexpr int kRN = kRH * 64;             // padded score columns per tile
constexpr int kRK = 32;                   // features per LDS stage
constexpr int kRowBytes = kRK * 2;        // 64: four 16-byte chunks per row
constexpr int kABytes = kRM * kRowBytes;  // 16 KB of token rows per stage
constexpr int kBBytes = kRN * kRowBytes;  // 8 KB of weight rows per stage
constexpr int kRThreads = 256;
constexpr int kALoads = kRM / 16 / 4;     // direct-to-LDS loads per wave per stage (16 rows each)
constexpr int kBLoads = kRN / 16 / 4;
constexpr int kLoadsPerStage = kALoads + kBLoads;

struct RouterArgs {
    const uint16_t *u;   // [M][D] bf16
    const uint16_t *w;   // [H][K][D] bf16
    int16_t *sel;        // [B][H][L]
    int64_t M, L, H;
    int K, D;
    uint32_t m_tiles, h_tiles;
};

// Position of 16-byte chunk c of row r inside the row: the chunks of rows two
// apart are rotated, so the fragment reads of eight consecutive rows (one
// LDS cycle of ds_read_b128) land on eight different 16-byte bank groups.
__device__ __forceinline__ int chunk_pos(int r, int c) { return c ^ ((r >> 1) & 3); }

// s_waitcnt with only the vector-memory count constrained (gfx9 encoding).
template <int N>
__device__ __forceinline__ void wait_vm()
{
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Three LDS stages, each its own variable so that the compiler can tell which
// stage a fragment read touches and waits only for that stage's loads.
__shared__ __attribute__((aligned(1024))) char s_stage0[kABytes + kBBytes];
__shared__ __attribute__((aligned(1024))) char s_stage1[kABytes + kBBytes];
__shared__ __attribute__((aligned(1024))) char s_stage2[kABytes + kBBytes];

template <int S>
__device__ __forceinline__ char *stage_buf()
{
    if constexpr (S == 0)
        return s_stage0;
    else if constexpr (S == 1)
        return s_stage1;
    else
        return s_stage2;
}

__global__ void __launch_bounds__(kRThreads, 2) router_kernel(RouterArgs a)
{
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

    // Direct-to-LDS loads: load j of this wave fills rows 16 g .. 16 g + 15 of
    // the stage (g = wave * loads + j), lane i writing the 16-byte slot i,
    // i.e. row 16 g + i / 4 at position i % 4, which holds the chunk
    // chunk_pos(row, i % 4) (the swizzle is its own inverse).  Rows past the
    // token count or padding score columns read row 0 instead: their results
    // are never used.
    const uint16_t *asrc[kALoads];
#pragma unroll
    for (int j = 0; j < kALoads; ++j) {
        const int r = 16 * (wave * kALoads + j) + (lane >> 2);
        const int64_t m = m0 + r;
        asrc[j] = a.u + (m < a.M ? m : 0) * (int64_t)D + chunk_pos(r, lane & 3) * 8;
    }
    const uint16_t *bsrc[kBLoads];
#pragma unroll
    for (int j = 0; j < kBLoads; ++j) {
        const int col = 16 * (wave * kBLoads + j) + (lane >> 2);
        const int64_t h = h0 + col / 64;
        const int k = col % 64;
        bsrc[j] = a.w + ((h < a.H && k < K) ? (h * K + k) : 0) * (int64_t)D + chunk_pos(col, lane & 3) * 8;
    }
    auto issue = [&](char *buf, int k0) {
        typedef __attribute__((address_space(3))) void lds_void;
#pragma unroll
        for (int j = 0; j < kALoads; ++j)
            __builtin_amdgcn_global_load_lds(asrc[j] + k0, (lds_void *)(buf + (wave * kALoads + j) * 1024), 16, 0, 0);
#pragma unroll
        for (int j = 0; j < kBLoads; ++j)
            __builtin_amdgcn_global_load_lds(bsrc[j] + k0, (lds_void *)(buf + kABytes + (wave * kBLoads + j) * 1024),
                                             16, 0, 0);
    };

    // This wave: tokens wm*128 .. +128 of the tile, head wn of the tile.
    const int wm = wave >> 1, wn = wave & 1;
    f32x16 acc[4][2];
#pragma unroll
    for (int mi = 0; mi < 4; ++mi)
#pragma unroll
        for (int ni = 0; ni < 2; ++ni)
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
    // The six fragment reads of a k-step are one asm block that waits for
    // them: written as C++, the compiler would make every LDS read wait for
    // all global-to-LDS loads in flight (it cannot tell the stages apart),
    // which would serialise the ring.
    auto compute = [&](const char *base) {
        const uint32_t ab = lds_addr(base) + (uint32_t)(wm * 128 * kRowBytes);
        const uint32_t bb = lds_addr(base) + (uint32_t)(kABytes + wn * 64 * kRowBytes);
#pragma unroll
        for (int ks = 0; ks < kRK / 16; ++ks) {
            typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
            u32x4 f0, f1, f2, f3, g0, g1;
            asm volatile(
                "ds_read_b128 %0, %6\n\t"
                "ds_read_b128 %1, %6 offset:2048\n\t"
                "ds_read_b128 %2, %6 offset:4096\n\t"
                "ds_read_b128 %3, %6 offset:6144\n\t"
                "ds_read_b128 %4, %7\n\t"
                "ds_read_b128 %5, %7 offset:2048\n\t"
                "s_waitcnt lgkmcnt(0)"
                : "=v"(f0), "=v"(f1), "=v"(f2), "=v"(f3), "=v"(g0), "=v"(g1)
                : "v"(ab + lane_off[ks]), "v"(bb + lane_off[ks])
                : "memory");
            bf16x8 af[4], bf[2];
            __builtin_memcpy(&af[0], &f0, 16);
            __builtin_memcpy(&af[1], &f1, 16);
            __builtin_memcpy(&af[2], &f2, 16);
            __builtin_memcpy(&af[3], &f3, 16);
            __builtin_memcpy(&bf[0], &g0, 16);
            __builtin_memcpy(&bf[1], &g1, 16);
#pragma unroll
            for (int mi = 0; mi < 4; ++mi)
#pragma unroll
                for (int ni = 0; ni < 2; ++ni)
                    acc[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[mi], bf[ni], acc[mi][ni], 0, 0, 0);
        }
    };

    // Three-stage ring: stage s is consumed while s + 1 and s + 2 load.
    // Before consuming s each wave waits for its own loads of s (the loads of
    // the two younger stages may stay in flight), then the barrier makes
    // every wave's rows of s visible and frees the buffer of s - 1, which
    // the loads of s + 2 then refill.
    const int stages = D / kRK;
    issue(stage_buf<0>(), 0);
    if (stages > 1)
        issue(stage_buf<1>(), kRK);
    auto step = [&](auto S, int s) {
        constexpr int cur = decltype(S)::value;
        constexpr int nxt = (cur + 2) % 3;
        if (s + 1 < stages)
            wait_vm<kLoadsPerStage>();
        else
            wait_vm<0>();
        __builtin_amdgcn_s_barrier();
        if (s + 2 < stages)
            issue(stage_buf<nxt>(), (s + 2) * kRK);
        compute(stage_buf<cur>());
    };
    for (int s = 0; s < stages; s += 3) {
        step(std::integral_constant<int, 0>(), s);
        if (s + 1 < stages)
            step(std::integral_constant<int, 1>(), s + 1);
        if (s + 2 < stages)
            step(std::integral_constant<int, 2>(), s + 2);
    }

    // Argmax per token over the head's K scores.  acc[mi][ni][e] is the
    // score of token wm*128 + mi*32 + 8*(e/4) + 4*(lane/32) + e%4 and entry
    // k = ni*32 + lane%32: compare the lane's two entries, then reduce over
    // the 32 lanes of each half-wave (ties to the lower index).
    const int64_t h = h0 + wn;
    int keep[2] = {0, 0};
#pragma unroll
    for (int mi = 0; mi < 4; ++mi) {
#pragma unroll
        for (int e = 0; e < 16; ++e) {
            const int k0 = lane & 31, k1 = 32 + (lane & 31);
            float bv = __uint_as_float(0xFF800000u);   // -inf, beaten by any score
            int bk = 64;
            if (k0 < K) {
                bv = acc[mi][0][e];
                bk = k0;
            }
            if (k1 < K && better(acc[mi][1][e], k1, bv, bk)) {
                bv = acc[mi][1][e];
                bk = k1;
            }
#pragma unroll
            for (int x = 1; x < 32; x <<= 1) {
                const float ov = __shfl_xor(bv, x, 64);
                const int ok = __shfl_xor(bk, x, 64);
                if (better(ov, ok, bv, bk)) {
                    bv = ov;
                    bk = ok;
                }
            }
            const int c = mi * 16 + e;   // lane c % 32 of each half keeps combination c
            if ((lane & 31) == (c & 31))
                keep[c >> 5] = bk;
        }
    }
    if (h < a.H) {
#pragma unroll
        for (int r = 0; r < 2; ++r) {
            const int c = r * 32 + (lane & 31), mi = c >> 4, e = c & 15;
            const int64_t m = m0 + wm * 128 + mi * 32 + 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3);
            if (m < a.M) {
                const int64_t b = m / a.L, t = m - b * a.L;
                a.sel[(b * a.H + h) * a.L + t] = (int16_t)keep[r];
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
    if (!u || !w || !sel_out)
        return PDSSM_ERR_NULL;
    if (B < 1 || L < 1 || H < 1 || K < 1 || K > 64 || D < kRK || (D % kRK) != 0)
        return PDSSM_ERR_DIM;
    const double tokens = (double)B * (double)L;
    const double m_tiles = (tokens + kRM - 1) / kRM, h_tiles = (double)((H + kRH - 1) / kRH);
    if (tokens > 2.0e9 || m_tiles * h_tiles > 2.0e9 || (double)H * K * D > 4.0e18)
        return PDSSM_ERR_DIM;
    if (flags != 0)
        return PDSSM_ERR_FLAGS;
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
