// pdssm_host.h -- host-side checks shared by the library's source files.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace pdssm {

// True when p is 16-byte aligned.
__attribute__((visibility("hidden"))) bool aligned16(const void *p);
// PDSSM_OK, or PDSSM_ERR_DIM when the sizes are out of the supported range.
__attribute__((visibility("hidden"))) int check_dims(int64_t B, int64_t H, int64_t L, int32_t N, int32_t K);
// PDSSM_OK for hipSuccess, else PDSSM_ERR_HIP (the HIP text goes to pdssm_strerror).
__attribute__((visibility("hidden"))) int hip_status(hipError_t e);
struct Header;
// Per-call preparation of a workspace on stream: a new epoch and a zero
// ticket counter in hdr (on first use, or when the epoch wraps, the n16
// 16-byte words of records at recs are cleared first), and the scatter
// entry table tab[h][k][0..NP) of every dictionary entry.
__attribute__((visibility("hidden"))) int launch_prep(Header *hdr, void *recs, int64_t n16, const int32_t *dict,
                                                      uint16_t *tab, int64_t entries, int N, int NP,
                                                      hipStream_t stream);
// dst[0..n) = src[0..n) (fp32), or zeros when src is NULL, on stream; nothing when n <= 0.
__attribute__((visibility("hidden"))) int launch_state_fill(const void *src, void *dst, int64_t n,
                                                            hipStream_t stream);

}  // namespace pdssm
