// LOCKS page-summary builds and the KV append (gfx950): the host-side entry
// of the build, and the append kernel.
//
// [N] = LOCKS reading notes (zhongzhuzhou.org 2026-07-29), §4.1 eq. 2-3 and
// §4.3 Algorithm 1. Every build, from the 8 pages a decode step completes to
// the 65536 pages of a 128K-token layer at the prefill boundary, runs the
// one-wave-per-page kernel of locks_build_page.hip: with its keys held in
// registers it fits 16 waves per compute unit, and on whole layers it builds
// more pages per second than a form that shared a wave between 4 pages
// (30.7 against 22.8 M pages/s at r = 8).
#include "locks_build_common.h"

namespace locks {

// ---------------------------------------------------------------------------
// append: one token per sequence into the paged cache
// ---------------------------------------------------------------------------
__global__ void append_kernel(const uint16_t* __restrict__ knew, const uint16_t* __restrict__ vnew,
                              uint16_t* __restrict__ kpool, uint16_t* __restrict__ vpool,
                              int64_t num_blocks, const int32_t* __restrict__ table,
                              const int32_t* __restrict__ lens, int H, int MP) {
  const int s = blockIdx.x;
  const int len = lens[s];
  if (len < 1 || len > MP * kPage) return;
  const int pos = len - 1;
  const int blk = table[(int64_t)s * MP + pos / kPage];
  if (blk < 0 || blk >= num_blocks) return;
  for (int idx = threadIdx.x; idx < H * (kHeadDim / 8); idx += blockDim.x) {
    const int h = idx / (kHeadDim / 8), c = idx % (kHeadDim / 8);
    const int64_t src = ((int64_t)s * H + h) * kHeadDim + 8 * c;
    const int64_t dst = (((int64_t)blk * H + h) * kPage + pos % kPage) * kHeadDim + 8 * c;
    *reinterpret_cast<uint4*>(kpool + dst) = *reinterpret_cast<const uint4*>(knew + src);
    *reinterpret_cast<uint4*>(vpool + dst) = *reinterpret_cast<const uint4*>(vnew + src);
  }
}

hipError_t launch_build_page(int r, const void* kpool, int64_t nb, int H, const int32_t* ids, int n,
                             const int32_t* table, const int32_t* lens, int MP, void* summ,
                             const void* knew, const void* vnew, void* vpool, int bits,
                             hipStream_t st);

// knew/vnew (filled-page mode only, may be null): append the new token too.
hipError_t launch_build(int r, const void* kpool, int64_t nb, int H, const int32_t* ids, int n,
                        const int32_t* table, const int32_t* lens, int MP, void* summ,
                        const void* knew, const void* vnew, void* vpool, int bits, hipStream_t st) {
  if (bits != 2 && bits != 4 && bits != 8) return hipErrorInvalidValue;
  return launch_build_page(r, kpool, nb, H, ids, n, table, lens, MP, summ, knew, vnew, vpool, bits, st);
}

hipError_t launch_append(const void* knew, const void* vnew, void* kpool, void* vpool, int64_t nb,
                         const int32_t* table, const int32_t* lens, int S, int H, int MP,
                         hipStream_t st) {
  if (S == 0) return hipSuccess;
  hipLaunchKernelGGL(append_kernel, dim3(S), dim3(128), 0, st,
                     static_cast<const uint16_t*>(knew), static_cast<const uint16_t*>(vnew),
                     static_cast<uint16_t*>(kpool), static_cast<uint16_t*>(vpool), nb, table, lens,
                     H, MP);
  return hipGetLastError();
}

}  // namespace locks
