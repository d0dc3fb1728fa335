// LOCKS page scores on the matrix cores (gfx950), for ranks 4, 8 and 16: the
// score kernel (one 128-page tile of one (sequence, KV head) per 256-thread
// workgroup, one Z partial per tile) and its launcher. The tile itself, with
// the description of its stages, is in locks_score_tile.h.
#include "locks_score_tile.h"

namespace locks {

// TPW tiles per workgroup (4 waves each).
template <int R, int G, int TPW>
__global__ __launch_bounds__(256 * TPW) void score_mfma_kernel(
    const uint16_t* __restrict__ q, const uint8_t* __restrict__ summ,
    const int32_t* __restrict__ table, const int32_t* __restrict__ seq_lens,
    float* __restrict__ scores, int64_t num_blocks, int H, int MP,
    int flags, float2* __restrict__ zpart, const uint16_t* __restrict__ knew,
    const uint16_t* __restrict__ vnew, uint16_t* __restrict__ kpool,
    uint16_t* __restrict__ vpool, float* __restrict__ mxout, CoopZero coop) {
  const int s = blockIdx.z, h = blockIdx.x;
  zero_coop_mailbox(coop, (int64_t)s * H + h, blockIdx.y, gridDim.y);
  const int sub = (TPW == 1) ? 0 : (int)(threadIdx.x >> 8);
  const int tile = blockIdx.y * TPW + sub;
  const int tid = threadIdx.x & 255, wave = tid >> 6, lane = tid & 63;
  const int ntiles = (MP + kScorePagesPerWg - 1) / kScorePagesPerWg;
  float zm = -__builtin_inff(), zs = 0.f;
  if (tile < ntiles)
    score_tile<R, G>(q, summ, table, seq_lens, scores, num_blocks, H, MP, MP, flags,
                     knew, vnew, kpool, vpool, mxout, s, h, tile, wave, tid, zm, zs);
  if (zpart) {
    __shared__ float zred[TPW][4][4][2];
    if (lane < G) { zred[sub][wave][lane][0] = zm; zred[sub][wave][lane][1] = zs; }
    __syncthreads();
    if (tid < G && tile < ntiles) {
      float m = zred[sub][0][tid][0], t = zred[sub][0][tid][1];
      for (int w = 1; w < 4; ++w) lse2_merge(m, t, zred[sub][w][tid][0], zred[sub][w][tid][1]);
      zpart[(((int64_t)s * H + h) * ntiles + tile) * G + tid] = make_float2(m, t);
    }
  }
}

template <int R, int G>
static hipError_t launch_r_g(const uint16_t* q, const uint8_t* summ, const int32_t* table,
                             const int32_t* lens, float* scores, int64_t nb, int S, int H, int MP,
                             int flags, float2* zpart, const void* knew, const void* vnew,
                             void* kpool, void* vpool, float* mxout, CoopZero coop,
                             hipStream_t st) {
  constexpr int TPW = 1;
  const int ntiles = (MP + kScorePagesPerWg - 1) / kScorePagesPerWg;
  dim3 grid(H, (ntiles + TPW - 1) / TPW, S);  // heads first: 8 heads -> one XCD each
  hipLaunchKernelGGL((score_mfma_kernel<R, G, TPW>), grid, dim3(256 * TPW), 0, st, q, summ, table, lens,
                     scores, nb, H, MP, flags, zpart, static_cast<const uint16_t*>(knew),
                     static_cast<const uint16_t*>(vnew), static_cast<uint16_t*>(kpool),
                     static_cast<uint16_t*>(vpool), mxout, coop);
  return hipGetLastError();
}

bool score_mfma_supported(int r) { return r == 4 || r == 8 || r == 16; }

hipError_t launch_score_mfma(int r, int G, const void* q, const void* summ, const int32_t* table,
                             const int32_t* lens, float* scores, int64_t nb, int S, int H, int MP,
                             int flags, float2* zpart, const void* knew, const void* vnew,
                             void* kpool, void* vpool, float* mxout, CoopZero coop,
                             hipStream_t st) {
  const uint16_t* qq = static_cast<const uint16_t*>(q);
  const uint8_t* ss = static_cast<const uint8_t*>(summ);
#define LOCKS_ARGS qq, ss, table, lens, scores, nb, S, H, MP, flags, zpart, knew, vnew, kpool, vpool, mxout, coop, st
#define LOCKS_G(RR)                                  \
  switch (G) {                                       \
    case 1: return launch_r_g<RR, 1>(LOCKS_ARGS);    \
    case 2: return launch_r_g<RR, 2>(LOCKS_ARGS);    \
    case 4: return launch_r_g<RR, 4>(LOCKS_ARGS);    \
    default: return hipErrorInvalidValue;            \
  }
  switch (r) {
    case 4: LOCKS_G(4)
    case 8: LOCKS_G(8)
    case 16: LOCKS_G(16)
    default: return hipErrorInvalidValue;
  }
#undef LOCKS_G
#undef LOCKS_ARGS
}

}  // namespace locks
