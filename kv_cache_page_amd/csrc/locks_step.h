// Launch arguments of the decode step's selection + attention kernel (host
// side, shared by its launcher and the C-ABI implementation).
#pragma once

#include "locks_device.h"

namespace locks {

// Row length in pages of a fused launch's score outputs (e per page and query,
// page maxima): MP rounded up to 32, so that each tile's outputs fill whole
// 128-byte lines of their own for any table width.
__host__ __device__ constexpr int step_row_pages(int MP) { return (MP + 31) / 32 * 32; }

struct StepLaunch {
  float* escore;        // per page and query e = 2^(s - m) (decode layout)
  float* pmax;          // per page m = max_g s (base 2)
  float2* zpart;        // per score tile and query, base-2 (max, sum)
  int ntiles;           // 128-page tiles (a fused launch with a score part sets its own)
  const int32_t* lens;
  const int32_t* budgets;
  const void* q;
  void* kpool;
  void* vpool;
  const int32_t* table;
  int64_t nb;
  int S, H, MP, KB, nsplit, slice, per_wg;
  int lag;              // 1: only the pages full before the current token are scored
  int rule;             // GQA merge rule of the selection keys (kMergeShare, ...)
  int hdiv;             // head divisor of the K/V and summary pools (score_head_div; 0 or 1: none)
  uint32_t* mbox;
  float* out;
  float* lse_out;
  int32_t* sel;
  int32_t* cnt;
  // fused score part: rank r in {4, 8, 16} scores the pages in the same
  // launch (summ, and knew / vnew for the append when no page build runs);
  // r = 0: the scores come from a separate score kernel
  int r;
  const void* summ;
  const void* knew;
  const void* vnew;
  CoopZero coop;
};

}  // namespace locks
