// LOCKS page-summary build and KV append kernels (gfx950).
//
// [N] = LOCKS reading notes (zhongzhuzhou.org 2026-07-29), §4.1 eq. 2-3 and
// §4.3 Algorithm 1: centre the page's keys (mu, D = K - 1 mu^T), form the
// B x B Gram D D^T, eigendecompose it (descending), keep the top r
// components as basis V = D^T U_r Sigma_r^{-1} and coefficients C = U_r
// Sigma_r, then store an int4 basis (one scale per column) and int8
// coefficients (one scale per token row) and centroid (one scale).
//
// Mapping: a 64-lane wave builds 4 pages; 16 lanes serve one page, lane i
// owning row i of the Gram matrix and of the eigenvector matrix U. The keys
// are bf16, so K K^T accumulated in fp64 is exact to rounding of the sums,
// and the Gram is formed as C (K K^T) C with the centring matrix
// C = I - 11^T/B. The eigendecomposition is a cyclic two-sided Jacobi in
// fp64 (rotation angles evaluated in fp32 and made orthogonal to fp64
// rounding, as in the one-page form): round m (m = 1..15) rotates the 8
// disjoint pairs (i, i xor m), so a
// sweep visits each of the 120 pairs once. Lane i keeps its rows permuted as
// b[x] = A[i][i xor x]; then the diagonal is b[0], the pair element is b[m]
// and every exchange is a xor lane shuffle. Sweeps stop when the off-diagonal
// mass of all 4 pages is below 1e-28 of the Frobenius mass (at most 12).
#include "locks_build_common.h"

namespace locks {

constexpr int kBuildPages = 4;    // pages per wave
constexpr int kRowPad = 132;      // fp32 LDS row stride of the key tile
constexpr int kMaxSweeps = 12;

__device__ __forceinline__ double shfl_xor_d(double v, int m) { return __shfl_xor(v, m, 64); }

// One Jacobi round: rotate the 8 pairs (p, p xor M) of the page's 16 rows.
// Lane i holds b[x] = A[i][i^x] and ub[x] = U[i][i^x].
template <int M>
__device__ __forceinline__ void jacobi_round(double (&b)[kPage], double (&ub)[kPage], int i) {
  constexpr int HB = (M >= 8) ? 8 : (M >= 4) ? 4 : (M >= 2) ? 2 : 1;  // top bit of M
  const bool lo = (i & HB) == 0;  // this row is the lower index of its pair
  const double aii = b[0], ajj = shfl_xor_d(b[0], M);
  const double apq = 0.5 * (b[M] + shfl_xor_d(b[M], M));
  double c, s;
  rotation_fast(lo ? aii : ajj, lo ? ajj : aii, apq, c, s);
  // Signed sine: +s on the lower lane of the pair, -s on the upper one. For
  // column j of this row the pair's rotation enters with the sign that lane j
  // itself holds, so fetching (c, sr) from lane j = i^x needs no lane masks.
  const double sr = lo ? s : -s;
  // columns: the pair (x, x^M) of the permuted row
#pragma unroll
  for (int x = 0; x < kPage; ++x) {
    if (x & HB) continue;
    const double cx = (x == 0) ? c : shfl_xor_d(c, x);
    const double sg = (x == 0) ? sr : shfl_xor_d(sr, x);
    const double b0 = b[x], b1 = b[x ^ M];
    b[x] = cx * b0 - sg * b1;
    b[x ^ M] = cx * b1 + sg * b0;
    const double u0 = ub[x], u1 = ub[x ^ M];
    ub[x] = cx * u0 - sg * u1;
    ub[x ^ M] = cx * u1 + sg * u0;
  }
  // rows: row_i <- c row_i -+ s row_partner; the partner's row is read in its
  // own permuted order (A[i^M][i^x] is the partner's b[x^M])
  double pr[kPage];
#pragma unroll
  for (int x = 0; x < kPage; ++x) pr[x] = shfl_xor_d(b[x ^ M], M);
#pragma unroll
  for (int x = 0; x < kPage; ++x) b[x] = c * b[x] - sr * pr[x];
}

// Pages come from a list of block ids (ids != nullptr: all H heads of each)
// or, in filled-page mode, from the sequences whose length is a multiple of
// the page size (their last page). In filled-page mode knew/vnew (optional)
// carry the token at position len - 1 of every sequence: it is appended to
// kdst/vdst (the pools) and, where it completes a page, taken as that page's
// last key straight from knew.
template <int R>
__global__ __launch_bounds__(64) void build_kernel(
    const uint16_t* __restrict__ kpool, int64_t num_blocks, int H,
    const int32_t* __restrict__ ids, int n, const int32_t* __restrict__ table,
    const int32_t* __restrict__ lens, int MP, uint8_t* __restrict__ summ,
    const uint16_t* __restrict__ knew, const uint16_t* __restrict__ vnew,
    uint16_t* __restrict__ kdst, uint16_t* __restrict__ vdst, int bits) {
  const SlotLayout L = slot_layout(R, bits);
  const int vq_max = basis_qmax(bits);
  __shared__ float kt[kBuildPages][kPage][kRowPad];
  __shared__ double urow[kBuildPages][kPage][kPage + 1];
  __shared__ double lam_s[kBuildPages][kPage];
  __shared__ int perm_s[kBuildPages][kPage];
  __shared__ double sig_s[kBuildPages][kPage];

  const int lane = threadIdx.x, pg = lane >> 4, i = lane & 15;
  const int64_t item = (int64_t)blockIdx.x * kBuildPages + pg;
  // ---- which page this lane group builds
  int64_t slot = -1;
  int blk = 0, head = 0;
  const uint8_t* last_key = nullptr;  // row 15 of the page, when it comes from knew
  {
    if (ids) {
      if (item < (int64_t)n * H) {
        const int b = ids[item / H];
        head = (int)(item % H);
        if (b >= 0 && b < num_blocks) { blk = b; slot = (int64_t)b * H + head; }
      }
    } else {
      // filled-page mode: item = seq * H + head
      if (item < (int64_t)n * H) {
        const int sq = (int)(item / H);
        head = (int)(item % H);
        const int len = lens[sq];
        const int64_t src = ((int64_t)sq * H + head) * kHeadDim;
        if (knew && len >= 1 && len <= MP * kPage) {
          const int b = table[(int64_t)sq * MP + (len - 1) / kPage];
          if (b >= 0 && b < num_blocks) {
            const int64_t dst =
                (((int64_t)b * H + head) * kPage + (len - 1) % kPage) * kHeadDim + 8 * i;
            *reinterpret_cast<uint4*>(kdst + dst) = *reinterpret_cast<const uint4*>(knew + src + 8 * i);
            *reinterpret_cast<uint4*>(vdst + dst) = *reinterpret_cast<const uint4*>(vnew + src + 8 * i);
          }
        }
        if (len > 0 && len % kPage == 0 && len / kPage <= MP) {
          const int b = table[(int64_t)sq * MP + len / kPage - 1];
          if (b >= 0 && b < num_blocks) {
            blk = b;
            slot = (int64_t)b * H + head;
            if (knew) last_key = reinterpret_cast<const uint8_t*>(knew + src);
          }
        }
      }
    }
  }
  const int64_t kofs = ((int64_t)blk * H + head) * (kPage * kHeadDim);

  // ---- phase 0: keys -> LDS (fp32, exact for bf16); centroid dims 8i..8i+7
  double mu[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) mu[e] = 0.0;
  {
    const uint8_t* kb = reinterpret_cast<const uint8_t*>(kpool + kofs);
#pragma unroll 4
    for (int t = 0; t < kPage; ++t) {
      const uint8_t* rowp = (last_key && t == kPage - 1) ? last_key : kb + t * 256;
      const uint4 w = (slot >= 0) ? *reinterpret_cast<const uint4*>(rowp + 16 * i)
                                  : make_uint4(0u, 0u, 0u, 0u);
      const uint32_t ww[4] = {w.x, w.y, w.z, w.w};
      float f[8];
#pragma unroll
      for (int e = 0; e < 4; ++e) { f[2 * e] = bf16_lo(ww[e]); f[2 * e + 1] = bf16_hi(ww[e]); }
#pragma unroll
      for (int e = 0; e < 8; ++e) mu[e] += (double)f[e];
      *reinterpret_cast<float4*>(&kt[pg][t][8 * i]) = make_float4(f[0], f[1], f[2], f[3]);
      *reinterpret_cast<float4*>(&kt[pg][t][8 * i + 4]) = make_float4(f[4], f[5], f[6], f[7]);
    }
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) mu[e] *= (1.0 / kPage);
  __syncthreads();

  // ---- phase 1: M = K K^T (row i, permuted: Mb[x] = M[i][i^x]), G = C M C
  double b[kPage];
#pragma unroll
  for (int x = 0; x < kPage; ++x) b[x] = 0.0;
  for (int d = 0; d < kHeadDim; d += 4) {
    const float4 ki = *reinterpret_cast<const float4*>(&kt[pg][i][d]);
    const double k0 = ki.x, k1 = ki.y, k2 = ki.z, k3 = ki.w;
#pragma unroll
    for (int x = 0; x < kPage; ++x) {
      const float4 kj = *reinterpret_cast<const float4*>(&kt[pg][i ^ x][d]);
      double a = b[x];
      a = fma(k0, (double)kj.x, a);
      a = fma(k1, (double)kj.y, a);
      a = fma(k2, (double)kj.z, a);
      a = fma(k3, (double)kj.w, a);
      b[x] = a;
    }
  }
  double energy = b[0];  // sum_i |k_i|^2 after the group reduction below
  double rmean = 0.0;
#pragma unroll
  for (int x = 0; x < kPage; ++x) rmean += b[x];
  rmean *= (1.0 / kPage);
  double tall = rmean;
#pragma unroll
  for (int m = 1; m < kPage; m <<= 1) {
    tall += shfl_xor_d(tall, m);
    energy += shfl_xor_d(energy, m);
  }
  tall *= (1.0 / kPage);
#pragma unroll
  for (int x = 0; x < kPage; ++x) {
    const double rj = (x == 0) ? rmean : shfl_xor_d(rmean, x);
    b[x] = (b[x] - (rmean + rj)) + tall;
  }
  double trace = b[0];
#pragma unroll
  for (int m = 1; m < kPage; m <<= 1) trace += shfl_xor_d(trace, m);

  // ---- phase 2: cyclic Jacobi, U accumulated in the same permuted order
  double ub[kPage];
#pragma unroll
  for (int x = 0; x < kPage; ++x) ub[x] = (x == 0) ? 1.0 : 0.0;
  for (int sweep = 0; sweep < kMaxSweeps; ++sweep) {
    double off = 0.0, tot = 0.0;
#pragma unroll
    for (int x = 0; x < kPage; ++x) {
      const double v = b[x] * b[x];
      tot += v;
      if (x) off += v;
    }
#pragma unroll
    for (int m = 1; m < kPage; m <<= 1) {
      off += shfl_xor_d(off, m);
      tot += shfl_xor_d(tot, m);
    }
    const bool done = !(off > 1e-28 * tot);
    if (__all(done)) break;
    jacobi_round<1>(b, ub, i);
    jacobi_round<2>(b, ub, i);
    jacobi_round<3>(b, ub, i);
    jacobi_round<4>(b, ub, i);
    jacobi_round<5>(b, ub, i);
    jacobi_round<6>(b, ub, i);
    jacobi_round<7>(b, ub, i);
    jacobi_round<8>(b, ub, i);
    jacobi_round<9>(b, ub, i);
    jacobi_round<10>(b, ub, i);
    jacobi_round<11>(b, ub, i);
    jacobi_round<12>(b, ub, i);
    jacobi_round<13>(b, ub, i);
    jacobi_round<14>(b, ub, i);
    jacobi_round<15>(b, ub, i);
  }

  // ---- phase 3: order eigenvalues (descending, lower index first on ties)
  const double lam = b[0];
  int rank = 0;
#pragma unroll
  for (int x = 1; x < kPage; ++x) {
    const double o = shfl_xor_d(lam, x);
    const int j = i ^ x;
    rank += (o > lam || (o == lam && j < i)) ? 1 : 0;
  }
  lam_s[pg][rank & (kPage - 1)] = lam;
  perm_s[pg][rank & (kPage - 1)] = i;
#pragma unroll
  for (int x = 0; x < kPage; ++x) urow[pg][i][i ^ x] = ub[x];
  __syncthreads();

  uint8_t* sl = (slot >= 0) ? summ + slot * (int64_t)L.stride : nullptr;
  const double thr = fmax(1e-6 * trace, 1e-12 * energy);

  // ---- phase 4: basis columns (lane i owns dims 8i..8i+7), sign, int4 codes
#pragma unroll 1
  for (int k = 0; k < R; ++k) {
    const double lk = lam_s[pg][k];
    const int ck = perm_s[pg][k] & (kPage - 1);
    const bool act = lk > thr;
    const double sig = act ? sqrt(lk) : 1.0;
    double v[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = 0.0;
#pragma unroll 2
    for (int t = 0; t < kPage; ++t) {
      const double u = urow[pg][t][ck];
      const float4 a = *reinterpret_cast<const float4*>(&kt[pg][t][8 * i]);
      const float4 c4 = *reinterpret_cast<const float4*>(&kt[pg][t][8 * i + 4]);
      const float kk[8] = {a.x, a.y, a.z, a.w, c4.x, c4.y, c4.z, c4.w};
#pragma unroll
      for (int e = 0; e < 8; ++e) v[e] = fma((double)kk[e] - mu[e], u, v[e]);
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = act ? v[e] / sig : 0.0;
    // largest |v| (lowest dim on ties) and its sign, across the 16 lanes
    double amax = -1.0, aval = 0.0;
    int aidx = 0;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const double av = fabs(v[e]);
      if (av > amax) { amax = av; aval = v[e]; aidx = 8 * i + e; }
    }
#pragma unroll
    for (int m = 1; m < kPage; m <<= 1) {
      const double oa = shfl_xor_d(amax, m), ov = shfl_xor_d(aval, m);
      const int oi = __shfl_xor(aidx, m, 64);
      if (oa > amax || (oa == amax && oi < aidx)) { amax = oa; aval = ov; aidx = oi; }
    }
    const double flip = (aval < 0.0) ? -1.0 : 1.0;
    if (i == 0) {
      sig_s[pg][k] = act ? sig * flip : 0.0;  // coefficient multiplier, 0 if inactive
    }
    const uint16_t sbits = act ? fp16_scale_bits(amax, (float)vq_max) : (uint16_t)0;
    const float scale = (float)__builtin_bit_cast(_Float16, sbits);
    int code[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) code[e] = quant_code(v[e] * flip, scale, vq_max);
    if (sl) {
      if (bits == 4) {
        // bytes carry the dim pairs (0,1), (4,5), (2,3), (6,7), low nibble first
        int c4[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) c4[e] = code[e] & 0xF;
        const uint32_t word = (uint32_t)(c4[0] | c4[1] << 4) | (uint32_t)(c4[4] | c4[5] << 4) << 8 |
                              (uint32_t)(c4[2] | c4[3] << 4) << 16 | (uint32_t)(c4[6] | c4[7] << 4) << 24;
        *reinterpret_cast<uint32_t*>(sl + 64 * k + 4 * i) = word;
      } else if (bits == 8) {  // one byte per dim, dim order
        uint32_t lo = 0, hi = 0;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          lo |= (uint32_t)(code[e] & 0xFF) << (8 * e);
          hi |= (uint32_t)(code[e + 4] & 0xFF) << (8 * e);
        }
        *reinterpret_cast<uint2*>(sl + 128 * k + 8 * i) = make_uint2(lo, hi);
      } else {  // two bits per dim, dim order from the lowest bits
        uint32_t h = 0;
#pragma unroll
        for (int e = 0; e < 8; ++e) h |= (uint32_t)(code[e] & 0x3) << (2 * e);
        *reinterpret_cast<uint16_t*>(sl + 32 * k + 2 * i) = (uint16_t)h;
      }
      if (i == 0) *reinterpret_cast<uint16_t*>(sl + L.sv + 2 * k) = sbits;
    }
  }
  __syncthreads();

  // ---- coefficients: lane t owns row c_t = U[t][c_k] sigma_k (signed), int8
  {
    double cr[R];
    double amax = 0.0;
#pragma unroll
    for (int k = 0; k < R; ++k) {
      const double f = sig_s[pg][k];
      cr[k] = (f != 0.0) ? urow[pg][i][perm_s[pg][k] & (kPage - 1)] * fabs(f) * (f < 0.0 ? -1.0 : 1.0) : 0.0;
      amax = fmax(amax, fabs(cr[k]));
    }
    const uint16_t sbits = amax > 0.0 ? fp16_scale_bits(amax, 127.f) : (uint16_t)0;
    const float scale = (float)__builtin_bit_cast(_Float16, sbits);
    if (sl) {
#pragma unroll
      for (int k = 0; k < R; ++k) sl[L.c + i * R + k] = (uint8_t)(quant_code(cr[k], scale, 127) & 0xFF);
      *reinterpret_cast<uint16_t*>(sl + L.sc + 2 * i) = sbits;
    }
  }

  // ---- centroid: lane i owns dims 8i..8i+7, one scale for the page
  {
    double amax = 0.0;
#pragma unroll
    for (int e = 0; e < 8; ++e) amax = fmax(amax, fabs(mu[e]));
#pragma unroll
    for (int m = 1; m < kPage; m <<= 1) amax = fmax(amax, shfl_xor_d(amax, m));
    const uint16_t sbits = amax > 0.0 ? fp16_scale_bits(amax, 127.f) : (uint16_t)0;
    const float scale = (float)__builtin_bit_cast(_Float16, sbits);
    uint32_t lo = 0, hi = 0;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      lo |= (uint32_t)(quant_code(mu[e], scale, 127) & 0xFF) << (8 * e);
      hi |= (uint32_t)(quant_code(mu[e + 4], scale, 127) & 0xFF) << (8 * e);
    }
    if (sl) {
      *reinterpret_cast<uint2*>(sl + L.mu + 8 * i) = make_uint2(lo, hi);
      if (i == 0) {
        *reinterpret_cast<uint16_t*>(sl + L.smu) = sbits;
        for (int p = L.payload; p < L.stride; ++p) sl[p] = 0;
      }
    }
  }
}

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

template <int R>
static hipError_t launch_build_r(const uint16_t* kpool, int64_t nb, int H, const int32_t* ids,
                                 int n, const int32_t* table, const int32_t* lens, int MP,
                                 uint8_t* summ, const uint16_t* knew, const uint16_t* vnew,
                                 uint16_t* kdst, uint16_t* vdst, int bits, hipStream_t st) {
  const int64_t items = (int64_t)n * H;
  if (items == 0) return hipSuccess;
  const int64_t grid = (items + kBuildPages - 1) / kBuildPages;
  hipLaunchKernelGGL(build_kernel<R>, dim3((unsigned)grid), dim3(64), 0, st, kpool, nb, H, ids, n,
                     table, lens, MP, summ, knew, vnew, kdst, vdst, bits);
  return hipGetLastError();
}

hipError_t launch_build_page(int r, const void* kpool, int64_t nb, int H, const int32_t* ids, int n,
                             const int32_t* table, const int32_t* lens, int MP, void* summ,
                             const void* knew, const void* vnew, void* vpool, int bits,
                             hipStream_t st);

// Up to this many pages go to the one-page-per-wave form (shorter time to a
// summary); larger lists to the 4-pages-per-wave form.
constexpr int64_t kPageFormMaxItems = 4096;

// knew/vnew (filled-page mode only, may be null): append the new token too.
hipError_t launch_build(int r, const void* kpool, int64_t nb, int H, const int32_t* ids, int n,
                        const int32_t* table, const int32_t* lens, int MP, void* summ,
                        const void* knew, const void* vnew, void* vpool, int bits, hipStream_t st) {
  if (bits != 2 && bits != 4 && bits != 8) return hipErrorInvalidValue;
  if (!ids || (int64_t)n * H <= kPageFormMaxItems)
    return launch_build_page(r, kpool, nb, H, ids, n, table, lens, MP, summ, knew, vnew, vpool, bits,
                             st);
  const uint16_t* kp = static_cast<const uint16_t*>(kpool);
  uint8_t* sm = static_cast<uint8_t*>(summ);
  const uint16_t* kn = static_cast<const uint16_t*>(knew);
  const uint16_t* vn = static_cast<const uint16_t*>(vnew);
  uint16_t* kd = const_cast<uint16_t*>(kp);
  uint16_t* vd = static_cast<uint16_t*>(vpool);
  switch (r) {
#define LOCKS_R(RR) \
  case RR:          \
    return launch_build_r<RR>(kp, nb, H, ids, n, table, lens, MP, sm, kn, vn, kd, vd, bits, st);
    LOCKS_R(1) LOCKS_R(2) LOCKS_R(3) LOCKS_R(4) LOCKS_R(5) LOCKS_R(6) LOCKS_R(7) LOCKS_R(8)
    LOCKS_R(9) LOCKS_R(10) LOCKS_R(11) LOCKS_R(12) LOCKS_R(13) LOCKS_R(14) LOCKS_R(15) LOCKS_R(16)
#undef LOCKS_R
    default:
      return hipErrorInvalidValue;
  }
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
