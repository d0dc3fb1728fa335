// LOCKS page-summary build: one 64-lane wave per page (gfx950).
//
// [N] = LOCKS reading notes (zhongzhuzhou.org 2026-07-29), §4.1 eq. 2-3 and
// §4.3 Algorithm 1: centroid mu, deviations D = K - 1 mu^T, Gram D D^T,
// descending eigendecomposition, basis V = D^T U_r Sigma_r^{-1}, coefficients
// C = U_r Sigma_r, int4 basis (int8 / int2 for the precision ablation) /
// int8 coefficients / int8 centroid. Serves every build: the few pages a
// decode step completes (time to one summary) and whole layers (pages per
// second: the keys stay in registers, so the kernel needs 9.7 KB of LDS and
// at most 128 registers, and 16 of its waves fit on a compute unit).
//
// Mapping (one wave, lane l):
//   keys  : lane l loads dims 32 (l / 16) .. +31 of token l % 16 (its Gram
//           operands) and, after the eigensolve, dims 2l, 2l+1 of every
//           token (its share of the centroid and the basis);
//   Gram  : K K^T on v_mfma_f64_16x16x4f64, 32 chunks of 4 dims: lane l feeds
//           K[l % 16][32 (l / 16) + c] as both operands; the result lands as
//           rows l / 16 + 4 i, column l % 16; centring G = C (K K^T) C;
//   Jacobi: lane 16 c + i holds entries x = 4c .. 4c+3 of row i in the
//           permuted order b[e] = A[i][i xor x] (and U likewise); round M
//           rotates the 8 pairs (p, p xor M) at once, with the diagonal, the
//           pair elements, the rotations and the partner rows exchanged
//           through LDS. Rotation angles are evaluated in fp32 (on operands
//           scaled to a common exponent) and c = 1/sqrt(1 + t^2) is brought
//           to fp64 accuracy, so every rotation is orthogonal to fp64
//           rounding while a visit leaves |a_pq| at about 1e-7 of its value;
//           sweeps stop when the off-diagonal mass falls below 1e-28 of the
//           total (at most 12);
//   basis : lane l owns dims 2l, 2l+1 of every basis column; coefficients:
//           lane t < 16 owns token row t.
#include "locks_build_common.h"

namespace locks {

typedef double double4v __attribute__((ext_vector_type(4)));

constexpr int kPgMaxSweeps = 12;


// LDS exchange area of the 64-lane Jacobi.
constexpr int kApStride = kPage + 2;  // 16-byte aligned rows, rows spread over banks
struct JacobiLds {
  double2 cs[kPage];              // (c, signed s) of the pair of row i
  double ap[kPage][kApStride];    // rows in permuted order: ap[i][x] = A[i][i ^ x]
  double up[kPage][kApStride];    // the same for U
};

__device__ __forceinline__ void store4(double* p, const double (&v)[4]) {
  reinterpret_cast<double2*>(p)[0] = make_double2(v[0], v[1]);
  reinterpret_cast<double2*>(p)[1] = make_double2(v[2], v[3]);
}
template <int EM>
__device__ __forceinline__ void load4_perm(double (&v)[4], const double* p) {
  const double2 a = reinterpret_cast<const double2*>(p)[0];
  const double2 b = reinterpret_cast<const double2*>(p)[1];
  const double t[4] = {a.x, a.y, b.x, b.y};
#pragma unroll
  for (int e = 0; e < 4; ++e) v[e] = t[e ^ EM];
}

// Wave-wide max / sum of a double: DPP inside rows of 16, then the rows
// pairwise by lane permutes (rows 0-1 and 2-3, then the two halves). Each
// permute hands both lanes of a pair the same (lower row, upper row) values,
// so every lane ends with the same bits.
template <int C>
__device__ __forceinline__ double dpp_d(double v) {
  const uint64_t u = (uint64_t)__double_as_longlong(v);
  const uint32_t lo = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)u, C, 0xF, 0xF, false);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)(u >> 32), C, 0xF, 0xF, false);
  return __longlong_as_double((long long)(((uint64_t)hi << 32) | lo));
}
__device__ __forceinline__ double join_d(uint32_t lo, uint32_t hi) {
  return __longlong_as_double((long long)(((uint64_t)hi << 32) | lo));
}
// (lower, upper) of the row pair (xor 16) or half pair (xor 32) holding v
template <bool kHalves>
__device__ __forceinline__ void pair_d(double v, double& a, double& b) {
  const uint64_t u = (uint64_t)__double_as_longlong(v);
  const uint32_t lo = (uint32_t)u, hi = (uint32_t)(u >> 32);
  if (kHalves) {
    const auto l = __builtin_amdgcn_permlane32_swap(lo, lo, false, false);
    const auto h = __builtin_amdgcn_permlane32_swap(hi, hi, false, false);
    a = join_d(l[0], h[0]);
    b = join_d(l[1], h[1]);
  } else {
    const auto l = __builtin_amdgcn_permlane16_swap(lo, lo, false, false);
    const auto h = __builtin_amdgcn_permlane16_swap(hi, hi, false, false);
    a = join_d(l[0], h[0]);
    b = join_d(l[1], h[1]);
  }
}
// One round of the 64-lane cyclic Jacobi: the 8 pairs (p, p xor M) at once.
// Lane (i, qc) holds b[e] = A[i][i ^ x], x = 4 qc + e, and U likewise.
// Column j = i ^ x turns with the rotation of row j's pair: b[x] <- c_j b[x]
// - s_j b[x ^ M], s_j signed as row j holds it (+s on the lower row of a
// pair, -s on the upper); then row i mixes with row i ^ M. The partner row's
// column-turned entry is formed here from its pre-round entries, so a round
// needs two exchanges: the pre-round rows (which also give the rotation
// parameters), then the rotations.
template <int M>
__device__ __forceinline__ void jacobi64_round(double (&b)[4], double (&ub)[4], int i, int qc,
                                               JacobiLds& sh) {
  constexpr int HB = (M >= 8) ? 8 : (M >= 4) ? 4 : (M >= 2) ? 2 : 1;  // top bit of M
  constexpr int QM = M >> 2, EM = M & 3;
  store4(&sh.ap[i][4 * qc], b);
  if (QM != 0) store4(&sh.up[i][4 * qc], ub);
  __syncthreads();
  const double aii = sh.ap[i][0], ajj = sh.ap[i ^ M][0];
  const double apq = 0.5 * (sh.ap[i][M] + sh.ap[i ^ M][M]);
  double pb[4], pu[4], px[4], pxm[4];
  load4_perm<0>(px, &sh.ap[i ^ M][4 * qc]);  // partner row, entries x
  if (QM == 0) {
#pragma unroll
    for (int e = 0; e < 4; ++e) { pb[e] = b[e ^ EM]; pu[e] = ub[e ^ EM]; pxm[e] = px[e ^ EM]; }
  } else {
    load4_perm<EM>(pb, &sh.ap[i][4 * (qc ^ QM)]);
    load4_perm<EM>(pu, &sh.up[i][4 * (qc ^ QM)]);
    load4_perm<EM>(pxm, &sh.ap[i ^ M][4 * (qc ^ QM)]);  // partner row, entries x ^ M
  }
  const bool lo = (i & HB) == 0;
  double cr, s0;
  rotation_fast(lo ? aii : ajj, lo ? ajj : aii, apq, cr, s0);
  const double sr = lo ? s0 : -s0;
  if (qc == 0) sh.cs[i] = make_double2(cr, sr);
  __syncthreads();
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const double2 r = sh.cs[i ^ (4 * qc + e)];
    const double b1 = r.x * b[e] - r.y * pb[e];      // own row, column turned
    const double p1 = r.x * pxm[e] - r.y * px[e];    // partner row at column i ^ x, turned
    ub[e] = r.x * ub[e] - r.y * pu[e];
    b[e] = cr * b1 - sr * p1;
  }
}

__device__ __forceinline__ double wave_max_d(double v) {
  v = fmax(v, dpp_d<0xB1>(v));   // xor 1
  v = fmax(v, dpp_d<0x4E>(v));   // xor 2
  v = fmax(v, dpp_d<0x141>(v));  // half-row mirror: quads 0/1, 2/3
  v = fmax(v, dpp_d<0x140>(v));  // row mirror: halves of the row
  double a, b;
  pair_d<false>(v, a, b);
  pair_d<true>(fmax(a, b), a, b);
  return fmax(a, b);
}
__device__ __forceinline__ double wave_sum_d(double v) {
  v += dpp_d<0xB1>(v);
  v += dpp_d<0x4E>(v);
  v += dpp_d<0x141>(v);
  v += dpp_d<0x140>(v);
  double a, b;
  pair_d<false>(v, a, b);
  pair_d<true>(a + b, a, b);
  return a + b;
}
__device__ __forceinline__ double readlane_d(double v, int src) {
  const uint64_t u = (uint64_t)__double_as_longlong(v);
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)u, src);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(u >> 32), src);
  return __longlong_as_double((long long)(((uint64_t)hi << 32) | lo));
}

template <int R>
__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(4))) void build_page_kernel(
    const uint16_t* __restrict__ kpool, int64_t num_blocks, int H,
    const int32_t* __restrict__ ids, int n, const int32_t* __restrict__ table,
    const int32_t* __restrict__ lens, int MP, uint8_t* __restrict__ summ,
    const uint16_t* __restrict__ knew, const uint16_t* __restrict__ vnew,
    uint16_t* __restrict__ kdst, uint16_t* __restrict__ vdst, int bits) {
  const SlotLayout L = slot_layout(R, bits);
  const int vq_max = basis_qmax(bits);
  __shared__ double g_s[kPage][kPage + 1];
  __shared__ double u_s[kPage][kPage + 1];
  __shared__ double lam_s[kPage];
  __shared__ int perm_s[kPage];
  __shared__ double sig_s[kPage];
  __shared__ double rm_s[kPage];
  __shared__ JacobiLds jl;

  const int lane = threadIdx.x;
  const int64_t item = blockIdx.x;
  // ---- which page: block ids[item / H] (all heads), or in filled-page mode
  // the last page of sequence item / H when its length is a multiple of the
  // page size (the new token, appended here too, is that page's last key)
  int64_t slot = -1;
  int blk = 0, head = (int)(item % H);
  const uint8_t* last_key = nullptr;
  if (ids) {
    const int b = ids[item / H];
    if (b >= 0 && b < num_blocks) { blk = b; slot = (int64_t)b * H + head; }
  } else {
    const int sq = (int)(item / H);
    const int len = lens[sq];
    const int64_t src = ((int64_t)sq * H + head) * kHeadDim;
    if (knew && len >= 1 && len <= MP * kPage && lane < 2 * (kHeadDim / 8)) {
      const int b = table[(int64_t)sq * MP + (len - 1) / kPage];
      if (b >= 0 && b < num_blocks) {
        const int c8 = lane % (kHeadDim / 8);
        const int64_t dst = (((int64_t)b * H + head) * kPage + (len - 1) % kPage) * kHeadDim + 8 * c8;
        if (lane < kHeadDim / 8)
          *reinterpret_cast<uint4*>(kdst + dst) = *reinterpret_cast<const uint4*>(knew + src + 8 * c8);
        else
          *reinterpret_cast<uint4*>(vdst + dst) = *reinterpret_cast<const uint4*>(vnew + src + 8 * c8);
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
  if (slot < 0) return;  // whole wave: nothing to build
  uint8_t* sl = summ + slot * (int64_t)L.stride;

  // ---- keys, straight into registers (no LDS copy): lane (t = lane % 16,
  // kg = lane / 16) takes dims 32 kg .. 32 kg + 31 of row t, its operands of
  // the Gram product (and, after the eigensolve, dims 2 lane, 2 lane + 1 of
  // every row, its share of the centroid and the basis); energy = sum of
  // squares of all keys
  const int t = lane & 15, kg = lane >> 4;
  auto row_of = [&](int tt) -> const uint8_t* {
    return (last_key && tt == kPage - 1)
               ? last_key
               : reinterpret_cast<const uint8_t*>(kpool + (((int64_t)blk * H + head) * kPage + tt) * kHeadDim);
  };
  uint4 wg4[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) wg4[e] = *reinterpret_cast<const uint4*>(row_of(t) + 64 * kg + 16 * e);
  double energy = 0.0;
  float kv[32];  // dims 32 kg + c, c = 0..31, of row t
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const uint32_t ww[4] = {wg4[e].x, wg4[e].y, wg4[e].z, wg4[e].w};
#pragma unroll
    for (int h2 = 0; h2 < 4; ++h2) {
      kv[8 * e + 2 * h2] = bf16_lo(ww[h2]);
      kv[8 * e + 2 * h2 + 1] = bf16_hi(ww[h2]);
    }
  }
#pragma unroll
  for (int c = 0; c < 32; ++c) energy = fma((double)kv[c], (double)kv[c], energy);
  energy = wave_sum_d(energy);

  // ---- Gram K K^T on the fp64 matrix core: rows l/16 + 4i, column l%16
  double4v mk = {0.0, 0.0, 0.0, 0.0};
#pragma unroll
  for (int c = 0; c < 32; ++c) mk = __builtin_amdgcn_mfma_f64_16x16x4f64((double)kv[c], (double)kv[c], mk, 0, 0, 0);
  // centring: G = M - rm 1^T - 1 rm^T + mean(rm), rm = row means (M symmetric)
  {
    const int col = lane & 15, rg = lane >> 4;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      double v = mk[i];  // row sum inside the 16-lane row
      v += dpp_d<0xB1>(v);
      v += dpp_d<0x4E>(v);
      v += dpp_d<0x141>(v);
      v += dpp_d<0x140>(v);
      if (col == 0) rm_s[rg + 4 * i] = v * (1.0 / kPage);
    }
    __syncthreads();
    double tall = 0.0;
#pragma unroll
    for (int r = 0; r < kPage; ++r) tall += rm_s[r];
    tall *= (1.0 / kPage);
    const double rc = rm_s[col];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = rg + 4 * i;
      g_s[row][col] = (mk[i] - (rm_s[row] + rc)) + tall;
    }
  }
  __syncthreads();

  // ---- Jacobi
  const int ii = lane & 15, qc = lane >> 4;
  double b[4], ub[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    b[e] = g_s[ii][ii ^ (4 * qc + e)];
    ub[e] = (qc == 0 && e == 0) ? 1.0 : 0.0;
  }
  const double trace = wave_sum_d((qc == 0) ? b[0] : 0.0);
  for (int sweep = 0; sweep < kPgMaxSweeps; ++sweep) {
    double off = 0.0, tot = 0.0;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const double v = b[e] * b[e];
      tot += v;
      if (qc != 0 || e != 0) off += v;
    }
    off = wave_sum_d(off);
    tot = wave_sum_d(tot);
    if (!(off > 1e-28 * tot)) break;  // the same value in every lane
    jacobi64_round<1>(b, ub, ii, qc, jl);
    jacobi64_round<2>(b, ub, ii, qc, jl);
    jacobi64_round<3>(b, ub, ii, qc, jl);
    jacobi64_round<4>(b, ub, ii, qc, jl);
    jacobi64_round<5>(b, ub, ii, qc, jl);
    jacobi64_round<6>(b, ub, ii, qc, jl);
    jacobi64_round<7>(b, ub, ii, qc, jl);
    jacobi64_round<8>(b, ub, ii, qc, jl);
    jacobi64_round<9>(b, ub, ii, qc, jl);
    jacobi64_round<10>(b, ub, ii, qc, jl);
    jacobi64_round<11>(b, ub, ii, qc, jl);
    jacobi64_round<12>(b, ub, ii, qc, jl);
    jacobi64_round<13>(b, ub, ii, qc, jl);
    jacobi64_round<14>(b, ub, ii, qc, jl);
    jacobi64_round<15>(b, ub, ii, qc, jl);
  }
  // eigenvalues (diagonal) and eigenvectors (columns of U) to LDS
  if (qc == 0) lam_s[ii] = b[0];
#pragma unroll
  for (int e = 0; e < 4; ++e) u_s[ii][ii ^ (4 * qc + e)] = ub[e];
  __syncthreads();
  // descending order, lower index first on ties
  if (lane < kPage) {
    const double lam = lam_s[lane];
    int rank = 0;
#pragma unroll
    for (int j = 0; j < kPage; ++j) {
      const double o = lam_s[j];
      rank += (o > lam || (o == lam && j < lane)) ? 1 : 0;
    }
    perm_s[rank & (kPage - 1)] = lane;
  }
  __syncthreads();

  const double thr = fmax(1e-6 * trace, 1e-12 * energy);
  // the lane's dims of every row (read again: the page was just fetched)
  uint32_t wc[kPage];
#pragma unroll
  for (int tt = 0; tt < kPage; ++tt) wc[tt] = *reinterpret_cast<const uint32_t*>(row_of(tt) + 4 * lane);
  // ---- centroid (dims 2l, 2l+1) and the page's deviations in those dims
  double mu[2];
#pragma unroll
  for (int e = 0; e < 2; ++e) mu[e] = 0.0;
#pragma unroll
  for (int tt = 0; tt < kPage; ++tt) {
    mu[0] += (double)bf16_lo(wc[tt]);
    mu[1] += (double)bf16_hi(wc[tt]);
  }
  mu[0] *= (1.0 / kPage);
  mu[1] *= (1.0 / kPage);
  double dv[kPage][2];
#pragma unroll
  for (int tt = 0; tt < kPage; ++tt) {
    dv[tt][0] = (double)bf16_lo(wc[tt]) - mu[0];
    dv[tt][1] = (double)bf16_hi(wc[tt]) - mu[1];
  }

  // ---- basis columns: v_k = D^T u_k / sigma_k, canonical sign, int4 codes
  const int wq = lane >> 2, pq = lane & 3;           // word of 8 dims, pair inside it
  const int byte_of_pair = (pq == 0) ? 0 : (pq == 1) ? 2 : (pq == 2) ? 1 : 3;
#pragma unroll
  for (int k = 0; k < R; ++k) {
    const int ck = perm_s[k] & (kPage - 1);
    const double lk = lam_s[ck];
    const bool act = lk > thr;
    const double sig = act ? sqrt(lk) : 1.0;
    double v0 = 0.0, v1 = 0.0;
#pragma unroll
    for (int t = 0; t < kPage; ++t) {
      const double u = u_s[t][ck];
      v0 = fma(dv[t][0], u, v0);
      v1 = fma(dv[t][1], u, v1);
    }
    v0 = act ? v0 / sig : 0.0;
    v1 = act ? v1 / sig : 0.0;
    // largest |v| over the 128 dims, and its value at the lowest such dim
    // (dims 2l, 2l+1 live in lane l)
    const double a0 = fabs(v0), a1 = fabs(v1);
    const double amax = wave_max_d(fmax(a0, a1));
    const uint64_t m0 = __ballot(a0 == amax), m1 = __ballot(a1 == amax);
    const int l0 = m0 ? __builtin_ctzll(m0) : 64, l1 = m1 ? __builtin_ctzll(m1) : 64;
    const double aval = (l0 <= l1) ? readlane_d(v0, l0) : readlane_d(v1, l1);
    const double flip = (aval < 0.0) ? -1.0 : 1.0;
    if (lane == 0) sig_s[k] = act ? sig * flip : 0.0;
    const uint16_t sbits = act ? fp16_scale_bits(amax, (float)vq_max) : (uint16_t)0;
    const float scale = (float)__builtin_bit_cast(_Float16, sbits);
    const int qc0 = quant_code(v0 * flip, scale, vq_max);
    const int qc1 = quant_code(v1 * flip, scale, vq_max);
    if (bits == 4) {
      const int code0 = qc0 & 0xF, code1 = qc1 & 0xF;
      // the 4 pairs of a word: bytes hold the pairs (0,1), (4,5), (2,3), (6,7)
      const uint32_t byte = (uint32_t)(code0 | (code1 << 4)) << (8 * byte_of_pair);
      uint32_t word = byte | (uint32_t)__builtin_amdgcn_update_dpp(0, (int)byte, 0xB1, 0xF, 0xF, false);
      word |= (uint32_t)__builtin_amdgcn_update_dpp(0, (int)word, 0x4E, 0xF, 0xF, false);
      if (pq == 0) *reinterpret_cast<uint32_t*>(sl + L.v + 64 * k + 4 * wq) = word;
    } else if (bits == 8) {  // one byte per dim, dim order
      *reinterpret_cast<uint16_t*>(sl + L.v + 128 * k + 2 * lane) =
          (uint16_t)((qc0 & 0xFF) | ((qc1 & 0xFF) << 8));
    } else {  // two bits per dim: lanes 2b and 2b + 1 share byte b
      const int nib = (qc0 & 0x3) | ((qc1 & 0x3) << 2);
      const int other = __builtin_amdgcn_update_dpp(0, nib, 0xB1, 0xF, 0xF, false);  // lane ^ 1
      if ((lane & 1) == 0) sl[L.v + 32 * k + (lane >> 1)] = (uint8_t)(nib | (other << 4));
    }
    if (lane == 0) *reinterpret_cast<uint16_t*>(sl + L.sv + 2 * k) = sbits;
  }
  __syncthreads();

  // ---- coefficients: lane t owns row c_t = U[t][c_k] sigma_k (signed), int8
  if (lane < kPage) {
    double cr[R];
    double amax = 0.0;
#pragma unroll
    for (int k = 0; k < R; ++k) {
      const double f = sig_s[k];
      cr[k] = (f != 0.0) ? u_s[lane][perm_s[k] & (kPage - 1)] * fabs(f) * (f < 0.0 ? -1.0 : 1.0) : 0.0;
      amax = fmax(amax, fabs(cr[k]));
    }
    const uint16_t sbits = amax > 0.0 ? fp16_scale_bits(amax, 127.f) : (uint16_t)0;
    const float scale = (float)__builtin_bit_cast(_Float16, sbits);
#pragma unroll
    for (int k = 0; k < R; ++k) sl[L.c + lane * R + k] = (uint8_t)(quant_code(cr[k], scale, 127) & 0xFF);
    *reinterpret_cast<uint16_t*>(sl + L.sc + 2 * lane) = sbits;
  }

  // ---- centroid: one scale for the page
  {
    const double amax = wave_max_d(fmax(fabs(mu[0]), fabs(mu[1])));
    const uint16_t sbits = amax > 0.0 ? fp16_scale_bits(amax, 127.f) : (uint16_t)0;
    const float scale = (float)__builtin_bit_cast(_Float16, sbits);
    const uint32_t lo = (uint32_t)(quant_code(mu[0], scale, 127) & 0xFF);
    const uint32_t hi = (uint32_t)(quant_code(mu[1], scale, 127) & 0xFF);
    *reinterpret_cast<uint16_t*>(sl + L.mu + 2 * lane) = (uint16_t)(lo | (hi << 8));
    if (lane == 0) *reinterpret_cast<uint16_t*>(sl + L.smu) = sbits;
    for (int p = L.payload + lane; p < L.stride; p += 64) sl[p] = 0;
  }
}

template <int R>
static hipError_t launch_build_page_r(const uint16_t* kpool, int64_t nb, int H, const int32_t* ids,
                                      int n, const int32_t* table, const int32_t* lens, int MP,
                                      uint8_t* summ, const uint16_t* knew, const uint16_t* vnew,
                                      uint16_t* kdst, uint16_t* vdst, int bits, hipStream_t st) {
  const int64_t items = (int64_t)n * H;
  if (items == 0) return hipSuccess;
  hipLaunchKernelGGL(build_page_kernel<R>, dim3((unsigned)items), dim3(64), 0, st, kpool, nb, H, ids,
                     n, table, lens, MP, summ, knew, vnew, kdst, vdst, bits);
  return hipGetLastError();
}

hipError_t launch_build_page(int r, const void* kpool, int64_t nb, int H, const int32_t* ids, int n,
                             const int32_t* table, const int32_t* lens, int MP, void* summ,
                             const void* knew, const void* vnew, void* vpool, int bits,
                             hipStream_t st) {
  const uint16_t* kp = static_cast<const uint16_t*>(kpool);
  uint8_t* sm = static_cast<uint8_t*>(summ);
  const uint16_t* kn = static_cast<const uint16_t*>(knew);
  const uint16_t* vn = static_cast<const uint16_t*>(vnew);
  uint16_t* kd = const_cast<uint16_t*>(kp);
  uint16_t* vd = static_cast<uint16_t*>(vpool);
  switch (r) {
#define LOCKS_R(RR) \
  case RR:          \
    return launch_build_page_r<RR>(kp, nb, H, ids, n, table, lens, MP, sm, kn, vn, kd, vd, bits, st);
    LOCKS_R(1) LOCKS_R(2) LOCKS_R(3) LOCKS_R(4) LOCKS_R(5) LOCKS_R(6) LOCKS_R(7) LOCKS_R(8)
    LOCKS_R(9) LOCKS_R(10) LOCKS_R(11) LOCKS_R(12) LOCKS_R(13) LOCKS_R(14) LOCKS_R(15) LOCKS_R(16)
#undef LOCKS_R
    default:
      return hipErrorInvalidValue;
  }
}

}  // namespace locks
