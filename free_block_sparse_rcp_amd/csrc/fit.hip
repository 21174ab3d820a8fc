// Probe-fitted residual reconstruction: the fit (arxivdaily 2608.18484,
// English abstract: weighted ridge regression of the dense-minus-sparse
// differences of the probe rows on the sparse output; skillfed article and
// peercurrent abstract: an affine map, call-specific, a small linear map from
// the sparse output within the output subspace seen in the probe residuals).
//
// All in fp64, for the m probe rows with s_i the sparse output and
// r_i = o_i - s_i:
//   k_fit_prep (many workgroups per head): w_i = ||o_i||^-2 / sum ||o||^-2,
//     Sigma = sum w_i r_i r_i^T, the Gram G = sum w_i [s_i;1][s_i;1]^T and
//     sum w_i [s_i;1] r_i^T, a block of 8 rows per workgroup;
//   k_fit (one workgroup per head): top-k_eff eigenvectors U of Sigma by
//     Householder tridiagonalisation in LDS, Sturm-count multisection,
//     inverse iteration on the tridiagonal, classical Gram-Schmidt twice and
//     the back-transform through the reflectors. The map's inputs are the
//     subspace coordinates z = U^T s, so its normal equations are those of
//     [z;1] on the targets U^T r: G_z = T^T G T and T^T (sum w [s;1] r^T) U
//     with T = diag(U, 1). The bias is eliminated (its row of the normal
//     equations is exact), leaving (C + lambda_eff I) B = rhs with the
//     weighted covariance C of z and lambda_eff = lambda tr(C) / (k sum w),
//     i.e. lambda times the mean weighted variance of the inputs; B comes
//     from a packed Cholesky factorisation in LDS with forward and backward
//     substitution, the bias from the eliminated row. The map is returned on
//     [s; 1]: Theta = [U B; bias].
#include "common.hpp"
#include "internal.hpp"

namespace spr {

constexpr int kFitThreads = 512;

// Cross-lane moves of a double, 32 bits at a time (the builtins' results go
// through integer casts, as in lane_half_swap): a DPP pattern within rows of
// 16 lanes.
template <int CTRL>
__device__ __forceinline__ double dpp_f64(double v) {
  const uint64_t b = __builtin_bit_cast(uint64_t, v);
  const unsigned lo = (unsigned)__builtin_amdgcn_update_dpp(0, (int)(unsigned)b, CTRL, 0xF, 0xF, false);
  const unsigned hi = (unsigned)__builtin_amdgcn_update_dpp(0, (int)(unsigned)(b >> 32), CTRL, 0xF, 0xF, false);
  return __builtin_bit_cast(double, ((uint64_t)hi << 32) | lo);
}
// v(l & ~B) + v(l | B) in every lane l, B = 16 or 32: the two results of
// v_permlane16_swap / v_permlane32_swap with both operands v are exactly these
// two values, so both lanes of a pair get the same bits.
__device__ __forceinline__ double u64_to_f64(unsigned lo, unsigned hi) {
  return __builtin_bit_cast(double, ((uint64_t)hi << 32) | lo);
}
__device__ __forceinline__ double pair_sum16_f64(double v) {
  const uint64_t b = __builtin_bit_cast(uint64_t, v);
  const unsigned l0 = (unsigned)b, h0 = (unsigned)(b >> 32);
  const auto sl = __builtin_amdgcn_permlane16_swap(l0, l0, false, false);
  const auto sh = __builtin_amdgcn_permlane16_swap(h0, h0, false, false);
  const unsigned la = (unsigned)sl[0], lb = (unsigned)sl[1];
  const unsigned ha = (unsigned)sh[0], hb = (unsigned)sh[1];
  return u64_to_f64(la, ha) + u64_to_f64(lb, hb);
}
__device__ __forceinline__ double pair_sum32_f64(double v) {
  const uint64_t b = __builtin_bit_cast(uint64_t, v);
  const unsigned l0 = (unsigned)b, h0 = (unsigned)(b >> 32);
  const auto sl = __builtin_amdgcn_permlane32_swap(l0, l0, false, false);
  const auto sh = __builtin_amdgcn_permlane32_swap(h0, h0, false, false);
  const unsigned la = (unsigned)sl[0], lb = (unsigned)sl[1];
  const unsigned ha = (unsigned)sh[0], hb = (unsigned)sh[1];
  return u64_to_f64(la, ha) + u64_to_f64(lb, hb);
}

// Sum over each aligned group of 16 lanes; every lane of the group gets the
// same bits (pairwise exchanges within quads, then the half-row and row
// mirrors, which pair lanes whose partial sums already agree).
__device__ __forceinline__ double sum16_f64(double v) {
  v += dpp_f64<0xB1>(v);    // quad_perm [1, 0, 3, 2]
  v += dpp_f64<0x4E>(v);    // quad_perm [2, 3, 0, 1]
  v += dpp_f64<0x141>(v);   // row_half_mirror
  v += dpp_f64<0x140>(v);   // row_mirror
  return v;
}

// Sum over the wave, identical in every lane: rows of 16, then rows r and
// r + 2 (lanes l and l ^ 32), then the two results read from lanes 0 and 16.
__device__ __forceinline__ double wave_sum_f64(double v) {
  v = sum16_f64(v);
  v = pair_sum32_f64(v);
  const uint64_t b = __builtin_bit_cast(uint64_t, v);
  const unsigned a0 = (unsigned)__builtin_amdgcn_readlane((int)(unsigned)b, 0);
  const unsigned a1 = (unsigned)__builtin_amdgcn_readlane((int)(unsigned)(b >> 32), 0);
  const unsigned c0 = (unsigned)__builtin_amdgcn_readlane((int)(unsigned)b, 16);
  const unsigned c1 = (unsigned)__builtin_amdgcn_readlane((int)(unsigned)(b >> 32), 16);
  return __builtin_bit_cast(double, ((uint64_t)a1 << 32) | a0) +
         __builtin_bit_cast(double, ((uint64_t)c1 << 32) | c0);
}

// Workgroup sum with one barrier. The wave partials go to one of two slots
// that alternate between calls: a slot is rewritten only two calls later,
// behind a barrier that every thread reaches after reading it.
constexpr int kFitWaves = kFitThreads / 64;
__device__ __forceinline__ double wg_sum1(double v, double* red2, int& slot) {
  v = wave_sum_f64(v);
  double* red = red2 + slot * kFitWaves;
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  double s = 0.0;
#pragma unroll
  for (int i = 0; i < kFitWaves; ++i) s += red[i];
  slot ^= 1;
  return s;
}
// 1/q from the hardware reciprocal refined by one Newton step: enough for the
// Sturm counts, which use only the signs of their recurrence.
__device__ __forceinline__ double rcp_nr(double q) {
  const double r = __builtin_amdgcn_rcp(q);
  return fma(r, fma(-q, r, 1.0), r);
}

// A second Newton step (the error squares again), for the multipliers and
// pivots of the inverse iteration.
__device__ __forceinline__ double rcp_nr2(double q) {
  const double r = rcp_nr(q);
  return fma(r, fma(-q, r, 1.0), r);
}

// Number of eigenvalues of the symmetric tridiagonal (a, b) below x, counted
// as the negative pivots of the LDL^T factorisation of T - x I (tiny pivots
// replaced by -pivmin).
__device__ int sturm_count(const double* a, const double* b2, int n, double x, double pivmin) {
  int cnt = 0;
  double q = a[0] - x;
  if (fabs(q) < pivmin) q = -pivmin;
  cnt += q < 0.0;
  for (int i = 1; i < n; ++i) {
    q = (a[i] - x) - b2[i - 1] * rcp_nr(q);
    if (fabs(q) < pivmin) q = -pivmin;
    cnt += q < 0.0;
  }
  return cnt;
}

// Per-head scratch layout (doubles) in the workspace.
struct FitScratch {
  double *sig, *gram, *xtwr, *hv, *rhs;
};
__host__ __device__ inline size_t fit_doubles_per_head(int m, int D, int k) {
  const size_t NX = (size_t)D + 1;
  (void)m;
  return (size_t)D * D + NX * NX + NX * D + (size_t)D * D + NX * (size_t)(k > 0 ? k : 1) + 64;
}
__device__ inline FitScratch fit_scratch(double* base, int m, int D, int k) {
  const size_t NX = (size_t)D + 1;
  (void)m;
  (void)k;
  FitScratch f;
  f.sig = base;
  f.gram = f.sig + (size_t)D * D;
  f.xtwr = f.gram + NX * NX;
  f.hv = f.xtwr + NX * D;
  f.rhs = f.hv + (size_t)D * D;
  return f;
}

__device__ __forceinline__ double row_inv_norm2(const float* row, int D) {
  double n2 = 0.0;
  for (int e = 0; e < D; ++e) {
    const double o = row[e];
    n2 += o * o;
  }
  return n2 > 0.0 ? 1.0 / n2 : 0.0;
}

// ---------------------------------------------------------------- prep
// grid (H, ceil((d+1)/8)), block 512. Workgroup b accumulates rows [8b, 8b+8)
// of Sigma (rows < d), of sum w [s;1] r^T and of the Gram (rows < d+1) over
// chunks of 256 probe rows staged in LDS. S_probe row i is s_i (fp32).
template <int D>
__global__ __launch_bounds__(kFitThreads) void k_fit_prep(const float* S_probe, const float* O_probe,
                                                          int m, int kmax, double* scratch) {
  constexpr int NT = kFitThreads;
  constexpr int NX = D + 1;
  constexpr int RB = 8;
  constexpr int CH = 256;          // probe rows per chunk
  __shared__ double ra[CH][RB];    // w_i * r_i[a] for the block's rows a
  __shared__ double xa[CH][RB];    // w_i * x_i[a]
  __shared__ double w_s[CH];
  __shared__ double red2[2 * NT / 64];
  const int h = blockIdx.x, b = blockIdx.y, t = threadIdx.x;
  const float* Sh = S_probe + (size_t)h * m * D;
  const float* Op = O_probe + (size_t)h * m * D;
  FitScratch f = fit_scratch(scratch + (size_t)h * fit_doubles_per_head(m, D, kmax), m, D, kmax);
  int slot = 0;
  double wpart = 0.0;
  for (int i = t; i < m; i += NT) wpart += row_inv_norm2(Op + (size_t)i * D, D);
  const double wsum = wg_sum1(wpart, red2, slot);
  const int a0 = RB * b;
  for (int i0 = 0; i0 < m; i0 += CH) {
    const int mi = min(CH, m - i0);
    __syncthreads();
    if (t < mi) {
      const double wi = row_inv_norm2(Op + (size_t)(i0 + t) * D, D);
      w_s[t] = wsum > 0.0 ? wi / wsum : 0.0;
    }
    __syncthreads();
    for (int idx = t; idx < mi * RB; idx += NT) {
      const int i = idx / RB, u = idx % RB, a = a0 + u;
      double rv = 0.0, xv = 0.0;
      if (a < D) {
        const double s = Sh[(size_t)(i0 + i) * D + a];
        rv = (double)Op[(size_t)(i0 + i) * D + a] - s;
        xv = s;
      } else if (a == D) {
        xv = 1.0;
      }
      ra[i][u] = w_s[i] * rv;
      xa[i][u] = w_s[i] * xv;
    }
    __syncthreads();
    // jobs: Sigma columns [0, D), X^T W R columns [D, 2D), Gram columns [2D, 2D + NX)
    for (int job = t; job < 2 * D + NX; job += NT) {
      const int kind = job < D ? 0 : (job < 2 * D ? 1 : 2);
      const int c = kind == 0 ? job : (kind == 1 ? job - D : job - 2 * D);
      double acc[RB];
#pragma unroll
      for (int u = 0; u < RB; ++u) acc[u] = 0.0;
      for (int i = 0; i < mi; ++i) {
        double col;
        if (kind == 2) col = c < D ? (double)Sh[(size_t)(i0 + i) * D + c] : 1.0;
        else col = (double)Op[(size_t)(i0 + i) * D + c] - (double)Sh[(size_t)(i0 + i) * D + c];
        const double* rowv = kind == 0 ? ra[i] : xa[i];
#pragma unroll
        for (int u = 0; u < RB; ++u) acc[u] += rowv[u] * col;
      }
#pragma unroll
      for (int u = 0; u < RB; ++u) {
        const int a = a0 + u;
        double* dst = nullptr;
        if (kind == 0) dst = a < D ? f.sig + (size_t)a * D + c : nullptr;
        else if (kind == 1) dst = a < NX ? f.xtwr + (size_t)a * D + c : nullptr;
        else dst = a < NX ? f.gram + (size_t)a * NX + c : nullptr;
        if (dst == nullptr) continue;
        *dst = (i0 == 0 ? 0.0 : *dst) + acc[u];
      }
    }
  }
}

// ---------------------------------------------------------------- fit
template <int D>
__global__ __launch_bounds__(kFitThreads) void k_fit(int m, int kmax, double lambda, float* U_out,
                                                     float* Th_out, int32_t* rank_eff,
                                                     double* scratch) {
  constexpr int NT = kFitThreads;
  constexpr int PA = D + 1;                // pitch of the eigen matrix
  constexpr int NX = D + 1;                // rows of the Gram on [s; 1]
  constexpr int BIG = (D + 1) * (D + 2);
  __shared__ double big[BIG];
  __shared__ double dg[D], od[D], od2[D], beta[D], vv[D], pv[D];
  __shared__ double lam_top[D + 1];   // eigenvalues, later 1 / L_ii of the ridge factor
  __shared__ double red2[2 * NT / 64];
  __shared__ double dots[D];
  constexpr int NSEG = NT / D;             // segments of the Householder product
  static_assert(NSEG >= 1 && NT % D == 0, "threads must cover whole rows");
  __shared__ double pseg[NSEG > 1 ? NSEG - 1 : 1][D];
  const int h = blockIdx.x, t = threadIdx.x;
  float* Uh = U_out + (size_t)h * D * kmax;
  float* Th = Th_out + (size_t)h * (D + 1) * kmax;
  const int keff = min(kmax, min(m, D));
  FitScratch f = fit_scratch(scratch + (size_t)h * fit_doubles_per_head(m, D, kmax), m, D, kmax);
  int slot = 0;

  for (int i = t; i < D * kmax; i += NT) Uh[i] = 0.f;
  for (int i = t; i < (D + 1) * kmax; i += NT) Th[i] = 0.f;
  if (keff <= 0) {
    if (t == 0) rank_eff[h] = 0;
    return;
  }
  double* A = big;
  for (int idx = t; idx < D * D; idx += NT) A[(idx / D) * PA + idx % D] = f.sig[idx];
  __syncthreads();
  double trpart = 0.0;
  for (int i = t; i < D; i += NT) trpart += A[i * PA + i];
  const double trace = wg_sum1(trpart, red2, slot);
  if (!(trace > 0.0)) {
    if (t == 0) rank_eff[h] = 0;
    return;
  }
  // ---- Householder tridiagonalisation on the lower triangle of A (the upper
  // triangle is not read after the copy); reflector k is stored in column k
  // below the diagonal. Three barriers per step: the sum v^T p, q ready, and
  // the end of the update, whose sum carries the next column's squared norm.
  constexpr int NC = D / 32;   // update columns per thread (registers)
  double sig2;
  {
    double part = 0.0;
    for (int i = 2 + t; i < D; i += NT) {
      const double x = A[i * PA];
      part += x * x;
    }
    sig2 = wg_sum1(part, red2, slot);
  }
  for (int k = 0; k < D - 2; ++k) {
    const int L = D - k - 1;
    const double x0 = A[(k + 1) * PA + k];
    if (sig2 == 0.0) {
      if (t == 0) {
        beta[k] = 0.0;
        od[k] = x0;
      }
      // nothing is updated in this step; the next column's norm is read directly
      double part = 0.0;
      for (int i = k + 3 + t; i < D; i += NT) {
        const double x = A[i * PA + k + 1];
        part += x * x;
      }
      sig2 = wg_sum1(part, red2, slot);
      continue;
    }
    const double alpha = -copysign(sqrt(x0 * x0 + sig2), x0);
    const double v0 = x0 - alpha;
    const double bk = 2.0 / (v0 * v0 + sig2);
    // p = beta A22 v with v_0 = v0, v_j = A[k+1+j][k]; entry (i, j) of A22 is
    // read from row max(i, j), column min(i, j). Row i of the product is split
    // over NSEG waves by segments of j; v^T p comes from the partials directly.
    const int i = t & (D - 1), seg = t / D;
    const int jm = (L + NSEG - 1) / NSEG;
    double* A22 = A + (k + 1) * PA + (k + 1);
    double s = 0.0;
    if (i < L) {
      const int j0 = min(L, seg * jm), j1 = min(L, j0 + jm);
      // four independent partial sums keep several LDS reads in flight
      double s4[4] = {0.0, 0.0, 0.0, 0.0};
      int j = j0;
      if (j == 0) {
        s4[0] = A22[i * PA] * v0;
        j = 1;
      }
      for (; j + 3 < j1; j += 4) {
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int jj = j + u;
          const int r = max(i, jj), c = min(i, jj);
          s4[u] += A22[r * PA + c] * A[(k + 1 + jj) * PA + k];
        }
      }
      for (; j < j1; ++j) {
        const int r = max(i, j), c = min(i, j);
        s4[0] += A22[r * PA + c] * A[(k + 1 + j) * PA + k];
      }
      s = (s4[0] + s4[1]) + (s4[2] + s4[3]);
    }
    const double v_i = i == 0 ? v0 : (i < L ? A[(k + 1 + i) * PA + k] : 0.0);
    if (seg > 0 && i < L) pseg[seg - 1][i] = s;   // partials of the later segments
    const double vp = i < L ? v_i * bk * s : 0.0;
    const double K = 0.5 * bk * wg_sum1(vp, red2, slot);
    if (seg == 0 && i < L) {
      double st = s;
#pragma unroll
      for (int q = 0; q < NSEG - 1; ++q) st += pseg[q][i];
      const double p_i = bk * st;
      pv[i] = p_i - K * v_i;   // q
      vv[i] = v_i;
    }
    if (t == 0) {
      beta[k] = bk;
      od[k] = alpha;
      A[(k + 1) * PA + k] = v0;   // x0 and the column are no longer read in this step
    }
    __syncthreads();
    // A22 -= v q^T + q v^T on the lower triangle: a thread keeps v and q of its
    // columns jc + 32 c and of its rows t / 32 + 16 r in registers, and reads
    // all of its old values before writing any. Column 0 of A22 (rows 2..) is
    // the next step's column; its squared norm is summed here.
    {
      constexpr int RM = D / 16;   // rows per thread at most
      static_assert(NT / 32 == 16, "16 row groups");
      const int jc = t & 31, i20 = t >> 5;
      double vcol[NC], qcol[NC], vrow[RM], qrow[RM], old[RM][NC];
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        const int j2 = jc + 32 * c;
        vcol[c] = j2 < L ? vv[j2] : 0.0;
        qcol[c] = j2 < L ? pv[j2] : 0.0;
      }
#pragma unroll
      for (int r = 0; r < RM; ++r) {
        const int i2 = i20 + 16 * r;
        vrow[r] = i2 < L ? vv[i2] : 0.0;
        qrow[r] = i2 < L ? pv[i2] : 0.0;
#pragma unroll
        for (int c = 0; c < NC; ++c) {
          const int j2 = jc + 32 * c;
          old[r][c] = (i2 < L && j2 <= i2) ? A22[i2 * PA + j2] : 0.0;
        }
      }
      double part = 0.0;
#pragma unroll
      for (int r = 0; r < RM; ++r) {
        const int i2 = i20 + 16 * r;
#pragma unroll
        for (int c = 0; c < NC; ++c) {
          const int j2 = jc + 32 * c;
          if (i2 < L && j2 <= i2) {
            const double nv = old[r][c] - (vrow[r] * qcol[c] + qrow[r] * vcol[c]);
            A22[i2 * PA + j2] = nv;
            if (c == 0 && jc == 0 && i2 >= 2) part += nv * nv;
          }
        }
      }
      sig2 = wg_sum1(part, red2, slot);
    }
  }
  for (int i = t; i < D; i += NT) dg[i] = A[i * PA + i];
  if (t == 0) {
    od[D - 2] = A[(D - 1) * PA + (D - 2)];
    od[D - 1] = 0.0;
  }
  __syncthreads();
  for (int i = t; i < D; i += NT) od2[i] = od[i] * od[i];
  __syncthreads();
  // ---- eigenvalues r = 0..keff-1 from the top by multisection of the
  // Gershgorin interval with Sturm counts
  double glo = 1e300, ghi = -1e300, maxb2 = 0.0, tnorm = 0.0;
  for (int i = 0; i < D; ++i) {
    const double bl = i > 0 ? fabs(od[i - 1]) : 0.0;
    const double br = i < D - 1 ? fabs(od[i]) : 0.0;
    glo = fmin(glo, dg[i] - bl - br);
    ghi = fmax(ghi, dg[i] + bl + br);
    maxb2 = fmax(maxb2, od2[i]);
    tnorm = fmax(tnorm, fabs(dg[i]) + bl + br);
  }
  const double pivmin = 2.2250738585072014e-308 * fmax(1.0, maxb2);
  const double pad = 2.2e-16 * fmax(tnorm, 1e-300) + pivmin;
  glo -= pad;
  ghi += pad;
  // P-point multisection per eigenvalue, one point per thread: P the largest
  // power of two with P keff <= NT (at most 32), so one pass covers every
  // eigenvalue. The interval shrinks by (P + 1)^iters > 2^40 (the eigenvalues
  // serve only as inverse-iteration shifts); the new bracket comes from a
  // ballot of the points' sides of the eigenvalue.
  int P = 32;
  while (P * keff > NT) P >>= 1;
  const int iters = P == 32 ? 8 : (P == 16 ? 10 : (P == 8 ? 13 : 18));
  {
    const int r = t / P, sub = t % P;
    const int j = D - 1 - (r < keff ? r : 0);  // ascending eigenvalue index
    const int gl = (t & 63) & ~(P - 1);        // the group's first lane in the wave
    const uint64_t pmask = P == 32 ? 0xffffffffull : ((1ull << P) - 1);
    const double dp = (double)(P + 1);
    double lo = glo, hi = ghi;
    for (int iter = 0; iter < iters; ++iter) {
      const double w = hi - lo;
      const double x = lo + w * (double)(sub + 1) / dp;
      const int cnt = sturm_count(dg, od2, D, x, pivmin);
      // bit s: point s (x = lo + w (s + 1) / (P + 1)) lies left of the eigenvalue
      const uint64_t left = (__ballot(cnt <= j) >> gl) & pmask;
      const uint64_t right = ~left & pmask;
      double nlo = lo, nhi = hi;
      if (left) nlo = fmax(nlo, lo + w * (double)(64 - __clzll((long long)left)) / dp);
      if (right) nhi = fmin(nhi, lo + w * (double)__ffsll((long long)right) / dp);
      lo = nlo;
      hi = nhi;
    }
    if (r < keff && sub == 0) lam_top[r] = 0.5 * (lo + hi);
  }
  __syncthreads();
  // ---- reflectors to the workspace, one per row (reflector k at [k][e], zero
  // for e <= k); the LDS block is reused from here on
  for (int idx = t; idx < (D - 2) * D; idx += NT) {
    const int k = idx / D, e = idx % D;
    f.hv[idx] = e > k ? A[e * PA + k] : 0.0;
  }
  __syncthreads();
  // ---- inverse iteration on the tridiagonal, one thread per eigenvector,
  // factors in LDS interleaved across the batch ([i][r]) so lanes hit distinct
  // banks; the vectors collect in the rhs scratch ([e][r], pitch kmax)
  const double pe = 2.2e-16 * fmax(tnorm, 1e-300);
  constexpr int KB = D / 4;   // 4 arrays of D x KB doubles fit the LDS block
  static_assert(4 * D * KB <= BIG, "inverse-iteration batch exceeds LDS");
  double* Xg = f.rhs;
  for (int b0 = 0; b0 < keff; b0 += KB) {
    const int nbt = min(KB, keff - b0);
    double* U1 = big;
    double* U2 = U1 + D * KB;
    double* U3 = U2 + D * KB;
    double* Z = U3 + D * KB;
    if (t < nbt) {
      const int r = b0 + t;
      const double lam = lam_top[r];
      for (int i = 0; i < D; ++i) {
        const uint32_t hsh = (uint32_t)(i * 2654435761u) ^ (uint32_t)(r * 40503u + 12345u);
        Z[i * KB + t] = 0.5 + (double)(hsh % 1000u) / 1000.0;
      }
      // three passes; a pass's normalisation is applied as the next pass (or
      // the copy out) reads the vector
      double inv = 1.0;
      for (int pass = 0; pass < 3; ++pass) {
        // LU with partial pivoting of T - lam I; U1 keeps the reciprocal pivots.
        // The next right-hand-side entry is read one step ahead.
        double cd = dg[0] - lam, cu = od[0], cu2 = 0.0, cr = Z[t] * inv;
        double znext = Z[KB + t];
        for (int i = 0; i < D - 1; ++i) {
          const double nl = od[i], nd = dg[i + 1] - lam, nu = (i + 1 < D - 1) ? od[i + 1] : 0.0;
          const double nr = znext * inv;
          if (i + 2 < D) znext = Z[(i + 2) * KB + t];
          const bool keep = fabs(cd) >= fabs(nl);   // no row swap
          if (keep && cd == 0.0) cd = pe;
          const double rp = rcp_nr2(keep ? cd : nl);
          if (keep) {
            const double mlt = nl * rp;
            U1[i * KB + t] = rp; U2[i * KB + t] = cu; U3[i * KB + t] = cu2; Z[i * KB + t] = cr;
            cd = nd - mlt * cu;
            cu = nu - mlt * cu2;
            cu2 = 0.0;
            cr = nr - mlt * cr;
          } else {
            const double mlt = cd * rp;
            U1[i * KB + t] = rp; U2[i * KB + t] = nd; U3[i * KB + t] = nu; Z[i * KB + t] = nr;
            const double ncd = cu - mlt * nd;
            const double ncu = cu2 - mlt * nu;
            cr = cr - mlt * nr;
            cd = ncd;
            cu = ncu;
            cu2 = 0.0;
          }
        }
        if (fabs(cd) < pe) cd = cd < 0.0 ? -pe : pe;
        double y1 = cr * rcp_nr2(cd), y2 = 0.0;
        double nrm = y1 * y1;
        Z[(D - 1) * KB + t] = y1;
        // back substitution, the factors of the next row read one step ahead
        double zn = Z[(D - 2) * KB + t], u1n = U1[(D - 2) * KB + t];
        double u2n = U2[(D - 2) * KB + t], u3n = U3[(D - 2) * KB + t];
        for (int i = D - 2; i >= 0; --i) {
          const double zi = zn, u1 = u1n, u2 = u2n, u3 = u3n;
          if (i > 0) {
            zn = Z[(i - 1) * KB + t];
            u1n = U1[(i - 1) * KB + t];
            u2n = U2[(i - 1) * KB + t];
            u3n = U3[(i - 1) * KB + t];
          }
          const double y = (zi - u2 * y1 - u3 * y2) * u1;
          Z[i * KB + t] = y;
          nrm += y * y;
          y2 = y1;
          y1 = y;
        }
        inv = 1.0 / sqrt(nrm);
      }
      dots[t] = inv;   // the last pass's normalisation, applied on the copy out
    }
    __syncthreads();
    for (int idx = t; idx < D * nbt; idx += NT) {
      const int i = idx / nbt, r = idx % nbt;
      Xg[(size_t)i * kmax + b0 + r] = Z[i * KB + r] * dots[r];
    }
    __syncthreads();
  }
  // ---- eigenvector block in LDS: X[e][r], pitch keff + 1
  const int PXK = keff + 1;
  double* X = big;
  for (int idx = t; idx < D * keff; idx += NT) {
    const int e = idx / keff, r = idx % keff;
    X[e * PXK + r] = Xg[(size_t)e * kmax + r];
  }
  __syncthreads();
  // ---- classical Gram-Schmidt, twice, in eigenvalue order, by wave 0 alone
  // (wave-ordered LDS, no workgroup barriers): 16 lanes per column, rows
  // part + 16 u; every lane group holds the column being orthogonalised and
  // the four groups take the earlier columns in turn.
  constexpr int NR = D / 16;
  if (t < 64) {
    const int g = t >> 4, part = t & 15;
    for (int j = 1; j < keff; ++j) {
      double xj[NR];
#pragma unroll
      for (int u = 0; u < NR; ++u) xj[u] = X[(part + 16 * u) * PXK + j];
      for (int pass = 0; pass < 2; ++pass) {
        double acc[NR];
#pragma unroll
        for (int u = 0; u < NR; ++u) acc[u] = 0.0;
        // four earlier columns per lane group at a time: 16 per round
        for (int i0 = 0; i0 < j; i0 += 16) {
          double xc[4][NR], sc[4];
          // unconditional loads (a valid column in place of a missing one),
          // then the missing columns zeroed
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int ic = i0 + 4 * q + g;
            const int icl = ic < j ? ic : 0;
#pragma unroll
            for (int u = 0; u < NR; ++u) {
              const double x = X[(part + 16 * u) * PXK + icl];
              xc[q][u] = ic < j ? x : 0.0;
            }
          }
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            sc[q] = 0.0;
#pragma unroll
            for (int u = 0; u < NR; ++u) sc[q] += xc[q][u] * xj[u];
          }
#pragma unroll
          for (int q = 0; q < 4; ++q) sc[q] = sum16_f64(sc[q]);
#pragma unroll
          for (int u = 0; u < NR; ++u)
#pragma unroll
            for (int q = 0; q < 4; ++q) acc[u] += sc[q] * xc[q][u];
        }
#pragma unroll
        for (int u = 0; u < NR; ++u) {
          acc[u] = pair_sum32_f64(pair_sum16_f64(acc[u]));
          xj[u] -= acc[u];
        }
      }
      double n2 = 0.0;
#pragma unroll
      for (int u = 0; u < NR; ++u) n2 += xj[u] * xj[u];
      const double nrm = sqrt(sum16_f64(n2));
      if (g == 0) {
#pragma unroll
        for (int u = 0; u < NR; ++u) X[(part + 16 * u) * PXK + j] = xj[u] / nrm;
      }
      // the next column reads this one: keep the LDS accesses in program order
      __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    }
  }
  __syncthreads();
  // ---- back-transform through the reflectors: X <- H_0 H_1 ... H_{D-3} X.
  // Each wave applies every reflector to its own columns (16 lanes per column,
  // rows part + 16 u, in registers); the reflectors are read from LDS, so the
  // loop has no workgroup barriers.
  {
    constexpr int NPM = D / 32;   // column slots per lane (keff <= D)
    const int lane = t & 63, wv = t >> 6, g = lane >> 4, part = lane & 15;
    const int npass = (keff + 31) / 32;
    double xr[NPM][NR];
#pragma unroll
    for (int pp = 0; pp < NPM; ++pp) {
      const int c = 32 * pp + 4 * wv + g;
#pragma unroll
      for (int u = 0; u < NR; ++u) xr[pp][u] = c < keff ? X[(part + 16 * u) * PXK + c] : 0.0;
    }
    __syncthreads();
    double* HV = big;   // reflector k at HV[k * D + e]
    for (int idx = t; idx < (D - 2) * D; idx += NT) HV[idx] = f.hv[idx];
    __syncthreads();
    for (int k = D - 3; k >= 0; --k) {
      const double bk = beta[k];
      if (bk == 0.0) continue;
      double vr[NR];
#pragma unroll
      for (int u = 0; u < NR; ++u) vr[u] = HV[k * D + part + 16 * u];
#pragma unroll
      for (int pp = 0; pp < NPM; ++pp) {
        if (pp < npass) {
          double s = 0.0;
#pragma unroll
          for (int u = 0; u < NR; ++u) s += vr[u] * xr[pp][u];
          const double dc = bk * sum16_f64(s);
#pragma unroll
          for (int u = 0; u < NR; ++u) xr[pp][u] -= dc * vr[u];
        }
      }
    }
    __syncthreads();
#pragma unroll
    for (int pp = 0; pp < NPM; ++pp) {
      const int c = 32 * pp + 4 * wv + g;
      if (c < keff) {
#pragma unroll
        for (int u = 0; u < NR; ++u) X[(part + 16 * u) * PXK + c] = xr[pp][u];
      }
    }
    __syncthreads();
  }
  for (int idx = t; idx < D * keff; idx += NT) {
    const int e = idx / keff, cc = idx % keff;
    Uh[(size_t)e * kmax + cc] = (float)X[e * PXK + cc];
  }
  // U in fp64 to the workspace (pitch keff): the reflectors are no longer needed
  for (int idx = t; idx < D * keff; idx += NT) f.hv[idx] = X[(idx / keff) * PXK + idx % keff];
  // ---- products with U in 4 x 4 register tiles: rows [0, D] of
  // F = (sum w [s;1] r^T) U into rhs (pitch kmax), and rows [0, D) of
  // H = G[:, 0:D] U into sig (pitch keff); row D of H is the bias column g
  {
    const int ntr = (NX + 3) / 4, ntc = (keff + 3) / 4;
    for (int tile = t; tile < 2 * ntr * ntc; tile += NT) {
      const bool isF = tile < ntr * ntc;
      const int tt = isF ? tile : tile - ntr * ntc;
      const int r0 = 4 * (tt / ntc), c0 = 4 * (tt % ntc);
      const double* src = isF ? f.xtwr : f.gram;
      const int pitch = isF ? D : NX;
      double acc[4][4];
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int v = 0; v < 4; ++v) acc[u][v] = 0.0;
      // unrolled so that many workspace loads are in flight at once
#pragma unroll 8
      for (int e = 0; e < D; ++e) {
        double xr[4], uc[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) xr[u] = r0 + u < NX ? src[(size_t)(r0 + u) * pitch + e] : 0.0;
#pragma unroll
        for (int v = 0; v < 4; ++v) uc[v] = c0 + v < keff ? X[e * PXK + c0 + v] : 0.0;
#pragma unroll
        for (int u = 0; u < 4; ++u)
#pragma unroll
          for (int v = 0; v < 4; ++v) acc[u][v] += xr[u] * uc[v];
      }
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const int r = r0 + u, c = c0 + v;
          if (r >= NX || c >= keff) continue;
          if (isF) f.rhs[(size_t)r * kmax + c] = acc[u][v];
          else if (r < D) f.sig[(size_t)r * keff + c] = acc[u][v];
          else dots[c] = acc[u][v];     // g_c = sum_i G[D][i] U[i][c]
        }
    }
  }
  __syncthreads();
  // ---- the bias-eliminated system in LDS (X is dead from here on):
  //   C   = U^T H - g g^T / G_DD          packed lower triangle, keff rows
  //   rhs = U^T F[0:D] - g F[D] / G_DD    keff x keff (in LDS when it fits)
  const int NPZ = keff * (keff + 1) / 2;
  const bool rhs_lds = NPZ + keff * keff <= BIG;
  double* rz = rhs_lds ? big + NPZ : f.xtwr;   // sum w [s;1] r^T is no longer read
  const double gdd = f.gram[(size_t)D * NX + D];   // sum of the weights
  const double igdd = gdd > 0.0 ? 1.0 / gdd : 0.0;
  for (int job = t; job < NPZ + keff * keff; job += NT) {
    int a, b;
    const bool isC = job < NPZ;
    if (isC) {
      a = (int)((sqrt(8.0 * job + 1.0) - 1.0) * 0.5);
      while (a * (a + 1) / 2 > job) --a;
      while ((a + 1) * (a + 2) / 2 <= job) ++a;
      b = job - a * (a + 1) / 2;
    } else {
      a = (job - NPZ) / keff;
      b = (job - NPZ) % keff;
    }
    const double* col = isC ? f.sig : f.rhs;
    const int pitch = isC ? keff : kmax;
    double s2[2] = {0.0, 0.0};
#pragma unroll 4
    for (int e = 0; e < D; e += 2) {
      s2[0] += f.hv[(size_t)e * keff + a] * col[(size_t)e * pitch + b];
      s2[1] += f.hv[(size_t)(e + 1) * keff + a] * col[(size_t)(e + 1) * pitch + b];
    }
    const double tail = isC ? dots[b] : f.rhs[(size_t)D * kmax + b];
    const double v = (s2[0] + s2[1]) - dots[a] * tail * igdd;
    if (isC) big[job] = v;
    else rz[(size_t)a * keff + b] = v;
  }
  __syncthreads();
  // ---- penalty: lambda times the mean weighted variance of the inputs. An
  // input set without spread (trace of C at the rounding level of the
  // uncentred Gram) leaves the slopes at 0 and the bias at the weighted mean.
  double trc_part = 0.0, trg_part = 0.0;
  for (int a = t; a < keff; a += NT) {
    trc_part += big[a * (a + 1) / 2 + a];
    trg_part += big[a * (a + 1) / 2 + a] + dots[a] * dots[a] * igdd;
  }
  const double trc = wg_sum1(trc_part, red2, slot);
  const double trg = wg_sum1(trg_part, red2, slot);
  const bool spread = trc > 64.0 * 2.220446049250313e-16 * trg && gdd > 0.0;
  if (spread) {
    const double lam_eff = lambda * trc * igdd / (double)keff;
    for (int a = t; a < keff; a += NT) big[a * (a + 1) / 2 + a] += lam_eff;
  } else {
    for (int idx = t; idx < keff * keff; idx += NT) rz[idx] = 0.0;
  }
  __syncthreads();
  if (spread) {
    // ---- Cholesky, right-looking, one barrier per column: the trailing
    // update uses the unscaled column j and 1/d_j; column j is scaled in the
    // next step, when it is no longer read.
    double dprev = 1.0;
    for (int j = 0; j < keff; ++j) {
      double dj = big[j * (j + 1) / 2 + j];
      dj = dj > 0.0 ? dj : 1e-300;
      const double rd = 1.0 / dj;
      if (j > 0) {
        const double sc = 1.0 / sqrt(dprev);
        for (int i = j + t; i < keff; i += NT) big[i * (i + 1) / 2 + (j - 1)] *= sc;
        if (t == 0) big[(j - 1) * j / 2 + (j - 1)] = sqrt(dprev);
      }
      for (int i = j + 1 + (t >> 5); i < keff; i += NT / 32) {
        double* row = big + i * (i + 1) / 2;
        const double lij = row[j] * rd;
        for (int l = j + 1 + (t & 31); l <= i; l += 32) row[l] -= lij * big[l * (l + 1) / 2 + j];
      }
      dprev = dj;
      __syncthreads();
    }
    if (t == 0) big[(keff - 1) * keff / 2 + (keff - 1)] = sqrt(dprev);
    __syncthreads();
    double* rdiag = lam_top;   // free again: 1 / L_ii for the substitutions
    for (int i = t; i < keff; i += NT) rdiag[i] = 1.0 / big[i * (i + 1) / 2 + i];
    __syncthreads();
    // ---- L y = b, then L^T x = y: sixteen lanes per right-hand-side column,
    // each column handled by one wave, so only wave-level ordering is needed
    constexpr int LPC = 16;                    // lanes per column
    constexpr int NU = (D + LPC - 1) / LPC;    // terms per lane at most
    const int lane = t & 63, wv = t >> 6;
    const int part = lane & (LPC - 1);
    for (int cb = 0; cb < keff; cb += (64 / LPC) * (NT / 64)) {
      const int cc = cb + (64 / LPC) * wv + lane / LPC;
      const bool on = cc < keff;
      for (int i = 0; i < keff; ++i) {
        double sacc = 0.0;
        if (on) {
          const double* row = big + i * (i + 1) / 2;
          // all of the lane's terms are read at once (one LDS round trip)
          double s2[2] = {0.0, 0.0};
#pragma unroll
          for (int u = 0; u < NU; ++u) {
            const int l = part + u * LPC;
            if (l < i) s2[u & 1] += row[l] * rz[(size_t)l * keff + cc];
          }
          sacc = s2[0] + s2[1];
        }
        sacc = sum16_f64(sacc);
        if (on && part == 0) rz[(size_t)i * keff + cc] = (rz[(size_t)i * keff + cc] - sacc) * rdiag[i];
        if (rhs_lds) __builtin_amdgcn_wave_barrier();
        else __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "workgroup");
      }
      for (int i = keff - 1; i >= 0; --i) {
        double sacc = 0.0;
        if (on) {
          double s2[2] = {0.0, 0.0};
#pragma unroll
          for (int u = 0; u < NU; ++u) {
            const int l = i + 1 + part + u * LPC;
            if (l < keff) s2[u & 1] += big[l * (l + 1) / 2 + i] * rz[(size_t)l * keff + cc];
          }
          sacc = s2[0] + s2[1];
        }
        sacc = sum16_f64(sacc);
        if (on && part == 0) rz[(size_t)i * keff + cc] = (rz[(size_t)i * keff + cc] - sacc) * rdiag[i];
        if (rhs_lds) __builtin_amdgcn_wave_barrier();
        else __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "workgroup");
      }
    }
    __syncthreads();
  }
  // ---- the map on [s; 1]: slopes U B (rows < D), bias (F[D] - g^T B) / G_DD
  for (int idx = t; idx < NX * keff; idx += NT) {
    const int r = idx / keff, cc = idx % keff;
    double v = 0.0;
    if (r < D) {
#pragma unroll 8
      for (int a = 0; a < keff; ++a) v += f.hv[(size_t)r * keff + a] * rz[(size_t)a * keff + cc];
    } else {
      double gb = 0.0;
      for (int a = 0; a < keff; ++a) gb += dots[a] * rz[(size_t)a * keff + cc];
      v = (f.rhs[(size_t)D * kmax + cc] - gb) * igdd;
    }
    Th[(size_t)r * kmax + cc] = (float)v;
  }
  if (t == 0) rank_eff[h] = keff;
}

size_t fit_ws_per_head(const Dims& d) {
  return fit_doubles_per_head(d.m, d.D, d.k) * sizeof(double);
}

hipError_t launch_fit(const Dims& d, const float* S_probe, const float* O_probe, float* U,
                      float* Theta, int32_t* rank_eff, char* fit_ws, hipStream_t st) {
  double* scratch = reinterpret_cast<double*>(fit_ws);
  const dim3 pgrid(d.H, (d.D + 1 + 7) / 8);
#define SPR_FIT(DD)                                                                         \
  do {                                                                                      \
    k_fit_prep<DD><<<pgrid, kFitThreads, 0, st>>>(S_probe, O_probe, d.m, d.k, scratch);     \
    k_fit<DD><<<d.H, kFitThreads, 0, st>>>(d.m, d.k, d.lam, U, Theta, rank_eff, scratch);   \
  } while (0)
  if (d.D == 128) SPR_FIT(128);
  else SPR_FIT(64);
#undef SPR_FIT
  return hipGetLastError();
}

}  // namespace spr
