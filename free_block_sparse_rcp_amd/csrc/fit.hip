// Probe-fitted residual reconstruction: the fit (arxivdaily 2608.18484,
// English abstract: weighted ridge regression of the dense-minus-sparse
// differences of the probe rows on the sparse output; skillfed article and
// peercurrent abstract: an affine map, call-specific, restricted to the output
// subspace seen in the probe residuals).
//
// All in fp64, with X = [s, 1] and r_i = o_i - s_i for the m probe rows:
//   k_fit_prep (many workgroups per head): w_i = ||o_i||^-2 / sum ||o||^-2,
//     Sigma = sum w_i r_i r_i^T, the ridge Gram X^T W X + lambda I~ (bias row
//     unpenalised) and X^T W R, a block of 8 rows per workgroup;
//   k_fit (one workgroup per head): top-k_eff eigenvectors U of Sigma by
//     Householder tridiagonalisation in LDS, Sturm-count multisection,
//     inverse iteration on the tridiagonal, classical Gram-Schmidt twice and
//     the back-transform through the reflectors; then the right-hand side
//     X^T W (R U) = (X^T W R) U and Theta by a packed Cholesky factorisation
//     in LDS with forward and backward substitution.
#include "common.hpp"
#include "internal.hpp"

namespace spr {

constexpr int kFitThreads = 512;

__device__ __forceinline__ double wave_sum_f64(double v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

// Workgroup sum with one barrier. The wave partials go to one of two slots
// that alternate between calls: a slot is rewritten only two calls later,
// behind a barrier that every thread reaches after reading it.
__device__ __forceinline__ double wg_sum1(double v, double* red2, int& slot) {
  v = wave_sum_f64(v);
  double* red = red2 + slot * (kFitThreads / 64);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  double s = 0.0;
#pragma unroll
  for (int i = 0; i < kFitThreads / 64; ++i) s += red[i];
  slot ^= 1;
  return s;
}

// Number of eigenvalues of the symmetric tridiagonal (a, b) below x.
// 1/q from the hardware reciprocal and one Newton step (relative error near
// the double rounding unit); only the signs of the recurrence are used.
__device__ __forceinline__ double rcp_nr(double q) {
  const double r = __builtin_amdgcn_rcp(q);
  return fma(r, fma(-q, r, 1.0), r);
}

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

__device__ __forceinline__ int probe_pos(int i, int N, int m) {
  return (int)(((2LL * i + 1) * N) / (2LL * m));
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
// grid (H, ceil((d+1)/8)), block 256. Workgroup b accumulates rows [8b, 8b+8)
// of Sigma (rows < d), of X^T W R and of the Gram (rows < d+1) over chunks of
// 256 probe rows staged in LDS.
template <int D>
__global__ __launch_bounds__(kFitThreads) void k_fit_prep(const float* S_out, const float* O_probe,
                                                          int N, int m, int kmax, double lambda,
                                                          double* scratch) {
  constexpr int NT = kFitThreads;
  constexpr int NX = D + 1;
  constexpr int RB = 8;
  constexpr int CH = 256;          // probe rows per chunk
  __shared__ double ra[CH][RB];    // w_i * r_i[a] for the block's rows a
  __shared__ double xa[CH][RB];    // w_i * x_i[a]
  __shared__ double w_s[CH];
  __shared__ int pos_s[CH];
  __shared__ double red2[2 * NT / 64];
  const int h = blockIdx.x, b = blockIdx.y, t = threadIdx.x;
  const float* Sh = S_out + (size_t)h * N * D;
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
      pos_s[t] = probe_pos(i0 + t, N, m);
    }
    __syncthreads();
    for (int idx = t; idx < mi * RB; idx += NT) {
      const int i = idx / RB, u = idx % RB, a = a0 + u;
      const int p = pos_s[i];
      double rv = 0.0, xv = 0.0;
      if (a < D) {
        const double s = Sh[(size_t)p * D + a];
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
        const int p = pos_s[i];
        double col;
        if (kind == 2) col = c < D ? (double)Sh[(size_t)p * D + c] : 1.0;
        else col = (double)Op[(size_t)(i0 + i) * D + c] - (double)Sh[(size_t)p * D + c];
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
        double v = (i0 == 0 ? 0.0 : *dst) + acc[u];
        if (kind == 2 && i0 + mi == m && a == c && a < D) v += lambda;
        *dst = v;
      }
    }
  }
}

// ---------------------------------------------------------------- fit
template <int D>
__global__ __launch_bounds__(kFitThreads) void k_fit(int m, int kmax, float* U_out, float* Th_out,
                                                     int32_t* rank_eff, double* scratch) {
  constexpr int NT = kFitThreads;
  constexpr int PA = D + 1;                // pitch of the eigen matrix
  constexpr int NX = D + 1;                // ridge unknowns (d weights + bias)
  constexpr int NP = NX * (NX + 1) / 2;    // packed lower triangle of the ridge matrix
  constexpr int BIG = (D + 1) * (D + 2);
  __shared__ double big[BIG];
  __shared__ double dg[D], od[D], od2[D], beta[D], vv[D], pv[D], vn[D];
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
  // ---- Householder tridiagonalisation; reflector k stored in column k below
  // the diagonal. Four barriers per step: two sums, q ready, update done.
  for (int k = 0; k < D - 2; ++k) {
    const int L = D - k - 1;
    double part = 0.0;
    for (int i = 1 + t; i < L; i += NT) {
      const double x = A[(k + 1 + i) * PA + k];
      part += x * x;
    }
    const double sig2 = wg_sum1(part, red2, slot);
    const double x0 = A[(k + 1) * PA + k];
    if (sig2 == 0.0) {
      if (t == 0) {
        beta[k] = 0.0;
        od[k] = x0;
      }
      continue;   // nothing is updated in this step
    }
    const double alpha = -copysign(sqrt(x0 * x0 + sig2), x0);
    const double v0 = x0 - alpha;
    const double bk = 2.0 / (v0 * v0 + sig2);
    // p = beta A22 v with v_0 = v0, v_j = A[k+1+j][k]. Row i of the product is
    // split over NSEG waves by segments of j; every step of a partial sum reads
    // one row of A22 across the wave. v^T p comes from the partials directly.
    const int i = t & (D - 1), seg = t / D;
    const int jm = (L + NSEG - 1) / NSEG;
    double s = 0.0;
    if (i < L) {
      const int j0 = min(L, seg * jm), j1 = min(L, j0 + jm);
      // four independent partial sums keep several LDS reads in flight
      double s4[4] = {0.0, 0.0, 0.0, 0.0};
      int j = j0;
      if (j == 0) {
        s4[0] = A[(k + 1) * PA + (k + 1 + i)] * v0;
        j = 1;
      }
      for (; j + 3 < j1; j += 4) {
#pragma unroll
        for (int u = 0; u < 4; ++u)
          s4[u] += A[(k + 1 + j + u) * PA + (k + 1 + i)] * A[(k + 1 + j + u) * PA + k];
      }
      for (; j < j1; ++j) s4[0] += A[(k + 1 + j) * PA + (k + 1 + i)] * A[(k + 1 + j) * PA + k];
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
    for (int i2 = t >> 5; i2 < L; i2 += NT / 32) {
      const double vi2 = vv[i2], qi2 = pv[i2];
      double* row = A + (k + 1 + i2) * PA + (k + 1);
      for (int j2 = t & 31; j2 < L; j2 += 32) row[j2] -= vi2 * pv[j2] + qi2 * vv[j2];
    }
    __syncthreads();
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
  // P-point multisection per eigenvalue, P = 32, 16 or 8 as keff allows; the
  // interval shrinks by (P + 1)^iters > 2^50
  const int P = keff <= NT / 32 ? 32 : (keff <= NT / 16 ? 16 : 8);
  const int iters = P == 32 ? 10 : (P == 16 ? 13 : 16);
  for (int base = 0; base < keff; base += NT / P) {
    const int r = base + t / P, sub = t % P;
    const int j = D - 1 - (r < keff ? r : 0);  // ascending eigenvalue index
    double lo = glo, hi = ghi;
    for (int iter = 0; iter < iters; ++iter) {
      const double x = lo + (hi - lo) * (double)(sub + 1) / (double)(P + 1);
      const int cnt = sturm_count(dg, od2, D, x, pivmin);
      double nlo = lo, nhi = hi;
      for (int sp = 0; sp < P; ++sp) {
        const double xs = __shfl(x, (t & ~(P - 1)) + sp);
        const int cs = __shfl(cnt, (t & ~(P - 1)) + sp);
        if (cs <= j) nlo = fmax(nlo, xs);
        else nhi = fmin(nhi, xs);
      }
      lo = nlo;
      hi = nhi;
    }
    if (r < keff && sub == 0) lam_top[r] = 0.5 * (lo + hi);
  }
  __syncthreads();
  // ---- reflectors to the workspace; the LDS block is reused from here on
  for (int idx = t; idx < D * D; idx += NT) {
    const int i = idx / D, k = idx % D;
    if (i > k && k < D - 2) f.hv[(size_t)i * D + k] = A[i * PA + k];
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
      for (int pass = 0; pass < 3; ++pass) {
        double cd = dg[0] - lam, cu = od[0], cu2 = 0.0, cr = Z[t];
        for (int i = 0; i < D - 1; ++i) {
          const double nl = od[i], nd = dg[i + 1] - lam, nu = (i + 1 < D - 1) ? od[i + 1] : 0.0;
          const double nr = Z[(i + 1) * KB + t];
          if (fabs(cd) >= fabs(nl)) {
            if (cd == 0.0) cd = pe;
            const double mlt = nl / cd;
            U1[i * KB + t] = cd; U2[i * KB + t] = cu; U3[i * KB + t] = cu2; Z[i * KB + t] = cr;
            cd = nd - mlt * cu;
            cu = nu - mlt * cu2;
            cu2 = 0.0;
            cr = nr - mlt * cr;
          } else {
            const double mlt = cd / nl;
            U1[i * KB + t] = nl; U2[i * KB + t] = nd; U3[i * KB + t] = nu; Z[i * KB + t] = nr;
            const double ncd = cu - mlt * nd;
            const double ncu = cu2 - mlt * nu;
            cr = cr - mlt * nr;
            cd = ncd;
            cu = ncu;
            cu2 = 0.0;
          }
        }
        if (fabs(cd) < pe) cd = cd < 0.0 ? -pe : pe;
        double y1 = cr / cd, y2 = 0.0;
        double nrm = y1 * y1;
        Z[(D - 1) * KB + t] = y1;
        for (int i = D - 2; i >= 0; --i) {
          const double y = (Z[i * KB + t] - U2[i * KB + t] * y1 - U3[i * KB + t] * y2) / U1[i * KB + t];
          Z[i * KB + t] = y;
          nrm += y * y;
          y2 = y1;
          y1 = y;
        }
        const double inv = 1.0 / sqrt(nrm);
        for (int i = 0; i < D; ++i) Z[i * KB + t] *= inv;
      }
    }
    __syncthreads();
    for (int idx = t; idx < D * nbt; idx += NT) {
      const int i = idx / nbt, r = idx % nbt;
      Xg[(size_t)i * kmax + b0 + r] = Z[i * KB + r];
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
  // ---- classical Gram-Schmidt, twice, in eigenvalue order
  for (int j = 1; j < keff; ++j) {
    for (int pass = 0; pass < 2; ++pass) {
      for (int i0 = 0; i0 < j; i0 += NT / 8) {
        const int i = i0 + t / 8, sub = t % 8;
        double sacc = 0.0;
        if (i < j)
          for (int e = sub; e < D; e += 8) sacc += X[e * PXK + i] * X[e * PXK + j];
        sacc += __shfl_xor(sacc, 1);
        sacc += __shfl_xor(sacc, 2);
        sacc += __shfl_xor(sacc, 4);
        if (i < j && sub == 0) dots[i] = sacc;
      }
      __syncthreads();
      for (int e = t; e < D; e += NT) {
        double x = X[e * PXK + j];
        for (int i = 0; i < j; ++i) x -= dots[i] * X[e * PXK + i];
        X[e * PXK + j] = x;
      }
      __syncthreads();
    }
    double part = 0.0;
    for (int e = t; e < D; e += NT) {
      const double x = X[e * PXK + j];
      part += x * x;
    }
    const double nrm = sqrt(wg_sum1(part, red2, slot));
    for (int e = t; e < D; e += NT) X[e * PXK + j] /= nrm;
    __syncthreads();
  }
  // ---- back-transform through the reflectors: X <- H_0 H_1 ... H_{D-3} X.
  // The next reflector is fetched from the workspace while this one is applied.
  for (int i = t; i < 2; i += NT) vv[i] = f.hv[(size_t)(D - 2 + i) * D + (D - 3)];
  __syncthreads();
  for (int k = D - 3; k >= 0; --k) {
    const int L = D - k - 1;
    double* vc = ((D - 3 - k) & 1) ? vn : vv;
    double* vnx = ((D - 3 - k) & 1) ? vv : vn;
    double nxt = 0.0;
    if (k > 0 && t < L + 1) nxt = f.hv[(size_t)(k + t) * D + (k - 1)];
    const double bk = beta[k];
    for (int c0 = 0; c0 < keff; c0 += NT / 16) {
      const int cc = c0 + t / 16, sub = t % 16;
      double sacc = 0.0;
      if (cc < keff && bk != 0.0) {
        double s2[2] = {0.0, 0.0};
        int i = sub;
        for (; i + 16 < L; i += 32) {
          s2[0] += vc[i] * X[(k + 1 + i) * PXK + cc];
          s2[1] += vc[i + 16] * X[(k + 17 + i) * PXK + cc];
        }
        for (; i < L; i += 16) s2[0] += vc[i] * X[(k + 1 + i) * PXK + cc];
        sacc = s2[0] + s2[1];
      }
      sacc += __shfl_xor(sacc, 1);
      sacc += __shfl_xor(sacc, 2);
      sacc += __shfl_xor(sacc, 4);
      sacc += __shfl_xor(sacc, 8);
      if (cc < keff && sub == 0) dots[cc] = bk * sacc;
    }
    __syncthreads();
    if (bk != 0.0) {
      for (int cc = t & 31; cc < keff; cc += 32) {
        const double dc = dots[cc];
        for (int i = t >> 5; i < L; i += NT / 32) X[(k + 1 + i) * PXK + cc] -= dc * vc[i];
      }
    }
    if (k > 0 && t < L + 1) vnx[t] = nxt;
    __syncthreads();
  }
  for (int idx = t; idx < D * keff; idx += NT) {
    const int e = idx / keff, cc = idx % keff;
    Uh[(size_t)e * kmax + cc] = (float)X[e * PXK + cc];
  }
  // ---- right-hand side (X^T W R) U in 4 x 4 register tiles, into the
  // workspace (it is copied behind the packed ridge matrix when it fits)
  {
    const int ntr = (NX + 3) / 4, ntc = (keff + 3) / 4;
    for (int tile = t; tile < ntr * ntc; tile += NT) {
      const int r0 = 4 * (tile / ntc), c0 = 4 * (tile % ntc);
      double acc[4][4];
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int v = 0; v < 4; ++v) acc[u][v] = 0.0;
      for (int e = 0; e < D; ++e) {
        double xr[4], uc[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) xr[u] = r0 + u < NX ? f.xtwr[(size_t)(r0 + u) * D + e] : 0.0;
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
        for (int v = 0; v < 4; ++v)
          if (r0 + u < NX && c0 + v < keff) f.rhs[(size_t)(r0 + u) * kmax + c0 + v] = acc[u][v];
    }
  }
  __syncthreads();
  const bool rhs_lds = NP + NX * keff <= BIG;
  double* rhs = rhs_lds ? big + NP : f.rhs;
  const int rstride = rhs_lds ? keff : kmax;
  // ---- packed ridge matrix P(i, j) = i (i + 1) / 2 + j, j <= i
  for (int idx = t; idx < NX * NX; idx += NT) {
    const int i = idx / NX, j = idx % NX;
    if (j <= i) big[i * (i + 1) / 2 + j] = f.gram[idx];
  }
  if (rhs_lds)
    for (int idx = t; idx < NX * keff; idx += NT) rhs[idx] = f.rhs[(size_t)(idx / keff) * kmax + idx % keff];
  __syncthreads();
  // ---- Cholesky, right-looking, one barrier per column: the trailing update
  // uses the unscaled column j and 1/d_j; column j is scaled in the next step,
  // when it is no longer read.
  double dprev = 1.0;
  for (int j = 0; j < NX; ++j) {
    double dj = big[j * (j + 1) / 2 + j];
    dj = dj > 0.0 ? dj : 1e-300;
    const double rd = 1.0 / dj;
    if (j > 0) {
      const double sc = 1.0 / sqrt(dprev);
      for (int i = j + t; i < NX; i += NT) big[i * (i + 1) / 2 + (j - 1)] *= sc;
      if (t == 0) big[(j - 1) * j / 2 + (j - 1)] = sqrt(dprev);
    }
    for (int i = j + 1 + (t >> 5); i < NX; i += NT / 32) {
      double* row = big + i * (i + 1) / 2;
      const double lij = row[j] * rd;
      for (int l = j + 1 + (t & 31); l <= i; l += 32) row[l] -= lij * big[l * (l + 1) / 2 + j];
    }
    dprev = dj;
    __syncthreads();
  }
  if (t == 0) big[(NX - 1) * NX / 2 + (NX - 1)] = sqrt(dprev);
  __syncthreads();
  double* rdiag = lam_top;   // free again: 1 / L_ii for the substitutions
  static_assert(NX <= D + 1, "reciprocal diagonal fits in lam_top");
  for (int i = t; i < NX; i += NT) rdiag[i] = 1.0 / big[i * (i + 1) / 2 + i];
  __syncthreads();
  // ---- L y = b, then L^T x = y: sixteen lanes per right-hand-side column,
  // each column handled by one wave, so only wave-level ordering is needed
  {
    constexpr int LPC = 16;                     // lanes per column
    constexpr int NU = (NX + LPC - 1) / LPC;    // terms per lane at most
    const int lane = t & 63, w = t >> 6;
    const int part = lane & (LPC - 1);
    for (int cb = 0; cb < keff; cb += (64 / LPC) * (NT / 64)) {
      const int cc = cb + (64 / LPC) * w + lane / LPC;
      const bool on = cc < keff;
      for (int i = 0; i < NX; ++i) {
        double s = 0.0;
        if (on) {
          const double* row = big + i * (i + 1) / 2;
          // all of the lane's terms are read at once (one LDS round trip)
          double s2[2] = {0.0, 0.0};
#pragma unroll
          for (int u = 0; u < NU; ++u) {
            const int l = part + u * LPC;
            if (l < i) s2[u & 1] += row[l] * rhs[(size_t)l * rstride + cc];
          }
          s = s2[0] + s2[1];
        }
        s += __shfl_xor(s, 1);
        s += __shfl_xor(s, 2);
        s += __shfl_xor(s, 4);
        s += __shfl_xor(s, 8);
        if (on && part == 0)
          rhs[(size_t)i * rstride + cc] = (rhs[(size_t)i * rstride + cc] - s) * rdiag[i];
        if (rhs_lds) __builtin_amdgcn_wave_barrier();
        else __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "workgroup");
      }
      for (int i = NX - 1; i >= 0; --i) {
        double s = 0.0;
        if (on) {
          double s2[2] = {0.0, 0.0};
#pragma unroll
          for (int u = 0; u < NU; ++u) {
            const int l = i + 1 + part + u * LPC;
            if (l < NX) s2[u & 1] += big[l * (l + 1) / 2 + i] * rhs[(size_t)l * rstride + cc];
          }
          s = s2[0] + s2[1];
        }
        s += __shfl_xor(s, 1);
        s += __shfl_xor(s, 2);
        s += __shfl_xor(s, 4);
        s += __shfl_xor(s, 8);
        if (on && part == 0)
          rhs[(size_t)i * rstride + cc] = (rhs[(size_t)i * rstride + cc] - s) * rdiag[i];
        if (rhs_lds) __builtin_amdgcn_wave_barrier();
        else __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "workgroup");
      }
    }
  }
  __syncthreads();
  for (int idx = t; idx < NX * keff; idx += NT) {
    const int ra = idx / keff, cc = idx % keff;
    Th[(size_t)ra * kmax + cc] = (float)rhs[(size_t)ra * rstride + cc];
  }
  if (t == 0) rank_eff[h] = keff;
}

size_t fit_ws_per_head(const Dims& d) {
  return fit_doubles_per_head(d.m, d.D, d.k) * sizeof(double);
}

hipError_t launch_fit(const Dims& d, const float* S_out, const float* O_probe, float* U,
                      float* Theta, int32_t* rank_eff, char* fit_ws, hipStream_t st) {
  double* scratch = reinterpret_cast<double*>(fit_ws);
  const dim3 pgrid(d.H, (d.D + 1 + 7) / 8);
#define SPR_FIT(DD)                                                                         \
  do {                                                                                      \
    k_fit_prep<DD><<<pgrid, kFitThreads, 0, st>>>(S_out, O_probe, d.N, d.m, d.k, d.lam,     \
                                                   scratch);                                \
    k_fit<DD><<<d.H, kFitThreads, 0, st>>>(d.m, d.k, U, Theta, rank_eff, scratch);          \
  } while (0)
  if (d.D == 128) SPR_FIT(128);
  else SPR_FIT(64);
#undef SPR_FIT
  return hipGetLastError();
}

}  // namespace spr
