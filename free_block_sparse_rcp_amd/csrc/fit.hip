// Probe-fitted residual reconstruction: the fit (arxivdaily 2608.18484,
// English abstract: weighted ridge regression of the dense-minus-sparse
// differences of the probe rows on the sparse output; skillfed article and
// peercurrent abstract: an affine map, call-specific, restricted to the output
// subspace seen in the probe residuals).
//
// One workgroup per head, all in fp64:
//   r_i = o_i - s_i, w_i = ||o_i||^-2 / sum ||o||^-2, Sigma = sum w_i r_i r_i^T;
//   top-k_eff eigenvectors of Sigma: Householder tridiagonalisation in LDS,
//   eigenvalues by Sturm-count multisection, eigenvectors of the tridiagonal
//   by inverse iteration, re-orthonormalised (classical Gram-Schmidt twice)
//   and mapped back through the reflectors;
//   Theta from (X^T W X + lambda I~) Theta = X^T W (R U), X = [s, 1], by
//   Cholesky in LDS with an unpenalised bias row.
#include "common.hpp"
#include "internal.hpp"

namespace spr {

constexpr int kFitThreads = 256;

__device__ __forceinline__ double wave_sum_f64(double v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

// Workgroup sum with two barriers (wave shuffles, then one LDS exchange).
__device__ __forceinline__ double wg_sum(double v, double* red) {
  v = wave_sum_f64(v);
  const int w = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) red[w] = v;
  __syncthreads();
  double s = 0.0;
#pragma unroll
  for (int i = 0; i < kFitThreads / 64; ++i) s += red[i];
  __syncthreads();
  return s;
}

// Number of eigenvalues of the symmetric tridiagonal (a, b) below x.
__device__ int sturm_count(const double* a, const double* b2, int n, double x, double pivmin) {
  int cnt = 0;
  double q = a[0] - x;
  if (fabs(q) < pivmin) q = -pivmin;
  cnt += q < 0.0;
  for (int i = 1; i < n; ++i) {
    q = (a[i] - x) - b2[i - 1] / q;
    if (fabs(q) < pivmin) q = -pivmin;
    cnt += q < 0.0;
  }
  return cnt;
}

// Per-head scratch layout (doubles) in the workspace.
struct FitScratch {
  double *R, *S, *w, *X, *hv, *Y, *rhs;
};
__host__ __device__ inline size_t fit_doubles_per_head(int m, int D, int k) {
  return (size_t)2 * m * D + m + (size_t)D * k + (size_t)D * D + (size_t)m * k +
         (size_t)(D + 1) * k + 64;
}
__device__ inline FitScratch fit_scratch(double* base, int m, int D, int k) {
  FitScratch f;
  f.R = base;
  f.S = f.R + (size_t)m * D;
  f.w = f.S + (size_t)m * D;
  f.X = f.w + m;
  f.hv = f.X + (size_t)D * k;
  f.Y = f.hv + (size_t)D * D;
  f.rhs = f.Y + (size_t)m * k;
  return f;
}

template <int D>
__global__ __launch_bounds__(kFitThreads) void k_fit(const float* S_out_in, const float* O_probe,
                                                     int N, int m, int kmax, double lambda,
                                                     float* U_out, float* Th_out,
                                                     int32_t* rank_eff, double* scratch) {
  constexpr int NT = kFitThreads;
  constexpr int PA = D + 1;       // pitch of the eigen matrix
  constexpr int PX = D + 2;       // pitch of the ridge matrix
  constexpr int NX = D + 1;       // ridge unknowns (d weights + bias)
  __shared__ double big[(D + 1) * (D + 2)];
  __shared__ double dg[D], od[D], od2[D], beta[D], vv[D], pv[D];
  __shared__ double lam_top[D];
  __shared__ double red[NT / 64];
  __shared__ double dots[D];
  const int h = blockIdx.x, t = threadIdx.x;
  const float* S_out = S_out_in + (size_t)h * N * D;
  const float* Op = O_probe + (size_t)h * m * D;
  float* Uh = U_out + (size_t)h * D * kmax;
  float* Th = Th_out + (size_t)h * (D + 1) * kmax;
  int keff = min(kmax, min(m, D));
  FitScratch f = fit_scratch(scratch + (size_t)h * fit_doubles_per_head(m, D, kmax), m, D, kmax);

  for (int i = t; i < D * kmax; i += NT) Uh[i] = 0.f;
  for (int i = t; i < (D + 1) * kmax; i += NT) Th[i] = 0.f;
  if (keff <= 0) {
    if (t == 0) rank_eff[h] = 0;
    return;
  }
  // ---- probes: residuals, weights
  for (int idx = t; idx < m * D; idx += NT) {
    const int i = idx / D, e = idx % D;
    const int p = (int)(((2LL * i + 1) * N) / (2LL * m));
    const double s = S_out[(size_t)p * D + e];
    const double o = Op[(size_t)i * D + e];
    f.S[idx] = s;
    f.R[idx] = o - s;
  }
  double wpart = 0.0;
  for (int i = t; i < m; i += NT) {
    double n2 = 0.0;
    for (int e = 0; e < D; ++e) {
      const double o = Op[(size_t)i * D + e];
      n2 += o * o;
    }
    const double wi = n2 > 0.0 ? 1.0 / n2 : 0.0;
    f.w[i] = wi;
    wpart += wi;
  }
  const double wsum = wg_sum(wpart, red);
  for (int i = t; i < m; i += NT) f.w[i] = wsum > 0.0 ? f.w[i] / wsum : 0.0;
  __syncthreads();
  // ---- Sigma = sum_i w_i r_i r_i^T into LDS, 8 x 8 tiles per thread
  double* A = big;
  {
    constexpr int NTB = D / 8;
    for (int tile = t; tile < NTB * NTB; tile += NT) {
      const int a0 = 8 * (tile / NTB), b0 = 8 * (tile % NTB);
      double acc[8][8];
#pragma unroll
      for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[i][j] = 0.0;
      for (int i = 0; i < m; ++i) {
        const double wi = f.w[i];
        const double* Ri = f.R + (size_t)i * D;
        double ra[8], rb[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          ra[u] = wi * Ri[a0 + u];
          rb[u] = Ri[b0 + u];
        }
#pragma unroll
        for (int u = 0; u < 8; ++u)
#pragma unroll
          for (int v = 0; v < 8; ++v) acc[u][v] += ra[u] * rb[v];
      }
#pragma unroll
      for (int u = 0; u < 8; ++u)
#pragma unroll
        for (int v = 0; v < 8; ++v) A[(a0 + u) * PA + b0 + v] = acc[u][v];
    }
  }
  __syncthreads();
  double trpart = 0.0;
  for (int i = t; i < D; i += NT) trpart += A[i * PA + i];
  const double trace = wg_sum(trpart, red);
  if (!(trace > 0.0)) {
    if (t == 0) rank_eff[h] = 0;
    return;
  }
  // ---- Householder tridiagonalisation; reflector k stored in column k below the diagonal
  for (int k = 0; k < D - 2; ++k) {
    const int L = D - k - 1;
    double part = 0.0;
    for (int i = 1 + t; i < L; i += NT) {
      const double x = A[(k + 1 + i) * PA + k];
      part += x * x;
    }
    const double sig2 = wg_sum(part, red);
    const double x0 = A[(k + 1) * PA + k];
    if (sig2 == 0.0) {
      if (t == 0) {
        beta[k] = 0.0;
        od[k] = x0;
      }
      __syncthreads();
      continue;
    }
    const double alpha = -copysign(sqrt(x0 * x0 + sig2), x0);
    const double v0 = x0 - alpha;
    const double bk = 2.0 / (v0 * v0 + sig2);
    for (int i = t; i < L; i += NT) vv[i] = i == 0 ? v0 : A[(k + 1 + i) * PA + k];
    __syncthreads();
    if (t == 0) {
      beta[k] = bk;
      od[k] = alpha;
      A[(k + 1) * PA + k] = v0;
    }
    // p = beta * A22 v (column access of the symmetric trailing block)
    double vp = 0.0;
    for (int i = t; i < L; i += NT) {
      double s = 0.0;
      for (int j = 0; j < L; ++j) s += A[(k + 1 + j) * PA + (k + 1 + i)] * vv[j];
      pv[i] = bk * s;
      vp += vv[i] * pv[i];
    }
    const double K = 0.5 * bk * wg_sum(vp, red);
    for (int i = t; i < L; i += NT) pv[i] = pv[i] - K * vv[i];  // q
    __syncthreads();
    for (int idx = t; idx < L * L; idx += NT) {
      const int i = idx / L, j = idx % L;
      A[(k + 1 + i) * PA + (k + 1 + j)] -= vv[i] * pv[j] + pv[i] * vv[j];
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
  // ---- eigenvalues r = 0..keff-1 from the top: 8-point multisection per eigenvalue
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
  for (int base = 0; base < keff; base += NT / 8) {
    const int r = base + t / 8, sub = t % 8;
    const int j = D - 1 - (r < keff ? r : 0);  // ascending eigenvalue index
    double lo = glo, hi = ghi;
    for (int iter = 0; iter < 22; ++iter) {
      const double x = lo + (hi - lo) * (double)(sub + 1) / 9.0;
      const int cnt = sturm_count(dg, od2, D, x, pivmin);
      double nlo = lo, nhi = hi;
      for (int s = 0; s < 8; ++s) {
        const double xs = __shfl(x, (t & ~7) + s);
        const int cs = __shfl(cnt, (t & ~7) + s);
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
  // factors in LDS interleaved across the batch ([i][r]) so lanes hit distinct banks
  const double pe = 2.2e-16 * fmax(tnorm, 1e-300);
  constexpr int KB = D / 4;   // 4 arrays of D x KB doubles fit the (D+1)(D+2) LDS block
  static_assert(4 * D * KB <= (D + 1) * (D + 2), "inverse-iteration batch exceeds LDS");
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
      f.X[(size_t)i * kmax + b0 + r] = Z[i * KB + r];
    }
    __syncthreads();
  }
  // ---- eigenvector block in LDS: X[e][r], pitch keff + 1
  const int PXK = keff + 1;
  double* X = big;
  for (int idx = t; idx < D * keff; idx += NT) {
    const int e = idx / keff, r = idx % keff;
    X[e * PXK + r] = f.X[(size_t)e * kmax + r];
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
    const double nrm = sqrt(wg_sum(part, red));
    for (int e = t; e < D; e += NT) X[e * PXK + j] /= nrm;
    __syncthreads();
  }
  // ---- back-transform through the reflectors: X <- H_0 H_1 ... H_{D-3} X
  for (int k = D - 3; k >= 0; --k) {
    const double bk = beta[k];
    if (bk == 0.0) continue;
    const int L = D - k - 1;
    for (int i = t; i < L; i += NT) vv[i] = f.hv[(size_t)(k + 1 + i) * D + k];
    __syncthreads();
    for (int c0 = 0; c0 < keff; c0 += NT / 8) {
      const int cc = c0 + t / 8, sub = t % 8;
      double sacc = 0.0;
      if (cc < keff)
        for (int i = sub; i < L; i += 8) sacc += vv[i] * X[(k + 1 + i) * PXK + cc];
      sacc += __shfl_xor(sacc, 1);
      sacc += __shfl_xor(sacc, 2);
      sacc += __shfl_xor(sacc, 4);
      if (cc < keff && sub == 0) dots[cc] = bk * sacc;
    }
    __syncthreads();
    for (int idx = t; idx < L * keff; idx += NT) {
      const int i = idx / keff, cc = idx % keff;
      X[(k + 1 + i) * PXK + cc] -= dots[cc] * vv[i];
    }
    __syncthreads();
  }
  for (int idx = t; idx < D * keff; idx += NT) {
    const int e = idx / keff, cc = idx % keff;
    f.X[(size_t)e * kmax + cc] = X[e * PXK + cc];
    Uh[(size_t)e * kmax + cc] = (float)X[e * PXK + cc];
  }
  __syncthreads();
  // ---- Y = R U
  for (int idx = t; idx < m * keff; idx += NT) {
    const int i = idx / keff, cc = idx % keff;
    double s = 0.0;
    for (int e = 0; e < D; ++e) s += f.R[(size_t)i * D + e] * f.X[(size_t)e * kmax + cc];
    f.Y[(size_t)i * kmax + cc] = s;
  }
  __syncthreads();
  // ---- normal equations in LDS (the eigen matrix is no longer needed)
  double* Xn = big;
  {
    constexpr int NTB = (NX + 7) / 8;
    for (int tile = t; tile < NTB * NTB; tile += NT) {
      const int a0 = 8 * (tile / NTB), b0 = 8 * (tile % NTB);
      double acc[8][8];
#pragma unroll
      for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[i][j] = 0.0;
      for (int i = 0; i < m; ++i) {
        const double wi = f.w[i];
        const double* Si = f.S + (size_t)i * D;
        double xa[8], xb[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          const int a = a0 + u, b = b0 + u;
          xa[u] = wi * (a < D ? Si[a] : (a == D ? 1.0 : 0.0));
          xb[u] = b < D ? Si[b] : (b == D ? 1.0 : 0.0);
        }
#pragma unroll
        for (int u = 0; u < 8; ++u)
#pragma unroll
          for (int v = 0; v < 8; ++v) acc[u][v] += xa[u] * xb[v];
      }
#pragma unroll
      for (int u = 0; u < 8; ++u)
#pragma unroll
        for (int v = 0; v < 8; ++v) {
          const int a = a0 + u, b = b0 + v;
          if (a < NX && b < NX) Xn[a * PX + b] = acc[u][v] + ((a == b && a < D) ? lambda : 0.0);
        }
    }
  }
  for (int idx = t; idx < NX * keff; idx += NT) {
    const int ra = idx / keff, cc = idx % keff;
    double s = 0.0;
    for (int i = 0; i < m; ++i) {
      const double xa = ra < D ? f.S[(size_t)i * D + ra] : 1.0;
      s += f.w[i] * xa * f.Y[(size_t)i * kmax + cc];
    }
    f.rhs[(size_t)ra * kmax + cc] = s;
  }
  __syncthreads();
  // ---- Cholesky (lower, right-looking)
  for (int j = 0; j < NX; ++j) {
    if (t == 0) {
      const double dj = Xn[j * PX + j];
      Xn[j * PX + j] = sqrt(dj > 0.0 ? dj : 1e-300);
    }
    __syncthreads();
    const double ljj = Xn[j * PX + j];
    for (int i = j + 1 + t; i < NX; i += NT) Xn[i * PX + j] /= ljj;
    __syncthreads();
    const int L = NX - j - 1;
    for (int idx = t; idx < L * L; idx += NT) {
      const int i = j + 1 + idx / L, l = j + 1 + idx % L;
      if (l <= i) Xn[i * PX + l] -= Xn[i * PX + j] * Xn[l * PX + j];
    }
    __syncthreads();
  }
  // ---- forward then backward substitution, parallel over right-hand sides
  for (int i = 0; i < NX; ++i) {
    const double lii = Xn[i * PX + i];
    for (int cc = t; cc < keff; cc += NT) f.rhs[(size_t)i * kmax + cc] /= lii;
    __syncthreads();
    for (int idx = t; idx < (NX - i - 1) * keff; idx += NT) {
      const int l = i + 1 + idx / keff, cc = idx % keff;
      f.rhs[(size_t)l * kmax + cc] -= Xn[l * PX + i] * f.rhs[(size_t)i * kmax + cc];
    }
    __syncthreads();
  }
  for (int i = NX - 1; i >= 0; --i) {
    const double lii = Xn[i * PX + i];
    for (int cc = t; cc < keff; cc += NT) f.rhs[(size_t)i * kmax + cc] /= lii;
    __syncthreads();
    for (int idx = t; idx < i * keff; idx += NT) {
      const int l = idx / keff, cc = idx % keff;
      f.rhs[(size_t)l * kmax + cc] -= Xn[i * PX + l] * f.rhs[(size_t)i * kmax + cc];
    }
    __syncthreads();
  }
  for (int idx = t; idx < NX * keff; idx += NT) {
    const int ra = idx / keff, cc = idx % keff;
    Th[(size_t)ra * kmax + cc] = (float)f.rhs[(size_t)ra * kmax + cc];
  }
  if (t == 0) rank_eff[h] = keff;
}

size_t fit_ws_per_head(const Dims& d) {
  return fit_doubles_per_head(d.m, d.D, d.k) * sizeof(double);
}

hipError_t launch_fit(const Dims& d, const float* S_out, const float* O_probe, float* U,
                      float* Theta, int32_t* rank_eff, char* fit_ws, hipStream_t st) {
  double* scratch = reinterpret_cast<double*>(fit_ws);
#define SPR_FIT(DD)                                                                       \
  k_fit<DD><<<d.H, kFitThreads, 0, st>>>(S_out, O_probe, d.N, d.m, d.k, d.lam, U, Theta, \
                                         rank_eff, scratch)
  if (d.D == 128) SPR_FIT(128); else SPR_FIT(64);
#undef SPR_FIT
  return hipGetLastError();
}

}  // namespace spr
