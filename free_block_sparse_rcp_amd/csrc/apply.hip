// Residual apply and return to token order (arxivdaily 2608.18484, English
// abstract: the fitted map predicts a residual for each unprobed query, which
// is added to its sparse output).
//
// For 64 query positions per workgroup: y = Theta^T [s; 1] (k values), then
// o = s + U y, in fp32; probe positions take their exact output instead. The
// rank is processed in chunks of 32 columns so LDS stays small for any k.
#include "common.hpp"
#include "internal.hpp"

namespace spr {

constexpr int kApplyRows = 64;
constexpr int kApplyChunk = 32;

__device__ __forceinline__ int probe_index(int pos, int N, int m) {
  if (m <= 0) return -1;
  const int64_t c = ((int64_t)pos * m) / N;
  for (int64_t i = c - 1; i <= c + 1; ++i) {
    if (i < 0 || i >= m) continue;
    if ((int)(((2 * i + 1) * N) / (2LL * m)) == pos) return (int)i;
  }
  return -1;
}

template <bool BF16, int D>
__global__ __launch_bounds__(256) void k_apply(const float* S, const int32_t* query_perm,
                                               const float* O_probe, const float* U,
                                               const float* Theta, const int32_t* rank_eff,
                                               int N, int m, int kmax, void* Ov) {
  using E = Elt<BF16>;
  constexpr int DU = D / 4;
  __shared__ float s_t[kApplyRows][D + 1];
  __shared__ float th[(D + 1) * kApplyChunk];
  __shared__ float ut[D * kApplyChunk];
  __shared__ float y_t[kApplyRows][kApplyChunk + 1];
  const int h = blockIdx.y, t = threadIdx.x;
  const int p0 = blockIdx.x * kApplyRows;
  const int nrow = min(N, p0 + kApplyRows) - p0;
  S += (size_t)h * N * D;
  typename E::T* O = static_cast<typename E::T*>(Ov) + (size_t)h * N * D;
  const float* Uh = U + (size_t)h * D * kmax;
  const float* Th = Theta + (size_t)h * (D + 1) * kmax;
  const int keff = rank_eff[h];
  for (int idx = t; idx < kApplyRows * D; idx += 256) {
    const int r = idx / D, e = idx % D;
    s_t[r][e] = r < nrow ? S[(size_t)(p0 + r) * D + e] : 0.f;
  }
  const int r = t >> 2, q = t & 3;
  float corr[DU];
#pragma unroll
  for (int u = 0; u < DU; ++u) corr[u] = 0.f;
  for (int c0 = 0; c0 < keff; c0 += kApplyChunk) {
    const int nc = min(kApplyChunk, keff - c0);
    __syncthreads();
    for (int idx = t; idx < (D + 1) * kApplyChunk; idx += 256) {
      const int a = idx / kApplyChunk, j = idx % kApplyChunk;
      th[idx] = j < nc ? Th[(size_t)a * kmax + c0 + j] : 0.f;
    }
    for (int idx = t; idx < D * kApplyChunk; idx += 256) {
      const int e = idx / kApplyChunk, j = idx % kApplyChunk;
      ut[idx] = j < nc ? Uh[(size_t)e * kmax + c0 + j] : 0.f;
    }
    __syncthreads();
    // y[r][j] for j = q + 4v
#pragma unroll
    for (int v = 0; v < kApplyChunk / 4; ++v) {
      const int j = q + 4 * v;
      float acc = th[D * kApplyChunk + j];
      for (int e = 0; e < D; ++e) acc = fmaf(s_t[r][e], th[e * kApplyChunk + j], acc);
      y_t[r][j] = acc;
    }
    __syncthreads();
#pragma unroll
    for (int u = 0; u < DU; ++u) {
      const int e = q + 4 * u;
      float acc = corr[u];
      for (int j = 0; j < kApplyChunk; ++j) acc = fmaf(ut[e * kApplyChunk + j], y_t[r][j], acc);
      corr[u] = acc;
    }
  }
  __syncthreads();
  if (r >= nrow) return;
  const int pos = p0 + r;
  const int tok = clamp_idx(query_perm[(size_t)h * N + pos], N);
  const int pi = probe_index(pos, N, m);
  if (pi >= 0) {
    const float* op = O_probe + ((size_t)h * m + pi) * D;
#pragma unroll
    for (int u = 0; u < DU; ++u) E::st(O, (size_t)tok * D + q + 4 * u, op[q + 4 * u]);
  } else {
#pragma unroll
    for (int u = 0; u < DU; ++u) E::st(O, (size_t)tok * D + q + 4 * u, s_t[r][q + 4 * u] + corr[u]);
  }
}

hipError_t launch_apply(const Dims& d, const float* S_out, const int32_t* query_perm,
                        const float* O_probe, const float* U, const float* Theta,
                        const int32_t* rank_eff, void* O, hipStream_t st) {
  const dim3 grid((d.N + kApplyRows - 1) / kApplyRows, d.H);
#define SPR_APPLY(B, DD)                                                                   \
  k_apply<B, DD><<<grid, 256, 0, st>>>(S_out, query_perm, O_probe, U, Theta, rank_eff, d.N, \
                                        d.m, d.k, O)
  if (d.bf16) {
    if (d.D == 128) SPR_APPLY(true, 128); else SPR_APPLY(true, 64);
  } else {
    if (d.D == 128) SPR_APPLY(false, 128); else SPR_APPLY(false, 64);
  }
#undef SPR_APPLY
  return hipGetLastError();
}

}  // namespace spr
