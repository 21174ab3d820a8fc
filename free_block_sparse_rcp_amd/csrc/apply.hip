// Residual apply and return to token order (arxivdaily 2608.18484, English
// abstract: the fitted map predicts a residual for each unprobed query, which
// is added to its sparse output).
//
// For 64 query positions per workgroup: y = Theta^T [s; 1] (k values), then
// o = s + U y, in fp32; probe positions take their exact output instead. The
// rank is processed in chunks of 32 columns so LDS stays small for any k;
// threads are register-blocked (4 rows x 2 columns, then 4 rows x d/16
// contiguous outputs) and write whole 8/16-byte pieces of each output row.
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
  constexpr int EPT = D / 16;          // output elements per thread (contiguous)
  constexpr int CH = kApplyChunk;
  __shared__ float s_t[kApplyRows][D + 1];
  __shared__ float th[(D + 1) * CH];   // [a][j]
  __shared__ float ut[D * (CH + 1)];   // [e][j], padded
  __shared__ float y_t[kApplyRows][CH + 1];
  const int h = blockIdx.y, t = threadIdx.x;
  const int p0 = blockIdx.x * kApplyRows;
  const int nrow = min(N, p0 + kApplyRows) - p0;
  S += (size_t)h * N * D;
  typename E::T* O = static_cast<typename E::T*>(Ov) + (size_t)h * N * D;
  const float* Uh = U + (size_t)h * D * kmax;
  const float* Th = Theta + (size_t)h * (D + 1) * kmax;
  const int keff = rank_eff[h];
  for (int idx = t; idx < kApplyRows * D / 4; idx += 256) {
    const int r = idx / (D / 4), e4 = idx % (D / 4);
    f32x4 v = {0.f, 0.f, 0.f, 0.f};
    if (r < nrow) v = *reinterpret_cast<const f32x4*>(S + (size_t)(p0 + r) * D + 4 * e4);
    s_t[r][4 * e4] = v[0];
    s_t[r][4 * e4 + 1] = v[1];
    s_t[r][4 * e4 + 2] = v[2];
    s_t[r][4 * e4 + 3] = v[3];
  }
  const int rg = t & 15;               // rows rg + 16 i
  const int cg = t >> 4;               // phase 1: columns cg, cg + 16; phase 2: e in [EPT cg, EPT cg + EPT)
  float corr[4][EPT];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int u = 0; u < EPT; ++u) corr[i][u] = 0.f;
  for (int c0 = 0; c0 < keff; c0 += CH) {
    const int nc = min(CH, keff - c0);
    __syncthreads();
    for (int idx = t; idx < (D + 1) * CH; idx += 256) {
      const int a = idx / CH, j = idx % CH;
      th[idx] = j < nc ? Th[(size_t)a * kmax + c0 + j] : 0.f;
    }
    for (int idx = t; idx < D * CH; idx += 256) {
      const int e = idx / CH, j = idx % CH;
      ut[e * (CH + 1) + j] = j < nc ? Uh[(size_t)e * kmax + c0 + j] : 0.f;
    }
    __syncthreads();
    // y = [s, 1] Theta for this chunk: 4 rows x 2 columns per thread
    float y[4][2];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      y[i][0] = th[D * CH + cg];
      y[i][1] = th[D * CH + cg + 16];
    }
    for (int e = 0; e < D; ++e) {
      const float t0 = th[e * CH + cg], t1 = th[e * CH + cg + 16];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float sv = s_t[rg + 16 * i][e];
        y[i][0] = fmaf(sv, t0, y[i][0]);
        y[i][1] = fmaf(sv, t1, y[i][1]);
      }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      y_t[rg + 16 * i][cg] = y[i][0];
      y_t[rg + 16 * i][cg + 16] = y[i][1];
    }
    __syncthreads();
    // corr += y U^T: 4 rows x EPT contiguous elements per thread
    for (int j = 0; j < CH; ++j) {
      float uv[EPT];
#pragma unroll
      for (int u = 0; u < EPT; ++u) uv[u] = ut[(EPT * cg + u) * (CH + 1) + j];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float yv = y_t[rg + 16 * i][j];
#pragma unroll
        for (int u = 0; u < EPT; ++u) corr[i][u] = fmaf(uv[u], yv, corr[i][u]);
      }
    }
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = rg + 16 * i;
    if (r >= nrow) continue;
    const int pos = p0 + r;
    const int tok = clamp_idx(query_perm[(size_t)h * N + pos], N);
    const int pi = probe_index(pos, N, m);
    float v[EPT];
    if (pi >= 0) {
      const float* op = O_probe + ((size_t)h * m + pi) * D + EPT * cg;
#pragma unroll
      for (int u = 0; u < EPT; ++u) v[u] = op[u];
    } else {
#pragma unroll
      for (int u = 0; u < EPT; ++u) v[u] = s_t[r][EPT * cg + u] + corr[i][u];
    }
    typename E::T* dst = O + (size_t)tok * D + EPT * cg;
    if (BF16) {
#pragma unroll
      for (int u = 0; u < EPT; u += 4) {
        const f32x2 f0 = {v[u], v[u + 1]};
        const f32x2 f1 = {v[u + 2], v[u + 3]};
        const bf16x2 b0 = __builtin_convertvector(f0, bf16x2);
        const bf16x2 b1 = __builtin_convertvector(f1, bf16x2);
        const bf16x4 bv = {b0[0], b0[1], b1[0], b1[1]};
        *reinterpret_cast<bf16x4*>(reinterpret_cast<uint16_t*>(dst) + u) = bv;
      }
    } else {
#pragma unroll
      for (int u = 0; u < EPT; u += 4) {
        const f32x4 fv = {v[u], v[u + 1], v[u + 2], v[u + 3]};
        *reinterpret_cast<f32x4*>(reinterpret_cast<float*>(dst) + u) = fv;
      }
    }
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
