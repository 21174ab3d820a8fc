// Residual apply and return to token order (arxivdaily 2608.18484, English
// abstract: the fitted map predicts a residual for each unprobed query, which
// is added to its sparse output).
//
// For 64 query positions per workgroup: y = Theta^T [s; 1] (k values), then
// o = s + U y, in fp32; probe positions take their exact output instead. The
// rank is processed in chunks of 32 columns so LDS stays small for any k;
// threads are register-blocked (4 rows x 2 columns, then 4 rows x d/16
// contiguous outputs) and write whole 8/16-byte pieces of each output row.
#include <algorithm>

#include "common.hpp"
#include "internal.hpp"

namespace spr {

constexpr int kApplyRows = 64;
constexpr int kApplyChunk = 32;

template <bool BF16, int D>
__global__ __launch_bounds__(256) void k_apply(const float* S, const int32_t* query_perm,
                                               const float* O_probe, const float* U,
                                               const float* Theta, const int32_t* rank_eff,
                                               const int32_t* ppos, int N, int m, int kmax,
                                               void* Ov) {
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
    const int pi = probe_index(ppos, pos, N, m);
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

// bf16 path on MFMA. The correction is linear in [s; 1], so it is folded into
// one matrix per head, W = Theta U^T ((d+1) x d): o = s + s W[:d] + W[d].
// k_apply_weights forms W^T once per head (fp32, stored as bf16 hi + lo parts)
// and the bias W[d]; k_apply_mfma copies them into LDS and runs the product
// O^T = W^T S^T as v_mfma_f32_32x32x16_bf16 on the bf16 sparse output
// (hi*s + lo*s: the correction keeps near-fp32 accuracy). Each wave takes 32
// query positions at a time, with the rows of its next two tiles in flight;
// the copy of s in the output layout for the final sum comes from lane-half
// swaps of the loaded rows, and the output tile is staged in LDS so that every
// row (token order) is written whole.
constexpr int kApplyTilesPerWg = 128;  // most 32-row tiles per workgroup
constexpr int kApplyWaves = 8;

// grid (H), block 256. wt: [H][2][d][d] bf16 (hi, lo) of W^T; bias: [H][d].
// Entry (e, a) of W^T (a = d is the bias) accumulates in LDS over chunks of
// 32 rank columns staged in LDS.
template <int D>
__global__ __launch_bounds__(256) void k_apply_weights(const float* U, const float* Theta,
                                                       const int32_t* rank_eff, int kmax,
                                                       uint16_t* wt, float* bias) {
  constexpr int CJ = 32;
  constexpr int UP = CJ + 1;
  constexpr int NE = D * (D + 1);
  __shared__ float ust[D * UP];
  __shared__ float tst[(D + 1) * UP];
  __shared__ float wacc[NE];
  const int h = blockIdx.x, t = threadIdx.x;
  int keff = rank_eff[h];
  keff = keff < 0 ? 0 : (keff > kmax ? kmax : keff);
  const float* Uh = U + (size_t)h * D * kmax;
  const float* Th = Theta + (size_t)h * (D + 1) * kmax;
  for (int i = t; i < NE; i += 256) wacc[i] = 0.f;
  for (int j0 = 0; j0 < keff; j0 += CJ) {
    __syncthreads();
    for (int i = t; i < D * CJ; i += 256) {
      const int r = i / CJ, j = i % CJ;
      ust[r * UP + j] = j0 + j < keff ? Uh[(size_t)r * kmax + j0 + j] : 0.f;
    }
    for (int i = t; i < (D + 1) * CJ; i += 256) {
      const int r = i / CJ, j = i % CJ;
      tst[r * UP + j] = j0 + j < keff ? Th[(size_t)r * kmax + j0 + j] : 0.f;
    }
    __syncthreads();
#pragma unroll 1
    for (int idx = t; idx < NE; idx += 256) {
      const int e = idx % D, aa = idx / D;
      float s = wacc[idx];
#pragma unroll 8
      for (int j = 0; j < CJ; ++j) s = fmaf(ust[e * UP + j], tst[aa * UP + j], s);
      wacc[idx] = s;
    }
  }
  __syncthreads();
  uint16_t* whi = wt + (size_t)h * 2 * D * D;
  uint16_t* wlo = whi + D * D;
  for (int idx = t; idx < NE; idx += 256) {
    const int e = idx % D, aa = idx / D;
    const float v = wacc[idx];
    if (aa == D) {
      bias[(size_t)h * D + e] = v;
    } else {
      const uint16_t hi = f32_to_bf16(v);
      whi[e * D + aa] = hi;
      wlo[e * D + aa] = f32_to_bf16(v - bf16_to_f32(hi));
    }
  }
}

template <int D>
__global__ __launch_bounds__(kApplyWaves * 64) void k_apply_mfma(const uint16_t* S, const int32_t* query_perm,
                                                    const float* O_probe, const uint16_t* wt,
                                                    const float* bias, const int32_t* ppos,
                                                    int N, int m, int wg_per_head, uint16_t* O) {
  constexpr int WP = D + 8;            // bf16 elements per LDS row of W^T (conflict-free b128 reads)
  constexpr int NKK = D / 16, NDT = D / 32;
  constexpr int CPR = D / 8;           // 16-byte chunks per row
  constexpr int OP = D + 8;            // bf16 elements per staged output row
  constexpr int NW = kApplyWaves;
  __shared__ __attribute__((aligned(16))) uint16_t wt_hi[D * WP];
  __shared__ __attribute__((aligned(16))) uint16_t wt_lo[D * WP];
  __shared__ float wbias[D];
  __shared__ __attribute__((aligned(16))) uint16_t ostage[NW][32 * OP];
  const int h = blockIdx.x / wg_per_head, part = blockIdx.x % wg_per_head;
  const int t = threadIdx.x, lane = t & 63, hl = lane >> 5, ql = lane & 31;
  const int w = __builtin_amdgcn_readfirstlane(t >> 6);
  {
    const uint16_t* src = wt + (size_t)h * 2 * D * D;
    for (int i = t; i < 2 * D * CPR; i += NW * 64) {
      const int arr = i / (D * CPR), rem = i % (D * CPR);
      const int r = rem / CPR, c = rem % CPR;
      const u32x4 v = *reinterpret_cast<const u32x4*>(src + (size_t)arr * D * D + r * D + 8 * c);
      *reinterpret_cast<u32x4*>((arr ? wt_lo : wt_hi) + r * WP + 8 * c) = v;
    }
    if (t < D) wbias[t] = bias[(size_t)h * D + t];
  }
  __syncthreads();

  const int ntile = (N + 31) / 32;
  const int per = (ntile + wg_per_head - 1) / wg_per_head;
  const int t0 = part * per, t1 = min(ntile, t0 + per);
  const uint16_t* Sh = S + (size_t)h * N * D;
  uint16_t* Oh = O + (size_t)h * N * D;
  uint16_t* stg = ostage[w];
  // A tile's s, as the MFMA operand: lane (ql, hl) holds columns 16 kk + 8 hl
  // .. + 7 of its row, one 16-byte load per k-step.
  auto load_tile = [&](u32x4 (&buf)[NKK], int tile) {
    const int pos = tile * 32 + ql;
    const bool ok = pos < N;
    const uint16_t* srow = Sh + (size_t)(ok ? pos : 0) * D;
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) {
      u32x4 v = {0u, 0u, 0u, 0u};
      if (ok) v = *reinterpret_cast<const u32x4*>(srow + 16 * kk + 8 * hl);
      buf[kk] = v;
    }
  };
  // One tile from buf; then buf takes the tile three rounds ahead.
  auto run_tile = [&](u32x4 (&buf)[NKK], int tile) {
    const int pos = tile * 32 + ql;
    const bool valid = pos < N;
    // token of this lane's row, read early; the store loop takes each row's
    // token from the lane that owns the row
    const int tok = valid ? clamp_idx(query_perm[(size_t)h * N + pos], N) : 0;
    const int pi = valid ? probe_index(ppos, pos, N, m) : -1;
    // W fragments are re-read from LDS every tile: kept opaque so that the
    // compiler does not hoist all of them into registers (occupancy)
    int woff = ql * WP + 8 * hl;
    asm volatile("" : "+v"(woff));
#pragma unroll
    for (int nt = 0; nt < NDT; ++nt) {
      f32x16 acc;
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[r] = 0.f;
      const uint16_t* whr = wt_hi + 32 * nt * WP + woff;
      const uint16_t* wlr = wt_lo + 32 * nt * WP + woff;
#pragma unroll
      for (int kk = 0; kk < NKK; ++kk) {
        const bf16x8 ahi = *reinterpret_cast<const bf16x8*>(whr + 16 * kk);
        const bf16x8 alo = *reinterpret_cast<const bf16x8*>(wlr + 16 * kk);
        const bf16x8 sv = __builtin_bit_cast(bf16x8, buf[kk]);
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ahi, sv, acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(alo, sv, acc, 0, 0, 0);
      }
      if (!valid) continue;
#pragma unroll
      for (int a = 0; a < 2; ++a) {
        // s of output rows 8 q + 4 hl + u, q = 2 a + b, from k-step 2 nt + a:
        // lane hl keeps or receives the dwords that hold them (b = 0: lo)
        // (scalar copies first: a __builtin_bit_cast of a vector element
        // names element 0 whichever element is written)
        const u32x4 x = buf[2 * nt + a];
        const uint32_t x0 = x[0], x1 = x[1], x2 = x[2], x3 = x[3];
        float lo0, hi0, lo1, hi1;
        lane_half_swap(__builtin_bit_cast(float, x0), __builtin_bit_cast(float, x2), lo0, hi0);
        lane_half_swap(__builtin_bit_cast(float, x1), __builtin_bit_cast(float, x3), lo1, hi1);
#pragma unroll
        for (int b = 0; b < 2; ++b) {
          const int q = 2 * a + b;
          const int d0 = 32 * nt + 8 * q + 4 * hl;
          f32x4 v;
          if (pi >= 0) {
            v = *reinterpret_cast<const f32x4*>(O_probe + ((size_t)h * m + pi) * D + d0);
          } else {
            const uint32_t p0 = __builtin_bit_cast(uint32_t, b ? hi0 : lo0);
            const uint32_t p1 = __builtin_bit_cast(uint32_t, b ? hi1 : lo1);
            const float sv4[4] = {__builtin_bit_cast(float, p0 << 16),
                                  __builtin_bit_cast(float, p0 & 0xffff0000u),
                                  __builtin_bit_cast(float, p1 << 16),
                                  __builtin_bit_cast(float, p1 & 0xffff0000u)};
#pragma unroll
            for (int u = 0; u < 4; ++u) v[u] = sv4[u] + acc[4 * q + u] + wbias[d0 + u];
          }
          const f32x2 f0 = {v[0], v[1]};
          const f32x2 f1 = {v[2], v[3]};
          const bf16x2 b0 = __builtin_convertvector(f0, bf16x2);
          const bf16x2 b1 = __builtin_convertvector(f1, bf16x2);
          const bf16x4 bv = {b0[0], b0[1], b1[0], b1[1]};
          *reinterpret_cast<bf16x4*>(stg + ql * OP + d0) = bv;
        }
      }
    }
    // every use of buf is issued: it takes the tile three rounds ahead
    if (tile + 3 * NW < t1) load_tile(buf, tile + 3 * NW);
    // whole output rows from the wave's staged tile: 16-byte pieces, one row per D/8 lanes
    __builtin_amdgcn_wave_barrier();
    constexpr int LPR = D / 8;          // lanes per row
    constexpr int RPI = 64 / LPR;       // rows per store instruction
#pragma unroll
    for (int r0 = 0; r0 < 32; r0 += RPI) {
      const int r = r0 + lane / LPR, c = lane % LPR;
      const int rpos = tile * 32 + r;
      const int rtok = __shfl(tok, r);
      if (rpos < N) {
        const u32x4 v = *reinterpret_cast<const u32x4*>(stg + r * OP + 8 * c);
        *reinterpret_cast<u32x4*>(Oh + (size_t)rtok * D + 8 * c) = v;
      }
    }
    __builtin_amdgcn_wave_barrier();
  };
  // three register buffers in rotation: tiles w, w + 8 and w + 16 of this
  // workgroup's range are in flight before the first is used
  u32x4 b0[NKK], b1[NKK], b2[NKK];
  const int tw = t0 + w;
  if (tw < t1) load_tile(b0, tw);
  if (tw + NW < t1) load_tile(b1, tw + NW);
  if (tw + 2 * NW < t1) load_tile(b2, tw + 2 * NW);
  for (int tile = tw; tile < t1; tile += 3 * NW) {
    run_tile(b0, tile);
    if (tile + NW < t1) run_tile(b1, tile + NW);
    if (tile + 2 * NW < t1) run_tile(b2, tile + 2 * NW);
  }
}

hipError_t launch_apply(const Dims& d, const void* S_out, const int32_t* query_perm,
                        const float* O_probe, const float* U, const float* Theta,
                        const int32_t* rank_eff, void* O, char* ws, hipStream_t st) {
  if (d.bf16) {
    const ApplyWs L = apply_ws(d);
    uint16_t* wt = reinterpret_cast<uint16_t*>(ws + L.wt);
    float* bias = reinterpret_cast<float*>(ws + L.bias);
    // workgroups per head: at most kApplyTilesPerWg tiles each, and the grid
    // filled up to whole rounds of resident workgroups (W and the output
    // staging allow one per CU at d = 128, two at d = 64; 256 CUs)
    const int ntile = (d.N + 31) / 32;
    const int base = (ntile + kApplyTilesPerWg - 1) / kApplyTilesPerWg;
    const int slots = 256 * (d.D == 128 ? 1 : 2);
    const int rounds = (d.H * base + slots - 1) / slots;
    int wgph = std::max(base, rounds * slots / d.H);
    wgph = std::min(wgph, std::max(base, (ntile + kApplyWaves - 1) / kApplyWaves));  // a tile per wave at least
    uint16_t* Ob = static_cast<uint16_t*>(O);
    const uint16_t* Sb = static_cast<const uint16_t*>(S_out);
    if (d.D == 128) {
      k_apply_weights<128><<<d.H, 256, 0, st>>>(U, Theta, rank_eff, d.k, wt, bias);
      k_apply_mfma<128><<<d.H * wgph, kApplyWaves * 64, 0, st>>>(Sb, query_perm, O_probe, wt, bias,
                                                                 d.ppos, d.N, d.m, wgph, Ob);
    } else {
      k_apply_weights<64><<<d.H, 256, 0, st>>>(U, Theta, rank_eff, d.k, wt, bias);
      k_apply_mfma<64><<<d.H * wgph, kApplyWaves * 64, 0, st>>>(Sb, query_perm, O_probe, wt, bias,
                                                                d.ppos, d.N, d.m, wgph, Ob);
    }
    return hipGetLastError();
  }
  const dim3 grid((d.N + kApplyRows - 1) / kApplyRows, d.H);
#define SPR_APPLY(B, DD)                                                                   \
  k_apply<B, DD><<<grid, 256, 0, st>>>(static_cast<const float*>(S_out), query_perm, O_probe, \
                                        U, Theta, rank_eff, d.ppos, d.N, \
                                        d.m, d.k, O)
  if (d.D == 128) SPR_APPLY(false, 128); else SPR_APPLY(false, 64);
#undef SPR_APPLY
  return hipGetLastError();
}

}  // namespace spr
