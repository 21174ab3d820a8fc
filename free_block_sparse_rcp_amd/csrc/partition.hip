// Response-coupled partitioning of the keys (arxivdaily 2608.18484, English
// abstract: keys grouped by how they respond to sampled queries; cpu3d
// summary: paired K/V groups).
//
// Lloyd k-means of the key response profiles r_j = tau * Q_s k_j is run with
// key-space centroids kbar_g: since profiles are linear in k,
//   ||r_j - c_g||^2 - ||r_j||^2 = kbar_g^T M kbar_g - 2 k_j^T (M kbar_g),
//   M = tau^2 Q_s^T Q_s,
// so each assignment is a [N x d] x [d x G] contraction plus a bias and a
// row-wise argmin. Every reduction runs in a fixed order, so labels and
// centroids are bit-identical from run to run.
#include "common.hpp"
#include "internal.hpp"

namespace spr {

// ---------------------------------------------------------------- metric M
// M[h] = tau_h^2 * sum_s q_s q_s^T in fp64 (samples added in increasing s).
// Chunks of 32 sampled rows are read with 16-byte loads into a double buffer
// in LDS; the next chunk's loads are in flight while this one is summed.
// grid (H, D/16), block 256.
template <bool BF16, int D>
__global__ __launch_bounds__(256) void k_metric(const void* Qv, const float* scale,
                                                const int32_t* sample_idx, int S, int N,
                                                double* M) {
  using T = typename Elt<BF16>::T;
  constexpr int ROWB = D * (int)sizeof(T);
  constexpr int CPR = ROWB / 16;             // 16-byte chunks per row
  constexpr int EPC = 16 / (int)sizeof(T);   // elements per chunk
  constexpr int LPT = (32 * CPR + 255) / 256;  // loads per thread per chunk of rows
  const char* Q = static_cast<const char*>(Qv) + (size_t)blockIdx.x * N * ROWB;
  __shared__ float xs[2][32][D];
  const int t = threadIdx.x;
  const int i = blockIdx.y * 16 + t / 16;
  const int jl = t % 16;
  constexpr int U = D / 16;
  double acc[U];
#pragma unroll
  for (int u = 0; u < U; ++u) acc[u] = 0.0;
  u32x4 raw[LPT];
  auto fetch = [&](int s0) {
    const int ns = min(32, S - s0);
#pragma unroll
    for (int l = 0; l < LPT; ++l) {
      const int e = t + 256 * l, ss = e / CPR, c = e % CPR;
      raw[l] = u32x4{0u, 0u, 0u, 0u};
      if (e < 32 * CPR && ss < ns)
        raw[l] = *reinterpret_cast<const u32x4*>(Q + (size_t)clamp_idx(sample_idx[s0 + ss], N) * ROWB + c * 16);
    }
  };
  auto stash = [&](int buf) {
#pragma unroll
    for (int l = 0; l < LPT; ++l) {
      const int e = t + 256 * l, ss = e / CPR, c = e % CPR;
      if (e >= 32 * CPR) continue;
      float* dst = &xs[buf][ss][c * EPC];
      if (BF16) {
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          dst[2 * u] = __uint_as_float(raw[l][u] << 16);
          dst[2 * u + 1] = __uint_as_float(raw[l][u] & 0xffff0000u);
        }
      } else {
#pragma unroll
        for (int u = 0; u < 4; ++u) dst[u] = __uint_as_float(raw[l][u]);
      }
    }
  };
  if (S > 0) {
    fetch(0);
    stash(0);
  }
  __syncthreads();
  int buf = 0;
  for (int s0 = 0; s0 < S; s0 += 32) {
    const int ns = min(32, S - s0);
    if (s0 + 32 < S) fetch(s0 + 32);
    for (int ss = 0; ss < ns; ++ss) {
      const double xi = xs[buf][ss][i];
#pragma unroll
      for (int u = 0; u < U; ++u) acc[u] += xi * (double)xs[buf][ss][jl + 16 * u];
    }
    if (s0 + 32 < S) stash(buf ^ 1);
    __syncthreads();
    buf ^= 1;
  }
  const double tau = scale[blockIdx.x];
  double* Mh = M + (size_t)blockIdx.x * D * D;
#pragma unroll
  for (int u = 0; u < U; ++u) Mh[(size_t)i * D + jl + 16 * u] = tau * tau * acc[u];
}

// kbar[h][g] = K[h][init_idx[g]]. grid (G, H), block D.
template <bool BF16, int D>
__global__ void k_centroid_init(const void* Kv, const int32_t* init_idx, int N, int G,
                                float* kbar) {
  using E = Elt<BF16>;
  const int g = blockIdx.x, h = blockIdx.y, e = threadIdx.x;
  const typename E::T* K = static_cast<const typename E::T*>(Kv) + (size_t)h * N * D;
  kbar[((size_t)h * G + g) * D + e] = E::ld(K, (size_t)clamp_idx(init_idx[g], N) * D + e);
}

// P_g = M kbar_g (fp64 accumulate), b_g = kbar_g^T M kbar_g. Stores P in fp32
// and as a bf16 pair P ~ hi + lo (rows [H][G][2][D]), so that a bf16 MFMA with
// exact bf16 keys recovers the product to ~2^-18 relative. Eight groups per
// workgroup, so that M is read once per eight groups: thread (e, set) forms
// P_g[e] for its set's groups in increasing j, and b_g is reduced over e with a
// pairwise tree. grid (ceil(G / 8), H), block 256.
constexpr int kPrepGroups = 8;

template <int D>
__global__ __launch_bounds__(256) void k_centroid_prep_g8(const double* M, const float* kbar, int G,
                                                          float* P, uint16_t* Phl, float* bvec) {
  constexpr int NG = kPrepGroups;
  constexpr int NSET = 256 / D;        // thread sets
  constexpr int GPT = NG / NSET;       // groups per thread
  __shared__ double kb[NG][D];
  __shared__ double rb[NG][D];
  const int h = blockIdx.y, g0 = blockIdx.x * NG, t = threadIdx.x;
  for (int i = t; i < NG * D; i += 256) {
    const int k = i / D, e = i - k * D;
    kb[k][e] = g0 + k < G ? (double)kbar[((size_t)h * G + g0 + k) * D + e] : 0.0;
  }
  __syncthreads();
  const int e = t % D, set = t / D;
  const double* Mh = M + (size_t)h * D * D;
  double p[GPT];
#pragma unroll
  for (int k = 0; k < GPT; ++k) p[k] = 0.0;
  for (int j = 0; j < D; ++j) {
    const double m = Mh[(size_t)j * D + e];   // M symmetric: column e
#pragma unroll
    for (int k = 0; k < GPT; ++k) p[k] += m * kb[set * GPT + k][j];
  }
#pragma unroll
  for (int k = 0; k < GPT; ++k) {
    const int gl = set * GPT + k, g = g0 + gl;
    rb[gl][e] = kb[gl][e] * p[k];
    if (g < G) {
      const size_t o = ((size_t)h * G + g) * D + e;
      P[o] = (float)p[k];
      const uint16_t hi = f32_to_bf16((float)p[k]);
      const uint16_t lo = f32_to_bf16((float)(p[k] - (double)bf16_to_f32(hi)));
      uint16_t* ph = Phl + ((size_t)h * G + g) * 2 * D;
      ph[e] = hi;
      ph[D + e] = lo;
    }
  }
  __syncthreads();
  for (int off = D / 2; off > 0; off >>= 1) {
    for (int i = t; i < NG * off; i += 256) {
      const int k = i / off, x = i - k * off;
      rb[k][x] += rb[k][x + off];
    }
    __syncthreads();
  }
  if (t < NG && g0 + t < G) bvec[(size_t)h * G + g0 + t] = (float)rb[t][0];
}

// ------------------------------------------------- row x centroid argselect
// MODE 0 (assign): score(j,g) = b_g - 2 * (x_j . P_g), argmin, lowest g wins.
// MODE 1 (coords): score(q,g) = tau * (x_q . P_g) over non-empty g, argmax.
// One workgroup = 64 rows; 256 threads, each 4 rows x 4 groups per chunk of
// 64 groups. fp32 dot products accumulated in increasing dimension order.
template <bool BF16, int D, int MODE>
__global__ __launch_bounds__(256) void k_rowvec_argsel(const void* Xv, const float* P,
                                                       const float* bvec, const float* scale,
                                                       const int32_t* group_off, int N, int G,
                                                       int32_t* best_idx, float* best_val,
                                                       float* dbg) {
  using E = Elt<BF16>;
  const int h = blockIdx.y;
  const int r0 = blockIdx.x * 64;
  const int t = threadIdx.x;
  const typename E::T* X = static_cast<const typename E::T*>(Xv) + (size_t)h * N * D;
  __shared__ float xs[64][D + 1];
  __shared__ float ps[64][D + 1];
  __shared__ float bs[64];
  __shared__ int ok[64];
  __shared__ float rv[16][64];
  __shared__ int rg[16][64];
  for (int idx = t; idx < 64 * D; idx += 256) {
    const int r = idx / D, c = idx % D;
    xs[r][c] = (r0 + r < N) ? E::ld(X, (size_t)(r0 + r) * D + c) : 0.f;
  }
  const float tau = MODE == 1 ? scale[h] : 0.f;
  const int ki = t % 16, gi = t / 16;
  float best[4];
  int bestg[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    best[i] = MODE == 0 ? __builtin_inff() : -__builtin_inff();
    bestg[i] = G;  // sentinel: replaced by the first finite candidate
  }
  for (int g0 = 0; g0 < G; g0 += 64) {
    __syncthreads();
    for (int idx = t; idx < 64 * D; idx += 256) {
      const int r = idx / D, c = idx % D;
      ps[r][c] = (g0 + r < G) ? P[((size_t)h * G + g0 + r) * D + c] : 0.f;
    }
    if (t < 64) {
      const int g = g0 + t;
      if (MODE == 0) {
        bs[t] = g < G ? bvec[(size_t)h * G + g] : 0.f;
        ok[t] = g < G;
      } else {
        ok[t] = g < G && group_off[(size_t)h * (G + 1) + g + 1] > group_off[(size_t)h * (G + 1) + g];
      }
    }
    __syncthreads();
    float acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[i][j] = 0.f;
    for (int e = 0; e < D; ++e) {
      float a[4], p[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) a[i] = xs[ki + 16 * i][e];
#pragma unroll
      for (int j = 0; j < 4; ++j) p[j] = ps[gi + 16 * j][e];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(a[i], p[j], acc[i][j]);
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int gl = gi + 16 * j;
      const int g = g0 + gl;
      if (g >= G) continue;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = r0 + ki + 16 * i;
        float s;
        if (MODE == 0) {
          s = bs[gl] - 2.0f * acc[i][j];
        } else {
          s = ok[gl] ? tau * acc[i][j] : -__builtin_inff();
        }
        if (dbg != nullptr && row < N) dbg[((size_t)h * N + row) * G + g] = s;
        if (MODE == 0) {
          if (s < best[i]) { best[i] = s; bestg[i] = g; }
        } else if (ok[gl]) {
          if (s > best[i]) { best[i] = s; bestg[i] = g; }
        }
      }
    }
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    rv[gi][ki + 16 * i] = best[i];
    rg[gi][ki + 16 * i] = bestg[i];
  }
  __syncthreads();
  if (t < 64 && r0 + t < N) {
    float bv = rv[0][t];
    int bg = rg[0][t];
    for (int q = 1; q < 16; ++q) {
      const float s = rv[q][t];
      const int g = rg[q][t];
      if (g == G) continue;
      const bool better = MODE == 0 ? (s < bv || (s == bv && g < bg)) : (s > bv || (s == bv && g < bg));
      if (bg == G || better) { bv = s; bg = g; }
    }
    if (bg == G) bg = 0;  // only if every score was NaN
    best_idx[(size_t)h * N + r0 + t] = bg;
    if (best_val) best_val[(size_t)h * N + r0 + t] = bv;
  }
}

// ------------------------------------------------ row x centroid argselect, MFMA
// Same scores as k_rowvec_argsel for bf16 rows, on v_mfma_f32_32x32x16_bf16:
// the centroid-side vectors are split P = hi + lo (bf16) and both halves are
// multiplied by the exact bf16 rows with fp32 accumulation. The product is
// formed transposed (groups x keys) so that each lane holds one key and 16
// groups. Each workgroup covers 256 groups (8 waves x 32, operands held in
// registers) for a chunk of kRvKeys keys streamed through padded LDS tiles.
// The kernel fits 128 VGPRs, so two workgroups share a CU: the tile's two
// 32-key halves are scored one after the other, the group biases are read
// from LDS, and tile loads use 32-bit offsets from the head's base. The
// per-key winner over its groups is merged into best[h][key] with a 64-bit
// atomicMin on (orderable score << 32 | g), which is order independent, so
// results are deterministic and ties go to the lowest g.
//   MODE 0 (assign): score = b_g - 2 k.P_g, minimised.
//   MODE 1 (coords): score = tau q.kbar_g over non-empty groups, maximised.
constexpr int kRvWaves = 8;
constexpr int kRvKeys = 2048;
constexpr int kRvTile = 64;

template <int D, int MODE>
__global__ __launch_bounds__(kRvWaves * 64) __attribute__((amdgpu_waves_per_eu(4, 4))) void k_rowvec_mfma(
    const uint16_t* X, const uint16_t* Phl, const float* bvec, const float* scale,
    const int32_t* group_off, int N, int G, int nkc, unsigned long long* best, float* dbg) {
  constexpr int NKK = D / 16;
  constexpr int KP = 2 * D + 16;
  constexpr int KCH = KP / 16;
  constexpr int TILEB = kRvTile * KP;
  constexpr int NINS = (TILEB + 1023) / 1024;
  __shared__ __attribute__((aligned(1024))) char kt0[NINS * 1024];
  __shared__ __attribute__((aligned(1024))) char kt1[NINS * 1024];
  __shared__ unsigned long long red[2][kRvWaves][kRvTile];
  __shared__ __attribute__((aligned(16))) float bsh[32 * kRvWaves];
  const int h = blockIdx.y;
  const int kc = blockIdx.x % nkc, gt = blockIdx.x / nkc;
  const int t = threadIdx.x, lane = t & 63, hl = lane >> 5, ql = lane & 31;
  const int w = __builtin_amdgcn_readfirstlane(t >> 6);
  const uint16_t* Xh = X + (size_t)h * N * D;
  // A operands: 32 groups of this wave, rows of hi and lo
  const int gA = gt * (32 * kRvWaves) + 32 * w + ql;
  bf16x8 phi[NKK], plo[NKK];
  {
    const bool ok = gA < G;
    const uint16_t* ph = Phl + ((size_t)h * G + (ok ? gA : 0)) * 2 * D;
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) {
      phi[kk] = *reinterpret_cast<const bf16x8*>(ph + 16 * kk + 8 * hl);
      plo[kk] = *reinterpret_cast<const bf16x8*>(ph + D + 16 * kk + 8 * hl);
      if (!ok) {
        phi[kk] = bf16x8{};
        plo[kk] = bf16x8{};
      }
    }
  }
  // output rows of this lane: groups g(r) = base + 8(r/4) + 4 hl + r%4, increasing in r.
  // Scores are minimised in the form  sgn * acc + bias  (MODE 0: -2 k.P_g + b_g;
  // MODE 1: -tau q.kbar_g); slots that must never win get bias = +inf.
  const int gbase = gt * (32 * kRvWaves) + 32 * w + 4 * hl;
  // per-group bias of this workgroup's groups, in LDS (read back 4 at a time in
  // the epilogue, so that it holds no registers across the tile loop)
  for (int i = t; i < 32 * kRvWaves; i += kRvWaves * 64) {
    const int g = gt * (32 * kRvWaves) + i;
    bool ok = g < G;
    float v;
    if (MODE == 0) {
      v = ok ? bvec[(size_t)h * G + g] : __builtin_inff();
    } else {
      if (ok) ok = group_off[(size_t)h * (G + 1) + g + 1] > group_off[(size_t)h * (G + 1) + g];
      v = ok ? 0.f : __builtin_inff();
    }
    bsh[i] = v;
  }
  const float* brow = bsh + 32 * w + 4 * hl;   // slot r: brow[8 (r / 4) + r % 4]
  const float sgn = MODE == 0 ? -2.0f : -scale[h];
  const int k0 = kc * kRvKeys, k1 = min(N, k0 + kRvKeys);
  const int ntile = (k1 - k0 + kRvTile - 1) / kRvTile;

  auto issue = [&](int tile, char* dst) {
#pragma unroll
    for (int u0 = 0; u0 < NINS; u0 += kRvWaves) {
      const int u = u0 + w;
      const int q = 64 * u + lane;
      if (u < NINS && q * 16 < TILEB) {
        const int r = q / KCH, cc = q - r * KCH;
        // uniform head base + 32-bit lane offset (N d < 2^31 keeps it in range)
        const uint32_t key = (uint32_t)min(k0 + tile * kRvTile + r, N - 1);
        const uint32_t off = key * (uint32_t)(2 * D) + (uint32_t)((cc < D / 8 ? cc : 0) * 16);
        __builtin_amdgcn_global_load_lds((const void*)(reinterpret_cast<const char*>(Xh) + off),
                                         (__attribute__((address_space(3))) void*)(dst + u * 1024),
                                         16, 0, 0);
      }
    }
  };
  // scores of one tile, one 32-key half at a time; the per-key winner of this
  // wave goes to red[tile & 1][w]
  auto compute = [&](int tile, const char* __restrict__ buf) {
    const char* kb = buf + ql * KP + hl * 16;
#pragma unroll
    for (int hk = 0; hk < 2; ++hk) {
      f32x16 acc;
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[r] = 0.f;
#pragma unroll
      for (int kk = 0; kk < NKK; ++kk) {
        const bf16x8 kop = *reinterpret_cast<const bf16x8*>(kb + 32 * hk * KP + 32 * kk);
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(phi[kk], kop, acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(plo[kk], kop, acc, 0, 0, 0);
      }
      const int key = k0 + tile * kRvTile + 32 * hk + ql;
      // lowest-slot minimum of the 16 scores by a pairwise tree (the left
      // operand holds the lower slots and keeps ties), so that the compares of
      // one level are independent; slots whose bias is +inf never win
      float sv[16];
      int si[16];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const f32x4 b4 = *reinterpret_cast<const f32x4*>(brow + 8 * j);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          sv[4 * j + i] = fmaf(sgn, acc[4 * j + i], b4[i]);
          si[4 * j + i] = 4 * j + i;
        }
      }
#pragma unroll
      for (int width = 8; width >= 1; width >>= 1) {
#pragma unroll
        for (int p = 0; p < width; ++p) {
          const bool right = sv[2 * p + 1] < sv[2 * p];
          sv[p] = right ? sv[2 * p + 1] : sv[2 * p];
          si[p] = right ? si[2 * p + 1] : si[2 * p];
        }
      }
      const float bs = sv[0];
      const int br = bs < __builtin_inff() ? si[0] : -1;
      if (dbg != nullptr && key < k1) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const f32x4 b4 = *reinterpret_cast<const f32x4*>(brow + 8 * j);
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int g = gbase + 8 * j + i;
            const float sc = fmaf(sgn, acc[4 * j + i], b4[i]);
            if (g < G) dbg[((size_t)h * N + key) * G + g] = MODE == 0 ? sc : -sc;
          }
        }
      }
      unsigned long long bk = ~0ull;
      if (br >= 0) {
        const int g = gbase + 8 * (br >> 2) + (br & 3);
        const uint32_t ob = MODE == 0 ? float_order_bits(bs) : float_desc_bits(-bs);
        bk = (static_cast<unsigned long long>(ob) << 32) | (uint32_t)g;
      }
      const unsigned long long other = __shfl_xor(bk, 32);
      bk = other < bk ? other : bk;
      if (hl == 0) red[tile & 1][w][32 * hk + ql] = bk;
    }
  };
  // after the barrier that ends a tile, one wave folds that tile's per-wave winners
  auto merge = [&](int tile) {
    if (w == (tile & (kRvWaves - 1))) {
      const int key = k0 + tile * kRvTile + lane;
      unsigned long long m = red[tile & 1][0][lane];
#pragma unroll
      for (int ww = 1; ww < kRvWaves; ++ww) m = red[tile & 1][ww][lane] < m ? red[tile & 1][ww][lane] : m;
      if (key < k1 && m != ~0ull) atomicMin(&best[(size_t)h * N + key], m);
    }
  };

  if (ntile > 0) issue(0, kt0);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  for (int tile = 0; tile < ntile; tile += 2) {
    if (tile + 1 < ntile) issue(tile + 1, kt1);
    compute(tile, kt0);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    merge(tile);
    if (tile + 1 >= ntile) break;
    if (tile + 2 < ntile) issue(tile + 2, kt0);
    compute(tile + 1, kt1);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    merge(tile + 1);
  }
}

__global__ void k_fill_u64(unsigned long long* p, size_t n, unsigned long long v) {
  const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (i < n) p[i] = v;
}

// best -> label (and, for coordinates, the winning value as fp32).
__global__ void k_best_to_label(const unsigned long long* best, size_t n, int descending,
                                int32_t* label, float* value) {
  const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n) return;
  const unsigned long long b = best[i];
  label[i] = b == ~0ull ? 0 : (int32_t)(b & 0xffffffffu);
  if (value != nullptr) {
    uint32_t ob = (uint32_t)(b >> 32);
    if (descending) ob = ~ob;
    const uint32_t bits = (ob & 0x80000000u) ? (ob & 0x7fffffffu) : ~ob;
    value[i] = __uint_as_float(bits);
  }
}

// hi/lo bf16 split of fp32 rows: dst[row][0][:] = hi, dst[row][1][:] = lo.
__global__ void k_split_hilo(const float* src, size_t rows, int D, uint16_t* dst) {
  const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= rows * D) return;
  const size_t r = i / D, e = i % D;
  const float x = src[i];
  const uint16_t hi = f32_to_bf16(x);
  dst[r * 2 * D + e] = hi;
  dst[r * 2 * D + D + e] = f32_to_bf16(x - bf16_to_f32(hi));
}

hipError_t launch_rowvec_mfma(const Dims& d, int mode, const void* X, const uint16_t* Phl,
                              const float* bvec, const float* scale, const int32_t* group_off,
                              unsigned long long* best, float* dbg, hipStream_t st) {
  const size_t n = (size_t)d.H * d.N;
  k_fill_u64<<<(unsigned)((n + 255) / 256), 256, 0, st>>>(best, n, ~0ull);
  const int nkc = (d.N + kRvKeys - 1) / kRvKeys;
  const int ngt = (d.G + 32 * kRvWaves - 1) / (32 * kRvWaves);
  const dim3 grid(nkc * ngt, d.H);
  const uint16_t* Xb = static_cast<const uint16_t*>(X);
  if (d.D == 128) {
    if (mode == 0) k_rowvec_mfma<128, 0><<<grid, kRvWaves * 64, 0, st>>>(Xb, Phl, bvec, scale, group_off, d.N, d.G, nkc, best, dbg);
    else k_rowvec_mfma<128, 1><<<grid, kRvWaves * 64, 0, st>>>(Xb, Phl, bvec, scale, group_off, d.N, d.G, nkc, best, dbg);
  } else {
    if (mode == 0) k_rowvec_mfma<64, 0><<<grid, kRvWaves * 64, 0, st>>>(Xb, Phl, bvec, scale, group_off, d.N, d.G, nkc, best, dbg);
    else k_rowvec_mfma<64, 1><<<grid, kRvWaves * 64, 0, st>>>(Xb, Phl, bvec, scale, group_off, d.N, d.G, nkc, best, dbg);
  }
  return hipGetLastError();
}

hipError_t launch_best_to_label(const Dims& d, const unsigned long long* best, bool descending,
                                int32_t* label, float* value, hipStream_t st) {
  const size_t n = (size_t)d.H * d.N;
  k_best_to_label<<<(unsigned)((n + 255) / 256), 256, 0, st>>>(best, n, descending ? 1 : 0, label, value);
  return hipGetLastError();
}

hipError_t launch_split_hilo(const float* src, size_t rows, int D, uint16_t* dst, hipStream_t st) {
  const size_t n = rows * D;
  k_split_hilo<<<(unsigned)((n + 255) / 256), 256, 0, st>>>(src, rows, D, dst);
  return hipGetLastError();
}

// ------------------------------------------------ stable counting-sort pass
// (kSortChunk, the elements per workgroup of the histogram and scatter passes,
// is declared with the dimensions.)
__device__ __forceinline__ uint32_t digit_of(int32_t key, int shift, uint32_t mask) {
  return (static_cast<uint32_t>(key) >> shift) & mask;
}
__device__ __forceinline__ uint32_t digit_of(uint64_t key, int shift, uint32_t mask) {
  return static_cast<uint32_t>(key >> shift) & mask;
}

// counts layout [H][nbuckets][nchunk]; chunks of kSortChunk elements, taken
// as kSortChunk / 256 consecutive sub-chunks of 256. grid (nchunk, H).
template <typename KeyT>
__global__ __launch_bounds__(256) void k_digit_hist(const KeyT* keys, int N, int nchunk,
                                                    int shift, int bits, int32_t* counts) {
  __shared__ int hist[1024];
  const int nbuckets = 1 << bits;
  const uint32_t mask = nbuckets - 1;
  const int h = blockIdx.y, c = blockIdx.x, t = threadIdx.x;
  for (int b = t; b < nbuckets; b += 256) hist[b] = 0;
  __syncthreads();
#pragma unroll
  for (int sub = 0; sub < kSortChunk / 256; ++sub) {
    const int i = c * kSortChunk + sub * 256 + t;
    if (i < N) atomicAdd(&hist[digit_of(keys[(size_t)h * N + i], shift, mask)], 1);
  }
  __syncthreads();
  for (int b = t; b < nbuckets; b += 256) counts[((size_t)h * nbuckets + b) * nchunk + c] = hist[b];
}

// Exclusive scan over the chunks of each bucket, in place. grid (nbuckets, H).
__global__ __launch_bounds__(256) void k_scan_chunks(int32_t* counts, int nchunk, int nbuckets,
                                                     int32_t* totals) {
  __shared__ int tmp[256];
  const int h = blockIdx.y, b = blockIdx.x;
  int32_t* row = counts + ((size_t)h * nbuckets + b) * nchunk;
  int carry = 0;
  for (int base = 0; base < nchunk; base += 256) {
    const int i = base + threadIdx.x;
    const int v = i < nchunk ? row[i] : 0;
    int tot;
    const int ex = block_exclusive_scan<256>(v, tmp, &tot);
    if (i < nchunk) row[i] = carry + ex;
    carry += tot;
  }
  if (threadIdx.x == 0) totals[(size_t)h * nbuckets + b] = carry;
}

// Exclusive scan over buckets; optionally the group offsets. grid (H), block 1024.
__global__ __launch_bounds__(1024) void k_scan_buckets(const int32_t* totals, int nbuckets,
                                                       int32_t* starts, int32_t* group_off, int G,
                                                       int N) {
  __shared__ int tmp[1024];
  const int h = blockIdx.x, t = threadIdx.x;
  const int v = t < nbuckets ? totals[(size_t)h * nbuckets + t] : 0;
  int tot;
  const int ex = block_exclusive_scan<1024>(v, tmp, &tot);
  if (t < nbuckets) starts[(size_t)h * nbuckets + t] = ex;
  if (group_off != nullptr) {
    if (t < G) group_off[(size_t)h * (G + 1) + t] = ex;
    if (t == 0) group_off[(size_t)h * (G + 1) + G] = N;
  }
}

// Stable scatter: the chunk's sub-chunks of 256 are taken in order; in each,
// a key's rank comes from wavefront ballots over the digit bits and per-wave
// digit counts in LDS, after the keys of that digit in the earlier sub-chunks
// (running count). grid (nchunk, H).
template <typename KeyT, bool WRITE_KEYS>
__global__ __launch_bounds__(256) void k_digit_scatter(const KeyT* keys_in, KeyT* keys_out,
                                                       const int32_t* vals_in, int32_t* vals_out,
                                                       int N, int nchunk, int shift, int bits,
                                                       const int32_t* counts,
                                                       const int32_t* starts) {
  __shared__ int wcnt[4 * 1024];
  __shared__ int running[1024];
  const int nbuckets = 1 << bits;
  const uint32_t mask = nbuckets - 1;
  const int h = blockIdx.y, c = blockIdx.x, t = threadIdx.x, w = t >> 6;
  for (int b = t; b < 4 * nbuckets; b += 256) wcnt[b] = 0;
  for (int b = t; b < nbuckets; b += 256) running[b] = 0;
  __syncthreads();
  const uint64_t lt = lanemask_lt();
  for (int sub = 0; sub < kSortChunk / 256; ++sub) {
    const int i = c * kSortChunk + sub * 256 + t;
    if (c * kSortChunk + sub * 256 >= N) break;   // uniform: no key left in the chunk
    const bool valid = i < N;
    const KeyT key = valid ? keys_in[(size_t)h * N + i] : KeyT(0);
    const uint32_t dg = digit_of(key, shift, mask);
    uint64_t match = __ballot(valid);
    for (int bit = 0; bit < bits; ++bit) {
      const bool set = (dg >> bit) & 1u;
      const uint64_t bb = __ballot(valid && set);
      match &= set ? bb : ~bb;
    }
    const int rank = __popcll(match & lt);
    const bool leader = valid && (match & lt) == 0;
    if (leader) wcnt[w * nbuckets + dg] = __popcll(match);
    __syncthreads();
    if (valid) {
      int before = running[dg];
      for (int ww = 0; ww < w; ++ww) before += wcnt[ww * nbuckets + dg];
      const int pos = starts[(size_t)h * nbuckets + dg] +
                      counts[((size_t)h * nbuckets + dg) * nchunk + c] + before + rank;
      if (WRITE_KEYS) keys_out[(size_t)h * N + pos] = key;
      vals_out[(size_t)h * N + pos] = vals_in ? vals_in[(size_t)h * N + i] : i;
    }
    __syncthreads();
    if (leader) {
      atomicAdd(&running[dg], __popcll(match));
      wcnt[w * nbuckets + dg] = 0;
    }
    __syncthreads();
  }
}

// ------------------------------------------------ deterministic group means
// kbar_g = mean of the rows of group g (positions [off_g, off_g+1) of the
// group-contiguous order), for non-empty groups; empty groups keep kbar. Each
// row is read once: a row is split into 16-byte chunks over CPR threads, and
// the workgroup's 256 / CPR row slots take rows slot, slot + 256 / CPR, ... in
// increasing order; the slots are then added in slot order, so the sum order is
// fixed. GATHER (the final grouping): each chunk read is also written to its
// group-contiguous place in Kp, and the same chunk of V to Vp, so the paired
// K/V groups cost no second read of K. grid (G, H), block 256.
template <bool BF16, int D, bool GATHER>
__global__ __launch_bounds__(256) void k_group_mean(const void* Kv, const int32_t* key_perm,
                                                    const int32_t* group_off, int N, int G,
                                                    float* kbar, const void* Vv, void* Kpv,
                                                    void* Vpv) {
  using T = typename Elt<BF16>::T;
  constexpr int ROWB = D * (int)sizeof(T);
  constexpr int CPR = ROWB / 16;              // threads per row
  constexpr int EPC = 16 / (int)sizeof(T);    // elements per chunk
  constexpr int RPP = 256 / CPR;              // rows per pass
  constexpr int U = 8;                        // row loads in flight per thread
  constexpr int PCH = 64 * RPP;               // key indices staged per chunk (a multiple of RPP)
  __shared__ float red[RPP * D];
  __shared__ int pidx[PCH];
  const int g = blockIdx.x, h = blockIdx.y, t = threadIdx.x;
  const int32_t* off = group_off + (size_t)h * (G + 1);
  const int b = off[g], e = off[g + 1];
  if (e <= b) return;
  const int cc = t % CPR, slot = t / CPR;
  const char* K = static_cast<const char*>(Kv) + (size_t)h * N * ROWB + cc * 16;
  const char* V = GATHER ? static_cast<const char*>(Vv) + (size_t)h * N * ROWB + cc * 16 : nullptr;
  char* Kp = GATHER ? static_cast<char*>(Kpv) + (size_t)h * N * ROWB + cc * 16 : nullptr;
  char* Vp = GATHER ? static_cast<char*>(Vpv) + (size_t)h * N * ROWB + cc * 16 : nullptr;
  const int32_t* perm = key_perm + (size_t)h * N;
  float acc[EPC];
#pragma unroll
  for (int j = 0; j < EPC; ++j) acc[j] = 0.f;
  auto add = [&](const u32x4 raw) {
    if (BF16) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        acc[2 * j] += __uint_as_float(raw[j] << 16);
        acc[2 * j + 1] += __uint_as_float(raw[j] & 0xffff0000u);
      }
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[j] += __uint_as_float(raw[j]);
    }
  };
  // The group's key indices are staged in LDS a chunk at a time, so the row
  // loads do not wait behind dependent index loads. Thread (slot, cc) adds
  // rows b + slot, b + slot + RPP, ... in that order whatever the chunking
  // (PCH is a multiple of RPP), so the sum is the same as a plain loop.
  for (int c0 = b; c0 < e; c0 += PCH) {
    const int n = min(PCH, e - c0);
    __syncthreads();
    for (int j = t; j < n; j += 256) pidx[j] = clamp_idx(perm[c0 + j], N);
    __syncthreads();
    int i = slot;
    for (; i + (U - 1) * RPP < n; i += U * RPP) {
      u32x4 raw[U], vraw[U];
#pragma unroll
      for (int u = 0; u < U; ++u)
        raw[u] = *reinterpret_cast<const u32x4*>(K + (size_t)pidx[i + u * RPP] * ROWB);
      if (GATHER) {
#pragma unroll
        for (int u = 0; u < U; ++u)
          vraw[u] = *reinterpret_cast<const u32x4*>(V + (size_t)pidx[i + u * RPP] * ROWB);
      }
#pragma unroll
      for (int u = 0; u < U; ++u) add(raw[u]);
      if (GATHER) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const size_t dst = (size_t)(c0 + i + u * RPP) * ROWB;
          *reinterpret_cast<u32x4*>(Kp + dst) = raw[u];
          *reinterpret_cast<u32x4*>(Vp + dst) = vraw[u];
        }
      }
    }
    for (; i < n; i += RPP) {
      const u32x4 raw = *reinterpret_cast<const u32x4*>(K + (size_t)pidx[i] * ROWB);
      add(raw);
      if (GATHER) {
        const size_t dst = (size_t)(c0 + i) * ROWB;
        *reinterpret_cast<u32x4*>(Kp + dst) = raw;
        *reinterpret_cast<u32x4*>(Vp + dst) =
            *reinterpret_cast<const u32x4*>(V + (size_t)pidx[i] * ROWB);
      }
    }
  }
#pragma unroll
  for (int j = 0; j < EPC; ++j) red[slot * D + cc * EPC + j] = acc[j];
  __syncthreads();
  if (t < D) {
    float s = 0.f;
    for (int k = 0; k < RPP; ++k) s += red[k * D + t];
    kbar[((size_t)h * G + g) * D + t] = s / (float)(e - b);
  }
}

// Random-block variant: label of key perm[i] is the run g with
// floor(gN/G) <= i < floor((g+1)N/G). grid (ceil(N/256), H).
// M = I per head (d x d, fp64). grid (ceil(d*d/256), H), block 256.
__global__ void k_identity_f64(int D, double* M) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i < D * D) M[(size_t)blockIdx.y * D * D + i] = (i / D == i % D) ? 1.0 : 0.0;
}

__global__ void k_random_labels(const int32_t* perm, int N, int G, int32_t* labels) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i >= N) return;
  int64_t g = ((int64_t)i * G) / N;
  while (g + 1 < G && ((g + 1) * (int64_t)N) / G <= i) ++g;
  while (g > 0 && (g * (int64_t)N) / G > i) --g;
  labels[(size_t)blockIdx.y * N + clamp_idx(perm[i], N)] = (int32_t)g;
}

__global__ void k_fill_i32(int32_t* p, size_t n, int32_t v) {
  const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (i < n) p[i] = v;
}
__global__ void k_fill_f32(float* p, size_t n, float v) {
  const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (i < n) p[i] = v;
}

// ------------------------------------------------------------- launchers
#define SPR_CHECK_LAUNCH()                              \
  do {                                                  \
    hipError_t e__ = hipGetLastError();                 \
    if (e__ != hipSuccess) return e__;                  \
  } while (0)

hipError_t launch_sort_pass_u32(const Dims& d, const int32_t* keys_in, int bits,
                                const int32_t* vals_in, int32_t* vals_out, int32_t* counts,
                                int32_t* totals, int32_t* starts, int32_t* group_off_out,
                                hipStream_t st) {
  const int nb = 1 << bits;
  k_digit_hist<int32_t><<<dim3(d.nchunk, d.H), 256, 0, st>>>(keys_in, d.N, d.nchunk, 0, bits,
                                                              counts);
  SPR_CHECK_LAUNCH();
  k_scan_chunks<<<dim3(nb, d.H), 256, 0, st>>>(counts, d.nchunk, nb, totals);
  SPR_CHECK_LAUNCH();
  k_scan_buckets<<<d.H, 1024, 0, st>>>(totals, nb, starts, group_off_out, d.G, d.N);
  SPR_CHECK_LAUNCH();
  k_digit_scatter<int32_t, false><<<dim3(d.nchunk, d.H), 256, 0, st>>>(
      keys_in, nullptr, vals_in, vals_out, d.N, d.nchunk, 0, bits, counts, starts);
  SPR_CHECK_LAUNCH();
  return hipSuccess;
}

hipError_t launch_sort_pass_u64(const Dims& d, const uint64_t* keys_in, uint64_t* keys_out,
                                int shift, int bits, const int32_t* vals_in, int32_t* vals_out,
                                int32_t* counts, int32_t* totals, int32_t* starts,
                                hipStream_t st) {
  const int nb = 1 << bits;
  k_digit_hist<uint64_t><<<dim3(d.nchunk, d.H), 256, 0, st>>>(keys_in, d.N, d.nchunk, shift,
                                                               bits, counts);
  SPR_CHECK_LAUNCH();
  k_scan_chunks<<<dim3(nb, d.H), 256, 0, st>>>(counts, d.nchunk, nb, totals);
  SPR_CHECK_LAUNCH();
  k_scan_buckets<<<d.H, 1024, 0, st>>>(totals, nb, starts, nullptr, d.G, d.N);
  SPR_CHECK_LAUNCH();
  if (keys_out != nullptr) {
    k_digit_scatter<uint64_t, true><<<dim3(d.nchunk, d.H), 256, 0, st>>>(
        keys_in, keys_out, vals_in, vals_out, d.N, d.nchunk, shift, bits, counts, starts);
  } else {
    k_digit_scatter<uint64_t, false><<<dim3(d.nchunk, d.H), 256, 0, st>>>(
        keys_in, nullptr, vals_in, vals_out, d.N, d.nchunk, shift, bits, counts, starts);
  }
  SPR_CHECK_LAUNCH();
  return hipSuccess;
}

template <bool BF16, int D>
static hipError_t partition_impl(const Dims& d, const void* Q, const void* K, const void* V,
                                 const float* scale, const int32_t* sample_idx,
                                 const int32_t* init_idx, const int32_t* rand_key_perm,
                                 int32_t* key_label, int32_t* key_perm, int32_t* group_off,
                                 float* kbar, void* Kp, void* Vp, float* dbg, char* ws,
                                 hipStream_t st) {
  const PartitionWs L = partition_ws(d);
  double* M = reinterpret_cast<double*>(ws + L.M);
  float* P = reinterpret_cast<float*>(ws + L.P);
  uint16_t* Phl = reinterpret_cast<uint16_t*>(ws + L.Phl);
  float* bvec = reinterpret_cast<float*>(ws + L.bvec);
  int32_t* counts = reinterpret_cast<int32_t*>(ws + L.counts);
  int32_t* totals = reinterpret_cast<int32_t*>(ws + L.totals);
  int32_t* starts = reinterpret_cast<int32_t*>(ws + L.starts);
  unsigned long long* best = reinterpret_cast<unsigned long long*>(ws + L.best);
  const dim3 rows64((d.N + 63) / 64, d.H);
  const dim3 per_group(d.G, d.H);

  // groups from the labels, then their means; the final grouping also forms
  // the paired K/V groups (when they are wanted) in the same pass over K
  auto regroup = [&](bool last) -> hipError_t {
    hipError_t e = launch_sort_pass_u32(d, key_label, d.gbits, nullptr, key_perm, counts, totals,
                                        starts, group_off, st);
    if (e != hipSuccess) return e;
    if (last && Kp != nullptr)
      k_group_mean<BF16, D, true><<<per_group, 256, 0, st>>>(K, key_perm, group_off, d.N, d.G,
                                                             kbar, V, Kp, Vp);
    else
      k_group_mean<BF16, D, false><<<per_group, 256, 0, st>>>(K, key_perm, group_off, d.N, d.G,
                                                              kbar, nullptr, nullptr, nullptr);
    SPR_CHECK_LAUNCH();
    return hipSuccess;
  };

  if (d.mode != SPARSEPR_RANDOM_BLOCK) {
    if (d.mode == SPARSEPR_RESPONSE_COUPLED) {
      k_metric<BF16, D><<<dim3(d.H, D / 16), 256, 0, st>>>(Q, scale, sample_idx, d.S, d.N, M);
    } else {
      // semantic mode: plain squared distances between raw rows
      k_identity_f64<<<dim3((D * D + 255) / 256, d.H), 256, 0, st>>>(D, M);
    }
    SPR_CHECK_LAUNCH();
    k_centroid_init<BF16, D><<<per_group, D, 0, st>>>(K, init_idx, d.N, d.G, kbar);
    SPR_CHECK_LAUNCH();
    for (int it = 0; it < d.T; ++it) {
      k_centroid_prep_g8<D><<<dim3((d.G + kPrepGroups - 1) / kPrepGroups, d.H), 256, 0, st>>>(
          M, kbar, d.G, P, Phl, bvec);
      SPR_CHECK_LAUNCH();
      float* dbg_it = (it == d.T - 1) ? dbg : nullptr;
      if (BF16) {
        hipError_t e = launch_rowvec_mfma(d, 0, K, Phl, bvec, nullptr, nullptr, best, dbg_it, st);
        if (e == hipSuccess) e = launch_best_to_label(d, best, false, key_label, nullptr, st);
        if (e != hipSuccess) return e;
      } else {
        k_rowvec_argsel<BF16, D, 0><<<rows64, 256, 0, st>>>(K, P, bvec, nullptr, nullptr, d.N, d.G,
                                                             key_label, nullptr, dbg_it);
        SPR_CHECK_LAUNCH();
      }
      hipError_t e = regroup(it == d.T - 1);
      if (e != hipSuccess) return e;
    }
  } else {
    const size_t nl = (size_t)d.H * d.N;
    k_fill_i32<<<(unsigned)((nl + 255) / 256), 256, 0, st>>>(key_label, nl, 0);
    SPR_CHECK_LAUNCH();
    const size_t nk = (size_t)d.H * d.G * D;
    k_fill_f32<<<(unsigned)((nk + 255) / 256), 256, 0, st>>>(kbar, nk, 0.f);
    SPR_CHECK_LAUNCH();
    k_random_labels<<<dim3((d.N + 255) / 256, d.H), 256, 0, st>>>(rand_key_perm, d.N, d.G,
                                                                   key_label);
    SPR_CHECK_LAUNCH();
    hipError_t e = regroup(true);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

hipError_t launch_partition(const Dims& d, const void* Q, const void* K, const void* V,
                            const float* scale, const int32_t* sample_idx, const int32_t* init_idx,
                            const int32_t* rand_key_perm, int32_t* key_label, int32_t* key_perm,
                            int32_t* group_off, float* kbar, void* Kp, void* Vp, float* dbg,
                            char* ws, hipStream_t st) {
#define SPR_PART(B, DD)                                                                       \
  return partition_impl<B, DD>(d, Q, K, V, scale, sample_idx, init_idx, rand_key_perm,        \
                               key_label, key_perm, group_off, kbar, Kp, Vp, dbg, ws, st)
  if (d.bf16) {
    if (d.D == 128) SPR_PART(true, 128);
    SPR_PART(true, 64);
  } else {
    if (d.D == 128) SPR_PART(false, 128);
    SPR_PART(false, 64);
  }
#undef SPR_PART
}

hipError_t launch_fill_i32(int32_t* p, size_t n, int32_t v, hipStream_t st) {
  if (n == 0) return hipSuccess;
  k_fill_i32<<<(unsigned)((n + 255) / 256), 256, 0, st>>>(p, n, v);
  return hipGetLastError();
}
hipError_t launch_fill_f32(float* p, size_t n, float v, hipStream_t st) {
  if (n == 0) return hipSuccess;
  k_fill_f32<<<(unsigned)((n + 255) / 256), 256, 0, st>>>(p, n, v);
  return hipGetLastError();
}

// Coordinates argmax is shared with route.hip through this launcher.
hipError_t launch_coords_valu(const Dims& d, const void* Q, const float* kbar, const float* scale,
                              const int32_t* group_off, int32_t* g1, float* v, float* dbg,
                              hipStream_t st) {
  const dim3 rows64((d.N + 63) / 64, d.H);
#define SPR_COORD(B, DD)                                                                        \
  k_rowvec_argsel<B, DD, 1><<<rows64, 256, 0, st>>>(Q, kbar, nullptr, scale, group_off, d.N, d.G, \
                                                    g1, v, dbg)
  if (d.bf16) {
    if (d.D == 128) SPR_COORD(true, 128); else SPR_COORD(true, 64);
  } else {
    if (d.D == 128) SPR_COORD(false, 128); else SPR_COORD(false, 64);
  }
#undef SPR_COORD
  return hipGetLastError();
}

}  // namespace spr
