// Query coordinates, query grouping and shared routing (arxivdaily
// 2608.18484, English abstract: queries grouped by their responses to the
// key-group centroids for shared sparse routing; peercurrent abstract: the
// centroids induce query-response coordinates).
#include "common.hpp"
#include "internal.hpp"

namespace spr {

hipError_t launch_coords_valu(const Dims& d, const void* Q, const float* kbar, const float* scale,
                              const int32_t* group_off, int32_t* g1, float* v, float* dbg,
                              hipStream_t st);

// Sort key of a query: (dominant group ascending, value descending); the
// stable passes keep token order for equal keys. grid (ceil(N/256), H).
__global__ void k_make_qkeys(const int32_t* g1, const float* v, int N, uint64_t* keys,
                             int32_t* dbg_dom, float* dbg_val) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i >= N) return;
  const size_t o = (size_t)blockIdx.y * N + i;
  const int g = g1[o];
  const float x = v[o];
  keys[o] = (static_cast<uint64_t>(static_cast<uint32_t>(g)) << 32) | float_desc_bits(x);
  if (dbg_dom) dbg_dom[o] = g;
  if (dbg_val) dbg_val[o] = x;
}

// out[h] = perm (head stride 0: one order shared by every head) or perm[h]
// (head stride N: an order per head).
__global__ void k_copy_perm(const int32_t* perm, size_t head_stride, int N, int32_t* out) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i < N) out[(size_t)blockIdx.y * N + i] = clamp_idx(perm[blockIdx.y * head_stride + i], N);
}

// Mean query of each block and its scores against every group:
// sigma[b,g] = tau * qbar_b . kbar_g over non-empty groups (-inf for empty).
// A workgroup takes kRsBlocks consecutive blocks: their query rows are
// gathered with 16-byte loads and summed per column (row groups combined in a
// fixed order); the scores of the 16 blocks against kRsGroups groups at a time
// are fp32 MFMA tiles (16 x 16 per wave), centroids read from L2.
// grid (ceil(nb / kRsBlocks), H), block 256.
constexpr int kRsBlocks = 16;
constexpr int kRsGroups = 64;

template <bool BF16, int D>
__global__ __launch_bounds__(256) void k_route_scores(const void* Qv, const int32_t* query_perm,
                                                      const float* kbar, const float* scale,
                                                      const int32_t* group_off, int N, int BQ,
                                                      int nb, int G, float* sigma, float* dbg) {
  using T = typename Elt<BF16>::T;
  constexpr int ROWB = D * (int)sizeof(T);
  constexpr int CPR = ROWB / 16;             // 16-byte chunks per row
  constexpr int EPC = 16 / (int)sizeof(T);   // elements per chunk
  constexpr int RG = 256 / CPR;              // row groups
  __shared__ float qb[kRsBlocks][D];
  __shared__ float part[RG][D];
  const int h = blockIdx.y, b0 = blockIdx.x * kRsBlocks, t = threadIdx.x;
  const char* Q = static_cast<const char*>(Qv) + (size_t)h * N * ROWB;
  const int32_t* qp = query_perm + (size_t)h * N;
  const int nblk = min(kRsBlocks, nb - b0);
  {
    const int c = t % CPR, rg = t / CPR;
    // one round of eight row chunks of block j starting at row r0 (rows past
    // the block's end re-read its last row and are not added)
    auto load_round = [&](int j, int r0, u32x4* raw) {
      const int p0 = (b0 + j) * BQ, n = min(N, p0 + BQ) - p0;
#pragma unroll
      for (int v = 0; v < 8; ++v) {
        const int r = r0 + v * RG;
        const int tok = clamp_idx(qp[p0 + min(r, n - 1)], N);
        raw[v] = *reinterpret_cast<const u32x4*>(Q + (size_t)tok * ROWB + c * 16);
      }
    };
    // the next block's first round is issued as soon as this block's last
    // round has been added, so it is in flight during the reduction below
    u32x4 raw[8];
    if (nblk > 0) load_round(0, rg, raw);
    for (int j = 0; j < nblk; ++j) {
      const int p0 = (b0 + j) * BQ, n = min(N, p0 + BQ) - p0;
      float acc[EPC];
#pragma unroll
      for (int u = 0; u < EPC; ++u) acc[u] = 0.f;
      // rows rg, rg + RG, ... in increasing order, eight loads in flight
      for (int r0 = rg;; r0 += 8 * RG) {
        if (r0 != rg) load_round(j, r0, raw);
#pragma unroll
        for (int v = 0; v < 8; ++v) {
          if (r0 + v * RG >= n) break;
          if (BF16) {
#pragma unroll
            for (int u = 0; u < 4; ++u) {
              acc[2 * u] += __uint_as_float(raw[v][u] << 16);
              acc[2 * u + 1] += __uint_as_float(raw[v][u] & 0xffff0000u);
            }
          } else {
#pragma unroll
            for (int u = 0; u < 4; ++u) acc[u] += __uint_as_float(raw[v][u]);
          }
        }
        if (r0 + 8 * RG >= n) {
          if (j + 1 < nblk) load_round(j + 1, rg, raw);
          break;
        }
      }
#pragma unroll
      for (int u = 0; u < EPC; ++u) part[rg][c * EPC + u] = acc[u];
      __syncthreads();
      if (t < D) {
        float s = 0.f;
        for (int i = 0; i < RG; ++i) s += part[i][t];
        qb[j][t] = s / (float)n;
      }
      __syncthreads();
    }
  }
  const float tau = scale[h];
  const int32_t* off = group_off + (size_t)h * (G + 1);
  const int lane = t & 63, w = t >> 6, r16 = lane & 15, kq = lane >> 4;
  static_assert(kRsBlocks == 16 && kRsGroups == 64 && D % 4 == 0, "16 x 64 score tiles on four waves");
  for (int g0 = 0; g0 < G; g0 += kRsGroups) {
    // wave w: the 16 blocks x groups [g0 + 16 w, g0 + 16 w + 16) with
    // v_mfma_f32_16x16x4_f32 (fp32 products and sums); lane (r16, kq) feeds
    // block r16 (LDS) and group 16 w + r16 (read from L2) at d = k0 + kq, and
    // receives blocks 4 kq .. 4 kq + 3 of group 16 w + r16
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    const float* arow = &qb[r16][kq];
    const float* brow = kbar + ((size_t)h * G + min(g0 + 16 * w + r16, G - 1)) * D + kq;
    float bv[D / 4];
#pragma unroll
    for (int u = 0; u < D / 4; ++u) bv[u] = brow[4 * u];
#pragma unroll
    for (int u = 0; u < D / 4; ++u)
      acc = __builtin_amdgcn_mfma_f32_16x16x4f32(arow[4 * u], bv[u], acc, 0, 0, 0);
    const int g = g0 + 16 * w + r16;
    if (g < G) {
      const bool ne = off[g + 1] > off[g];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int j = 4 * kq + u;
        if (j < nblk) {
          const float sc = ne ? tau * acc[u] : -__builtin_inff();
          sigma[((size_t)h * nb + b0 + j) * G + g] = sc;
          if (dbg) dbg[((size_t)h * nb + b0 + j) * G + g] = sc;
        }
      }
    }
  }
}

// Per block: rank non-empty groups by (sigma desc, g asc) with a bitonic sort
// in LDS, take the longest ranked prefix with total size <= kappa (at least
// one group), and list the chosen groups in ascending g.
// grid (nb, H), block 256; G <= 1024.
__global__ __launch_bounds__(256) void k_block_select(const float* sigma,
                                                      const int32_t* group_off, int G,
                                                      int64_t kappa, int32_t* sel,
                                                      int32_t* selcnt, int64_t* blkkeys) {
  constexpr int NT = 256;
  const int b = blockIdx.x, h = blockIdx.y, nb = gridDim.x, t = threadIdx.x;
  __shared__ uint64_t key[1024];
  __shared__ int flag[1024];
  __shared__ int tmp[NT];
  __shared__ int s_keys;
  int GP = 1;
  while (GP < G) GP <<= 1;
  const int32_t* off = group_off + (size_t)h * (G + 1);
  const float* sg = sigma + ((size_t)h * nb + b) * G;
  for (int i = t; i < GP; i += NT) {
    uint64_t k = ~0ull;
    if (i < G && off[i + 1] > off[i]) k = (static_cast<uint64_t>(float_desc_bits(sg[i])) << 32) | (uint32_t)i;
    key[i] = k;
    if (i < G) flag[i] = 0;
  }
  __syncthreads();
  for (int k = 2; k <= GP; k <<= 1) {
    for (int j = k >> 1; j > 0; j >>= 1) {
      for (int i = t; i < GP; i += NT) {
        const int ixj = i ^ j;
        if (ixj > i) {
          const uint64_t a = key[i], c = key[ixj];
          const bool up = (i & k) == 0;
          if ((a > c) == up) {
            key[i] = c;
            key[ixj] = a;
          }
        }
      }
      __syncthreads();
    }
  }
  // inclusive prefix of sizes in ranked order; each thread owns E consecutive entries
  const int E = (GP + NT - 1) / NT;
  int loc[4];
  int own = 0;
  for (int u = 0; u < E; ++u) {
    const int i = t * E + u;
    int sz = 0;
    if (i < GP && key[i] != ~0ull) {
      const int g = (int)(key[i] & 0xffffffffu);
      sz = off[g + 1] - off[g];
    }
    loc[u] = sz;
    own += sz;
  }
  int total;
  const int ex = block_exclusive_scan<NT>(own, tmp, &total);
  int fits = 0;
  int incl = ex;
  int inclv[4];
  for (int u = 0; u < E; ++u) {
    const int i = t * E + u;
    incl += loc[u];
    inclv[u] = incl;
    if (i < GP && key[i] != ~0ull && (int64_t)incl <= kappa) ++fits;
  }
  int nfit;
  (void)block_exclusive_scan<NT>(fits, tmp, &nfit);
  const int count = nfit > 0 ? nfit : 1;
  for (int u = 0; u < E; ++u)
    if (t * E + u == count - 1) s_keys = inclv[u];
  for (int i = t; i < count; i += NT) flag[(int)(key[i] & 0xffffffffu)] = 1;
  __syncthreads();
  // ascending compaction of the chosen groups
  int32_t* out = sel + ((size_t)h * nb + b) * G;
  int base = 0;
  for (int g0 = 0; g0 < G; g0 += NT) {
    const int g = g0 + t;
    const int f = g < G ? flag[g] : 0;
    int tot;
    const int ex = block_exclusive_scan<NT>(f, tmp, &tot);
    if (f) out[base + ex] = g;
    base += tot;
  }
  if (t == 0) {
    selcnt[(size_t)h * nb + b] = count;
    blkkeys[(size_t)h * nb + b] = s_keys;
  }
}

// block_ptr = exclusive scan of the per-block counts; executed pairs =
// sum_b n_b |K(b)| + m N. grid (H), block 1024.
__global__ __launch_bounds__(1024) void k_csr_scan(const int32_t* selcnt, const int64_t* blkkeys,
                                                   int nb, int N, int BQ, int m,
                                                   int32_t* block_ptr, int64_t* executed) {
  constexpr int NT = 1024;
  __shared__ int tmp[NT];
  __shared__ long long red[NT];
  const int h = blockIdx.x, t = threadIdx.x;
  int carry = 0;
  long long pairs = 0;
  for (int base = 0; base < nb; base += NT) {
    const int b = base + t;
    const int v = b < nb ? selcnt[(size_t)h * nb + b] : 0;
    int tot;
    const int ex = block_exclusive_scan<NT>(v, tmp, &tot);
    if (b < nb) {
      block_ptr[(size_t)h * (nb + 1) + b] = carry + ex;
      const int nrow = min(N, (b + 1) * BQ) - b * BQ;
      pairs += (long long)nrow * blkkeys[(size_t)h * nb + b];
    }
    carry += tot;
  }
  red[t] = pairs;
  __syncthreads();
  for (int o = NT / 2; o > 0; o >>= 1) {
    if (t < o) red[t] += red[t + o];
    __syncthreads();
  }
  if (t == 0) {
    block_ptr[(size_t)h * (nb + 1) + nb] = carry;
    executed[h] = red[0] + (long long)m * N;
  }
}

// Copy each block's chosen groups into the CSR. grid (nb, H), block 256.
__global__ void k_csr_copy(const int32_t* sel, const int32_t* selcnt, const int32_t* block_ptr,
                           int G, int32_t* block_groups) {
  const int b = blockIdx.x, h = blockIdx.y, nb = gridDim.x;
  const int cnt = selcnt[(size_t)h * nb + b];
  const int p = block_ptr[(size_t)h * (nb + 1) + b];
  const int32_t* src = sel + ((size_t)h * nb + b) * G;
  int32_t* dst = block_groups + (size_t)h * nb * G + p;
  for (int i = threadIdx.x; i < cnt; i += 256) dst[i] = src[i];
}

#define SPR_CHECK_LAUNCH()                              \
  do {                                                  \
    hipError_t e__ = hipGetLastError();                 \
    if (e__ != hipSuccess) return e__;                  \
  } while (0)

hipError_t launch_route(const Dims& d, const void* Q, const float* scale, const float* kbar,
                        const int32_t* group_off, const int32_t* rand_query_perm,
                        int32_t* query_perm, int32_t* block_ptr, int32_t* block_groups,
                        int64_t* executed_pairs, float* dbg_coords, int32_t* dbg_dom,
                        float* dbg_domval, float* dbg_sigma, char* ws, hipStream_t st) {
  const RouteWs L = route_ws(d);
  uint64_t* keysA = reinterpret_cast<uint64_t*>(ws + L.keysA);
  uint64_t* keysB = reinterpret_cast<uint64_t*>(ws + L.keysB);
  int32_t* valsA = reinterpret_cast<int32_t*>(ws + L.valsA);
  int32_t* valsB = reinterpret_cast<int32_t*>(ws + L.valsB);
  int32_t* counts = reinterpret_cast<int32_t*>(ws + L.counts);
  int32_t* totals = reinterpret_cast<int32_t*>(ws + L.totals);
  int32_t* starts = reinterpret_cast<int32_t*>(ws + L.starts);
  float* sigma = reinterpret_cast<float*>(ws + L.sigma);
  int32_t* sel = reinterpret_cast<int32_t*>(ws + L.sel);
  int32_t* selcnt = reinterpret_cast<int32_t*>(ws + L.selcnt);
  int64_t* blkkeys = reinterpret_cast<int64_t*>(ws + L.blkkeys);
  const dim3 rows256((d.N + 255) / 256, d.H);
  const bool response = d.mode == SPARSEPR_RESPONSE_COUPLED;

  if (response || dbg_coords || dbg_dom || dbg_domval) {
    // g1 -> valsA, v -> valsB (reinterpreted) before the sort reuses them
    int32_t* g1 = valsA;
    float* v = reinterpret_cast<float*>(valsB);
    hipError_t e;
    if (d.bf16) {
      uint16_t* chl = reinterpret_cast<uint16_t*>(ws + L.chl);
      unsigned long long* best = reinterpret_cast<unsigned long long*>(ws + L.best);
      e = launch_split_hilo(kbar, (size_t)d.H * d.G, d.D, chl, st);
      if (e == hipSuccess)
        e = launch_rowvec_mfma(d, 1, Q, chl, nullptr, scale, group_off, best, dbg_coords, st);
      if (e == hipSuccess) e = launch_best_to_label(d, best, true, g1, v, st);
    } else {
      e = launch_coords_valu(d, Q, kbar, scale, group_off, g1, v, dbg_coords, st);
    }
    if (e != hipSuccess) return e;
    k_make_qkeys<<<rows256, 256, 0, st>>>(g1, v, d.N, keysA, dbg_dom, dbg_domval);
    SPR_CHECK_LAUNCH();
  }
  if (response) {
    // LSD radix sort: 4 passes over the value key (8 bits each), then the group bits.
    const int npass = 4 + (d.gbits > 0 ? 1 : 0);
    uint64_t* kin = keysA;
    uint64_t* kout = keysB;
    const int32_t* vin = nullptr;
    int32_t* vbuf[2] = {valsA, valsB};
    for (int ps = 0; ps < npass; ++ps) {
      const bool last = ps == npass - 1;
      const int shift = ps < 4 ? 8 * ps : 32;
      const int bits = ps < 4 ? 8 : d.gbits;
      int32_t* vout = last ? query_perm : vbuf[ps & 1];
      hipError_t e = launch_sort_pass_u64(d, kin, last ? nullptr : kout, shift, bits, vin, vout,
                                          counts, totals, starts, st);
      if (e != hipSuccess) return e;
      vin = vout;
      uint64_t* tk = kin;
      kin = kout;
      kout = tk;
    }
  } else {
    const size_t stride = d.mode == SPARSEPR_SEMANTIC ? (size_t)d.N : 0;
    k_copy_perm<<<rows256, 256, 0, st>>>(rand_query_perm, stride, d.N, query_perm);
    SPR_CHECK_LAUNCH();
  }
  const dim3 blocks(d.nb, d.H);
  const dim3 sblocks((d.nb + kRsBlocks - 1) / kRsBlocks, d.H);
#define SPR_RS(B, DD)                                                                          \
  k_route_scores<B, DD><<<sblocks, 256, 0, st>>>(Q, query_perm, kbar, scale, group_off, d.N,    \
                                                  d.BQ, d.nb, d.G, sigma, dbg_sigma)
  if (d.bf16) {
    if (d.D == 128) SPR_RS(true, 128); else SPR_RS(true, 64);
  } else {
    if (d.D == 128) SPR_RS(false, 128); else SPR_RS(false, 64);
  }
#undef SPR_RS
  SPR_CHECK_LAUNCH();
  k_block_select<<<blocks, 256, 0, st>>>(sigma, group_off, d.G, d.kappa, sel, selcnt, blkkeys);
  SPR_CHECK_LAUNCH();
  k_csr_scan<<<d.H, 1024, 0, st>>>(selcnt, blkkeys, d.nb, d.N, d.BQ, d.m, block_ptr,
                                    executed_pairs);
  SPR_CHECK_LAUNCH();
  k_csr_copy<<<blocks, 256, 0, st>>>(sel, selcnt, block_ptr, d.G, block_groups);
  SPR_CHECK_LAUNCH();
  return hipSuccess;
}

}  // namespace spr
