// Attention kernels: block-sparse over routed key groups, dense, and the
// split-key pass for the exact probe rows (arxivdaily 2608.18484, English
// abstract: attention only between selected groups; exact attention on a
// small set of query rows).
//
// bf16 path (gfx950 MFMA, v_mfma_f32_32x32x16_bf16). One workgroup owns one
// query block of BQ rows; each wavefront owns 32 query rows. Keys stream in
// tiles of KT through double-buffered LDS: 32 in the sparse and probe modes,
// where the smaller buffers let three workgroups share a CU, and 64 in dense
// mode, where the longer tile between barriers pays more. The product is
// formed transposed, S^T = K Q^T, so each lane holds the logits of ONE query
// (lane % 32) for 16 keys of each 32-key part of the tile: the online-softmax
// statistics are per-lane scalars, and the probabilities are already in the
// B-operand layout of O^T = V^T P^T. V stays row-major in LDS (rows padded)
// and is read transposed with ds_read_b64_tr_b16. The key list of a block is the
// concatenation of its routed groups' ranges in the group-contiguous Kp/Vp;
// tiles run across group boundaries, so only the block's last tile is ragged.
// Given the caller's work-queue counters, the sparse and dense launches are
// persistent grids that take query blocks from per-XCD queues (take_item).
#include <atomic>

#include "common.hpp"
#include "internal.hpp"

namespace spr {

// Routed groups that are adjacent in the group-contiguous key order are merged
// into one range; with at most 1024 groups there are at most 512 ranges.
constexpr int kMaxRanges = 512;
constexpr int kMaxGroups = 1024;

// LDS tiles hold 64 key rows with padded pitches: K rows at 2D+16 bytes (MFMA
// A-operand reads of 16 consecutive rows hit distinct banks), V rows at 2D+64
// bytes (the transposing ds_read_b64_tr_b16 reads 4 rows x 64 bytes per 32
// lanes, and the pitch puts those rows on disjoint banks). Both keep every
// LDS read address affine in the loop indices.
// LDS geometry of one KT-key tile. A buffer is rounded up to whole 1 KB
// loads; load lanes past the tile's data re-read chunk 0 of the tile's first
// row into that padding.
template <int D, int KT>
struct TileGeom {
  static_assert(KT == 32 || KT == 64, "tiles of 32 or 64 keys");
  static constexpr int ROWB = 2 * D;
  static constexpr int KP = ROWB + 16;
  static constexpr int VP = ROWB + 64;
  static constexpr int KCH = KP / 16;          // 16-byte chunks per padded K row
  static constexpr int VCH = VP / 16;
  static constexpr int KBYTES = (KT * KP + 1023) / 1024 * 1024;
  static constexpr int VBYTES = (KT * VP + 1023) / 1024 * 1024;
  static constexpr int KINS = KBYTES / 1024;   // 1 KB direct loads per tile
  static constexpr int VINS = VBYTES / 1024;
};

template <int MODE>
constexpr int tile_keys() { return MODE == ATTN_DENSE ? 64 : 32; }

// Decoded work item of one workgroup.
struct Item {
  int h, b, sp;
};

template <int MODE>
__device__ __forceinline__ Item decode_item(const AttnArgs& a, int nqb) {
  Item it;
  if (MODE != ATTN_PROBE && a.xcd_chunk > 0) {
    // dispatch w runs on XCD w % 8; XCD x takes blocks [x c, x c + c) of every
    // head, heads in order, so all XCDs stream the same head's keys together
    const int c = a.xcd_chunk;
    const int x = blockIdx.x & 7, i = blockIdx.x >> 3;
    it.h = i / c;
    it.b = x * c + i % c;
    it.sp = 0;
    if (it.b >= nqb) it.h = a.H;  // padding dispatch: no work
    return it;
  }
  const int total = (MODE == ATTN_PROBE ? nqb * a.nsplit : nqb) * a.H;
  const int L = xcd_remap(blockIdx.x, total);
  if (MODE == ATTN_PROBE) {
    const int per = nqb * a.nsplit;
    it.h = L / per;
    const int r = L % per;
    it.b = r / a.nsplit;
    it.sp = r % a.nsplit;
  } else {
    it.h = L / nqb;
    it.b = L % nqb;
    it.sp = 0;
  }
  return it;
}

// Work queues of the persistent grid: one counter per XCD, kQueueStride ints
// apart (one per 128-byte line), over the same per-XCD slices as the static
// mapping above: queue x holds blocks [x c, x c + c) of every head, heads in
// order. A workgroup takes from its own XCD's queue while it lasts, then from
// the others, so XCDs that run faster take over the last blocks of the
// slower ones. Counters only grow (an index at or past lim means empty; a
// workgroup that finds every queue empty has added at most 8 in all).
// Returns x * lim + index, or -1 once every queue is empty.
__device__ __forceinline__ int take_item(int* ctr, int lim) {
  const int x = blockIdx.x & 7;
  int code = -1;
  for (int y = 0; y < 8 && code < 0; ++y) {
    const int z = (x + y) & 7;
    const int i = atomicAdd(&ctr[z * kQueueStride], 1);
    if (i < lim) code = z * lim + i;
  }
  return code;
}

__global__ void k_clear_queues(int* ctr) {
  if (threadIdx.x < 8) ctr[threadIdx.x * kQueueStride] = 0;
}

// Whether query block b (positions [b B_q, b B_q + B_q)) holds a probe
// position: the caller's first position at or after the block start, or for
// p_i = floor((2i + 1) N / (2m)) the first such probe i0 = ceil((2m lo - N) / (2N)).
__device__ __forceinline__ bool block_has_probe(const int32_t* ppos, int b, int N, int m, int BQ) {
  if (m <= 0) return false;
  const int64_t lo = (int64_t)b * BQ;
  const int64_t hi = lo + BQ < N ? lo + BQ : N;
  if (ppos != nullptr) {
    const int i = probe_lower_bound(ppos, (int)lo, N, m);
    return i < m && clamp_idx(ppos[i], N) < hi;
  }
  const int64_t num = 2LL * m * lo - N;
  const int64_t i0 = num <= 0 ? 0 : (num + 2LL * N - 1) / (2LL * N);
  if (i0 >= m) return false;
  return ((2 * i0 + 1) * (int64_t)N) / (2LL * m) < hi;
}

// Token of query row qi of the work item; sets *pos to the output row.
template <int MODE, int BQ>
__device__ __forceinline__ int query_token(const AttnArgs& a, const Item& it, int qi, int* pos,
                                           bool* valid) {
  if (MODE == ATTN_PROBE) {
    const int pi = it.b * BQ + qi;
    *valid = pi < a.m;
    *pos = pi;
    if (!*valid) return 0;
    const int p = probe_position(a.ppos, pi, a.N, a.m);
    return clamp_idx(a.query_perm[(size_t)it.h * a.N + p], a.N);
  }
  const int p = it.b * BQ + qi;
  *pos = p;
  *valid = p < a.N;
  if (!*valid) return 0;
  if (MODE == ATTN_SPARSE) return clamp_idx(a.query_perm[(size_t)it.h * a.N + p], a.N);
  return p;
}

// Fills r_start / r_cum (exclusive prefix, r_cum[ng] = total) in LDS and
// returns the number of ranges. Contains __syncthreads().
template <int MODE, int NT>
__device__ __forceinline__ int build_ranges(const AttnArgs& a, const Item& it, int* r_start,
                                            int* r_cum, int* tmp) {
  const int t = threadIdx.x;
  if (MODE != ATTN_SPARSE) {
    if (t == 0) {
      int lo = 0, hi = a.N;
      if (MODE == ATTN_PROBE) {
        lo = it.sp * a.split_len;
        hi = min(a.N, lo + a.split_len);
      }
      r_start[0] = lo;
      r_cum[0] = 0;
      r_cum[1] = hi - lo;
    }
    __syncthreads();
    return 1;
  }
  const int32_t* bp = a.block_ptr + (size_t)it.h * (a.nb + 1);
  const int p0 = bp[it.b];
  int ng = bp[it.b + 1] - p0;
  ng = ng < 0 ? 0 : (ng > kMaxGroups ? kMaxGroups : ng);
  const int32_t* grp = a.block_groups + (size_t)it.h * a.nb * a.G + p0;
  const int32_t* off = a.group_off + (size_t)it.h * (a.G + 1);
  int carry_len = 0, carry_rng = 0;
  for (int base = 0; base < ng; base += NT) {
    const int i = base + t;
    int len = 0, st = 0, fresh = 0;
    if (i < ng) {
      const int g = clamp_idx(grp[i], a.G);
      st = off[g];
      len = max(0, off[g + 1] - st);
      // a range starts unless this group begins where the previous one ended
      fresh = (i == 0) || (off[clamp_idx(grp[i - 1], a.G) + 1] != st);
    }
    int tot_len, tot_rng;
    const int ex_len = block_exclusive_scan<NT>(len, tmp, &tot_len);
    const int ex_rng = block_exclusive_scan<NT>(fresh, tmp, &tot_rng);
    const int ri = carry_rng + ex_rng;
    if (i < ng && fresh && ri < kMaxRanges) {
      r_start[ri] = st;
      r_cum[ri] = carry_len + ex_len;
    }
    carry_len += tot_len;
    carry_rng += tot_rng;
  }
  const int nr = carry_rng < kMaxRanges ? carry_rng : kMaxRanges;
  if (t == 0) r_cum[nr] = carry_len;
  __syncthreads();
  return nr;
}

// Row of Kp/Vp at key position p of the block's list (cursor advances
// monotonically across tiles).
__device__ __forceinline__ int key_row(int p, int total, int ng, const int* r_start,
                                       const int* r_cum, int& cur) {
  if (p >= total) return r_start[0];
  while (cur + 1 < ng && r_cum[cur + 1] <= p) ++cur;
  return r_start[cur] + (p - r_cum[cur]);
}

// One KT-key tile of the flash loop: S^T = K Q^T, online softmax, O^T += V^T P^T.
// Ktile / Vtile point at distinct __shared__ buffers, so the compiler can see
// that these reads do not alias the direct loads filling the other buffer.
// RSUM (sparse and probe modes): the row sum adds the bf16-rounded
// probabilities that P V uses, two per v_dot2_f32_bf16, so each output row is
// a convex combination of its V rows with exactly those weights; the
// log-sum-exp then differs from the exact one by at most log(1 + 2^-9). The
// dense mode sums the fp32 probabilities.
template <int D, int KT, bool RSUM>
__device__ __forceinline__ void attn_tile(const char* __restrict__ kb, const char* __restrict__ vb,
                                          const bf16x8* qreg, f32x16* acc_o, float& m_run,
                                          float& l_run, float c, int kbase, int total, int hl) {
  using TG = TileGeom<D, KT>;
  constexpr int NKT = KT / 32;   // 32-key parts of the tile
  constexpr int NDT = D / 32;
  constexpr int NKK = D / 16;
  f32x16 s[NKT];
#pragma unroll
  for (int kt = 0; kt < NKT; ++kt) {
#pragma unroll
    for (int r = 0; r < 16; ++r) s[kt][r] = 0.f;
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) {
      const bf16x8 kop = *reinterpret_cast<const bf16x8*>(kb + 32 * kt * TG::KP + 32 * kk);
      s[kt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kop, qreg[kk], s[kt], 0, 0, 0);
    }
  }
  // online softmax in log2 units; the max is only re-based when it grows by > 8
  if (kbase + KT > total) {
#pragma unroll
    for (int kt = 0; kt < NKT; ++kt)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int kp = kbase + 32 * kt + 8 * (r >> 2) + 4 * hl + (r & 3);
        if (kp >= total) s[kt][r] = -__builtin_inff();
      }
  }
  float mx = -__builtin_inff();
#pragma unroll
  for (int kt = 0; kt < NKT; ++kt)
#pragma unroll
    for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kt][r]);
  {
    // lanes l and l ^ 32 hold the two halves of one query row (the helper
    // reads both swap results through integer casts: a bit_cast of a vector
    // element straight from the builtin's result reads element 0 twice)
    float lo, hi;
    lane_half_swap(mx, mx, lo, hi);
    mx = (lo > hi ? lo : hi) * c;
  }
  const float m_new = fmaxf(m_run, mx);
  const bool need = m_new > m_run + 8.0f;
  if (__any(need)) {
    const float alpha = need ? __builtin_amdgcn_exp2f(m_run - m_new) : 1.0f;
    l_run *= alpha;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc_o[dt][r] *= alpha;
    if (need) m_run = m_new;
  }
  const float neg_m = -m_run;
  bf16x8 pk[NKT][2];
#pragma unroll
  for (int kt = 0; kt < NKT; ++kt)
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
      float pv[8];
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        pv[q] = __builtin_amdgcn_exp2f(fmaf(s[kt][8 * hf + q], c, neg_m));
        if (!RSUM) l_run += pv[q];
      }
#pragma unroll
      for (int q = 0; q < 8; q += 2) {
        const f32x2 f = {pv[q], pv[q + 1]};
        const bf16x2 bb = __builtin_convertvector(f, bf16x2);
        pk[kt][hf][q] = bb[0];
        pk[kt][hf][q + 1] = bb[1];
        if (RSUM) {
          const bf16x2 one = {(__bf16)1.0f, (__bf16)1.0f};
          l_run = __builtin_amdgcn_fdot2_f32_bf16(bb, one, l_run, false);
        }
      }
    }
  // V^T operand via transposing LDS reads
#pragma unroll
  for (int kt = 0; kt < NKT; ++kt)
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
      const int chunk = 32 * kt + 16 * hf;
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) {
        const char* p1 = vb + chunk * TG::VP + 64 * dt;
        const char* p2 = p1 + 8 * TG::VP;
        const s16x4 v1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) s16x4*)(p1));
        const s16x4 v2 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) s16x4*)(p2));
        const s16x8 vv = __builtin_shufflevector(v1, v2, 0, 1, 2, 3, 4, 5, 6, 7);
        acc_o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, vv),
                                                            pk[kt][hf], acc_o[dt], 0, 0, 0);
      }
    }
}

template <int D, int BQ, int MODE>
__global__ __launch_bounds__(BQ * 2)
__attribute__((amdgpu_waves_per_eu(BQ == 128 ? (tile_keys<MODE>() == 32 ? 3 : 2) : 1,
                                   BQ == 128 ? (tile_keys<MODE>() == 32 ? 3 : 2) : 1)))
void k_attn_mfma(AttnArgs args) {
  constexpr int KT = tile_keys<MODE>();
  using TG = TileGeom<D, KT>;
  constexpr int NT = BQ * 2;
  constexpr int NW = BQ / 32;
  constexpr int ROWB = TG::ROWB;
  constexpr int CPR = ROWB / 16;             // data chunks per row
  constexpr int NDT = D / 32;                // 32-wide output d tiles
  constexpr int NKK = D / 16;                // k-steps of the QK^T product
  // one stage = a tile's K rows (KBYTES) followed by its V rows (VBYTES);
  // two stages in distinct arrays, so the compiler sees that the compute reads
  // of one never alias the direct loads filling the other
  constexpr int NLOAD = TG::KINS + TG::VINS;   // 1 KB direct loads per tile
  constexpr int SLOTS = (NLOAD + NW - 1) / NW; // the same number for every wave
  constexpr int CHT = 16;                      // tiles per row-table chunk
  constexpr bool kTable = MODE == ATTN_SPARSE; // dense and probe keys are one contiguous range
  __shared__ __attribute__((aligned(1024))) char lds_s0[NLOAD * 1024];
  __shared__ __attribute__((aligned(1024))) char lds_s1[NLOAD * 1024];
  __shared__ int ridx[2][kTable ? CHT * KT : 1];
  __shared__ int r_start[kMaxRanges + 1];
  __shared__ int r_cum[kMaxRanges + 2];
  // scan scratch of the range builder; during the tile loop it absorbs the
  // loads of the slots past NLOAD (never read)
  __shared__ __attribute__((aligned(1024))) int tmp[NT > 256 ? NT : 256];
  char* const lds_pad = reinterpret_cast<char*>(tmp);
  char* const lds_k0 = lds_s0;
  char* const lds_v0 = lds_s0 + TG::KBYTES;
  char* const lds_k1 = lds_s1;
  char* const lds_v1 = lds_s1 + TG::KBYTES;

  __shared__ int s_item;
  // One item (query block, or probe split) per trip. With work queues the grid
  // is persistent and loops until they are empty; without, each workgroup runs
  // the item its id names.
  const bool queued = MODE != ATTN_PROBE && args.qctr != nullptr;
  for (int trip = 0;; ++trip) {
  // The arguments are re-read on each trip from the kernel-argument segment
  // (the struct is the kernel's only argument, at offset 0), through an offset
  // the compiler cannot prove zero, so that no value derived from them is held
  // from one item to the next (it would not fit the register budget).
  int kz = 0;
  asm volatile("" : "+s"(kz));
  const AttnArgs a = *(const AttnArgs*)((const char*)__builtin_amdgcn_kernarg_segment_ptr() + kz);
  const int nqb = MODE == ATTN_PROBE ? (a.m + BQ - 1) / BQ : a.nb;
  Item it;
  if (queued) {
    __syncthreads();   // every wave is done with the previous item's LDS and s_item
    if (threadIdx.x == 0) s_item = take_item(a.qctr, a.xcd_chunk * a.H);
    __syncthreads();
    const int code = s_item;
    if (code < 0) break;
    const int lim = a.xcd_chunk * a.H, x = code / lim, i = code - x * lim;
    it.h = i / a.xcd_chunk;
    it.b = x * a.xcd_chunk + i % a.xcd_chunk;
    it.sp = 0;
    if (it.b >= nqb) continue;   // padding slot of the last slice
  } else {
    if (trip > 0) break;
    it = decode_item<MODE>(a, nqb);
    if (it.h >= a.H) break;
  }
  if (MODE == ATTN_SPARSE && a.subset != 0 && block_has_probe(a.ppos, it.b, a.N, a.m, BQ) != (a.subset == 1))
    continue;
  const int t = threadIdx.x;
  const int lane = t & 63;
  const int w = __builtin_amdgcn_readfirstlane(t >> 6);   // uniform across the wave
  const int hl = lane >> 5;       // which half of the wave
  const int ql = lane & 31;       // query within the wave
  const size_t hoff = (size_t)it.h * a.N * D;
  const uint16_t* Qh = static_cast<const uint16_t*>(a.Q) + hoff;
  const char* Kh = static_cast<const char*>(a.K) + hoff * 2;
  const char* Vh = static_cast<const char*>(a.V) + hoff * 2;

  const int ng = build_ranges<MODE, NT>(a, it, r_start, r_cum, tmp);
  const int total = r_cum[ng];

  // Q operand: B of S^T = K Q^T; lane holds query ql, d = 16 kk + 8 hl + 0..7
  int qpos;
  bool qvalid;
  const int qtok = query_token<MODE, BQ>(a, it, w * 32 + ql, &qpos, &qvalid);
  bf16x8 qreg[NKK];
#pragma unroll
  for (int kk = 0; kk < NKK; ++kk)
    qreg[kk] = *reinterpret_cast<const bf16x8*>(Qh + (size_t)qtok * D + 16 * kk + 8 * hl);

  // The online softmax scales each tile's largest raw logit by c, which is the
  // largest scaled logit only when c >= 0. For a negative scale the Q operand
  // is negated (an exact sign flip of every bf16 element), so that the kernel
  // runs with |c| on the same scaled logits.
  float c = a.scale[it.h] * kLog2e;
  if (c < 0.f) {
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) {
      u32x4 bits = __builtin_bit_cast(u32x4, qreg[kk]);
      bits ^= 0x80008000u;
      qreg[kk] = __builtin_bit_cast(bf16x8, bits);
    }
    c = -c;
  }
  // Masked keys carry a raw logit of -inf, which a zero scale would turn into
  // NaN. The smallest normal scale gives the same result as zero: every scaled
  // logit is then below 2^-100 in magnitude, so each exponential rounds to 1.
  if (c == 0.f) c = __FLT_MIN__;
  float m_run = -__builtin_inff();   // running max of the scaled logits (log2 units)
  float l_run = 0.f;
  f32x16 acc_o[NDT];
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc_o[dt][r] = 0.f;

  const int ntiles = (total + KT - 1) / KT;
  int cursor = 0;
  // Sparse mode: the row table holds the byte offset in Kp/Vp of each key
  // position, CHT tiles per chunk, two chunks; all threads fill a chunk at
  // once (each thread's positions increase, so its range cursor only moves
  // forward). Dense and probe modes read one contiguous key range from row0.
  const int row0 = r_start[0];
  auto fill_chunk = [&](int chunk) {
    int* dst = ridx[chunk & 1];
#pragma unroll
    for (int e0 = 0; e0 < CHT * KT; e0 += NT) {
      const int e = e0 + t;
      if (e < CHT * KT) {
        const int r = key_row(chunk * CHT * KT + e, total, ng, r_start, r_cum, cursor);
        dst[e] = (int)((uint32_t)r * ROWB);
      }
    }
  };
  // A tile is NLOAD direct global->LDS loads of 1 KB (K rows, then V rows),
  // dealt out SLOTS per wave so that every wave runs the same branch-free
  // sequence; a slot past NLOAD re-reads chunk 0 of the tile's first row into
  // a buffer nobody reads. Lane i of load u moves chunk 64 (u mod tile part)
  // + i; its word packs 4x its row in the tile (low 16 bits) and the byte
  // offset of its 16-byte chunk in the row (high 16 bits; chunks past a row's
  // data re-read chunk 0). Keys past the list's end re-read a valid row.
  int sw[SLOTS];
  const char* sbase[SLOTS];
  int sdst[SLOTS];
#pragma unroll
  for (int j = 0; j < SLOTS; ++j) {
    const int u = w * SLOTS + j;
    const bool isk = u < TG::KINS;
    const int ul = isk ? u : u - TG::KINS;
    const int ch = isk ? TG::KCH : TG::VCH;
    const int q0 = 64 * ul + lane;
    const int q = (u < NLOAD && q0 < KT * ch) ? q0 : 0;
    const int r = q / ch, cc = q - r * ch;
    sw[j] = (4 * r) | (((cc < CPR ? cc : 0) * 16) << 16);
    sbase[j] = isk ? Kh : Vh;
    sdst[j] = u < NLOAD ? u * 1024 : -1;
  }
  auto issue_slots = [&](int tile, char* stage) {
    uint32_t ro[SLOTS];
    if constexpr (kTable) {
      const char* tab = reinterpret_cast<const char*>(ridx[(tile / CHT) & 1]) + (tile % CHT) * KT * 4;
#pragma unroll
      for (int j = 0; j < SLOTS; ++j)
        ro[j] = *reinterpret_cast<const uint32_t*>(tab + (sw[j] & 0xffff)) + ((uint32_t)sw[j] >> 16);
    } else {
#pragma unroll
      for (int j = 0; j < SLOTS; ++j) {
        const int pk = min(tile * KT + ((sw[j] & 0xffff) >> 2), total - 1);
        ro[j] = (uint32_t)(row0 + pk) * (uint32_t)ROWB + ((uint32_t)sw[j] >> 16);
      }
    }
#pragma unroll
    for (int j = 0; j < SLOTS; ++j) {
      char* dst = sdst[j] >= 0 ? stage + sdst[j] : lds_pad;
      __builtin_amdgcn_global_load_lds((const void*)(sbase[j] + ro[j]),
                                       (__attribute__((address_space(3))) void*)dst, 16, 0, 0);
    }
  };
#define NEXT_ROWS(TILE)                                                                    \
  do {                                                                                     \
    if constexpr (kTable) {                                                                \
      if ((TILE) % CHT == 0) fill_chunk((TILE) / CHT + 1);                                 \
    }                                                                                      \
  } while (0)

  if constexpr (kTable) fill_chunk(0);
  __syncthreads();
  if (ntiles > 0) issue_slots(0, lds_s0);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();

  const int grp = lane >> 4, gl = lane & 15;
  // per-lane LDS byte offsets (the tile loop adds only compile-time constants)
  const int koff = ql * TG::KP + hl * 16;
  const int voff = (4 * (grp >> 1) + (gl >> 2)) * TG::VP + (16 * (grp & 1) + 4 * (gl & 3)) * 2;
  // two tiles per trip: even tiles live in stage 0, odd tiles in stage 1
  for (int tile = 0; tile < ntiles; tile += 2) {
    if (tile + 1 < ntiles) issue_slots(tile + 1, lds_s1);
    NEXT_ROWS(tile);
    attn_tile<D, KT, MODE != ATTN_DENSE>(lds_k0 + koff, lds_v0 + voff, qreg, acc_o, m_run, l_run, c, tile * KT, total, hl);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (tile + 1 >= ntiles) break;
    if (tile + 2 < ntiles) issue_slots(tile + 2, lds_s0);
    NEXT_ROWS(tile + 1);
    attn_tile<D, KT, MODE != ATTN_DENSE>(lds_k1 + koff, lds_v1 + voff, qreg, acc_o, m_run, l_run, c, (tile + 1) * KT, total, hl);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  }

#undef NEXT_ROWS
  // ---- epilogue
  const float l_tot = l_run + __shfl_xor(l_run, 32);
  const float inv = l_tot > 0.f ? 1.0f / l_tot : 0.f;
  const float lse = l_tot > 0.f ? (m_run + log2f(l_tot)) * kLn2 : -__builtin_inff();
  if (qvalid) {
  if (MODE == ATTN_PROBE) {
    float* op = a.opart + (((size_t)it.h * a.nsplit + it.sp) * a.m + qpos) * D;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int d0 = 32 * dt + 8 * j + 4 * hl;
        const f32x4 v = {acc_o[dt][4 * j] * inv, acc_o[dt][4 * j + 1] * inv,
                         acc_o[dt][4 * j + 2] * inv, acc_o[dt][4 * j + 3] * inv};
        *reinterpret_cast<f32x4*>(op + d0) = v;
      }
    if (hl == 0) a.lsepart[((size_t)it.h * a.nsplit + it.sp) * a.m + qpos] = lse;
  } else {
    // bf16 rows: S_out at the query position (sparse), O at the token (dense)
    uint16_t* out = static_cast<uint16_t*>(a.out) + hoff + (size_t)qpos * D;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int d0 = 32 * dt + 8 * j + 4 * hl;
        const f32x2 f0 = {acc_o[dt][4 * j] * inv, acc_o[dt][4 * j + 1] * inv};
        const f32x2 f1 = {acc_o[dt][4 * j + 2] * inv, acc_o[dt][4 * j + 3] * inv};
        const bf16x2 b0 = __builtin_convertvector(f0, bf16x2);
        const bf16x2 b1 = __builtin_convertvector(f1, bf16x2);
        const bf16x4 bv = {b0[0], b0[1], b1[0], b1[1]};
        *reinterpret_cast<bf16x4*>(out + d0) = bv;
      }
    // a probe position's row also goes out unrounded, for the fit
    const int pi = MODE == ATTN_SPARSE && a.sprobe != nullptr ? probe_index(a.ppos, qpos, a.N, a.m) : -1;
    if (pi >= 0) {
      float* sp = a.sprobe + ((size_t)it.h * a.m + pi) * D;
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int d0 = 32 * dt + 8 * j + 4 * hl;
          const f32x4 v = {acc_o[dt][4 * j] * inv, acc_o[dt][4 * j + 1] * inv,
                           acc_o[dt][4 * j + 2] * inv, acc_o[dt][4 * j + 3] * inv};
          *reinterpret_cast<f32x4*>(sp + d0) = v;
        }
    }
  }
  if (MODE != ATTN_PROBE) {
    if (hl == 0 && a.lse != nullptr) a.lse[(size_t)it.h * a.N + qpos] = lse;
  }
  }  // qvalid
  }  // trips
}

// fp32 path: 64 query rows per workgroup, 4 lanes per query (dims 4u + lane%4),
// key tiles of 32 rows in LDS; online softmax per tile.
template <int D, int MODE>
__global__ __launch_bounds__(256) void k_attn_valu(AttnArgs a, int BQ) {
  constexpr int NT = 256;
  constexpr int KT = 32;
  constexpr int DU = D / 4;
  __shared__ float kt_s[KT][D];
  __shared__ float vt_s[KT][D];
  __shared__ int r_start[kMaxRanges + 1];
  __shared__ int r_cum[kMaxRanges + 2];
  __shared__ int tmp[NT];
  const int sub_per_block = BQ / 64;
  const int nqb = MODE == ATTN_PROBE ? (a.m + BQ - 1) / BQ : a.nb;
  const int total_items = (MODE == ATTN_PROBE ? nqb * a.nsplit : nqb) * a.H * sub_per_block;
  const int Lw = xcd_remap(blockIdx.x, total_items);
  const int sub = Lw % sub_per_block;
  const int L = Lw / sub_per_block;
  Item it;
  if (MODE == ATTN_PROBE) {
    const int per = nqb * a.nsplit;
    it.h = L / per;
    it.b = (L % per) / a.nsplit;
    it.sp = (L % per) % a.nsplit;
  } else {
    it.h = L / nqb;
    it.b = L % nqb;
    it.sp = 0;
  }
  if (MODE == ATTN_SPARSE && a.subset != 0 && block_has_probe(a.ppos, it.b, a.N, a.m, BQ) != (a.subset == 1))
    return;
  const int t = threadIdx.x;
  const int qq = t & 3;
  const int qi = sub * 64 + (t >> 2);
  const size_t hoff = (size_t)it.h * a.N * D;
  const float* Qh = static_cast<const float*>(a.Q) + hoff;
  const float* Kh = static_cast<const float*>(a.K) + hoff;
  const float* Vh = static_cast<const float*>(a.V) + hoff;

  const int ng = build_ranges<MODE, NT>(a, it, r_start, r_cum, tmp);
  const int total = r_cum[ng];
  int qpos;
  bool qvalid;
  int qtok;
  if (MODE == ATTN_PROBE) {
    const int pi = it.b * BQ + qi;
    qvalid = pi < a.m;
    qpos = pi;
    qtok = qvalid ? clamp_idx(a.query_perm[(size_t)it.h * a.N +
                                           probe_position(a.ppos, pi, a.N, a.m)], a.N) : 0;
  } else {
    qpos = it.b * BQ + qi;
    qvalid = qpos < a.N;
    qtok = !qvalid ? 0 : (MODE == ATTN_SPARSE ? clamp_idx(a.query_perm[(size_t)it.h * a.N + qpos], a.N) : qpos);
  }
  float q[DU], o[DU];
#pragma unroll
  for (int u = 0; u < DU; ++u) {
    q[u] = Qh[(size_t)qtok * D + 4 * u + qq];
    o[u] = 0.f;
  }
  const float c = a.scale[it.h] * kLog2e;
  float m_run = -__builtin_inff(), l_run = 0.f;
  int cursor = 0;
  const int ntiles = (total + KT - 1) / KT;
  for (int tile = 0; tile < ntiles; ++tile) {
    __syncthreads();
    for (int f = t; f < KT * DU; f += NT) {
      const int r = f / DU, c4 = f % DU;
      // rows are visited in increasing order by each thread, so the cursor is monotone
      const int row = key_row(tile * KT + r, total, ng, r_start, r_cum, cursor);
      *reinterpret_cast<f32x4*>(&kt_s[r][4 * c4]) = *reinterpret_cast<const f32x4*>(Kh + (size_t)row * D + 4 * c4);
      *reinterpret_cast<f32x4*>(&vt_s[r][4 * c4]) = *reinterpret_cast<const f32x4*>(Vh + (size_t)row * D + 4 * c4);
    }
    __syncthreads();
    float x[KT];
    float mx = -__builtin_inff();
#pragma unroll
    for (int j = 0; j < KT; ++j) {
      float part = 0.f;
#pragma unroll
      for (int u = 0; u < DU; ++u) part = fmaf(q[u], kt_s[j][4 * u + qq], part);
      part += __shfl_xor(part, 1);
      part += __shfl_xor(part, 2);
      x[j] = (tile * KT + j < total) ? part * c : -__builtin_inff();
      mx = fmaxf(mx, x[j]);
    }
    const float m_new = fmaxf(m_run, mx);
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
    l_run *= alpha;
#pragma unroll
    for (int u = 0; u < DU; ++u) o[u] *= alpha;
    m_run = m_new;
#pragma unroll
    for (int j = 0; j < KT; ++j) {
      const float p = __builtin_amdgcn_exp2f(x[j] - m_run);
      l_run += p;
#pragma unroll
      for (int u = 0; u < DU; ++u) o[u] = fmaf(p, vt_s[j][4 * u + qq], o[u]);
    }
  }
  const float inv = l_run > 0.f ? 1.0f / l_run : 0.f;
  const float lse = l_run > 0.f ? (m_run + log2f(l_run)) * kLn2 : -__builtin_inff();
  if (!qvalid) return;
  if (MODE == ATTN_PROBE) {
    float* op = a.opart + (((size_t)it.h * a.nsplit + it.sp) * a.m + qpos) * D;
#pragma unroll
    for (int u = 0; u < DU; ++u) op[4 * u + qq] = o[u] * inv;
    if (qq == 0) a.lsepart[((size_t)it.h * a.nsplit + it.sp) * a.m + qpos] = lse;
  } else {
    float* out = static_cast<float*>(a.out) + hoff + (size_t)qpos * D;
#pragma unroll
    for (int u = 0; u < DU; ++u) out[4 * u + qq] = o[u] * inv;
    if (qq == 0 && a.lse != nullptr) a.lse[(size_t)it.h * a.N + qpos] = lse;
    // a probe position's row also goes to the fit's copy
    const int pi = MODE == ATTN_SPARSE && a.sprobe != nullptr ? probe_index(a.ppos, qpos, a.N, a.m) : -1;
    if (pi >= 0) {
      float* sp = a.sprobe + ((size_t)it.h * a.m + pi) * D;
#pragma unroll
      for (int u = 0; u < DU; ++u) sp[4 * u + qq] = o[u] * inv;
    }
  }
}

// O_probe = LSE-weighted merge of the split partials. grid (m, H), block D.
template <int D>
__global__ void k_probe_merge(const float* opart, const float* lsepart, int m, int nsplit,
                              float* O_probe) {
  const int i = blockIdx.x, h = blockIdx.y, e = threadIdx.x;
  float mx = -__builtin_inff();
  for (int s = 0; s < nsplit; ++s) mx = fmaxf(mx, lsepart[((size_t)h * nsplit + s) * m + i]);
  float wsum = 0.f, acc = 0.f;
  for (int s = 0; s < nsplit; ++s) {
    const float ls = lsepart[((size_t)h * nsplit + s) * m + i];
    const float wgt = ls == -__builtin_inff() ? 0.f : expf(ls - mx);
    wsum += wgt;
    acc += wgt * opart[(((size_t)h * nsplit + s) * m + i) * D + e];
  }
  O_probe[((size_t)h * m + i) * D + e] = wsum > 0.f ? acc / wsum : 0.f;
}

// Workgroups of k_attn_mfma<D, BQ, MODE> that the current device holds at once
// (0 if the runtime cannot say), looked up once per instantiation and device.
template <int D, int BQ, int MODE>
static int resident_workgroups() {
  static std::atomic<int> cache[16];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  if (dev < 16) {
    const int c = cache[dev].load(std::memory_order_relaxed);
    if (c > 0) return c;
  }
  int cus = 0, per = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      hipOccupancyMaxActiveBlocksPerMultiprocessor(&per, k_attn_mfma<D, BQ, MODE>, BQ * 2, 0) !=
          hipSuccess)
    return 0;
  const int n = cus * per;
  if (dev < 16 && n > 0) cache[dev].store(n, std::memory_order_relaxed);
  return n;
}

// Matrix-core launch. With work queues the grid is the resident workgroup
// count (at most one per item) and the queues are cleared first on the same
// stream; without, one workgroup per item.
template <int D, int BQ, int MODE>
static void launch_mfma(AttnArgs aa, int items, hipStream_t st) {
  int grid = items;
  if (aa.qctr != nullptr) {
    const int res = resident_workgroups<D, BQ, MODE>();
    if (res > 0) {
      k_clear_queues<<<1, 64, 0, st>>>(aa.qctr);
      grid = items < res ? items : res;
    } else {
      aa.qctr = nullptr;
    }
  }
  k_attn_mfma<D, BQ, MODE><<<grid, BQ * 2, 0, st>>>(aa);
}

hipError_t launch_attention(const Dims& d, AttnMode mode, const AttnArgs& a, hipStream_t st) {
  const int nqb = mode == ATTN_PROBE ? (d.m + d.BQ - 1) / d.BQ : (d.N + d.BQ - 1) / d.BQ;
  int items = (mode == ATTN_PROBE ? nqb * d.nsplit : nqb) * d.H;
  AttnArgs aa = a;
  aa.nb = mode == ATTN_PROBE ? a.nb : nqb;
  aa.xcd_chunk = 0;
  if (d.bf16) {
    if (mode != ATTN_PROBE) {
      // head-synchronous XCD mapping (padding items exit at once)
      aa.xcd_chunk = (nqb + 7) / 8;
      items = 8 * aa.xcd_chunk * d.H;
    } else {
      aa.qctr = nullptr;
    }
#define SPR_MFMA(DD, BB)                                                   \
  do {                                                                     \
    if (mode == ATTN_SPARSE) launch_mfma<DD, BB, ATTN_SPARSE>(aa, items, st); \
    else if (mode == ATTN_DENSE) launch_mfma<DD, BB, ATTN_DENSE>(aa, items, st); \
    else launch_mfma<DD, BB, ATTN_PROBE>(aa, items, st);                  \
  } while (0)
    if (d.D == 128) {
      if (d.BQ == 128) SPR_MFMA(128, 128); else SPR_MFMA(128, 64);
    } else {
      if (d.BQ == 128) SPR_MFMA(64, 128); else SPR_MFMA(64, 64);
    }
#undef SPR_MFMA
  } else {
    const int witems = items * (d.BQ / 64);
#define SPR_VALU(DD)                                                                        \
  do {                                                                                      \
    if (mode == ATTN_SPARSE) k_attn_valu<DD, ATTN_SPARSE><<<witems, 256, 0, st>>>(aa, d.BQ); \
    else if (mode == ATTN_DENSE) k_attn_valu<DD, ATTN_DENSE><<<witems, 256, 0, st>>>(aa, d.BQ); \
    else k_attn_valu<DD, ATTN_PROBE><<<witems, 256, 0, st>>>(aa, d.BQ);                     \
  } while (0)
    if (d.D == 128) SPR_VALU(128); else SPR_VALU(64);
#undef SPR_VALU
  }
  return hipGetLastError();
}

hipError_t launch_probe_merge(const Dims& d, const float* opart, const float* lsepart,
                              float* O_probe, hipStream_t st) {
  if (d.m == 0) return hipSuccess;
  if (d.D == 128)
    k_probe_merge<128><<<dim3(d.m, d.H), 128, 0, st>>>(opart, lsepart, d.m, d.nsplit, O_probe);
  else
    k_probe_merge<64><<<dim3(d.m, d.H), 64, 0, st>>>(opart, lsepart, d.m, d.nsplit, O_probe);
  return hipGetLastError();
}

}  // namespace spr
