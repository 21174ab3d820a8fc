// Support and mass diagnostics of routed query blocks (skillfed article,
// paragraphs on the two problems of block-sparse attention: queries sharing a
// block route may prefer different keys, and keeping most of the attention
// mass need not keep the output; arxivdaily 2608.18484, English abstract:
// partition choice affects the overlap of grouped queries' preferred supports).
//
// For each row q of a sampled block b (all N keys, p_qj = softmax_j(tau q.k_j)):
//   lse_q      = log sum_j exp(tau q.k_j)
//   mass_q     = sum of p_qj over the block's routed keys K(b)
//   theta_q    = largest logit t with sum_{x_qj >= t} p_qj >= mu
//   support_q  = #{j : x_qj >= theta_q}   (the fewest keys holding mass mu)
//   routed_q   = #{j in K(b) : x_qj >= theta_q}
// and per block the pooled support |union_q {j : x_qj >= theta_q}| and its part
// inside K(b). Logits are fp32 (exact bf16 or fp32 inputs, fp32 accumulation);
// sums over keys are accumulated in fp64.
#include "common.hpp"
#include "internal.hpp"

namespace spr {

constexpr int kSupRows = 16;  // query rows per workgroup of the logits kernel

// Key j's group is routed to the block: bit label_j of the block's group mask.
__device__ __forceinline__ bool routed(const uint32_t* sel, int g) {
  return (sel[g >> 5] >> (g & 31)) & 1u;
}

// The block's routed groups as a bit mask in LDS (G <= 1024 bits). Contains
// __syncthreads().
__device__ __forceinline__ void load_group_mask(const SupportArgs& a, int b, uint32_t* sel) {
  const int t = threadIdx.x;
  for (int i = t; i < 32; i += blockDim.x) sel[i] = 0u;
  __syncthreads();
  const int32_t* bp = a.block_ptr + (size_t)a.head * (a.nb + 1);
  const int32_t* grp = a.block_groups + (size_t)a.head * a.nb * a.G;
  const int p0 = bp[b];
  const int n = max(0, min(bp[b + 1] - p0, a.G));
  for (int i = t; i < n; i += blockDim.x) {
    const int g = clamp_idx(grp[p0 + i], a.G);
    atomicOr(&sel[g >> 5], 1u << (g & 31));
  }
  __syncthreads();
}

// Logits of kSupRows query rows against every key. grid (n_blocks *
// ceil(B_q / kSupRows)), block 256. xs[(i B_q + r) N + j] for sampled block i,
// row r of the block (rows past N are written as -inf).
template <bool BF16, int D>
__global__ __launch_bounds__(256) void k_support_logits(SupportArgs a) {
  using IO = Elt<BF16>;
  using T = typename IO::T;
  __shared__ float qs[kSupRows][D];
  const int per = (a.BQ + kSupRows - 1) / kSupRows;
  const int i = blockIdx.x / per, r0 = (blockIdx.x % per) * kSupRows;
  const int b = clamp_idx(a.blocks[i], a.nb);
  const int t = threadIdx.x;
  const T* Qh = static_cast<const T*>(a.Q) + (size_t)a.head * a.N * D;
  const T* Kh = static_cast<const T*>(a.K) + (size_t)a.head * a.N * D;
  const float tau = a.scale[a.head];
  for (int e = t; e < kSupRows * D; e += 256) {
    const int r = e / D, c = e % D;
    const int p = b * a.BQ + r0 + r;
    float v = 0.f;
    if (r0 + r < a.BQ && p < a.N) {
      const int q = clamp_idx(a.query_perm[(size_t)a.head * a.N + p], a.N);
      v = IO::ld(Qh, (size_t)q * D + c);
    }
    qs[r][c] = v;
  }
  __syncthreads();
  for (int j = t; j < a.N; j += 256) {
    float acc[kSupRows];
#pragma unroll
    for (int r = 0; r < kSupRows; ++r) acc[r] = 0.f;
    for (int c = 0; c < D; c += 8) {
      float k[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) k[u] = IO::ld(Kh, (size_t)j * D + c + u);
#pragma unroll
      for (int r = 0; r < kSupRows; ++r)
#pragma unroll
        for (int u = 0; u < 8; ++u) acc[r] = fmaf(qs[r][c + u], k[u], acc[r]);
    }
#pragma unroll
    for (int r = 0; r < kSupRows; ++r) {
      const int p = b * a.BQ + r0 + r;
      if (r0 + r < a.BQ)
        a.xs[((size_t)i * a.BQ + r0 + r) * a.N + j] = p < a.N ? tau * acc[r] : -__builtin_inff();
    }
  }
}

template <int NT>
__device__ __forceinline__ float block_max_f32(float v, float* tmp) {
  const int t = threadIdx.x;
  tmp[t] = v;
  __syncthreads();
  for (int off = NT / 2; off > 0; off >>= 1) {
    if (t < off) tmp[t] = fmaxf(tmp[t], tmp[t + off]);
    __syncthreads();
  }
  const float r = tmp[0];
  __syncthreads();
  return r;
}

template <int NT>
__device__ __forceinline__ float block_min_f32(float v, float* tmp) {
  return -block_max_f32<NT>(-v, tmp);
}

__device__ __forceinline__ float float_from_order(uint32_t u) {
  return __uint_as_float((u & 0x80000000u) ? (u & 0x7fffffffu) : ~u);
}

// Per row: lse, routed mass, support threshold and sizes. grid (n_blocks B_q),
// block 256.
__global__ __launch_bounds__(256) void k_support_row(SupportArgs a) {
  constexpr int NT = 256;
  __shared__ uint32_t sel[32];
  __shared__ float tf[NT];
  __shared__ double td[NT];
  const int row = blockIdx.x, i = row / a.BQ, r = row % a.BQ;
  const int b = clamp_idx(a.blocks[i], a.nb);
  const int p = b * a.BQ + r;
  const int t = threadIdx.x;
  if (p >= a.N) {
    if (t == 0) {
      a.lse[row] = -__builtin_inff();
      a.mass[row] = 0.f;
      a.support[row] = 0;
      a.support_routed[row] = 0;
      a.thr[row] = __builtin_inff();
    }
    return;
  }
  load_group_mask(a, b, sel);
  const float* x = a.xs + (size_t)row * a.N;
  const int32_t* lab = a.key_label + (size_t)a.head * a.N;
  float mx = -__builtin_inff(), mn = __builtin_inff();
  for (int j = t; j < a.N; j += NT) {
    mx = fmaxf(mx, x[j]);
    mn = fminf(mn, x[j]);
  }
  mx = block_max_f32<NT>(mx, tf);
  mn = block_min_f32<NT>(mn, tf);
  double z = 0.0;
  for (int j = t; j < a.N; j += NT) z += (double)expf(x[j] - mx);
  z = block_sum_f64<NT>(z, td);
  const float lse = mx + (float)log(z);
  // probabilities as fp64 from the fp32 logits: p_j = exp(x_j - max) / z
  double in = 0.0;
  for (int j = t; j < a.N; j += NT)
    if (routed(sel, clamp_idx(lab[j], a.G))) in += (double)expf(x[j] - mx);
  in = block_sum_f64<NT>(in, td) / z;
  // largest t (over the float order) with mass(x >= t) >= mu; the mass only
  // changes at logit values, so the answer is one of the logits
  uint32_t lo = float_order_bits(mn), hi = float_order_bits(mx);
  const double target = a.mu * z;
  while (lo < hi) {
    const uint32_t mid = (uint32_t)(((uint64_t)lo + hi + 1) / 2);
    const float th = float_from_order(mid);
    double s = 0.0;
    for (int j = t; j < a.N; j += NT)
      if (x[j] >= th) s += (double)expf(x[j] - mx);
    s = block_sum_f64<NT>(s, td);
    if (s >= target) lo = mid; else hi = mid - 1;
  }
  const float th = float_from_order(lo);
  int cnt = 0, cnt_r = 0;
  for (int j = t; j < a.N; j += NT)
    if (x[j] >= th) {
      ++cnt;
      cnt_r += routed(sel, clamp_idx(lab[j], a.G)) ? 1 : 0;
    }
  cnt = (int)block_sum_f64<NT>((double)cnt, td);
  cnt_r = (int)block_sum_f64<NT>((double)cnt_r, td);
  if (t == 0) {
    a.lse[row] = lse;
    a.mass[row] = (float)in;
    a.support[row] = cnt;
    a.support_routed[row] = cnt_r;
    a.thr[row] = th;
  }
}

// Pooled support of each sampled block: keys inside some row's support.
// grid (n_blocks, ceil(N / 256)), block 256; pooled counts start at zero.
__global__ __launch_bounds__(256) void k_support_pool(SupportArgs a) {
  __shared__ uint32_t sel[32];
  __shared__ double td[256];
  const int i = blockIdx.x;
  const int b = clamp_idx(a.blocks[i], a.nb);
  load_group_mask(a, b, sel);
  const int j = blockIdx.y * 256 + threadIdx.x;
  int in = 0, in_r = 0;
  if (j < a.N) {
    for (int r = 0; r < a.BQ; ++r) {
      const size_t row = (size_t)i * a.BQ + r;
      if (a.xs[row * a.N + j] >= a.thr[row]) {
        in = 1;
        break;
      }
    }
    in_r = in && routed(sel, clamp_idx(a.key_label[(size_t)a.head * a.N + j], a.G));
  }
  const int c = (int)block_sum_f64<256>((double)in, td);
  const int cr = (int)block_sum_f64<256>((double)in_r, td);
  if (threadIdx.x == 0) {
    if (c) atomicAdd(&a.pooled[i], c);
    if (cr) atomicAdd(&a.pooled_routed[i], cr);
  }
}

hipError_t launch_support(const Dims& d, const SupportArgs& a, hipStream_t st) {
  const int per = (d.BQ + kSupRows - 1) / kSupRows;
  const dim3 g1(a.n_blocks * per);
  if (d.bf16) {
    if (d.D == 128) k_support_logits<true, 128><<<g1, 256, 0, st>>>(a);
    else k_support_logits<true, 64><<<g1, 256, 0, st>>>(a);
  } else {
    if (d.D == 128) k_support_logits<false, 128><<<g1, 256, 0, st>>>(a);
    else k_support_logits<false, 64><<<g1, 256, 0, st>>>(a);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  k_support_row<<<a.n_blocks * d.BQ, 256, 0, st>>>(a);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if ((e = launch_fill_i32(a.pooled, (size_t)a.n_blocks, 0, st)) != hipSuccess) return e;
  if ((e = launch_fill_i32(a.pooled_routed, (size_t)a.n_blocks, 0, st)) != hipSuccess) return e;
  k_support_pool<<<dim3(a.n_blocks, (d.N + 255) / 256), 256, 0, st>>>(a);
  return hipGetLastError();
}

}  // namespace spr
