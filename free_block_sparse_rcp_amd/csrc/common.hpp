// Shared device helpers for the SparsePR gfx950 kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace spr {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef short s16x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// Round-to-nearest-even conversion (v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  __bf16 h = static_cast<__bf16>(f);
  return __builtin_bit_cast(uint16_t, h);
}

// Element access for the two storage types of Q/K/V/S/O.
template <bool BF16>
struct Elt;
template <>
struct Elt<true> {
  using T = uint16_t;
  static __device__ __forceinline__ float ld(const T* p, size_t i) { return bf16_to_f32(p[i]); }
  static __device__ __forceinline__ void st(T* p, size_t i, float v) { p[i] = f32_to_bf16(v); }
};
template <>
struct Elt<false> {
  using T = float;
  static __device__ __forceinline__ float ld(const T* p, size_t i) { return p[i]; }
  static __device__ __forceinline__ void st(T* p, size_t i, float v) { p[i] = v; }
};

__device__ __forceinline__ int clamp_idx(int i, int n) { return i < 0 ? 0 : (i >= n ? n - 1 : i); }

// Orderable bit pattern of a float: ascending uint order == ascending value.
// -0.0 is folded onto +0.0 so that equal values give equal keys.
__device__ __forceinline__ uint32_t float_order_bits(float f) {
  if (f == 0.0f) f = 0.0f;
  uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
// Key that sorts floats in DESCENDING order when sorted ascending.
__device__ __forceinline__ uint32_t float_desc_bits(float f) { return ~float_order_bits(f); }

// Query position of probe i < m: ppos[i] (clamped into [0, N)) when the
// caller gave positions, else floor((2 i + 1) N / (2 m)).
__device__ __forceinline__ int probe_position(const int32_t* ppos, int i, int N, int m) {
  if (ppos != nullptr) return clamp_idx(ppos[i], N);
  return (int)(((2LL * i + 1) * N) / (2LL * m));
}

// Lowest i < m whose given position is >= pos (m if none): binary search over
// the caller's increasing positions; every read stays inside [0, m).
__device__ __forceinline__ int probe_lower_bound(const int32_t* ppos, int pos, int N, int m) {
  int lo = 0, hi = m;
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if (clamp_idx(ppos[mid], N) < pos) lo = mid + 1;
    else hi = mid;
  }
  return lo;
}

// Index i of the probe at query position pos (probe i sits at
// floor((2 i + 1) N / (2 m))), or -1 when pos holds no probe.
__device__ __forceinline__ int probe_index(int pos, int N, int m) {
  if (m <= 0) return -1;
  const int64_t c = ((int64_t)pos * m) / N;
  for (int64_t i = c - 1; i <= c + 1; ++i) {
    if (i < 0 || i >= m) continue;
    if ((int)(((2 * i + 1) * N) / (2LL * m)) == pos) return (int)i;
  }
  return -1;
}

// The same with the caller's positions when ppos is not null.
__device__ __forceinline__ int probe_index(const int32_t* ppos, int pos, int N, int m) {
  if (ppos == nullptr) return probe_index(pos, N, m);
  if (m <= 0) return -1;
  const int i = probe_lower_bound(ppos, pos, N, m);
  return i < m && clamp_idx(ppos[i], N) == pos ? i : -1;
}

// Workgroups are dispatched round-robin over the 8 XCDs; this maps the
// dispatch id to a logical id so that each XCD receives one contiguous run of
// logical work items (neighbouring blocks share keys, so they share its L2).
__device__ __forceinline__ int xcd_remap(int w, int total) {
  const int q = total / 8, rem = total % 8;
  const int xcd = w % 8, idx = w / 8;
  return xcd < rem ? xcd * (q + 1) + idx : rem * (q + 1) + (xcd - rem) * q + idx;
}

// v_permlane32_swap on two floats: lo gets a in lanes 0-31 and b of lane
// l - 32 in lanes 32-63; hi gets a of lane l + 32 in lanes 0-31 and b in lanes
// 32-63. Scalar arguments and results: the builtin mis-lowers when fed vector
// elements directly. And a __builtin_bit_cast of any vector element (of this
// builtin's result or of a loaded vector) reads element 0 whichever element is
// named, so each element goes through an integer copy or cast first.
__device__ __forceinline__ void lane_half_swap(float a, float b, float& lo, float& hi) {
  const auto sw = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(unsigned, a),
                                                   __builtin_bit_cast(unsigned, b), false, false);
  lo = __builtin_bit_cast(float, (unsigned)sw[0]);
  hi = __builtin_bit_cast(float, (unsigned)sw[1]);
}

// Workgroup barrier for LDS-only exchange: waits for this wave's LDS
// operations, not for its outstanding global loads (which __syncthreads()'s
// fence would drain, stalling a prefetch in flight).
__device__ __forceinline__ void lds_barrier() {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0); vmcnt and expcnt untouched
  __builtin_amdgcn_s_barrier();
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

__device__ __forceinline__ uint64_t lanemask_lt() {
  const int lane = __lane_id();
  return lane == 0 ? 0ull : (~0ull >> (64 - lane));
}

// Exclusive scan of one int per thread across a workgroup of NT threads
// (whole waves): a scan inside each wave by lane shifts, then the wave totals
// through `tmp` (at least NT / 64 ints of shared memory). Returns the
// exclusive prefix and writes the total to *total. Contains two
// __syncthreads(); `tmp` may be reused right after it returns.
template <int NT>
__device__ __forceinline__ int block_exclusive_scan(int v, int* tmp, int* total) {
  static_assert(NT % 64 == 0, "whole waves");
  constexpr int NW = NT / 64;
  const int t = threadIdx.x, lane = t & 63, w = t >> 6;
  int x = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int y = __shfl_up(x, off);
    if (lane >= off) x += y;
  }
  if (lane == 63) tmp[w] = x;
  __syncthreads();
  int before = 0, all = 0;
#pragma unroll
  for (int i = 0; i < NW; ++i) {
    const int s = tmp[i];
    before += i < w ? s : 0;
    all += s;
  }
  *total = all;
  __syncthreads();
  return before + x - v;
}

template <int NT>
__device__ __forceinline__ double block_sum_f64(double v, double* tmp) {
  const int t = threadIdx.x;
  tmp[t] = v;
  __syncthreads();
  for (int off = NT / 2; off > 0; off >>= 1) {
    if (t < off) tmp[t] += tmp[t + off];
    __syncthreads();
  }
  double r = tmp[0];
  __syncthreads();
  return r;
}

}  // namespace spr
