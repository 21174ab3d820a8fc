// Host-side launchers shared between the C-ABI (api.hip) and the kernel files.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/sparsepr.h"

namespace spr {

// Sizes derived from sparsepr_params, computed once per call on the host.
constexpr int kSortChunk = 2048;   // elements per workgroup of a counting-sort pass

struct Dims {
  int H, N, D, G, S, T, BQ, nb, m, k;
  bool bf16;
  int mode;
  double rho, lam;
  int64_t kappa;
  int nchunk;     // ceil(N / kSortChunk): chunks of the counting-sort passes
  int gbits;      // bits needed for a group index (0 when G == 1)
  int nsplit;     // probe attention: key splits
  int split_len;  // probe attention: keys per split (multiple of 64)
  const int32_t* ppos;  // probe positions [m] (device), or null for the default rule
};

// ---- workspace layout (byte offsets; one workspace serves every stage)
struct PartitionWs {
  size_t M, P, Phl, bvec, counts, totals, starts, best, end;
};
struct RouteWs {
  size_t keysA, keysB, valsA, valsB, counts, totals, starts, sigma, sel, selcnt, blkkeys,
      chl, best, end;
};
struct ProbeWs {
  size_t opart, lsepart, fit, fit_per_head, end;
};
struct ApplyWs {
  size_t wt, bias, end;   // W^T as bf16 hi/lo [H][2][d][d]; bias [H][d] fp32
};
PartitionWs partition_ws(const Dims& d);
RouteWs route_ws(const Dims& d);
ProbeWs probe_ws(const Dims& d);
ApplyWs apply_ws(const Dims& d);
size_t fit_ws_per_head(const Dims& d);

// ---- partition.hip
hipError_t launch_partition(const Dims& d, const void* Q, const void* K, const void* V,
                            const float* scale, const int32_t* sample_idx, const int32_t* init_idx,
                            const int32_t* rand_key_perm, int32_t* key_label, int32_t* key_perm,
                            int32_t* group_off, float* kbar, void* Kp, void* Vp, float* dbg,
                            char* ws, hipStream_t st);

// counting-sort pass used by partition (labels) and route (query keys)
hipError_t launch_sort_pass_u32(const Dims& d, const int32_t* keys_in, int bits,
                                const int32_t* vals_in, int32_t* vals_out, int32_t* counts,
                                int32_t* totals, int32_t* starts, int32_t* group_off_out,
                                hipStream_t st);
hipError_t launch_sort_pass_u64(const Dims& d, const uint64_t* keys_in, uint64_t* keys_out,
                                int shift, int bits, const int32_t* vals_in, int32_t* vals_out,
                                int32_t* counts, int32_t* totals, int32_t* starts, hipStream_t st);

// row x centroid arg-selection on MFMA (bf16 rows): mode 0 argmin of
// b - 2 x.P, mode 1 argmax of tau x.P over non-empty groups
hipError_t launch_rowvec_mfma(const Dims& d, int mode, const void* X, const uint16_t* Phl,
                              const float* bvec, const float* scale, const int32_t* group_off,
                              unsigned long long* best, float* dbg, hipStream_t st);
hipError_t launch_best_to_label(const Dims& d, const unsigned long long* best, bool descending,
                                int32_t* label, float* value, hipStream_t st);
hipError_t launch_split_hilo(const float* src, size_t rows, int D, uint16_t* dst, hipStream_t st);

// fills by kernel (no memset nodes, so callers may capture the stream)
hipError_t launch_fill_i32(int32_t* p, size_t n, int32_t v, hipStream_t st);
hipError_t launch_fill_f32(float* p, size_t n, float v, hipStream_t st);

// ---- route.hip
hipError_t launch_route(const Dims& d, const void* Q, const float* scale, const float* kbar,
                        const int32_t* group_off, const int32_t* rand_query_perm,
                        int32_t* query_perm, int32_t* block_ptr, int32_t* block_groups,
                        int64_t* executed_pairs, float* dbg_coords, int32_t* dbg_dom,
                        float* dbg_domval, float* dbg_sigma, char* ws, hipStream_t st);

// ---- attention.hip
enum AttnMode { ATTN_SPARSE = 0, ATTN_DENSE = 1, ATTN_PROBE = 2 };
struct AttnArgs {
  const void* Q;
  const void* K;
  const void* V;
  const float* scale;
  int H, N, m, nsplit, split_len, G, nb;
  const int32_t* query_perm;   // sparse / probe
  const int32_t* block_ptr;    // sparse
  const int32_t* block_groups; // sparse
  const int32_t* group_off;    // sparse
  void* out;                   // sparse: S_out dtype (query order); dense: O dtype (token order)
  float* sprobe;               // sparse: fp32 rows of the probe positions [H][m][d] (or null)
  float* lse;                  // sparse / dense (may be null for dense)
  float* opart;                // probe: [H, nsplit, m, D] fp32
  float* lsepart;              // probe: [H, nsplit, m]
  int xcd_chunk;               // > 0: head-synchronous XCD mapping with this many blocks per XCD
  int subset;                  // sparse: 0 all blocks, 1 blocks holding a probe row, 2 the others
  int* qctr;                   // sparse / dense, bf16: 8 work-queue counters kQueueStride ints
                               // apart (persistent grid), or null (one item per workgroup)
  const int32_t* ppos;         // sparse / probe: probe positions [m], or null (default rule)
};
// Spacing of the attention's work-queue counters (ints): one per 128-byte line.
constexpr int kQueueStride = 32;
hipError_t launch_attention(const Dims& d, AttnMode mode, const AttnArgs& a, hipStream_t st);
hipError_t launch_probe_merge(const Dims& d, const float* opart, const float* lsepart,
                              float* O_probe, hipStream_t st);

// ---- support.hip
struct SupportArgs {
  const void* Q;
  const void* K;               // token order
  const float* scale;
  const int32_t* key_label;
  const int32_t* query_perm;
  const int32_t* block_ptr;
  const int32_t* block_groups;
  const int32_t* blocks;       // [n_blocks] sampled block indices
  int n_blocks, head, N, nb, G, BQ;
  double mu;                   // target mass
  float* xs;                   // workspace: [n_blocks * B_q, N] logits
  float* thr;                  // workspace: [n_blocks * B_q] support thresholds
  float* lse;                  // [n_blocks * B_q]
  float* mass;                 // [n_blocks * B_q]
  int32_t* support;            // [n_blocks * B_q]
  int32_t* support_routed;     // [n_blocks * B_q]
  int32_t* pooled;             // [n_blocks]
  int32_t* pooled_routed;      // [n_blocks]
};
hipError_t launch_support(const Dims& d, const SupportArgs& a, hipStream_t st);

// ---- fit.hip
hipError_t launch_fit(const Dims& d, const float* S_probe, const float* O_probe, float* U,
                      float* Theta, int32_t* rank_eff, char* fit_ws, hipStream_t st);

// ---- apply.hip
hipError_t launch_apply(const Dims& d, const void* S_out, const int32_t* query_perm,
                        const float* O_probe, const float* U, const float* Theta,
                        const int32_t* rank_eff, void* O, char* ws, hipStream_t st);

}  // namespace spr
