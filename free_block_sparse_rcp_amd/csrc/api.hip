// C-ABI of the SparsePR operator: host-side validation, workspace layout and
// the stage launch sequences. Every check happens before the first launch.
#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>

#include "internal.hpp"

namespace spr {

static thread_local char g_last_error[512] = "";

static int32_t fail(int32_t code, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
static int32_t fail(int32_t code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
  va_end(ap);
  return code;
}

static size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

struct Bump {
  size_t off = 0;
  size_t take(size_t bytes) {
    const size_t o = align256(off);
    off = o + bytes;
    return o;
  }
};

static int bits_for(int n) {
  int b = 0;
  while ((1 << b) < n) ++b;
  return b;
}

PartitionWs partition_ws(const Dims& d) {
  Bump b;
  PartitionWs L;
  const size_t H = d.H, G = d.G, D = d.D;
  const size_t nbk = size_t(1) << d.gbits;
  L.M = b.take(H * D * D * sizeof(double));
  L.P = b.take(H * G * D * sizeof(float));
  L.Phl = b.take(H * G * D * 2 * sizeof(uint16_t));
  L.bvec = b.take(H * G * sizeof(float));
  L.counts = b.take(H * nbk * d.nchunk * sizeof(int32_t));
  L.totals = b.take(H * nbk * sizeof(int32_t));
  L.starts = b.take(H * nbk * sizeof(int32_t));
  L.best = b.take(H * (size_t)d.N * sizeof(unsigned long long));
  L.end = align256(b.off);
  return L;
}

RouteWs route_ws(const Dims& d) {
  Bump b;
  RouteWs L;
  const size_t H = d.H, N = d.N, G = d.G, nb = d.nb;
  const size_t nbk = std::max<size_t>(256, size_t(1) << d.gbits);
  L.keysA = b.take(H * N * 8);
  L.keysB = b.take(H * N * 8);
  L.valsA = b.take(H * N * 4);
  L.valsB = b.take(H * N * 4);
  L.counts = b.take(H * nbk * d.nchunk * 4);
  L.totals = b.take(H * nbk * 4);
  L.starts = b.take(H * nbk * 4);
  L.sigma = b.take(H * nb * G * 4);
  L.sel = b.take(H * nb * G * 4);
  L.selcnt = b.take(H * nb * 4);
  L.blkkeys = b.take(H * nb * 8);
  L.chl = b.take(H * G * d.D * 2 * 2);
  L.best = b.take(H * N * 8);
  L.end = align256(b.off);
  return L;
}

ProbeWs probe_ws(const Dims& d) {
  Bump b;
  ProbeWs L;
  const size_t H = d.H, m = d.m;
  L.opart = b.take(H * d.nsplit * m * d.D * 4);
  L.lsepart = b.take(H * d.nsplit * m * 4);
  L.fit_per_head = fit_ws_per_head(d);
  L.fit = b.take(H * L.fit_per_head);
  L.end = align256(b.off);
  return L;
}

ApplyWs apply_ws(const Dims& d) {
  Bump b;
  ApplyWs L;
  const size_t H = d.H, D = d.D;
  L.wt = b.take(H * 2 * D * D * 2);
  L.bias = b.take(H * D * 4);
  L.end = align256(b.off);
  return L;
}

constexpr int kProbeSlots = 768;   // resident probe-attention workgroups: 3 per CU x 256 CUs

// Validation of the parameters; `full` also checks the fields that only the
// sparse stages use.
static int32_t make_dims(const sparsepr_params* p, bool full, Dims* d) {
  if (p == nullptr) return fail(SPARSEPR_ERR_INVALID_ARG, "params is NULL");
  if (p->heads < 1) return fail(SPARSEPR_ERR_INVALID_ARG, "heads must be >= 1 (got %d)", p->heads);
  // heads are the second grid dimension of several launches
  if (p->heads > 65535) return fail(SPARSEPR_ERR_UNSUPPORTED, "heads must be <= 65535 (got %d)", p->heads);
  if (p->n_tokens < 1) return fail(SPARSEPR_ERR_INVALID_ARG, "n_tokens must be >= 1 (got %d)", p->n_tokens);
  if (p->head_dim != 64 && p->head_dim != 128)
    return fail(SPARSEPR_ERR_UNSUPPORTED, "head_dim must be 64 or 128 (got %d)", p->head_dim);
  if (p->dtype != SPARSEPR_F32 && p->dtype != SPARSEPR_BF16)
    return fail(SPARSEPR_ERR_INVALID_ARG, "dtype must be SPARSEPR_F32 or SPARSEPR_BF16 (got %d)", p->dtype);
  if (p->q_block != 64 && p->q_block != 128)
    return fail(SPARSEPR_ERR_UNSUPPORTED, "q_block must be 64 or 128 (got %d)", p->q_block);
  if ((int64_t)p->heads * p->n_tokens * p->head_dim > (int64_t(1) << 40))
    return fail(SPARSEPR_ERR_UNSUPPORTED, "H*N*d too large");
  if ((int64_t)p->n_tokens * p->head_dim >= (int64_t(1) << 31))
    return fail(SPARSEPR_ERR_UNSUPPORTED, "N*d must fit in 31 bits");
  d->H = p->heads;
  d->N = p->n_tokens;
  d->D = p->head_dim;
  d->bf16 = p->dtype == SPARSEPR_BF16;
  d->BQ = p->q_block;
  d->nb = (d->N + d->BQ - 1) / d->BQ;
  d->nchunk = (d->N + kSortChunk - 1) / kSortChunk;
  d->G = 1;
  d->S = 1;
  d->T = 1;
  d->m = 0;
  d->k = 0;
  d->mode = 0;
  d->rho = 1.0;
  d->lam = 1.0;
  d->kappa = d->N;
  d->gbits = 0;
  d->nsplit = 1;
  d->split_len = d->N;
  d->ppos = nullptr;
  if (!full) return SPARSEPR_OK;
  if (p->reserved != 0) return fail(SPARSEPR_ERR_INVALID_ARG, "reserved must be 0");
  if (p->partition_mode != SPARSEPR_RESPONSE_COUPLED && p->partition_mode != SPARSEPR_RANDOM_BLOCK &&
      p->partition_mode != SPARSEPR_SEMANTIC)
    return fail(SPARSEPR_ERR_INVALID_ARG, "partition_mode must be 0, 1 or 2 (got %d)", p->partition_mode);
  if (p->n_groups < 1 || p->n_groups > 1024 || p->n_groups > p->n_tokens)
    return fail(SPARSEPR_ERR_INVALID_ARG, "n_groups must be in [1, min(N, 1024)] (got %d)", p->n_groups);
  if (p->partition_mode == SPARSEPR_RESPONSE_COUPLED &&
      (p->n_samples < 1 || p->n_samples > p->n_tokens))
    return fail(SPARSEPR_ERR_INVALID_ARG, "n_samples must be in [1, N] (got %d)", p->n_samples);
  if (p->partition_mode != SPARSEPR_RANDOM_BLOCK) {
    if (p->kmeans_iters < 1)
      return fail(SPARSEPR_ERR_INVALID_ARG, "kmeans_iters must be >= 1 (got %d)", p->kmeans_iters);
  }
  if (!(p->density > 0.0 && p->density <= 1.0))
    return fail(SPARSEPR_ERR_INVALID_ARG, "density must be in (0, 1] (got %g)", p->density);
  if (p->n_probes < 0 || p->n_probes > p->n_tokens)
    return fail(SPARSEPR_ERR_INVALID_ARG, "n_probes must be in [0, N] (got %d)", p->n_probes);
  if (p->rank < 0 || p->rank > p->head_dim)
    return fail(SPARSEPR_ERR_INVALID_ARG, "rank must be in [0, d] (got %d)", p->rank);
  if (!(p->ridge_lambda > 0.0) || !std::isfinite(p->ridge_lambda))
    return fail(SPARSEPR_ERR_INVALID_ARG, "ridge_lambda must be > 0 (got %g)", p->ridge_lambda);
  const double kap = std::floor(p->density * (double)p->n_tokens - (double)p->n_probes);
  if (kap < 1.0)
    return fail(SPARSEPR_ERR_INVALID_ARG,
                "key budget floor(density*N - n_probes) = %.0f must be >= 1", kap);
  d->G = p->n_groups;
  d->S = p->n_samples;
  d->T = p->kmeans_iters;
  d->m = p->n_probes;
  d->ppos = d->m > 0 ? p->probe_pos : nullptr;   // device array, not read here
  d->k = p->rank;
  d->mode = p->partition_mode;
  d->rho = p->density;
  d->lam = p->ridge_lambda;
  d->kappa = (int64_t)kap;
  d->gbits = bits_for(d->G);
  if (d->m > 0) {
    // key splits of the exact probe rows: as many workgroups as fit on the chip
    // at once (three per CU on 256 CUs), so that the pass runs in one round
    const int nqb = (d->m + d->BQ - 1) / d->BQ;
    const int items = d->H * nqb;
    int nsplit = kProbeSlots / items;
    nsplit = std::max(1, std::min(nsplit, (d->N + 255) / 256));
    int len = (d->N + nsplit - 1) / nsplit;
    len = (len + 63) / 64 * 64;
    d->split_len = len;
    d->nsplit = (d->N + len - 1) / len;
  }
  return SPARSEPR_OK;
}

static size_t total_ws(const Dims& d) {
  return std::max(std::max(partition_ws(d).end, route_ws(d).end),
                  std::max(probe_ws(d).end, apply_ws(d).end));
}

#define SPR_REQUIRE(ptr, name) \
  if ((ptr) == nullptr) return fail(SPARSEPR_ERR_INVALID_ARG, "%s is NULL", name)

static int32_t check_ws(const Dims& d, const void* ws, size_t ws_bytes) {
  const size_t need = total_ws(d);
  if (ws == nullptr || ws_bytes < need)
    return fail(SPARSEPR_ERR_WORKSPACE, "workspace of %zu bytes needed (got %zu%s)", need, ws_bytes,
                ws == nullptr ? ", NULL" : "");
  return SPARSEPR_OK;
}

// The attention's work queues: optional; when given, SPARSEPR_QUEUE_BYTES of
// 4-byte aligned device memory (8 counters, one per 128-byte line).
static_assert(SPARSEPR_QUEUE_BYTES == 8 * kQueueStride * sizeof(int), "queue layout");
static int32_t check_queue(const void* queue, size_t queue_bytes) {
  if (queue == nullptr) return SPARSEPR_OK;
  if (reinterpret_cast<uintptr_t>(queue) % 4 != 0)
    return fail(SPARSEPR_ERR_INVALID_ARG, "queue must be 4-byte aligned");
  if (queue_bytes < SPARSEPR_QUEUE_BYTES)
    return fail(SPARSEPR_ERR_WORKSPACE, "queue of %d bytes needed (got %zu)", SPARSEPR_QUEUE_BYTES,
                queue_bytes);
  return SPARSEPR_OK;
}

static int32_t hip_status(hipError_t e, const char* stage) {
  if (e == hipSuccess) {
    g_last_error[0] = 0;
    return SPARSEPR_OK;
  }
  return fail(SPARSEPR_ERR_HIP, "%s: %s", stage, hipGetErrorString(e));
}

// ---- fixed scratch of sparsepr_apply_noalloc: the per-head matrix Theta U^T
// (bf16 hi/lo parts) and bias that sparsepr_apply keeps in the workspace live
// here instead. Each device holds its own copy for the life of the process.
// In host code `scratch` is only a stand-in for the symbol: kernels receive
// the device address looked up below, never the array's name.
static __device__ __align__(256) char scratch[SPARSEPR_APPLY_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
static std::mutex g_scratch_mu;
static char* g_scratch_ptr[kMaxDevices] = {};

// Device address of `scratch` on the current device, looked up once per device
// (with that device current) and kept.
static int32_t scratch_address(char** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(SPARSEPR_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices)
    return fail(SPARSEPR_ERR_UNSUPPORTED, "device index %d beyond %d", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || ptr == nullptr)
      return fail(SPARSEPR_ERR_HIP, "hipGetSymbolAddress(scratch) on device %d: %s", dev,
                  hipGetErrorString(e));
    g_scratch_ptr[dev] = static_cast<char*>(ptr);
  }
  *out = g_scratch_ptr[dev];
  return SPARSEPR_OK;
}

}  // namespace spr

using namespace spr;

extern "C" {

int32_t sparsepr_abi_version(void) { return SPARSEPR_ABI_VERSION; }

const char* sparsepr_status_string(int32_t status) {
  switch (status) {
    case SPARSEPR_OK: return "SPARSEPR_OK";
    case SPARSEPR_ERR_INVALID_ARG: return "SPARSEPR_ERR_INVALID_ARG";
    case SPARSEPR_ERR_UNSUPPORTED: return "SPARSEPR_ERR_UNSUPPORTED";
    case SPARSEPR_ERR_WORKSPACE: return "SPARSEPR_ERR_WORKSPACE";
    case SPARSEPR_ERR_HIP: return "SPARSEPR_ERR_HIP";
    default: return "SPARSEPR_UNKNOWN_STATUS";
  }
}

const char* sparsepr_last_error(void) { return g_last_error; }

int32_t sparsepr_workspace_bytes(const sparsepr_params* params, size_t* bytes) {
  Dims d;
  const int32_t s = make_dims(params, true, &d);
  if (s != SPARSEPR_OK) return s;
  SPR_REQUIRE(bytes, "bytes");
  *bytes = total_ws(d);
  return SPARSEPR_OK;
}

int32_t sparsepr_partition(const sparsepr_params* params, const void* Q, const void* K,
                           const void* V, const float* scale, const int32_t* sample_idx,
                           const int32_t* init_idx, const int32_t* rand_key_perm,
                           int32_t* key_label, int32_t* key_perm, int32_t* group_off,
                           float* key_centroid, void* Kp, void* Vp, float* dbg_assign_scores,
                           void* workspace, size_t workspace_bytes, void* stream) {
  Dims d;
  int32_t s = make_dims(params, true, &d);
  if (s != SPARSEPR_OK) return s;
  SPR_REQUIRE(K, "K");
  if ((Kp == nullptr) != (Vp == nullptr))
    return fail(SPARSEPR_ERR_INVALID_ARG, "Kp and Vp must both be given or both be NULL");
  if (Kp != nullptr) SPR_REQUIRE(V, "V");
  if (d.mode == SPARSEPR_RESPONSE_COUPLED) {
    SPR_REQUIRE(Q, "Q");
    SPR_REQUIRE(scale, "scale");
    SPR_REQUIRE(sample_idx, "sample_idx");
    SPR_REQUIRE(init_idx, "init_idx");
  } else if (d.mode == SPARSEPR_SEMANTIC) {
    SPR_REQUIRE(init_idx, "init_idx");
  } else {
    SPR_REQUIRE(rand_key_perm, "rand_key_perm");
  }
  SPR_REQUIRE(key_label, "key_label");
  SPR_REQUIRE(key_perm, "key_perm");
  SPR_REQUIRE(group_off, "group_off");
  SPR_REQUIRE(key_centroid, "key_centroid");
  if ((s = check_ws(d, workspace, workspace_bytes)) != SPARSEPR_OK) return s;
  return hip_status(launch_partition(d, Q, K, V, scale, sample_idx, init_idx, rand_key_perm,
                                     key_label, key_perm, group_off, key_centroid, Kp, Vp,
                                     dbg_assign_scores, static_cast<char*>(workspace),
                                     static_cast<hipStream_t>(stream)),
                    "sparsepr_partition");
}

int32_t sparsepr_route(const sparsepr_params* params, const void* Q, const float* scale,
                       const float* key_centroid, const int32_t* group_off,
                       const int32_t* rand_query_perm, int32_t* query_perm, int32_t* block_ptr,
                       int32_t* block_groups, int64_t* executed_pairs, float* dbg_coords,
                       int32_t* dbg_dominant, float* dbg_dominant_val, float* dbg_block_score,
                       void* workspace, size_t workspace_bytes, void* stream) {
  Dims d;
  int32_t s = make_dims(params, true, &d);
  if (s != SPARSEPR_OK) return s;
  SPR_REQUIRE(Q, "Q");
  SPR_REQUIRE(scale, "scale");
  SPR_REQUIRE(key_centroid, "key_centroid");
  SPR_REQUIRE(group_off, "group_off");
  if (d.mode != SPARSEPR_RESPONSE_COUPLED) SPR_REQUIRE(rand_query_perm, "rand_query_perm");
  SPR_REQUIRE(query_perm, "query_perm");
  SPR_REQUIRE(block_ptr, "block_ptr");
  SPR_REQUIRE(block_groups, "block_groups");
  SPR_REQUIRE(executed_pairs, "executed_pairs");
  if ((s = check_ws(d, workspace, workspace_bytes)) != SPARSEPR_OK) return s;
  return hip_status(launch_route(d, Q, scale, key_centroid, group_off, rand_query_perm,
                                 query_perm, block_ptr, block_groups, executed_pairs, dbg_coords,
                                 dbg_dominant, dbg_dominant_val, dbg_block_score,
                                 static_cast<char*>(workspace), static_cast<hipStream_t>(stream)),
                    "sparsepr_route");
}

int32_t sparsepr_attend_subset(const sparsepr_params* params, const void* Q, const void* Kp,
                               const void* Vp, const float* scale, const int32_t* group_off,
                               const int32_t* query_perm, const int32_t* block_ptr,
                               const int32_t* block_groups, void* S_out, float* S_probe,
                               float* lse, int32_t subset, void* queue, size_t queue_bytes,
                               void* stream) {
  Dims d;
  int32_t s = make_dims(params, true, &d);
  if (s != SPARSEPR_OK) return s;
  if (subset < SPARSEPR_BLOCKS_ALL || subset > SPARSEPR_BLOCKS_WITHOUT_PROBE)
    return fail(SPARSEPR_ERR_INVALID_ARG, "subset must be 0, 1 or 2 (got %d)", subset);
  if ((s = check_queue(queue, queue_bytes)) != SPARSEPR_OK) return s;
  SPR_REQUIRE(Q, "Q");
  SPR_REQUIRE(Kp, "Kp");
  SPR_REQUIRE(Vp, "Vp");
  SPR_REQUIRE(scale, "scale");
  SPR_REQUIRE(group_off, "group_off");
  SPR_REQUIRE(query_perm, "query_perm");
  SPR_REQUIRE(block_ptr, "block_ptr");
  SPR_REQUIRE(block_groups, "block_groups");
  SPR_REQUIRE(S_out, "S_out");
  if (d.m > 0) SPR_REQUIRE(S_probe, "S_probe");
  SPR_REQUIRE(lse, "lse");
  AttnArgs a{};
  a.Q = Q;
  a.K = Kp;
  a.V = Vp;
  a.scale = scale;
  a.H = d.H;
  a.N = d.N;
  a.m = d.m;
  a.ppos = d.ppos;
  a.nsplit = 1;
  a.split_len = d.N;
  a.G = d.G;
  a.nb = d.nb;
  a.query_perm = query_perm;
  a.block_ptr = block_ptr;
  a.block_groups = block_groups;
  a.group_off = group_off;
  a.out = S_out;
  a.sprobe = d.m > 0 ? S_probe : nullptr;
  a.lse = lse;
  a.subset = subset;
  a.qctr = static_cast<int*>(queue);
  return hip_status(launch_attention(d, ATTN_SPARSE, a, static_cast<hipStream_t>(stream)),
                    "sparsepr_attend");
}

int32_t sparsepr_attend(const sparsepr_params* params, const void* Q, const void* Kp,
                        const void* Vp, const float* scale, const int32_t* group_off,
                        const int32_t* query_perm, const int32_t* block_ptr,
                        const int32_t* block_groups, void* S_out, float* S_probe, float* lse,
                        void* queue, size_t queue_bytes, void* stream) {
  return sparsepr_attend_subset(params, Q, Kp, Vp, scale, group_off, query_perm, block_ptr,
                                block_groups, S_out, S_probe, lse, SPARSEPR_BLOCKS_ALL, queue,
                                queue_bytes, stream);
}

int32_t sparsepr_support_stats(const sparsepr_params* params, int32_t head, const void* Q,
                               const void* K, const float* scale, const int32_t* key_label,
                               const int32_t* query_perm, const int32_t* block_ptr,
                               const int32_t* block_groups, const int32_t* blocks,
                               int32_t n_blocks, double mass, float* lse, float* routed_mass,
                               int32_t* support, int32_t* support_routed, int32_t* pooled,
                               int32_t* pooled_routed, void* workspace, size_t workspace_bytes,
                               void* stream) {
  Dims d;
  int32_t s = make_dims(params, true, &d);
  if (s != SPARSEPR_OK) return s;
  if (head < 0 || head >= d.H)
    return fail(SPARSEPR_ERR_INVALID_ARG, "head must be in [0, H) (got %d)", head);
  if (n_blocks < 1 || n_blocks > d.nb)
    return fail(SPARSEPR_ERR_INVALID_ARG, "n_blocks must be in [1, nb] (got %d)", n_blocks);
  if (!(mass > 0.0 && mass <= 1.0))
    return fail(SPARSEPR_ERR_INVALID_ARG, "mass must be in (0, 1] (got %g)", mass);
  // the pooled-support pass puts 256-key slices of a row on the grid's second dimension
  if ((d.N + 255) / 256 > 65535)
    return fail(SPARSEPR_ERR_UNSUPPORTED, "support statistics need N <= 16776960 (got %d)", d.N);
  SPR_REQUIRE(Q, "Q");
  SPR_REQUIRE(K, "K");
  SPR_REQUIRE(scale, "scale");
  SPR_REQUIRE(key_label, "key_label");
  SPR_REQUIRE(query_perm, "query_perm");
  SPR_REQUIRE(block_ptr, "block_ptr");
  SPR_REQUIRE(block_groups, "block_groups");
  SPR_REQUIRE(blocks, "blocks");
  SPR_REQUIRE(lse, "lse");
  SPR_REQUIRE(routed_mass, "routed_mass");
  SPR_REQUIRE(support, "support");
  SPR_REQUIRE(support_routed, "support_routed");
  SPR_REQUIRE(pooled, "pooled");
  SPR_REQUIRE(pooled_routed, "pooled_routed");
  const size_t rows = (size_t)n_blocks * d.BQ;
  const size_t need = rows * ((size_t)d.N + 1) * sizeof(float);
  if (workspace == nullptr || workspace_bytes < need)
    return fail(SPARSEPR_ERR_WORKSPACE, "workspace of %zu bytes needed (got %zu%s)", need,
                workspace_bytes, workspace == nullptr ? ", NULL" : "");
  SupportArgs a{};
  a.Q = Q;
  a.K = K;
  a.scale = scale;
  a.key_label = key_label;
  a.query_perm = query_perm;
  a.block_ptr = block_ptr;
  a.block_groups = block_groups;
  a.blocks = blocks;
  a.n_blocks = n_blocks;
  a.head = head;
  a.N = d.N;
  a.nb = d.nb;
  a.G = d.G;
  a.BQ = d.BQ;
  a.mu = mass;
  a.xs = static_cast<float*>(workspace);
  a.thr = a.xs + rows * (size_t)d.N;
  a.lse = lse;
  a.mass = routed_mass;
  a.support = support;
  a.support_routed = support_routed;
  a.pooled = pooled;
  a.pooled_routed = pooled_routed;
  return hip_status(launch_support(d, a, static_cast<hipStream_t>(stream)),
                    "sparsepr_support_stats");
}

int32_t sparsepr_probe_fit(const sparsepr_params* params, const void* Q, const void* K,
                           const void* V, const float* scale, const int32_t* query_perm,
                           const float* S_probe, float* O_probe, float* U, float* Theta,
                           int32_t* rank_eff, void* workspace, size_t workspace_bytes,
                           void* stream) {
  Dims d;
  int32_t s = make_dims(params, true, &d);
  if (s != SPARSEPR_OK) return s;
  SPR_REQUIRE(rank_eff, "rank_eff");
  if (d.m > 0) {
    SPR_REQUIRE(Q, "Q");
    SPR_REQUIRE(K, "K");
    SPR_REQUIRE(V, "V");
    SPR_REQUIRE(scale, "scale");
    SPR_REQUIRE(query_perm, "query_perm");
    SPR_REQUIRE(S_probe, "S_probe");
    SPR_REQUIRE(O_probe, "O_probe");
  }
  if (d.k > 0) {
    SPR_REQUIRE(U, "U");
    SPR_REQUIRE(Theta, "Theta");
  }
  if ((s = check_ws(d, workspace, workspace_bytes)) != SPARSEPR_OK) return s;
  const hipStream_t st = static_cast<hipStream_t>(stream);
  const ProbeWs L = probe_ws(d);
  char* ws = static_cast<char*>(workspace);
  hipError_t e = hipSuccess;
  if (d.m > 0) {
    AttnArgs a{};
    a.Q = Q;
    a.K = K;
    a.V = V;
    a.scale = scale;
    a.H = d.H;
    a.N = d.N;
    a.m = d.m;
  a.ppos = d.ppos;
    a.nsplit = d.nsplit;
    a.split_len = d.split_len;
    a.G = d.G;
    a.nb = d.nb;
    a.query_perm = query_perm;
    a.opart = reinterpret_cast<float*>(ws + L.opart);
    a.lsepart = reinterpret_cast<float*>(ws + L.lsepart);
    e = launch_attention(d, ATTN_PROBE, a, st);
    if (e == hipSuccess) e = launch_probe_merge(d, a.opart, a.lsepart, O_probe, st);
  }
  if (e == hipSuccess) {
    if (d.m > 0 && d.k > 0) {
      e = launch_fit(d, S_probe, O_probe, U, Theta, rank_eff, ws + L.fit, st);
    } else {
      e = launch_fill_i32(rank_eff, (size_t)d.H, 0, st);
      if (e == hipSuccess && d.k > 0) e = launch_fill_f32(U, (size_t)d.H * d.D * d.k, 0.f, st);
      if (e == hipSuccess && d.k > 0)
        e = launch_fill_f32(Theta, (size_t)d.H * (d.D + 1) * d.k, 0.f, st);
    }
  }
  return hip_status(e, "sparsepr_probe_fit");
}

int32_t sparsepr_apply(const sparsepr_params* params, const void* S_out,
                       const int32_t* query_perm, const float* O_probe, const float* U,
                       const float* Theta, const int32_t* rank_eff, void* O, void* workspace,
                       size_t workspace_bytes, void* stream) {
  Dims d;
  int32_t s = make_dims(params, true, &d);
  if (s != SPARSEPR_OK) return s;
  SPR_REQUIRE(S_out, "S_out");
  SPR_REQUIRE(query_perm, "query_perm");
  SPR_REQUIRE(rank_eff, "rank_eff");
  SPR_REQUIRE(O, "O");
  if (d.m > 0) SPR_REQUIRE(O_probe, "O_probe");
  if (d.k > 0) {
    SPR_REQUIRE(U, "U");
    SPR_REQUIRE(Theta, "Theta");
  }
  if ((s = check_ws(d, workspace, workspace_bytes)) != SPARSEPR_OK) return s;
  return hip_status(launch_apply(d, S_out, query_perm, O_probe, U, Theta, rank_eff, O,
                                 static_cast<char*>(workspace), static_cast<hipStream_t>(stream)),
                    "sparsepr_apply");
}

int32_t sparsepr_apply_noalloc(const sparsepr_params* params, const void* S_out,
                               const int32_t* query_perm, const float* O_probe, const float* U,
                               const float* Theta, const int32_t* rank_eff, void* O,
                               void* stream) {
  Dims d;
  int32_t s = make_dims(params, true, &d);
  if (s != SPARSEPR_OK) return s;
  SPR_REQUIRE(S_out, "S_out");
  SPR_REQUIRE(query_perm, "query_perm");
  SPR_REQUIRE(rank_eff, "rank_eff");
  SPR_REQUIRE(O, "O");
  if (d.m > 0) SPR_REQUIRE(O_probe, "O_probe");
  if (d.k > 0) {
    SPR_REQUIRE(U, "U");
    SPR_REQUIRE(Theta, "Theta");
  }
  const size_t need = d.bf16 ? apply_ws(d).end : 0;
  if (need > SPARSEPR_APPLY_SCRATCH_BYTES)
    return fail(SPARSEPR_ERR_WORKSPACE,
                "sparsepr_apply_noalloc needs %zu bytes of scratch for %d heads of dimension %d; "
                "its fixed scratch holds %zu (use sparsepr_apply with a workspace)",
                need, d.H, d.D, (size_t)SPARSEPR_APPLY_SCRATCH_BYTES);
  char* ws = nullptr;
  if ((s = scratch_address(&ws)) != SPARSEPR_OK) return s;
  return hip_status(launch_apply(d, S_out, query_perm, O_probe, U, Theta, rank_eff, O, ws,
                                 static_cast<hipStream_t>(stream)),
                    "sparsepr_apply_noalloc");
}

int32_t sparsepr_dense_attention(const sparsepr_params* params, const void* Q, const void* K,
                                 const void* V, const float* scale, void* O, float* lse,
                                 void* queue, size_t queue_bytes, void* stream) {
  Dims d;
  int32_t s = make_dims(params, false, &d);
  if (s != SPARSEPR_OK) return s;
  SPR_REQUIRE(Q, "Q");
  SPR_REQUIRE(K, "K");
  SPR_REQUIRE(V, "V");
  SPR_REQUIRE(scale, "scale");
  SPR_REQUIRE(O, "O");
  if ((s = check_queue(queue, queue_bytes)) != SPARSEPR_OK) return s;
  AttnArgs a{};
  a.Q = Q;
  a.K = K;
  a.V = V;
  a.scale = scale;
  a.H = d.H;
  a.N = d.N;
  a.nsplit = 1;
  a.split_len = d.N;
  a.G = 1;
  a.nb = d.nb;
  a.out = O;
  a.lse = lse;
  a.qctr = static_cast<int*>(queue);
  return hip_status(launch_attention(d, ATTN_DENSE, a, static_cast<hipStream_t>(stream)),
                    "sparsepr_dense_attention");
}

}  // extern "C"
