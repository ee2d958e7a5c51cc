// sv_api.hip -- the C ABI of libspecverify: argument validation (before any
// HIP call), workspace carving and the stream-ordered launches.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include <atomic>
#include <mutex>

#include "specverify.h"
#include "sv_internal.hpp"

// Scratch of sv_verify_batch_noalloc: one copy per device, allocated by the
// HIP runtime when the code object is loaded and held until the process
// ends.  In host code `scratch` names a host-side stand-in, not the device
// array: host code only ever uses the device address that
// hipGetSymbolAddress returns for the current device (scratch_address).
static __device__ __align__(256) unsigned char scratch[SV_NOALLOC_SCRATCH_BYTES];

namespace {

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Compute units of the current device (one persistent row-pass workgroup
// each); cached per device.
constexpr int kMaxDevices = 64;
std::atomic<int> g_cu_count[kMaxDevices];

// Device address of `scratch` on each device, resolved once per device (with
// that device current) on the first sv_verify_batch_noalloc call there.
std::mutex g_scratch_mu;
std::atomic<void*> g_scratch_ptr[kMaxDevices];

void* scratch_address() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  void* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (p) return p;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  p = g_scratch_ptr[dev].load(std::memory_order_relaxed);
  if (p) return p;
  void* q = nullptr;
  if (hipGetSymbolAddress(&q, HIP_SYMBOL(scratch)) != hipSuccess || q == nullptr) return nullptr;
  g_scratch_ptr[dev].store(q, std::memory_order_release);
  return q;
}

int device_cu_count() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return -1;
  if (dev < kMaxDevices) {
    const int cached = g_cu_count[dev].load(std::memory_order_relaxed);
    if (cached > 0) return cached;
  }
  int cus = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return -1;
  if (dev < kMaxDevices) g_cu_count[dev].store(cus, std::memory_order_relaxed);
  return cus;
}

// row_width: the elements of a row held by one buffer (V, or the shard width).
sv_status validate_verify(const sv_verify_args* a, int64_t row_width, size_t* need) {
  if (!a) return SV_ERR_INVALID_ARGUMENT;
  if (a->B < 0 || a->D_max < 0 || a->D_max > SV_MAX_DEPTH) return SV_ERR_INVALID_ARGUMENT;
  if (a->V < 1 || a->V > INT32_MAX || a->row_stride < row_width) return SV_ERR_INVALID_ARGUMENT;
  if (a->dtype != SV_DTYPE_BF16 && a->dtype != SV_DTYPE_FP32) return SV_ERR_UNSUPPORTED;
  if (a->flags & ~(SV_FLAG_FORCE_FP64_DRAW | SV_FLAG_STREAMING_ROW_PASS |
                   SV_FLAG_EXACT_FP64_MASSES | SV_FLAG_TEAM_WAIT_GIVE_UP))
    return SV_ERR_UNSUPPORTED;
  if ((int64_t)a->B * (a->D_max + 1) > (int64_t)INT32_MAX / 64) return SV_ERR_INVALID_ARGUMENT;
  // the float64 draw numbers its (queue entry, tile) items in 32 bits
  if ((int64_t)a->B * ((a->V + sv::kDrawTile - 1) / sv::kDrawTile) > (int64_t)INT32_MAX)
    return SV_ERR_INVALID_ARGUMENT;
  if (a->B == 0) {
    *need = 0;
    return SV_OK;
  }
  if (!a->target_logits || !a->target_row0 || !a->depth || !a->temperature ||
      !a->accepted_len || !a->out_tokens || !a->num_out)
    return SV_ERR_INVALID_ARGUMENT;
  if (a->D_max > 0 && !a->draft_tokens) return SV_ERR_INVALID_ARGUMENT;
  if ((a->draft_logits == nullptr) != (a->draft_row0 == nullptr)) return SV_ERR_INVALID_ARGUMENT;
  const int64_t vec = (a->dtype == SV_DTYPE_BF16) ? 8 : 4;
  if (!aligned16(a->target_logits) || (a->draft_logits && !aligned16(a->draft_logits)) ||
      a->row_stride % vec != 0)
    return SV_ERR_UNSUPPORTED;
  *need = sv::workspace_layout(a->B, a->D_max, a->V).total;
  if (!a->workspace || (reinterpret_cast<uintptr_t>(a->workspace) & 255u) != 0)
    return SV_ERR_INVALID_ARGUMENT;
  if (a->workspace_bytes < *need) return SV_ERR_WORKSPACE_TOO_SMALL;
  return SV_OK;
}

}  // namespace

extern "C" {

const char* sv_status_string(sv_status status) {
  switch (status) {
    case SV_OK: return "ok";
    case SV_ERR_INVALID_ARGUMENT: return "invalid argument";
    case SV_ERR_UNSUPPORTED: return "unsupported layout, dtype or flag";
    case SV_ERR_WORKSPACE_TOO_SMALL: return "workspace too small";
    case SV_ERR_DEVICE: return "device launch failed";
    case SV_ERR_SCRATCH_TOO_SMALL:
      return "batch needs more scratch than the no-allocation entry point holds";
  }
  return "unknown status";
}

const char* sv_version(void) { return "specverify 0.1.0 gfx950"; }

int64_t sv_k_rho(int32_t B, int32_t D, double rho) {
  if (B < 0 || D < 0 || !(rho >= 0.0 && rho <= 1.0)) return -1;
  const double k = ceil(rho * (double)B * (double)(D + 1));
  const int64_t kk = (int64_t)k;
  return kk > B ? kk : (int64_t)B;
}

size_t sv_verify_workspace_bytes(int32_t B, int32_t D_max, int64_t V) {
  if (B < 0 || D_max < 0 || D_max > SV_MAX_DEPTH || V < 1 || V > INT32_MAX) return 0;
  return sv::workspace_layout(B, D_max, V).total;
}

}  // extern "C"

namespace {

sv_status run_verify(const sv_verify_args* a, int32_t nshard, int64_t shard_w,
                     const void* const* tsh, const void* const* dsh, void* stream) {
  sv::VerifyParams p{};
  p.nshard = nshard;
  p.shard_w = shard_w;
  for (int32_t s = 0; s < nshard && nshard > 1; ++s) {
    p.tsh[s] = tsh[s];
    p.dsh[s] = dsh ? dsh[s] : nullptr;
  }
  p.dtype = a->dtype;
  p.B = a->B;
  p.D = a->D_max;
  p.V = a->V;
  p.stride = a->row_stride;
  sv::stats_geometry(p.B, p.D, p.V, &p.S1, &p.seg1);
  sv::draw_geometry(p.V, &p.S2, &p.seg2);
  p.seed_lo = (uint32_t)(a->seed & 0xffffffffull);
  p.seed_hi = (uint32_t)(a->seed >> 32);
  p.step = a->step;
  p.flags = a->flags;
  p.target = a->target_logits;
  p.draft = a->draft_logits;
  p.target_row0 = a->target_row0;
  p.draft_row0 = a->draft_row0;
  p.tokens = a->draft_tokens;
  p.depth = a->depth;
  p.temperature = a->temperature;
  p.request_id = a->request_id;
  p.accepted_len = a->accepted_len;
  p.out_tokens = a->out_tokens;
  p.num_out = a->num_out;
  p.alpha = a->alpha;
  p.diag = a->diag;
  p.stats_expected_len = a->stats_expected_len;
  p.stats_per_depth = a->stats_per_depth;
  p.stats_summary = a->stats_summary;
  p.events = a->stage_events;
  const sv::WorkspaceLayout L = sv::workspace_layout(p.B, p.D, p.V);
  char* ws = static_cast<char*>(a->workspace);
  p.part_p = reinterpret_cast<float2*>(ws + L.part_p);
  p.part_q = reinterpret_cast<float2*>(ws + L.part_q);
  p.part_a = reinterpret_cast<float*>(ws + L.part_a);
  p.pair_p = reinterpret_cast<float2*>(ws + L.pair_p);
  p.pair_q = reinterpret_cast<float2*>(ws + L.pair_q);
  p.seg_zp64 = reinterpret_cast<double*>(ws + L.seg_zp64);
  p.seg_zq64 = reinterpret_cast<double*>(ws + L.seg_zq64);
  p.seg_w64 = reinterpret_cast<double*>(ws + L.seg_w64);
  p.seg_a64 = reinterpret_cast<double*>(ws + L.seg_a64);
  p.seg_t64 = reinterpret_cast<double*>(ws + L.seg_t64);
  p.seg_u32 = reinterpret_cast<int32_t*>(ws + L.seg_u32);
  p.seg_e64 = reinterpret_cast<double*>(ws + L.seg_e64);
  p.seg_h64 = reinterpret_cast<double*>(ws + L.seg_h64);
  p.fb_count = reinterpret_cast<int32_t*>(ws + L.fb_count);
  p.fb_jobs = reinterpret_cast<sv::DrawJob*>(ws + L.fb_jobs);
  p.fb_done = reinterpret_cast<int32_t*>(ws + L.fb_done);
  p.plan_pairs = reinterpret_cast<sv::PlanItem*>(ws + L.plan_pairs);
  p.plan_singles = reinterpret_cast<sv::PlanItem*>(ws + L.plan_singles);
  p.plan_counts = reinterpret_cast<int32_t*>(ws + L.plan_counts);
  p.team_xch = reinterpret_cast<uint64_t*>(ws + L.team_xch);
  p.sync_error = reinterpret_cast<int32_t*>(ws + L.sync_error);
  p.shard_tab = reinterpret_cast<const void**>(ws + L.shard_tab);
  const int grid = device_cu_count();
  if (grid <= 0) return SV_ERR_DEVICE;
  if (nshard > 1) {  // the sharded path has no streaming fallback
    int32_t T, nv, slice;
    if (grid > sv::kMaxTeamGrid || !sv::team_geometry(p.dtype, p.V, grid, &T, &nv, &slice))
      return SV_ERR_UNSUPPORTED;
  }
  const hipError_t e = sv::launch_verify(p, grid, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? SV_OK : SV_ERR_DEVICE;
}

}  // namespace

extern "C" {

sv_status sv_verify_batch(const sv_verify_args* a, void* stream) {
  size_t need = 0;
  const sv_status st = validate_verify(a, a ? a->V : 0, &need);
  if (st != SV_OK) return st;
  if (a->B == 0) return SV_OK;
  return run_verify(a, 1, a->V, nullptr, nullptr, stream);
}

sv_status sv_verify_batch_noalloc(const sv_verify_args* a, void* stream) {
  if (!a) return SV_ERR_INVALID_ARGUMENT;
  // Size check first, on the host, before the device is touched.
  const size_t need = sv_verify_workspace_bytes(a->B, a->D_max, a->V);
  if (need > (size_t)SV_NOALLOC_SCRATCH_BYTES) return SV_ERR_SCRATCH_TOO_SMALL;
  sv_verify_args b = *a;
  b.workspace = nullptr;
  b.workspace_bytes = 0;
  if (b.B > 0) {
    void* ptr = scratch_address();
    if (!ptr) return SV_ERR_DEVICE;
    b.workspace = ptr;
    b.workspace_bytes = SV_NOALLOC_SCRATCH_BYTES;
  }
  size_t need2 = 0;
  const sv_status st = validate_verify(&b, b.V, &need2);
  if (st != SV_OK) return st;
  if (b.B == 0) return SV_OK;
  return run_verify(&b, 1, b.V, nullptr, nullptr, stream);
}

sv_status sv_verify_batch_sharded(const sv_verify_args* a, int32_t n_shards, int64_t shard_width,
                                  const void* const* target_shards,
                                  const void* const* draft_shards, void* stream) {
  if (!a || !target_shards || n_shards < 1 || n_shards > SV_MAX_SHARDS)
    return SV_ERR_INVALID_ARGUMENT;
  if (shard_width < 8 || shard_width % 8 != 0) return SV_ERR_UNSUPPORTED;
  if (a->V < 1 || (a->V + shard_width - 1) / shard_width != n_shards)
    return SV_ERR_INVALID_ARGUMENT;
  for (int32_t s = 0; s < n_shards; ++s) {
    if (!target_shards[s] || !aligned16(target_shards[s])) return SV_ERR_INVALID_ARGUMENT;
    if (draft_shards && (!draft_shards[s] || !aligned16(draft_shards[s])))
      return SV_ERR_INVALID_ARGUMENT;
  }
  sv_verify_args b = *a;
  b.target_logits = target_shards[0];
  b.draft_logits = draft_shards ? draft_shards[0] : nullptr;
  if ((b.draft_logits == nullptr) != (b.draft_row0 == nullptr)) return SV_ERR_INVALID_ARGUMENT;
  size_t need = 0;
  const sv_status st = validate_verify(&b, n_shards > 1 ? shard_width : a->V, &need);
  if (st != SV_OK) return st;
  if (b.B == 0) return SV_OK;
  if (n_shards == 1) return run_verify(&b, 1, b.V, nullptr, nullptr, stream);
  return run_verify(&b, n_shards, shard_width, target_shards, draft_shards, stream);
}

sv_status sv_allocate_budget(const float* conf, int32_t B, int32_t D_max,
                             const int32_t* max_depth, int64_t K, int32_t* depth,
                             int64_t* draft_row0, int64_t* target_row0, float* utility,
                             void* stream) {
  if (B < 0 || D_max < 0) return SV_ERR_INVALID_ARGUMENT;
  if (B > SV_MAX_BUDGET_POSITIONS || (int64_t)B * D_max > SV_MAX_BUDGET_POSITIONS)
    return SV_ERR_INVALID_ARGUMENT;
  if (B == 0) return SV_OK;
  if (!depth || (D_max > 0 && !conf)) return SV_ERR_INVALID_ARGUMENT;
  const hipError_t e = sv::launch_budget(conf, B, D_max, max_depth, K, depth, draft_row0,
                                         target_row0, utility, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? SV_OK : SV_ERR_DEVICE;
}

sv_status sv_allocate_fixed_depth(const float* conf, int32_t B, int32_t D_max, int64_t K,
                                  int32_t* depth, int64_t* draft_row0, int64_t* target_row0,
                                  float* utility, void* stream) {
  if (B < 0 || D_max < 0) return SV_ERR_INVALID_ARGUMENT;
  if (B > SV_MAX_BUDGET_POSITIONS || (int64_t)B * D_max > SV_MAX_BUDGET_POSITIONS)
    return SV_ERR_INVALID_ARGUMENT;
  if (B == 0) return SV_OK;
  if (!depth || (D_max > 0 && !conf)) return SV_ERR_INVALID_ARGUMENT;
  const hipError_t e = sv::launch_budget_fixed(conf, B, D_max, K, depth, draft_row0, target_row0,
                                               utility, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? SV_OK : SV_ERR_DEVICE;
}

size_t sv_draft_confidence_workspace_bytes(sv_dtype dtype, int32_t B, int32_t D_max, int64_t V) {
  if (B < 0 || D_max < 0 || V < 1 || V > INT32_MAX) return 0;
  if (dtype != SV_DTYPE_BF16 && dtype != SV_DTYPE_FP32) return 0;
  const int64_t rows = (int64_t)B * D_max;
  const int64_t nstate = sv::confidence_states(dtype, V);  // per row
  if (rows * nstate > (int64_t)INT32_MAX) return 0;
  const size_t bytes = (size_t)rows * (size_t)nstate * sizeof(float2);
  return bytes == 0 ? 256 : (bytes + 255) / 256 * 256;
}

sv_status sv_draft_confidence(sv_dtype dtype, int32_t B, int32_t D_max, int64_t V,
                              int64_t row_stride, const void* draft_logits,
                              const int64_t* draft_row0, const int32_t* draft_tokens,
                              const int32_t* depth, const float* temperature, float* conf,
                              void* workspace, size_t workspace_bytes, void* stream) {
  if (dtype != SV_DTYPE_BF16 && dtype != SV_DTYPE_FP32) return SV_ERR_UNSUPPORTED;
  if (B < 0 || D_max < 0 || V < 1 || V > INT32_MAX || row_stride < V)
    return SV_ERR_INVALID_ARGUMENT;
  const size_t need = sv_draft_confidence_workspace_bytes(dtype, B, D_max, V);
  if (need == 0) return SV_ERR_INVALID_ARGUMENT;
  if ((int64_t)B * D_max == 0) return SV_OK;
  if (!draft_logits || !draft_row0 || !draft_tokens || !temperature || !conf)
    return SV_ERR_INVALID_ARGUMENT;
  const int64_t vec = (dtype == SV_DTYPE_BF16) ? 8 : 4;
  if (!aligned16(draft_logits) || row_stride % vec != 0) return SV_ERR_UNSUPPORTED;
  if (!workspace || (reinterpret_cast<uintptr_t>(workspace) & 255u) != 0)
    return SV_ERR_INVALID_ARGUMENT;
  if (workspace_bytes < need) return SV_ERR_WORKSPACE_TOO_SMALL;
  sv::ConfParams c{};
  c.dtype = dtype;
  c.B = B;
  c.D = D_max;
  c.V = V;
  c.stride = row_stride;
  c.logits = draft_logits;
  c.row0 = draft_row0;
  c.tokens = draft_tokens;
  c.depth = depth;
  c.temperature = temperature;
  c.conf = conf;
  c.part = static_cast<float2*>(workspace);
  c.nseg = sv::confidence_segments(dtype, V);
  const hipError_t e = sv::launch_confidence(c, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? SV_OK : SV_ERR_DEVICE;
}

sv_status sv_select_budget_ratio(const float* conf, int32_t B, int32_t D_max,
                                 const int32_t* max_depth, int32_t n_ratios,
                                 const double* ratios, int32_t n_batch,
                                 const int32_t* table_batch, const float* table_latency,
                                 int32_t* choice, int64_t* K_chosen, float* projected,
                                 int32_t* depth, int64_t* draft_row0, int64_t* target_row0,
                                 float* utility, void* stream) {
  if (B < 0 || D_max < 0) return SV_ERR_INVALID_ARGUMENT;
  if (B > SV_MAX_BUDGET_POSITIONS || (int64_t)B * D_max > SV_MAX_BUDGET_POSITIONS)
    return SV_ERR_INVALID_ARGUMENT;
  if (n_ratios < 1 || n_ratios > SV_MAX_RATIOS || !ratios) return SV_ERR_INVALID_ARGUMENT;
  if (n_batch < 1 || !table_batch || !table_latency) return SV_ERR_INVALID_ARGUMENT;
  for (int32_t j = 0; j < n_ratios; ++j)
    if (!(ratios[j] >= 0.0 && ratios[j] <= 1.0)) return SV_ERR_INVALID_ARGUMENT;
  for (int32_t i = 0; i < n_batch; ++i) {
    if (i > 0 && !(table_batch[i] > table_batch[i - 1])) return SV_ERR_INVALID_ARGUMENT;
    for (int32_t j = 0; j < n_ratios; ++j) {
      const float l = table_latency[(int64_t)i * n_ratios + j];
      if (!(l > 0.0f && l < INFINITY)) return SV_ERR_INVALID_ARGUMENT;
    }
  }
  if (!choice || !K_chosen || !depth || (B > 0 && D_max > 0 && !conf))
    return SV_ERR_INVALID_ARGUMENT;
  if (B == 0) return SV_OK;
  // Latency of each ratio at this batch size: linear in the batch size
  // between the two nearest profiled sizes, clamped at the table's ends.
  sv::RatioArgs ra{};
  ra.n = n_ratios;
  int32_t lo = 0;
  while (lo + 1 < n_batch && table_batch[lo + 1] < B) ++lo;
  for (int32_t j = 0; j < n_ratios; ++j) {
    ra.ratio[j] = ratios[j];
    const double a = table_latency[(int64_t)lo * n_ratios + j];
    if (B <= table_batch[0]) {
      ra.latency[j] = (double)table_latency[j];
    } else if (B >= table_batch[n_batch - 1]) {
      ra.latency[j] = (double)table_latency[(int64_t)(n_batch - 1) * n_ratios + j];
    } else {
      const double b = table_latency[(int64_t)(lo + 1) * n_ratios + j];
      const double f = (double)(B - table_batch[lo]) / (double)(table_batch[lo + 1] - table_batch[lo]);
      ra.latency[j] = a + (b - a) * f;
    }
  }
  const hipError_t e = sv::launch_budget_ratio(conf, B, D_max, max_depth, ra, choice, K_chosen,
                                               projected, depth, draft_row0, target_row0, utility,
                                               static_cast<hipStream_t>(stream));
  return e == hipSuccess ? SV_OK : SV_ERR_DEVICE;
}

sv_status sv_sample_rows(sv_dtype dtype, int32_t B, int64_t V, int64_t row_stride,
                         const void* logits, int64_t row_base, const int32_t* row_index,
                         int64_t index_stride, const float* temperature,
                         const uint32_t* request_id, uint64_t seed, uint32_t step,
                         uint32_t position, int32_t* tokens, int64_t token_stride, void* stream) {
  if (dtype != SV_DTYPE_BF16 && dtype != SV_DTYPE_FP32) return SV_ERR_UNSUPPORTED;
  if (B < 0 || V < 1 || V > INT32_MAX || row_stride < V || row_base < 0 || index_stride < 0 ||
      token_stride < 1)
    return SV_ERR_INVALID_ARGUMENT;
  if (B == 0) return SV_OK;
  if (!logits || !row_index || !temperature || !tokens) return SV_ERR_INVALID_ARGUMENT;
  sv::SampleParams p{};
  p.dtype = dtype;
  p.B = B;
  p.V = V;
  p.stride = row_stride;
  p.logits = logits;
  p.row_base = row_base;
  p.row_index = row_index;
  p.index_stride = index_stride;
  p.temperature = temperature;
  p.request_id = request_id;
  p.seed_lo = (uint32_t)(seed & 0xffffffffull);
  p.seed_hi = (uint32_t)(seed >> 32);
  p.step = step;
  p.position = position;
  p.tokens = tokens;
  p.token_stride = token_stride;
  const hipError_t e = sv::launch_sample(p, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? SV_OK : SV_ERR_DEVICE;
}

sv_status sv_accept_stats(const int32_t* depth, const float* alpha, const int32_t* accepted_len,
                          int32_t B, int32_t D_max, float* expected_len, float* per_depth,
                          float* summary, void* stream) {
  if (B < 0 || D_max < 0 || D_max > SV_MAX_DEPTH) return SV_ERR_INVALID_ARGUMENT;
  if (B == 0) return SV_OK;
  if (!depth || !accepted_len) return SV_ERR_INVALID_ARGUMENT;
  const hipError_t e = sv::launch_stats(depth, alpha, accepted_len, B, D_max, expected_len,
                                        per_depth, summary, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? SV_OK : SV_ERR_DEVICE;
}

sv_status sv_accept_stats_accumulate(const int32_t* depth, const float* alpha,
                                     const int32_t* accepted_len, int32_t B, int32_t D_max,
                                     double* accum, float* summary, void* stream) {
  if (B < 0 || D_max < 0 || D_max > SV_MAX_DEPTH || !accum) return SV_ERR_INVALID_ARGUMENT;
  if (B > 0 && (!depth || !accepted_len)) return SV_ERR_INVALID_ARGUMENT;
  const hipError_t e = sv::launch_accumulate(depth, alpha, accepted_len, B, D_max, accum, summary,
                                             static_cast<hipStream_t>(stream));
  return e == hipSuccess ? SV_OK : SV_ERR_DEVICE;
}

}  // extern "C"
