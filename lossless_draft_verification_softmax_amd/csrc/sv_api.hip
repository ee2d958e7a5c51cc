// sv_api.hip -- the C ABI of libspecverify: argument validation (before any
// HIP call), workspace carving and the stream-ordered launches.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include <atomic>

#include "specverify.h"
#include "sv_internal.hpp"

namespace {

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Compute units of the current device (one persistent row-pass workgroup
// each); cached per device.
constexpr int kMaxDevices = 64;
std::atomic<int> g_cu_count[kMaxDevices];

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

sv_status validate_verify(const sv_verify_args* a, size_t* need) {
  if (!a) return SV_ERR_INVALID_ARGUMENT;
  if (a->B < 0 || a->D_max < 0 || a->D_max > SV_MAX_DEPTH) return SV_ERR_INVALID_ARGUMENT;
  if (a->V < 1 || a->V > INT32_MAX || a->row_stride < a->V) return SV_ERR_INVALID_ARGUMENT;
  if (a->dtype != SV_DTYPE_BF16 && a->dtype != SV_DTYPE_FP32) return SV_ERR_UNSUPPORTED;
  if (a->flags & ~(SV_FLAG_FORCE_FP64_DRAW | SV_FLAG_STREAMING_ROW_PASS | SV_FLAG_EXACT_FP64_MASSES))
    return SV_ERR_UNSUPPORTED;
  if ((int64_t)a->B * (a->D_max + 1) > (int64_t)INT32_MAX / 64) return SV_ERR_INVALID_ARGUMENT;
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

sv_status sv_verify_batch(const sv_verify_args* a, void* stream) {
  size_t need = 0;
  const sv_status st = validate_verify(a, &need);
  if (st != SV_OK) return st;
  if (a->B == 0) return SV_OK;
  sv::VerifyParams p{};
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
  p.events = a->stage_events;
  const sv::WorkspaceLayout L = sv::workspace_layout(p.B, p.D, p.V);
  char* ws = static_cast<char*>(a->workspace);
  p.part_p = reinterpret_cast<float2*>(ws + L.part_p);
  p.part_q = reinterpret_cast<float2*>(ws + L.part_q);
  p.part_a = reinterpret_cast<float*>(ws + L.part_a);
  p.req = reinterpret_cast<sv::DrawState*>(ws + L.req);
  p.seg_w32 = reinterpret_cast<float*>(ws + L.seg_w32);
  p.seg_zp64 = reinterpret_cast<double*>(ws + L.seg_zp64);
  p.seg_zq64 = reinterpret_cast<double*>(ws + L.seg_zq64);
  p.seg_w64 = reinterpret_cast<double*>(ws + L.seg_w64);
  p.seg_a64 = reinterpret_cast<double*>(ws + L.seg_a64);
  p.seg_t64 = reinterpret_cast<double*>(ws + L.seg_t64);
  p.seg_u32 = reinterpret_cast<int32_t*>(ws + L.seg_u32);
  p.seg_e64 = reinterpret_cast<double*>(ws + L.seg_e64);
  p.fb_count = reinterpret_cast<int32_t*>(ws + L.fb_count);
  p.fb_list = reinterpret_cast<int32_t*>(ws + L.fb_list);
  p.plan_pairs = reinterpret_cast<sv::PlanItem*>(ws + L.plan_pairs);
  p.plan_singles = reinterpret_cast<sv::PlanItem*>(ws + L.plan_singles);
  p.plan_counts = reinterpret_cast<int32_t*>(ws + L.plan_counts);
  p.team_xch = reinterpret_cast<uint64_t*>(ws + L.team_xch);
  p.sync_error = reinterpret_cast<int32_t*>(ws + L.sync_error);
  const int grid = device_cu_count();
  if (grid <= 0) return SV_ERR_DEVICE;
  const hipError_t e = sv::launch_verify(p, grid, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? SV_OK : SV_ERR_DEVICE;
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

}  // extern "C"
