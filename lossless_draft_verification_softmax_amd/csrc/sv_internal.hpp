// sv_internal.hpp -- launch parameters, per-request draw state and the
// workspace layout of libspecverify.  Used by the library's own sources only.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "specverify.h"

namespace sv {

enum DrawMode : int32_t { kDrawNone = 0, kDrawResidual = 1, kDrawBonus = 2 };

// Elements per draw tile (256 threads x 8).
constexpr int kDrawTile = 2048;
// float64 draw: uncertain-sign elements kept per tile (more: the tile is
// recomputed directly)
constexpr int kDrawKeep64 = 16;
constexpr int kMaxShards = SV_MAX_SHARDS;
// Largest grid of the team row pass, and most members per row.
constexpr int kMaxTeamGrid = 1024;
constexpr int kMaxTeam = 64;
// Team exchange: per workgroup of the team grid, four ring slots of one
// four-word record.
constexpr int kTeamXchWords = kMaxTeamGrid * 4 * 4;

// The draw of one request, as the accept phase of k_accept_draw leaves it
// for the float32 draw of the same kernel.
struct DrawState {
  int32_t mode;     // DrawMode
  int32_t tau;      // position of the emitted draw
  int64_t prow;     // target row of the draw
  int64_t qrow;     // draft row (residual draws)
  float sl;         // log2(e) / T
  float T;          // temperature
  float mp, lzp;    // target row: max and log2 of sum 2^(x sl - R(max))
  float mq, lzq;    // draft row: the same
  float zp;         // target row: sum 2^(x sl - R(max))
  float u;          // draw uniform (word 1 of the Philox block at tau)
};

// A draw queued for the float64 recompute: everything the float64 kernel
// needs, in one 64-byte entry, so that its workgroups read one entry before
// the logits.
struct DrawJob {
  int64_t prow, qrow;  // target row; draft row (residual draws, else 0)
  double invT;         // 1 / T in float64
  double rho_e;        // Zq / Zp from the float32 row states (residual draws)
  float mp, mq;        // row maxima (the float64 exponentials are taken against them)
  float u;             // draw uniform
  int32_t mode;        // kDrawResidual or kDrawBonus
  int32_t r, tau;      // request and position of the draw
  int32_t y32;         // token of the float32 draw (-1: none): its tile is prefetched
  int32_t pad;
};
static_assert(sizeof(DrawJob) == 64, "one 64-byte queue entry");

// One row-pass work item, written by the planner so that a workgroup can
// issue a unit's loads from a single 32-byte read.
struct PlanItem {
  int64_t trow;   // target row index
  int64_t drow;   // draft row index (row pairs)
  uint32_t code;  // request << 7 | position
  float T;        // temperature
  float sl;       // log2(e) / T (0 at T = 0)
  uint32_t pad;
};

struct VerifyParams {
  sv_dtype dtype;
  int32_t B, D;            // batch, D_max
  int64_t V, stride;       // vocabulary, row stride (elements)
  int32_t S1, seg1;        // row pass: partial-state slots per row, segment length
  // Slices of a draw row, as the row pass leaves them: slot s of a row pair
  // (a single row) holds the state of columns [s len, min(V, (s + 1) len)) of
  // its target row and, for a pair, the sum of min(p, q) over them.
  int32_t pair_ns, single_ns;    // slices per row pair / per single row
  int64_t pair_len, single_len;  // slice length (elements)
  int32_t team, nteams;    // team row pass: members per row, teams
  int64_t team_len;        // team row pass: slice length (elements)
  int32_t S2, seg2;        // draw: tiles per row, tile length
  uint32_t seed_lo, seed_hi, step, flags;
  const void* target;
  const void* draft;
  // Vocabulary shards (sv_verify_batch_sharded): nshard > 1 buffers, shard s
  // holding columns [s W, min(V, (s + 1) W)) of every row at row stride
  // `stride`; target / draft then hold shard 0 (null draft: no draft
  // shards) and the kernels read the shard pointers from shard_tab (target
  // shards, then draft shards), written by k_plan.
  int32_t nshard;
  int64_t shard_w;
  const void* tsh[kMaxShards];
  const void* dsh[kMaxShards];
  const int64_t* target_row0;
  const int64_t* draft_row0;
  const int32_t* tokens;
  const int32_t* depth;
  const float* temperature;
  const uint32_t* request_id;
  int32_t* accepted_len;
  int32_t* out_tokens;
  int32_t* num_out;
  float* alpha;
  sv_diag* diag;
  // acceptance statistics of the batch (sv_accept_stats outputs), each
  // optional; computed by one extra workgroup of k_draw_tile64
  float* stats_expected_len;  // [B]
  float* stats_per_depth;     // [3 D]
  float* stats_summary;       // [4]
  void* const* events;     // SV_NUM_STAGE_EVENTS hipEvent_t or null
  // workspace
  float2* part_p;    // [U][S1]  (max, sum) or (max, arg max bits) at T = 0
  float2* part_q;    // [U][S1]
  float* part_a;     // [U][S1]  partial sum min(p, q)
  float2* pair_p;    // [U]      row state of a pair's target row (the normaliser its rates used)
  float2* pair_q;    // [U]      row state of a pair's draft row
  // float64 tile partials, indexed by queue entry
  double* seg_zp64;  // [B][S2]
  double* seg_zq64;  // [B][S2]
  double* seg_w64;   // [B][S2]  float64 tile masses (first the sums D of the one-pass split)
  double* seg_a64;   // [B][S2]  float64 sums A of the one-pass split
  double* seg_t64;   // [B][S2]  float64 sums of ep over equal logit pairs
  int32_t* seg_u32;  // [B][S2]  elements of a tile whose residual sign was not certain
  double* seg_e64;   // [B][S2][kDrawKeep64][2]  their (ep, eq), in element order
  double* seg_h64;   // [B][2][kDrawTile]  exponentials of the float32 draw's tile
  int32_t* fb_count; // draws queued for the float64 recompute
  DrawJob* fb_jobs;  // [B]  the queue
  int32_t* fb_done;  // [B]  tiles of queue entry j done (zeroed by k_plan)
  PlanItem* plan_pairs;    // [B * D]        row pairs at T > 0
  PlanItem* plan_singles;  // [B * (D + 1)]  single rows
  int32_t* plan_counts;    // [2]
  uint64_t* team_xch;      // [kMaxTeamGrid * 4][4] tagged slice states exchanged in a team
  int32_t* sync_error;     // set if a team wait expired
  const void** shard_tab;  // [2 * kMaxShards] shard pointers (written by k_plan)
};

// ---- launch geometry (host) -------------------------------------------------

// Single rows (bonus rows, T = 0 rows) are cut into S1 segments so that the
// row pass has several times more items than CUs; segments hold at least
// 2048 elements.
inline void stats_geometry(int32_t B, int32_t D, int64_t V, int32_t* S1, int32_t* seg1) {
  const int64_t units = (int64_t)B * (D + 1);
  int64_t s = units > 0 ? (4096 + units - 1) / units : 1;
  int64_t by_len = V / 2048;
  if (by_len < 1) by_len = 1;
  if (s > by_len) s = by_len;
  if (s > 64) s = 64;
  if (s < 1) s = 1;
  int64_t len = (V + s - 1) / s;
  len = (len + 7) / 8 * 8;
  *S1 = (int32_t)s;
  *seg1 = (int32_t)len;
}

// Draw: tiles of kDrawTile elements.
inline void draw_geometry(int64_t V, int32_t* S2, int32_t* seg2) {
  *S2 = (int32_t)((V + kDrawTile - 1) / kDrawTile);
  *seg2 = kDrawTile;
}

inline size_t align256(size_t x) { return (x + 255) / 256 * 256; }

struct WorkspaceLayout {
  size_t part_p, part_q, part_a, pair_p, pair_q, seg_zp64, seg_zq64, seg_w64, seg_a64, seg_t64,
      seg_u32, seg_e64, seg_h64, fb_count, fb_jobs, fb_done,
      plan_pairs, plan_singles, plan_counts, team_xch, shard_tab, sync_error, total;
  int32_t slots;
};

inline WorkspaceLayout workspace_layout(int32_t B, int32_t D, int64_t V) {
  int32_t S1, seg1, S2, seg2;
  stats_geometry(B, D, V, &S1, &seg1);
  draw_geometry(V, &S2, &seg2);
  const size_t U = (size_t)B * (size_t)(D + 1);
  const size_t slots = (size_t)(S1 > kMaxTeam ? S1 : kMaxTeam);
  WorkspaceLayout L;
  L.slots = (int32_t)slots;
  size_t off = 0;
  L.part_p = off; off += align256(U * slots * sizeof(float2));
  L.part_q = off; off += align256(U * slots * sizeof(float2));
  L.part_a = off; off += align256(U * slots * sizeof(float));
  L.pair_p = off; off += align256(U * sizeof(float2));
  L.pair_q = off; off += align256(U * sizeof(float2));
  L.seg_zp64 = off; off += align256((size_t)B * S2 * sizeof(double));
  L.seg_zq64 = off; off += align256((size_t)B * S2 * sizeof(double));
  L.seg_w64 = off; off += align256((size_t)B * S2 * sizeof(double));
  L.seg_a64 = off; off += align256((size_t)B * S2 * sizeof(double));
  L.seg_t64 = off; off += align256((size_t)B * S2 * sizeof(double));
  L.seg_u32 = off; off += align256((size_t)B * S2 * sizeof(int32_t));
  L.seg_e64 = off; off += align256((size_t)B * S2 * kDrawKeep64 * 2 * sizeof(double));
  L.seg_h64 = off; off += align256((size_t)B * 2 * kDrawTile * sizeof(double));
  L.fb_count = off; off += align256(sizeof(int32_t));
  L.fb_jobs = off; off += align256((size_t)B * sizeof(DrawJob));
  L.fb_done = off; off += align256((size_t)B * sizeof(int32_t));
  L.plan_pairs = off; off += align256((size_t)B * (size_t)D * sizeof(PlanItem));
  L.plan_singles = off; off += align256(U * sizeof(PlanItem));
  L.plan_counts = off; off += align256(2 * sizeof(int32_t));
  L.team_xch = off; off += align256((size_t)kTeamXchWords * sizeof(uint64_t));
  L.shard_tab = off; off += align256(2 * kMaxShards * sizeof(void*));
  L.sync_error = off; off += align256(sizeof(int32_t));
  L.total = off;
  return L;
}

hipError_t launch_verify(VerifyParams& p, int grid, hipStream_t stream);
bool team_geometry(sv_dtype dtype, int64_t V, int grid, int32_t* T, int32_t* NV,
                   int32_t* slice_len);
hipError_t launch_rowteam(VerifyParams& p, int grid, int nv, hipStream_t stream);
void launch_plan(const VerifyParams& p, hipStream_t stream);
void launch_rowpass(const VerifyParams& p, int grid, hipStream_t stream);
void launch_draw(const VerifyParams& p, int cus, hipStream_t stream);
hipError_t launch_budget(const float* conf, int32_t B, int32_t D, const int32_t* max_depth,
                         int64_t K, int32_t* depth, int64_t* draft_row0, int64_t* target_row0,
                         float* utility, hipStream_t stream);
hipError_t launch_budget_fixed(const float* conf, int32_t B, int32_t D, int64_t K, int32_t* depth,
                               int64_t* draft_row0, int64_t* target_row0, float* utility,
                               hipStream_t stream);
hipError_t launch_accumulate(const int32_t* depth, const float* alpha, const int32_t* accepted_len,
                             int32_t B, int32_t D, double* accum, float* summary,
                             hipStream_t stream);
hipError_t launch_stats(const int32_t* depth, const float* alpha, const int32_t* accepted_len,
                        int32_t B, int32_t D, float* expected_len, float* per_depth,
                        float* summary, hipStream_t stream);

// Drafter confidence (sv_confidence.hip).
struct ConfParams {
  sv_dtype dtype;
  int32_t B, D;
  int64_t V, stride;
  const void* logits;
  const int64_t* row0;     // [B] first draft row of each request
  const int32_t* tokens;   // [B, D]
  const int32_t* depth;    // [B] or null (= D)
  const float* temperature;
  float* conf;             // [B, D]
  float2* part;            // [B * D][nseg][waves] wavefront states (workspace)
  int64_t nseg;            // segments per row
};
int64_t confidence_segments(sv_dtype dtype, int64_t V);
int64_t confidence_states(sv_dtype dtype, int64_t V);
hipError_t launch_confidence(const ConfParams& c, hipStream_t stream);

// Keep-ratio choice (sv_budget.hip): the candidate ratios and their
// latencies at this batch size.
constexpr int kMaxRatios = SV_MAX_RATIOS;
struct RatioArgs {
  int32_t n;
  double ratio[kMaxRatios];
  double latency[kMaxRatios];
};
hipError_t launch_budget_ratio(const float* conf, int32_t B, int32_t D, const int32_t* max_depth,
                               const RatioArgs& ra, int32_t* choice, int64_t* K_chosen,
                               float* projected, int32_t* depth, int64_t* draft_row0,
                               int64_t* target_row0, float* utility, hipStream_t stream);

// Token sampler (sv_sample.hip).
struct SampleParams {
  sv_dtype dtype;
  int32_t B;
  int64_t V, stride;
  const void* logits;
  int64_t row_base;
  const int32_t* row_index;  // row of request r: row_base + row_index[r * index_stride]
  int64_t index_stride;
  const float* temperature;
  const uint32_t* request_id;  // or null: r
  uint32_t seed_lo, seed_hi, step, position;
  int32_t* tokens;             // token of request r at tokens[r * token_stride]
  int64_t token_stride;
};
hipError_t launch_sample(const SampleParams& p, hipStream_t stream);

}  // namespace sv
