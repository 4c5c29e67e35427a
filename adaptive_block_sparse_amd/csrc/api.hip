// C ABI entry points: argument validation, workspace layout, launches.
#include <hip/hip_runtime.h>

#include <math.h>
#include <string.h>

#include "abs.h"
#include "internal.h"
#include "route_internal.h"

namespace abs_impl {

Geo make_geo(const abs_plan* plan) {
  Geo g;
  const abs_shape& s = plan->s;
  g.B = s.batch;
  g.H = s.heads;
  g.d = s.head_dim;
  g.T = s.grid[0];
  g.Hg = s.grid[1];
  g.W = s.grid[2];
  g.bt = s.block[0];
  g.bh = s.block[1];
  g.bw = s.block[2];
  g.nbt = plan->nblk[0];
  g.nbh = plan->nblk[1];
  g.nbw = plan->nblk[2];
  g.nb = plan->num_blocks;
  g.Bt = plan->block_tokens;
  g.N = (int)plan->tokens;
  g.rows = (int)plan->rows;
  g.words = (g.nb + 31) / 32;
  // pair along t (closest kept sets), the left-over plane along h, its
  // left-over row along w
  g.groups_per_head = groups_per_head_of(g.nbt, g.nbh, g.nbw);
  g.groups = g.B * g.H * g.groups_per_head;
  return g;
}

RouteWs route_ws_layout(const Geo& g, bool slack, bool frames) {
  RouteWs L;
  size_t off = 0;
  auto take = [&](size_t bytes) { size_t at = off; off = align256(off + bytes); return at; };
  const size_t pooled = (size_t)g.B * g.H * g.nb * g.d * sizeof(float);
  L.qp = take(pooled);
  L.kp = take(pooled);
  L.prob = take(slack ? (size_t)g.rows * g.nb * sizeof(float) : 0);
  L.bitmap = take((size_t)g.rows * g.words * sizeof(uint32_t));
  L.count = take((size_t)g.rows * sizeof(int));
  const size_t heads = (size_t)g.B * g.H;
  L.gsum = take(heads * route_groups_per_head(g.nb) * sizeof(int));
  L.kf = take(frames ? heads * g.nb * g.bt * g.d * sizeof(float) : 0);
  L.fbitmap = take(frames ? (size_t)g.rows * route_frame_words(g) * sizeof(uint32_t) : 0);
  L.fcount = take(frames ? (size_t)g.rows * sizeof(int) : 0);
  L.hist = take(slack ? heads * 2048 * sizeof(uint32_t) : 0);
  L.sel = take(slack ? heads * 4 * sizeof(int) : 0);
  L.eqcnt = take(slack ? (size_t)g.rows * sizeof(int) : 0);
  L.eqoff = take(slack ? (size_t)g.rows * sizeof(int) : 0);
  L.total = off;
  return L;
}

AttendWs attend_ws_layout(const Geo& g, int dtype, int max_parts) {
  AttendWs L;
  size_t off = 0;
  auto take = [&](size_t bytes) { size_t at = off; off = align256(off + bytes); return at; };
  const bool split = max_parts >= 0;
  const size_t queue = split ? (size_t)g.groups + (size_t)max_parts : (size_t)g.rows;
  const size_t order = queue > (size_t)g.rows ? queue : (size_t)g.rows;
  // split mode: the unit table comes first (its placement is part of the ABI)
  L.units = split ? take(queue * 4 * sizeof(int)) : 0;
  L.stab = split ? take((size_t)g.groups * 4 * sizeof(int)) : 0;
  L.sched = take(order * sizeof(int));
  L.counter = take(512 * sizeof(int));
  L.sort_a = take(order * sizeof(int));
  L.sort_b = take(order * sizeof(int));
  if (dtype == ABS_BF16) {
    L.kc = take((size_t)g.B * g.H * g.nb * g.Bt * g.d * 2);
    L.vc = take((size_t)g.B * g.H * g.nb * g.Bt * g.d * 2);
    L.tlist = take((size_t)g.groups * tlist_cap(g) * sizeof(int));
    L.tcount = take((size_t)g.groups * sizeof(int));
    L.icost = take((size_t)g.groups * sizeof(int));
    L.kn = take((size_t)g.rows * sizeof(float));
  } else {
    L.kc = take(0);
    L.vc = take((size_t)g.B * g.N * g.H * g.d * sizeof(float));
    L.tlist = take(0);
    L.tcount = take(0);
    L.icost = take(0);
    L.kn = take(0);
  }
  L.part = take(split ? (size_t)max_parts * part_floats(g) * sizeof(float) : 0);
  L.total = off;
  return L;
}

}  // namespace abs_impl

using namespace abs_impl;

static bool plan_ok(const abs_plan* plan) {
  return plan && plan->num_blocks > 0 && plan->rows > 0 && plan->block_tokens > 0 &&
         (plan->s.dtype == ABS_F32 || plan->s.dtype == ABS_BF16) && plan->heads_per_phase >= 1;
}

static bool mask_ok(const abs_mask* m) {
  return m && m->row_ptr && m->col_idx && m->head_nnz;
}

extern "C" {

const char* abs_status_string(abs_status st) {
  switch (st) {
    case ABS_OK: return "ok";
    case ABS_EINVAL: return "invalid argument";
    case ABS_ENOTSUP: return "unsupported shape or dtype";
    case ABS_ENOSPACE: return "workspace too small";
    case ABS_EHIP: return "HIP launch error";
    case ABS_ETOOBIG: return "plan too large for the static no-allocation scratch";
  }
  return "unknown status";
}

abs_status abs_plan_init(const abs_shape* shape, abs_plan* out) {
  if (!shape || !out) return ABS_EINVAL;
  const abs_shape& s = *shape;
  if (s.batch <= 0 || s.heads <= 0 || s.head_dim <= 0) return ABS_EINVAL;
  for (int a = 0; a < 3; ++a)
    if (s.grid[a] <= 0 || s.block[a] <= 0) return ABS_EINVAL;
  if (s.dtype != ABS_F32 && s.dtype != ABS_BF16) return ABS_ENOTSUP;
  if (s.head_dim != 64 && s.head_dim != 128) return ABS_ENOTSUP;
  for (int a = 0; a < 3; ++a)
    if (s.block[a] > 255 || s.grid[a] > (1 << 20)) return ABS_ENOTSUP;
  const long long bt_tokens = (long long)s.block[0] * s.block[1] * s.block[2];
  if (bt_tokens != 32 && bt_tokens != 64 && bt_tokens != 128) return ABS_ENOTSUP;
  abs_plan p;
  memset(&p, 0, sizeof(p));
  p.s = s;
  long long nb = 1;
  for (int a = 0; a < 3; ++a) {
    p.nblk[a] = (s.grid[a] + s.block[a] - 1) / s.block[a];
    p.padded[a] = p.nblk[a] * s.block[a];
    nb *= p.nblk[a];
  }
  if (nb > MAX_NB) return ABS_ENOTSUP;
  const long long tokens = (long long)s.grid[0] * s.grid[1] * s.grid[2];
  const long long rows = (long long)s.batch * s.heads * nb;
  // int32 indices: token numbers, CSR positions (rows * nb bounds nnz) and the
  // per-item key-block lists; element offsets are 64-bit
  if (rows * nb >= (1ll << 31) || tokens >= (1ll << 31)) return ABS_ENOTSUP;
  p.num_blocks = (int32_t)nb;
  p.block_tokens = (int32_t)bt_tokens;
  p.tokens = tokens;
  p.rows = rows;
  p.col_capacity = rows * nb;
  // phase width for the head-phased queue: keep the phase's K and V within
  // about 24 MB, well inside the last-level cache (at 480p, 20 MB a head, one
  // head a phase ran 0.6-1.3 % faster than two and 1 % faster than three or
  // four; at 720p, 39 MB a head, one head ran 0.8 % faster than two and 2.5 %
  // faster than four)
  const double per_head = 2.0 * (double)tokens * s.head_dim * (s.dtype == ABS_BF16 ? 2 : 4);
  long long hpp = (long long)(24.0e6 / per_head);
  if (hpp < 1) hpp = 1;
  if (hpp > (long long)s.batch * s.heads) hpp = (long long)s.batch * s.heads;
  p.heads_per_phase = (int32_t)hpp;
  Geo g = make_geo(&p);
  p.route_ws_bytes = route_ws_layout(g, true, true).total;
  p.attend_ws_bytes = attend_ws_layout(g, s.dtype).total;
  *out = p;
  return ABS_OK;
}

abs_status abs_route(const abs_plan* plan, const void* q, const void* k, float p,
                     int32_t k_floor, float slack, const abs_mask* mask, void* ws,
                     size_t ws_bytes, void* stream) {
  if (!plan_ok(plan) || !q || !k || !mask_ok(mask) || !ws) return ABS_EINVAL;
  if (!(p > 0.0f && p <= 1.0f)) return ABS_EINVAL;  // also rejects NaN
  if (k_floor < 1) return ABS_EINVAL;
  if (!(slack >= 0.0f && slack < 1.0f)) return ABS_EINVAL;
  Geo g = make_geo(plan);
  RouteWs L = route_ws_layout(g, slack > 0.0f);
  if (ws_bytes < L.total) return ABS_ENOSPACE;
  const int kf = k_floor > g.nb ? g.nb : k_floor;
  hipError_t e = launch_route(g, plan->s.dtype, q, k, p, kf, slack, mask, (char*)ws, L,
                              (hipStream_t)stream);
  return e == hipSuccess ? ABS_OK : ABS_EHIP;
}

abs_status abs_route_dynamic(const abs_plan* plan, const void* q, const void* k, float p,
                             int32_t k_floor, float theta, const int64_t* budget,
                             const abs_mask* mask, void* ws, size_t ws_bytes, void* stream) {
  if (!plan_ok(plan) || !q || !k || !budget || !mask_ok(mask) || !ws) return ABS_EINVAL;
  if (!(p > 0.0f && p <= 1.0f)) return ABS_EINVAL;
  if (k_floor < 1) return ABS_EINVAL;
  if (!(theta >= 0.0f && theta <= 1.0f)) return ABS_EINVAL;
  Geo g = make_geo(plan);
  RouteWs L = route_ws_layout(g, true);
  if (ws_bytes < L.total) return ABS_ENOSPACE;
  const int kf = k_floor > g.nb ? g.nb : k_floor;
  hipError_t e = launch_route_dynamic(g, plan->s.dtype, q, k, p, kf, theta,
                                      (const long long*)budget, mask, (char*)ws, L,
                                      (hipStream_t)stream);
  return e == hipSuccess ? ABS_OK : ABS_EHIP;
}

abs_status abs_route_frames(const abs_plan* plan, const void* q, const void* k, float p,
                            int32_t k_floor, float p_frame, const abs_mask* mask,
                            int32_t* frame_mask, void* ws, size_t ws_bytes, void* stream) {
  if (!plan_ok(plan) || !q || !k || !mask_ok(mask) || !frame_mask || !ws) return ABS_EINVAL;
  if (!(p > 0.0f && p <= 1.0f) || !(p_frame > 0.0f && p_frame <= 1.0f)) return ABS_EINVAL;
  if (k_floor < 1) return ABS_EINVAL;
  Geo g = make_geo(plan);
  if (g.bt > MAX_FRAMES || (long)g.nb * g.bt > MAX_FRAME_KEYS) return ABS_ENOTSUP;
  RouteWs L = route_ws_layout(g, false, true);
  if (ws_bytes < L.total) return ABS_ENOSPACE;
  hipError_t e = launch_route_frames(g, plan->s.dtype, q, k, p, k_floor, p_frame, mask,
                                     frame_mask, (char*)ws, L, (hipStream_t)stream);
  return e == hipSuccess ? ABS_OK : ABS_EHIP;
}

abs_status abs_attend_frames(const abs_plan* plan, const void* q, const void* k, const void* v,
                             const abs_mask* mask, const int32_t* frame_mask, void* o,
                             int32_t sched, void* ws, size_t ws_bytes, int64_t* telemetry,
                             void* stream) {
  if (!plan_ok(plan) || !q || !k || !v || !o || !mask_ok(mask) || !frame_mask || !ws)
    return ABS_EINVAL;
  if (sched < ABS_SCHED_NNZ_SORTED || sched > ABS_SCHED_XCD_LOCAL) return ABS_EINVAL;
  if (plan->s.dtype != ABS_BF16 || plan->block_tokens != 128) return ABS_ENOTSUP;
  Geo g = make_geo(plan);
  if (g.bt > MAX_FRAMES) return ABS_ENOTSUP;
  AttendWs L = attend_ws_layout(g, plan->s.dtype);
  if (ws_bytes < L.total) return ABS_ENOSPACE;
  const int grid = attend_grid(g, plan->s.dtype, sched);
  if (grid <= 0) return ABS_EHIP;
  hipStream_t s = (hipStream_t)stream;
  hipError_t e = launch_attend_relayout(g, plan->s.dtype, k, v, (char*)ws, L, s);
  if (e == hipSuccess)
    e = launch_attend_schedule(g, plan->s.dtype, mask, sched, plan->heads_per_phase, (char*)ws,
                               L, s, frame_mask);
  if (e == hipSuccess)
    e = launch_attend_run(g, plan->s.dtype, q, k, mask, o, sched, (char*)ws, L, telemetry, grid, s,
                          true);
  return e == hipSuccess ? ABS_OK : ABS_EHIP;
}

abs_status abs_slack_budget(const abs_plan* plan, int32_t sched, const int64_t* telemetry,
                            float fill, int64_t max_pairs, int64_t* budget, void* stream) {
  if (!plan_ok(plan) || !telemetry || !budget) return ABS_EINVAL;
  if (sched != ABS_SCHED_NNZ_SORTED && sched != ABS_SCHED_HEAD_PHASED &&
      sched != ABS_SCHED_XCD_LOCAL)
    return ABS_EINVAL;   // the records must come from a persistent launch
  if (!(fill >= 0.0f && fill <= 1.0f) || max_pairs < 0) return ABS_EINVAL;
  if (plan->s.dtype != ABS_BF16) return ABS_ENOTSUP;
  Geo g = make_geo(plan);
  const int n = attend_grid(g, plan->s.dtype, sched);
  if (n <= 0) return ABS_EHIP;
  hipError_t e = launch_slack_budget((const long long*)telemetry, n, fill, (long long)max_pairs,
                                     (long long*)budget, (hipStream_t)stream);
  return e == hipSuccess ? ABS_OK : ABS_EHIP;
}

abs_status abs_attend_prepare(const abs_plan* plan, const void* k, const void* v,
                              const abs_mask* mask, int32_t sched, void* ws, size_t ws_bytes,
                              void* stream) {
  if (!plan_ok(plan) || !k || !v || !mask_ok(mask) || !ws) return ABS_EINVAL;
  if (sched < ABS_SCHED_NNZ_SORTED || sched > ABS_SCHED_XCD_LOCAL) return ABS_EINVAL;
  Geo g = make_geo(plan);
  AttendWs L = attend_ws_layout(g, plan->s.dtype);
  if (ws_bytes < L.total) return ABS_ENOSPACE;
  hipError_t e = launch_attend_prepare(g, plan->s.dtype, k, v, mask, sched, plan->heads_per_phase,
                                       (char*)ws, L, (hipStream_t)stream);
  return e == hipSuccess ? ABS_OK : ABS_EHIP;
}

abs_status abs_attend_relayout(const abs_plan* plan, const void* k, const void* v, void* ws,
                               size_t ws_bytes, void* stream) {
  if (!plan_ok(plan) || !k || !v || !ws) return ABS_EINVAL;
  Geo g = make_geo(plan);
  AttendWs L = attend_ws_layout(g, plan->s.dtype);
  if (ws_bytes < L.total) return ABS_ENOSPACE;
  hipError_t e = launch_attend_relayout(g, plan->s.dtype, k, v, (char*)ws, L,
                                        (hipStream_t)stream);
  return e == hipSuccess ? ABS_OK : ABS_EHIP;
}

abs_status abs_attend_schedule(const abs_plan* plan, const abs_mask* mask, int32_t sched,
                               void* ws, size_t ws_bytes, void* stream) {
  if (!plan_ok(plan) || !mask_ok(mask) || !ws) return ABS_EINVAL;
  if (sched < ABS_SCHED_NNZ_SORTED || sched > ABS_SCHED_XCD_LOCAL) return ABS_EINVAL;
  Geo g = make_geo(plan);
  AttendWs L = attend_ws_layout(g, plan->s.dtype);
  if (ws_bytes < L.total) return ABS_ENOSPACE;
  hipError_t e = launch_attend_schedule(g, plan->s.dtype, mask, sched, plan->heads_per_phase,
                                        (char*)ws, L, (hipStream_t)stream);
  return e == hipSuccess ? ABS_OK : ABS_EHIP;
}

abs_status abs_attend_default_sched(const abs_plan* plan, int32_t* sched) {
  if (!plan_ok(plan) || !sched) return ABS_EINVAL;
  // With phases of about 48 MB of K and V (a few heads at 480p, one at 720p
  // and on the 81-frame shape), the head-phased queue measured fastest on every
  // workload: 0.5 % ahead of XCD-local at 480p, 1-2 % on the head-imbalance
  // stress, 5-6 % at 720p and on the 81-frame shape.
  *sched = ABS_SCHED_HEAD_PHASED;
  return ABS_OK;
}

abs_status abs_attend_grid(const abs_plan* plan, int32_t sched, int32_t* workgroups) {
  if (!plan_ok(plan) || !workgroups) return ABS_EINVAL;
  if (sched < ABS_SCHED_NNZ_SORTED || sched > ABS_SCHED_XCD_LOCAL) return ABS_EINVAL;
  Geo g = make_geo(plan);
  const int n = attend_grid(g, plan->s.dtype, sched);
  if (n <= 0) return ABS_EHIP;
  *workgroups = n;
  return ABS_OK;
}

abs_status abs_attend_run(const abs_plan* plan, const void* q, const void* k,
                          const abs_mask* mask, void* o, int32_t sched, void* ws,
                          size_t ws_bytes, int64_t* telemetry, void* stream) {
  if (!plan_ok(plan) || !q || !k || !o || !mask_ok(mask) || !ws) return ABS_EINVAL;
  if (sched < ABS_SCHED_NNZ_SORTED || sched > ABS_SCHED_XCD_LOCAL) return ABS_EINVAL;
  Geo g = make_geo(plan);
  AttendWs L = attend_ws_layout(g, plan->s.dtype);
  if (ws_bytes < L.total) return ABS_ENOSPACE;
  const int grid = attend_grid(g, plan->s.dtype, sched);
  if (grid <= 0) return ABS_EHIP;
  hipError_t e = launch_attend_run(g, plan->s.dtype, q, k, mask, o, sched, (char*)ws, L,
                                   telemetry, grid, (hipStream_t)stream);
  return e == hipSuccess ? ABS_OK : ABS_EHIP;
}

abs_status abs_attend(const abs_plan* plan, const void* q, const void* k, const void* v,
                      const abs_mask* mask, void* o, int32_t sched, void* ws, size_t ws_bytes,
                      int64_t* telemetry, void* stream) {
  if (!q || !k || !o) return ABS_EINVAL;
  abs_status st = abs_attend_prepare(plan, k, v, mask, sched, ws, ws_bytes, stream);
  if (st != ABS_OK) return st;
  return abs_attend_run(plan, q, k, mask, o, sched, ws, ws_bytes, telemetry, stream);
}

// split-and-merge entry points: persistent sorted queues, bf16 only
static abs_status split_args(const abs_plan* plan, int32_t sched, int32_t max_parts) {
  if (!plan_ok(plan)) return ABS_EINVAL;
  if (sched != ABS_SCHED_NNZ_SORTED && sched != ABS_SCHED_HEAD_PHASED) return ABS_EINVAL;
  if (max_parts < 0 || max_parts > MAX_SPLIT_PARTS) return ABS_EINVAL;
  if (plan->s.dtype != ABS_BF16) return ABS_ENOTSUP;
  return ABS_OK;
}

abs_status abs_attend_split_ws_bytes(const abs_plan* plan, int32_t max_parts, size_t* bytes) {
  if (!bytes) return ABS_EINVAL;
  const abs_status st = split_args(plan, ABS_SCHED_NNZ_SORTED, max_parts);
  if (st != ABS_OK) return st;
  *bytes = attend_ws_layout(make_geo(plan), plan->s.dtype, max_parts).total;
  return ABS_OK;
}

abs_status abs_attend_prepare_split(const abs_plan* plan, const void* k, const void* v,
                                    const abs_mask* mask, int32_t sched, int32_t split_tiles,
                                    int32_t max_parts, void* ws, size_t ws_bytes, void* stream) {
  if (!plan_ok(plan) || !k || !v || !mask_ok(mask) || !ws) return ABS_EINVAL;
  if (split_tiles < 1) return ABS_EINVAL;
  const abs_status st = split_args(plan, sched, max_parts);
  if (st != ABS_OK) return st;
  Geo g = make_geo(plan);
  AttendWs L = attend_ws_layout(g, plan->s.dtype, max_parts);
  if (ws_bytes < L.total) return ABS_ENOSPACE;
  hipError_t e = launch_attend_prepare_split(g, k, v, mask, sched, plan->heads_per_phase,
                                             split_tiles, max_parts, (char*)ws, L,
                                             (hipStream_t)stream);
  return e == hipSuccess ? ABS_OK : ABS_EHIP;
}

abs_status abs_attend_run_split(const abs_plan* plan, const void* q, const abs_mask* mask,
                                void* o, int32_t sched, int32_t max_parts, void* ws,
                                size_t ws_bytes, int64_t* telemetry, void* stream) {
  if (!plan_ok(plan) || !q || !o || !mask_ok(mask) || !ws) return ABS_EINVAL;
  const abs_status st = split_args(plan, sched, max_parts);
  if (st != ABS_OK) return st;
  Geo g = make_geo(plan);
  AttendWs L = attend_ws_layout(g, plan->s.dtype, max_parts);
  if (ws_bytes < L.total) return ABS_ENOSPACE;
  const int grid = attend_grid(g, plan->s.dtype, sched);
  if (grid <= 0) return ABS_EHIP;
  hipError_t e = launch_attend_run_split(g, q, mask, o, max_parts, (char*)ws, L, telemetry, grid,
                                         (hipStream_t)stream);
  return e == hipSuccess ? ABS_OK : ABS_EHIP;
}

}  // extern "C"
