// Internal declarations shared by the library's translation units.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "abs.h"

namespace abs_impl {

// Block geometry passed by value to every kernel.
struct Geo {
  int B, H, d;
  int T, Hg, W;        // real latent grid
  int bt, bh, bw;      // block dims
  int nbt, nbh, nbw;   // blocks per axis
  int nb, Bt;          // blocks per head, tokens per block
  int N;               // tokens
  int rows;            // B*H*nb
  int words;           // 32-bit words of one row bitmap, ceil(nb/32)
  // Attention work items pair two query blocks that are neighbours (they keep
  // most of the same key blocks, so one K/V tile copy serves both): along t,
  // then in a left-over last t-plane along h, then in a left-over last h-row of
  // that plane along w; a block left over after that stands alone.
  int groups_per_head; // work items per head
  int groups;          // B*H*groups_per_head
};

// Work items of one head, in this order:
//   (nbt/2) * nbh * nbw  t-pairs    (2tp, h, w) + (2tp+1, h, w);
//   if nbt is odd, in plane t = nbt-1:
//     (nbh/2) * nbw      h-pairs    (t, 2hp, w) + (t, 2hp+1, w);
//     if nbh is odd, in row h = nbh-1:
//       nbw/2            w-pairs    (t, h, 2wp) + (t, h, 2wp+1);
//       if nbw is odd    the block  (t, h, nbw-1) alone.
__host__ __device__ inline int groups_per_head_of(int nbt, int nbh, int nbw) {
  return (nbt / 2) * nbh * nbw +
         (nbt % 2) * ((nbh / 2) * nbw + (nbh % 2) * (nbw / 2 + nbw % 2));
}

// Leader block and partner (or -1) of work item gl of a head (order above).
__host__ __device__ inline void group_blocks(const Geo& g, int gl, int* lead, int* partner) {
  const int plane = g.nbh * g.nbw;
  const int n_t = (g.nbt / 2) * plane;
  if (gl < n_t) {
    const int tp = gl / plane;
    *lead = gl + tp * plane;          // (2tp) * plane + (gl % plane)
    *partner = *lead + plane;
    return;
  }
  gl -= n_t;
  int base = (g.nbt - 1) * plane;     // the last t-plane (nbt odd)
  const int n_h = (g.nbh / 2) * g.nbw;
  if (gl < n_h) {
    const int hp = gl / g.nbw, wb = gl % g.nbw;
    *lead = base + 2 * hp * g.nbw + wb;
    *partner = *lead + g.nbw;
    return;
  }
  gl -= n_h;
  base += (g.nbh - 1) * g.nbw;        // its last h-row (nbh odd)
  if (gl < g.nbw / 2) {
    *lead = base + 2 * gl;
    *partner = *lead + 1;
    return;
  }
  *lead = base + g.nbw - 1;           // nbw odd: the last block alone
  *partner = -1;
}

// Attend workspace layout.
struct AttendWs {
  size_t sched;           // int32 [rows], or [groups + max_parts] work units when split
  size_t counter;         // int32 [512]: [0] queue head; [32..40] XCD queue offsets;
                          // [64 + 32x] head of XCD queue x (own cache line each)
  size_t sort_a, sort_b;  // int32, as sched, radix-sort ping-pong
  size_t kc, vc;          // bf16: chunk-major K and V block tiles [B*H*nb*Bt*d] each;
                          // float32: vc holds a token-major copy of V, kc is empty
  size_t tlist, tcount;   // bf16: per work item, the union of its rows' kept key
                          // blocks with owners, int32 [groups * 2 nb], and the count [groups]
  size_t icost;           // bf16: per work item, the kept-block count of its rows [groups]
  size_t kn;              // bf16: per key block, the largest norm of its keys, float [B*H*nb]
  // split-and-merge mode only (sizes 0 otherwise):
  size_t units;           // int4 [groups + max_parts]: {item, t0, t1, slot or -1}
  size_t stab;            // int4 [groups]: per split item {item, first slot, parts, 0}
  size_t part;            // float32 slots [max_parts]: partial O^T [2][Bt][d], m [2][Bt],
                          // l [2][Bt] (see part_floats)
  size_t total;
};

Geo make_geo(const abs_plan* plan);
// max_parts < 0: the plain layout; >= 0: with the split-and-merge buffers
AttendWs attend_ws_layout(const Geo& g, int dtype, int max_parts = -1);

// Launchers (return hipSuccess or the launch error).
hipError_t launch_attend_relayout(const Geo& g, int dtype, const void* k, const void* v,
                                  char* ws, const AttendWs& L, hipStream_t s);
hipError_t launch_attend_schedule(const Geo& g, int dtype, const abs_mask* mask, int sched,
                                  int heads_per_phase, char* ws, const AttendWs& L,
                                  hipStream_t s, const int* frame_mask = nullptr);
hipError_t launch_attend_prepare(const Geo& g, int dtype, const void* k, const void* v,
                                 const abs_mask* mask,
                                 int sched, int heads_per_phase, char* ws, const AttendWs& L,
                                 hipStream_t s);
hipError_t launch_attend_run(const Geo& g, int dtype, const void* q, const void* k,
                             const abs_mask* mask, void* o, int sched, char* ws,
                             const AttendWs& L, int64_t* telemetry, int grid, hipStream_t s,
                             bool frames = false);
// Split-and-merge variants (bf16): heavy work items cut into parts along their
// union tile lists, partial results merged by log-sum-exp weights.
hipError_t launch_attend_prepare_split(const Geo& g, const void* k, const void* v,
                                       const abs_mask* mask, int sched, int heads_per_phase,
                                       int split_tiles, int max_parts, char* ws,
                                       const AttendWs& L, hipStream_t s);
hipError_t launch_attend_run_split(const Geo& g, const void* q, const abs_mask* mask, void* o,
                                   int max_parts, char* ws, const AttendWs& L,
                                   int64_t* telemetry, int grid, hipStream_t s);
int attend_grid(const Geo& g, int dtype, int sched);

inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

constexpr int NXCD = 8;          // XCDs (L2 domains) of an MI355X
constexpr int QOFF = 32;         // counter[QOFF + x]: start of XCD queue x (x = 0..NXCD)
constexpr int QHEAD = 64;        // counter[QHEAD + 32 x]: pull counter of XCD queue x
constexpr int MAX_LPT_HEADS = 1024;
constexpr int NUNITS = 48;       // counter[NUNITS]: work units of the split-and-merge queue
constexpr int NSPLIT = 49;       // counter[NSPLIT]: items cut into two or more parts
constexpr int MAX_SPLIT_PARTS = 1 << 24;   // bound on max_parts (slot indices stay int32)
constexpr int MAX_NB = 8192;     // key blocks per head supported by the plan
constexpr int MAX_FRAMES = 6;    // fine-grained routing: frames per block (block[0])
constexpr int MAX_FRAME_KEYS = 1024;   // fine-grained routing: frames per head (nb * bt)
inline int tlist_cap(const Geo& g) { return 2 * g.nb; }   // union entries per item
// floats of one partial-result slot: O^T for the item's two query blocks, then
// the reference maximum (exp2 domain) and the sum of each query
inline size_t part_floats(const Geo& g) { return (size_t)2 * g.Bt * g.d + 4 * (size_t)g.Bt; }

}  // namespace abs_impl
