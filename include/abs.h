/*
 * abs.h - C ABI of the adaptive block-sparse video attention library (MI355X,
 * gfx950).  Plain pointers and sizes only; every device pointer is memory the
 * caller owns (for instance torch tensors); the library never allocates, frees
 * or synchronises, and launches all work asynchronously on the given stream.
 *
 * The method is the one described by the FVAttn explainer ("FVAttn: adaptive
 * sparse attention with runtime load balancing, for video generation", an
 * explainer of arXiv 2607.16190), section "Core method":
 *   part 1, sparse-routing frontend: 3D video blocks, per-head Top-p routing
 *           over a cheap approximate similarity, a Top-k safety floor, and a
 *           repair of holes in the materialised mask;
 *   part 2, runtime load balancing: measure each head's mask size before the
 *           kernel runs and give the heaviest work out first (here: across the
 *           compute units of one GPU instead of across ranks);
 *   part 3, slack-aware augmentation: fill spare capacity with the highest
 *           scoring blocks (here: a fixed per-head block budget, or a budget
 *           derived on the device from the idle time a persistent launch
 *           measured, abs_slack_budget / abs_route_dynamic).
 * Heavy work items can also be cut into parts whose partial softmax results
 * are merged by log-sum-exp (abs_attend_*_split), the merge the APB-V paper
 * notes use across hosts.
 *
 * Tensor layout.  q, k, v and o are contiguous [B, N, H, d] with the N = T*H*W
 * latent tokens in row-major (t, h, w) order, the layout a DiT's QKV projection
 * emits.  Element type is float32 (ABS_F32) or bfloat16 (ABS_BF16); o has the
 * type of q.  The softmax scale is 1/sqrt(d).
 *
 * Blocks.  Each axis of the latent grid is padded up to a whole number of
 * (bt, bh, bw) blocks.  Block index ((t/bt)*nbh + h/bh)*nbw + w/bw and slot
 * ((t%bt)*bh + h%bh)*bw + w%bw are row-major at both levels; query and key
 * blocks share this blocking.  Padding tokens do not exist: they are excluded
 * from the pooled means, masked as keys and produce no output.  (Inside the
 * attention workspace a cut block's tile stores its real tokens first; that
 * order is internal and changes nothing above.)
 *
 * Errors.  Every entry point validates its arguments on the host before any
 * launch and returns ABS_EINVAL / ABS_ENOTSUP / ABS_ENOSPACE without touching
 * the device.  ABS_EHIP reports a launch error from the HIP runtime.  Nothing
 * throws across this interface.  Calls on distinct streams with distinct
 * workspaces are independent (the library holds no mutable global state apart
 * from a per-device cache of the compute-unit count and occupancy).
 */
#ifndef ABS_H
#define ABS_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  ABS_OK = 0,
  ABS_EINVAL = 1,   /* null pointer, non-positive size, p outside (0,1], ... */
  ABS_ENOTSUP = 2,  /* head_dim, block size, dtype or size outside the built kernels */
  ABS_ENOSPACE = 3, /* workspace smaller than the plan requires */
  ABS_EHIP = 4,     /* HIP launch error */
  ABS_ETOOBIG = 5   /* the plan needs more than the static scratch of abs_route_noalloc */
} abs_status;

typedef enum { ABS_F32 = 0, ABS_BF16 = 1 } abs_dtype;

/* Order in which (batch, head, query-block) items are processed by attend.
 *   NNZ_SORTED : persistent workgroups pull work items from one queue sorted
 *                by kept-block count, largest first, ties by item index
 *                (load balancing of the explainer's "Core method" part 2,
 *                recast over compute units);
 *   HEAD_MAJOR : one workgroup per work item in natural order, scheduled
 *                by the hardware dispatcher (the unbalanced baseline);
 *   HEAD_PHASED: persistent queue; heads are taken in phases of a few heads
 *                (so their K/V stay cache resident), largest items first
 *                inside a phase, ties by item index.
 *   XCD_LOCAL  : heads are placed on the GPU's 8 XCDs (longest head first onto
 *                the least loaded XCD); each XCD has its own queue of its
 *                heads' work items in natural (spatial) order, so neighbouring
 *                items that share key blocks run together under one L2; a
 *                workgroup pops from the queue of the XCD it runs on (read from
 *                the hardware XCC id) and steals from the others once that
 *                queue is empty.
 * All of them give bitwise identical outputs: every row has one owner and a
 * fixed key-block order. */
typedef enum {
  ABS_SCHED_NNZ_SORTED = 0,
  ABS_SCHED_HEAD_MAJOR = 1,
  ABS_SCHED_HEAD_PHASED = 2,
  ABS_SCHED_XCD_LOCAL = 3
} abs_sched;

typedef struct {
  int32_t batch, heads, head_dim;
  int32_t grid[3];  /* T, H, W latent grid */
  int32_t block[3]; /* bt, bh, bw */
  int32_t dtype;    /* abs_dtype */
} abs_shape;

/* Host-side plan, filled by abs_plan_init.  Read-only afterwards. */
typedef struct {
  abs_shape s;
  int32_t padded[3];       /* grid rounded up to whole blocks */
  int32_t nblk[3];         /* blocks per axis */
  int32_t num_blocks;      /* nb, blocks per head */
  int32_t block_tokens;    /* Bt = bt*bh*bw */
  int32_t heads_per_phase; /* phase width used by ABS_SCHED_HEAD_PHASED (heads whose
                              K and V fit in about 24 MB, at least one) */
  int32_t reserved;
  int64_t tokens;          /* N = T*H*W */
  int64_t rows;            /* B*H*nb rows of the block mask */
  int64_t col_capacity;    /* rows*nb: worst-case col_idx length */
  size_t route_ws_bytes;   /* workspace abs_route needs */
  size_t attend_ws_bytes;  /* workspace abs_attend needs */
} abs_plan;

/* Per-head CSR block mask, device buffers owned by the caller:
 *   row_ptr  int32 [rows + 1]       rows r = (b*H + h)*nb + i
 *   col_idx  int32 [col_capacity]   kept key blocks of row r, ascending, in
 *                                   col_idx[row_ptr[r] .. row_ptr[r+1])
 *   head_nnz int32 [B*H]            kept blocks per head                   */
typedef struct {
  int32_t* row_ptr;
  int32_t* col_idx;
  int32_t* head_nnz;
} abs_mask;

/* Fill *out for the given shape.  Host only, synchronous, no device access.
 * Supported: head_dim in {64, 128}; bt*bh*bw in {32, 64, 128}; nb <= 8192;
 * rows*nb < 2^31 (CSR positions are int32).  Element offsets are 64-bit, so
 * Q, K, V and O may hold more than 2^31 elements (for example 40 heads of an
 * 81-frame 1080p latent grid, 81x68x120 tokens: nb = 5535, 3.4e9 elements). */
abs_status abs_plan_init(const abs_shape* shape, abs_plan* out);

/* Routing (explainer "Core method" part 1, and part 3 when slack > 0).
 * For every row (b, h, i): Qp_i, Kp_j = means of q, k over the real tokens of
 * block i, j; P_ij = softmax_j(Qp_i . Kp_j / sqrt(d)) in float32; blocks
 * ordered by P descending (ties: lower j first); m = smallest count whose
 * cumulative mass reaches p (>= p; p == 1 keeps all); keep the first
 * min(nb, max(m, k_floor)) blocks plus block i itself.  With slack > 0 every
 * head is then topped up to ceil(slack * nb^2) kept pairs with its unkept
 * pairs of largest P (ties: lowest i*nb + j).  Writes the CSR into *mask.
 *   q, k   : device [B, N, H, d] of the plan's dtype
 *   p      : in (0, 1];  k_floor >= 1 (values above nb keep every block)
 *   slack  : in [0, 1), 0 disables the fill
 *   ws     : device workspace of at least plan->route_ws_bytes bytes.  On
 *            return (stream order) it starts with the pooled means, float32
 *            Qp [B, H, nb, d] followed by Kp [B, H, nb, d].
 *   stream : hipStream_t (NULL = default stream)                         */
abs_status abs_route(const abs_plan* plan, const void* q, const void* k, float p,
                     int32_t k_floor, float slack, const abs_mask* mask, void* ws,
                     size_t ws_bytes, void* stream);

/* Routing with a dynamic slack fill (explainer "Core method" part 3: after
 * balancing, workers off the critical path still go idle, and that capacity is
 * filled with high-scoring blocks; "Lessons for engineering" item 5: only
 * blocks above a score threshold are used, and the injected amount is the knob
 * to turn down).  Base routing as abs_route with slack = 0, then, over the
 * whole batch at once, the unkept pairs with P >= theta are ranked by P
 * descending (ties: lowest linear index ((b*H + h)*nb + i)*nb + j) and the
 * first min(*budget, number of such pairs) are added.  The budget is read on
 * the device, in stream order, so it can come straight from
 * abs_slack_budget without a host round trip.
 *   theta  : in [0, 1]
 *   budget : device int64 [1]; values below 0 count as 0
 *   ws     : as abs_route (plan->route_ws_bytes); the pooled means are at its
 *            start on return, as there.
 * Errors as abs_route, plus ABS_EINVAL for theta outside [0, 1] or a null
 * budget. */
abs_status abs_route_dynamic(const abs_plan* plan, const void* q, const void* k, float p,
                             int32_t k_floor, float theta, const int64_t* budget,
                             const abs_mask* mask, void* ws, size_t ws_bytes, void* stream);

/* Pair budget for abs_route_dynamic from the telemetry of one persistent
 * attention launch of this plan (abs_attend_run or abs_attend_run_split with
 * the same sched; abs_attend_grid(plan, sched) records).  With T = the largest
 * busy count, idle = sum over workgroups of (T - busy) ticks; at the launch's
 * mean cost per kept tile this is idle * sum(tiles) / sum(busy) tiles, and
 * *budget = floor(fill * that) clamped to [0, max_pairs] (integer product,
 * then one float64 multiply and one divide).  Written on the device in stream
 * order.
 *   telemetry : device int64 records as abs_attend_run writes them
 *   fill      : in [0, 1]; max_pairs >= 0
 *   budget    : device int64 [1], written
 * Errors: ABS_EINVAL for a null pointer, sched HEAD_MAJOR (its workgroups are
 * not persistent workers) or out-of-range fill / max_pairs; ABS_ENOTSUP for
 * float32 plans (their attention is not persistent). */
abs_status abs_slack_budget(const abs_plan* plan, int32_t sched, const int64_t* telemetry,
                            float fill, int64_t max_pairs, int64_t* budget, void* stream);

/* Attention prologue: re-lays k and v block-major for the attention kernel
 * (bf16) and builds the order of `sched` over the attention work items from
 * the mask's row lengths (explainer "Core method" part 2: profile the mask
 * size per head, heaviest first).  A bf16 work item is a pair of
 * neighbouring query blocks of one head.  Items are numbered head by head:
 * first the t-pairs (the block with an even t coordinate and its successor;
 * plane pair by plane pair, blocks in row-major (h, w) order); if nbt is odd,
 * the last t-plane's h-pairs (even h and its successor; row pair by row pair,
 * w ascending); if nbh is odd too, that plane's last row's w-pairs (even w and
 * its successor); if nbw is odd as well, its last block alone.  An item's cost
 * is the kept-block count of its rows.  On
 * return (stream order) the workspace starts with the item order, int32
 * [items].  Float32 plans process rows in natural order.
 *   k, v : device [B, N, H, d] of the plan's dtype
 *   ws   : device workspace of at least plan->attend_ws_bytes bytes; it must
 *          be passed unchanged to abs_attend_run.                          */
abs_status abs_attend_prepare(const abs_plan* plan, const void* k, const void* v,
                              const abs_mask* mask, int32_t sched, void* ws, size_t ws_bytes,
                              void* stream);

/* The two halves of abs_attend_prepare, for callers that overlap the first
 * with routing (it does not depend on the mask).  abs_attend_relayout does the
 * K/V re-layout (bf16) or the V copy (float32) into ws; abs_attend_schedule
 * builds the work items' key-block lists and the order of `sched` from the
 * mask.  Both, in either order or on different streams, followed by
 * abs_attend_run in stream order after both (the caller orders the streams,
 * for instance with events), leave ws exactly as abs_attend_prepare does.
 * Arguments and errors as abs_attend_prepare. */
abs_status abs_attend_relayout(const abs_plan* plan, const void* k, const void* v, void* ws,
                               size_t ws_bytes, void* stream);
abs_status abs_attend_schedule(const abs_plan* plan, const abs_mask* mask, int32_t sched,
                               void* ws, size_t ws_bytes, void* stream);

/* Block-sparse attention over the kept blocks (explainer "Core method" part 1
 * and "The real problem"): for each real query token of block i, one softmax
 * over the real keys of all kept blocks of row (b, h, i), scale 1/sqrt(d),
 * output written to o [B, N, H, d].  Requires abs_attend_prepare on the same
 * ws, mask and sched earlier in stream order.
 *   telemetry : NULL, or device int64 [abs_attend_grid(...) * 4]: per
 *               workgroup {hardware id register, XCC id, kept tiles processed,
 *               busy clock ticks}.                                          */
abs_status abs_attend_run(const abs_plan* plan, const void* q, const void* k,
                          const abs_mask* mask, void* o, int32_t sched, void* ws,
                          size_t ws_bytes, int64_t* telemetry, void* stream);

/* abs_attend_prepare followed by abs_attend_run. */
abs_status abs_attend(const abs_plan* plan, const void* q, const void* k, const void* v,
                      const abs_mask* mask, void* o, int32_t sched, void* ws,
                      size_t ws_bytes, int64_t* telemetry, void* stream);

/* The schedule that measured fastest for this plan's shape on MI355X.  With
 * phases that keep at most about 24 MB of K and V in flight (one head at the
 * 480p, 720p and 81-frame shapes), HEAD_PHASED led on every workload measured
 * (480p by 0.5 % over XCD_LOCAL, the head-imbalance stress by 1-2 %, 720p and
 * the 81-frame 1.3B shape by 5-6 %), so it is returned for every plan; the
 * query stays so that callers need not hard-code it.  Host query. */
abs_status abs_attend_default_sched(const abs_plan* plan, int32_t* sched);

/* Number of workgroups abs_attend_run launches for this plan and schedule on
 * the current device (the telemetry record count).  Host query. */
abs_status abs_attend_grid(const abs_plan* plan, int32_t sched, int32_t* workgroups);

/* Split-and-merge attention (bf16 plans; persistent sorted queues, i.e. sched
 * ABS_SCHED_NNZ_SORTED or ABS_SCHED_HEAD_PHASED).  Load balancing over compute
 * units (explainer "Core method" part 2) is limited by the size of the largest
 * work item; this mode cuts heavy items into parts that run on different
 * workgroups and combines the parts' partial softmax results by their
 * log-sum-exp, the merge the APB-V paper notes ("APB-V: Accelerating
 * Long-Video Understanding via Sequence-Parallelism-aware Approximate
 * Attention", key design 2) use to join one query block's attention computed
 * on several hosts.
 *
 * A work item (see abs_attend_prepare) walks the ascending union of its two
 * rows' kept key blocks, nt entries.  With split_tiles = S, an item with
 * nt > S wants P = ceil(nt / S) parts, part p taking union entries
 * [p*nt/P, (p+1)*nt/P) (integer division).  Items are cut heaviest first (nt
 * descending, ties by lower item index) while the running sum of their P stays
 * within max_parts; the first that does not fit ends the cutting, and the rest
 * stay whole.  Slots are numbered over the cut items in item order.  Each
 * part writes float32 partials (O not yet normalised, its reference maximum
 * and its sum, per query); a merge kernel
 * then writes o for the cut items.  The result is the same softmax up to
 * rounding (parts' partials are float32, combined in ascending part order), is
 * bitwise independent of the queue order, and equals abs_attend_run's output
 * bitwise for items that are not cut.  The queue is sorted by part length (in
 * union entries), longest first.
 *
 * On return (stream order) from abs_attend_prepare_split the workspace starts
 * with the work-unit table, int32 [items + max_parts][4]: one entry
 * {item, t0, t1, slot} per unit (slot -1 for an item that is not cut), units
 * of an item consecutive, items in ascending order; entries past the last
 * unit are unspecified.
 *
 * Workspace: abs_attend_split_ws_bytes(plan, max_parts) bytes, which holds
 * max_parts slots of (2*Bt*d + 4*Bt) floats each (133 120 bytes for Bt = 128,
 * d = 128) on top of the plain attend workspace; a slot count above 2^24 is
 * rejected (ABS_EINVAL).  The same ws, mask, sched and max_parts go to
 * abs_attend_prepare_split and then abs_attend_run_split, in stream order.
 * Telemetry has abs_attend_grid(plan, sched) records, tiles counting the kept
 * (row, key block) pairs each workgroup processed.  Errors: ABS_EINVAL for
 * another sched, split_tiles < 1, max_parts outside [0, 2^24] or null
 * pointers; ABS_ENOTSUP for float32 plans; ABS_ENOSPACE for a small ws. */
abs_status abs_attend_split_ws_bytes(const abs_plan* plan, int32_t max_parts, size_t* bytes);
abs_status abs_attend_prepare_split(const abs_plan* plan, const void* k, const void* v,
                                    const abs_mask* mask, int32_t sched, int32_t split_tiles,
                                    int32_t max_parts, void* ws, size_t ws_bytes, void* stream);
abs_status abs_attend_run_split(const abs_plan* plan, const void* q, const abs_mask* mask,
                                void* o, int32_t sched, int32_t max_parts, void* ws,
                                size_t ws_bytes, int64_t* telemetry, void* stream);

/* Bytes of the static device scratch that abs_route_noalloc works in. */
#define ABS_ROUTE_NOALLOC_SCRATCH_BYTES (64ull << 20)

/* abs_route for callers that cannot allocate device memory: code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc.  Same
 * arguments, computation and result as abs_route, but no workspace argument:
 * the route workspace is a static device array of
 * ABS_ROUTE_NOALLOC_SCRATCH_BYTES (64 MiB) that the library holds on every GPU
 * it runs on until the process ends.  The call allocates and frees nothing
 * (no hipMalloc, hipFree or allocating library routine).
 *   Size limit: the workspace abs_route needs for this plan and slack must fit
 *   the scratch; plan->route_ws_bytes (the need with the fill) bounds it.
 *   A larger plan returns ABS_ETOOBIG before any device call.
 *   Sharing: every call on one GPU works in that GPU's one array, which keeps
 *   the last call's contents (nothing in it has to start at zero: each call
 *   writes what it reads).  Calls that overlap in time on one GPU (several
 *   streams or host threads) race and give undefined masks; order them on one
 *   stream or with events.
 *   stream : hipStream_t of the current device (NULL = its default stream);
 *            a stream of another device returns ABS_EINVAL.
 * Errors as abs_route (ABS_ENOSPACE cannot occur), plus ABS_ETOOBIG, and
 * ABS_EHIP if the scratch address cannot be obtained. */
abs_status abs_route_noalloc(const abs_plan* plan, const void* q, const void* k, float p,
                             int32_t k_floor, float slack, const abs_mask* mask, void* stream);

/* Fine-grained Top-p inside the kept blocks (explainer "Core method" part 1,
 * video-aware block organisation: block-level decisions are combined with
 * Top-p's fine-grained decisions; the fact-check table repeats "block-level
 * decisions combined with fine-grained Top-p").  Block routing as abs_route
 * (no slack fill), then Top-p again over frames: frame tau of key block j is
 * the part of the block at temporal offset tau (its real tokens with
 * t % bt == tau).  For every row (b, h, i), the candidates are the frames with
 * real tokens of the blocks the row keeps; their masses are the softmax, over
 * the candidates only, of Qp_i . Kf_(j,tau) / sqrt(d) (Kf = mean of k over
 * the frame's real tokens); ordered by mass (ties: lower j*bt + tau first),
 * the smallest prefix whose mass reaches p_frame is kept (p_frame == 1 keeps
 * every candidate), never fewer than k_floor frames, and every frame of block
 * i.  A kept block may keep no frame.
 *   p_frame    : in (0, 1]
 *   frame_mask : device int32 [plan->col_capacity], written: entry e (aligned
 *                with mask->col_idx) has bit tau set when frame tau of block
 *                col_idx[e] is kept
 *   ws         : route workspace of at least plan->route_ws_bytes bytes
 * Supported: block[0] (frames per block) <= 6 and nb * block[0] <= 1024
 * (ABS_ENOTSUP otherwise).  Other errors as abs_route. */
abs_status abs_route_frames(const abs_plan* plan, const void* q, const void* k, float p,
                            int32_t k_floor, float p_frame, const abs_mask* mask,
                            int32_t* frame_mask, void* ws, size_t ws_bytes, void* stream);

/* Block-sparse attention restricted to kept frames: as abs_attend, but each
 * real query token of block i attends to the real keys of the kept frames
 * (frame_mask from abs_route_frames) of the kept blocks of its row.  Runs the
 * prologue (K/V re-layout, key-block lists with each row's frames, schedule)
 * and the attention.  bf16 plans with 128-token blocks, block[0] <= 6
 * (ABS_ENOTSUP otherwise); any sched; ws of at least plan->attend_ws_bytes
 * bytes.  Telemetry as abs_attend_run (tiles count kept blocks). */
abs_status abs_attend_frames(const abs_plan* plan, const void* q, const void* k, const void* v,
                             const abs_mask* mask, const int32_t* frame_mask, void* o,
                             int32_t sched, void* ws, size_t ws_bytes, int64_t* telemetry,
                             void* stream);

/* Static description of a status code. */
const char* abs_status_string(abs_status status);

#ifdef __cplusplus
}
#endif

#endif /* ABS_H */
