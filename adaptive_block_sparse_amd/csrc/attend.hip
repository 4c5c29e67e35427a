// Attention kernels: V re-layout, work schedule, and block-sparse flash-style
// attention over the kept key blocks.  Source: FVAttn explainer ("FVAttn:
// adaptive sparse attention with runtime load balancing, for video
// generation"), "Core method" part 1 (attention restricted to the routed KV
// blocks) and part 2 (runtime load balancing: per-head mask sizes measured
// before the kernel, heaviest work first), recast from ranks to the compute
// units of one GPU.
#include <hip/hip_runtime.h>

#include <math.h>

#include <type_traits>

#include "device_common.h"
#include "internal.h"

// the LDS copies set M0 inside inline asm (declared as clobbered)
#pragma clang diagnostic ignored "-Winline-asm"

namespace abs_impl {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

#define LDS_PTR(p) ((__attribute__((address_space(3))) void*)(p))

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}
// Workgroup barrier that does not drain outstanding global loads (the HIP
// __syncthreads() also waits for every in-flight vector memory operation,
// which would serialise the K/V prefetch with the math).
__device__ __forceinline__ void wg_barrier() { asm volatile("s_barrier" ::: "memory"); }

// Key order inside each 16-key group of the re-laid V: positions 0-7 hold keys
// {0-3, 8-11} and positions 8-15 hold keys {4-7, 12-15}, which is the order in
// which a 32x32 MFMA accumulator hands the softmax probabilities to the next
// MFMA as its B operand.  Swapping bits 2 and 3 maps a key to its position and
// back.
__host__ __device__ __forceinline__ int vt_perm(int k) {
  return (k & ~12) | ((k >> 1) & 4) | ((k << 1) & 8);
}

// ---------------------------------------------------------------------------
// Slot order inside a block tile: the block's real tokens come first, in
// row-major (t, h, w) order over the block's real extent Tl x Hl x Wl, and the
// padding slots follow.  For a whole block this is the row-major slot order of
// the blocking; in a block cut by the grid edge it packs the real tokens, so
// that whole 64-key chunks and 32-query subtiles of padding can be skipped.
// Returns the token's offset ((st * Hg + sh) * W + sw) from the block's first
// token, for slot s < Tl * Hl * Wl.
// ---------------------------------------------------------------------------
__device__ __forceinline__ int packed_slot_offset(const Geo& g, int s, int Hl, int Wl) {
  const int st = s / (Hl * Wl), r = s - st * (Hl * Wl);
  const int sh = r / Wl, sw = r - sh * Wl;
  return (st * g.Hg + sh) * g.W + sw;
}

// Maximum of two scores.  The IEEE maximum (NaN propagating) needs no
// quieting of its inputs, so chains of it become v_maximum3_f32; fmaxf would
// first canonicalise every MFMA result.  Scores are finite.
__device__ __forceinline__ float vmax(float a, float b) {
  return __builtin_elementwise_maximum(a, b);
}

// Real extent of block j: Tl | Hl << 8 | Wl << 16.
__device__ __forceinline__ int block_extent(const Geo& g, int j) {
  const int tb = j / (g.nbh * g.nbw), hb = (j / g.nbw) % g.nbh, wb = j % g.nbw;
  const int Tl = min(g.bt, g.T - tb * g.bt), Hl = min(g.bh, g.Hg - hb * g.bh),
            Wl = min(g.bw, g.W - wb * g.bw);
  return Tl | (Hl << 8) | (Wl << 16);
}

// ---------------------------------------------------------------------------
// K/V re-layout into the attention kernel's chunk-major block tiles (bf16):
//   Kc[b, h, blk, c, key, 8]: 16-byte chunk c (d = 8c .. 8c+7) of every key;
//   Vc[b, h, blk, c, d, 8]  : for every d, the 8 keys of key chunk c, in
//                             vt_perm order;
// slots in the packed order above, zeros in padding slots.  A tile is then one
// contiguous BT*D*2-byte copy into
// LDS, and every MFMA operand read is (lane base + compile-time offset).  One
// workgroup per (block, b*h, K|V).
// ---------------------------------------------------------------------------
template <int D, int BT>
__global__ __launch_bounds__(256) void kv_relayout_kernel(Geo g, const bf16_t* __restrict__ k,
                                                          const bf16_t* __restrict__ v,
                                                          bf16_t* __restrict__ kc,
                                                          bf16_t* __restrict__ vc,
                                                          float* __restrict__ kn) {
  constexpr int RW = D / 2 + 4;  // row stride in 32-bit words (16-byte aligned, padded)
  __shared__ __attribute__((aligned(16))) uint32_t tile[BT * RW];
  const int blk = blockIdx.x, bh = blockIdx.y, which = blockIdx.z;
  const int b = bh / g.H, h = bh % g.H;
  const int tb = blk / (g.nbh * g.nbw), hb = (blk / g.nbw) % g.nbh, wb = blk % g.nbw;
  const int Tl = min(g.bt, g.T - tb * g.bt), Hl = min(g.bh, g.Hg - hb * g.bh),
            Wl = min(g.bw, g.W - wb * g.bw);
  const int nreal = Tl * Hl * Wl;
  const long n0 = ((long)(tb * g.bt) * g.Hg + hb * g.bh) * g.W + wb * g.bw;
  const bf16_t* src = which == 0 ? k : v;
  // every load of this thread is issued before the first LDS store
  constexpr int NIT = (BT * (D / 8) + 255) / 256;
  uint4 val[NIT];
#pragma unroll
  for (int it = 0; it < NIT; ++it) {
    const int e = threadIdx.x + 256 * it;
    const int s = e / (D / 8), c = e % (D / 8);
    val[it] = make_uint4(0, 0, 0, 0);
    if (e < BT * (D / 8) && s < nreal) {
      const long n = n0 + packed_slot_offset(g, s, Hl, Wl);
      val[it] = *reinterpret_cast<const uint4*>(src + (((long)b * g.N + n) * g.H + h) * D + c * 8);
    }
  }
#pragma unroll
  for (int it = 0; it < NIT; ++it) {
    const int e = threadIdx.x + 256 * it;
    if (e < BT * (D / 8))
      *reinterpret_cast<uint4*>(&tile[(e / (D / 8)) * RW + (e % (D / 8)) * 4]) = val[it];
  }
  __syncthreads();
  const long tile_off = ((long)bh * g.nb + blk) * (long)(D * BT);
  if (which == 0) {
    // largest norm of the block's keys (padding slots are zero), rounded up by
    // a relative 2^-12 so that it bounds the norm of the bf16 key exactly
    {
      constexpr int TPK = 256 / BT;   // threads per key
      const int key = threadIdx.x / TPK, part = threadIdx.x % TPK;
      float ss = 0.f;
      for (int w = part; w < D / 2; w += TPK) {
        const uint32_t x = tile[key * RW + w];
        const float lo = __uint_as_float(x << 16), hi = __uint_as_float(x & 0xffff0000u);
        ss = fmaf(lo, lo, ss);
        ss = fmaf(hi, hi, ss);
      }
      for (int o = 1; o < TPK; o <<= 1) ss += __shfl_xor(ss, o);
      for (int o = TPK; o < 64; o <<= 1) ss = fmaxf(ss, __shfl_xor(ss, o));
      __shared__ float wmax[4];
      if ((threadIdx.x & 63) == 0) wmax[threadIdx.x >> 6] = ss;
      __syncthreads();
      if (threadIdx.x == 0)
        kn[(long)bh * g.nb + blk] =
            sqrtf(fmaxf(fmaxf(wmax[0], wmax[1]), fmaxf(wmax[2], wmax[3]))) * (1.0f + 0x1p-12f);
    }
    uint4* out = reinterpret_cast<uint4*>(kc + tile_off);
    for (int e = threadIdx.x; e < BT * (D / 8); e += 256) {
      const int c = e / BT, key = e % BT;
      out[e] = *reinterpret_cast<const uint4*>(&tile[key * RW + c * 4]);
    }
  } else {
    uint4* out = reinterpret_cast<uint4*>(vc + tile_off);
    for (int e = threadIdx.x; e < D * (BT / 8); e += 256) {
      const int c = e / D, d = e % D;
      uint32_t w[4];
#pragma unroll
      for (int x = 0; x < 4; ++x) {
        const int k0 = vt_perm(c * 8 + 2 * x), k1 = vt_perm(c * 8 + 2 * x + 1);
        const uint32_t lo = (tile[k0 * RW + (d >> 1)] >> ((d & 1) * 16)) & 0xffffu;
        const uint32_t hi = (tile[k1 * RW + (d >> 1)] >> ((d & 1) * 16)) & 0xffffu;
        w[x] = lo | (hi << 16);
      }
      out[e] = make_uint4(w[0], w[1], w[2], w[3]);
    }
  }
}

// ---------------------------------------------------------------------------
// Work schedule over attention work items (groups of one or two paired query
// blocks of one head, see group_blocks), or over split-and-merge units.  A
// stable LSD radix sort (4-bit digits, one workgroup per sorted range) by key:
//   NNZ_SORTED : key = 2nb - cost (largest first);
//   HEAD_PHASED: key = phase * (2nb + 1) + 2nb - cost, phase = head / hpp
//                (work items: each phase's range sorted by its own workgroup);
//   HEAD_MAJOR : natural order;
//   XCD_LOCAL  : no sort; heads placed on XCDs, one queue per XCD (below).
// cost = kept blocks of the group's rows (a unit: its number of union
// entries).  Ties keep item order.  Also resets the persistent queue heads.
// ---------------------------------------------------------------------------
__device__ __forceinline__ int group_cost(const Geo& g, const int* row_ptr, int item) {
  const int bh = item / g.groups_per_head, gl = item % g.groups_per_head;
  int lead, partner;
  group_blocks(g, gl, &lead, &partner);
  const int r = bh * g.nb + lead;
  int c = row_ptr[r + 1] - row_ptr[r];
  if (partner >= 0) c += row_ptr[r - lead + partner + 1] - row_ptr[r - lead + partner];
  return c;
}

// Key of queue entry r: a work item (cost from the per-item table the bf16
// prologue writes, else from the CSR), or (split-and-merge) a work unit whose
// cost is the length of its range of the item's union list (at most 2nb).
__device__ __forceinline__ unsigned sched_key(const Geo& g, const int* row_ptr, const int* icost,
                                              const int* units, int r, int phased, int hpp) {
  int item, cost;
  if (units) {
    item = units[4 * r];
    cost = units[4 * r + 2] - units[4 * r + 1];
  } else {
    item = r;
    cost = icost ? icost[r] : group_cost(g, row_ptr, r);
  }
  const unsigned k = (unsigned)(2 * g.nb - cost);
  return phased ? (unsigned)((item / g.groups_per_head) / hpp) * (unsigned)(2 * g.nb + 1) + k : k;
}

__global__ __launch_bounds__(512) void schedule_kernel(Geo g, const int* __restrict__ row_ptr,
                                                       int mode, int hpp, int* __restrict__ sched,
                                                       int* __restrict__ buf_a,
                                                       int* __restrict__ buf_b,
                                                       int* __restrict__ counter,
                                                       const int* __restrict__ units,
                                                       const int* __restrict__ icost) {
  constexpr int NT = 512;
  __shared__ unsigned offs[16][NT];
  __shared__ unsigned stmp[NT / 64 + 1];
  // queue entries: work items, or the split units counted by split_units_kernel
  const int items = units ? counter[NUNITS] : g.groups;
  if (blockIdx.x == 0) {
    if (threadIdx.x == 0) counter[0] = 0;
    if (threadIdx.x < NXCD) counter[QHEAD + 32 * threadIdx.x] = 0;
  }
  if (mode == ABS_SCHED_HEAD_MAJOR) {
    for (int r = threadIdx.x; r < items; r += NT) sched[r] = r;
    return;
  }
  if (mode == ABS_SCHED_XCD_LOCAL) {
    // head costs, then LPT placement of heads on XCDs (longest first onto the
    // least loaded XCD, ties to the lower index); beyond MAX_LPT_HEADS heads,
    // head h goes to XCD h % NXCD
    __shared__ int hcost[MAX_LPT_HEADS];
    __shared__ int hbase[MAX_LPT_HEADS];
    __shared__ int qlen[NXCD];
    const int heads = g.B * g.H;
    const bool lpt = heads <= MAX_LPT_HEADS;
    if (lpt) {
      // every thread adds its items' costs to their heads (integer sums: the
      // result does not depend on the order)
      for (int hh = threadIdx.x; hh < heads; hh += NT) hcost[hh] = 0;
      __syncthreads();
      for (int it = threadIdx.x; it < items; it += NT)
        atomicAdd(&hcost[it / g.groups_per_head], icost ? icost[it] : group_cost(g, row_ptr, it));
    }
    __syncthreads();
    // heads in (cost desc, index asc) order: each thread ranks its heads
    __shared__ int horder[MAX_LPT_HEADS];
    if (lpt) {
      for (int hh = threadIdx.x; hh < heads; hh += NT) {
        const int c = hcost[hh];
        int r = 0;
        for (int o = 0; o < heads; ++o) {
          const int co = hcost[o];
          r += (co > c || (co == c && o < hh)) ? 1 : 0;
        }
        horder[r] = hh;
      }
    }
    __syncthreads();
    if (threadIdx.x == 0) {
      long long load[NXCD];
      int rank[NXCD];
      for (int x = 0; x < NXCD; ++x) { load[x] = 0; rank[x] = 0; }
      for (int n = 0; n < heads && lpt; ++n) {
        const int best = horder[n];
        int xm = 0;
        for (int x = 1; x < NXCD; ++x)
          if (load[x] < load[xm]) xm = x;
        load[xm] += hcost[best];
        hbase[best] = xm * MAX_LPT_HEADS + rank[xm]++;   // (xcd, rank) packed
      }
      for (int x = 0; x < NXCD; ++x) qlen[x] = 0;
      if (lpt) {
        for (int x = 0; x < NXCD; ++x) qlen[x] = rank[x] * g.groups_per_head;
      } else {
        for (int hh = 0; hh < heads; ++hh) qlen[hh % NXCD] += g.groups_per_head;
      }
      int off = 0;
      for (int x = 0; x < NXCD; ++x) { counter[QOFF + x] = off; off += qlen[x]; }
      counter[QOFF + NXCD] = off;
      for (int x = 0; x < NXCD; ++x) qlen[x] = counter[QOFF + x];   // now queue starts
    }
    __syncthreads();
    for (int it = threadIdx.x; it < items; it += NT) {
      const int hh = it / g.groups_per_head, gl = it % g.groups_per_head;
      int pos;
      if (lpt) {
        const int x = hbase[hh] / MAX_LPT_HEADS, rk = hbase[hh] % MAX_LPT_HEADS;
        pos = qlen[x] + rk * g.groups_per_head + gl;
      } else {
        pos = qlen[hh % NXCD] + (hh / NXCD) * g.groups_per_head + gl;
      }
      sched[pos] = it;
    }
    return;
  }
  // Work items (not split units) sit head by head, so under HEAD_PHASED each
  // phase is a contiguous range of them and the queue is that range sorted by
  // cost alone: one workgroup per phase (the launch's grid) sorts its range.
  int phased = mode == ABS_SCHED_HEAD_PHASED;
  int base = 0, n = items;
  if (phased && !units) {
    base = blockIdx.x * hpp * g.groups_per_head;
    n = min(items - base, hpp * g.groups_per_head);
    phased = 0;
    if (n <= 0) return;
  }
  const int nphase = phased ? (g.B * g.H + hpp - 1) / hpp : 1;
  const unsigned maxkey = (unsigned)nphase * (unsigned)(2 * g.nb + 1);
  int passes = 1;
  while (passes < 8 && (maxkey >> (4 * passes)) != 0u) ++passes;
  const int per = (n + NT - 1) / NT;
  const int lo = base + threadIdx.x * per, hi = min(base + n, lo + per);
  for (int pass = 0; pass < passes; ++pass) {
    const int* src = pass == 0 ? nullptr : ((pass & 1) ? buf_a : buf_b);
    int* dst = pass == passes - 1 ? sched : ((pass & 1) ? buf_b : buf_a);
    const int sh = 4 * pass;
    unsigned cnt[16];
#pragma unroll
    for (int x = 0; x < 16; ++x) cnt[x] = 0u;
    for (int e = lo; e < hi; ++e) {
      const int r = src ? src[e] : e;
      const unsigned dg = (sched_key(g, row_ptr, icost, units, r, phased, hpp) >> sh) & 15u;
#pragma unroll
      for (int x = 0; x < 16; ++x) cnt[x] += (dg == (unsigned)x) ? 1u : 0u;
    }
#pragma unroll
    for (int x = 0; x < 16; ++x) offs[x][threadIdx.x] = cnt[x];
    __syncthreads();
    // exclusive scan of the flattened [digit][thread] table: thread t owns
    // the 16 consecutive entries 16t .. 16t+15
    unsigned loc[16];
    unsigned run = 0u;
#pragma unroll
    for (int x = 0; x < 16; ++x) {
      const int f = threadIdx.x * 16 + x;
      loc[x] = run;
      run += offs[f / NT][f % NT];
    }
    unsigned tot;
    const unsigned pre = block_exclusive_scan<NT>(run, stmp, &tot);
#pragma unroll
    for (int x = 0; x < 16; ++x) {
      const int f = threadIdx.x * 16 + x;
      offs[f / NT][f % NT] = pre + loc[x];
    }
    __syncthreads();
    for (int e = lo; e < hi; ++e) {
      const int r = src ? src[e] : e;
      const unsigned dg = (sched_key(g, row_ptr, icost, units, r, phased, hpp) >> sh) & 15u;
      const unsigned pos = offs[dg][threadIdx.x]++;
      dst[base + pos] = r;
    }
    __syncthreads();
  }
}

// ---------------------------------------------------------------------------
// Per attention work item (a pair of query blocks of one head, or a single
// block), the union of its rows' kept key-block lists in ascending order, each
// entry j | (short) << 16 | (kept by the first block) << 17 | (kept by the
// second) << 18, where short marks a key block whose real tokens all sit in the
// first 64 slots of its tile (at most 64 real tokens, packed first).  One
// workgroup per item: the two rows are marked in two LDS bitmaps of nb bits, a
// workgroup scan of the union's word popcounts gives each word's first list
// position, and every kept block is written in ascending order from there.  The
// list of item i starts at tlist[i * cap], cap = 2 nb, with tcount[i] entries.
// ---------------------------------------------------------------------------
//
// With frame masks (fine-grained routing: frame_mask[e] bit tau = frame tau of
// col_idx[e] kept), a row owns a block only if it keeps one of its frames, the
// entry also holds the kept frames of the first block's row << 19 and of the
// second's << 25 (at most 6 frames a block), and short also marks a block whose
// kept frames (of either row) all sit in the first 64 slots.
template <bool FR = false>
__global__ __launch_bounds__(256) void tile_list_kernel(Geo g, const int* __restrict__ row_ptr,
                                                        const int* __restrict__ col_idx, int cap,
                                                        int* __restrict__ tlist,
                                                        int* __restrict__ tcount,
                                                        int* __restrict__ icost,
                                                        const int* __restrict__ frame_mask = nullptr) {
  constexpr int NT = 256, MAXW = MAX_NB / 32;
  static_assert(MAXW <= NT, "one bitmap word per thread");
  __shared__ uint32_t bA[MAXW], bB[MAXW], bS[MAXW];   // kept by A, by B; short blocks
  __shared__ int woff[MAXW];                           // list position of each word's first
  __shared__ int tmp[NT / 64 + 1];
  __shared__ uint8_t fA[FR ? MAX_NB : 1], fB[FR ? MAX_NB : 1];   // frames kept by A, by B
  const int item = blockIdx.x;
  const int bhh = item / g.groups_per_head, gl = item % g.groups_per_head;
  int lead, partner;
  group_blocks(g, gl, &lead, &partner);
  const int rA = bhh * g.nb + lead;
  const int pA = row_ptr[rA], nA = row_ptr[rA + 1] - pA;
  int pB = 0, nB = 0;
  if (partner >= 0) {
    const int rB = bhh * g.nb + partner;
    pB = row_ptr[rB];
    nB = row_ptr[rB + 1] - pB;
  }
  const int W = (g.nb + 31) / 32;
  for (int w = threadIdx.x; w < W; w += NT) { bA[w] = 0u; bB[w] = 0u; bS[w] = 0u; }
  __syncthreads();
  if constexpr (FR)
    for (int j = threadIdx.x; j < g.nb; j += NT) { fA[j] = 0; fB[j] = 0; }
  if constexpr (!FR)
    for (int j = threadIdx.x; j < g.nb; j += NT) {
      const int e = block_extent(g, j);
      if ((e & 255) * ((e >> 8) & 255) * ((e >> 16) & 255) <= 64)
        atomicOr(&bS[j >> 5], 1u << (j & 31));
    }
  for (int i = threadIdx.x; i < nA; i += NT) {
    const int v = col_idx[pA + i];
    if (FR) {
      const int fm = frame_mask[pA + i];
      if (fm == 0) continue;
      fA[v] = (uint8_t)fm;
    }
    atomicOr(&bA[v >> 5], 1u << (v & 31));
  }
  for (int i = threadIdx.x; i < nB; i += NT) {
    const int v = col_idx[pB + i];
    if (FR) {
      const int fm = frame_mask[pB + i];
      if (fm == 0) continue;
      fB[v] = (uint8_t)fm;
    }
    atomicOr(&bB[v >> 5], 1u << (v & 31));
  }
  __syncthreads();
  if constexpr (FR)
    for (int j = threadIdx.x; j < g.nb; j += NT) {
      // short: the real tokens of every kept frame lie in the first 64 slots
      const int e = block_extent(g, j);
      const int fs = ((e >> 8) & 255) * ((e >> 16) & 255);   // tokens per frame
      const int u = fA[j] | fB[j];
      const int top = u ? 31 - __clz(u) : 0;                 // highest kept frame
      if (u && (top + 1) * fs <= 64) atomicOr(&bS[j >> 5], 1u << (j & 31));
    }
  __syncthreads();
  {
    const int w = threadIdx.x;
    const uint32_t u = w < W ? (bA[w] | bB[w]) : 0u;
    int tot;
    const int off = block_exclusive_scan<NT>((int)__popc(u), tmp, &tot);
    if (w < W) woff[w] = off;
    if (threadIdx.x == 0) tcount[item] = tot;
  }
  __syncthreads();
  // every block of the union: its place is its word's offset plus the kept
  // blocks below it in the word
  int* out = tlist + (long)item * cap;
  for (int j = threadIdx.x; j < g.nb; j += NT) {
    const int wj = j >> 5, bit = j & 31;
    const uint32_t a = bA[wj], b = bB[wj];
    if (!(((a | b) >> bit) & 1u)) continue;
    const int pos = woff[wj] + __popc((a | b) & ((1u << bit) - 1u));
    const int owners = (int)((a >> bit) & 1u) | ((int)((b >> bit) & 1u) << 1);
    int ent = j | ((int)((bS[wj] >> bit) & 1u) << 16) | (owners << 17);
    if constexpr (FR) ent |= ((int)fA[j] << 19) | ((int)fB[j] << 25);
    out[pos] = ent;
  }
  if (threadIdx.x == 0) icost[item] = nA + nB;
}

// ---------------------------------------------------------------------------
// Split-and-merge queue (one workgroup).  A work item whose union list holds
// nt > split entries wants P = ceil(nt / split) parts, part q covering entries
// [q nt / P, (q+1) nt / P) (integer division, every part non-empty).  Items
// are cut heaviest first (nt descending, ties by item index) while the running
// sum of their P stays within max_parts; the first item that does not fit ends
// the cutting.  Found without sorting: with w(v) = (items with nt == v) x P(v)
// and the suffix sums S(v) = sum over u >= v of w(u), the cut is every item
// with nt > tau plus the first floor((max_parts - S(tau+1)) / P(tau)) items
// (in item order) with nt == tau, where tau is the largest v with
// S(v) > max_parts (no tau: every heavy item is cut).  Each part owns one
// partial-result slot (slots numbered over the cut items in item order); an
// item that is not cut is one unit that writes its output directly.
//   units[u] = {item, t0, t1, slot or -1}, units of an item consecutive, items
//              in order;
//   stab[s]  = {item, first slot, P, 0} for the s-th cut item (item order);
//   counter[NUNITS], counter[NSPLIT] = number of units, of cut items.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(1024) void split_units_kernel(Geo g, const int* __restrict__ tcount,
                                                           int split, int max_parts,
                                                           int4* __restrict__ units,
                                                           int4* __restrict__ stab,
                                                           int* __restrict__ counter) {
  constexpr int NT = 1024, VPT = (2 * MAX_NB + 1 + NT - 1) / NT;   // values per thread
  __shared__ int cnt[2 * MAX_NB + 1];
  __shared__ int tmp[NT / 64 + 1];
  __shared__ int s_tau, s_allow;
  const int nv = 2 * g.nb + 1;   // union counts 0 .. 2nb
  auto parts_of = [&](int nt) { return nt > split ? (nt + split - 1) / split : 1; };
  for (int v = threadIdx.x; v < nv; v += NT) cnt[v] = 0;
  if (threadIdx.x == 0) { s_tau = -1; s_allow = 0; }
  __syncthreads();
  for (int i = threadIdx.x; i < g.groups; i += NT) {
    const int nt = tcount[i];
    if (nt > split) atomicAdd(&cnt[nt], 1);
  }
  __syncthreads();
  // suffix sums over values, high to low: thread t owns reversed positions
  // r = VPT t .. VPT t + VPT - 1, value v = nv - 1 - r
  int wv[VPT], loc = 0;
#pragma unroll
  for (int e = 0; e < VPT; ++e) {
    const int v = nv - 1 - (VPT * (int)threadIdx.x + e);
    wv[e] = (v > split && v >= 0) ? cnt[v] * parts_of(v) : 0;
    loc += wv[e];
  }
  int total;
  int run = block_exclusive_scan<NT>(loc, tmp, &total);   // S(v) of values above this chunk
#pragma unroll
  for (int e = 0; e < VPT; ++e) {
    const int v = nv - 1 - (VPT * (int)threadIdx.x + e);
    const int above = run;           // S(v + 1)
    run += wv[e];                    // S(v)
    if (v > split && run > max_parts && above <= max_parts) {
      s_tau = v;
      s_allow = (max_parts - above) / parts_of(v);
    }
  }
  __syncthreads();
  const int tau = s_tau, allow = s_allow;
  int slot_base = 0, unit_base = 0, split_base = 0, eq_base = 0;
  for (int i0 = 0; i0 < g.groups; i0 += NT) {
    const int i = i0 + threadIdx.x;
    const int nt = i < g.groups ? tcount[i] : 0;
    const int P = parts_of(nt);
    const bool at_tau = i < g.groups && nt > split && nt == tau;
    int eq_tot;
    const int eq_rank = eq_base + block_exclusive_scan<NT>(at_tau ? 1 : 0, tmp, &eq_tot);
    const bool cut = i < g.groups && nt > split && (nt > tau || (at_tau && eq_rank < allow));
    const int nu = i < g.groups ? (cut ? P : 1) : 0;
    int utot, stot, ctot;
    const int upre = block_exclusive_scan<NT>(nu, tmp, &utot);
    const int spre = block_exclusive_scan<NT>(cut ? 1 : 0, tmp, &stot);
    const int cpre = block_exclusive_scan<NT>(cut ? P : 0, tmp, &ctot);
    if (i < g.groups) {
      const int u0 = unit_base + upre, slot0 = slot_base + cpre;
      if (cut) {
        for (int q = 0; q < P; ++q)
          units[u0 + q] = make_int4(i, (q * nt) / P, ((q + 1) * nt) / P, slot0 + q);
        stab[split_base + spre] = make_int4(i, slot0, P, 0);
      } else {
        units[u0] = make_int4(i, 0, nt, -1);
      }
    }
    eq_base += eq_tot;
    slot_base += ctot;
    unit_base += utot;
    split_base += stot;
  }
  if (threadIdx.x == 0) {
    counter[NUNITS] = unit_base;
    counter[NSPLIT] = split_base;
  }
}

__global__ void reset_counter_kernel(int* counter) {
  if (threadIdx.x == 0) counter[0] = 0;
  if (threadIdx.x < NXCD) counter[QHEAD + 32 * threadIdx.x] = 0;
}

// ---------------------------------------------------------------------------
// bf16 block-sparse attention.  A workgroup handles one work item: a pair of
// neighbouring query blocks of one head (or a single block, see
// group_blocks), 4 waves per
// query block (BT = 128), wave w owning one 32-query subtile of block w/NW1
// (subtile w%NW1, rotated by two in the second block).  The workgroup walks
// the union of the two ascending kept-block lists
// (precomputed per item by tile_list_kernel and read two entries ahead);
// each K/V tile is copied into LDS once and serves both blocks that keep it
// (neighbouring blocks keep nearly the same key blocks: at 480p a copy serves
// 1.85 blocks on average).  Per kept key block j, for the waves whose block keeps j, in chunks
// of 64 keys:
//   S^T (keys x queries) = K_j Q^T with v_mfma_f32_32x32x16_bf16 (Q^T held in
//     registers as the B operand, K_j read from LDS as the A operand);
//   padding keys get -1e30 through one extra MFMA k-step (bias column times a
//     ones row), so no per-element masking is needed; a cut block's real
//     tokens come first in its tile, so chunks and 32-key subtiles of padding
//     keys, and waves of padding queries, skip their products (and a short
//     block the copies of its second chunk);
//   softmax per query column, running sum in float32.  When the
//     Cauchy-Schwarz bound on the item's scores (query norms times the head's
//     largest key norm, K norms from the re-layout) proves that exp2 of every
//     score lies in [2^-32, 2^32], the probabilities are taken against the
//     reference 0, with log2(e)/sqrt(d) folded into the bf16 Q operand: one
//     exp2 per score, no maxima (FAST walk).
//     Otherwise (EXACT walk) the reference is a lazily moved running maximum:
//     a lane's reference moves to the chunk maximum only when that maximum
//     exceeds it by more than 8 in the exp2 domain, otherwise the chunk's
//     probabilities are taken against the old reference (at most 2^8) and O^T
//     needs no rescale.  Either way O^T and the sum stay relative to one
//     common reference per query, so the result is the same softmax;
//   O^T (d x queries) += Vt_j P^T, the probabilities converted to bf16 straight
//     from the accumulator layout (see vt_perm).
// K/V tiles are double buffered: the direct global->LDS copies of the next
// union block (global_load_lds_dwordx4) run while the current one is
// computed; one barrier per block.  PERSIST: workgroups pull work items from
// an atomic queue (sched order; XCD-local: the queue of the XCD they run on,
// then the others) until it is exhausted.  SPLIT: the queue holds work units,
// each a range of an item's union list; a unit that is a part writes float32
// partials (O^T before normalisation, its reference and its sum) to its slot
// for merge_parts_kernel instead of the output.
// ---------------------------------------------------------------------------
template <int D, int BT>
struct AttnCfg {
  static constexpr int NW1 = BT / 32;               // waves per query block
  static constexpr int NW = 2 * NW1, NT = 64 * NW;   // waves / threads per workgroup
  static constexpr int TILE = BT * D * 2;            // bytes of one K or V tile
  static constexpr int INSTR = TILE / 1024;          // 1 KB per wave-wide copy
  static constexpr int ROUNDS = INSTR / NW;          // copies per thread per tile
  static constexpr int KS = D / 16, NSUB = BT / 32, DSUB = D / 32;
  static constexpr int CHS = NSUB < 2 ? NSUB : 2;    // 32-key subtiles per softmax chunk
  static constexpr int NCH = NSUB / CHS;
  static_assert(ROUNDS * NW == INSTR, "tile split");
};

struct AttnArgs {
  Geo g;
  const bf16_t* q;
  const bf16_t* kc;
  const bf16_t* vc;
  const int* row_ptr;
  const int* col_idx;
  const int* sched;
  int* counter;
  bf16_t* o;
  long long* telem;
  float c;  // log2(e) / sqrt(d)
  int head_major;
  int xcd_local;
  const int* tlist;   // per item: union of the kept key blocks with owners (tile_list_kernel)
  const int* tcount;  // per item: number of entries
  const float* kn;    // per key block: the largest norm of its keys
  int tlist_cap;      // entries reserved per item
  // split-and-merge mode: queue entries are units {item, t0, t1, slot}
  const int* units;
  float* part;        // partial-result slots
  long part_floats;   // floats per slot
};

typedef __attribute__((address_space(4))) const int cint_t;  // scalar-loadable
__device__ __forceinline__ int ld_scalar(const int* p, long i) {
  return ((cint_t*)(const void*)p)[i];
}

// Copy 16 bytes per lane from global memory at base + voff into LDS at
// lds_base + 16*lane; base and lds_base are the same in every lane.  Written as
// inline asm so that the compiler does not treat the transfer as an LDS store
// it must wait for before every LDS read; completion is tracked explicitly
// with s_waitcnt vmcnt.  The instruction writes no registers.  The address is
// a scalar base plus a 32-bit offset per lane: issuing a copy holds up the
// issuing wave, and this form, with half the per-lane address data of a full
// 64-bit address, issues faster.
__device__ __forceinline__ void dma16(const void* base, uint32_t voff, uint32_t lds_base) {
  const uint64_t b = (uint64_t)base;
  // (readfirstlane returns int: each half goes through uint32_t so that the
  // low half is zero-extended, not sign-extended, into the 64-bit base)
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)b);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(b >> 32));
  const uint64_t sb = ((uint64_t)hi << 32) | (uint64_t)lo;
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
               :
               : "v"(voff), "s"(sb), "s"(__builtin_amdgcn_readfirstlane(lds_base))
               : "memory", "m0");
}

template <int D, int BT, bool PERSIST, bool SPLIT = false, bool FRAMES = false>
__global__ __launch_bounds__(128 * (BT / 32), 2) void attn_bf16_kernel(AttnArgs a) {
  static_assert(PERSIST || !SPLIT, "split units come from the persistent queue");
  static_assert(!FRAMES || (BT == 128 && !SPLIT), "frame masks: 128-token blocks, whole items");
  using C = AttnCfg<D, BT>;
  __shared__ __attribute__((aligned(1024))) char sK[2][C::TILE];
  __shared__ __attribute__((aligned(1024))) char sV[2][C::TILE];
  // per key block: its number of real tokens (128-token blocks; smaller blocks
  // run two workgroups per CU and keep their LDS)
  constexpr bool BINFO = BT == 128;
  // (a real count fits a byte; with frame masks, nb * bt <= MAX_FRAME_KEYS, the
  // table holds the subtiles' frame ranges as well)
  using binfo_t = std::conditional_t<FRAMES, int, uint8_t>;
  __shared__ binfo_t s_binfo[BINFO ? (FRAMES ? MAX_FRAME_KEYS : MAX_NB) : 1];
  __shared__ int s_item;
  __shared__ int s_exact;   // some real query of the item needs the running maximum

  const Geo& g = a.g;
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int half = w / C::NW1, wq = w % C::NW1;   // query block of the pair, wave in block
  const int hf = lane >> 5, l32 = lane & 31;
  // 32-query subtile of this wave.  Waves w and w + NW1 share a SIMD; with four
  // subtiles per block the second block's waves take them rotated by two, so
  // that when a cut block has only its first subtiles real, the busy waves of
  // the pair sit on different SIMDs.
  const int qsub = C::NW1 == 4 ? (wq + 2 * half) & 3 : wq;
  auto block_info = [&](int j) {
    const int e = block_extent(g, j);
    return (e & 255) * ((e >> 8) & 255) * ((e >> 16) & 255);   // real tokens
  };
  // fine-grained routing: beside the real count (bits 0-7), for each 32-key
  // subtile t of the tile the first and last frame its real keys belong to
  // (3 bits each, at bit 8 + 6t)
  auto block_info_frames = [&](int j) {
    const int e = block_extent(g, j);
    const int fs = ((e >> 8) & 255) * ((e >> 16) & 255);   // real tokens per frame
    const int nreal = (e & 255) * fs;
    int info = nreal;
#pragma unroll
    for (int t = 0; t < 4; ++t)
      if (32 * t < nreal) {
        const int fa = (32 * t) / fs, fb = (min(32 * t + 32, nreal) - 1) / fs;
        info |= (fa | (fb << 3)) << (8 + 6 * t);
      }
    return info;
  };
  if constexpr (BINFO)
    for (int j = tid; j < g.nb; j += C::NT)
      s_binfo[j] = (binfo_t)(FRAMES ? block_info_frames(j) : block_info(j));
  // (the persistent loop clears it again before each item's first barrier)
  if (tid == 0) s_exact = 0;
  __syncthreads();

  const uint32_t sK_base = (uint32_t)(size_t)(__attribute__((address_space(3))) void*)&sK[0][0];
  const uint32_t sV_base = (uint32_t)(size_t)(__attribute__((address_space(3))) void*)&sV[0][0];
  // per-lane LDS byte offsets of the MFMA A operands (see the re-layout)
  const int kread = hf * (BT * 16) + l32 * 16;
  const int vread = hf * (D * 16) + l32 * 16;
  const long long t_start = (long long)wall_clock64();
  long long tiles = 0;

  // queue length: work items, or the split units (written by the prologue)
  const int qlen = SPLIT ? ld_scalar(a.counter, NUNITS) : g.groups;
  // claim of a queue position (thread 0 only); past the end: >= qlen
  auto pull = [&]() {
    if (a.xcd_local) {
      // own XCD's queue first, then steal from the others in turn
      const int x0 = (int)(xcc_id_reg() & (NXCD - 1));
      int found = g.groups;
      for (int k = 0; k < NXCD; ++k) {
        const int x = (x0 + k) & (NXCD - 1);
        const int q0 = a.counter[QOFF + x], q1 = a.counter[QOFF + x + 1];
        if (q0 == q1) continue;
        const int idx = atomicAdd(&a.counter[QHEAD + 32 * x], 1);
        if (q0 + idx < q1) { found = q0 + idx; break; }
      }
      return found;
    }
    return atomicAdd(a.counter, 1);
  };
  // the next position is claimed before the previous item's output stores, so
  // that its round trip overlaps them, and the workgroup meets at a barrier
  // that waits for LDS only: those stores stay in flight into the next item
  int claimed = 0;
  int iter = 0;
  while (true) {
    int item;
    if (PERSIST) {
      if (tid == 0) {
        s_item = iter == 0 ? pull() : claimed;
        s_exact = 0;
      }
      asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
      item = __builtin_amdgcn_readfirstlane(s_item);
      if (item >= qlen) break;
      item = ld_scalar(a.sched, item);
    } else {
      if (iter > 0) break;
      item = a.head_major ? (int)blockIdx.x : ld_scalar(a.sched, blockIdx.x);
    }
    ++iter;
    item = __builtin_amdgcn_readfirstlane(item);
    // split-and-merge: this unit covers entries [t0, t1) of the item's list and
    // writes its partial result to a slot (slot < 0: the whole item, final output)
    int t0 = 0, t1 = 0, slot = -1;
    if constexpr (SPLIT) {
      const int u = item;
      item = __builtin_amdgcn_readfirstlane(ld_scalar(a.units, 4l * u));
      t0 = __builtin_amdgcn_readfirstlane(ld_scalar(a.units, 4l * u + 1));
      t1 = __builtin_amdgcn_readfirstlane(ld_scalar(a.units, 4l * u + 2));
      slot = __builtin_amdgcn_readfirstlane(ld_scalar(a.units, 4l * u + 3));
    }

    const int bhh = item / g.groups_per_head, gl = item % g.groups_per_head;
    int lead, partner;
    group_blocks(g, gl, &lead, &partner);
    const int b = bhh / g.H, h = bhh % g.H;
    const long tok_base = (long)b * g.N;
    const int rA = bhh * g.nb + lead;
    const int rB = partner >= 0 ? bhh * g.nb + partner : -1;
    const int pA = ld_scalar(a.row_ptr, rA), nA = ld_scalar(a.row_ptr, rA + 1) - pA;
    const int pB = rB >= 0 ? ld_scalar(a.row_ptr, rB) : 0;
    const int nB = rB >= 0 ? ld_scalar(a.row_ptr, rB + 1) - pB : 0;
    const bool active = half == 0 || rB >= 0;     // this wave's query block exists
    const int iq = half == 0 ? lead : partner;
    const char* kc_head = (const char*)(a.kc + (long)bhh * g.nb * (D * BT));
    const char* vc_head = (const char*)(a.vc + (long)bhh * g.nb * (D * BT));

    // copies of the tile of union entry ent into buffer buf.  A short block
    // (flag bit 16) has real tokens only in its first 64-key chunk, the only
    // chunk the products read: the 1 KB copies that hold only keys of the second
    // chunk are skipped.  In Kc a KB is 64 keys of one d chunk, so with 128-key
    // tiles the odd waves copy only second-chunk keys; in Vc the second chunk
    // starts at round V2 (a whole round, for D = 64 and 128).
    auto issue = [&](int ent, int buf) {
      const int jblk = ent & 0xffff;
      constexpr bool SKIP = C::NCH == 2;   // 128-key tiles, two 64-key chunks
      constexpr int V2 = SKIP ? 8 * (D * 16) / (C::NW * 1024) : C::ROUNDS;
      static_assert(!SKIP || (BT * 16 == 2048 && (8 * D * 16) % (C::NW * 1024) == 0),
                    "second-chunk copies: odd K waves and whole V rounds");
      const bool short_blk = SKIP && ((ent >> 16) & 1) != 0;
      const char* ks = kc_head + (long)jblk * C::TILE;
      const char* vs = vc_head + (long)jblk * C::TILE;
      if (!(short_blk && (w & 1))) {
#pragma unroll
        for (int rr = 0; rr < C::ROUNDS; ++rr) {
          const int off = (rr * C::NW + w) * 1024;
          dma16(ks, off + lane * 16, sK_base + buf * C::TILE + off);
        }
      }
#pragma unroll
      for (int rr = 0; rr < C::ROUNDS; ++rr) {
        if (rr < V2 || !short_blk) {
          const int off = (rr * C::NW + w) * 1024;
          dma16(vs, off + lane * 16, sV_base + buf * C::TILE + off);
        }
      }
    };

    // walk over the item's precomputed union list, read two entries ahead
    const int* tl = a.tlist + (long)item * a.tlist_cap + t0;
    const int nt = SPLIT ? t1 - t0 : ld_scalar(a.tcount, item);
    if (nt > 0) issue(ld_scalar(tl, 0), 0);   // the first copy, ahead of the item set-up

    // largest key norm of the head (its loads in flight beside the Q loads)
    float kmx = 0.f;
    {
      const float* knh = a.kn + (long)bhh * g.nb;
      for (int base = 0; base < g.nb; base += 512) {
        float kv[8];
#pragma unroll
        for (int x = 0; x < 8; ++x) {
          const int t = base + lane + 64 * x;
          kv[x] = t < g.nb ? knh[t] : 0.f;
        }
#pragma unroll
        for (int x = 0; x < 8; ++x) kmx = fmaxf(kmx, kv[x]);
      }
    }

    // this lane's query slot (packed slot order, see packed_slot_offset)
    const int tq = iq / (g.nbh * g.nbw), hq = (iq / g.nbw) % g.nbh, wqb = iq % g.nbw;
    const int n0q = ((tq * g.bt) * g.Hg + hq * g.bh) * g.W + wqb * g.bw;
    const int extQ = block_extent(g, iq);
    const int HlQ = (extQ >> 8) & 255, WlQ = (extQ >> 16) & 255;
    const int nrealQ = (extQ & 255) * HlQ * WlQ;
    const int qs = 32 * qsub + l32;
    const bool qvalid = active && qs < nrealQ;
    const long nq = n0q + (qvalid ? packed_slot_offset(g, qs, HlQ, WlQ) : 0);
    const bool wave_has_q = __any(qvalid);   // some real query in this wave's 32 slots

    // Q^T as the B operand: lane holds 8 consecutive d of query slot qs
    bf16x8_t qop[C::KS];
    {
      const bf16_t* qrow = a.q + ((tok_base + nq) * g.H + h) * D + 8 * hf;
#pragma unroll
      for (int ks = 0; ks < C::KS; ++ks) {
        u32x4_t v = {0u, 0u, 0u, 0u};
        if (qvalid) v = *reinterpret_cast<const u32x4_t*>(qrow + 16 * ks);
        qop[ks] = __builtin_bit_cast(bf16x8_t, v);
      }
      // Consume the Q registers here so that the compiler waits for their
      // loads once per item and not at the top of every key-block iteration.
#pragma unroll
      for (int ks = 0; ks < C::KS; ++ks) asm volatile("" ::"v"(qop[ks]));
    }

    // Exponent range.  With c = log2(e)/sqrt(d), every score of query q in the
    // exp2 domain lies within B = c |q| max_j |k_j| of zero (Cauchy-Schwarz over
    // the head's keys; the norms are taken from the bf16 values in float32 and
    // rounded up, and B carries a relative 2^-10 margin for the products'
    // float32 sums).  When B <= 32 for every real query of the work item, the
    // probabilities exp2(c s) lie in [2^-32, 2^32], far inside bf16 and float
    // range, and the softmax needs no running maximum: the item is walked
    // against the reference 0 (the FAST walk).  Otherwise (or with NaN inputs)
    // it is walked with the lazily moved running maximum (the EXACT walk).  The
    // choice is the same for every part of a cut item (it depends on the
    // queries and the head only).
    {
      float q2 = 0.f;
#pragma unroll
      for (int ks = 0; ks < C::KS; ++ks)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float x = (float)qop[ks][e];
          q2 = fmaf(x, x, q2);
        }
      const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(q2), __float_as_uint(q2),
                                                       false, false);
      q2 = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
#pragma unroll
      for (int o2 = 1; o2 < 64; o2 <<= 1) kmx = fmaxf(kmx, __shfl_xor(kmx, o2));
      // (1 + 2^-7): the FAST walk multiplies the bf16 queries by c and rounds
      // them to bf16 again, which changes each by at most 2^-8 relative
      const float bound =
          a.c * (sqrtf(q2) * (1.0f + 0x1p-12f)) * kmx * ((1.0f + 0x1p-10f) * (1.0f + 0x1p-7f));
      if (__builtin_amdgcn_ballot_w64(qvalid && !(bound <= 32.0f)) != 0 && lane == 0) s_exact = 1;
    }
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    const bool exact_item = __builtin_amdgcn_readfirstlane(s_exact) != 0;
    bool any_kept = false;   // the wave's row keeps a block of the walk (wave-uniform)

    f32x16_t o[C::DSUB];
    float m_run = -INFINITY, l_run = 0.f;   // reference (score units) and sum

    // one walk over the item's union list, read two entries ahead
    auto walk = [&](auto exact_tag) __attribute__((always_inline)) {
      constexpr bool EXACT = decltype(exact_tag)::value;
      int e0 = nt > 0 ? ld_scalar(tl, 0) : -1;
      int e1 = nt > 1 ? ld_scalar(tl, 1) : -1;
      int e2 = nt > 2 ? ld_scalar(tl, 2) : -1;
#pragma unroll
      for (int u = 0; u < C::DSUB; ++u)
#pragma unroll
        for (int e = 0; e < 16; ++e) o[u][e] = 0.f;
      m_run = EXACT ? -INFINITY : 0.f;
      l_run = 0.f;
      int buf = 0;
      for (int t = 0; t < nt; ++t) {
        const int j = e0 & 0xffff;
        const bool mine = ((e0 >> (17 + half)) & 1) != 0;
        // fine-grained routing: this wave's row's kept frames of block j
        const int fmw = FRAMES ? (e0 >> (19 + 6 * half)) & 63 : 0;
        const int en = e1;
        if constexpr (SPLIT) tiles += ((e0 >> 17) & 1) + ((e0 >> 18) & 1);   // owned tiles
        any_kept = any_kept || mine;
        e0 = e1;
        e1 = e2;
        e2 = __builtin_amdgcn_readfirstlane(t + 3 < nt ? ld_scalar(tl, t + 3) : -1);

        wait_vmcnt<0>();      // this thread's copies of block j have landed
        wg_barrier();         // ... everyone's; and block j-1's buffer is free
        if (en >= 0) issue(en, buf ^ 1);

        if (mine && wave_has_q) {
          const int info = __builtin_amdgcn_readfirstlane(BINFO ? (int)s_binfo[j] : block_info(j));
          const int nreal = FRAMES ? (info & 255) : info;
          // fine-grained routing: fpart when this wave's row keeps only some of
          // the block's frames (the last real key's frame is the last frame); else
          // the tile runs as without frame masks
          bool fpart = false;
          if constexpr (FRAMES) {
            const int last = (info >> (11 + 6 * ((nreal - 1) >> 5))) & 7;
            fpart = fmw != (2 << last) - 1;
          }
          // kept frames among the real keys of subtiles ta..tb (ta <= tb, both
          // holding real keys): 2 all, 1 some, 0 none
          auto frames_in = [&](int ta, int tb) {
            const int fa = (info >> (8 + 6 * ta)) & 7, fb = (info >> (11 + 6 * tb)) & 7;
            const int m = ((2 << fb) - 1) & ~((1 << fa) - 1);
            return (fmw & m) == m ? 2 : ((fmw & m) != 0 ? 1 : 0);
          };
          const char* kb = sK[buf] + kread;
          const char* vb = sV[buf] + vread;
#pragma unroll
          for (int hc = 0; hc < C::NCH; ++hc) {
            // a chunk whose first slot lies beyond the block's real tokens holds
            // only padding keys: nothing to add
            if (hc * C::CHS * 32 >= nreal) continue;
            // fine-grained routing: a chunk none of whose real keys lies in a kept
            // frame of this wave's row adds nothing either
            if (FRAMES && fpart &&
                frames_in(hc * C::CHS, (hc * C::CHS + 1) * 32 < nreal ? hc * C::CHS + C::CHS - 1
                                                                       : hc * C::CHS) == 0)
              continue;
            // only when the chunk's second subtile holds real keys (of kept
            // frames) are its score and PV products run (else its scores are the
            // bias alone and its probabilities zero)
            bool two = C::CHS == 1 || (hc * C::CHS + 1) * 32 < nreal;
            if (FRAMES && fpart && two && C::CHS == 2) two = frames_in(hc * 2 + 1, hc * 2 + 1) != 0;
            // Waves w and w + NW1 share a SIMD and would otherwise run the same
            // phases in step.  Their priorities alternate: chunk by chunk, one
            // half leads the score products and the other the softmax and PV
            // products, so that neither trails the other into the tile barrier.
            const bool lead_qk = ((hc + half) & 1) != 0;
            if (lead_qk) __builtin_amdgcn_s_setprio(1); else __builtin_amdgcn_s_setprio(0);
            // ---- S^T = K Q^T for the CHS key subtiles of this chunk
            f32x16_t s[C::CHS];
            // K operands read from LDS 4 products ahead of use (the order of the
            // reads and products is pinned)
            constexpr int NQ = C::CHS * C::KS, PDK = 4 < NQ ? 4 : NQ;
            auto kaddr = [&](int i) {
              return reinterpret_cast<const bf16x8_t*>(kb + (i % C::KS) * (2 * BT * 16) +
                                                       (hc * C::CHS + i / C::KS) * 512);
            };
            bf16x8_t kf[PDK];
#pragma unroll
            for (int i = 0; i < PDK; ++i) kf[i] = *kaddr(i);
#pragma unroll
            for (int t2 = 0; t2 < C::CHS; ++t2) {
              const int t = hc * C::CHS + t2;
              // padding keys: add -1e30 through one extra k-step (bias column x ones row).
              // fmode (fine-grained routing): 1 also masks the keys of frames the
              // row does not keep, 2 masks every key of the subtile
              auto add_bias = [&](const f32x16_t& acc, int fmode) {
                bool ok = 32 * t + l32 < nreal;
                if (FRAMES && fmode == 2) ok = false;
                if (FRAMES && fmode == 1) {
                  const int e = block_extent(g, j);
                  const float fs = (float)(((e >> 8) & 255) * ((e >> 16) & 255));
                  // frame of the lane's key slot: floor((s + 1/2) / fs) is exact in
                  // float32 for slots and frame sizes below 256
                  const int f = (int)(((float)(32 * t + l32) + 0.5f) / fs);
                  ok = ok && ((fmw >> f) & 1);
                }
                bf16x8_t bias, ones;
#pragma unroll
                for (int e = 0; e < 8; ++e) { bias[e] = (__bf16)0.0f; ones[e] = (__bf16)0.0f; }
                if (hf == 0) ones[0] = (__bf16)1.0f;
                if (hf == 0 && !ok) bias[0] = (__bf16)(-1.0e30f);
                return __builtin_amdgcn_mfma_f32_32x32x16_bf16(bias, ones, acc, 0, 0, 0);
              };
              f32x16_t zero;
#pragma unroll
              for (int e = 0; e < 16; ++e) zero[e] = 0.f;
              if (t2 == 0 || two) {
                s[t2] = zero;
#pragma unroll
                for (int ks = 0; ks < C::KS; ++ks) {
                  const int i = t2 * C::KS + ks;
                  const bf16x8_t av = kf[i % PDK];
                  if (i + PDK < NQ) kf[i % PDK] = *kaddr(i + PDK);
                  s[t2] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, qop[ks], s[t2], 0, 0, 0);
                  __builtin_amdgcn_sched_barrier(0);
                }
                // only the subtile that holds the block's last real key also
                // holds padding keys (and, with frame masks, a subtile that
                // holds keys of a frame its row does not keep)
                const bool fsub = FRAMES && fpart && frames_in(t, t) != 2;
                if (32 * (t + 1) > nreal || fsub) s[t2] = add_bias(s[t2], fsub ? 1 : 0);
              } else {
                // padding keys only (or, with frame masks, keys of frames the row
                // does not keep): the scores are the bias alone
                s[t2] = add_bias(zero, 2);
              }
            }

            if (lead_qk) __builtin_amdgcn_s_setprio(0); else __builtin_amdgcn_s_setprio(1);
            bf16x8_t pop[2 * C::CHS];
            if constexpr (EXACT) {
              // ---- online softmax over the chunk's keys, per query column
              // four independent partial maxima (short dependency chains)
              float mq[4];
#pragma unroll
              for (int r = 0; r < 4; ++r) mq[r] = s[0][r];
#pragma unroll
              for (int t2 = 0; t2 < C::CHS; ++t2)
#pragma unroll
                for (int e = (t2 == 0 ? 4 : 0); e < 16; ++e) mq[e & 3] = vmax(mq[e & 3], s[t2][e]);
              float mt = vmax(vmax(mq[0], mq[1]), vmax(mq[2], mq[3]));
              {
                // the other half of the query column lives in lane l ^ 32
                const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(mt),
                                                                 __float_as_uint(mt), false, false);
                mt = vmax(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
              }
              // lazily moved reference: only when the chunk maximum exceeds it by
              // more than 8 in the exp2 domain (probabilities stay <= 2^8)
              const bool up = !((mt - m_run) * a.c <= 8.0f);   // also true while m_run = -inf
              const float m_new = up ? mt : m_run;
              const float alpha = up ? __builtin_amdgcn_exp2f((m_run - m_new) * a.c) : 1.0f;
              const float mc = m_new * a.c;
              float pq[4];   // four independent partial sums
#pragma unroll
              for (int t2 = 0; t2 < C::CHS; ++t2)
#pragma unroll
                for (int e = 0; e < 16; ++e) {
                  const float pv = __builtin_amdgcn_exp2f(fmaf(s[t2][e], a.c, -mc));
                  pq[e & 3] = t2 == 0 && e < 4 ? pv : pq[e & 3] + pv;
                  pop[2 * t2 + e / 8][e % 8] = (__bf16)pv;
                }
              const float psum = (pq[0] + pq[1]) + (pq[2] + pq[3]);
              l_run = l_run * alpha + psum;
              if (up) {
#pragma unroll
                for (int u = 0; u < C::DSUB; ++u)
#pragma unroll
                  for (int e = 0; e < 16; ++e) o[u][e] *= alpha;
              }
              m_run = m_new;
            } else {
              // ---- softmax against the reference 0 (see the exponent range above)
              float pq[4];   // four independent partial sums
#pragma unroll
              for (int t2 = 0; t2 < C::CHS; ++t2)
#pragma unroll
                for (int e = 0; e < 16; ++e) {
                  const float pv = __builtin_amdgcn_exp2f(s[t2][e]);
                  pq[e & 3] = t2 == 0 && e < 4 ? pv : pq[e & 3] + pv;
                  pop[2 * t2 + e / 8][e % 8] = (__bf16)pv;
                }
              l_run += (pq[0] + pq[1]) + (pq[2] + pq[3]);
            }

            // ---- O^T += Vt P^T over the chunk's keys, subtile by subtile (each
            // o[u] still sums its 16-key steps in order)
#pragma unroll
            for (int t2 = 0; t2 < C::CHS; ++t2) {
              if (t2 > 0 && !two) break;
#pragma unroll
              for (int u = 0; u < C::DSUB; ++u) {
#pragma unroll
                for (int st2 = 2 * t2; st2 < 2 * t2 + 2; ++st2) {
                  const int st = hc * 2 * C::CHS + st2;
                  const bf16x8_t av =
                      *reinterpret_cast<const bf16x8_t*>(vb + st * (2 * D * 16) + u * 512);
                  o[u] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, pop[st2], o[u], 0, 0, 0);
                }
              }
            }
          }
        }
        buf ^= 1;
      }
    };
    if (exact_item) {
      walk(std::true_type{});
    } else {
      // FAST walk: c folded into the Q operand, so the products give the
      // scores in the exp2 domain and each probability is one exp2
#pragma unroll
      for (int ks = 0; ks < C::KS; ++ks)
#pragma unroll
        for (int e = 0; e < 8; ++e) qop[ks][e] = (__bf16)((float)qop[ks][e] * a.c);
      walk(std::false_type{});
    }
    // the reference of O^T and the sum, exp2 domain (-inf: no key)
    const float m_out = exact_item ? m_run * a.c : (any_kept ? 0.f : -INFINITY);
    if constexpr (!SPLIT) tiles += nA + nB;
    if (PERSIST && tid == 0) claimed = pull();

    // ---- epilogue: normalise and store the real query rows
    const float l_tot = l_run + __shfl_xor(l_run, 32);
    const float inv = l_tot > 0.f ? 1.0f / l_tot : 0.f;
    if (SPLIT && slot >= 0) {
      // partial result of this part, every query slot of the pair: O^T relative
      // to the reference m (not normalised), m in the exp2 domain, and the sum
      float* ps = a.part + (long)slot * a.part_floats;
      const int qi = half * BT + qs;
      float* prow = ps + (long)qi * D + 4 * hf;
#pragma unroll
      for (int u = 0; u < C::DSUB; ++u)
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4)
          *reinterpret_cast<float4*>(prow + 32 * u + 8 * g4) =
              make_float4(o[u][4 * g4 + 0], o[u][4 * g4 + 1], o[u][4 * g4 + 2], o[u][4 * g4 + 3]);
      if (hf == 0) {
        ps[2 * BT * D + qi] = m_out;
        ps[2 * BT * D + 2 * BT + qi] = l_tot;
      }
    } else if (qvalid) {
      bf16_t* orow = a.o + ((tok_base + nq) * g.H + h) * D + 4 * hf;
#pragma unroll
      for (int u = 0; u < C::DSUB; ++u)
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          __bf16 v0 = (__bf16)(o[u][4 * g4 + 0] * inv), v1 = (__bf16)(o[u][4 * g4 + 1] * inv);
          __bf16 v2 = (__bf16)(o[u][4 * g4 + 2] * inv), v3 = (__bf16)(o[u][4 * g4 + 3] * inv);
          const uint32_t w0 = (uint32_t)__builtin_bit_cast(uint16_t, v0) |
                              ((uint32_t)__builtin_bit_cast(uint16_t, v1) << 16);
          const uint32_t w1 = (uint32_t)__builtin_bit_cast(uint16_t, v2) |
                              ((uint32_t)__builtin_bit_cast(uint16_t, v3) << 16);
          *reinterpret_cast<uint2*>(orow + 32 * u + 8 * g4) = make_uint2(w0, w1);
        }
    }
    if (PERSIST) __syncthreads();  // s_item is rewritten by the next pull
  }
  if (tid == 0 && a.telem) {
    long long* t = a.telem + (long)blockIdx.x * 4;
    t[0] = (long long)hw_id_reg();
    t[1] = (long long)xcc_id_reg();
    t[2] = tiles;
    t[3] = (long long)wall_clock64() - t_start;
  }
}

// ---------------------------------------------------------------------------
// Merge of the parts of every cut work item.  Part p left, per query,
// O_p = sum over its keys of 2^(c s - m_p) v, its sum l_p and its reference
// m_p (exp2 domain, -inf when the part had no key of the query's row).  With
// M = max_p m_p and weights w_p = 2^(m_p - M), the softmax over the union of
// the parts' keys is
//   O = (sum_p w_p O_p) / (sum_p w_p l_p),
// the same log-sum-exp combination as merging attention computed over
// disjoint key sets.  Parts are combined in ascending order, so the result does
// not depend on the schedule.  Workgroup x = (cut item, chunk of 256 float4
// columns of the item's 2 Bt x d output); one thread per 4 consecutive d of one
// query, so every load of a workgroup is in flight at once.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void merge_parts_kernel(Geo g, const int* __restrict__ stab,
                                                          const int* __restrict__ counter,
                                                          const float* __restrict__ part,
                                                          long pf, int chunks,
                                                          bf16_t* __restrict__ o) {
  const int sidx = blockIdx.x / chunks, chunk = blockIdx.x % chunks;
  if (sidx >= counter[NSPLIT]) return;
  const int BT = g.Bt, D = g.d, C4 = D / 4;
  const int f = chunk * 256 + threadIdx.x;
  if (f >= 2 * BT * C4) return;
  const int item = stab[4 * sidx], slot0 = stab[4 * sidx + 1], P = stab[4 * sidx + 2];
  const int bhh = item / g.groups_per_head, gl = item % g.groups_per_head;
  int lead, partner;
  group_blocks(g, gl, &lead, &partner);
  const int qi = f / C4, c4 = f % C4;
  const int half = qi / BT, qs = qi % BT;
  const int blk = half ? partner : lead;
  if (blk < 0) return;
  const int tb = blk / (g.nbh * g.nbw), hb = (blk / g.nbw) % g.nbh, wb = blk % g.nbw;
  const int ext = block_extent(g, blk);
  const int Hl = (ext >> 8) & 255, Wl = (ext >> 16) & 255;
  if (qs >= (ext & 255) * Hl * Wl) return;   // padding slot: no output
  const long n = ((long)(tb * g.bt) * g.Hg + hb * g.bh) * g.W + wb * g.bw +
                 packed_slot_offset(g, qs, Hl, Wl);
  const int b = bhh / g.H, h = bhh % g.H;
  const float* base = part + (long)slot0 * pf;
  const long mo = 2l * BT * D, lo = mo + 2 * BT;
  float M = -INFINITY;
  for (int p = 0; p < P; ++p) M = fmaxf(M, base[p * pf + mo + qi]);
  float L = 0.f;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  if (M > -INFINITY) {
    for (int p = 0; p < P; ++p) {
      const float* sp = base + p * pf;
      const float wgt = __builtin_amdgcn_exp2f(sp[mo + qi] - M);
      L = fmaf(wgt, sp[lo + qi], L);
      const float4 v = *reinterpret_cast<const float4*>(sp + (long)qi * D + 4 * c4);
      acc.x = fmaf(wgt, v.x, acc.x);
      acc.y = fmaf(wgt, v.y, acc.y);
      acc.z = fmaf(wgt, v.z, acc.z);
      acc.w = fmaf(wgt, v.w, acc.w);
    }
  }
  const float inv = L > 0.f ? 1.0f / L : 0.f;
  const __bf16 v0 = (__bf16)(acc.x * inv), v1 = (__bf16)(acc.y * inv);
  const __bf16 v2 = (__bf16)(acc.z * inv), v3 = (__bf16)(acc.w * inv);
  const uint32_t w0 = (uint32_t)__builtin_bit_cast(uint16_t, v0) |
                      ((uint32_t)__builtin_bit_cast(uint16_t, v1) << 16);
  const uint32_t w1 = (uint32_t)__builtin_bit_cast(uint16_t, v2) |
                      ((uint32_t)__builtin_bit_cast(uint16_t, v3) << 16);
  *reinterpret_cast<uint2*>(o + (((long)b * g.N + n) * g.H + h) * D + 4 * c4) =
      make_uint2(w0, w1);
}

// ---------------------------------------------------------------------------
// float32 block-sparse attention (scalar FMA path, tiny and fp32 workloads):
// one workgroup per item, one thread per query slot, keys in chunks of 32.
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(128) void attn_f32_kernel(Geo g, const float* __restrict__ q,
                                                       const float* __restrict__ k,
                                                       const float* __restrict__ v,
                                                       const int* __restrict__ row_ptr,
                                                       const int* __restrict__ col_idx,
                                                       const int* __restrict__ sched,
                                                       int head_major, float* __restrict__ o,
                                                       long long* __restrict__ telem,
                                                       float scale) {
  __shared__ float sk[32][D + 1];
  __shared__ float sv[32][D];
  __shared__ int kval[32];
  const long long t_start = (long long)wall_clock64();
  const int r = (int)blockIdx.x;  // rows in natural order (small float32 workloads)
  (void)sched;
  (void)head_major;
  const int bhh = r / g.nb, iq = r % g.nb;
  const int b = bhh / g.H, h = bhh % g.H;
  const int plane = g.bh * g.bw;
  auto tok = [&](int blk, int s, bool* ok) -> long {
    const int tb = blk / (g.nbh * g.nbw), hb = (blk / g.nbw) % g.nbh, wb = blk % g.nbw;
    const int st = s / plane, sh = (s / g.bw) % g.bh, sw = s % g.bw;
    const int t = tb * g.bt + st, hh = hb * g.bh + sh, ww = wb * g.bw + sw;
    *ok = t < g.T && hh < g.Hg && ww < g.W;
    return ((long)t * g.Hg + hh) * g.W + ww;
  };
  const int qs = threadIdx.x;
  bool qok = false;
  long nq = 0;
  if (qs < g.Bt) nq = tok(iq, qs, &qok);
  float qv[D], acc[D];
#pragma unroll
  for (int x = 0; x < D; ++x) {
    qv[x] = qok ? q[(((long)b * g.N + nq) * g.H + h) * D + x] * scale : 0.f;
    acc[x] = 0.f;
  }
  float m_run = -INFINITY, l_run = 0.f;
  const int rp0 = row_ptr[r], rp1 = row_ptr[r + 1];
  for (int jj = rp0; jj < rp1; ++jj) {
    const int j = col_idx[jj];
    for (int k0 = 0; k0 < g.Bt; k0 += 32) {
      __syncthreads();
      for (int e = threadIdx.x; e < 32 * D; e += 128) {
        const int kk = e / D, x = e % D;
        bool ok = false;
        long n = 0;
        if (k0 + kk < g.Bt) n = tok(j, k0 + kk, &ok);
        const long off = (((long)b * g.N + n) * g.H + h) * D + x;
        sk[kk][x] = ok ? k[off] : 0.f;
        sv[kk][x] = ok ? v[off] : 0.f;
        if (x == 0) kval[kk] = ok ? 1 : 0;
      }
      __syncthreads();
      float sc[32];
      float mt = -INFINITY;
      for (int kk = 0; kk < 32; ++kk) {
        float d = 0.f;
#pragma unroll
        for (int x = 0; x < D; ++x) d = fmaf(qv[x], sk[kk][x], d);
        sc[kk] = kval[kk] ? d : -INFINITY;
        mt = fmaxf(mt, sc[kk]);
      }
      const float m_new = fmaxf(m_run, mt);
      if (m_new == -INFINITY) continue;
      const float alpha = expf(m_run - m_new);
      l_run *= alpha;
#pragma unroll
      for (int x = 0; x < D; ++x) acc[x] *= alpha;
      for (int kk = 0; kk < 32; ++kk) {
        const float pw = expf(sc[kk] - m_new);
        l_run += pw;
#pragma unroll
        for (int x = 0; x < D; ++x) acc[x] = fmaf(pw, sv[kk][x], acc[x]);
      }
      m_run = m_new;
    }
  }
  if (qok) {
    const float inv = 1.0f / l_run;
#pragma unroll
    for (int x = 0; x < D; ++x) o[(((long)b * g.N + nq) * g.H + h) * D + x] = acc[x] * inv;
  }
  if (threadIdx.x == 0 && telem) {
    long long* t = telem + (long)blockIdx.x * 4;
    t[0] = (long long)hw_id_reg();
    t[1] = (long long)xcc_id_reg();
    t[2] = rp1 - rp0;
    t[3] = (long long)wall_clock64() - t_start;
  }
}

// ---------------------------------------------------------------------------
// Launchers
// ---------------------------------------------------------------------------
template <int D, int BT>
static void launch_relayout(const Geo& g, const void* k, const void* v, bf16_t* kc, bf16_t* vc,
                            float* kn, hipStream_t s) {
  hipLaunchKernelGGL((kv_relayout_kernel<D, BT>), dim3(g.nb, g.B * g.H, 2), dim3(256), 0, s, g,
                     (const bf16_t*)k, (const bf16_t*)v, kc, vc, kn);
}

static void launch_relayout_bf16(const Geo& g, const void* k, const void* v, char* ws,
                                 const AttendWs& L, hipStream_t s) {
  bf16_t* kc = (bf16_t*)(ws + L.kc);
  bf16_t* vc = (bf16_t*)(ws + L.vc);
  float* kn = (float*)(ws + L.kn);
  if (g.d == 128) {
    if (g.Bt == 128) launch_relayout<128, 128>(g, k, v, kc, vc, kn, s);
    else if (g.Bt == 64) launch_relayout<128, 64>(g, k, v, kc, vc, kn, s);
    else launch_relayout<128, 32>(g, k, v, kc, vc, kn, s);
  } else {
    if (g.Bt == 128) launch_relayout<64, 128>(g, k, v, kc, vc, kn, s);
    else if (g.Bt == 64) launch_relayout<64, 64>(g, k, v, kc, vc, kn, s);
    else launch_relayout<64, 32>(g, k, v, kc, vc, kn, s);
  }
}

hipError_t launch_attend_relayout(const Geo& g, int dtype, const void* k, const void* v,
                                  char* ws, const AttendWs& L, hipStream_t s) {
  if (dtype == ABS_BF16) {
    launch_relayout_bf16(g, k, v, ws, L, s);
  } else {
    // float32 path: the attention kernel reads V token-major from the workspace
    const size_t bytes = (size_t)g.B * g.N * g.H * g.d * sizeof(float);
    hipError_t e = hipMemcpyAsync(ws + L.vc, v, bytes, hipMemcpyDeviceToDevice, s);
    if (e != hipSuccess) return e;
  }
  return hipGetLastError();
}

hipError_t launch_attend_prepare(const Geo& g, int dtype, const void* k, const void* v,
                                 const abs_mask* mask, int sched, int heads_per_phase, char* ws,
                                 const AttendWs& L, hipStream_t s) {
  hipError_t e = launch_attend_relayout(g, dtype, k, v, ws, L, s);
  if (e != hipSuccess) return e;
  return launch_attend_schedule(g, dtype, mask, sched, heads_per_phase, ws, L, s);
}

hipError_t launch_attend_schedule(const Geo& g, int dtype, const abs_mask* mask, int sched,
                                  int heads_per_phase, char* ws, const AttendWs& L,
                                  hipStream_t s, const int* frame_mask) {
  if (dtype == ABS_BF16 && frame_mask)
    hipLaunchKernelGGL(tile_list_kernel<true>, dim3(g.groups), dim3(256), 0, s, g, mask->row_ptr,
                       mask->col_idx, tlist_cap(g), (int*)(ws + L.tlist), (int*)(ws + L.tcount),
                       (int*)(ws + L.icost), frame_mask);
  else if (dtype == ABS_BF16)
    hipLaunchKernelGGL(tile_list_kernel<false>, dim3(g.groups), dim3(256), 0, s, g, mask->row_ptr,
                       mask->col_idx, tlist_cap(g), (int*)(ws + L.tlist), (int*)(ws + L.tcount),
                       (int*)(ws + L.icost), (const int*)nullptr);
  // head-phased work items: one workgroup per phase
  const int grid = sched == ABS_SCHED_HEAD_PHASED
                       ? (g.B * g.H + heads_per_phase - 1) / heads_per_phase : 1;
  hipLaunchKernelGGL(schedule_kernel, dim3(grid), dim3(512), 0, s, g, mask->row_ptr, sched,
                     heads_per_phase, (int*)(ws + L.sched), (int*)(ws + L.sort_a),
                     (int*)(ws + L.sort_b), (int*)(ws + L.counter), (const int*)nullptr,
                     dtype == ABS_BF16 ? (const int*)(ws + L.icost) : (const int*)nullptr);
  return hipGetLastError();
}

hipError_t launch_attend_prepare_split(const Geo& g, const void* k, const void* v,
                                       const abs_mask* mask, int sched, int heads_per_phase,
                                       int split_tiles, int max_parts, char* ws,
                                       const AttendWs& L, hipStream_t s) {
  launch_relayout_bf16(g, k, v, ws, L, s);
  hipLaunchKernelGGL(tile_list_kernel<false>, dim3(g.groups), dim3(256), 0, s, g, mask->row_ptr,
                     mask->col_idx, tlist_cap(g), (int*)(ws + L.tlist), (int*)(ws + L.tcount),
                     (int*)(ws + L.icost), (const int*)nullptr);
  hipLaunchKernelGGL(split_units_kernel, dim3(1), dim3(1024), 0, s, g, (const int*)(ws + L.tcount),
                     split_tiles, max_parts, (int4*)(ws + L.units), (int4*)(ws + L.stab),
                     (int*)(ws + L.counter));
  hipLaunchKernelGGL(schedule_kernel, dim3(1), dim3(512), 0, s, g, mask->row_ptr, sched,
                     heads_per_phase, (int*)(ws + L.sched), (int*)(ws + L.sort_a),
                     (int*)(ws + L.sort_b), (int*)(ws + L.counter), (const int*)(ws + L.units),
                     (const int*)(ws + L.icost));
  return hipGetLastError();
}

template <int D, int BT>
static int persistent_grid() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  static int cache_cu[64] = {0};
  static int cache_occ[64][6] = {{0}};
  int cu = dev < 64 ? __atomic_load_n(&cache_cu[dev], __ATOMIC_RELAXED) : 0;
  if (cu == 0) {
    if (hipDeviceGetAttribute(&cu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
      return 0;
    if (dev < 64) __atomic_store_n(&cache_cu[dev], cu, __ATOMIC_RELAXED);
  }
  const int slot = (D == 128 ? 0 : 3) + (BT == 128 ? 0 : (BT == 64 ? 1 : 2));
  int occ = dev < 64 ? __atomic_load_n(&cache_occ[dev][slot], __ATOMIC_RELAXED) : 0;
  if (occ == 0) {
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(
            &occ, reinterpret_cast<const void*>(&attn_bf16_kernel<D, BT, true>), 4 * BT, 0) !=
            hipSuccess ||
        occ < 1)
      occ = 1;
    if (dev < 64) __atomic_store_n(&cache_occ[dev][slot], occ, __ATOMIC_RELAXED);
  }
  return cu * occ;
}

int attend_grid(const Geo& g, int dtype, int sched) {
  if (dtype != ABS_BF16) return g.rows;           // float32: one workgroup per row
  if (sched == ABS_SCHED_HEAD_MAJOR) return g.groups;
  if (g.d == 128) {
    if (g.Bt == 128) return persistent_grid<128, 128>();
    if (g.Bt == 64) return persistent_grid<128, 64>();
    return persistent_grid<128, 32>();
  }
  if (g.Bt == 128) return persistent_grid<64, 128>();
  if (g.Bt == 64) return persistent_grid<64, 64>();
  return persistent_grid<64, 32>();
}

template <int D, int BT, bool FR = false>
static void launch_bf16(const AttnArgs& a, bool persist, int grid, hipStream_t s) {
  if (persist)
    hipLaunchKernelGGL((attn_bf16_kernel<D, BT, true, false, FR>), dim3(grid), dim3(4 * BT), 0, s,
                       a);
  else
    hipLaunchKernelGGL((attn_bf16_kernel<D, BT, false, false, FR>), dim3(grid), dim3(4 * BT), 0,
                       s, a);
}

template <int D, int BT>
static void launch_bf16_split(const AttnArgs& a, int grid, hipStream_t s) {
  hipLaunchKernelGGL((attn_bf16_kernel<D, BT, true, true>), dim3(grid), dim3(4 * BT), 0, s, a);
}

hipError_t launch_attend_run(const Geo& g, int dtype, const void* q, const void* k,
                             const abs_mask* mask, void* o, int sched, char* ws,
                             const AttendWs& L, int64_t* telemetry, int grid, hipStream_t s,
                             bool frames) {
  const int* sch = (const int*)(ws + L.sched);
  const bool head_major = sched == ABS_SCHED_HEAD_MAJOR;
  if (dtype == ABS_BF16) {
    AttnArgs a = {};
    a.g = g;
    a.q = (const bf16_t*)q;
    a.kc = (const bf16_t*)(ws + L.kc);
    a.vc = (const bf16_t*)(ws + L.vc);
    a.row_ptr = mask->row_ptr;
    a.col_idx = mask->col_idx;
    a.sched = sch;
    a.counter = (int*)(ws + L.counter);
    a.o = (bf16_t*)o;
    a.telem = (long long*)telemetry;
    a.c = (float)(1.4426950408889634 / sqrt((double)g.d));
    a.head_major = head_major ? 1 : 0;
    const bool persist = !head_major;
    a.xcd_local = sched == ABS_SCHED_XCD_LOCAL ? 1 : 0;
    a.tlist = (const int*)(ws + L.tlist);
    a.kn = (const float*)(ws + L.kn);
    a.tcount = (const int*)(ws + L.tcount);
    a.tlist_cap = tlist_cap(g);
    if (persist) hipLaunchKernelGGL(reset_counter_kernel, dim3(1), dim3(64), 0, s, a.counter);
    if (frames) {
      if (g.d == 128) launch_bf16<128, 128, true>(a, persist, grid, s);
      else launch_bf16<64, 128, true>(a, persist, grid, s);
    } else if (g.d == 128) {
      if (g.Bt == 128) launch_bf16<128, 128>(a, persist, grid, s);
      else if (g.Bt == 64) launch_bf16<128, 64>(a, persist, grid, s);
      else launch_bf16<128, 32>(a, persist, grid, s);
    } else {
      if (g.Bt == 128) launch_bf16<64, 128>(a, persist, grid, s);
      else if (g.Bt == 64) launch_bf16<64, 64>(a, persist, grid, s);
      else launch_bf16<64, 32>(a, persist, grid, s);
    }
  } else {
    const float scale = (float)(1.0 / sqrt((double)g.d));
    if (g.d == 128)
      hipLaunchKernelGGL(attn_f32_kernel<128>, dim3(g.rows), dim3(128), 0, s, g, (const float*)q,
                         (const float*)k, (const float*)(ws + L.vc), mask->row_ptr, mask->col_idx,
                         sch, head_major ? 1 : 0, (float*)o, (long long*)telemetry, scale);
    else
      hipLaunchKernelGGL(attn_f32_kernel<64>, dim3(g.rows), dim3(128), 0, s, g, (const float*)q,
                         (const float*)k, (const float*)(ws + L.vc), mask->row_ptr, mask->col_idx,
                         sch, head_major ? 1 : 0, (float*)o, (long long*)telemetry, scale);
  }
  return hipGetLastError();
}

hipError_t launch_attend_run_split(const Geo& g, const void* q, const abs_mask* mask, void* o,
                                   int max_parts, char* ws, const AttendWs& L,
                                   int64_t* telemetry, int grid, hipStream_t s) {
  AttnArgs a = {};
  a.g = g;
  a.q = (const bf16_t*)q;
  a.kc = (const bf16_t*)(ws + L.kc);
  a.vc = (const bf16_t*)(ws + L.vc);
  a.row_ptr = mask->row_ptr;
  a.col_idx = mask->col_idx;
  a.sched = (const int*)(ws + L.sched);
  a.counter = (int*)(ws + L.counter);
  a.o = (bf16_t*)o;
  a.telem = (long long*)telemetry;
  a.c = (float)(1.4426950408889634 / sqrt((double)g.d));
  a.tlist = (const int*)(ws + L.tlist);
  a.kn = (const float*)(ws + L.kn);
  a.tcount = (const int*)(ws + L.tcount);
  a.tlist_cap = tlist_cap(g);
  a.units = (const int*)(ws + L.units);
  a.part = (float*)(ws + L.part);
  a.part_floats = (long)part_floats(g);
  hipLaunchKernelGGL(reset_counter_kernel, dim3(1), dim3(64), 0, s, a.counter);
  if (g.d == 128) {
    if (g.Bt == 128) launch_bf16_split<128, 128>(a, grid, s);
    else if (g.Bt == 64) launch_bf16_split<128, 64>(a, grid, s);
    else launch_bf16_split<128, 32>(a, grid, s);
  } else {
    if (g.Bt == 128) launch_bf16_split<64, 128>(a, grid, s);
    else if (g.Bt == 64) launch_bf16_split<64, 64>(a, grid, s);
    else launch_bf16_split<64, 32>(a, grid, s);
  }
  // every cut item has at least two parts
  const long most = (long)max_parts / 2 < (long)g.groups ? (long)max_parts / 2 : (long)g.groups;
  const int chunks = (2 * g.Bt * (g.d / 4) + 255) / 256;
  if (most > 0)
    hipLaunchKernelGGL(merge_parts_kernel, dim3((unsigned)(most * chunks)), dim3(256), 0, s, g,
                       (const int*)(ws + L.stab), (const int*)(ws + L.counter),
                       (const float*)(ws + L.part), (long)part_floats(g), chunks, (bf16_t*)o);
  return hipGetLastError();
}

}  // namespace abs_impl
