// Routing kernels: 3D-block mean pooling, pooled block scores, per-row Top-p
// selection with a Top-k floor and own-block repair, per-head slack fill, and
// CSR compaction.  Source: FVAttn explainer ("FVAttn: adaptive sparse
// attention with runtime load balancing, for video generation"), "Core method"
// part 1 (sparse-routing frontend) and part 3 (slack-aware augmentation).
#include <hip/hip_runtime.h>

#include <math.h>

#include "device_common.h"
#include "internal.h"

namespace abs_impl {

// ---------------------------------------------------------------------------
// Pooling: mean of Q and K over the real tokens of each 3D block (the cheap
// approximate similarity the routing runs on, explainer "Highlights and
// limitations").  One workgroup per (block, batch*head); 16-byte coalesced
// loads of each token's d-vector; float32 sums in a fixed order.
// ---------------------------------------------------------------------------
template <typename T, int D>
__global__ __launch_bounds__(256) void pool_kernel(Geo g, const T* __restrict__ q,
                                                   const T* __restrict__ k,
                                                   float* __restrict__ qp,
                                                   float* __restrict__ kp) {
  constexpr int E = Chunk<T>::E;   // elements per 16-byte chunk
  constexpr int C = D / E;         // chunks per token row
  constexpr int G = 256 / C;       // token groups
  __shared__ float red[G][D];
  const int blk = blockIdx.x, bh = blockIdx.y;
  const int b = bh / g.H, h = bh % g.H;
  const int tb = blk / (g.nbh * g.nbw), hb = (blk / g.nbw) % g.nbh, wb = blk % g.nbw;
  const int Tl = min(g.bt, g.T - tb * g.bt), Hl = min(g.bh, g.Hg - hb * g.bh),
            Wl = min(g.bw, g.W - wb * g.bw);
  const float inv = 1.0f / (float)(Tl * Hl * Wl);
  const int c = threadIdx.x % C, grp = threadIdx.x / C;
  const int plane = g.bh * g.bw;
#pragma unroll 1
  for (int which = 0; which < 2; ++which) {
    const T* src = which == 0 ? q : k;
    float* dst = which == 0 ? qp : kp;
    float acc[E];
#pragma unroll
    for (int e = 0; e < E; ++e) acc[e] = 0.f;
    // every load of this thread is issued before the first sum (the slots a
    // thread visits are at most 128 / G); padding slots contribute zeros, and
    // the sums run in slot order
    constexpr int MAXIT = 128 / G;
    uint4 raw[MAXIT];
#pragma unroll
    for (int it = 0; it < MAXIT; ++it) {
      const int s = grp + it * G;
      raw[it] = make_uint4(0u, 0u, 0u, 0u);
      const int st = s / plane, sh = (s / g.bw) % g.bh, sw = s % g.bw;
      if (s < g.Bt && st < Tl && sh < Hl && sw < Wl) {
        const long n = ((long)(tb * g.bt + st) * g.Hg + hb * g.bh + sh) * g.W + wb * g.bw + sw;
        raw[it] = *reinterpret_cast<const uint4*>(src + (((long)b * g.N + n) * g.H + h) * D + c * E);
      }
    }
#pragma unroll
    for (int it = 0; it < MAXIT; ++it) {
      float v[E];
      Chunk<T>::unpack(raw[it], v);
#pragma unroll
      for (int e = 0; e < E; ++e) acc[e] += v[e];
    }
#pragma unroll
    for (int e = 0; e < E; ++e) red[grp][c * E + e] = acc[e];
    __syncthreads();
    for (int dd = threadIdx.x; dd < D; dd += 256) {
      float s = 0.f;
      for (int gg = 0; gg < G; ++gg) s += red[gg][dd];
      dst[((long)bh * g.nb + blk) * D + dd] = s * inv;
    }
    __syncthreads();
  }
}

// ---------------------------------------------------------------------------
// Pooled block scores S[b,h,i,j] = Qp_i . Kp_j / sqrt(d), float32.  64x64
// output tile per workgroup, 4x4 per thread, d consumed in slices of 32.
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(256) void scores_kernel(Geo g, const float* __restrict__ qp,
                                                     const float* __restrict__ kp,
                                                     float* __restrict__ score, float scale) {
  __shared__ float As[32][64 + 4];
  __shared__ float Bs[32][64 + 4];
  const int bh = blockIdx.z;
  const int i0 = blockIdx.y * 64, j0 = blockIdx.x * 64;
  const int tx = threadIdx.x % 16, ty = threadIdx.x / 16;
  const float* Q = qp + (long)bh * g.nb * D;
  const float* K = kp + (long)bh * g.nb * D;
  float acc[4][4];
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int c = 0; c < 4; ++c) acc[a][c] = 0.f;
  for (int d0 = 0; d0 < D; d0 += 32) {
    // 64 rows x 32 columns of each operand, stored transposed (d-major)
    for (int e = threadIdx.x; e < 64 * 32; e += 256) {
      const int r = e / 32, dd = e % 32;
      As[dd][r] = (i0 + r < g.nb) ? Q[(long)(i0 + r) * D + d0 + dd] : 0.f;
      Bs[dd][r] = (j0 + r < g.nb) ? K[(long)(j0 + r) * D + d0 + dd] : 0.f;
    }
    __syncthreads();
#pragma unroll 8
    for (int dd = 0; dd < 32; ++dd) {
      float a[4], bb[4];
#pragma unroll
      for (int x = 0; x < 4; ++x) { a[x] = As[dd][ty * 4 + x]; bb[x] = Bs[dd][tx * 4 + x]; }
#pragma unroll
      for (int x = 0; x < 4; ++x)
#pragma unroll
        for (int y = 0; y < 4; ++y) acc[x][y] = fmaf(a[x], bb[y], acc[x][y]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int x = 0; x < 4; ++x) {
    const int i = i0 + ty * 4 + x;
    if (i >= g.nb) continue;
#pragma unroll
    for (int y = 0; y < 4; ++y) {
      const int j = j0 + tx * 4 + y;
      if (j < g.nb) score[((long)bh * g.nb + i) * g.nb + j] = acc[x][y] * scale;
    }
  }
}

// ---------------------------------------------------------------------------
// Per-row selection.  P = softmax of the score row; blocks sorted by
// (P descending, index ascending) with a bitonic sort of 64-bit keys in LDS;
// an inclusive scan of the sorted masses finds m, the smallest count reaching
// p; keep the first min(nb, max(m, k_floor)) blocks plus the own block.
// Output: the row's kept-block bitmap and count (and P, for the slack fill).
// ---------------------------------------------------------------------------
template <int NBP>
__global__ __launch_bounds__(256) void select_kernel(Geo g, float* __restrict__ score,
                                                     uint32_t* __restrict__ bitmap,
                                                     int* __restrict__ count, float p,
                                                     int k_floor, int write_prob) {
  constexpr int NT = 256;
  __shared__ unsigned long long keys[NBP];
  __shared__ float ev[NBP];
  __shared__ uint32_t bits[NBP / 32];
  __shared__ float ftmp[NT / 64 + 1];
  __shared__ int itmp[NT / 64 + 1];
  const int row = blockIdx.x;
  const int nb = g.nb;
  const int i = row % nb;
  float* srow = score + (long)row * nb;

  float mx = -INFINITY;
  for (int j = threadIdx.x; j < nb; j += NT) mx = fmaxf(mx, srow[j]);
  mx = block_max<NT>(mx, ftmp);
  float part = 0.f;
  for (int j = threadIdx.x; j < nb; j += NT) {
    const float e = expf(srow[j] - mx);
    ev[j] = e;
    part += e;
  }
  const float z = block_sum<NT>(part, ftmp);
  for (int j = threadIdx.x; j < NBP; j += NT) {
    unsigned long long key = ~0ull;
    if (j < nb) {
      const float pj = ev[j] / z;
      if (write_prob) srow[j] = pj;
      key = ((unsigned long long)(~__float_as_uint(pj)) << 32) | (unsigned)j;
    }
    keys[j] = key;
  }
  for (int w = threadIdx.x; w < NBP / 32; w += NT) bits[w] = 0u;
  __syncthreads();

  // bitonic sort, ascending keys = P descending then index ascending
  for (int size = 2; size <= NBP; size <<= 1) {
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      for (int t = threadIdx.x; t < NBP / 2; t += NT) {
        const int lo = 2 * t - (t & (stride - 1));
        const int hi = lo + stride;
        const bool up = (lo & size) == 0;
        const unsigned long long a = keys[lo], c = keys[hi];
        if ((a > c) == up) { keys[lo] = c; keys[hi] = a; }
      }
      __syncthreads();
    }
  }

  // inclusive scan of the sorted masses; first position reaching p
  constexpr int PER = (NBP + NT - 1) / NT;
  const int r0 = threadIdx.x * PER;
  float loc[PER];
  float run = 0.f;
#pragma unroll
  for (int e = 0; e < PER; ++e) {
    const int r = r0 + e;
    const float v = (r < nb) ? __uint_as_float(~(uint32_t)(keys[r] >> 32)) : 0.f;
    run += v;
    loc[e] = run;
  }
  float tot;
  const float pre = block_exclusive_scan<NT>(run, ftmp, &tot);
  int first = nb;  // count m (1-based) of the first prefix reaching p
#pragma unroll
  for (int e = PER - 1; e >= 0; --e) {
    const int r = r0 + e;
    if (r < nb && pre + loc[e] >= p) first = r + 1;
  }
  first = -first;
  {
    int x = first;
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) x = max(x, __shfl_xor(x, o));
    if ((threadIdx.x & 63) == 0) itmp[threadIdx.x >> 6] = x;
    __syncthreads();
    int r = itmp[0];
#pragma unroll
    for (int w = 1; w < NT / 64; ++w) r = max(r, itmp[w]);
    first = -r;
  }
  const int m = (p >= 1.0f) ? nb : first;
  const int m2 = min(nb, max(m, k_floor));
  for (int r = threadIdx.x; r < m2; r += NT) {
    const int j = (int)(keys[r] & 0xffffffffu);
    atomicOr(&bits[j >> 5], 1u << (j & 31));
  }
  if (threadIdx.x == 0) atomicOr(&bits[i >> 5], 1u << (i & 31));
  __syncthreads();
  int pc = 0;
  for (int w = threadIdx.x; w < g.words; w += NT) {
    const uint32_t v = bits[w];
    bitmap[(long)row * g.words + w] = v;
    pc += __popc(v);
  }
  pc = wave_sum_int(pc);
  if ((threadIdx.x & 63) == 0) itmp[threadIdx.x >> 6] = pc;
  __syncthreads();
  if (threadIdx.x == 0) {
    int c = 0;
    for (int w = 0; w < NT / 64; ++w) c += itmp[w];
    count[row] = c;
  }
}

// ---------------------------------------------------------------------------
// The same per-row selection with one wave per row (nb <= 2048), no LDS sort
// and no workgroup barriers: element e = lane * KPL + r of the row lives in
// register r of lane `lane`, and the bitonic network compares in registers for
// strides below KPL and across lanes (shuffles) above.  Same keys, so the same
// order; the float32 sums run in another order than the workgroup version.
// ---------------------------------------------------------------------------
template <int NBP>
__global__ __launch_bounds__(256) void select_wave_kernel(Geo g, float* __restrict__ score,
                                                          uint32_t* __restrict__ bitmap,
                                                          int* __restrict__ count, float p,
                                                          int k_floor, int write_prob) {
  constexpr int KPL = NBP / 64;   // keys per lane
  static_assert(KPL >= 1 && KPL <= 32, "one wave per row up to 2048 blocks");
  __shared__ uint32_t bits[4][NBP / 32 > 1 ? NBP / 32 : 1];
  const int wv = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int row = blockIdx.x * 4 + wv;
  if (row >= g.rows) return;   // whole wave: no workgroup barrier below
  const int nb = g.nb;
  const int i = row % nb;
  float* srow = score + (long)row * nb;
  float sv[KPL];
  float mx = -INFINITY;
#pragma unroll
  for (int r = 0; r < KPL; ++r) {
    const int j = lane * KPL + r;
    sv[r] = j < nb ? srow[j] : -INFINITY;
    mx = fmaxf(mx, sv[r]);
  }
  mx = wave_max(mx);
  float part = 0.f;
#pragma unroll
  for (int r = 0; r < KPL; ++r) {
    const int j = lane * KPL + r;
    sv[r] = j < nb ? expf(sv[r] - mx) : 0.f;
    part += sv[r];
  }
  const float z = wave_sum(part);
  unsigned long long key[KPL];
#pragma unroll
  for (int r = 0; r < KPL; ++r) {
    const int j = lane * KPL + r;
    key[r] = ~0ull;
    if (j < nb) {
      const float pj = sv[r] / z;
      if (write_prob) srow[j] = pj;
      key[r] = ((unsigned long long)(~__float_as_uint(pj)) << 32) | (unsigned)j;
    }
  }
  // bitonic sort, ascending keys = P descending then index ascending
#pragma unroll
  for (int size = 2; size <= NBP; size <<= 1) {
#pragma unroll
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      if (stride >= KPL) {
        const int ls = stride / KPL;
#pragma unroll
        for (int r = 0; r < KPL; ++r) {
          const unsigned long long o = __shfl_xor(key[r], ls);
          const int e = lane * KPL + r;
          const bool lower = (e & stride) == 0, up = (e & size) == 0;
          const unsigned long long lo = key[r] < o ? key[r] : o, hi = key[r] < o ? o : key[r];
          key[r] = (lower == up) ? lo : hi;
        }
      } else {
#pragma unroll
        for (int r = 0; r < KPL; ++r) {
          if (r & stride) continue;
          const int e = lane * KPL + r;
          const bool up = (e & size) == 0;
          const unsigned long long a = key[r], c = key[r + stride];
          if ((a > c) == up) { key[r] = c; key[r + stride] = a; }
        }
      }
    }
  }
  // inclusive scan of the sorted masses; first position reaching p
  float loc[KPL];
  float run = 0.f;
#pragma unroll
  for (int r = 0; r < KPL; ++r) {
    const int e = lane * KPL + r;
    run += (e < nb) ? __uint_as_float(~(uint32_t)(key[r] >> 32)) : 0.f;
    loc[r] = run;
  }
  const float pre = wave_inclusive_scan(run) - run;
  int first = nb;
#pragma unroll
  for (int r = KPL - 1; r >= 0; --r) {
    const int e = lane * KPL + r;
    if (e < nb && pre + loc[r] >= p) first = e + 1;
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) first = min(first, __shfl_xor(first, o));
  const int m = (p >= 1.0f) ? nb : first;
  const int m2 = min(nb, max(m, k_floor));
  uint32_t* wb = bits[wv];
  for (int w = lane; w < NBP / 32; w += 64) wb[w] = 0u;
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
#pragma unroll
  for (int r = 0; r < KPL; ++r) {
    const int e = lane * KPL + r;
    if (e < m2) {
      const int j = (int)(key[r] & 0xffffffffu);
      atomicOr(&wb[j >> 5], 1u << (j & 31));
    }
  }
  if (lane == 0) atomicOr(&wb[i >> 5], 1u << (i & 31));
  __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
  __builtin_amdgcn_wave_barrier();
  int pc = 0;
  for (int w = lane; w < g.words; w += 64) {
    const uint32_t v = wb[w];
    bitmap[(long)row * g.words + w] = v;
    pc += __popc(v);
  }
  pc = wave_sum_int(pc);
  if (lane == 0) count[row] = pc;
}

// ---------------------------------------------------------------------------
// Slack fill over groups of gr consecutive rows: in each group, add the `need`
// unkept pairs with the largest P among those with P >= theta (ties: lowest
// linear index).  Exact selection by a three-pass radix select on the float
// bits of P (non-negative floats order like their bit patterns): 11 + 11 + 10
// bits.  Groups are heads (fixed per-head budget, gr = nb, theta = 0) or the
// whole batch (dynamic fill, gr = rows).
// sel[group] = {need (remaining), prefix, active, need_total}
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void slack_init_kernel(Geo g, const int* __restrict__ count,
                                                         int* __restrict__ sel,
                                                         uint32_t* __restrict__ hist,
                                                         long long budget) {
  __shared__ int itmp[8];
  const int bh = blockIdx.x;
  int s = 0;
  for (int i = threadIdx.x; i < g.nb; i += 256) s += count[bh * g.nb + i];
  s = wave_sum_int(s);
  if ((threadIdx.x & 63) == 0) itmp[threadIdx.x >> 6] = s;
  for (int x = threadIdx.x; x < 2048; x += 256) hist[bh * 2048 + x] = 0u;
  __syncthreads();
  if (threadIdx.x == 0) {
    const long long nnz = (long long)itmp[0] + itmp[1] + itmp[2] + itmp[3];
    const long long need = budget - nnz;
    sel[bh * 4 + 0] = need > 0 ? (int)need : 0;
    sel[bh * 4 + 1] = 0;
    sel[bh * 4 + 2] = need > 0 ? 1 : 0;
    sel[bh * 4 + 3] = need > 0 ? (int)need : 0;
  }
}

// Dynamic fill, one group (the whole batch): need = the device-side budget.
__global__ __launch_bounds__(256) void dslack_init_kernel(int* __restrict__ sel,
                                                          uint32_t* __restrict__ hist,
                                                          const long long* __restrict__ budget) {
  for (int x = threadIdx.x; x < 2048; x += 256) hist[x] = 0u;
  if (threadIdx.x == 0) {
    long long need = *budget;
    need = need < 0 ? 0 : (need > 0x7fffffffll ? 0x7fffffffll : need);
    sel[0] = (int)need;
    sel[1] = 0;
    sel[2] = need > 0 ? 1 : 0;
    sel[3] = (int)need;
  }
}

// shift/width of the digit examined in each pass; prefix holds the bits above
__device__ __forceinline__ void slack_digit(int pass, int* shift, int* width) {
  *shift = pass == 0 ? 21 : (pass == 1 ? 10 : 0);
  *width = pass == 2 ? 10 : 11;
}

// Rows-per-workgroup chunks of one group; histogram of the current digit over
// candidate pairs (unkept, P >= theta) whose higher bits equal the prefix
// chosen so far.
__global__ __launch_bounds__(256) void slack_hist_kernel(Geo g, const float* __restrict__ prob,
                                                         const uint32_t* __restrict__ bitmap,
                                                         const int* __restrict__ sel,
                                                         uint32_t* __restrict__ hist, int pass,
                                                         int rows_per_wg, int gr, float theta) {
  __shared__ uint32_t lh[2048];
  const int bh = blockIdx.y;
  if (sel[bh * 4 + 2] == 0) return;
  int shift, width;
  slack_digit(pass, &shift, &width);
  const uint32_t prefix = (uint32_t)sel[bh * 4 + 1];
  const int hshift = shift + width;  // bits above the digit
  for (int x = threadIdx.x; x < 2048; x += 256) lh[x] = 0u;
  __syncthreads();
  const int i0 = blockIdx.x * rows_per_wg;
  const int i1 = min(gr, i0 + rows_per_wg);
  for (int i = i0; i < i1; ++i) {
    const long row = (long)bh * gr + i;
    for (int j = threadIdx.x; j < g.nb; j += 256) {
      if ((bitmap[row * g.words + (j >> 5)] >> (j & 31)) & 1u) continue;
      const float pv = prob[row * g.nb + j];
      if (!(pv >= theta)) continue;
      const uint32_t key = __float_as_uint(pv);
      if (pass > 0 && (key >> hshift) != prefix) continue;
      atomicAdd(&lh[(key >> shift) & ((1u << width) - 1u)], 1u);
    }
  }
  __syncthreads();
  for (int x = threadIdx.x; x < (1 << width); x += 256)
    if (lh[x]) atomicAdd(&hist[bh * 2048 + x], lh[x]);
}

// One workgroup per head: find the digit holding the need-th largest key.
__global__ __launch_bounds__(256) void slack_pick_kernel(int* __restrict__ sel,
                                                         uint32_t* __restrict__ hist, int pass) {
  __shared__ int itmp[8];
  const int bh = blockIdx.x;
  if (sel[bh * 4 + 2] == 0) return;
  int shift, width;
  slack_digit(pass, &shift, &width);
  const int nbins = 1 << width;
  const int per = nbins / 256;
  // thread t owns bins counted from the top: [nbins-1-t*per, nbins-(t+1)*per]
  int loc = 0;
  for (int e = 0; e < per; ++e) loc += (int)hist[bh * 2048 + nbins - 1 - (threadIdx.x * per + e)];
  int tot;
  const int above = block_exclusive_scan<256>(loc, itmp, &tot);
  int need = sel[bh * 4 + 0];
  if (pass == 0 && need > tot) need = tot;   // fewer candidates than the budget
  __syncthreads();
  if (need == 0) {
    if (threadIdx.x == 0) { sel[bh * 4 + 0] = 0; sel[bh * 4 + 2] = 0; }
    for (int x = threadIdx.x; x < 2048; x += 256) hist[bh * 2048 + x] = 0u;
    return;
  }
  if (above < need && need <= above + loc) {
    int run = above;
    for (int e = 0; e < per; ++e) {
      const int bin = nbins - 1 - (threadIdx.x * per + e);
      const int c = (int)hist[bh * 2048 + bin];
      if (need <= run + c) {
        sel[bh * 4 + 0] = need - run;
        sel[bh * 4 + 1] = (int)(((uint32_t)sel[bh * 4 + 1] << width) | (uint32_t)bin);
        break;
      }
      run += c;
    }
  }
  __syncthreads();
  for (int x = threadIdx.x; x < 2048; x += 256) hist[bh * 2048 + x] = 0u;
}

// Per row: number of unkept pairs whose key equals the threshold key.
__global__ __launch_bounds__(256) void slack_eqcount_kernel(Geo g, const float* __restrict__ prob,
                                                            const uint32_t* __restrict__ bitmap,
                                                            const int* __restrict__ sel,
                                                            int* __restrict__ eqcnt, int gr,
                                                            float theta) {
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (row >= g.rows) return;
  const int bh = row / gr;
  int c = 0;
  if (sel[bh * 4 + 2]) {
    const uint32_t thr = (uint32_t)sel[bh * 4 + 1];
    for (int j = lane; j < g.nb; j += 64) {
      if ((bitmap[(long)row * g.words + (j >> 5)] >> (j & 31)) & 1u) continue;
      const float pv = prob[(long)row * g.nb + j];
      if (pv >= theta && __float_as_uint(pv) == thr) ++c;
    }
  }
  c = wave_sum_int(c);
  if (lane == 0) eqcnt[row] = c;
}

// Per group: exclusive scan of the per-row equal counts (row order = linear order).
__global__ __launch_bounds__(256) void slack_eqscan_kernel(Geo g, const int* __restrict__ eqcnt,
                                                           int* __restrict__ eqoff, int gr) {
  __shared__ int itmp[8];
  const int bh = blockIdx.x;
  int carry = 0;
  for (int base = 0; base < gr; base += 256) {
    const int i = base + threadIdx.x;
    const long r = (long)bh * gr + i;
    const int v = i < gr ? eqcnt[r] : 0;
    int tot;
    const int ex = block_exclusive_scan<256>(v, itmp, &tot);
    if (i < gr) eqoff[r] = carry + ex;
    carry += tot;
  }
}

// Per row (one wave): set the bits of the selected pairs and update the count.
__global__ __launch_bounds__(256) void slack_mark_kernel(Geo g, const float* __restrict__ prob,
                                                         uint32_t* __restrict__ bitmap,
                                                         int* __restrict__ count,
                                                         const int* __restrict__ sel,
                                                         const int* __restrict__ eqoff, int gr,
                                                         float theta) {
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (row >= g.rows) return;
  const int bh = row / gr;
  if (!sel[bh * 4 + 2]) return;
  const uint32_t thr = (uint32_t)sel[bh * 4 + 1];
  const int need_eq = sel[bh * 4 + 0];
  int eq_rank = eqoff[row];
  int added = 0;
  for (int c0 = 0; c0 < g.nb; c0 += 64) {
    const int j = c0 + lane;
    uint32_t* wp = bitmap + (long)row * g.words + (c0 >> 5);
    bool take = false, eq = false;
    if (j < g.nb) {
      const bool kept = (wp[lane >> 5] >> (lane & 31)) & 1u;
      const float pv = kept ? 0.f : prob[(long)row * g.nb + j];
      if (!kept && pv >= theta) {
        const uint32_t key = __float_as_uint(pv);
        take = key > thr;
        eq = key == thr;
      }
    }
    const unsigned long long eqm = __ballot(eq);
    if (eq) {
      const int rank = eq_rank + __popcll(eqm & ((1ull << lane) - 1ull));
      take = rank < need_eq;
    }
    eq_rank += __popcll(eqm);
    const unsigned long long tm = __ballot(take);
    added += __popcll(tm);
    if (lane == 0) {
      if ((uint32_t)tm) wp[0] |= (uint32_t)tm;
      if ((uint32_t)(tm >> 32) && c0 + 32 < g.nb) wp[1] |= (uint32_t)(tm >> 32);
    }
  }
  if (lane == 0) count[row] += added;
}

// ---------------------------------------------------------------------------
// Dynamic slack budget from the telemetry of one persistent attention launch
// (one workgroup): records {hw id, xcc id, tiles, busy ticks} per workgroup.
// T = max busy; idle = n T - sum(busy) ticks, worth idle * sum(tiles) /
// sum(busy) tiles; budget = floor(fill * that), clamped to [0, max_pairs].
// The integer product is exact; then one float64 multiply and one divide.
// Source: FVAttn explainer, "Core method" part 3 (capacity that non-critical
// workers leave idle after balancing is filled).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void slack_budget_kernel(const long long* __restrict__ telem,
                                                           int n, float fill, long long max_pairs,
                                                           long long* __restrict__ budget) {
  __shared__ long long s_sum[4], s_tiles[4], s_max[4];
  long long sum = 0, tiles = 0, mx = 0;
  for (int w = threadIdx.x; w < n; w += 256) {
    const long long b = telem[4l * w + 3];
    sum += b;
    tiles += telem[4l * w + 2];
    mx = b > mx ? b : mx;
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    sum += __shfl_xor(sum, o);
    tiles += __shfl_xor(tiles, o);
    const long long om = __shfl_xor(mx, o);
    mx = om > mx ? om : mx;
  }
  if ((threadIdx.x & 63) == 0) {
    s_sum[threadIdx.x >> 6] = sum;
    s_tiles[threadIdx.x >> 6] = tiles;
    s_max[threadIdx.x >> 6] = mx;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    sum = tiles = mx = 0;
    for (int w = 0; w < 4; ++w) {
      sum += s_sum[w];
      tiles += s_tiles[w];
      mx = s_max[w] > mx ? s_max[w] : mx;
    }
    long long out = 0;
    if (sum > 0 && tiles > 0) {
      const long long idle_tiles = ((long long)n * mx - sum) * tiles;
      const double v = floor((double)fill * (double)idle_tiles / (double)sum);
      out = v <= 0.0 ? 0 : (v >= (double)max_pairs ? max_pairs : (long long)v);
    }
    *budget = out;
  }
}

// ---------------------------------------------------------------------------
// CSR: exclusive scan of the row counts (one workgroup), then per-row
// emission of ascending column indices from the bitmap (one wave per row).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(1024) void csr_scan_kernel(Geo g, const int* __restrict__ count,
                                                        int* __restrict__ row_ptr,
                                                        int* __restrict__ head_nnz) {
  __shared__ int itmp[17];
  constexpr int PER = 8;
  int carry = 0;
  for (int base = 0; base < g.rows; base += 1024 * PER) {
    const int r0 = base + threadIdx.x * PER;
    int v[PER];
    int run = 0;
#pragma unroll
    for (int e = 0; e < PER; ++e) {
      v[e] = (r0 + e < g.rows) ? count[r0 + e] : 0;
      run += v[e];
    }
    int tot;
    int ex = block_exclusive_scan<1024>(run, itmp, &tot) + carry;
#pragma unroll
    for (int e = 0; e < PER; ++e) {
      if (r0 + e < g.rows) row_ptr[r0 + e] = ex;
      ex += v[e];
    }
    carry += tot;
  }
  if (threadIdx.x == 0) row_ptr[g.rows] = carry;
  __syncthreads();
  for (int bh = threadIdx.x; bh < g.B * g.H; bh += 1024)
    head_nnz[bh] = row_ptr[(bh + 1) * g.nb] - row_ptr[bh * g.nb];
}

__global__ __launch_bounds__(256) void csr_emit_kernel(Geo g, const uint32_t* __restrict__ bitmap,
                                                       const int* __restrict__ row_ptr,
                                                       int* __restrict__ col_idx) {
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (row >= g.rows) return;
  int* out = col_idx + row_ptr[row];
  for (int c0 = 0; c0 < g.nb; c0 += 64) {
    const int j = c0 + lane;
    const bool bit = j < g.nb && ((bitmap[(long)row * g.words + (j >> 5)] >> (j & 31)) & 1u);
    const unsigned long long m = __ballot(bit);
    if (bit) out[__popcll(m & ((1ull << lane) - 1ull))] = j;
    out += __popcll(m);
  }
}

// ---------------------------------------------------------------------------
template <typename T>
static void launch_pool(const Geo& g, const void* q, const void* k, float* qp, float* kp,
                        hipStream_t s) {
  dim3 grid(g.nb, g.B * g.H);
  if (g.d == 128)
    hipLaunchKernelGGL((pool_kernel<T, 128>), grid, dim3(256), 0, s, g, (const T*)q,
                       (const T*)k, qp, kp);
  else
    hipLaunchKernelGGL((pool_kernel<T, 64>), grid, dim3(256), 0, s, g, (const T*)q,
                       (const T*)k, qp, kp);
}

template <int NBP>
static void launch_select_n(const Geo& g, float* score, uint32_t* bm, int* cnt, float p,
                            int kf, int wp, hipStream_t s) {
  hipLaunchKernelGGL((select_kernel<NBP>), dim3(g.rows), dim3(256), 0, s, g, score, bm, cnt, p,
                     kf, wp);
}

template <int NBP>
static void launch_select_wave(const Geo& g, float* score, uint32_t* bm, int* cnt, float p,
                               int kf, int wp, hipStream_t s) {
  hipLaunchKernelGGL((select_wave_kernel<NBP>), dim3((g.rows + 3) / 4), dim3(256), 0, s, g, score,
                     bm, cnt, p, kf, wp);
}

static void launch_select(const Geo& g, float* score, uint32_t* bm, int* cnt, float p, int kf,
                          int wp, hipStream_t s) {
  if (g.nb <= 64) launch_select_wave<64>(g, score, bm, cnt, p, kf, wp, s);
  else if (g.nb <= 128) launch_select_wave<128>(g, score, bm, cnt, p, kf, wp, s);
  else if (g.nb <= 256) launch_select_wave<256>(g, score, bm, cnt, p, kf, wp, s);
  else if (g.nb <= 512) launch_select_wave<512>(g, score, bm, cnt, p, kf, wp, s);
  else if (g.nb <= 1024) launch_select_wave<1024>(g, score, bm, cnt, p, kf, wp, s);
  else if (g.nb <= 2048) launch_select_wave<2048>(g, score, bm, cnt, p, kf, wp, s);
  else launch_select_n<4096>(g, score, bm, cnt, p, kf, wp, s);
}

hipError_t launch_route(const Geo& g, int dtype, const void* q, const void* k, float p,
                        int k_floor, float slack, const abs_mask* mask, char* ws,
                        const RouteWs& L, hipStream_t s) {
  float* qp = (float*)(ws + L.qp);
  float* kp = (float*)(ws + L.kp);
  float* score = (float*)(ws + L.score);
  uint32_t* bm = (uint32_t*)(ws + L.bitmap);
  int* cnt = (int*)(ws + L.count);
  if (dtype == ABS_BF16) launch_pool<bf16_t>(g, q, k, qp, kp, s);
  else launch_pool<float>(g, q, k, qp, kp, s);
  {
    dim3 grid((g.nb + 63) / 64, (g.nb + 63) / 64, g.B * g.H);
    const float scale = (float)(1.0 / sqrt((double)g.d));
    if (g.d == 128)
      hipLaunchKernelGGL(scores_kernel<128>, grid, dim3(256), 0, s, g, qp, kp, score, scale);
    else
      hipLaunchKernelGGL(scores_kernel<64>, grid, dim3(256), 0, s, g, qp, kp, score, scale);
  }
  const bool do_slack = slack > 0.f;
  launch_select(g, score, bm, cnt, p, k_floor, do_slack ? 1 : 0, s);
  if (do_slack) {
    const long long budget = (long long)ceil((double)slack * (double)g.nb * (double)g.nb);
    uint32_t* hist = (uint32_t*)(ws + L.hist);
    int* sel = (int*)(ws + L.sel);
    int* eqcnt = (int*)(ws + L.eqcnt);
    int* eqoff = (int*)(ws + L.eqoff);
    const int heads = g.B * g.H;
    hipLaunchKernelGGL(slack_init_kernel, dim3(heads), dim3(256), 0, s, g, cnt, sel, hist, budget);
    const int rpw = 8;
    for (int pass = 0; pass < 3; ++pass) {
      hipLaunchKernelGGL(slack_hist_kernel, dim3((g.nb + rpw - 1) / rpw, heads), dim3(256), 0, s,
                         g, score, bm, sel, hist, pass, rpw, g.nb, 0.0f);
      hipLaunchKernelGGL(slack_pick_kernel, dim3(heads), dim3(256), 0, s, sel, hist, pass);
    }
    const int wg4 = (g.rows + 3) / 4;
    hipLaunchKernelGGL(slack_eqcount_kernel, dim3(wg4), dim3(256), 0, s, g, score, bm, sel, eqcnt,
                       g.nb, 0.0f);
    hipLaunchKernelGGL(slack_eqscan_kernel, dim3(heads), dim3(256), 0, s, g, eqcnt, eqoff, g.nb);
    hipLaunchKernelGGL(slack_mark_kernel, dim3(wg4), dim3(256), 0, s, g, score, bm, cnt, sel,
                       eqoff, g.nb, 0.0f);
  }
  hipLaunchKernelGGL(csr_scan_kernel, dim3(1), dim3(1024), 0, s, g, cnt, mask->row_ptr,
                     mask->head_nnz);
  hipLaunchKernelGGL(csr_emit_kernel, dim3((g.rows + 3) / 4), dim3(256), 0, s, g, bm,
                     mask->row_ptr, mask->col_idx);
  return hipGetLastError();
}

hipError_t launch_route_dynamic(const Geo& g, int dtype, const void* q, const void* k, float p,
                                int k_floor, float theta, const long long* budget,
                                const abs_mask* mask, char* ws, const RouteWs& L, hipStream_t s) {
  float* qp = (float*)(ws + L.qp);
  float* kp = (float*)(ws + L.kp);
  float* score = (float*)(ws + L.score);
  uint32_t* bm = (uint32_t*)(ws + L.bitmap);
  int* cnt = (int*)(ws + L.count);
  if (dtype == ABS_BF16) launch_pool<bf16_t>(g, q, k, qp, kp, s);
  else launch_pool<float>(g, q, k, qp, kp, s);
  {
    dim3 grid((g.nb + 63) / 64, (g.nb + 63) / 64, g.B * g.H);
    const float scale = (float)(1.0 / sqrt((double)g.d));
    if (g.d == 128)
      hipLaunchKernelGGL(scores_kernel<128>, grid, dim3(256), 0, s, g, qp, kp, score, scale);
    else
      hipLaunchKernelGGL(scores_kernel<64>, grid, dim3(256), 0, s, g, qp, kp, score, scale);
  }
  launch_select(g, score, bm, cnt, p, k_floor, 1, s);
  // one group: the whole batch
  uint32_t* hist = (uint32_t*)(ws + L.hist);
  int* sel = (int*)(ws + L.sel);
  int* eqcnt = (int*)(ws + L.eqcnt);
  int* eqoff = (int*)(ws + L.eqoff);
  hipLaunchKernelGGL(dslack_init_kernel, dim3(1), dim3(256), 0, s, sel, hist, budget);
  const int rpw = 64;
  for (int pass = 0; pass < 3; ++pass) {
    hipLaunchKernelGGL(slack_hist_kernel, dim3((g.rows + rpw - 1) / rpw, 1), dim3(256), 0, s, g,
                       score, bm, sel, hist, pass, rpw, g.rows, theta);
    hipLaunchKernelGGL(slack_pick_kernel, dim3(1), dim3(256), 0, s, sel, hist, pass);
  }
  const int wg4 = (g.rows + 3) / 4;
  hipLaunchKernelGGL(slack_eqcount_kernel, dim3(wg4), dim3(256), 0, s, g, score, bm, sel, eqcnt,
                     g.rows, theta);
  hipLaunchKernelGGL(slack_eqscan_kernel, dim3(1), dim3(256), 0, s, g, eqcnt, eqoff, g.rows);
  hipLaunchKernelGGL(slack_mark_kernel, dim3(wg4), dim3(256), 0, s, g, score, bm, cnt, sel, eqoff,
                     g.rows, theta);
  hipLaunchKernelGGL(csr_scan_kernel, dim3(1), dim3(1024), 0, s, g, cnt, mask->row_ptr,
                     mask->head_nnz);
  hipLaunchKernelGGL(csr_emit_kernel, dim3((g.rows + 3) / 4), dim3(256), 0, s, g, bm,
                     mask->row_ptr, mask->col_idx);
  return hipGetLastError();
}

hipError_t launch_slack_budget(const long long* telem, int n, float fill, long long max_pairs,
                               long long* budget, hipStream_t s) {
  hipLaunchKernelGGL(slack_budget_kernel, dim3(1), dim3(256), 0, s, telem, n, fill, max_pairs,
                     budget);
  return hipGetLastError();
}

}  // namespace abs_impl
