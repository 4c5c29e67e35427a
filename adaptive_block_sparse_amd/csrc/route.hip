// Routing kernels: 3D-block mean pooling, pooled block scores with a row
// softmax and the per-row Top-p selection (Top-k floor, own-block repair) in
// one pass, per-head slack fill, and CSR compaction.  Source: FVAttn explainer
// ("FVAttn: adaptive sparse attention with runtime load balancing, for video
// generation"), "Core method" part 1 (sparse-routing frontend) and part 3
// (slack-aware augmentation).
#include <hip/hip_runtime.h>

#include <math.h>

#include "device_common.h"
#include "internal.h"
#include "route_internal.h"

namespace abs_impl {

// ---------------------------------------------------------------------------
// Pooling: mean of Q and K over the real tokens of each 3D block (the cheap
// approximate similarity the routing runs on, explainer "Highlights and
// limitations").  One workgroup per (3D block, group of hg heads of one batch
// entry).  In the [B, N, H, d] layout a token's heads sit side by side, so for
// every real token of the block the workgroup reads one contiguous run of
// hg*d elements, and the workgroups of the other head groups of the same block
// (launched next to it) read the rest of those tokens' rows.  Each thread owns
// one 16-byte chunk of the run and a residue class of the block's slots; it
// keeps 16 loads in flight and sums in slot order, then the classes are summed
// in a fixed order through LDS.
// ---------------------------------------------------------------------------
template <typename T, int D>
__global__ __launch_bounds__(256) void pool_kernel(Geo g, const T* __restrict__ q,
                                                   const T* __restrict__ k,
                                                   float* __restrict__ qp,
                                                   float* __restrict__ kp, int hg) {
  constexpr int E = Chunk<T>::E;   // elements per 16-byte chunk
  constexpr int C = D / E;         // chunks per head
  constexpr int BATCH = 8;         // slots per batch of loads (per tensor)
  __shared__ float red[2][256 * E];
  const int run = hg * C;          // chunks per token run; divides 256
  const int tpp = 256 / run;       // slots per pass
  const int ngrp = g.H / hg;
  const int b = blockIdx.x / ngrp, h0 = (blockIdx.x % ngrp) * hg;
  const int blk = blockIdx.y;
  const int tb = blk / (g.nbh * g.nbw), hb = (blk / g.nbw) % g.nbh, wb = blk % g.nbw;
  const int Tl = min(g.bt, g.T - tb * g.bt), Hl = min(g.bh, g.Hg - hb * g.bh),
            Wl = min(g.bw, g.W - wb * g.bw);
  const float inv = 1.0f / (float)(Tl * Hl * Wl);
  const int c = threadIdx.x % run, sub = threadIdx.x / run;
  const int plane = g.bh * g.bw;
  const long tok = (long)g.H * D;                  // elements per token row
  const long base = (long)b * g.N * tok + (long)h0 * D + c * E;
  float aq[E], ak[E];
#pragma unroll
  for (int e = 0; e < E; ++e) aq[e] = ak[e] = 0.f;
  for (int s0 = sub; s0 < g.Bt; s0 += BATCH * tpp) {
    uint4 rq[BATCH], rk[BATCH];
#pragma unroll
    for (int u = 0; u < BATCH; ++u) {
      const int s = s0 + u * tpp;
      rq[u] = rk[u] = make_uint4(0u, 0u, 0u, 0u);
      const int st = s / plane, sh = (s / g.bw) % g.bh, sw = s % g.bw;
      if (s < g.Bt && st < Tl && sh < Hl && sw < Wl) {
        const long n = ((long)(tb * g.bt + st) * g.Hg + hb * g.bh + sh) * g.W + wb * g.bw + sw;
        rq[u] = *reinterpret_cast<const uint4*>(q + base + n * tok);
        rk[u] = *reinterpret_cast<const uint4*>(k + base + n * tok);
      }
    }
#pragma unroll
    for (int u = 0; u < BATCH; ++u) {
      float vq[E], vk[E];
      Chunk<T>::unpack(rq[u], vq);
      Chunk<T>::unpack(rk[u], vk);
#pragma unroll
      for (int e = 0; e < E; ++e) {
        aq[e] += vq[e];
        ak[e] += vk[e];
      }
    }
  }
  // thread (sub, c) holds outputs o = c*E + e of the run: head h0 + o / D, dim o % D
#pragma unroll
  for (int e = 0; e < E; ++e) {
    red[0][threadIdx.x * E + e] = aq[e];
    red[1][threadIdx.x * E + e] = ak[e];
  }
  __syncthreads();
  const int outs = run * E;
  for (int o = threadIdx.x; o < 2 * outs; o += 256) {
    const int which = o / outs, oo = o % outs;
    float sum = 0.f;
    for (int s = 0; s < tpp; ++s) sum += red[which][s * outs + oo];
    float* dst = which == 0 ? qp : kp;
    dst[(((long)b * g.H + h0 + oo / D) * g.nb + blk) * D + oo % D] = sum * inv;
  }
}

// ---------------------------------------------------------------------------
// Frame means of K (fine-grained routing): for every 3D block and temporal
// offset tau < bt, the mean of K over the block's real tokens at that offset
// (bh x bw tokens, fewer in a block cut by the grid edge); 0 for a frame with
// no real token (a block cut along t).  Grid and thread layout as pool_kernel;
// the frames are summed one after the other.
// ---------------------------------------------------------------------------
template <typename T, int D>
__global__ __launch_bounds__(256) void frame_pool_kernel(Geo g, const T* __restrict__ k,
                                                         float* __restrict__ kf, int hg) {
  constexpr int E = Chunk<T>::E;
  constexpr int C = D / E;
  constexpr int BATCH = 8;
  __shared__ float red[256 * E];
  const int run = hg * C, tpp = 256 / run;
  const int ngrp = g.H / hg;
  const int b = blockIdx.x / ngrp, h0 = (blockIdx.x % ngrp) * hg;
  const int blk = blockIdx.y;
  const int tb = blk / (g.nbh * g.nbw), hb = (blk / g.nbw) % g.nbh, wb = blk % g.nbw;
  const int Tl = min(g.bt, g.T - tb * g.bt), Hl = min(g.bh, g.Hg - hb * g.bh),
            Wl = min(g.bw, g.W - wb * g.bw);
  const float inv = 1.0f / (float)(Hl * Wl);
  const int c = threadIdx.x % run, sub = threadIdx.x / run;
  const int plane = g.bh * g.bw;   // slots of one frame
  const long tok = (long)g.H * D;
  const long base = (long)b * g.N * tok + (long)h0 * D + c * E;
  const int outs = run * E;
  for (int tau = 0; tau < g.bt; ++tau) {
    float ak[E];
#pragma unroll
    for (int e = 0; e < E; ++e) ak[e] = 0.f;
    if (tau < Tl) {
      for (int s0 = sub; s0 < plane; s0 += BATCH * tpp) {
        uint4 rk[BATCH];
#pragma unroll
        for (int u = 0; u < BATCH; ++u) {
          const int s = s0 + u * tpp;
          rk[u] = make_uint4(0u, 0u, 0u, 0u);
          const int sh = s / g.bw, sw = s % g.bw;
          if (s < plane && sh < Hl && sw < Wl) {
            const long n = ((long)(tb * g.bt + tau) * g.Hg + hb * g.bh + sh) * g.W + wb * g.bw + sw;
            rk[u] = *reinterpret_cast<const uint4*>(k + base + n * tok);
          }
        }
#pragma unroll
        for (int u = 0; u < BATCH; ++u) {
          float vk[E];
          Chunk<T>::unpack(rk[u], vk);
#pragma unroll
          for (int e = 0; e < E; ++e) ak[e] += vk[e];
        }
      }
    }
#pragma unroll
    for (int e = 0; e < E; ++e) red[threadIdx.x * E + e] = ak[e];
    __syncthreads();
    for (int o = threadIdx.x; o < outs; o += 256) {
      float sum = 0.f;
      for (int s = 0; s < tpp; ++s) sum += red[s * outs + o];
      kf[((((long)b * g.H + h0 + o / D) * g.nb + blk) * g.bt + tau) * D + o % D] =
          tau < Tl ? sum * inv : 0.f;
    }
    __syncthreads();
  }
}

// ---------------------------------------------------------------------------
// Wave-wide sum and maximum through DPP row operations (quad swaps, half-row
// and row mirrors) and the four row results read out in a fixed order, so
// every lane receives the same value.
// ---------------------------------------------------------------------------
template <int CTRL>
__device__ __forceinline__ float dpp_f(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xf, 0xf, false));
}
__device__ __forceinline__ float row_lanes(float x, int l) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), l));
}
__device__ __forceinline__ float wave_sum_dpp(float x) {
  x += dpp_f<0xb1>(x);    // quad_perm [1,0,3,2]
  x += dpp_f<0x4e>(x);    // quad_perm [2,3,0,1]
  x += dpp_f<0x141>(x);   // row_half_mirror
  x += dpp_f<0x140>(x);   // row_mirror: every lane of a row of 16 holds the row sum
  return (row_lanes(x, 0) + row_lanes(x, 16)) + (row_lanes(x, 32) + row_lanes(x, 48));
}
__device__ __forceinline__ float wave_max_dpp(float x) {
  x = fmaxf(x, dpp_f<0xb1>(x));
  x = fmaxf(x, dpp_f<0x4e>(x));
  x = fmaxf(x, dpp_f<0x141>(x));
  x = fmaxf(x, dpp_f<0x140>(x));
  return fmaxf(fmaxf(row_lanes(x, 0), row_lanes(x, 16)),
               fmaxf(row_lanes(x, 32), row_lanes(x, 48)));
}
__device__ __forceinline__ int popc_ballot(bool b) { return __popcll(__ballot(b)); }

typedef float v4f __attribute__((ext_vector_type(4)));

// Sum and maximum over each row of 16 lanes (DPP quad swaps, half-row and row
// mirrors): every lane of a row receives its row's result.
template <int CTRL>
__device__ __forceinline__ int dpp_i(int x) {
  return __builtin_amdgcn_update_dpp(0, x, CTRL, 0xf, 0xf, false);
}
__device__ __forceinline__ float row16_sum(float x) {
  x += dpp_f<0xb1>(x);
  x += dpp_f<0x4e>(x);
  x += dpp_f<0x141>(x);
  x += dpp_f<0x140>(x);
  return x;
}
__device__ __forceinline__ int row16_sum_int(int x) {
  x += dpp_i<0xb1>(x);
  x += dpp_i<0x4e>(x);
  x += dpp_i<0x141>(x);
  x += dpp_i<0x140>(x);
  return x;
}
__device__ __forceinline__ int row16_max_int(int x) {
  x = max(x, dpp_i<0xb1>(x));
  x = max(x, dpp_i<0x4e>(x));
  x = max(x, dpp_i<0x141>(x));
  x = max(x, dpp_i<0x140>(x));
  return x;
}
__device__ __forceinline__ int row16_min_int(int x) {
  x = min(x, dpp_i<0xb1>(x));
  x = min(x, dpp_i<0x4e>(x));
  x = min(x, dpp_i<0x141>(x));
  x = min(x, dpp_i<0x140>(x));
  return x;
}
__device__ __forceinline__ float row16_max(float x) {
  x = fmaxf(x, dpp_f<0xb1>(x));
  x = fmaxf(x, dpp_f<0x4e>(x));
  x = fmaxf(x, dpp_f<0x141>(x));
  x = fmaxf(x, dpp_f<0x140>(x));
  return x;
}

// ---------------------------------------------------------------------------
// Scores, softmax and Top-p selection of 16 rows (query blocks) of one head,
// nb <= 64*NC <= 1024 (one workgroup; wave w owns rows 4w..4w+3 of the group).
//
// Scores: Kp of the head streams through LDS in chunks of 64 key blocks, and
// each wave multiplies the group's 16 Qp rows by 16 of a chunk's keys on the
// fp32 matrix cores.  The scores then pass through LDS so that row r of wave w
// (group row 4w + r) lives in lanes 16r..16r+15 (one DPP row), element
// j = 16e + (lane & 15) in register e.  Every step below works on the wave's
// four rows at once and reduces within DPP rows.
//
// Selection.  The probabilities are never sorted.  The order (P descending,
// then j ascending) is only needed through two of its consequences, both found
// by bisection over the float32 bit pattern of P (non-negative floats order
// like their bits; 30 halvings of [0, bits(1.0) + 1]):
//   mass:  the largest t with S(t) = sum of P_j over bits(P_j) >= t at least
//          p is the bit pattern of the m-th largest P, where m is the size of
//          the smallest prefix of the order reaching p; the blocks above it are
//          kept, and of the blocks equal to it the lowest-index ones the prefix
//          needs;
//   floor: when m is below k_floor, the largest t with at least k_floor blocks
//          at or above it, the ties again by lowest index.
// p = 1, or a total that rounding left below p, keeps every block.  The own
// block is added last.  Output: the rows' bitmaps and counts, the group's
// total count (for the CSR offsets) and, for slack fills, P.
// ---------------------------------------------------------------------------
//
// FR: the same selection one level down (fine-grained Top-p inside the kept
// blocks): the keys are the frames f = j*bt + tau of the blocks (kp then holds
// the frame means of K, nk = nb*bt per head), and only the real frames of the
// blocks the row keeps in `cand` (the block-level bitmaps) are candidates.  The
// floor counts frames, every frame of the own block is kept, and the output is
// the row's frame bitmap.
template <int D, int NC, bool FR = false>
__global__ __launch_bounds__(256) void route_select_kernel(
    Geo g, const float* __restrict__ qp, const float* __restrict__ kp,
    uint32_t* __restrict__ bitmap, int* __restrict__ count, int* __restrict__ gsum,
    float* __restrict__ prob, float p, int k_floor, float scale,
    const uint32_t* __restrict__ cand, int nk, int words_out) {
  constexpr int KS = D + 4;          // padded LDS row of one key block's mean
  constexpr int TS = 64 * NC + 16;   // padded LDS row of one row's scores
  constexpr int E = 4 * NC;          // elements per lane in the 16-lane layout
  constexpr int KD = D / 4;          // MFMA k-steps (4 dimensions each)
  constexpr int LDS_F = 64 * KS > 16 * TS ? 64 * KS : 16 * TS;
  __shared__ float lds[LDS_F];
  __shared__ int wsum[4];
  const int bh = blockIdx.y;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int nb = g.nb;
  const int nch = (nk + 63) >> 6;    // key chunks present (<= NC)
  const int ig = blockIdx.x * 16;    // first row of the group
  const float* K = kp + (long)bh * nk * D;
  // Scores on the fp32 matrix cores (v_mfma_f32_16x16x4_f32): the group's 16
  // rows against 16 keys per wave and chunk.  Lane l supplies A[l % 16][l / 16]
  // and B[l / 16][l % 16] and receives D[4 (l / 16) + r][l % 16] in register r.
  // k-step s gives slot l / 16 the dimension KD (l / 16) + s, so each lane's A
  // values (its row's Qp) are KD consecutive floats, loaded once.
  const int a16 = lane & 15, kq = lane >> 4;
  float a[KD];
  {
    const float4* src = reinterpret_cast<const float4*>(
        qp + ((long)bh * nb + min(ig + a16, nb - 1)) * D + KD * kq);
#pragma unroll
    for (int s = 0; s < KD / 4; ++s) {
      const float4 v = src[s];
      a[4 * s] = v.x; a[4 * s + 1] = v.y; a[4 * s + 2] = v.z; a[4 * s + 3] = v.w;
    }
  }
  // chunk c + 1 of Kp is loaded into registers while chunk c is multiplied
  constexpr int PER = 64 * (D / 4) / 256;   // float4 per thread per chunk
  float4 nxt[PER];
  auto load_chunk = [&](int c) {
#pragma unroll
    for (int u = 0; u < PER; ++u) {
      const int f = threadIdx.x + 256 * u;
      const int kb = f / (D / 4), d4 = f % (D / 4);
      const int j = c * 64 + kb;
      nxt[u] = make_float4(0.f, 0.f, 0.f, 0.f);
      if (j < nk) nxt[u] = *reinterpret_cast<const float4*>(K + (long)j * D + d4 * 4);
    }
  };
  load_chunk(0);
  v4f acc[NC];
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    acc[c] = v4f{0.f, 0.f, 0.f, 0.f};
    if (c < nch) {
      __syncthreads();
#pragma unroll
      for (int u = 0; u < PER; ++u) {
        const int f = threadIdx.x + 256 * u;
        *reinterpret_cast<float4*>(lds + (f / (D / 4)) * KS + (f % (D / 4)) * 4) = nxt[u];
      }
      if (c + 1 < nch) load_chunk(c + 1);
      __syncthreads();
      const float* brow = lds + (16 * wv + a16) * KS + KD * kq;
#pragma unroll
      for (int s = 0; s < KD; s += 4) {
        const float4 bv = *reinterpret_cast<const float4*>(brow + s);
        acc[c] = __builtin_amdgcn_mfma_f32_16x16x4f32(a[s], bv.x, acc[c], 0, 0, 0);
        acc[c] = __builtin_amdgcn_mfma_f32_16x16x4f32(a[s + 1], bv.y, acc[c], 0, 0, 0);
        acc[c] = __builtin_amdgcn_mfma_f32_16x16x4f32(a[s + 2], bv.z, acc[c], 0, 0, 0);
        acc[c] = __builtin_amdgcn_mfma_f32_16x16x4f32(a[s + 3], bv.w, acc[c], 0, 0, 0);
      }
    }
  }
  __syncthreads();   // every wave is done with the staged keys
  // scores to LDS, row-major over the group's 16 rows
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    const int j = c * 64 + 16 * wv + a16;
#pragma unroll
    for (int r = 0; r < 4; ++r)
      lds[(4 * kq + r) * TS + j] = c < nch && j < nk ? acc[c][r] * scale : -INFINITY;
  }
  __syncthreads();
  const float* T = lds + wv * 4 * TS;
  const int i0 = ig + 4 * wv;
  const int rr = lane >> 4, l16 = lane & 15;
  const int i = i0 + rr;             // this lane's row
  const bool live = i < nb;
  const int row = bh * nb + i;
  float x[E];
  bool valid[E];
  int nc = nb;                       // candidates of the row
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const int f = 16 * e + l16;
    valid[e] = f < nk;
    if constexpr (FR) {
      // a frame of a block the row keeps, and a frame with real tokens
      const int j = f / g.bt, tau = f - j * g.bt;
      const int tl = min(g.bt, g.T - (j / (g.nbh * g.nbw)) * g.bt);
      valid[e] = valid[e] && live && tau < tl &&
                 ((cand[(long)row * g.words + (j >> 5)] >> (j & 31)) & 1u);
    }
    x[e] = valid[e] ? T[rr * TS + f] : -INFINITY;
  }
  if constexpr (FR) {
    int n = 0;
#pragma unroll
    for (int e = 0; e < E; ++e) n += valid[e] ? 1 : 0;
    nc = row16_sum_int(n);
  }

  // softmax over the row's candidates; keys = bit patterns of P, -1 elsewhere
  float mx = -INFINITY;
#pragma unroll
  for (int e = 0; e < E; ++e) mx = fmaxf(mx, x[e]);
  mx = row16_max(mx);
  float part = 0.f;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    x[e] = expf(x[e] - mx);
    part += x[e];
  }
  const float rz = 1.0f / row16_sum(part);
  int key[E];
  part = 0.f;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const int j = 16 * e + l16;
    const float pj = x[e] * rz;
    if (prob && live && j < nb) prob[(long)row * nb + j] = pj;
    key[e] = valid[e] ? __float_as_int(pj) : -1;
    part += valid[e] ? pj : 0.f;
  }
  const float total = row16_sum(part);

  // mass bisection.  Bracket: S(lo) >= p > S(hi) = shi, clo and chi blocks at
  // or above lo and hi.  It starts at [bits(min P), bits(max P) + 1) and stops
  // once one block is left inside it (its P is the cut) or it is one bit wide
  // (the blocks inside are ties).
  int kmin = 0x7fffffff, kmax = -1;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    kmin = key[e] >= 0 ? min(kmin, key[e]) : kmin;
    kmax = max(kmax, key[e]);
  }
  int lo = row16_min_int(kmin), hi = row16_max_int(kmax) + 1;
  int clo = nc, chi = 0;
  float shi = 0.f;
  bool active = clo - chi > 1 && hi - lo > 1;
  for (int step = 0; step < 31; ++step) {
    if (!__ballot(active)) break;
    const int mid = lo + ((hi - lo) >> 1);
    float sp = 0.f;
    int cnt = 0;
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const bool ge = key[e] >= mid;
      sp += ge ? __int_as_float(key[e]) : 0.f;
      cnt += ge ? 1 : 0;
    }
    const float sm = row16_sum(sp);
    cnt = row16_sum_int(cnt);
    const bool up = sm >= p;
    if (active) {
      lo = up ? mid : lo;
      clo = up ? cnt : clo;
      hi = up ? hi : mid;
      chi = up ? chi : cnt;
      shi = up ? shi : sm;
    }
    active = clo - chi > 1 && hi - lo > 1;
  }
  // the cut: the largest P below hi; the blocks above it, and its ties
  int kcut = -1;
#pragma unroll
  for (int e = 0; e < E; ++e) kcut = key[e] < hi ? max(kcut, key[e]) : kcut;
  lo = row16_max_int(kcut);
  const int cg = chi, ct = clo - chi;
  const float v = __int_as_float(lo);
  int need = ct;
  if (v > 0.f) {
    const float t = ceilf((p - shi) / v);
    need = t < 1.f ? 1 : (t < (float)ct ? (int)t : ct);
  }
  const int m = cg + need;
  const int m2 = min(nc, max(m, k_floor));
  const bool all = p >= 1.0f || !(total >= p) || m2 >= nc;
  const bool floor_row = !all && m2 > m;
  int thr = all ? -1 : lo;           // keep key > thr, and the first ktie keys == thr
  int ktie = all ? 0 : need;
  if (__ballot(floor_row && live)) {
    // floor: the largest t with at least m2 blocks at or above it
    int a = 0, b = 0x3f800001;
    for (int step = 0; step < 30; ++step) {
      const int mid = a + ((b - a) >> 1);
      int cnt = 0;
#pragma unroll
      for (int e = 0; e < E; ++e) cnt += key[e] >= mid ? 1 : 0;
      cnt = row16_sum_int(cnt);
      const bool up = cnt >= m2;
      a = up ? mid : a;
      b = up ? b : mid;
    }
    int above = 0;
#pragma unroll
    for (int e = 0; e < E; ++e) above += key[e] > a ? 1 : 0;
    above = row16_sum_int(above);
    if (floor_row) {
      thr = a;
      ktie = m2 - above;
    }
  }

  // kept bits: register e holds keys 16e .. 16e+15 of each row (16 bits of a
  // 64-bit ballot), so registers 2w and 2w+1 make bitmap word w
  const uint32_t below = (1u << l16) - 1u;
  const int sh = 16 * rr;
  int tie_seen = 0, kept = 0;
  uint32_t half = 0;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const int j = 16 * e + l16;
    const bool eq = thr >= 0 && key[e] == thr;
    const uint32_t eg = (uint32_t)(__ballot(eq) >> sh) & 0xffffu;
    const int rank = tie_seen + __popc(eg & below);
    tie_seen += __popc(eg);
    const bool own = FR ? j / g.bt == i : j == i;
    const bool keep = valid[e] && (key[e] > thr || (eq && rank < ktie) || own);
    const uint32_t kg = (uint32_t)(__ballot(keep) >> sh) & 0xffffu;
    kept += __popc(kg);
    if (e & 1) {
      if (live && l16 == 0 && (e >> 1) < words_out)
        bitmap[(long)row * words_out + (e >> 1)] = half | (kg << 16);
    } else {
      half = kg;
    }
  }
  if (live && l16 == 0) count[row] = kept;
  const int mine = live ? kept : 0;  // the same in all 16 lanes of a row
  const int wtot = __builtin_amdgcn_readlane(mine, 0) + __builtin_amdgcn_readlane(mine, 16) +
                   __builtin_amdgcn_readlane(mine, 32) + __builtin_amdgcn_readlane(mine, 48);
  if (lane == 0) wsum[wv] = wtot;
  __syncthreads();
  if (threadIdx.x == 0 && gsum)
    gsum[bh * gridDim.x + blockIdx.x] = wsum[0] + wsum[1] + wsum[2] + wsum[3];
}

// ---------------------------------------------------------------------------
// The same scores and selection for nb > 1024 with one wave per row (RPW = 1):
// element j = 64c + l of the row lives in register c of lane l, and each
// bisection step reduces across the whole wave.  Same results as above up to
// the order of float32 sums.
// ---------------------------------------------------------------------------
template <int D, int KPL, int RPW>
__global__ __launch_bounds__(256) void route_select_wide_kernel(
    Geo g, const float* __restrict__ qp, const float* __restrict__ kp,
    uint32_t* __restrict__ bitmap, int* __restrict__ count, int* __restrict__ gsum,
    float* __restrict__ prob, float p, int k_floor, float scale) {
  constexpr int KS = D + 4;          // padded LDS row of one key block's mean
  __shared__ float kt[64 * KS];
  __shared__ int wsum[4];
  const int bh = blockIdx.y;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int nb = g.nb;
  const int nch = (nb + 63) >> 6;    // key chunks present (<= KPL)
  const int i0 = (blockIdx.x * 4 + wv) * RPW;
  const float* K = kp + (long)bh * nb * D;
  const float4* Qr[RPW];
#pragma unroll
  for (int r = 0; r < RPW; ++r)
    Qr[r] = reinterpret_cast<const float4*>(qp + ((long)bh * nb + min(i0 + r, nb - 1)) * D);

  // scores -> keys: key = bit pattern of P_j, or -1 past nb
  int key[RPW][KPL];
#pragma unroll
  for (int c = 0; c < KPL; ++c) {
    if (c < nch) {
      __syncthreads();
      for (int f = threadIdx.x; f < 64 * (D / 4); f += 256) {
        const int kb = f / (D / 4), d4 = f % (D / 4);
        const int j = c * 64 + kb;
        float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
        if (j < nb) v = *reinterpret_cast<const float4*>(K + (long)j * D + d4 * 4);
        *reinterpret_cast<float4*>(kt + kb * KS + d4 * 4) = v;
      }
      __syncthreads();
      float acc[RPW];
#pragma unroll
      for (int r = 0; r < RPW; ++r) acc[r] = 0.f;
#pragma unroll 8
      for (int d4 = 0; d4 < D / 4; ++d4) {
        const float4 kv = *reinterpret_cast<const float4*>(kt + lane * KS + d4 * 4);
#pragma unroll
        for (int r = 0; r < RPW; ++r) {
          const float4 qv = Qr[r][d4];
          acc[r] = fmaf(qv.x, kv.x, acc[r]);
          acc[r] = fmaf(qv.y, kv.y, acc[r]);
          acc[r] = fmaf(qv.z, kv.z, acc[r]);
          acc[r] = fmaf(qv.w, kv.w, acc[r]);
        }
      }
#pragma unroll
      for (int r = 0; r < RPW; ++r)
        key[r][c] = __float_as_int(c * 64 + lane < nb ? acc[r] * scale : -INFINITY);
    } else {
#pragma unroll
      for (int r = 0; r < RPW; ++r) key[r][c] = __float_as_int(-INFINITY);
    }
  }

  // softmax over the row's nb blocks; keys become the bit patterns of P
  float total[RPW];
#pragma unroll
  for (int r = 0; r < RPW; ++r) {
    float mx = -INFINITY;
#pragma unroll
    for (int c = 0; c < KPL; ++c) mx = fmaxf(mx, __int_as_float(key[r][c]));
    mx = wave_max_dpp(mx);
    float part = 0.f;
#pragma unroll
    for (int c = 0; c < KPL; ++c) {
      const float e = c < nch ? expf(__int_as_float(key[r][c]) - mx) : 0.f;
      key[r][c] = __float_as_int(e);
      part += e;
    }
    const float z = wave_sum_dpp(part);
    const int row = bh * nb + i0 + r;
    const bool live = i0 + r < nb;
    part = 0.f;
#pragma unroll
    for (int c = 0; c < KPL; ++c) {
      const int j = c * 64 + lane;
      const float pj = __int_as_float(key[r][c]) / z;
      if (prob && live && j < nb) prob[(long)row * nb + j] = pj;
      key[r][c] = j < nb ? __float_as_int(pj) : -1;
      part += j < nb ? pj : 0.f;
    }
    total[r] = wave_sum_dpp(part);
  }

  // mass bisection, the wave's rows in lockstep
  int lo[RPW], hi[RPW];
  float shi[RPW];
#pragma unroll
  for (int r = 0; r < RPW; ++r) { lo[r] = 0; hi[r] = 0x3f800001; shi[r] = 0.f; }
  for (int step = 0; step < 30; ++step) {
#pragma unroll
    for (int r = 0; r < RPW; ++r) {
      const int mid = lo[r] + ((hi[r] - lo[r]) >> 1);
      float part = 0.f;
#pragma unroll
      for (int c = 0; c < KPL; ++c)
        if (c < nch) part += key[r][c] >= mid ? __int_as_float(key[r][c]) : 0.f;
      const float sm = wave_sum_dpp(part);
      if (sm >= p) lo[r] = mid;
      else { hi[r] = mid; shi[r] = sm; }
    }
  }

  int mine = 0;   // kept blocks of this wave's live rows
#pragma unroll
  for (int r = 0; r < RPW; ++r) {
    const int i = i0 + r;
    if (i >= nb) continue;   // wave-uniform
    const int row = bh * nb + i;
    int thr, ktie;           // keep key > thr, and the first ktie blocks with key == thr
    if (p >= 1.0f || !(total[r] >= p)) {
      thr = -1; ktie = 0;    // every block (p = 1, or rounding left the total below p)
    } else {
      int cg = 0, ct = 0;
#pragma unroll
      for (int c = 0; c < KPL; ++c)
        if (c < nch) {
          cg += popc_ballot(key[r][c] > lo[r]);
          ct += popc_ballot(key[r][c] == lo[r]);
        }
      const float v = __int_as_float(lo[r]);
      int need = ct;
      if (v > 0.f) {
        const float t = ceilf((p - shi[r]) / v);
        need = t < 1.f ? 1 : (t < (float)ct ? (int)t : ct);
      }
      const int m = cg + need;
      const int m2 = min(nb, max(m, k_floor));
      if (m2 >= nb) {
        thr = -1; ktie = 0;
      } else if (m2 == m) {
        thr = lo[r]; ktie = need;
      } else {
        // floor: the largest t with at least m2 blocks at or above it
        int a = 0, bnd = 0x3f800001;
        for (int step = 0; step < 30; ++step) {
          const int mid = a + ((bnd - a) >> 1);
          int cnt = 0;
#pragma unroll
          for (int c = 0; c < KPL; ++c)
            if (c < nch) cnt += popc_ballot(key[r][c] >= mid);
          if (cnt >= m2) a = mid;
          else bnd = mid;
        }
        int above = 0;
#pragma unroll
        for (int c = 0; c < KPL; ++c)
          if (c < nch) above += popc_ballot(key[r][c] > a);
        thr = a; ktie = m2 - above;
      }
    }
    int kept = 0, tie_seen = 0;
#pragma unroll
    for (int c = 0; c < KPL; ++c) {
      if (c >= nch) continue;
      const int j = c * 64 + lane;
      const bool eq = key[r][c] == thr && thr >= 0;
      const unsigned long long em = __ballot(eq);
      const int rank = tie_seen + __popcll(em & ((1ull << lane) - 1ull));
      tie_seen += __popcll(em);
      const bool keep = j < nb && (key[r][c] > thr || (eq && rank < ktie) || j == i);
      const unsigned long long km = __ballot(keep);
      kept += __popcll(km);
      uint32_t* wp = bitmap + (long)row * g.words + 2 * c;
      if (lane == 0) wp[0] = (uint32_t)km;
      if (lane == 1 && 2 * c + 1 < g.words) wp[1] = (uint32_t)(km >> 32);
    }
    if (lane == 0) count[row] = kept;
    mine += kept;
  }
  if (lane == 0) wsum[wv] = mine;
  __syncthreads();
  if (threadIdx.x == 0)
    gsum[bh * gridDim.x + blockIdx.x] = wsum[0] + wsum[1] + wsum[2] + wsum[3];
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
// Kept blocks per row group (one thread per group), after a slack fill has
// changed the row counts.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void route_gsum_kernel(Geo g, const int* __restrict__ count,
                                                         int* __restrict__ gsum, int rpg,
                                                         int gph) {
  const int x = blockIdx.x * 256 + threadIdx.x;
  if (x >= g.B * g.H * gph) return;
  const int bh = x / gph, i0 = (x % gph) * rpg;
  int s = 0;
  for (int i = i0; i < min(g.nb, i0 + rpg); ++i) s += count[bh * g.nb + i];
  gsum[x] = s;
}

// ---------------------------------------------------------------------------
// CSR over the row groups of route_select_kernel (same grid): a group's first
// position is the sum of the totals of all groups before it (read from gsum),
// its rows follow in order, and each row's columns are its bitmap's set bits
// in ascending order (one wave per row, 64 columns per ballot).  The first
// group of a head also writes the head's total, the last group the end of
// row_ptr.
// ---------------------------------------------------------------------------
// With frame bitmaps (fine-grained routing, fwords words a row) every entry
// also gets its kept frames: frame_mask[e] bit tau = frame tau of that block.
__global__ __launch_bounds__(256) void route_csr_kernel(Geo g, const uint32_t* __restrict__ bitmap,
                                                        const int* __restrict__ count,
                                                        const int* __restrict__ gsum, int rpg,
                                                        int* __restrict__ row_ptr,
                                                        int* __restrict__ col_idx,
                                                        int* __restrict__ head_nnz,
                                                        const uint32_t* __restrict__ fbitmap,
                                                        int fwords, int* __restrict__ frame_mask) {
  __shared__ int tmp[8];
  __shared__ int roff[17];
  const int bh = blockIdx.y, x = blockIdx.x, gph = gridDim.x;
  const int lin = bh * gph + x;
  const int wv = threadIdx.x >> 6, lane = threadIdx.x & 63;
  int a = 0, hs = 0;
  for (int w = threadIdx.x; w < lin; w += 256) a += gsum[w];
  if (x == 0)
    for (int w = threadIdx.x; w < gph; w += 256) hs += gsum[bh * gph + w];
  a = wave_sum_int(a);
  hs = wave_sum_int(hs);
  if (lane == 0) { tmp[wv] = a; tmp[4 + wv] = hs; }
  const int i0 = x * rpg, n = min(rpg, g.nb - i0);
  if (threadIdx.x == 0) {
    int run = 0;
    for (int r = 0; r < n; ++r) {
      roff[r] = run;
      run += count[bh * g.nb + i0 + r];
    }
    roff[n] = run;
  }
  __syncthreads();
  const int base = tmp[0] + tmp[1] + tmp[2] + tmp[3];
  if (threadIdx.x == 0) {
    if (x == 0) head_nnz[bh] = tmp[4] + tmp[5] + tmp[6] + tmp[7];
    if (lin == g.B * g.H * gph - 1) row_ptr[g.rows] = base + roff[n];
  }
  for (int r = wv; r < n; r += 4) {
    const int row = bh * g.nb + i0 + r;
    const int start = base + roff[r];
    if (lane == 0) row_ptr[row] = start;
    int pos = start;
    for (int c0 = 0; c0 < g.nb; c0 += 64) {
      const int j = c0 + lane;
      const bool bit = j < g.nb && ((bitmap[(long)row * g.words + (j >> 5)] >> (j & 31)) & 1u);
      const unsigned long long m = __ballot(bit);
      if (bit) {
        const int at = pos + __popcll(m & ((1ull << lane) - 1ull));
        col_idx[at] = j;
        if (frame_mask) {
          const uint32_t* fb = fbitmap + (long)row * fwords;
          const int f0 = j * g.bt, w0 = f0 >> 5, sh = f0 & 31;
          uint32_t v = fb[w0] >> sh;
          if (sh + g.bt > 32) v |= fb[w0 + 1] << (32 - sh);
          frame_mask[at] = (int)(v & ((1u << g.bt) - 1u));
        }
      }
      pos += __popcll(m);
    }
  }
}

// ---------------------------------------------------------------------------
template <typename T>
static void launch_pool(const Geo& g, const void* q, const void* k, float* qp, float* kp,
                        hipStream_t s) {
  // widest head group (at most 8 heads) that divides H, fits 256 chunks and
  // still gives at least 4096 workgroups (480p: 2 heads, 6160 workgroups; 1,
  // 2, 4 and 8 heads measured 138, 133, 136 and 141 us there)
  const int chunks_per_head = g.d * (int)sizeof(T) / 16;
  int hg = 8;
  while (hg > 1 && (g.H % hg != 0 || hg * chunks_per_head > 256 ||
                    (long)g.B * (g.H / hg) * g.nb < 4096))
    hg /= 2;
  dim3 grid(g.B * (g.H / hg), g.nb);
  if (g.d == 128)
    hipLaunchKernelGGL((pool_kernel<T, 128>), grid, dim3(256), 0, s, g, (const T*)q,
                       (const T*)k, qp, kp, hg);
  else
    hipLaunchKernelGGL((pool_kernel<T, 64>), grid, dim3(256), 0, s, g, (const T*)q,
                       (const T*)k, qp, kp, hg);
}

template <int D, int KPL>
static void launch_select_wide(const Geo& g, dim3 grid, const float* qp, const float* kp,
                               uint32_t* bm, int* cnt, int* gsum, float* prob, float p, int kf,
                               float scale, hipStream_t s) {
  hipLaunchKernelGGL((route_select_wide_kernel<D, KPL, 1>), grid, dim3(256), 0, s, g, qp, kp, bm,
                     cnt, gsum, prob, p, kf, scale);
}

template <int D, int NC>
static void launch_select16(const Geo& g, dim3 grid, const float* qp, const float* kp,
                            uint32_t* bm, int* cnt, int* gsum, float* prob, float p, int kf,
                            float scale, hipStream_t s) {
  hipLaunchKernelGGL((route_select_kernel<D, NC>), grid, dim3(256), 0, s, g, qp, kp, bm, cnt, gsum,
                     prob, p, kf, scale, (const uint32_t*)nullptr, g.nb, g.words);
}

template <int D>
static void launch_select_d(const Geo& g, dim3 grid, const float* qp, const float* kp,
                            uint32_t* bm, int* cnt, int* gsum, float* prob, float p, int kf,
                            float scale, hipStream_t s) {
  const int nch = (g.nb + 63) / 64;
#define ABS_SEL16(NC_)                                                                   \
  if (nch <= NC_) {                                                                      \
    launch_select16<D, NC_>(g, grid, qp, kp, bm, cnt, gsum, prob, p, kf, scale, s);      \
    return;                                                                              \
  }
  ABS_SEL16(1) ABS_SEL16(2) ABS_SEL16(3) ABS_SEL16(4) ABS_SEL16(5) ABS_SEL16(6)
  ABS_SEL16(8) ABS_SEL16(10) ABS_SEL16(12) ABS_SEL16(16)
#undef ABS_SEL16
  if (nch <= 32) launch_select_wide<D, 32>(g, grid, qp, kp, bm, cnt, gsum, prob, p, kf, scale, s);
  else if (nch <= 64) launch_select_wide<D, 64>(g, grid, qp, kp, bm, cnt, gsum, prob, p, kf, scale, s);
  else launch_select_wide<D, 128>(g, grid, qp, kp, bm, cnt, gsum, prob, p, kf, scale, s);
}

// pooling, then scores + softmax + selection (P kept for a slack fill when
// `prob` is given)
static void launch_route_front(const Geo& g, int dtype, const void* q, const void* k, float p,
                               int k_floor, char* ws, const RouteWs& L, float* prob,
                               hipStream_t s) {
  float* qp = (float*)(ws + L.qp);
  float* kp = (float*)(ws + L.kp);
  if (dtype == ABS_BF16) launch_pool<bf16_t>(g, q, k, qp, kp, s);
  else launch_pool<float>(g, q, k, qp, kp, s);
  static_assert(MAX_NB <= 64 * 128, "one wave's registers hold a row of at most 8192 blocks");
  const dim3 grid(route_groups_per_head(g.nb), g.B * g.H);
  const float scale = (float)(1.0 / sqrt((double)g.d));
  uint32_t* bm = (uint32_t*)(ws + L.bitmap);
  int* cnt = (int*)(ws + L.count);
  int* gsum = (int*)(ws + L.gsum);
  if (g.d == 128) launch_select_d<128>(g, grid, qp, kp, bm, cnt, gsum, prob, p, k_floor, scale, s);
  else launch_select_d<64>(g, grid, qp, kp, bm, cnt, gsum, prob, p, k_floor, scale, s);
}

static void launch_route_csr(const Geo& g, char* ws, const RouteWs& L, bool recount,
                             const abs_mask* mask, hipStream_t s, int* frame_mask = nullptr) {
  const int rpg = route_group_rows(g.nb), gph = route_groups_per_head(g.nb);
  int* cnt = (int*)(ws + L.count);
  int* gsum = (int*)(ws + L.gsum);
  if (recount) {
    const int groups = g.B * g.H * gph;
    hipLaunchKernelGGL(route_gsum_kernel, dim3((groups + 255) / 256), dim3(256), 0, s, g, cnt,
                       gsum, rpg, gph);
  }
  hipLaunchKernelGGL(route_csr_kernel, dim3(gph, g.B * g.H), dim3(256), 0, s, g,
                     (const uint32_t*)(ws + L.bitmap), cnt, gsum, rpg, mask->row_ptr,
                     mask->col_idx, mask->head_nnz, (const uint32_t*)(ws + L.fbitmap),
                     route_frame_words(g), frame_mask);
}

hipError_t launch_route(const Geo& g, int dtype, const void* q, const void* k, float p,
                        int k_floor, float slack, const abs_mask* mask, char* ws,
                        const RouteWs& L, hipStream_t s) {
  const bool do_slack = slack > 0.f;
  float* prob = do_slack ? (float*)(ws + L.prob) : nullptr;
  launch_route_front(g, dtype, q, k, p, k_floor, ws, L, prob, s);
  uint32_t* bm = (uint32_t*)(ws + L.bitmap);
  int* cnt = (int*)(ws + L.count);
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
                         g, prob, bm, sel, hist, pass, rpw, g.nb, 0.0f);
      hipLaunchKernelGGL(slack_pick_kernel, dim3(heads), dim3(256), 0, s, sel, hist, pass);
    }
    const int wg4 = (g.rows + 3) / 4;
    hipLaunchKernelGGL(slack_eqcount_kernel, dim3(wg4), dim3(256), 0, s, g, prob, bm, sel, eqcnt,
                       g.nb, 0.0f);
    hipLaunchKernelGGL(slack_eqscan_kernel, dim3(heads), dim3(256), 0, s, g, eqcnt, eqoff, g.nb);
    hipLaunchKernelGGL(slack_mark_kernel, dim3(wg4), dim3(256), 0, s, g, prob, bm, cnt, sel,
                       eqoff, g.nb, 0.0f);
  }
  launch_route_csr(g, ws, L, do_slack, mask, s);
  return hipGetLastError();
}

hipError_t launch_route_dynamic(const Geo& g, int dtype, const void* q, const void* k, float p,
                                int k_floor, float theta, const long long* budget,
                                const abs_mask* mask, char* ws, const RouteWs& L, hipStream_t s) {
  float* prob = (float*)(ws + L.prob);
  launch_route_front(g, dtype, q, k, p, k_floor, ws, L, prob, s);
  uint32_t* bm = (uint32_t*)(ws + L.bitmap);
  int* cnt = (int*)(ws + L.count);
  // one group: the whole batch
  uint32_t* hist = (uint32_t*)(ws + L.hist);
  int* sel = (int*)(ws + L.sel);
  int* eqcnt = (int*)(ws + L.eqcnt);
  int* eqoff = (int*)(ws + L.eqoff);
  hipLaunchKernelGGL(dslack_init_kernel, dim3(1), dim3(256), 0, s, sel, hist, budget);
  const int rpw = 64;
  for (int pass = 0; pass < 3; ++pass) {
    hipLaunchKernelGGL(slack_hist_kernel, dim3((g.rows + rpw - 1) / rpw, 1), dim3(256), 0, s, g,
                       prob, bm, sel, hist, pass, rpw, g.rows, theta);
    hipLaunchKernelGGL(slack_pick_kernel, dim3(1), dim3(256), 0, s, sel, hist, pass);
  }
  const int wg4 = (g.rows + 3) / 4;
  hipLaunchKernelGGL(slack_eqcount_kernel, dim3(wg4), dim3(256), 0, s, g, prob, bm, sel, eqcnt,
                     g.rows, theta);
  hipLaunchKernelGGL(slack_eqscan_kernel, dim3(1), dim3(256), 0, s, g, eqcnt, eqoff, g.rows);
  hipLaunchKernelGGL(slack_mark_kernel, dim3(wg4), dim3(256), 0, s, g, prob, bm, cnt, sel, eqoff,
                     g.rows, theta);
  launch_route_csr(g, ws, L, true, mask, s);
  return hipGetLastError();
}

template <int D, int NC>
static void launch_select_frames_nc(const Geo& g, dim3 grid, const float* qp, const float* kf,
                                    const uint32_t* cand, uint32_t* fbm, int* fcnt, float p,
                                    int k_floor, float scale, hipStream_t s) {
  hipLaunchKernelGGL((route_select_kernel<D, NC, true>), grid, dim3(256), 0, s, g, qp, kf, fbm,
                     fcnt, (int*)nullptr, (float*)nullptr, p, k_floor, scale, cand, g.nb * g.bt,
                     route_frame_words(g));
}

template <int D>
static void launch_select_frames(const Geo& g, dim3 grid, const float* qp, const float* kf,
                                 const uint32_t* cand, uint32_t* fbm, int* fcnt, float p,
                                 int k_floor, float scale, hipStream_t s) {
  const int nch = (g.nb * g.bt + 63) / 64;
#define ABS_SELF(NC_)                                                                     \
  if (nch <= NC_) {                                                                       \
    launch_select_frames_nc<D, NC_>(g, grid, qp, kf, cand, fbm, fcnt, p, k_floor, scale, s); \
    return;                                                                               \
  }
  ABS_SELF(2) ABS_SELF(4) ABS_SELF(6) ABS_SELF(8) ABS_SELF(10) ABS_SELF(12) ABS_SELF(16)
#undef ABS_SELF
}

hipError_t launch_route_frames(const Geo& g, int dtype, const void* q, const void* k, float p,
                               int k_floor, float p_frame, const abs_mask* mask, int* frame_mask,
                               char* ws, const RouteWs& L, hipStream_t s) {
  launch_route_front(g, dtype, q, k, p, k_floor, ws, L, nullptr, s);
  // frame means of K
  float* kf = (float*)(ws + L.kf);
  {
    const int cph = g.d * (dtype == ABS_BF16 ? 2 : 4) / 16;
    int hg = 8;
    while (hg > 1 && (g.H % hg != 0 || hg * cph > 256 || (long)g.B * (g.H / hg) * g.nb < 4096))
      hg /= 2;
    dim3 grid(g.B * (g.H / hg), g.nb);
    if (dtype == ABS_BF16) {
      if (g.d == 128)
        hipLaunchKernelGGL((frame_pool_kernel<bf16_t, 128>), grid, dim3(256), 0, s, g,
                           (const bf16_t*)k, kf, hg);
      else
        hipLaunchKernelGGL((frame_pool_kernel<bf16_t, 64>), grid, dim3(256), 0, s, g,
                           (const bf16_t*)k, kf, hg);
    } else {
      if (g.d == 128)
        hipLaunchKernelGGL((frame_pool_kernel<float, 128>), grid, dim3(256), 0, s, g,
                           (const float*)k, kf, hg);
      else
        hipLaunchKernelGGL((frame_pool_kernel<float, 64>), grid, dim3(256), 0, s, g,
                           (const float*)k, kf, hg);
    }
  }
  const dim3 grid(route_groups_per_head(g.nb), g.B * g.H);
  const float scale = (float)(1.0 / sqrt((double)g.d));
  const float* qp = (const float*)(ws + L.qp);
  const uint32_t* cand = (const uint32_t*)(ws + L.bitmap);
  uint32_t* fbm = (uint32_t*)(ws + L.fbitmap);
  int* fcnt = (int*)(ws + L.fcount);
  if (g.d == 128)
    launch_select_frames<128>(g, grid, qp, kf, cand, fbm, fcnt, p_frame, k_floor, scale, s);
  else
    launch_select_frames<64>(g, grid, qp, kf, cand, fbm, fcnt, p_frame, k_floor, scale, s);
  launch_route_csr(g, ws, L, false, mask, s, frame_mask);
  return hipGetLastError();
}

hipError_t launch_slack_budget(const long long* telem, int n, float fill, long long max_pairs,
                               long long* budget, hipStream_t s) {
  hipLaunchKernelGGL(slack_budget_kernel, dim3(1), dim3(256), 0, s, telem, n, fill, max_pairs,
                     budget);
  return hipGetLastError();
}

}  // namespace abs_impl
