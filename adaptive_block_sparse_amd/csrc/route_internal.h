// Routing declarations shared by the library's translation units (the
// attention path does not use them).
#pragma once

#include "internal.h"

namespace abs_impl {

// Routing selects the rows of one head in groups of route_group_rows(nb)
// consecutive query blocks, one workgroup of four waves per group: four rows a
// wave (16 lanes a row) up to 1024 key blocks, one row a wave beyond.
__host__ __device__ inline int route_rows_per_wave(int nb) { return nb <= 1024 ? 4 : 1; }
__host__ __device__ inline int route_group_rows(int nb) { return 4 * route_rows_per_wave(nb); }
__host__ __device__ inline int route_groups_per_head(int nb) {
  return (nb + route_group_rows(nb) - 1) / route_group_rows(nb);
}

// Route workspace layout (byte offsets, all 256-aligned).
struct RouteWs {
  size_t qp, kp;          // float [B*H*nb*d] each
  size_t prob;            // float [rows*nb] probabilities (slack fills only)
  size_t bitmap;          // uint32 [rows*words]
  size_t count;           // int32 [rows]
  size_t gsum;            // int32 [B*H*route_groups_per_head(nb)]: kept blocks per row group
  size_t kf;              // float [B*H*nb*bt*d] frame means of K (fine-grained routing only)
  size_t fbitmap;         // uint32 [rows*route_frame_words]: kept frames (fine-grained only)
  size_t fcount;          // int32 [rows]: kept frames per row (fine-grained only)
  size_t hist;            // uint32 [B*H*2048] slack radix histogram
  size_t sel;             // int32 [B*H*4] slack selection state
  size_t eqcnt, eqoff;    // int32 [rows] each
  size_t total;
};

// 32-bit words of one row's frame bitmap (nb*bt frames)
__host__ __device__ inline int route_frame_words(const Geo& g) { return (g.nb * g.bt + 31) / 32; }

RouteWs route_ws_layout(const Geo& g, bool slack, bool frames = false);

hipError_t launch_route(const Geo& g, int dtype, const void* q, const void* k, float p,
                        int k_floor, float slack, const abs_mask* mask, char* ws,
                        const RouteWs& L, hipStream_t s);
hipError_t launch_route_dynamic(const Geo& g, int dtype, const void* q, const void* k, float p,
                                int k_floor, float theta, const long long* budget,
                                const abs_mask* mask, char* ws, const RouteWs& L, hipStream_t s);
hipError_t launch_route_frames(const Geo& g, int dtype, const void* q, const void* k, float p,
                               int k_floor, float p_frame, const abs_mask* mask, int* frame_mask,
                               char* ws, const RouteWs& L, hipStream_t s);
hipError_t launch_slack_budget(const long long* telem, int n, float fill, long long max_pairs,
                               long long* budget, hipStream_t s);

}  // namespace abs_impl
