// Internal launch interface between the C ABI (api.hip) and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace pisa {

struct AttnArgs {
  const void* Q;
  const void* K;
  const void* V;
  const int32_t* idx;
  int kmax;
  const float* centroid;
  const float* vsum;
  const float* hbar;
  const void* packed;   // nullable bf16 pack of the statistics
  const void* ht;       // bf16 H_j^T per block (FIRST order, bf16 path)
  const float* H;       // fp32 H_j per block (FIRST order, fp32 path)
  int approx;           // 0: keep-or-drop, 1: add the unselected blocks
  int order;            // with approx: kOrderMixed / kOrderZeroth / kOrderFirst
  float scale;
  void* O;
  int bh;   // batch * heads
  int nb;   // blocks per sequence
  int D;
  int BLK;
  const int32_t* lens;  // nullable device [batch]: valid length of each sequence
  int heads;
  hipStream_t stream;
  // in-kernel routing (bf16): route_k > 0 selects each query block's route_k
  // blocks inside the attention kernel (idx unused); idx_out receives them
  const float* M;
  int route_k;
  double route_scale;
  double route_lam;
  int32_t* idx_out;     // nullable
  // split work items (bf16): cap > 0 runs an item whose exact list holds more
  // than cap blocks as several parts and merges them (split_ws: workspace)
  int split_cap;
  void* split_ws;
};

struct StatsArgs {
  const void* K;
  const void* V;
  float* centroid;
  float* vsum;
  float* H;      // nullable
  float* hbar;
  float* M;
  void* packed;  // nullable bf16 pack of the statistics
  void* ht;      // nullable bf16 H_j^T per block
  void* ws;
  int spectral;  // M_j as the largest singular value (bf16 path: needs H)
  int bh;
  int nb;
  int D;
  int BLK;
  const int32_t* lens;
  int heads;
  hipStream_t stream;
};

struct RouteArgs {
  const void* Q;
  const float* centroid;
  const float* M;
  int k;
  double scale;
  double lam;
  int32_t* idx;
  int bh;
  int nb;
  int D;
  int BLK;
  const int32_t* lens;
  int heads;
  hipStream_t stream;
};

// first-order treatment of the unselected blocks
constexpr int kOrderMixed = 0;    // global Hbar correction
constexpr int kOrderZeroth = 1;   // none
constexpr int kOrderFirst = 2;    // per-block H_j

// largest nb (= L / block) the kernels accept
constexpr int kMaxBlocks = 2048;

size_t stats_workspace_bf16(int bh, int nb, int D, int BLK);
size_t stats_workspace_f32(int bh, int nb, int D);
size_t stats_packed_bytes(int bh, int nb, int D, int BLK);

hipError_t launch_attn_bf16(const AttnArgs& a);
// workspace bytes of a split attention launch (bf16)
size_t attn_split_workspace(int D, int BLK, int bh, int nb, int kmax, int cap);
// largest nb whose in-kernel routing fits the attention kernel's LDS (bf16)
int fused_route_max_blocks(int D, int BLK);
// in-kernel routing (bf16): the launch's work items, and how many of its
// workgroups the current device holds at once over all CUs (<= 0 when the
// runtime cannot say)
int fused_route_items(int D, int BLK, int bh, int nb);
int fused_route_resident(int D, int BLK);
hipError_t launch_attn_f32(const AttnArgs& a);
hipError_t launch_stats_bf16(const StatsArgs& a);
hipError_t launch_stats_f32(const StatsArgs& a);
hipError_t launch_route_bf16(const RouteArgs& a);
hipError_t launch_route_f32(const RouteArgs& a);

}  // namespace pisa
