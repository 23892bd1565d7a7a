// Host-side dispatch rules of the Beam MoE library: which kernel family a call takes and how its
// work is cut. Plain C++ (no kernels), shared by the library and its sanitizer build.
#include <algorithm>

#include "common.h"

namespace beam {

int small_block_rows() { return kSmallBlockRows; }
int tiled_block_rows(bool) { return kPipeBlockRows; }
int boundary_max_hidden() { return kBoundaryMaxHidden; }

int router_partial_chunks(const Shape& s) { return s.H / kRouterChunk; }

bool use_partial_route(const Shape& s) {
  return s.T <= kPartialRouteT && router_partial_chunks(s) <= kRouterMaxChunks;
}

bool use_fused_router(const Shape& s, bool x_bf16) {
  return x_bf16 && !use_partial_route(s) && s.E <= 256 && s.E % 16 == 0 &&
         s.H % kRouterChunk == 0 && s.G <= 64 && s.K <= 64;
}

int down_ksplit(int64_t tiles, int64_t k_stages, int n_cu) {
  // Workgroups run one per CU, dealt to the 8 XCDs in contiguous ranges; a grid whose last round
  // is nearly empty leaves most CUs idle for one workgroup's time. Choose the K split (1, 2 or 4)
  // with the fewest rounds per unit of work, charging each extra part a little for its partial-sum
  // traffic; parts keep at least 16 stages.
  const int64_t cu_per_xcd = std::max(1, n_cu / 8);
  int best = 1;
  double best_cost = 1e30;
  for (int ks = 1; ks <= 4; ks *= 2) {
    if (k_stages % ks != 0 || k_stages / ks < 16) continue;
    const int64_t per_xcd = ceil_div(tiles * ks, 8);
    const double rounds = (double)ceil_div(per_xcd, cu_per_xcd);
    const double cost = rounds / ks + 0.05 * (ks - 1);
    if (cost < best_cost - 1e-9) {
      best_cost = cost;
      best = ks;
    }
  }
  return best;
}

}  // namespace beam
