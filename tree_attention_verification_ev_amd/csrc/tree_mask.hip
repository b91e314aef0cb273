// Ancestor bitmask of each drafted tree ([TR] sec. 2, mask equation M: node i may attend
// to tree node j exactly when j is i itself or one of its ancestors).
//
// One wavefront per sequence, lane i owns node i (T <= 64).  The mask is built by pointer
// doubling over the parent links: after round r every lane knows the set of its
// ancestors within distance 2^r and the node 2^r levels up, so six rounds cover any
// 64-node tree.  depth[i] is the popcount of the final set minus one.
#include "ev_internal.h"

namespace ev {

__global__ __launch_bounds__(64) void tree_mask_kernel(const int32_t *__restrict__ parent,
                                                        int32_t T, uint64_t *__restrict__ anc,
                                                        int32_t *__restrict__ depth,
                                                        int32_t *dev_status) {
  args_in_sgprs(parent, T, anc, depth);
  const int b = blockIdx.x;
  const int i = threadIdx.x;
  const bool live = i < T;
  int p = live ? parent[(int64_t)b * T + i] : -1;
  // Topological check: the root has parent -1, every other node an earlier node.
  bool ok = !live || (i == 0 ? p == -1 : (p >= 0 && p < i));
  if (__any(!ok)) {
    if (i == 0) report(dev_status, EV_DERR_PARENT);
    return;
  }
  // set = nodes within distance 2^r above i (including i); up = node 2^r levels up or -1
  uint64_t set = live ? (1ull << i) : 0ull;
  int up = p;
  for (int r = 0; r < 6; ++r) {
    int src = up < 0 ? i : up;
    uint64_t s_up = __shfl(set, src);   // ancestors of `up` within distance 2^r
    int up_up = __shfl(up, src);
    if (up >= 0) {
      set |= s_up;
      up = up_up;
    }
  }
  if (live) {
    anc[(int64_t)b * T + i] = set;
    if (depth) depth[(int64_t)b * T + i] = __popcll(set) - 1;
  }
}

}  // namespace ev

EV_API ev_status ev_tree_mask_build(const int32_t *parent, int32_t B, int32_t T,
                                    uint64_t *anc_mask, int32_t *depth, int32_t *dev_status,
                                    hipStream_t stream) {
  if (B < 0 || T < 1 || T > ev::kMaxNodes) return EV_ERR_SHAPE;
  if (B == 0) return EV_OK;
  if (!parent || !anc_mask) return EV_ERR_NULL;
  hipLaunchKernelGGL(ev::tree_mask_kernel, dim3(B), dim3(64), 0, stream, parent, T, anc_mask,
                     depth, dev_status);
  return ev::launch_status();
}
