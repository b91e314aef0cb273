// Accepted-path KV compaction ([TR] sec. 2 sequence diagram: the target keeps the KV of
// the approved branch and discards the wrong branches).
//
// The tree's KV sits in slots L .. L+T-1 in node order; keeping the accepted path
// 0 = a_0 < a_1 < ... < a_k moves slot L + a_m to slot L + m (m = 1..k).  Because a
// destination L + m can be the source of another move (a_{m'} = m), one workgroup owns a
// whole (sequence, layer, KV head, K|V) slice and gathers every source row into LDS
// before it writes any destination.  This is a bandwidth-bound copy: 16-byte loads and
// stores, one row per 16 (bf16, d = 128) lanes.
#include "ev_internal.h"

namespace ev {

constexpr int kCompactThreads = 256;
constexpr int kMaxRowBytes = 128 * 4;

struct CompactArgs {
  char *k;
  char *v;
  KvAddr kv;
  int esz;                 // element size in bytes
  int64_t layer_stride;    // elements
  int n_layers;
  const int32_t *prefix_len;
  const int32_t *path;
  const int32_t *accept_len;
  int T;
  int32_t *new_len;
  int32_t *dev_status;
};

__global__ __launch_bounds__(kCompactThreads) void kv_compact_kernel(CompactArgs a) {
  __shared__ __attribute__((aligned(16))) char stage[(kMaxNodes - 1) * kMaxRowBytes];
  __shared__ int bad;
  const int b = blockIdx.x;
  const int z = blockIdx.y;
  const int which = z & 1;
  const int g = (z >> 1) % a.kv.hkv;
  const int layer = (z >> 1) / a.kv.hkv;
  const int tid = threadIdx.x;
  const int L = a.prefix_len[b];
  const int k = a.accept_len[b];
  const int32_t *path = a.path + (int64_t)b * a.T;

  // Validate the path: node 0 first, strictly increasing, inside the tree.
  bool ok = k >= 0 && k < a.T && path[0] == 0;
  for (int m = 1; ok && m <= k; ++m) ok = path[m] > path[m - 1] && path[m] < a.T;
  if (!ok) {
    if (tid == 0 && z == 0) report(a.dev_status, EV_DERR_PATH);
    return;
  }
  if (L < 0 || !a.kv.fits(L + a.T)) {
    if (tid == 0 && z == 0) report(a.dev_status, EV_DERR_BOUNDS);
    return;
  }
  if (tid == 0) bad = 0;
  if (z == 0 && tid == 0) a.new_len[b] = L + k + 1;
  __syncthreads();
  if (k == 0) return;

  char *base = (which ? a.v : a.k) + (int64_t)layer * a.layer_stride * a.esz;
  const int row_bytes = a.kv.d * a.esz;
  const int cpr = row_bytes / 16;           // 16-byte chunks per row
  const int total = k * cpr;
  // gather
  for (int c = tid; c < total; c += kCompactThreads) {
    int m = c / cpr + 1, ch = c % cpr;
    int64_t off = a.kv.slot_offset(b, g, L + path[m]);
    f32x4 val = {};
    if (off >= 0) val = *(const f32x4 *)(base + off * a.esz + ch * 16);
    else bad = 1;
    *(f32x4 *)(stage + (m - 1) * row_bytes + ch * 16) = val;
  }
  __syncthreads();
  if (bad) {
    if (tid == 0) report(a.dev_status, EV_DERR_BOUNDS);
    return;
  }
  // scatter
  for (int c = tid; c < total; c += kCompactThreads) {
    int m = c / cpr + 1, ch = c % cpr;
    int64_t off = a.kv.slot_offset(b, g, L + m);
    if (off >= 0)
      *(f32x4 *)(base + off * a.esz + ch * 16) = *(const f32x4 *)(stage + (m - 1) * row_bytes + ch * 16);
  }
}

}  // namespace ev

EV_API ev_status ev_kv_compact(const ev_kv_desc *kv, const int32_t *prefix_len, const int32_t *path,
                               const int32_t *accept_len, int32_t B, int32_t T, int32_t *new_len,
                               int32_t *dev_status, hipStream_t stream) {
  ev::KvAddr addr;
  ev_status st = ev::make_kv_addr(kv, &addr);
  if (st != EV_OK) return st;
  if (B < 0 || T < 1 || T > ev::kMaxNodes) return EV_ERR_SHAPE;
  if ((int64_t)kv->n_layers * kv->n_kv_heads * 2 > 65535) return EV_ERR_SHAPE;
  if (kv->n_layers > 1 && kv->layer_stride <= 0) return EV_ERR_SHAPE;
  if (B == 0) return EV_OK;
  if (!prefix_len || !path || !accept_len || !new_len) return EV_ERR_NULL;
  ev::CompactArgs a{};
  a.k = (char *)kv->k;
  a.v = (char *)kv->v;
  a.kv = addr;
  a.esz = kv->dtype == EV_F32 ? 4 : 2;
  a.layer_stride = kv->layer_stride;
  a.n_layers = kv->n_layers;
  a.prefix_len = prefix_len;
  a.path = path;
  a.accept_len = accept_len;
  a.T = T;
  a.new_len = new_len;
  a.dev_status = dev_status;
  dim3 grid(B, kv->n_layers * kv->n_kv_heads * 2);
  hipLaunchKernelGGL(ev::kv_compact_kernel, grid, dim3(ev::kCompactThreads), 0, stream, a);
  return ev::launch_status();
}
