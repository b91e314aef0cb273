// Accepted-path KV compaction ([TR] sec. 2 sequence diagram: the target keeps the KV of
// the approved branch and discards the wrong branches).
//
// The tree's KV sits in slots L .. L+T-1 in node order; keeping the accepted path
// 0 = a_0 < a_1 < ... < a_k moves slot L + a_m to slot L + m (m = 1..k).  Because a
// destination L + m can be the source of another move (a_{m'} = m), a workgroup reads
// every source row of a layer into registers before it writes any destination of that
// layer.  One workgroup covers a (sequence, KV head, K|V) slice across a group of layers,
// sized so a launch has about 2048 workgroups; 16-byte loads and stores.
#include "ev_internal.h"

#include <algorithm>

namespace ev {

constexpr int kCompactThreads = 256;
constexpr int kStageChunks = 2048;     // 16-byte chunks staged in LDS (32 KB): a layer's
                                       // rows at most, 63 rows of 512 bytes
constexpr int kCompactWGs = 2048;      // workgroups one launch aims for

struct CompactArgs {
  char *k;
  char *v;
  float *k_scale;          // INT4 caches: one scale per row, moved with it
  float *v_scale;
  KvAddr kv;
  int row_bytes;           // bytes of one (slot, KV head) row
  int64_t layer_stride;    // values
  int n_layers;
  int layers_per_wg;
  const int32_t *prefix_len;
  const int32_t *path;
  const int32_t *accept_len;
  int T;
  int32_t *new_len;
  int32_t *dev_status;
  const uint64_t *copy_mask;   // slots L + m copied (bit m), sequence b at b * mask_stride;
  int mask_stride;             // null: every m (and the path is validated here)
};

// One workgroup per (sequence, KV head, K|V, group of layers).  The rows of one layer are
// all read into LDS before any of them is written (a destination L + m can be the source
// of another move); layers are disjoint, so a pass stages as many whole layers as fit.
__global__ __launch_bounds__(kCompactThreads) void kv_compact_kernel(CompactArgs a) {
  __shared__ f32x4 stage[kStageChunks];
  __shared__ float stage_s[kStageChunks / 2];
  __shared__ int s_path[kMaxNodes];
  __shared__ int s_list[kMaxNodes];
  __shared__ int s_n, s_bad;
  const int b = blockIdx.x;
  const int z = blockIdx.y;
  const int which = z & 1;
  const int g = (z >> 1) % a.kv.hkv;
  const int group = (z >> 1) / a.kv.hkv;
  const int tid = threadIdx.x;
  // the arguments in one batch, then the sequence's copy mask, length, accepted count and
  // path together (loaded where first used they were five dependent round trips)
  args_in_sgprs(a.copy_mask, a.mask_stride, a.prefix_len, a.accept_len, a.path, a.T, a.kv.hkv,
                a.kv.d, a.kv.paged, a.kv.cap, a.n_layers, a.layers_per_wg, a.row_bytes,
                a.layer_stride, a.k, a.v, a.k_scale, a.v_scale);
  const uint64_t mask = a.copy_mask ? a.copy_mask[(int64_t)b * a.mask_stride] : ~0ull;
  const int L = a.prefix_len[b];
  const int k = a.accept_len[b];
  const int pth = tid < kMaxNodes && tid < a.T ? a.path[(int64_t)b * a.T + tid] : -1;
  args_in_sgprs(mask, L, k);
  if (mask == 0) return;                 // remap mode: nothing to copy (or an invalid tree)
  if (tid < kMaxNodes) s_path[tid] = pth;
  if (tid == 0) s_bad = 0;
  __syncthreads();
  if (!a.copy_mask) {
    // validate the path (node 0 first, strictly increasing, inside the tree), the slots
    // and, for a paged cache, the table entries of the tree's blocks
    bool bad_path = k < 0 || k >= a.T || s_path[0] != 0;
    if (!bad_path && tid >= 1 && tid <= k)
      bad_path = !(s_path[tid] > s_path[tid - 1] && s_path[tid] < a.T);
    bool bad_slot = L < 0 || !a.kv.fits(L + a.T);
    if (!bad_slot && a.kv.paged) {
      const int bs = 1 << a.kv.block_shift;
      const int X = L / bs + tid;
      if (X <= (L + a.T - 1) / bs) {
        const int blk = a.kv.table[(int64_t)b * a.kv.max_blocks + X];
        bad_slot = blk < 0 || blk >= a.kv.n_blocks;
      }
    }
    if (bad_path) atomicOr(&s_bad, 1);
    if (bad_slot) atomicOr(&s_bad, 2);
    __syncthreads();
    const int bad = s_bad;
    if (bad) {
      if (tid == 0 && z == 0) report(a.dev_status, (bad & 1) ? EV_DERR_PATH : EV_DERR_BOUNDS);
      return;
    }
    if (z == 0 && tid == 0) a.new_len[b] = L + k + 1;
  }
  // the moves this call makes, in ascending m
  if (tid < 64) {
    const bool mv = tid >= 1 && tid <= k && ((mask >> tid) & 1);
    const uint64_t bal = __ballot(mv);
    if (mv) s_list[__popcll(bal & ((1ull << tid) - 1ull))] = tid;
    if (tid == 0) s_n = __popcll(bal);
  }
  __syncthreads();
  const int n = s_n;
  if (n == 0) return;
  const int l_lo = group * a.layers_per_wg;
  const int l_hi = min(a.n_layers, l_lo + a.layers_per_wg);
  const int cpr = a.row_bytes / 16;      // 16-byte chunks per row: 2 .. 32
  const int cshift = __ffs(cpr) - 1;
  const int dshift = __ffs(a.kv.d) - 1;  // element offset -> row
  const int per_layer = n * cpr;
  const int lpp = max(1, kStageChunks / per_layer);      // whole layers per pass
  const int64_t layer_rows = a.layer_stride >> dshift;
  char *base = which ? a.v : a.k;
  float *scales = which ? a.v_scale : a.k_scale;
  for (int l0 = l_lo; l0 < l_hi; l0 += lpp) {
    const int nl = min(lpp, l_hi - l0);
    for (int li = 0; li < nl; ++li) {
      const int64_t lrow = (int64_t)(l0 + li) * layer_rows;
      for (int r = tid; r < per_layer; r += kCompactThreads) {
        const int mi = r >> cshift, ch = r & (cpr - 1);
        const int64_t row = lrow + (a.kv.slot_offset(b, g, L + s_path[s_list[mi]]) >> dshift);
        stage[li * per_layer + r] = *(const f32x4 *)(base + row * a.row_bytes + ch * 16);
        if (scales && ch == 0) stage_s[li * n + mi] = scales[row];
      }
    }
    __syncthreads();                     // every source of these layers read
    for (int li = 0; li < nl; ++li) {
      const int64_t lrow = (int64_t)(l0 + li) * layer_rows;
      for (int r = tid; r < per_layer; r += kCompactThreads) {
        const int mi = r >> cshift, ch = r & (cpr - 1);
        const int64_t row = lrow + (a.kv.slot_offset(b, g, L + s_list[mi]) >> dshift);
        *(f32x4 *)(base + row * a.row_bytes + ch * 16) = stage[li * per_layer + r];
        if (scales && ch == 0) scales[row] = stage_s[li * n + mi];
      }
    }
    __syncthreads();                     // the stage is refilled by the next pass
  }
}

// Layers per workgroup so that one launch has about kCompactWGs workgroups.
inline int compact_layers_per_wg(int B, int hkv, int n_layers) {
  const int64_t slices = (int64_t)B * hkv * 2;
  const int64_t groups = std::max<int64_t>(1, std::min<int64_t>(n_layers, (kCompactWGs + slices - 1) / slices));
  return (int)((n_layers + groups - 1) / groups);
}

// Zero-copy compaction of a paged cache ([TR] sec. 4: KV fragmentation and the radix
// cache; sec. 2: keep the accepted branch's KV).  Destination slots L+1 .. L+k lie in
// logical blocks X.  A block wholly past the root whose moves share one offset
// D = a_m - m, a multiple of the block size, needs no data movement: D = 0 keeps it in
// place, D > 0 gives X the physical block of X + D/bs.  The other destination blocks are
// written by copying rows, and a remap whose source block receives copies falls back to
// a copy (repeated until stable).  Three launches: the plan (one wavefront per sequence,
// lane j = logical block L/bs + j), the row copies through the unchanged table, and the
// table commit.
struct RemapWs {                       // per sequence, in the caller's workspace
  uint64_t copy_mask;
  int32_t n_stage;                     // table entries to commit from block L / bs on
  int32_t pad;
  int32_t stage[kMaxNodes];
};

enum : int { kBlkNone = 0, kBlkCopy = 1, kBlkKeep = 2, kBlkRemap = 3 };

struct RemapArgs {
  int32_t *table;                      // [B][max_blocks], updated in place by the commit
  int bs, max_blocks, n_blocks;
  const int32_t *prefix_len;
  const int32_t *path;
  const int32_t *accept_len;
  int T;
  RemapWs *ws;
  int32_t *new_len, *freed, *freed_count, *copied;
  int32_t *dev_status;
};

__global__ __launch_bounds__(64) void kv_remap_plan_kernel(RemapArgs a) {
  __shared__ int s_path[kMaxNodes];
  __shared__ int s_cls[kMaxNodes];
  __shared__ int s_ref[kMaxNodes];
  __shared__ int s_old[kMaxNodes];
  const int b = blockIdx.x;
  const int lane = threadIdx.x;
  const int L = a.prefix_len[b];
  const int k = a.accept_len[b];
  const int32_t *path = a.path + (int64_t)b * a.T;
  RemapWs *w = a.ws + b;
  const int pv = lane < a.T ? path[lane] : -1;
  s_path[lane] = pv;
  // node 0 first, strictly increasing, inside the tree (lane m checks step m)
  const int prev = __shfl(pv, max(lane - 1, 0));
  bool ok = k >= 0 && k < a.T && __shfl(pv, 0) == 0;
  ok = ok && !__any(lane >= 1 && lane <= k && !(pv > prev && pv < a.T));
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  const int bs = a.bs;
  const int n_old = L >= 0 ? (L + a.T + bs - 1) / bs : 0;
  if (ok && (L < 0 || n_old > a.max_blocks)) {
    if (lane == 0) report(a.dev_status, EV_DERR_BOUNDS);
    ok = false;
  } else if (!ok && lane == 0) {
    report(a.dev_status, EV_DERR_PATH);
  }
  const int X0 = ok ? L / bs : 0;
  const int X = X0 + lane;
  const bool in_tree = ok && X < n_old;
  const int old = in_tree ? a.table[(int64_t)b * a.max_blocks + X] : -1;
  if (ok && __any(in_tree && (old < 0 || old >= a.n_blocks))) {
    if (lane == 0) report(a.dev_status, EV_DERR_BOUNDS);
    ok = false;
  }
  if (!ok) {                           // nothing is copied or committed
    if (lane == 0) {
      w->copy_mask = 0;
      w->n_stage = 0;
    }
    return;
  }
  // class of block X
  const int m_lo = max(1, X * bs - L), m_hi = min(k, X * bs + bs - 1 - L);
  int cls = kBlkNone, src = -1;
  if (in_tree && m_lo <= m_hi) {
    if (X * bs <= L) {
      cls = kBlkCopy;
    } else {
      const int D = s_path[m_lo] - m_lo;
      bool same = true;
      for (int m = m_lo + 1; m <= m_hi; ++m) same = same && (s_path[m] - m == D);
      if (!same || D % bs != 0) cls = kBlkCopy;
      else if (D == 0) cls = kBlkKeep;
      else {
        cls = kBlkRemap;
        src = X + D / bs;                // < n_old, so src - X0 < 64
      }
    }
  }
  s_cls[lane] = cls;
  s_old[lane] = old;
  // a remap whose source block receives copies becomes a copy, until none is left
  for (;;) {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    const bool demote = cls == kBlkRemap && s_cls[max(src - X0, 0)] == kBlkCopy;
    if (!__any(demote)) break;
    __builtin_amdgcn_wave_barrier();
    if (demote) {
      cls = kBlkCopy;
      s_cls[lane] = cls;
    }
  }
  // copies: slot L + m (lane m) when its block is a copy block
  const bool copy_m = lane >= 1 && lane <= k && s_cls[(L + lane) / bs - X0] == kBlkCopy;
  const uint64_t mask = __ballot(copy_m);
  // the new table of the tree's blocks
  const int n_new = (L + k + 1 + bs - 1) / bs;
  int nw = old;
  if (in_tree) {
    if (X >= n_new) nw = -1;
    else if (cls == kBlkRemap) nw = s_old[max(src - X0, 0)];
  }
  // freed: the tree's old blocks no live block references any more.  A live block keeps
  // its own entry unless it is remapped, in which case it takes its source's entry (the
  // entries of a sequence's blocks are distinct, as an allocator hands them out).
  s_ref[lane] = 0;
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  if (in_tree && X < n_new) s_ref[cls == kBlkRemap ? max(src - X0, 0) : lane] = 1;
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  const bool fr = in_tree && !s_ref[lane];
  const uint64_t fm = __ballot(fr);
  if (fr) a.freed[(int64_t)b * a.max_blocks + __popcll(fm & ((1ull << lane) - 1ull))] = old;
  w->stage[lane] = nw;
  if (lane == 0) {
    w->copy_mask = mask;
    w->n_stage = n_old - X0;
    a.new_len[b] = L + k + 1;
    a.freed_count[b] = __popcll(fm);
    a.copied[b] = __popcll(mask);
  }
}

__global__ __launch_bounds__(64) void kv_remap_commit_kernel(RemapArgs a) {
  const int b = blockIdx.x;
  const RemapWs *w = a.ws + b;
  const int lane = threadIdx.x;
  if (lane < w->n_stage)
    a.table[(int64_t)b * a.max_blocks + a.prefix_len[b] / a.bs + lane] = w->stage[lane];
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
  if (kv->n_layers > 1 && (kv->layer_stride <= 0 || kv->layer_stride % kv->head_dim)) return EV_ERR_SHAPE;
  if (B == 0) return EV_OK;
  if (!prefix_len || !path || !accept_len || !new_len) return EV_ERR_NULL;
  ev::CompactArgs a{};
  a.k = (char *)kv->k;
  a.v = (char *)kv->v;
  a.kv = addr;
  a.row_bytes = kv->dtype == EV_F32 ? 4 * kv->head_dim
               : kv->dtype == EV_BF16 ? 2 * kv->head_dim : kv->head_dim / 2;
  a.k_scale = kv->dtype == EV_INT4 ? const_cast<float *>(kv->k_scale) : nullptr;
  a.v_scale = kv->dtype == EV_INT4 ? const_cast<float *>(kv->v_scale) : nullptr;
  a.layer_stride = kv->layer_stride;
  a.n_layers = kv->n_layers;
  a.prefix_len = prefix_len;
  a.path = path;
  a.accept_len = accept_len;
  a.T = T;
  a.new_len = new_len;
  a.dev_status = dev_status;
  a.layers_per_wg = ev::compact_layers_per_wg(B, kv->n_kv_heads, kv->n_layers);
  const int groups = (kv->n_layers + a.layers_per_wg - 1) / a.layers_per_wg;
  dim3 grid(B, groups * kv->n_kv_heads * 2);
  hipLaunchKernelGGL(ev::kv_compact_kernel, grid, dim3(ev::kCompactThreads), 0, stream, a);
  return ev::launch_status();
}

EV_API size_t ev_kv_compact_remap_workspace(int32_t B) {
  if (B < 1) return 0;
  return ev::align_up((size_t)B * sizeof(ev::RemapWs), 256);
}

EV_API ev_status ev_kv_compact_remap(const ev_kv_desc *kv, const int32_t *prefix_len,
                                     const int32_t *path, const int32_t *accept_len, int32_t B,
                                     int32_t T, int32_t *new_len, int32_t *freed,
                                     int32_t *freed_count, int32_t *copied, void *ws,
                                     size_t ws_bytes, int32_t *dev_status, hipStream_t stream) {
  ev::KvAddr addr;
  ev_status st = ev::make_kv_addr(kv, &addr);
  if (st != EV_OK) return st;
  if (!kv->paged) return EV_ERR_ARG;
  if (B < 0 || T < 1 || T > ev::kMaxNodes) return EV_ERR_SHAPE;
  if ((int64_t)kv->n_layers * kv->n_kv_heads * 2 > 65535) return EV_ERR_SHAPE;
  if (kv->n_layers > 1 && (kv->layer_stride <= 0 || kv->layer_stride % kv->head_dim)) return EV_ERR_SHAPE;
  if (B == 0) return EV_OK;
  if (!prefix_len || !path || !accept_len || !new_len || !freed || !freed_count || !copied)
    return EV_ERR_NULL;
  if (!ws || ws_bytes < ev_kv_compact_remap_workspace(B)) return EV_ERR_WORKSPACE;
  // the table the descriptor points to is the caller's writable device array
  ev::RemapArgs r{const_cast<int32_t *>(kv->block_table), kv->block_size, kv->max_blocks_per_seq, kv->n_blocks,
                  prefix_len, path, accept_len, T, (ev::RemapWs *)ws, new_len, freed,
                  freed_count, copied, dev_status};
  hipLaunchKernelGGL(ev::kv_remap_plan_kernel, dim3(B), dim3(64), 0, stream, r);
  ev::CompactArgs a{};
  a.k = (char *)kv->k;
  a.v = (char *)kv->v;
  a.kv = addr;
  a.row_bytes = kv->dtype == EV_F32 ? 4 * kv->head_dim
               : kv->dtype == EV_BF16 ? 2 * kv->head_dim : kv->head_dim / 2;
  a.k_scale = kv->dtype == EV_INT4 ? const_cast<float *>(kv->k_scale) : nullptr;
  a.v_scale = kv->dtype == EV_INT4 ? const_cast<float *>(kv->v_scale) : nullptr;
  a.layer_stride = kv->layer_stride;
  a.n_layers = kv->n_layers;
  a.prefix_len = prefix_len;
  a.path = path;
  a.accept_len = accept_len;
  a.T = T;
  a.new_len = new_len;
  a.dev_status = dev_status;
  a.copy_mask = &((const ev::RemapWs *)ws)->copy_mask;
  static_assert(sizeof(ev::RemapWs) % sizeof(uint64_t) == 0, "mask stride");
  a.mask_stride = (int)(sizeof(ev::RemapWs) / sizeof(uint64_t));
  a.layers_per_wg = ev::compact_layers_per_wg(B, kv->n_kv_heads, kv->n_layers);
  const int groups = (kv->n_layers + a.layers_per_wg - 1) / a.layers_per_wg;
  dim3 grid(B, groups * kv->n_kv_heads * 2);
  hipLaunchKernelGGL(ev::kv_compact_kernel, grid, dim3(ev::kCompactThreads), 0, stream, a);
  hipLaunchKernelGGL(ev::kv_remap_commit_kernel, dim3(B), dim3(64), 0, stream, r);
  return ev::launch_status();
}
