// Tree-masked attention over a KV prefix plus each node's ancestors.
//
// What is computed ([TR] sec. 2, sequence diagram and mask equation M; [EX] "Core idea"):
// for sequence b, query head h (KV head g = h / G) and tree node i, the keys are every
// prefix slot 0..L_b-1 and the tree slots L_b + j with bit j of anc[b][i] set; the result
// is softmax(sm_scale * q k^T) v and the natural-log normaliser LSE.
//
// gfx950 design (bf16):
//   * Work unit = (sequence, KV head, block of query rows, range of key tiles).  The rows
//     of a unit are the T*G (node, q-head-in-group) pairs that share one KV head, so a
//     grouped-query layer reuses each K/V byte G*T times.
//   * A workgroup of NW wavefronts stages 64-key tiles of K (row-major) and V (transposed)
//     in LDS; each wavefront owns QT tiles of 32 query rows.
//   * Scores are computed transposed, S^T = K Q^T, with v_mfma_f32_32x32x16_bf16:
//     the accumulator column is the query, so every lane holds 16 keys of ONE query and
//     the softmax statistics, the rescale of the output and the final normalisation are
//     lane-local (only the row max crosses the two wave halves).
//   * K rows are fed to the matrix core in a permuted order (bits 2 and 3 of the row
//     index swapped) so that the score accumulator, converted to bf16, is directly the
//     B operand of O^T += V^T P^T for 16 consecutive keys — no shuffle of P.
//   * The output accumulator is O^T (head_dim x 32 queries), again lane-local per query.
//   * The online softmax runs in float32 in base 2 (scale folded into one FMA before
//     exp2); only tiles that reach past the prefix apply the ancestor bitmask.
//   * Long prefixes are split across workgroups; each split writes a partial (O, LSE)
//     in float32 and a merge kernel combines them.
// float32 path: a plain VALU kernel (one wavefront per (sequence, head, node)).
#include "ev_internal.h"

#include <math.h>

namespace ev {

constexpr int kKT = 64;                 // keys per tile
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

struct AttnArgs {
  const void *q;
  const void *k;
  const void *v;
  KvAddr kv;
  const int32_t *prefix_len;
  const uint64_t *anc;
  int B, T, Hq, G;
  float scale_log2;        // sm_scale * log2(e)
  int tiles_per_split;
  int n_splits;
  void *out;               // final O (n_splits == 1)
  float *lse;              // final LSE (n_splits == 1)
  float *part_o;           // [n_splits][B][T][Hq][D] (n_splits > 1)
  float *part_lse;         // [n_splits][B][T][Hq]
  int32_t *dev_status;
};

// Is logical slot `slot` visible to a query whose ancestor row is `anc` (prefix length L)?
__device__ inline bool visible(int slot, int L, uint64_t anc) {
  int j = slot - L;
  return j < 0 || (j < 64 && ((anc >> j) & 1ull));
}

// MFMA row index -> key within a 32-key subtile: swap bits 2 and 3.
__device__ inline int swap23(int r) { return (r & ~12) | ((r & 4) << 1) | ((r & 8) >> 1); }

template <int D, int QT, int NW>
__global__ __launch_bounds__(NW * 64) void tree_attn_bf16_kernel(AttnArgs a) {
  constexpr int KS = D / 16;            // k-steps of the score product
  constexpr int DT = D / 32;            // 32-row tiles of O^T
  constexpr int KP = D + 8;             // LDS pitch of the K tile (elements)
  constexpr int VP = kKT + 8;           // LDS pitch of the V^T tile (elements)
  constexpr int NT = NW * 64;
  __shared__ __attribute__((aligned(16))) __bf16 sK[kKT * KP];
  __shared__ __attribute__((aligned(16))) __bf16 sV[D * VP];

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int qn = lane & 31;             // query column of this lane
  const int hh = lane >> 5;             // wave half

  const int split = blockIdx.x;
  const int rb = blockIdx.y;
  const int b = blockIdx.z / a.kv.hkv;
  const int g = blockIdx.z % a.kv.hkv;
  const int L = a.prefix_len[b];
  const int nkeys = L + a.T;
  if (L < 0 || !a.kv.fits(nkeys)) {
    if (threadIdx.x == 0) report(a.dev_status, EV_DERR_BOUNDS);
    return;
  }
  const int ntiles = (nkeys + kKT - 1) / kKT;
  const int t_begin = split * a.tiles_per_split;
  const int t_end = min(t_begin + a.tiles_per_split, ntiles);
  if (t_begin >= t_end) return;         // this split lies beyond the sequence

  const int rows = a.T * a.G;
  const int row0 = (rb * NW + wave) * QT * 32;
  const __bf16 *Q = (const __bf16 *)a.q;
  const __bf16 *K = (const __bf16 *)a.k;
  const __bf16 *V = (const __bf16 *)a.v;

  // Q^T fragments (B operand): lane holds query row qn, 8 head-dim elements per k-step.
  bf16x8 qf[QT][KS];
  uint64_t anc_q[QT];
#pragma unroll
  for (int t = 0; t < QT; ++t) {
    int r = row0 + t * 32 + qn;
    bool ok = r < rows;
    int node = ok ? r / a.G : 0;
    int head = g * a.G + (ok ? r % a.G : 0);
    const __bf16 *src = Q + (((int64_t)b * a.T + node) * a.Hq + head) * D + 8 * hh;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      bf16x8 z = {};
      qf[t][ks] = ok ? *(const bf16x8 *)(src + 16 * ks) : z;
    }
    anc_q[t] = ok ? a.anc[(int64_t)b * a.T + node] : 0ull;
  }

  f32x16 o[QT][DT];
  float m[QT], l[QT];
#pragma unroll
  for (int t = 0; t < QT; ++t) {
    m[t] = -INFINITY;
    l[t] = 0.f;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) o[t][dt] = f32x16{};
  }

  for (int tile = t_begin; tile < t_end; ++tile) {
    const int key0 = tile * kKT;
    __syncthreads();
    // ---- stage K tile (row-major) ----
    for (int c = threadIdx.x; c < kKT * (D / 8); c += NT) {
      int key = c / (D / 8), dc = c % (D / 8);
      int slot = key0 + key;
      bf16x8 val = {};
      if (slot < nkeys) {
        int64_t off = a.kv.slot_offset(b, g, slot);
        if (off >= 0) val = *(const bf16x8 *)(K + off + dc * 8);
        else report(a.dev_status, EV_DERR_BOUNDS);
      }
      *(bf16x8 *)(sK + key * KP + dc * 8) = val;
    }
    // ---- stage V tile transposed: 4 keys x 8 dims per item ----
    for (int c = threadIdx.x; c < (kKT / 4) * (D / 8); c += NT) {
      int kq = c % (kKT / 4), dc = c / (kKT / 4);
      bf16x8 rows4[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        int slot = key0 + 4 * kq + r;
        bf16x8 val = {};
        if (slot < nkeys) {
          int64_t off = a.kv.slot_offset(b, g, slot);
          if (off >= 0) val = *(const bf16x8 *)(V + off + dc * 8);
        }
        rows4[r] = val;
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        bf16x4 col = {rows4[0][e], rows4[1][e], rows4[2][e], rows4[3][e]};
        *(bf16x4 *)(sV + (dc * 8 + e) * VP + 4 * kq) = col;
      }
    }
    __syncthreads();

    const bool need_mask = key0 + kKT > L;
    // ---- S^T = K Q^T for two 32-key subtiles ----
    f32x16 s[QT][2];
#pragma unroll
    for (int st = 0; st < 2; ++st) {
#pragma unroll
      for (int t = 0; t < QT; ++t) s[t][st] = f32x16{};
      const __bf16 *krow = sK + (st * 32 + swap23(qn)) * KP + 8 * hh;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        bf16x8 kf = *(const bf16x8 *)(krow + 16 * ks);
#pragma unroll
        for (int t = 0; t < QT; ++t)
          s[t][st] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[t][ks], s[t][st], 0, 0, 0);
      }
    }

    // ---- online softmax (base 2), lane-local per query ----
    bf16x8 pf[QT][2][2];
#pragma unroll
    for (int t = 0; t < QT; ++t) {
      if (need_mask) {
#pragma unroll
        for (int st = 0; st < 2; ++st)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            int j = r >> 2, i = r & 3;
            int key = st * 32 + (j >> 1) * 16 + hh * 8 + (j & 1) * 4 + i;
            if (!visible(key0 + key, L, anc_q[t])) s[t][st][r] = -INFINITY;
          }
      }
      float mx = -INFINITY;
#pragma unroll
      for (int st = 0; st < 2; ++st)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[t][st][r]);
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      const float m_new = fmaxf(m[t], mx);
      const float m_use = m_new == -INFINITY ? 0.f : m_new;
      const float alpha = exp2f((m[t] - m_use) * a.scale_log2);
      const float nb = -m_use * a.scale_log2;
      float sum = 0.f;
#pragma unroll
      for (int st = 0; st < 2; ++st)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          float p = exp2f(fmaf(s[t][st][r], a.scale_log2, nb));
          s[t][st][r] = p;
          sum += p;
        }
      l[t] = l[t] * alpha + sum;
      m[t] = m_new;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) o[t][dt] *= alpha;
#pragma unroll
      for (int st = 0; st < 2; ++st)
#pragma unroll
        for (int kk = 0; kk < 2; ++kk)
#pragma unroll
          for (int e = 0; e < 8; ++e) pf[t][st][kk][e] = (__bf16)s[t][st][kk * 8 + e];
    }

    // ---- O^T += V^T P^T, 16 keys per step ----
#pragma unroll
    for (int st = 0; st < 2; ++st)
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
          bf16x8 vf = *(const bf16x8 *)(sV + (dt * 32 + qn) * VP + st * 32 + kk * 16 + 8 * hh);
#pragma unroll
          for (int t = 0; t < QT; ++t)
            o[t][dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pf[t][st][kk], o[t][dt], 0, 0, 0);
        }
      }
  }

  // ---- epilogue: normalise and write (final or partial) ----
#pragma unroll
  for (int t = 0; t < QT; ++t) {
    int r = row0 + t * 32 + qn;
    float ltot = l[t] + __shfl_xor(l[t], 32);
    if (r >= rows) continue;
    int node = r / a.G;
    int head = g * a.G + r % a.G;
    int64_t orow = ((int64_t)b * a.T + node) * a.Hq + head;
    float inv = ltot > 0.f ? 1.f / ltot : 0.f;
    float lse = ltot > 0.f ? (m[t] * a.scale_log2 + log2f(ltot)) * kLn2 : -INFINITY;
    if (a.n_splits == 1) {
      __bf16 *dst = (__bf16 *)a.out + orow * D;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          bf16x4 w;
#pragma unroll
          for (int i = 0; i < 4; ++i) w[i] = (__bf16)(o[t][dt][4 * j + i] * inv);
          *(bf16x4 *)(dst + dt * 32 + 8 * j + 4 * hh) = w;
        }
      if (hh == 0) a.lse[orow] = lse;
    } else {
      int64_t prow = (int64_t)split * a.B * a.T * a.Hq + orow;
      float *dst = a.part_o + prow * D;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          f32x4 w;
#pragma unroll
          for (int i = 0; i < 4; ++i) w[i] = o[t][dt][4 * j + i] * inv;
          *(f32x4 *)(dst + dt * 32 + 8 * j + 4 * hh) = w;
        }
      if (hh == 0) a.part_lse[prow] = lse;
    }
  }
}

// Combine split partials: lse = log sum_s exp(lse_s), O = sum_s exp(lse_s - lse) O_s.
// One row (sequence, node, head) per 32 lanes, 4 head-dim elements per lane.
template <int D, typename OutT>
__global__ __launch_bounds__(256) void attn_merge_kernel(AttnArgs a) {
  const int64_t nrows = (int64_t)a.B * a.T * a.Hq;
  const int64_t row = (int64_t)blockIdx.x * 8 + (threadIdx.x >> 5);
  const int c = threadIdx.x & 31;
  if (row >= nrows) return;
  const int b = (int)(row / ((int64_t)a.T * a.Hq));
  const int L = a.prefix_len[b];
  if (L < 0 || !a.kv.fits(L + a.T)) return;
  const int ntiles = (L + a.T + kKT - 1) / kKT;
  const int nvalid = min(a.n_splits, (ntiles + a.tiles_per_split - 1) / a.tiles_per_split);
  const int64_t stride = nrows;
  float mx = -INFINITY;
  for (int s = 0; s < nvalid; ++s) mx = fmaxf(mx, a.part_lse[s * stride + row]);
  float acc[D / 32] = {};
  float wsum = 0.f;
  for (int s = 0; s < nvalid; ++s) {
    float ls = a.part_lse[s * stride + row];
    float w = ls == -INFINITY ? 0.f : exp2f((ls - mx) * kLog2e);
    wsum += w;
    if (w == 0.f) continue;
    const float *src = a.part_o + (s * stride + row) * D;
#pragma unroll
    for (int k = 0; k < D / 32; ++k) acc[k] += w * src[c + 32 * k];
  }
  float inv = wsum > 0.f ? 1.f / wsum : 0.f;
  OutT *dst = (OutT *)a.out + row * D;
#pragma unroll
  for (int k = 0; k < D / 32; ++k) dst[c + 32 * k] = (OutT)(acc[k] * inv);
  if (c == 0) a.lse[row] = wsum > 0.f ? mx + logf(wsum) : -INFINITY;
}

// float32 path: one wavefront per (sequence, q-head, node); lane j scores key j of each
// 64-key tile, the tile's probabilities go through LDS, lane d accumulates O[d].
template <int D>
__global__ __launch_bounds__(64) void tree_attn_f32_kernel(AttnArgs a) {
  __shared__ float sq[D];
  __shared__ float sp[64];
  const int lane = threadIdx.x;
  const int node = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int g = h / a.G;
  const int L = a.prefix_len[b];
  const int nkeys = L + a.T;
  if (L < 0 || !a.kv.fits(nkeys)) {
    if (lane == 0) report(a.dev_status, EV_DERR_BOUNDS);
    return;
  }
  const float *Q = (const float *)a.q;
  const float *K = (const float *)a.k;
  const float *V = (const float *)a.v;
  const int64_t orow = ((int64_t)b * a.T + node) * a.Hq + h;
  for (int d = lane; d < D; d += 64) sq[d] = Q[orow * D + d];
  const uint64_t anc = a.anc[(int64_t)b * a.T + node];
  __syncthreads();
  float m = -INFINITY, l = 0.f;
  float o[D / 64] = {};
  for (int key0 = 0; key0 < nkeys; key0 += 64) {
    int slot = key0 + lane;
    float sc = -INFINITY;
    if (slot < nkeys && visible(slot, L, anc)) {
      int64_t off = a.kv.slot_offset(b, g, slot);
      if (off >= 0) {
        float acc = 0.f;
        for (int d = 0; d < D; ++d) acc = fmaf(sq[d], K[off + d], acc);
        sc = acc * a.scale_log2;
      } else {
        report(a.dev_status, EV_DERR_BOUNDS);
      }
    }
    float mx = sc;
    for (int w = 32; w >= 1; w >>= 1) mx = fmaxf(mx, __shfl_xor(mx, w));
    float m_new = fmaxf(m, mx);
    float m_use = m_new == -INFINITY ? 0.f : m_new;
    float alpha = exp2f(m - m_use);
    float p = exp2f(sc - m_use);
    float ps = p;
    for (int w = 32; w >= 1; w >>= 1) ps += __shfl_xor(ps, w);
    l = l * alpha + ps;
    m = m_new;
    __syncthreads();
    sp[lane] = p;
    __syncthreads();
    int cnt = min(64, nkeys - key0);
#pragma unroll
    for (int k = 0; k < D / 64; ++k) o[k] *= alpha;
    for (int j = 0; j < cnt; ++j) {
      float pj = sp[j];
      if (pj == 0.f) continue;
      int64_t off = a.kv.slot_offset(b, g, key0 + j);
#pragma unroll
      for (int k = 0; k < D / 64; ++k) o[k] = fmaf(pj, V[off + lane + 64 * k], o[k]);
    }
  }
  float inv = l > 0.f ? 1.f / l : 0.f;
  float lse = l > 0.f ? (m + log2f(l)) * kLn2 : -INFINITY;
  if (a.n_splits == 1) {
#pragma unroll
    for (int k = 0; k < D / 64; ++k) ((float *)a.out)[orow * D + lane + 64 * k] = o[k] * inv;
    if (lane == 0) a.lse[orow] = lse;
  }
}

// ---------------------------------------------------------------------------------------
// Launch policy.
struct Plan {
  int qt, nw;            // query tiles per wave, waves per workgroup
  int row_blocks;
  int tiles_per_split, n_splits;
};

static int max_slots(const KvAddr &kv) {
  if (!kv.paged) return (int)std::min<int64_t>(kv.cap, 1 << 30);
  return kv.max_blocks << kv.block_shift;
}

static Plan make_plan(const KvAddr &kv, int dtype, int B, int T, int Hq) {
  Plan p{};
  if (dtype == EV_F32) {
    p.qt = p.nw = p.row_blocks = 1;
    p.tiles_per_split = 1 << 30;
    p.n_splits = 1;
    return p;
  }
  const int G = Hq / kv.hkv;
  const int rows = T * G;
  p.qt = rows >= 256 ? 2 : 1;
  const int wave_rows = 32 * p.qt;
  const int waves_needed = (rows + wave_rows - 1) / wave_rows;
  p.nw = waves_needed >= 4 ? 4 : waves_needed;
  p.row_blocks = (waves_needed + p.nw - 1) / p.nw;
  const int max_tiles = (max_slots(kv) + kKT - 1) / kKT;
  const int units = B * kv.hkv * p.row_blocks;
  // Aim for about two workgroups per compute unit, at least 4 tiles per split.
  const int target_wgs = 512;
  int splits = (target_wgs + units - 1) / units;
  int tps = (max_tiles + splits - 1) / splits;
  if (tps < 4) tps = 4;
  p.tiles_per_split = tps;
  p.n_splits = (max_tiles + tps - 1) / tps;
  if (p.n_splits < 1) p.n_splits = 1;
  return p;
}

static size_t workspace_bytes(const Plan &p, int B, int T, int Hq, int D) {
  if (p.n_splits <= 1) return 0;
  size_t rows = (size_t)p.n_splits * B * T * Hq;
  return align_up(rows * D * sizeof(float), 256) + align_up(rows * sizeof(float), 256);
}

template <int D>
static void launch_bf16(const Plan &p, const AttnArgs &a, hipStream_t stream) {
  dim3 grid(p.n_splits, p.row_blocks, a.B * a.kv.hkv);
  if (p.qt == 2) {
    hipLaunchKernelGGL((tree_attn_bf16_kernel<D, 2, 4>), grid, dim3(256), 0, stream, a);
  } else if (p.nw == 4) {
    hipLaunchKernelGGL((tree_attn_bf16_kernel<D, 1, 4>), grid, dim3(256), 0, stream, a);
  } else if (p.nw == 2) {
    hipLaunchKernelGGL((tree_attn_bf16_kernel<D, 1, 2>), grid, dim3(128), 0, stream, a);
  } else if (p.nw == 3) {
    hipLaunchKernelGGL((tree_attn_bf16_kernel<D, 1, 3>), grid, dim3(192), 0, stream, a);
  } else {
    hipLaunchKernelGGL((tree_attn_bf16_kernel<D, 1, 1>), grid, dim3(64), 0, stream, a);
  }
  if (p.n_splits > 1) {
    int64_t nrows = (int64_t)a.B * a.T * a.Hq;
    hipLaunchKernelGGL((attn_merge_kernel<D, __bf16>), dim3((unsigned)((nrows + 7) / 8)),
                       dim3(256), 0, stream, a);
  }
}

}  // namespace ev

EV_API size_t ev_tree_attention_workspace(const ev_kv_desc *kv, int32_t B, int32_t T, int32_t Hq) {
  ev::KvAddr addr;
  if (ev::make_kv_addr(kv, &addr) != EV_OK || B < 1 || T < 1 || T > ev::kMaxNodes || Hq < 1 ||
      Hq % kv->n_kv_heads)
    return 0;
  ev::Plan p = ev::make_plan(addr, kv->dtype, B, T, Hq);
  return ev::workspace_bytes(p, B, T, Hq, kv->head_dim);
}

EV_API ev_status ev_tree_attention(const void *q, const ev_kv_desc *kv, const int32_t *prefix_len,
                                   const uint64_t *anc_mask, int32_t B, int32_t T, int32_t Hq,
                                   float sm_scale, void *out, float *lse, void *ws,
                                   size_t ws_bytes, int32_t *dev_status, hipStream_t stream) {
  ev::KvAddr addr;
  ev_status st = ev::make_kv_addr(kv, &addr);
  if (st != EV_OK) return st;
  if (B < 0 || T < 1 || T > ev::kMaxNodes || Hq < 1 || Hq % kv->n_kv_heads) return EV_ERR_SHAPE;
  if (!(sm_scale > 0.f) || !isfinite(sm_scale)) return EV_ERR_ARG;
  if (B == 0) return EV_OK;
  if (!q || !prefix_len || !anc_mask || !out || !lse) return EV_ERR_NULL;
  ev::Plan p = ev::make_plan(addr, kv->dtype, B, T, Hq);
  size_t need = ev::workspace_bytes(p, B, T, Hq, kv->head_dim);
  if (ws_bytes < need || (need && !ws)) return EV_ERR_WORKSPACE;

  ev::AttnArgs a{};
  a.q = q;
  a.k = kv->k;
  a.v = kv->v;
  a.kv = addr;
  a.prefix_len = prefix_len;
  a.anc = anc_mask;
  a.B = B;
  a.T = T;
  a.Hq = Hq;
  a.G = Hq / kv->n_kv_heads;
  a.scale_log2 = sm_scale * ev::kLog2e;
  a.tiles_per_split = p.tiles_per_split;
  a.n_splits = p.n_splits;
  a.out = out;
  a.lse = lse;
  a.dev_status = dev_status;
  if (need) {
    size_t rows = (size_t)p.n_splits * B * T * Hq;
    a.part_o = (float *)ws;
    a.part_lse = (float *)((char *)ws + ev::align_up(rows * kv->head_dim * sizeof(float), 256));
  }
  if (kv->dtype == EV_F32) {
    dim3 grid(T, Hq, B);
    if (kv->head_dim == 64)
      hipLaunchKernelGGL(ev::tree_attn_f32_kernel<64>, grid, dim3(64), 0, stream, a);
    else
      hipLaunchKernelGGL(ev::tree_attn_f32_kernel<128>, grid, dim3(64), 0, stream, a);
  } else {
    if (kv->head_dim == 64)
      ev::launch_bf16<64>(p, a, stream);
    else
      ev::launch_bf16<128>(p, a, stream);
  }
  return ev::launch_status();
}
