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
//     grouped-query layer reuses each K/V byte G*T times inside one workgroup.
//   * bf16 with d = 128 (tree_attn_dma_kernel): workgroups of 2, 4 or 8 wavefronts of 32
//     query rows; 64-key K and V tiles go global -> LDS by direct-to-LDS loads through a
//     4-stage ring (three tiles in flight), XOR-swizzled so the fragment reads are
//     bank-conflict-free; V fragments come from the LDS transpose read.  The query rows
//     and ancestor masks also arrive by DMA, and the output rows leave through LDS as whole
//     rows, so the kernel issues no ordinary global loads.
//   * d = 64 and the INT4 cache (tree_attn_bf16_kernel): the same products with tiles
//     staged through registers (the INT4 tile dequantised on its way to LDS), double
//     buffered, the next tile's loads in flight while the current one is computed.
//   * Scores are computed transposed, S^T = K Q^T, with v_mfma_f32_32x32x16_bf16: the
//     accumulator column is the query, so each lane holds 16 keys of ONE query and the
//     softmax statistics, the output rescale and the final normalisation are lane-local
//     (only the tile max crosses the two wave halves).
//   * K rows enter the matrix core with bits 2 and 3 of the row index swapped, so that the
//     score accumulator, converted to bf16, is directly the B operand of O^T += V^T P^T
//     for 16 consecutive keys — no data movement for P.
//   * Online softmax in float32, base 2, scale folded into one FMA before v_exp_f32.  The
//     reference max is only raised when a tile's max exceeds it by more than 8 (a factor
//     256 in probability), so the O rescale runs on a handful of tiles, not on every one.
//   * Only tiles reaching past the prefix apply the ancestor bitmask.
//   * 1-D grid with an XCD-aware order: the row blocks of one (sequence, head, split) are
//     dispatched to the same XCD and so share its L2 for the K/V tiles.
//   * Long prefixes are split across workgroups (sized for one workgroup per CU in the DMA
//     kernel); each split writes its normalised partial O in fp16 (pre-divided by
//     max(1, |O|max) of the row, the divisor kept in float32) and its LSE, adjacent to the
//     other splits of the same row; a merge kernel combines them.
// float32 path: a VALU kernel, one workgroup per (sequence, KV head, block of query rows),
// K and V tiles staged in LDS.
#include "ev_internal.h"
#include "rowstream.h"

#include <algorithm>
#include <math.h>
#include <mutex>
#include <type_traits>

namespace ev {

constexpr int kKT = 64;                 // keys per tile
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kRescaleSlack = 8.0f;   // log2 headroom before the reference max is raised
constexpr int kXcds = 8;
constexpr int kMaxSplits = 32;          // split-L partials per output row, at most

struct AttnArgs {
  const void *q;
  const void *k;
  const void *v;
  KvAddr kv;
  const int32_t *prefix_len;
  const uint64_t *anc;
  int B, T, Hq, G;
  int max_prefix;          // host bound of every prefix_len[b]; splits cover its key range
  int max_tiles;           // 64-key tiles of that range (the plan's)
  float scale_log2;        // sm_scale * log2(e)
  int row_blocks;
  int tiles_per_split;
  int n_splits;
  int n_work;              // B * Hkv * row_blocks * n_splits
  void *out;               // final O (n_splits == 1)
  float *lse;              // final LSE (n_splits == 1)
  _Float16 *part_o;        // [B][T][Hq][n_splits][D], scaled by 1 / its scale
  uint64_t *part_ls;       // [B][T][Hq][n_splits]: partial LSE bits | scale bits << 32
  int32_t *dev_status;
  const float *k_scale;    // INT4 caches: one scale per (slot, KV head) row
  const float *v_scale;
  const int32_t *parent;   // set: the DMA kernel builds the masks itself from the parents
  uint64_t *anc_out;       //   and writes them (and depth_out, if set) once per sequence
  int32_t *depth_out;
};

// Row of split `split`'s partial for output row `orow` ((sequence, node, head) order): the
// partials of one output row are adjacent, so the merge reads one contiguous block.
__device__ inline int64_t part_row(const AttnArgs &a, int64_t orow, int split) {
  return orow * a.n_splits + split;
}

// A split's partial LSE and the divisor its fp16 row was stored with, as one 64-bit word.
__device__ inline uint64_t pack_ls(float lse, float scale) {
  return (uint64_t)__float_as_uint(lse) | ((uint64_t)__float_as_uint(scale) << 32);
}
__device__ inline float ls_lse(uint64_t w) { return __uint_as_float((uint32_t)w); }
__device__ inline float ls_scale(uint64_t w) { return __uint_as_float((uint32_t)(w >> 32)); }

// Is logical slot `slot` visible to a query whose ancestor row is `anc` (prefix length L)?
__device__ inline bool visible(int slot, int L, uint64_t anc) {
  int j = slot - L;
  return j < 0 || (j < 64 && ((anc >> j) & 1ull));
}

// MFMA row index -> key within a 32-key subtile: swap bits 2 and 3.
__device__ inline int swap23(int r) { return (r & ~12) | ((r & 4) << 1) | ((r & 8) >> 1); }

// S^T = K Q^T of NST 32-key subtiles of a 64-key tile (both, or the one a wavefront of a
// key-split workgroup owns); kfrag(st, ks) returns the K fragment (A operand) of local
// subtile st, head-dim step ks for this lane.
template <int QT, int KS, int NST, typename KFrag>
__device__ __forceinline__ void tile_scores(f32x16 (&s)[QT][NST], const bf16x8 (&qf)[QT][KS],
                                            KFrag kfrag) {
#pragma unroll
  for (int st = 0; st < NST; ++st)
#pragma unroll
    for (int t = 0; t < QT; ++t) s[t][st] = f32x16{};
  // With two subtiles they alternate, so consecutive products accumulate into different
  // registers and do not wait on each other.  Each K fragment is read four products ahead:
  // the scheduling groups below keep that order (left to itself the scheduler put each
  // read one product ahead and waited for it).
  constexpr int AHEAD = 4;
  bf16x8 kf[AHEAD];
#pragma unroll
  for (int i = 0; i < AHEAD; ++i) kf[i] = kfrag(i % NST, i / NST);
#pragma unroll
  for (int i = 0; i < NST * KS; ++i) {
    const int st = i % NST, ks = i / NST;
    const bf16x8 cur = kf[i % AHEAD];
    if (i + AHEAD < NST * KS) kf[i % AHEAD] = kfrag((i + AHEAD) % NST, (i + AHEAD) / NST);
#pragma unroll
    for (int t = 0; t < QT; ++t)
      s[t][st] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(cur, qf[t][ks], s[t][st], 0, 0, 0);
  }
  __builtin_amdgcn_sched_group_barrier(0x100, AHEAD, 0);     // LDS reads
#pragma unroll
  for (int i = 0; i < NST * KS; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, QT, 0);      // matrix products
    if (i + AHEAD < NST * KS) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
  }
}

// Ancestor mask of a tile reaching past the prefix, applied in place to the scores: a key
// that is neither a prefix slot nor an ancestor-or-self tree slot of the lane's query gets
// -inf.  Register r of local subtile st holds key key0 + st*32 + 16*(r>>3) + 8*hh +
// 4*((r>>2)&1) + (r&3) (the K rows were fed with bits 2 and 3 of the row index swapped).
template <int QT, int NST>
__device__ __forceinline__ void tile_mask(f32x16 (&s)[QT][NST], const uint64_t (&anc_q)[QT],
                                          int key0, int L, int hh) {
#pragma unroll
  for (int t = 0; t < QT; ++t)
#pragma unroll
    for (int st = 0; st < NST; ++st)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = st * 32 + (r >> 3) * 16 + hh * 8 + ((r >> 2) & 1) * 4 + (r & 3);
        if (!visible(key0 + key, L, anc_q[t])) s[t][st][r] = -INFINITY;
      }
}

// Online softmax (base 2, float32) of one tile's (masked) scores, lane-local per query,
// in two parts so that independent matrix-core work can be scheduled between them:
// tile_rescale takes the tile max and raises the reference max (rescaling O and the sum)
// only when the tile could overflow 2^8 of headroom; tile_exp forms the probabilities,
// their sum and the bf16 P fragments.  Each 8-register group of a subtile is 8 consecutive
// keys, so the fragments are directly the B operand of O^T += V^T P^T.
template <int QT, int DT, int NST>
__device__ __forceinline__ void tile_rescale(const f32x16 (&s)[QT][NST], f32x16 (&o)[QT][DT],
                                             float (&mref)[QT], float (&l)[QT], float scale_log2) {
#pragma unroll
  for (int t = 0; t < QT; ++t) {
    float mx = -INFINITY;
#pragma unroll
    for (int st = 0; st < NST; ++st)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[t][st][r]);
    mx = halves_max(mx) * scale_log2;
    if (__any(mx > mref[t] + kRescaleSlack)) {
      const float mnew = fmaxf(mref[t], mx);
      const float alpha = mnew == -INFINITY ? 1.f : __builtin_amdgcn_exp2f(mref[t] - mnew);
      l[t] *= alpha;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) o[t][dt] *= alpha;
      mref[t] = mnew;
    }
  }
}

template <int QT, int NST>
__device__ __forceinline__ void tile_exp(const f32x16 (&s)[QT][NST], bf16x8 (&pf)[QT][NST][2],
                                         const float (&mref)[QT], float (&l)[QT], float scale_log2) {
#pragma unroll
  for (int t = 0; t < QT; ++t) {
    const float nb = mref[t] == -INFINITY ? 0.f : -mref[t];
    float sum = -0.f;                            // the additive identity: no leading add
#pragma unroll
    for (int st = 0; st < NST; ++st) {
      f32x16 p;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        p[r] = __builtin_amdgcn_exp2f(fmaf(s[t][st][r], scale_log2, nb));
        sum += p[r];
      }
#pragma unroll
      for (int kk = 0; kk < 2; ++kk)
        pf[t][st][kk] = bf16x8{(__bf16)p[8 * kk + 0], (__bf16)p[8 * kk + 1], (__bf16)p[8 * kk + 2],
                               (__bf16)p[8 * kk + 3], (__bf16)p[8 * kk + 4], (__bf16)p[8 * kk + 5],
                               (__bf16)p[8 * kk + 6], (__bf16)p[8 * kk + 7]};
    }
    l[t] += sum;
  }
}

// O^T += V^T P^T over NST subtiles; vfrag(st, kk, dt) returns the V^T fragment (A operand)
// of local subtile st: head dims dt*32 + qn, keys st*32 + kk*16 + 8*hh + 0..7.
template <int QT, int DT, int NST, typename VFrag>
__device__ __forceinline__ void tile_pv(f32x16 (&o)[QT][DT], const bf16x8 (&pf)[QT][NST][2],
                                        VFrag vfrag) {
#pragma unroll
  for (int st = 0; st < NST; ++st)
#pragma unroll
    for (int kk = 0; kk < 2; ++kk)
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        const bf16x8 vf = vfrag(st, kk, dt);
#pragma unroll
        for (int t = 0; t < QT; ++t)
          o[t][dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pf[t][st][kk], o[t][dt], 0, 0, 0);
      }
}

// Normalise this lane's query rows and write them: the final O (bf16) and LSE when the
// sequence is not split, else an fp16 partial O pre-divided by max(1, |O|max of the row)
// (the divisor kept in float32 so the partial cannot overflow) plus the partial LSE.
template <int D, int QT>
__device__ __forceinline__ void write_rows(const AttnArgs &a, const f32x16 (&o)[QT][D / 32],
                                           const float (&mref)[QT], const float (&l)[QT],
                                           int row0, int b, int g, int split, int qn, int hh) {
  constexpr int DT = D / 32;
  const int rows = a.T * a.G;
#pragma unroll
  for (int t = 0; t < QT; ++t) {
    const int r = row0 + t * 32 + qn;
    const float ltot = halves_sum(l[t]);
    const float inv = ltot > 0.f ? 1.f / ltot : 0.f;
    const float lse = ltot > 0.f ? (mref[t] + __log2f(ltot)) * kLn2 : -INFINITY;
    const bool ok = r < rows;
    const int node = ok ? r / a.G : 0;
    const int head = g * a.G + (ok ? r % a.G : 0);
    const int64_t orow = ((int64_t)b * a.T + node) * a.Hq + head;
    if (a.n_splits == 1) {
      if (!ok) continue;
      __bf16 *dst = (__bf16 *)a.out + orow * D;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const f32x16 &ov = o[t][dt];
          *(bf16x4 *)(dst + dt * 32 + 8 * j + 4 * hh) =
              bf16x4{(__bf16)(ov[4 * j] * inv), (__bf16)(ov[4 * j + 1] * inv),
                     (__bf16)(ov[4 * j + 2] * inv), (__bf16)(ov[4 * j + 3] * inv)};
        }
      if (hh == 0) a.lse[orow] = lse;
    } else {
      float amax = 0.f;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int i = 0; i < 16; ++i) amax = fmaxf(amax, fabsf(o[t][dt][i]));
      amax = halves_max(amax) * inv;
      const float scale = fmaxf(1.f, amax);
      const float k = inv / scale;
      if (!ok) continue;
      const int64_t prow = part_row(a, orow, split);
      _Float16 *dst = a.part_o + prow * D;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const f32x16 &ov = o[t][dt];
          *(f16x4 *)(dst + dt * 32 + 8 * j + 4 * hh) =
              f16x4{(_Float16)(ov[4 * j] * k), (_Float16)(ov[4 * j + 1] * k),
                    (_Float16)(ov[4 * j + 2] * k), (_Float16)(ov[4 * j + 3] * k)};
        }
      if (hh == 0) a.part_ls[prow] = pack_ls(lse, scale);
    }
  }
}

// Block ids of one split's paged tiles, cached in LDS by the workgroup.
constexpr int kTableCache = 1024;

// Global -> register staging of one 64-key tile; registers -> LDS after the compute.
// Thread `tid` always owns the same (key, 8-dim chunk) positions of a tile, so a full
// contiguous tile is one uniform base pointer plus fixed per-thread offsets; a paged tile
// reads its block ids from the LDS cache.  Only the last tile of a sequence is partial.
// V is transposed on its way to LDS in items of KPI keys x 8 dims (one item per thread
// for 256- and 512-thread workgroups).
// Eight values of an INT4 row chunk (4 bytes, element 2j in the low nibble of byte j)
// times the row's scale, each float32 product rounded to bfloat16, packed in pairs.
__device__ inline u32x4 dequant8(uint32_t w, float s) {
  u32x4 out;
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const int lo = ((int)(w << (28 - 8 * p))) >> 28;
    const int hi = ((int)(w << (24 - 8 * p))) >> 28;
    const __bf16 a = (__bf16)(s * (float)lo), b = (__bf16)(s * (float)hi);
    out[p] = (uint32_t)__builtin_bit_cast(uint16_t, a) | ((uint32_t)__builtin_bit_cast(uint16_t, b) << 16);
  }
  return out;
}

template <int D, int NT, bool PAGED, bool Q4 = false>
struct TileStage {
  static constexpr int DC = D / 8;                     // 8-value chunks per key row
  static constexpr int KCHUNKS = kKT * DC;             // K chunks per tile
  static constexpr int KPI = NT >= 512 ? 2 : 4;        // keys per V item
  static constexpr int VITEMS = (kKT / KPI) * DC;      // V items per tile
  static constexpr int KPT = (KCHUNKS + NT - 1) / NT;
  static constexpr int VPT = (VITEMS + NT - 1) / NT;
  static constexpr int KSTEP = NT / DC;                // key stride between a thread's K chunks
  static constexpr int KP = D + 8;                     // LDS pitch of the K tile (elements)
  static constexpr int VP = kKT + 8;                   // LDS pitch of the V^T tile (elements)
  static_assert(NT % DC == 0 && NT % (kKT / KPI) == 0, "thread count must tile the stage");
  // Staged tile: bf16 chunks, or for Q4 the packed words and their rows' scales
  // (dequantised when stored, so a prefetch holds only the raw bytes).
  u32x4 kr[Q4 ? 1 : KPT];
  u32x4 vr[Q4 ? 1 : VPT][KPI];
  uint32_t kw[Q4 ? KPT : 1];
  float ks[Q4 ? KPT : 1];
  uint32_t vw[Q4 ? VPT : 1][KPI];
  float vs[Q4 ? VPT : 1][KPI];

  // Row index (slot row of KV head g) of logical slot `slot` (PAGED: -1 for a bad block).
  __device__ static inline int64_t slot_row(const KvAddr &kv, int64_t seq_row, const int *stbl,
                                            int blk0, int g, int slot) {
    if (!PAGED) return seq_row + slot;
    const int blk = stbl[(slot >> kv.block_shift) - blk0];
    if (blk < 0) return -1;
    return (((int64_t)blk * kv.hkv + g) << kv.block_shift) | (slot & ((1 << kv.block_shift) - 1));
  }

  __device__ inline void load(const AttnArgs &a, const void *K, const void *V, int64_t seq_row,
                              const int *stbl, int blk0, int g, int key0, int nkeys) {
    const int tid = threadIdx.x;
    const bool full = key0 + kKT <= nkeys;
    const int dc = tid % DC;
    if constexpr (Q4) {
#pragma unroll
      for (int i = 0; i < KPT; ++i) {
        const int key = tid / DC + i * KSTEP;
        const bool live = key < kKT && (full || key0 + key < nkeys);
        const int64_t row = live ? slot_row(a.kv, seq_row, stbl, blk0, g, key0 + key) : -1;
        kw[i] = row >= 0 ? *(const uint32_t *)((const uint8_t *)K + row * (D / 2) + dc * 4) : 0u;
        ks[i] = row >= 0 ? a.k_scale[row] : 0.f;
      }
#pragma unroll
      for (int i = 0; i < VPT; ++i) {
        const int c = tid + i * NT;
        const int kq = c % (kKT / KPI), vdc = c / (kKT / KPI);
#pragma unroll
        for (int r = 0; r < KPI; ++r) {
          const int key = KPI * kq + r;
          const bool live = c < VITEMS && (full || key0 + key < nkeys);
          const int64_t row = live ? slot_row(a.kv, seq_row, stbl, blk0, g, key0 + key) : -1;
          vw[i][r] = row >= 0 ? *(const uint32_t *)((const uint8_t *)V + row * (D / 2) + vdc * 4) : 0u;
          vs[i][r] = row >= 0 ? a.v_scale[row] : 0.f;
        }
      }
    } else {
#pragma unroll
      for (int i = 0; i < KPT; ++i) {
        const int key = tid / DC + i * KSTEP;
        u32x4 val = {};
        if (key < kKT && (full || key0 + key < nkeys)) {
          const int64_t row = slot_row(a.kv, seq_row, stbl, blk0, g, key0 + key);
          if (row >= 0) val = *(const u32x4 *)((const __bf16 *)K + row * D + dc * 8);
        }
        kr[i] = val;
      }
#pragma unroll
      for (int i = 0; i < VPT; ++i) {
        const int c = tid + i * NT;
        const int kq = c % (kKT / KPI), vdc = c / (kKT / KPI);
#pragma unroll
        for (int r = 0; r < KPI; ++r) {
          u32x4 val = {};
          const int key = KPI * kq + r;
          if (c < VITEMS && (full || key0 + key < nkeys)) {
            const int64_t row = slot_row(a.kv, seq_row, stbl, blk0, g, key0 + key);
            if (row >= 0) val = *(const u32x4 *)((const __bf16 *)V + row * D + vdc * 8);
          }
          vr[i][r] = val;
        }
      }
    }
  }

  __device__ inline u32x4 kchunk(int i) const { return Q4 ? dequant8(kw[i], ks[i]) : kr[i]; }
  __device__ inline u32x4 vchunk(int i, int r) const {
    return Q4 ? dequant8(vw[i][r], vs[i][r]) : vr[i][r];
  }

  __device__ inline void store(__bf16 *sK, __bf16 *sV) const {
    const int tid = threadIdx.x;
#pragma unroll
    for (int i = 0; i < KPT; ++i) {
      const int key = tid / DC + i * KSTEP;
      if (key < kKT) *(u32x4 *)(sK + key * KP + (tid % DC) * 8) = kchunk(i);
    }
#pragma unroll
    for (int i = 0; i < VPT; ++i) {
      const int c = tid + i * NT;
      if (c >= VITEMS) continue;
      const int kq = c % (kKT / KPI), vdc = c / (kKT / KPI);
      // dim e of the item's keys: the low (even e) or high (odd e) half of word e / 2
#pragma unroll
      for (int wd = 0; wd < 4; ++wd) {
        if (KPI == 4) {
          const u32x4 r0 = vchunk(i, 0), r1 = vchunk(i, 1), r2 = vchunk(i, KPI - 2),
                      r3 = vchunk(i, KPI - 1);
          u32x2 lo = {__builtin_amdgcn_perm(r1[wd], r0[wd], 0x05040100u),
                      __builtin_amdgcn_perm(r3[wd], r2[wd], 0x05040100u)};
          u32x2 hi = {__builtin_amdgcn_perm(r1[wd], r0[wd], 0x07060302u),
                      __builtin_amdgcn_perm(r3[wd], r2[wd], 0x07060302u)};
          *(u32x2 *)(sV + (vdc * 8 + 2 * wd) * VP + KPI * kq) = lo;
          *(u32x2 *)(sV + (vdc * 8 + 2 * wd + 1) * VP + KPI * kq) = hi;
        } else {
          const u32x4 r0 = vchunk(i, 0), r1 = vchunk(i, 1);
          *(uint32_t *)(sV + (vdc * 8 + 2 * wd) * VP + KPI * kq) =
              __builtin_amdgcn_perm(r1[wd], r0[wd], 0x05040100u);
          *(uint32_t *)(sV + (vdc * 8 + 2 * wd + 1) * VP + KPI * kq) =
              __builtin_amdgcn_perm(r1[wd], r0[wd], 0x07060302u);
        }
      }
    }
  }
};

template <int D, int QT, int NW, bool PAGED, bool Q4 = false>
__global__ __launch_bounds__(NW * 64) void tree_attn_bf16_kernel(AttnArgs a) {
  constexpr int NT = NW * 64;
  using Stage = TileStage<D, NT, PAGED, Q4>;
  constexpr int KS = D / 16;            // k-steps of the score product
  constexpr int DT = D / 32;            // 32-row tiles of O^T
  constexpr int KP = Stage::KP;
  constexpr int VP = Stage::VP;
  constexpr int KBUF = kKT * KP;        // elements per K buffer
  constexpr int VBUF = D * VP;          // elements per V^T buffer
  __shared__ __attribute__((aligned(16))) __bf16 sK[KBUF];
  __shared__ __attribute__((aligned(16))) __bf16 sV[VBUF];
  __shared__ int stbl[PAGED ? kTableCache : 1];

  // XCD-aware work order: consecutive work items (the row blocks of one split) land on the
  // same XCD, whose L2 then serves their shared K/V tiles.
  const int per_xcd = gridDim.x / kXcds;
  const int w = (blockIdx.x % kXcds) * per_xcd + blockIdx.x / kXcds;
  if (w >= a.n_work) return;
  const int rb = w % a.row_blocks;
  const int split = (w / a.row_blocks) % a.n_splits;
  const int bg = w / (a.row_blocks * a.n_splits);
  const int b = bg / a.kv.hkv;
  const int g = bg % a.kv.hkv;

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int qn = lane & 31;             // query column of this lane
  const int hh = lane >> 5;             // wave half

  const int L = a.prefix_len[b];
  const int nkeys = L + a.T;
  if (L < 0 || L > a.max_prefix || !a.kv.fits(nkeys)) {
    if (threadIdx.x == 0) report(a.dev_status, EV_DERR_BOUNDS);
    return;
  }
  const int ntiles = (nkeys + kKT - 1) / kKT;
  const int t_begin = split * a.tiles_per_split;
  const int t_end = min(t_begin + a.tiles_per_split, ntiles);
  const int rows = a.T * a.G;
  const int row0 = (rb * NW + wave) * QT * 32;
  if (t_begin >= t_end) {               // this split lies beyond the sequence: no weight
    if (a.n_splits > 1 && hh == 0) {
#pragma unroll
      for (int t = 0; t < QT; ++t) {
        const int r = row0 + t * 32 + qn;
        if (r >= rows) continue;
        const int64_t orow = ((int64_t)b * a.T + r / a.G) * a.Hq + g * a.G + r % a.G;
        a.part_ls[part_row(a, orow, split)] = pack_ls(-INFINITY, 1.f);
      }
    }
    return;
  }
  const __bf16 *Q = (const __bf16 *)a.q;
  const void *K = a.k;
  const void *V = a.v;
  const int64_t seq_row = PAGED ? 0 : (int64_t)(b * a.kv.hkv + g) * a.kv.cap;

  int blk0 = 0;
  if (PAGED) {
    blk0 = (t_begin * kKT) >> a.kv.block_shift;
    const int nblk = ((min(t_end * kKT, nkeys) - 1) >> a.kv.block_shift) - blk0 + 1;
    bool bad = false;
    for (int i = threadIdx.x; i < nblk; i += NT) {
      const int blk = a.kv.table[(int64_t)b * a.kv.max_blocks + blk0 + i];
      const bool ok = blk >= 0 && blk < a.kv.n_blocks;
      bad |= !ok;
      stbl[i] = ok ? blk : -1;
    }
    if (__any(bad) && lane == 0) report(a.dev_status, EV_DERR_BOUNDS);
    __syncthreads();
  }

  Stage s0;
  s0.load(a, K, V, seq_row, stbl, blk0, g, t_begin * kKT, nkeys);

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
  float mref[QT], l[QT];                // reference max (log2 units) and lane-partial sum
#pragma unroll
  for (int t = 0; t < QT; ++t) {
    mref[t] = -INFINITY;
    l[t] = 0.f;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) o[t][dt] = f32x16{};
  }

  auto kfrag = [&](int st, int ks) {
    return *(const bf16x8 *)(sK + (st * 32 + swap23(qn)) * KP + 8 * hh + 16 * ks);
  };
  auto vfrag = [&](int st, int kk, int dt) {
    return *(const bf16x8 *)(sV + (dt * 32 + qn) * VP + st * 32 + kk * 16 + 8 * hh);
  };
  s0.store(sK, sV);
  __syncthreads();
  for (int tile = t_begin; tile < t_end; ++tile) {
    // INT4: the next tile's raw bytes are requested before this tile is computed (they are
    // small enough to stay in registers meanwhile); bf16 keeps load-after-compute.
    if (Q4 && tile + 1 < t_end) s0.load(a, K, V, seq_row, stbl, blk0, g, (tile + 1) * kKT, nkeys);
    f32x16 sc[QT][2];
    bf16x8 pf[QT][2][2];
    tile_scores<QT, KS, 2>(sc, qf, kfrag);
    if (tile * kKT + kKT > L) tile_mask(sc, anc_q, tile * kKT, L, hh);
    tile_rescale(sc, o, mref, l, a.scale_log2);
    tile_exp(sc, pf, mref, l, a.scale_log2);
    tile_pv(o, pf, vfrag);
    if (tile + 1 < t_end) {
      if (!Q4) s0.load(a, K, V, seq_row, stbl, blk0, g, (tile + 1) * kKT, nkeys);
      __syncthreads();
      s0.store(sK, sV);
      __syncthreads();
    }
  }

  write_rows<D, QT>(a, o, mref, l, row0, b, g, split, qn, hh);
}

// ---------------------------------------------------------------------------------------
// Direct-to-LDS pipeline (head_dim 128, 2-8 wavefronts of 32 query rows).
//
// K and V tiles travel HBM -> LDS with global_load_lds_dwordx4 (no staging registers): lane
// l of a wave-instruction fills LDS chunk base + l, so the LDS layout is chosen on the global
// side.  Both matrices are stored row-major by key with the 16-byte chunks of each row
// XOR-swizzled (K: chunk ^ (key & 15); V: chunk ^ 2*(key & 7)), which makes the K fragment
// reads and the transposing V reads (ds_read_b64_tr_b16: within 16 lanes, lane 4a+c receives
// element c of the 4-element rows addressed by lanes a, a+4, a+8, a+12) bank-conflict-free.
// Four LDS stages hold tiles j (P V), j+1 (Q K^T, overlapping the softmax of j) and j+2, j+3
// (in flight).  Completion is tracked with explicit vmcnt waits, one barrier per tile.
constexpr int kStages = 4;

__device__ __forceinline__ void dma16(const __bf16 *g, __bf16 *l) {
  __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void *)g,
                                   (__attribute__((address_space(3))) void *)l, 16, 0, 0);
}

template <int N>
__device__ __forceinline__ void wait_vm() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

__device__ __forceinline__ void wg_barrier() { asm volatile("s_barrier" ::: "memory"); }

typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;

// Transposing LDS read of a V fragment.  The restrict-qualified pointer gives the read
// alias-scope information; without it the compiler treats the read as possibly aliasing
// every direct-to-LDS load in flight and puts a full vmcnt(0) before it, which would wait
// out the tiles prefetched three steps ahead.  Ordering against the DMA is the kernel's
// own: explicit vmcnt waits plus a barrier before any tile is read.
__device__ __forceinline__ bf16x4 lds_read_tr(lds_bf16x4 *__restrict__ p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4bf16(p);
}

// Output row (sequence, node, head order) of query row r of KV head g.
__device__ inline int64_t out_row(const AttnArgs &a, int b, int g, int r) {
  return ((int64_t)b * a.T + r / a.G) * a.Hq + g * a.G + r % a.G;
}

// write_rows for the DMA kernel (one query tile per wave): the wave's 32 normalised rows
// go through an idle 8 KB of LDS (chunk-swizzled like a K tile) so that the global stores
// are whole rows, 16 bytes per lane and four rows per instruction, instead of 8-byte pieces
// scattered over 32 rows.  A split partial is fp16, pre-divided by max(1, |O|max) of its
// row, with its LSE and divisor as one word; with NT its rows are stored non-temporally (the
// merge reads each once).
template <int D, bool NT>
__device__ __forceinline__ void write_rows_staged(const AttnArgs &a, const f32x16 (&o)[1][D / 32],
                                                  float mref, float l, int row0, int b, int g,
                                                  int split, int qn, int hh, uint16_t *stage) {
  constexpr int DT = D / 32, DCH = D / 8;
  const int lane = threadIdx.x & 63;
  const int rows = a.T * a.G;
  const float ltot = halves_sum(l);
  const float inv = ltot > 0.f ? 1.f / ltot : 0.f;
  const float lse = ltot > 0.f ? (mref + __log2f(ltot)) * kLn2 : -INFINITY;
  const bool part = a.n_splits > 1;
  float k = inv, scale = 1.f;
  if (part) {
    float amax = 0.f;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int i = 0; i < 16; ++i) amax = fmaxf(amax, fabsf(o[0][dt][i]));
    amax = halves_max(amax) * inv;
    scale = fmaxf(1.f, amax);
    k = inv / scale;
  }
  // The partial / final choice is made once, outside the loops, the eight row reads go
  // out before the first store, and the output rows are stepped rather than divided out
  // per row: one wavefront does all of this after the last tile, so its branches, LDS
  // round trips and integer divisions were the call's tail (2.3 -> 1.8 us per wave, 26- and
  // 128-row workgroups; 16.5 -> 15.9 us per call with 32 MHA heads x 26 rows).
  auto store = [&](auto is_part) {
    constexpr bool P = decltype(is_part)::value;
    using H = typename std::conditional<P, f16x4, bf16x4>::type;
    using E = typename std::conditional<P, _Float16, __bf16>::type;
    // this lane's values: row qn, head dims dt*32 + 8j + 4hh + 0..3 = half hh of chunk 4dt + j
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const f32x16 &ov = o[0][dt];
        const H h = H{(E)(ov[4 * j] * k), (E)(ov[4 * j + 1] * k), (E)(ov[4 * j + 2] * k),
                      (E)(ov[4 * j + 3] * k)};
        const int pc = (4 * dt + j) ^ (qn & 15);
        *(u32x2 *)(stage + qn * D + pc * 8 + 4 * hh) = __builtin_bit_cast(u32x2, h);
      }
    // whole rows back out, all read before the first store: lane takes row 4i + lane/16,
    // chunk lane%16
    constexpr int NI = 32 * DCH / 64;
    const int cc = lane & 15;
    u32x4 v[NI];
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int rr = 4 * i + (lane >> 4);
      v[i] = *(const u32x4 *)(stage + rr * D + ((cc ^ (rr & 15)) << 3));
    }
    // output row of query row r = node * G + m, stepped four rows at a time
    int r = row0 + (lane >> 4);
    int node = r / a.G, m = r % a.G;
    const int dnode = 4 / a.G, dm = 4 % a.G;
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      if (r < rows) {
        const int64_t orow = ((int64_t)b * a.T + node) * a.Hq + g * a.G + m;
        if constexpr (P) {
          u32x4 *dst = (u32x4 *)(a.part_o + part_row(a, orow, split) * D + cc * 8);
          if constexpr (NT)
            __builtin_nontemporal_store(v[i], dst);
          else
            *dst = v[i];
        } else {
          *(u32x4 *)((__bf16 *)a.out + orow * D + cc * 8) = v[i];
        }
      }
      r += 4;
      node += dnode;
      m += dm;
      if (m >= a.G) {
        m -= a.G;
        ++node;
      }
    }
  };
  if (part)
    store(std::true_type{});
  else
    store(std::false_type{});
  const int r = row0 + qn;
  if (hh == 0 && r < rows) {
    const int64_t orow = out_row(a, b, g, r);
    if (part)
      a.part_ls[part_row(a, orow, split)] = pack_ls(lse, scale);
    else
      a.lse[orow] = lse;
  }
}

// The end of a key-split group: wavefront kh holds the online-softmax state (reference
// max m, partial sums l, accumulators o) of its half of every tile's keys, for all 32 rows
// and all head dimensions.  Each finishes half of the head dimensions (dt = 2kh, 2kh + 1):
// it hands the other half, with m, l and its max |o|, to its partner through `xch`, takes
// the partner's values for its own dimensions, and writes the combined, normalised values
// into the group's 32 staging rows (`stage`, chunk-swizzled like a K tile); after a
// barrier each stores 16 of the 32 rows whole.  Both compute the row scalars in the same
// order, so they agree bit for bit.  A split partial's divisor is max(1, bound) with the
// bound a0 max|o_0| + a1 max|o_1| over the row sum, which is at least the row's max |O|,
// so the fp16 row cannot overflow.  Every wavefront of the workgroup calls this (it holds
// two barriers).  KH is a template argument so that the accumulators are only ever indexed
// by constants (a run-time index put them in scratch memory).
template <int D, bool NT, int KH>
__device__ __forceinline__ void finish_pair(const AttnArgs &a, const f32x16 (&o)[1][D / 32],
                                            float m, float l, int row0, int b, int g,
                                            int split, int qn, int hh, float *xch,
                                            uint16_t *stage) {
  constexpr int kh = KH;
  constexpr int DT = D / 32, DH = DT / 2, DCH = D / 8;
  constexpr int XF = 3 + DH * 16;                // floats one wavefront hands over per lane
  const int lane = threadIdx.x & 63;
  const int rows = a.T * a.G;
  const bool part = a.n_splits > 1;
  float am = 0.f;
  if (part) {
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int i = 0; i < 16; ++i) am = fmaxf(am, fabsf(o[0][dt][i]));
    am = halves_max(am);
  }
  float *mine = xch + kh * XF * 64;
  const float *theirs = xch + (1 - kh) * XF * 64;
  mine[lane] = m;
  mine[64 + lane] = l;
  mine[128 + lane] = am;
#pragma unroll
  for (int h = 0; h < DH; ++h)
#pragma unroll
    for (int i = 0; i < 16; ++i) mine[(3 + h * 16 + i) * 64 + lane] = o[0][(1 - kh) * DH + h][i];
  __syncthreads();
  const float m2 = theirs[lane], l2 = theirs[64 + lane], am2 = theirs[128 + lane];
  const float m0 = kh == 0 ? m : m2, m1 = kh == 0 ? m2 : m;
  const float l0 = kh == 0 ? l : l2, l1 = kh == 0 ? l2 : l;
  const float am0 = kh == 0 ? am : am2, am1 = kh == 0 ? am2 : am;
  const float mnew = fmaxf(m0, m1);
  const float a0 = m0 == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m0 - mnew);
  const float a1 = m1 == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m1 - mnew);
  const float ltot = halves_sum(l0 * a0 + l1 * a1);
  const float inv = ltot > 0.f ? 1.f / ltot : 0.f;
  const float lse = ltot > 0.f ? (mnew + __log2f(ltot)) * kLn2 : -INFINITY;
  float k = inv, scale = 1.f;
  if (part) {
    scale = fmaxf(1.f, (a0 * am0 + a1 * am1) * inv);
    k = inv / scale;
  }
  const float km = k * (kh == 0 ? a0 : a1), kt = k * (kh == 0 ? a1 : a0);
  auto store = [&](auto is_part) {
    constexpr bool P = decltype(is_part)::value;
    using H = typename std::conditional<P, f16x4, bf16x4>::type;
    using E = typename std::conditional<P, _Float16, __bf16>::type;
    // this lane's values: row qn, head dims dt*32 + 8j + 4hh + 0..3 = half hh of chunk 4dt + j
#pragma unroll
    for (int h = 0; h < DH; ++h)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int dt = kh * DH + h;
        const f32x16 &ov = o[0][dt];
        float v[4];
#pragma unroll
        for (int e = 0; e < 4; ++e)
          v[e] = fmaf(ov[4 * j + e], km, theirs[(3 + h * 16 + 4 * j + e) * 64 + lane] * kt);
        const H hv = H{(E)v[0], (E)v[1], (E)v[2], (E)v[3]};
        const int pc = (4 * dt + j) ^ (qn & 15);
        *(u32x2 *)(stage + qn * D + pc * 8 + 4 * hh) = __builtin_bit_cast(u32x2, hv);
      }
    __syncthreads();                             // both halves of every row staged
    // rows 16kh .. 16kh + 15 back out whole: lane takes row 16kh + 4i + lane/16, chunk lane%16
    constexpr int NI = 32 * DCH / 64 / 2;
    const int cc = lane & 15;
    u32x4 w[NI];
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int rr = 16 * kh + 4 * i + (lane >> 4);
      w[i] = *(const u32x4 *)(stage + rr * D + ((cc ^ (rr & 15)) << 3));
    }
    int r = row0 + 16 * kh + (lane >> 4);
    int node = r / a.G, mm = r % a.G;
    const int dnode = 4 / a.G, dm = 4 % a.G;
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      if (r < rows) {
        const int64_t orow = ((int64_t)b * a.T + node) * a.Hq + g * a.G + mm;
        if constexpr (P) {
          u32x4 *dst = (u32x4 *)(a.part_o + part_row(a, orow, split) * D + cc * 8);
          if constexpr (NT)
            __builtin_nontemporal_store(w[i], dst);
          else
            *dst = w[i];
        } else {
          *(u32x4 *)((__bf16 *)a.out + orow * D + cc * 8) = w[i];
        }
      }
      r += 4;
      node += dnode;
      mm += dm;
      if (mm >= a.G) {
        mm -= a.G;
        ++node;
      }
    }
  };
  if (part)
    store(std::true_type{});
  else
    store(std::false_type{});
  const int r = row0 + qn;
  if (kh == 0 && hh == 0 && r < rows) {
    const int64_t orow = out_row(a, b, g, r);
    if (part)
      a.part_ls[part_row(a, orow, split)] = pack_ls(lse, scale);
    else
      a.lse[orow] = lse;
  }
}

// Direct-to-LDS tree attention kernel, head_dim 128.  Without KSPLIT: NW wavefronts of 32
// query rows each.  KSPLIT: NW / 2 groups of 32 rows, two wavefronts per group (one per
// 32-key half of every tile, so each scores and accumulates half the keys), the halves
// combined through LDS at the end; with NW = 2 it serves heads of at most 32 rows, with
// NW = 8 it halves the rows per workgroup of short split plans (more row blocks, fewer
// splits, fewer partial rows).
// Ancestor masks of sequence b from its parents in LDS (one wavefront, lane i = node i),
// by pointer doubling over the parent links as ev_tree_mask_build does ([TR] sec. 2, mask
// equation M): after round r a lane holds its ancestors within distance 2^r, so six rounds
// cover 64 nodes.  The masks go to LDS; `writer` also stores them (and the depths) to
// anc_out / depth_out, or reports a parent array that is not a tree (whose outputs are
// then unspecified, like every output of a sequence with a device error).
__device__ void build_masks(const AttnArgs &a, int b, const int32_t *s_par, uint64_t *s_anc,
                            bool writer) {
  const int i = threadIdx.x & 63;
  const bool live = i < a.T;
  int p = live ? s_par[i] : -1;
  const bool ok = !live || (i == 0 ? p == -1 : (p >= 0 && p < i));
  const bool tree_ok = !__any(!ok);
  if (!ok) p = -1;
  uint64_t set = live ? (1ull << i) : 0ull;
  int up = p;
  for (int r = 0; r < 6; ++r) {
    const int src = up < 0 ? i : up;
    const uint64_t s_up = __shfl(set, src);
    const int up_up = __shfl(up, src);
    if (up >= 0) {
      set |= s_up;
      up = up_up;
    }
  }
  if (live) s_anc[i] = set;
  if (writer) {
    if (!tree_ok) {
      if (i == 0) report(a.dev_status, EV_DERR_PARENT);
    } else if (live) {
      a.anc_out[(int64_t)b * a.T + i] = set;
      if (a.depth_out) a.depth_out[(int64_t)b * a.T + i] = __popcll(set) - 1;
    }
  }
}

// MASKS: the masks are built from a.parent (ev_tree_mask_attention) instead of read from
// a.anc; a separate instantiation, so that ev_tree_attention's kernels are unchanged.
template <int NW, bool PAGED, bool KSPLIT, bool MASKS>
__global__ __launch_bounds__(NW * 64) void tree_attn_dma_kernel(AttnArgs a) {
  constexpr int D = 128;
  constexpr int QT = 1;
  constexpr int NST = KSPLIT ? 1 : 2;            // 32-key subtiles this wave computes
  constexpr int KS = D / 16, DT = D / 32, DCH = D / 8;
  constexpr int MAT = kKT * D;                   // bf16 elements of one K or V tile
  constexpr int IPW = kKT * DCH / 64 / NW;       // DMA instructions per wave per matrix
  constexpr int PER = 2 * IPW;                   // per wave per tile
  static_assert(IPW >= 1 && 2 * PER <= 63, "vmcnt range");
  static_assert(!KSPLIT || NW == 2 || NW == 8, "key-split workgroups have two or eight wavefronts");
  constexpr int RG = KSPLIT ? NW / 2 : NW;       // groups of 32 query rows per workgroup
  constexpr int NT = NW * 64;
  // kStages K|V tile pairs, then the sequence's ancestor masks (64 x 8 bytes)
  // (then the parents, when the kernel builds the masks: 64 x 4 bytes)
  __shared__ __attribute__((aligned(1024))) __bf16 lds[kStages * 2 * MAT + kMaxNodes * (MASKS ? 6 : 4)];
  __shared__ int stbl[PAGED ? kTableCache : 1];

  args_in_sgprs(gridDim.x, a.n_work, a.row_blocks, a.n_splits, a.kv.hkv, a.kv.cap, a.T, a.G, a.Hq,
                a.q, a.k, a.v, a.anc, a.prefix_len, a.tiles_per_split, a.max_tiles, a.max_prefix);
  const int per_xcd = gridDim.x / kXcds;
  const int w = (blockIdx.x % kXcds) * per_xcd + blockIdx.x / kXcds;
  if (w >= a.n_work) return;
  const int rb = w % a.row_blocks;
  const int split = (w / a.row_blocks) % a.n_splits;
  const int bg = w / (a.row_blocks * a.n_splits);
  const int b = bg / a.kv.hkv;
  const int g = bg % a.kv.hkv;
  // The prefix length, as a scalar load ahead of every DMA: read after them it became a
  // vector load that could only be waited for together with all of them.
  const int L = scalar_load(a.prefix_len, b);
  const int lane = threadIdx.x & 63;
  // (uniform; said so for eight-wavefront workgroups, whose tile DMA addresses are scalar)
  const int wave = NW == 8 ? __builtin_amdgcn_readfirstlane(threadIdx.x >> 6) : threadIdx.x >> 6;
  const int qn = lane & 31;
  const int hh = lane >> 5;
  const int rows = a.T * a.G;
  const int rg = wave % RG;                      // this wave's row group
  const int kh = wave / RG;                      // KSPLIT: this wave's half of each tile
  const int row0 = (rb * RG + rg) * 32;
  const int st0 = KSPLIT ? kh : 0;               // first 32-key subtile of this wave

  const __bf16 *Q = (const __bf16 *)a.q;
  const __bf16 *K = (const __bf16 *)a.k;
  const __bf16 *V = (const __bf16 *)a.v;
  const int64_t seq_base = PAGED ? 0 : (int64_t)(b * a.kv.hkv + g) * a.kv.cap * D;
  const int t_begin = split * a.tiles_per_split;

  bf16x8 qf[QT][KS];                             // filled from LDS in the prologue
  uint64_t anc_q[QT];                            // likewise
  // The sequence's ancestor masks, also global -> LDS by DMA (wave 0, 4-byte pieces),
  // into the same LDS array as the tiles.
  uint64_t *s_anc = (uint64_t *)(lds + kStages * 2 * MAT);
  // With a.parent set, the sequence's parents come instead (one 4-byte piece per node,
  // after the masks' area) and the masks are built from them in the prologue.
  int32_t *s_par = (int32_t *)(s_anc + kMaxNodes);
  auto issue_anc = [&]() {
    if constexpr (MASKS) {
      if (lane < a.T)
        __builtin_amdgcn_global_load_lds(
            (const __attribute__((address_space(1))) void *)(a.parent + (int64_t)b * a.T + lane),
            (__attribute__((address_space(3))) void *)s_par, 4, 0, 0);
      return;
    }
    const uint32_t *src = (const uint32_t *)(a.anc + (int64_t)b * a.T);
#pragma unroll
    for (int i = 0; i < 2; ++i)
      if (64 * i + lane < 2 * a.T)
        __builtin_amdgcn_global_load_lds(
            (const __attribute__((address_space(1))) void *)(src + 64 * i + lane),
            (__attribute__((address_space(3))) void *)((uint32_t *)s_anc + 64 * i), 4, 0, 0);
  };
  // This wave's 32 query rows travel global -> LDS by DMA, whole rows at a time and
  // chunk-swizzled like a K tile, into the area of stages 2 and 3 (idle until the third
  // tile is issued); the Q^T fragments are then read from there.  Fetched as ordinary
  // loads they would be scattered 16-byte gathers queued ahead of the K/V traffic, and
  // the compiler would drain every DMA in flight before their first use.  Rows past the
  // last one repeat it: their results are never written.  The two wavefronts of a
  // key-split group fetch 16 of the group's rows each.
  __bf16 *qlds = lds + 2 * 2 * MAT + rg * 32 * D;
  auto issue_q = [&]() {
    constexpr int NQ = 32 * DCH / 64;            // DMA instructions for 32 whole rows
    constexpr int QI = KSPLIT ? NQ / 2 : NQ;
#pragma unroll
    for (int ii = 0; ii < QI; ++ii) {
      const int i = KSPLIT ? kh * QI + ii : ii;
      const int rr = 4 * i + (lane >> 4), pc = lane & 15;
      const int r = min(row0 + rr, rows - 1);
      const int node = r / a.G, head = g * a.G + r % a.G;
      dma16(Q + (((int64_t)b * a.T + node) * a.Hq + head) * D + ((pc ^ (rr & 15)) << 3),
            qlds + i * 512);
    }
  };

  // Lane-constant parts of this wave's DMA: instruction i fills 1 KB block wave*IPW + i of
  // a tile, i.e. key rows 4*(wave*IPW + i) .. +3; lane l takes row key_i, physical chunk
  // l % 16, and so fetches logical chunk (l % 16) ^ swizzle(key_i).
  int dkey[IPW], doffK[IPW], doffV[IPW];
#pragma unroll
  for (int i = 0; i < IPW; ++i) {
    const int q = (wave * IPW + i) * 64 + lane;
    const int key = q / DCH, pc = q % DCH;
    dkey[i] = key;
    doffK[i] = ((pc ^ swap23(key & 15)) << 3);
    doffV[i] = ((pc ^ ((5 * (key & 3)) & 15)) << 3);
  }
  // DMA of one tile's K and V rows into stage stg, from element offsets row_of(slot).
  auto issue_rows = [&](int tile, int stg, auto row_of) {
    __bf16 *kd = lds + stg * 2 * MAT;
#pragma unroll
    for (int i = 0; i < IPW; ++i) {
      const int64_t off = row_of(tile * kKT + dkey[i]);
      const int blk = wave * IPW + i;
      dma16(K + off + doffK[i], kd + blk * 512);
      dma16(V + off + doffV[i], kd + MAT + blk * 512);
    }
  };

  // Prologue, first part: the masks, the query rows and, for a contiguous cache, the
  // split's first two tiles go out before the prefix length is known (its load is a
  // dependent round trip).  The speculative tiles read slots up to the end of the planned
  // key range, clamped into the cache; slots past the sequence are dealt with once the
  // length is known (V rows zeroed, scores masked).
  if (wave == 0) issue_anc();
  issue_q();
  int n_early = 0;                               // tiles issued before the length is known
  if constexpr (!PAGED) {
    auto spec_row = [&](int slot) {
      return seq_base + (int64_t)min<int64_t>(slot, a.kv.cap - 1) * D;
    };
    issue_rows(t_begin, 0, spec_row);
    n_early = 1;
    if (t_begin + 1 < a.max_tiles) {
      issue_rows(t_begin + 1, 1, spec_row);
      n_early = 2;
    }
  }

  const int nkeys = L + a.T;
  if (L < 0 || L > a.max_prefix || !a.kv.fits(nkeys)) {
    if (threadIdx.x == 0) report(a.dev_status, EV_DERR_BOUNDS);
    wait_vm<0>();                                // no DMA into LDS outlives the wave
    return;
  }
  const int ntiles = (nkeys + kKT - 1) / kKT;
  const int t_end = min(t_begin + a.tiles_per_split, ntiles);
  if (t_begin >= t_end) {
    // an empty split (a shorter sequence of the batch): its partial carries no weight
    if (a.n_splits > 1 && hh == 0 && row0 + qn < rows && kh == 0)
      a.part_ls[part_row(a, out_row(a, b, g, row0 + qn), split)] = pack_ls(-INFINITY, 1.f);
    wait_vm<0>();
    return;
  }

  int blk0 = 0;
  if (PAGED) {
    blk0 = (t_begin * kKT) >> a.kv.block_shift;
    const int nblk = ((min(t_end * kKT, nkeys) - 1) >> a.kv.block_shift) - blk0 + 1;
    bool bad = false;
    for (int i = threadIdx.x; i < nblk; i += NT) {
      const int blk = a.kv.table[(int64_t)b * a.kv.max_blocks + blk0 + i];
      const bool ok = blk >= 0 && blk < a.kv.n_blocks;
      bad |= !ok;
      stbl[i] = ok ? blk : -1;
    }
    if (__any(bad) && lane == 0) report(a.dev_status, EV_DERR_BOUNDS);
    __syncthreads();
  }

  // Element offset of a slot's row (PAGED: from the LDS block-id cache; bad ids read row 0,
  // already reported).
  auto row_off = [&](int slot) -> int64_t {
    if (!PAGED) return seq_base + (int64_t)slot * D;
    const int blk = stbl[(slot >> a.kv.block_shift) - blk0];
    if (blk < 0) return 0;
    return ((((int64_t)blk * a.kv.hkv + g) << a.kv.block_shift) |
            (slot & ((1 << a.kv.block_shift) - 1))) * D;
  };
  // A full tile whose DMA instructions each stay within one page (pages of 4 or more
  // tokens; a contiguous cache always): every instruction reads 4 consecutive slots, so
  // its address is a wave-uniform base (scalar arithmetic; a paged cache's block id from
  // a scalar load of the table, issued by page_ids ahead of the barrier that precedes the
  // DMA) plus a lane-constant offset.  Other tiles go slot by slot.
  const bool whole_pages = NW == 8 && (!PAGED || a.kv.block_shift >= 2);
  const int lrow = (lane >> 4) * D;              // slot within the instruction's four
  struct PageIds { int id[IPW]; };
  auto page_ids = [&](int tile) {
    PageIds p;
#pragma unroll
    for (int i = 0; i < IPW; ++i) {
      p.id[i] = 0;
      if constexpr (PAGED) {
        const int kq = tile * kKT + 4 * (wave * IPW + i);
        const int64_t e = (int64_t)b * a.kv.max_blocks + (min(kq, nkeys - 1) >> a.kv.block_shift);
        p.id[i] = scalar_load(a.kv.table, e);
      }
    }
    return p;
  };
  auto issue = [&](int tile, int stg, const PageIds &p) {
    const int key0 = tile * kKT;
    const bool full = key0 + kKT <= nkeys;
    if (full && whole_pages) {
      __bf16 *kd = lds + stg * 2 * MAT;
#pragma unroll
      for (int i = 0; i < IPW; ++i) {
        const int blk = wave * IPW + i;
        const int kq = key0 + 4 * blk;           // first slot of this instruction
        int64_t base;
        if constexpr (PAGED) {
          const int id = p.id[i] < 0 || p.id[i] >= a.kv.n_blocks ? 0 : p.id[i];   // reported
          base = ((((int64_t)id * a.kv.hkv + g) << a.kv.block_shift) +
                  (kq & ((1 << a.kv.block_shift) - 1))) * D;
        } else {
          base = seq_base + (int64_t)kq * D;
        }
        dma16(K + base + (uint32_t)(lrow + doffK[i]), kd + blk * 512);
        dma16(V + base + (uint32_t)(lrow + doffV[i]), kd + MAT + blk * 512);
      }
      return;
    }
    issue_rows(tile, stg, [&](int slot) {
      // past the sequence: finite data, masked out
      return row_off(!full && slot >= nkeys ? key0 : slot);
    });
  };
  // A speculatively issued tile that reaches past the sequence: once it has landed, each
  // wave zeroes the V rows past the sequence among those it fetched (a zero probability
  // times a stale value must not make NaN); the scores of those keys are masked anyway.
  auto fix_tail = [&](int tile, int stg) {
    const int key0 = tile * kKT;
    if (key0 + kKT <= nkeys) return;
    __bf16 *vd = lds + stg * 2 * MAT + MAT;
#pragma unroll
    for (int i = 0; i < IPW; ++i)
      if (key0 + dkey[i] >= nkeys) *(u32x4 *)(vd + (wave * IPW + i) * 512 + lane * 8) = u32x4{};
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  };
  // Wait until the tile `newer` tiles older than the newest issued one has landed.
  auto landed = [&](int newer) {
    if (newer >= 2) wait_vm<2 * PER>();
    else if (newer == 1) wait_vm<PER>();
    else wait_vm<0>();
  };

  // Lane-constant LDS offsets (elements) of the fragments within a stage.
  const int krow = swap23(qn);                   // key row within a subtile
  int koff[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) koff[ks] = krow * D + ((((2 * ks) | hh) ^ (qn & 15)) << 3);
  const int r16 = lane & 15, grp16 = lane >> 4;
  int voff[DT][2];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
#pragma unroll
    for (int hr = 0; hr < 2; ++hr) {
      const int rr = (r16 >> 2) + 4 * hr;        // key within the 8-key group
      const int d = dt * 32 + 16 * (grp16 & 1) + 4 * (r16 & 3);
      voff[dt][hr] = (8 * hh + rr) * D + (((d >> 3) ^ ((5 * (rr & 3)) & 15)) << 3) + (d & 7);
    }

  f32x16 o[QT][DT];
  float mref[QT] = {-INFINITY}, l[QT] = {0.f};
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) o[0][dt] = f32x16{};

  // Stage index is a compile-time constant in every call below, so all LDS addresses are
  // a lane-constant register plus an immediate offset (plus the subtile of a key-split
  // wave).
  auto scores_of = [&](f32x16 (&sc)[QT][NST], auto stg) {
    const __bf16 *kb = lds + decltype(stg)::value * 2 * MAT + st0 * 32 * D;
    tile_scores<QT, KS, NST>(sc, qf, [&](int st, int ks) {
      return *(const bf16x8 *)(kb + st * 32 * D + koff[ks]);
    });
  };
  auto pv_of = [&](const bf16x8 (&pf)[QT][NST][2], auto stg) {
    const __bf16 *vb = lds + decltype(stg)::value * 2 * MAT + MAT + st0 * 32 * D;
    tile_pv<QT, DT, NST>(o, pf, [&](int st, int kk, int dt) {
      const __bf16 *base = vb + (st * 32 + kk * 16) * D;
      const bf16x4 lo = lds_read_tr((lds_bf16x4 *)(base + voff[dt][0]));
      const bf16x4 hi = lds_read_tr((lds_bf16x4 *)(base + voff[dt][1]));
      return bf16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    });
  };
  using S0 = std::integral_constant<int, 0>;
  using S1 = std::integral_constant<int, 1>;
  using S2 = std::integral_constant<int, 2>;
  using S3 = std::integral_constant<int, 3>;

  // One pipeline step for tile j in stage STG: make tile j+1 visible, refill the stage of
  // j-1 with tile j+3, and compute the scores of j+1 (into sn; the matrix cores run them
  // while the wave continues) before the softmax and P V of j.  Returns false when j was
  // the last tile.
  auto step = [&](int j, f32x16 (&sc)[QT][NST], f32x16 (&sn)[QT][NST], auto stg) -> bool {
    constexpr int STG = decltype(stg)::value;
    using NEXT = std::integral_constant<int, (STG + 1) % kStages>;
    using REFILL = std::integral_constant<int, (STG + 3) % kStages>;
    const bool more = j + 1 < t_end;
    if (more) {
      const PageIds ids = page_ids(j + 3);       // in flight while the tile lands
      landed(min(t_end - 1, j + 2) - (j + 1));
      if constexpr (!PAGED)
        if (j == t_begin) fix_tail(j + 1, NEXT::value);   // the second early tile
      wg_barrier();                              // tile j+1 visible; stage of j-1 free
      // A contiguous cache issues the next tile's score products before the refill DMA
      // (GQA 64/8 L=4096: 19.61 -> 19.35 us per call).  With a paged cache that order
      // made the compiler wait for the refill before the V reads of every step.
      if constexpr (PAGED) {
        if (j + 3 < t_end) issue(j + 3, REFILL::value, ids);
        scores_of(sn, NEXT{});
      } else {
        scores_of(sn, NEXT{});
        if (j + 3 < t_end) issue(j + 3, REFILL::value, ids);
      }
    }
    if (j * kKT + kKT > L) tile_mask(sc, anc_q, j * kKT + st0 * 32, L, hh);
    tile_rescale(sc, o, mref, l, a.scale_log2);
    bf16x8 pf[QT][NST][2];
    tile_exp(sc, pf, mref, l, a.scale_log2);
    pv_of(pf, stg);
    return more;
  };

  // Prologue, second part: a paged cache's first two tiles (their block ids are in LDS
  // now).  Once this wave's Q rows have landed its fragments are read, and after every
  // wave has them the third tile goes into the area they occupied; then the scores of the
  // first tile.
  if constexpr (PAGED) {
    issue(t_begin, 0, page_ids(t_begin));
    n_early = 1;
    if (t_begin + 1 < t_end) {
      issue(t_begin + 1, 1, page_ids(t_begin + 1));
      n_early = 2;
    }
  }
  if (n_early == 2) wait_vm<2 * PER>();          // masks and Q landed (this wave's own rows)
  else wait_vm<PER>();
  if constexpr (KSPLIT) wg_barrier();            // and the other half of the group's rows
#pragma unroll
  for (int ks = 0; ks < KS; ++ks)
    qf[0][ks] = *(const bf16x8 *)(qlds + qn * D + ((((2 * ks) | hh) ^ (qn & 15)) << 3));
  // Masks from the parents (their DMA has landed with this wave's Q rows): only workgroups
  // whose keys reach the tree slots use them, so only those build them; the one holding
  // the sequence's last tile for KV head 0 and row block 0 also writes them out.
  if constexpr (MASKS)
    if (wave == 0 && t_end * kKT > L)
      build_masks(a, b, s_par, s_anc, g == 0 && rb == 0 && t_end == ntiles);
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  wg_barrier();                                  // every wave holds its Q: stages 2, 3 free
  anc_q[0] = row0 + qn < rows ? s_anc[(row0 + qn) / a.G] : 0ull;
  if (t_begin + 2 < t_end) issue(t_begin + 2, 2, page_ids(t_begin + 2));
  // (with an early second tile beyond t_end this waits for everything in flight)
  landed(min(t_end - 1, t_begin + 2) - t_begin);
  if constexpr (!PAGED) fix_tail(t_begin, 0);
  wg_barrier();
  f32x16 sa[QT][NST], sb[QT][NST];
  scores_of(sa, S0{});
  for (int j = t_begin;; j += 4) {
    if (!step(j, sa, sb, S0{})) break;
    if (!step(j + 1, sb, sa, S1{})) break;
    if (!step(j + 2, sa, sb, S2{})) break;
    if (!step(j + 3, sb, sa, S3{})) break;
  }
  // Once a wave has left the loop, the others are at most one step behind: they may still
  // read the stages of the last two tiles, never the two after them, and no DMA is in
  // flight.  Those two stages hold the waves' output rows (8 KB each).
  const int last = (t_end - 1 - t_begin) % kStages;
  if constexpr (KSPLIT) {
    // exchange areas: with one group the two stages after the last tile's (no wave reads
    // them any more); with four (72 KB), stages 0-2 once every wave is past its last tile;
    // the staging rows of the groups follow in stage 3
    float *xch;
    uint16_t *gstage;
    if constexpr (NW == 2) {
      xch = (float *)(lds + ((last + 2) % kStages) * 2 * MAT);
      gstage = (uint16_t *)(lds + ((last + 1) % kStages) * 2 * MAT);
    } else {
      __syncthreads();
      xch = (float *)lds + rg * 2 * (3 + DT / 2 * 16) * 64;
      gstage = (uint16_t *)(lds + 3 * 2 * MAT + rg * 32 * D);
    }
    if (__builtin_amdgcn_readfirstlane(kh) == 0)
      finish_pair<D, RG * 32 >= 128, 0>(a, o, mref[0], l[0], row0, b, g, split, qn, hh, xch, gstage);
    else
      finish_pair<D, RG * 32 >= 128, 1>(a, o, mref[0], l[0], row0, b, g, split, qn, hh, xch, gstage);
    return;
  }
  uint16_t *stage = (uint16_t *)(lds + ((last + 1 + (wave >> 2)) % kStages) * 2 * MAT +
                                 (wave & 3) * 32 * D);
  // Partial rows go non-temporally from workgroups of 128 rows or more; a split plan of
  // smaller workgroups writes at most 256 x 64 partial rows (4 MB), which stay cached
  // (measured: 8 MB of partials, 8 splits of 4096 rows, 22.3 us per call non-temporal
  // against 22.9 cached; 1.5 MB, 7 splits of 832 rows, 18.9 against 18.6).
  write_rows_staged<D, RG * 32 >= 128>(a, o, mref[0], l[0], row0, b, g, split, qn, hh, stage);
}

// Combine split partials: lse = log sum_s exp(lse_s), O = sum_s exp(lse_s - lse) O_s.
// D/E lanes per row (sequence, node, head), E head-dim elements per lane; the partials are
// read in batches of BATCH splits (all loads of a batch in flight together) and combined
// with a running maximum.
template <int D, int E, int BATCH>
__global__ __launch_bounds__(256) void attn_merge_kernel(AttnArgs a) {
  constexpr int LPR = D / E;             // lanes per row
  constexpr int RPB = 256 / LPR;         // rows per workgroup
  args_in_sgprs(a.B, a.T, a.Hq, a.n_splits, a.part_o, a.part_ls, a.out, a.lse);
  typedef _Float16 hE __attribute__((ext_vector_type(E)));
  typedef __bf16 bE __attribute__((ext_vector_type(E)));
  const int64_t nrows = (int64_t)a.B * a.T * a.Hq;
  const int64_t row = (int64_t)blockIdx.x * RPB + threadIdx.x / LPR;
  const int c = threadIdx.x % LPR;
  if (row >= nrows) return;
  // Every split wrote its partial LSE (an empty split -inf), so all n_splits are read
  // without waiting for the sequence length.
  const int nvalid = a.n_splits;
  float mx = -INFINITY, wsum = 0.f;
  float acc[E] = {};
  for (int s0 = 0; s0 < nvalid; s0 += BATCH) {
    float ls[BATCH], sc[BATCH];
    hE x[BATCH];
#pragma unroll
    for (int u = 0; u < BATCH; ++u) {
      const int s = s0 + u;
      const bool ok = s < nvalid;
      const uint64_t w = ok ? a.part_ls[row * nvalid + s] : pack_ls(-INFINITY, 0.f);
      ls[u] = ls_lse(w);
      sc[u] = ls_scale(w);
      x[u] = ok ? *(const hE *)(a.part_o + (row * nvalid + s) * D + c * E) : hE{};
    }
    float bm = mx;
#pragma unroll
    for (int u = 0; u < BATCH; ++u) bm = fmaxf(bm, ls[u]);
    if (bm == -INFINITY) continue;
    const float r = mx == -INFINITY ? 0.f : exp2f((mx - bm) * kLog2e);
    wsum *= r;
#pragma unroll
    for (int e = 0; e < E; ++e) acc[e] *= r;
#pragma unroll
    for (int u = 0; u < BATCH; ++u) {
      // a split without weight (LSE -inf) may hold unwritten partials: select, not multiply
      const bool live = ls[u] != -INFINITY;
      const float w = live ? exp2f((ls[u] - bm) * kLog2e) : 0.f;
      wsum += w;
      const float ws = w * sc[u];
#pragma unroll
      for (int e = 0; e < E; ++e) acc[e] += live ? ws * (float)x[u][e] : 0.f;
    }
    mx = bm;
  }
  const float inv = wsum > 0.f ? 1.f / wsum : 0.f;
  bE o;
#pragma unroll
  for (int e = 0; e < E; ++e) o[e] = (__bf16)(acc[e] * inv);
  *(bE *)((__bf16 *)a.out + row * D + c * E) = o;
  if (c == 0) a.lse[row] = wsum > 0.f ? mx + logf(wsum) : -INFINITY;
}

// float32 path: one workgroup per (sequence, KV head, block of R query rows): 8 wavefronts
// for a block of 8 rows (one row each), 4 for a block of 32.
// 64-key K and V tiles reach LDS through coalesced 16-byte loads, the next tile's loads in
// flight in registers while the current one is computed.  Scores: lane k of wavefront w
// scores key k against rows w, w + NWV, ... (query rows are broadcast reads), so a row's 64
// scores lie across one wavefront and its max and sum are wavefront (DPP) reductions.  P V:
// thread t owns head dimension t % D of rows t / D, t / D + 256 / D, ...
// Workgroup barrier for LDS data only: the wave's LDS accesses complete, then s_barrier.
// Unlike __syncthreads it does not wait for global loads, so a tile prefetched into
// registers stays in flight across it.

template <int D, int R, bool PAGED, int NT>
__global__ __launch_bounds__(NT) void tree_attn_f32_kernel(AttnArgs a) {
  constexpr int NWV = NT / 64;              // wavefronts
  constexpr int C4 = D / 4;                 // 16-byte pieces per row
  constexpr int LPT = kKT * C4 / NT;        // pieces per thread per K or V tile
  constexpr int KP = D + 4;                 // K tile pitch: 16-byte reads of row k by lane k
                                            // cover all 64 banks across 16 lanes
  constexpr int RW = R / NWV;               // score rows per wavefront
  constexpr int RSTEP = NT / D;             // row stride of a thread's P V rows
  constexpr int RPT = R / RSTEP;            // P V rows per thread
  static_assert(R % NWV == 0 && R % RSTEP == 0, "row block must tile the workgroup");
  // the 8-row block unrolls its LDS loops fully (all reads in flight together, and its
  // register-held query rows indexed by constants); the 32-row block would run out of
  // registers doing so
  constexpr bool QREG = RW * D <= 128 && D == 64;   // query rows held in registers
  constexpr int UNR = QREG ? D / 4 : (R == 8 ? 8 : 2);
  __shared__ __attribute__((aligned(16))) float sQ[R * D];
  __shared__ __attribute__((aligned(16))) float sK[kKT * KP];
  __shared__ __attribute__((aligned(16))) float sV[kKT * D];
  __shared__ __attribute__((aligned(16))) float sP[R * kKT];
  __shared__ float sA[R], sM[R], sL[R];

  args_in_sgprs(a.row_blocks, a.kv.hkv, a.kv.cap, a.T, a.G, a.Hq, a.q, a.k, a.v, a.anc,
                a.prefix_len, a.max_prefix);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int rb = blockIdx.x % a.row_blocks;
  const int bg = blockIdx.x / a.row_blocks;
  const int b = bg / a.kv.hkv, g = bg % a.kv.hkv;
  const int L = scalar_load(a.prefix_len, b);   // waited for after the first loads
  const int rows = a.T * a.G;
  const int row0 = rb * R;
  const int nrow = min(R, rows - row0);
  const float *Q = (const float *)a.q;
  const float *K = (const float *)a.k;
  const float *V = (const float *)a.v;
  auto orow_of = [&](int r) {               // output row of block row r (r < nrow)
    const int rr = row0 + r;
    return ((int64_t)b * a.T + rr / a.G) * a.Hq + g * a.G + rr % a.G;
  };

  // Loads that do not need the prefix length go out before it is known: the block's query
  // rows (zero past the last row), the ancestor masks and, for a contiguous cache, the
  // first K/V tile (slots clamped into the cache; keys past the sequence are zeroed when
  // stored and masked when scored).
  constexpr int QPT = (R * C4 + NT - 1) / NT;
  f32x4 qx[QPT];
#pragma unroll
  for (int u = 0; u < QPT; ++u) {
    const int i = tid + u * NT, r = i / C4, c = i % C4;
    qx[u] = f32x4{};
    if (i < R * C4 && r < nrow) qx[u] = *(const f32x4 *)(Q + orow_of(r) * D + 4 * c);
  }
  uint64_t anc[RW];
#pragma unroll
  for (int i = 0; i < RW; ++i) {
    const int r = wave + NWV * i;
    anc[i] = r < nrow ? a.anc[(int64_t)b * a.T + (row0 + r) / a.G] : 0ull;
  }

  // Every piece is loaded unconditionally from an in-bounds address (contiguous: a slot
  // past the cache reloads its last slot; paged, loaded once the length is known: a slot
  // past the sequence reloads its last slot, a bad block id reads the cache's first row)
  // and masked only when stored: a load under a per-lane branch made the compiler wait
  // for it at once.
  f32x4 kr[LPT], vr[LPT];
  bool bad = false;
  int key0_loaded = 0;
  int nkeys = 0;
  auto load = [&](int key0) {
    key0_loaded = key0;
#pragma unroll
    for (int i = 0; i < LPT; ++i) {
      const int piece = tid + i * NT, key = piece / C4, c = piece % C4;
      int64_t off;
      if constexpr (PAGED) {
        off = a.kv.slot_offset(b, g, min(key0 + key, nkeys - 1));
        bad |= off < 0;
        off = off < 0 ? 0 : off;
      } else {
        off = ((int64_t)(b * a.kv.hkv + g) * a.kv.cap + min<int64_t>(key0 + key, a.kv.cap - 1)) * D;
      }
      kr[i] = *(const f32x4 *)(K + off + 4 * c);
      vr[i] = *(const f32x4 *)(V + off + 4 * c);
    }
  };
  auto store = [&]() {
#pragma unroll
    for (int i = 0; i < LPT; ++i) {
      const int piece = tid + i * NT, key = piece / C4, c = piece % C4;
      const bool live = key0_loaded + key < nkeys;
      *(f32x4 *)(sK + key * KP + 4 * c) = live ? kr[i] : f32x4{};
      *(f32x4 *)(sV + key * D + 4 * c) = live ? vr[i] : f32x4{};
    }
  };
  if constexpr (!PAGED) load(0);

  nkeys = L + a.T;
  if (L < 0 || L > a.max_prefix || !a.kv.fits(nkeys)) {
    if (tid == 0) report(a.dev_status, EV_DERR_BOUNDS);
    if constexpr (!PAGED)
#pragma unroll
      for (int i = 0; i < LPT; ++i) asm volatile("" ::"v"(kr[i]), "v"(vr[i]));   // keeps the
      // early tile's loads above this branch (the compiler sank them past it otherwise)
    return;
  }
  if constexpr (PAGED) load(0);
#pragma unroll
  for (int u = 0; u < QPT; ++u) {
    const int i = tid + u * NT;
    if (i < R * C4) *(f32x4 *)(sQ + i * 4) = qx[u];
  }

  float m[RW], l[RW], o[RPT];
#pragma unroll
  for (int i = 0; i < RW; ++i) m[i] = -INFINITY, l[i] = 0.f;
#pragma unroll
  for (int j = 0; j < RPT; ++j) o[j] = 0.f;
  const int dim = tid % D, prow = tid / D;

  // With at most two rows of 64 dimensions per wavefront the query rows are held in
  // registers (up to 128 per lane) instead of being re-read from LDS for every key tile:
  // a broadcast read still moves 1 KB through the LDS per instruction.
  f32x4 qr[QREG ? RW : 1][QREG ? D / 4 : 1];
  const int ntiles = (nkeys + kKT - 1) / kKT;
  if constexpr (QREG) {
    lds_barrier();                          // the query rows are in LDS
#pragma unroll
    for (int i = 0; i < RW; ++i)
#pragma unroll
      for (int c = 0; c < D / 4; ++c)
        qr[i][c] = *(const f32x4 *)(sQ + (wave + NWV * i < nrow ? wave + NWV * i : 0) * D + 4 * c);
  }
  for (int t = 0; t < ntiles; ++t) {
    lds_barrier();                          // the previous tile's P V is done with sK/sV/sP
    store();
    lds_barrier();
    if (t + 1 < ntiles) load((t + 1) * kKT);
    const int slot = t * kKT + lane;
    float s[RW];
#pragma unroll
    for (int i = 0; i < RW; ++i) s[i] = 0.f;
    // rows past the block's last read row 0's query (broadcast) and are never used
#pragma unroll UNR
    for (int d = 0; d < D; d += 4) {
      const f32x4 kv = *(const f32x4 *)(sK + lane * KP + d);
#pragma unroll
      for (int i = 0; i < RW; ++i) {
        const f32x4 qv = QREG ? qr[i][d / 4]
                              : *(const f32x4 *)(sQ + (wave + NWV * i < nrow ? wave + NWV * i : 0) * D + d);
        s[i] = fmaf(qv[0], kv[0], fmaf(qv[1], kv[1], fmaf(qv[2], kv[2], fmaf(qv[3], kv[3], s[i]))));
      }
    }
#pragma unroll
    for (int i = 0; i < RW; ++i) {
      const int r = wave + NWV * i;
      if (r >= nrow) continue;             // uniform across the wavefront
      const bool ok = slot < nkeys && visible(slot, L, anc[i]);
      const float x = ok ? s[i] * a.scale_log2 : -INFINITY;
      const float mnew = fmaxf(m[i], wave_max_f(x));
      const float alpha = mnew == -INFINITY ? 1.f : exp2f(m[i] - mnew);
      const float p = ok ? exp2f(x - mnew) : 0.f;
      l[i] = l[i] * alpha + wave_sum_f(p);
      m[i] = mnew;
      sP[r * kKT + lane] = p;
      if (lane == 0) sA[r] = alpha;
    }
    lds_barrier();
    // keys in the outer loop: each V element read once feeds all of the thread's rows
#pragma unroll
    for (int j = 0; j < RPT; ++j) {
      const int r = prow + RSTEP * j;
      o[j] *= r < nrow ? sA[r] : 1.f;
    }
#pragma unroll UNR
    for (int k = 0; k < kKT; k += 4) {
      const float v0 = sV[k * D + dim], v1 = sV[(k + 1) * D + dim];
      const float v2 = sV[(k + 2) * D + dim], v3 = sV[(k + 3) * D + dim];
#pragma unroll
      for (int j = 0; j < RPT; ++j) {
        const int r = prow + RSTEP * j;
        const f32x4 pv = *(const f32x4 *)(sP + (r < nrow ? r : 0) * kKT + k);
        o[j] = fmaf(pv[0], v0, fmaf(pv[1], v1, fmaf(pv[2], v2, fmaf(pv[3], v3, o[j]))));
      }
    }
  }
  if (__any(bad) && lane == 0) report(a.dev_status, EV_DERR_BOUNDS);
#pragma unroll
  for (int i = 0; i < RW; ++i) {
    const int r = wave + NWV * i;
    if (r < nrow && lane == 0) {
      sM[r] = m[i];
      sL[r] = l[i];
      a.lse[orow_of(r)] = l[i] > 0.f ? (m[i] + log2f(l[i])) * kLn2 : -INFINITY;
    }
  }
  lds_barrier();
#pragma unroll
  for (int j = 0; j < RPT; ++j) {
    const int r = prow + RSTEP * j;
    if (r >= nrow) continue;
    const float lt = sL[r];
    ((float *)a.out)[orow_of(r) * D + dim] = lt > 0.f ? o[j] / lt : 0.f;
  }
}

// ---------------------------------------------------------------------------------------
// Launch policy.
constexpr int kCUs = 256;
constexpr int kShortSplit = 16;   // tiles per split up to which GQA plans halve their row blocks

struct Plan {
  int nw;                // waves per workgroup
  bool dma;              // bf16 d = 128: the direct-to-LDS kernel
  bool ksplit;           // DMA kernel whose wave pairs split each tile's keys
  int row_blocks;
  int tiles_per_split, n_splits;
  int max_tiles;         // 64-key tiles of the planned key range
  int n_work, grid;
};

// Query rows per float32 workgroup: 8 for small groups (the fp32 configuration has 8 rows
// per KV head), else 32.
static int f32_rows(int rows) { return rows <= 8 ? 8 : 32; }

static int64_t max_slots(const KvAddr &kv) {
  if (!kv.paged) return kv.cap;
  return (int64_t)kv.max_blocks << kv.block_shift;
}

// Key slots the plan covers: the longest prefix the call may see plus the tree, never more
// than the cache holds (a longer sequence cannot fit and is reported by the kernel).
static int plan_slots(const KvAddr &kv, int T, int64_t max_prefix_len) {
  const int64_t want = std::min<int64_t>(max_prefix_len, 1 << 30) + T;
  return (int)std::min<int64_t>(std::min<int64_t>(want, max_slots(kv)), 1 << 30);
}

// Splits are sized so that one round of workgroups fills the chip (GQA: one 8-wave
// workgroup per CU; MHA: four 1-wave workgroups per CU), at most kMaxSplits of them, over
// the key range of the longest prefix the call may see; a paged split's block ids must
// fit the LDS cache.
static Plan make_plan(const KvAddr &kv, int dtype, int B, int T, int Hq, int64_t max_prefix_len) {
  Plan p{};
  const int G = Hq / kv.hkv;
  const int rows = T * G;
  if (dtype == EV_F32) {
    p.nw = 4;
    p.row_blocks = (rows + f32_rows(rows) - 1) / f32_rows(rows);
    p.n_splits = 1;
    p.tiles_per_split = 1 << 30;
    p.max_tiles = (plan_slots(kv, T, max_prefix_len) + kKT - 1) / kKT;
    p.n_work = B * kv.hkv * p.row_blocks;
    p.grid = p.n_work;
    return p;
  }
  // Waves of 32 query rows, up to 8 per workgroup (two waves per SIMD, no accumulator
  // spill to AGPRs).
  const int waves_needed = (rows + 31) / 32;
  p.nw = waves_needed >= 8 ? 8 : waves_needed >= 4 ? 4 : (waves_needed >= 2 ? 2 : 1);
  // An INT4 tile is dequantised by every thread of the workgroup while staging: at least
  // four wavefronts share that work even when fewer own query rows.
  if (dtype == EV_INT4) p.nw = std::max(p.nw, 4);
  // bf16 with d = 128 always takes the direct-to-LDS kernel, whose smallest workgroup has
  // two wavefronts (with at most 32 rows per KV head the second owns none and only shares
  // the DMA issue); its 128 KB of LDS leave room for one workgroup per CU.
  const bool dma = dtype == EV_BF16 && kv.d == 128;
  if (dma) p.nw = std::max(p.nw, 2);
  p.dma = dma;
  p.ksplit = dma && waves_needed == 1;
  const int max_tiles = (plan_slots(kv, T, max_prefix_len) + kKT - 1) / kKT;
  const int slots = dma || p.nw >= 4 ? kCUs : (p.nw == 2 ? 2 * kCUs : 4 * kCUs);
  // split the planned key range over enough workgroups to fill `slots`
  auto split_plan = [&](int groups_per_wg) {
    p.row_blocks = (waves_needed + groups_per_wg - 1) / groups_per_wg;
    const int units = B * kv.hkv * p.row_blocks;
    int splits = std::max(1, slots / units);
    splits = std::min(splits, std::min(kMaxSplits, max_tiles));
    int tps = (max_tiles + splits - 1) / splits;
    if (kv.paged) {
      // a split's block ids must fit the LDS cache
      const int blocks_per_tile = std::max(1, kKT >> kv.block_shift);
      tps = std::min(tps, (kTableCache - 1) / blocks_per_tile);
    }
    p.tiles_per_split = tps;
    p.n_splits = (max_tiles + tps - 1) / tps;
    p.n_work = units * p.n_splits;
  };
  split_plan(p.ksplit ? 1 : p.nw);
  // Short split loops (a few tiles per workgroup, the partials a large part of the
  // traffic): eight-wave workgroups take 128 rows instead of 256, their wave pairs
  // splitting every tile's keys, when that still fits one round of workgroups.
  if (dma && p.nw == 8 && p.n_splits > 1 && p.tiles_per_split <= kShortSplit &&
      (int64_t)B * kv.hkv * ((waves_needed + 3) / 4) <= kCUs) {
    p.ksplit = true;
    split_plan(4);
  }
  p.max_tiles = max_tiles;
  p.grid = (p.n_work + kXcds - 1) / kXcds * kXcds;
  return p;
}

static size_t part_rows(const Plan &p, int B, int T, int Hq) {
  return (size_t)p.n_splits * B * T * Hq;
}

// Workspace of a split plan: the fp16 partial rows, then their (LSE, divisor) words.
static size_t workspace_bytes(const Plan &p, int B, int T, int Hq, int D) {
  if (p.n_splits <= 1) return 0;
  size_t rows = part_rows(p, B, T, Hq);
  return align_up(rows * D * sizeof(_Float16), 256) + align_up(rows * sizeof(uint64_t), 256);
}

template <bool PAGED, bool MASKS>
static void launch_dma(const Plan &p, const AttnArgs &a, dim3 grid, hipStream_t stream) {
  if (p.nw == 8 && p.ksplit)
    hipLaunchKernelGGL((tree_attn_dma_kernel<8, PAGED, true, MASKS>), grid, dim3(512), 0, stream, a);
  else if (p.nw == 8)
    hipLaunchKernelGGL((tree_attn_dma_kernel<8, PAGED, false, MASKS>), grid, dim3(512), 0, stream, a);
  else if (p.nw == 4)
    hipLaunchKernelGGL((tree_attn_dma_kernel<4, PAGED, false, MASKS>), grid, dim3(256), 0, stream, a);
  else if (p.ksplit)
    hipLaunchKernelGGL((tree_attn_dma_kernel<2, PAGED, true, MASKS>), grid, dim3(128), 0, stream, a);
  else
    hipLaunchKernelGGL((tree_attn_dma_kernel<2, PAGED, false, MASKS>), grid, dim3(128), 0, stream, a);
}

template <int D, bool PAGED, bool Q4>
static void launch_main(const Plan &p, const AttnArgs &a, hipStream_t stream) {
  dim3 grid(p.grid);
  if constexpr (!Q4 && D == 128) {
    // bf16 with d = 128: the direct-to-LDS kernel (the plan gives it at least 2 waves)
    if (a.parent)
      launch_dma<PAGED, true>(p, a, grid, stream);
    else
      launch_dma<PAGED, false>(p, a, grid, stream);
  } else if (p.nw == 8) {
    hipLaunchKernelGGL((tree_attn_bf16_kernel<D, 1, 8, PAGED, Q4>), grid, dim3(512), 0, stream, a);
  } else if (p.nw == 4) {
    hipLaunchKernelGGL((tree_attn_bf16_kernel<D, 1, 4, PAGED, Q4>), grid, dim3(256), 0, stream, a);
  } else if constexpr (!Q4) {
    // d = 64 bf16 only: INT4 plans have at least four waves
    if (p.nw == 2)
      hipLaunchKernelGGL((tree_attn_bf16_kernel<D, 1, 2, PAGED, Q4>), grid, dim3(128), 0, stream, a);
    else
      hipLaunchKernelGGL((tree_attn_bf16_kernel<D, 1, 1, PAGED, Q4>), grid, dim3(64), 0, stream, a);
  }
}

template <int D>
static void launch_bf16(const Plan &p, const AttnArgs &a, bool q4, hipStream_t stream) {
  if (q4) {
    if (a.kv.paged)
      launch_main<D, true, true>(p, a, stream);
    else
      launch_main<D, false, true>(p, a, stream);
  } else if (a.kv.paged) {
    launch_main<D, true, false>(p, a, stream);
  } else {
    launch_main<D, false, false>(p, a, stream);
  }
  if (p.n_splits > 1) {
    constexpr int E = 4 * D / 128;
    const int64_t nrows = (int64_t)a.B * a.T * a.Hq;
    const int rows_per_wg = 256 / (D / E);
    dim3 mgrid((unsigned)((nrows + rows_per_wg - 1) / rows_per_wg));
    hipLaunchKernelGGL((attn_merge_kernel<D, E, 8>), mgrid, dim3(256), 0, stream, a);
  }
}

template <bool PAGED>
static void launch_f32(const Plan &p, const AttnArgs &a, int T, hipStream_t stream) {
  const bool small = f32_rows(T * a.G) == 8;
  dim3 grid(p.grid);
  if (a.kv.d == 64 && small)
    hipLaunchKernelGGL((tree_attn_f32_kernel<64, 8, PAGED, 512>), grid, dim3(512), 0, stream, a);
  else if (a.kv.d == 64)
    hipLaunchKernelGGL((tree_attn_f32_kernel<64, 32, PAGED, 256>), grid, dim3(256), 0, stream, a);
  else if (small)
    hipLaunchKernelGGL((tree_attn_f32_kernel<128, 8, PAGED, 512>), grid, dim3(512), 0, stream, a);
  else
    hipLaunchKernelGGL((tree_attn_f32_kernel<128, 32, PAGED, 256>), grid, dim3(256), 0, stream, a);
}

}  // namespace ev

EV_API size_t ev_tree_attention_workspace(const ev_kv_desc *kv, int32_t B, int32_t T, int32_t Hq,
                                          int64_t max_prefix_len) {
  ev::KvAddr addr;
  if (ev::make_kv_addr(kv, &addr) != EV_OK || B < 1 || T < 1 || T > ev::kMaxNodes || Hq < 1 ||
      Hq % kv->n_kv_heads || max_prefix_len < 0)
    return 0;
  ev::Plan p = ev::make_plan(addr, kv->dtype, B, T, Hq, max_prefix_len);
  return ev::workspace_bytes(p, B, T, Hq, kv->head_dim);
}

namespace ev {

// ev_tree_attention's work with the workspace given; scratch_call: the workspace is the
// fixed scratch array, so a plan that needs more than ws_bytes is EV_ERR_SCRATCH.
// With `parent` set (ev_tree_mask_attention) the masks are built from it and written to
// anc_out (and depth_out): inside the direct-to-LDS kernel, else by the mask kernel
// launched first.
static ev_status attention_call(const void *q, const ev_kv_desc *kv, const int32_t *prefix_len,
                                const uint64_t *anc_mask, int32_t B, int32_t T, int32_t Hq,
                                int64_t max_prefix_len, float sm_scale, void *out, float *lse,
                                void *ws, size_t ws_bytes, int32_t *dev_status,
                                hipStream_t stream, bool scratch_call,
                                const int32_t *parent = nullptr, uint64_t *anc_out = nullptr,
                                int32_t *depth_out = nullptr) {
  ev::KvAddr addr;
  ev_status st = ev::make_kv_addr(kv, &addr);
  if (st != EV_OK) return st;
  if (B < 0 || T < 1 || T > ev::kMaxNodes || Hq < 1 || Hq % kv->n_kv_heads || max_prefix_len < 0)
    return EV_ERR_SHAPE;
  if (!(sm_scale > 0.f) || !isfinite(sm_scale)) return EV_ERR_ARG;
  if (B == 0) return EV_OK;
  if (!q || !prefix_len || !out || !lse) return EV_ERR_NULL;
  if (parent ? !anc_out : !anc_mask) return EV_ERR_NULL;
  // rows of q, out and the cache are read and written in 16-byte pieces
  if (((uintptr_t)q | (uintptr_t)out | (uintptr_t)kv->k | (uintptr_t)kv->v) & 15) return EV_ERR_ARG;
  if ((int64_t)B * kv->n_kv_heads > (1 << 24)) return EV_ERR_SHAPE;
  ev::Plan p = ev::make_plan(addr, kv->dtype, B, T, Hq, max_prefix_len);
  size_t need = ev::workspace_bytes(p, B, T, Hq, kv->head_dim);
  if (ws_bytes < need || (need && !ws)) return scratch_call ? EV_ERR_SCRATCH : EV_ERR_WORKSPACE;

  ev::AttnArgs a{};
  a.q = q;
  a.k = kv->k;
  a.v = kv->v;
  a.k_scale = kv->k_scale;
  a.v_scale = kv->v_scale;
  a.kv = addr;
  a.prefix_len = prefix_len;
  a.anc = anc_mask;
  a.B = B;
  a.T = T;
  a.Hq = Hq;
  a.G = Hq / kv->n_kv_heads;
  a.max_prefix = (int)std::min<int64_t>(max_prefix_len, 1 << 30);
  a.max_tiles = p.max_tiles;
  a.scale_log2 = sm_scale * ev::kLog2e;
  a.row_blocks = p.row_blocks;
  a.tiles_per_split = p.tiles_per_split;
  a.n_splits = p.n_splits;
  a.n_work = p.n_work;
  a.out = out;
  a.lse = lse;
  a.dev_status = dev_status;
  if (parent) {
    if (p.dma) {
      a.parent = parent;
      a.anc_out = anc_out;
      a.depth_out = depth_out;
    } else {
      st = ev_tree_mask_build(parent, B, T, anc_out, depth_out, dev_status, stream);
      if (st != EV_OK) return st;
      a.anc = anc_out;
    }
  }
  if (need) {
    size_t rows = ev::part_rows(p, B, T, Hq);
    char *base = (char *)ws;
    const size_t o_bytes = ev::align_up(rows * kv->head_dim * sizeof(_Float16), 256);
    a.part_o = (_Float16 *)base;
    a.part_ls = (uint64_t *)(base + o_bytes);
  }
  if (kv->dtype == EV_F32) {
    if (kv->paged)
      ev::launch_f32<true>(p, a, T, stream);
    else
      ev::launch_f32<false>(p, a, T, stream);
  } else {
    const bool q4 = kv->dtype == EV_INT4;
    if (kv->head_dim == 64)
      ev::launch_bf16<64>(p, a, q4, stream);
    else
      ev::launch_bf16<128>(p, a, q4, stream);
  }
  return ev::launch_status();
}

// Workspace of the no-allocation entry point: one fixed array per GPU, holding the split
// partials of the call in progress.  In host code its name stands for no device address;
// the address comes from hipGetSymbolAddress, once per device.
constexpr size_t kScratchBytes = size_t(32) << 20;
constexpr int kScratchDevices = 64;
static std::mutex g_scratch_mu;
static void *g_scratch_ptr[kScratchDevices];

}  // namespace ev

static __device__ __align__(256) unsigned char scratch[ev::kScratchBytes];

namespace ev {
// Device address of this GPU's scratch array (the current device's), looked up on the
// first call on that device.
static ev_status scratch_pointer(void **out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kScratchDevices) return EV_ERR_SCRATCH;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void *ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return EV_ERR_SCRATCH;
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return EV_OK;
}
}  // namespace ev

EV_API ev_status ev_tree_attention(const void *q, const ev_kv_desc *kv, const int32_t *prefix_len,
                                   const uint64_t *anc_mask, int32_t B, int32_t T, int32_t Hq,
                                   int64_t max_prefix_len, float sm_scale, void *out, float *lse,
                                   void *ws, size_t ws_bytes, int32_t *dev_status,
                                   hipStream_t stream) {
  return ev::attention_call(q, kv, prefix_len, anc_mask, B, T, Hq, max_prefix_len, sm_scale, out,
                            lse, ws, ws_bytes, dev_status, stream, false);
}

EV_API ev_status ev_tree_attention_noalloc(const void *q, const ev_kv_desc *kv,
                                           const int32_t *prefix_len, const uint64_t *anc_mask,
                                           int32_t B, int32_t T, int32_t Hq,
                                           int64_t max_prefix_len, float sm_scale, void *out,
                                           float *lse, int32_t *dev_status, hipStream_t stream) {
  void *ws = nullptr;
  const ev_status st = ev::scratch_pointer(&ws);
  if (st != EV_OK) return st;
  return ev::attention_call(q, kv, prefix_len, anc_mask, B, T, Hq, max_prefix_len, sm_scale, out,
                            lse, ws, ev::kScratchBytes, dev_status, stream, true);
}

EV_API size_t ev_tree_attention_noalloc_limit(void) { return ev::kScratchBytes; }

EV_API ev_status ev_tree_mask_attention(const void *q, const ev_kv_desc *kv,
                                        const int32_t *prefix_len, const int32_t *parent,
                                        uint64_t *anc_mask, int32_t *depth, int32_t B, int32_t T,
                                        int32_t Hq, int64_t max_prefix_len, float sm_scale,
                                        void *out, float *lse, void *ws, size_t ws_bytes,
                                        int32_t *dev_status, hipStream_t stream) {
  if (!parent) return EV_ERR_NULL;
  return ev::attention_call(q, kv, prefix_len, nullptr, B, T, Hq, max_prefix_len, sm_scale, out,
                            lse, ws, ws_bytes, dev_status, stream, false, parent, anc_mask, depth);
}

