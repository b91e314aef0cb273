// Tree acceptance: greedy longest match and distribution-preserving rejection sampling.
//
// [EX] "Core idea": the target verifies every branch and keeps the longest accepted
// prefix; [SN] case 1: k accepted drafts emit k + 1 tokens; [EX] "Why it works" and [SN]
// case 3: drafts are accepted or rejected-and-resampled so that the emitted tokens follow
// the target's own distribution.  Drafts are point masses (the draft head takes an argmax,
// [TR] sec. 2), so at node a with residual mass Z a child drafting x is accepted iff
// u * Z < p_a(x); a rejected token leaves the residual (Z -= p_a(x)); when every child
// fails, the emitted token is an inverse-CDF draw from the residual.
//
// The walk is sequential, but the outcome at a node depends only on that node's logit
// row, its children's draft tokens and their uniforms — not on how the walk got there.  So
// everything happens in ONE launch over (row = node, 1024-logit chunk) wavefronts:
//   * each wavefront streams its chunk of float32 logits once and stores the chunk's
//     statistics — greedy: (max, lowest argmax); rejection: float64 (M_c = max s,
//     S_c = sum exp(s - M_c)), s = logit/tau;
//   * the workgroup that completes a row's last chunk (a device-scope counter per row)
//     reduces the row and settles that node's outcome: its argmax / accepted child,
//     residual mass, rejected children and their probabilities;
//   * the workgroup that completes a sequence's last row (a counter per sequence) follows
//     accepted children from the root and draws the bonus token at the last node (greedy:
//     its argmax; rejection: the residual inverse CDF, located through the chunk masses,
//     then one 1024-logit chunk scanned in float64).
// The counters live in the caller's workspace, which must be zero-filled before its first
// use; every call leaves them at zero again.
#include "ev_internal.h"
#include "rowstream.h"

#include <limits.h>
#include <algorithm>
#include <type_traits>
#include <math.h>

namespace ev {

// Compaction of the accepted path in the acceptance launch (the *_compact entry points):
// the cache (ev_kv_desc as KvAddr plus the raw pointers), its row size and layers.
struct CompactSeq {
  char *k;
  char *v;
  float *k_scale;                        // INT4 caches: one scale per row, moved with it
  float *v_scale;
  KvAddr kv;
  int row_bytes;                         // bytes of one (slot, KV head) row
  int64_t layer_rows;                    // rows from one layer to the next
  int n_layers;
  const int32_t *prefix_len;
  int32_t *new_len;
};

struct AcceptArgs {
  const float *logits;
  const int32_t *tokens;
  const int32_t *parent;
  int B, T, V, n_chunks;
  double inv_tau;
  const double *uniforms;
  void *stats;                           // [B*T][n_chunks] chunk statistics
  int32_t *row_cnt;                      // [B*T] arrivals per row
  int32_t *seq_cnt;                      // [B] settled rows per sequence
  uint64_t *node_out;                    // [B*T] (accepted child | bonus token << 32)
  int32_t *accept_len;
  int32_t *path;
  int32_t *out_tokens;
  int32_t *dev_status;
  CompactSeq cmp;                        // used by the compacting kernels only
};

__device__ inline uint64_t pack_node(int next, int bonus) {
  return (uint64_t)(uint32_t)next | ((uint64_t)(uint32_t)bonus << 32);
}

// Inverse-CDF draw from the residual of a node, t = u0 * Z (one wavefront).  Rejected
// tokens: lanes set in `rej` hold them in `tok` and their probabilities in `prej`.  The
// chunk whose cumulative residual mass first exceeds t is found from the chunk statistics
// (cs, strided as in row_stats_regs); that chunk is then scanned element by element.
// Values of one lane at a wave-uniform index are read with readlane (a scalar-register
// move), not a shuffle (an LDS round trip each); the settle and walk are chains of them.
__device__ int residual_draw(const float *row, int V, int nc, double inv_tau,
                             const RejStat (&cs)[kChunkRegs], double M, double S,
                             uint64_t rej, int tok, double prej, double t, const double *tab) {
  const int lane = threadIdx.x & 63;
  const double inv_S = 1.0 / S;
  double mass[kChunkRegs], xm[kChunkRegs], em[kChunkRegs];
#pragma unroll
  for (int r = 0; r < kChunkRegs; ++r) xm[r] = cs[r].M - M;
  exp_nonpos_n(xm, em, tab);
#pragma unroll
  for (int r = 0; r < kChunkRegs; ++r) mass[r] = cs[r].S > 0.0 ? cs[r].S * em[r] * inv_S : 0.0;
  for (uint64_t rr = rej; rr; rr &= rr - 1) {
    const int src = __ffsll((unsigned long long)rr) - 1;
    const int x = lane_i(tok, src);
    const double px = lane_d(prej, src);
#pragma unroll
    for (int r = 0; r < kChunkRegs; ++r)
      if (lane + 64 * r == x / kChunk) mass[r] -= px;
  }
  int cstar = -1;
  double cbefore = -INFINITY, base = 0.0;
#pragma unroll
  for (int r = 0; r < kChunkRegs; ++r) {
    if (cstar < 0 && 64 * r < nc) {
      const double incl = wave_inclusive_sum(mass[r]);
      const uint64_t hit = __ballot(lane + 64 * r < nc && base + incl > t);
      if (hit) {
        const int hl = __ffsll((unsigned long long)hit) - 1;
        cstar = hl + 64 * r;
        cbefore = base + lane_d(incl - mass[r], hl);
      }
      base += lane_d(incl, 63);
    }
  }
  if (cstar < 0) cstar = nc - 1;          // rounding left t beyond the total: last chunk
  for (;;) {
    const int y0 = cstar * kChunk + lane * 16;   // lane scans 16 consecutive ids
    double pv[16];
    float lv[16];
#pragma unroll
    for (int e = 0; e < 16; ++e) lv[e] = row[min(y0 + e, V - 1)];
    // table reads in batches of 4, each batch issued before any of it is used (a larger
    // batch raised the kernel's register count and cost the logit stream occupancy)
#pragma unroll
    for (int h = 0; h < 16; h += 4) {
      ExpParts ep[4];
      double tj[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) ep[e] = exp_split(shifted(lv[h + e], inv_tau, M));
#pragma unroll
      for (int e = 0; e < 4; ++e) tj[e] = tab[exp_slot(ep[e].k)];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const double pe = exp_join(ep[e], tj[e]) * inv_S;
        pv[h + e] = y0 + h + e < V ? pe : 0.0;
      }
    }
    for (uint64_t rr = rej; rr; rr &= rr - 1) {
      const int x = lane_i(tok, __ffsll((unsigned long long)rr) - 1);
#pragma unroll
      for (int e = 0; e < 16; ++e)
        if (y0 + e == x) pv[e] = 0.0;
    }
    double lsum = 0.0;
#pragma unroll
    for (int e = 0; e < 16; ++e) lsum += pv[e];
    const double li = wave_inclusive_sum(lsum);
    double C = cbefore + (li - lsum);
    int first = -1, last = -1;
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      C += pv[e];
      if (first < 0 && pv[e] > 0.0 && C > t) first = y0 + e;
      if (pv[e] > 0.0) last = y0 + e;
    }
    const uint64_t fh = __ballot(first >= 0);
    if (fh) return lane_i(first, __ffsll((unsigned long long)fh) - 1);
    // no crossing (rounding at a chunk edge or beyond the total): largest positive id
    const uint64_t lh = __ballot(last >= 0);
    if (lh) return lane_i(last, 63 - __clzll((long long)lh));
    if (cstar == 0) return 0;
    --cstar;                             // empty chunk (all rejected / underflow): go down
    cbefore = -INFINITY;
  }
}

struct WsLayout {
  size_t row_cnt, seq_cnt, stats, node_out, total;
};

inline WsLayout ws_layout(int B, int T, int V) {
  WsLayout w;
  const size_t rows = (size_t)B * T;
  w.row_cnt = 0;
  w.seq_cnt = kCounterBytes / 2;
  w.stats = kCounterBytes;
  w.node_out = w.stats + align_up(rows * n_chunks_of(V) * sizeof(RejStat), 256);
  w.total = w.node_out + align_up(rows * sizeof(uint64_t), 256);
  return w;
}

// Outcome of node n of sequence b (one wavefront; lane i holds parent, token and uniform
// of node i): greedy — the row's lowest argmax y, the lowest-index child drafting y, and y
// as the bonus; rejection — the tests of its children in ascending index, and, when none
// is accepted, the bonus drawn from the residual.  The bonus is only used if the walk
// ends here, but it depends on nothing else, so every row draws its own in parallel.
template <bool REJ>
__device__ void settle_node(const AcceptArgs &a, int b, int n, int par, int tok, double ul,
                            const double *tab) {
  const int lane = threadIdx.x & 63;
  const int T = a.T, nc = a.n_chunks;
  const int64_t row_id = (int64_t)b * T + n;
  const bool live = lane < T;
  const bool pok = !live || (lane == 0 ? par == -1 : (par >= 0 && par < lane));
  int next = -2, bonus = 0;              // -2: invalid tree, the sequence is skipped
  if (__any(!pok)) {
    if (lane == 0) report(a.dev_status, EV_DERR_PARENT);
  } else if (__any(live && lane > 0 && (tok < 0 || tok >= a.V))) {
    if (lane == 0) report(a.dev_status, EV_DERR_TOKEN);
  } else {
    const uint64_t kids = __ballot(live && par == n);
    if (!REJ) {
      const uint64_t *st = (const uint64_t *)a.stats + row_id * nc;
      float v = -INFINITY;
      int i = INT_MAX;
      for (int c = lane; c < nc; c += 64) {
        const GreedyStat g = unpack(observe(&st[c]));
        better(v, i, g.val, g.idx);
      }
      wave_argmax(v, i);
      const uint64_t match = kids & __ballot(live && tok == i);
      next = match ? __ffsll((unsigned long long)match) - 1 : -1;
      bonus = i;
    } else {
      const RejStat *st = (const RejStat *)a.stats + row_id * nc;
      const float *row = a.logits + row_id * a.V;
      RejStat cs[kChunkRegs];
#pragma unroll
      for (int r = 0; r < kChunkRegs; ++r) {
        const int c = lane + 64 * r;
        cs[r] = c < nc ? RejStat{observe(&st[c].M), observe(&st[c].S)} : RejStat{-INFINITY, 0.0};
      }
      const float lg = ((kids >> lane) & 1) ? row[tok] : 0.f;
      double M, S;
      row_stats_regs(cs, tab, M, S);
      const double inv_S = 1.0 / S;
      // every child's target probability at once, in its own lane (in the loop below, one
      // exp per child, each waiting for its table read, made wide nodes the slowest rows)
      const double pk = exp_nonpos(shifted(lg, a.inv_tau, M), tab) * inv_S;
      double Z = 1.0, myp = 0.0;
      uint64_t rej = 0;
      next = -1;
      for (uint64_t kk = kids; kk; kk &= kk - 1) {
        const int c = __ffsll((unsigned long long)kk) - 1;
        const int x = lane_i(tok, c);
        if (__ballot(((rej >> lane) & 1) && tok == x)) continue;   // already rejected here
        const double p = lane_d(pk, c);
        if (lane_d(ul, c) * Z < p) {
          next = c;
          break;
        }
        rej |= 1ull << c;
        if (lane == c) myp = p;
        Z -= p;
      }
      bonus = next >= 0 ? -1
                        : residual_draw(row, a.V, nc, a.inv_tau, cs, M, S, rej, tok, myp,
                                        lane_d(ul, 0) * Z, tab);
    }
  }
  if (lane == 0) publish(&a.node_out[row_id], pack_node(next, bonus));
}

// Follow accepted children from the root of sequence b and emit the bonus token of the
// last node (one wavefront; lane i holds the token of node i).
// With s_path set, the path and k also go to LDS for the compaction that follows (k = -1
// for an invalid tree).
template <class Args>
__device__ void finish_sequence(const Args &a, int b, int tok, int *s_path = nullptr,
                                int *s_k = nullptr) {
  const int lane = threadIdx.x & 63;
  const int T = a.T;
  const bool live = lane < T;
  const uint64_t w = live ? observe(&a.node_out[(int64_t)b * T + lane]) : pack_node(-1, -1);
  const int next_l = (int)(uint32_t)w, bonus_l = (int)(uint32_t)(w >> 32);
  if (__any(next_l == -2)) {             // invalid tree, already reported
    if (s_k && lane == 0) *s_k = -1;
    return;
  }
  int node = 0, k = 0;
  int my_path = lane == 0 ? 0 : -1;      // lane m holds path[m]
  int my_out = -1;                       // lane m holds out_tokens[m]
  for (;;) {
    const int nxt = lane_i(next_l, node);
    if (nxt < 0) break;
    const int drafted = lane_i(tok, nxt);
    if (lane == k) my_out = drafted;
    ++k;
    if (lane == k) my_path = nxt;
    node = nxt;
  }
  const int bonus = lane_i(bonus_l, node);
  if (lane == k) my_out = bonus;
  if (live) {
    a.path[(int64_t)b * T + lane] = my_path;
    a.out_tokens[(int64_t)b * T + lane] = my_out;
  }
  if (lane == 0) a.accept_len[b] = k;
  if (s_path) {
    if (live) s_path[lane] = my_path;
    if (lane == 0) *s_k = k;
  }
}

// Row index (within layer 0) of logical slot `slot` of sequence b, KV head g; a paged
// cache's block ids come from s_blk, which holds those of blocks blk0, blk0 + 1, ...
__device__ inline int64_t slot_row(const CompactSeq &c, const int *s_blk, int blk0, int b, int g,
                                   int slot) {
  if (!c.kv.paged) return (int64_t)(b * c.kv.hkv + g) * c.kv.cap + slot;
  const int blk = s_blk[(slot >> c.kv.block_shift) - blk0];
  return (((int64_t)blk * c.kv.hkv + g) << c.kv.block_shift) | (slot & ((1 << c.kv.block_shift) - 1));
}

// Whether the slots of sequence b's tree, [L, L + T), fall outside the cache; for a paged
// cache thread t also loads the id of the tree's t-th block into s_blk (every source and
// destination slot of the compaction lies in that range).  Run by the wavefronts that do
// not walk, while the walk runs.
__device__ inline bool tree_slots_bad(const CompactSeq &c, int b, int T, int L, int t,
                                      int *s_blk) {
  if (L < 0 || !c.kv.fits(L + T)) return t == 0;
  if (!c.kv.paged) return false;
  const int blk0 = L >> c.kv.block_shift;
  if (blk0 + t > (L + T - 1) >> c.kv.block_shift) return false;
  const int blk = c.kv.table[(int64_t)b * c.kv.max_blocks + blk0 + t];
  s_blk[t] = blk;
  return blk < 0 || blk >= c.kv.n_blocks;
}

// Accepted-path KV compaction of sequence b ([TR] sec. 2: keep the accepted branch's KV)
// by the whole workgroup, as ev_kv_compact does it: slot L + path[m] moves to slot L + m,
// m = 1 .. k, in every layer, KV head, K and V.  The moves go in rounds of up to 4 x 256
// 16-byte pieces, ordered by m; a round reads all its pieces into registers before it
// writes any, since a destination L + m can be the source of an earlier move of the same
// round (path[m'] = m, m' < m).  It is never the source of a later round: path[m'] >= m'
// for every move, so later sources lie above every destination written before them.
// `bad`: the tree's slots [L, L + T) are not all in the cache (tree_slots_bad).
__device__ void compact_sequence(const CompactSeq &c, int b, int T, int L, int k, bool bad,
                                 const int *s_path, const int *s_blk, int32_t *dev_status) {
  if (k < 0) return;                     // invalid tree, already reported
  const int tid = threadIdx.x;
  const int blk0 = c.kv.paged ? L >> c.kv.block_shift : 0;
  if (bad) {
    if (tid == 0) report(dev_status, EV_DERR_BOUNDS);
    return;
  }
  if (tid == 0) c.new_len[b] = L + k + 1;
  const int cpr = c.row_bytes / 16;      // 16-byte pieces per row: 2 .. 32
  const int cshift = __ffs(cpr) - 1;
  const int hk2 = c.kv.hkv * 2;
  const int per_move = c.n_layers * hk2;
  const int n_pieces = k * per_move * cpr;
  constexpr int R = 4;
  for (int base = 0; base < n_pieces; base += R * 256) {
    u32x4 val[R];
    float sc[R];
    int64_t dst[R];
#pragma unroll
    for (int i = 0; i < R; ++i) {
      const int idx = base + tid + 256 * i;
      dst[i] = -1;
      if (idx < n_pieces) {
        const int row = idx >> cshift, ch = idx & (cpr - 1);
        const int m = 1 + row / per_move, r2 = row % per_move;
        const int l = r2 / hk2, g = (r2 % hk2) >> 1, which = r2 & 1;
        const int64_t lrow = (int64_t)l * c.layer_rows;
        const int64_t src = lrow + slot_row(c, s_blk, blk0, b, g, L + s_path[m]);
        const int64_t dr = lrow + slot_row(c, s_blk, blk0, b, g, L + m);
        const char *basep = which ? c.v : c.k;
        val[i] = *(const u32x4 *)(basep + src * c.row_bytes + ch * 16);
        const float *scales = which ? c.v_scale : c.k_scale;
        sc[i] = scales && ch == 0 ? scales[src] : 0.f;
        dst[i] = dr * cpr + ch + ((int64_t)which << 60);   // destination piece, K or V
      }
    }
    __syncthreads();                     // every piece of the round read
#pragma unroll
    for (int i = 0; i < R; ++i) {
      if (dst[i] < 0) continue;
      const int which = (int)(dst[i] >> 60);
      const int64_t piece = dst[i] & (((int64_t)1 << 60) - 1);
      const int64_t dr = piece >> cshift;
      const int ch = (int)(piece & (cpr - 1));
      char *basep = which ? c.v : c.k;
      *(u32x4 *)(basep + dr * c.row_bytes + ch * 16) = val[i];
      float *scales = which ? c.v_scale : c.k_scale;
      if (scales && ch == 0) scales[dr] = sc[i];
    }
  }
}

// Statistics of one 1024-logit chunk (already in registers), the same in every lane:
// greedy, the (max, lowest argmax) word; rejection, float64 (M_c = max s, S_c = sum exp(s - M_c)).
template <bool REJ>
using ChunkStat = typename std::conditional<REJ, RejStat, uint64_t>::type;

template <bool REJ, int XB>
__device__ __forceinline__ ChunkStat<REJ> chunk_stats(const AcceptArgs &a, int chunk,
                                                      const float (&v)[16], const double *tab) {
  const int lane = threadIdx.x & 63;
  if constexpr (!REJ) {
    // a lane visits its ids in increasing order, so a strict > keeps the lowest index; it
    // starts from its first id when that lies in the row, so a row of -inf logits still
    // yields its lowest id (0), as the argmax definition does
    float best = -INFINITY;
    const int first = chunk * kChunk + lane * 4;
    int bi = first < a.V ? first : INT_MAX;
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const bool gt = v[e] > best;
      best = gt ? v[e] : best;
      bi = gt ? chunk * kChunk + ((e >> 2) * 64 + lane) * 4 + (e & 3) : bi;
    }
    wave_argmax(best, bi);
    return pack(GreedyStat{best, bi});
  } else {
    float best = -INFINITY;
#pragma unroll
    for (int e = 0; e < 16; ++e) best = fmaxf(best, v[e]);
    const double M = (double)wave_max_f(best) * a.inv_tau;
    // Padding past V holds -inf: its term is clamped to at most 5e-324, which vanishes
    // next to the chunk's own maximum term (1), so no per-element test is needed.
    const double sum = exp_sum<16, XB>([&](int e) { return shifted(v[e], a.inv_tau, M); }, tab);
    return RejStat{M, wave_sum(sum)};
  }
}

__device__ inline void publish_stat(const AcceptArgs &a, int64_t row, int chunk, uint64_t st) {
  publish((uint64_t *)a.stats + row * a.n_chunks + chunk, st);
}
__device__ inline void publish_stat(const AcceptArgs &a, int64_t row, int chunk, RejStat st) {
  RejStat *dst = (RejStat *)a.stats + row * a.n_chunks + chunk;
  publish(&dst->M, st.M);
  publish(&dst->S, st.S);
}

// grid (chunk groups, rows); a workgroup's four wavefronts stream CPW chunks each, the
// wavefronts of a workgroup interleaved chunk by chunk, with the next chunk's loads in
// flight while the current one is reduced.
// COMPACT: the workgroup that walks a sequence then compacts its accepted path's KV.
template <bool REJ, int CPW, bool VEC, bool COMPACT>
__global__ __launch_bounds__(256) void accept_kernel(AcceptArgs a) {
  __shared__ double tab[kExpTab];
  __shared__ int s_last;
  __shared__ int s_path[COMPACT ? kMaxNodes : 1];
  __shared__ int s_blk[COMPACT ? kMaxNodes + 1 : 1];
  __shared__ int s_k;
  __shared__ int s_bad;
  args_in_sgprs(a.n_chunks, a.T, a.V, a.logits, a.parent, a.tokens, a.uniforms, a.inv_tau,
                a.stats, a.row_cnt);
  if (COMPACT && threadIdx.x == 0) s_bad = 0;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int64_t row = blockIdx.y;
  const int nc = a.n_chunks;
  const int b = (int)row / a.T, n = (int)row % a.T;   // row < 2^31

  // ---- this wavefront's chunk statistics ----
  const float *lrow = a.logits + row * a.V;
  // the wavefront's first chunk, uniform across its lanes (so are the branches below)
  const int c0 = __builtin_amdgcn_readfirstlane(blockIdx.x * kChunksPerWG * CPW + wave);
  float v[2][16];
  int idx_unused[16];
  // Non-temporal loads with one or two chunks per wavefront, cached loads with four
  // (measured against cached loads: 64 rows x 128256 logits, two chunks, 18.4 -> 17.5 us;
  // 26 rows x 32000, one chunk, 6.47 -> 6.28 us; 256 rows x 128256, four chunks, 39.5 ->
  // 41.0 us).
  constexpr bool kNT = CPW <= 2;
  // Every wavefront issues all CPW chunk loads, each while the chunk before it is being
  // reduced, and publishes its statistics only at the end: a load or store under a branch,
  // or a store between the loads, made the compiler wait for the chunk still in flight.
  // A chunk past the row's end (last workgroup of a row) loads the row's last chunk and is
  // not reduced.  With one chunk per wavefront its loads go out before the exp table is
  // filled (26 rows x 32000: 6.38 -> 5.98 us); with two or four they go out after the
  // barrier (issued before it, 64 rows x 128256 took 16.15 -> 16.48 us, same-box pairs).
  ChunkStat<REJ> st[CPW];
  // exp table reads issued 8 (four chunks per wavefront: 4) at a time; 8 with four chunks
  // took the kernel past the register count that keeps six wavefronts per SIMD
  constexpr int kExpBatch = CPW == 4 ? 4 : 8;
  if constexpr (CPW == 1) load_chunk_raw<kNT, VEC>(lrow, a.V, min(c0, nc - 1) * kChunk, v[0]);

  if (REJ) fill_exp_table(tab);
  // The tree of this sequence, for the settle and walk steps below (loaded up front so
  // that its latency hides behind the logit stream).
  int par = -2, tok = -1;
  double ul = 0.0;
  if (wave == 0 && lane < a.T) {
    par = a.parent[(int64_t)b * a.T + lane];
    tok = a.tokens[(int64_t)b * a.T + lane];
    if (REJ) ul = a.uniforms[(int64_t)b * a.T + lane];
  }
  lds_barrier();                          // the exp table
  if constexpr (CPW != 1) load_chunk_raw<kNT, VEC>(lrow, a.V, min(c0, nc - 1) * kChunk, v[0]);
#pragma unroll
  for (int m = 0; m < CPW; ++m) {
    const int c = c0 + kChunksPerWG * m;
    if (m + 1 < CPW)
      load_chunk_raw<kNT, VEC>(lrow, a.V, min(c + kChunksPerWG, nc - 1) * kChunk, v[(m + 1) & 1]);
    if (c < nc) {
      mask_chunk(a.V, c * kChunk, v[m & 1], idx_unused);
      st[m] = chunk_stats<REJ, kExpBatch>(a, c, v[m & 1], tab);
    }
  }
  if (lane == 0) {
#pragma unroll
    for (int m = 0; m < CPW; ++m)
      if (c0 + kChunksPerWG * m < nc) publish_stat(a, row, c0 + kChunksPerWG * m, st[m]);
  }
  if (!last_arrival(&a.row_cnt[counter_slot(row)], gridDim.x, &s_last)) return;

  // ---- last workgroup of this row: settle the node ----
  if (wave == 0) settle_node<REJ>(a, b, n, par, tok, ul, tab);
  if (!last_arrival(&a.seq_cnt[counter_slot(b)], a.T, &s_last)) return;

  // ---- last row of this sequence: walk (and compaction) ----
  if constexpr (COMPACT) {
    const int L = scalar_load(a.cmp.prefix_len, b);
    if (wave == 0) {
      finish_sequence(a, b, tok, s_path, &s_k);
    } else if (tree_slots_bad(a.cmp, b, a.T, L, (int)threadIdx.x - 64, s_blk)) {
      s_bad = 1;
    }
    __syncthreads();
    compact_sequence(a.cmp, b, a.T, L, s_k, s_bad != 0, s_path, s_blk, a.dev_status);
  } else if (wave == 0) {
    finish_sequence(a, b, tok);
  }
}

static ev_status check_common(const float *logits, const int32_t *tokens, const int32_t *parent,
                              int32_t B, int32_t T, int32_t V, int32_t *accept_len,
                              int32_t *path, int32_t *out_tokens, void *ws, size_t ws_bytes) {
  if (B < 0 || T < 1 || T > kMaxNodes || V < 1 || V > 64 * kChunkRegs * kChunk) return EV_ERR_SHAPE;
  if ((int64_t)B * T > kMaxRows) return EV_ERR_SHAPE;
  if (B == 0) return EV_OK;
  if (!logits || !tokens || !parent || !accept_len || !path || !out_tokens) return EV_ERR_NULL;
  if (ws_bytes < ws_layout(B, T, V).total || !ws) return EV_ERR_WORKSPACE;
  return EV_OK;
}

static ev_status launch_accept(bool rej, const float *logits, const int32_t *tokens,
                               const int32_t *parent, int32_t B, int32_t T, int32_t V,
                               double inv_tau, const double *uniforms, int32_t *accept_len,
                               int32_t *path, int32_t *out_tokens, void *ws,
                               int32_t *dev_status, hipStream_t stream,
                               const CompactSeq *cmp = nullptr) {
  const WsLayout w = ws_layout(B, T, V);
  char *base = (char *)ws;
  AcceptArgs a{logits, tokens, parent, B, T, V, n_chunks_of(V), inv_tau, uniforms,
               base + w.stats, (int32_t *)(base + w.row_cnt), (int32_t *)(base + w.seq_cnt),
               (uint64_t *)(base + w.node_out), accept_len, path, out_tokens, dev_status, {}};
  if (cmp) a.cmp = *cmp;
  // Chunks per wavefront: as many as keep at least 1024 workgroups in the grid (four per
  // CU), so that the streams run with the next chunk's loads in flight behind the reduction
  // while every workgroup stays resident at once.
  const int64_t rows = (int64_t)B * T;
  int cpw = 4;
  while (cpw > 1 && rows * ((a.n_chunks + kChunksPerWG * cpw - 1) / (kChunksPerWG * cpw)) < 1024)
    cpw /= 2;
  dim3 grid((a.n_chunks + kChunksPerWG * cpw - 1) / (kChunksPerWG * cpw), (unsigned)rows);
  const bool vec = (V & 3) == 0;          // rows start 16-byte aligned
#define EV_LAUNCH_ACCEPT(R, C)                                                                \
  do {                                                                                        \
    if (cmp) {                                                                                \
      if (vec) hipLaunchKernelGGL((accept_kernel<R, C, true, true>), grid, dim3(256), 0, stream, a); \
      else hipLaunchKernelGGL((accept_kernel<R, C, false, true>), grid, dim3(256), 0, stream, a); \
    } else {                                                                                  \
      if (vec) hipLaunchKernelGGL((accept_kernel<R, C, true, false>), grid, dim3(256), 0, stream, a); \
      else hipLaunchKernelGGL((accept_kernel<R, C, false, false>), grid, dim3(256), 0, stream, a); \
    }                                                                                         \
  } while (0)
  if (rej) {
    if (cpw == 4) EV_LAUNCH_ACCEPT(true, 4);
    else if (cpw == 2) EV_LAUNCH_ACCEPT(true, 2);
    else EV_LAUNCH_ACCEPT(true, 1);
  } else {
    if (cpw == 4) EV_LAUNCH_ACCEPT(false, 4);
    else if (cpw == 2) EV_LAUNCH_ACCEPT(false, 2);
    else EV_LAUNCH_ACCEPT(false, 1);
  }
#undef EV_LAUNCH_ACCEPT
  return launch_status();
}

// ---------------------------------------------------------------------------------------
// Acceptance with drafts sampled from a draft distribution q (one per node, from its own
// logit row at its own temperature).  At a node the children are tested in ascending
// index against the residual r = W / Z, W(y) = max(0, p(y) - s q(y)), Z = sum W: a child
// drafting x is accepted iff u * q(x) * Z < W(x); a rejection grows s by Z.  When no
// child is accepted the bonus token is drawn from W.  Z changes with every rejection, so
// each rejection needs one more pass over the node's row: the work runs in rounds, one
// launch per round, every launch one pass over the rows still being decided (a row
// whose node is settled returns at once).  The statistics launch already takes each
// node's first decision: with s = 0 the residual is p itself, whose mass per chunk
// follows from the chunk statistics, so leaves draw their bonus and first children are
// tested there.  A node with c children is therefore settled by round c, and the
// caller's bound on children per node fixes the number of launches.
struct SampledRow {
  double Mp, Sp, Mq, Sq;                 // row statistics of the target and draft rows
  double s;                              // residual shift after the rejections so far
  int32_t active;                        // still being decided
  int32_t tried;                         // children tested so far
};

// A row still undecided after a round, with its state: the next round's work list.
struct SampledEntry {
  SampledRow st;
  int64_t row;
  int64_t pad;
};
static_assert(sizeof(SampledEntry) == 64, "one list entry per 64 bytes");
constexpr int kMaxLaunches = kMaxNodes + 1;   // the statistics launch and up to T rounds

struct SampledArgs {
  const float *logits;
  const float *draft;
  const int32_t *tokens;
  const int32_t *parent;
  int B, T, V, n_chunks, max_children;
  double inv_tau, inv_tau_q;
  const double *uniforms;
  RejStat *pstat;                        // [B*T][n_chunks]
  RejStat *qstat;                        // [B*T][n_chunks]
  double *wpart;                         // [B*T][n_chunks] residual mass per chunk, current pass
  SampledRow *state;                     // [B*T]
  int32_t *row_cnt;
  int32_t *seq_cnt;
  uint64_t *node_out;
  int32_t *accept_len;
  int32_t *path;
  int32_t *out_tokens;
  int32_t *dev_status;
  SampledEntry *list[2];                 // rows still undecided after round r: list[r & 1]
  int32_t *list_cnt;                     // [kMaxLaunches] their number, per round
  int round;                             // 0: the statistics launch
  int reset_lists;                       // the statistics launch clears the list counters
};

struct SampledWs {
  size_t row_cnt, seq_cnt, pstat, qstat, wpart, state, node_out, list_cnt, list, total;
};

inline SampledWs sampled_ws_layout(int B, int T, int V) {
  SampledWs w;
  const size_t rows = (size_t)B * T, per_chunk = rows * n_chunks_of(V);
  w.row_cnt = 0;
  w.seq_cnt = kCounterBytes / 2;
  w.pstat = kCounterBytes;
  w.qstat = w.pstat + align_up(per_chunk * sizeof(RejStat), 256);
  w.wpart = w.qstat + align_up(per_chunk * sizeof(RejStat), 256);
  w.state = w.wpart + align_up(per_chunk * sizeof(double), 256);
  w.node_out = w.state + align_up(rows * sizeof(SampledRow), 256);
  w.list_cnt = w.node_out + align_up(rows * sizeof(uint64_t), 256);
  w.list = w.list_cnt + align_up(kMaxLaunches * sizeof(int32_t), 256);
  w.total = w.list + 2 * rows * sizeof(SampledEntry);
  return w;
}

// Residual weight of logit pair (target, draft) under row state st (shift s).
__device__ inline double residual_weight(float lp, float lq, const SampledArgs &a,
                                         const SampledRow &st, double inv_sp, double inv_sq,
                                         const double *tab) {
  const double p = exp_nonpos(shifted(lp, a.inv_tau, st.Mp), tab) * inv_sp;
  const double q = exp_nonpos(shifted(lq, a.inv_tau_q, st.Mq), tab) * inv_sq;
  return fmax(0.0, fma(-st.s, q, p));
}

// Bonus token of a node from its residual W: the chunk whose cumulative residual mass
// first exceeds t is found from the chunk masses (lane-strided as in row_stats_regs),
// then that chunk is scanned element by element (one wavefront).
__device__ int sampled_draw(const SampledArgs &a, int64_t row, const SampledRow &st,
                            const double (&mass)[kChunkRegs], double t, const double *tab) {
  const int lane = threadIdx.x & 63;
  const int nc = a.n_chunks;
  int cstar = -1;
  double cbefore = -INFINITY, base = 0.0;
#pragma unroll
  for (int r = 0; r < kChunkRegs; ++r) {
    if (cstar < 0 && 64 * r < nc) {
      const double incl = wave_inclusive_sum(mass[r]);
      const uint64_t hit = __ballot(lane + 64 * r < nc && base + incl > t);
      if (hit) {
        const int hl = __ffsll((unsigned long long)hit) - 1;
        cstar = hl + 64 * r;
        cbefore = base + __shfl(incl - mass[r], hl);
      }
      base += __shfl(incl, 63);
    }
  }
  if (cstar < 0) cstar = nc - 1;
  const double inv_sp = 1.0 / st.Sp, inv_sq = 1.0 / st.Sq;
  const float *lp = a.logits + row * a.V;
  const float *lq = a.draft + row * a.V;
  for (;;) {
    const int y0 = cstar * kChunk + lane * 16;
    double w[16];
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int y = min(y0 + e, a.V - 1);
      const double we = residual_weight(lp[y], lq[y], a, st, inv_sp, inv_sq, tab);
      w[e] = y0 + e < a.V ? we : 0.0;
    }
    double lsum = 0.0;
#pragma unroll
    for (int e = 0; e < 16; ++e) lsum += w[e];
    const double li = wave_inclusive_sum(lsum);
    double C = cbefore + (li - lsum);
    int first = -1, last = -1;
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      C += w[e];
      if (first < 0 && w[e] > 0.0 && C > t) first = y0 + e;
      if (w[e] > 0.0) last = y0 + e;
    }
    const uint64_t fh = __ballot(first >= 0);
    if (fh) return __shfl(first, __ffsll((unsigned long long)fh) - 1);
    const uint64_t lh = __ballot(last >= 0);
    if (lh) return __shfl(last, 63 - __clzll((long long)lh));
    if (cstar == 0) return 0;
    --cstar;
    cbefore = -INFINITY;
  }
}

// What the decision of node n needs besides the residual, loaded by wave 0 of every
// workgroup before its pass over the row so that these loads overlap the pass: lane i
// holds node i's parent and token; then the next untested child, the two logits at its
// drafted token, and the uniforms of the child test and of the bonus draw.  The token
// index is clamped for the load (the tree is validated only after the pass).
struct NodeView {
  int par, tok;                          // of node `lane`
  int c;                                 // next untested child of n, -1 if none
  float lpx, lqx;                        // target and draft logits at c's token
  double uc, u0;
};

__device__ inline NodeView node_view(const SampledArgs &a, int64_t row, int b, int n,
                                     int tried) {
  const int lane = threadIdx.x & 63;
  const bool live = lane < a.T;
  NodeView v;
  v.par = live ? a.parent[(int64_t)b * a.T + lane] : -2;
  v.tok = live ? a.tokens[(int64_t)b * a.T + lane] : -1;
  uint64_t kids = __ballot(live && v.par == n);
  for (int i = 0; i < tried; ++i) kids &= kids - 1;     // children tested already
  v.c = kids ? __ffsll((unsigned long long)kids) - 1 : -1;
  const int x = min(max(__shfl(v.tok, max(v.c, 0)), 0), a.V - 1);
  v.lpx = a.logits[row * a.V + x];
  v.lqx = a.draft[row * a.V + x];
  v.uc = a.uniforms[(int64_t)b * a.T + max(v.c, 0)];
  v.u0 = a.uniforms[(int64_t)b * a.T];
  return v;
}

// Decision of node n (row `row`) once the residual at shift st.s is known through its
// chunk masses: the next untested child is accepted or rejected, or, with no child left,
// the bonus token is drawn.  One wavefront.  Returns whether the node is settled (its
// node_out published); a rejection instead advances the row state, in state[] or (LIST)
// in the entry that lists the row for the next round.
template <bool LIST>
__device__ bool sampled_decide(const SampledArgs &a, int64_t row, const SampledRow &st,
                               const NodeView &v, const double (&mass)[kChunkRegs],
                               const double *tab) {
  const int lane = threadIdx.x & 63;
  double Z = 0.0;
#pragma unroll
  for (int r = 0; r < kChunkRegs; ++r) Z += mass[r];
  Z = wave_sum(Z);
  int next = -1, bonus = -1;
  if (v.c >= 0) {
    const double inv_sp = 1.0 / st.Sp, inv_sq = 1.0 / st.Sq;
    const double qx = exp_nonpos(shifted(v.lqx, a.inv_tau_q, st.Mq), tab) * inv_sq;
    const double wx = residual_weight(v.lpx, v.lqx, a, st, inv_sp, inv_sq, tab);
    if (!(v.uc * qx * Z < wx)) {
      if (lane == 0) {
        SampledRow nst = st;
        nst.s = st.s + Z;
        nst.tried = st.tried + 1;
        nst.active = 1;
        if constexpr (!LIST) {
          a.state[row] = nst;              // read by the next round
        } else {                           // listed for the next round
          const int i = __hip_atomic_fetch_add(&a.list_cnt[a.round], 1, __ATOMIC_RELAXED,
                                               __HIP_MEMORY_SCOPE_AGENT);
          a.list[a.round & 1][i] = SampledEntry{nst, row, 0};
        }
      }
      return false;
    }
    next = v.c;
  } else {
    bonus = sampled_draw(a, row, st, mass, v.u0 * Z, tab);
  }
  if (lane == 0) {
    if constexpr (!LIST) {
      SampledRow nst = st;
      nst.active = 0;
      a.state[row] = nst;
    }
    publish(&a.node_out[row], pack_node(next, bonus));
  }
  return true;
}

// Statistics launch: per-chunk (M, S) of both rows; the row's last workgroup validates
// the tree and sets up the row state.
template <int CPW, bool VEC>
__global__ __launch_bounds__(256) void sampled_stats_kernel(SampledArgs a) {
  constexpr int XB = 4;                  // exp table reads issued 4 at a time
  __shared__ double tab[kExpTab];
  __shared__ int s_last;
  fill_exp_table(tab);
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int64_t row = blockIdx.y;
  const int nc = a.n_chunks;
  const int b = (int)(row / a.T), n = (int)(row % a.T);
  NodeView v{};
  if (wave == 0) v = node_view(a, row, b, n, 0);
  __syncthreads();
  const float *lp = a.logits + row * a.V;
  const float *lq = a.draft + row * a.V;
  int idx_unused[16];
  const int c0 = __builtin_amdgcn_readfirstlane(blockIdx.x * kChunksPerWG * CPW + wave);
  // As in the acceptance stream: the next chunk's loads of both rows are issued before the
  // current chunk is reduced, unconditionally (a chunk past the row's end reloads the last
  // one and is not reduced), and the statistics are stored once at the end.
  float vp[2][16], vq[2][16];
  RejStat stp[CPW], stq[CPW];
  load_chunk_raw<false, VEC>(lp, a.V, min(c0, nc - 1) * kChunk, vp[0]);
  load_chunk_raw<false, VEC>(lq, a.V, min(c0, nc - 1) * kChunk, vq[0]);
  __builtin_amdgcn_sched_barrier(0);     // keep the first chunk's loads ahead of the next's
#pragma unroll
  for (int m = 0; m < CPW; ++m) {
    const int c = c0 + kChunksPerWG * m;
    if (m + 1 < CPW) {
      const int cn = min(c + kChunksPerWG, nc - 1) * kChunk;
      load_chunk_raw<false, VEC>(lp, a.V, cn, vp[(m + 1) & 1]);
      load_chunk_raw<false, VEC>(lq, a.V, cn, vq[(m + 1) & 1]);
    }
    if (c < nc) {
      float (&xp)[16] = vp[m & 1];
      float (&xq)[16] = vq[m & 1];
      mask_chunk(a.V, c * kChunk, xp, idx_unused);
      mask_chunk(a.V, c * kChunk, xq, idx_unused);
      float bp = -INFINITY, bq = -INFINITY;
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        bp = fmaxf(bp, xp[e]);
        bq = fmaxf(bq, xq[e]);
      }
      const double Mp = (double)wave_max_f(bp) * a.inv_tau;
      const double Mq = (double)wave_max_f(bq) * a.inv_tau_q;
      const double sp = exp_sum<16, XB>([&](int e) { return shifted(xp[e], a.inv_tau, Mp); }, tab);
      const double sq = exp_sum<16, XB>([&](int e) { return shifted(xq[e], a.inv_tau_q, Mq); }, tab);
      stp[m] = RejStat{Mp, wave_sum(sp)};
      stq[m] = RejStat{Mq, wave_sum(sq)};
    }
  }
  if (lane == 0) {
#pragma unroll
    for (int m = 0; m < CPW; ++m) {
      const int c = c0 + kChunksPerWG * m;
      if (c < nc) {
        publish(&a.pstat[row * nc + c].M, stp[m].M);
        publish(&a.pstat[row * nc + c].S, stp[m].S);
        publish(&a.qstat[row * nc + c].M, stq[m].M);
        publish(&a.qstat[row * nc + c].S, stq[m].S);
      }
    }
  }
  const bool row_done = last_arrival(&a.row_cnt[counter_slot(row)], gridDim.x, &s_last);
  // the rounds' list counters start at zero (no round runs before this launch ends)
  if (a.reset_lists && blockIdx.x == 0 && blockIdx.y == 0 && threadIdx.x < kMaxLaunches)
    publish(&a.list_cnt[threadIdx.x], 0);
  if (!row_done) return;
  if (wave == 0) {
    const bool live = lane < a.T;
    const int par = v.par, tok = v.tok;
    const bool pok = !live || (lane == 0 ? par == -1 : (par >= 0 && par < lane));
    bool ok = true;
    if (__any(!pok)) {
      if (lane == 0) report(a.dev_status, EV_DERR_PARENT);
      ok = false;
    } else if (__any(live && lane > 0 && (tok < 0 || tok >= a.V))) {
      if (lane == 0) report(a.dev_status, EV_DERR_TOKEN);
      ok = false;
    } else if (__popcll(__ballot(live && par == n)) > a.max_children) {
      if (lane == 0) report(a.dev_status, EV_DERR_WIDTH);
      ok = false;
    }
    if (ok) {
      // Row statistics of both rows.  Before any rejection (s = 0) the residual is p, so
      // its chunk masses follow from the chunk statistics and the first decision needs
      // no further pass over the row.
      RejStat cp[kChunkRegs], cq[kChunkRegs];
#pragma unroll
      for (int r = 0; r < kChunkRegs; ++r) {
        const int c = lane + 64 * r;
        const RejStat *sp = a.pstat + row * nc + c, *sq = a.qstat + row * nc + c;
        cp[r] = c < nc ? RejStat{observe(&sp->M), observe(&sp->S)} : RejStat{-INFINITY, 0.0};
        cq[r] = c < nc ? RejStat{observe(&sq->M), observe(&sq->S)} : RejStat{-INFINITY, 0.0};
      }
      SampledRow st{};
      row_stats_regs(cp, tab, st.Mp, st.Sp);
      row_stats_regs(cq, tab, st.Mq, st.Sq);
      const double inv_sp = 1.0 / st.Sp;
      double mass[kChunkRegs], xm[kChunkRegs], em[kChunkRegs];
#pragma unroll
      for (int r = 0; r < kChunkRegs; ++r) xm[r] = cp[r].M - st.Mp;
      exp_nonpos_n(xm, em, tab);
#pragma unroll
      for (int r = 0; r < kChunkRegs; ++r) mass[r] = cp[r].S > 0.0 ? cp[r].S * em[r] * inv_sp : 0.0;
      const bool done = sampled_decide<false>(a, row, st, v, mass, tab);
      if (lane == 0) s_last = done ? 1 : 0;
    } else if (lane == 0) {
      a.state[row] = SampledRow{};       // inactive
      publish(&a.node_out[row], pack_node(-2, 0));
      s_last = 1;                        // an invalid tree settles the row at once
    }
  }
  __syncthreads();
  if (!s_last) return;
  // the sequence is skipped by the walk (its outputs are left as they were)
  if (!last_arrival(&a.seq_cnt[counter_slot(b)], a.T, &s_last)) return;
  if (wave == 0) finish_sequence(a, b, v.tok);
}

// A round over every row (the first round, or every round when one chunk per wavefront
// covers the rows): every row still being decided takes one pass over its target and
// draft logits for the residual mass at its current shift; its last workgroup then
// decides.  Rows settled earlier return at once.
template <int CPW, bool LIST>
__global__ __launch_bounds__(256) void sampled_round_kernel(SampledArgs a) {
  __shared__ double tab[kExpTab];
  __shared__ int s_last;
  const int64_t row = blockIdx.y;
  const SampledRow st = a.state[row];    // written by an earlier launch
  if (!st.active) return;                // settled: no workgroup of this row arrives
  fill_exp_table(tab);
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int nc = a.n_chunks;
  const int b = (int)(row / a.T), n = (int)(row % a.T);
  NodeView v{};
  if (wave == 0) v = node_view(a, row, b, n, st.tried);
  __syncthreads();
  const float *lp = a.logits + row * a.V;
  const float *lq = a.draft + row * a.V;
  const bool vec_ok = (a.V & 3) == 0;
  const double inv_sp = 1.0 / st.Sp, inv_sq = 1.0 / st.Sq;
  int idx_unused[16];
  const int c0 = __builtin_amdgcn_readfirstlane(blockIdx.x * kChunksPerWG * CPW + wave);
#pragma unroll
  for (int m = 0; m < CPW; ++m) {
    const int c = c0 + kChunksPerWG * m;
    if (c >= nc) continue;
    float vp[16], vq[16];
    load_pair(lp, lq, a.V, c * kChunk, vec_ok, vp, vq, idx_unused);
    double w = 0.0;
#pragma unroll
    for (int e = 0; e < 16; ++e) w += residual_weight(vp[e], vq[e], a, st, inv_sp, inv_sq, tab);
    w = wave_sum(w);
    if (lane == 0) publish(&a.wpart[row * nc + c], w);
  }
  if (!last_arrival(&a.row_cnt[counter_slot(row)], gridDim.x, &s_last)) return;
  if (wave == 0) {
    double mass[kChunkRegs];
#pragma unroll
    for (int r = 0; r < kChunkRegs; ++r) {
      const int c = lane + 64 * r;
      mass[r] = c < nc ? observe(&a.wpart[row * nc + c]) : 0.0;
    }
    const bool done = sampled_decide<LIST>(a, row, st, v, mass, tab);
    if (lane == 0) s_last = done ? 1 : 0;
  }
  __syncthreads();
  if (!s_last) return;
  if (!last_arrival(&a.seq_cnt[counter_slot(b)], a.T, &s_last)) return;
  if (wave == 0) finish_sequence(a, b, v.tok);
}

// Later rounds: work item (i, j) is chunk group j of the i-th row listed by the round
// before (one chunk per wavefront), and a fixed grid strides over the items.  A round with
// few rows spreads each of them over many workgroups, and an empty round costs one load.
// The list's count and a workgroup's first entry are loaded together.
__global__ __launch_bounds__(256) void sampled_list_round_kernel(SampledArgs a) {
  __shared__ double tab[kExpTab];
  __shared__ int s_last;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const SampledEntry *list = a.list[(a.round - 1) & 1];
  const int nc = a.n_chunks;
  const int gpr = (nc + kChunksPerWG - 1) / kChunksPerWG;
  const int64_t rows = (int64_t)a.B * a.T;
  const int64_t i0 = min((int64_t)blockIdx.x / gpr, rows - 1);
  SampledEntry e = list[i0];             // speculative: valid if i0 < the count
  const int64_t n_items = (int64_t)observe(&a.list_cnt[a.round - 1]) * gpr;
  if ((int64_t)blockIdx.x >= n_items) return;
  fill_exp_table(tab);
  const bool vec_ok = (a.V & 3) == 0;
  for (int64_t it = blockIdx.x; it < n_items; it += gridDim.x) {
    const int64_t i = it / gpr;
    if (i != i0) e = list[i];
    const int c = (int)(it % gpr) * kChunksPerWG + wave;
    const int64_t row = e.row;
    const SampledRow st = e.st;
    const int b = (int)(row / a.T), n = (int)(row % a.T);
    NodeView v{};
    if (wave == 0) v = node_view(a, row, b, n, st.tried);
    __syncthreads();                     // the exp table; the previous item's LDS flag read
    if (c < nc) {
      const float *lp = a.logits + row * a.V;
      const float *lq = a.draft + row * a.V;
      const double inv_sp = 1.0 / st.Sp, inv_sq = 1.0 / st.Sq;
      int idx_unused[16];
      float vp[16], vq[16];
      load_pair(lp, lq, a.V, c * kChunk, vec_ok, vp, vq, idx_unused);
      double w = 0.0;
#pragma unroll
      for (int k = 0; k < 16; ++k) w += residual_weight(vp[k], vq[k], a, st, inv_sp, inv_sq, tab);
      w = wave_sum(w);
      if (lane == 0) publish(&a.wpart[row * nc + c], w);
    }
    if (!last_arrival(&a.row_cnt[counter_slot(row)], gpr, &s_last)) continue;
    if (wave == 0) {
      double mass[kChunkRegs];
#pragma unroll
      for (int r = 0; r < kChunkRegs; ++r) {
        const int cc = lane + 64 * r;
        mass[r] = cc < nc ? observe(&a.wpart[row * nc + cc]) : 0.0;
      }
      const bool done = sampled_decide<true>(a, row, st, v, mass, tab);
      if (lane == 0) s_last = done ? 1 : 0;
    }
    __syncthreads();
    if (!s_last) continue;
    if (!last_arrival(&a.seq_cnt[counter_slot(b)], a.T, &s_last)) continue;
    if (wave == 0) finish_sequence(a, b, v.tok);
  }
}

// Workgroups of a later round's launch (at most).
constexpr int kRoundGrid = 1024;

static ev_status launch_sampled(const float *logits, const float *draft, const int32_t *tokens,
                                const int32_t *parent, int32_t B, int32_t T, int32_t V,
                                double inv_tau, double inv_tau_q, const double *uniforms,
                                int32_t max_children, int32_t *accept_len, int32_t *path,
                                int32_t *out_tokens, void *ws, int32_t *dev_status,
                                hipStream_t stream) {
  const SampledWs w = sampled_ws_layout(B, T, V);
  char *base = (char *)ws;
  SampledArgs a{logits, draft, tokens, parent, B, T, V, n_chunks_of(V), max_children, inv_tau,
                inv_tau_q, uniforms, (RejStat *)(base + w.pstat), (RejStat *)(base + w.qstat),
                (double *)(base + w.wpart), (SampledRow *)(base + w.state),
                (int32_t *)(base + w.row_cnt), (int32_t *)(base + w.seq_cnt),
                (uint64_t *)(base + w.node_out), accept_len, path, out_tokens, dev_status,
                {(SampledEntry *)(base + w.list), (SampledEntry *)(base + w.list) + (int64_t)B * T},
                (int32_t *)(base + w.list_cnt), 0, 0};
  const int64_t rows = (int64_t)B * T;
  int cpw = 4;
  while (cpw > 1 && rows * ((a.n_chunks + kChunksPerWG * cpw - 1) / (kChunksPerWG * cpw)) < 2048)
    cpw /= 2;
  dim3 grid((a.n_chunks + kChunksPerWG * cpw - 1) / (kChunksPerWG * cpw), (unsigned)rows);
  // Rounds.  With one chunk per wavefront the grid over every row already spreads a few
  // undecided rows as widely as a list would, so every round takes it.  With more, a
  // wavefront would reduce its chunks one after another however few rows are left, so
  // after the first round (where most rows are still undecided) the rounds run over a
  // list of the undecided rows, one chunk per wavefront.
  const bool lists = cpw > 1 && max_children > 1;
  a.reset_lists = lists;
#define EV_LAUNCH_SAMPLED(C)                                                                  \
  do {                                                                                        \
    if (lists) hipLaunchKernelGGL((sampled_round_kernel<C, true>), grid, dim3(256), 0, stream, a); \
    else hipLaunchKernelGGL((sampled_round_kernel<C, false>), grid, dim3(256), 0, stream, a); \
  } while (0)
#define EV_LAUNCH_STATS(C)                                                                    \
  do {                                                                                        \
    if ((V & 3) == 0) hipLaunchKernelGGL((sampled_stats_kernel<C, true>), grid, dim3(256), 0, stream, a); \
    else hipLaunchKernelGGL((sampled_stats_kernel<C, false>), grid, dim3(256), 0, stream, a); \
  } while (0)
  if (cpw == 4) EV_LAUNCH_STATS(4);
  else if (cpw == 2) EV_LAUNCH_STATS(2);
  else EV_LAUNCH_STATS(1);
#undef EV_LAUNCH_STATS
  const int64_t items = rows * ((a.n_chunks + kChunksPerWG - 1) / kChunksPerWG);
  const dim3 lgrid((unsigned)std::min<int64_t>(items, kRoundGrid));
  for (int r = 1; r <= max_children; ++r) {
    a.round = r;
    if (r > 1 && lists)
      hipLaunchKernelGGL(sampled_list_round_kernel, lgrid, dim3(256), 0, stream, a);
    else if (cpw == 4) EV_LAUNCH_SAMPLED(4);
    else if (cpw == 2) EV_LAUNCH_SAMPLED(2);
    else EV_LAUNCH_SAMPLED(1);
  }
#undef EV_LAUNCH_SAMPLED
  return launch_status();
}
}  // namespace ev

EV_API size_t ev_accept_workspace(int32_t B, int32_t T, int32_t V) {
  if (B < 1 || T < 1 || V < 1) return 0;
  return ev::ws_layout(B, T, V).total;
}

EV_API ev_status ev_accept_greedy(const float *logits, const int32_t *tokens, const int32_t *parent,
                                  int32_t B, int32_t T, int32_t V, int32_t *accept_len,
                                  int32_t *path, int32_t *out_tokens, void *ws, size_t ws_bytes,
                                  int32_t *dev_status, hipStream_t stream) {
  ev_status st = ev::check_common(logits, tokens, parent, B, T, V, accept_len, path, out_tokens,
                                  ws, ws_bytes);
  if (st != EV_OK || B == 0) return st;
  return ev::launch_accept(false, logits, tokens, parent, B, T, V, 0.0, nullptr, accept_len, path,
                           out_tokens, ws, dev_status, stream);
}

EV_API ev_status ev_accept_rejection(const float *logits, const int32_t *tokens,
                                     const int32_t *parent, int32_t B, int32_t T, int32_t V,
                                     float temperature, const double *uniforms,
                                     int32_t *accept_len, int32_t *path, int32_t *out_tokens,
                                     void *ws, size_t ws_bytes, int32_t *dev_status,
                                     hipStream_t stream) {
  if (!(temperature > 0.f) || !isfinite(temperature)) return EV_ERR_ARG;
  ev_status st = ev::check_common(logits, tokens, parent, B, T, V, accept_len, path, out_tokens,
                                  ws, ws_bytes);
  if (st != EV_OK || B == 0) return st;
  if (!uniforms) return EV_ERR_NULL;
  return ev::launch_accept(true, logits, tokens, parent, B, T, V, 1.0 / (double)temperature,
                           uniforms, accept_len, path, out_tokens, ws, dev_status, stream);
}

namespace ev {

// The walking workgroup compacts the cache itself when one accepted node's rows (every
// layer, KV head, K and V) are at most this many 16-byte pieces, so that a typical path of
// a few nodes fits one round of its 1024 pieces; larger moves go to the compaction
// kernel's grid of workgroups (32 MHA heads of 256-byte rows, 1024 pieces a node, took the
// fused Llama-2-7B-shaped step from 30.1 to 34.1 us).
constexpr int kFusedCompactPieces = 256;

// Acceptance followed by compaction of each accepted path: one launch when the cache has
// few layers, else the acceptance launch and then ev_kv_compact.
static ev_status accept_and_compact(bool rej, const float *logits, const int32_t *tokens,
                                    const int32_t *parent, int32_t B, int32_t T, int32_t V,
                                    double inv_tau, const double *uniforms, int32_t *accept_len,
                                    int32_t *path, int32_t *out_tokens, const ev_kv_desc *kv,
                                    const int32_t *prefix_len, int32_t *new_len, void *ws,
                                    int32_t *dev_status, hipStream_t stream) {
  KvAddr addr;
  ev_status st = make_kv_addr(kv, &addr);
  if (st != EV_OK) return st;
  if ((int64_t)kv->n_layers * kv->n_kv_heads * 2 > 65535) return EV_ERR_SHAPE;
  if (kv->n_layers > 1 && (kv->layer_stride <= 0 || kv->layer_stride % kv->head_dim))
    return EV_ERR_SHAPE;
  if (!prefix_len || !new_len) return EV_ERR_NULL;
  const int row_bytes = kv->dtype == EV_F32 ? 4 * kv->head_dim
                      : kv->dtype == EV_BF16 ? 2 * kv->head_dim : kv->head_dim / 2;
  const int64_t pieces_per_move = (int64_t)kv->n_layers * kv->n_kv_heads * 2 * (row_bytes / 16);
  if (pieces_per_move > kFusedCompactPieces) {
    st = launch_accept(rej, logits, tokens, parent, B, T, V, inv_tau, uniforms, accept_len, path,
                       out_tokens, ws, dev_status, stream);
    if (st != EV_OK) return st;
    return ev_kv_compact(kv, prefix_len, path, accept_len, B, T, new_len, dev_status, stream);
  }
  CompactSeq c{};
  c.k = (char *)kv->k;
  c.v = (char *)kv->v;
  c.k_scale = kv->dtype == EV_INT4 ? const_cast<float *>(kv->k_scale) : nullptr;
  c.v_scale = kv->dtype == EV_INT4 ? const_cast<float *>(kv->v_scale) : nullptr;
  c.kv = addr;
  c.row_bytes = row_bytes;
  c.layer_rows = kv->n_layers > 1 ? kv->layer_stride / kv->head_dim : 0;
  c.n_layers = kv->n_layers;
  c.prefix_len = prefix_len;
  c.new_len = new_len;
  return launch_accept(rej, logits, tokens, parent, B, T, V, inv_tau, uniforms, accept_len, path,
                       out_tokens, ws, dev_status, stream, &c);
}

}  // namespace ev

EV_API ev_status ev_accept_greedy_compact(const float *logits, const int32_t *tokens,
                                          const int32_t *parent, int32_t B, int32_t T, int32_t V,
                                          int32_t *accept_len, int32_t *path, int32_t *out_tokens,
                                          const ev_kv_desc *kv, const int32_t *prefix_len,
                                          int32_t *new_len, void *ws, size_t ws_bytes,
                                          int32_t *dev_status, hipStream_t stream) {
  ev_status st = ev::check_common(logits, tokens, parent, B, T, V, accept_len, path, out_tokens,
                                  ws, ws_bytes);
  if (st != EV_OK || B == 0) return st;
  return ev::accept_and_compact(false, logits, tokens, parent, B, T, V, 0.0, nullptr, accept_len,
                                path, out_tokens, kv, prefix_len, new_len, ws, dev_status, stream);
}

EV_API ev_status ev_accept_rejection_compact(const float *logits, const int32_t *tokens,
                                             const int32_t *parent, int32_t B, int32_t T,
                                             int32_t V, float temperature,
                                             const double *uniforms, int32_t *accept_len,
                                             int32_t *path, int32_t *out_tokens,
                                             const ev_kv_desc *kv, const int32_t *prefix_len,
                                             int32_t *new_len, void *ws, size_t ws_bytes,
                                             int32_t *dev_status, hipStream_t stream) {
  if (!(temperature > 0.f) || !isfinite(temperature)) return EV_ERR_ARG;
  ev_status st = ev::check_common(logits, tokens, parent, B, T, V, accept_len, path, out_tokens,
                                  ws, ws_bytes);
  if (st != EV_OK || B == 0) return st;
  if (!uniforms) return EV_ERR_NULL;
  return ev::accept_and_compact(true, logits, tokens, parent, B, T, V, 1.0 / (double)temperature,
                                uniforms, accept_len, path, out_tokens, kv, prefix_len, new_len,
                                ws, dev_status, stream);
}

EV_API size_t ev_accept_sampled_workspace(int32_t B, int32_t T, int32_t V) {
  if (B < 1 || T < 1 || V < 1) return 0;
  return ev::sampled_ws_layout(B, T, V).total;
}

EV_API ev_status ev_accept_sampled(const float *logits, const float *draft_logits,
                                   const int32_t *tokens, const int32_t *parent, int32_t B,
                                   int32_t T, int32_t V, float temperature,
                                   float draft_temperature, const double *uniforms,
                                   int32_t max_children, int32_t *accept_len, int32_t *path,
                                   int32_t *out_tokens, void *ws, size_t ws_bytes,
                                   int32_t *dev_status, hipStream_t stream) {
  if (!(temperature > 0.f) || !isfinite(temperature)) return EV_ERR_ARG;
  if (!(draft_temperature > 0.f) || !isfinite(draft_temperature)) return EV_ERR_ARG;
  if (B < 0 || T < 1 || T > ev::kMaxNodes || V < 1 || V > 64 * ev::kChunkRegs * ev::kChunk)
    return EV_ERR_SHAPE;
  if ((int64_t)B * T > ev::kMaxRows || max_children < 0 || max_children >= T + 1)
    return EV_ERR_SHAPE;
  if (B == 0) return EV_OK;
  if (!logits || !draft_logits || !tokens || !parent || !uniforms || !accept_len || !path ||
      !out_tokens)
    return EV_ERR_NULL;
  if (!ws || ws_bytes < ev::sampled_ws_layout(B, T, V).total) return EV_ERR_WORKSPACE;
  return ev::launch_sampled(logits, draft_logits, tokens, parent, B, T, V,
                            1.0 / (double)temperature, 1.0 / (double)draft_temperature, uniforms,
                            max_children, accept_len, path, out_tokens, ws, dev_status, stream);
}
