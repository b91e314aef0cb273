// Dynamic draft-tree construction: entropy-guided beam expansion and the final rerank.
//
// [TR] sec. 2 (sequence diagram; "Dynamic Tree-Attention Masking"): the drafter grows the
// candidate tree depth by depth (4 to 6 deep), judges each prediction by the entropy of
// its distribution, prunes weak branches with a beam search, and hands the verifier a
// tree of at most 64 nodes.  The rules (the plainest reading of the page):
//   * frontier node n with q_n = softmax(draft_logits_n / tau) gets
//     k_n = min(k_max, max(1, floor(exp(H(q_n)) + 1/2))) children, its k_n most probable
//     tokens (equal logits: lower token id first) -- one child when the prediction is
//     near-certain, k_max when it is flat;
//   * a node's value is the product of the draft probabilities along its path (root 1);
//   * each depth keeps the W best new candidates as the next frontier (the beam);
//   * the tree is the root plus the N - 1 best candidates of all depths, numbered by
//     depth, then by value rank.  Equal values go to the lower candidate id, and ids run
//     depth by depth, frontier slot, child rank.
//
// Expansion is two launches per depth:
//   * over (chunk group, frontier row) workgroups, each wavefront streams one 1024-logit
//     chunk and stores float64 (M_c, S_c, T_c), S_c = sum e, T_c = sum e (s - M_c),
//     e = exp(s - M_c), s = logit / tau, and the chunk's best (logit, token);
//   * one workgroup per frontier row then merges them.  The entropy is
//     H = log S - T / S, so the perplexity is exp(H) = S / exp(T / S) (T <= 0).  The
//     row's k best tokens lie in the k chunks with the best maxima, which it re-reads;
//     their probabilities follow from (M, S);
//   * the workgroup that completes a sequence's frontier forms the new candidates, one
//     per lane (frontier slot = lane / 8, child rank = lane % 8), stores them and keeps
//     the best W as the next frontier.
// The rerank is one wavefront per sequence.  The workspace keeps the tree under
// construction between calls; the frontier state is double-buffered by depth parity so
// that a launch never reads what its own last workgroup rewrites.
#include "ev_internal.h"
#include "rowstream.h"

namespace ev {

constexpr int kTreeTop = 8;            // most children per node, widest beam
// the float64 exp's table: 64 entries (small, latency-bound launches; see rowstream.h)
constexpr int kTreeExpBits = 6;
constexpr int kMaxExpansions = 16;     // deepest tree under construction
constexpr int kCandSlots = 64;         // candidates per depth: kTreeTop frontier x kTreeTop

struct TreeChunk {
  double M, S, T;
};
struct TreeRow {                       // one frontier row after its merge
  int32_t k;
  int32_t tok[kTreeTop];
  double q[kTreeTop];
};
struct TreeCand {
  double value;
  int32_t parent;                      // candidate id of the parent, -1: the root
  int32_t token;
};
struct TreeFront {
  int32_t count;
  int32_t id[kTreeTop];                // candidate ids
  double value[kTreeTop];
};

struct TreeWs {
  size_t row_cnt, seq_cnt, chunk, top, rows, front, cand, cand_rank, cand_count, n_exp, total;
};

inline TreeWs tree_ws_layout(int B, int W, int V) {
  TreeWs w;
  const size_t rows = (size_t)B * W, per_chunk = rows * n_chunks_of(V);
  w.row_cnt = 0;
  w.seq_cnt = kCounterBytes / 2;
  w.chunk = kCounterBytes;
  w.top = w.chunk + align_up(per_chunk * sizeof(TreeChunk), 256);
  w.rows = w.top + align_up(per_chunk * sizeof(uint64_t), 256);
  w.front = w.rows + align_up(rows * sizeof(TreeRow), 256);
  w.cand = w.front + align_up(2 * (size_t)B * sizeof(TreeFront), 256);
  w.cand_rank = w.cand + align_up((size_t)B * kMaxExpansions * kCandSlots * sizeof(TreeCand), 256);
  w.cand_count = w.cand_rank + align_up((size_t)B * kMaxExpansions * kCandSlots * sizeof(int32_t), 256);
  w.n_exp = w.cand_count + align_up((size_t)B * kMaxExpansions * sizeof(int32_t), 256);
  w.total = w.n_exp + align_up((size_t)B * sizeof(int32_t), 256);
  return w;
}

struct ExpandArgs {
  const float *logits;                 // [B][W][V]
  int B, W, V, n_chunks, depth, k_max;
  double inv_tau;
  TreeChunk *chunk;                    // [B*W][n_chunks]
  uint64_t *top;                       // [B*W][n_chunks] packed best (logit, token)
  TreeRow *rows;                       // [B*W]
  const TreeFront *front_in;           // [B], this depth's frontier (depth >= 1)
  TreeFront *front_out;                // [B], the next one
  TreeCand *cand;                      // [B][kMaxExpansions][kCandSlots]
  int32_t *cand_rank;                  // [B][kMaxExpansions][kCandSlots]: slot of each rank
  int32_t *cand_count;                 // [B][kMaxExpansions]
  int32_t *n_exp;                      // [B] expansions done
  int32_t *row_cnt, *seq_cnt;
  int32_t *out_tokens, *out_slots, *out_count;
  int32_t *dev_status;
};

// Is (v, i) after (lv, li) in the order "larger logit first, then lower token id"?
__device__ inline bool after(float v, int i, float lv, int li) {
  return (v < lv) | ((v == lv) & (i > li));
}

// A lane's best two (value, index) pairs, best first.
struct Top2 {
  float v1;
  int i1;
  float v2;
  int i2;
};

__device__ inline bool beats(float v, int i, float v2, int i2) {
  return (v > v2) | ((v == v2) & (i < i2));
}

// Best two of two best-two lists: the winner of the two leaders, then the better of the
// losing leader and the winner's runner-up.
__device__ inline Top2 merge_top2(const Top2 &a, const Top2 &b) {
  const bool bw = beats(b.v1, b.i1, a.v1, a.i1);
  const float lv = bw ? a.v1 : b.v1, sv = bw ? b.v2 : a.v2;
  const int li = bw ? a.i1 : b.i1, si = bw ? b.i2 : a.i2;
  const bool sw = beats(sv, si, lv, li);
  return Top2{bw ? b.v1 : a.v1, bw ? b.i1 : a.i1, sw ? sv : lv, sw ? si : li};
}

// The lane's two best of its N (value, index) pairs that come after (lv, li), by a
// tournament (log2 N dependent merge levels).
template <int N>
__device__ inline void best_two_after(const float (&v)[N], const int (&idx)[N], float lv, int li,
                                      float &v1, int &i1, float &v2, int &i2) {
  static_assert((N & (N - 1)) == 0, "power of two");
  Top2 t[N];
#pragma unroll
  for (int e = 0; e < N; ++e) {
    const bool ok = after(v[e], idx[e], lv, li);
    t[e] = Top2{ok ? v[e] : -INFINITY, ok ? idx[e] : INT_MAX, -INFINITY, INT_MAX};
  }
#pragma unroll
  for (int n = N / 2; n >= 1; n /= 2) {
#pragma unroll
    for (int p = 0; p < n; ++p) t[p] = merge_top2(t[p], t[p + n]);
  }
  v1 = t[0].v1;
  i1 = t[0].i1;
  v2 = t[0].v2;
  i2 = t[0].i2;
}

// The wave's `rounds` best pairs over the lanes' arrays, best first, into (tv, ti) (wave-
// uniform).  Each lane keeps its best two; a lane whose two are both taken rescans its
// array for the best after its last taken pair (rare: 3 of the winners in one lane).
template <int N>
__device__ inline void wave_top(const float (&v)[N], const int (&idx)[N], int rounds,
                                float (&tv)[kTreeTop], int (&ti)[kTreeTop]) {
  float h1, h2;
  int j1, j2;
  best_two_after(v, idx, INFINITY, -1, h1, j1, h2, j2);
  int used = 0;                         // of the lane's current pair
#pragma unroll
  for (int r = 0; r < kTreeTop; ++r) {
    if (r < rounds) {
      float wv = h1;
      int wi = j1;
      wave_argmax(wv, wi);
      tv[r] = wv;
      ti[r] = wi;
      const bool mine = (j1 == wi) & (h1 == wv);
      if (mine) {
        h1 = h2;
        j1 = j2;
        ++used;
      }
      if (__any(mine && used == 2)) {
        if (mine && used == 2) {
          best_two_after(v, idx, wv, wi, h1, j1, h2, j2);
          used = 0;
        }
      }
    } else {
      tv[r] = -INFINITY;
      ti[r] = INT_MAX;
    }
  }
}

__device__ inline void better_d(double &v, int &i, double v2, int i2) {
  const bool take = (v2 > v) | ((v2 == v) & (i2 < i));
  v = take ? v2 : v;
  i = take ? i2 : i;
}

// Wave-wide best (largest value, then lowest id) of one (value, id) per lane.
__device__ inline void wave_best_d(double &v, int &i) {
  better_d(v, i, dpp_d<kDppQuadSwap1>(v), dpp_i<kDppQuadSwap1>(i));
  better_d(v, i, dpp_d<kDppQuadSwap2>(v), dpp_i<kDppQuadSwap2>(i));
  better_d(v, i, dpp_d<kDppHalfMirror>(v), dpp_i<kDppHalfMirror>(i));
  better_d(v, i, dpp_d<kDppMirror>(v), dpp_i<kDppMirror>(i));
  double bv = lane_d(v, 0);
  int bi = lane_i(i, 0);
#pragma unroll
  for (int r = 16; r < 64; r += 16) better_d(bv, bi, lane_d(v, r), lane_i(i, r));
  v = bv;
  i = bi;
}

// Merge of a streamed row (the whole workgroup of kTreeTop wavefronts): statistics,
// width, best tokens.  The row's k best tokens lie in the k chunks whose own best tokens
// rank first: a token in any other chunk is preceded by at least k chunk maxima.
// Wavefront 0 finds those chunks; wavefront j re-reads the j-th (from cache) and takes
// its best tokens among those not after the k-th chunk maximum; each of the at most
// k * k pairs then finds its rank among all of them.
constexpr int kMergeThreads = 64 * kTreeTop;

struct MergeShared {
  double M, S;
  int k;
  float tv;                            // the k-th best chunk maximum
  int ti;
  int chunk[kTreeTop];
  uint64_t ent[kTreeTop * kTreeTop];   // the wavefronts' lists, packed
};

__device__ void merge_row(const ExpandArgs &a, int64_t row, const double *tab, MergeShared &sh) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int nc = a.n_chunks;
  if (wave == 0) {
    // row statistics from the chunk statistics (lane holds chunks lane, lane + 64, ...)
    TreeChunk cs[kChunkRegs];
    float cv[kChunkRegs];
    int ci[kChunkRegs];
    double M = -INFINITY;
#pragma unroll
    for (int r = 0; r < kChunkRegs; ++r) {
      const int c = lane + 64 * r;
      cs[r] = c < nc ? a.chunk[row * nc + c] : TreeChunk{-INFINITY, 0.0, 0.0};
      const GreedyStat g = c < nc ? unpack(a.top[row * nc + c]) : GreedyStat{-INFINITY, INT_MAX};
      cv[r] = g.val;
      ci[r] = g.idx;
      M = fmax(M, cs[r].M);
    }
    M = wave_max(M);
    double S = 0.0, T = 0.0, xf[kChunkRegs], ef[kChunkRegs];
#pragma unroll
    for (int r = 0; r < kChunkRegs; ++r) xf[r] = cs[r].M - M;
    exp_nonpos_n<kChunkRegs, kTreeExpBits>(xf, ef, tab);
#pragma unroll
    for (int r = 0; r < kChunkRegs; ++r) {
      if (cs[r].S > 0.0) {
        const double f = ef[r];
        S += cs[r].S * f;
        T += f * fma(cs[r].M - M, cs[r].S, cs[r].T);
      }
    }
    S = wave_sum(S);
    T = wave_sum(T);
    const double ppl = S / exp_nonpos<kTreeExpBits>(T / S, tab);
    const double half_up = ppl + 0.5;
    const int k = half_up >= (double)a.k_max ? a.k_max : max(1, (int)floor(half_up));
    // the k chunks whose maxima rank first (k rounds over the lanes' chunk maxima); the
    // k-th of them bounds the row's k best tokens: none comes after it
    float tv[kTreeTop];
    int ti[kTreeTop];
    wave_top(cv, ci, k, tv, ti);
    if (lane == 0) {
      sh.M = M;
      sh.S = S;
      sh.k = k;
      const bool full = ti[k - 1] >= 0 && ti[k - 1] < a.V;
      sh.tv = full ? tv[k - 1] : -INFINITY;   // fewer than k chunks: every token qualifies
      sh.ti = full ? ti[k - 1] : INT_MAX;
#pragma unroll
      for (int r = 0; r < kTreeTop; ++r)
        sh.chunk[r] = (r < k && ti[r] >= 0 && ti[r] < a.V) ? ti[r] / kChunk : -1;
    }
  }
  __syncthreads();
  const int k = sh.k;
  {
    const int c = wave < k ? sh.chunk[wave] : -1;
    float tv[kTreeTop];
    int ti[kTreeTop];
    int n_cand = 0;
    if (c >= 0) {
      float v[16];
      int idx[16];
      load_chunk(a.logits + row * a.V, a.V, c * kChunk, (a.V & 3) == 0, v, idx);
      const float thv = sh.tv;
      const int thi = sh.ti;
      int mine = 0;
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const bool keep = !after(v[e], idx[e], thv, thi);
        v[e] = keep ? v[e] : -INFINITY;
        idx[e] = keep ? idx[e] : INT_MAX;
        mine += keep ? 1 : 0;
      }
      // rounds needed: the chunk's qualifying tokens (a wave sum of `mine`, bit by bit),
      // at most k
      int total = 0;
#pragma unroll
      for (int m = 1; m <= 16; m <<= 1) total += __popcll(__ballot((mine & m) != 0)) * m;
      n_cand = min(total, k);
      wave_top(v, idx, n_cand, tv, ti);
    }
    if (lane == 0) {
#pragma unroll
      for (int r = 0; r < kTreeTop; ++r)
        sh.ent[wave * kTreeTop + r] = pack(r < n_cand ? GreedyStat{tv[r], ti[r]}
                                                      : GreedyStat{-INFINITY, INT_MAX});
    }
  }
  __syncthreads();
  if (wave != 0) return;
  // entry e = lane goes to its rank among all the lists' entries; the lane holding rank r
  // writes the row's r-th token
  const GreedyStat me = unpack(sh.ent[lane]);
  int rank = 0;
#pragma unroll
  for (int f = 0; f < kTreeTop * kTreeTop; ++f) {
    const GreedyStat o = unpack(sh.ent[f]);
    rank += beats(o.val, o.idx, me.val, me.idx) ? 1 : 0;
  }
  const bool real = me.idx != INT_MAX;
  const int n_real = __popcll(__ballot(real));
  TreeRow *out = a.rows + row;
  if (lane == 0) publish(&out->k, k);
  if (real && rank < k) {
    publish(&out->tok[rank], me.idx);
    publish(&out->q[rank], exp_nonpos<kTreeExpBits>(shifted(me.val, a.inv_tau, sh.M), tab) / sh.S);
  }
  if (lane < kTreeTop && lane >= min(k, n_real)) {
    if (lane < k) report(a.dev_status, EV_DERR_TOKEN);   // only NaN logits: too few tokens
    publish(&out->tok[lane], lane < k ? a.V - 1 : -1);
    publish(&out->q[lane], 0.0);
  }
}

// New candidates of a sequence and the next frontier (one wavefront).
__device__ void expand_sequence(const ExpandArgs &a, int b, int count, double *sval) {
  const int lane = threadIdx.x & 63;
  const int w = lane >> 3, j = lane & 7;
  const bool live_slot = w < count;
  const TreeRow *rr = a.rows + (int64_t)b * a.W + min(w, count - 1);
  const int k = observe(&rr->k);
  const bool valid = live_slot && j < k;
  const double q = valid ? observe(&rr->q[j]) : 0.0;
  const int tok = valid ? observe(&rr->tok[j]) : -1;
  double pval = 1.0;
  int pid = -1;
  if (a.depth > 0 && live_slot) {
    pval = a.front_in[b].value[w];
    pid = a.front_in[b].id[w];
  }
  const double value = pval * q;
  const uint64_t vmask = __ballot(valid);
  const int slot = __popcll(vmask & ((1ull << lane) - 1ull));
  const int n_valid = __popcll(vmask);
  const int64_t cbase = ((int64_t)b * kMaxExpansions + a.depth) * kCandSlots;
  if (valid) a.cand[cbase + slot] = TreeCand{value, pid, tok};
  if (lane == 0) {
    a.cand_count[(int64_t)b * kMaxExpansions + a.depth] = n_valid;
    a.n_exp[b] = a.depth + 1;
  }
  // the beam: each candidate's rank among the valid ones (ties: lower lane = lower id),
  // counted against all lanes' values staged in LDS
  sval[lane] = valid ? value : -1.0;
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  int rank = 0;
#pragma unroll 8
  for (int f = 0; f < 64; ++f) {
    const double vf = sval[f];
    rank += ((vf > value) | ((vf == value) & (f < lane))) ? 1 : 0;
  }
  if (valid) a.cand_rank[cbase + rank] = slot;   // the depth's candidates best first
  const int n_sel = min(a.W, n_valid);
  TreeFront *fo = a.front_out + b;
  if (valid && rank < n_sel) {
    fo->id[rank] = a.depth * kCandSlots + slot;
    fo->value[rank] = value;
    a.out_tokens[(int64_t)b * a.W + rank] = tok;
    a.out_slots[(int64_t)b * a.W + rank] = w;
  }
  if (lane >= n_sel && lane < a.W) {
    a.out_tokens[(int64_t)b * a.W + lane] = -1;
    a.out_slots[(int64_t)b * a.W + lane] = -1;
  }
  if (lane == 0) {
    fo->count = n_sel;
    a.out_count[b] = n_sel;
  }
}

// Streaming launch: one 1024-logit chunk per wavefront per step.
template <int CPW>
__global__ __launch_bounds__(256) void tree_chunk_kernel(ExpandArgs a) {
  __shared__ double tab[1 << kTreeExpBits];
  const int64_t row = blockIdx.y;
  const int b = (int)(row / a.W), w = (int)(row % a.W);
  const int count = a.depth == 0 ? 1 : a.front_in[b].count;   // written by the last depth
  if (w >= count) return;              // unused frontier slot
  fill_exp_table<kTreeExpBits>(tab);
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int nc = a.n_chunks;
  __syncthreads();
  const float *lr = a.logits + row * a.V;
  const bool vec_ok = (a.V & 3) == 0;
  const int c0 = blockIdx.x * kChunksPerWG * CPW + wave;
#pragma unroll
  for (int m = 0; m < CPW; ++m) {
    const int c = c0 + kChunksPerWG * m;
    if (c >= nc) continue;
    float v[16];
    int idx[16];
    load_chunk(lr, a.V, c * kChunk, vec_ok, v, idx);
    float bv = -INFINITY;
    int bi = INT_MAX;
#pragma unroll
    for (int e = 0; e < 16; ++e) better(bv, bi, v[e], idx[e]);
    wave_argmax(bv, bi);               // the chunk's best (largest logit, lowest token)
    const double M = (double)bv * a.inv_tau;
    double S = 0.0, T = 0.0;
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const double d = shifted(v[e], a.inv_tau, M);
      const double ex = exp_nonpos<kTreeExpBits>(d, tab);
      S += ex;
      T += d >= -745.0 ? ex * d : 0.0;  // e * d -> 0 as d -> -inf (padding, -inf logits)
    }
    S = wave_sum(S);
    T = wave_sum(T);
    if (lane == 0) {
      a.chunk[row * nc + c] = TreeChunk{M, S, T};
      a.top[row * nc + c] = pack(GreedyStat{bv, bi});
    }
  }
}

// Merge launch: one workgroup per frontier row; the workgroup that completes a
// sequence's frontier forms its candidates and the next beam.
__global__ __launch_bounds__(kMergeThreads) void tree_merge_kernel(ExpandArgs a) {
  __shared__ double tab[1 << kTreeExpBits];
  __shared__ int s_last;
  __shared__ MergeShared sh;
  __shared__ double s_rank[64];
  const int64_t row = blockIdx.x;
  const int b = (int)(row / a.W), w = (int)(row % a.W);
  const int count = a.depth == 0 ? 1 : a.front_in[b].count;
  if (w >= count) return;
  fill_exp_table<kTreeExpBits>(tab);
  __syncthreads();
  merge_row(a, row, tab, sh);
  if (!last_arrival(&a.seq_cnt[counter_slot(b)], count, &s_last)) return;
  if ((threadIdx.x >> 6) == 0) expand_sequence(a, b, count, s_rank);
}

struct FinalArgs {
  const int32_t *root_tokens;
  int B, n_nodes;
  const TreeCand *cand;
  const int32_t *cand_rank;
  const int32_t *cand_count;
  const int32_t *n_exp;
  int32_t *parent, *tokens, *tree_size;
};

// The tree of each sequence: the n_nodes - 1 best candidates, numbered by depth, then by
// value rank.  One workgroup per sequence.  The order is "larger value first, then lower
// id" (id = depth * 64 + slot); each depth's candidates are already listed in that order
// (expand_sequence ranks them for its beam), so a candidate's place in the whole order is
// its rank in its own depth plus, for every other depth, the number of that depth's
// candidates before it, found by binary search.  Only candidates ranked below
// n_nodes - 1 in their own depth can be among the best n_nodes - 1.  (A full bitonic sort
// of all candidates took 55 dependent LDS stages.)  One wavefront then numbers them.
constexpr int kFinalThreads = 512;
constexpr int kFinalKeys = kMaxExpansions * kCandSlots;

__device__ inline bool key_before(double v, int i, double v2, int i2) {
  return (v > v2) | ((v == v2) & (i < i2));
}

__global__ __launch_bounds__(kFinalThreads) void tree_finalize_kernel(FinalArgs a) {
  __shared__ double kv[kFinalKeys];
  __shared__ int ki[kCandSlots];
  __shared__ int srt[kFinalKeys];
  __shared__ int pos_of[kFinalKeys];
  const int tid = threadIdx.x;
  const int b = blockIdx.x;
  __shared__ int s_cc[kMaxExpansions];
  // every load at once: the expansion count, the per-depth counts, all candidate values
  // and the rank-order lists
  const int n_exp_raw = a.n_exp[b];
  const TreeCand *cb = a.cand + (int64_t)b * kMaxExpansions * kCandSlots;
  const int32_t *cr = a.cand_rank + (int64_t)b * kMaxExpansions * kCandSlots;
  const int32_t *cc = a.cand_count + (int64_t)b * kMaxExpansions;
  if (tid < kMaxExpansions) s_cc[tid] = cc[tid];
  double cval[kFinalKeys / kFinalThreads];
  int crank[kFinalKeys / kFinalThreads];
#pragma unroll
  for (int r = 0; r < kFinalKeys / kFinalThreads; ++r) {
    cval[r] = cb[tid + r * kFinalThreads].value;
    crank[r] = cr[tid + r * kFinalThreads];
  }
  const int n_exp = max(0, min(n_exp_raw, kMaxExpansions));
  __syncthreads();
  int total = 0;
  for (int e = 0; e < n_exp; ++e) total += min(max(s_cc[e], 0), kCandSlots);
  const int n_sel = min(a.n_nodes - 1, total);
#pragma unroll
  for (int r = 0; r < kFinalKeys / kFinalThreads; ++r) {
    const int i = tid + r * kFinalThreads;
    const int e = i / kCandSlots, slot = i % kCandSlots;
    const bool valid = e < n_exp && slot < s_cc[e];
    kv[i] = valid ? cval[r] : -1.0;    // values are >= 0
    srt[i] = (e << 6) | (crank[r] & (kCandSlots - 1));   // id of the rank-slot-th best
    pos_of[i] = 0;
  }
  if (tid < kCandSlots) ki[tid] = INT_MAX;
  __syncthreads();
  // candidate (depth e, own rank r): place = r + sum over the other depths of the number
  // of their candidates before it
#pragma unroll
  for (int q = 0; q < kFinalKeys / kFinalThreads; ++q) {
    const int i = tid + q * kFinalThreads;
    const int e = i / kCandSlots, r = i % kCandSlots;
    if (e >= n_exp || r >= min(s_cc[e], kCandSlots) || r >= n_sel) continue;
    const int id = srt[i];
    const double v = kv[id];
    int place = r;
    for (int e2 = 0; e2 < n_exp; ++e2) {
      if (e2 == e) continue;
      int lo = 0, hi = min(max(s_cc[e2], 0), kCandSlots);
      while (lo < hi) {                  // first of depth e2 not before (v, id)
        const int mid = (lo + hi) >> 1;
        const int id2 = srt[e2 * kCandSlots + mid];
        if (key_before(kv[id2], id2, v, id)) lo = mid + 1;
        else hi = mid;
      }
      place += lo;
    }
    if (place < n_sel) ki[place] = id;
  }
  __syncthreads();
  // numbering (wavefront 0): by depth, then by rank (lane r holds the r-th best)
  const int lane = tid & 63;
  int id = INT_MAX, pos = 0, n_tree = 1;
  bool mine = false;
  if (tid < 64) {
    id = lane < n_sel ? ki[lane] : INT_MAX;
    mine = id < n_exp * kCandSlots;     // false only for NaN-valued leftovers
    const int dep = mine ? id / kCandSlots : kMaxExpansions;
    int before = 0;
    for (int e = 0; e < n_exp; ++e) {
      const uint64_t m = __ballot(mine && dep == e);
      if (e < dep) before += __popcll(m);
      if (e == dep) before += __popcll(m & ((1ull << lane) - 1ull));
    }
    n_tree = 1 + __popcll(__ballot(mine));
    pos = 1 + before;
    if (mine) pos_of[id] = pos;
  }
  __syncthreads();
  if (tid >= 64) return;
  int32_t *par = a.parent + (int64_t)b * a.n_nodes;
  int32_t *tok = a.tokens + (int64_t)b * a.n_nodes;
  if (mine) {
    const TreeCand c = cb[id];
    const int pp = c.parent;
    par[pos] = (pp < 0 || pp >= kFinalKeys) ? 0 : pos_of[pp];
    tok[pos] = c.token;
  }
  if (lane == 0) {
    par[0] = -1;
    tok[0] = a.root_tokens[b];
    a.tree_size[b] = n_tree;
  }
  if (lane >= n_tree && lane < a.n_nodes) {
    par[lane] = -1;
    tok[lane] = -1;
  }
}

}  // namespace ev

EV_API size_t ev_draft_tree_workspace(int32_t B, int32_t beam, int32_t V) {
  if (B < 1 || beam < 1 || beam > ev::kTreeTop || V < 1) return 0;
  return ev::tree_ws_layout(B, beam, V).total;
}

EV_API ev_status ev_draft_tree_expand(const float *draft_logits, int32_t B, int32_t beam,
                                      int32_t V, int32_t depth, float temperature,
                                      int32_t k_max, int32_t *frontier_tokens,
                                      int32_t *frontier_slots, int32_t *frontier_count,
                                      void *ws, size_t ws_bytes, int32_t *dev_status,
                                      hipStream_t stream) {
  using namespace ev;
  if (!(temperature > 0.f) || !isfinite(temperature)) return EV_ERR_ARG;
  if (B < 0 || beam < 1 || beam > kTreeTop || k_max < 1 || k_max > kTreeTop || V < 1 ||
      V > 64 * kChunkRegs * kChunk || depth < 0 || depth >= kMaxExpansions)
    return EV_ERR_SHAPE;
  if ((int64_t)B * beam > kMaxRows) return EV_ERR_SHAPE;
  if (B == 0) return EV_OK;
  if (!draft_logits || !frontier_tokens || !frontier_slots || !frontier_count) return EV_ERR_NULL;
  const TreeWs w = tree_ws_layout(B, beam, V);
  if (!ws || ws_bytes < w.total) return EV_ERR_WORKSPACE;
  char *base = (char *)ws;
  TreeFront *fronts = (TreeFront *)(base + w.front);
  ExpandArgs a{draft_logits, B, beam, V, n_chunks_of(V), depth, k_max,
               1.0 / (double)temperature, (TreeChunk *)(base + w.chunk),
               (uint64_t *)(base + w.top), (TreeRow *)(base + w.rows),
               fronts + (size_t)(depth & 1) * B, fronts + (size_t)((depth + 1) & 1) * B,
               (TreeCand *)(base + w.cand), (int32_t *)(base + w.cand_rank),
               (int32_t *)(base + w.cand_count),
               (int32_t *)(base + w.n_exp), (int32_t *)(base + w.row_cnt),
               (int32_t *)(base + w.seq_cnt), frontier_tokens, frontier_slots, frontier_count,
               dev_status};
  const int64_t rows = (int64_t)B * beam;
  int cpw = 4;
  while (cpw > 1 && rows * ((a.n_chunks + kChunksPerWG * cpw - 1) / (kChunksPerWG * cpw)) < 2048)
    cpw /= 2;
  dim3 grid((a.n_chunks + kChunksPerWG * cpw - 1) / (kChunksPerWG * cpw), (unsigned)rows);
  if (cpw == 4) hipLaunchKernelGGL((tree_chunk_kernel<4>), grid, dim3(256), 0, stream, a);
  else if (cpw == 2) hipLaunchKernelGGL((tree_chunk_kernel<2>), grid, dim3(256), 0, stream, a);
  else hipLaunchKernelGGL((tree_chunk_kernel<1>), grid, dim3(256), 0, stream, a);
  hipLaunchKernelGGL(tree_merge_kernel, dim3((unsigned)rows), dim3(kMergeThreads), 0, stream, a);
  return launch_status();
}

EV_API ev_status ev_draft_tree_finalize(const int32_t *root_tokens, int32_t B, int32_t beam,
                                        int32_t V, int32_t n_nodes, int32_t *parent,
                                        int32_t *tokens, int32_t *tree_size, void *ws,
                                        size_t ws_bytes, hipStream_t stream) {
  using namespace ev;
  if (B < 0 || beam < 1 || beam > kTreeTop || V < 1 || V > 64 * kChunkRegs * kChunk ||
      n_nodes < 1 || n_nodes > kMaxNodes)
    return EV_ERR_SHAPE;
  if ((int64_t)B * beam > kMaxRows) return EV_ERR_SHAPE;
  if (B == 0) return EV_OK;
  if (!root_tokens || !parent || !tokens || !tree_size) return EV_ERR_NULL;
  const TreeWs w = tree_ws_layout(B, beam, V);
  if (!ws || ws_bytes < w.total) return EV_ERR_WORKSPACE;
  char *base = (char *)ws;
  FinalArgs a{root_tokens, B, n_nodes, (const TreeCand *)(base + w.cand),
              (const int32_t *)(base + w.cand_rank), (const int32_t *)(base + w.cand_count),
              (const int32_t *)(base + w.n_exp), parent, tokens, tree_size};
  hipLaunchKernelGGL(tree_finalize_kernel, dim3(B), dim3(kFinalThreads), 0, stream, a);
  return launch_status();
}
