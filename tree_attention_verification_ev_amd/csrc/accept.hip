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
// Two launches per call:
//   1. stats: one wavefront per (row, 1024-logit chunk) streams the float32 logits once.
//      greedy    -> (max, lowest argmax) per chunk
//      rejection -> float64 (M_c = max s, S_c = sum exp(s - M_c)) per chunk, s = logit/tau
//   2. walk: one wavefront per sequence; lane i holds node i (T <= 64).  Children of the
//      current node come from a ballot over parent[]; per-node statistics are reduced
//      from the chunk table; the bonus draw locates its chunk from the chunk masses and
//      then scans only that chunk in float64.
#include "ev_internal.h"

#include <limits.h>
#include <math.h>

namespace ev {

constexpr int kChunk = 1024;       // logits per wavefront chunk (16 per lane)
constexpr int kChunksPerWG = 4;

struct GreedyStat {
  float val;
  int idx;
};
struct RejStat {
  double M;
  double S;
};

__host__ __device__ inline int n_chunks_of(int V) { return (V + kChunk - 1) / kChunk; }

// Lane's 16 logits of chunk `base`: element (k*64 + lane)*4 + e, k < 4, e < 4 (coalesced).
__device__ inline void load_chunk(const float *row, int V, int base, bool vec_ok, float v[16],
                                  int idx[16]) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    int i0 = base + (k * 64 + lane) * 4;
    if (vec_ok && i0 + 3 < V) {
      f32x4 x = *(const f32x4 *)(row + i0);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        v[4 * k + e] = x[e];
        idx[4 * k + e] = i0 + e;
      }
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        int i = i0 + e;
        v[4 * k + e] = i < V ? row[i] : -INFINITY;
        idx[4 * k + e] = i < V ? i : INT_MAX;
      }
    }
  }
}

// (value, index) pairs: larger value wins, equal values keep the lower index.
__device__ inline void better(float &v, int &i, float v2, int i2) {
  if (v2 > v || (v2 == v && i2 < i)) {
    v = v2;
    i = i2;
  }
}

__device__ inline void wave_argmax(float &v, int &i) {
#pragma unroll
  for (int w = 32; w >= 1; w >>= 1) {
    float v2 = __shfl_xor(v, w);
    int i2 = __shfl_xor(i, w);
    better(v, i, v2, i2);
  }
}

__device__ inline double wave_sum(double x) {
#pragma unroll
  for (int w = 32; w >= 1; w >>= 1) x += __shfl_xor(x, w);
  return x;
}

__device__ inline double wave_max(double x) {
#pragma unroll
  for (int w = 32; w >= 1; w >>= 1) x = fmax(x, __shfl_xor(x, w));
  return x;
}

template <bool REJ>
__global__ __launch_bounds__(256) void accept_stats_kernel(const float *__restrict__ logits, int V,
                                                           int n_chunks, double inv_tau,
                                                           void *__restrict__ stats) {
  const int lane = threadIdx.x & 63;
  const int chunk = blockIdx.x * kChunksPerWG + (threadIdx.x >> 6);
  const int64_t row = blockIdx.y;
  if (chunk >= n_chunks) return;
  const float *src = logits + row * V;
  const bool vec_ok = (V & 3) == 0;
  float v[16];
  int idx[16];
  load_chunk(src, V, chunk * kChunk, vec_ok, v, idx);
  float best = -INFINITY;
  int bi = INT_MAX;
#pragma unroll
  for (int e = 0; e < 16; ++e) better(best, bi, v[e], idx[e]);
  wave_argmax(best, bi);
  if (!REJ) {
    if (lane == 0) ((GreedyStat *)stats)[row * n_chunks + chunk] = GreedyStat{best, bi};
    return;
  }
  const double M = (double)best * inv_tau;
  double s = 0.0;
#pragma unroll
  for (int e = 0; e < 16; ++e)
    if (idx[e] != INT_MAX) s += exp((double)v[e] * inv_tau - M);
  s = wave_sum(s);
  if (lane == 0) ((RejStat *)stats)[row * n_chunks + chunk] = RejStat{M, s};
}

struct WalkArgs {
  const float *logits;
  const int32_t *tokens;
  const int32_t *parent;
  int T, V, n_chunks;
  double inv_tau;
  const double *uniforms;
  const void *stats;
  int32_t *accept_len;
  int32_t *path;
  int32_t *out_tokens;
  int32_t *dev_status;
};

// p_a(y) under the float64 contract.
__device__ inline double prob(const float *row, int y, double inv_tau, double M, double S) {
  return exp((double)row[y] * inv_tau - M) / S;
}

// Inverse-CDF draw from the residual of node row `row` (rejected tokens: lanes set in
// `rej` hold them in `tok`, with their probabilities in `prej`).
__device__ int residual_draw(const WalkArgs &a, const float *row, const RejStat *st, double M,
                             double S, uint64_t rej, int tok, double prej, double t) {
  const int lane = threadIdx.x;
  const int nc = a.n_chunks;
  const int cpl = (nc + 63) / 64;      // contiguous chunks per lane
  // chunk masses with the rejected tokens removed
  double mass[4];                       // cpl <= 4 for V <= 262144
  double tot = 0.0;
  for (int r = 0; r < cpl; ++r) {
    int c = lane * cpl + r;
    mass[r] = c < nc ? st[c].S * exp(st[c].M - M) / S : 0.0;
  }
  for (uint64_t rr = rej; rr; rr &= rr - 1) {
    int src = __ffsll((unsigned long long)rr) - 1;
    int x = __shfl(tok, src);
    double px = __shfl(prej, src);
    int c = x / kChunk;
    for (int r = 0; r < cpl; ++r)
      if (lane * cpl + r == c) mass[r] -= px;
  }
  for (int r = 0; r < cpl; ++r) tot += mass[r];
  // exclusive scan of lane totals
  double incl = tot;
#pragma unroll
  for (int w = 1; w < 64; w <<= 1) {
    double y = __shfl_up(incl, w);
    if (lane >= w) incl += y;
  }
  double excl = incl - tot;
  uint64_t hit = __ballot(incl > t);
  int cstar = -1;
  double cbefore = 0.0;
  if (hit) {
    int hl = __ffsll((unsigned long long)hit) - 1;
    if (lane == hl) {
      double acc = excl;
      for (int r = 0; r < cpl; ++r) {
        if (acc + mass[r] > t || r == cpl - 1) {
          cstar = lane * cpl + r;
          cbefore = acc;
          break;
        }
        acc += mass[r];
      }
      if (cstar >= nc) cstar = nc - 1;
    }
    cstar = __shfl(cstar, hl);
    cbefore = __shfl(cbefore, hl);
  } else {
    cstar = nc - 1;                      // rounding left t beyond the total: last chunk
    cbefore = -INFINITY;
  }
  // scan the chosen chunk element by element (lane owns 16 consecutive ids)
  for (;;) {
    const int y0 = cstar * kChunk + lane * 16;
    double pv[16];
    double lsum = 0.0;
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      int y = y0 + e;
      pv[e] = y < a.V ? prob(row, y, a.inv_tau, M, S) : 0.0;
    }
    for (uint64_t rr = rej; rr; rr &= rr - 1) {
      int src = __ffsll((unsigned long long)rr) - 1;
      int x = __shfl(tok, src);
#pragma unroll
      for (int e = 0; e < 16; ++e)
        if (y0 + e == x) pv[e] = 0.0;
    }
#pragma unroll
    for (int e = 0; e < 16; ++e) lsum += pv[e];
    double li = lsum;
#pragma unroll
    for (int w = 1; w < 64; w <<= 1) {
      double y = __shfl_up(li, w);
      if (lane >= w) li += y;
    }
    double C = cbefore + (li - lsum);
    int first = -1, last = -1;
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      C += pv[e];
      if (first < 0 && pv[e] > 0.0 && C > t) first = y0 + e;
      if (pv[e] > 0.0) last = y0 + e;
    }
    uint64_t fh = __ballot(first >= 0);
    if (fh) return __shfl(first, __ffsll((unsigned long long)fh) - 1);
    // no crossing (rounding at a chunk edge or beyond the total): largest positive id
    uint64_t lh = __ballot(last >= 0);
    if (lh) return __shfl(last, 63 - __clzll((long long)lh));
    if (cstar == 0) return 0;
    --cstar;                             // empty chunk (all rejected / underflow): go down
    cbefore = -INFINITY;
  }
}

template <bool REJ>
__global__ __launch_bounds__(64) void accept_walk_kernel(WalkArgs a) {
  const int b = blockIdx.x;
  const int lane = threadIdx.x;
  const int T = a.T;
  const bool live = lane < T;
  const int par = live ? a.parent[(int64_t)b * T + lane] : -2;
  const int tok = live ? a.tokens[(int64_t)b * T + lane] : -1;
  bool ok = !live || (lane == 0 ? par == -1 : (par >= 0 && par < lane));
  if (__any(!ok)) {
    if (lane == 0) report(a.dev_status, EV_DERR_PARENT);
    return;
  }
  if (__any(live && lane > 0 && (tok < 0 || tok >= a.V))) {
    if (lane == 0) report(a.dev_status, EV_DERR_TOKEN);
    return;
  }
  const int nc = a.n_chunks;
  int node = 0;
  int k = 0;
  int my_path = lane == 0 ? 0 : -1;    // lane m holds path[m]
  int my_out = -1;                      // lane m holds out_tokens[m]
  for (;;) {
    const int64_t row_id = (int64_t)b * T + node;
    const float *row = a.logits + row_id * a.V;
    const uint64_t kids = __ballot(live && par == node);
    int emitted;
    int next = -1;
    if (!REJ) {
      const GreedyStat *st = (const GreedyStat *)a.stats + row_id * nc;
      float v = -INFINITY;
      int i = INT_MAX;
      for (int c = lane; c < nc; c += 64) better(v, i, st[c].val, st[c].idx);
      wave_argmax(v, i);
      emitted = i;
      uint64_t match = kids & __ballot(live && tok == i);
      if (match) next = __ffsll((unsigned long long)match) - 1;
    } else {
      const RejStat *st = (const RejStat *)a.stats + row_id * nc;
      double M = -INFINITY;
      for (int c = lane; c < nc; c += 64) M = fmax(M, st[c].M);
      M = wave_max(M);
      double S = 0.0;
      for (int c = lane; c < nc; c += 64) S += st[c].S * exp(st[c].M - M);
      S = wave_sum(S);
      double Z = 1.0;
      uint64_t rej = 0;
      double prej = 0.0;                // lane c: p of its token if rejected here
      const double *u = a.uniforms + (int64_t)b * T;
      for (uint64_t kk = kids; kk; kk &= kk - 1) {
        int c = __ffsll((unsigned long long)kk) - 1;
        int x = __shfl(tok, c);
        if (__ballot(((rej >> lane) & 1) && tok == x)) continue;   // already rejected here
        double p = prob(row, x, a.inv_tau, M, S);
        if (u[c] * Z < p) {
          next = c;
          break;
        }
        rej |= 1ull << c;
        if (lane == c) prej = p;
        Z -= p;
      }
      if (next >= 0) {
        emitted = __shfl(tok, next);
      } else {
        emitted = residual_draw(a, row, st, M, S, rej, tok, prej, u[0] * Z);
      }
    }
    if (lane == k) my_out = emitted;
    if (next < 0) break;
    ++k;
    if (lane == k) my_path = next;
    node = next;
  }
  if (live) {
    a.path[(int64_t)b * T + lane] = my_path;
    a.out_tokens[(int64_t)b * T + lane] = my_out;
  }
  if (lane == 0) a.accept_len[b] = k;
}

static ev_status check_common(const float *logits, const int32_t *tokens, const int32_t *parent,
                              int32_t B, int32_t T, int32_t V, int32_t *accept_len,
                              int32_t *path, int32_t *out_tokens, void *ws, size_t ws_bytes) {
  if (B < 0 || T < 1 || T > kMaxNodes || V < 1 || V > 64 * 4 * kChunk) return EV_ERR_SHAPE;
  if (B == 0) return EV_OK;
  if (!logits || !tokens || !parent || !accept_len || !path || !out_tokens) return EV_ERR_NULL;
  size_t need = (size_t)B * T * n_chunks_of(V) * sizeof(RejStat);
  if (ws_bytes < need || !ws) return EV_ERR_WORKSPACE;
  return EV_OK;
}

}  // namespace ev

EV_API size_t ev_accept_workspace(int32_t B, int32_t T, int32_t V) {
  if (B < 1 || T < 1 || V < 1) return 0;
  return (size_t)B * T * ev::n_chunks_of(V) * sizeof(ev::RejStat);
}

EV_API ev_status ev_accept_greedy(const float *logits, const int32_t *tokens, const int32_t *parent,
                                  int32_t B, int32_t T, int32_t V, int32_t *accept_len,
                                  int32_t *path, int32_t *out_tokens, void *ws, size_t ws_bytes,
                                  int32_t *dev_status, hipStream_t stream) {
  ev_status st = ev::check_common(logits, tokens, parent, B, T, V, accept_len, path, out_tokens,
                                  ws, ws_bytes);
  if (st != EV_OK || B == 0) return st;
  const int nc = ev::n_chunks_of(V);
  dim3 grid((nc + ev::kChunksPerWG - 1) / ev::kChunksPerWG, B * T);
  hipLaunchKernelGGL(ev::accept_stats_kernel<false>, grid, dim3(256), 0, stream, logits, V, nc,
                     0.0, ws);
  ev::WalkArgs a{logits, tokens, parent, T, V, nc, 0.0, nullptr, ws,
                 accept_len, path, out_tokens, dev_status};
  hipLaunchKernelGGL(ev::accept_walk_kernel<false>, dim3(B), dim3(64), 0, stream, a);
  return ev::launch_status();
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
  const int nc = ev::n_chunks_of(V);
  const double inv_tau = 1.0 / (double)temperature;
  dim3 grid((nc + ev::kChunksPerWG - 1) / ev::kChunksPerWG, B * T);
  hipLaunchKernelGGL(ev::accept_stats_kernel<true>, grid, dim3(256), 0, stream, logits, V, nc,
                     inv_tau, ws);
  ev::WalkArgs a{logits, tokens, parent, T, V, nc, inv_tau, uniforms, ws,
                 accept_len, path, out_tokens, dev_status};
  hipLaunchKernelGGL(ev::accept_walk_kernel<true>, dim3(B), dim3(64), 0, stream, a);
  return ev::launch_status();
}
