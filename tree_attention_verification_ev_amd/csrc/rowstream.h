// Device helpers for kernels that stream logit rows in 1024-logit chunks, one chunk per
// wavefront, and hand results between the workgroups of a launch through arrival
// counters: chunk loads, float64 exp, wave-wide DPP reductions, agent-scope publication
// and the counter slots.
#pragma once

#include <limits.h>
#include <math.h>

#include "ev_internal.h"

namespace ev {

constexpr int kChunk = 1024;       // logits per wavefront chunk (16 per lane)
constexpr int kChunksPerWG = 4;    // wavefronts per workgroup (one chunk each per step)

struct GreedyStat {                      // stored as one 64-bit word: value bits, index
  float val;
  int idx;
};
__device__ inline uint64_t pack(GreedyStat g) {
  return (uint64_t)__float_as_uint(g.val) | ((uint64_t)(uint32_t)g.idx << 32);
}
__device__ inline GreedyStat unpack(uint64_t w) {
  return GreedyStat{__uint_as_float((uint32_t)w), (int)(uint32_t)(w >> 32)};
}
struct RejStat {
  double M;
  double S;
};

__host__ __device__ inline int n_chunks_of(int V) { return (V + kChunk - 1) / kChunk; }

// exp(x) for x <= 0 in float64 by the table-driven method of P. T. P. Tang (ACM TOMS 15(2),
// 1989): x = (N m + j) ln2/N + r with |r| <= ln2/(2N), exp(x) = 2^m 2^(j/N) exp(r), the
// last factor by its Taylor polynomial: to r^4 with N = 256 (kExpTabBits 8), to r^5 with
// N = 64 (6); truncation below 4e-17 either way.  tab[j] = 2^(j/N).  The larger table saves
// a float64 FMA per argument (the statistics streams: acceptance 3-5 % faster); the small
// latency-bound draft-tree launches were 2.5 % slower with it, so they keep N = 64.  The nearest integer to
// N x / ln2 comes from adding and removing 1.5 * 2^52, whose low word then holds it as a
// two's-complement integer.  Arguments below -745 (results below the smallest subnormal)
// are clamped there, so they return at most 5e-324.  The method in two halves, so that a
// caller can issue the table reads of several arguments before it combines any of them
// (each read is an LDS round trip): exp_nonpos(x) = exp_join(exp_split(x), tab[exp_slot(k)]).
constexpr int kExpTabBits = 8;                 // the acceptance kernels' table
constexpr int kExpTab = 1 << kExpTabBits;
template <int TB> struct ExpReduction;
template <> struct ExpReduction<8> {
  static constexpr double kInvLn2xN = 369.3299304675746;     // 256 / ln 2
  static constexpr double kLn2dNHi = 0.0027076061740622863;  // ln2/256 rounded to double
  static constexpr double kLn2dNLo = 9.058776616587108e-20;  // ln2/256 - kLn2dNHi
};
template <> struct ExpReduction<6> {
  static constexpr double kInvLn2xN = 92.33248261689366;     // 64 / ln 2
  static constexpr double kLn2dNHi = 0.010830424696249145;   // ln2/64 rounded to double
  static constexpr double kLn2dNLo = 3.623510646634843e-19;  // ln2/64 - kLn2dNHi
};
struct ExpParts {
  double p;                                                   // exp(r) - 1
  int k;                                                      // 2^TB m + j
};
template <int TB = kExpTabBits>
__device__ inline ExpParts exp_split(double x) {
  using R = ExpReduction<TB>;
  constexpr double kShifter = 6755399441055744.0;             // 1.5 * 2^52
  x = fmax(x, -745.0);
  const double t = fma(x, R::kInvLn2xN, kShifter);
  const double kf = t - kShifter;
  const int k = (int)(uint32_t)__double_as_longlong(t);
  double r = fma(-kf, R::kLn2dNHi, x);
  r = fma(-kf, R::kLn2dNLo, r);
  double p;
  if constexpr (TB >= 8) {
    p = fma(r, 1.0 / 24.0, 1.0 / 6.0);
  } else {
    p = fma(r, 1.0 / 120.0, 1.0 / 24.0);
    p = fma(r, p, 1.0 / 6.0);
  }
  p = fma(r, p, 0.5);
  p = fma(r, p, 1.0);
  return ExpParts{p * r, k};
}
template <int TB = kExpTabBits>
__device__ inline int exp_slot(int k) { return k & ((1 << TB) - 1); }
template <int TB = kExpTabBits>
__device__ inline double exp_join(ExpParts e, double tj) {
  return ldexp(fma(tj, e.p, tj), e.k >> TB);
}
template <int TB = kExpTabBits>
__device__ inline double exp_nonpos(double x, const double *tab) {
  const ExpParts e = exp_split<TB>(x);
  return exp_join<TB>(e, tab[exp_slot<TB>(e.k)]);
}
// exp_nonpos of N arguments, their table reads issued together.
template <int N, int TB = kExpTabBits>
__device__ __forceinline__ void exp_nonpos_n(const double (&x)[N], double (&y)[N],
                                             const double *tab) {
  ExpParts ep[N];
  double tj[N];
#pragma unroll
  for (int i = 0; i < N; ++i) ep[i] = exp_split<TB>(x[i]);
#pragma unroll
  for (int i = 0; i < N; ++i) tj[i] = tab[exp_slot<TB>(ep[i].k)];
#pragma unroll
  for (int i = 0; i < N; ++i) y[i] = exp_join<TB>(ep[i], tj[i]);
}
// sum of exp_nonpos(x(e)), e = 0 .. N-1 in order, the table reads of every XB arguments
// issued before any of them is used (with XB = 1, one read at a time, each waited for
// before the next argument begins).  The arithmetic does not depend on XB.
template <int N, int XB, class F>
__device__ __forceinline__ double exp_sum(F x, const double *tab) {
  static_assert(N % XB == 0, "whole batches");
  double sum = 0.0;
#pragma unroll
  for (int h = 0; h < N; h += XB) {
    ExpParts ep[XB];
    double tj[XB];
#pragma unroll
    for (int e = 0; e < XB; ++e) ep[e] = exp_split(x(h + e));
#pragma unroll
    for (int e = 0; e < XB; ++e) tj[e] = tab[exp_slot(ep[e].k)];
#pragma unroll
    for (int e = 0; e < XB; ++e) sum += exp_join(ep[e], tj[e]);
  }
  return sum;
}

// s - M for a logit at inverse temperature inv_tau (one rounding).
__device__ inline double shifted(float logit, double inv_tau, double M) {
  return fma((double)logit, inv_tau, -M);
}

// Lane's 16 logits of chunk `base` are elements (k*64 + lane)*4 + e, k < 4, e < 4
// (coalesced).  load_chunk_raw only issues the loads: an element past the row's end loads
// an in-bounds address instead, and mask_chunk later turns it into -inf.  No load sits
// under a lane-dependent branch, and the selects come after the caller has issued its next
// loads.  (A per-lane branch around each load, with the selects inside it, made the
// compiler wait for every load in flight, a prefetched chunk's included, before each new
// load.)  VEC: V is a multiple of 4, so each 16-byte piece lies wholly inside the row or
// wholly past its end.  NT: non-temporal loads, for a row read once by a launch.
template <bool NT, bool VEC>
__device__ inline void load_chunk_raw(const float *row, int V, int base, float v[16]) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int i0 = base + (k * 64 + lane) * 4;
    if constexpr (VEC) {
      const f32x4 *p = (const f32x4 *)(row + min(i0, V - 4));
      const f32x4 x = NT ? __builtin_nontemporal_load(p) : *p;
#pragma unroll
      for (int e = 0; e < 4; ++e) v[4 * k + e] = x[e];
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) v[4 * k + e] = row[min(i0 + e, V - 1)];
    }
  }
}

__device__ inline void mask_chunk(int V, int base, float v[16], int idx[16]) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int k = 0; k < 4; ++k)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int i = base + (k * 64 + lane) * 4 + e;
      v[4 * k + e] = i < V ? v[4 * k + e] : -INFINITY;
      idx[4 * k + e] = i < V ? i : INT_MAX;
    }
}

// The same chunk of two rows: both rows' loads are in flight before either is masked.
__device__ inline void load_pair(const float *ra, const float *rb, int V, int base, bool vec_ok,
                                 float va[16], float vb[16], int idx[16]) {
  if (vec_ok) {
    load_chunk_raw<false, true>(ra, V, base, va);
    load_chunk_raw<false, true>(rb, V, base, vb);
  } else {
    load_chunk_raw<false, false>(ra, V, base, va);
    load_chunk_raw<false, false>(rb, V, base, vb);
  }
  mask_chunk(V, base, va, idx);
  mask_chunk(V, base, vb, idx);
}

// Both steps at once; vec_ok (V a multiple of 4) is the same for every lane.
__device__ inline void load_chunk(const float *row, int V, int base, bool vec_ok, float v[16],
                                  int idx[16]) {
  if (vec_ok) load_chunk_raw<false, true>(row, V, base, v);
  else load_chunk_raw<false, false>(row, V, base, v);
  mask_chunk(V, base, v, idx);
}

// (value, index) pairs: larger value wins, equal values keep the lower index (selects,
// no branches).
__device__ inline void better(float &v, int &i, float v2, int i2) {
  const bool take = (v2 > v) | ((v2 == v) & (i2 < i));
  v = take ? v2 : v;
  i = take ? i2 : i;
}

// Whole-wavefront reductions (every lane active).  Within each row of 16 lanes, DPP
// moves exchange with the neighbour in the pair, then the other pair of the quad, then
// the mirrored quad of the half-row, then the mirrored half of the row, so every lane of
// a row holds the row's result.  Two row broadcasts then fold row 0 into row 1 and row 2
// into row 3, and row 1 into row 3; lane 63 holds ((r3 . r2) . (r1 . r0)), read into a
// scalar.  The combination order is fixed, so results are reproducible.
constexpr int kDppQuadSwap1 = 0xB1;      // quad_perm [1,0,3,2]
constexpr int kDppQuadSwap2 = 0x4E;      // quad_perm [2,3,0,1]
constexpr int kDppHalfMirror = 0x141;    // row_half_mirror
constexpr int kDppMirror = 0x140;        // row_mirror
constexpr int kDppRowBcast15 = 0x142;    // lane 15 of each row to the next row
constexpr int kDppRowBcast31 = 0x143;    // lane 31 to rows 2 and 3
constexpr int kRows13 = 0xa;             // row masks
constexpr int kRows23 = 0xc;

template <int CTRL>
__device__ inline int dpp_i(int x) {
  return __builtin_amdgcn_mov_dpp(x, CTRL, 0xf, 0xf, true);
}
template <int CTRL>
__device__ inline float dpp_f(float x) {
  return __int_as_float(dpp_i<CTRL>(__float_as_int(x)));
}
template <int CTRL>
__device__ inline double dpp_d(double x) {
  const uint64_t b = (uint64_t)__double_as_longlong(x);
  const uint32_t lo = (uint32_t)dpp_i<CTRL>((int)(uint32_t)b);
  const uint32_t hi = (uint32_t)dpp_i<CTRL>((int)(uint32_t)(b >> 32));
  return __longlong_as_double((long long)(((uint64_t)hi << 32) | lo));
}
__device__ inline int lane_i(int x, int l) { return __builtin_amdgcn_readlane(x, l); }
__device__ inline float lane_f(float x, int l) { return __int_as_float(lane_i(__float_as_int(x), l)); }
__device__ inline double lane_d(double x, int l) {
  const uint64_t b = (uint64_t)__double_as_longlong(x);
  const uint32_t lo = (uint32_t)lane_i((int)(uint32_t)b, l);
  const uint32_t hi = (uint32_t)lane_i((int)(uint32_t)(b >> 32), l);
  return __longlong_as_double((long long)(((uint64_t)hi << 32) | lo));
}

// DPP move into the rows of ROWS only; lanes of the other rows receive `old`.
template <int CTRL, int ROWS>
__device__ inline int bcast_i(int old, int x) {
  return __builtin_amdgcn_update_dpp(old, x, CTRL, ROWS, 0xf, false);
}
template <int CTRL, int ROWS>
__device__ inline float bcast_f(float old, float x) {
  return __int_as_float(bcast_i<CTRL, ROWS>(__float_as_int(old), __float_as_int(x)));
}
template <int CTRL, int ROWS>
__device__ inline double bcast_d(double old, double x) {
  const uint64_t o = (uint64_t)__double_as_longlong(old), b = (uint64_t)__double_as_longlong(x);
  const uint32_t lo = (uint32_t)bcast_i<CTRL, ROWS>((int)(uint32_t)o, (int)(uint32_t)b);
  const uint32_t hi = (uint32_t)bcast_i<CTRL, ROWS>((int)(uint32_t)(o >> 32), (int)(uint32_t)(b >> 32));
  return __longlong_as_double((long long)(((uint64_t)hi << 32) | lo));
}

// Inclusive prefix sum over the 64 lanes: Hillis-Steele within each row of 16 (row_shr
// by 1, 2, 4, 8; lanes shifted in from outside the row read 0), then each row adds the
// totals of the rows before it.
template <int SHR>
__device__ inline double dpp_shr_d(double x) {
  return dpp_d<0x110 + SHR>(x);
}
__device__ inline double wave_inclusive_sum(double x) {
  x += dpp_shr_d<1>(x);
  x += dpp_shr_d<2>(x);
  x += dpp_shr_d<4>(x);
  x += dpp_shr_d<8>(x);
  const double t0 = lane_d(x, 15), t1 = lane_d(x, 31), t2 = lane_d(x, 47);
  const int row = (threadIdx.x & 63) >> 4;
  const double off = row == 0 ? 0.0 : row == 1 ? t0 : row == 2 ? t0 + t1 : (t0 + t1) + t2;
  return x + off;
}

template <int CTRL>
__device__ inline void argmax_step(float &v, int &i) {
  better(v, i, dpp_f<CTRL>(v), dpp_i<CTRL>(i));
}
__device__ inline void wave_argmax(float &v, int &i) {
  argmax_step<kDppQuadSwap1>(v, i);
  argmax_step<kDppQuadSwap2>(v, i);
  argmax_step<kDppHalfMirror>(v, i);
  argmax_step<kDppMirror>(v, i);
  better(v, i, bcast_f<kDppRowBcast15, kRows13>(-INFINITY, v), bcast_i<kDppRowBcast15, kRows13>(INT_MAX, i));
  better(v, i, bcast_f<kDppRowBcast31, kRows23>(-INFINITY, v), bcast_i<kDppRowBcast31, kRows23>(INT_MAX, i));
  v = lane_f(v, 63);
  i = lane_i(i, 63);
}

__device__ inline double wave_sum(double x) {
  x += dpp_d<kDppQuadSwap1>(x);
  x += dpp_d<kDppQuadSwap2>(x);
  x += dpp_d<kDppHalfMirror>(x);
  x += dpp_d<kDppMirror>(x);
  x += bcast_d<kDppRowBcast15, kRows13>(0.0, x);
  x += bcast_d<kDppRowBcast31, kRows23>(0.0, x);
  return lane_d(x, 63);
}

__device__ inline float wave_max_f(float x) {
  x = fmaxf(x, dpp_f<kDppQuadSwap1>(x));
  x = fmaxf(x, dpp_f<kDppQuadSwap2>(x));
  x = fmaxf(x, dpp_f<kDppHalfMirror>(x));
  x = fmaxf(x, dpp_f<kDppMirror>(x));
  x = fmaxf(x, bcast_f<kDppRowBcast15, kRows13>(-INFINITY, x));
  x = fmaxf(x, bcast_f<kDppRowBcast31, kRows23>(-INFINITY, x));
  return lane_f(x, 63);
}

__device__ inline float wave_sum_f(float x) {
  x += dpp_f<kDppQuadSwap1>(x);
  x += dpp_f<kDppQuadSwap2>(x);
  x += dpp_f<kDppHalfMirror>(x);
  x += dpp_f<kDppMirror>(x);
  x += bcast_f<kDppRowBcast15, kRows13>(0.f, x);
  x += bcast_f<kDppRowBcast31, kRows23>(0.f, x);
  return lane_f(x, 63);
}

__device__ inline double wave_max(double x) {
  x = fmax(x, dpp_d<kDppQuadSwap1>(x));
  x = fmax(x, dpp_d<kDppQuadSwap2>(x));
  x = fmax(x, dpp_d<kDppHalfMirror>(x));
  x = fmax(x, dpp_d<kDppMirror>(x));
  x = fmax(x, bcast_d<kDppRowBcast15, kRows13>(-INFINITY, x));
  x = fmax(x, bcast_d<kDppRowBcast31, kRows23>(-INFINITY, x));
  return lane_d(x, 63);
}

// 2^(j/N), j < N = 2^TB, into LDS, one entry per thread (every workgroup that calls it
// has at least 256 threads; a loop over blockDim made each launch fetch the dispatch
// packet first).
template <int TB = kExpTabBits>
__device__ inline void fill_exp_table(double *tab) {
  constexpr int N = 1 << TB;
  if (threadIdx.x < N) tab[threadIdx.x] = exp2((double)threadIdx.x / N);
}

// Data handed from one workgroup to another within a launch (chunk statistics, node
// outcomes) moves through agent-scope atomic stores and loads, which are coherent across
// the XCDs' separate L2 caches without the whole-L2 write-back and invalidate that an
// agent-scope fence costs.  A writer waits for its stores to complete before it bumps an
// arrival counter; a reader loads only after its own increment has returned the final
// count, so every store it reads has already reached the coherence point.
template <class X>
__device__ inline void publish(X *p, X v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
template <class X>
__device__ inline X observe(const X *p) {
  return __hip_atomic_load(const_cast<X *>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ inline void stores_complete() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// Returns true in the one workgroup whose arrival completes `expected` arrivals; that
// workgroup also resets the counter for the next call.  Call with the whole workgroup.
__device__ inline bool last_arrival(int32_t *cnt, int expected, int *s_flag) {
  stores_complete();
  __syncthreads();
  if (threadIdx.x == 0) {
    const int old = __hip_atomic_fetch_add(cnt, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const bool last = old == expected - 1;
    if (last) publish(cnt, 0);
    *s_flag = last;
  }
  __syncthreads();
  asm volatile("" ::: "memory");
  return *s_flag;
}

// Row statistics (max s, sum exp(s - max)) from chunk statistics held in registers: lane
// holds chunks lane, lane + 64, ... (kChunkRegs of them, so V <= 256 Ki logits).
constexpr int kChunkRegs = 4;
__device__ inline void row_stats_regs(const RejStat (&cs)[kChunkRegs], const double *tab,
                                      double &M, double &S) {
  M = -INFINITY;
#pragma unroll
  for (int r = 0; r < kChunkRegs; ++r) M = fmax(M, cs[r].M);
  M = wave_max(M);
  double x[kChunkRegs], e[kChunkRegs];
#pragma unroll
  for (int r = 0; r < kChunkRegs; ++r) x[r] = cs[r].M - M;
  exp_nonpos_n(x, e, tab);
  S = 0.0;
#pragma unroll
  for (int r = 0; r < kChunkRegs; ++r)
    if (cs[r].S > 0.0) S += cs[r].S * e[r];
  S = wave_sum(S);
}

// Workspace: the counters sit at fixed offsets at its start, sized for the largest
// launch (B * T <= 65535 rows, B <= 65535 sequences), so that a workspace left at zero by
// one call is still zero where a call of any other shape looks for its counters.
constexpr int kMaxRows = 65535;
constexpr size_t kCounterBytes = 2 * align_up((kMaxRows + 1) * sizeof(int32_t), 256);

// Counter slot of row (or sequence) r: up to 4096 consecutive ids land on distinct 64-byte
// lines (ids r and r + 4096 share one).  Arrivals on one line serialise in the memory
// system, so packing the counters of neighbouring rows together would make every
// workgroup of a launch queue on a handful of lines.
__device__ inline int counter_slot(int64_t r) { return (int)((r & 4095) * 16 + (r >> 12)); }

}  // namespace ev
