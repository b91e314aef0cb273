// Internal helpers shared by the gfx950 kernels and their host launchers.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "ev.h"

#define EV_API extern "C" __attribute__((visibility("default")))

namespace ev {

constexpr int kWave = 64;
constexpr int kMaxNodes = 64;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// First device error wins.
__device__ inline void report(int32_t *dev_status, int32_t code) {
  if (dev_status) atomicCAS(dev_status, 0, code);
}

// Element offset of logical slot `slot` of sequence b, KV head g, in a cache layer.
// Returns -1 when the slot's block id is out of range (paged) — the caller must not read.
struct KvAddr {
  int paged;
  int hkv;
  int d;
  int64_t cap;
  const int32_t *table;
  int block_shift;   // log2(block_size)
  int max_blocks;
  int n_blocks;

  __device__ inline int64_t slot_offset(int b, int g, int slot) const {
    if (!paged) return ((int64_t)(b * hkv + g) * cap + slot) * d;
    int blk = table[(int64_t)b * max_blocks + (slot >> block_shift)];
    if (blk < 0 || blk >= n_blocks) return -1;
    int bs = 1 << block_shift;
    return (((int64_t)blk * hkv + g) * bs + (slot & (bs - 1))) * d;
  }

  // Can slots [0, n) of sequence b exist in this cache?
  __device__ inline bool fits(int n) const {
    if (!paged) return n <= cap;
    return ((n + (1 << block_shift) - 1) >> block_shift) <= max_blocks;
  }
};

inline int ilog2_exact(int x) {
  int s = 0;
  while ((1 << s) < x) ++s;
  return (1 << s) == x ? s : -1;
}

// Host-side validation of a KV descriptor; fills `a` on success.
inline ev_status make_kv_addr(const ev_kv_desc *kv, KvAddr *a) {
  if (!kv || !kv->k || !kv->v) return EV_ERR_NULL;
  if (kv->dtype != EV_F32 && kv->dtype != EV_BF16 && kv->dtype != EV_INT4) return EV_ERR_DTYPE;
  if (kv->dtype == EV_INT4 && (!kv->k_scale || !kv->v_scale)) return EV_ERR_NULL;
  if (kv->n_kv_heads < 1 || (kv->head_dim != 64 && kv->head_dim != 128)) return EV_ERR_SHAPE;
  if (kv->n_layers < 1) return EV_ERR_SHAPE;
  a->paged = kv->paged ? 1 : 0;
  a->hkv = kv->n_kv_heads;
  a->d = kv->head_dim;
  a->cap = kv->cap;
  a->table = kv->block_table;
  a->block_shift = 0;
  a->max_blocks = kv->max_blocks_per_seq;
  a->n_blocks = kv->n_blocks;
  if (a->paged) {
    if (!kv->block_table) return EV_ERR_NULL;
    int s = kv->block_size >= 1 && kv->block_size <= 256 ? ilog2_exact(kv->block_size) : -1;
    if (s < 0 || kv->max_blocks_per_seq < 1 || kv->n_blocks < 1) return EV_ERR_SHAPE;
    a->block_shift = s;
  } else {
    if (kv->cap < 1) return EV_ERR_SHAPE;
  }
  return EV_OK;
}

inline ev_status launch_status() {
  return hipGetLastError() == hipSuccess ? EV_OK : EV_ERR_LAUNCH;
}

constexpr size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// Workgroup barrier for LDS data only: waits for this wave's LDS operations, not for its
// global loads in flight (__syncthreads waits for those as well).
// A lane's value combined with that of the lane 32 away (the other half of the wavefront),
// through the cross-half swap of gfx950: a vector-unit operation, where a shuffle
// (ds_bpermute) is an LDS round trip.  Lane l < 32 gets op(x[l], x[l+32]), lane l >= 32
// op(x[l-32], x[l]), so both halves hold the same bits.
__device__ __forceinline__ float halves_max(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float halves_sum(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Uses each value in scalar registers at this point of the program.  Listing the kernel
// arguments a prologue needs here makes the compiler fetch them in one batch at entry,
// where it would otherwise load each where it is first used, a dependent round trip
// through the scalar cache each time.
template <typename T>
__device__ __forceinline__ void in_sgprs(T x) {
  asm volatile("" ::"s"(x));
}
template <typename... Ts>
__device__ __forceinline__ void args_in_sgprs(const Ts &...xs) {
  (in_sgprs(xs), ...);
}

// A uniform load through the scalar cache: from the constant address space the compiler
// may use a scalar load even after stores or inline assembly earlier in the kernel (read
// through a global pointer there, it issues a vector load).  Only for data no kernel of
// the call writes.
template <typename T>
__device__ __forceinline__ T scalar_load(const T *p, int64_t i) {
  return ((const __attribute__((address_space(4))) T *)p)[i];
}

}  // namespace ev
