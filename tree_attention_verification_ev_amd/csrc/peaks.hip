// Calibration kernels: the bf16 matrix-core rate and the copy bandwidth one MI355X
// sustains, measured so that rooflines can be stated against the box as well as against
// the published peaks.  Not part of the verification pass.
#include "ev_internal.h"
#include "ev_peaks.h"

namespace ev {

// Four independent accumulators per wavefront, so consecutive products never wait on
// each other; operands come from the thread index (not constants the compiler could fold).
__global__ __launch_bounds__(256) void mfma_peak_kernel(int iters, float *sink) {
  const int lane = threadIdx.x & 63;
  bf16x8 a, b;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = (__bf16)(0.001f * (float)((lane * 8 + i) & 127) - 0.06f);
    b[i] = (__bf16)(0.002f * (float)((lane * 3 + i * 5) & 63) - 0.05f);
  }
  f32x16 c0 = {}, c1 = {}, c2 = {}, c3 = {};
  for (int it = 0; it < iters; ++it) {
    c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c0, 0, 0, 0);
    c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(b, a, c1, 0, 0, 0);
    c2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, a, c2, 0, 0, 0);
    c3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(b, b, c3, 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < 16; ++i) s += c0[i] + c1[i] + c2[i] + c3[i];
  if (threadIdx.x == 0) sink[blockIdx.x] = s;
}

// Grid-stride copy, four 16-byte pieces in flight per thread, non-temporal on both sides
// (the fastest of the shapes tried on MI355X: 5.2 TB/s against 4.7-4.8 for cached copies).
__global__ __launch_bounds__(256) void copy_peak_kernel(const u32x4 *src, u32x4 *dst, size_t n) {
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  for (; i + 3 * stride < n; i += 4 * stride) {
    u32x4 x[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) x[u] = __builtin_nontemporal_load(src + i + u * stride);
#pragma unroll
    for (int u = 0; u < 4; ++u) __builtin_nontemporal_store(x[u], dst + i + u * stride);
  }
  for (; i < n; i += stride) dst[i] = src[i];
}

// Grid-stride read of n 16-byte pieces, four in flight per thread, folded by XOR into one
// word per workgroup (sink) so that the loads stay live.
__global__ __launch_bounds__(256) void read_peak_kernel(const u32x4 *src, size_t n, uint32_t *sink) {
  __shared__ uint32_t red[256];
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  u32x4 acc = {};
  for (; i + 3 * stride < n; i += 4 * stride) {
    u32x4 x[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) x[u] = __builtin_nontemporal_load(src + i + u * stride);
#pragma unroll
    for (int u = 0; u < 4; ++u) acc ^= x[u];
  }
  for (; i < n; i += stride) acc ^= src[i];
  red[threadIdx.x] = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t r = 0;
    for (int t = 0; t < 256; ++t) r ^= red[t];
    sink[blockIdx.x] = r;
  }
}

}  // namespace ev

EV_API ev_status ev_peak_mfma_bf16(int32_t n_workgroups, int32_t iters, float *sink,
                                   hipStream_t stream) {
  if (n_workgroups < 1 || iters < 1) return EV_ERR_SHAPE;
  if (!sink) return EV_ERR_NULL;
  hipLaunchKernelGGL(ev::mfma_peak_kernel, dim3(n_workgroups), dim3(256), 0, stream, iters, sink);
  return ev::launch_status();
}

EV_API ev_status ev_peak_copy(const void *src, void *dst, size_t bytes, hipStream_t stream) {
  if (!src || !dst) return EV_ERR_NULL;
  if (((uintptr_t)src | (uintptr_t)dst | bytes) & 15) return EV_ERR_ARG;
  if (bytes == 0) return EV_OK;
  const size_t n = bytes / 16;
  const unsigned grid = (unsigned)std::min<size_t>((n + 255) / 256, 64 * 256);
  hipLaunchKernelGGL(ev::copy_peak_kernel, dim3(grid), dim3(256), 0, stream,
                     (const ev::u32x4 *)src, (ev::u32x4 *)dst, n);
  return ev::launch_status();
}

EV_API ev_status ev_peak_read(const void *src, size_t bytes, uint32_t *sink, int32_t n_workgroups,
                              hipStream_t stream) {
  if (!src || !sink) return EV_ERR_NULL;
  if (((uintptr_t)src | bytes) & 15) return EV_ERR_ARG;
  if (n_workgroups < 1) return EV_ERR_SHAPE;
  if (bytes == 0) return EV_OK;
  hipLaunchKernelGGL(ev::read_peak_kernel, dim3(n_workgroups), dim3(256), 0, stream,
                     (const ev::u32x4 *)src, bytes / 16, sink);
  return ev::launch_status();
}
