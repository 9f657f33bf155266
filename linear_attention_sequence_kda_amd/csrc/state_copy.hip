// State checkpoint / rollback: a plain device copy of fp32 states ("xhh.club" tag page
// 结构, entry on the structure's system implications: state rollback is one of KDA's
// three execution forms, and the prefix cache keeps state checkpoints).
#include "internal.h"
#include "kda_device.h"

namespace kda {
namespace {

__global__ __launch_bounds__(256) void copy_vec4(float4 *__restrict__ dst,
                                                 const float4 *__restrict__ src, int64_t n4) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n4; i += stride)
    dst[i] = src[i];
}

__global__ __launch_bounds__(256) void copy_scalar(float *__restrict__ dst,
                                                   const float *__restrict__ src, int64_t n) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride)
    dst[i] = src[i];
}

__global__ __launch_bounds__(256) void fill_zero(float *__restrict__ dst, int64_t n) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride) dst[i] = 0.f;
}

unsigned grid_for(int64_t n) {
  const int64_t blocks = (n + 255) / 256;
  return static_cast<unsigned>(blocks < 4096 ? (blocks < 1 ? 1 : blocks) : 4096);
}

}  // namespace

hipError_t launch_state_copy(float *dst, const float *src, int64_t n, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  const bool aligned = ((reinterpret_cast<uintptr_t>(dst) | reinterpret_cast<uintptr_t>(src)) & 15u) == 0;
  if (aligned && (n & 3) == 0) {
    const int64_t n4 = n / 4;
    hipLaunchKernelGGL(copy_vec4, dim3(grid_for(n4)), dim3(256), 0, s,
                       reinterpret_cast<float4 *>(dst), reinterpret_cast<const float4 *>(src), n4);
  } else {
    hipLaunchKernelGGL(copy_scalar, dim3(grid_for(n)), dim3(256), 0, s, dst, src, n);
  }
  return hipGetLastError();
}

hipError_t launch_fill_zero(float *dst, int64_t n, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(fill_zero, dim3(grid_for(n)), dim3(256), 0, s, dst, n);
  return hipGetLastError();
}

}  // namespace kda
