// State checkpoint / rollback: a plain device copy of fp32 states ("xhh.club" tag page
// 结构, entry on the structure's system implications: state rollback is one of KDA's
// three execution forms, and the prefix cache keeps state checkpoints).
//
// The indexed copy moves whole states between slots of two state arrays (a serving
// pool, a batch, the checkpoints of a prefill, or pinned host memory for write-back):
// dst[dst_slots[i]] = src[src_slots[i]].
#include "internal.h"
#include "kda_device.h"

namespace kda {
namespace {

typedef float v4f __attribute__((ext_vector_type(4)));

// Non-temporal stores: a copy writes each line once and does not read it back.  With
// them and at most 1024 workgroups a 1 GiB copy reaches about 6 TB/s on MI355X (5.2 TB/s
// with ordinary stores and 4096 workgroups).
__global__ __launch_bounds__(256) void copy_vec4(float4 *__restrict__ dst,
                                                 const float4 *__restrict__ src, int64_t n4) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n4; i += stride) {
    const float4 v = src[i];
    __builtin_nontemporal_store(v4f{v.x, v.y, v.z, v.w}, reinterpret_cast<v4f *>(dst + i));
  }
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

// One workgroup copies one 16 KiB piece (1024 float4) of one state pair; the pair and
// the piece come from the block index, so there is no per-element division.
__global__ __launch_bounds__(256) void copy_indexed_vec4(float4 *__restrict__ dst,
                                                         const int32_t *__restrict__ dst_slots,
                                                         int64_t dst_count,
                                                         const float4 *__restrict__ src,
                                                         const int32_t *__restrict__ src_slots,
                                                         int64_t src_count, int64_t elems4,
                                                         int64_t pieces) {
  const int64_t blk = blockIdx.x;
  const int64_t i = blk / pieces, piece = blk % pieces;
  const int64_t d = dst_slots ? (int64_t)dst_slots[i] : i;
  const int64_t s = src_slots ? (int64_t)src_slots[i] : i;
  if (d < 0 || d >= dst_count || s < 0 || s >= src_count) return;
  const int64_t begin = piece * 1024, end = begin + 1024 < elems4 ? begin + 1024 : elems4;
  float4 *out = dst + d * elems4;
  const float4 *in = src + s * elems4;
  for (int64_t x = begin + threadIdx.x; x < end; x += 256) out[x] = in[x];
}

__global__ __launch_bounds__(256) void copy_indexed_scalar(float *__restrict__ dst,
                                                           const int32_t *__restrict__ dst_slots,
                                                           int64_t dst_count,
                                                           const float *__restrict__ src,
                                                           const int32_t *__restrict__ src_slots,
                                                           int64_t src_count, int64_t elems,
                                                           int64_t pieces) {
  const int64_t blk = blockIdx.x;
  const int64_t i = blk / pieces, piece = blk % pieces;
  const int64_t d = dst_slots ? (int64_t)dst_slots[i] : i;
  const int64_t s = src_slots ? (int64_t)src_slots[i] : i;
  if (d < 0 || d >= dst_count || s < 0 || s >= src_count) return;
  const int64_t begin = piece * 1024, end = begin + 1024 < elems ? begin + 1024 : elems;
  for (int64_t x = begin + threadIdx.x; x < end; x += 256) dst[d * elems + x] = src[s * elems + x];
}

unsigned grid_for(int64_t n) {
  const int64_t blocks = (n + 255) / 256;
  return static_cast<unsigned>(blocks < 1024 ? (blocks < 1 ? 1 : blocks) : 1024);
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

hipError_t launch_state_copy_indexed(float *dst, const int32_t *dst_slots, int64_t dst_count,
                                     const float *src, const int32_t *src_slots, int64_t src_count,
                                     int64_t n, int64_t elems, hipStream_t s) {
  if (n <= 0 || elems <= 0) return hipSuccess;
  const bool aligned = ((reinterpret_cast<uintptr_t>(dst) | reinterpret_cast<uintptr_t>(src)) & 15u) == 0;
  if (aligned && (elems & 3) == 0) {
    const int64_t elems4 = elems / 4, pieces = (elems4 + 1023) / 1024;
    hipLaunchKernelGGL(copy_indexed_vec4, dim3(static_cast<unsigned>(n * pieces)), dim3(256), 0, s,
                       reinterpret_cast<float4 *>(dst), dst_slots, dst_count,
                       reinterpret_cast<const float4 *>(src), src_slots, src_count, elems4, pieces);
  } else {
    const int64_t pieces = (elems + 1023) / 1024;
    hipLaunchKernelGGL(copy_indexed_scalar, dim3(static_cast<unsigned>(n * pieces)), dim3(256), 0, s,
                       dst, dst_slots, dst_count, src, src_slots, src_count, elems, pieces);
  }
  return hipGetLastError();
}

hipError_t launch_fill_zero(float *dst, int64_t n, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(fill_zero, dim3(grid_for(n)), dim3(256), 0, s, dst, n);
  return hipGetLastError();
}

}  // namespace kda
