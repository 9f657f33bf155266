// Launchers shared between the host ABI layer (api.cpp) and the kernel files.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stddef.h>
#include <stdint.h>

#include "kda.h"

namespace kda {

constexpr int kCUs = 256;   // compute units of MI355X: launches aim at one workgroup per CU

// slots: null for the plain form (state [N, H, d_k, d_v]); else the pool slot of each
// sequence (state [pool, H, d_k, d_v]).
hipError_t launch_decode(const kda_decode_desc &d, const int32_t *slots, int32_t pool, hipStream_t s);
// dst[dst_slots[i]] = src[src_slots[i]] for i < n (identity where a slot array is null),
// states of `elems` floats; pairs with a slot outside [0, count) are skipped.
hipError_t launch_state_copy_indexed(float *dst, const int32_t *dst_slots, int64_t dst_count,
                                     const float *src, const int32_t *src_slots, int64_t src_count,
                                     int64_t n, int64_t elems, hipStream_t s);
hipError_t launch_state_copy(float *dst, const float *src, int64_t n_floats, hipStream_t s);
hipError_t launch_fill_zero(float *dst, int64_t n_floats, hipStream_t s);

// Execution plan of one prefill call, decided on the host.
struct PrefillPlan {
  int n_seg;        // segments per sequence (1 = no context parallelism)
  int seg_chunks;   // chunks per segment (last segment may be shorter)
  int n_chunks;     // chunks per sequence
  int v_split;      // workgroups per (sequence, head, segment) over the value columns
  bool split_norm;  // norm/gate epilogue runs as a separate pass (v_split > 1 with a gate)
  size_t ws_rec;    // bytes: per-chunk records [B,H,n_chunks] written by the prep kernel
  size_t ws_maps;   // bytes: segment maps [B,H,n_seg,d_k,2*d_v] fp32
  size_t ws_sin;    // bytes: states entering each segment [B,H,n_seg,d_k,d_v] fp32
  int scan_grp;     // segments per group of the scan (n_seg: a single chain)
  size_t ws_gmaps;  // bytes: composed maps of the scan's groups [B,H,groups-1,d_k,2 d_v] fp32
  size_t ws_norm;   // bytes: raw fp32 outputs [B,T,H,d_v] for the separate norm pass (bf16 out)
  size_t off_rec, off_maps, off_sin, off_gmaps, off_norm;   // byte offsets in the workspace
  size_t ws_total;
};

// Bytes of one per-chunk record (chunk 16 or 64; fp32 inputs use chunk 16).
size_t prefill_record_bytes(int chunk, bool f32);

// Pass 0 of the prefill: records of every (sequence, head, chunk).
hipError_t launch_prefill_prep(const kda_prefill_desc &d, int n_chunks, void *records, hipStream_t s);

hipError_t launch_prefill(const kda_prefill_desc &d, const PrefillPlan &p, hipStream_t s);

// Backward pass: workspace bytes, and the four kernels (chunk quantities, state sweep,
// gradient sweep, per-chunk gradients) on the stream.
size_t backward_workspace_bytes(int B, int T, int H);
hipError_t launch_backward(const kda_backward_desc &d, hipStream_t s);

}  // namespace kda
