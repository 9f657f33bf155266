// MFMA operand plumbing shared by the chunkwise prefill kernels (gfx950, wave64).
//
// MFMA 16x16x32 (f16/bf16) operand layouts:  A operand: lane l holds row (l & 15),
// contraction indices 8(l >> 4) .. +7;  B operand: column (l & 15), same indices;
// result (D): lane l holds rows 4(l >> 4) + r, r = 0..3, column (l & 15).
#pragma once

#include <type_traits>

#include "kda_device.h"

namespace kda {

constexpr int D = 128;          // d_k = d_v
constexpr int NTHREADS = 256;   // 4 waves per workgroup

typedef __attribute__((__vector_size__(8 * sizeof(float)))) float f32x8;

// ---------------------------------------------------------------------------
// operand types and the 16x16 (x K=32) MFMA step
// ---------------------------------------------------------------------------
template <bool F32> struct Op;
template <> struct Op<false> {   // fp16 operands
  using T = _Float16;
  using V8 = f16x8;
  static __device__ __forceinline__ T cvt(float x) { return static_cast<_Float16>(x); }
  static __device__ __forceinline__ f32x4 mma(f32x4 c, V8 a, V8 b) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
  }
  static __device__ __forceinline__ V8 load(const T *p) { return *reinterpret_cast<const V8 *>(p); }
  static __device__ __forceinline__ void store(T *p, V8 v) { *reinterpret_cast<V8 *>(p) = v; }
};
template <> struct Op<true> {    // fp32 operands
  using T = float;
  using V8 = f32x8;
  static __device__ __forceinline__ T cvt(float x) { return x; }
  // The 32-long contraction as 8 MFMAs of K=4.  Lane group g supplies contraction
  // index 8g+e to MFMA e (the same permutation on both operands).
  static __device__ __forceinline__ f32x4 mma(f32x4 c, V8 a, V8 b) {
#pragma unroll
    for (int e = 0; e < 8; ++e) c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[e], b[e], c, 0, 0, 0);
    return c;
  }
  static __device__ __forceinline__ V8 load(const T *p) {
    const float4 a = reinterpret_cast<const float4 *>(p)[0], b = reinterpret_cast<const float4 *>(p)[1];
    return V8{a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
  }
  static __device__ __forceinline__ void store(T *p, V8 v) {
    reinterpret_cast<float4 *>(p)[0] = make_float4(v[0], v[1], v[2], v[3]);
    reinterpret_cast<float4 *>(p)[1] = make_float4(v[4], v[5], v[6], v[7]);
  }
};

__device__ __forceinline__ f32x4 zero4() { return f32x4{0.f, 0.f, 0.f, 0.f}; }

// Swizzled row-major LDS buffer.  Element (row, col) of a row of ROWLEN elements sits
// in 16-byte chunk (col / EPC) XOR (row mod min(16, chunks per row)) of its row, so
// lanes that read or write the same logical column of consecutive rows hit distinct
// banks.
template <typename T, int ROWLEN>
struct Swz {
  static constexpr int EPC = 16 / (int)sizeof(T);      // elements per 16-byte chunk
  static constexpr int NCH = ROWLEN / EPC;             // chunks per row
  static constexpr int MASK = (NCH < 16 ? NCH : 16) - 1;
  static __device__ __forceinline__ int at(int row, int col) {
    return row * ROWLEN + (((col / EPC) ^ (row & MASK)) * EPC) + (col % EPC);
  }
};

typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

// Operand read, normal form: lane l gets 8 consecutive elements of row row0 + (l&15)
// starting at column k0 + 8(l>>4)  (an [m][k] or [n][k] buffer, k contiguous).
template <bool F32, int RL>
__device__ __forceinline__ typename Op<F32>::V8 ld_n(const typename Op<F32>::T *buf, int row0, int k0, int lane) {
  using S = Swz<typename Op<F32>::T, RL>;
  const int row = row0 + (lane & 15), col = k0 + 8 * (lane >> 4);
  if constexpr (F32) {
    const float4 a = *reinterpret_cast<const float4 *>(buf + S::at(row, col));
    const float4 b = *reinterpret_cast<const float4 *>(buf + S::at(row, col + 4));
    return typename Op<F32>::V8{a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
  } else {
    return *reinterpret_cast<const typename Op<F32>::V8 *>(buf + S::at(row, col));
  }
}

// Operand read, transposed form: from a [k][m] buffer (m contiguous), lane l gets
// X[k0 + 8(l>>4) + e][m0 + (l&15)], e = 0..7.  For 16-bit data this is two LDS
// transpose reads: within each 16-lane group, lanes 4e..4e+3 address the four 8-byte
// words of row e and lane j receives column j of those four rows.
template <bool F32, int RL>
__device__ __forceinline__ typename Op<F32>::V8 ld_t(const typename Op<F32>::T *buf, int k0, int m0, int lane) {
  using S = Swz<typename Op<F32>::T, RL>;
  const int g = lane >> 4;
  if constexpr (F32) {
    typename Op<F32>::V8 v;
    const int m = m0 + (lane & 15);
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = buf[S::at(k0 + 8 * g + e, m)];
    return v;
  } else {
    const int q = lane & 15, e4 = q >> 2, w = q & 3;
    const _Float16 *p0 = buf + S::at(k0 + 8 * g + e4, m0 + 4 * w);
    const _Float16 *p1 = buf + S::at(k0 + 8 * g + 4 + e4, m0 + 4 * w);
    const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)(p0));
    const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)(p1));
    const f16x4 a = __builtin_bit_cast(f16x4, lo), b = __builtin_bit_cast(f16x4, hi);
    return typename Op<F32>::V8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
  }
}

// The same two reads with the contraction index in split order: lane group g's eight
// elements are contraction indices k0 + 4g + (0..3) and k0 + 16 + 4g + (0..3).  In
// this order the two 16x16 MFMA result tiles covering rows k0..k0+15 and
// k0+16..k0+31 give the lane exactly its operand elements (lane (l&15, g) holds rows
// 4g..4g+3 of each tile), so results feed later products without leaving registers.
// Every operand of the state recurrence uses this order.
template <bool F32, int RL>
__device__ __forceinline__ typename Op<F32>::V8 ld_n_split(const typename Op<F32>::T *buf, int row0, int k0, int lane) {
  using S = Swz<typename Op<F32>::T, RL>;
  const int row = row0 + (lane & 15), g = lane >> 4;
  if constexpr (F32) {
    const float4 a = *reinterpret_cast<const float4 *>(buf + S::at(row, k0 + 4 * g));
    const float4 b = *reinterpret_cast<const float4 *>(buf + S::at(row, k0 + 16 + 4 * g));
    return typename Op<F32>::V8{a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
  } else {
    const f16x4 a = *reinterpret_cast<const f16x4 *>(buf + S::at(row, k0 + 4 * g));
    const f16x4 b = *reinterpret_cast<const f16x4 *>(buf + S::at(row, k0 + 16 + 4 * g));
    return typename Op<F32>::V8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
  }
}

template <bool F32, int RL>
__device__ __forceinline__ typename Op<F32>::V8 ld_t_split(const typename Op<F32>::T *buf, int k0, int m0, int lane) {
  using S = Swz<typename Op<F32>::T, RL>;
  const int g = lane >> 4;
  if constexpr (F32) {
    typename Op<F32>::V8 v;
    const int m = m0 + (lane & 15);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      v[e] = buf[S::at(k0 + 4 * g + e, m)];
      v[4 + e] = buf[S::at(k0 + 16 + 4 * g + e, m)];
    }
    return v;
  } else {
    const int q = lane & 15, e4 = q >> 2, w = q & 3;
    const _Float16 *p0 = buf + S::at(k0 + 4 * g + e4, m0 + 4 * w);
    const _Float16 *p1 = buf + S::at(k0 + 16 + 4 * g + e4, m0 + 4 * w);
    const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)(p0));
    const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)(p1));
    const f16x4 a = __builtin_bit_cast(f16x4, lo), b = __builtin_bit_cast(f16x4, hi);
    return typename Op<F32>::V8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
  }
}

// Operand in split order from two 16x16 results in MFMA output layout: x holds rows
// k0..k0+15, y rows k0+16..k0+31 (see ld_n_split).
template <bool F32>
__device__ __forceinline__ typename Op<F32>::V8 frag_from(f32x4 x, f32x4 y) {
  using T = typename Op<F32>::T;
  return typename Op<F32>::V8{(T)x[0], (T)x[1], (T)x[2], (T)x[3], (T)y[0], (T)y[1], (T)y[2], (T)y[3]};
}

// store 4 consecutive elements (row, col..col+3), col a multiple of 4
template <bool F32, int RL>
__device__ __forceinline__ void st4(typename Op<F32>::T *buf, int row, int col, float x0, float x1, float x2, float x3) {
  using S = Swz<typename Op<F32>::T, RL>;
  if constexpr (F32) {
    *reinterpret_cast<float4 *>(buf + S::at(row, col)) = make_float4(x0, x1, x2, x3);
  } else {
    *reinterpret_cast<f16x4 *>(buf + S::at(row, col)) =
        f16x4{(_Float16)x0, (_Float16)x1, (_Float16)x2, (_Float16)x3};
  }
}

// store 8 consecutive elements (row, col..col+7), col a multiple of 8
template <bool F32, int RL>
__device__ __forceinline__ void st8(typename Op<F32>::T *buf, int row, int col, const float *x) {
  using S = Swz<typename Op<F32>::T, RL>;
  if constexpr (F32) {
    *reinterpret_cast<float4 *>(buf + S::at(row, col)) = make_float4(x[0], x[1], x[2], x[3]);
    *reinterpret_cast<float4 *>(buf + S::at(row, col + 4)) = make_float4(x[4], x[5], x[6], x[7]);
  } else {
    *reinterpret_cast<f16x8 *>(buf + S::at(row, col)) =
        f16x8{(_Float16)x[0], (_Float16)x[1], (_Float16)x[2], (_Float16)x[3],
              (_Float16)x[4], (_Float16)x[5], (_Float16)x[6], (_Float16)x[7]};
  }
}

// ---------------------------------------------------------------------------
// 8 consecutive inputs of a bf16 or fp32 tensor (bf16 kept packed until used)
// ---------------------------------------------------------------------------
template <bool F32>
using Q8 = typename std::conditional<F32, f32x8, uint4>::type;

template <bool F32>
__device__ __forceinline__ Q8<F32> load_q8(const void *p, size_t idx) {
  if constexpr (F32) {
    const float4 a = *reinterpret_cast<const float4 *>(static_cast<const float *>(p) + idx);
    const float4 b = *reinterpret_cast<const float4 *>(static_cast<const float *>(p) + idx + 4);
    return f32x8{a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
  } else {
    return *reinterpret_cast<const uint4 *>(static_cast<const uint16_t *>(p) + idx);
  }
}

// 8 inputs in split order: elements idx .. idx+3 and idx+16 .. idx+19
template <bool F32>
__device__ __forceinline__ Q8<F32> load_q8_split(const void *p, size_t idx) {
  if constexpr (F32) {
    const float4 a = *reinterpret_cast<const float4 *>(static_cast<const float *>(p) + idx);
    const float4 b = *reinterpret_cast<const float4 *>(static_cast<const float *>(p) + idx + 16);
    return f32x8{a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
  } else {
    const uint2 a = *reinterpret_cast<const uint2 *>(static_cast<const uint16_t *>(p) + idx);
    const uint2 b = *reinterpret_cast<const uint2 *>(static_cast<const uint16_t *>(p) + idx + 16);
    return make_uint4(a.x, a.y, b.x, b.y);
  }
}

template <bool F32>
__device__ __forceinline__ Q8<F32> zero_q8() {
  if constexpr (F32) return f32x8{0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  else return make_uint4(0u, 0u, 0u, 0u);
}

// element e of 8 inputs, widened to fp32 exactly
template <bool F32>
__device__ __forceinline__ float q8_at(const Q8<F32> &x, int e) {
  if constexpr (F32) {
    return x[e];
  } else {
    const uint32_t w = e < 2 ? x.x : e < 4 ? x.y : e < 6 ? x.z : x.w;
    return __uint_as_float((e & 1) ? (w & 0xffff0000u) : (w << 16));
  }
}

__device__ __forceinline__ void f8_from(float *dst, float4 a, float4 b) {
  dst[0] = a.x; dst[1] = a.y; dst[2] = a.z; dst[3] = a.w;
  dst[4] = b.x; dst[5] = b.y; dst[6] = b.z; dst[7] = b.w;
}

// ---------------------------------------------------------------------------
// per-chunk record written by the prep kernel and read by the state kernel.
// Every matrix is stored as whole MFMA operand fragments with the contraction index
// in split order (see ld_n_split): fragment f holds 512 elements, lane l's 8 elements
// at f * 512 + 8 l, so a wave reads a fragment with one 16-byte (fp16) or 32-byte
// (fp32) access per lane.
//   -W      [t][i]   token tile t, key block i (stored negated: U = T V + (-W) S)
//   T       [t][j]   token tile t, token block j; only blocks on or below the diagonal
//   Kdec^T  [i][j]   key tile i, token block j
//   e^{G_C}          per key channel, fp32
//   Qt      [t][i]
//   P       [t][j]   only blocks on or below the diagonal
// The state map of a chunk needs only the first four (the prefix of `trans` bytes);
// the outputs need all.  Both sizes are whole KiB, so the record is copied to LDS in
// 1 KiB wave-wide pieces.
// ---------------------------------------------------------------------------
template <int C, bool F32>
struct Rec {
  using T = typename Op<F32>::T;
  static constexpr int NT = C / 16;                   // 16-token tiles
  static constexpr int KB = (C < 32 ? 32 : C) / 32;   // 32-token contraction blocks
  static constexpr size_t FRAG = 512 * sizeof(T);
  // fragment (token tile tb, token block kb) is zero when the block lies wholly above
  // the diagonal of a lower triangular C x C matrix
  static constexpr bool nz(int tb, int kb) { return 32 * kb <= 16 * tb + 15; }
  static constexpr int count_tri() {
    int n = 0;
    for (int tb = 0; tb < NT; ++tb)
      for (int kb = 0; kb < KB; ++kb) n += nz(tb, kb) ? 1 : 0;
    return n;
  }
  // position of a nonzero (tb, kb) fragment of T or P among the stored ones
  static constexpr int tri(int tb, int kb) {
    int n = 0;
    for (int t = 0; t < NT; ++t)
      for (int k = 0; k < KB; ++k) {
        if (t == tb && k == kb) return n;
        n += nz(t, k) ? 1 : 0;
      }
    return -1;
  }
  static constexpr int nW = NT * 4;
  static constexpr int nT = count_tri();
  static constexpr int nK = 8 * KB;
  static constexpr int nQ = NT * 4;
  static constexpr int nP = count_tri();
  static constexpr size_t kib(size_t x) { return (x + 1023) & ~size_t(1023); }
  static constexpr size_t oW = 0;
  static constexpr size_t oT = oW + nW * FRAG;
  static constexpr size_t oK = oT + nT * FRAG;
  static constexpr size_t oDec = oK + nK * FRAG;
  static constexpr size_t trans = kib(oDec + D * 4);
  static constexpr size_t oQ = trans;
  static constexpr size_t oP = oQ + nQ * FRAG;
  static constexpr size_t bytes = kib(oP + nP * FRAG);
  static __device__ __forceinline__ size_t frag(size_t off, int f, int lane) {
    return off + (size_t)f * FRAG + (size_t)lane * 8 * sizeof(T);
  }
};

}  // namespace kda
