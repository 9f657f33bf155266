// Chunkwise KDA prefill for gfx950.
//
// The sequence is cut into chunks; chunks are linked by the state recurrence and
// computed inside with matrix products ("xhh.club" tag page 结构, entry on the chunkwise
// algorithm).  Per chunk of C tokens entering with state S (d_k x d_v), with G the
// inclusive cumulative sum of the floored log-decay over the chunk (per key channel):
//
//   A  = StrictLower(diag(beta) (K e^G)(K e^-G)^T)      C x C   (decay-weighted K K^T)
//   P  = Lower((Q e^G)(K e^-G)^T)                       C x C   (decay-weighted Q K^T)
//   T  = (I + A)^-1 diag(beta)                          triangular solve (WY/UT form)
//   W  = T (K e^G),   U = T V - W S                      U holds the per-token writes u_t
//   O  = (Q e^G) S + P U
//   S <- Diag(e^{G_C}) S + (K e^{G_C - G})^T U
//
// Numerics ("xhh.club", chunkwise entry; "nlpx.cn" K3 guide section 6).  e^{+-G} over a
// whole chunk over/underflows fp32, so A and P are formed on 16-token tiles with a
// tile-local reference point r: for a diagonal tile the row factor e^{G_t - r} lies in
// [e^-80, 1] and the column factor e^{r - G_j} in [1, e^80] only because every step's
// log-decay is floored at -5 (16 * 5 = 80 < ln(FLT_MAX) = 88.7).  Those factors need a
// wide exponent, so diagonal tiles run as BF16 MFMA with each operand split into bf16
// high and low parts (three products).  In off-diagonal tiles both factors are <= 1
// and every other product has operands bounded by |q|, |k|, |v| or |S|; those run as
// fp16 MFMA.  All accumulation is fp32 and the state is carried in fp32 accumulators.
// With fp32 inputs every product runs as fp32 MFMA instead.
//
// One workgroup (4 waves) owns one (sequence, head, segment, value-column slice) and
// walks its chunks in order.  MODE_TRANSITION computes a segment's state map for the
// associative scan of context parallelism instead of outputs (see segment_scan).
#include <atomic>
#include <type_traits>

#include "internal.h"
#include "kda_device.h"

namespace kda {
namespace {

constexpr int D = 128;          // d_k = d_v
constexpr int NTHREADS = 256;   // 4 waves
constexpr int MODE_OUTPUT = 0;
constexpr int MODE_TRANSITION = 1;

typedef __attribute__((__vector_size__(8 * sizeof(float)))) float f32x8;

// ---------------------------------------------------------------------------
// operand types and the 16x16 (x K=32) MFMA step
// ---------------------------------------------------------------------------
template <bool F32> struct Op;
template <> struct Op<false> {   // fp16 operands in LDS
  using T = _Float16;
  using V8 = f16x8;
  static __device__ __forceinline__ V8 ld8(const T *p) { return *reinterpret_cast<const V8 *>(p); }
  static __device__ __forceinline__ T cvt(float x) { return static_cast<_Float16>(x); }
  static __device__ __forceinline__ f32x4 mma(f32x4 c, V8 a, V8 b) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
  }
};
template <> struct Op<true> {    // fp32 operands in LDS
  using T = float;
  using V8 = f32x8;
  static __device__ __forceinline__ V8 ld8(const T *p) {
    const float4 a = reinterpret_cast<const float4 *>(p)[0], b = reinterpret_cast<const float4 *>(p)[1];
    return V8{a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
  }
  static __device__ __forceinline__ T cvt(float x) { return x; }
  // The 32-long contraction as 8 MFMAs of K=4.  Lane group g supplies contraction
  // index 8g+e to MFMA e (the same permutation on both operands).
  static __device__ __forceinline__ f32x4 mma(f32x4 c, V8 a, V8 b) {
#pragma unroll
    for (int e = 0; e < 8; ++e) c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[e], b[e], c, 0, 0, 0);
    return c;
  }
};

// Swizzled row-major buffer.  Element (row, col) of a row of ROWLEN elements sits in
// 16-byte chunk (col / EPC) XOR (row mod min(16, chunks per row)) of its row, so lanes
// that read or write the same logical column of consecutive rows hit distinct banks.
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

__device__ __forceinline__ f32x4 zero4() { return f32x4{0.f, 0.f, 0.f, 0.f}; }

// Inclusive prefix sum over the 16 lanes of each DPP row.
__device__ __forceinline__ float row_scan16(float x) {
  x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x111, 0xf, 0xf, false));
  x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x112, 0xf, 0xf, false));
  x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x114, 0xf, 0xf, false));
  x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x118, 0xf, 0xf, false));
  return x;
}

// one step of the 16-lane inclusive scan on 8 independent values (DPP row shift right)
template <int CTRL>
__device__ __forceinline__ void scan_step(float *x) {
  float sv[8];
#pragma unroll
  for (int e = 0; e < 8; ++e)
    sv[e] = __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x[e]), CTRL, 0xf, 0xf, false));
#pragma unroll
  for (int e = 0; e < 8; ++e) x[e] += sv[e];
}

__device__ __forceinline__ void f8_from(float *dst, float4 a, float4 b) {
  dst[0] = a.x; dst[1] = a.y; dst[2] = a.z; dst[3] = a.w;
  dst[4] = b.x; dst[5] = b.y; dst[6] = b.z; dst[7] = b.w;
}

// ---------------------------------------------------------------------------
// shared-memory layout (all MFMA operand buffers row-major and swizzled)
// ---------------------------------------------------------------------------
template <int C, int NC, bool F32>
struct Layout {
  using T = typename Op<F32>::T;
  static constexpr int NT = C / 16;                  // 16-token tiles per chunk
  static constexpr int KC = C < 32 ? 32 : C;         // token contraction extent (zero padded)
  static constexpr bool ALIAS = (KC == C);           // buffers may share storage (no padding)
  static constexpr size_t E = sizeof(T);
  static constexpr size_t cmax(size_t a, size_t b) { return a > b ? a : b; }
  static constexpr size_t al(size_t x) { return (x + 15) & ~size_t(15); }
  // sizes in bytes
  static constexpr size_t bST = (size_t)NC * D * E;  // S^T    [c][i]
  static constexpr size_t bQT = (size_t)C * D * E;   // Qt     [t][i]
  static constexpr size_t bKD = (size_t)KC * D * E;  // Kdec   [t][i]  (rows >= C zero)
  static constexpr size_t bV = (size_t)KC * NC * E;  // V      [t][c]  (rows >= C zero)
  static constexpr size_t bPt = (size_t)KC * C * E;  // P^T    [j][t]  (rows >= C zero)
  static constexpr size_t bA = (size_t)C * C * 4;    // A fp32 [t][j]
  static constexpr size_t bUT = (size_t)NC * KC * E; // U^T    [c][t]  (cols >= C zero)
  static constexpr size_t bKF = (size_t)C * D * E;   // KF [t][i], then W [t][i]
  static constexpr size_t bKT = (size_t)KC * D * E;  // Kt     [t][i]  (rows >= C zero)
  static constexpr size_t bX = (size_t)NT * 256 * 4; // diagonal blocks of (I+A)^-1, fp32
  static constexpr size_t bTt = (size_t)KC * C * E;  // T^T    [j][t]  (rows >= C zero)
  static constexpr size_t bO = (size_t)C * D * 4;    // O staging fp32 [t][c]
  // byte offsets
  static constexpr size_t oST = 0;
  static constexpr size_t oQT = al(oST + bST);
  static constexpr size_t oKD = al(oQT + bQT);
  static constexpr size_t oV = al(oKD + bKD);
  static constexpr size_t oPt = al(oV + bV);
  static constexpr size_t oA = al(oPt + bPt);
  static constexpr size_t oUT = ALIAS ? oA : al(oA + bA);
  static constexpr size_t oKF = al(ALIAS ? oA + cmax(bA, bUT) : oUT + bUT);
  static constexpr size_t oKT = al(oKF + bKF);
  static constexpr size_t oX = al(oKT + bKT);
  static constexpr size_t oTt = al(oX + bX);
  static constexpr size_t oO = ALIAS ? oKT : al(oTt + bTt);        // staging over Kt + X + T^T
  static constexpr size_t endBig = ALIAS ? cmax(oTt + bTt, oKT + bO) : oO + bO;
  static constexpr int NFAC = NT > 2 ? (NT - 1) * (NT - 2) / 2 : 1;   // tile pairs w - s' >= 2
  // per-tile decay products; they are dead before T^T is written, so with aliasing
  // they live in the T^T buffer
  static constexpr size_t bVec = (2 * NT + NFAC) * D * 4;
  static_assert(!ALIAS || bVec <= bTt, "tile vectors must fit in the T^T buffer");
  static constexpr size_t oDpow = al(endBig);                       // D_m = e^{tile m total}
  static constexpr size_t oVec = ALIAS ? oTt : oDpow + NT * D * 4;
  static constexpr size_t oPre = oVec;                              // prod_{m<w} D_m
  static constexpr size_t oPost = oPre + NT * D * 4;                // prod_{m>w} D_m
  static constexpr size_t oFac = oPost + NT * D * 4;                // prod_{s'<m<w} D_m
  static constexpr size_t oBeta = ALIAS ? oDpow + NT * D * 4 : oFac + NFAC * D * 4;
  static constexpr size_t oDecay = oBeta + KC * 4;
  static constexpr size_t bytes = al(oDecay + D * 4);
};

// Raw inputs of one chunk held in registers between the load and their use, so the
// next chunk's loads can be issued while the current one is still being computed.
template <int C, int NC, bool F32>
struct RawChunk {
  static constexpr int NVG = C * NC / 8;                          // 8-column value groups
  static constexpr int NVPT = (NVG + NTHREADS - 1) / NTHREADS;    // groups per thread
  using Q8 = typename std::conditional<F32, f32x8, uint4>::type;  // 8 inputs (fp32 or bf16)
  float4 g[8];          // log-decay of this lane's token, channels 32kb + 8lg + (0..7)
  Q8 k[4], q[4];
  float beta;
  Q8 v[NVPT];
};

template <bool F32>
__device__ __forceinline__ typename std::conditional<F32, f32x8, uint4>::type load_q8(const void *p, size_t idx) {
  if constexpr (F32) {
    const float4 a = *reinterpret_cast<const float4 *>(static_cast<const float *>(p) + idx);
    const float4 b = *reinterpret_cast<const float4 *>(static_cast<const float *>(p) + idx + 4);
    return f32x8{a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
  } else {
    return *reinterpret_cast<const uint4 *>(static_cast<const uint16_t *>(p) + idx);
  }
}

template <bool F32>
__device__ __forceinline__ typename std::conditional<F32, f32x8, uint4>::type zero_q8() {
  if constexpr (F32) return f32x8{0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  else return make_uint4(0u, 0u, 0u, 0u);
}

// element e of 8 inputs, widened to fp32 exactly
template <bool F32>
__device__ __forceinline__ float q8_at(const typename std::conditional<F32, f32x8, uint4>::type &x, int e) {
  if constexpr (F32) {
    return x[e];
  } else {
    const uint32_t w = e < 2 ? x.x : e < 4 ? x.y : e < 6 ? x.z : x.w;
    return __uint_as_float((e & 1) ? (w & 0xffff0000u) : (w << 16));
  }
}

struct PrefillArgs {
  const void *q, *k, *v, *gate;
  const float *g, *beta, *S0, *norm_weight;
  float *S_final, *ckpt;
  void *o;
  float *maps;        // [units][D][2D] segment maps (transition mode)
  const float *sin;   // [units][D][D] states entering each segment (segmented output mode)
  float eps;
  int B, T, H;
  int n_seg, seg_chunks, n_chunks;
  int ckpt_every, n_ckpt;
  int out_bf16, fused_gate, raw_out;   // raw_out: write raw o for a separate norm pass
  int n_units;        // B * H * n_seg
};

// Issue the global loads of one chunk (zero-filled past the sequence end).  Addresses
// are a uniform chunk base plus per-lane 32-bit offsets that do not change between
// chunks; full chunks take a branch-free path.
template <int C, int NC, bool F32, int MODE>
__device__ __forceinline__ void load_chunk(RawChunk<C, NC, F32> &r, const PrefillArgs &a, int b, int h,
                                           int t0, int c0, int tid) {
  constexpr int NT = C / 16;
  constexpr int per_tok = NC / 8;
  constexpr int NVPT = RawChunk<C, NC, F32>::NVPT, NVG = RawChunk<C, NC, F32>::NVG;
  using E = typename std::conditional<F32, float, uint16_t>::type;
  const int wave = tid >> 6, lane = tid & 63, lr = lane & 15, lg = lane >> 4;
  const int tok_stride = a.H * D;
  const size_t base = ((size_t)b * a.T + t0) * tok_stride + (size_t)h * D;   // uniform
  const float *gb = a.g + base;
  const E *kb_ = static_cast<const E *>(a.k) + base;
  const E *qb = static_cast<const E *>(a.q) + base;
  const E *vb = static_cast<const E *>(a.v) + base;
  const float *bb = a.beta + ((size_t)b * a.T + t0) * a.H + h;
  const int tt = 16 * wave + lr;
  const uint32_t off = (uint32_t)tt * tok_stride + 8 * lg;
  auto vcol = [&](int x) { return MODE == MODE_OUTPUT ? c0 + (x % per_tok) * 8 : c0 + (x % per_tok) * 8 - D; };
  if (t0 + C <= a.T) {                                   // full chunk
    if (wave < NT) {
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        r.g[2 * kb] = *reinterpret_cast<const float4 *>(gb + off + 32 * kb);
        r.g[2 * kb + 1] = *reinterpret_cast<const float4 *>(gb + off + 32 * kb + 4);
        r.k[kb] = load_q8<F32>(kb_, off + 32 * kb);
        r.q[kb] = load_q8<F32>(qb, off + 32 * kb);
      }
      r.beta = bb[(uint32_t)tt * a.H];
    }
#pragma unroll
    for (int u = 0; u < NVPT; ++u) {
      const int x = tid + u * NTHREADS;
      const bool ok = (NVG % NTHREADS == 0 || x < NVG) && (MODE == MODE_OUTPUT || c0 + (x % per_tok) * 8 >= D);
      r.v[u] = ok ? load_q8<F32>(vb, (uint32_t)(x / per_tok) * tok_stride + vcol(x)) : zero_q8<F32>();
    }
    return;
  }
  const int nval = a.T - t0;                             // ragged last chunk
  const bool tok_ok = wave < NT && tt < nval;
#pragma unroll
  for (int kb = 0; kb < 4; ++kb) {
    if (tok_ok) {
      r.g[2 * kb] = *reinterpret_cast<const float4 *>(gb + off + 32 * kb);
      r.g[2 * kb + 1] = *reinterpret_cast<const float4 *>(gb + off + 32 * kb + 4);
      r.k[kb] = load_q8<F32>(kb_, off + 32 * kb);
      r.q[kb] = load_q8<F32>(qb, off + 32 * kb);
    } else {
      r.g[2 * kb] = r.g[2 * kb + 1] = make_float4(0.f, 0.f, 0.f, 0.f);
      r.k[kb] = zero_q8<F32>();
      r.q[kb] = zero_q8<F32>();
    }
  }
  r.beta = tok_ok ? bb[(uint32_t)tt * a.H] : 0.f;
#pragma unroll
  for (int u = 0; u < NVPT; ++u) {
    const int x = tid + u * NTHREADS;
    const int t = x / per_tok;
    const bool ok = x < NVG && t < nval && (MODE == MODE_OUTPUT || c0 + (x % per_tok) * 8 >= D);
    r.v[u] = ok ? load_q8<F32>(vb, (uint32_t)t * tok_stride + vcol(x)) : zero_q8<F32>();
  }
}

// ---------------------------------------------------------------------------
// the kernel
// ---------------------------------------------------------------------------
template <int C, int NC, bool F32, int MODE>
__global__ __launch_bounds__(NTHREADS, 1) void prefill_kernel(PrefillArgs a) {
  using L = Layout<C, NC, F32>;
  using T = typename Op<F32>::T;
  using V8 = typename Op<F32>::V8;
  constexpr int NT = L::NT, KC = L::KC;
  static_assert(!F32 || C == 16, "fp32 operands are used with 16-token chunks only");
  constexpr int NCB = NC / 16;                         // 16-column blocks per workgroup
  constexpr int VS = (MODE == MODE_TRANSITION ? 2 * D : D) / NC;   // workgroups per unit
  extern __shared__ __align__(16) unsigned char smem[];
  T *sST = reinterpret_cast<T *>(smem + L::oST);       // rows of D
  T *sQT = reinterpret_cast<T *>(smem + L::oQT);       // rows of D
  T *sKD = reinterpret_cast<T *>(smem + L::oKD);       // rows of D
  T *sV = reinterpret_cast<T *>(smem + L::oV);         // rows of NC
  T *sPt = reinterpret_cast<T *>(smem + L::oPt);       // rows of C
  float *sA = reinterpret_cast<float *>(smem + L::oA);
  T *sUT = reinterpret_cast<T *>(smem + L::oUT);       // rows of KC
  T *sKF = reinterpret_cast<T *>(smem + L::oKF);       // rows of D
  T *sW = sKF;                                         // W [t][i], after KF is dead
  T *sKT = reinterpret_cast<T *>(smem + L::oKT);       // rows of D
  float *sX = reinterpret_cast<float *>(smem + L::oX);
  T *sTt = reinterpret_cast<T *>(smem + L::oTt);       // rows of C
  float *sO = reinterpret_cast<float *>(smem + L::oO);
  float *sDpow = reinterpret_cast<float *>(smem + L::oDpow);
  float *sPre = reinterpret_cast<float *>(smem + L::oPre);
  float *sPost = reinterpret_cast<float *>(smem + L::oPost);
  float *sFac = reinterpret_cast<float *>(smem + L::oFac);
  float *sBeta = reinterpret_cast<float *>(smem + L::oBeta);
  float *sDecay = reinterpret_cast<float *>(smem + L::oDecay);

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int lr = lane & 15, lg = lane >> 4;

  // XCD-aware placement: consecutive workgroup ids go to different XCDs, so the
  // column slices of one unit get ids that are equal modulo 8 (same XCD, shared L2).
  const int bid = blockIdx.x;
  const int xcd = bid & 7, rest = bid >> 3;
  const int slice = rest % VS;
  const int unit = (rest / VS) * 8 + xcd;
  if (unit >= a.n_units) return;
  const int seg = unit % a.n_seg;
  if (MODE == MODE_TRANSITION && seg == a.n_seg - 1) return;   // last map is never used
  const int bh = unit / a.n_seg;
  const int h = bh % a.H, b = bh / a.H;
  const int c0 = slice * NC;                           // first (virtual) column of this slice
  const size_t tok_stride = (size_t)a.H * D;           // elements between consecutive tokens
  const size_t state_off = (size_t)bh * D * D;

  // zero the padded token range of the contraction buffers once (only when KC > C)
  if constexpr (!L::ALIAS) {
    for (int x = tid; x < KC * D; x += NTHREADS) { sKD[x] = T(0); sKT[x] = T(0); }
    for (int x = tid; x < KC * NC; x += NTHREADS) { sV[x] = T(0); sUT[x] = T(0); }
    for (int x = tid; x < KC * C; x += NTHREADS) { sPt[x] = T(0); sTt[x] = T(0); }
  }

  // ---- initial state: fp32 accumulators in MFMA output layout + transposed LDS copy
  // wave w owns key-row blocks {2w, 2w+1} x all NCB column blocks.
  f32x4 S[2][NCB];
#pragma unroll
  for (int ib = 0; ib < 2; ++ib)
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) {
      const int i0 = (2 * wave + ib) * 16 + 4 * lg, c = c0 + cb * 16 + lr;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int i = i0 + r;
        float x;
        if constexpr (MODE == MODE_TRANSITION) {
          x = (c < D && i == c) ? 1.f : 0.f;           // [A | B] starts at [I | 0]
        } else if (a.n_seg > 1) {
          x = a.sin[(size_t)unit * D * D + (size_t)i * D + c];   // from the segment scan
        } else {
          x = a.S0 ? a.S0[state_off + (size_t)i * D + c] : 0.f;
        }
        S[ib][cb][r] = x;
      }
      st4<F32, D>(sST, cb * 16 + lr, i0, S[ib][cb][0], S[ib][cb][1], S[ib][cb][2], S[ib][cb][3]);
    }

  const int ch_begin = seg * a.seg_chunks;
  const int ch_end = min(a.n_chunks, ch_begin + a.seg_chunks);
  const int tt = 16 * wave + lr;                       // this lane's token in phase A

  RawChunk<C, NC, F32> raw;
  load_chunk<C, NC, F32, MODE>(raw, a, b, h, ch_begin * C, c0, tid);

  for (int chunk = ch_begin; chunk < ch_end; ++chunk) {
    const int t0 = chunk * C;
    const int nval = min(C, a.T - t0);
    const size_t tok0 = ((size_t)b * a.T + t0) * tok_stride + (size_t)h * D;   // (b, t0, h, 0)

    // ===== phase A1: tile-relative cumulative log-decay, V =====
    // wave w < NT handles token tile w; lane: token tt = 16w + lr, channels 32kb + 8lg + e.
    float Lc[32];                                      // tile-relative cumulative log2-decay
    if (wave < NT) {
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        const int ch = 32 * kb + 8 * lg;
        float gg[8];
        f8_from(gg, raw.g[2 * kb], raw.g[2 * kb + 1]);
#pragma unroll
        for (int e = 0; e < 8; ++e) Lc[8 * kb + e] = log2_decay(gg[e]);
        // inclusive scan over the 16 tokens of the tile (DPP row shifts), 8 channels at once
        scan_step<0x111>(Lc + 8 * kb);
        scan_step<0x112>(Lc + 8 * kb);
        scan_step<0x114>(Lc + 8 * kb);
        scan_step<0x118>(Lc + 8 * kb);
        if (lr == 15) {                                  // tile decays D_w = e^{tile total}
          float dp[8];
#pragma unroll
          for (int e = 0; e < 8; ++e) dp[e] = exp2_fast(Lc[8 * kb + e]);
          float *pp = sDpow + wave * D + ch;
          reinterpret_cast<float4 *>(pp)[0] = make_float4(dp[0], dp[1], dp[2], dp[3]);
          reinterpret_cast<float4 *>(pp)[1] = make_float4(dp[4], dp[5], dp[6], dp[7]);
        }
      }
      if (lg == 0) sBeta[tt] = raw.beta;
    }
    // value columns of this slice, token-major (transition mode: columns < D belong to
    // the A part of the map and carry no value; they were loaded as zeros)
    {
      constexpr int per_tok = NC / 8;
#pragma unroll
      for (int u = 0; u < RawChunk<C, NC, F32>::NVPT; ++u) {
        const int x = tid + u * NTHREADS;
        if (x < RawChunk<C, NC, F32>::NVG) {
          float vv[8];
#pragma unroll
          for (int e = 0; e < 8; ++e) vv[e] = q8_at<F32>(raw.v[u], e);
          st8<F32, NC>(sV, x / per_tok, (x % per_tok) * 8, vv);
        }
      }
    }
    __syncthreads();   // tile totals, beta, V visible

    // per (tile, channel): prefix and suffix decay products, chunk decay, and the
    // factors between tiles two or more apart (all products of the tile decays D_m)
    if constexpr (NT > 1) {
      const int ch = tid & (D - 1), half = tid >> 7;
      float dp[NT];
#pragma unroll
      for (int m = 0; m < NT; ++m) dp[m] = sDpow[m * D + ch];
      if (half == 0) {
        float p = 1.f;
#pragma unroll
        for (int m = 0; m < NT; ++m) { sPre[m * D + ch] = p; p *= dp[m]; }
        sDecay[ch] = p;
        int pi = 0;
#pragma unroll
        for (int w = 2; w < NT; ++w)
#pragma unroll
          for (int sp = 0; sp + 2 <= w; ++sp) {
            float f = 1.f;
#pragma unroll
            for (int m = sp + 1; m < w; ++m) f *= dp[m];
            sFac[pi * D + ch] = f;
            ++pi;
          }
      } else {
        float p = 1.f;
#pragma unroll
        for (int m = NT - 1; m >= 0; --m) { sPost[m * D + ch] = p; p *= dp[m]; }
      }
    } else {
      if (tid < D) { sPre[tid] = 1.f; sPost[tid] = 1.f; sDecay[tid] = sDpow[tid]; }
    }
    __syncthreads();

    // ===== phase A2: decay factors, diagonal tile, chunk-level operands =====
    T rkx[32], rqx[32];                                // k e^{G_t - r_w}, q e^{G_t - r_w}
    if (wave < NT) {
      f32x4 accAd = zero4(), accPd = zero4();          // diagonal tile (w, w)
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        const int ch = 32 * kb + 8 * lg;
        float pre[8], post[8], dw[8];
        f8_from(pre, *reinterpret_cast<const float4 *>(sPre + wave * D + ch),
                *reinterpret_cast<const float4 *>(sPre + wave * D + ch + 4));
        f8_from(post, *reinterpret_cast<const float4 *>(sPost + wave * D + ch),
                *reinterpret_cast<const float4 *>(sPost + wave * D + ch + 4));
        f8_from(dw, *reinterpret_cast<const float4 *>(sDpow + wave * D + ch),
                *reinterpret_cast<const float4 *>(sDpow + wave * D + ch + 4));
        float rk[8], rq[8], yd[8], xq[8], xk[8], xd[8], xf[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float Lv = Lc[8 * kb + e], kk = q8_at<F32>(raw.k[kb], e), qq = q8_at<F32>(raw.q[kb], e);
          const float E = exp2_fast(Lv);               // e^{G_t - r_w}      in [e^-80, 1]
          const float En = exp2_fast(-Lv);             // e^{r_w - G_t}      in [1, e^80]
          rk[e] = kk * E;
          rq[e] = qq * E;
          yd[e] = kk * En;                             // k e^{r_w - G_t}
          xf[e] = yd[e] * dw[e];                       // k e^{r_{w+1} - G_t}, in [e^-75, 1] |k|
          xq[e] = rq[e] * pre[e];                      // q e^{G_t}
          xk[e] = rk[e] * pre[e];                      // k e^{G_t}
          xd[e] = xf[e] * post[e];                     // k e^{G_C - G_t}
          rkx[8 * kb + e] = Op<F32>::cvt(rk[e]);       // kept for the off-diagonal tiles
          rqx[8 * kb + e] = Op<F32>::cvt(rq[e]);
        }
        st8<F32, D>(sQT, tt, ch, xq);
        st8<F32, D>(sKT, tt, ch, xk);
        st8<F32, D>(sKD, tt, ch, xd);
        st8<F32, D>(sKF, tt, ch, xf);
        // diagonal tile (w, w) straight from registers: A in bf16, P with bf16 hi/lo
        if constexpr (F32) {
          const V8 va{rk[0], rk[1], rk[2], rk[3], rk[4], rk[5], rk[6], rk[7]};
          const V8 vq{rq[0], rq[1], rq[2], rq[3], rq[4], rq[5], rq[6], rq[7]};
          const V8 vy{yd[0], yd[1], yd[2], yd[3], yd[4], yd[5], yd[6], yd[7]};
          accAd = Op<true>::mma(accAd, va, vy);
          if constexpr (MODE == MODE_OUTPUT) accPd = Op<true>::mma(accPd, vq, vy);
        } else {
          bf16x8 kh, yh;
#pragma unroll
          for (int e = 0; e < 8; ++e) { kh[e] = static_cast<__bf16>(rk[e]); yh[e] = static_cast<__bf16>(yd[e]); }
          accAd = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kh, yh, accAd, 0, 0, 0);
          if constexpr (MODE == MODE_OUTPUT) {
            bf16x8 qh, ql, yl;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
              qh[e] = static_cast<__bf16>(rq[e]);
              ql[e] = static_cast<__bf16>(rq[e] - static_cast<float>(qh[e]));
              yl[e] = static_cast<__bf16>(yd[e] - static_cast<float>(yh[e]));
            }
            accPd = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qh, yh, accPd, 0, 0, 0);
            accPd = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qh, yl, accPd, 0, 0, 0);
            accPd = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ql, yh, accPd, 0, 0, 0);
          }
        }
      }
      // store the diagonal tile: A (beta rows, strictly lower), P^T (lower incl.), and
      // P's zero blocks above the diagonal of this tile row
      {
        float pv[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int ti = 4 * lg + r, t = 16 * wave + ti;
          sA[t * C + 16 * wave + lr] = ti > lr ? accAd[r] * sBeta[t] : 0.f;
          pv[r] = ti >= lr ? accPd[r] : 0.f;
        }
        if constexpr (MODE == MODE_OUTPUT) {
          st4<F32, C>(sPt, 16 * wave + lr, 16 * wave + 4 * lg, pv[0], pv[1], pv[2], pv[3]);
#pragma unroll
          for (int sp = 1; sp < NT; ++sp)
            if (sp > wave) st4<F32, C>(sPt, 16 * sp + lr, 16 * wave + 4 * lg, 0.f, 0.f, 0.f, 0.f);
        }
      }
    }
    __syncthreads();   // KF, Qt, Kt, Kdec, decay, diagonal A/P visible

    // gate logits of this chunk for the fused epilogue (tokens 4w + lg + 16n, columns
    // 8lr..8lr+7), then the next chunk's inputs: both arrive while the solve and the
    // state products run
    typename RawChunk<C, NC, F32>::Q8 gate_cur[C / 16];
    if constexpr (MODE == MODE_OUTPUT && NC == D) {
      if (a.fused_gate) {
#pragma unroll
        for (int n = 0; n < C / 16; ++n) {
          const int t = 4 * wave + lg + 16 * n;
          gate_cur[n] = t < nval ? load_q8<F32>(a.gate, tok0 + (size_t)t * tok_stride + 8 * lr) : zero_q8<F32>();
        }
      }
    }
    if (chunk + 1 < ch_end) load_chunk<C, NC, F32, MODE>(raw, a, b, h, t0 + C, c0, tid);

    // ===== phase A3: wave 0 inverts every diagonal block of I + A (one column per lane);
    // waves w >= 1 compute the off-diagonal tiles (w, s'), s' < w, with row operand
    // k e^{G_t - r_w} prod_{s'<m<w} D_m and column operand KF of tile s' (both <= 1) ====
    if (wave == 0) {
      if (lane < 16 * NT) {
        const int bb = lane >> 4, j = lane & 15;
        float x[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          float arow[16];
#pragma unroll
          for (int m4 = 0; m4 < 4; ++m4)
            *reinterpret_cast<float4 *>(arow + 4 * m4) =
                *reinterpret_cast<const float4 *>(sA + (16 * bb + i) * C + 16 * bb + 4 * m4);
          float acc = (i == j) ? 1.f : 0.f;
#pragma unroll
          for (int m = 0; m < i; ++m) acc -= arow[m] * x[m];
          x[i] = acc;
        }
#pragma unroll
        for (int i = 0; i < 16; ++i) sX[bb * 256 + i * 16 + j] = x[i];
      }
    } else if (wave < NT) {
      f32x4 accA[NT], accP[NT];
#pragma unroll
      for (int sp = 0; sp < NT; ++sp) { accA[sp] = zero4(); accP[sp] = zero4(); }
#pragma unroll
      for (int sp = 0; sp < NT - 1; ++sp) {
        if (sp < wave) {
#pragma unroll
          for (int kb = 0; kb < 4; ++kb) {
            const int ch = 32 * kb + 8 * lg;
            V8 va, vq;
#pragma unroll
            for (int e = 0; e < 8; ++e) { va[e] = rkx[8 * kb + e]; vq[e] = rqx[8 * kb + e]; }
            if (sp + 1 < wave) {                         // tiles two or more apart: scale by
              const int pi = (wave - 2) * (wave - 1) / 2 + sp;   // prod_{s'<m<w} D_m
              float fac[8];
              f8_from(fac, *reinterpret_cast<const float4 *>(sFac + pi * D + ch),
                      *reinterpret_cast<const float4 *>(sFac + pi * D + ch + 4));
              V8 vf;
#pragma unroll
              for (int e = 0; e < 8; ++e) vf[e] = Op<F32>::cvt(fac[e]);
              va = va * vf;
              vq = vq * vf;
            }
            const V8 vb = ld_n<F32, D>(sKF, 16 * sp, 32 * kb, lane);
            accA[sp] = Op<F32>::mma(accA[sp], va, vb);
            if constexpr (MODE == MODE_OUTPUT) accP[sp] = Op<F32>::mma(accP[sp], vq, vb);
          }
        }
      }
#pragma unroll
      for (int sp = 0; sp < NT - 1; ++sp) {
        if (sp < wave) {
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int t = 16 * wave + 4 * lg + r;
            sA[t * C + 16 * sp + lr] = accA[sp][r] * sBeta[t];
          }
          if constexpr (MODE == MODE_OUTPUT)
            st4<F32, C>(sPt, 16 * sp + lr, 16 * wave + 4 * lg, accP[sp][0], accP[sp][1], accP[sp][2], accP[sp][3]);
        }
      }
    }
    __syncthreads();   // A, P, diagonal inverses complete

    // ===== solve: wave w walks down column block w of X = (I + A)^-1:
    // X_{s,w} = -X_ss sum_{w<=m<s} A_{s,m} X_{m,w}; a 16x16 result in MFMA output layout
    // is the B operand layout of the K=16 MFMA, so the blocks stay in registers.
    // Then T[:, block w] = X[:, block w] diag(beta), stored as T^T [j][t]. =====
    if (wave < NT) {
      const int n = lr;                                 // column within the block
      const float bj = sBeta[16 * wave + n];
      f32x4 xc[NT];
#pragma unroll
      for (int s = 0; s < NT; ++s) {
        if (s == wave) {
#pragma unroll
          for (int r = 0; r < 4; ++r) xc[s][r] = sX[wave * 256 + (4 * lg + r) * 16 + n];
        } else {
          xc[s] = zero4();
        }
      }
      if constexpr (NT > 1 && !F32) {
#pragma unroll
        for (int s = 1; s < NT; ++s) {
          if (s > wave) {
            f32x4 y = zero4();
#pragma unroll
            for (int m = 0; m < NT - 1; ++m) {
              if (m >= wave && m < s) {
                const float4 av = *reinterpret_cast<const float4 *>(sA + (16 * s + lr) * C + 16 * m + 4 * lg);
                const f16x4 a4{(_Float16)av.x, (_Float16)av.y, (_Float16)av.z, (_Float16)av.w};
                const f16x4 b4{(_Float16)xc[m][0], (_Float16)xc[m][1], (_Float16)xc[m][2], (_Float16)xc[m][3]};
                y = __builtin_amdgcn_mfma_f32_16x16x16f16(a4, b4, y, 0, 0, 0);
              }
            }
            const float4 xv = *reinterpret_cast<const float4 *>(sX + s * 256 + lr * 16 + 4 * lg);
            const f16x4 a4{(_Float16)xv.x, (_Float16)xv.y, (_Float16)xv.z, (_Float16)xv.w};
            const f16x4 b4{(_Float16)y[0], (_Float16)y[1], (_Float16)y[2], (_Float16)y[3]};
            const f32x4 z = __builtin_amdgcn_mfma_f32_16x16x16f16(a4, b4, zero4(), 0, 0, 0);
#pragma unroll
            for (int r = 0; r < 4; ++r) xc[s][r] = -z[r];
          }
        }
      }
#pragma unroll
      for (int s = 0; s < NT; ++s) {
        const bool on = s >= wave;
        st4<F32, C>(sTt, 16 * wave + n, 16 * s + 4 * lg, on ? xc[s][0] * bj : 0.f, on ? xc[s][1] * bj : 0.f,
                    on ? xc[s][2] * bj : 0.f, on ? xc[s][3] * bj : 0.f);
      }
    }
    __syncthreads();   // T complete

    // ===== W^T = Kt^T T^T  ->  W [t][i] (overwrites KF) =====
    {
      constexpr int NTILE = 8 * NT;                    // (i-block, t-block)
#pragma unroll 2
      for (int it = 0; it < (NTILE + 3) / 4; ++it) {
        const int tile = wave + 4 * it;
        if (tile < NTILE) {
          const int ib = tile / NT, tb = tile % NT;
          f32x4 acc = zero4();
#pragma unroll
          for (int kb = 0; kb < KC / 32; ++kb)
            acc = Op<F32>::mma(acc, ld_t<F32, D>(sKT, 32 * kb, 16 * ib, lane),
                               ld_t<F32, C>(sTt, 32 * kb, 16 * tb, lane));
          // acc[r] = W^T[16ib + 4lg + r][16tb + lr]
          st4<F32, D>(sW, 16 * tb + lr, 16 * ib + 4 * lg, acc[0], acc[1], acc[2], acc[3]);
        }
      }
    }
    __syncthreads();

    // ===== U = T V - W S  ->  U^T[c][t] =====
    {
      constexpr int NTILE = NT * NCB;
#pragma unroll 2
      for (int it = 0; it < (NTILE + 3) / 4; ++it) {
        const int tile = wave + 4 * it;
        if (tile < NTILE) {
          const int tb = tile / NCB, cb = tile % NCB;
          f32x4 acc = zero4();
#pragma unroll
          for (int kb = 0; kb < 4; ++kb)
            acc = Op<F32>::mma(acc, ld_n<F32, D>(sW, 16 * tb, 32 * kb, lane),
                               ld_n<F32, D>(sST, 16 * cb, 32 * kb, lane));
#pragma unroll
          for (int r = 0; r < 4; ++r) acc[r] = -acc[r];
#pragma unroll
          for (int kb = 0; kb < KC / 32; ++kb)
            acc = Op<F32>::mma(acc, ld_t<F32, C>(sTt, 32 * kb, 16 * tb, lane),
                               ld_t<F32, NC>(sV, 32 * kb, 16 * cb, lane));
          // acc[r] = U[16tb + 4lg + r][16cb + lr]
          st4<F32, KC>(sUT, 16 * cb + lr, 16 * tb + 4 * lg, acc[0], acc[1], acc[2], acc[3]);
        }
      }
    }
    __syncthreads();

    // ===== O = Qt S + P U  (output mode) =====
    if constexpr (MODE == MODE_OUTPUT) {
      constexpr int NTILE = NT * NCB;
#pragma unroll 2
      for (int it = 0; it < (NTILE + 3) / 4; ++it) {
        const int tile = wave + 4 * it;
        if (tile < NTILE) {
          const int tb = tile / NCB, cb = tile % NCB;
          f32x4 acc = zero4();
#pragma unroll
          for (int kb = 0; kb < 4; ++kb)
            acc = Op<F32>::mma(acc, ld_n<F32, D>(sQT, 16 * tb, 32 * kb, lane),
                               ld_n<F32, D>(sST, 16 * cb, 32 * kb, lane));
#pragma unroll
          for (int kb = 0; kb < KC / 32; ++kb)
            acc = Op<F32>::mma(acc, ld_t<F32, C>(sPt, 32 * kb, 16 * tb, lane),
                               ld_n<F32, KC>(sUT, 16 * cb, 32 * kb, lane));
          const int cl = 16 * cb + lr;
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int t = 16 * tb + 4 * lg + r;
            if (a.fused_gate) {
              sO[t * D + cl] = acc[r];
            } else if (t < nval) {
              const size_t idx = tok0 + (size_t)t * tok_stride + c0 + cl;
              if (a.out_bf16 && !a.raw_out)
                static_cast<uint16_t *>(a.o)[idx] = f32_to_bf16_bits(acc[r]);
              else
                static_cast<float *>(a.o)[idx] = acc[r];
            }
          }
        }
      }
      __syncthreads();   // O reads of S^T complete (and staging visible)
      if (a.fused_gate) {
        // per-head RMSNorm over the 128 value columns, then the sigmoid gate:
        // 4 tokens per wave pass, 16 lanes x 8 columns per token
#pragma unroll
        for (int n = 0; n < C / 16; ++n) {
          const int t = 4 * wave + lg + 16 * n;
          float ov[8];
          float ss = 0.f;
#pragma unroll
          for (int e = 0; e < 8; ++e) { ov[e] = sO[t * D + 8 * lr + e]; ss += ov[e] * ov[e]; }
          ss += __shfl_xor(ss, 1, 64);
          ss += __shfl_xor(ss, 2, 64);
          ss += __shfl_xor(ss, 4, 64);
          ss += __shfl_xor(ss, 8, 64);
          if (t < nval) {
            const float inv = rsqrtf(ss * (1.0f / D) + a.eps);
            const size_t base = tok0 + (size_t)t * tok_stride + 8 * lr;
            float gv[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) gv[e] = q8_at<F32>(gate_cur[n], e);
            float res[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
              const float w = a.norm_weight ? a.norm_weight[8 * lr + e] : 1.f;
              res[e] = ov[e] * inv * w * sigmoidf_(gv[e]);
            }
            if (a.out_bf16) {
              store4<true>(a.o, base, make_float4(res[0], res[1], res[2], res[3]));
              store4<true>(a.o, base + 4, make_float4(res[4], res[5], res[6], res[7]));
            } else {
              store4<false>(a.o, base, make_float4(res[0], res[1], res[2], res[3]));
              store4<false>(a.o, base + 4, make_float4(res[4], res[5], res[6], res[7]));
            }
          }
        }
      }
    }

    // ===== S <- Diag(e^{G_C}) S + Kdec^T U =====
#pragma unroll
    for (int ib = 0; ib < 2; ++ib) {
      const int i0 = (2 * wave + ib) * 16;
      const float4 dec = *reinterpret_cast<const float4 *>(sDecay + i0 + 4 * lg);
#pragma unroll
      for (int cb = 0; cb < NCB; ++cb) {
        f32x4 acc = S[ib][cb];
        acc[0] *= dec.x; acc[1] *= dec.y; acc[2] *= dec.z; acc[3] *= dec.w;
#pragma unroll
        for (int kb = 0; kb < KC / 32; ++kb)
          acc = Op<F32>::mma(acc, ld_t<F32, D>(sKD, 32 * kb, i0, lane),
                             ld_n<F32, KC>(sUT, 16 * cb, 32 * kb, lane));
        S[ib][cb] = acc;
        st4<F32, D>(sST, 16 * cb + lr, i0 + 4 * lg, acc[0], acc[1], acc[2], acc[3]);
      }
    }
    // checkpoint: state after a multiple of ckpt_every tokens
    if constexpr (MODE == MODE_OUTPUT) {
      const int tend = t0 + nval;
      if (a.ckpt_every > 0 && nval == C && tend % a.ckpt_every == 0) {
        const int m = tend / a.ckpt_every - 1;
        float *dst = a.ckpt + (((size_t)b * a.n_ckpt + m) * a.H + h) * (size_t)D * D;
#pragma unroll
        for (int ib = 0; ib < 2; ++ib)
#pragma unroll
          for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
            for (int r = 0; r < 4; ++r)
              dst[(size_t)((2 * wave + ib) * 16 + 4 * lg + r) * D + c0 + 16 * cb + lr] = S[ib][cb][r];
      }
    }
    __syncthreads();   // chunk done: LDS may be refilled
  }

  // ---- results: final state (last segment) or the segment map
  if constexpr (MODE == MODE_OUTPUT) {
    if (a.S_final && seg == a.n_seg - 1) {
#pragma unroll
      for (int ib = 0; ib < 2; ++ib)
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
          for (int r = 0; r < 4; ++r)
            a.S_final[state_off + (size_t)((2 * wave + ib) * 16 + 4 * lg + r) * D + c0 + 16 * cb + lr] =
                S[ib][cb][r];
    }
  } else {
    float *dst = a.maps + (size_t)unit * D * (2 * D);
#pragma unroll
    for (int ib = 0; ib < 2; ++ib)
#pragma unroll
      for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          dst[(size_t)((2 * wave + ib) * 16 + 4 * lg + r) * (2 * D) + c0 + 16 * cb + lr] = S[ib][cb][r];
  }
}

// ---------------------------------------------------------------------------
// associative scan of segment maps: S_in[0] = S0, S_in[s+1] = A_s S_in[s] + B_s
// ("xhh.club" structure entry: context parallelism by an associative prefix scan; the
// states entering later segments are composed, never summed).  One workgroup per
// (sequence, head, 16-column block); the map product runs as fp32 MFMA.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(NTHREADS, 1) void segment_scan(const float *__restrict__ maps,
                                                           const float *__restrict__ S0,
                                                           float *__restrict__ sin, int n_seg,
                                                           int n_bh) {
  __shared__ __align__(16) float sXt[16][D + 4];      // current state block, transposed [n][i]
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int lr = lane & 15, lg = lane >> 4;
  const int bh = blockIdx.x / (D / 16), cb = blockIdx.x % (D / 16);
  if (bh >= n_bh) return;
  const int c0 = cb * 16;
  // S_in[0] = S0 (or zeros)
  for (int x = tid; x < 16 * D; x += NTHREADS) {
    const int i = x / 16, n = x % 16;
    const float v = S0 ? S0[(size_t)bh * D * D + (size_t)i * D + c0 + n] : 0.f;
    sXt[n][i] = v;
    sin[((size_t)bh * n_seg) * D * D + (size_t)i * D + c0 + n] = v;
  }
  __syncthreads();
  for (int s = 0; s + 1 < n_seg; ++s) {
    const float *A = maps + ((size_t)bh * n_seg + s) * D * (2 * D);
    f32x4 acc[2];
    // wave w computes rows 32w..32w+31 (two 16-row tiles); lane group g supplies
    // contraction indices 32g .. 32g+31 (one per MFMA).
#pragma unroll
    for (int it = 0; it < 2; ++it) {
      const int i = (2 * wave + it) * 16 + lr;
      f32x4 c = zero4();
      const float *arow = A + (size_t)i * (2 * D) + 32 * lg;
#pragma unroll
      for (int q4 = 0; q4 < 8; ++q4) {
        const float4 av = *reinterpret_cast<const float4 *>(arow + 4 * q4);
        const float4 bv = *reinterpret_cast<const float4 *>(&sXt[lr][32 * lg + 4 * q4]);
        c = __builtin_amdgcn_mfma_f32_16x16x4f32(av.x, bv.x, c, 0, 0, 0);
        c = __builtin_amdgcn_mfma_f32_16x16x4f32(av.y, bv.y, c, 0, 0, 0);
        c = __builtin_amdgcn_mfma_f32_16x16x4f32(av.z, bv.z, c, 0, 0, 0);
        c = __builtin_amdgcn_mfma_f32_16x16x4f32(av.w, bv.w, c, 0, 0, 0);
      }
      acc[it] = c;
    }
    __syncthreads();   // all reads of the old block done
    float *dst = sin + ((size_t)bh * n_seg + s + 1) * D * D;
#pragma unroll
    for (int it = 0; it < 2; ++it)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int i = (2 * wave + it) * 16 + 4 * lg + r;
        const float v = acc[it][r] + A[(size_t)i * (2 * D) + D + c0 + lr];
        sXt[lr][i] = v;
        dst[(size_t)i * D + c0 + lr] = v;
      }
    __syncthreads();
  }
}

// ---------------------------------------------------------------------------
// RMSNorm + sigmoid gate over raw outputs (used when the value columns of a head are
// split across workgroups): one wave per 4 (token, head) rows.
// ---------------------------------------------------------------------------
template <bool IN_BF16, bool OUT_BF16>
__global__ __launch_bounds__(NTHREADS) void norm_gate_kernel(const float *__restrict__ raw,
                                                             const void *__restrict__ gate,
                                                             const float *__restrict__ w,
                                                             void *__restrict__ out, int64_t rows,
                                                             float eps) {
  const int lane = threadIdx.x & 63, lr = lane & 15, lg = lane >> 4;
  const int64_t row = ((int64_t)blockIdx.x * (NTHREADS / 64) + (threadIdx.x >> 6)) * 4 + lg;
  if (row >= rows) return;
  const size_t base = (size_t)row * D + 8 * lr;
  const float4 a0 = *reinterpret_cast<const float4 *>(raw + base);
  const float4 a1 = *reinterpret_cast<const float4 *>(raw + base + 4);
  const float ov[8] = {a0.x, a0.y, a0.z, a0.w, a1.x, a1.y, a1.z, a1.w};
  float ss = 0.f;
#pragma unroll
  for (int e = 0; e < 8; ++e) ss += ov[e] * ov[e];
  ss += __shfl_xor(ss, 1, 64);
  ss += __shfl_xor(ss, 2, 64);
  ss += __shfl_xor(ss, 4, 64);
  ss += __shfl_xor(ss, 8, 64);
  const float inv = rsqrtf(ss * (1.0f / D) + eps);
  const float4 g0 = load4<IN_BF16>(gate, base), g1 = load4<IN_BF16>(gate, base + 4);
  const float gv[8] = {g0.x, g0.y, g0.z, g0.w, g1.x, g1.y, g1.z, g1.w};
  float res[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) res[e] = ov[e] * inv * (w ? w[8 * lr + e] : 1.f) * sigmoidf_(gv[e]);
  store4<OUT_BF16>(out, base, make_float4(res[0], res[1], res[2], res[3]));
  store4<OUT_BF16>(out, base + 4, make_float4(res[4], res[5], res[6], res[7]));
}

// ---------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------
template <int C, int NC, bool F32, int MODE>
hipError_t launch_one(const PrefillArgs &a, hipStream_t s) {
  using L = Layout<C, NC, F32>;
  static_assert(L::bytes <= 160 * 1024, "LDS budget exceeded");
  auto kern = prefill_kernel<C, NC, F32, MODE>;
  static std::atomic<bool> attr_set{false};   // the attribute is per function, set once
  if (!attr_set.load(std::memory_order_acquire)) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)L::bytes);
    if (e != hipSuccess) return e;
    attr_set.store(true, std::memory_order_release);
  }
  constexpr int VS = (MODE == MODE_TRANSITION ? 2 * D : D) / NC;
  const int groups = (a.n_units + 7) / 8;
  const unsigned grid = static_cast<unsigned>(groups) * 8u * VS;
  hipLaunchKernelGGL(kern, dim3(grid), dim3(NTHREADS), L::bytes, s, a);
  return hipGetLastError();
}

template <int C, bool F32, int MODE>
hipError_t launch_nc(const PrefillArgs &a, int nc, hipStream_t s) {
  if constexpr (!F32) {   // the fp32 path keeps at most 64 columns per workgroup (LDS)
    if (nc == 128) return launch_one<C, 128, F32, MODE>(a, s);
  }
  if (nc == 64) return launch_one<C, 64, F32, MODE>(a, s);
  if (nc == 32) return launch_one<C, 32, F32, MODE>(a, s);
  return hipErrorInvalidValue;
}

template <int MODE>
hipError_t launch_mode(const PrefillArgs &a, int chunk, bool f32, int nc, hipStream_t s) {
  if (f32) return launch_nc<16, true, MODE>(a, nc, s);
  if (chunk == 16) return launch_nc<16, false, MODE>(a, nc, s);
  return launch_nc<64, false, MODE>(a, nc, s);
}

}  // namespace

hipError_t launch_prefill(const kda_prefill_desc &d, const PrefillPlan &p, hipStream_t s) {
  const bool f32 = d.in_dtype == KDA_F32;
  const int64_t units = (int64_t)d.B * d.H;
  unsigned char *ws = static_cast<unsigned char *>(d.workspace);
  auto up = [](size_t x) { return (x + 255) & ~static_cast<size_t>(255); };
  float *maps = p.ws_maps ? reinterpret_cast<float *>(ws) : nullptr;
  float *sin = p.ws_sin ? reinterpret_cast<float *>(ws + up(p.ws_maps)) : nullptr;

  if (d.T == 0) {
    // no tokens: the final state is the initial state
    if (d.S_final && d.S_final != d.S0) {
      if (d.S0) return launch_state_copy(d.S_final, d.S0, units * d.d_k * d.d_v, s);
      return launch_fill_zero(d.S_final, units * d.d_k * d.d_v, s);
    }
    return hipSuccess;
  }

  PrefillArgs a{};
  a.q = d.q; a.k = d.k; a.v = d.v; a.gate = d.gate;
  a.g = d.g; a.beta = d.beta; a.S0 = d.S0; a.norm_weight = d.norm_weight;
  a.S_final = d.S_final; a.ckpt = d.ckpt; a.o = d.o;
  a.maps = maps; a.sin = sin; a.eps = d.norm_eps;
  a.B = d.B; a.T = d.T; a.H = d.H;
  a.n_seg = p.n_seg; a.seg_chunks = p.seg_chunks; a.n_chunks = p.n_chunks;
  a.ckpt_every = d.ckpt_every;
  a.n_ckpt = d.ckpt_every > 0 ? d.T / d.ckpt_every : 0;
  a.out_bf16 = d.out_dtype == KDA_BF16;
  a.n_units = static_cast<int>(units * p.n_seg);
  const int nc = D / p.v_split;
  a.fused_gate = d.gate != nullptr && !p.split_norm;
  a.raw_out = p.split_norm;
  float *raw = nullptr;
  if (p.split_norm) {
    // raw o goes to fp32 storage first: the output itself when it is fp32
    raw = d.out_dtype == KDA_F32 ? static_cast<float *>(d.o)
                                 : reinterpret_cast<float *>(ws + up(p.ws_maps) + up(p.ws_sin));
    if (!raw) return hipErrorInvalidValue;
    a.o = raw;
  }

  hipError_t e;
  if (p.n_seg > 1) {
    // pass 1: maps of all segments but the last
    PrefillArgs t = a;
    t.n_units = static_cast<int>(units * p.n_seg);
    t.fused_gate = 0;
    // the map [A | B] has 2 x 128 columns: two workgroups per segment (fp32 operands: four)
    e = launch_mode<MODE_TRANSITION>(t, d.chunk, f32, f32 ? 64 : D, s);
    if (e != hipSuccess) return e;
    // pass 2: states entering each segment
    const unsigned grid = static_cast<unsigned>(units * (D / 16));
    hipLaunchKernelGGL(segment_scan, dim3(grid), dim3(NTHREADS), 0, s, maps, d.S0, sin, p.n_seg,
                       static_cast<int>(units));
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  // pass 3 (or the single pass): outputs, checkpoints, final state
  e = launch_mode<MODE_OUTPUT>(a, d.chunk, f32, nc, s);
  if (e != hipSuccess) return e;
  if (p.split_norm) {
    const int64_t rows = (int64_t)d.B * d.T * d.H;
    const unsigned grid = static_cast<unsigned>((rows + 15) / 16);
    const bool ib = d.in_dtype == KDA_BF16, ob = d.out_dtype == KDA_BF16;
    if (ib && ob) hipLaunchKernelGGL((norm_gate_kernel<true, true>), dim3(grid), dim3(NTHREADS), 0, s, raw, d.gate, d.norm_weight, d.o, rows, d.norm_eps);
    else if (ib) hipLaunchKernelGGL((norm_gate_kernel<true, false>), dim3(grid), dim3(NTHREADS), 0, s, raw, d.gate, d.norm_weight, d.o, rows, d.norm_eps);
    else if (ob) hipLaunchKernelGGL((norm_gate_kernel<false, true>), dim3(grid), dim3(NTHREADS), 0, s, raw, d.gate, d.norm_weight, d.o, rows, d.norm_eps);
    else hipLaunchKernelGGL((norm_gate_kernel<false, false>), dim3(grid), dim3(NTHREADS), 0, s, raw, d.gate, d.norm_weight, d.o, rows, d.norm_eps);
    e = hipGetLastError();
  }
  return e;
}

}  // namespace kda
