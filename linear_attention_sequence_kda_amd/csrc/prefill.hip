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

// C[16x16] += A[16 x 32] * B[32 x 16] where lane l supplies row (l&15) of A and column
// (l&15) of B, contraction elements 8(l>>4)..+7: both read from row-major buffers whose
// contraction index is contiguous (A: [m][k], B stored as [n][k]).
template <bool F32>
__device__ __forceinline__ f32x4 mma_lds(f32x4 c, const typename Op<F32>::T *a, int lda,
                                         const typename Op<F32>::T *b, int ldb, int lane) {
  const int r = lane & 15, k = 8 * (lane >> 4);
  return Op<F32>::mma(c, Op<F32>::ld8(a + r * lda + k), Op<F32>::ld8(b + r * ldb + k));
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

// ---------------------------------------------------------------------------
// shared-memory layout
// ---------------------------------------------------------------------------
template <int C, int NC, bool F32>
struct Layout {
  using T = typename Op<F32>::T;
  static constexpr int NT = C / 16;                  // 16-token tiles per chunk
  static constexpr int KC = C < 32 ? 32 : C;         // token contraction extent (zero padded)
  static constexpr bool ALIAS = (KC == C);           // buffers may share storage (no padding)
  static constexpr size_t E = sizeof(T);
  // element counts
  static constexpr size_t nST = (size_t)NC * D;      // S^T   [c][i]
  static constexpr size_t nQT = (size_t)C * D;       // Qt    [t][i]
  static constexpr size_t nKD = (size_t)D * KC;      // Kdec^T[i][t]
  static constexpr size_t nVT = (size_t)NC * KC;     // V^T   [c][t]
  static constexpr size_t nP = (size_t)C * KC;       // P     [t][j]
  static constexpr size_t nKF = (size_t)C * D;       // KF    [t][i]  then -W [t][i]
  static constexpr size_t nKT = (size_t)D * KC;      // Kt^T  [i][t]
  static constexpr size_t bA = (size_t)C * C * 4;    // A fp32 [t][j]
  static constexpr size_t bUT = nVT * E;             // U^T   [c][t]
  static constexpr size_t bX = (size_t)C * C * 4;    // X fp32 [t][j]
  static constexpr size_t bTT = (size_t)C * KC * E;  // T     [t][j]
  static constexpr size_t bO = (size_t)C * D * 4;    // O staging fp32 [t][c]
  static constexpr size_t cmax(size_t a, size_t b) { return a > b ? a : b; }
  static constexpr size_t al(size_t x) { return (x + 15) & ~size_t(15); }
  // byte offsets
  static constexpr size_t oST = 0;
  static constexpr size_t oQT = al(oST + nST * E);
  static constexpr size_t oKD = al(oQT + nQT * E);
  static constexpr size_t oVT = al(oKD + nKD * E);
  static constexpr size_t oP = al(oVT + nVT * E);
  static constexpr size_t oAU = al(oP + nP * E);
  static constexpr size_t szAU = ALIAS ? cmax(bA, bUT) : 0;
  static constexpr size_t oA = oAU;
  static constexpr size_t oUT = ALIAS ? oAU : al(oAU + bA);
  static constexpr size_t oKFW = al(ALIAS ? oAU + szAU : oUT + bUT);
  static constexpr size_t oKT = al(oKFW + nKF * E);
  static constexpr size_t oXT = al(oKT + nKT * E);
  static constexpr size_t szXT = ALIAS ? cmax(bX, bTT) : bX;
  static constexpr size_t oTT = ALIAS ? oXT : al(oXT + bX);
  static constexpr size_t oO = ALIAS ? oKT : al(oTT + bTT);        // staging over Kt^T + X
  static constexpr size_t endBig = ALIAS ? cmax(oXT + szXT, oKT + bO) : oO + bO;
  static constexpr size_t oDelta = al(endBig);
  static constexpr size_t oDpow = oDelta + NT * D * 4;
  static constexpr size_t oDinv = oDpow + NT * D * 4;
  static constexpr size_t oBeta = oDinv + NT * D * 4;
  static constexpr size_t oDecay = oBeta + KC * 4;
  static constexpr size_t bytes = al(oDecay + D * 4);
};

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

// ---------------------------------------------------------------------------
// the kernel
// ---------------------------------------------------------------------------
template <int C, int NC, bool F32, int MODE>
__global__ __launch_bounds__(NTHREADS, 1) void prefill_kernel(PrefillArgs a) {
  using L = Layout<C, NC, F32>;
  using T = typename Op<F32>::T;
  constexpr int NT = L::NT, KC = L::KC;
  constexpr int NCB = NC / 16;                         // 16-column blocks per workgroup
  constexpr int VS = (MODE == MODE_TRANSITION ? 2 * D : D) / NC;   // workgroups per unit
  extern __shared__ __align__(16) unsigned char smem[];
  T *sST = reinterpret_cast<T *>(smem + L::oST);
  T *sQT = reinterpret_cast<T *>(smem + L::oQT);
  T *sKD = reinterpret_cast<T *>(smem + L::oKD);
  T *sVT = reinterpret_cast<T *>(smem + L::oVT);
  T *sP = reinterpret_cast<T *>(smem + L::oP);
  float *sA = reinterpret_cast<float *>(smem + L::oA);
  T *sUT = reinterpret_cast<T *>(smem + L::oUT);
  T *sKF = reinterpret_cast<T *>(smem + L::oKFW);
  T *sW = sKF;                                         // -W, after KF is dead
  T *sKT = reinterpret_cast<T *>(smem + L::oKT);
  float *sX = reinterpret_cast<float *>(smem + L::oXT);
  T *sTT = reinterpret_cast<T *>(smem + L::oTT);
  float *sO = reinterpret_cast<float *>(smem + L::oO);
  float *sDelta = reinterpret_cast<float *>(smem + L::oDelta);
  float *sDpow = reinterpret_cast<float *>(smem + L::oDpow);
  float *sDinv = reinterpret_cast<float *>(smem + L::oDinv);
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
    for (int x = tid; x < D * KC; x += NTHREADS) { sKD[x] = T(0); sKT[x] = T(0); }
    for (int x = tid; x < NC * KC; x += NTHREADS) { sVT[x] = T(0); sUT[x] = T(0); }
    for (int x = tid; x < C * KC; x += NTHREADS) { sP[x] = T(0); sTT[x] = T(0); }
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
    }
#pragma unroll
  for (int ib = 0; ib < 2; ++ib)
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) {
      const int i0 = (2 * wave + ib) * 16 + 4 * lg, cl = cb * 16 + lr;
#pragma unroll
      for (int r = 0; r < 4; ++r) sST[cl * D + i0 + r] = Op<F32>::cvt(S[ib][cb][r]);
    }

  const int ch_begin = seg * a.seg_chunks;
  const int ch_end = min(a.n_chunks, ch_begin + a.seg_chunks);

  for (int chunk = ch_begin; chunk < ch_end; ++chunk) {
    const int t0 = chunk * C;
    const int nval = min(C, a.T - t0);
    const size_t tok0 = ((size_t)b * a.T + t0) * tok_stride + (size_t)h * D;   // (b, t0, h, 0)

    // ===== phase A: decay factors and operands (wave w handles token tile w) =====
    // lane: token tt = 16w + lr, channels ch(kb, e) = 32kb + 8lg + e.
    float Lc[32];                 // tile-relative cumulative log2-decay
    float kx[32], qx[32];
    const int tt = 16 * wave + lr;
    const bool tok_ok = (wave < NT) && (tt < nval);
    if (wave < NT) {
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        const int ch = 32 * kb + 8 * lg;
        float gg[8];
        if (tok_ok) {
          const size_t base = tok0 + (size_t)tt * tok_stride + ch;
          const float4 g0 = *reinterpret_cast<const float4 *>(a.g + base);
          const float4 g1 = *reinterpret_cast<const float4 *>(a.g + base + 4);
          gg[0] = g0.x; gg[1] = g0.y; gg[2] = g0.z; gg[3] = g0.w;
          gg[4] = g1.x; gg[5] = g1.y; gg[6] = g1.z; gg[7] = g1.w;
          const float4 k0 = load4<!F32>(a.k, base), k1 = load4<!F32>(a.k, base + 4);
          const float4 q0 = load4<!F32>(a.q, base), q1 = load4<!F32>(a.q, base + 4);
          kx[8 * kb + 0] = k0.x; kx[8 * kb + 1] = k0.y; kx[8 * kb + 2] = k0.z; kx[8 * kb + 3] = k0.w;
          kx[8 * kb + 4] = k1.x; kx[8 * kb + 5] = k1.y; kx[8 * kb + 6] = k1.z; kx[8 * kb + 7] = k1.w;
          qx[8 * kb + 0] = q0.x; qx[8 * kb + 1] = q0.y; qx[8 * kb + 2] = q0.z; qx[8 * kb + 3] = q0.w;
          qx[8 * kb + 4] = q1.x; qx[8 * kb + 5] = q1.y; qx[8 * kb + 6] = q1.z; qx[8 * kb + 7] = q1.w;
        } else {
#pragma unroll
          for (int e = 0; e < 8; ++e) { gg[e] = 0.f; kx[8 * kb + e] = 0.f; qx[8 * kb + e] = 0.f; }
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) Lc[8 * kb + e] = row_scan16(tok_ok ? log2_decay(gg[e]) : 0.f);
      }
      if (lr == 15) {
#pragma unroll
        for (int kb = 0; kb < 4; ++kb)
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const int ch = 32 * kb + 8 * lg + e;
            const float dl = Lc[8 * kb + e];
            sDelta[wave * D + ch] = dl;
            sDpow[wave * D + ch] = exp2_fast(dl);
            sDinv[wave * D + ch] = exp2_fast(-dl);
          }
      }
      if (lg == 0) sBeta[tt] = tok_ok ? a.beta[((size_t)b * a.T + t0 + tt) * a.H + h] : 0.f;
    }
    // value columns of this slice, transposed: V^T[c][t] (transition mode: columns < D
    // belong to the A part of the map and carry no value)
    {
      constexpr int per_tok = NC / 8;                  // 8-column groups per token
      for (int x = tid; x < C * per_tok; x += NTHREADS) {
        const int t = x / per_tok, cgrp = (x % per_tok) * 8;
        const int c = c0 + cgrp;
        float vv[8];
        const bool ok = t < nval && (MODE == MODE_OUTPUT || c >= D);
        if (ok) {
          const int cv = MODE == MODE_OUTPUT ? c : c - D;
          const size_t base = tok0 + (size_t)t * tok_stride + cv;
          const float4 v0 = load4<!F32>(a.v, base), v1 = load4<!F32>(a.v, base + 4);
          vv[0] = v0.x; vv[1] = v0.y; vv[2] = v0.z; vv[3] = v0.w;
          vv[4] = v1.x; vv[5] = v1.y; vv[6] = v1.z; vv[7] = v1.w;
        } else {
#pragma unroll
          for (int e = 0; e < 8; ++e) vv[e] = 0.f;
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) sVT[(cgrp + e) * KC + t] = Op<F32>::cvt(vv[e]);
      }
    }
    __syncthreads();   // tile totals, beta, V^T visible

    // per-lane operands from the tile factors
    using DiagV = typename Op<F32>::V8;
    f32x4 accA[NT], accP[NT];          // off-diagonal tiles (w, s'), compile-time index s'
    f32x4 accAd = zero4(), accPd = zero4();   // diagonal tile (w, w)
    float rkx[32], rqx[32];            // k e^{G_t - r_w}, q e^{G_t - r_w}
#pragma unroll
    for (int s = 0; s < NT; ++s) { accA[s] = zero4(); accP[s] = zero4(); }
    if (wave < NT) {
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        float E[8], F[8];
        float rk[8], rq[8], yd[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int ch = 32 * kb + 8 * lg + e;
          const float dl = sDelta[wave * D + ch];
          const float Lv = Lc[8 * kb + e];
          E[e] = exp2_fast(Lv);                      // e^{G_t - r_w}      in [e^-80, 1]
          F[e] = exp2_fast(dl - Lv);                 // e^{r_{w+1} - G_t}  in [e^-75, 1]
          float pre = 1.f, post = 1.f;
#pragma unroll
          for (int m = 0; m < NT; ++m) {
            const float dp = sDpow[m * D + ch];
            if (m < wave) pre *= dp;
            if (m > wave) post *= dp;
          }
          const float kk = kx[8 * kb + e], qq = qx[8 * kb + e];
          rk[e] = kk * E[e];
          rq[e] = qq * E[e];
          yd[e] = kk * F[e] * sDinv[wave * D + ch];   // k e^{r_w - G_t} in [0, e^80]|k|
          // chunk-level operands
          sQT[tt * D + ch] = Op<F32>::cvt(rq[e] * pre);                 // q e^{G_t}
          sKT[ch * KC + tt] = Op<F32>::cvt(rk[e] * pre);                // (k e^{G_t})^T
          sKD[ch * KC + tt] = Op<F32>::cvt(kk * F[e] * post);           // (k e^{G_C - G_t})^T
          sKF[tt * D + ch] = Op<F32>::cvt(kk * F[e]);                   // k e^{r_{w+1} - G_t}
          if (wave == 0 && lr == 0) {
            float dec = 1.f;
#pragma unroll
            for (int m = 0; m < NT; ++m) dec *= sDpow[m * D + ch];
            sDecay[ch] = dec;                                           // e^{G_C}
          }
        }
        // diagonal tile (w, w): operands straight from registers
        if constexpr (F32) {
          DiagV va{rk[0], rk[1], rk[2], rk[3], rk[4], rk[5], rk[6], rk[7]};
          DiagV vq{rq[0], rq[1], rq[2], rq[3], rq[4], rq[5], rq[6], rq[7]};
          DiagV vy{yd[0], yd[1], yd[2], yd[3], yd[4], yd[5], yd[6], yd[7]};
          accAd = Op<true>::mma(accAd, va, vy);
          if constexpr (MODE == MODE_OUTPUT) accPd = Op<true>::mma(accPd, vq, vy);
        } else {
          bf16x8 kh, kl, qh, ql, yh, yl;
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            kh[e] = static_cast<__bf16>(rk[e]);
            kl[e] = static_cast<__bf16>(rk[e] - static_cast<float>(kh[e]));
            qh[e] = static_cast<__bf16>(rq[e]);
            ql[e] = static_cast<__bf16>(rq[e] - static_cast<float>(qh[e]));
            yh[e] = static_cast<__bf16>(yd[e]);
            yl[e] = static_cast<__bf16>(yd[e] - static_cast<float>(yh[e]));
          }
          accAd = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kh, yh, accAd, 0, 0, 0);
          accAd = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kh, yl, accAd, 0, 0, 0);
          accAd = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kl, yh, accAd, 0, 0, 0);
          if constexpr (MODE == MODE_OUTPUT) {
            accPd = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qh, yh, accPd, 0, 0, 0);
            accPd = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qh, yl, accPd, 0, 0, 0);
            accPd = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ql, yh, accPd, 0, 0, 0);
          }
        }
        // off-diagonal row operands: scaled to the end of column tile s' (both <= 1)
        // their column operands (KF of tile s') are read after the barrier below
#pragma unroll
        for (int e = 0; e < 8; ++e) { rkx[8 * kb + e] = rk[e]; rqx[8 * kb + e] = rq[e]; }
      }
    }
    __syncthreads();   // KF, Qt, Kt^T, Kdec^T, decay visible

    // off-diagonal tiles (w, s'), s' < w: row operand k e^{G_t - r_w} * prod_{s'<m<w} D_m
    if (wave < NT) {
#pragma unroll
      for (int sp = 0; sp < NT - 1; ++sp) {
        if (sp < wave) {
#pragma unroll
          for (int kb = 0; kb < 4; ++kb) {
            typename Op<F32>::V8 va, vq;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
              const int ch = 32 * kb + 8 * lg + e;
              float fac = 1.f;
#pragma unroll
              for (int m = 0; m < NT; ++m)
                if (m > sp && m < wave) fac *= sDpow[m * D + ch];
              va[e] = Op<F32>::cvt(rkx[8 * kb + e] * fac);
              vq[e] = Op<F32>::cvt(rqx[8 * kb + e] * fac);
            }
            const typename Op<F32>::V8 vb = Op<F32>::ld8(sKF + (16 * sp + lr) * D + 32 * kb + 8 * lg);
            accA[sp] = Op<F32>::mma(accA[sp], va, vb);
            if constexpr (MODE == MODE_OUTPUT) accP[sp] = Op<F32>::mma(accP[sp], vq, vb);
          }
        }
      }
      // scale rows by beta, mask, store A (fp32) and P; P's blocks above the diagonal
      // are stored as zeros (A's are never read)
#pragma unroll
      for (int sp = 0; sp < NT; ++sp) {
        if (sp > wave) {
          if constexpr (MODE == MODE_OUTPUT) {
#pragma unroll
            for (int r = 0; r < 4; ++r) sP[(16 * wave + 4 * lg + r) * KC + 16 * sp + lr] = Op<F32>::cvt(0.f);
          }
        } else {
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int ti = 4 * lg + r;                 // row within the tile
            const int t = 16 * wave + ti, j = 16 * sp + lr;
            const bool diag = sp == wave;
            const float av = diag ? (ti > lr ? accAd[r] * sBeta[t] : 0.f) : accA[sp][r] * sBeta[t];
            const float pv = diag ? (ti >= lr ? accPd[r] : 0.f) : accP[sp][r];
            sA[t * C + j] = av;
            if constexpr (MODE == MODE_OUTPUT) sP[t * KC + j] = Op<F32>::cvt(pv);
          }
        }
      }
    }
    __syncthreads();   // A complete

    // ===== solve: X = (I + A)^-1 (blocked), T = X diag(beta) =====
    // diagonal blocks: forward substitution, one column per lane (lanes 0..15)
    if (wave < NT && lane < 16) {
      const int j = lane;
      float x[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        float acc = (i == j) ? 1.f : 0.f;
#pragma unroll
        for (int m = 0; m < i; ++m) acc -= sA[(16 * wave + i) * C + 16 * wave + m] * x[m];
        x[i] = acc;
      }
#pragma unroll
      for (int i = 0; i < 16; ++i) sX[(16 * wave + i) * C + 16 * wave + j] = x[i];
    }
    __syncthreads();
    // off-diagonal blocks by block diagonal d: X_{s,s-d} = -X_ss sum_m A_{s,m} X_{m,s-d}
#pragma unroll
    for (int d = 1; d < NT; ++d) {
      const int s = wave + d;                          // wave w computes block (w+d, w)
      if (s < NT) {
        const int cs = 16 * (s - d);
        f32x4 y = zero4();
        for (int kk = 0; kk < 4 * d; ++kk) {
          const int kidx = cs + 4 * kk + lg;
          y = __builtin_amdgcn_mfma_f32_16x16x4f32(sA[(16 * s + lr) * C + kidx],
                                                  sX[kidx * C + cs + lr], y, 0, 0, 0);
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) sX[(16 * s + 4 * lg + r) * C + cs + lr] = y[r];
        f32x4 z = zero4();
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
          const int kidx = 16 * s + 4 * kk + lg;
          z = __builtin_amdgcn_mfma_f32_16x16x4f32(sX[(16 * s + lr) * C + kidx],
                                                  sX[kidx * C + cs + lr], z, 0, 0, 0);
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) sX[(16 * s + 4 * lg + r) * C + cs + lr] = -z[r];
      }
      __syncthreads();
    }
    // T[t][j] = X[t][j] beta_j on and below the diagonal (X's upper part is not stored)
    {
      constexpr int PER = (C * KC + NTHREADS - 1) / NTHREADS;
      float tv[PER];
#pragma unroll
      for (int u = 0; u < PER; ++u) {
        const int x = tid + u * NTHREADS;
        const int t = x / KC, j = x % KC;
        tv[u] = (x < C * KC && j < C && (j >> 4) <= (t >> 4)) ? sX[t * C + j] * sBeta[j] : 0.f;
      }
      if constexpr (L::ALIAS) __syncthreads();
#pragma unroll
      for (int u = 0; u < PER; ++u) {
        const int x = tid + u * NTHREADS;
        if (x < C * KC) sTT[x] = Op<F32>::cvt(tv[u]);
      }
    }
    __syncthreads();

    // ===== W^T = Kt^T T^T  ->  store -W[t][i] (overwrites KF) =====
    {
      constexpr int NTILE = 8 * NT;                      // (i-block, t-block)
      for (int tile = wave; tile < NTILE; tile += 4) {
        const int ib = tile / NT, tb = tile % NT;
        f32x4 acc = zero4();
#pragma unroll
        for (int kb = 0; kb < KC / 32; ++kb)
          acc = mma_lds<F32>(acc, sKT + (16 * ib) * KC + 32 * kb, KC, sTT + (16 * tb) * KC + 32 * kb, KC, lane);
        // acc[r] = W^T[16ib + 4lg + r][16tb + lr]
#pragma unroll
        for (int r = 0; r < 4; ++r) sW[(16 * tb + lr) * D + 16 * ib + 4 * lg + r] = Op<F32>::cvt(-acc[r]);
      }
    }
    __syncthreads();

    // ===== U = T V - W S  ->  U^T[c][t] =====
    {
      constexpr int NTILE = NT * NCB;
      for (int tile = wave; tile < NTILE; tile += 4) {
        const int tb = tile / NCB, cb = tile % NCB;
        f32x4 acc = zero4();
#pragma unroll
        for (int kb = 0; kb < KC / 32; ++kb)
          acc = mma_lds<F32>(acc, sTT + (16 * tb) * KC + 32 * kb, KC, sVT + (16 * cb) * KC + 32 * kb, KC, lane);
#pragma unroll
        for (int kb = 0; kb < 4; ++kb)
          acc = mma_lds<F32>(acc, sW + (16 * tb) * D + 32 * kb, D, sST + (16 * cb) * D + 32 * kb, D, lane);
        // acc[r] = U[16tb + 4lg + r][16cb + lr]
#pragma unroll
        for (int r = 0; r < 4; ++r) sUT[(16 * cb + lr) * KC + 16 * tb + 4 * lg + r] = Op<F32>::cvt(acc[r]);
      }
    }
    __syncthreads();

    // ===== O = Qt S + P U  (output mode) =====
    if constexpr (MODE == MODE_OUTPUT) {
      constexpr int NTILE = NT * NCB;
      for (int tile = wave; tile < NTILE; tile += 4) {
        const int tb = tile / NCB, cb = tile % NCB;
        f32x4 acc = zero4();
#pragma unroll
        for (int kb = 0; kb < 4; ++kb)
          acc = mma_lds<F32>(acc, sQT + (16 * tb) * D + 32 * kb, D, sST + (16 * cb) * D + 32 * kb, D, lane);
#pragma unroll
        for (int kb = 0; kb < KC / 32; ++kb)
          acc = mma_lds<F32>(acc, sP + (16 * tb) * KC + 32 * kb, KC, sUT + (16 * cb) * KC + 32 * kb, KC, lane);
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
      __syncthreads();   // O reads of S^T complete (and staging visible)
      if (a.fused_gate) {
        // per-head RMSNorm over the 128 value columns, then the sigmoid gate:
        // 4 tokens per wave pass, 16 lanes x 8 columns per token
        for (int t = 4 * wave + lg; t < C; t += 16) {
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
            const float4 g0 = load4<!F32>(a.gate, base), g1 = load4<!F32>(a.gate, base + 4);
            const float gv[8] = {g0.x, g0.y, g0.z, g0.w, g1.x, g1.y, g1.z, g1.w};
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
      float dec[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) dec[r] = sDecay[i0 + 4 * lg + r];
#pragma unroll
      for (int cb = 0; cb < NCB; ++cb) {
        f32x4 acc = S[ib][cb];
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[r] *= dec[r];
#pragma unroll
        for (int kb = 0; kb < KC / 32; ++kb)
          acc = mma_lds<F32>(acc, sKD + i0 * KC + 32 * kb, KC, sUT + (16 * cb) * KC + 32 * kb, KC, lane);
        S[ib][cb] = acc;
#pragma unroll
        for (int r = 0; r < 4; ++r) sST[(16 * cb + lr) * D + i0 + 4 * lg + r] = Op<F32>::cvt(acc[r]);
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
    e = launch_mode<MODE_TRANSITION>(t, d.chunk, f32, nc, s);
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
