// Chunkwise KDA prefill, part 1: the per-chunk work that does not depend on the state.
//
// The sequence is cut into chunks; chunks are linked by the state recurrence and
// computed inside with matrix products ("xhh.club" tag page 结构, entry on the chunkwise
// algorithm).  For a chunk of C tokens, with G the inclusive cumulative sum of the
// floored log-decay over the chunk (per key channel):
//
//   A  = StrictLower(diag(beta) (K e^G)(K e^-G)^T)      C x C   (decay-weighted K K^T)
//   P  = Lower((Q e^G)(K e^-G)^T)                       C x C   (decay-weighted Q K^T)
//   T  = (I + A)^-1 diag(beta)                          triangular solve (WY/UT form)
//   W  = T (K e^G),   Qt = Q e^G,   Kdec = K e^{G_C - G},   decay = e^{G_C}
//
// None of these depends on the state entering the chunk, so every (sequence, head,
// chunk) is prepared independently here, fully in parallel, and written to a record
// (see Rec in tiles.h) that the sequential state kernel reads.
//
// Numerics ("xhh.club", chunkwise entry; "nlpx.cn" K3 guide section 6).  e^{+-G} over a
// whole chunk over/underflows fp32, so A and P are formed on 16-token tiles with a
// tile-local reference point r: for a diagonal tile the row factor e^{G_t - r} lies in
// [e^-80, 1] and the column factor e^{r - G_j} in [1, e^80] only because every step's
// log-decay is floored at -5 (16 * 5 = 80 < ln(FLT_MAX) = 88.7).  Those factors need a
// wide exponent, so diagonal tiles run as BF16 MFMA, P's with each operand split into
// bf16 high and low parts (three products).  In off-diagonal tiles both factors are
// <= 1 and run as fp16 MFMA, as do the solve and W; all accumulation is fp32.  With
// fp32 inputs every product runs as fp32 MFMA instead.
#include <atomic>
#include <utility>

#include "internal.h"
#include "tiles.h"

namespace kda {
namespace {

struct PrepArgs {
  const void *q, *k;
  const float *g, *beta;
  unsigned char *rec;     // n_recs records of Rec<C, F32>::bytes
  int T, H, n_chunks;
  int64_t n_recs;         // B * H * n_chunks
  int chunk_major;        // workgroup order: all heads of a chunk, then the next chunk
};

template <int C, bool F32>
struct PrepLayout {
  using T = typename Op<F32>::T;
  static constexpr int NT = C / 16;
  static constexpr int KC = C < 32 ? 32 : C;          // token contraction extent (zero padded)
  static constexpr size_t E = sizeof(T);
  static constexpr size_t al(size_t x) { return (x + 15) & ~size_t(15); }
  static constexpr size_t cmax(size_t a, size_t b) { return a > b ? a : b; }
  static constexpr int NFAC = NT > 2 ? (NT - 1) * (NT - 2) / 2 : 1;   // tile pairs w - s' >= 2
  static constexpr int NBO = NT * (NT - 1) / 2;       // off-diagonal blocks of A below the diagonal
  static constexpr size_t bKT = (size_t)KC * D * E;   // K e^G      [t][i]  (rows >= C zero)
  static constexpr size_t bKF = (size_t)KC * D * E;   // KF         [t][i]  (rows >= C zero)
  static constexpr size_t bTt = (size_t)KC * C * E;   // T^T        [j][t]  (rows >= C zero)
  static constexpr size_t bAd = (size_t)NT * 256 * 4; // diagonal blocks of A, fp32
  static constexpr size_t bVec = (size_t)(3 * NT + NFAC) * D * 4;   // per-tile decay vectors
  static constexpr size_t bAo = NBO > 0 ? (size_t)NBO * 256 * 2 : 0;   // A, off-diagonal blocks, fp16
  static constexpr size_t bX = (size_t)NT * 256 * E;  // inverses of the diagonal blocks of I + A
  // K e^G is written only after KF is dead (from the raw k still in registers), so it
  // shares KF's storage
  static constexpr size_t oKF = 0;
  static constexpr size_t oKT = oKF;
  // T^T is written only after the diagonal A blocks and the per-tile vectors are dead,
  // so it shares their storage
  static constexpr size_t oTt = al(oKF + (bKF > bKT ? bKF : bKT));
  static constexpr size_t oAd = oTt;
  static constexpr size_t oDpow = oAd + bAd;                    // D_m = e^{tile m total}
  static constexpr size_t oPre = oDpow + (size_t)NT * D * 4;    // prod_{m<w} D_m
  static constexpr size_t oPost = oPre + (size_t)NT * D * 4;    // prod_{m>w} D_m
  static constexpr size_t oFac = oPost + (size_t)NT * D * 4;    // prod_{s'<m<w} D_m
  static constexpr size_t oAo = al(oTt + cmax(bTt, bAd + bVec));
  static constexpr size_t oX = al(oAo + bAo);
  static constexpr size_t oBeta = al(oX + bX);
  static constexpr size_t oDecay = oBeta + (size_t)KC * 4;
  static constexpr size_t bytes = al(oDecay + D * 4);
};

// Raw inputs of one chunk held in registers between the load and their use.
template <bool F32>
struct RawPrep {
  float4 g[8];          // log-decay of this lane's token: g[2kb] channels 32kb + 4lg + (0..3),
                        // g[2kb + 1] channels 32kb + 16 + 4lg + (0..3)
  Q8<F32> k[4], q[4];
  float beta;
  bool ok;              // the lane's token lies in the sequence (else its inputs read as 0)
};

// Global loads of one chunk, zero-filled past the sequence end.  Wave w < NT loads
// token tile w: lane (lr, lg) gets token 16w + lr and, per 32-channel block kb, the
// channels of the split contraction order, 32kb + 4lg + (0..3) and 32kb + 16 + 4lg +
// (0..3) (see ld_n_split): every operand built from them is already in that order.
template <int C, bool F32>
__device__ __forceinline__ void load_prep(RawPrep<F32> &r, const PrepArgs &a, int64_t rec, int tid) {
  constexpr int NT = C / 16;
  const int wave = tid >> 6, lane = tid & 63, lr = lane & 15, lg = lane >> 4;
  const int bh = (int)(rec / a.n_chunks), chunk = (int)(rec % a.n_chunks);
  const int b = bh / a.H, h = bh % a.H;
  const int t0 = chunk * C;
  const int tt = 16 * wave + lr;
  const bool ok = wave < NT && t0 + tt < a.T;
  // Lanes past the sequence end (or of waves without a tile) load the chunk's first
  // token instead and use zeros, so the loads are branch-free.  They are issued in the
  // order of first use (beta and g in the decay scan, then k and q): the wait counter
  // completes in issue order, so the scan does not wait for k and q.
  const size_t tok = (size_t)b * a.T + t0 + (ok ? tt : 0);
  const size_t base = (tok * a.H + h) * D + 4 * lg;
  r.ok = ok;
  r.beta = a.beta[tok * a.H + h];
#pragma unroll
  for (int kb = 0; kb < 4; ++kb) {
    r.g[2 * kb] = *reinterpret_cast<const float4 *>(a.g + base + 32 * kb);
    r.g[2 * kb + 1] = *reinterpret_cast<const float4 *>(a.g + base + 32 * kb + 16);
  }
  __builtin_amdgcn_sched_barrier(0);   // keep this order
#pragma unroll
  for (int kb = 0; kb < 4; ++kb) r.k[kb] = load_q8_split<F32>(a.k, base + 32 * kb);
#pragma unroll
  for (int kb = 0; kb < 4; ++kb) r.q[kb] = load_q8_split<F32>(a.q, base + 32 * kb);
}

// Workgroup barrier for LDS only: waits for this wave's LDS accesses, not for its global
// loads, so that loads issued earlier stay in flight across it (the kernel never reads
// global memory it writes).
__device__ __forceinline__ void lds_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0); vmcnt and expcnt not waited for
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
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

// Column j of the inverse of a unit lower triangular 16x16 block I + A by forward
// substitution, x_i = [i == j] - sum_{m<i} A[i][m] x_m.  Lane j of each 16-lane row
// holds row j of its block's A in rowA; A[i][m] is broadcast from lane i of the row.
template <int I>
__device__ __forceinline__ void invert_row(const float *rowA, float *x, int j) {
  float acc = 0.f;
#pragma unroll
  for (int m = 0; m < I; ++m) {
    const float a = __builtin_bit_cast(
        float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, rowA[m]), 0x150 + I, 0xf, 0xf, false));
    acc = fmaf(a, x[m], acc);
  }
  x[I] = (I == j ? 1.f : 0.f) - acc;
  __builtin_amdgcn_sched_barrier(0);   // keep the broadcasts of later rows from being hoisted
}

template <int... Is>
__device__ __forceinline__ void invert_unit_lower(const float *rowA, float *x, int j, std::integer_sequence<int, Is...>) {
  (invert_row<Is>(rowA, x, j), ...);
}

template <int C, bool F32>
// 34 KB of LDS and at most 128 VGPRs at C = 64: four workgroups share a CU, and one's
// loads overlap the others' arithmetic
__global__ __launch_bounds__(NTHREADS, F32 ? 1 : (C == 64 ? 4 : 2)) void chunk_prep_kernel(PrepArgs a) {
  using L = PrepLayout<C, F32>;
  using R = Rec<C, F32>;
  using T = typename Op<F32>::T;
  using V8 = typename Op<F32>::V8;
  constexpr int NT = L::NT, KC = L::KC, KB = R::KB;
  static_assert(!F32 || C == 16, "fp32 operands are used with 16-token chunks only");
  extern __shared__ __align__(16) unsigned char smem[];
  T *sKT = reinterpret_cast<T *>(smem + L::oKT);       // rows of D
  T *sKF = reinterpret_cast<T *>(smem + L::oKF);       // rows of D
  T *sTt = reinterpret_cast<T *>(smem + L::oTt);       // rows of C
  float *sAd = reinterpret_cast<float *>(smem + L::oAd);
  _Float16 *sAo = reinterpret_cast<_Float16 *>(smem + L::oAo);
  T *sX = reinterpret_cast<T *>(smem + L::oX);
  float *sDpow = reinterpret_cast<float *>(smem + L::oDpow);
  float *sPre = reinterpret_cast<float *>(smem + L::oPre);
  float *sPost = reinterpret_cast<float *>(smem + L::oPost);
  float *sFac = reinterpret_cast<float *>(smem + L::oFac);
  float *sBeta = reinterpret_cast<float *>(smem + L::oBeta);
  float *sDecay = reinterpret_cast<float *>(smem + L::oDecay);

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int lr = lane & 15, lg = lane >> 4;
  const int tt = 16 * wave + lr;                       // this lane's token in phase A

  // zero the padded token range of the contraction buffers (only when KC > C; the
  // rows of T^T past the chunk are cleared in the solve, when its storage is free)
  if constexpr (KC > C) {
    for (int x = tid; x < (KC - C) * D; x += NTHREADS) { sKT[C * D + x] = T(0); sKF[C * D + x] = T(0); }
  }

  if ((int64_t)blockIdx.x >= a.n_recs) return;
  int64_t rec = blockIdx.x;                            // records stay [B * H][n_chunks]
  if (a.chunk_major) {
    const int64_t n_bh = a.n_recs / a.n_chunks;
    rec = ((int64_t)blockIdx.x % n_bh) * a.n_chunks + (int64_t)blockIdx.x / n_bh;
  }
  RawPrep<F32> raw;
  load_prep<C, F32>(raw, a, rec, tid);
  {
    unsigned char *out = a.rec + (size_t)rec * R::bytes;

    // ===== A1: tile-relative cumulative log2-decay; tile totals; beta =====
    float Lc[32];
    if (wave < NT) {
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        const int ch = 32 * kb + 4 * lg;               // channels ch + (0..3), ch + 16 + (0..3)
        float gg[8];
        f8_from(gg, raw.g[2 * kb], raw.g[2 * kb + 1]);
#pragma unroll
        for (int e = 0; e < 8; ++e) gg[e] = raw.ok ? gg[e] : 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) Lc[8 * kb + e] = log2_decay(gg[e]);
        scan_step<0x111>(Lc + 8 * kb);
        scan_step<0x112>(Lc + 8 * kb);
        scan_step<0x114>(Lc + 8 * kb);
        scan_step<0x118>(Lc + 8 * kb);
        if (lr == 15) {                                  // tile decays D_w = e^{tile total}
          float dp[8];
#pragma unroll
          for (int e = 0; e < 8; ++e) dp[e] = exp2_fast(Lc[8 * kb + e]);
          float *pp = sDpow + wave * D + ch;
          *reinterpret_cast<float4 *>(pp) = make_float4(dp[0], dp[1], dp[2], dp[3]);
          *reinterpret_cast<float4 *>(pp + 16) = make_float4(dp[4], dp[5], dp[6], dp[7]);
        }
      }
      if (lg == 0) sBeta[tt] = raw.ok ? raw.beta : 0.f;
    }
    lds_barrier();   // k and q may still be in flight

    // ===== per (tile, channel): prefix and suffix decay products, the chunk decay,
    // and the factors between tiles two or more apart =====
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
    lds_barrier();

    // ===== A2: decay factors, diagonal tile, chunk-level operands =====
    V8 rkx[4], rqx[4];                                 // k e^{G_t - r_w}, q e^{G_t - r_w}
    // P is formed transposed: a P^T tile (s, w) in MFMA output layout holds, per lane,
    // token 16w + lr and keys 16s + 4lg + r, which are exactly the lane's elements of
    // P's split-order operand fragment, so P is exported without going through LDS
    f32x4 accPd = zero4(), accP[NT];                   // P^T tiles (w, w) and (s', w)
#pragma unroll
    for (int sp = 0; sp < NT; ++sp) accP[sp] = zero4();
    if (wave < NT) {
      f32x4 accAd = zero4();                           // diagonal tile (w, w) of A
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        const int ch = 32 * kb + 4 * lg;               // channels ch + (0..3), ch + 16 + (0..3)
        float pre[8], dw[8];
        f8_from(pre, *reinterpret_cast<const float4 *>(sPre + wave * D + ch),
                *reinterpret_cast<const float4 *>(sPre + wave * D + ch + 16));
        f8_from(dw, *reinterpret_cast<const float4 *>(sDpow + wave * D + ch),
                *reinterpret_cast<const float4 *>(sDpow + wave * D + ch + 16));
        float rk[8], rq[8], yd[8], xf[8];
        V8 xq;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float Lv = Lc[8 * kb + e];
          const float kk = raw.ok ? q8_at<F32>(raw.k[kb], e) : 0.f, qq = raw.ok ? q8_at<F32>(raw.q[kb], e) : 0.f;
          const float E = exp2_fast(Lv);               // e^{G_t - r_w}      in [e^-80, 1]
          const float En = exp2_fast(-Lv);             // e^{r_w - G_t}      in [1, e^80]
          rk[e] = kk * E;
          rq[e] = qq * E;
          yd[e] = kk * En;                             // k e^{r_w - G_t}
          xf[e] = yd[e] * dw[e];                       // k e^{r_{w+1} - G_t}, in [e^-75, 1] |k|
          xq[e] = Op<F32>::cvt(rq[e] * pre[e]);        // q e^{G_t}
          rkx[kb][e] = Op<F32>::cvt(rk[e]);            // kept for the off-diagonal tiles
          rqx[kb][e] = Op<F32>::cvt(rq[e]);
        }
        // Qt goes out directly: this lane layout is the operand fragment (tile w, kb)
        Op<F32>::store(reinterpret_cast<T *>(out + R::frag(R::oQ, wave * 4 + kb, lane)), xq);
        st4<F32, D>(sKF, tt, ch, xf[0], xf[1], xf[2], xf[3]);
        st4<F32, D>(sKF, tt, ch + 16, xf[4], xf[5], xf[6], xf[7]);
        // diagonal tile (w, w) straight from registers: A in bf16, P with bf16 hi/lo
        if constexpr (F32) {
          const V8 va{rk[0], rk[1], rk[2], rk[3], rk[4], rk[5], rk[6], rk[7]};
          const V8 vq{rq[0], rq[1], rq[2], rq[3], rq[4], rq[5], rq[6], rq[7]};
          const V8 vy{yd[0], yd[1], yd[2], yd[3], yd[4], yd[5], yd[6], yd[7]};
          accAd = Op<true>::mma(accAd, va, vy);
          accPd = Op<true>::mma(accPd, vy, vq);
        } else {
          bf16x8 kh, yh, qh, ql, yl;
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            kh[e] = static_cast<__bf16>(rk[e]);
            yh[e] = static_cast<__bf16>(yd[e]);
            qh[e] = static_cast<__bf16>(rq[e]);
            ql[e] = static_cast<__bf16>(rq[e] - static_cast<float>(qh[e]));
            yl[e] = static_cast<__bf16>(yd[e] - static_cast<float>(yh[e]));
          }
          accAd = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kh, yh, accAd, 0, 0, 0);
          accPd = __builtin_amdgcn_mfma_f32_16x16x32_bf16(yh, qh, accPd, 0, 0, 0);
          accPd = __builtin_amdgcn_mfma_f32_16x16x32_bf16(yl, qh, accPd, 0, 0, 0);
          accPd = __builtin_amdgcn_mfma_f32_16x16x32_bf16(yh, ql, accPd, 0, 0, 0);
        }
      }
      // diagonal tile: A (beta rows, strictly lower, fp32); P^T keeps keys j <= t
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int ti = 4 * lg + r, t = 16 * wave + ti;
        sAd[wave * 256 + ti * 16 + lr] = ti > lr ? accAd[r] * sBeta[t] : 0.f;
        accPd[r] = ti <= lr ? accPd[r] : 0.f;
      }
    }
    lds_barrier();   // KF, Kt, decay, diagonal A/P visible

    // ===== A3: wave 0 inverts every diagonal block of I + A (one column per lane);
    // waves w >= 1 compute the off-diagonal tiles (w, s'), s' < w, with row operand
    // k e^{G_t - r_w} prod_{s'<m<w} D_m and column operand KF of tile s' (both <= 1) ====
    if (wave == 0) {
      const int bb = lane >> 4, j = lane & 15;
      float rowA[16], x[16];
      if (bb < NT) {
#pragma unroll
        for (int m4 = 0; m4 < 4; ++m4) {
          const float4 v = *reinterpret_cast<const float4 *>(sAd + bb * 256 + j * 16 + 4 * m4);
          rowA[4 * m4] = v.x; rowA[4 * m4 + 1] = v.y; rowA[4 * m4 + 2] = v.z; rowA[4 * m4 + 3] = v.w;
        }
      } else {
#pragma unroll
        for (int m = 0; m < 16; ++m) rowA[m] = 0.f;
      }
      invert_unit_lower(rowA, x, j, std::make_integer_sequence<int, 16>{});
      if (bb < NT) {
#pragma unroll
        for (int i = 0; i < 16; ++i) sX[bb * 256 + i * 16 + j] = static_cast<T>(x[i]);
      }
    } else if (wave < NT) {
      f32x4 accA[NT];
#pragma unroll
      for (int sp = 0; sp < NT; ++sp) accA[sp] = zero4();
#pragma unroll
      for (int sp = 0; sp < NT - 1; ++sp) {
        if (sp < wave) {
#pragma unroll
          for (int kb = 0; kb < 4; ++kb) {
            const int ch = 32 * kb + 4 * lg;
            V8 va = rkx[kb], vq = rqx[kb];
            if (sp + 1 < wave) {                         // tiles two or more apart: scale by
              const int pi = (wave - 2) * (wave - 1) / 2 + sp;   // prod_{s'<m<w} D_m
              float fac[8];
              f8_from(fac, *reinterpret_cast<const float4 *>(sFac + pi * D + ch),
                      *reinterpret_cast<const float4 *>(sFac + pi * D + ch + 16));
              V8 vf;
#pragma unroll
              for (int e = 0; e < 8; ++e) vf[e] = Op<F32>::cvt(fac[e]);
              va = va * vf;
              vq = vq * vf;
            }
            const V8 vb = ld_n_split<F32, D>(sKF, 16 * sp, 32 * kb, lane);
            accA[sp] = Op<F32>::mma(accA[sp], va, vb);
            accP[sp] = Op<F32>::mma(accP[sp], vb, vq);
          }
        }
      }
#pragma unroll
      for (int sp = 0; sp < NT - 1; ++sp) {
        if (sp < wave) {
#pragma unroll
          for (int r = 0; r < 4; ++r) {               // block (w, s'), row 4lg + r, column lr
            const int t = 16 * wave + 4 * lg + r;
            sAo[((wave * (wave - 1)) / 2 + sp) * 256 + (4 * lg + r) * 16 + lr] =
                static_cast<_Float16>(accA[sp][r] * sBeta[t]);
          }
        }
      }
    }
    // P fragments (tile w, kb) from the P^T tiles (2kb, w) and (2kb + 1, w)
    if (wave < NT) {
      auto pt = [&](int sp) __attribute__((always_inline)) {
        return sp < wave ? accP[sp] : sp == wave ? accPd : zero4();
      };
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
        if (R::nz(wave, kb))                           // blocks above the diagonal are not stored
          Op<F32>::store(reinterpret_cast<T *>(out + R::frag(R::oP, R::tri(wave, kb), lane)),
                         frag_from<F32>(pt(2 * kb), pt(2 * kb + 1)));
    }

    // Kdec^T fragments: Kdec = KF * prod_{m>w} D_m, read transposed from KF.  Lane
    // (lr, lg) of fragment (ib, kb) holds channel 16ib + lr of tokens 32kb + 4lg + e
    // (tile 2kb) and 32kb + 16 + 4lg + e (tile 2kb + 1).
    for (int f = wave; f < R::nK; f += 4) {
      const int ib = f / KB, kb = f % KB;
      const float post0 = sPost[(2 * kb) * D + 16 * ib + lr];
      const float post1 = 2 * kb + 1 < NT ? sPost[(2 * kb + 1) * D + 16 * ib + lr] : 0.f;
      V8 v = ld_t_split<F32, D>(sKF, 32 * kb, 16 * ib, lane);
#pragma unroll
      for (int e = 0; e < 8; ++e) v[e] = Op<F32>::cvt(static_cast<float>(v[e]) * (e < 4 ? post0 : post1));
      Op<F32>::store(reinterpret_cast<T *>(out + R::frag(R::oK, f, lane)), v);
    }
    lds_barrier();   // A, P, diagonal inverses complete; KF dead
    // K e^G = (k e^{G_t - r_w}) prod_{m<w} D_m into KF's storage, for W
    if (wave < NT) {
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        const int ch = 32 * kb + 4 * lg;
        float pre[8];
        f8_from(pre, *reinterpret_cast<const float4 *>(sPre + wave * D + ch),
                *reinterpret_cast<const float4 *>(sPre + wave * D + ch + 16));
        float xk[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) xk[e] = static_cast<float>(rkx[kb][e]) * pre[e];
        st4<F32, D>(sKT, tt, ch, xk[0], xk[1], xk[2], xk[3]);
        st4<F32, D>(sKT, tt, ch + 16, xk[4], xk[5], xk[6], xk[7]);
      }
    }
    lds_barrier();   // K e^G complete; the per-tile vectors are dead

    // ===== solve: wave w walks down column block w of X = (I + A)^-1:
    // X_{s,w} = -X_ss sum_{w<=m<s} A_{s,m} X_{m,w}; a 16x16 result in MFMA output layout
    // is the B operand layout of the K=16 MFMA, so the blocks stay in registers.
    // Then T[:, block w] = X[:, block w] diag(beta), stored as T^T [j][t]. =====
    if constexpr (KC > C) {                           // T^T rows past the chunk
      for (int x = tid; x < (KC - C) * C; x += NTHREADS) sTt[C * C + x] = T(0);
    }
    if (wave < NT) {
      const int n = lr;                                 // column within the block
      const float bj = sBeta[16 * wave + n];
      f32x4 xc[NT];
#pragma unroll
      for (int s = 0; s < NT; ++s) {
        if (s == wave) {
#pragma unroll
          for (int r = 0; r < 4; ++r) xc[s][r] = static_cast<float>(sX[wave * 256 + (4 * lg + r) * 16 + n]);
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
                const f16x4 a4 = *reinterpret_cast<const f16x4 *>(sAo + ((s * (s - 1)) / 2 + m) * 256 + lr * 16 + 4 * lg);
                const f16x4 b4{(_Float16)xc[m][0], (_Float16)xc[m][1], (_Float16)xc[m][2], (_Float16)xc[m][3]};
                y = __builtin_amdgcn_mfma_f32_16x16x16f16(a4, b4, y, 0, 0, 0);
              }
            }
            const f16x4 a4 = *reinterpret_cast<const f16x4 *>(reinterpret_cast<const _Float16 *>(sX) + s * 256 + lr * 16 + 4 * lg);
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
    lds_barrier();   // T complete

    // ===== W = T (K e^G): fragment (tb, kb) straight from the two W^T tiles (2kb, tb)
    // and (2kb + 1, tb), each W^T = Kt^T T^T over the chunk's tokens =====
#pragma unroll
    for (int m = 0; m < R::nW / 4; ++m) {
      const int f = wave + 4 * m, tb = f / 4, kb = f % 4;
      f32x4 w0 = zero4(), w1 = zero4();
#pragma unroll
      for (int kc = 0; kc < KB; ++kc) {
        const V8 b = ld_t<F32, C>(sTt, 32 * kc, 16 * tb, lane);
        w0 = Op<F32>::mma(w0, ld_t<F32, D>(sKT, 32 * kc, 32 * kb, lane), b);
        w1 = Op<F32>::mma(w1, ld_t<F32, D>(sKT, 32 * kc, 32 * kb + 16, lane), b);
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) {                   // stored negated
        w0[r] = -w0[r];
        w1[r] = -w1[r];
      }
      Op<F32>::store(reinterpret_cast<T *>(out + R::frag(R::oW, f, lane)), frag_from<F32>(w0, w1));
    }
    // T fragments and the chunk decay
    for (int f = wave; f < NT * KB; f += 4) {
      const int tb = f / KB, kb = f % KB;
      if (R::nz(tb, kb))                               // blocks above the diagonal are not stored
        Op<F32>::store(reinterpret_cast<T *>(out + R::frag(R::oT, R::tri(tb, kb), lane)),
                       ld_t_split<F32, C>(sTt, 32 * kb, 16 * tb, lane));
    }
    if (tid < D / 4)
      reinterpret_cast<float4 *>(out + R::oDec)[tid] = reinterpret_cast<const float4 *>(sDecay)[tid];
  }
}

template <int C, bool F32>
hipError_t launch_prep_t(const PrepArgs &a, hipStream_t s) {
  using L = PrepLayout<C, F32>;
  static_assert(F32 || C != 64 || L::bytes <= 40 * 1024, "four workgroups per CU must fit in LDS");
  static_assert(L::bytes <= 53 * 1024, "three workgroups per CU must fit in LDS");
  auto kern = chunk_prep_kernel<C, F32>;
  static std::atomic<bool> attr_set{false};   // the attribute is per function, set once
  if (!attr_set.load(std::memory_order_acquire)) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)L::bytes);
    if (e != hipSuccess) return e;
    attr_set.store(true, std::memory_order_release);
  }
  // one workgroup per record; several resident per CU overlap one's loads with
  // another's arithmetic
  hipLaunchKernelGGL(kern, dim3(static_cast<unsigned>(a.n_recs)), dim3(NTHREADS), L::bytes, s, a);
  return hipGetLastError();
}

}  // namespace

size_t prefill_record_bytes(int chunk, bool f32) {
  if (f32) return Rec<16, true>::bytes;
  return chunk == 16 ? Rec<16, false>::bytes : Rec<64, false>::bytes;
}

hipError_t launch_prefill_prep(const kda_prefill_desc &d, int n_chunks, void *records, hipStream_t s) {
  PrepArgs a{};
  a.q = d.q; a.k = d.k; a.g = d.g; a.beta = d.beta;
  a.rec = static_cast<unsigned char *>(records);
  a.T = d.T; a.H = d.H; a.n_chunks = n_chunks;
  a.n_recs = (int64_t)d.B * d.H * n_chunks;
  if (a.n_recs == 0) return hipSuccess;
  // The workgroups resident at one time (four per CU) are consecutive ids.  In head-major
  // order, with 1024 or more chunks per head they all read one head: 256 bytes of every
  // token row of q, k and g.  Chunk-major order then makes them read whole token rows
  // (131k workload: prep 829 -> 778 us).  With fewer chunks head-major order already
  // spans several heads and measured slightly faster for the passes after it.
  a.chunk_major = n_chunks >= 4 * kCUs;
  if (d.in_dtype == KDA_F32) return launch_prep_t<16, true>(a, s);
  if (d.chunk == 16) return launch_prep_t<16, false>(a, s);
  return launch_prep_t<64, false>(a, s);
}

}  // namespace kda
