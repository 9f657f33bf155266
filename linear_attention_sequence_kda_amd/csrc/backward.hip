// Backward pass of the chunkwise KDA prefill (gfx950, fp32 arithmetic throughout).
//
// The pages fix the forward only (xhh.club tag page 结构: the recurrent form, and the
// chunkwise form used for training and prefill).  The gradient here is reverse-mode
// differentiation of that chunkwise form, per 64-token chunk with
//   gt = min(0, max(-5, g)),  G_t = sum_{u <= t} gt_u (per key channel),  Gam = G_63,
//   KK[t][j] = sum_i k_ti k_ji e^{G_ti - G_ji}  (j < t),  P[t][j] = same with q_t (j <= t),
//   M = (I + diag(beta) KK)^-1,  T = M diag(beta),
//   W = T (k e^G),  U~ = T v,  Q~ = q e^G,  K_dec = k e^{Gam - G},  D = e^{Gam},
//   U = U~ - W S,  S_next = D S + K_dec^T U,  O = Q~ S + P U.
// Given dO (gradient of the raw outputs) and dS_T, the chain rule gives, per chunk,
//   dU = P^T dO + K_dec dS_next,   dS = D dS_next + Q~^T dO - W^T dU      (reverse sweep)
//   dP = Lower(dO U^T), dQ~ = dO S^T, dW = -dU S^T, dK_dec = U dS_next^T,
//   dD = rowsum(dS_next * S), dT = dU v^T + dW (k e^G)^T, dv = T^T dU, d(k e^G) = T^T dW,
//   dbeta_j = sum_t dT[t][j] M[t][j] + sum_i dA[j][i] KK[j][i],
//   dA = -M^T (dT diag(beta)) M^T (strictly lower),  dKK = diag(beta) dA,
// and the pairwise terms of dKK and dP into dk, dq and dG, the elementwise terms of
// Q~, k e^G and K_dec, then dg_u = [-5 <= g_u <= 0] (sum_{t >= u} dG_t + dGam).
//
// Pairwise decays e^{G_t - G_j} (j <= t) are factored through the first token R of a
// 16-token block: e^{G_t - G_R} e^{G_R - G_j}, with R the start of j's block or of t's
// block.  Each factor stays inside fp32 range because every step's log-decay is at least
// -5 (15 steps within a block: at most e^75), the bound the forward's 16-token diagonal
// tiles rely on; a factor that underflows multiplies a term below fp32 resolution.
//
// Four kernels:
//   bwd_prep    one workgroup per chunk: G, K_dec, Q~, P^T, KK, M, W, U~, D -> record
//   bwd_fwd     per (sequence, head, 32 value columns): states entering every chunk, U
//   bwd_rev     same split, reverse order: dS after every chunk, dU, and dS0
//   bwd_grad    one workgroup per chunk: dq, dk, dv, dg, dbeta of the chunk's tokens
#include <type_traits>

#include "internal.h"
#include "kda_device.h"

namespace kda {
namespace {

constexpr int D = 128;        // d_k = d_v
constexpr int C = 64;         // tokens per chunk
constexpr int LD = D + 4;     // LDS row stride of [C][D] tiles
constexpr int LS = C + 4;     // LDS row stride of [C][C] tiles

// per-chunk record, floats.  P is kept transposed (the chunk kernel's MFMA output
// fragments hold four consecutive rows of it, the gradient sweep reads its columns).
constexpr int R_G = 0;                // [C][D] G in log2 units
constexpr int R_KD = R_G + C * D;     // [C][D] K_dec
constexpr int R_W = R_KD + C * D;     // [C][D] W
constexpr int R_UT = R_W + C * D;     // [C][D] U~ (column-blocked), replaced by U = U~ - W S
                                      // in the state sweep
constexpr int R_QT = R_UT + C * D;    // [C][D] Q~
constexpr int R_PT = R_QT + C * D;    // [C][C] P^T (zero below the diagonal)
constexpr int R_M = R_PT + C * C;     // [C][C] M (zero above the diagonal)
constexpr int R_KK = R_M + C * C;     // [C][C] KK (zero on and above the diagonal)
constexpr int R_D = R_KK + C * C;     // [D] e^{Gam}
constexpr int REC = R_D + D;

struct BwdArgs {
  const void *q, *k, *v;
  const float *g, *beta, *S0, *dO, *dSf;
  float *dq, *dk, *dv, *dg, *dbeta, *dS0;
  float *rec, *sin, *dsa, *du;
  int B, T, H, NC;
};

__device__ __forceinline__ f32x4 mfma4(float a, float b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}
// One 16-long contraction block: lane group q supplies contraction index 4q+e to the
// e-th MFMA (the same permutation on both operands).
__device__ __forceinline__ f32x4 mma16(f32x4 c, float4 a, float4 b) {
  c = mfma4(a.x, b.x, c);
  c = mfma4(a.y, b.y, c);
  c = mfma4(a.z, b.z, c);
  return mfma4(a.w, b.w, c);
}
__device__ __forceinline__ float4 ld4(const float *p) { return *reinterpret_cast<const float4 *>(p); }
// p[0], p[ld], p[2 ld], p[3 ld]
__device__ __forceinline__ float4 col4(const float *p, int ld) {
  return make_float4(p[0], p[ld], p[2 * ld], p[3 * ld]);
}
__device__ __forceinline__ float4 mul4(float4 a, float4 b) {
  return make_float4(a.x * b.x, a.y * b.y, a.z * b.z, a.w * b.w);
}
__device__ __forceinline__ f32x4 zero4() { return f32x4{0.f, 0.f, 0.f, 0.f}; }

// Column-blocked layout of the per-chunk states, their gradients, U and dU: element
// (row, col) of a [rows][D] matrix sits at (col / 16) [rows] [16] + (row, col % 16), so a
// sweep workgroup's 16 columns are one contiguous block (whole-line stores) and a
// 16-byte piece of a row stays contiguous for the per-chunk kernel.
__device__ __forceinline__ int cblk(int row, int col, int rows) {
  return (col >> 4) * rows * 16 + row * 16 + (col & 15);
}

// element offset of token t of a [B,T,H,D] array, head h
__device__ __forceinline__ size_t tok_off(const BwdArgs &a, int b, int h, int t) {
  return (static_cast<size_t>(b) * a.T + t) * a.H * D + static_cast<size_t>(h) * D;
}

// Barrier that orders LDS accesses only: it waits for this wave's LDS operations, not for
// its global loads in flight (the prefetches of the next phase) nor its global stores.
// The kernels below never read global memory they write, so LDS is all a barrier orders.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0); vmcnt and expcnt not waited for
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// ---------------------------------------------------------------------------
// bwd_prep: per-chunk quantities of the forward (one workgroup of 512 per chunk)
// ---------------------------------------------------------------------------
template <bool BF16>
__global__ __launch_bounds__(512, 1) void bwd_prep(BwdArgs a) {
  __shared__ __align__(16) float sG[C * LD];    // G (log2), then beta k e^G
  __shared__ __align__(16) float sX[C * LD];    // KR = k e^{G - G_R}, then QR, then beta v
  __shared__ __align__(16) float sY[C * LD];    // KL = k e^{G_R - G}
  __shared__ __align__(16) float sA[C * LS];    // beta_t KK[t][j]
  __shared__ __align__(16) float sM[C * LS];    // M
  __shared__ __align__(16) float sDel[6 * D];   // e^{G_R(a) - G_R(b)}, a > b
  __shared__ __align__(16) float sGa[4 * D];    // G at the four block starts
  __shared__ float sBeta[C];
  __shared__ float sZ[4][16 * 17];

  const int tid = threadIdx.x, lane = tid & 63, r = lane & 15, q = lane >> 4;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int ch = blockIdx.x, bh = ch / a.NC, c = ch % a.NC, b = bh / a.H, h = bh % a.H;
  const int t0 = c * C, Tc = min(C, a.T - t0);
  float *rec = a.rec + static_cast<size_t>(ch) * REC;

  // Every input of the chunk is loaded here, so that the k, q and v loads overlap the
  // decay scan; k, q and v stay in their input format until used.
  using Raw4 = typename std::conditional<BF16, uint2, float4>::type;
  Raw4 kraw[4], qraw[4], vraw[4];
  auto widen = [](const Raw4 &x) __attribute__((always_inline)) {
    if constexpr (BF16) {
      return make_float4(__uint_as_float(x.x << 16), __uint_as_float(x.x & 0xffff0000u),
                         __uint_as_float(x.y << 16), __uint_as_float(x.y & 0xffff0000u));
    } else {
      return x;
    }
  };
  // decays (log2 units) and beta; tokens past the sequence end are zero.  beta and g
  // are loaded first: the in-order wait counter then lets their first use proceed while
  // k, q and v are still in flight.
  const float beta_t = tid < Tc ? a.beta[(static_cast<size_t>(b) * a.T + t0 + tid) * a.H + h] : 0.f;
  {
    float4 gv[4];
#pragma unroll
    for (int x = 0; x < 4; ++x) {
      const int e = tid + 512 * x, t = e >> 5, i = (e & 31) * 4;
      gv[x] = ld4(a.g + tok_off(a, b, h, t0 + min(t, Tc - 1)) + i);
    }
    using E = typename std::conditional<BF16, uint16_t, float>::type;
#pragma unroll
    for (int x = 0; x < 4; ++x) {
      const int e = tid + 512 * x, t = e >> 5, i = (e & 31) * 4;
      const size_t o = tok_off(a, b, h, t0 + min(t, Tc - 1)) + i;
      kraw[x] = *reinterpret_cast<const Raw4 *>(static_cast<const E *>(a.k) + o);
      qraw[x] = *reinterpret_cast<const Raw4 *>(static_cast<const E *>(a.q) + o);
      vraw[x] = *reinterpret_cast<const Raw4 *>(static_cast<const E *>(a.v) + o);
    }
#pragma unroll
    for (int x = 0; x < 4; ++x) {
      const int e = tid + 512 * x, t = e >> 5, i = (e & 31) * 4;
      if (t >= Tc) gv[x] = make_float4(0.f, 0.f, 0.f, 0.f);
      float *d = sG + t * LD + i;
      d[0] = log2_decay(gv[x].x); d[1] = log2_decay(gv[x].y); d[2] = log2_decay(gv[x].z); d[3] = log2_decay(gv[x].w);
    }
  }
  for (int e = tid; e < C * LS; e += 512) { sA[e] = 0.f; sM[e] = 0.f; }
  if (tid < C) sBeta[tid] = beta_t;
  lds_barrier();
  {   // inclusive scan over the chunk: four 16-token parts per channel, then offsets
    float *sTot = &sZ[0][0];   // part totals [4][D] (sZ is free until the solve)
    const int i = tid & (D - 1), part = tid >> 7;
    float s = 0.f;
#pragma unroll
    for (int t = 16 * part; t < 16 * part + 16; ++t) { s += sG[t * LD + i]; sG[t * LD + i] = s; }
    sTot[part * D + i] = s;
    lds_barrier();
    float off = 0.f;
    for (int p = 0; p < part; ++p) off += sTot[p * D + i];
    if (part > 0) {
#pragma unroll
      for (int t = 16 * part; t < 16 * part + 16; ++t) sG[t * LD + i] += off;
    }
  }
  lds_barrier();
  if (tid < D) {
    const int i = tid;
    for (int blk = 0; blk < 4; ++blk) sGa[blk * D + i] = sG[16 * blk * LD + i];
    int p = 0;
    for (int x = 1; x < 4; ++x)
      for (int y = 0; y < x; ++y, ++p) sDel[p * D + i] = exp2_fast(sG[16 * x * LD + i] - sG[16 * y * LD + i]);
    rec[R_D + i] = exp2_fast(sG[(C - 1) * LD + i]);
  }
  lds_barrier();

  // pass 1: KR, KL, Q~, K_dec, G; k and q stay in registers for pass 2
  float4 kv[4], qv[4];
#pragma unroll
  for (int x = 0; x < 4; ++x) {
    kv[x] = widen(kraw[x]);
    qv[x] = widen(qraw[x]);
  }
#pragma unroll
  for (int x = 0; x < 4; ++x) {
    const int e = tid + 512 * x, t = e >> 5, i = (e & 31) * 4;
    if (t >= Tc) { kv[x] = make_float4(0.f, 0.f, 0.f, 0.f); qv[x] = kv[x]; }
    const float kk[4] = {kv[x].x, kv[x].y, kv[x].z, kv[x].w}, qq[4] = {qv[x].x, qv[x].y, qv[x].z, qv[x].w};
    float kr[4], kl[4], qt[4], kd[4], gg[4];
#pragma unroll
    for (int y = 0; y < 4; ++y) {
      const float G = sG[t * LD + i + y], Ga = sGa[(t >> 4) * D + i + y], Gm = sG[(C - 1) * LD + i + y];
      kr[y] = kk[y] * exp2_fast(G - Ga);
      kl[y] = kk[y] * exp2_fast(Ga - G);
      qt[y] = qq[y] * exp2_fast(G);
      kd[y] = kk[y] * exp2_fast(Gm - G);
      gg[y] = G;
    }
    *reinterpret_cast<float4 *>(sX + t * LD + i) = make_float4(kr[0], kr[1], kr[2], kr[3]);
    *reinterpret_cast<float4 *>(sY + t * LD + i) = make_float4(kl[0], kl[1], kl[2], kl[3]);
    *reinterpret_cast<float4 *>(rec + R_QT + t * D + i) = make_float4(qt[0], qt[1], qt[2], qt[3]);
    *reinterpret_cast<float4 *>(rec + R_KD + t * D + i) = make_float4(kd[0], kd[1], kd[2], kd[3]);
    *reinterpret_cast<float4 *>(rec + R_G + t * D + i) = make_float4(gg[0], gg[1], gg[2], gg[3]);
  }
  // zero tiles above the block diagonal of KK and P
  for (int e = tid; e < C * C; e += 512) {
    const int t = e >> 6, j = e & 63;
    if ((j >> 4) > (t >> 4)) { rec[R_KK + t * C + j] = 0.f; rec[R_PT + j * C + t] = 0.f; }
  }
  lds_barrier();

  // KK and P: tile (ta, tb), ta >= tb: rows t of block ta, columns j of block tb,
  //   sum_i (X_ti e^{G_R(ta) - G_R(tb)}) KL_ji  with X = KR (KK) or QR (P)
  auto pair_tiles = [&](bool is_p) {
    for (int tt = w; tt < 10; tt += 8) {   // tiles in the order (0,0) (1,0) (1,1) (2,0) ...
      const int ta = tt < 1 ? 0 : tt < 3 ? 1 : tt < 6 ? 2 : 3, tb = tt - ta * (ta + 1) / 2;
      const float *ar = sX + (16 * ta + r) * LD + 4 * q;
      const float *br = sY + (16 * tb + r) * LD + 4 * q;
      const float *dl = sDel + (ta * (ta - 1) / 2 + tb) * D + 4 * q;
      f32x4 acc = zero4();
#pragma unroll 4
      for (int k0 = 0; k0 < D; k0 += 16) {
        float4 av = ld4(ar + k0);
        if (ta != tb) av = mul4(av, ld4(dl + k0));
        acc = mma16(acc, av, ld4(br + k0));
      }
      if (is_p) {   // P^T[j][t], the lane's four t contiguous
        const int j = 16 * tb + r, t4 = 16 * ta + 4 * q;
        *reinterpret_cast<float4 *>(rec + R_PT + j * C + t4) =
            make_float4(j <= t4 ? acc[0] : 0.f, j <= t4 + 1 ? acc[1] : 0.f, j <= t4 + 2 ? acc[2] : 0.f,
                        j <= t4 + 3 ? acc[3] : 0.f);
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int t = 16 * ta + 4 * q + e, j = 16 * tb + r;
        if (!is_p) {
          const float v = j < t ? acc[e] : 0.f;
          rec[R_KK + t * C + j] = v;
          sA[t * LS + j] = sBeta[t] * v;
        }
      }
    }
  };
  pair_tiles(false);
  lds_barrier();

  // pass 2: QR over KR; beta k e^G over G (each element by the thread that reads it)
#pragma unroll
  for (int x = 0; x < 4; ++x) {
    const int e = tid + 512 * x, t = e >> 5, i = (e & 31) * 4;
    const float kk[4] = {kv[x].x, kv[x].y, kv[x].z, kv[x].w}, qq[4] = {qv[x].x, qv[x].y, qv[x].z, qv[x].w};
    const float bt = sBeta[t];
#pragma unroll
    for (int y = 0; y < 4; ++y) {
      const float G = sG[t * LD + i + y], Ga = sGa[(t >> 4) * D + i + y];
      sX[t * LD + i + y] = qq[y] * exp2_fast(G - Ga);
      sG[t * LD + i + y] = bt * kk[y] * exp2_fast(G);
    }
  }
  lds_barrier();
  pair_tiles(true);

  // M = (I + A)^-1, A = diag(beta) KK strictly lower: 16x16 diagonal blocks by
  // forward substitution (one wave per block, lane = column), then the blocks below
  //   M_xy = -M_xx sum_{y <= z < x} A_xz M_zy
  if (w < 4) {
    const int blk = w, cc = lane & 15;
    float x[16];
#pragma unroll
    for (int t = 0; t < 16; ++t) {
      float s = t == cc ? 1.f : 0.f;
#pragma unroll
      for (int j = 0; j < t; ++j) s -= sA[(16 * blk + t) * LS + 16 * blk + j] * x[j];
      x[t] = s;
    }
    if (lane < 16)
#pragma unroll
      for (int t = 0; t < 16; ++t) sM[(16 * blk + t) * LS + 16 * blk + cc] = x[t];
  }
  lds_barrier();
  for (int xb = 1; xb < 4; ++xb) {
    if (w < xb) {
      const int yb = w;
      f32x4 z = zero4();
      for (int zb = yb; zb < xb; ++zb) {
        const float4 av = ld4(sA + (16 * xb + r) * LS + 16 * zb + 4 * q);
        const float4 bv = col4(sM + (16 * zb + 4 * q) * LS + 16 * yb + r, LS);
        z = mma16(z, av, bv);
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) sZ[w][(4 * q + e) * 17 + r] = z[e];
      const float4 av = ld4(sM + (16 * xb + r) * LS + 16 * xb + 4 * q);
      const float4 bv = col4(&sZ[w][(4 * q) * 17 + r], 17);
      const f32x4 y = mma16(zero4(), av, bv);
#pragma unroll
      for (int e = 0; e < 4; ++e) sM[(16 * xb + 4 * q + e) * LS + 16 * yb + r] = -y[e];
    }
    lds_barrier();
  }
  for (int e = tid; e < C * C; e += 512) rec[R_M + e] = sM[(e >> 6) * LS + (e & 63)];

  // beta v over QR
  {
    float4 vv[4];
#pragma unroll
    for (int x = 0; x < 4; ++x) vv[x] = widen(vraw[x]);
#pragma unroll
    for (int x = 0; x < 4; ++x) {
      const int e = tid + 512 * x, t = e >> 5, i = (e & 31) * 4;
      const float bt = sBeta[t];   // zero past the sequence end
      *reinterpret_cast<float4 *>(sX + t * LD + i) = make_float4(bt * vv[x].x, bt * vv[x].y, bt * vv[x].z, bt * vv[x].w);
    }
  }
  lds_barrier();

  // W = M (beta k e^G), U~ = M (beta v): wave w rows 16(w&3).., column tiles (w>>2)+2i
  const int tm = w & 3, tn0 = w >> 2;
  f32x4 accW[4], accU[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) { accW[i] = zero4(); accU[i] = zero4(); }
  for (int k0 = 0; k0 <= 16 * tm; k0 += 16) {    // M[t][j] = 0 for j > t
    const float4 av = ld4(sM + (16 * tm + r) * LS + k0 + 4 * q);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int n = 16 * (tn0 + 2 * i) + r;
      accW[i] = mma16(accW[i], av, col4(sG + (k0 + 4 * q) * LD + n, LD));
      accU[i] = mma16(accU[i], av, col4(sX + (k0 + 4 * q) * LD + n, LD));
    }
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int n = 16 * (tn0 + 2 * i) + r;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int t = 16 * tm + 4 * q + e;
      rec[R_W + t * D + n] = accW[i][e];
      rec[R_UT + cblk(t, n, C)] = accU[i][e];
    }
  }
}

// (sequence, head) and column unit of a sweep workgroup (NU units of 128/NU columns per
// head).  The units of a (sequence, head) share one XCD (workgroups are dealt to XCDs
// round robin), so the chunk records they all read are fetched into one L2.
template <int NU>
__device__ __forceinline__ bool sweep_unit(int BH, int &bh, int &cb) {
  const int x = blockIdx.x, xcd = x & 7, slot = x >> 3;
  bh = (slot / NU) * 8 + xcd;
  cb = slot % NU;
  return bh < BH;
}

// ---------------------------------------------------------------------------
// bwd_fwd: states entering every chunk, for 16 CB value columns of one (sequence, head)
// ---------------------------------------------------------------------------
// Eight waves per unit.  Each chunk step has two phases: U = U~ - W S (wave w: rows
// 16(w&3).. of U over half of the contraction, (w>>2), for all CB column blocks), then
// S = D S + K_dec^T U (wave w: state rows 16w..).  The record fragments of a phase are
// loaded one step ahead, so their latency overlaps the other phase, and each fragment
// serves the unit's CB column blocks (the record is read once per 16 CB columns).  S and
// the two partial sums of U are kept in LDS transposed ([column][row], double buffered),
// so that an MFMA operand is one 16-byte read and a step needs two barriers; state and U
// rows go to global memory as 16-byte stores from those copies.
constexpr int LT = D + 4;   // row stride of a transposed [16][D] block
constexpr int LU = C + 4;   // row stride of a transposed [16][C] block

template <int CB> struct FwdA { float4 w[4]; float ut[CB][4]; };
struct FwdB { float4 kd[4]; float4 d; };

template <int CB>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(4 / CB))) void bwd_fwd(BwdArgs a) {
  constexpr int NU = 8 / CB, NCOL = 16 * CB;
  __shared__ __align__(16) float sSt[2][NCOL * LT];
  __shared__ __align__(16) float sUt[2][2][NCOL * LU];
  int bh, cb;
  if (!sweep_unit<NU>(a.B * a.H, bh, cb)) return;
  const int tid = threadIdx.x, lane = tid & 63, r = lane & 15, q = lane >> 4;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int ta = w & 3, kh = w >> 2;
  const int c0 = NCOL * cb;
  float *recs = a.rec + static_cast<size_t>(bh) * a.NC * REC;
  auto loadA = [&](FwdA<CB> &x, int c) {
    const float *rec = recs + static_cast<size_t>(c) * REC;
#pragma unroll
    for (int j = 0; j < 4; ++j) x.w[j] = ld4(rec + R_W + (16 * ta + r) * D + 16 * (4 * kh + j) + 4 * q);
#pragma unroll
    for (int j = 0; j < CB; ++j)
#pragma unroll
      for (int e = 0; e < 4; ++e) x.ut[j][e] = rec[R_UT + cblk(16 * ta + 4 * q + e, c0 + 16 * j + r, C)];
  };
  auto loadB = [&](FwdB &x, int c) {
    const float *rec = recs + static_cast<size_t>(c) * REC;
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) x.kd[kb] = col4(rec + R_KD + (16 * kb + 4 * q) * D + 16 * w + r, D);
    x.d = ld4(rec + R_D + 16 * w + 4 * q);
  };
  // state rows 16w + 4q + e, columns c0 + 16j + r
  f32x4 S[CB];
#pragma unroll
  for (int j = 0; j < CB; ++j) {
#pragma unroll
    for (int e = 0; e < 4; ++e)
      S[j][e] = a.S0 ? a.S0[(static_cast<size_t>(bh) * D + 16 * w + 4 * q + e) * D + c0 + 16 * j + r] : 0.f;
    *reinterpret_cast<float4 *>(&sSt[0][(16 * j + r) * LT + 16 * w + 4 * q]) = make_float4(S[j][0], S[j][1], S[j][2], S[j][3]);
  }
  FwdA<CB> A;
  FwdB Bf;
  loadA(A, 0);
  loadB(Bf, 0);
  __syncthreads();
  for (int c = 0; c < a.NC; ++c) {
    const int p = c & 1, cn = min(c + 1, a.NC - 1);   // the last step reloads its own chunk
    float *rec = recs + static_cast<size_t>(c) * REC;
    // partial U over this wave's half of the contraction (two chains per column block)
#pragma unroll
    for (int j = 0; j < CB; ++j) {
      const float *bs = &sSt[p][(16 * j + r) * LT + 64 * kh + 4 * q];
      f32x4 u0 = zero4(), u1 = zero4();
      u0 = mma16(u0, A.w[0], ld4(bs));
      u1 = mma16(u1, A.w[1], ld4(bs + 16));
      u0 = mma16(u0, A.w[2], ld4(bs + 32));
      u1 = mma16(u1, A.w[3], ld4(bs + 48));
      float u[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) u[e] = (kh == 0 ? A.ut[j][e] : 0.f) - (u0[e] + u1[e]);
      *reinterpret_cast<float4 *>(&sUt[p][kh][(16 * j + r) * LU + 16 * ta + 4 * q]) = make_float4(u[0], u[1], u[2], u[3]);
    }
    loadA(A, cn);
    lds_barrier();
    if (tid < 256 * CB) {   // U replaces U~ (its columns are this workgroup's alone)
      const int t = (tid >> 2) & (C - 1), c4 = 4 * (tid & 3) + 16 * (tid >> 8);
      const float *s0p = &sUt[p][0][c4 * LU + t], *s1p = &sUt[p][1][c4 * LU + t];
      *reinterpret_cast<float4 *>(rec + R_UT + cblk(t, c0 + c4, C)) =
          make_float4(s0p[0] + s1p[0], s0p[LU] + s1p[LU], s0p[2 * LU] + s1p[2 * LU], s0p[3 * LU] + s1p[3 * LU]);
    }
    // S = D S + K_dec^T U, rows 16w..
#pragma unroll
    for (int j = 0; j < CB; ++j) {
      const float *bu0 = &sUt[p][0][(16 * j + r) * LU + 4 * q], *bu1 = &sUt[p][1][(16 * j + r) * LU + 4 * q];
      f32x4 s0, s1 = zero4();
      s0[0] = Bf.d.x * S[j][0];
      s0[1] = Bf.d.y * S[j][1];
      s0[2] = Bf.d.z * S[j][2];
      s0[3] = Bf.d.w * S[j][3];
#pragma unroll
      for (int kb = 0; kb < 4; kb += 2) {
        const float4 x0 = ld4(bu0 + 16 * kb), y0 = ld4(bu1 + 16 * kb);
        const float4 x1 = ld4(bu0 + 16 * kb + 16), y1 = ld4(bu1 + 16 * kb + 16);
        s0 = mma16(s0, Bf.kd[kb], make_float4(x0.x + y0.x, x0.y + y0.y, x0.z + y0.z, x0.w + y0.w));
        s1 = mma16(s1, Bf.kd[kb + 1], make_float4(x1.x + y1.x, x1.y + y1.y, x1.z + y1.z, x1.w + y1.w));
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) S[j][e] = s0[e] + s1[e];
      *reinterpret_cast<float4 *>(&sSt[p ^ 1][(16 * j + r) * LT + 16 * w + 4 * q]) =
          make_float4(S[j][0], S[j][1], S[j][2], S[j][3]);
    }
    loadB(Bf, cn);
    {   // the state entering this chunk, rows of 16 columns from its LDS copy (unchanged
        // this step).  Issued after the prefetches: the wait counter completes in issue
        // order, so no wait for a prefetched fragment also waits for this store.
      float *sin = a.sin + (static_cast<size_t>(bh) * a.NC + c) * D * D;
#pragma unroll
      for (int x = 0; x < CB; ++x) {
        const int i = tid >> 2, c4 = 4 * (tid & 3) + 16 * x;
        const float *src = &sSt[p][c4 * LT + i];
        *reinterpret_cast<float4 *>(sin + cblk(i, c0 + c4, D)) = make_float4(src[0], src[LT], src[2 * LT], src[3 * LT]);
      }
    }
    lds_barrier();
  }
}

// ---------------------------------------------------------------------------
// bwd_rev: dS after every chunk (reverse order), dU, and dS0
// ---------------------------------------------------------------------------
// Eight waves per unit, as the state sweep.  Phases: dU = P^T dO + K_dec dS (wave w: rows
// 16(w&3).. of dU; the twelve 16-long blocks of the contraction split six and six by
// (w>>2)), then dS = D dS + Q~^T dO - W^T dU (wave w: rows 16w..).  Record fragments and
// the dO block of the next (earlier) chunk are loaded one step ahead (D with the phase-A
// set, so that its early use does not wait for the phase-B set); dS, dO and the two
// partial sums of dU are kept in LDS transposed and double buffered.
struct RevA { float4 f[6]; float4 d; };
struct RevB { float4 qt[4]; float4 wt[4]; };

template <int CB>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(4 / CB))) void bwd_rev(BwdArgs a) {
  constexpr int NU = 8 / CB, NCOL = 16 * CB;
  __shared__ __align__(16) float sdSt[2][NCOL * LT];
  __shared__ __align__(16) float sdOt[2][NCOL * LU];
  __shared__ __align__(16) float sdUt[2][2][NCOL * LU];
  int bh, cb;
  if (!sweep_unit<NU>(a.B * a.H, bh, cb)) return;
  const int tid = threadIdx.x, lane = tid & 63, r = lane & 15, q = lane >> 4;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int ta = w & 3, kh = w >> 2;
  const int c0 = NCOL * cb, b = bh / a.H, h = bh % a.H;
  const float *recs = a.rec + static_cast<size_t>(bh) * a.NC * REC;
  // contraction blocks of dU: kh = 0 takes P^T blocks 0..3 (over t) and K_dec blocks 0..1
  // (over i); kh = 1 takes K_dec blocks 2..7
  auto loadA = [&](RevA &x, int c) {
    const float *rec = recs + static_cast<size_t>(c) * REC;
    if (kh == 0) {
#pragma unroll
      for (int j = 0; j < 4; ++j) x.f[j] = ld4(rec + R_PT + (16 * ta + r) * C + 16 * j + 4 * q);
#pragma unroll
      for (int j = 0; j < 2; ++j) x.f[4 + j] = ld4(rec + R_KD + (16 * ta + r) * D + 16 * j + 4 * q);
    } else {
#pragma unroll
      for (int j = 0; j < 6; ++j) x.f[j] = ld4(rec + R_KD + (16 * ta + r) * D + 16 * (j + 2) + 4 * q);
    }
    x.d = ld4(rec + R_D + 16 * w + 4 * q);
  };
  auto loadB = [&](RevB &x, int c) {
    const float *rec = recs + static_cast<size_t>(c) * REC;
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      x.qt[kb] = col4(rec + R_QT + (16 * kb + 4 * q) * D + 16 * w + r, D);
      x.wt[kb] = col4(rec + R_W + (16 * kb + 4 * q) * D + 16 * w + r, D);
    }
  };
  // one float4 of a chunk's dO block [64][16 CB] for each of the first 256 CB threads
  // (rows past the end read 0), stored transposed; the other threads (CB = 1) load a
  // duplicate inside the unit's columns and store nothing
  const int ot = (tid >> 2) & (C - 1), ox = 4 * (tid & 3) + 16 * ((tid >> 8) & (CB - 1));
  auto loadO = [&](int c) {
    const int t = c * C + ot;
    float4 v = ld4(a.dO + tok_off(a, b, h, min(t, a.T - 1)) + c0 + ox);
    if (t >= a.T) v = make_float4(0.f, 0.f, 0.f, 0.f);
    return v;
  };
  auto storeO = [&](float *dst, float4 v) {
    if (tid < 256 * CB) {
      dst[(ox + 0) * LU + ot] = v.x;
      dst[(ox + 1) * LU + ot] = v.y;
      dst[(ox + 2) * LU + ot] = v.z;
      dst[(ox + 3) * LU + ot] = v.w;
    }
  };
  f32x4 dS[CB];
#pragma unroll
  for (int j = 0; j < CB; ++j) {
#pragma unroll
    for (int e = 0; e < 4; ++e)
      dS[j][e] = a.dSf ? a.dSf[(static_cast<size_t>(bh) * D + 16 * w + 4 * q + e) * D + c0 + 16 * j + r] : 0.f;
    *reinterpret_cast<float4 *>(&sdSt[0][(16 * j + r) * LT + 16 * w + 4 * q]) =
        make_float4(dS[j][0], dS[j][1], dS[j][2], dS[j][3]);
  }
  if (a.NC > 0) {
    RevA A;
    RevB Bf;
    storeO(sdOt[0], loadO(a.NC - 1));
    loadA(A, a.NC - 1);
    loadB(Bf, a.NC - 1);
    __syncthreads();
    for (int c = a.NC - 1, p = 0; c >= 0; --c, p ^= 1) {
      const int cn = max(c - 1, 0);   // the last step reloads its own chunk
      const float4 ov = loadO(cn);
      // partial dU over this wave's six contraction blocks
#pragma unroll
      for (int j = 0; j < CB; ++j) {
        f32x4 u0 = zero4(), u1 = zero4();
        if (kh == 0) {
          const float *bo = &sdOt[p][(16 * j + r) * LU + 4 * q], *bs = &sdSt[p][(16 * j + r) * LT + 4 * q];
          u0 = mma16(u0, A.f[0], ld4(bo));
          u1 = mma16(u1, A.f[1], ld4(bo + 16));
          u0 = mma16(u0, A.f[2], ld4(bo + 32));
          u1 = mma16(u1, A.f[3], ld4(bo + 48));
          u0 = mma16(u0, A.f[4], ld4(bs));
          u1 = mma16(u1, A.f[5], ld4(bs + 16));
        } else {
          const float *bs = &sdSt[p][(16 * j + r) * LT + 32 + 4 * q];
#pragma unroll
          for (int x = 0; x < 6; x += 2) {
            u0 = mma16(u0, A.f[x], ld4(bs + 16 * x));
            u1 = mma16(u1, A.f[x + 1], ld4(bs + 16 * x + 16));
          }
        }
        *reinterpret_cast<float4 *>(&sdUt[p][kh][(16 * j + r) * LU + 16 * ta + 4 * q]) =
            make_float4(u0[0] + u1[0], u0[1] + u1[1], u0[2] + u1[2], u0[3] + u1[3]);
      }
      const float4 dcur = A.d;
      loadA(A, cn);
      lds_barrier();
      if (tid < 256 * CB) {   // dU rows from the LDS partial sums
        float *du = a.du + (static_cast<size_t>(bh) * a.NC + c) * C * D;
        const int t = (tid >> 2) & (C - 1), c4 = 4 * (tid & 3) + 16 * (tid >> 8);
        const float *s0p = &sdUt[p][0][c4 * LU + t], *s1p = &sdUt[p][1][c4 * LU + t];
        *reinterpret_cast<float4 *>(du + cblk(t, c0 + c4, C)) =
            make_float4(s0p[0] + s1p[0], s0p[LU] + s1p[LU], s0p[2 * LU] + s1p[2 * LU], s0p[3 * LU] + s1p[3 * LU]);
      }
      // dS = D dS + Q~^T dO - W^T dU, rows 16w..
#pragma unroll
      for (int j = 0; j < CB; ++j) {
        const float *bo = &sdOt[p][(16 * j + r) * LU + 4 * q];
        const float *bu0 = &sdUt[p][0][(16 * j + r) * LU + 4 * q], *bu1 = &sdUt[p][1][(16 * j + r) * LU + 4 * q];
        f32x4 s0, s1 = zero4();
        s0[0] = dcur.x * dS[j][0];
        s0[1] = dcur.y * dS[j][1];
        s0[2] = dcur.z * dS[j][2];
        s0[3] = dcur.w * dS[j][3];
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) {
          const float4 x = ld4(bu0 + 16 * kb), y = ld4(bu1 + 16 * kb);
          s0 = mma16(s0, Bf.qt[kb], ld4(bo + 16 * kb));
          s1 = mma16(s1, Bf.wt[kb], make_float4(-(x.x + y.x), -(x.y + y.y), -(x.z + y.z), -(x.w + y.w)));
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) dS[j][e] = s0[e] + s1[e];
        *reinterpret_cast<float4 *>(&sdSt[p ^ 1][(16 * j + r) * LT + 16 * w + 4 * q]) =
            make_float4(dS[j][0], dS[j][1], dS[j][2], dS[j][3]);
      }
      storeO(sdOt[p ^ 1], ov);
      loadB(Bf, cn);
      {   // dS after this chunk (unchanged this step), after the prefetches as in the
          // state sweep
        float *dsa = a.dsa + (static_cast<size_t>(bh) * a.NC + c) * D * D;
#pragma unroll
        for (int x = 0; x < CB; ++x) {
          const int i = tid >> 2, c4 = 4 * (tid & 3) + 16 * x;
          const float *src = &sdSt[p][c4 * LT + i];
          *reinterpret_cast<float4 *>(dsa + cblk(i, c0 + c4, D)) = make_float4(src[0], src[LT], src[2 * LT], src[3 * LT]);
        }
      }
      lds_barrier();
    }
  }
  if (a.dS0)
#pragma unroll
    for (int j = 0; j < CB; ++j)
#pragma unroll
      for (int e = 0; e < 4; ++e)
        a.dS0[(static_cast<size_t>(bh) * D + 16 * w + 4 * q + e) * D + c0 + 16 * j + r] = dS[j][e];
}

// ---------------------------------------------------------------------------
// bwd_grad: gradients of one chunk's tokens (one workgroup of 512 per chunk)
// ---------------------------------------------------------------------------
// Every [C][D] product below uses one tile map: wave w owns rows 16(w&3)+4q+e and the
// columns 16((w>>2)+2i)+r, i < 4, so the gradient accumulators dq, dk, dG stay in
// registers across all of them.  [C][C] products use columns 16((w>>2)+2i)+r, i < 2.
template <bool BF16>
__global__ __launch_bounds__(512, 1) void bwd_grad(BwdArgs a) {
  __shared__ __align__(16) float s1[C * LD];    // U, then k e^G, then dM M^T, then KL; then dG
  __shared__ __align__(16) float s2[C * LD];    // dU, then KR; then dK_dec * K_dec
  __shared__ __align__(16) float s3[C * LD];    // dO, then dW, then QR
  __shared__ __align__(16) float sP[C * LS];    // dP; then partial sums of the dg scan
  __shared__ __align__(16) float sT[C * LS];    // dT, then dT diag(beta), then dKK
  __shared__ __align__(16) float sM[C * LS];    // M
  __shared__ __align__(16) float sGa[4 * D];    // G at the block starts
  __shared__ float sBeta[C], sdD[D], sB1[C], sB2[2][C];

  const int tid = threadIdx.x, lane = tid & 63, r = lane & 15, q = lane >> 4;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int tm = w & 3, tn0 = w >> 2;
  const int ch = blockIdx.x, bh = ch / a.NC, c = ch % a.NC, b = bh / a.H, h = bh % a.H;
  const int t0 = c * C, Tc = min(C, a.T - t0);
  const float *rec = a.rec + static_cast<size_t>(ch) * REC;
  const float *S = a.sin + static_cast<size_t>(ch) * D * D;
  const float *dSn = a.dsa + static_cast<size_t>(ch) * D * D;

  auto row = [&](int e) { return 16 * tm + 4 * q + e; };
  auto col = [&](int i) { return 16 * (tn0 + 2 * i) + r; };

  // stage dO, U and dU (both written by the sweeps), M, beta, block-start G; every
  // global load of the staging is issued before the first LDS store
  const float *Ug = rec + R_UT;   // U~ replaced by U in the state sweep
  const float *dUg = a.du + static_cast<size_t>(ch) * C * D;
  const float bt = a.beta[(static_cast<size_t>(b) * a.T + t0 + min(tid & 63, Tc - 1)) * a.H + h];
  const float ga = rec[R_G + 16 * (tid >> 7) * D + (tid & 127)];
  float4 vo[4], vu[4], vd[4], vm[2];
#pragma unroll
  for (int x = 0; x < 4; ++x) {
    const int e = tid + 512 * x, t = e >> 5, i = (e & 31) * 4;
    vo[x] = ld4(a.dO + tok_off(a, b, h, t0 + min(t, Tc - 1)) + i);
    if (t >= Tc) vo[x] = make_float4(0.f, 0.f, 0.f, 0.f);
    vu[x] = ld4(Ug + 4 * e);    // column-blocked: consecutive threads, consecutive bytes
    vd[x] = ld4(dUg + 4 * e);
  }
#pragma unroll
  for (int x = 0; x < 2; ++x) vm[x] = ld4(rec + R_M + 4 * (tid + 512 * x));
  // per-lane G, k, q at the lane's 16 elements of the tile map, and Gam of its columns
  f32x4 Gr[4], kr[4], qr[4], DQ[4], DK[4], DG[4], KT[4];
  float Gam[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    Gam[i] = rec[R_G + (C - 1) * D + col(i)];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int t = row(e);
      Gr[i][e] = rec[R_G + t * D + col(i)];
      const size_t o = tok_off(a, b, h, t0 + min(t, Tc - 1)) + col(i);
      kr[i][e] = load1<BF16>(a.k, o);
      qr[i][e] = load1<BF16>(a.q, o);
    }
    DQ[i] = DK[i] = DG[i] = KT[i] = zero4();
  }
#pragma unroll
  for (int x = 0; x < 4; ++x) {
    const int e = tid + 512 * x, t = e >> 5, i = (e & 31) * 4;
    *reinterpret_cast<float4 *>(s3 + t * LD + i) = vo[x];
    const int tb = (e >> 2) & (C - 1), ib = 16 * (e >> 8) + 4 * (e & 3);   // element 4e, blocked
    *reinterpret_cast<float4 *>(s1 + tb * LD + ib) = vu[x];
    *reinterpret_cast<float4 *>(s2 + tb * LD + ib) = vd[x];
  }
#pragma unroll
  for (int x = 0; x < 2; ++x) {
    const int e = 4 * (tid + 512 * x);
    *reinterpret_cast<float4 *>(sM + (e >> 6) * LS + (e & 63)) = vm[x];
  }
  if (tid < C) sBeta[tid] = tid < Tc ? bt : 0.f;
  sGa[tid] = ga;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int e = 0; e < 4; ++e)
      if (row(e) >= Tc) { kr[i][e] = 0.f; qr[i][e] = 0.f; }
  lds_barrier();

  // dP = Lower(dO U^T)  -> sP
  {
    f32x4 p[2] = {zero4(), zero4()};
    const float *ar = s3 + (16 * tm + r) * LD + 4 * q;
#pragma unroll 2
    for (int k0 = 0; k0 < D; k0 += 16) {
      const float4 av = ld4(ar + k0);
#pragma unroll
      for (int i = 0; i < 2; ++i)
        if (tn0 + 2 * i <= tm) p[i] = mma16(p[i], av, ld4(s1 + col(i) * LD + k0 + 4 * q));
    }
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int e = 0; e < 4; ++e) sP[row(e) * LS + col(i)] = col(i) <= row(e) ? p[i][e] : 0.f;
  }

  // One pass over the chunk's state S and state gradient dS_next, both as transposed
  // right operands (B(k, n) = X[n][k], the lane's four rows of X loaded one 16-long block
  // ahead of their MFMAs):  dQ~ = dO S^T,  dW = -dU S^T,  dK_dec = U dS_next^T,  and
  // dD = rowsum(dS_next * S) from the same fragments (waves with tm = 0 cover all rows).
  f32x4 aq[4], aw[4], ak[4];
  float dd[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int i = 0; i < 4; ++i) { aq[i] = zero4(); aw[i] = zero4(); ak[i] = zero4(); }
  {
    auto load_bt = [&](float4 (&bt4)[4], const float *X, int kb) {
#pragma unroll
      for (int i = 0; i < 4; ++i) bt4[i] = ld4(X + kb * D * 16 + col(i) * 16 + 4 * q);   // (col(i), 16 kb + 4q)
    };
    float4 sc[4], sn[4], dc[4], dn[4];
    load_bt(sc, S, 0);
    load_bt(dc, dSn, 0);
    const float *ao = s3 + (16 * tm + r) * LD + 4 * q, *adu = s2 + (16 * tm + r) * LD + 4 * q;
    const float *au = s1 + (16 * tm + r) * LD + 4 * q;
#pragma unroll 2
    for (int kb = 0; kb < 8; ++kb) {
      load_bt(sn, S, min(kb + 1, 7));
      load_bt(dn, dSn, min(kb + 1, 7));
      const float4 xo = ld4(ao + 16 * kb), xdu = ld4(adu + 16 * kb), xu = ld4(au + 16 * kb);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        aq[i] = mma16(aq[i], xo, sc[i]);
        aw[i] = mma16(aw[i], xdu, sc[i]);
        ak[i] = mma16(ak[i], xu, dc[i]);
        dd[i] += sc[i].x * dc[i].x + sc[i].y * dc[i].y + sc[i].z * dc[i].z + sc[i].w * dc[i].w;
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) { sc[i] = sn[i]; dc[i] = dn[i]; }
    }
  }
  if (tm == 0) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float x = dd[i];
      x += __shfl_xor(x, 16);
      x += __shfl_xor(x, 32);
      if (q == 0) sdD[col(i)] = x;
    }
  }
  // dq += dQ~ e^G, dG += dQ~ * Q~;  dk += dK_dec e^{Gam - G}, keep dK_dec * K_dec
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float eg = exp2_fast(Gr[i][e]), f = exp2_fast(Gam[i] - Gr[i][e]);
      DQ[i][e] += aq[i][e] * eg;
      DG[i][e] += aq[i][e] * qr[i][e] * eg;
      DK[i][e] += ak[i][e] * f;
      KT[i][e] = ak[i][e] * kr[i][e] * f;
    }
  lds_barrier();   // dO (s3) and U (s1) no longer read

  // dW -> s3;  k e^G -> s1
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      s3[row(e) * LD + col(i)] = -aw[i][e];
      s1[row(e) * LD + col(i)] = kr[i][e] * exp2_fast(Gr[i][e]);
    }
  lds_barrier();

  // dT = dU v^T + dW (k e^G)^T -> sT (lower, with the diagonal); v rows one block ahead
  {
    f32x4 p[2] = {zero4(), zero4()};
    const float *ar = s2 + (16 * tm + r) * LD + 4 * q;
    const float *aw4p = s3 + (16 * tm + r) * LD + 4 * q;
    auto load_v = [&](float4 (&v4)[2], int kb) {
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int j = col(i);
        v4[i] = load4<BF16>(a.v, tok_off(a, b, h, t0 + min(j, Tc - 1)) + 16 * kb + 4 * q);
        if (j >= Tc) v4[i] = make_float4(0.f, 0.f, 0.f, 0.f);
      }
    };
    float4 vc[2], vn[2];
    load_v(vc, 0);
#pragma unroll
    for (int kb = 0; kb < 8; ++kb) {
      load_v(vn, min(kb + 1, 7));
      const float4 av = ld4(ar + 16 * kb), aw4 = ld4(aw4p + 16 * kb);
#pragma unroll
      for (int i = 0; i < 2; ++i)
        if (tn0 + 2 * i <= tm) {
          p[i] = mma16(p[i], av, vc[i]);
          p[i] = mma16(p[i], aw4, ld4(s1 + col(i) * LD + 16 * kb + 4 * q));
        }
#pragma unroll
      for (int i = 0; i < 2; ++i) vc[i] = vn[i];
    }
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int e = 0; e < 4; ++e) sT[row(e) * LS + col(i)] = col(i) <= row(e) ? p[i][e] : 0.f;
  }
  // dv = T^T dU (out);  d(k e^G) = T^T dW: dk += . e^G, dG += . k e^G
  {
    f32x4 av_acc[4], aw_acc[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) { av_acc[i] = zero4(); aw_acc[i] = zero4(); }
    for (int k0 = 16 * tm; k0 < C; k0 += 16) {   // M[t][j] = 0 for t < j
      const float4 am = col4(sM + (k0 + 4 * q) * LS + 16 * tm + r, LS);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        av_acc[i] = mma16(av_acc[i], am, col4(s2 + (k0 + 4 * q) * LD + col(i), LD));
        aw_acc[i] = mma16(aw_acc[i], am, col4(s3 + (k0 + 4 * q) * LD + col(i), LD));
      }
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int j = row(e);
      const float bj = sBeta[j];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if (j < Tc) a.dv[tok_off(a, b, h, t0 + j) + col(i)] = bj * av_acc[i][e];
        const float eg = exp2_fast(Gr[i][e]), x = bj * aw_acc[i][e];
        DK[i][e] += x * eg;
        DG[i][e] += x * kr[i][e] * eg;
      }
    }
  }
  lds_barrier();   // dT complete; k e^G (s1) no longer read

  // dbeta_j, first part: sum_t dT[t][j] M[t][j]; then dT -> dT diag(beta) in place
  {
    const int j = tid >> 3, part = tid & 7;
    float sum = 0.f;
    const float bj = sBeta[j];
#pragma unroll
    for (int x = 0; x < 8; ++x) {
      const int t = 8 * part + x;
      const float v = sT[t * LS + j];
      sum += v * sM[t * LS + j];
      sT[t * LS + j] = v * bj;
    }
    sum += __shfl_xor(sum, 1);
    sum += __shfl_xor(sum, 2);
    sum += __shfl_xor(sum, 4);
    if (part == 0) sB1[j] = sum;
  }
  lds_barrier();
  // Y = dM M^T -> s1 (row stride LS; only blocks on and below the diagonal are used)
  float *sYm = s1;
  {
    f32x4 p[2] = {zero4(), zero4()};
    const float *ar = sT + (16 * tm + r) * LS + 4 * q;
    for (int k0 = 0; k0 < C; k0 += 16) {
      const float4 av = ld4(ar + k0);
#pragma unroll
      for (int i = 0; i < 2; ++i)
        if (tn0 + 2 * i <= tm) p[i] = mma16(p[i], av, ld4(sM + col(i) * LS + k0 + 4 * q));
    }
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int e = 0; e < 4; ++e) sYm[row(e) * LS + col(i)] = p[i][e];
  }
  lds_barrier();
  // dA = -M^T Y (strictly lower): dKK = beta_t dA -> sT; dbeta_t += sum_j dA[t][j] KK[t][j]
  {
    float kk[2][4];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int e = 0; e < 4; ++e) kk[i][e] = rec[R_KK + row(e) * C + col(i)];
    f32x4 p[2] = {zero4(), zero4()};
    for (int k0 = 16 * tm; k0 < C; k0 += 16) {   // M[u][t] = 0 for u < t
      const float4 am = col4(sM + (k0 + 4 * q) * LS + 16 * tm + r, LS);
#pragma unroll
      for (int i = 0; i < 2; ++i)
        if (tn0 + 2 * i <= tm) p[i] = mma16(p[i], am, col4(sYm + (k0 + 4 * q) * LS + col(i), LS));
    }
    float part[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int t = row(e), j = col(i);
        const float da = j < t ? -p[i][e] : 0.f;
        sT[t * LS + j] = sBeta[t] * da;
        part[e] += da * kk[i][e];
      }
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      float x = part[e];
      x += __shfl_xor(x, 1);
      x += __shfl_xor(x, 2);
      x += __shfl_xor(x, 4);
      x += __shfl_xor(x, 8);
      if (r == 0) sB2[tn0][row(e)] = x;
    }
  }
  lds_barrier();   // Y (s1) no longer read
  // KL -> s1, KR -> s2, QR -> s3 (block start of each row's own 16-token block)
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float g0 = sGa[tm * D + col(i)], G = Gr[i][e];
      const float up = exp2_fast(G - g0), dn = exp2_fast(g0 - G);
      s1[row(e) * LD + col(i)] = kr[i][e] * dn;
      s2[row(e) * LD + col(i)] = kr[i][e] * up;
      s3[row(e) * LD + col(i)] = qr[i][e] * up;
    }
  lds_barrier();

  // pairwise terms, rows t (j in blocks bb <= t's block):
  //   sum_j dKK[t][j] e^{G_t-G_j} k_j = sum_bb e^{G_t - G_R(bb)} (dKK[t, bb] KL[bb])
  for (int bb = 0; bb <= tm; ++bb) {
    f32x4 x[4], y[4];
    const float4 akk = ld4(sT + (16 * tm + r) * LS + 16 * bb + 4 * q);
    const float4 ap = ld4(sP + (16 * tm + r) * LS + 16 * bb + 4 * q);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float4 bl = col4(s1 + (16 * bb + 4 * q) * LD + col(i), LD);
      x[i] = mma16(zero4(), akk, bl);
      y[i] = mma16(zero4(), ap, bl);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float gr = sGa[bb * D + col(i)];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float f = exp2_fast(fminf(0.f, Gr[i][e] - gr));
        const float xs = x[i][e] * f, ys = y[i][e] * f;
        DK[i][e] += xs;
        DQ[i][e] += ys;
        DG[i][e] += xs * kr[i][e] + ys * qr[i][e];
      }
    }
  }
  // rows j (t in blocks aa >= j's block):
  //   sum_t dKK[t][j] e^{G_t-G_j} k_t = sum_aa e^{G_R(aa) - G_j} (dKK[aa, j]^T KR[aa]), same for dP, q
  for (int aa = tm; aa < 4; ++aa) {
    f32x4 x[4];
    const float4 akk = col4(sT + (16 * aa + 4 * q) * LS + 16 * tm + r, LS);
    const float4 ap = col4(sP + (16 * aa + 4 * q) * LS + 16 * tm + r, LS);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      x[i] = mma16(zero4(), akk, col4(s2 + (16 * aa + 4 * q) * LD + col(i), LD));
      x[i] = mma16(x[i], ap, col4(s3 + (16 * aa + 4 * q) * LD + col(i), LD));
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float gr = sGa[aa * D + col(i)];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float v = x[i][e] * exp2_fast(gr - Gr[i][e]);
        DK[i][e] += v;
        DG[i][e] -= v * kr[i][e];
      }
    }
  }
  // decays of the dg scan, loaded ahead: thread (channel si, quarter sp) owns tokens
  // 16 sp .. 16 sp + 15 of channel si
  const int si = tid & 127, sp = tid >> 7;
  float gq[16];
#pragma unroll
  for (int x = 0; x < 16; ++x) gq[x] = a.g[tok_off(a, b, h, t0 + min(16 * sp + x, Tc - 1)) + si];
  const float Dsi = rec[R_D + si];
  lds_barrier();   // s1, s2, sP free

  // outputs dq, dk; dG - dK_dec*K_dec -> s1, dK_dec*K_dec -> s2
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int t = row(e);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if (t < Tc) {
        const size_t o = tok_off(a, b, h, t0 + t) + col(i);
        a.dq[o] = DQ[i][e];
        a.dk[o] = DK[i][e];
      }
      s1[t * LD + col(i)] = DG[i][e] - KT[i][e];
      s2[t * LD + col(i)] = KT[i][e];
    }
  }
  if (tid < C) {
    const int t = tid;
    if (t < Tc) a.dbeta[(static_cast<size_t>(b) * a.T + t0 + t) * a.H + h] = sB1[t] + sB2[0][t] + sB2[1][t];
  }
  lds_barrier();
  // dg_u = mask_u (sum_{t >= u} dG_t + dGam),  dGam = sum_t dK_dec*K_dec + dD e^{Gam}:
  // quarter sums, then each quarter's suffix scan from its offset
  {
    float ps = 0.f, ks = 0.f;
#pragma unroll
    for (int x = 0; x < 16; ++x) {
      ps += s1[(16 * sp + x) * LD + si];
      ks += s2[(16 * sp + x) * LD + si];
    }
    sP[sp * D + si] = ps;
    sP[4 * D + sp * D + si] = ks;
  }
  lds_barrier();
  {
    float off = sdD[si] * Dsi;
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      off += sP[4 * D + p * D + si];
      if (p > sp) off += sP[p * D + si];
    }
#pragma unroll
    for (int x = 15; x >= 0; --x) {
      const int u = 16 * sp + x;
      off += s1[u * LD + si];
      if (u < Tc) {
        const float g = gq[x];
        a.dg[tok_off(a, b, h, t0 + u) + si] = (g >= kFloor && g <= 0.f) ? off : 0.f;
      }
    }
  }
}

}  // namespace

size_t backward_workspace_bytes(int B, int T, int H) {
  const size_t nc = T > 0 ? (static_cast<size_t>(T) + C - 1) / C : 0;
  return static_cast<size_t>(B) * H * nc * (static_cast<size_t>(REC) + 2 * D * D + C * D) * sizeof(float);
}

hipError_t launch_backward(const kda_backward_desc &d, hipStream_t s) {
  BwdArgs a;
  a.q = d.q; a.k = d.k; a.v = d.v; a.g = d.g; a.beta = d.beta; a.S0 = d.S0;
  a.dO = d.dO; a.dSf = d.dS_final;
  a.dq = d.dq; a.dk = d.dk; a.dv = d.dv; a.dg = d.dg; a.dbeta = d.dbeta; a.dS0 = d.dS0;
  a.B = d.B; a.T = d.T; a.H = d.H;
  a.NC = d.T > 0 ? (d.T + C - 1) / C : 0;
  const size_t nch = static_cast<size_t>(d.B) * d.H * a.NC;
  float *ws = static_cast<float *>(d.workspace);
  a.rec = ws;
  a.sin = ws + nch * REC;
  a.dsa = a.sin + nch * D * D;
  a.du = a.dsa + nch * D * D;
  const int BH = d.B * d.H;
  if (BH == 0) return hipSuccess;
  const bool bf16 = d.in_dtype == KDA_BF16;
  if (nch > 0) {
    if (bf16) bwd_prep<true><<<dim3(static_cast<unsigned>(nch)), dim3(512), 0, s>>>(a);
    else bwd_prep<false><<<dim3(static_cast<unsigned>(nch)), dim3(512), 0, s>>>(a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  // Sweep units of 32 columns (each record fragment a wave loads serves two column
  // blocks) when there are enough of them to give every CU one; with few (sequence,
  // head) pairs, as in a long single sequence, units of 16 columns double the parallelism.
  int dev = 0, ncu = 256;
  if (hipGetDevice(&dev) == hipSuccess) {
    int v = 0;
    if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && v > 0) ncu = v;
  }
  const bool wide = static_cast<int64_t>(BH) * 4 >= ncu;
  const unsigned sweep_grid = static_cast<unsigned>((BH + 7) / 8 * 8 * (wide ? 4 : 8));
  if (nch > 0) {
    if (wide) bwd_fwd<2><<<dim3(sweep_grid), dim3(512), 0, s>>>(a);
    else bwd_fwd<1><<<dim3(sweep_grid), dim3(512), 0, s>>>(a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (wide) bwd_rev<2><<<dim3(sweep_grid), dim3(512), 0, s>>>(a);
  else bwd_rev<1><<<dim3(sweep_grid), dim3(512), 0, s>>>(a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (nch > 0) {
    if (bf16) bwd_grad<true><<<dim3(static_cast<unsigned>(nch)), dim3(512), 0, s>>>(a);
    else bwd_grad<false><<<dim3(static_cast<unsigned>(nch)), dim3(512), 0, s>>>(a);
    e = hipGetLastError();
  }
  return e;
}

}  // namespace kda
