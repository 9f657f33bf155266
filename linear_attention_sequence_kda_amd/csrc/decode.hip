// KDA recurrent decode step (the recurrent form; "xhh.club" tag page 结构, entries on
// the recurrent form and on the chunkwise algorithm: decode uses the recurrent form).
//
// One workgroup owns one (sequence, head) state of 128 x 128 fp32 (64 KB).  The state
// is the only large operand, so the step is bound by HBM: it is read once and written
// once, in place, with 16-byte loads and stores that cover whole 512-byte rows per half
// wave.  Both reductions over the key axis come from one read of the state, using
//     o = S_new^T q = S'^T q + u (k . q),   with  S' = Diag(alpha) S,
// so e = S'^T k and f = S'^T q are reduced together, then u = beta (v - e) and the
// write S_new = S' + k u^T reuse the values still held in registers.
//
// Thread layout (256 threads): column group cg = tid % 32 owns columns 4cg..4cg+3;
// row phase rp = tid / 32 owns rows rp, rp+8, ..., rp+120 (16 rows).
//
// Small batches (fewer states than CUs, no gate): the value columns of a state are
// independent (u_j, o_j and column j of the update use column j of S only), so a state
// is split into four slices of 32 columns, one workgroup each, and a step over a few
// states spreads over four times as many CUs.  Each slice row is a whole 128-byte line,
// and the four slices of a state run on one XCD.  Column group cg = tid % 8, row phase
// rp = tid / 8 owns rows rp, rp+32, rp+64, rp+96.  The per-head RMSNorm of the gated
// form needs all 128 columns, so the gated step always takes whole states.
//
// The state is read and written with non-temporal accesses: a decode step streams every
// state once, so caching it only displaces other lines.  Measured on MI355X with the
// states of four 256-sequence x 16-head batches stepped in turn (each step's 256 MiB
// read from DRAM): 92.7 us per step with non-temporal loads and stores against 107.0 us
// with ordinary ones (5.87 against 5.09 TB/s of algorithmic traffic); non-temporal loads
// alone give 102.3 us, stores alone 109.5 us.
//
// Pooled form (serving): the states live in a pool of slots and sequence n of the
// batch uses slot slots[n]; everything else is as above.  A slot outside the pool
// leaves the pool untouched and gives NaN outputs for that sequence.
#include "internal.h"
#include "kda_device.h"

namespace kda {
namespace {

constexpr int D = 128;
constexpr int NT = 256;
typedef float v4f __attribute__((ext_vector_type(4)));

// the slice of a state one workgroup owns: COLS value columns
template <int COLS>
struct Slice {
  static constexpr int CG = COLS / 4;     // column groups of 4
  static constexpr int RP = NT / CG;      // row phases
  static constexpr int RPT = D / RP;      // rows per thread
  static constexpr int NSL = D / COLS;    // slices per state
};

struct DecodeArgs {
  const void *q, *k, *v, *gate;
  const float *g, *beta, *norm_weight;
  float *state;
  void *o;
  float eps;
  const int32_t *slots;   // pooled form: slot of each sequence, or null
  int32_t pool, H;        // pool size (slots), heads
};

template <bool IN_BF16, bool OUT_BF16, bool GATE, int COLS>
__global__ __launch_bounds__(NT) void decode_kernel(DecodeArgs a, int64_t n_states) {
  static_assert(!GATE || COLS == D, "the gated step normalises whole states");
  using SL = Slice<COLS>;
  constexpr int CG = SL::CG, RP = SL::RP, RPT = SL::RPT, NSL = SL::NSL;
  __shared__ float s_alpha[D], s_k[D], s_q[D];
  __shared__ float s_red[4][CG][9];
  __shared__ float s_sq[4];

  const int tid = threadIdx.x;
  const int cg = tid % CG, rp = tid / CG, wave = tid >> 6, lane = tid & 63;
  // blocks of eight states in turn, slice-major inside a block, so that the slices of
  // one state share an XCD (consecutive block ids go to consecutive XCDs)
  const int64_t bid = blockIdx.x;
  const int xcd = (int)(bid & 7);
  const int64_t rest = bid >> 3;
  const int sl = (int)(rest % NSL);
  const int64_t nh64 = (rest / NSL) * 8 + xcd;        // sequence * H + head
  if (nh64 >= n_states) return;
  const size_t nh = (size_t)nh64;
  const int c0 = sl * COLS;                            // first column of the slice
  size_t sh = nh;                                      // state index in the pool
  if (a.slots) {
    const int n = (int)(nh / a.H), h = (int)(nh % a.H);
    const int slot = a.slots[n];
    if (slot < 0 || slot >= a.pool) {                  // not a slot of the pool
      if (tid < CG) store4<OUT_BF16>(a.o, nh * D + c0 + 4 * tid, make_float4(__builtin_nanf(""), __builtin_nanf(""), __builtin_nanf(""), __builtin_nanf("")));
      return;
    }
    sh = (size_t)slot * a.H + h;
  }
  float *S = a.state + sh * (size_t)(D * D) + c0;

  // Issue the state loads first so their latency overlaps the small vector loads.
  float4 s[RPT];
#pragma unroll
  for (int m = 0; m < RPT; ++m) {
    const v4f w = __builtin_nontemporal_load(reinterpret_cast<const v4f *>(S + (size_t)(rp + RP * m) * D + 4 * cg));
    s[m] = make_float4(w.x, w.y, w.z, w.w);
  }

  if (tid < D) {
    const size_t i = nh * D + tid;
    s_alpha[tid] = exp2_fast(log2_decay(a.g[i]));
    s_k[tid] = load1<IN_BF16>(a.k, i);
    s_q[tid] = load1<IN_BF16>(a.q, i);
  }
  const float4 vv = load4<IN_BF16>(a.v, nh * D + c0 + 4 * cg);
  const float bt = a.beta[nh];
  __syncthreads();

  // Decay the rows, then partial reductions e = S'^T k, f = S'^T q and k.q.
  float4 e = make_float4(0.f, 0.f, 0.f, 0.f), f = e;
  float kq = 0.f;
#pragma unroll
  for (int m = 0; m < RPT; ++m) {
    const int i = rp + RP * m;
    const float al = s_alpha[i], kk = s_k[i], qq = s_q[i];
    s[m].x *= al; s[m].y *= al; s[m].z *= al; s[m].w *= al;
    e.x += s[m].x * kk; e.y += s[m].y * kk; e.z += s[m].z * kk; e.w += s[m].w * kk;
    f.x += s[m].x * qq; f.y += s[m].y * qq; f.z += s[m].z * qq; f.w += s[m].w * qq;
    kq += kk * qq;
  }
  // Sum the row phases of this wave (lanes l, l ^ CG, ...), then the four waves.
  float r[9] = {e.x, e.y, e.z, e.w, f.x, f.y, f.z, f.w, kq};
#pragma unroll
  for (int off = CG; off < 64; off <<= 1)
#pragma unroll
    for (int j = 0; j < 9; ++j) r[j] += __shfl_xor(r[j], off, 64);
  if (lane < CG) {
#pragma unroll
    for (int j = 0; j < 9; ++j) s_red[wave][cg][j] = r[j];
  }
  __syncthreads();
#pragma unroll
  for (int j = 0; j < 9; ++j) r[j] = s_red[0][cg][j] + s_red[1][cg][j] + s_red[2][cg][j] + s_red[3][cg][j];

  const float4 u = make_float4(bt * (vv.x - r[0]), bt * (vv.y - r[1]), bt * (vv.z - r[2]),
                               bt * (vv.w - r[3]));
  kq = r[8];
  // Write S_new = S' + k u^T.
#pragma unroll
  for (int m = 0; m < RPT; ++m) {
    const int i = rp + RP * m;
    const float kk = s_k[i];
    float4 x = s[m];
    x.x += kk * u.x; x.y += kk * u.y; x.z += kk * u.z; x.w += kk * u.w;
    __builtin_nontemporal_store(v4f{x.x, x.y, x.z, x.w}, reinterpret_cast<v4f *>(S + (size_t)i * D + 4 * cg));
  }

  float4 o = make_float4(r[4] + u.x * kq, r[5] + u.y * kq, r[6] + u.z * kq, r[7] + u.w * kq);
  if constexpr (GATE) {
    // Per-head RMSNorm over the 128 value columns, then the sigmoid gate.
    float sq = o.x * o.x + o.y * o.y + o.z * o.z + o.w * o.w;
#pragma unroll
    for (int off = 16; off >= 1; off >>= 1) sq += __shfl_xor(sq, off, 64);
    if (tid == 0) s_sq[0] = sq;
    __syncthreads();
    const float inv = rsqrtf(s_sq[0] * (1.0f / D) + a.eps);
    const float4 gt = load4<IN_BF16>(a.gate, nh * D + 4 * cg);
    float4 w = make_float4(1.f, 1.f, 1.f, 1.f);
    if (a.norm_weight) w = *reinterpret_cast<const float4 *>(a.norm_weight + 4 * cg);
    o.x *= inv * w.x * sigmoidf_(gt.x);
    o.y *= inv * w.y * sigmoidf_(gt.y);
    o.z *= inv * w.z * sigmoidf_(gt.z);
    o.w *= inv * w.w * sigmoidf_(gt.w);
  }
  if (rp == 0) store4<OUT_BF16>(a.o, nh * D + c0 + 4 * cg, o);
}

// states below which an ungated step splits each state into 32-column slices
constexpr int64_t kSplitBelow = 256;

template <bool IN_BF16, bool OUT_BF16, bool GATE>
hipError_t launch3(const DecodeArgs &a, int64_t n, hipStream_t s) {
  const int64_t groups = (n + 7) / 8;                 // blocks of eight states
  if (!GATE && n < kSplitBelow) {
    const unsigned grid = static_cast<unsigned>(groups * 8 * Slice<32>::NSL);
    hipLaunchKernelGGL((decode_kernel<IN_BF16, OUT_BF16, false, 32>), dim3(grid), dim3(NT), 0, s, a, n);
  } else {
    const unsigned grid = static_cast<unsigned>(groups * 8);
    hipLaunchKernelGGL((decode_kernel<IN_BF16, OUT_BF16, GATE, D>), dim3(grid), dim3(NT), 0, s, a, n);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_decode(const kda_decode_desc &d, const int32_t *slots, int32_t pool, hipStream_t s) {
  const int64_t n = (int64_t)d.N * d.H;
  if (n == 0) return hipSuccess;
  DecodeArgs a{d.q, d.k, d.v, d.gate, d.g, d.beta, d.norm_weight, d.state, d.o, d.norm_eps,
               slots, pool, d.H};
  const bool ib = d.in_dtype == KDA_BF16, ob = d.out_dtype == KDA_BF16, gt = d.gate != nullptr;
  const int64_t nb = n;
  if (ib) {
    if (ob) return gt ? launch3<true, true, true>(a, nb, s) : launch3<true, true, false>(a, nb, s);
    return gt ? launch3<true, false, true>(a, nb, s) : launch3<true, false, false>(a, nb, s);
  }
  if (ob) return gt ? launch3<false, true, true>(a, nb, s) : launch3<false, true, false>(a, nb, s);
  return gt ? launch3<false, false, true>(a, nb, s) : launch3<false, false, false>(a, nb, s);
}

}  // namespace kda
