// Chunkwise KDA prefill, part 2: the state recurrence between chunks.
//
// Per chunk, with the record written by the prep kernel (W, Qt, P, T, Kdec, e^{G_C};
// see prefill_prep.hip) and the state S (d_k x d_v) entering the chunk
// ("xhh.club" tag page 结构, entry on the chunkwise algorithm: recurrence between
// chunks, matrix products inside them):
//
//   U  = T V - W S                    the per-token writes u_t of the delta rule
//   O  = Qt S + P U                   outputs (then the optional per-head RMSNorm and
//                                     sigmoid gate, same page, entry on KDA's form)
//   S <- Diag(e^{G_C}) S + Kdec^T U
//
// Value columns are independent in all three products, so each wave owns NC/4
// columns of the state and runs its own recurrence on them: S and U stay in MFMA
// accumulators and feed the next products straight from registers (the record's
// operands are stored with the contraction index in the matching split order).  The
// only data shared by the waves of a workgroup is the chunk's record, which is
// copied into LDS once per workgroup by asynchronous global->LDS loads (one chunk ahead
// into two buffers for outputs, two chunks ahead into three for state maps), and the
// chunk's values V.  All products are fp16 MFMA with
// fp32 accumulation (fp32 MFMA for fp32 inputs).  MODE_TRANSITION computes a
// segment's state map for the associative scan of context parallelism instead of
// outputs.
#include <type_traits>

#include "internal.h"
#include "tiles.h"

namespace kda {
namespace {

constexpr int MODE_OUTPUT = 0;
constexpr int MODE_TRANSITION = 1;

struct StateArgs {
  const void *v, *gate;
  const float *S0, *norm_weight;
  const unsigned char *rec;   // prep records, [B*H][n_chunks]
  float *S_final, *ckpt;
  void *o;
  float *maps;        // [units][D][2D] segment maps (transition mode)
  const float *sin;   // [units][D][D] states entering each segment (segmented output mode)
  float eps;
  int T, H;
  int n_seg, seg_chunks, n_chunks;
  int ckpt_every, n_ckpt;
  int out_bf16, fused_gate, raw_out;   // raw_out: write raw fp32 o for a separate norm pass
  int n_units;        // B * H * n_seg
};

// Workgroup shape for NC state columns: up to 8 waves, 16 or 32 columns each.  VC
// value columns come with them: all NC for outputs; for a state map ([A | B], 2D
// columns) only the D columns of the B part carry values.
template <int NC, int MODE>
struct Shape {
  static constexpr int NW = NC / 16 < 8 ? NC / 16 : 8;
  static constexpr int NTH = NW * 64;
  static constexpr int NCW = NC / NW;                  // state columns per wave
  static constexpr int VC = MODE == MODE_OUTPUT ? NC : D;
  static constexpr int VOFF = MODE == MODE_OUTPUT ? 0 : D;   // first state column with values
};

// value columns of one chunk for this workgroup: groups of 8 columns, token-major
template <int C, int NC, bool F32, int MODE>
struct VRaw {
  static constexpr int NTH = Shape<NC, MODE>::NTH;
  static constexpr int VC = Shape<NC, MODE>::VC;
  static constexpr int NVG = C * VC / 8;
  static constexpr int NVPT = (NVG + NTH - 1) / NTH;
  Q8<F32> v[NVPT];
};

// x where ok, else zeros, without a branch
template <bool F32>
__device__ __forceinline__ Q8<F32> keep_if(Q8<F32> x, bool ok) {
  const uint32_t m = ok ? 0xffffffffu : 0u;
  if constexpr (F32) {
#pragma unroll
    for (int e = 0; e < 8; ++e) x[e] = __uint_as_float(__float_as_uint(x[e]) & m);
    return x;
  } else {
    return make_uint4(x.x & m, x.y & m, x.z & m, x.w & m);
  }
}

// Branch-free loads with addresses clamped into the chunk; values past the chunk (and
// the A part of a transition map, which carries no value) are zeroed when stored to
// LDS, so that a load is never consumed right after it is issued.
template <int C, int NC, bool F32, int MODE>
__device__ __forceinline__ void load_v(VRaw<C, NC, F32, MODE> &r, const StateArgs &a, size_t tok0, int nval,
                                       int c0, int tid) {
  using VR = VRaw<C, NC, F32, MODE>;
  constexpr int per_tok = VR::VC / 8;
  const size_t tok_stride = (size_t)a.H * D;
  const int cv = MODE == MODE_OUTPUT ? c0 : 0;
  using E = typename std::conditional<F32, float, uint16_t>::type;
  const E *vb = static_cast<const E *>(a.v) + tok0 + cv;     // uniform
#pragma unroll
  for (int u = 0; u < VR::NVPT; ++u) {
    const int x = tid + u * VR::NTH;
    const uint32_t tc = (uint32_t)min(x / per_tok, nval - 1);
    r.v[u] = load_q8<F32>(vb, tc * (uint32_t)tok_stride + (uint32_t)(x % per_tok) * 8u);
  }
}

// fp32 values are stored as they are; bf16 values as their bf16 bits, which each wave
// turns into fp16 operands with the scale of its columns (see the state kernel)
template <int C, int NC, bool F32, int MODE>
__device__ __forceinline__ void store_v(typename Op<F32>::T *sV, const VRaw<C, NC, F32, MODE> &r, int nval,
                                        int tid) {
  using VR = VRaw<C, NC, F32, MODE>;
  constexpr int per_tok = VR::VC / 8;
#pragma unroll
  for (int u = 0; u < VR::NVPT; ++u) {
    const int x = tid + u * VR::NTH;
    if (VR::NVG % VR::NTH == 0 || x < VR::NVG) {
      const Q8<F32> q = keep_if<F32>(r.v[u], x / per_tok < nval);
      if constexpr (F32) {
        float vv[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) vv[e] = q8_at<F32>(q, e);
        st8<F32, VR::VC>(sV, x / per_tok, (x % per_tok) * 8, vv);
      } else {
        using S = Swz<typename Op<F32>::T, VR::VC>;
        *reinterpret_cast<uint4 *>(sV + S::at(x / per_tok, (x % per_tok) * 8)) = q;
      }
    }
  }
}

// 4 consecutive inputs of a bf16 or fp32 tensor
template <bool F32>
using Q4 = typename std::conditional<F32, float4, uint2>::type;

template <bool F32>
__device__ __forceinline__ Q4<F32> load_q4(const void *p, size_t idx) {
  if constexpr (F32) return *reinterpret_cast<const float4 *>(static_cast<const float *>(p) + idx);
  else return *reinterpret_cast<const uint2 *>(static_cast<const uint16_t *>(p) + idx);
}

template <bool F32>
__device__ __forceinline__ float q4_at(const Q4<F32> &x, int e) {
  if constexpr (F32) {
    return e == 0 ? x.x : e == 1 ? x.y : e == 2 ? x.z : x.w;
  } else {
    const uint32_t w = e < 2 ? x.x : x.y;
    return __uint_as_float((e & 1) ? (w & 0xffff0000u) : (w << 16));
  }
}

// Byte offsets (within a record) of the operand fragments one chunk step reads, in
// the order it reads them: -W (key block outer, token tile inner), T, Kdec^T, then for
// outputs Qt and P.  Blocks of T and P above the diagonal are zero and not stored.
template <int C, bool F32, bool OUT>
struct SeqFrags {
  using R = Rec<C, F32>;
  static constexpr int NT = C / 16, KB = R::KB;
  struct List {
    int off[R::nW + R::nT + R::nK + R::nQ + R::nP];
    int n;
  };
  static constexpr List make() {
    List l{};
    int n = 0;
    for (int kb = 0; kb < 4; ++kb)
      for (int tb = 0; tb < NT; ++tb) l.off[n++] = (int)(R::oW + (size_t)(tb * 4 + kb) * R::FRAG);
    for (int kb = 0; kb < KB; ++kb)
      for (int tb = 0; tb < NT; ++tb)
        if (R::nz(tb, kb)) l.off[n++] = (int)(R::oT + (size_t)R::tri(tb, kb) * R::FRAG);
    for (int kb = 0; kb < KB; ++kb)
      for (int ib = 0; ib < 8; ++ib) l.off[n++] = (int)(R::oK + (size_t)(ib * KB + kb) * R::FRAG);
    if (OUT) {
      for (int kb = 0; kb < 4; ++kb)
        for (int tb = 0; tb < NT; ++tb) l.off[n++] = (int)(R::oQ + (size_t)(tb * 4 + kb) * R::FRAG);
      for (int kb = 0; kb < KB; ++kb)
        for (int tb = 0; tb < NT; ++tb)
          if (R::nz(tb, kb)) l.off[n++] = (int)(R::oP + (size_t)R::tri(tb, kb) * R::FRAG);
    }
    l.n = n;
    return l;
  }
  static constexpr List seq = make();
  static constexpr int n = seq.n;
};

// Largest of a non-negative float (given as its bits, which order as the values do)
// over the wave: within rows of 16 lanes by DPP (pairs, quads, half rows, rows), then
// the four row results through scalar registers.  All 64 lanes must be active.
__device__ __forceinline__ int wave_max_nonneg(int v) {
  v = max(v, __builtin_amdgcn_update_dpp(0, v, 0xB1, 0xf, 0xf, false));    // quad_perm 1,0,3,2
  v = max(v, __builtin_amdgcn_update_dpp(0, v, 0x4E, 0xf, 0xf, false));    // quad_perm 2,3,0,1
  v = max(v, __builtin_amdgcn_update_dpp(0, v, 0x141, 0xf, 0xf, false));   // row_half_mirror
  v = max(v, __builtin_amdgcn_update_dpp(0, v, 0x140, 0xf, 0xf, false));   // row_mirror
  return max(max(__builtin_amdgcn_readlane(v, 0), __builtin_amdgcn_readlane(v, 16)),
             max(__builtin_amdgcn_readlane(v, 32), __builtin_amdgcn_readlane(v, 48)));
}

// Operand range.  With bf16 inputs the values, the state copy and U enter the products
// as fp16 operands, whose range ends at 65504, while bf16 values and the fp32 state can
// be far larger.  Every product is linear in (values, state) column by column, so each
// 16-column block of a wave carries a power-of-two scale 2^-e: the fp32 state is held
// as S 2^-e, values enter as v 2^-e, and outputs, checkpoints, final states and maps
// are multiplied back by 2^e.  e is 0 (no scaling at all) while every |S| and |v| of the
// block stays below 2^9; otherwise each step sets it so that the block's largest
// magnitude lies in [2^8, 2^9).  The bound that makes this enough: for keys of unit
// norm, beta in [0, 1] and decays at most 1, one token changes a state column's 2-norm
// by at most |v| (I - beta k k^T has norm at most 1), and |u| is at most |v| plus that
// norm.  Over a chunk of 64 from entries below 2^9 this gives |u| and |S| below
// 2^9 (1 + 128^(1/2) + 63) < 38600, inside fp16, and the same argument bounds every
// record entry (W, T, P, Kdec, Q~) by 1.  Powers of two change no rounding.
//
// GATE: the output pass of a whole head (NC = 128) with the fused RMSNorm and gate
template <int C, int NC, bool F32, int MODE, bool GATE>
__global__ __launch_bounds__((Shape<NC, MODE>::NTH), 1) void chunk_state_kernel(StateArgs a) {
  using R = Rec<C, F32>;
  using T = typename Op<F32>::T;
  using V8 = typename Op<F32>::V8;
  constexpr int KC = C < 32 ? 32 : C;
  constexpr int KB = R::KB, NT = C / 16;
  using SH = Shape<NC, MODE>;
  constexpr int NW = SH::NW, NTH = SH::NTH;            // two waves per SIMD for NC >= 128
  constexpr int NCW = SH::NCW;                         // state columns per wave
  constexpr int CBW = NCW / 16;                        // 16-column blocks per wave
  constexpr int VC = SH::VC;                           // value columns in LDS
  static_assert(!GATE || (MODE == MODE_OUTPUT && NC == D), "the fused epilogue needs whole heads");
  static_assert(MODE == MODE_OUTPUT || (NC == 2 * D && CBW == 2), "a state map is one workgroup, two blocks per wave");
  constexpr int VS = (MODE == MODE_TRANSITION ? 2 * D : D) / NC;   // workgroups per unit
  // KiB of the record this pass copies (the state map needs only its prefix)
  constexpr int NBLK = (int)((MODE == MODE_TRANSITION ? R::trans : R::bytes) / 1024);
  // Values and norm partials are double buffered (chunks alternate), records double
  // buffered for outputs and triple buffered for state maps (the copy of chunk n+2 is
  // in flight during chunk n: a map step has less work to hide it behind).  Each
  // buffer is a separate LDS object, so the compiler sees that reads of one buffer do
  // not depend on the asynchronous copy in flight into another.
  constexpr int NRB = MODE == MODE_TRANSITION ? 3 : 2;
  __shared__ __align__(16) unsigned char recA[NBLK * 1024];
  __shared__ __align__(16) unsigned char recB[NBLK * 1024];
  __shared__ __align__(16) unsigned char recC[NRB == 3 ? NBLK * 1024 : 16];
  __shared__ __align__(16) T sVA[KC * VC];             // V [t][c] (rows >= C zero)
  __shared__ __align__(16) T sVB[KC * VC];
  __shared__ __align__(16) float sNormA[GATE ? C * NW : 1];   // per-token, per-wave sums of squares
  __shared__ __align__(16) float sNormB[GATE ? C * NW : 1];

  // the wave index is uniform: branches on it are scalar (MFMAs ignore the lane mask,
  // so a product skipped by a wave must be skipped by a real branch)
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lr = lane & 15, lg = lane >> 4;

  // XCD-aware placement: consecutive workgroup ids go to different XCDs, so the
  // column slices of one unit get ids that are equal modulo 8 (same XCD, shared L2
  // for the record they both read).
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
  const int cw = wave * NCW;                           // this wave's first column in the slice
  // First column of 16-column block j of this wave.  A state map gives each wave one
  // block of the A part and the matching block of the B part, so that every wave has
  // the same work (only B blocks carry values).
  auto colb = [&](int j) __attribute__((always_inline)) {
    return MODE == MODE_TRANSITION ? j * D + 16 * wave : c0 + cw + 16 * j;
  };
  const size_t tok_stride = (size_t)a.H * D;
  const size_t state_off = (size_t)bh * D * D;
  const unsigned char *rec_bh = a.rec + (size_t)bh * a.n_chunks * R::bytes;
  auto tok_base = [&](int chunk) __attribute__((always_inline)) {
    return ((size_t)b * a.T + (size_t)chunk * C) * tok_stride + (size_t)h * D;
  };

  // V rows past the chunk stay zero (only when KC > C)
  if constexpr (KC > C) {
    for (int x = tid; x < (KC - C) * VC; x += NTH) sVA[C * VC + x] = sVB[C * VC + x] = T(0);
  }

  // ---- initial state: S[ib][j] holds rows 16ib + 4lg + r, column colb(j) + lr
  f32x4 S[8][CBW];
#pragma unroll
  for (int ib = 0; ib < 8; ++ib)
#pragma unroll
    for (int j = 0; j < CBW; ++j) {
      const int c = colb(j) + lr;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int i = 16 * ib + 4 * lg + r;
        float x;
        if constexpr (MODE == MODE_TRANSITION) {
          x = (c < D && i == c) ? 1.f : 0.f;           // [A | B] starts at [I | 0]
        } else if (a.n_seg > 1) {
          x = a.sin[(size_t)unit * D * D + (size_t)i * D + c];   // from the segment scan
        } else {
          x = a.S0 ? a.S0[state_off + (size_t)i * D + c] : 0.f;
        }
        S[ib][j][r] = x;
      }
    }

  // power-of-two scale exponent of each 16-column block (wave-uniform; always 0 with
  // fp32 operands)
  int esc[CBW];
#pragma unroll
  for (int j = 0; j < CBW; ++j) esc[j] = 0;

  // asynchronous copy of one chunk's record into an LDS buffer: one KiB per wave
  // instruction, lane l's 16 bytes landing at offset 16 l of that KiB (every wave
  // issues the same number of copies, the last KiB possibly twice, so the count of
  // memory operations in flight is known at compile time)
  constexpr int NCOPY = (NBLK + NW - 1) / NW;          // copies per wave and chunk
  auto copy_rec = [&](unsigned char *dst, int chunk, int n0, int n1) __attribute__((always_inline)) {
    const unsigned char *src = rec_bh + (size_t)chunk * R::bytes;   // uniform
#pragma unroll
    for (int n = n0; n < n1; ++n) {
      const int blk = min(wave + NW * n, NBLK - 1);
      // non-temporal (cache policy 2): a record is read once per pass, and caching it only
      // displaces other lines (1% on the 8k workload)
      __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void *)(src + (uint32_t)(blk * 1024 + 16 * lane)),
                                       (__attribute__((address_space(3))) void *)(dst + (size_t)blk * 1024), 16, 0, 2);
    }
  };
  // gate logits for the fused epilogue: token 16tb + lr, columns cw + 16j + 4lg .. +3
  auto load_gate = [&](Q4<F32> (&gt)[NT][CBW], int chunk) __attribute__((always_inline)) {
    const int nv = min(C, a.T - chunk * C);
    using E = typename std::conditional<F32, float, uint16_t>::type;
    const E *gb = static_cast<const E *>(a.gate) + tok_base(chunk) + cw;   // uniform
#pragma unroll
    for (int tb = 0; tb < NT; ++tb)
#pragma unroll
      for (int j = 0; j < CBW; ++j) {
        const uint32_t t = (uint32_t)min(16 * tb + lr, nv - 1);   // rows past the end are never used
        gt[tb][j] = load_q4<F32>(gb, t * (uint32_t)tok_stride + (uint32_t)(16 * j + 4 * lg));
      }
  };

  const int ch_begin = seg * a.seg_chunks;
  const int ch_end = min(a.n_chunks, ch_begin + a.seg_chunks);

  // Pipeline.  Within one chunk no register loaded during that chunk is consumed:
  // with loads, stores and LDS copies in flight together the compiler can only wait
  // for all of them, so every wait happens at the top of a chunk, where the record
  // copy has to be complete anyway.  Per chunk n, after the one barrier of the step:
  // the norm and gate of chunk n-1 are applied (its per-wave sums of squares were
  // written at the end of n-1), the gate of n is loaded, the values of n+1 (loaded
  // during n-1) go to the other V buffer and those of n+2 are loaded, the record of
  // n+1 is copied, and the outputs of n-1 are stored between the products.
  VRaw<C, NC, F32, MODE> vr;
  Q4<F32> gq[NT][CBW];                                 // gate logits of one chunk
  f32x4 op[NT][CBW];                                   // outputs of the previous chunk
  float wv[CBW][4];                                    // RMSNorm weights of this wave's columns
  if constexpr (GATE) {
#pragma unroll
    for (int j = 0; j < CBW; ++j)
#pragma unroll
      for (int r = 0; r < 4; ++r) wv[j][r] = a.norm_weight ? a.norm_weight[cw + 16 * j + 4 * lg + r] : 1.f;
  }
  const int ch_last = ch_end - 1;
  load_v<C, NC, F32, MODE>(vr, a, tok_base(ch_begin), min(C, a.T - ch_begin * C), c0, tid);
  copy_rec(recA, ch_begin, 0, NCOPY);
  __builtin_amdgcn_s_waitcnt(0x0F70);
  store_v<C, NC, F32, MODE>(sVA, vr, min(C, a.T - ch_begin * C), tid);
  {
    const int n1 = min(ch_begin + 1, ch_last);
    load_v<C, NC, F32, MODE>(vr, a, tok_base(n1), min(C, a.T - n1 * C), c0, tid);
    if constexpr (NRB == 3) copy_rec(recB, n1, 0, NCOPY);
  }
  // With three record buffers, every memory operation but the record copy issued last
  // (two buffers ahead) has to be complete at the top of a step.  The count is exact:
  // every wave issues NCOPY copies per step, after its value loads.
  static_assert(NRB == 2 || NCOPY < 16, "vmcnt field");

  // per-head RMSNorm over the 128 value columns, then the sigmoid gate, applied to the
  // raw outputs op of one chunk, with that chunk's sums of squares and gate logits
  auto norm_gate = [&](const float *sn) __attribute__((always_inline)) {
#pragma unroll
    for (int tb = 0; tb < NT; ++tb) {
      const int t = 16 * tb + lr;
      float tot = 0.f;
#pragma unroll
      for (int w4 = 0; w4 < NW / 4; ++w4) {
        const float4 x = *reinterpret_cast<const float4 *>(sn + t * NW + 4 * w4);
        tot += (x.x + x.y) + (x.z + x.w);
      }
      const float inv = rsqrtf(tot * (1.0f / D) + a.eps);
#pragma unroll
      for (int j = 0; j < CBW; ++j)
#pragma unroll
        for (int r = 0; r < 4; ++r) op[tb][j][r] *= inv * wv[j][r] * sigmoidf_(q4_at<F32>(gq[tb][j], r));
    }
  };

  // outputs of token tile tb of one chunk (lane: token 16tb + lr, columns
  // c0 + cw + 16j + 4lg .. +3)
  auto store_tile = [&](int chunk, int tb) __attribute__((always_inline)) {
    const int nv = min(C, a.T - chunk * C);
    const size_t base = tok_base(chunk) + c0 + cw;                      // uniform
    const bool ok = 16 * tb + lr < nv;
    if (a.out_bf16 && !a.raw_out) {
      uint16_t *ob = static_cast<uint16_t *>(a.o) + base;
#pragma unroll
      for (int j = 0; j < CBW; ++j)
        if (ok)
          store4<true>(ob, (uint32_t)(16 * tb + lr) * (uint32_t)tok_stride + (uint32_t)(16 * j + 4 * lg),
                       make_float4(op[tb][j][0], op[tb][j][1], op[tb][j][2], op[tb][j][3]));
    } else {
      float *ob = static_cast<float *>(a.o) + base;
#pragma unroll
      for (int j = 0; j < CBW; ++j)
        if (ok)
          *reinterpret_cast<float4 *>(ob + ((uint32_t)(16 * tb + lr) * (uint32_t)tok_stride + (uint32_t)(16 * j + 4 * lg))) =
              make_float4(op[tb][j][0], op[tb][j][1], op[tb][j][2], op[tb][j][3]);
    }
  };
  // checkpoint: the state after a chunk that ends on a multiple of ckpt_every tokens
  auto store_ckpt = [&](int chunk) __attribute__((always_inline)) {
    const int t0 = chunk * C, nv = min(C, a.T - t0);
    if (a.ckpt_every > 0 && nv == C && (t0 + C) % a.ckpt_every == 0) {
      const int m = (t0 + C) / a.ckpt_every - 1;
      float *dst = a.ckpt + (((size_t)b * a.n_ckpt + m) * a.H + h) * (size_t)D * D;
#pragma unroll
      for (int ib = 0; ib < 8; ++ib)
#pragma unroll
        for (int j = 0; j < CBW; ++j)
#pragma unroll
          for (int r = 0; r < 4; ++r)
            dst[(size_t)(16 * ib + 4 * lg + r) * D + c0 + cw + 16 * j + lr] = ldexpf(S[ib][j][r], esc[j]);
    }
  };

  // one chunk, reading record buffer RB and value buffer BUF (A or B) and filling the
  // others: the record copy goes to the buffer NRB - 1 ahead
  auto recbuf = [&](int i) __attribute__((always_inline)) { return i == 0 ? recA : i == 1 ? recB : recC; };
  auto step = [&](auto bufc, auto rbc, int chunk) __attribute__((always_inline)) {
    constexpr int BUF = decltype(bufc)::value;
    constexpr int RB = decltype(rbc)::value;
    unsigned char *rc = recbuf(RB);
    unsigned char *rn = recbuf((RB + NRB - 1) % NRB);
    const T *sV = BUF == 0 ? sVA : sVB;
    T *sVn = BUF == 0 ? sVB : sVA;
    if constexpr (NRB == 2) {
      // This wave's loads and record copies landed: all but the previous step's output
      // stores, issued last (NT * CBW of them when that step had outputs to store), then
      // a barrier without a memory fence (a fence would wait for the stores too).
      static_assert(NT * CBW < 16, "vmcnt field");
      asm volatile("" ::: "memory");
      if (MODE == MODE_OUTPUT && chunk - 1 > ch_begin) __builtin_amdgcn_s_waitcnt(0x0070 | (NT * CBW));
      else __builtin_amdgcn_s_waitcnt(0x0070);       // vmcnt(0) lgkmcnt(0)
      __builtin_amdgcn_s_barrier();
      asm volatile("" ::: "memory");
    } else {
      // The same with the record copy issued last still in flight, and a barrier without
      // a memory fence (a fence would wait for it): every exchange through LDS is
      // complete once lgkmcnt and vmcnt have counted it.  Nothing of the step moves above
      // the barrier, where a use of the value registers would again wait for everything.
      asm volatile("" ::: "memory");
      __builtin_amdgcn_s_waitcnt(0x0070 | NCOPY);      // vmcnt(NCOPY) lgkmcnt(0)
      __builtin_amdgcn_s_barrier();
      asm volatile("" ::: "memory");
      __builtin_amdgcn_sched_barrier(0);
    }

    const bool prev = MODE == MODE_OUTPUT && chunk > ch_begin;
    if constexpr (GATE) {
      if (prev) norm_gate(BUF == 0 ? sNormB : sNormA);
      load_gate(gq, chunk);
    }
    const int nx = min(chunk + 1, ch_last);            // the last chunk reloads its own
    {                                                  // values of chunk+1 (loaded a chunk ago)
      store_v<C, NC, F32, MODE>(sVn, vr, min(C, a.T - nx * C), tid);
      const int n2 = min(chunk + 2, ch_last);
      load_v<C, NC, F32, MODE>(vr, a, tok_base(n2), min(C, a.T - n2 * C), c0, tid);
    }
    if (prev) store_ckpt(chunk - 1);

    // Record fragments are read from LDS through a ring of PF registers, PF fragments
    // ahead of the product that consumes them, in the order the products below take
    // them (SeqFrags), so that LDS latency overlaps the matrix cores.
    using SF = SeqFrags<C, F32, MODE == MODE_OUTPUT>;
    // (fp32 fragments are twice as wide: a two-deep ring keeps the gated fp32 pass
    // within its registers, with no scratch)
    constexpr int PF_MAX = F32 && GATE ? 2 : 4;
    constexpr int PF = SF::n < PF_MAX ? SF::n : PF_MAX;
    auto fetch = [&](int i) __attribute__((always_inline)) {
      return Op<F32>::load(reinterpret_cast<const T *>(rc + SF::seq.off[i] + lane * 8 * sizeof(T)));
    };
    V8 ring[PF];
#pragma unroll
    for (int i = 0; i < PF; ++i) ring[i] = fetch(i);
    // A later record's copy is issued late in the step: while an asynchronous copy into
    // LDS is in flight the compiler waits for all outstanding LDS reads at every use,
    // which defeats the read-ahead.  The state map pass (three buffers) copies the record
    // after next once its last fragment read is issued.  The outputs pass copies the
    // next record once the reads of the state products are issued, before the output
    // stores of the previous chunk: the next step then waits for the copy with those
    // stores still in flight.
    constexpr int COPY_AT = MODE == MODE_OUTPUT ? R::nW + R::nT + R::nK : SF::n - 1;
    auto take = [&](int i) __attribute__((always_inline)) {
      const V8 f = ring[i % PF];
      if (i + PF < SF::n) ring[i % PF] = fetch(i + PF);
      if (i + PF == COPY_AT) copy_rec(rn, NRB == 2 ? nx : min(chunk + 2, ch_last), 0, NCOPY);
      __builtin_amdgcn_sched_barrier(0);             // keep the read PF products ahead
      return f;
    };
    // the A part of a state map (block 0 of each wave) carries no values: no T V product
    // there
    auto has_v = [&](int j) __attribute__((always_inline)) { return MODE == MODE_OUTPUT || j == 1; };
    // S and V as operands (contraction over key channels / tokens, split order)
    V8 sf[4][CBW], vf[KB][CBW] = {};
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
      for (int j = 0; j < CBW; ++j) sf[kb][j] = frag_from<F32>(S[2 * kb][j], S[2 * kb + 1][j]);
    if constexpr (F32) {
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int j = 0; j < CBW; ++j)
          if (has_v(j)) vf[kb][j] = ld_t_split<F32, VC>(sV, 32 * kb, colb(j) - SH::VOFF - c0, lane);
    } else {
#pragma unroll
      for (int j = 0; j < CBW; ++j) {
        // the block's values (bf16 bits in LDS) as unscaled operands, and their largest
        // magnitude
        auto vraw = [&](int kb) __attribute__((always_inline)) {
          // the whole vector reinterpreted: a bit cast of one vector element reads the
          // vector's first element
          return __builtin_bit_cast(uint4, ld_t_split<F32, VC>(sV, 32 * kb, colb(j) - SH::VOFF - c0, lane));
        };
        float lm = 0.f;
        if (has_v(j)) {
#pragma unroll
          for (int kb = 0; kb < KB; ++kb) {
            const uint4 w = vraw(kb);
#pragma unroll
            for (int e = 0; e < 8; ++e) {
              const float x = q8_at<false>(w, e);
              lm = fmaxf(lm, fabsf(x));
              vf[kb][j][e] = Op<F32>::cvt(x);
            }
          }
        }
        float ls = 0.f;                                // scaled state
#pragma unroll
        for (int ib = 0; ib < 8; ++ib)
#pragma unroll
          for (int r = 0; r < 4; ++r) ls = fmaxf(ls, fabsf(S[ib][j][r]));
        const float lim = 512.f;                       // 2^9
        if (esc[j] != 0 || __any(lm >= lim || ls >= lim)) {
          // largest magnitude of the block, in true units, over the wave, and the
          // exponent en that brings it into [2^8, 2^9)
          const int mb = wave_max_nonneg(max(__float_as_int(ldexpf(ls, esc[j])), __float_as_int(lm)));
          const int en = mb >= 0x44000000 ? min(((mb >> 23) & 0xff) - 135, 120) : 0;
          if (en != esc[j]) {
#pragma unroll
            for (int ib = 0; ib < 8; ++ib)
#pragma unroll
              for (int r = 0; r < 4; ++r) S[ib][j][r] = ldexpf(S[ib][j][r], esc[j] - en);
#pragma unroll
            for (int kb = 0; kb < 4; ++kb) sf[kb][j] = frag_from<F32>(S[2 * kb][j], S[2 * kb + 1][j]);
            esc[j] = en;
          }
          if (has_v(j) && esc[j] != 0) {               // the values again, scaled
            const float sc = __int_as_float((127 - esc[j]) << 23);   // 2^-e, e <= 120
#pragma unroll
            for (int kb = 0; kb < KB; ++kb) {
              const uint4 w = vraw(kb);
#pragma unroll
              for (int e = 0; e < 8; ++e) vf[kb][j][e] = Op<F32>::cvt(q8_at<false>(w, e) * sc);
            }
          }
        }
      }
    }

    // The products run as independent accumulation chains, one per output tile, stepped
    // together over the contraction blocks, so that consecutive MFMAs do not wait on
    // each other.
    int fi = 0;                                        // next fragment of the sequence
    // ===== U = T V + (-W) S: lane holds U[16tb + 4lg + r][cw + 16j + lr] =====
    f32x4 U[NT][CBW];
#pragma unroll
    for (int tb = 0; tb < NT; ++tb)
#pragma unroll
      for (int j = 0; j < CBW; ++j) U[tb][j] = zero4();
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
#pragma unroll
      for (int tb = 0; tb < NT; ++tb) {
        const V8 wf = take(fi++);
#pragma unroll
        for (int j = 0; j < CBW; ++j) U[tb][j] = Op<F32>::mma(U[tb][j], wf, sf[kb][j]);
      }
    }
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
      for (int tb = 0; tb < NT; ++tb) {
        if (!R::nz(tb, kb)) continue;                  // T is lower triangular
        const V8 tf = take(fi++);
#pragma unroll
        for (int j = 0; j < CBW; ++j)
          if (has_v(j)) U[tb][j] = Op<F32>::mma(U[tb][j], tf, vf[kb][j]);
      }
    // U as an operand (contraction over tokens; tokens past the chunk are zero)
    V8 uf[KB][CBW];
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
      for (int j = 0; j < CBW; ++j) uf[kb][j] = frag_from<F32>(U[2 * kb][j], 2 * kb + 1 < NT ? U[2 * kb + 1][j] : zero4());

    // ===== S <- Diag(e^{G_C}) S + Kdec^T U (S as an operand was taken above) =====
#pragma unroll
    for (int ib = 0; ib < 8; ++ib) {
      const float4 dec = *reinterpret_cast<const float4 *>(rc + R::oDec + 4 * (16 * ib + 4 * lg));
#pragma unroll
      for (int j = 0; j < CBW; ++j) {
        S[ib][j][0] *= dec.x; S[ib][j][1] *= dec.y; S[ib][j][2] *= dec.z; S[ib][j][3] *= dec.w;
      }
    }
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
      for (int ib = 0; ib < 8; ++ib) {
        const V8 kf = take(fi++);
#pragma unroll
        for (int j = 0; j < CBW; ++j) S[ib][j] = Op<F32>::mma(S[ib][j], kf, uf[kb][j]);
      }

    // ===== O^T = S^T Qt^T + U^T P^T: lane holds O[16tb + lr][cw + 16j + 4lg + r] =====
    f32x4 O[NT][CBW];
    if constexpr (MODE == MODE_OUTPUT) {
#pragma unroll
      for (int tb = 0; tb < NT; ++tb)
#pragma unroll
        for (int j = 0; j < CBW; ++j) O[tb][j] = zero4();
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
#pragma unroll
        for (int tb = 0; tb < NT; ++tb) {
          const V8 qf = take(fi++);
#pragma unroll
          for (int j = 0; j < CBW; ++j) O[tb][j] = Op<F32>::mma(O[tb][j], sf[kb][j], qf);
        }
        if (prev && kb < NT) store_tile(chunk - 1, kb);
      }
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int tb = 0; tb < NT; ++tb) {
          if (!R::nz(tb, kb)) continue;                // P is lower triangular
          const V8 pf = take(fi++);
#pragma unroll
          for (int j = 0; j < CBW; ++j) O[tb][j] = Op<F32>::mma(O[tb][j], uf[kb][j], pf);
        }
    }

    if constexpr (MODE == MODE_OUTPUT) {
#pragma unroll
      for (int tb = 0; tb < NT; ++tb)
#pragma unroll
        for (int j = 0; j < CBW; ++j) op[tb][j] = O[tb][j];
#pragma unroll
      for (int j = 0; j < CBW; ++j)
        if (esc[j] != 0) {                             // outputs in true units
#pragma unroll
          for (int tb = 0; tb < NT; ++tb)
#pragma unroll
            for (int r = 0; r < 4; ++r) op[tb][j][r] = ldexpf(op[tb][j][r], esc[j]);
        }
    }
    // per-token sums of squares of this wave's columns for the fused RMSNorm
    if constexpr (GATE) {
      float *sn = BUF == 0 ? sNormA : sNormB;
#pragma unroll
      for (int tb = 0; tb < NT; ++tb) {
        float ss = 0.f;
#pragma unroll
        for (int j = 0; j < CBW; ++j)
#pragma unroll
          for (int r = 0; r < 4; ++r) ss += op[tb][j][r] * op[tb][j][r];   // true units
        ss += __shfl_xor(ss, 16, 64);
        ss += __shfl_xor(ss, 32, 64);
        if (lg == 0) sn[(16 * tb + lr) * NW + wave] = ss;
      }
    }
  };
  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  using I2 = std::integral_constant<int, 2>;
  if constexpr (NRB == 2) {
    for (int chunk = ch_begin; chunk < ch_end; chunk += 2) {
      step(I0{}, I0{}, chunk);
      if (chunk + 1 < ch_end) step(I1{}, I1{}, chunk + 1);
    }
  } else {
    // (the loop is left as soon as the chunks run out, so that no path skips a step and
    // runs a later one: the compiler's wait counts stay exact at every step; segments are
    // never empty, so the first step always runs)
    for (int chunk = ch_begin;; chunk += 6) {
      step(I0{}, I0{}, chunk);
      if (chunk + 1 >= ch_end) break;
      step(I1{}, I1{}, chunk + 1);
      if (chunk + 2 >= ch_end) break;
      step(I0{}, I2{}, chunk + 2);
      if (chunk + 3 >= ch_end) break;
      step(I1{}, I0{}, chunk + 3);
      if (chunk + 4 >= ch_end) break;
      step(I0{}, I1{}, chunk + 4);
      if (chunk + 5 >= ch_end) break;
      step(I1{}, I2{}, chunk + 5);
      if (chunk + 6 >= ch_end) break;
    }
  }
  if constexpr (MODE == MODE_OUTPUT) {
    __builtin_amdgcn_s_waitcnt(0x0F70);                // gate of the last chunk
    __syncthreads();                                   // its sums of squares
    if constexpr (GATE) norm_gate(((ch_last - ch_begin) & 1) == 0 ? sNormA : sNormB);
#pragma unroll
    for (int tb = 0; tb < NT; ++tb) store_tile(ch_last, tb);
    store_ckpt(ch_last);
  }

  // ---- results: the final state (last segment) or the segment map
  if constexpr (MODE == MODE_OUTPUT) {
    if (a.S_final && seg == a.n_seg - 1) {
#pragma unroll
      for (int ib = 0; ib < 8; ++ib)
#pragma unroll
        for (int j = 0; j < CBW; ++j)
#pragma unroll
          for (int r = 0; r < 4; ++r)
            a.S_final[state_off + (size_t)(16 * ib + 4 * lg + r) * D + c0 + cw + 16 * j + lr] = ldexpf(S[ib][j][r], esc[j]);
    }
  } else {
    float *dst = a.maps + (size_t)unit * D * (2 * D);
#pragma unroll
    for (int ib = 0; ib < 8; ++ib)
#pragma unroll
      for (int j = 0; j < CBW; ++j)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          dst[(size_t)(16 * ib + 4 * lg + r) * (2 * D) + colb(j) + lr] = ldexpf(S[ib][j][r], esc[j]);
  }
  // the copies of the last iteration (a reload of the last chunk) complete before the
  // workgroup's LDS is released
  __builtin_amdgcn_s_waitcnt(0x0F70);
}

// ---------------------------------------------------------------------------
// Associative scan of segment maps ("xhh.club" structure entry: context parallelism by
// an associative prefix scan; the states entering later segments are composed, never
// summed).  A segment map is S -> A S + B, stored [D][2D] as [A | B]; two maps compose
// as (A2, B2) o (A1, B1) = (A2 A1, A2 B1 + B2).
//
// map_chain runs chains of map applications in parallel.  A chain starts from a block
// X of 16 columns (of a state, or of a map [A | B]) and applies its maps in order,
// X <- A_j X (+ B_j's matching columns for state columns and for the B part of a map).
// With n segments the states entering them come from three launches of it (n >= 32:
// 3 (m - 1) dependent steps instead of n - 1, groups of m ~ sqrt(n) segments):
//   1. compose:  the maps of every group but the last, composed in parallel per group
//   2. groups:   S_in at the first segment of every group, one chain over the group maps
//   3. within:   S_in at every other segment, one chain per group from its first state
// and from one launch of the third kind over a single group for smaller n.
//
// One workgroup per (chain, one or two 16-column blocks); the map product runs as fp32
// MFMA.  The workgroups of a chain share an XCD (ids equal modulo 8), so each map is
// fetched from memory once into that XCD's L2.  The next map's rows are loaded while the
// current product runs; each 16x16 result tile accumulates in four independent chains
// over the 128-long contraction.  The contraction index of MFMA k-slot s (lane group
// s = lane / 16) at step q4, element e is 16 q4 + 4 s + e, so the four lanes of a map
// row read 64 contiguous bytes per load.
// ---------------------------------------------------------------------------
template <int NB>
struct MapRows {
  float4 a[2][8];     // A rows (2 tiles), contraction 16 q4 + 4 lg + (0..3)
  float b[NB][2][4];  // B at rows 4lg + r of each tile, this lane's column of each block
};

struct ChainArgs {
  const float *maps;            // [D][2D] maps: step j of chain (bh, g) reads the map at
                                // maps + bh * map_bh + g * map_grp + map_off + j * D * 2D
  const float *x0;              // the chain's first block: x0 + bh * x0_bh + g * x0_grp (row
                                // stride x0_ld), or null for zeros
  float *out;                   // the block after step j at out + bh * out_bh + g * out_grp +
                                // (j + 1) * out_step (row stride out_ld); with store_all = 0
                                // only the last step's block, at out + bh * out_bh + g * out_grp
  int64_t map_bh, map_grp, map_off, x0_bh, x0_grp, out_bh, out_grp, out_step;
  int x0_ld, out_ld;
  int n_bh, n_grp;              // chains: n_bh x n_grp
  int grp_len, n_total;         // chain g applies min(grp_len, n_total - g grp_len) - 1 maps
  int ncb;                      // column blocks per chain: 8 (a state) or 16 (a map, A then B)
  int store_x0, store_all;      // store the first block too (at the chain's output base)
};

// NB: 16-column blocks per workgroup (the A rows a wave loads serve all of them)
// (no __restrict__ on the maps: with it the compiler sinks the prefetch loads of the
// next map to their uses, exposing their latency at every step)
template <int NB>
__global__ __launch_bounds__(NTHREADS, 1) void map_chain(ChainArgs a) {
  constexpr int NCOL = 16 * NB;
  __shared__ __align__(16) float sXt[2][NCOL][D + 4];   // the block, transposed [n][i], double buffered
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int lr = lane & 15, lg = lane >> 4;
  const int xcd = blockIdx.x & 7, rest = blockIdx.x >> 3;
  const int nwg = a.ncb / NB;                          // workgroups per chain
  const int cb = (rest % nwg) * NB, chain = (rest / nwg) * 8 + xcd;
  if (chain >= a.n_bh * a.n_grp) return;
  const int bh = chain / a.n_grp, g = chain % a.n_grp;
  const int steps = min(a.grp_len, a.n_total - g * a.grp_len) - 1;
  const int c0 = cb * 16;
  const bool add_b = a.ncb == 8 || cb >= 8;            // state columns, or the B part of a map
  const int bcol = D + (cb & 7) * 16;
  const float *map0 = a.maps + bh * a.map_bh + g * a.map_grp + a.map_off;
  const float *x0 = a.x0 ? a.x0 + bh * a.x0_bh + g * a.x0_grp + c0 : nullptr;
  float *out0 = a.out + bh * a.out_bh + g * a.out_grp + c0;
  // wave w computes rows 32w .. 32w + 31 (two 16-row tiles)
  auto load_map = [&](MapRows<NB> &m, int j) __attribute__((always_inline)) {
    const float *A = map0 + (size_t)j * D * (2 * D);
#pragma unroll
    for (int it = 0; it < 2; ++it) {
      const int row0 = (2 * wave + it) * 16;
      const float *arow = A + (size_t)(row0 + lr) * (2 * D) + 4 * lg;
#pragma unroll
      for (int q4 = 0; q4 < 8; ++q4) m.a[it][q4] = *reinterpret_cast<const float4 *>(arow + 16 * q4);
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          m.b[nb][it][r] = add_b ? A[(size_t)(row0 + 4 * lg + r) * (2 * D) + bcol + 16 * nb + lr] : 0.f;
    }
  };
  // Two map buffers in fixed roles per half of the unrolled loop (no register copies
  // between them), so that the waits for one map's rows do not cover the loads of the
  // next one.
  MapRows<NB> m0, m1;
  if (steps > 0) load_map(m0, 0);                      // in flight while the first block loads
  // all loads of the first block before any store: written as one loop, the compiler
  // waited for each load before the next (x0 and out may alias as far as it knows)
  constexpr int XPT = NCOL * D / NTHREADS;
  float xv[XPT];
#pragma unroll
  for (int u = 0; u < XPT; ++u) {
    const int x = tid + u * NTHREADS, i = x / NCOL, n = x % NCOL;
    xv[u] = x0 ? x0[(size_t)i * a.x0_ld + n] : 0.f;
  }
#pragma unroll
  for (int u = 0; u < XPT; ++u) {
    const int x = tid + u * NTHREADS, i = x / NCOL, n = x % NCOL;
    sXt[0][n][i] = xv[u];
    if (a.store_x0) out0[(size_t)i * a.out_ld + n] = xv[u];
  }
  if (steps <= 0) return;                              // the whole workgroup leaves
  __syncthreads();
  auto step = [&](MapRows<NB> &cur, MapRows<NB> &nxt, int j) __attribute__((always_inline)) {
    // unconditional (the last step reloads the last map), so that the compiler's waits
    // for cur count exactly the loads issued after it
    load_map(nxt, min(j + 1, steps - 1));
    asm volatile("" ::: "memory");                     // keeps those loads ahead of the products
    f32x4 res[NB][2];
#pragma unroll
    for (int it = 0; it < 2; ++it) {
      f32x4 c[NB][4];
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) c[nb][0] = c[nb][1] = c[nb][2] = c[nb][3] = zero4();
#pragma unroll
      for (int q4 = 0; q4 < 8; ++q4) {
        const float4 av = cur.a[it][q4];
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
          const float4 bv = *reinterpret_cast<const float4 *>(&sXt[j & 1][16 * nb + lr][16 * q4 + 4 * lg]);
          c[nb][0] = __builtin_amdgcn_mfma_f32_16x16x4f32(av.x, bv.x, c[nb][0], 0, 0, 0);
          c[nb][1] = __builtin_amdgcn_mfma_f32_16x16x4f32(av.y, bv.y, c[nb][1], 0, 0, 0);
          c[nb][2] = __builtin_amdgcn_mfma_f32_16x16x4f32(av.z, bv.z, c[nb][2], 0, 0, 0);
          c[nb][3] = __builtin_amdgcn_mfma_f32_16x16x4f32(av.w, bv.w, c[nb][3], 0, 0, 0);
        }
      }
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          res[nb][it][r] = ((c[nb][0][r] + c[nb][1][r]) + (c[nb][2][r] + c[nb][3][r])) + cur.b[nb][it][r];
    }
    const bool st = a.store_all || j == steps - 1;
    float *dst = out0 + (a.store_all ? (j + 1) * a.out_step : 0);
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int it = 0; it < 2; ++it)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int i = (2 * wave + it) * 16 + 4 * lg + r;
          sXt[(j + 1) & 1][16 * nb + lr][i] = res[nb][it][r];   // the other buffer: no wait for readers of this one
          if (st) dst[(size_t)i * a.out_ld + 16 * nb + lr] = res[nb][it][r];
        }
    // the new block visible to all waves; a barrier without a memory fence, so that the
    // global stores of the block are not waited for
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(0xC07F);                // lgkmcnt(0)
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
  };
  for (int j = 0; j < steps; j += 2) {
    step(m0, m1, j);
    if (j + 1 < steps) step(m1, m0, j + 1);
  }
}

// Two column blocks per workgroup halve the map rows read per step (the A rows serve
// both), at one workgroup per CU; worth it while that still gives every CU a workgroup.
hipError_t launch_chain(const ChainArgs &a, hipStream_t s) {
  const int64_t chains = (int64_t)a.n_bh * a.n_grp;
  const int64_t slots = (chains + 7) / 8 * 8;
  if (slots * (a.ncb / 2) >= 256) {
    hipLaunchKernelGGL(map_chain<2>, dim3(static_cast<unsigned>(slots * (a.ncb / 2))), dim3(NTHREADS), 0, s, a);
  } else {
    hipLaunchKernelGGL(map_chain<1>, dim3(static_cast<unsigned>(slots * a.ncb)), dim3(NTHREADS), 0, s, a);
  }
  return hipGetLastError();
}

// The states entering every segment: sin[bh][s] for s < n_seg, from the maps of
// segments 0..n_seg-2 and S0 (null: zeros).  gmaps: workspace for the group maps when
// grp_len < n_seg, [n_bh][n_seg / grp_len rounded up - 1][D][2D].
hipError_t segment_scan(const float *maps, const float *S0, float *sin, float *gmaps, int n_seg,
                        int grp_len, int n_bh, hipStream_t s) {
  const int64_t DD = (int64_t)D * D, D2D = (int64_t)D * 2 * D;
  const int G = (n_seg + grp_len - 1) / grp_len;
  ChainArgs w{};                                       // within groups (or the only chain)
  w.maps = maps; w.map_bh = n_seg * D2D; w.map_grp = grp_len * D2D; w.map_off = 0;
  w.out = sin; w.out_bh = n_seg * DD; w.out_grp = grp_len * DD; w.out_step = DD;
  w.out_ld = D; w.x0_ld = D;
  w.n_bh = n_bh; w.n_grp = G; w.grp_len = grp_len; w.n_total = n_seg;
  w.ncb = D / 16; w.store_all = 1;
  if (G == 1) {
    w.x0 = S0; w.x0_bh = DD; w.store_x0 = 1;
    return launch_chain(w, s);
  }
  ChainArgs c{};                                       // compose the maps of groups 0..G-2
  c.maps = maps; c.map_bh = n_seg * D2D; c.map_grp = grp_len * D2D; c.map_off = D2D;
  c.x0 = maps; c.x0_bh = n_seg * D2D; c.x0_grp = grp_len * D2D; c.x0_ld = 2 * D;
  c.out = gmaps; c.out_bh = (G - 1) * D2D; c.out_grp = D2D; c.out_ld = 2 * D;
  c.n_bh = n_bh; c.n_grp = G - 1; c.grp_len = grp_len; c.n_total = (G - 1) * grp_len;
  c.ncb = 2 * D / 16; c.store_x0 = 0; c.store_all = 0;
  hipError_t e = launch_chain(c, s);
  if (e != hipSuccess) return e;
  ChainArgs q{};                                       // states entering the groups
  q.maps = gmaps; q.map_bh = (G - 1) * D2D;
  q.x0 = S0; q.x0_bh = DD; q.x0_ld = D;
  q.out = sin; q.out_bh = n_seg * DD; q.out_step = grp_len * DD; q.out_ld = D;
  q.n_bh = n_bh; q.n_grp = 1; q.grp_len = G; q.n_total = G;
  q.ncb = D / 16; q.store_x0 = 1; q.store_all = 1;
  e = launch_chain(q, s);
  if (e != hipSuccess) return e;
  w.x0 = sin; w.x0_bh = n_seg * DD; w.x0_grp = grp_len * DD; w.store_x0 = 0;
  return launch_chain(w, s);
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
template <int C, int NC, bool F32, int MODE, bool GATE>
hipError_t launch_one(const StateArgs &a, hipStream_t s) {
  constexpr int VS = (MODE == MODE_TRANSITION ? 2 * D : D) / NC;
  const int groups = (a.n_units + 7) / 8;
  const unsigned grid = static_cast<unsigned>(groups) * 8u * VS;
  hipLaunchKernelGGL((chunk_state_kernel<C, NC, F32, MODE, GATE>), dim3(grid), dim3(Shape<NC, MODE>::NTH), 0, s, a);
  return hipGetLastError();
}

template <int C, bool F32, int MODE>
hipError_t launch_nc(const StateArgs &a, int nc, hipStream_t s) {
  // a state map [A | B] (2D columns) is one workgroup of 8 waves x 32 columns
  if constexpr (MODE == MODE_TRANSITION) {
    (void)nc;
    return launch_one<C, 2 * D, F32, MODE, false>(a, s);
  } else {
    if (nc == 128) {
      if (a.fused_gate) return launch_one<C, 128, F32, MODE, true>(a, s);
      return launch_one<C, 128, F32, MODE, false>(a, s);
    }
    if (nc == 64) return launch_one<C, 64, F32, MODE, false>(a, s);
    return hipErrorInvalidValue;
  }
}

template <int MODE>
hipError_t launch_mode(const StateArgs &a, int chunk, bool f32, int nc, hipStream_t s) {
  if (f32) return launch_nc<16, true, MODE>(a, nc, s);
  if (chunk == 16) return launch_nc<16, false, MODE>(a, nc, s);
  return launch_nc<64, false, MODE>(a, nc, s);
}

}  // namespace

hipError_t launch_prefill(const kda_prefill_desc &d, const PrefillPlan &p, hipStream_t s) {
  const bool f32 = d.in_dtype == KDA_F32;
  const int64_t units = (int64_t)d.B * d.H;

  if (d.T == 0) {
    // no tokens: the final state is the initial state
    if (d.S_final && d.S_final != d.S0) {
      if (d.S0) return launch_state_copy(d.S_final, d.S0, units * d.d_k * d.d_v, s);
      return launch_fill_zero(d.S_final, units * d.d_k * d.d_v, s);
    }
    return hipSuccess;
  }

  unsigned char *ws = static_cast<unsigned char *>(d.workspace);
  unsigned char *rec = ws + p.off_rec;
  float *maps = p.ws_maps ? reinterpret_cast<float *>(ws + p.off_maps) : nullptr;
  float *sin = p.ws_sin ? reinterpret_cast<float *>(ws + p.off_sin) : nullptr;

  // pass 0: per-chunk records, all chunks in parallel
  hipError_t e = launch_prefill_prep(d, p.n_chunks, rec, s);
  if (e != hipSuccess) return e;

  StateArgs a{};
  a.v = d.v; a.gate = d.gate;
  a.S0 = d.S0; a.norm_weight = d.norm_weight;
  a.rec = rec;
  a.S_final = d.S_final; a.ckpt = d.ckpt; a.o = d.o;
  a.maps = maps; a.sin = sin; a.eps = d.norm_eps;
  a.T = d.T; a.H = d.H;
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
    raw = d.out_dtype == KDA_F32 ? static_cast<float *>(d.o) : reinterpret_cast<float *>(ws + p.off_norm);
    a.o = raw;
  }

  if (p.n_seg > 1) {
    // pass 1: maps of all segments but the last
    StateArgs t = a;
    t.fused_gate = 0;
    e = launch_mode<MODE_TRANSITION>(t, d.chunk, f32, 2 * D, s);
    if (e != hipSuccess) return e;
    // pass 2: states entering each segment
    float *gmaps = p.ws_gmaps ? reinterpret_cast<float *>(ws + p.off_gmaps) : nullptr;
    e = segment_scan(maps, d.S0, sin, gmaps, p.n_seg, p.scan_grp, static_cast<int>(units), s);
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
