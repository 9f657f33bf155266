// C ABI of the KDA library: argument validation, execution planning, dispatch.
// Validation is synchronous and launches nothing on error; every launch is
// asynchronous on the caller's stream.  No exception crosses the boundary.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cstring>

#include "internal.h"
#include "kda.h"

namespace {

using kda::PrefillPlan;

// ---------------------------------------------------------------------------
// device check: gfx950 only, cached per device ordinal
// ---------------------------------------------------------------------------
constexpr int kMaxDevices = 64;
std::atomic<int> g_dev_state[kMaxDevices];  // 0 unknown, 1 gfx950, 2 other

kda_status check_device() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return KDA_ERR_DEVICE;
  if (dev >= kMaxDevices) return KDA_ERR_DEVICE;
  int st = g_dev_state[dev].load(std::memory_order_acquire);
  if (st == 0) {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return KDA_ERR_DEVICE;
    st = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : 2;
    g_dev_state[dev].store(st, std::memory_order_release);
  }
  return st == 1 ? KDA_OK : KDA_ERR_DEVICE;
}

// [p, p + n) and [q, q + m) overlap (empty ranges never overlap).
bool overlap(const void *p, size_t n, const void *q, size_t m) {
  if (!p || !q || n == 0 || m == 0) return false;
  const uintptr_t a = reinterpret_cast<uintptr_t>(p), b = reinterpret_cast<uintptr_t>(q);
  return a < b + m && b < a + n;
}

size_t esize(int32_t dt) { return dt == KDA_BF16 ? 2 : 4; }

bool valid_dtype(int32_t dt) { return dt == KDA_F32 || dt == KDA_BF16; }

// ---------------------------------------------------------------------------
// prefill planning
// ---------------------------------------------------------------------------

kda_status plan_prefill(const kda_prefill_desc &d, PrefillPlan *p) {
  std::memset(p, 0, sizeof(*p));
  const int64_t n_chunks = d.T > 0 ? (static_cast<int64_t>(d.T) + d.chunk - 1) / d.chunk : 0;
  const int64_t units = static_cast<int64_t>(d.B) * d.H;
  p->n_chunks = static_cast<int>(n_chunks);

  // columns per workgroup: whole heads unless the caller asks for a split (a split
  // head re-reads every chunk record once per workgroup and needs a separate norm
  // pass); parallelism beyond the (sequence, head) units comes from segments
  const int vs = d.v_split != 0 ? d.v_split : 1;
  p->v_split = vs;

  // segments: context parallelism until the chip is covered, keeping >= 8 chunks each
  int64_t ns = d.n_segments;
  if (ns > 1 && ns > n_chunks) return KDA_ERR_SHAPE;
  if (ns == 0) {
    ns = 1;
    while (units * vs * ns < kda::kCUs && n_chunks / (ns * 2) >= 8) ns *= 2;
  }
  if (ns < 1) ns = 1;
  int64_t seg_chunks = n_chunks > 0 ? (n_chunks + ns - 1) / ns : 0;
  if (seg_chunks > 0) ns = (n_chunks + seg_chunks - 1) / seg_chunks;  // no empty segments
  p->n_seg = static_cast<int>(ns);
  p->seg_chunks = static_cast<int>(seg_chunks);
  p->split_norm = d.gate != nullptr && vs > 1;

  const size_t dkdv = static_cast<size_t>(d.d_k) * d.d_v;
  p->ws_rec = static_cast<size_t>(units) * static_cast<size_t>(n_chunks) *
              kda::prefill_record_bytes(d.chunk, d.in_dtype == KDA_F32);
  p->scan_grp = p->n_seg;
  if (p->n_seg > 1) {
    p->ws_maps = static_cast<size_t>(units) * p->n_seg * dkdv * 2 * sizeof(float);
    p->ws_sin = static_cast<size_t>(units) * p->n_seg * dkdv * sizeof(float);
    // from 32 segments on, the scan runs in groups of about sqrt(n_seg) segments:
    // 3 (m - 1) dependent map applications instead of n_seg - 1
    if (p->n_seg >= 32) {
      int m = 1;
      while (m * m < p->n_seg) ++m;
      const int groups = (p->n_seg + m - 1) / m;
      p->scan_grp = m;
      p->ws_gmaps = static_cast<size_t>(units) * (groups - 1) * dkdv * 2 * sizeof(float);
    }
  }
  if (p->split_norm && d.out_dtype == KDA_BF16)
    p->ws_norm = static_cast<size_t>(units) * static_cast<size_t>(d.T) * d.d_v * sizeof(float);
  auto up = [](size_t x) { return (x + 255) & ~static_cast<size_t>(255); };
  p->off_rec = 0;
  p->off_maps = p->off_rec + up(p->ws_rec);
  p->off_sin = p->off_maps + up(p->ws_maps);
  p->off_gmaps = p->off_sin + up(p->ws_sin);
  p->off_norm = p->off_gmaps + up(p->ws_gmaps);
  p->ws_total = p->off_norm + up(p->ws_norm);
  return KDA_OK;
}

kda_status validate_sizes(const kda_prefill_desc *d) {
  if (!d) return KDA_ERR_NULL;
  if (d->B < 0 || d->T < 0 || d->H < 0) return KDA_ERR_SHAPE;
  if (d->d_k != 128 || d->d_v != 128) return KDA_ERR_UNSUPPORTED;
  if (d->chunk != 16 && d->chunk != 64) return KDA_ERR_UNSUPPORTED;
  if (!valid_dtype(d->in_dtype) || !valid_dtype(d->out_dtype)) return KDA_ERR_UNSUPPORTED;
  if (d->in_dtype == KDA_F32 && d->chunk != 16) return KDA_ERR_UNSUPPORTED;
  if (d->v_split != 0 && d->v_split != 1 && d->v_split != 2)
    return KDA_ERR_UNSUPPORTED;
  if (d->n_segments < 0) return KDA_ERR_SHAPE;
  if (d->ckpt_every < 0 || (d->ckpt_every > 0 && d->ckpt_every % d->chunk != 0)) return KDA_ERR_SHAPE;
  // one prep workgroup per (sequence, head, chunk): the grid is 32-bit
  const int64_t n_chunks = (static_cast<int64_t>(d->T) + d->chunk - 1) / d->chunk;
  if (static_cast<int64_t>(d->B) * d->H * n_chunks >= (int64_t(1) << 31)) return KDA_ERR_SHAPE;
  return KDA_OK;
}

kda_status validate_prefill(const kda_prefill_desc *d, PrefillPlan *p) {
  kda_status st0 = validate_sizes(d);
  if (st0 != KDA_OK) return st0;
  const size_t ntok = static_cast<size_t>(d->B) * d->T * d->H;
  const size_t nstate = static_cast<size_t>(d->B) * d->H;
  const int64_t n_ckpt = d->ckpt_every > 0 ? d->T / d->ckpt_every : 0;
  if (ntok > 0 && (!d->q || !d->k || !d->v || !d->g || !d->beta || !d->o)) return KDA_ERR_NULL;
  if (n_ckpt > 0 && nstate > 0 && !d->ckpt) return KDA_ERR_NULL;
  kda_status st = plan_prefill(*d, p);
  if (st != KDA_OK) return st;

  // aliasing
  const size_t ie = esize(d->in_dtype), oe = esize(d->out_dtype);
  const size_t dk = d->d_k, dv = d->d_v, sbytes = nstate * dk * dv * 4;
  const size_t o_bytes = ntok * dv * oe;
  const size_t ck_bytes = static_cast<size_t>(n_ckpt) * sbytes;
  struct R { const void *p; size_t n; } in[] = {
      {d->q, ntok * dk * ie}, {d->k, ntok * dk * ie}, {d->v, ntok * dv * ie},
      {d->g, ntok * dk * 4},  {d->beta, ntok * 4},    {d->gate, d->gate ? ntok * dv * ie : 0},
      {d->S0, d->S0 ? sbytes : 0}, {d->norm_weight, d->norm_weight ? dv * 4 : 0}};
  for (const R &r : in)
    if (overlap(d->o, o_bytes, r.p, r.n)) return KDA_ERR_ALIAS;
  if (overlap(d->o, o_bytes, d->S_final, d->S_final ? sbytes : 0)) return KDA_ERR_ALIAS;
  if (overlap(d->o, o_bytes, d->ckpt, ck_bytes)) return KDA_ERR_ALIAS;
  if (d->S_final) {
    for (int i = 0; i < 8; ++i)
      if (i != 6 && overlap(d->S_final, sbytes, in[i].p, in[i].n)) return KDA_ERR_ALIAS;
    if (d->S0 && d->S_final != d->S0 && overlap(d->S_final, sbytes, d->S0, sbytes)) return KDA_ERR_ALIAS;
    if (overlap(d->S_final, sbytes, d->ckpt, ck_bytes)) return KDA_ERR_ALIAS;
  }
  if (d->ckpt) {
    for (const R &r : in)
      if (overlap(d->ckpt, ck_bytes, r.p, r.n)) return KDA_ERR_ALIAS;
  }
  if (p->ws_total > 0) {
    if (!d->workspace || d->workspace_bytes < p->ws_total) return KDA_ERR_WORKSPACE;
    for (const R &r : in)
      if (overlap(d->workspace, p->ws_total, r.p, r.n)) return KDA_ERR_ALIAS;
    if (overlap(d->workspace, p->ws_total, d->o, o_bytes) ||
        overlap(d->workspace, p->ws_total, d->S_final, d->S_final ? sbytes : 0) ||
        overlap(d->workspace, p->ws_total, d->ckpt, ck_bytes))
      return KDA_ERR_ALIAS;
  }
  return KDA_OK;
}

// n_state: states in d->state (N for the plain form, the pool size for the pooled one)
kda_status validate_decode(const kda_decode_desc *d, int64_t n_state) {
  if (!d) return KDA_ERR_NULL;
  if (d->N < 0 || d->H < 0 || n_state < 0) return KDA_ERR_SHAPE;
  if (static_cast<int64_t>(d->N) * d->H >= (int64_t(1) << 31)) return KDA_ERR_SHAPE;   // one workgroup per state
  if (d->d_k != 128 || d->d_v != 128) return KDA_ERR_UNSUPPORTED;
  if (!valid_dtype(d->in_dtype) || !valid_dtype(d->out_dtype)) return KDA_ERR_UNSUPPORTED;
  const size_t n = static_cast<size_t>(d->N) * d->H;
  if (n == 0) return KDA_OK;
  if (!d->q || !d->k || !d->v || !d->g || !d->beta || !d->state || !d->o) return KDA_ERR_NULL;
  const size_t ie = esize(d->in_dtype), oe = esize(d->out_dtype);
  const size_t dk = d->d_k, dv = d->d_v;
  const size_t o_bytes = n * dv * oe;
  const size_t s_bytes = static_cast<size_t>(n_state) * d->H * dk * dv * 4;
  struct R { const void *p; size_t n; } in[] = {
      {d->q, n * dk * ie}, {d->k, n * dk * ie}, {d->v, n * dv * ie}, {d->g, n * dk * 4},
      {d->beta, n * 4},    {d->gate, d->gate ? n * dv * ie : 0},
      {d->norm_weight, d->norm_weight ? dv * 4 : 0}, {d->state, s_bytes}};
  for (const R &r : in)
    if (overlap(d->o, o_bytes, r.p, r.n)) return KDA_ERR_ALIAS;
  for (int i = 0; i < 7; ++i)
    if (overlap(d->state, s_bytes, in[i].p, in[i].n)) return KDA_ERR_ALIAS;
  return KDA_OK;
}

kda_status validate_copy(const float *a, const float *b, int64_t n_states, int32_t dk, int32_t dv) {
  if (n_states < 0 || dk < 1 || dv < 1) return KDA_ERR_SHAPE;
  if (n_states == 0) return KDA_OK;
  if (!a || !b) return KDA_ERR_NULL;
  const size_t bytes = static_cast<size_t>(n_states) * dk * dv * 4;
  if (overlap(a, bytes, b, bytes)) return KDA_ERR_ALIAS;
  return KDA_OK;
}

kda_status validate_copy_indexed(const float *dst, int64_t dst_count, const int32_t *dst_slots,
                                 const float *src, int64_t src_count, const int32_t *src_slots,
                                 int64_t n, int64_t elems) {
  if (n < 0 || dst_count < 0 || src_count < 0 || elems < 0) return KDA_ERR_SHAPE;
  if ((!dst_slots && n > dst_count) || (!src_slots && n > src_count)) return KDA_ERR_SHAPE;
  if (n == 0 || elems == 0) return KDA_OK;
  if (!dst || !src) return KDA_ERR_NULL;
  const int64_t pieces = (elems + 1023) / 1024;            // workgroups per state (grid size)
  if (pieces > (int64_t(1) << 31) / n) return KDA_ERR_SHAPE;
  return KDA_OK;
}

kda_status validate_backward_sizes(const kda_backward_desc *d) {
  if (!d) return KDA_ERR_NULL;
  if (d->B < 0 || d->T < 0 || d->H < 0) return KDA_ERR_SHAPE;
  if (d->d_k != 128 || d->d_v != 128 || d->chunk != 64) return KDA_ERR_UNSUPPORTED;
  if (!valid_dtype(d->in_dtype)) return KDA_ERR_UNSUPPORTED;
  const int64_t n_chunks = (static_cast<int64_t>(d->T) + 63) / 64;
  if (static_cast<int64_t>(d->B) * d->H * n_chunks >= (int64_t(1) << 31)) return KDA_ERR_SHAPE;
  return KDA_OK;
}

kda_status validate_backward(const kda_backward_desc *d, size_t *ws) {
  kda_status st = validate_backward_sizes(d);
  if (st != KDA_OK) return st;
  const size_t ntok = static_cast<size_t>(d->B) * d->T * d->H;
  const size_t nstate = static_cast<size_t>(d->B) * d->H;
  if (ntok > 0 && (!d->q || !d->k || !d->v || !d->g || !d->beta || !d->dO || !d->dq || !d->dk ||
                   !d->dv || !d->dg || !d->dbeta))
    return KDA_ERR_NULL;
  *ws = kda::backward_workspace_bytes(d->B, d->T, d->H);
  if (*ws > 0 && (!d->workspace || d->workspace_bytes < *ws)) return KDA_ERR_WORKSPACE;
  const size_t ie = esize(d->in_dtype), sb = nstate * 128 * 128 * 4, tb = ntok * 128 * 4;
  struct R { const void *p; size_t n; };
  const R in[] = {{d->q, ntok * 128 * ie}, {d->k, ntok * 128 * ie}, {d->v, ntok * 128 * ie},
                  {d->g, tb}, {d->beta, ntok * 4}, {d->S0, d->S0 ? sb : 0}, {d->dO, tb},
                  {d->dS_final, d->dS_final ? sb : 0}};
  const R out[] = {{d->dq, tb}, {d->dk, tb}, {d->dv, tb}, {d->dg, tb}, {d->dbeta, ntok * 4},
                   {d->dS0, d->dS0 ? sb : 0}, {d->workspace, *ws}};
  for (size_t i = 0; i < sizeof(out) / sizeof(out[0]); ++i) {
    for (const R &r : in)
      if (overlap(out[i].p, out[i].n, r.p, r.n)) return KDA_ERR_ALIAS;
    for (size_t j = 0; j < i; ++j)
      if (overlap(out[i].p, out[i].n, out[j].p, out[j].n)) return KDA_ERR_ALIAS;
  }
  return KDA_OK;
}

kda_status from_hip(hipError_t e) { return e == hipSuccess ? KDA_OK : KDA_ERR_HIP; }

// ---------------------------------------------------------------------------
// the prefill's workspace for callers that cannot allocate: one array in device memory
// per GPU, reserved when the library is loaded and held until the process ends
// ---------------------------------------------------------------------------
static __device__ __align__(256) unsigned char scratch[KDA_NOALLOC_WORKSPACE_BYTES];

// Device address of `scratch` on each device, looked up once per device with that
// device current.  In host code `scratch` names a host-side stand-in, never the device
// memory: only these addresses are passed to kernels.
std::atomic<void *> g_scratch[kMaxDevices];
std::atomic<int> g_scratch_state[kMaxDevices];   // 0 not looked up, 1 ok, 2 failed

kda_status scratch_of_current_device(void **ptr) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return KDA_ERR_DEVICE;
  int st = g_scratch_state[dev].load(std::memory_order_acquire);
  if (st == 0) {
    void *p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e == hipSuccess && p) g_scratch[dev].store(p, std::memory_order_release);
    st = e == hipSuccess && p ? 1 : 2;
    // concurrent first calls look up the same address; either store is correct
    g_scratch_state[dev].store(st, std::memory_order_release);
  }
  if (st != 1) return KDA_ERR_HIP;
  *ptr = g_scratch[dev].load(std::memory_order_acquire);
  return KDA_OK;
}

}  // namespace

extern "C" {

kda_status kda_prefill_workspace_size(const kda_prefill_desc *d, size_t *bytes) {
  if (!bytes) return KDA_ERR_NULL;
  kda_status st = validate_sizes(d);
  if (st != KDA_OK) return st;
  PrefillPlan p;
  st = plan_prefill(*d, &p);
  if (st != KDA_OK) return st;
  *bytes = p.ws_total;
  return KDA_OK;
}

kda_status kda_prefill_chunked(const kda_prefill_desc *d, hipStream_t stream) {
  PrefillPlan p;
  kda_status st = validate_prefill(d, &p);
  if (st != KDA_OK) return st;
  if (static_cast<int64_t>(d->B) * d->H == 0) return KDA_OK;
  st = check_device();
  if (st != KDA_OK) return st;
  return from_hip(kda::launch_prefill(*d, p, stream));
}

kda_status kda_prefill_chunked_noalloc(const kda_prefill_desc *d, hipStream_t stream) {
  kda_status st = validate_sizes(d);
  if (st != KDA_OK) return st;
  PrefillPlan p;
  st = plan_prefill(*d, &p);
  if (st != KDA_OK) return st;
  if (p.ws_total > static_cast<size_t>(KDA_NOALLOC_WORKSPACE_BYTES)) return KDA_ERR_WORKSPACE;
  if (static_cast<int64_t>(d->B) * d->H == 0) return validate_prefill(d, &p);
  st = check_device();
  if (st != KDA_OK) return st;
  void *ws = nullptr;
  st = scratch_of_current_device(&ws);
  if (st != KDA_OK) return st;
  kda_prefill_desc dd = *d;                  // the caller's workspace fields are ignored
  dd.workspace = ws;
  dd.workspace_bytes = KDA_NOALLOC_WORKSPACE_BYTES;
  st = validate_prefill(&dd, &p);
  if (st != KDA_OK) return st;
  return from_hip(kda::launch_prefill(dd, p, stream));
}

kda_status kda_decode_step(const kda_decode_desc *d, hipStream_t stream) {
  kda_status st = validate_decode(d, d ? d->N : 0);
  if (st != KDA_OK) return st;
  if (static_cast<int64_t>(d->N) * d->H == 0) return KDA_OK;
  st = check_device();
  if (st != KDA_OK) return st;
  return from_hip(kda::launch_decode(*d, nullptr, 0, stream));
}

kda_status kda_decode_step_pooled(const kda_decode_desc *d, const int32_t *slots, int32_t pool_size,
                                  hipStream_t stream) {
  kda_status st = validate_decode(d, pool_size);
  if (st != KDA_OK) return st;
  if (static_cast<int64_t>(d->N) * d->H == 0) return KDA_OK;
  if (!slots) return KDA_ERR_NULL;
  st = check_device();
  if (st != KDA_OK) return st;
  return from_hip(kda::launch_decode(*d, slots, pool_size, stream));
}

kda_status kda_state_copy_indexed(float *dst, const int32_t *dst_slots, int64_t dst_count,
                                  const float *src, const int32_t *src_slots, int64_t src_count,
                                  int64_t n, int64_t state_elems, hipStream_t stream) {
  kda_status st = validate_copy_indexed(dst, dst_count, dst_slots, src, src_count, src_slots, n, state_elems);
  if (st != KDA_OK || n == 0 || state_elems == 0) return st;
  st = check_device();
  if (st != KDA_OK) return st;
  return from_hip(kda::launch_state_copy_indexed(dst, dst_slots, dst_count, src, src_slots, src_count, n,
                                                  state_elems, stream));
}

kda_status kda_state_checkpoint(const float *state, float *ckpt, int64_t n_states, int32_t d_k,
                                int32_t d_v, hipStream_t stream) {
  kda_status st = validate_copy(state, ckpt, n_states, d_k, d_v);
  if (st != KDA_OK || n_states == 0) return st;
  st = check_device();
  if (st != KDA_OK) return st;
  return from_hip(kda::launch_state_copy(ckpt, state, n_states * d_k * d_v, stream));
}

kda_status kda_state_rollback(float *state, const float *ckpt, int64_t n_states, int32_t d_k,
                              int32_t d_v, hipStream_t stream) {
  kda_status st = validate_copy(state, ckpt, n_states, d_k, d_v);
  if (st != KDA_OK || n_states == 0) return st;
  st = check_device();
  if (st != KDA_OK) return st;
  return from_hip(kda::launch_state_copy(state, ckpt, n_states * d_k * d_v, stream));
}

kda_status kda_backward_workspace_size(const kda_backward_desc *d, size_t *bytes) {
  if (!bytes) return KDA_ERR_NULL;
  kda_status st = validate_backward_sizes(d);
  if (st != KDA_OK) return st;
  *bytes = kda::backward_workspace_bytes(d->B, d->T, d->H);
  return KDA_OK;
}

kda_status kda_prefill_backward(const kda_backward_desc *d, hipStream_t stream) {
  size_t ws = 0;
  kda_status st = validate_backward(d, &ws);
  if (st != KDA_OK) return st;
  if (static_cast<int64_t>(d->B) * d->H == 0) return KDA_OK;
  st = check_device();
  if (st != KDA_OK) return st;
  return from_hip(kda::launch_backward(*d, stream));
}

const char *kda_status_string(kda_status s) {
  switch (s) {
    case KDA_OK: return "ok";
    case KDA_ERR_NULL: return "a required pointer is NULL";
    case KDA_ERR_SHAPE: return "invalid or inconsistent sizes";
    case KDA_ERR_UNSUPPORTED: return "unsupported configuration (d_k/d_v must be 128; chunk 16 or 64, 64 for the backward; dtype f32 or bf16)";
    case KDA_ERR_WORKSPACE: return "workspace missing or too small";
    case KDA_ERR_ALIAS: return "an output buffer overlaps a buffer it must not overlap";
    case KDA_ERR_DEVICE: return "current HIP device is not gfx950 (MI355X) or cannot be queried";
    case KDA_ERR_HIP: return "HIP kernel launch failed";
  }
  return "unknown status";
}

int32_t kda_abi_version(void) { return KDA_ABI_VERSION; }

}  // extern "C"
