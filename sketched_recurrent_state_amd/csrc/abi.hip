// abi.hip -- the extern "C" entry points of libsketchssm.so: argument checks
// on the host, then one asynchronous launch on the caller's stream. Nothing
// here allocates, frees or synchronises. See include/sketchssm.h.
#include <stdarg.h>
#include <stdint.h>
#include <stdio.h>

#include <string>

#include "launch.hpp"
#include "sketchssm.h"

namespace {

thread_local std::string g_last_error;

constexpr long long kMaxUnits = 1LL << 24;  // keeps every grid below 2^32 threads

ssm_status fail(ssm_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}

ssm_status ok() {
  g_last_error.clear();
  return SSM_OK;
}

bool in_set(int x, std::initializer_list<int> s) {
  for (int v : s)
    if (v == x) return true;
  return false;
}

ssm_status check_dims(const ssm_dims* d, const char* fn) {
  if (d == nullptr) return fail(SSM_E_NULL, "%s: dims is NULL", fn);
  if (d->rule < SSM_MAMBA2 || d->rule > SSM_KDA)
    return fail(SSM_E_RANGE, "%s: rule %d is not 0 (Mamba-2), 1 (GDN) or 2 (KDA)", fn, d->rule);
  if (d->in_dtype != SSM_IN_BF16 && d->in_dtype != SSM_IN_F32)
    return fail(SSM_E_RANGE, "%s: in_dtype %d is not 0 (bf16) or 1 (fp32)", fn, d->in_dtype);
  if (d->sketch_dtype != SSM_SKETCH_F32 && d->sketch_dtype != SSM_SKETCH_BF16)
    return fail(SSM_E_RANGE, "%s: sketch_dtype %d is not 0 (fp32) or 1 (bf16)", fn,
                d->sketch_dtype);
  if (d->batch < 0) return fail(SSM_E_SHAPE, "%s: batch %d < 0", fn, d->batch);
  if (d->heads < 1) return fail(SSM_E_SHAPE, "%s: heads %d < 1", fn, d->heads);
  if (!in_set(d->d_k, {16, 32, 64, 128}))
    return fail(SSM_E_SHAPE, "%s: d_k %d not in {16, 32, 64, 128}", fn, d->d_k);
  if (!in_set(d->d_v, {16, 32, 64, 128}))
    return fail(SSM_E_SHAPE, "%s: d_v %d not in {16, 32, 64, 128}", fn, d->d_v);
  if (d->window < 1 || d->window > 16)
    return fail(SSM_E_SHAPE, "%s: window %d not in [1, 16]", fn, d->window);
  const int rmax = d->d_k < 32 ? d->d_k : 32;
  if (d->rank < 1 || d->rank > rmax)
    return fail(SSM_E_SHAPE, "%s: rank %d not in [1, %d]", fn, d->rank, rmax);
  if ((long long)d->batch * d->heads >= kMaxUnits)
    return fail(SSM_E_SHAPE, "%s: batch*heads = %lld >= %lld", fn,
                (long long)d->batch * d->heads, kMaxUnits);
  return SSM_OK;
}

struct Arr {
  const void* p;
  size_t bytes;
  bool output;
  const char* name;
  unsigned align = 16;
};

ssm_status check_arrays(const char* fn, std::initializer_list<Arr> arrs) {
  for (const Arr& a : arrs) {
    if (a.p != nullptr && (reinterpret_cast<uintptr_t>(a.p) & (a.align - 1)) != 0)
      return fail(SSM_E_ALIGN, "%s: %s (%p) is not %u-byte aligned", fn, a.name, a.p, a.align);
  }
  for (const Arr& a : arrs) {
    if (a.p == nullptr || a.bytes == 0) continue;
    for (const Arr& b : arrs) {
      if (&a == &b || b.p == nullptr || b.bytes == 0) continue;
      if (!a.output && !b.output) continue;
      const uintptr_t a0 = reinterpret_cast<uintptr_t>(a.p), a1 = a0 + a.bytes;
      const uintptr_t b0 = reinterpret_cast<uintptr_t>(b.p), b1 = b0 + b.bytes;
      if (a0 < b1 && b0 < a1)
        return fail(SSM_E_ALIAS, "%s: %s overlaps %s", fn, a.name, b.name);
    }
  }
  return SSM_OK;
}

struct Sizes {
  size_t units, elem, sk_elem, state, sketch, basis, kbuf, vbuf, dbuf, bbuf, qk, v, dtok, btok, y;
};

Sizes sizes_of(const ssm_dims& d) {
  Sizes z;
  z.units = (size_t)d.batch * (size_t)d.heads;
  z.elem = d.in_dtype == SSM_IN_BF16 ? 2 : 4;
  z.sk_elem = d.sketch_dtype == SSM_SKETCH_BF16 ? 2 : 4;
  const size_t dstr = d.rule == SSM_KDA ? (size_t)d.d_k : 1;
  const size_t W = (size_t)d.window;
  z.state = z.units * d.d_k * d.d_v * 4;
  z.sketch = z.units * d.rank * d.d_v * z.sk_elem;
  z.basis = (size_t)d.heads * d.rank * d.d_k * 4;
  z.kbuf = z.units * W * d.d_k * z.elem;
  z.vbuf = z.units * W * d.d_v * z.elem;
  z.dbuf = z.units * W * dstr * 4;
  z.bbuf = z.units * W * 4;
  z.qk = z.units * d.d_k * z.elem;
  z.v = z.units * d.d_v * z.elem;
  z.dtok = z.units * dstr * 4;
  z.btok = z.units * 4;
  z.y = z.units * d.d_v * 4;
  return z;
}

ssm_status check_beta(const ssm_dims& d, const void* beta, const char* what, const char* fn) {
  if (d.rule == SSM_MAMBA2 && beta != nullptr)
    return fail(SSM_E_RANGE, "%s: %s must be NULL for Mamba-2", fn, what);
  if (d.rule != SSM_MAMBA2 && beta == nullptr)
    return fail(SSM_E_NULL, "%s: %s is NULL (required by the delta rules)", fn, what);
  return SSM_OK;
}

// The current-token pointers of a fused append: all present or all absent.
ssm_status check_token(const ssm_dims& d, const void* k_t, const void* v_t, const void* d_t,
                       const void* b_t, const char* fn) {
  if (k_t == nullptr) {
    if (v_t != nullptr || d_t != nullptr || b_t != nullptr)
      return fail(SSM_E_RANGE, "%s: k_t is NULL but v_t/decay_t/beta_t are not", fn);
    return SSM_OK;
  }
  if (v_t == nullptr) return fail(SSM_E_NULL, "%s: v_t is NULL", fn);
  if (d_t == nullptr) return fail(SSM_E_NULL, "%s: decay_t is NULL", fn);
  return check_beta(d, b_t, "beta_t", fn);
}

ssm_status check_buffers(const ssm_dims& d, const void* k_buf, const void* v_buf,
                         const void* decay_buf, const void* beta_buf, const char* fn) {
  if (k_buf == nullptr) return fail(SSM_E_NULL, "%s: k_buf is NULL", fn);
  if (v_buf == nullptr) return fail(SSM_E_NULL, "%s: v_buf is NULL", fn);
  if (decay_buf == nullptr) return fail(SSM_E_NULL, "%s: decay_buf is NULL", fn);
  return check_beta(d, beta_buf, "beta_buf", fn);
}

// Per-head rank table (host array of heads + 1 prefix offsets).
ssm_status check_rank_offsets(const ssm_dims& d, const int32_t* off, const char* fn) {
  if (off == nullptr) return fail(SSM_E_NULL, "%s: rank_offsets is NULL", fn);
  if (d.heads > ssm::kMaxRankedHeads)
    return fail(SSM_E_SHAPE, "%s: %d heads > %d supported with per-head ranks", fn, d.heads,
                ssm::kMaxRankedHeads);
  if (off[0] != 0) return fail(SSM_E_RANGE, "%s: rank_offsets[0] = %d, not 0", fn, off[0]);
  const int rmax = d.d_k < 32 ? d.d_k : 32;
  for (int h = 0; h < d.heads; ++h) {
    const long long r = (long long)off[h + 1] - off[h];
    if (r < 1 || r > rmax)
      return fail(SSM_E_RANGE, "%s: head %d has rank %lld, not in [1, %d]", fn, h, r, rmax);
  }
  return SSM_OK;
}

// Sketch and basis bytes for a per-head rank table (or the uniform rank when off is NULL).
void apply_ranks(const ssm_dims& d, const int32_t* off, Sizes& z) {
  if (off == nullptr) return;
  const size_t R = (size_t)off[d.heads];
  z.sketch = z.units / (size_t)d.heads * R * d.d_v * z.sk_elem;
  z.basis = R * d.d_k * 4;
}

// A variable-length call: `batch` rows mapped onto a pool of num_slots persistent slots.
ssm_status check_pool(const ssm_dims& d, int32_t num_slots, const int32_t* slot,
                      const int32_t* counts, const char* what, const char* fn) {
  if (num_slots < 1) return fail(SSM_E_SHAPE, "%s: num_slots %d < 1", fn, num_slots);
  if ((long long)num_slots * d.heads >= kMaxUnits)
    return fail(SSM_E_SHAPE, "%s: num_slots*heads = %lld >= %lld", fn,
                (long long)num_slots * d.heads, kMaxUnits);
  if (slot == nullptr && d.batch > num_slots)
    return fail(SSM_E_SHAPE, "%s: %d rows but %d slots and no slot map", fn, d.batch, num_slots);
  if (counts == nullptr) return fail(SSM_E_NULL, "%s: %s is NULL", fn, what);
  return SSM_OK;
}

// Sizes of the persistent arrays (state, sketch, window buffer) for a pool of slots.
Sizes pool_sizes(const ssm_dims& d, int32_t num_slots) {
  ssm_dims p = d;
  p.batch = num_slots;
  const Sizes zp = sizes_of(p);
  Sizes z = sizes_of(d);
  z.state = zp.state;
  z.sketch = zp.sketch;
  z.kbuf = zp.kbuf;
  z.vbuf = zp.vbuf;
  z.dbuf = zp.dbuf;
  z.bbuf = zp.bbuf;
  return z;
}

ssm_status launched(hipError_t e, const char* fn) {
  if (e != hipSuccess) return fail(SSM_E_LAUNCH, "%s: launch failed: %s", fn, hipGetErrorString(e));
  return ok();
}

}  // namespace

extern "C" {

int32_t ssm_abi_version(void) { return SSM_ABI_VERSION; }

const char* ssm_status_string(int32_t status) {
  switch (status) {
    case SSM_OK: return "ok";
    case SSM_E_NULL: return "a required pointer is NULL";
    case SSM_E_SHAPE: return "unsupported or inconsistent dimensions";
    case SSM_E_ALIGN: return "a pointer is not 16-byte aligned";
    case SSM_E_RANGE: return "an argument is out of range";
    case SSM_E_ALIAS: return "an output overlaps an input";
    case SSM_E_LAUNCH: return "kernel launch failed";
  }
  return "unknown status";
}

const char* ssm_last_error(void) { return g_last_error.c_str(); }

ssm_status ssm_buffer_append(const ssm_dims* d, const void* k_t, const void* v_t,
                             const float* decay_t, const float* beta_t, void* k_buf, void* v_buf,
                             float* decay_buf, float* beta_buf, int32_t slot, void* stream) {
  static const char* fn = "ssm_buffer_append";
  ssm_status st = check_dims(d, fn);
  if (st != SSM_OK) return st;
  if (slot < 0 || slot >= d->window)
    return fail(SSM_E_RANGE, "%s: slot %d not in [0, %d)", fn, slot, d->window);
  if (d->batch == 0) return ok();
  if (k_t == nullptr) return fail(SSM_E_NULL, "%s: k_t is NULL", fn);
  if ((st = check_token(*d, k_t, v_t, decay_t, beta_t, fn)) != SSM_OK) return st;
  if ((st = check_buffers(*d, k_buf, v_buf, decay_buf, beta_buf, fn)) != SSM_OK) return st;
  const Sizes z = sizes_of(*d);
  st = check_arrays(fn, {{k_t, z.qk, false, "k_t"}, {v_t, z.v, false, "v_t"},
                         {decay_t, z.dtok, false, "decay_t"}, {beta_t, z.btok, false, "beta_t"},
                         {k_buf, z.kbuf, true, "k_buf"}, {v_buf, z.vbuf, true, "v_buf"},
                         {decay_buf, z.dbuf, true, "decay_buf"},
                         {beta_buf, z.bbuf, true, "beta_buf"}});
  if (st != SSM_OK) return st;
  (void)hipGetLastError();
  return launched(ssm::launch_buffer_append(*d, k_t, v_t, decay_t, beta_t, k_buf, v_buf,
                                            decay_buf, beta_buf, slot,
                                            reinterpret_cast<hipStream_t>(stream)),
                  fn);
}

static ssm_status update_refresh_impl(const char* fn, const ssm_dims* d, const int32_t* rank_offsets,
                               float* state, void* sketch, const float* basis, const void* k_buf,
                               const void* v_buf, const float* decay_buf, const float* beta_buf,
                               int32_t n_tokens, void* stream, bool ranked,
                               float* read_map = nullptr, bool ls = false) {
  ssm_status st = check_dims(d, fn);
  if (st != SSM_OK) return st;
  if (ranked && (st = check_rank_offsets(*d, rank_offsets, fn)) != SSM_OK) return st;
  if (n_tokens < 0 || n_tokens > d->window)
    return fail(SSM_E_RANGE, "%s: n_tokens %d not in [0, %d]", fn, n_tokens, d->window);
  if (d->batch == 0) return ok();
  if (state == nullptr) return fail(SSM_E_NULL, "%s: state is NULL", fn);
  if (ls) {
    if (d->sketch_dtype != SSM_SKETCH_F32)
      return fail(SSM_E_RANGE, "%s: least-squares coefficients need an fp32 sketch", fn);
    if (sketch == nullptr) return fail(SSM_E_NULL, "%s: sketch_q is NULL", fn);
    if (read_map == nullptr) return fail(SSM_E_NULL, "%s: read_map is NULL", fn);
  }
  if (sketch != nullptr && basis == nullptr)
    return fail(SSM_E_NULL, "%s: basis is NULL but a sketch is requested", fn);
  if (n_tokens > 0) {
    if ((st = check_buffers(*d, k_buf, v_buf, decay_buf, beta_buf, fn)) != SSM_OK) return st;
  }
  if (n_tokens == 0 && sketch == nullptr) return ok();  // nothing to apply, nothing to store
  Sizes z = sizes_of(*d);
  apply_ranks(*d, rank_offsets, z);
  const bool tok = n_tokens > 0;
  const size_t map_bytes = z.units * d->rank * d->d_k * 4;
  st = check_arrays(fn, {{state, z.state, true, "state"}, {sketch, z.sketch, true, ls ? "sketch_q" : "sketch"},
                         {read_map, map_bytes, true, "read_map"},
                         {basis, z.basis, false, "basis"},
                         {tok ? k_buf : nullptr, z.kbuf, false, "k_buf"},
                         {tok ? v_buf : nullptr, z.vbuf, false, "v_buf"},
                         {tok ? decay_buf : nullptr, z.dbuf, false, "decay_buf"},
                         {tok ? beta_buf : nullptr, z.bbuf, false, "beta_buf"}});
  if (st != SSM_OK) return st;
  (void)hipGetLastError();
  return launched(ssm::launch_update_refresh(*d, rank_offsets, state, sketch, basis, k_buf, v_buf, decay_buf,
                                             beta_buf, n_tokens,
                                             reinterpret_cast<hipStream_t>(stream), nullptr,
                                             read_map),
                  fn);
}

static ssm_status sketch_decode_impl(const char* fn, const ssm_dims* d, const int32_t* rank_offsets,
                              const void* sketch, const float* basis, const void* q,
                              const void* k_t, const void* v_t, const float* decay_t,
                              const float* beta_t, void* k_buf, void* v_buf, float* decay_buf,
                              float* beta_buf, int32_t tau, float* y, void* stream, bool ranked,
                              bool ls = false) {
  ssm_status st = check_dims(d, fn);
  if (st != SSM_OK) return st;
  if (ranked && (st = check_rank_offsets(*d, rank_offsets, fn)) != SSM_OK) return st;
  if (tau < 1 || tau > d->window)
    return fail(SSM_E_RANGE, "%s: tau %d not in [1, %d]", fn, tau, d->window);
  if (d->batch == 0) return ok();
  if (ls && d->sketch_dtype != SSM_SKETCH_F32)
    return fail(SSM_E_RANGE, "%s: least-squares coefficients need an fp32 sketch", fn);
  if (sketch == nullptr) return fail(SSM_E_NULL, "%s: %s is NULL", fn, ls ? "sketch_q" : "sketch");
  if (basis == nullptr) return fail(SSM_E_NULL, "%s: %s is NULL", fn, ls ? "read_map" : "basis");
  if (q == nullptr) return fail(SSM_E_NULL, "%s: q is NULL", fn);
  if (y == nullptr) return fail(SSM_E_NULL, "%s: y is NULL", fn);
  if ((st = check_token(*d, k_t, v_t, decay_t, beta_t, fn)) != SSM_OK) return st;
  if ((st = check_buffers(*d, k_buf, v_buf, decay_buf, beta_buf, fn)) != SSM_OK) return st;
  Sizes z = sizes_of(*d);
  apply_ranks(*d, rank_offsets, z);
  if (ls) z.basis = z.units * d->rank * d->d_k * 4;  // the per-unit read map
  const bool fused = k_t != nullptr;
  st = check_arrays(fn, {{sketch, z.sketch, false, ls ? "sketch_q" : "sketch"},
                         {basis, z.basis, false, ls ? "read_map" : "basis"},
                         {q, z.qk, false, "q"}, {k_t, z.qk, false, "k_t"}, {v_t, z.v, false, "v_t"},
                         {decay_t, z.dtok, false, "decay_t"}, {beta_t, z.btok, false, "beta_t"},
                         {k_buf, z.kbuf, fused, "k_buf"}, {v_buf, z.vbuf, fused, "v_buf"},
                         {decay_buf, z.dbuf, fused, "decay_buf"},
                         {beta_buf, z.bbuf, fused, "beta_buf"}, {y, z.y, true, "y"}});
  if (st != SSM_OK) return st;
  (void)hipGetLastError();
  return launched(ssm::launch_sketch_decode(*d, rank_offsets, sketch, basis, q, k_t, v_t, decay_t, beta_t,
                                            k_buf, v_buf, decay_buf, beta_buf, tau, y,
                                            reinterpret_cast<hipStream_t>(stream), nullptr, ls),
                  fn);
}

ssm_status ssm_full_read_decode_step(const ssm_dims* d, const float* state, const void* q,
                                     const void* k_t, const void* v_t, const float* decay_t,
                                     const float* beta_t, void* k_buf, void* v_buf,
                                     float* decay_buf, float* beta_buf, int32_t tau, float* y,
                                     void* stream) {
  static const char* fn = "ssm_full_read_decode_step";
  ssm_status st = check_dims(d, fn);
  if (st != SSM_OK) return st;
  if (tau < 1 || tau > d->window)
    return fail(SSM_E_RANGE, "%s: tau %d not in [1, %d]", fn, tau, d->window);
  if (d->batch == 0) return ok();
  if (state == nullptr) return fail(SSM_E_NULL, "%s: state is NULL", fn);
  if (q == nullptr) return fail(SSM_E_NULL, "%s: q is NULL", fn);
  if (y == nullptr) return fail(SSM_E_NULL, "%s: y is NULL", fn);
  if ((st = check_token(*d, k_t, v_t, decay_t, beta_t, fn)) != SSM_OK) return st;
  if ((st = check_buffers(*d, k_buf, v_buf, decay_buf, beta_buf, fn)) != SSM_OK) return st;
  const Sizes z = sizes_of(*d);
  const bool fused = k_t != nullptr;
  st = check_arrays(fn, {{state, z.state, false, "state"}, {q, z.qk, false, "q"},
                         {k_t, z.qk, false, "k_t"}, {v_t, z.v, false, "v_t"},
                         {decay_t, z.dtok, false, "decay_t"}, {beta_t, z.btok, false, "beta_t"},
                         {k_buf, z.kbuf, fused, "k_buf"}, {v_buf, z.vbuf, fused, "v_buf"},
                         {decay_buf, z.dbuf, fused, "decay_buf"},
                         {beta_buf, z.bbuf, fused, "beta_buf"}, {y, z.y, true, "y"}});
  if (st != SSM_OK) return st;
  (void)hipGetLastError();
  return launched(ssm::launch_full_read_decode(*d, state, q, k_t, v_t, decay_t, beta_t, k_buf,
                                               v_buf, decay_buf, beta_buf, tau, y,
                                               reinterpret_cast<hipStream_t>(stream)),
                  fn);
}

ssm_status ssm_recurrent_decode_step(const ssm_dims* d, float* state, const void* q,
                                     const void* k_t, const void* v_t, const float* decay_t,
                                     const float* beta_t, float* y, void* stream) {
  static const char* fn = "ssm_recurrent_decode_step";
  ssm_status st = check_dims(d, fn);
  if (st != SSM_OK) return st;
  if (d->batch == 0) return ok();
  if (state == nullptr) return fail(SSM_E_NULL, "%s: state is NULL", fn);
  if (q == nullptr) return fail(SSM_E_NULL, "%s: q is NULL", fn);
  if (y == nullptr) return fail(SSM_E_NULL, "%s: y is NULL", fn);
  if (k_t == nullptr) return fail(SSM_E_NULL, "%s: k_t is NULL", fn);
  if ((st = check_token(*d, k_t, v_t, decay_t, beta_t, fn)) != SSM_OK) return st;
  const Sizes z = sizes_of(*d);
  st = check_arrays(fn, {{state, z.state, true, "state"}, {q, z.qk, false, "q"},
                         {k_t, z.qk, false, "k_t"}, {v_t, z.v, false, "v_t"},
                         {decay_t, z.dtok, false, "decay_t"}, {beta_t, z.btok, false, "beta_t"},
                         {y, z.y, true, "y"}});
  if (st != SSM_OK) return st;
  (void)hipGetLastError();
  return launched(ssm::launch_recurrent_step(*d, state, q, k_t, v_t, decay_t, beta_t, y,
                                             reinterpret_cast<hipStream_t>(stream)),
                  fn);
}

ssm_status ssm_fit_basis(const ssm_dims* d, const void* samples, int32_t n_samples,
                         float* basis, void* stream) {
  static const char* fn = "ssm_fit_basis";
  ssm_status st = check_dims(d, fn);
  if (st != SSM_OK) return st;
  if (samples == nullptr) return fail(SSM_E_NULL, "%s: samples is NULL", fn);
  if (basis == nullptr) return fail(SSM_E_NULL, "%s: basis is NULL", fn);
  if (n_samples < 1 || n_samples > (1 << 24))
    return fail(SSM_E_SHAPE, "%s: n_samples %d not in [1, 2^24]", fn, n_samples);
  const Sizes z = sizes_of(*d);
  const size_t sample_bytes = (size_t)d->heads * (size_t)n_samples * d->d_k * z.elem;
  st = check_arrays(fn, {{samples, sample_bytes, false, "samples"}, {basis, z.basis, true, "basis"}});
  if (st != SSM_OK) return st;
  (void)hipGetLastError();
  return launched(ssm::launch_fit_basis(*d, samples, n_samples, basis,
                                        reinterpret_cast<hipStream_t>(stream)),
                  fn);
}

ssm_status ssm_stream_probe(float* buf, int64_t n_tiles, int32_t shape, void* stream) {
  static const char* fn = "ssm_stream_probe";
  if (buf == nullptr) return fail(SSM_E_NULL, "%s: buf is NULL", fn);
  if (shape != 0 && shape != 1) return fail(SSM_E_RANGE, "%s: shape %d is not 0 or 1", fn, shape);
  if (n_tiles < 1 || n_tiles >= kMaxUnits)
    return fail(SSM_E_SHAPE, "%s: n_tiles %lld not in [1, 2^24)", fn, (long long)n_tiles);
  if (shape == 1 && (n_tiles & 1))
    return fail(SSM_E_SHAPE, "%s: shape 1 needs an even n_tiles (got %lld)", fn, (long long)n_tiles);
  ssm_status st = check_arrays(fn, {{buf, (size_t)n_tiles * 65536, true, "buf"}});
  if (st != SSM_OK) return st;
  (void)hipGetLastError();
  return launched(ssm::launch_stream_probe(buf, (long long)n_tiles, shape,
                                           reinterpret_cast<hipStream_t>(stream)),
                  fn);
}

ssm_status ssm_window_update_refresh(const ssm_dims* d, float* state, void* sketch,
                                     const float* basis, const void* k_buf, const void* v_buf,
                                     const float* decay_buf, const float* beta_buf,
                                     int32_t n_tokens, void* stream) {
  return update_refresh_impl("ssm_window_update_refresh", d, nullptr, state, sketch, basis, k_buf,
                             v_buf, decay_buf, beta_buf, n_tokens, stream, false);
}

ssm_status ssm_window_update_refresh_ranked(const ssm_dims* d, const int32_t* rank_offsets,
                                            float* state, void* sketch, const float* basis,
                                            const void* k_buf, const void* v_buf,
                                            const float* decay_buf, const float* beta_buf,
                                            int32_t n_tokens, void* stream) {
  return update_refresh_impl("ssm_window_update_refresh_ranked", d, rank_offsets, state, sketch,
                             basis, k_buf, v_buf, decay_buf, beta_buf, n_tokens, stream, true);
}

ssm_status ssm_sketch_decode_step(const ssm_dims* d, const void* sketch, const float* basis,
                                  const void* q, const void* k_t, const void* v_t,
                                  const float* decay_t, const float* beta_t, void* k_buf,
                                  void* v_buf, float* decay_buf, float* beta_buf, int32_t tau,
                                  float* y, void* stream) {
  return sketch_decode_impl("ssm_sketch_decode_step", d, nullptr, sketch, basis, q, k_t, v_t,
                            decay_t, beta_t, k_buf, v_buf, decay_buf, beta_buf, tau, y, stream,
                            false);
}

ssm_status ssm_sketch_decode_step_ranked(const ssm_dims* d, const int32_t* rank_offsets,
                                         const void* sketch, const float* basis, const void* q,
                                         const void* k_t, const void* v_t, const float* decay_t,
                                         const float* beta_t, void* k_buf, void* v_buf,
                                         float* decay_buf, float* beta_buf, int32_t tau, float* y,
                                         void* stream) {
  return sketch_decode_impl("ssm_sketch_decode_step_ranked", d, rank_offsets, sketch, basis, q,
                            k_t, v_t, decay_t, beta_t, k_buf, v_buf, decay_buf, beta_buf, tau, y,
                            stream, true);
}

ssm_status ssm_window_update_refresh_ls(const ssm_dims* d, float* state, float* sketch_q,
                                        float* read_map, const float* basis, const void* k_buf,
                                        const void* v_buf, const float* decay_buf,
                                        const float* beta_buf, int32_t n_tokens, void* stream) {
  return update_refresh_impl("ssm_window_update_refresh_ls", d, nullptr, state, sketch_q, basis,
                             k_buf, v_buf, decay_buf, beta_buf, n_tokens, stream, false, read_map,
                             true);
}

ssm_status ssm_sketch_decode_step_ls(const ssm_dims* d, const float* sketch_q,
                                     const float* read_map, const void* q, const void* k_t,
                                     const void* v_t, const float* decay_t,
                                     const float* beta_t, void* k_buf, void* v_buf,
                                     float* decay_buf, float* beta_buf, int32_t tau, float* y,
                                     void* stream) {
  return sketch_decode_impl("ssm_sketch_decode_step_ls", d, nullptr, sketch_q, read_map, q, k_t,
                            v_t, decay_t, beta_t, k_buf, v_buf, decay_buf, beta_buf, tau, y,
                            stream, false, true);
}

ssm_status ssm_window_update_refresh_varlen(const ssm_dims* d, int32_t num_slots,
                                            const int32_t* slot, const int32_t* n_tokens,
                                            float* state, void* sketch, const float* basis,
                                            const void* k_buf, const void* v_buf,
                                            const float* decay_buf, const float* beta_buf,
                                            void* stream) {
  static const char* fn = "ssm_window_update_refresh_varlen";
  ssm_status st = check_dims(d, fn);
  if (st != SSM_OK) return st;
  if (d->batch == 0) return ok();
  if ((st = check_pool(*d, num_slots, slot, n_tokens, "n_tokens", fn)) != SSM_OK) return st;
  if (state == nullptr) return fail(SSM_E_NULL, "%s: state is NULL", fn);
  if (sketch != nullptr && basis == nullptr)
    return fail(SSM_E_NULL, "%s: basis is NULL but a sketch is requested", fn);
  if ((st = check_buffers(*d, k_buf, v_buf, decay_buf, beta_buf, fn)) != SSM_OK) return st;
  const Sizes z = pool_sizes(*d, num_slots);
  const size_t rows = (size_t)d->batch * 4;
  st = check_arrays(fn, {{state, z.state, true, "state"}, {sketch, z.sketch, true, "sketch"},
                         {basis, z.basis, false, "basis"}, {k_buf, z.kbuf, false, "k_buf"},
                         {v_buf, z.vbuf, false, "v_buf"}, {decay_buf, z.dbuf, false, "decay_buf"},
                         {beta_buf, z.bbuf, false, "beta_buf"},
                         {slot, rows, false, "slot", 4}, {n_tokens, rows, false, "n_tokens", 4}});
  if (st != SSM_OK) return st;
  const ssm::Varlen vl{slot, n_tokens, num_slots, 0, d->window};
  (void)hipGetLastError();
  return launched(ssm::launch_update_refresh(*d, nullptr, state, sketch, basis, k_buf, v_buf,
                                             decay_buf, beta_buf, 0,
                                             reinterpret_cast<hipStream_t>(stream), &vl),
                  fn);
}

ssm_status ssm_sketch_decode_step_varlen(const ssm_dims* d, int32_t num_slots,
                                         const int32_t* slot, const int32_t* tau,
                                         const void* sketch, const float* basis, const void* q,
                                         const void* k_t, const void* v_t, const float* decay_t,
                                         const float* beta_t, void* k_buf, void* v_buf,
                                         float* decay_buf, float* beta_buf, float* y,
                                         void* stream) {
  static const char* fn = "ssm_sketch_decode_step_varlen";
  ssm_status st = check_dims(d, fn);
  if (st != SSM_OK) return st;
  if (d->batch == 0) return ok();
  if ((st = check_pool(*d, num_slots, slot, tau, "tau", fn)) != SSM_OK) return st;
  if (sketch == nullptr) return fail(SSM_E_NULL, "%s: sketch is NULL", fn);
  if (basis == nullptr) return fail(SSM_E_NULL, "%s: basis is NULL", fn);
  if (q == nullptr) return fail(SSM_E_NULL, "%s: q is NULL", fn);
  if (y == nullptr) return fail(SSM_E_NULL, "%s: y is NULL", fn);
  if ((st = check_token(*d, k_t, v_t, decay_t, beta_t, fn)) != SSM_OK) return st;
  if ((st = check_buffers(*d, k_buf, v_buf, decay_buf, beta_buf, fn)) != SSM_OK) return st;
  const Sizes z = pool_sizes(*d, num_slots);
  const size_t rows = (size_t)d->batch * 4;
  const bool fused = k_t != nullptr;
  st = check_arrays(fn, {{sketch, z.sketch, false, "sketch"}, {basis, z.basis, false, "basis"},
                         {q, z.qk, false, "q"}, {k_t, z.qk, false, "k_t"}, {v_t, z.v, false, "v_t"},
                         {decay_t, z.dtok, false, "decay_t"}, {beta_t, z.btok, false, "beta_t"},
                         {k_buf, z.kbuf, fused, "k_buf"}, {v_buf, z.vbuf, fused, "v_buf"},
                         {decay_buf, z.dbuf, fused, "decay_buf"},
                         {beta_buf, z.bbuf, fused, "beta_buf"}, {y, z.y, true, "y"},
                         {slot, rows, false, "slot", 4}, {tau, rows, false, "tau", 4}});
  if (st != SSM_OK) return st;
  const ssm::Varlen vl{slot, tau, num_slots, 1, d->window};
  (void)hipGetLastError();
  return launched(ssm::launch_sketch_decode(*d, nullptr, sketch, basis, q, k_t, v_t, decay_t,
                                            beta_t, k_buf, v_buf, decay_buf, beta_buf, 0, y,
                                            reinterpret_cast<hipStream_t>(stream), &vl),
                  fn);
}

ssm_status ssm_decode_step_varlen(const ssm_dims* d, int32_t num_slots, const int32_t* slot,
                                  const int32_t* tau, const int32_t* parity, int32_t n_update,
                                  const int32_t* update_rows, float* state, void* sketch0,
                                  void* sketch1, const float* basis, const void* q,
                                  const void* k_t, const void* v_t, const float* decay_t,
                                  const float* beta_t, void* k_buf, void* v_buf,
                                  float* decay_buf, float* beta_buf, float* y, void* stream) {
  static const char* fn = "ssm_decode_step_varlen";
  ssm_status st = check_dims(d, fn);
  if (st != SSM_OK) return st;
  if (n_update < 0 || n_update > d->batch)
    return fail(SSM_E_RANGE, "%s: n_update %d not in [0, batch = %d]", fn, n_update, d->batch);
  if (d->batch == 0) return ok();
  if ((st = check_pool(*d, num_slots, slot, tau, "tau", fn)) != SSM_OK) return st;
  if (parity == nullptr) return fail(SSM_E_NULL, "%s: parity is NULL", fn);
  if (n_update > 0 && update_rows == nullptr)
    return fail(SSM_E_NULL, "%s: update_rows is NULL with n_update = %d", fn, n_update);
  if (state == nullptr) return fail(SSM_E_NULL, "%s: state is NULL", fn);
  if (sketch0 == nullptr) return fail(SSM_E_NULL, "%s: sketch0 is NULL", fn);
  if (sketch1 == nullptr) return fail(SSM_E_NULL, "%s: sketch1 is NULL", fn);
  if (basis == nullptr) return fail(SSM_E_NULL, "%s: basis is NULL", fn);
  if (q == nullptr) return fail(SSM_E_NULL, "%s: q is NULL", fn);
  if (y == nullptr) return fail(SSM_E_NULL, "%s: y is NULL", fn);
  if (k_t == nullptr)
    return fail(SSM_E_NULL, "%s: k_t is NULL (the step appends the current token)", fn);
  if ((st = check_token(*d, k_t, v_t, decay_t, beta_t, fn)) != SSM_OK) return st;
  if ((st = check_buffers(*d, k_buf, v_buf, decay_buf, beta_buf, fn)) != SSM_OK) return st;
  const Sizes z = pool_sizes(*d, num_slots);
  const size_t rows = (size_t)d->batch * 4;
  st = check_arrays(fn, {{state, z.state, true, "state"}, {sketch0, z.sketch, true, "sketch0"},
                         {sketch1, z.sketch, true, "sketch1"}, {basis, z.basis, false, "basis"},
                         {q, z.qk, false, "q"}, {k_t, z.qk, false, "k_t"}, {v_t, z.v, false, "v_t"},
                         {decay_t, z.dtok, false, "decay_t"}, {beta_t, z.btok, false, "beta_t"},
                         {k_buf, z.kbuf, true, "k_buf"}, {v_buf, z.vbuf, true, "v_buf"},
                         {decay_buf, z.dbuf, true, "decay_buf"},
                         {beta_buf, z.bbuf, true, "beta_buf"}, {y, z.y, true, "y"},
                         {slot, rows, false, "slot", 4}, {tau, rows, false, "tau", 4},
                         {parity, rows, false, "parity", 4},
                         {update_rows, (size_t)n_update * 4, false, "update_rows", 4}});
  if (st != SSM_OK) return st;
  (void)hipGetLastError();
  return launched(ssm::launch_decode_step(*d, num_slots, slot, tau, parity, n_update,
                                          update_rows, state, sketch0, sketch1, basis, q, k_t,
                                          v_t, decay_t, beta_t, k_buf, v_buf, decay_buf,
                                          beta_buf, y, reinterpret_cast<hipStream_t>(stream)),
                  fn);
}

}  // extern "C"
