// C ABI of the KDA library: argument validation, state handles, dispatch.
// Every entry point validates fully before it enqueues anything, returns a
// kda_status, and never lets a C++ exception escape.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <mutex>
#include <new>

#include "kda_common.h"

struct kda_state {
  kda_dims dims;
  float* S;
  void* ring;
  bool own_S;
  bool own_ring;
  void* ws;         // prefill workspace owned by the handle (grown on demand)
  size_t ws_bytes;
};

namespace {

thread_local char g_err[512] = "";

kda_status fail(kda_status st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return st;
}

kda_status hip_fail(hipError_t e, const char* what) {
  return fail(KDA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool supported_width(int32_t d) { return d == 16 || d == 32 || d == 64 || d == 128; }

size_t io_size(kda_dtype io) { return io == KDA_BF16 ? 2 : 4; }

// The io field of validated dims as the enum (check_dims has rejected every
// other value).
kda_dtype io_of(const kda_dims* d) { return static_cast<kda_dtype>(d->io); }

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }
bool aligned16(const void* p) { return aligned(p, 16); }

// Checks dims; on success fills the element counts used by the calls.
kda_status check_dims(const kda_dims* d) {
  if (!d) return fail(KDA_ERR_INVALID, "dims is NULL");
  if (d->batch < 1 || d->heads < 1)
    return fail(KDA_ERR_INVALID, "batch (%d) and heads (%d) must be >= 1", d->batch, d->heads);
  if (d->batch > 65535 || d->heads > 65535)
    return fail(KDA_ERR_UNSUPPORTED, "batch and heads are limited to 65535 each");
  if (d->conv_width != 4)
    return fail(KDA_ERR_INVALID, "conv_width must be 4 (got %d)", d->conv_width);
  if (d->io != KDA_F32 && d->io != KDA_BF16)
    return fail(KDA_ERR_INVALID, "io dtype %d is not KDA_F32 or KDA_BF16", d->io);
  if (!supported_width(d->d_k) || !supported_width(d->d_v))
    return fail(KDA_ERR_UNSUPPORTED, "d_k=%d d_v=%d: supported widths are 16, 32, 64, 128",
                d->d_k, d->d_v);
  return KDA_OK;
}

size_t ctot_of(const kda_dims* d) {
  return (size_t)d->heads * (size_t)(2 * d->d_k + d->d_v);
}

size_t s_bytes_of(const kda_dims* d) {
  return (size_t)d->batch * d->heads * d->d_k * d->d_v * sizeof(float);
}

size_t ring_bytes_of(const kda_dims* d) {
  return (size_t)d->batch * 3 * ctot_of(d) * io_size(io_of(d));
}

// `allowed` is the set of flag bits the entry point understands.
kda_status check_flags(uint32_t flags, uint32_t allowed) {
  if (flags & ~allowed)
    return fail(KDA_ERR_INVALID, "flag bits 0x%x are not valid for this call", flags & ~allowed);
  return KDA_OK;
}

constexpr uint32_t kPrologueFlags = KDA_F_SKIP_CONV | KDA_F_SKIP_L2;
constexpr uint32_t kStepFlags =
    KDA_F_SKIP_CONV | KDA_F_SKIP_L2 | KDA_F_SCALAR_G | KDA_F_RAW_GATES;

// Token tensors, g, beta and o are accessed per element (natural alignment);
// conv weights, S, the ring and the workspace are accessed 16 bytes at a time.
#define KDA_REQUIRE_PTR(p, name, align)                                              \
  do {                                                                               \
    if (!(p)) return fail(KDA_ERR_INVALID, "%s is NULL", name);                      \
    if (!aligned((p), (align)))                                                      \
      return fail(KDA_ERR_INVALID, "%s is not %d-byte aligned", name, (int)(align)); \
  } while (0)

constexpr size_t kDefaultWsCap = (size_t)2 << 30;  // 2 GiB

kda_status check_eps(float eps) {
  if (!(eps > 0.0f) || !(eps < INFINITY))
    return fail(KDA_ERR_INVALID, "eps = %g must be finite and > 0", (double)eps);
  return KDA_OK;
}

// Shared by kda_decode_step and kda_decode_step_gated (gate == NULL: plain).
kda_status decode_common(kda_state* stt, const void* q, const void* k, const void* v,
                         const float* g, const float* beta, const float* conv_w,
                         const void* gate, const float* norm_w, float eps, void* o,
                         uint32_t flags, hipStream_t stream) {
  const kda_dims* d = &stt->dims;
  const size_t esz = io_size(io_of(d));
  KDA_REQUIRE_PTR(q, "q", esz);
  KDA_REQUIRE_PTR(k, "k", esz);
  KDA_REQUIRE_PTR(v, "v", esz);
  KDA_REQUIRE_PTR(g, "g", 4);
  KDA_REQUIRE_PTR(beta, "beta", 4);
  KDA_REQUIRE_PTR(o, "o", esz);
  if (!(flags & KDA_F_SKIP_CONV)) KDA_REQUIRE_PTR(conv_w, "conv_w", 16);
  kda::DecodeArgs a{stt->S, stt->ring, q, k, v, g, beta, conv_w, o,
                    d->batch, d->heads, d->d_k, d->d_v, flags, gate, norm_w, eps};
  hipError_t e = kda::launch_decode(a, io_of(d), stream);
  if (e != hipSuccess) return hip_fail(e, "decode launch");
  return KDA_OK;
}

}  // namespace

extern "C" {

const char* kda_last_error(void) { return g_err; }

const char* kda_version(void) { return "kda-gfx950 0.1"; }

size_t kda_state_bytes(const kda_dims* dims, size_t* ring_bytes) {
  if (check_dims(dims) != KDA_OK) {
    if (ring_bytes) *ring_bytes = 0;
    return 0;
  }
  if (ring_bytes) *ring_bytes = ring_bytes_of(dims);
  return s_bytes_of(dims);
}

kda_status kda_state_alloc(const kda_dims* dims, void* s_mem, void* ring_mem,
                           kda_state** out) {
  g_err[0] = 0;
  if (!out) return fail(KDA_ERR_INVALID, "out is NULL");
  *out = nullptr;
  kda_status st = check_dims(dims);
  if (st != KDA_OK) return st;
  if (s_mem && !aligned16(s_mem)) return fail(KDA_ERR_INVALID, "s_mem is not 16-byte aligned");
  if (ring_mem && !aligned16(ring_mem))
    return fail(KDA_ERR_INVALID, "ring_mem is not 16-byte aligned");
  kda_state* h = new (std::nothrow) kda_state();
  if (!h) return fail(KDA_ERR_OOM, "host allocation of the handle failed");
  h->dims = *dims;
  h->S = static_cast<float*>(s_mem);
  h->ring = ring_mem;
  if (!h->S) {
    if (hipMalloc(reinterpret_cast<void**>(&h->S), s_bytes_of(dims)) != hipSuccess) {
      delete h;
      return fail(KDA_ERR_OOM, "hipMalloc of %zu state bytes failed", s_bytes_of(dims));
    }
    h->own_S = true;
  }
  if (!h->ring) {
    if (hipMalloc(&h->ring, ring_bytes_of(dims)) != hipSuccess) {
      if (h->own_S) (void)hipFree(h->S);
      delete h;
      return fail(KDA_ERR_OOM, "hipMalloc of %zu ring bytes failed", ring_bytes_of(dims));
    }
    h->own_ring = true;
  }
  *out = h;
  return KDA_OK;
}

void kda_state_free(kda_state* st) {
  if (!st) return;
  if (st->own_S) (void)hipFree(st->S);
  if (st->own_ring) (void)hipFree(st->ring);
  if (st->ws) (void)hipFree(st->ws);
  delete st;
}

float* kda_state_S(kda_state* st) { return st ? st->S : nullptr; }

void* kda_state_ring(kda_state* st) { return st ? st->ring : nullptr; }

kda_status kda_state_get_dims(const kda_state* st, kda_dims* out) {
  if (!st || !out) return fail(KDA_ERR_INVALID, "NULL argument");
  *out = st->dims;
  return KDA_OK;
}

kda_status kda_state_reset(kda_state* st, const int32_t* seq_ids, int32_t n,
                           hipStream_t stream) {
  g_err[0] = 0;
  if (!st) return fail(KDA_ERR_INVALID, "state is NULL");
  const kda_dims* d = &st->dims;
  if (seq_ids) {
    if (n < 0) return fail(KDA_ERR_INVALID, "n = %d is negative", n);
    for (int32_t i = 0; i < n; ++i)
      if (seq_ids[i] < 0 || seq_ids[i] >= d->batch)
        return fail(KDA_ERR_INVALID, "seq_ids[%d] = %d is outside [0, %d)", i, seq_ids[i],
                    d->batch);
  }
  const size_t s_seq = s_bytes_of(d) / d->batch;
  const size_t r_seq = ring_bytes_of(d) / d->batch;
  hipError_t e;
  if (!seq_ids) {
    if ((e = kda::launch_fill_zero(st->S, s_bytes_of(d), stream)) != hipSuccess)
      return hip_fail(e, "reset of S");
    if ((e = kda::launch_fill_zero(st->ring, ring_bytes_of(d), stream)) != hipSuccess)
      return hip_fail(e, "reset of the ring");
    return KDA_OK;
  }
  for (int32_t i = 0; i < n; ++i) {
    uint8_t* s = reinterpret_cast<uint8_t*>(st->S) + (size_t)seq_ids[i] * s_seq;
    uint8_t* r = reinterpret_cast<uint8_t*>(st->ring) + (size_t)seq_ids[i] * r_seq;
    if ((e = kda::launch_fill_zero(s, s_seq, stream)) != hipSuccess)
      return hip_fail(e, "reset of S");
    if ((e = kda::launch_fill_zero(r, r_seq, stream)) != hipSuccess)
      return hip_fail(e, "reset of the ring");
  }
  return KDA_OK;
}

kda_status kda_conv_prologue(const kda_dims* dims, int32_t T, const void* q, const void* k,
                             const void* v, const float* conv_w, void* ring, float* q_out,
                             float* k_out, float* v_out, uint32_t flags, hipStream_t stream) {
  g_err[0] = 0;
  kda_status st = check_dims(dims);
  if (st != KDA_OK) return st;
  if ((st = check_flags(flags, kPrologueFlags)) != KDA_OK) return st;
  if (T < 0) return fail(KDA_ERR_INVALID, "T = %d is negative", T);
  if (T == 0) return KDA_OK;
  if ((long long)dims->batch * T * dims->heads > (1LL << 31) * 3)
    return fail(KDA_ERR_UNSUPPORTED, "B*T*H too large for one launch");
  const size_t esz = io_size(io_of(dims));
  KDA_REQUIRE_PTR(q, "q", esz);
  KDA_REQUIRE_PTR(k, "k", esz);
  KDA_REQUIRE_PTR(v, "v", esz);
  KDA_REQUIRE_PTR(q_out, "q_out", 4);
  KDA_REQUIRE_PTR(k_out, "k_out", 4);
  KDA_REQUIRE_PTR(v_out, "v_out", 4);
  if (!(flags & KDA_F_SKIP_CONV)) {
    KDA_REQUIRE_PTR(conv_w, "conv_w", 16);
    KDA_REQUIRE_PTR(ring, "ring", esz);
  }
  kda::PrologueArgs a{q, k, v, conv_w, ring, q_out, k_out, v_out,
                      dims->batch, T, dims->heads, dims->d_k, dims->d_v, flags};
  hipError_t e = kda::launch_prologue(a, io_of(dims), stream);
  if (e != hipSuccess) return hip_fail(e, "prologue launch");
  if (!(flags & KDA_F_SKIP_CONV)) {
    e = kda::launch_ring_advance(q, k, v, ring, dims->batch, T, dims->heads, dims->d_k,
                                 dims->d_v, io_of(dims), stream);
    if (e != hipSuccess) return hip_fail(e, "ring advance launch");
  }
  return KDA_OK;
}

kda_status kda_decode_step(kda_state* stt, const void* q, const void* k, const void* v,
                           const float* g, const float* beta, const float* conv_w, void* o,
                           uint32_t flags, hipStream_t stream) {
  g_err[0] = 0;
  if (!stt) return fail(KDA_ERR_INVALID, "state is NULL");
  kda_status st = check_flags(flags, kStepFlags);
  if (st != KDA_OK) return st;
  return decode_common(stt, q, k, v, g, beta, conv_w, nullptr, nullptr, 0.0f, o, flags,
                       stream);
}

kda_status kda_decode_step_gated(kda_state* stt, const void* q, const void* k, const void* v,
                                 const float* g, const float* beta, const float* conv_w,
                                 const void* gate, const float* norm_w, float eps, void* o,
                                 uint32_t flags, hipStream_t stream) {
  g_err[0] = 0;
  if (!stt) return fail(KDA_ERR_INVALID, "state is NULL");
  kda_status st = check_flags(flags, kStepFlags);
  if (st != KDA_OK) return st;
  if ((st = check_eps(eps)) != KDA_OK) return st;
  KDA_REQUIRE_PTR(gate, "gate", io_size(io_of(&stt->dims)));
  KDA_REQUIRE_PTR(norm_w, "norm_w", 4);
  return decode_common(stt, q, k, v, g, beta, conv_w, gate, norm_w, eps, o, flags, stream);
}

kda_status kda_gated_rmsnorm(const kda_dims* dims, int32_t T, const void* x, const void* gate,
                             const float* norm_w, float eps, void* out, hipStream_t stream) {
  g_err[0] = 0;
  kda_status st = check_dims(dims);
  if (st != KDA_OK) return st;
  if (T < 0) return fail(KDA_ERR_INVALID, "T = %d is negative", T);
  if ((st = check_eps(eps)) != KDA_OK) return st;
  if (T == 0) return KDA_OK;
  KDA_REQUIRE_PTR(x, "x", 16);
  KDA_REQUIRE_PTR(gate, "gate", 16);
  KDA_REQUIRE_PTR(norm_w, "norm_w", 16);
  KDA_REQUIRE_PTR(out, "out", 16);
  const long rows = (long)dims->batch * T * dims->heads;
  const size_t bytes = (size_t)rows * dims->d_v * io_size(io_of(dims));
  const uintptr_t xo = reinterpret_cast<uintptr_t>(x), oo = reinterpret_cast<uintptr_t>(out),
                  go = reinterpret_cast<uintptr_t>(gate);
  if (oo != xo && oo < xo + bytes && xo < oo + bytes)
    return fail(KDA_ERR_INVALID, "out overlaps x without being x");
  if (oo < go + bytes && go < oo + bytes)
    return fail(KDA_ERR_INVALID, "out overlaps gate");
  hipError_t e = kda::launch_gated_rmsnorm(x, gate, norm_w, eps, out, rows, dims->d_v, io_of(dims),
                                           stream);
  if (e != hipSuccess) return hip_fail(e, "gated rmsnorm launch");
  return KDA_OK;
}

size_t kda_prefill_workspace_bytes(const kda_dims* dims, int32_t T, int32_t chunk) {
  if (check_dims(dims) != KDA_OK) return 0;
  if (T < 0 || (chunk != 16 && chunk != 32 && chunk != 64)) return 0;
  const size_t nchunks = ((size_t)T + chunk - 1) / chunk;
  return nchunks *
         kda::prefill_ws_bytes_per_chunk(dims->heads, dims->batch, dims->d_k, dims->d_v, chunk,
                                         io_of(dims));
}

namespace {

// Validation shared by the prefill entry points; on success *per_chunk and
// *nchunks give the workspace one chunk of all B*H chunk-heads needs and the
// chunk count of the call.
kda_status check_prefill(const kda_state* stt, int32_t T, const void* q, const void* k,
                         const void* v, const float* g, const float* beta, const float* conv_w,
                         const void* o, int32_t chunk, uint32_t flags, size_t* per_chunk,
                         size_t* nchunks) {
  if (!stt) return fail(KDA_ERR_INVALID, "state is NULL");
  kda_status st = check_flags(flags, kStepFlags);
  if (st != KDA_OK) return st;
  const kda_dims* d = &stt->dims;
  if (T < 0) return fail(KDA_ERR_INVALID, "T = %d is negative", T);
  if (chunk != 16 && chunk != 32 && chunk != 64)
    return fail(KDA_ERR_UNSUPPORTED, "chunk = %d: supported chunks are 16, 32, 64", chunk);
  *per_chunk = kda::prefill_ws_bytes_per_chunk(d->heads, d->batch, d->d_k, d->d_v, chunk, io_of(d));
  *nchunks = ((size_t)T + chunk - 1) / chunk;
  if (T == 0) return KDA_OK;
  const size_t esz = io_size(io_of(d));
  KDA_REQUIRE_PTR(q, "q", esz);
  KDA_REQUIRE_PTR(k, "k", esz);
  KDA_REQUIRE_PTR(v, "v", esz);
  KDA_REQUIRE_PTR(g, "g", 4);
  KDA_REQUIRE_PTR(beta, "beta", 4);
  KDA_REQUIRE_PTR(o, "o", esz);
  if (!(flags & KDA_F_SKIP_CONV)) KDA_REQUIRE_PTR(conv_w, "conv_w", 16);
  return KDA_OK;
}

// The prefill itself, once the workspace is chosen: the chunked kernels,
// which also advance the ring.
kda_status run_prefill(kda_state* stt, int32_t T, const void* q, const void* k, const void* v,
                       const float* g, const float* beta, const float* conv_w, void* o,
                       int32_t chunk, void* workspace, size_t workspace_bytes, uint32_t flags,
                       hipStream_t stream) {
  const kda_dims* d = &stt->dims;
  kda::PrefillArgs a{stt->S, stt->ring, q, k, v, g, beta, conv_w, o,
                     d->batch, T, d->heads, d->d_k, d->d_v, chunk, flags};
  hipError_t e = kda::launch_prefill(a, io_of(d), workspace, workspace_bytes, stream);
  if (e != hipSuccess) return hip_fail(e, "prefill launch");
  return KDA_OK;
}

}  // namespace

kda_status kda_chunk_prefill(kda_state* stt, int32_t T, const void* q, const void* k,
                             const void* v, const float* g, const float* beta,
                             const float* conv_w, void* o, int32_t chunk, void* workspace,
                             size_t workspace_bytes, uint32_t flags, hipStream_t stream) {
  g_err[0] = 0;
  size_t per_chunk = 0, nchunks = 0;
  kda_status st = check_prefill(stt, T, q, k, v, g, beta, conv_w, o, chunk, flags, &per_chunk,
                                &nchunks);
  if (st != KDA_OK || T == 0) return st;
  if (workspace) {
    if (!aligned16(workspace)) return fail(KDA_ERR_INVALID, "workspace is not 16-byte aligned");
    if (workspace_bytes < per_chunk)
      return fail(KDA_ERR_INVALID, "workspace of %zu bytes is below the %zu bytes of one chunk",
                  workspace_bytes, per_chunk);
  } else {
    size_t want = nchunks * per_chunk;
    if (want > kDefaultWsCap) want = (kDefaultWsCap / per_chunk) * per_chunk;
    if (want < per_chunk) want = per_chunk;
    if (stt->ws_bytes < want) {
      // The handle's workspace grows here. hipFree waits for work already
      // queued that may still read the old buffer.
      if (stt->ws) (void)hipFree(stt->ws);
      stt->ws = nullptr;
      stt->ws_bytes = 0;
      if (hipMalloc(&stt->ws, want) != hipSuccess)
        return fail(KDA_ERR_OOM, "hipMalloc of a %zu-byte prefill workspace failed", want);
      stt->ws_bytes = want;
    }
    workspace = stt->ws;
    workspace_bytes = stt->ws_bytes;
  }
  return run_prefill(stt, T, q, k, v, g, beta, conv_w, o, chunk, workspace, workspace_bytes,
                     flags, stream);
}

// ---- allocation-free prefill ----------------------------------------------
// The workspace of kda_chunk_prefill_noalloc: one fixed array per device,
// loaded with the library's code object and held until the process ends.
// Host code uses only the device address obtained for it below, never the
// array's name (which on the host is a stand-in, not a device address).
static __device__ __align__(256) unsigned char scratch[KDA_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];  // device address of `scratch` on each device

// The device address of `scratch` on the device of `stream`, looked up once
// per device (with that device current, as the call requires).
kda_status scratch_for(hipStream_t stream, void** out) {
  int cur = -1;
  hipError_t e = hipGetDevice(&cur);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  hipDevice_t sdev = cur;
  if (stream) {
    e = hipStreamGetDevice(stream, &sdev);
    if (e != hipSuccess) return hip_fail(e, "hipStreamGetDevice");
  }
  if (sdev != cur)
    return fail(KDA_ERR_INVALID, "the stream belongs to device %d but device %d is current",
                (int)sdev, cur);
  if (cur < 0 || cur >= kMaxDevices)
    return fail(KDA_ERR_UNSUPPORTED, "device %d: at most %d devices", cur, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[cur]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress of the static scratch");
    if (!p) return fail(KDA_ERR_HIP, "hipGetSymbolAddress returned NULL for the static scratch");
    g_scratch_ptr[cur] = p;
  }
  *out = g_scratch_ptr[cur];
  return KDA_OK;
}

}  // namespace

kda_status kda_chunk_prefill_noalloc(kda_state* stt, int32_t T, const void* q, const void* k,
                                     const void* v, const float* g, const float* beta,
                                     const float* conv_w, void* o, int32_t chunk, uint32_t flags,
                                     hipStream_t stream) {
  g_err[0] = 0;
  size_t per_chunk = 0, nchunks = 0;
  kda_status st = check_prefill(stt, T, q, k, v, g, beta, conv_w, o, chunk, flags, &per_chunk,
                                &nchunks);
  if (st != KDA_OK || T == 0) return st;
  if (per_chunk > (size_t)KDA_NOALLOC_SCRATCH_BYTES)
    return fail(KDA_ERR_UNSUPPORTED,
                "one chunk of %d sequences x %d heads needs %zu bytes of workspace, more than "
                "the %zu-byte static scratch of kda_chunk_prefill_noalloc",
                stt->dims.batch, stt->dims.heads, per_chunk, (size_t)KDA_NOALLOC_SCRATCH_BYTES);
  void* ws = nullptr;
  st = scratch_for(stream, &ws);
  if (st != KDA_OK) return st;
  return run_prefill(stt, T, q, k, v, g, beta, conv_w, o, chunk, ws,
                     (size_t)KDA_NOALLOC_SCRATCH_BYTES, flags, stream);
}

kda_status kda_stream_rmw(void* buf, size_t bytes, float scale, hipStream_t stream) {
  g_err[0] = 0;
  if (!buf) return fail(KDA_ERR_INVALID, "buf is NULL");
  if (!aligned16(buf) || bytes % 16 != 0)
    return fail(KDA_ERR_INVALID, "buf must be 16-byte aligned and bytes a multiple of 16");
  hipError_t e = kda::launch_stream_rmw(buf, bytes, scale, stream);
  if (e != hipSuccess) return hip_fail(e, "stream probe launch");
  return KDA_OK;
}

size_t kda_backward_workspace_bytes(const kda_dims* d, int32_t T, int32_t chunk) {
  if (check_dims(d) != KDA_OK || T < 0 || (chunk != 16 && chunk != 32 && chunk != 64)) return 0;
  return kda::backward_ws_bytes(d->batch, T, d->heads, d->d_k, d->d_v, chunk);
}

size_t kda_backward_workspace_min_bytes(const kda_dims* d, int32_t T, int32_t chunk) {
  if (check_dims(d) != KDA_OK || T < 0 || (chunk != 16 && chunk != 32 && chunk != 64)) return 0;
  return kda::backward_ws_min_bytes(d->batch, T, d->heads, d->d_k, d->d_v, chunk);
}

kda_status kda_chunk_backward(const kda_dims* d, int32_t T, const void* q, const void* k,
                              const void* v, const float* g, const float* beta, const float* S0,
                              const void* dO, const float* dST, void* dq, void* dk, void* dv,
                              float* dg, float* dbeta, float* dS0, int32_t chunk,
                              void* workspace, size_t workspace_bytes, uint32_t flags,
                              hipStream_t stream) {
  g_err[0] = 0;
  kda_status st = check_dims(d);
  if (st != KDA_OK) return st;
  if (flags != 0) return fail(KDA_ERR_INVALID, "kda_chunk_backward takes no flags (got 0x%x)", flags);
  if (T < 0) return fail(KDA_ERR_INVALID, "T = %d is negative", T);
  if (chunk != 16 && chunk != 32 && chunk != 64)
    return fail(KDA_ERR_UNSUPPORTED, "chunk = %d: supported chunks are 16, 32, 64", chunk);
  const size_t nc = ((size_t)T + chunk - 1) / chunk;
  if (nc * (size_t)d->batch * d->heads > 0x7fffffffu)
    return fail(KDA_ERR_UNSUPPORTED, "T = %d: too many (chunk, sequence, head) items", T);
  if (S0 && !aligned16(S0)) return fail(KDA_ERR_INVALID, "S0 is not 16-byte aligned");
  if (dST && !aligned16(dST)) return fail(KDA_ERR_INVALID, "dST is not 16-byte aligned");
  if (dS0 && !aligned16(dS0)) return fail(KDA_ERR_INVALID, "dS0 is not 16-byte aligned");
  const size_t need = kda::backward_ws_min_bytes(d->batch, T, d->heads, d->d_k, d->d_v, chunk);
  if (T > 0) {
    const size_t esz = io_size(io_of(d));
    // q, k, v, g and dO are read 16 bytes (or 8 for bf16) at a time
    KDA_REQUIRE_PTR(q, "q", 16);
    KDA_REQUIRE_PTR(k, "k", 16);
    KDA_REQUIRE_PTR(v, "v", 16);
    KDA_REQUIRE_PTR(g, "g", 16);
    KDA_REQUIRE_PTR(beta, "beta", 4);
    KDA_REQUIRE_PTR(dO, "dO", 16);
    KDA_REQUIRE_PTR(dq, "dq", esz);
    KDA_REQUIRE_PTR(dk, "dk", esz);
    KDA_REQUIRE_PTR(dv, "dv", esz);
    KDA_REQUIRE_PTR(dg, "dg", 4);
    KDA_REQUIRE_PTR(dbeta, "dbeta", 4);
    KDA_REQUIRE_PTR(workspace, "workspace", 16);
    if (workspace_bytes < need)
      return fail(KDA_ERR_INVALID, "workspace of %zu bytes is below the %zu bytes needed",
                  workspace_bytes, need);
  } else if (!dS0) {
    return KDA_OK;  // nothing to compute
  }
  kda::BackwardArgs a{q,  k,  v,     g,   beta,       S0,         dO,         dST,
                      dq, dk, dv,    dg,  dbeta,      dS0,        d->batch,   T,
                      d->heads, d->d_k, d->d_v, chunk, 0, 0, nullptr, nullptr, nullptr,
                      nullptr};
  hipError_t e = kda::launch_backward(a, io_of(d), workspace, T > 0 ? workspace_bytes : 0, stream);
  if (e != hipSuccess) return hip_fail(e, "backward launch");
  return KDA_OK;
}

size_t kda_prologue_backward_workspace_bytes(const kda_dims* d, int32_t T) {
  if (check_dims(d) != KDA_OK || T < 0) return 0;
  return (size_t)d->batch * kda::prologue_bwd_segments(T) * ctot_of(d) * 4 * sizeof(float);
}

kda_status kda_prologue_backward(const kda_dims* d, int32_t T, const void* q, const void* k,
                                 const void* v, const float* conv_w, const void* ring,
                                 const void* dq_hat, const void* dk_hat, const void* dv_hat,
                                 void* dq, void* dk, void* dv, float* dconv_w, float* dring,
                                 void* workspace, size_t workspace_bytes, uint32_t flags,
                                 hipStream_t stream) {
  g_err[0] = 0;
  kda_status st = check_dims(d);
  if (st != KDA_OK) return st;
  if (flags != 0)
    return fail(KDA_ERR_INVALID, "kda_prologue_backward takes no flags (got 0x%x)", flags);
  if (T < 0) return fail(KDA_ERR_INVALID, "T = %d is negative", T);
  if ((size_t)d->batch * d->heads * kda::prologue_bwd_segments(T) > 0x7fffffffu)
    return fail(KDA_ERR_UNSUPPORTED, "T = %d: too many (sequence, head, segment) items", T);
  const size_t esz = io_size(io_of(d));
  KDA_REQUIRE_PTR(conv_w, "conv_w", 16);
  KDA_REQUIRE_PTR(dconv_w, "dconv_w", 16);
  // q, k, v, the ring and the activation gradients are read 16 (fp32) or 8
  // (bf16) bytes at a time
  if (ring && !aligned16(ring)) return fail(KDA_ERR_INVALID, "ring is not 16-byte aligned");
  if (dring && !aligned(dring, 4)) return fail(KDA_ERR_INVALID, "dring is misaligned");
  if (T > 0) {
    KDA_REQUIRE_PTR(q, "q", 16);
    KDA_REQUIRE_PTR(k, "k", 16);
    KDA_REQUIRE_PTR(v, "v", 16);
    KDA_REQUIRE_PTR(dq_hat, "dq_hat", 16);
    KDA_REQUIRE_PTR(dk_hat, "dk_hat", 16);
    KDA_REQUIRE_PTR(dv_hat, "dv_hat", 16);
    KDA_REQUIRE_PTR(dq, "dq", esz);
    KDA_REQUIRE_PTR(dk, "dk", esz);
    KDA_REQUIRE_PTR(dv, "dv", esz);
    KDA_REQUIRE_PTR(workspace, "workspace", 16);
    const size_t need = kda_prologue_backward_workspace_bytes(d, T);
    if (workspace_bytes < need)
      return fail(KDA_ERR_INVALID, "workspace of %zu bytes is below the %zu bytes needed",
                  workspace_bytes, need);
  }
  hipError_t e;
  if (T == 0 && dring) {  // no tokens: the history's gradient is zero
    e = kda::launch_fill_zero(dring, (size_t)d->batch * 3 * ctot_of(d) * sizeof(float), stream);
    if (e != hipSuccess) return hip_fail(e, "fill launch");
  }
  kda::PrologueBwdArgs a{q,      k,      v,      conv_w, ring,     dq_hat,
                         dk_hat, dv_hat, dq,     dk,     dv,       dconv_w,
                         dring,  static_cast<float*>(workspace), d->batch, T,
                         d->heads, d->d_k, d->d_v, kda::prologue_bwd_segments(T)};
  e = kda::launch_prologue_backward(a, io_of(d), stream);
  if (e != hipSuccess) return hip_fail(e, "prologue backward launch");
  return KDA_OK;
}

}  // extern "C"
