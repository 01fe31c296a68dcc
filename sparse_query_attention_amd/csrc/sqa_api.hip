// C ABI of libsqa (declared in include/sqa.h): argument validation on the
// host, the stream-ordered workspace of sqa_forward (or the fixed device array
// of sqa_forward_noalloc), and dispatch to the three gfx950 kernels
// (projection, attention core, output projection).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <mutex>
#include <unordered_map>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "sqa.h"
#include "sqa_internal.h"

namespace {

thread_local char g_err[256] = "";

sqa_status fail(sqa_status s, const char* msg) {
  snprintf(g_err, sizeof(g_err), "%s", msg);
  return s;
}

sqa_status fail_hip(hipError_t e, const char* where) {
  snprintf(g_err, sizeof(g_err), "%s: %s", where, hipGetErrorString(e));
  return e == hipErrorOutOfMemory ? SQA_ERR_OUT_OF_MEMORY : SQA_ERR_HIP;
}

sqa_status ok() {
  g_err[0] = '\0';
  return SQA_OK;
}

size_t elem_size(sqa_dtype dt) { return dt == SQA_DTYPE_BF16 ? 2 : 4; }

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

// a*b without overflow into out; false on overflow or negative factors.
bool mul_ok(int64_t a, int64_t b, int64_t* out) {
  if (a < 0 || b < 0) return false;
  if (a != 0 && b > INT64_MAX / a) return false;
  *out = a * b;
  return true;
}

bool overlap(const void* a, size_t na, const void* b, size_t nb) {
  const uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
  return x < y + nb && y < x + na;
}

struct Shape {
  int64_t B, N, d_model, H, H_q, H_kv, d;
};

// Shared checks of the head configuration (pure host, no HIP call).
sqa_status check_heads(const Shape& s, bool need_h) {
  if (s.B < 0 || s.N < 0) return fail(SQA_ERR_INVALID_ARG, "B and N must be >= 0");
  if (s.N > SQA_MAX_N) return fail(SQA_ERR_UNSUPPORTED, "N exceeds SQA_MAX_N");
  if (s.B > (int64_t)1 << 20) return fail(SQA_ERR_UNSUPPORTED, "B exceeds 2^20");
  if (s.H_kv < 1 || s.H_q < s.H_kv) return fail(SQA_ERR_INVALID_ARG, "need 1 <= H_kv <= H_q");
  if (s.H_q % s.H_kv != 0) return fail(SQA_ERR_INVALID_ARG, "H_q must be a multiple of H_kv");
  if (s.H_q > 1024) return fail(SQA_ERR_UNSUPPORTED, "H_q exceeds 1024");
  if (need_h) {
    if (s.H < s.H_q) return fail(SQA_ERR_INVALID_ARG, "need H_q <= H");
    int64_t dm;
    if (!mul_ok(s.H, s.d, &dm) || dm != s.d_model)
      return fail(SQA_ERR_INVALID_ARG, "d_model must equal H * d_head");
  }
  if (s.d != 32 && s.d != 64) return fail(SQA_ERR_UNSUPPORTED, "d_head must be 32 or 64");
  return SQA_OK;
}

sqa_status check_dtype(sqa_dtype dt) {
  if (dt != SQA_DTYPE_FP32 && dt != SQA_DTYPE_BF16)
    return fail(SQA_ERR_UNSUPPORTED, "dtype must be SQA_DTYPE_FP32 or SQA_DTYPE_BF16");
  return SQA_OK;
}

sqa_status check_ptr(const void* p, const char* msg_null, const char* msg_align) {
  if (!p) return fail(SQA_ERR_INVALID_ARG, msg_null);
  if (!aligned16(p)) return fail(SQA_ERR_INVALID_ARG, msg_align);
  return SQA_OK;
}

#define SQA_TRY(expr)            \
  do {                           \
    sqa_status _s = (expr);      \
    if (_s != SQA_OK) return _s; \
  } while (0)

// Byte sizes of the intermediates, with overflow checks.
struct Sizes {
  int64_t Np, q, kv, a;  // bytes of q, of k (= of vt), of a
};

sqa_status sizes_for(const Shape& s, sqa_dtype dt, Sizes* out) {
  out->Np = sqa::padded_length(s.N);
  int64_t t, es = (int64_t)elem_size(dt);
  if (!mul_ok(s.B, out->Np, &t) || !mul_ok(t, s.d * es, &t)) return fail(SQA_ERR_UNSUPPORTED, "size overflow");
  int64_t qb, kb;
  if (!mul_ok(t, s.H_q, &qb) || !mul_ok(t, s.H_kv, &kb)) return fail(SQA_ERR_UNSUPPORTED, "size overflow");
  int64_t ab;
  if (!mul_ok(s.B, s.N, &ab) || !mul_ok(ab, s.H_q * s.d * es, &ab))
    return fail(SQA_ERR_UNSUPPORTED, "size overflow");
  out->q = qb; out->kv = kb; out->a = ab;
  return SQA_OK;
}

int64_t round256(int64_t x) { return (x + 255) / 256 * 256; }

constexpr int kMaxDevices = 64;

// The workspace of sqa_forward_noalloc: a fixed device array that every device
// the library runs on holds from the module's load until the process ends.
// Host code never passes its name to a kernel or a copy (in host code the name
// stands for a host-side shadow, not the device array): the device address is
// looked up once per device with hipGetSymbolAddress and kept in
// g_scratch_ptr.
static __device__ __align__(256) unsigned char scratch[SQA_NOALLOC_SCRATCH_BYTES];
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// The device address of `scratch` on the device of `stream`, looked up on the
// first call for that device with that device current.
sqa_status noalloc_scratch(hipStream_t stream, void** out) {
  int dev = 0;
  hipError_t e = stream ? hipStreamGetDevice(stream, &dev) : hipGetDevice(&dev);
  if (e != hipSuccess) return fail_hip(e, "device of stream");
  if (dev < 0 || dev >= kMaxDevices) return fail(SQA_ERR_UNSUPPORTED, "device index too large");
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    int cur = 0;
    e = hipGetDevice(&cur);
    if (e != hipSuccess) return fail_hip(e, "hipGetDevice");
    if (cur != dev && (e = hipSetDevice(dev)) != hipSuccess) return fail_hip(e, "hipSetDevice");
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    const hipError_t er = cur != dev ? hipSetDevice(cur) : hipSuccess;
    if (e != hipSuccess) return fail_hip(e, "hipGetSymbolAddress(scratch)");
    if (er != hipSuccess) return fail_hip(er, "hipSetDevice");
    if (!ptr) return fail(SQA_ERR_HIP, "hipGetSymbolAddress(scratch) returned null");
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return SQA_OK;
}

// One stream-ordered pool per device. Freed workspace stays in the pool for
// reuse (release threshold = max) instead of going back to the driver.
std::mutex g_pool_mu;
hipMemPool_t g_pools[kMaxDevices] = {};

sqa_status pool_for(hipStream_t stream, hipMemPool_t* out) {
  int dev = 0;
  hipError_t e = stream ? hipStreamGetDevice(stream, &dev) : hipGetDevice(&dev);
  if (e != hipSuccess) return fail_hip(e, "device of stream");
  if (dev < 0 || dev >= kMaxDevices) return fail(SQA_ERR_UNSUPPORTED, "device index too large");
  std::lock_guard<std::mutex> lock(g_pool_mu);
  if (!g_pools[dev]) {
    hipMemPoolProps props;
    memset(&props, 0, sizeof(props));
    props.allocType = hipMemAllocationTypePinned;
    props.handleTypes = hipMemHandleTypeNone;
    props.location.type = hipMemLocationTypeDevice;
    props.location.id = dev;
    hipMemPool_t pool;
    e = hipMemPoolCreate(&pool, &props);
    if (e != hipSuccess) return fail_hip(e, "hipMemPoolCreate");
    uint64_t thr = UINT64_MAX;
    e = hipMemPoolSetAttribute(pool, hipMemPoolAttrReleaseThreshold, &thr);
    if (e != hipSuccess) {
      (void)hipMemPoolDestroy(pool);
      return fail_hip(e, "hipMemPoolSetAttribute");
    }
    g_pools[dev] = pool;
  }
  *out = g_pools[dev];
  return SQA_OK;
}

// Per-stream workspace, kept between calls. A stream-ordered allocation and
// release per call cost about 2.5 us of device time (a decode step takes about
// 60 us), and while the pool grows they make the host wait for the device
// (about 270 us per call with earlier work still running). So a workspace of
// up to kStreamWsMax bytes stays with its stream instead: calls on one stream
// run in order, so each finds the previous one's use finished. A larger
// request takes a new buffer of at least twice the size; the old one is kept
// too, never freed, since a call on the same stream from another host thread
// may still be about to launch work on it (at most twice the largest
// workspace per stream in all). Buffers are held until the process ends.
constexpr size_t kStreamWsMax = SQA_STREAM_WORKSPACE_MAX;
std::mutex g_stream_ws_mu;
struct StreamWs { void* ptr; size_t bytes; };   // the current buffer; earlier ones stay allocated
std::unordered_map<hipStream_t, StreamWs> g_stream_ws;

sqa_status stream_workspace(hipStream_t stream, size_t bytes, void** out) {
  std::lock_guard<std::mutex> lock(g_stream_ws_mu);
  StreamWs& w = g_stream_ws[stream];
  if (w.ptr && w.bytes >= bytes) {
    *out = w.ptr;
    return SQA_OK;
  }
  hipMemPool_t pool;
  SQA_TRY(pool_for(stream, &pool));
  const size_t want = std::min(kStreamWsMax, std::max(bytes, 2 * w.bytes));
  void* p = nullptr;
  const hipError_t e = hipMallocFromPoolAsync(&p, want, pool, stream);
  if (e != hipSuccess) return fail_hip(e, "workspace allocation");
  w.ptr = p;
  w.bytes = want;
  *out = p;
  return SQA_OK;
}

// The workspace of one call: the stream's kept buffer up to kStreamWsMax
// bytes, else stream-ordered memory from the device's pool, released on the
// same stream after the call's launches.
struct Workspace {
  void* ptr = nullptr;
  hipStream_t stream = nullptr;
  bool pooled = false;
  sqa_status acquire(size_t bytes, hipStream_t s) {
    stream = s;
    if (bytes <= kStreamWsMax) return stream_workspace(s, bytes, &ptr);
    hipMemPool_t pool;
    SQA_TRY(pool_for(s, &pool));
    const hipError_t e = hipMallocFromPoolAsync(&ptr, bytes, pool, s);
    if (e != hipSuccess) { ptr = nullptr; return fail_hip(e, "workspace allocation"); }
    pooled = true;
    return SQA_OK;
  }
  hipError_t release() {
    if (!pooled || !ptr) return hipSuccess;
    const hipError_t e = hipFreeAsync(ptr, stream);
    ptr = nullptr;
    return e;
  }
};

// Checks a caller's buffer of saved training activations: its size, its
// alignment, and that it overlaps none of the given buffers.
sqa_status check_saved(const void* saved, size_t saved_bytes, const Shape& s, sqa_dtype dt,
                       const void* const* bufs, const size_t* sizes, int n) {
  if (!saved) return fail(SQA_ERR_INVALID_ARG, "saved is null");
  if (!aligned16(saved)) return fail(SQA_ERR_INVALID_ARG, "saved is not 16-byte aligned");
  const int64_t need =
      sqa::saved_layout((int64_t)elem_size(dt), s.B, s.N, sqa::padded_length(s.N), s.H_q, s.H_kv, s.d).total;
  if (saved_bytes < (size_t)need) return fail(SQA_ERR_INVALID_ARG, "saved_bytes is too small");
  for (int j = 0; j < n; ++j)
    if (overlap(saved, (size_t)need, bufs[j], sizes[j]))
      return fail(SQA_ERR_INVALID_ARG, "saved overlaps another buffer");
  return SQA_OK;
}

// sqa_forward (varlen false, lens unused), sqa_forward_varlen, sqa_prefill
// (kc, vc non-null: the caches [B, H_kv, N_max, d_head] receive K and V),
// sqa_forward_train (saved non-null: the activations stay there, with each
// row's log-sum-exp, instead of in the workspace) and sqa_forward_noalloc
// (no_alloc: the workspace is the fixed device array `scratch`).
sqa_status forward_impl(const void* x, const void* Wq, const void* Wk, const void* Wv,
                        const void* Wo, void* out, bool varlen, const int32_t* lens, void* kc,
                        void* vc, int64_t N_max, int64_t B, int64_t N, int64_t d_model, int64_t H,
                        int64_t H_q, int64_t H_kv, int64_t d_head, int causal, sqa_dtype dtype,
                        hipStream_t stream, void* saved = nullptr, size_t saved_bytes = 0,
                        bool no_alloc = false) {
  const Shape s{B, N, d_model, H, H_q, H_kv, d_head};
  SQA_TRY(check_dtype(dtype));
  SQA_TRY(check_heads(s, true));
  if (causal != 0 && causal != 1) return fail(SQA_ERR_INVALID_ARG, "causal must be 0 or 1");
  if (B * N == 0) return ok();
  SQA_TRY(check_ptr(x, "x is null", "x is not 16-byte aligned"));
  SQA_TRY(check_ptr(Wq, "Wq is null", "Wq is not 16-byte aligned"));
  SQA_TRY(check_ptr(Wk, "Wk is null", "Wk is not 16-byte aligned"));
  SQA_TRY(check_ptr(Wv, "Wv is null", "Wv is not 16-byte aligned"));
  SQA_TRY(check_ptr(Wo, "Wo is null", "Wo is not 16-byte aligned"));
  SQA_TRY(check_ptr(out, "out is null", "out is not 16-byte aligned"));
  if (!varlen) {
    lens = nullptr;
  } else if (lens == nullptr) {
    return fail(SQA_ERR_INVALID_ARG, "lens is null");
  } else if (reinterpret_cast<uintptr_t>(lens) & 3u) {
    return fail(SQA_ERR_INVALID_ARG, "lens is not 4-byte aligned");
  }
  Sizes z;
  SQA_TRY(sizes_for(s, dtype, &z));
  const size_t es = elem_size(dtype);
  const size_t yb = (size_t)(B * N * d_model) * es;
  const size_t wqb = (size_t)(d_model * H_q * d_head) * es, wkb = (size_t)(d_model * H_kv * d_head) * es;
  const void* ins[5] = {x, Wq, Wk, Wv, Wo};
  const size_t inb[5] = {yb, wqb, wkb, wkb, wqb};
  for (int j = 0; j < 5; ++j)
    if (overlap(out, yb, ins[j], inb[j])) return fail(SQA_ERR_INVALID_ARG, "out overlaps an input");
  if (lens && overlap(out, yb, lens, (size_t)B * sizeof(int32_t)))
    return fail(SQA_ERR_INVALID_ARG, "out overlaps lens");
  if (kc) {
    if (N > N_max) return fail(SQA_ERR_INVALID_ARG, "N exceeds N_max");
    int64_t cb;
    if (!mul_ok(B * H_kv, N_max, &cb) || !mul_ok(cb, d_head * (int64_t)es, &cb))
      return fail(SQA_ERR_UNSUPPORTED, "size overflow");
    if (overlap(kc, (size_t)cb, vc, (size_t)cb)) return fail(SQA_ERR_INVALID_ARG, "k_cache overlaps v_cache");
    for (void* c : {kc, vc}) {
      if (overlap(c, (size_t)cb, out, yb)) return fail(SQA_ERR_INVALID_ARG, "a cache overlaps out");
      for (int j = 0; j < 5; ++j)
        if (overlap(c, (size_t)cb, ins[j], inb[j])) return fail(SQA_ERR_INVALID_ARG, "a cache overlaps an input");
    }
  }

  if (saved) {
    const void* bufs[6] = {x, Wq, Wk, Wv, Wo, out};
    const size_t sizes[6] = {yb, wqb, wkb, wkb, wqb, yb};
    SQA_TRY(check_saved(saved, saved_bytes, s, dtype, bufs, sizes, 6));
  }
  // q, k, vt, a in the workspace, or in `saved` (then only the weight transposes are)
  const int64_t act = saved ? 0 : 1;
  const int64_t off_k = act * round256(z.q), off_v = off_k + act * round256(z.kv);
  const int64_t off_a = off_v + act * round256(z.kv), off_w1 = off_a + act * round256(z.a);
  const int64_t off_w3 = off_w1 + round256((int64_t)sqa::qkv_wt_bytes(dtype, d_model, H_q, H_kv, d_head));
  const int64_t off_ord = off_w3 + round256((int64_t)sqa::out_wt_bytes(dtype, H_q * d_head, d_model));
  const int64_t off_split = off_ord + (lens ? round256((int64_t)sqa::attention_order_bytes(B, N, H_q)) : 0);
  const int64_t split_b = (int64_t)sqa::attention_split_bytes(dtype, B, N, H_q, H_kv, d_head, causal != 0,
                                                              lens != nullptr, stream);
  const int64_t total = off_split + round256(split_b);
  void* ws = nullptr;
  Workspace wsp;
  hipError_t e = hipSuccess;
  if (no_alloc) {
    if ((uint64_t)total > (uint64_t)SQA_NOALLOC_SCRATCH_BYTES) {
      snprintf(g_err, sizeof(g_err),
               "the workspace of %lld bytes exceeds SQA_NOALLOC_SCRATCH_BYTES (%llu)",
               (long long)total, (unsigned long long)SQA_NOALLOC_SCRATCH_BYTES);
      return SQA_ERR_UNSUPPORTED;
    }
    SQA_TRY(noalloc_scratch(stream, &ws));
  } else {
    SQA_TRY(wsp.acquire((size_t)total, stream));
    ws = wsp.ptr;
  }
  char* base = (char*)ws;
  void *q = base, *k = base + off_k, *vt = base + off_v, *a = base + off_a;
  void *w1 = base + off_w1, *w3 = base + off_w3;
  int32_t* order = lens ? (int32_t*)(base + off_ord) : nullptr;
  float* split_ws = split_b > 0 ? (float*)(base + off_split) : nullptr;
  float* lse = nullptr;
  float* o32 = nullptr;
  if (saved) {
    const sqa::SavedLayout S = sqa::saved_layout((int64_t)es, B, N, z.Np, H_q, H_kv, d_head);
    char* sv = (char*)saved;
    q = sv + S.q; k = sv + S.k; vt = sv + S.vt; a = sv + S.a;
    lse = (float*)(sv + S.lse);
    o32 = (float*)(sv + S.o32);
  }

  e = sqa::launch_qkv_projection(dtype, x, Wq, Wk, Wv, w1, q, k, vt, B, N, z.Np, d_model, H_q,
                                 H_kv, d_head, lens, stream);
  if (e == hipSuccess && kc)
    e = sqa::launch_fill_cache(dtype, k, vt, kc, vc, B, H_kv, N, z.Np, N_max, d_head, stream);
  if (e == hipSuccess)
    e = sqa::launch_attention(dtype, q, k, vt, a, B, N, z.Np, H_q, H_kv, d_head, causal != 0, lens,
                              stream, lse, order, o32, split_ws);
  if (e == hipSuccess)
    e = sqa::launch_output_projection(dtype, a, Wo, w3, out, B * N, H_q * d_head, d_model, lens, N,
                                      stream);
  const hipError_t ef = wsp.release();
  if (e != hipSuccess) return fail_hip(e, "kernel launch");
  if (ef != hipSuccess) return fail_hip(ef, "workspace release");
  return ok();
}

sqa_status backward_impl(const void* x, const void* Wq, const void* Wk, const void* Wv,
                         const void* Wo, const void* dy, const void* saved, size_t saved_bytes,
                         void* dx, void* dWq, void* dWk, void* dWv,
                         void* dWo, int64_t B, int64_t N, int64_t d_model, int64_t H, int64_t H_q,
                         int64_t H_kv, int64_t d_head, int causal, sqa_dtype dtype,
                         hipStream_t stream) {
  const Shape s{B, N, d_model, H, H_q, H_kv, d_head};
  SQA_TRY(check_dtype(dtype));
  SQA_TRY(check_heads(s, true));
  if (causal != 0 && causal != 1) return fail(SQA_ERR_INVALID_ARG, "causal must be 0 or 1");
  if (B * N == 0) return ok();
  const void* ins[6] = {x, Wq, Wk, Wv, Wo, dy};
  const char* in_names[6] = {"x", "Wq", "Wk", "Wv", "Wo", "dy"};
  void* outs[5] = {dx, dWq, dWk, dWv, dWo};
  const char* out_names[5] = {"dx", "dWq", "dWk", "dWv", "dWo"};
  char msg[64];
  for (int j = 0; j < 6; ++j) {
    snprintf(msg, sizeof(msg), "%s is null or not 16-byte aligned", in_names[j]);
    if (!ins[j] || !aligned16(ins[j])) return fail(SQA_ERR_INVALID_ARG, msg);
  }
  for (int j = 0; j < 5; ++j) {
    snprintf(msg, sizeof(msg), "%s is null or not 16-byte aligned", out_names[j]);
    if (!outs[j] || !aligned16(outs[j])) return fail(SQA_ERR_INVALID_ARG, msg);
  }
  Sizes z;
  SQA_TRY(sizes_for(s, dtype, &z));
  const int64_t es = (int64_t)elem_size(dtype);
  // the largest workspace regions are token-major copies of widths up to
  // d_model + (H_q + 2 H_kv) d_head; keep every byte count far from overflow
  int64_t t;
  if (!mul_ok(B, z.Np, &t) || !mul_ok(t, d_model + (H_q + 2 * H_kv) * d_head, &t) ||
      !mul_ok(t, 64 * es, &t))
    return fail(SQA_ERR_UNSUPPORTED, "size overflow");
  const size_t xb = (size_t)(B * N * d_model * es);
  const size_t wqb = (size_t)(d_model * H_q * d_head * es), wkb = (size_t)(d_model * H_kv * d_head * es);
  const size_t inb[6] = {xb, wqb, wkb, wkb, wqb, xb};
  const size_t outb[5] = {xb, wqb, wkb, wkb, wqb};
  for (int j = 0; j < 5; ++j) {
    for (int i = 0; i < 6; ++i)
      if (overlap(outs[j], outb[j], ins[i], inb[i]))
        return fail(SQA_ERR_INVALID_ARG, "an output overlaps an input");
    for (int i = 0; i < j; ++i)
      if (overlap(outs[j], outb[j], outs[i], outb[i]))
        return fail(SQA_ERR_INVALID_ARG, "two outputs overlap");
  }
  if (saved) SQA_TRY(check_saved(saved, saved_bytes, s, dtype, outs, outb, 5));
  Workspace ws;
  SQA_TRY(ws.acquire(sqa::backward_workspace_bytes(dtype, B, N, z.Np, d_model, H_q, H_kv, d_head,
                                                   saved != nullptr, causal != 0),
                     stream));
  const hipError_t e = sqa::launch_backward(dtype, x, Wq, Wk, Wv, Wo, dy, saved, dx, dWq, dWk, dWv, dWo,
                                            B, N, z.Np, d_model, H_q, H_kv, d_head, causal != 0,
                                            ws.ptr, stream);
  const hipError_t ef = ws.release();
  if (e != hipSuccess) return fail_hip(e, "kernel launch");
  if (ef != hipSuccess) return fail_hip(ef, "workspace release");
  return ok();
}

}  // namespace

extern "C" {

const char* sqa_status_string(sqa_status s) {
  switch (s) {
    case SQA_OK: return "SQA_OK";
    case SQA_ERR_INVALID_ARG: return "SQA_ERR_INVALID_ARG: invalid argument";
    case SQA_ERR_UNSUPPORTED: return "SQA_ERR_UNSUPPORTED: configuration not supported";
    case SQA_ERR_HIP: return "SQA_ERR_HIP: a HIP runtime call failed";
    case SQA_ERR_OUT_OF_MEMORY: return "SQA_ERR_OUT_OF_MEMORY: workspace allocation failed";
  }
  return "unknown sqa_status";
}

const char* sqa_last_error_message(void) { return g_err; }

int64_t sqa_padded_length(int64_t N) { return N < 0 ? -1 : sqa::padded_length(N); }

sqa_status sqa_qkv_projection(const void* x, const void* Wq, const void* Wk, const void* Wv,
                              void* q, void* k, void* vt, int64_t B, int64_t N, int64_t d_model,
                              int64_t H, int64_t H_q, int64_t H_kv, int64_t d_head,
                              sqa_dtype dtype, hipStream_t stream) {
  const Shape s{B, N, d_model, H, H_q, H_kv, d_head};
  SQA_TRY(check_dtype(dtype));
  SQA_TRY(check_heads(s, true));
  if (B * N == 0) return ok();
  SQA_TRY(check_ptr(x, "x is null", "x is not 16-byte aligned"));
  SQA_TRY(check_ptr(Wq, "Wq is null", "Wq is not 16-byte aligned"));
  SQA_TRY(check_ptr(Wk, "Wk is null", "Wk is not 16-byte aligned"));
  SQA_TRY(check_ptr(Wv, "Wv is null", "Wv is not 16-byte aligned"));
  SQA_TRY(check_ptr(q, "q is null", "q is not 16-byte aligned"));
  SQA_TRY(check_ptr(k, "k is null", "k is not 16-byte aligned"));
  SQA_TRY(check_ptr(vt, "vt is null", "vt is not 16-byte aligned"));
  Sizes z;
  SQA_TRY(sizes_for(s, dtype, &z));
  const size_t es = elem_size(dtype);
  const size_t xb = (size_t)(B * N * d_model) * es;
  const size_t wqb = (size_t)(d_model * H_q * d_head) * es, wkb = (size_t)(d_model * H_kv * d_head) * es;
  const void* ins[4] = {x, Wq, Wk, Wv};
  const size_t inb[4] = {xb, wqb, wkb, wkb};
  void* outs[3] = {q, k, vt};
  const size_t outb[3] = {(size_t)z.q, (size_t)z.kv, (size_t)z.kv};
  for (int i = 0; i < 3; ++i) {
    for (int j = 0; j < 4; ++j)
      if (overlap(outs[i], outb[i], ins[j], inb[j]))
        return fail(SQA_ERR_INVALID_ARG, "an output of the projection overlaps an input");
    for (int j = i + 1; j < 3; ++j)
      if (overlap(outs[i], outb[i], outs[j], outb[j]))
        return fail(SQA_ERR_INVALID_ARG, "q, k and vt must not overlap");
  }
  Workspace wt;
  SQA_TRY(wt.acquire(sqa::qkv_wt_bytes(dtype, d_model, H_q, H_kv, d_head), stream));
  hipError_t e = sqa::launch_qkv_projection(dtype, x, Wq, Wk, Wv, wt.ptr, q, k, vt, B, N, z.Np,
                                            d_model, H_q, H_kv, d_head, nullptr, stream);
  const hipError_t ef = wt.release();
  if (e != hipSuccess) return fail_hip(e, "qkv projection launch");
  if (ef != hipSuccess) return fail_hip(ef, "scratch release");
  return ok();
}

sqa_status sqa_attention(const void* q, const void* k, const void* vt, void* a, int64_t B,
                         int64_t N, int64_t H_q, int64_t H_kv, int64_t d_head, int causal,
                         sqa_dtype dtype, hipStream_t stream) {
  const Shape s{B, N, H_q * d_head, H_q, H_q, H_kv, d_head};
  SQA_TRY(check_dtype(dtype));
  SQA_TRY(check_heads(s, false));
  if (causal != 0 && causal != 1) return fail(SQA_ERR_INVALID_ARG, "causal must be 0 or 1");
  if (B * N == 0) return ok();
  SQA_TRY(check_ptr(q, "q is null", "q is not 16-byte aligned"));
  SQA_TRY(check_ptr(k, "k is null", "k is not 16-byte aligned"));
  SQA_TRY(check_ptr(vt, "vt is null", "vt is not 16-byte aligned"));
  SQA_TRY(check_ptr(a, "a is null", "a is not 16-byte aligned"));
  Sizes z;
  SQA_TRY(sizes_for(s, dtype, &z));
  if (overlap(a, z.a, q, z.q) || overlap(a, z.a, k, z.kv) || overlap(a, z.a, vt, z.kv))
    return fail(SQA_ERR_INVALID_ARG, "a overlaps q, k or vt");
  Workspace ws;   // the key-split parts of a partial last round, if any
  const size_t split_b =
      sqa::attention_split_bytes(dtype, B, N, H_q, H_kv, d_head, causal != 0, false, stream);
  if (split_b > 0) SQA_TRY(ws.acquire(split_b, stream));
  hipError_t e = sqa::launch_attention(dtype, q, k, vt, a, B, N, z.Np, H_q, H_kv, d_head,
                                       causal != 0, nullptr, stream, nullptr, nullptr, nullptr,
                                       (float*)ws.ptr);
  const hipError_t ef = ws.release();
  if (e != hipSuccess) return fail_hip(e, "attention launch");
  if (ef != hipSuccess) return fail_hip(ef, "workspace release");
  return ok();
}

sqa_status sqa_output_projection(const void* a, const void* Wo, void* out, int64_t M, int64_t K,
                                 int64_t d_model, sqa_dtype dtype, hipStream_t stream) {
  SQA_TRY(check_dtype(dtype));
  if (M < 0) return fail(SQA_ERR_INVALID_ARG, "M must be >= 0");
  if (K < 32 || K % 32 != 0) return fail(SQA_ERR_UNSUPPORTED, "K must be a positive multiple of 32");
  if (d_model < 32 || d_model % 32 != 0)
    return fail(SQA_ERR_UNSUPPORTED, "d_model must be a positive multiple of 32");
  if (K > 65536 || d_model > 65536) return fail(SQA_ERR_UNSUPPORTED, "K or d_model exceeds 65536");
  if (M > ((int64_t)1 << 40)) return fail(SQA_ERR_UNSUPPORTED, "M too large");
  if (M == 0) return ok();
  SQA_TRY(check_ptr(a, "a is null", "a is not 16-byte aligned"));
  SQA_TRY(check_ptr(Wo, "Wo is null", "Wo is not 16-byte aligned"));
  SQA_TRY(check_ptr(out, "out is null", "out is not 16-byte aligned"));
  const size_t es = elem_size(dtype);
  if (overlap(out, (size_t)(M * d_model) * es, a, (size_t)(M * K) * es) ||
      overlap(out, (size_t)(M * d_model) * es, Wo, (size_t)(K * d_model) * es))
    return fail(SQA_ERR_INVALID_ARG, "out overlaps a or Wo");
  Workspace wt;
  SQA_TRY(wt.acquire(sqa::out_wt_bytes(dtype, K, d_model), stream));
  hipError_t e = sqa::launch_output_projection(dtype, a, Wo, wt.ptr, out, M, K, d_model, nullptr, 1,
                                               stream);
  const hipError_t ef = wt.release();
  if (e != hipSuccess) return fail_hip(e, "output projection launch");
  if (ef != hipSuccess) return fail_hip(ef, "scratch release");
  return ok();
}

sqa_status sqa_forward(const void* x, const void* Wq, const void* Wk, const void* Wv,
                       const void* Wo, void* out, int64_t B, int64_t N, int64_t d_model,
                       int64_t H, int64_t H_q, int64_t H_kv, int64_t d_head, int causal,
                       sqa_dtype dtype, hipStream_t stream) {
  return forward_impl(x, Wq, Wk, Wv, Wo, out, false, nullptr, nullptr, nullptr, 0, B, N, d_model, H, H_q, H_kv, d_head, causal,
                      dtype, stream);
}

sqa_status sqa_forward_noalloc(const void* x, const void* Wq, const void* Wk, const void* Wv,
                               const void* Wo, void* out, int64_t B, int64_t N, int64_t d_model,
                               int64_t H, int64_t H_q, int64_t H_kv, int64_t d_head, int causal,
                               sqa_dtype dtype, hipStream_t stream) {
  return forward_impl(x, Wq, Wk, Wv, Wo, out, false, nullptr, nullptr, nullptr, 0, B, N, d_model,
                      H, H_q, H_kv, d_head, causal, dtype, stream, nullptr, 0, true);
}

sqa_status sqa_forward_varlen(const void* x, const void* Wq, const void* Wk, const void* Wv,
                              const void* Wo, void* out, const int32_t* lens, int64_t B, int64_t N,
                              int64_t d_model, int64_t H, int64_t H_q, int64_t H_kv,
                              int64_t d_head, int causal, sqa_dtype dtype, hipStream_t stream) {
  return forward_impl(x, Wq, Wk, Wv, Wo, out, true, lens, nullptr, nullptr, 0, B, N, d_model, H, H_q, H_kv, d_head, causal,
                      dtype, stream);
}

sqa_status sqa_prefill(const void* x, const void* Wq, const void* Wk, const void* Wv,
                       const void* Wo, void* out, void* k_cache, void* v_cache, int64_t B,
                       int64_t N, int64_t N_max, int64_t d_model, int64_t H, int64_t H_q,
                       int64_t H_kv, int64_t d_head, sqa_dtype dtype, hipStream_t stream) {
  if (N_max < 1 || N_max > SQA_MAX_N) return fail(SQA_ERR_UNSUPPORTED, "N_max must be in [1, SQA_MAX_N]");
  if (B * N != 0) {
    SQA_TRY(check_ptr(k_cache, "k_cache is null", "k_cache is not 16-byte aligned"));
    SQA_TRY(check_ptr(v_cache, "v_cache is null", "v_cache is not 16-byte aligned"));
  }
  return forward_impl(x, Wq, Wk, Wv, Wo, out, false, nullptr, k_cache, v_cache, N_max, B, N,
                      d_model, H, H_q, H_kv, d_head, 1, dtype, stream);
}

size_t sqa_training_saved_bytes(int64_t B, int64_t N, int64_t H_q, int64_t H_kv, int64_t d_head,
                                sqa_dtype dtype) {
  const Shape s{B, N, H_q * d_head, H_q, H_q, H_kv, d_head};
  if (check_dtype(dtype) != SQA_OK || check_heads(s, false) != SQA_OK) return 0;
  Sizes z;
  if (sizes_for(s, dtype, &z) != SQA_OK) return 0;
  return (size_t)sqa::saved_layout((int64_t)elem_size(dtype), B, N, z.Np, H_q, H_kv, d_head).total;
}

sqa_status sqa_forward_train(const void* x, const void* Wq, const void* Wk, const void* Wv,
                             const void* Wo, void* out, void* saved, size_t saved_bytes, int64_t B,
                             int64_t N, int64_t d_model, int64_t H, int64_t H_q, int64_t H_kv,
                             int64_t d_head, int causal, sqa_dtype dtype, hipStream_t stream) {
  if (B * N != 0 && !saved) return fail(SQA_ERR_INVALID_ARG, "saved is null");
  return forward_impl(x, Wq, Wk, Wv, Wo, out, false, nullptr, nullptr, nullptr, 0, B, N, d_model,
                      H, H_q, H_kv, d_head, causal, dtype, stream, saved, saved_bytes);
}

sqa_status sqa_backward(const void* x, const void* Wq, const void* Wk, const void* Wv,
                        const void* Wo, const void* dy, const void* saved, size_t saved_bytes,
                        void* dx, void* dWq, void* dWk, void* dWv, void* dWo, int64_t B, int64_t N,
                        int64_t d_model, int64_t H, int64_t H_q, int64_t H_kv, int64_t d_head,
                        int causal, sqa_dtype dtype, hipStream_t stream) {
  return backward_impl(x, Wq, Wk, Wv, Wo, dy, saved, saved_bytes, dx, dWq, dWk, dWv, dWo, B, N,
                       d_model, H, H_q, H_kv, d_head, causal, dtype, stream);
}

sqa_status sqa_decode_step(const void* x_new, const void* Wq, const void* Wk, const void* Wv,
                           const void* Wo, void* out, void* k_cache, void* v_cache,
                           const int32_t* pos, int64_t B, int64_t N_max, int64_t d_model,
                           int64_t H, int64_t H_q, int64_t H_kv, int64_t d_head, sqa_dtype dtype,
                           hipStream_t stream) {
  // Shape checks as for one sequence of B tokens (head counts, d_head, sizes).
  const Shape s{1, B, d_model, H, H_q, H_kv, d_head};
  SQA_TRY(check_dtype(dtype));
  SQA_TRY(check_heads(s, true));
  if (N_max < 1 || N_max > SQA_MAX_N) return fail(SQA_ERR_UNSUPPORTED, "N_max must be in [1, SQA_MAX_N]");
  if (B > 65535) return fail(SQA_ERR_UNSUPPORTED, "B exceeds 65535 for a decode step");
  if (B == 0) return ok();
  SQA_TRY(check_ptr(x_new, "x_new is null", "x_new is not 16-byte aligned"));
  SQA_TRY(check_ptr(Wq, "Wq is null", "Wq is not 16-byte aligned"));
  SQA_TRY(check_ptr(Wk, "Wk is null", "Wk is not 16-byte aligned"));
  SQA_TRY(check_ptr(Wv, "Wv is null", "Wv is not 16-byte aligned"));
  SQA_TRY(check_ptr(Wo, "Wo is null", "Wo is not 16-byte aligned"));
  SQA_TRY(check_ptr(out, "out is null", "out is not 16-byte aligned"));
  SQA_TRY(check_ptr(k_cache, "k_cache is null", "k_cache is not 16-byte aligned"));
  SQA_TRY(check_ptr(v_cache, "v_cache is null", "v_cache is not 16-byte aligned"));
  if (!pos) return fail(SQA_ERR_INVALID_ARG, "pos is null");
  if (reinterpret_cast<uintptr_t>(pos) & 3u) return fail(SQA_ERR_INVALID_ARG, "pos is not 4-byte aligned");
  Sizes z;
  SQA_TRY(sizes_for(s, dtype, &z));
  const size_t es = elem_size(dtype);
  int64_t cb;
  if (!mul_ok(B * H_kv, N_max, &cb) || !mul_ok(cb, d_head * (int64_t)es, &cb))
    return fail(SQA_ERR_UNSUPPORTED, "size overflow");
  const size_t yb = (size_t)(B * d_model) * es;
  const size_t wqb = (size_t)(d_model * H_q * d_head) * es, wkb = (size_t)(d_model * H_kv * d_head) * es;
  const void* ins[6] = {x_new, Wq, Wk, Wv, Wo, pos};
  const size_t inb[6] = {yb, wqb, wkb, wkb, wqb, (size_t)B * sizeof(int32_t)};
  for (int j = 0; j < 6; ++j) {
    if (overlap(out, yb, ins[j], inb[j])) return fail(SQA_ERR_INVALID_ARG, "out overlaps an input");
    if (overlap(k_cache, (size_t)cb, ins[j], inb[j]) || overlap(v_cache, (size_t)cb, ins[j], inb[j]))
      return fail(SQA_ERR_INVALID_ARG, "a cache overlaps an input");
  }
  if (overlap(k_cache, (size_t)cb, v_cache, (size_t)cb)) return fail(SQA_ERR_INVALID_ARG, "k_cache overlaps v_cache");
  if (overlap(out, yb, k_cache, (size_t)cb) || overlap(out, yb, v_cache, (size_t)cb))
    return fail(SQA_ERR_INVALID_ARG, "out overlaps a cache");

  // Workspace: q and a [B, H_q*d_head], then the decode attention's fp32
  // partial states of its key chunks.
  const int64_t qa_b = B * H_q * d_head * (int64_t)es;
  const int64_t scratch_b = (int64_t)sqa::decode_partial_bytes(dtype, B, H_q, H_kv, N_max, d_head);
  const int64_t off_a = round256(qa_b), off_p = off_a + round256(qa_b);
  const int64_t total = off_p + round256(scratch_b);
  Workspace ws;
  SQA_TRY(ws.acquire((size_t)total, stream));
  char* base = (char*)ws.ptr;
  void *q = base, *a = base + off_a, *part = base + off_p;
  hipError_t e;
  e = sqa::launch_decode_qkv(dtype, x_new, Wq, Wk, Wv, pos, q, k_cache, v_cache, B, d_model, H_q,
                             H_kv, d_head, N_max, stream);
  // The merge of the attention's key chunks runs inside the output
  // projection where its LDS row fits, else as a launch of its own.
  const bool fused = sqa::decode_merge_out_fits(dtype, B, N_max, H_q, H_kv, d_head, d_model);
  if (e == hipSuccess)
    e = sqa::launch_decode_attention(dtype, q, k_cache, v_cache, pos, fused ? nullptr : a, part, B,
                                     N_max, H_q, H_kv, d_head, stream);
  if (e == hipSuccess)
    e = fused ? sqa::launch_decode_merge_out(dtype, part, pos, Wo, out, B, N_max, H_q, H_kv, d_head,
                                             d_model, stream)
              : sqa::launch_decode_out(dtype, a, Wo, out, B, H_q * d_head, d_model, stream);
  const hipError_t ef = ws.release();
  if (e != hipSuccess) return fail_hip(e, "kernel launch");
  if (ef != hipSuccess) return fail_hip(ef, "workspace release");
  return ok();
}

}  // extern "C"
