// ssd_api.hip -- the C ABI of libssd: argument validation, algorithm choice,
// scratch management and kernel launches.  Declarations and the contract
// are in include/ssd.h.
//
// Every check runs on the host before the first HIP call, so a rejected
// call has no side effect on the device and can be exercised without a GPU.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <algorithm>
#include <atomic>
#include <cmath>
#include <mutex>
#include <string>
#include <vector>

#include "ssd.h"
#include "ssd_internal.h"

// Scratch of the allocation-free entry point ssd_scan_fwd_noalloc: a fixed
// array in the code object's device memory, one copy per device, kept until
// the process ends.  Host code never passes the array's name to a kernel (in
// host code it is a stand-in, not a device address): it takes the device
// address with hipGetSymbolAddress once per device (fixed_scratch_ptr).
#define SSD_FIXED_SCRATCH_BYTES ((size_t)64 << 20)
static __device__ __align__(256) unsigned char scratch[SSD_FIXED_SCRATCH_BYTES];

namespace {

thread_local std::string g_last_error;

int fail(int status, const char *fmt, ...) __attribute__((format(printf, 2, 3)));
int fail(int status, const char *fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return status;
}

int elem_size(int dtype) { return dtype == SSD_BF16 ? 2 : 4; }

int64_t numel(const ssd_tensor *t) {
  int64_t n = 1;
  for (int i = 0; i < t->ndim; ++i) n *= t->shape[i];
  return n;
}

struct Range {
  uintptr_t lo = 0, hi = 0; // [lo, hi)
  bool empty() const { return hi <= lo; }
};

Range range_of(const ssd_tensor *t) {
  Range r;
  if (!t || !t->data) return r;
  r.lo = (uintptr_t)t->data;
  r.hi = r.lo + (uintptr_t)(numel(t) * elem_size(t->dtype));
  return r;
}

bool overlap(const Range &a, const Range &b) {
  return !a.empty() && !b.empty() && a.lo < b.hi && b.lo < a.hi;
}

// Checks presence, dtype, rank, exact shape, dense row-major strides and
// 16-byte alignment.  `want_dtype` < 0 accepts f32 or bf16.
int check_tensor(const ssd_tensor *t, const char *name, int want_dtype, int ndim,
                 const int64_t *shape) {
  if (!t) return fail(SSD_ERR_NULL, "%s: descriptor is NULL", name);
  if (!t->data) return fail(SSD_ERR_NULL, "%s: data pointer is NULL", name);
  if (t->dtype != SSD_F32 && t->dtype != SSD_BF16)
    return fail(SSD_ERR_DTYPE, "%s: unknown dtype %d", name, t->dtype);
  if (want_dtype >= 0 && t->dtype != want_dtype)
    return fail(SSD_ERR_DTYPE, "%s: dtype %s, expected %s", name,
                t->dtype == SSD_BF16 ? "bf16" : "f32", want_dtype == SSD_BF16 ? "bf16" : "f32");
  if (t->ndim != ndim)
    return fail(SSD_ERR_SHAPE, "%s: rank %d, expected %d", name, t->ndim, ndim);
  for (int i = 0; i < ndim; ++i)
    if (t->shape[i] != shape[i])
      return fail(SSD_ERR_SHAPE, "%s: dim %d is %lld, expected %lld", name, i,
                  (long long)t->shape[i], (long long)shape[i]);
  int64_t stride = 1;
  for (int i = ndim - 1; i >= 0; --i) {
    if (t->shape[i] != 1 && t->strides[i] != stride)
      return fail(SSD_ERR_LAYOUT, "%s: stride of dim %d is %lld, expected %lld (dense row-major)",
                  name, i, (long long)t->strides[i], (long long)stride);
    stride *= t->shape[i];
  }
  if (((uintptr_t)t->data) % 16 != 0)
    return fail(SSD_ERR_LAYOUT, "%s: data pointer is not 16-byte aligned", name);
  return SSD_OK;
}

#define SSD_CHECK(expr)                                                                   \
  do {                                                                                    \
    int _s = (expr);                                                                      \
    if (_s != SSD_OK) return _s;                                                          \
  } while (0)

bool valid_pn(int64_t v) { return v == 16 || v == 32 || v == 64 || v == 128; }

constexpr int64_t kMaxL = (int64_t)1 << 24;   // tokens per sequence
constexpr int64_t kMaxRow = (int64_t)1 << 22; // elements of x (H*P) or B/C (G*N) per token

struct ScanShape {
  int64_t b, L, H, P, G, N;
};

int validate_scan(const ssd_tensor *x, const ssd_tensor *dt, const ssd_tensor *dt_bias,
                  const ssd_tensor *A, const ssd_tensor *B, const ssd_tensor *C,
                  const ssd_tensor *D, const ssd_tensor *init, const ssd_tensor *out,
                  const ssd_tensor *fin, int chunk, ScanShape *s, const char *out_name = "out",
                  bool out_written = true) {
  if (!x) return fail(SSD_ERR_NULL, "x: descriptor is NULL");
  if (!B) return fail(SSD_ERR_NULL, "B: descriptor is NULL");
  if (x->ndim != 4) return fail(SSD_ERR_SHAPE, "x: rank %d, expected 4 [b,L,H,P]", x->ndim);
  if (B->ndim != 4) return fail(SSD_ERR_SHAPE, "B: rank %d, expected 4 [b,L,G,N]", B->ndim);
  s->b = x->shape[0]; s->L = x->shape[1]; s->H = x->shape[2]; s->P = x->shape[3];
  s->G = B->shape[2]; s->N = B->shape[3];
  if (s->b < 1 || s->L < 1 || s->H < 1 || s->G < 1)
    return fail(SSD_ERR_SHAPE, "empty problem: b=%lld L=%lld H=%lld G=%lld", (long long)s->b,
                (long long)s->L, (long long)s->H, (long long)s->G);
  if (s->H % s->G != 0)
    return fail(SSD_ERR_SHAPE, "H=%lld is not a multiple of G=%lld", (long long)s->H, (long long)s->G);
  if (!valid_pn(s->P)) return fail(SSD_ERR_UNSUPPORTED, "P=%lld not in {16,32,64,128}", (long long)s->P);
  if (!valid_pn(s->N)) return fail(SSD_ERR_UNSUPPORTED, "N=%lld not in {16,32,64,128}", (long long)s->N);
  if (x->dtype == SSD_F32 && s->P > 64)
    return fail(SSD_ERR_UNSUPPORTED, "P=%lld with fp32 inputs: fp32 supports P in {16,32,64}", (long long)s->P);
  if (chunk < 64 || chunk > 65536 || (chunk & (chunk - 1)) != 0)
    return fail(SSD_ERR_UNSUPPORTED, "chunk=%d is not a power of two in [64, 65536]", chunk);
  if (s->b * s->L * s->H * s->P > ((int64_t)1 << 40) || s->b * s->L > INT32_MAX / 2 ||
      s->b * s->H * ((s->L + 63) / 64) > INT32_MAX / 2)
    return fail(SSD_ERR_UNSUPPORTED, "problem too large for 32-bit workgroup indexing");
  // Kernels address one 64-token tile (and the row walk one sequence of
  // score tiles) through 32-bit byte ranges.
  if (s->L > kMaxL)
    return fail(SSD_ERR_UNSUPPORTED, "L=%lld above the supported %lld tokens", (long long)s->L,
                (long long)kMaxL);
  if (s->H * s->P > kMaxRow || s->G * s->N > kMaxRow)
    return fail(SSD_ERR_UNSUPPORTED, "H*P=%lld or G*N=%lld above the supported %lld per token",
                (long long)(s->H * s->P), (long long)(s->G * s->N), (long long)kMaxRow);
  const int xd = x->dtype;
  const int64_t sx[4] = {s->b, s->L, s->H, s->P}, sdt[3] = {s->b, s->L, s->H},
                sh[1] = {s->H}, sbc[4] = {s->b, s->L, s->G, s->N},
                sst[4] = {s->b, s->H, s->P, s->N};
  SSD_CHECK(check_tensor(x, "x", -1, 4, sx));
  SSD_CHECK(check_tensor(dt, "dt", SSD_F32, 3, sdt));
  if (dt_bias) SSD_CHECK(check_tensor(dt_bias, "dt_bias", SSD_F32, 1, sh));
  SSD_CHECK(check_tensor(A, "A", SSD_F32, 1, sh));
  SSD_CHECK(check_tensor(B, "B", xd, 4, sbc));
  SSD_CHECK(check_tensor(C, "C", xd, 4, sbc));
  if (D) SSD_CHECK(check_tensor(D, "D", SSD_F32, 1, sh));
  if (init) SSD_CHECK(check_tensor(init, "init_state", SSD_F32, 4, sst));
  SSD_CHECK(check_tensor(out, out_name, xd, 4, sx));
  if (fin) SSD_CHECK(check_tensor(fin, "final_state", SSD_F32, 4, sst));
  if (!out_written) return SSD_OK;

  const Range ro = range_of(out), rf = range_of(fin);
  const ssd_tensor *ins[] = {x, dt, dt_bias, A, B, C, D, init};
  const char *names[] = {"x", "dt", "dt_bias", "A", "B", "C", "D", "init_state"};
  for (int i = 0; i < 8; ++i) {
    const Range ri = range_of(ins[i]);
    if (overlap(ro, ri)) return fail(SSD_ERR_ALIAS, "out overlaps %s", names[i]);
    if (i == 7 && fin && init && fin->data == init->data) continue; // in-place state
    if (overlap(rf, ri)) return fail(SSD_ERR_ALIAS, "final_state overlaps %s", names[i]);
  }
  if (overlap(ro, rf)) return fail(SSD_ERR_ALIAS, "out overlaps final_state");
  return SSD_OK;
}

int hip_fail(hipError_t e, const char *what) {
  return fail(SSD_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

// Scratch memory.  A stream-ordered allocate/free pair on every call makes the
// host wait inside the runtime for the stream's earlier work (measured on
// MI355X: about 160 us of host time per scan call of the 2.7B layer, as long
// as the scan, so the GPU idled between back-to-back calls).  The library
// instead keeps one buffer per (device, stream) and hands it to every call on
// that stream, which uses it in stream order.  An event recorded after the
// call's last launch, and waited on by the next call that takes the buffer,
// also orders uses when a destroyed stream's handle is handed out again (or
// when one handle names several streams, as the per-thread default stream
// does).  A buffer grows, stream-ordered, to the largest request up to
// kScratchKeepMax; a larger request is allocated and freed on the stream for
// that call alone.  At most kScratchSlots buffers holding at most
// kScratchTotal bytes are kept: a call that needs a new one first frees the
// least recently used idle buffers (after waiting for their last use) until
// both limits hold.  ssd_release_scratch() frees every kept buffer.
constexpr size_t kScratchKeepMax = (size_t)4 << 30;
constexpr size_t kScratchGranule = (size_t)1 << 20;
constexpr size_t kScratchSlots = 16;
constexpr size_t kScratchTotal = (size_t)8 << 30;

struct ScratchSlot {
  int dev;
  hipStream_t st;
  int tag;
  void *p;
  size_t cap;
  hipEvent_t done;
  bool pending;       // done has been recorded after the last use
  bool busy;          // held by a call in progress (this thread, an outer call)
  uint64_t last_use;  // for least-recently-used eviction
};

// Recursive: a call may hold one buffer (tag 1) while the calls it makes take
// another (tag 0) on the same stream.
std::recursive_mutex g_scratch_mu;
std::vector<ScratchSlot> g_scratch;
uint64_t g_scratch_clock = 0;

// The allocation-free entry point points every call it makes at the fixed
// device array instead (set for the duration of that call on this thread).
struct FixedScratch {
  void *p = nullptr;
  size_t cap = 0;
};
thread_local FixedScratch g_fixed;

// Frees slot i (waiting for its last use first) and removes it.  Called with
// the lock held.
int drop_slot(size_t i) {
  ScratchSlot s = g_scratch[i];
  g_scratch.erase(g_scratch.begin() + (ptrdiff_t)i);
  int cur = 0;
  hipError_t e = hipGetDevice(&cur);
  if (e != hipSuccess) return hip_fail(e, "scratch eviction: current device");
  int status = SSD_OK;
  e = hipSetDevice(s.dev);
  if (e == hipSuccess && s.pending) e = hipEventSynchronize(s.done);
  if (e == hipSuccess && s.p) e = hipFree(s.p);
  if (e == hipSuccess) e = hipEventDestroy(s.done);
  if (e != hipSuccess) status = hip_fail(e, "scratch eviction");
  e = hipSetDevice(cur);
  if (e != hipSuccess && status == SSD_OK) status = hip_fail(e, "scratch eviction: restore device");
  return status;
}

// Evicts idle slots, least recently used first, until `more_slots` more
// slots and `more_bytes` more bytes fit both limits.  Called with the lock
// held.
int make_room(size_t more_slots, size_t more_bytes) {
  for (;;) {
    size_t total = more_bytes;
    for (const ScratchSlot &s : g_scratch) total += s.cap;
    if (g_scratch.size() + more_slots <= kScratchSlots && total <= kScratchTotal) return SSD_OK;
    size_t victim = g_scratch.size();
    for (size_t i = 0; i < g_scratch.size(); ++i)
      if (!g_scratch[i].busy && (victim == g_scratch.size() || g_scratch[i].last_use < g_scratch[victim].last_use))
        victim = i;
    if (victim == g_scratch.size()) return SSD_OK; // every kept buffer is in use by this thread
    SSD_CHECK(drop_slot(victim));
  }
}

// One call's scratch.  get() returns the buffer; the lock on the kept
// buffers is held from get() until finish() (or destruction), so the event
// is recorded after the call's launches and before another call takes the
// buffer.
class Scratch {
public:
  explicit Scratch(hipStream_t st, int tag = 0) : st_(st), tag_(tag) {}
  Scratch(const Scratch &) = delete;
  Scratch &operator=(const Scratch &) = delete;
  ~Scratch() { (void)finish(); }

  int get(size_t bytes, void **out) {
    *out = nullptr;
    if (g_fixed.p) {
      // allocation-free call: the fixed array, shared by every such call on
      // this device
      if (bytes > g_fixed.cap)
        return fail(SSD_ERR_NOMEM, "this call needs %zu bytes of scratch; the fixed scratch array holds %zu",
                    bytes, g_fixed.cap);
      *out = g_fixed.p;
      return SSD_OK;
    }
    if (bytes > kScratchKeepMax) {
      const hipError_t e = hipMallocAsync(&own_, bytes, st_);
      if (e != hipSuccess || !own_) {
        (void)hipGetLastError();
        own_ = nullptr;
        return fail(SSD_ERR_NOMEM, "scratch of %zu bytes: %s", bytes, hipGetErrorString(e));
      }
      *out = own_;
      return SSD_OK;
    }
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e, "scratch: current device");
    lock_ = std::unique_lock<std::recursive_mutex>(g_scratch_mu);
    const size_t want = (bytes + kScratchGranule - 1) / kScratchGranule * kScratchGranule;
    size_t i = 0;
    while (i < g_scratch.size() &&
           !(g_scratch[i].dev == dev && g_scratch[i].st == st_ && g_scratch[i].tag == tag_))
      ++i;
    if (i == g_scratch.size()) {
      SSD_CHECK(make_room(1, want));
      hipEvent_t ev = nullptr;
      // No system-scope fence: the event orders later device work on the
      // same device (and the host's wait before a free), so a device-scope
      // release suffices; the system-scope one writes back the L2 at every
      // call end (about 2 us per back-to-back 2.7B-layer call).
      e = hipEventCreateWithFlags(&ev, hipEventDisableTiming | hipEventDisableSystemFence);
      if (e != hipSuccess) return hip_fail(e, "scratch: event");
      g_scratch.push_back(ScratchSlot{dev, st_, tag_, nullptr, 0, ev, false, false, 0});
      i = g_scratch.size() - 1;
    } else if (g_scratch[i].cap < bytes) {
      // growing: keep the other buffers within the byte limit
      g_scratch[i].busy = true;
      int st = make_room(0, want - g_scratch[i].cap);
      g_scratch[i].busy = false;
      SSD_CHECK(st);
      while (i < g_scratch.size() &&
             !(g_scratch[i].dev == dev && g_scratch[i].st == st_ && g_scratch[i].tag == tag_))
        ++i;
      if (i == g_scratch.size()) return fail(SSD_ERR_NOMEM, "scratch: slot lost while growing");
    }
    ScratchSlot &s = g_scratch[i];
    if (s.pending) {
      e = hipStreamWaitEvent(st_, s.done, 0);
      if (e != hipSuccess) return hip_fail(e, "scratch: wait for its last use");
    }
    if (s.cap < bytes) {
      if (s.p) {
        e = hipFreeAsync(s.p, st_);
        s.p = nullptr;
        s.cap = 0;
        if (e != hipSuccess) return hip_fail(e, "scratch: free to grow");
      }
      e = hipMallocAsync(&s.p, want, st_);
      if (e != hipSuccess || !s.p) {
        (void)hipGetLastError();
        s.p = nullptr;
        return fail(SSD_ERR_NOMEM, "scratch of %zu bytes: %s", want, hipGetErrorString(e));
      }
      s.cap = want;
    }
    s.busy = true;
    s.last_use = ++g_scratch_clock;
    slot_dev_ = dev;
    slot_st_ = st_;
    slot_ = 1;
    *out = s.p;
    return SSD_OK;
  }

  // After the launches that use the buffer.
  int finish() {
    int status = SSD_OK;
    if (own_) {
      const hipError_t e = hipFreeAsync(own_, st_);
      own_ = nullptr;
      if (e != hipSuccess) status = hip_fail(e, "scratch free");
    }
    if (slot_ >= 0) {
      // find the slot again: a nested call may have evicted others meanwhile
      for (ScratchSlot &s : g_scratch) {
        if (s.dev == slot_dev_ && s.st == slot_st_ && s.tag == tag_) {
          const hipError_t e = hipEventRecord(s.done, st_);
          s.pending = true;
          s.busy = false;
          if (e != hipSuccess) status = hip_fail(e, "scratch: record its use");
          break;
        }
      }
      slot_ = -1;
    }
    if (lock_.owns_lock()) lock_.unlock();
    return status;
  }

private:
  hipStream_t st_;
  int tag_;
  std::unique_lock<std::recursive_mutex> lock_;
  int slot_ = -1;
  int slot_dev_ = 0;
  hipStream_t slot_st_ = nullptr;
  void *own_ = nullptr;
};

// Device address of this device's copy of the fixed scratch array, looked up
// once per device (with that device current) and kept.
std::mutex g_fixed_mu;
void *g_fixed_ptr[64] = {};

int fixed_scratch_ptr(void **out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "fixed scratch: current device");
  if (dev < 0 || dev >= 64) return fail(SSD_ERR_UNSUPPORTED, "device %d: at most 64 devices", dev);
  std::lock_guard<std::mutex> lock(g_fixed_mu);
  if (!g_fixed_ptr[dev]) {
    void *p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p) {
      (void)hipGetLastError();
      return fail(SSD_ERR_HIP, "fixed scratch: hipGetSymbolAddress: %s", hipGetErrorString(e));
    }
    g_fixed_ptr[dev] = p;
  }
  *out = g_fixed_ptr[dev];
  return SSD_OK;
}

// Points this thread's scratch requests at the fixed array for one call.
class FixedScratchScope {
public:
  FixedScratchScope(void *p, size_t cap) { g_fixed = FixedScratch{p, cap}; }
  ~FixedScratchScope() { g_fixed = FixedScratch{}; }
};

// Number of buffers kept and their total bytes (tests).
void scratch_usage(size_t *slots, size_t *bytes) {
  std::lock_guard<std::recursive_mutex> lock(g_scratch_mu);
  *slots = g_scratch.size();
  size_t t = 0;
  for (const ScratchSlot &s : g_scratch) t += s.cap;
  *bytes = t;
}

// Every tensor must be memory the current device can address: device memory
// of the current device, managed memory, or pinned host memory.  Pageable
// host memory or another device's memory is refused here, before any launch
// (a kernel would fault on it).
int check_addressable(const ssd_tensor *const *ts, const char *const *names, int n) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) {
    (void)hipGetLastError();
    return fail(SSD_ERR_LAYOUT, "no current HIP device");
  }
  for (int i = 0; i < n; ++i) {
    if (!ts[i]) continue;
    hipPointerAttribute_t a;
    if (hipPointerGetAttributes(&a, ts[i]->data) != hipSuccess) {
      (void)hipGetLastError();
      return fail(SSD_ERR_LAYOUT, "%s: not memory a HIP device can address (pageable host memory?)", names[i]);
    }
    if (a.type == hipMemoryTypeUnregistered)
      return fail(SSD_ERR_LAYOUT, "%s: not memory a HIP device can address (pageable host memory?)", names[i]);
    if (a.type == hipMemoryTypeDevice && a.device != dev)
      return fail(SSD_ERR_LAYOUT, "%s: on device %d, but device %d is current", names[i], a.device, dev);
  }
  return SSD_OK;
}

int run_fused(const ssd_tensor *x, const ssd_tensor *dt, const ssd_tensor *dt_bias,
              const ssd_tensor *A, const ssd_tensor *B, const ssd_tensor *C,
              const ssd_tensor *D, const ssd_tensor *z, const ssd_tensor *init, ssd_tensor *out,
              ssd_tensor *fin, const ScanShape &s, hipStream_t st) {
  ssd::WalkParams p{};
  p.x = x->data; p.dt = (const float *)dt->data;
  p.dt_bias = dt_bias ? (const float *)dt_bias->data : nullptr;
  p.A = (const float *)A->data; p.B = B->data; p.C = C->data;
  p.D = D ? (const float *)D->data : nullptr;
  p.init = init ? (const float *)init->data : nullptr;
  p.out = out->data;
  p.z = z ? z->data : nullptr;
  p.state_out = fin ? (float *)fin->data : nullptr;
  p.b = (int)s.b; p.L = (int)s.L; p.H = (int)s.H; p.G = (int)s.G;
  p.seg_len = (int)s.L; p.nseg = 1;
  hipError_t e = ssd::launch_walk(x->dtype, (int)s.P, (int)s.N, ssd::kWalkFull, p, st);
  return e == hipSuccess ? SSD_OK : hip_fail(e, "fused walk launch");
}

// The quadratic path takes L <= 256 and every P the fused walk takes
// except 128 with fp32 inputs.
bool quad_supported(int dtype, const ScanShape &s) {
  return s.L <= ssd::kQuadMaxL && (s.P <= 64 || dtype == SSD_BF16);
}

int run_quad(const ssd_tensor *x, const ssd_tensor *dt, const ssd_tensor *dt_bias,
             const ssd_tensor *A, const ssd_tensor *B, const ssd_tensor *C,
             const ssd_tensor *D, const ssd_tensor *z, const ssd_tensor *init, ssd_tensor *out,
             ssd_tensor *fin, const ScanShape &s, hipStream_t st) {
  ssd::WalkParams p{};
  p.x = x->data; p.dt = (const float *)dt->data;
  p.dt_bias = dt_bias ? (const float *)dt_bias->data : nullptr;
  p.A = (const float *)A->data; p.B = B->data; p.C = C->data;
  p.D = D ? (const float *)D->data : nullptr;
  p.init = init ? (const float *)init->data : nullptr;
  p.out = out->data;
  p.z = z ? z->data : nullptr;
  p.final_state = fin ? (float *)fin->data : nullptr;
  p.b = (int)s.b; p.L = (int)s.L; p.H = (int)s.H; p.G = (int)s.G;
  p.seg_len = (int)s.L; p.nseg = 1;
  hipError_t e = ssd::launch_quad(x->dtype, (int)s.P, (int)s.N, p, st);
  return e == hipSuccess ? SSD_OK : hip_fail(e, "quadratic path launch");
}

int run_chunked(const ssd_tensor *x, const ssd_tensor *dt, const ssd_tensor *dt_bias,
                const ssd_tensor *A, const ssd_tensor *B, const ssd_tensor *C,
                const ssd_tensor *D, const ssd_tensor *z, const ssd_tensor *init, ssd_tensor *out,
                ssd_tensor *fin, const ScanShape &s, int chunk, hipStream_t st) {
  const int64_t nc = (s.L + chunk - 1) / chunk;
  const int64_t PN = s.P * s.N;
  const size_t n_tok = (size_t)(s.b * s.H * s.L);
  const size_t n_seg = (size_t)(s.b * s.H * nc);
  // scratch: Delta [b,H,L] | chunk log2 decays [b,H,nc] (padded) | chunk states [b,H,nc,P,N]
  const size_t off_dec = n_tok * sizeof(float);
  const size_t off_states = off_dec + ((n_seg * sizeof(float) + 255) / 256) * 256;
  const size_t total = off_states + n_seg * (size_t)PN * sizeof(float);
  Scratch sc(st);
  void *ws = nullptr;
  SSD_CHECK(sc.get(total, &ws));
  hipError_t e;
  float *delta = (float *)ws;
  float *seg_decay = (float *)((char *)ws + off_dec);
  float *states = (float *)((char *)ws + off_states);
  int status = SSD_OK;
  do {
    // 1. step sizes Delta (head-major)
    e = ssd::launch_delta((const float *)dt->data, dt_bias ? (const float *)dt_bias->data : nullptr,
                          delta, (int)s.b, (int)s.L, (int)s.H, st);
    if (e != hipSuccess) { status = hip_fail(e, "delta launch"); break; }

    // 2. each chunk's own end state from a zero start, and its total decay
    //    (all chunks but the last)
    ssd::WalkParams p{};
    p.x = x->data; p.dt = delta; p.dt_bias = nullptr; p.A = (const float *)A->data;
    p.B = B->data; p.C = C->data; p.D = D ? (const float *)D->data : nullptr;
    p.b = (int)s.b; p.L = (int)s.L; p.H = (int)s.H; p.G = (int)s.G;
    p.seg_len = chunk; p.nseg = (int)nc;
    p.init = nullptr; p.out = nullptr; p.state_out = states; p.final_state = nullptr;
    p.seg_decay = seg_decay;
    if (nc > 1) {
      e = ssd::launch_walk(x->dtype, (int)s.P, (int)s.N, ssd::kWalkChunkState, p, st);
      if (e != hipSuccess) { status = hip_fail(e, "chunk-state launch"); break; }
    }

    // 3. state entering every chunk (sequential over chunks)
    e = ssd::launch_state_pass(states, seg_decay, init ? (const float *)init->data : nullptr,
                               (int)s.b, (int)s.H, (int)PN, (int)nc, st);
    if (e != hipSuccess) { status = hip_fail(e, "state-pass launch"); break; }

    // 4. outputs of every chunk from its entering state; the last chunk's
    //    walk leaves the final state
    p.init = states; p.out = out->data; p.z = z ? z->data : nullptr; p.state_out = nullptr; p.seg_decay = nullptr;
    p.final_state = fin ? (float *)fin->data : nullptr;
    e = ssd::launch_walk(x->dtype, (int)s.P, (int)s.N, ssd::kWalkChunkOut, p, st);
    if (e != hipSuccess) { status = hip_fail(e, "chunk-output launch"); break; }
  } while (0);
  const int fs = sc.finish();
  return status != SSD_OK ? status : fs;
}

bool rows_supported(int dtype, int64_t N) {
  return dtype == SSD_BF16 && (N == 32 || N == 64 || N == 128);
}

// Waves per workgroup of the row-sliced walk: the workgroups of a pass run
// one per compute unit (LDS), and a workgroup of W waves retires a
// sub-block in about 1 + 0.1 W units of time (shared LDS and issue), so
// take the W with the fewest ceil(workgroups / CUs) * (1 + 0.1 W).
int rows_waves(const ScanShape &s, int cus) {
  const int64_t rg = (s.H / s.G) * s.P;
  double best = 1e300;
  int best_w = 4;
  for (int W = 1; W <= 8; ++W) {
    const int64_t nwg = s.b * s.G * ((rg + 16 * W - 1) / (16 * W));
    const double t = (double)((nwg + cus - 1) / cus) * (1.0 + 0.1 * W);
    if (t < best) {
      best = t;
      best_w = W;
    }
  }
  return best_w;
}

int run_rows(const ssd_tensor *x, const ssd_tensor *dt, const ssd_tensor *dt_bias,
             const ssd_tensor *A, const ssd_tensor *B, const ssd_tensor *C, const ssd_tensor *D,
             const ssd_tensor *z, const ssd_tensor *init, ssd_tensor *out, ssd_tensor *fin,
             const ScanShape &s, int W, hipStream_t st) {
  const int64_t nsub = (s.L + 63) / 64;
  const size_t rec_bytes = (size_t)(s.b * s.G * nsub) * (size_t)ssd::prep_record_blocks((int)s.N) * 1024;
  const size_t bytes = rec_bytes + (size_t)(s.b * s.H * nsub * 64) * 4;
  Scratch sc(st);
  void *ws = nullptr;
  SSD_CHECK(sc.get(bytes, &ws));
  float *dtT = reinterpret_cast<float *>(static_cast<char *>(ws) + rec_bytes);
  int status = SSD_OK;
  hipError_t e;
  do {
    // the plain walk reads Delta, the gated walk the raw dt (its softplus in
    // the walk measured faster there)
    e = ssd::launch_prep(B->data, C->data, ws, (const float *)dt->data,
                         dt_bias ? (const float *)dt_bias->data : nullptr, z ? 0 : 1, dtT, (int)s.b, (int)s.L, (int)s.H,
                         (int)s.G, (int)s.N, st);
    if (e != hipSuccess) { status = hip_fail(e, "operand record launch"); break; }
    ssd::RWalkParams p{};
    p.x = x->data; p.dt = (const float *)dt->data;
    p.dt_bias = dt_bias ? (const float *)dt_bias->data : nullptr;
    p.A = (const float *)A->data; p.B = B->data; p.C = C->data;
    p.D = D ? (const float *)D->data : nullptr;
    p.rec = ws;
    p.dtT = dtT;
    p.init = init ? (const float *)init->data : nullptr;
    p.out = out->data;
    p.z = z ? z->data : nullptr;
    p.final_state = fin ? (float *)fin->data : nullptr;
    p.b = (int)s.b; p.L = (int)s.L; p.H = (int)s.H; p.G = (int)s.G; p.P = (int)s.P;
    p.rows_per_bg = (int)((s.H / s.G) * s.P);
    p.wg_per_bg = (p.rows_per_bg + 16 * W - 1) / (16 * W);
    e = ssd::launch_rwalk((int)s.N, W, p, st);
    if (e != hipSuccess) { status = hip_fail(e, "row walk launch"); break; }
  } while (0);
  const int fs = sc.finish();
  return status != SSD_OK ? status : fs;
}

// Compute units of the current device (queried once per device).
// Safe to call from several threads at once (each slot is written with the
// same value by whichever thread gets there first).
int device_cus() {
  static std::atomic<int> cache[64] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) {
    (void)hipGetLastError();
    return 256;
  }
  int cu = cache[dev].load(std::memory_order_relaxed);
  if (cu == 0) {
    if (hipDeviceGetAttribute(&cu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cu <= 0) {
      (void)hipGetLastError();
      cu = 256;
    }
    cache[dev].store(cu, std::memory_order_relaxed);
  }
  return cu;
}

// Plan for SSD_ALGO_AUTO, from measured costs on MI355X.  The walks of the
// fused and chunked algorithms retire about one 64-token sub-block of one
// (batch, head) walk per compute unit every 2 us whether a unit holds one
// walk or several, so a pass of U walks of n sub-blocks costs
// ceil(U / CUs) * n * 2 us.  The row-sliced walk (bf16) costs
// ceil(workgroups / CUs) * n * t_rows(W).  Splitting sequences into S
// segments gives a pass of b*H*S output walks, a state-only pass over S-1
// segments (0.7 of an output walk), the step-size kernel, the state-passing
// pass (2 * b*H*S*P*N*4 bytes at ~4 TB/s) and launch gaps; a split is
// taken only when predicted at least 10% faster than the single pass.
struct Plan {
  int algo;
  int seg_len;
};

Plan choose_plan(const ScanShape &s, int dtype, int cus) {
  // Cost model in microseconds, fitted to MI355X measurements of the three
  // plans.  Walks that share a compute unit (more walks than units) cost
  // about 0.78 x ceil(walks per unit) of a lone walk.
  const bool bf16 = dtype == SSD_BF16;
  const double t_full = bf16 ? 3.3 : 11.0;  // one 64-token sub-block of a whole-sequence walk
  const double t_seg = bf16 ? 2.3 : 9.2;    // the same inside a segment walk
  const double state_rel = 0.7;             // state-only walk relative to an output walk
  const double pass_bw = 4.0e12;
  const double fixed_us = 10.0;             // step-size kernel and extra launches
  auto share = [](double n) { return n <= 1.0 ? 1.0 : 0.78 * std::ceil(n); };
  const int64_t units = s.b * s.H;
  const int64_t nsub = (s.L + 63) / 64;
  Plan best{SSD_ALGO_FUSED, (int)std::min<int64_t>(s.L, 65536)};
  double single_t = share((double)units / cus) * nsub * t_full;
  if (rows_supported(dtype, s.N)) {
    // row walk: one workgroup per unit and round; a sub-block takes longer
    // with more waves per workgroup and with more units busy
    const int W = rows_waves(s, cus);
    const int64_t nwg = s.b * s.G * (((s.H / s.G) * s.P + 16 * W - 1) / (16 * W));
    const double fill = std::min(1.0, (double)nwg / cus);
    const double rows_t = (double)((nwg + cus - 1) / cus) * nsub * (2.0 + 0.15 * W) * (0.55 + 0.45 * fill) + 6.0;
    if (rows_t < single_t) {
      single_t = rows_t;
      best.algo = SSD_ALGO_ROWS;
    }
  }
  // Quadratic path (L <= 256): one workgroup per (batch, head, query block)
  // with no chain of blocks; taken when those workgroups fit one pass over
  // the units and there is a chain to avoid (two or more blocks).  Measured
  // kernel times: fp32 b=1, L=256, H=4, P=N=16 12.0 us against 19.6 us for
  // one walk per head; bf16 b=1, L=256, H=80 (320 workgroups, two passes)
  // 15.4 us against 16.6 us, and b=8, L=256, H=32 (1024 workgroups) 33.5
  // us against 18.6 us.
  if (quad_supported(dtype, s) && nsub >= 2 && s.b * s.H * nsub <= cus)
    return Plan{SSD_ALGO_QUAD, (int)s.L};
  double best_t = 0.9 * single_t;
  for (int seg = 65536; seg >= 256; seg /= 2) {
    const int64_t S = (s.L + seg - 1) / seg;
    if (S < 2) continue;
    const double sub = (double)(seg / 64);
    const double walk = share((double)(units * S) / cus) * sub * t_seg;
    const double state = state_rel * share((double)(units * (S - 1)) / cus) * sub * t_seg;
    const double pass = 2.0 * units * S * s.P * s.N * 4.0 / pass_bw * 1e6;
    const double t = walk + state + pass + fixed_us;
    if (t < best_t) {
      best_t = t;
      best = Plan{SSD_ALGO_CHUNKED, seg};
    }
  }
  return best;
}

int scan_dispatch(const ssd_tensor *x, const ssd_tensor *dt, const ssd_tensor *dt_bias,
                  const ssd_tensor *A, const ssd_tensor *B, const ssd_tensor *C,
                  const ssd_tensor *D, const ssd_tensor *z, const ssd_tensor *init_state,
                  ssd_tensor *out, ssd_tensor *final_state, const ScanShape &s, int chunk, int algo,
                  void *stream) {
  if (algo != SSD_ALGO_AUTO && algo != SSD_ALGO_FUSED && algo != SSD_ALGO_CHUNKED &&
      algo != SSD_ALGO_ROWS && algo != SSD_ALGO_QUAD)
    return fail(SSD_ERR_UNSUPPORTED, "unknown algorithm %d", algo);
  if (algo == SSD_ALGO_ROWS && !rows_supported(x->dtype, s.N))
    return fail(SSD_ERR_UNSUPPORTED, "row-sliced walk needs bf16 inputs and N in {32,64,128}");
  if (algo == SSD_ALGO_QUAD && !quad_supported(x->dtype, s))
    return fail(SSD_ERR_UNSUPPORTED, "quadratic path needs L <= %d (L=%lld) and P <= 64 with fp32 inputs",
                ssd::kQuadMaxL, (long long)s.L);
  {
    const ssd_tensor *ts[] = {x, dt, dt_bias, A, B, C, D, z, init_state, out, final_state};
    const char *nm[] = {"x", "dt", "dt_bias", "A", "B", "C", "D", "z", "init_state", "out", "final_state"};
    SSD_CHECK(check_addressable(ts, nm, 11));
  }
  const int cus = device_cus();
  if (algo == SSD_ALGO_AUTO) {
    const Plan plan = choose_plan(s, x->dtype, cus);
    algo = plan.algo;
    chunk = plan.seg_len;
  }
  hipStream_t st = (hipStream_t)stream;
  if (algo == SSD_ALGO_ROWS)
    return run_rows(x, dt, dt_bias, A, B, C, D, z, init_state, out, final_state, s, rows_waves(s, cus), st);
  if (algo == SSD_ALGO_FUSED)
    return run_fused(x, dt, dt_bias, A, B, C, D, z, init_state, out, final_state, s, st);
  if (algo == SSD_ALGO_QUAD)
    return run_quad(x, dt, dt_bias, A, B, C, D, z, init_state, out, final_state, s, st);
  return run_chunked(x, dt, dt_bias, A, B, C, D, z, init_state, out, final_state, s, chunk, st);
}

// The gate input z: same shape and element type as x, dense; neither out
// nor final_state may overlap it.
int validate_gate(const ssd_tensor *z, const ssd_tensor *x, const ssd_tensor *out,
                  const ssd_tensor *fin, const ScanShape &s) {
  const int64_t sx[4] = {s.b, s.L, s.H, s.P};
  SSD_CHECK(check_tensor(z, "z", x->dtype, 4, sx));
  const Range rz = range_of(z);
  if (overlap(range_of(out), rz)) return fail(SSD_ERR_ALIAS, "out overlaps z");
  if (overlap(range_of(fin), rz)) return fail(SSD_ERR_ALIAS, "final_state overlaps z");
  return SSD_OK;
}

// Checks of ssd_scan_bwd's arguments (and, for the gated call, z and dz);
// every check runs on the host before any HIP call.
int validate_bwd(const ssd_tensor *x, const ssd_tensor *dt, const ssd_tensor *dt_bias,
                 const ssd_tensor *A, const ssd_tensor *B, const ssd_tensor *C,
                 const ssd_tensor *D, const ssd_tensor *init_state, const ssd_tensor *dout,
                 const ssd_tensor *dfinal_state, const ssd_tensor *dx, const ssd_tensor *ddt,
                 const ssd_tensor *ddt_bias, const ssd_tensor *dA, const ssd_tensor *dB,
                 const ssd_tensor *dC, const ssd_tensor *dD, const ssd_tensor *dinit_state,
                 const ssd_tensor *z, const ssd_tensor *dz, ScanShape &s) {
  SSD_CHECK(validate_scan(x, dt, dt_bias, A, B, C, D, init_state, dout, nullptr, 64, &s, "dout", false));
  if (s.P > 64)
    return fail(SSD_ERR_UNSUPPORTED, "backward: P=%lld not in {16,32,64}", (long long)s.P);
  const int64_t sx[4] = {s.b, s.L, s.H, s.P}, sdt[3] = {s.b, s.L, s.H}, sh[1] = {s.H},
                sbc[4] = {s.b, s.L, s.G, s.N}, sst[4] = {s.b, s.H, s.P, s.N};
  if (dfinal_state) SSD_CHECK(check_tensor(dfinal_state, "dfinal_state", SSD_F32, 4, sst));
  SSD_CHECK(check_tensor(dx, "dx", SSD_F32, 4, sx));
  SSD_CHECK(check_tensor(ddt, "ddt", SSD_F32, 3, sdt));
  if (ddt_bias) SSD_CHECK(check_tensor(ddt_bias, "ddt_bias", SSD_F32, 1, sh));
  SSD_CHECK(check_tensor(dA, "dA", SSD_F32, 1, sh));
  SSD_CHECK(check_tensor(dB, "dB", SSD_F32, 4, sbc));
  SSD_CHECK(check_tensor(dC, "dC", SSD_F32, 4, sbc));
  if (dD) SSD_CHECK(check_tensor(dD, "dD", SSD_F32, 1, sh));
  if (dinit_state) SSD_CHECK(check_tensor(dinit_state, "dinit_state", SSD_F32, 4, sst));
  if (z) {
    SSD_CHECK(check_tensor(z, "z", x->dtype, 4, sx));
    if (!dz) return fail(SSD_ERR_NULL, "dz: descriptor is NULL");
    SSD_CHECK(check_tensor(dz, "dz", SSD_F32, 4, sx));
  }
  // inputs 0..10, outputs 11..19 (z and dz only for the gated call)
  const ssd_tensor *ts[] = {x, dt, dt_bias, A, B, C, D, init_state, dout, dfinal_state, z,
                            dx, ddt, ddt_bias, dA, dB, dC, dD, dinit_state, dz};
  const char *nm[] = {"x", "dt", "dt_bias", "A", "B", "C", "D", "init_state", "dout", "dfinal_state", "z",
                      "dx", "ddt", "ddt_bias", "dA", "dB", "dC", "dD", "dinit_state", "dz"};
  // no output may overlap an input or another output
  for (int i = 11; i < 20; ++i) {
    const Range ri = range_of(ts[i]);
    for (int j = 0; j < 20; ++j)
      if (j != i && overlap(ri, range_of(ts[j])))
        return fail(SSD_ERR_ALIAS, "%s overlaps %s", nm[i], nm[j]);
  }
  SSD_CHECK(check_addressable(ts, nm, 20));
  return SSD_OK;
}


// The backward after validation: dout is the gradient at the scan output y.
int run_bwd(const ssd_tensor *x, const ssd_tensor *dt, const ssd_tensor *dt_bias,
            const ssd_tensor *A, const ssd_tensor *B, const ssd_tensor *C, const ssd_tensor *D,
            const ssd_tensor *init_state, const void *dout, const ssd_tensor *dfinal_state,
            ssd_tensor *dx, ssd_tensor *ddt, ssd_tensor *ddt_bias, ssd_tensor *dA, ssd_tensor *dB,
            ssd_tensor *dC, ssd_tensor *dD, ssd_tensor *dinit_state, const ScanShape &s,
            hipStream_t st) {
  const int64_t nc = (s.L + 63) / 64, PN = s.P * s.N, nbh = s.b * s.H;
  // the two state walks run as 2*b*H*nseg workgroups: cut the sequence into
  // segments when b*H alone would leave the GPU short of work
  const int64_t seg_chunks = (nc + std::min<int64_t>(nc, std::max<int64_t>(1, (256 + nbh - 1) / nbh)) - 1) /
                             std::min<int64_t>(nc, std::max<int64_t>(1, (256 + nbh - 1) / nbh));
  const int64_t nseg = (nc + seg_chunks - 1) / seg_chunks;
  auto al = [](size_t v) { return (v + 255) / 256 * 256; };
  const size_t o_adj = al((size_t)(nbh * nc * PN) * 4);
  const size_t o_part = o_adj + al((size_t)(nbh * nc * PN) * 4);
  const size_t o_pre = o_part + al((size_t)(nbh * nc * 3) * 4);
  const size_t o_seg = o_pre + 2 * al((size_t)(nbh * nc) * 4);
  const size_t o_sdec = o_seg + 2 * al((size_t)(nbh * nseg * PN) * 4);
  const size_t total = o_sdec + 2 * al((size_t)(nbh * nseg) * 4) + al((size_t)nbh * 4);
  Scratch sc(st);
  void *ws = nullptr;
  SSD_CHECK(sc.get(total, &ws));
  char *base = (char *)ws;
  ssd::BwdParams bp{};
  bp.x = x->data; bp.dt = (const float *)dt->data;
  bp.dt_bias = dt_bias ? (const float *)dt_bias->data : nullptr;
  bp.A = (const float *)A->data; bp.B = B->data; bp.C = C->data;
  bp.D = D ? (const float *)D->data : nullptr;
  bp.dy = dout; bp.dfinal = dfinal_state ? (const float *)dfinal_state->data : nullptr;
  bp.states_init = init_state ? (const float *)init_state->data : nullptr;
  bp.states = (float *)base; bp.adj = (float *)(base + o_adj); bp.part = (float *)(base + o_part);
  bp.nseg = (int)nseg; bp.seg_chunks = (int)seg_chunks;
  bp.fpre = (float *)(base + o_pre); bp.rpre = (float *)(base + o_pre + al((size_t)(nbh * nc) * 4));
  bp.segend_f = (float *)(base + o_seg); bp.segend_r = (float *)(base + o_seg + al((size_t)(nbh * nseg * PN) * 4));
  bp.segdec_f = (float *)(base + o_sdec); bp.segdec_r = (float *)(base + o_sdec + al((size_t)(nbh * nseg) * 4));
  bp.rdec0 = (float *)(base + o_sdec + 2 * al((size_t)(nbh * nseg) * 4));
  bp.dx = (float *)dx->data; bp.ddt = (float *)ddt->data; bp.dB = (float *)dB->data;
  bp.dC = (float *)dC->data; bp.dA = (float *)dA->data;
  bp.dD = dD ? (float *)dD->data : nullptr;
  bp.ddt_bias = ddt_bias ? (float *)ddt_bias->data : nullptr;
  bp.dinit = dinit_state ? (float *)dinit_state->data : nullptr;
  bp.b = (int)s.b; bp.L = (int)s.L; bp.H = (int)s.H; bp.G = (int)s.G; bp.nc = (int)nc;
  int status = SSD_OK;
  const hipError_t e = ssd::launch_bwd(x->dtype, (int)s.P, (int)s.N, bp, st);
  if (e != hipSuccess) status = hip_fail(e, "backward launch");
  const int fs = sc.finish();
  return status != SSD_OK ? status : fs;
}


} // namespace

extern "C" {

int ssd_scan_fwd_algo(const ssd_tensor *x, const ssd_tensor *dt, const ssd_tensor *dt_bias,
                      const ssd_tensor *A, const ssd_tensor *B, const ssd_tensor *C,
                      const ssd_tensor *D, const ssd_tensor *init_state, ssd_tensor *out,
                      ssd_tensor *final_state, int chunk, int algo, void *stream) {
  g_last_error.clear();
  ScanShape s;
  SSD_CHECK(validate_scan(x, dt, dt_bias, A, B, C, D, init_state, out, final_state, chunk, &s));
  return scan_dispatch(x, dt, dt_bias, A, B, C, D, nullptr, init_state, out, final_state, s, chunk, algo,
                       stream);
}

int ssd_scan_fwd_gated(const ssd_tensor *x, const ssd_tensor *dt, const ssd_tensor *dt_bias,
                       const ssd_tensor *A, const ssd_tensor *B, const ssd_tensor *C,
                       const ssd_tensor *D, const ssd_tensor *z, const ssd_tensor *init_state,
                       ssd_tensor *out, ssd_tensor *final_state, int chunk, int algo, void *stream) {
  g_last_error.clear();
  ScanShape s;
  SSD_CHECK(validate_scan(x, dt, dt_bias, A, B, C, D, init_state, out, final_state, chunk, &s));
  if (!z) return fail(SSD_ERR_NULL, "z: descriptor is NULL");
  SSD_CHECK(validate_gate(z, x, out, final_state, s));
  return scan_dispatch(x, dt, dt_bias, A, B, C, D, z, init_state, out, final_state, s, chunk, algo, stream);
}

int ssd_scan_fwd(const ssd_tensor *x, const ssd_tensor *dt, const ssd_tensor *dt_bias,
                 const ssd_tensor *A, const ssd_tensor *B, const ssd_tensor *C,
                 const ssd_tensor *D, const ssd_tensor *init_state, ssd_tensor *out,
                 ssd_tensor *final_state, int chunk, void *stream) {
  return ssd_scan_fwd_algo(x, dt, dt_bias, A, B, C, D, init_state, out, final_state, chunk,
                           SSD_ALGO_AUTO, stream);
}

int ssd_scan_fwd_noalloc(const ssd_tensor *x, const ssd_tensor *dt, const ssd_tensor *dt_bias,
                         const ssd_tensor *A, const ssd_tensor *B, const ssd_tensor *C,
                         const ssd_tensor *D, const ssd_tensor *init_state, ssd_tensor *out,
                         ssd_tensor *final_state, int chunk, void *stream) {
  g_last_error.clear();
  ScanShape s;
  SSD_CHECK(validate_scan(x, dt, dt_bias, A, B, C, D, init_state, out, final_state, chunk, &s));
  void *p = nullptr;
  SSD_CHECK(fixed_scratch_ptr(&p));
  FixedScratchScope scope(p, SSD_FIXED_SCRATCH_BYTES);
  return scan_dispatch(x, dt, dt_bias, A, B, C, D, nullptr, init_state, out, final_state, s, chunk,
                       SSD_ALGO_AUTO, stream);
}

int64_t ssd_fixed_scratch_bytes(void) { return (int64_t)SSD_FIXED_SCRATCH_BYTES; }

int ssd_scratch_stats(int64_t *buffers, int64_t *bytes) {
  g_last_error.clear();
  if (!buffers || !bytes) return fail(SSD_ERR_NULL, "buffers/bytes: NULL");
  size_t n = 0, t = 0;
  scratch_usage(&n, &t);
  *buffers = (int64_t)n;
  *bytes = (int64_t)t;
  return SSD_OK;
}

int ssd_scan_fwd_rows(const ssd_tensor *x, const ssd_tensor *dt, const ssd_tensor *dt_bias,
                      const ssd_tensor *A, const ssd_tensor *B, const ssd_tensor *C,
                      const ssd_tensor *D, const ssd_tensor *init_state, ssd_tensor *out,
                      ssd_tensor *final_state, int waves, void *stream) {
  g_last_error.clear();
  ScanShape s;
  SSD_CHECK(validate_scan(x, dt, dt_bias, A, B, C, D, init_state, out, final_state, 64, &s));
  if (!rows_supported(x->dtype, s.N))
    return fail(SSD_ERR_UNSUPPORTED, "row-sliced walk needs bf16 inputs and N in {32,64,128}");
  if (waves < 0 || waves > 8) return fail(SSD_ERR_UNSUPPORTED, "waves=%d not in 0..8", waves);
  {
    const ssd_tensor *ts[] = {x, dt, dt_bias, A, B, C, D, init_state, out, final_state};
    const char *nm[] = {"x", "dt", "dt_bias", "A", "B", "C", "D", "init_state", "out", "final_state"};
    SSD_CHECK(check_addressable(ts, nm, 10));
  }
  const int W = waves ? waves : rows_waves(s, device_cus());
  return run_rows(x, dt, dt_bias, A, B, C, D, nullptr, init_state, out, final_state, s, W,
                  (hipStream_t)stream);
}

int ssd_step(ssd_tensor *state, const ssd_tensor *x, const ssd_tensor *dt, const ssd_tensor *A,
             const ssd_tensor *B, const ssd_tensor *C, const ssd_tensor *D, ssd_tensor *out,
             void *stream) {
  g_last_error.clear();
  if (!state) return fail(SSD_ERR_NULL, "state: descriptor is NULL");
  if (!B) return fail(SSD_ERR_NULL, "B: descriptor is NULL");
  if (state->ndim != 4) return fail(SSD_ERR_SHAPE, "state: rank %d, expected 4 [b,H,P,N]", state->ndim);
  if (B->ndim != 3) return fail(SSD_ERR_SHAPE, "B: rank %d, expected 3 [b,G,N]", B->ndim);
  const int64_t b = state->shape[0], H = state->shape[1], P = state->shape[2],
                N = state->shape[3], G = B->shape[1];
  if (b < 1 || H < 1 || P < 1 || G < 1)
    return fail(SSD_ERR_SHAPE, "empty problem: b=%lld H=%lld P=%lld G=%lld", (long long)b,
                (long long)H, (long long)P, (long long)G);
  if (H % G != 0) return fail(SSD_ERR_SHAPE, "H=%lld is not a multiple of G=%lld", (long long)H, (long long)G);
  if (N != 16 && N != 32 && N != 64 && N != 128 && N != 256)
    return fail(SSD_ERR_UNSUPPORTED, "N=%lld not in {16,32,64,128,256}", (long long)N);
  if (b * H > INT32_MAX / 2 || P > (1 << 20))
    return fail(SSD_ERR_UNSUPPORTED, "problem too large");
  if (!x) return fail(SSD_ERR_NULL, "x: descriptor is NULL");
  const int xd = x->dtype;
  const int64_t sst[4] = {b, H, P, N}, sx[3] = {b, H, P}, sdt[2] = {b, H}, sh[1] = {H},
                sbc[3] = {b, G, N};
  SSD_CHECK(check_tensor(state, "state", SSD_F32, 4, sst));
  SSD_CHECK(check_tensor(x, "x", -1, 3, sx));
  SSD_CHECK(check_tensor(dt, "dt", SSD_F32, 2, sdt));
  SSD_CHECK(check_tensor(A, "A", SSD_F32, 1, sh));
  SSD_CHECK(check_tensor(B, "B", xd, 3, sbc));
  SSD_CHECK(check_tensor(C, "C", xd, 3, sbc));
  if (D) SSD_CHECK(check_tensor(D, "D", SSD_F32, 1, sh));
  SSD_CHECK(check_tensor(out, "out", xd, 3, sx));
  const Range ro = range_of(out), rs = range_of(state);
  const ssd_tensor *ins[] = {x, dt, A, B, C, D};
  const char *names[] = {"x", "dt", "A", "B", "C", "D"};
  for (int i = 0; i < 6; ++i) {
    const Range ri = range_of(ins[i]);
    if (overlap(ro, ri)) return fail(SSD_ERR_ALIAS, "out overlaps %s", names[i]);
    if (overlap(rs, ri)) return fail(SSD_ERR_ALIAS, "state overlaps %s", names[i]);
  }
  if (overlap(ro, rs)) return fail(SSD_ERR_ALIAS, "out overlaps state");
  {
    const ssd_tensor *ts[] = {state, x, dt, A, B, C, D, out};
    const char *nm[] = {"state", "x", "dt", "A", "B", "C", "D", "out"};
    SSD_CHECK(check_addressable(ts, nm, 8));
  }
  hipError_t e = ssd::launch_step(xd, (int)N, (float *)state->data, x->data,
                                  (const float *)dt->data, (const float *)A->data, B->data,
                                  C->data, D ? (const float *)D->data : nullptr, out->data,
                                  (int)b, (int)H, (int)P, (int)G, (hipStream_t)stream);
  return e == hipSuccess ? SSD_OK : hip_fail(e, "step launch");
}

int ssd_selective_scan_fwd(const ssd_tensor *x, const ssd_tensor *dt, const ssd_tensor *dt_bias,
                           const ssd_tensor *A, const ssd_tensor *B, const ssd_tensor *C,
                           const ssd_tensor *D, const ssd_tensor *init_state, ssd_tensor *out,
                           ssd_tensor *final_state, int segments, void *stream) {
  g_last_error.clear();
  if (!x) return fail(SSD_ERR_NULL, "x: descriptor is NULL");
  if (!A) return fail(SSD_ERR_NULL, "A: descriptor is NULL");
  if (!B) return fail(SSD_ERR_NULL, "B: descriptor is NULL");
  if (x->ndim != 3) return fail(SSD_ERR_SHAPE, "x: rank %d, expected 3 [b,L,D]", x->ndim);
  if (A->ndim != 2) return fail(SSD_ERR_SHAPE, "A: rank %d, expected 2 [D,N]", A->ndim);
  if (B->ndim != 4) return fail(SSD_ERR_SHAPE, "B: rank %d, expected 4 [b,L,G,N]", B->ndim);
  const int64_t b = x->shape[0], L = x->shape[1], Dc = x->shape[2], G = B->shape[2],
                N = B->shape[3];
  if (b < 1 || L < 1 || Dc < 1 || G < 1)
    return fail(SSD_ERR_SHAPE, "empty problem: b=%lld L=%lld D=%lld G=%lld", (long long)b,
                (long long)L, (long long)Dc, (long long)G);
  if (Dc % G != 0) return fail(SSD_ERR_SHAPE, "D=%lld is not a multiple of G=%lld", (long long)Dc, (long long)G);
  if ((Dc / G) % 64 != 0)
    return fail(SSD_ERR_UNSUPPORTED, "channels per group D/G=%lld is not a multiple of 64",
                (long long)(Dc / G));
  if (N != 4 && N != 8 && N != 16) return fail(SSD_ERR_UNSUPPORTED, "N=%lld not in {4,8,16}", (long long)N);
  if (L > kMaxL) return fail(SSD_ERR_UNSUPPORTED, "L=%lld above the supported %lld tokens", (long long)L, (long long)kMaxL);
  if (Dc > kMaxRow || b * L > INT32_MAX / 2 || b * (Dc / 64) > INT32_MAX / 64)
    return fail(SSD_ERR_UNSUPPORTED, "problem too large");
  if (segments < 0) return fail(SSD_ERR_UNSUPPORTED, "segments=%d is negative", segments);
  const int xd = x->dtype;
  const int64_t sx[3] = {b, L, Dc}, sd[1] = {Dc}, sa[2] = {Dc, N}, sbc[4] = {b, L, G, N},
                sst[3] = {b, Dc, N};
  SSD_CHECK(check_tensor(x, "x", -1, 3, sx));
  SSD_CHECK(check_tensor(dt, "dt", SSD_F32, 3, sx));
  if (dt_bias) SSD_CHECK(check_tensor(dt_bias, "dt_bias", SSD_F32, 1, sd));
  SSD_CHECK(check_tensor(A, "A", SSD_F32, 2, sa));
  SSD_CHECK(check_tensor(B, "B", xd, 4, sbc));
  SSD_CHECK(check_tensor(C, "C", xd, 4, sbc));
  if (D) SSD_CHECK(check_tensor(D, "D", SSD_F32, 1, sd));
  if (init_state) SSD_CHECK(check_tensor(init_state, "init_state", SSD_F32, 3, sst));
  SSD_CHECK(check_tensor(out, "out", xd, 3, sx));
  if (final_state) SSD_CHECK(check_tensor(final_state, "final_state", SSD_F32, 3, sst));
  {
    const Range ro = range_of(out), rf = range_of(final_state);
    const ssd_tensor *ins[] = {x, dt, dt_bias, A, B, C, D, init_state};
    const char *names[] = {"x", "dt", "dt_bias", "A", "B", "C", "D", "init_state"};
    for (int i = 0; i < 8; ++i) {
      const Range ri = range_of(ins[i]);
      if (overlap(ro, ri)) return fail(SSD_ERR_ALIAS, "out overlaps %s", names[i]);
      if (i == 7 && final_state && init_state && final_state->data == init_state->data) continue;
      if (overlap(rf, ri)) return fail(SSD_ERR_ALIAS, "final_state overlaps %s", names[i]);
    }
    if (overlap(ro, rf)) return fail(SSD_ERR_ALIAS, "out overlaps final_state");
  }
  // Segments: about five waves per SIMD (each wave owns 64 channels of one
  // batch row; the kernel is bound by the vector ALU, and a multiple of the
  // SIMD count avoids a partial last round -- measured on MI355X: 16
  // segments for 320 (batch, channel-block) pairs run in 274 us, 13 in 320);
  // segments are whole 8-token steps.
  const int64_t waves_per_seg = b * (Dc / 64);
  const int64_t steps = (L + 7) / 8;
  int64_t nseg = segments;
  if (nseg == 0) {
    const int64_t want = 20LL * device_cus();
    nseg = std::max<int64_t>(1, (want + waves_per_seg / 2) / waves_per_seg);
  }
  // A wave addresses its segment of x, dt and out through 32-bit byte
  // ranges: at least enough segments to keep one segment under 2 GiB.
  const int64_t min_nseg = (L * Dc * 4 + ((int64_t)1 << 31) - 1) >> 31;
  nseg = std::max<int64_t>(nseg, min_nseg);
  nseg = std::min<int64_t>(std::min<int64_t>(nseg, steps), 1024);
  const int64_t seg_len = ((steps + nseg - 1) / nseg) * 8;
  nseg = (L + seg_len - 1) / seg_len;
  if (seg_len * Dc * 4 >= ((int64_t)1 << 31) || b * (Dc / 64) * nseg > INT32_MAX)
    return fail(SSD_ERR_UNSUPPORTED, "problem too large");

  {
    const ssd_tensor *ts[] = {x, dt, dt_bias, A, B, C, D, init_state, out, final_state};
    const char *nm[] = {"x", "dt", "dt_bias", "A", "B", "C", "D", "init_state", "out", "final_state"};
    SSD_CHECK(check_addressable(ts, nm, 10));
  }
  ssd::SScanParams p{};
  p.x = x->data; p.dt = (const float *)dt->data;
  p.dt_bias = dt_bias ? (const float *)dt_bias->data : nullptr;
  p.A = (const float *)A->data; p.B = B->data; p.C = C->data;
  p.D = D ? (const float *)D->data : nullptr;
  p.init = init_state ? (const float *)init_state->data : nullptr;
  p.out = out->data; p.final_state = final_state ? (float *)final_state->data : nullptr;
  p.b = (int)b; p.L = (int)L; p.Dc = (int)Dc; p.G = (int)G; p.seg_len = (int)seg_len; p.nseg = (int)nseg;
  hipStream_t st = (hipStream_t)stream;
  Scratch sc(st);
  void *ws = nullptr;
  if (nseg > 1) {
    // scratch: segment end states [b,nseg,D,N] | segment Delta sums [b,nseg,D] | staged init [b,D,N]
    const size_t n_end = (size_t)(b * nseg * Dc);
    const size_t off_sd = ((n_end * N * sizeof(float) + 255) / 256) * 256;
    const size_t off_hc = off_sd + ((n_end * sizeof(float) + 255) / 256) * 256;
    const size_t total = off_hc + (size_t)(b * Dc * N) * sizeof(float);
    SSD_CHECK(sc.get(total, &ws));
    p.hend = (float *)ws;
    p.sdelta = (float *)((char *)ws + off_sd);
    p.hcopy = (float *)((char *)ws + off_hc);
  }
  int status = SSD_OK;
  hipError_t e = ssd::launch_sscan(xd, (int)N, p, st);
  if (e != hipSuccess) status = hip_fail(e, "selective scan launch");
  const int fs = sc.finish();
  return status != SSD_OK ? status : fs;
}

int ssd_scan_bwd(const ssd_tensor *x, const ssd_tensor *dt, const ssd_tensor *dt_bias,
                 const ssd_tensor *A, const ssd_tensor *B, const ssd_tensor *C,
                 const ssd_tensor *D, const ssd_tensor *init_state, const ssd_tensor *dout,
                 const ssd_tensor *dfinal_state, ssd_tensor *dx, ssd_tensor *ddt,
                 ssd_tensor *ddt_bias, ssd_tensor *dA, ssd_tensor *dB, ssd_tensor *dC,
                 ssd_tensor *dD, ssd_tensor *dinit_state, void *stream) {
  g_last_error.clear();
  ScanShape s;
  SSD_CHECK(validate_bwd(x, dt, dt_bias, A, B, C, D, init_state, dout, dfinal_state, dx, ddt, ddt_bias,
                         dA, dB, dC, dD, dinit_state, nullptr, nullptr, s));
  return run_bwd(x, dt, dt_bias, A, B, C, D, init_state, dout->data, dfinal_state, dx, ddt, ddt_bias, dA,
                 dB, dC, dD, dinit_state, s, (hipStream_t)stream);
}

int ssd_scan_bwd_gated(const ssd_tensor *x, const ssd_tensor *dt, const ssd_tensor *dt_bias,
                       const ssd_tensor *A, const ssd_tensor *B, const ssd_tensor *C,
                       const ssd_tensor *D, const ssd_tensor *z, const ssd_tensor *init_state,
                       const ssd_tensor *dout, const ssd_tensor *dfinal_state, ssd_tensor *dx,
                       ssd_tensor *ddt, ssd_tensor *ddt_bias, ssd_tensor *dA, ssd_tensor *dB,
                       ssd_tensor *dC, ssd_tensor *dD, ssd_tensor *dz, ssd_tensor *dinit_state,
                       void *stream) {
  g_last_error.clear();
  if (!z) return fail(SSD_ERR_NULL, "z: descriptor is NULL");
  ScanShape s;
  SSD_CHECK(validate_bwd(x, dt, dt_bias, A, B, C, D, init_state, dout, dfinal_state, dx, ddt, ddt_bias,
                         dA, dB, dC, dD, dinit_state, z, dz, s));
  hipStream_t st = (hipStream_t)stream;
  // y (the scan output before the gate) and the gradient at it, in x's dtype
  const size_t n = (size_t)(s.b * s.L * s.H * s.P), es = (size_t)elem_size(x->dtype);
  const size_t half = (n * es + 255) / 256 * 256;
  Scratch keep(st, 1);
  void *ws = nullptr;
  SSD_CHECK(keep.get(2 * half, &ws));
  ssd_tensor yt = *x;
  yt.data = ws;
  int status = scan_dispatch(x, dt, dt_bias, A, B, C, D, nullptr, init_state, &yt, nullptr, s, 256,
                             SSD_ALGO_AUTO, stream);
  void *dyg = (char *)ws + half;
  if (status == SSD_OK) {
    const hipError_t e = ssd::launch_gate_bwd(x->dtype, ws, z->data, dout->data, dyg, (float *)dz->data,
                                              (int64_t)n, st);
    if (e != hipSuccess) status = hip_fail(e, "gate backward launch");
  }
  if (status == SSD_OK)
    status = run_bwd(x, dt, dt_bias, A, B, C, D, init_state, dyg, dfinal_state, dx, ddt, ddt_bias, dA, dB,
                     dC, dD, dinit_state, s, st);
  const int fs = keep.finish();
  return status != SSD_OK ? status : fs;
}

int ssd_scan_plan(int64_t b, int64_t L, int64_t H, int64_t P, int64_t G, int64_t N, int dtype,
                  int cus, int *algo, int *seg_len) {
  g_last_error.clear();
  if (!algo || !seg_len) return fail(SSD_ERR_NULL, "algo/seg_len: NULL");
  if (b < 1 || L < 1 || H < 1 || G < 1 || H % G != 0)
    return fail(SSD_ERR_SHAPE, "invalid shape b=%lld L=%lld H=%lld G=%lld", (long long)b,
                (long long)L, (long long)H, (long long)G);
  ScanShape s{b, L, H, P, G, N};
  if (dtype != SSD_F32 && dtype != SSD_BF16) return fail(SSD_ERR_DTYPE, "dtype %d", dtype);
  const Plan plan = choose_plan(s, dtype, cus > 0 ? cus : 256);
  *algo = plan.algo;
  *seg_len = plan.seg_len;
  return SSD_OK;
}

const char *ssd_status_string(int status) {
  switch (status) {
  case SSD_OK: return "ok";
  case SSD_ERR_NULL: return "null pointer";
  case SSD_ERR_SHAPE: return "shape mismatch";
  case SSD_ERR_DTYPE: return "dtype mismatch";
  case SSD_ERR_LAYOUT: return "layout not dense row-major or misaligned";
  case SSD_ERR_UNSUPPORTED: return "unsupported size or option";
  case SSD_ERR_ALIAS: return "output aliases an input";
  case SSD_ERR_NOMEM: return "scratch allocation failed";
  case SSD_ERR_HIP: return "HIP runtime error";
  }
  return "unknown status";
}

const char *ssd_last_error(void) { return g_last_error.c_str(); }

int ssd_version(void) { return SSD_VERSION; }

int ssd_release_scratch(void) {
  g_last_error.clear();
  std::lock_guard<std::recursive_mutex> lock(g_scratch_mu);
  if (g_scratch.empty()) return SSD_OK;
  int cur = 0;
  hipError_t e = hipGetDevice(&cur);
  if (e != hipSuccess) return hip_fail(e, "release scratch: current device");
  int status = SSD_OK;
  for (ScratchSlot &s : g_scratch) {
    e = hipSetDevice(s.dev);
    if (e == hipSuccess && s.pending) e = hipEventSynchronize(s.done);
    if (e == hipSuccess && s.p) e = hipFreeAsync(s.p, nullptr);
    if (e == hipSuccess) e = hipStreamSynchronize(nullptr);
    if (e == hipSuccess) e = hipEventDestroy(s.done);
    if (e != hipSuccess && status == SSD_OK) status = hip_fail(e, "release scratch");
  }
  g_scratch.clear();
  e = hipSetDevice(cur);
  if (e != hipSuccess && status == SSD_OK) status = hip_fail(e, "release scratch: restore device");
  return status;
}

} // extern "C"
