// C ABI of the ReTopK decode-step attention library: handle management,
// argument checks, launch sequencing and host-side state exchange.
// The interface and its contracts are documented in include/retopk.h.

#include "retopk.h"
#include "retopk_internal.h"

#include <cmath>
#include <cstring>
#include <string>
#include <vector>

using namespace retopk;

namespace {

constexpr int kMaxTimed = 65536;

thread_local std::string g_last_error;

retopk_status fail(retopk_status s, const std::string& msg) {
  g_last_error = msg;
  return s;
}

retopk_status hip_fail(hipError_t e, const char* what) {
  return fail(RETOPK_HIP_ERROR, std::string(what) + ": " + hipGetErrorString(e));
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// Makes the handle's device current for the duration of a call.
class DeviceGuard {
 public:
  explicit DeviceGuard(int dev) {
    if (hipGetDevice(&old_) != hipSuccess) old_ = -1;
    if (old_ != dev) (void)hipSetDevice(dev);
    dev_ = dev;
  }
  ~DeviceGuard() {
    if (old_ >= 0 && old_ != dev_) (void)hipSetDevice(old_);
  }

 private:
  int old_ = -1, dev_ = -1;
};

}  // namespace

namespace {

constexpr int kMaxGroupLayers = 1024;

// Device allocations of one owner, zero-filled, freed together.
struct Allocs {
  std::vector<void*> ptrs;
  size_t bytes = 0;

  template <typename T>
  hipError_t alloc(T** ptr, size_t count) {
    const size_t n = count * sizeof(T);
    void* raw = nullptr;
    hipError_t e = hipMalloc(&raw, n > 0 ? n : 16);
    if (e != hipSuccess) return e;
    ptrs.push_back(raw);
    bytes += n;
    *ptr = static_cast<T*>(raw);
    return hipMemset(raw, 0, n > 0 ? n : 16);
  }
  void release() {
    for (void* a : ptrs) (void)hipFree(a);
    ptrs.clear();
    bytes = 0;
  }
};

// The per-call workspaces of k_step (everything in Bufs but a layer's cache
// and statistics ring), the dense partials, the launch-hint word, the control
// words of graph-replayed steps and the call sequence. A handle owns one, or
// the layers of a group share one (calls on them are serialised on one stream).
struct Workspace {
  Allocs mem;
  Bufs b{};                         // the shared fields filled, the per-layer ones NULL
  float* dense_part = nullptr;      // dense attention's row-slice partials [B*Hq, dense_max_split, kDensePart]
  int32_t* hint_host = nullptr;     // pinned, device-mapped word behind Bufs::hint
  int32_t* ctl = nullptr;           // {length, t_dec, seq, pad}: position of graph-replayed steps
  int call_seq = 0;                 // sequence number of the last k_step launch on the workspace

  // Tag of the next launch's decision flags: 2 * seq, seq counting 1, 2, ... mod
  // 2^29 (an even modulus, so bit 1, which selects the histogram half,
  // alternates from call to call, and no tag repeats the previous one).
  int next_call_flag() {
    call_seq = (call_seq + 1) & kSeqMask;
    return 2 * call_seq;
  }

  hipError_t create(const Dims& d) {
    const size_t BH = static_cast<size_t>(d.B) * d.Hq;
    hipError_t e = hipSuccess;
    auto A = [&](auto** ptr, size_t n) {
      if (e == hipSuccess) e = mem.alloc(ptr, n);
    };
    A(&b.path, BH);
    A(&b.rho, BH);
    A(&b.ret, BH * d.R);
    A(&b.retslot, BH * d.R);
    A(&b.m, BH);
    A(&b.cand, BH * d.cand_cap);
    A(&b.score, BH * d.score_stride);
    A(&b.hist, BH * 2 * kNumBins);
    A(&b.hits, BH * d.max_len);
    A(&b.ccnt, BH * d.n_cu);
    A(&b.dec, BH * kFlagStride);
    A(&b.err, 1);
    A(&b.wdone, static_cast<size_t>(d.n_cu) * kFlagStride);
    A(&b.bkeys, BH * d.max_len);
    A(&b.sel, BH * d.K);
    A(&b.selsc, BH * d.K);
    A(&b.sellen, BH);
    A(&dense_part, BH * static_cast<size_t>(dense_max_split(d)) * kDensePart);
    A(&ctl, 4);
    if (e == hipSuccess) e = hipHostMalloc(reinterpret_cast<void**>(&hint_host), 64, hipHostMallocMapped);
    if (e == hipSuccess) {
      *hint_host = 0;
      e = hipHostGetDevicePointer(reinterpret_cast<void**>(&b.hint), hint_host, 0);
    }
    return e;
  }
  void release() {
    mem.release();
    if (hint_host != nullptr) (void)hipHostFree(hint_host);
    hint_host = nullptr;
  }
};

}  // namespace

struct retopk_group;

struct retopk_handle {
  retopk_params p{};
  Dims d{};
  Bufs b{};
  int device = 0;
  Allocs mem;                       // this layer's cache, statistics ring and table copy
  Workspace own;                    // the workspace of a stand-alone handle
  Workspace* ws = &own;             // the workspace in use (a group's, for its layers)
  retopk_group* group = nullptr;    // the owning group, or NULL
  bool stats = true;
  bool timing = false;
  std::vector<hipEvent_t> events;   // pairs (start, stop)
  std::vector<int> event_kernel;    // kernel id of each recorded pair
  int timed = 0;                    // pairs recorded since the last read

  int next_call_flag() { return ws->next_call_flag(); }

  // This layer's own buffers, and its table (the workspace's fields beside
  // them) copied to the device.
  hipError_t create_layer() {
    const size_t BH = static_cast<size_t>(d.B) * d.Hq, D = kHeadDim;
    Bufs t = ws->b;
    hipError_t e = hipSuccess;
    auto A = [&](auto** ptr, size_t n) {
      if (e == hipSuccess) e = mem.alloc(ptr, n);
    };
    A(&t.cache_qbar, BH * d.C * D);
    A(&t.cache_supp, BH * d.C * d.K);
    A(&t.cache_len, BH * d.C);
    A(&t.fifo, BH * 2);
    A(&t.st_path, BH * kStatsCap);
    A(&t.st_rho, BH * kStatsCap);
    A(&t.st_m, BH * kStatsCap);
    A(&t.self, 1);
    if (e == hipSuccess) e = hipMemcpy(t.self, &t, sizeof(Bufs), hipMemcpyHostToDevice);
    b = t;
    return e;
  }

  size_t bytes() const { return mem.bytes + (group == nullptr ? own.mem.bytes : 0); }

  void release() {
    mem.release();
    own.release();
    for (hipEvent_t e : events) (void)hipEventDestroy(e);
    events.clear();
  }

  // Run one kernel launch, bracketing it with timing events when enabled.
  template <typename F>
  retopk_status run(int id, hipStream_t s, F&& launch) {
    bool timed_launch = false;
    if (timing && timed < kMaxTimed) {
      if (static_cast<int>(events.size()) < 2 * (timed + 1)) {
        for (int i = 0; i < 256; ++i) {
          hipEvent_t ev;
          if (hipEventCreate(&ev) != hipSuccess) break;
          events.push_back(ev);
        }
        event_kernel.resize(events.size() / 2);
      }
      if (static_cast<int>(events.size()) >= 2 * (timed + 1)) {
        timed_launch = hipEventRecord(events[2 * timed], s) == hipSuccess;
      }
    }
    const hipError_t e = launch();
    if (e != hipSuccess) return hip_fail(e, kernel_name(id));
    if (timed_launch && hipEventRecord(events[2 * timed + 1], s) == hipSuccess) {
      event_kernel[timed] = id;
      ++timed;
    }
    return RETOPK_OK;
  }
};

// Layers sharing one workspace, and the HIP graph of one decode token over
// all of them.
struct retopk_group {
  retopk_params p{};
  Dims d{};
  int device = 0;
  Workspace ws;
  std::vector<retopk_handle*> layers;
  hipGraph_t graph = nullptr;
  hipGraphExec_t exec = nullptr;
  int next_len = 0, next_tdec = 0;  // position of the next replayed token (0: not set)
  bool ctl_stale = true;            // the control words need setting before the next replay
  int seq_at_replay = -1;           // the workspace's call sequence after the last replay

  void release() {
    if (exec != nullptr) (void)hipGraphExecDestroy(exec);
    if (graph != nullptr) (void)hipGraphDestroy(graph);
    exec = nullptr;
    graph = nullptr;
    for (retopk_handle* h : layers) {
      h->release();
      delete h;
    }
    layers.clear();
    ws.release();
  }
};

namespace {

// Argument checks shared by retopk_create and retopk_group_create.
retopk_status check_params(const retopk_params& p, const char* who) {
  const std::string w(who);
  if (p.batch < 1 || p.n_q_heads < 1 || p.n_kv_heads < 1)
    return fail(RETOPK_INVALID_ARG, w + ": batch and head counts must be >= 1");
  if (p.n_q_heads % p.n_kv_heads != 0)
    return fail(RETOPK_INVALID_ARG, w + ": n_q_heads must be a multiple of n_kv_heads");
  if (p.n_q_heads / p.n_kv_heads > kMaxGroup)
    return fail(RETOPK_INVALID_ARG, w + ": at most 16 query heads per KV head");
  if (p.head_dim != kHeadDim) return fail(RETOPK_INVALID_ARG, w + ": head_dim must be 128");
  if (p.max_len < 1 || p.max_len > (1 << 24))
    return fail(RETOPK_OUT_OF_RANGE, w + ": max_len must be in 1 .. 2^24");
  if (p.top_k < 1 || p.top_k > 8192) return fail(RETOPK_OUT_OF_RANGE, w + ": top_k must be in 1 .. 8192");
  if (p.cache_cap < 1 || p.cache_cap > 64)
    return fail(RETOPK_OUT_OF_RANGE, w + ": cache_cap must be in 1 .. 64");
  if (p.window < 0) return fail(RETOPK_OUT_OF_RANGE, w + ": window must be >= 0");
  if (p.top_r < 1 || p.top_r > p.cache_cap)
    return fail(RETOPK_OUT_OF_RANGE, w + ": top_r must be in 1 .. cache_cap");
  if (p.refresh_every < 0) return fail(RETOPK_OUT_OF_RANGE, w + ": refresh_every must be >= 0");
  if (std::isnan(p.tau)) return fail(RETOPK_INVALID_ARG, w + ": tau is NaN");
  if (p.retrieval != RETOPK_RETRIEVE_SIMILAR && p.retrieval != RETOPK_RETRIEVE_RECENT)
    return fail(RETOPK_INVALID_ARG, w + ": retrieval must be RETOPK_RETRIEVE_SIMILAR or _RECENT");
  const long long cand = static_cast<long long>(p.top_r) * p.top_k + p.window;
  if (cand > kMaxCand) return fail(RETOPK_OUT_OF_RANGE, w + ": top_r * top_k + window must be <= 16384");
  {
    Dims probe{};
    probe.K = p.top_k;
    probe.G = p.n_q_heads / p.n_kv_heads;
    probe.cand_cap = static_cast<int>(cand);
    probe.n_cu = kHeadThreads;  // the most score work groups a call has
    if (head_lds_bytes(probe) > static_cast<size_t>(kLdsLimit) ||
        finish_lds_bytes(probe) > static_cast<size_t>(kLdsLimit) ||
        score_lds_bytes(probe) > static_cast<size_t>(kLdsLimit))
      return fail(RETOPK_OUT_OF_RANGE, w + ": top_k / top_r / window need more LDS than a work group has");
  }
  const long long bh = static_cast<long long>(p.batch) * p.n_q_heads;
  if (bh > (1 << 20)) return fail(RETOPK_OUT_OF_RANGE, w + ": batch * n_q_heads too large");
  if (static_cast<long long>(p.batch) * p.n_kv_heads > 1024)
    return fail(RETOPK_OUT_OF_RANGE, w + ": batch * n_kv_heads must be <= 1024");
  return RETOPK_OK;
}

retopk_status current_device(int* dev, int* n_cu, const char* who) {
  int ndev = 0;
  if (hipGetDeviceCount(&ndev) != hipSuccess || ndev < 1) {
    (void)hipGetLastError();
    return fail(RETOPK_NO_DEVICE, std::string(who) + ": no HIP device visible");
  }
  if (hipGetDevice(dev) != hipSuccess) return fail(RETOPK_NO_DEVICE, std::string(who) + ": hipGetDevice failed");
  if (hipDeviceGetAttribute(n_cu, hipDeviceAttributeMultiprocessorCount, *dev) != hipSuccess || *n_cu < 1)
    return fail(RETOPK_NO_DEVICE, std::string(who) + ": cannot read the compute unit count");
  return RETOPK_OK;
}

Dims make_dims(const retopk_params& p, int n_cu) {
  Dims d{};
  d.B = p.batch;
  d.Hq = p.n_q_heads;
  d.Hkv = p.n_kv_heads;
  d.G = p.n_q_heads / p.n_kv_heads;
  d.max_len = p.max_len;
  d.score_stride = (p.max_len + 15) / 16 * 16;
  d.K = p.top_k;
  d.C = p.cache_cap;
  d.W = p.window;
  d.R = p.top_r;
  d.Tr = p.refresh_every;
  d.cand_cap = p.top_r * p.top_k + p.window;
  d.n_cu = n_cu;
  d.recent = p.retrieval == RETOPK_RETRIEVE_RECENT ? 1 : 0;
  d.tau = p.tau;
  return d;
}

}  // namespace

extern "C" {

const char* retopk_status_string(retopk_status s) {
  switch (s) {
    case RETOPK_OK: return "ok";
    case RETOPK_INVALID_ARG: return "invalid argument";
    case RETOPK_OUT_OF_RANGE: return "argument out of range";
    case RETOPK_HIP_ERROR: return "HIP runtime error";
    case RETOPK_NOT_INITIALIZED: return "handle not initialised";
    case RETOPK_NO_DEVICE: return "no GPU device";
  }
  return "unknown status";
}

const char* retopk_last_error(void) { return g_last_error.c_str(); }

int32_t retopk_kernel_count(void) { return kNumKernels; }

const char* retopk_kernel_name(int32_t id) { return kernel_name(id); }

size_t retopk_device_bytes(const retopk_handle* h) { return h ? h->bytes() : 0; }

retopk_status retopk_read_device_error(retopk_handle* h, int32_t* word) {
  if (h == nullptr) return fail(RETOPK_NOT_INITIALIZED, "retopk_read_device_error: NULL handle");
  if (word == nullptr) return fail(RETOPK_INVALID_ARG, "retopk_read_device_error: NULL output");
  DeviceGuard guard(h->device);
  hipError_t e = hipDeviceSynchronize();
  if (e == hipSuccess) e = hipMemcpy(word, h->b.err, sizeof(int32_t), hipMemcpyDeviceToHost);
  if (e == hipSuccess) e = hipMemset(h->b.err, 0, sizeof(int32_t));
  if (e == hipSuccess) e = hipDeviceSynchronize();
  return e == hipSuccess ? RETOPK_OK : hip_fail(e, "retopk_read_device_error");
}

retopk_status retopk_create(const retopk_params* params, retopk_handle** out) {
  if (out == nullptr) return fail(RETOPK_INVALID_ARG, "retopk_create: out is NULL");
  *out = nullptr;
  if (params == nullptr) return fail(RETOPK_INVALID_ARG, "retopk_create: params is NULL");
  retopk_status st = check_params(*params, "retopk_create");
  if (st != RETOPK_OK) return st;
  int dev = 0, n_cu = 0;
  st = current_device(&dev, &n_cu, "retopk_create");
  if (st != RETOPK_OK) return st;
  auto* h = new (std::nothrow) retopk_handle();
  if (h == nullptr) return fail(RETOPK_HIP_ERROR, "retopk_create: out of host memory");
  h->p = *params;
  h->device = dev;
  h->d = make_dims(*params, n_cu);
  hipError_t e = h->own.create(h->d);
  if (e == hipSuccess) e = h->create_layer();
  if (e == hipSuccess) e = configure_kernels(h->d);
  if (e == hipSuccess) e = hipDeviceSynchronize();
  if (e != hipSuccess) {
    h->release();
    delete h;
    return hip_fail(e, "retopk_create: device allocation");
  }
  *out = h;
  return RETOPK_OK;
}

void retopk_destroy(retopk_handle* h) {
  if (h == nullptr || h->group != nullptr) return;  // a group's layers go with the group
  {
    DeviceGuard guard(h->device);
    (void)hipDeviceSynchronize();
    h->release();
  }
  delete h;
}

retopk_status retopk_group_create(const retopk_params* params, int32_t n_layers, retopk_group** out) {
  if (out == nullptr) return fail(RETOPK_INVALID_ARG, "retopk_group_create: out is NULL");
  *out = nullptr;
  if (params == nullptr) return fail(RETOPK_INVALID_ARG, "retopk_group_create: params is NULL");
  if (n_layers < 1 || n_layers > kMaxGroupLayers)
    return fail(RETOPK_OUT_OF_RANGE, "retopk_group_create: n_layers must be in 1 .. 1024");
  retopk_status st = check_params(*params, "retopk_group_create");
  if (st != RETOPK_OK) return st;
  int dev = 0, n_cu = 0;
  st = current_device(&dev, &n_cu, "retopk_group_create");
  if (st != RETOPK_OK) return st;
  auto* g = new (std::nothrow) retopk_group();
  if (g == nullptr) return fail(RETOPK_HIP_ERROR, "retopk_group_create: out of host memory");
  g->p = *params;
  g->device = dev;
  g->d = make_dims(*params, n_cu);
  hipError_t e = g->ws.create(g->d);
  for (int l = 0; l < n_layers && e == hipSuccess; ++l) {
    auto* h = new (std::nothrow) retopk_handle();
    if (h == nullptr) {
      e = hipErrorOutOfMemory;
      break;
    }
    h->p = *params;
    h->device = dev;
    h->d = g->d;
    h->ws = &g->ws;
    h->group = g;
    g->layers.push_back(h);
    e = h->create_layer();
  }
  if (e == hipSuccess) e = configure_kernels(g->d);
  if (e == hipSuccess) e = hipDeviceSynchronize();
  if (e != hipSuccess) {
    g->release();
    delete g;
    return hip_fail(e, "retopk_group_create: device allocation");
  }
  *out = g;
  return RETOPK_OK;
}

void retopk_group_destroy(retopk_group* g) {
  if (g == nullptr) return;
  {
    DeviceGuard guard(g->device);
    (void)hipDeviceSynchronize();
    g->release();
  }
  delete g;
}

retopk_handle* retopk_group_layer(retopk_group* g, int32_t layer) {
  if (g == nullptr || layer < 0 || layer >= static_cast<int32_t>(g->layers.size())) return nullptr;
  return g->layers[layer];
}

size_t retopk_group_device_bytes(const retopk_group* g) {
  if (g == nullptr) return 0;
  size_t n = g->ws.mem.bytes;
  for (const retopk_handle* h : g->layers) n += h->mem.bytes;
  return n;
}

retopk_status retopk_group_set_position(retopk_group* g, int32_t length, int32_t t_dec) {
  if (g == nullptr) return fail(RETOPK_NOT_INITIALIZED, "retopk_group_set_position: NULL group");
  if (length < 1 || length > g->d.max_len)
    return fail(RETOPK_OUT_OF_RANGE, "retopk_group_set_position: length must be in 1 .. max_len");
  if (t_dec < 1) return fail(RETOPK_OUT_OF_RANGE, "retopk_group_set_position: t_dec must be >= 1");
  g->next_len = length;
  g->next_tdec = t_dec;
  g->ctl_stale = true;
  return RETOPK_OK;
}

retopk_status retopk_group_capture(retopk_group* g, const uint16_t* const* q, const uint16_t* const* k,
                                   const uint16_t* const* v, float* const* out, void* stream) {
  if (g == nullptr) return fail(RETOPK_NOT_INITIALIZED, "retopk_group_capture: NULL group");
  if (q == nullptr || k == nullptr || v == nullptr || out == nullptr)
    return fail(RETOPK_INVALID_ARG, "retopk_group_capture: NULL pointer array");
  if (stream == nullptr) return fail(RETOPK_INVALID_ARG, "retopk_group_capture: needs a created stream (not NULL)");
  const int n = static_cast<int>(g->layers.size());
  for (int l = 0; l < n; ++l) {
    if (q[l] == nullptr || k[l] == nullptr || v[l] == nullptr || out[l] == nullptr)
      return fail(RETOPK_INVALID_ARG, "retopk_group_capture: NULL tensor");
    if (!aligned(q[l], 16) || !aligned(k[l], 16) || !aligned(v[l], 16) || !aligned(out[l], 4))
      return fail(RETOPK_INVALID_ARG, "retopk_group_capture: misaligned tensor");
  }
  DeviceGuard guard(g->device);
  auto s = static_cast<hipStream_t>(stream);
  const Dims& d = g->d;
  const long q_sb = static_cast<long>(d.Hq) * kHeadDim, q_sh = kHeadDim;
  const bool wide = 2 * *static_cast<volatile int32_t*>(g->ws.hint_host) >= d.B * d.Hkv;
  hipGraph_t graph = nullptr;
  hipError_t e = hipStreamBeginCapture(s, hipStreamCaptureModeThreadLocal);
  if (e != hipSuccess) return hip_fail(e, "retopk_group_capture: hipStreamBeginCapture");
  hipError_t le = launch_advance(g->ws.ctl, n, s);
  for (int l = 0; l < n && le == hipSuccess; ++l) {
    const retopk_handle* h = g->layers[l];
    // sized for the longest length a replay can have; the position and the
    // call flag are read from the control words
    le = launch_step(d, h->b, q[l], q_sb, q_sh, k[l], v[l], out[l], nullptr, d.max_len, 0, kModeDecode,
                     h->stats ? 0 : -1, 1, 0, wide, s, g->ws.ctl, l);
  }
  e = hipStreamEndCapture(s, &graph);
  if (le != hipSuccess) {
    if (graph != nullptr) (void)hipGraphDestroy(graph);
    return hip_fail(le, "retopk_group_capture: launch");
  }
  if (e != hipSuccess) return hip_fail(e, "retopk_group_capture: hipStreamEndCapture");
  hipGraphExec_t exec = nullptr;
  e = hipGraphInstantiate(&exec, graph, nullptr, nullptr, 0);
  if (e != hipSuccess) {
    (void)hipGraphDestroy(graph);
    return hip_fail(e, "retopk_group_capture: hipGraphInstantiate");
  }
  if (g->exec != nullptr) (void)hipGraphExecDestroy(g->exec);
  if (g->graph != nullptr) (void)hipGraphDestroy(g->graph);
  g->graph = graph;
  g->exec = exec;
  return RETOPK_OK;
}

retopk_status retopk_group_replay(retopk_group* g, void* stream) {
  if (g == nullptr) return fail(RETOPK_NOT_INITIALIZED, "retopk_group_replay: NULL group");
  if (g->exec == nullptr) return fail(RETOPK_INVALID_ARG, "retopk_group_replay: nothing captured");
  if (g->next_len < 1) return fail(RETOPK_INVALID_ARG, "retopk_group_replay: no position set");
  if (g->next_len > g->d.max_len)
    return fail(RETOPK_OUT_OF_RANGE, "retopk_group_replay: the next token's length exceeds max_len");
  DeviceGuard guard(g->device);
  auto s = static_cast<hipStream_t>(stream);
  const int n = static_cast<int>(g->layers.size());
  hipError_t e = hipSuccess;
  if (g->ctl_stale || g->ws.call_seq != g->seq_at_replay) {
    // the words the replay's k_advance moves on to this token's position and to
    // the call sequence an eager call would take next
    e = launch_set_position(g->ws.ctl, g->next_len - 1, g->next_tdec - 1, g->ws.call_seq + 1 - n, s);
    if (e != hipSuccess) return hip_fail(e, "retopk_group_replay: control words");
  }
  e = hipGraphLaunch(g->exec, s);
  if (e != hipSuccess) return hip_fail(e, "retopk_group_replay: hipGraphLaunch");
  g->ws.call_seq = (g->ws.call_seq + n) & kSeqMask;
  g->seq_at_replay = g->ws.call_seq;
  g->ctl_stale = false;
  g->next_len += 1;
  g->next_tdec += 1;
  return RETOPK_OK;
}

retopk_status retopk_init_from_prefill(retopk_handle* h, const uint16_t* q_tail, const uint16_t* k,
                                       int32_t prompt_len, void* stream) {
  if (h == nullptr) return fail(RETOPK_NOT_INITIALIZED, "retopk_init_from_prefill: NULL handle");
  if (q_tail == nullptr || k == nullptr)
    return fail(RETOPK_INVALID_ARG, "retopk_init_from_prefill: NULL tensor");
  if (!aligned(q_tail, 16) || !aligned(k, 16))
    return fail(RETOPK_INVALID_ARG, "retopk_init_from_prefill: q_tail and k must be 16-byte aligned");
  if (prompt_len < 1 || prompt_len > h->d.max_len)
    return fail(RETOPK_OUT_OF_RANGE, "retopk_init_from_prefill: prompt_len must be in 1 .. max_len");
  DeviceGuard guard(h->device);
  const Dims& d = h->d;
  const Bufs& b = h->b;
  auto s = static_cast<hipStream_t>(stream);
  const int n0 = prompt_len < d.C ? prompt_len : d.C;
  const long q_sb = static_cast<long>(d.Hq) * n0 * kHeadDim, q_sh = static_cast<long>(n0) * kHeadDim;
  retopk_status st = h->run(kKReset, s, [&] { return launch_reset(d, b, s); });
  for (int i = 0; i < n0 && st == RETOPK_OK; ++i) {
    const int len = prompt_len - n0 + i + 1;  // causal: keys 0 .. p
    const uint16_t* qi = q_tail + static_cast<long>(i) * kHeadDim;
    const int flag = h->next_call_flag();
    st = h->run(kKStep, s, [&] {
      return launch_step(d, b, qi, q_sb, q_sh, k, nullptr, nullptr, nullptr, len, 0, kModeExact, -1, 1, flag, false,
                         s, nullptr, 0);
    });
  }
  return st;
}

retopk_status retopk_decode_step(retopk_handle* h, const uint16_t* q, const uint16_t* k,
                                 const uint16_t* v, int32_t length, int32_t t_dec, float* out,
                                 void* stream) {
  if (h == nullptr) return fail(RETOPK_NOT_INITIALIZED, "retopk_decode_step: NULL handle");
  if (q == nullptr || k == nullptr || v == nullptr || out == nullptr)
    return fail(RETOPK_INVALID_ARG, "retopk_decode_step: NULL tensor");
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(out, 4))
    return fail(RETOPK_INVALID_ARG, "retopk_decode_step: misaligned tensor");
  if (length < 1 || length > h->d.max_len)
    return fail(RETOPK_OUT_OF_RANGE, "retopk_decode_step: length must be in 1 .. max_len");
  if (t_dec < 1) return fail(RETOPK_OUT_OF_RANGE, "retopk_decode_step: t_dec must be >= 1");
  DeviceGuard guard(h->device);
  const Dims& d = h->d;
  const Bufs& b = h->b;
  auto s = static_cast<hipStream_t>(stream);
  const int slot = h->stats ? (t_dec - 1) % kStatsCap : -1;
  const long q_sb = static_cast<long>(d.Hq) * kHeadDim, q_sh = kHeadDim;
  const int flag = h->next_call_flag();
  // exact KV groups of a recent step, written by the device into host-mapped
  // memory (possibly stale; it only sizes the launch)
  const int recent_exact = *static_cast<volatile int32_t*>(h->ws->hint_host);
  const bool wide = 2 * recent_exact >= d.B * d.Hkv;
  retopk_status st = h->run(kKStep, s, [&] {
    return launch_step(d, b, q, q_sb, q_sh, k, v, out, nullptr, length, t_dec, kModeDecode, slot, 1, flag, wide, s,
                       nullptr, 0);
  });
  return st;
}

retopk_status retopk_exact_topk_attn(retopk_handle* h, const uint16_t* q, const uint16_t* k,
                                     const uint16_t* v, int32_t length, float* out, int32_t* sel_out,
                                     void* stream) {
  if (h == nullptr) return fail(RETOPK_NOT_INITIALIZED, "retopk_exact_topk_attn: NULL handle");
  if (q == nullptr || k == nullptr || v == nullptr || out == nullptr)
    return fail(RETOPK_INVALID_ARG, "retopk_exact_topk_attn: NULL tensor");
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(out, 4) ||
      (sel_out != nullptr && !aligned(sel_out, 4)))
    return fail(RETOPK_INVALID_ARG, "retopk_exact_topk_attn: misaligned tensor");
  if (length < 1 || length > h->d.max_len)
    return fail(RETOPK_OUT_OF_RANGE, "retopk_exact_topk_attn: length must be in 1 .. max_len");
  DeviceGuard guard(h->device);
  const Dims& d = h->d;
  const Bufs& b = h->b;
  auto s = static_cast<hipStream_t>(stream);
  const long q_sb = static_cast<long>(d.Hq) * kHeadDim, q_sh = kHeadDim;
  const int flag = h->next_call_flag();
  retopk_status st = h->run(kKStep, s, [&] {
    return launch_step(d, b, q, q_sb, q_sh, k, v, out, sel_out, length, 0, kModeExact, -1, 0, flag, false, s,
                       nullptr, 0);
  });
  return st;
}

retopk_status retopk_dense_attn(retopk_handle* h, const uint16_t* q, const uint16_t* k, const uint16_t* v,
                                int32_t length, float* out, void* stream) {
  if (h == nullptr) return fail(RETOPK_NOT_INITIALIZED, "retopk_dense_attn: NULL handle");
  if (q == nullptr || k == nullptr || v == nullptr || out == nullptr)
    return fail(RETOPK_INVALID_ARG, "retopk_dense_attn: NULL tensor");
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(out, 4))
    return fail(RETOPK_INVALID_ARG, "retopk_dense_attn: misaligned tensor");
  if (length < 1 || length > h->d.max_len)
    return fail(RETOPK_OUT_OF_RANGE, "retopk_dense_attn: length must be in 1 .. max_len");
  if (h->d.G > kDenseMaxGroup)
    return fail(RETOPK_OUT_OF_RANGE, "retopk_dense_attn: at most 8 query heads per KV head");
  DeviceGuard guard(h->device);
  auto s = static_cast<hipStream_t>(stream);
  retopk_status st = h->run(kKDense, s, [&] { return launch_dense(h->d, q, k, v, out, length, h->ws->dense_part, s, 0); });
  if (st != RETOPK_OK) return st;
  return h->run(kKDenseMerge, s, [&] { return launch_dense(h->d, q, k, v, out, length, h->ws->dense_part, s, 1); });
}

retopk_status retopk_dense_attn_noalloc(int32_t batch, int32_t n_q_heads, int32_t n_kv_heads, int32_t max_len,
                                        const uint16_t* q, const uint16_t* k, const uint16_t* v, int32_t length,
                                        float* out, void* stream) {
  if (q == nullptr || k == nullptr || v == nullptr || out == nullptr)
    return fail(RETOPK_INVALID_ARG, "retopk_dense_attn_noalloc: NULL tensor");
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(out, 4))
    return fail(RETOPK_INVALID_ARG, "retopk_dense_attn_noalloc: misaligned tensor");
  if (batch < 1 || n_q_heads < 1 || n_kv_heads < 1 || n_q_heads % n_kv_heads != 0)
    return fail(RETOPK_INVALID_ARG, "retopk_dense_attn_noalloc: batch and head counts must be >= 1, "
                                    "n_q_heads a multiple of n_kv_heads");
  if (n_q_heads / n_kv_heads > kDenseMaxGroup)
    return fail(RETOPK_OUT_OF_RANGE, "retopk_dense_attn_noalloc: at most 8 query heads per KV head");
  if (max_len < 1 || max_len > (1 << 24) || length < 1 || length > max_len)
    return fail(RETOPK_OUT_OF_RANGE, "retopk_dense_attn_noalloc: need 1 <= length <= max_len <= 2^24");
  if (static_cast<long long>(batch) * n_kv_heads > 1024)
    return fail(RETOPK_OUT_OF_RANGE, "retopk_dense_attn_noalloc: batch * n_kv_heads must be <= 1024");
  int dev = 0, n_cu = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&n_cu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n_cu < 1) {
    (void)hipGetLastError();
    return fail(RETOPK_NO_DEVICE, "retopk_dense_attn_noalloc: no usable device");
  }
  Dims d{};
  d.B = batch;
  d.Hq = n_q_heads;
  d.Hkv = n_kv_heads;
  d.G = n_q_heads / n_kv_heads;
  d.max_len = max_len;
  d.n_cu = n_cu;
  const size_t need = static_cast<size_t>(batch) * n_q_heads * dense_max_split(d) * kDensePart;
  if (need > kNoAllocScratchFloats)
    return fail(RETOPK_OUT_OF_RANGE, "retopk_dense_attn_noalloc: needs " + std::to_string(need * 4) +
                                         " bytes of scratch, more than its 4 MiB");
  float* part = nullptr;
  hipError_t e = dense_scratch(&part);
  if (e != hipSuccess) return hip_fail(e, "retopk_dense_attn_noalloc: scratch address");
  auto s = static_cast<hipStream_t>(stream);
  e = launch_dense(d, q, k, v, out, length, part, s, 0);
  if (e == hipSuccess) e = launch_dense(d, q, k, v, out, length, part, s, 1);
  return e == hipSuccess ? RETOPK_OK : hip_fail(e, "retopk_dense_attn_noalloc");
}

retopk_status retopk_stream_read(const void* buf, size_t bytes, uint32_t* sink, void* stream) {
  if (buf == nullptr || sink == nullptr) return fail(RETOPK_INVALID_ARG, "retopk_stream_read: NULL pointer");
  if (!aligned(buf, 16) || bytes % 16 != 0 || !aligned(sink, 4))
    return fail(RETOPK_INVALID_ARG, "retopk_stream_read: buf must be 16-byte aligned, bytes a multiple of 16");
  int dev = 0, n_cu = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&n_cu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n_cu < 1)
    return fail(RETOPK_NO_DEVICE, "retopk_stream_read: no usable device");
  if (bytes == 0) return RETOPK_OK;
  const hipError_t e = launch_stream_read(buf, bytes, sink, n_cu, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? RETOPK_OK : hip_fail(e, "retopk_stream_read");
}

retopk_status retopk_score_probe(int32_t use_mfma, const uint16_t* k, int64_t n_rows, const uint16_t* q,
                                float* sink, void* stream) {
  if (k == nullptr || q == nullptr || sink == nullptr)
    return fail(RETOPK_INVALID_ARG, "retopk_score_probe: NULL pointer");
  if (use_mfma != 0 && use_mfma != 1) return fail(RETOPK_INVALID_ARG, "retopk_score_probe: use_mfma must be 0 or 1");
  if (n_rows < 1 || n_rows > (int64_t(1) << 30))
    return fail(RETOPK_OUT_OF_RANGE, "retopk_score_probe: n_rows out of range");
  if (!aligned(k, 16) || !aligned(q, 16) || !aligned(sink, 4))
    return fail(RETOPK_INVALID_ARG, "retopk_score_probe: k and q must be 16-byte aligned");
  int dev = 0, n_cu = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&n_cu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n_cu < 1)
    return fail(RETOPK_NO_DEVICE, "retopk_score_probe: no usable device");
  const hipError_t e = launch_score_probe(use_mfma, k, static_cast<long>(n_rows), q, sink, n_cu,
                                          static_cast<hipStream_t>(stream));
  return e == hipSuccess ? RETOPK_OK : hip_fail(e, "retopk_score_probe");
}

retopk_status retopk_read_state(retopk_handle* h, float* qbar, int32_t* supp, int32_t* supp_len,
                                int32_t* count) {
  if (h == nullptr) return fail(RETOPK_NOT_INITIALIZED, "retopk_read_state: NULL handle");
  if (qbar == nullptr || supp == nullptr || supp_len == nullptr || count == nullptr)
    return fail(RETOPK_INVALID_ARG, "retopk_read_state: NULL buffer");
  DeviceGuard guard(h->device);
  const Dims& d = h->d;
  const size_t BH = static_cast<size_t>(d.B) * d.Hq, C = d.C, K = d.K, D = kHeadDim;
  std::vector<float> rq(BH * C * D);
  std::vector<int32_t> rs(BH * C * K), rl(BH * C), rf(BH * 2);
  hipError_t e = hipDeviceSynchronize();
  if (e == hipSuccess) e = hipMemcpy(rq.data(), h->b.cache_qbar, rq.size() * 4, hipMemcpyDeviceToHost);
  if (e == hipSuccess) e = hipMemcpy(rs.data(), h->b.cache_supp, rs.size() * 4, hipMemcpyDeviceToHost);
  if (e == hipSuccess) e = hipMemcpy(rl.data(), h->b.cache_len, rl.size() * 4, hipMemcpyDeviceToHost);
  if (e == hipSuccess) e = hipMemcpy(rf.data(), h->b.fifo, rf.size() * 4, hipMemcpyDeviceToHost);
  if (e != hipSuccess) return hip_fail(e, "retopk_read_state");
  std::memset(qbar, 0, BH * C * D * 4);
  std::memset(supp, 0, BH * C * K * 4);
  std::memset(supp_len, 0, BH * C * 4);
  for (size_t bh = 0; bh < BH; ++bh) {
    const int head = rf[2 * bh], n = rf[2 * bh + 1];
    const int oldest = (head - n + d.C) % d.C;
    count[bh] = n;
    for (int i = 0; i < n; ++i) {
      const size_t src = bh * C + (oldest + i) % d.C, dst = bh * C + i;
      std::memcpy(qbar + dst * D, rq.data() + src * D, D * 4);
      const int len = rl[src];
      supp_len[dst] = len;
      std::memcpy(supp + dst * K, rs.data() + src * K, static_cast<size_t>(len) * 4);
    }
  }
  return RETOPK_OK;
}

retopk_status retopk_write_state(retopk_handle* h, const float* qbar, const int32_t* supp,
                                 const int32_t* supp_len, const int32_t* count) {
  if (h == nullptr) return fail(RETOPK_NOT_INITIALIZED, "retopk_write_state: NULL handle");
  if (qbar == nullptr || supp == nullptr || supp_len == nullptr || count == nullptr)
    return fail(RETOPK_INVALID_ARG, "retopk_write_state: NULL buffer");
  const Dims& d = h->d;
  const size_t BH = static_cast<size_t>(d.B) * d.Hq, C = d.C, K = d.K, D = kHeadDim;
  std::vector<int32_t> rs(BH * C * K, 0), rl(BH * C, 0), rf(BH * 2, 0);
  std::vector<float> rq(BH * C * D, 0.f);
  for (size_t bh = 0; bh < BH; ++bh) {
    const int n = count[bh];
    if (n < 0 || n > d.C) return fail(RETOPK_OUT_OF_RANGE, "retopk_write_state: count out of range");
    for (int i = 0; i < n; ++i) {
      const size_t e = bh * C + i;
      const int len = supp_len[e];
      if (len < 0 || len > d.K) return fail(RETOPK_OUT_OF_RANGE, "retopk_write_state: supp_len out of range");
      for (int j = 0; j < len; ++j) {
        const int x = supp[e * K + j];
        if (x < 0 || x >= d.max_len) return fail(RETOPK_OUT_OF_RANGE, "retopk_write_state: support index out of range");
        if (j > 0 && x <= rs[e * K + j - 1])
          return fail(RETOPK_INVALID_ARG, "retopk_write_state: a support is not strictly ascending");
        rs[e * K + j] = x;
      }
      rl[e] = len;
      std::memcpy(rq.data() + e * D, qbar + e * D, D * 4);
    }
    rf[2 * bh] = n % d.C;
    rf[2 * bh + 1] = n;
  }
  DeviceGuard guard(h->device);
  hipError_t e = hipDeviceSynchronize();
  if (e == hipSuccess) e = hipMemcpy(h->b.cache_qbar, rq.data(), rq.size() * 4, hipMemcpyHostToDevice);
  if (e == hipSuccess) e = hipMemcpy(h->b.cache_supp, rs.data(), rs.size() * 4, hipMemcpyHostToDevice);
  if (e == hipSuccess) e = hipMemcpy(h->b.cache_len, rl.data(), rl.size() * 4, hipMemcpyHostToDevice);
  if (e == hipSuccess) e = hipMemcpy(h->b.fifo, rf.data(), rf.size() * 4, hipMemcpyHostToDevice);
  if (e == hipSuccess) e = hipDeviceSynchronize();
  if (e != hipSuccess) return hip_fail(e, "retopk_write_state");
  return RETOPK_OK;
}

retopk_status retopk_read_step_info(retopk_handle* h, int32_t* path, double* rho_max, int32_t* retrieved,
                                    int32_t* n_cand, int32_t* cand, int32_t* sel, int32_t* sel_len,
                                    float* sel_scores) {
  if (h == nullptr) return fail(RETOPK_NOT_INITIALIZED, "retopk_read_step_info: NULL handle");
  DeviceGuard guard(h->device);
  const Dims& d = h->d;
  const size_t BH = static_cast<size_t>(d.B) * d.Hq;
  hipError_t e = hipDeviceSynchronize();
  auto copy = [&](void* dst, const void* src, size_t n) {
    if (e == hipSuccess && dst != nullptr) e = hipMemcpy(dst, src, n, hipMemcpyDeviceToHost);
  };
  copy(path, h->b.path, BH * 4);
  copy(rho_max, h->b.rho, BH * 8);
  copy(retrieved, h->b.ret, BH * d.R * 4);
  copy(n_cand, h->b.m, BH * 4);
  copy(cand, h->b.cand, BH * d.cand_cap * 4);
  copy(sel, h->b.sel, BH * d.K * 4);
  copy(sel_len, h->b.sellen, BH * 4);
  copy(sel_scores, h->b.selsc, BH * d.K * 4);
  if (e != hipSuccess) return hip_fail(e, "retopk_read_step_info");
  return RETOPK_OK;
}

retopk_status retopk_read_stats(retopk_handle* h, int32_t first_t_dec, int32_t n_steps, uint8_t* path,
                                double* rho_max, int32_t* n_cand) {
  if (h == nullptr) return fail(RETOPK_NOT_INITIALIZED, "retopk_read_stats: NULL handle");
  if (path == nullptr || rho_max == nullptr || n_cand == nullptr)
    return fail(RETOPK_INVALID_ARG, "retopk_read_stats: NULL buffer");
  if (first_t_dec < 1 || n_steps < 0 || n_steps > kStatsCap)
    return fail(RETOPK_OUT_OF_RANGE, "retopk_read_stats: first_t_dec >= 1 and n_steps <= 4096 required");
  DeviceGuard guard(h->device);
  const size_t BH = static_cast<size_t>(h->d.B) * h->d.Hq;
  hipError_t e = hipDeviceSynchronize();
  for (int i = 0; i < n_steps && e == hipSuccess; ++i) {
    const size_t slot = static_cast<size_t>(first_t_dec - 1 + i) % kStatsCap;
    e = hipMemcpy(path + i * BH, h->b.st_path + slot * BH, BH, hipMemcpyDeviceToHost);
    if (e == hipSuccess) e = hipMemcpy(rho_max + i * BH, h->b.st_rho + slot * BH, BH * 8, hipMemcpyDeviceToHost);
    if (e == hipSuccess) e = hipMemcpy(n_cand + i * BH, h->b.st_m + slot * BH, BH * 4, hipMemcpyDeviceToHost);
  }
  if (e != hipSuccess) return hip_fail(e, "retopk_read_stats");
  return RETOPK_OK;
}

retopk_status retopk_set_stats(retopk_handle* h, int32_t enabled) {
  if (h == nullptr) return fail(RETOPK_NOT_INITIALIZED, "retopk_set_stats: NULL handle");
  h->stats = enabled != 0;
  return RETOPK_OK;
}

retopk_status retopk_set_timing(retopk_handle* h, int32_t enabled) {
  if (h == nullptr) return fail(RETOPK_NOT_INITIALIZED, "retopk_set_timing: NULL handle");
  h->timing = enabled != 0;
  return RETOPK_OK;
}

retopk_status retopk_read_kernel_times(retopk_handle* h, int32_t n, double* total_ms, int64_t* launches) {
  if (h == nullptr) return fail(RETOPK_NOT_INITIALIZED, "retopk_read_kernel_times: NULL handle");
  if (n < 0 || n > kNumKernels || (n > 0 && (total_ms == nullptr || launches == nullptr)))
    return fail(RETOPK_INVALID_ARG, "retopk_read_kernel_times: bad output buffers");
  DeviceGuard guard(h->device);
  hipError_t e = hipDeviceSynchronize();
  if (e != hipSuccess) return hip_fail(e, "retopk_read_kernel_times");
  for (int i = 0; i < n; ++i) {
    total_ms[i] = 0.0;
    launches[i] = 0;
  }
  for (int i = 0; i < h->timed; ++i) {
    float ms = 0.f;
    e = hipEventElapsedTime(&ms, h->events[2 * i], h->events[2 * i + 1]);
    if (e != hipSuccess) return hip_fail(e, "retopk_read_kernel_times: hipEventElapsedTime");
    const int id = h->event_kernel[i];
    if (id < n) {
      total_ms[id] += ms;
      launches[id] += 1;
    }
  }
  h->timed = 0;
  return RETOPK_OK;
}

}  // extern "C"
