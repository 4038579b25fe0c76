// Engine of the persistent decode megakernel: device memory of a bound
// schedule, the device task table, launches and region statistics.
#include <mutex>

#include "vm.h"

namespace amk {

// Streaming read of `bytes` (multiple of 16) at the rate the memory system
// sustains for this access pattern: workgroup b of G (512 threads) reads one
// contiguous 1/G of the buffer in 1 KB slabs (64 lanes x 16 bytes), its 8
// waves taking every 8th slab, 16 non-temporal loads per lane in flight.
// Loads past `bytes` return zero (buffer range check).  One word per
// workgroup is stored only if the data hash hits a constant, which keeps the
// loads live.
constexpr int kStreamDepth = 16;
__global__ void __launch_bounds__(512) amk_stream_read(const uint8_t* __restrict__ src, uint32_t bytes,
                                                        float* __restrict__ out) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const uint64_t nslab = ((uint64_t)bytes + 1023) / 1024;
  const uint64_t s0 = nslab * blockIdx.x / gridDim.x, s1 = nslab * (blockIdx.x + 1) / gridDim.x;
  const __amdgpu_buffer_rsrc_t r = rsrc(src, bytes);
  uint32_t acc = 0;
  u32x4 buf[kStreamDepth];
  auto off = [&](uint64_t k) {  // k-th slab of this wave
    const uint64_t sl = s0 + (uint64_t)w + 8 * k;
    return sl < s1 ? (uint32_t)(sl * 1024 + (uint64_t)lane * 16) : kOob;
  };
  const uint64_t n = (s1 - s0 + 7 - (uint64_t)w) / 8;  // slabs of this wave
#pragma unroll
  for (int k = 0; k < kStreamDepth; ++k) buf[k] = bload(r, off(k));
  for (uint64_t i = 0; i < n; i += kStreamDepth) {
#pragma unroll
    for (int k = 0; k < kStreamDepth; ++k) {
      acc ^= buf[k].x ^ buf[k].y ^ buf[k].z ^ buf[k].w;
      if (i + kStreamDepth + k < n) buf[k] = bload(r, off(i + kStreamDepth + k));
    }
  }
  if (acc == 0x9E3779B9u) out[blockIdx.x] = 1.0f;
}

// Zero `n` 32-bit words (grid-stride).  Used where the engine clears device
// state inside a caller's stream, in place of a memset node.
__global__ void __launch_bounds__(256) amk_fill_zero(uint32_t* __restrict__ p, uint64_t n) {
  for (uint64_t i = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (uint64_t)gridDim.x * blockDim.x)
    p[i] = 0u;
}

// enqueue amk_fill_zero over `bytes` (a multiple of 4) at p
hipError_t fill_zero(void* p, size_t bytes, hipStream_t st) {
  const uint64_t n = bytes / 4;
  const unsigned blocks = (unsigned)std::min<uint64_t>(1024, (n + 255) / 256 + 1);
  hipLaunchKernelGGL(amk_fill_zero, dim3(blocks), dim3(256), 0, st, static_cast<uint32_t*>(p), n);
  return hipGetLastError();
}

}  // namespace amk


// =================================================================== engine
namespace amk {
namespace {

#define HIP_TRY(call)                                                                          \
  do {                                                                                         \
    hipError_t e_ = (call);                                                                    \
    if (e_ != hipSuccess) return fail(AMK_ERR_HIP, std::string(#call) + ": " + hipGetErrorString(e_)); \
  } while (0)

template <int D>
const void* kernel_for_format(int wfmt, bool multi) {
  switch (wfmt) {
    case AMK_W_INT8_ROW: return vm_kernel<D, AMK_W_INT8_ROW>(multi);
    case AMK_W_INT4_G128: return vm_kernel<D, AMK_W_INT4_G128>(multi);
    default: return vm_kernel<D, AMK_W_BF16>(multi);
  }
}

// the single-step kernel (multi = false) or the greedy multi-step one
const void* kernel_for(int depth, int wfmt, bool multi) {
  switch (depth) {
    case 4: return kernel_for_format<4>(wfmt, multi);
    case 8: return kernel_for_format<8>(wfmt, multi);
    default: return kernel_for_format<16>(wfmt, multi);
  }
}

}  // namespace
}  // namespace amk

namespace amk {

// ---- the static scratch of amk_engine_create_noalloc -------------------
// One array per device (each device that loads the library holds its own
// copy until the process ends).  Host code never passes `scratch` itself to
// the device: its name is a host-side stand-in; the device address is
// looked up once per device with hipGetSymbolAddress and kept in
// g_noalloc[device].base.
constexpr size_t kNoAllocScratchBytes = (size_t)AMK_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) uint8_t scratch[kNoAllocScratchBytes];

constexpr int kMaxDevices = 64;
struct NoAllocDevice {
  uint8_t* base = nullptr;         // device address of `scratch` on this device
  const amk_engine* owner = nullptr;  // the engine whose regions the scratch holds
};
std::mutex g_noalloc_mu;
NoAllocDevice g_noalloc[kMaxDevices];

// The scratch's device address on device `dev` (the current device), looked
// up on the first call for that device.
amk_status noalloc_base(int dev, uint8_t** out) {
  if (dev < 0 || dev >= kMaxDevices) return fail(AMK_ERR_UNSUPPORTED, "device index beyond the static scratch table");
  std::lock_guard<std::mutex> lock(g_noalloc_mu);
  if (!g_noalloc[dev].base) {
    void* p = nullptr;
    const hipError_t err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (err != hipSuccess || !p)
      return fail(AMK_ERR_HIP, std::string("hipGetSymbolAddress(scratch): ") + hipGetErrorString(err));
    g_noalloc[dev].base = static_cast<uint8_t*>(p);
  }
  *out = g_noalloc[dev].base;
  return AMK_OK;
}

}  // namespace amk

struct amk_engine {
  amk_model_config model{};
  amk_schedule_config config{};
  int device = 0;
  const void* kernel = nullptr;        // one decode step per launch
  const void* kernel_multi = nullptr;  // greedy steps with on-device token feedback
  size_t lds_bytes = 0;
  amk::VmParams params{};
  // device allocations owned by the engine
  std::vector<void*> owned;
  uint32_t max_prod = 1;
  int32_t n_counters = 1;
  int64_t written = 0;  // positions 0..written-1 hold KV rows
  int64_t steps = 0;
  int wallclock_khz = 100000;
  int32_t n_tasks = 0;
  std::vector<int32_t> task_type, task_layer;  // host copies for the region statistics
  uint64_t* d_trace = nullptr;  // allocated on first amk_engine_set_trace(e, 1)
  // tagged activations: one arena, zeroed at creation (tag 0 is never a launch's)
  uint64_t* tag_arena = nullptr;
  size_t tag_arena_words = 0;
  std::vector<size_t> tag_words;
  // the schedule passes amk_multistep_check (amk_decode_steps allowed)
  bool multistep_ok = false;
  // num_cus + 1 zeros: queue offsets of a launch in which every queue is
  // empty (amk_engine_launch_empty)
  int32_t* qoff_empty = nullptr;
  // amk_engine_create_noalloc: every device region of the engine is carved
  // from this device's static scratch array (nothing allocated, nothing
  // freed); null for engines whose regions were allocated
  uint8_t* scratch = nullptr;
};

namespace amk {
namespace {

template <typename T>
amk_status dev_alloc(amk_engine* e, T** out, size_t count) {
  void* p = nullptr;
  const size_t bytes = std::max<size_t>(count * sizeof(T), 256);
  hipError_t err = hipMalloc(&p, bytes);
  if (err != hipSuccess) return fail(AMK_ERR_NOMEM, std::string("hipMalloc: ") + hipGetErrorString(err));
  e->owned.push_back(p);
  err = hipMemset(p, 0, bytes);
  if (err != hipSuccess) return fail(AMK_ERR_HIP, std::string("hipMemset: ") + hipGetErrorString(err));
  *out = static_cast<T*>(p);
  return AMK_OK;
}

// One device region of an engine: its size, where its address goes, and
// the host bytes it starts with (null: zeros).  An engine's regions are
// listed first and placed together, so that a schedule too large for the
// static scratch is refused before any of it is written.
struct Region {
  void** dst;
  size_t bytes;       // at least 256
  const void* host;   // host_bytes <= bytes copied in after zeroing
  size_t host_bytes;
};

template <typename T>
void add_region(std::vector<Region>* r, T** dst, size_t count) {
  r->push_back({reinterpret_cast<void**>(dst), std::max<size_t>(count * sizeof(T), 256), nullptr, 0});
}

template <typename T>
void add_region(std::vector<Region>* r, T** dst, const std::vector<T>& host) {
  r->push_back({reinterpret_cast<void**>(dst), std::max<size_t>(host.size() * sizeof(T), 256), host.data(),
                host.size() * sizeof(T)});
}

constexpr size_t kRegionAlign = 256;
inline size_t align_up(size_t v) { return (v + kRegionAlign - 1) & ~(kRegionAlign - 1); }

size_t regions_bytes(const std::vector<Region>& rs) {
  size_t off = 0;
  for (const Region& r : rs) off = align_up(off) + r.bytes;
  return off;
}

// Place, zero and fill the regions: from e->scratch when set, else each
// allocated (and owned by the engine).
amk_status place_regions(amk_engine* e, const std::vector<Region>& rs) {
  size_t off = 0;
  for (const Region& r : rs) {
    void* p = nullptr;
    if (e->scratch) {
      off = align_up(off);
      p = e->scratch + off;
      off += r.bytes;
    } else {
      const hipError_t err = hipMalloc(&p, r.bytes);
      if (err != hipSuccess) return fail(AMK_ERR_NOMEM, std::string("hipMalloc: ") + hipGetErrorString(err));
      e->owned.push_back(p);
    }
    HIP_TRY(hipMemset(p, 0, r.bytes));
    if (r.host_bytes) HIP_TRY(hipMemcpy(p, r.host, r.host_bytes, hipMemcpyHostToDevice));
    *r.dst = p;
  }
  return AMK_OK;
}

// whether engine e may use its device regions: always for allocated
// engines; for engines in the static scratch, only while the scratch of its
// device still holds its regions
bool regions_live(const amk_engine* e);

void free_engine(amk_engine* e) {
  for (void* p : e->owned) (void)hipFree(p);
  if (e->scratch) {
    std::lock_guard<std::mutex> lock(g_noalloc_mu);
    if (g_noalloc[e->device].owner == e) g_noalloc[e->device].owner = nullptr;
  }
  delete e;
}

bool regions_live(const amk_engine* e) {
  if (!e->scratch) return true;
  std::lock_guard<std::mutex> lock(g_noalloc_mu);
  return g_noalloc[e->device].owner == e;
}

amk_status check_live(const amk_engine* e) {
  if (!regions_live(e))
    return fail(AMK_ERR_INVALID_ARG, "a later amk_engine_create_noalloc on this device took over the static "
                                     "scratch that held this engine's state");
  return AMK_OK;
}

// The kernel derives every address from (type, params) and the standard
// buffer layout; refuse descriptions it cannot execute exactly as validated.
// The weight rows a GEMV task streams (rpu = 0 for other task types); must
// agree with the task functions of the kernel.
struct GemvShape {
  int32_t tensor = -1, rpu = 0;
  int64_t row0 = 0, nunits = 0, K = 0, rows_total = 0;
};
GemvShape gemv_shape(const amk_model_config& m, const Task& t) {
  const int64_t H = m.hidden, F = m.ffn, qd = (int64_t)m.n_heads * m.head_dim;
  const int64_t qkv_rows = (int64_t)(m.n_heads + 2 * m.n_kv_heads) * m.head_dim;
  GemvShape g;
  const int32_t l = t.p[0];
  switch (t.type) {
    case AMK_TASK_QKV: g = {3 + 6 * l + LB_QKV, 2, 2 * (int64_t)t.p[1], (int64_t)t.p[2] - t.p[1], H, qkv_rows}; break;
    case AMK_TASK_OPROJ: g = {3 + 6 * l + LB_O, 1, t.p[1], (int64_t)t.p[2] - t.p[1], qd, H}; break;
    case AMK_TASK_GATEUP: g = {3 + 6 * l + LB_GATEUP, 2, 2 * (int64_t)t.p[1], (int64_t)t.p[2] - t.p[1], H, 2 * F}; break;
    case AMK_TASK_DOWN: g = {3 + 6 * l + LB_DOWN, 1, t.p[1], (int64_t)t.p[2] - t.p[1], F, H}; break;
    case AMK_TASK_LMHEAD: g = {2, 1, t.p[0], (int64_t)t.p[1] - t.p[0], H, m.vocab}; break;
    default: break;
  }
  // O, down and LM-head rows go in pairs when their count is even
  if ((t.type == AMK_TASK_OPROJ || t.type == AMK_TASK_DOWN || t.type == AMK_TASK_LMHEAD) && g.nunits % 2 == 0) {
    g.rpu = 2;
    g.nunits /= 2;
  }
  return g;
}

// output rows a projection task holds in LDS (0 for the other task types)
int64_t task_res_rows(const Task& t) {
  switch (t.type) {
    case AMK_TASK_QKV: return 2 * ((int64_t)t.p[2] - t.p[1]);
    case AMK_TASK_GATEUP: return 2 * ((int64_t)t.p[2] - t.p[1]);
    case AMK_TASK_OPROJ:
    case AMK_TASK_DOWN: return (int64_t)t.p[2] - t.p[1];
    case AMK_TASK_LMHEAD: return (int64_t)t.p[1] - t.p[0];
    default: return 0;
  }
}

amk_status check_executable(const amk_schedule& s) {
  amk_schedule_config rc;
  if (resolve_config(s.model, s.config, &rc) != AMK_OK) return AMK_ERR_UNSUPPORTED;
  if (std::memcmp(&rc, &s.config, sizeof rc) != 0)
    return fail(AMK_ERR_UNSUPPORTED, "schedule config is not in resolved form");
  if ((int64_t)s.queues.size() != s.config.num_cus)
    return fail(AMK_ERR_UNSUPPORTED, "queue count differs from num_cus");
  if (3 + 6 * (int64_t)s.model.n_layers > 32767)
    return fail(AMK_ERR_UNSUPPORTED, "too many layers for the device task record");
  const std::vector<Buffer> std_buffers = buffer_table(s.model, s.config.attn_splits);
  if (s.buffers.size() != std_buffers.size())
    return fail(AMK_ERR_UNSUPPORTED, "buffer table differs from the library layout");
  for (size_t b = 0; b < std_buffers.size(); ++b)
    if (s.buffers[b].size != std_buffers[b].size || s.buffers[b].kind != std_buffers[b].kind)
      return fail(AMK_ERR_UNSUPPORTED, "buffer table differs from the library layout");
  const int64_t kmax = std::max({(int64_t)s.model.hidden, (int64_t)s.model.ffn,
                                 (int64_t)s.model.n_heads * s.model.head_dim});
  for (const Task& t : s.tasks) {
    // a NOP task only waits and signals: accesses it declares are never made
    if (t.type == AMK_TASK_NOP && !t.acc.empty())
      return fail(AMK_ERR_UNSUPPORTED, "a NOP task declares memory accesses the kernel would not make");
    // a task's weight rows are addressed with 32-bit buffer offsets
    if (task_res_rows(t) * kmax * 2 + 4096 > ((int64_t)1 << 31))
      return fail(AMK_ERR_UNSUPPORTED, "a task's weight rows exceed 2 GiB");
    if ((int)t.waits.size() > kMaxWaits || (int)t.sigs.size() > kMaxSigs)
      return fail(AMK_ERR_UNSUPPORTED, "a task has more than 4 waits or signals");
    if ((t.type == AMK_TASK_ATTN && t.p[3] != s.config.attn_splits) ||
        (t.type == AMK_TASK_MERGE && t.p[2] != s.config.attn_splits))
      return fail(AMK_ERR_UNSUPPORTED, "attention split count differs from the schedule config");
  }
  return AMK_OK;
}

}  // namespace
}  // namespace amk

using namespace amk;

namespace amk {
namespace {

// One cooperative launch of n steps starting at (token, pos).
amk_status launch_steps(amk_engine* e, int32_t token, int32_t pos, int32_t n, int32_t* tokens_out, void* stream) {
  if (!e) return fail(AMK_ERR_INVALID_ARG, "null engine");
  if (token < 0 || token >= e->model.vocab) return fail(AMK_ERR_OUT_OF_RANGE, "token out of range");
  if (pos < 0 || pos >= e->model.max_ctx) return fail(AMK_ERR_OUT_OF_RANGE, "pos out of range");
  if (n < 1 || (int64_t)pos + n > e->model.max_ctx)
    return fail(AMK_ERR_OUT_OF_RANGE, "steps must be >= 1 and end within max_ctx");
  if (pos > e->written)
    return fail(AMK_ERR_INVALID_ARG, "pos " + std::to_string(pos) + " leaves a gap: only " +
                                         std::to_string(e->written) + " positions are written");
  amk_status live = check_live(e);
  if (live != AMK_OK) return live;
  hipStream_t st = static_cast<hipStream_t>(stream);
  // (the clears below are fill kernels, not memset nodes, so that a caller
  // may capture these launches in a HIP graph)
  // counters are monotonic across launches; restart them well before u32 wraps
  if ((uint64_t)(e->params.epoch + n + 2) * e->max_prod >= (1ull << 31)) {
    HIP_TRY(fill_zero(e->params.ctr, sizeof(uint32_t) * kCounterStride * e->n_counters, st));
    e->params.epoch = 0;
  }
  // a launch's tags are never reused while words of an earlier launch may
  // hold them: near the wrap the tagged words are cleared and tags start
  // again from 1
  if ((uint64_t)e->params.tag + (uint64_t)n >= 0xFFFFFFFFull) {
    if (e->tag_arena) HIP_TRY(fill_zero(e->tag_arena, e->tag_arena_words * sizeof(uint64_t), st));
    HIP_TRY(fill_zero(e->params.targ, sizeof(uint64_t) * 2 * std::max(1, e->params.n_lm), st));
    e->params.tag = 1;
  }
  e->params.token = token;
  e->params.pos = pos;
  e->params.n_steps = n;
  e->params.tokens_out = tokens_out;
  void* args[] = {&e->params};
  HIP_TRY(hipLaunchCooperativeKernel(tokens_out ? e->kernel_multi : e->kernel, dim3(e->config.num_cus), dim3(kThreads), args,
                                     (unsigned)e->lds_bytes, st));
  e->params.epoch += (uint32_t)n;
  e->params.tag += (uint32_t)n;
  e->written = (int64_t)pos + n;
  e->steps += n;
  return AMK_OK;
}

}  // namespace
}  // namespace amk

namespace amk {
namespace {

// amk_engine_create (noalloc = false) and amk_engine_create_noalloc (true):
// the same engine, with its device regions allocated or carved from the
// device's static scratch.
amk_status create_engine(const amk_schedule* s, const amk_device_buffers* bufs, amk_engine** out, bool noalloc) {
  if (!s || !bufs || !out) return fail(AMK_ERR_INVALID_ARG, "null argument");
  *out = nullptr;
  amk_verdict v;
  amk_status st = amk_validate(s, &v);
  if (st != AMK_OK) return st;  // unsafe schedules never reach the GPU
  st = check_model(s->model);
  if (st != AMK_OK) return st;
  st = check_executable(*s);
  if (st != AMK_OK) return st;
  const amk_model_config& m = s->model;
  const amk_schedule_config& c = s->config;
  const int32_t npacked = 3 + 6 * m.n_layers;
  if (!bufs->weights || bufs->n_weights != npacked || !bufs->kv_cache || !bufs->logits)
    return fail(AMK_ERR_INVALID_ARG, "device buffers: need " + std::to_string(npacked) +
                                         " packed weights, a KV cache and a logits buffer");
  for (int32_t k = 0; k < npacked; ++k)
    if (!bufs->weights[k]) return fail(AMK_ERR_INVALID_ARG, "packed weight " + std::to_string(k) + " is null");

  int dev = 0;
  HIP_TRY(hipGetDevice(&dev));
  hipDeviceProp_t prop;
  HIP_TRY(hipGetDeviceProperties(&prop, dev));
  if (!prop.cooperativeLaunch) return fail(AMK_ERR_UNSUPPORTED, "device lacks cooperative launch");

  amk_engine* e = new (std::nothrow) amk_engine();
  if (!e) return fail(AMK_ERR_NOMEM, "out of host memory");
  e->model = m;
  e->config = c;
  e->device = dev;
  e->multistep_ok = multistep_unsafe_task(*s) == -1;
  auto bail = [&](amk_status code) {
    free_engine(e);
    return code;
  };
  if (noalloc && (st = noalloc_base(dev, &e->scratch)) != AMK_OK) return bail(st);

  // ---- LDS plan (floats).  Every task uses [0, lower(task)): the head, then
  // a GEMV task's staged input and partial tables, or the attention scratch.
  // Weight prefetch areas sit at the top of the workgroup's LDS.
  const int64_t hd = m.head_dim;
  const int64_t E = m.wfmt == AMK_W_BF16 ? 8 : (m.wfmt == AMK_W_INT8_ROW ? 16 : 32);
  auto xs_fl = [&](int64_t K) {
    const int64_t padded = (K + E * 64 - 1) / (E * 64) * (E * 64);
    return (padded + padded / 32 + 3) / 4 * 4;
  };
  // attention: the larger of the two lane layouts' scratch
  // (attn_lds_floats); merge: [S][hd + 1]
  const int64_t att_floats =
      std::max<int64_t>(attn_lds_floats(m.n_heads / m.n_kv_heads, (int)hd), (int64_t)c.attn_splits * (hd + 1));
  const int64_t lds_att = kHead;
  auto lower = [&](const Task& t) -> int64_t {
    const GemvShape g = gemv_shape(m, t);
    if (g.rpu) return kHead + xs_fl(g.K) + (g.nunits * g.rpu + 3) / 4 * 4 * (1 + kWaves);
    if (t.type == AMK_TASK_ATTN || t.type == AMK_TASK_MERGE) return lds_att + att_floats;
    return kHead;
  };
  int64_t total_floats = kHead;
  for (const Task& t : s->tasks) total_floats = std::max(total_floats, lower(t));
  const bool prefetch = c.prefetch_kb > 0 || c.prefetch_attn_kb > 0;
  const int64_t lds_total = std::min<int64_t>((int64_t)prop.sharedMemPerBlock, 163840);
  e->lds_bytes = prefetch ? (size_t)lds_total : (size_t)total_floats * 4;
  if ((int64_t)total_floats * 4 > lds_total)
    return (free_engine(e), fail(AMK_ERR_UNSUPPORTED, "schedule needs " + std::to_string(total_floats * 4) +
                                                          " bytes of LDS per workgroup; device allows " +
                                                          std::to_string(lds_total)));
  if (e->lds_bytes > (size_t)prop.sharedMemPerBlock)
    return (free_engine(e), fail(AMK_ERR_UNSUPPORTED, "schedule needs " + std::to_string(e->lds_bytes) +
                                                          " bytes of LDS per workgroup; device allows " +
                                                          std::to_string(prop.sharedMemPerBlock)));
  e->kernel = kernel_for(c.pipeline_depth, m.wfmt, false);
  e->kernel_multi = kernel_for(c.pipeline_depth, m.wfmt, true);
  for (const void* k : {e->kernel, e->kernel_multi}) {
    if (e->lds_bytes > 65536) {
      hipError_t err = hipFuncSetAttribute(k, hipFuncAttributeMaxDynamicSharedMemorySize, (int)e->lds_bytes);
      if (err != hipSuccess) return bail(fail(AMK_ERR_HIP, std::string("hipFuncSetAttribute: ") + hipGetErrorString(err)));
    }
    int per_cu = 0;
    hipError_t oerr = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, k, kThreads, e->lds_bytes);
    if (oerr != hipSuccess) return bail(fail(AMK_ERR_HIP, std::string("occupancy query: ") + hipGetErrorString(oerr)));
    if ((int64_t)per_cu * prop.multiProcessorCount < c.num_cus)
      return bail(fail(AMK_ERR_UNSUPPORTED, std::to_string(c.num_cus) + " queues exceed the " +
                                                std::to_string(per_cu * prop.multiProcessorCount) +
                                                " co-resident workgroups of this device"));
  }
  int khz = 0;
  if (hipDeviceGetAttribute(&khz, hipDeviceAttributeWallClockRate, dev) == hipSuccess && khz > 0)
    e->wallclock_khz = khz;

  // ---- device task table
  std::vector<uint32_t> P = counter_producers(*s);
  e->max_prod = 1;
  for (uint32_t p : P) e->max_prod = std::max(e->max_prod, p);
  e->n_counters = std::max(1, s->n_counters);
  e->n_tasks = (int32_t)s->tasks.size();
  e->task_type.resize(s->tasks.size());
  e->task_layer.resize(s->tasks.size());
  for (size_t i = 0; i < s->tasks.size(); ++i) {
    e->task_type[i] = s->tasks[i].type;
    e->task_layer[i] = s->tasks[i].type == AMK_TASK_LMHEAD ? m.n_layers : s->tasks[i].p[0];
  }
  std::vector<DevTask> dt(s->tasks.size());
  int32_t n_lm = 0;
  for (size_t i = 0; i < s->tasks.size(); ++i) {
    const Task& t = s->tasks[i];
    DevTask d{};
    d.type = t.type;
    d.id = (int32_t)i;
    d.qslot = 0;
    d.nwait = (int8_t)t.waits.size();
    d.nsig = (int8_t)t.sigs.size();
    std::copy(t.p, t.p + 6, d.p);
    for (size_t k = 0; k < t.waits.size(); ++k) {
      d.wctr[k] = t.waits[k].ctr;
      d.wthr[k] = t.waits[k].thr;
      d.wprod[k] = P[t.waits[k].ctr];
    }
    for (size_t k = 0; k < t.sigs.size(); ++k) d.sctr[k] = t.sigs[k];
    if (t.type == AMK_TASK_LMHEAD) d.p[2] = n_lm++;  // slot of its argmax partial
    dt[i] = d;
  }
  for (const auto& q : s->queues)
    for (size_t k = 0; k < q.size(); ++k) dt[q[k]].qslot = (int32_t)(k & 1);
  // weight prefetch: the task before a GEMV task in its queue copies the
  // GEMV's first slabs into LDS above everything the tasks from the issuer
  // to the GEMV use, and at most ~56 DMA loads outstanding per issuing wave.
  // MERGE tasks are stepped over (the task before them issues the copy, so
  // a merge's loads do not queue behind it); the budget is prefetch_attn_kb
  // when attention work precedes the GEMV in its queue, else prefetch_kb.
  if (prefetch)
    for (const auto& q : s->queues)
      for (size_t k = 1; k < q.size(); ++k) {
        const Task& b = s->tasks[q[k]];
        const GemvShape g = gemv_shape(m, b);
        if (!g.rpu) continue;
        // the issuer steps back over MERGE tasks (and, with DMA waves,
        // over ATTN tasks too: their input reads and the copy are in
        // different waves, so the O projection streams during attention)
        const bool dma3 = c.poll_mode == 3;
        auto skip = [&](int32_t ty) { return ty == AMK_TASK_MERGE || (dma3 && ty == AMK_TASK_ATTN); };
        size_t j = k - 1;
        int64_t used_f = lower(b);
        while (j > 0 && skip(s->tasks[q[j]].type)) used_f = std::max(used_f, lower(s->tasks[q[j--]]));
        used_f = std::max(used_f, lower(s->tasks[q[j]]));
        const int32_t prev_ty = s->tasks[q[k - 1]].type;
        const int32_t kb = prev_ty == AMK_TASK_ATTN || prev_ty == AMK_TASK_MERGE ? c.prefetch_attn_kb : c.prefetch_kb;
        if (kb <= 0) continue;
        const int64_t per_row = 1024 + (m.wfmt == AMK_W_INT4_G128 ? 256 : 0);
        const int64_t step = g.rpu * per_row;
        const int64_t used = 4 * used_f;
        const int64_t avail = std::min<int64_t>(lds_total - used - 64, (int64_t)kb * 1024);
        // DMA loads outstanding per issuing wave: about 56 when waves 1..7
        // each copy their own steps and a seventh of wave 0's; at most 60
        // when each of the two DMA waves copies the steps of four waves
        const int64_t loads_per_step = g.rpu * (m.wfmt == AMK_W_INT4_G128 ? 2 : 1);
        const int64_t dma_cap = dma3 ? 60 / (4 * loads_per_step) : 49 / loads_per_step;
        const int64_t steps = std::min<int64_t>(avail / (kWaves * step), dma_cap);
        if (steps < 1) continue;
        const int64_t off = lds_total - kWaves * steps * step;
        DevTask& d = dt[q[k]];
        d.pf_have = (int8_t)steps;
        d.pf_lds = (int32_t)off;
        DevTask& a = dt[q[j]];
        a.pfn_tensor = (int16_t)g.tensor;
        a.pfn_row0 = (int32_t)g.row0;
        a.pfn_nunits = (int32_t)g.nunits;
        a.pfn_rpu = (int8_t)g.rpu;
        a.pfn_K = (int32_t)g.K;
        a.pfn_steps = (int8_t)steps;
        a.pfn_lds = (int32_t)off;
        a.pfn_rows_total = (int32_t)g.rows_total;
      }
  std::vector<int32_t> qoff(1, 0), queue;
  for (const auto& q : s->queues) {
    queue.insert(queue.end(), q.begin(), q.end());
    qoff.push_back((int32_t)queue.size());
  }
  // RoPE table in double, stored fp32: (cos, sin)(pos * theta^(-2i/hd))
  const int64_t half = hd / 2;
  std::vector<float2> rope((size_t)m.max_ctx * half);
  for (int64_t p = 0; p < m.max_ctx; ++p)
    for (int64_t i = 0; i < half; ++i) {
      const double ang = (double)p * std::pow((double)m.rope_theta, -2.0 * (double)i / (double)hd);
      rope[p * half + i] = make_float2((float)std::cos(ang), (float)std::sin(ang));
    }
  std::vector<const uint8_t*> wptr(npacked);
  for (int32_t k = 0; k < npacked; ++k) wptr[k] = static_cast<const uint8_t*>(bufs->weights[k]);

  VmParams& pr = e->params;
  DevTask* d_tasks = nullptr;
  int32_t *d_qoff = nullptr, *d_queue = nullptr, *d_qoff_empty = nullptr;
  const uint8_t** d_wptr = nullptr;
  float2* d_rope = nullptr;
  const int64_t L = m.n_layers, S = c.attn_splits, H = m.hidden, F = m.ffn;
  const int64_t qd = (int64_t)m.n_heads * m.head_dim;
  pr.tagged = c.sync_mode != 0;
  pr.a_tagged = c.sync_mode == 1;
  pr.tag = 1;
  pr.n_steps = 1;
  pr.n_lm = n_lm;
  pr.tokens_out = nullptr;
  const std::vector<int32_t> qoff_empty((size_t)c.num_cus + 1, 0);
  std::vector<Region> regions;
  add_region(&regions, &d_tasks, dt);
  add_region(&regions, &d_qoff, qoff);
  add_region(&regions, &d_qoff_empty, qoff_empty);
  add_region(&regions, &d_queue, queue);
  add_region(&regions, &d_wptr, wptr);
  add_region(&regions, &d_rope, rope);
  add_region(&regions, &pr.x, (size_t)(L * 2 * H));
  add_region(&regions, &pr.q, (size_t)(L * qd));
  add_region(&regions, &pr.part, (size_t)(L * m.n_heads * S * (hd + 2)));
  add_region(&regions, &pr.o, (size_t)(L * qd));
  add_region(&regions, &pr.a, (size_t)(L * F));
  add_region(&regions, &pr.ctr, (size_t)std::max(1, s->n_counters) * kCounterStride);
  add_region(&regions, &pr.err, 64);
  add_region(&regions, &pr.targ, (size_t)std::max(1, n_lm) * 2);
  uint64_t* arena = nullptr;
  e->tag_words.clear();
  if (pr.tagged) {
    const int64_t nkvd = (int64_t)m.n_kv_heads * hd;
    size_t n = 0;
    for (int64_t w : {L * 2 * H, L * qd, L * 2 * nkvd, L * m.n_heads * S * (hd + 2), L * qd, L * F}) {
      e->tag_words.push_back((size_t)w);
      n += (size_t)w;
    }
    add_region(&regions, &arena, n);
    e->tag_arena_words = n;
  }
  if (e->scratch && regions_bytes(regions) > kNoAllocScratchBytes)
    return bail(fail(AMK_ERR_UNSUPPORTED, "the engine needs " + std::to_string(regions_bytes(regions)) +
                                              " bytes of device scratch; amk_engine_create_noalloc holds at most " +
                                              std::to_string(kNoAllocScratchBytes)));
  if ((st = place_regions(e, regions)) != AMK_OK) return bail(st);
  if (pr.tagged) {
    e->tag_arena = arena;
    uint64_t** dst[] = {&pr.tx, &pr.tq, &pr.tkv, &pr.tpart, &pr.to, &pr.ta};
    size_t off = 0;
    for (int k = 0; k < 6; ++k) {
      *dst[k] = arena + off;
      off += e->tag_words[k];
    }
  }
  pr.tasks = d_tasks;
  pr.queue_off = d_qoff;
  e->qoff_empty = d_qoff_empty;
  pr.queue = d_queue;
  pr.wptr = d_wptr;
  pr.rope = d_rope;
  pr.kv = static_cast<uint16_t*>(bufs->kv_cache);
  pr.logits = bufs->logits;
  pr.L = m.n_layers;
  pr.H = m.hidden;
  pr.nq = m.n_heads;
  pr.nkv = m.n_kv_heads;
  pr.hd = m.head_dim;
  pr.F = m.ffn;
  pr.V = m.vocab;
  pr.mc = m.max_ctx;
  pr.S = c.attn_splits;
  pr.wfmt = m.wfmt;
  pr.act_bf16 = m.act_bf16;
  pr.eps = m.rms_eps;
  pr.lds_att = (int32_t)lds_att;
  pr.poll_late = c.poll_mode;
  pr.rel0 = c.release_mode;
  pr.spin_ticks = (uint64_t)2000000 * (uint64_t)e->wallclock_khz / 1000u;
  if (noalloc) {
    // the scratch now holds this engine's regions: an earlier engine made
    // by amk_engine_create_noalloc on this device can no longer run
    std::lock_guard<std::mutex> lock(g_noalloc_mu);
    g_noalloc[dev].owner = e;
  }
  *out = e;
  return AMK_OK;
}

}  // namespace
}  // namespace amk

extern "C" {

amk_status amk_engine_create(const amk_schedule* s, const amk_device_buffers* bufs, amk_engine** out) {
  return amk::create_engine(s, bufs, out, false);
}

amk_status amk_engine_create_noalloc(const amk_schedule* s, const amk_device_buffers* bufs, amk_engine** out) {
  return amk::create_engine(s, bufs, out, true);
}

amk_status amk_decode_step(amk_engine* e, int32_t token, int32_t pos, void* stream) {
  return amk::launch_steps(e, token, pos, 1, nullptr, stream);
}

amk_status amk_decode_steps(amk_engine* e, int32_t token, int32_t pos, int32_t n_steps, int32_t* tokens_out,
                            void* stream) {
  if (!tokens_out) return fail(AMK_ERR_INVALID_ARG, "null tokens_out");
  if (e && !e->multistep_ok)
    return fail(AMK_ERR_UNSUPPORTED, "the engine's schedule fails amk_multistep_check: a multi-step launch could "
                                     "start a step while a task of the previous one still runs");
  return amk::launch_steps(e, token, pos, n_steps, tokens_out, stream);
}

amk_status amk_engine_launch_empty(amk_engine* e, void* stream) {
  if (!e) return fail(AMK_ERR_INVALID_ARG, "null engine");
  amk_status live = check_live(e);
  if (live != AMK_OK) return live;
  amk::VmParams p = e->params;
  p.queue_off = e->qoff_empty;
  p.n_steps = 1;
  p.tokens_out = nullptr;
  void* args[] = {&p};
  HIP_TRY(hipLaunchCooperativeKernel(e->kernel, dim3(e->config.num_cus), dim3(kThreads), args, (unsigned)e->lds_bytes,
                                     static_cast<hipStream_t>(stream)));
  return AMK_OK;
}

amk_status amk_engine_check(amk_engine* e) {
  if (!e) return fail(AMK_ERR_INVALID_ARG, "null engine");
  amk_status live = check_live(e);
  if (live != AMK_OK) return live;
  int32_t err = 0;
  HIP_TRY(hipMemcpy(&err, e->params.err, sizeof(err), hipMemcpyDeviceToHost));
  if (err != 0) {
    // counters of an aborted launch are inconsistent: restart from zero
    HIP_TRY(hipMemset(e->params.ctr, 0, sizeof(uint32_t) * kCounterStride * e->n_counters));
    HIP_TRY(hipMemset(e->params.err, 0, sizeof(int32_t)));
    e->params.epoch = 0;
    return fail(AMK_ERR_TIMEOUT, "a device-side wait exceeded its spin budget");
  }
  return AMK_OK;
}

amk_status amk_engine_set_kv_length(amk_engine* e, int32_t n) {
  if (!e) return fail(AMK_ERR_INVALID_ARG, "null engine");
  if (n < 0 || n > e->model.max_ctx) return fail(AMK_ERR_OUT_OF_RANGE, "kv length out of range");
  e->written = n;
  return AMK_OK;
}

amk_status amk_engine_set_trace(amk_engine* e, int32_t enable) {
  if (!e) return fail(AMK_ERR_INVALID_ARG, "null engine");
  if (e->scratch && enable)
    return fail(AMK_ERR_UNSUPPORTED, "tracing allocates its stamp buffer: not available on an engine made by "
                                     "amk_engine_create_noalloc");
  if (enable && !e->d_trace) {
    amk_status st = dev_alloc(e, &e->d_trace, (size_t)std::max(1, e->n_tasks) * 4);
    if (st != AMK_OK) return st;
  }
  e->params.trace = enable ? e->d_trace : nullptr;
  return AMK_OK;
}

amk_status amk_engine_read_trace(amk_engine* e, uint64_t* out, int64_t n_values, int32_t* clock_khz) {
  if (!e || !out) return fail(AMK_ERR_INVALID_ARG, "null argument");
  if (!e->d_trace) return fail(AMK_ERR_INVALID_ARG, "tracing was never enabled");
  if (n_values != (int64_t)e->n_tasks * 4) return fail(AMK_ERR_INVALID_ARG, "need 4 values per task");
  HIP_TRY(hipMemcpy(out, e->d_trace, sizeof(uint64_t) * n_values, hipMemcpyDeviceToHost));
  if (clock_khz) *clock_khz = e->wallclock_khz;
  return AMK_OK;
}

amk_status amk_engine_region_stats(amk_engine* e, amk_region_stat* out) {
  if (!e || !out) return fail(AMK_ERR_INVALID_ARG, "null argument");
  if (!e->d_trace) return fail(AMK_ERR_INVALID_ARG, "tracing was never enabled");
  const size_t n = (size_t)e->n_tasks;
  std::vector<uint64_t> st(4 * n);
  HIP_TRY(hipMemcpy(st.data(), e->d_trace, sizeof(uint64_t) * st.size(), hipMemcpyDeviceToHost));
  const double us = 1e3 / (double)e->wallclock_khz;
  for (int k = 0; k < AMK_TASK_NTYPES; ++k) out[k] = amk_region_stat{};
  uint64_t t0 = UINT64_MAX;
  for (size_t i = 0; i < n; ++i) t0 = std::min(t0, st[4 * i]);
  // the phases of a layer in dependency order; a phase's span runs from the
  // last signal of the phase before it (or the launch start) to its own
  static const int32_t order[] = {AMK_TASK_QKV, AMK_TASK_ATTN, AMK_TASK_MERGE, AMK_TASK_OPROJ, AMK_TASK_GATEUP,
                                  AMK_TASK_DOWN};
  const int32_t L = e->model.n_layers;
  std::vector<uint64_t> last((size_t)(L + 1) * AMK_TASK_NTYPES, 0);
  for (size_t i = 0; i < n; ++i) {
    const int32_t ty = e->task_type[i];
    amk_region_stat& r = out[ty];
    r.n_tasks += 1;
    r.wait_us += (double)(st[4 * i + 1] - st[4 * i]) * us;
    r.work_us += (double)(st[4 * i + 2] - st[4 * i + 1]) * us;
    r.signal_us += (double)(st[4 * i + 3] - st[4 * i + 2]) * us;
    uint64_t& l = last[(size_t)e->task_layer[i] * AMK_TASK_NTYPES + ty];
    l = std::max(l, st[4 * i + 3]);
  }
  uint64_t prev = t0;
  for (int32_t l = 0; l <= L; ++l) {
    for (int32_t ty : order) {
      if (l == L) break;
      const uint64_t end = last[(size_t)l * AMK_TASK_NTYPES + ty];
      if (end == 0) continue;
      out[ty].span_us += (double)(std::max(end, prev) - prev) * us;
      prev = std::max(end, prev);
    }
    if (l == L) {
      const uint64_t end = last[(size_t)L * AMK_TASK_NTYPES + AMK_TASK_LMHEAD];
      if (end != 0) out[AMK_TASK_LMHEAD].span_us += (double)(std::max(end, prev) - prev) * us;
    }
  }
  return AMK_OK;
}

amk_status amk_engine_set_spin_budget(amk_engine* e, int64_t us) {
  if (!e || us <= 0) return fail(AMK_ERR_INVALID_ARG, "bad engine or budget");
  e->params.spin_ticks = (uint64_t)us * (uint64_t)e->wallclock_khz / 1000u;
  return AMK_OK;
}

amk_status amk_engine_steps(const amk_engine* e, int64_t* out) {
  if (!e || !out) return fail(AMK_ERR_INVALID_ARG, "null argument");
  *out = e->steps;
  return AMK_OK;
}

amk_status amk_stream_read_probe(const void* src, size_t bytes, float* out, int32_t blocks, void* stream) {
  if (!src || !out || blocks < 1 || bytes % 16 || bytes == 0 || bytes >= ((size_t)1 << 31))
    return fail(AMK_ERR_INVALID_ARG, "bad probe arguments");
  hipLaunchKernelGGL(amk_stream_read, dim3(blocks), dim3(512), 0, static_cast<hipStream_t>(stream),
                     static_cast<const uint8_t*>(src), (uint32_t)bytes, out);
  HIP_TRY(hipGetLastError());
  return AMK_OK;
}

amk_status amk_engine_destroy(amk_engine* e) {
  if (!e) return AMK_OK;
  free_engine(e);
  return AMK_OK;
}

}  // extern "C"
