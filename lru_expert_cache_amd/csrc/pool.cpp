// Host runtime of the offloaded MoE layer: pool creation, the per-call
// orchestration (router -> resolve -> miss copies -> FFN -> combine), prefill
// double-buffered staging, the hybrid host worker, statistics.
//
// Pages (FreeToken, by title and section): experts in host RAM, a GPU LRU
// cache of expert slots, misses streamed over PCIe, hybrid split of a step's
// misses, one global pool across layers -- devpik article "FreeToken: Run
// Frontier MoE Models on Your Own GPU, and the RAM It Takes", section "Why a
// Huge MoE Model Fits on One Consumer GPU"; prefill copies every expert of a
// layer per chunk, layer N+1 copied while N computes, warning when the cache
// cannot hold the two staging layers -- same article, "Long Prompts Are the
// Bottleneck"; pinned host memory -- same article, "The Real Requirement Is
// System RAM".
#include <algorithm>
#include <chrono>
#include <cmath>
#include <cstdarg>
#include <cstdlib>
#include <functional>
#include <map>
#include <memory>
#include <thread>

#include "common.h"

namespace ftmoe {

static thread_local std::string g_err;

void set_error(const char* fmt, ...) {
  char buf[1024];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_err = buf;
}
const char* get_error() { return g_err.c_str(); }

bool ffn_shape_ok(int fmt, int hidden, int inter);

}  // namespace ftmoe

using namespace ftmoe;

struct ft_moe_pool {
  int L = 0, H = 0, I = 0, E = 0, k = 0, shared = 0, device = 0, cpu_threads = 8;
  std::unique_ptr<WorkerPool> workers;  // host threads of the hybrid split (created on first use)
  int64_t C = 0;
  std::vector<int32_t> fmt;
  ExpertLayout lay[4];
  int64_t canon_bytes[4] = {0, 0, 0, 0};
  int64_t slot_bytes = 0;
  double share_fmt[4] = {0.0, 0.0, 0.0, 0.0};  // hybrid share of each weight format (index FT_FMT_*)
  double gpu_rate[4] = {0.0, 0.0, 0.0, 0.0};   // device FFN bytes/s from the last mode measurement
  // in-situ observations of the hybrid path since the last share change
  // (ft_moe_rebalance): host-computed and streamed expert bytes and times
  struct Obs {
    double host_bytes = 0.0, host_sec = 0.0, copy_bytes = 0.0, copy_ms = 0.0;
  } obs[4];

  // pinned host store (device layout), one entry per distinct (blob, format)
  uint8_t* host_store = nullptr;
  const uint8_t* host_store_dev = nullptr;  // its device-visible address
  int64_t host_bytes = 0;
  std::vector<int64_t> key_off;     // [L*E]
  int64_t* key_off_dev = nullptr;   // [L*E] device copy (device-driven miss copies)
  std::vector<uint8_t> layer_contig;

  // Decode runs device-driven (the GPU copies its own misses; the host never
  // waits) unless the call needs the host: hybrid split, several waves, or
  // FT_MOE_DECODE_PATH=host / injected copy failures.
  bool dev_decode = true;
  int copy_wgs = 64;                // workgroups of the miss-copy kernel (a sweep measured 64 best)
  // debug (env FT_MOE_POISON at creation): every slot is filled with 0xFF
  // bytes (NaN block scales) just before a copy into it, so a reader that
  // races a copy produces NaN instead of stale values
  bool poison = false;
  // debug (env FT_MOE_DEBUG_CHECKSUM at creation): before an FFN reads a slot,
  // a kernel recomputes the slot's checksum and compares it with the key's
  // blob in the host store; each call then waits and reports a mismatch
  bool checksum = false;
  uint64_t* key_sum_dev = nullptr;  // [L*E] checksum of each key's blob (device layout)
  uint64_t* bad_dev = nullptr;      // [2] first mismatch: 1 + key, slot
  int64_t corrupt_copy = -1;        // FT_MOE_FAULT=corrupt:<n>: the n-th miss copy lands damaged (tests)
  // env FT_MOE_LOG=<n>: a counters line on stderr every n forward calls
  int log_every = 0;
  uint64_t log_calls = 0;

  // device memory
  uint8_t* arena = nullptr;
  uint8_t* shared_dev = nullptr;
  int64_t shared_stride = 0;
  float* router_dev = nullptr;
  DevTable tab{};

  // work buffers (grow with T)
  int cap_T = 0;
  double* z = nullptr;
  int32_t* sel = nullptr;
  float* w = nullptr;
  double* gap = nullptr;
  uint8_t* pair_flag = nullptr;
  int32_t* pair_slot = nullptr;
  int32_t* pair_row = nullptr;
  int32_t* row_tok = nullptr;
  float* row_w = nullptr;
  GroupDesc* groups = nullptr;
  int32_t* glist = nullptr;
  GroupDesc* gdesc = nullptr;  // descriptors in run order (what the FFN and copy kernels read)
  int32_t* count_max = nullptr;  // device INT32_MAX: the device count of a launch whose count the host knows
  int32_t* dev_header = nullptr;
  uint16_t* hbuf = nullptr;
  uint16_t* pbuf = nullptr;
  uint8_t* rb_host = nullptr;
  uint8_t* rb_dev = nullptr;
  int64_t rb_cap = 0;
  uint16_t* x_host = nullptr;       // pinned copy of x for host-computed experts
  uint16_t* cpu_out = nullptr;      // pinned result rows of host-computed experts
  int32_t* fail_dev = nullptr;      // [2*E] keys and slots whose copy failed
  // prefill MX activation modes
  int32_t* row_slot = nullptr;      // [rows] prefill: each row's slot in the MX GEMM activation tiles
  uint8_t* xq_codes = nullptr;      // [cap][H] (FP8) or [cap][H/2] (FP4): quantised x, row-major
  uint8_t* xq_scales = nullptr;     // [cap][H/32]
  uint8_t* tq_codes = nullptr;      // MX GEMM activation tiles (allocated at the first MX call): x
  uint8_t* tq_scales = nullptr;
  uint8_t* hq_codes = nullptr;      // and h, written by the gate/up GEMM while x tiles are read
  int64_t hq_blocks = 0;            // (tile, K step) blocks of the h tiles
  uint8_t* hq_scales = nullptr;
  int32_t* tiles = nullptr;         // [2 * max_tiles]
  int32_t* stage_agg = nullptr;     // staged resolve scratch (stage_agg_ints)
  int32_t max_tiles = 0;

  // Miss copies rotate over n_copy streams (several DMA queues overlap the
  // per-copy setup of one copy with the transfer of another); copy[0] also
  // carries the prefill staging copies.
  static constexpr int kMaxCopyStreams = 4;
  int n_copy = 2;
  hipStream_t copy[kMaxCopyStreams] = {nullptr, nullptr, nullptr, nullptr};
  hipEvent_t ev_copy_done[kMaxCopyStreams] = {nullptr, nullptr, nullptr, nullptr};
  hipStream_t copy_stream = nullptr;  // == copy[0]
  hipEvent_t ev_resolved = nullptr, ev_copied = nullptr, ev_sync = nullptr, ev_cpu_copied = nullptr;
  hipEvent_t ev_done[2] = {nullptr, nullptr}, ev_staged[2] = {nullptr, nullptr};
  bool cpu_copy_pending = false;

  int32_t stamp = 0;
  int prefill_next = 0;
  bool prefill_hit = false;          // the current chunk skips resident experts
  std::vector<int32_t> prefill_res;  // [L*E] slot of each resident key at chunk start (outside staging), else -1
  uint64_t copy_counter = 0;
  int64_t fault_copy = -1;
  // fault injection (FT_MOE_FAULT): fail the n-th device allocation of the
  // per-call work buffers / of the MX activation tiles, once (1-based)
  int fault_work_alloc = -1, fault_mx_alloc = -1;
  int work_allocs = 0, mx_allocs = 0;

  // copy time (ft_moe_stats::copy_ms): device-driven copies measure
  // themselves on the device wall clock (copy_clk scratch, copy_ticks per
  // layer); host-issued copies are bracketed by events, folded in per layer
  uint64_t* copy_clk = nullptr;    // [3]
  uint64_t* copy_ticks = nullptr;  // [L]
  double wall_khz = 0.0;
  std::vector<double> copy_ms_host;  // [L]
  struct CopyRec {
    int layer;
    hipEvent_t a, b;
    double bytes;  // streamed expert bytes (decode calls) for the in-situ rates, else 0
  };
  std::vector<CopyRec> copy_pending;

  // miss lists of the latest call; after a device-driven call they are read
  // from the resolve kernel's mapped readback when first asked for
  mutable std::vector<int32_t> last_se, last_ss, last_ce;
  mutable bool last_pending = false;

  // calls on different streams are ordered through this event
  hipEvent_t ev_call_done = nullptr;
  hipStream_t last_stream = nullptr;
  bool any_call = false;

  // stage timing (ft_moe_set_profiling)
  struct ProfRec {
    int stage;
    hipEvent_t a, b;
    double bytes, flops;
  };
  int32_t prof_mask = 0;  // bit i: time stage i
  std::vector<ProfRec> prof_pending;
  std::vector<hipEvent_t> prof_free;
  ft_moe_profile prof{};
  // device-driven calls: groups and rows behind the timed FFN and copy
  // stages are counted on the device (ResolveArgs::prof_cnt)
  uint64_t* prof_cnt_dev = nullptr;  // [3][4][2]
  uint64_t prof_cnt_seen[24] = {};
};

namespace {

struct DeviceGuard {
  int prev = -1;
  explicit DeviceGuard(int dev) {
    if (hipGetDevice(&prev) != hipSuccess) prev = -1;
    if (prev != dev) (void)hipSetDevice(dev);
  }
  ~DeviceGuard() {
    if (prev >= 0) (void)hipSetDevice(prev);
  }
};

template <typename T>
int dev_alloc(T** p, int64_t n) {
  if (hipMalloc(reinterpret_cast<void**>(p), size_t(n) * sizeof(T) + 16) != hipSuccess) {
    *p = nullptr;
    (void)hipGetLastError();
    set_error("device allocation of %lld bytes failed", (long long)(n * sizeof(T)));
    return FT_E_OOM_DEVICE;
  }
  return FT_OK;
}

void parallel_for(int n, int threads, const std::function<void(int, int)>& fn) {
  threads = std::max(1, std::min(threads, n));
  if (threads == 1) {
    fn(0, n);
    return;
  }
  std::vector<std::thread> th;
  const int chunk = (n + threads - 1) / threads;
  for (int t = 0; t < threads; ++t) {
    const int b = t * chunk, e = std::min(n, b + chunk);
    if (b >= e) break;
    th.emplace_back(fn, b, e);
  }
  for (auto& x : th) x.join();
}

template <typename T>
void dev_free(T*& q) {
  if (q) (void)hipFree(q);
  q = nullptr;
}

// A device allocation of the work buffers; fails when it is the pool's
// injected fault (FT_MOE_FAULT=work_alloc:<n>, once).
template <typename T>
int work_alloc(ft_moe_pool* p, T** q, int64_t n) {
  if (++p->work_allocs == p->fault_work_alloc) {
    p->fault_work_alloc = -1;
    *q = nullptr;
    set_error("injected failure of work-buffer allocation %d", p->work_allocs);
    return FT_E_OOM_DEVICE;
  }
  return dev_alloc(q, n);
}

void free_work_buffers(ft_moe_pool* p) {
  dev_free(p->z); dev_free(p->sel); dev_free(p->w); dev_free(p->gap); dev_free(p->pair_flag);
  dev_free(p->pair_slot); dev_free(p->pair_row); dev_free(p->row_tok); dev_free(p->row_w);
  dev_free(p->hbuf); dev_free(p->pbuf);
  dev_free(p->row_slot); dev_free(p->tiles); dev_free(p->xq_codes); dev_free(p->xq_scales);
  dev_free(p->stage_agg);
  dev_free(p->tq_codes); dev_free(p->tq_scales); dev_free(p->hq_codes); dev_free(p->hq_scales);
  if (p->rb_host) (void)hipHostFree(p->rb_host);
  if (p->x_host) (void)hipHostFree(p->x_host);
  if (p->cpu_out) (void)hipHostFree(p->cpu_out);
  p->rb_host = nullptr;
  p->rb_dev = nullptr;
  p->x_host = nullptr;
  p->cpu_out = nullptr;
  p->cap_T = 0;
}

// Grows the per-call buffers to T tokens.  Every buffer is freed and nulled
// first, and cap_T stays 0 until all of them exist, so a failed allocation
// leaves no dangling pointer and the next call simply tries again.
int ensure_capacity(ft_moe_pool* p, int T) {
  if (T <= p->cap_T) return FT_OK;
  const int cap = std::max(T, 64);
  FT_HIP_CHECK(hipDeviceSynchronize());  // earlier calls may still use the old buffers
  free_work_buffers(p);
  const int64_t pairs = int64_t(cap) * p->k;
  const int64_t rows = pairs + (p->shared ? cap : 0);
  const int tr = mx_gemm_rows_per_tile();
  p->max_tiles = int32_t((pairs + tr - 1) / tr + p->E + (cap + tr - 1) / tr + 2);
  int rc;
  if ((rc = work_alloc(p, &p->z, int64_t(cap) * p->E)) || (rc = work_alloc(p, &p->sel, pairs)) ||
      (rc = work_alloc(p, &p->w, pairs)) || (rc = work_alloc(p, &p->gap, cap)) ||
      (rc = work_alloc(p, &p->pair_flag, pairs)) || (rc = work_alloc(p, &p->pair_slot, pairs)) ||
      (rc = work_alloc(p, &p->pair_row, pairs)) || (rc = work_alloc(p, &p->row_tok, rows)) ||
      (rc = work_alloc(p, &p->row_w, rows)) || (rc = work_alloc(p, &p->hbuf, rows * p->I)) ||
      (rc = work_alloc(p, &p->pbuf, rows * p->H)) || (rc = work_alloc(p, &p->row_slot, rows)) ||
      (rc = work_alloc(p, &p->xq_codes, int64_t(cap) * p->H)) ||
      (rc = work_alloc(p, &p->xq_scales, int64_t(cap) * p->H / 32)) ||
      (rc = work_alloc(p, &p->tiles, 2 * int64_t(p->max_tiles))) ||
      (rc = work_alloc(p, &p->stage_agg, stage_agg_ints(pairs, p->E)))) {
    free_work_buffers(p);
    return rc;
  }
  p->rb_cap = int64_t(sizeof(ResolveHeader)) + 5 * 4 * int64_t(p->E) + 8 * pairs + 64;
  if (hipHostMalloc(reinterpret_cast<void**>(&p->rb_host), p->rb_cap, hipHostMallocMapped | hipHostMallocCoherent) !=
      hipSuccess) {
    (void)hipGetLastError();
    p->rb_host = nullptr;
    free_work_buffers(p);
    set_error("pinned readback allocation failed");
    return FT_E_OOM_PINNED;
  }
  if (hipHostGetDevicePointer(reinterpret_cast<void**>(&p->rb_dev), p->rb_host, 0) != hipSuccess) {
    (void)hipGetLastError();
    free_work_buffers(p);
    set_error("pinned readback buffer is not mapped for the device");
    return FT_E_HIP;
  }
  if (hipHostMalloc(reinterpret_cast<void**>(&p->x_host), size_t(cap) * p->H * 2, hipHostMallocDefault) !=
          hipSuccess ||
      hipHostMalloc(reinterpret_cast<void**>(&p->cpu_out), size_t(pairs) * p->H * 2, hipHostMallocDefault) !=
          hipSuccess) {
    (void)hipGetLastError();
    free_work_buffers(p);
    set_error("pinned staging allocation failed");
    return FT_E_OOM_PINNED;
  }
  p->cap_T = cap;
  return FT_OK;
}

int fail_copies(ft_moe_pool* p, int layer, const int32_t* se, const int32_t* ss, int from, int n,
                hipStream_t s) {
  const std::string msg = get_error();
  std::vector<int32_t> buf;
  for (int i = from; i < n; ++i) buf.push_back(layer * p->E + se[i]);
  for (int i = from; i < n; ++i) buf.push_back(ss[i]);
  const int m = n - from;
  if (m > 0) {
    FT_HIP_CHECK(hipMemcpy(p->fail_dev, buf.data(), buf.size() * 4, hipMemcpyHostToDevice));
    FT_HIP_CHECK(launch_uncommit(p->tab, p->fail_dev, p->fail_dev + m, m, int(p->C), s));
    FT_HIP_CHECK(hipStreamSynchronize(s));
  }
  set_error("%s", msg.c_str());
  return FT_E_HIP;
}

int issue_copy(ft_moe_pool* p, void* dst, const void* src, size_t bytes, hipStream_t cs) {
  ++p->copy_counter;
  if (p->fault_copy >= 0 && int64_t(p->copy_counter) == p->fault_copy) {
    set_error("injected failure of miss copy %llu", (unsigned long long)p->copy_counter);
    return FT_E_HIP;
  }
  if (p->poison) FT_HIP_CHECK(hipMemsetAsync(dst, 0xFF, bytes, cs));
  FT_HIP_CHECK(hipMemcpyAsync(dst, src, bytes, hipMemcpyHostToDevice, cs));
  if (int64_t(p->copy_counter) == p->corrupt_copy)  // damaged copy (tests): 256 bytes of 0xA5
    FT_HIP_CHECK(hipMemsetAsync(dst, 0xA5, std::min<size_t>(bytes, 256), cs));
  return FT_OK;
}

// Debug checksums: groups g0 .. min(g1, *n_dev) - 1 of the run list must
// hold their key's weights (FT_MOE_DEBUG_CHECKSUM).
int verify_groups(ft_moe_pool* p, int layer, int g0, int g1, const int32_t* n_dev, hipStream_t s) {
  if (!p->checksum) return FT_OK;
  FT_HIP_CHECK(launch_verify_slots(p->gdesc, g0, g1, n_dev, p->key_sum_dev, layer * p->E,
                                   p->lay[p->fmt[layer]].bytes, p->bad_dev, s));
  return FT_OK;
}

FfnArgs ffn_args(ft_moe_pool* p, int layer, int list_off, int n, const int32_t* n_dev) {
  FfnArgs a{};
  a.gdesc = p->gdesc + list_off;
  a.n_list = n;
  a.n_list_dev = n_dev != nullptr ? n_dev : p->count_max;
  a.row_tok = p->row_tok;
  a.row_w = p->row_w;
  a.hidden = p->H;
  a.inter = p->I;
  a.lay = p->lay[p->fmt[layer]];
  a.act_mode = 0;
  return a;
}

double mat_bytes(int fmt, double rows, double cols);
hipEvent_t prof_begin(ft_moe_pool* p, hipStream_t s, int stage);
void prof_end(ft_moe_pool* p, int stage, hipEvent_t a, hipStream_t s, double bytes, double flops);
Ev prof_pair(ft_moe_pool* p, hipStream_t s, int stage);
void prof_push(ft_moe_pool* p, int stage, Ev ev, double bytes, double flops);

// groups / rows: how many expert groups and rows this launch runs (for the
// algorithmic byte and flop counts of the stage timers; 0 when the device
// counts them).
int run_ffn(ft_moe_pool* p, int layer, const void* x, int list_off, int n, const int32_t* n_dev, hipStream_t s,
            double groups, double rows, int max_group_rows = 1 << 30) {
  // nothing to run (a count known on the host): no launch, and no timing record
  // (its recycled events would still hold an earlier launch's timestamps)
  if (n_dev == nullptr && n <= 0) return FT_OK;
  FfnArgs a = ffn_args(p, layer, list_off, n, n_dev);
  a.max_rows = max_group_rows <= 64 ? max_group_rows : 0;
  const int f = p->fmt[layer];
  const double H = p->H, I = p->I;
  a.x = static_cast<const uint16_t*>(x);
  a.out = p->hbuf;
  Ev ev = prof_pair(p, s, FT_STAGE_FFN_GATEUP);
  FT_HIP_CHECK(launch_ffn_gateup(a, s, ev));
  prof_push(p, FT_STAGE_FFN_GATEUP, ev, groups * 2 * mat_bytes(f, I, H) + rows * (H + I) * 2, rows * 4 * H * I);
  a.x = p->hbuf;
  a.out = p->pbuf;
  ev = prof_pair(p, s, FT_STAGE_FFN_DOWN);
  FT_HIP_CHECK(launch_ffn_down(a, s, ev));
  prof_push(p, FT_STAGE_FFN_DOWN, ev, groups * mat_bytes(f, H, I) + rows * (I + H) * 2, rows * 2 * H * I);
  return FT_OK;
}

ResolveArgs resolve_args(ft_moe_pool* p, int layer, int T, int t0, int mode) {
  ResolveArgs a{};
  a.z = p->z;
  a.do_topk = (mode == 0 && t0 == 0) ? 1 : 0;
  a.sel = p->sel;
  a.w = p->w;
  a.gap = p->gap;
  a.t0 = t0;
  a.T = T;
  a.k = p->k;
  a.E = p->E;
  a.layer = layer;
  a.C = int(p->C);
  a.mode = mode;
  a.stamp = p->stamp++;
  a.share = p->share_fmt[p->fmt[layer]];
  a.expert_bytes = p->canon_bytes[p->fmt[layer]];
  a.hidden = p->H;
  a.arena = reinterpret_cast<uint64_t>(p->arena);
  a.slot_bytes = p->slot_bytes;
  a.shared_ptr = p->shared ? reinterpret_cast<uint64_t>(p->shared_dev + int64_t(layer) * p->shared_stride) : 0;
  a.tab = p->tab;
  a.pair_flag = p->pair_flag;
  a.pair_slot = p->pair_slot;
  a.pair_row = p->pair_row;
  a.row_tok = p->row_tok;
  a.row_w = p->row_w;
  a.groups = p->groups;
  a.glist = p->glist;
  a.gdesc = p->gdesc;
  a.dev_header = p->dev_header;
  a.host_rb = mode == 0 ? p->rb_dev : nullptr;
  a.host_rb_cap = p->rb_cap;
  a.host_wait = mode == 0 ? 1 : 0;
  a.tiles = mode == 1 ? p->tiles : nullptr;
  a.row_slot = mode == 1 ? p->row_slot : nullptr;
  a.tile_rows = mx_gemm_rows_per_tile();
  if (mode == 1) {
    a.agg = p->stage_agg;
    a.nchunks = int32_t((int64_t(T) * p->k + kStageChunk - 1) / kStageChunk);
  }
  return a;
}

// ---- stage timing
hipEvent_t prof_event(ft_moe_pool* p) {
  if (!p->prof_free.empty()) {
    hipEvent_t e = p->prof_free.back();
    p->prof_free.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) return nullptr;
  return e;
}

hipEvent_t prof_begin(ft_moe_pool* p, hipStream_t s, int stage) {
  if (!(p->prof_mask & (1 << stage))) return nullptr;
  hipEvent_t e = prof_event(p);
  if (e) (void)hipEventRecord(e, s);
  return e;
}

void prof_end(ft_moe_pool* p, int stage, hipEvent_t a, hipStream_t s, double bytes, double flops = 0.0) {
  if (!a) return;
  hipEvent_t b = prof_event(p);
  if (!b) return;
  (void)hipEventRecord(b, s);
  p->prof_pending.push_back({stage, a, b, bytes, flops});
}

// Event pair for a kernel launched through ft_launch (bracketing the kernel itself).
Ev prof_pair(ft_moe_pool* p, hipStream_t s, int stage) {
  (void)s;
  Ev ev;
  if (!(p->prof_mask & (1 << stage))) return ev;
  ev.a = prof_event(p);
  ev.b = prof_event(p);
  if (!ev.a || !ev.b) ev = Ev{};
  return ev;
}

void prof_push(ft_moe_pool* p, int stage, Ev ev, double bytes, double flops) {
  if (ev.a) p->prof_pending.push_back({stage, ev.a, ev.b, bytes, flops});
}

// Copy-time events of host-issued copies (always on; ft_moe_stats::copy_ms).
hipEvent_t copy_timer_begin(ft_moe_pool* p, hipStream_t s) {
  hipEvent_t e = prof_event(p);
  if (e && hipEventRecord(e, s) != hipSuccess) {
    (void)hipGetLastError();
    p->prof_free.push_back(e);
    return nullptr;
  }
  return e;
}

void copy_timer_end(ft_moe_pool* p, int layer, hipEvent_t a, hipStream_t s, double obs_bytes = 0.0) {
  if (!a) return;
  hipEvent_t b = prof_event(p);
  if (!b || hipEventRecord(b, s) != hipSuccess) {
    (void)hipGetLastError();
    p->prof_free.push_back(a);
    if (b) p->prof_free.push_back(b);
    return;
  }
  p->copy_pending.push_back({layer, a, b, obs_bytes});
}

void copy_drain(ft_moe_pool* p, bool wait) {
  std::vector<ft_moe_pool::CopyRec> keep;
  for (auto& r : p->copy_pending) {
    if (wait)
      (void)hipEventSynchronize(r.b);
    else if (hipEventQuery(r.b) != hipSuccess) {
      keep.push_back(r);
      continue;
    }
    float ms = 0.f;
    if (hipEventElapsedTime(&ms, r.a, r.b) == hipSuccess) {
      p->copy_ms_host[r.layer] += ms;
      if (r.bytes > 0.0) {
        ft_moe_pool::Obs& o = p->obs[p->fmt[r.layer]];
        o.copy_ms += ms;
        o.copy_bytes += r.bytes;
      }
    }
    p->prof_free.push_back(r.a);
    p->prof_free.push_back(r.b);
  }
  (void)hipGetLastError();
  p->copy_pending.swap(keep);
}

// Fold finished records into the sums (all of them if wait).
void prof_drain(ft_moe_pool* p, bool wait) {
  std::vector<ft_moe_pool::ProfRec> keep;
  for (auto& r : p->prof_pending) {
    if (wait)
      (void)hipEventSynchronize(r.b);
    else if (hipEventQuery(r.b) != hipSuccess) {
      keep.push_back(r);
      continue;
    }
    float ms = 0.f;
    if (hipEventElapsedTime(&ms, r.a, r.b) == hipSuccess) {
      p->prof.ms[r.stage] += ms;
      p->prof.bytes[r.stage] += r.bytes;
      p->prof.flops[r.stage] += r.flops;
      p->prof.launches[r.stage] += 1;
    }
    p->prof_free.push_back(r.a);
    p->prof_free.push_back(r.b);
  }
  (void)hipGetLastError();
  p->prof_pending.swap(keep);
}

// Algorithmic bytes of the weights of one matrix (codes + block scales).
double mat_bytes(int fmt, double rows, double cols) {
  const double n = rows * cols;
  switch (fmt) {
    case FT_FMT_MXFP4: return n / 2 + n / 32;
    case FT_FMT_NVFP4: return n / 2 + n / 16;
    default: return n + n / 128 * 4;
  }
}

int copy_layer_staging(ft_moe_pool* p, int layer) {
  const int E = p->E;
  const int half = layer & 1;
  uint8_t* dst = p->arena + int64_t(half) * E * p->slot_bytes;
  const ExpertLayout& L = p->lay[p->fmt[layer]];
  hipEvent_t e0 = prof_begin(p, p->copy_stream, FT_STAGE_COPY);
  hipEvent_t ct = copy_timer_begin(p, p->copy_stream);
  int copied = 0;
  if (p->poison) {
    // every slot of the half that this call copies into
    for (int e = 0; e < E; ++e)
      if (!(p->prefill_hit && p->prefill_res[int64_t(layer) * E + e] >= 0))
        FT_HIP_CHECK(hipMemsetAsync(dst + int64_t(e) * p->slot_bytes, 0xFF, size_t(L.bytes), p->copy_stream));
  }
  if (p->prefill_hit) {
    // runs of consecutive experts that are not resident in the pool
    const int32_t* res = p->prefill_res.data() + int64_t(layer) * E;
    for (int e = 0; e < E;) {
      if (res[e] >= 0) {
        ++e;
        continue;
      }
      int e1 = e + 1;
      while (e1 < E && res[e1] < 0) ++e1;
      if (p->layer_contig[layer]) {
        FT_HIP_CHECK(hipMemcpyAsync(dst + int64_t(e) * p->slot_bytes, p->host_store + p->key_off[int64_t(layer) * E + e],
                                    size_t(e1 - e - 1) * p->slot_bytes + size_t(L.bytes), hipMemcpyHostToDevice,
                                    p->copy_stream));
      } else {
        for (int j = e; j < e1; ++j)
          FT_HIP_CHECK(hipMemcpyAsync(dst + int64_t(j) * p->slot_bytes,
                                      p->host_store + p->key_off[int64_t(layer) * E + j], size_t(L.bytes),
                                      hipMemcpyHostToDevice, p->copy_stream));
      }
      copied += e1 - e;
      e = e1;
    }
  } else if (p->layer_contig[layer]) {
    FT_HIP_CHECK(hipMemcpyAsync(dst, p->host_store + p->key_off[int64_t(layer) * E], size_t(E) * p->slot_bytes,
                                hipMemcpyHostToDevice, p->copy_stream));
    copied = E;
  } else {
    for (int e = 0; e < E; ++e)
      FT_HIP_CHECK(hipMemcpyAsync(dst + int64_t(e) * p->slot_bytes, p->host_store + p->key_off[int64_t(layer) * E + e],
                                  size_t(L.bytes), hipMemcpyHostToDevice, p->copy_stream));
    copied = E;
  }
  prof_end(p, FT_STAGE_COPY, e0, p->copy_stream, double(copied) * double(p->canon_bytes[p->fmt[layer]]), 0.0);
  copy_timer_end(p, layer, ct, p->copy_stream);
  FT_HIP_CHECK(hipEventRecord(p->ev_staged[half], p->copy_stream));
  return FT_OK;
}

// The gate/up GEMM's activation tiles: x of a prefill chunk (T rows, K = H)
// is quantised row-major (one row per token) and copied into the tiles of
// every expert row that reads it.  Timed as one stage.  (h is quantised by
// the gate/up GEMM into the down GEMM's tiles.)
int mx_act_tiles(ft_moe_pool* p, const uint16_t* src, int nrows, int K, bool fp4, hipStream_t s) {
  hipEvent_t e0 = prof_begin(p, s, FT_STAGE_ACT_QUANT);
  MxQuantArgs q{};
  q.in = src;
  q.rows = nrows;
  q.K = K;
  q.out_codes = p->xq_codes;
  q.out_scales = p->xq_scales;
  FT_HIP_CHECK(launch_mx_quant(q, fp4, s));
  const double per = fp4 ? 0.5 + 1.0 / 32 : 1.0 + 1.0 / 32;
  double bytes = double(nrows) * K * (2.0 + per);
  MxTileArgs t{};
  t.codes = p->xq_codes;
  t.scales = p->xq_scales;
  t.K = K;
  t.row_map = p->row_tok;
  t.groups = p->groups;
  t.tiles = p->tiles;
  t.n_tiles_dev = p->dev_header + 10;
  t.max_tiles = p->max_tiles;
  t.out_codes = p->tq_codes;
  t.out_scales = p->tq_scales;
  FT_HIP_CHECK(launch_mx_tile_gather(t, fp4, s));
  bytes += 2.0 * double(nrows) * p->k * K * per;
  prof_end(p, FT_STAGE_ACT_QUANT, e0, s, bytes, 0.0);
  return FT_OK;
}

// The prefill expert FFN of an MXFP4 layer on the grouped GEMM: act is
// FT_ACT_* >> 4.  MX modes quantise x into the GEMM's activation tiles, and
// the gate/up GEMM writes h quantised into the down GEMM's tiles; bf16 reads
// the activations from their rows (x by token, h by row).
int run_mx_ffn(ft_moe_pool* p, int layer, const void* x, int T, int act, hipStream_t s) {
  const int rows = T * p->k + (p->shared ? T : 0);
  const double H = p->H, I = p->I;
  const bool mx = act != 0, fp4 = act == (FT_ACT_MXFP4 >> 4);
  // activation bytes per element as the GEMM reads them
  const double per = !mx ? 2.0 : fp4 ? 0.5 + 1.0 / 32 : 1.0 + 1.0 / 32;
  if (mx && !(p->tq_codes && p->tq_scales && p->hq_codes && p->hq_scales)) {
    // sized for FP8 codes (x: K = H, h: K = I); freed with the per-call
    // buffers.  All four exist or none does: a failed allocation frees the
    // others, so a later call never runs with part of them.
    const int64_t xb = int64_t(p->max_tiles) * (p->H / kTileK), hb = int64_t(p->max_tiles) * (p->I / kTileK);
    auto mx_alloc = [p](uint8_t** q, int64_t n) -> int {
      if (++p->mx_allocs == p->fault_mx_alloc) {
        p->fault_mx_alloc = -1;
        *q = nullptr;
        set_error("injected failure of MX tile allocation %d", p->mx_allocs);
        return FT_E_OOM_DEVICE;
      }
      return dev_alloc(q, n);
    };
    dev_free(p->tq_codes); dev_free(p->tq_scales); dev_free(p->hq_codes); dev_free(p->hq_scales);
    int rc;
    if ((rc = mx_alloc(&p->tq_codes, xb * mx_tile_code_bytes(false))) ||
        (rc = mx_alloc(&p->tq_scales, xb * kMxTileScaleBytes)) ||
        (rc = mx_alloc(&p->hq_codes, hb * mx_tile_code_bytes(false))) ||
        (rc = mx_alloc(&p->hq_scales, hb * kMxTileScaleBytes))) {
      dev_free(p->tq_codes); dev_free(p->tq_scales); dev_free(p->hq_codes); dev_free(p->hq_scales);
      p->hq_blocks = 0;
      return rc;
    }
    p->hq_blocks = hb;
  }
  int rc;
  if (mx && (rc = mx_act_tiles(p, static_cast<const uint16_t*>(x), T, p->H, fp4, s))) return rc;
  MxGemmArgs a{};
  a.groups = p->groups;
  a.tiles = p->tiles;
  a.n_tiles_dev = p->dev_header + 10;
  a.max_tiles = p->max_tiles;
  a.act_codes = p->tq_codes;
  a.act_scales = p->tq_scales;
  a.act_rows = static_cast<const uint16_t*>(x);
  a.row_tok = p->row_tok;
  a.row_w = p->row_w;
  a.out = p->hbuf;
  a.hidden = p->H;
  a.inter = p->I;
  a.lay = p->lay[p->fmt[layer]];
  if (mx) {
    // h leaves the gate/up GEMM quantised, in the down GEMM's activation tiles
    a.h_codes = p->hq_codes;
    a.h_scales = p->hq_scales;
    a.row_slot = p->row_slot;
  }
  Ev ev = prof_pair(p, s, FT_STAGE_FFN_GATEUP);
  FT_HIP_CHECK(launch_mx_gemm(a, true, act, s, ev));
  prof_push(p, FT_STAGE_FFN_GATEUP, ev, (p->E + p->shared) * 2 * mat_bytes(FT_FMT_MXFP4, I, H) + rows * I * per +
            T * H * per, rows * 4 * H * I);
  a.act_codes = p->hq_codes;
  a.act_scales = p->hq_scales;
  a.h_codes = a.h_scales = nullptr;
  a.act_rows = p->hbuf;
  a.row_tok = nullptr;
  a.out = p->pbuf;
  ev = prof_pair(p, s, FT_STAGE_FFN_DOWN);
  FT_HIP_CHECK(launch_mx_gemm(a, false, act, s, ev));
  prof_push(p, FT_STAGE_FFN_DOWN, ev, (p->E + p->shared) * mat_bytes(FT_FMT_MXFP4, H, I) + rows * H * 2.0 +
            rows * I * per, rows * 2 * H * I);
  return FT_OK;
}

int forward_prefill(ft_moe_pool* p, int layer, int T, const void* x, void* out, hipStream_t s, int act,
                    bool hit_d2d) {
  const int L = p->L, E = p->E;
  if (act != 0 && p->fmt[layer] != FT_FMT_MXFP4) {
    set_error("MX activation modes need MXFP4 expert weights (layer %d)", layer);
    return FT_E_INVALID;
  }
  if (p->C < 2 * int64_t(E)) {
    set_error("prefill staging needs 2*E = %d slots, pool has %lld", 2 * E, (long long)p->C);
    return FT_E_INVALID;
  }
  if (!(layer == 0 || layer == p->prefill_next)) {
    set_error("prefill layer %d out of order (expected 0 or %d)", layer, p->prefill_next);
    return FT_E_STATE;
  }
  if (layer > 0 && hit_d2d != p->prefill_hit) {
    set_error("prefill layer %d: the hit-D2D option must match the chunk's layer 0", layer);
    return FT_E_STATE;
  }
  if (layer == 0) {
    p->prefill_hit = hit_d2d;
    if (hit_d2d) {
      // residency outside the staging region, fixed for the whole chunk
      // (layer 0 clears the staging region; decode calls wait for the chunk)
      const int64_t LE = int64_t(L) * E;
      p->prefill_res.resize(size_t(LE));
      FT_HIP_CHECK(hipStreamSynchronize(s));
      FT_HIP_CHECK(hipMemcpy(p->prefill_res.data(), p->tab.key2slot, size_t(LE) * 4, hipMemcpyDeviceToHost));
      for (auto& v : p->prefill_res)
        if (v < 2 * E) v = -1;
    }
  }
  // the layer's experts are streamed into its staging half (resident ones
  // are skipped with the hit-D2D option)
  p->last_pending = false;
  p->last_se.clear();
  p->last_ss.clear();
  p->last_ce.clear();
  for (int e = 0; e < E; ++e) {
    if (p->prefill_hit && p->prefill_res[int64_t(layer) * E + e] >= 0) continue;
    p->last_se.push_back(e);
    p->last_ss.push_back((layer & 1) * E + e);
  }
  // table: the staging halves lose their LRU residents
  FT_HIP_CHECK(launch_stage_table(p->tab, E, int(p->C), layer, L, T * p->k, 0, s));
  if (layer == 0) {
    // first copy of the chunk: after every earlier reader of half 0 on s
    FT_HIP_CHECK(hipEventRecord(p->ev_sync, s));
    FT_HIP_CHECK(hipStreamWaitEvent(p->copy_stream, p->ev_sync, 0));
    int rc = copy_layer_staging(p, 0);
    if (rc) return rc;
  }
  if (layer + 1 < L) {
    // half (layer+1)%2 was last read by layer-1 (or by earlier decode work)
    if (layer >= 1) {
      FT_HIP_CHECK(hipStreamWaitEvent(p->copy_stream, p->ev_done[(layer - 1) & 1], 0));
    }
    int rc = copy_layer_staging(p, layer + 1);
    if (rc) return rc;
  }
  FT_HIP_CHECK(hipStreamWaitEvent(s, p->ev_staged[layer & 1], 0));
  ResolveArgs ra = resolve_args(p, layer, T, 0, 1);
  ra.stage_hits = p->prefill_hit ? 1 : 0;
  Ev er = prof_pair(p, s, FT_STAGE_RESOLVE);
  FT_HIP_CHECK(launch_resolve(ra, s, er));
  prof_push(p, FT_STAGE_RESOLVE, er, 0.0, 0.0);
  if (int rc = verify_groups(p, layer, 0, E + 1, p->dev_header + 9, s)) return rc;
  const double rows = double(T) * p->k + (p->shared ? T : 0);
  // MXFP4 layers run the grouped GEMM (bf16 or MX activations); others the FFN kernels
  int rc = p->fmt[layer] == FT_FMT_MXFP4 ? run_mx_ffn(p, layer, x, T, act, s)
                                         : run_ffn(p, layer, x, 0, E + 1, p->dev_header + 9, s, E + p->shared, rows);
  if (rc) return rc;
  Ev ev = prof_pair(p, s, FT_STAGE_COMBINE);
  FT_HIP_CHECK(launch_combine(p->pbuf, p->pair_row, 0, T, p->k, p->H, p->shared ? T * p->k : -1,
                              static_cast<uint16_t*>(out), s, ev));
  prof_push(p, FT_STAGE_COMBINE, ev, (rows + T) * p->H * 2.0, 0.0);
  FT_HIP_CHECK(hipEventRecord(p->ev_done[layer & 1], s));
  p->prefill_next = layer + 1 == L ? 0 : layer + 1;
  return FT_OK;
}

// Decode with device-driven misses (one wave: T*k <= C), enqueued on s with
// no host wait: resolve -> miss copy -> FFN of every group -> combine.  The
// copy overwrites victim slots only, and every earlier reader of those slots
// precedes the resolve kernel on s.  Everything stays on one stream: waits
// across queues cost more than the FFN of the hits that could overlap the
// copy, and an FFN sharing CUs with the copy's PCIe loads is starved.
int forward_decode_dev(ft_moe_pool* p, int layer, int T, const void* x, void* out, hipStream_t s) {
  const int E = p->E, k = p->k;
  const int f = p->fmt[layer];
  if (p->prof_mask) prof_drain(p, false);
  ResolveArgs ra = resolve_args(p, layer, T, 0, 0);
  ra.host_wait = 0;  // nobody spins: the readback is read after a stream sync
  const int bits = ((p->prof_mask >> FT_STAGE_FFN_GATEUP) & 1) | (((p->prof_mask >> FT_STAGE_FFN_DOWN) & 1) << 1) |
                   (((p->prof_mask >> FT_STAGE_COPY) & 1) << 2);
  if (bits) {
    ra.prof_cnt = p->prof_cnt_dev;
    ra.prof_stages = bits;
    ra.fmt = f;
  }
  Ev er = prof_pair(p, s, FT_STAGE_RESOLVE);
  FT_HIP_CHECK(launch_resolve(ra, s, er));
  prof_push(p, FT_STAGE_RESOLVE, er, 0.0, 0.0);

  MissCopyArgs ca{};
  ca.host = p->host_store_dev;
  ca.key_off = p->key_off_dev;
  ca.dev_header = p->dev_header;
  ca.gdesc = p->gdesc;
  ca.layer = layer;
  ca.E = E;
  ca.bytes = p->lay[f].bytes;
  ca.clk = p->copy_clk;
  ca.ticks = p->copy_ticks + layer;
  if (p->poison) FT_HIP_CHECK(launch_poison_slots(ca, p->copy_wgs, s));
  Ev ec = prof_pair(p, s, FT_STAGE_COPY);
  FT_HIP_CHECK(launch_miss_copy(ca, p->copy_wgs, s, ec));
  prof_push(p, FT_STAGE_COPY, ec, 0.0, 0.0);

  // all groups (hit list, then streamed misses; no host-computed ones here)
  const int pairs = T * k;
  const int bound = std::min(pairs, E) + p->shared;
  if (int rc = verify_groups(p, layer, 0, bound, p->dev_header + 9, s)) return rc;
  // a group has at most one row per token
  int rc = run_ffn(p, layer, x, 0, bound, p->dev_header + 9, s, 0.0, 0.0, T);
  if (rc) return rc;
  const int rows = pairs + (p->shared ? T : 0);
  Ev eb = prof_pair(p, s, FT_STAGE_COMBINE);
  FT_HIP_CHECK(launch_combine(p->pbuf, p->pair_row, 0, T, k, p->H, p->shared ? pairs : -1,
                              static_cast<uint16_t*>(out), s, eb));
  prof_push(p, FT_STAGE_COMBINE, eb, (double(rows) + T) * p->H * 2.0, 0.0);
  p->last_pending = true;
  return FT_OK;
}

// Miss lists of the latest device-driven call, from the resolve kernel's
// mapped readback (waits for the stream of that call).
int read_pending_misses(const ft_moe_pool* p) {
  if (!p->last_pending) return FT_OK;
  FT_HIP_CHECK(hipStreamSynchronize(p->last_stream));
  const ResolveHeader h = *reinterpret_cast<const ResolveHeader*>(p->rb_host);
  const int32_t* se = reinterpret_cast<const int32_t*>(p->rb_host + sizeof(ResolveHeader));
  const int32_t* ss = se + p->E;
  p->last_se.assign(se, se + h.n_stream);
  p->last_ss.assign(ss, ss + h.n_stream);
  p->last_ce.clear();
  p->last_pending = false;
  return FT_OK;
}

int forward_decode(ft_moe_pool* p, int layer, int T, const void* x, void* out, hipStream_t s) {
  const int E = p->E, k = p->k;
  if (!p->copy_pending.empty()) copy_drain(p, false);
  const ExpertLayout& L = p->lay[p->fmt[layer]];
  p->last_se.clear();
  p->last_ss.clear();
  p->last_ce.clear();
  p->last_pending = false;
  int t0 = 0;
  while (t0 < T) {
    ResolveArgs ra = resolve_args(p, layer, T, t0, 0);
    volatile uint32_t* seq = &reinterpret_cast<ResolveHeader*>(p->rb_host)->seq;
    *seq = uint32_t(ra.stamp) ^ 0x80000000u;
    Ev er = prof_pair(p, s, FT_STAGE_RESOLVE);
    FT_HIP_CHECK(launch_resolve(ra, s, er));
    prof_push(p, FT_STAGE_RESOLVE, er, 0.0, 0.0);
    FT_HIP_CHECK(hipEventRecord(p->ev_resolved, s));
    // The kernel publishes the wave's stamp in mapped memory after its other
    // writes; spinning on it returns sooner than an event wait.  A stream
    // error (or a very long wait) falls back to the event, which reports it.
    {
      const auto t_start = std::chrono::steady_clock::now();
      uint32_t n = 0;
      while (*seq != uint32_t(ra.stamp)) {
        __builtin_ia32_pause();
        if ((++n & 0xFFF) == 0) {
          const hipError_t q = hipEventQuery(p->ev_resolved);
          if (q != hipErrorNotReady && *seq != uint32_t(ra.stamp)) {
            FT_HIP_CHECK(hipEventSynchronize(p->ev_resolved));
            if (*seq != uint32_t(ra.stamp)) {
              set_error("resolve finished without publishing its results");
              return FT_E_HIP;
            }
          }
          if (std::chrono::steady_clock::now() - t_start > std::chrono::seconds(30)) {
            FT_HIP_CHECK(hipEventSynchronize(p->ev_resolved));
          }
        }
      }
      std::atomic_thread_fence(std::memory_order_acquire);
    }
    if (p->prof_mask) prof_drain(p, false);
    const ResolveHeader h = *reinterpret_cast<const ResolveHeader*>(p->rb_host);
    const int32_t* se = reinterpret_cast<const int32_t*>(p->rb_host + sizeof(ResolveHeader));
    const int32_t* ss = se + E;
    const int32_t* ce = ss + E;
    const int32_t* cb = ce + E;
    const int32_t* cc = cb + E;
    const int32_t* ct = cc + E;
    const float* cw = reinterpret_cast<const float*>(ct + int64_t(T) * k);
    if (h.t1 <= t0 || h.t1 > T) {
      set_error("resolve returned an invalid wave end %d (t0 %d, T %d)", h.t1, t0, T);
      return FT_E_HIP;
    }
    for (int i = 0; i < h.n_stream; ++i) {
      p->last_se.push_back(se[i]);
      p->last_ss.push_back(ss[i]);
    }
    for (int i = 0; i < h.n_cpu; ++i) p->last_ce.push_back(ce[i]);

    // the activation rows the host-computed experts need, then the host work,
    // both before the streamed copies are queued: behind the copies the small
    // device-to-host copy would wait for the whole transfer, and issuing the
    // copies (tens of microseconds of API time each) would delay the host work
    std::thread cpu_thread;
    struct JoinGuard {
      std::thread& t;
      ~JoinGuard() {
        if (t.joinable()) t.join();
      }
    } join_guard{cpu_thread};  // every return below waits for the host work
    std::vector<int64_t> cpu_base;
    double host_sec = 0.0;
    if (h.n_cpu > 0) {
      if (p->cpu_copy_pending) FT_HIP_CHECK(hipEventSynchronize(p->ev_cpu_copied));
      FT_HIP_CHECK(hipMemcpyAsync(p->x_host, x, size_t(T) * p->H * 2, hipMemcpyDeviceToHost, s));
      FT_HIP_CHECK(hipStreamSynchronize(s));
      int64_t base = 0;
      for (int j = 0; j < h.n_cpu; ++j) {
        cpu_base.push_back(base);
        base += cc[j];
      }
      if (!p->workers) p->workers = std::make_unique<WorkerPool>(p->cpu_threads);
      std::vector<int32_t> toks(ct, ct + h.cpu_rows);
      std::vector<float> wts(cw, cw + h.cpu_rows);
      std::vector<int32_t> experts(ce, ce + h.n_cpu), counts(cc, cc + h.n_cpu);
      cpu_thread = std::thread([p, layer, toks, wts, experts, counts, cpu_base, &L, &host_sec]() {
        const auto t0 = std::chrono::steady_clock::now();
        std::vector<uint16_t> xr(toks.size() * size_t(p->H));
        for (size_t r = 0; r < toks.size(); ++r)
          std::memcpy(&xr[r * p->H], p->x_host + int64_t(toks[r]) * p->H, size_t(p->H) * 2);
        std::vector<HostExpertJob> jobs(experts.size());
        for (size_t j = 0; j < experts.size(); ++j)
          jobs[j] = HostExpertJob{p->host_store + p->key_off[int64_t(layer) * p->E + experts[j]],
                                  xr.data() + cpu_base[j] * p->H, wts.data() + cpu_base[j], counts[j],
                                  p->cpu_out + cpu_base[j] * p->H};
        host_experts(L, jobs.data(), int(jobs.size()), *p->workers);
        host_sec = std::chrono::duration<double>(std::chrono::steady_clock::now() - t0).count();
      });
    }

    // streamed misses: one contiguous copy per expert, rotating over the copy
    // streams.  Everything earlier on s (the readers of the victim slots) has
    // finished: the resolve kernel that published this list ran after it.
    const int ncs = std::min(p->n_copy, std::max(h.n_stream, 1));
    hipEvent_t ec = h.n_stream > 0 ? prof_begin(p, p->copy[0], FT_STAGE_COPY) : nullptr;
    hipEvent_t et = h.n_stream > 0 ? copy_timer_begin(p, p->copy[0]) : nullptr;
    if (et)
      for (int c = 1; c < ncs; ++c) FT_HIP_CHECK(hipStreamWaitEvent(p->copy[c], et, 0));
    for (int i = 0; i < h.n_stream; ++i) {
      const int64_t key = int64_t(layer) * E + se[i];
      int rc = issue_copy(p, p->arena + int64_t(ss[i]) * p->slot_bytes, p->host_store + p->key_off[key],
                          size_t(L.bytes), p->copy[i % ncs]);
      if (rc) {
        for (int c = 0; c < ncs; ++c) (void)hipStreamSynchronize(p->copy[c]);
        return fail_copies(p, layer, se, ss, i, h.n_stream, s);
      }
    }
    if (h.n_stream > 0) {
      for (int c = 1; c < ncs; ++c) {
        FT_HIP_CHECK(hipEventRecord(p->ev_copy_done[c], p->copy[c]));
        FT_HIP_CHECK(hipStreamWaitEvent(p->copy[0], p->ev_copy_done[c], 0));
      }
      prof_end(p, FT_STAGE_COPY, ec, p->copy[0], double(h.n_stream) * double(p->canon_bytes[p->fmt[layer]]), 0.0);
      copy_timer_end(p, layer, et, p->copy[0], double(h.n_stream) * double(p->canon_bytes[p->fmt[layer]]));
      FT_HIP_CHECK(hipEventRecord(p->ev_copied, p->copy[0]));
    }

    int rc = verify_groups(p, layer, 0, h.n_hit_list, nullptr, s);
    if (rc == FT_OK) rc = run_ffn(p, layer, x, 0, h.n_hit_list, nullptr, s, h.n_hit_list, h.rows_hit_list, T);
    if (rc == FT_OK && h.n_stream > 0) {
      FT_HIP_CHECK(hipStreamWaitEvent(s, p->ev_copied, 0));
      rc = verify_groups(p, layer, h.n_hit_list, h.n_hit_list + h.n_stream, nullptr, s);
      if (rc == FT_OK)
        rc = run_ffn(p, layer, x, h.n_hit_list, h.n_stream, nullptr, s, h.n_stream, h.rows_stream, T);
    }
    if (cpu_thread.joinable()) {
      cpu_thread.join();
      p->obs[p->fmt[layer]].host_sec += host_sec;
      p->obs[p->fmt[layer]].host_bytes += double(h.n_cpu) * double(p->canon_bytes[p->fmt[layer]]);
      if (p->prof_mask & (1 << FT_STAGE_HOST_FFN)) {
        p->prof.ms[FT_STAGE_HOST_FFN] += host_sec * 1e3;
        p->prof.bytes[FT_STAGE_HOST_FFN] += double(h.n_cpu) * double(p->canon_bytes[p->fmt[layer]]);
        p->prof.flops[FT_STAGE_HOST_FFN] += double(h.cpu_rows) * 6.0 * p->H * p->I;
        p->prof.launches[FT_STAGE_HOST_FFN] += 1;
      }
    }
    if (rc) return rc;
    if (h.n_cpu > 0) {
      // one copy per run of host experts whose rows are adjacent in pbuf
      for (int j = 0; j < h.n_cpu;) {
        int j1 = j + 1;
        int64_t rows = cc[j];
        while (j1 < h.n_cpu && int64_t(cb[j1]) == int64_t(cb[j]) + rows) rows += cc[j1++];
        FT_HIP_CHECK(hipMemcpyAsync(p->pbuf + int64_t(cb[j]) * p->H, p->cpu_out + cpu_base[j] * p->H,
                                    size_t(rows) * p->H * 2, hipMemcpyHostToDevice, s));
        j = j1;
      }
      FT_HIP_CHECK(hipEventRecord(p->ev_cpu_copied, s));
      p->cpu_copy_pending = true;
    }
    Ev eb = prof_pair(p, s, FT_STAGE_COMBINE);
    FT_HIP_CHECK(launch_combine(p->pbuf, p->pair_row, t0, h.t1, k, p->H, p->shared ? h.pairs : -1,
                                static_cast<uint16_t*>(out), s, eb));
    prof_push(p, FT_STAGE_COMBINE, eb, (double(h.rows) + (h.t1 - t0)) * p->H * 2.0, 0.0);
    t0 = h.t1;
  }
  return FT_OK;
}

}  // namespace

extern "C" {

const char* ft_moe_last_error(void) { return get_error(); }

int ft_moe_init_pool(const ft_moe_config* cfg, const ft_moe_weights* wts, ft_moe_pool** out) {
  try {
    if (!out) {
      set_error("out is NULL");
      return FT_E_INVALID;
    }
    *out = nullptr;
    if (!cfg || !wts || !wts->expert || !wts->router_w || !cfg->layer_fmt) {
      set_error("NULL config, weights or layer_fmt");
      return FT_E_INVALID;
    }
    const int L = cfg->num_layers, H = cfg->hidden, I = cfg->inter, E = cfg->num_experts, k = cfg->top_k;
    if (L < 1 || H < 128 || I < 128 || H % 128 || I % 128 || H > 8192 || I > 16384) {
      set_error("bad shape: L=%d H=%d I=%d (H, I multiples of 128, H <= 8192)", L, H, I);
      return FT_E_INVALID;
    }
    if (E < 1 || E > kMaxExperts || k < 1 || k > kMaxTopK || k > E) {
      set_error("bad experts/top_k: E=%d k=%d (E <= %d, k <= %d)", E, k, kMaxExperts, kMaxTopK);
      return FT_E_INVALID;
    }
    if (cfg->hybrid_cpu_share < 0.0 || cfg->hybrid_cpu_share > 1.0) {
      set_error("hybrid_cpu_share must be in [0,1]");
      return FT_E_INVALID;
    }
    if (cfg->has_shared_expert && !wts->shared) {
      set_error("has_shared_expert set but shared blobs are NULL");
      return FT_E_INVALID;
    }
    for (int l = 0; l < L; ++l) {
      const int f = cfg->layer_fmt[l];
      if (f < FT_FMT_MXFP4 || f > FT_FMT_FP8_B128) {
        set_error("layer %d: unknown format %d", l, f);
        return FT_E_INVALID;
      }
      if (!ffn_shape_ok(f, H, I)) {
        set_error("layer %d: H=%d I=%d not supported by the expert kernels", l, H, I);
        return FT_E_INVALID;
      }
    }
    for (int64_t i = 0; i < int64_t(L) * E; ++i)
      if (!wts->expert[i]) {
        set_error("expert blob %lld is NULL", (long long)i);
        return FT_E_INVALID;
      }
    auto p = std::make_unique<ft_moe_pool>();
    p->L = L; p->H = H; p->I = I; p->E = E; p->k = k;
    p->shared = cfg->has_shared_expert ? 1 : 0;
    p->device = cfg->device;
    p->cpu_threads = cfg->cpu_threads > 0 ? cfg->cpu_threads : 8;
    for (double& v : p->share_fmt) v = cfg->hybrid_cpu_share;
    p->fmt.assign(cfg->layer_fmt, cfg->layer_fmt + L);
    for (int f = 1; f <= 3; ++f) {
      p->lay[f] = make_layout(f, H, I);
      p->canon_bytes[f] = canonical_bytes(f, H, I);
    }
    for (int l = 0; l < L; ++l) p->slot_bytes = std::max(p->slot_bytes, p->lay[p->fmt[l]].bytes);
    p->C = cfg->pool_slots > 0 ? cfg->pool_slots : (cfg->pool_bytes > 0 ? cfg->pool_bytes / p->slot_bytes : 0);
    if (p->C < k || p->C > kMaxSlots) {
      set_error("pool of %lld slots: need top_k = %d <= slots <= %d", (long long)p->C, k, kMaxSlots);
      return FT_E_INVALID;
    }
    const char* fault = std::getenv("FT_MOE_FAULT");
    if (fault && std::strncmp(fault, "copy:", 5) == 0) p->fault_copy = std::atoll(fault + 5);
    if (fault && std::strncmp(fault, "work_alloc:", 11) == 0) p->fault_work_alloc = std::atoi(fault + 11);
    if (fault && std::strncmp(fault, "mx_alloc:", 9) == 0) p->fault_mx_alloc = std::atoi(fault + 9);
    if (fault && std::strncmp(fault, "corrupt:", 8) == 0) p->corrupt_copy = std::atoll(fault + 8);
    if (const char* cs = std::getenv("FT_MOE_DEBUG_CHECKSUM")) p->checksum = cs[0] != '\0' && std::strcmp(cs, "0");
    if (const char* lg = std::getenv("FT_MOE_LOG")) p->log_every = std::max(0, std::atoi(lg));

    // ---- pinned host store: one entry per distinct (blob pointer, format)
    std::map<std::pair<const void*, int>, int64_t> seen;
    p->key_off.resize(size_t(L) * E);
    std::vector<std::pair<const void*, int>> order;
    int64_t off = 0;
    for (int l = 0; l < L; ++l)
      for (int e = 0; e < E; ++e) {
        const auto key = std::make_pair(wts->expert[int64_t(l) * E + e], p->fmt[l]);
        auto it = seen.find(key);
        if (it == seen.end()) {
          seen[key] = off;
          order.push_back(key);
          p->key_off[int64_t(l) * E + e] = off;
          off += p->slot_bytes;
        } else {
          p->key_off[int64_t(l) * E + e] = it->second;
        }
      }
    p->layer_contig.assign(L, 0);
    for (int l = 0; l < L; ++l) {
      bool c = p->lay[p->fmt[l]].bytes == p->slot_bytes;
      for (int e = 1; e < E && c; ++e)
        c = p->key_off[int64_t(l) * E + e] == p->key_off[int64_t(l) * E] + int64_t(e) * p->slot_bytes;
      p->layer_contig[l] = c;
    }
    p->host_bytes = off;
    DeviceGuard dg(p->device);
    // the static scratch of ft_moe_layer_forward_noalloc: its device address
    // on this device, looked up once (a failure is reported by that call)
    {
      const std::string keep = get_error();
      if (scratch_register_device(p->device) != FT_OK) set_error("%s", keep.c_str());
    }
    if (fault && std::strcmp(fault, "pinned_alloc") == 0) {
      set_error("injected pinned allocation failure (%lld bytes)", (long long)off);
      return FT_E_OOM_PINNED;
    }
    if (hipHostMalloc(reinterpret_cast<void**>(&p->host_store), size_t(off), hipHostMallocDefault) != hipSuccess) {
      (void)hipGetLastError();
      p->host_store = nullptr;
      set_error("pinned host allocation of %lld bytes failed", (long long)off);
      return FT_E_OOM_PINNED;
    }
    {
      void* hd = nullptr;
      if (hipHostGetDevicePointer(&hd, p->host_store, 0) != hipSuccess) {
        (void)hipGetLastError();
        ft_moe_destroy_pool(p.release());
        set_error("pinned host store is not mapped for the device");
        return FT_E_HIP;
      }
      p->host_store_dev = static_cast<const uint8_t*>(hd);
    }
    {
      const int nthr = std::max(1, std::min(16, int(std::thread::hardware_concurrency())));
      parallel_for(int(order.size()), nthr, [&](int b, int e) {
        for (int i = b; i < e; ++i) {
          const auto& key = order[i];
          repack_expert(p->lay[key.second], static_cast<const uint8_t*>(key.first), p->host_store + seen[key]);
        }
      });
    }

    // ---- device memory
    int rc;
    if ((rc = dev_alloc(&p->arena, p->C * p->slot_bytes))) {
      ft_moe_destroy_pool(p.release());
      return rc;
    }
    const int64_t rsz = int64_t(L) * E * H;
    if ((rc = dev_alloc(&p->router_dev, rsz))) {
      ft_moe_destroy_pool(p.release());
      return rc;
    }
    FT_HIP_CHECK(hipMemcpy(p->router_dev, wts->router_w, size_t(rsz) * 4, hipMemcpyHostToDevice));
    if (p->shared) {
      p->shared_stride = p->slot_bytes;
      if ((rc = dev_alloc(&p->shared_dev, int64_t(L) * p->shared_stride))) {
        ft_moe_destroy_pool(p.release());
        return rc;
      }
      std::vector<uint8_t> tmp(p->slot_bytes);
      for (int l = 0; l < L; ++l) {
        repack_expert(p->lay[p->fmt[l]], static_cast<const uint8_t*>(wts->shared[l]), tmp.data());
        FT_HIP_CHECK(hipMemcpy(p->shared_dev + int64_t(l) * p->shared_stride, tmp.data(),
                               size_t(p->lay[p->fmt[l]].bytes), hipMemcpyHostToDevice));
      }
    }
    const int64_t C = p->C;
    if ((rc = dev_alloc(&p->tab.key2slot, int64_t(L) * E)) || (rc = dev_alloc(&p->tab.slot_key, C)) ||
        (rc = dev_alloc(&p->tab.slot_last, C)) || (rc = dev_alloc(&p->tab.lru[0], C)) ||
        (rc = dev_alloc(&p->tab.lru[1], C)) || (rc = dev_alloc(&p->tab.lru_cur, 1)) ||
        (rc = dev_alloc(&p->tab.clock, 1)) || (rc = dev_alloc(&p->tab.stats, int64_t(L) * ST_COUNT)) ||
        (rc = dev_alloc(&p->tab.min_gap, L)) || (rc = dev_alloc(&p->groups, E + 2)) ||
        (rc = dev_alloc(&p->glist, E + 2)) || (rc = dev_alloc(&p->gdesc, E + 2)) ||
        (rc = dev_alloc(&p->count_max, 1)) || (rc = dev_alloc(&p->dev_header, 16)) ||
        (rc = dev_alloc(&p->fail_dev, 2 * E + 2)) || (rc = dev_alloc(&p->key_off_dev, int64_t(L) * E)) ||
        (rc = dev_alloc(&p->prof_cnt_dev, 24)) || (rc = dev_alloc(&p->copy_clk, 3)) ||
        (rc = dev_alloc(&p->copy_ticks, L))) {
      ft_moe_destroy_pool(p.release());
      return rc;
    }
    FT_HIP_CHECK(hipMemset(p->tab.key2slot, 0xFF, size_t(L) * E * 4));
    FT_HIP_CHECK(hipMemset(p->gdesc, 0, size_t(E + 2) * sizeof(GroupDesc)));
    FT_HIP_CHECK(hipMemset(p->tab.slot_key, 0xFF, size_t(C) * 4));
    FT_HIP_CHECK(hipMemset(p->tab.lru_cur, 0, 4));
    FT_HIP_CHECK(hipMemset(p->tab.slot_last, 0, size_t(C) * 8));
    FT_HIP_CHECK(hipMemset(p->tab.clock, 0, 8));
    FT_HIP_CHECK(hipMemset(p->tab.stats, 0, size_t(L) * ST_COUNT * 8));
    FT_HIP_CHECK(hipMemset(p->prof_cnt_dev, 0, 24 * 8));
    FT_HIP_CHECK(hipMemset(p->copy_ticks, 0, size_t(L) * 8));
    {
      const uint64_t clk0[3] = {~0ull, 0ull, 0ull};
      FT_HIP_CHECK(hipMemcpy(p->copy_clk, clk0, sizeof(clk0), hipMemcpyHostToDevice));
      int khz = 0;
      FT_HIP_CHECK(hipDeviceGetAttribute(&khz, hipDeviceAttributeWallClockRate, p->device));
      p->wall_khz = double(khz);
      p->copy_ms_host.assign(L, 0.0);
    }
    {
      const int32_t big = INT32_MAX;
      FT_HIP_CHECK(hipMemcpy(p->count_max, &big, 4, hipMemcpyHostToDevice));
    }
    FT_HIP_CHECK(hipMemcpy(p->key_off_dev, p->key_off.data(), p->key_off.size() * 8, hipMemcpyHostToDevice));
    for (int f = 1; f <= 3; ++f)
      if (p->lay[f].bytes % 16) p->dev_decode = false;
    if (const char* dp = std::getenv("FT_MOE_DECODE_PATH")) p->dev_decode = p->dev_decode && std::strcmp(dp, "host");
    if (p->fault_copy >= 0 || p->corrupt_copy >= 0) p->dev_decode = false;  // injected copy faults: host path only
    if (p->checksum) {
      // checksum of every key's blob as the pinned store holds it
      std::vector<uint64_t> sums(size_t(L) * E);
      const int nthr = std::max(1, std::min(16, int(std::thread::hardware_concurrency())));
      parallel_for(L * E, nthr, [&](int b, int e) {
        for (int i = b; i < e; ++i)
          sums[i] = slot_checksum(p->host_store + p->key_off[i], p->lay[p->fmt[i / E]].bytes);
      });
      if ((rc = dev_alloc(&p->key_sum_dev, int64_t(L) * E)) || (rc = dev_alloc(&p->bad_dev, 2))) {
        ft_moe_destroy_pool(p.release());
        return rc;
      }
      FT_HIP_CHECK(hipMemcpy(p->key_sum_dev, sums.data(), sums.size() * 8, hipMemcpyHostToDevice));
      FT_HIP_CHECK(hipMemset(p->bad_dev, 0, 16));
    }
    if (const char* pz = std::getenv("FT_MOE_POISON")) p->poison = pz[0] != '\0' && std::strcmp(pz, "0") != 0;
    {
      std::vector<int32_t> lru(C);
      for (int64_t i = 0; i < C; ++i) lru[i] = int32_t(i);
      FT_HIP_CHECK(hipMemcpy(p->tab.lru[0], lru.data(), size_t(C) * 4, hipMemcpyHostToDevice));
      std::vector<double> g(L, INFINITY);
      FT_HIP_CHECK(hipMemcpy(p->tab.min_gap, g.data(), size_t(L) * 8, hipMemcpyHostToDevice));
    }
    for (int c = 0; c < p->n_copy; ++c) {
      FT_HIP_CHECK(hipStreamCreateWithFlags(&p->copy[c], hipStreamNonBlocking));
      FT_HIP_CHECK(hipEventCreateWithFlags(&p->ev_copy_done[c], hipEventDisableTiming));
    }
    p->copy_stream = p->copy[0];
    for (hipEvent_t* e : {&p->ev_resolved, &p->ev_copied, &p->ev_sync, &p->ev_cpu_copied, &p->ev_done[0],
                          &p->ev_done[1], &p->ev_staged[0], &p->ev_staged[1], &p->ev_call_done})
      FT_HIP_CHECK(hipEventCreateWithFlags(e, hipEventDisableTiming));
    FT_HIP_CHECK(hipDeviceSynchronize());
    *out = p.release();
    return (*out)->C < 2 * int64_t(E) ? FT_WARN_STAGING_SMALL : FT_OK;
  } catch (const std::exception& ex) {
    set_error("init failed: %s", ex.what());
    return FT_E_INVALID;
  }
}

}  // extern "C"

namespace {

// Per-call buffers of a device-driven decode call carved from `base` (256-byte
// aligned regions, in this order); with base null only the size is computed.
struct ScratchCarve {
  double* z;
  int32_t *sel, *pair_slot, *pair_row, *row_tok;
  float *w, *row_w;
  double* gap;
  uint8_t* pair_flag;
  uint16_t *hbuf, *pbuf;
  int64_t bytes;
};

ScratchCarve carve_scratch(const ft_moe_pool* p, int T, uint8_t* base) {
  ScratchCarve c{};
  int64_t off = 0;
  auto take = [&](int64_t n) -> uint8_t* {
    uint8_t* q = base ? base + off : nullptr;
    off += (n + 255) & ~int64_t(255);
    return q;
  };
  const int64_t pairs = int64_t(T) * p->k, rows = pairs + (p->shared ? T : 0);
  c.z = reinterpret_cast<double*>(take(int64_t(T) * p->E * 8));
  c.sel = reinterpret_cast<int32_t*>(take(pairs * 4));
  c.w = reinterpret_cast<float*>(take(pairs * 4));
  c.gap = reinterpret_cast<double*>(take(int64_t(T) * 8));
  c.pair_flag = take(pairs);
  c.pair_slot = reinterpret_cast<int32_t*>(take(pairs * 4));
  c.pair_row = reinterpret_cast<int32_t*>(take(pairs * 4));
  c.row_tok = reinterpret_cast<int32_t*>(take(rows * 4));
  c.row_w = reinterpret_cast<float*>(take(rows * 4));
  c.hbuf = reinterpret_cast<uint16_t*>(take(rows * p->I * 2));
  c.pbuf = reinterpret_cast<uint16_t*>(take(rows * p->H * 2));
  c.bytes = off;
  return c;
}

// Points the pool's per-call buffers at a carve of the scratch for one call
// (no mapped readback: the resolve kernel then publishes no miss lists) and
// puts them back afterwards.
struct ScratchView {
  ft_moe_pool* p;
  double *z, *gap;
  int32_t *sel, *pair_slot, *pair_row, *row_tok;
  float *w, *row_w;
  uint8_t *pair_flag, *rb_dev;
  uint16_t *hbuf, *pbuf;
  bool last_pending;
  ScratchView(ft_moe_pool* pp, const ScratchCarve& c)
      : p(pp), z(pp->z), gap(pp->gap), sel(pp->sel), pair_slot(pp->pair_slot), pair_row(pp->pair_row),
        row_tok(pp->row_tok), w(pp->w), row_w(pp->row_w), pair_flag(pp->pair_flag), rb_dev(pp->rb_dev),
        hbuf(pp->hbuf), pbuf(pp->pbuf), last_pending(pp->last_pending) {
    p->z = c.z; p->gap = c.gap; p->sel = c.sel; p->pair_slot = c.pair_slot; p->pair_row = c.pair_row;
    p->row_tok = c.row_tok; p->w = c.w; p->row_w = c.row_w; p->pair_flag = c.pair_flag; p->rb_dev = nullptr;
    p->hbuf = c.hbuf; p->pbuf = c.pbuf;
  }
  ~ScratchView() {
    p->z = z; p->gap = gap; p->sel = sel; p->pair_slot = pair_slot; p->pair_row = pair_row; p->row_tok = row_tok;
    p->w = w; p->row_w = row_w; p->pair_flag = pair_flag; p->rb_dev = rb_dev; p->hbuf = hbuf; p->pbuf = pbuf;
    // the mapped readback still holds the lists of the call before this one
    p->last_pending = last_pending;
  }
};

int forward_impl(ft_moe_pool* p, int32_t layer, int32_t num_tokens, const void* x_bf16, const float* router_bias,
                 void* out_bf16, int32_t flags, void* hip_stream, ft_moe_trace* trace, bool noalloc) {
  {
    if (!p || !x_bf16 || !out_bf16) {
      set_error("NULL pool, x or out");
      return FT_E_INVALID;
    }
    if (layer < 0 || layer >= p->L || num_tokens < 0) {
      set_error("bad layer %d or token count %d", layer, num_tokens);
      return FT_E_INVALID;
    }
    if ((reinterpret_cast<uintptr_t>(x_bf16) | reinterpret_cast<uintptr_t>(out_bf16)) & 15) {
      set_error("x and out must be 16-byte aligned");
      return FT_E_INVALID;
    }
    const int mode = flags & FT_FWD_MODE_MASK;
    const int act = (flags & FT_ACT_MASK) >> 4;
    const bool hit_d2d = (flags & FT_FWD_PREFILL_HIT_D2D) != 0;
    if (mode > FT_FWD_PREFILL_STAGED || act > 2 ||
        (flags & ~(FT_FWD_MODE_MASK | FT_ACT_MASK | FT_FWD_PREFILL_HIT_D2D)) ||
        (hit_d2d && mode != FT_FWD_PREFILL_STAGED)) {
      set_error("bad flags 0x%x", flags);
      return FT_E_INVALID;
    }
    if (act != 0 && mode == FT_FWD_DECODE) {
      set_error("MX activation modes apply to prefill calls only");
      return FT_E_INVALID;
    }
    if (mode == FT_FWD_DECODE && p->prefill_next != 0) {
      set_error("decode call while prefill chunk is at layer %d", p->prefill_next);
      return FT_E_STATE;
    }
    if (num_tokens == 0) return FT_OK;
    const int T = num_tokens, E = p->E, k = p->k;
    const bool dev_path = mode == FT_FWD_DECODE && p->dev_decode && p->share_fmt[p->fmt[layer]] == 0.0 && int64_t(T) * k <= p->C;
    ScratchCarve carve{};
    if (noalloc) {
      if (!dev_path || flags != FT_FWD_DECODE) {
        set_error("ft_moe_layer_forward_noalloc runs device-driven decode calls only: flags FT_FWD_DECODE, no "
                  "hybrid share, T*top_k <= pool slots (T=%d, flags 0x%x, share %g)", T, flags,
                  p->share_fmt[p->fmt[layer]]);
        return FT_E_INVALID;
      }
      carve = carve_scratch(p, T, nullptr);
      if (carve.bytes > kScratchBytes) {
        set_error("ft_moe_layer_forward_noalloc: %d tokens need %lld bytes of scratch, the maximum is %lld", T,
                  (long long)carve.bytes, (long long)kScratchBytes);
        return FT_E_INVALID;
      }
    }
    DeviceGuard dg(p->device);
    hipStream_t s = static_cast<hipStream_t>(hip_stream);
    hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
    FT_HIP_CHECK(hipStreamIsCapturing(s, &cap));
    const bool capturing = cap != hipStreamCaptureStatusNone;
    if (capturing && p->checksum) {
      set_error("the debug checksum mode (FT_MOE_DEBUG_CHECKSUM) waits after each call: no graph capture");
      return FT_E_INVALID;
    }
    if (capturing && !noalloc && (!dev_path || T > p->cap_T)) {
      set_error("a captured call must be a device-driven decode call of at most the reserved %d tokens "
                "(T=%d, mode %d)", p->cap_T, T, mode);
      return FT_E_INVALID;
    }
    int rc;
    std::unique_ptr<ScratchView> view;
    if (noalloc) {
      uint8_t* base = scratch_device_ptr(p->device);
      if (base == nullptr) {
        if ((rc = scratch_register_device(p->device))) return rc;
        base = scratch_device_ptr(p->device);
      }
      view = std::make_unique<ScratchView>(p, carve_scratch(p, T, base));
    } else if ((rc = ensure_capacity(p, num_tokens))) {
      return rc;
    }
    const int32_t prof_saved = p->prof_mask;
    // no event records inside a graph; the no-alloc call creates no events
    if (capturing || noalloc) p->prof_mask = 0;
    struct Restore {
      ft_moe_pool* p;
      int32_t m;
      ~Restore() { p->prof_mask = m; }
    } restore{p, prof_saved};
    if (p->any_call && s != p->last_stream && !capturing) {
      // a call on another stream: order it after everything enqueued so far
      FT_HIP_CHECK(hipEventRecord(p->ev_call_done, p->last_stream));
      FT_HIP_CHECK(hipStreamWaitEvent(s, p->ev_call_done, 0));
    }
    Ev e0 = prof_pair(p, s, FT_STAGE_ROUTER);
    FT_HIP_CHECK(launch_router_logits(static_cast<const uint16_t*>(x_bf16), p->router_dev + int64_t(layer) * E * p->H,
                                      router_bias, p->z, T, p->H, E, s, e0));
    prof_push(p, FT_STAGE_ROUTER, e0, double(E) * p->H * 4 + double(T) * p->H * 2, 2.0 * T * E * p->H);
    if (mode == FT_FWD_PREFILL_STAGED) {
      // decode folds the top-k into its resolve kernel
      e0 = prof_pair(p, s, FT_STAGE_TOPK);
      FT_HIP_CHECK(launch_topk(p->z, T, E, k, p->sel, p->w, p->gap, s, e0));
      prof_push(p, FT_STAGE_TOPK, e0, double(T) * E * 8, 0.0);
    }
    if (mode == FT_FWD_DECODE) {
      rc = dev_path ? forward_decode_dev(p, layer, T, x_bf16, out_bf16, s)
                    : forward_decode(p, layer, T, x_bf16, out_bf16, s);
    } else {
      rc = forward_prefill(p, layer, T, x_bf16, out_bf16, s, act, hit_d2d);
    }
    if (rc) return rc;
    if (!capturing) {
      p->last_stream = s;
      p->any_call = true;
    } else {
      p->last_pending = false;  // the lists belong to a replay, not to this call
    }
    if (trace) {
      const size_t n = size_t(T) * k;
      if (trace->sel) FT_HIP_CHECK(hipMemcpyAsync(trace->sel, p->sel, n * 4, hipMemcpyDeviceToDevice, s));
      if (trace->w) FT_HIP_CHECK(hipMemcpyAsync(trace->w, p->w, n * 4, hipMemcpyDeviceToDevice, s));
      if (trace->slot) FT_HIP_CHECK(hipMemcpyAsync(trace->slot, p->pair_slot, n * 4, hipMemcpyDeviceToDevice, s));
      if (trace->flag) FT_HIP_CHECK(hipMemcpyAsync(trace->flag, p->pair_flag, n, hipMemcpyDeviceToDevice, s));
      if (trace->row) FT_HIP_CHECK(hipMemcpyAsync(trace->row, p->pair_row, n * 4, hipMemcpyDeviceToDevice, s));
    }
    if (p->checksum && !capturing) {
      uint64_t bad[2] = {0, 0};
      FT_HIP_CHECK(hipStreamSynchronize(s));
      FT_HIP_CHECK(hipMemcpy(bad, p->bad_dev, 16, hipMemcpyDeviceToHost));
      if (bad[0] != 0) {
        FT_HIP_CHECK(hipMemset(p->bad_dev, 0, 16));
        const int64_t key = int64_t(bad[0]) - 1;
        set_error("slot checksum mismatch: key %lld (layer %lld, expert %lld) in slot %lld does not hold its weights",
                  (long long)key, (long long)(key / E), (long long)(key % E), (long long)bad[1]);
        return FT_E_HIP;
      }
    }
    if (p->log_every > 0 && !capturing && ++p->log_calls % uint64_t(p->log_every) == 0) {
      ft_moe_stats st;
      if (ft_moe_pool_stats(p, -1, &st, 0) == FT_OK)
        std::fprintf(stderr,
                     "ftmoe: %llu calls, pair hit rate %.4f, experts %llu hit / %llu missed (%llu on host), "
                     "%llu evictions, %.3f GB copied in %.1f ms, slots %lld / %lld\n",
                     (unsigned long long)st.calls,
                     double(st.pair_hits) / double(std::max<uint64_t>(st.pair_hits + st.pair_misses, 1)),
                     (unsigned long long)st.expert_hits, (unsigned long long)st.expert_misses,
                     (unsigned long long)st.cpu_misses, (unsigned long long)st.evictions, double(st.bytes_h2d) * 1e-9,
                     st.copy_ms, (long long)st.slots_used, (long long)st.slots_total);
    }
    return FT_OK;
  }
}

}  // namespace

extern "C" {

int ft_moe_layer_forward(ft_moe_pool* p, int32_t layer, int32_t num_tokens, const void* x_bf16,
                         const float* router_bias, void* out_bf16, int32_t flags, void* hip_stream,
                         ft_moe_trace* trace) {
  try {
    return forward_impl(p, layer, num_tokens, x_bf16, router_bias, out_bf16, flags, hip_stream, trace, false);
  } catch (const std::exception& ex) {
    set_error("forward failed: %s", ex.what());
    return FT_E_INVALID;
  }
}

int ft_moe_layer_forward_noalloc(ft_moe_pool* p, int32_t layer, int32_t num_tokens, const void* x_bf16,
                                 const float* router_bias, void* out_bf16, int32_t flags, void* hip_stream,
                                 ft_moe_trace* trace) {
  try {
    return forward_impl(p, layer, num_tokens, x_bf16, router_bias, out_bf16, flags, hip_stream, trace, true);
  } catch (const std::exception& ex) {
    set_error("forward failed: %s", ex.what());
    return FT_E_INVALID;
  }
}

int ft_moe_pool_stats(ft_moe_pool* p, int32_t layer, ft_moe_stats* out, int32_t reset) {
  if (!p || !out || layer < -1 || layer >= p->L) {
    set_error("bad pool, layer or output");
    return FT_E_INVALID;
  }
  DeviceGuard dg(p->device);
  FT_HIP_CHECK(hipDeviceSynchronize());
  std::vector<uint64_t> st(size_t(p->L) * ST_COUNT);
  std::vector<double> g(p->L);
  std::vector<int32_t> sk(p->C);
  std::vector<uint64_t> ticks(p->L);
  copy_drain(p, true);
  FT_HIP_CHECK(hipMemcpy(st.data(), p->tab.stats, st.size() * 8, hipMemcpyDeviceToHost));
  FT_HIP_CHECK(hipMemcpy(ticks.data(), p->copy_ticks, ticks.size() * 8, hipMemcpyDeviceToHost));
  FT_HIP_CHECK(hipMemcpy(g.data(), p->tab.min_gap, g.size() * 8, hipMemcpyDeviceToHost));
  FT_HIP_CHECK(hipMemcpy(sk.data(), p->tab.slot_key, sk.size() * 4, hipMemcpyDeviceToHost));
  std::memset(out, 0, sizeof(*out));
  out->min_topk_gap = INFINITY;
  for (int l = 0; l < p->L; ++l) {
    if (layer >= 0 && l != layer) continue;
    const uint64_t* s = &st[size_t(l) * ST_COUNT];
    out->pair_hits += s[ST_PAIR_HITS];
    out->pair_misses += s[ST_PAIR_MISSES];
    out->expert_hits += s[ST_EXPERT_HITS];
    out->expert_misses += s[ST_EXPERT_MISSES];
    out->cpu_misses += s[ST_CPU_MISSES];
    out->evictions += s[ST_EVICTIONS];
    out->bytes_h2d += s[ST_BYTES_H2D];
    out->calls += s[ST_CALLS];
    out->min_topk_gap = std::min(out->min_topk_gap, g[l]);
    out->copy_ms += (p->wall_khz > 0 ? double(ticks[l]) / p->wall_khz : 0.0) + p->copy_ms_host[l];
  }
  out->slots_total = p->C;
  for (int32_t v : sk) out->slots_used += v >= 0;
  if (reset) {
    FT_HIP_CHECK(hipMemset(p->tab.stats, 0, st.size() * 8));
    FT_HIP_CHECK(hipMemset(p->copy_ticks, 0, ticks.size() * 8));
    std::fill(p->copy_ms_host.begin(), p->copy_ms_host.end(), 0.0);
    std::vector<double> inf(p->L, INFINITY);
    FT_HIP_CHECK(hipMemcpy(p->tab.min_gap, inf.data(), inf.size() * 8, hipMemcpyHostToDevice));
  }
  return FT_OK;
}

int ft_moe_last_misses(const ft_moe_pool* p, int32_t* stream_expert, int32_t* stream_slot, int32_t* n_stream,
                       int32_t* cpu_expert, int32_t* n_cpu, int32_t cap) {
  if (!p) {
    set_error("NULL pool");
    return FT_E_INVALID;
  }
  {
    DeviceGuard dg(p->device);
    const int rc = read_pending_misses(p);
    if (rc) return rc;
  }
  if (n_stream) *n_stream = int32_t(p->last_se.size());
  if (n_cpu) *n_cpu = int32_t(p->last_ce.size());
  for (size_t i = 0; i < p->last_se.size() && int32_t(i) < cap; ++i) {
    if (stream_expert) stream_expert[i] = p->last_se[i];
    if (stream_slot) stream_slot[i] = p->last_ss[i];
  }
  for (size_t i = 0; i < p->last_ce.size() && int32_t(i) < cap; ++i)
    if (cpu_expert) cpu_expert[i] = p->last_ce[i];
  return FT_OK;
}

int ft_moe_pool_table(ft_moe_pool* p, int32_t* slot_key, uint64_t* slot_last, uint64_t* clock, int64_t* slots) {
  if (!p) {
    set_error("NULL pool");
    return FT_E_INVALID;
  }
  DeviceGuard dg(p->device);
  FT_HIP_CHECK(hipDeviceSynchronize());
  if (slot_key) FT_HIP_CHECK(hipMemcpy(slot_key, p->tab.slot_key, size_t(p->C) * 4, hipMemcpyDeviceToHost));
  if (slot_last) FT_HIP_CHECK(hipMemcpy(slot_last, p->tab.slot_last, size_t(p->C) * 8, hipMemcpyDeviceToHost));
  if (clock) FT_HIP_CHECK(hipMemcpy(clock, p->tab.clock, 8, hipMemcpyDeviceToHost));
  if (slots) *slots = p->C;
  return FT_OK;
}

// Elastic resize (the pages: VRAM moves between the expert cache and other
// memory while the engine runs -- dev.to article "FreeToken uses
// bandwidth-adaptive CPU-GPU co-execution on your desktop", section "Memory
// that moves while the engine runs").  The new_slots most recently used
// residents survive; a survivor keeps its slot if it still exists, the others
// (ascending old slot) move to the lowest free slots below new_slots.  Last
// uses and the clock are unchanged.  Everything new is allocated before the
// pool changes, so a failed allocation leaves the pool as it was.
int ft_moe_resize_pool(ft_moe_pool* p, int64_t new_slots) {
  if (!p) {
    set_error("NULL pool");
    return FT_E_INVALID;
  }
  if (new_slots < p->k || new_slots > kMaxSlots) {
    set_error("pool of %lld slots: need top_k = %d <= slots <= %d", (long long)new_slots, p->k, kMaxSlots);
    return FT_E_INVALID;
  }
  if (p->prefill_next != 0) {
    set_error("resize while a prefill chunk is at layer %d", p->prefill_next);
    return FT_E_STATE;
  }
  DeviceGuard dg(p->device);
  FT_HIP_CHECK(hipDeviceSynchronize());
  const int64_t C = p->C, NC = new_slots, LE = int64_t(p->L) * p->E;
  std::vector<int32_t> key(C), k2s(LE);
  std::vector<uint64_t> last(C);
  FT_HIP_CHECK(hipMemcpy(key.data(), p->tab.slot_key, size_t(C) * 4, hipMemcpyDeviceToHost));
  FT_HIP_CHECK(hipMemcpy(last.data(), p->tab.slot_last, size_t(C) * 8, hipMemcpyDeviceToHost));
  FT_HIP_CHECK(hipMemcpy(k2s.data(), p->tab.key2slot, size_t(LE) * 4, hipMemcpyDeviceToHost));

  std::vector<int64_t> res;
  for (int64_t sl = 0; sl < C; ++sl)
    if (key[sl] >= 0) res.push_back(sl);
  // ties in last use go to the lower slot, as in the victim order of a call
  std::sort(res.begin(), res.end(),
            [&](int64_t a, int64_t b) { return last[a] != last[b] ? last[a] < last[b] : a < b; });
  const size_t n_ev = res.size() > size_t(NC) ? res.size() - size_t(NC) : 0;
  std::vector<int64_t> keep, move;
  for (size_t i = n_ev; i < res.size(); ++i) (res[i] < NC ? keep : move).push_back(res[i]);
  std::sort(keep.begin(), keep.end());
  std::sort(move.begin(), move.end());
  std::vector<int32_t> nkey(NC, -1);
  std::vector<uint64_t> nlast(NC, 0);
  for (int64_t sl : keep) {
    nkey[sl] = key[sl];
    nlast[sl] = last[sl];
  }
  std::vector<std::pair<int64_t, int64_t>> moves;  // old slot -> new slot
  {
    int64_t hole = 0;
    for (int64_t sl : move) {
      while (nkey[hole] >= 0) ++hole;
      nkey[hole] = key[sl];
      nlast[hole] = last[sl];
      moves.emplace_back(sl, hole);
      ++hole;
    }
  }
  for (size_t i = 0; i < n_ev; ++i) k2s[key[res[i]]] = -1;
  for (auto& mv : moves) k2s[key[mv.first]] = int32_t(mv.second);
  // recency order: free slots ascending, then residents by last use
  std::vector<int32_t> order;
  for (int64_t sl = 0; sl < NC; ++sl)
    if (nkey[sl] < 0) order.push_back(int32_t(sl));
  {
    std::vector<int32_t> r;
    for (int64_t sl = 0; sl < NC; ++sl)
      if (nkey[sl] >= 0) r.push_back(int32_t(sl));
    std::sort(r.begin(), r.end(),
              [&](int32_t a, int32_t b) { return nlast[a] != nlast[b] ? nlast[a] < nlast[b] : a < b; });
    order.insert(order.end(), r.begin(), r.end());
  }

  // new device memory first
  uint8_t* arena = nullptr;
  int32_t *sk = nullptr, *l0 = nullptr, *l1 = nullptr;
  uint64_t* sla = nullptr;
  int rc;
  if ((rc = dev_alloc(&arena, NC * p->slot_bytes)) || (rc = dev_alloc(&sk, NC)) || (rc = dev_alloc(&sla, NC)) ||
      (rc = dev_alloc(&l0, NC)) || (rc = dev_alloc(&l1, NC))) {
    hipFree(arena); hipFree(sk); hipFree(sla); hipFree(l0); hipFree(l1);
    return rc;
  }
  for (int64_t sl : keep)
    FT_HIP_CHECK(hipMemcpyAsync(arena + sl * p->slot_bytes, p->arena + sl * p->slot_bytes, size_t(p->slot_bytes),
                                hipMemcpyDeviceToDevice, nullptr));
  for (auto& mv : moves)
    FT_HIP_CHECK(hipMemcpyAsync(arena + mv.second * p->slot_bytes, p->arena + mv.first * p->slot_bytes,
                                size_t(p->slot_bytes), hipMemcpyDeviceToDevice, nullptr));
  FT_HIP_CHECK(hipMemcpy(sk, nkey.data(), size_t(NC) * 4, hipMemcpyHostToDevice));
  FT_HIP_CHECK(hipMemcpy(sla, nlast.data(), size_t(NC) * 8, hipMemcpyHostToDevice));
  FT_HIP_CHECK(hipMemcpy(l0, order.data(), size_t(NC) * 4, hipMemcpyHostToDevice));
  FT_HIP_CHECK(hipMemcpy(p->tab.key2slot, k2s.data(), size_t(LE) * 4, hipMemcpyHostToDevice));
  FT_HIP_CHECK(hipMemset(p->tab.lru_cur, 0, 4));
  FT_HIP_CHECK(hipDeviceSynchronize());
  hipFree(p->arena); hipFree(p->tab.slot_key); hipFree(p->tab.slot_last); hipFree(p->tab.lru[0]);
  hipFree(p->tab.lru[1]);
  p->arena = arena;
  p->tab.slot_key = sk;
  p->tab.slot_last = sla;
  p->tab.lru[0] = l0;
  p->tab.lru[1] = l1;
  p->C = NC;
  return NC < 2 * int64_t(p->E) ? FT_WARN_STAGING_SMALL : FT_OK;
}

int ft_moe_reserve(ft_moe_pool* p, int32_t max_tokens) {
  if (!p || max_tokens < 0) {
    set_error("bad pool or token count");
    return FT_E_INVALID;
  }
  DeviceGuard dg(p->device);
  return ensure_capacity(p, max_tokens);
}

int ft_moe_set_hybrid_share(ft_moe_pool* p, double share) {
  if (!p || !(share >= 0.0 && share <= 1.0)) {
    set_error("share must be in [0,1]");
    return FT_E_INVALID;
  }
  for (double& v : p->share_fmt) v = share;
  for (auto& o : p->obs) o = ft_moe_pool::Obs{};
  return FT_OK;
}

int ft_moe_set_hybrid_share_format(ft_moe_pool* p, int32_t fmt, double share) {
  if (!p || fmt < FT_FMT_MXFP4 || fmt > FT_FMT_FP8_B128 || !(share >= 0.0 && share <= 1.0)) {
    set_error("need a pool, a format FT_FMT_* and a share in [0,1]");
    return FT_E_INVALID;
  }
  p->share_fmt[fmt] = share;
  p->obs[fmt] = ft_moe_pool::Obs{};
  return FT_OK;
}

int ft_moe_get_hybrid_share(const ft_moe_pool* p, int32_t fmt, double* share) {
  if (!p || fmt < FT_FMT_MXFP4 || fmt > FT_FMT_FP8_B128 || !share) {
    set_error("need a pool, a format FT_FMT_* and an output");
    return FT_E_INVALID;
  }
  *share = p->share_fmt[fmt];
  return FT_OK;
}

int ft_moe_rebalance(ft_moe_pool* p, int32_t apply, ft_moe_rebalance_report* out) {
  if (!p || !out) {
    set_error("need a pool and a report");
    return FT_E_INVALID;
  }
  DeviceGuard dg(p->device);
  copy_drain(p, true);
  ft_moe_rebalance_report r{};
  for (int f = FT_FMT_MXFP4; f <= FT_FMT_FP8_B128; ++f) {
    const ft_moe_pool::Obs& o = p->obs[f];
    r.host_bytes[f] = o.host_bytes;
    r.host_seconds[f] = o.host_sec;
    r.copy_bytes[f] = o.copy_bytes;
    r.copy_seconds[f] = o.copy_ms * 1e-3;
    r.gpu_bytes_per_s[f] = p->gpu_rate[f];
    r.share[f] = p->share_fmt[f];
    if (o.host_bytes > 0.0 && o.host_sec > 0.0 && o.copy_bytes > 0.0 && o.copy_ms > 0.0) {
      // seconds per expert byte on each side, as in the one-time decision
      const double ts = o.copy_ms * 1e-3 / o.copy_bytes + (p->gpu_rate[f] > 0.0 ? 1.0 / p->gpu_rate[f] : 0.0);
      const double tc = o.host_sec / o.host_bytes;
      r.share[f] = ts / (ts + tc);
      r.changed[f] = 1;
    }
  }
  if (apply)
    for (int f = FT_FMT_MXFP4; f <= FT_FMT_FP8_B128; ++f)
      if (r.changed[f]) p->share_fmt[f] = r.share[f];
  for (auto& o : p->obs) o = ft_moe_pool::Obs{};
  *out = r;
  return FT_OK;
}

int ft_moe_host_expert_rate(ft_moe_pool* p, int32_t layer, int32_t tokens, int32_t iters, double* bytes_per_s) {
  if (!p || layer < 0 || layer >= p->L || tokens < 1 || iters < 1 || !bytes_per_s) {
    set_error("bad arguments");
    return FT_E_INVALID;
  }
  const ExpertLayout& L = p->lay[p->fmt[layer]];
  std::vector<uint16_t> x(size_t(tokens) * p->H, 0x3F80), out(size_t(tokens) * p->H);
  std::vector<float> w(tokens, 1.0f);
  const uint8_t* blob = p->host_store + p->key_off[int64_t(layer) * p->E];
  if (!p->workers) p->workers = std::make_unique<WorkerPool>(p->cpu_threads);
  const HostExpertJob job{blob, x.data(), w.data(), tokens, out.data()};
  const auto t0 = std::chrono::steady_clock::now();
  for (int i = 0; i < iters; ++i) host_experts(L, &job, 1, *p->workers);
  const double sec = std::chrono::duration<double>(std::chrono::steady_clock::now() - t0).count();
  *bytes_per_s = double(p->canon_bytes[p->fmt[layer]]) * iters / std::max(sec, 1e-9);
  return FT_OK;
}

int ft_moe_mfma_rate(int32_t kind, int32_t iters, void* hip_stream, double* flops_per_s) {
  if (kind < 0 || kind > 4 || iters < 1 || iters > (1 << 20) || !flops_per_s) {
    set_error("bad arguments");
    return FT_E_INVALID;
  }
  hipStream_t s = static_cast<hipStream_t>(hip_stream);
  float* out = nullptr;
  if (hipMalloc(&out, mfma_peak_out_bytes()) != hipSuccess) {
    (void)hipGetLastError();
    set_error("device allocation of %zu bytes failed", mfma_peak_out_bytes());
    return FT_E_OOM_DEVICE;
  }
  hipEvent_t e0 = nullptr, e1 = nullptr;
  int rc = FT_OK;
  float ms = 0.f;
  auto run = [&]() -> int {
    FT_HIP_CHECK(hipEventCreate(&e0));
    FT_HIP_CHECK(hipEventCreate(&e1));
    FT_HIP_CHECK(launch_mfma_peak(kind, iters, 0, out, s));  // warm-up (clocks, code load)
    FT_HIP_CHECK(hipEventRecord(e0, s));
    FT_HIP_CHECK(launch_mfma_peak(kind, iters, 1, out, s));
    FT_HIP_CHECK(hipEventRecord(e1, s));
    FT_HIP_CHECK(hipEventSynchronize(e1));
    FT_HIP_CHECK(hipEventElapsedTime(&ms, e0, e1));
    return FT_OK;
  };
  rc = run();
  if (e0) (void)hipEventDestroy(e0);
  if (e1) (void)hipEventDestroy(e1);
  (void)hipFree(out);
  if (rc != FT_OK) return rc;
  *flops_per_s = mfma_peak_flops(kind, iters) / (double(std::max(ms, 1e-6f)) * 1e-3);
  return FT_OK;
}

int ft_moe_decide_mode(ft_moe_mode_report* r) {
  if (!r) {
    set_error("NULL report");
    return FT_E_INVALID;
  }
  double ts = 0.0, tc = 0.0;
  for (int f = 1; f <= 3; ++f) {
    if (r->layers[f] < 0) {
      set_error("negative layer count for format %d", f);
      return FT_E_INVALID;
    }
    if (r->layers[f] == 0) continue;
    const double b = r->expert_bytes[f], h = r->h2d_bytes_per_s[f], g = r->gpu_bytes_per_s[f],
                 c = r->cpu_bytes_per_s[f];
    if (!(b > 0.0) || !(h > 0.0) || !(g > 0.0) || !(c > 0.0) || !std::isfinite(b) || std::isnan(h) ||
        std::isnan(g) || std::isnan(c)) {
      set_error("format %d: expert bytes and rates must be positive", f);
      return FT_E_INVALID;
    }
    for (int l = 0; l < r->layers[f]; ++l) {
      ts += b / h + b / g;
      tc += b / c;
    }
  }
  r->t_stream = ts;
  r->t_cpu = tc;
  r->balanced_share = ts / (ts + tc);
  if (r->pool_slots >= r->all_experts) {
    r->mode = FT_MODE_FUSED;
    r->share = 0.0;
  } else if (tc < ts) {
    r->mode = FT_MODE_HYBRID;
    r->share = ts / (ts + tc);
  } else {
    r->mode = FT_MODE_OFFLOAD;
    r->share = 0.0;
  }
  return FT_OK;
}

int ft_moe_measure_mode(ft_moe_pool* p, int32_t tokens, int32_t apply, ft_moe_mode_report* out) {
  if (!p || !out || tokens < 1 || tokens > 64) {
    set_error("bad arguments (need a pool, a report and 1 <= tokens <= 64)");
    return FT_E_INVALID;
  }
  if (p->prefill_next != 0) {
    set_error("mode measurement while a prefill chunk is at layer %d", p->prefill_next);
    return FT_E_STATE;
  }
  DeviceGuard dg(p->device);
  ft_moe_mode_report r{};
  r.tokens = tokens;
  r.pool_slots = p->C;
  r.all_experts = int64_t(p->L) * p->E;
  const int n = std::min(p->E, 16), T = tokens, H = p->H;
  int rc = read_pending_misses(p);
  if (rc) return rc;
  if ((rc = ensure_capacity(p, (n * T + p->k - 1) / p->k))) return rc;
  FT_HIP_CHECK(hipDeviceSynchronize());
  uint8_t* tmp = nullptr;
  uint16_t* xd = nullptr;
  if ((rc = dev_alloc(&tmp, int64_t(n) * p->slot_bytes)) || (rc = dev_alloc(&xd, int64_t(T) * H))) {
    hipFree(tmp);
    return rc;
  }
  hipStream_t s = p->copy[0];
  hipEvent_t e0 = nullptr, e1 = nullptr;
  struct Cleanup {
    hipEvent_t& e0;
    hipEvent_t& e1;
    uint8_t* tmp;
    uint16_t* xd;
    ~Cleanup() {
      if (e0) hipEventDestroy(e0);
      if (e1) hipEventDestroy(e1);
      hipFree(tmp);
      hipFree(xd);
    }
  } guard{e0, e1, tmp, xd};
  FT_HIP_CHECK(hipEventCreate(&e0));
  FT_HIP_CHECK(hipEventCreate(&e1));
  {
    std::vector<uint16_t> ones(size_t(T) * H, 0x3F80);  // bf16 1.0
    FT_HIP_CHECK(hipMemcpy(xd, ones.data(), ones.size() * 2, hipMemcpyHostToDevice));
  }
  const int32_t prof_saved = p->prof_mask;
  p->prof_mask = 0;
  struct Restore {
    ft_moe_pool* p;
    int32_t m;
    ~Restore() { p->prof_mask = m; }
  } restore{p, prof_saved};
  constexpr int kReps = 3;
  double sec = 0.0;
  auto timed = [&](auto&& body) -> int {  // sec = seconds per repetition, after one warm-up
    body();
    FT_HIP_CHECK(hipEventRecord(e0, s));
    for (int i = 0; i < kReps; ++i) body();
    FT_HIP_CHECK(hipEventRecord(e1, s));
    FT_HIP_CHECK(hipEventSynchronize(e1));
    float ms = 0.0f;
    FT_HIP_CHECK(hipEventElapsedTime(&ms, e0, e1));
    sec = std::max(double(ms), 1e-6) * 1e-3 / kReps;
    return FT_OK;
  };
  for (int f = 1; f <= 3; ++f) {
    int layer = -1;
    for (int l = 0; l < p->L; ++l)
      if (p->fmt[l] == f) {
        if (layer < 0) layer = l;
        ++r.layers[f];
      }
    if (layer < 0) continue;
    const int64_t b = p->canon_bytes[f];
    r.expert_bytes[f] = double(b);
    // pinned host -> device
    hipError_t cerr = hipSuccess;
    if ((rc = timed([&]() {
           for (int e = 0; e < n; ++e) {
             const hipError_t ce =
                 hipMemcpyAsync(tmp + e * p->slot_bytes, p->host_store + p->key_off[int64_t(layer) * p->E + e],
                                size_t(b), hipMemcpyHostToDevice, s);
             if (cerr == hipSuccess) cerr = ce;
           }
         })))
      return rc;
    FT_HIP_CHECK(cerr);
    r.h2d_bytes_per_s[f] = double(n) * double(b) / sec;
    // the device's grouped FFN on the n experts, T rows each
    {
      std::vector<GroupDesc> g(n);
      std::vector<int32_t> rt(size_t(n) * T);
      std::vector<float> rw(size_t(n) * T, 1.0f);
      for (int e = 0; e < n; ++e) {
        g[e].wptr = reinterpret_cast<uint64_t>(tmp + e * p->slot_bytes);
        g[e].row_begin = e * T;
        g[e].row_count = T;
        g[e].expert = e;
        g[e].slot = -1;
        for (int t = 0; t < T; ++t) rt[size_t(e) * T + t] = t;
        for (int t = 0; t < kGroupTok; ++t) g[e].tok[t] = uint16_t(t < T ? t : 0);
      }
      FT_HIP_CHECK(hipMemcpy(p->gdesc, g.data(), g.size() * sizeof(GroupDesc), hipMemcpyHostToDevice));
      FT_HIP_CHECK(hipMemcpy(p->row_tok, rt.data(), rt.size() * 4, hipMemcpyHostToDevice));
      FT_HIP_CHECK(hipMemcpy(p->row_w, rw.data(), rw.size() * 4, hipMemcpyHostToDevice));
    }
    int frc = FT_OK;
    if ((rc = timed([&]() {
           if (frc == FT_OK) frc = run_ffn(p, layer, xd, 0, n, nullptr, s, n, double(n) * T, T);
         })))
      return rc;
    if (frc) return frc;
    r.gpu_bytes_per_s[f] = double(n) * double(b) / sec;
    // the host expert path on the same n experts, in one batched call as a
    // step's host-computed misses run
    {
      std::vector<uint16_t> x(size_t(T) * H, 0x3F80), o(size_t(n) * T * H);
      std::vector<float> w(T, 1.0f);
      if (!p->workers) p->workers = std::make_unique<WorkerPool>(p->cpu_threads);
      std::vector<HostExpertJob> jobs(n);
      for (int e = 0; e < n; ++e)
        jobs[e] = HostExpertJob{p->host_store + p->key_off[int64_t(layer) * p->E + e], x.data(), w.data(), T,
                                o.data() + size_t(e) * T * H};
      host_experts(p->lay[f], jobs.data(), n, *p->workers);  // warm-up
      const auto t0 = std::chrono::steady_clock::now();
      int it = 0;
      double el = 0.0;
      do {
        host_experts(p->lay[f], jobs.data(), n, *p->workers);
        ++it;
        el = std::chrono::duration<double>(std::chrono::steady_clock::now() - t0).count();
      } while (it < kReps && el < 0.25);
      r.cpu_bytes_per_s[f] = double(n) * double(b) * it / std::max(el, 1e-9);
    }
  }
  FT_HIP_CHECK(hipDeviceSynchronize());
  if ((rc = ft_moe_decide_mode(&r))) return rc;
  for (int f = 1; f <= 3; ++f) p->gpu_rate[f] = r.gpu_bytes_per_s[f];
  if (apply) {
    for (double& v : p->share_fmt) v = r.share;
    for (auto& o : p->obs) o = ft_moe_pool::Obs{};
  }
  *out = r;
  return FT_OK;
}

const char* ft_moe_ffn_kernel_name(int32_t stage) {
  if (stage == FT_STAGE_FFN_GATEUP) return ffn_last_kernel(true);
  if (stage == FT_STAGE_FFN_DOWN) return ffn_last_kernel(false);
  return "";
}

int ft_moe_set_profiling(ft_moe_pool* p, int32_t stage_mask) {
  if (!p) {
    set_error("NULL pool");
    return FT_E_INVALID;
  }
  p->prof_mask = stage_mask & ((1 << FT_STAGE_COUNT) - 1);
  return FT_OK;
}

int ft_moe_profile_read(ft_moe_pool* p, ft_moe_profile* out, int32_t reset) {
  if (!p || !out) {
    set_error("NULL pool or output");
    return FT_E_INVALID;
  }
  DeviceGuard dg(p->device);
  prof_drain(p, true);
  {
    // work of device-driven calls, counted by their resolve kernels
    uint64_t cnt[24];
    FT_HIP_CHECK(hipDeviceSynchronize());
    FT_HIP_CHECK(hipMemcpy(cnt, p->prof_cnt_dev, sizeof(cnt), hipMemcpyDeviceToHost));
    const double H = p->H, I = p->I;
    for (int f = 1; f <= 3; ++f) {
      double d[3][2];
      for (int st = 0; st < 3; ++st)
        for (int j = 0; j < 2; ++j) {
          const int i = (st * 4 + f) * 2 + j;
          d[st][j] = double(cnt[i] - p->prof_cnt_seen[i]);
          p->prof_cnt_seen[i] = cnt[i];
        }
      p->prof.bytes[FT_STAGE_FFN_GATEUP] += d[0][0] * 2 * mat_bytes(f, I, H) + d[0][1] * (H + I) * 2;
      p->prof.flops[FT_STAGE_FFN_GATEUP] += d[0][1] * 4 * H * I;
      p->prof.bytes[FT_STAGE_FFN_DOWN] += d[1][0] * mat_bytes(f, H, I) + d[1][1] * (I + H) * 2;
      p->prof.flops[FT_STAGE_FFN_DOWN] += d[1][1] * 2 * H * I;
      p->prof.bytes[FT_STAGE_COPY] += d[2][0] * double(p->canon_bytes[f]);
    }
  }
  *out = p->prof;
  if (reset) p->prof = ft_moe_profile{};
  return FT_OK;
}

int ft_moe_debug_read(ft_moe_pool* p, int32_t what, void* dst, int64_t bytes) {
  if (!p || !dst || bytes < 0) {
    set_error("need a pool, a destination and a byte count");
    return FT_E_INVALID;
  }
  const void* src = nullptr;
  int64_t cap = 0;
  if (what == FT_DBG_H_CODES) {
    src = p->hq_codes;
    cap = p->hq_codes ? p->hq_blocks * mx_tile_code_bytes(false) : 0;
  } else if (what == FT_DBG_H_SCALES) {
    src = p->hq_scales;
    cap = p->hq_scales ? p->hq_blocks * kMxTileScaleBytes : 0;
  } else if (what == FT_DBG_ROW_SLOT) {
    src = p->row_slot;
    cap = p->row_slot ? (int64_t(p->cap_T) * p->k + (p->shared ? p->cap_T : 0)) * 4 : 0;
  } else {
    set_error("unknown buffer %d", what);
    return FT_E_INVALID;
  }
  if (src == nullptr || bytes > cap) {
    set_error("buffer %d holds %lld bytes, %lld asked", what, (long long)cap, (long long)bytes);
    return FT_E_INVALID;
  }
  DeviceGuard dg(p->device);
  FT_HIP_CHECK(hipDeviceSynchronize());
  FT_HIP_CHECK(hipMemcpy(dst, src, size_t(bytes), hipMemcpyDeviceToHost));
  return FT_OK;
}

void ft_moe_destroy_pool(ft_moe_pool* p) {
  if (!p) return;
  DeviceGuard dg(p->device);
  (void)hipDeviceSynchronize();
  prof_drain(p, true);
  copy_drain(p, true);
  for (hipEvent_t e : p->prof_free) hipEventDestroy(e);
  hipFree(p->arena); hipFree(p->shared_dev); hipFree(p->router_dev);
  hipFree(p->tab.key2slot); hipFree(p->tab.slot_key); hipFree(p->tab.slot_last); hipFree(p->tab.lru[0]);
  hipFree(p->tab.lru[1]); hipFree(p->tab.lru_cur); hipFree(p->tab.clock); hipFree(p->tab.stats);
  hipFree(p->tab.min_gap);
  hipFree(p->z); hipFree(p->sel); hipFree(p->w); hipFree(p->gap); hipFree(p->pair_flag); hipFree(p->pair_slot);
  hipFree(p->pair_row); hipFree(p->row_tok); hipFree(p->row_w); hipFree(p->groups); hipFree(p->glist); hipFree(p->gdesc); hipFree(p->count_max);
  hipFree(p->dev_header); hipFree(p->hbuf); hipFree(p->pbuf); hipFree(p->fail_dev);
  hipFree(p->key_off_dev); hipFree(p->prof_cnt_dev); hipFree(p->copy_clk); hipFree(p->copy_ticks);
  hipFree(p->key_sum_dev); hipFree(p->bad_dev);
  hipFree(p->row_slot); hipFree(p->tiles); hipFree(p->xq_codes); hipFree(p->xq_scales);
  hipFree(p->tq_codes); hipFree(p->tq_scales);
  hipFree(p->hq_codes); hipFree(p->hq_scales);
  if (p->rb_host) hipHostFree(p->rb_host);
  if (p->x_host) hipHostFree(p->x_host);
  if (p->cpu_out) hipHostFree(p->cpu_out);
  if (p->host_store) hipHostFree(p->host_store);
  for (int c = 0; c < ft_moe_pool::kMaxCopyStreams; ++c) {
    if (p->copy[c]) hipStreamDestroy(p->copy[c]);
    if (p->ev_copy_done[c]) hipEventDestroy(p->ev_copy_done[c]);
  }
  for (hipEvent_t e : {p->ev_resolved, p->ev_copied, p->ev_sync, p->ev_cpu_copied, p->ev_done[0], p->ev_done[1],
                       p->ev_staged[0], p->ev_staged[1], p->ev_call_done})
    if (e) hipEventDestroy(e);
  delete p;
}

}  // extern "C"
