// Host runtime of the C ABI declared in include/tlsync.h: argument checks,
// tile-configuration choice, workspace management, work-order tables,
// launches (one persistent launch, or two stream-ordered launches for the
// serial baseline) and device status read-back.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cstdint>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <unordered_map>
#include <vector>

#include "../../include/tlsync.h"
#include "internal.h"
#include "runtime_internal.h"

namespace tls {

// ---------------------------------------------------------------------------
// Error bookkeeping.
// ---------------------------------------------------------------------------
static std::atomic<int> g_last_hip{0};
static std::atomic<int64_t> g_last_timeout_item{-1};
static std::atomic<int> g_last_timeout_kind{-1};

chain_status hip_fail(hipError_t e) {
  g_last_hip.store((int)e);
  (void)hipGetLastError();  // clear the sticky non-fatal error state
  return CHAIN_EHIP;
}

// ---------------------------------------------------------------------------
// Per-device state: CU count, occupancy per kernel, library-owned workspace.
// ---------------------------------------------------------------------------
struct DevState {
  bool init = false;
  int cus = 0;
  std::unordered_map<int, int> occ;  // kernel key -> workgroups per CU
  void* ws = nullptr;
  size_t ws_bytes = 0;
};

static std::mutex g_mu;
static std::vector<DevState> g_dev;
// Order table last uploaded into a workspace (keyed by the workspace base).
static std::unordered_map<uintptr_t, uint64_t> g_order_key;

chain_status current_device(int* dev) {
  hipError_t e = hipGetDevice(dev);
  if (e != hipSuccess) return hip_fail(e);
  return CHAIN_OK;
}

static DevState& dev_state(int dev) {
  if ((int)g_dev.size() <= dev) g_dev.resize(dev + 1);
  return g_dev[dev];
}

chain_status device_cus(int dev, int* cus) {
  std::lock_guard<std::mutex> lk(g_mu);
  DevState& d = dev_state(dev);
  if (!d.init) {
    int n = 0;
    hipError_t e = hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return hip_fail(e);
    d.cus = n;
    d.init = true;
  }
  *cus = d.cus;
  return CHAIN_OK;
}

chain_status kernel_occupancy(int dev, int key, hipError_t (*query)(int, int*), int cfg,
                              int* occ) {
  {
    std::lock_guard<std::mutex> lk(g_mu);
    DevState& d = dev_state(dev);
    auto it = d.occ.find(key);
    if (it != d.occ.end()) {
      *occ = it->second;
      return CHAIN_OK;
    }
  }
  int n = 0;
  hipError_t e = query(cfg, &n);
  if (e != hipSuccess) return hip_fail(e);
  std::lock_guard<std::mutex> lk(g_mu);
  dev_state(dev).occ[key] = n;
  *occ = n;
  return CHAIN_OK;
}

// Library-owned workspace of the current device, grown on demand and zeroed
// when (re)allocated.
chain_status library_workspace(int dev, size_t need, void** ws) {
  std::lock_guard<std::mutex> lk(g_mu);
  DevState& d = dev_state(dev);
  if (d.ws_bytes < need) {
    if (d.ws) {
      hipError_t e = hipDeviceSynchronize();
      if (e != hipSuccess) return hip_fail(e);
      e = hipFree(d.ws);
      g_order_key.erase((uintptr_t)d.ws);
      d.ws = nullptr;
      d.ws_bytes = 0;
      if (e != hipSuccess) return hip_fail(e);
    }
    const size_t bytes = align_up(std::max(need, (size_t)(8u << 20)), 1u << 20);
    void* p = nullptr;
    hipError_t e = hipMalloc(&p, bytes);
    if (e != hipSuccess) {
      (void)hipGetLastError();
      return CHAIN_ENOMEM;
    }
    e = hipMemset(p, 0, bytes);
    if (e == hipSuccess) e = hipDeviceSynchronize();
    if (e != hipSuccess) {
      (void)hipFree(p);
      return hip_fail(e);
    }
    d.ws = p;
    d.ws_bytes = bytes;
  }
  *ws = d.ws;
  return CHAIN_OK;
}

static void* library_workspace_if_any(int dev) {
  std::lock_guard<std::mutex> lk(g_mu);
  if ((int)g_dev.size() <= dev) return nullptr;
  return g_dev[dev].ws;
}

// ---------------------------------------------------------------------------
// Work orders.  Groups of items are listed in an order where every consumer
// follows all producers it reads (the condition for deadlock freedom of the
// persistent scheduler); a seed permutes items inside each group.
// ---------------------------------------------------------------------------
static uint64_t splitmix64(uint64_t& s) {
  uint64_t z = (s += 0x9E3779B97F4A7C15ull);
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

void shuffle_range(std::vector<uint32_t>* v, size_t first, size_t last, uint64_t* state) {
  for (size_t i = last; i > first + 1; --i) {
    const size_t j = first + (size_t)(splitmix64(*state) % (uint64_t)(i - first));
    std::swap((*v)[i - 1], (*v)[j]);
  }
}

chain_status upload_order(void* ws, size_t offset, const std::vector<uint32_t>& order,
                          uint64_t key, hipStream_t stream) {
  {
    std::lock_guard<std::mutex> lk(g_mu);
    auto it = g_order_key.find((uintptr_t)ws);
    if (it != g_order_key.end() && it->second == key) return CHAIN_OK;
  }
  // Ordered after earlier work on the stream, and complete before return so
  // the host vector may go away.
  hipError_t e = hipStreamSynchronize(stream);
  if (e == hipSuccess)
    e = hipMemcpy((char*)ws + offset, order.data(), order.size() * 4, hipMemcpyHostToDevice);
  if (e != hipSuccess) return hip_fail(e);
  std::lock_guard<std::mutex> lk(g_mu);
  g_order_key[(uintptr_t)ws] = key;
  return CHAIN_OK;
}

// Host mirror of the device slab order (sched.h): item i of queue q.
static uint32_t host_slab_item(const SchedParams& s, int ph, int q, uint32_t i) {
  const uint32_t nt = (uint32_t)s.cols[ph], nr = (uint32_t)s.rows[ph];
  uint32_t r, c;
  if (s.slab_rows) {
    const uint32_t r0 = slab_begin(q, nr), n = slab_begin(q + 1, nr) - r0;
    if (s.col_major[ph]) {
      c = i / n;
      r = r0 + i % n;
    } else {
      r = r0 + i / nt;
      c = i % nt;
    }
  } else {
    const uint32_t c0 = slab_begin(q, nt), nc = slab_begin(q + 1, nt) - c0;
    if (s.col_major[ph]) {
      c = c0 + i / nr;
      r = i % nr;
    } else {
      r = i / nc;
      c = c0 + i % nc;
    }
  }
  return s.base[ph] + r * nt + c;
}

// Items of one phase's tile grid in a global order (base + r * cols + c for
// row r, column c): row-major, column-major, or row-major with the columns of
// each row visited with a stride (c, c + s, c + 2s, ..., then c + 1, ...).
static void phase_items(const SchedParams& sp, int ph, int order_mode, int stride,
                        std::vector<uint32_t>* out) {
  const uint32_t nr = (uint32_t)sp.rows[ph], nc = (uint32_t)sp.cols[ph], b = sp.base[ph];
  if (order_mode == CHAIN_ORDER_COL_MAJOR) {
    for (uint32_t c = 0; c < nc; ++c)
      for (uint32_t r = 0; r < nr; ++r) out->push_back(b + r * nc + c);
    return;
  }
  const uint32_t s = order_mode == CHAIN_ORDER_STRIDED && stride > 1 ? (uint32_t)stride : 1u;
  for (uint32_t r = 0; r < nr; ++r)
    for (uint32_t j = 0; j < s; ++j)
      for (uint32_t c = j; c < nc; c += s) out->push_back(b + r * nc + c);
}

chain_status plan_sched_phases(SchedParams* sp, int order_mode, uint64_t seed, int stride,
                               int nphase, const int* rows, const int* cols, const int* col_major,
                               bool slab_rows, bool separate_launches, const int* dep_last,
                               std::vector<uint32_t>* tab) {
  std::memset(sp, 0, sizeof(*sp));
  tab->clear();
  uint32_t total = 0;
  for (int ph = 0; ph < nphase; ++ph) {
    sp->base[ph] = total;
    sp->rows[ph] = rows[ph];
    sp->cols[ph] = cols[ph];
    sp->col_major[ph] = col_major ? col_major[ph] : 0;
    total += (uint32_t)rows[ph] * (uint32_t)cols[ph];
  }
  sp->slab_rows = slab_rows ? 1 : 0;
  sp->first_phase = 0;
  sp->last_phase = nphase - 1;
  sp->t_begin = 0;
  sp->t_end = total;
  if (order_mode == CHAIN_ORDER_XCD) {
    sp->sched = 1;
    for (int ph = 0; ph < nphase; ++ph)
      for (int q = 0; q < kNumQueues; ++q)
        sp->qcount[ph][q] =
            slab_rows ? (slab_begin(q + 1, rows[ph]) - slab_begin(q, rows[ph])) * (uint32_t)cols[ph]
                      : (uint32_t)rows[ph] * (slab_begin(q + 1, cols[ph]) - slab_begin(q, cols[ph]));
    if (seed == 0) return CHAIN_OK;
    tab->reserve(total);
    uint64_t st = seed;
    for (int ph = 0; ph < nphase; ++ph)
      for (int q = 0; q < kNumQueues; ++q) {
        sp->qstart[ph][q] = (uint32_t)tab->size();
        const size_t first = tab->size();
        for (uint32_t i = 0; i < sp->qcount[ph][q]; ++i)
          tab->push_back(host_slab_item(*sp, ph, q, i));
        shuffle_range(tab, first, tab->size(), &st);
      }
    return CHAIN_OK;
  }
  sp->sched = 0;
  if (order_mode == CHAIN_ORDER_ROW_MAJOR && seed == 0) return CHAIN_OK;  // t itself
  // Groups of items in table order; a seed permutes the items inside each
  // group.  Every group of consumer items follows the producer items it reads.
  std::vector<size_t> ends;
  uint64_t st = seed;
  auto close_group = [&]() {
    const size_t first = ends.empty() ? 0 : ends.back();
    if (seed != 0) shuffle_range(tab, first, tab->size(), &st);
    ends.push_back(tab->size());
  };
  if (order_mode != CHAIN_ORDER_INTERLEAVED || separate_launches || nphase != 2) {
    // One group per phase (separate stream-ordered launches take their
    // phase's table positions, so the interleaved order falls back to this).
    const int mode = order_mode == CHAIN_ORDER_INTERLEAVED ? CHAIN_ORDER_ROW_MAJOR : order_mode;
    for (int ph = 0; ph < nphase; ++ph) {
      phase_items(*sp, ph, mode, stride, tab);
      close_group();
    }
    return CHAIN_OK;
  }
  // Interleaved: producer row r, then every consumer row whose last producer
  // row (dep_last, default its own row) is r - 1: one row of lag behind the
  // last producer row it reads, and rows whose dependencies end at the last
  // producer row come after it.  A consumer row is thus listed after every
  // producer row it depends on, whatever its halo, which keeps the chain
  // live with any number of resident workgroups.
  const int mt = rows[0], mc = rows[1];
  std::vector<std::vector<int>> after(mt);
  for (int c = 0; c < mc; ++c) {
    int last = dep_last ? dep_last[c] : c;
    last = std::min(std::max(last, 0), mt - 1);
    after[std::min(last + 1, mt - 1)].push_back(c);
  }
  for (int r = 0; r < mt; ++r) {
    for (int c = 0; c < cols[0]; ++c) tab->push_back(sp->base[0] + (uint32_t)(r * cols[0] + c));
    close_group();
    if (after[r].empty()) continue;
    for (int cr : after[r])
      for (int c = 0; c < cols[1]; ++c)
        tab->push_back(sp->base[1] + (uint32_t)(cr * cols[1] + c));
    close_group();
  }
  return CHAIN_OK;
}

void set_first_items(SchedParams* sp, FirstItems* f, bool on, int grid, uint32_t begin,
                     uint32_t end, uint32_t P, bool skip) {
  sp->t_begin = begin;
  sp->t_end = end;
  f->n = 0;
  f->base = begin;
  f->sweep_at = kNoItem;
  f->skip = skip ? 1u : 0u;
  if (!on || begin >= P || grid <= 0) return;
  f->n = std::min<uint32_t>((uint32_t)grid, P - begin);
  sp->t_begin = begin + f->n;
  f->sweep_at = P;
}

chain_status install_order(SchedParams* sp, const std::vector<uint32_t>& tab, void* ws,
                           size_t order_off, hipStream_t stream) {
  sp->ctl = (Ctl*)ws;
  sp->order = nullptr;
  if (tab.empty()) return CHAIN_OK;
  // The table's own contents key the upload: a workspace that already holds
  // this table at this offset is not written again.
  uint64_t key = hash_words({(uint64_t)order_off, (uint64_t)tab.size()});
  for (size_t i = 0; i < tab.size(); i += 2)
    key = hash_words({key, tab[i], i + 1 < tab.size() ? tab[i + 1] : 0u});
  chain_status st = upload_order(ws, order_off, tab, key, stream);
  if (st != CHAIN_OK) return st;
  sp->order = (const uint32_t*)((char*)ws + order_off);
  return CHAIN_OK;
}

chain_status setup_sched_phases(SchedParams* sp, int order_mode, uint64_t seed, int stride,
                                int nphase, const int* rows, const int* cols, const int* col_major,
                                bool slab_rows, void* ws, size_t order_off, hipStream_t stream,
                                bool separate_launches) {
  std::vector<uint32_t> tab;
  chain_status st = plan_sched_phases(sp, order_mode, seed, stride, nphase, rows, cols, col_major,
                                      slab_rows, separate_launches, nullptr, &tab);
  if (st != CHAIN_OK) return st;
  return install_order(sp, tab, ws, order_off, stream);
}

void order_sequence(const SchedParams& sp, const std::vector<uint32_t>& tab,
                    std::vector<uint32_t>* seq) {
  seq->clear();
  if (sp.sched) {
    for (int ph = sp.first_phase; ph <= sp.last_phase; ++ph)
      for (int q = 0; q < kNumQueues; ++q)
        for (uint32_t i = 0; i < sp.qcount[ph][q]; ++i)
          seq->push_back(tab.empty() ? host_slab_item(sp, ph, q, i) : tab[sp.qstart[ph][q] + i]);
    return;
  }
  for (uint32_t t = sp.t_begin; t < sp.t_end; ++t) seq->push_back(tab.empty() ? t : tab[t]);
}

chain_status export_sequence(const std::vector<uint32_t>& seq, uint32_t* items, size_t capacity,
                             size_t* count) {
  if (count) *count = seq.size();
  if (!items) return CHAIN_OK;
  if (capacity < seq.size()) return CHAIN_EINVAL;
  std::memcpy(items, seq.data(), seq.size() * sizeof(uint32_t));
  return CHAIN_OK;
}

uint64_t hash_words(std::initializer_list<uint64_t> w) {
  uint64_t h = 0x243F6A8885A308D3ull;
  for (uint64_t x : w) {
    h ^= x + 0x9E3779B97F4A7C15ull + (h << 6) + (h >> 2);
    h *= 0xff51afd7ed558ccdull;
  }
  return h;
}

chain_status ring_validate(const void* ring, int slots, int policy, const void* out) {
  if (!ring) return CHAIN_OK;
  if (policy != CHAIN_SENTINEL || out || !aligned16(ring)) return CHAIN_EINVAL;
  if (slots < 2 || slots > 16) return CHAIN_EINVAL;
  return CHAIN_OK;
}

RingPick ring_pick(void* ring, int slots, uint32_t index, size_t slot_bytes) {
  const uint32_t n = (uint32_t)slots;
  RingPick r;
  r.z = (char*)ring + (size_t)(index % n) * slot_bytes;
  r.zfill = (char*)ring + (size_t)((index + 1u) % n) * slot_bytes;
  r.fill_bytes = (uint32_t)slot_bytes;
  r.prime = index == 0;
  return r;
}

// ---------------------------------------------------------------------------
// Fill kernel for the sentinel: a plain kernel (not a memset node), so the
// call stays capturable in a HIP graph.
// ---------------------------------------------------------------------------
__global__ void fill_u32_kernel(uint32_t* p, uint32_t v, size_t n) {
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride) p[i] = v;
}

chain_status fill_u32(void* p, uint32_t v, size_t bytes, hipStream_t s) {
  const size_t n = bytes / 4;
  if (n == 0) return CHAIN_OK;
  const int blocks = (int)std::min<size_t>((n + 255) / 256, 4096);
  hipLaunchKernelGGL(fill_u32_kernel, dim3(blocks), dim3(256), 0, s, (uint32_t*)p, v, n);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return hip_fail(e);
  return CHAIN_OK;
}

// ---------------------------------------------------------------------------
// Status read-back.
// ---------------------------------------------------------------------------
chain_status read_status(void* ws, hipStream_t stream) {
  hipError_t e = hipStreamSynchronize(stream);
  if (e != hipSuccess) return hip_fail(e);
  if (!ws) return CHAIN_OK;
  Ctl host;
  e = hipMemcpy(&host, ws, sizeof(Ctl), hipMemcpyDeviceToHost);
  if (e != hipSuccess) return hip_fail(e);
  if (host.status == kStatusOk) return CHAIN_OK;
  g_last_timeout_item.store((int64_t)host.status_item);
  g_last_timeout_kind.store((int)host.status_kind);
  const uint32_t zero[4] = {0, 0, 0, 0};
  e = hipMemcpy((char*)ws + offsetof(Ctl, status), zero, sizeof(zero), hipMemcpyHostToDevice);
  if (e != hipSuccess) return hip_fail(e);
  return CHAIN_ETIMEOUT;
}

bool sync_mode() {
  static const bool on = [] {
    const char* v = std::getenv("TLSYNC_SYNC");
    return v && v[0] == '1';
  }();
  return on;
}

chain_status finish_call(void* ws, hipStream_t stream) {
  if (!sync_mode()) return CHAIN_OK;
  return read_status(ws, stream);
}

}  // namespace tls

using namespace tls;

// ===========================================================================
// C ABI
// ===========================================================================
extern "C" {

chain_status chain_trace_clock_khz(int* khz) {
  if (!khz) return CHAIN_EINVAL;
  int dev = 0;
  chain_status st = current_device(&dev);
  if (st != CHAIN_OK) return st;
  hipError_t e = hipDeviceGetAttribute(khz, hipDeviceAttributeWallClockRate, dev);
  return e == hipSuccess ? CHAIN_OK : hip_fail(e);
}

const char* chain_strerror(chain_status s) {
  switch (s) {
    case CHAIN_OK: return "success";
    case CHAIN_EINVAL: return "invalid argument (null or misaligned pointer, bad size)";
    case CHAIN_EUNSUPPORTED: return "unsupported shape, dtype or policy";
    case CHAIN_EHIP: return "HIP runtime error";
    case CHAIN_ETIMEOUT: return "a device wait exceeded its poll limit";
    case CHAIN_ENOMEM: return "workspace allocation failed or workspace too small";
    case CHAIN_ESCRATCH:
      return "the call needs more workspace than the static scratch array of the "
             "allocation-free entry point holds";
    default: return "unknown status";
  }
}

int chain_last_hip_error(void) { return g_last_hip.load(); }

chain_status chain_last_timeout(int64_t* item, int* kind) {
  const int64_t it = g_last_timeout_item.load();
  if (it < 0) return CHAIN_EINVAL;
  if (item) *item = it;
  if (kind) *kind = g_last_timeout_kind.load();
  return CHAIN_OK;
}

chain_status chain_workspace_reset(void* workspace, size_t bytes, void* stream) {
  if (!workspace || bytes < kFixedBytes) return CHAIN_EINVAL;
  // A fill kernel rather than a memset node, so the call may be captured
  // into a HIP graph and replayed.
  chain_status st = fill_u32(workspace, 0u, bytes & ~(size_t)3, (hipStream_t)stream);
  if (st != CHAIN_OK) return st;
  std::lock_guard<std::mutex> lk(g_mu);
  g_order_key.erase((uintptr_t)workspace);
  return CHAIN_OK;
}

chain_status chain_workspace_status(void* workspace, void* stream) {
  if (!workspace) return CHAIN_EINVAL;
  return read_status(workspace, (hipStream_t)stream);
}

chain_status chain_sync(void* stream) {
  int dev = 0;
  chain_status st = current_device(&dev);
  if (st != CHAIN_OK) return st;
  return read_status(library_workspace_if_any(dev), (hipStream_t)stream);
}

void chain_release(void) {
  std::lock_guard<std::mutex> lk(g_mu);
  int cur = 0;
  (void)hipGetDevice(&cur);
  for (size_t d = 0; d < g_dev.size(); ++d) {
    if (!g_dev[d].ws) continue;
    (void)hipSetDevice((int)d);
    (void)hipDeviceSynchronize();
    (void)hipFree(g_dev[d].ws);
    g_order_key.erase((uintptr_t)g_dev[d].ws);
    g_dev[d].ws = nullptr;
    g_dev[d].ws_bytes = 0;
  }
  (void)hipSetDevice(cur);
}

chain_status chain_wave_model(const int64_t* blocks, int n, int64_t slots, double* frac,
                              int64_t* serial_waves, double* fused_waves) {
  if (!blocks || n <= 0 || slots <= 0) return CHAIN_EINVAL;
  int64_t serial = 0, total = 0;
  for (int i = 0; i < n; ++i) {
    if (blocks[i] < 0) return CHAIN_EINVAL;
    if (frac) frac[i] = (double)blocks[i] / (double)slots;
    serial += (blocks[i] + slots - 1) / slots;
    total += blocks[i];
  }
  if (serial_waves) *serial_waves = serial;
  if (fused_waves) *fused_waves = (double)total / (double)slots;
  return CHAIN_OK;
}

}  // extern "C"
