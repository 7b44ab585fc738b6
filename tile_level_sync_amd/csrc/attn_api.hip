// C ABI of the attention-score chain: argument checks, workspace layout,
// scheduling and launches.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstring>
#include <vector>

#include "internal.h"
#include "runtime_internal.h"

namespace tls {

hipError_t attn_launch(const AttnParams& p, int policy, int grid, hipStream_t s);
hipError_t attn_occupancy(int, int* blocks);

namespace {

constexpr int kAttnOccKey = 300;
constexpr int kBM = 128, kBN = 128, kD = 128;

struct AttnLayout {
  size_t tileflags, order, sc, total;
};

// nflags: one readiness flag per (row block, key block) score tile.
AttnLayout attn_layout(int64_t rows_total, int64_t S, uint32_t nflags, uint32_t P, uint32_t C,
                       bool sc_in_ws) {
  AttnLayout L;
  (void)nflags;
  L.tileflags = kTileFlagOffset;
  L.order = kFixedBytes;
  L.sc = align_up(L.order + (size_t)(P + C) * 4, 256);
  L.total = align_up(L.sc + (sc_in_ws ? (size_t)rows_total * S * 2 : 0), 256);
  return L;
}

chain_status attn_check(const chain_attn_args* a) {
  if (!a || !a->Q || !a->K || !a->V || !a->O) return CHAIN_EINVAL;
  if (!aligned16(a->Q) || !aligned16(a->K) || !aligned16(a->V) || !aligned16(a->O))
    return CHAIN_EINVAL;
  if (a->s_out && !aligned16(a->s_out)) return CHAIN_EINVAL;
  if (a->B <= 0 || a->heads <= 0 || a->S <= 0 || a->d <= 0) return CHAIN_EINVAL;
  if (a->d != kD || a->S % kBM) return CHAIN_EUNSUPPORTED;
  const int64_t rows_total = (int64_t)a->B * a->heads * a->S;
  const int64_t lim = (int64_t)1 << 31;
  if (rows_total * a->S * 2 >= lim || rows_total * a->d * 2 >= lim) return CHAIN_EUNSUPPORTED;
  if (a->dtype != CHAIN_F16 && a->dtype != CHAIN_BF16) return CHAIN_EUNSUPPORTED;
  switch (a->policy) {
    case CHAIN_STREAM_SERIAL:
    case CHAIN_TILESYNC:
    case CHAIN_ROWSYNC:
    case CHAIN_SENTINEL:
      break;
    default:
      return CHAIN_EUNSUPPORTED;
  }
  if (a->order < CHAIN_ORDER_XCD || a->order > CHAIN_ORDER_STRIDED || a->order_stride < 0)
    return CHAIN_EINVAL;
  if (a->grid < 0 || a->debug_skip_producer < 0 || a->tile_cfg < 0 || a->tile_cfg > 1)
    return CHAIN_EINVAL;
  if (a->debug_first_skip < 0 || a->debug_first_skip > 1) return CHAIN_EINVAL;
  if (a->policy == CHAIN_TILESYNC && (rows_total / kBM) * (a->S / kBN) > (int64_t)kMaxTileFlags)
    return CHAIN_EUNSUPPORTED;
  if (a->policy == CHAIN_ROWSYNC && rows_total / kBM > (int64_t)kMaxRowCounters)
    return CHAIN_EUNSUPPORTED;
  if (a->trace && (!aligned16(a->trace) ||
                   (uint64_t)a->trace_capacity < 2u * (uint64_t)(rows_total / kBM)))
    return CHAIN_EINVAL;
  return ring_validate(a->s_ring, a->ring_slots, a->policy, a->s_out);
}

// Scheduler parameters and order table of a call.  The tile grid is
// (batch, head) pairs x row blocks of 128 queries, item = pair * S / 128 +
// block (the row block's index in the stacked rows).  The default order runs
// as one global counter over the rows: per-XCD queues (row slabs, and rows
// dealt round-robin alike) measured 5-15 % slower for every policy of this
// chain.
chain_status attn_sched_plan(const chain_attn_args* a, SchedParams* sp,
                             std::vector<uint32_t>* tab) {
  const int order = a->order == CHAIN_ORDER_XCD ? CHAIN_ORDER_ROW_MAJOR : a->order;
  const int pairs = a->B * a->heads, blocks = a->S / kBM;
  const int rows[2] = {pairs, pairs}, cols[2] = {blocks, blocks};
  return plan_sched_phases(sp, order, a->order_seed,
                           a->order_stride ? a->order_stride : kDefaultOrderStride, 2, rows,
                           cols, nullptr, true, a->policy == CHAIN_STREAM_SERIAL, nullptr, tab);
}

}  // namespace
}  // namespace tls

using namespace tls;

extern "C" {

size_t chain_attn_workspace_bytes(int B, int heads, int S, int d, int policy, int dtype,
                                  int tile_cfg) {
  (void)tile_cfg;
  chain_attn_args a;
  std::memset(&a, 0, sizeof(a));
  static const char dummy[16] __attribute__((aligned(16))) = {0};
  a.Q = a.K = a.V = dummy;
  a.O = (void*)dummy;
  a.B = B; a.heads = heads; a.S = S; a.d = d; a.policy = policy; a.dtype = dtype;
  if (attn_check(&a) != CHAIN_OK) return 0;
  const int64_t rows_total = (int64_t)B * heads * S;
  const uint32_t rows = (uint32_t)(rows_total / kBM), ntj = (uint32_t)(S / kBN);
  return attn_layout(rows_total, S, rows * ntj, rows, rows, true).total;
}

chain_status chain_attn_ex(const chain_attn_args* a) {
  chain_status st = attn_check(a);
  if (st != CHAIN_OK) return st;
  const hipStream_t stream = (hipStream_t)a->stream;
  const int64_t rows_total = (int64_t)a->B * a->heads * a->S;
  const int rows = (int)(rows_total / kBM), ntj = a->S / kBN;
  // Producer items are whole score rows (a row block against every key
  // block); consumer items are the same row blocks.
  const uint32_t P = (uint32_t)rows, C = (uint32_t)rows;

  int dev = 0;
  if ((st = current_device(&dev)) != CHAIN_OK) return st;
  int cus = 0;
  if ((st = device_cus(dev, &cus)) != CHAIN_OK) return st;
  // Every policy's kernel runs two workgroups per CU.
  const int kpol = a->policy;
  int occ = 0;
  if ((st = kernel_occupancy(dev, kAttnOccKey + kpol, attn_occupancy, kpol, &occ)) != CHAIN_OK)
    return st;
  if (occ <= 0) return CHAIN_EUNSUPPORTED;

  const AttnLayout L =
      attn_layout(rows_total, a->S, (uint32_t)rows * ntj, P, C,
                  a->s_out == nullptr && a->s_ring == nullptr);
  void* ws = a->workspace;
  if (ws) {
    if (!aligned16(ws)) return CHAIN_EINVAL;
    if (a->workspace_bytes < L.total) return CHAIN_ENOMEM;
  } else if ((st = library_workspace(dev, L.total, &ws)) != CHAIN_OK) {
    return st;
  }
  char* base = (char*)ws;

  AttnParams p;
  std::memset(&p, 0, sizeof(p));
  {
    std::vector<uint32_t> tab;
    if ((st = attn_sched_plan(a, &p.sp, &tab)) != CHAIN_OK) return st;
    if ((st = install_order(&p.sp, tab, ws, L.order, stream)) != CHAIN_OK) return st;
  }
  p.Q = a->Q;
  p.K = a->K;
  p.V = a->V;
  const size_t sbytes = (size_t)rows_total * a->S * 2;
  p.Sc = a->s_out ? a->s_out : (void*)(base + L.sc);
  bool prime = a->policy == CHAIN_SENTINEL;
  if (a->s_ring) {
    const RingPick r = ring_pick(a->s_ring, a->ring_slots, a->ring_index, sbytes);
    p.Sc = r.z;
    p.zfill = r.zfill;
    p.fill_bytes = r.fill_bytes;
    prime = r.prime;
  }
  p.O = a->O;
  p.B = a->B;
  p.heads = a->heads;
  p.S = a->S;
  p.d = a->d;
  p.scale = a->scale;
  p.rows = rows;
  p.ntj = ntj;
  p.trace = (TraceRec*)a->trace;
  p.trace_cap = a->trace ? a->trace_capacity : 0u;
  p.bf16 = a->dtype == CHAIN_BF16 ? 1 : 0;
  p.P = P;
  p.Cn = C;
  p.ctl = (Ctl*)base;
  p.tileflags = (uint32_t*)(base + L.tileflags);
  p.rowcnt = (uint32_t*)(base + kRowCntOffset);
  p.poll_limit = a->poll_limit ? a->poll_limit : kDefaultPollLimit;
  p.skip_producer = a->debug_skip_producer - 1;
  p.delay = a->debug_delay;
  // Whole 128-byte lines per tile (row strides are multiples of 128 bytes).
  p.light_acquire = ((uintptr_t)p.Sc % 128u) == 0 ? 1u : 0u;

  const int slots = cus * occ;
  if (prime) {  // a ring slot after the first was filled by the call before
    if ((st = fill_u32(p.Sc, 0xFFFFFFFFu, sbytes, stream)) != CHAIN_OK) return st;
  }
  // With the default order (the shared counter, no table) a launch's first
  // claims go through the eight per-XCD counters (FirstItems).
  const bool spread = p.sp.sched == 0 && p.sp.order == nullptr;
  const bool skip = a->debug_first_skip != 0;
  hipError_t e;
  if (a->policy == CHAIN_STREAM_SERIAL) {
    const int g1 = a->grid ? a->grid : std::min<int>((int)P, slots);
    set_first_items(&p.sp, &p.first, spread, g1, 0, P, P, skip);
    p.sp.first_phase = p.sp.last_phase = 0;
    e = attn_launch(p, kpol, g1, stream);
    if (e != hipSuccess) return hip_fail(e);
    set_first_items(&p.sp, &p.first, false, 0, P, P + C, P, skip);
    p.sp.first_phase = p.sp.last_phase = 1;
    e = attn_launch(p, kpol, a->grid ? a->grid : std::min<int>((int)C, slots), stream);
    if (e != hipSuccess) return hip_fail(e);
  } else {
    const int g = a->grid ? a->grid : std::min<int>((int)(P + C), slots);
    set_first_items(&p.sp, &p.first, spread, g, p.sp.t_begin, p.sp.t_end, P, skip);
    e = attn_launch(p, kpol, g, stream);
    if (e != hipSuccess) return hip_fail(e);
  }
  return finish_call(ws, stream);
}

chain_status chain_attn_order(const chain_attn_args* a, uint32_t* items, size_t capacity,
                              size_t* count) {
  if (!count) return CHAIN_EINVAL;
  chain_status st = attn_check(a);
  if (st != CHAIN_OK) return st;
  SchedParams sp;
  std::vector<uint32_t> tab, seq;
  if ((st = attn_sched_plan(a, &sp, &tab)) != CHAIN_OK) return st;
  order_sequence(sp, tab, &seq);
  return export_sequence(seq, items, capacity, count);
}

chain_status chain_attn(const void* Q, const void* K, const void* V, void* O, int B, int heads,
                        int S, int d, float scale, int policy) {
  chain_attn_args a;
  std::memset(&a, 0, sizeof(a));
  a.Q = Q; a.K = K; a.V = V; a.O = O;
  a.B = B; a.heads = heads; a.S = S; a.d = d; a.scale = scale; a.policy = policy;
  return chain_attn_ex(&a);
}

}  // extern "C"
