// Host-side helpers shared by the runtime and the per-chain API files.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>
#include <initializer_list>
#include <cstring>
#include <vector>

#include "../../include/tlsync.h"
#include "internal.h"

namespace tls {

chain_status hip_fail(hipError_t e);
chain_status current_device(int* dev);
chain_status device_cus(int dev, int* cus);
// Workgroups per CU of a kernel, cached per (device, key).
chain_status kernel_occupancy(int dev, int key, hipError_t (*query)(int, int*), int cfg,
                              int* occ);
chain_status library_workspace(int dev, size_t need, void** ws);
chain_status fill_u32(void* p, uint32_t v, size_t bytes, hipStream_t s);
chain_status read_status(void* ws, hipStream_t stream);
chain_status finish_call(void* ws, hipStream_t stream);
bool sync_mode();

// Fisher-Yates shuffle of [first, last) with a splitmix64 stream.
void shuffle_range(std::vector<uint32_t>* v, size_t first, size_t last, uint64_t* state);
chain_status upload_order(void* ws, size_t offset, const std::vector<uint32_t>& order,
                          uint64_t key, hipStream_t stream);
uint64_t hash_words(std::initializer_list<uint64_t> w);

// Scheduler of an n-stage chain: phase ph has a rows[ph] x cols[ph] tile
// grid; items are numbered phase after phase (base[ph] + r * cols[ph] + c).
// plan_sched_phases fills the parameters and, when the order needs one, the
// order table (host only, no device call); every order lists each consumer
// item after all producer items it reads.  dep_last (two-phase chains,
// optional) gives per consumer row the last producer row it reads (default:
// its own row); the interleaved order uses it.  stride is the column stride
// of CHAIN_ORDER_STRIDED.  setup_sched_phases also uploads the table into
// the workspace at order_off.
chain_status plan_sched_phases(SchedParams* sp, int order_mode, uint64_t seed, int stride,
                               int nphase, const int* rows, const int* cols, const int* col_major,
                               bool slab_rows, bool separate_launches, const int* dep_last,
                               std::vector<uint32_t>* table);
// Points sp at the workspace and uploads the order table (if any) to
// ws + order_off, skipping the copy when that table is already there.
chain_status install_order(SchedParams* sp, const std::vector<uint32_t>& tab, void* ws,
                           size_t order_off, hipStream_t stream);

// Items [begin, end) of one global-counter launch whose producer items end at
// P: with `on` (the default order, begin == 0) the first min(grid, P) items
// go out through the per-XCD counters (FirstItems, device side in sched.h)
// and the shared counter starts after them; otherwise plain [begin, end).
void set_first_items(SchedParams* sp, FirstItems* f, bool on, int grid, uint32_t begin,
                     uint32_t end, uint32_t P, bool skip);
chain_status setup_sched_phases(SchedParams* sp, int order_mode, uint64_t seed, int stride,
                                int nphase, const int* rows, const int* cols, const int* col_major,
                                bool slab_rows, void* ws, size_t order_off, hipStream_t stream,
                                bool separate_launches);
// The items in the order workgroups take them: the global sequence, or for
// per-XCD queues the queue lists, phase after phase.
void order_sequence(const SchedParams& sp, const std::vector<uint32_t>& tab,
                    std::vector<uint32_t>* seq);
// Copy a sequence to a caller array (count always set; items may be NULL to
// ask for the count; CHAIN_EINVAL if capacity is short).
chain_status export_sequence(const std::vector<uint32_t>& seq, uint32_t* items, size_t capacity,
                             size_t* count);

// Default column stride of CHAIN_ORDER_STRIDED.
constexpr int kDefaultOrderStride = 2;

inline bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

// Workspace bytes a chain_mlp_ex call with these arguments needs (the same
// checks as the call; no device call).
chain_status mlp_workspace_need(const chain_mlp_args* a, size_t* need);

// Sentinel ring of intermediate buffers (slots of slot_bytes back to back):
// argument checks (host only, before any device call) and, per call, the slot
// consumed, the slot refilled inside the launch and whether the consumed slot
// must first be filled on the stream (the ring's first call).
chain_status ring_validate(const void* ring, int slots, int policy, const void* out);
struct RingPick {
  void* z;
  void* zfill;
  uint32_t fill_bytes;
  bool prime;
};
RingPick ring_pick(void* ring, int slots, uint32_t index, size_t slot_bytes);

}  // namespace tls
