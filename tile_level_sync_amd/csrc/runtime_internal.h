// Host-side helpers shared by the runtime and the per-chain API files.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>
#include <initializer_list>
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

struct OrderGroup {
  uint32_t first;
  uint32_t count;
};
// Fisher-Yates shuffle of [first, last) with a splitmix64 stream.
void shuffle_range(std::vector<uint32_t>* v, size_t first, size_t last, uint64_t* state);
void build_order(const std::vector<OrderGroup>& groups, uint64_t seed,
                 std::vector<uint32_t>* out);
chain_status upload_order(void* ws, size_t offset, const std::vector<uint32_t>& order,
                          uint64_t key, hipStream_t stream);
uint64_t hash_words(std::initializer_list<uint64_t> w);

// Fill the scheduler parameters of a two-phase chain (mt row tiles, nt1
// producer and nt2 consumer column tiles) for the requested order; uploads an
// order table into the workspace at order_off when the order needs one.
// Producers of all queues precede every consumer in every order.
// Scheduler of an n-stage chain: phase ph has a rows[ph] x cols[ph] tile
// grid; items are numbered phase after phase.
chain_status setup_sched_phases(SchedParams* sp, int order_mode, uint64_t seed, int nphase,
                                const int* rows, const int* cols, const int* col_major,
                                bool slab_rows, void* ws, size_t order_off, hipStream_t stream,
                                uint64_t key_salt, bool separate_launches);
chain_status setup_sched(SchedParams* sp, int order_mode, uint64_t seed, int mt, int nt1,
                         int nt2, bool slab_rows, void* ws, size_t order_off,
                         hipStream_t stream, uint64_t key_salt, bool two_launches);

inline bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

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
