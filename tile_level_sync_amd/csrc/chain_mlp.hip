// Persistent MLP chain kernel: Z = act(X W1) (producer tiles), Y = Z W2
// (consumer tiles), both in one launch.
//
// Scheduling (cuSync paper, sections "Stage Processing Order" and "Tile
// Processing Order"): each workgroup repeatedly takes the next work item from
// a global atomic counter; items [0, P) are producer tiles and [P, P + C)
// consumer tiles, optionally permuted by an order table that keeps every
// consumer after all the producers it reads.  A consumer therefore only waits
// on tiles already taken by running workgroups, and producers never wait, so
// the chain cannot deadlock however many workgroups are resident.  This
// replaces the paper's wait-kernel, whose purpose was exactly this ordering.
//
// Policies (section "Synchronization Policies"):
//   TileSync  flag per producer tile, set to the call's epoch; a consumer
//             waits for flag (row, j) before its K loop enters column tile j.
//   RowSync   counter per producer row, +1 per finished tile; a consumer waits
//             once, before its first K step, for the whole row.
//   Sentinel  (sentinel guide, 4.6.4) Z was filled with 0xFFFF; the consumer
//             loads Z with agent-coherent loads and re-loads any 16-byte chunk
//             that still holds the sentinel.
//   Serial    two launches over [0, P) and [P, P + C) on one stream.
#include "gemm_tile.h"

namespace tls {

// Dense row-major A operand [rows][ld] (bytes past the buffer read as zero).
struct DenseA {
  __amdgpu_buffer_rsrc_t rs;
  uint32_t ld;    // elements
  uint32_t row0;  // first row of the tile
  __device__ __forceinline__ u32x4 load(int r, int kc, int kt) const {
    return bload16<kAuxNone>(rs, ((row0 + r) * ld + kt * 64 + kc) * 2u);
  }
  __device__ __forceinline__ void fix(u32x4*, int) const {}
};

// Sentinel A operand: agent-coherent loads, and every loaded chunk that still
// holds the sentinel is re-loaded (bounded by the poll limit; a watchdog
// expiry abandons the re-polls and reports a timeout).
template <int NCH>
struct SentinelA {
  __amdgpu_buffer_rsrc_t rs;
  uint32_t ld;
  uint32_t row0;
  uint32_t limit;
  Ctl* ctl;
  uint32_t item;
  bool gave_up;
  __device__ __forceinline__ u32x4 load(int r, int kc, int kt) const {
    return bload16<kAuxAgent>(rs, ((row0 + r) * ld + kt * 64 + kc) * 2u);
  }
  __device__ __forceinline__ void fix(u32x4* ra, int kt) {
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
      if (!has_sentinel16(ra[i]) || gave_up) continue;
      const int c = threadIdx.x + i * 256;
      for (uint32_t it = 0;; ++it) {
        if (it >= limit || ((it & 63u) == 63u && ld_relaxed_agent(&ctl->abort))) {
          gave_up = true;
          record_timeout(ctl, item, 1u);
          break;
        }
        __builtin_amdgcn_s_sleep(1);
        ra[i] = load(c >> 3, (c & 7) * 8, kt);
        if (!has_sentinel16(ra[i])) break;
      }
    }
  }
};

// Row-major [K][ld] B operand (the weights as written).
struct DenseB {
  __amdgpu_buffer_rsrc_t rs;
  uint32_t ld;    // elements (N of the product)
  uint32_t col0;  // first column of the tile
  __device__ __forceinline__ u32x4 load(int kr, int nc, int kt) const {
    return bload16<kAuxNone>(rs, ((kt * 64 + kr) * ld + col0 + nc) * 2u);
  }
};

struct TileSyncWait {
  const uint32_t* flags;  // first flag of the producer row
  int steps_per_tile;     // K steps per producer column tile
  uint32_t epoch;
  uint32_t limit;
  Ctl* ctl;
  uint32_t item;
  int* s_ok;
  __device__ __forceinline__ bool before(int kt) {
    if (kt % steps_per_tile) return true;
    return wg_wait(flags + (kt / steps_per_tile) * kFlagStride, epoch, limit, ctl, item, s_ok);
  }
};

struct RowSyncWait {
  const uint32_t* counter;
  uint32_t target;
  uint32_t limit;
  Ctl* ctl;
  uint32_t item;
  int* s_ok;
  __device__ __forceinline__ bool before(int kt) {
    if (kt != 0) return true;
    return wg_wait(counter, target, limit, ctl, item, s_ok);
  }
};

template <int BM, int BN1, int BN2>
struct MlpShapes {
  using T1 = TileShape<BM, BN1>;
  using T2 = TileShape<BM, BN2>;
  static constexpr int SMEM = T1::SMEM_HALFS > T2::SMEM_HALFS ? T1::SMEM_HALFS : T2::SMEM_HALFS;
};

template <class T>
__device__ __forceinline__ void mlp_producer(const MlpParams& p, f16* smem, uint32_t item,
                                             uint32_t epoch) {
  const int tm = item / p.nt1, tn = item % p.nt1;
  const uint32_t row0 = tm * T::BM, col0 = tn * T::BN;
  DenseA al{make_rsrc(p.X, (uint32_t)p.M * p.H * 2u), (uint32_t)p.H, row0};
  DenseB bl{make_rsrc(p.W1, (uint32_t)p.H * p.F * 2u), (uint32_t)p.F, col0};
  NoWait w;
  Gemm<T> g;
  gemm_mainloop<T>(g, smem, p.H / 64, al, bl, w);
  debug_delay(item, p.delay);
  const bool skip = (int32_t)item == p.skip_producer;
  auto zr = make_rsrc(p.Z, (uint32_t)p.M * p.F * 2u);
  auto store = [&](int r, int c, u32x4 v) {
    if (skip && p.policy == kSentinel) return;  // leave the sentinel in place (test knob)
    bstore16(zr, ((row0 + r) * (uint32_t)p.F + col0 + c) * 2u, v);
  };
  float* dbg = p.zdbg;
  auto dbgfn = [&](int r, int c, const float* v) {
    if (row0 + r >= (uint32_t)p.M) return;
    f32x4* d = reinterpret_cast<f32x4*>(dbg + (size_t)(row0 + r) * p.F + col0 + c);
    d[0] = f32x4{v[0], v[1], v[2], v[3]};
    d[1] = f32x4{v[4], v[5], v[6], v[7]};
  };
  gemm_epilogue<T>(g, smem, p.act, 1.0f, store, dbgfn, dbg != nullptr);
  // Post: all stores of the tile complete, then one release.
  drain_vmem();
  __syncthreads();
  if (threadIdx.x == 0 && !skip) {
    if (p.policy == kTileSync) {
      st_release_agent(p.tileflags + item * kFlagStride, epoch);
    } else if (p.policy == kRowSync) {
      add_release_agent(p.rowcnt + tm * kFlagStride, 1u);
    } else if (p.policy == kSentinel) {
      fence_release_agent();
    }
  }
}

template <class T, int BN1>
__device__ __forceinline__ void mlp_consumer(const MlpParams& p, f16* smem, uint32_t citem,
                                             uint32_t epoch, int* s_ok) {
  const int tm = citem / p.nt2, tn = citem % p.nt2;
  const uint32_t row0 = tm * T::BM, col0 = tn * T::BN;
  const uint32_t item = p.P + citem;
  DenseB bl{make_rsrc(p.W2, (uint32_t)p.F * p.H * 2u), (uint32_t)p.H, col0};
  const auto zr = make_rsrc(p.Z, (uint32_t)p.M * p.F * 2u);
  Gemm<T> g;
  bool ok = true;
  const int KT = p.F / 64;
  if (p.policy == kTileSync) {
    DenseA al{zr, (uint32_t)p.F, row0};
    TileSyncWait w{p.tileflags + (size_t)tm * p.nt1 * kFlagStride, BN1 / 64, epoch, p.poll_limit,
                   p.ctl, item, s_ok};
    ok = gemm_mainloop<T>(g, smem, KT, al, bl, w);
  } else if (p.policy == kRowSync) {
    DenseA al{zr, (uint32_t)p.F, row0};
    RowSyncWait w{p.rowcnt + (size_t)tm * kFlagStride, (uint32_t)p.nt1, p.poll_limit, p.ctl, item,
                  s_ok};
    ok = gemm_mainloop<T>(g, smem, KT, al, bl, w);
  } else if (p.policy == kSentinel) {
    SentinelA<T::A_CHUNKS> al{zr, (uint32_t)p.F, row0, p.poll_limit, p.ctl, item, false};
    NoWait w;
    ok = gemm_mainloop<T>(g, smem, KT, al, bl, w);
  } else {
    DenseA al{zr, (uint32_t)p.F, row0};
    NoWait w;
    ok = gemm_mainloop<T>(g, smem, KT, al, bl, w);
  }
  if (ok) {
    auto yr = make_rsrc(p.Y, (uint32_t)p.M * p.H * 2u);
    auto store = [&](int r, int c, u32x4 v) {
      bstore16(yr, ((row0 + r) * (uint32_t)p.H + col0 + c) * 2u, v);
    };
    auto nodbg = [](int, int, const float*) {};
    gemm_epilogue<T>(g, smem, kActNone, 1.0f, store, nodbg, false);
  }
  __syncthreads();  // LDS reuse by the next tile
}

template <int BM, int BN1, int BN2>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 2)))
mlp_chain_kernel(MlpParams p) {
  using S = MlpShapes<BM, BN1, BN2>;
  __shared__ __attribute__((aligned(16))) f16 smem[S::SMEM];
  __shared__ uint32_t s_item;
  __shared__ int s_ok;
  __shared__ int s_last;
  const uint32_t epoch = p.ctl->epoch + 1u;
  for (;;) {
    if (threadIdx.x == 0) {
      uint32_t t = p.t_begin + add_relaxed_agent(&p.ctl->work, 1u);
      if (t < p.t_end && ld_relaxed_agent(&p.ctl->abort)) t = p.t_end;
      s_item = t;
    }
    __syncthreads();
    const uint32_t t = s_item;
    if (t >= p.t_end) break;
    const uint32_t item = p.order ? p.order[t] : t;
    if (item < p.P)
      mlp_producer<typename S::T1>(p, smem, item, epoch);
    else
      mlp_consumer<typename S::T2, BN1>(p, smem, item - p.P, epoch, &s_ok);
  }
  // Exit: the last workgroup out resets the counters (and RowSync counters)
  // so the next launch starts from zero without a memset, and publishes the
  // epoch of a sync-policy call.
  if (threadIdx.x == 0) {
    const uint32_t d = add_relaxed_agent(&p.ctl->done, 1u);
    s_last = (d == gridDim.x - 1) ? 1 : 0;
  }
  __syncthreads();
  if (s_last) {
    fence_acquire_agent();
    if (p.policy == kRowSync) {
      for (int r = threadIdx.x; r < p.mt; r += blockDim.x) p.rowcnt[r * kFlagStride] = 0u;
    }
    if (threadIdx.x == 0) {
      p.ctl->work = 0u;
      p.ctl->done = 0u;
      p.ctl->abort = 0u;
      if (p.policy == kTileSync) p.ctl->epoch = epoch;
    }
  }
}

// ---------------------------------------------------------------------------
// Host-side launch helpers (one template instance per tile configuration).
// ---------------------------------------------------------------------------
template <int BM, int BN1, int BN2>
static hipError_t launch_cfg(const MlpParams& p, int grid, hipStream_t s) {
  hipLaunchKernelGGL((mlp_chain_kernel<BM, BN1, BN2>), dim3(grid), dim3(256), 0, s, p);
  return hipGetLastError();
}

template <int BM, int BN1, int BN2>
static hipError_t occ_cfg(int* blocks) {
  return hipOccupancyMaxActiveBlocksPerMultiprocessor(blocks, mlp_chain_kernel<BM, BN1, BN2>,
                                                      256, 0);
}

hipError_t mlp_launch(int cfg, const MlpParams& p, int grid, hipStream_t s) {
  switch (cfg) {
    case 0: return launch_cfg<64, 64, 64>(p, grid, s);
    case 1: return launch_cfg<128, 128, 128>(p, grid, s);
    case 2: return launch_cfg<256, 128, 128>(p, grid, s);
    case 3: return launch_cfg<128, 64, 64>(p, grid, s);
    case 4: return launch_cfg<64, 128, 128>(p, grid, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t mlp_occupancy(int cfg, int* blocks) {
  switch (cfg) {
    case 0: return occ_cfg<64, 64, 64>(blocks);
    case 1: return occ_cfg<128, 128, 128>(blocks);
    case 2: return occ_cfg<256, 128, 128>(blocks);
    case 3: return occ_cfg<128, 64, 64>(blocks);
    case 4: return occ_cfg<64, 128, 128>(blocks);
    default: return hipErrorInvalidValue;
  }
}

int mlp_lds_bytes(int cfg) {
  switch (cfg) {
    case 0: return MlpShapes<64, 64, 64>::SMEM * 2;
    case 1: return MlpShapes<128, 128, 128>::SMEM * 2;
    case 2: return MlpShapes<256, 128, 128>::SMEM * 2;
    case 3: return MlpShapes<128, 64, 64>::SMEM * 2;
    case 4: return MlpShapes<64, 128, 128>::SMEM * 2;
    default: return 0;
  }
}

}  // namespace tls
