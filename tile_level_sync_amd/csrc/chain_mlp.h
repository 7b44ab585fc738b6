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
//   TileSync  flag per producer tile, set to the call's epoch; before its K
//             loop enters producer column tile j, a consumer needs flag
//             (row, j).  Wave 0 scans the remaining flags of the row in
//             parallel and acquires once per newly ready run of tiles.
//   RowSync   counter per producer row, +1 per finished tile; a consumer waits
//             once, before its first K step, for the whole row.
//   Sentinel  (sentinel guide, 4.6.4) Z was filled with 0xFFFF; the consumer
//             checks every 16-byte chunk it loaded and re-loads (past the
//             caches) any chunk that still holds the sentinel.
//   Serial    two launches over [0, P) and [P, P + C) on one stream.
#pragma once
#include "gemm_tile.h"
#include "sched.h"
#include "waits.h"

namespace tls {

template <int BM, int BN1, int BN2, int BK, int NS, int WM, int WN, bool BF16 = false, int NSB = 0>
struct MlpShapes {
  using T1 = TileShape<BM, BN1, NS, BK, WM, WN, false, BF16, NSB>;
  using T2 = TileShape<BM, BN2, NS, BK, WM, WN, false, BF16, NSB>;
  static constexpr int NT = T1::NT;
  static constexpr int SMEM = T1::SMEM > T2::SMEM ? T1::SMEM : T2::SMEM;
};

template <class T, int POL>
__device__ __forceinline__ void mlp_producer(const MlpParams& p, char* smem, uint32_t item,
                                             uint32_t epoch, int* s_flag) {
  // Work item = (tile, K split); split s covers K steps [s*KS, (s+1)*KS).
  const uint32_t tile = item / (uint32_t)p.ks1;
  const int split = (int)(item % (uint32_t)p.ks1);
  const int tm = tile / p.nt1, tn = tile % p.nt1;
  const uint32_t row0 = tm * T::BM, col0 = tn * T::BN;
  const int KS = p.H / T::BK / p.ks1;
  const uint32_t k0 = (uint32_t)(split * KS * T::BK);  // first K element of the split
  PlainRows<T> al;
  al.init((const char*)p.X + k0 * 2u, (uint32_t)p.M * p.H * 2u - k0 * 2u, row0, (uint32_t)p.H);
  RowMajorKN<T> bl;
  bl.init((const char*)p.W1 + (size_t)k0 * p.F * 2u, (uint32_t)(p.H - k0) * p.F * 2u, col0,
          (uint32_t)p.F);
  NoWait w;
  Gemm<T> g;
  gemm_mainloop<T>(g, smem, KS, al, bl, w);
  const bool skip = (int32_t)item == p.skip_producer;
  if (p.ks1 > 1) {
    if (skip) {  // this split never arrives (test knob): the tile never completes
      __syncthreads();
      return;
    }
    if (!split_k_reduce<T>(g, p.part1, p.part1_bytes, tile, split, p.ks1, p.splitcnt + tile * kFlagStride,
                           s_flag, (uint32_t)p.M - row0))
      return;
  }
  debug_delay(item, p.delay);
  const auto zr = make_rsrc(p.Z, (uint32_t)p.M * p.F * 2u);
  auto store = [&](int r, int c, u32x4 v) {
    if (POL == kSentinel && skip) return;  // leave the sentinel in place (test knob)
    publish16(zr, ((row0 + r) * (uint32_t)p.F + col0 + c) * 2u, v);
  };
  float* dbg = p.zdbg;
  auto dbgfn = [&](int r, int c, const float* v) {
    if (row0 + r >= (uint32_t)p.M) return;
    f32x4* d = reinterpret_cast<f32x4*>(dbg + (size_t)(row0 + r) * p.F + col0 + c);
    d[0] = f32x4{v[0], v[1], v[2], v[3]};
    d[1] = f32x4{v[4], v[5], v[6], v[7]};
  };
  gemm_epilogue<T>(g, smem, p.act, 1.0f, store, dbgfn, dbg != nullptr);
  // Post: every wave's device-scope stores complete, then one lane posts.
  // Under the sentinel protocol the stored values are the signal.
  drain_vmem();
  __syncthreads();
  if (threadIdx.x == 0 && !skip) {
    if constexpr (POL == kTileSync) {
      post_store(p.tileflags + tile * kFlagStride, epoch);
    } else if constexpr (POL == kRowSync) {
      post_add(p.rowcnt + tm * kFlagStride, 1u);
    }
  }
}

template <class T, int BN1, int POL>
__device__ __forceinline__ void mlp_consumer(const MlpParams& p, char* smem, uint32_t citem,
                                             uint32_t epoch, int* s_ok, uint64_t* s_tready) {
  const uint32_t tile = citem / (uint32_t)p.ks2;
  const int split = (int)(citem % (uint32_t)p.ks2);
  const int tm = tile / p.nt2, tn = tile % p.nt2;
  const uint32_t row0 = tm * T::BM, col0 = tn * T::BN;
  const uint32_t item = p.P + citem;
  const int KS = p.F / T::BK / p.ks2;
  const int kt0 = split * KS;                       // first K step of the split
  const uint32_t k0 = (uint32_t)(kt0 * T::BK);
  RowMajorKN<T> bl;
  bl.init((const char*)p.W2 + (size_t)k0 * p.H * 2u, (uint32_t)(p.F - k0) * p.H * 2u, col0,
          (uint32_t)p.H);
  const char* zbase = (const char*)p.Z + k0 * 2u;
  const uint32_t zbytes = (uint32_t)p.M * p.F * 2u - k0 * 2u;
  Gemm<T> g;
  bool ok = true;
  const int KT = KS;
  if constexpr (POL == kTileSync && T::SPLIT_RING) {
    // The split-ring tile (256 x 192, the largest M) waits for every tile of
    // its row before step 0: a per-step wait in its main loop spilled and ran
    // behind the serialised launches.
    PlainRows<T> al;
    al.init(zbase, zbytes, row0, (uint32_t)p.F);
    TileRowWait w{p.tileflags + (size_t)tm * p.nt1 * kFlagStride, p.nt1, epoch, p.poll_limit,
                  p.ctl, item, s_ok, p.light_acquire != 0};
    TracedWait<TileRowWait> tw{w, s_tready};
    ok = gemm_mainloop<T>(g, smem, KT, al, bl, tw);
  } else if constexpr (POL == kTileSync) {
    PlainRows<T> al;
    al.init(zbase, zbytes, row0, (uint32_t)p.F);
    TileSyncWait w{p.tileflags + (size_t)tm * p.nt1 * kFlagStride, BN1 / T::BK, p.nt1, epoch,
                   p.poll_limit, p.ctl, item, s_ok, 0, p.light_acquire != 0, kt0};
    TracedWait<TileSyncWait> tw{w, s_tready};
    ok = gemm_mainloop<T>(g, smem, KT, al, bl, tw);
  } else if constexpr (POL == kRowSync) {
    PlainRows<T> al;
    al.init(zbase, zbytes, row0, (uint32_t)p.F);
    RowSyncWait w{p.rowcnt + (size_t)tm * kFlagStride, (uint32_t)p.nt1, p.poll_limit, p.ctl, item,
                  s_ok, p.light_acquire != 0};
    TracedWait<RowSyncWait> tw{w, s_tready};
    ok = gemm_mainloop<T>(g, smem, KT, al, bl, tw);
  } else if constexpr (POL == kSentinel) {
    SentinelRows<T> al;
    al.init(zbase, zbytes, row0, (uint32_t)p.F);
    al.limit = p.poll_limit;
    al.ctl = p.ctl;
    al.item = item;
    al.gave_up = false;
    NoWait w;
    ok = gemm_mainloop<T>(g, smem, KT, al, bl, w);
  } else {
    PlainRows<T> al;
    al.init(zbase, zbytes, row0, (uint32_t)p.F);
    NoWait w;
    ok = gemm_mainloop<T>(g, smem, KT, al, bl, w);
  }
  if (ok && p.ks2 > 1)
    ok = split_k_reduce<T>(g, p.part2, p.part2_bytes, tile, split, p.ks2,
                           p.splitcnt + (p.P / p.ks1 + tile) * kFlagStride, s_ok,
                           (uint32_t)p.M - row0);
  if (ok) {
    const auto yr = make_rsrc(p.Y, (uint32_t)p.M * p.H * 2u);
    auto store = [&](int r, int c, u32x4 v) {
      store_out16(yr, ((row0 + r) * (uint32_t)p.H + col0 + c) * 2u, v);
    };
    auto nodbg = [](int, int, const float*) {};
    gemm_epilogue<T>(g, smem, kActNone, 1.0f, store, nodbg, false);
  }
  __syncthreads();  // LDS reuse by the next tile
}

template <int BM, int BN1, int BN2, int BK, int NS, int WM, int WN, int POL, bool BF16 = false,
          int NSB = 0>
__global__ void __launch_bounds__(64 * WM * WN)
mlp_chain_kernel(MlpParams p) {
  using S = MlpShapes<BM, BN1, BN2, BK, NS, WM, WN, BF16, NSB>;
  __shared__ __attribute__((aligned(1024))) char smem[S::SMEM];
  __shared__ uint32_t s_item;
  __shared__ int s_ok;
  __shared__ int s_last;
  __shared__ uint64_t s_tready;
  const uint32_t epoch = p.ctl->epoch + 1u;
  const bool tracing = p.trace != nullptr;
  SchedState st;
  st.init(p.sp);
  for (;;) {
    if (threadIdx.x == 0) s_item = st.next(p.sp);
    __syncthreads();
    const uint32_t item = s_item;
    if (item == kNoItem) break;
    uint64_t t0 = 0;
    if (tracing && threadIdx.x == 0) s_tready = t0 = now_rt();
    if (item < p.P)
      mlp_producer<typename S::T1, POL>(p, smem, item, epoch, &s_ok);
    else
      mlp_consumer<typename S::T2, BN1, POL>(p, smem, item - p.P, epoch, &s_ok,
                                             tracing ? &s_tready : nullptr);
    if (tracing && threadIdx.x == 0 && item < p.trace_cap)
      p.trace[item] = TraceRec{item, (uint16_t)blockIdx.x, hw_location(), t0, s_tready, now_rt()};
  }
  if constexpr (POL == kSentinel) sentinel_refill(p.ctl, p.zfill, p.fill_bytes, &s_item);
  sched_finish(p.sp, &s_last, POL == kRowSync, p.rowcnt, p.mt, POL == kTileSync, epoch,
               p.splitcnt, (p.ks1 > 1 || p.ks2 > 1) ? (int)(p.P / p.ks1 + p.C / p.ks2) : 0);
}

// ---------------------------------------------------------------------------
// Tile configurations (the table mirrors kMlpCfgs) and the policy dispatch.
// ---------------------------------------------------------------------------
#define TLS_MLP_CFGS_A(X) \
  X(0, 64, 64, 64, 64, 4, 2, 2, 0) \
  X(1, 128, 128, 128, 64, 4, 2, 2, 0) \
  X(2, 256, 128, 128, 64, 3, 2, 2, 0) \
  X(3, 128, 64, 64, 64, 3, 2, 2, 0) \
  X(4, 64, 128, 128, 64, 3, 2, 2, 0) \
  X(5, 256, 256, 256, 64, 2, 2, 2, 0) \
  X(6, 256, 128, 128, 64, 3, 4, 2, 0) \
  X(7, 128, 128, 128, 64, 4, 2, 4, 0) \
  X(8, 256, 192, 192, 64, 2, 2, 2, 0)

#define TLS_MLP_CFGS_B(X) \
  X(9, 128, 192, 192, 64, 3, 2, 2, 0) \
  X(10, 64, 192, 192, 64, 4, 2, 2, 0) \
  X(11, 128, 256, 256, 64, 3, 2, 2, 0) \
  X(12, 256, 192, 192, 64, 2, 4, 2, 0) \
  X(13, 256, 256, 256, 32, 4, 2, 4, 0) \
  X(14, 256, 192, 192, 32, 4, 2, 2, 0) \
  X(15, 128, 192, 192, 32, 5, 2, 2, 0) \
  X(16, 256, 256, 256, 32, 4, 2, 2, 0)

// 256 x 192 with the split ring (A three slots deep, B two: 144 KB of LDS).
#define TLS_MLP_CFGS_C(X) \
  X(17, 256, 192, 192, 64, 3, 2, 2, 2) \
  X(18, 256, 192, 192, 64, 3, 4, 2, 2)

#define TLS_MLP_CFGS(X) TLS_MLP_CFGS_A(X) TLS_MLP_CFGS_B(X) TLS_MLP_CFGS_C(X)

// bf16 instances exist for the configurations the automatic plan picks and
// their fallbacks (mlp_bf16_cfg tells the host which).
#define TLS_MLP_BF16_CFGS(X)           \
  X(0, 64, 64, 64, 64, 4, 2, 2, 0)        \
  X(1, 128, 128, 128, 64, 4, 2, 2, 0)     \
  X(6, 256, 128, 128, 64, 3, 4, 2, 0)     \
  X(7, 128, 128, 128, 64, 4, 2, 4, 0)     \
  X(9, 128, 192, 192, 64, 3, 2, 2, 0)     \
  X(12, 256, 192, 192, 64, 2, 4, 2, 0)    \
  X(17, 256, 192, 192, 64, 3, 2, 2, 2)

template <int BM, int BN1, int BN2, int BK, int NS, int WM, int WN, bool BF16, int NSB>
static hipError_t launch_pol(const MlpParams& p, int grid, hipStream_t s) {
  const dim3 blk(64 * WM * WN);
  switch (p.policy) {
    case kSerial:
      hipLaunchKernelGGL((mlp_chain_kernel<BM, BN1, BN2, BK, NS, WM, WN, kSerial, BF16, NSB>), dim3(grid), blk, 0, s, p);
      break;
    case kTileSync:
      hipLaunchKernelGGL((mlp_chain_kernel<BM, BN1, BN2, BK, NS, WM, WN, kTileSync, BF16, NSB>), dim3(grid), blk, 0, s, p);
      break;
    case kRowSync:
      hipLaunchKernelGGL((mlp_chain_kernel<BM, BN1, BN2, BK, NS, WM, WN, kRowSync, BF16, NSB>), dim3(grid), blk, 0, s, p);
      break;
    case kSentinel:
      hipLaunchKernelGGL((mlp_chain_kernel<BM, BN1, BN2, BK, NS, WM, WN, kSentinel, BF16, NSB>), dim3(grid), blk, 0, s, p);
      break;
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}


// Launch and occupancy entry points of one translation unit's instances.
#define TLS_MLP_UNIT(NAME, CFGS, BF16)                                                     \
  hipError_t mlp_launch_##NAME(int cfg, const MlpParams& p, int grid, hipStream_t s) {   \
    switch (cfg) {                                                                       \
      CFGS(TLS_MLP_UNIT_LAUNCH_CASE_##BF16)                                              \
      default:                                                                           \
        return hipErrorInvalidValue;                                                     \
    }                                                                                    \
  }                                                                                      \
  hipError_t mlp_occupancy_##NAME(int cfg, int* blocks) {                                \
    switch (cfg) {                                                                       \
      CFGS(TLS_MLP_UNIT_OCC_CASE_##BF16)                                                 \
      default:                                                                           \
        return hipErrorInvalidValue;                                                     \
    }                                                                                    \
  }
#define TLS_MLP_UNIT_LAUNCH_CASE_0(i, bm, bn1, bn2, bk, ns, wm, wn, nsb) \
  case i:                                                               \
    return launch_pol<bm, bn1, bn2, bk, ns, wm, wn, false, nsb>(p, grid, s);
#define TLS_MLP_UNIT_LAUNCH_CASE_1(i, bm, bn1, bn2, bk, ns, wm, wn, nsb) \
  case i:                                                               \
    return launch_pol<bm, bn1, bn2, bk, ns, wm, wn, true, nsb>(p, grid, s);
// Occupancy of a configuration: its RowSync instance stands for all policies
// (they share the LDS footprint and launch shape).
#define TLS_MLP_UNIT_OCC_CASE_0(i, bm, bn1, bn2, bk, ns, wm, wn, nsb)                      \
  case i:                                                                                 \
    return hipOccupancyMaxActiveBlocksPerMultiprocessor(                                  \
        blocks, mlp_chain_kernel<bm, bn1, bn2, bk, ns, wm, wn, kRowSync, false, nsb>,      \
        64 * wm * wn, 0);
#define TLS_MLP_UNIT_OCC_CASE_1(i, bm, bn1, bn2, bk, ns, wm, wn, nsb)                      \
  case i:                                                                                 \
    return hipOccupancyMaxActiveBlocksPerMultiprocessor(                                  \
        blocks, mlp_chain_kernel<bm, bn1, bn2, bk, ns, wm, wn, kRowSync, true, nsb>,       \
        64 * wm * wn, 0);

hipError_t mlp_launch_f16a(int cfg, const MlpParams& p, int grid, hipStream_t s);
hipError_t mlp_launch_f16b(int cfg, const MlpParams& p, int grid, hipStream_t s);
hipError_t mlp_launch_f16c(int cfg, const MlpParams& p, int grid, hipStream_t s);
hipError_t mlp_launch_bf16(int cfg, const MlpParams& p, int grid, hipStream_t s);
hipError_t mlp_occupancy_f16a(int cfg, int* blocks);
hipError_t mlp_occupancy_f16b(int cfg, int* blocks);
hipError_t mlp_occupancy_f16c(int cfg, int* blocks);
hipError_t mlp_occupancy_bf16(int cfg, int* blocks);

}  // namespace tls
