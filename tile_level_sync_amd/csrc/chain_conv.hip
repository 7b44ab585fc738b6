// Persistent conv-pair chain kernel: Z = ReLU(conv(X, Wa)) (producer tiles),
// Y = conv(Z, Wb) (consumer tiles), "same" 2-D convolutions (stride 1,
// 2 * pad = R - 1 = S - 1) computed as implicit GEMMs in one launch.
//
// Implicit GEMM (cuSync paper, section "Tile based Computations": libraries
// compute convolutions with their GeMM tiles): GEMM rows are output pixels
// m = (n, p, q) flattened over NHWC, columns are output channels, and the
// reduction index is (tap r*S + s, input channel c), which is exactly the row
// index of the RSCK filter viewed as a [R*S*Cin][K] matrix.  A K step of BK
// covers BK channels of one tap; its A chunk for pixel m is the 8-channel
// vector of input pixel (n, p + r - pad, q + s - pad), or zeros outside the
// image (an out-of-range buffer offset loads zeros).
//
// Dependencies (section "Synchronization Policies", Conv2DTileSync, in its
// halo-aware reading): consumer pixel tile i reads intermediate pixels whose
// flattened index lies within pad*Ww + pad of its own; it waits, before its
// first K step, for every producer tile of that range (all channel tiles).
//   Conv2DTileSync  flag per producer tile (epoch);
//   RowSync         counter per producer pixel tile (+1 per channel tile);
//   Sentinel        Z pre-filled with 0xFFFF, cached first loads and
//                   agent-coherent re-polls of sentinel chunks;
//   Serial          two stream-ordered launches.
#include "gemm_tile.h"
#include "sched.h"
#include "waits.h"

namespace tls {

// NHWC gather operand for the implicit GEMM.
template <class T, int AUX>
struct ConvRows {
  using Shape = T;
  static constexpr int NI = T::BM * T::CPA / T::NT;
  i32x4 rs;
  int32_t pq[NI];     // (p << 16) | q of the tile row's pixel, -1 past the last pixel
  uint32_t base[NI];  // element offset of the pixel's chunk: m * Cin + chunk * 8
  int32_t Hh, Ww, Cin, S, pad, cpt;
  // k / cpt and tap / S as a multiply and a shift: floor(k * (2^20 / d + 1) / 2^20)
  // equals floor(k / d) for every divisor up to 64 and k up to 7 * 7 * 64
  // (checked exhaustively), far beyond the K steps of a supported conv.
  uint32_t cpt_mul, s_mul;
  int32_t kt0;  // absolute K step of the loop's step 0 (K splits)
  __device__ __forceinline__ void init(const void* ptr, uint32_t bytes, int m0, int npix,
                                       int Hh_, int Ww_, int Cin_, int S_, int pad_) {
    rs = make_srd(ptr, bytes);
    Hh = Hh_;
    Ww = Ww_;
    Cin = Cin_;
    S = S_;
    pad = pad_;
    cpt = Cin_ / T::BK;
    cpt_mul = (1u << 20) / (uint32_t)cpt + 1u;
    s_mul = (1u << 20) / (uint32_t)S_ + 1u;
    kt0 = 0;
#pragma unroll
    for (int j = 0; j < NI; ++j) {
      const int P = dma_position<T::NW>(j);
      const int r = P / T::CPA, c = (P % T::CPA) ^ swz_a<T::CPA>(r);
      const int m = m0 + r;
      if (m < npix) {
        const int rem = m % (Hh_ * Ww_);
        pq[j] = ((rem / Ww_) << 16) | (rem % Ww_);
        base[j] = (uint32_t)(m * Cin_ + c * 8);
      } else {
        pq[j] = -1;
        base[j] = 0;
      }
    }
  }
  // Byte offset of chunk j at loop step ktl, or an offset past the buffer
  // (which loads zeros) where the tap falls outside the image.  The step's
  // tap and channel block are wave-uniform; the per-lane part is a select,
  // not a branch, so a step's loads stay in one basic block.
  __device__ __forceinline__ uint32_t offset(int j, int ktl) const {
    const uint32_t k = (uint32_t)(ktl + kt0);
    const uint32_t tap = (k * cpt_mul) >> 20, cb = k - tap * (uint32_t)cpt;
    const uint32_t r = (tap * s_mul) >> 20, sx = tap - r * (uint32_t)S;
    const int dy = (int)r - pad, dx = (int)sx - pad;
    const int shift = (dy * Ww + dx) * Cin + (int)cb * T::BK;
    const int v = pq[j];
    const int p = v >> 16, q = v & 0xFFFF;
    const bool ok = (v >= 0) & ((unsigned)(p + dy) < (unsigned)Hh) & ((unsigned)(q + dx) < (unsigned)Ww);
    const uint32_t o = (uint32_t)(((int)base[j] + shift) * 2);
    return ok ? o : 0x80000000u;
  }
  __device__ __forceinline__ void issue_one(int j, char* region, int kt) const {
    dma16<AUX>(rs, region + dma_block<T::NW>(j), offset(j, kt));
  }
  // The same chunk again, agent-coherent (misses any stale cached copy).
  __device__ __forceinline__ void repoll_one(int j, char* region, int kt) const {
    dma16<kAuxAgent>(rs, region + dma_block<T::NW>(j), offset(j, kt));
  }
  __device__ __forceinline__ void issue(char* region, int kt) const {
#pragma unroll
    for (int j = 0; j < NI; ++j) issue_one(j, region, kt);
  }
};

template <class T>
struct PlainConv : ConvRows<T, kAuxNone>, NoFix {};
template <class T>
using SentinelConv = SentinelFix<ConvRows<T, kAuxNone>>;

// Wait, before the first K step, for every producer tile of the halo range:
// wave 0 checks all the flags in parallel (lane l takes flags l, l+64, ...),
// then one acquire and the workgroup barrier.
struct HaloWait {
  const uint32_t* flags;  // tile flags (Conv2DTileSync) or row counters (RowSync)
  int lo, hi;             // producer pixel tiles of the halo range
  int nt1;                // producer channel tiles
  bool per_row;           // RowSync counters: one per pixel tile, target nt1
  uint32_t target;
  uint32_t limit;
  Ctl* ctl;
  uint32_t item;
  int* s_ok;
  bool light;  // light acquire (see acquire_after_poll)
  // Waits only before step 0 (the prologue): nothing left in the main loop.
  __device__ __forceinline__ bool all_ready() const { return true; }
  __device__ __forceinline__ bool before(int kt) {
    if (kt != 0) return true;
    if (threadIdx.x < 64) {
      const int lane = threadIdx.x;
      const int n = per_row ? (hi - lo + 1) : (hi - lo + 1) * nt1;
      const int ok = wave_wait_all(
                         [&]() {
                           bool mine = true;
                           for (int f = lane; f < n; f += 64) {
                             const uint32_t* fp =
                                 per_row ? flags + (lo + f) * kFlagStride
                                         : flags + ((lo + f / nt1) * nt1 + f % nt1) * kFlagStride;
                             mine = mine && reached(ld_relaxed_agent(fp), target);
                           }
                           return mine;
                         },
                         limit, ctl)
                         ? 1
                         : 0;
      if (lane == 0) {
        if (ok)
          acquire_after_poll(light);
        else
          record_timeout(ctl, item, 1u);
        *s_ok = ok;
      }
    }
    wg_barrier();
    return *s_ok != 0;
  }
};

template <int BM, int BN, int NS, int WM, int WN, int BK, bool BF16 = false>
struct ConvShapes {
  using T = TileShape<BM, BN, NS, BK, WM, WN, false, BF16>;
};

template <class T, int POL>
__device__ __forceinline__ void conv_producer(const ConvParams& p, char* smem, uint32_t item,
                                              uint32_t epoch, int* s_flag) {
  // Work item = (tile, K split); the K steps run over taps, then channel blocks.
  const uint32_t tile = item / (uint32_t)p.ks1;
  const int split = (int)(item % (uint32_t)p.ks1);
  const int tm = tile / p.nt1, tn = tile % p.nt1;
  const int m0 = tm * T::BM;
  const uint32_t col0 = tn * T::BN;
  const int KS = p.R * p.S * (p.C / T::BK) / p.ks1;
  const int kt0 = split * KS;
  PlainConv<T> al;
  al.init(p.X, (uint32_t)p.npix * p.C * 2u, m0, p.npix, p.Hh, p.Ww, p.C, p.S, p.pad);
  al.kt0 = kt0;
  RowMajorKN<T> bl;
  bl.init((const char*)p.Wa + (size_t)kt0 * T::BK * p.K * 2u,
          (uint32_t)(p.R * p.S * p.C - kt0 * T::BK) * p.K * 2u, col0, (uint32_t)p.K);
  NoWait w;
  Gemm<T> g;
  gemm_mainloop<T>(g, smem, KS, al, bl, w);
  if (p.ks1 > 1) {
    if ((int32_t)item == p.skip_producer) {  // this split never arrives (test knob)
      __syncthreads();
      return;
    }
    // Pixel tiles are full but the last: the plain partial offsets (fewer
    // registers, the occupancy of the two-stage 128 x 64 tile).
    if (!split_k_reduce<T, false>(g, p.part1, p.part1_bytes, tile, split, p.ks1,
                                  p.splitcnt + tile * kFlagStride, s_flag, T::BM))
      return;
  }
  debug_delay(item, p.delay);
  const bool skip = (int32_t)item == p.skip_producer;
  const auto zr = make_rsrc(p.Z, (uint32_t)p.npix * p.K * 2u);
  auto store = [&](int r, int c, u32x4 v) {
    if (POL == kSentinel && skip) return;  // leave the sentinel in place (test knob)
    publish16(zr, ((m0 + r) * (uint32_t)p.K + col0 + c) * 2u, v);
  };
  float* dbg = p.zdbg;
  auto dbgfn = [&](int r, int c, const float* v) {
    if (m0 + r >= p.npix) return;
    f32x4* d = reinterpret_cast<f32x4*>(dbg + (size_t)(m0 + r) * p.K + col0 + c);
    d[0] = f32x4{v[0], v[1], v[2], v[3]};
    d[1] = f32x4{v[4], v[5], v[6], v[7]};
  };
  // one epilogue per activation (a constant inside its chunk loop)
  switch (p.act) {
    case kGeluErf:
      gemm_epilogue<T, kGeluErf>(g, smem, p.act, 1.0f, store, dbgfn, dbg != nullptr);
      break;
    case kGeluTanh:
      gemm_epilogue<T, kGeluTanh>(g, smem, p.act, 1.0f, store, dbgfn, dbg != nullptr);
      break;
    case kRelu:
      gemm_epilogue<T, kRelu>(g, smem, p.act, 1.0f, store, dbgfn, dbg != nullptr);
      break;
    default:
      gemm_epilogue<T, kActNone>(g, smem, p.act, 1.0f, store, dbgfn, dbg != nullptr);
      break;
  }
  // Post (device-scope stores drained; the sentinel protocol posts nothing).
  drain_vmem();
  __syncthreads();
  if (threadIdx.x == 0 && !skip) {
    if constexpr (POL == kConvTileSync) {
      post_store(p.tileflags + tile * kFlagStride, epoch);
    } else if constexpr (POL == kRowSync) {
      post_add(p.rowcnt + tm * kFlagStride, 1u);
    }
  }
}

template <class T, int POL>
__device__ __forceinline__ void conv_consumer(const ConvParams& p, char* smem, uint32_t citem,
                                              uint32_t epoch, int* s_ok, uint64_t* s_tready) {
  const uint32_t tile = citem / (uint32_t)p.ks2;
  const int split = (int)(citem % (uint32_t)p.ks2);
  const int tm = tile / p.nt2, tn = tile % p.nt2;
  const int m0 = tm * T::BM;
  const uint32_t col0 = tn * T::BN;
  const uint32_t item = p.P + citem;
  const int KT = p.R * p.S * (p.K / T::BK) / p.ks2;
  const int kt0 = split * KT;
  RowMajorKN<T> bl;
  bl.init((const char*)p.Wb + (size_t)kt0 * T::BK * p.K * 2u,
          (uint32_t)(p.R * p.S * p.K - kt0 * T::BK) * p.K * 2u, col0, (uint32_t)p.K);
  const uint32_t zbytes = (uint32_t)p.npix * p.K * 2u;
  Gemm<T> g;
  bool ok = true;
  if constexpr (POL == kSentinel) {
    SentinelConv<T> al;
    al.init(p.Z, zbytes, m0, p.npix, p.Hh, p.Ww, p.K, p.S, p.pad);
    al.kt0 = kt0;
    al.limit = p.poll_limit;
    al.ctl = p.ctl;
    al.item = item;
    al.gave_up = false;
    NoWait w;
    ok = gemm_mainloop<T>(g, smem, KT, al, bl, w);
  } else {
    PlainConv<T> al;
    al.init(p.Z, zbytes, m0, p.npix, p.Hh, p.Ww, p.K, p.S, p.pad);
    al.kt0 = kt0;
    if constexpr (POL == kConvTileSync || POL == kRowSync) {
      int64_t lo, hi;
      conv_dep_range(tm, p.npix, p.Ww, T::BM, p.pad, &lo, &hi);
      HaloWait w{POL == kRowSync ? p.rowcnt : p.tileflags,
                 (int)lo,
                 (int)hi,
                 p.nt1,
                 POL == kRowSync,
                 POL == kRowSync ? (uint32_t)p.nt1 : epoch,
                 p.poll_limit,
                 p.ctl,
                 item,
                 s_ok,
                 p.light_acquire != 0};
      TracedWait<HaloWait> tw{w, s_tready};
      ok = gemm_mainloop<T>(g, smem, KT, al, bl, tw);
    } else {
      NoWait w;
      ok = gemm_mainloop<T>(g, smem, KT, al, bl, w);
    }
  }
  if (ok && p.ks2 > 1)
    ok = split_k_reduce<T, false>(g, p.part2, p.part2_bytes, tile, split, p.ks2,
                                  p.splitcnt + (p.P / p.ks1 + tile) * kFlagStride, s_ok, T::BM);
  if (ok) {
    const auto yr = make_rsrc(p.Y, (uint32_t)p.npix * p.K * 2u);
    auto store = [&](int r, int c, u32x4 v) {
      store_out16(yr, ((m0 + r) * (uint32_t)p.K + col0 + c) * 2u, v);
    };
    auto nodbg = [](int, int, const float*) {};
    gemm_epilogue<T>(g, smem, kActNone, 1.0f, store, nodbg, false);
  }
  __syncthreads();
}

// WPE > 0 asks the compiler to fit WPE waves per SIMD (registers within
// 512 / WPE per lane), for the configurations whose LDS footprint allows more
// workgroups per CU than their default register use would.
template <int BM, int BN, int NS, int WM, int WN, int BK, int WPE, int POL, bool BF16 = false>
__global__ void __launch_bounds__(64 * WM * WN)
    __attribute__((amdgpu_waves_per_eu(WPE > 0 ? WPE : 1))) conv_chain_kernel(ConvParams p) {
  using T = typename ConvShapes<BM, BN, NS, WM, WN, BK, BF16>::T;
  __shared__ __attribute__((aligned(1024))) char smem[T::SMEM];
  __shared__ uint32_t s_item;
  __shared__ int s_ok;
  __shared__ int s_last;
  __shared__ uint64_t s_tready;
  __shared__ int s_sweep;
  __shared__ uint32_t s_first[kNumQueues];
  const uint32_t epoch = p.ctl->epoch + 1u;
  const bool tracing = p.trace != nullptr;
  SchedState st;
  st.init(p.sp);
  bool first = true;
  for (;;) {
    if (threadIdx.x == 0) {
      int sweep;
      s_item = next_item(st, p.sp, p.first, first, &sweep);
      s_sweep = sweep;
    }
    first = false;
    __syncthreads();
    const uint32_t item = s_item;
    if (s_sweep) {
      __syncthreads();  // s_item read before the sweep reuses the shared state
      sweep_first(p.first, p.ctl, s_first, &s_last, [&](uint32_t it) {
        uint64_t ts = 0;
        if (tracing && threadIdx.x == 0) ts = now_rt();
        conv_producer<T, POL>(p, smem, it, epoch, &s_ok);
        if (tracing && threadIdx.x == 0 && it < p.trace_cap)
          p.trace[it] = TraceRec{it, (uint16_t)blockIdx.x, hw_location(), ts, ts, now_rt()};
      });
    }
    if (item == kNoItem) break;
    uint64_t t0 = 0;
    if (tracing && threadIdx.x == 0) s_tready = t0 = now_rt();
    if (item < p.P)
      conv_producer<T, POL>(p, smem, item, epoch, &s_ok);
    else
      conv_consumer<T, POL>(p, smem, item - p.P, epoch, &s_ok, tracing ? &s_tready : nullptr);
    if (tracing && threadIdx.x == 0 && item < p.trace_cap)
      p.trace[item] = TraceRec{item, (uint16_t)blockIdx.x, hw_location(), t0, s_tready, now_rt()};
  }
  if constexpr (POL == kSentinel) sentinel_refill(p.ctl, p.zfill, p.fill_bytes, &s_item);
  sched_finish(p.sp, &s_last, POL == kRowSync, p.rowcnt, p.mt, POL == kConvTileSync, epoch,
               p.splitcnt, (p.ks1 > 1 || p.ks2 > 1) ? (int)(p.P / p.ks1 + p.Cn / p.ks2) : 0);
}

#define TLS_CONV_CFGS(X)          \
  X(0, 128, 64, 3, 2, 2, 64, 0)   \
  X(1, 256, 64, 3, 4, 1, 64, 0)   \
  X(2, 128, 128, 3, 2, 2, 64, 0)  \
  X(3, 64, 64, 4, 2, 2, 64, 0)    \
  X(4, 128, 64, 2, 2, 2, 64, 0)   \
  X(5, 64, 64, 3, 2, 2, 64, 0)    \
  X(6, 64, 64, 2, 2, 2, 64, 0)    \
  X(7, 128, 128, 2, 2, 2, 64, 0)  \
  X(8, 128, 64, 3, 2, 2, 32, 4)   \
  X(9, 128, 64, 4, 2, 2, 32, 3)   \
  X(10, 64, 64, 4, 2, 2, 32, 4)

template <int BM, int BN, int NS, int WM, int WN, int BK, int WPE, bool BF16>
static hipError_t conv_launch_pol(const ConvParams& p, int policy, int grid, hipStream_t s) {
  const dim3 blk(64 * WM * WN);
  switch (policy) {
    case kSerial:
      hipLaunchKernelGGL((conv_chain_kernel<BM, BN, NS, WM, WN, BK, WPE, kSerial, BF16>), dim3(grid),
                         blk, 0, s, p);
      break;
    case kConvTileSync:
      hipLaunchKernelGGL((conv_chain_kernel<BM, BN, NS, WM, WN, BK, WPE, kConvTileSync, BF16>),
                         dim3(grid), blk, 0, s, p);
      break;
    case kRowSync:
      hipLaunchKernelGGL((conv_chain_kernel<BM, BN, NS, WM, WN, BK, WPE, kRowSync, BF16>), dim3(grid),
                         blk, 0, s, p);
      break;
    case kSentinel:
      hipLaunchKernelGGL((conv_chain_kernel<BM, BN, NS, WM, WN, BK, WPE, kSentinel, BF16>), dim3(grid),
                         blk, 0, s, p);
      break;
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

// bf16 instances exist for the automatic configurations (conv_auto_cfg).
#define TLS_CONV_BF16_CFGS(X)    \
  X(0, 128, 64, 3, 2, 2, 64, 0)  \
  X(3, 64, 64, 4, 2, 2, 64, 0)   \
  X(4, 128, 64, 2, 2, 2, 64, 0)  \
  X(9, 128, 64, 4, 2, 2, 32, 3)

bool conv_bf16_cfg(int cfg) {
  switch (cfg) {
#define X(i, bm, bn, ns, wm, wn, bk, wpe) \
  case i:                                 \
    return true;
    TLS_CONV_BF16_CFGS(X)
#undef X
    default:
      return false;
  }
}

hipError_t conv_launch(int cfg, const ConvParams& p, int policy, int grid, hipStream_t s) {
  if (p.bf16) {
    switch (cfg) {
#define X(i, bm, bn, ns, wm, wn, bk, wpe) \
  case i:                                 \
    return conv_launch_pol<bm, bn, ns, wm, wn, bk, wpe, true>(p, policy, grid, s);
      TLS_CONV_BF16_CFGS(X)
#undef X
      default:
        return hipErrorInvalidValue;
    }
  }
  switch (cfg) {
#define X(i, bm, bn, ns, wm, wn, bk, wpe) \
  case i:                                 \
    return conv_launch_pol<bm, bn, ns, wm, wn, bk, wpe, false>(p, policy, grid, s);
    TLS_CONV_CFGS(X)
#undef X
    default:
      return hipErrorInvalidValue;
  }
}

// Occupancy of a configuration: its fp16 RowSync instance stands for every
// policy and dtype (they share the LDS footprint and launch shape).
hipError_t conv_occupancy(int cfg, int* blocks) {
  switch (cfg) {
#define X(i, bm, bn, ns, wm, wn, bk, wpe)                                              \
  case i:                                                                              \
    return hipOccupancyMaxActiveBlocksPerMultiprocessor(                               \
        blocks, conv_chain_kernel<bm, bn, ns, wm, wn, bk, wpe, kRowSync>, 64 * wm * wn, 0);
    TLS_CONV_CFGS(X)
#undef X
    default:
      return hipErrorInvalidValue;
  }
}

}  // namespace tls
