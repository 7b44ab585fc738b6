// Persistent attention-score chain kernel, per (batch, head):
//   producer item, row block i:  Sc[i, j] = fp16(scale * Q_i K_j^T) for every key block j
//   consumer item, row block i:  O_i = softmax_rows(Sc[i, :]) V
// in one launch (cuSync paper, section "GPT Models", Fig. "Architecture of two
// building blocks of GPT models" (b), the dot-product/softmax kernel that
// depends on whole rows of the first product; RowSync in "Synchronization
// Policies").  Rows of all heads are stacked: Q, K, V, O are [B*heads*S, d]
// and Sc is [B*heads*S, S].
//
// The consumer streams its score rows in blocks of 64 keys together with the
// matching 64 rows of V through the LDS ring and keeps an online softmax:
// per query row a running maximum m and sum l; each block rescales the
// accumulator by exp(m_old - m_new).  It computes O^T = V^T P^T on the
// matrix cores, so every accumulator a lane holds belongs to the one query
// row whose scores that lane reads: the rescale needs no data exchange beyond
// the pair of lanes sharing a row.  Softmax arithmetic is fp32; P enters the
// MFMA in the storage type, fp16 or bf16 (values in [0, 1]).
#include "gemm_tile.h"
#include "sched.h"
#include "waits.h"

namespace tls {

constexpr int kAttnBM = 128;  // query rows per tile
constexpr int kAttnBN = 128;  // keys per producer tile
constexpr int kAttnD = 128;   // head dimension

// TileSync posts one flag per (row block, key block).
template <int POL>
constexpr bool kTileFlags = POL == kTileSync;

// The producer's LDS: a two-slot ring of half key blocks (128 keys x 64 of d,
// 16-bit) and, after it, the score epilogue's staging area.
constexpr int kAttnKSlot = kAttnBN * 64 * 2;  // half a key block: 128 keys x 64 of d, 16-bit

template <class T>
constexpr int attn_producer_smem() {
  return 2 * kAttnKSlot + T::EPI_BYTES;
}

template <int NSC, bool BF16 = false>
struct AttnShapes {
  // producer: Q rows x K rows (K^T read like A), K-loop over d
  using TP = TileShape<kAttnBM, kAttnBN, 2, 64, 2, 2, true, BF16>;
  // consumer stages: [128 rows x 64 keys] of Sc (A layout) and [64 keys x 128 d] of V (KN)
  using TC = TileShape<kAttnBM, kAttnD, NSC, 64, 2, 2, false, BF16>;
  static constexpr int SMEM = attn_producer_smem<TP>() > TC::SMEM ? attn_producer_smem<TP>() : TC::SMEM;
};

// Producer work item: one row block (128 queries of one head) against every
// key block, Sc[i, j] = fp16(scale * Q_i K_j^T) for j = 0 .. S/128 - 1.  Whole
// rows per item keep the number of posts at one per row for RowSync.  The
// query tile is read once per item into registers (each wave's A fragments
// for all of d: 64 registers per lane); the keys stream through a two-slot
// LDS ring of half key blocks (128 keys x 64 of d), loaded one step ahead,
// so a block's first half lands during the score epilogue of the block
// before, which stages through its own LDS area after the ring.  Under
// TileSync the flag of key block j is published at the second step of block
// j + 1: that step's wait covers every earlier memory operation of the wave
// (the device-scope score stores of block j included) and its barrier those
// of every wave, so the post needs no workgroup-wide drain.
template <class T>
__device__ __forceinline__ void attn_mfma(f32x16& acc, const f16x8& a, const f16x8& b) {
  if constexpr (T::BF16)
    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                  __builtin_bit_cast(bf16x8, b), acc, 0, 0, 0);
  else
    acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, acc, 0, 0, 0);
}

template <class T, int POL>
__device__ __forceinline__ void attn_producer(const AttnParams& p, char* smem, uint32_t row,
                                              uint32_t epoch) {
  static_assert(T::BM == kAttnBM && T::BN == kAttnBN && T::BK == 64 && T::B_NK,
                "producer tile: 128 queries x 128 keys, d in steps of 64, K rows as B");
  static_assert(T::EPI_BYTES >= (kAttnD / T::BK) * T::A_BYTES, "Q staged in the epilogue area");
  constexpr int KS = kAttnD / T::BK;  // d steps per key block
  constexpr int KK = T::BK / 16;      // MFMA k sub-steps per step
  using KRows = RowMajorRows<T, T::BN, kAuxNone>;
  constexpr int NI = KRows::NI;  // direct loads per thread per half block
  // Score stores per thread in one epilogue: the 128 x 128 16-bit tile in
  // 16-byte chunks.  A half block's keys were loaded before the previous
  // block's epilogue, so its wait may leave exactly these in flight.
  constexpr int kEpiStores = T::BM * T::BN * 2 / (T::NT * 16);
  static_assert(KS == 2 && kEpiStores == 8, "two half blocks per key block, 8 stores");
  const int nti = p.S / kAttnBM;
  const int bh = row / nti, ti = row % nti;
  const uint32_t qkv_bytes = (uint32_t)p.B * p.heads * p.S * p.d * 2u;
  const bool skip = (int32_t)row == p.skip_producer;
  const uint32_t sc_bytes = (uint32_t)p.B * p.heads * p.S * p.S * 2u;
  const auto sr = make_rsrc(p.Sc, sc_bytes);
  const uint32_t srow0 = (uint32_t)(bh * p.S + ti * kAttnBM);
  uint32_t* flags = p.tileflags + (size_t)row * p.ntj * kFlagStride;
  char* epi = smem + 2 * kAttnKSlot;  // the Q tile first, then the epilogue's staging
  PlainRows<T> al;
  al.init(p.Q, qkv_bytes, srow0, (uint32_t)p.d);
#pragma unroll
  for (int h = 0; h < KS; ++h) al.issue(epi + h * T::A_BYTES, h);
  // Keys of this head from its first row; half block s = (block s / 2, d half
  // s % 2) sits (s / 2) * 128 rows and (s % 2) * 64 elements further on.
  KRows bl;
  bl.init(p.K, qkv_bytes, (uint32_t)(bh * p.S), (uint32_t)p.d);
  const int nsteps = KS * p.ntj;
  auto issue_keys = [&](int s) {
    char* slot = smem + (s & 1) * kAttnKSlot;
    const uint32_t soff =
        (uint32_t)(s >> 1) * (uint32_t)kAttnBN * p.d * 2u + (uint32_t)(s & 1) * (T::BK * 2u);
#pragma unroll
    for (int q = 0; q < NI; ++q)
      dma16s<kAuxNone>(bl.rs, slot + dma_block<T::NW>(q), bl.voff[q], soff);
  };
  issue_keys(0);
  wait_vmcnt<NI>();  // the Q tile landed; the first keys may still be in flight
  wg_barrier();
  Gemm<T> g;
  f16x8 aq[KS * KK][T::FM];
  {
    f16x8 unused[T::FN];
#pragma unroll
    for (int h = 0; h < KS; ++h)
#pragma unroll
      for (int kk = 0; kk < KK; ++kk)
        g.template read_frags<0>(epi + h * T::A_BYTES, nullptr, kk, aq[h * KK + kk], unused);
  }
  g.zero();
  auto nodbg = [](int, int, const float*) {};
  // Key block j in two steps, half h of d each (h is a constant, so the Q
  // fragments of the half stay registers, not an indexed stack array).
  for (int j = 0; j < p.ntj; ++j) {
#pragma unroll
    for (int h = 0; h < KS; ++h) {
      const int s = KS * j + h;
      if (h == 0 && j > 0)
        wait_vmcnt<kEpiStores>();  // this step's keys (issued before the stores)
      else
        wait_vmcnt<0>();
      // Every wave's keys of step s landed and every wave finished reading
      // the slot step s + 1 fills (step s - 1's), and at s = 0 its Q fragments.
      wg_barrier();
      if constexpr (kTileFlags<POL>) {
        if (h == 1 && j > 0 && threadIdx.x == 0 && !skip)
          post_store(flags + (j - 1) * kFlagStride, epoch);
      }
      if (s + 1 < nsteps) issue_keys(s + 1);
      const char* sb = smem + h * kAttnKSlot;
      f16x8 b[2][T::FN];
      f16x8 unused[T::FM];
      g.template read_frags<1>(nullptr, sb, 0, unused, b[0]);
#pragma unroll
      for (int kk = 0; kk < KK; ++kk) {
        if (kk + 1 < KK) g.template read_frags<1>(nullptr, sb, kk + 1, unused, b[(kk + 1) & 1]);
#pragma unroll
        for (int fm = 0; fm < T::FM; ++fm)
#pragma unroll
          for (int fn = 0; fn < T::FN; ++fn)
            attn_mfma<T>(g.acc[fm][fn], aq[h * KK + kk][fm], b[kk & 1][fn]);
      }
    }
    debug_delay(row * p.ntj + j, p.delay);
    const uint32_t scol0 = (uint32_t)(j * kAttnBN);
    auto store = [&](int r, int c, u32x4 v) {
      // Device-scope stores: the scores go through to the level every XCD
      // reads, so a drained relaxed post publishes them.  The sentinel test
      // knob leaves the sentinel in place by storing past the buffer
      // (dropped), which keeps the count of stores the waits rely on.
      const bool keep = POL == kSentinel && skip;
      publish16(sr, keep ? sc_bytes : ((srow0 + r) * (uint32_t)p.S + scol0 + c) * 2u, v);
    };
    gemm_epilogue<T>(g, epi, kActNone, p.scale, store, nodbg, false);
    g.zero();
  }
  drain_vmem();
  __syncthreads();
  if (threadIdx.x == 0 && !skip) {
    if constexpr (kTileFlags<POL>) {
      post_store(flags + (p.ntj - 1) * kFlagStride, epoch);
    } else if constexpr (POL == kRowSync) {
      post_add(p.rowcnt + row * kFlagStride, 1u);
    }
  }
}

// Online-softmax P.V over the stages of one consumer row block.
template <class T>
struct AttnConsumerStep {
  f32x16 acc[kAttnD / 32];  // O^T blocks: d rows fm*32.., query columns of this wave
  float m, l;               // running max / partial sum of this lane's query row
  __device__ __forceinline__ void init() {
#pragma unroll
    for (int i = 0; i < kAttnD / 32; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][r] = 0.0f;
    m = -__builtin_inff();
    l = 0.0f;
  }
  template <class LOADS>
  __device__ __forceinline__ void operator()(char* cur, int, LOADS& loads) {
    loads.all();
    constexpr float kLog2e = 1.4426950408889634f;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const char* sS = cur;
    const char* sV = cur + T::A_BYTES;
    // This lane's scores: query row wave*32 + (lane & 31), keys 16kk + 8*(lane>>5) + 0..7.
    const int fa = swz_a<8>(lane & 15);
    const char* arow = sS + (wave * 32 + (lane & 31)) * 128;
    f16x8 sv[4];
#pragma unroll
    for (int kk = 0; kk < 4; ++kk)
      sv[kk] = *reinterpret_cast<const f16x8*>(arow + (((kk * 2 + (lane >> 5)) ^ fa) * 16));
    // The scores as fp32 (bf16: the stored 16 bits are the upper half of the
    // fp32 pattern; whole-vector casts, see the compiler note in gemm_tile.h).
    float sf[4][8];
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      if constexpr (T::BF16) {
        const u16x8 b = __builtin_bit_cast(u16x8, sv[kk]);
#pragma unroll
        for (int e = 0; e < 8; ++e) sf[kk][e] = __builtin_bit_cast(float, (uint32_t)b[e] << 16);
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) sf[kk][e] = (float)sv[kk][e];
      }
    }
    float bmax = -__builtin_inff();
#pragma unroll
    for (int kk = 0; kk < 4; ++kk)
#pragma unroll
      for (int e = 0; e < 8; ++e) bmax = fmaxf(bmax, sf[kk][e]);
    bmax = fmaxf(bmax, __shfl_xor(bmax, 32));
    const float mnew = fmaxf(m, bmax);
    const float alpha = exp2f((m - mnew) * kLog2e);
    l *= alpha;
#pragma unroll
    for (int i = 0; i < kAttnD / 32; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][r] *= alpha;
    m = mnew;
    // P enters the MFMA in the storage type (fp16 or bf16, values in [0, 1]);
    // l sums the rounded values, so the normalisation matches what was used.
    f16x8 pf[4];
    u16x8 pb[4];
#pragma unroll
    for (int kk = 0; kk < 4; ++kk)
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float pv = exp2f((sf[kk][e] - mnew) * kLog2e);
        if constexpr (T::BF16) {
          const uint16_t h = f32_to_bf16_canon(pv);
          l += __builtin_bit_cast(float, (uint32_t)h << 16);
          pb[kk][e] = h;
        } else {
          const f16 ph = (f16)pv;
          l += (float)ph;
          pf[kk][e] = ph;
        }
      }
    // A = V^T fragments through the transposing read of the KN-staged V.
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      const int g = lane >> 4, i = lane & 15;
      const int k = kk * 16 + (g >> 1) * 8 + (i >> 2);
#pragma unroll
      for (int fm = 0; fm < kAttnD / 32; ++fm) {
        const int n = fm * 32 + (g & 1) * 16 + (i & 3) * 4;
        const int off = k * (kAttnD * 2) + (((n >> 3) ^ swz_b<kAttnD / 8>(k)) * 16) + (n & 7) * 2;
        fp16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4f16((TLS_LDS_AS fp16x4*)(sV + off));
        fp16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4f16(
            (TLS_LDS_AS fp16x4*)(sV + off + 4 * kAttnD * 2));
        if constexpr (T::BF16) {
          // the transposing read moves 16-bit patterns: bf16 V as it is stored
          const u16x4 l4 = __builtin_bit_cast(u16x4, lo), h4 = __builtin_bit_cast(u16x4, hi);
          const u16x8 a16 = {l4[0], l4[1], l4[2], l4[3], h4[0], h4[1], h4[2], h4[3]};
          acc[fm] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
              __builtin_bit_cast(bf16x8, a16), __builtin_bit_cast(bf16x8, pb[kk]), acc[fm], 0,
              0, 0);
        } else {
          f16x8 a;
          a[0] = (f16)lo[0]; a[1] = (f16)lo[1]; a[2] = (f16)lo[2]; a[3] = (f16)lo[3];
          a[4] = (f16)hi[0]; a[5] = (f16)hi[1]; a[6] = (f16)hi[2]; a[7] = (f16)hi[3];
          acc[fm] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, pf[kk], acc[fm], 0, 0, 0);
        }
      }
    }
  }
};

// Consumer row block: online softmax over the stored score rows with the
// matching V rows, then O (normalised once) to HBM.  `W` is the dependency
// waiter (NoWait, RowSyncWait, TileRowWait); the sentinel protocol checks
// the scores themselves (SentinelRows).
template <class T, bool SENTINEL, class W>
__device__ __forceinline__ void attn_consumer_body(const AttnParams& p, char* smem, uint32_t row,
                                                   W& w0, uint64_t* s_tready) {
  TracedWait<W> w{w0, s_tready};
  const int nti = p.S / kAttnBM;
  const int bh = row / nti, ti = row % nti;
  const uint32_t item = p.P + row;
  const uint32_t sc_bytes = (uint32_t)p.B * p.heads * p.S * p.S * 2u;
  const uint32_t srow0 = (uint32_t)(bh * p.S + ti * kAttnBM);
  RowMajorKN<T> bl;  // V rows of this head: [S keys][d]
  bl.init((const char*)p.V + (size_t)bh * p.S * p.d * 2, (uint32_t)p.S * p.d * 2u, 0u,
          (uint32_t)p.d);
  const int KT = p.S / T::BK;
  AttnConsumerStep<T> cs;
  cs.init();
  bool ok;
  if constexpr (SENTINEL) {
    SentinelRows<T> al;
    al.init(p.Sc, sc_bytes, srow0, (uint32_t)p.S);
    al.limit = p.poll_limit;
    al.ctl = p.ctl;
    al.item = item;
    al.gave_up = false;
    ok = pipeline<T>(smem, KT, al, bl, w, cs);
  } else {
    PlainRows<T> al;
    al.init(p.Sc, sc_bytes, srow0, (uint32_t)p.S);
    ok = pipeline<T>(smem, KT, al, bl, w, cs);
  }
  if (ok) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const float lt = cs.l + __shfl_xor(cs.l, 32);
    const float inv = 1.0f / lt;
    const auto orr = make_rsrc(p.O, (uint32_t)p.B * p.heads * p.S * p.d * 2u);
    const uint32_t orow = srow0 + wave * 32 + (lane & 31);
#pragma unroll
    for (int fm = 0; fm < kAttnD / 32; ++fm)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int d0 = fm * 32 + 8 * q + 4 * (lane >> 5);
        auto cvt = [](float v) -> uint32_t {
          if constexpr (T::BF16)
            return f32_to_bf16_canon(v);
          else
            return f32_to_f16_canon(v);
        };
        u32x2 o;
        o[0] = cvt(cs.acc[fm][4 * q + 0] * inv) | (cvt(cs.acc[fm][4 * q + 1] * inv) << 16);
        o[1] = cvt(cs.acc[fm][4 * q + 2] * inv) | (cvt(cs.acc[fm][4 * q + 3] * inv) << 16);
        store_out8(orr, (orow * (uint32_t)p.d + d0) * 2u, o);
      }
  }
}

template <class T, int POL>
__device__ __forceinline__ void attn_consumer(const AttnParams& p, char* smem, uint32_t row,
                                              uint32_t epoch, int* s_ok, uint64_t* s_tready) {
  if constexpr (POL == kSentinel) {
    NoWait w;  // no dependency wait: the trace's ready time stays the start
    attn_consumer_body<T, true>(p, smem, row, w, nullptr);
  } else if constexpr (POL == kTileSync) {
    // The consumer waits for the whole row before its loop: its softmax runs
    // over every key, and a wait before each key block inside that loop did
    // not fit beside the softmax state in 256 registers (it spilled in the
    // loop and ran behind the serialised launches).
    TileRowWait w{p.tileflags + (size_t)row * p.ntj * kFlagStride, p.ntj, epoch, p.poll_limit,
                  p.ctl, p.P + row, s_ok, p.light_acquire != 0};
    attn_consumer_body<T, false>(p, smem, row, w, s_tready);
  } else if constexpr (POL == kRowSync) {
    RowSyncWait w{p.rowcnt + (size_t)row * kFlagStride, 1u, p.poll_limit, p.ctl, p.P + row, s_ok,
                  p.light_acquire != 0};
    attn_consumer_body<T, false>(p, smem, row, w, s_tready);
  } else {
    NoWait w;
    attn_consumer_body<T, false>(p, smem, row, w, nullptr);
  }
  __syncthreads();
}

// Two workgroups of four waves per CU (at most 256 registers per lane).
template <int NSC, int POL, bool BF16 = false>
__global__ void __launch_bounds__(256, 2) attn_chain_kernel(AttnParams p) {
  using S = AttnShapes<NSC, BF16>;
  __shared__ __attribute__((aligned(1024))) char smem[S::SMEM];
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
        attn_producer<typename S::TP, POL>(p, smem, it, epoch);
        if (tracing && threadIdx.x == 0 && it < p.trace_cap)
          p.trace[it] = TraceRec{it, (uint16_t)blockIdx.x, hw_location(), ts, ts, now_rt()};
      });
    }
    if (item == kNoItem) break;
    uint64_t t0 = 0;
    if (tracing && threadIdx.x == 0) s_tready = t0 = now_rt();
    if (item < p.P)
      attn_producer<typename S::TP, POL>(p, smem, item, epoch);
    else
      attn_consumer<typename S::TC, POL>(p, smem, item - p.P, epoch, &s_ok,
                                         tracing ? &s_tready : nullptr);
    if (tracing && threadIdx.x == 0 && item < p.trace_cap)
      p.trace[item] = TraceRec{item, (uint16_t)blockIdx.x, hw_location(), t0, s_tready, now_rt()};
  }
  if constexpr (POL == kSentinel) sentinel_refill(p.ctl, p.zfill, p.fill_bytes, &s_item);
  sched_finish(p.sp, &s_last, POL == kRowSync, p.rowcnt, p.rows, kTileFlags<POL>, epoch);
}

constexpr int kAttnNSC = 2;

template <bool BF16>
static hipError_t attn_launch_t(const AttnParams& p, int policy, int grid, hipStream_t s) {
  switch (policy) {
    case kSerial:
      hipLaunchKernelGGL((attn_chain_kernel<kAttnNSC, kSerial, BF16>), dim3(grid), dim3(256), 0, s,
                         p);
      break;
    case kTileSync:
      hipLaunchKernelGGL((attn_chain_kernel<kAttnNSC, kTileSync, BF16>), dim3(grid), dim3(256), 0,
                         s, p);
      break;
    case kRowSync:
      hipLaunchKernelGGL((attn_chain_kernel<kAttnNSC, kRowSync, BF16>), dim3(grid), dim3(256), 0,
                         s, p);
      break;
    case kSentinel:
      hipLaunchKernelGGL((attn_chain_kernel<kAttnNSC, kSentinel, BF16>), dim3(grid), dim3(256), 0,
                         s, p);
      break;
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t attn_launch(const AttnParams& p, int policy, int grid, hipStream_t s) {
  return p.bf16 ? attn_launch_t<true>(p, policy, grid, s) : attn_launch_t<false>(p, policy, grid, s);
}

// Occupancy per policy: the fp16 instance stands for both element types (the
// same LDS footprint and launch bounds).
hipError_t attn_occupancy(int policy, int* blocks) {
  switch (policy) {
    case kSerial:
      return hipOccupancyMaxActiveBlocksPerMultiprocessor(
          blocks, attn_chain_kernel<kAttnNSC, kSerial>, 256, 0);
    case kTileSync:
      return hipOccupancyMaxActiveBlocksPerMultiprocessor(
          blocks, attn_chain_kernel<kAttnNSC, kTileSync>, 256, 0);
    case kRowSync:
      return hipOccupancyMaxActiveBlocksPerMultiprocessor(
          blocks, attn_chain_kernel<kAttnNSC, kRowSync>, 256, 0);
    case kSentinel:
      return hipOccupancyMaxActiveBlocksPerMultiprocessor(
          blocks, attn_chain_kernel<kAttnNSC, kSentinel>, 256, 0);
    default:
      return hipErrorInvalidValue;
  }
}

}  // namespace tls
