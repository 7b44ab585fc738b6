// MFMA tile engine for gfx950.  One workgroup (4 waves, 2 x 2) computes a
// BM x BN tile of C = A B with fp16 operands and fp32 accumulation.  Tiles
// follow the cuSync paper, section "Tile based Computations": tile C^{xy}
// multiplies BM rows of A with BN columns of B.
//
// Data movement: the K dimension is consumed in steps of 64 from a ring of
// NS LDS stages.  Operands travel global -> LDS with the gfx950 direct loads
// (buffer_load_dwordx4 ... lds: every lane moves 16 bytes and a wave fills
// 1 KiB of LDS contiguously), so no registers hold staged data and NS - 1
// steps are in flight while the matrix cores consume the current one.  Waits
// are explicit (s_waitcnt vmcnt(N)) and barriers are raw s_barrier, so the
// prefetches are never drained by a fence.
//
// LDS layouts (16-byte chunks, XOR-swizzled so the MFMA-pattern reads are
// bank-conflict free both with 128-byte and 256-byte LDS cycles):
//   A   [BM rows][BK/8 chunks]: chunk c of row r at r*(BK/8) + (c ^ fA(r))
//       (fA below); read with ds_read_b128.
//   B   "KN" (the weight layout as written, N contiguous) [64 k][BN/8]:
//       chunk c of row k at k*(BN/8) + (c ^ sB(k)); read with the transposing
//       ds_read_b64_tr_b16, which hands each lane 4 consecutive k of one
//       column.  "NK" (K contiguous, e.g. K^T of attention) is laid out and
//       read like A.
// MFMA: v_mfma_f32_32x32x16_f16, each wave owns a (BM/2) x (BN/2) block.
#pragma once

#include <type_traits>

#include "device.h"

namespace tls {

// Raw workgroup barrier: waits for this wave's LDS operations, not for its
// outstanding global loads (the prefetches stay in flight).
__device__ __forceinline__ void wg_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N <= 63, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

typedef int32_t i32x4 __attribute__((ext_vector_type(4)));

// Buffer descriptor in SGPRs for the inline-asm direct loads: raw buffer over
// [base, base + bytes), loads past the end return zero.
__device__ __forceinline__ i32x4 make_srd(const void* base, uint32_t bytes) {
  const uint64_t a = (uint64_t)(uintptr_t)base;
  i32x4 d;
  d[0] = __builtin_amdgcn_readfirstlane((int32_t)(uint32_t)a);
  d[1] = __builtin_amdgcn_readfirstlane((int32_t)(uint32_t)(a >> 32) & 0xFFFF);
  d[2] = __builtin_amdgcn_readfirstlane((int32_t)bytes);
  d[3] = 0x00020000;
  return d;
}

// One 16-byte-per-lane direct load into LDS at lds_wave_base + lane * 16.
// Written as inline asm on purpose: the compiler then neither counts it nor
// inserts a drain (s_waitcnt vmcnt(0)) before every LDS read that it cannot
// prove disjoint from the pending load; the explicit waits below own the
// ordering.  AUX = kAuxAgent makes the load agent-coherent (sc1).
// The LDS address for M0 is the low half of the generic pointer: a generic
// address into LDS is the shared aperture base (low 32 bits zero) plus the
// LDS offset, and the address-space cast adds only a null check, which would
// cost a compare and select before every load.  The base is wave-uniform
// (dma_block uses the scalar wave index), so no readfirstlane is emitted.
template <int AUX>
__device__ __forceinline__ void dma16(i32x4 srd, char* lds_wave_base, uint32_t voff) {
  const int32_t m0v = __builtin_amdgcn_readfirstlane((int32_t)(uint32_t)(uintptr_t)lds_wave_base);
  if constexpr (AUX == kAuxAgent) {
    asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen sc1 lds"
                 ::"s"(m0v), "v"(voff), "s"(srd)
                 : "memory");
  } else {
    asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
                 ::"s"(m0v), "v"(voff), "s"(srd)
                 : "memory");
  }
}

// The same with a wave-uniform byte offset soff in the instruction's scalar
// offset: a loader's per-step advance then costs no vector add per load.
// Only for loaders whose rows past the buffer end are decided by voff alone
// (the step advance stays inside every row, or inside the buffer): the
// buffer range check need not count the scalar offset.  A loader whose step
// advance itself walks past the end (the self-attention key rows past the
// last token) keeps dma16.
template <int AUX>
__device__ __forceinline__ void dma16s(i32x4 srd, char* lds_wave_base, uint32_t voff,
                                       uint32_t soff) {
  const int32_t m0v = __builtin_amdgcn_readfirstlane((int32_t)(uint32_t)(uintptr_t)lds_wave_base);
  const int32_t so = __builtin_amdgcn_readfirstlane((int32_t)soff);
  if constexpr (AUX == kAuxAgent) {
    asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, %3 offen sc1 lds"
                 ::"s"(m0v), "v"(voff), "s"(srd), "s"(so)
                 : "memory");
  } else {
    asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds"
                 ::"s"(m0v), "v"(voff), "s"(srd), "s"(so)
                 : "memory");
  }
}

// A-side swizzle of the 16-byte chunk index within a row of CPA chunks
// (CPA = BK / 8).  Conflict-free for ds_read_b128 of 8 or 16 consecutive
// rows at one chunk column.
template <int CPA>
__device__ __forceinline__ int swz_a(int r) {
  if constexpr (CPA == 8) {
    return (r & 7) ^ ((r >> 3) & 1);
  } else {
    return ((r >> 1) ^ (r >> 2)) & 3;
  }
}

template <int CPR>  // chunks per B row
__device__ __forceinline__ int swz_b(int k) {
  static_assert(CPR % 8 == 0, "B rows must hold a multiple of 8 chunks");
  if constexpr (CPR % 16 == 0) {
    return ((k & 3) << 2) | (k & 2);  // k & 3 = 0, 1, 2, 3 -> 0, 4, 10, 14
  } else {
    return 2 * (k & 3);  // stays inside each aligned group of 8 chunks (e.g. BN = 192)
  }
}

// NS is the depth of the A-operand ring; NSB_ (0 = NS) that of the B ring.
// With equal depths a stage holds A then B (one region per ring slot); with a
// shallower B ring the A slots come first, then the B slots, so that a tile
// whose two operands do not fit three stages deep can still run its A loads
// (the operand that comes from farther away) two steps ahead.
template <int BM_, int BN_, int NS_, int BK_ = 64, int WM_ = 2, int WN_ = 2, bool B_NK_ = false,
          bool BF16_ = false, int NSB_ = 0>
struct TileShape {
  static constexpr int BM = BM_, BN = BN_, BK = BK_, NS = NS_;
  static constexpr int NSB = NSB_ == 0 ? NS_ : NSB_;
  static constexpr bool SPLIT_RING = NSB != NS;
  // Operand element type: fp16, or bf16 (the MFMA and the epilogue's rounding
  // differ; loads, LDS layout and fragments only move 16-bit patterns).
  static constexpr bool BF16 = BF16_;
  static_assert(BK == 32 || BK == 64, "BK");
  static constexpr int CPA = BK / 8;                   // chunks per A (or NK B) row
  static constexpr int WM = WM_, WN = WN_;
  static constexpr int NW = WM * WN;                   // waves per workgroup
  static constexpr int NT = 64 * NW;
  static constexpr int WTM = BM / WM, WTN = BN / WN;
  static constexpr int FM = WTM / 32, FN = WTN / 32;
  static constexpr bool B_NK = B_NK_;
  static constexpr int CPR_B = BN / 8;                 // KN: chunks per B row
  static constexpr int A_BYTES = BM * BK * 2;
  static constexpr int B_BYTES = BK * BN * 2;
  static constexpr int STAGE = A_BYTES + B_BYTES;
  static constexpr int A_INSTR = A_BYTES / (NT * 16);  // direct loads per thread per stage
  static constexpr int B_INSTR = B_BYTES / (NT * 16);
  static constexpr int LOADS = A_INSTR + B_INSTR;
  // The MFMAs of each 16-wide k sub-step are issued in SPLIT groups; the
  // direct loads of the next stage are spread over the gaps between groups.
  static constexpr int SPLIT = ((FM * FN) % 2 == 0) ? 2 : 1;
  static constexpr int SLOTS = (BK / 16) * SPLIT;
  static constexpr int RING = SPLIT_RING ? NS * A_BYTES + NSB * B_BYTES : NS * STAGE;
  static constexpr int LDCF = BN + 4;                  // fp32 epilogue staging row stride
  static constexpr int EPI_PASSES = (BM * LDCF * 4 <= RING) ? 1 : WM;
  static constexpr int EPI_BYTES = (BM / EPI_PASSES) * LDCF * 4;
  static constexpr int SMEM = (RING > EPI_BYTES) ? RING : EPI_BYTES;
  static_assert(FM >= 1 && FN >= 1, "tile too small for the waves' 32x32 blocks");
  static_assert(A_INSTR >= 1 && B_INSTR >= 1, "tile too small for the direct loads");
  static_assert(A_BYTES % (NT * 16) == 0 && B_BYTES % (NT * 16) == 0, "load chunking");
  static_assert(NS >= 2 && (NS - 2) * LOADS <= 63, "stages vs vmcnt range");
  static_assert(!SPLIT_RING || (NS == 3 && NSB == 2), "split rings: A three deep, B two deep");
  // Byte offsets of ring slot s of each operand.
  static constexpr int a_off(int s) { return SPLIT_RING ? (s % NS) * A_BYTES : (s % NS) * STAGE; }
  static constexpr int b_off(int s) {
    return SPLIT_RING ? NS * A_BYTES + (s % NSB) * B_BYTES : (s % NS) * STAGE + A_BYTES;
  }
};

// Row / column of the element that accumulator register r of `lane` holds in
// a 32 x 32 MFMA block: rows advance in groups of 4 per half-wave.
__device__ __forceinline__ int acc_row(int lane, int r) {
  return 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
}
__device__ __forceinline__ int acc_col(int lane) { return lane & 31; }

// 16-byte chunk position filled by this lane's direct load j: instruction j
// of wave w covers positions (j*NW + w)*64 + lane of a stage region.
template <int NW>
__device__ __forceinline__ int dma_position(int j) {
  return (j * NW + (threadIdx.x >> 6)) * 64 + (threadIdx.x & 63);
}
// Wave index as a scalar (uniform by construction), so that addresses built
// from it stay in SGPRs.
__device__ __forceinline__ int wave_id() {
  return __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
}
template <int NW>
__device__ __forceinline__ int dma_block(int j) {
  return (j * NW + wave_id()) * 1024;
}

// Dense row-major operand whose rows are the tile's M (or N for NK) rows:
// element (row, k) at base + (row0 + row) * ld + k.  Rows past the buffer end
// read as zero (buffer range check).
template <class T, int ROWS, int AUX>
struct RowMajorRows {
  using Shape = T;
  static constexpr int NI = ROWS * T::CPA / (T::NT);  // instructions per thread
  i32x4 rs;
  uint32_t voff[NI];
  __device__ __forceinline__ void init(const void* base, uint32_t bytes, uint32_t row0,
                                       uint32_t ld) {
    rs = make_srd(base, bytes);
#pragma unroll
    for (int j = 0; j < NI; ++j) {
      const int P = dma_position<T::NW>(j);
      const int r = P / T::CPA, c = (P % T::CPA) ^ swz_a<T::CPA>(r);
      voff[j] = ((row0 + r) * ld + c * 8) * 2u;
    }
  }
  __device__ __forceinline__ void issue_one(int j, char* region, int kt) const {
    dma16s<AUX>(rs, region + dma_block<T::NW>(j), voff[j], kt * (uint32_t)(T::BK * 2));
  }
  // The same chunk again, agent-coherent (misses any stale cached copy).
  __device__ __forceinline__ void repoll_one(int j, char* region, int kt) const {
    dma16s<kAuxAgent>(rs, region + dma_block<T::NW>(j), voff[j], kt * (uint32_t)(T::BK * 2));
  }
  __device__ __forceinline__ void issue(char* region, int kt) const {
#pragma unroll
    for (int j = 0; j < NI; ++j) issue_one(j, region, kt);
  }
};

// Dense row-major [K][ld] operand (N contiguous), tile columns col0.
template <class T>
struct RowMajorKN {
  static constexpr int NI = T::B_INSTR;
  i32x4 rs;
  uint32_t voff[NI];
  uint32_t kstep;  // bytes per K step of 64 rows
  __device__ __forceinline__ void init(const void* base, uint32_t bytes, uint32_t col0,
                                       uint32_t ld) {
    rs = make_srd(base, bytes);
    kstep = (uint32_t)T::BK * ld * 2u;
#pragma unroll
    for (int j = 0; j < NI; ++j) {
      const int P = dma_position<T::NW>(j);
      const int k = P / T::CPR_B, c = (P % T::CPR_B) ^ swz_b<T::CPR_B>(k);
      voff[j] = (k * ld + col0 + c * 8) * 2u;
    }
  }
  __device__ __forceinline__ void issue_one(int j, char* region, int kt) const {
    dma16s<kAuxNone>(rs, region + dma_block<T::NW>(j), voff[j], kt * kstep);
  }
  __device__ __forceinline__ void issue(char* region, int kt) const {
#pragma unroll
    for (int j = 0; j < NI; ++j) issue_one(j, region, kt);
  }
};

// A operands with nothing to fix after landing.
struct NoFix {
  __device__ __forceinline__ void fix(char*, int) {}
};

// Loaders whose stage check can be split into an early read-back and a late
// test (SentinelFix) declare kEarlyFix.
template <class L, class = void>
struct HasEarlyFix {
  static constexpr bool value = false;
};
template <class L>
struct HasEarlyFix<L, decltype((void)L::kEarlyFix)> {
  static constexpr bool value = L::kEarlyFix;
};

// Sentinel handoff on top of a direct-load operand L (sentinel guide, 4.6.4.4
// Consumer Check, with a software per-element check): after a step has landed
// every lane re-reads the chunks it loaded and re-issues (for itself only) any
// chunk that still holds the sentinel, bounded by the poll limit; an expired
// wait is reported and the remaining re-polls of the workgroup are abandoned.
// The first load of a chunk is an ordinary cached load and only the re-polls
// are agent-coherent.  That is safe because every 16-byte chunk of the
// intermediate is written once, whole, with its final value, and the launch
// began with invalidated caches: a cached copy of a chunk holds either the
// sentinel (caught here, then re-read past the cache) or the final value.
template <class L>
struct SentinelFix : L {
  static constexpr bool kEarlyFix = true;
  uint32_t limit;
  Ctl* ctl;
  uint32_t item;
  bool gave_up;
  u32x4 early[L::NI];  // this lane's chunks of the next stage, read back early
  __device__ __forceinline__ const u32x4* chunk(const char* region, int j) const {
    return reinterpret_cast<const u32x4*>(region + dma_block<L::Shape::NW>(j) +
                                          (threadIdx.x & 63) * 16);
  }
  // Per-chunk re-poll of every chunk that still holds the sentinel.
  __device__ __forceinline__ void repoll(char* region, int kt) {
#pragma unroll
    for (int j = 0; j < L::NI; ++j) {
      const u32x4* mine = chunk(region, j);
      if (gave_up || !has_sentinel16(*mine)) continue;
      for (uint32_t it = 0;; ++it) {
        if (it >= limit || ((it & 63u) == 63u && ld_relaxed_agent(&ctl->abort))) {
          gave_up = true;
          record_timeout(ctl, item, 1u);
          break;
        }
        poll_pause(it);
        this->repoll_one(j, region, kt);
        wait_vmcnt<0>();
        if (!has_sentinel16(*mine)) break;
      }
    }
  }
  // Whole check at the stage boundary: all of this lane's chunks read back at
  // once, one wait, one test; the re-poll runs only if a sentinel is present.
  __device__ __forceinline__ void fix(char* region, int kt) {
    uint32_t m = 0;
#pragma unroll
    for (int j = 0; j < L::NI; ++j) m |= sentinel_bits(*chunk(region, j));
    if (__builtin_expect(m == 0u, 1) || gave_up) return;
    repoll(region, kt);
  }
  // The same check in two halves: fix_begin reads the chunks back once this
  // lane's loads of the stage have landed (while the MFMAs of the step
  // before still run), fix_end tests them at the boundary.  Nothing writes
  // the stage in between (its loads are complete, re-polls happen only in
  // fix_end), so the values are the ones fix would read.
  __device__ __forceinline__ void fix_begin(const char* region) {
#pragma unroll
    for (int j = 0; j < L::NI; ++j) early[j] = *chunk(region, j);
  }
  __device__ __forceinline__ void fix_end(char* region, int kt) {
    uint32_t m = 0;
#pragma unroll
    for (int j = 0; j < L::NI; ++j) m |= sentinel_bits(early[j]);
    if (__builtin_expect(m == 0u, 1) || gave_up) return;
    repoll(region, kt);
  }
};

template <class T>
struct Gemm {
  f32x16 acc[T::FM][T::FN];

  __device__ __forceinline__ void zero() {
#pragma unroll
    for (int i = 0; i < T::FM; ++i)
#pragma unroll
      for (int j = 0; j < T::FN; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;
  }

  // Fragments of one 16-wide k sub-step read from an LDS stage: PART 0 the
  // A fragments, PART 1 the B fragments, PART -1 both.
  template <int PART = -1>
  __device__ __forceinline__ void read_frags(const char* sa, const char* sb, int kk,
                                             f16x8 (&a)[T::FM], f16x8 (&b)[T::FN]) const {
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int wm = wave / T::WN, wn = wave % T::WN;
    // A: row r = wm*WTM + fm*32 + (lane & 31) -> r & 15 == lane & 15.
    constexpr int ROWB = T::BK * 2;  // bytes per A row in LDS
    const int fa = swz_a<T::CPA>(lane & 15);
    const int ca = ((kk * 2 + (lane >> 5)) ^ fa) * 16;
    if constexpr (PART != 1) {
      const char* arow = sa + (wm * T::WTM + (lane & 31)) * ROWB;
#pragma unroll
      for (int fm = 0; fm < T::FM; ++fm)
        a[fm] = *reinterpret_cast<const f16x8*>(arow + fm * 32 * ROWB + ca);
    }
    if constexpr (PART != 0) {
#pragma unroll
      for (int fn = 0; fn < T::FN; ++fn) {
        if constexpr (T::B_NK) {
          const char* brow = sb + (wn * T::WTN + fn * 32 + (lane & 31)) * ROWB;
          b[fn] = *reinterpret_cast<const f16x8*>(brow + ca);
        } else {
          // Transposing read: in each group of 16 lanes, lane (r, c) = 4r + c
          // names 4 consecutive halfs of k row r; lane j receives column j of
          // the 4 x 16 block.  Lanes 0-31 take k rows 0-7 of this 16-step,
          // lanes 32-63 rows 8-15; columns 0-15 / 16-31 by (lane >> 4) & 1.
          const int g = lane >> 4, i = lane & 15;
          const int k = kk * 16 + (g >> 1) * 8 + (i >> 2);
          const int n = wn * T::WTN + fn * 32 + (g & 1) * 16 + (i & 3) * 4;
          const int off = k * (T::BN * 2) + (((n >> 3) ^ swz_b<T::CPR_B>(k)) * 16) + (n & 7) * 2;
          const char* p0 = sb + off;
          const char* p1 = p0 + 4 * T::BN * 2;  // k + 4: same swizzle (k & 3 unchanged)
          fp16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4f16((TLS_LDS_AS fp16x4*)(p0));
          fp16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4f16((TLS_LDS_AS fp16x4*)(p1));
          f16x8 v;
          v[0] = (f16)lo[0]; v[1] = (f16)lo[1]; v[2] = (f16)lo[2]; v[3] = (f16)lo[3];
          v[4] = (f16)hi[0]; v[5] = (f16)hi[1]; v[6] = (f16)hi[2]; v[7] = (f16)hi[3];
          b[fn] = v;
        }
      }
    }
  }

  // One BK step of MFMAs from an LDS stage.  The fragments of sub-step 0 are
  // already in a[0], b[0]; those of sub-step kk+1 are read (into the other
  // buffer) while the MFMAs of sub-step kk run.  After each of the SPLIT MFMA
  // groups of a sub-step, `loads.slot(i)` issues its share of the next
  // stage's direct loads: spreading them keeps every wave's loads flowing
  // while the matrix cores work, instead of a burst that stalls the waves on a
  // full address queue at the top of each stage.  `boundary()` runs once the
  // last sub-step's MFMAs are issued: it crosses into the next stage (wait,
  // barrier, that stage's first fragments into a[0], b[0]) while those MFMAs
  // still execute.  BK / 16 is even, so sub-step 0 always uses buffer 0.
  template <class LOADS, class BOUNDARY>
  __device__ __forceinline__ void compute(const char* sa, const char* sb, LOADS& loads,
                                          f16x8 (&a)[2][T::FM], f16x8 (&b)[2][T::FN],
                                          BOUNDARY&& boundary) {
    constexpr int KK = T::BK / 16;
    static_assert(KK % 2 == 0, "fragment buffer parity across stages");
    constexpr int NMFMA = T::FM * T::FN;
    constexpr int G = NMFMA / T::SPLIT;
    constexpr int NRA = T::FM, NRB = T::B_NK ? T::FN : 2 * T::FN;  // LDS reads per part
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
      const int cur = kk & 1;
#pragma unroll
      for (int h = 0; h < T::SPLIT; ++h) {
        // The next sub-step's fragments: B during the first group, A during
        // the last (both in the single group when SPLIT = 1).  The next
        // sub-step's first group multiplies the first A fragments with every
        // B fragment, so B is read first and the A fragments in the order
        // they are used: each read then has a whole group of MFMAs to land.
        if (kk + 1 < KK) {
          if (T::SPLIT == 1) {
            read_frags(sa, sb, kk + 1, a[cur ^ 1], b[cur ^ 1]);
          } else if (h == 0) {
            read_frags<1>(sa, sb, kk + 1, a[cur ^ 1], b[cur ^ 1]);
          } else if (h == T::SPLIT - 1) {
            read_frags<0>(sa, sb, kk + 1, a[cur ^ 1], b[cur ^ 1]);
          }
        }
#pragma unroll
        for (int q = h * G; q < (h + 1) * G; ++q) {
          const int fm = q / T::FN, fn = q % T::FN;
          if constexpr (T::BF16)
            acc[fm][fn] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                __builtin_bit_cast(bf16x8, a[cur][fm]), __builtin_bit_cast(bf16x8, b[cur][fn]),
                acc[fm][fn], 0, 0, 0);
          else
            acc[fm][fn] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a[cur][fm], b[cur][fn],
                                                                 acc[fm][fn], 0, 0, 0);
        }
        if (kk + 1 < KK) {
          // one LDS read after each MFMA of the group, the rest at the end
          constexpr int NR = T::SPLIT == 1 ? NRA + NRB : 0;
          const int nr = T::SPLIT == 1 ? NR : (h == 0 ? NRB : (h == T::SPLIT - 1 ? NRA : 0));
#pragma unroll
          for (int i = 0; i < G; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
            if (i < nr) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // one LDS read
          }
#pragma unroll
          for (int i = G; i < nr; ++i) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        }
        loads.slot(kk * T::SPLIT + h);
        // Keep the scheduler from hoisting the next group's reads above this
        // point: that only lengthens live ranges (register spills) without
        // hiding more latency than the interleave above already does.
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    boundary();
  }
};

// Waiters: called uniformly by all threads before the A loads of step kt
// are issued; return false when a wait expired (the tile is abandoned).
// `all_ready()` says that no later step will wait (the main loop then runs
// without the wait's code in it).  A waiter that may wait at steps after the
// first declares `kStepWaits = true`.
struct NoWait {
  __device__ __forceinline__ bool all_ready() const { return true; }
  __device__ __forceinline__ bool before(int) { return true; }
};

template <class W, class = void>
struct StepWaits {
  static constexpr bool value = false;
};
template <class W>
struct StepWaits<W, decltype((void)W::kStepWaits)> {
  static constexpr bool value = W::kStepWaits;
};

// s_waitcnt vmcnt(n) for an n that is a constant after unrolling.
template <int I = 0>
__device__ __forceinline__ void wait_vmcnt_n(int n) {
  if constexpr (I <= 63) {
    if (n == I) {
      wait_vmcnt<I>();
      return;
    }
    wait_vmcnt_n<I + 1>(n);
  }
}

template <class T, int I = 0>
__device__ __forceinline__ void wait_stage(int later) {
  if constexpr (I <= T::NS - 2) {
    if (later == I) {
      wait_vmcnt<I * T::LOADS>();
      return;
    }
    wait_stage<T, I + 1>(later);
  }
}

// The direct loads of one future stage, B then A.  `slot(i)` issues the loads
// that fall into slot i of T::SLOTS (called with compile-time i by the
// unrolled MFMA loop); `all()` issues everything at once.  The dependency
// wait of the stage has already succeeded when these are issued.
template <class T, class AL, class BL>
struct StageLoads {
  static constexpr int NB = BL::NI, NA = AL::NI, N = NB + NA;
  static_assert(N == T::LOADS, "loads per stage");
  AL& al;
  BL& bl;
  char* st;
  int nxt;
  __device__ __forceinline__ void issue(int j) {
    if (j < NB)
      bl.issue_one(j, st + T::A_BYTES, nxt);
    else
      al.issue_one(j - NB, st, nxt);
  }
  // With a two-stage ring the loads of a stage are consumed right after the
  // step that issues them, so they go out over the first half of its slots
  // (measured on the 256 x 192 tile: 13 % faster than the whole step, whose
  // last loads then land late; a quarter is slower again, the address queue
  // backs up).  With more stages there is a step of slack: the whole step.
  static constexpr int SPAN = T::NS == 2 ? (T::SLOTS + 1) / 2 : T::SLOTS;
  __device__ __forceinline__ void slot(int i) {
#pragma unroll
    for (int j = 0; j < N; ++j)
      if ((j * SPAN) / N == i) issue(j);
  }
  __device__ __forceinline__ void all() {
#pragma unroll
    for (int j = 0; j < N; ++j) issue(j);
  }
};

// StageLoads of step kt that also start the sentinel check of stage kt + 1
// (rings of three or more stages): after the loads of slot CHECK this
// thread waits until its loads of stage kt + 1 have landed (every load issued
// after them may stay in flight: the NS - 3 whole stages between and this
// step's loads so far) and reads its chunks back; the last groups of MFMAs
// of the step then cover the read latency, and the boundary only tests.
template <class T, class AL, class BL>
struct CheckedStageLoads : StageLoads<T, AL, BL> {
  using Base = StageLoads<T, AL, BL>;
  const char* next_stage;
  static constexpr int CHECK = T::SLOTS >= 4 ? T::SLOTS - 3 : T::SLOTS - 1;
  static constexpr int issued_through(int i) {
    int c = 0;
    for (int j = 0; j < Base::N; ++j)
      if ((j * Base::SPAN) / Base::N <= i) ++c;
    return c;
  }
  __device__ __forceinline__ void slot(int i) {
    Base::slot(i);
    if (i == CHECK) {
      wait_vmcnt_n((T::NS - 3) * T::LOADS + issued_through(CHECK));
      this->al.fix_begin(next_stage);
    }
  }
};

// The last NS - 1 steps have nothing left to load.
struct NoLoads {
  __device__ __forceinline__ void slot(int) {}
  __device__ __forceinline__ void all() {}
};

// Pipelined loop over KT steps of an NS-stage LDS ring: stage s holds the A
// operand (A_BYTES) then the B operand.  `step(stage, kt, loads)` consumes a
// landed stage and issues the loads of stage kt + NS - 1 through `loads`
// (into the ring slot that step kt - 1 used, free after the barrier).
// Returns false if a wait expired (the tile is abandoned).
template <class T, class = void>
struct IsSplitRing {
  static constexpr bool value = false;
};
template <class T>
struct IsSplitRing<T, decltype((void)T::SPLIT_RING)> {
  static constexpr bool value = T::SPLIT_RING;
};

template <class T, class AL, class BL, class W, class STEP>
__device__ __forceinline__ bool pipeline(char* smem, int KT, AL& al, BL& bl, W& w, STEP&& step) {
  static_assert(!IsSplitRing<T>::value, "pipeline() runs rings of equal depth");
  // Prologue: stages 0 .. NS-2.  The independent operand B is issued before
  // the dependency wait of each stage, so its loads overlap the wait (the
  // "+R" reordering of the cuSync paper, section "Reorder Tile Loads and
  // Synchronization").
#pragma unroll
  for (int s = 0; s < T::NS - 1; ++s) {
    if (s < KT) {
      char* st = smem + s * T::STAGE;
      bl.issue(st + T::A_BYTES, s);
      if (!w.before(s)) {
        wait_vmcnt<0>();
        return false;
      }
      al.issue(st, s);
    }
  }
  // Steps whose successor stage NS - 1 ahead still has to be loaded, then the
  // last NS - 1 steps.  Separate loops rather than a branch per step, so that
  // the accumulators flow straight through without a join.  A waiter that
  // waits at later steps keeps its wait in the first loop only while some
  // producer tile is still outstanding; the second loop carries no wait code.
  constexpr bool kSplitLoop = StepWaits<W>::value;
  int kt = 0;
  for (; kt + T::NS - 1 < KT && !(kSplitLoop && w.all_ready()); ++kt) {
    const int later = min(T::NS - 2, KT - 1 - kt);
    wait_stage<T>(later);  // this thread's loads of step kt have landed
    char* cur = smem + (kt % T::NS) * T::STAGE;
    al.fix(cur, kt);
    wg_barrier();  // everyone's loads of step kt landed; step kt-1 consumed
    const int nxt = kt + T::NS - 1;
    if (!w.before(nxt)) {
      wait_vmcnt<0>();
      return false;
    }
    StageLoads<T, AL, BL> ld{al, bl, smem + (nxt % T::NS) * T::STAGE, nxt};
    step(cur, kt, ld);
  }
  if constexpr (kSplitLoop) {
    for (; kt + T::NS - 1 < KT; ++kt) {
      const int later = min(T::NS - 2, KT - 1 - kt);
      wait_stage<T>(later);
      char* cur = smem + (kt % T::NS) * T::STAGE;
      al.fix(cur, kt);
      wg_barrier();
      const int nxt = kt + T::NS - 1;
      StageLoads<T, AL, BL> ld{al, bl, smem + (nxt % T::NS) * T::STAGE, nxt};
      step(cur, kt, ld);
    }
  }
  for (; kt < KT; ++kt) {
    wait_stage<T>(KT - 1 - kt);
    char* cur = smem + (kt % T::NS) * T::STAGE;
    al.fix(cur, kt);
    wg_barrier();
    NoLoads ld;
    step(cur, kt, ld);
  }
  return true;
}

// The loads one step of a split ring issues: those of B for step bkt (the
// next one) first, then, with HAS_A, those of A for step akt (two ahead),
// spread over the step's MFMA slots in that order.  Issuing every B load
// before any A load is what lets the boundary into the next step wait with
// vmcnt(A_INSTR): only this step's A loads may then still be in flight.
template <class T, class AL, class BL, bool HAS_A>
struct SplitStageLoads {
  static constexpr int NB = BL::NI, NA = HAS_A ? AL::NI : 0, N = NB + NA;
  AL& al;
  BL& bl;
  char* smem;
  int bkt, akt;
  __device__ __forceinline__ void issue(int j) {
    if (j < NB)
      bl.issue_one(j, smem + T::b_off(bkt), bkt);
    else
      al.issue_one(j - NB, smem + T::a_off(akt), akt);
  }
  __device__ __forceinline__ void slot(int i) {
#pragma unroll
    for (int j = 0; j < N; ++j)
      if ((j * T::SLOTS) / N == i) issue(j);
  }
};

// Main loop of a split ring (A three slots deep, B two): the A operand of
// step kt + 2 and the B operand of step kt + 1 are loaded during step kt, so
// A loads, which come from farther away (the activations are read by every
// column tile, the weight panel mostly from this XCD's L2), have two steps
// to land.  Slots and barriers as in gemm_mainloop: the slot written during
// step kt is the one step kt - 1 read, free after the barrier that entered
// step kt.  Accumulation order, hence the bits, is the same as with any
// other ring.
template <class T, class AL, class BL, class W>
__device__ __forceinline__ bool gemm_mainloop_split(Gemm<T>& g, char* smem, int KT, AL& al,
                                                    BL& bl, W& w) {
  static_assert(T::SPLIT_RING && T::NS == 3 && T::NSB == 2, "split ring shape");
  g.zero();
  if (KT <= 0) return true;
  // Prologue: B(0), A(0), A(1); B before the dependency wait (+R).
  bl.issue(smem + T::b_off(0), 0);
  if (!w.before(0)) {
    wait_vmcnt<0>();
    return false;
  }
  al.issue(smem + T::a_off(0), 0);
  if (KT > 1) {
    if (!w.before(1)) {
      wait_vmcnt<0>();
      return false;
    }
    al.issue(smem + T::a_off(1), 1);
  }
  f16x8 a[2][T::FM], b[2][T::FN];
  // Enter step s: its A and B have landed once at most the A loads of step
  // s + 1 (issued after them) are outstanding.
  auto enter = [&](int s, bool a_next_pending) {
    if (a_next_pending)
      wait_vmcnt<T::A_INSTR>();
    else
      wait_vmcnt<0>();
    al.fix(smem + T::a_off(s), s);
    wg_barrier();
    g.read_frags(smem + T::a_off(s), smem + T::b_off(s), 0, a[0], b[0]);
  };
  enter(0, KT > 1);
  constexpr bool kStep = StepWaits<W>::value;
  int kt = 0;
  // Steps that load both operands: first while a step wait may still be
  // needed, then without the wait's code (as in gemm_mainloop).
  for (; kt + 2 < KT && !(kStep && w.all_ready()); ++kt) {
    if (!w.before(kt + 2)) {
      wait_vmcnt<0>();
      return false;
    }
    SplitStageLoads<T, AL, BL, true> ld{al, bl, smem, kt + 1, kt + 2};
    g.compute(smem + T::a_off(kt), smem + T::b_off(kt), ld, a, b,
              [&]() { enter(kt + 1, true); });
  }
  if constexpr (kStep) {
    for (; kt + 2 < KT; ++kt) {
      SplitStageLoads<T, AL, BL, true> ld{al, bl, smem, kt + 1, kt + 2};
      g.compute(smem + T::a_off(kt), smem + T::b_off(kt), ld, a, b,
                [&]() { enter(kt + 1, true); });
    }
  }
  if (kt + 1 < KT) {  // step KT - 2: only the last B is left to load
    SplitStageLoads<T, AL, BL, false> ld{al, bl, smem, kt + 1, 0};
    g.compute(smem + T::a_off(kt), smem + T::b_off(kt), ld, a, b,
              [&]() { enter(kt + 1, false); });
    ++kt;
  }
  NoLoads ld;
  g.compute(smem + T::a_off(kt), smem + T::b_off(kt), ld, a, b, []() {});
  return true;
}

// Tile GEMM main loop: accumulators zeroed, then one MFMA step per stage of
// an NS-stage LDS ring (the prologue and load issue as in pipeline()).  The
// stage boundary sits inside the last k sub-step of the step before: once a
// wave has issued that sub-step's MFMAs it waits for its loads of the next
// stage, meets the others at the barrier and reads the next stage's first
// fragments, all while its MFMAs still run, so the matrix cores do not idle
// across the barrier.  The barrier also frees the ring slot of the step just
// finished (every wave's reads of it completed before its last MFMAs), which
// is where the loads of step kt + NS are issued during step kt + 1.
// Returns false if a wait expired (the tile is abandoned).
template <class T, class AL, class BL, class W>
__device__ __forceinline__ bool gemm_mainloop(Gemm<T>& g, char* smem, int KT, AL& al, BL& bl,
                                              W& w) {
  if constexpr (T::SPLIT_RING) return gemm_mainloop_split<T>(g, smem, KT, al, bl, w);
  g.zero();
#pragma unroll
  for (int s = 0; s < T::NS - 1; ++s) {
    if (s < KT) {
      char* st = smem + s * T::STAGE;
      bl.issue(st + T::A_BYTES, s);
      if (!w.before(s)) {
        wait_vmcnt<0>();
        return false;
      }
      al.issue(st, s);
    }
  }
  f16x8 a[2][T::FM], b[2][T::FN];
  // Enter stage `s` (all of its loads issued, those of up to `later`
  // stages after it may still be in flight): wait, check, barrier, first
  // fragments.
  // A sentinel loader on a ring of three or more stages has its check
  // started inside the step before (CheckedStageLoads); `checked` says so.
  constexpr bool kEarly = HasEarlyFix<AL>::value && T::NS >= 3;
  auto enter = [&](int s, int later, bool checked) {
    wait_stage<T>(later);
    char* st = smem + (s % T::NS) * T::STAGE;
    if constexpr (kEarly) {
      if (checked)
        al.fix_end(st, s);
      else
        al.fix(st, s);
    } else {
      al.fix(st, s);
    }
    wg_barrier();
    g.read_frags(st, st + T::A_BYTES, 0, a[0], b[0]);
  };
  using Loads = typename std::conditional<kEarly, CheckedStageLoads<T, AL, BL>,
                                          StageLoads<T, AL, BL>>::type;
  auto stage_loads = [&](int kt, int nxt) {
    if constexpr (kEarly)
      return Loads{{al, bl, smem + (nxt % T::NS) * T::STAGE, nxt},
                   smem + ((kt + 1) % T::NS) * T::STAGE};
    else
      return Loads{al, bl, smem + (nxt % T::NS) * T::STAGE, nxt};
  };
  if (KT <= 0) return true;
  enter(0, min(T::NS - 2, KT - 1), false);
  // Steps whose successor stage NS - 1 ahead still has to be loaded, then the
  // last NS - 1 steps.  Separate loops rather than a branch per step, so that
  // the accumulators flow straight through without a join.  The first loop
  // keeps the dependency wait and runs only while the waiter still has
  // something to wait for (a TileSync consumer that started before its row
  // was complete); the second carries no wait code at all, which keeps the
  // wait's registers and its barrier out of the steady-state loop.  Only the
  // two-stage rings leave the first loop early (the 256 x 192 8-wave tile,
  // whose waiting loop spills: 1.3x faster at M = 2048); with three or more
  // stages the first loop runs to the end and the second is unreachable,
  // which measured fastest for every other tile (the compiler's code for the
  // waiting loop depends on the whole function; measured, not derived).
  constexpr bool kWaitFreeLoop = T::NS == 2;
  int kt = 0;
  for (; kt + T::NS - 1 < KT && !(kWaitFreeLoop && w.all_ready()); ++kt) {
    char* cur = smem + (kt % T::NS) * T::STAGE;
    const int nxt = kt + T::NS - 1;
    if (!w.before(nxt)) {
      wait_vmcnt<0>();
      return false;
    }
    Loads ld = stage_loads(kt, nxt);
    g.compute(cur, cur + T::A_BYTES, ld, a, b, [&]() { enter(kt + 1, T::NS - 2, kEarly); });
  }
  for (; kt + T::NS - 1 < KT; ++kt) {
    char* cur = smem + (kt % T::NS) * T::STAGE;
    const int nxt = kt + T::NS - 1;
    Loads ld = stage_loads(kt, nxt);
    g.compute(cur, cur + T::A_BYTES, ld, a, b, [&]() { enter(kt + 1, T::NS - 2, kEarly); });
  }
  for (; kt < KT; ++kt) {
    char* cur = smem + (kt % T::NS) * T::STAGE;
    NoLoads ld;
    g.compute(cur, cur + T::A_BYTES, ld, a, b, [&]() {
      if (kt + 1 < KT) enter(kt + 1, KT - 2 - kt, false);
    });
  }
  return true;
}

// Deterministic split-K.  Split s of S of tile `tile` stores its fp32 partial
// accumulators to part (as a register image: chunk v of thread t at
// ((tile * S + s) * NV + v) * NT + t, 16 bytes each, so every store and load
// instruction of a wave covers 1 KiB contiguously), then counts its arrival.
// The workgroup whose arrival completes the tile becomes the reducer: it sums
// the S partials in split order, p0 + p1 + ... + p(S-1), whoever arrives
// last, so the result does not depend on timing, and returns true with the
// sum in g.acc.  The others return false.  Partials are written with
// device-scope stores and drained before the arrival (arrive_agent), and the
// completing arrival acquires, so the reducer sees every partial whichever
// XCD wrote it.  Only the chunks that hold rows below `rows` (the tile's rows
// inside the output; the others are never stored) move: a dead chunk's
// offset is pushed past the buffer, where the range check drops the store
// and makes the load read zero, without a branch per chunk.  A batch of one
// row moves 1/32 of the 8-wave 128 x 128 tile's partial.  The per-chunk
// offsets cost 8-20 registers; DEAD_ROWS = false keeps the plain offsets for
// chains whose tiles are all full but the last.  Called by all threads.
template <class T, bool DEAD_ROWS = true>
__device__ __forceinline__ bool split_k_reduce(Gemm<T>& g, float* part, uint32_t part_bytes,
                                               uint32_t tile, int s, int S, uint32_t* cnt,
                                               int* s_flag, uint32_t rows) {
  constexpr int NV = T::FM * T::FN * 4;  // f32x4 chunks per thread
  const uint32_t dead = part_bytes;       // the first offset past the buffer
  const auto pr = make_rsrc(part, part_bytes);
  const uint32_t tid = threadIdx.x;
  const uint32_t tbase = tile * (uint32_t)S * NV;
  // First of the four rows chunk v of this thread holds: accumulator
  // registers 4q .. 4q + 3 of block (fm, fn) (acc_row).
  const uint32_t rbase = (tid >> 6) / T::WN * T::WTM + 4 * ((tid & 63) >> 5);
  auto off = [&](int t, int v) {
    const uint32_t r = rbase + (uint32_t)(v / (T::FN * 4)) * 32u + 8u * (uint32_t)(v % 4);
    return r < rows ? (((tbase + (uint32_t)t * NV + v) * T::NT) + tid) * 16u : dead;
  };
#pragma unroll
  for (int v = 0; v < NV; ++v) {
    const int fm = v / (T::FN * 4), fn = (v / 4) % T::FN, q = v % 4;
    // Whole-vector bit cast: this compiler miscompiles __builtin_bit_cast of
    // a single vector element (it reads element 0 whatever the index).
    const f32x4 f = {g.acc[fm][fn][4 * q + 0], g.acc[fm][fn][4 * q + 1], g.acc[fm][fn][4 * q + 2],
                     g.acc[fm][fn][4 * q + 3]};
    const u32x4 w = __builtin_bit_cast(u32x4, f);
    if constexpr (DEAD_ROWS)
      publish16(pr, off(s, v), w);
    else
      publish16(pr, (((tbase + (uint32_t)s * NV + v) * T::NT) + tid) * 16u, w);
  }
  drain_vmem();
  __syncthreads();
  if (tid == 0) {
    const uint32_t before = arrive_agent(cnt, (uint32_t)S);
    *s_flag = (before + 1u == (uint32_t)S) ? 1 : 0;
  }
  __syncthreads();
  if (!*s_flag) return false;
  // The last arrival's acquire invalidated this CU's and XCD's caches, so
  // plain loads see every split's partial.
  const f32x4* pp = reinterpret_cast<const f32x4*>(part);
#pragma unroll
  for (int v = 0; v < NV; ++v) {
    const int fm = v / (T::FN * 4), fn = (v / 4) % T::FN, q = v % 4;
    f32x4 sum;
    if constexpr (DEAD_ROWS) {
      sum = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                          pr, (int)off(0, v), 0, kAuxNone));
      for (int t = 1; t < S; ++t)
        sum += __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                             pr, (int)off(t, v), 0, kAuxNone));
    } else {
      sum = pp[(tbase + v) * T::NT + tid];
      for (int t = 1; t < S; ++t) sum += pp[(tbase + (uint32_t)t * NV + v) * T::NT + tid];
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) g.acc[fm][fn][4 * q + e] = sum[e];
  }
  return true;
}

// Epilogue: the raw fp32 accumulators are staged through LDS (row-major, in
// one or two passes of wave rows), then every thread takes 8 consecutive
// values of a row, applies scale and activation, rounds to fp16 (NaN
// canonicalised) and hands a 16-byte chunk to `store(row, col, u32x4)` in
// tile-local coordinates.  `dbg(row, col, const float* v8)` receives the
// fp32 values before rounding when want_dbg is set.  Doing the activation
// here, one chunk at a time, keeps it out of the register-heavy accumulator
// phase.  ACT >= 0 fixes the activation at compile time (`act` is then
// ignored): a uniform switch per element cost the conv pair's producer tiles
// 2 of a 3.5 us epilogue.  The 256 x 192 MLP tile keeps the runtime switch:
// one epilogue copy per activation pushes it into spills that cost far more.
// The caller synchronises before smem is reused.
template <class T, int ACT = -1, class StoreFn, class DbgFn>
__device__ __forceinline__ void gemm_epilogue(Gemm<T>& g, char* smem, int act, float scale,
                                              StoreFn&& store, DbgFn&& dbg, bool want_dbg) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int wm = wave / T::WN, wn = wave % T::WN;
  float* Cs = reinterpret_cast<float*>(smem);
  constexpr int ROWS = T::BM / T::EPI_PASSES;
  constexpr int CPR = T::BN / 8;  // chunks per row
  constexpr int CH = ROWS * CPR / T::NT;
  static_assert((ROWS * CPR) % T::NT == 0, "epilogue chunking");
  wg_barrier();  // every wave is done reading the last stage
#pragma unroll
  for (int pass = 0; pass < T::EPI_PASSES; ++pass) {
    if (T::EPI_PASSES == 1 || wm == pass) {
#pragma unroll
      for (int fm = 0; fm < T::FM; ++fm)
#pragma unroll
        for (int fn = 0; fn < T::FN; ++fn)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int row = wm * T::WTM + fm * 32 + acc_row(lane, r) - pass * ROWS;
            const int col = wn * T::WTN + fn * 32 + acc_col(lane);
            Cs[row * T::LDCF + col] = g.acc[fm][fn][r];
          }
    }
    wg_barrier();
#pragma unroll 1
    for (int i = 0; i < CH; ++i) {
      const int c = threadIdx.x + i * T::NT;
      const int row = c / CPR, col = (c % CPR) * 8;
      const f32x4 lo = *reinterpret_cast<const f32x4*>(Cs + row * T::LDCF + col);
      const f32x4 hi = *reinterpret_cast<const f32x4*>(Cs + row * T::LDCF + col + 4);
      float v[8] = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
#pragma unroll
      for (int e = 0; e < 8; ++e) v[e] = apply_act(ACT >= 0 ? ACT : act, v[e] * scale);
      if (want_dbg) dbg(pass * ROWS + row, col, v);
      u32x4 o;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        if constexpr (T::BF16)
          o[e] = (uint32_t)f32_to_bf16_canon(v[2 * e]) |
                 ((uint32_t)f32_to_bf16_canon(v[2 * e + 1]) << 16);
        else
          o[e] = (uint32_t)f32_to_f16_canon(v[2 * e]) |
                 ((uint32_t)f32_to_f16_canon(v[2 * e + 1]) << 16);
      }
      store(pass * ROWS + row, col, o);
    }
    if (pass + 1 < T::EPI_PASSES) wg_barrier();
  }
}

}  // namespace tls
