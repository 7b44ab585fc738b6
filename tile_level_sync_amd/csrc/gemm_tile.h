// MFMA tile engine for gfx950: one workgroup computes a BM x BN tile of
// C = A B with fp16 operands and fp32 accumulation, K staged in steps of 64
// through two LDS buffers (the next step's global loads are in flight while
// the matrix cores consume the current one).  Tiles follow the cuSync paper,
// section "Tile based Computations": tile C^{xy} multiplies BM rows of A with
// BN columns of B; here each of the 2 x 2 waves owns a (BM/2) x (BN/2) block
// made of 32 x 32 MFMA blocks (v_mfma_f32_32x32x16_f16).
//
// Operand layouts:
//   A   row-major [rows][K] (K contiguous): read from LDS with ds_read_b128.
//   B   "KN" row-major [K][N] (N contiguous, the weight layout as written):
//       staged as is and read with the gfx950 transposing LDS read
//       ds_read_b64_tr_b16, which hands each lane 4 consecutive K values of
//       one column.  "NK" [N][K] (K contiguous, e.g. K^T of attention) is
//       read like A.
#pragma once

#include "device.h"

namespace tls {

template <int BM_, int BN_, bool B_NK_ = false>
struct TileShape {
  static constexpr int BM = BM_, BN = BN_, BK = 64;
  static constexpr int WM = 2, WN = 2;
  static constexpr int NT = 64 * WM * WN;
  static constexpr int WTM = BM / WM, WTN = BN / WN;
  static constexpr int FM = WTM / 32, FN = WTN / 32;
  static constexpr bool B_NK = B_NK_;
  // LDS row strides in halfs; the padding spreads rows over the banks.
  static constexpr int LDA = BK + 8;
  static constexpr int LDB = B_NK ? BK + 8 : BN + 16;
  static constexpr int LDCF = BN + 4;  // fp32 epilogue staging row stride
  static constexpr int A_STAGE = BM * LDA;
  static constexpr int B_STAGE = B_NK ? BN * LDB : BK * LDB;
  static constexpr int STAGE = A_STAGE + B_STAGE;
  static constexpr int A_CHUNKS = BM * BK / 8 / NT;  // 16-byte chunks per thread
  static constexpr int B_CHUNKS = BK * BN / 8 / NT;
  // The fp32 staging of the epilogue takes one pass, or two passes of wave
  // rows when a full tile would not fit in the K-loop's LDS footprint.
  static constexpr int EPI_PASSES = (BM * LDCF * 2 <= 2 * STAGE) ? 1 : WM;
  static constexpr int EPI_HALFS = (BM / EPI_PASSES) * LDCF * 2;
  static constexpr int SMEM_HALFS = (2 * STAGE > EPI_HALFS) ? 2 * STAGE : EPI_HALFS;
  static_assert(FM >= 1 && FN >= 1, "tile too small for 2x2 waves of 32x32 blocks");
  static_assert(A_CHUNKS >= 1 && B_CHUNKS >= 1, "tile too small");
  static_assert((BM * BK / 8) % NT == 0 && (BK * BN / 8) % NT == 0, "chunking");
};

// Row / column of the element that accumulator register r of `lane` holds in
// a 32 x 32 MFMA block: rows advance in groups of 4 per half-wave.
__device__ __forceinline__ int acc_row(int lane, int r) {
  return 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
}
__device__ __forceinline__ int acc_col(int lane) { return lane & 31; }

template <class T>
struct Gemm {
  f32x16 acc[T::FM][T::FN];
  u32x4 ra[T::A_CHUNKS];
  u32x4 rb[T::B_CHUNKS];

  __device__ __forceinline__ void zero() {
#pragma unroll
    for (int i = 0; i < T::FM; ++i)
#pragma unroll
      for (int j = 0; j < T::FN; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;
  }

  template <class AL>
  __device__ __forceinline__ void load_a(AL& al, int kt) {
#pragma unroll
    for (int i = 0; i < T::A_CHUNKS; ++i) {
      const int c = threadIdx.x + i * T::NT;
      ra[i] = al.load(c >> 3, (c & 7) * 8, kt);
    }
  }

  template <class BL>
  __device__ __forceinline__ void load_b(BL& bl, int kt) {
#pragma unroll
    for (int i = 0; i < T::B_CHUNKS; ++i) {
      const int c = threadIdx.x + i * T::NT;
      if constexpr (T::B_NK)
        rb[i] = bl.load(c >> 3, (c & 7) * 8, kt);  // (n row, k col)
      else
        rb[i] = bl.load(c / (T::BN / 8), (c % (T::BN / 8)) * 8, kt);  // (k row, n col)
    }
  }

  __device__ __forceinline__ void store_a(f16* As) const {
#pragma unroll
    for (int i = 0; i < T::A_CHUNKS; ++i) {
      const int c = threadIdx.x + i * T::NT;
      *reinterpret_cast<u32x4*>(As + (c >> 3) * T::LDA + (c & 7) * 8) = ra[i];
    }
  }

  __device__ __forceinline__ void store_b(f16* Bs) const {
#pragma unroll
    for (int i = 0; i < T::B_CHUNKS; ++i) {
      const int c = threadIdx.x + i * T::NT;
      if constexpr (T::B_NK)
        *reinterpret_cast<u32x4*>(Bs + (c >> 3) * T::LDB + (c & 7) * 8) = rb[i];
      else
        *reinterpret_cast<u32x4*>(Bs + (c / (T::BN / 8)) * T::LDB + (c % (T::BN / 8)) * 8) =
            rb[i];
    }
  }

  // One BK step of MFMAs from an LDS stage.
  __device__ __forceinline__ void compute(const f16* As, const f16* Bs) {
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int wm = wave / T::WN, wn = wave % T::WN;
#pragma unroll
    for (int kk = 0; kk < T::BK / 16; ++kk) {
      f16x8 a[T::FM], b[T::FN];
#pragma unroll
      for (int fm = 0; fm < T::FM; ++fm) {
        const f16* p = As + (wm * T::WTM + fm * 32 + (lane & 31)) * T::LDA + kk * 16 +
                       (lane >> 5) * 8;
        a[fm] = *reinterpret_cast<const f16x8*>(p);
      }
#pragma unroll
      for (int fn = 0; fn < T::FN; ++fn) {
        if constexpr (T::B_NK) {
          const f16* p = Bs + (wn * T::WTN + fn * 32 + (lane & 31)) * T::LDB + kk * 16 +
                         (lane >> 5) * 8;
          b[fn] = *reinterpret_cast<const f16x8*>(p);
        } else {
          // Transposing read: in each group of 16 lanes, lane (r, c) = 4r + c
          // names 4 consecutive halfs of row r; lane j receives column j of
          // the 4 x 16 block.  Lanes 0-31 take K rows 0-7 of this 16-step,
          // lanes 32-63 rows 8-15; columns 0-15 / 16-31 by (lane >> 4) & 1.
          const int g = lane >> 4, i = lane & 15;
          const int row = kk * 16 + (g >> 1) * 8 + (i >> 2);
          const int col = wn * T::WTN + fn * 32 + (g & 1) * 16 + (i & 3) * 4;
          const f16* p0 = Bs + row * T::LDB + col;
          const f16* p1 = p0 + 4 * T::LDB;
          fp16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4f16((TLS_LDS_AS fp16x4*)(p0));
          fp16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4f16((TLS_LDS_AS fp16x4*)(p1));
          f16x8 v;
          v[0] = (f16)lo[0]; v[1] = (f16)lo[1]; v[2] = (f16)lo[2]; v[3] = (f16)lo[3];
          v[4] = (f16)hi[0]; v[5] = (f16)hi[1]; v[6] = (f16)hi[2]; v[7] = (f16)hi[3];
          b[fn] = v;
        }
      }
#pragma unroll
      for (int fm = 0; fm < T::FM; ++fm)
#pragma unroll
        for (int fn = 0; fn < T::FN; ++fn)
          acc[fm][fn] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a[fm], b[fn], acc[fm][fn], 0, 0, 0);
    }
  }
};

// Waiters: called uniformly by all threads before the A slice of step kt is
// loaded; return false when the wait expired (the tile is abandoned).
struct NoWait {
  __device__ __forceinline__ bool before(int) { return true; }
};

// Fix-up of loaded A chunks before they are staged (sentinel re-poll); the
// plain loaders have nothing to fix.
struct NoFix {};

// Double-buffered main loop.  Returns false if a wait expired.
template <class T, class AL, class BL, class W>
__device__ __forceinline__ bool gemm_mainloop(Gemm<T>& g, f16* smem, int KT, AL& al, BL& bl,
                                              W& w) {
  g.zero();
  f16* A0 = smem;
  f16* B0 = smem + T::A_STAGE;
  f16* A1 = smem + T::STAGE;
  f16* B1 = A1 + T::A_STAGE;
  // Independent operand first, then the (possibly) dependent one: the B
  // loads overlap the wait (the "+R" reordering of the cuSync paper, section
  // "Reorder Tile Loads and Synchronization").
  g.load_b(bl, 0);
  if (!w.before(0)) return false;
  g.load_a(al, 0);
  al.fix(g.ra, 0);
  g.store_a(A0);
  g.store_b(B0);
  __syncthreads();
  for (int kt = 0; kt < KT; ++kt) {
    const bool nxt = kt + 1 < KT;
    if (nxt) {
      g.load_b(bl, kt + 1);
      if (!w.before(kt + 1)) return false;
      g.load_a(al, kt + 1);
    }
    const bool odd = kt & 1;
    g.compute(odd ? A1 : A0, odd ? B1 : B0);
    if (nxt) {
      al.fix(g.ra, kt + 1);
      g.store_a(odd ? A0 : A1);
      g.store_b(odd ? B0 : B1);
    }
    __syncthreads();
  }
  return true;
}

// Epilogue: the raw fp32 accumulators are staged through LDS (row-major,
// in one or two passes of wave rows), then every thread takes 8 consecutive
// values of a row, applies scale and activation, rounds to fp16 (NaN
// canonicalised) and hands a 16-byte chunk to `store(row, col, u32x4)` in
// tile-local coordinates.  `dbg(row, col, const float* v8)` receives the
// fp32 values before rounding when want_dbg is set.  Doing the activation
// here, one chunk at a time, keeps it out of the register-heavy accumulator
// phase.  The caller synchronises before smem is reused.
template <class T, class StoreFn, class DbgFn>
__device__ __forceinline__ void gemm_epilogue(Gemm<T>& g, f16* smem, int act, float scale,
                                              StoreFn&& store, DbgFn&& dbg, bool want_dbg) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int wm = wave / T::WN, wn = wave % T::WN;
  float* Cs = reinterpret_cast<float*>(smem);
  constexpr int ROWS = T::BM / T::EPI_PASSES;
  constexpr int CPR = T::BN / 8;  // chunks per row
  constexpr int CH = ROWS * CPR / T::NT;
  static_assert((ROWS * CPR) % T::NT == 0, "epilogue chunking");
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
    __syncthreads();
#pragma unroll 2
    for (int i = 0; i < CH; ++i) {
      const int c = threadIdx.x + i * T::NT;
      const int row = c / CPR, col = (c % CPR) * 8;
      const f32x4 lo = *reinterpret_cast<const f32x4*>(Cs + row * T::LDCF + col);
      const f32x4 hi = *reinterpret_cast<const f32x4*>(Cs + row * T::LDCF + col + 4);
      float v[8] = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
#pragma unroll
      for (int e = 0; e < 8; ++e) v[e] = apply_act(act, v[e] * scale);
      if (want_dbg) dbg(pass * ROWS + row, col, v);
      u32x4 o;
#pragma unroll
      for (int e = 0; e < 4; ++e)
        o[e] = (uint32_t)f32_to_f16_canon(v[2 * e]) |
               ((uint32_t)f32_to_f16_canon(v[2 * e + 1]) << 16);
      store(pass * ROWS + row, col, o);
    }
    if (pass + 1 < T::EPI_PASSES) __syncthreads();
  }
}

}  // namespace tls
