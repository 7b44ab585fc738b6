// Persistent three-stage self-attention chain (cuSync paper, Fig.
// "Architecture of two building blocks of GPT models" (b), one GPU's share of
// the model-parallel layer; section "Self-Attention" and paragraph
// StridedSync of "Synchronization Policies"):
//   stage 1  XQKV[M, 3 Hs] = X Wqkv, tiles of 128 x 128: column tile c of the
//            first slice holds head c's queries, the same column of the second
//            and third slices its score and value operands;
//   stage 2  per (block of 256 queries, head h): the fused dot product
//            O = softmax(scale * Q S2^T) S3 over every token, into XDot[M, Hs];
//   stage 3  Y = XDot W2, tiles of 128 x 128.
// Stage 2 of head h reads column tile h of all three slices for every row
// tile.  Under StridedSync those 3 x (M/128) tiles, `heads` columns apart,
// share one counter and stage 2 waits once for it; stage 1 hands out its
// tiles head group by head group (the three slices of a head, all rows) so
// the first heads complete early.  Under TileSync stage 2 scans the tiles'
// own flags.  Stage 3 waits per head (TileSync on the XDot tiles of its row
// block) as its K loop reaches each head's columns.
//
// When the (query block, head) items of stage 2 do not fill the chip, each is
// split into S items over contiguous ranges of 64-key blocks; every split
// leaves its unnormalised softmax state and the last to finish merges them
// in split order, so the bits do not depend on timing.
//
// Stage 2 is a flash-style kernel: the queries stay in registers as the B
// operand of S^T = S2_j Q^T (keys x queries, so every accumulator a lane
// holds belongs to its one query), an online softmax in base 2, and
// O^T += S3_j^T P^T with P fed straight from the S^T accumulators: the MFMA
// contraction over keys runs in the order the accumulators hold them (keys
// 0-3, 8-11 in lanes 0-31 and 4-7, 12-15 in lanes 32-63 of each 16), so the
// S3 fragments are read in that same order.
#include "gemm_tile.h"
#include "sched.h"
#include "waits.h"

namespace tls {

constexpr int kSaD = 128;    // head dimension
constexpr int kSaBQ = 256;   // queries per stage-2 item: 8 waves x 32
constexpr int kSaBK = 64;    // keys per stage-2 pipeline step
// stage 1 and 3 GEMM tiles, 8 waves; fp16 or bf16 storage
template <bool BF16>
using SaTile = TileShape<128, 128, 4, 64, 2, 4, false, BF16>;
using SaT = SaTile<false>;

// One stage-2 pipeline step in LDS: 64 keys x 128 of the score operand (A
// layout, chunk c of row r at c ^ (r & 15)), then 64 keys x 128 of the value
// operand (KN layout, read transposed).
struct FlashShape {
  static constexpr int NS = 3, NW = 8, NT = 512;
  static constexpr int A_BYTES = kSaBK * kSaD * 2;
  static constexpr int B_BYTES = A_BYTES;
  static constexpr int STAGE = A_BYTES + B_BYTES;
  static constexpr int LOADS = (A_BYTES + B_BYTES) / (NT * 16);
  static constexpr int SLOTS = 4;
};

template <bool VALUE>
struct SaKeyRows : NoFix {
  static constexpr int NI = FlashShape::A_BYTES / (FlashShape::NT * 16);
  i32x4 rs;
  uint32_t voff[NI];
  uint32_t kstep;
  __device__ __forceinline__ void init(const void* qkv, uint32_t bytes, uint32_t col0,
                                       uint32_t ld) {
    rs = make_srd(qkv, bytes);
    kstep = (uint32_t)kSaBK * ld * 2u;
#pragma unroll
    for (int j = 0; j < NI; ++j) {
      const int P = dma_position<FlashShape::NW>(j);
      const int r = P / 16, cl = P % 16;
      const int cg = VALUE ? (cl ^ swz_b<16>(r)) : (cl ^ (r & 15));
      voff[j] = (r * ld + col0 + cg * 8) * 2u;
    }
  }
  __device__ __forceinline__ void issue_one(int j, char* region, int kt) const {
    dma16<kAuxNone>(rs, region + dma_block<FlashShape::NW>(j), voff[j] + kt * kstep);
  }
  __device__ __forceinline__ void issue(char* region, int kt) const {
#pragma unroll
    for (int j = 0; j < NI; ++j) issue_one(j, region, kt);
  }
};

// BF16: the operands are bf16 patterns (held in f16x8 registers as bits) and
// P enters the second product in bf16.
template <bool BF16>
struct FlashStep {
  f16x8 qf[kSaD / 16];  // this wave's 32 queries as the B operand, one per 16 of d
  f32x16 o[kSaD / 32];  // O^T: d blocks of 32 x 32 queries
  float m, l;           // running max (base-2 units) and partial sum of this lane's query
  float sl2e;           // scale * log2(e)
  int M;                // tokens: keys at or past M (the last block's tail) are masked
  int kb0;              // first key block of this item's key range
  template <class LOADS>
  __device__ __forceinline__ void operator()(char* cur, int kt, LOADS& loads) {
    loads.all();
    const int lane = threadIdx.x & 63;
    const char* sK = cur;
    const char* sV = cur + FlashShape::A_BYTES;
    f32x16 s[kSaBK / 32];
#pragma unroll
    for (int fm = 0; fm < kSaBK / 32; ++fm)
#pragma unroll
      for (int r = 0; r < 16; ++r) s[fm][r] = 0.0f;
#pragma unroll
    for (int kk = 0; kk < kSaD / 16; ++kk) {
#pragma unroll
      for (int fm = 0; fm < kSaBK / 32; ++fm) {
        const int row = fm * 32 + (lane & 31);
        const f16x8 a = *reinterpret_cast<const f16x8*>(
            sK + row * (kSaD * 2) + (((2 * kk + (lane >> 5)) ^ (row & 15)) * 16));
        if constexpr (BF16)
          s[fm] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                          __builtin_bit_cast(bf16x8, qf[kk]),
                                                          s[fm], 0, 0, 0);
        else
          s[fm] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, qf[kk], s[fm], 0, 0, 0);
      }
    }
    float bmax = -__builtin_inff();
#pragma unroll
    for (int fm = 0; fm < kSaBK / 32; ++fm)
#pragma unroll
      for (int r = 0; r < 16; ++r) s[fm][r] *= sl2e;
    // Keys past the last token (read as zero rows) take no probability: -inf
    // scores.  Only the last block can hold them, and it keeps at least one
    // valid key; every key split starts below the last token, so the running
    // max of every split stays finite.
    const int key0 = (kb0 + kt) * kSaBK;
    if (key0 + kSaBK > M) {
#pragma unroll
      for (int fm = 0; fm < kSaBK / 32; ++fm)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (key0 + fm * 32 + acc_row(lane, r) >= M) s[fm][r] = -__builtin_inff();
    }
#pragma unroll
    for (int fm = 0; fm < kSaBK / 32; ++fm)
#pragma unroll
      for (int r = 0; r < 16; ++r) bmax = fmaxf(bmax, s[fm][r]);
    bmax = fmaxf(bmax, __shfl_xor(bmax, 32));
    const float mnew = fmaxf(m, bmax);
    const float alpha = exp2f(m - mnew);
    l *= alpha;
#pragma unroll
    for (int i = 0; i < kSaD / 32; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r) o[i][r] *= alpha;
    m = mnew;
    // l sums the rounded probabilities, the values the product uses.
    f16x8 pf[kSaBK / 16];
    u16x8 pb[kSaBK / 16];
#pragma unroll
    for (int kk = 0; kk < kSaBK / 16; ++kk)
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float pv = exp2f(s[kk / 2][8 * (kk % 2) + e] - mnew);
        if constexpr (BF16) {
          const uint16_t hb = f32_to_bf16_canon(pv);
          l += __builtin_bit_cast(float, (uint32_t)hb << 16);
          pb[kk][e] = hb;
        } else {
          const f16 ph = (f16)pv;
          l += (float)ph;
          pf[kk][e] = ph;
        }
      }
    // O^T += S3^T P^T: A fragments of S3 read transposed, keys in the order of pf.
#pragma unroll
    for (int kk = 0; kk < kSaBK / 16; ++kk) {
      const int g = lane >> 4, i = lane & 15;
      const int k = kk * 16 + (g >> 1) * 4 + (i >> 2);  // keys 0-3 / 4-7, then + 8
#pragma unroll
      for (int fd = 0; fd < kSaD / 32; ++fd) {
        const int n = fd * 32 + (g & 1) * 16 + (i & 3) * 4;
        const int off = k * (kSaD * 2) + (((n >> 3) ^ swz_b<kSaD / 8>(k)) * 16) + (n & 7) * 2;
        fp16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4f16((TLS_LDS_AS fp16x4*)(sV + off));
        fp16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4f16(
            (TLS_LDS_AS fp16x4*)(sV + off + 8 * kSaD * 2));
        if constexpr (BF16) {
          // the transposing read moves 16-bit patterns: bf16 S3 as stored
          const u16x4 l4 = __builtin_bit_cast(u16x4, lo), h4 = __builtin_bit_cast(u16x4, hi);
          const u16x8 a16 = {l4[0], l4[1], l4[2], l4[3], h4[0], h4[1], h4[2], h4[3]};
          o[fd] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
              __builtin_bit_cast(bf16x8, a16), __builtin_bit_cast(bf16x8, pb[kk]), o[fd], 0, 0, 0);
        } else {
          f16x8 a;
          a[0] = (f16)lo[0]; a[1] = (f16)lo[1]; a[2] = (f16)lo[2]; a[3] = (f16)lo[3];
          a[4] = (f16)hi[0]; a[5] = (f16)hi[1]; a[6] = (f16)hi[2]; a[7] = (f16)hi[3];
          o[fd] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, pf[kk], o[fd], 0, 0, 0);
        }
      }
    }
  }
};

// Stage 1 work item = (tile, K split), tile = (row tile, virtual column).
// Virtual column v lists the head groups: head v / 3, slice v % 3.  The
// splits of a tile are adjacent items; the last to arrive sums the partials
// in split order (deterministic) and finishes the tile.  Tiles below
// tail_begin have ks1 splits, the rest (the tail, last in item order)
// ks_tail, with their partials indexed from the first tail tile.
template <int POL, bool BF16>
__device__ __forceinline__ void sa_stage1(const SaParams& p, char* smem, uint32_t item,
                                          uint32_t epoch, int* s_flag) {
  using T = SaTile<BF16>;
  const uint32_t head_items = p.tail_begin * (uint32_t)p.ks1;
  uint32_t tile, pidx;
  int split, S;
  if (item < head_items) {
    tile = item / (uint32_t)p.ks1;
    split = (int)(item % (uint32_t)p.ks1);
    S = p.ks1;
    pidx = tile;
  } else {
    const uint32_t t = item - head_items;
    pidx = t / (uint32_t)p.ks_tail;
    tile = p.tail_begin + pidx;
    split = (int)(t % (uint32_t)p.ks_tail);
    S = p.ks_tail;
  }
  const int r = tile / p.nc1, v = tile % p.nc1;
  const int head = v / 3, c = (v % 3) * p.heads + head;
  const uint32_t row0 = r * T::BM, col0 = c * T::BN, ld = 3u * p.Hs;
  const int KS = p.H / T::BK / S;
  const uint32_t k0 = (uint32_t)(split * KS * T::BK);  // first K element of the split
  PlainRows<T> al;
  al.init((const char*)p.X + k0 * 2u, (uint32_t)p.M * p.H * 2u - k0 * 2u, row0, (uint32_t)p.H);
  RowMajorKN<T> bl;
  bl.init((const char*)p.Wqkv + (size_t)k0 * ld * 2u, (uint32_t)(p.H - k0) * ld * 2u, col0, ld);
  NoWait w;
  Gemm<T> g;
  gemm_mainloop<T>(g, smem, KS, al, bl, w);
  const bool skip = (int32_t)item == p.skip_producer;
  if (S > 1) {
    if (skip) {  // this split never arrives (test knob): the tile never completes
      __syncthreads();
      return;
    }
    if (!split_k_reduce<T>(g, p.part1, p.part1_bytes, pidx, split, S,
                           p.splitcnt + tile * kFlagStride, s_flag, (uint32_t)p.M - row0))
      return;
  }
  debug_delay(item, p.delay);
  const auto qr = make_rsrc(p.QKV, (uint32_t)p.M * ld * 2u);
  auto store = [&](int rr, int cc, u32x4 v4) {
    publish16(qr, ((row0 + rr) * ld + col0 + cc) * 2u, v4);
  };
  auto nodbg = [](int, int, const float*) {};
  gemm_epilogue<T>(g, smem, kActNone, 1.0f, store, nodbg, false);
  drain_vmem();
  __syncthreads();
  if (threadIdx.x == 0 && !skip) {
    if constexpr (POL == kStrided) {
      post_add(p.sem + head * kFlagStride, 1u);
    } else if constexpr (POL == kTileSync) {
      post_store(p.flags1 + (r * p.nc1 + c) * kFlagStride, epoch);
    }
  }
}

// Stage 2 wait under TileSync: every stage-1 tile of head h's three column
// tiles over all row tiles, checked by wave 0 in parallel.
struct SaGroupWait {
  const uint32_t* flags;
  int mt1, nc1, heads, head;
  uint32_t epoch, limit;
  Ctl* ctl;
  uint32_t item;
  int* s_ok;
  bool light;
  __device__ __forceinline__ bool wait() {
    if (threadIdx.x < 64) {
      const int lane = threadIdx.x, n = 3 * mt1;
      const int ok = wave_wait_all(
                         [&]() {
                           bool mine = true;
                           for (int f = lane; f < n; f += 64) {
                             const int r = f / 3, c = (f % 3) * heads + head;
                             mine = mine && reached(ld_relaxed_agent(flags + (r * nc1 + c) * kFlagStride),
                                                    epoch);
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

// Merge of the key splits of one stage-2 item (flash-decoding style): split
// s left its unnormalised O^T, running max m_s (base 2) and partial sum l_s
// as a register image; the last split to arrive reads all of them back in
// split order and rescales each to the common max, so the result does not
// depend on which split came last.  Chunk v of thread t of split s of pair
// q sits at ((q * S + s) * kSaChunks + v) * 512 + t (16 bytes each).
constexpr int kSaChunks = kSaD / 32 * 4 + 1;  // 16 chunks of O^T, then (m, l, 0, 0)

template <class FS>
__device__ __forceinline__ void sa_store_partial(const SaParams& p, const FS& fs,
                                                 uint32_t pair, int split) {
  const auto pr = make_rsrc(p.part2, p.part2_bytes);
  const uint32_t base = (pair * (uint32_t)p.ks2 + (uint32_t)split) * kSaChunks;
#pragma unroll
  for (int v = 0; v < kSaChunks; ++v) {
    f32x4 f;
    if (v < kSaChunks - 1) {
      const int i = v / 4, q = v % 4;
      f = f32x4{fs.o[i][4 * q], fs.o[i][4 * q + 1], fs.o[i][4 * q + 2], fs.o[i][4 * q + 3]};
    } else {
      f = f32x4{fs.m, fs.l, 0.0f, 0.0f};
    }
    publish16(pr, ((base + v) * 512u + threadIdx.x) * 16u, __builtin_bit_cast(u32x4, f));
  }
}

template <class FS>
__device__ __forceinline__ void sa_merge_partials(const SaParams& p, FS& fs,
                                                  uint32_t pair) {
  const f32x4* pp = reinterpret_cast<const f32x4*>(p.part2);
  const uint32_t base = pair * (uint32_t)p.ks2 * kSaChunks;
  float m = -__builtin_inff();
  for (int s = 0; s < p.ks2; ++s)
    m = fmaxf(m, pp[(base + s * kSaChunks + kSaChunks - 1) * 512u + threadIdx.x][0]);
  float l = 0.0f;
#pragma unroll
  for (int i = 0; i < kSaD / 32; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) fs.o[i][r] = 0.0f;
  for (int s = 0; s < p.ks2; ++s) {
    const uint32_t b = base + s * kSaChunks;
    const f32x4 ml = pp[(b + kSaChunks - 1) * 512u + threadIdx.x];
    const float a = exp2f(ml[0] - m);
    l += ml[1] * a;
#pragma unroll
    for (int v = 0; v < kSaChunks - 1; ++v) {
      const f32x4 f = pp[(b + v) * 512u + threadIdx.x];
      const int i = v / 4, q = v % 4;
#pragma unroll
      for (int e = 0; e < 4; ++e) fs.o[i][4 * q + e] += f[e] * a;
    }
  }
  fs.m = m;
  fs.l = l;
}

template <int POL, bool BF16>
__device__ __forceinline__ void sa_stage2(const SaParams& p, char* smem, uint32_t it,
                                          uint32_t epoch, int* s_ok, uint64_t* s_tready) {
  // Item = ((query block, head), key split); the splits of a pair are adjacent.
  const uint32_t pair = it / (uint32_t)p.ks2;
  const int split = (int)(it % (uint32_t)p.ks2);
  const int qb = pair / p.heads, h = pair % p.heads;
  const uint32_t item = p.P1 + it;
  bool ok = true;
  if constexpr (POL == kStrided) {
    RowSyncWait w{p.sem + h * kFlagStride, 3u * (uint32_t)p.mt1, p.poll_limit, p.ctl, item, s_ok,
                  p.light_acquire != 0};
    ok = w.before(0);
  } else if constexpr (POL == kTileSync) {
    SaGroupWait w{p.flags1, p.mt1, p.nc1, p.heads, h, epoch, p.poll_limit, p.ctl, item, s_ok,
                  p.light_acquire != 0};
    ok = w.wait();
  }
  if (POL != kSerial && s_tready != nullptr && threadIdx.x == 0) *s_tready = now_rt();
  if (ok) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const uint32_t ld = 3u * p.Hs;
    const uint32_t q = (uint32_t)(qb * kSaBQ + wave * 32 + (lane & 31));
    const uint32_t qkv_bytes = (uint32_t)p.M * ld * 2u;
    FlashStep<BF16> fs;
    // Queries past the last token read as zero (range-checked loads); their
    // outputs are dropped by the store's range check.
    const auto qr = make_rsrc(p.QKV, qkv_bytes);
    const uint32_t qoff = (q * ld + (uint32_t)(h * kSaD + 8 * (lane >> 5))) * 2u;
#pragma unroll
    for (int kk = 0; kk < kSaD / 16; ++kk)
      fs.qf[kk] = __builtin_bit_cast(
          f16x8, __builtin_amdgcn_raw_buffer_load_b128(qr, (int)(qoff + kk * 32u), 0, 0));
#pragma unroll
    for (int i = 0; i < kSaD / 32; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r) fs.o[i][r] = 0.0f;
    fs.m = -__builtin_inff();
    fs.l = 0.0f;
    fs.sl2e = p.scale_log2e;
    fs.M = p.M;
    // This split's key blocks [kb0, kb1): contiguous, every split non-empty.
    const int per = (p.nkb + p.ks2 - 1) / p.ks2;
    const int kb0 = split * per, kb1 = min(p.nkb, kb0 + per);
    fs.kb0 = kb0;
    const uint32_t koff = (uint32_t)kb0 * kSaBK * ld * 2u;  // byte offset of the first key row
    SaKeyRows<false> kl;
    kl.init((const char*)p.QKV + koff, qkv_bytes - koff, (uint32_t)(p.Hs + h * kSaD), ld);
    SaKeyRows<true> vl;
    vl.init((const char*)p.QKV + koff, qkv_bytes - koff, (uint32_t)(2 * p.Hs + h * kSaD), ld);
    NoWait nw;
    pipeline<FlashShape>(smem, kb1 - kb0, kl, vl, nw, fs);
    if (p.ks2 > 1) {
      if ((int32_t)item == p.skip_producer) {  // this split never arrives (test knob)
        __syncthreads();
        return;
      }
      sa_store_partial(p, fs, pair, split);
      drain_vmem();
      __syncthreads();
      if (threadIdx.x == 0) {
        const uint32_t before = arrive_agent(p.splitcnt + (p.T1 + pair) * kFlagStride, p.ks2);
        *s_ok = (before + 1u == (uint32_t)p.ks2) ? 1 : 0;
      }
      __syncthreads();
      if (!*s_ok) return;  // another split finishes the pair
      // The last arrival's acquire invalidated this CU's and XCD's caches, so
      // plain loads see every split's partial.
      sa_merge_partials(p, fs, pair);
    }
    const float lt = fs.l + __shfl_xor(fs.l, 32);
    const float inv = 1.0f / lt;
    const auto dr = make_rsrc(p.Dot, (uint32_t)p.M * p.Hs * 2u);
#pragma unroll
    for (int fd = 0; fd < kSaD / 32; ++fd)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d0 = h * kSaD + fd * 32 + 8 * g + 4 * (lane >> 5);
        auto cvt = [](float v) -> uint32_t {
          if constexpr (BF16)
            return f32_to_bf16_canon(v);
          else
            return f32_to_f16_canon(v);
        };
        u32x2 o2;
        o2[0] = cvt(fs.o[fd][4 * g + 0] * inv) | (cvt(fs.o[fd][4 * g + 1] * inv) << 16);
        o2[1] = cvt(fs.o[fd][4 * g + 2] * inv) | (cvt(fs.o[fd][4 * g + 3] * inv) << 16);
        publish8(dr, (q * (uint32_t)p.Hs + d0) * 2u, o2);
      }
    debug_delay(item, p.delay);
    drain_vmem();
  }
  __syncthreads();
  if (ok && threadIdx.x == 0 && (int32_t)item != p.skip_producer && POL != kSerial)
    post_store(p.flags2 + pair * kFlagStride, epoch);
}

template <int POL, bool BF16>
__device__ __forceinline__ void sa_stage3(const SaParams& p, char* smem, uint32_t it,
                                          uint32_t epoch, int* s_ok, uint64_t* s_tready) {
  using T = SaTile<BF16>;
  const int r = it / p.nc3, c = it % p.nc3;
  const uint32_t row0 = r * T::BM, col0 = c * T::BN;
  const uint32_t item = p.P1 + p.P2 + it;
  PlainRows<T> al;
  al.init(p.Dot, (uint32_t)p.M * p.Hs * 2u, row0, (uint32_t)p.Hs);
  RowMajorKN<T> bl;
  bl.init(p.W2, (uint32_t)p.Hs * p.H * 2u, col0, (uint32_t)p.H);
  Gemm<T> g;
  bool ok;
  const int KT = p.Hs / T::BK;
  if constexpr (POL == kSerial) {
    NoWait w;
    ok = gemm_mainloop<T>(g, smem, KT, al, bl, w);
  } else {
    const int qb = row0 / kSaBQ;
    TileSyncWait w{p.flags2 + (size_t)qb * p.heads * kFlagStride, kSaD / T::BK, p.heads, epoch,
                   p.poll_limit, p.ctl, item, s_ok, 0, p.light_acquire != 0, 0};
    TracedWait<TileSyncWait> tw{w, s_tready};
    ok = gemm_mainloop<T>(g, smem, KT, al, bl, tw);
  }
  if (ok) {
    const auto yr = make_rsrc(p.Y, (uint32_t)p.M * p.H * 2u);
    auto store = [&](int rr, int cc, u32x4 v4) {
      store_out16(yr, ((row0 + rr) * (uint32_t)p.H + col0 + cc) * 2u, v4);
    };
    auto nodbg = [](int, int, const float*) {};
    gemm_epilogue<T>(g, smem, kActNone, 1.0f, store, nodbg, false);
  }
  __syncthreads();
}

template <int POL, bool BF16>
__global__ void __launch_bounds__(512) selfattn_chain_kernel(SaParams p) {
  constexpr int SMEM = SaT::SMEM > FlashShape::NS * FlashShape::STAGE
                           ? SaT::SMEM
                           : FlashShape::NS * FlashShape::STAGE;
  __shared__ __attribute__((aligned(1024))) char smem[SMEM];
  __shared__ uint32_t s_item;
  __shared__ int s_ok;
  __shared__ int s_last;
  __shared__ uint64_t s_tready;
  const uint32_t epoch = p.ctl->epoch + 1u;
  const bool tracing = p.trace != nullptr;
  uint64_t* const tr = tracing ? &s_tready : nullptr;
  SchedState st;
  st.init(p.sp);
  for (;;) {
    if (threadIdx.x == 0) s_item = st.next(p.sp);
    __syncthreads();
    const uint32_t item = s_item;
    if (item == kNoItem) break;
    uint64_t t0 = 0;
    if (tracing && threadIdx.x == 0) s_tready = t0 = now_rt();
    if (item < p.P1)
      sa_stage1<POL, BF16>(p, smem, item, epoch, &s_ok);
    else if (item < p.P1 + p.P2)
      sa_stage2<POL, BF16>(p, smem, item - p.P1, epoch, &s_ok, tr);
    else
      sa_stage3<POL, BF16>(p, smem, item - p.P1 - p.P2, epoch, &s_ok, tr);
    if (tracing && threadIdx.x == 0 && item < p.trace_cap)
      p.trace[item] = TraceRec{item, (uint16_t)blockIdx.x, hw_location(), t0, s_tready, now_rt()};
  }
  sched_finish(p.sp, &s_last, POL == kStrided, p.sem, p.heads, POL != kSerial, epoch,
               p.splitcnt,
               (p.ks1 > 1 || p.ks_tail > 1 || p.ks2 > 1) ? (int)(p.T1 + (uint32_t)p.nq * p.heads)
                                                          : 0);
}

template <bool BF16>
static hipError_t selfattn_launch_t(const SaParams& p, int grid, hipStream_t s) {
  switch (p.policy) {
    case kSerial:
      hipLaunchKernelGGL((selfattn_chain_kernel<kSerial, BF16>), dim3(grid), dim3(512), 0, s, p);
      break;
    case kStrided:
      hipLaunchKernelGGL((selfattn_chain_kernel<kStrided, BF16>), dim3(grid), dim3(512), 0, s,
                         p);
      break;
    case kTileSync:
      hipLaunchKernelGGL((selfattn_chain_kernel<kTileSync, BF16>), dim3(grid), dim3(512), 0, s,
                         p);
      break;
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t selfattn_launch(const SaParams& p, int grid, hipStream_t s) {
  return p.bf16 ? selfattn_launch_t<true>(p, grid, s) : selfattn_launch_t<false>(p, grid, s);
}

// The fp16 instance stands for both element types (the same LDS footprint and
// launch bounds).
hipError_t selfattn_occupancy(int, int* blocks) {
  return hipOccupancyMaxActiveBlocksPerMultiprocessor(
      blocks, selfattn_chain_kernel<kStrided, false>, 512, 0);
}

}  // namespace tls
