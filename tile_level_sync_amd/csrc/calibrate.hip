// Measurement calibration: the sustained dense fp16 MFMA rate and shader
// clock of the current device.  Every wave of a persistent grid (one or two
// four-wave workgroups per CU) runs `iters` rounds of eight independent
// v_mfma_f32_32x32x16_f16 chains on pseudo-random register operands (four
// operand sets used in turn, so consecutive instructions see different bits,
// as in a GEMM), with nothing else in the loop: the MFMA ceiling a GEMM
// engine could reach on this chip under its power management.  The clock is
// the shader clock counter (s_memtime) over the constant 100 MHz realtime
// counter (s_memrealtime) across the loop, averaged over the waves.  Every
// thread stores one float so that the loop is not removed; lane 0 of every
// wave stores its two counter deltas.
#include <hip/hip_runtime.h>

#include <vector>

#include "../../include/tlsync.h"
#include "device.h"
#include "internal.h"
#include "runtime_internal.h"

namespace tls {
namespace {

typedef _Float16 c_f16x8 __attribute__((ext_vector_type(8)));
typedef float c_f32x16 __attribute__((ext_vector_type(16)));
constexpr int kChains = 8;
constexpr double kFlopsPerMfma = 2.0 * 32 * 32 * 16;

__global__ void __launch_bounds__(256) mfma_ceiling_kernel(float* out, uint64_t* clk, int iters) {
  c_f16x8 av[4], bv[4];
  uint32_t x = 2463534242u ^ (threadIdx.x * 747796405u) ^ (blockIdx.x * 2891336453u);
  for (int k = 0; k < 4; ++k)
    for (int i = 0; i < 8; ++i) {
      x ^= x << 13; x ^= x >> 17; x ^= x << 5;
      av[k][i] = (_Float16)((float)(x & 0xFFFFu) * (1.0f / 65536.0f) - 0.5f);
      x ^= x << 13; x ^= x >> 17; x ^= x << 5;
      bv[k][i] = (_Float16)((float)(x & 0xFFFFu) * (1.0f / 65536.0f) - 0.5f);
    }
  c_f32x16 acc[kChains];
  for (int c = 0; c < kChains; ++c)
    for (int r = 0; r < 16; ++r) acc[c][r] = 0.0f;
  const uint64_t t0 = __builtin_amdgcn_s_memtime();
  const uint64_t r0 = __builtin_amdgcn_s_memrealtime();
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int c = 0; c < kChains; ++c)
      acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_f16(av[c & 3], bv[(c + (c >> 2)) & 3], acc[c],
                                                      0, 0, 0);
  }
  const uint64_t t1 = __builtin_amdgcn_s_memtime();
  const uint64_t r1 = __builtin_amdgcn_s_memrealtime();
  float s = 0.0f;
  for (int c = 0; c < kChains; ++c)
    for (int r = 0; r < 16; ++r) s += acc[c][r];
  const size_t gid = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  out[gid] = s;
  if ((threadIdx.x & 63u) == 0u) {
    const size_t w = gid / 64;
    clk[2 * w] = t1 - t0;
    clk[2 * w + 1] = r1 - r0;
  }
}

// Plain copy with the chain kernels' access style (16-byte buffer loads and
// stores with the default cache policy), grid-stride over 16-byte chunks.
__global__ void __launch_bounds__(256) copy16_kernel(const void* in, void* out, uint32_t chunks) {
  const auto rs = make_rsrc(in, chunks * 16u);
  const auto rd = make_rsrc(out, chunks * 16u);
  for (uint32_t i = blockIdx.x * blockDim.x + threadIdx.x; i < chunks;
       i += gridDim.x * blockDim.x) {
    const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(rs, (int)(i * 16u), 0, 0);
    store_out16(rd, i * 16u, v);
  }
}

}  // namespace
}  // namespace tls

using namespace tls;

extern "C" {

chain_status chain_calibrate_mfma(int waves_per_simd, int iters, void* scratch,
                                  size_t scratch_bytes, void* stream, double* tflops,
                                  double* ghz, double* ms) {
  if (waves_per_simd < 1 || waves_per_simd > 2 || iters <= 0 || !scratch || !tflops || !ghz ||
      !ms)
    return CHAIN_EINVAL;
  int dev = 0, cus = 0;
  chain_status st = current_device(&dev);
  if (st != CHAIN_OK) return st;
  if ((st = device_cus(dev, &cus)) != CHAIN_OK) return st;
  const int grid = cus * waves_per_simd;
  const size_t threads = (size_t)grid * 256, waves = threads / 64;
  const size_t out_bytes = threads * sizeof(float), clk_bytes = waves * 2 * sizeof(uint64_t);
  if (scratch_bytes < out_bytes + clk_bytes || ((uintptr_t)scratch & 15u)) return CHAIN_EINVAL;
  float* out = (float*)scratch;
  uint64_t* clk = (uint64_t*)((char*)scratch + out_bytes);
  const hipStream_t s = (hipStream_t)stream;
  hipEvent_t e0 = nullptr, e1 = nullptr;
  hipError_t e = hipEventCreate(&e0);
  if (e == hipSuccess) e = hipEventCreate(&e1);
  if (e == hipSuccess) e = hipEventRecord(e0, s);
  if (e == hipSuccess) {
    hipLaunchKernelGGL(mfma_ceiling_kernel, dim3(grid), dim3(256), 0, s, out, clk, iters);
    e = hipGetLastError();
  }
  if (e == hipSuccess) e = hipEventRecord(e1, s);
  if (e == hipSuccess) e = hipEventSynchronize(e1);
  float t = 0.0f;
  if (e == hipSuccess) e = hipEventElapsedTime(&t, e0, e1);
  std::vector<uint64_t> h(waves * 2);
  if (e == hipSuccess) e = hipMemcpy(h.data(), clk, clk_bytes, hipMemcpyDeviceToHost);
  if (e0) (void)hipEventDestroy(e0);
  if (e1) (void)hipEventDestroy(e1);
  if (e != hipSuccess) return hip_fail(e);
  double cyc = 0.0, rt = 0.0;
  for (size_t w = 0; w < waves; ++w) {
    cyc += (double)h[2 * w];
    rt += (double)h[2 * w + 1];
  }
  *ms = t;
  *ghz = rt > 0.0 ? cyc / rt * 0.1 : 0.0;  // realtime counter at 100 MHz
  *tflops = (double)waves * iters * kChains * kFlopsPerMfma / (t * 1e-3) / 1e12;
  return CHAIN_OK;
}

chain_status chain_calibrate_copy(const void* src, void* dst, size_t bytes, void* stream) {
  if (!src || !dst || !aligned16(src) || !aligned16(dst) || bytes == 0 || (bytes & 15u) ||
      bytes >= ((size_t)1 << 31))
    return CHAIN_EINVAL;
  int dev = 0, cus = 0;
  chain_status st = current_device(&dev);
  if (st != CHAIN_OK) return st;
  if ((st = device_cus(dev, &cus)) != CHAIN_OK) return st;
  hipLaunchKernelGGL(copy16_kernel, dim3(cus * 8), dim3(256), 0, (hipStream_t)stream, src, dst,
                     (uint32_t)(bytes / 16));
  const hipError_t e = hipGetLastError();
  return e == hipSuccess ? CHAIN_OK : hip_fail(e);
}

}  // extern "C"
