// Measured hardware ceilings for the roofline (not part of the attention
// library or its C ABI; built as libfa_probes.so and called by the benchmark).
//
//   fa_probe_mfma_bf16: sustained v_mfma_f32_32x32x16_bf16 throughput of the
//     whole chip, two waves per SIMD, eight independent accumulators per
//     wave, operands held in registers.  The operands are either hashed
//     bf16 values (random sign and mantissa, exponent near 1) or zeros: the
//     matrix cores draw far less power on zeros, and on a power-limited part
//     that changes the clock, so the random figure is the relevant ceiling
//     for attention on random data.
//   fa_probe_hbm_read(_hint): read-only streaming bandwidth over a device
//     buffer with 16-byte loads, eight in flight per thread, with or without
//     the non-temporal load hint.
//
// Both allocate their own buffers and synchronise the device; they are
// measurement tools, not for use inside a timed region.
#include <hip/hip_runtime.h>
#include <cstdint>

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ uint32_t mix32(uint32_t x) {
  x ^= x >> 16;
  x *= 0x7feb352dU;
  x ^= x >> 15;
  x *= 0x846ca68bU;
  x ^= x >> 16;
  return x;
}

constexpr int kPeakThreads = 256;

template <bool ZERO>
__global__ __launch_bounds__(kPeakThreads) void mfma_peak_kernel(float* out, long long* clk, int iters) {
  const uint32_t id = blockIdx.x * kPeakThreads + threadIdx.x;
  u32x4 ra[4], rb[4];
  for (int i = 0; i < 4; ++i)
    for (int j = 0; j < 4; ++j) {
      const uint32_t h = mix32(id * 131u + i * 17u + j);
      const uint32_t g = mix32(h);
      // bf16 pairs: exponent of 0.5..1, random sign and mantissa bits
      ra[i][j] = ZERO ? 0u : ((0x3f00u | (h & 0x807fu)) | ((0x3f00u | ((h >> 16) & 0x807fu)) << 16));
      rb[i][j] = ZERO ? 0u : ((0x3f00u | (g & 0x807fu)) | ((0x3f00u | ((g >> 16) & 0x807fu)) << 16));
    }
  f32x16 c[8];
  for (int i = 0; i < 8; ++i) c[i] = f32x16{};
  const long long t0 = __builtin_amdgcn_s_memtime();
  const long long r0 = __builtin_amdgcn_s_memrealtime();
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int i = 0; i < 8; ++i)
      c[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, ra[(i + it) & 3]),
                                                     __builtin_bit_cast(bf16x8, rb[(i + 2 * it) & 3]), c[i], 0, 0, 0);
  }
  const long long t1 = __builtin_amdgcn_s_memtime();
  const long long r1 = __builtin_amdgcn_s_memrealtime();
  float s = 0.f;
  for (int i = 0; i < 8; ++i)
    for (int j = 0; j < 16; ++j) s += c[i][j];
  out[id] = s;
  if (threadIdx.x == 0) {
    clk[2 * blockIdx.x] = t1 - t0;
    clk[2 * blockIdx.x + 1] = r1 - r0;
  }
}

constexpr int kReadThreads = 256;
constexpr int kReadUnroll = 8;

// NT: loads carry the non-temporal hint (evict-first), as a one-pass stream would.
template <bool NT>
__global__ __launch_bounds__(kReadThreads) void hbm_read_kernel(const u32x4* __restrict__ p, size_t n16,
                                                                uint32_t* out) {
  uint32_t acc = 0;
  const size_t stride = (size_t)gridDim.x * kReadThreads * kReadUnroll;
  for (size_t i = (size_t)blockIdx.x * kReadThreads * kReadUnroll + threadIdx.x; i < n16; i += stride) {
    u32x4 v[kReadUnroll];
#pragma unroll
    for (int u = 0; u < kReadUnroll; ++u)
      v[u] = (i + (size_t)u * kReadThreads < n16)
                 ? (NT ? __builtin_nontemporal_load(&p[i + (size_t)u * kReadThreads]) : p[i + (size_t)u * kReadThreads])
                 : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
    for (int u = 0; u < kReadUnroll; ++u) acc ^= v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3];
  }
  if (acc == 0x9e3779b9u) out[0] = acc;  // keeps the loads live
}

struct Events {
  hipEvent_t a = nullptr, b = nullptr;
  ~Events() {
    if (a) (void)hipEventDestroy(a);
    if (b) (void)hipEventDestroy(b);
  }
};

}  // namespace

extern "C" {

// Sustained dense bf16 MFMA rate of the whole device (TFLOP/s) and the mean
// shader clock of workgroup 0 during the run (GHz, from s_memtime against
// the 100 MHz s_memrealtime).  iters: MFMA groups per wave (8 MFMAs each).
// Returns 0 on success, 1 on a HIP error.
int fa_probe_mfma_bf16(int zero_operands, int iters, double* tflops, double* shader_ghz) {
  if (iters <= 0 || tflops == nullptr || shader_ghz == nullptr) return 1;
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 1;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 1;
  const int blocks = 2 * cus;  // 4 waves per workgroup -> two waves per SIMD
  float* out = nullptr;
  long long* clk = nullptr;
  if (hipMalloc(&out, (size_t)blocks * kPeakThreads * sizeof(float)) != hipSuccess) return 1;
  if (hipMalloc(&clk, (size_t)blocks * 2 * sizeof(long long)) != hipSuccess) {
    (void)hipFree(out);
    return 1;
  }
  int rc = 1;
  Events e;
  do {
    if (hipEventCreate(&e.a) != hipSuccess || hipEventCreate(&e.b) != hipSuccess) break;
    auto launch = [&] {
      if (zero_operands)
        hipLaunchKernelGGL(mfma_peak_kernel<true>, dim3(blocks), dim3(kPeakThreads), 0, 0, out, clk, iters);
      else
        hipLaunchKernelGGL(mfma_peak_kernel<false>, dim3(blocks), dim3(kPeakThreads), 0, 0, out, clk, iters);
    };
    launch();  // warm-up (clocks ramp)
    if (hipDeviceSynchronize() != hipSuccess) break;
    if (hipEventRecord(e.a, 0) != hipSuccess) break;
    launch();
    if (hipEventRecord(e.b, 0) != hipSuccess) break;
    if (hipEventSynchronize(e.b) != hipSuccess) break;
    float ms = 0.f;
    if (hipEventElapsedTime(&ms, e.a, e.b) != hipSuccess || ms <= 0.f) break;
    long long c[2];
    if (hipMemcpy(c, clk, sizeof(c), hipMemcpyDeviceToHost) != hipSuccess) break;
    const double flops = (double)blocks * (kPeakThreads / 64) * iters * 8 * (2.0 * 32 * 32 * 16);
    *tflops = flops / (ms * 1e-3) / 1e12;
    *shader_ghz = c[1] > 0 ? (double)c[0] / ((double)c[1] / 100e6) / 1e9 : 0.0;
    rc = 0;
  } while (false);
  (void)hipFree(out);
  (void)hipFree(clk);
  return rc;
}

// Read-only HBM bandwidth (GB/s, decimal) over a buffer of `bytes` bytes
// (rounded down to 16), averaged over `reps` passes after one warm-up; with
// `nontemporal` the loads carry the non-temporal hint.
int fa_probe_hbm_read_hint(size_t bytes, int reps, int nontemporal, double* gbs) {
  if (bytes < 16 || reps <= 0 || gbs == nullptr) return 1;
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 1;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 1;
  const size_t n16 = bytes / 16;
  u32x4* buf = nullptr;
  uint32_t* out = nullptr;
  if (hipMalloc(&buf, n16 * 16) != hipSuccess) return 1;
  if (hipMalloc(&out, 64) != hipSuccess) {
    (void)hipFree(buf);
    return 1;
  }
  int rc = 1;
  Events e;
  do {
    if (hipMemset(buf, 1, n16 * 16) != hipSuccess) break;
    if (hipEventCreate(&e.a) != hipSuccess || hipEventCreate(&e.b) != hipSuccess) break;
    const int blocks = 8 * cus;
    auto launch = [&] {
      if (nontemporal)
        hipLaunchKernelGGL(hbm_read_kernel<true>, dim3(blocks), dim3(kReadThreads), 0, 0, buf, n16, out);
      else
        hipLaunchKernelGGL(hbm_read_kernel<false>, dim3(blocks), dim3(kReadThreads), 0, 0, buf, n16, out);
    };
    launch();
    if (hipDeviceSynchronize() != hipSuccess) break;
    if (hipEventRecord(e.a, 0) != hipSuccess) break;
    for (int r = 0; r < reps; ++r) launch();
    if (hipEventRecord(e.b, 0) != hipSuccess) break;
    if (hipEventSynchronize(e.b) != hipSuccess) break;
    float ms = 0.f;
    if (hipEventElapsedTime(&ms, e.a, e.b) != hipSuccess || ms <= 0.f) break;
    *gbs = (double)n16 * 16 * reps / (ms * 1e-3) / 1e9;
    rc = 0;
  } while (false);
  (void)hipFree(buf);
  (void)hipFree(out);
  return rc;
}

// The same without the hint.
int fa_probe_hbm_read(size_t bytes, int reps, double* gbs) { return fa_probe_hbm_read_hint(bytes, reps, 0, gbs); }

}  // extern "C"
