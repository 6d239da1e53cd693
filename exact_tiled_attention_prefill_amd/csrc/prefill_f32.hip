// fp32 prefill: the same tiled running-softmax method in plain fp32 vector
// arithmetic, for callers that need fp32 inputs and fp32 results.
//
// Method: tiles of keys/values are staged in LDS and consumed one at a time
// while each query row keeps its running max and running sum ("11.4d
// FlashAttention", "Tiling" and "Online Softmax"); scale, mask, normalisation
// and aggregation are fused ("How Does Flash Attention Reduce Memory Traffic
// During Local Inference?", "Kernel Fusion Keeps More of the Attention Chain
// in One Execution Path").
//
// Layout: one thread per query row, 128 rows per workgroup; the output
// accumulator in registers, the rows' q in LDS (padded by one word, so the
// 128 threads' reads of their own rows fall in different banks), 32-key fp32
// K/V tiles in LDS read as broadcasts.
//
// Precision: fp32 inputs and outputs, fp64 sums.  The scores q.k, the
// running max, the output accumulator and the running sum are fp64, and the
// exponentials exp2f of the (fp64-formed) arguments are fp32.  In fp32 a row's
// sum of N terms p * v grows a rounding error like sqrt(N) * 2^-24 * |o|
// (about 1e-5 at N = 2800, |o| = 4), and the 128-term fp32 dot product puts
// ~5e-6 (log2 units) into each exponent at |scale| = 0.45, which a sharp
// softmax turns into ~1e-5 of output error; products of fp32 values are exact
// in fp64.  The coefficient c = |scale| log2(e) is formed in fp64 too: in
// fp32 its rounding (2^-24 relative) times a row max of a few hundred (log2
// units) moves lse by ~1e-5.  What is left is the fp32 exponentials, about
// 1e-6 of the output, and lse's own fp32 rounding.
#include "common.h"
#include "kernels.h"

namespace fa {
namespace {

constexpr int kF32Rows = 128;
constexpr int kF32Keys = 32;

template <int D, bool CAUSAL>
__global__ __launch_bounds__(128) void prefill_f32_kernel(
    const float* __restrict__ q, const float* __restrict__ k, const float* __restrict__ v,
    float* __restrict__ o, float* __restrict__ lse, int Hq, int Hkv, int N, int n_qtiles, int BH,
    double cd, float qsign) {
  __shared__ float qs[kF32Rows][D + 1];
  __shared__ float ks[kF32Keys][D];
  __shared__ float vs[kF32Keys][D];
  const int tid = threadIdx.x;
  const int bid = blockIdx.x;
  const int qtile = CAUSAL ? (n_qtiles - 1 - bid / BH) : (bid / BH);
  const int bh = bid % BH;
  const int b = bh / Hq;
  const int h = bh - b * Hq;
  const int g = h / (Hq / Hkv);
  const float* qh = q + (size_t)bh * N * D;
  const float* kh = k + ((size_t)b * Hkv + g) * N * D;
  const float* vh = v + ((size_t)b * Hkv + g) * N * D;

  const int q0 = qtile * kF32Rows;
  const int row = q0 + tid;
  const bool live = row < N;

  double acc[D];
  // q rows of the workgroup into LDS (coalesced: consecutive threads read
  // consecutive elements)
  for (int e = tid; e < kF32Rows * D; e += kF32Rows) {
    const int r = e / D, cc = e % D;
    qs[r][cc] = q0 + r < N ? qsign * qh[(size_t)(q0 + r) * D + cc] : 0.f;
  }
#pragma unroll
  for (int i = 0; i < D; ++i) acc[i] = 0.0;
  double m_run = -INFINITY;  // running max of c * (q . k), log2 units
  double l_run = 0.0;

  const int kv_end = CAUSAL ? min(N, q0 + kF32Rows) : N;
  for (int k0 = 0; k0 < kv_end; k0 += kF32Keys) {
    __syncthreads();
    for (int i = tid; i < kF32Keys * D; i += kF32Rows) {
      const int r = i / D, cc = i % D;
      const bool ok = k0 + r < N;
      ks[r][cc] = ok ? kh[(size_t)(k0 + r) * D + cc] : 0.f;
      vs[r][cc] = ok ? vh[(size_t)(k0 + r) * D + cc] : 0.f;
    }
    __syncthreads();
    // s[j] = q . k_j in fp64, summed over i in order
    double s[kF32Keys];
#pragma unroll
    for (int j = 0; j < kF32Keys; ++j) s[j] = 0.0;
    for (int i = 0; i < D; ++i) {
      const double qi = (double)qs[tid][i];
#pragma unroll
      for (int j = 0; j < kF32Keys; ++j) s[j] = fma(qi, (double)ks[j][i], s[j]);
    }
    double mx = -INFINITY;
#pragma unroll
    for (int j = 0; j < kF32Keys; ++j) {
      const int key = k0 + j;
      const bool masked = key >= N || (CAUSAL && key > row);
      s[j] = masked ? -INFINITY : s[j];
      mx = fmax(mx, s[j]);
    }
    const double mn = fmax(m_run, mx * cd);
    if (mn == -INFINITY) continue;  // nothing visible yet (padding rows only)
    const double alpha = (double)exp2f((float)(m_run - mn));
    l_run *= alpha;
#pragma unroll
    for (int i = 0; i < D; ++i) acc[i] *= alpha;
    m_run = mn;
#pragma unroll
    for (int j = 0; j < kF32Keys; ++j) {
      const double p = (double)exp2f((float)fma(s[j], cd, -mn));
      l_run += p;
#pragma unroll
      for (int i = 0; i < D; ++i) acc[i] = fma(p, (double)vs[j][i], acc[i]);
    }
  }
  if (!live) return;
  const double inv = 1.0 / l_run;
#pragma unroll
  for (int i = 0; i < D; ++i) o[(size_t)bh * N * D + (size_t)row * D + i] = (float)(acc[i] * inv);
  if (lse != nullptr) lse[(size_t)bh * N + row] = (float)(m_run * 0.6931471805599453 + log(l_run));
}

// c = |scale| log2(e) in fp64, clamped below at kMinC as the bf16 kernels' c is
// (so that c * (-inf) stays -inf at a zero scale)
double f32_coeff(float scale_abs) {
  const double c = (double)scale_abs * 1.4426950408889634074;
  return c < (double)kMinC ? (double)kMinC : c;
}

template <int D, bool CAUSAL>
hipError_t launch(const PrefillArgs& a, hipStream_t stream) {
  const int n_qtiles = (a.N + kF32Rows - 1) / kF32Rows;
  const int BH = a.B * a.Hq;
  const long long blocks = (long long)n_qtiles * BH;
  if (blocks > 0x7fffffffLL) return hipErrorInvalidValue;
  hipLaunchKernelGGL((prefill_f32_kernel<D, CAUSAL>), dim3((unsigned)blocks), dim3(kF32Rows), 0, stream,
                     static_cast<const float*>(a.q), static_cast<const float*>(a.k),
                     static_cast<const float*>(a.v), static_cast<float*>(a.o), a.lse, a.Hq, a.Hkv, a.N,
                     n_qtiles, BH, f32_coeff(a.scale_abs), a.neg ? -1.0f : 1.0f);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_prefill_f32(const PrefillArgs& a, hipStream_t stream) {
  if (a.d == 128) return a.causal ? launch<128, true>(a, stream) : launch<128, false>(a, stream);
  if (a.d == 64) return a.causal ? launch<64, true>(a, stream) : launch<64, false>(a, stream);
  return hipErrorInvalidValue;
}

}  // namespace fa
