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
// Layout: one thread per query row (q and the output accumulator in VGPRs),
// 128 rows per workgroup, 32-key fp32 K/V tiles in LDS read as broadcasts.
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
    float c, float qsign) {
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

  float qr[D], acc[D];
#pragma unroll
  for (int i = 0; i < D; ++i) {
    qr[i] = live ? qsign * qh[(size_t)row * D + i] : 0.f;
    acc[i] = 0.f;
  }
  float m_run = -INFINITY, l_run = 0.f;

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
    float s[kF32Keys];
    float mx = -INFINITY;
#pragma unroll
    for (int j = 0; j < kF32Keys; ++j) {
      float dot = 0.f;
#pragma unroll
      for (int i = 0; i < D; ++i) dot = fmaf(qr[i], ks[j][i], dot);
      const int key = k0 + j;
      const bool masked = key >= N || (CAUSAL && key > row);
      s[j] = masked ? -INFINITY : dot;
      mx = fmaxf(mx, s[j]);
    }
    const float mn = fmaxf(m_run, mx * c);
    if (mn == -INFINITY) continue;  // nothing visible yet (padding rows only)
    const float alpha = fast_exp2(m_run - mn);
    l_run *= alpha;
#pragma unroll
    for (int i = 0; i < D; ++i) acc[i] *= alpha;
    m_run = mn;
#pragma unroll
    for (int j = 0; j < kF32Keys; ++j) {
      const float p = exp2f(fmaf(s[j], c, -mn));
      l_run += p;
#pragma unroll
      for (int i = 0; i < D; ++i) acc[i] = fmaf(p, vs[j][i], acc[i]);
    }
  }
  if (!live) return;
  const float inv = 1.0f / l_run;
#pragma unroll
  for (int i = 0; i < D; ++i) o[(size_t)bh * N * D + (size_t)row * D + i] = acc[i] * inv;
  if (lse != nullptr) lse[(size_t)bh * N + row] = m_run * kLn2 + logf(l_run);
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
                     n_qtiles, BH, a.c, a.neg ? -1.0f : 1.0f);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_prefill_f32(const PrefillArgs& a, hipStream_t stream) {
  if (a.d == 128) return a.causal ? launch<128, true>(a, stream) : launch<128, false>(a, stream);
  if (a.d == 64) return a.causal ? launch<64, true>(a, stream) : launch<64, false>(a, stream);
  return hipErrorInvalidValue;
}

}  // namespace fa
