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
// Layout: a workgroup takes 16 query rows of one head; each of its 4, 8 or 16
// waves covers all 16 rows (4 lanes per row, each lane a quarter of d in
// interleaved 16-byte pieces) and takes every 4th (8th, 16th) 8-key batch of the keys,
// keeping its own running max, sum and output for the rows.  q and the output
// accumulator stay in registers (fp64); K and V rows come straight from
// memory, the 16 rows of a wave reading the same 16-byte pieces.  The
// waves' states are merged through LDS at the end with weights 2^(m_w - M)
// (the running-softmax rule applied to whole key subsets).  Small problems
// thus still spread over many waves: one head of 256 rows is 128 waves.
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

constexpr int kF32Rows = kPrefillF32Rows;  // query rows per workgroup
constexpr int kF32Batch = 8;   // keys per batch (one max and one rescale per batch)
// Waves per workgroup (SPLIT), each taking every SPLIT-th key batch: 8 while
// the grid is small (one head of 256 rows: 57 -> 36 us on MI355X), 16 for the
// smallest d = 64 grids, 4 for large grids, where at d = 128 the 8-wave form
// fits only one workgroup per CU (3-7% slower there).
constexpr int kF32SmallGrid = 4096;  // workgroups below which 8 waves are used
constexpr int kF32TinyGrid = 1024;   // d = 64: workgroups below which 16 waves are used

__device__ __forceinline__ double shfl_xor_d(double x, int m) { return __shfl_xor(x, m, 64); }

template <int D, bool CAUSAL, int SPLIT>
__global__ __launch_bounds__(64 * SPLIT) void prefill_f32_kernel(
    const float* __restrict__ q, const float* __restrict__ k, const float* __restrict__ v,
    float* __restrict__ o, float* __restrict__ lse, int Hq, int Hkv, int N, int n_qtiles, int BH,
    double cd, float qsign) {
  constexpr int kC = D / 16;  // 16-byte pieces of a row per lane
  constexpr int kL = D / 4;   // elements of a row per lane
  __shared__ double red_m[SPLIT][kF32Rows];
  __shared__ double red_l[SPLIT][kF32Rows];
  __shared__ double red_o[SPLIT][kF32Rows][D];
  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int rl = lane >> 2;   // row of the workgroup
  const int part = lane & 3;  // quarter of d: elements 16c + 4part + e
  const int bid = blockIdx.x;
  const int qtile = CAUSAL ? (n_qtiles - 1 - bid / BH) : (bid / BH);  // causal: long rows first
  const int bh = bid % BH;
  const int b = bh / Hq;
  const int h = bh - b * Hq;
  const int g = h / (Hq / Hkv);
  const float* kh = k + ((size_t)b * Hkv + g) * N * D;
  const float* vh = v + ((size_t)b * Hkv + g) * N * D;

  const int q0 = qtile * kF32Rows;
  const int row = q0 + rl;  // rows past N compute on row N-1 and are not stored
  double qd[kL];
  {
    const float* qr = q + ((size_t)bh * N + min(row, N - 1)) * D + 4 * part;
#pragma unroll
    for (int c = 0; c < kC; ++c) {
      const f32x4 x = *reinterpret_cast<const f32x4*>(qr + 16 * c);
#pragma unroll
      for (int e = 0; e < 4; ++e) qd[4 * c + e] = (double)(qsign * x[e]);
    }
  }
  double acc[kL];
#pragma unroll
  for (int i = 0; i < kL; ++i) acc[i] = 0.0;
  double m_run = -INFINITY;  // running max of c * (q . k), log2 units
  double l_run = 0.0;

  const int kv_end = CAUSAL ? min(N, q0 + kF32Rows) : N;
  const int nb = (kv_end + kF32Batch - 1) / kF32Batch;
  for (int bt = wave; bt < nb; bt += SPLIT) {
    const int k0 = bt * kF32Batch;
    // s[j] = q . k_j in fp64: a quarter of the terms per lane, then the
    // quarters summed across the row's 4 lanes (the same value in each)
    double s[kF32Batch];
#pragma unroll
    for (int j = 0; j < kF32Batch; ++j) {
      const int key = k0 + j;
      const float* kr = kh + (size_t)min(key, N - 1) * D + 4 * part;
      double a = 0.0;
#pragma unroll
      for (int c = 0; c < kC; ++c) {
        const f32x4 x = *reinterpret_cast<const f32x4*>(kr + 16 * c);
#pragma unroll
        for (int e = 0; e < 4; ++e) a = fma(qd[4 * c + e], (double)x[e], a);
      }
      a += shfl_xor_d(a, 1);
      a += shfl_xor_d(a, 2);
      const bool masked = key >= N || (CAUSAL && key > row);
      s[j] = masked ? -INFINITY : a;
    }
    double mx = -INFINITY;
#pragma unroll
    for (int j = 0; j < kF32Batch; ++j) mx = fmax(mx, s[j]);
    const double mn = fmax(m_run, mx * cd);
    // a row that has seen no key yet keeps m = -inf, l = 0, o = 0
    const double mref = mn == -INFINITY ? 0.0 : mn;
    const double alpha = (double)exp2f((float)(m_run - mref));
    l_run *= alpha;
#pragma unroll
    for (int i = 0; i < kL; ++i) acc[i] *= alpha;
    m_run = mn;
#pragma unroll
    for (int j = 0; j < kF32Batch; ++j) {
      const double p = (double)exp2f((float)fma(s[j], cd, -mref));
      l_run += p;
      const float* vr = vh + (size_t)min(k0 + j, N - 1) * D + 4 * part;
#pragma unroll
      for (int c = 0; c < kC; ++c) {
        const f32x4 x = *reinterpret_cast<const f32x4*>(vr + 16 * c);
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[4 * c + e] = fma(p, (double)x[e], acc[4 * c + e]);
      }
    }
  }

  // merge the waves' states of each row
  if (part == 0) {
    red_m[wave][rl] = m_run;
    red_l[wave][rl] = l_run;
  }
#pragma unroll
  for (int c = 0; c < kC; ++c)
#pragma unroll
    for (int e = 0; e < 4; ++e) red_o[wave][rl][16 * c + 4 * part + e] = acc[4 * c + e];
  __syncthreads();
  constexpr int kTPR = 64 * SPLIT / kF32Rows;  // merge threads per row
  static_assert(D % kTPR == 0, "a row's columns split evenly over its threads");
  const int rr = tid / kTPR;  // columns cc, cc + kTPR, ...
  const int cc = tid % kTPR;
  const int orow = q0 + rr;
  if (orow >= N) return;
  double M = red_m[0][rr];
#pragma unroll
  for (int w = 1; w < SPLIT; ++w) M = fmax(M, red_m[w][rr]);  // finite: wave 0 saw key 0
  double wgt[SPLIT];
  double l = 0.0;
#pragma unroll
  for (int w = 0; w < SPLIT; ++w) {
    wgt[w] = exp2(red_m[w][rr] - M);  // 0 for a wave that saw none of the row's keys
    l += wgt[w] * red_l[w][rr];
  }
  const double inv = 1.0 / l;
  float* orow_p = o + ((size_t)bh * N + orow) * D;
#pragma unroll
  for (int i = 0; i < D / kTPR; ++i) {
    const int col = cc + kTPR * i;
    double a = 0.0;
#pragma unroll
    for (int w = 0; w < SPLIT; ++w) a = fma(wgt[w], red_o[w][rr][col], a);
    orow_p[col] = (float)(a * inv);
  }
  if (lse != nullptr && cc == 0) lse[(size_t)bh * N + orow] = (float)(M * 0.6931471805599453 + log(l));
}

// c = |scale| log2(e) in fp64, clamped below at kMinC as the bf16 kernels' c is
// (so that c * (-inf) stays -inf at a zero scale)
double f32_coeff(float scale_abs) {
  const double c = (double)scale_abs * 1.4426950408889634074;
  return c < (double)kMinC ? (double)kMinC : c;
}

template <int D, bool CAUSAL, int SPLIT>
hipError_t launch_split(const PrefillArgs& a, hipStream_t stream, int n_qtiles, int BH, unsigned blocks) {
  hipLaunchKernelGGL((prefill_f32_kernel<D, CAUSAL, SPLIT>), dim3(blocks), dim3(64 * SPLIT), 0, stream,
                     static_cast<const float*>(a.q), static_cast<const float*>(a.k),
                     static_cast<const float*>(a.v), static_cast<float*>(a.o), a.lse, a.Hq, a.Hkv, a.N,
                     n_qtiles, BH, f32_coeff(a.scale_abs), a.neg ? -1.0f : 1.0f);
  return hipGetLastError();
}

template <int D, bool CAUSAL>
hipError_t launch(const PrefillArgs& a, hipStream_t stream) {
  const int n_qtiles = (a.N + kF32Rows - 1) / kF32Rows;
  const int BH = a.B * a.Hq;
  const long long blocks = (long long)n_qtiles * BH;
  if (blocks > 0x7fffffffLL) return hipErrorInvalidValue;
  if constexpr (D == 64) {
    // at d = 64 sixteen waves fit a CU (128 VGPRs, a 132 KB merge buffer)
    if (blocks < kF32TinyGrid) return launch_split<D, CAUSAL, 16>(a, stream, n_qtiles, BH, (unsigned)blocks);
  }
  return blocks < kF32SmallGrid ? launch_split<D, CAUSAL, 8>(a, stream, n_qtiles, BH, (unsigned)blocks)
                                : launch_split<D, CAUSAL, 4>(a, stream, n_qtiles, BH, (unsigned)blocks);
}

}  // namespace

hipError_t launch_prefill_f32(const PrefillArgs& a, hipStream_t stream) {
  if (a.d == 128) return a.causal ? launch<128, true>(a, stream) : launch<128, false>(a, stream);
  if (a.d == 64) return a.causal ? launch<64, true>(a, stream) : launch<64, false>(a, stream);
  return hipErrorInvalidValue;
}

}  // namespace fa
