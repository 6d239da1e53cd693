// Decode: one new query token per sequence against its contiguous KV cache.
//
// Generating a token re-reads the sequence's whole cache including the new
// entry, so the cost is linear in cache length and the step is bound by
// memory bandwidth (forum comment item 45450456, paragraphs on KV caching and
// on its implications; forum thread item 42793451 on causal LMs being memory
// bound at inference).  The cache is retained by the caller and only read
// here ("How Does Flash Attention Reduce Memory Traffic During Local
// Inference?", "Reduced IO Is Not the Same as Eliminating KV Cache").
//
// Split-KV design for gfx950:
//   kernel 1 (split): one workgroup per (sequence, key/value head, query-head
//     slice, 512-key chunk).  Every K/V byte of the chunk is read from HBM
//     exactly once and used for all query heads of the GQA group ("Optimizing
//     memory requirements for inference in large language models", GQA
//     paragraph).  Scores: 4 lanes per cache row (64 contiguous bytes each),
//     all loads of a pass issued before use; values: 16 lanes per row.  The
//     chunk's softmax statistics are reduced in-wave and across waves in
//     LDS.  Output per chunk: its normalised partial o_s and its log-sum-exp.
//   kernel 2 (combine): per (sequence, query head), the partials are merged
//     with weights exp(lse_s - max lse) -- the running-softmax rule applied to
//     whole chunks ("11.4d FlashAttention", "Online Softmax").
// seqlens is read only on the device; chunks at or past a sequence's length
// exit at once, rows past the length are never loaded.
#include "common.h"
#include "kernels.h"

namespace fa {
namespace {

constexpr int kChunk = kDecodeChunk;  // keys per split
constexpr int kWaves = 4;
constexpr int kRowsPerWave = kChunk / kWaves;  // 128

template <typename T>
struct Elem;
template <>
struct Elem<uint16_t> {  // bf16 storage
  static constexpr int kPer16B = 8;
  __device__ static inline void widen(const u32x4& w, float* f) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f[2 * i] = bf16lo_to_f32(w[i]);
      f[2 * i + 1] = bf16hi_to_f32(w[i]);
    }
  }
  __device__ static inline float load1(const uint16_t* p) { return __uint_as_float((uint32_t)(*p) << 16); }
  __device__ static inline void store1(uint16_t* p, float x) {
    *p = (uint16_t)(pack_bf16x2(x, 0.f) & 0xffffu);
  }
};
template <>
struct Elem<float> {
  static constexpr int kPer16B = 4;
  __device__ static inline void widen(const u32x4& w, float* f) {
#pragma unroll
    for (int i = 0; i < 4; ++i) f[i] = __uint_as_float(w[i]);
  }
  __device__ static inline float load1(const float* p) { return *p; }
  __device__ static inline void store1(float* p, float x) { *p = x; }
};

__device__ __forceinline__ float shfl_xor_f(float x, int m) { return __shfl_xor(x, m, 64); }

// grid: x = chunk index, y = kv head * (G/GT) + head slice, z = sequence.
template <typename T, int D, int GT>
__global__ __launch_bounds__(256) void decode_split_kernel(
    const T* __restrict__ q, const T* __restrict__ kc, const T* __restrict__ vc,
    const int32_t* __restrict__ seqlens, float* __restrict__ part_o, float* __restrict__ part_lse,
    int Hq, int Hkv, int maxlen, int nsplit, float c, float qsign) {
  using E = Elem<T>;
  constexpr int kE = E::kPer16B;            // elements per 16-byte load
  constexpr int kLaneElems = D / 4;         // score phase: d-range per lane
  constexpr int kSLoads = kLaneElems / kE;  // 16-byte loads per row per lane
  constexpr int kVLanes = D / kE;           // value phase: lanes per row
  constexpr int kVSlots = 64 / kVLanes;     // rows per wave per pass
  static_assert(64 % kVLanes == 0, "row must split over lanes");

  __shared__ float p_lds[kChunk][GT];
  __shared__ float red_m[kWaves][GT];
  __shared__ float red_l[kWaves][GT];
  __shared__ float o_lds[kWaves][GT][D];

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int split = blockIdx.x;
  const int G = Hq / Hkv;
  const int slices = G / GT;
  const int kvh = blockIdx.y / slices;
  const int h0 = kvh * G + (blockIdx.y % slices) * GT;
  const int b = blockIdx.z;

  const int L = min(max(seqlens[b], 0), maxlen);
  const int kbeg = split * kChunk;
  if (kbeg >= L) return;
  const int n = min(kChunk, L - kbeg);

  const size_t cbase = (((size_t)b * Hkv + kvh) * maxlen + kbeg) * D;
  const T* kp = kc + cbase;
  const T* vp = vc + cbase;

  // ---------------- scores: 4 lanes per row ----------------
  const int rs = lane >> 2;  // row slot 0..15
  const int jq = lane & 3;   // quarter of the row
  float qv[GT][kLaneElems];
#pragma unroll
  for (int g = 0; g < GT; ++g) {
    const T* qrow = q + ((size_t)b * Hq + h0 + g) * D;
#pragma unroll
    for (int cc = 0; cc < kSLoads; ++cc)
#pragma unroll
      for (int e = 0; e < kE; ++e)
        qv[g][cc * kE + e] = qsign * E::load1(qrow + cc * (4 * kE) + jq * kE + e);
  }

  constexpr int kPasses = kRowsPerWave / 16;  // 8 passes of 16 rows per wave
  // passes whose loads are issued together (<= 128 VGPRs of loads in flight)
  constexpr int kSB = (32 / kSLoads) < kPasses ? (32 / kSLoads) : kPasses;
  static_assert(kPasses % kSB == 0, "score passes must batch evenly");
  float sc[kPasses][GT];
#pragma unroll
  for (int p0 = 0; p0 < kPasses; p0 += kSB) {
    u32x4 buf[kSB][kSLoads];
#pragma unroll
    for (int i = 0; i < kSB; ++i) {
      const int row = wave * kRowsPerWave + (p0 + i) * 16 + rs;
#pragma unroll
      for (int cc = 0; cc < kSLoads; ++cc) {
        if (row < n)
          buf[i][cc] = *reinterpret_cast<const u32x4*>(kp + (size_t)row * D + cc * (4 * kE) + jq * kE);
        else
          buf[i][cc] = u32x4{0u, 0u, 0u, 0u};
      }
    }
#pragma unroll
    for (int i = 0; i < kSB; ++i) {
      float acc[GT];
#pragma unroll
      for (int g = 0; g < GT; ++g) acc[g] = 0.f;
#pragma unroll
      for (int cc = 0; cc < kSLoads; ++cc) {
        float kf[kE];
        E::widen(buf[i][cc], kf);
#pragma unroll
        for (int e = 0; e < kE; ++e)
#pragma unroll
          for (int g = 0; g < GT; ++g) acc[g] = fmaf(kf[e], qv[g][cc * kE + e], acc[g]);
      }
      const int row = wave * kRowsPerWave + (p0 + i) * 16 + rs;
#pragma unroll
      for (int g = 0; g < GT; ++g) {
        float a = acc[g];
        a += shfl_xor_f(a, 1);
        a += shfl_xor_f(a, 2);
        sc[p0 + i][g] = row < n ? a * c : -INFINITY;
      }
    }
  }

  // chunk max per head
  float mloc[GT];
#pragma unroll
  for (int g = 0; g < GT; ++g) {
    float mx = -INFINITY;
#pragma unroll
    for (int p = 0; p < kPasses; ++p) mx = fmaxf(mx, sc[p][g]);
    mx = fmaxf(mx, shfl_xor_f(mx, 4));
    mx = fmaxf(mx, shfl_xor_f(mx, 8));
    mx = fmaxf(mx, shfl_xor_f(mx, 16));
    mx = fmaxf(mx, shfl_xor_f(mx, 32));
    mloc[g] = mx;
  }
  if (lane == 0) {
#pragma unroll
    for (int g = 0; g < GT; ++g) red_m[wave][g] = mloc[g];
  }
  __syncthreads();
  float M[GT];
#pragma unroll
  for (int g = 0; g < GT; ++g) {
    float mx = red_m[0][g];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) mx = fmaxf(mx, red_m[w][g]);
    M[g] = mx;  // finite: the chunk has at least one row
  }
  // probabilities to LDS, partial sums
  float lpart[GT];
#pragma unroll
  for (int g = 0; g < GT; ++g) lpart[g] = 0.f;
#pragma unroll
  for (int p = 0; p < kPasses; ++p) {
    const int row = wave * kRowsPerWave + p * 16 + rs;
#pragma unroll
    for (int g = 0; g < GT; ++g) {
      const float e = fast_exp2(sc[p][g] - M[g]);
      if (jq == 0) {
        p_lds[row][g] = e;
        lpart[g] += e;
      }
    }
  }
#pragma unroll
  for (int g = 0; g < GT; ++g) {
    float s = lpart[g];
    s += shfl_xor_f(s, 4);
    s += shfl_xor_f(s, 8);
    s += shfl_xor_f(s, 16);
    s += shfl_xor_f(s, 32);
    if (lane == 0) red_l[wave][g] = s;
  }
  __syncthreads();

  // ---------------- values: kVLanes lanes per row ----------------
  const int vs = lane / kVLanes;  // row slot
  const int vd = lane % kVLanes;  // 16-byte column
  float oacc[GT][kE];
#pragma unroll
  for (int g = 0; g < GT; ++g)
#pragma unroll
    for (int e = 0; e < kE; ++e) oacc[g][e] = 0.f;
  constexpr int kVPasses = kRowsPerWave / kVSlots;
  constexpr int kBatch = 16;
  static_assert(kVPasses % kBatch == 0, "value passes must batch evenly");
#pragma unroll 1
  for (int p0 = 0; p0 < kVPasses; p0 += kBatch) {
    u32x4 vb[kBatch];
#pragma unroll
    for (int i = 0; i < kBatch; ++i) {
      const int row = wave * kRowsPerWave + (p0 + i) * kVSlots + vs;
      if (row < n)
        vb[i] = *reinterpret_cast<const u32x4*>(vp + (size_t)row * D + vd * kE);
      else
        vb[i] = u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int i = 0; i < kBatch; ++i) {
      const int row = wave * kRowsPerWave + (p0 + i) * kVSlots + vs;
      if (row < n) {
        float vf[kE];
        E::widen(vb[i], vf);
#pragma unroll
        for (int g = 0; g < GT; ++g) {
          const float pg = p_lds[row][g];
#pragma unroll
          for (int e = 0; e < kE; ++e) oacc[g][e] = fmaf(pg, vf[e], oacc[g][e]);
        }
      }
    }
  }
  // reduce over row slots inside the wave (lanes differing in the slot bits)
#pragma unroll
  for (int g = 0; g < GT; ++g)
#pragma unroll
    for (int e = 0; e < kE; ++e) {
      float a = oacc[g][e];
#pragma unroll
      for (int m = kVLanes; m < 64; m <<= 1) a += shfl_xor_f(a, m);
      oacc[g][e] = a;
    }
  if (vs == 0) {
#pragma unroll
    for (int g = 0; g < GT; ++g)
#pragma unroll
      for (int e = 0; e < kE; ++e) o_lds[wave][g][vd * kE + e] = oacc[g][e];
  }
  __syncthreads();
  // final: thread t handles (g, d) pairs
  for (int i = tid; i < GT * D; i += 256) {
    const int g = i / D, d = i % D;
    float l = 0.f, a = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      l += red_l[w][g];
      a += o_lds[w][g][d];
    }
    const size_t pidx = ((size_t)b * Hq + h0 + g) * nsplit + split;
    part_o[pidx * D + d] = a / l;
    if (d == 0) part_lse[pidx] = M[g] * kLn2 + __logf(l);
  }
}

// grid: x = query head, y = sequence; block = D threads.
template <typename T, int D>
__global__ __launch_bounds__(128) void decode_combine_kernel(
    const float* __restrict__ part_o, const float* __restrict__ part_lse,
    const int32_t* __restrict__ seqlens, T* __restrict__ o, int Hq, int maxlen, int nsplit) {
  using E = Elem<T>;
  const int h = blockIdx.x, b = blockIdx.y;
  const int L = min(max(seqlens[b], 0), maxlen);
  const int ns = (L + kChunk - 1) / kChunk;
  const size_t base = ((size_t)b * Hq + h) * nsplit;
  for (int d = threadIdx.x; d < D; d += blockDim.x) {
    float out = 0.f;
    if (ns > 0) {
      float mx = -INFINITY;
      for (int s = 0; s < ns; ++s) mx = fmaxf(mx, part_lse[base + s]);
      float wsum = 0.f, acc = 0.f;
      for (int s = 0; s < ns; ++s) {
        const float w = __expf(part_lse[base + s] - mx);
        wsum += w;
        acc = fmaf(w, part_o[(base + s) * D + d], acc);
      }
      out = acc / wsum;
    }
    E::store1(o + ((size_t)b * Hq + h) * D + d, out);
  }
}

template <typename T, int D, int GT>
hipError_t launch_t(const DecodeArgs& a, hipStream_t stream) {
  const int nsplit = (a.maxlen + kChunk - 1) / kChunk;
  const int G = a.Hq / a.Hkv;
  float* part_o = static_cast<float*>(a.ws);
  const size_t po_bytes = (size_t)a.B * a.Hq * nsplit * D * sizeof(float);
  float* part_lse = reinterpret_cast<float*>(static_cast<char*>(a.ws) + ((po_bytes + 255) & ~(size_t)255));
  dim3 g1(nsplit, a.Hkv * (G / GT), a.B);
  if (g1.y > 65535u || g1.z > 65535u) return hipErrorInvalidValue;
  hipLaunchKernelGGL((decode_split_kernel<T, D, GT>), g1, dim3(256), 0, stream, static_cast<const T*>(a.q),
                     static_cast<const T*>(a.k), static_cast<const T*>(a.v), a.seqlens, part_o, part_lse,
                     a.Hq, a.Hkv, a.maxlen, nsplit, a.c, a.neg ? -1.0f : 1.0f);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((decode_combine_kernel<T, D>), dim3(a.Hq, a.B), dim3(128), 0, stream, part_o, part_lse,
                     a.seqlens, static_cast<T*>(a.o), a.Hq, a.maxlen, nsplit);
  return hipGetLastError();
}

template <typename T, int D>
hipError_t launch_g(const DecodeArgs& a, hipStream_t stream) {
  const int G = a.Hq / a.Hkv;
  if (G % 4 == 0) return launch_t<T, D, 4>(a, stream);
  if (G % 2 == 0) return launch_t<T, D, 2>(a, stream);
  return launch_t<T, D, 1>(a, stream);
}

}  // namespace

size_t decode_workspace_bytes(int B, int Hq, int maxlen, int d) {
  const size_t nsplit = ((size_t)maxlen + kChunk - 1) / kChunk;
  const size_t po = (size_t)B * Hq * nsplit * d * sizeof(float);
  const size_t pl = (size_t)B * Hq * nsplit * sizeof(float);
  return ((po + 255) & ~(size_t)255) + ((pl + 255) & ~(size_t)255);
}

hipError_t launch_decode_bf16(const DecodeArgs& a, hipStream_t stream) {
  if (a.d == 128) return launch_g<uint16_t, 128>(a, stream);
  if (a.d == 64) return launch_g<uint16_t, 64>(a, stream);
  return hipErrorInvalidValue;
}

hipError_t launch_decode_f32(const DecodeArgs& a, hipStream_t stream) {
  if (a.d == 128) return launch_g<float, 128>(a, stream);
  if (a.d == 64) return launch_g<float, 64>(a, stream);
  return hipErrorInvalidValue;
}

}  // namespace fa
