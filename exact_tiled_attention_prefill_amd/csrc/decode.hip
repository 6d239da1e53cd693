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
//     slice, chunk of keys).  Every K/V byte of the chunk is read from HBM
//     exactly once and used for all query heads of the GQA group ("Optimizing
//     memory requirements for inference in large language models", GQA
//     paragraph).  Output per chunk: its normalised partial o_s and its
//     log-sum-exp.
//     bf16 path (chunks of 4096, 2048, 1024, 512 or 256 keys, the largest
//       that still gives 1024 workgroups): one workgroup serves the whole GQA
//       group
//       (up to 32 query heads).  Each of its four waves streams its own
//       32-key tiles of the chunk through a private two-slot LDS ring, copied
//       HBM -> LDS by global_load_lds_dwordx4 (no VGPR staging, no per-tile
//       barrier), and computes S^T = K Q^T and O^T += V^T P^T on
//       v_mfma_f32_32x32x16_bf16 with the group's heads as the columns -- the
//       prefill kernel's register and LDS layouts.  The products cost the same
//       per key whatever the number of heads, so the group's K/V is read once
//       and the matrix cores stay far below their rate at HBM speed.  Each
//       wave keeps its own running max / sum per head (lazy rescale); the
//       four waves are merged once per chunk through LDS.
//     Each (sequence, head) row's chunk order is rotated by the row index so
//     that the XCDs receive equal shares of real chunks.
//     fp32 path (512-key chunks, up to 4 query heads per workgroup): VGPR
//       loads, 8 lanes per row for scores and 16 (or 32) lanes per row for
//       values; the score dot products, chunk max, probability sum and P.V
//       sums are taken in fp64 (fp32 inputs, fp32 probabilities from exp2f)
//       and the chunk log-sum-exps stored in fp64, so that rounding stays far
//       below fp32 output tolerance even where large scores amplify it.  The
//       fp64 scores of a chunk are kept in LDS, which leaves registers for two
//       waves per SIMD.
//     Both paths load the cache with the non-temporal hint: every byte is read
//     once, and marking its lines evict-first raised the bf16 split kernel
//     from ~5.6 to ~6.0 TB/s on MI355X (a plain read stream reaches ~6.3 TB/s,
//     a non-temporal one ~6.8).
//   kernel 2 (combine): per (sequence, query head), the partials are merged
//     with weights exp(lse_s - max lse) -- the running-softmax rule applied to
//     whole chunks ("11.4d FlashAttention", "Online Softmax"); every load in
//     it is independent of the others, so a sequence's partials stream in at
//     once.
// seqlens is read only on the device; chunks at or past a sequence's length
// exit at once, rows past the length are never loaded.
#include <mutex>
#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace fa {
namespace {

constexpr int kChunk = kDecodeChunk;  // keys per split of the fp32 path
constexpr int kWaves = 4;
constexpr int kRowsPerWave = kChunk / kWaves;  // 128

// Bytes of the split-KV partials ([B,Hq,nsplit,d] fp32 outputs, then
// [B,Hq,nsplit] log-sum-exps of lse_bytes each -- fp64 on the fp32 path, fp32
// on the bf16 path -- each padded to 256 bytes) for a chunk size.
size_t partials_bytes(int B, int Hq, int maxlen, int d, int chunk, size_t lse_bytes) {
  const size_t nsplit = ((size_t)maxlen + chunk - 1) / chunk;
  const size_t po = (size_t)B * Hq * nsplit * d * sizeof(float);
  const size_t pl = (size_t)B * Hq * nsplit * lse_bytes;
  return ((po + 255) & ~(size_t)255) + ((pl + 255) & ~(size_t)255);
}

// Chunk handled by this workgroup.  Workgroups go to the 8 XCDs round-robin
// by linear id, with x (the split) fastest, and only a prefix of each
// (sequence, head) row's splits has keys -- a prefix whose length varies by
// sequence.  Without a rotation, split s of every row lands on XCD s % 8 when
// the split count is a multiple of 8, so the low XCDs get every row's odd
// remainder (about 10% more work than the average for uniform random
// lengths); rotating each row's chunk order by its row index spreads them.
__device__ __forceinline__ int split_of_block(int nsplit) {
  const int row = blockIdx.y + gridDim.y * blockIdx.z;
  return (nsplit & 7) == 0 ? (int)((blockIdx.x + (unsigned)row) % (unsigned)nsplit) : (int)blockIdx.x;
}

template <typename T>
struct Elem;
template <>
struct Elem<uint16_t> {  // bf16 storage: only the combine's output store
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

// Log-sum-exp of a chunk partial: fp64 on the fp32 path (at |lse| above 128
// the fp32 half-ulp, 7.6e-6, moves the combine's weights by as much, which a
// sharp softmax carries into the output), fp32 on the bf16 path.
template <typename T>
using LseT = typename std::conditional<std::is_same<T, float>::value, double, float>::type;

__device__ __forceinline__ float shfl_xor_f(float x, int m) { return __shfl_xor(x, m, 64); }
__device__ __forceinline__ double shfl_xor_d(double x, int m) { return __shfl_xor(x, m, 64); }

// grid: x = chunk index, y = kv head * (G/GT) + head slice, z = sequence.
template <typename T, int D, int GT>
__global__ __launch_bounds__(256) void decode_split_kernel(
    const T* __restrict__ q, const T* __restrict__ kc, const T* __restrict__ vc,
    const int32_t* __restrict__ seqlens, float* __restrict__ part_o, LseT<T>* __restrict__ part_lse,
    int Hq, int Hkv, int maxlen, int nsplit, float c, float qsign) {
  using E = Elem<T>;
  constexpr int kE = E::kPer16B;            // elements per 16-byte load
  constexpr int kSL = 8;                    // score phase: lanes per row
  constexpr int kRowSlots = 64 / kSL;       // score phase: rows per wave per pass
  constexpr int kLaneElems = D / kSL;       // score phase: d-range per lane
  constexpr int kSLoads = kLaneElems / kE;  // 16-byte loads per row per lane
  constexpr int kVLanes = D / kE;           // value phase: lanes per row
  constexpr int kVSlots = 64 / kVLanes;     // rows per wave per pass
  static_assert(64 % kVLanes == 0, "row must split over lanes");

  __shared__ double s_lds[kChunk][GT];  // scores c * (q . k), log2 units
  __shared__ float p_lds[kChunk][GT];
  __shared__ double red_m[kWaves][GT];
  __shared__ double red_l[kWaves][GT];
  __shared__ double o_lds[kWaves][GT][D];

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int split = split_of_block(nsplit);
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

  // ---------------- scores: kSL lanes per row ----------------
  const int rs = lane / kSL;  // row slot
  const int jq = lane % kSL;  // the lane's 16-byte pieces of the row: jq, jq + kSL, ...
  float qv[GT][kLaneElems];
#pragma unroll
  for (int g = 0; g < GT; ++g) {
    const T* qrow = q + ((size_t)b * Hq + h0 + g) * D;
#pragma unroll
    for (int cc = 0; cc < kSLoads; ++cc)
#pragma unroll
      for (int e = 0; e < kE; ++e)
        qv[g][cc * kE + e] = qsign * E::load1(qrow + cc * (kSL * kE) + jq * kE + e);
  }

  constexpr int kPasses = kRowsPerWave / kRowSlots;  // 16 passes of 8 rows per wave
  // passes whose loads are issued together (64 VGPRs of loads in flight)
  constexpr int kSB = (16 / kSLoads) < kPasses ? (16 / kSLoads) : kPasses;
  static_assert(kPasses % kSB == 0, "score passes must batch evenly");
  double mloc[GT];  // running chunk max per head (the same in the kSL lanes of a row)
#pragma unroll
  for (int g = 0; g < GT; ++g) mloc[g] = -INFINITY;
  // one batch of loads at a time (not unrolled: the scores go to LDS, and an
  // unrolled loop lets later batches' loads move up and spill), and only the
  // batches that hold rows of the chunk (wave-uniform)
  const int wave_rows = min(max(n - wave * kRowsPerWave, 0), kRowsPerWave);
  const int n_pass = (wave_rows + kRowSlots - 1) / kRowSlots;
#pragma unroll 1
  for (int p0 = 0; p0 < n_pass; p0 += kSB) {
    u32x4 buf[kSB][kSLoads];
#pragma unroll
    for (int i = 0; i < kSB; ++i) {
      const int row = wave * kRowsPerWave + (p0 + i) * kRowSlots + rs;
#pragma unroll
      for (int cc = 0; cc < kSLoads; ++cc) {
        if (row < n)
          buf[i][cc] = __builtin_nontemporal_load(
              reinterpret_cast<const u32x4*>(kp + (size_t)row * D + cc * (kSL * kE) + jq * kE));
        else
          buf[i][cc] = u32x4{0u, 0u, 0u, 0u};
      }
    }
#pragma unroll
    for (int i = 0; i < kSB; ++i) {
      double acc[GT];
#pragma unroll
      for (int g = 0; g < GT; ++g) acc[g] = 0.0;
#pragma unroll
      for (int cc = 0; cc < kSLoads; ++cc) {
        float kf[kE];
        E::widen(buf[i][cc], kf);
#pragma unroll
        for (int e = 0; e < kE; ++e)
#pragma unroll
          for (int g = 0; g < GT; ++g) acc[g] = fma((double)kf[e], (double)qv[g][cc * kE + e], acc[g]);
      }
      const int row = wave * kRowsPerWave + (p0 + i) * kRowSlots + rs;
#pragma unroll
      for (int g = 0; g < GT; ++g) {
        double a = acc[g];
#pragma unroll
        for (int m = 1; m < kSL; m <<= 1) a += shfl_xor_d(a, m);
        const double sv = row < n ? a * (double)c : -INFINITY;
        mloc[g] = fmax(mloc[g], sv);
        if (jq == 0) s_lds[row][g] = sv;
      }
    }
  }

  // chunk max per head
#pragma unroll
  for (int g = 0; g < GT; ++g) {
    double mx = mloc[g];
#pragma unroll
    for (int m = kSL; m < 64; m <<= 1) mx = fmax(mx, shfl_xor_d(mx, m));
    mloc[g] = mx;
  }
  if (lane == 0) {
#pragma unroll
    for (int g = 0; g < GT; ++g) red_m[wave][g] = mloc[g];
  }
  __syncthreads();
  double M[GT];
#pragma unroll
  for (int g = 0; g < GT; ++g) {
    double mx = red_m[0][g];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) mx = fmax(mx, red_m[w][g]);
    M[g] = mx;  // finite: the chunk has at least one row
  }
  // probabilities to LDS, partial sums: each lane takes rows lane and
  // lane + 64 of its wave's (rows past the length give 0; their scores were
  // written only up to the end of their batch)
  double lpart[GT];
#pragma unroll
  for (int g = 0; g < GT; ++g) lpart[g] = 0.0;
#pragma unroll
  for (int i = 0; i < kRowsPerWave / 64; ++i) {
    const int row = wave * kRowsPerWave + i * 64 + lane;
#pragma unroll
    for (int g = 0; g < GT; ++g) {
      const float e = row < n ? exp2f((float)(s_lds[row][g] - M[g])) : 0.f;
      p_lds[row][g] = e;
      lpart[g] += e;
    }
  }
#pragma unroll
  for (int g = 0; g < GT; ++g) {
    double s = lpart[g];
    s += shfl_xor_d(s, 1);
    s += shfl_xor_d(s, 2);
    s += shfl_xor_d(s, 4);
    s += shfl_xor_d(s, 8);
    s += shfl_xor_d(s, 16);
    s += shfl_xor_d(s, 32);
    if (lane == 0) red_l[wave][g] = s;
  }
  __syncthreads();

  // ---------------- values: kVLanes lanes per row ----------------
  const int vs = lane / kVLanes;  // row slot
  const int vd = lane % kVLanes;  // 16-byte column
  double oacc[GT][kE];
#pragma unroll
  for (int g = 0; g < GT; ++g)
#pragma unroll
    for (int e = 0; e < kE; ++e) oacc[g][e] = 0.0;
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
        vb[i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(vp + (size_t)row * D + vd * kE));
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
          for (int e = 0; e < kE; ++e) oacc[g][e] = fma((double)pg, (double)vf[e], oacc[g][e]);
        }
      }
    }
  }
  // reduce over row slots inside the wave (lanes differing in the slot bits)
#pragma unroll
  for (int g = 0; g < GT; ++g)
#pragma unroll
    for (int e = 0; e < kE; ++e) {
      double a = oacc[g][e];
#pragma unroll
      for (int m = kVLanes; m < 64; m <<= 1) a += shfl_xor_d(a, m);
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
    double l = 0.0, a = 0.0;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      l += red_l[w][g];
      a += o_lds[w][g][d];
    }
    const size_t pidx = ((size_t)b * Hq + h0 + g) * nsplit + split;
    part_o[pidx * D + d] = (float)(a / l);
    if (d == 0) part_lse[pidx] = (LseT<T>)(M[g] * 0.6931471805599453 + log(l));
  }
}

// grid: x = query head, y = sequence; block = 256 threads.
// The chunk partials of one (sequence, query head) are merged with weights
// exp(lse_s - max lse).  All loads are independent of one another: the max
// is a strided block reduction, the weights go through LDS in batches, and
// thread group sg (256 / D groups of D threads, one column each) accumulates
// splits sg, sg + 256/D, ... with unrolled, coalesced row loads.
constexpr int kCombThreads = 256;
constexpr int kCombBatch = 1024;  // weights staged in LDS per batch

template <typename T, int D>
__global__ __launch_bounds__(kCombThreads) void decode_combine_kernel(
    const float* __restrict__ part_o, const LseT<T>* __restrict__ part_lse,
    const int32_t* __restrict__ seqlens, T* __restrict__ o, int Hq, int maxlen, int nsplit, int chunk) {
  using E = Elem<T>;
  using L_ = LseT<T>;
  constexpr int NG = kCombThreads / D;  // split groups
  __shared__ float w_lds[kCombBatch];
  __shared__ L_ red_mx[kCombThreads / 64];
  __shared__ float red[kCombThreads / 64];
  __shared__ float acc_lds[NG][D];
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int h = blockIdx.x, b = blockIdx.y;
  const int L = min(max(seqlens[b], 0), maxlen);
  const int ns = (L + chunk - 1) / chunk;
  T* orow = o + ((size_t)b * Hq + h) * D;
  if (ns == 0) {
    if (tid < D) E::store1(orow + tid, 0.f);
    return;
  }
  const size_t base = ((size_t)b * Hq + h) * nsplit;
  const L_* lse = part_lse + base;
  const float* po = part_o + base * D;

  // block max of the log-sum-exps
  L_ mx = -INFINITY;
  for (int s = tid; s < ns; s += kCombThreads) mx = fmax(mx, lse[s]);
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) mx = fmax(mx, (L_)__shfl_xor(mx, off, 64));
  if (lane == 0) red_mx[wave] = mx;
  __syncthreads();
  mx = red_mx[0];
#pragma unroll
  for (int w = 1; w < kCombThreads / 64; ++w) mx = fmax(mx, red_mx[w]);

  const int d = tid % D, sg = tid / D;
  float acc = 0.f, wpart = 0.f;
  for (int s0 = 0; s0 < ns; s0 += kCombBatch) {
    const int nb = min(kCombBatch, ns - s0);
    __syncthreads();  // previous batch's weights fully read (and red[] read above)
    for (int i = tid; i < nb; i += kCombThreads) {
      // the fp32 path takes the fp64 exponential of the fp64 difference, bf16
      // the fast one, whose error grows with |argument|
      float w;
      if constexpr (std::is_same<T, float>::value) w = (float)exp(lse[s0 + i] - mx);
      else w = __expf(lse[s0 + i] - mx);
      w_lds[i] = w;
      wpart += w;
    }
    __syncthreads();
    const float* pb = po + (size_t)s0 * D + d;
    int i = sg;
    for (; i + 3 * NG < nb; i += 4 * NG) {
      const float a0 = pb[(size_t)i * D];
      const float a1 = pb[(size_t)(i + NG) * D];
      const float a2 = pb[(size_t)(i + 2 * NG) * D];
      const float a3 = pb[(size_t)(i + 3 * NG) * D];
      acc = fmaf(w_lds[i], a0, acc);
      acc = fmaf(w_lds[i + NG], a1, acc);
      acc = fmaf(w_lds[i + 2 * NG], a2, acc);
      acc = fmaf(w_lds[i + 3 * NG], a3, acc);
    }
    for (; i < nb; i += NG) acc = fmaf(w_lds[i], pb[(size_t)i * D], acc);
  }
  // block sum of the weights, group sum of the accumulators
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) wpart += __shfl_xor(wpart, off, 64);
  __syncthreads();  // every thread is past its last read of red[] and w_lds
  if (lane == 0) red[wave] = wpart;
  acc_lds[sg][d] = acc;
  __syncthreads();
  if (tid < D) {
    float wsum = red[0];
#pragma unroll
    for (int w = 1; w < kCombThreads / 64; ++w) wsum += red[w];
    float a = acc_lds[0][tid];
#pragma unroll
    for (int g = 1; g < NG; ++g) a += acc_lds[g][tid];
    E::store1(orow + tid, a / wsum);
  }
}

// ---------------------------------------------------------------------------
// bf16 split kernel helpers.
constexpr float kTauB = 8.0f;   // lazy-rescale threshold (log2 units)

template <int n>
__device__ __forceinline__ void dec_wait_vmem_le() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(n) : "memory");
}
// lane l's 16 bytes from base + off land at lds_wave_base + 16*l (inline asm:
// the compiler does not track it; completion is ordered by vmcnt + barrier).
// The copies carry the non-temporal hint (nt): the cache is read once.
// The compiler applies no hazard rule to inline asm: s_nop 0 gives the m0
// write just before the copy its one wait state, and the build checks the
// generated code for a VALU write of the base SGPRs fewer than 5 wait
// states before a copy (isa_check.py).
__device__ __forceinline__ void dec_dma16(const void* base, uint32_t off, uint8_t* lds_wave_base) {
  const uint32_t m0 = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) uint8_t*)lds_wave_base;
  asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, %2 nt" ::"v"(off), "{m0}"(m0), "s"(base) : "memory");
}
// the same copy from a per-lane 64-bit address (paged caches: the rows of one
// stage may come from different pages)
__device__ __forceinline__ void dec_dma16_addr(const void* addr, uint8_t* lds_wave_base) {
  const uint32_t m0 = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) uint8_t*)lds_wave_base;
  asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, off nt" ::"v"(addr), "{m0}"(m0) : "memory");
}
// Longest bf16 chunk (keys), and the most pool pages one chunk touches: its
// keys over pages of >= 16 keys, plus one page for a chunk that does not start
// on a page boundary.
constexpr int kMaxChunkB = 4096;
constexpr int kMaxChunkPages = kMaxChunkB / 16 + 1;
typedef short dec_i16x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ u32x2 dec_read_tr(const uint8_t* p) {
  typedef __attribute__((address_space(3))) dec_i16x4 lds_t;
  return __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_t*)(p)));
}
// ---------------------------------------------------------------------------
// bf16 split kernel: matrix cores.  S^T = K Q^T and O^T += V^T P^T run on
// v_mfma_f32_32x32x16_bf16 with the query heads of one GQA group (up to 32)
// as the columns; unused columns hold zero queries.  The products cost the
// same per key whatever the number of heads, so every K/V byte is read once
// for the whole group and the matrix cores stay far below their rate at HBM
// speed.  (A VALU kernel with v_dot2_f32_bf16 grew with the heads served and
// saturated from 8 heads on.)  Each wave streams its own 32-key tiles (tiles
// w, w+4, ... of the chunk) through a private two-slot LDS ring, so no
// barrier runs per tile; the four waves' (m, l, o) are merged once per chunk.
// The register and LDS layouts are those of the prefill kernel: K rows read
// with ds_read_b128 from 16-byte chunks XOR-swizzled by row, V read transposed
// with ds_read_b64_tr_b16, P packed from the accumulator into the B operand, a
// lazily rescaled running max per head.
template <int D>
__device__ __forceinline__ int mk_swz(int row) {  // K: 16 rows x one chunk per read
  return D == 128 ? (row & 15) : ((row >> 1) & 7);
}
template <int D>
__device__ __forceinline__ int mv_swz(int row) {  // V: 4 rows x 4 chunks per transposed read
  return D == 128 ? 4 * (row & 3) : 4 * ((row >> 1) & 1);
}

// gm (1..32) query heads of one GQA group per workgroup: columns 0..gm-1.
template <int D, bool PAGED>
__global__ __launch_bounds__(256, D >= 128 ? 1 : 2) void decode_bf16_mfma_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ kc, const uint16_t* __restrict__ vc,
    const int32_t* __restrict__ seqlens, float* __restrict__ part_o, float* __restrict__ part_lse,
    int Hq, int Hkv, int maxlen, int nsplit, int chunk, float c, uint32_t qflip, PagedKV pg, int gm) {
  constexpr int GM = 32;            // columns (heads) per workgroup, gm of them live
  constexpr int KS = D / 16;        // k-steps of S^T = K Q^T
  constexpr int MD = D / 32;        // 32-row blocks of O^T
  constexpr int RC = D / 8;         // 16-byte chunks per cache row
  constexpr int TILE = 32 * D * 2;  // bytes per 32-key K (or V) tile
  constexpr int RPI = 64 / RC;      // rows per copy instruction (a wave moves 1 KB)
  constexpr int NCP = 32 / RPI;     // copy instructions per K (or V) tile
  // [wave][slot][K, V]; after the key loop it holds the waves' outputs
  __shared__ __attribute__((aligned(1024))) uint8_t ring[4][2][2][TILE];
  __shared__ float m_w[4][GM], l_w[4][GM];
  __shared__ int pid_lds[PAGED ? kMaxChunkPages : 1];
  static_assert(4 * GM * D * 4 <= 4 * 2 * 2 * TILE, "wave outputs must fit in the ring");

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int x = lane & 31;
  const int hi = lane >> 5;
  const int wave_s = __builtin_amdgcn_readfirstlane(wave);
  const int split = split_of_block(nsplit);
  const int G = Hq / Hkv;
  const int slices = G / gm;
  const int kvh = blockIdx.y / slices;
  const int h0 = kvh * G + (blockIdx.y % slices) * gm;
  const int b = blockIdx.z;

  const int L = min(max(seqlens[b], 0), maxlen);
  const int kbeg = split * chunk;
  if (kbeg >= L) return;
  const int n = min(chunk, L - kbeg);
  const int ntile = (n + 31) / 32;
  const size_t cbase = PAGED ? 0 : (((size_t)b * Hkv + kvh) * maxlen + kbeg) * D;
  const uint8_t* kp = reinterpret_cast<const uint8_t*>(kc + cbase);
  const uint8_t* vp = reinterpret_cast<const uint8_t*>(vc + cbase);
  // paged: this chunk's slice of the block table, pool ids clamped into the
  // pool so that a bad table can never address outside it
  const int slot0 = PAGED ? (kbeg >> pg.page_shift) : 0;
  if (PAGED) {
    const int nslots = ((kbeg + n - 1) >> pg.page_shift) - slot0 + 1;  // <= kMaxChunkPages
    for (int i = tid; i < nslots; i += 256)
      pid_lds[i] = min(max(pg.block_table[(size_t)b * pg.max_pages + slot0 + i], 0), pg.num_pages - 1);
    __syncthreads();
  }

  // Q^T fragments (B operand): column x = head h0 + x (zero past gm),
  // d = 16ks + 8hi + 0..7.  Used at once, so their loads are waited for here
  // and not inside the key loop (where the counter also sees the copies).
  bf16x8 qf[KS];
  {
    const uint16_t* qr = q + ((size_t)b * Hq + h0 + min(x, gm - 1)) * D + hi * 8;
    u32x4 w[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) w[ks] = *reinterpret_cast<const u32x4*>(qr + ks * 16);
    const uint32_t keep = x < gm ? 0xffffffffu : 0u;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) qf[ks] = __builtin_bit_cast(bf16x8, (w[ks] ^ qflip) & keep);
  }
  // LDS read offsets within a tile: K row x, chunk (2ks + hi); V^T rows
  // 4hi + (i>>2) (+8, +16ks2), chunk of column block md
  int koff[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) koff[ks] = x * (D * 2) + (((2 * ks + hi) ^ mk_swz<D>(x)) << 4);
  int voff[MD];
  {
    const int i = lane & 15;
    const int row = 4 * hi + (i >> 2);
    const int colc = 2 * ((lane >> 4) & 1) + ((i & 3) >> 1);
#pragma unroll
    for (int md = 0; md < MD; ++md) voff[md] = row * (D * 2) + (((4 * md + colc) ^ mv_swz<D>(row)) << 4) + 8 * (i & 1);
  }

  // Copy instruction i of a tile moves rows RPI*i .. RPI*i + RPI - 1: lane l
  // fills physical chunk l % RC of row RPI*i + l / RC, which holds logical
  // chunk (l % RC) ^ swz(row).  Rows past the chunk end re-read its last key
  // (never past it: the cache there may hold anything); their scores are
  // masked.
  const int crow = lane / RC, ccp = lane % RC;
  const int pmask = PAGED ? (1 << pg.page_shift) - 1 : 0;
  auto issue = [&](int t, int slot) {
    uint8_t* kl = &ring[wave_s][slot][0][0];
    uint8_t* vl = &ring[wave_s][slot][1][0];
    const int r0 = 32 * t;
#pragma unroll
    for (int i = 0; i < NCP; ++i) {
      const int row = RPI * i + crow;
      const int rs = min(row, n - 1 - r0);
      const uint32_t kch = (uint32_t)((ccp ^ mk_swz<D>(row)) << 4);
      const uint32_t vch = (uint32_t)((ccp ^ mv_swz<D>(row)) << 4);
      if (PAGED) {
        const int key = kbeg + r0 + rs;
        const int pid = pid_lds[(key >> pg.page_shift) - slot0];
        const size_t rb = ((((size_t)pid * Hkv + kvh) << pg.page_shift) | (size_t)(key & pmask)) * (D * 2);
        dec_dma16_addr(kp + rb + kch, kl + i * 1024);
        dec_dma16_addr(vp + rb + vch, vl + i * 1024);
      } else {
        dec_dma16(kp + (size_t)r0 * D * 2, (uint32_t)(rs * D * 2) + kch, kl + i * 1024);
        dec_dma16(vp + (size_t)r0 * D * 2, (uint32_t)(rs * D * 2) + vch, vl + i * 1024);
      }
    }
  };

  f32x16 oacc[MD];
#pragma unroll
  for (int md = 0; md < MD; ++md) oacc[md] = f32x16{};
  float m_run = -INFINITY, l_run = 0.f;
  const int myn = ntile > wave_s ? (ntile - 1 - wave_s) / 4 + 1 : 0;  // tiles w, w+4, ... of the chunk
  if (myn > 0) issue(wave_s, 0);
  for (int j = 0; j < myn; ++j) {
    const int t = wave_s + 4 * j;
    const int slot = j & 1;
    if (j + 1 < myn) {
      issue(t + 4, slot ^ 1);      // that slot's reads (tile j-1) finished at its end
      dec_wait_vmem_le<2 * NCP>();  // tile j landed; tile j+1 may be in flight
    } else {
      dec_wait_vmem_le<0>();
    }
    const uint8_t* kl = &ring[wave_s][slot][0][0];
    const uint8_t* vl = &ring[wave_s][slot][1][0];
    // S^T = K Q^T: lane (x, hi) holds keys 8(r/4) + 4hi + r%4 of the tile for head x
    f32x16 s = f32x16{};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) s = mfma32x32x16(*reinterpret_cast<const bf16x8*>(kl + koff[ks]), qf[ks], s);
    const int k0 = 32 * t;
    if (k0 + 32 > n) {
      const int lim = n - 1 - k0 - 4 * hi;
#pragma unroll
      for (int r = 0; r < 16; ++r) s[r] = (8 * (r >> 2) + (r & 3) > lim) ? -INFINITY : s[r];
    }
    // running max per head (lazy rescale against a stale max, as in prefill)
    float mx = s[0];
#pragma unroll
    for (int r = 1; r < 16; ++r) mx = fmaxf(mx, s[r]);
    mx = max_halves(mx) * c;  // -inf stays -inf (c > 0)
    if (__any(mx > m_run + kTauB)) {
      const float mn = fmaxf(m_run, mx);
      const float alpha = fast_exp2(m_run - mn);  // 0 on the first tile (m_run = -inf, mn finite)
      l_run *= alpha;
#pragma unroll
      for (int md = 0; md < MD; ++md) oacc[md] *= alpha;
      m_run = mn;
    }
    bf16x8 pf[2];
#pragma unroll
    for (int ks2 = 0; ks2 < 2; ++ks2) {
      float tmp[8];
#pragma unroll
      for (int jj = 0; jj < 8; ++jj) {
        const float p = fast_exp2(fmaf(s[8 * ks2 + jj], c, -m_run));
        l_run += p;
        tmp[jj] = p;
      }
      pf[ks2] = pack_bf16x8(tmp);
    }
    // O^T += V^T P^T over the tile's two 16-key steps
#pragma unroll
    for (int ks2 = 0; ks2 < 2; ++ks2)
#pragma unroll
      for (int md = 0; md < MD; ++md) {
        const u32x2 a0 = dec_read_tr(vl + voff[md] + (16 * ks2) * D * 2);
        const u32x2 a1 = dec_read_tr(vl + voff[md] + (16 * ks2 + 8) * D * 2);
        const u32x4 a = {a0[0], a0[1], a1[0], a1[1]};
        oacc[md] = mfma32x32x16(__builtin_bit_cast(bf16x8, a), pf[ks2], oacc[md]);
      }
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // this slot may be refilled next
  }

  // ---- merge the four waves' (m, l, o) through the ring ----
  const float lt = sum_halves(l_run);
  __syncthreads();  // every copy landed and every read finished: the ring is free
  float(&o_w)[4][GM][D] = *reinterpret_cast<float(*)[4][GM][D]>(&ring[0][0][0][0]);
  if (x < gm) {
#pragma unroll
    for (int md = 0; md < MD; ++md)
#pragma unroll
      for (int r = 0; r < 16; ++r) o_w[wave_s][x][32 * md + 8 * (r >> 2) + 4 * hi + (r & 3)] = oacc[md][r];
    if (hi == 0) {
      m_w[wave_s][x] = m_run;  // -inf for a wave without tiles (then l = 0, o = 0)
      l_w[wave_s][x] = lt;
    }
  }
  __syncthreads();
  for (int i = tid; i < gm * D; i += 256) {
    const int g = i / D, d = i % D;
    float M = m_w[0][g];
#pragma unroll
    for (int w = 1; w < 4; ++w) M = fmaxf(M, m_w[w][g]);
    float l = 0.f, a = 0.f;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const float f = fast_exp2(m_w[w][g] - M);  // 0 for a wave that saw no key
      l = fmaf(l_w[w][g], f, l);
      a = fmaf(o_w[w][g][d], f, a);
    }
    const size_t pidx = ((size_t)b * Hq + h0 + g) * nsplit + split;
    part_o[pidx * D + d] = a / l;
    if (d == 0) part_lse[pidx] = M * kLn2 + __logf(l);
  }
}

// Query heads per bf16 split workgroup for a GQA group of G heads: the whole
// group up to 32 (every K/V byte is then read once), else the largest divisor
// of G that fits the 32 matrix columns.
int bf16_group_tile(int G) {
  if (G <= 32) return G;
  for (int t = 32; t > 1; --t)
    if (G % t == 0) return t;
  return 1;
}

// Keys per bf16 split workgroup: the largest of 4096, 2048, 1024, 512, 256
// that still gives at least 1024 workgroups (four rounds of one workgroup per
// CU) when every sequence is maxlen long; long chunks amortise the per-chunk
// prologue and partials, short ones keep small batches parallel.  (GQA B64
// Hkv8 workload, lengths 1K-32K, 4 and 8 heads per group: 4096 keys 6.66 /
// 6.41 TB/s, 2048 6.48 / 6.17, 1024 5.50 / 5.02, 8192 5.08 / 5.02.  Asking
// for 1024 rather than 2048 workgroups doubles the chunk for small batches
// and short caches: +2-3% there; asking for 4096 loses 6-10%.)
int bf16_decode_chunk(int B, int Hq, int Hkv, int maxlen) {
  const long long rows = (long long)B * Hkv * ((Hq / Hkv) / bf16_group_tile(Hq / Hkv));
  static_assert(kMaxChunkB == 4096, "the longest chunk sizes the page-id table");
  for (int chunk : {4096, 2048, 1024, 512}) {
    if (rows * ((maxlen + chunk - 1) / chunk) >= 1024) return chunk;
  }
  return 256;
}

template <int D, bool PAGED>
hipError_t launch_bf16_mfma(const DecodeArgs& a, hipStream_t stream) {
  const int gm = bf16_group_tile(a.Hq / a.Hkv);
  const int chunk = bf16_decode_chunk(a.B, a.Hq, a.Hkv, a.maxlen);
  if (partials_bytes(a.B, a.Hq, a.maxlen, D, chunk, sizeof(float)) > a.ws_bytes) return hipErrorInvalidValue;
  const int nsplit = (a.maxlen + chunk - 1) / chunk;
  const int G = a.Hq / a.Hkv;
  float* part_o = static_cast<float*>(a.ws);
  const size_t po_bytes = (size_t)a.B * a.Hq * nsplit * D * sizeof(float);
  float* part_lse = reinterpret_cast<float*>(static_cast<char*>(a.ws) + ((po_bytes + 255) & ~(size_t)255));
  dim3 g1(nsplit, a.Hkv * (G / gm), a.B);
  if (g1.y > 65535u || g1.z > 65535u) return hipErrorInvalidValue;
  hipLaunchKernelGGL((decode_bf16_mfma_kernel<D, PAGED>), g1, dim3(256), 0, stream,
                     static_cast<const uint16_t*>(a.q), static_cast<const uint16_t*>(a.k),
                     static_cast<const uint16_t*>(a.v), a.seqlens, part_o, part_lse, a.Hq, a.Hkv, a.maxlen,
                     nsplit, chunk, a.c, a.neg ? 0x80008000u : 0u, a.paged, gm);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((decode_combine_kernel<uint16_t, D>), dim3(a.Hq, a.B), dim3(kCombThreads), 0, stream, part_o,
                     part_lse, a.seqlens, static_cast<uint16_t*>(a.o), a.Hq, a.maxlen, nsplit, chunk);
  return hipGetLastError();
}

template <int D, bool PAGED>
hipError_t launch_bf16_g(const DecodeArgs& a, hipStream_t stream) {
  return launch_bf16_mfma<D, PAGED>(a, stream);
}

template <typename T, int D, int GT>
hipError_t launch_t(const DecodeArgs& a, hipStream_t stream) {
  if (partials_bytes(a.B, a.Hq, a.maxlen, D, kChunk, sizeof(LseT<T>)) > a.ws_bytes) return hipErrorInvalidValue;
  const int nsplit = (a.maxlen + kChunk - 1) / kChunk;
  const int G = a.Hq / a.Hkv;
  float* part_o = static_cast<float*>(a.ws);
  const size_t po_bytes = (size_t)a.B * a.Hq * nsplit * D * sizeof(float);
  LseT<T>* part_lse = reinterpret_cast<LseT<T>*>(static_cast<char*>(a.ws) + ((po_bytes + 255) & ~(size_t)255));
  dim3 g1(nsplit, a.Hkv * (G / GT), a.B);
  if (g1.y > 65535u || g1.z > 65535u) return hipErrorInvalidValue;
  hipLaunchKernelGGL((decode_split_kernel<T, D, GT>), g1, dim3(256), 0, stream, static_cast<const T*>(a.q),
                     static_cast<const T*>(a.k), static_cast<const T*>(a.v), a.seqlens, part_o, part_lse,
                     a.Hq, a.Hkv, a.maxlen, nsplit, a.c, a.neg ? -1.0f : 1.0f);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((decode_combine_kernel<T, D>), dim3(a.Hq, a.B), dim3(kCombThreads), 0, stream, part_o, part_lse,
                     a.seqlens, static_cast<T*>(a.o), a.Hq, a.maxlen, nsplit, kChunk);
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

size_t decode_workspace_bytes(int B, int Hq, int Hkv, int maxlen, int d) {
  // large enough for either path's chunking
  const size_t a = partials_bytes(B, Hq, maxlen, d, kChunk, sizeof(double));
  const size_t b = partials_bytes(B, Hq, maxlen, d, bf16_decode_chunk(B, Hq, Hkv, maxlen), sizeof(float));
  return a > b ? a : b;
}

hipError_t launch_decode_bf16(const DecodeArgs& a, hipStream_t stream) {
  if (a.paged.block_table != nullptr) {
    if (a.paged.page_shift < 4 || a.paged.num_pages <= 0 || a.paged.max_pages <= 0 ||
        a.maxlen != (a.paged.max_pages << a.paged.page_shift))
      return hipErrorInvalidValue;
    if (a.d == 128) return launch_bf16_g<128, true>(a, stream);
    if (a.d == 64) return launch_bf16_g<64, true>(a, stream);
    return hipErrorInvalidValue;
  }
  if (a.d == 128) return launch_bf16_g<128, false>(a, stream);
  if (a.d == 64) return launch_bf16_g<64, false>(a, stream);
  return hipErrorInvalidValue;
}

hipError_t launch_decode_f32(const DecodeArgs& a, hipStream_t stream) {
  if (a.d == 128) return launch_g<float, 128>(a, stream);
  if (a.d == 64) return launch_g<float, 64>(a, stream);
  return hipErrorInvalidValue;
}

size_t decode_noalloc_bytes(int B, int Hq, int Hkv, int maxlen, int d) {
  return partials_bytes(B, Hq, maxlen, d, bf16_decode_chunk(B, Hq, Hkv, maxlen), sizeof(float));
}

}  // namespace fa

// Fixed partials array of the allocation-free decode entry point.  In host
// code `scratch` names a host-side stand-in, not device memory: the device
// address comes from hipGetSymbolAddress, once per device, and only that
// address is ever passed to a kernel.  Every partial the combine reads is
// written by the split kernel of the same call, so nothing needs clearing.
static __device__ __align__(256) uint8_t scratch[fa::kDecodeScratchBytes];

namespace fa {
namespace {
constexpr int kMaxScratchDevices = 64;
std::mutex g_scratch_mutex;
void* g_scratch_ptr[kMaxScratchDevices] = {};
}  // namespace

hipError_t decode_scratch_address(void** ptr) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxScratchDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));  // the current device's copy
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return hipSuccess;
}

}  // namespace fa
