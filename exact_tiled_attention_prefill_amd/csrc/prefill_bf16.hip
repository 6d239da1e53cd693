// bf16 prefill: tiled exact attention with a running softmax on gfx950 MFMA.
//
// Method (sources cited by page title and section):
//   * Tiles of queries, keys and values sized for on-chip memory are finished
//     one at a time and nothing N x N reaches HBM ("11.4d FlashAttention",
//     "Tiling"; "How Does Flash Attention Reduce Memory Traffic During Local
//     Inference?", "Flash Attention Tiles the Problem Into On-Chip Working
//     Sets").
//   * A running max and running sum per query row normalise incrementally
//     ("11.4d FlashAttention", "Online Softmax"; the same page pair's
//     "Online Softmax Avoids Storing the Full Score Matrix").
//   * Score, scale, mask, normalisation and value aggregation run in one
//     kernel ("Kernel Fusion Keeps More of the Attention Chain in One
//     Execution Path").
//   * Loads of the next key/value tile overlap compute on the current one
//     (double buffering, forum comment item 45450456, paragraph on the
//     implications for prefill and token generation).
//
// gfx950 design (one workgroup = 4 waves = 256 query rows of one head):
//   * Each wave owns 64 query rows (two 32-column MFMA blocks).  Q lives in
//     VGPRs for the whole kernel.
//   * Scores are computed transposed, S^T = K Q^T, with
//     v_mfma_f32_32x32x16_bf16: a lane then holds 16 keys of ONE query per
//     block, so the row max and row sum are mostly in-lane, with one
//     v_permlane32_swap to join the two wave halves.
//   * The fp32 S^T accumulator, packed to bf16, is directly the B operand of
//     O^T += V^T P^T (the contraction index is the key, whose order inside a
//     16-key step may be permuted freely as long as V^T uses the same order),
//     so P never goes through LDS.  O^T keeps a lane's query in the lane, so
//     the per-row rescale is a lane-local multiply.
//   * K tiles sit in LDS row-major with 16-byte chunks XOR-swizzled by row;
//     V tiles are stored transposed (d-major, 8-byte key slots rotated by row)
//     so that each MFMA A fragment is two ds_read_b64.  Both are
//     double-buffered: tile t+1 is fetched from HBM into VGPRs while tile t
//     is computed, then written to the idle LDS buffer.
//   * The running max is updated lazily: the output is rescaled only when a
//     row max grows by more than 2^8, otherwise exponents are taken against
//     the stale max (p <= 256, exact after the final division by l).
//   * Causal: tiles above the diagonal are never loaded; a wave whose rows
//     are all before a tile skips its MFMAs; masks are applied only on
//     diagonal and ragged tail tiles.  Heavy (late) query tiles launch first.
#include "common.h"
#include "kernels.h"

namespace fa {
namespace {

template <int D>
struct Bf16Cfg {
  static constexpr int kThreads = 256;
  static constexpr int kWaveRows = 64;                  // query rows per wave
  static constexpr int kBR = 256;                       // query rows per workgroup
  static constexpr int kBC = 64;                        // keys per tile
  static constexpr int kKS = D / 16;                    // k-steps of S^T = K Q^T
  static constexpr int kMD = D / 32;                    // 32-row blocks of O^T
  static constexpr int kRowChunks = D / 8;              // 16-byte chunks per K row
  static constexpr int kKChunks = kBC * kRowChunks;     // per K tile
  static constexpr int kKPerThread = kKChunks / kThreads;
  static constexpr int kVTasks = (kBC / 4) * (D / 8);   // 4-key x 8-d blocks per V tile
  static constexpr int kTileBytes = kBC * D * 2;
  static_assert(kKChunks % kThreads == 0, "K tile must split evenly");
  static_assert(kVTasks <= kThreads, "one V block per thread at most");
};

constexpr float kTau = 8.0f;  // lazy-rescale threshold (log2 units)

// K tile: row = key (D*2 bytes), 16-byte chunk c stored at c ^ (row & mask).
template <int D>
__device__ __forceinline__ int k_lds_off(int row, int chunk) {
  constexpr int mask = (D / 8) - 1;
  return row * (D * 2) + ((chunk ^ (row & mask)) << 4);
}

// V^T tile: row = d (64 keys = 128 bytes), 8-byte slot s (keys 4s..4s+3)
// stored at (s + rot(row)) & 15 with rot spreading both the transposing
// writes (rows 8b+e, fixed e) and the fragment reads (32 consecutive rows)
// over distinct banks.
__device__ __forceinline__ int v_lds_off(int row, int slot) {
  const int rot = ((row >> 3) + 2 * (row & 7)) & 15;
  return row * 128 + (((slot + rot) & 15) << 3);
}

template <int D, bool CAUSAL>
__global__ __launch_bounds__(256, 1) void prefill_bf16_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, uint16_t* __restrict__ o, float* __restrict__ lse,
    int Hq, int Hkv, int N, int n_qtiles, int BH, float c, uint32_t qflip) {
  using Cfg = Bf16Cfg<D>;
  __shared__ __attribute__((aligned(16))) uint8_t smem_k[2][Cfg::kTileBytes];
  __shared__ __attribute__((aligned(16))) uint8_t smem_v[2][Cfg::kTileBytes];

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int x = lane & 31;
  const int hi = lane >> 5;

  // Work item: heavy query tiles first when causal.
  const int bid = blockIdx.x;
  const int qtile = CAUSAL ? (n_qtiles - 1 - bid / BH) : (bid / BH);
  const int bh = bid % BH;
  const int b = bh / Hq;
  const int h = bh - b * Hq;
  const int g = h / (Hq / Hkv);
  const size_t qbase = (size_t)bh * N * D;
  const size_t kvbase = ((size_t)b * Hkv + g) * N * D;
  const uint16_t* qh = q + qbase;
  const uint16_t* kh = k + kvbase;
  const uint16_t* vh = v + kvbase;

  const int q0 = qtile * Cfg::kBR;
  const int qw = q0 + wave * Cfg::kWaveRows;
  const bool wave_has_rows = qw < N;
  const int wave_last_row = min(qw + Cfg::kWaveRows - 1, N - 1);

  // Q fragments (B operand of S^T = K Q^T): column x of block nb, d = 16ks + 8hi + 0..7.
  bf16x8 qf[2][Cfg::kKS];
#pragma unroll
  for (int nb = 0; nb < 2; ++nb) {
    const int row = qw + nb * 32 + x;
#pragma unroll
    for (int ks = 0; ks < Cfg::kKS; ++ks) {
      u32x4 w = {0u, 0u, 0u, 0u};
      if (row < N) {
        w = *reinterpret_cast<const u32x4*>(qh + (size_t)row * D + ks * 16 + hi * 8);
        w ^= qflip;
      }
      qf[nb][ks] = __builtin_bit_cast(bf16x8, w);
    }
  }

  f32x16 oacc[2][Cfg::kMD];
#pragma unroll
  for (int nb = 0; nb < 2; ++nb)
#pragma unroll
    for (int md = 0; md < Cfg::kMD; ++md) oacc[nb][md] = f32x16{};
  float m_run[2] = {-INFINITY, -INFINITY};
  float l_run[2] = {0.f, 0.f};

  const int kv_end = CAUSAL ? min(N, q0 + Cfg::kBR) : N;
  const int ntiles = (kv_end + Cfg::kBC - 1) / Cfg::kBC;

  // ---- global -> VGPR prefetch and VGPR -> LDS store of one K/V tile ----
  u32x4 kreg[Cfg::kKPerThread];
  u32x4 vreg[4];
  const bool v_task = tid < Cfg::kVTasks;
  const int va = tid / (D / 8);  // 4-key group
  const int vb = tid % (D / 8);  // 8-d group

  auto load_tile = [&](int t) {
    const int k0 = t * Cfg::kBC;
#pragma unroll
    for (int i = 0; i < Cfg::kKPerThread; ++i) {
      const int idx = i * Cfg::kThreads + tid;
      const int row = idx / Cfg::kRowChunks;
      const int ch = idx % Cfg::kRowChunks;
      if (k0 + row < N)
        kreg[i] = *reinterpret_cast<const u32x4*>(kh + (size_t)(k0 + row) * D + ch * 8);
      else
        kreg[i] = u32x4{0u, 0u, 0u, 0u};
    }
    if (v_task) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = k0 + va * 4 + i;
        if (row < N)
          vreg[i] = *reinterpret_cast<const u32x4*>(vh + (size_t)row * D + vb * 8);
        else
          vreg[i] = u32x4{0u, 0u, 0u, 0u};
      }
    }
  };

  auto store_tile = [&](int buf) {
#pragma unroll
    for (int i = 0; i < Cfg::kKPerThread; ++i) {
      const int idx = i * Cfg::kThreads + tid;
      const int row = idx / Cfg::kRowChunks;
      const int ch = idx % Cfg::kRowChunks;
      *reinterpret_cast<u32x4*>(&smem_k[buf][k_lds_off<D>(row, ch)]) = kreg[i];
    }
    if (v_task) {
      // 4 keys x 8 d  ->  8 rows of V^T, each 4 consecutive keys (8 bytes).
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        const uint32_t w0 = vreg[0][p], w1 = vreg[1][p], w2 = vreg[2][p], w3 = vreg[3][p];
        u32x2 lo = {(w0 & 0xffffu) | (w1 << 16), (w2 & 0xffffu) | (w3 << 16)};
        u32x2 hv = {(w0 >> 16) | (w1 & 0xffff0000u), (w2 >> 16) | (w3 & 0xffff0000u)};
        const int r0 = vb * 8 + 2 * p;
        *reinterpret_cast<u32x2*>(&smem_v[buf][v_lds_off(r0, va)]) = lo;
        *reinterpret_cast<u32x2*>(&smem_v[buf][v_lds_off(r0 + 1, va)]) = hv;
      }
    }
  };

  load_tile(0);
  store_tile(0);
  __syncthreads();

  for (int t = 0; t < ntiles; ++t) {
    const int buf = t & 1;
    if (t + 1 < ntiles) load_tile(t + 1);
    const int k0 = t * Cfg::kBC;
    const bool active = wave_has_rows && (!CAUSAL || k0 <= wave_last_row);
    if (active) {
      const uint8_t* ks_lds = smem_k[buf];
      const uint8_t* vs_lds = smem_v[buf];
      // ---- S^T = K Q^T : s[mb][nb] covers keys 32mb.., queries 32nb.. ----
      f32x16 s[2][2];
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int nb = 0; nb < 2; ++nb) s[mb][nb] = f32x16{};
#pragma unroll
      for (int ks = 0; ks < Cfg::kKS; ++ks) {
#pragma unroll
        for (int mb = 0; mb < 2; ++mb) {
          const bf16x8 kf = *reinterpret_cast<const bf16x8*>(
              ks_lds + k_lds_off<D>(mb * 32 + x, ks * 2 + hi));
#pragma unroll
          for (int nb = 0; nb < 2; ++nb) s[mb][nb] = mfma32x32x16(kf, qf[nb][ks], s[mb][nb]);
        }
      }
      // ---- mask: keys past the end, and keys after the query when causal ----
      const bool need_mask = (k0 + Cfg::kBC > N) || (CAUSAL && k0 + Cfg::kBC - 1 > qw);
      if (need_mask) {
#pragma unroll
        for (int mb = 0; mb < 2; ++mb)
#pragma unroll
          for (int nb = 0; nb < 2; ++nb) {
            const int qrow = qw + nb * 32 + x;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              const int key = k0 + mb * 32 + 8 * (r >> 2) + 4 * hi + (r & 3);
              const bool masked = (key >= N) || (CAUSAL && key > qrow);
              s[mb][nb][r] = masked ? -INFINITY : s[mb][nb][r];
            }
          }
      }
      // ---- running softmax ----
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) {
        float mx = -INFINITY;
#pragma unroll
        for (int mb = 0; mb < 2; ++mb)
#pragma unroll
          for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[mb][nb][r]);
        mx = max_halves(mx);
        const float mxs = mx * c;  // -inf stays -inf (c > 0)
        const bool grow = mxs > m_run[nb] + kTau;
        if (__any(grow)) {
          const float mn = fmaxf(m_run[nb], mxs);
          const float alpha = fast_exp2(m_run[nb] - mn);
          l_run[nb] *= alpha;
#pragma unroll
          for (int md = 0; md < Cfg::kMD; ++md) oacc[nb][md] *= alpha;
          m_run[nb] = mn;
        }
        const float negm = -m_run[nb];
        float lsum = 0.f;
#pragma unroll
        for (int mb = 0; mb < 2; ++mb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const float p = fast_exp2(fmaf(s[mb][nb][r], c, negm));
            s[mb][nb][r] = p;
            lsum += p;
          }
        l_run[nb] += lsum;
      }
      // ---- O^T += V^T P^T over four 16-key steps ----
#pragma unroll
      for (int ks2 = 0; ks2 < Cfg::kBC / 16; ++ks2) {
        bf16x8 pf[2];
#pragma unroll
        for (int nb = 0; nb < 2; ++nb) {
          float tmp[8];
#pragma unroll
          for (int j = 0; j < 8; ++j) tmp[j] = s[ks2 >> 1][nb][8 * (ks2 & 1) + j];
          pf[nb] = pack_bf16x8(tmp);
        }
#pragma unroll
        for (int md = 0; md < Cfg::kMD; ++md) {
          const int row = md * 32 + x;
          const u32x2 a0 = *reinterpret_cast<const u32x2*>(vs_lds + v_lds_off(row, 4 * ks2 + hi));
          const u32x2 a1 = *reinterpret_cast<const u32x2*>(vs_lds + v_lds_off(row, 4 * ks2 + 2 + hi));
          const u32x4 a = {a0[0], a0[1], a1[0], a1[1]};
          const bf16x8 vf = __builtin_bit_cast(bf16x8, a);
#pragma unroll
          for (int nb = 0; nb < 2; ++nb) oacc[nb][md] = mfma32x32x16(vf, pf[nb], oacc[nb][md]);
        }
      }
    }
    if (t + 1 < ntiles) store_tile(buf ^ 1);
    __syncthreads();
  }

  // ---- epilogue: O = O^T / l, lse = m ln2 + ln l ----
  if (!wave_has_rows) return;
#pragma unroll
  for (int nb = 0; nb < 2; ++nb) {
    const float lt = sum_halves(l_run[nb]);
    const float inv = 1.0f / lt;
    const int row = qw + nb * 32 + x;
    if (row < N) {
      uint16_t* orow = o + qbase + (size_t)row * D;
#pragma unroll
      for (int md = 0; md < Cfg::kMD; ++md)
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          const int d0 = md * 32 + 8 * g4 + 4 * hi;
          u32x2 w = {pack_bf16x2(oacc[nb][md][4 * g4 + 0] * inv, oacc[nb][md][4 * g4 + 1] * inv),
                     pack_bf16x2(oacc[nb][md][4 * g4 + 2] * inv, oacc[nb][md][4 * g4 + 3] * inv)};
          *reinterpret_cast<u32x2*>(orow + d0) = w;
        }
      if (lse != nullptr && hi == 0) lse[(size_t)bh * N + row] = m_run[nb] * kLn2 + __logf(lt);
    }
  }
}

template <int D, bool CAUSAL>
hipError_t launch(const PrefillArgs& a, hipStream_t stream) {
  using Cfg = Bf16Cfg<D>;
  const int n_qtiles = (a.N + Cfg::kBR - 1) / Cfg::kBR;
  const int BH = a.B * a.Hq;
  const long long blocks = (long long)n_qtiles * BH;
  if (blocks > 0x7fffffffLL) return hipErrorInvalidValue;
  hipLaunchKernelGGL((prefill_bf16_kernel<D, CAUSAL>), dim3((unsigned)blocks), dim3(Cfg::kThreads), 0,
                     stream, static_cast<const uint16_t*>(a.q), static_cast<const uint16_t*>(a.k),
                     static_cast<const uint16_t*>(a.v), static_cast<uint16_t*>(a.o), a.lse, a.Hq,
                     a.Hkv, a.N, n_qtiles, BH, a.c, a.neg ? 0x80008000u : 0u);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_prefill_bf16(const PrefillArgs& a, hipStream_t stream) {
  if (a.d == 128) return a.causal ? launch<128, true>(a, stream) : launch<128, false>(a, stream);
  if (a.d == 64) return a.causal ? launch<64, true>(a, stream) : launch<64, false>(a, stream);
  return hipErrorInvalidValue;
}

}  // namespace fa
