// bf16 prefill: tiled exact attention with a running softmax on gfx950 MFMA.
//
// Method (sources cited by page title and section):
//   * Tiles of queries, keys and values sized for on-chip memory are finished
//     one at a time and nothing N x N reaches HBM ("11.4d FlashAttention",
//     "Tiling"; "How Does Flash Attention Reduce Memory Traffic During Local
//     Inference?", "Flash Attention Tiles the Problem Into On-Chip Working
//     Sets").
//   * A running max and running sum per query row normalise incrementally
//     ("11.4d FlashAttention", "Online Softmax"; "How Does Flash Attention
//     Reduce Memory Traffic ...", "Online Softmax Avoids Storing the Full Score
//     Matrix").
//   * Score, scale, mask, normalisation and value aggregation run in one
//     kernel ("Kernel Fusion Keeps More of the Attention Chain in One
//     Execution Path").
//   * The next key/value tile is loaded while the current one is computed
//     (double buffering, forum comment item 45450456, paragraph on the
//     implications for prefill and token generation).
//
// gfx950 design:
//   * Workgroup = 4 waves = 128 query rows of one head; each wave owns 32
//     rows.  Two workgroups share a CU, so every SIMD runs two waves whose
//     softmax (VALU) and matrix products (MFMA) interleave.  Q stays in VGPRs.
//   * Scores are computed transposed, S^T = K Q^T, with
//     v_mfma_f32_32x32x16_bf16: a lane then holds 16 keys of ONE query per
//     32-key block, so row max and row sum are in-lane plus one
//     v_permlane32_swap.  The fp32 accumulator, packed to bf16, is directly
//     the B operand of O^T += V^T P^T (inside a 16-key step the key order may
//     be permuted freely as long as V^T uses the same order), so P never
//     touches LDS, and O^T keeps each query's output in its own lane.
//   * K and V tiles (64 keys) are copied HBM -> LDS by global_load_lds_dwordx4
//     (no VGPR staging), double-buffered.  K is read with ds_read_b128, V with
//     the gfx950 transposing ds_read_b64_tr_b16 straight into the MFMA A
//     operand layout.  16-byte chunks are XOR-swizzled by row so both reads
//     are bank-conflict free; the DMA source addresses apply the same swizzle.
//   * The running max is updated lazily: the output is rescaled only when a
//     row max grows by more than 2^8; otherwise exponents are taken against
//     the stale max (p <= 256; exact after the final division by l).
//   * Causal: tiles above the diagonal are never loaded, a wave whose rows all
//     precede a tile skips it, masks run only on diagonal and ragged tiles.
//   * Scheduling: workgroup ids are dealt round-robin to the 8 XCDs, so each
//     XCD is given a contiguous range of work items; within it the items are
//     ordered (KV head group, query tile heaviest-first, query head of the
//     group), so the query heads sharing K/V -- and neighbouring query tiles
//     streaming the same K/V tiles -- run together on one XCD's L2.
#include "common.h"
#include "kernels.h"

namespace fa {
namespace {

constexpr int kThreads = 256;
constexpr int kBR = 128;  // query rows per workgroup
constexpr int kBC = 64;   // keys per tile
constexpr float kTau = 8.0f;  // lazy-rescale threshold (log2 units)

// Chunk swizzles (16-byte chunks within a tile row of D/8 chunks).
// K rows are read 16 rows x one chunk at a time -> spread consecutive rows.
template <int D>
__device__ __forceinline__ int k_swz(int row) {
  return D == 128 ? (row & 15) : ((row >> 1) & 7);
}
// V rows are read 4 rows x 4 chunks at a time (transposing reads).
template <int D>
__device__ __forceinline__ int v_swz(int row) {
  return D == 128 ? 4 * (row & 3) : 4 * ((row >> 1) & 1);
}

__device__ __forceinline__ void wait_vmem() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

typedef short i16x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ u32x2 ds_read_tr(const uint8_t* lds_byte_ptr) {
  typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
  const lds_i16x4* p = (const lds_i16x4*)(lds_byte_ptr);
  return __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16(const_cast<lds_i16x4*>(p)));
}

__device__ __forceinline__ void dma16(const void* gsrc, uint8_t* lds_wave_base) {
  __builtin_amdgcn_global_load_lds(gsrc, (__attribute__((address_space(3))) void*)lds_wave_base, 16, 0, 0);
}

template <int D, bool CAUSAL>
__global__ __launch_bounds__(kThreads, 2) void prefill_bf16_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, uint16_t* __restrict__ o, float* __restrict__ lse,
    int Hq, int Hkv, int N, int n_qtiles, int n_items, float c, uint32_t qflip) {
  constexpr int KS = D / 16;              // k-steps of S^T = K Q^T
  constexpr int MD = D / 32;              // 32-row blocks of O^T
  constexpr int RC = D / 8;               // 16-byte chunks per row
  constexpr int TILE = kBC * D * 2;       // bytes per K (or V) tile
  constexpr int CPT = kBC * RC / kThreads;  // DMA chunks per thread per tile
  static_assert(CPT * kThreads == kBC * RC, "tile must split evenly");
  // Four distinct LDS objects (K/V x two buffers) so that the compiler can
  // tell the DMA target of the next tile from the buffer being read.
  __shared__ __attribute__((aligned(1024))) uint8_t k_lds0[TILE];
  __shared__ __attribute__((aligned(1024))) uint8_t k_lds1[TILE];
  __shared__ __attribute__((aligned(1024))) uint8_t v_lds0[TILE];
  __shared__ __attribute__((aligned(1024))) uint8_t v_lds1[TILE];

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int x = lane & 31;
  const int hi = lane >> 5;

  // ---- work item: XCD-contiguous ranges, (group, tile heavy-first, head) ----
  int item = blockIdx.x;
  if ((n_items & 7) == 0) item = (blockIdx.x & 7) * (n_items >> 3) + (blockIdx.x >> 3);
  const int G = Hq / Hkv;
  const int per_group = n_qtiles * G;
  const int grp = item / per_group;  // (b, kv head)
  const int rem = item - grp * per_group;
  const int tslot = rem / G;
  const int qtile = CAUSAL ? (n_qtiles - 1 - tslot) : tslot;
  const int b = grp / Hkv;
  const int g = grp - b * Hkv;
  const int h = g * G + (rem - tslot * G);
  const int bh = b * Hq + h;
  const size_t qbase = (size_t)bh * N * D;
  const uint16_t* qh = q + qbase;
  const uint16_t* kh = k + (size_t)grp * N * D;
  const uint16_t* vh = v + (size_t)grp * N * D;

  const int q0 = qtile * kBR;
  const int qw = q0 + wave * 32;
  const bool wave_has_rows = qw < N;
  const int wave_last_row = min(qw + 31, N - 1);

  // Q fragments (B operand of S^T = K Q^T): column x, d = 16ks + 8hi + 0..7.
  bf16x8 qf[KS];
  {
    const int row = qw + x;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      u32x4 w = {0u, 0u, 0u, 0u};
      if (row < N) {
        w = *reinterpret_cast<const u32x4*>(qh + (size_t)row * D + ks * 16 + hi * 8);
        w ^= qflip;
      }
      qf[ks] = __builtin_bit_cast(bf16x8, w);
    }
  }

  // ---- per-lane LDS read offsets (the tile base and ks/mb/ks2 parts are immediates) ----
  int koff[KS];  // K: row x (+32 mb), chunk (2ks + hi) swizzled
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) koff[ks] = x * (D * 2) + (((2 * ks + hi) ^ k_swz<D>(x)) << 4);
  int voff[MD];  // V^T fragments: row 4hi + (i>>2) (+16ks2 + 8half), chunk of column md*32 + ...
  {
    const int i = lane & 15;
    const int row = 4 * hi + (i >> 2);
    const int colc = 2 * ((lane >> 4) & 1) + ((i & 3) >> 1);  // chunk within the 32-column block
#pragma unroll
    for (int md = 0; md < MD; ++md)
      voff[md] = row * (D * 2) + (((4 * md + colc) ^ v_swz<D>(row)) << 4) + 8 * (i & 1);
  }

  // ---- DMA: chunk p = i*256 + wave*64 + lane of the tile ----
  int dma_row[CPT], dma_kc[CPT], dma_vc[CPT];
#pragma unroll
  for (int i = 0; i < CPT; ++i) {
    const int p = i * kThreads + wave * 64 + lane;
    const int r = p / RC, cp = p % RC;
    dma_row[i] = r;
    dma_kc[i] = (cp ^ k_swz<D>(r)) * 8;
    dma_vc[i] = (cp ^ v_swz<D>(r)) * 8;
  }
  auto issue_tile = [&](int t, uint8_t* kl, uint8_t* vl) {
    const int k0 = t * kBC;
    const bool full = k0 + kBC <= N;
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      // rows past the end re-read the last row: finite, and masked out below
      const int row = full ? k0 + dma_row[i] : min(k0 + dma_row[i], N - 1);
      dma16(kh + (size_t)row * D + dma_kc[i], kl + (i * kThreads + wave * 64) * 16);
      dma16(vh + (size_t)row * D + dma_vc[i], vl + (i * kThreads + wave * 64) * 16);
    }
  };

  f32x16 oacc[MD];
#pragma unroll
  for (int md = 0; md < MD; ++md) oacc[md] = f32x16{};
  float m_run = -INFINITY, l_run = 0.f;

  const int kv_end = CAUSAL ? min(N, q0 + kBR) : N;
  const int ntiles = (kv_end + kBC - 1) / kBC;

  issue_tile(0, k_lds0, v_lds0);
  wait_vmem();
  __syncthreads();

  // One tile step: prefetch tile t+1 into (kn, vn) while computing tile t from (kl, vl).
  auto step = [&](int t, const uint8_t* kl, const uint8_t* vl, uint8_t* kn, uint8_t* vn) {
    if (t + 1 < ntiles) issue_tile(t + 1, kn, vn);
    const int k0 = t * kBC;
    const bool active = wave_has_rows && (!CAUSAL || k0 <= wave_last_row);
    if (active) {
      // ---- S^T = K Q^T : s[mb] covers keys 32mb + (8(r/4) + 4hi + r%4), query x ----
      f32x16 s[2] = {f32x16{}, f32x16{}};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
#pragma unroll
        for (int mb = 0; mb < 2; ++mb) {
          const bf16x8 kf = *reinterpret_cast<const bf16x8*>(kl + koff[ks] + mb * 32 * D * 2);
          s[mb] = mfma32x32x16(kf, qf[ks], s[mb]);
        }
      // ---- mask: keys past the end, and keys after the query when causal ----
      if ((k0 + kBC > N) || (CAUSAL && k0 + kBC - 1 > qw)) {
        const int qrow = qw + x;
#pragma unroll
        for (int mb = 0; mb < 2; ++mb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int key = k0 + mb * 32 + 8 * (r >> 2) + 4 * hi + (r & 3);
            const bool masked = (key >= N) || (CAUSAL && key > qrow);
            s[mb][r] = masked ? -INFINITY : s[mb][r];
          }
      }
      // ---- running softmax (base 2, lazy rescale) ----
      float mx = -INFINITY;
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[mb][r]);
      mx = max_halves(mx);
      const float mxs = mx * c;  // -inf stays -inf (c > 0)
      if (__any(mxs > m_run + kTau)) {
        const float mn = fmaxf(m_run, mxs);
        const float alpha = fast_exp2(m_run - mn);
        l_run *= alpha;
#pragma unroll
        for (int md = 0; md < MD; ++md) oacc[md] *= alpha;
        m_run = mn;
      }
      const float negm = -m_run;
      float lsum = 0.f;
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float p = fast_exp2(fmaf(s[mb][r], c, negm));
          s[mb][r] = p;
          lsum += p;
        }
      l_run += lsum;
      // ---- O^T += V^T P^T over four 16-key steps ----
#pragma unroll
      for (int ks2 = 0; ks2 < kBC / 16; ++ks2) {
        float tmp[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) tmp[j] = s[ks2 >> 1][8 * (ks2 & 1) + j];
        const bf16x8 pf = pack_bf16x8(tmp);
#pragma unroll
        for (int md = 0; md < MD; ++md) {
          const u32x2 a0 = ds_read_tr(vl + voff[md] + (16 * ks2) * D * 2);
          const u32x2 a1 = ds_read_tr(vl + voff[md] + (16 * ks2 + 8) * D * 2);
          const u32x4 a = {a0[0], a0[1], a1[0], a1[1]};
          oacc[md] = mfma32x32x16(__builtin_bit_cast(bf16x8, a), pf, oacc[md]);
        }
      }
    }
    wait_vmem();
    __syncthreads();
  };
  for (int t = 0; t < ntiles; t += 2) {
    step(t, k_lds0, v_lds0, k_lds1, v_lds1);
    if (t + 1 < ntiles) step(t + 1, k_lds1, v_lds1, k_lds0, v_lds0);
  }

  // ---- epilogue: O = O^T / l, lse = m ln2 + ln l ----
  if (!wave_has_rows) return;
  const float lt = sum_halves(l_run);
  const float inv = 1.0f / lt;
  const int row = qw + x;
  if (row < N) {
    uint16_t* orow = o + qbase + (size_t)row * D;
#pragma unroll
    for (int md = 0; md < MD; ++md)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int d0 = md * 32 + 8 * g4 + 4 * hi;
        u32x2 w = {pack_bf16x2(oacc[md][4 * g4 + 0] * inv, oacc[md][4 * g4 + 1] * inv),
                   pack_bf16x2(oacc[md][4 * g4 + 2] * inv, oacc[md][4 * g4 + 3] * inv)};
        *reinterpret_cast<u32x2*>(orow + d0) = w;
      }
    if (lse != nullptr && hi == 0) lse[(size_t)bh * N + row] = m_run * kLn2 + __logf(lt);
  }
}

template <int D, bool CAUSAL>
hipError_t launch(const PrefillArgs& a, hipStream_t stream) {
  const int n_qtiles = (a.N + kBR - 1) / kBR;
  const long long items = (long long)n_qtiles * a.B * a.Hq;
  if (items > 0x7fffffffLL) return hipErrorInvalidValue;
  hipLaunchKernelGGL((prefill_bf16_kernel<D, CAUSAL>), dim3((unsigned)items), dim3(kThreads), 0, stream,
                     static_cast<const uint16_t*>(a.q), static_cast<const uint16_t*>(a.k),
                     static_cast<const uint16_t*>(a.v), static_cast<uint16_t*>(a.o), a.lse, a.Hq, a.Hkv,
                     a.N, n_qtiles, (int)items, a.c, a.neg ? 0x80008000u : 0u);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_prefill_bf16(const PrefillArgs& a, hipStream_t stream) {
  if (a.d == 128) return a.causal ? launch<128, true>(a, stream) : launch<128, false>(a, stream);
  if (a.d == 64) return a.causal ? launch<64, true>(a, stream) : launch<64, false>(a, stream);
  return hipErrorInvalidValue;
}

}  // namespace fa
