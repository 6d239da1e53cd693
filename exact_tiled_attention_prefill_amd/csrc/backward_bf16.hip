// bf16 attention backward on gfx950 MFMA: dQ, dK, dV from Q, K, V, O, dO and
// the forward's log-sum-exp.
//
// Method: the probabilities are recomputed tile by tile from Q, K and the
// saved log-sum-exp instead of being stored ("11.4d FlashAttention", section
// "Recomputation"); with s = scale q.k, p = exp(s - lse):
//     dV = P^T dO,   dP = dO V^T,   dS = P o (dP - D),   D_i = dO_i . O_i,
//     dQ = scale dS K,   dK = scale dS^T Q
// (D_i is the row sum of P o dP).  Under GQA a key/value head's dK, dV sum
// over the query heads that share it.
//
// Two kernels on the caller's stream:
//   dQ:    one workgroup per 128 query rows (as the forward).  It first
//          computes D_i of its rows and writes -D_i and -lse_i*log2(e) to a
//          workspace padded to 64-row multiples (so the dK/dV kernel's tile
//          copies never leave it).  Key tiles then stream through an LDS ring;
//          per 64-key tile and wave S^T = K Q^T, P^T, dP^T = V dO^T, dS^T,
//          then dQ^T += K^T dS^T, with dS^T packed to bf16 straight from the
//          accumulator layout into the B operand (48 MFMAs).  dP^T starts at
//          -D, the exponentials run under the dP^T products and dS^T under
//          the dQ^T products;
//   dK/dV: one workgroup of 8 waves per 128 keys of one key/value head,
//          looping over the group's query heads and their 64-row query
//          tiles.  Waves w and w+4 own the same 32 keys and split each tile's
//          rows; per wave S = Q K^T and dP = dO V^T (K fragments in registers,
//          the block's V rows in LDS), then dV += P^T dO and dK += dS^T Q with
//          the packed P / dS as the A operand (32 MFMAs).  The dP
//          accumulator starts at -D of its rows, so dS = P dP takes one
//          product, and the exponentials (and dS) run under the dP (and dV)
//          matrix products.  No atomics: every output element has
//          one writer, so results are deterministic.
// In both kernels the per-element causal / end-of-sequence mask runs only on
// tiles that some row of the wave does not see in full, and the tile loops
// are unrolled by two so that ring slots are immediates.
// Q, dO (dK/dV kernel) and K (dQ kernel) are read from LDS both row-wise
// (ds_read_b128) and transposed (ds_read_b64_tr_b16); their 16-byte chunks
// use one XOR swizzle that leaves both access patterns free of bank
// conflicts (dQ's V tile, read row-wise only, shares it).
#include "common.h"
#include "kernels.h"
#include <type_traits>

namespace fa {
namespace {

constexpr int kBThreads = 256;  // 4 waves
constexpr int kBQRows = 128;    // dQ kernel: query rows per workgroup
constexpr int kBKeys = 128;     // dK/dV kernel: keys per workgroup (32 per wave)
constexpr int kBTile = 64;      // rows per streamed K/V (dQ) or Q/dO (dK/dV) tile

// Row-read swizzle (chunk ^ f(row)) for tiles only read row-wise.
template <int D>
__device__ __forceinline__ int swz_row(int row) {
  return D == 128 ? (row & 15) : ((row >> 1) & 7);
}
// Swizzle for tiles read both row-wise and transposed: for rows 0..15 (the
// 16 rows of one row read) it is a permutation, and the 4 consecutive rows of
// a transposed read get 4 different values of its bits 2-3.
template <int D>
__device__ __forceinline__ int swz_both(int row) {
  return D == 128 ? ((4 * (row & 3)) | ((row >> 2) & 3)) : ((4 * ((row >> 1) & 1)) | ((row >> 2) & 3));
}

template <int n>
__device__ __forceinline__ void bwait_vmem_le() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(n) : "memory");
}
__device__ __forceinline__ void bbarrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}
// lane l's 16 bytes from base + off land at lds_wave_base + 16*l (inline asm:
// not tracked by the compiler; completion is ordered by vmcnt + barrier).
// The compiler applies no hazard rule to inline asm: s_nop 0 gives the m0
// write just before the copy its one wait state, and the build checks the
// generated code for a VALU write of the base SGPRs fewer than 5 wait
// states before a copy (isa_check.py).
__device__ __forceinline__ void bdma16(const void* base, uint32_t off, uint8_t* lds_wave_base) {
  const uint32_t m0 = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) uint8_t*)lds_wave_base;
  asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, %2" ::"v"(off), "{m0}"(m0), "s"(base) : "memory");
}
// A wave-uniform pointer forced into scalar registers (the copy takes its
// base address from SGPRs).
__device__ __forceinline__ const void* sgpr_ptr(const void* p) {
  const uint64_t a = (uint64_t)(uintptr_t)p;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)a);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
  return (const void*)(uintptr_t)(((uint64_t)hi << 32) | lo);
}
typedef short bi16x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ u32x2 bread_tr(const uint8_t* p) {
  typedef __attribute__((address_space(3))) bi16x4 lds_t;
  return __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_t*)(p)));
}

// ---------------------------------------------------------------------------
// dQ kernel.
// Before its key loop it also computes, for its own rows, D_i = dO_i . O_i,
// and writes -D_i and -lse_i * log2(e) to the workspace for the dK/dV kernel
// (rows N .. Npad-1 of the padded workspace get 0).
template <int D, bool CAUSAL>
__global__ __launch_bounds__(kBThreads, 2) void bwd_dq_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    const uint16_t* __restrict__ o, const uint16_t* __restrict__ dout, const float* __restrict__ lse,
    float* __restrict__ nlsw, float* __restrict__ ndw, uint16_t* __restrict__ dq, int Hq, int Hkv, int N,
    int Npad, int n_qtiles, int n_items, float cs, float scale) {
  constexpr int KS = D / 16;
  constexpr int MD = D / 32;
  constexpr int RC = D / 8;
  constexpr int TILE = kBTile * D * 2;
  constexpr int CPT = kBTile * RC / kBThreads;
  static_assert(CPT * kBThreads == kBTile * RC, "tile must split evenly");
  __shared__ __attribute__((aligned(1024))) uint8_t ring[2][2][TILE];  // [stage][K, V]

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int x = lane & 31;
  const int hi = lane >> 5;

  int item = blockIdx.x;
  if ((n_items & 7) == 0) item = (blockIdx.x & 7) * (n_items >> 3) + (blockIdx.x >> 3);
  const int G = Hq / Hkv;
  const int per_group = n_qtiles * G;
  const int grp = item / per_group;
  const int rem = item - grp * per_group;
  const int tslot = rem / G;
  const int qtile = CAUSAL ? (n_qtiles - 1 - tslot) : tslot;
  const int b = grp / Hkv;
  const int g = grp - b * Hkv;
  const int h = g * G + (rem - tslot * G);
  const int bh = b * Hq + h;
  const size_t qbase = (size_t)bh * N * D;
  const uint16_t* kh = k + (size_t)grp * N * D;
  const uint16_t* vh = v + (size_t)grp * N * D;

  const int q0 = qtile * kBQRows;
  const int qrow = q0 + wave + 4 * x;  // rows interleaved over the waves, as in the forward
  const int wave_first = q0 + wave;
  const int wave_last_row = min(q0 + wave + 4 * 31, N - 1);
  const bool wave_has_rows = wave_first < N;
  const int qr = min(qrow, N - 1);

  // Q and dO fragments: column x = row qrow, d = 16ks + 8hi + 0..7
  bf16x8 qf[KS], df[KS];
  {
    const uint16_t* qp = q + qbase + (size_t)qr * D + hi * 8;
    const uint16_t* dp = dout + qbase + (size_t)qr * D + hi * 8;
    u32x4 wq[KS], wd[KS];
#pragma unroll
    for (int t = 0; t < KS; ++t) {
      wq[t] = *reinterpret_cast<const u32x4*>(qp + t * 16);
      wd[t] = *reinterpret_cast<const u32x4*>(dp + t * 16);
    }
    const uint32_t keep = qrow < N ? 0xffffffffu : 0u;
#pragma unroll
    for (int t = 0; t < KS; ++t) {
      qf[t] = __builtin_bit_cast(bf16x8, wq[t] & keep);
      df[t] = __builtin_bit_cast(bf16x8, wd[t] & keep);
    }
  }
  // D and lse*log2(e) of row qrow: each half-wave lane holds half of the
  // row's d elements (the same split as df), the other half is in lane x^32
  float dd, l2;
  {
    const uint16_t* op = o + qbase + (size_t)qr * D + hi * 8;
    u32x4 wo[KS];
#pragma unroll
    for (int t = 0; t < KS; ++t) wo[t] = *reinterpret_cast<const u32x4*>(op + t * 16);
    float a = 0.f;
#pragma unroll
    for (int t = 0; t < KS; ++t) {
      const u32x4 dv4 = __builtin_bit_cast(u32x4, df[t]);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        a = fmaf(bf16lo_to_f32(wo[t][e]), bf16lo_to_f32(dv4[e]), a);
        a = fmaf(bf16hi_to_f32(wo[t][e]), bf16hi_to_f32(dv4[e]), a);
      }
    }
    dd = sum_halves(a);
    l2 = qrow < N ? lse[(size_t)bh * N + qr] * kLog2e : 0.f;
    if (hi == 0 && qrow < Npad) {
      ndw[(size_t)bh * Npad + qrow] = -dd;  // 0 past N: dO was zeroed there
      nlsw[(size_t)bh * Npad + qrow] = -l2;
    }
  }

  // LDS read offsets.  K and V rows: row x (+32mb), chunk (2ks+hi)^swz_both.
  // V is only read row-wise, but sharing K's swizzle (a permutation over any
  // 16 rows, so row reads stay conflict-free) lets both use one offset set.
  int koff[KS];
#pragma unroll
  for (int t = 0; t < KS; ++t) koff[t] = x * (D * 2) + (((2 * t + hi) ^ swz_both<D>(x)) << 4);
  // K^T transposed reads: rows 4hi + (i>>2) (+8 for the second half, +16ks2),
  // column block md; the swizzle depends on row bits 0..3, so the +8 half
  // has its own offset (+16 rows leave it unchanged)
  int ktr[MD][2];
  {
    const int i = lane & 15;
    const int colc = 2 * ((lane >> 4) & 1) + ((i & 3) >> 1);
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
      const int row = 4 * hi + (i >> 2) + 8 * hf;
#pragma unroll
      for (int md = 0; md < MD; ++md)
        ktr[md][hf] = row * (D * 2) + (((4 * md + colc) ^ swz_both<D>(row)) << 4) + 8 * (i & 1);
    }
  }
  // DMA: chunk p = i*256 + tid -> row p / RC, chunk p % RC.  A lane's chunks
  // are kRowStep rows apart and both swizzles depend on the row only modulo
  // 16, so one offset serves every chunk; the row step goes into the base.
  const int wave_s = __builtin_amdgcn_readfirstlane(wave);
  constexpr int kRowStep = kBThreads / RC;
  static_assert(kRowStep % 16 == 0, "row step keeps the swizzle");
  const int drow = (wave * 64 + lane) / RC, dcp = lane % RC;
  const uint32_t d_off = (uint32_t)(drow * D * 2 + ((dcp ^ swz_both<D>(drow)) << 4));
  auto issue = [&](int t, uint8_t* kdst, uint8_t* vdst) {
    const int k0 = t * kBTile;
    const uint8_t* kb = reinterpret_cast<const uint8_t*>(kh) + (size_t)k0 * D * 2;
    const uint8_t* vb = reinterpret_cast<const uint8_t*>(vh) + (size_t)k0 * D * 2;
    if (k0 + kBTile <= N) {
#pragma unroll
      for (int i = 0; i < CPT; ++i) {
        bdma16(kb + (size_t)i * kRowStep * D * 2, d_off, kdst + (i * kBThreads + wave_s * 64) * 16);
        bdma16(vb + (size_t)i * kRowStep * D * 2, d_off, vdst + (i * kBThreads + wave_s * 64) * 16);
      }
    } else {
#pragma unroll
      for (int i = 0; i < CPT; ++i) {
        // rows past the end re-read the last row; the offset is taken from
        // the tile base and the clamped row is >= 0, so it never wraps
        const int delta = (min(drow + i * kRowStep, N - 1 - k0) - drow) * D * 2;
        bdma16(kb, d_off + delta, kdst + (i * kBThreads + wave_s * 64) * 16);
        bdma16(vb, d_off + delta, vdst + (i * kBThreads + wave_s * 64) * 16);
      }
    }
  };

  f32x16 acc[MD];
#pragma unroll
  for (int md = 0; md < MD; ++md) acc[md] = f32x16{};

  const int kv_end = CAUSAL ? min(N, q0 + kBQRows) : N;
  const int ntiles = (kv_end + kBTile - 1) / kBTile;
  // Every row of this wave sees every key of tile k0 (no per-element mask):
  // the tile lies below the causal diagonal of the wave's first row and
  // inside the sequence.  Wave-uniform.
  const int wave_first_s = q0 + wave_s;
  auto tile_all_visible = [&](int k0) {
    return k0 + kBTile <= N && (!CAUSAL || k0 + kBTile - 1 <= wave_first_s);
  };
  // One tile step; the ring slot is a compile-time constant (the loop is
  // unrolled by two), so the LDS reads take immediate offsets.
  auto step = [&](int t, auto slot_c) {
    constexpr int SL = decltype(slot_c)::value;
    if (t + 1 < ntiles) issue(t + 1, ring[SL ^ 1][0], ring[SL ^ 1][1]);
    const uint8_t* kl = ring[SL][0];
    const uint8_t* vl = ring[SL][1];
    const int k0 = t * kBTile;
    if (wave_has_rows && (!CAUSAL || k0 <= wave_last_row)) {
      // S^T, and dP^T from -D of the lane's row, so dS^T = P^T dP^T.  The
      // regions are fenced (sched_barrier) so that each one's grouping hints
      // see only its own instructions.
      f32x16 s[2] = {f32x16{}, f32x16{}}, dp[2];
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int r = 0; r < 16; ++r) dp[mb][r] = -dd;
      // region 1: S^T = K Q^T (the dP^T initialisation runs alongside)
#pragma unroll
      for (int t2 = 0; t2 < KS; ++t2)
#pragma unroll
        for (int mb = 0; mb < 2; ++mb) {
          const bf16x8 kf = *reinterpret_cast<const bf16x8*>(kl + koff[t2] + mb * 32 * D * 2);
          s[mb] = mfma32x32x16(kf, qf[t2], s[mb]);
        }
#pragma unroll
      for (int i = 0; i < 2 * KS; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, 2, 0);
      }
      __builtin_amdgcn_sched_barrier(0);
      // region 2: dP^T = V dO^T - D || P^T = exp2(cs S^T - lse log2 e), in
      // two fenced halves (half the k-steps with one score block's
      // exponentials each: one group pattern over all of it went unfilled)
#pragma unroll
      for (int hk = 0; hk < 2; ++hk) {
#pragma unroll
        for (int t2 = hk * KS / 2; t2 < (hk + 1) * KS / 2; ++t2)
#pragma unroll
          for (int mb = 0; mb < 2; ++mb) {
            const bf16x8 vf = *reinterpret_cast<const bf16x8*>(vl + koff[t2] + mb * 32 * D * 2);
            dp[mb] = mfma32x32x16(vf, df[t2], dp[mb]);
          }
#pragma unroll
        for (int r = 0; r < 16; ++r) s[hk][r] = fast_exp2(fmaf(s[hk][r], cs, -l2));
#pragma unroll
        for (int i = 0; i < KS; ++i) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x002, 32 / KS, 0);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
      if (!tile_all_visible(k0)) {
        // key of (mb, r) = k0 + 4hi + 32mb + 8(r/4) + r%4; visible when <= lim
        // (a select, not a product: a masked exponent may be +inf)
        const int lim = (CAUSAL ? min(qrow, N - 1) : N - 1) - k0 - 4 * hi;
#pragma unroll
        for (int mb = 0; mb < 2; ++mb)
#pragma unroll
          for (int r = 0; r < 16; ++r) s[mb][r] = 32 * mb + 8 * (r >> 2) + (r & 3) <= lim ? s[mb][r] : 0.f;
      }
      // region 3: dQ^T += K^T dS^T || dS^T = P^T dP^T, packed per 16 keys
#pragma unroll
      for (int ks2 = 0; ks2 < kBTile / 16; ++ks2) {
        float tmp[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) tmp[j] = s[ks2 >> 1][8 * (ks2 & 1) + j] * dp[ks2 >> 1][8 * (ks2 & 1) + j];
        const bf16x8 pf = pack_bf16x8(tmp);
#pragma unroll
        for (int md = 0; md < MD; ++md) {
          const u32x2 a0 = bread_tr(kl + ktr[md][0] + (16 * ks2) * D * 2);
          const u32x2 a1 = bread_tr(kl + ktr[md][1] + (16 * ks2) * D * 2);
          const u32x4 a = {a0[0], a0[1], a1[0], a1[1]};
          acc[md] = mfma32x32x16(__builtin_bit_cast(bf16x8, a), pf, acc[md]);
        }
      }
      // the first 16 keys' dS^T and packs, then one matrix product and three
      // VALU ops per step
      __builtin_amdgcn_sched_group_barrier(0x002, 12, 0);
#pragma unroll
      for (int i = 0; i < MD * kBTile / 16; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, 3, 0);
      }
    }
    if (t + 1 < ntiles) bwait_vmem_le<0>();
    bbarrier();
  };
  issue(0, ring[0][0], ring[0][1]);
  bwait_vmem_le<0>();
  bbarrier();
  // unrolled by two; an odd last tile is the loop's skipped second half (a
  // workgroup-uniform branch), so there is no separate tail copy of the step
  for (int t = 0; t < ntiles; t += 2) {
    step(t, std::integral_constant<int, 0>{});
    if (t + 1 < ntiles) step(t + 1, std::integral_constant<int, 1>{});
  }
  if (wave_has_rows && qrow < N) {
    uint16_t* orow = dq + qbase + (size_t)qrow * D;
#pragma unroll
    for (int md = 0; md < MD; ++md)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int d0 = md * 32 + 8 * g4 + 4 * hi;
        u32x2 w = {pack_bf16x2(acc[md][4 * g4 + 0] * scale, acc[md][4 * g4 + 1] * scale),
                   pack_bf16x2(acc[md][4 * g4 + 2] * scale, acc[md][4 * g4 + 3] * scale)};
        *reinterpret_cast<u32x2*>(orow + d0) = w;
      }
  }
}

// ---------------------------------------------------------------------------
// dK/dV kernel: 8 waves, two per SIMD.  Waves w and w+4 own the same 32 keys
// (k0b + 32(w&3) + x) and split every 64-row query tile: wave w takes rows
// 0..31, wave w+4 rows 32..63.  K fragments stay in registers; the block's
// 128 V rows (read row-wise as the B operand of dP) are copied to LDS once.
// The two halves' dV and dK are summed through LDS at the end.
constexpr int kBKThreads = 512;

template <int D, bool CAUSAL>
__global__ __launch_bounds__(kBKThreads, 1) void bwd_dkdv_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    const uint16_t* __restrict__ dout, const float* __restrict__ nlsw, const float* __restrict__ ndw,
    uint16_t* __restrict__ dk, uint16_t* __restrict__ dv, int Hq, int Hkv, int N, int Npad, int n_kblocks,
    int n_items, float cs, float scale) {
  constexpr int KS = D / 16;
  constexpr int MD = D / 32;
  constexpr int RC = D / 8;
  constexpr int TILE = kBTile * D * 2;
  constexpr int CPT = kBTile * RC / kBKThreads;    // Q (and dO) chunks per thread per tile
  constexpr int VPT = kBKeys * RC / kBKThreads;    // V-block chunks per thread
  static_assert(CPT >= 1 && CPT * kBKThreads == kBTile * RC, "tile must split evenly");
  static_assert(VPT * kBKThreads == kBKeys * RC, "V block must split evenly");
  // [stage][Q, dO] tiles; at the end the ring holds the upper waves' partial sums
  __shared__ __attribute__((aligned(1024))) uint8_t ring[2][2][TILE];
  __shared__ __attribute__((aligned(1024))) uint8_t vblk[kBKeys * D * 2];
  __shared__ __attribute__((aligned(16))) float rowv[2][2][kBTile];  // [stage][-lse*log2(e), -D][row]
  static_assert(4 * 32 * D * 4 <= 2 * 2 * TILE, "partial sums must fit in the ring");

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int x = lane & 31;
  const int hi = lane >> 5;
  const int kw = wave & 3;    // key sub-block
  const int half = wave >> 2;  // query rows 32*half .. +31 of every tile

  int item = blockIdx.x;
  if ((n_items & 7) == 0) item = (blockIdx.x & 7) * (n_items >> 3) + (blockIdx.x >> 3);
  const int grp = item / n_kblocks;       // (b, kv head)
  const int kb = item - grp * n_kblocks;  // key block; causal: low blocks see the most queries
  const int b = grp / Hkv;
  const int g = grp - b * Hkv;
  const int G = Hq / Hkv;
  const int k0b = kb * kBKeys;
  const int key = k0b + 32 * kw + x;      // this lane's key (column x of the sub-block)
  const int kr = min(key, N - 1);
  const size_t kvbase = (size_t)grp * N * D;
  const int wave_s = __builtin_amdgcn_readfirstlane(wave);

  // K fragments as the B operand of S = Q K^T: column x = key, d = 16ks + 8hi + 0..7
  bf16x8 kf[KS];
  {
    const uint16_t* kp = k + kvbase + (size_t)kr * D + hi * 8;
#pragma unroll
    for (int t = 0; t < KS; ++t) kf[t] = *reinterpret_cast<const bf16x8*>(kp + t * 16);
  }
  // the block's V rows into LDS (rows past N re-read row N-1), swizzled for row reads
  {
    const uint8_t* vb = reinterpret_cast<const uint8_t*>(v + kvbase) + (size_t)k0b * D * 2;
#pragma unroll
    for (int i = 0; i < VPT; ++i) {
      const int p = i * kBKThreads + wave * 64 + lane;
      const int r = p / RC, cp = p % RC;
      const int rr = min(r, N - 1 - k0b);
      bdma16(vb, (uint32_t)(rr * D * 2 + ((cp ^ swz_row<D>(r)) << 4)), vblk + (i * kBKThreads + wave_s * 64) * 16);
    }
  }
  int voffb[KS];  // V rows as the B operand of dP = dO V^T: row 32kw + x, chunk (2ks + hi)
#pragma unroll
  for (int t = 0; t < KS; ++t)
    voffb[t] = (32 * kw + x) * (D * 2) + (((2 * t + hi) ^ swz_row<D>(x)) << 4);
  // Q / dO rows 32*half + x for row reads; transposed reads as in the dQ kernel
  int roff[KS];
#pragma unroll
  for (int t = 0; t < KS; ++t)
    roff[t] = (32 * half + x) * (D * 2) + (((2 * t + hi) ^ swz_both<D>(x)) << 4);
  int trr[MD][2];
  {
    const int i = lane & 15;
    const int colc = 2 * ((lane >> 4) & 1) + ((i & 3) >> 1);
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
      const int row = 4 * hi + (i >> 2) + 8 * hf;
#pragma unroll
      for (int md = 0; md < MD; ++md)
        trr[md][hf] = (32 * half + row) * (D * 2) + (((4 * md + colc) ^ swz_both<D>(row)) << 4) + 8 * (i & 1);
    }
  }
  // one DMA offset per lane: its chunks are kRowStep rows apart and the
  // swizzle depends on the row only modulo 16
  constexpr int kRowStep = kBKThreads / RC;
  static_assert(kRowStep % 16 == 0, "row step keeps the swizzle");
  const int drow = (wave * 64 + lane) / RC;
  const uint32_t d_off = (uint32_t)(drow * D * 2 + (((lane % RC) ^ swz_both<D>(drow)) << 4));

  f32x16 dva[MD], dka[MD];
#pragma unroll
  for (int md = 0; md < MD; ++md) {
    dva[md] = f32x16{};
    dka[md] = f32x16{};
  }

  const int n_qt = (N + kBTile - 1) / kBTile;
  const int qt0 = CAUSAL ? (k0b / kBTile) : 0;  // query tiles that can see this key block
  const int per_head = n_qt - qt0;
  const int total = per_head * G;               // (head, query tile) steps
  // step u: head h = g*G + u / per_head, query tile qt0 + u % per_head
  auto issue = [&](int u, auto st_c) {
    constexpr int st = decltype(st_c)::value;
    const int h = g * G + u / per_head;
    const int q0 = (qt0 + u % per_head) * kBTile;
    const size_t hb = ((size_t)b * Hq + h);
    const uint8_t* qb = reinterpret_cast<const uint8_t*>(q + hb * N * D) + (size_t)q0 * D * 2;
    const uint8_t* ob = reinterpret_cast<const uint8_t*>(dout + hb * N * D) + (size_t)q0 * D * 2;
    if (q0 + kBTile <= N) {
#pragma unroll
      for (int i = 0; i < CPT; ++i) {
        bdma16(qb + (size_t)i * kRowStep * D * 2, d_off, ring[st][0] + (i * kBKThreads + wave_s * 64) * 16);
        bdma16(ob + (size_t)i * kRowStep * D * 2, d_off, ring[st][1] + (i * kBKThreads + wave_s * 64) * 16);
      }
    } else {
#pragma unroll
      for (int i = 0; i < CPT; ++i) {
        // clamped row >= 0 relative to the tile base: the offset never wraps
        const int delta = (min(drow + i * kRowStep, N - 1 - q0) - drow) * D * 2;
        bdma16(qb, d_off + delta, ring[st][0] + (i * kBKThreads + wave_s * 64) * 16);
        bdma16(ob, d_off + delta, ring[st][1] + (i * kBKThreads + wave_s * 64) * 16);
      }
    }
    // -lse*log2(e) and -D of the tile's 64 rows (padded workspace, always in
    // range): waves 0-1 copy the first, waves 2-3 the second, 8 lanes x 16
    // bytes each
    if (wave_s < 4) {
      const void* src = sgpr_ptr((wave_s < 2 ? nlsw : ndw) + hb * Npad + q0 + 32 * (wave_s & 1));
      // the lane id is taken afresh (mbcnt): a value kept live across the
      // loop was spilled, and its reload's vmcnt wait stalled on the copies
      const uint32_t ln = __builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u));
      if (ln < 8)
        bdma16(src, ln * 16, reinterpret_cast<uint8_t*>(&rowv[st][wave_s >> 1][32 * (wave_s & 1)]));
    }
  };

  // Every (row, key) pair of this wave in the tile at q0 is visible (no
  // per-element mask): the wave's rows lie inside the sequence and, causal,
  // at or below the diagonal of its last key.  Wave-uniform.
  const int wkey_last = k0b + 32 * (wave_s & 3) + 31;
  const int wrow_off = 32 * (wave_s >> 2);
  auto tile_all_visible = [&](int q0) {
    return q0 + wrow_off + 31 < N && (!CAUSAL || wkey_last <= q0 + wrow_off);
  };
  // One (head, query tile) step; the ring slot is a compile-time constant
  // (the loop is unrolled by two), so the LDS reads take immediate offsets.
  auto step = [&](int u, auto slot_c) {
    constexpr int SL = decltype(slot_c)::value;
    if (u + 1 < total) issue(u + 1, std::integral_constant<int, SL ^ 1>{});
    const uint8_t* ql = ring[SL][0];
    const uint8_t* ol = ring[SL][1];
    const float* nlt = rowv[SL][0];
    const float* ndt = rowv[SL][1];
    const int q0 = (qt0 + u % per_head) * kBTile;
    // S[q, key] = Q K^T and dP[q, key] = dO V^T - D over rows
    // q0 + 32half + 8(r/4) + 4hi + r%4: the dP accumulator starts at the
    // rows' -D, so dS = P dP.
    f32x16 s = f32x16{}, dp;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const f32x4 d4 = *reinterpret_cast<const f32x4*>(ndt + 32 * half + 8 * j + 4 * hi);
#pragma unroll
      for (int e = 0; e < 4; ++e) dp[4 * j + e] = d4[e];
    }
    // The regions below are fenced (sched_barrier) so that each one's
    // grouping hints see only its own instructions.
    // region 1: S (and the rows' -lse log2 e)
#pragma unroll
    for (int t2 = 0; t2 < KS; ++t2) {
      const bf16x8 a = *reinterpret_cast<const bf16x8*>(ql + roff[t2]);
      s = mfma32x32x16(a, kf[t2], s);
    }
    f32x4 l4[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) l4[j] = *reinterpret_cast<const f32x4*>(nlt + 32 * half + 8 * j + 4 * hi);
    __builtin_amdgcn_sched_barrier(0);
    // region 2: dP || P = exp2(cs S - lse log2 e)
#pragma unroll
    for (int t2 = 0; t2 < KS; ++t2) {
      const bf16x8 a = *reinterpret_cast<const bf16x8*>(ol + roff[t2]);
      const bf16x8 bv = *reinterpret_cast<const bf16x8*>(vblk + voffb[t2]);
      dp = mfma32x32x16(a, bv, dp);
    }
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int e = 0; e < 4; ++e) s[4 * j + e] = fast_exp2(fmaf(s[4 * j + e], cs, l4[j][e]));
    // one matrix product and four VALU ops per step
#pragma unroll
    for (int i = 0; i < KS; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);
    }
    __builtin_amdgcn_sched_barrier(0);
    // visible: row < N and, causal, key <= row (a select: a masked exponent
    // may be +inf)
    if (!tile_all_visible(q0)) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = q0 + 32 * half + 8 * (r >> 2) + 4 * hi + (r & 3);
        const bool vis = row < N && (!CAUSAL || key <= row);
        s[r] = vis ? s[r] : 0.f;
      }
    }
    // region 3: dV += P^T dO || dS = P dP
    bf16x8 pa[2], da[2];
#pragma unroll
    for (int ks2 = 0; ks2 < 2; ++ks2) {
      float tp[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) tp[j] = s[8 * ks2 + j];
      pa[ks2] = pack_bf16x8(tp);
    }
#pragma unroll
    for (int ks2 = 0; ks2 < 2; ++ks2)
#pragma unroll
      for (int md = 0; md < MD; ++md) {
        const u32x2 o0 = bread_tr(ol + trr[md][0] + (16 * ks2) * D * 2);
        const u32x2 o1 = bread_tr(ol + trr[md][1] + (16 * ks2) * D * 2);
        const u32x4 ob = {o0[0], o0[1], o1[0], o1[1]};
        dva[md] = mfma32x32x16(pa[ks2], __builtin_bit_cast(bf16x8, ob), dva[md]);
      }
#pragma unroll
    for (int ks2 = 0; ks2 < 2; ++ks2) {
      float td[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) td[j] = s[8 * ks2 + j] * dp[8 * ks2 + j];
      da[ks2] = pack_bf16x8(td);
    }
    // the first probabilities' packs, then one matrix product and three VALU
    // ops per step
    __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);
#pragma unroll
    for (int i = 0; i < 2 * MD; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x002, 3, 0);
    }
    __builtin_amdgcn_sched_barrier(0);
    // region 4: dK += dS^T Q
#pragma unroll
    for (int ks2 = 0; ks2 < 2; ++ks2)
#pragma unroll
      for (int md = 0; md < MD; ++md) {
        const u32x2 q0r = bread_tr(ql + trr[md][0] + (16 * ks2) * D * 2);
        const u32x2 q1r = bread_tr(ql + trr[md][1] + (16 * ks2) * D * 2);
        const u32x4 qbv = {q0r[0], q0r[1], q1r[0], q1r[1]};
        dka[md] = mfma32x32x16(da[ks2], __builtin_bit_cast(bf16x8, qbv), dka[md]);
      }
    if (u + 1 < total) bwait_vmem_le<0>();
    bbarrier();
  };
  if (total > 0) issue(0, std::integral_constant<int, 0>{});
  bwait_vmem_le<0>();  // the V block (and tile 0)
  // The K fragments' loads have landed too.  A use of them here lets the
  // compiler settle their wait before the loop; otherwise it waits inside
  // the loop, where its vmcnt also counts the next tile's copies.
#pragma unroll
  for (int t = 0; t < KS; ++t) asm volatile("" ::"v"(__builtin_bit_cast(u32x4, kf[t])));
  bbarrier();
  // unrolled by two; an odd last step is the loop's skipped second half
  // (a workgroup-uniform branch), so no separate tail copy of the step keeps
  // its per-lane offsets live (and spilled) past the loop
  for (int u = 0; u < total; u += 2) {
    step(u, std::integral_constant<int, 0>{});
    if (u + 1 < total) step(u + 1, std::integral_constant<int, 1>{});
  }

  // Sum the two halves through LDS (every wave is past the last barrier, no
  // copy is in flight), then the lower waves store.  Register r of block md
  // holds key k0b + 32kw + 8(r/4) + 4hi + r%4 and column d = 32md + x.  The
  // lane id is taken afresh (mbcnt, in volatile asm so that it is not
  // hoisted) and the wave split comes from the scalar wave index, so no
  // per-lane epilogue address stays live (and spilled) through the loop.
  int le;
  asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(le));
  const int xe = le & 31, he = le >> 5;
  const int kw_e = wave_s & 3, half_e = wave_s >> 2;
  float* red = reinterpret_cast<float*>(&ring[0][0][0]);
  auto red_idx = [&](int md, int r) { return (kw_e * 32 + 8 * (r >> 2) + 4 * he + (r & 3)) * D + 32 * md + xe; };
  auto reduce_store = [&](f32x16(&acc)[MD], uint16_t* out, float mul) {
    if (half_e == 1) {
#pragma unroll
      for (int md = 0; md < MD; ++md)
#pragma unroll
        for (int r = 0; r < 16; ++r) red[red_idx(md, r)] = acc[md][r];
    }
    __syncthreads();
    if (half_e == 0) {
#pragma unroll
      for (int md = 0; md < MD; ++md)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int kk = k0b + 32 * kw_e + 8 * (r >> 2) + 4 * he + (r & 3);
          const float val = (acc[md][r] + red[red_idx(md, r)]) * mul;
          if (kk < N) out[kvbase + (size_t)kk * D + 32 * md + xe] = (uint16_t)(pack_bf16x2(val, 0.f) & 0xffffu);
        }
    }
    __syncthreads();
  };
  reduce_store(dva, dv, 1.0f);
  reduce_store(dka, dk, scale);
}

template <int D, bool CAUSAL>
hipError_t launch_bwd(const BackwardArgs& a, hipStream_t stream) {
  const int Npad = (a.N + kBTile - 1) / kBTile * kBTile;
  float* nlsw = static_cast<float*>(a.ws);  // -lse/scale, then -D, per padded row
  float* ndw = nlsw + (size_t)a.B * a.Hq * Npad;
  const float cs = a.scale * kLog2e;  // signed: exp2(s_raw * cs - lse * log2 e)
  const int n_qtiles = (a.N + kBQRows - 1) / kBQRows;
  const long long dq_items = (long long)n_qtiles * a.B * a.Hq;
  const int n_kblocks = (a.N + kBKeys - 1) / kBKeys;
  const long long kv_items = (long long)n_kblocks * a.B * a.Hkv;
  if (dq_items > 0x7fffffffLL || kv_items > 0x7fffffffLL) return hipErrorInvalidValue;
  hipLaunchKernelGGL((bwd_dq_kernel<D, CAUSAL>), dim3((unsigned)dq_items), dim3(kBThreads), 0, stream,
                     static_cast<const uint16_t*>(a.q), static_cast<const uint16_t*>(a.k),
                     static_cast<const uint16_t*>(a.v), static_cast<const uint16_t*>(a.o),
                     static_cast<const uint16_t*>(a.dout), a.lse, nlsw, ndw, static_cast<uint16_t*>(a.dq), a.Hq,
                     a.Hkv, a.N, Npad, n_qtiles, (int)dq_items, cs, a.scale);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((bwd_dkdv_kernel<D, CAUSAL>), dim3((unsigned)kv_items), dim3(kBKThreads), 0, stream,
                     static_cast<const uint16_t*>(a.q), static_cast<const uint16_t*>(a.k),
                     static_cast<const uint16_t*>(a.v), static_cast<const uint16_t*>(a.dout), nlsw, ndw,
                     static_cast<uint16_t*>(a.dk), static_cast<uint16_t*>(a.dv), a.Hq, a.Hkv, a.N, Npad, n_kblocks,
                     (int)kv_items, cs, a.scale);
  return hipGetLastError();
}

}  // namespace

size_t backward_workspace_bytes(int B, int Hq, int N) {
  const size_t Npad = ((size_t)N + kBTile - 1) / kBTile * kBTile;
  return 2 * (size_t)B * Hq * Npad * sizeof(float) + 256;
}

hipError_t launch_backward_bf16(const BackwardArgs& a, hipStream_t stream) {
  if (a.ws_bytes < backward_workspace_bytes(a.B, a.Hq, a.N)) return hipErrorInvalidValue;
  if (a.d == 128) return a.causal ? launch_bwd<128, true>(a, stream) : launch_bwd<128, false>(a, stream);
  if (a.d == 64) return a.causal ? launch_bwd<64, true>(a, stream) : launch_bwd<64, false>(a, stream);
  return hipErrorInvalidValue;
}

}  // namespace fa
