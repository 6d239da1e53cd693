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
//   * Workgroup = 4 waves = 128 query rows of one head; two workgroups share
//     a CU, so every SIMD runs two waves from different workgroups whose
//     softmax (VALU) and matrix products (MFMA) interleave.  Rows that see
//     4K keys or more on average use 8 waves = 256 rows instead (one
//     workgroup per CU, half the K/V copies per row).  Wave w of W owns rows
//     q0 + w + Wj (j = 0..31): interleaving the rows gives every wave the
//     same causal work, so the per-tile barrier never waits on a wave with
//     more tiles.  Q stays in VGPRs.
//   * Scores are computed transposed, S^T = K Q^T, with
//     v_mfma_f32_32x32x16_bf16: a lane then holds 16 keys of ONE query per
//     32-key block, so row max and row sum are in-lane plus one
//     v_permlane32_swap.  The fp32 accumulator, packed to bf16, is directly
//     the B operand of O^T += V^T P^T (inside a 16-key step the key order may
//     be permuted freely as long as V^T uses the same order), so P never
//     touches LDS, and O^T keeps each query's output in its own lane.
//   * K and V tiles (64 keys) are copied HBM -> LDS by global_load_lds_dwordx4
//     (no VGPR staging) into a ring: with four waves two slots (K of the tile
//     after next and V of the next tile stream in while the current ones are
//     read; a workgroup barrier after every tile), with eight waves four slots
//     (a barrier after every second tile; the copies of a step are issued by
//     one half of the waves, alternating, so one wave of every SIMD keeps the
//     matrix cores busy while the other issues copies).  The barrier does not
//     drain in-flight DMA.  K is read
//     with ds_read_b128, V with the gfx950 transposing ds_read_b64_tr_b16
//     straight into the MFMA A operand layout.  16-byte chunks are
//     XOR-swizzled by row so both reads are bank-conflict free; the DMA source
//     addresses apply the same swizzle.
//   * Software pipeline inside each wave: while the matrix cores compute the
//     scores of tile t+1, the VALU turns the scores of tile t into
//     probabilities; while the V-side products of tile t run, the VALU takes
//     the row max of tile t+1.  Scheduling-group hints interleave the two
//     instruction streams, and the ring slots are compile-time constants (the
//     loop is unrolled by two), so no address arithmetic runs per tile.
//   * The running max is updated lazily: the output is rescaled only when a
//     row max grows by more than 2^8; otherwise exponents are taken against
//     the stale max (p <= 256; exact after the final division by l).
//   * Causal: tiles above the diagonal are never loaded; masks run only on
//     diagonal, ragged and window tiles.  Under a sliding window every query
//     tile sees about the same number of keys, so its tiles are not paired.
//   * Scheduling: workgroup ids are dealt round-robin to the 8 XCDs, so each
//     XCD is given a contiguous range of work items; within it the items are
//     ordered (block of KV head groups, slot, group, query head of the group),
//     so the query heads sharing K/V -- and neighbouring query tiles
//     streaming the same K/V tiles -- run together on one XCD's L2.  Causal:
//     a slot runs query tile n-1-s and then its mirror s, so every workgroup
//     streams about n+1 key-tile pairs.
#include "common.h"
#include "kernels.h"
#include <algorithm>
#include <type_traits>

namespace fa {
namespace {

// Launch shape: waves per workgroup (a template parameter, 4 or 8) and keys
// per tile (compile-time).  Eight waves (256 query rows sharing each K/V
// tile, one workgroup per CU, four ring slots) halve the L2 -> LDS traffic
// and gain ~2% when the average query row sees 4K keys or more, but lose
// 2-20% on shorter rows (causal MHA 2K and 4K, 1K-key windows), where one
// workgroup per CU leaves its prologue and the wider causal diagonal
// exposed.  The launcher picks the width per call (FA_PREFILL_WAVES=4 or 8
// forces one, for testing).  32-key tiles are ~3% slower.
#ifndef FA_PREFILL_WAVES
#define FA_PREFILL_WAVES 0
#endif
#ifndef FA_PREFILL_BC
#define FA_PREFILL_BC 64
#endif
// K/V ring slots of the eight-wave kernel (2 or 4; 4 takes one workgroup
// barrier per two key tiles instead of one per tile).
#ifndef FA_PREFILL_RING8
#define FA_PREFILL_RING8 4
#endif
static_assert(FA_PREFILL_RING8 == 2 || FA_PREFILL_RING8 == 4, "ring slots: 2 or 4");
// Causal packed sequences under a window: pair query tiles as without one (1)
// or run one tile per slot (0).
#ifndef FA_WINDOW_PAIR
#define FA_WINDOW_PAIR 0
#endif
// With four slots, half of the waves copy the tiles of each step (1), or all
// of them (0).
#ifndef FA_PREFILL_HALFCOPY
#define FA_PREFILL_HALFCOPY 1
#endif
static_assert(FA_PREFILL_WAVES == 0 || FA_PREFILL_WAVES == 4 || FA_PREFILL_WAVES == 8, "waves: 0 (choose), 4 or 8");
constexpr int kBC = FA_PREFILL_BC;     // keys per tile (64, or 32)
constexpr int kMB = kBC / 32;          // 32-key MFMA blocks per tile
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

// Wait until at most n vector-memory operations of this wave are outstanding.
template <int n>
__device__ __forceinline__ void wait_vmem_le() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(n) : "memory");
}

// Workgroup barrier that does not drain the DMA ring.  The caller has
// already waited (vmcnt) for the tiles the next step reads and (lgkmcnt) for
// its own LDS reads, so only the s_barrier itself is needed; the empty asm
// statements keep the compiler from moving memory operations across it.
__device__ __forceinline__ void ring_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

typedef short i16x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ u32x2 ds_read_tr(const uint8_t* lds_byte_ptr) {
  typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
  const lds_i16x4* p = (const lds_i16x4*)(lds_byte_ptr);
  return __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16(const_cast<lds_i16x4*>(p)));
}

// One 16-byte-per-lane global -> LDS copy: lane l's 16 bytes from
// base + off land at lds_wave_base + 16*l.  Written as inline asm so that the
// compiler does not track it as a pending LDS write (its conservative
// tracking would otherwise wait for every in-flight ring tile before each LDS
// read); completion is ordered explicitly by wait_vmem_le() and the ring
// barrier.  The asm has no register outputs.
// The compiler applies no hazard rule to inline asm: s_nop 0 gives the m0
// write just before the copy its one wait state, and the build checks the
// generated code for a VALU write of the base SGPRs fewer than 5 wait
// states before a copy (isa_check.py).
__device__ __forceinline__ void dma16(const void* base, uint32_t off, uint8_t* lds_wave_base) {
  const uint32_t m0 = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) uint8_t*)lds_wave_base;
  asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, %2" ::"v"(off), "{m0}"(m0), "s"(base) : "memory");
}

// VARLEN: packed variable-length sequences (VarlenRef); N is then the longest
// sequence's query count, which sizes the grid.
template <int D, bool CAUSAL, bool VARLEN, int WAVES>
__global__ __launch_bounds__(64 * WAVES, 8 / WAVES) void prefill_bf16_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, uint16_t* __restrict__ o, float* __restrict__ lse,
    int Hq, int Hkv, int N, int n_qtiles, int n_items, int block_heads, float c, uint32_t qflip,
    VarlenRef vr) {
  constexpr int kWaves = WAVES;
  constexpr int kBR = 32 * kWaves;          // query rows per workgroup
  constexpr int KS = D / 16;                // k-steps of S^T = K Q^T
  constexpr int MD = D / 32;                // 32-row blocks of O^T
  constexpr int RC = D / 8;                 // 16-byte chunks per row
  constexpr int TILE = kBC * D * 2;         // bytes per K (or V) tile
  // Ring of K and V tiles; tile t lives in slot t % kRing.  Four-wave
  // workgroups (two per CU) keep two slots and take the workgroup barrier
  // after every tile; eight-wave workgroups (one per CU) keep four slots and
  // take it after every second tile (+0.5 to +1.3% on long rows), except the
  // non-causal packed kernel, whose tile loop spills registers with four.
  // The DMA into the ring is inline asm, so the compiler does not track it;
  // ordering is explicit (vmcnt + lgkmcnt + barrier).
  constexpr int kRing = (kWaves == 8 && (CAUSAL || !VARLEN)) ? FA_PREFILL_RING8 : 2;
  constexpr int kPer = kRing / 2;  // tiles per barrier
  // Waves that copy a tile: all of them, or (four slots) one half per step,
  // waves 0-3 in even steps and 4-7 in odd ones, so that one wave of every
  // SIMD runs its matrix products while the other issues copies.
  constexpr int kCopyWaves = (kRing == 4 && FA_PREFILL_HALFCOPY) ? kWaves / 2 : kWaves;
  constexpr int kCopyThreads = 64 * kCopyWaves;
  constexpr int CPT = kBC * RC / kCopyThreads;  // DMA chunks per copying thread per K (or V) tile
  static_assert(CPT * kCopyThreads == kBC * RC, "tile must split evenly");
  __shared__ __attribute__((aligned(1024))) uint8_t ring[kRing * 2 * TILE];
  // Byte offsets of slot s's K and V tiles.  Two slots: (K, V) pairs.  Four
  // slots: the K tiles, then the V tiles, so that every K read and (with the
  // V region's base in the lane's V offsets) every V read stays within the
  // 16-bit immediate offset of ds_read.
  constexpr auto kslot = [](int sl) { return kRing == 2 ? 2 * sl * TILE : sl * TILE; };
  constexpr auto vslot = [](int sl) { return kRing == 2 ? (2 * sl + 1) * TILE : (kRing + sl) * TILE; };
  constexpr auto vread = [](int sl) { return kRing == 2 ? (2 * sl + 1) * TILE : sl * TILE; };

  const int wave = (int)threadIdx.x >> 6;

  // ---- work item: XCD-contiguous ranges of (block of KV groups, slot, group
  // in the block, head).  A block holds at least block_heads query heads so
  // that short sequences still spread a block over an XCD's slots. ----
  int item = blockIdx.x;
  if ((n_items & 7) == 0) item = (blockIdx.x & 7) * (n_items >> 3) + (blockIdx.x >> 3);
  const int G = Hq / Hkv;
  // causal: slot s of a head runs query tiles n-1-s and s (equal work per slot)
  // Causal tiles are paired (below) unless a window gives every query tile
  // about the same number of keys.
  const bool pair = CAUSAL && !(VARLEN && !FA_WINDOW_PAIR && vr.window >= 0);
  const int n_slots = pair ? (n_qtiles + 1) / 2 : n_qtiles;
  const int n_groups = n_items / (n_slots * G);  // B * Hkv
  const int BG = G >= block_heads ? 1 : (block_heads + G - 1) / G;  // KV groups per block
  const int per_block = BG * G * n_slots;
  const int blk = item / per_block;
  const int rem = item - blk * per_block;
  const int gib = min(BG, n_groups - blk * BG);  // groups in this block (the last may be partial)
  const int tslot = rem / (gib * G);
  const int r2 = rem - tslot * gib * G;
  const int gi = r2 / G;
  const int grp = blk * BG + gi;  // (b, kv head)
  const int b = grp / Hkv;
  const int g = grp - b * Hkv;
  const int h = g * G + (r2 - gi * G);
  const int bh = b * Hq + h;

  // ---- sequence geometry: Lq queries (the last Lq positions) against Lk keys;
  // causal row i sees keys up to i + off, a window W >= 0 none before i + off - W.
  // Dense: Lq = Lk = N, off = 0, no window; packed rows have stride H*D. ----
  int Lq = N, Lk = N, qstart = 0, kstart = 0;
  if (VARLEN) {
    qstart = min(max(vr.cu_q[b], 0), vr.total_q);
    const int qe = min(max(vr.cu_q[b + 1], qstart), vr.total_q);
    kstart = min(max(vr.cu_k[b], 0), vr.total_k);
    const int ke = min(max(vr.cu_k[b + 1], kstart), vr.total_k);
    Lq = qe - qstart;
    Lk = ke - kstart;
  }
  const int off = Lk - Lq;
  const int W = VARLEN ? vr.window : -1;
  const int q_rs = VARLEN ? Hq * D : D;   // row strides (elements)
  const int kv_rs = VARLEN ? Hkv * D : D;
  const size_t qbase = VARLEN ? ((size_t)qstart * Hq + h) * D : (size_t)bh * N * D;
  const uint16_t* qh = q + qbase;
  const uint16_t* kh = k + (VARLEN ? ((size_t)kstart * Hkv + g) * D : (size_t)grp * N * D);
  const uint16_t* vh = v + (VARLEN ? ((size_t)kstart * Hkv + g) * D : (size_t)grp * N * D);

  // Causal: a slot pairs a heavy query tile with its light mirror (n-1-s, then
  // s), so every workgroup streams about the same number of key tiles and the
  // XCDs do not finish on a tail of long workgroups.
  const int n_qt = VARLEN ? (Lq + kBR - 1) / kBR : n_qtiles;  // this sequence's query tiles
  const int n_pass = pair ? 2 : 1;
  for (int pass = 0; pass < n_pass; ++pass) {
  const int qtile = !pair ? tslot : (pass == 0 ? n_qt - 1 - tslot : tslot);
  // pass 1 only when the mirror is a different tile; past a shorter
  // sequence's tiles the whole workgroup skips the pass
  if (pair && (tslot > n_qt - 1 - tslot || (pass == 1 && tslot == n_qt - 1 - tslot))) continue;
  if (VARLEN && !pair && tslot >= n_qt) continue;

  // Every lane-dependent value of the pass derives from the lane id taken
  // here (mbcnt, in volatile asm so that it is not hoisted), so the compiler
  // recomputes such values per pass instead of keeping them live (and
  // spilled) across the pass loop.
  int lp;
  asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(lp));
  const int xp = lp & 31, hp = lp >> 5;
  const int wave_s = __builtin_amdgcn_readfirstlane(wave);  // scalar: LDS bases go to M0 directly

  // Rows of this wave: q0 + wave + kWaves*j; lane column x holds row q0 + wave + kWaves*x.
  const int q0 = qtile * kBR;
  const int qrow = q0 + wave_s + kWaves * xp;
  const int wave_first = q0 + wave_s;
  const bool wave_has_rows = wave_first < Lq;
  const int wave_last_row = min(q0 + wave_s + kWaves * 31, Lq - 1);

  // Q fragments (B operand of S^T = K Q^T): column x, d = 16ks + 8hi + 0..7.
  // All loads are issued before any is used (rows past the end read the last
  // row and are zeroed afterwards).
  bf16x8 qf[KS];
  {
    const uint16_t* qr = qh + (size_t)min(qrow, Lq - 1) * q_rs + hp * 8;
    u32x4 w[KS];
#pragma unroll
    for (int kq = 0; kq < KS; ++kq) w[kq] = *reinterpret_cast<const u32x4*>(qr + kq * 16);
    const uint32_t keep = qrow < Lq ? 0xffffffffu : 0u;
#pragma unroll
    for (int kq = 0; kq < KS; ++kq) qf[kq] = __builtin_bit_cast(bf16x8, (w[kq] ^ qflip) & keep);
  }

  // ---- per-lane LDS read offsets (tile base and ks/mb/ks2 parts are immediates) ----
  int koff[KS];  // K: row x (+32 mb), chunk (2ks + hi) swizzled
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) koff[ks] = xp * (D * 2) + (((2 * ks + hp) ^ k_swz<D>(xp)) << 4);
  int voff[MD];  // V^T fragments: row 4hi + (i>>2) (+16ks2 + 8half), chunk of column md*32 + ...
  {
    // four slots: the V region's base, kept opaque so that it stays in the
    // offsets instead of being folded into the reads' immediates
    int vbase = kRing == 2 ? 0 : kRing * TILE;
    if constexpr (kRing != 2) asm volatile("" : "+v"(vbase));
    const int i = lp & 15;
    const int row = 4 * hp + (i >> 2);
    const int colc = 2 * ((lp >> 4) & 1) + ((i & 3) >> 1);  // chunk within the 32-column block
#pragma unroll
    for (int md = 0; md < MD; ++md)
      voff[md] = vbase + row * (D * 2) + (((4 * md + colc) ^ v_swz<D>(row)) << 4) + 8 * (i & 1);
  }

  // ---- DMA: chunk p = i*kCopyThreads + cw*64 + lane of the tile; byte offsets within the tile ----
  // rows of chunk i are dma_row + i*kRowStep; the swizzle depends on the row
  // only modulo 16, so one offset serves every chunk of a lane
  constexpr int kRowStep = kCopyThreads / RC;
  static_assert(kRowStep % 16 == 0, "row step keeps the swizzle");
  const int cw = wave_s % kCopyWaves;  // the wave's place among the copying waves
  const int dma_row = (cw * 64 + lp) / RC;
  const int dma_cp = lp % RC;
  const uint32_t dk_off = (uint32_t)(dma_row * kv_rs * 2 + ((dma_cp ^ k_swz<D>(dma_row)) << 4));
  const uint32_t dv_off = (uint32_t)(dma_row * kv_rs * 2 + ((dma_cp ^ v_swz<D>(dma_row)) << 4));
  f32x16 oacc[MD];
#pragma unroll
  for (int md = 0; md < MD; ++md) oacc[md] = f32x16{};
  float m_run = -INFINITY, l_run = 0.f;

  // Key tiles t_begin .. t_end-1: up to the last key any row of the tile may
  // see, from the first key of the earliest row's window.
  const int kv_end = CAUSAL ? min(Lk, q0 + kBR + off) : Lk;
  const int t_begin = W >= 0 ? max(0, q0 + off - W) / kBC : 0;
  const int ntiles = max((max(kv_end, 0) + kBC - 1) / kBC - t_begin, 0);

  // Does this wave copy the tiles of a step of parity p (wave-uniform)?
  auto copies_of = [&](int p) { return kCopyWaves == kWaves || wave_s / kCopyWaves == p; };
  // Copy rows [k0, k0+64) of the K (IS_K) or V head slab into an LDS tile.
  // Rows past the end re-read the last row (finite values whose scores are
  // masked).
  auto issue_half = [&](int t, auto is_k, uint8_t* lds) {
    constexpr bool IS_K = decltype(is_k)::value;
    const int k0 = (t_begin + t) * kBC;
    const uint8_t* base = reinterpret_cast<const uint8_t*>(IS_K ? kh : vh) + (size_t)k0 * kv_rs * 2;
    const uint32_t doff = IS_K ? dk_off : dv_off;
    if (k0 + kBC <= Lk) {
#pragma unroll
      for (int i = 0; i < CPT; ++i) {
        // half-wave copies: one scalar base per tile and the chunk's row
        // step in the lane offset, which keeps the copy bases out of the
        // SGPRs the compiler would otherwise spill to VGPR lanes
        if constexpr (kCopyWaves < kWaves)
          dma16(base, doff + (uint32_t)(i * kRowStep * kv_rs * 2), lds + (i * kCopyThreads + cw * 64) * 16);
        else
          dma16(base + (size_t)i * kRowStep * kv_rs * 2, doff, lds + (i * kCopyThreads + cw * 64) * 16);
      }
    } else {
#pragma unroll
      for (int i = 0; i < CPT; ++i) {
        // offset from the tile base: the clamped row is >= 0, so the unsigned
        // 32-bit offset never wraps
        const int r = min(dma_row + i * kRowStep, Lk - 1 - k0);
        dma16(base, doff + (r - dma_row) * kv_rs * 2, lds + (i * kCopyThreads + cw * 64) * 16);
      }
    }
  };

  // Keys past the end, after the query (causal) or before its window: only
  // diagonal, ragged and window tiles need the mask.
  auto needs_mask = [&](int k0) {
    return (k0 + kBC > Lk) || (CAUSAL && k0 + kBC - 1 > wave_first + off) ||
           (W >= 0 && k0 < wave_last_row + off - W);
  };
  // key = k0 + 4hi + o, o = 32mb + 8(r/4) + r%4: masked when o > lim (or o < lim_lo)
  auto mask_scores = [&](f32x16 (&s)[kMB], int k0) {
    const int lim = (CAUSAL ? min(qrow + off, Lk - 1) : Lk - 1) - k0 - 4 * hp;
    if (W >= 0) {
      const int lim_lo = qrow + off - W - k0 - 4 * hp;
#pragma unroll
      for (int mb = 0; mb < kMB; ++mb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int o_ = 32 * mb + 8 * (r >> 2) + (r & 3);
          s[mb][r] = (o_ > lim || o_ < lim_lo) ? -INFINITY : s[mb][r];
        }
    } else {
#pragma unroll
      for (int mb = 0; mb < kMB; ++mb)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          s[mb][r] = (32 * mb + 8 * (r >> 2) + (r & 3) > lim) ? -INFINITY : s[mb][r];
    }
  };
  // Row max of a score tile: four independent chains of three-input maxima
  // over the lane's scores, then the other half-wave's.
  auto rowmax = [&](const f32x16 (&s)[kMB]) {
    float m4[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      constexpr int per = 16 * kMB / 4;
      const int e0 = j * per;
      float m = fmaxf(s[e0 >> 4][e0 & 15], s[(e0 + 1) >> 4][(e0 + 1) & 15]);
#pragma unroll
      for (int e = e0 + 2; e + 1 < e0 + per; e += 2)
        m = fmaxf(fmaxf(m, s[e >> 4][e & 15]), s[(e + 1) >> 4][(e + 1) & 15]);
      m4[j] = m;
    }
    return max_halves(fmaxf(fmaxf(m4[0], m4[1]), fmaxf(m4[2], m4[3])));
  };
  // S^T = K Q^T for one tile: s[mb] covers keys 32mb + (8(r/4) + 4hi + r%4), query x
  auto scores = [&](f32x16 (&s)[kMB], const uint8_t* kl) {
#pragma unroll
    for (int mb = 0; mb < kMB; ++mb) s[mb] = f32x16{};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
#pragma unroll
      for (int mb = 0; mb < kMB; ++mb) {
        const bf16x8 kf = *reinterpret_cast<const bf16x8*>(kl + koff[ks] + mb * 32 * D * 2);
        s[mb] = mfma32x32x16(kf, qf[ks], s[mb]);
      }
  };
  // Every LDS read of this wave has returned (so a slot may be refilled
  // after the following barrier).
  auto lds_reads_done = [] { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); };

  // Software pipeline over key tiles: iteration t finishes tile t (its
  // probabilities and O^T += V^T P^T) while the matrix cores already compute
  // the scores of tile t+1, and takes the row max of tile t+1 while the
  // V-side products of tile t run.  Ring slot t%2 holds K(t) and V(t); during
  // iteration t, K(t+2) and V(t+1) stream into the slots that tiles t (K) and
  // t-1 (V) no longer need.
  // Score tiles alternate between two register sets (no copies): iteration t
  // finishes sc (tile t) and fills sn (tile t+1); mx_c / mx_n are their row
  // maxima (unscaled).
  f32x16 sA[kMB], sB[kMB];
  float mxA = -INFINITY, mxB = -INFINITY;

  auto iter = [&](int t, f32x16 (&sc)[kMB], f32x16 (&sn)[kMB], float& mx_c, float& mx_n, auto slot_c,
                  auto full_c) {
    constexpr int SL = decltype(slot_c)::value;     // t % kRing
    constexpr bool FULL = decltype(full_c)::value;  // tile t+1 exists
    // the barrier closes every kPer-th step and the last one (four slots:
    // after the loop)
    constexpr bool BAR = SL % kPer == kPer - 1 || !FULL;
    // K runs kPer + 1 tiles ahead, V kPer tiles: their slots were last read
    // before the previous barrier
    if (copies_of(SL & 1)) {
      if (t + kPer + 1 < ntiles) issue_half(t + kPer + 1, std::true_type{}, ring + kslot((SL + kPer + 1) % kRing));
      if (t + kPer < ntiles) issue_half(t + kPer, std::false_type{}, ring + vslot((SL + kPer) % kRing));
    }
    // lazy rescale against tile t's row max
    {
      const float mxs = mx_c * c;  // -inf stays -inf (c > 0)
      if (__any(mxs > m_run + kTau)) {
        const float mn = fmaxf(m_run, mxs);
        // packed sequences and windows: a row may still have seen no key
        const float alpha = (VARLEN && mn == -INFINITY) ? 1.0f : fast_exp2(m_run - mn);
        l_run *= alpha;
#pragma unroll
        for (int md = 0; md < MD; ++md) oacc[md] *= alpha;
        m_run = mn;
      }
    }
    const float negm = (VARLEN && m_run == -INFINITY) ? 0.f : -m_run;
    // ---- region A: scores of tile t+1 || probabilities of tile t ----
    if constexpr (FULL) scores(sn, ring + kslot((SL + 1) % kRing));
    bf16x8 pf[kBC / 16];
    {
      float lsum[2] = {0.f, 0.f};
#pragma unroll
      for (int mb = 0; mb < kMB; ++mb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float p = fast_exp2(fmaf(sc[mb][r], c, negm));
          sc[mb][r] = p;
          lsum[r & 1] += p;
        }
      l_run += lsum[0] + lsum[1];
#pragma unroll
      for (int ks2 = 0; ks2 < kBC / 16; ++ks2) {
        float tmp[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) tmp[j] = sc[ks2 >> 1][8 * (ks2 & 1) + j];
        pf[ks2] = pack_bf16x8(tmp);
      }
    }
    if constexpr (FULL) {
      // one K-fragment read and about seven VALU ops per matrix product
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
#pragma unroll
      for (int i = 0; i < KS * kMB; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, 7, 0);
        if (i + 2 < KS * kMB) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      }
      // keep the probabilities in this block: without a use here the
      // compiler sinks them past the mask branch, next to their products
#pragma unroll
      for (int ks2 = 0; ks2 < kBC / 16; ++ks2) asm volatile("" ::"v"(__builtin_bit_cast(u32x4, pf[ks2])));
      asm volatile("" ::"v"(l_run));
      const int k1 = (t_begin + t + 1) * kBC;
      if (needs_mask(k1)) mask_scores(sn, k1);
    }
    // ---- region B: O^T += V^T P^T for tile t || row max of tile t+1 ----
    const uint8_t* vl = ring + vread(SL);
#pragma unroll
    for (int ks2 = 0; ks2 < kBC / 16; ++ks2)
#pragma unroll
      for (int md = 0; md < MD; ++md) {
        const u32x2 a0 = ds_read_tr(vl + voff[md] + (16 * ks2) * D * 2);
        const u32x2 a1 = ds_read_tr(vl + voff[md] + (16 * ks2 + 8) * D * 2);
        const u32x4 a = {a0[0], a0[1], a1[0], a1[1]};
        oacc[md] = mfma32x32x16(__builtin_bit_cast(bf16x8, a), pf[ks2], oacc[md]);
      }
    if constexpr (FULL) {
      mx_n = rowmax(sn);
      __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
      for (int i = 0; i < MD * kBC / 16; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, 2, 0);
        if (i + 2 < MD * kBC / 16) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
      }
    }
    if constexpr (BAR) {
      if (t + 1 < ntiles) wait_vmem_le<0>();
      lds_reads_done();
      ring_barrier();
    }
  };

  if (ntiles > 0) {
    // prologue: K(0..kPer) and V(0..kPer-1) in flight; scores and row max of tile 0
    if (copies_of(0)) {
      issue_half(0, std::true_type{}, ring + kslot(0));
      issue_half(0, std::false_type{}, ring + vslot(0));
    }
    if (copies_of(1) && ntiles > 1) issue_half(1, std::true_type{}, ring + kslot(1));
    if constexpr (kPer == 2) {
      if (copies_of(1) && ntiles > 1) issue_half(1, std::false_type{}, ring + vslot(1));
      if (copies_of(0) && ntiles > 2) issue_half(2, std::true_type{}, ring + kslot(2));
    }
    wait_vmem_le<0>();
    ring_barrier();
    scores(sA, ring + kslot(0));
    if (needs_mask(t_begin * kBC)) mask_scores(sA, t_begin * kBC);
    mxA = rowmax(sA);
    lds_reads_done();
    ring_barrier();  // K(0)'s slot is refilled by the first steps
    // unrolled by kRing: ring slots are immediates in every LDS access
    using I0 = std::integral_constant<int, 0>;
    using I1 = std::integral_constant<int, 1>;
    using I2 = std::integral_constant<int, 2>;
    using I3 = std::integral_constant<int, 3>;
    using T_ = std::true_type;
    using F_ = std::false_type;
    int t = 0;
    if constexpr (kRing == 2) {
      for (; t + 2 < ntiles; t += 2) {
        iter(t, sA, sB, mxA, mxB, I0{}, T_{});
        iter(t + 1, sB, sA, mxB, mxA, I1{}, T_{});
      }
      if (t + 1 < ntiles) {
        iter(t, sA, sB, mxA, mxB, I0{}, T_{});
        iter(t + 1, sB, sA, mxB, mxA, I1{}, F_{});
      } else {
        iter(t, sA, sB, mxA, mxB, I0{}, F_{});
      }
    } else {
      // Four slots: the last step also computes the scores of the slot after
      // it (stale keys no copy is writing), which nothing uses; one code copy
      // per slot serves every tile count.
      for (; t < ntiles; t += 4) {
        iter(t, sA, sB, mxA, mxB, I0{}, T_{});
        if (t + 1 >= ntiles) break;
        iter(t + 1, sB, sA, mxB, mxA, I1{}, T_{});
        if (t + 2 >= ntiles) break;
        iter(t + 2, sA, sB, mxA, mxB, I2{}, T_{});
        if (t + 3 >= ntiles) break;
        iter(t + 3, sB, sA, mxB, mxA, I3{}, T_{});
      }
      // no copy is in flight after the last step
      lds_reads_done();
      ring_barrier();
    }
  }

  // ---- epilogue: O = O^T / l, lse = m ln2 + ln l ----
  if (wave_has_rows) {
  // the row and the output addresses come from the lane id taken afresh, so
  // that no 64-bit address stays live (and spilled) through the tile loop
  int le;
  asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(le));
  const int row_e = q0 + wave_s + kWaves * (le & 31);
  const int he = le >> 5;
  const float lt = sum_halves(l_run);
  // a packed causal row with i + off < 0 (or a sequence without keys) sees no
  // key: o = 0, lse = -inf, decided by position, not by arithmetic
  const bool empty = VARLEN && ((CAUSAL && row_e + off < 0) || Lk == 0);
  const float inv = empty ? 0.f : 1.0f / lt;
  if (row_e < Lq) {
    uint16_t* orow = o + qbase + (size_t)row_e * q_rs;
#pragma unroll
    for (int md = 0; md < MD; ++md)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int d0 = md * 32 + 8 * g4 + 4 * he;
        u32x2 w = {pack_bf16x2(oacc[md][4 * g4 + 0] * inv, oacc[md][4 * g4 + 1] * inv),
                   pack_bf16x2(oacc[md][4 * g4 + 2] * inv, oacc[md][4 * g4 + 3] * inv)};
        if (empty) w = u32x2{0u, 0u};
        *reinterpret_cast<u32x2*>(orow + d0) = w;
      }
    if (lse != nullptr && he == 0) {
      // one rounding (fma), whatever the surrounding code
      const float lv = empty ? -INFINITY : fmaf(m_run, kLn2, __logf(lt));
      if (VARLEN)
        lse[(size_t)h * vr.total_q + qstart + row_e] = lv;
      else
        lse[(size_t)bh * N + row_e] = lv;
    }
  }
  }  // wave_has_rows
  }  // pass
}

// Query heads per scheduling block.  With causal tiles paired, every slot of
// a head carries about the same work, so one head per block suffices once a
// head has 16 or more slots; short sequences group 4 heads so that a block
// still spans an XCD's ~64 workgroup slots (measured on causal MHA d128,
// N 1K..16K: within 1% of the best block size at every length).
int block_heads_for(int n_slots) { return n_slots < 16 ? 4 : 1; }

template <int D, bool CAUSAL, bool VARLEN, int WAVES>
hipError_t launch(const PrefillArgs& a, hipStream_t stream) {
  constexpr int kBR = 32 * WAVES;  // query rows per workgroup
  const int n_qtiles = (a.N + kBR - 1) / kBR;
  // causal slots pair two query tiles, except under a window (as in the kernel)
  const bool pair = CAUSAL && !(VARLEN && !FA_WINDOW_PAIR && a.varlen.window >= 0);
  const int n_slots = pair ? (n_qtiles + 1) / 2 : n_qtiles;
  const long long items = (long long)n_slots * a.B * a.Hq;
  if (items > 0x7fffffffLL) return hipErrorInvalidValue;
  const int block_heads = block_heads_for(n_slots);
  hipLaunchKernelGGL((prefill_bf16_kernel<D, CAUSAL, VARLEN, WAVES>), dim3((unsigned)items), dim3(64 * WAVES), 0,
                     stream,
                     static_cast<const uint16_t*>(a.q), static_cast<const uint16_t*>(a.k),
                     static_cast<const uint16_t*>(a.v), static_cast<uint16_t*>(a.o), a.lse, a.Hq, a.Hkv,
                     a.N, n_qtiles, (int)items, block_heads, a.c, a.neg ? 0x80008000u : 0u, a.varlen);
  return hipGetLastError();
}

// Eight waves when the average query row sees at least 4096 keys (d = 128;
// the wider workgroup was measured there only).  Dense rows see N keys, or
// (N + 1) / 2 on average under the causal mask.  Packed sequences of average
// lengths Lq = total_q / B, Lk = total_k / B see Lk keys, or Lk - (Lq - 1) / 2
// under the bottom-right causal mask (the dense value for one full-length
// sequence, so both entry points pick the same width and agree bit for bit);
// a window caps them at window_left + 1.
bool wide_launch(const PrefillArgs& a) {
  if (FA_PREFILL_WAVES != 0) return FA_PREFILL_WAVES == 8;
  if (a.d != 128 || a.B <= 0) return false;
  double keys;
  if (a.varlen.cu_q != nullptr) {
    keys = (double)a.varlen.total_k / a.B - (a.causal ? 0.5 * ((double)a.varlen.total_q / a.B - 1.0) : 0.0);
    if (a.varlen.window >= 0) keys = std::min(keys, (double)a.varlen.window + 1);
  } else {
    keys = a.causal ? 0.5 * ((double)a.N + 1) : (double)a.N;
  }
  return keys >= 4096.0;
}

template <int D, bool VARLEN>
hipError_t launch_c(const PrefillArgs& a, hipStream_t stream) {
  if (wide_launch(a))
    return a.causal ? launch<D, true, VARLEN, 8>(a, stream) : launch<D, false, VARLEN, 8>(a, stream);
  return a.causal ? launch<D, true, VARLEN, 4>(a, stream) : launch<D, false, VARLEN, 4>(a, stream);
}

}  // namespace

hipError_t launch_prefill_bf16(const PrefillArgs& a, hipStream_t stream) {
  const bool varlen = a.varlen.cu_q != nullptr;
  if (varlen && (a.varlen.cu_k == nullptr || a.varlen.total_q <= 0 || a.varlen.total_k <= 0 || a.varlen.window < -1))
    return hipErrorInvalidValue;
  if (a.d == 128) return varlen ? launch_c<128, true>(a, stream) : launch_c<128, false>(a, stream);
  if (a.d == 64) return varlen ? launch_c<64, true>(a, stream) : launch_c<64, false>(a, stream);
  return hipErrorInvalidValue;
}

}  // namespace fa
