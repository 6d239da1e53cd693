// Internal launch interface between the C-ABI layer (fa_api.hip) and the
// kernels.  All sizes are validated by the caller; pointers are device memory.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/fa.h"

namespace fa {

// Softmax runs in base 2: exp(scale*s) = exp2(c*s) with c = |scale|*log2(e),
// and a negative scale is applied by flipping the sign of q (exact).  c is
// clamped below at kMinC so that c*(-inf) stays -inf (a zero scale would
// otherwise turn masked scores into NaN); at that size c*s rounds every
// exponent of a finite score to 0 exactly as a zero scale would.
constexpr float kMinC = 1e-30f;

// Packed variable-length sequences: q/o [total_q, Hq, d], k/v [total_k, Hkv, d],
// lse [Hq, total_q]; sequence b owns query rows cu_q[b] .. cu_q[b+1]-1 and key
// rows cu_k[b] .. cu_k[b+1]-1 (device arrays; clamped into range on the
// device).  Its queries are the last n_q positions (causal row i sees keys up
// to i + n_k - n_q); window >= 0 also drops keys before that bound - window.
struct VarlenRef {
  const int32_t* cu_q = nullptr;
  const int32_t* cu_k = nullptr;
  int total_q = 0;
  int total_k = 0;
  int window = -1;
};

struct PrefillArgs {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;  // may be null
  int B, Hq, Hkv, N, d;  // varlen: N = the longest sequence's query count
  bool causal;
  float c;       // |scale| * log2(e), >= kMinC
  bool neg;      // scale < 0: use -q
  VarlenRef varlen;  // cu_q == nullptr: dense [B, H, N, d] layout (bf16 only otherwise)
  float scale_abs = 0.f;  // |scale|: the fp32 kernel forms its coefficient in fp64 from it
};

// Paged KV cache: k/v point at page pools [num_pages, Hkv, page_size, d];
// block_table [B, max_pages] maps a sequence's logical page i (cache entries
// i*page_size .. (i+1)*page_size - 1) to a pool page.  block_table == nullptr
// means the contiguous layout [B, Hkv, maxlen, d].
struct PagedKV {
  const int32_t* block_table = nullptr;
  int max_pages = 0;
  int num_pages = 0;
  int page_shift = 0;  // page_size = 1 << page_shift
};

struct DecodeArgs {
  const void* q;
  const void* k;
  const void* v;
  const int32_t* seqlens;
  void* o;
  int B, Hq, Hkv, maxlen, d;  // paged: maxlen = max_pages * page_size
  float c;
  bool neg;
  void* ws;        // >= decode_workspace_bytes(...)
  size_t ws_bytes; // size of ws; each launch checks its own partial layout fits
  PagedKV paged;   // bf16 only
};

// Backward: q, o, dout, dq [B, Hq, N, d]; k, v, dk, dv [B, Hkv, N, d] (bf16);
// lse [B, Hq, N] fp32 (natural log, from the forward).
struct BackwardArgs {
  const void* q;
  const void* k;
  const void* v;
  const void* o;
  const void* dout;
  const float* lse;
  void* dq;
  void* dk;
  void* dv;
  int B, Hq, Hkv, N, d;
  bool causal;
  float scale;      // signed
  void* ws;         // >= backward_workspace_bytes(B, Hq, N)
  size_t ws_bytes;
};

hipError_t launch_prefill_bf16(const PrefillArgs& a, hipStream_t stream);
hipError_t launch_backward_bf16(const BackwardArgs& a, hipStream_t stream);
size_t backward_workspace_bytes(int B, int Hq, int N);
hipError_t launch_prefill_f32(const PrefillArgs& a, hipStream_t stream);
hipError_t launch_decode_bf16(const DecodeArgs& a, hipStream_t stream);
hipError_t launch_decode_f32(const DecodeArgs& a, hipStream_t stream);

// Keys per split-KV chunk of the fp32 decode path (the bf16 path picks its
// chunk per launch).
constexpr int kDecodeChunk = 512;

// Query rows per workgroup: the bf16 prefill kernels' tile (4 waves; 8-wave
// launches take 256, so 128 bounds the grid) and the fp32 prefill kernel's.
constexpr int kPrefillBf16Rows = 128;
constexpr int kPrefillF32Rows = 16;
size_t decode_workspace_bytes(int B, int Hq, int Hkv, int maxlen, int d);

// Allocation-free bf16 decode: the partials live in a fixed device array of
// kDecodeScratchBytes (one per GPU, for the life of the process).
constexpr size_t kDecodeScratchBytes = FA_DECODE_NOALLOC_SCRATCH_BYTES;
// Bytes of that array a bf16 decode of these sizes uses.
size_t decode_noalloc_bytes(int B, int Hq, int Hkv, int maxlen, int d);
// Device address of the current device's array (looked up once per device).
hipError_t decode_scratch_address(void** ptr);

}  // namespace fa
