// C-ABI layer of libfa.so: argument validation, device check, dispatch.
// Every check that can fail on arguments alone runs before any HIP call.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <mutex>
#include <vector>

#include "../../include/fa.h"
#include "common.h"
#include "kernels.h"

namespace {

constexpr int kMaxDevices = 64;
// 0 = unknown, 1 = gfx950, 2 = other architecture
int g_arch_state[kMaxDevices] = {0};
std::mutex g_arch_mutex;

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

int check_device() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return FA_ERR_HIP;
  if (dev < 0 || dev >= kMaxDevices) return FA_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_arch_mutex);
  if (g_arch_state[dev] == 0) {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return FA_ERR_HIP;
    const char* want = "gfx950";
    bool ok = true;
    for (int i = 0; want[i] != '\0'; ++i)
      if (prop.gcnArchName[i] != want[i]) ok = false;
    g_arch_state[dev] = ok ? 1 : 2;
  }
  return g_arch_state[dev] == 1 ? FA_OK : FA_ERR_UNSUPPORTED;
}

float softmax_coeff(float scale) {
  float c = std::fabs(scale) * fa::kLog2e;
  return c < fa::kMinC ? fa::kMinC : c;
}

int check_common(int B, int Hq, int Hkv, int d, float scale) {
  if (B <= 0 || Hq <= 0 || Hkv <= 0 || d <= 0) return FA_ERR_INVALID_ARG;
  if (Hq % Hkv != 0) return FA_ERR_INVALID_ARG;
  // the kernels exponentiate in base 2 with the coefficient |scale| log2(e),
  // which must itself be a finite fp32 number
  if (!std::isfinite(scale) || !std::isfinite(std::fabs(scale) * fa::kLog2e)) return FA_ERR_INVALID_ARG;
  if (d != 64 && d != 128) return FA_ERR_UNSUPPORTED;
  return FA_OK;
}

int prefill_common(const void* q, const void* k, const void* v, void* o, float* lse, int B, int Hq,
                   int Hkv, int N, int d, int causal, float scale, void* stream, bool bf16) {
  if (q == nullptr || k == nullptr || v == nullptr || o == nullptr) return FA_ERR_INVALID_ARG;
  if (N <= 0 || (causal != 0 && causal != 1)) return FA_ERR_INVALID_ARG;
  int st = check_common(B, Hq, Hkv, d, scale);
  if (st != FA_OK) return st;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16)) return FA_ERR_INVALID_ARG;
  if (lse != nullptr && !aligned(lse, 4)) return FA_ERR_INVALID_ARG;
  // grid limits: B*Hq*ceil(N/rows) workgroups must fit in 31 bits
  const int rows = bf16 ? fa::kPrefillBf16Rows : fa::kPrefillF32Rows;
  if ((long long)B * Hq * ((N + rows - 1) / rows) > 0x7fffffffLL) return FA_ERR_INVALID_ARG;
  st = check_device();
  if (st != FA_OK) return st;
  fa::PrefillArgs a{q, k, v, o, lse, B, Hq, Hkv, N, d, causal != 0, softmax_coeff(scale), scale < 0.f};
  a.scale_abs = std::fabs(scale);
  hipError_t e = bf16 ? fa::launch_prefill_bf16(a, static_cast<hipStream_t>(stream))
                      : fa::launch_prefill_f32(a, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? FA_OK : FA_ERR_HIP;
}

int decode_check(const void* q, const void* kc, const void* vc, const int32_t* seqlens, void* o, int B,
                 int Hq, int Hkv, int maxlen, int d, float scale) {
  if (q == nullptr || kc == nullptr || vc == nullptr || seqlens == nullptr || o == nullptr)
    return FA_ERR_INVALID_ARG;
  if (maxlen <= 0) return FA_ERR_INVALID_ARG;
  int st = check_common(B, Hq, Hkv, d, scale);
  if (st != FA_OK) return st;
  if (B > 65535 || Hq > 65535) return FA_ERR_INVALID_ARG;
  if (!aligned(q, 16) || !aligned(kc, 16) || !aligned(vc, 16) || !aligned(o, 16) || !aligned(seqlens, 4))
    return FA_ERR_INVALID_ARG;
  return FA_OK;
}

int decode_run(const void* q, const void* kc, const void* vc, const int32_t* seqlens, void* o, int B, int Hq,
               int Hkv, int maxlen, int d, float scale, void* ws, size_t ws_bytes, void* stream, bool bf16,
               fa::PagedKV paged = fa::PagedKV{}) {
  int st = decode_check(q, kc, vc, seqlens, o, B, Hq, Hkv, maxlen, d, scale);
  if (st != FA_OK) return st;
  const size_t need = fa::decode_workspace_bytes(B, Hq, Hkv, maxlen, d);
  hipStream_t s = static_cast<hipStream_t>(stream);
  bool owned = false;
  if (ws != nullptr) {
    if (ws_bytes < need || !aligned(ws, 256)) return FA_ERR_INVALID_ARG;
    st = check_device();
    if (st != FA_OK) return st;
  } else {
    st = check_device();
    if (st != FA_OK) return st;
    if (hipMallocAsync(&ws, need, s) != hipSuccess) {
      (void)hipGetLastError();
      return FA_ERR_NO_MEMORY;
    }
    owned = true;
  }
  fa::DecodeArgs a{q, kc, vc, seqlens, o, B, Hq, Hkv, maxlen, d, softmax_coeff(scale), scale < 0.f, ws,
                   owned ? need : ws_bytes, paged};
  hipError_t e = bf16 ? fa::launch_decode_bf16(a, s) : fa::launch_decode_f32(a, s);
  if (owned) {
    hipError_t f = hipFreeAsync(ws, s);
    if (e == hipSuccess) e = f;
  }
  return e == hipSuccess ? FA_OK : FA_ERR_HIP;
}

// Paged-cache geometry: page_size a power of two in [16, 2^20], logical
// length max_pages * page_size within int.  Returns the page shift, or -1.
int paged_shift(int num_pages, int page_size, int max_pages) {
  if (num_pages <= 0 || max_pages <= 0 || page_size < 16 || page_size > (1 << 20)) return -1;
  if ((page_size & (page_size - 1)) != 0) return -1;
  if ((long long)max_pages * page_size > 0x7fffffffLL) return -1;
  int shift = 0;
  while ((1 << shift) < page_size) ++shift;
  return shift;
}

}  // namespace

extern "C" {

const char* fa_strerror(int status) {
  switch (status) {
    case FA_OK:
      return "FA_OK: success";
    case FA_ERR_INVALID_ARG:
      return "FA_ERR_INVALID_ARG: invalid argument";
    case FA_ERR_UNSUPPORTED:
      return "FA_ERR_UNSUPPORTED: head dimension or device not supported";
    case FA_ERR_HIP:
      return "FA_ERR_HIP: HIP runtime or launch failure";
    case FA_ERR_NO_MEMORY:
      return "FA_ERR_NO_MEMORY: workspace allocation failed";
    case FA_ERR_TOO_LARGE:
      return "FA_ERR_TOO_LARGE: sizes exceed the fixed scratch of fa_decode_noalloc";
    default:
      return "unknown fa_status";
  }
}

int fa_version(void) { return 100; }

int fa_prefill(const void* q, const void* k, const void* v, void* o, float* lse, int B, int Hq, int Hkv,
               int N, int d, int causal, float scale, void* stream) {
  return prefill_common(q, k, v, o, lse, B, Hq, Hkv, N, d, causal, scale, stream, true);
}

int fa_prefill_f32(const float* q, const float* k, const float* v, float* o, float* lse, int B, int Hq,
                   int Hkv, int N, int d, int causal, float scale, void* stream) {
  return prefill_common(q, k, v, o, lse, B, Hq, Hkv, N, d, causal, scale, stream, false);
}

int fa_prefill_varlen(const void* q, const void* k, const void* v, void* o, float* lse,
                      const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k, int B, int Hq, int Hkv,
                      int total_q, int total_k, int max_seqlen_q, int d, int causal, int window_left,
                      float scale, void* stream) {
  if (q == nullptr || k == nullptr || v == nullptr || o == nullptr || cu_seqlens_q == nullptr ||
      cu_seqlens_k == nullptr)
    return FA_ERR_INVALID_ARG;
  if (causal != 0 && causal != 1) return FA_ERR_INVALID_ARG;
  if (total_q <= 0 || total_k <= 0 || max_seqlen_q <= 0 || max_seqlen_q > total_q || window_left < -1)
    return FA_ERR_INVALID_ARG;
  int st = check_common(B, Hq, Hkv, d, scale);
  if (st != FA_OK) return st;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16) || !aligned(cu_seqlens_q, 4) ||
      !aligned(cu_seqlens_k, 4))
    return FA_ERR_INVALID_ARG;
  if (lse != nullptr && !aligned(lse, 4)) return FA_ERR_INVALID_ARG;
  // one 64-key tile of packed K rows must be addressable with 32-bit offsets
  if ((long long)64 * Hkv * d * 2 > 0x7fffffffLL) return FA_ERR_INVALID_ARG;
  if ((long long)B * Hq * ((max_seqlen_q + 127) / 128) > 0x7fffffffLL) return FA_ERR_INVALID_ARG;
  st = check_device();
  if (st != FA_OK) return st;
  fa::PrefillArgs a{q, k, v, o, lse, B, Hq, Hkv, max_seqlen_q, d, causal != 0, softmax_coeff(scale), scale < 0.f};
  a.varlen.cu_q = cu_seqlens_q;
  a.varlen.cu_k = cu_seqlens_k;
  a.varlen.total_q = total_q;
  a.varlen.total_k = total_k;
  a.varlen.window = window_left;
  return fa::launch_prefill_bf16(a, static_cast<hipStream_t>(stream)) == hipSuccess ? FA_OK : FA_ERR_HIP;
}

size_t fa_prefill_backward_workspace_bytes(int B, int Hq, int N) {
  if (B <= 0 || Hq <= 0 || N <= 0) return 0;
  return fa::backward_workspace_bytes(B, Hq, N);
}

int fa_prefill_backward(const void* q, const void* k, const void* v, const void* o, const void* dout,
                        const float* lse, void* dq, void* dk, void* dv, int B, int Hq, int Hkv, int N, int d,
                        int causal, float scale, void* workspace, size_t workspace_bytes, void* stream) {
  if (q == nullptr || k == nullptr || v == nullptr || o == nullptr || dout == nullptr || lse == nullptr ||
      dq == nullptr || dk == nullptr || dv == nullptr)
    return FA_ERR_INVALID_ARG;
  if (N <= 0 || (causal != 0 && causal != 1)) return FA_ERR_INVALID_ARG;
  int st = check_common(B, Hq, Hkv, d, scale);
  if (st != FA_OK) return st;
  const void* p16[] = {q, k, v, o, dout, dq, dk, dv};
  for (const void* p : p16)
    if (!aligned(p, 16)) return FA_ERR_INVALID_ARG;
  if (!aligned(lse, 4)) return FA_ERR_INVALID_ARG;
  if ((long long)B * Hq * ((N + 127) / 128) > 0x7fffffffLL) return FA_ERR_INVALID_ARG;
  const size_t need = fa::backward_workspace_bytes(B, Hq, N);
  hipStream_t s = static_cast<hipStream_t>(stream);
  bool owned = false;
  if (workspace != nullptr) {
    if (workspace_bytes < need || !aligned(workspace, 256)) return FA_ERR_INVALID_ARG;
    st = check_device();
    if (st != FA_OK) return st;
  } else {
    st = check_device();
    if (st != FA_OK) return st;
    if (hipMallocAsync(&workspace, need, s) != hipSuccess) {
      (void)hipGetLastError();
      return FA_ERR_NO_MEMORY;
    }
    owned = true;
  }
  fa::BackwardArgs a{q, k, v, o, dout, lse, dq, dk, dv, B, Hq, Hkv, N, d, causal != 0, scale, workspace,
                     owned ? need : workspace_bytes};
  hipError_t e = fa::launch_backward_bf16(a, s);
  if (owned) {
    hipError_t f = hipFreeAsync(workspace, s);
    if (e == hipSuccess) e = f;
  }
  return e == hipSuccess ? FA_OK : FA_ERR_HIP;
}

size_t fa_decode_workspace_bytes(int B, int Hq, int Hkv, int maxlen, int d) {
  if (B <= 0 || Hq <= 0 || Hkv <= 0 || maxlen <= 0 || (d != 64 && d != 128) || Hq % Hkv != 0) return 0;
  return fa::decode_workspace_bytes(B, Hq, Hkv, maxlen, d);
}

int fa_decode(const void* q, const void* kcache, const void* vcache, const int32_t* seqlens, void* o, int B,
              int Hq, int Hkv, int maxlen, int d, float scale, void* stream) {
  return decode_run(q, kcache, vcache, seqlens, o, B, Hq, Hkv, maxlen, d, scale, nullptr, 0, stream, true);
}

int fa_decode_ws(const void* q, const void* kcache, const void* vcache, const int32_t* seqlens, void* o,
                 int B, int Hq, int Hkv, int maxlen, int d, float scale, void* workspace,
                 size_t workspace_bytes, void* stream) {
  if (workspace == nullptr) return FA_ERR_INVALID_ARG;
  return decode_run(q, kcache, vcache, seqlens, o, B, Hq, Hkv, maxlen, d, scale, workspace, workspace_bytes,
                    stream, true);
}

int fa_decode_noalloc(const void* q, const void* kcache, const void* vcache, const int32_t* seqlens, void* o,
                      int B, int Hq, int Hkv, int maxlen, int d, float scale, void* stream) {
  int st = decode_check(q, kcache, vcache, seqlens, o, B, Hq, Hkv, maxlen, d, scale);
  if (st != FA_OK) return st;
  if (fa::decode_noalloc_bytes(B, Hq, Hkv, maxlen, d) > fa::kDecodeScratchBytes) return FA_ERR_TOO_LARGE;
  st = check_device();
  if (st != FA_OK) return st;
  void* ws = nullptr;
  if (fa::decode_scratch_address(&ws) != hipSuccess) return FA_ERR_HIP;
  fa::DecodeArgs a{q, kcache, vcache, seqlens, o, B, Hq, Hkv, maxlen, d, softmax_coeff(scale), scale < 0.f, ws,
                   fa::kDecodeScratchBytes, fa::PagedKV{}};
  return fa::launch_decode_bf16(a, static_cast<hipStream_t>(stream)) == hipSuccess ? FA_OK : FA_ERR_HIP;
}

size_t fa_decode_paged_workspace_bytes(int B, int Hq, int Hkv, int page_size, int max_pages, int d) {
  if (paged_shift(1, page_size, max_pages) < 0) return 0;
  return fa_decode_workspace_bytes(B, Hq, Hkv, max_pages * page_size, d);
}

int fa_decode_paged(const void* q, const void* kpages, const void* vpages, const int32_t* block_table,
                    const int32_t* seqlens, void* o, int B, int Hq, int Hkv, int num_pages, int page_size,
                    int max_pages, int d, float scale, void* workspace, size_t workspace_bytes, void* stream) {
  const int shift = paged_shift(num_pages, page_size, max_pages);
  if (shift < 0 || block_table == nullptr || !aligned(block_table, 4)) return FA_ERR_INVALID_ARG;
  fa::PagedKV pg;
  pg.block_table = block_table;
  pg.max_pages = max_pages;
  pg.num_pages = num_pages;
  pg.page_shift = shift;
  return decode_run(q, kpages, vpages, seqlens, o, B, Hq, Hkv, max_pages * page_size, d, scale, workspace,
                    workspace_bytes, stream, true, pg);
}

int fa_decode_f32(const float* q, const float* kcache, const float* vcache, const int32_t* seqlens, float* o,
                  int B, int Hq, int Hkv, int maxlen, int d, float scale, void* stream) {
  return decode_run(q, kcache, vcache, seqlens, o, B, Hq, Hkv, maxlen, d, scale, nullptr, 0, stream, false);
}

int fa_decode_f32_ws(const float* q, const float* kcache, const float* vcache, const int32_t* seqlens,
                     float* o, int B, int Hq, int Hkv, int maxlen, int d, float scale, void* workspace,
                     size_t workspace_bytes, void* stream) {
  if (workspace == nullptr) return FA_ERR_INVALID_ARG;
  return decode_run(q, kcache, vcache, seqlens, o, B, Hq, Hkv, maxlen, d, scale, workspace, workspace_bytes,
                    stream, false);
}

}  // extern "C"
