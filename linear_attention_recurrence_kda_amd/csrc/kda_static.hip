// kda_chunk_prefill_static: kda_chunk_prefill with its workspace in a
// file-scope device array instead of a caller buffer, for callers that cannot
// allocate device memory.  The array is this library's on every GPU it runs
// on (each GPU holds its own copy until the process ends); host code reaches
// it only through the address hipGetSymbolAddress returns for the current
// device, looked up once per device.
#include <hip/hip_runtime.h>

#include <cstdio>
#include <mutex>

#include "kda_hostutil.hpp"

using namespace kda_host;

namespace {

constexpr size_t kScratchBytes = size_t{KDA_STATIC_SCRATCH_MB} << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_ptr[kMaxDevices] = {};

// The scratch array's device address on the current device (looked up on the
// first call there).
int scratch_ptr(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_status(e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices) return fail(KDA_EUNSUPPORTED, "device %d beyond %d", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_mu);
  if (g_ptr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_status(e, "hipGetSymbolAddress(scratch)");
    g_ptr[dev] = p;
  }
  *out = g_ptr[dev];
  return KDA_OK;
}

}  // namespace

extern "C" {

int kda_chunk_prefill_static(const void* q, const void* k, const void* v, const void* a,
                             const void* beta, kda_dtype in_dtype, int32_t H, int32_t dk, int32_t dv,
                             int32_t chunk, const int32_t* cu_seqlens_host, int32_t n_seqs,
                             const float* s0, void* o, float* s_final, const int32_t* ckpt_cu_host,
                             const int32_t* ckpt_pos_host, const int32_t* ckpt_slot_host,
                             int64_t n_ckpt, float* page_pool, int64_t page_elems, int64_t n_slots,
                             int32_t* err_flag, void* stream) {
  void* ws = nullptr;
  int st = scratch_ptr(&ws);
  if (st) return st;
  st = kda_chunk_prefill(q, k, v, a, beta, in_dtype, H, dk, dv, chunk, cu_seqlens_host, n_seqs, s0, o,
                         s_final, ckpt_cu_host, ckpt_pos_host, ckpt_slot_host, n_ckpt, page_pool, page_elems,
                         n_slots, ws, kScratchBytes, err_flag, stream);
  if (st == KDA_EWORKSPACE) {
    const std::string why = kda_last_error();
    return fail(KDA_EWORKSPACE, "the call does not fit the static scratch of %zu bytes (%s)", kScratchBytes,
                why.c_str());
  }
  return st;
}

size_t kda_static_scratch_bytes(void) { return kScratchBytes; }

}  // extern "C"
