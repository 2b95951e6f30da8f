// The raw-input ring (RawInputRing of the "Serve 模块交互式演示" page, Tab 4
// "ReplaySSM"): during verification each draft step's raw inputs
// (q, k, v, a, beta) of a session are written into that session's ring of
// fixed capacity, overwriting the oldest entry once it is full; window()
// hands the held entries back oldest first in the draft-projection layout
// (draft, B, H, D) that verify-and-replay reads; commit replays the accepted
// prefix and resets the ring.
//
// Layout: per field a [n_slots][capacity][H][D] array in the input dtype (D =
// dk for q, k, a, dv for v, 1 for beta) and count [n_slots], the pushes since
// the last reset.  One workgroup per session moves that session's whole
// step: 16-byte pieces where the field's row is a whole number of them, then
// element by element for the rest.
#include "kda_device.hpp"
#include "kda_internal.hpp"

namespace kda {
namespace {

constexpr int kRingThreads = 256;

// Copy n elements of es bytes (es = 2 or 4); src and dst 16-byte aligned.
__device__ __forceinline__ void copy_elems(char* dst, const char* src, int64_t n, int es) {
  const int64_t bytes = n * es, n16 = bytes / 16;
  for (int64_t i = threadIdx.x; i < n16; i += blockDim.x)
    reinterpret_cast<uint4*>(dst)[i] = reinterpret_cast<const uint4*>(src)[i];
  for (int64_t i = n16 * 16 / 2 + threadIdx.x; i < bytes / 2; i += blockDim.x)
    reinterpret_cast<uint16_t*>(dst)[i] = reinterpret_cast<const uint16_t*>(src)[i];
}
__device__ __forceinline__ void zero_elems(char* dst, int64_t n, int es) {
  const int64_t bytes = n * es, n16 = bytes / 16;
  for (int64_t i = threadIdx.x; i < n16; i += blockDim.x)
    reinterpret_cast<uint4*>(dst)[i] = make_uint4(0, 0, 0, 0);
  for (int64_t i = n16 * 16 / 2 + threadIdx.x; i < bytes / 2; i += blockDim.x)
    reinterpret_cast<uint16_t*>(dst)[i] = 0;
}

__global__ __launch_bounds__(kRingThreads) void ring_push_kernel(RingArgs r, const int32_t* __restrict__ slot,
                                                             int B, RingStep in) {
  const int b = blockIdx.x;
  const int s = slot[b];
  if (s < 0 || s >= r.n_slots) {  // the whole workgroup skips the session
    if (threadIdx.x == 0 && r.err_flag != nullptr) *r.err_flag = 1;
    return;
  }
  const int pos = r.count[s] % r.capacity;
  for (int f = 0; f < 5; ++f) {
    const int64_t e = r.elems[f];  // elements of one entry (H * D)
    copy_elems(static_cast<char*>(r.field[f]) + ((static_cast<int64_t>(s) * r.capacity + pos) * e) * r.es,
               static_cast<const char*>(in.field[f]) + static_cast<int64_t>(b) * e * r.es, e, r.es);
  }
  __syncthreads();  // every thread has read count[s]
  if (threadIdx.x == 0) r.count[s] = r.count[s] + 1;
}

__global__ __launch_bounds__(kRingThreads) void ring_window_kernel(RingArgs r, const int32_t* __restrict__ slot,
                                                               int B, RingStep out, int32_t* n_valid) {
  const int b = blockIdx.x, i = blockIdx.y;  // session, row of the window
  const int s = slot[b];
  const bool ok = s >= 0 && s < r.n_slots;
  if (!ok && i == 0 && threadIdx.x == 0 && r.err_flag != nullptr) *r.err_flag = 1;
  const int c = ok ? r.count[s] : 0;
  const int n = c < r.capacity ? c : r.capacity;
  if (i == 0 && threadIdx.x == 0 && n_valid != nullptr) n_valid[b] = n;
  const int pos = (c - n + i) % r.capacity;
  for (int f = 0; f < 5; ++f) {
    const int64_t e = r.elems[f];
    char* dst = static_cast<char*>(out.field[f]) + ((static_cast<int64_t>(i) * B + b) * e) * r.es;
    if (i < n)
      copy_elems(dst, static_cast<const char*>(r.field[f]) + ((static_cast<int64_t>(s) * r.capacity + pos) * e) * r.es,
                 e, r.es);
    else
      zero_elems(dst, e, r.es);
  }
}

__global__ void ring_reset_kernel(RingArgs r, const int32_t* __restrict__ slot, int B) {
  const int b = blockIdx.x * blockDim.x + threadIdx.x;
  if (b >= B) return;
  const int s = slot[b];
  if (s < 0 || s >= r.n_slots) {
    if (r.err_flag != nullptr) *r.err_flag = 1;
    return;
  }
  r.count[s] = 0;
}

}  // namespace

hipError_t launch_ring_push(const RingArgs& r, const int32_t* slot, int B, const RingStep& in) {
  if (B == 0) return hipSuccess;
  hipLaunchKernelGGL(ring_push_kernel, dim3(B), dim3(kRingThreads), 0, r.stream, r, slot, B, in);
  return hipGetLastError();
}

hipError_t launch_ring_window(const RingArgs& r, const int32_t* slot, int B, const RingStep& out,
                              int32_t* n_valid) {
  if (B == 0) return hipSuccess;
  hipLaunchKernelGGL(ring_window_kernel, dim3(B, r.capacity), dim3(kRingThreads), 0, r.stream, r, slot, B, out,
                     n_valid);
  return hipGetLastError();
}

hipError_t launch_ring_reset(const RingArgs& r, const int32_t* slot, int B) {
  if (B == 0) return hipSuccess;
  hipLaunchKernelGGL(ring_reset_kernel, dim3((B + 255) / 256), dim3(256), 0, r.stream, r, slot, B);
  return hipGetLastError();
}

}  // namespace kda
