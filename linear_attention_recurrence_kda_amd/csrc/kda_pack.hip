// Head packing into flat page slots and the inverse, bit-exact.
//
// A page slot holds one state flattened head after head: element
// h*dk*dv + i*dv + j holds S[h, i, j] (i over dk, j over dv), and the rest of
// the page is zero ("Serve 模块交互式演示" page, §1.5 pack_heads/unpack_heads,
// and Tab 7: the state is written flat into the page, followed by zero
// padding).  From the canonical [.., dk, dv] layout this is a streaming copy
// (float4, coalesced); from or to the transposed [.., dv, dk] layout it is a
// per-head transpose staged through LDS in 32x32 tiles.  Elements are fp32,
// or 16-bit (a bf16 state in bf16 pages), copied bit for bit either way.
#include "kda_device.hpp"
#include "kda_internal.hpp"

namespace kda {
namespace {

constexpr int kCopyThreads = 256;

// Canonical layout: page[slot[b]][e] = state[b][e] for e < hkv, 0 beyond
// (pack); state[b][e] = page[slot[b]][e] (unpack).  16 bytes per thread.
template <bool UNPACK, typename E>
__global__ __launch_bounds__(kCopyThreads) void copy_kernel(
    const E* __restrict__ src, E* __restrict__ dst, const int32_t* __restrict__ slot,
    int64_t hkv, int64_t page_elems, int64_t n_slots, int32_t* __restrict__ err_flag) {
  constexpr int VE = 16 / static_cast<int>(sizeof(E));
  const int b = blockIdx.y;
  const int64_t s = slot[b];
  if (s < 0 || s >= n_slots) {
    if (err_flag != nullptr && threadIdx.x == 0 && blockIdx.x == 0) *err_flag = 1;
    return;
  }
  const int64_t e = (static_cast<int64_t>(blockIdx.x) * kCopyThreads + threadIdx.x) * VE;
  if (UNPACK) {
    if (e >= hkv) return;
    const uint4 x = *reinterpret_cast<const uint4*>(src + s * page_elems + e);
    *reinterpret_cast<uint4*>(dst + b * hkv + e) = x;
  } else {
    if (e >= page_elems) return;
    uint4 x = make_uint4(0, 0, 0, 0);
    if (e < hkv) x = *reinterpret_cast<const uint4*>(src + b * hkv + e);
    *reinterpret_cast<uint4*>(dst + s * page_elems + e) = x;
  }
}

// Zero page[slot[b]][hkv .. page_elems) (the padding after a transposing pack).
template <typename E>
__global__ __launch_bounds__(kCopyThreads) void zero_tail_kernel(
    E* __restrict__ pool, const int32_t* __restrict__ slot, int64_t hkv, int64_t page_elems,
    int64_t n_slots) {
  constexpr int VE = 16 / static_cast<int>(sizeof(E));
  const int b = blockIdx.y;
  const int64_t s = slot[b];
  if (s < 0 || s >= n_slots) return;  // flagged by the transpose kernel
  const int64_t e = hkv + (static_cast<int64_t>(blockIdx.x) * kCopyThreads + threadIdx.x) * VE;
  if (e < page_elems) *reinterpret_cast<uint4*>(pool + s * page_elems + e) = make_uint4(0, 0, 0, 0);
}

constexpr int kTile = 32;

// Per (b, h): dst[c][r] = src[r][c] for an R x C head matrix.  The slot
// indirection sits on the page side: the destination for pack, the source
// for unpack.
template <bool UNPACK, typename E>
__global__ __launch_bounds__(256) void transpose_kernel(
    const E* __restrict__ src, E* __restrict__ dst, const int32_t* __restrict__ slot,
    int H, int R, int C, int64_t page_elems, int64_t n_slots, int32_t* __restrict__ err_flag) {
  __shared__ E tile[kTile][kTile + 1];
  const int b = blockIdx.z, h = blockIdx.y;
  const int64_t s = slot[b];
  if (s < 0 || s >= n_slots) {
    if (err_flag != nullptr && threadIdx.x == 0 && blockIdx.x == 0 && h == 0) *err_flag = 1;
    return;
  }
  const int64_t rc = static_cast<int64_t>(R) * C;
  const int64_t hkv = rc * H;
  const E* sp = src + (UNPACK ? s * page_elems : b * hkv) + h * rc;
  E* dp = dst + (UNPACK ? b * hkv : s * page_elems) + h * rc;
  const int tiles_c = (C + kTile - 1) / kTile;
  const int r0 = (blockIdx.x / tiles_c) * kTile, c0 = (blockIdx.x % tiles_c) * kTile;
  const int tx = threadIdx.x % kTile, ty = threadIdx.x / kTile;  // 32 x 8
  for (int y = ty; y < kTile; y += 8) {
    const int r = r0 + y, c = c0 + tx;
    if (r < R && c < C) tile[y][tx] = sp[static_cast<int64_t>(r) * C + c];
  }
  __syncthreads();
  for (int y = ty; y < kTile; y += 8) {
    const int c = c0 + y, r = r0 + tx;
    if (r < R && c < C) dp[static_cast<int64_t>(c) * R + r] = tile[tx][y];
  }
}

template <typename E>
hipError_t launch_pack_t(const PackArgs& p) {
  constexpr int VE = 16 / static_cast<int>(sizeof(E));
  const E* src = static_cast<const E*>(p.src);
  E* dst = static_cast<E*>(p.dst);
  const int64_t hkv = static_cast<int64_t>(p.H) * p.dk * p.dv;
  if (!p.vk) {
    const int64_t n = p.unpack ? hkv : p.page_elems;
    const dim3 grid(static_cast<unsigned>((n / VE + kCopyThreads - 1) / kCopyThreads), p.B);
    if (p.unpack)
      hipLaunchKernelGGL((copy_kernel<true, E>), grid, dim3(kCopyThreads), 0, p.stream, src, dst,
                         p.slot, hkv, p.page_elems, p.n_slots, p.err_flag);
    else
      hipLaunchKernelGGL((copy_kernel<false, E>), grid, dim3(kCopyThreads), 0, p.stream, src, dst,
                         p.slot, hkv, p.page_elems, p.n_slots, p.err_flag);
    return hipGetLastError();
  }
  // Pack from VK: the head matrix read is [dv][dk]; unpack to VK: it is [dk][dv].
  const int R = p.unpack ? p.dk : p.dv, C = p.unpack ? p.dv : p.dk;
  const dim3 grid(static_cast<unsigned>(((R + kTile - 1) / kTile) * ((C + kTile - 1) / kTile)),
                  p.H, p.B);
  if (p.unpack) {
    hipLaunchKernelGGL((transpose_kernel<true, E>), grid, dim3(256), 0, p.stream, src, dst, p.slot,
                       p.H, R, C, p.page_elems, p.n_slots, p.err_flag);
  } else {
    hipLaunchKernelGGL((transpose_kernel<false, E>), grid, dim3(256), 0, p.stream, src, dst,
                       p.slot, p.H, R, C, p.page_elems, p.n_slots, p.err_flag);
    const int64_t tail = p.page_elems - hkv;
    if (tail > 0) {
      const dim3 g2(static_cast<unsigned>((tail / VE + kCopyThreads - 1) / kCopyThreads), p.B);
      hipLaunchKernelGGL((zero_tail_kernel<E>), g2, dim3(kCopyThreads), 0, p.stream, dst, p.slot,
                         hkv, p.page_elems, p.n_slots);
    }
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_pack(const PackArgs& p) {
  return p.es == 2 ? launch_pack_t<uint16_t>(p) : launch_pack_t<float>(p);
}

}  // namespace kda
