// Corrections for sequences split into segments inside one fused prefill
// (context parallelism on one GPU).
//
// The recurrence is affine in the state ("Kimi Linear 的 KDA 缓存" page,
// "KDA 的递推与充分状态"; the "Serve 模块交互式演示" page reduces a segment
// of a long sequence to a fixed-size summary in §1.7 and composes them in
// §7.2): after t tokens of a segment that starts at S_in,
//   S_t = X_t S_in + B_t,
// with X_t the product of the token maps' linear parts (the state reached
// from the identity with v = 0) and B_t the state reached from zero.  The
// output o_t = S_t^T q_t is then B_t^T q_t + S_in^T (X_t^T q_t).  The fused
// prefill runs a split sequence's later segments from zero (giving B_t^T q_t
// and the checkpoints B_ck) and from the identity (giving qhat_t = X_t^T q_t,
// whose dk entries are that chain's outputs, and the checkpoints X_ck), all
// at once beside the first segment; once the segments' start states are
// known (the composition of the segment maps, compose_kernel), this kernel
// adds S_in^T qhat_t to every output row of the segment and writes every
// checkpoint of it as X_ck S_in + B_ck.
//
// o rows: bf16 MFMA (16x16x32) on S_in rounded to bf16, the operand
// precision the prefill's own output products use, accumulated in fp32 onto
// the stored row.  Formed transposed (o^T += S_in^T qhat^T), so that a lane
// holds four consecutive columns of one output row and moves them as one
// 8-byte piece, and reads qhat as 16-byte pieces of one row.  Checkpoints:
// fp32 products on the vector units (a few per call).
#include "kda_prefill_slab.hpp"

namespace kda {
namespace {

constexpr int kFixThreads = 256;
constexpr int kFixD = 128;     // dk = dv
constexpr int kFixCkRows = 32;  // state rows per checkpoint workgroup

// o += S_in^T qhat for kFixTokens tokens of one head of one segment.  Wave w
// takes output columns 64 (w & 1) .. +63 and tokens 32 (w >> 1) .. +31 of each
// 64-token block: four 16-column tiles (nt) by two 16-token tiles (tt).
__device__ __forceinline__ void fix_rows(const FixArgs& p, int item) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int l16 = lane & 15, g = lane >> 4;
  const int sg = ld_const(p.owgs, 3 * item), h = ld_const(p.owgs, 3 * item + 1);
  const int t0 = ld_const(p.owgs, 3 * item + 2);
  const int lo = ld_const(p.segs, 4 * sg), len = ld_const(p.segs, 4 * sg + 1);
  const int qrow = ld_const(p.segs, 4 * sg + 2), si = ld_const(p.segs, 4 * sg + 3);
  const float* S = p.tstate + (static_cast<int64_t>(si) * p.H + h) * kFixD * kFixD;
  const int n0 = 64 * (wave & 1);
  // A operands: S_in^T, rows = output columns n0 + 16 nt + l16, contraction
  // k = 32 ks + 8 g + e.
  bf16x8 sa[4][4];
#pragma unroll
  for (int nt = 0; nt < 4; ++nt)
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
#pragma unroll
      for (int e = 0; e < 8; ++e)
        sa[nt][ks][e] = static_cast<__bf16>(S[(32 * ks + 8 * g + e) * kFixD + n0 + 16 * nt + l16]);

  const uint32_t rs = static_cast<uint32_t>(p.H) * kFixD * 2;  // token row stride of qhat and o, bytes
  for (int b = 0; b < kFixTokens; b += 64) {
    const int r0 = t0 + b;                 // first token of the block within the segment
    const int nrows = min(64, len - r0);   // rows past it read zero and are not written
    const uint32_t range = nrows > 0 ? static_cast<uint32_t>(nrows - 1) * rs + kFixD * 2 : 0u;
    const __amdgpu_buffer_rsrc_t rq = buf_rsrc(
        static_cast<const char*>(p.qhat) + ((static_cast<int64_t>(qrow) + r0) * p.H + h) * kFixD * 2, range);
    const __amdgpu_buffer_rsrc_t ro = buf_rsrc(
        static_cast<char*>(p.o) + ((static_cast<int64_t>(lo) + r0) * p.H + h) * kFixD * 2, range);
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
      const uint32_t row = static_cast<uint32_t>(32 * (wave >> 1) + 16 * tt + l16) * rs;
      bf16x8 qb[4];
#pragma unroll
      for (int ks = 0; ks < 4; ++ks)
        qb[ks] = __builtin_bit_cast(
            bf16x8, __builtin_amdgcn_raw_buffer_load_b128(rq, row + (32 * ks + 8 * g) * 2, 0, 0));
      i32x2 ov[4];
#pragma unroll
      for (int nt = 0; nt < 4; ++nt)
        ov[nt] = __builtin_bit_cast(
            i32x2, __builtin_amdgcn_raw_buffer_load_b64(ro, row + (n0 + 16 * nt + 4 * g) * 2, 0, 0));
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) {
        const bf16x4 o4 = __builtin_bit_cast(bf16x4, ov[nt]);
        f32x4 acc;
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[i] = static_cast<float>(o4[i]);
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) acc = mma(sa[nt][ks], qb[ks], acc);
        bf16x4 r4;
#pragma unroll
        for (int i = 0; i < 4; ++i) r4[i] = static_cast<__bf16>(acc[i]);
        __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(i32x2, r4), ro,
                                              row + (n0 + 16 * nt + 4 * g) * 2, 0, 0);
      }
    }
  }
}

// One checkpoint of a segment, one head, kFixCkRows state rows:
// page = X_ck S_in + B_ck in fp32.  Thread t: column t % 128, rows
// 16 (t / 128) .. +15 of the block (uniform per wave, so the rows of X are
// LDS broadcasts).
__device__ __forceinline__ void fix_ckpt(const FixArgs& p, int item, float (*xs)[kFixD]) {
  const int tid = threadIdx.x;
  const int rb = item % (kFixD / kFixCkRows);
  const int h = (item / (kFixD / kFixCkRows)) % p.H;
  const int ck = item / (kFixD / kFixCkRows) / p.H;
  const int64_t slot = ld_const(p.cks, 4 * ck);
  const int bi = ld_const(p.cks, 4 * ck + 1), xi = ld_const(p.cks, 4 * ck + 2), si = ld_const(p.cks, 4 * ck + 3);
  const int64_t hkv = static_cast<int64_t>(p.H) * kFixD * kFixD, hoff = static_cast<int64_t>(h) * kFixD * kFixD;
  const float* X = p.xpool + xi * hkv + hoff;
  const float* B = p.xpool + bi * hkv + hoff;
  const float* S = p.tstate + si * hkv + hoff;
  float* dst = p.page_pool + slot * p.page_elems + hoff;
  const int r0 = kFixCkRows * rb;
  for (int e = tid; e < kFixCkRows * kFixD; e += kFixThreads) xs[e / kFixD][e % kFixD] = X[(r0 + e / kFixD) * kFixD + e % kFixD];
  __syncthreads();
  const int c = tid % kFixD, rh = 16 * (tid / kFixD);
  float acc[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) acc[i] = B[(r0 + rh + i) * kFixD + c];
  for (int k = 0; k < kFixD; k += 4) {
    const float s0 = S[k * kFixD + c], s1 = S[(k + 1) * kFixD + c];
    const float s2 = S[(k + 2) * kFixD + c], s3 = S[(k + 3) * kFixD + c];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const float4 x = *reinterpret_cast<const float4*>(&xs[rh + i][k]);
      acc[i] = fmaf(x.x, s0, acc[i]);
      acc[i] = fmaf(x.y, s1, acc[i]);
      acc[i] = fmaf(x.z, s2, acc[i]);
      acc[i] = fmaf(x.w, s3, acc[i]);
    }
  }
#pragma unroll
  for (int i = 0; i < 16; ++i) dst[(r0 + rh + i) * kFixD + c] = acc[i];
  // The page's padding past the H heads is zero (once per checkpoint).
  if (h == 0 && rb == 0)
    for (int64_t e = hkv + tid; e < p.page_elems; e += kFixThreads) (p.page_pool + slot * p.page_elems)[e] = 0.f;
}

__global__ __launch_bounds__(kFixThreads) void fix_kernel(FixArgs p) {
  __shared__ __attribute__((aligned(16))) float xs[kFixCkRows][kFixD];
  if (ld_const(p.flag, 0) != 0) return;  // a decay out of range: nothing is corrected
  const int b = blockIdx.x;
  if (b < p.n_owg) fix_rows(p, b);
  else fix_ckpt(p, b - p.n_owg, xs);
}

}  // namespace

hipError_t launch_fix(const FixArgs& p) {
  if (p.dk != kFixD || p.dv != kFixD) return hipErrorInvalidValue;
  const int64_t n = p.n_owg + static_cast<int64_t>(p.n_cks) * p.H * (kFixD / kFixCkRows);
  if (n == 0) return hipSuccess;
  if (n >= (int64_t{1} << 31)) return hipErrorInvalidValue;
  hipLaunchKernelGGL(fix_kernel, dim3(static_cast<unsigned>(n)), dim3(kFixThreads), 0, p.stream, p);
  return hipGetLastError();
}

}  // namespace kda
