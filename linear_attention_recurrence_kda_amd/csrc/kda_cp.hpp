// Corrections for sequences split into segments inside one fused prefill
// (context parallelism on one GPU): the device code that the fused kernel's
// tail workgroups run (kda_fused.hip, fused_tail).
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
// known (the composition of the segment maps, compose_kernel), the
// correction adds S_in^T qhat_t to every output row of the segment and writes every
// checkpoint of it as X_ck S_in + B_ck (and, for a sequence in two segments,
// its final state as A S_in + B: the composition of one map).
//
// o rows: bf16 MFMA (16x16x32) on S_in rounded to bf16, the operand
// precision the prefill's own output products use, accumulated in fp32 onto
// the stored row.  Formed transposed (o^T += S_in^T qhat^T), with the rows
// of two column tiles interleaved so that a lane holds eight consecutive
// columns of one output row and moves them as one 16-byte piece; qhat is read
// as 16-byte pieces of one row.  States: fp32 MFMA (16x16x4).
#pragma once

#include "kda_prefill_slab.hpp"

namespace kda {
namespace {

constexpr int kFixD = 128;           // dk = dv
constexpr int kStPitch = kFixD + 8;  // bf16 per row of S_in^T in LDS (16 bytes of padding)
// States: X (pitch 132) and S_in (pitch 144) in LDS, pitches that put the
// lanes of an MFMA operand read on distinct banks.
constexpr int kXPitch = kFixD + 4, kSPitch = kFixD + 16;
constexpr int kFixDepth = 3;  // row blocks in flight per wave
constexpr int kRowsLds = kFixD * kStPitch * 2;              // bytes of LDS of the output rows
constexpr int kFullLds = kFixD * (kXPitch + kSPitch) * 4;   // of a state

struct FixView {
  void* o;
  const void* qhat;
  float* tstate;  // (start states are written into it)
  const float* xpool;
  float* page_pool;
  float* s_final;
  int64_t page_elems;
  int H;
};

// Output column of row r (0..15) of column tile 2p + j of S_in^T: the two
// tiles of pair p give a lane (rows 4g .. 4g + 3 of each) the eight
// consecutive columns 32p + 8g .. + 7 of its output row, one 16-byte piece.
__device__ __forceinline__ int fix_col(int p, int j, int r) { return 32 * p + 8 * (r >> 2) + 4 * j + (r & 3); }

// o += S_in^T qhat for tokens [t0, t1) of one head of one segment (first
// token lo, len tokens, qhat rows from qrow, S_in = tstate state si), by the
// NW waves of the workgroup, in blocks of 16 NW tokens: wave w takes tokens
// 16w .. 16w + 15 of a block and every column.  S_in^T waits in LDS as bf16
// (rows = output columns, 16-byte fragment reads, read again for every block
// so that few registers stay live); kFixDepth blocks' qhat and o are in
// flight per wave.
template <int NW>
__device__ __forceinline__ void fix_rows(const FixView& p, int lo, int len, int qrow, int si, int h, int t0, int t1,
                                         char* lds) {
  constexpr int NB = 16 * NW;  // tokens per block
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l16 = lane & 15, g = lane >> 4;
  const float* S = p.tstate + (static_cast<int64_t>(si) * p.H + h) * kFixD * kFixD;
  __bf16* st = reinterpret_cast<__bf16*>(lds);
  const uint32_t rs = static_cast<uint32_t>(p.H) * kFixD * 2;  // token row stride of qhat and o, bytes
  const int end = min(len, t1);
  const uint32_t row = static_cast<uint32_t>(16 * wave + l16) * rs;
  struct Blk {
    i32x4 q[4], o[4];
  };
  // Block starting at token r0 of the segment; rows past the range (or a
  // block past it: r0 >= end) read as zero and are not written.
  auto rsrc = [&](const void* base, int64_t first, int r0) {
    const int n = min(NB, end - r0);
    return buf_rsrc(static_cast<const char*>(base) + ((first + r0) * p.H + h) * kFixD * 2,
                    n > 0 ? static_cast<uint32_t>(n - 1) * rs + kFixD * 2 : 0u);
  };
  auto load = [&](int r0, Blk& b) {
    const __amdgpu_buffer_rsrc_t rq = rsrc(p.qhat, qrow, r0), ro = rsrc(p.o, lo, r0);
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
      b.q[ks] = __builtin_bit_cast(i32x4, __builtin_amdgcn_raw_buffer_load_b128(rq, row + (32 * ks + 8 * g) * 2, 0, 0));
#pragma unroll
    for (int pp = 0; pp < 4; ++pp)
      b.o[pp] = __builtin_bit_cast(i32x4, __builtin_amdgcn_raw_buffer_load_b128(ro, row + (32 * pp + 8 * g) * 2, 0, 0));
  };
  Blk buf[kFixDepth];
#pragma unroll
  for (int j = 0; j < kFixDepth; ++j) load(t0 + j * NB, buf[j]);
  // (every load of S_in issued before the first store: one memory round trip)
  constexpr int N4 = kFixD * kFixD / 4, IT = (N4 + 64 * NW - 1) / (64 * NW);
  float4 sx[IT];
#pragma unroll
  for (int i = 0; i < IT; ++i) {
    const int e = tid + i * 64 * NW;
    if (e < N4) sx[i] = *reinterpret_cast<const float4*>(&S[4 * e]);
  }
#pragma unroll
  for (int i = 0; i < IT; ++i) {
    const int e = tid + i * 64 * NW;
    if (e >= N4) continue;
    const int k = e / (kFixD / 4), n4 = 4 * (e % (kFixD / 4));
    st[(n4 + 0) * kStPitch + k] = static_cast<__bf16>(sx[i].x);
    st[(n4 + 1) * kStPitch + k] = static_cast<__bf16>(sx[i].y);
    st[(n4 + 2) * kStPitch + k] = static_cast<__bf16>(sx[i].z);
    st[(n4 + 3) * kStPitch + k] = static_cast<__bf16>(sx[i].w);
  }
  __syncthreads();
  // Groups of kFixDepth blocks, unrolled so that every buffer is a fixed set
  // of registers: block r0 + j NB comes from buf[j], which then takes block
  // r0 + (j + kFixDepth) NB (operations past the range have empty ranges, so
  // there is no branch and the waits count exactly what they need).
  for (int r0 = t0; r0 < end; r0 += kFixDepth * NB) {
#pragma unroll
    for (int j = 0; j < kFixDepth; ++j) {
      const int rb = r0 + j * NB;
      asm volatile("" ::: "memory");  // (S_in^T is read from LDS per block, not held in registers)
      const __amdgpu_buffer_rsrc_t ro = rsrc(p.o, lo, rb);
#pragma unroll
      for (int pp = 0; pp < 4; ++pp) {
        const bf16x8 o8 = __builtin_bit_cast(bf16x8, buf[j].o[pp]);
        f32x4 acc[2];
#pragma unroll
        for (int jj = 0; jj < 2; ++jj)
#pragma unroll
          for (int i = 0; i < 4; ++i) acc[jj][i] = static_cast<float>(o8[4 * jj + i]);
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
          const bf16x8 qb = __builtin_bit_cast(bf16x8, buf[j].q[ks]);
#pragma unroll
          for (int jj = 0; jj < 2; ++jj) {
            const bf16x8 sa = *reinterpret_cast<const bf16x8*>(&st[fix_col(pp, jj, l16) * kStPitch + 32 * ks + 8 * g]);
            acc[jj] = mma(sa, qb, acc[jj]);
          }
        }
        bf16x8 r8;
#pragma unroll
        for (int jj = 0; jj < 2; ++jj)
#pragma unroll
          for (int i = 0; i < 4; ++i) r8[4 * jj + i] = static_cast<__bf16>(acc[jj][i]);
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(i32x4, r8), ro, row + (32 * pp + 8 * g) * 2, 0, 0);
      }
      load(rb + kFixDepth * NB, buf[j]);
    }
  }
}

// One head's state dst = X S_in + B (dst, X, B, S_in point at the head's
// [dk][dv] block), by a workgroup of NW >= 8 waves with kFullLds bytes of
// LDS: X and S_in are loaded into LDS together (one memory round trip), then
// wave w < 8 forms rows 16w .. 16w + 15, all 128 columns (eight 16x16
// tiles), in fp32 MFMA (16x16x4).
template <int NW>
__device__ __forceinline__ void fix_state(float* dst, const float* X, const float* B, const float* S, char* lds) {
  static_assert(NW >= 8, "eight waves form the sixteen-row tiles");
  float* xs = reinterpret_cast<float*>(lds);
  float* ss = xs + kFixD * kXPitch;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, l16 = lane & 15, g = lane >> 4;
  // Loads of B (into the accumulators: D tile ct holds rows 16 wave + 4g + i,
  // column 16 ct + l16), X and S_in all issued before the first LDS store:
  // one memory round trip.
  f32x4 acc[8];
  if (wave < 8)
#pragma unroll
    for (int ct = 0; ct < 8; ++ct)
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[ct][i] = B[(16 * wave + 4 * g + i) * kFixD + 16 * ct + l16];
  constexpr int N4 = kFixD * kFixD / 4, IT = (N4 + 64 * NW - 1) / (64 * NW);
  float4 x[IT], y[IT];
#pragma unroll
  for (int i = 0; i < IT; ++i) {
    const int e = tid + i * 64 * NW;
    if (e < N4) {
      x[i] = *reinterpret_cast<const float4*>(&X[4 * e]);
      y[i] = *reinterpret_cast<const float4*>(&S[4 * e]);
    }
  }
#pragma unroll
  for (int i = 0; i < IT; ++i) {
    const int e = tid + i * 64 * NW;
    if (e >= N4) continue;
    const int r = e / (kFixD / 4), c4 = 4 * (e % (kFixD / 4));
    float* dx = &xs[r * kXPitch + c4];
    float* dy = &ss[r * kSPitch + c4];
    dx[0] = x[i].x; dx[1] = x[i].y; dx[2] = x[i].z; dx[3] = x[i].w;
    dy[0] = y[i].x; dy[1] = y[i].y; dy[2] = y[i].z; dy[3] = y[i].w;
  }
  __syncthreads();
  if (wave >= 8) return;
  for (int ks = 0; ks < kFixD / 4; ++ks) {
    const int k = 4 * ks + g;
    const float a = xs[(16 * wave + l16) * kXPitch + k];
#pragma unroll
    for (int ct = 0; ct < 8; ++ct)
      acc[ct] = __builtin_amdgcn_mfma_f32_16x16x4f32(a, ss[k * kSPitch + 16 * ct + l16], acc[ct], 0, 0, 0);
  }
#pragma unroll
  for (int ct = 0; ct < 8; ++ct)
#pragma unroll
    for (int i = 0; i < 4; ++i) dst[(16 * wave + 4 * g + i) * kFixD + 16 * ct + l16] = acc[ct][i];
}

// A state item of head h: X S_in + B into a page slot (dkind 0, page zero
// padding included), the final state of sequence didx (dkind 1) or tstate
// state didx (dkind 2: a later segment's start state); B and X from tstate
// when in_t, else from xpool; S_in = tstate state si.
template <int NW>
__device__ __forceinline__ void fix_state_item(const FixView& p, int dkind, int64_t didx, int bi, int xi, int si,
                                               bool in_t, int h, char* lds) {
  const int64_t hkv = static_cast<int64_t>(p.H) * kFixD * kFixD, hoff = static_cast<int64_t>(h) * kFixD * kFixD;
  const float* pool = in_t ? p.tstate : p.xpool;
  float* base = dkind == 0 ? p.page_pool + didx * p.page_elems
                           : (dkind == 1 ? p.s_final : p.tstate) + didx * hkv;
  fix_state<NW>(base + hoff, pool + xi * hkv + hoff, pool + bi * hkv + hoff, p.tstate + si * hkv + hoff, lds);
  if (dkind == 0 && h == 0)
    for (int64_t e = hkv + threadIdx.x; e < p.page_elems; e += 64 * NW) base[e] = 0.f;
}

}  // namespace
}  // namespace kda
