// Segment summaries for context-parallel prefill, and their composition.
//
// [Serve demo] §7.2 ("KCP 前缀扫描") and §1.7 reduce each segment of a long
// sequence to what the next segment needs from it, a fixed-size quantity
// independent of the segment's length.  The recurrence is affine in the state
// (each token maps S to (I - beta k k^T) diag(e^a) S + beta k v^T), so a
// segment is the map S_end = A S_start + B, with A (dk x dk) the product of
// the token maps' linear parts and B (dk x dv) the end state from S_start = 0.
// Both come from the prefill's own chunk machinery: one local pass over the
// segment's chunks, then the propagation from the zero state (B) and from the
// identity with v = 0 (A, dk columns: column j of A is the end state of the
// start e_j).  The composition (A2, B2) o (A1, B1) = (A2 A1, A2 B1 + B2) makes
// the start of every segment an exclusive scan over the segments before it.
#include "kda_prefill_kernels.hpp"

namespace kda {
namespace {

template <int DK, typename InT, int MODE>
hipError_t prop_cols(const PrefillArgs& a) {
  if (a.slab) return launch_slab_prop(a, MODE);
  switch (a.dv / a.dv_tiles) {
    case 16: return launch_prop<DK, 16, InT, MODE>(a);
    case 32: if constexpr (MODE != 2 || DK >= 32) return launch_prop<DK, 32, InT, MODE>(a); break;
    case 64: if constexpr (MODE != 2 || DK >= 64) return launch_prop<DK, 64, InT, MODE>(a); break;
  }
  return hipErrorInvalidValue;
}

template <int DK, typename InT>
hipError_t summary_dk(const PrefillArgs& a, float* a_out, int a_tiles) {
  if (a.n_chunks > 0) {
    const hipError_t e = launch_local<DK, InT>(a);
    if (e != hipSuccess) return e;
  }
  PrefillArgs b = a;  // B: from the zero state
  b.q = nullptr;
  b.s0 = nullptr;
  b.o = nullptr;
  hipError_t e = prop_cols<DK, InT, 1>(b);
  if (e != hipSuccess) return e;
  PrefillArgs m = b;  // A: from the identity, v = 0
  m.v = nullptr;
  m.dv = DK;
  m.dv_tiles = a_tiles;
  m.s_final = a_out;
  return prop_cols<DK, InT, 2>(m);
}

template <typename InT>
hipError_t summary_in(const PrefillArgs& a, float* a_out, int a_tiles) {
  switch (a.dk) {
    case 16: return summary_dk<16, InT>(a, a_out, a_tiles);
    case 32: return summary_dk<32, InT>(a, a_out, a_tiles);
    case 64: return summary_dk<64, InT>(a, a_out, a_tiles);
    case 128: return summary_dk<128, InT>(a, a_out, a_tiles);
  }
  return hipErrorInvalidValue;
}

// One workgroup of four waves per (head, 16 columns of the state): the
// column tile of S stays in LDS across the segments, and each segment's
// S <- A S + B is a 16-column fp32 MFMA product (v_mfma_f32_16x16x4_f32).
// Wave w takes the 16-row tiles w, w+4, ...  The contraction index is
// permuted so that every lane's A operands are contiguous: in k-step s the
// lane group g = lane/16 contributes k = (DK/4) g + s, so a lane holds
// A[row][(DK/4) g .. (DK/4) g + DK/4 - 1] and loads it as float4s.  A and B
// of the next segment are loaded while the current one is multiplied.
constexpr int kComposeThreads = 256;
constexpr int kComposeCols = 16;

template <int DK>
__global__ __launch_bounds__(kComposeThreads) void compose_kernel(ComposeArgs p) {
  constexpr int RT = DK / 16;           // 16-row tiles of S
  constexpr int RPW = (RT + 3) / 4;     // row tiles per wave
  constexpr int KS = DK / 4;            // k-steps; lane group g covers k = KS g + s
  constexpr int NV = KS / 4;            // float4s of A per row tile and lane
  __shared__ float S[DK][kComposeCols + 1];
  const int tiles = p.dv / kComposeCols;
  const int h = blockIdx.x / tiles, j0 = (blockIdx.x % tiles) * kComposeCols;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = lane & 15, g = lane >> 4;
  const int dv = p.dv, H = p.H;
  for (int e = tid; e < DK * kComposeCols; e += kComposeThreads) {
    const int r = e / kComposeCols, c = e % kComposeCols;
    S[r][c] = p.s_in ? p.s_in[(static_cast<size_t>(h) * DK + r) * dv + j0 + c] : 0.f;
  }
  // Row tiles of this wave (clamped: a wave past the last tile repeats it
  // and discards the result).
  int rt[RPW];
  bool active[RPW];
#pragma unroll
  for (int t = 0; t < RPW; ++t) {
    rt[t] = min(wave + 4 * t, RT - 1);
    active[t] = wave + 4 * t < RT;
  }

  float4 a[RPW][NV];
  float b[RPW][4];
  auto load = [&](int i) {
    const size_t hb = static_cast<size_t>(i) * H + h;
    const float* A = p.A + hb * DK * DK;
    const float* B = p.B + hb * DK * dv;
#pragma unroll
    for (int t = 0; t < RPW; ++t) {
      const float4* row = reinterpret_cast<const float4*>(A + static_cast<size_t>(16 * rt[t] + col) * DK + KS * g);
#pragma unroll
      for (int v = 0; v < NV; ++v) a[t][v] = row[v];
#pragma unroll
      for (int rr = 0; rr < 4; ++rr)
        b[t][rr] = B[static_cast<size_t>(16 * rt[t] + 4 * g + rr) * dv + j0 + col];
    }
  };
  if (p.n > 0) load(0);
  __syncthreads();
  for (int i = 0; i < p.n; ++i) {
    const size_t hb = static_cast<size_t>(i) * H + h;
    float4 an[RPW][NV];
    float bn[RPW][4];
#pragma unroll
    for (int t = 0; t < RPW; ++t) {
#pragma unroll
      for (int v = 0; v < NV; ++v) an[t][v] = a[t][v];
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) bn[t][rr] = b[t][rr];
    }
    if (i + 1 < p.n) load(i + 1);
    f32x4 acc[RPW];
#pragma unroll
    for (int t = 0; t < RPW; ++t) acc[t] = f32x4{bn[t][0], bn[t][1], bn[t][2], bn[t][3]};
#pragma unroll
    for (int v = 0; v < NV; ++v) {
      const float x0 = S[KS * g + 4 * v][col], x1 = S[KS * g + 4 * v + 1][col];
      const float x2 = S[KS * g + 4 * v + 2][col], x3 = S[KS * g + 4 * v + 3][col];
#pragma unroll
      for (int t = 0; t < RPW; ++t) {
        acc[t] = __builtin_amdgcn_mfma_f32_16x16x4f32(an[t][v].x, x0, acc[t], 0, 0, 0);
        acc[t] = __builtin_amdgcn_mfma_f32_16x16x4f32(an[t][v].y, x1, acc[t], 0, 0, 0);
        acc[t] = __builtin_amdgcn_mfma_f32_16x16x4f32(an[t][v].z, x2, acc[t], 0, 0, 0);
        acc[t] = __builtin_amdgcn_mfma_f32_16x16x4f32(an[t][v].w, x3, acc[t], 0, 0, 0);
      }
    }
    // starts[i] = the S that entered this segment; then S <- A S + B.
#pragma unroll
    for (int t = 0; t < RPW; ++t) {
      if (active[t]) {
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
          const int r = 16 * rt[t] + 4 * g + rr;
          p.starts[(hb * DK + r) * dv + j0 + col] = S[r][col];
        }
      }
    }
    __syncthreads();
#pragma unroll
    for (int t = 0; t < RPW; ++t) {
      if (active[t]) {
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) S[16 * rt[t] + 4 * g + rr][col] = acc[t][rr];
      }
    }
    __syncthreads();
  }
  if (p.s_end) {
    for (int e = tid; e < DK * kComposeCols; e += kComposeThreads) {
      const int r = e / kComposeCols, c = e % kComposeCols;
      p.s_end[(static_cast<size_t>(h) * DK + r) * dv + j0 + c] = S[r][c];
    }
  }
}

template <int DK>
hipError_t compose_dk(const ComposeArgs& a) {
  const dim3 grid(static_cast<unsigned>(a.H) * static_cast<unsigned>(a.dv / kComposeCols));
  hipLaunchKernelGGL((compose_kernel<DK>), grid, dim3(kComposeThreads), 0, a.stream, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_segment_summary(const PrefillArgs& a, float* a_out, int a_tiles) {
  return a.bf16 ? summary_in<bf16raw>(a, a_out, a_tiles) : summary_in<float>(a, a_out, a_tiles);
}

hipError_t launch_compose(const ComposeArgs& a) {
  switch (a.dk) {
    case 16: return compose_dk<16>(a);
    case 32: return compose_dk<32>(a);
    case 64: return compose_dk<64>(a);
    case 128: return compose_dk<128>(a);
  }
  return hipErrorInvalidValue;
}

}  // namespace kda
