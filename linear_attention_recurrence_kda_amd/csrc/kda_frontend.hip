// The KDA front end in one pass: causal depthwise short convolution, SiLU,
// L2Norm of q and k, and the gates, from a layer's mixed q|k|v projections
// and gate logits to the recurrence inputs q, k, v, a, beta; plus the
// convolution window a checkpoint keeps next to the recurrent state.
//
// The "Kimi Linear 的 KDA 缓存" page ("KDA 的递推与充分状态") names the steps
// (projection, causal short convolution, activation, then L2Norm of Q and K)
// and its checkpoint section takes the convolution checkpoint as the last
// kernel_size - 1 rows of mixed_qkv before the boundary; the "Serve 模块交互式
// 演示" page (§1.3) gives a = g_min * sigmoid(.) and beta = sigmoid(.).  The
// readings for what the pages leave open: mixed rows hold the q channels of
// all heads, then k, then v; the convolution is depthwise, causal, without
// bias, weight w[c][K-1] on the current token; the activation is SiLU;
// L2Norm divides by sqrt(sum u^2 + 1e-6).
//
// One workgroup per (tile of up to 64 tokens of one sequence, group of
// neighbouring heads), four waves: q, k and v of those heads, and the gates.
// A lane owns 16 bytes of one head's channels and the lane groups of a wave
// are neighbouring heads, so every load and store moves a contiguous run of
// a token's row; a lane walks the tile's tokens in order with the three
// previous raw rows in registers (each row is read once, plus a three-row
// halo per tile), and q and k take their L2 sums with a butterfly inside the
// head's lane group.  Loads and stores in the token loop are unconditional
// (groups past the heads repeat the last one and store identical values), so
// the compiler's waits count only what they
// need.  In step mode a tile is one decode token of one session, the rows
// before it come from the session's window, and the window comes back
// shifted by one row.
#include <algorithm>

#include "kda_device.hpp"
#include "kda_internal.hpp"

namespace kda {
namespace {

constexpr float kL2Eps = 1e-6f;

// VEC consecutive elements (16 bytes) as floats.
template <typename InT>
struct Vec {
  static constexpr int N = 16 / static_cast<int>(sizeof(InT));
};
__device__ __forceinline__ void ld16(const float* p, float* v) {
  const float4 x = *reinterpret_cast<const float4*>(p);
  v[0] = x.x; v[1] = x.y; v[2] = x.z; v[3] = x.w;
}
__device__ __forceinline__ void ld16(const bf16raw* p, float* v) {
  const uint4 u = *reinterpret_cast<const uint4*>(p);
  const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[2 * i] = __uint_as_float(w[i] << 16);
    v[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
  }
}
__device__ __forceinline__ void st16(float* p, const float* v) {
  *reinterpret_cast<float4*>(p) = make_float4(v[0], v[1], v[2], v[3]);
}
__device__ __forceinline__ void st16(bf16raw* p, const float* v) {
  uint32_t w[4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
    w[i] = static_cast<uint32_t>(f32_to_bf16_bits(v[2 * i])) |
           (static_cast<uint32_t>(f32_to_bf16_bits(v[2 * i + 1])) << 16);
  *reinterpret_cast<uint4*>(p) = make_uint4(w[0], w[1], w[2], w[3]);
}

__device__ __forceinline__ float sigmoid_f(float z) { return 1.f / (1.f + fast_exp(-z)); }

struct Tile {
  int seq, t0, rows, s0;  // sequence, first token, tokens, the sequence's first token
};

// Lane layout: a lane owns VEC consecutive channels (16 bytes) of one head,
// LPT = D / VEC lanes cover a head's D channels, and the lane groups of a
// wave are neighbouring heads, so one load or store moves a contiguous run of
// the token's row.  A workgroup covers HG heads (the group count of the
// widest part); groups past them, or past H, repeat the last head (same
// loads, same values, same addresses).
template <int D, typename InT>
struct Lanes {
  static constexpr int VEC = Vec<InT>::N;
  static constexpr int LPT = D / VEC;
  static constexpr int G = 64 / LPT;
  static_assert(D % VEC == 0 && LPT <= 64, "lane layout");
};
template <int DK, int DV, typename InT>
struct HeadGroup {
  static constexpr int HG = Lanes<(DK > DV ? DK : DV), InT>::G;
};

// One part (q, k or v) over a tile for the heads h0 .. h0 + HG - 1: D
// channels of head h start at channel cbase + h * D of the mixed rows, and go
// to out[t][h][*].  A lane walks the tile's tokens in order with the three
// raw rows before the current one in registers.
template <int D, int HG, typename InT, bool STEP>
__device__ __forceinline__ void conv_part(const FrontParams& p, const Tile& tl, int h0, int cbase,
                                          InT* __restrict__ out, bool l2) {
  using L = Lanes<D, InT>;
  constexpr int VEC = L::VEC, LPT = L::LPT;
  const int lane = threadIdx.x & 63;
  const int C = p.C, K = p.K, H = p.H;
  const int h = min(h0 + min(lane / LPT, HG - 1), H - 1);
  const int cl = (lane % LPT) * VEC;
  const int ch = cbase + h * D + cl;
  const InT* __restrict__ x = static_cast<const InT*>(p.x);
  const InT* __restrict__ w = static_cast<const InT*>(p.w);
  const InT* __restrict__ win = static_cast<const InT*>(p.win_in);

  // Weight of slot s (0: the current row, 1..3: the rows before it) is tap K-1-s.
  float wr[4][VEC];
#pragma unroll
  for (int v = 0; v < VEC; ++v)
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const int tap = K - 1 - s;
      const float wv = to_f32(w[static_cast<size_t>(ch + v) * K + max(tap, 0)]);
      wr[s][v] = tap >= 0 ? wv : 0.f;
    }
  // The three raw rows before the tile: from x inside the sequence, else row j
  // of the carried window (j = row - s0 + K - 1), else zero (a branch on
  // values shared by the whole wave).
  float prev[3][VEC];
#pragma unroll
  for (int s = 1; s <= 3; ++s) {
    const int row = tl.t0 - s;
    const int j = row - tl.s0 + K - 1;
#pragma unroll
    for (int v = 0; v < VEC; ++v) prev[s - 1][v] = 0.f;
    if (!STEP && row >= tl.s0) ld16(x + static_cast<size_t>(row) * C + ch, prev[s - 1]);
    else if (win != nullptr && j >= 0 && s <= K - 1)
      ld16(win + (static_cast<size_t>(tl.seq) * (K - 1) + j) * C + ch, prev[s - 1]);
  }

  const size_t xrow0 = STEP ? static_cast<size_t>(tl.seq) : static_cast<size_t>(tl.t0);
#pragma unroll 4
  for (int r = 0; r < tl.rows; ++r) {
    float xc[VEC], y[VEC];
    ld16(x + (xrow0 + r) * C + ch, xc);
    float ss = 0.f;
#pragma unroll
    for (int v = 0; v < VEC; ++v) {
      const float u = wr[0][v] * xc[v] + wr[1][v] * prev[0][v] + wr[2][v] * prev[1][v] +
                      wr[3][v] * prev[2][v];
      prev[2][v] = prev[1][v];
      prev[1][v] = prev[0][v];
      prev[0][v] = xc[v];
      y[v] = u * sigmoid_f(u);  // SiLU
      ss += y[v] * y[v];
    }
    if (l2) {
#pragma unroll
      for (int off = LPT / 2; off > 0; off >>= 1) ss += __shfl_xor(ss, off);
      const float sc = rsqrtf(ss + kL2Eps);
#pragma unroll
      for (int v = 0; v < VEC; ++v) y[v] *= sc;
    }
    st16(out + ((tl.t0 + r) * static_cast<size_t>(H) + h) * D + cl, y);
  }

  if constexpr (STEP) {
    // The window after the token: row j is the raw row K-2-j rows back (row
    // K-2 is the token itself).
    InT* wout = static_cast<InT*>(p.win_step);
    for (int j = 0; j < K - 1; ++j) {
      const int s = K - 2 - j;  // 0..2
      float val[VEC];
#pragma unroll
      for (int v = 0; v < VEC; ++v) val[v] = s == 0 ? prev[0][v] : (s == 1 ? prev[1][v] : prev[2][v]);
      st16(wout + (static_cast<size_t>(tl.seq) * (K - 1) + j) * C + ch, val);
    }
  }
}

template <int DK, int HG, typename InT>
__device__ __forceinline__ void gate_part(const FrontParams& p, const Tile& tl, int h0) {
  using L = Lanes<DK, InT>;
  constexpr int VEC = L::VEC, LPT = L::LPT;
  const int lane = threadIdx.x & 63;
  const int H = p.H;
  const int h = min(h0 + min(lane / LPT, HG - 1), H - 1);
  const int cl = (lane % LPT) * VEC;
  const InT* __restrict__ za = static_cast<const InT*>(p.z_a);
  const InT* __restrict__ zb = static_cast<const InT*>(p.z_b);
  InT* __restrict__ a = static_cast<InT*>(p.a);
  InT* __restrict__ beta = static_cast<InT*>(p.beta);
#pragma unroll 4
  for (int r = 0; r < tl.rows; ++r) {
    const size_t th = static_cast<size_t>(tl.t0 + r) * H + h;
    float z[VEC], gv[VEC];
    ld16(za + th * DK + cl, z);
#pragma unroll
    for (int v = 0; v < VEC; ++v) gv[v] = p.g_min * sigmoid_f(z[v]);
    st16(a + th * DK + cl, gv);
    // Every lane of the head's group writes its beta (same value, same address).
    beta[th] = from_f32<InT>(sigmoid_f(to_f32(zb[th])));
  }
}

template <int DK, int DV, typename InT, bool STEP>
__global__ __launch_bounds__(256) void front_kernel(FrontParams p) {
  constexpr int HG = HeadGroup<DK, DV, InT>::HG;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int n_hg = (p.H + HG - 1) / HG;
  const int unit = blockIdx.x / n_hg, h0 = (blockIdx.x % n_hg) * HG;
  Tile tl;
  if constexpr (STEP) {
    tl = Tile{unit, unit, 1, unit};
  } else {
    const int32_t* tr = p.tiles + 4 * unit;
    tl.seq = __builtin_amdgcn_readfirstlane(tr[0]);
    tl.t0 = __builtin_amdgcn_readfirstlane(tr[1]);
    tl.rows = __builtin_amdgcn_readfirstlane(tr[2]);
    tl.s0 = __builtin_amdgcn_readfirstlane(tr[3]);
  }
  const int H = p.H;
  switch (wave) {
    case 0: conv_part<DK, HG, InT, STEP>(p, tl, h0, 0, static_cast<InT*>(p.q), true); break;
    case 1: conv_part<DK, HG, InT, STEP>(p, tl, h0, H * DK, static_cast<InT*>(p.k), true); break;
    case 2: conv_part<DV, HG, InT, STEP>(p, tl, h0, 2 * H * DK, static_cast<InT*>(p.v), false); break;
    default: gate_part<DK, HG, InT>(p, tl, h0); break;
  }
}

// Convolution windows at sequence boundaries: boundary b (seq, p, slot) takes
// the K-1 raw rows before token p of sequence seq (from x, or from the carried
// window where p < K-1) into page slot `slot` of the window pool (zero-padded
// past (K-1)*C), or into win_out[seq] when slot < 0.
template <typename InT>
__global__ __launch_bounds__(256) void conv_window_kernel(WindowParams p) {
  for (int b = blockIdx.y; b < p.n_bnd; b += gridDim.y) {
  const int32_t* bd = p.bnd + 4 * b;
  const int seq = bd[0], pos = bd[1], slot = bd[2], s0 = bd[3];
  const int K = p.K, C = p.C;
  const int64_t n = static_cast<int64_t>(K - 1) * C;
  const InT* x = static_cast<const InT*>(p.x);
  const InT* win = static_cast<const InT*>(p.win_in);
  InT* dst = slot >= 0 ? static_cast<InT*>(p.pool) + static_cast<int64_t>(slot) * p.pool_elems
                       : static_cast<InT*>(p.win_out) + static_cast<int64_t>(seq) * n;
  const int64_t total = slot >= 0 ? p.pool_elems : n;
  for (int64_t e = blockIdx.x * static_cast<int64_t>(blockDim.x) + threadIdx.x; e < total;
       e += static_cast<int64_t>(gridDim.x) * blockDim.x) {
    InT val = from_f32<InT>(0.f);
    if (e < n) {
      const int j = static_cast<int>(e / C), c = static_cast<int>(e % C);
      const int t = pos - (K - 1) + j;
      if (t >= 0) val = x[static_cast<size_t>(s0 + t) * C + c];
      else if (win != nullptr) val = win[(static_cast<size_t>(seq) * (K - 1) + (K - 1 + t)) * C + c];
    }
    dst[e] = val;
  }
  }
}

template <int DK, int DV, typename InT>
hipError_t launch_t(const FrontParams& p, int units, bool step) {
  constexpr int HG = HeadGroup<DK, DV, InT>::HG;
  const dim3 grid(static_cast<unsigned>(units) * static_cast<unsigned>((p.H + HG - 1) / HG));
  if (step) hipLaunchKernelGGL((front_kernel<DK, DV, InT, true>), grid, dim3(256), 0, p.stream, p);
  else hipLaunchKernelGGL((front_kernel<DK, DV, InT, false>), grid, dim3(256), 0, p.stream, p);
  return hipGetLastError();
}

template <int DK, typename InT>
hipError_t launch_dv(const FrontParams& p, int units, bool step) {
  switch (p.dv) {
    case 16: return launch_t<DK, 16, InT>(p, units, step);
    case 32: return launch_t<DK, 32, InT>(p, units, step);
    case 64: return launch_t<DK, 64, InT>(p, units, step);
    case 128: return launch_t<DK, 128, InT>(p, units, step);
  }
  return hipErrorInvalidValue;
}

template <typename InT>
hipError_t launch_dk(const FrontParams& p, int units, bool step) {
  switch (p.dk) {
    case 16: return launch_dv<16, InT>(p, units, step);
    case 32: return launch_dv<32, InT>(p, units, step);
    case 64: return launch_dv<64, InT>(p, units, step);
    case 128: return launch_dv<128, InT>(p, units, step);
  }
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_front(const FrontParams& p, int units, bool step) {
  return p.bf16 ? launch_dk<bf16raw>(p, units, step) : launch_dk<float>(p, units, step);
}

hipError_t launch_windows(const WindowParams& p) {
  if (p.n_bnd == 0) return hipSuccess;
  const int64_t per = std::max<int64_t>(p.pool_elems, static_cast<int64_t>(p.K - 1) * p.C);
  const dim3 grid(static_cast<unsigned>(std::max<int64_t>(1, std::min<int64_t>((per + 255) / 256, 64))),
                  static_cast<unsigned>(std::min(p.n_bnd, 65535)));
  if (p.bf16) hipLaunchKernelGGL((conv_window_kernel<bf16raw>), grid, dim3(256), 0, p.stream, p);
  else hipLaunchKernelGGL((conv_window_kernel<float>), grid, dim3(256), 0, p.stream, p);
  return hipGetLastError();
}

}  // namespace kda
