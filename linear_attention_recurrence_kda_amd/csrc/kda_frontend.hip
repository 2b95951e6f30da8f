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
// head's lane group.  Rows are loaded in batches, the next batch before the
// current one is computed and stored, and loads and stores in the token loop
// are unconditional (groups past the heads repeat the last one and store
// identical values; loads past a tile's end repeat its last row), so the
// compiler's waits count only what they need.  For bf16 inputs the
// convolution runs on packed bf16 pairs with dot2 products (conv_part_bf16).
// In step mode a tile is one decode token of one session, the rows before it
// come from the session's window, and the window comes back shifted by one
// row.
#include <algorithm>
#include <type_traits>

#include "kda_device.hpp"
#include "kda_internal.hpp"

namespace kda {
namespace {

constexpr float kL2Eps = 1e-6f;
constexpr int kBatch = 8;  // rows per load batch
typedef __bf16 bf16x2v __attribute__((ext_vector_type(2)));

// VEC consecutive elements (16 bytes) as floats.
template <typename InT>
struct Vec {
  static constexpr int N = 16 / static_cast<int>(sizeof(InT));
};
// A lane's 16 bytes as loaded (raw) and as floats.
template <typename InT>
struct Raw;
template <>
struct Raw<float> {
  using T = float4;
};
template <>
struct Raw<bf16raw> {
  using T = uint4;
};
template <typename InT>
__device__ __forceinline__ typename Raw<InT>::T ldraw(const InT* p) {
  return *reinterpret_cast<const typename Raw<InT>::T*>(p);
}
__device__ __forceinline__ void unpack(const float4& x, float* v) {
  v[0] = x.x; v[1] = x.y; v[2] = x.z; v[3] = x.w;
}
__device__ __forceinline__ void unpack(const uint4& u, float* v) {
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

__device__ __forceinline__ float sigmoid_f(float z) { return fast_rcp(1.f + fast_exp(-z)); }

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
  // of the carried window (j = row - s0 + K - 1), else zero.  The source is
  // chosen per row (values shared by the whole wave) and the three loads are
  // issued together; a zero row loads the tile's first row and drops it.
  const size_t xrow0 = STEP ? static_cast<size_t>(tl.seq) : static_cast<size_t>(tl.t0);
  float prev[3][VEC];
  {
    typename Raw<InT>::T hr[3];
    bool keep[3];
#pragma unroll
    for (int s = 1; s <= 3; ++s) {
      const int row = tl.t0 - s;
      const int j = row - tl.s0 + K - 1;
      const bool from_x = !STEP && row >= tl.s0;
      const bool from_w = !from_x && win != nullptr && j >= 0 && s <= K - 1;
      const InT* src = from_x ? x + static_cast<size_t>(row) * C + ch
                       : from_w ? win + (static_cast<size_t>(tl.seq) * (K - 1) + j) * C + ch
                                : x + xrow0 * C + ch;
      hr[s - 1] = ldraw(src);
      keep[s - 1] = from_x || from_w;
    }
#pragma unroll
    for (int s = 0; s < 3; ++s) {
      unpack(hr[s], prev[s]);
#pragma unroll
      for (int v = 0; v < VEC; ++v) prev[s][v] = keep[s] ? prev[s][v] : 0.f;
    }
  }

  // Rows go in batches of kBatch: the loads of the next batch are issued
  // before the current batch is computed and stored, so a wave keeps a batch
  // of loads in flight and never waits on its own stores (vector-memory
  // counters also count stores).  Past the tile's end the loads repeat its
  // last row.
  const int last = tl.rows - 1;
  using RT = typename Raw<InT>::T;
  RT nxt[kBatch];
#pragma unroll
  for (int i = 0; i < kBatch; ++i) nxt[i] = ldraw(x + (xrow0 + min(i, last)) * C + ch);
  for (int r0 = 0; r0 < tl.rows; r0 += kBatch) {
    RT cur[kBatch];
#pragma unroll
    for (int i = 0; i < kBatch; ++i) {
      cur[i] = nxt[i];
      nxt[i] = ldraw(x + (xrow0 + min(r0 + kBatch + i, last)) * C + ch);
    }
#pragma unroll
    for (int i = 0; i < kBatch; ++i) {
      if (r0 + i > last) break;
      float xc[VEC], y[VEC];
      unpack(cur[i], xc);
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
      st16(out + ((tl.t0 + r0 + i) * static_cast<size_t>(H) + h) * D + cl, y);
    }
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

// The bf16 form of conv_part.  A lane keeps its channels as packed bf16: for
// channel c, the pair (x_t[c], x_{t-1}[c]) is one 32-bit word made with a byte
// permute, and the convolution is two dot2 products, with the weights of the
// current and previous rows (taps K-1, K-2) and with the pair of two rows
// back and taps K-3, K-4 (products exact, sums in fp32).
__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2v, a), __builtin_bit_cast(bf16x2v, b), c,
                                        false);
}
// Pairs of the even / odd channel of words cur (row t) and prv (row t-1):
// low half from cur, high half from prv.
__device__ __forceinline__ uint32_t pair_even(uint32_t prv, uint32_t cur) {
  return __builtin_amdgcn_perm(prv, cur, 0x05040100u);
}
__device__ __forceinline__ uint32_t pair_odd(uint32_t prv, uint32_t cur) {
  return __builtin_amdgcn_perm(prv, cur, 0x07060302u);
}
// The row in the high halves of the pairs of channels 2i (lo) and 2i+1 (hi).
__device__ __forceinline__ uint32_t high_row(uint32_t hi, uint32_t lo) {
  return __builtin_amdgcn_perm(hi, lo, 0x07060302u);
}

template <int D, int HG, bool STEP>
__device__ __forceinline__ void conv_part_bf16(const FrontParams& p, const Tile& tl, int h0, int cbase,
                                               bf16raw* __restrict__ out, bool l2) {
  using L = Lanes<D, bf16raw>;
  constexpr int LPT = L::LPT;
  static_assert(L::VEC == 8, "8 channels a lane");
  const int lane = threadIdx.x & 63;
  const int C = p.C, K = p.K, H = p.H;
  const int h = min(h0 + min(lane / LPT, HG - 1), H - 1);
  const int cl = (lane % LPT) * 8;
  const int ch = cbase + h * D + cl;
  const bf16raw* __restrict__ x = static_cast<const bf16raw*>(p.x);
  const uint16_t* __restrict__ w = reinterpret_cast<const uint16_t*>(p.w);
  const bf16raw* __restrict__ win = static_cast<const bf16raw*>(p.win_in);

  // w1[c] = (tap K-1, tap K-2), w2[c] = (tap K-3, tap K-4); missing taps are 0.
  uint32_t w1[8], w2[8];
#pragma unroll
  for (int c = 0; c < 8; ++c) {
    uint32_t tw[4];
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const int tap = K - 1 - s;
      const uint32_t wv = w[static_cast<size_t>(ch + c) * K + max(tap, 0)];
      tw[s] = tap >= 0 ? wv : 0u;
    }
    w1[c] = tw[0] | (tw[1] << 16);
    w2[c] = tw[2] | (tw[3] << 16);
  }
  // The three raw rows before the tile, as in conv_part (zero rows are 0).
  const size_t xrow0 = STEP ? static_cast<size_t>(tl.seq) : static_cast<size_t>(tl.t0);
  uint32_t hw[3][4];
  {
    uint4 hr[3];
    bool keep[3];
#pragma unroll
    for (int s = 1; s <= 3; ++s) {
      const int row = tl.t0 - s;
      const int j = row - tl.s0 + K - 1;
      const bool from_x = !STEP && row >= tl.s0;
      const bool from_w = !from_x && win != nullptr && j >= 0 && s <= K - 1;
      const bf16raw* src = from_x ? x + static_cast<size_t>(row) * C + ch
                           : from_w ? win + (static_cast<size_t>(tl.seq) * (K - 1) + j) * C + ch
                                    : x + xrow0 * C + ch;
      hr[s - 1] = ldraw(src);
      keep[s - 1] = from_x || from_w;
    }
#pragma unroll
    for (int s = 0; s < 3; ++s) {
      hw[s][0] = keep[s] ? hr[s].x : 0u;
      hw[s][1] = keep[s] ? hr[s].y : 0u;
      hw[s][2] = keep[s] ? hr[s].z : 0u;
      hw[s][3] = keep[s] ? hr[s].w : 0u;
    }
  }
  // History: r1 = raw row t-1; pa = pairs (t-1, t-2), pb = pairs (t-2, t-3).
  uint32_t r1[4], pa[8], pb[8];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    r1[i] = hw[0][i];
    pa[2 * i] = pair_even(hw[1][i], hw[0][i]);
    pa[2 * i + 1] = pair_odd(hw[1][i], hw[0][i]);
    pb[2 * i] = pair_even(hw[2][i], hw[1][i]);
    pb[2 * i + 1] = pair_odd(hw[2][i], hw[1][i]);
  }

  // Batched loads as in conv_part.
  const int last = tl.rows - 1;
  uint4 nxt[kBatch];
#pragma unroll
  for (int i = 0; i < kBatch; ++i) nxt[i] = ldraw(x + (xrow0 + min(i, last)) * C + ch);
  for (int r0 = 0; r0 < tl.rows; r0 += kBatch) {
    uint4 cur[kBatch];
#pragma unroll
    for (int i = 0; i < kBatch; ++i) {
      cur[i] = nxt[i];
      nxt[i] = ldraw(x + (xrow0 + min(r0 + kBatch + i, last)) * C + ch);
    }
#pragma unroll
    for (int i = 0; i < kBatch; ++i) {
      if (r0 + i > last) break;
      const uint32_t xw[4] = {cur[i].x, cur[i].y, cur[i].z, cur[i].w};
      float y[8];
      float ss = 0.f;
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        const uint32_t pc = (c & 1) ? pair_odd(r1[c / 2], xw[c / 2]) : pair_even(r1[c / 2], xw[c / 2]);
        const float u = dot2_bf16(pc, w1[c], dot2_bf16(pb[c], w2[c], 0.f));
        pb[c] = pa[c];
        pa[c] = pc;
        y[c] = u * sigmoid_f(u);  // SiLU
        ss += y[c] * y[c];
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) r1[j] = xw[j];
      if (l2) {
#pragma unroll
        for (int off = LPT / 2; off > 0; off >>= 1) ss += __shfl_xor(ss, off);
        const float sc = rsqrtf(ss + kL2Eps);
#pragma unroll
        for (int c = 0; c < 8; ++c) y[c] *= sc;
      }
      st16(out + ((tl.t0 + r0 + i) * static_cast<size_t>(H) + h) * D + cl, y);
    }
  }

  if constexpr (STEP) {
    // The window after the token: row j is the raw row K-2-j rows back: the
    // token (r1), then the high halves of pa (row t-1) and pb (row t-2).
    bf16raw* wout = static_cast<bf16raw*>(p.win_step);
    for (int j = 0; j < K - 1; ++j) {
      const int s = K - 2 - j;  // 0..2
      uint32_t o[4];
#pragma unroll
      for (int i = 0; i < 4; ++i)
        o[i] = s == 0 ? r1[i] : (s == 1 ? high_row(pa[2 * i + 1], pa[2 * i]) : high_row(pb[2 * i + 1], pb[2 * i]));
      *reinterpret_cast<uint4*>(wout + (static_cast<size_t>(tl.seq) * (K - 1) + j) * C + ch) =
          make_uint4(o[0], o[1], o[2], o[3]);
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
  const int last = tl.rows - 1;
  using RT = typename Raw<InT>::T;
  auto za_at = [&](int r) { return za + (static_cast<size_t>(tl.t0 + min(r, last)) * H + h) * DK + cl; };
  RT nxt[kBatch];
#pragma unroll
  for (int i = 0; i < kBatch; ++i) nxt[i] = ldraw(za_at(i));
  for (int r0 = 0; r0 < tl.rows; r0 += kBatch) {
    RT cur[kBatch];
#pragma unroll
    for (int i = 0; i < kBatch; ++i) {
      cur[i] = nxt[i];
      nxt[i] = ldraw(za_at(r0 + kBatch + i));
    }
#pragma unroll
    for (int i = 0; i < kBatch; ++i) {
      if (r0 + i > last) break;
      float z[VEC], gv[VEC];
      unpack(cur[i], z);
#pragma unroll
      for (int v = 0; v < VEC; ++v) gv[v] = p.g_min * sigmoid_f(z[v]);
      st16(a + (static_cast<size_t>(tl.t0 + r0 + i) * H + h) * DK + cl, gv);
    }
  }
  // beta: one lane per (row, head) of the tile's HG heads.
  for (int e = lane; e < tl.rows * HG; e += 64) {
    const int hb = h0 + e % HG;
    if (hb < H) {
      const size_t th = static_cast<size_t>(tl.t0 + e / HG) * H + hb;
      beta[th] = from_f32<InT>(sigmoid_f(to_f32(zb[th])));
    }
  }
}

template <int D, int HG, typename InT, bool STEP>
__device__ __forceinline__ void conv(const FrontParams& p, const Tile& tl, int h0, int cbase, InT* out, bool l2) {
  if constexpr (std::is_same<InT, bf16raw>::value) conv_part_bf16<D, HG, STEP>(p, tl, h0, cbase, out, l2);
  else conv_part<D, HG, InT, STEP>(p, tl, h0, cbase, out, l2);
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
    case 0: conv<DK, HG, InT, STEP>(p, tl, h0, 0, static_cast<InT*>(p.q), true); break;
    case 1: conv<DK, HG, InT, STEP>(p, tl, h0, H * DK, static_cast<InT*>(p.k), true); break;
    case 2: conv<DV, HG, InT, STEP>(p, tl, h0, 2 * H * DK, static_cast<InT*>(p.v), false); break;
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
