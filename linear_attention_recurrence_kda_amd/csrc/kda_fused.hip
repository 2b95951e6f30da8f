// Fused chunked prefill: one kernel, one workgroup per (sequence, head, dv
// tile) chain, 32-token chunks, bf16 inputs, fp32 state, dk = 128.
//
// The chunk form (derived from the per-token recurrence; "Kimi Linear 的 KDA
// 缓存" page, sections "KDA 的递推与充分状态" and "预填充为什么能分块并行"):
// per chunk of n <= 32 tokens, with G the running sum of the log-decays
// inside the chunk, G_m its value after the first 16 rows (the reference)
// and G_n its value at the chunk's end,
//   Kp = k e^{G - G_m},  Qp = q e^{G - G_m},  Km = k e^{G_m - G}
//   T  = (I + diag(beta) strict_lower(Kp Km^T))^{-1}
//   S' = diag(e^{G_m}) S                       (the state at the reference)
//   U  = T diag(beta) (V - Kp S'), by 16-row blocks:
//        U_0 = T_00 diag(beta_0) Z_0,  U_1 = T_11 diag(beta_1) (Z_1 - A_10 U_0)
//        (Z = V - Kp S', A = Kp Km^T; block 10 of T never needs forming)
//   O  = Qp S' + lower(Qp Km^T) U
//   S <- diag(e^{G_n - G_m}) (S' + Km^T U)
// (Kp S' = (k e^G) S and Km^T U scaled by e^{G_n - G_m} is (k e^{G_n - G})^T U:
// the same products as the per-token form, taken with one reference.)  The
// scaled operands stay within e^{+-80} for a >= -160/32 = -5, and both
// scalings of the state are applied one after the other, so neither
// underflows where their product would.
//
// Why one kernel: the chunk-local work (the decay sums, the scaled operands,
// the Gram products and the triangular solve) needs no state, but passing it
// through HBM from a separate kernel costs more than twice the compulsory
// bytes (a record of about 50 KB per chunk and head, written once and read
// back).  Here the workgroup that carries the state builds each chunk's
// record in LDS ahead of use, so HBM sees only q, k, a, beta, v, the outputs
// and the states.  The operands Kp, Qp, Km are exactly the bf16 operands of
// the Gram products, so a record costs two exponentials, three products and
// the bf16 rounding per element, and the state carries the two per-channel
// scalings.
//
// Twelve waves, three per SIMD:
//  - waves 0..3, the propagation ("P") waves: the column-slab chunk step on
//    register-resident state (16 or 32 state columns per wave; narrow tiles
//    leave some P waves without state), and (16 columns per wave) the
//    diagonal solves of the next chunk's record;
//  - waves 4..11, the local ("L") waves: L wave w builds token rows
//    16 (w / 4) .. +15 of key channels 32 (w % 4) .. +31.  A lane holds one
//    token row and eight channels, loaded from HBM in 16-byte pieces through
//    a buffer resource that ends at the chunk's last row (rows past it read
//    as zero: zero decay, zero key, query, value and beta, so they drop out of
//    every product).  The running sums of a are row scans across 16 lanes
//    (DPP); with the reference at row 16 the two halves need nothing from
//    each other.  The Gram operands are MFMA fragments already: each wave
//    forms its 32 channels' share of the diagonal blocks of A_kk and A_qk,
//    and after M the first-half wave forms the off-diagonal ones from the
//    other half's rows in LDS (all as transposes, so that a lane ends with
//    one row of a block: the layout the triangular solve wants).
//
// Per chunk c every wave passes two barriers, M (mid-chunk) and A (the
// hand-over).  Before M: P runs chunk c's state-independent half and inverts
// chunk c+1's diagonal blocks (I + L_RR), two waves per block, two of each
// lane's four columns each (forward substitution by rows, each step a DPP
// broadcast of one row within the lane row); the L waves issue the loads of
// chunk c+3 (q, k, a, beta) and c+2 (v) and build chunk c+2 (the second-half
// waves only its Kp and Qp rows).  After M: P runs the rest of chunk c; the
// first-half L waves form chunk c+2's off-diagonal Gram shares, the
// second-half ones the rest of their build (Km^T, diagonal shares,
// e^{G_n - G_m}), and two first-half waves write chunk c+1's lower(A_qk) and
// A_10; all L waves store chunk c-1's outputs and move chunk c+1's v into
// LDS.  (With 32 state columns per P wave the second-half L waves also do
// the inversion, after M.)  So a record is built across one chunk's two
// intervals, finished in the next chunk's and read in the one after.
//
// With the gate fused in, a and beta arrive as logits and the L waves apply
// a = g_min sigmoid(z_a), beta = sigmoid(z_b) in fp32 as they build ("Serve 模
// 块交互式演示" page, §1.3, for the gates; the "Kimi Linear 的 KDA 缓存" page's
// vLLM path fuses them the same way).
//
// A decay outside [a_lo, 0] (or a NaN) found while building chunk x raises
// the error flags and stops that chain at the barrier that would hand chunk x
// over: the outputs and checkpoints of the chunks before x stay written,
// nothing after them (nor the final state) is.
//
// Long sequences may arrive cut into segments (the host decides): a later
// segment's chains run from the zero state and, as width code 4, from the
// identity with v taken as zero, whose outputs are q mapped through the
// segment's linear part.  The workgroups listed after the chains (the tail,
// fused_tail below) then compose the segments' maps into their start states
// and correct the later segments' outputs and checkpoints (kda_cp.hpp).
#include <climits>
#include <cstddef>
#include <type_traits>

#include "kda_cp.hpp"
#include "kda_prefill_slab.hpp"

namespace kda {
namespace {

constexpr int kFC = 32;  // tokens per chunk

typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));
typedef float f32x8 __attribute__((ext_vector_type(8)));

// One chunk's operands in LDS.  kp, qp: 32 token rows of 16 pieces (16
// bytes, slab_col channel order), piece q of row m at q ^ (m & 7); km: Km^T,
// dk channel rows of 4 pieces (32 tokens in slab_col order), piece q of row m
// at q ^ ((m >> 1) & 3); em, en: e^{G_m} and e^{G_n - G_m} per channel.
template <int DK>
struct FRec {
  i32x4 kp[kFC * DK / 8];
  i32x4 qp[kFC * DK / 8];
  i32x4 km[DK * 4];
  float em[DK];
  float en[DK];
};
// T diag(beta) with its block 10 zero, and lower(A_qk), of one chunk: 32 rows
// of 4 pieces, columns in slab_col order, swizzled as km; A_10 (the Gram block
// of rows 16.. against rows ..15): 16 rows of the left halves of 4 pieces (the
// right halves, columns 16.., are zero and not stored).
struct FTri {
  i32x4 tb[kFC * 4];
  i32x4 aq[kFC * 4];
  i32x2 ka[16 * 4];
};

template <int DK>
struct FusedSmem {
  FRec<DK> rec[3];
  FTri tri[2];
  __bf16 vb[2][kFC * 128];         // v of a chunk ([32][DVT], row-swizzled pieces), then its outputs
  f32x4 part[2][DK / 32][6][64];   // per chunk and channel group: shares of A_kk (tiles 00, 10, 11) and A_qk
  float lr[2][16][20];             // full rows of -diag(beta) strict_lower(A_kk): blocks 00 and 11
  float beta[2][kFC];
  // stop[x % 3]: a decay out of range in chunk x.  Set while chunk x is built
  // (two intervals before it is used), read by every wave after the barrier
  // that would hand chunk x over; the writes of the interval after that
  // barrier go to another slot, so all waves read the same value and leave
  // the loop together.
  int stop[3];
};

__device__ __forceinline__ int swz4(int m, int q) { return q ^ ((m >> 1) & 3); }
__device__ __forceinline__ int swz16(int m, int q) { return q ^ (m & 7); }

// Inclusive prefix sum over the 16 lanes of each row (DPP row shifts; lanes
// shifted in from outside the row contribute 0).
template <int N>
__device__ __forceinline__ float row_shr(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x110 + N, 0xF,
                                                               0xF, false));
}
__device__ __forceinline__ float row_scan(float x) {
  x += row_shr<1>(x);
  x += row_shr<2>(x);
  x += row_shr<4>(x);
  x += row_shr<8>(x);
  return x;
}
// The value of lane I of this lane's row of 16 lanes (DPP row_newbcast; every
// lane has a source, so the move can fold into the instruction that uses it).
template <int I>
__device__ __forceinline__ float row_bcast(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), 0x150 + I, 0xF, 0xF, true));
}
__device__ __forceinline__ float row_last(float x) { return row_bcast<15>(x); }

// f(integral_constant<int, I>) for I = B .. E - 1, unrolled at compile time.
template <int B, int E, typename Fn>
__device__ __forceinline__ void static_for(Fn&& f) {
  if constexpr (B < E) {
    f(std::integral_constant<int, B>{});
    static_for<B + 1, E>(f);
  }
}

// (Vector elements reach these by value: a bit cast of a vector element in
// place reads the wrong element with this compiler.)
__device__ __forceinline__ u16x2 as_u16x2(int w) { return __builtin_bit_cast(u16x2, w); }
__device__ __forceinline__ i32x4 ld128(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(i32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}

struct FusedParams {
  const void *q, *k, *v, *a, *beta;
  const float* s0;
  void* o;
  float* s_final;
  float* page_pool;
  int64_t page_elems;
  const int32_t *chains, *seqinfo, *ck_pos, *ck_slot, *wgs;
  int32_t* wsflag;
  int32_t* err_flag;
  float a_lo;
  bool gate;    // a, beta are logits: a = g_min * sigmoid(a), beta = sigmoid(beta)
  float g_min;
  int H, dv;
  // Sequences split into segments (null segx: none).  segx [entries][6] =
  // (index of the start state in s0, index of the end state in s_final or
  // tstate, mode bits kSeg*, first row in qhat, completion counter of head 0
  // or -1, unused) per entry of seqinfo; state indices count H*dk*dv
  // elements.  Identity chains (width code 4) start from the identity with v
  // taken as zero, write their outputs (q mapped through the segment's linear
  // part) to qhat rows, their checkpoints to xpool and their end state to
  // tstate.
  const int32_t* segx;
  void* qhat;
  float* xpool;
  float* tstate;
  // Tail workgroups (width code 5): the correction of split sequences,
  // items titems [n][kTailInts] (see fused_tail), each waiting for what it
  // reads through tcnt (counters in the workspace, zero on entry).
  const int32_t* titems;
  int32_t* tcnt;
};

// Loads of one chunk for one L lane: q, k, a of its token row (eight
// channels, 16 bytes each), and one beta.
// Rows t .. t + n - 1 of a chunk.
struct Span {
  int t, n;
};

struct Raw {
  i32x4 q, k, a;
  uint32_t b;
  int n;  // the chunk's rows
};

template <int DK>
struct Fused {
  static constexpr int NCG = DK / 32;   // channel groups of 32
  static constexpr int NLW = 2 * NCG;   // L waves: two token halves per channel group
  static constexpr int NPW = 4;         // P waves
  static constexpr int NT = 64 * (NPW + NLW);
  static constexpr int NR = DK / 16, NKS = DK / 32;
};

// ---------------------------------------------------------------------------
// The chain of one workgroup.  NPA P waves are active with NJ column tiles of
// 16 each (tile width DVT = 16 * NJ * NPA).
template <int DK, int NPA, int NJ, bool ID = false>
__device__ __forceinline__ void fused_chain(const FusedParams& p, int chain, int tile, FusedSmem<DK>& sm) {
  using F = Fused<DK>;
  constexpr int NR = F::NR, NKS = F::NKS, NCG = F::NCG, NLW = F::NLW;
  constexpr int DVT = 16 * NJ * NPA;
  constexpr int VPR = DVT / 8;                // 16-byte pieces per v row
  constexpr int VSW = VPR < 4 ? VPR - 1 : 3;  // v row swizzle: piece q of row r at q ^ ((r >> 2) & VSW)
  static_assert(DK == 128, "the L waves cover 32 channels each: dk = 128 is the tuned shape");
  static_assert(kFC * VPR <= 64 * NLW, "one v piece per L lane");
  // Who inverts the diagonal blocks: the P waves before M when a wave holds
  // 16 state columns, the second-half L waves after M when it holds 32 (its
  // registers are full).
  constexpr bool kPSolve = NJ == 1;

  const int tid = threadIdx.x, lane = tid & 63, grp = lane >> 4, col = lane & 15;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const bool lw = wave >= F::NPW;  // uniform
  const int H = p.H, dv = p.dv;

  const int seq = ld_const(p.chains, 2 * chain), h = ld_const(p.chains, 2 * chain + 1);
  if (seq < 0) return;
  const int lo = ld_const(p.seqinfo, 6 * seq), hi = ld_const(p.seqinfo, 6 * seq + 1);
  const int ck_lo = ld_const(p.seqinfo, 6 * seq + 2), ck_hi = ld_const(p.seqinfo, 6 * seq + 3);
  const int c_lo = ld_const(p.seqinfo, 6 * seq + 4), c_hi = ld_const(p.seqinfo, 6 * seq + 5);
  const int64_t hkv = static_cast<int64_t>(H) * DK * dv;
  // The entry's mode and state index (a sequence that is not split: its own
  // index, mode 0).
  auto seg_field = [&](int f, int dflt) { return p.segx != nullptr ? ld_const(p.segx, kSegxInts * seq + f) : dflt; };
  const int mode = ID ? kSegZeroStart | kSegFinalTemp | kSegCkTemp : seg_field(2, 0);
  const size_t state_off = (static_cast<size_t>(seg_field(0, seq)) * H + h) * DK * dv;
  const uint32_t rsv = static_cast<uint32_t>(H) * dv * 2;  // token row stride of v and o, bytes

  auto ck_at = [&](int k) { return k < ck_hi ? lo + ld_const(p.ck_pos, k) : INT_MAX; };
  auto first_chunk = [&]() {
    ChunkWalk w{lo, 0, ck_at(ck_lo), ck_lo};
    w.n = min(min(kFC, hi - lo), w.nck - lo);
    return w;
  };
  // (past the last chunk a walker stays on it: the work on it is repeated
  // into buffers nobody reads, so no memory operation needs a branch)
  auto next_chunk = [&](ChunkWalk& w) {
    if (w.t + w.n >= hi) return;
    if (w.t + w.n == w.nck) w.nck = ck_at(++w.ck);
    w.t += w.n;
    w.n = min(min(kFC, hi - w.t), w.nck - w.t);
  };
  auto b2 = [&](int c) { return (c - c_lo) & 1; };
  auto b3 = [&](int c) { return (c - c_lo) % 3; };
  auto inc3 = [](int r) { return r == 2 ? 0 : r + 1; };

  // Zero the page padding of this sequence's checkpoint slots (once per sequence).
  if (tile == 0 && h == 0 && p.page_elems > hkv && !(mode & kSegCkTemp)) {
    for (int c = ck_lo; c < ck_hi; ++c) {
      float* pg = p.page_pool + static_cast<int64_t>(ld_const(p.ck_slot, c)) * p.page_elems;
      for (int64_t e = hkv + tid; e < p.page_elems; e += F::NT) pg[e] = 0.f;
    }
  }
  if (c_lo >= c_hi) {  // an empty sequence: the final state is s0 (segments are never empty)
    if (!ID && !lw && wave < NPA && p.s_final != nullptr && mode == 0) {
      const int jw = tile * DVT + 16 * NJ * wave;
      for (int e = lane; e < DK * 16 * NJ; e += 64) {
        const int c = e / (16 * NJ), j = jw + e % (16 * NJ);
        const size_t off = state_off + static_cast<size_t>(c) * dv + j;
        p.s_final[off] = p.s0 != nullptr ? p.s0[off] : 0.f;
      }
    }
    return;
  }
  if (tid < 3) sm.stop[tid] = 0;
  slab_barrier();  // (every wave passes 5 + 2 * chunks barriers)

  // 8-byte piece of a [32][32] tile: row m, columns 4 g .. +3 of the left
  // (hi = 0) or right (hi = 1) 16 columns (slab_col order puts them side by
  // side in piece g).
  auto piece8 = [&](i32x4* t, int m, int hi) {
    return reinterpret_cast<char*>(&t[4 * m + swz4(m, grp)]) + 8 * hi;
  };

  // ---- finishing a chunk's record (shares B2 -> tiles tri[B2]) -------------
  // "Row layout": lane (col, grp) holds row col of a 16x16 block, columns
  // 4 grp .. 4 grp + 3.  The diagonal blocks are inverted by solve_half, the
  // rest is written by the L waves after M (finish).
  auto sum_part = [&](int B2, int t) {
    f32x4 s = sm.part[B2][0][t][lane];
#pragma unroll
    for (int u = 1; u < NCG; ++u) s += sm.part[B2][u][t][lane];
    return s;
  };
  auto pack4 = [](float a0, float a1, float a2, float a3) {
    bf16x4 v;
    v[0] = static_cast<__bf16>(a0); v[1] = static_cast<__bf16>(a1);
    v[2] = static_cast<__bf16>(a2); v[3] = static_cast<__bf16>(a3);
    return v;
  };
  // (I + L_RR)^{-1} diag(beta_R) of diagonal block R, columns
  // 4 grp + NC hc .. + NC - 1 of each lane's four (NC = 2 or 4): by rows,
  // step i folds row i (final by then; lane i of this lane's row of 16) into
  // every row below it.  The rows of -L are gathered through LDS (two waves
  // of a block write the same values).  The block beside it in tb is zero.
  auto solve = [&](auto ncc, int B2, int R, int hc) {
    constexpr int NC = decltype(ncc)::value;
    FTri& tri = sm.tri[B2];
    const float* beta = sm.beta[B2];
    const f32x4 a = sum_part(B2, R == 0 ? 0 : 2);
    const float br = -beta[16 * R + col];
    float l[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) l[t] = 4 * grp + t < col ? br * a[t] : 0.f;
    *reinterpret_cast<float4*>(&sm.lr[R][col][4 * grp]) = make_float4(l[0], l[1], l[2], l[3]);
    wave_sync();
    float nL[16];
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      const float4 x4 = *reinterpret_cast<const float4*>(&sm.lr[R][col][4 * q4]);
      nL[4 * q4] = x4.x; nL[4 * q4 + 1] = x4.y; nL[4 * q4 + 2] = x4.z; nL[4 * q4 + 3] = x4.w;
    }
    const int c0 = 4 * grp + NC * hc;
    float T[NC];
#pragma unroll
    for (int u = 0; u < NC; ++u) T[u] = c0 + u == col ? 1.f : 0.f;
    static_for<0, 15>([&](auto ic) {
      constexpr int i = decltype(ic)::value;
#pragma unroll
      for (int u = 0; u < NC; ++u) T[u] = fmaf(row_bcast<i>(T[u]), nL[i], T[u]);
    });
    using BV = std::conditional_t<NC == 4, bf16x4, bf16x2>;
    using ZV = std::conditional_t<NC == 4, i32x2, int>;
    BV tv;
#pragma unroll
    for (int u = 0; u < NC; ++u) tv[u] = static_cast<__bf16>(T[u] * beta[16 * R + c0 + u]);
    *reinterpret_cast<BV*>(piece8(tri.tb, 16 * R + col, R) + 2 * NC * hc) = tv;
    *reinterpret_cast<ZV*>(piece8(tri.tb, 16 * R + col, 1 - R) + 2 * NC * hc) = ZV{};
  };
  using I2 = std::integral_constant<int, 2>;
  using I4 = std::integral_constant<int, 4>;
  if (lw) {
    // ======================= L waves ==========================================
    // With two or fewer P waves holding state, the L waves' build bounds the
    // interval before M, where the P waves have slack: the L waves then take
    // issue priority on their SIMDs before M, and give it back after M, where
    // the P waves' step is the longer one.  (With four, priority only starves
    // the P waves' longer step.)
    auto prio = [](auto pc) {
      if constexpr (NPA <= 2) __builtin_amdgcn_s_setprio(decltype(pc)::value);
    };
    const int w = wave - F::NPW, X = w / NCG, cw = w % NCG;  // uniform
    const int r16 = col, g4 = grp, m = 16 * X + r16;
    const int cb = 32 * cw + 8 * g4;  // this lane's first channel
    const int ltid = tid - 64 * F::NPW;
    const uint32_t rsk = static_cast<uint32_t>(H) * DK * 2;  // token row stride of q, k, a, bytes
    const uint32_t vo = m * rsk + cb * 2;
    const uint32_t vob = static_cast<uint32_t>(lane & 31) * H * 2;
    // This lane's v / output piece: row ve / VPR, stored piece ve % VPR.
    // Lanes past the tile's pieces move nothing: their global offset is out
    // of every range (loads read zero, stores are dropped) and they skip the
    // LDS write (the output piece they would read is refilled in the same
    // interval by its own lane).
    const bool vlane = ltid < kFC * VPR;
    const int ve = min(ltid, kFC * VPR - 1), vrow = ve / VPR, vpq = ve % VPR;
    const uint32_t vso = vlane ? vrow * rsv + 16 * (vpq ^ ((vrow >> 2) & VSW)) : 0x80000000u;
    // Buffer resource over the chunk's rows of one head of a token-major
    // tensor (rows past the chunk's end read as zero).
    auto tok_rsrc = [&](const void* base, const auto& x, uint32_t row_bytes, uint32_t lane_bytes,
                        uint32_t head_off) {
      return buf_rsrc(static_cast<const char*>(base) + static_cast<size_t>(x.t) * row_bytes + head_off,
                      static_cast<uint32_t>(x.n - 1) * row_bytes + lane_bytes);
    };
    auto load_raw = [&](const auto& x, Raw& r) {
      const uint32_t ho = static_cast<uint32_t>(h) * DK * 2;
      r.q = ld128(tok_rsrc(p.q, x, rsk, DK * 2, ho), vo);
      r.k = ld128(tok_rsrc(p.k, x, rsk, DK * 2, ho), vo);
      r.a = ld128(tok_rsrc(p.a, x, rsk, DK * 2, ho), vo);
      const __amdgpu_buffer_rsrc_t rb = tok_rsrc(p.beta, x, static_cast<uint32_t>(H) * 2, 2, h * 2);
      r.b = __builtin_amdgcn_raw_buffer_load_b16(rb, vob, 0, 0);
      r.n = x.n;
    };
    auto load_v = [&](const auto& x, i32x4& vr) {
      if constexpr (ID) vr = i32x4{0, 0, 0, 0};
      else vr = ld128(tok_rsrc(p.v, x, rsv, DVT * 2, (h * dv + tile * DVT) * 2), vso);
    };
    auto put_v = [&](int b, const i32x4& vr) {
      if (vlane) *reinterpret_cast<i32x4*>(&sm.vb[b][8 * ve]) = vr;
    };
    // Outputs of a chunk from vb[b] to global memory through a buffer resource
    // that ends at the chunk's last row (any = false: an empty range, every
    // store is dropped, so the call sites need no branch around it).
    auto read_o = [&](int b) { return *reinterpret_cast<const i32x4*>(&sm.vb[b][8 * ve]); };
    // (identity chains: row t of the segment [lo, hi) goes to qhat row
    // t - lo + its first row)
    char* const obase = ID ? static_cast<char*>(p.qhat) + (static_cast<int64_t>(seg_field(3, 0)) - lo) * rsv
                           : static_cast<char*>(p.o);
    auto store_o = [&](const auto& x, const i32x4& ov, bool any) {
      const __amdgpu_buffer_rsrc_t ro =
          buf_rsrc(obase + (static_cast<size_t>(x.t) * H + h) * dv * 2 + tile * DVT * 2,
                   any ? (x.n - 1) * rsv + DVT * 2 : 0u);
      __builtin_amdgcn_raw_buffer_store_b128(ov, ro, vso, 0, 0);
    };

    // ---- building a chunk's operands (chunk x, loads r, record set R3, shares B2)
    // The running sums of a are kept in log2 units (times log2 e), so every
    // exponential is one v_exp_f32.
    constexpr float kLog2e = 1.4426950408889634f;
    auto exp2f_ = [](float x) { return __builtin_amdgcn_exp2f(x); };
    auto unpack = [](const i32x4& v, int j) {
      const uint32_t u = static_cast<uint32_t>(v[j >> 1]);
      return __uint_as_float(j & 1 ? u & 0xffff0000u : u << 16);
    };
    // bf16 bit patterns of the decay range: a in [a_lo, 0] (-0 and +0 too) is
    // a pattern u with u <= bits(a_lo) as unsigned, where u >= 0x8000, or u =
    // 0; every positive value and every NaN fails one of the two tests below.
    const uint32_t a_lo_bits = __float_as_uint(p.a_lo) >> 16;
    // Slab_col positions of this lane's channels cb + 0..3 and cb + 4..7 in a
    // row of kp or qp: pieces 4 cw + 2 (g4 & 1) and the next, half g4 >> 1.
    const int q0 = 4 * cw + 2 * (g4 & 1), half = 8 * (g4 >> 1);
    auto row_piece = [&](i32x4* base, int mm, int s) {
      return reinterpret_cast<char*>(&base[16 * mm]) + 16 * swz16(mm, q0 + s) + half;
    };
    bf16x8 km0;  // this lane's Km fragment, kept for the shares formed after M
    bf16x8 kp1, qp1;  // (second-half waves) its Kp, Qp fragments, likewise
    f32x8 ref1;       // (second-half waves) G_n - G_m of its channels
    // The part of chunk x's build that needs only this wave's rows: the
    // decay range and sums (build1a), then the operands and Gram shares
    // (build1b).
    // e^{G_m} (first half) or e^{G_n - G_m} (second half) of channel
    // cb + (r16 & 7), stored by lanes 0..7 of the row: select the channel,
    // then one exponential.
    auto put_scale = [&](float* dst, f32x8 ref) {
      const bool s0 = r16 & 1, s1 = r16 & 2, s2 = r16 & 4;
      const float a01 = s0 ? ref[1] : ref[0], a23 = s0 ? ref[3] : ref[2];
      const float a45 = s0 ? ref[5] : ref[4], a67 = s0 ? ref[7] : ref[6];
      const float b03 = s1 ? a23 : a01, b47 = s1 ? a67 : a45;
      const float e = exp2f_(s2 ? b47 : b03);
      dst[cb + (r16 & 7)] = e;  // (rows r16 and r16 + 8 write the same value)
    };
    auto build1a = [&](int R3, const Raw& r, float* G) {
      FRec<DK>& rec = sm.rec[R3];
      bool bad;
      if (p.gate) {
        // a = g_min sigmoid(z) (in [g_min, 0] for finite z; zero past the
        // chunk's end), in log2 units; a NaN logit makes a NaN.
        const float gl = p.g_min * kLog2e;
        const bool in = m < r.n;
        bad = false;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const float s = __builtin_amdgcn_rcpf(1.f + exp2f_(-kLog2e * unpack(r.a, j)));
          G[j] = in ? gl * s : 0.f;
          bad |= G[j] != G[j];
        }
      } else {
        // The decay range, on the bit patterns (two per word).
        u16x2 mx = {0, 0}, mn = {0xffff, 0xffff};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const u16x2 u = as_u16x2(r.a[i]);
          mx = __builtin_elementwise_max(mx, u);
          mn = __builtin_elementwise_min(mn, u - u16x2{1, 1});  // +0 -> 0xffff; positives below 0x7fff
        }
        const uint32_t mx1 = max(static_cast<uint32_t>(mx.x), static_cast<uint32_t>(mx.y));
        const uint32_t mn1 = min(static_cast<uint32_t>(mn.x), static_cast<uint32_t>(mn.y));
        bad = mx1 > a_lo_bits || mn1 < 0x7fffu;
#pragma unroll
        for (int j = 0; j < 8; ++j) G[j] = unpack(r.a, j) * kLog2e;
      }
      if (__builtin_amdgcn_ballot_w64(bad) != 0 && lane == 0) {
        *p.wsflag = 1;
        if (p.err_flag != nullptr) *p.err_flag = 1;
        sm.stop[R3] = 1;
      }
      // Running sums over this half's 16 rows.  The first half's total is G_m
      // (with n <= 16 that is G_n: the zero rows add nothing): its rows take
      // G - G_m, and the second half's own sums are already G - G_m.
      float ref[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) G[j] = row_scan(G[j]);
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        ref[j] = row_last(G[j]);  // G_m (first half) or G_n - G_m (second half)
        if (X == 0) G[j] -= ref[j];
      }
      const f32x8 rv = {ref[0], ref[1], ref[2], ref[3], ref[4], ref[5], ref[6], ref[7]};
      if (X == 0) put_scale(rec.em, rv);
      else ref1 = rv;
    };
    // Km^T: row = channel cb + j (cb is a multiple of 8, so the swizzle of
    // row cb + j is j >> 1), token m at slab position 8 (m%16 / 4) + 4 X + m % 4.
    auto put_km = [&](FRec<DK>& rec, const bf16x8& km) {
      char* kt = reinterpret_cast<char*>(&rec.km[4 * cb]) + 2 * (4 * X + (r16 & 3));
#pragma unroll
      for (int j = 0; j < 8; ++j)
        *reinterpret_cast<__bf16*>(kt + 16 * (4 * j + ((r16 >> 2) ^ (j >> 1)))) = km[j];
    };
    // Shares of the diagonal blocks over this wave's channels, formed as
    // transposes (Km first): lane (r16, g4) then holds row r16 of the tile,
    // columns 4 g4 .. 4 g4 + 3.  Tiles: 0 = A_kk 00, 1 = A_kk 10,
    // 2 = A_kk 11, 3..5 = the same of A_qk.
    auto gram_diag = [&](int B2, const bf16x8& km, const bf16x8& kp, const bf16x8& qp) {
      const f32x4 z = zero4();
      sm.part[B2][cw][X == 0 ? 0 : 2][lane] = mma(km, kp, z);
      sm.part[B2][cw][X == 0 ? 3 : 5][lane] = mma(km, qp, z);
    };
    auto build1b = [&](int R3, int B2, const Raw& r, const float* G) {
      FRec<DK>& rec = sm.rec[R3];
      // Kp, Qp rows (slab_col order) and Km^T, and the Gram fragments.
      bf16x8 kp, qp, km;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const float kv = unpack(r.k, j), qv = unpack(r.q, j);
        const float up = exp2f_(G[j]), dn = exp2f_(-G[j]);
        kp[j] = static_cast<__bf16>(kv * up);
        qp[j] = static_cast<__bf16>(qv * up);
        km[j] = static_cast<__bf16>(kv * dn);
      }
      const i32x4 kw = __builtin_bit_cast(i32x4, kp), qw = __builtin_bit_cast(i32x4, qp);
      *reinterpret_cast<i32x2*>(row_piece(rec.kp, m, 0)) = i32x2{kw[0], kw[1]};
      *reinterpret_cast<i32x2*>(row_piece(rec.kp, m, 1)) = i32x2{kw[2], kw[3]};
      *reinterpret_cast<i32x2*>(row_piece(rec.qp, m, 0)) = i32x2{qw[0], qw[1]};
      *reinterpret_cast<i32x2*>(row_piece(rec.qp, m, 1)) = i32x2{qw[2], qw[3]};
      km0 = km;
      if (X == 0) {
        put_km(rec, km);
        gram_diag(B2, km, kp, qp);
      } else {
        kp1 = kp;
        qp1 = qp;
      }
      if (w == 0) {  // (lanes 32.. hold the same tokens' beta as lanes ..31)
        float b = __uint_as_float(r.b << 16);
        if (p.gate) b = (lane & 31) < r.n ? __builtin_amdgcn_rcpf(1.f + exp2f_(-kLog2e * b)) : 0.f;
        sm.beta[B2][lane & 31] = b;
      }
    };
    auto build1 = [&](int R3, int B2, const Raw& r) {
      float G[8];
      build1a(R3, r, G);
      build1b(R3, B2, r, G);
    };
    // After M: (second-half waves) the rest of build1b and build1a, which
    // the P waves need two intervals later at the earliest; (first-half
    // waves) the off-diagonal shares Km0 Kp1^T and Km0 Qp1^T, with rows 16..
    // of kp and qp read back from LDS.
    auto build2 = [&](int R3, int B2) {
      if (X != 0) {
        FRec<DK>& rec = sm.rec[R3];
        put_km(rec, km0);
        gram_diag(B2, km0, kp1, qp1);
        put_scale(rec.en, ref1);
        return;
      }
      const FRec<DK>& rec = sm.rec[R3];
      auto frag_of = [&](const i32x4* base) {
        const i32x2 lo2 = *reinterpret_cast<const i32x2*>(row_piece(const_cast<i32x4*>(base), 16 + r16, 0));
        const i32x2 hi2 = *reinterpret_cast<const i32x2*>(row_piece(const_cast<i32x4*>(base), 16 + r16, 1));
        return __builtin_bit_cast(bf16x8, i32x4{lo2[0], lo2[1], hi2[0], hi2[1]});
      };
      const bf16x8 kpo = frag_of(rec.kp), qpo = frag_of(rec.qp);
      const f32x4 z = zero4();
      sm.part[B2][cw][1][lane] = mma(km0, kpo, z);
      sm.part[B2][cw][4][lane] = mma(km0, qpo, z);
    };

    // After M: first-half wave 2 writes lower(A_qk), wave 3 A_10 (their SIMDs
    // host the P waves that narrow tiles leave without state).
    auto finish = [&](int B2) {
      FTri& tri = sm.tri[B2];
      if (!kPSolve && X == 1) {
        solve(I2{}, B2, cw >> 1, cw & 1);
      } else if (X == 0 && cw == 2) {
        const f32x4 a00 = sum_part(B2, 3), a10 = sum_part(B2, 4), a11 = sum_part(B2, 5);
        float m00[4], m11[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const bool on = 4 * g4 + t <= r16;
          m00[t] = on ? a00[t] : 0.f;
          m11[t] = on ? a11[t] : 0.f;
        }
        *reinterpret_cast<bf16x4*>(piece8(tri.aq, r16, 0)) = pack4(m00[0], m00[1], m00[2], m00[3]);
        *reinterpret_cast<bf16x4*>(piece8(tri.aq, 16 + r16, 0)) = pack4(a10[0], a10[1], a10[2], a10[3]);
        *reinterpret_cast<bf16x4*>(piece8(tri.aq, 16 + r16, 1)) = pack4(m11[0], m11[1], m11[2], m11[3]);
        *reinterpret_cast<bf16x4*>(piece8(tri.aq, r16, 1)) = pack4(0.f, 0.f, 0.f, 0.f);
      } else if (X == 0 && cw == 3) {
        const f32x4 a10 = sum_part(B2, 1);
        tri.ka[4 * r16 + swz4(r16, g4)] = __builtin_bit_cast(i32x2, pack4(a10[0], a10[1], a10[2], a10[3]));
      }
    };

    // The walker wr is on the chunk whose q, k, a, beta are loaded next; the
    // spans of the chunks it passed are kept for the v loads and the output
    // stores (in iteration c: h0 = chunk c + 2, h1 = c + 1, h2 = c,
    // h3 = c - 1).
    Raw rs[2];
    i32x4 vs[2];
    ChunkWalk wr = first_chunk();
    auto take = [&]() {
      const Span x{wr.t, wr.n};
      next_chunk(wr);
      return x;
    };
    // Prologue: chunk c_lo complete and chunk c_lo + 1 built, in four steps.
    load_raw(wr, rs[0]);
    const Span x0 = take();
    load_raw(wr, rs[1]);
    const Span x1 = take();
    load_v(x0, vs[0]);
    build1(b3(c_lo), b2(c_lo), rs[0]);
    slab_barrier();
    build2(b3(c_lo), b2(c_lo));
    put_v(b2(c_lo), vs[0]);
    load_v(x1, vs[1]);
    slab_barrier();
    build1(b3(c_lo + 1), b2(c_lo + 1), rs[1]);
    slab_barrier();
    build2(b3(c_lo + 1), b2(c_lo + 1));
    finish(b2(c_lo));
    load_raw(wr, rs[0]);  // chunk c_lo + 2
    Span h0 = take(), h1 = x1, h2 = x0, h3 = x0;
    slab_barrier();  // A: chunk c_lo complete
    const bool live = sm.stop[b3(c_lo)] == 0;
    int last = c_lo;  // the last chunk the P waves processed
    if (live) {
      // Chunk c is processed by the P waves during iteration c.  The loads of
      // chunk x go to register set (x - c_lo) & 1: with K = (c - c_lo) & 1,
      // set K holds q, k, a, beta of chunk c + 2 (built now) and set K ^ 1
      // those of chunk c + 1 (built during the previous iteration, so it takes
      // chunk c + 3's at once); v of chunk c + 1 (moved to LDS now) is in set
      // K ^ 1 and v of chunk c (in LDS already) leaves set K to chunk c + 2.
      using std::integral_constant;
      auto iter = [&](auto kc, int c, int r3) {  // r3 = b3(c)
        constexpr int K = decltype(kc)::value, K1 = K ^ 1;
        const int r3n = inc3(r3), r3nn = inc3(r3n);
        const bool go = sm.stop[r3n] == 0;  // (final since chunk c + 1 was built)
        // Every memory operation here is unconditional (the output store of
        // the first iteration has an empty range), so the compiler can count
        // what is in flight and waits for the loads it needs, not for
        // everything issued before.
        prio(integral_constant<int, 2>{});
        load_raw(wr, rs[K1]);  // chunk c + 3
        const Span x3 = take();
        load_v(h0, vs[K]);  // chunk c + 2
        build1(r3nn, b2(c + 2), rs[K]);
        slab_barrier();  // M
        prio(integral_constant<int, 0>{});
        const i32x4 ov = read_o(b2(c - 1));  // (vb[b2(c + 1)], before put_v refills it)
        build2(r3nn, b2(c + 2));
        finish(b2(c + 1));
        store_o(h3, ov, c > c_lo);
        put_v(b2(c + 1), vs[K1]);
        h3 = h2;
        h2 = h1;
        h1 = h0;
        h0 = x3;
        slab_barrier();  // A: chunk c + 1 complete
        last = c;
        return go;
      };
      int r3 = 0;
      for (int c = c_lo; c < c_hi; c += 2) {
        if (!iter(integral_constant<int, 0>{}, c, r3)) break;
        r3 = inc3(r3);
        if (c + 1 >= c_hi || !iter(integral_constant<int, 1>{}, c + 1, r3)) break;
        r3 = inc3(r3);
      }
    }
    // The outputs of the last chunk the P waves processed (h3 is on it).
    if (live) store_o(h3, read_o(b2(last)), true);
    return;
  }

  // ========================= P waves ==========================================
  const bool active = wave < NPA;
  // The diagonal solves (16 columns per wave): with two or fewer waves holding
  // state, waves 2 and 3 (none) invert a block each; otherwise every P wave
  // takes two columns of a block.
  auto p_solve = [&](int B2) {
    if constexpr (kPSolve) {
      if constexpr (NPA <= 2) {
        if (wave >= 2) solve(I4{}, B2, wave - 2, 0);
      } else {
        solve(I2{}, B2, wave >> 1, wave & 1);
      }
    }
  };
  const int jl = 16 * NJ * (active ? wave : 0);  // first column of this wave's slab within the tile
  const int jw = tile * DVT + jl;

  // S tile (R, J): rows 16R + 4 grp + i, column jw + slab_jcol(J, col).
  f32x4 S[NR][NJ];
#pragma unroll
  for (int R = 0; R < NR; ++R)
#pragma unroll
    for (int J = 0; J < NJ; ++J) {
      S[R][J] = zero4();
      if constexpr (ID) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
          S[R][J][i] = 16 * R + 4 * grp + i == jw + slab_jcol<NJ>(J, col) ? 1.f : 0.f;
      } else if (active && p.s0 != nullptr && !(mode & kSegZeroStart)) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int c = 16 * R + 4 * grp + i, j = jw + slab_jcol<NJ>(J, col);
          S[R][J][i] = p.s0[state_off + static_cast<size_t>(c) * dv + j];
        }
      }
    }
  uint32_t slane[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) slane[i] = ((4 * grp + i) * dv + jw + slab_jcol<NJ>(0, col)) * 4;
  auto store_state = [&](float* dst) {
#pragma unroll
    for (int R = 0; R < NR; ++R) {
      const __amdgpu_buffer_rsrc_t rs = buf_rsrc(dst + static_cast<size_t>(16 * R) * dv, 16u * dv * 4);
#pragma unroll
      for (int J = 0; J < NJ; ++J)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          __builtin_amdgcn_raw_buffer_store_b32(__float_as_int(S[R][J][i]), rs, slane[i] + 16 * J, 0, 0);
    }
  };
  // The state's rows scaled by a per-channel factor (rows 16R + 4 grp + i).
  auto scale_rows = [&](const float* f) {
#pragma unroll
    for (int R = 0; R < NR; ++R) {
      const float4 g = *reinterpret_cast<const float4*>(&f[16 * R + 4 * grp]);
#pragma unroll
      for (int J = 0; J < NJ; ++J) {
        S[R][J][0] *= g.x;
        S[R][J][1] *= g.y;
        S[R][J][2] *= g.z;
        S[R][J][3] *= g.w;
      }
    }
  };
  using OV = std::conditional_t<NJ == 2, i32x4, i32x2>;
  auto vaddr = [&](int r, int j) { return r * DVT + (((j >> 3) ^ ((r >> 2) & VSW)) << 3) + (j & 7); };
  auto stage_o = [&](int b, int T, const OV& ov) {
    *reinterpret_cast<OV*>(&sm.vb[b][vaddr(16 * T + col, jl + 4 * NJ * grp)]) = ov;
  };
  auto vval = [&](int b, int T, int J, int i) {
    if constexpr (ID) return 0.f;
    return static_cast<float>(sm.vb[b][vaddr(16 * T + 4 * grp + i, jl + slab_jcol<NJ>(J, col))]);
  };
  auto frag16 = [&](const i32x4* base, int m, int q) { return __builtin_bit_cast(bf16x8, base[16 * m + swz16(m, q)]); };
  auto frag4 = [&](const i32x4* base, int m, int q) { return __builtin_bit_cast(bf16x8, base[4 * m + swz4(m, q)]); };

  // The prologue's four steps (the L waves build chunks c_lo and c_lo + 1).
  slab_barrier();
  slab_barrier();
  p_solve(b2(c_lo));
  slab_barrier();
  slab_barrier();  // A: chunk c_lo complete
  bool done = sm.stop[b3(c_lo)] != 0;
  ChunkWalk w = first_chunk();
  for (int c = c_lo; c < c_hi && !done; ++c) {
    const int b = b2(c);
    const FRec<DK>& r = sm.rec[b3(c)];
    const FTri& tri = sm.tri[b];
    const bool is_ck = w.t + w.n == w.nck;
    const bool stop_next = sm.stop[b3(c + 1)] != 0;  // (final since chunk c + 1 was built)
    bf16x8 bU[NJ];
    // S' rounded to bf16 as MFMA operands (kept across M when a wave holds 16
    // columns; rebuilt after it otherwise, for the registers).
    constexpr bool kKeepS = NJ == 1;
    bf16x8 bSk[NKS][NJ];
    if (active) {
      scale_rows(r.em);  // S' = e^{G_m} S
      // ---- P = Kp S', Z = V - P, U = T diag(beta) Z ---------------------------
      f32x4 P[2][NJ];
#pragma unroll
      for (int T = 0; T < 2; ++T)
#pragma unroll
        for (int J = 0; J < NJ; ++J) P[T][J] = zero4();
#pragma unroll
      for (int s = 0; s < NKS; ++s) {
        bf16x8 bS[NJ];
#pragma unroll
        for (int J = 0; J < NJ; ++J) {
          bS[J] = pack_frag(S[2 * s][J], S[2 * s + 1][J]);
          if (kKeepS) bSk[s][J] = bS[J];
        }
#pragma unroll
        for (int T = 0; T < 2; ++T) {
          const bf16x8 ak = frag16(r.kp, 16 * T + col, 4 * s + grp);
#pragma unroll
          for (int J = 0; J < NJ; ++J) P[T][J] = mma(ak, bS[J], P[T][J]);
        }
      }
      // U_0 = T_00 diag(beta_0) Z_0 (row block 0 of tb: its block 01 is zero),
      // Y = Z_1 - A_10 U_0, U_1 = T_11 diag(beta_1) Y (row block 1 of tb: its
      // block 10 is zero); the zero halves of the A operands make the other
      // halves of the B operands irrelevant.
      const bf16x8 at0 = frag4(tri.tb, col, grp), at1 = frag4(tri.tb, 16 + col, grp);
      const i32x2 kl = tri.ka[4 * col + swz4(col, grp)];
      const bf16x8 a10 = __builtin_bit_cast(bf16x8, i32x4{kl[0], kl[1], 0, 0});
#pragma unroll
      for (int J = 0; J < NJ; ++J) {
        f32x4 z0, z1;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          z0[i] = vval(b, 0, J, i) - P[0][J][i];
          z1[i] = vval(b, 1, J, i) - P[1][J][i];
        }
        const f32x4 U0 = mma(at0, pack_frag(z0, z1), zero4());
        const f32x4 W = mma(a10, pack_frag(U0, U0), zero4());
        const f32x4 y = z1 - W;
        const f32x4 U1 = mma(at1, pack_frag(y, y), zero4());
        bU[J] = pack_frag(U0, U1);
      }
    }
    p_solve(b2(c + 1));
    slab_barrier();  // M (v of this chunk is dead from here on: the outputs take its place)
    if (active) {
      // ---- O^T = S'^T Qp^T + U^T A_qk^T ---------------------------------------
      f32x4 OT[NJ][2];
#pragma unroll
      for (int T = 0; T < 2; ++T)
#pragma unroll
        for (int J = 0; J < NJ; ++J) OT[J][T] = zero4();
#pragma unroll
      for (int s = 0; s < NKS; ++s) {
        bf16x8 bS[NJ];
#pragma unroll
        for (int J = 0; J < NJ; ++J) bS[J] = kKeepS ? bSk[s][J] : pack_frag(S[2 * s][J], S[2 * s + 1][J]);
#pragma unroll
        for (int T = 0; T < 2; ++T) {
          const bf16x8 aq = frag16(r.qp, 16 * T + col, 4 * s + grp);
#pragma unroll
          for (int J = 0; J < NJ; ++J) OT[J][T] = mma(bS[J], aq, OT[J][T]);
        }
      }
#pragma unroll
      for (int T = 0; T < 2; ++T) {
        const bf16x8 aa = frag4(tri.aq, 16 * T + col, grp);
        bf16x4 ov[NJ];
#pragma unroll
        for (int J = 0; J < NJ; ++J) {
          OT[J][T] = mma(bU[J], aa, OT[J][T]);
#pragma unroll
          for (int i = 0; i < 4; ++i) ov[J][i] = static_cast<__bf16>(OT[J][T][i]);
        }
        stage_o(b, T, __builtin_bit_cast(OV, ov));
      }
      // ---- S <- e^{G_n - G_m} (S' + Km^T U) -----------------------------------
#pragma unroll
      for (int R = 0; R < NR; ++R) {
        const bf16x8 a0 = frag4(r.km, 16 * R + col, grp);
#pragma unroll
        for (int J = 0; J < NJ; ++J) S[R][J] = mma(a0, bU[J], S[R][J]);
      }
      scale_rows(r.en);
      if (is_ck) {
        const int64_t slot = ld_const(p.ck_slot, w.ck);
        store_state((ID || (seg_field(2, 0) & kSegCkTemp) ? p.xpool + slot * hkv
                                                          : p.page_pool + slot * p.page_elems) +
                    static_cast<int64_t>(h) * DK * dv);
      }
    }
    slab_barrier();  // A
    done = stop_next;
    next_chunk(w);
  }
  if (active && !done) {
    float* const fin = ID || (seg_field(2, 0) & kSegFinalTemp) ? p.tstate : p.s_final;
    if (fin != nullptr) store_state(fin + (static_cast<size_t>(seg_field(1, seq)) * H + h) * DK * dv);
  }
}

// ---------------------------------------------------------------------------
// The tail: the correction of split sequences (kda_cp.hpp) by workgroups
// listed after every chain they read, so that they start only once those
// have started (workgroups start in list order), and then wait, as the
// chains finish, on a counter per (sequence, later segment, head).  The
// chains of a segment raise it when their stores are complete (1, or
// 0x10000 for a chain that stopped at a decay out of range), and so does the
// item that forms the segment's start state; an item forming a start state
// raises the next segment's counter when done (0x10000 when it corrected
// nothing), so every wait ends.  The wait is bounded too: past kTailSpin
// polls the workgroup raises the error flags and corrects nothing.  The
// split chains are the longest and start first, so they end well before
// the launch's last chains and the correction runs beside them.
//   titems [kTailInts]: rows: (0, first token, tokens, first qhat row,
//   tstate index of S_in, head, first and end token within the segment,
//   counter, count, -1, 0); states: (1, destination kind, index, B, X,
//   tstate index of S_in, 1: B and X in tstate / 0: in xpool, head,
//   counter, count, counter raised when done or -1, 0).
constexpr int kTailSpin = 1 << 24;  // polls of about 0.3 us: a few seconds

template <int DK>
__device__ __forceinline__ void fused_tail(const FusedParams& p, int item, FusedSmem<DK>& sm) {
  constexpr int NW = Fused<DK>::NT / 64;
  auto f = [&](int i) { return ld_const(p.titems, kTailInts * item + i); };
  if (threadIdx.x == 0) {
    const int want = f(9);
    int c = 0;
    for (int n = 0; n < kTailSpin; ++n) {
      c = __hip_atomic_load(p.tcnt + f(8), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if (c >= want) break;
      __builtin_amdgcn_s_sleep(8);
    }
    if (c < want) {  // (never, while every chain of the launch ends)
      *p.wsflag = 1;
      if (p.err_flag != nullptr) *p.err_flag = 1;
    }
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");  // the chains' stores are visible from here on
    sm.stop[0] = c == want;
  }
  __syncthreads();
  const bool good = sm.stop[0] != 0;
  const FixView v{p.o, p.qhat, p.tstate, p.xpool, p.page_pool, p.s_final, p.page_elems, p.H};
  char* lds = reinterpret_cast<char*>(&sm);  // (up to kFullLds bytes from its start, clear of stop[])
  if (f(0) == 0) {
    if (good) fix_rows<NW>(v, f(1), f(2), f(3), f(4), f(5), f(6), f(7), lds);
    return;
  }
  if (good) fix_state_item<NW>(v, f(1), f(2), f(3), f(4), f(5), f(6) != 0, f(7), lds);
  const int sig = f(10);
  if (sig >= 0) {  // a start state: its stores complete (every wave), then one release and the count
    vm_drain();
    __syncthreads();
    if (threadIdx.x == 0) {
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");  // (L2 written back)
      vm_drain();  // (and the write-back complete before the count)
      atomicAdd(p.tcnt + sig, good ? 1 : 0x10000);
    }
  }
}

// Entry bid of p.wgs: chain << 8 | width code << 4 | tile; width code 0: 32
// columns, 1: 64, 2: 128, 3: 16, 4: 128 from the identity (a segment's
// linear part), 5: tail item (in place of the chain), 15: no work.
template <int DK>
__global__ __launch_bounds__(Fused<DK>::NT, 1) void fused_kernel(FusedParams p) {
  __shared__ __attribute__((aligned(16))) FusedSmem<DK> sm;
  static_assert(offsetof(FusedSmem<DK>, stop) >= kRowsLds && offsetof(FusedSmem<DK>, stop) >= kFullLds,
                "the tail's LDS block lies clear of stop[]");
  const int e = ld_const(p.wgs, blockIdx.x);
  const int chain = e >> 8, code = (e >> 4) & 15, tile = e & 15;
  if (code == 5) {
    fused_tail<DK>(p, chain, sm);
    return;
  }
  if (code == 0) fused_chain<DK, 2, 1>(p, chain, tile, sm);
  else if (code == 1) fused_chain<DK, 4, 1>(p, chain, tile, sm);
  else if (code == 2) fused_chain<DK, 4, 2>(p, chain, tile, sm);
  else if (code == 3) fused_chain<DK, 1, 1>(p, chain, tile, sm);
  else if (code == 4) fused_chain<DK, 4, 2, true>(p, chain, tile, sm);
  // A chain that tail workgroups read: its stores complete (every wave),
  // then one release and the count.
  if (code <= 4 && p.segx != nullptr) {
    const int seq = ld_const(p.chains, 2 * chain);
    const int cb = seq >= 0 ? ld_const(p.segx, kSegxInts * seq + 4) : -1;
    if (cb >= 0) {
      vm_drain();
      __syncthreads();
      if (threadIdx.x == 0) {
        const bool stopped = (sm.stop[0] | sm.stop[1] | sm.stop[2]) != 0;
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");  // (L2 written back)
        vm_drain();  // (and the write-back complete before the count)
        atomicAdd(p.tcnt + cb + ld_const(p.chains, 2 * chain + 1), stopped ? 0x10000 : 1);
      }
    }
  }
}

}  // namespace

hipError_t launch_fused(const PrefillArgs& a) {
  if (a.dk != 128 || !a.bf16 || a.chunk != kFC) return hipErrorInvalidValue;
  FusedParams prm;
  prm.q = a.q; prm.k = a.k; prm.v = a.v; prm.a = a.a; prm.beta = a.beta;
  prm.s0 = a.s0; prm.o = a.o; prm.s_final = a.s_final;
  prm.page_pool = a.page_pool; prm.page_elems = a.page_elems;
  prm.chains = a.chains; prm.seqinfo = a.seqinfo; prm.ck_pos = a.ck_pos; prm.ck_slot = a.ck_slot;
  prm.wgs = a.wgs;
  prm.wsflag = a.wsflag; prm.err_flag = a.err_flag; prm.a_lo = a.a_lo;
  prm.gate = a.gate; prm.g_min = a.g_min;
  prm.H = a.H; prm.dv = a.dv;
  prm.segx = a.segx; prm.qhat = a.qhat; prm.xpool = a.xpool; prm.tstate = a.tstate;
  prm.titems = a.titems; prm.tcnt = a.tcnt;
  if (a.n_wg == 0) return hipSuccess;
  hipLaunchKernelGGL((fused_kernel<128>), dim3(static_cast<unsigned>(a.n_wg)), dim3(Fused<128>::NT), 0, a.stream,
                     prm);
  return hipGetLastError();
}

}  // namespace kda
