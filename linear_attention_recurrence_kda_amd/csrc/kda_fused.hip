// Fused chunked prefill: one kernel, one workgroup per (sequence, head, dv
// tile) chain, 32-token chunks, bf16 inputs, fp32 state, dk = 128.
//
// The chunk form is the one of kda_prefill_kernels.hpp (derived from the
// per-token recurrence; "Kimi Linear 的 KDA 缓存" page, sections "KDA 的递推与
// 充分状态" and "预填充为什么能分块并行"): per chunk of n <= 32 tokens, with
// G the running sum of the log-decays inside the chunk and G_m the reference
// (the sum over the first 16 rows when n > 16, else 0),
//   L = diag(beta) strict_lower(Kp Km^T),  Kp = k e^{G - G_m},  Km = k e^{G_m - G}
//   T = (I + L)^{-1}
//   U = T diag(beta) (V - (k e^G) S)
//   O = (q e^G) S + lower(Qp Km^T) U,       Qp = q e^{G - G_m}
//   S <- diag(e^{G_n}) S + (k e^{G_n - G})^T U
//
// What is new here is where the chunk-local part runs.  The two-kernel path
// computes T diag(beta), lower(A_qk) and the scaled operands of every chunk in
// a first kernel and passes them through HBM (a 66 KB record per chunk and
// head, written once and read back by the sequential kernel: more than twice
// the compulsory bytes).  Here the workgroup that carries the state builds
// each chunk's record in LDS ahead of use, so HBM sees only q, k, a, beta, v,
// the outputs and the states.  A 32-token chunk keeps the records in flight
// (three operand sets of 24.5 KB, two of the small tiles, two of the Gram
// shares) inside 160 KB of LDS.
//
// Eight waves, two per SIMD:
//  - waves 0..3, the propagation ("P") waves: the column-slab chunk step of
//    kda_prefill_slab.hpp on register-resident state (16 or 32 state columns
//    per wave; narrow tiles leave some P waves idle);
//  - waves 4..7, the local ("L") waves: wave w owns key channels 32w..32w+31.
//    A lane holds one token row (16 lanes per 16-row block) and eight
//    channels, loaded straight from HBM in 16-byte pieces, so the chunk's
//    running sums of a are row scans across 16 lanes (DPP), the Gram operands
//    are MFMA fragments already, and each wave forms its 32 channels' share
//    of A_kk and A_qk with six MFMAs (as transposes, so that a lane ends with
//    one row of a block: the layout the triangular solve wants).
//
// Per chunk c every wave passes two barriers, M (mid-chunk) and A (the
// hand-over); P runs chunk c's state-independent half before M and the rest
// after.  In the same interval the L waves
//  - finish chunk c+1: before M, L wave 0 inverts the diagonal block
//    (I + L_00), L wave 1 the block (I + L_11) (forward substitution by rows,
//    each step a DPP broadcast of one row within the lane row), L wave 2 adds
//    the shares of A_qk and writes lower(A_qk), L wave 3 forms L_10; after M,
//    L wave 3 forms the off-diagonal block T_10 = -T_11 L_10 T_00 with two
//    fp32 MFMA products;
//  - build chunk c+2's scaled operands and Gram shares, the first 16 token
//    rows before M, the other 16 after;
//  - store chunk c-1's outputs, move chunk c+1's v into LDS, and issue the
//    loads of chunk c+3 (q, k, a, beta) and c+2 (v) into registers.
// So a record is built over two chunk intervals and read in the third.
//
// A decay outside [a_lo, 0] (or a NaN) found while building chunk x raises
// the error flags and stops that chain at the barrier that would hand chunk x
// over: the outputs and checkpoints of the chunks before x stay written,
// nothing after them (nor the final state) is.
#include <climits>
#include <type_traits>

#include "kda_prefill_slab.hpp"

namespace kda {
namespace {

constexpr int kFC = 32;  // tokens per chunk

// One chunk's operands in LDS.  kg, qg: 32 token rows of 16 pieces (16
// bytes, slab_col channel order), piece q of row m at q ^ (m & 7); kh: dk
// channel rows of 4 pieces (32 tokens in slab_col order), piece q of row m at
// q ^ ((m >> 1) & 3).
template <int DK>
struct FRec {
  i32x4 kg[kFC * DK / 8];
  i32x4 qg[kFC * DK / 8];
  i32x4 kh[DK * 4];
  float gn[DK];
};
// T diag(beta) and lower(A_qk) of one chunk: 32 rows of 4 pieces, columns in
// slab_col order, swizzled as kh.
struct FTri {
  i32x4 tb[kFC * 4];
  i32x4 aq[kFC * 4];
};

template <int DK>
struct FusedSmem {
  FRec<DK> rec[3];
  FTri tri[2];
  __bf16 vb[2][kFC * 128];        // v of a chunk ([32][DVT], row-swizzled pieces), then its outputs
  f32x4 part[2][DK / 32][6][64];  // per chunk and L wave: shares of A_kk (tiles 00, 10, 11) and A_qk
  float lr[2][16][20];            // full rows of diag(beta) strict_lower(A_kk): blocks 00 and 11
  float t00[16][20], t11[16][20], l10[16][20];
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
// The value of lane I of this lane's row of 16 lanes (DPP row_newbcast).
template <int I>
__device__ __forceinline__ float row_bcast(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x150 + I, 0xF, 0xF,
                                                               false));
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

__device__ __forceinline__ void st_bf16(void* base, int byte_off, float x) {
  *reinterpret_cast<__bf16*>(static_cast<char*>(base) + byte_off) = static_cast<__bf16>(x);
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
  int H, dv;
};

// Loads of one chunk for one L lane: q, k, a of rows r16 and 16 + r16, this
// wave's eight channels (16 bytes each), and one beta.
struct Raw {
  i32x4 q[2], k[2], a[2];
  uint32_t b;
};
// v of one chunk: at most two 16-byte pieces per L lane (128 columns).
struct VRaw {
  i32x4 x[2];
};
// What the first half of a chunk's build hands to the second.
struct Mid {
  float G1[8], em[8], en[8];
  bf16x8 km0;
};

template <int DK>
struct Fused {
  static constexpr int NLW = DK / 32;  // L waves
  static constexpr int NPW = 4;        // P waves
  static constexpr int NT = 64 * (NPW + NLW);
  static constexpr int NR = DK / 16, NKS = DK / 32;
};

// ---------------------------------------------------------------------------
// The chain of one workgroup.  NPA P waves are active with NJ column tiles of
// 16 each (tile width DVT = 16 * NJ * NPA).
template <int DK, int NPA, int NJ>
__device__ __forceinline__ void fused_chain(const FusedParams& p, int chain, int tile, FusedSmem<DK>& sm) {
  using F = Fused<DK>;
  constexpr int NR = F::NR, NKS = F::NKS, NLW = F::NLW;
  constexpr int DVT = 16 * NJ * NPA;
  constexpr int VPR = DVT / 8;                // 16-byte pieces per v row
  constexpr int VSW = VPR < 4 ? VPR - 1 : 3;  // v row swizzle: piece q of row r at q ^ ((r >> 2) & VSW)
  constexpr int NVP = (kFC * VPR + 64 * NLW - 1) / (64 * NLW);  // v pieces per L lane
  static_assert(DK == 128, "the L waves cover 32 channels each: dk = 128 is the tuned shape");
  static_assert(NVP <= 2, "v pieces per lane");

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
  const size_t state_off = (static_cast<size_t>(seq) * H + h) * DK * dv;
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

  // Zero the page padding of this sequence's checkpoint slots (once per sequence).
  if (tile == 0 && h == 0 && p.page_elems > hkv) {
    for (int c = ck_lo; c < ck_hi; ++c) {
      float* pg = p.page_pool + static_cast<int64_t>(ld_const(p.ck_slot, c)) * p.page_elems;
      for (int64_t e = hkv + tid; e < p.page_elems; e += F::NT) pg[e] = 0.f;
    }
  }
  if (c_lo >= c_hi) {  // an empty sequence: the final state is s0
    if (!lw && wave < NPA && p.s_final != nullptr) {
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
  slab_barrier();  // (every wave passes 4 + 2 * chunks barriers)

  if (lw) {
    // ======================= L waves ==========================================
    const int w = wave - F::NPW, r16 = col, g4 = grp;
    const int cb = 32 * w + 8 * g4;  // this lane's first channel
    const int ltid = tid - 64 * F::NPW;

    auto load_raw = [&](const ChunkWalk& x, Raw& r) {
#pragma unroll
      for (int X = 0; X < 2; ++X) {
        const int row = min(16 * X + r16, x.n - 1);
        const size_t off = ((static_cast<size_t>(x.t + row) * H + h) * DK + cb) * 2;
        r.q[X] = *reinterpret_cast<const i32x4*>(static_cast<const char*>(p.q) + off);
        r.k[X] = *reinterpret_cast<const i32x4*>(static_cast<const char*>(p.k) + off);
        r.a[X] = *reinterpret_cast<const i32x4*>(static_cast<const char*>(p.a) + off);
      }
      const int row = min(lane & 31, x.n - 1);
      r.b = *reinterpret_cast<const uint16_t*>(static_cast<const char*>(p.beta) +
                                               (static_cast<size_t>(x.t + row) * H + h) * 2);
    };
    // v piece e (of 32 * VPR): row e / VPR, stored piece e % VPR.
    auto load_v = [&](const ChunkWalk& x, VRaw& vr) {
      const char* vt = static_cast<const char*>(p.v) + (static_cast<size_t>(x.t) * H + h) * dv * 2 + tile * DVT * 2;
#pragma unroll
      for (int i = 0; i < NVP; ++i) {
        const int e = min(ltid + 64 * NLW * i, kFC * VPR - 1), row = e / VPR, pq = e % VPR;
        const int src = pq ^ ((row >> 2) & VSW);
        vr.x[i] = *reinterpret_cast<const i32x4*>(vt + min(row, x.n - 1) * rsv + 16 * src);
      }
    };
    auto put_v = [&](int b, const VRaw& vr) {
#pragma unroll
      for (int i = 0; i < NVP; ++i) {
        const int e = min(ltid + 64 * NLW * i, kFC * VPR - 1);
        *reinterpret_cast<i32x4*>(&sm.vb[b][8 * e]) = vr.x[i];
      }
    };
    // Outputs of a chunk from vb[b] to global memory through a buffer resource
    // that ends at the chunk's last row (any = false: an empty range, every
    // store is dropped, so the call sites need no branch around it).
    auto store_o = [&](const ChunkWalk& x, int b, bool any) {
      i32x4 ov[NVP];
#pragma unroll
      for (int i = 0; i < NVP; ++i) {
        const int e = min(ltid + 64 * NLW * i, kFC * VPR - 1);
        ov[i] = *reinterpret_cast<const i32x4*>(&sm.vb[b][8 * e]);
      }
      const __amdgpu_buffer_rsrc_t ro =
          buf_rsrc(static_cast<char*>(p.o) + (static_cast<size_t>(x.t) * H + h) * dv * 2 + tile * DVT * 2,
                   any ? (x.n - 1) * rsv + DVT * 2 : 0u);
#pragma unroll
      for (int i = 0; i < NVP; ++i) {
        const int e = min(ltid + 64 * NLW * i, kFC * VPR - 1), r = e / VPR, pq = e % VPR;
        __builtin_amdgcn_raw_buffer_store_b128(ov[i], ro, r * rsv + 16 * (pq ^ ((r >> 2) & VSW)), 0, 0);
      }
    };

    // ---- building a chunk's operands (chunk x, loads r, record set R3, shares B2)
    // The running sums of a are kept in log2 units (times log2 e), so every
    // exponential is one v_exp_f32.  Rows past the chunk's end repeat its
    // last row (finite values): their a counts as 0, their beta is 0, so every
    // product they enter is zeroed by T diag(beta), and no k or q needs masking.
    constexpr float kLog2e = 1.4426950408889634f;
    auto exp2f_ = [](float x) { return __builtin_amdgcn_exp2f(x); };
    auto unpack = [](const i32x4& v, int j) {
      const uint32_t u = static_cast<uint32_t>(v[j >> 1]);
      return __uint_as_float(j & 1 ? u & 0xffff0000u : u << 16);
    };
    // Token rows 16 X + r16 (X = 0 or 1) of the record: kg, qg, kh, and the
    // bf16 fragments kp, qp, km of the Gram products.
    auto rows = [&](FRec<DK>& rec, int X, const Raw& r, const float* G, const float* em, const float* en,
                    bf16x8& kp, bf16x8& qp, bf16x8& km) {
      const int m = 16 * X + r16;
      bf16x4 kg0, kg1, qg0, qg1;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const float kv = unpack(r.k[X], j), qv = unpack(r.q[X], j);
        const float up = exp2f_(G[j]), dn = exp2f_(-G[j]);
        const float kpv = kv * up, qpv = qv * up, kmv = kv * dn;
        kp[j] = static_cast<__bf16>(kpv);
        qp[j] = static_cast<__bf16>(qpv);
        km[j] = static_cast<__bf16>(kmv);
        if (j < 4) {
          kg0[j] = static_cast<__bf16>(kpv * em[j]);
          qg0[j] = static_cast<__bf16>(qpv * em[j]);
        } else {
          kg1[j - 4] = static_cast<__bf16>(kpv * em[j]);
          qg1[j - 4] = static_cast<__bf16>(qpv * em[j]);
        }
        // (k e^{G_n - G})^T: row = channel, token m at slab position
        // 8 (m%16 / 4) + 4 X + m % 4.
        const int ch = cb + j;
        st_bf16(&rec.kh[4 * ch + swz4(ch, r16 >> 2)], 2 * (4 * X + (r16 & 3)), kmv * en[j]);
      }
      // Channels cb + 0..3 and cb + 4..7 in slab_col order: pieces
      // 4w + 2 (g4 & 1) and the next, half g4 >> 1 of each.
      const int q0 = 4 * w + 2 * (g4 & 1), half = 8 * (g4 >> 1);
      char* kr = reinterpret_cast<char*>(&rec.kg[16 * m]);
      char* qr = reinterpret_cast<char*>(&rec.qg[16 * m]);
      *reinterpret_cast<bf16x4*>(kr + 16 * swz16(m, q0) + half) = kg0;
      *reinterpret_cast<bf16x4*>(kr + 16 * swz16(m, q0 + 1) + half) = kg1;
      *reinterpret_cast<bf16x4*>(qr + 16 * swz16(m, q0) + half) = qg0;
      *reinterpret_cast<bf16x4*>(qr + 16 * swz16(m, q0 + 1) + half) = qg1;
    };
    // The shares of A_kk and A_qk over this wave's channels are formed as
    // transposes (K- as the first operand): lane (r16, g4) then holds row r16
    // of tile (R, I), columns 4 g4 .. 4 g4 + 3.  Tiles: 0 = A_kk 00,
    // 1 = A_kk 10, 2 = A_kk 11, 3..5 = the same of A_qk.
    auto build1 = [&](const ChunkWalk& x, int R3, int B2, const Raw& r, Mid& md) {
      FRec<DK>& rec = sm.rec[R3];
      float G0[8];
      float amin = 0.f, amax = 0.f;
      const bool v0 = r16 < x.n, v1 = 16 + r16 < x.n;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const float a0 = unpack(r.a[0], j), a1 = unpack(r.a[1], j);
        amin = fminf(amin, fminf(a0, a1));  // (repeated rows hold real values too)
        amax = fmaxf(amax, fmaxf(a0, a1));
        G0[j] = v0 ? a0 * kLog2e : 0.f;
        md.G1[j] = v1 ? a1 * kLog2e : 0.f;
      }
      bool nan = false;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        G0[j] = row_scan(G0[j]);
        const float c0 = row_last(G0[j]);  // sum over rows 0..15
        md.G1[j] = row_scan(md.G1[j]) + c0;
        const float gm = x.n > 16 ? c0 : 0.f;  // the reference G_m
        const float gn = row_last(md.G1[j]);   // the sum over the chunk (NaN if any a is)
        nan |= gn != gn;
        md.em[j] = exp2f_(gm);
        md.en[j] = exp2f_(gn - gm);
        G0[j] -= gm;
        md.G1[j] -= gm;
      }
      // (fminf/fmaxf drop NaNs; a NaN shows in the chunk's sums instead)
      if (__builtin_amdgcn_ballot_w64(nan || !(amin >= p.a_lo) || !(amax <= 0.f)) != 0 && lane == 0) {
        *p.wsflag = 1;
        if (p.err_flag != nullptr) *p.err_flag = 1;
        sm.stop[R3] = 1;
      }
      bf16x8 kp0, qp0;
      rows(rec, 0, r, G0, md.em, md.en, kp0, qp0, md.km0);
      if (r16 == 0) {
        float4 g0, g1;
        g0.x = md.em[0] * md.en[0]; g0.y = md.em[1] * md.en[1]; g0.z = md.em[2] * md.en[2]; g0.w = md.em[3] * md.en[3];
        g1.x = md.em[4] * md.en[4]; g1.y = md.em[5] * md.en[5]; g1.z = md.em[6] * md.en[6]; g1.w = md.em[7] * md.en[7];
        *reinterpret_cast<float4*>(&rec.gn[cb]) = g0;
        *reinterpret_cast<float4*>(&rec.gn[cb + 4]) = g1;
      }
      const f32x4 z = zero4();
      sm.part[B2][w][0][lane] = mma(md.km0, kp0, z);
      sm.part[B2][w][3][lane] = mma(md.km0, qp0, z);
      if (w == 0 && lane < 32) sm.beta[B2][lane] = lane < x.n ? __uint_as_float(r.b << 16) : 0.f;
    };
    auto build2 = [&](int R3, int B2, const Raw& r, const Mid& md) {
      bf16x8 kp1, qp1, km1;
      rows(sm.rec[R3], 1, r, md.G1, md.em, md.en, kp1, qp1, km1);
      const f32x4 z = zero4();
      sm.part[B2][w][1][lane] = mma(md.km0, kp1, z);
      sm.part[B2][w][2][lane] = mma(km1, kp1, z);
      sm.part[B2][w][4][lane] = mma(md.km0, qp1, z);
      sm.part[B2][w][5][lane] = mma(km1, qp1, z);
    };

    // ---- finishing a chunk (shares B2 -> tiles tri[B2]) ---------------------
    // "Row layout": lane (r16, g4) holds row r16 of a 16x16 block, columns
    // 4 g4 .. 4 g4 + 3; "column layout": column r16, rows 4 g4 .. 4 g4 + 3
    // (the layout of an MFMA result).
    auto sum_part = [&](int B2, int t) {
      f32x4 s = sm.part[B2][0][t][lane];
#pragma unroll
      for (int u = 1; u < NLW; ++u) s += sm.part[B2][u][t][lane];
      return s;
    };
    // 8-byte piece of a [32][32] tile: row m, columns 4 g4 .. +3 of the left
    // (hi = 0) or right (hi = 1) 16 columns (slab_col order puts them side by
    // side in piece g4).
    auto piece8 = [&](i32x4* t, int m, int hi) {
      return reinterpret_cast<bf16x4*>(reinterpret_cast<char*>(&t[4 * m + swz4(m, g4)]) + 8 * hi);
    };
    auto pack4 = [](float a0, float a1, float a2, float a3) {
      bf16x4 v;
      v[0] = static_cast<__bf16>(a0); v[1] = static_cast<__bf16>(a1);
      v[2] = static_cast<__bf16>(a2); v[3] = static_cast<__bf16>(a3);
      return v;
    };
    // (I + L_RR)^{-1} of diagonal block R (L wave R): by rows, step i folds
    // row i (final by then; lane i of this lane's row of 16) into every row
    // below it.
    auto solve_diag = [&](int B2, int R) {
      FTri& tri = sm.tri[B2];
      const float* beta = sm.beta[B2];
      const f32x4 a = sum_part(B2, R == 0 ? 0 : 2);
      const float br = beta[16 * R + r16];
      const float4 bc = *reinterpret_cast<const float4*>(&beta[16 * R + 4 * g4]);
      float l[4];
#pragma unroll
      for (int t = 0; t < 4; ++t) l[t] = 4 * g4 + t < r16 ? br * a[t] : 0.f;
      *reinterpret_cast<float4*>(&sm.lr[R][r16][4 * g4]) = make_float4(l[0], l[1], l[2], l[3]);
      wave_sync();
      float L[16];
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const float4 x4 = *reinterpret_cast<const float4*>(&sm.lr[R][r16][4 * q4]);
        L[4 * q4] = x4.x; L[4 * q4 + 1] = x4.y; L[4 * q4 + 2] = x4.z; L[4 * q4 + 3] = x4.w;
      }
      float T[4];
#pragma unroll
      for (int t = 0; t < 4; ++t) T[t] = 4 * g4 + t == r16 ? 1.f : 0.f;
      static_for<0, 15>([&](auto ic) {
        constexpr int i = decltype(ic)::value;
#pragma unroll
        for (int t = 0; t < 4; ++t) T[t] -= L[i] * row_bcast<i>(T[t]);
      });
      float(*tt)[20] = R == 0 ? sm.t00 : sm.t11;
      *reinterpret_cast<float4*>(&tt[r16][4 * g4]) = make_float4(T[0], T[1], T[2], T[3]);
      *piece8(tri.tb, 16 * R + r16, R) = pack4(T[0] * bc.x, T[1] * bc.y, T[2] * bc.z, T[3] * bc.w);
      if (R == 0) *piece8(tri.tb, r16, 1) = pack4(0.f, 0.f, 0.f, 0.f);  // the upper-right block
    };
    auto finish1 = [&](int B2) {  // before M
      if (w == 0 || w == 1) {
        solve_diag(B2, w);
      } else if (w == 2) {
        FTri& tri = sm.tri[B2];
        const f32x4 a00 = sum_part(B2, 3), a10 = sum_part(B2, 4), a11 = sum_part(B2, 5);
        float m00[4], m11[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const bool on = 4 * g4 + t <= r16;
          m00[t] = on ? a00[t] : 0.f;
          m11[t] = on ? a11[t] : 0.f;
        }
        *piece8(tri.aq, r16, 0) = pack4(m00[0], m00[1], m00[2], m00[3]);
        *piece8(tri.aq, 16 + r16, 0) = pack4(a10[0], a10[1], a10[2], a10[3]);
        *piece8(tri.aq, 16 + r16, 1) = pack4(m11[0], m11[1], m11[2], m11[3]);
        *piece8(tri.aq, r16, 1) = pack4(0.f, 0.f, 0.f, 0.f);
      } else {
        const f32x4 a10 = sum_part(B2, 1);
        const float br = sm.beta[B2][16 + r16];
        *reinterpret_cast<float4*>(&sm.l10[r16][4 * g4]) =
            make_float4(br * a10[0], br * a10[1], br * a10[2], br * a10[3]);
      }
    };
    // After M (L wave 3): T_10 = -T_11 (L_10 T_00), two fp32 MFMA products
    // (16x16x4, contraction index 4 g4 + kb); the result is in column layout.
    auto finish2 = [&](int B2) {
      if (w != 3) return;
      f32x4 W = zero4();
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
        W = __builtin_amdgcn_mfma_f32_16x16x4f32(sm.l10[r16][4 * g4 + kb], sm.t00[4 * g4 + kb][r16], W, 0, 0, 0);
      f32x4 T10 = zero4();
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
        T10 = __builtin_amdgcn_mfma_f32_16x16x4f32(sm.t11[r16][4 * g4 + kb], W[kb], T10, 0, 0, 0);
      const float bc = sm.beta[B2][r16];
      char* tb = reinterpret_cast<char*>(sm.tri[B2].tb);
      const int sp = slab_col(r16);
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const int row = 16 + 4 * g4 + t;
        *reinterpret_cast<__bf16*>(tb + 16 * (4 * row + swz4(row, sp >> 3)) + 2 * (sp & 7)) =
            static_cast<__bf16>(-T10[t] * bc);
      }
    };

    // Walkers: wr the chunk whose q, k, a, beta are loaded next, wv whose v,
    // wb whose operands are built next, wo whose outputs are stored next.
    Raw rs[2];
    VRaw vs[2];
    Mid md;
    ChunkWalk wr = first_chunk(), wv = wr, wb = wr, wo = wr;
    // Prologue: chunk c_lo complete and chunk c_lo + 1 built, in three steps.
    load_raw(wr, rs[0]);
    next_chunk(wr);
    load_raw(wr, rs[1]);
    next_chunk(wr);
    load_v(wv, vs[0]);
    next_chunk(wv);
    load_v(wv, vs[1]);
    next_chunk(wv);
    build1(wb, b3(c_lo), b2(c_lo), rs[0], md);
    build2(b3(c_lo), b2(c_lo), rs[0], md);
    slab_barrier();
    next_chunk(wb);
    finish1(b2(c_lo));
    build1(wb, b3(c_lo + 1), b2(c_lo + 1), rs[1], md);
    load_raw(wr, rs[0]);  // chunk c_lo + 2
    next_chunk(wr);
    slab_barrier();
    finish2(b2(c_lo));
    build2(b3(c_lo + 1), b2(c_lo + 1), rs[1], md);
    put_v(b2(c_lo), vs[0]);
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
      auto iter = [&](auto kc, int c) {
        constexpr int K = decltype(kc)::value, K1 = K ^ 1;
        // Every memory operation here is unconditional (the output store of
        // the first iteration has an empty range), so the compiler can count
        // what is in flight and waits for the loads it needs, not for
        // everything issued before.
        store_o(wo, b2(c - 1), c > c_lo);
        if (c > c_lo) next_chunk(wo);
        load_raw(wr, rs[K1]);  // chunk c + 3
        next_chunk(wr);
        load_v(wv, vs[K]);  // chunk c + 2
        next_chunk(wv);
        finish1(b2(c + 1));
        next_chunk(wb);
        build1(wb, b3(c + 2), b2(c + 2), rs[K], md);
        slab_barrier();  // M
        finish2(b2(c + 1));
        build2(b3(c + 2), b2(c + 2), rs[K], md);
        put_v(b2(c + 1), vs[K1]);
        slab_barrier();  // A: chunk c + 1 complete
        last = c;
        return sm.stop[b3(c + 1)] == 0;
      };
      for (int c = c_lo; c < c_hi; c += 2) {
        if (!iter(integral_constant<int, 0>{}, c)) break;
        if (c + 1 >= c_hi || !iter(integral_constant<int, 1>{}, c + 1)) break;
      }
    }
    // The outputs of the last chunk the P waves processed (wo points at it).
    if (live) store_o(wo, b2(last), true);
    return;
  }

  // ========================= P waves ==========================================
  const bool active = wave < NPA;
  const int jl = 16 * NJ * (active ? wave : 0);  // first column of this wave's slab within the tile
  const int jw = tile * DVT + jl;

  // S tile (R, J): rows 16R + 4 grp + i, column jw + slab_jcol(J, col).
  f32x4 S[NR][NJ];
#pragma unroll
  for (int R = 0; R < NR; ++R)
#pragma unroll
    for (int J = 0; J < NJ; ++J) {
      S[R][J] = zero4();
      if (active && p.s0 != nullptr) {
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
  using OV = std::conditional_t<NJ == 2, i32x4, i32x2>;
  auto vaddr = [&](int r, int j) { return r * DVT + (((j >> 3) ^ ((r >> 2) & VSW)) << 3) + (j & 7); };
  auto stage_o = [&](int b, int T, const OV& ov) {
    *reinterpret_cast<OV*>(&sm.vb[b][vaddr(16 * T + col, jl + 4 * NJ * grp)]) = ov;
  };
  auto vval = [&](int b, int T, int J, int i) {
    return static_cast<float>(sm.vb[b][vaddr(16 * T + 4 * grp + i, jl + slab_jcol<NJ>(J, col))]);
  };
  auto frag16 = [&](const i32x4* base, int m, int q) { return __builtin_bit_cast(bf16x8, base[16 * m + swz16(m, q)]); };
  auto frag4 = [&](const i32x4* base, int m, int q) { return __builtin_bit_cast(bf16x8, base[4 * m + swz4(m, q)]); };

  slab_barrier();  // the prologue's three steps
  slab_barrier();
  slab_barrier();  // A: chunk c_lo complete (the L waves built it)
  bool done = sm.stop[b3(c_lo)] != 0;
  ChunkWalk w = first_chunk();
  for (int c = c_lo; c < c_hi && !done; ++c) {
    const int b = b2(c);
    const FRec<DK>& r = sm.rec[b3(c)];
    const FTri& tri = sm.tri[b];
    const bool is_ck = w.t + w.n == w.nck;
    if (active) {
      // ---- P = (k g) S, Z = V - P, U = T diag(beta) Z --------------------------
      f32x4 P[2][NJ];
#pragma unroll
      for (int T = 0; T < 2; ++T)
#pragma unroll
        for (int J = 0; J < NJ; ++J) P[T][J] = zero4();
#pragma unroll
      for (int s = 0; s < NKS; ++s) {
        bf16x8 bS[NJ];
#pragma unroll
        for (int J = 0; J < NJ; ++J) bS[J] = pack_frag(S[2 * s][J], S[2 * s + 1][J]);
#pragma unroll
        for (int T = 0; T < 2; ++T) {
          const bf16x8 ak = frag16(r.kg, 16 * T + col, 4 * s + grp);
#pragma unroll
          for (int J = 0; J < NJ; ++J) P[T][J] = mma(ak, bS[J], P[T][J]);
        }
      }
      bf16x8 bU[NJ];
      {
        bf16x8 bZ[NJ];
#pragma unroll
        for (int J = 0; J < NJ; ++J) {
          f32x4 z0, z1;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            z0[i] = vval(b, 0, J, i) - P[0][J][i];
            z1[i] = vval(b, 1, J, i) - P[1][J][i];
          }
          bZ[J] = pack_frag(z0, z1);
        }
        f32x4 U[2][NJ];
#pragma unroll
        for (int T = 0; T < 2; ++T) {
          const bf16x8 at = frag4(tri.tb, 16 * T + col, grp);
#pragma unroll
          for (int J = 0; J < NJ; ++J) U[T][J] = mma(at, bZ[J], zero4());
        }
#pragma unroll
        for (int J = 0; J < NJ; ++J) bU[J] = pack_frag(U[0][J], U[1][J]);
      }
      slab_barrier();  // M (v of this chunk is dead from here on: the outputs take its place)
      // ---- O^T = S^T (q g)^T + U^T A_qk^T --------------------------------------
      f32x4 OT[NJ][2];
#pragma unroll
      for (int T = 0; T < 2; ++T)
#pragma unroll
        for (int J = 0; J < NJ; ++J) OT[J][T] = zero4();
#pragma unroll
      for (int s = 0; s < NKS; ++s) {
        bf16x8 bS[NJ];
#pragma unroll
        for (int J = 0; J < NJ; ++J) bS[J] = pack_frag(S[2 * s][J], S[2 * s + 1][J]);
#pragma unroll
        for (int T = 0; T < 2; ++T) {
          const bf16x8 aq = frag16(r.qg, 16 * T + col, 4 * s + grp);
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
      // ---- S <- diag(g_n) S + (k g_n/g)^T U -----------------------------------
#pragma unroll
      for (int R = 0; R < NR; ++R) {
        const float4 gn = *reinterpret_cast<const float4*>(&r.gn[16 * R + 4 * grp]);
        const bf16x8 a0 = frag4(r.kh, 16 * R + col, grp);
#pragma unroll
        for (int J = 0; J < NJ; ++J) {
          S[R][J][0] *= gn.x;
          S[R][J][1] *= gn.y;
          S[R][J][2] *= gn.z;
          S[R][J][3] *= gn.w;
          S[R][J] = mma(a0, bU[J], S[R][J]);
        }
      }
      if (is_ck)
        store_state(p.page_pool + static_cast<int64_t>(ld_const(p.ck_slot, w.ck)) * p.page_elems +
                    static_cast<int64_t>(h) * DK * dv);
    } else {
      slab_barrier();  // M
    }
    slab_barrier();  // A
    done = sm.stop[b3(c + 1)] != 0;
    next_chunk(w);
  }
  if (active && !done && p.s_final != nullptr) store_state(p.s_final + state_off);
}

// Entry bid of p.wgs: chain << 8 | width code << 4 | tile; width code 0: 32
// columns, 1: 64, 2: 128, 3: 16, 15: no work.
template <int DK>
__global__ __launch_bounds__(Fused<DK>::NT, 1) void fused_kernel(FusedParams p) {
  __shared__ __attribute__((aligned(16))) FusedSmem<DK> sm;
  const int e = ld_const(p.wgs, blockIdx.x);
  const int chain = e >> 8, code = (e >> 4) & 15, tile = e & 15;
  if (code == 0) fused_chain<DK, 2, 1>(p, chain, tile, sm);
  else if (code == 1) fused_chain<DK, 4, 1>(p, chain, tile, sm);
  else if (code == 2) fused_chain<DK, 4, 2>(p, chain, tile, sm);
  else if (code == 3) fused_chain<DK, 1, 1>(p, chain, tile, sm);
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
  prm.H = a.H; prm.dv = a.dv;
  if (a.n_wg == 0) return hipSuccess;
  hipLaunchKernelGGL((fused_kernel<128>), dim3(static_cast<unsigned>(a.n_wg)), dim3(Fused<128>::NT), 0, a.stream,
                     prm);
  return hipGetLastError();
}

}  // namespace kda
