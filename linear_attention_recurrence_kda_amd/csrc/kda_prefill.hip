// Chunked KDA prefill with checkpoint emission, bf16 MFMA on gfx950.
//
// Math.  The "Kimi Linear 的 KDA 缓存" page (section "预填充为什么能分块并行")
// notes that inside a chunk every state transition is a diagonal matrix minus
// a rank-one matrix, so a chunk compresses, via a WY representation and a UT
// transform, into matrix products and a small lower-triangular solve.  The
// form used here is derived from the per-token recurrence (decay, then error,
// then write; section "KDA 的递推与充分状态").  For one head and a chunk of
// n rows with start state S (dk x dv):
//   G_r = sum_{i<=r} a_i (per key channel),  g_r = exp(G_r)
//   L   = diag(beta) strict_lower(Kp Km^T),   Kp_r = k_r*e^{G_r-G_m}, Km_i = k_i*e^{G_m-G_i}
//   T   = (I + L)^{-1}                        (unit lower triangular)
//   W   = T diag(beta) (k*g),   Ut = T diag(beta) V
//   U   = Ut - W S
//   O   = (q*g) S + lower(Qp Km^T) U,         Qp_r = q_r*e^{G_r-G_m}
//   S  <- diag(g_n) S + (k*g_n/g)^T U
// The reference row m sits mid-chunk, so every scaled operand stays within
// e^{+-|a|*C/2}: finite in bf16/fp32 for per-token log-decays a >= -2.5 at a
// chunk of 64.  Every other scaled operand is bounded by 1.
//
// Mapping.  One workgroup (4 waves) runs one (sequence, head) chain over a
// DVT-wide tile of the dv columns (the columns of S are independent in the
// recurrence, so a chain can be split over several workgroups that each redo
// the key-side work).  The fp32 state tile lives in MFMA accumulators for the
// whole sequence; a bf16 transposed copy in LDS feeds the contractions.  All
// contractions use v_mfma_f32_16x16x32_bf16 with operands staged in LDS.
// T is inverted in fp32: the four 16x16 diagonal blocks by forward
// substitution, the off-diagonal blocks by block recursion.
// Workgroups are placed so the tiles of one chain share an XCD (and its L2),
// and chains run longest sequence first.
#include "kda_device.hpp"
#include "kda_internal.hpp"

namespace kda {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef int i32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;

// Operand storage: bf16 (bf16 inputs, chunk up to 64) or fp32 (fp32 inputs,
// chunk up to 32).  Rows of LDS operand buffers are padded by 16 bytes.
template <typename ST>
struct Op;
template <>
struct Op<__bf16> {
  static constexpr int MAXC = 64, PAD = 8;
};
template <>
struct Op<float> {
  static constexpr int MAXC = 32, PAD = 4;
};

__device__ __forceinline__ void put(__bf16* p, float x) { *p = static_cast<__bf16>(x); }
__device__ __forceinline__ void put(float* p, float x) { *p = x; }
__device__ __forceinline__ void put2(__bf16* p, float x, float y) {
  bf16x2 r;
  r[0] = static_cast<__bf16>(x);
  r[1] = static_cast<__bf16>(y);
  *reinterpret_cast<bf16x2*>(p) = r;
}
__device__ __forceinline__ void put2(float* p, float x, float y) {
  *reinterpret_cast<float2*>(p) = make_float2(x, y);
}
__device__ __forceinline__ void put4(__bf16* p, const float* x) {
  bf16x4 r;
#pragma unroll
  for (int i = 0; i < 4; ++i) r[i] = static_cast<__bf16>(x[i]);
  *reinterpret_cast<bf16x4*>(p) = r;
}
__device__ __forceinline__ void put4(float* p, const float* x) {
  *reinterpret_cast<float4*>(p) = make_float4(x[0], x[1], x[2], x[3]);
}
__device__ __forceinline__ void put8(__bf16* p, const float* x) {
  bf16x8 r;
#pragma unroll
  for (int i = 0; i < 8; ++i) r[i] = static_cast<__bf16>(x[i]);
  *reinterpret_cast<bf16x8*>(p) = r;
}
__device__ __forceinline__ void put8(float* p, const float* x) {
  *reinterpret_cast<float4*>(p) = make_float4(x[0], x[1], x[2], x[3]);
  *reinterpret_cast<float4*>(p + 4) = make_float4(x[4], x[5], x[6], x[7]);
}

struct Params {
  const void *q, *k, *v, *a, *beta;
  const float* s0;
  void* o;
  float* s_final;
  float* page_pool;
  int64_t page_elems;
  const int32_t* chains;   // [n_chains][2] = (sequence or -1, head)
  const int32_t* seqinfo;  // [n_seqs][4]  = (tok_lo, tok_hi, ck_lo, ck_hi)
  const int32_t* ck_pos;   // [n_ckpt] token counts from the sequence start
  const int32_t* ck_slot;  // [n_ckpt]
  int H, dv, chunk, dv_tiles;
};

template <int DK, int DVT, typename ST>
struct Smem {
  static constexpr int MAXC = Op<ST>::MAXC;
  static constexpr int LDK = DK + Op<ST>::PAD;   // row length of [*][DK] buffers
  static constexpr int LC = MAXC + Op<ST>::PAD;  // row length of [*][chunk] buffers
  static constexpr int LF = MAXC + 1;            // row length of fp32 [chunk][chunk]
  union {
    struct {  // key-side operands of the Gram products (mid-chunk reference)
      ST kpm[MAXC][LDK], qpm[MAXC][LDK], kmm[MAXC][LDK];
    } gram;
    struct {  // chunk-start scaled operands of the propagation
      ST bkpT[DK][LC];      // (beta * k * g)^T
      ST qp[MAXC][LDK];     // q * g
      ST khT[DK][LC];       // (k * g_n / g)^T
    } prop;
  } u;
  ST bvT[DVT][LC];          // (beta * v)^T, this workgroup's columns
  ST sT[DVT][LDK];          // S^T
  union {
    float Lf[MAXC][LF];     // diag(beta) strict_lower(A_kk), fp32
    ST w[MAXC][LDK];        // W, row-major
  } lw;
  float Tf[MAXC][LF];       // T in fp32 (upper blocks: scratch)
  ST Tb[MAXC][LC];          // T
  ST aqk[MAXC][LC];         // lower(Qp Km^T)
  ST uT[DVT][LC];           // U^T
  float tot[MAXC / 16][DK]; // per-16-row-block sums of a
  float gmid[DK], gend[DK], gexp[DK];
  float beta[MAXC];
};

__device__ __forceinline__ bf16x8 zero8() { return __builtin_bit_cast(bf16x8, i32x4{0, 0, 0, 0}); }

// acc += A[0:16, 0:kvalid] * Bt[0:16, 0:kvalid]^T for 16-row slabs A (row
// stride lda) and Bt (row stride ldb) in LDS.  Lane l ends with rows
// 4*(l/16)+0..3 of column l%16 of the 16x16 result.
__device__ __forceinline__ f32x4 tile_mma(f32x4 acc, const __bf16* A, int lda, const __bf16* Bt,
                                          int ldb, int kvalid, int lane) {
  const int row = lane & 15, kk = (lane >> 4) * 8;
  const __bf16* ap = A + row * lda + kk;
  const __bf16* bp = Bt + row * ldb + kk;
  for (int k0 = 0; k0 < kvalid; k0 += 32) {
    bf16x8 fa = zero8(), fb = zero8();
    if (k0 + kk < kvalid) {
      fa = *reinterpret_cast<const bf16x8*>(ap + k0);
      fb = *reinterpret_cast<const bf16x8*>(bp + k0);
    }
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa, fb, acc, 0, 0, 0);
  }
  return acc;
}

// fp32 operands: x = hi + lo with hi = bf16(x), lo = bf16(x - hi); the product
// keeps hi*hi + hi*lo + lo*hi.
__device__ __forceinline__ void split8(const float* p, bf16x8& hi, bf16x8& lo) {
  const float4 x0 = *reinterpret_cast<const float4*>(p);
  const float4 x1 = *reinterpret_cast<const float4*>(p + 4);
  const float x[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    hi[i] = static_cast<__bf16>(x[i]);
    lo[i] = static_cast<__bf16>(x[i] - static_cast<float>(hi[i]));
  }
}

__device__ __forceinline__ f32x4 tile_mma(f32x4 acc, const float* A, int lda, const float* Bt,
                                          int ldb, int kvalid, int lane) {
  const int row = lane & 15, kk = (lane >> 4) * 8;
  const float* ap = A + row * lda + kk;
  const float* bp = Bt + row * ldb + kk;
  for (int k0 = 0; k0 < kvalid; k0 += 32) {
    bf16x8 ah = zero8(), al = zero8(), bh = zero8(), bl = zero8();
    if (k0 + kk < kvalid) {
      split8(ap + k0, ah, al);
      split8(bp + k0, bh, bl);
    }
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(al, bh, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, bl, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, bh, acc, 0, 0, 0);
  }
  return acc;
}

__device__ __forceinline__ float ld(const float* p, size_t i) { return p[i]; }
__device__ __forceinline__ float ld(const bf16raw* p, size_t i) { return to_f32(p[i]); }


template <typename InT>
struct StoreOf {
  using type = __bf16;
};
template <>
struct StoreOf<float> {
  using type = float;
};

template <int DK, int DVT, typename InT>
__global__ __launch_bounds__(kThreads, 1) void prefill_kernel(Params p) {
  using ST = typename StoreOf<InT>::type;
  using SM = Smem<DK, DVT, ST>;
  constexpr int HK = DK / 2;  // channel pairs
  constexpr int LDK = SM::LDK, LC = SM::LC;
  constexpr int NCT = DK / 16, NJT = DVT / 16;
  constexpr int NST = NCT * NJT, NS = (NST + 3) / 4;
  __shared__ __attribute__((aligned(16))) SM sm;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int H = p.H, dv = p.dv;

  // Workgroup -> (chain, dv tile): the tiles of a chain land on one XCD.
  const int bid = blockIdx.x, xcd = bid & 7, local = bid >> 3;
  const int chain = 8 * (local / p.dv_tiles) + xcd, tile = local % p.dv_tiles;
  const int seq = p.chains[2 * chain], h = p.chains[2 * chain + 1];
  if (seq < 0) return;
  const int lo = p.seqinfo[4 * seq], hi = p.seqinfo[4 * seq + 1];
  const int ck_lo = p.seqinfo[4 * seq + 2], ck_hi = p.seqinfo[4 * seq + 3];
  const int j0 = tile * DVT;
  const int64_t hkv = static_cast<int64_t>(H) * DK * dv;
  const size_t state_off = (static_cast<size_t>(seq) * H + h) * DK * dv;

  const InT* __restrict__ gq = static_cast<const InT*>(p.q);
  const InT* __restrict__ gk = static_cast<const InT*>(p.k);
  const InT* __restrict__ gv = static_cast<const InT*>(p.v);
  const InT* __restrict__ ga = static_cast<const InT*>(p.a);
  const InT* __restrict__ gb = static_cast<const InT*>(p.beta);
  InT* __restrict__ go = static_cast<InT*>(p.o);

  // State tile: accumulator tile s = wave + 4u covers rows 16*(s/NJT) and
  // columns j0 + 16*(s%NJT).
  f32x4 S[NS];
#pragma unroll
  for (int u = 0; u < NS; ++u) {
    const int s = wave + 4 * u;
    S[u] = f32x4{0.f, 0.f, 0.f, 0.f};
    if (s < NST && p.s0 != nullptr) {
      const int c0 = 16 * (s / NJT) + 4 * (lane >> 4), j = j0 + 16 * (s % NJT) + (lane & 15);
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) S[u][rr] = p.s0[state_off + static_cast<size_t>(c0 + rr) * dv + j];
    }
  }
  auto write_sT = [&]() {
#pragma unroll
    for (int u = 0; u < NS; ++u) {
      const int s = wave + 4 * u;
      if (s < NST) {
        const int c0 = 16 * (s / NJT) + 4 * (lane >> 4), jl = 16 * (s % NJT) + (lane & 15);
        const float x[4] = {S[u][0], S[u][1], S[u][2], S[u][3]};
        put4(&sm.sT[jl][c0], x);
      }
    }
  };
  auto store_state = [&](float* dst) {  // dst points at this head's [DK][dv] block
#pragma unroll
    for (int u = 0; u < NS; ++u) {
      const int s = wave + 4 * u;
      if (s < NST) {
        const int c0 = 16 * (s / NJT) + 4 * (lane >> 4), j = j0 + 16 * (s % NJT) + (lane & 15);
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) dst[static_cast<size_t>(c0 + rr) * dv + j] = S[u][rr];
      }
    }
  };
  write_sT();

  // Zero the page padding of this sequence's checkpoint slots (once per sequence).
  if (tile == 0 && h == 0 && p.page_elems > hkv) {
    for (int c = ck_lo; c < ck_hi; ++c) {
      float* pg = p.page_pool + static_cast<int64_t>(p.ck_slot[c]) * p.page_elems;
      for (int64_t e = hkv + tid; e < p.page_elems; e += kThreads) pg[e] = 0.f;
    }
  }

  // Prep mapping: thread -> channel pair cp, 16-row block g.
  const int cp = tid % HK, g = tid / HK;
  const int c0p = 2 * cp;

  int t0 = lo, ck = ck_lo;
  while (t0 < hi) {
    int end = min(t0 + p.chunk, hi);
    if (ck < ck_hi) end = min(end, lo + p.ck_pos[ck]);
    const int n = end - t0;
    const int nb = (n + 15) >> 4;
    const bool act = g < nb;

    // ---- load the chunk; per-block cumulative sums of a -------------------
    float kr[16][2], qr[16][2], gr[16][2];
    if (act) {
      float run0 = 0.f, run1 = 0.f;
#pragma unroll
      for (int rr = 0; rr < 16; ++rr) {
        const int r = 16 * g + rr;
        float k0 = 0.f, k1 = 0.f, q0 = 0.f, q1 = 0.f, a0 = 0.f, a1 = 0.f;
        if (r < n) {
          const size_t off = (static_cast<size_t>(t0 + r) * H + h) * DK + c0p;
          k0 = ld(gk, off); k1 = ld(gk, off + 1);
          q0 = ld(gq, off); q1 = ld(gq, off + 1);
          a0 = ld(ga, off); a1 = ld(ga, off + 1);
        }
        run0 += a0; run1 += a1;
        kr[rr][0] = k0; kr[rr][1] = k1; qr[rr][0] = q0; qr[rr][1] = q1;
        gr[rr][0] = run0; gr[rr][1] = run1;
      }
      sm.tot[g][c0p] = run0;
      sm.tot[g][c0p + 1] = run1;
    }
    if (tid < 16 * nb) sm.beta[tid] = tid < n ? ld(gb, static_cast<size_t>(t0 + tid) * H + h) : 0.f;
    // (beta * v)^T for this tile: thread -> (column j, 8 consecutive rows).
    for (int idx = tid; idx < DVT * 2 * nb; idx += kThreads) {
      const int j = idx % DVT, rb = idx / DVT;
      float x[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int r = 8 * rb + e;
        x[e] = 0.f;
        if (r < n) {
          const size_t tr = static_cast<size_t>(t0 + r) * H + h;
          x[e] = ld(gb, tr) * ld(gv, tr * dv + j0 + j);
        }
      }
      put8(&sm.bvT[j][8 * rb], x);
    }
    __syncthreads();

    // ---- cumulative sums across blocks; reference rows --------------------
    const int mrow = 8 * nb;  // mid-chunk reference row
    if (act) {
      float pre0 = 0.f, pre1 = 0.f;
      for (int gg = 0; gg < g; ++gg) { pre0 += sm.tot[gg][c0p]; pre1 += sm.tot[gg][c0p + 1]; }
#pragma unroll
      for (int rr = 0; rr < 16; ++rr) { gr[rr][0] += pre0; gr[rr][1] += pre1; }
      if (g == (mrow >> 4)) {
#pragma unroll
        for (int rr = 0; rr < 16; ++rr)
          if (rr == (mrow & 15)) { sm.gmid[c0p] = gr[rr][0]; sm.gmid[c0p + 1] = gr[rr][1]; }
      }
      if (g == nb - 1) {
        sm.gend[c0p] = gr[15][0]; sm.gend[c0p + 1] = gr[15][1];
        sm.gexp[c0p] = fast_exp(gr[15][0]); sm.gexp[c0p + 1] = fast_exp(gr[15][1]);
      }
    }
    __syncthreads();

    // ---- Gram operands (mid-chunk reference) ------------------------------
    if (act) {
      const float m0 = sm.gmid[c0p], m1 = sm.gmid[c0p + 1];
#pragma unroll
      for (int rr = 0; rr < 16; ++rr) {
        const int r = 16 * g + rr;
        const float d0 = gr[rr][0] - m0, d1 = gr[rr][1] - m1;
        const float up0 = fast_exp(d0), up1 = fast_exp(d1);
        const float dn0 = fast_exp(-d0), dn1 = fast_exp(-d1);
        put2(&sm.u.gram.kpm[r][c0p], kr[rr][0] * up0, kr[rr][1] * up1);
        put2(&sm.u.gram.qpm[r][c0p], qr[rr][0] * up0, qr[rr][1] * up1);
        put2(&sm.u.gram.kmm[r][c0p], kr[rr][0] * dn0, kr[rr][1] * dn1);
      }
    }
    __syncthreads();

    // ---- Gram products: L = diag(beta) strict_lower(A_kk), Aqk = lower(A_qk)
    {
      const int ntri = nb * (nb + 1) / 2;
      for (int tt = wave; tt < 2 * ntri; tt += 4) {
        const bool qk = tt >= ntri;
        int x = qk ? tt - ntri : tt, R = 0;
        while (x > R) { x -= R + 1; ++R; }
        const int I = x;
        const ST* A = qk ? &sm.u.gram.qpm[16 * R][0] : &sm.u.gram.kpm[16 * R][0];
        f32x4 acc = tile_mma(f32x4{0.f, 0.f, 0.f, 0.f}, A, LDK, &sm.u.gram.kmm[16 * I][0], LDK,
                             DK, lane);
        const int col = 16 * I + (lane & 15);
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
          const int row = 16 * R + 4 * (lane >> 4) + rr;
          if (qk) put(&sm.aqk[row][col], row >= col ? acc[rr] : 0.f);
          else sm.lw.Lf[row][col] = row > col ? sm.beta[row] * acc[rr] : 0.f;
        }
      }
    }
    __syncthreads();

    // ---- propagation operands (chunk-start reference) ---------------------
    if (act) {
      const float n0 = sm.gend[c0p], n1 = sm.gend[c0p + 1];
      float bk0[16], bk1[16], kh0[16], kh1[16];
#pragma unroll
      for (int rr = 0; rr < 16; ++rr) {
        const int r = 16 * g + rr;
        const float e0 = fast_exp(gr[rr][0]), e1 = fast_exp(gr[rr][1]);
        const float b = sm.beta[r];
        bk0[rr] = b * kr[rr][0] * e0;
        bk1[rr] = b * kr[rr][1] * e1;
        kh0[rr] = kr[rr][0] * fast_exp(n0 - gr[rr][0]);
        kh1[rr] = kr[rr][1] * fast_exp(n1 - gr[rr][1]);
        put2(&sm.u.prop.qp[r][c0p], qr[rr][0] * e0, qr[rr][1] * e1);
      }
#pragma unroll
      for (int hb = 0; hb < 2; ++hb) {
        put8(&sm.u.prop.bkpT[c0p][16 * g + 8 * hb], bk0 + 8 * hb);
        put8(&sm.u.prop.bkpT[c0p + 1][16 * g + 8 * hb], bk1 + 8 * hb);
        put8(&sm.u.prop.khT[c0p][16 * g + 8 * hb], kh0 + 8 * hb);
        put8(&sm.u.prop.khT[c0p + 1][16 * g + 8 * hb], kh1 + 8 * hb);
      }
    }
    // ---- T = (I + L)^{-1}: diagonal 16x16 blocks by forward substitution --
    if (wave < nb && lane < 16) {
      const int R = wave, j = lane;
      float x[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float s = (r == j) ? 1.f : 0.f;
#pragma unroll
        for (int i = 0; i < r; ++i) s -= sm.lw.Lf[16 * R + r][16 * R + i] * x[i];
        x[r] = s;
      }
#pragma unroll
      for (int r = 0; r < 16; ++r) sm.Tf[16 * R + r][16 * R + j] = x[r];
    }
    __syncthreads();
    // Off-diagonal blocks by distance d: T_RI = -T_RR * sum_{J=I}^{R-1} L_RJ T_JI.
    for (int d = 1; d < nb; ++d) {
      for (int e = tid; e < (nb - d) * 256; e += kThreads) {
        const int I = e >> 8, R = I + d, r = (e >> 4) & 15, jc = e & 15;
        float s = 0.f;
        for (int J = I; J < R; ++J)
#pragma unroll
          for (int x = 0; x < 16; ++x) s += sm.lw.Lf[16 * R + r][16 * J + x] * sm.Tf[16 * J + x][16 * I + jc];
        sm.Tf[16 * I + r][16 * R + jc] = s;  // upper block (I, R): scratch
      }
      __syncthreads();
      for (int e = tid; e < (nb - d) * 256; e += kThreads) {
        const int I = e >> 8, R = I + d, r = (e >> 4) & 15, jc = e & 15;
        float s = 0.f;
#pragma unroll
        for (int x = 0; x < 16; ++x) s -= sm.Tf[16 * R + r][16 * R + x] * sm.Tf[16 * I + x][16 * R + jc];
        sm.Tf[16 * R + r][16 * I + jc] = s;
      }
      __syncthreads();
    }
    for (int e = tid; e < 16 * nb * 16 * nb; e += kThreads) {
      const int r = e / (16 * nb), i = e % (16 * nb);
      put(&sm.Tb[r][i], i <= r ? sm.Tf[r][i] : 0.f);
    }
    __syncthreads();

    // ---- W^T = (beta k g)^T T^T (stored as W row-major); Ut = T (beta V) ---
    for (int tw = wave; tw < NCT * nb; tw += 4) {
      const int ct = tw / nb, R = tw % nb;
      const f32x4 acc = tile_mma(f32x4{0.f, 0.f, 0.f, 0.f}, &sm.u.prop.bkpT[16 * ct][0], LC,
                                 &sm.Tb[16 * R][0], LC, 16 * (R + 1), lane);
      const float x[4] = {acc[0], acc[1], acc[2], acc[3]};
      put4(&sm.lw.w[16 * R + (lane & 15)][16 * ct + 4 * (lane >> 4)], x);
    }
    f32x4 ut[NJT];
    if (wave < nb) {
#pragma unroll
      for (int jt = 0; jt < NJT; ++jt)
        ut[jt] = tile_mma(f32x4{0.f, 0.f, 0.f, 0.f}, &sm.Tb[16 * wave][0], LC, &sm.bvT[16 * jt][0],
                          LC, 16 * (wave + 1), lane);
    }
    __syncthreads();

    // ---- U = Ut - W S  (stored transposed) --------------------------------
    if (wave < nb) {
#pragma unroll
      for (int jt = 0; jt < NJT; ++jt) {
        const f32x4 ws = tile_mma(f32x4{0.f, 0.f, 0.f, 0.f}, &sm.lw.w[16 * wave][0], LDK,
                                  &sm.sT[16 * jt][0], LDK, DK, lane);
        float x[4];
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) x[rr] = ut[jt][rr] - ws[rr];
        put4(&sm.uT[16 * jt + (lane & 15)][16 * wave + 4 * (lane >> 4)], x);
      }
    }
    __syncthreads();

    // ---- O = (q g) S + Aqk U;  S <- diag(g_n) S + (k g_n/g)^T U ------------
    if (wave < nb) {
#pragma unroll
      for (int jt = 0; jt < NJT; ++jt) {
        f32x4 acc = tile_mma(f32x4{0.f, 0.f, 0.f, 0.f}, &sm.u.prop.qp[16 * wave][0], LDK,
                             &sm.sT[16 * jt][0], LDK, DK, lane);
        acc = tile_mma(acc, &sm.aqk[16 * wave][0], LC, &sm.uT[16 * jt][0], LC, 16 * (wave + 1),
                       lane);
        const int j = j0 + 16 * jt + (lane & 15);
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
          const int r = 16 * wave + 4 * (lane >> 4) + rr;
          if (r < n) go[(static_cast<size_t>(t0 + r) * H + h) * dv + j] = from_f32<InT>(acc[rr]);
        }
      }
    }
#pragma unroll
    for (int u = 0; u < NS; ++u) {
      const int s = wave + 4 * u;
      if (s < NST) {
        const int ct = s / NJT, jt = s % NJT;
        const int c0 = 16 * ct + 4 * (lane >> 4);
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) S[u][rr] *= sm.gexp[c0 + rr];
        S[u] = tile_mma(S[u], &sm.u.prop.khT[16 * ct][0], LC, &sm.uT[16 * jt][0], LC, 16 * nb, lane);
      }
    }
    __syncthreads();
    write_sT();

    if (ck < ck_hi && end == lo + p.ck_pos[ck]) {
      store_state(p.page_pool + static_cast<int64_t>(p.ck_slot[ck]) * p.page_elems +
                  static_cast<int64_t>(h) * DK * dv);
      ++ck;
    }
    t0 = end;
  }
  if (p.s_final != nullptr) store_state(p.s_final + state_off);
}

template <int DK, int DVT, typename InT>
hipError_t launch_t(const PrefillArgs& a, const Params& prm) {
  const dim3 grid(static_cast<unsigned>(a.n_chains) * static_cast<unsigned>(a.dv_tiles));
  hipLaunchKernelGGL((prefill_kernel<DK, DVT, InT>), grid, dim3(kThreads), 0, a.stream, prm);
  return hipGetLastError();
}

template <int DK, int DVT>
hipError_t launch_dt(const PrefillArgs& a, const Params& prm) {
  return a.bf16 ? launch_t<DK, DVT, bf16raw>(a, prm) : launch_t<DK, DVT, float>(a, prm);
}

template <int DK>
hipError_t launch_dvt(const PrefillArgs& a, const Params& prm) {
  switch (a.dv / a.dv_tiles) {
    case 16: return launch_dt<DK, 16>(a, prm);
    case 32: return launch_dt<DK, 32>(a, prm);
    case 64: return launch_dt<DK, 64>(a, prm);
  }
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_prefill(const PrefillArgs& a) {
  Params prm;
  prm.q = a.q; prm.k = a.k; prm.v = a.v; prm.a = a.a; prm.beta = a.beta;
  prm.s0 = a.s0; prm.o = a.o; prm.s_final = a.s_final;
  prm.page_pool = a.page_pool; prm.page_elems = a.page_elems;
  prm.chains = a.chains; prm.seqinfo = a.seqinfo; prm.ck_pos = a.ck_pos; prm.ck_slot = a.ck_slot;
  prm.H = a.H; prm.dv = a.dv; prm.chunk = a.chunk; prm.dv_tiles = a.dv_tiles;
  switch (a.dk) {
    case 16: return launch_dvt<16>(a, prm);
    case 32: return launch_dvt<32>(a, prm);
    case 64: return launch_dvt<64>(a, prm);
    case 128: return launch_dvt<128>(a, prm);
  }
  return hipErrorInvalidValue;
}

}  // namespace kda
