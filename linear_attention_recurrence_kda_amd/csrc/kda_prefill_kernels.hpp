// Kernels of the chunked KDA prefill (and of the segment summaries built on
// the same propagation), MFMA on gfx950.  Included by kda_prefill.hip and
// kda_segments.hip; everything here has internal linkage.
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
//   U   = T diag(beta) (V - (k*g) S)          (T applied to the residual at the chunk start)
//   O   = (q*g) S + lower(Qp Km^T) U,         Qp_r = q_r*e^{G_r-G_m}
//   S  <- diag(g_n) S + (k*g_n/g)^T U
// (U = T diag(beta) V - (T diag(beta) (k*g)) S is the WY form; applying T to
// the residual needs no W = T diag(beta) (k*g) at all.)  The reference G_m is
// the cumulative sum through the middle 16-row block boundary, so every
// scaled Gram operand stays within e^{+-|a|*C/2}: finite in bf16/fp32 for
// per-token log-decays a >= -2.5 at a chunk of 64.  Every other scaled
// operand is bounded by 1.
//
// Two kernels.  T diag(beta) and lower(Qp Km^T) depend on the chunk's own
// keys, queries, decays and betas only, never on the state, so the "local"
// kernel computes them for every (chunk, head) at once, with as many
// workgroups as there are such pairs, and stores them in the workspace.  The
// "propagation" kernel then runs each (sequence, head) chain through its
// chunks in order and does only the state-dependent products; its per-chunk
// latency, multiplied by the longest sequence's chunk count, is the critical
// path of the whole prefill.
//
// Propagation mapping.  One workgroup (8 waves) runs one chain over a
// DVT-wide tile of the dv columns (the columns of S are independent in the
// recurrence, so a chain can be split over several workgroups).  The fp32
// state tile lives in MFMA accumulators for the whole sequence; a transposed
// copy in LDS feeds the contractions.  All contractions use
// v_mfma_f32_16x16x32_bf16 with operands staged in LDS: bf16 inputs stage
// bf16 operands; fp32 inputs stage fp32 operands and split each into a bf16
// high and low part, taking three products (hi*hi + hi*lo + lo*hi, about
// 2^-16 relative error) so that fp32 I/O keeps fp32-level accuracy (fp32
// operands double the LDS footprint, so that path caps the chunk at 32 rows).
// The next chunk's inputs, T and A_qk are loaded into registers while the
// current chunk computes.  Workgroups are placed so the tiles of one chain
// share an XCD (and its L2), and chains run longest sequence first.
//
// Local mapping.  T is built per wave without workgroup barriers: wave I
// inverts the 16x16 diagonal blocks it needs by forward substitution (64
// lanes = 4 blocks x 16 columns) and then its block column
// T_RI = -T_RR sum_J L_RJ T_JI with MFMA.
#pragma once

#include "kda_device.hpp"
#include "kda_internal.hpp"

namespace kda {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x2 __attribute__((ext_vector_type(2)));

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
template <int N, typename ST>
__device__ __forceinline__ void putn(ST* p, const float* x) {
  if constexpr (N == 8) put8(p, x);
  else if constexpr (N == 4) put4(p, x);
  else if constexpr (N == 2) put2(p, x[0], x[1]);
  else put(p, x[0]);
}

// Column order of the [*][DK] matrices and the two tiles of records read by
// the column-slab propagation kernel: inside every 32-column group, column
// 16h + 4g + i is stored at 8g + 4h + i, so that lane group g of an MFMA
// operand fragment finds its eight contraction indices {4g..4g+3,
// 16+4g..16+4g+3} in one 16-byte piece.
__device__ __forceinline__ int slab_col(int c) {
  return (c & ~31) | ((c & 12) << 1) | ((c & 16) >> 2) | (c & 3);
}

__device__ __forceinline__ bf16x8 zero8() { return __builtin_bit_cast(bf16x8, i32x4{0, 0, 0, 0}); }
__device__ __forceinline__ f32x4 zero4() { return f32x4{0.f, 0.f, 0.f, 0.f}; }

// Orders this wave's LDS writes before its later LDS reads across lanes.
__device__ __forceinline__ void wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  __builtin_amdgcn_wave_barrier();
}

// acc_t += A_t[0:16, 0:kvalid] * Bt_t[0:16, 0:kvalid]^T for NT independent
// tiles sharing one K loop (16-row slabs in LDS, row strides lda / ldb).
// Lane l ends with rows 4*(l/16)+0..3 of column l%16 of each 16x16 result.
template <int NT>
__device__ __forceinline__ void tiles_mma(f32x4* acc, const __bf16* const* A, int lda,
                                          const __bf16* const* Bt, int ldb, int kvalid, int lane) {
  const int row = lane & 15, kk = (lane >> 4) * 8;
  for (int k0 = 0; k0 < kvalid; k0 += 32) {
    bf16x8 fa[NT], fb[NT];
    const bool ok = k0 + kk < kvalid;
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      fa[t] = ok ? *reinterpret_cast<const bf16x8*>(A[t] + row * lda + kk + k0) : zero8();
      fb[t] = ok ? *reinterpret_cast<const bf16x8*>(Bt[t] + row * ldb + kk + k0) : zero8();
    }
#pragma unroll
    for (int t = 0; t < NT; ++t)
      acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa[t], fb[t], acc[t], 0, 0, 0);
  }
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

template <int NT>
__device__ __forceinline__ void tiles_mma(f32x4* acc, const float* const* A, int lda,
                                          const float* const* Bt, int ldb, int kvalid, int lane) {
  const int row = lane & 15, kk = (lane >> 4) * 8;
  for (int k0 = 0; k0 < kvalid; k0 += 32) {
    const bool ok = k0 + kk < kvalid;
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      bf16x8 ah = zero8(), al = zero8(), bh = zero8(), bl = zero8();
      if (ok) {
        split8(A[t] + row * lda + kk + k0, ah, al);
        split8(Bt[t] + row * ldb + kk + k0, bh, bl);
      }
      acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(al, bh, acc[t], 0, 0, 0);
      acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, bl, acc[t], 0, 0, 0);
      acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, bh, acc[t], 0, 0, 0);
    }
  }
}

// acc_t += A_t * Bt^T for NT tiles that share one B operand: B's fragment is
// read from LDS once per k-step instead of once per tile.
template <int NT>
__device__ __forceinline__ void tiles_mma_sb(f32x4* acc, const __bf16* const* A, int lda,
                                             const __bf16* Bt, int ldb, int kvalid, int lane) {
  const int row = lane & 15, kk = (lane >> 4) * 8;
  for (int k0 = 0; k0 < kvalid; k0 += 32) {
    const bool ok = k0 + kk < kvalid;
    const bf16x8 fb = ok ? *reinterpret_cast<const bf16x8*>(Bt + row * ldb + kk + k0) : zero8();
    bf16x8 fa[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t)
      fa[t] = ok ? *reinterpret_cast<const bf16x8*>(A[t] + row * lda + kk + k0) : zero8();
#pragma unroll
    for (int t = 0; t < NT; ++t)
      acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa[t], fb, acc[t], 0, 0, 0);
  }
}

template <int NT>
__device__ __forceinline__ void tiles_mma_sb(f32x4* acc, const float* const* A, int lda,
                                             const float* Bt, int ldb, int kvalid, int lane) {
  const int row = lane & 15, kk = (lane >> 4) * 8;
  for (int k0 = 0; k0 < kvalid; k0 += 32) {
    const bool ok = k0 + kk < kvalid;
    bf16x8 bh = zero8(), bl = zero8();
    if (ok) split8(Bt + row * ldb + kk + k0, bh, bl);
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      bf16x8 ah = zero8(), al = zero8();
      if (ok) split8(A[t] + row * lda + kk + k0, ah, al);
      acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(al, bh, acc[t], 0, 0, 0);
      acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, bl, acc[t], 0, 0, 0);
      acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, bh, acc[t], 0, 0, 0);
    }
  }
}

// fp32 operands rounded once to bf16.
__device__ __forceinline__ void round8(const float* p, bf16x8& hi) {
  const float4 x0 = *reinterpret_cast<const float4*>(p);
  const float4 x1 = *reinterpret_cast<const float4*>(p + 4);
  const float x[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
#pragma unroll
  for (int i = 0; i < 8; ++i) hi[i] = static_cast<__bf16>(x[i]);
}

template <typename ST>
__device__ __forceinline__ f32x4 tile_mma(f32x4 acc, const ST* A, int lda, const ST* Bt, int ldb,
                                          int kvalid, int lane) {
  tiles_mma<1>(&acc, &A, lda, &Bt, ldb, kvalid, lane);
  return acc;
}

// A fp32 (LDS) times B stored as bf16: A rounded once to bf16.
__device__ __forceinline__ f32x4 tile_mma_fb(f32x4 acc, const float* A, int lda, const __bf16* Bt,
                                             int ldb, int kvalid, int lane) {
  const int row = lane & 15, kk = (lane >> 4) * 8;
  for (int k0 = 0; k0 < kvalid; k0 += 32) {
    bf16x8 ah = zero8(), bh = zero8();
    if (k0 + kk < kvalid) {
      round8(A + row * lda + kk + k0, ah);
      bh = *reinterpret_cast<const bf16x8*>(Bt + row * ldb + kk + k0);
    }
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, bh, acc, 0, 0, 0);
  }
  return acc;
}
// A fp32 times B fp32: hi/lo split (fp32 inputs).
__device__ __forceinline__ f32x4 tile_mma_fb(f32x4 acc, const float* A, int lda, const float* Bt,
                                             int ldb, int kvalid, int lane) {
  return tile_mma<float>(acc, A, lda, Bt, ldb, kvalid, lane);
}

struct LocalParams {
  const void *q, *k, *a, *beta;  // a, beta: gate logits when the gate is fused
  float g_min;
  int perm;                // record columns in the column-slab order (slab_col)
  const int32_t* chunks;   // [n_chunks][2] = (first token, rows)
  void* tq;                // [n_chunks][H] unit records (UnitLayout)
  int H, ld;
  int32_t* wsflag;         // raised (with *err_flag when not null) on a decay outside [a_lo, 0]
  int32_t* err_flag;
  float a_lo;
};

struct PropParams {
  const void* v;
  const void* tq;            // unit records (UnitLayout)
  const float* s0;
  void* o;
  float* s_final;
  float* page_pool;
  int64_t page_elems;
  const int32_t* chains;   // [n_chains][2] = (sequence or -1, head)
  const int32_t* seqinfo;  // [n_seqs][6]  = (tok_lo, tok_hi, ck_lo, ck_hi, chunk_lo, chunk_hi)
  const int32_t* ck_pos;   // [n_ckpt] token counts from the sequence start
  const int32_t* ck_slot;  // [n_ckpt]
  const int32_t* chunks;   // [n_chunks][2]
  const int32_t* wgs;      // per-workgroup (chain, width, tile) of the mixed-width slab launch
  const int32_t* wsflag;   // nonzero: a decay was out of range, the prefill writes nothing
  int H, dv, ld, dv_tiles;
};

template <typename ST>
struct TScratch {  // one wave's workspace for its block column of T
  static constexpr int MAXC = Op<ST>::MAXC, PAD = Op<ST>::PAD;
  ST diag[MAXC / 16][16][16 + PAD];  // T_RR, row-major, for R = I .. nb-1
  ST colT[16][MAXC + PAD];    // colT[i][j] = T[j][16 I + i]
  ST PT[16][16 + PAD];        // P^T of the current step
};

template <int DK, typename ST, int NG>
struct LocalSmem {
  static constexpr int MAXC = Op<ST>::MAXC;
  static constexpr int LDK = DK + Op<ST>::PAD;   // row length of [*][DK] buffers
  static constexpr int LC = MAXC + Op<ST>::PAD;  // row length of [*][chunk] buffers
  static constexpr int LF = MAXC + 4;            // row length of fp32 [chunk][chunk]
  __attribute__((aligned(16))) float beta[MAXC];
  float tot[NG][DK];        // per-row-group sums of a
  float Lf[MAXC][LF];       // diag(beta) strict_lower(A_kk), fp32
  union __attribute__((aligned(16))) {
    struct {  // scaled Gram operands (mid-chunk reference)
      ST kpm[MAXC][LDK], qpm[MAXC][LDK], kmm[MAXC][LDK];
    } gram;
    struct {  // after the Gram products
      TScratch<ST> ts[MAXC / 16];  // block columns of T
      ST tb[MAXC][LC];             // T diag(beta)
      ST aqk[MAXC][LC];            // lower(Qp Km^T)
    } out;
  } u;
};

template <int DK, int DVT, typename ST>
struct PropSmem {
  static constexpr int MAXC = Op<ST>::MAXC;
  static constexpr int LDK = DK + Op<ST>::PAD;
  static constexpr int LC = MAXC + Op<ST>::PAD;
  static constexpr int LV = DVT + Op<ST>::PAD;
  float gexp[DK];           // g_n
  ST tb[MAXC][LC];          // T diag(beta)
  ST aqk[MAXC][LC];         // lower(Qp Km^T)
  ST sT[DVT][LDK];          // S^T
  union {                   // v is dead once Z is formed; U^T follows it
    ST v[MAXC][LV];         // v, this workgroup's columns, row-major
    ST uT[DVT][LC];         // U^T
  } buf;
  ST zT[DVT][LC];           // Z^T = (V - (k g) S)^T
  // This chunk's outputs, row-major.  They are written to HBM only after the
  // next chunk's first barrier and loads, so that a later wait on those loads
  // (vector-memory counters also count stores) never waits on fresh stores.
  __attribute__((aligned(16))) ST o[MAXC][LV];
  ST kp[MAXC][LDK];         // k * g
  ST qp[MAXC][LDK];         // q * g
  ST khT[DK][LC];           // (k * g_n / g)^T
};

template <typename InT>
struct Traits;
template <>
struct Traits<bf16raw> {
  using ST = __bf16;
  using Pair = uint32_t;  // two consecutive bf16 values
  static __device__ __forceinline__ Pair load(const char* p) {
    return *reinterpret_cast<const uint32_t*>(p);
  }
  static __device__ __forceinline__ float2 unpack(Pair x) {
    return make_float2(__uint_as_float(x << 16), __uint_as_float(x & 0xffff0000u));
  }
  static __device__ __forceinline__ Pair zero() { return 0u; }
};
template <>
struct Traits<float> {
  using ST = float;
  using Pair = float2;
  static __device__ __forceinline__ Pair load(const char* p) {
    return *reinterpret_cast<const float2*>(p);
  }
  static __device__ __forceinline__ float2 unpack(Pair x) { return x; }
  static __device__ __forceinline__ Pair zero() { return make_float2(0.f, 0.f); }
};

// Thread and tile mappings of one workgroup of NW waves.
template <int DK, int DVT, typename ST, int NW>
struct Shape {
  static constexpr int NT = 64 * NW;                  // threads
  static constexpr int MAXC = Op<ST>::MAXC;
  static constexpr int HK = DK / 2;                   // channel pairs
  static constexpr int RPG = (MAXC * HK / NT) > 0 ? MAXC * HK / NT : 1;  // rows per prep thread
  static constexpr int NG = MAXC / RPG;               // prep row groups
  static constexpr int VP = DVT / 2;                  // column pairs of the tile
  static constexpr int RV = (MAXC * VP / NT) > 0 ? MAXC * VP / NT : 1;   // rows per v thread
  static constexpr int NCT = DK / 16, NJT = DVT / 16;
  static constexpr int NST = NCT * NJT;               // state tiles
  static constexpr int NS = (NST + NW - 1) / NW;      // state tiles per wave
  static constexpr int NUT = (4 * NJT + NW - 1) / NW; // (row block, column tile) pairs per wave
  static constexpr int NTRI = (MAXC / 16) * (MAXC / 16 + 1) / 2;  // lower block tiles
  static constexpr int NGT = (NTRI + NW - 1) / NW;    // Gram tile pairs per wave
  static_assert(RPG <= 8 && RV <= 8 && 16 % RPG == 0, "mapping");
};

// ---------------------------------------------------------------------------
// Local kernel: T diag(beta) and lower(A_qk) of one (chunk, head).

// GATE: a and beta arrive as logits z_a, z_b and the gate is applied on load,
// a = g_min * sigmoid(z_a), beta = sigmoid(z_b) ("Serve 模块交互式演示" page,
// §1.3), in fp32 (the fused gate of the "Kimi Linear 的 KDA 缓存" page's vLLM
// path, "chunk_kda_with_fused_gate").
template <int DK, typename InT, int NW, bool GATE>
__global__ __launch_bounds__(64 * NW, 2) void local_kernel(LocalParams p) {
  using TR = Traits<InT>;
  using ST = typename TR::ST;
  using Pair = typename TR::Pair;
  using SH = Shape<DK, 16, ST, NW>;
  using SM = LocalSmem<DK, ST, SH::NG>;
  constexpr int NT = SH::NT, MAXC = SH::MAXC, HK = SH::HK, RPG = SH::RPG, NG = SH::NG, NGT = SH::NGT;
  constexpr int LDK = SM::LDK, LF = SM::LF;
  constexpr uint32_t ES = sizeof(InT);
  __shared__ __attribute__((aligned(16))) SM sm;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int H = p.H;
  const int unit = blockIdx.x, c = unit / H, h = unit - c * H;
  const int t0 = p.chunks[2 * c], n = p.chunks[2 * c + 1];
  const int nb = (n + 15) >> 4, ngc = 16 * nb / RPG;
  const int cp = tid % HK, g = tid / HK;
  const int c0p = 2 * cp, r0 = g * RPG;
  const bool act = g < ngc;
  const size_t row0 = static_cast<size_t>(t0) * H + h;
  const InT* __restrict__ gb = static_cast<const InT*>(p.beta);

  // ---- loads; per-group cumulative sums of a ------------------------------
  Pair kr[RPG], qr[RPG];
  float gr[RPG][2];
  bool bad = false;  // a log-decay of this thread outside [a_lo, 0]
  if (act) {
    const uint32_t rsk = static_cast<uint32_t>(H) * DK * ES;
    const uint32_t ok0 = r0 * rsk + c0p * ES, okl = (n - 1) * rsk + c0p * ES;
    const char* bk = reinterpret_cast<const char*>(static_cast<const InT*>(p.k) + row0 * DK);
    const char* bq = reinterpret_cast<const char*>(static_cast<const InT*>(p.q) + row0 * DK);
    const char* ba = reinterpret_cast<const char*>(static_cast<const InT*>(p.a) + row0 * DK);
    Pair ar[RPG];
#pragma unroll
    for (int rr = 0; rr < RPG; ++rr) {
      const uint32_t off = min(ok0 + rr * rsk, okl);
      kr[rr] = TR::load(bk + off);
      qr[rr] = TR::load(bq + off);
      ar[rr] = TR::load(ba + off);
    }
    float run0 = 0.f, run1 = 0.f;
#pragma unroll
    for (int rr = 0; rr < RPG; ++rr) {
      const bool valid = r0 + rr < n;
      if (!valid) { kr[rr] = TR::zero(); qr[rr] = TR::zero(); }
      float2 aa = TR::unpack(valid ? ar[rr] : TR::zero());
      if constexpr (GATE) {
        aa.x = valid ? p.g_min * fast_rcp(1.f + fast_exp(-aa.x)) : 0.f;
        aa.y = valid ? p.g_min * fast_rcp(1.f + fast_exp(-aa.y)) : 0.f;
      }
      // (a NaN fails both comparisons)
      bad |= !(aa.x >= p.a_lo && aa.x <= 0.f && aa.y >= p.a_lo && aa.y <= 0.f);
      run0 += aa.x; run1 += aa.y;
      gr[rr][0] = run0; gr[rr][1] = run1;
    }
    sm.tot[g][c0p] = run0;
    sm.tot[g][c0p + 1] = run1;
  }
  if (tid < 16 * nb) {
    float b = tid < n ? to_f32(gb[row0 + static_cast<size_t>(tid) * H]) : 0.f;
    if constexpr (GATE) b = tid < n ? fast_rcp(1.f + fast_exp(-b)) : 0.f;
    sm.beta[tid] = b;
  }
  // One store per wave that saw a decay out of range.
  if (__builtin_amdgcn_ballot_w64(bad) != 0 && lane == 0) {
    *p.wsflag = 1;
    if (p.err_flag != nullptr) *p.err_flag = 1;
  }
  __syncthreads();

  // ---- scaled Gram operands (reference: end of 16-row block nb/2 - 1) into
  // LDS; the chunk-start operands k*g, q*g, (k*g_n/g)^T and g_n into this
  // unit's record for the propagation kernel ---------------------------------
  const UnitLayout lay(p.ld, DK, static_cast<int>(ES));
  char* rec = static_cast<char*>(p.tq) + static_cast<size_t>(unit) * lay.bytes;
  if (act) {
    float pre0 = 0.f, pre1 = 0.f, rf0 = 0.f, rf1 = 0.f, ge0 = 0.f, ge1 = 0.f;
    const int gref = 16 * (nb >> 1) / RPG;
    // All group sums are read at once (one LDS latency, not one per group).
#pragma unroll
    for (int gg = 0; gg < NG; ++gg) {
      const float2 t = *reinterpret_cast<const float2*>(&sm.tot[gg][c0p]);
      if (gg < g) { pre0 += t.x; pre1 += t.y; }
      if (gg < gref) { rf0 += t.x; rf1 += t.y; }
      if (gg < ngc) { ge0 += t.x; ge1 += t.y; }
    }
    // e^{G} = e^{G - G_m} e^{G_m},  e^{G_n - G} = e^{G_m - G} e^{G_n - G_m}.
    const float em0 = fast_exp(rf0), em1 = fast_exp(rf1);
    const float en0 = fast_exp(ge0 - rf0), en1 = fast_exp(ge1 - rf1);
    ST* okp = reinterpret_cast<ST*>(rec + lay.kp);
    ST* oqp = reinterpret_cast<ST*>(rec + lay.qp);
    ST* okh = reinterpret_cast<ST*>(rec + lay.kh);
    if (g == 0) {
      float* ogx = reinterpret_cast<float*>(rec + lay.gexp);
      ogx[c0p] = fast_exp(ge0);
      ogx[c0p + 1] = fast_exp(ge1);
    }
    const int kc = p.perm ? slab_col(c0p) : c0p;  // c0p, c0p + 1 stay adjacent
    float kh0[RPG], kh1[RPG];
#pragma unroll
    for (int rr = 0; rr < RPG; ++rr) {
      const int r = r0 + rr;
      const float d0 = gr[rr][0] + pre0 - rf0, d1 = gr[rr][1] + pre1 - rf1;
      const float up0 = fast_exp(d0), up1 = fast_exp(d1);
      const float dn0 = fast_exp(-d0), dn1 = fast_exp(-d1);
      const float2 kk = TR::unpack(kr[rr]), qq = TR::unpack(qr[rr]);
      put2(&sm.u.gram.kpm[r][c0p], kk.x * up0, kk.y * up1);
      put2(&sm.u.gram.qpm[r][c0p], qq.x * up0, qq.y * up1);
      put2(&sm.u.gram.kmm[r][c0p], kk.x * dn0, kk.y * dn1);
      const float e0 = up0 * em0, e1 = up1 * em1;
      put2(okp + r * DK + kc, kk.x * e0, kk.y * e1);
      put2(oqp + r * DK + kc, qq.x * e0, qq.y * e1);
      kh0[rr] = kk.x * (dn0 * en0);
      kh1[rr] = kk.y * (dn1 * en1);
    }
    putn<RPG>(okh + c0p * p.ld + r0, kh0);
    putn<RPG>(okh + (c0p + 1) * p.ld + r0, kh1);
  } else if (r0 < p.ld) {
    // Rows past the chunk's last 16-row block are written as zeros, so a
    // reader may run its products over the whole chunk.
    ST* okp = reinterpret_cast<ST*>(rec + lay.kp);
    ST* oqp = reinterpret_cast<ST*>(rec + lay.qp);
    ST* okh = reinterpret_cast<ST*>(rec + lay.kh);
    const float zr[RPG] = {};
#pragma unroll
    for (int rr = 0; rr < RPG; ++rr) {
      put2(okp + (r0 + rr) * DK + c0p, 0.f, 0.f);  // a zero row is a zero row in any order
      put2(oqp + (r0 + rr) * DK + c0p, 0.f, 0.f);
    }
    putn<RPG>(okh + c0p * p.ld + r0, zr);
    putn<RPG>(okh + (c0p + 1) * p.ld + r0, zr);
  }
  __syncthreads();

  // ---- Gram products: L = diag(beta) strict_lower(A_kk) into LDS; A_qk kept
  // in registers until the operands are dead.  Tile x of the lower triangle
  // pairs the A_kk and A_qk products that share the Km block.
  const int ntri = nb * (nb + 1) / 2;
  f32x4 aq[NGT];
  int aR[NGT], aI[NGT];
#pragma unroll
  for (int m = 0; m < NGT; ++m) {
    const int x0 = wave + NW * m;
    aq[m] = zero4();
    aR[m] = 0; aI[m] = 0;
    if (x0 < ntri) {
      int x = x0, R = 0;
      while (x > R) { x -= R + 1; ++R; }
      aR[m] = R; aI[m] = x;
      f32x4 acc[2] = {zero4(), zero4()};
      const ST* A[2] = {&sm.u.gram.kpm[16 * R][0], &sm.u.gram.qpm[16 * R][0]};
      tiles_mma_sb<2>(acc, A, LDK, &sm.u.gram.kmm[16 * x][0], LDK, DK, lane);
      aq[m] = acc[1];
      const int col = 16 * x + (lane & 15), row0t = 16 * R + 4 * (lane >> 4);
      const float4 bt = *reinterpret_cast<const float4*>(&sm.beta[row0t]);
      const float b4[4] = {bt.x, bt.y, bt.z, bt.w};
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) sm.Lf[row0t + rr][col] = row0t + rr > col ? b4[rr] * acc[0][rr] : 0.f;
    }
  }
  __syncthreads();

#pragma unroll
  for (int m = 0; m < NGT; ++m) {
    if (wave + NW * m < ntri) {
      const int col = 16 * aI[m] + (lane & 15), row0t = 16 * aR[m] + 4 * (lane >> 4);
      const int cs = p.perm ? slab_col(col) : col;  // the tiles are kept in the record's column order
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) put(&sm.u.out.aqk[row0t + rr][cs], row0t + rr >= col ? aq[m][rr] : 0.f);
    }
  }
  // ---- T = (I + L)^{-1}, one block column per wave; stored as T diag(beta)
  if (wave < nb) {
    const int I = wave;
    TScratch<ST>& ts = sm.u.out.ts[wave];
    constexpr int LD = 16 + Op<ST>::PAD, LCT = MAXC + Op<ST>::PAD;
    const float bcol = sm.beta[16 * I + (lane & 15)];
    // Diagonal inverses T_RR for R = I .. nb-1: lane = 16*(R-I) + column.
    {
      const int blk = lane >> 4, R = I + blk, j = lane & 15;
      if (R < nb) {
        // Right-looking: once x[i] is final, fold it into every later row.
        // Column i+1 of L is loaded while column i is applied; the
        // scheduling barrier keeps at most two columns in registers.
        float x[16], lc[16], ln[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) x[r] = (r == j) ? 1.f : 0.f;
#pragma unroll
        for (int r = 1; r < 16; ++r) lc[r] = sm.Lf[16 * R + r][16 * R];
#pragma unroll
        for (int i = 0; i < 15; ++i) {
          if (i + 1 < 15) {
#pragma unroll
            for (int r = i + 2; r < 16; ++r) ln[r] = sm.Lf[16 * R + r][16 * R + i + 1];
          }
#pragma unroll
          for (int r = i + 1; r < 16; ++r) x[r] -= lc[r] * x[i];
          __builtin_amdgcn_sched_barrier(0);
#pragma unroll
          for (int r = i + 2; r < 16; ++r) lc[r] = ln[r];
        }
#pragma unroll
        for (int r = 0; r < 16; ++r) put(&ts.diag[blk][r][j], x[r]);
        if (blk == 0) {
#pragma unroll
          for (int r = 0; r < 16; r += 4) put4(&ts.colT[j][16 * I + r], x + r);
          const int cs = p.perm ? slab_col(16 * I + j) : 16 * I + j;
#pragma unroll
          for (int r = 0; r < 16; ++r) put(&sm.u.out.tb[16 * I + r][cs], x[r] * bcol);
        }
      }
    }
    wave_sync();
    // Block column: T_RI = -T_RR * sum_{J=I}^{R-1} L_RJ T_JI.
    const int tcol = p.perm ? slab_col(16 * I + (lane & 15)) : 16 * I + (lane & 15);
    for (int R = I + 1; R < nb; ++R) {
      const f32x4 P = tile_mma_fb(zero4(), &sm.Lf[16 * R][16 * I], LF, &ts.colT[0][16 * I], LCT,
                                  16 * (R - I), lane);
      const float pv[4] = {P[0], P[1], P[2], P[3]};
      put4(&ts.PT[lane & 15][4 * (lane >> 4)], pv);
      wave_sync();
      const f32x4 Tn = tile_mma<ST>(zero4(), &ts.diag[R - I][0][0], LD, &ts.PT[0][0], LD, 16, lane);
      const float tv[4] = {-Tn[0], -Tn[1], -Tn[2], -Tn[3]};
      put4(&ts.colT[lane & 15][16 * R + 4 * (lane >> 4)], tv);
#pragma unroll
      for (int rr = 0; rr < 4; ++rr)
        put(&sm.u.out.tb[16 * R + 4 * (lane >> 4) + rr][tcol], tv[rr] * bcol);
      wave_sync();
    }
  }
  __syncthreads();

  // ---- both tiles to the workspace, 16 bytes per store; entries right of
  // the diagonal block and rows past the chunk's last 16-row block are written
  // as zeros, so a reader may run its products over any range ---------------
  {
    const int ld = p.ld, ppr = ld * static_cast<int>(ES) / 16;  // 16-byte pieces per row
    constexpr int EP = 16 / static_cast<int>(ES);                // elements per piece
    char* dst = rec;
    const int npc = ld * ppr;
    // Entry (r, c) is built in LDS when r < 16 nb and c is in a block on or
    // left of the diagonal; the rest is zero.
    auto built = [&](int r, int c) { return r < 16 * nb && c < 16 * (r / 16 + 1); };
    for (int x = tid; x < 2 * npc; x += NT) {
      const int m = x >= npc, y = x - m * npc, r = y / ppr, cc = (y - r * ppr) * EP;
      const ST* row = m ? &sm.u.out.aqk[r][0] : &sm.u.out.tb[r][0];
      char* drow = dst + (static_cast<size_t>(m) * ld * ld + r * ld) * ES;
      if constexpr (ES == 2) {
        if (p.perm) {
          // The tiles are in LDS in slab_col order: piece cc = 32s + 8g holds
          // columns 32s + 4g .. +3 and 32s + 16 + 4g .. +3.  The upper-right
          // 32x32 quadrant is left unwritten (the slab kernel never reads it).
          if (r < 32 && cc >= 32) continue;
          const int c1 = (cc & ~31) + ((cc & 31) >> 1), c2 = c1 + 16;
          i32x4 val = *reinterpret_cast<const i32x4*>(row + cc);
          if (!built(r, c1)) val[0] = val[1] = 0;
          if (!built(r, c2)) val[2] = val[3] = 0;
          *reinterpret_cast<i32x4*>(drow + cc * ES) = val;
          continue;
        }
      }
      const i32x4 val = built(r, cc) ? *reinterpret_cast<const i32x4*>(row + cc) : i32x4{0, 0, 0, 0};
      *reinterpret_cast<i32x4*>(drow + cc * ES) = val;
    }
  }
}

// ---------------------------------------------------------------------------
// Propagation kernel: one (sequence, head, dv tile) chain through its chunks.

// The propagation kernel's per-chunk inputs, loaded into registers one chunk
// ahead as 16-byte pieces: the unit record's scaled operands and tiles (see
// UnitLayout) and this workgroup's columns of v.
template <int NPK, int NPV>
struct Pieces {
  i32x4 kp[NPK], qp[NPK], kh[NPK];  // k*g, q*g rows; (k*g_n/g)^T rows
  i32x4 t, a, g;                     // T diag(beta), lower(A_qk), g_n
  i32x4 v[NPV];
};

// One chunk: copy its pieces into LDS; Z = V - (k g) S and QS = (q g) S;
// U = T diag(beta) Z; O = QS + A_qk U and S <- diag(g_n) S + (k g_n/g)^T U;
// then S^T, O and checkpoint stores (four workgroup barriers).
// MODE 0: prefill.  MODE 1: a segment's B, the end state from the start state
// s0 (zero when s0 is null), without outputs.  MODE 2: a segment's A, the end
// state from the identity (dv = dk) with v taken as zero, without outputs.
template <int DK, int DVT, typename InT, int NW, int MODE>
__global__ __launch_bounds__(64 * NW, 1) void prop_kernel(PropParams p) {
  using TR = Traits<InT>;
  using ST = typename TR::ST;
  using SH = Shape<DK, DVT, ST, NW>;
  using SM = PropSmem<DK, DVT, ST>;
  constexpr int NT = SH::NT, MAXC = SH::MAXC, NJT = SH::NJT;
  constexpr int NST = SH::NST, NS = SH::NS, NUT = SH::NUT;
  constexpr int LDK = SM::LDK, LC = SM::LC;
  constexpr uint32_t ES = sizeof(InT);
  constexpr int EP = 16 / static_cast<int>(ES);        // elements per 16-byte piece
  constexpr int PKR = DK / EP;                         // pieces per [*][DK] row
  constexpr int PVR = DVT / EP;                        // pieces per v row of the tile
  constexpr int NPK = (MAXC * PKR + NT - 1) / NT;      // k*g pieces per thread
  constexpr int NPV = (MAXC * PVR + NT - 1) / NT;      // v pieces per thread
  __shared__ __attribute__((aligned(16))) SM sm;

  const int tid = threadIdx.x, lane = tid & 63;
  // Wave index in a scalar register, so per-wave tile loops branch on scalars.
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int H = p.H, dv = p.dv, ld = p.ld;

  // Workgroup -> (chain, dv tile): the tiles of a chain land on one XCD.
  const int bid = blockIdx.x, xcd = bid & 7, local = bid >> 3;
  const int chain = 8 * (local / p.dv_tiles) + xcd, tile = local % p.dv_tiles;
  const int seq = p.chains[2 * chain], h = p.chains[2 * chain + 1];
  if (seq < 0) return;
  if (MODE == 0 && *p.wsflag != 0) return;  // a decay out of range: write nothing
  const int* si = p.seqinfo + 6 * seq;
  const int lo = si[0], ck_lo = si[2], ck_hi = si[3], c_lo = si[4], c_hi = si[5];
  const int j0 = tile * DVT;
  const int64_t hkv = static_cast<int64_t>(H) * DK * dv;
  const size_t state_off = (static_cast<size_t>(seq) * H + h) * DK * dv;
  const InT* __restrict__ gv = static_cast<const InT*>(p.v);
  InT* __restrict__ go = static_cast<InT*>(p.o);
  const UnitLayout lay(ld, DK, static_cast<int>(ES));

  // State tile: accumulator tile s = wave + NW*u covers rows 16*(s/NJT) and
  // columns j0 + 16*(s%NJT).
  f32x4 S[NS];
#pragma unroll
  for (int u = 0; u < NS; ++u) {
    const int s = wave + NW * u;
    S[u] = zero4();
    if constexpr (MODE == 2) {
      const int c0 = 16 * (s / NJT) + 4 * (lane >> 4), j = j0 + 16 * (s % NJT) + (lane & 15);
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) S[u][rr] = c0 + rr == j ? 1.f : 0.f;
    } else if (s < NST && p.s0 != nullptr) {
      const int c0 = 16 * (s / NJT) + 4 * (lane >> 4), j = j0 + 16 * (s % NJT) + (lane & 15);
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) S[u][rr] = p.s0[state_off + static_cast<size_t>(c0 + rr) * dv + j];
    }
  }
  auto write_sT = [&]() {
#pragma unroll
    for (int u = 0; u < NS; ++u) {
      const int s = wave + NW * u;
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
      const int s = wave + NW * u;
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
      for (int64_t e = hkv + tid; e < p.page_elems; e += NT) pg[e] = 0.f;
    }
  }

  // Piece mappings (loop-invariant).  T / A_qk / (k g_n/g)^T rows are ld
  // elements long (ppr pieces); k*g / q*g rows DK elements; v rows DVT.
  // Every load, LDS copy and output store below is unconditional: a thread
  // past the end of a piece list takes the last piece again (the same data
  // to the same place), and v / output rows past n repeat row n-1.  With no
  // per-thread branches around them, the compiler can count exactly which
  // memory operations are still in flight and wait only for the ones needed
  // (a conditional load or store would make it wait for all of them,
  // including the previous chunk's output stores).
  const int ppr = ld / EP;
  const int tpc = min(tid, ld * ppr - 1);
  const int tr = tpc / ppr, tc = (tpc - tr * ppr) * EP;  // T, A_qk piece
  const int gpc = min(tid, DK / 4 - 1);                   // g_n piece
  const uint32_t rsv = static_cast<uint32_t>(H) * dv * ES;  // v row stride, bytes

  // Issue all loads of chunk c (first token t, n rows) into registers.
  Pieces<NPK, NPV> pc;
  auto issue = [&](int c, int t, int n) {
    const char* rc = static_cast<const char*>(p.tq) + (static_cast<size_t>(c) * H + h) * lay.bytes;
    pc.t = *reinterpret_cast<const i32x4*>(rc + (tr * ld + tc) * ES);
    pc.a = *reinterpret_cast<const i32x4*>(rc + lay.aqk + (tr * ld + tc) * ES);
    pc.g = *reinterpret_cast<const i32x4*>(rc + lay.gexp + gpc * 16);
    // v rows past n repeat row n-1: T diag(beta) has zero columns there, so
    // they never reach U.
    if constexpr (MODE != 2) {
      const char* bv = reinterpret_cast<const char*>(gv + (static_cast<size_t>(t) * H + h) * dv + j0);
#pragma unroll
      for (int i = 0; i < NPV; ++i) {
        const int x = min(tid + NT * i, MAXC * PVR - 1), r = x / PVR, cc = (x - r * PVR) * EP;
        pc.v[i] = *reinterpret_cast<const i32x4*>(bv + min(r, n - 1) * rsv + cc * ES);
      }
    }
#pragma unroll
    for (int i = 0; i < NPK; ++i) {
      const int xk = min(tid + NT * i, ld * PKR - 1), xh = min(tid + NT * i, DK * ppr - 1);
      pc.kp[i] = *reinterpret_cast<const i32x4*>(rc + lay.kp + xk * 16);
      pc.qp[i] = *reinterpret_cast<const i32x4*>(rc + lay.qp + xk * 16);
      pc.kh[i] = *reinterpret_cast<const i32x4*>(rc + lay.kh + xh * 16);
    }
  };
  // Output rows of a chunk (first token t, n rows) from sm.o, 16 bytes per
  // thread and store.
  auto store_o = [&](int t, int n_) {
    char* bo = reinterpret_cast<char*>(go + (static_cast<size_t>(t) * H + h) * dv + j0);
#pragma unroll
    for (int i = 0; i < NPV; ++i) {
      const int x = min(tid + NT * i, n_ * PVR - 1), r = x / PVR, cc = (x - r * PVR) * EP;
      *reinterpret_cast<i32x4*>(bo + r * rsv + cc * ES) = *reinterpret_cast<const i32x4*>(&sm.o[r][cc]);
    }
  };

  int ck = ck_lo;
  int t0 = 0, n = 0;
  if (c_lo < c_hi) {
    t0 = __builtin_amdgcn_readfirstlane(p.chunks[2 * c_lo]);
    n = __builtin_amdgcn_readfirstlane(p.chunks[2 * c_lo + 1]);
    issue(c_lo, t0, n);
  }
  // The previous chunk, whose outputs are still in sm.o.  Before the first
  // chunk it is the first chunk itself: its rows then receive whatever sm.o
  // holds and are rewritten by the same threads with the real outputs one
  // chunk later (one thread's stores to one address stay in order).
  int pt0 = t0, pn = n;

  static_assert(NW % NJT == 0, "pair mapping");
  const int jtw = wave % NJT;  // the column tile shared by this wave's tiles
  for (int c = c_lo; c < c_hi; ++c) {
    // The next chunk, or this one again at the end of the chain (the loads
    // stay unconditional).
    const int cn = c + 1 < c_hi ? c + 1 : c;
    const int tn = __builtin_amdgcn_readfirstlane(p.chunks[2 * cn]);
    const int nn = __builtin_amdgcn_readfirstlane(p.chunks[2 * cn + 1]);
    const int nb = (n + 15) >> 4;
    const bool is_ck = ck < ck_hi && t0 + n == lo + p.ck_pos[ck];

    // ---- pieces into LDS ----------------------------------------------------
    *reinterpret_cast<i32x4*>(&sm.tb[tr][tc]) = pc.t;
    *reinterpret_cast<i32x4*>(&sm.aqk[tr][tc]) = pc.a;
    *reinterpret_cast<i32x4*>(&sm.gexp[4 * gpc]) = pc.g;
    if constexpr (MODE != 2) {
#pragma unroll
      for (int i = 0; i < NPV; ++i) {
        const int x = min(tid + NT * i, MAXC * PVR - 1), r = x / PVR, cc = (x - r * PVR) * EP;
        *reinterpret_cast<i32x4*>(&sm.buf.v[r][cc]) = pc.v[i];
      }
    }
#pragma unroll
    for (int i = 0; i < NPK; ++i) {
      const int xk = min(tid + NT * i, ld * PKR - 1), xh = min(tid + NT * i, DK * ppr - 1);
      const int rk = xk / PKR, ck_ = (xk - rk * PKR) * EP;
      const int rh = xh / ppr, ch = (xh - rh * ppr) * EP;
      *reinterpret_cast<i32x4*>(&sm.kp[rk][ck_]) = pc.kp[i];
      *reinterpret_cast<i32x4*>(&sm.qp[rk][ck_]) = pc.qp[i];
      *reinterpret_cast<i32x4*>(&sm.khT[rh][ch]) = pc.kh[i];
    }
    __syncthreads();
    // The next chunk's loads, then the previous chunk's output stores.
    issue(cn, tn, nn);
    if constexpr (MODE == 0) store_o(pt0, pn);

    // ---- Z = V - (k g) S (stored transposed); QS = (q g) S ----------------
    // The pairs of a wave share the column tile jtw (NJT divides NW), so all
    // their products read one B operand, S^T's tile jtw.
    const bool all_pairs = wave + NW * (NUT - 1) < nb * NJT;  // wave-uniform
    const int kmax = 16 * min(nb, (wave + NW * (NUT - 1)) / NJT + 1);  // row extent of the last pair
    // Products per pair: (k g) S, and (q g) S when outputs are formed.
    constexpr int NA = MODE == 0 ? 2 : 1;
    auto zval = [&](int i, int jl, float ks) {  // Z = V - (k g) S (V = 0 for MODE 2)
      if constexpr (MODE == 2) return -ks;
      else return static_cast<float>(sm.buf.v[i][jl]) - ks;
    };
    f32x4 qs[NUT];
    if (all_pairs) {
      f32x4 acc[NA * NUT];
      const ST* A[NA * NUT];
#pragma unroll
      for (int m = 0; m < NUT; ++m) {
        const int R = (wave + NW * m) / NJT;
        acc[NA * m] = zero4();
        A[NA * m] = &sm.kp[16 * R][0];
        if constexpr (NA == 2) {
          acc[2 * m + 1] = zero4();
          A[2 * m + 1] = &sm.qp[16 * R][0];
        }
      }
      tiles_mma_sb<NA * NUT>(acc, A, LDK, &sm.sT[16 * jtw][0], LDK, DK, lane);
#pragma unroll
      for (int m = 0; m < NUT; ++m) {
        const int R = (wave + NW * m) / NJT;
        if constexpr (NA == 2) qs[m] = acc[2 * m + 1];
        const int jl = 16 * jtw + (lane & 15), i0 = 16 * R + 4 * (lane >> 4);
        float z[4];
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) z[rr] = zval(i0 + rr, jl, acc[NA * m][rr]);
        put4(&sm.zT[jl][i0], z);
      }
    } else {
#pragma unroll
      for (int m = 0; m < NUT; ++m) {
        const int x = wave + NW * m;
        qs[m] = zero4();
        if (x < nb * NJT) {
          const int R = x / NJT;
          f32x4 acc[NA];
          const ST* A[NA];
          acc[0] = zero4();
          A[0] = &sm.kp[16 * R][0];
          if constexpr (NA == 2) {
            acc[1] = zero4();
            A[1] = &sm.qp[16 * R][0];
          }
          tiles_mma_sb<NA>(acc, A, LDK, &sm.sT[16 * jtw][0], LDK, DK, lane);
          if constexpr (NA == 2) qs[m] = acc[1];
          const int jl = 16 * jtw + (lane & 15), i0 = 16 * R + 4 * (lane >> 4);
          float z[4];
#pragma unroll
          for (int rr = 0; rr < 4; ++rr) z[rr] = zval(i0 + rr, jl, acc[0][rr]);
          put4(&sm.zT[jl][i0], z);
        }
      }
    }
    __syncthreads();

    // ---- U = T diag(beta) Z  (stored transposed) ----------------------------
    // T diag(beta) is zero right of each diagonal block, so the pairs of a
    // wave can share one run over the last pair's row extent.
    if (all_pairs) {
      f32x4 acc[NUT];
      const ST* A[NUT];
#pragma unroll
      for (int m = 0; m < NUT; ++m) {
        acc[m] = zero4();
        A[m] = &sm.tb[16 * ((wave + NW * m) / NJT)][0];
      }
      tiles_mma_sb<NUT>(acc, A, LC, &sm.zT[16 * jtw][0], LC, kmax, lane);
#pragma unroll
      for (int m = 0; m < NUT; ++m) {
        const int R = (wave + NW * m) / NJT;
        const float uv[4] = {acc[m][0], acc[m][1], acc[m][2], acc[m][3]};
        put4(&sm.buf.uT[16 * jtw + (lane & 15)][16 * R + 4 * (lane >> 4)], uv);
      }
    } else {
#pragma unroll
      for (int m = 0; m < NUT; ++m) {
        const int x = wave + NW * m;
        if (x < nb * NJT) {
          const int R = x / NJT;
          const f32x4 u4 = tile_mma<ST>(zero4(), &sm.tb[16 * R][0], LC, &sm.zT[16 * jtw][0], LC, 16 * (R + 1), lane);
          const float uv[4] = {u4[0], u4[1], u4[2], u4[3]};
          put4(&sm.buf.uT[16 * jtw + (lane & 15)][16 * R + 4 * (lane >> 4)], uv);
        }
      }
    }
    __syncthreads();

    // ---- O = QS + Aqk U;  S <- diag(g_n) S + (k g_n/g)^T U -----------------
    if constexpr (MODE == 0) {
    if (all_pairs) {
      const ST* A[NUT];
#pragma unroll
      for (int m = 0; m < NUT; ++m) A[m] = &sm.aqk[16 * ((wave + NW * m) / NJT)][0];
      tiles_mma_sb<NUT>(qs, A, LC, &sm.buf.uT[16 * jtw][0], LC, kmax, lane);
#pragma unroll
      for (int m = 0; m < NUT; ++m) {
        const int jl = 16 * jtw + (lane & 15), i0 = 16 * ((wave + NW * m) / NJT) + 4 * (lane >> 4);
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) put(&sm.o[i0 + rr][jl], qs[m][rr]);
      }
    } else {
#pragma unroll
      for (int m = 0; m < NUT; ++m) {
        const int x = wave + NW * m;
        if (x < nb * NJT) {
          const int R = x / NJT;
          const f32x4 acc = tile_mma<ST>(qs[m], &sm.aqk[16 * R][0], LC, &sm.buf.uT[16 * jtw][0], LC, 16 * (R + 1), lane);
          const int jl = 16 * jtw + (lane & 15), i0 = 16 * R + 4 * (lane >> 4);
#pragma unroll
          for (int rr = 0; rr < 4; ++rr) put(&sm.o[i0 + rr][jl], acc[rr]);
        }
      }
    }
    }
    {
      // The state tiles of a wave share the column tile jtw, so the update
      // reads one B operand, U^T's tile jtw.
      const ST* A[NS];
#pragma unroll
      for (int u = 0; u < NS; ++u) {
        const int s = min(wave + NW * u, NST - 1);
        const int ct = s / NJT;
        const int c0 = 16 * ct + 4 * (lane >> 4);
        if (wave + NW * u < NST) {
#pragma unroll
          for (int rr = 0; rr < 4; ++rr) S[u][rr] *= sm.gexp[c0 + rr];
        }
        A[u] = &sm.khT[16 * ct][0];
      }
      const ST* B = &sm.buf.uT[16 * jtw][0];
      // Batches of at most four tiles keep the operand fragments in registers.
      constexpr int NB4 = NS < 4 ? NS : 4;
#pragma unroll
      for (int u0 = 0; u0 < NS; u0 += NB4) {
        if (wave + NW * (u0 + NB4 - 1) < NST) {
          tiles_mma_sb<NB4>(S + u0, A + u0, LC, B, LC, 16 * nb, lane);
        } else {
#pragma unroll
          for (int u = u0; u < u0 + NB4; ++u)
            if (wave + NW * u < NST) S[u] = tile_mma<ST>(S[u], A[u], LC, B, LC, 16 * nb, lane);
        }
      }
    }
    __syncthreads();

    // ---- S^T; this chunk's output rows (16 bytes per store); checkpoint -----
    write_sT();
    if (is_ck) {
      store_state(p.page_pool + static_cast<int64_t>(p.ck_slot[ck]) * p.page_elems +
                  static_cast<int64_t>(h) * DK * dv);
      ++ck;
    }
    pt0 = t0;
    pn = n;
    t0 = tn;
    n = nn;
  }
  if constexpr (MODE == 0) {
    if (c_hi > c_lo) store_o(pt0, pn);
  }
  if (p.s_final != nullptr) store_state(p.s_final + state_off);
}

constexpr int kWaves = 8;

template <int DK, typename InT>
hipError_t launch_local(const PrefillArgs& a) {
  LocalParams prm;
  prm.q = a.q; prm.k = a.k; prm.a = a.a; prm.beta = a.beta; prm.g_min = a.g_min;
  prm.perm = a.slab ? 1 : 0;
  prm.chunks = a.chunks; prm.tq = a.tq; prm.H = a.H; prm.ld = a.chunk;
  prm.wsflag = a.wsflag; prm.err_flag = a.err_flag; prm.a_lo = a.a_lo;
  const dim3 grid(static_cast<unsigned>(a.n_chunks) * static_cast<unsigned>(a.H));
  if (a.gate)
    hipLaunchKernelGGL((local_kernel<DK, InT, kWaves, true>), grid, dim3(64 * kWaves), 0, a.stream, prm);
  else
    hipLaunchKernelGGL((local_kernel<DK, InT, kWaves, false>), grid, dim3(64 * kWaves), 0, a.stream, prm);
  return hipGetLastError();
}

template <int DK, int DVT, typename InT, int MODE>
hipError_t launch_prop(const PrefillArgs& a) {
  PropParams prm;
  prm.v = a.v; prm.tq = a.tq;
  prm.s0 = a.s0; prm.o = a.o; prm.s_final = a.s_final;
  prm.page_pool = a.page_pool; prm.page_elems = a.page_elems;
  prm.chains = a.chains; prm.seqinfo = a.seqinfo; prm.ck_pos = a.ck_pos; prm.ck_slot = a.ck_slot;
  prm.chunks = a.chunks; prm.wsflag = a.wsflag;
  prm.H = a.H; prm.dv = a.dv; prm.ld = a.chunk; prm.dv_tiles = a.dv_tiles;
  const dim3 grid(static_cast<unsigned>(a.n_chains) * static_cast<unsigned>(a.dv_tiles));
  hipLaunchKernelGGL((prop_kernel<DK, DVT, InT, kWaves, MODE>), grid, dim3(64 * kWaves), 0, a.stream, prm);
  return hipGetLastError();
}

}  // namespace
}  // namespace kda
