// Column-slab propagation kernel of the chunked prefill and of the segment
// summaries (bf16 inputs, chunk 64, dk a multiple of 32), MFMA on gfx950.
// It runs the chunk step of prop_kernel (derivation at the top of
// kda_prefill_kernels.hpp):
//   Z = V - (k*g) S,  U = T diag(beta) Z,  O = (q*g) S + lower(A_qk) U,
//   S <- diag(g_n) S + (k*g_n/g)^T U,
// with another mapping.  Every column of S evolves on its own: Z, U and O
// column j need only S column j.  So each wave owns a slab of 16*NJ columns
// of S (all dk rows) for the whole chain and runs the step for its slab
// alone; the waves of a workgroup share nothing but the chunk's record.
//
// Operands stay in registers.  A 16x16 accumulator tile holds, in lane l,
// rows 4(l/16)..+3 of column l%16.  Two such tiles stacked along the
// contraction index are the B operand of v_mfma_f32_16x16x32_bf16 (lane l:
// eight k values of column l%16) and, read as S^T, its A operand, when the
// k values of lane group g = l/16 are taken in the order {4g..4g+3,
// 16+4g..16+4g+3}.  The local kernel writes the record with its columns in
// that order (slab_col), so a fragment of k*g, q*g or the two tiles is one
// 16-byte LDS read ((k*g_n/g)^T keeps its token order: two 8-byte reads),
// and S, Z and U feed the next product straight from the accumulators
// (rounded to bf16, as the LDS-staged path rounds them).
//
// Two loader waves do every move between global memory and LDS
// (global_load_lds_dwordx4 in, buffer stores out): a wave stalls while the
// memory pipeline accepts its operations, and a CU streams about 17 bytes
// per clock from HBM, so the loads live in waves of their own, and start
// early.  The record is split by when it is read: the early part (k*g,
// T diag(beta)) before the mid-chunk barrier M, the late part after it.
// Each part and v (this tile's columns) are double-buffered; the early part
// of chunk c+2 streams in from M of chunk c, the late part and v of chunk
// c+1 from the start of chunk c, and the barrier A at the end of chunk c
// hands chunk c+1 over.  The compute waves write the outputs into v's
// buffer, and the loader waves store them.  The LDS copies have no padding:
// 16-byte pieces are XOR-swizzled by row so that the rows of a fragment read
// fall on distinct banks, and the two 64x64 tiles keep only their lower
// 32x32-block triangle.
//
// O is formed transposed (O^T = S^T (q g)^T + U^T A_qk^T), so a lane holds
// consecutive columns of one output row: with the column order of slab_jcol,
// eight of them over its two column tiles, one 16-byte piece.  o is
// addressed through a buffer resource that ends at the chunk's last row, so
// stores past it are dropped and the partial last chunk of a sequence needs
// no per-lane branches.
//
// MODE 0: prefill.  MODE 1: a segment's B, the end state from s0 (zero when
// null), no outputs.  MODE 2: a segment's A, the end state from the identity
// (dv = dk) with v taken as zero, no outputs.
//
// slab_kernel runs one tile width for every chain.  slab_mixed_kernel (the
// prefill at dv = 128) takes a width per workgroup from a host-built list,
// so that the longest sequences run in narrow tiles (a shorter chain per
// chunk) and the short ones in wide tiles (the record read once per chain):
// with one long sequence among short ones the propagation is bounded by that
// sequence's chain, not by the total work.
#pragma once

#include <climits>
#include <type_traits>

#include "kda_prefill_kernels.hpp"

namespace kda {
namespace {

// Buffer resource over [base, base + bytes) (raw, stride 0).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buf_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), static_cast<short>(0),
                                           static_cast<int>(bytes), 0x00020000);
}

// The work list is written before the launch and only read by the kernel: read
// it through the constant address space, so uniform indices become scalar
// loads instead of vector loads that later waits would have to count.
__device__ __forceinline__ int ld_const(const int32_t* p, int i) {
  return ((const __attribute__((address_space(4))) int32_t*)(p))[i];
}

// 16 bytes per lane from gbase + voff (lane offset) to LDS at lds + 16 *
// lane, issued as inline assembly: the compiler then cannot tell that it
// writes LDS and does not hold every later LDS read of the other buffer
// until it lands (it cannot tell the buffers apart), and LDS reads of the
// current buffer may be scheduled across it.  Completion is awaited
// explicitly (vm_drain) before the barrier that hands the buffer over; for
// the compiler's own waits an unseen load only makes them count more loads
// in flight, never fewer.  M0 holds the LDS address; one wait state separates
// its write from the load that reads it.
__device__ __forceinline__ void dma16(const void* gbase, uint32_t voff, const void* lds) {
  const uint32_t la = static_cast<uint32_t>(
      reinterpret_cast<uintptr_t>((const __attribute__((address_space(3))) void*)(lds)));
  asm volatile(
      "s_mov_b32 m0, %0\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %1, %2"
      :
      : "s"(la), "v"(voff), "s"(gbase)
      : "m0");
}

// One chunk's record matrices in LDS as 16-byte pieces, row-major, the
// pieces of row m stored at q ^ (m mod min(pieces per row, 8)), so that the
// rows of a fragment read fall on distinct banks.  T diag(beta) and
// lower(A_qk) are zero right of their diagonal 32x32 blocks, which are never
// read: rows 0..31 keep columns 0..31 (4 pieces), rows 32..63 all 8.
template <int DK>
struct SlabRec {
  static constexpr int WK = DK / 8;                        // pieces per DK-column row
  static constexpr int TB0 = 0, TB1 = 128, AQ0 = 384, AQ1 = 512, KP = 768;
  static constexpr int QP = KP + 8 * DK, KH = QP + 8 * DK, NU = KH + 8 * DK;
  i32x4 u[NU];
};

template <int W>
__device__ __forceinline__ int swz(int m, int q) {
  return q ^ (m & (W < 8 ? W - 1 : 7));
}

// Fragment of a record matrix stored at piece BASE with W pieces per row:
// row m (of the stored part), contraction pieces q = 4s + g.
template <int BASE, int W, int DK>
__device__ __forceinline__ bf16x8 frag(const SlabRec<DK>& r, int m, int q) {
  return __builtin_bit_cast(bf16x8, r.u[BASE + m * W + swz<W>(m, q)]);
}
// (k g_n/g)^T keeps the natural token order (its rows are written 16 bytes
// at a time by the local kernel): the fragment's two halves, tokens
// 32s + 4g .. +3 and 32s + 16 + 4g .. +3, are two 8-byte reads.
template <int BASE, int DK>
__device__ __forceinline__ bf16x8 frag_kh(const SlabRec<DK>& r, int m, int s, int g) {
  const char* row = reinterpret_cast<const char*>(&r.u[BASE + 8 * m]);
  const int q1 = 4 * s + (g >> 1), q2 = q1 + 2, off = 8 * (g & 1);
  const i32x2 lo = *reinterpret_cast<const i32x2*>(row + 16 * swz<8>(m, q1) + off);
  const i32x2 hi = *reinterpret_cast<const i32x2*>(row + 16 * swz<8>(m, q2) + off);
  return __builtin_bit_cast(bf16x8, i32x4{lo[0], lo[1], hi[0], hi[1]});
}
// T diag(beta) or lower(A_qk) (LO, HI: the two stored parts), row block T,
// k-step s <= T / 2.
template <int LO, int HI, int DK>
__device__ __forceinline__ bf16x8 frag_tri(const SlabRec<DK>& r, int T, int s, int col, int grp) {
  return T < 2 ? frag<LO, 4>(r, 16 * T + col, grp) : frag<HI, 8>(r, 16 * (T - 2) + col, 4 * s + grp);
}

// Two accumulator tiles (rows 16*2s.. and 16*(2s+1).. of one column tile) as
// one MFMA operand fragment, rounded to bf16.
__device__ __forceinline__ bf16x8 pack_frag(const f32x4& lo, const f32x4& hi) {
  bf16x8 r;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    r[i] = static_cast<__bf16>(lo[i]);
    r[4 + i] = static_cast<__bf16>(hi[i]);
  }
  return r;
}

__device__ __forceinline__ f32x4 mma(const bf16x8& a, const bf16x8& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// Waits for every vector memory operation of this wave, including direct
// loads into LDS (s_waitcnt vmcnt(0), other counters left alone).
__device__ __forceinline__ void vm_drain() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// Workgroup barrier for the slab kernel's two hand-overs, without the fences
// of __syncthreads (whose acquire side would make every wave wait for its own
// output stores): the LDS reads of this wave are complete (lgkmcnt(0)), and
// the compiler keeps memory operations on their side of it.  Direct loads
// into LDS are waited for explicitly (vm_drain) by the waves that issue them.
__device__ __forceinline__ void slab_barrier() {
  __builtin_amdgcn_s_waitcnt(0xC07F);
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// The chunks of one sequence in order, as the host lays them out: 64 tokens,
// cut at the sequence end and at each checkpoint position (so no table read
// is needed per chunk).  nck is the next checkpoint's token (INT_MAX when
// none is left), ck its index.
struct ChunkWalk {
  int t, n, nck, ck;
};

__device__ __forceinline__ float bf16_bits_to_f32(short x) {
  return __uint_as_float(static_cast<uint32_t>(static_cast<uint16_t>(x)) << 16);
}

// Column of a wave's slab held by lane column `col` of column tile J.  Any
// order works (the columns are independent); with two tiles this one gives a
// lane of O^T the eight consecutive columns 8g..8g+7 (g = lane / 16) over
// its two tiles, stored as one 16-byte piece.
template <int NJ>
__device__ __forceinline__ int slab_jcol(int J, int col) {
  return NJ == 2 ? 8 * (col >> 2) + 4 * J + (col & 3) : col;
}

// One workgroup per (sequence, head, 16*NJ*NWV-column tile): NWV compute
// waves and NLW loader waves.
constexpr int kLoaders = 2;
template <int DK, int NWV, int NJ, int MODE>
__device__ __forceinline__ void slab_body(const PropParams& p, int chain, int tile, SlabRec<DK>* sm,
                                          float (*gx)[256], __bf16* vbase) {
  constexpr int NLW = kLoaders;
  constexpr int NT = 64 * (NWV + NLW), DVT = 16 * NJ * NWV;
  constexpr int NR = DK / 16;   // 16-row blocks of S
  constexpr int NKS = DK / 32;  // k-steps over dk
  using Rec = SlabRec<DK>;
  constexpr int WK = Rec::WK;
  constexpr int VPR = DVT / 8;                // 16-byte pieces per row of the v tile
  constexpr int VSW = VPR < 4 ? VPR - 1 : 3;  // v row swizzle: piece q of row r at q ^ ((r >> 2) & VSW)
  static_assert(DK % 32 == 0, "dk a multiple of 32");
  __bf16 (*vb)[64 * DVT] = reinterpret_cast<__bf16 (*)[64 * DVT]>(vbase);  // v of a chunk, this tile

  const int tid = threadIdx.x, lane = tid & 63, grp = lane >> 4, col = lane & 15;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const bool loader = wave >= NWV;  // uniform
  const int lw = wave - NWV;         // loader index
  const int H = p.H, dv = p.dv;

  const int seq = ld_const(p.chains, 2 * chain), h = ld_const(p.chains, 2 * chain + 1);
  if (seq < 0) return;
  if (MODE == 0 && ld_const(p.wsflag, 0) != 0) return;  // a decay out of range: write nothing
  const int lo = ld_const(p.seqinfo, 6 * seq), hi = ld_const(p.seqinfo, 6 * seq + 1);
  const int ck_lo = ld_const(p.seqinfo, 6 * seq + 2);
  const int ck_hi = ld_const(p.seqinfo, 6 * seq + 3), c_lo = ld_const(p.seqinfo, 6 * seq + 4);
  const int c_hi = ld_const(p.seqinfo, 6 * seq + 5);
  const int jl = 16 * NJ * (loader ? 0 : wave);  // first column of this wave's slab within the tile
  const int jw = tile * DVT + jl;                // ... within the state
  const int64_t hkv = static_cast<int64_t>(H) * DK * dv;
  const size_t state_off = (static_cast<size_t>(seq) * H + h) * DK * dv;
  const UnitLayout lay(64, DK, 2);
  const uint32_t rsv = static_cast<uint32_t>(H) * dv * 2;  // token row stride of v and o, bytes

  // S tile (R, J): rows 16R + 4 grp + i, column jw + slab_jcol(J, col)
  // (compute waves).
  f32x4 S[NR][NJ];
#pragma unroll
  for (int R = 0; R < NR; ++R)
#pragma unroll
    for (int J = 0; J < NJ; ++J) {
      S[R][J] = zero4();
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int c = 16 * R + 4 * grp + i, j = jw + slab_jcol<NJ>(J, col);
        if constexpr (MODE == 2) S[R][J][i] = c == j ? 1.f : 0.f;
        else if (!loader && p.s0 != nullptr) S[R][J][i] = p.s0[state_off + static_cast<size_t>(c) * dv + j];
      }
    }
  // dst points at this head's [DK][dv] block.  One buffer resource per
  // 16-row block; the lane offsets of its four rows in registers.
  uint32_t slane[4];  // column tile 0; tile 1 is 4 columns on (two tiles) or absent
#pragma unroll
  for (int i = 0; i < 4; ++i) slane[i] = ((4 * grp + i) * dv + jw + slab_jcol<NJ>(0, col)) * 4;
  auto store_state = [&](float* dst) {
#pragma unroll
    for (int R = 0; R < NR; ++R) {
      const __amdgpu_buffer_rsrc_t rs = buf_rsrc(dst + static_cast<size_t>(16 * R) * dv, 16u * dv * 4);
#pragma unroll
      for (int J = 0; J < NJ; ++J)
#pragma unroll
        for (int i = 0; i < 4; ++i)  // (the store takes the 32 bits as an integer, by value)
          __builtin_amdgcn_raw_buffer_store_b32(__float_as_int(S[R][J][i]), rs, slane[i] + 16 * J, 0, 0);
    }
  };

  auto ck_at = [&](int k) { return k < ck_hi ? lo + ld_const(p.ck_pos, k) : INT_MAX; };
  auto first_chunk = [&]() {
    ChunkWalk w{lo, 0, ck_at(ck_lo), ck_lo};
    w.n = min(min(64, hi - lo), w.nck - lo);
    return w;
  };
  auto next_chunk = [&](ChunkWalk& w) {
    if (w.t + w.n == w.nck) w.nck = ck_at(++w.ck);
    w.t += w.n;
    w.n = min(min(64, hi - w.t), w.nck - w.t);
  };

  // Zero the page padding of this sequence's checkpoint slots (once per sequence).
  if (tile == 0 && h == 0 && p.page_elems > hkv) {
    for (int c = ck_lo; c < ck_hi; ++c) {
      float* pg = p.page_pool + static_cast<int64_t>(ld_const(p.ck_slot, c)) * p.page_elems;
      for (int64_t e = hkv + tid; e < p.page_elems; e += NT) pg[e] = 0.f;
    }
  }

  if (c_lo < c_hi) {
    if (loader && lw >= NLW) {
      // ---- spare wave (a narrow tile in a workgroup sized for a wider one):
      // it issues no memory operation at all and only passes the same
      // barriers as the loader waves (one before the chain, two per chunk).
      slab_barrier();
      for (int c = c_lo; c < c_hi; ++c) {
        slab_barrier();
        slab_barrier();
      }
    } else if (loader) {
      // ---- loader wave: every global->LDS move of the chain ----------------
      // Record of chunk c: LDS piece x of a stored part (W pieces per row,
      // rows from row R0 of a record matrix whose rows are GW pieces long)
      // is local row m = x / W, stored piece pq; its source is piece
      // pq ^ (m mod min(W, 8)) of record row R0 + m.  The parts are moved in
      // 64-piece blocks, shared out between the loader waves.
      auto region = [&](const char* rc, auto lds_c, auto w_c, auto g_c, auto gw_c, auto pieces_c, int b) {
        constexpr int LDS = decltype(lds_c)::value, W = decltype(w_c)::value;
        constexpr int GB = decltype(g_c)::value, GW = decltype(gw_c)::value;  // record piece of row R0, row length
        constexpr int NB = decltype(pieces_c)::value / 64;
        static_assert(decltype(pieces_c)::value % 64 == 0, "whole blocks");
#pragma unroll
        for (int blk = 0; blk < NB; ++blk) {
          if (blk % NLW != lw) continue;
          const int m = (64 / W) * blk + lane / W, pq = lane % W;
          dma16(rc + 16 * (GB + (64 / W) * blk * GW), 16 * ((lane / W) * GW + swz<W>(m, pq)),
                &sm[b].u[LDS + 64 * blk]);
        }
      };
      // The early part of a chunk's record (k*g and T diag(beta), read before
      // the mid-chunk barrier) and the late part (the rest, read after it).
      using std::integral_constant;
      using I4 = integral_constant<int, 4>;
      using I8 = integral_constant<int, 8>;
      using IK = integral_constant<int, WK>;
      auto rec_at = [&](int c) {
        return static_cast<const char*>(p.tq) + (static_cast<size_t>(c) * H + h) * lay.bytes;
      };
      auto load_E = [&](int c, int b) {
        const char* rc = rec_at(c);
        region(rc, integral_constant<int, Rec::TB0>{}, I4{}, integral_constant<int, 0>{}, I8{},
               integral_constant<int, 128>{}, b);
        region(rc, integral_constant<int, Rec::TB1>{}, I8{}, integral_constant<int, 256>{}, I8{},
               integral_constant<int, 256>{}, b);
        region(rc, integral_constant<int, Rec::KP>{}, IK{}, integral_constant<int, 1024>{}, IK{},
               integral_constant<int, 8 * DK>{}, b);
      };
      // Direct loads one loader wave issues per load_E (the blocks split evenly).
      constexpr int NE = (2 + 4 + DK / 8) / NLW;
      static_assert(2 % NLW == 0 && 4 % NLW == 0 && (DK / 8) % NLW == 0, "even split of the early part");
      // g_n: 4 floats per lane; lanes past DK/4 repeat the last piece into
      // the landing room.
      auto load_L = [&](int c, int b) {
        const char* rc = rec_at(c);
        region(rc, integral_constant<int, Rec::KH>{}, I8{}, integral_constant<int, 1024 + 16 * DK>{}, I8{},
               integral_constant<int, 8 * DK>{}, b);
        if constexpr (MODE == 0) {  // the output side
          region(rc, integral_constant<int, Rec::AQ0>{}, I4{}, integral_constant<int, 512>{}, I8{},
                 integral_constant<int, 128>{}, b);
          region(rc, integral_constant<int, Rec::AQ1>{}, I8{}, integral_constant<int, 768>{}, I8{},
                 integral_constant<int, 256>{}, b);
          region(rc, integral_constant<int, Rec::QP>{}, IK{}, integral_constant<int, 1024 + 8 * DK>{}, IK{},
                 integral_constant<int, 8 * DK>{}, b);
        }
        // (every loader writes the same bytes)
        dma16(rc + lay.gexp, 16 * min(lane, DK / 4 - 1), &gx[b][0]);
      };
      // v of a chunk (first token t, n rows), this tile's columns: LDS piece
      // x is row r = x / VPR, stored piece pq, whose source is piece
      // pq ^ ((r >> 2) & VSW) of row r; rows past n repeat row n - 1 (their
      // T diag(beta) columns are zero, so they never reach U).
      auto load_v = [&](int t, int n, int b) {
        const char* vt = static_cast<const char*>(p.v) + (static_cast<size_t>(t) * H + h) * dv * 2 + tile * DVT * 2;
#pragma unroll
        for (int i = 0; i < VPR; ++i) {
          if (i % NLW != lw) continue;
          const int x = 64 * i + lane, r = x / VPR, pq = x % VPR;
          const uint32_t off = min(r, n - 1) * rsv + 16 * (pq ^ ((r >> 2) & VSW));
          dma16(vt, off, &vb[b][512 * i]);
        }
      };

      // Output rows of a chunk, staged by the compute waves in X[b] with v's
      // piece order: read into registers (this loader's pieces i = lw, lw +
      // NLW, ...), then stored to global memory through a buffer resource
      // that ends at the chunk's last row (first token t, n rows).
      constexpr int NOP = (VPR + NLW - 1) / NLW;  // pieces per lane
      i32x4 ov[NOP];
      auto read_o = [&](int b) {
#pragma unroll
        for (int k = 0; k < NOP; ++k) {
          const int i = lw + NLW * k;
          if (i < VPR) ov[k] = *reinterpret_cast<const i32x4*>(&vb[b][8 * (64 * i + lane)]);
        }
      };
      auto store_o = [&](int t, int n) {
        const __amdgpu_buffer_rsrc_t ro =
            buf_rsrc(static_cast<char*>(p.o) + (static_cast<size_t>(t) * H + h) * dv * 2 + tile * DVT * 2,
                     (n - 1) * rsv + DVT * 2);
#pragma unroll
        for (int k = 0; k < NOP; ++k) {
          const int i = lw + NLW * k;
          if (i >= VPR) continue;
          const int x = 64 * i + lane, r = x / VPR, pq = x % VPR;
          __builtin_amdgcn_raw_buffer_store_b128(ov[k], ro, r * rsv + 16 * (pq ^ ((r >> 2) & VSW)), 0, 0);
        }
      };

      // Chunk c's early part is in LDS from the middle of chunk c - 2 on,
      // its late part and v from the start of chunk c - 1 on: every load has
      // more than a chunk's time to land.
      ChunkWalk wv = first_chunk();  // the chunk whose v is loaded next
      ChunkWalk wo = wv;             // the chunk whose outputs are stored next
      load_E(c_lo, 0);
      load_E(min(c_lo + 1, c_hi - 1), 1);
      load_L(c_lo, 0);
      if constexpr (MODE != 2) load_v(wv.t, wv.n, 0);
      vm_drain();
      slab_barrier();  // A: chunk c_lo in LDS
      for (int c = c_lo; c < c_hi; ++c) {
        const int b = (c - c_lo) & 1;
        // Chunk c - 1's outputs leave X[b ^ 1] for registers, then chunk
        // c + 1's v and late part move in (this chunk again at the end of the
        // chain); the outputs are stored after the mid-chunk barrier.
        if constexpr (MODE == 0) {
          if (c > c_lo) read_o(b ^ 1);
          __builtin_amdgcn_s_waitcnt(0xC07F);  // the reads are done before v lands there
        }
        if (c + 1 < c_hi) next_chunk(wv);
        if constexpr (MODE != 2) load_v(wv.t, wv.n, b ^ 1);
        load_L(min(c + 1, c_hi - 1), b ^ 1);
        slab_barrier();  // M: the compute waves are done with chunk c's early part
        if constexpr (MODE == 0) {
          if (c > c_lo) {
            store_o(wo.t, wo.n);
            next_chunk(wo);
          }
        }
        load_E(min(c + 2, c_hi - 1), b);
        // Everything issued before the early part just issued: the loads land
        // in order, so at most the NE newest operations are pending only when
        // all older loads are done.
        __builtin_amdgcn_s_waitcnt((NE & 15) | ((NE >> 4) << 14) | 0x0F70);
        slab_barrier();  // A: chunk c + 1 in LDS; chunk c's late part and v free
      }
      if constexpr (MODE == 0) {
        read_o((c_hi - 1 - c_lo) & 1);
        store_o(wo.t, wo.n);
      }
    } else {
      // ---- compute waves ------------------------------------------------------
      // Output rows go to X[b] (v's place, consumed by then) for the loader
      // waves to store: a lane holds tile columns jl + 8g .. +7 (two column
      // tiles) or jl + 4g .. +3 (one) of row 16T + col.
      using OV = std::conditional_t<NJ == 2, i32x4, i32x2>;
      auto stage_o = [&](int b, int T, const OV& ov) {
        const int r = 16 * T + col, j = jl + 4 * NJ * grp;
        __bf16* dst = &vb[b][r * DVT + (((j >> 3) ^ ((r >> 2) & VSW)) << 3) + (j & 7)];
        *reinterpret_cast<OV*>(dst) = ov;
      };
      // v of tile (T, J) row i of this lane: row 16T + 4 grp + i, tile
      // column jl + 16J + col.
      auto vval = [&](int b, int T, int J, int i) {
        const int r = 16 * T + 4 * grp + i, j = jl + slab_jcol<NJ>(J, col);
        return static_cast<float>(vb[b][r * DVT + (((j >> 3) ^ ((r >> 2) & VSW)) << 3) + (j & 7)]);
      };

      ChunkWalk w = first_chunk();
      slab_barrier();  // A: chunk c_lo in LDS
      for (int c = c_lo; c < c_hi; ++c) {
        const int b = (c - c_lo) & 1;
        const Rec& r = sm[b];
        const bool is_ck = w.t + w.n == w.nck;

        // ---- P = (k g) S over dk -------------------------------------------
        f32x4 P[4][NJ];
#pragma unroll
        for (int T = 0; T < 4; ++T)
#pragma unroll
          for (int J = 0; J < NJ; ++J) P[T][J] = zero4();
#pragma unroll
        for (int s = 0; s < NKS; ++s) {
          bf16x8 bS[NJ];
#pragma unroll
          for (int J = 0; J < NJ; ++J) bS[J] = pack_frag(S[2 * s][J], S[2 * s + 1][J]);
#pragma unroll
          for (int T = 0; T < 4; ++T) {
            const bf16x8 ak = frag<Rec::KP, WK>(r, 16 * T + col, 4 * s + grp);
#pragma unroll
            for (int J = 0; J < NJ; ++J) P[T][J] = mma(ak, bS[J], P[T][J]);
          }
        }
        // ---- Z = V - P (V = 0 for MODE 2) ----------------------------------
        bf16x8 bZ[2][NJ];
#pragma unroll
        for (int s = 0; s < 2; ++s)
#pragma unroll
          for (int J = 0; J < NJ; ++J) {
            f32x4 z0, z1;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              if constexpr (MODE == 2) {
                z0[i] = -P[2 * s][J][i];
                z1[i] = -P[2 * s + 1][J][i];
              } else {
                z0[i] = vval(b, 2 * s, J, i) - P[2 * s][J][i];
                z1[i] = vval(b, 2 * s + 1, J, i) - P[2 * s + 1][J][i];
              }
            }
            bZ[s][J] = pack_frag(z0, z1);
          }

        // ---- U = T diag(beta) Z (block lower triangular) -----------------
        f32x4 U[4][NJ];
#pragma unroll
        for (int T = 0; T < 4; ++T) {
#pragma unroll
          for (int J = 0; J < NJ; ++J) U[T][J] = zero4();
#pragma unroll
          for (int s = 0; s <= T / 2; ++s) {
            const bf16x8 at = frag_tri<Rec::TB0, Rec::TB1>(r, T, s, col, grp);
#pragma unroll
            for (int J = 0; J < NJ; ++J) U[T][J] = mma(at, bZ[s][J], U[T][J]);
          }
        }
        bf16x8 bU[2][NJ];
#pragma unroll
        for (int s = 0; s < 2; ++s)
#pragma unroll
          for (int J = 0; J < NJ; ++J) bU[s][J] = pack_frag(U[2 * s][J], U[2 * s + 1][J]);
        slab_barrier();  // M: done with this chunk's early part

        // ---- O^T = S^T (q g)^T + U^T A_qk^T -------------------------------
        if constexpr (MODE == 0) {
          f32x4 OT[NJ][4];
#pragma unroll
          for (int T = 0; T < 4; ++T)
#pragma unroll
            for (int J = 0; J < NJ; ++J) OT[J][T] = zero4();
#pragma unroll
          for (int s = 0; s < NKS; ++s) {
            bf16x8 bS[NJ];
#pragma unroll
            for (int J = 0; J < NJ; ++J) bS[J] = pack_frag(S[2 * s][J], S[2 * s + 1][J]);
#pragma unroll
            for (int T = 0; T < 4; ++T) {
              const bf16x8 aq = frag<Rec::QP, WK>(r, 16 * T + col, 4 * s + grp);
#pragma unroll
              for (int J = 0; J < NJ; ++J) OT[J][T] = mma(bS[J], aq, OT[J][T]);
            }
          }
#pragma unroll
          for (int T = 0; T < 4; ++T) {
#pragma unroll
            for (int s = 0; s <= T / 2; ++s) {
              const bf16x8 aa = frag_tri<Rec::AQ0, Rec::AQ1>(r, T, s, col, grp);
#pragma unroll
              for (int J = 0; J < NJ; ++J) OT[J][T] = mma(bU[s][J], aa, OT[J][T]);
            }
            bf16x4 ov[NJ];
#pragma unroll
            for (int J = 0; J < NJ; ++J)
#pragma unroll
              for (int i = 0; i < 4; ++i) ov[J][i] = static_cast<__bf16>(OT[J][T][i]);
            stage_o(b, T, __builtin_bit_cast(OV, ov));
          }
        }

        // ---- S <- diag(g_n) S + (k g_n/g)^T U ----------------------------
#pragma unroll
        for (int R = 0; R < NR; ++R) {
          const float4 gn = *reinterpret_cast<const float4*>(&gx[b][16 * R + 4 * grp]);
          const bf16x8 a0 = frag_kh<Rec::KH>(r, 16 * R + col, 0, grp);
          const bf16x8 a1 = frag_kh<Rec::KH>(r, 16 * R + col, 1, grp);
#pragma unroll
          for (int J = 0; J < NJ; ++J) {
            S[R][J][0] *= gn.x;
            S[R][J][1] *= gn.y;
            S[R][J][2] *= gn.z;
            S[R][J][3] *= gn.w;
            S[R][J] = mma(a0, bU[0][J], S[R][J]);
            S[R][J] = mma(a1, bU[1][J], S[R][J]);
          }
        }
        if (is_ck) {
          store_state(p.page_pool + static_cast<int64_t>(ld_const(p.ck_slot, w.ck)) * p.page_elems +
                      static_cast<int64_t>(h) * DK * dv);
        }
        slab_barrier();  // A: the next chunk is in LDS; this one's late part and v free
        if (c + 1 < c_hi) next_chunk(w);
      }
    }
  }
  if (!loader && p.s_final != nullptr) store_state(p.s_final + state_off);
}

// One tile width for every workgroup: workgroup -> (chain, dv tile), the
// tiles of a chain on one XCD.
template <int DK, int NWV, int NJ, int MODE>
__global__ __launch_bounds__(64 * (NWV + kLoaders), 1) void slab_kernel(PropParams p) {
  __shared__ __attribute__((aligned(16))) SlabRec<DK> sm[2];
  __shared__ __attribute__((aligned(16))) float gx[2][256];                  // g_n, then landing room
  __shared__ __attribute__((aligned(16))) __bf16 vb[2 * 64 * 16 * NJ * NWV];  // v of a chunk, this tile
  const int bid = blockIdx.x, xcd = bid & 7, local = bid >> 3;
  const int chain = 8 * (local / p.dv_tiles) + xcd, tile = local % p.dv_tiles;
  slab_body<DK, NWV, NJ, MODE>(p, chain, tile, sm, gx, vb);
}

// A tile width per workgroup (prefill): entry bid of p.wgs is chain << 8 |
// width code << 4 | tile (width code 0: 32 columns, 1: 64, 2: 128; 15: no
// work).  Six waves for every width: a 32-column tile has two compute and
// two loader waves, and its two spare waves only pass the barriers.
template <int DK>
__global__ __launch_bounds__(64 * (4 + kLoaders), 1) void slab_mixed_kernel(PropParams p) {
  __shared__ __attribute__((aligned(16))) SlabRec<DK> sm[2];
  __shared__ __attribute__((aligned(16))) float gx[2][256];
  __shared__ __attribute__((aligned(16))) __bf16 vb[2 * 64 * 128];
  const int e = ld_const(p.wgs, blockIdx.x);
  const int chain = e >> 8, code = (e >> 4) & 15, tile = e & 15;
  if (code == 0) slab_body<DK, 2, 1, 0>(p, chain, tile, sm, gx, vb);
  else if (code == 1) slab_body<DK, 4, 1, 0>(p, chain, tile, sm, gx, vb);
  else if (code == 2) slab_body<DK, 4, 2, 0>(p, chain, tile, sm, gx, vb);
}

template <int DK, int NWV, int NJ, int MODE>
hipError_t launch_slab_t(const PrefillArgs& a) {
  PropParams prm;
  prm.v = a.v; prm.tq = a.tq;
  prm.s0 = a.s0; prm.o = a.o; prm.s_final = a.s_final;
  prm.page_pool = a.page_pool; prm.page_elems = a.page_elems;
  prm.chains = a.chains; prm.seqinfo = a.seqinfo; prm.ck_pos = a.ck_pos; prm.ck_slot = a.ck_slot;
  prm.chunks = a.chunks; prm.wsflag = a.wsflag;
  prm.H = a.H; prm.dv = a.dv; prm.ld = a.chunk; prm.dv_tiles = a.dv_tiles;
  const dim3 grid(static_cast<unsigned>(a.n_chains) * static_cast<unsigned>(a.dv_tiles));
  hipLaunchKernelGGL((slab_kernel<DK, NWV, NJ, MODE>), grid, dim3(64 * (NWV + kLoaders)), 0, a.stream, prm);
  return hipGetLastError();
}

// Tile widths 16, 32, 64 and 128 columns: one 16-column tile per compute
// wave up to 64 columns (more waves share the chunk's work), two at 128.
template <int DK>
hipError_t launch_slab_mixed(const PrefillArgs& a) {
  PropParams prm;
  prm.v = a.v; prm.tq = a.tq;
  prm.s0 = a.s0; prm.o = a.o; prm.s_final = a.s_final;
  prm.page_pool = a.page_pool; prm.page_elems = a.page_elems;
  prm.chains = a.chains; prm.seqinfo = a.seqinfo; prm.ck_pos = a.ck_pos; prm.ck_slot = a.ck_slot;
  prm.chunks = a.chunks; prm.wgs = a.wgs; prm.wsflag = a.wsflag;
  prm.H = a.H; prm.dv = a.dv; prm.ld = a.chunk; prm.dv_tiles = a.dv_tiles;
  hipLaunchKernelGGL((slab_mixed_kernel<DK>), dim3(static_cast<unsigned>(a.n_wg)), dim3(64 * (4 + kLoaders)), 0,
                     a.stream, prm);
  return hipGetLastError();
}

template <int DK, int MODE>
hipError_t launch_slab(const PrefillArgs& a) {
  switch (a.dv / a.dv_tiles) {
    case 16: return launch_slab_t<DK, 1, 1, MODE>(a);
    case 32: return launch_slab_t<DK, 2, 1, MODE>(a);
    case 64: return launch_slab_t<DK, 4, 1, MODE>(a);
    case 128: return launch_slab_t<DK, 4, 2, MODE>(a);
  }
  return hipErrorInvalidValue;
}

}  // namespace
}  // namespace kda
