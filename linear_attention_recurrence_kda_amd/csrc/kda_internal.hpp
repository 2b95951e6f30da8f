// Host-side launch interface between the C ABI layer (kda_api.cpp) and the
// kernel files.  Arguments arrive here already validated.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace kda {

// Decode (t_draft = 1, n_accepted = nullptr, s_in == s_out) and replay.
struct SweepArgs {
  const void* s_in;   // fp32, or bf16 when state_bf16
  void* s_out;
  bool state_bf16;
  const void *q, *k, *v, *a, *beta;
  const int32_t* n_accepted;  // nullptr: every session runs t_draft steps
  int t_draft, B, H, dk, dv;
  bool bf16;
  void* o;
  int o_steps;  // rows per (b, h) in o: 1 for decode, t_draft for replay
  int32_t* err_flag;
  hipStream_t stream;
};
hipError_t launch_sweep(const SweepArgs& p);

// Pack (state -> pages) and unpack (pages -> state).
struct PackArgs {
  const void* src;  // elements of es bytes (4: fp32, 2: bf16)
  void* dst;
  int es;
  const int32_t* slot;
  int B, H, dk, dv;
  bool vk;      // the state side uses the [.., dv, dk] layout
  bool unpack;  // pages -> state
  int64_t page_elems, n_slots;
  int32_t* err_flag;
  hipStream_t stream;
};
hipError_t launch_pack(const PackArgs& p);

// Chunked prefill.  The work list lives in the caller's workspace; the host
// layer (kda_api_prefill.cpp) builds it:
//   chains [n_chains][2]  (sequence or -1 for padding, head), longest first,
//                         n_chains a multiple of 8 (one XCD round)
//   seqinfo [n_seqs][6]   (first token, end token, first ckpt, end ckpt,
//                         first chunk, end chunk)
//   ck_pos / ck_slot      per-sequence token counts and page slots
//   chunks [n_chunks][2]  (first token, rows)
// followed by one record per (chunk, head) unit, written by the local kernel
// and read by the propagation kernel (elements of the operand type, bf16 for
// bf16 inputs and fp32 for fp32 inputs; ld = chunk):
//   T diag(beta) [ld][ld], lower(A_qk) [ld][ld], k*g [ld][dk], q*g [ld][dk],
//   (k*g_n/g)^T [dk][ld], then g_n [dk] in fp32.
// Rows and columns past the chunk's last 16-row block are zero, and so are
// the entries right of each diagonal 16x16 block of the two [ld][ld] tiles.
// Slab-format records (PrefillArgs::slab: bf16, chunk 64, dk % 32 == 0, read
// by the column-slab kernel) store the columns of the two tiles, k*g and q*g
// in slab_col order ((k*g_n/g)^T keeps its token order) and leave the
// upper-right 32x32 quadrant of the two tiles unwritten (that kernel never
// reads it).
struct UnitLayout {
  size_t aqk, kp, qp, kh, gexp, bytes;  // byte offsets within a record, record size
  __host__ __device__ UnitLayout(int ld, int dk, int es) {
    const size_t sq = static_cast<size_t>(ld) * ld * es, rk = static_cast<size_t>(ld) * dk * es;
    aqk = sq;
    kp = 2 * sq;
    qp = kp + rk;
    kh = qp + rk;
    gexp = kh + rk;
    bytes = gexp + static_cast<size_t>(dk) * 4;
  }
};
struct PrefillArgs {
  const void *q, *k, *v, *a, *beta;
  bool bf16;
  bool gate;    // a, beta are logits; a = g_min * sigmoid(a), beta = sigmoid(beta)
  bool slab;    // slab-format records and the column-slab propagation kernel
  bool fused;   // the fused kernel (kda_fused.hip): bf16, chunk 32, dk 128, no records
  float g_min;
  int H, dk, dv, chunk;
  const float* s0;
  void* o;
  float* s_final;
  float* page_pool;
  int64_t page_elems;
  const int32_t *chains, *seqinfo, *ck_pos, *ck_slot;
  const int32_t* chunks;  // [n_chunks][2] = (first token, rows)
  void* tq;               // [n_chunks][H] unit records (UnitLayout)
  int n_chunks;
  int n_chains;  // padded
  int dv_tiles;  // workgroups per chain (split of dv)
  const int32_t* wgs;  // mixed tile widths (slab prefill): [n_wg] entries (slab_mixed_kernel), or n_wg = 0
  int n_wg;
  // Decay range: the local kernel raises *wsflag (a word of the workspace,
  // zero on entry) and *err_flag (the caller's, or null) when a log-decay lies
  // outside [a_lo, 0] or is not a number; the prefill's propagation then
  // writes nothing.
  int32_t* wsflag;
  int32_t* err_flag;
  float a_lo;
  // Segments of split sequences (fused path; see launch_fused): null segx
  // when no sequence is split.
  const int32_t* segx;
  void* qhat;
  float* xpool;
  float* tstate;
  const int32_t* titems;  // tail items of sequences in two segments
  int32_t* tcnt;          // their completion counters (zero on entry)
  hipStream_t stream;
};
hipError_t launch_prefill(const PrefillArgs& p);

// Mode bits of a segment entry (PrefillArgs::segx): start from the zero state
// instead of s0; end state to tstate instead of s_final; checkpoints to xpool
// (stride H*dk*dv) instead of the page pool.
enum : int { kSegZeroStart = 1, kSegFinalTemp = 2, kSegCkTemp = 4 };
constexpr int kSegxInts = 6;  // ints per segx entry
// The fused prefill (one kernel, records in LDS): p.wgs lists one entry per
// workgroup, chain << 8 | width code << 4 | tile (width code 0: 32 columns,
// 1: 64, 2: 128, 3: 16, 4: 128 columns from the identity with v = 0).
hipError_t launch_fused(const PrefillArgs& p);
// The column-slab propagation (p.slab): mode 0 prefill, 1 a segment's B, 2 its A.
hipError_t launch_slab_prop(const PrefillArgs& p, int mode);

// Segment summaries: the work list and records of a prefill over the segments
// (q unused, o and s0 null), then two propagations: p.s_final receives B (the
// end state from the zero state) and a_out [n_seqs][H][dk][dk] receives A (the
// end state from the identity with v = 0), propagated in a_tiles column tiles.
hipError_t launch_segment_summary(const PrefillArgs& p, float* a_out, int a_tiles);

// Exclusive scan of segment maps: starts[i] = A[i-1] starts[i-1] + B[i-1].
struct ComposeArgs {
  const float *A, *B, *s_in;
  float *starts, *s_end;
  int n, H, dk, dv;
  hipStream_t stream;
};

// Tail items of the fused launch (kda_fused.hip, fused_tail): int32 each.
constexpr int kTailInts = 12;
hipError_t launch_compose(const ComposeArgs& p);

// Front end (convolution, SiLU, L2Norm, gates).  Prefill: one unit per tile
// [n_tiles][4] = (sequence, first token, tokens, the sequence's first token),
// carried windows win_in [N][K-1][C] or null.  Step: one unit per session,
// x [B][C], the window win_in [B][K-1][C] read and written back to win_step.
struct FrontParams {
  const void *x, *z_a, *z_b, *w, *win_in;
  void* win_step;
  void *q, *k, *v, *a, *beta;
  const int32_t* tiles;
  float g_min;
  int H, dk, dv, K, C;
  bool bf16;
  hipStream_t stream;
};
hipError_t launch_front(const FrontParams& p, int units, bool step);

// Convolution windows at boundaries [n_bnd][4] = (sequence, token count p,
// pool slot or -1 for win_out, the sequence's first token).
struct WindowParams {
  const void *x, *win_in;
  void *win_out, *pool;
  int64_t pool_elems;
  const int32_t* bnd;
  int n_bnd, K, C;
  bool bf16;
  hipStream_t stream;
};
hipError_t launch_windows(const WindowParams& p);

// Raw-input rings: field f in (q, k, v, a, beta) is [n_slots][capacity][elems[f]]
// in elements of es bytes; count [n_slots].
struct RingArgs {
  void* field[5];
  int64_t elems[5];
  int32_t* count;
  int64_t n_slots;
  int capacity, es;
  int32_t* err_flag;
  hipStream_t stream;
};
// One step's inputs [B][elems[f]] (push) or the window [capacity][B][elems[f]].
struct RingStep {
  void* field[5];
};
hipError_t launch_ring_push(const RingArgs& r, const int32_t* slot, int B, const RingStep& in);
hipError_t launch_ring_window(const RingArgs& r, const int32_t* slot, int B, const RingStep& out,
                              int32_t* n_valid);
hipError_t launch_ring_reset(const RingArgs& r, const int32_t* slot, int B);

}  // namespace kda
