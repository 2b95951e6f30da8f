/*
 * kda.h — C ABI of the KDA (Kimi Delta Attention) state-recurrence library
 * for AMD MI355X (gfx950).
 *
 * Pages cited (titles as published; sections as named on the page):
 *   [Serve demo]  "【轻量化复刻大模型 / KIMI K3】Serve 模块交互式演示"
 *   [KDA cache]   "Kimi Linear 的 KDA 缓存：SGLang、vLLM 与 Mooncake Store 全链路"
 *
 * The recurrence, per head, with state S (dk x dv, fp32):
 *   decay    S~ = diag(exp(a_t)) S                 a_t: one log-decay per key channel
 *   error    d  = v_t - S~^T k_t                   (formed after the decay)
 *   write    S  = S~ + beta_t k_t d^T
 *   readout  o_t = S^T q_t                         (after the write)
 * [KDA cache] "KDA 的递推与充分状态" fixes decay-then-error; [Serve demo] §1.3
 * bounds a_t to [g_min, 0] (a log value, hence the exp) and beta_t to [0, 1].
 *
 * Conventions shared by every entry point
 *  - Tensors are caller-owned device memory (any allocator), dense row-major,
 *    in the shapes stated per call.  The library never allocates device
 *    memory; the prefill work list lives in a caller-provided workspace.
 *  - Token-indexed tensors are token-packed: q, k, a [T, H, dk], v [T, H, dv],
 *    beta [T, H], o [T, H, dv].
 *  - States are fp32 in the canonical layout [.., H, dk, dv] (dv fastest).
 *  - Inputs q, k, v, a, beta share one dtype (KDA_F32 or KDA_BF16); the
 *    output o has that dtype too.  Arithmetic is fp32 (prefill contractions
 *    take bf16 operands with fp32 accumulation; see kda_chunk_prefill).
 *  - Supported head sizes: dk, dv in {16, 32, 64, 128}.
 *  - stream is a hipStream_t (NULL = the null stream).  Calls only enqueue
 *    work; they return before it runs.  They hold no state between calls and
 *    may be called from several host threads.
 *  - Errors: every argument a call can see on the host is validated before
 *    anything is enqueued, so a non-zero status means nothing was written.
 *    Values that live in device memory (n_accepted, slots) cannot be checked
 *    there; they are checked by the kernel, which skips the offending item
 *    and raises *err_flag (when err_flag is not NULL).  No call throws.
 */
#ifndef KDA_H
#define KDA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  KDA_OK = 0,
  KDA_EINVAL = -1,       /* a bad shape, size, pointer or offset array        */
  KDA_EUNSUPPORTED = -2, /* valid request outside what the kernels cover      */
  KDA_EALIAS = -3,       /* an output overlaps an input that must stay intact */
  KDA_EWORKSPACE = -4,   /* workspace missing or smaller than required        */
  KDA_EHIP = -5          /* the HIP runtime reported an error on enqueue      */
} kda_status;

/* The two range markers of each enum below make every int a value of the
 * type, so an out-of-range value from a caller in another language is
 * well-defined (and refused with KDA_EINVAL). */
typedef enum { KDA_F32 = 0, KDA_BF16 = 1, KDA_DTYPE_MIN_ = -2147483647 - 1, KDA_DTYPE_MAX_ = 2147483647 } kda_dtype;

/* State layouts: KV = [.., dk, dv] (canonical), VK = [.., dv, dk] (the
 * transposed layout some kernels and state pools use, [KDA cache] "先统一记号"). */
typedef enum {
  KDA_LAYOUT_KV = 0,
  KDA_LAYOUT_VK = 1,
  KDA_LAYOUT_MIN_ = -2147483647 - 1,
  KDA_LAYOUT_MAX_ = 2147483647
} kda_layout;

/* Version of the page layout written by pack and by checkpoint emission. */
#define KDA_PAGE_LAYOUT_VERSION 1

const char* kda_status_string(int status);

/* Text describing the most recent failure on the calling host thread ("" if
 * none).  The pointer stays valid until the next call on that thread. */
const char* kda_last_error(void);

/* Largest chunk the prefill accepts, and the chunk it is tuned for. */
#define KDA_MAX_CHUNK 64

/*
 * kda_snapshot_cost_ratio — bytes of one per-step state snapshot over bytes of
 * one per-step draft projection, H*dk*dv / (H*(3*dk + dv + 1)); independent of
 * the draft length ([Serve demo] §1.1).  Host-only helper; returns a negative
 * value for non-positive sizes.
 */
double kda_snapshot_cost_ratio(int32_t H, int32_t dk, int32_t dv);

/*
 * kda_decode_step — one token per session, state updated IN PLACE
 * ([Serve demo] §1.3 kda_step).
 *   q, k, a : [B, H, dk]   v : [B, H, dv]   beta : [B, H]   (in_dtype)
 *   state   : [B, H, dk, dv] fp32, read and overwritten
 *   o       : [B, H, dv] (in_dtype), must not overlap state or the inputs
 * B may be 0 (nothing is enqueued).
 */
int kda_decode_step(const void* q, const void* k, const void* v, const void* a,
                    const void* beta, kda_dtype in_dtype, int32_t B, int32_t H,
                    int32_t dk, int32_t dv, float* state, void* o, void* stream);

/*
 * kda_verify_and_replay — clone the committed state and replay the first
 * n_accepted[b] draft steps of session b ([Serve demo] §1.2; Tab 3 §6.4 for
 * the n = partial / all / 0 cases).
 *   committed : [B, H, dk, dv] fp32, READ ONLY (shared in the cache; never written)
 *   q, k, a   : [t_draft, B, H, dk]   v : [t_draft, B, H, dv]   beta : [t_draft, B, H]
 *               (the draft-projection layout (draft, B, H, D), [Serve demo] Tab 4)
 *   n_accepted: device int32 [B]; values outside 0..t_draft are clamped and
 *               raise *err_flag
 *   s_new     : [B, H, dk, dv] fp32, the state after n_accepted[b] steps
 *               (a bit-exact copy of committed[b] when n_accepted[b] = 0)
 *   o         : [B, H, t_draft, dv] (in_dtype); rows i >= n_accepted[b] are 0
 *   err_flag  : device int32, may be NULL; set to 1 on a clamped n_accepted
 * s_new and o must not overlap committed (KDA_EALIAS) nor each other.
 */
int kda_verify_and_replay(const float* committed, const void* q, const void* k,
                          const void* v, const void* a, const void* beta,
                          kda_dtype in_dtype, const int32_t* n_accepted, int32_t B,
                          int32_t H, int32_t dk, int32_t dv, int32_t t_draft,
                          float* s_new, void* o, int32_t* err_flag, void* stream);

/*
 * kda_pack_heads — write state[b] into page slot slot[b] of a flat page pool,
 * head after head, and zero the rest of the page ([Serve demo] §1.5 pack_heads
 * and Tab 7 store_kda: "the rest of the page is zero padding").
 *   state     : [B, H, dk, dv] (KV) or [B, H, dv, dk] (VK), fp32
 *   slot      : device int32 [B]; out-of-range slots are skipped and raise *err_flag
 *   page_pool : fp32 [n_slots, page_elems], page_elems >= H*dk*dv
 *   Page element h*dk*dv + i*dv + j holds S[h, i, j] (i over dk, j over dv).
 * Distinct b must name distinct slots (not checked: slots live on the device).
 */
int kda_pack_heads(const float* state, kda_layout src_layout, int32_t B, int32_t H,
                   int32_t dk, int32_t dv, const int32_t* slot, float* page_pool,
                   int64_t page_elems, int64_t n_slots, int32_t* err_flag, void* stream);

/* kda_unpack_heads — the inverse: page slot slot[b] -> state[b] in dst_layout.
 * Bit-exact ([Serve demo] §1.5 unpack_heads, "lossless"). */
int kda_unpack_heads(const float* page_pool, int64_t page_elems, int64_t n_slots,
                     const int32_t* slot, int32_t B, int32_t H, int32_t dk, int32_t dv,
                     kda_layout dst_layout, float* state, int32_t* err_flag, void* stream);

/*
 * bf16 states and pages (a variant: the pages keep the recurrent state in
 * FP32, [KDA cache] "检查点状态池的内存成本"; a bf16 state halves the bytes
 * decode streams).  With state_dtype = KDA_BF16 the state (and committed,
 * s_new, the page pool) holds bfloat16 values: they are widened exactly on
 * load, the arithmetic stays fp32, and stored values are rounded to the
 * nearest bfloat16, ties to even.  A decode call rounds after its step; a
 * replay call rounds once, at its end (n_accepted = 0 leaves a bit-exact
 * copy).  Pages of a bf16 state hold bf16 elements in the pack layout; pack
 * and unpack copy them bit for bit; page_elems must then be a multiple of 8.
 * state_dtype = KDA_F32 is exactly the call without the suffix.
 */
int kda_decode_step_ex(const void* q, const void* k, const void* v, const void* a,
                       const void* beta, kda_dtype in_dtype, int32_t B, int32_t H, int32_t dk,
                       int32_t dv, kda_dtype state_dtype, void* state, void* o, void* stream);

int kda_verify_and_replay_ex(const void* committed, const void* q, const void* k, const void* v,
                             const void* a, const void* beta, kda_dtype in_dtype,
                             const int32_t* n_accepted, int32_t B, int32_t H, int32_t dk,
                             int32_t dv, int32_t t_draft, kda_dtype state_dtype, void* s_new,
                             void* o, int32_t* err_flag, void* stream);

int kda_pack_heads_ex(const void* state, kda_dtype state_dtype, kda_layout src_layout, int32_t B,
                      int32_t H, int32_t dk, int32_t dv, const int32_t* slot, void* page_pool,
                      int64_t page_elems, int64_t n_slots, int32_t* err_flag, void* stream);

int kda_unpack_heads_ex(const void* page_pool, kda_dtype state_dtype, int64_t page_elems,
                        int64_t n_slots, const int32_t* slot, int32_t B, int32_t H, int32_t dk,
                        int32_t dv, kda_layout dst_layout, void* state, int32_t* err_flag,
                        void* stream);

/*
 * kda_chunk_prefill — token-packed variable-length prefill from committed
 * states, with exact checkpoints written into page slots.
 *
 * The chunked form ([KDA cache] "预填充为什么能分块并行": transitions inside a
 * chunk are diagonal-minus-rank-one and compress, through a WY representation
 * and a UT transform, into matrix products plus a small lower-triangular
 * solve) gives the recurrence's result up to rounding.  Contractions use bf16
 * MFMA operands with fp32 accumulation; the state is carried in fp32.
 *
 *   q, k, a  : [T_tot, H, dk]   v : [T_tot, H, dv]   beta : [T_tot, H]  (in_dtype)
 *   chunk    : a multiple of 16 up to KDA_MAX_CHUNK (64 is the tuned size for
 *              bf16); fp32 inputs take at most 32 (their operands stay fp32,
 *              split into bf16 high and low parts, so fp32 I/O keeps
 *              fp32-level accuracy)
 *   Log-decays must lie in [-160/chunk, 0] per token and channel ([Serve demo]
 *   §1.3 bounds a to [g_min, 0]; the lower end is -2.5 at chunk 64, -5 at
 *   chunk 32): the chunk's scaled operands, referenced to the middle row of
 *   the chunk, then stay below e^80 and are finite in bf16 and fp32.  Every
 *   a is checked on the device (a NaN fails the check too); one out of range
 *   raises *err_flag, and no wrong record is written (the [kv_prefix] page's
 *   rule that a failure never leaves a partial or wrong record).  On the
 *   two-kernel path (chunk other than 32, fp32 inputs or dk other than 128)
 *   the call then writes nothing: o, s_final and the page slots keep their
 *   contents.  On the fused path (bf16, chunk 32, dk = 128) the (sequence,
 *   head) holding the value keeps the outputs and checkpoints of the chunks
 *   before it and writes no later checkpoint and no final state; for a
 *   sequence the call cuts into segments (kda_chunk_prefill_split) that
 *   head's output rows after its first segment are then unspecified.  Every
 *   other (sequence, head) is complete.
 *   cu_seqlens_host : host int32 [n_seqs + 1]; cu[0] = 0, non-decreasing,
 *              cu[n_seqs] = T_tot.  Zero-length sequences are allowed.
 *   s0       : [n_seqs, H, dk, dv] fp32 committed states, READ ONLY, or NULL
 *              for zero states.  Outputs must not overlap it (KDA_EALIAS).
 *   o        : [T_tot, H, dv] (in_dtype), 16-byte aligned (KDA_EINVAL otherwise)
 *   s_final  : [n_seqs, H, dk, dv] fp32 or NULL
 *   Checkpoints ([KDA cache] "Kimi K3 预览版与 vLLM 的细粒度检查点": one slot
 *   holds one exact boundary, e.g. the tail C(P6976)):
 *   ckpt_cu_host   : host int32 [n_seqs + 1], offsets into the two arrays below
 *                    (NULL when n_ckpt = 0)
 *   ckpt_pos_host  : host int32 [n_ckpt]; per sequence strictly increasing token
 *                    counts p, 1 <= p <= len: the state after exactly p tokens
 *   ckpt_slot_host : host int32 [n_ckpt]; page slot of each checkpoint, distinct,
 *                    0 <= slot < n_slots
 *   page_pool      : fp32 [n_slots, page_elems], page_elems >= H*dk*dv; a slot
 *                    is written in the pack layout and zero-padded
 *   workspace      : device memory of at least kda_chunk_prefill_workspace_size
 *                    bytes, 256-byte aligned; contents on entry are ignored.  It
 *                    holds the work list and, on the two-kernel path, one
 *                    record per (chunk, head),
 *                    written by a first kernel that handles all chunks at once
 *                    and read by the sequential one: T diag(beta) and
 *                    lower(A_qk) (chunk^2 elements each), k*g, q*g and
 *                    (k*g_n/g)^T (chunk*dk elements each) in in_dtype, and g_n
 *                    (dk fp32).  That is about
 *                    (T_tot / chunk + n_seqs + n_ckpt) * H * (2 chunk^2 +
 *                    3 chunk dk) * 2 bytes for bf16 (4.3 GB for 128k tokens,
 *                    H = 32, dk = 128, chunk 64).  On the fused path it holds
 *                    the work list and, where the call cuts long sequences
 *                    into segments, their buffers: the later segments' rows
 *                    of q mapped through their linear parts (bf16, H dk per
 *                    token of those segments), their checkpoints from zero
 *                    and from the identity, and a few states per segment.
 *                    The size function's figure covers that for any lengths
 *                    (about the size of q, plus 4 MiB per checkpoint at
 *                    H = 32, d = 128); a smaller workspace that still holds
 *                    the work list makes the call run without segments.
 *   err_flag       : device int32, may be NULL; set to 1 when a log-decay is
 *                    out of range (above); never cleared by the library
 * Sizes: T_tot < 2^31 tokens, H*dk*dv < 2^31, H*max(dk, dv) <= 2^24, and
 * (number of chunks) * H < 2^31.
 * The work list is copied from pageable host memory into the workspace
 * (hipMemcpyAsync), so the call may block the host while the runtime stages
 * those few kilobytes; everything else is enqueued.
 */
int kda_chunk_prefill_workspace_size(int32_t n_seqs, int64_t total_tokens, int32_t H,
                                     int32_t dk, int32_t dv, int32_t chunk, int64_t n_ckpt,
                                     kda_dtype in_dtype, size_t* bytes);

int kda_chunk_prefill(const void* q, const void* k, const void* v, const void* a,
                      const void* beta, kda_dtype in_dtype, int32_t H, int32_t dk,
                      int32_t dv, int32_t chunk, const int32_t* cu_seqlens_host,
                      int32_t n_seqs, const float* s0, void* o, float* s_final,
                      const int32_t* ckpt_cu_host, const int32_t* ckpt_pos_host,
                      const int32_t* ckpt_slot_host, int64_t n_ckpt, float* page_pool,
                      int64_t page_elems, int64_t n_slots, void* workspace,
                      size_t workspace_bytes, int32_t* err_flag, void* stream);

/*
 * kda_chunk_prefill_split — kda_chunk_prefill with an explicit number of
 * workgroups per (sequence, head) chain: the dv columns of the state are
 * independent in the recurrence (column j of S depends only on column j of
 * v), so a chain can be split into dv_split column tiles that each redo the
 * chunk's key-side work.  dv_split in {1, 2, 4, 8} with dv / dv_split one
 * of 16, 32 or 64, and also 128 for bf16 inputs at chunk 64 with dk a
 * multiple of 32 (the configurations served by the column-slab kernel, whose
 * default is one tile per head), or 0 to let the library choose, or -1 for a
 * tile width per sequence (32, 64 or 128 columns, from the library's cost
 * model, in one launch) where the column-slab kernel runs with dv = 128; the
 * automatic choice (0) takes that form where the model predicts it faster.
 * On the fused path (bf16, chunk 32, dk = dv = 128) the automatic choice
 * also cuts sequences whose chain would bound the call into segments
 * ([Serve demo] §1.7: a segment is the affine map S_end = A S_start + B of its
 * start state): a later segment's chains run from the zero state and from
 * the identity beside the first one, and the launch's last workgroups
 * compose the maps and correct the later segments' outputs and checkpoints
 * (the same result up to rounding).  dv_split = -n, 2 <= n <= 8, cuts every
 * sequence of at least n * 512 tokens into n segments (at most eight later
 * segments per call), with the widths of the automatic choice.
 * Other values: KDA_EUNSUPPORTED.
 */
int kda_chunk_prefill_split(const void* q, const void* k, const void* v, const void* a,
                            const void* beta, kda_dtype in_dtype, int32_t H, int32_t dk,
                            int32_t dv, int32_t chunk, const int32_t* cu_seqlens_host,
                            int32_t n_seqs, const float* s0, void* o, float* s_final,
                            const int32_t* ckpt_cu_host, const int32_t* ckpt_pos_host,
                            const int32_t* ckpt_slot_host, int64_t n_ckpt, float* page_pool,
                            int64_t page_elems, int64_t n_slots, void* workspace,
                            size_t workspace_bytes, int32_t dv_split, int32_t* err_flag,
                            void* stream);

/*
 * kda_chunk_prefill_plan — what kda_chunk_prefill_split would launch for these
 * shapes, without launching anything: tile_cols_out [n_seqs] (may be NULL)
 * receives the dv columns per workgroup of each sequence's chains, and
 * kernels_out (may be NULL) the NUL-terminated names of the kernels, cut to
 * kernels_bytes.  Validates the same arguments as the prefill (dtype, sizes,
 * cu_seqlens, checkpoint offsets and positions) with the same status codes.
 */
int kda_chunk_prefill_plan(kda_dtype in_dtype, int32_t H, int32_t dk, int32_t dv, int32_t chunk,
                           const int32_t* cu_seqlens_host, int32_t n_seqs,
                           const int32_t* ckpt_cu_host, const int32_t* ckpt_pos_host,
                           int64_t n_ckpt, int32_t dv_split, int32_t* tile_cols_out,
                           char* kernels_out, size_t kernels_bytes);

/*
 * kda_chunk_prefill_static — kda_chunk_prefill without a workspace argument,
 * for callers that cannot allocate device memory (code under graph capture,
 * tight serving loops, harnesses that forbid hipMalloc).  The workspace is a
 * device array of KDA_STATIC_SCRATCH_MB MiB inside the library, one per GPU
 * (held until the process ends); the call allocates no device memory and
 * calls no allocating routine.  A call whose workspace need (that of
 * kda_chunk_prefill for the same arguments) exceeds the array is refused
 * with KDA_EWORKSPACE before anything is enqueued.  The fused path (bf16,
 * chunk 32, dk 128) needs only its work list (about 50 KB for 16 sequences,
 * H = 32), and cuts long sequences into segments only where the array also
 * holds their buffers (else it runs them whole); the two-kernel path also
 * needs its chunk records (66 KB per
 * chunk and head at chunk 64, dk 128), so there it serves prefills of about
 * a thousand (chunk, head) pairs.  Every call on one GPU uses that GPU's one
 * array: calls that overlap on one GPU (other streams or host threads) race,
 * and must be serialized by the caller.  Each call clears what must start at
 * zero (its work list is rewritten from the host every call).
 */
#define KDA_STATIC_SCRATCH_MB 64
int kda_chunk_prefill_static(const void* q, const void* k, const void* v, const void* a,
                             const void* beta, kda_dtype in_dtype, int32_t H, int32_t dk,
                             int32_t dv, int32_t chunk, const int32_t* cu_seqlens_host,
                             int32_t n_seqs, const float* s0, void* o, float* s_final,
                             const int32_t* ckpt_cu_host, const int32_t* ckpt_pos_host,
                             const int32_t* ckpt_slot_host, int64_t n_ckpt, float* page_pool,
                             int64_t page_elems, int64_t n_slots, int32_t* err_flag, void* stream);

/* Size in bytes of the static workspace of kda_chunk_prefill_static. */
size_t kda_static_scratch_bytes(void);

/*
 * kda_chunk_prefill_gated — kda_chunk_prefill_split with the gate fused in
 * (the [KDA cache] page's vLLM path calls its prefill "chunk_kda_with_fused_gate"):
 * z_a [T_tot, H, dk] and z_b [T_tot, H] (in_dtype) are gate logits, and the
 * prefill uses a = g_min * sigmoid(z_a), beta = sigmoid(z_b) ([Serve demo]
 * §1.3), computed in fp32 as the logits are loaded.  g_min finite and <= 0.
 * The decay bound of kda_chunk_prefill applies to the gated a: g_min below
 * -160/chunk is refused (KDA_EUNSUPPORTED), and a logit that makes a NaN
 * raises *err_flag as for kda_chunk_prefill.  Everything else is as for
 * kda_chunk_prefill_split.
 */
int kda_chunk_prefill_gated(const void* q, const void* k, const void* v, const void* z_a,
                            const void* z_b, float g_min, kda_dtype in_dtype, int32_t H,
                            int32_t dk, int32_t dv, int32_t chunk, const int32_t* cu_seqlens_host,
                            int32_t n_seqs, const float* s0, void* o, float* s_final,
                            const int32_t* ckpt_cu_host, const int32_t* ckpt_pos_host,
                            const int32_t* ckpt_slot_host, int64_t n_ckpt, float* page_pool,
                            int64_t page_elems, int64_t n_slots, void* workspace,
                            size_t workspace_bytes, int32_t dv_split, int32_t* err_flag,
                            void* stream);

/*
 * Segment summaries for context-parallel prefill ([Serve demo] §7.2 "KCP 前缀扫描",
 * §1.7: what a segment of a long sequence passes on has a size independent of
 * its length).  Each token maps the state affinely,
 *   S -> (I - beta k k^T) diag(exp(a)) S + beta k v^T,
 * so a segment maps its start state to its end state as S_end = A S_start + B.
 *
 * kda_segment_summary — (A, B) of every segment of a token-packed input.
 *   k, a : [T_tot, H, dk]   v : [T_tot, H, dv]   beta : [T_tot, H]   (in_dtype)
 *   cu_seg_host : host int32 [n_seg + 1], segment boundaries as for cu_seqlens
 *   A_out : [n_seg, H, dk, dk] fp32, the linear part (identity for an empty segment)
 *   B_out : [n_seg, H, dk, dv] fp32, the end state from the zero start state
 *   workspace : at least kda_segment_summary_workspace_size bytes, 256-byte aligned
 * chunk, the decay bound (here a precondition: the summary does not check
 * it), dtypes and size limits are those of kda_chunk_prefill (same chunk form: B is the prefill's final state from s0 = 0, and A is the
 * same propagation run from the identity with v = 0), plus H*dk*dk < 2^31.
 * Outputs must not overlap the inputs or each other (KDA_EALIAS).
 */
int kda_segment_summary_workspace_size(int32_t n_seg, int64_t total_tokens, int32_t H,
                                       int32_t dk, int32_t dv, int32_t chunk,
                                       kda_dtype in_dtype, size_t* bytes);

int kda_segment_summary(const void* k, const void* v, const void* a, const void* beta,
                        kda_dtype in_dtype, int32_t H, int32_t dk, int32_t dv, int32_t chunk,
                        const int32_t* cu_seg_host, int32_t n_seg, float* A_out, float* B_out,
                        void* workspace, size_t workspace_bytes, void* stream);

/*
 * kda_compose_segments — the exclusive scan of segment maps under
 * (A2, B2) o (A1, B1) = (A2 A1, A2 B1 + B2): the start state of every segment
 * of one sequence, given the sequence's start state.
 *   A : [n_seg, H, dk, dk] fp32, 16-byte aligned   B : [n_seg, H, dk, dv] fp32
 *   s_in     : [H, dk, dv] fp32 start state of segment 0, or NULL for zero
 *   s_starts : [n_seg, H, dk, dv] fp32; s_starts[0] = s_in,
 *              s_starts[i+1] = A[i] s_starts[i] + B[i]
 *   s_end    : [H, dk, dv] fp32 or NULL; A[n-1] s_starts[n-1] + B[n-1]
 *              (s_in when n_seg = 0)
 * fp32 arithmetic, sums in a fixed order (deterministic).  Running
 * kda_chunk_prefill over the segments as sequences with s0 = s_starts gives
 * the outputs and states of one pass over the whole sequence.
 */
int kda_compose_segments(const float* A, const float* B, int32_t n_seg, int32_t H, int32_t dk,
                         int32_t dv, const float* s_in, float* s_starts, float* s_end,
                         void* stream);

/*
 * The front end: from a layer's projections to the recurrence inputs, and the
 * convolution window a checkpoint keeps next to the recurrent state
 * ([KDA cache] "KDA 的递推与充分状态": projection, causal short convolution,
 * activation, then L2Norm of Q and K, so the recurrent matrix alone cannot
 * continue the next token; its checkpoint section: the convolution checkpoint
 * is the last kernel_size - 1 rows of mixed_qkv before the boundary;
 * [Serve demo] §1.3: a = g_min * sigmoid(.), beta = sigmoid(.)).  Readings:
 *   - mixed rows x hold, per token, the q channels of all heads, then the k
 *     channels, then the v channels: C = H*(2*dk + dv), head-major in a part;
 *   - the convolution is depthwise and causal, kernel size K (1..4), weights
 *     conv_w [C, K] with conv_w[c][K-1] on the current token, no bias:
 *       u[t][c] = sum_j conv_w[c][j] * x[t-(K-1)+j][c];
 *   - then SiLU, u * sigmoid(u), on all parts;
 *   - q and k are divided per (token, head) by sqrt(sum over dk of u^2 + 1e-6);
 *   - a = g_min * sigmoid(z_a) per key channel, beta = sigmoid(z_b) per head.
 * A window is [K-1, C]: the K-1 raw rows before a boundary, oldest first,
 * in dtype (rows before a fresh sequence are zero).  Arithmetic is fp32;
 * outputs are rounded to dtype.
 *
 * kda_front_end — token-packed sequences.
 *   x : [T_tot, C]   z_a : [T_tot, H, dk]   z_b : [T_tot, H]   conv_w : [C, K]
 *   cu_seqlens_host : host int32 [n_seqs + 1] as for kda_chunk_prefill
 *   win_in  : [n_seqs, K-1, C] windows carried into the sequences, or NULL (zero)
 *   win_out : [n_seqs, K-1, C] the window after each sequence, or NULL
 *   checkpoints (ckpt_cu/pos/slot as for kda_chunk_prefill): the window
 *     after p tokens goes into slot ckpt_slot of conv_pool [n_slots,
 *     conv_elems] (dtype), conv_elems >= (K-1)*C, the rest of the slot zero;
 *     the same slot index as the state's page keeps the two halves of one
 *     checkpoint together
 *   q, k, a : [T_tot, H, dk]   v : [T_tot, H, dv]   beta : [T_tot, H]  (dtype)
 *   workspace : kda_front_end_workspace_size bytes, 16-byte aligned
 * x, z_a, win_in, q, k, v, a 16-byte aligned (rows move in 16-byte pieces).
 * Outputs must not overlap the inputs or each other (KDA_EALIAS).
 */
int kda_front_end_workspace_size(int32_t n_seqs, int64_t total_tokens, int64_t n_ckpt,
                                 size_t* bytes);

int kda_front_end(const void* x, const void* z_a, const void* z_b, const void* conv_w,
                  kda_dtype dtype, int32_t H, int32_t dk, int32_t dv, int32_t K, float g_min,
                  const int32_t* cu_seqlens_host, int32_t n_seqs, const void* win_in,
                  void* win_out, const int32_t* ckpt_cu_host, const int32_t* ckpt_pos_host,
                  const int32_t* ckpt_slot_host, int64_t n_ckpt, void* conv_pool,
                  int64_t conv_elems, int64_t n_slots, void* q, void* k, void* v, void* a,
                  void* beta, void* workspace, size_t workspace_bytes, void* stream);

/*
 * kda_front_end_step — one decode token per session, the window updated IN
 * PLACE (it supplies the K-1 rows before the token and comes back shifted by
 * one row, the token's raw row last).  x, z_a, window, q, k, v, a 16-byte
 * aligned.
 *   x : [B, C]   z_a : [B, H, dk]   z_b : [B, H]   conv_w : [C, K]
 *   window : [B, K-1, C] (dtype), read and overwritten (may be NULL when K = 1)
 *   q, k, a : [B, H, dk]   v : [B, H, dv]   beta : [B, H]
 */
int kda_front_end_step(const void* x, const void* z_a, const void* z_b, const void* conv_w,
                       kda_dtype dtype, int32_t B, int32_t H, int32_t dk, int32_t dv, int32_t K,
                       float g_min, void* window, void* q, void* k, void* v, void* a, void* beta,
                       void* stream);

/*
 * The raw-input ring ([Serve demo] Tab 4 "ReplaySSM", §7.1-7.3: during
 * verification each draft step's raw inputs (q, k, v, g, beta) are written,
 * as they arrive, into a per-slot ring window; once full a push overwrites
 * the oldest entry; window() returns the held entries oldest first in the
 * draft-projection layout (draft, B, H, D), row i the i-th entry; commit
 * replays the accepted prefix with kda_verify_and_replay, the same engine as
 * the batch path, and the ring starts over (kda_ring_reset)).  Rollback by
 * full state snapshots (route A of [Serve demo] §1.1) needs no new call: it is
 * kda_pack_heads of the state after every step and kda_unpack_heads of the
 * accepted one.
 *
 * A ring is caller-owned device memory described by kda_ring:
 *   q, k, a : [n_slots, capacity, H, dk]   v : [n_slots, capacity, H, dv]
 *   beta    : [n_slots, capacity, H]      (dtype; each 16-byte aligned)
 *   count   : int32 [n_slots], pushes since the last reset (zero it once
 *             when the ring is created)
 * Slot values live on the device: out-of-range slots are skipped and raise
 * *err_flag (when not NULL).  The slots of one call must be distinct.
 */
#define KDA_RING_MAX_CAPACITY 1024

typedef struct {
  void *q, *k, *v, *a, *beta;
  int32_t* count;
  int64_t n_slots;
  int32_t capacity, H, dk, dv;
  kda_dtype dtype;
} kda_ring;

/* kda_ring_push — append one draft step: entry b (q, k, a [B, H, dk],
 * v [B, H, dv], beta [B, H], 16-byte aligned, ring dtype) goes to slot slot[b]
 * at position count % capacity, then count[slot[b]] += 1. */
int kda_ring_push(const kda_ring* ring, const int32_t* slot, int32_t B, const void* q,
                  const void* k, const void* v, const void* a, const void* beta,
                  int32_t* err_flag, void* stream);

/* kda_ring_window — the windows of B slots, oldest first: q, k, a
 * [capacity, B, H, dk], v [capacity, B, H, dv], beta [capacity, B, H]
 * (16-byte aligned); rows past the held entries are zero; n_valid [B] (may be
 * NULL) receives min(count, capacity). */
int kda_ring_window(const kda_ring* ring, const int32_t* slot, int32_t B, void* q, void* k,
                    void* v, void* a, void* beta, int32_t* n_valid, int32_t* err_flag,
                    void* stream);

/* kda_ring_reset — empty the rings of B slots (count = 0). */
int kda_ring_reset(const kda_ring* ring, const int32_t* slot, int32_t B, int32_t* err_flag,
                   void* stream);

#ifdef __cplusplus
}
#endif

#endif /* KDA_H */
