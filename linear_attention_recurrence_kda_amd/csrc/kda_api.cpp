// The extern "C" entry points of include/kda.h: argument validation (all of
// it before the first enqueue, so a failing call writes nothing), the prefill
// work list, and dispatch to the kernel launchers.
#include "../../include/kda.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <numeric>
#include <string>
#include <unordered_set>
#include <vector>

#include "kda_hostutil.hpp"
#include "kda_internal.hpp"

using namespace kda_host;

extern "C" {

const char* kda_status_string(int status) {
  switch (status) {
    case KDA_OK: return "ok";
    case KDA_EINVAL: return "invalid argument";
    case KDA_EUNSUPPORTED: return "unsupported configuration";
    case KDA_EALIAS: return "output aliases a protected input";
    case KDA_EWORKSPACE: return "workspace missing or too small";
    case KDA_EHIP: return "HIP runtime error";
  }
  return "unknown status";
}

const char* kda_last_error(void) { return g_last_error.c_str(); }

double kda_snapshot_cost_ratio(int32_t H, int32_t dk, int32_t dv) {
  if (H <= 0 || dk <= 0 || dv <= 0) return -1.0;
  const double snap = static_cast<double>(H) * dk * dv;
  const double proj = static_cast<double>(H) * (3.0 * dk + dv + 1.0);
  return snap / proj;
}

int kda_decode_step_ex(const void* q, const void* k, const void* v, const void* a,
                       const void* beta, kda_dtype in_dtype, int32_t B, int32_t H, int32_t dk,
                       int32_t dv, kda_dtype state_dtype, void* state, void* o, void* stream) {
  if (!valid_dtype(in_dtype)) return fail(KDA_EINVAL, "in_dtype %d", static_cast<int>(in_dtype));
  if (!valid_dtype(state_dtype)) return fail(KDA_EINVAL, "state_dtype %d", static_cast<int>(state_dtype));
  if (B < 0 || H <= 0) return fail(KDA_EINVAL, "B=%d H=%d", B, H);
  if (!supported_dim(dk) || !supported_dim(dv))
    return fail(KDA_EUNSUPPORTED, "dk=%d dv=%d (supported: 16, 32, 64, 128)", dk, dv);
  if (B == 0) return ok();
  if (!q || !k || !v || !a || !beta || !state || !o) return fail(KDA_EINVAL, "null pointer");
  if (!aligned16(state)) return fail(KDA_EINVAL, "state must be 16-byte aligned");
  const size_t es = elem_size(in_dtype), bh = static_cast<size_t>(B) * H;
  const std::vector<Range> ins = {{q, bh * dk * es, "q"},   {k, bh * dk * es, "k"},
                                  {v, bh * dv * es, "v"},   {a, bh * dk * es, "a"},
                                  {beta, bh * es, "beta"}};
  const size_t ss = elem_size(state_dtype);
  int st = check_disjoint({{state, bh * dk * dv * ss, "state"}, {o, bh * dv * es, "o"}}, ins);
  if (st) return st;
  kda::SweepArgs p{};
  p.s_in = state;
  p.s_out = state;
  p.state_bf16 = state_dtype == KDA_BF16;
  p.q = q; p.k = k; p.v = v; p.a = a; p.beta = beta;
  p.n_accepted = nullptr;
  p.t_draft = 1; p.B = B; p.H = H; p.dk = dk; p.dv = dv;
  p.bf16 = in_dtype == KDA_BF16;
  p.o = o; p.o_steps = 1;
  p.err_flag = nullptr;
  p.stream = static_cast<hipStream_t>(stream);
  return hip_status(kda::launch_sweep(p), "decode launch");
}

int kda_decode_step(const void* q, const void* k, const void* v, const void* a,
                    const void* beta, kda_dtype in_dtype, int32_t B, int32_t H, int32_t dk,
                    int32_t dv, float* state, void* o, void* stream) {
  return kda_decode_step_ex(q, k, v, a, beta, in_dtype, B, H, dk, dv, KDA_F32, state, o, stream);
}

int kda_verify_and_replay_ex(const void* committed, const void* q, const void* k, const void* v,
                             const void* a, const void* beta, kda_dtype in_dtype,
                             const int32_t* n_accepted, int32_t B, int32_t H, int32_t dk,
                             int32_t dv, int32_t t_draft, kda_dtype state_dtype, void* s_new,
                             void* o, int32_t* err_flag, void* stream) {
  if (!valid_dtype(in_dtype)) return fail(KDA_EINVAL, "in_dtype %d", static_cast<int>(in_dtype));
  if (!valid_dtype(state_dtype)) return fail(KDA_EINVAL, "state_dtype %d", static_cast<int>(state_dtype));
  if (B < 0 || H <= 0 || t_draft <= 0) return fail(KDA_EINVAL, "B=%d H=%d t_draft=%d", B, H, t_draft);
  if (!supported_dim(dk) || !supported_dim(dv))
    return fail(KDA_EUNSUPPORTED, "dk=%d dv=%d (supported: 16, 32, 64, 128)", dk, dv);
  if (B == 0) return ok();
  if (!committed || !q || !k || !v || !a || !beta || !n_accepted || !s_new || !o)
    return fail(KDA_EINVAL, "null pointer");
  if (!aligned16(committed) || !aligned16(s_new))
    return fail(KDA_EINVAL, "committed and s_new must be 16-byte aligned");
  const size_t es = elem_size(in_dtype), bh = static_cast<size_t>(B) * H;
  const size_t tb = static_cast<size_t>(t_draft) * bh;
  const size_t ss = elem_size(state_dtype);
  const std::vector<Range> ins = {
      {committed, bh * dk * dv * ss, "committed"}, {q, tb * dk * es, "q"}, {k, tb * dk * es, "k"},
      {v, tb * dv * es, "v"}, {a, tb * dk * es, "a"}, {beta, tb * es, "beta"},
      {n_accepted, static_cast<size_t>(B) * 4, "n_accepted"}};
  std::vector<Range> outs = {{s_new, bh * dk * dv * ss, "s_new"}, {o, tb * dv * es, "o"}};
  if (err_flag) outs.push_back({err_flag, 4, "err_flag"});
  int st = check_disjoint(outs, ins);
  if (st) return st;
  kda::SweepArgs p{};
  p.s_in = committed;
  p.s_out = s_new;
  p.state_bf16 = state_dtype == KDA_BF16;
  p.q = q; p.k = k; p.v = v; p.a = a; p.beta = beta;
  p.n_accepted = n_accepted;
  p.t_draft = t_draft; p.B = B; p.H = H; p.dk = dk; p.dv = dv;
  p.bf16 = in_dtype == KDA_BF16;
  p.o = o; p.o_steps = t_draft;
  p.err_flag = err_flag;
  p.stream = static_cast<hipStream_t>(stream);
  return hip_status(kda::launch_sweep(p), "replay launch");
}

int kda_verify_and_replay(const float* committed, const void* q, const void* k, const void* v,
                          const void* a, const void* beta, kda_dtype in_dtype,
                          const int32_t* n_accepted, int32_t B, int32_t H, int32_t dk,
                          int32_t dv, int32_t t_draft, float* s_new, void* o,
                          int32_t* err_flag, void* stream) {
  return kda_verify_and_replay_ex(committed, q, k, v, a, beta, in_dtype, n_accepted, B, H, dk, dv,
                                  t_draft, KDA_F32, s_new, o, err_flag, stream);
}

static int pack_common(const void* src, void* dst, kda_dtype state_dtype, kda_layout layout,
                       int32_t B, int32_t H, int32_t dk, int32_t dv, const int32_t* slot,
                       int64_t page_elems, int64_t n_slots, int32_t* err_flag, bool unpack,
                       void* stream) {
  if (!valid_dtype(state_dtype)) return fail(KDA_EINVAL, "state_dtype %d", static_cast<int>(state_dtype));
  if (layout != KDA_LAYOUT_KV && layout != KDA_LAYOUT_VK)
    return fail(KDA_EINVAL, "layout %d", static_cast<int>(layout));
  if (B < 0 || H <= 0 || n_slots < 0) return fail(KDA_EINVAL, "B=%d H=%d n_slots=%lld", B, H,
                                                  static_cast<long long>(n_slots));
  if (!supported_dim(dk) || !supported_dim(dv))
    return fail(KDA_EUNSUPPORTED, "dk=%d dv=%d (supported: 16, 32, 64, 128)", dk, dv);
  const int64_t hkv = static_cast<int64_t>(H) * dk * dv;
  if (page_elems < hkv) return fail(KDA_EINVAL, "page_elems %lld < H*dk*dv %lld",
                                    static_cast<long long>(page_elems), static_cast<long long>(hkv));
  const size_t ss = elem_size(state_dtype);
  if (page_elems % static_cast<int64_t>(16 / ss))
    return fail(KDA_EUNSUPPORTED, "page_elems must be a multiple of %d (16 bytes)", static_cast<int>(16 / ss));
  if (B > kMaxGridY || H > kMaxGridY) return fail(KDA_EUNSUPPORTED, "B or H above 65535");
  if (B == 0) return ok();
  if (!src || !dst || !slot) return fail(KDA_EINVAL, "null pointer");
  if (!aligned16(src) || !aligned16(dst)) return fail(KDA_EINVAL, "buffers must be 16-byte aligned");
  const size_t state_bytes = static_cast<size_t>(B) * hkv * ss;
  const size_t pool_bytes = static_cast<size_t>(n_slots) * page_elems * ss;
  const Range state_r{unpack ? dst : src, state_bytes, "state"};
  const Range pool_r{unpack ? src : dst, pool_bytes, "page_pool"};
  const Range slot_r{slot, static_cast<size_t>(B) * 4, "slot"};
  std::vector<Range> outs = {unpack ? state_r : pool_r};
  if (err_flag) outs.push_back({err_flag, 4, "err_flag"});
  int st = check_disjoint(outs, {unpack ? pool_r : state_r, slot_r});
  if (st) return st;
  kda::PackArgs p{};
  p.src = src; p.dst = dst; p.es = static_cast<int>(ss); p.slot = slot;
  p.B = B; p.H = H; p.dk = dk; p.dv = dv;
  p.vk = layout == KDA_LAYOUT_VK;
  p.unpack = unpack;
  p.page_elems = page_elems; p.n_slots = n_slots;
  p.err_flag = err_flag;
  p.stream = static_cast<hipStream_t>(stream);
  return hip_status(kda::launch_pack(p), unpack ? "unpack launch" : "pack launch");
}

int kda_pack_heads(const float* state, kda_layout src_layout, int32_t B, int32_t H, int32_t dk,
                   int32_t dv, const int32_t* slot, float* page_pool, int64_t page_elems,
                   int64_t n_slots, int32_t* err_flag, void* stream) {
  return pack_common(state, page_pool, KDA_F32, src_layout, B, H, dk, dv, slot, page_elems,
                     n_slots, err_flag, false, stream);
}

int kda_unpack_heads(const float* page_pool, int64_t page_elems, int64_t n_slots,
                     const int32_t* slot, int32_t B, int32_t H, int32_t dk, int32_t dv,
                     kda_layout dst_layout, float* state, int32_t* err_flag, void* stream) {
  return pack_common(page_pool, state, KDA_F32, dst_layout, B, H, dk, dv, slot, page_elems,
                     n_slots, err_flag, true, stream);
}

int kda_pack_heads_ex(const void* state, kda_dtype state_dtype, kda_layout src_layout, int32_t B,
                      int32_t H, int32_t dk, int32_t dv, const int32_t* slot, void* page_pool,
                      int64_t page_elems, int64_t n_slots, int32_t* err_flag, void* stream) {
  return pack_common(state, page_pool, state_dtype, src_layout, B, H, dk, dv, slot, page_elems,
                     n_slots, err_flag, false, stream);
}

int kda_unpack_heads_ex(const void* page_pool, kda_dtype state_dtype, int64_t page_elems,
                        int64_t n_slots, const int32_t* slot, int32_t B, int32_t H, int32_t dk,
                        int32_t dv, kda_layout dst_layout, void* state, int32_t* err_flag,
                        void* stream) {
  return pack_common(page_pool, state, state_dtype, dst_layout, B, H, dk, dv, slot, page_elems,
                     n_slots, err_flag, true, stream);
}

int kda_compose_segments(const float* A, const float* B, int32_t n_seg, int32_t H, int32_t dk,
                         int32_t dv, const float* s_in, float* s_starts, float* s_end,
                         void* stream) {
  if (n_seg < 0 || H <= 0) return fail(KDA_EINVAL, "n_seg=%d H=%d", n_seg, H);
  if (!supported_dim(dk) || !supported_dim(dv))
    return fail(KDA_EUNSUPPORTED, "dk=%d dv=%d (supported: 16, 32, 64, 128)", dk, dv);
  const int64_t hkv = static_cast<int64_t>(H) * dk * dv, hkk = static_cast<int64_t>(H) * dk * dk;
  if (std::max(hkv, hkk) >= (int64_t{1} << 31))
    return fail(KDA_EUNSUPPORTED, "H*dk*max(dk, dv) must be below 2^31");
  if (n_seg > 0 && (!A || !B || !s_starts)) return fail(KDA_EINVAL, "A, B and s_starts must not be null");
  if (n_seg == 0 && !s_end) return ok();
  if (!aligned16(A)) return fail(KDA_EINVAL, "A must be 16-byte aligned");
  const size_t n = static_cast<size_t>(n_seg), sb = static_cast<size_t>(hkv) * 4;
  const std::vector<Range> ins = {{A, n * static_cast<size_t>(hkk) * 4, "A"}, {B, n * sb, "B"},
                                  {s_in, s_in ? sb : 0, "s_in"}};
  const std::vector<Range> outs = {{s_starts, n * sb, "s_starts"}, {s_end, s_end ? sb : 0, "s_end"}};
  const int st = check_disjoint(outs, ins);
  if (st) return st;
  kda::ComposeArgs p{A, B, s_in, s_starts, s_end, n_seg, H, dk, dv, static_cast<hipStream_t>(stream)};
  return hip_status(kda::launch_compose(p), "compose launch");
}

}  // extern "C"
