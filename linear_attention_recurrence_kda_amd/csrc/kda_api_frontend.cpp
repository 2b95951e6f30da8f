// extern "C" front-end entry points: validation of every host-visible
// argument, the tile and boundary tables (built on the host, copied into the
// caller's workspace), and the launches.
#include <hip/hip_runtime.h>

#include <cmath>
#include <unordered_set>
#include <vector>

#include "kda_hostutil.hpp"
#include "kda_internal.hpp"

using namespace kda_host;

namespace {

constexpr int kFrontRows = 64;  // tokens per tile of the front-end kernel
constexpr int kMaxConv = 4;     // largest convolution kernel size

// Tiles never cross a sequence end: at most T / rows + N of them.
int64_t max_tiles(int32_t n_seqs, int64_t total_tokens) { return total_tokens / kFrontRows + n_seqs; }
size_t front_ints(int32_t n_seqs, int64_t total_tokens, int64_t n_ckpt) {
  return static_cast<size_t>(4 * max_tiles(n_seqs, total_tokens) + 4 * (n_seqs + n_ckpt));
}

int check_common(kda_dtype dtype, int32_t H, int32_t dk, int32_t dv, int32_t K, float g_min) {
  if (!valid_dtype(dtype)) return fail(KDA_EINVAL, "dtype %d", static_cast<int>(dtype));
  if (H <= 0) return fail(KDA_EINVAL, "H=%d", H);
  if (!supported_dim(dk) || !supported_dim(dv))
    return fail(KDA_EUNSUPPORTED, "dk=%d dv=%d (supported: 16, 32, 64, 128)", dk, dv);
  if (K < 1 || K > kMaxConv) return fail(KDA_EUNSUPPORTED, "kernel size %d (1..%d)", K, kMaxConv);
  if (!std::isfinite(g_min) || g_min > 0.f) return fail(KDA_EINVAL, "g_min must be finite and <= 0");
  if (static_cast<int64_t>(H) * (2 * dk + dv) >= (int64_t{1} << 31))
    return fail(KDA_EUNSUPPORTED, "H*(2*dk+dv) must be below 2^31");
  return KDA_OK;
}

}  // namespace

extern "C" {

int kda_front_end_workspace_size(int32_t n_seqs, int64_t total_tokens, int64_t n_ckpt,
                                 size_t* bytes) {
  if (!bytes) return fail(KDA_EINVAL, "bytes is null");
  if (n_seqs < 0 || total_tokens < 0 || n_ckpt < 0)
    return fail(KDA_EINVAL, "n_seqs=%d total_tokens=%lld n_ckpt=%lld", n_seqs,
                static_cast<long long>(total_tokens), static_cast<long long>(n_ckpt));
  *bytes = front_ints(n_seqs, total_tokens, n_ckpt) * 4;
  return ok();
}

int kda_front_end(const void* x, const void* z_a, const void* z_b, const void* conv_w,
                  kda_dtype dtype, int32_t H, int32_t dk, int32_t dv, int32_t K, float g_min,
                  const int32_t* cu, int32_t n_seqs, const void* win_in, void* win_out,
                  const int32_t* ck_cu, const int32_t* ck_pos, const int32_t* ck_slot,
                  int64_t n_ckpt, void* conv_pool, int64_t conv_elems, int64_t n_slots, void* q,
                  void* k, void* v, void* a, void* beta, void* workspace, size_t workspace_bytes,
                  void* stream) {
  int st = check_common(dtype, H, dk, dv, K, g_min);
  if (st) return st;
  if (n_seqs < 0 || n_ckpt < 0) return fail(KDA_EINVAL, "n_seqs=%d n_ckpt=%lld", n_seqs,
                                            static_cast<long long>(n_ckpt));
  if (n_seqs == 0) return ok();
  if (!cu) return fail(KDA_EINVAL, "cu_seqlens is null");
  if (cu[0] != 0) return fail(KDA_EINVAL, "cu_seqlens[0] = %d, must be 0", cu[0]);
  for (int32_t i = 0; i < n_seqs; ++i)
    if (cu[i + 1] < cu[i]) return fail(KDA_EINVAL, "cu_seqlens decreases at %d", i);
  const int64_t T = cu[n_seqs];
  const int64_t C = static_cast<int64_t>(H) * (2 * dk + dv);
  const int64_t wrow = static_cast<int64_t>(K - 1) * C;  // elements of one window

  // Checkpoints.
  if (n_ckpt > 0 && (!ck_cu || !ck_pos || !ck_slot || !conv_pool))
    return fail(KDA_EINVAL, "checkpoints need ckpt_cu, ckpt_pos, ckpt_slot and conv_pool");
  if (ck_cu) {
    if (ck_cu[0] != 0 || ck_cu[n_seqs] != n_ckpt)
      return fail(KDA_EINVAL, "ckpt_cu must start at 0 and end at n_ckpt");
    for (int32_t i = 0; i < n_seqs; ++i) {
      if (ck_cu[i + 1] < ck_cu[i]) return fail(KDA_EINVAL, "ckpt_cu decreases at %d", i);
      const int32_t len = cu[i + 1] - cu[i];
      for (int32_t c = ck_cu[i]; c < ck_cu[i + 1]; ++c) {
        if (ck_pos[c] < 1 || ck_pos[c] > len)
          return fail(KDA_EINVAL, "checkpoint %d of sequence %d at %d outside 1..%d", c - ck_cu[i],
                      i, ck_pos[c], len);
      }
    }
  } else if (n_ckpt != 0) {
    return fail(KDA_EINVAL, "n_ckpt > 0 without ckpt_cu");
  }
  if (n_ckpt > 0) {
    if (conv_elems < wrow)
      return fail(KDA_EINVAL, "conv_elems %lld < (K-1)*C %lld", static_cast<long long>(conv_elems),
                  static_cast<long long>(wrow));
    std::unordered_set<int32_t> seen;
    for (int64_t c = 0; c < n_ckpt; ++c) {
      if (ck_slot[c] < 0 || ck_slot[c] >= n_slots)
        return fail(KDA_EINVAL, "checkpoint slot %d outside 0..%lld", ck_slot[c],
                    static_cast<long long>(n_slots) - 1);
      if (!seen.insert(ck_slot[c]).second) return fail(KDA_EINVAL, "checkpoint slot %d repeated", ck_slot[c]);
    }
  }

  // Buffers.
  const size_t es = elem_size(dtype);
  if (T > 0 && (!x || !z_a || !z_b || !conv_w || !q || !k || !v || !a || !beta))
    return fail(KDA_EINVAL, "null input or output");
  // Rows are read and written in 16-byte pieces.
  for (const void* ptr : {x, z_a, win_in, static_cast<const void*>(q), static_cast<const void*>(k),
                          static_cast<const void*>(v), static_cast<const void*>(a)})
    if (!aligned16(ptr)) return fail(KDA_EINVAL, "x, z_a, win_in, q, k, v, a must be 16-byte aligned");
  const int64_t n_tiles_max = max_tiles(n_seqs, T);
  if (n_tiles_max * H >= (int64_t{1} << 31)) return fail(KDA_EUNSUPPORTED, "too many (tile, head) pairs");
  const size_t need = front_ints(n_seqs, T, n_ckpt) * 4;
  if (!workspace || workspace_bytes < need)
    return fail(KDA_EWORKSPACE, "workspace of %zu bytes, need %zu", workspace_bytes, need);
  if (reinterpret_cast<uintptr_t>(workspace) % 16) return fail(KDA_EINVAL, "workspace must be 16-byte aligned");
  const size_t th = static_cast<size_t>(T) * H;
  const size_t wbytes = static_cast<size_t>(n_seqs) * wrow * es;
  const std::vector<Range> ins = {{x, static_cast<size_t>(T) * C * es, "x"},
                                  {z_a, th * dk * es, "z_a"},
                                  {z_b, th * es, "z_b"},
                                  {conv_w, static_cast<size_t>(C) * K * es, "conv_w"},
                                  {win_in, win_in ? wbytes : 0, "win_in"}};
  const std::vector<Range> outs = {
      {q, th * dk * es, "q"}, {k, th * dk * es, "k"}, {v, th * dv * es, "v"},
      {a, th * dk * es, "a"}, {beta, th * es, "beta"}, {win_out, win_out ? wbytes : 0, "win_out"},
      {conv_pool, n_ckpt > 0 ? static_cast<size_t>(n_slots) * conv_elems * es : 0, "conv_pool"},
      {workspace, need, "workspace"}};
  st = check_disjoint(outs, ins);
  if (st) return st;

  // Tiles and boundaries.
  std::vector<int32_t> work;
  work.reserve(front_ints(n_seqs, T, n_ckpt));
  int64_t n_tiles = 0;
  for (int32_t i = 0; i < n_seqs; ++i)
    for (int32_t t = cu[i]; t < cu[i + 1]; t += kFrontRows, ++n_tiles) {
      work.push_back(i);
      work.push_back(t);
      work.push_back(std::min(kFrontRows, cu[i + 1] - t));
      work.push_back(cu[i]);
    }
  const size_t bnd_off = work.size();
  int32_t n_bnd = 0;
  for (int32_t i = 0; i < n_seqs; ++i) {
    if (ck_cu)
      for (int32_t c = ck_cu[i]; c < ck_cu[i + 1]; ++c, ++n_bnd) {
        work.push_back(i);
        work.push_back(ck_pos[c]);
        work.push_back(ck_slot[c]);
        work.push_back(cu[i]);
      }
    if (win_out) {
      work.push_back(i);
      work.push_back(cu[i + 1] - cu[i]);
      work.push_back(-1);
      work.push_back(cu[i]);
      ++n_bnd;
    }
  }
  hipStream_t hs = static_cast<hipStream_t>(stream);
  if (!work.empty()) {
    // Pageable source: the runtime has consumed it when the call returns.
    const hipError_t e = hipMemcpyAsync(workspace, work.data(), work.size() * 4, hipMemcpyHostToDevice, hs);
    if (e != hipSuccess) return hip_status(e, "work list copy");
  }
  const int32_t* dwork = static_cast<const int32_t*>(workspace);
  if (n_tiles > 0) {
    kda::FrontParams p{};
    p.x = x; p.z_a = z_a; p.z_b = z_b; p.w = conv_w; p.win_in = win_in; p.win_step = nullptr;
    p.q = q; p.k = k; p.v = v; p.a = a; p.beta = beta;
    p.tiles = dwork;
    p.g_min = g_min;
    p.H = H; p.dk = dk; p.dv = dv; p.K = K; p.C = static_cast<int>(C);
    p.bf16 = dtype == KDA_BF16;
    p.stream = hs;
    st = hip_status(kda::launch_front(p, static_cast<int>(n_tiles), false), "front-end launch");
    if (st) return st;
  }
  kda::WindowParams wp{};
  wp.x = x; wp.win_in = win_in; wp.win_out = win_out; wp.pool = conv_pool;
  wp.pool_elems = conv_elems;
  wp.bnd = dwork + bnd_off;
  wp.n_bnd = n_bnd; wp.K = K; wp.C = static_cast<int>(C);
  wp.bf16 = dtype == KDA_BF16;
  wp.stream = hs;
  return hip_status(kda::launch_windows(wp), "window launch");
}

int kda_front_end_step(const void* x, const void* z_a, const void* z_b, const void* conv_w,
                       kda_dtype dtype, int32_t B, int32_t H, int32_t dk, int32_t dv, int32_t K,
                       float g_min, void* window, void* q, void* k, void* v, void* a, void* beta,
                       void* stream) {
  int st = check_common(dtype, H, dk, dv, K, g_min);
  if (st) return st;
  if (B < 0) return fail(KDA_EINVAL, "B=%d", B);
  if (B == 0) return ok();
  if (static_cast<int64_t>(B) * H >= (int64_t{1} << 31)) return fail(KDA_EUNSUPPORTED, "B*H too large");
  if (!x || !z_a || !z_b || !conv_w || !q || !k || !v || !a || !beta || (K > 1 && !window))
    return fail(KDA_EINVAL, "null input or output");
  const size_t es = elem_size(dtype);
  for (const void* ptr : {x, z_a, static_cast<const void*>(q), static_cast<const void*>(k),
                          static_cast<const void*>(v), static_cast<const void*>(a),
                          static_cast<const void*>(window)})
    if (!aligned16(ptr)) return fail(KDA_EINVAL, "x, z_a, window, q, k, v, a must be 16-byte aligned");
  const int64_t C = static_cast<int64_t>(H) * (2 * dk + dv);
  const size_t bh = static_cast<size_t>(B) * H;
  const std::vector<Range> ins = {{x, static_cast<size_t>(B) * C * es, "x"}, {z_a, bh * dk * es, "z_a"},
                                  {z_b, bh * es, "z_b"}, {conv_w, static_cast<size_t>(C) * K * es, "conv_w"}};
  const std::vector<Range> outs = {
      {q, bh * dk * es, "q"}, {k, bh * dk * es, "k"}, {v, bh * dv * es, "v"}, {a, bh * dk * es, "a"},
      {beta, bh * es, "beta"},
      {window, static_cast<size_t>(B) * (K - 1) * C * es, "window"}};
  st = check_disjoint(outs, ins);
  if (st) return st;
  kda::FrontParams p{};
  p.x = x; p.z_a = z_a; p.z_b = z_b; p.w = conv_w; p.win_in = window; p.win_step = window;
  p.q = q; p.k = k; p.v = v; p.a = a; p.beta = beta;
  p.tiles = nullptr;
  p.g_min = g_min;
  p.H = H; p.dk = dk; p.dv = dv; p.K = K; p.C = static_cast<int>(C);
  p.bf16 = dtype == KDA_BF16;
  p.stream = static_cast<hipStream_t>(stream);
  return hip_status(kda::launch_front(p, B, true), "front-end step launch");
}

}  // extern "C"
