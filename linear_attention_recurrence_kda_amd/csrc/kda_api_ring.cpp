// extern "C" entry points of the raw-input ring: validation of the ring
// description and of every host-visible argument, then the launches.
#include <hip/hip_runtime.h>

#include <vector>

#include "kda_hostutil.hpp"
#include "kda_internal.hpp"

using namespace kda_host;

namespace {

int check_ring(const kda_ring* r, kda::RingArgs* out, int32_t* err_flag, void* stream) {
  if (!r) return fail(KDA_EINVAL, "ring is null");
  if (!valid_dtype(r->dtype)) return fail(KDA_EINVAL, "ring dtype %d", static_cast<int>(r->dtype));
  if (r->H <= 0 || r->n_slots <= 0) return fail(KDA_EINVAL, "ring H=%d n_slots=%lld", r->H,
                                                static_cast<long long>(r->n_slots));
  if (!supported_dim(r->dk) || !supported_dim(r->dv))
    return fail(KDA_EUNSUPPORTED, "ring dk=%d dv=%d (supported: 16, 32, 64, 128)", r->dk, r->dv);
  if (r->capacity < 1 || r->capacity > KDA_RING_MAX_CAPACITY)
    return fail(KDA_EUNSUPPORTED, "ring capacity %d (1..%d)", r->capacity, KDA_RING_MAX_CAPACITY);
  if (r->n_slots >= (int64_t{1} << 31)) return fail(KDA_EUNSUPPORTED, "too many ring slots");
  const void* fields[5] = {r->q, r->k, r->v, r->a, r->beta};
  for (const void* f : fields)
    if (!f || !aligned16(f)) return fail(KDA_EINVAL, "ring arrays must be non-null and 16-byte aligned");
  if (!r->count) return fail(KDA_EINVAL, "ring count is null");
  const int64_t e[5] = {int64_t{r->H} * r->dk, int64_t{r->H} * r->dk, int64_t{r->H} * r->dv,
                        int64_t{r->H} * r->dk, int64_t{r->H}};
  const size_t es = elem_size(r->dtype);
  // The ring arrays and the counts must not overlap one another.
  std::vector<Range> parts;
  const char* names[5] = {"ring q", "ring k", "ring v", "ring a", "ring beta"};
  for (int f = 0; f < 5; ++f)
    parts.push_back({fields[f], static_cast<size_t>(r->n_slots) * r->capacity * e[f] * es, names[f]});
  parts.push_back({r->count, static_cast<size_t>(r->n_slots) * 4, "ring count"});
  int st = check_disjoint(parts, {});
  if (st) return st;
  kda::RingArgs a{};
  for (int f = 0; f < 5; ++f) {
    a.field[f] = const_cast<void*>(fields[f]);
    a.elems[f] = e[f];
  }
  a.count = r->count;
  a.n_slots = r->n_slots;
  a.capacity = r->capacity;
  a.es = static_cast<int>(es);
  a.err_flag = err_flag;
  a.stream = static_cast<hipStream_t>(stream);
  *out = a;
  return KDA_OK;
}

std::vector<Range> ring_ranges(const kda::RingArgs& a) {
  std::vector<Range> v;
  const char* names[5] = {"ring q", "ring k", "ring v", "ring a", "ring beta"};
  for (int f = 0; f < 5; ++f)
    v.push_back({a.field[f], static_cast<size_t>(a.n_slots) * a.capacity * a.elems[f] * a.es, names[f]});
  v.push_back({a.count, static_cast<size_t>(a.n_slots) * 4, "ring count"});
  return v;
}

}  // namespace

extern "C" {

int kda_ring_push(const kda_ring* ring, const int32_t* slot, int32_t B, const void* q,
                  const void* k, const void* v, const void* a, const void* beta,
                  int32_t* err_flag, void* stream) {
  kda::RingArgs r;
  int st = check_ring(ring, &r, err_flag, stream);
  if (st) return st;
  if (B < 0) return fail(KDA_EINVAL, "B=%d", B);
  if (B == 0) return ok();
  const void* in[5] = {q, k, v, a, beta};
  for (const void* p : in)
    if (!p || !aligned16(p)) return fail(KDA_EINVAL, "step inputs must be non-null and 16-byte aligned");
  if (!slot) return fail(KDA_EINVAL, "slot is null");
  std::vector<Range> ins;
  const char* names[5] = {"q", "k", "v", "a", "beta"};
  for (int f = 0; f < 5; ++f) ins.push_back({in[f], static_cast<size_t>(B) * r.elems[f] * r.es, names[f]});
  ins.push_back({slot, static_cast<size_t>(B) * 4, "slot"});
  std::vector<Range> outs = ring_ranges(r);
  if (err_flag) outs.push_back({err_flag, 4, "err_flag"});
  st = check_disjoint(outs, ins);
  if (st) return st;
  kda::RingStep s{};
  for (int f = 0; f < 5; ++f) s.field[f] = const_cast<void*>(in[f]);
  return hip_status(kda::launch_ring_push(r, slot, B, s), "ring push launch");
}

int kda_ring_window(const kda_ring* ring, const int32_t* slot, int32_t B, void* q, void* k, void* v,
                    void* a, void* beta, int32_t* n_valid, int32_t* err_flag, void* stream) {
  kda::RingArgs r;
  int st = check_ring(ring, &r, err_flag, stream);
  if (st) return st;
  if (B < 0) return fail(KDA_EINVAL, "B=%d", B);
  if (B == 0) return ok();
  void* out[5] = {q, k, v, a, beta};
  for (void* p : out)
    if (!p || !aligned16(p)) return fail(KDA_EINVAL, "window outputs must be non-null and 16-byte aligned");
  if (!slot) return fail(KDA_EINVAL, "slot is null");
  std::vector<Range> outs;
  const char* names[5] = {"q", "k", "v", "a", "beta"};
  for (int f = 0; f < 5; ++f)
    outs.push_back({out[f], static_cast<size_t>(r.capacity) * B * r.elems[f] * r.es, names[f]});
  if (n_valid) outs.push_back({n_valid, static_cast<size_t>(B) * 4, "n_valid"});
  if (err_flag) outs.push_back({err_flag, 4, "err_flag"});
  std::vector<Range> ins = ring_ranges(r);
  ins.push_back({slot, static_cast<size_t>(B) * 4, "slot"});
  st = check_disjoint(outs, ins);
  if (st) return st;
  kda::RingStep s{};
  for (int f = 0; f < 5; ++f) s.field[f] = out[f];
  return hip_status(kda::launch_ring_window(r, slot, B, s, n_valid), "ring window launch");
}

int kda_ring_reset(const kda_ring* ring, const int32_t* slot, int32_t B, int32_t* err_flag,
                   void* stream) {
  kda::RingArgs r;
  int st = check_ring(ring, &r, err_flag, stream);
  if (st) return st;
  if (B < 0) return fail(KDA_EINVAL, "B=%d", B);
  if (B == 0) return ok();
  if (!slot) return fail(KDA_EINVAL, "slot is null");
  return hip_status(kda::launch_ring_reset(r, slot, B), "ring reset launch");
}

}  // extern "C"
