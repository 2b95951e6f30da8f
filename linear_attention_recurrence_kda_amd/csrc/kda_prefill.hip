// Chunked KDA prefill: the local kernel over every (chunk, head), then the
// propagation kernel over every (sequence, head, dv tile) chain (kernels in
// kda_prefill_kernels.hpp; the column-slab kernel in kda_slab.hip).
#include "kda_prefill_kernels.hpp"

namespace kda {
namespace {

template <int DK, typename InT>
hipError_t launch_dk(const PrefillArgs& a) {
  if (a.n_chunks > 0) {
    const hipError_t e = launch_local<DK, InT>(a);
    if (e != hipSuccess) return e;
  }
  // Slab-format records (bf16 inputs, chunk 64, dk a multiple of 32): the
  // column-slab kernel (kda_slab.hip).
  if (a.slab) return launch_slab_prop(a, 0);
  switch (a.dv / a.dv_tiles) {
    case 16: return launch_prop<DK, 16, InT, 0>(a);
    case 32: return launch_prop<DK, 32, InT, 0>(a);
    case 64: return launch_prop<DK, 64, InT, 0>(a);
  }
  return hipErrorInvalidValue;
}

template <typename InT>
hipError_t launch_in(const PrefillArgs& a) {
  switch (a.dk) {
    case 16: return launch_dk<16, InT>(a);
    case 32: return launch_dk<32, InT>(a);
    case 64: return launch_dk<64, InT>(a);
    case 128: return launch_dk<128, InT>(a);
  }
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_prefill(const PrefillArgs& a) {
  if (a.fused) return launch_fused(a);
  return a.bf16 ? launch_in<bf16raw>(a) : launch_in<float>(a);
}

}  // namespace kda
