// The column-slab propagation kernel (kda_prefill_slab.hpp), instantiated
// for dk = 32, 64, 128 and the three modes.  Built on its own with MFMA
// results kept in ordinary vector registers (the kernel scales and rounds
// them with vector ALU instructions every chunk, which cannot read the
// accumulation registers).
#include "kda_prefill_slab.hpp"

namespace kda {

hipError_t launch_slab_prop(const PrefillArgs& a, int mode) {
  if (mode == 0 && a.n_wg > 0) {
    switch (a.dk) {
      case 32: return launch_slab_mixed<32>(a);
      case 64: return launch_slab_mixed<64>(a);
      case 128: return launch_slab_mixed<128>(a);
    }
    return hipErrorInvalidValue;
  }
  switch (a.dk) {
    case 32:
      return mode == 0 ? launch_slab<32, 0>(a) : mode == 1 ? launch_slab<32, 1>(a) : launch_slab<32, 2>(a);
    case 64:
      return mode == 0 ? launch_slab<64, 0>(a) : mode == 1 ? launch_slab<64, 1>(a) : launch_slab<64, 2>(a);
    case 128:
      return mode == 0 ? launch_slab<128, 0>(a) : mode == 1 ? launch_slab<128, 1>(a) : launch_slab<128, 2>(a);
  }
  return hipErrorInvalidValue;
}

}  // namespace kda
