// fix_kernel: the correction of split sequences as a launch of its own, for
// sequences in more than two segments (after compose_kernel has formed the
// later segments' start states); sequences in two segments are corrected
// by the fused kernel's tail workgroups.  The device code is in kda_cp.hpp.
#include "kda_cp.hpp"

namespace kda {
namespace {

constexpr int kFixThreads = 256;

__global__ __launch_bounds__(kFixThreads) void fix_kernel(FixArgs p) {
  __shared__ __attribute__((aligned(16))) char lds[kFixLds];
  const FixView v{p.o, p.qhat, p.tstate, p.xpool, p.page_pool, p.s_final, p.page_elems, p.H};
  const int b = blockIdx.x;
  // (a chain of this sequence and head stopped at a decay out of range:
  // nothing of it is corrected)
  auto stopped = [&](int cb, int h) { return p.cnt[cb + h] >= 0x10000; };
  if (b < p.n_owg) {
    const int sg = ld_const(p.owgs, 3 * b), h = ld_const(p.owgs, 3 * b + 1), t0 = ld_const(p.owgs, 3 * b + 2);
    if (stopped(ld_const(p.segs, 5 * sg + 4), h)) return;
    fix_rows<kFixThreads / 64>(v, ld_const(p.segs, 5 * sg), ld_const(p.segs, 5 * sg + 1), ld_const(p.segs, 5 * sg + 2),
                               ld_const(p.segs, 5 * sg + 3), h, t0, t0 + kFixTokens, lds);
  } else {
    const int item = b - p.n_owg, rb = item % (kFixD / kFixCkRows);
    const int h = (item / (kFixD / kFixCkRows)) % p.H, ck = item / (kFixD / kFixCkRows) / p.H;
    if (stopped(ld_const(p.cks, 6 * ck + 5), h)) return;
    fix_state_item<kFixThreads / 64>(v, ld_const(p.cks, 6 * ck), ld_const(p.cks, 6 * ck + 1), ld_const(p.cks, 6 * ck + 2),
                   ld_const(p.cks, 6 * ck + 3), ld_const(p.cks, 6 * ck + 4) != 0, h, rb, lds);
  }
}

}  // namespace

hipError_t launch_fix(const FixArgs& p) {
  if (p.dk != kFixD || p.dv != kFixD) return hipErrorInvalidValue;
  const int64_t n = p.n_owg + static_cast<int64_t>(p.n_cks) * p.H * (kFixD / kFixCkRows);
  if (n == 0) return hipSuccess;
  if (n >= (int64_t{1} << 31)) return hipErrorInvalidValue;
  hipLaunchKernelGGL(fix_kernel, dim3(static_cast<unsigned>(n)), dim3(kFixThreads), 0, p.stream, p);
  return hipGetLastError();
}

}  // namespace kda
