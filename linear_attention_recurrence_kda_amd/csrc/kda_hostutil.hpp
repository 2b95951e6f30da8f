// Host-side helpers of the C ABI layer: status reporting, argument checks.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <string>
#include <vector>

#include "../../include/kda.h"

namespace kda_host {

inline thread_local std::string g_last_error;

inline int fail(int status, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return status;
}

inline int ok() {
  g_last_error.clear();
  return KDA_OK;
}

inline bool supported_dim(int32_t d) { return d == 16 || d == 32 || d == 64 || d == 128; }

inline size_t elem_size(kda_dtype t) { return t == KDA_BF16 ? 2 : 4; }

inline bool valid_dtype(int t) { return t == KDA_F32 || t == KDA_BF16; }

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

struct Range {
  const void* p;
  size_t bytes;
  const char* name;
};

inline bool overlap(const Range& x, const Range& y) {
  if (x.p == nullptr || y.p == nullptr || x.bytes == 0 || y.bytes == 0) return false;
  const uintptr_t a0 = reinterpret_cast<uintptr_t>(x.p), a1 = a0 + x.bytes;
  const uintptr_t b0 = reinterpret_cast<uintptr_t>(y.p), b1 = b0 + y.bytes;
  return a0 < b1 && b0 < a1;
}

// Every output must be disjoint from every input and from every other output.
inline int check_disjoint(const std::vector<Range>& outs, const std::vector<Range>& ins) {
  for (size_t i = 0; i < outs.size(); ++i) {
    for (const Range& in : ins)
      if (overlap(outs[i], in))
        return fail(KDA_EALIAS, "output '%s' overlaps input '%s'", outs[i].name, in.name);
    for (size_t j = i + 1; j < outs.size(); ++j)
      if (overlap(outs[i], outs[j]))
        return fail(KDA_EALIAS, "outputs '%s' and '%s' overlap", outs[i].name, outs[j].name);
  }
  return KDA_OK;
}

inline int hip_status(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(KDA_EHIP, "%s: %s", what, hipGetErrorString(e));
  return ok();
}

inline constexpr int64_t kMaxGridY = 65535;

}  // namespace kda_host
