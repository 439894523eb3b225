// Host-side checks of the index arrays the kernels trust: packed sequence
// offsets and state-pool indices.  The C ABI runs them on a
// host copy of the device array when GDR_DEBUG_CHECKS is set (include/gdr.h);
// they are plain C++ so that the sanitizer build tests them without a GPU.
#pragma once

#include <stdint.h>
#include <stdio.h>

#include <vector>

namespace gdr {

// Sequence offsets of a packed batch: cu[0] == 0, non-decreasing, and
// cu[N] == the token count.  On failure writes a message to msg.
inline bool check_cu_seqlens(const int32_t* cu, int N, long long tokens, const char* what, char* msg, size_t n) {
  if (N < 0) {
    snprintf(msg, n, "%s: negative sequence count %d", what, N);
    return false;
  }
  if (cu[0] != 0) {
    snprintf(msg, n, "%s[0] = %d, must be 0", what, cu[0]);
    return false;
  }
  for (int i = 0; i < N; ++i) {
    if (cu[i + 1] < cu[i]) {
      snprintf(msg, n, "%s decreases at %d: %d -> %d", what, i, cu[i], cu[i + 1]);
      return false;
    }
  }
  if ((long long)cu[N] != tokens) {
    snprintf(msg, n, "%s[%d] = %d, must equal the token count %lld", what, N, cu[N], tokens);
    return false;
  }
  return true;
}

// State-pool indices: every index inside [0, pool) names its own slot (an
// index outside the range marks a padding row).
inline bool check_state_indices(const int32_t* idx, int N, int pool, char* msg, size_t n) {
  std::vector<unsigned char> seen(pool > 0 ? (size_t)pool : 0, 0);
  for (int i = 0; i < N; ++i) {
    const int32_t s = idx[i];
    if (s < 0 || s >= pool) continue;
    if (seen[(size_t)s]) {
      snprintf(msg, n, "state_indices: slot %d is named twice (row %d)", s, i);
      return false;
    }
    seen[(size_t)s] = 1;
  }
  return true;
}

}  // namespace gdr
