// Matrix-core decode path for bf16, head_dim 128 (declarations).
#pragma once

#include "pa_common.hpp"
#include "pa.h"

namespace pa {
namespace mfma {

inline bool eligible(int dtype, int head_dim, int group) {
  (void)dtype; (void)head_dim; (void)group;
  return false;
}
inline int chunk_for(int max_live) { (void)max_live; return 256; }
inline int launch(const DecodeArgs&, hipStream_t) { return -1; }

}  // namespace mfma
}  // namespace pa
