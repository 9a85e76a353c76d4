// Optional launch instrumentation: hipEvents recorded on the caller's stream
// around every kernel launch, read back per kernel kind.  Off by default; when
// off, each hook costs one relaxed atomic load.
#pragma once

#include <hip/hip_runtime.h>

namespace evo {

enum KernelKind { K_FWD = 0, K_BWD_PRE = 1, K_BWD_KV = 2, K_BWD_Q = 3, K_BWD_FIN = 4, K_COUNT = 5 };

void prof_begin(KernelKind k, hipStream_t s);
void prof_end(KernelKind k, hipStream_t s);

}  // namespace evo
