// Kernel launches of libsfa's HIP sources: SFA_LAUNCH hands the events of
// a recording ProfileScope to the dispatch it launches.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include "sfa_internal.h"

// A kernel launch that hands the recording scope's events, if any, to the
// dispatch (the first launch of the scope; later ones launch plainly).
#define SFA_LAUNCH(kernel, grid, block, lds, st, ...)                                                          \
  do {                                                                                                         \
    ::sfa::ProfileScope* sfa_ps_ = ::sfa::active_profile_scope();                                            \
    if (sfa_ps_ && sfa_ps_->launches++ == 0)                                                                 \
      hipExtLaunchKernelGGL(kernel, grid, block, lds, st, static_cast<hipEvent_t>(sfa_ps_->ev0),             \
                            static_cast<hipEvent_t>(sfa_ps_->ev1), 0, __VA_ARGS__);                          \
    else                                                                                                       \
      hipLaunchKernelGGL(kernel, grid, block, lds, st, __VA_ARGS__);                                          \
  } while (0)
