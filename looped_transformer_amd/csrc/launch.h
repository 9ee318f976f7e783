// Launch macro of the library's kernels: a plain launch, or with a kernel timer
// installed on this thread (kernels.h), a launch whose event pair the runtime
// stamps with the kernel's own start and end.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include "kernels.h"

#define TL_LAUNCH(K, grid, block, lds, s, ...)                                    \
  do {                                                                           \
    hipEvent_t tl_t0_, tl_t1_;                                                   \
    KernelTimer* tl_kt_ = kernel_timer();                                        \
    if (tl_kt_ && tl_kt_->take(&tl_t0_, &tl_t1_))                                \
      hipExtLaunchKernelGGL(K, grid, block, lds, s, tl_t0_, tl_t1_, 0, __VA_ARGS__); \
    else                                                                         \
      hipLaunchKernelGGL(K, grid, block, lds, s, __VA_ARGS__);                   \
  } while (0)
