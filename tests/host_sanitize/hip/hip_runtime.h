/* Host-only stand-in for <hip/hip_runtime.h> (see hip_runtime_api.h). */
#pragma once
#include "hip_runtime_api.h"

#define __device__
#define __align__(n) __attribute__((aligned(n)))
#define HIP_SYMBOL(x) (&(x))
