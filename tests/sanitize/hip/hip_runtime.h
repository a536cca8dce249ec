/* A host-only stand-in for <hip/hip_runtime.h>, for building the C ABI's
 * validation code with the host compiler's sanitizers: the few types and
 * runtime calls that convrot_api.cpp names, and nothing that runs on a GPU.
 * Test infrastructure only. */
#pragma once

#include <stddef.h>
#include <stdint.h>

typedef enum hipError_t { hipSuccess = 0, hipErrorInvalidValue = 1 } hipError_t;
typedef struct ihipStream_t *hipStream_t;

#define __device__
#define __forceinline__ inline

inline hipError_t hipGetLastError(void) { return hipSuccess; }

/* wave_lds_sync in the internal header names these device builtins */
#define __builtin_amdgcn_fence(order, scope) ((void)0)
#define __builtin_amdgcn_wave_barrier() ((void)0)
