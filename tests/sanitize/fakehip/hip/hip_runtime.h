/*
 * Stand-in for <hip/hip_runtime.h> in the host-only sanitizer build of the
 * C ABI layer (tests/test_sanitizers_cpu.py): just the names api.hip and
 * launch.h use, with HIP's device qualifiers compiled away.  Nothing here
 * touches a GPU; the launchers are stubs (stub_launch.cpp).
 */
#pragma once
#include <stddef.h>
#include <stdint.h>

#define __device__
#define __host__
#define __global__
#define __forceinline__ inline
#define __align__(x) __attribute__((aligned(x)))

typedef struct ihipStream_t *hipStream_t;
typedef enum { hipSuccess = 0, hipErrorInvalidValue = 1 } hipError_t;

hipError_t hipGetLastError(void);
hipError_t hipGetDevice(int *device);
hipError_t hipGetSymbolAddress(void **devPtr, const void *symbol);
#define HIP_SYMBOL(x) ((const void *)&(x))
