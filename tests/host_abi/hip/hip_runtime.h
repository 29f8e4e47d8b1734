// Host-only stand-in for <hip/hip_runtime.h>, for a CPU build of the library's host code (api.cpp) under the
// address and undefined-behaviour sanitizers. It declares only what that code uses; stubs.cpp defines the
// functions, with failures that the test driver injects. No device code is compiled against it.
#pragma once
#include <stddef.h>

typedef enum hipError_t {
  hipSuccess = 0,
  hipErrorInvalidValue = 1,
  hipErrorOutOfMemory = 2,
  hipErrorInvalidDevice = 101,
  hipErrorInvalidSymbol = 13,
  hipErrorLaunchFailure = 719,
  hipErrorIllegalAddress = 700,
} hipError_t;

typedef struct ihipStream_t* hipStream_t;
typedef struct ihipEvent_t* hipEvent_t;

// a __device__ array becomes an ordinary host array; HIP_SYMBOL names it by address
#define __device__
#define __align__(n) __attribute__((aligned(n)))
#define HIP_SYMBOL(x) ((const void*)&(x))

hipError_t hipEventRecord(hipEvent_t event, hipStream_t stream);
hipError_t hipGetDevice(int* device);
hipError_t hipGetSymbolAddress(void** ptr, const void* symbol);
hipError_t hipStreamSynchronize(hipStream_t stream);
hipError_t hipGetLastError(void);
const char* hipGetErrorString(hipError_t e);
