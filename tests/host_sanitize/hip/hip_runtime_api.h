/*
 * Host-only stand-in for the HIP runtime API, for the CPU sanitizer build of
 * the library's host layer (flce_api.hip compiled by g++ with AddressSanitizer
 * and UndefinedBehaviorSanitizer).  TEST INFRASTRUCTURE: declares only what
 * that file uses; stub_runtime.cpp defines the functions.  Nothing here
 * touches a device.
 */
#pragma once
#include <stddef.h>
#include <stdint.h>

typedef struct ihipStream_t* hipStream_t;
typedef struct ihipEvent_t* hipEvent_t;
typedef int hipDevice_t;

typedef enum hipError_t {
  hipSuccess = 0,
  hipErrorInvalidValue = 1,
  hipErrorInvalidSymbol = 13,
  hipErrorInvalidDevice = 101
} hipError_t;

typedef enum hipMemcpyKind {
  hipMemcpyHostToHost = 0,
  hipMemcpyHostToDevice = 1,
  hipMemcpyDeviceToHost = 2,
  hipMemcpyDeviceToDevice = 3,
  hipMemcpyDefault = 4
} hipMemcpyKind;

#ifdef __cplusplus
extern "C" {
#endif
hipError_t hipEventRecord(hipEvent_t event, hipStream_t stream);
hipError_t hipMemcpyAsync(void* dst, const void* src, size_t bytes, hipMemcpyKind kind,
                          hipStream_t stream);
hipError_t hipGetDevice(int* device);
hipError_t hipSetDevice(int device);
hipError_t hipStreamGetDevice(hipStream_t stream, hipDevice_t* device);
hipError_t hipGetSymbolAddress(void** dev_ptr, const void* symbol);
#ifdef __cplusplus
}
#endif
