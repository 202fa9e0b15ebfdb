// Host-only stand-in for the parts of the HIP runtime header that the library's host code uses, so that
// onela_host.cpp builds with g++ and the sanitizers.  Test infrastructure: no GPU, no device code.
#pragma once

#include <cstddef>
#include <cstdint>

typedef enum hipError_t {
  hipSuccess = 0,
  hipErrorInvalidValue = 1,
  hipErrorInvalidDevice = 101,
  hipErrorLaunchFailure = 719,
} hipError_t;

typedef struct ihipStream_t* hipStream_t;

typedef enum hipMemcpyKind {
  hipMemcpyHostToHost = 0,
  hipMemcpyHostToDevice = 1,
  hipMemcpyDeviceToHost = 2,
  hipMemcpyDeviceToDevice = 3,
  hipMemcpyDefault = 4,
} hipMemcpyKind;

typedef enum hipDeviceAttribute_t {
  hipDeviceAttributeMaxSharedMemoryPerBlock = 1,
  hipDeviceAttributeMultiprocessorCount = 2,
} hipDeviceAttribute_t;

hipError_t hipGetDevice(int* device);
hipError_t hipDeviceGetAttribute(int* value, hipDeviceAttribute_t attr, int device);
const char* hipGetErrorString(hipError_t e);
hipError_t hipGetLastError();
hipError_t hipMemcpyAsync(void* dst, const void* src, size_t bytes, hipMemcpyKind kind, hipStream_t s);
hipError_t hipStreamSynchronize(hipStream_t s);
