// Stand-in for <hip/hip_runtime.h> in the GPU-less sanitizer build of the C
// ABI's host code (tests/test_sanitize_host.py).  It declares only what
// moe_permute_api.cpp and moe_launch.h use; launch_stub.cpp defines it.  No
// device code is compiled in that build.
#pragma once

#include <cstddef>

typedef enum hipError_t { hipSuccess = 0, hipErrorInvalidValue = 1, hipErrorNoDevice = 100 } hipError_t;
typedef struct ihipStream_t* hipStream_t;

typedef struct hipDeviceProp_t {
    char gcnArchName[256];
    int multiProcessorCount;
} hipDeviceProp_t;

typedef enum hipDeviceAttribute_t {
    hipDeviceAttributeMultiprocessorCount,
    hipDeviceAttributeMaxSharedMemoryPerMultiprocessor,
} hipDeviceAttribute_t;

extern "C" {
hipError_t hipGetDeviceCount(int* count);
hipError_t hipGetDevice(int* device);
hipError_t hipGetDeviceProperties(hipDeviceProp_t* prop, int device);
hipError_t hipDeviceGetAttribute(int* value, hipDeviceAttribute_t attr, int device);
}
