/* Host-only stand-in for <hip/hip_runtime.h>, used by the sanitizer build of
 * the C-ABI layer (api.cpp) in tests/test_host_sanitizers.py: the few HIP
 * runtime types that api.cpp and internal.h name, nothing else.  The device
 * code is not built in that test; its launch functions are replaced by the
 * recording stubs of tests/csrc/abi_host_check.cpp. */
#pragma once
#include <stddef.h>
#include <stdint.h>
typedef enum hipError_t { hipSuccess = 0, hipErrorInvalidValue = 1 } hipError_t;
typedef struct ihipStream_t* hipStream_t;
