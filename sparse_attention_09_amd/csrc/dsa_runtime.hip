// HIP runtime services of the host code: reading caller memory back for the
// DSA_VALIDATE checks.
#include <hip/hip_runtime.h>

#include <string>

#include "dsa_internal.h"

namespace dsa {

dsa_status copy_to_host(void* dst, const void* src, size_t bytes, void* stream) {
  if (bytes == 0) return DSA_OK;
  hipError_t e = hipStreamSynchronize(static_cast<hipStream_t>(stream));
  if (e == hipSuccess) e = hipMemcpy(dst, src, bytes, hipMemcpyDefault);
  if (e != hipSuccess)
    return fail(DSA_ERR_HIP, std::string("DSA_VALIDATE: reading the batch description failed: ") +
                                 hipGetErrorString(e));
  return DSA_OK;
}

}  // namespace dsa
