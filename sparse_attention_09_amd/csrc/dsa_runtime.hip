// HIP runtime services of the host code: reading caller memory back for the
// DSA_VALIDATE checks, and the read-bandwidth probe the rooflines are
// measured against.
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

namespace {

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

// Grid-stride read of n16 16-byte pieces, four per thread per trip, every load
// bounds-checked; one XOR per workgroup keeps the loads live.
__global__ __launch_bounds__(256) void read_probe_kernel(const u32x4_t* __restrict__ p, int64_t n16,
                                                         uint32_t* __restrict__ out) {
  uint32_t acc = 0;
  const int64_t stride = int64_t(gridDim.x) * 256 * 4;
  for (int64_t i = int64_t(blockIdx.x) * 256 * 4 + threadIdx.x; i < n16; i += stride) {
    u32x4_t v[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int64_t j = i + 256 * u;
      v[u] = j < n16 ? p[j] : u32x4_t{0, 0, 0, 0};
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) acc ^= v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3];
  }
  __shared__ uint32_t red[256];
  red[threadIdx.x] = acc;
  __syncthreads();
  if (threadIdx.x < 64) {
    uint32_t x = red[threadIdx.x] ^ red[threadIdx.x + 64] ^ red[threadIdx.x + 128] ^
                 red[threadIdx.x + 192];
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) x ^= uint32_t(__shfl_xor(int(x), off));
    if (threadIdx.x == 0) out[blockIdx.x] = x;
  }
}

}  // namespace

extern "C" dsa_status dsa_read_probe(const void* buf, int64_t bytes, uint32_t* out,
                                     int32_t num_blocks, void* stream) {
  if (!buf || !out || bytes < 0 || bytes % 16 != 0 || (reinterpret_cast<uintptr_t>(buf) & 15) != 0 ||
      num_blocks < 1 || num_blocks > 65536)
    return dsa::fail(DSA_ERR_INVALID_ARG,
                     "dsa_read_probe: need buf and out, buf 16-byte aligned, bytes >= 0 and a "
                     "multiple of 16, 1 <= num_blocks <= 65536");
  if (bytes == 0) return dsa::ok();
  hipLaunchKernelGGL(read_probe_kernel, dim3(num_blocks), dim3(256), 0,
                     static_cast<hipStream_t>(stream), static_cast<const u32x4_t*>(buf), bytes / 16,
                     out);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess)
    return dsa::fail(DSA_ERR_HIP, std::string("dsa_read_probe: launch failed: ") + hipGetErrorString(e));
  return dsa::ok();
}
