// Measurement helper: a plain streaming read of device memory, the HBM
// ceiling that the decode attention kernel's bandwidth is compared with.
// Not part of the attention arithmetic.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "mla.h"
#include "mla_device.h"

namespace mla {
namespace {

constexpr int SR_THREADS = 256;
constexpr int SR_UNROLL = 4;  // 16-byte loads in flight per thread

// Grid-stride read of n16 16-byte words; the XOR of everything read is
// compared with a value it cannot take in practice, so the loads stay live
// and nothing is written.
__global__ __launch_bounds__(SR_THREADS) void stream_read_kernel(const u32x4* __restrict__ src, int64_t n16,
                                                                 uint32_t* __restrict__ sink) {
  const int64_t stride = (int64_t)gridDim.x * SR_THREADS;
  int64_t i = (int64_t)blockIdx.x * SR_THREADS + threadIdx.x;
  u32x4 acc = zero16();
  for (; i + (SR_UNROLL - 1) * stride < n16; i += SR_UNROLL * stride) {
    u32x4 v[SR_UNROLL];
#pragma unroll
    for (int u = 0; u < SR_UNROLL; ++u) v[u] = __builtin_nontemporal_load(src + i + u * stride);
#pragma unroll
    for (int u = 0; u < SR_UNROLL; ++u) acc ^= v[u];
  }
  for (; i < n16; i += stride) acc ^= src[i];
  const uint32_t x = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
  if (x == 0x9E3779B9u && sink) sink[0] = x;
}

}  // namespace
}  // namespace mla

extern "C" mla_status mla_stream_read(const void* src, int64_t bytes, void* sink, void* stream) {
  if (!src || bytes <= 0 || (bytes & 15) || ((uintptr_t)src & 15)) return MLA_ERR_INVALID_ARG;
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return MLA_ERR_HIP;
  const int64_t n16 = bytes / 16;
  int64_t blocks = (int64_t)cus * 8;  // eight workgroups of four waves per CU
  const int64_t need = (n16 + mla::SR_THREADS - 1) / mla::SR_THREADS;
  if (blocks > need) blocks = need;
  hipLaunchKernelGGL(mla::stream_read_kernel, dim3((unsigned)blocks), dim3(mla::SR_THREADS), 0, (hipStream_t)stream,
                     (const mla::u32x4*)src, n16, (uint32_t*)sink);
  return hipGetLastError() == hipSuccess ? MLA_OK : MLA_ERR_HIP;
}
