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
constexpr int SR_PER = 9;                          // 16-byte loads per thread and tile
constexpr int SR_TILE = SR_THREADS * SR_PER;       // 16-byte words per tile (36 KB)

// One workgroup per CU reads whole 36 KB tiles (workgroup w: tiles w, w + G,
// w + 2G, ..., so the grid sweeps memory front to back), two tiles in flight,
// with non-temporal 16-byte loads; then the words past the last whole tile.
// The XOR of everything read is compared with a value it cannot take in
// practice, so the loads stay live and nothing is written.  (A grid-stride
// loop over 16-byte words with eight workgroups per CU and four loads in
// flight per thread reached 6.1 TB/s; this shape reaches 7.0-7.2 TB/s, with
// pages of two tiles read in shuffled order as well.)
__global__ __launch_bounds__(SR_THREADS) void stream_read_kernel(const u32x4* __restrict__ src, int64_t n16,
                                                                 uint32_t* __restrict__ sink) {
  const int64_t G = gridDim.x, ntiles = n16 / SR_TILE;
  const int tid = threadIdx.x;
  u32x4 acc = zero16();
  u32x4 a[SR_PER], b[SR_PER];
  auto load = [&](u32x4 (&v)[SR_PER], int64_t t) {
    const u32x4* p = src + t * SR_TILE + tid;
#pragma unroll
    for (int k = 0; k < SR_PER; ++k) v[k] = __builtin_nontemporal_load(p + SR_THREADS * k);
  };
  auto use = [&](const u32x4 (&v)[SR_PER]) {
#pragma unroll
    for (int k = 0; k < SR_PER; ++k) acc ^= v[k];
  };
  int64_t t = blockIdx.x;
  if (t < ntiles) load(a, t);
  if (t + G < ntiles) load(b, t + G);
  for (; t < ntiles; t += 2 * G) {
    use(a);
    if (t + 2 * G < ntiles) load(a, t + 2 * G);
    if (t + G < ntiles) {
      use(b);
      if (t + 3 * G < ntiles) load(b, t + 3 * G);
    }
  }
  for (int64_t i = ntiles * SR_TILE + (int64_t)blockIdx.x * SR_THREADS + tid; i < n16; i += G * SR_THREADS)
    acc ^= src[i];
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
  const int64_t blocks = cus;  // one workgroup of four waves per CU
  hipLaunchKernelGGL(mla::stream_read_kernel, dim3((unsigned)blocks), dim3(mla::SR_THREADS), 0, (hipStream_t)stream,
                     (const mla::u32x4*)src, n16, (uint32_t*)sink);
  return hipGetLastError() == hipSuccess ? MLA_OK : MLA_ERR_HIP;
}
