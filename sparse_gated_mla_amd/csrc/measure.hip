// HBM read probe: a plain streaming read of a device buffer, in the access
// pattern the indexer uses for its keys (each wave instruction reads 1 KiB of
// contiguous memory with the streaming cache policy; each workgroup walks one
// contiguous chunk with eight 4 KiB steps in flight). It measures the read
// rate this GPU reaches, to set beside its published HBM peak; it is not a
// step of the method.
#include <stdint.h>

#include "sga.h"
#include "sga_device.h"

namespace sga {
namespace {

constexpr int kProbeThreads = 256;
constexpr int kProbeSteps = 8;          // 4 KiB steps in flight per workgroup
constexpr uint32_t kProbeStep = 4096;   // bytes per workgroup step
constexpr int kProbeWgs = 1024;         // four workgroups per compute unit
constexpr int kStreaming = 2;           // cache-policy bit: read-once data

__global__ __launch_bounds__(kProbeThreads) void hbm_read_kernel(const uint8_t* src, uint64_t bytes,
                                                                uint64_t chunk, uint32_t* sink) {
  const uint64_t begin = (uint64_t)blockIdx.x * chunk;
  if (begin >= bytes) return;
  const uint32_t len = (uint32_t)(bytes - begin < chunk ? bytes - begin : chunk);
  const rsrc_t r = make_rsrc(src + begin, len);   // past len the loads read zeros
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  u32x4 acc = {0u, 0u, 0u, 0u};
  for (uint32_t s = 0; s < len; s += kProbeSteps * kProbeStep) {
    u32x4 v[kProbeSteps];
#pragma unroll
    for (int i = 0; i < kProbeSteps; ++i)
      v[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                           r, (int)(s + i * kProbeStep + wave * 1024 + lane * 16), 0, kStreaming));
#pragma unroll
    for (int i = 0; i < kProbeSteps; ++i) acc ^= v[i];
  }
  const uint32_t x = acc.x ^ acc.y ^ acc.z ^ acc.w;
  // a store no input is expected to trigger, so the loads cannot be dropped
  if (x == 0x5EA7F00Du) sink[blockIdx.x * kProbeThreads + threadIdx.x] = x;
}

}  // namespace
}  // namespace sga

extern "C" SGA_API sga_status sga_hbm_read_probe(const void* src, size_t bytes, uint32_t* sink,
                                                 hipStream_t stream) {
  if (!src || !sink || bytes == 0 || bytes % sga::kProbeStep != 0) return SGA_ERR_INVALID_ARG;
  const uint64_t per = (bytes + sga::kProbeWgs - 1) / sga::kProbeWgs;
  const uint64_t chunk = (per + sga::kProbeStep - 1) / sga::kProbeStep * sga::kProbeStep;
  if (chunk > 0xFFFFFFFFull - sga::kProbeSteps * sga::kProbeStep) return SGA_ERR_UNSUPPORTED;
  const unsigned grid = (unsigned)((bytes + chunk - 1) / chunk);
  sga::hbm_read_kernel<<<grid, sga::kProbeThreads, 0, stream>>>(static_cast<const uint8_t*>(src),
                                                               (uint64_t)bytes, chunk, sink);
  return hipGetLastError() == hipSuccess ? SGA_OK : SGA_ERR_HIP;
}
