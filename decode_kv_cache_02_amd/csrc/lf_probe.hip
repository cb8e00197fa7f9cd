// Measurement probes (include/longflow_probe.h). Streaming read: every
// workgroup reads its own contiguous region once with 16-byte non-temporal
// buffer loads, the same loads the decode kernel uses for K and V, and XORs
// what it read. HBM attributes: the device's own memory clock and bus width.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/longflow_probe.h"

namespace {

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
constexpr int kThreads = 256;
constexpr int kUnroll = 4;           // loads in flight per thread
constexpr int kRsrcWord3 = 0x00020000;
constexpr int kNonTemporal = 3;      // the decode kernel's K/V cache policy

constexpr int kHwRegXccId = (15 << 11) | 20;
constexpr int kHwRegHwId = (31 << 11) | 4;

__global__ __launch_bounds__(kThreads) void stream_read_kernel(const char* buf, uint32_t region,
                                                               u32x4_t* sink, uint64_t* records) {
  const uint64_t start = records ? __builtin_amdgcn_s_memrealtime() : 0;
  const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<char*>(buf) + static_cast<size_t>(blockIdx.x) * region, 0,
      static_cast<int>(region), kRsrcWord3);
  u32x4_t acc = {0u, 0u, 0u, 0u};
  for (uint32_t off = threadIdx.x * 16u; off < region; off += kThreads * 16u * kUnroll) {
    u32x4_t v[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u)
      v[u] = __builtin_amdgcn_raw_buffer_load_b128(r, static_cast<int>(off + u * kThreads * 16u), 0,
                                                   kNonTemporal);
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) acc ^= v[u];
  }
  sink[static_cast<size_t>(blockIdx.x) * kThreads + threadIdx.x] = acc;
  if (records && threadIdx.x == 0) {
    uint64_t* rec = records + 4 * static_cast<size_t>(blockIdx.x);
    rec[0] = start;
    rec[1] = __builtin_amdgcn_s_memrealtime();
    rec[2] = static_cast<uint64_t>(__builtin_amdgcn_s_getreg(kHwRegXccId)) |
             (static_cast<uint64_t>(__builtin_amdgcn_s_getreg(kHwRegHwId)) << 32);
    rec[3] = blockIdx.x;
  }
}

lf_status launch_read(const void* buf, size_t bytes, int32_t workgroups, void* sink, uint64_t* records,
                      void* stream) {
  if (!buf || !sink || workgroups < 1) return LF_ERR_INVALID_ARG;
  if ((reinterpret_cast<uintptr_t>(buf) & 15u) || (reinterpret_cast<uintptr_t>(sink) & 15u))
    return LF_ERR_INVALID_ARG;
  const size_t unit = 16u * static_cast<size_t>(workgroups);
  if (bytes == 0 || bytes % unit) return LF_ERR_INVALID_ARG;
  const size_t region = bytes / static_cast<size_t>(workgroups);
  if (region >= (size_t{1} << 31)) return LF_ERR_INVALID_ARG;
  hipLaunchKernelGGL(stream_read_kernel, dim3(workgroups), dim3(kThreads), 0,
                     static_cast<hipStream_t>(stream), static_cast<const char*>(buf),
                     static_cast<uint32_t>(region), static_cast<u32x4_t*>(sink), records);
  return hipGetLastError() == hipSuccess ? LF_OK : LF_ERR_HIP;
}

}  // namespace

extern "C" lf_status lf_probe_stream_read(const void* buf, size_t bytes, int32_t workgroups,
                                          void* sink, void* stream) {
  return launch_read(buf, bytes, workgroups, sink, nullptr, stream);
}

extern "C" lf_status lf_probe_stream_read_timing(const void* buf, size_t bytes, int32_t workgroups,
                                                 void* sink, uint64_t* records, void* stream) {
  if (!records) return LF_ERR_INVALID_ARG;
  return launch_read(buf, bytes, workgroups, sink, records, stream);
}

extern "C" lf_status lf_probe_hbm_attributes(int32_t* mem_clock_khz, int32_t* bus_width_bits) {
  if (!mem_clock_khz || !bus_width_bits) return LF_ERR_INVALID_ARG;
  int dev = 0, clock = 0, width = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&clock, hipDeviceAttributeMemoryClockRate, dev) != hipSuccess ||
      hipDeviceGetAttribute(&width, hipDeviceAttributeMemoryBusWidth, dev) != hipSuccess) {
    (void)hipGetLastError();
    return LF_ERR_HIP;
  }
  *mem_clock_khz = clock;
  *bus_width_bits = width;
  return LF_OK;
}
