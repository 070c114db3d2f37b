// Plain streaming read of a device buffer (include/iq_probe.h): the read
// rate this GPU reaches, against which the decode kernels' rates are set.
#include "iq.h"
#include "iq_probe.h"

#include <algorithm>

namespace {

constexpr int kProbeThreads = 256;
constexpr int kProbeGroupsPerCu = 8;
constexpr uint32_t kProbeMagic = 0x9E3779B9u;

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// Thread t of the grid reads 16-byte words t, t + S, t + 2S, ... (S = the
// grid's thread count) with non-temporal loads, one in flight per lane: of
// the launch shapes tried (1 to 8 loads in flight per lane, 2 to 32
// workgroups per compute unit, with and without the non-temporal hint) this
// reads fastest; more loads per lane spread each wave's requests further
// apart in memory and read slower.
__global__ __launch_bounds__(kProbeThreads) void stream_read_kernel(const u32x4 *__restrict__ p, size_t n,
                                                                    uint32_t *sink) {
  const size_t s = (size_t)gridDim.x * kProbeThreads;
  uint32_t acc = 0;
  for (size_t i = (size_t)blockIdx.x * kProbeThreads + threadIdx.x; i < n; i += s) {
    const u32x4 v = __builtin_nontemporal_load(p + i);
    acc ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  if (acc == kProbeMagic) *sink = acc;
}

}  // namespace

extern "C" int iq_probe_stream_read(const void *buf, size_t bytes, uint32_t *sink, hipStream_t stream) {
  if (buf == nullptr || sink == nullptr || bytes == 0 || bytes % 16 != 0) return IQ_ERR_INVALID_ARG;
  if (reinterpret_cast<uintptr_t>(buf) % 16 != 0) return IQ_ERR_MISALIGNED;
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
    return IQ_ERR_HIP;
  const size_t n = bytes / 16;
  const size_t need = (n + kProbeThreads - 1) / kProbeThreads;
  const unsigned grid = (unsigned)std::min<size_t>((size_t)cus * kProbeGroupsPerCu, need);
  hipLaunchKernelGGL(stream_read_kernel, dim3(grid), dim3(kProbeThreads), 0, stream,
                     static_cast<const u32x4 *>(buf), n, sink);
  return hipGetLastError() == hipSuccess ? IQ_OK : IQ_ERR_HIP;
}
