// Measurement probes: a plain 16-byte streaming read and a plain copy.
// They give the bandwidth the memory system sustains for a simple stream,
// the ceiling the decode kernels are compared with.  And the upload copy
// (pa_upload): the same loop reading device-mapped host memory.
#include "pa_device.h"
#include "pa_internal.h"

namespace pa {
namespace {

constexpr int kProbeThreads = 256;
// 8 workgroups of 4 waves per CU on a 256-CU part: every wave resident at
// once (32 per CU).  A sweep on MI355X read 4 GiB at 6.39 TB/s this way and
// at 5.94-5.99 TB/s with twice the workgroups (two rounds of residency).
constexpr int kProbeBlocks = 256 * 8;

__global__ __launch_bounds__(kProbeThreads) void probe_read_kernel(const uint4* buf, int64_t n16, uint4* sink) {
  uint4 acc = make_uint4(0, 0, 0, 0);
  const int64_t stride = (int64_t)gridDim.x * kProbeThreads;
  for (int64_t i = (int64_t)blockIdx.x * kProbeThreads + threadIdx.x; i < n16; i += stride) {
    const uint4 v = buf[i];
    acc.x ^= v.x; acc.y ^= v.y; acc.z ^= v.z; acc.w ^= v.w;
  }
  // fold the workgroup's lanes so the loads stay live; one 16-byte word per workgroup
  __shared__ uint4 red[kProbeThreads];
  red[threadIdx.x] = acc;
  __syncthreads();
  for (int s = kProbeThreads / 2; s > 0; s >>= 1) {
    if (threadIdx.x < s) {
      uint4 o = red[threadIdx.x + s];
      red[threadIdx.x].x ^= o.x; red[threadIdx.x].y ^= o.y;
      red[threadIdx.x].z ^= o.z; red[threadIdx.x].w ^= o.w;
    }
    __syncthreads();
  }
  if (threadIdx.x == 0) sink[blockIdx.x] = red[0];
}

__global__ __launch_bounds__(kProbeThreads) void probe_copy_kernel(uint4* dst, const uint4* src, int64_t n16) {
  const int64_t stride = (int64_t)gridDim.x * kProbeThreads;
  for (int64_t i = (int64_t)blockIdx.x * kProbeThreads + threadIdx.x; i < n16; i += stride) dst[i] = src[i];
}

// Upload: a grid-stride 16-byte copy from device-mapped host memory.
constexpr int kUploadThreads = 256;

__global__ __launch_bounds__(kUploadThreads) void upload_kernel(uint4* dst, const uint4* src, int64_t n16) {
  const int64_t stride = (int64_t)gridDim.x * kUploadThreads;
  for (int64_t i = (int64_t)blockIdx.x * kUploadThreads + threadIdx.x; i < n16; i += stride) dst[i] = src[i];
}

}  // namespace

hipError_t launch_upload(void* dst, const void* src, size_t bytes, hipStream_t stream) {
  const int64_t n16 = (int64_t)(bytes / 16);
  const int64_t want = (n16 + kUploadThreads - 1) / kUploadThreads;
  const int grid = (int)(want < 64 ? (want < 1 ? 1 : want) : 64);     // a few workgroups: the reads cross PCIe
  hipLaunchKernelGGL(upload_kernel, dim3(grid), dim3(kUploadThreads), 0, stream, reinterpret_cast<uint4*>(dst),
                     reinterpret_cast<const uint4*>(src), n16);
  return hipGetLastError();
}

size_t probe_sink_bytes() { return (size_t)kProbeBlocks * 16; }

hipError_t launch_probe_stream_read(const void* buf, size_t bytes, void* sink, hipStream_t stream) {
  hipLaunchKernelGGL(probe_read_kernel, dim3(kProbeBlocks), dim3(kProbeThreads), 0, stream,
                     reinterpret_cast<const uint4*>(buf), (int64_t)(bytes / 16), reinterpret_cast<uint4*>(sink));
  return hipGetLastError();
}

hipError_t launch_probe_copy(void* dst, const void* src, size_t bytes, hipStream_t stream) {
  hipLaunchKernelGGL(probe_copy_kernel, dim3(kProbeBlocks), dim3(kProbeThreads), 0, stream,
                     reinterpret_cast<uint4*>(dst), reinterpret_cast<const uint4*>(src), (int64_t)(bytes / 16));
  return hipGetLastError();
}

}  // namespace pa
