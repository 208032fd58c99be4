// A plain streaming read of a device buffer: the practical HBM read ceiling
// of the device, measured beside the attention kernels.  Every lane reads
// 16-byte chunks with the nontemporal policy the decode kernels use, eight
// loads in flight, and folds them into a checksum so that no load can be
// dropped; each workgroup writes one word.
#include "common.h"

namespace pkv {
namespace {

constexpr int kProbeThreads = 256;
constexpr int kProbeUnroll = 8;

__global__ __launch_bounds__(kProbeThreads) void stream_read_kernel(const uint4* __restrict__ src,
                                                                    int64_t chunks,
                                                                    uint32_t* __restrict__ sink) {
  const int64_t stride = (int64_t)gridDim.x * kProbeThreads;
  int64_t i = (int64_t)blockIdx.x * kProbeThreads + threadIdx.x;
  uint32_t acc = 0;
  // whole rounds of kProbeUnroll chunks per lane, all loads issued first
  for (; i + (kProbeUnroll - 1) * stride < chunks; i += kProbeUnroll * stride) {
    uint4 v[kProbeUnroll];
#pragma unroll
    for (int u = 0; u < kProbeUnroll; ++u) v[u] = load_stream(src + i + u * stride);
#pragma unroll
    for (int u = 0; u < kProbeUnroll; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  for (; i < chunks; i += stride) {
    const uint4 v = load_stream(src + i);
    acc ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  // each wave folds its lanes and its lane 0 writes the wave's word (four
  // words per workgroup)
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) acc ^= __shfl_xor(acc, off);
  if ((threadIdx.x & 63) == 0) sink[(int64_t)blockIdx.x * (kProbeThreads / 64) + (threadIdx.x >> 6)] = acc;
}

}  // namespace

int stream_read_sink_words(int workgroups) { return workgroups * (kProbeThreads / 64); }

hipError_t launch_stream_read(const void* buf, int64_t bytes, uint32_t* sink, int workgroups,
                              hipStream_t st) {
  hipLaunchKernelGGL(stream_read_kernel, dim3(workgroups), dim3(kProbeThreads), 0, st,
                     reinterpret_cast<const uint4*>(buf), bytes / 16, sink);
  return hipGetLastError();
}

}  // namespace pkv
