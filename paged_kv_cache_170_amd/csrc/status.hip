// Status strings and per-device host state of libpagedkv.
#include <mutex>

#include "common.hpp"

extern "C" const char* pkv_status_string(pkv_status status) {
  switch (status) {
    case PKV_OK: return "ok";
    case PKV_ERR_INVALID_ARG: return "invalid argument";
    case PKV_ERR_UNSUPPORTED: return "unsupported dtype, head_dim, head ratio or block size";
    case PKV_ERR_WORKSPACE_TOO_SMALL: return "decode workspace too small";
    case PKV_ERR_HIP: return "HIP kernel launch failed";
    case PKV_ERR_NO_SPACE: return "not enough free blocks";
    case PKV_ERR_SCRATCH_TOO_SMALL: return "shapes need more than the no-alloc decode's static scratch";
  }
  return "unknown status";
}

namespace pkv_host {

namespace {
constexpr int kMaxDevices = 64;
std::once_flag g_once[kMaxDevices];
int g_cu[kMaxDevices];
}  // namespace

int cu_count() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return 256;
  std::call_once(g_once[dev], [dev] {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    g_cu[dev] = n;
  });
  return g_cu[dev];
}

pkv_status launch_status() { return hipGetLastError() == hipSuccess ? PKV_OK : PKV_ERR_HIP; }

}  // namespace pkv_host

// Streaming-read reference: every byte of the buffer is read once with non-temporal 16-byte loads
// (four in flight per thread, two workgroups per CU) and folded
// into one word per workgroup, which is XOR-ed into *sink.  Used to measure the bandwidth a plain
// read stream reaches on the device, next to the decode's.
namespace {
__global__ __launch_bounds__(256) void stream_read_kernel(const uint4* __restrict__ p, size_t n16,
                                                          uint32_t* __restrict__ sink) {
  uint32_t acc = 0;
  const size_t stride = static_cast<size_t>(gridDim.x) * blockDim.x;
  size_t i = static_cast<size_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  for (; i + 3 * stride < n16; i += 4 * stride) {
    const uint4 a = pkv::ld16_nt(p + i), b = pkv::ld16_nt(p + i + stride), c = pkv::ld16_nt(p + i + 2 * stride),
                d = pkv::ld16_nt(p + i + 3 * stride);
    acc ^= a.x ^ a.w ^ b.y ^ b.z ^ c.x ^ c.w ^ d.y ^ d.z;
  }
  for (; i < n16; i += stride) acc ^= p[i].x ^ p[i].w;
  __shared__ uint32_t red[256];
  red[threadIdx.x] = acc;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t r = 0;
    for (int k = 0; k < 256; ++k) r ^= red[k];
    atomicXor(sink, r);
  }
}
}  // namespace

extern "C" pkv_status pkv_stream_read_probe(const void* buf, size_t bytes, uint32_t* sink, void* stream) {
  if (!buf || !sink || bytes % 16 != 0 || (reinterpret_cast<uintptr_t>(buf) % 16) != 0) return PKV_ERR_INVALID_ARG;
  if (bytes == 0) return PKV_OK;
  const int blocks = pkv_host::cu_count() * 2;  // the fastest plain read stream measured on MI355X
  hipLaunchKernelGGL(stream_read_kernel, dim3(blocks), dim3(256), 0, static_cast<hipStream_t>(stream),
                     static_cast<const uint4*>(buf), bytes / 16, sink);
  return pkv_host::launch_status();
}
