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

// Matrix-core reference: independent MFMA chains on every SIMD, nothing else (see pagedkv.h).
namespace {
__global__ __launch_bounds__(512) void mfma_peak_kernel(int iters, float* __restrict__ sink) {
  // Eight A and eight B fragments of pseudo-random bf16 values in [-2, 2) per lane (a per-thread
  // xorshift), so that consecutive MFMAs see different operands: the switching activity of real
  // data, which sets the power, and so the clock, the matrix cores hold.  (Constant operands run
  // at a markedly higher rate than any real kernel can.)
  uint32_t h = (blockIdx.x * 512u + threadIdx.x) * 2654435761u + 0x9e3779b9u;
  auto rnd = [&]() {
    h ^= h << 13;
    h ^= h >> 17;
    h ^= h << 5;
    return static_cast<__bf16>(static_cast<float>(static_cast<int32_t>(h)) * 0x1p-30f);
  };
  pkv::bf16x8 A[8], B[8];
#pragma unroll
  for (int f = 0; f < 8; ++f)
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      A[f][i] = rnd();
      B[f][i] = rnd();
    }
  pkv::floatx16 acc[4];
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[j][e] = 0.f;
  // Four independent accumulator chains; 64 MFMAs (16 iterations' worth) cycle through the 64
  // operand pairs.
  int it = 0;
  for (; it + 16 <= iters; it += 16)
#pragma unroll
    for (int b = 0; b < 8; ++b)
#pragma unroll
      for (int a = 0; a < 8; ++a)
        acc[(a + b) & 3] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A[a], B[b], acc[(a + b) & 3], 0, 0, 0);
  for (; it < iters; ++it)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A[j], B[j], acc[j], 0, 0, 0);
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int e = 0; e < 16; ++e) s += acc[j][e];
  if (s == -1.2345e-30f) sink[0] = s;  // never true; keeps the chains
}
}  // namespace

extern "C" pkv_status pkv_mfma_peak_probe(int32_t iters, float* sink, void* stream) {
  if (iters <= 0 || !sink) return PKV_ERR_INVALID_ARG;
  hipLaunchKernelGGL(mfma_peak_kernel, dim3(pkv_host::cu_count()), dim3(512), 0, static_cast<hipStream_t>(stream),
                     iters, sink);
  return pkv_host::launch_status();
}

extern "C" int32_t pkv_device_cu_count(void) { return pkv_host::cu_count(); }
