// Plain streaming read of a device buffer: the device's achievable HBM read rate, measured
// next to the projection kernels (which move the same head bytes) so that their bandwidth
// can be read against what a kernel that does nothing but read reaches on the same device.
// Every 16-byte chunk is read once with lane-contiguous loads (a wave reads 1 KB per
// instruction); the chunks are XOR-folded into one word per wave so that no load can be
// dropped.
#include "jet_internal.h"

// One workgroup per CU, eight 16-byte loads in flight per lane, non-temporal loads (the
// buffer is read once): the fastest combination measured, 7.06 TB/s over a 1.27 GB buffer
// (6.3 without the non-temporal hint; 512 or 2048 workgroups and 4 or 16 loads gave
// 4.6-6.2).
#ifndef JET_STREAM_GRID
#define JET_STREAM_GRID 256
#endif
#ifndef JET_STREAM_UNROLL
#define JET_STREAM_UNROLL 8
#endif

namespace jet {
namespace {

constexpr int kStreamUnroll = JET_STREAM_UNROLL;

__global__ __launch_bounds__(256) void k_stream_read(const u32x4* __restrict__ p, long long n16,
                                                     uint32_t* __restrict__ out) {
  const long long stride = (long long)gridDim.x * 256;
  long long i = (long long)blockIdx.x * 256 + threadIdx.x;
  uint32_t x = 0u;
  for (; i + (kStreamUnroll - 1) * stride < n16; i += kStreamUnroll * stride) {
    u32x4 v[kStreamUnroll];
#pragma unroll
    for (int u = 0; u < kStreamUnroll; ++u) v[u] = __builtin_nontemporal_load(&p[i + u * stride]);
#pragma unroll
    for (int u = 0; u < kStreamUnroll; ++u) x ^= v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3];
  }
  for (; i < n16; i += stride) {
    const u32x4 a = __builtin_nontemporal_load(&p[i]);
    x ^= a[0] ^ a[1] ^ a[2] ^ a[3];
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) x ^= (uint32_t)__shfl_xor((int)x, off);
  if ((threadIdx.x & 63) == 0) atomicXor(out, x);
}

}  // namespace
}  // namespace jet

extern "C" JET_API jet_status jet_stream_read(const void* buf, size_t bytes, uint32_t* out,
                                              void* stream) {
  if (!buf || !out) return JET_E_NULL;
  if (bytes % 16 != 0 || ((uintptr_t)buf & 15u)) return JET_E_SHAPE;
  const long long n16 = (long long)(bytes / 16);
  if (n16 == 0) return JET_OK;
  hipLaunchKernelGGL(jet::k_stream_read, dim3(JET_STREAM_GRID), dim3(256), 0, static_cast<hipStream_t>(stream),
                     static_cast<const jet::u32x4*>(buf), n16, out);
  return hipGetLastError() == hipSuccess ? JET_OK : JET_E_HIP;
}
