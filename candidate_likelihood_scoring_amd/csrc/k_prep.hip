// Operand staging before the projection (for most plans nothing to do).
//
//  * fp32 H with a bf16 head, for the tiled and fallback kernels: H = hi + lo,
//    hi = bf16_rne(H), lo = bf16_rne(H - hi).  The subtraction is exact in fp32, so hi + lo
//    differs from H by at most one bf16 rounding of the residual (about 2^-17 relative).
//    The streaming kernel splits fp32 H itself.
//  * Fewer rows than one tile of the tiled kernel: the kernel runs one whole row tile, so
//    the split planes (fp32 H) or a copy of H (bf16 H) get zero rows appended up to it; the
//    padding rows' partials are never merged.
#include "jet_internal.h"

namespace jet {
namespace {

__device__ inline void split_range(const float* __restrict__ H, long long n, long long n_out,
                                   uint16_t* __restrict__ hi, uint16_t* __restrict__ lo,
                                   long long i0, long long stride) {
  for (long long i = i0; i < n_out; i += stride) {
    const float x = i < n ? H[i] : 0.f;
    const uint16_t h = f32_to_bf16_rne(x);
    hi[i] = h;
    lo[i] = f32_to_bf16_rne(x - bf16_to_f32(h));
  }
}

__global__ __launch_bounds__(256) void k_split(const float* __restrict__ H, long long n,
                                               long long n_out, uint16_t* __restrict__ hi,
                                               uint16_t* __restrict__ lo) {
  split_range(H, n, n_out, hi, lo, (long long)blockIdx.x * 256 + threadIdx.x,
              (long long)gridDim.x * 256);
}

// bf16 H with fewer rows than one tile of the tiled kernel: copied whole, then zero rows up
// to the tile (16-byte chunks: n16 copied, n16_out in all).
__global__ __launch_bounds__(256) void k_pad_rows(const u32x4* __restrict__ src, long long n16,
                                                  long long n16_out, u32x4* __restrict__ dst) {
  for (long long i = (long long)blockIdx.x * 256 + threadIdx.x; i < n16_out;
       i += (long long)gridDim.x * 256)
    dst[i] = i < n16 ? src[i] : u32x4{0u, 0u, 0u, 0u};
}

int split_blocks(long long n, int threads) {
  long long b = (n + threads - 1) / threads;
  if (b > 2048) b = 2048;
  return (int)b;
}

}  // namespace

hipError_t launch_prep(const ScoreArgs& a) {
  const jet_problem* p = a.p;
  const Plan& pl = *a.plan;
  char* ws = a.ws;
  if (pl.hilo && !pl.stream) {
    const hipError_t e = launch_split(static_cast<const float*>(p->H), (long long)p->n_rows * p->d,
                                      (long long)pl.rows_k * p->d,
                                      reinterpret_cast<uint16_t*>(ws + pl.off_hhi),
                                      reinterpret_cast<uint16_t*>(ws + pl.off_hlo), a.stream);
    if (e != hipSuccess) return e;
  }
  if (pl.pad_h) {  // bf16 H: d is a multiple of 64, so rows are whole 16-byte chunks
    const long long n16 = (long long)p->n_rows * p->d / 8, n16_out = (long long)pl.rows_k * p->d / 8;
    hipLaunchKernelGGL(k_pad_rows, dim3(split_blocks(n16_out, 256)), dim3(256), 0, a.stream,
                       static_cast<const u32x4*>(p->H), n16, n16_out,
                       reinterpret_cast<u32x4*>(ws + pl.off_hpad));
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

hipError_t launch_split(const float* H, long long n_elems, long long n_out, uint16_t* hi,
                        uint16_t* lo, hipStream_t stream) {
  if (n_out <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_split, dim3(split_blocks(n_out, 256)), dim3(256), 0, stream, H, n_elems,
                     n_out, hi, lo);
  return hipGetLastError();
}

}  // namespace jet
