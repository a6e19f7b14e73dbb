// Decision sensitivity of layer skips (FastJEV Sec. 3.4, Eq. 5-6, "Calibration Guided
// Selection"), for a calibration set of logit vectors.
//
// k_sens_d: one wave per (layer l, input x), over input x's entries [a, b):
//     delta = z_skip[l] - z ;  d[l][x] = rms(delta - mean delta) / max(eps, rms(z - mean z))
//   two passes (means, then centred sums of squares), lane-strided sums in index order
//   combined by a fixed xor tree: the result is bitwise reproducible.
// k_sens_select: one workgroup.  J[l] = (sum over x of d[l][x]) / n_inputs in the same fixed
//   order, then the rank of layer l in the order (J, index) -- NaN ranks as +inf -- so the
//   k smallest are written to selected[0..k) with ties resolved by layer index.  Ranks are
//   distinct, so every slot is written exactly once.
#include "jet_internal.h"

namespace jet {
namespace {

__device__ inline float wave_sum(float x) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) x += __shfl_xor(x, off);
  return x;
}

__global__ void k_sens_clear(int32_t* __restrict__ flags) {
  if (threadIdx.x == 0) flags[0] = 0;
}

__global__ __launch_bounds__(256) void k_sens_d(const float* __restrict__ z,
                                                const float* __restrict__ z_skip,
                                                const int* __restrict__ seg_off, int n_inputs,
                                                int n_values, int n_layers, float eps,
                                                float* __restrict__ d, int32_t* __restrict__ flags) {
  const int lane = threadIdx.x & 63;
  const long long w = (long long)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (w >= (long long)n_inputs * n_layers) return;
  const int l = (int)(w / n_inputs), x = (int)(w % n_inputs);
  const int a = seg_off[x], b = seg_off[x + 1];
  float* out = d + (size_t)l * n_inputs + x;
  if (a < 0 || b > n_values || b <= a) {
    if (lane == 0) {
      *out = __builtin_nanf("");
      if (flags) flag_or(flags, JET_FLAG_BAD_OFFSETS);
    }
    return;
  }
  const float* zs = z_skip + (size_t)l * n_values;
  float sz = 0.f, sd = 0.f;
  for (int i = a + lane; i < b; i += 64) {
    sz += z[i];
    sd += zs[i] - z[i];
  }
  const float m = (float)(b - a);
  const float mz = wave_sum(sz) / m, md = wave_sum(sd) / m;
  float qz = 0.f, qd = 0.f;
  for (int i = a + lane; i < b; i += 64) {
    const float u = z[i] - mz, v = (zs[i] - z[i]) - md;
    qz = fmaf(u, u, qz);
    qd = fmaf(v, v, qd);
  }
  const float rz = sqrtf(wave_sum(qz) / m), rd = sqrtf(wave_sum(qd) / m);
  if (lane == 0) *out = rd / fmaxf(eps, rz);
}

constexpr int kMaxLayers = 4096;

__global__ __launch_bounds__(1024) void k_sens_select(const float* __restrict__ d, int n_inputs,
                                                      int n_layers, int k, float* __restrict__ J,
                                                      int32_t* __restrict__ selected) {
  __shared__ float sJ[kMaxLayers];
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  for (int l = wv; l < n_layers; l += 16) {
    float s = 0.f;
    for (int x = lane; x < n_inputs; x += 64) s += d[(size_t)l * n_inputs + x];
    const float j = wave_sum(s) / (float)n_inputs;
    if (lane == 0) {
      J[l] = j;
      sJ[l] = j != j ? INFINITY : j;
    }
  }
  __syncthreads();
  for (int l = tid; l < n_layers; l += 1024) {
    const float j = sJ[l];
    int rank = 0;
    for (int o = 0; o < n_layers; ++o) {
      const float v = sJ[o];
      rank += (v < j) || (v == j && o < l);
    }
    if (rank < k) selected[rank] = l;
  }
}

}  // namespace

int sensitivity_max_layers() { return kMaxLayers; }

hipError_t launch_sensitivity(const float* z, const float* z_skip, const int* seg_off,
                              int n_inputs, int n_values, int n_layers, float eps, int k,
                              float* d, float* J, int32_t* selected, int32_t* flags,
                              hipStream_t stream) {
  hipError_t e;
  if (flags) {
    hipLaunchKernelGGL(k_sens_clear, dim3(1), dim3(64), 0, stream, flags);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  const long long waves = (long long)n_inputs * n_layers;
  hipLaunchKernelGGL(k_sens_d, dim3((unsigned)((waves + 3) / 4)), dim3(256), 0, stream, z, z_skip,
                     seg_off, n_inputs, n_values, n_layers, eps, d, flags);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL(k_sens_select, dim3(1), dim3(1024), 0, stream, d, n_inputs, n_layers, k, J,
                     selected);
  return hipGetLastError();
}

}  // namespace jet
