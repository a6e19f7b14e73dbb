// Temperature fitting: the T in [T_min, T_max] minimising the mean gold NLL over labelled
// questions (gemma-e2b doc, "Output contracts": temperature fitting; nimble, "V2
// probability default": T scales candidate scores once, before the softmax).  The gold NLL
// is the decision's: LSE(s/T) - LSE(s/T over the candidates of the gold text).
//
// One workgroup of 16 waves.  Each round evaluates 64 temperatures spaced evenly in log T
// over the current interval, one per lane: wave w takes questions w, w + 16, ... and every
// lane accumulates its temperature's NLL over them in question order; the 16 wave partials
// are added in wave order.  Wave 0 takes the argmin (lowest index on ties, NaN last) and
// narrows the interval to the two neighbouring grid points.  Six rounds shrink the spacing
// from ln(T_max / T_min) / 63 by (2/63)^5, below fp32 resolution of ln T.  Questions with
// no label (gold id < 0) or no candidate of the gold text are not counted.
#include "jet_internal.h"

namespace jet {
namespace {

constexpr int kGrid = 64, kRounds = 6, kWaves = 16;

__global__ __launch_bounds__(1024) void k_fit_temperature(
    const float* __restrict__ s, const int* __restrict__ q_cand_off, int n_q, int n_cand,
    const int* __restrict__ text, const int* __restrict__ gold, float lo0, float hi0,
    float* __restrict__ T_out, float* __restrict__ nll_out, int32_t* __restrict__ flags) {
  __shared__ float part[kWaves][kGrid];
  __shared__ int cnt[kWaves];
  __shared__ float iv[2];
  const int tid = threadIdx.x, g = tid & 63, wv = tid >> 6;
  if (tid == 0) {
    iv[0] = lo0;
    iv[1] = hi0;
  }
  __syncthreads();
  bool bad = false;
  for (int round = 0; round < kRounds; ++round) {
    const float lo = iv[0], hi = iv[1];
    const float u = lo + (hi - lo) * (float)g / (float)(kGrid - 1);
    const float inv_t = expf(-u);
    float acc = 0.f;
    int used = 0;
    for (int q = wv; q < n_q; q += kWaves) {
      const int c0 = q_cand_off[q], c1 = q_cand_off[q + 1];
      if (c0 < 0 || c1 > n_cand || c1 <= c0) {
        bad = true;
        continue;
      }
      const int gt = gold[q];
      if (gt < 0) continue;
      float M = -INFINITY, Mg = -INFINITY;
      for (int c = c0; c < c1; ++c) {
        const float a = s[c] * inv_t;
        M = fmaxf(M, a);
        if (text[c] == gt) Mg = fmaxf(Mg, a);
      }
      if (Mg == -INFINITY) continue;  // no candidate of the gold text
      float Z = 0.f, Zg = 0.f;
      for (int c = c0; c < c1; ++c) {
        const float a = s[c] * inv_t;
        Z += expf(a - M);
        if (text[c] == gt) Zg += expf(a - Mg);
      }
      acc += (M + logf(Z)) - (Mg + logf(Zg));
      ++used;
    }
    part[wv][g] = acc;
    if (g == 0) cnt[wv] = used;
    __syncthreads();
    if (wv == 0) {
      float tot = 0.f;
      int n = 0;
      for (int w = 0; w < kWaves; ++w) {
        tot += part[w][g];
        n += cnt[w];
      }
      const float f = n ? tot / (float)n : __builtin_nanf("");
      float bv = f != f ? INFINITY : f;
      int bi = g;
#pragma unroll
      for (int off = 32; off >= 1; off >>= 1) {
        const float ov = __shfl_xor(bv, off);
        const int oi = __shfl_xor(bi, off);
        if (ov < bv || (ov == bv && oi < bi)) {
          bv = ov;
          bi = oi;
        }
      }
      if (g == bi) {
        if (round + 1 < kRounds) {
          const float step = (hi - lo) / (float)(kGrid - 1);
          iv[0] = bi > 0 ? u - step : u;
          iv[1] = bi < kGrid - 1 ? u + step : u;
        } else {
          T_out[0] = n ? expf(u) : __builtin_nanf("");
          nll_out[0] = f;
        }
      }
    }
    __syncthreads();
  }
  if (bad && g == 0 && flags) flag_or(flags, JET_FLAG_BAD_OFFSETS);
}

__global__ void k_temp_clear(int32_t* __restrict__ flags) {
  if (threadIdx.x == 0) flags[0] = 0;
}

}  // namespace

hipError_t launch_fit_temperature(const float* s, const int* q_cand_off, int n_q, int n_cand,
                                  const int* text, const int* gold, float T_min, float T_max,
                                  float* T_out, float* nll_out, int32_t* flags,
                                  hipStream_t stream) {
  hipError_t e;
  if (flags) {
    hipLaunchKernelGGL(k_temp_clear, dim3(1), dim3(64), 0, stream, flags);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  hipLaunchKernelGGL(k_fit_temperature, dim3(1), dim3(1024), 0, stream, s, q_cand_off, n_q, n_cand,
                     text, gold, logf(T_min), logf(T_max), T_out, nll_out, flags);
  return hipGetLastError();
}

}  // namespace jet
