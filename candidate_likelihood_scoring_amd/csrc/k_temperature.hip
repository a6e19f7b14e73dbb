// Temperature fitting: the T in [T_min, T_max] minimising the mean gold NLL over labelled
// questions (gemma-e2b doc, "Output contracts": temperature fitting; nimble, "V2
// probability default": T scales candidate scores once, before the softmax).  The gold NLL
// is the decision's: LSE(s/T) - LSE(s/T over the candidates of the gold text).
//
// Each round evaluates 64 temperatures spaced evenly in log T over the current interval,
// one per lane.  k_fit_partial: wave w of the launch takes questions w, w + W, ... (W waves
// in all) and every lane accumulates its temperature's NLL over them in question order; a
// workgroup adds its 4 waves in order into one partial per temperature.  There are up to
// 1024 workgroups, one wave per question up to 4096 questions: a wave's questions run one
// after another, so the question count per wave sets the kernel's length.  k_fit_reduce (16
// waves): wave w adds the partials of the w-th contiguous slice of workgroups in order, wave
// 0 adds the 16 slice sums in order, takes the argmin (lowest index on ties, NaN last) and
// narrows the interval to the two neighbouring grid points, kept in the workspace for the
// next round.  Six rounds shrink the spacing from ln(T_max / T_min) / 63
// by (2/63)^5, below fp32 resolution of ln T.  Questions with no label (gold id < 0) or no
// candidate of the gold text are not counted.  The result is bitwise reproducible.
#include <algorithm>

#include "jet_internal.h"

namespace jet {
namespace {

constexpr int kGrid = 64, kRounds = 6, kMaxBlocks = 1024, kReduceWaves = 16;

__device__ inline float grid_point(float lo, float hi, int g) {
  return lo + (hi - lo) * (float)g / (float)(kGrid - 1);
}

__global__ __launch_bounds__(256) void k_fit_partial(
    const float* __restrict__ s, const int* __restrict__ q_cand_off, int n_q, int n_cand,
    const int* __restrict__ text, const int* __restrict__ gold, const float* __restrict__ iv,
    float lo0, float hi0, float* __restrict__ part, int* __restrict__ cnt,
    int32_t* __restrict__ flags) {
  __shared__ float wpart[4][kGrid];
  __shared__ int wcnt[4];
  const int g = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const float lo = iv ? iv[0] : lo0, hi = iv ? iv[1] : hi0;
  const float inv_t = expf(-grid_point(lo, hi, g));
  const int W = gridDim.x * 4;
  float acc = 0.f;
  int used = 0;
  bool bad = false;
  for (int q = blockIdx.x * 4 + wv; q < n_q; q += W) {
    const int c0 = q_cand_off[q], c1 = q_cand_off[q + 1];
    if (c0 < 0 || c1 > n_cand || c1 <= c0) {
      bad = true;
      continue;
    }
    const int gt = gold[q];
    if (gt < 0) continue;
    // The question's scores and text ids arrive 64 at a time, one per lane, in one coalesced
    // load; each candidate is then broadcast from its lane, so the loops below wait on one
    // load per 64 candidates instead of one per candidate.  Candidates are visited in order.
    float M = -INFINITY, Mg = -INFINITY;
    for (int b = c0; b < c1; b += kGrid) {
      const int n = min(kGrid, c1 - b);
      const float sv = g < n ? s[b + g] : 0.f;
      const int tv = g < n ? text[b + g] : 0;
      for (int j = 0; j < n; ++j) {
        const float a = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(sv), j)) * inv_t;
        M = fmaxf(M, a);
        if (__builtin_amdgcn_readlane(tv, j) == gt) Mg = fmaxf(Mg, a);
      }
    }
    if (Mg == -INFINITY) continue;  // no candidate of the gold text
    float Z = 0.f, Zg = 0.f;
    for (int b = c0; b < c1; b += kGrid) {
      const int n = min(kGrid, c1 - b);
      const float sv = g < n ? s[b + g] : 0.f;
      const int tv = g < n ? text[b + g] : 0;
      for (int j = 0; j < n; ++j) {
        const float a = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(sv), j)) * inv_t;
        Z += expf(a - M);
        if (__builtin_amdgcn_readlane(tv, j) == gt) Zg += expf(a - Mg);
      }
    }
    acc += (M + logf(Z)) - (Mg + logf(Zg));
    ++used;
  }
  if (bad && g == 0 && flags) flag_or(flags, JET_FLAG_BAD_OFFSETS);
  wpart[wv][g] = acc;
  if (g == 0) wcnt[wv] = used;
  __syncthreads();
  if (wv == 0) {
    part[(size_t)blockIdx.x * kGrid + g] = ((wpart[0][g] + wpart[1][g]) + wpart[2][g]) + wpart[3][g];
    if (g == 0) cnt[blockIdx.x] = wcnt[0] + wcnt[1] + wcnt[2] + wcnt[3];
  }
}

__global__ __launch_bounds__(kReduceWaves * 64) void k_fit_reduce(
    const float* __restrict__ part, const int* __restrict__ cnt, int nb, float* __restrict__ iv,
    float lo0, float hi0, int first, int last, float* __restrict__ T_out,
    float* __restrict__ nll_out) {
  __shared__ float wsum[kReduceWaves][kGrid];
  __shared__ int wn[kReduceWaves];
  const int g = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int per = (nb + kReduceWaves - 1) / kReduceWaves;
  const int b0 = min(nb, w * per), b1 = min(nb, b0 + per);
  float tot = 0.f;
  int n = 0;
#pragma unroll 8
  for (int b = b0; b < b1; ++b) {
    tot += part[(size_t)b * kGrid + g];
    n += cnt[b];
  }
  wsum[w][g] = tot;
  if (g == 0) wn[w] = n;
  __syncthreads();
  if (w != 0) return;
  tot = 0.f;
  n = 0;
  for (int v = 0; v < kReduceWaves; ++v) {
    tot += wsum[v][g];
    n += wn[v];
  }
  const float lo = first ? lo0 : iv[0], hi = first ? hi0 : iv[1];
  const float u = grid_point(lo, hi, g);
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
  if (g == bi) {  // every lane has read the interval above: the wave runs in lockstep
    if (!last) {
      const float step = (hi - lo) / (float)(kGrid - 1);
      iv[0] = bi > 0 ? u - step : u;
      iv[1] = bi < kGrid - 1 ? u + step : u;
    } else {
      T_out[0] = n ? expf(u) : __builtin_nanf("");
      nll_out[0] = f;
    }
  }
}

__global__ void k_temp_clear(int32_t* __restrict__ flags) {
  if (threadIdx.x == 0) flags[0] = 0;
}

int fit_blocks(int n_q) { return std::max(1, std::min(kMaxBlocks, (n_q + 3) / 4)); }

}  // namespace

size_t fit_temperature_workspace(int n_q) {
  const size_t nb = (size_t)fit_blocks(n_q);
  return (nb * kGrid * 4 + 255) / 256 * 256 + (nb * 4 + 255) / 256 * 256 + 256;
}

hipError_t launch_fit_temperature(const float* s, const int* q_cand_off, int n_q, int n_cand,
                                  const int* text, const int* gold, float T_min, float T_max,
                                  float* T_out, float* nll_out, int32_t* flags, char* ws,
                                  hipStream_t stream) {
  hipError_t e;
  const int nb = fit_blocks(n_q);
  float* part = reinterpret_cast<float*>(ws);
  int* cnt = reinterpret_cast<int*>(ws + ((size_t)nb * kGrid * 4 + 255) / 256 * 256);
  float* iv = reinterpret_cast<float*>(reinterpret_cast<char*>(cnt) + ((size_t)nb * 4 + 255) / 256 * 256);
  if (flags) {
    hipLaunchKernelGGL(k_temp_clear, dim3(1), dim3(64), 0, stream, flags);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  const float lo0 = logf(T_min), hi0 = logf(T_max);
  for (int round = 0; round < kRounds; ++round) {
    hipLaunchKernelGGL(k_fit_partial, dim3(nb), dim3(256), 0, stream, s, q_cand_off, n_q, n_cand,
                       text, gold, round ? iv : nullptr, lo0, hi0, part, cnt, flags);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    hipLaunchKernelGGL(k_fit_reduce, dim3(1), dim3(kReduceWaves * 64), 0, stream, part, cnt, nb, iv, lo0, hi0,
                       round == 0 ? 1 : 0, round + 1 == kRounds ? 1 : 0, T_out, nll_out);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace jet
