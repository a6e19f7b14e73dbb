// Fused LM-head projection + online full-vocabulary logsumexp + target-logit capture for
// up to 32 predictor rows per row tile ("small-row" kernel, HBM-bound on the head).
//
// What it computes (JET paper, Eq. 1-2; FastJEV Sec. 3.3, candidate-preserving readout):
// for each row r of a 32-row tile and every vocabulary entry v, z[r,v] = <H[r], W[v]>
// with fp32 accumulation on the matrix cores; the logits stay in registers.  Each wave
// folds its logits into a running (max, sum of exp) per row, and writes the logit of
// every scored (row, target) pair that falls in its vocabulary range ("only candidate
// log-probabilities leave the kernel", JET Sec. on GPU scoring).  A workgroup's waves
// merge their running states in a fixed order and store one (m, s) partial per row.
//
// Matrix-core mapping (gfx950, 64-lane waves): the head is the A operand (vocabulary as
// M), the hidden states are the B operand (rows as N), both K(=d)-contiguous.  One
// v_mfma_f32_32x32x16_bf16 consumes a 32x16 slice of W and a 16x32 slice of H; lane l
// supplies row m = l % 32 and 8 consecutive k of its half (l / 32).  K is permuted per
// 32-wide block so that each lane loads 32 contiguous bytes of its row: in block kb the
// lane's half h holds k = kb + 16 h + 8 j + e for MFMA step j in {0, 1}.  A and B use the
// same permutation, so the sum over the block is unchanged.  Output element (m, n) of a
// 32x32 tile lives in lane n + 32 * ((m >> 2) & 1), register 4 * (m >> 3) + (m & 3).
//
// fp32 H with a bf16 head: H = hi + lo with hi = bf16(H), lo = bf16(H - hi); two MFMAs
// accumulate W*hi + W*lo, keeping about 16 significant bits of H (the page's systems use
// bf16 weights with fp32 accumulation, nimble "Correctness and limits").
#include "jet_internal.h"

namespace jet {
namespace {

constexpr int kWpb = 4;  // waves per workgroup

struct Frag32B {
  uint4 x, y;
};

__device__ inline Frag32B ld32(const uint16_t* p) {
  const uint4* q = reinterpret_cast<const uint4*>(p);
  Frag32B f;
  f.x = q[0];
  f.y = q[1];
  return f;
}

__device__ inline bf16x8 as_bf16x8(uint4 v) { return __builtin_bit_cast(bf16x8, v); }

// Vocabulary index (relative to the tile) held by register i of lane half h.
__device__ inline int tile_m(int i, int h) { return 8 * (i >> 2) + 4 * h + (i & 3); }

template <int NT>
struct Acc {
  f32x16 t[NT];
};

// Fold one group's logits into the lane's running (m, s) state; capture the targets in
// the group.  Shared by the bf16 and fp32 kernels.
template <int NT>
__device__ inline void epilogue_lse(const Acc<NT>& acc, int v0, int V, int n, int half,
                                    int row0, const int* __restrict__ b_off,
                                    const int* __restrict__ b_tok, int bkey,
                                    const int* __restrict__ tok_row,
                                    const int* __restrict__ tok_target,
                                    float* __restrict__ z_tgt, float& m_run, float& s_run) {
  float gm = -INFINITY;
#pragma unroll
  for (int t = 0; t < NT; ++t)
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int v = v0 + 32 * t + tile_m(i, half);
      if (v < V) gm = fmaxf(gm, acc.t[t][i]);
    }
  const float mn = fmaxf(m_run, gm);
  if (mn != -INFINITY) {
    const float mb = mn * kLog2e;
    float sum = 0.f;
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int v = v0 + 32 * t + tile_m(i, half);
        if (v < V) sum += exp2f(fmaf(acc.t[t][i], kLog2e, -mb));
      }
    s_run = s_run * exp2f((m_run - mn) * kLog2e) + sum;
    m_run = mn;
  }
  // Target capture: the bucket lists the tokens whose (row tile, vocabulary group) is
  // this one; the lane holding (row, target) writes the raw logit.
  const int e0 = b_off[bkey], e1 = b_off[bkey + 1];
  for (int e = e0; e < e1; ++e) {
    const int k = b_tok[e];
    const int r = tok_row ? tok_row[k] : k;
    const int lv = tok_target[k] - v0;
    const int mm = lv & 31;
    if (n == r - row0 && half == ((mm >> 2) & 1)) {
      const int tt = lv >> 5, ii = ((mm >> 3) << 2) | (mm & 3);
      float val = 0.f;
#pragma unroll
      for (int t = 0; t < NT; ++t)
#pragma unroll
        for (int i = 0; i < 16; ++i)
          if (t == tt && i == ii) val = acc.t[t][i];
      z_tgt[k] = val;
    }
  }
}

// Merge the two lane halves, then the workgroup's waves in wave order; store one partial
// per row of the tile.
__device__ inline void store_partial(float m_run, float s_run, int n, int half, int wid,
                                     int row0, int n_rows, float2* __restrict__ part,
                                     float2 (*red)[32]) {
  {
    const float m2 = __shfl_xor(m_run, 32);
    const float s2 = __shfl_xor(s_run, 32);
    lse_merge(m_run, s_run, m2, s2);
  }
  if (half == 0) red[wid][n] = make_float2(m_run, s_run);
  __syncthreads();
  if (threadIdx.x < 32) {
    float m = red[0][n].x, s = red[0][n].y;
#pragma unroll
    for (int w = 1; w < kWpb; ++w) lse_merge(m, s, red[w][n].x, red[w][n].y);
    const int row = row0 + n;
    if (row < n_rows) part[(size_t)blockIdx.x * n_rows + row] = make_float2(m, s);
  }
}

// Store epilogue (restricted path): Z[row][v] for valid rows and vocabulary entries.
template <int NT>
__device__ inline void epilogue_store(const Acc<NT>& acc, int v0, int V, int n, int half,
                                      int row0, int n_rows, float* __restrict__ Z) {
  const int row = row0 + n;
  if (row >= n_rows) return;
#pragma unroll
  for (int t = 0; t < NT; ++t)
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int v = v0 + 32 * t + tile_m(i, half);
      if (v < V) Z[(size_t)row * V + v] = acc.t[t][i];
    }
}

// ------------------------------------------------------------------------------------
// bf16 head
// ------------------------------------------------------------------------------------
template <int NT, bool HILO, bool STORE>
__global__ __launch_bounds__(256) void k_project_small_bf16(
    const uint16_t* __restrict__ W, int V, int d, const uint16_t* __restrict__ Hhi,
    const uint16_t* __restrict__ Hlo, int n_rows, int n_groups, const int* __restrict__ b_off,
    const int* __restrict__ b_tok, const int* __restrict__ tok_row,
    const int* __restrict__ tok_target, float* __restrict__ z_tgt, float2* __restrict__ part,
    float* __restrict__ Z) {
  __shared__ float2 red[kWpb][32];
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const int n = lane & 31, half = lane >> 5;
  const int rt = blockIdx.y, row0 = rt * 32;
  const int hrow = min(row0 + n, n_rows - 1);
  const uint16_t* hp = Hhi + (size_t)hrow * d + half * 16;
  const uint16_t* lp = HILO ? Hlo + (size_t)hrow * d + half * 16 : nullptr;
  const long long nw = (long long)gridDim.x * kWpb;
  const long long w = (long long)blockIdx.x * kWpb + wid;
  const int g0 = (int)(w * n_groups / nw), g1 = (int)((w + 1) * n_groups / nw);
  float m_run = -INFINITY, s_run = 0.f;

  for (int g = g0; g < g1; ++g) {
    const int v0 = g * (32 * NT);
    const uint16_t* wp[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) wp[t] = W + (size_t)min(v0 + 32 * t + n, V - 1) * d + half * 16;
    Acc<NT> acc;
#pragma unroll
    for (int t = 0; t < NT; ++t) acc.t[t] = f32x16{};

    Frag32B a0[NT], a1[NT], bh0, bh1, bl0, bl1;
#define JET_LOAD(A, BH, BL, KB)                                    \
  {                                                                \
    _Pragma("unroll") for (int t = 0; t < NT; ++t) A[t] = ld32(wp[t] + (KB)); \
    BH = ld32(hp + (KB));                                          \
    if (HILO) BL = ld32(lp + (KB));                                \
  }
#define JET_MMA(A, BH, BL)                                                                   \
  {                                                                                          \
    _Pragma("unroll") for (int t = 0; t < NT; ++t) {                                         \
      acc.t[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(A[t].x), as_bf16x8(BH.x), \
                                                        acc.t[t], 0, 0, 0);                  \
      if (HILO)                                                                              \
        acc.t[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(A[t].x),                \
                                                          as_bf16x8(BL.x), acc.t[t], 0, 0, 0); \
      acc.t[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(A[t].y), as_bf16x8(BH.y), \
                                                        acc.t[t], 0, 0, 0);                  \
      if (HILO)                                                                              \
        acc.t[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(A[t].y),                \
                                                          as_bf16x8(BL.y), acc.t[t], 0, 0, 0); \
    }                                                                                        \
  }
    JET_LOAD(a0, bh0, bl0, 0);
    for (int kb = 0; kb < d; kb += 64) {
      if (kb + 32 < d) JET_LOAD(a1, bh1, bl1, kb + 32);
      JET_MMA(a0, bh0, bl0);
      if (kb + 64 < d) JET_LOAD(a0, bh0, bl0, kb + 64);
      if (kb + 32 < d) JET_MMA(a1, bh1, bl1);
    }
#undef JET_LOAD
#undef JET_MMA
    if (STORE)
      epilogue_store<NT>(acc, v0, V, n, half, row0, n_rows, Z);
    else
      epilogue_lse<NT>(acc, v0, V, n, half, row0, b_off, b_tok, rt * n_groups + g, tok_row,
                       tok_target, z_tgt, m_run, s_run);
  }
  if (!STORE) store_partial(m_run, s_run, n, half, wid, row0, n_rows, part, red);
}

// ------------------------------------------------------------------------------------
// fp32 head and fp32 hidden states: v_mfma_f32_32x32x2_f32, one k per lane half per
// step; lane half h loads 4 consecutive k (a float4) of its row per 8-wide block and
// step j uses k = kb + 4 h + j.
// ------------------------------------------------------------------------------------
template <int NT, bool STORE>
__global__ __launch_bounds__(256) void k_project_small_f32(
    const float* __restrict__ W, int V, int d, const float* __restrict__ H, int n_rows,
    int n_groups, const int* __restrict__ b_off, const int* __restrict__ b_tok,
    const int* __restrict__ tok_row, const int* __restrict__ tok_target,
    float* __restrict__ z_tgt, float2* __restrict__ part, float* __restrict__ Z) {
  __shared__ float2 red[kWpb][32];
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const int n = lane & 31, half = lane >> 5;
  const int rt = blockIdx.y, row0 = rt * 32;
  const int hrow = min(row0 + n, n_rows - 1);
  const float* hp = H + (size_t)hrow * d + half * 4;
  const long long nw = (long long)gridDim.x * kWpb;
  const long long w = (long long)blockIdx.x * kWpb + wid;
  const int g0 = (int)(w * n_groups / nw), g1 = (int)((w + 1) * n_groups / nw);
  float m_run = -INFINITY, s_run = 0.f;
  for (int g = g0; g < g1; ++g) {
    const int v0 = g * (32 * NT);
    const float* wp[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) wp[t] = W + (size_t)min(v0 + 32 * t + n, V - 1) * d + half * 4;
    Acc<NT> acc;
#pragma unroll
    for (int t = 0; t < NT; ++t) acc.t[t] = f32x16{};
    float4 a0[NT], a1[NT], b0, b1;
    auto load = [&](float4* A, float4& B, int kb) {
#pragma unroll
      for (int t = 0; t < NT; ++t) A[t] = *reinterpret_cast<const float4*>(wp[t] + kb);
      B = *reinterpret_cast<const float4*>(hp + kb);
    };
    auto mma = [&](const float4* A, const float4& B) {
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        acc.t[t] = __builtin_amdgcn_mfma_f32_32x32x2f32(A[t].x, B.x, acc.t[t], 0, 0, 0);
        acc.t[t] = __builtin_amdgcn_mfma_f32_32x32x2f32(A[t].y, B.y, acc.t[t], 0, 0, 0);
        acc.t[t] = __builtin_amdgcn_mfma_f32_32x32x2f32(A[t].z, B.z, acc.t[t], 0, 0, 0);
        acc.t[t] = __builtin_amdgcn_mfma_f32_32x32x2f32(A[t].w, B.w, acc.t[t], 0, 0, 0);
      }
    };
    load(a0, b0, 0);
    for (int kb = 0; kb < d; kb += 16) {
      if (kb + 8 < d) load(a1, b1, kb + 8);
      mma(a0, b0);
      if (kb + 16 < d) load(a0, b0, kb + 16);
      if (kb + 8 < d) mma(a1, b1);
    }
    if (STORE)
      epilogue_store<NT>(acc, v0, V, n, half, row0, n_rows, Z);
    else
      epilogue_lse<NT>(acc, v0, V, n, half, row0, b_off, b_tok, rt * n_groups + g, tok_row,
                       tok_target, z_tgt, m_run, s_run);
  }
  if (!STORE) store_partial(m_run, s_run, n, half, wid, row0, n_rows, part, red);
}

}  // namespace

// Tiles per vocabulary group of the small-row kernels (a group is 32 * NT entries).  Two
// tiles keep the bf16 kernel at 2 resident waves per SIMD.
#ifndef JET_SMALL_NT
#define JET_SMALL_NT 2
#endif
constexpr int kSmallNT = JET_SMALL_NT;
constexpr int kSmallNTf32 = 2;

hipError_t launch_project(const ScoreArgs& a) {
  const jet_problem* p = a.p;
  const Plan& pl = *a.plan;
  const int* b_off = reinterpret_cast<const int*>(a.ws + pl.off_boff);
  const int* b_tok = reinterpret_cast<const int*>(a.ws + pl.off_btok);
  float* z_tgt = reinterpret_cast<float*>(a.ws + pl.off_ztgt);
  float2* part = reinterpret_cast<float2*>(a.ws + pl.off_part);
  dim3 grid(pl.grid_x, pl.n_rtiles), block(256);
  if (pl.variant == VAR_SMALL_BF16) {
    const uint16_t* W = static_cast<const uint16_t*>(p->W);
    if (pl.hilo) {
      const uint16_t* hhi = reinterpret_cast<const uint16_t*>(a.ws + pl.off_hhi);
      const uint16_t* hlo = reinterpret_cast<const uint16_t*>(a.ws + pl.off_hlo);
      hipLaunchKernelGGL((k_project_small_bf16<kSmallNT, true, false>), grid, block, 0, a.stream,
                         W, p->V, p->d, hhi, hlo, p->n_rows, pl.n_vgroups, b_off, b_tok,
                         p->tok_row, p->tok_target, z_tgt, part, nullptr);
    } else {
      const uint16_t* h = static_cast<const uint16_t*>(p->H);
      hipLaunchKernelGGL((k_project_small_bf16<kSmallNT, false, false>), grid, block, 0,
                         a.stream, W, p->V, p->d, h, nullptr, p->n_rows, pl.n_vgroups, b_off,
                         b_tok, p->tok_row, p->tok_target, z_tgt, part, nullptr);
    }
  } else if (pl.variant == VAR_SMALL_F32) {
    hipLaunchKernelGGL((k_project_small_f32<kSmallNTf32, false>), grid, block, 0, a.stream,
                       static_cast<const float*>(p->W), p->V, p->d,
                       static_cast<const float*>(p->H), p->n_rows, pl.n_vgroups, b_off, b_tok,
                       p->tok_row, p->tok_target, z_tgt, part, nullptr);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

int small_group_size(int variant) { return 32 * (variant == VAR_SMALL_F32 ? kSmallNTf32 : kSmallNT); }

static int store_grid(int n_groups) {
  int g = (n_groups + kWpb - 1) / kWpb;
  return g < 1 ? 1 : g;
}

hipError_t launch_project_store_bf16(const uint16_t* Wu, int U, int d, const uint16_t* Hhi,
                                     const uint16_t* Hlo, int n_rows, float* Z,
                                     hipStream_t stream) {
  const int n_groups = (U + 31) / 32;
  dim3 grid(store_grid(n_groups), (n_rows + 31) / 32), block(256);
  if (Hlo)
    hipLaunchKernelGGL((k_project_small_bf16<1, true, true>), grid, block, 0, stream, Wu, U, d,
                       Hhi, Hlo, n_rows, n_groups, nullptr, nullptr, nullptr, nullptr, nullptr,
                       nullptr, Z);
  else
    hipLaunchKernelGGL((k_project_small_bf16<1, false, true>), grid, block, 0, stream, Wu, U, d,
                       Hhi, nullptr, n_rows, n_groups, nullptr, nullptr, nullptr, nullptr,
                       nullptr, nullptr, Z);
  return hipGetLastError();
}

hipError_t launch_project_store_f32(const float* Wu, int U, int d, const float* H, int n_rows,
                                    float* Z, hipStream_t stream) {
  const int n_groups = (U + 31) / 32;
  dim3 grid(store_grid(n_groups), (n_rows + 31) / 32), block(256);
  hipLaunchKernelGGL((k_project_small_f32<1, true>), grid, block, 0, stream, Wu, U, d, H, n_rows,
                     n_groups, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, Z);
  return hipGetLastError();
}

}  // namespace jet
