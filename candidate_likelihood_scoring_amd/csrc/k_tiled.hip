// Large-row fused projection + online full-vocabulary logsumexp + target capture
// (matrix-core bound when rows >> 300: 2 * rows flop per head byte).
//
// Computes the same quantities as the small-row kernels (JET paper, Eq. 1-2; FastJEV
// Sec. 3.3): z[r, v] = <H[r], W[v]> with fp32 accumulation, folded into a running
// (max, sum of exp) per row, plus the logit of every scored (row, target) pair.
//
// Tiling (gfx950): a workgroup of 4 waves owns a 256-row tile of H and sweeps a contiguous
// range of 256-entry vocabulary tiles.  Each wave computes a 128 x 128 quadrant (vocabulary
// x rows) as 4 x 4 tiles of v_mfma_f32_32x32x16_bf16, i.e. 256 fp32 accumulators per lane.
// K advances in BK-wide stages staged through LDS, double buffered: the next stage is
// loaded into registers with lane-contiguous 16-byte loads (8 lanes cover one 128-byte row
// segment) while the current stage feeds the matrix cores, then written to the other
// buffer; one barrier per stage.  LDS chunk (row r, 16-byte chunk c) lives at
// r * CH + (c ^ ((r / (8 / CH)) % CH)), which keeps the row-wise writes and the 32-row
// fragment reads conflict-free.  Fragment k layout: lane half h, sub-step kk reads chunk
// 2 kk + h of its row for both operands (any k permutation shared by A and B gives the
// same dot product).
//
// H in one bf16 plane (bf16 hidden states) or two (fp32 hidden states split into hi + lo,
// each product accumulated twice); with two planes BK halves so a stage still fits.
#include "jet_internal.h"

namespace jet {
namespace {

constexpr int TBM = 256;  // vocabulary entries per block tile
constexpr int TBN = 256;  // rows per block tile

__device__ inline int tm_of(int i, int h) { return 8 * (i >> 2) + 4 * h + (i & 3); }

template <int CH>
__device__ inline int lds_slot(int r, int c) {
  constexpr int RPL = 8 / CH;  // rows per 128-byte bank line
  return r * CH + (c ^ ((r / RPL) % CH));
}

template <int NP>
__global__ __launch_bounds__(256, 1) void k_project_tiled_bf16(
    const uint16_t* __restrict__ W, int V, int d, const uint16_t* __restrict__ H0,
    const uint16_t* __restrict__ H1, int n_rows, int n_vtiles, const int* __restrict__ b_off,
    const int* __restrict__ b_tok, const int* __restrict__ tok_row,
    const int* __restrict__ tok_target, float* __restrict__ z_tgt, float2* __restrict__ part) {
  constexpr int BK = NP == 1 ? 64 : 32;
  constexpr int CH = BK / 8;          // 16-byte chunks per row per stage
  constexpr int KK = BK / 16;         // MFMA k sub-steps per stage
  constexpr int LA = TBM * CH / 256;  // A chunks loaded per thread per stage
  constexpr int LB = TBN * CH / 256;  // B chunks per plane per thread per stage
  __shared__ u32x4 sA[2][TBM * CH];
  __shared__ u32x4 sB[2][NP][TBN * CH];
  __shared__ float2 red[2][TBN];

  const int tid = threadIdx.x, wid = tid >> 6, lane = tid & 63;
  const int wm = wid & 1, wn = wid >> 1;
  const int n = lane & 31, h = lane >> 5;
  const int rt = blockIdx.y, row0 = rt * TBN;
  const int t0 = (int)((long long)blockIdx.x * n_vtiles / gridDim.x);
  const int t1 = (int)((long long)(blockIdx.x + 1) * n_vtiles / gridDim.x);
  const int nk = d / BK;

  // global -> LDS mapping: chunk q = i * 256 + tid -> tile row q / CH, chunk q % CH
  const uint16_t* hsrc[NP][LB];
  int b_slot[LB];
#pragma unroll
  for (int i = 0; i < LB; ++i) {
    const int q = i * 256 + tid, r = q / CH, c = q % CH;
    const size_t off = (size_t)min(row0 + r, n_rows - 1) * d + c * 8;
    hsrc[0][i] = H0 + off;
    if (NP == 2) hsrc[NP - 1][i] = H1 + off;
    b_slot[i] = lds_slot<CH>(r, c);
  }
  int a_slot[LA], a_row[LA], a_c[LA];
#pragma unroll
  for (int i = 0; i < LA; ++i) {
    const int q = i * 256 + tid;
    a_row[i] = q / CH;
    a_c[i] = q % CH;
    a_slot[i] = lds_slot<CH>(a_row[i], a_c[i]);
  }

  // running (max, sum) of the lane's 4 rows: row0 + wn*128 + nt*32 + n
  float m_run[4], s_run[4];
#pragma unroll
  for (int nt = 0; nt < 4; ++nt) {
    m_run[nt] = -INFINITY;
    s_run[nt] = 0.f;
  }

  for (int vt = t0; vt < t1; ++vt) {
    const int v0 = vt * TBM;
    const uint16_t* wsrc[LA];
#pragma unroll
    for (int i = 0; i < LA; ++i) wsrc[i] = W + (size_t)min(v0 + a_row[i], V - 1) * d + a_c[i] * 8;

    f32x16 acc[4][4];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) acc[mt][nt] = f32x16{};

    u32x4 ra[LA], rb[NP][LB];
    // stage 0 -> buffer 0
#pragma unroll
    for (int i = 0; i < LA; ++i) ra[i] = *reinterpret_cast<const u32x4*>(wsrc[i]);
#pragma unroll
    for (int p = 0; p < NP; ++p)
#pragma unroll
      for (int i = 0; i < LB; ++i) rb[p][i] = *reinterpret_cast<const u32x4*>(hsrc[p][i]);
#pragma unroll
    for (int i = 0; i < LA; ++i) sA[0][a_slot[i]] = ra[i];
#pragma unroll
    for (int p = 0; p < NP; ++p)
#pragma unroll
      for (int i = 0; i < LB; ++i) sB[0][p][b_slot[i]] = rb[p][i];
    __syncthreads();

    for (int ks = 0; ks < nk; ++ks) {
      const int buf = ks & 1;
      const int kn = min(ks + 1, nk - 1) * BK;  // next stage (re-reads the last at the end)
#pragma unroll
      for (int i = 0; i < LA; ++i) ra[i] = *reinterpret_cast<const u32x4*>(wsrc[i] + kn);
#pragma unroll
      for (int p = 0; p < NP; ++p)
#pragma unroll
        for (int i = 0; i < LB; ++i) rb[p][i] = *reinterpret_cast<const u32x4*>(hsrc[p][i] + kn);

#pragma unroll
      for (int kk = 0; kk < KK; ++kk) {
        const int c = 2 * kk + h;
        bf16x8 fa[4], fb[NP][4];
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
          fa[mt] = __builtin_bit_cast(bf16x8, sA[buf][lds_slot<CH>(wm * 128 + mt * 32 + n, c)]);
#pragma unroll
        for (int p = 0; p < NP; ++p)
#pragma unroll
          for (int nt = 0; nt < 4; ++nt)
            fb[p][nt] = __builtin_bit_cast(bf16x8, sB[buf][p][lds_slot<CH>(wn * 128 + nt * 32 + n, c)]);
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
#pragma unroll
          for (int nt = 0; nt < 4; ++nt)
#pragma unroll
            for (int p = 0; p < NP; ++p)
              acc[mt][nt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[mt], fb[p][nt], acc[mt][nt], 0, 0, 0);
      }
      // the other buffer was last read before the previous barrier
#pragma unroll
      for (int i = 0; i < LA; ++i) sA[buf ^ 1][a_slot[i]] = ra[i];
#pragma unroll
      for (int p = 0; p < NP; ++p)
#pragma unroll
        for (int i = 0; i < LB; ++i) sB[buf ^ 1][p][b_slot[i]] = rb[p][i];
      __syncthreads();
    }

    // online logsumexp over this tile's 128 vocabulary entries per lane row
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) {
      float gm = -INFINITY;
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int i = 0; i < 16; ++i)
          if (v0 + wm * 128 + mt * 32 + tm_of(i, h) < V) gm = fmaxf(gm, acc[mt][nt][i]);
      const float mn = fmaxf(m_run[nt], gm);
      if (mn != -INFINITY) {
        const float mb = mn * kLog2e;
        float sum = 0.f;
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
#pragma unroll
          for (int i = 0; i < 16; ++i)
            if (v0 + wm * 128 + mt * 32 + tm_of(i, h) < V)
              sum += exp2f(fmaf(acc[mt][nt][i], kLog2e, -mb));
        s_run[nt] = s_run[nt] * exp2f((m_run[nt] - mn) * kLog2e) + sum;
        m_run[nt] = mn;
      }
    }
    // target capture: tokens whose (row tile, vocabulary tile) is this block tile
    const int bkey = rt * n_vtiles + vt;
    const int e0 = b_off[bkey], e1 = b_off[bkey + 1];
    for (int e = e0; e < e1; ++e) {
      const int k = b_tok[e];
      const int lr = (tok_row ? tok_row[k] : k) - row0;
      const int lv = tok_target[k] - v0;
      if (lv < 0 || lv >= TBM || lr < 0 || lr >= TBN) continue;
      if ((lv >> 7) != wm || (lr >> 7) != wn) continue;  // wave-uniform
      const int tmt = (lv >> 5) & 3, tnt = (lr >> 5) & 3, mm = lv & 31;
      if (n == (lr & 31) && h == ((mm >> 2) & 1)) {
        const int ti = ((mm >> 3) << 2) | (mm & 3);
        float val = 0.f;
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
#pragma unroll
          for (int nt = 0; nt < 4; ++nt)
            if (mt == tmt && nt == tnt) {
#pragma unroll
              for (int i = 0; i < 16; ++i)
                if (i == ti) val = acc[mt][nt][i];
            }
        z_tgt[k] = val;
      }
    }
  }

  // merge lane halves, then the two vocabulary halves (wm = 0 then 1) of each row
#pragma unroll
  for (int nt = 0; nt < 4; ++nt) {
    const float m2 = __shfl_xor(m_run[nt], 32), s2 = __shfl_xor(s_run[nt], 32);
    lse_merge(m_run[nt], s_run[nt], m2, s2);
    if (h == 0) red[wm][wn * 128 + nt * 32 + n] = make_float2(m_run[nt], s_run[nt]);
  }
  __syncthreads();
  {
    const int r = tid;  // 256 threads, 256 rows
    float m = red[0][r].x, s = red[0][r].y;
    lse_merge(m, s, red[1][r].x, red[1][r].y);
    if (row0 + r < n_rows) part[(size_t)blockIdx.x * n_rows + row0 + r] = make_float2(m, s);
  }
}

}  // namespace

int tiled_bk(bool hilo) { return hilo ? 32 : 64; }

hipError_t launch_project_tiled(const ScoreArgs& a) {
  const jet_problem* p = a.p;
  const Plan& pl = *a.plan;
  const int* b_off = reinterpret_cast<const int*>(a.ws + pl.off_boff);
  const int* b_tok = reinterpret_cast<const int*>(a.ws + pl.off_btok);
  float* z_tgt = reinterpret_cast<float*>(a.ws + pl.off_ztgt);
  float2* part = reinterpret_cast<float2*>(a.ws + pl.off_part);
  dim3 grid(pl.grid_x, pl.n_rtiles), block(256);
  const uint16_t* W = static_cast<const uint16_t*>(p->W);
  if (pl.hilo) {
    const uint16_t* hhi = reinterpret_cast<const uint16_t*>(a.ws + pl.off_hhi);
    const uint16_t* hlo = reinterpret_cast<const uint16_t*>(a.ws + pl.off_hlo);
    hipLaunchKernelGGL((k_project_tiled_bf16<2>), grid, block, 0, a.stream, W, p->V, p->d, hhi,
                       hlo, p->n_rows, pl.n_vgroups, b_off, b_tok, p->tok_row, p->tok_target,
                       z_tgt, part);
  } else {
    hipLaunchKernelGGL((k_project_tiled_bf16<1>), grid, block, 0, a.stream, W, p->V, p->d,
                       static_cast<const uint16_t*>(p->H), nullptr, p->n_rows, pl.n_vgroups,
                       b_off, b_tok, p->tok_row, p->tok_target, z_tgt, part);
  }
  return hipGetLastError();
}

}  // namespace jet
