// Fused LM-head projection + online full-vocabulary logsumexp for few predictor rows
// ("small-row" kernels, HBM-bound on the head).
//
// What it computes (JET paper, Eq. 1-2; FastJEV Sec. 3.3, candidate-preserving readout):
// for each row r of a row tile and every vocabulary entry v, z[r,v] = <H[r], W[v]>
// with fp32 accumulation on the matrix cores; the logits stay in registers and never
// reach memory (the JET paper's GPU scoring likewise hands back only the candidates'
// log-probabilities).  Each wave folds its logits into a running (max, sum of exp) per row;
// a workgroup's waves merge their running states in a fixed order and store one (m, s)
// partial per row.  The scored (row, target) logits are computed after the projection,
// one dot product per token (k_token_logp).
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


__device__ inline bf16x8 as_bf16x8(uint4 v) { return __builtin_bit_cast(bf16x8, v); }
__device__ inline bf16x8 as_bf16x8v(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

// Vocabulary index (relative to the tile) held by register i of lane half h.
__device__ inline int tile_m(int i, int h) { return 8 * (i >> 2) + 4 * h + (i & 3); }

template <int NT>
struct Acc {
  f32x16 t[NT];
};

// Fold one group's logits into the lane's running (m, s) state.  Shared by the bf16 and fp32
// kernels; no target logit is captured here (k_token_logp computes them after the
// projection).
template <int NT>
__device__ inline void epilogue_lse(const Acc<NT>& acc, int v0, int V, int half, float& m_run,
                                    float& s_run) {
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
}

// Merge the two lane halves, then the workgroup's waves in wave order; store one partial
// per row of the tile: at part[blockIdx.x * n_rows + row], or, ROW_MAJOR (the streaming
// kernel, whose merge reads a row's partials as one contiguous run), at
// part[row * gridDim.x + blockIdx.x].
template <int NW = kWpb, bool ROW_MAJOR = false>
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
    for (int w = 1; w < NW; ++w) lse_merge(m, s, red[w][n].x, red[w][n].y);
    const int row = row0 + n;
    if (row < n_rows)
      part[ROW_MAJOR ? (size_t)row * gridDim.x + blockIdx.x : (size_t)blockIdx.x * n_rows + row] =
          make_float2(m, s);
  }
}

// Store epilogue (restricted path with an fp32 head): Z[row][v] for valid rows and
// vocabulary entries.
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
// K pipeline.  A stage holds one KB-wide block of k: lane half h covers
// [kb + h*KB/2, kb + h*KB/2 + KB/2), i.e. KB bytes (bf16) of its W row and of its H row.
// S stages rotate through registers; loads are issued S-1 blocks ahead of use and are
// never predicated (a block past the end re-reads the last block, which the caches
// serve), so the compiler can wait for exactly the block it is about to consume.
// ------------------------------------------------------------------------------------
template <int KB>
struct FragK {
  uint4 v[KB / 16];
};

template <int KB>
__device__ inline FragK<KB> ldk(const uint16_t* p) {
  FragK<KB> f;
  const uint4* q = reinterpret_cast<const uint4*>(p);
#pragma unroll
  for (int j = 0; j < KB / 16; ++j) f.v[j] = q[j];
  return f;
}

// ------------------------------------------------------------------------------------
// bf16 head
// ------------------------------------------------------------------------------------
template <int NT, int KB, int S, bool HILO>
__global__ __launch_bounds__(256) void k_project_small_bf16(
    const uint16_t* __restrict__ W, int V, int d, const uint16_t* __restrict__ Hhi,
    const uint16_t* __restrict__ Hlo, int n_rows, int n_groups, int32_t* __restrict__ flags,
    float2* __restrict__ part) {
  static_assert(KB % 32 == 0 && S >= 2, "stage shape");
  __shared__ float2 red[kWpb][32];
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const int n = lane & 31, half = lane >> 5;
  const int rt = blockIdx.y, row0 = rt * 32;
  const int hrow = min(row0 + n, n_rows - 1);
  const uint16_t* hp = Hhi + (size_t)hrow * d + half * (KB / 2);
  const uint16_t* lp = HILO ? Hlo + (size_t)hrow * d + half * (KB / 2) : nullptr;
  const long long nw = (long long)gridDim.x * kWpb;
  const long long w = (long long)blockIdx.x * kWpb + wid;
  const int g0 = (int)(w * n_groups / nw), g1 = (int)((w + 1) * n_groups / nw);
  const int nkb = d / KB;
  float m_run = -INFINITY, s_run = 0.f;
  if (blockIdx.x == 0 && blockIdx.y == 0 && threadIdx.x == 0) flags[0] = 0;

  for (int g = g0; g < g1; ++g) {
    const int v0 = g * (32 * NT);
    const uint16_t* wp[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t)
      wp[t] = W + (size_t)min(v0 + 32 * t + n, V - 1) * d + half * (KB / 2);
    Acc<NT> acc;
#pragma unroll
    for (int t = 0; t < NT; ++t) acc.t[t] = f32x16{};

    FragK<KB> A[S][NT], BH[S], BL[S];
#pragma unroll
    for (int s = 0; s < S - 1; ++s) {
      const int off = min(s, nkb - 1) * KB;
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int t = 0; t < NT; ++t) A[s][t] = ldk<KB>(wp[t] + off);
      BH[s] = ldk<KB>(hp + off);
      if (HILO) BL[s] = ldk<KB>(lp + off);
    }
    for (int i = 0; i < nkb; i += S) {
#pragma unroll
      for (int s = 0; s < S; ++s) {
        const int ls = (s + S - 1) % S;
        const int off = min(i + s + S - 1, nkb - 1) * KB;
        // Keep each stage's loads ahead of its matrix ops and in source order, so every
        // path into the loop sees the same number of younger loads at each wait.
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int t = 0; t < NT; ++t) A[ls][t] = ldk<KB>(wp[t] + off);
        BH[ls] = ldk<KB>(hp + off);
        if (HILO) BL[ls] = ldk<KB>(lp + off);
        __builtin_amdgcn_sched_barrier(0);
        if (i + s < nkb) {
#pragma unroll
          for (int j = 0; j < KB / 16; ++j)
#pragma unroll
            for (int t = 0; t < NT; ++t) {
              acc.t[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                  as_bf16x8(A[s][t].v[j]), as_bf16x8(BH[s].v[j]), acc.t[t], 0, 0, 0);
              if (HILO)
                acc.t[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                    as_bf16x8(A[s][t].v[j]), as_bf16x8(BL[s].v[j]), acc.t[t], 0, 0, 0);
            }
        }
      }
    }
    epilogue_lse<NT>(acc, v0, V, half, m_run, s_run);
  }
  store_partial(m_run, s_run, n, half, wid, row0, n_rows, part, red);
}

// ------------------------------------------------------------------------------------
// Streaming kernel for d a multiple of 64 (the HBM-bound small-row case).
//
// Every global load is lane-contiguous: 16 lanes cover 256 contiguous bytes of one row and
// an instruction reads four rows, i.e. 8 whole cache lines per 1 KB.  (Loading operands
// directly in the matrix-core layout instead touches 32-64 lines per instruction, and the
// per-line cost then bounds the stream well below HBM bandwidth.)  The workgroup's waves
// advance through K in lockstep, 128 k per stage:
//   * each wave owns one 32-row tile of the head and moves each stage of it through its
//     own LDS tile into the MFMA A layout;
//   * the 32 x 128 stage of H (hi and lo planes) is loaded once per workgroup, each wave
//     fetching WPB-th of it, into a double-buffered LDS stage shared by all waves.
// LDS chunk (row r, 16-byte chunk c) of a 32x128 bf16 tile lives at r * 16 + (c ^ (r & 15)):
// sixteen consecutive rows at the same c fall into sixteen different 16-byte bank groups,
// so the row-wise writes and the column-wise fragment reads are both conflict-free.
// K permutation inside a stage: lane half h, MFMA step j covers k = kb + 64 h + 8 j + e,
// i.e. chunk 8 h + j of the row, for both operands.  When d % 128 = 64 the last stage holds
// 64 k: its chunks 8..15 re-read chunks 0..7 of the same head rows (in bounds, lines the
// stage already fetches) and meet zero H chunks, so they add nothing.  Register stages
// rotate S deep; loads run S-1 stages ahead and are never predicated (a stage past the end
// re-reads the last one), so the compiler waits exactly for the stage it consumes.
// ------------------------------------------------------------------------------------
// NT: head loads carry the non-temporal hint (the head streams through once, with no reuse
// the caches could serve: one row tile, or a head larger than the last-level cache).
// Measured on binary_enum (1.27 GB head, one row tile): 220 -> 207 us per launch, the plain
// read of the same bytes 6.34 -> 7.06 TB/s.
// Its first workgroup clears the flag word (no launch before it does).
// NR: 32-row tiles of H per workgroup (1, 2 or 4): each head fragment is multiplied into NR
// accumulator tiles, so the head is read once for 32 NR rows.  The H stage holds NR x 32
// rows (LDS: 64 KB of head tiles + 2 x NP x NR x 8 KB of H stages, twice that with PAIR;
// at most 128 KB).
// HALF: d % 128 = 64, the last stage 64 wide (a separate instance, so that the loads of the
// d % 128 = 0 instances stay as they were: the run-time test cost binary_enum 15%).
// PAIR (one row tile): the per-stage barrier only guards the shared H stage, so two H stages
// share a buffer and a barrier: stages 2p and 2p + 1 are written at stage 2p and 2p + 1 runs
// without a barrier.  A stage's H loads are then issued before its head loads, so writing
// H one stage early waits only for loads the current stage needs anyway.  Measured 1-4%
// faster (binary_enum 202.6 -> 199.4 us).
template <int WPB, int S, bool HF32, bool NT, int NR, bool HALF, bool PAIR>
__global__ __launch_bounds__(WPB * 64) void k_project_wg_bf16(
    const uint16_t* __restrict__ W, int V, int d, const void* __restrict__ Hsrc, int n_rows,
    int n_groups, int32_t* __restrict__ flags, float2* __restrict__ part) {
  constexpr int KC = 128;                 // k per stage
  constexpr int NP = HF32 ? 2 : 1;        // H planes in LDS (hi, lo)
  constexpr int HQ = (HF32 ? 16 : 8) * NR / WPB;  // H load instructions per wave per stage
  static_assert(HQ >= 1 && ((HF32 ? 16 : 8) * NR) % WPB == 0, "H stage split");
  static_assert(NP * NR * (PAIR ? 2 : 1) <= 4, "H stages within the LDS budget");
  constexpr int HP = NR * 512;            // 16-byte slots per H plane
  constexpr int HS = PAIR ? 2 : 1;        // H stages per buffer (and per barrier)
  __shared__ u32x4 wt[WPB][512];          // per-wave 32-row head tile
  __shared__ u32x4 hb[2][HS][NP][HP];     // H stages, double buffered
  __shared__ float2 red[NR][WPB][32];
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const int n = lane & 31, half = lane >> 5;
  const int lrow = lane >> 4, lch = lane & 15;
  const int rt = blockIdx.y, row0 = rt * 32 * NR;
  const int g0 = (int)((long long)blockIdx.x * n_groups / gridDim.x);
  const int g1 = (int)((long long)(blockIdx.x + 1) * n_groups / gridDim.x);
  const int nst = HALF ? (d + KC - 1) / KC : d / KC;  // with HALF the last stage holds 64 k
  u32x4* my = wt[wid];
  float m_run[NR], s_run[NR];
#pragma unroll
  for (int t = 0; t < NR; ++t) {
    m_run[t] = -INFINITY;
    s_run[t] = 0.f;
  }
  if (blockIdx.x == 0 && blockIdx.y == 0 && threadIdx.x == 0) flags[0] = 0;

  // H stage loads.  bf16 H: instruction hq reads stage rows 4 hq + lane / 16, 16-byte chunk
  // lane % 16.  fp32 H: instruction hq reads rows 2 hq + lane / 32, four values at
  // 4 (lane % 32), i.e. half of chunk (lane % 32) / 2; they are split into bf16 hi and lo
  // (hi = rne(x), lo = rne(x - hi)) on the way into LDS.
  int h_r[HQ];
  const char* h_src[HQ];
#pragma unroll
  for (int i = 0; i < HQ; ++i) {
    const int hq = wid * HQ + i;
    h_r[i] = HF32 ? 2 * hq + (lane >> 5) : 4 * hq + lrow;
    const int hrow = min(row0 + h_r[i], n_rows - 1);
    h_src[i] = HF32 ? (const char*)((const float*)Hsrc + (size_t)hrow * d + (lane & 31) * 4)
                    : (const char*)((const uint16_t*)Hsrc + (size_t)hrow * d + lch * 8);
  }
  const int h_chunk = HF32 ? ((lane & 31) >> 1) : lch;
  // lanes whose H values sit in chunks 8..15 of a stage (k 64..127 of it)
  const bool h_upper = HF32 ? (lane & 31) >= 16 : lch >= 8;

  for (int g = g0; g < g1; ++g) {
    const int v0 = g * (WPB * 32) + wid * 32;
    Acc<NR> acc;
#pragma unroll
    for (int t = 0; t < NR; ++t) acc.t[t] = f32x16{};
    u32x4 R[S][8], Hr[S][HQ];
    // H loads of a stage: after its head loads, or with PAIR before them (a stage's H is
    // written to LDS one stage early, so its wait must not cover that stage's head loads)
#define JET_STAGE_LOAD_H(SLOT, ST)                                                          \
  _Pragma("unroll") for (int i = 0; i < HQ; ++i) {                                          \
    const u32x4 hv_ = *reinterpret_cast<const u32x4*>(                                      \
        h_src[i] + ((size_t)(ST) * KC - (hz_ ? 64 : 0)) * (HF32 ? 4 : 2));                  \
    Hr[SLOT][i] = hz_ ? u32x4{0u, 0u, 0u, 0u} : hv_;                                        \
  }
#define JET_STAGE_LOAD(SLOT, ST)                                                            \
  {                                                                                         \
    const bool up_ = HALF && (ST) == nst - 1; /* a 64-wide last stage */                    \
    const int ko_ = (ST) * KC + (up_ ? (lch & 7) : lch) * 8;                                \
    const bool hz_ = up_ && h_upper;                                                        \
    if (PAIR) JET_STAGE_LOAD_H(SLOT, ST);                                                   \
    _Pragma("unroll") for (int q = 0; q < 8; ++q) {                                         \
      const u32x4* src_ = reinterpret_cast<const u32x4*>(                                   \
          W + (size_t)min(v0 + 4 * q + lrow, V - 1) * d + ko_);                             \
      R[SLOT][q] = NT ? __builtin_nontemporal_load(src_) : *src_;                           \
    }                                                                                       \
    if (!PAIR) JET_STAGE_LOAD_H(SLOT, ST);                                                  \
  }
    // H of the stage in register slot HSLOT, split into hi and lo for fp32 H, to the LDS
    // stage at DST
#define JET_STAGE_WRITE_H(HSLOT, DST)                                                       \
  _Pragma("unroll") for (int i = 0; i < HQ; ++i) {                                          \
    const int slot_ = h_r[i] * 16 + (h_chunk ^ (h_r[i] & 15));                               \
    if (HF32) {                                                                             \
      const u32x4 x = Hr[HSLOT][i];                                                         \
      uint32_t h01, l01, h23, l23;                                                          \
      split_pair(__uint_as_float(x[0]), __uint_as_float(x[1]), h01, l01);                   \
      split_pair(__uint_as_float(x[2]), __uint_as_float(x[3]), h23, l23);                   \
      uint2* dh = reinterpret_cast<uint2*>(&(DST)[slot_]) + (lane & 1);                     \
      uint2* dl = reinterpret_cast<uint2*>(&(DST)[HP + slot_]) + (lane & 1);                \
      *dh = make_uint2(h01, h23);                                                           \
      *dl = make_uint2(l01, l23);                                                           \
    } else {                                                                                \
      (DST)[slot_] = Hr[HSLOT][i];                                                          \
    }                                                                                       \
  }
#define JET_STAGE_MMA(SLOT, ST)                                                             \
  {                                                                                         \
    _Pragma("unroll") for (int q = 0; q < 8; ++q) {                                         \
      const int r = 4 * q + lrow;                                                           \
      my[r * 16 + (lch ^ (r & 15))] = R[SLOT][q];                                            \
    }                                                                                       \
    /* PAIR: stages 2p and 2p + 1 share buffer p & 1 and one barrier, both written at 2p */ \
    u32x4* hbuf = PAIR ? &hb[((ST) >> 1) & 1][(ST) & 1][0][0] : &hb[(ST) & 1][0][0][0];     \
    if (!PAIR || ((ST) & 1) == 0) { /* uniform over the workgroup */                        \
      JET_STAGE_WRITE_H(SLOT, hbuf);                                                        \
      if (PAIR) JET_STAGE_WRITE_H(((SLOT) + 1) % S, hbuf + NP * HP);                        \
      __syncthreads();                                                                      \
    }                                                                                       \
    _Pragma("unroll") for (int j = 0; j < 8; ++j) {                                         \
      const int c = ((half * 8 + j) ^ (n & 15)) + n * 16;                                    \
      const bf16x8 a = as_bf16x8v(my[c]);                                                   \
      _Pragma("unroll") for (int t = 0; t < NR; ++t) {                                       \
        acc.t[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, as_bf16x8v(hbuf[t * 512 + c]), acc.t[t], 0, 0, 0); \
        if (HF32)                                                                           \
          acc.t[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, as_bf16x8v(hbuf[HP + t * 512 + c]), acc.t[t], 0, 0, 0); \
      }                                                                                     \
    }                                                                                       \
  }
#pragma unroll
    for (int s = 0; s < S - 1; ++s) {
      __builtin_amdgcn_sched_barrier(0);
      JET_STAGE_LOAD(s, min(s, nst - 1));
    }
    // Main loop over a multiple of S stages: every prefetched slot is consumed, so no load
    // sits behind a condition (which would let it sink to its use).
    const int nmain = nst - nst % S;
    for (int st0 = 0; st0 < nmain; st0 += S) {
#pragma unroll
      for (int s = 0; s < S; ++s) {
        __builtin_amdgcn_sched_barrier(0);
        JET_STAGE_LOAD((s + S - 1) % S, min(st0 + s + S - 1, nst - 1));
        __builtin_amdgcn_sched_barrier(0);
        JET_STAGE_MMA(s, st0 + s);
      }
    }
    // The last nst % S (< S) stages are already in slots 0 .. nst % S - 1.
#pragma unroll
    for (int s = 0; s < S - 1; ++s)
      if (s < nst - nmain) JET_STAGE_MMA(s, nmain + s);  // uniform over the workgroup
#undef JET_STAGE_MMA
#undef JET_STAGE_WRITE_H
#undef JET_STAGE_LOAD
#undef JET_STAGE_LOAD_H
#pragma unroll
    for (int t = 0; t < NR; ++t) {
      Acc<1> one;
      one.t[0] = acc.t[t];
      epilogue_lse<1>(one, v0, V, half, m_run[t], s_run[t]);
    }
    // The H stage buffer is hb[stage & 1] (PAIR: hb[(stage / 2) & 1]) and the stage count
    // restarts with every group.  With an odd number of buffer uses the group's last and the
    // next group's first share buffer 0, so no wave may write the next group's first stage
    // before every wave has read the last: one barrier per group (uniform; an even count
    // alternates across the boundary and needs none).
    if ((PAIR ? (nst + 1) >> 1 : nst) & 1) __syncthreads();
  }
#pragma unroll
  for (int t = 0; t < NR; ++t)
    store_partial<WPB, true>(m_run[t], s_run[t], n, half, wid, row0 + 32 * t, n_rows, part, red[t]);
}

// ------------------------------------------------------------------------------------
// Streaming kernel for an fp32 head (fp32 H).  The loads of the bf16 streaming kernel: 16
// lanes read 256 contiguous bytes (64 k) of one row and an instruction reads four rows, so
// every head byte moves in whole cache lines; each wave owns a 32-row head tile per
// vocabulary group and moves each stage of it through its own LDS tile into the operand
// layout of the matrix op.  The 32 x 64 stage of H is loaded once per workgroup (four rows
// per wave) into a double-buffered stage shared by all waves.  LDS chunk (row r, 16-byte
// chunk c) sits at r * 16 + (c ^ (r & 15)), as in the bf16 kernel.  HALF: d % 64 = 32, the
// last stage holds 32 k; its chunks 8..15 re-read chunks 0..7 of the same head rows (in
// bounds) and meet zero H chunks.
// fp32 matrix ops run at a sixteenth of the bf16 rate: at a full 32-row tile the matrix work
// of a stage takes about as long as its head bytes take to arrive at HBM speed, so a tile
// of 16 rows serves up to 16 rows at half the matrix work.
// The workgroup walks its vocabulary groups as one flat stream of (group, stage) steps: loads
// run ahead across group boundaries (3-10% faster than restarting the pipeline per group at
// d <= 1024 and few rows, 3% slower with one group per workgroup and many row tiles).
//   RT = 32: v_mfma_f32_32x32x2f32, lane l supplies row l % 32 and one k of its half l / 32;
//            K is permuted inside a stage so that half h takes k = 32 h + s at step s.
//   RT = 16: v_mfma_f32_16x16x4f32 on two 16-entry vocabulary tiles, lane l supplies row
//            l % 16 and one k of its quarter q = l / 16, k = 16 q + s at step s; output
//            (m, n) of a 16 x 16 tile sits in lane n + 16 (m / 4), register m % 4.
// Both operands take the same permutation, and one 16-byte LDS read serves four steps.
template <int WPB, int S, bool NT, bool HALF, int RT>
__global__ __launch_bounds__(WPB * 64) void k_project_wg_f32(
    const float* __restrict__ W, int V, int d, const float* __restrict__ H, int n_rows,
    int n_groups, int32_t* __restrict__ flags, float2* __restrict__ part) {
  constexpr int KC = 64;  // k per stage
  static_assert(WPB == 8, "four H rows per wave per stage");
  static_assert(RT == 16 || RT == 32, "row tile");
  __shared__ u32x4 wt[WPB][512];  // per-wave 32-row head tile
  __shared__ u32x4 hb[2][512];    // H stage, double buffered
  __shared__ float2 red[WPB][32];
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const int n = lane & 31, half = lane >> 5;
  const int n16 = lane & 15, quarter = lane >> 4;
  const int lrow = lane >> 4, lch = lane & 15;
  const int row0 = blockIdx.y * RT;
  const int g0 = (int)((long long)blockIdx.x * n_groups / gridDim.x);
  const int g1 = (int)((long long)(blockIdx.x + 1) * n_groups / gridDim.x);
  const int nst = HALF ? (d + KC - 1) / KC : d / KC;
  u32x4* my = wt[wid];
  float m_run = -INFINITY, s_run = 0.f;
  if (blockIdx.x == 0 && blockIdx.y == 0 && threadIdx.x == 0) flags[0] = 0;
  // H stage rows 4 wid + lane / 16, chunk lane % 16 (rows past the last, and with RT = 16
  // stage rows 16..31, repeat a valid row: their products are not used)
  const int h_r = 4 * wid + lrow;
  const float* h_src = H + (size_t)min(row0 + h_r, n_rows - 1) * d + lch * 4;
  const bool h_upper = lch >= 8;  // k 32..63 of a stage
  const int h_slot = h_r * 16 + (lch ^ (h_r & 15));

  // One flat stream of (group, stage) steps over the workgroup's groups: loads run S - 1
  // steps ahead across group boundaries, and each group's epilogue follows its last stage
  // (a group of few stages would otherwise refill the pipeline every time).  Loads past the
  // last step re-read the last group's stages (in bounds) and are not used.
  const int total = (g1 - g0) * nst;
  f32x16 acc = {};
  f32x4 acc16[2] = {};
  u32x4 R[S][8], Hr[S];
  int lg = g0, lst = 0;  // next step to load
  int mg = g0, mst = 0;  // next step to multiply
#define JET_F32_LOAD(SLOT)                                                                  \
  {                                                                                         \
    const int lv0_ = min(lg, g1 - 1) * (WPB * 32) + wid * 32;                               \
    const bool up_ = HALF && lst == nst - 1; /* a 32-wide last stage */                     \
    const int ko_ = lst * KC + (up_ ? (lch & 7) : lch) * 4;                                 \
    _Pragma("unroll") for (int q = 0; q < 8; ++q) {                                         \
      const u32x4* src_ = reinterpret_cast<const u32x4*>(                                   \
          W + (size_t)min(lv0_ + 4 * q + lrow, V - 1) * d + ko_);                           \
      R[SLOT][q] = NT ? __builtin_nontemporal_load(src_) : *src_;                           \
    }                                                                                       \
    const bool hz_ = up_ && h_upper;                                                        \
    const u32x4 hv_ =                                                                       \
        *reinterpret_cast<const u32x4*>(h_src + (size_t)lst * KC - (hz_ ? 32 : 0));         \
    Hr[SLOT] = hz_ ? u32x4{0u, 0u, 0u, 0u} : hv_;                                           \
    if (++lst == nst) { lst = 0; ++lg; }                                                    \
  }
#define JET_F32_MMA(SLOT, F)                                                                \
  {                                                                                         \
    _Pragma("unroll") for (int q = 0; q < 8; ++q) {                                         \
      const int r = 4 * q + lrow;                                                           \
      my[r * 16 + (lch ^ (r & 15))] = R[SLOT][q];                                            \
    }                                                                                       \
    u32x4* hbuf = &hb[(F) & 1][0];                                                          \
    hbuf[h_slot] = Hr[SLOT];                                                                \
    __syncthreads();                                                                        \
    if constexpr (RT == 32) {                                                               \
      _Pragma("unroll") for (int j = 0; j < 8; ++j) {                                       \
        const int c = ((half * 8 + j) ^ (n & 15)) + n * 16;                                  \
        const u32x4 a4 = my[c], b4 = hbuf[c];                                               \
        _Pragma("unroll") for (int e = 0; e < 4; ++e)                                       \
          acc = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a4[e]),                \
                                                     __uint_as_float(b4[e]), acc, 0, 0, 0); \
      }                                                                                     \
    } else {                                                                                \
      _Pragma("unroll") for (int j = 0; j < 4; ++j) {                                       \
        const int c = ((quarter * 4 + j) ^ n16) + n16 * 16;                                  \
        const u32x4 a0 = my[c], a1 = my[c + 256], b4 = hbuf[c];                             \
        _Pragma("unroll") for (int e = 0; e < 4; ++e) {                                     \
          acc16[0] = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a0[e]),           \
                                                          __uint_as_float(b4[e]), acc16[0], \
                                                          0, 0, 0);                         \
          acc16[1] = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a1[e]),           \
                                                          __uint_as_float(b4[e]), acc16[1], \
                                                          0, 0, 0);                         \
        }                                                                                   \
      }                                                                                     \
    }                                                                                       \
    if (++mst == nst) { /* the group's last stage: fold its logits (uniform) */             \
      group_done(mg * (WPB * 32) + wid * 32);                                               \
      mst = 0;                                                                              \
      ++mg;                                                                                 \
    }                                                                                       \
  }
  auto group_done = [&](int v0) {
    if constexpr (RT == 32) {
      Acc<1> one;
      one.t[0] = acc;
      epilogue_lse<1>(one, v0, V, half, m_run, s_run);
      acc = f32x16{};
    } else {
      // register i of tile t: vocabulary entry v0 + 16 t + 4 quarter + i, row n16
      float gm = -INFINITY;
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (v0 + 16 * t + 4 * quarter + i < V) gm = fmaxf(gm, acc16[t][i]);
      const float mn = fmaxf(m_run, gm);
      if (mn != -INFINITY) {
        const float mb = mn * kLog2e;
        float sum = 0.f;
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            if (v0 + 16 * t + 4 * quarter + i < V) sum += exp2f(fmaf(acc16[t][i], kLog2e, -mb));
        s_run = s_run * exp2f((m_run - mn) * kLog2e) + sum;
        m_run = mn;
      }
      acc16[0] = f32x4{};
      acc16[1] = f32x4{};
    }
  };
#pragma unroll
  for (int s = 0; s < S - 1; ++s) {
    __builtin_amdgcn_sched_barrier(0);
    JET_F32_LOAD(s);
  }
  // main loop over a multiple of S steps, so that no load sits behind a condition; the H
  // stage buffer alternates with every step, so group boundaries need no barrier of their own
  const int nmain = total - total % S;
  for (int f0 = 0; f0 < nmain; f0 += S) {
#pragma unroll
    for (int s = 0; s < S; ++s) {
      __builtin_amdgcn_sched_barrier(0);
      JET_F32_LOAD((s + S - 1) % S);
      __builtin_amdgcn_sched_barrier(0);
      JET_F32_MMA(s, f0 + s);
    }
  }
  // the last total % S (< S) steps are already in slots 0 .. total % S - 1
#pragma unroll
  for (int s = 0; s < S - 1; ++s)
    if (s < total - nmain) JET_F32_MMA(s, nmain + s);  // uniform over the workgroup
#undef JET_F32_MMA
#undef JET_F32_LOAD
  if constexpr (RT == 32) {
    store_partial<WPB, true>(m_run, s_run, n, half, wid, row0, n_rows, part, red);
  } else {
    // lanes n16, n16 + 16, n16 + 32 and n16 + 48 hold row n16: merge them, then the waves
    // in wave order
#pragma unroll
    for (int x = 16; x <= 32; x *= 2) {
      const float m2 = __shfl_xor(m_run, x);
      const float s2 = __shfl_xor(s_run, x);
      lse_merge(m_run, s_run, m2, s2);
    }
    if (lane < 16) red[wid][lane] = make_float2(m_run, s_run);
    __syncthreads();
    if (threadIdx.x < 16) {
      float m = red[0][n16].x, s = red[0][n16].y;
#pragma unroll
      for (int w = 1; w < WPB; ++w) lse_merge(m, s, red[w][n16].x, red[w][n16].y);
      const int row = row0 + n16;
      if (row < n_rows) part[(size_t)row * gridDim.x + blockIdx.x] = make_float2(m, s);
    }
  }
}

// ------------------------------------------------------------------------------------
// fp32 head and fp32 hidden states: v_mfma_f32_32x32x2_f32 takes one k per lane half.
// A workgroup takes one 32-entry vocabulary group at a time and its four waves split the
// k range: wave w takes the 16-wide blocks w, w + 4, ...; in a block, lane half h loads 8
// consecutive k (two float4) of its row, k = kb + 8 h + 4 q + c for float4 q and component
// c, each component one MFMA step.  (One wave over the whole row would make a 32 x 32 tile
// a chain of d / 2 dependent matrix ops; split four ways the chain is a quarter as long and
// four times as many waves are in flight.)  The waves' tiles are added in wave order
// through LDS, and wave 0 runs the epilogue.
// ------------------------------------------------------------------------------------
template <bool STORE>
__global__ __launch_bounds__(256) void k_project_small_f32(
    const float* __restrict__ W, int V, int d, const float* __restrict__ H, int n_rows,
    int n_groups, int32_t* __restrict__ flags, float2* __restrict__ part, float* __restrict__ Z) {
  constexpr int KB = 16, S = 2;
  __shared__ float2 red[kWpb][32];
  __shared__ f32x16 tiles[kWpb - 1][kWave];
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const int n = lane & 31, half = lane >> 5;
  const int rt = blockIdx.y, row0 = rt * 32;
  const int hrow = min(row0 + n, n_rows - 1);
  const float* hp = H + (size_t)hrow * d + half * (KB / 2);
  const int g0 = (int)((long long)blockIdx.x * n_groups / gridDim.x);
  const int g1 = (int)((long long)(blockIdx.x + 1) * n_groups / gridDim.x);
  const int nkb = d / KB;  // >= 2 (d is a multiple of 32)
  // this wave's blocks wid, wid + kWpb, ...: nmy of them (none when nkb <= wid)
  const int nmy = nkb > wid ? (nkb - wid + kWpb - 1) / kWpb : 0;
  // k offset of the wave's block j; past its last block (or with no block) the load
  // re-reads a valid block and is not used
  auto koff = [&](int j) { return min(wid + kWpb * j, nkb - 1) * KB; };
  float m_run = -INFINITY, s_run = 0.f;
  if (!STORE && blockIdx.x == 0 && blockIdx.y == 0 && threadIdx.x == 0) flags[0] = 0;
  for (int g = g0; g < g1; ++g) {
    const int v0 = g * 32;
    const float* wp = W + (size_t)min(v0 + n, V - 1) * d + half * (KB / 2);
    f32x16 acc = {};
    float4 A[S][2], B[S][2];
#pragma unroll
    for (int s = 0; s < S - 1; ++s) {
      const int off = koff(s);
      A[s][0] = *reinterpret_cast<const float4*>(wp + off);
      A[s][1] = *reinterpret_cast<const float4*>(wp + off + 4);
      B[s][0] = *reinterpret_cast<const float4*>(hp + off);
      B[s][1] = *reinterpret_cast<const float4*>(hp + off + 4);
    }
    for (int i = 0; i < nmy; i += S) {  // nmy is uniform over the wave
#pragma unroll
      for (int s = 0; s < S; ++s) {
        const int ls = (s + S - 1) % S;
        const int off = koff(i + s + S - 1);
        A[ls][0] = *reinterpret_cast<const float4*>(wp + off);
        A[ls][1] = *reinterpret_cast<const float4*>(wp + off + 4);
        B[ls][0] = *reinterpret_cast<const float4*>(hp + off);
        B[ls][1] = *reinterpret_cast<const float4*>(hp + off + 4);
        if (i + s < nmy) {
#pragma unroll
          for (int q = 0; q < 2; ++q) {
            acc = __builtin_amdgcn_mfma_f32_32x32x2f32(A[s][q].x, B[s][q].x, acc, 0, 0, 0);
            acc = __builtin_amdgcn_mfma_f32_32x32x2f32(A[s][q].y, B[s][q].y, acc, 0, 0, 0);
            acc = __builtin_amdgcn_mfma_f32_32x32x2f32(A[s][q].z, B[s][q].z, acc, 0, 0, 0);
            acc = __builtin_amdgcn_mfma_f32_32x32x2f32(A[s][q].w, B[s][q].w, acc, 0, 0, 0);
          }
        }
      }
    }
    if (wid > 0) tiles[wid - 1][lane] = acc;
    __syncthreads();
    if (wid == 0) {
      Acc<1> sum;
      sum.t[0] = acc;
#pragma unroll
      for (int w = 0; w < kWpb - 1; ++w) sum.t[0] += tiles[w][lane];
      if (STORE)
        epilogue_store<1>(sum, v0, V, n, half, row0, n_rows, Z);
      else
        epilogue_lse<1>(sum, v0, V, half, m_run, s_run);
    }
    __syncthreads();  // tiles is rewritten for the next group
  }
  // waves 1.. hold (-inf, 0), which the wave-order merge leaves unchanged
  if (!STORE) store_partial(m_run, s_run, n, half, wid, row0, n_rows, part, red);
}

}  // namespace

// Shape of the small-row bf16 kernel: NT 32-row tiles per vocabulary group (a group is
// 32 * NT entries), KB-wide k blocks, S pipeline stages.
#ifndef JET_SMALL_NT
#define JET_SMALL_NT 2
#endif
#ifndef JET_SMALL_KB
#define JET_SMALL_KB 32
#endif
#ifndef JET_SMALL_S
#define JET_SMALL_S 3
#endif
#ifndef JET_STREAM_PAIR
#define JET_STREAM_PAIR 1  // one row tile per workgroup: two H stages per barrier
#endif
#ifndef JET_STREAM_WPB
#define JET_STREAM_WPB 8
#endif
#ifndef JET_STREAM_S
#define JET_STREAM_S 3  // register stages (3 measured 1-2% faster than 2 with non-temporal
                        // head loads; 4 spills)
#endif
constexpr int kStreamWPB = JET_STREAM_WPB;
// heads at least this large (the last-level cache is 256 MB) are loaded non-temporally even
// when several row tiles read them
constexpr size_t kStreamNtBytes = (size_t)256 << 20;
constexpr int kStreamS = JET_STREAM_S;
constexpr int kSmallNT = JET_SMALL_NT;
constexpr int kSmallKB = JET_SMALL_KB;
constexpr int kSmallS = JET_SMALL_S;

hipError_t launch_project(const ScoreArgs& a) {
  const jet_problem* p = a.p;
  const Plan& pl = *a.plan;
  if (pl.variant == VAR_TILED_BF16) return launch_project_tiled(a);
  float2* part = reinterpret_cast<float2*>(a.ws + pl.off_part);
  dim3 grid(pl.grid_x, pl.n_rtiles), block(256);
  if (pl.variant == VAR_SMALL_BF16 && stream_d(p->d)) {
    const uint16_t* W = static_cast<const uint16_t*>(p->W);
    dim3 sblock(kStreamWPB * 64);
    // non-temporal head loads unless several row tiles could find a small head in a cache
    const bool nt = pl.n_rtiles == 1 || (size_t)p->V * p->d * 2 >= kStreamNtBytes;
#define JET_WG(HF, NTV, NRV, HALFV)                                                          \
  hipLaunchKernelGGL((k_project_wg_bf16<kStreamWPB, (NRV == 1 ? kStreamS : 2), HF, NTV, NRV,    \
                                        HALFV, (NRV == 1 && JET_STREAM_PAIR)>),                 \
                     grid, sblock, 0,                                                           \
                     a.stream, W, p->V, p->d, p->H, p->n_rows, pl.n_vgroups, a.flags, part)
#define JET_WG_H(HF, NTV, NRV) \
  if (p->d % 128) JET_WG(HF, NTV, NRV, true); else JET_WG(HF, NTV, NRV, false)
#define JET_WG_NT(HF, NRV) \
  if (nt) { JET_WG_H(HF, true, NRV); } else { JET_WG_H(HF, false, NRV); }
    if (pl.hilo) {
      if (pl.stream_nr == 1) { JET_WG_NT(true, 1); }
      else if (pl.stream_nr == 2) { JET_WG_NT(true, 2); }
      else return hipErrorInvalidValue;
    } else {
      if (pl.stream_nr == 1) { JET_WG_NT(false, 1); }
      else if (pl.stream_nr == 2) { JET_WG_NT(false, 2); }
      else if (pl.stream_nr == 4) { JET_WG_NT(false, 4); }
      else return hipErrorInvalidValue;
    }
#undef JET_WG_NT
#undef JET_WG_H
#undef JET_WG
  } else if (pl.variant == VAR_SMALL_BF16) {
    const uint16_t* W = static_cast<const uint16_t*>(p->W);
    if (pl.hilo) {
      const uint16_t* hhi = reinterpret_cast<const uint16_t*>(a.ws + pl.off_hhi);
      const uint16_t* hlo = reinterpret_cast<const uint16_t*>(a.ws + pl.off_hlo);
      hipLaunchKernelGGL((k_project_small_bf16<kSmallNT, kSmallKB, kSmallS, true>), grid, block, 0, a.stream,
                         W, p->V, p->d, hhi, hlo, p->n_rows, pl.n_vgroups, a.flags, part);
    } else {
      const uint16_t* h = static_cast<const uint16_t*>(p->H);
      hipLaunchKernelGGL((k_project_small_bf16<kSmallNT, kSmallKB, kSmallS, false>), grid, block, 0,
                         a.stream, W, p->V, p->d, h, nullptr, p->n_rows, pl.n_vgroups, a.flags,
                         part);
    }
  } else if (pl.variant == VAR_SMALL_F32 && pl.stream) {
    const float* W = static_cast<const float*>(p->W);
    const float* H = static_cast<const float*>(p->H);
    dim3 sblock(kStreamWPB * 64);
    const bool nt = pl.n_rtiles == 1 || (size_t)p->V * p->d * 4 >= kStreamNtBytes;
#define JET_WF(NTV, HALFV, RTV)                                                                \
  hipLaunchKernelGGL((k_project_wg_f32<kStreamWPB, kStreamS, NTV, HALFV, RTV>), grid, sblock,   \
                     0, a.stream, W, p->V, p->d, H, p->n_rows, pl.n_vgroups, a.flags, part)
#define JET_WF_H(NTV, RTV) \
  if (p->d % 64) JET_WF(NTV, true, RTV); else JET_WF(NTV, false, RTV)
#define JET_WF_NT(RTV) \
  if (nt) { JET_WF_H(true, RTV); } else { JET_WF_H(false, RTV); }
    if (pl.row_tile == 16) { JET_WF_NT(16); }
    else { JET_WF_NT(32); }
#undef JET_WF_NT
#undef JET_WF_H
#undef JET_WF
  } else if (pl.variant == VAR_SMALL_F32) {
    hipLaunchKernelGGL((k_project_small_f32<false>), grid, block, 0, a.stream,
                       static_cast<const float*>(p->W), p->V, p->d,
                       static_cast<const float*>(p->H), p->n_rows, pl.n_vgroups, a.flags, part,
                       nullptr);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

// The streaming kernel takes d in 128-wide stages, the last one 64 wide when d % 128 = 64.
bool stream_d(int d) { return d % 64 == 0; }

// Vocabulary entries per group and workgroups of the small-row path.
int small_group_size(int variant, bool stream) {
  if (stream) return 32 * kStreamWPB;
  return variant == VAR_SMALL_F32 ? 32 : 32 * kSmallNT;
}

int small_grid(int variant, bool stream, int n_groups, int max_waves) {
  if (stream) {
    int wg = max_waves / kStreamWPB;
    return n_groups < wg ? n_groups : wg;
  }
  if (variant == VAR_SMALL_F32) {  // one group at a time per workgroup
    const int cap = max_waves / kWpb;
    return n_groups < 1 ? 1 : (n_groups > cap ? cap : n_groups);
  }
  int gx = (n_groups + kWpb - 1) / kWpb;
  const int cap = max_waves / kWpb;
  return gx < 1 ? 1 : (gx > cap ? cap : gx);
}


hipError_t launch_project_store_f32(const float* Wu, int U, int d, const float* H, int n_rows,
                                    float* Z, hipStream_t stream) {
  const int n_groups = (U + 31) / 32;
  // one group at a time per workgroup, at most two workgroups per CU
  const int gx = n_groups < 1 ? 1 : (n_groups < 512 ? n_groups : 512);
  dim3 grid(gx, (n_rows + 31) / 32), block(256);
  hipLaunchKernelGGL((k_project_small_f32<true>), grid, block, 0, stream, Wu, U, d, H, n_rows,
                     n_groups, nullptr, nullptr, Z);
  return hipGetLastError();
}

}  // namespace jet
