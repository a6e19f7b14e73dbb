// Large-row fused projection + online full-vocabulary logsumexp + target capture
// (matrix-core bound when rows >> 300: 2 * rows flop per head byte).
//
// Computes the same quantities as the small-row kernels (JET paper, Eq. 1-2; FastJEV
// Sec. 3.3): z[r, v] = <H[r], W[v]> with fp32 accumulation, folded into a running
// (max, sum of exp) per row, plus the logit of every scored (row, target) pair.
//
// Tiling (gfx950): a workgroup of 4 waves owns a 256-row tile of H and sweeps a contiguous
// range of 256-entry vocabulary tiles.  Each wave computes a 128 x 128 quadrant (vocabulary
// x rows) as 4 x 4 tiles of v_mfma_f32_32x32x16_bf16, i.e. 256 fp32 accumulators per lane
// (all AGPRs; one wave per SIMD).
//
// Pipeline: K advances in 32-wide stages; the stages of all the split's vocabulary tiles
// form one stream, so the next tile's first stages are in flight during an epilogue.
//  * global -> registers: lane-contiguous 16-byte buffer loads (4 lanes cover one 64-byte
//    row segment), issued three stages ahead into two register sets;
//  * registers -> LDS: a ring of three buffers; stage g + 2 is written while stage g
//    computes, so the buffer of stage g + 1 was completed before the previous barrier and
//    its first fragments are read before this stage's barrier (no read-after-barrier
//    bubble); one barrier per stage;
//  * every MFMA is followed by one memory instruction (fragment read, LDS write or global
//    load), so with one wave per SIMD the memory traffic overlaps the matrix core instead
//    of stalling its issue in bursts.
// The last vocabulary tile (and row tile) is shifted back to end exactly at V (n_rows), so
// every load is in bounds; the overlap is masked in the epilogue and only the tile's own
// rows are reported.  LDS chunk (row r, 16-byte chunk c) lives at r * CH + (c ^ f(r)),
// which keeps the row-wise writes and the 32-row fragment reads conflict-free.
//
// Workgroup placement: workgroup L runs on XCD L % 8, and each XCD runs about 32 at a time
// (one per CU).  Launch index L is remapped so that those 32 form an SR x SS block of
// (row tile, vocabulary split) pairs: the SR row tiles' H tiles are shared SS ways and the
// SS splits' head tiles SR ways inside that XCD's L2.  Fragment k layout: lane half h,
// sub-step kk reads chunk 2 kk + h of its row for both operands (any k permutation shared
// by A and B gives the same dot product).
//
// H in one bf16 plane (bf16 hidden states) or two (fp32 hidden states split into hi + lo,
// each product accumulated twice).
#include "jet_internal.h"

#ifndef JET_TILED_NSET2
#define JET_TILED_NSET2 2
#endif

namespace jet {
namespace {

constexpr int TBM = 256;  // vocabulary entries per block tile
constexpr int TBN = 256;  // rows per block tile

__device__ inline int tm_of(int i, int h) { return 8 * (i >> 2) + 4 * h + (i & 3); }

// XOR swizzle of 16-byte chunks, a function of row & 15 only: 16 consecutive rows read at
// one chunk land in 16 different 16-byte bank groups, every aligned 8 rows in 8 different
// ones, and 32-row tiles 32 * CH apart share one swizzle (so their addresses differ by an
// immediate offset).
template <int CH>
__device__ inline int swz(int r) {
  return CH == 8 ? ((r ^ ((r >> 3) & 1)) & 7) : (((r >> 1) ^ (r >> 2)) & 3);
}

__device__ inline __amdgpu_buffer_rsrc_t rsrc_of(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

__device__ inline u32x4 bload(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)voff, (int)soff, 0));
}

// One BK = 32 stage of the block tile: LA head chunks and NP * LB hidden-state chunks per
// thread (16 bytes each), 16 KB per operand plane.
constexpr int BK = 32;
constexpr int CH = BK / 8;        // 16-byte chunks per row per stage
constexpr int KK = BK / 16;       // MFMA k sub-steps per stage
constexpr int RPI = 256 / CH;     // tile rows covered by one load round of 256 threads
constexpr int LA = TBM / RPI;     // head loads per thread per stage
constexpr int LB = TBN / RPI;     // hidden-state loads per plane per thread per stage
constexpr int NBUF = 3;           // LDS ring depth
constexpr int ASZ = TBM * CH;     // 16-byte slots per operand plane per buffer

template <int NP, int NSET>
__global__ __launch_bounds__(256, 1) void k_project_tiled_bf16(
    const uint16_t* __restrict__ W, int V, int d, const uint16_t* __restrict__ H0,
    const uint16_t* __restrict__ H1, int n_rows, int n_vtiles, const int* __restrict__ b_off,
    const int* __restrict__ b_tok, const int* __restrict__ tok_row,
    const int* __restrict__ tok_target, float* __restrict__ z_tgt, float2* __restrict__ part,
    int n_rtiles, int splits, int sr, int ss, int remap) {
  static_assert(KK == 2 && (NSET == 1 || NSET == 2), "stage layout");
  constexpr int BUFSZ = ASZ * (1 + NP);
  constexpr int NST = LA + NP * LB;  // LDS stores per thread per stage
  __shared__ u32x4 lds[NBUF * BUFSZ];
  __shared__ float2 red[2][TBN];

  const int tid = threadIdx.x, wid = tid >> 6, lane = tid & 63;
  const int wm = wid & 1, wn = wid >> 1;
  const int n = lane & 31, h = lane >> 5;
  int P = blockIdx.x;
  if (remap) {  // total is a multiple of 256: 8 XCDs x 32 concurrent workgroups
    const int xcd = blockIdx.x & 7, slot = blockIdx.x >> 3;
    P = (((slot >> 5) << 3) + xcd) * 32 + (slot & 31);
  }
  const int j = P / (sr * ss), w = P % (sr * ss);
  const int jr = j / (splits / ss), js = j % (splits / ss);
  const int rt = jr * sr + w / ss, split = js * ss + w % ss;
  const int row_nom = rt * TBN;                    // first row this tile reports
  const int row0 = min(row_nom, n_rows - TBN);     // rows loaded: [row0, row0 + 256), all valid
  const int t0 = (int)((long long)split * n_vtiles / splits);
  const int t1 = (int)((long long)(split + 1) * n_vtiles / splits);
  const int nk = d / BK;                           // even
  const uint32_t rowb = (uint32_t)d * 2;           // bytes per row (head and H planes)

  // load-side mapping: thread tid loads chunk tid % CH of tile rows tid / CH + i * RPI
  const int lr0 = tid / CH, lc = tid % CH;
  const uint32_t lvoff = (uint32_t)lr0 * rowb + lc * 16;
  const __amdgpu_buffer_rsrc_t rH0 = rsrc_of(H0, (uint32_t)n_rows * rowb);
  const __amdgpu_buffer_rsrc_t rH1 = rsrc_of(NP == 2 ? H1 : H0, (uint32_t)n_rows * rowb);
  const __amdgpu_buffer_rsrc_t rW = rsrc_of(W, (uint32_t)min((long long)V * rowb, 0xffffffffll));
  const uint32_t hrow = (uint32_t)row0 * rowb;
  // LDS write slot: rows lr0 + i * RPI share row & 15, hence one swizzle
  const int wslot = lr0 * CH + (lc ^ swz<CH>(lr0));
  // fragment read slots of sub-step kk: row (wm|wn)*128 + t*32 + n, chunk 2 kk + h
  int ra_slot[KK], rb_slot[KK];
#pragma unroll
  for (int kk = 0; kk < KK; ++kk) {
    ra_slot[kk] = (wm * 128 + n) * CH + ((2 * kk + h) ^ swz<CH>(n));
    rb_slot[kk] = ASZ + (wn * 128 + n) * CH + ((2 * kk + h) ^ swz<CH>(n));
  }

  float m_run[4], s_run[4];
#pragma unroll
  for (int nt = 0; nt < 4; ++nt) {
    m_run[nt] = -INFINITY;
    s_run[nt] = 0.f;
  }

  // The stages of all vocabulary tiles of this split form one stream g = 0 .. G - 1
  // (tile t0 + g / nk, k block g % nk).  Stage g + 1 + NSET is loaded at the top of stage
  // g; stage g + 2 is written to buffer (g + 2) % 3 while stage g computes.  Buffer
  // (g + 1) % 3 was completed before the previous barrier, so the first fragments of stage
  // g + 1 are read before this stage's barrier.  Past the end the cursor repeats the last
  // stage (in bounds; never consumed).
  const int G = (t1 - t0) * nk;
  int lt = t0, lk = 0, lg = 0;  // load cursor: tile, k block, stream index
  u32x4 ra[NSET][LA], rb[NSET][NP][LB];
  uint32_t l_ws = 0, l_hs = 0;  // byte offsets of the stage being loaded
#define JET_CURSOR()                                                                         \
  {                                                                                          \
    const uint32_t ko = (uint32_t)lk * (BK * 2);                                             \
    l_ws = __builtin_amdgcn_readfirstlane((uint32_t)min(lt * TBM, V - TBM) * rowb + ko);     \
    l_hs = __builtin_amdgcn_readfirstlane(hrow + ko);                                        \
    if (lg + 1 < G) {                                                                        \
      ++lg;                                                                                  \
      if (++lk == nk) {                                                                      \
        lk = 0;                                                                              \
        ++lt;                                                                                \
      }                                                                                      \
    }                                                                                        \
  }
  // loads u in [U0, U1) of the stage at the cursor into register set SET
#define JET_LOADU(SET, U0, U1)                                                               \
  {                                                                                          \
    _Pragma("unroll") for (int u = (U0); u < (U1); ++u) {                                    \
      if (u < LA) ra[SET][u] = bload(rW, lvoff, l_ws + u * RPI * rowb);                      \
      else                                                                                   \
        rb[SET][(u - LA) / LB][(u - LA) % LB] =                                              \
            bload((u - LA) / LB ? rH1 : rH0, lvoff, l_hs + ((u - LA) % LB) * RPI * rowb);    \
    }                                                                                        \
  }
#define JET_LOAD(SET)                                                                        \
  {                                                                                          \
    JET_CURSOR();                                                                            \
    JET_LOADU(SET, 0, NST);                                                                  \
  }
  // stores u in [U0, U1) of register set SET into the buffer at slot offset BOFF
#define JET_STORE(SET, BOFF, U0, U1)                                                         \
  {                                                                                          \
    _Pragma("unroll") for (int u = (U0); u < (U1); ++u) {                                    \
      if (u < LA) lds[(BOFF) + wslot + u * RPI * CH] = ra[SET][u];                           \
      else                                                                                   \
        lds[(BOFF) + ASZ * (1 + (u - LA) / LB) + wslot + ((u - LA) % LB) * RPI * CH] =        \
            rb[SET][(u - LA) / LB][(u - LA) % LB];                                           \
    }                                                                                        \
  }
  bf16x8 fa[KK][4], fb[KK][NP][4];
#define JET_FRAGS(F, BOFF, KK_)                                                              \
  {                                                                                          \
    _Pragma("unroll") for (int t = 0; t < 4; ++t)                                            \
      fa[F][t] = __builtin_bit_cast(bf16x8, lds[(BOFF) + ra_slot[KK_] + t * 32 * CH]);       \
    _Pragma("unroll") for (int p = 0; p < NP; ++p)                                           \
      _Pragma("unroll") for (int t = 0; t < 4; ++t)                                          \
        fb[F][p][t] = __builtin_bit_cast(bf16x8,                                             \
                                         lds[(BOFF) + p * ASZ + rb_slot[KK_] + t * 32 * CH]); \
  }
  // One MFMA sub-step with its memory slots, in issue order: MFMA i (vocabulary tile
  // i / (4 NP), row tile (i / NP) % 4, plane i % NP) is followed by memory slot i.  Slots
  // 0 .. NL - 1 hold the fragment reads of the next sub-step (read set RF, buffer RBOFF,
  // k sub-step RKK) with the NW LDS writes [W0, W0 + NW) of register set SSET spread evenly
  // among them; the next NLD slots issue loads [L0, L0 + NLD) into register set LSET.
  // Reads are ordered by first use: a0, all b, a1, a2, a3.
#define JET_SUBSTEP(F, RF, RBOFF, RKK, SSET, W0, NW, LSET, L0, NLD)                           \
  {                                                                                          \
    _Pragma("unroll") for (int i = 0; i < 16 * NP; ++i) {                                    \
      acc[i / (4 * NP)][(i / NP) % 4] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(              \
          fa[F][i / (4 * NP)], fb[F][i % NP][(i / NP) % 4], acc[i / (4 * NP)][(i / NP) % 4],  \
          0, 0, 0);                                                                          \
      constexpr int NL_ = NRD + (NW);                                                        \
      if (i < NL_) {                                                                         \
        const int nwb = (i * (NW)) / NL_;                                                    \
        if (((i + 1) * (NW)) / NL_ > nwb) {                                                  \
          JET_STORE(SSET, b_st, (W0) + nwb, (W0) + nwb + 1);                                 \
        } else {                                                                             \
          const int jr = i - nwb;                                                            \
          if (jr == 0) {                                                                     \
            fa[RF][0] = __builtin_bit_cast(bf16x8, lds[(RBOFF) + ra_slot[RKK]]);             \
          } else if (jr <= 4 * NP) {                                                         \
            const int pb = (jr - 1) % NP, tb = (jr - 1) / NP;                                \
            fb[RF][pb][tb] = __builtin_bit_cast(                                             \
                bf16x8, lds[(RBOFF) + pb * ASZ + rb_slot[RKK] + tb * 32 * CH]);              \
          } else {                                                                           \
            const int ta = jr - 4 * NP;                                                      \
            fa[RF][ta] = __builtin_bit_cast(bf16x8, lds[(RBOFF) + ra_slot[RKK] + ta * 32 * CH]); \
          }                                                                                  \
        }                                                                                    \
      } else if (i - NL_ < (NLD)) {                                                          \
        JET_LOADU(LSET, (L0) + i - NL_, (L0) + i - NL_ + 1);                                 \
      }                                                                                      \
      __builtin_amdgcn_sched_barrier(0);                                                     \
    }                                                                                        \
  }
  // One stage.  SLOAD receives stage g + 1 + NSET (half its loads per sub-step), SSTORE
  // (stage g + 2) is written to buffer (g + 2) % 3, half per sub-step with two sets, all in
  // the second with one.  Sub-step 0 also reads the fragments of k sub-step 1; sub-step 1
  // reads those of the next stage's sub-step 0.
  constexpr int NRD = 4 + 4 * NP;                  // fragment reads per sub-step
  constexpr int NW0 = NSET == 2 ? NST / 2 : 0;     // stores in sub-step 0
  static_assert(NRD + NW0 + NST / 2 <= 16 * NP &&
                    NRD + (NST - NW0) + (NST - NST / 2) <= 16 * NP,
                "every memory slot needs an MFMA");
#define JET_STAGE(SLOAD, SSTORE)                                                             \
  {                                                                                          \
    __builtin_amdgcn_sched_barrier(0);                                                       \
    JET_CURSOR();                                                                            \
    __builtin_amdgcn_sched_barrier(0);                                                       \
    JET_SUBSTEP(0, 1, b_cur, 1, SSTORE, 0, NW0, SLOAD, 0, NST / 2);                          \
    JET_SUBSTEP(1, 0, b_nxt, 0, SSTORE, NW0, NST - NW0, SLOAD, NST / 2, NST - NST / 2);      \
    __syncthreads();                                                                         \
    {                                                                                        \
      const int b_old = b_cur;                                                               \
      b_cur = b_nxt;                                                                         \
      b_nxt = b_st;                                                                          \
      b_st = b_old;                                                                          \
    }                                                                                        \
  }

  // prologue: stages 0 and 1 into buffers 0 and 1, stage 2 (two sets) in flight
  JET_LOAD(0);
  JET_STORE(0, 0, 0, NST);
  JET_LOAD(NSET - 1);
  JET_STORE(NSET - 1, BUFSZ, 0, NST);
  if (NSET == 2) JET_LOAD(0);
  __syncthreads();
  int b_cur = 0, b_nxt = BUFSZ, b_st = 2 * BUFSZ;  // slot offsets of buffers g, g+1, g+2 (mod 3)
  JET_FRAGS(0, b_cur, 0);

  for (int vt = t0; vt < t1; ++vt) {
    f32x16 acc[4][4];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) acc[mt][nt] = f32x16{};
    for (int kb = 0; kb < nk; kb += 2) {
      JET_STAGE(NSET - 1, 0);  // even stage: loads into the second set, stores the first
      JET_STAGE(0, NSET - 1);  // odd stage: loads into the first set, stores the second
    }

    // tile vt done: online logsumexp over its entries (the shifted last tile skips the ones
    // before v_nom, which the previous tile counted)
    const int v_nom = vt * TBM;
    const int v0 = min(v_nom, V - TBM);
    if (v0 == v_nom) {
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) {
        float gm = m_run[nt];
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
#pragma unroll
          for (int i = 0; i < 16; ++i) gm = fmaxf(gm, acc[mt][nt][i]);
        const float mb = gm * kLog2e;  // gm is finite: the tile holds 256 finite logits
        float sum = 0.f;
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
#pragma unroll
          for (int i = 0; i < 16; ++i) sum += exp2_hw(fmaf(acc[mt][nt][i], kLog2e, -mb));
        s_run[nt] = s_run[nt] * exp2f(m_run[nt] * kLog2e - mb) + sum;
        m_run[nt] = gm;
      }
    } else {
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) {
        float gm = -INFINITY;
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
#pragma unroll
          for (int i = 0; i < 16; ++i)
            if (v0 + wm * 128 + mt * 32 + tm_of(i, h) >= v_nom) gm = fmaxf(gm, acc[mt][nt][i]);
        const float mn = fmaxf(m_run[nt], gm);
        if (mn != -INFINITY) {
          const float mb = mn * kLog2e;
          float sum = 0.f;
#pragma unroll
          for (int mt = 0; mt < 4; ++mt)
#pragma unroll
            for (int i = 0; i < 16; ++i)
              if (v0 + wm * 128 + mt * 32 + tm_of(i, h) >= v_nom)
                sum += exp2_hw(fmaf(acc[mt][nt][i], kLog2e, -mb));
          s_run[nt] = s_run[nt] * exp2f((m_run[nt] - mn) * kLog2e) + sum;
          m_run[nt] = mn;
        }
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
#undef JET_LOAD
#undef JET_LOADU
#undef JET_CURSOR
#undef JET_STORE
#undef JET_FRAGS
#undef JET_STAGE
#undef JET_SUBSTEP

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
    const int row = row0 + r;
    if (row >= row_nom) part[(size_t)split * n_rows + row] = make_float2(m, s);
  }
}

}  // namespace

int tiled_bk(bool) { return 2 * BK; }  // nk = d / BK must be even

hipError_t launch_project_tiled(const ScoreArgs& a) {
  const jet_problem* p = a.p;
  const Plan& pl = *a.plan;
  const int* b_off = reinterpret_cast<const int*>(a.ws + pl.off_boff);
  const int* b_tok = reinterpret_cast<const int*>(a.ws + pl.off_btok);
  float* z_tgt = reinterpret_cast<float*>(a.ws + pl.off_ztgt);
  float2* part = reinterpret_cast<float2*>(a.ws + pl.off_part);
  // super-tile shape for the XCD-aware placement
  int sr = 1, ss = 1;
  const int S = pl.grid_x, R = pl.n_rtiles;
  const int total = S * R;
  int remap = 0;
  if (total % 256 == 0) {
    const int cand[3][2] = {{4, 8}, {2, 16}, {1, 32}};
    for (int i = 0; i < 3; ++i)
      if (R % cand[i][0] == 0 && S % cand[i][1] == 0) {
        sr = cand[i][0];
        ss = cand[i][1];
        remap = 1;
        break;
      }
  }
  if (!remap) {  // plain order: P = row tile * S + split
    sr = 1;
    ss = S;
  }
  dim3 grid(total), block(256);
  const uint16_t* W = static_cast<const uint16_t*>(p->W);
  if (pl.hilo) {
    const uint16_t* hhi = reinterpret_cast<const uint16_t*>(a.ws + pl.off_hhi);
    const uint16_t* hlo = reinterpret_cast<const uint16_t*>(a.ws + pl.off_hlo);
    hipLaunchKernelGGL((k_project_tiled_bf16<2, JET_TILED_NSET2>), grid, block, 0, a.stream, W, p->V, p->d, hhi,
                       hlo, p->n_rows, pl.n_vgroups, b_off, b_tok, p->tok_row, p->tok_target,
                       z_tgt, part, R, S, sr, ss, remap);
  } else {
    hipLaunchKernelGGL((k_project_tiled_bf16<1, 2>), grid, block, 0, a.stream, W, p->V, p->d,
                       static_cast<const uint16_t*>(p->H), nullptr, p->n_rows, pl.n_vgroups,
                       b_off, b_tok, p->tok_row, p->tok_target, z_tgt, part, R, S, sr, ss, remap);
  }
  return hipGetLastError();
}

}  // namespace jet
