// Large-row fused projection + online full-vocabulary logsumexp (matrix-core bound when
// rows >> 300: 2 * rows flop per head byte).
//
// Computes the same quantities as the small-row kernels (JET paper, Eq. 1-2; FastJEV
// Sec. 3.3): z[r, v] = <H[r], W[v]> with fp32 accumulation, folded into a running
// (max, sum of exp) per row; the scored (row, target) logits are computed after it, one
// dot product per token (k_token_logp).
//
// Tiling (gfx950): a workgroup of 4 waves (one per SIMD) owns a 256-row tile of H and
// sweeps a contiguous range of 256-entry vocabulary tiles; each wave computes a 128 x 128
// quadrant (vocabulary x rows), 256 fp32 accumulators per lane (all AGPRs).  The stages of
// all the range's vocabulary tiles form one stream, so the next tile's first stages are in
// flight during an epilogue.  Two kernels, d any multiple of 64 (64-wide stages, odd
// counts included):
//  * k_project_tiled_m16 (bf16 H): 8 x 8 blocks of v_mfma_f32_16x16x32_bf16 per wave;
//    stages loaded by the buffer unit straight into two LDS buffers; one barrier per
//    stage, at its midpoint (see the kernel);
//  * k_project_tiled_m16x2 (fp32 H as two bf16 planes, hi + lo): the same kernel with the
//    hi and lo rows of 128 rows as its 256 B-operand rows, both products of a row
//    accumulated into one accumulator.
// Every MFMA is followed by at most one memory instruction (fragment read or load), so with
// one wave per SIMD the memory traffic overlaps the matrix core instead of stalling its
// issue in bursts.  The last vocabulary tile (and row tile) is shifted back to end exactly
// at V (n_rows), so every load is in bounds; the overlap is masked in the epilogue and only
// the tile's own rows are reported.  LDS chunk (row r, 16-byte chunk c) lives at
// r * 8 + (c ^ swz16(r)), which keeps the fragment reads free of bank conflicts.
//
// Workgroup placement: workgroup L runs on XCD L % 8, and each XCD runs about 32 at a time
// (one per CU).  Launch index L is remapped so that those 32 form an SR x SS block of
// (row tile, vocabulary split) pairs: the SR row tiles' H tiles are shared SS ways and the
// SS splits' head tiles SR ways inside that XCD's L2.
#include "jet_internal.h"

namespace jet {
namespace {

constexpr int TBM = 256;  // vocabulary entries per block tile
constexpr int TBN = 256;  // rows per block tile

__device__ inline __amdgpu_buffer_rsrc_t rsrc_of(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

// Load 16 bytes per lane straight into LDS: lane l's bytes land at LDS byte address
// m0 + 16 l.  Issued as inline assembly so that the compiler's own LDS reads are not made
// to wait for every load in flight; completion is awaited explicitly (vm_wait) before
// the barrier that publishes the buffer.
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff,
                                      uint32_t m0) {
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds"
               :
               : "s"(m0), "v"(voff), "s"(r), "s"(soff)
               : "memory", "m0");
}
template <int N>
__device__ __forceinline__ void vm_wait() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// Workgroup -> (row tile, vocabulary split).  Launch index L runs on XCD L % 8, and each XCD
// runs about 32 workgroups at a time; with remap (launch size a multiple of 256) those 32
// form an sr x ss block of (row tile, split) pairs sharing tiles in that XCD's L2.  Blocks
// are numbered row group first: the eight XCDs, which start blocks together, work on the
// same vocabulary splits for different row groups, so a head tile fetched from HBM by one
// XCD is found by the others in the last-level cache.  Blocks past the last real one decode
// to row tiles >= n_rtiles or splits >= splits (padding).
__device__ __forceinline__ void tile_assign(int n_rtiles, int sr, int ss, int splits, int remap,
                                            int& rt, int& split) {
  int P = blockIdx.x;
  if (remap) {
    const int xcd = blockIdx.x & 7, slot = blockIdx.x >> 3;
    P = (((slot >> 5) << 3) + xcd) * 32 + (slot & 31);
  }
  const int j = P / (sr * ss), w = P % (sr * ss);
  const int n_rg = (n_rtiles + sr - 1) / sr;  // row groups; the last may hold padding
  const int jr = j % n_rg, js = j / n_rg;
  rt = jr * sr + w / ss;
  split = js * ss + w % ss;
}

// ------------------------------------------------------------------------------------
// bf16 hidden states on v_mfma_f32_16x16x32_bf16.  A stage is 64 columns of K for the
// 256-row head tile and the 256-row hidden-state tile (8 chunks of 16 bytes per row), two
// 64 KB buffers.  Every load instruction is issued by the buffer unit straight into LDS
// (1 KB: 8 rows x 8 chunks; lane l fetches the chunk that the swizzled layout puts in slot
// l).  Each wave's 128 x 128 quadrant is 8 x 8 blocks of 16 x 16 (4 accumulators per lane
// each).  On this matrix-core shape the chip sustains a higher clock under its power limit
// than with 32 x 32 blocks, which more than pays for the extra instructions.  Operand
// layout: lane l supplies row (A) or column (B) l % 16 and k = 8 (l / 16) + j, so a stage's
// k-step ks (32 wide) reads chunk 4 ks + l / 16 (swizzled by swz16).  Output register i of
// lane l holds vocabulary entry 4 (l / 16) + i and row l % 16 of its block.
// ------------------------------------------------------------------------------------
typedef __attribute__((ext_vector_type(4))) float f32x4;

// Chunk swizzle of the 16 x 16 kernel, a function of row & 15: logical chunk c of row r
// sits in slot c ^ swz16(r).  A quarter-wave reads 16 consecutive rows at one chunk, and
// lanes l and l + 32 are served together (the same 8 rows at chunks c and c + 2, c with
// bit 1 clear).  Both are conflict-free when the rows of one parity get distinct values
// and no two rows of one parity within an aligned group of 8 differ by 2 (XOR): value
// 4 b2 + 2 b3 + b1 of the row's bits.  A plain XOR with row & 7 doubled the LDS time of the
// fragment reads.
__device__ inline int swz16(int r) {
  return (((r >> 2) & 1) << 2) | (((r >> 3) & 1) << 1) | ((r >> 1) & 1);
}

// Clear the accumulators of block column nt once the epilogue has folded them.  The zeros
// are written to the accumulator registers and then made opaque to the compiler, so every
// stage of a tile, the first included, runs one loop body that accumulates in place.
// Seeding the first stage of each tile with an inline-constant zero instead (a peeled
// first stage) made the register allocator permute all 256 accumulators through vector
// registers in the stage after it, every tile: 344 register moves and stalled matrix ops
// that waited on their predecessors, 0.6% of the large-row kernel's time.
template <bool TWO>
__device__ __forceinline__ void zero_column(f32x4 (&acc)[8][TWO ? 4 : 8], int nt) {
#pragma unroll
  for (int mt = 0; mt < 8; ++mt) {
    acc[mt][nt] = f32x4{};
    asm volatile("" : "+a"(acc[mt][nt]));
  }
}

// Fold a finished block tile (vocabulary tile vt) into the running (max, sum of exp) of
// this lane's rows; no target logit is captured (k_token_logp computes them after the
// projection).  TWO (fp32 H as two planes): both planes' products of a row are in one
// accumulator, four block columns per wave (64 rows).  The shifted last vocabulary tile
// masks the entries before v_nom, which the previous tile counted.
template <bool TWO>
__device__ __forceinline__ void tile_epilogue16(
    f32x4 (&acc)[8][TWO ? 4 : 8], float (&m_run)[8], float (&s_run)[8], int vt, int V, int wm,
    int r16, int q) {
  constexpr int NR = TWO ? 4 : 8;          // block columns of distinct rows
  const int v_nom = vt * TBM;
  const int v0 = min(v_nom, V - TBM);
  if (v0 != v_nom) {
    // shifted last tile: add -inf to the entries below v_nom through the matrix core
    // (A: -inf at k = 0 for a dropped entry, B: 1 at k = 0; no 0 * inf is formed)
    const int thr = v_nom - v0 - wm * 128;
    bf16x8 bone = {};
    if (q == 0) bone[0] = (__bf16)1.0f;
#pragma unroll
    for (int mt = 0; mt < 8; ++mt) {
      bf16x8 amask = {};
      if (q == 0 && mt * 16 + r16 < thr) amask[0] = (__bf16)(-INFINITY);
#pragma unroll
      for (int nt = 0; nt < NR; ++nt)
        acc[mt][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(amask, bone, acc[mt][nt], 0, 0, 0);
    }
  }
#pragma unroll
  for (int nt = 0; nt < NR; ++nt) {
#pragma unroll
    for (int mt = 0; mt < 8; ++mt) asm volatile("" : "+a"(acc[mt][nt]));
    float gm = m_run[nt];
#pragma unroll
    for (int mt = 0; mt < 8; ++mt)
#pragma unroll
      for (int i = 0; i < 4; ++i) gm = fmaxf(gm, acc[mt][nt][i]);
    const float mb = gm == -INFINITY ? 0.f : gm * kLog2e;
    float ps[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int mt = 0; mt < 8; ++mt)
#pragma unroll
      for (int i = 0; i < 4; ++i) ps[i] += exp2_hw(fmaf(acc[mt][nt][i], kLog2e, -mb));
    s_run[nt] = s_run[nt] * exp2_hw(m_run[nt] * kLog2e - mb) + ((ps[0] + ps[1]) + (ps[2] + ps[3]));
    m_run[nt] = gm;
    zero_column<TWO>(acc, nt);  // folded: the next tile accumulates from zero
  }
}

// TWO (fp32 H as bf16 planes hi and lo, H = hi + lo): the B tile's 256 rows are, per
// 64-row quarter j, plane j & 1 of real rows 64 (j >> 1) .. + 63, so wave column wn holds
// the hi rows of its 64 real rows as fragments 0..3 and their lo rows as 4..7.  A k-step
// issues the 32 hi products (block (i / 4, i % 4)) and then the 32 lo products into the
// same 32 accumulators, 32 matrix ops apart.  A block tile covers 128 real rows with the
// matrix work of a 256-row bf16 tile and half its accumulators.
template <bool TWO>
__device__ __forceinline__ void project_m16(
    const uint16_t* __restrict__ W, int V, int d, const uint16_t* __restrict__ H,
    const uint16_t* __restrict__ Hlo, int n_rows, int n_vtiles, int32_t* __restrict__ flags,
    float2* __restrict__ part,
    int n_rtiles, int splits, int sr, int ss, int remap) {
  constexpr int BK = 64, CH = 8, RPD = 64 / CH;
  constexpr int NR = TWO ? 4 : 8;       // block columns of distinct rows per wave
  constexpr int RT = TWO ? 128 : TBN;   // real rows per block tile
  constexpr int ASZ = TBM * CH;  // 16-byte slots per operand half per buffer (32 KB)
  constexpr int BUFSZ = 2 * ASZ;
  constexpr int NDO = CH;        // load instructions per wave per operand per stage
  __shared__ u32x4 lds[2 * BUFSZ];
  __shared__ float2 red[2][TBN];
  __shared__ float2 runs[4][8][64];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wid & 1, wn = wid >> 1;
  const int r16 = lane & 15, q = lane >> 4;
  // the first launch index clears the flag word (no launch before this kernel does)
  if (blockIdx.x == 0 && threadIdx.x == 0) flags[0] = 0;
  int rt, split;
  tile_assign(n_rtiles, sr, ss, splits, remap, rt, split);
  if (rt >= n_rtiles || split >= splits) return;  // padding of the XCD-aware launch
  const int row_nom = rt * RT;
  const int row0 = min(row_nom, n_rows - RT);
  // consecutive ranges of L tiles (see the split choice); trailing ranges may be empty
  const int L = (n_vtiles + splits - 1) / splits;
  const int t0 = min(split * L, n_vtiles);
  const int t1 = min(t0 + L, n_vtiles);
  const int nk = d / BK;  // d is a multiple of BK
  const uint32_t rowb = (uint32_t)d * 2;
  // Buffer resources based at this workgroup's first H row and first head row, so that
  // every offset is local to its own tiles (32 bits suffice whatever the operand sizes):
  // H rows [row0, row0 + RT), head rows [vbase, vend) covering every tile of the range
  // (a tile starts at min(t * 256, V - 256); an empty range still loads one tile).
  const int vbase = min(t0 * TBM, V - TBM);
  const int vend = max(min(t1 * TBM, V), vbase + TBM);
  const __amdgpu_buffer_rsrc_t rH = rsrc_of(H + (size_t)row0 * d, (uint32_t)RT * rowb);
  const __amdgpu_buffer_rsrc_t rL = TWO ? rsrc_of(Hlo + (size_t)row0 * d, (uint32_t)RT * rowb) : rH;
  const __amdgpu_buffer_rsrc_t rW = rsrc_of(W + (size_t)vbase * d, (uint32_t)(vend - vbase) * rowb);
  const uint32_t hrow = 0;
  const int dr = wid * RPD + lane / CH;
  const uint32_t dvoff = (uint32_t)dr * rowb + (uint32_t)(((lane % CH) ^ swz16(dr)) * 16);
  const uint32_t m0_base = (uint32_t)(size_t)(__attribute__((address_space(3))) void*)lds +
                           (uint32_t)wid * 1024u;
  // fragment slot of k-step ks (0, 1) for block row 0 of this wave's half: row r16 of the
  // block, chunk 4 ks + q; blocks are 16 rows (128 slots) apart
  int fslot[2];
#pragma unroll
  for (int ks = 0; ks < 2; ++ks) fslot[ks] = r16 * CH + ((4 * ks + q) ^ swz16(r16));
  const int a_off = wm * 128 * CH, b_off_h = ASZ + wn * 128 * CH;

#pragma unroll
  for (int nt = 0; nt < 8; ++nt) runs[wid][nt][lane] = make_float2(-INFINITY, 0.f);

  const int G = (t1 - t0) * nk;
  int lt = t0, lk = 0, lg = 0;  // load cursor
  uint32_t l_ws = 0, l_hs = 0;
#define JET_CURSOR()                                                                         \
  {                                                                                          \
    const uint32_t ko = (uint32_t)lk * (BK * 2);                                             \
    l_ws = __builtin_amdgcn_readfirstlane((uint32_t)(min(lt * TBM, V - TBM) - vbase) * rowb + ko); \
    l_hs = __builtin_amdgcn_readfirstlane(hrow + ko);                                        \
    if (lg + 1 < G) {                                                                        \
      ++lg;                                                                                  \
      if (++lk == nk) {                                                                      \
        lk = 0;                                                                              \
        ++lt;                                                                                \
      }                                                                                      \
    }                                                                                        \
  }
  // load instruction Q (0 .. 2 NDO - 1): head rows first, then hidden-state rows.
  // Instruction jj of an operand fills B-tile rows 32 jj .. 32 jj + 31; with TWO those are
  // plane (jj >> 1) & 1 of real rows 64 (jj >> 2) + 32 (jj & 1) + 0 .. 31.
#define JET_DMA1(BI, Q)                                                                      \
  {                                                                                          \
    const int op_ = (Q) / NDO, jj_ = (Q) % NDO;                                              \
    const int hr_ = TWO ? 64 * (jj_ >> 2) + 32 * (jj_ & 1) : jj_ * 4 * RPD;                  \
    const __amdgpu_buffer_rsrc_t rb_ = (TWO && ((jj_ >> 1) & 1)) ? rL : rH;                  \
    dma16(op_ ? rb_ : rW, dvoff,                                                             \
          op_ ? l_hs + (uint32_t)hr_ * rowb : l_ws + (uint32_t)(jj_ * 4 * RPD) * rowb,         \
          m0_base + (uint32_t)(((BI) * BUFSZ + op_ * ASZ + jj_ * 256) * 16));                \
  }
  bf16x8 fa[2][8], fb[2][8];
  // fragment read JR (0 .. 15) of k-step KS_ into set F, in order of first use:
  // a0, b0..b7, a1..a7
#define JET_FRAG1(F, BOFF, KS_, JR)                                                          \
  {                                                                                          \
    if ((JR) >= 1 && (JR) <= 8) {                                                            \
      fb[F][(JR) - 1] = __builtin_bit_cast(                                                  \
          bf16x8, lds[(BOFF) + b_off_h + fslot[KS_] + ((JR) - 1) * 16 * CH]);                 \
    } else {                                                                                 \
      const int ta_ = (JR) == 0 ? 0 : (JR) - 8;                                              \
      fa[F][ta_] = __builtin_bit_cast(bf16x8, lds[(BOFF) + a_off + fslot[KS_] + ta_ * 16 * CH]); \
    }                                                                                        \
  }
  int bc = 0;
  // One stage g (buffer bc; the k-step 0 fragments of stage g already in set 0): two
  // k-steps of 64 MFMAs (block (i / 8, i % 8)).  k-step 0 reads the k-step 1 fragments at
  // every fourth slot.  Then every wave is done with buffer bc and stage g + 1 is awaited
  // (its loads were issued during the previous stage's k-step 1) behind the one barrier
  // of the stage.  k-step 1 reads the k-step 0 fragments of stage g + 1 (slots 0, 4, ..,
  // 60) and loads stage g + 2 into buffer bc (slots 2, 6, .., 62), so loads get half a
  // stage to a stage to land and no stage starts by waiting for LDS.
  // matrix op i of a k-step: A fragment MT_(i), B fragment FB_(i), accumulator (MT_, NT_)
#define MT_(i) (TWO ? ((i) % 32) / 4 : (i) / 8)
#define FB_(i) (TWO ? (i) % 4 + 4 * ((i) / 32) : (i) % 8)
#define NT_(i) (TWO ? (i) % 4 : (i) % 8)
#define JET_MSTAGE()                                                                         \
  {                                                                                          \
    const int b_nx = bc ^ 1;                                                                 \
    __builtin_amdgcn_sched_barrier(0);                                                       \
    _Pragma("unroll") for (int i = 0; i < 64; ++i) {                                         \
      acc[MT_(i)][NT_(i)] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(                         \
          fa[0][MT_(i)], fb[0][FB_(i)], acc[MT_(i)][NT_(i)], 0, 0, 0);                       \
      if (i % 4 == 0) JET_FRAG1(1, bc * BUFSZ, 1, i / 4);                                    \
      __builtin_amdgcn_sched_barrier(0);                                                     \
    }                                                                                        \
    vm_wait<0>();                                                                            \
    __syncthreads();                                                                         \
    JET_CURSOR();                                                                            \
    __builtin_amdgcn_sched_barrier(0);                                                       \
    _Pragma("unroll") for (int i = 0; i < 64; ++i) {                                         \
      acc[MT_(i)][NT_(i)] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(                         \
          fa[1][MT_(i)], fb[1][FB_(i)], acc[MT_(i)][NT_(i)], 0, 0, 0);                       \
      if (i % 4 == 0) {                                                                      \
        JET_FRAG1(0, b_nx * BUFSZ, 0, i / 4);                                                \
      } else if (i % 4 == 2) {                                                               \
        JET_DMA1(bc, i / 4);                                                                 \
      }                                                                                      \
      __builtin_amdgcn_sched_barrier(0);                                                     \
    }                                                                                        \
    bc = b_nx;                                                                               \
  }

  // prologue: stage 0 into buffer 0, stage 1 into buffer 1; stage 0 complete; its k-step 0
  // fragments into set 0
  JET_CURSOR();
#pragma unroll
  for (int qq = 0; qq < 2 * NDO; ++qq) JET_DMA1(0, qq);
  JET_CURSOR();
#pragma unroll
  for (int qq = 0; qq < 2 * NDO; ++qq) JET_DMA1(1, qq);
  vm_wait<2 * NDO>();
  __syncthreads();
#pragma unroll
  for (int jr = 0; jr < 16; ++jr) JET_FRAG1(0, 0, 0, jr);

  f32x4 acc[8][NR];
#pragma unroll
  for (int nt = 0; nt < NR; ++nt) zero_column<TWO>(acc, nt);
  for (int vt = t0; vt < t1; ++vt) {
    // two stages per trip (the buffer index alternates at run time, so an odd count only
    // adds one stage after the loop)
    for (int kb = 0; kb + 1 < nk; kb += 2) {
      JET_MSTAGE();
      JET_MSTAGE();
    }
    if (nk & 1) JET_MSTAGE();
    {
      // lane-derived values recomputed here (from the exec mask, in a form the compiler
      // cannot hoist) instead of being kept live across the stage loop: a spill reload
      // would make the epilogue wait for the loads in flight
      int lane_e;
      asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(lane_e));
      float m_run[8], s_run[8];
#pragma unroll
      for (int nt = 0; nt < NR; ++nt) {
        const float2 r = runs[wid][nt][lane_e];
        m_run[nt] = r.x;
        s_run[nt] = r.y;
      }
      tile_epilogue16<TWO>(acc, m_run, s_run, vt, V, wm, lane_e & 15, lane_e >> 4);
#pragma unroll
      for (int nt = 0; nt < NR; ++nt) runs[wid][nt][lane_e] = make_float2(m_run[nt], s_run[nt]);
    }
  }
  vm_wait<0>();  // no load may land in LDS after the workgroup ends
#undef JET_CURSOR
#undef JET_DMA1
#undef JET_FRAG1
#undef JET_MSTAGE
#undef MT_
#undef FB_
#undef NT_
  // merge the four lanes of each row (q = 0..3), then the two vocabulary halves (wm)
#pragma unroll
  for (int nt = 0; nt < NR; ++nt) {
    float m = runs[wid][nt][lane].x, sm = runs[wid][nt][lane].y;
    float m2 = __shfl_xor(m, 16), s2 = __shfl_xor(sm, 16);
    lse_merge(m, sm, m2, s2);
    m2 = __shfl_xor(m, 32);
    s2 = __shfl_xor(sm, 32);
    lse_merge(m, sm, m2, s2);
    if (q == 0) red[wm][wn * (16 * NR) + nt * 16 + r16] = make_float2(m, sm);
  }
  __syncthreads();
  if (tid < RT) {
    const int r = tid;
    float m = red[0][r].x, sm = red[0][r].y;
    lse_merge(m, sm, red[1][r].x, red[1][r].y);
    const int row = row0 + r;
    if (row >= row_nom) part[(size_t)split * n_rows + row] = make_float2(m, sm);
  }
}

__global__ __launch_bounds__(256, 1) void k_project_tiled_m16(
    const uint16_t* __restrict__ W, int V, int d, const uint16_t* __restrict__ H, int n_rows,
    int n_vtiles, int32_t* __restrict__ flags, float2* __restrict__ part, int n_rtiles,
    int splits, int sr, int ss, int remap) {
  project_m16<false>(W, V, d, H, nullptr, n_rows, n_vtiles, flags, part, n_rtiles, splits, sr,
                     ss, remap);
}

__global__ __launch_bounds__(256, 1) void k_project_tiled_m16x2(
    const uint16_t* __restrict__ W, int V, int d, const uint16_t* __restrict__ Hhi,
    const uint16_t* __restrict__ Hlo, int n_rows, int n_vtiles, int32_t* __restrict__ flags,
    float2* __restrict__ part,
    int n_rtiles, int splits, int sr, int ss, int remap) {
  project_m16<true>(W, V, d, Hhi, Hlo, n_rows, n_vtiles, flags, part, n_rtiles, splits, sr, ss,
                    remap);
}

}  // namespace

// d must be a whole number of 64-wide stages
int tiled_bk(bool hilo) { return 64; }

// fp32 H runs as two bf16 planes, 128 real rows per block tile
int tiled_row_tile(bool hilo, int d) { return hilo ? 128 : TBN; }

const char* tiled_kernel_name(bool hilo, int d) {
  return hilo ? "k_project_tiled_m16x2" : "k_project_tiled_m16";
}

hipError_t launch_project_tiled(const ScoreArgs& a) {
  const jet_problem* p = a.p;
  const Plan& pl = *a.plan;
  float2* part = reinterpret_cast<float2*>(a.ws + pl.off_part);
  // XCD-aware placement when the split count is a multiple of 8 and there are at least 2
  // row tiles: blocks of sr row tiles x ss splits per XCD, row tiles padded to a multiple of
  // sr and the launch to a multiple of 256; padding workgroups (row tile >= R) exit at once.
  // Otherwise the plain order P = rt * S + split.  One row tile has no head tile for a block
  // to share, and padding it to a block left 3 of 4 workgroups empty: 467 -> 352 us at
  // 256 rows, V = 248,320, d = 2560.  With 2 or 3 row tiles the blocks' sharing of each head
  // tile in L2 outweighs their padding (629 against 677 us at 384 rows).  bf16 H takes 8 x 4
  // blocks (each head tile shared 8 ways; 2% faster than 4 x 8 on large_batch) when that pads
  // at most 1/16 of the row tiles; the two-plane kernel, whose H tiles hold two planes, takes
  // 4 x 8 (with 8 x 4 it was no faster at 32 row tiles and 7% slower at 64).
  const int S = pl.grid_x, R = pl.n_rtiles;
  int sr = 1, ss = S, remap = 0, total = S * R;
  if (S % 8 == 0 && R >= 2) {
    sr = 4;
    ss = 8;
    if (!pl.hilo && R >= 8 && ((R + 7) / 8 * 8 - R) * 16 <= R) {
      sr = 8;
      ss = 4;
    }
    remap = 1;
    const int r_pad = (R + sr - 1) / sr * sr;
    total = (r_pad * S + 255) / 256 * 256;
  }
  dim3 grid(total), block(256);
  const uint16_t* W = static_cast<const uint16_t*>(p->W);
  // the kernels see rows_k rows (n_rows, or one whole row tile of zero-padded H); partials
  // are strided by rows_k
  const int rk = pl.rows_k;
  if (pl.hilo) {
    const uint16_t* hhi = reinterpret_cast<const uint16_t*>(a.ws + pl.off_hhi);
    const uint16_t* hlo = reinterpret_cast<const uint16_t*>(a.ws + pl.off_hlo);
    hipLaunchKernelGGL(k_project_tiled_m16x2, grid, block, 0, a.stream, W, p->V, p->d, hhi, hlo,
                       rk, pl.n_vgroups, a.flags, part, R, S, sr, ss, remap);
  } else {
    const uint16_t* H = pl.pad_h ? reinterpret_cast<const uint16_t*>(a.ws + pl.off_hpad)
                                 : static_cast<const uint16_t*>(p->H);
    hipLaunchKernelGGL(k_project_tiled_m16, grid, block, 0, a.stream, W, p->V, p->d, H, rk,
                       pl.n_vgroups, a.flags, part, R, S, sr, ss, remap);
  }
  return hipGetLastError();
}

}  // namespace jet
