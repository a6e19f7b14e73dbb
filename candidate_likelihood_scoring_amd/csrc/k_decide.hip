// Token log-probabilities and candidate decisions (k_token_logp: one wave per token, plus
// one per row whose LSE no token writes; k_decide: one wave per question); the shared device
// code is in jet_tail.h.
#include "jet_tail.h"

namespace jet {
namespace {

// Token log-probabilities after the projection, which captures no targets (JET paper,
// Eq. 1-2: l_k = z[r, y] - LSE_r with r = tok_row[k], y = tok_target[k]).  One wave per
// token: it loads row r's first partials, computes the target logit as one dot product of
// the operands the projection multiplies (a bf16 head with bf16 H, or with fp32 H as its
// bf16 hi + lo; an fp32 head with fp32 H; products and sums in fp32), merges the partials
// into LSE_r (merge_finish: the same bits for every wave that merges the row), and stores
// l_k.  The target's logit is one of the terms of LSE_r, so l_k <= 0; its dot product is
// summed in another order than the projection's, so l_k is clamped to 0 where rounding puts
// it above (NaN stays NaN).  An out-of-range row or target raises its flag and stores NaN.
// When token k is on row k (no row map), its wave also stores row_lse[k]; the waves past
// the tokens merge the rows no token wave stores (all rows when there is a row map).
// A head row is read whole by one wave: d / 8 chunks of 8 elements (16 bytes of a bf16
// head, 32 of an fp32 one), lane l taking chunks l, l + 64, ... (d is a multiple of 32).
struct TokArgs {
  const float2* part;  // partial j of row r at part[r * rs + j * ps]
  int n_parts;
  long long rs, ps;
  const void* W;
  int V, d;
  const void* H;
  int n_rows;
  const int* tok_row;
  const int* tok_target;
  int n_tok;
  float* tok_logp;
  float* row_lse;   // NULL: no row LSE is stored
  int row_first;    // first row a row wave merges (n_tok when token k is on row k)
  int32_t* flags;
};

template <bool WF32, bool HF32>
__device__ inline float target_dot(const TokArgs& a, int r, int y, int lane) {
  constexpr int kBatch = WF32 ? 4 : 8;  // 8-element chunks per lane in flight
  constexpr int WQ = WF32 ? 2 : 1, HQ = HF32 ? 2 : 1;  // 16-byte loads per chunk
  const int nch = a.d >> 3;
  const u32x4* wrow = reinterpret_cast<const u32x4*>(
      static_cast<const char*>(a.W) + (size_t)y * a.d * (WF32 ? 4 : 2));
  const u32x4* hrow = reinterpret_cast<const u32x4*>(
      static_cast<const char*>(a.H) + (size_t)r * a.d * (HF32 ? 4 : 2));
  float acc = 0.f;
  for (int c0 = 0; c0 < nch; c0 += 64 * kBatch) {
    u32x4 wv[kBatch][WQ], hv[kBatch][HQ];
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      const int c = min(c0 + lane + 64 * u, nch - 1);  // past the end: re-read, not used
#pragma unroll
      for (int q = 0; q < WQ; ++q) wv[u][q] = wrow[WQ * c + q];
#pragma unroll
      for (int q = 0; q < HQ; ++q) hv[u][q] = hrow[HQ * c + q];
    }
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      if (c0 + lane + 64 * u >= nch) continue;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        float wj, hj;
        if constexpr (WF32) {
          wj = __uint_as_float(wv[u][j >> 2][j & 3]);
        } else {
          const uint32_t wp = wv[u][0][j >> 1];
          wj = __uint_as_float((j & 1) ? (wp & 0xffff0000u) : (wp << 16));
        }
        if constexpr (HF32) {
          const float x = __uint_as_float(hv[u][j >> 2][j & 3]);
          if constexpr (WF32) {
            hj = x;  // fp32 head: fp32 products
          } else {
            const float hi = bf16_to_f32(f32_to_bf16_rne(x));
            hj = hi + bf16_to_f32(f32_to_bf16_rne(x - hi));  // hi + lo, exact in fp32
          }
        } else {
          const uint32_t hp = hv[u][0][j >> 1];
          hj = __uint_as_float((j & 1) ? (hp & 0xffff0000u) : (hp << 16));
        }
        acc = fmaf(hj, wj, acc);
      }
    }
  }
  return wave_sum(acc);
}

template <bool WF32, bool HF32>
__global__ __launch_bounds__(256) void k_token_logp(TokArgs a) {
  const int lane = threadIdx.x & 63;
  const long long w = (long long)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (w >= a.n_tok) {
    const long long row = a.row_first + (w - a.n_tok);
    if (row >= a.n_rows) return;
    const RowParts rp = merge_issue(a.part, a.n_parts, a.rs, a.ps, (int)row, lane);
    const float l = merge_finish(rp, a.part, a.n_parts, a.rs, a.ps, (int)row, lane);
    if (lane == 0) a.row_lse[row] = l;
    return;
  }
  const int k = (int)w;
  const int r = a.tok_row ? a.tok_row[k] : k;
  const int y = a.tok_target[k];
  const bool bad_target = y < 0 || y >= a.V;
  if (r < 0 || r >= a.n_rows) {
    if (lane == 0) {
      flag_or(a.flags, JET_FLAG_BAD_ROW | (bad_target ? (uint32_t)JET_FLAG_BAD_TARGET : 0u));
      a.tok_logp[k] = __builtin_nanf("");
    }
    return;
  }
  const RowParts rp = merge_issue(a.part, a.n_parts, a.rs, a.ps, r, lane);
  const float z = bad_target ? __builtin_nanf("") : target_dot<WF32, HF32>(a, r, y, lane);
  const float lse = merge_finish(rp, a.part, a.n_parts, a.rs, a.ps, r, lane);
  float l = z - lse;
  if (l > 0.f) l = 0.f;
  if (lane == 0) {
    if (bad_target) flag_or(a.flags, JET_FLAG_BAD_TARGET);
    a.tok_logp[k] = l;
    if (a.row_lse && !a.tok_row) a.row_lse[k] = lse;
  }
}

__global__ __launch_bounds__(256) void k_decide(DecideArgs a) {
  const int lane = threadIdx.x & 63;
  const int q = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (q >= a.n_q) return;
  decide_question(a, q, lane);
}

// The flag word when no projection runs (a problem without rows, hence without tokens).
__global__ void k_clear_flags(int32_t* __restrict__ flags) {
  if (threadIdx.x == 0) flags[0] = 0;
}

DecideArgs decide_args(const ScoreArgs& a) {
  const jet_problem* p = a.p;
  const jet_outputs* o = a.o;
  DecideArgs d;
  d.n_tok = p->n_tok;
  d.cand_tok_off = p->cand_tok_off;
  d.n_cand = p->n_cand;
  d.q_cand_off = p->q_cand_off;
  d.n_q = p->n_q;
  d.cand_text_id = p->cand_text_id;
  d.q_gold_text_id = p->q_gold_text_id;
  d.q_true_idx = p->q_true_idx;
  d.T = p->T;
  d.tok_logp = o->tok_logp;
  d.cand_s = o->cand_s;
  d.cand_q = o->cand_q;
  d.q_argmax = o->q_argmax;
  d.q_true = o->q_true;
  d.q_expect = o->q_expect;
  d.q_nll = o->q_gold_nll;
  d.q_conf = o->q_confidence;
  d.q_mass = o->q_mass;
  d.flags = a.flags;
  return d;
}

}  // namespace

hipError_t launch_token_logp(const ScoreArgs& a) {
  const jet_problem* p = a.p;
  const Plan& pl = *a.plan;
  if (p->n_rows == 0) {  // no tokens either: only the flag word needs its clear
    hipLaunchKernelGGL(k_clear_flags, dim3(1), dim3(64), 0, a.stream, a.flags);
    return hipGetLastError();
  }
  TokArgs t;
  t.part = reinterpret_cast<const float2*>(a.ws + pl.off_part);
  t.n_parts = pl.n_parts;
  // row-major partials (streaming kernel): row r's partials contiguous; the others: one
  // partial per row per workgroup, strided by the rows the projection kernel saw
  t.rs = pl.stream ? pl.n_parts : 1;
  t.ps = pl.stream ? 1 : pl.rows_k;
  t.W = p->W;
  t.V = p->V;
  t.d = p->d;
  t.H = p->H;
  t.n_rows = p->n_rows;
  t.tok_row = p->tok_row;
  t.tok_target = p->tok_target;
  t.n_tok = p->n_tok;
  t.tok_logp = a.o->tok_logp;
  t.row_lse = a.o->row_lse;
  // rows the token waves do not store: none without row_lse; rows past the tokens when
  // token k is on row k; every row with a row map
  t.row_first = !t.row_lse ? p->n_rows : (p->tok_row ? 0 : p->n_tok);
  t.flags = a.flags;
  const long long waves = (long long)t.n_tok + (p->n_rows - t.row_first);
  if (waves == 0) return hipSuccess;
  const dim3 grid((unsigned)((waves + 3) / 4));
  if (p->w_dtype == JET_F32)
    hipLaunchKernelGGL((k_token_logp<true, true>), grid, dim3(256), 0, a.stream, t);
  else if (pl.hilo)
    hipLaunchKernelGGL((k_token_logp<false, true>), grid, dim3(256), 0, a.stream, t);
  else
    hipLaunchKernelGGL((k_token_logp<false, false>), grid, dim3(256), 0, a.stream, t);
  return hipGetLastError();
}

hipError_t launch_decide(const ScoreArgs& a) {
  const jet_problem* p = a.p;
  if (p->n_q == 0) return hipSuccess;
  hipLaunchKernelGGL(k_decide, dim3((p->n_q + 3) / 4), dim3(256), 0, a.stream, decide_args(a));
  return hipGetLastError();
}

}  // namespace jet
