// Normaliser merge and candidate decisions (k_merge: one wave per row; k_token_logp: one
// wave per token; k_decide: one wave per question); the shared device code is in jet_tail.h.
#include "jet_tail.h"

namespace jet {
namespace {

__global__ __launch_bounds__(256) void k_merge(const float2* __restrict__ part, int n_parts,
                                               int n_rows, long long rs, long long ps,
                                               float* __restrict__ lse) {
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= n_rows) return;
  const float l = merge_row(part, n_parts, (size_t)rs, (size_t)ps, row, lane);
  if (lane == 0) lse[row] = l;
}

// Token log-probabilities of a streaming-kernel problem, whose projection captures no
// targets (JET paper, Eq. 1-2: l_k = z[r, y] - LSE_r with r = tok_row[k], y = tok_target[k]).
// One wave per token: it loads row r's partials, computes the target logit as one dot
// product of the operands the projection multiplies (bf16 H, or fp32 H as its bf16 hi + lo;
// products and sums in fp32), merges the partials into LSE_r (the same bits as a row wave's
// merge), and stores l_k.  The target's logit is one of the terms of LSE_r, so l_k <= 0;
// its dot product is summed in another order than the projection's, so l_k is clamped to 0
// where rounding puts it above (NaN stays NaN).  An out-of-range row or target raises its
// flag and stores NaN.  Waves past the tokens each merge one row for the caller's row_lse.
// The head's rows are read whole by one wave: d / 8 chunks of 16 bytes, lane l taking chunks
// l, l + 64, ... (d is a multiple of 128 on this path).
struct TokArgs {
  const float2* part;
  int n_parts;  // <= 64 * kMergeBatch (the streaming kernel has at most 256 workgroups)
  const uint16_t* W;
  int V, d;
  const void* H;
  int n_rows;
  const int* tok_row;
  const int* tok_target;
  int n_tok;
  float* tok_logp;
  float* row_lse;  // NULL: no row waves
  int n_lse_rows;
  int32_t* flags;
};

constexpr int kDotBatch = 8;  // 16-byte head chunks per lane in flight (d <= 4096: one batch)

template <bool HF32>
__global__ __launch_bounds__(256) void k_token_logp(TokArgs a) {
  const int lane = threadIdx.x & 63;
  const long long w = (long long)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (w >= a.n_tok) {
    const long long row = w - a.n_tok;
    if (row >= a.n_lse_rows) return;
    const float l = merge_finish(merge_issue(a.part, a.n_parts, (int)row, lane), a.n_parts, lane);
    if (lane == 0) a.row_lse[row] = l;
    return;
  }
  const int k = (int)w;
  const int r = a.tok_row ? a.tok_row[k] : k;
  const int y = a.tok_target[k];
  uint32_t bad = 0u;
  if (r < 0 || r >= a.n_rows) bad |= JET_FLAG_BAD_ROW;
  if (y < 0 || y >= a.V) bad |= JET_FLAG_BAD_TARGET;
  if (bad) {
    if (lane == 0) {
      flag_or(a.flags, bad);
      a.tok_logp[k] = __builtin_nanf("");
    }
    return;
  }
  const RowParts rp = merge_issue(a.part, a.n_parts, r, lane);
  const int nch = a.d >> 3;
  const u32x4* wrow = reinterpret_cast<const u32x4*>(a.W + (size_t)y * a.d);
  float acc = 0.f;
  for (int c0 = 0; c0 < nch; c0 += 64 * kDotBatch) {
    u32x4 wv[kDotBatch], hv[kDotBatch][HF32 ? 2 : 1];
#pragma unroll
    for (int u = 0; u < kDotBatch; ++u) {
      const int c = min(c0 + lane + 64 * u, nch - 1);  // past the end: re-read, not used
      wv[u] = wrow[c];
      if constexpr (HF32) {
        const u32x4* h = reinterpret_cast<const u32x4*>(static_cast<const float*>(a.H) + (size_t)r * a.d) + 2 * c;
        hv[u][0] = h[0];
        hv[u][1] = h[1];
      } else {
        hv[u][0] = reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(a.H) + (size_t)r * a.d)[c];
      }
    }
#pragma unroll
    for (int u = 0; u < kDotBatch; ++u) {
      if (c0 + lane + 64 * u >= nch) continue;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const uint32_t wp = wv[u][j >> 1];
        const float wj = __uint_as_float((j & 1) ? (wp & 0xffff0000u) : (wp << 16));
        float hj;
        if constexpr (HF32) {
          const float x = __uint_as_float(hv[u][j >> 2][j & 3]);
          const float hi = bf16_to_f32(f32_to_bf16_rne(x));
          hj = hi + bf16_to_f32(f32_to_bf16_rne(x - hi));  // hi + lo, exact in fp32
        } else {
          const uint32_t hp = hv[u][0][j >> 1];
          hj = __uint_as_float((j & 1) ? (hp & 0xffff0000u) : (hp << 16));
        }
        acc = fmaf(hj, wj, acc);
      }
    }
  }
  const float z = wave_sum(acc);
  const float lse = merge_finish(rp, a.n_parts, lane);
  float l = z - lse;
  if (l > 0.f) l = 0.f;
  if (lane == 0) a.tok_logp[k] = l;
}

__global__ __launch_bounds__(256) void k_decide(DecideArgs a) {
  const int lane = threadIdx.x & 63;
  const int q = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (q >= a.n_q) return;
  decide_question(a, q, lane);
}

DecideArgs decide_args(const ScoreArgs& a) {
  const jet_problem* p = a.p;
  const jet_outputs* o = a.o;
  const Plan& pl = *a.plan;
  DecideArgs d;
  d.z_tgt = reinterpret_cast<const float*>(a.ws + pl.off_ztgt);
  d.lse = a.lse;
  d.tok_row = p->tok_row;
  d.n_rows = p->n_rows;
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
  d.logp_ready = pl.direct;
  return d;
}

}  // namespace

hipError_t launch_merge(const ScoreArgs& a) {
  const jet_problem* p = a.p;
  const Plan& pl = *a.plan;
  if (p->n_rows == 0) return hipSuccess;
  // row-major partials (streaming kernel): row r's partials contiguous; the others: one
  // partial per row per workgroup, strided by the rows the projection kernel saw
  const long long rs = pl.stream ? pl.n_parts : 1, ps = pl.stream ? 1 : pl.rows_k;
  hipLaunchKernelGGL(k_merge, dim3((p->n_rows + 3) / 4), dim3(256), 0, a.stream,
                     reinterpret_cast<const float2*>(a.ws + pl.off_part), pl.n_parts, p->n_rows,
                     rs, ps, a.lse);
  return hipGetLastError();
}

hipError_t launch_token_logp(const ScoreArgs& a) {
  const jet_problem* p = a.p;
  const Plan& pl = *a.plan;
  TokArgs t;
  t.part = reinterpret_cast<const float2*>(a.ws + pl.off_part);
  t.n_parts = pl.n_parts;
  t.W = static_cast<const uint16_t*>(p->W);
  t.V = p->V;
  t.d = p->d;
  t.H = p->H;
  t.n_rows = p->n_rows;
  t.tok_row = p->tok_row;
  t.tok_target = p->tok_target;
  t.n_tok = p->n_tok;
  t.tok_logp = a.o->tok_logp;
  t.row_lse = a.o->row_lse;
  t.n_lse_rows = a.o->row_lse ? p->n_rows : 0;
  t.flags = a.flags;
  if (!pl.direct || p->d % 128 != 0 || pl.n_parts > 64 * kMergeBatch) return hipErrorInvalidValue;
  const long long waves = (long long)t.n_tok + t.n_lse_rows;
  if (waves == 0) return hipSuccess;
  const dim3 grid((unsigned)((waves + 3) / 4));
  if (pl.hilo)
    hipLaunchKernelGGL(k_token_logp<true>, grid, dim3(256), 0, a.stream, t);
  else
    hipLaunchKernelGGL(k_token_logp<false>, grid, dim3(256), 0, a.stream, t);
  return hipGetLastError();
}

hipError_t launch_decide(const ScoreArgs& a) {
  const jet_problem* p = a.p;
  if (p->n_q == 0) return hipSuccess;
  hipLaunchKernelGGL(k_decide, dim3((p->n_q + 3) / 4), dim3(256), 0, a.stream, decide_args(a));
  return hipGetLastError();
}

}  // namespace jet
