// Normaliser merge and candidate decisions (k_merge: one wave per row; k_decide: one wave
// per question); the device code is in jet_tail.h.
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
  return d;
}

}  // namespace

hipError_t launch_merge(const ScoreArgs& a) {
  const jet_problem* p = a.p;
  const Plan& pl = *a.plan;
  if (p->n_rows == 0) return hipSuccess;
  // row-major partials (streaming kernel): row r's partials contiguous
  const long long rs = pl.stream ? pl.n_parts : 1, ps = pl.stream ? 1 : p->n_rows;
  hipLaunchKernelGGL(k_merge, dim3((p->n_rows + 3) / 4), dim3(256), 0, a.stream,
                     reinterpret_cast<const float2*>(a.ws + pl.off_part), pl.n_parts, p->n_rows,
                     rs, ps, a.lse);
  return hipGetLastError();
}

hipError_t launch_decide(const ScoreArgs& a) {
  const jet_problem* p = a.p;
  if (p->n_q == 0) return hipSuccess;
  hipLaunchKernelGGL(k_decide, dim3((p->n_q + 3) / 4), dim3(256), 0, a.stream, decide_args(a));
  return hipGetLastError();
}

}  // namespace jet
