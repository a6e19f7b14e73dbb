// Normaliser merge and candidate decisions.
//
// k_merge: LSE_r = M + log sum_j s_j exp(m_j - M) over the row's (m_j, s_j) partials, one
//   wave per row; lane i folds partials i, i+64, ... in order, then a fixed xor-shuffle
//   tree combines the lanes (every lane ends with the same bits).  The result does not
//   depend on the row's position.  (JET paper, Eq. 2: the full-vocabulary denominator.)
//
// k_decide: one wave per question (JET Eq. 3-5 and the decision rules; gemma-e2b doc,
//   "Candidate likelihoods" and "Output contracts"):
//     l_k   = z[row_k, y_k] - LSE_{row_k}                (written to tok_logp)
//     s(c)  = sum of l_k over the candidate's tokens, in token order
//     a_c   = s(c) / T ;  q_c = exp(a_c - max a) / sum exp(a - max a)
//     argmax: lowest index among the exact maxima of a (fixed order)
//     q(true) = q at the true index (given, or 1 for K = 2)
//     E = sum_i i q_i ;  gold NLL = (M + log Z) - (Mg + log Zg) over gold-text candidates
//     confidence = 1 - H(q) / ln K (1 for K = 1) ; mass = sum_c exp s(c), summed as
//     exp(max s) * sum_c exp(s(c) - max s) so that terms far below the largest keep their bits
//   Candidates are handled lane-strided (candidate c by lane (c - c0) % 64), every sum
//   runs in candidate order per lane and then through a fixed xor tree, so results are
//   bitwise reproducible.
#include "jet_internal.h"

namespace jet {
namespace {

__device__ inline float wave_sum(float x) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) x += __shfl_xor(x, off);
  return x;
}

__device__ inline float wave_max(float x) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) x = fmaxf(x, __shfl_xor(x, off));
  return x;
}

// Lane i folds partials i, i + 64, ... in order; eight of them are loaded before any is
// folded, so the loads of a row overlap instead of waiting one after another.
constexpr int kMergeBatch = 8;

__global__ __launch_bounds__(256) void k_merge(const float2* __restrict__ part, int n_parts,
                                               int n_rows, float* __restrict__ lse) {
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= n_rows) return;
  float m = -INFINITY, s = 0.f;
  for (int j0 = lane; j0 < n_parts; j0 += 64 * kMergeBatch) {
    float2 v[kMergeBatch];
#pragma unroll
    for (int u = 0; u < kMergeBatch; ++u) {
      const int j = j0 + 64 * u;
      v[u] = j < n_parts ? part[(size_t)j * n_rows + row] : make_float2(-INFINITY, 0.f);
    }
#pragma unroll
    for (int u = 0; u < kMergeBatch; ++u)
      if (j0 + 64 * u < n_parts) lse_merge(m, s, v[u].x, v[u].y);
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    const float m2 = __shfl_xor(m, off), s2 = __shfl_xor(s, off);
    lse_merge(m, s, m2, s2);
  }
  if (lane == 0) lse[row] = m + logf(s);
}

__global__ __launch_bounds__(256) void k_decide(
    const float* __restrict__ z_tgt, const float* __restrict__ lse, const int* __restrict__ tok_row,
    int n_rows, int n_tok, const int* __restrict__ cand_tok_off, int n_cand,
    const int* __restrict__ q_cand_off, int n_q, const int* __restrict__ cand_text_id,
    const int* __restrict__ q_gold_text_id, const int* __restrict__ q_true_idx, float T,
    float* __restrict__ tok_logp, float* __restrict__ cand_s, float* __restrict__ cand_q,
    int* __restrict__ q_argmax, float* __restrict__ q_true, float* __restrict__ q_expect,
    float* __restrict__ q_nll, float* __restrict__ q_conf, float* __restrict__ q_mass,
    int32_t* __restrict__ flags) {
  const int lane = threadIdx.x & 63;
  const int q = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (q >= n_q) return;
  const float NaN = __builtin_nanf("");
  int c0 = q_cand_off[q], c1 = q_cand_off[q + 1];
  if (c0 < 0 || c1 > n_cand || c1 <= c0) {
    if (lane == 0) {
      flag_or(flags, JET_FLAG_BAD_OFFSETS);
      q_argmax[q] = -1;
      if (q_true) q_true[q] = NaN;
      if (q_expect) q_expect[q] = NaN;
      if (q_nll) q_nll[q] = NaN;
      if (q_conf) q_conf[q] = NaN;
      if (q_mass) q_mass[q] = NaN;
    }
    return;
  }
  const int K = c1 - c0;
  // pass 1: token log-probabilities, candidate sums, running argmax
  float best = -INFINITY, smax = -INFINITY;
  int best_c = c1;  // sentinel: no finite candidate seen
  bool bad_off = false;
  // with at most 64 candidates a lane holds one: its sum stays in a register for passes 2-3
  float s_mine = 0.f;
  for (int c = c0 + lane; c < c1; c += 64) {
    int t0 = cand_tok_off[c], t1 = cand_tok_off[c + 1];
    float s = 0.f;
    if (t0 < 0 || t1 > n_tok || t1 <= t0) {
      bad_off = true;
      s = NaN;
    } else {
      for (int k = t0; k < t1; ++k) {
        const int r = tok_row ? tok_row[k] : k;
        const float l = (r >= 0 && r < n_rows) ? z_tgt[k] - lse[r] : NaN;
        tok_logp[k] = l;
        s += l;
      }
    }
    cand_s[c] = s;
    s_mine = s;
    smax = fmaxf(smax, s);
    const float a = s / T;
    if (a > best || (a == best && c < best_c)) {
      best = a;
      best_c = c;
    }
  }
  if (bad_off) flag_or(flags, JET_FLAG_BAD_OFFSETS);
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    const float ob = __shfl_xor(best, off);
    const int oc = __shfl_xor(best_c, off);
    if (ob > best || (ob == best && oc < best_c)) {
      best = ob;
      best_c = oc;
    }
  }
  const float M = best;
  const float Ms = wave_max(smax);  // shift of the mass sum
  const bool have_text = cand_text_id && q_gold_text_id;
  const int gold = have_text ? q_gold_text_id[q] : 0;
  const bool one_each = K <= 64;
  // pass 2: normalisers (all candidates; gold-text candidates)
  float z_part = 0.f, mg = -INFINITY;
  for (int c = c0 + lane; c < c1; c += 64) {
    const float a = (one_each ? s_mine : cand_s[c]) / T;
    z_part += expf(a - M);
    if (have_text && cand_text_id[c] == gold) mg = fmaxf(mg, a);
  }
  const float Z = wave_sum(z_part);
  const float Mg = have_text ? wave_max(mg) : -INFINITY;
  int t_idx = q_true_idx ? q_true_idx[q] : (K == 2 ? 1 : -1);
  if (t_idx < -1 || t_idx >= K) {
    if (lane == 0) flag_or(flags, JET_FLAG_BAD_TRUE_IDX);
    t_idx = -1;
  }
  // pass 3: q, expectation, entropy, mass, gold sum
  float e_part = 0.f, h_part = 0.f, mass_part = 0.f, zg_part = 0.f;
  for (int c = c0 + lane; c < c1; c += 64) {
    const float s = one_each ? s_mine : cand_s[c];
    const float a = s / T;
    const float qc = expf(a - M) / Z;
    cand_q[c] = qc;
    e_part += (float)(c - c0) * qc;
    if (qc > 0.f) h_part -= qc * logf(qc);
    mass_part += expf(s - Ms);
    if (have_text && cand_text_id[c] == gold && Mg != -INFINITY) zg_part += expf(a - Mg);
    if (q_true && c - c0 == t_idx) q_true[q] = qc;
  }
  const float E = wave_sum(e_part);
  const float Hq = wave_sum(h_part);
  const float mass = Ms == -INFINITY ? 0.f : expf(Ms) * wave_sum(mass_part);
  const float Zg = wave_sum(zg_part);
  if (lane == 0) {
    q_argmax[q] = best_c < c1 ? best_c - c0 : -1;
    if (q_true && t_idx < 0) q_true[q] = NaN;
    if (q_expect) q_expect[q] = E;
    if (q_nll) {
      float nll = NaN;
      if (have_text) nll = (Mg == -INFINITY) ? INFINITY : (M + logf(Z)) - (Mg + logf(Zg));
      q_nll[q] = nll;
    }
    if (q_conf) q_conf[q] = K == 1 ? 1.f : 1.f - Hq / logf((float)K);
    if (q_mass) q_mass[q] = mass;
  }
}

}  // namespace

hipError_t launch_merge(const ScoreArgs& a) {
  const jet_problem* p = a.p;
  const Plan& pl = *a.plan;
  if (p->n_rows == 0) return hipSuccess;
  hipLaunchKernelGGL(k_merge, dim3((p->n_rows + 3) / 4), dim3(256), 0, a.stream,
                     reinterpret_cast<const float2*>(a.ws + pl.off_part), pl.n_parts, p->n_rows,
                     a.lse);
  return hipGetLastError();
}

hipError_t launch_decide(const ScoreArgs& a) {
  const jet_problem* p = a.p;
  const jet_outputs* o = a.o;
  if (p->n_q == 0) return hipSuccess;
  const Plan& pl = *a.plan;
  hipLaunchKernelGGL(k_decide, dim3((p->n_q + 3) / 4), dim3(256), 0, a.stream,
                     reinterpret_cast<const float*>(a.ws + pl.off_ztgt), a.lse, p->tok_row,
                     p->n_rows, p->n_tok, p->cand_tok_off, p->n_cand, p->q_cand_off, p->n_q,
                     p->cand_text_id, p->q_gold_text_id, p->q_true_idx, p->T, o->tok_logp,
                     o->cand_s, o->cand_q, o->q_argmax, o->q_true, o->q_expect, o->q_gold_nll,
                     o->q_confidence, o->q_mass, a.flags);
  return hipGetLastError();
}

}  // namespace jet
