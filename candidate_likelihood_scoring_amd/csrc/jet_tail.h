// Device code of the normaliser merge and the per-question decisions (k_token_logp, k_decide).
//
// merge_issue / merge_finish: LSE_r = M + log sum_j s_j exp(m_j - M) over the row's
//   (m_j, s_j) partials (JET paper, Eq. 2: the full-vocabulary denominator).  One wave per
//   row: lane i folds partials i, i + 64, ... in order, then a fixed lane tree
//   (wave_lse_merge) combines the lanes, so every lane ends with the same bits and the
//   result does not depend on the row's position.
// decide_question: one wave per question (JET Eq. 3-5 and the decision rules; gemma-e2b
//   doc, "Candidate likelihoods" and "Output contracts"), from the token log-probabilities
//   l_k = z[row_k, y_k] - LSE_{row_k} that k_token_logp stored in tok_logp:
//     s(c)  = sum of l_k over the candidate's tokens, in token order
//     a_c   = s(c) / T ;  q_c = exp(a_c - max a) / sum exp(a - max a)
//     argmax: lowest index among the exact maxima of a (fixed order)
//     q(true) = q at the true index (given, or 1 for K = 2)
//     E = sum_i i q_i ;  gold NLL = (M + log Z) - (Mg + log Zg) over gold-text candidates
//     confidence = 1 - H(q) / ln K (1 for K = 1) ; mass = sum_c exp s(c), summed as
//     exp(max s) * sum_c exp(s(c) - max s) so that terms far below the largest keep their bits
//   Candidates are handled lane-strided (candidate c by lane (c - c0) % 64), every sum runs
//   in candidate order per lane and then through a fixed lane tree, so results are bitwise
//   reproducible.
#pragma once

#include "jet_internal.h"

namespace jet {

// Wave reductions in a fixed tree, on lane moves within rows of 16 lanes (DPP: no LDS
// round trip) and then the four row results read from lanes 0, 16, 32, 48:
//   1. pair lanes l and l ^ 1 (quad_perm [1,0,3,2]);  2. pair l and l ^ 2 (quad_perm
//   [2,3,0,1]), after which the four lanes of a quad hold equal values;  3. pair the two
//   quads of each half-row (row_half_mirror, lane i with 7 - i);  4. pair the two half-rows
//   of each row (row_mirror, i with 15 - i);  5. (r0 op r1) op (r2 op r3) over the rows.
// Every operation used is commutative in its bits, so both lanes of a pair compute the same
// value, every lane returns the same result, and the result depends only on the lanes'
// values in lane order.  All 64 lanes must be active.
constexpr int kDppXor1 = 0xB1, kDppXor2 = 0x4E, kDppHalfMirror = 0x141, kDppMirror = 0x140;

template <int CTRL>
__device__ inline float dpp_f(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL,
                                                               0xF, 0xF, false));
}
template <int CTRL>
__device__ inline int dpp_i(int x) {
  return __builtin_amdgcn_update_dpp(0, x, CTRL, 0xF, 0xF, false);
}
__device__ inline float lane_f(float x, int l) {
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), l));
}

__device__ inline float wave_sum(float x) {
  x += dpp_f<kDppXor1>(x);
  x += dpp_f<kDppXor2>(x);
  x += dpp_f<kDppHalfMirror>(x);
  x += dpp_f<kDppMirror>(x);
  return (lane_f(x, 0) + lane_f(x, 16)) + (lane_f(x, 32) + lane_f(x, 48));
}

__device__ inline float wave_max(float x) {
  x = fmaxf(x, dpp_f<kDppXor1>(x));
  x = fmaxf(x, dpp_f<kDppXor2>(x));
  x = fmaxf(x, dpp_f<kDppHalfMirror>(x));
  x = fmaxf(x, dpp_f<kDppMirror>(x));
  return fmaxf(fmaxf(lane_f(x, 0), lane_f(x, 16)), fmaxf(lane_f(x, 32), lane_f(x, 48)));
}

// (value, index) with the larger value winning and the lower index winning ties
__device__ inline void argmax_pick(float& v, int& i, float v2, int i2) {
  if (v2 > v || (v2 == v && i2 < i)) {
    v = v2;
    i = i2;
  }
}
template <int CTRL>
__device__ inline void argmax_step(float& v, int& i) {
  argmax_pick(v, i, dpp_f<CTRL>(v), dpp_i<CTRL>(i));
}
__device__ inline void wave_argmax(float& v, int& i) {
  argmax_step<kDppXor1>(v, i);
  argmax_step<kDppXor2>(v, i);
  argmax_step<kDppHalfMirror>(v, i);
  argmax_step<kDppMirror>(v, i);
  float v0 = lane_f(v, 0), v2 = lane_f(v, 32);
  int i0 = __builtin_amdgcn_readlane(i, 0), i2 = __builtin_amdgcn_readlane(i, 32);
  argmax_pick(v0, i0, lane_f(v, 16), __builtin_amdgcn_readlane(i, 16));
  argmax_pick(v2, i2, lane_f(v, 48), __builtin_amdgcn_readlane(i, 48));
  argmax_pick(v0, i0, v2, i2);
  v = v0;
  i = i0;
}

// Online-logsumexp states (m, s) merged over the wave in the same tree (lse_merge is
// symmetric in its bits).
template <int CTRL>
__device__ inline void lse_step(float& m, float& s) {
  lse_merge(m, s, dpp_f<CTRL>(m), dpp_f<CTRL>(s));
}
__device__ inline void wave_lse_merge(float& m, float& s) {
  lse_step<kDppXor1>(m, s);
  lse_step<kDppXor2>(m, s);
  lse_step<kDppHalfMirror>(m, s);
  lse_step<kDppMirror>(m, s);
  float m0 = lane_f(m, 0), s0 = lane_f(s, 0), m2 = lane_f(m, 32), s2 = lane_f(s, 32);
  lse_merge(m0, s0, lane_f(m, 16), lane_f(s, 16));
  lse_merge(m2, s2, lane_f(m, 48), lane_f(s, 48));
  lse_merge(m0, s0, m2, s2);
  m = m0;
  s = s0;
}

// Partials loaded per lane before any is folded, so a row's loads overlap.
constexpr int kMergeBatch = 8;

// Full-vocabulary LSE of one row from its n_parts partials, partial j of the row at
// part[row * rs + j * ps] (the streaming kernel stores a row's partials contiguously, rs =
// n_parts, ps = 1; the other kernels one partial per row per workgroup, rs = 1, ps = the
// kernel's row count).  Lane i folds partials i, i + 64, ... in order, then a fixed lane tree
// (wave_lse_merge) combines the lanes, so every lane ends with the same bits and the result
// does not depend on the row's position.  In two halves, so a wave can put other loads in
// flight between them: merge_issue loads the first 64 * kMergeBatch partials into registers;
// merge_finish folds them, then loads and folds the rest kMergeBatch per lane at a time.
struct RowParts {
  float2 v[kMergeBatch];
};
__device__ inline RowParts merge_issue(const float2* __restrict__ part, int n_parts, size_t rs,
                                       size_t ps, int row, int lane) {
  RowParts r;
#pragma unroll
  for (int u = 0; u < kMergeBatch; ++u) {
    const int j = lane + 64 * u;
    r.v[u] = j < n_parts ? part[(size_t)row * rs + (size_t)j * ps] : make_float2(-INFINITY, 0.f);
  }
  return r;
}
__device__ inline float merge_finish(const RowParts& r, const float2* __restrict__ part,
                                     int n_parts, size_t rs, size_t ps, int row, int lane) {
  float m = -INFINITY, s = 0.f;
#pragma unroll
  for (int u = 0; u < kMergeBatch; ++u)
    if (lane + 64 * u < n_parts) lse_merge(m, s, r.v[u].x, r.v[u].y);
  for (int j0 = lane + 64 * kMergeBatch; j0 < n_parts; j0 += 64 * kMergeBatch) {
    const RowParts more = merge_issue(part + (size_t)(j0 - lane) * ps, n_parts - (j0 - lane), rs, ps, row, lane);
#pragma unroll
    for (int u = 0; u < kMergeBatch; ++u)
      if (j0 + 64 * u < n_parts) lse_merge(m, s, more.v[u].x, more.v[u].y);
  }
  wave_lse_merge(m, s);
  return m + logf(s);
}

// Everything decide_question reads and writes (device pointers; optional ones may be NULL).
struct DecideArgs {
  int n_tok;
  const int* cand_tok_off;
  int n_cand;
  const int* q_cand_off;
  int n_q;
  const int* cand_text_id;
  const int* q_gold_text_id;
  const int* q_true_idx;
  float T;
  const float* tok_logp;  // written by k_token_logp
  float* cand_s;
  float* cand_q;
  int* q_argmax;
  float* q_true;
  float* q_expect;
  float* q_nll;
  float* q_conf;
  float* q_mass;
  int32_t* flags;
};

// All outputs of question q, computed by one wave (every lane calls it with the same q).
__device__ inline void decide_question(const DecideArgs& a, int q, int lane) {
  const float NaN = __builtin_nanf("");
  // question-level inputs are loaded with the question's offsets, and each lane's candidate
  // text id with its token offsets, so that no load waits behind the token loop
  const bool have_text = a.cand_text_id && a.q_gold_text_id;
  const int gold = have_text ? a.q_gold_text_id[q] : 0;
  const int t_given = a.q_true_idx ? a.q_true_idx[q] : 0;
  int c0 = a.q_cand_off[q], c1 = a.q_cand_off[q + 1];
  if (c0 < 0 || c1 > a.n_cand || c1 <= c0) {
    if (lane == 0) {
      flag_or(a.flags, JET_FLAG_BAD_OFFSETS);
      a.q_argmax[q] = -1;
      if (a.q_true) a.q_true[q] = NaN;
      if (a.q_expect) a.q_expect[q] = NaN;
      if (a.q_nll) a.q_nll[q] = NaN;
      if (a.q_conf) a.q_conf[q] = NaN;
      if (a.q_mass) a.q_mass[q] = NaN;
    }
    return;
  }
  const int K = c1 - c0;
  // pass 1: token log-probabilities, candidate sums, running argmax
  float best = -INFINITY, smax = -INFINITY;
  int best_c = c1;  // sentinel: no finite candidate seen
  bool bad_off = false;
  // with at most 64 candidates a lane holds one: its sum and text id stay in registers for
  // passes 2-3
  float s_mine = 0.f;
  int text_mine = 0;
  for (int c = c0 + lane; c < c1; c += 64) {
    int t0 = a.cand_tok_off[c], t1 = a.cand_tok_off[c + 1];
    if (have_text) text_mine = a.cand_text_id[c];
    float s = 0.f;
    if (t0 < 0 || t1 > a.n_tok || t1 <= t0) {
      bad_off = true;
      s = NaN;
    } else {
      for (int k = t0; k < t1; ++k) s += a.tok_logp[k];
    }
    a.cand_s[c] = s;
    s_mine = s;
    smax = fmaxf(smax, s);
    const float av = s / a.T;
    if (av > best || (av == best && c < best_c)) {
      best = av;
      best_c = c;
    }
  }
  if (bad_off) flag_or(a.flags, JET_FLAG_BAD_OFFSETS);
  wave_argmax(best, best_c);
  const float M = best;
  const float Ms = wave_max(smax);  // shift of the mass sum
  const bool one_each = K <= 64;
  // pass 2: normalisers (all candidates; gold-text candidates)
  float z_part = 0.f, mg = -INFINITY;
  for (int c = c0 + lane; c < c1; c += 64) {
    const float av = (one_each ? s_mine : a.cand_s[c]) / a.T;
    z_part += expf(av - M);
    if (have_text && (one_each ? text_mine : a.cand_text_id[c]) == gold) mg = fmaxf(mg, av);
  }
  const float Z = wave_sum(z_part);
  const float Mg = have_text ? wave_max(mg) : -INFINITY;
  int t_idx = a.q_true_idx ? t_given : (K == 2 ? 1 : -1);
  if (t_idx < -1 || t_idx >= K) {
    if (lane == 0) flag_or(a.flags, JET_FLAG_BAD_TRUE_IDX);
    t_idx = -1;
  }
  // pass 3: q, expectation, entropy, mass, gold sum
  float e_part = 0.f, h_part = 0.f, mass_part = 0.f, zg_part = 0.f;
  for (int c = c0 + lane; c < c1; c += 64) {
    const float s = one_each ? s_mine : a.cand_s[c];
    const float av = s / a.T;
    const float qc = expf(av - M) / Z;
    a.cand_q[c] = qc;
    e_part += (float)(c - c0) * qc;
    if (qc > 0.f) h_part -= qc * logf(qc);
    mass_part += expf(s - Ms);
    if (have_text && (one_each ? text_mine : a.cand_text_id[c]) == gold && Mg != -INFINITY)
      zg_part += expf(av - Mg);
    if (a.q_true && c - c0 == t_idx) a.q_true[q] = qc;
  }
  const float E = wave_sum(e_part);
  const float Hq = wave_sum(h_part);
  const float mass = Ms == -INFINITY ? 0.f : expf(Ms) * wave_sum(mass_part);
  const float Zg = wave_sum(zg_part);
  if (lane == 0) {
    a.q_argmax[q] = best_c < c1 ? best_c - c0 : -1;
    if (a.q_true && t_idx < 0) a.q_true[q] = NaN;
    if (a.q_expect) a.q_expect[q] = E;
    if (a.q_nll) {
      float nll = NaN;
      if (have_text) nll = (Mg == -INFINITY) ? INFINITY : (M + logf(Z)) - (Mg + logf(Zg));
      a.q_nll[q] = nll;
    }
    if (a.q_conf) a.q_conf[q] = K == 1 ? 1.f : 1.f - Hq / logf((float)K);
    if (a.q_mass) a.q_mass[q] = mass;
  }
}

}  // namespace jet
