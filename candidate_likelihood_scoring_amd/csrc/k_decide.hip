// Token log-probabilities and candidate decisions (k_token_logp: one wave per token, plus
// one per row whose LSE no token writes; k_decide: one wave per question, or a whole
// workgroup for a question with more than 64 candidates); the shared device code is in
// jet_tail.h.
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

// Questions with more than 64 candidates (on problems where one could have more than
// 1,024, see launch_decide).  One wave walks a question's candidates three
// times, 64 at a time, with a dependent pair of loads (token offsets, then log-probabilities)
// per candidate; for a question of thousands of candidates that one wave takes milliseconds
// (3.1 ms for 131,072 single-token candidates).  Such a question is taken by all 16 waves of
// its workgroup instead: thread t takes candidates c0 + t, c0 + t + 1024, ..., loading the
// offsets and first tokens of four candidates before summing any; each sum runs in
// candidate order per thread, then through the wave tree and over the 16 waves in order, so
// the results are bitwise reproducible.  The same outputs and rules as decide_question.
constexpr int kDecideWaves = 16, kDecideThreads = kDecideWaves * 64, kDecideBatch = 4;

struct BlockRed {  // per-wave partials of the workgroup reductions
  float v[4][kDecideWaves];
  int i[kDecideWaves];
};

// N sums over the workgroup (each wave's tree, then waves 0..15 in order), every thread
// receiving the results
template <int N>
__device__ inline void block_sums(float (&x)[N], BlockRed& r, int lane, int wid) {
#pragma unroll
  for (int n = 0; n < N; ++n) {
    x[n] = wave_sum(x[n]);
    if (lane == 0) r.v[n][wid] = x[n];
  }
  __syncthreads();
#pragma unroll
  for (int n = 0; n < N; ++n) {
    float t = r.v[n][0];
    for (int w = 1; w < kDecideWaves; ++w) t += r.v[n][w];
    x[n] = t;
  }
  __syncthreads();
}

__device__ void decide_question_block(const DecideArgs& a, int q, BlockRed& red, int tid) {
  const int lane = tid & 63, wid = tid >> 6;
  const float NaN = __builtin_nanf("");
  const bool have_text = a.cand_text_id && a.q_gold_text_id;
  const int gold = have_text ? a.q_gold_text_id[q] : 0;
  const int t_given = a.q_true_idx ? a.q_true_idx[q] : 0;
  const int c0 = a.q_cand_off[q], c1 = a.q_cand_off[q + 1];  // valid, c1 - c0 > 64
  const int K = c1 - c0;
  // pass 1: candidate sums, running argmax, largest sum
  float best = -INFINITY, smax = -INFINITY;
  int best_c = c1;  // sentinel: no finite candidate seen
  bool bad_off = false;
  for (int cb = c0 + tid; cb < c1; cb += kDecideBatch * kDecideThreads) {
    int t0[kDecideBatch], t1[kDecideBatch];
#pragma unroll
    for (int u = 0; u < kDecideBatch; ++u) {
      const int c = cb + u * kDecideThreads;
      t0[u] = c < c1 ? a.cand_tok_off[c] : 0;
      t1[u] = c < c1 ? a.cand_tok_off[c + 1] : 0;
    }
    bool ok[kDecideBatch];
    float first[kDecideBatch];
#pragma unroll
    for (int u = 0; u < kDecideBatch; ++u) {
      ok[u] = t0[u] >= 0 && t1[u] <= a.n_tok && t1[u] > t0[u];
      first[u] = ok[u] ? a.tok_logp[t0[u]] : 0.f;
    }
#pragma unroll
    for (int u = 0; u < kDecideBatch; ++u) {
      const int c = cb + u * kDecideThreads;
      if (c < c1) {
        float s = NaN;
        if (!ok[u]) {
          bad_off = true;
        } else {
          s = 0.f;
          s += first[u];
          for (int k = t0[u] + 1; k < t1[u]; ++k) s += a.tok_logp[k];
        }
        a.cand_s[c] = s;
        smax = fmaxf(smax, s);
        const float av = s / a.T;
        if (av > best || (av == best && c < best_c)) {
          best = av;
          best_c = c;
        }
      }
    }
  }
  if (bad_off) flag_or(a.flags, JET_FLAG_BAD_OFFSETS);
  wave_argmax(best, best_c);
  smax = wave_max(smax);
  if (lane == 0) {
    red.v[0][wid] = best;
    red.i[wid] = best_c;
    red.v[1][wid] = smax;
  }
  __syncthreads();
  best = red.v[0][0];
  best_c = red.i[0];
  float Ms = red.v[1][0];
  for (int w = 1; w < kDecideWaves; ++w) {
    argmax_pick(best, best_c, red.v[0][w], red.i[w]);
    Ms = fmaxf(Ms, red.v[1][w]);
  }
  __syncthreads();
  const float M = best;
  // pass 2: normalisers (all candidates; gold-text candidates); a thread reads back only
  // the sums it stored
  float z_part = 0.f, mg = -INFINITY;
#pragma unroll 4
  for (int c = c0 + tid; c < c1; c += kDecideThreads) {
    const float av = a.cand_s[c] / a.T;
    z_part += expf(av - M);
    if (have_text && a.cand_text_id[c] == gold) mg = fmaxf(mg, av);
  }
  z_part = wave_sum(z_part);
  mg = wave_max(mg);
  if (lane == 0) {
    red.v[0][wid] = z_part;
    red.v[1][wid] = mg;
  }
  __syncthreads();
  float Z = red.v[0][0], Mg = red.v[1][0];
  for (int w = 1; w < kDecideWaves; ++w) {
    Z += red.v[0][w];
    Mg = fmaxf(Mg, red.v[1][w]);
  }
  __syncthreads();
  if (!have_text) Mg = -INFINITY;
  int t_idx = a.q_true_idx ? t_given : (K == 2 ? 1 : -1);
  if (t_idx < -1 || t_idx >= K) {
    if (tid == 0) flag_or(a.flags, JET_FLAG_BAD_TRUE_IDX);
    t_idx = -1;
  }
  // pass 3: q, expectation, entropy, mass, gold sum
  float part[4] = {0.f, 0.f, 0.f, 0.f};  // e, h, mass, zg
#pragma unroll 4
  for (int c = c0 + tid; c < c1; c += kDecideThreads) {
    const float s = a.cand_s[c];
    const float av = s / a.T;
    const float qc = expf(av - M) / Z;
    a.cand_q[c] = qc;
    part[0] += (float)(c - c0) * qc;
    if (qc > 0.f) part[1] -= qc * logf(qc);
    part[2] += expf(s - Ms);
    if (have_text && a.cand_text_id[c] == gold && Mg != -INFINITY) part[3] += expf(av - Mg);
    if (a.q_true && c - c0 == t_idx) a.q_true[q] = qc;
  }
  block_sums<4>(part, red, lane, wid);
  if (tid == 0) {
    const float E = part[0], Hq = part[1], Zg = part[3];
    const float mass = Ms == -INFINITY ? 0.f : expf(Ms) * part[2];
    a.q_argmax[q] = best_c < c1 ? best_c - c0 : -1;
    if (a.q_true && t_idx < 0) a.q_true[q] = NaN;
    if (a.q_expect) a.q_expect[q] = E;
    if (a.q_nll) {
      float nll = NaN;
      if (have_text) nll = (Mg == -INFINITY) ? INFINITY : (M + logf(Z)) - (Mg + logf(Zg));
      a.q_nll[q] = nll;
    }
    if (a.q_conf) a.q_conf[q] = 1.f - Hq / logf((float)K);
    if (a.q_mass) a.q_mass[q] = mass;
  }
}

// Four questions per workgroup, one wave each (waves 0..3, one per SIMD).  BIG = false:
// 4-wave workgroups, every question on its wave.  BIG = true: 16-wave workgroups; a
// question with more than 64 candidates is set aside by its wave and then taken by all 16
// waves, in question order.
template <bool BIG>
__global__ __launch_bounds__(BIG ? kDecideThreads : 256) void k_decide(DecideArgs a) {
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int q = blockIdx.x * 4 + wid;
  // The ends of both offset arrays (a question's own checks see only its interior): with
  // these and every question's and candidate's checks passed, the candidates partition the
  // tokens and the questions partition the candidates, so every output is written.
  if (blockIdx.x == 0 && tid == 0 &&
      (a.q_cand_off[0] != 0 || a.q_cand_off[a.n_q] != a.n_cand || a.cand_tok_off[0] != 0 ||
       a.cand_tok_off[a.n_cand] != a.n_tok))
    flag_or(a.flags, JET_FLAG_BAD_OFFSETS);
  if constexpr (!BIG) {
    if (q < a.n_q) decide_question(a, q, lane);
  } else {
    __shared__ BlockRed red;
    __shared__ int s_big[4];  // question set aside by wave w, or -1
    if (wid < 4) {
      int big_q = -1;
      if (q < a.n_q) {
        const int c0 = a.q_cand_off[q], c1 = a.q_cand_off[q + 1];
        if (c0 >= 0 && c1 <= a.n_cand && c1 - c0 > 64)
          big_q = q;
        else
          decide_question(a, q, lane);
      }
      if (lane == 0) s_big[wid] = big_q;
    }
    __syncthreads();
#pragma unroll 1
    for (int w = 0; w < 4; ++w)
      if (s_big[w] >= 0) decide_question_block(a, s_big[w], red, tid);
  }
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
  // Every valid question has at least one candidate, so none has more than
  // n_cand - (n_q - 1).  Past 1,024 the 16-wave workgroups, which take any question of more
  // than 64 candidates together, are launched; below, one wave decides a question of up to
  // 1,024 candidates in about 20 us, and the 4-wave kernel saves the larger workgroups'
  // 0.3 us (measured on 32 questions of at most 24 candidates: 4.6-4.8 us against 5.0 us).
  const bool big = (long long)p->n_cand - (p->n_q - 1) > 1024;
  if (big)
    hipLaunchKernelGGL(k_decide<true>, dim3((p->n_q + 3) / 4), dim3(kDecideThreads), 0,
                       a.stream, decide_args(a));
  else
    hipLaunchKernelGGL(k_decide<false>, dim3((p->n_q + 3) / 4), dim3(256), 0, a.stream,
                       decide_args(a));
  return hipGetLastError();
}

}  // namespace jet
