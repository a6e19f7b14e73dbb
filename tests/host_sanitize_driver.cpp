// Host-code driver for the address/undefined-behaviour sanitizer build of the library.
//
// It calls every entry point that does its work on the host (index validation, union and
// trie building, workspace-size and plan queries, the argument checks of the device entry
// points) on random and extreme inputs, and checks the results against properties that
// hold for every input.  No call here reaches a kernel launch, so it runs without a GPU.
// Exit status 0 = every check held; the sanitizers abort on any memory error or undefined
// behaviour.
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <map>
#include <vector>

#include "../include/jet.h"

namespace {

int g_fail = 0;

#define CHECK(cond)                                                           \
  do {                                                                        \
    if (!(cond)) {                                                            \
      std::fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #cond); \
      ++g_fail;                                                               \
    }                                                                         \
  } while (0)

// xorshift64* (Vigna), for reproducible random structures
struct Rng {
  uint64_t s;
  explicit Rng(uint64_t seed) : s(seed * 0x9E3779B97F4A7C15ull + 1) {}
  uint64_t next() {
    s ^= s >> 12;
    s ^= s << 25;
    s ^= s >> 27;
    return s * 2685821657736338717ull;
  }
  int uniform(int lo, int hi) { return lo + (int)(next() % (uint64_t)(hi - lo + 1)); }
};

struct Problem {
  std::vector<int32_t> tok_row, tok_target, cand_off, q_off, true_idx, text, gold;
  int n_rows = 0, V = 0;
};

// questions of K candidates with lengths 1..max_len; rows: one per token
Problem random_problem(Rng& r, int n_q, int max_k, int max_len, int V) {
  Problem p;
  p.V = V;
  p.cand_off.push_back(0);
  p.q_off.push_back(0);
  for (int g = 0; g < n_q; ++g) {
    const int K = r.uniform(1, max_k);
    for (int c = 0; c < K; ++c) {
      const int m = r.uniform(1, max_len);
      for (int t = 0; t < m; ++t) {
        p.tok_row.push_back((int32_t)p.tok_row.size());
        p.tok_target.push_back(r.uniform(0, V - 1));
      }
      p.cand_off.push_back((int32_t)p.tok_row.size());
      p.text.push_back(r.uniform(0, 3));
    }
    p.q_off.push_back((int32_t)p.cand_off.size() - 1);
    p.true_idx.push_back(r.uniform(-1, K - 1));
    p.gold.push_back(r.uniform(0, 3));
  }
  p.n_rows = (int)p.tok_row.size();
  return p;
}

jet_problem view(const Problem& q, const void* dummy, int d) {
  jet_problem p;
  std::memset(&p, 0, sizeof(p));
  p.H = dummy;
  p.h_dtype = JET_F32;
  p.n_rows = q.n_rows;
  p.W = dummy;
  p.w_dtype = JET_BF16;
  p.V = q.V;
  p.d = d;
  p.tok_row = q.tok_row.data();
  p.tok_target = q.tok_target.data();
  p.n_tok = (int32_t)q.tok_row.size();
  p.cand_tok_off = q.cand_off.data();
  p.n_cand = (int32_t)q.cand_off.size() - 1;
  p.q_cand_off = q.q_off.data();
  p.n_q = (int32_t)q.q_off.size() - 1;
  p.cand_text_id = q.text.data();
  p.q_gold_text_id = q.gold.data();
  p.q_true_idx = q.true_idx.data();
  p.T = 1.0f;
  return p;
}

void test_validate_and_plan(Rng& r) {
  alignas(16) static float dummy[64];
  for (int it = 0; it < 200; ++it) {
    Problem q = random_problem(r, r.uniform(1, 12), 9, 6, r.uniform(1, 300000));
    const int d = 32 * r.uniform(1, 96);
    jet_problem p = view(q, dummy, d);
    CHECK(jet_validate_host(&p) == JET_OK);
    CHECK(jet_score_workspace_size(&p) > 0);
    CHECK(jet_projection_kernel(&p) != nullptr);
    // one corrupted index per kind must be found
    Problem b = q;
    b.tok_target[r.uniform(0, (int)b.tok_target.size() - 1)] = q.V;
    jet_problem pb = view(b, dummy, d);
    CHECK(jet_validate_host(&pb) != JET_OK);
    b = q;
    b.tok_row[r.uniform(0, (int)b.tok_row.size() - 1)] = -1;
    pb = view(b, dummy, d);
    CHECK(jet_validate_host(&pb) != JET_OK);
    b = q;
    if (b.cand_off.size() > 2) {
      const int c = r.uniform(1, (int)b.cand_off.size() - 2);
      b.cand_off[c] = b.cand_off[c - 1];  // an empty candidate
      pb = view(b, dummy, d);
      CHECK(jet_validate_host(&pb) != JET_OK);
    }
    b = q;
    b.true_idx[0] = 1 << 20;
    pb = view(b, dummy, d);
    CHECK(jet_validate_host(&pb) != JET_OK);
  }
  // extreme scalars: sizes near every limit, never a crash or overflow
  const int32_t Vs[] = {1, 255, 256, 257, 248320, 1 << 30, (1 << 30) + 1, -1, 0};
  const int32_t ds[] = {32, 96, 128, 2560, 65536, 65568, 31, 0, -32};
  const int32_t rows[] = {0, 1, 255, 256, 26624, 1 << 21, (1 << 21) + 1, -1};
  std::vector<int32_t> off2 = {0, 1}, one = {0};
  for (int32_t V : Vs)
    for (int32_t d : ds)
      for (int32_t nr : rows)
        for (int hd = 0; hd < 2; ++hd) {
          jet_problem p;
          std::memset(&p, 0, sizeof(p));
          p.H = dummy;
          p.W = dummy;
          p.h_dtype = hd ? JET_BF16 : JET_F32;
          p.w_dtype = JET_BF16;
          p.n_rows = nr;
          p.V = V;
          p.d = d;
          p.tok_target = one.data();
          p.n_tok = nr > 0 ? 1 : 0;
          p.cand_tok_off = off2.data();
          p.n_cand = p.n_tok;
          p.q_cand_off = off2.data();
          p.n_q = p.n_tok;
          p.T = 1.0f;
          const size_t ws = jet_score_workspace_size(&p);
          const char* name = jet_projection_kernel(&p);
          CHECK((ws == 0) == (name == nullptr));
          jet_restricted_problem rp;
          std::memset(&rp, 0, sizeof(rp));
          rp.H = dummy;
          rp.W = dummy;
          rp.h_dtype = p.h_dtype;
          rp.w_dtype = JET_BF16;
          rp.n_rows = nr;
          rp.V = V;
          rp.d = d;
          rp.union_ids = one.data();
          rp.n_union = V > 0 ? (V < 832 ? V : 832) : 0;
          rp.T = 2.0f;
          (void)jet_restricted_workspace_size(&rp);
        }
  for (int32_t n : {-5, 0, 1, 4096, 1 << 20, 1 << 30}) (void)jet_fit_temperature_workspace_size(n);
}

void test_union(Rng& r) {
  for (int it = 0; it < 300; ++it) {
    const int n_f = r.uniform(0, 40), V = r.uniform(1, 5000);
    std::vector<int32_t> ids, off = {0};
    for (int f = 0; f < n_f; ++f) {
      const int K = r.uniform(1, 26);
      for (int k = 0; k < K; ++k) ids.push_back(r.uniform(0, V - 1));  // repeats allowed
      off.push_back((int32_t)ids.size());
    }
    const int n = (int)ids.size();
    std::vector<int32_t> uni(n + 1, -7), slot(n + 1, -7);
    int32_t n_union = -1;
    CHECK(jet_build_union(ids.data(), off.data(), n_f, V, uni.data(), &n_union, slot.data()) == JET_OK);
    CHECK(n_union >= 0 && n_union <= n);
    for (int j = 1; j < n_union; ++j) CHECK(uni[j - 1] < uni[j]);
    for (int j = 0; j < n; ++j) CHECK(slot[j] >= 0 && slot[j] < n_union && uni[slot[j]] == ids[j]);
    CHECK(uni[n] == -7 && slot[n] == -7);  // nothing written past the end
    if (n > 0) {
      std::vector<int32_t> bad = ids;
      bad[r.uniform(0, n - 1)] = r.uniform(0, 1) ? V : -1;
      CHECK(jet_build_union(bad.data(), off.data(), n_f, V, uni.data(), &n_union, slot.data()) == JET_E_INDEX);
    }
  }
  int32_t n_union = 0, x = 0;
  CHECK(jet_build_union(nullptr, nullptr, 1, 10, &x, &n_union, &x) != JET_OK);
}

void test_trie(Rng& r) {
  for (int it = 0; it < 300; ++it) {
    // small vocabularies so that histories repeat
    Problem q = random_problem(r, r.uniform(1, 8), 12, 5, r.uniform(1, 4));
    const int n_tok = (int)q.tok_target.size();
    const int n_cand = (int)q.cand_off.size() - 1, n_q = (int)q.q_off.size() - 1;
    std::vector<int32_t> tok_node(n_tok + 1, -7), node_tok(n_tok + 1, -7);
    int32_t n_nodes = -1;
    CHECK(jet_build_predictor_trie(q.tok_target.data(), q.cand_off.data(), n_cand, q.q_off.data(), n_q,
                                   tok_node.data(), node_tok.data(), &n_nodes) == JET_OK);
    CHECK(n_nodes >= 1 && n_nodes <= n_tok);
    CHECK(tok_node[n_tok] == -7 && node_tok[n_tok] == -7);
    // two tokens share a node exactly when they have the same question and history
    std::vector<int> qof(n_tok), pos(n_tok);
    std::vector<const int32_t*> start(n_tok);
    for (int g = 0; g < n_q; ++g)
      for (int c = q.q_off[g]; c < q.q_off[g + 1]; ++c)
        for (int k = q.cand_off[c]; k < q.cand_off[c + 1]; ++k) {
          qof[k] = g;
          pos[k] = k - q.cand_off[c];
          start[k] = q.tok_target.data() + q.cand_off[c];
        }
    for (int a = 0; a < n_tok; ++a) {
      CHECK(tok_node[a] >= 0 && tok_node[a] < n_nodes);
      for (int b = a + 1; b < n_tok && b < a + 64; ++b) {
        const bool same = qof[a] == qof[b] && pos[a] == pos[b] &&
                          std::memcmp(start[a], start[b], sizeof(int32_t) * pos[a]) == 0;
        CHECK(same == (tok_node[a] == tok_node[b]));
      }
    }
    for (int j = 0; j < n_nodes; ++j) CHECK(tok_node[node_tok[j]] == j);
  }
  int32_t n_nodes = 0;
  std::vector<int32_t> off = {0, 1}, t = {0}, tn(1), nt(1);
  CHECK(jet_build_predictor_trie(t.data(), off.data(), -1, off.data(), 1, tn.data(), nt.data(), &n_nodes) == JET_E_SHAPE);
  CHECK(jet_build_predictor_trie(nullptr, off.data(), 1, off.data(), 1, tn.data(), nt.data(), &n_nodes) == JET_E_NULL);
  std::vector<int32_t> neg = {-3};
  CHECK(jet_build_predictor_trie(neg.data(), off.data(), 1, off.data(), 1, tn.data(), nt.data(), &n_nodes) == JET_E_INDEX);
}

void test_restricted_validation(Rng& r) {
  alignas(16) static float dummy[64];
  for (int it = 0; it < 200; ++it) {
    const int n_f = r.uniform(1, 32), V = r.uniform(30, 248320);
    std::vector<int32_t> ids, off = {0}, frow;
    for (int f = 0; f < n_f; ++f) {
      const int K = r.uniform(1, 26);
      for (int k = 0; k < K; ++k) ids.push_back(r.uniform(0, V - 1));
      off.push_back((int32_t)ids.size());
      frow.push_back(f);
    }
    std::vector<int32_t> uni(ids.size()), slot(ids.size());
    int32_t n_union = 0;
    CHECK(jet_build_union(ids.data(), off.data(), n_f, V, uni.data(), &n_union, slot.data()) == JET_OK);
    jet_restricted_problem p;
    std::memset(&p, 0, sizeof(p));
    p.H = dummy;
    p.W = dummy;
    p.h_dtype = JET_F32;
    p.w_dtype = JET_BF16;
    p.n_rows = n_f;
    p.V = V;
    p.d = 32 * r.uniform(1, 80);
    p.union_ids = uni.data();
    p.n_union = n_union;
    p.field_row = frow.data();
    p.field_slot_off = off.data();
    p.slot_uidx = slot.data();
    p.n_fields = n_f;
    p.n_slots = (int32_t)ids.size();
    p.T = 2.0f;
    CHECK(jet_validate_restricted_host(&p) == JET_OK);
    CHECK(jet_restricted_workspace_size(&p) > 0);
    std::vector<int32_t> s2 = slot;
    s2[r.uniform(0, (int)s2.size() - 1)] = n_union;
    p.slot_uidx = s2.data();
    CHECK(jet_validate_restricted_host(&p) == JET_E_INDEX);
    p.slot_uidx = slot.data();
    std::vector<int32_t> f2 = frow;
    f2[r.uniform(0, n_f - 1)] = n_f;
    p.field_row = f2.data();
    CHECK(jet_validate_restricted_host(&p) == JET_E_INDEX);
  }
}

void test_argument_checks() {
  // every device entry point rejects bad scalars and pointers before enqueuing anything
  alignas(16) static float buf[64];
  CHECK(jet_score(nullptr, nullptr, nullptr, 0, nullptr) == JET_E_NULL);
  CHECK(jet_score_restricted(nullptr, nullptr, nullptr, 0, nullptr) == JET_E_NULL);
  CHECK(jet_stream_read(nullptr, 16, nullptr, nullptr) == JET_E_NULL);
  CHECK(jet_stream_read(buf, 15, reinterpret_cast<uint32_t*>(buf), nullptr) == JET_E_SHAPE);
  CHECK(jet_stream_read(reinterpret_cast<char*>(buf) + 4, 16, reinterpret_cast<uint32_t*>(buf), nullptr) == JET_E_SHAPE);
  CHECK(jet_stream_read(buf, 0, reinterpret_cast<uint32_t*>(buf), nullptr) == JET_OK);
  std::vector<int32_t> off = {0, 2};
  CHECK(jet_decision_sensitivity(buf, buf, off.data(), 1, 2, 0, 1e-8f, 0, buf, buf, nullptr, nullptr, nullptr) == JET_E_SHAPE);
  int32_t* sel = reinterpret_cast<int32_t*>(buf);
  CHECK(jet_decision_sensitivity(buf, buf, off.data(), 1, 2, 3, 1e-8f, 4, buf, buf, sel, nullptr, nullptr) == JET_E_SHAPE);
  CHECK(jet_decision_sensitivity(buf, buf, off.data(), 1, 2, 3, NAN, 1, buf, buf, sel, nullptr, nullptr) == JET_E_SHAPE);
  CHECK(jet_decision_sensitivity(buf, buf, off.data(), 1, 2, 3, 1e-8f, 1, buf, buf, nullptr, nullptr, nullptr) == JET_E_NULL);
  float T = 0.f, nll = 0.f;
  const int32_t* ib = reinterpret_cast<const int32_t*>(buf);
  CHECK(jet_fit_temperature(buf, off.data(), 1, 2, ib, ib, 2.0f, 1.0f, &T, &nll, nullptr, buf, 1 << 20, nullptr) == JET_E_TEMP);
  CHECK(jet_fit_temperature(buf, off.data(), 1, 2, nullptr, ib, 0.5f, 2.0f, &T, &nll, nullptr, buf, 1 << 20, nullptr) == JET_E_NULL);
  CHECK(jet_fit_temperature(buf, off.data(), 0, 2, ib, ib, 0.5f, 2.0f, &T, &nll, nullptr, buf, 1 << 20, nullptr) == JET_E_SHAPE);
  jet_problem p;
  std::memset(&p, 0, sizeof(p));
  p.H = buf;
  p.W = buf;
  p.w_dtype = JET_F32;
  p.h_dtype = JET_BF16;  // unsupported combination
  p.V = 10;
  p.d = 32;
  p.T = 1.0f;
  CHECK(jet_score_workspace_size(&p) == 0);
  jet_outputs o;
  std::memset(&o, 0, sizeof(o));
  CHECK(jet_score(&p, &o, buf, sizeof(buf), nullptr) == JET_E_DTYPE);
  int32_t bogus = 7;  // a dtype value no enumerator names, as a C or Python caller may pass
  std::memcpy(&p.h_dtype, &bogus, sizeof(bogus));
  CHECK(jet_score_workspace_size(&p) == 0);
  CHECK(jet_score(&p, &o, buf, sizeof(buf), nullptr) == JET_E_DTYPE);
  p.h_dtype = JET_F32;
  p.T = -1.0f;
  CHECK(jet_score(&p, &o, buf, sizeof(buf), nullptr) == JET_E_TEMP);
  for (int s = -10; s <= 1; ++s) CHECK(jet_status_string((jet_status)s) != nullptr);
}

}  // namespace

int main() {
  Rng r(20241202);
  test_validate_and_plan(r);
  test_union(r);
  test_trie(r);
  test_restricted_validation(r);
  test_argument_checks();
  if (g_fail) {
    std::fprintf(stderr, "%d checks failed\n", g_fail);
    return 1;
  }
  std::printf("host driver: all checks passed\n");
  return 0;
}
