// C ABI of libjet: host-side validation, execution planning and launch sequencing.
// Every check here runs on the host before anything is enqueued, so a call rejected by a
// check enqueues nothing.  JET_E_HIP alone comes after enqueueing may have begun: it
// reports a failed launch or event record, and the launches before it stay enqueued.  The
// device kernels bounds-check every index themselves.
#include <algorithm>
#include <cmath>
#include <mutex>
#include <unordered_map>
#include <vector>

#include "jet_internal.h"

// Workspace of jet_score_noalloc: static device memory, one copy per GPU the library runs
// on, held until the process ends.  Host code never passes this name to a kernel (on the
// host it is only a stand-in for the symbol); it uses the device address that
// hipGetSymbolAddress returns for the current device.
static constexpr size_t kNoallocScratchBytes = JET_NOALLOC_MAX_WORKSPACE;
static __device__ __align__(256) unsigned char scratch[kNoallocScratchBytes];

namespace jet {

int small_group_size(int variant, bool stream);
int small_grid(int variant, bool stream, int n_groups, int max_waves);

namespace {

constexpr int kMaxD = 65536;
constexpr int kMaxV = 1 << 30;
#ifndef JET_SMALL_WAVES
#define JET_SMALL_WAVES 2048  // 256 CUs x 8 resident waves
#endif
constexpr int kSmallWaves = JET_SMALL_WAVES;
// Rows the streaming kernel takes in one pass over the head: its workgroups carry up to 2
// (fp32 H, split into two planes) or 4 (bf16 H) 32-row tiles of H, as many as the LDS
// holds.  Past that the tiled (matrix-core) kernel takes the problem, and also past one
// 32-row tile when d rules the streaming kernel out (the fallback reads the whole head once
// per 32-row tile).  Measured at V = 248,320, d = 2560: the streaming kernel with one row
// tile per workgroup 194 us per 32-row tile (1.48 ms at 255 rows), one tiled row tile about
// 350 us.
int stream_max_row_tiles(bool hilo) { return hilo ? 2 : 4; }

// fp32 head: the streaming kernel k_project_wg_f32 when it has at least one workgroup per
// CU (256-entry vocabulary groups x row tiles of 16 rows up to 16 rows, else 32); smaller
// problems take k_project_small_f32, whose 32-entry groups and k split over four waves
// spread them over more CUs.  Measured with 8 rows: the streaming kernel 8.2 -> 13.3 us at
// V = 4096, d = 256 and 23 -> 40 us at V = 16,384, d = 1024 (16 and 64 groups), level at
// 128 groups, 26 -> 20 us at V = 65,536, d = 256 (256 groups); 109 us against 164 us at
// V = 128,000, d = 1024 with 4 rows.
constexpr long long kF32StreamMinWork = 256;
bool f32_streams(int V, int n_rows) {
  if (!JET_F32_STREAM) return false;
  const long long groups = (V + 255) / 256;
  const long long tiles = n_rows <= 16 ? 1 : (n_rows + 31) / 32;
  return groups * tiles >= kF32StreamMinWork;
}

size_t al256(size_t x) { return (x + 255) & ~(size_t)255; }

bool aligned16(const void* ptr) { return ((uintptr_t)ptr & 15u) == 0; }

jet_status check_dims(jet_dtype h_dtype, jet_dtype w_dtype, int n_rows, int V, int d,
                      const void* H, const void* W, float T) {
  if (!(w_dtype == JET_BF16 && (h_dtype == JET_BF16 || h_dtype == JET_F32)) &&
      !(w_dtype == JET_F32 && h_dtype == JET_F32))
    return JET_E_DTYPE;
  if (n_rows < 0 || V < 1 || V > kMaxV || d < 32 || d > kMaxD || d % 32 != 0) return JET_E_SHAPE;
  if (!W || (n_rows > 0 && !H)) return JET_E_NULL;
  if (!aligned16(W) || !aligned16(H)) return JET_E_SHAPE;
  if (!std::isfinite(T) || !(T > 0.f)) return JET_E_TEMP;
  return JET_OK;
}

jet_status check_problem(const jet_problem* p) {
  if (!p) return JET_E_NULL;
  jet_status st = check_dims(p->h_dtype, p->w_dtype, p->n_rows, p->V, p->d, p->H, p->W, p->T);
  if (st != JET_OK) return st;
  if (p->n_tok < 0 || p->n_cand < 0 || p->n_q < 0) return JET_E_SHAPE;
  if (p->n_cand < p->n_q || p->n_tok < p->n_cand) return JET_E_SHAPE;  // K >= 1, m_c >= 1
  // the offset arrays end at n_cand and n_tok: no candidates without questions, no tokens
  // without candidates
  if ((p->n_q == 0 && p->n_cand > 0) || (p->n_cand == 0 && p->n_tok > 0)) return JET_E_SHAPE;
  if (p->n_tok > 0 && p->n_rows == 0) return JET_E_SHAPE;
  if (!p->tok_row && p->n_tok > p->n_rows) return JET_E_SHAPE;
  if (p->n_rows > (1 << 21)) return JET_E_SHAPE;
  if (p->n_tok > 0 && !p->tok_target) return JET_E_NULL;
  if (p->n_cand > 0 && !p->cand_tok_off) return JET_E_NULL;
  if (p->n_q > 0 && !p->q_cand_off) return JET_E_NULL;
  return JET_OK;
}

jet_status check_outputs(const jet_problem* p, const jet_outputs* o) {
  if (!o) return JET_E_NULL;
  if (p->n_tok > 0 && !o->tok_logp) return JET_E_NULL;
  if (p->n_cand > 0 && (!o->cand_s || !o->cand_q)) return JET_E_NULL;
  if (p->n_q > 0 && !o->q_argmax) return JET_E_NULL;
  return JET_OK;
}

}  // namespace

void make_plan(const jet_problem* p, Plan* pl) {
  *pl = Plan{};
  pl->variant = p->w_dtype == JET_F32 ? VAR_SMALL_F32 : VAR_SMALL_BF16;
  pl->hilo = p->w_dtype == JET_BF16 && p->h_dtype == JET_F32;
  // tiled path: enough rows, whole stages, at least one full vocabulary tile (its buffer
  // offsets are local to a workgroup's tiles, so operands of any size take it); fewer rows
  // than one row tile run as one tile with zero rows appended to H
  const bool streams = pl->variant == VAR_SMALL_BF16 && stream_d(p->d);
  const int one_pass_rows = streams ? 32 * stream_max_row_tiles(pl->hilo) : 32;
  if (pl->variant == VAR_SMALL_BF16 && p->n_rows > one_pass_rows && p->V >= 256 &&
      p->d % tiled_bk(pl->hilo) == 0)
    pl->variant = VAR_TILED_BF16;
  pl->rows_k = p->n_rows;
  pl->stream = (pl->variant == VAR_SMALL_BF16 && stream_d(p->d)) ||
               (pl->variant == VAR_SMALL_F32 && f32_streams(p->V, p->n_rows));
  if (pl->variant == VAR_TILED_BF16) {
    pl->row_tile = tiled_row_tile(pl->hilo, p->d);
    pl->rows_k = std::max(p->n_rows, pl->row_tile);
    pl->pad_h = !pl->hilo && p->n_rows < pl->row_tile;  // fp32 H: its split planes are padded
    pl->n_rtiles = (pl->rows_k + pl->row_tile - 1) / pl->row_tile;
    pl->vgroup = 256;
    pl->n_vgroups = (p->V + 255) / 256;
    // Split count S (vocabulary ranges per row tile).  Every workgroup takes the same
    // number L of consecutive vocabulary tiles (the last range of a row tile may be shorter
    // or empty), 4 when there is work for many workgroups: workgroups of equal length
    // finish together, so each XCD's next 32 again form one block sharing its L2,
    // and short ones keep the eight XCDs on nearby head tiles.  (Measured on both tiled
    // kernels: runs of 4 tiles 1-3% faster than 8, 6-10% faster than balanced ranges of
    // unequal length; single tiles 2-3% slower.)  With less work than 4 tiles per CU, the
    // fewest tiles per workgroup that still fit every workgroup into one round on the 256
    // CUs.  S is rounded up to a multiple of 8 (XCD-aware placement, which needs at least 2
    // row tiles) when that adds few empty ranges.
    const int R = pl->n_rtiles, nvt = pl->n_vgroups;
    const long long work = (long long)R * nvt;
    int L = (int)std::min<long long>(4, std::max<long long>(1, (work + 255) / 256));
    L = std::min(L, nvt);
    int splits = (nvt + L - 1) / L;
    if (splits >= 32 && R >= 2) splits = (splits + 7) / 8 * 8;
    pl->grid_x = splits;
  } else {
    // streaming kernel: the fewest row tiles per workgroup (1, 2, 4) that cover the rows,
    // up to the LDS limit (more rows only with a vocabulary below one tiled tile)
    int nr = 1;
    if (pl->stream && pl->variant == VAR_SMALL_BF16)
      while (nr < stream_max_row_tiles(pl->hilo) && 32 * nr < p->n_rows) nr *= 2;
    pl->stream_nr = nr;
    pl->row_tile = 32 * nr;
    // fp32 head: up to 16 rows take the 16-row tile (half the matrix work of a 32-row one)
    if (pl->stream && pl->variant == VAR_SMALL_F32 && p->n_rows <= 16) pl->row_tile = 16;
    pl->n_rtiles = (p->n_rows + pl->row_tile - 1) / pl->row_tile;
    pl->vgroup = small_group_size(pl->variant, pl->stream);
    pl->n_vgroups = (p->V + pl->vgroup - 1) / pl->vgroup;
    pl->grid_x = std::max(1, small_grid(pl->variant, pl->stream, pl->n_vgroups, kSmallWaves));
  }
  pl->n_parts = pl->grid_x;
  // no target logit is captured by a projection kernel (k_token_logp computes them after
  // it), so the workspace holds operands, partials and the flag word only
  size_t off = 0;
  const size_t rows_k = (size_t)pl->rows_k, d = (size_t)p->d;
  const bool split_buffers = pl->hilo && !pl->stream;
  pl->off_hhi = off;
  if (split_buffers) off += al256(rows_k * d * 2);
  pl->off_hlo = off;
  if (split_buffers) off += al256(rows_k * d * 2);
  pl->off_hpad = off;
  if (pl->pad_h) off += al256(rows_k * d * 2);
  pl->off_part = off;
  off += al256((size_t)pl->n_parts * rows_k * 8);
  pl->off_flags = off;
  off += 256;
  pl->total = off;
}

}  // namespace jet

using namespace jet;

extern "C" {

const char* jet_status_string(jet_status s) {
  switch (s) {
    case JET_OK: return "ok";
    case JET_E_NULL: return "a required pointer is NULL";
    case JET_E_SHAPE: return "a size is out of range or an operand is misaligned";
    case JET_E_DTYPE: return "unsupported operand type combination";
    case JET_E_INDEX: return "an index is out of range or offsets are malformed";
    case JET_E_TEMP: return "temperature must be finite and > 0";
    case JET_E_WORKSPACE: return "workspace is NULL, too small or not 256-byte aligned";
    case JET_E_HIP: return "a HIP runtime call failed";
  }
  return "unknown status";
}

jet_status jet_decision_sensitivity(const float* z, const float* z_skip, const int32_t* seg_off,
                                    int32_t n_inputs, int32_t n_values, int32_t n_layers,
                                    float eps, int32_t k, float* d, float* J, int32_t* selected,
                                    int32_t* dev_flags, void* stream) {
  if (!z || !z_skip || !seg_off || !d || !J || (k > 0 && !selected)) return JET_E_NULL;
  if (n_inputs < 1 || n_values < 1 || n_layers < 1 || n_layers > sensitivity_max_layers() ||
      k < 0 || k > n_layers || !std::isfinite(eps) || !(eps > 0.f))
    return JET_E_SHAPE;
  const hipError_t e = launch_sensitivity(z, z_skip, seg_off, n_inputs, n_values, n_layers, eps,
                                          k, d, J, selected, dev_flags,
                                          static_cast<hipStream_t>(stream));
  return e == hipSuccess ? JET_OK : JET_E_HIP;
}

size_t jet_fit_temperature_workspace_size(int32_t n_q) {
  return n_q < 1 ? 0 : fit_temperature_workspace(n_q);
}

jet_status jet_fit_temperature(const float* cand_s, const int32_t* q_cand_off, int32_t n_q,
                               int32_t n_cand, const int32_t* cand_text_id,
                               const int32_t* q_gold_text_id, float T_min, float T_max,
                               float* T_fit, float* nll_fit, int32_t* dev_flags, void* workspace,
                               size_t workspace_bytes, void* stream) {
  if (!cand_s || !q_cand_off || !cand_text_id || !q_gold_text_id || !T_fit || !nll_fit)
    return JET_E_NULL;
  if (n_q < 1 || n_cand < 1) return JET_E_SHAPE;
  if (!std::isfinite(T_min) || !std::isfinite(T_max) || !(T_min > 0.f) || !(T_max > T_min))
    return JET_E_TEMP;
  if (!workspace || workspace_bytes < fit_temperature_workspace(n_q) ||
      ((uintptr_t)workspace & 255u))
    return JET_E_WORKSPACE;
  const hipError_t e = launch_fit_temperature(cand_s, q_cand_off, n_q, n_cand, cand_text_id,
                                              q_gold_text_id, T_min, T_max, T_fit, nll_fit,
                                              dev_flags, static_cast<char*>(workspace),
                                              static_cast<hipStream_t>(stream));
  return e == hipSuccess ? JET_OK : JET_E_HIP;
}

jet_status jet_build_predictor_trie(const int32_t* tok_target, const int32_t* cand_tok_off,
                                    int32_t n_cand, const int32_t* q_cand_off, int32_t n_q,
                                    int32_t* tok_node, int32_t* node_tok, int32_t* n_nodes) {
  if (!cand_tok_off || !q_cand_off || !n_nodes) return JET_E_NULL;
  if (n_cand < 0 || n_q < 0) return JET_E_SHAPE;
  if (cand_tok_off[0] != 0 || q_cand_off[0] != 0 || q_cand_off[n_q] != n_cand) return JET_E_SHAPE;
  for (int32_t g = 0; g < n_q; ++g)
    if (q_cand_off[g + 1] <= q_cand_off[g]) return JET_E_SHAPE;
  for (int32_t c = 0; c < n_cand; ++c)
    if (cand_tok_off[c + 1] <= cand_tok_off[c]) return JET_E_SHAPE;
  const int32_t n_tok = cand_tok_off[n_cand];
  if (n_tok > 0 && (!tok_target || !tok_node || !node_tok)) return JET_E_NULL;
  for (int32_t k = 0; k < n_tok; ++k)
    if (tok_target[k] < 0) return JET_E_INDEX;
  // tree nodes in creation order; number[v] = predictor index of tree node v, or -1
  std::vector<int32_t> number;
  number.reserve((size_t)n_tok + n_q);
  std::unordered_map<uint64_t, int32_t> child;
  child.reserve((size_t)n_tok * 2 + 1);
  int32_t nn = 0;
  for (int32_t g = 0; g < n_q; ++g) {
    const int32_t root = (int32_t)number.size();
    number.push_back(-1);
    for (int32_t c = q_cand_off[g]; c < q_cand_off[g + 1]; ++c) {
      int32_t v = root;
      for (int32_t k = cand_tok_off[c]; k < cand_tok_off[c + 1]; ++k) {
        if (number[v] < 0) {
          number[v] = nn;
          node_tok[nn++] = k;
        }
        tok_node[k] = number[v];
        const uint64_t key = ((uint64_t)(uint32_t)v << 32) | (uint32_t)tok_target[k];
        auto it = child.find(key);
        if (it == child.end()) {
          it = child.emplace(key, (int32_t)number.size()).first;
          number.push_back(-1);
        }
        v = it->second;
      }
    }
  }
  *n_nodes = nn;
  return JET_OK;
}

const char* jet_projection_kernel(const jet_problem* p) {
  if (check_problem(p) != JET_OK) return nullptr;
  Plan pl;
  make_plan(p, &pl);
  switch (pl.variant) {
    case VAR_TILED_BF16: return tiled_kernel_name(pl.hilo, p->d);
    case VAR_SMALL_F32: return pl.stream ? "k_project_wg_f32" : "k_project_small_f32";
    default: return pl.stream ? "k_project_wg_bf16" : "k_project_small_bf16";
  }
}

size_t jet_score_workspace_size(const jet_problem* p) {
  if (check_problem(p) != JET_OK) return 0;
  Plan pl;
  make_plan(p, &pl);
  return pl.total;
}

jet_status jet_score_profiled(const jet_problem* p, const jet_outputs* o, void* workspace,
                              size_t workspace_bytes, void* stream, void* ev_before,
                              void* ev_after) {
  jet_status st = check_problem(p);
  if (st != JET_OK) return st;
  if ((st = check_outputs(p, o)) != JET_OK) return st;
  Plan pl;
  make_plan(p, &pl);
  if (!workspace || workspace_bytes < pl.total || ((uintptr_t)workspace & 255u)) return JET_E_WORKSPACE;
  char* ws = static_cast<char*>(workspace);
  ScoreArgs a;
  a.p = p;
  a.o = o;
  a.plan = &pl;
  a.ws = ws;
  a.flags = o->dev_flags ? o->dev_flags : reinterpret_cast<int32_t*>(ws + pl.off_flags);
  a.stream = static_cast<hipStream_t>(stream);
  // operand staging (fp32 H split into planes, zero-padded H; none for most plans), the
  // projection (its first workgroup clears the flag word), token log-probabilities with the
  // row merges (also the flag word's clear when there are no rows), decisions
  if (launch_prep(a) != hipSuccess) return JET_E_HIP;
  if (ev_before && hipEventRecord(static_cast<hipEvent_t>(ev_before), a.stream) != hipSuccess)
    return JET_E_HIP;
  if (p->n_rows > 0 && launch_project(a) != hipSuccess) return JET_E_HIP;
  if (ev_after && hipEventRecord(static_cast<hipEvent_t>(ev_after), a.stream) != hipSuccess)
    return JET_E_HIP;
  if (launch_token_logp(a) != hipSuccess) return JET_E_HIP;
  if (launch_decide(a) != hipSuccess) return JET_E_HIP;
  return JET_OK;
}

jet_status jet_score(const jet_problem* p, const jet_outputs* o, void* workspace,
                     size_t workspace_bytes, void* stream) {
  return jet_score_profiled(p, o, workspace, workspace_bytes, stream, nullptr, nullptr);
}

}  // extern "C"

namespace {
constexpr int kNoallocMaxDevices = 256;
std::mutex g_scratch_mu;
void* g_scratch_dev[kNoallocMaxDevices];  // device address of scratch, per device ordinal

// Device address of the static scratch array on the current device, looked up once per
// device (with that device current) and kept; NULL if the lookup fails.
void* scratch_on_current_device() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kNoallocMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_dev[dev]) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess) return nullptr;
    g_scratch_dev[dev] = ptr;
  }
  return g_scratch_dev[dev];
}
}  // namespace

extern "C" {

jet_status jet_score_noalloc(const jet_problem* p, const jet_outputs* o, void* stream) {
  jet_status st = check_problem(p);
  if (st != JET_OK) return st;
  if ((st = check_outputs(p, o)) != JET_OK) return st;
  Plan pl;
  make_plan(p, &pl);
  if (pl.total > kNoallocScratchBytes) return JET_E_WORKSPACE;
  void* ws = scratch_on_current_device();
  if (!ws) return JET_E_HIP;
  return jet_score_profiled(p, o, ws, kNoallocScratchBytes, stream, nullptr, nullptr);
}

jet_status jet_validate_host(const jet_problem* p) {
  jet_status st = check_problem(p);
  if (st != JET_OK) return st;
  for (int k = 0; k < p->n_tok; ++k) {
    const int r = p->tok_row ? p->tok_row[k] : k;
    if (r < 0 || r >= p->n_rows) return JET_E_INDEX;
    if (p->tok_target[k] < 0 || p->tok_target[k] >= p->V) return JET_E_INDEX;
  }
  if (p->n_cand > 0) {
    if (p->cand_tok_off[0] != 0 || p->cand_tok_off[p->n_cand] != p->n_tok) return JET_E_INDEX;
    for (int c = 0; c < p->n_cand; ++c)
      if (p->cand_tok_off[c + 1] <= p->cand_tok_off[c]) return JET_E_INDEX;
  }
  if (p->n_q > 0) {
    if (p->q_cand_off[0] != 0 || p->q_cand_off[p->n_q] != p->n_cand) return JET_E_INDEX;
    for (int g = 0; g < p->n_q; ++g) {
      const int K = p->q_cand_off[g + 1] - p->q_cand_off[g];
      if (K < 1) return JET_E_INDEX;
      if (p->q_true_idx && (p->q_true_idx[g] < -1 || p->q_true_idx[g] >= K)) return JET_E_INDEX;
    }
  } else if (p->n_cand != 0) {
    return JET_E_INDEX;
  }
  return JET_OK;
}

jet_status jet_build_union(const int32_t* field_ids, const int32_t* field_off, int32_t n_fields,
                           int32_t V, int32_t* union_ids, int32_t* n_union, int32_t* slot_uidx) {
  if (!field_off || !n_union) return JET_E_NULL;
  if (n_fields < 0 || V < 1) return JET_E_SHAPE;
  if (field_off[0] != 0) return JET_E_INDEX;
  for (int f = 0; f < n_fields; ++f)
    if (field_off[f + 1] <= field_off[f]) return JET_E_INDEX;
  const int n_slots = field_off[n_fields];
  if (n_slots > 0 && (!field_ids || !union_ids || !slot_uidx)) return JET_E_NULL;
  std::vector<int32_t> u(field_ids, field_ids + n_slots);
  for (int32_t x : u)
    if (x < 0 || x >= V) return JET_E_INDEX;
  std::sort(u.begin(), u.end());
  u.erase(std::unique(u.begin(), u.end()), u.end());
  for (int j = 0; j < n_slots; ++j)
    slot_uidx[j] = (int32_t)(std::lower_bound(u.begin(), u.end(), field_ids[j]) - u.begin());
  std::copy(u.begin(), u.end(), union_ids);
  *n_union = (int32_t)u.size();
  return JET_OK;
}

static jet_status check_restricted(const jet_restricted_problem* p) {
  if (!p) return JET_E_NULL;
  jet_status st = check_dims(p->h_dtype, p->w_dtype, p->n_rows, p->V, p->d, p->H, p->W, p->T);
  if (st != JET_OK) return st;
  if (p->n_union < 0 || p->n_fields < 0 || p->n_slots < p->n_fields) return JET_E_SHAPE;
  if (p->n_fields == 0 && p->n_slots > 0) return JET_E_SHAPE;  // slots outside every field
  if (p->n_fields > 0 && (p->n_union < 1 || p->n_rows < 1)) return JET_E_SHAPE;
  if (p->n_union > p->V) return JET_E_SHAPE;
  if (p->n_rows > (1 << 21)) return JET_E_SHAPE;
  if (p->n_union > 0 && !p->union_ids) return JET_E_NULL;
  if (p->n_fields > 0 && (!p->field_row || !p->field_slot_off || !p->slot_uidx)) return JET_E_NULL;
  return JET_OK;
}

size_t jet_restricted_workspace_size(const jet_restricted_problem* p) {
  if (check_restricted(p) != JET_OK) return 0;
  RestrictedPlan pl;
  make_restricted_plan(p, &pl);
  return pl.total;
}

jet_status jet_score_restricted(const jet_restricted_problem* p, const jet_restricted_outputs* o,
                                void* workspace, size_t workspace_bytes, void* stream) {
  jet_status st = check_restricted(p);
  if (st != JET_OK) return st;
  if (!o) return JET_E_NULL;
  if (p->n_fields > 0 && (!o->slot_logit || !o->slot_q || !o->field_argmax)) return JET_E_NULL;
  RestrictedPlan pl;
  make_restricted_plan(p, &pl);
  if (!workspace || workspace_bytes < pl.total || ((uintptr_t)workspace & 255u)) return JET_E_WORKSPACE;
  char* ws = static_cast<char*>(workspace);
  int32_t* flags = o->dev_flags ? o->dev_flags : reinterpret_cast<int32_t*>(ws + pl.off_flags);
  if (launch_restricted(p, o, &pl, ws, flags, static_cast<hipStream_t>(stream)) != hipSuccess)
    return JET_E_HIP;
  return JET_OK;
}

jet_status jet_validate_restricted_host(const jet_restricted_problem* p) {
  jet_status st = check_restricted(p);
  if (st != JET_OK) return st;
  for (int j = 0; j < p->n_union; ++j) {
    if (p->union_ids[j] < 0 || p->union_ids[j] >= p->V) return JET_E_INDEX;
    if (j > 0 && p->union_ids[j] <= p->union_ids[j - 1]) return JET_E_INDEX;
  }
  if (p->n_fields > 0) {
    if (p->field_slot_off[0] != 0 || p->field_slot_off[p->n_fields] != p->n_slots) return JET_E_INDEX;
    for (int f = 0; f < p->n_fields; ++f) {
      if (p->field_slot_off[f + 1] <= p->field_slot_off[f]) return JET_E_INDEX;
      if (p->field_row[f] < 0 || p->field_row[f] >= p->n_rows) return JET_E_INDEX;
    }
    for (int j = 0; j < p->n_slots; ++j)
      if (p->slot_uidx[j] < 0 || p->slot_uidx[j] >= p->n_union) return JET_E_INDEX;
  }
  return JET_OK;
}

}  // extern "C"
