/*
 * jet.h - C ABI of the MI355X (gfx950) candidate-likelihood scoring library.
 *
 * The library implements the readout of teacher-forced candidate scoring:
 *
 *   z[r, v]  = <H[r, :], W[v, :]>                 LM-head projection of predictor row r
 *   LSE_r    = log sum_{v < V} exp z[r, v]          full-vocabulary normaliser
 *   l_k      = z[row_k, y_k] - LSE_{row_k}          token log-probability
 *   s(c)     = sum of l_k over the candidate's tokens (chain rule, no length normalisation)
 *   q(c)     = softmax over the question's candidates of s(c) / T
 *   argmax   lowest candidate index among the maxima of s / T
 *   q(true), E = sum_i i q(i), gold NLL = -log sum_{text(c) = gold} q(c)
 *
 * as defined by "JET: Justification Evaluation in Transformer" (Eq. 1-5 and the decision
 * rules after them), the gemma-e2b "Parallel decision inference" doc ("Candidate
 * likelihoods", "Output contracts"), FastJEV Sec. 3.3 ("Candidate Preserving Readout":
 * project each predictor node once, normalise over the full vocabulary, gather along
 * candidate paths) and, for the restricted-vocabulary entry point, the nimble page
 * "Parallel constrained scoring in MLX" (Execution, steps 5-6).
 *
 * Conventions for every entry point:
 *  - Pointers named in a *_problem / *_outputs struct are DEVICE pointers owned by the
 *    caller, except where a comment says HOST.  Nothing is allocated, freed or
 *    synchronised by the library; all work is enqueued on the caller's stream
 *    (a hipStream_t passed as void*, NULL = the null stream).
 *  - Matrices are row-major and densely packed: H[n_rows][d], W[V][d].
 *  - bf16 operands are IEEE bfloat16 bit patterns (uint16); fp32 are IEEE binary32.
 *  - Supported operand types: (W bf16, H bf16), (W bf16, H fp32: H is split exactly
 *    into two bf16 terms so the product keeps about 16 significant bits of H), and
 *    (W fp32, H fp32).  Anything else returns JET_E_DTYPE.
 *  - d must be a positive multiple of 32 (at most 65536); V >= 1; counts >= 0.
 *  - Errors: functions return a negative jet_status.  Every status except JET_E_HIP
 *    comes from a check made on the host before anything is enqueued, so such a call
 *    enqueues nothing.  JET_E_HIP reports a HIP runtime call (a kernel launch or an event
 *    record) that failed: the launches the same call enqueued before it stay enqueued
 *    (they read and write only the call's own buffers), and the outputs, the workspace and
 *    *dev_flags are then undefined.  Only scalars and pointers are checked on the host,
 *    since index arrays live on the device; use jet_validate_host (host copies) to check
 *    indices.  On the device every index is
 *    bounds-checked: an out-of-range row, target or offset never causes an out-of-bounds
 *    access; it sets a bit in *dev_flags (when given) and yields NaN in the affected
 *    outputs.  Outputs are defined only when the status is JET_OK and *dev_flags is 0.
 *  - The library is stateless and re-entrant; calls on different streams may overlap if
 *    their workspaces differ.
 */
#ifndef JET_H
#define JET_H

#include <stddef.h>
#include <stdint.h>

#if defined(__GNUC__) || defined(__clang__)
#define JET_API __attribute__((visibility("default")))
#else
#define JET_API
#endif

#ifdef __cplusplus
extern "C" {
#endif

/* Status and dtype values cross the ABI as 32-bit ints and may come from any caller; in
 * C++ the enums take int32_t as their underlying type so that every such value is a valid
 * enumerator-typed value (C enums are int already). */
#ifdef __cplusplus
#define JET_ENUM_INT : int32_t
#else
#define JET_ENUM_INT
#endif

typedef enum JET_ENUM_INT {
  JET_OK = 0,
  JET_E_NULL = -1,      /* a required pointer is NULL                                  */
  JET_E_SHAPE = -2,     /* a size is out of range (negative count, d % 32 != 0, ...)    */
  JET_E_DTYPE = -3,     /* unsupported operand type combination                         */
  JET_E_INDEX = -4,     /* host validation: index out of range or offsets not monotone  */
  JET_E_TEMP = -5,      /* T is not finite or not > 0                                   */
  JET_E_WORKSPACE = -6, /* workspace NULL, smaller than the size query, or misaligned   */
  JET_E_HIP = -7,       /* a HIP runtime call (launch, event record) failed; earlier
                           launches of the same call may already be enqueued            */
} jet_status;

typedef enum JET_ENUM_INT { JET_F32 = 0, JET_BF16 = 1 } jet_dtype;

/* Device flag bits written to *dev_flags (OR-ed; the buffer is cleared by each call). */
#define JET_FLAG_BAD_ROW 1u      /* tok_row[k] outside [0, n_rows)                        */
#define JET_FLAG_BAD_TARGET 2u   /* tok_target[k] outside [0, V)                          */
#define JET_FLAG_BAD_OFFSETS 4u  /* cand_tok_off / q_cand_off / field offsets malformed   */
#define JET_FLAG_BAD_TRUE_IDX 8u /* q_true_idx[q] outside [-1, K_q)                       */
#define JET_FLAG_BAD_UNION 16u   /* union id / slot index / field row out of range        */

/* Full-vocabulary problem (JET Eq. 1-5).  Token k is scored from predictor row
 * tok_row[k] against target tok_target[k]; tokens [cand_tok_off[c], cand_tok_off[c+1])
 * form candidate c in order; candidates [q_cand_off[g], q_cand_off[g+1]) form question g
 * in their fixed tie order.  One row may serve many tokens: e.g. the shared prefix row
 * scores the first token of every candidate (JET, hybrid execution) and one field row
 * scores every single-token choice of that field (gemma-e2b doc). */
typedef struct {
  const void* H;             /* [n_rows][d] predictor hidden states                      */
  jet_dtype h_dtype;
  int32_t n_rows;
  const void* W;             /* [V][d] LM head (tied embedding) rows                     */
  jet_dtype w_dtype;
  int32_t V;
  int32_t d;
  const int32_t* tok_row;    /* [n_tok] row of token k; NULL: token k uses row k          */
  const int32_t* tok_target; /* [n_tok] target id in [0, V)                                */
  int32_t n_tok;
  const int32_t* cand_tok_off; /* [n_cand+1]: 0 = off[0] < off[1] < ... = n_tok (m_c >= 1) */
  int32_t n_cand;
  const int32_t* q_cand_off;   /* [n_q+1]: 0 = off[0] < ... = n_cand (K_g >= 1)            */
  int32_t n_q;
  const int32_t* cand_text_id;   /* [n_cand] optional: equal id = identical answer text   */
  const int32_t* q_gold_text_id; /* [n_q] optional: text id of the gold answer            */
  const int32_t* q_true_idx;     /* [n_q] optional: local index of "true", -1 = none;
                                    NULL: index 1 when K_g == 2 ([false, true]), else none */
  float T;                       /* candidate temperature, finite and > 0 (default 1)     */
} jet_problem;

/* Outputs of jet_score (device buffers, fp32 unless noted).  Required: tok_logp, cand_s,
 * cand_q, q_argmax.  Optional outputs may be NULL. */
typedef struct {
  float* tok_logp;     /* [n_tok]  l_k (<= 0; NaN for an out-of-range row or target)       */
  float* row_lse;      /* [n_rows] LSE_r (optional)                                        */
  float* cand_s;       /* [n_cand] s(c)                                                    */
  float* cand_q;       /* [n_cand] q(c)                                                    */
  int32_t* q_argmax;   /* [n_q] local index of the decision (lowest index wins ties)      */
  float* q_true;       /* [n_q] q(true); NaN when the question has no true index (opt.)   */
  float* q_expect;     /* [n_q] sum_i i q(i), levels 0..K-1 in supplied order (optional)  */
  float* q_gold_nll;   /* [n_q] -log sum_{text = gold} q; NaN without text ids, +inf when
                          no candidate has the gold text (optional)                        */
  float* q_confidence; /* [n_q] 1 - H(q) / ln K, 1 when K = 1 (optional)                  */
  float* q_mass;       /* [n_q] sum_c exp s(c): full-vocabulary probability mass of the
                          complete candidate sequences (optional)                          */
  int32_t* dev_flags;  /* [1] JET_FLAG_* bits met on the device (optional)                 */
} jet_outputs;

/* Bytes of device workspace jet_score needs for this problem (depends only on the
 * problem's scalars: sizes and dtypes).  0 when the problem is invalid. */
JET_API size_t jet_score_workspace_size(const jet_problem* p);

/* Enqueue the whole path: operand staging, fused projection + online full-vocabulary
 * logsumexp (logits never stored), then per token its target logit (one dot product of the
 * operands the projection multiplies), the deterministic merge of its row's per-chunk
 * normalisers and its log-probability, then candidate sums and per-question decisions.  workspace: device memory of at least jet_score_workspace_size(p) bytes,
 * 256-byte aligned, not shared with a concurrent call.  Results are bitwise
 * reproducible for identical inputs and do not depend on a row's position. */
JET_API jet_status jet_score(const jet_problem* p, const jet_outputs* o, void* workspace,
                     size_t workspace_bytes, void* stream);

/* jet_score, additionally recording ev_before and ev_after (hipEvent_t as void*, may be
 * NULL) on the stream immediately before and after the projection kernel, so a caller
 * can time the dominant kernel alone. */
JET_API jet_status jet_score_profiled(const jet_problem* p, const jet_outputs* o, void* workspace,
                              size_t workspace_bytes, void* stream, void* ev_before,
                              void* ev_after);

/* For callers that cannot allocate device memory (code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc): jet_score with the workspace taken from
 * a static device array of JET_NOALLOC_MAX_WORKSPACE bytes inside the library, so neither
 * the caller nor the library allocates.  The caller still owns H, W, the index arrays and
 * the outputs, and passes a stream of the current device.
 *  - Each GPU holds one copy of the array from the library's first use on it until the
 *    process ends.  The first call on a device looks up the array's device address with
 *    that device current (a runtime query, no allocation) and keeps it.
 *  - Every call on a GPU shares that GPU's array: calls that overlap on one GPU (other
 *    streams, other threads) race on it and give undefined results; calls ordered on one
 *    stream are safe.  The array keeps the last call's contents; every call clears what
 *    must start at zero itself, with kernels (no memsets).
 *  - A problem whose workspace (jet_score_workspace_size) exceeds the array returns
 *    JET_E_WORKSPACE with nothing enqueued; JET_E_HIP also when the address lookup fails.
 *    Otherwise as jet_score: same checks, same kernels, same bits. */
#define JET_NOALLOC_MAX_WORKSPACE ((size_t)64 << 20)
JET_API jet_status jet_score_noalloc(const jet_problem* p, const jet_outputs* o, void* stream);

/* Name of the projection kernel jet_score launches for this problem (the plan depends
 * only on the problem's scalars), as profilers report it: "k_project_tiled_m16",
 * "k_project_tiled_m16x2", "k_project_wg_bf16", "k_project_small_bf16" or
 * "k_project_wg_f32".  NULL when the problem is invalid.  Host only; the string is
 * static. */
JET_API const char* jet_projection_kernel(const jet_problem* p);

/* Measurement helper, not part of scoring: reads every byte of buf (device memory, 16-byte
 * aligned, bytes a multiple of 16) once with plain coalesced loads and XORs a checksum of
 * the words into *out (device memory; not cleared).  Timed around the same bytes the
 * projection streams, it gives the device's achievable read rate next to the HBM spec.
 * Enqueued on stream; JET_E_NULL / JET_E_SHAPE on bad arguments, JET_E_HIP on a failed
 * launch. */
JET_API jet_status jet_stream_read(const void* buf, size_t bytes, uint32_t* out, void* stream);

/* Host-side validation of a problem whose index arrays (tok_row, tok_target,
 * cand_tok_off, q_cand_off, q_true_idx) are HOST pointers; H and W are not read.
 * Returns JET_OK or the first error found. */
JET_API jet_status jet_validate_host(const jet_problem* p);

/* HOST: predictor-row deduplication by history-consistent merging (FastJEV Sec. 3.3,
 * Eq. 4).  Token t of a candidate is predicted from the state after its preceding history
 * (the question's context, then the candidate's tokens 0..t-1).  Histories form one tree
 * per question, a child keyed by (parent node, token); depth fixes the position.  Tokens
 * share a predictor node exactly when they belong to the same question and have identical
 * preceding histories.
 *   tok_target[n_tok], cand_tok_off[n_cand+1], q_cand_off[n_q+1]: the problem's token and
 *     offset arrays (HOST copies; n_tok = cand_tok_off[n_cand]; offsets monotone from 0,
 *     every candidate and question non-empty, targets >= 0).
 *   tok_node[n_tok] (out): predictor node of each token, numbered 0.. in order of first use.
 *   node_tok[n_tok] (out): node_tok[j] = first token predicted from node j (its row in a
 *     one-row-per-token layout holds node j's state); entries >= *n_nodes are untouched.
 *   *n_nodes (out): number of predictor nodes.
 * Scoring with H' = rows of node_tok and tok_row = tok_node projects each node once and
 * gives the same outputs when equal histories have equal states.  Returns JET_E_NULL,
 * JET_E_SHAPE (malformed offsets) or JET_E_INDEX (a negative target) without writing. */
JET_API jet_status jet_build_predictor_trie(const int32_t* tok_target, const int32_t* cand_tok_off,
                                            int32_t n_cand, const int32_t* q_cand_off, int32_t n_q,
                                            int32_t* tok_node, int32_t* node_tok, int32_t* n_nodes);

/* Restricted-vocabulary scoring (nimble page, Execution steps 5-6): gather only the
 * allowed head rows (their sorted union), project the rows onto the union and take each
 * field's softmax over its own allowed ids at temperature T.  The full-vocabulary
 * normaliser is never computed, so there are no token log-probabilities. */

/* HOST: build the sorted unique union of every field's allowed ids and, per slot, the
 * index of its id in the union.  field_ids[field_off[n_fields]] and field_off[n_fields+1]
 * are inputs; union_ids must hold field_off[n_fields] entries; slot_uidx likewise.
 * Returns JET_E_INDEX for an id outside [0, V) or malformed offsets. */
JET_API jet_status jet_build_union(const int32_t* field_ids, const int32_t* field_off, int32_t n_fields,
                           int32_t V, int32_t* union_ids, int32_t* n_union, int32_t* slot_uidx);

typedef struct {
  const void* H;                /* [n_rows][d]                                              */
  jet_dtype h_dtype;
  int32_t n_rows;
  const void* W;                /* [V][d]                                                   */
  jet_dtype w_dtype;
  int32_t V;
  int32_t d;
  const int32_t* union_ids;     /* [n_union] sorted unique ids in [0, V)                    */
  int32_t n_union;
  const int32_t* field_row;     /* [n_fields] row of H scored for field f                  */
  const int32_t* field_slot_off;/* [n_fields+1] monotone, K_f >= 1, last = n_slots          */
  const int32_t* slot_uidx;     /* [n_slots] index into union_ids of slot j's allowed id   */
  int32_t n_fields;
  int32_t n_slots;
  float T;                      /* finite, > 0                                              */
} jet_restricted_problem;

typedef struct {
  float* slot_logit;      /* [n_slots] z[field_row[f], union_ids[slot_uidx[j]]]             */
  float* slot_q;          /* [n_slots] softmax over the field's slots of slot_logit / T     */
  int32_t* field_argmax;  /* [n_fields] local slot index of the decision (lowest wins ties) */
  int32_t* dev_flags;     /* [1] optional                                                   */
} jet_restricted_outputs;

/* Bytes of device workspace jet_score_restricted needs (from the scalars only; 0 when the
 * problem is invalid): a flag word, and with d > 16384 or more than 4096 slots also, for a
 * bf16 head, the fp32 partial sums of the projection over ceil(d / 512) groups of k,
 * [groups][n_union][n_rows], and for an fp32 head the gathered rows [n_union][d] and the
 * logits [n_rows][n_union]. */
JET_API size_t jet_restricted_workspace_size(const jet_restricted_problem* p);
/* Enqueue the restricted path: project the rows onto the union, then each field's softmax
 * and argmax over its slots.  A problem with d <= 16384 and at most 4096 slots takes one
 * launch (a workgroup per field computes its slots' logits, softmax and argmax, reading the
 * head rows through union_ids).  Larger ones take two with a bf16 head (read through
 * union_ids by the projection) and four with an fp32 head (its union rows gathered into the
 * workspace first).  workspace: at least jet_restricted_workspace_size(p) bytes,
 * 256-byte aligned, not shared with a concurrent call.  Host checks return JET_E_NULL,
 * JET_E_SHAPE, JET_E_DTYPE, JET_E_TEMP or JET_E_WORKSPACE and enqueue nothing.  On the
 * device an id outside [0, V) reads as a zero row and a slot index, field row or field
 * offset out of range yields NaN / -1 in that field; each raises its JET_FLAG_* bit. */
JET_API jet_status jet_score_restricted(const jet_restricted_problem* p, const jet_restricted_outputs* o,
                                void* workspace, size_t workspace_bytes, void* stream);
/* Host-side validation of a restricted problem whose index arrays are HOST pointers. */
JET_API jet_status jet_validate_restricted_host(const jet_restricted_problem* p);

/* Decision sensitivity of layer skips (FastJEV Sec. 3.4, Eq. 5-6), for a calibration set
 * of logit vectors (candidates and abstention, before any probability post-processing).
 *   z[n_values]: the inputs' logits back to back; input x owns z[seg_off[x] .. seg_off[x+1]).
 *   z_skip[n_layers][n_values]: the same logits with layer l skipped (row l).
 *   seg_off[n_inputs+1]: device offsets, each segment non-empty and inside [0, n_values).
 *   eps: floor of the denominator (the pages use 1e-8); finite and > 0.
 * Outputs (device, caller-owned):
 *   d[n_layers][n_inputs] = rms(ctr(z_skip[l] - z)) / max(eps, rms(ctr(z))) over input x's
 *     entries, with ctr(v) = v - mean(v) and rms(v) = ||v|| / sqrt(m);
 *   J[n_layers] = mean over inputs of d;
 *   selected[k] = the k layers with the smallest J, ties resolved by layer index, in that
 *     order (0 <= k <= n_layers; may be NULL when k = 0);
 *   dev_flags[1] (optional) = JET_FLAG_BAD_OFFSETS if a segment is malformed (its d and the
 *     J built on it are NaN; NaN ranks last).
 * Results are bitwise reproducible.  Host checks: JET_E_NULL, JET_E_SHAPE (n_inputs < 1,
 * n_values < 1, n_layers outside [1, 4096], k outside [0, n_layers], eps not finite > 0). */
JET_API jet_status jet_decision_sensitivity(const float* z, const float* z_skip,
                                            const int32_t* seg_off, int32_t n_inputs,
                                            int32_t n_values, int32_t n_layers, float eps,
                                            int32_t k, float* d, float* J, int32_t* selected,
                                            int32_t* dev_flags, void* stream);

/* Temperature fitting (gemma-e2b doc, "Output contracts"; nimble, "V2 probability
 * default": T scales candidate scores once, before the softmax): the T in [T_min, T_max]
 * minimising the mean over labelled questions of the gold NLL,
 *   LSE(s/T) - LSE(s/T over the candidates whose text id equals the gold text id).
 *   cand_s[n_cand] (device): candidate sequence scores s(c), e.g. jet_score's cand_s.
 *   q_cand_off[n_q+1], cand_text_id[n_cand], q_gold_text_id[n_q] (device): as in
 *     jet_problem; a question with gold id < 0 or no candidate of the gold text is not
 *     counted; a malformed question raises JET_FLAG_BAD_OFFSETS and is skipped.
 *   T_fit[1], nll_fit[1] (device out): the fitted T and the mean gold NLL there (NaN if no
 *     question is counted); dev_flags[1] optional.
 *   workspace: device memory of at least jet_fit_temperature_workspace_size(n_q) bytes,
 *     256-byte aligned, not shared with a concurrent call.
 * Search: 64 temperatures evenly spaced in log T, narrowed six times around the argmin
 * (lowest index on ties); bitwise reproducible.  Host checks: JET_E_NULL, JET_E_SHAPE
 * (n_q < 1 or n_cand < 1), JET_E_TEMP (0 < T_min < T_max, both finite), JET_E_WORKSPACE. */
JET_API size_t jet_fit_temperature_workspace_size(int32_t n_q);
JET_API jet_status jet_fit_temperature(const float* cand_s, const int32_t* q_cand_off, int32_t n_q,
                                       int32_t n_cand, const int32_t* cand_text_id,
                                       const int32_t* q_gold_text_id, float T_min, float T_max,
                                       float* T_fit, float* nll_fit, int32_t* dev_flags,
                                       void* workspace, size_t workspace_bytes, void* stream);

/* Static description of a status code. */
JET_API const char* jet_status_string(jet_status s);

#ifdef __cplusplus
}
#endif

#endif /* JET_H */
