// Internal declarations shared by the HIP translation units of libjet.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <math.h>

#include "../../include/jet.h"

namespace jet {

constexpr int kWave = 64;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(4))) unsigned u32x4;

// bf16 round-to-nearest-even of an fp32 value (gfx950 converts in hardware,
// v_cvt_pk_bf16_f32; NaN stays a NaN).
__device__ inline uint16_t f32_to_bf16_rne(float x) {
  return __builtin_bit_cast(uint16_t, (__bf16)x);
}

// Exact two-term split of two fp32 values: hi = bf16(x), lo = bf16(x - hi), packed as
// bf16 pairs (element 0 in the low half).  x - hi is exact in fp32.
__device__ inline void split_pair(float a, float b, uint32_t& hi, uint32_t& lo) {
  const __bf16 ha = (__bf16)a, hb = (__bf16)b;
  const __bf16 la = (__bf16)(a - (float)ha), lb = (__bf16)(b - (float)hb);
  hi = (uint32_t)__builtin_bit_cast(uint16_t, ha) | ((uint32_t)__builtin_bit_cast(uint16_t, hb) << 16);
  lo = (uint32_t)__builtin_bit_cast(uint16_t, la) | ((uint32_t)__builtin_bit_cast(uint16_t, lb) << 16);
}

__device__ inline float bf16_to_f32(uint16_t b) { return __uint_as_float(((uint32_t)b) << 16); }

// Merge two online-logsumexp states (m = running max, s = sum of exp(z - m)).
// Symmetric in its arguments bit-for-bit (max and + commute), so xor-shuffle trees give
// every lane the same result.
// Hardware base-2 exponential (v_exp_f32, about 1 ulp).  Results below 2^-126 may flush to
// zero; used for the terms of a sum of exp(z - max), which always holds a term equal to 1.
__device__ inline float exp2_hw(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ inline void lse_merge(float& m, float& s, float m2, float s2) {
  float M = fmaxf(m, m2);
  if (M == -INFINITY) return;
  s = s * exp2f((m - M) * kLog2e) + s2 * exp2f((m2 - M) * kLog2e);
  m = M;
}

__device__ inline void flag_or(int32_t* flags, uint32_t bit) {
  if (flags) atomicOr(flags, (int32_t)bit);
}

// ------------------------------------------------------------------------------------
// Execution plan of one jet_score call (derived from the scalars only)
// ------------------------------------------------------------------------------------
enum Variant { VAR_SMALL_BF16 = 0, VAR_SMALL_F32 = 1, VAR_TILED_BF16 = 2 };

// fp32 heads take the streaming kernel k_project_wg_f32 (0: the k-split kernel
// k_project_small_f32, kept for the restricted path's stored logits)
#ifndef JET_F32_STREAM
#define JET_F32_STREAM 1
#endif

struct Plan {
  int variant;
  bool hilo;          // fp32 H split into bf16 hi + lo
  bool stream;        // streaming kernel (bf16 head with d % 64 == 0, or an fp32 head):
                      // partials row-major; with a bf16 head it splits fp32 H itself
  int stream_nr;      // streaming kernel: 32-row tiles of H per workgroup (1, 2 or 4)
  int row_tile;       // rows per projection tile
  int rows_k;         // rows the projection kernel sees: n_rows, or one whole row tile of the
                      // tiled kernel when n_rows is smaller (H then padded with zero rows)
  bool pad_h;         // bf16 H copied into the workspace with zero rows up to rows_k
  int n_rtiles;
  int vgroup;         // vocabulary entries per group (a multiple of the kernel's tile)
  int n_vgroups;
  int grid_x;         // projection workgroups along the vocabulary
  int n_parts;        // (m, s) partials per row
  // workspace byte offsets
  size_t off_hhi, off_hlo, off_hpad, off_part, off_flags, total;
};

void make_plan(const jet_problem* p, Plan* plan);

// ------------------------------------------------------------------------------------
// Launchers (each returns hipSuccess or the launch error)
// ------------------------------------------------------------------------------------
struct ScoreArgs {
  const jet_problem* p;
  const jet_outputs* o;
  const Plan* plan;
  char* ws;
  int32_t* flags;    // device flag word (caller's or workspace)
  hipStream_t stream;
};

hipError_t launch_prep(const ScoreArgs& a);
hipError_t launch_project(const ScoreArgs& a);
hipError_t launch_project_tiled(const ScoreArgs& a);
bool stream_d(int d);  // d the streaming kernel takes (a multiple of 64)
int tiled_bk(bool hilo);
int tiled_row_tile(bool hilo, int d);
const char* tiled_kernel_name(bool hilo, int d);
int sensitivity_max_layers();
size_t fit_temperature_workspace(int n_q);
hipError_t launch_fit_temperature(const float* s, const int* q_cand_off, int n_q, int n_cand,
                                  const int* text, const int* gold, float T_min, float T_max,
                                  float* T_out, float* nll_out, int32_t* flags, char* ws,
                                  hipStream_t stream);
hipError_t launch_sensitivity(const float* z, const float* z_skip, const int* seg_off,
                              int n_inputs, int n_values, int n_layers, float eps, int k,
                              float* d, float* J, int32_t* selected, int32_t* flags,
                              hipStream_t stream);  // the tiled kernel launched for this plane count
hipError_t launch_token_logp(const ScoreArgs& a);  // also clears the flag word without rows
hipError_t launch_decide(const ScoreArgs& a);

struct RestrictedPlan {
  bool per_field;  // d <= 16384, <= 4096 slots: one launch, a workgroup per field
  bool fused;  // bf16 head: gather and split inside the projection, k-split partials of Z
  int n_kg;    // partial sums of Z (k groups)
  size_t off_wu, off_z, off_flags, total;
};
bool make_restricted_plan(const jet_restricted_problem* p, RestrictedPlan* plan);
hipError_t launch_restricted(const jet_restricted_problem* p, const jet_restricted_outputs* o,
                             const RestrictedPlan* plan, char* ws, int32_t* flags,
                             hipStream_t stream);

// H fp32 -> (hi, lo) bf16 planes for the tiled and fallback kernels; elements n_elems ..
// n_out - 1 of the planes are zero (padding rows).
hipError_t launch_split(const float* H, long long n_elems, long long n_out, uint16_t* hi,
                        uint16_t* lo, hipStream_t stream);

// Projection core of the restricted path with an fp32 head: Z[row][u] = <H[row], Wu[u]>
// for all rows and gathered union entries.
hipError_t launch_project_store_f32(const float* Wu, int U, int d, const float* H, int n_rows,
                                    float* Z, hipStream_t stream);

}  // namespace jet
