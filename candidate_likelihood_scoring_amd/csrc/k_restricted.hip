// Restricted-vocabulary scoring (nimble "Parallel constrained scoring in MLX", Execution
// steps 5-6): gather only the allowed head rows, project the hidden states onto their
// union, and let each field take a softmax over its own allowed ids at temperature T.
//
// d <= 16384 and at most 4096 slots, either head dtype: one launch, a workgroup per field
// (k_restricted_fields, k_restricted_fields_lds below).  Past those limits:
// bf16 head (two launches):
//   k_restricted_project: Z[r, j] = <H[r], W[union_ids[j]]> on the matrix cores, fp32
//                   accumulation, with the row gather and the fp32 split (H = hi + lo, both
//                   bf16) done in the operand loads, so the gathered rows never exist in
//                   memory; k is split over workgroups, which store fp32 partial sums.
//   k_field_softmax: one wave per field: slot_logit = the sum of the partials (in a fixed
//                   order) at (field_row, slot_uidx), a = logit/T, q = softmax(a) over the
//                   field's slots, argmax = lowest index among the exact maxima of a.
// fp32 head: k_gather_rows (Wu[j, :] = W[union_ids[j], :], 16-byte coalesced copies), the
// small-row fp32 kernel's store epilogue, then k_field_softmax.
#include "jet_tail.h"

namespace jet {
namespace {

__global__ __launch_bounds__(256) void k_gather_rows(const uint4* __restrict__ W, int V,
                                                     int row_vec, const int* __restrict__ ids,
                                                     int n_union, uint4* __restrict__ Wu,
                                                     int32_t* __restrict__ flags) {
  for (int j = blockIdx.x; j < n_union; j += gridDim.x) {
    const int id = ids[j];
    const bool ok = id >= 0 && id < V;
    if (!ok && threadIdx.x == 0) flag_or(flags, JET_FLAG_BAD_UNION);
    const uint4* src = W + (size_t)(ok ? id : 0) * row_vec;
    uint4* dst = Wu + (size_t)j * row_vec;
    for (int i = threadIdx.x; i < row_vec; i += 256) dst[i] = ok ? src[i] : make_uint4(0, 0, 0, 0);
  }
}

__global__ void k_clear_flag(int32_t* __restrict__ flags) {
  if (threadIdx.x == 0) flags[0] = 0;
}

// Projection onto the union for a bf16 head.  Tile (ut, rt, kg) covers union entries
// [32 ut, 32 ut + 32), rows [32 rt, 32 rt + 32) and k in [512 kg, 512 kg + 512); wave w of
// the workgroup takes the 128-wide k slice at 512 kg + 128 w and issues all of its loads
// before its first matrix op, so a tile costs one memory round trip.  Lane l supplies
// union entry l % 32 (A operand, read straight from the head row union_ids[.]) and row
// l % 32 (B operand); in each 32-wide block kb its half h = l / 32 covers k in
// [kb + 16 h, kb + 16 h + 16): 32 contiguous bytes of the head row and 32 (bf16 H) or 64
// (fp32 H) of the hidden row, consumed by two v_mfma_f32_32x32x16_bf16 (A and B use the
// same k order, so the sum is unchanged).  fp32 H is split on the fly, hi = bf16(x) and
// lo = bf16(x - hi), two products per step.  The four waves' 32x32 tiles are added in wave
// order through LDS and stored as the partial Zp[kg][u][row] (rows contiguous, so each
// store instruction writes two 128-byte runs).  An id outside [0, V) reads as a zero row;
// k_field_softmax reports it.  Workgroup 0 clears the flag word first: this kernel sets no
// flags, and the next launch on the stream does.
constexpr int kRkWave = 128, kRWaves = 4, kRkTile = kRkWave * kRWaves;

template <bool HF32>
__global__ __launch_bounds__(256) void k_restricted_project(
    const uint16_t* __restrict__ W, int V, int d, const int* __restrict__ ids, int n_union,
    const void* __restrict__ H, int n_rows, int n_ut, int n_rt, int n_kg,
    float* __restrict__ Zp, int32_t* __restrict__ flags) {
  __shared__ f32x16 red[kRWaves - 1][kWave];
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const int m = lane & 31, h = lane >> 5;
  if (blockIdx.x == 0 && threadIdx.x == 0) flags[0] = 0;
  const long long n_tiles = (long long)n_ut * n_rt * n_kg;
  for (long long tile = blockIdx.x; tile < n_tiles; tile += gridDim.x) {
    const int kg = (int)(tile % n_kg);
    const int rt = (int)((tile / n_kg) % n_rt);
    const int ut = (int)(tile / ((long long)n_kg * n_rt));
    const int u0 = ut * 32, row0 = rt * 32;
    const int id = ids[min(u0 + m, n_union - 1)];
    const bool id_ok = id >= 0 && id < V;
    const uint16_t* wrow = W + (size_t)(id_ok ? id : 0) * d;
    const int hr = min(row0 + m, n_rows - 1);
    const int k0 = kg * kRkTile + wid * kRkWave;
    // 32-wide blocks of this wave's slice inside [0, d) (d is a multiple of 32); blocks
    // past the end load the last block again (in bounds) and are not used
    const int nb = min(kRkWave, max(0, d - k0)) / 32;
    uint4 a[4][2], b[4][HF32 ? 4 : 2];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const int kb = min(k0 + 32 * t, d - 32) + 16 * h;
      const uint4* wp = reinterpret_cast<const uint4*>(wrow + kb);
      a[t][0] = wp[0];
      a[t][1] = wp[1];
      if constexpr (HF32) {
        const uint4* hp = reinterpret_cast<const uint4*>(static_cast<const float*>(H) + (size_t)hr * d + kb);
#pragma unroll
        for (int j = 0; j < 4; ++j) b[t][j] = hp[j];
      } else {
        const uint4* hp = reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(H) + (size_t)hr * d + kb);
#pragma unroll
        for (int j = 0; j < 2; ++j) b[t][j] = hp[j];
      }
    }
    f32x16 acc = {};
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      if (t < nb) {
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const uint4 av = id_ok ? a[t][j] : make_uint4(0, 0, 0, 0);
          if constexpr (HF32) {
            const uint4 x0 = b[t][2 * j], x1 = b[t][2 * j + 1];
            uint32_t h0, h1, h2, h3, l0, l1, l2, l3;
            split_pair(__uint_as_float(x0.x), __uint_as_float(x0.y), h0, l0);
            split_pair(__uint_as_float(x0.z), __uint_as_float(x0.w), h1, l1);
            split_pair(__uint_as_float(x1.x), __uint_as_float(x1.y), h2, l2);
            split_pair(__uint_as_float(x1.z), __uint_as_float(x1.w), h3, l3);
            const u32x4 hi = {h0, h1, h2, h3}, lo = {l0, l1, l2, l3};
            acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, av),
                                                          __builtin_bit_cast(bf16x8, hi), acc, 0, 0, 0);
            acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, av),
                                                          __builtin_bit_cast(bf16x8, lo), acc, 0, 0, 0);
          } else {
            acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, av),
                                                          __builtin_bit_cast(bf16x8, b[t][j]), acc, 0, 0, 0);
          }
        }
      }
    }
    if (wid > 0) red[wid - 1][lane] = acc;
    __syncthreads();
    if (wid == 0) {
#pragma unroll
      for (int w = 0; w < kRWaves - 1; ++w) acc += red[w][lane];
      // output (union entry, row) of register i: entry 8 (i / 4) + 4 h + i % 4, row lane % 32
      const int row = row0 + m;
      if (row < n_rows) {
        float* zp = Zp + (size_t)kg * n_union * n_rows;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int u = u0 + 8 * (i >> 2) + 4 * h + (i & 3);
          if (u < n_union) zp[(size_t)u * n_rows + row] = acc[i];
        }
      }
    }
    __syncthreads();  // red is rewritten by the next tile
  }
}

// Z holds n_part partial sums of the logits: z(r, u) = sum over p in order 0, 1, ... of
// Z[p * part_stride + u * u_stride + r * r_stride].  Every workgroup also checks a strided
// share of the union ids (an id outside [0, V) raises JET_FLAG_BAD_UNION).
__global__ __launch_bounds__(256) void k_field_softmax(
    const float* __restrict__ Z, int n_part, size_t part_stride, int u_stride, int r_stride,
    int n_rows, int n_union, const int* __restrict__ ids, int V,
    const int* __restrict__ field_row, const int* __restrict__ slot_off,
    const int* __restrict__ slot_uidx, int n_fields, int n_slots, float T,
    float* __restrict__ slot_logit, float* __restrict__ slot_q, int* __restrict__ f_argmax,
    int32_t* __restrict__ flags) {
  for (int j = blockIdx.x * blockDim.x + threadIdx.x; j < n_union; j += gridDim.x * blockDim.x) {
    const int id = ids[j];
    if (id < 0 || id >= V) flag_or(flags, JET_FLAG_BAD_UNION);
  }
  // the offsets' ends: with them and every field's own check, the fields partition the slots
  if (blockIdx.x == 0 && threadIdx.x == 0 && n_fields > 0 &&
      (slot_off[0] != 0 || slot_off[n_fields] != n_slots))
    flag_or(flags, JET_FLAG_BAD_OFFSETS);
  const int lane = threadIdx.x & 63;
  const int f = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (f >= n_fields) return;
  const float NaN = __builtin_nanf("");
  const int j0 = slot_off[f], j1 = slot_off[f + 1];
  const int r = field_row[f];
  if (j0 < 0 || j1 > n_slots || j1 <= j0) {
    if (lane == 0) {
      flag_or(flags, JET_FLAG_BAD_OFFSETS);
      f_argmax[f] = -1;
    }
    return;
  }
  const bool row_ok = r >= 0 && r < n_rows;
  if (!row_ok && lane == 0) flag_or(flags, JET_FLAG_BAD_UNION);
  float best = -INFINITY;
  int best_j = j1;
  bool bad = false;
  for (int j = j0 + lane; j < j1; j += 64) {
    const int u = slot_uidx[j];
    float z = NaN;
    if (row_ok && u >= 0 && u < n_union) {
      const float* zp = Z + (size_t)u * u_stride + (size_t)r * r_stride;
      z = zp[0];
      for (int q = 1; q < n_part; ++q) z += zp[q * part_stride];
    } else {
      bad = true;
    }
    slot_logit[j] = z;
    const float a = z / T;
    if (a > best) {
      best = a;
      best_j = j;
    }
  }
  if (bad) flag_or(flags, JET_FLAG_BAD_UNION);
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    const float ob = __shfl_xor(best, off);
    const int oj = __shfl_xor(best_j, off);
    if (ob > best || (ob == best && oj < best_j)) {
      best = ob;
      best_j = oj;
    }
  }
  float zp = 0.f;
  for (int j = j0 + lane; j < j1; j += 64) zp += expf(slot_logit[j] / T - best);
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) zp += __shfl_xor(zp, off);
  for (int j = j0 + lane; j < j1; j += 64) slot_q[j] = expf(slot_logit[j] / T - best) / zp;
  if (lane == 0) f_argmax[f] = best_j < j1 ? best_j - j0 : -1;
}

// One launch for d <= 16384 and at most 4096 slots (every problem of the common shapes):
// workgroup f scores field f alone.  Its 16 waves take the field's slots in turn; for a
// slot, lane l multiplies head row union_ids[slot_uidx[j]] by the field's hidden row at
// k = 512 c + 8 l .. + 7 for each 512-wide chunk c (fp32 products, accumulated in k order
// per lane, then the wave's fixed lane tree), so the logit is a full-length fp32 dot
// product.  A bf16 head up to d = 2560: the hidden row stays in registers for all the
// field's slots and the next slot's head row is loaded while the current one is summed
// (k_restricted_fields).  Past that, and for an fp32 head at any d: the row is staged once
// in LDS as fp32 and each slot's head row is loaded eight (bf16) or four (fp32) chunks at
// a time (k_restricted_fields_lds), the same products summed in the same order.  Then
// wave 0 takes the field's softmax at T and argmax (lowest index among the exact maxima).
// No workgroup needs another's results.
// Index checks: workgroup 0 checks every union id, field offset, field row and slot index
// and stores the flag word (a plain store of the whole word: no other workgroup writes it,
// so it needs no clearing first); each field treats its own bad indices as k_field_softmax
// does (an id outside [0, V) reads as a zero row; a bad slot index or row gives NaN; bad
// offsets give argmax -1).
constexpr int kFieldWaves = 16, kFieldMaxSlots = 4096, kFieldMaxD = 16384;
constexpr int kFieldThreads = kFieldWaves * 64;

struct FieldArgs {
  const void* W;
  int V, d;
  const int* ids;
  int n_union;
  const void* H;
  int n_rows;
  const int* field_row;
  const int* slot_off;
  const int* slot_uidx;
  int n_fields, n_slots;
  float T;
  float* slot_logit;
  float* slot_q;
  int* f_argmax;
  int32_t* flags;
};

// workgroup 0: every index array checked, the flag word stored whole
__device__ inline void fields_check(const FieldArgs& a, uint32_t* s_bits, int tid) {
  if (tid == 0) *s_bits = 0u;
  __syncthreads();
  uint32_t bits = 0u;
  for (int j = tid; j < a.n_union; j += kFieldThreads)
    if (a.ids[j] < 0 || a.ids[j] >= a.V) bits |= JET_FLAG_BAD_UNION;
  for (int g = tid; g < a.n_fields; g += kFieldThreads) {
    const int lo = a.slot_off[g], hi = a.slot_off[g + 1], r = a.field_row[g];
    if (lo < 0 || hi > a.n_slots || hi <= lo) bits |= JET_FLAG_BAD_OFFSETS;
    else if (r < 0 || r >= a.n_rows) bits |= JET_FLAG_BAD_UNION;
  }
  for (int j = tid; j < a.n_slots; j += kFieldThreads)
    if (a.slot_uidx[j] < 0 || a.slot_uidx[j] >= a.n_union) bits |= JET_FLAG_BAD_UNION;
  // the offsets' ends: with them and every field's own check, the fields partition the slots
  if (tid == 0 && a.n_fields > 0 && (a.slot_off[0] != 0 || a.slot_off[a.n_fields] != a.n_slots))
    bits |= JET_FLAG_BAD_OFFSETS;
  if (bits) atomicOr(s_bits, bits);
  __syncthreads();
  if (tid == 0) a.flags[0] = (int32_t)*s_bits;
}

// head row of slot j (its union entry valid or not, its id in range or not)
struct SlotRow {
  const char* row;  // row 0 for an id outside [0, V); not read then
  bool use;         // the union index is valid (else the logit is NaN)
  bool id_ok;       // the id is in [0, V) (else the row reads as zeros)
};

template <bool WF32>
__device__ inline SlotRow slot_row(const FieldArgs& a, int j) {
  const int u = a.slot_uidx[j];
  const bool u_ok = u >= 0 && u < a.n_union;
  const int id = u_ok ? a.ids[u] : 0;
  const bool id_ok = u_ok && id >= 0 && id < a.V;
  return SlotRow{static_cast<const char*>(a.W) + (size_t)(id_ok ? id : 0) * a.d * (WF32 ? 4 : 2),
                 u_ok, id_ok};
}

// lane's share of a chunk: 8 head values (bf16) times 8 hidden values, in k order
__device__ inline float chunk_dot(const uint4& w, const float (&h)[8], float acc) {
  const uint32_t w4[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    acc = fmaf(__uint_as_float(w4[e] << 16), h[2 * e], acc);
    acc = fmaf(__uint_as_float(w4[e] & 0xffff0000u), h[2 * e + 1], acc);
  }
  return acc;
}

// the same for 8 fp32 head values (two 16-byte loads)
__device__ inline float chunk_dot_f32(const uint4& w0, const uint4& w1, const float (&h)[8],
                                      float acc) {
  const uint32_t w8[8] = {w0.x, w0.y, w0.z, w0.w, w1.x, w1.y, w1.z, w1.w};
#pragma unroll
  for (int e = 0; e < 8; ++e) acc = fmaf(__uint_as_float(w8[e]), h[e], acc);
  return acc;
}

// the hidden row's 8 values at k (fp32, or bf16 widened exactly)
template <bool HF32>
__device__ inline void load_h8(const void* H, size_t off, float (&h)[8]) {
  if constexpr (HF32) {
    const float4* hp = reinterpret_cast<const float4*>(static_cast<const float*>(H) + off);
    const float4 x0 = hp[0], x1 = hp[1];
    h[0] = x0.x; h[1] = x0.y; h[2] = x0.z; h[3] = x0.w;
    h[4] = x1.x; h[5] = x1.y; h[6] = x1.z; h[7] = x1.w;
  } else {
    const uint4 x = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(H) + off);
    const uint32_t w4[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      h[2 * e] = __uint_as_float(w4[e] << 16);
      h[2 * e + 1] = __uint_as_float(w4[e] & 0xffff0000u);
    }
  }
}

// wave 0: the field's softmax at T over its K logits in s_logit, and its argmax
__device__ inline void fields_decide(const FieldArgs& a, const float* s_logit, int f, int j0,
                                     int K, int lane) {
  float best = -INFINITY;
  int bi = K;
  for (int i = lane; i < K; i += 64) {
    const float av = s_logit[i] / a.T;
    if (av > best) {  // increasing i: a lane keeps its lowest index among equal values
      best = av;
      bi = i;
    }
  }
  wave_argmax(best, bi);
  float zs = 0.f;
  for (int i = lane; i < K; i += 64) zs += expf(s_logit[i] / a.T - best);
  zs = wave_sum(zs);
  for (int i = lane; i < K; i += 64) a.slot_q[j0 + i] = expf(s_logit[i] / a.T - best) / zs;
  if (lane == 0) a.f_argmax[f] = bi < K ? bi : -1;
}

template <bool HF32, int NC>  // NC: 512-wide chunks of k in registers (d <= 512 NC)
__global__ __launch_bounds__(kFieldThreads) void k_restricted_fields(FieldArgs a) {
  __shared__ float s_logit[kFieldMaxSlots];
  __shared__ uint32_t s_bits;
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int f = blockIdx.x;
  if (f == 0) fields_check(a, &s_bits, tid);
  if (f >= a.n_fields) return;
  const int j0 = a.slot_off[f], j1 = a.slot_off[f + 1];
  if (j0 < 0 || j1 > a.n_slots || j1 <= j0) {
    if (tid == 0) a.f_argmax[f] = -1;
    return;
  }
  const int r = a.field_row[f];
  const bool row_ok = r >= 0 && r < a.n_rows;
  const int K = j1 - j0;  // <= n_slots <= kFieldMaxSlots (host check)
  // the field's hidden row: lane l's 8 values of each chunk (zero past d)
  float hv[NC][8];
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    const int k = 512 * c + 8 * lane;
    if (row_ok && k < a.d) {
      load_h8<HF32>(a.H, (size_t)r * a.d + k, hv[c]);
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) hv[c][e] = 0.f;
    }
  }
  // head row of slot j: its chunks (zero for an id outside [0, V), or past d)
  auto load_w = [&](int j, uint4 (&wv)[NC], bool& use) {
    const SlotRow s = slot_row<false>(a, j);
    use = s.use;
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      const int k = 512 * c + 8 * lane;
      wv[c] = (s.id_ok && k < a.d) ? *reinterpret_cast<const uint4*>(s.row + (size_t)k * 2)
                                   : make_uint4(0, 0, 0, 0);
    }
  };
  uint4 wv[NC], wn[NC];
  bool use = false, use_n = false;
  int j = j0 + wid;
  if (j < j1) load_w(j, wv, use);
  for (; j < j1; j += kFieldWaves) {
    const int jn = j + kFieldWaves;
    if (jn < j1) load_w(jn, wn, use_n);
    float acc = 0.f;
#pragma unroll
    for (int c = 0; c < NC; ++c) acc = chunk_dot(wv[c], hv[c], acc);
    acc = wave_sum(acc);
    const float z = (use && row_ok) ? acc : __builtin_nanf("");
    if (lane == 0) {
      s_logit[j - j0] = z;
      a.slot_logit[j] = z;
    }
#pragma unroll
    for (int c = 0; c < NC; ++c) wv[c] = wn[c];
    use = use_n;
  }
  __syncthreads();
  if (wid == 0) fields_decide(a, s_logit, f, j0, K, lane);
}

template <bool WF32, bool HF32>
__global__ __launch_bounds__(kFieldThreads) void k_restricted_fields_lds(FieldArgs a) {
  constexpr int NB = WF32 ? 4 : 8;  // 512-wide chunks of a head row in flight per wave
  constexpr int WQ = WF32 ? 2 : 1;  // 16-byte loads per lane per chunk
  __shared__ float4 s_h[kFieldMaxD / 4];
  __shared__ float s_logit[kFieldMaxSlots];
  __shared__ uint32_t s_bits;
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int f = blockIdx.x;
  if (f == 0) fields_check(a, &s_bits, tid);
  if (f >= a.n_fields) return;
  const int j0 = a.slot_off[f], j1 = a.slot_off[f + 1];
  if (j0 < 0 || j1 > a.n_slots || j1 <= j0) {
    if (tid == 0) a.f_argmax[f] = -1;
    return;
  }
  const int r = a.field_row[f];
  const bool row_ok = r >= 0 && r < a.n_rows;
  const int K = j1 - j0;  // <= n_slots <= kFieldMaxSlots (host check)
  const int d = a.d;      // <= kFieldMaxD, a multiple of 32 (host checks)
  // the field's hidden row in LDS as fp32 (zeros for a bad row, whose logits are NaN)
  for (int k = 8 * tid; k < d; k += 8 * kFieldThreads) {
    float h[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    if (row_ok) load_h8<HF32>(a.H, (size_t)r * d + k, h);
    s_h[k / 4] = make_float4(h[0], h[1], h[2], h[3]);
    s_h[k / 4 + 1] = make_float4(h[4], h[5], h[6], h[7]);
  }
  __syncthreads();
  const int nch = (d + 511) / 512;
  for (int j = j0 + wid; j < j1; j += kFieldWaves) {
    const SlotRow s = slot_row<WF32>(a, j);
    float acc = 0.f;
    for (int c0 = 0; c0 < nch; c0 += NB) {
      uint4 wv[NB][WQ];
#pragma unroll
      for (int u = 0; u < NB; ++u) {
        const int k = 512 * (c0 + u) + 8 * lane;
        const uint4* wp = reinterpret_cast<const uint4*>(s.row + (size_t)k * (WF32 ? 4 : 2));
#pragma unroll
        for (int q = 0; q < WQ; ++q) wv[u][q] = (s.id_ok && k < d) ? wp[q] : make_uint4(0, 0, 0, 0);
      }
#pragma unroll
      for (int u = 0; u < NB; ++u) {
        const int k = 512 * (c0 + u) + 8 * lane;
        if (k < d) {
          const float4 x0 = s_h[k / 4], x1 = s_h[k / 4 + 1];
          const float h[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
          if constexpr (WF32)
            acc = chunk_dot_f32(wv[u][0], wv[u][1], h, acc);
          else
            acc = chunk_dot(wv[u][0], h, acc);
        }
      }
    }
    acc = wave_sum(acc);
    const float z = (s.use && row_ok) ? acc : __builtin_nanf("");
    if (lane == 0) {
      s_logit[j - j0] = z;
      a.slot_logit[j] = z;
    }
  }
  __syncthreads();
  if (wid == 0) fields_decide(a, s_logit, f, j0, K, lane);
}

}  // namespace

bool make_restricted_plan(const jet_restricted_problem* p, RestrictedPlan* pl) {
  const size_t elt = p->w_dtype == JET_BF16 ? 2 : 4;
  auto al = [](size_t x) { return (x + 255) & ~(size_t)255; };
  // d <= 16384 (the hidden row in registers, or in LDS), at most 4096 slots: one launch,
  // a workgroup per field, no workspace but the flag word
  pl->per_field = p->d <= kFieldMaxD && p->n_slots <= kFieldMaxSlots;
  if (pl->per_field) {
    pl->fused = false;
    pl->n_kg = 0;
    pl->off_wu = pl->off_z = 0;
    pl->off_flags = 0;
    pl->total = 256;
    return true;
  }
  // otherwise, bf16 head: k-split partials of Z, no gathered copy; fp32 head: the gathered
  // rows and Z
  pl->fused = p->w_dtype == JET_BF16;
  pl->n_kg = pl->fused ? (p->d + kRkTile - 1) / kRkTile : 1;
  size_t off = 0;
  pl->off_wu = off;
  if (!pl->fused) off += al((size_t)p->n_union * p->d * elt);
  pl->off_z = off;
  off += al((size_t)pl->n_kg * p->n_rows * p->n_union * 4);
  pl->off_flags = off;
  off += 256;
  pl->total = off;
  return true;
}

// fp32 head: clear the flags, gather the union rows, project them with the small-row fp32
// kernel's store epilogue into Z[row][u].
static hipError_t launch_restricted_f32(const jet_restricted_problem* p, const RestrictedPlan* pl,
                                        char* ws, int32_t* flags, float* Z, hipStream_t stream) {
  const int row_vec = (int)((size_t)p->d * 4 / 16);
  hipError_t e;
  hipLaunchKernelGGL(k_clear_flag, dim3(1), dim3(64), 0, stream, flags);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if (p->n_union > 0) {
    const int grid = p->n_union < 4096 ? p->n_union : 4096;
    hipLaunchKernelGGL(k_gather_rows, dim3(grid), dim3(256), 0, stream,
                       static_cast<const uint4*>(p->W), p->V, row_vec, p->union_ids, p->n_union,
                       reinterpret_cast<uint4*>(ws + pl->off_wu), flags);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  if (p->n_union > 0 && p->n_rows > 0)
    return launch_project_store_f32(reinterpret_cast<const float*>(ws + pl->off_wu), p->n_union,
                                    p->d, static_cast<const float*>(p->H), p->n_rows, Z, stream);
  return hipSuccess;
}

template <bool HF32>
static hipError_t launch_fields(const jet_restricted_problem* p, const jet_restricted_outputs* o,
                                int32_t* flags, hipStream_t stream) {
  const dim3 grid(p->n_fields > 0 ? p->n_fields : 1), block(kFieldThreads);
  FieldArgs a;
  a.W = p->W;
  a.V = p->V;
  a.d = p->d;
  a.ids = p->union_ids;
  a.n_union = p->n_union;
  a.H = p->H;
  a.n_rows = p->n_rows;
  a.field_row = p->field_row;
  a.slot_off = p->field_slot_off;
  a.slot_uidx = p->slot_uidx;
  a.n_fields = p->n_fields;
  a.n_slots = p->n_slots;
  a.T = p->T;
  a.slot_logit = o->slot_logit;
  a.slot_q = o->slot_q;
  a.f_argmax = o->field_argmax;
  a.flags = flags;
  if constexpr (HF32) {  // an fp32 head comes with fp32 hidden states (host check)
    if (p->w_dtype == JET_F32) {
      hipLaunchKernelGGL((k_restricted_fields_lds<true, true>), grid, block, 0, stream, a);
      return hipGetLastError();
    }
  }
  if (p->d <= 1024)
    hipLaunchKernelGGL((k_restricted_fields<HF32, 2>), grid, block, 0, stream, a);
  else if (p->d <= 2560)
    hipLaunchKernelGGL((k_restricted_fields<HF32, 5>), grid, block, 0, stream, a);
  else
    hipLaunchKernelGGL((k_restricted_fields_lds<false, HF32>), grid, block, 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_restricted(const jet_restricted_problem* p, const jet_restricted_outputs* o,
                             const RestrictedPlan* pl, char* ws, int32_t* flags,
                             hipStream_t stream) {
  if (pl->per_field)
    return p->h_dtype == JET_F32 ? launch_fields<true>(p, o, flags, stream)
                                 : launch_fields<false>(p, o, flags, stream);
  // the flag word is cleared by the first kernel (no memset, so the sequence stays
  // capturable) and set only by kernels after it
  hipError_t e;
  float* Z = reinterpret_cast<float*>(ws + pl->off_z);
  size_t part_stride = 0;
  int u_stride = 1, r_stride = p->n_union;
  if (pl->fused) {
    // one launch whatever the sizes: its workgroup 0 clears the flag word
    const int n_ut = (p->n_union + 31) / 32, n_rt = (p->n_rows + 31) / 32;
    const long long n_tiles = (long long)n_ut * n_rt * pl->n_kg;
    const int grid = n_tiles < 1 ? 1 : (n_tiles > 65536 ? 65536 : (int)n_tiles);
    if (p->h_dtype == JET_F32)
      hipLaunchKernelGGL(k_restricted_project<true>, dim3(grid), dim3(256), 0, stream,
                         static_cast<const uint16_t*>(p->W), p->V, p->d, p->union_ids, p->n_union,
                         p->H, p->n_rows, n_ut, n_rt, pl->n_kg, Z, flags);
    else
      hipLaunchKernelGGL(k_restricted_project<false>, dim3(grid), dim3(256), 0, stream,
                         static_cast<const uint16_t*>(p->W), p->V, p->d, p->union_ids, p->n_union,
                         p->H, p->n_rows, n_ut, n_rt, pl->n_kg, Z, flags);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    part_stride = (size_t)p->n_union * p->n_rows;
    u_stride = p->n_rows;
    r_stride = 1;
  } else {
    if ((e = launch_restricted_f32(p, pl, ws, flags, Z, stream)) != hipSuccess) return e;
  }
  if (p->n_fields > 0 || p->n_union > 0) {
    const int grid = p->n_fields > 0 ? (p->n_fields + 3) / 4 : 1;
    hipLaunchKernelGGL(k_field_softmax, dim3(grid), dim3(256), 0, stream, Z, pl->n_kg,
                       part_stride, u_stride, r_stride, p->n_rows, p->n_union, p->union_ids, p->V,
                       p->field_row, p->field_slot_off, p->slot_uidx, p->n_fields, p->n_slots,
                       p->T, o->slot_logit, o->slot_q, o->field_argmax, flags);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace jet
