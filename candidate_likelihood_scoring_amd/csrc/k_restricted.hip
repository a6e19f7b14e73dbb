// Restricted-vocabulary scoring (nimble "Parallel constrained scoring in MLX", Execution
// steps 5-6): gather only the allowed head rows, project the hidden states onto their
// union, and let each field take a softmax over its own allowed ids at temperature T.
//
//   k_gather_rows : Wu[j, :] = W[union_ids[j], :], a bit-exact copy of each row with
//                   16-byte coalesced loads/stores (one workgroup per union row).
//   projection    : Z[r, j] = <H[r], Wu[j]> with the small-row matrix-core kernel's store
//                   epilogue (fp32 accumulation; fp32 H split into bf16 hi + lo).
//   k_field_softmax: one wave per field: slot_logit = Z[field_row, slot_uidx], a = logit/T,
//                   q = softmax(a) over the field's slots, argmax = lowest index among the
//                   exact maxima of a.
#include "jet_internal.h"

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

__global__ __launch_bounds__(256) void k_field_softmax(
    const float* __restrict__ Z, int n_rows, int n_union, const int* __restrict__ field_row,
    const int* __restrict__ slot_off, const int* __restrict__ slot_uidx, int n_fields, int n_slots,
    float T, float* __restrict__ slot_logit, float* __restrict__ slot_q, int* __restrict__ f_argmax,
    int32_t* __restrict__ flags) {
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
    if (row_ok && u >= 0 && u < n_union) z = Z[(size_t)r * n_union + u];
    else bad = true;
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

}  // namespace

bool make_restricted_plan(const jet_restricted_problem* p, RestrictedPlan* pl) {
  const size_t elt = p->w_dtype == JET_BF16 ? 2 : 4;
  auto al = [](size_t x) { return (x + 255) & ~(size_t)255; };
  pl->hilo = p->w_dtype == JET_BF16 && p->h_dtype == JET_F32;
  size_t off = 0;
  pl->off_wu = off;
  off += al((size_t)p->n_union * p->d * elt);
  pl->off_hhi = off;
  if (pl->hilo) off += al((size_t)p->n_rows * p->d * 2);
  pl->off_hlo = off;
  if (pl->hilo) off += al((size_t)p->n_rows * p->d * 2);
  pl->off_z = off;
  off += al((size_t)p->n_rows * p->n_union * 4);
  pl->off_flags = off;
  off += 256;
  pl->total = off;
  return true;
}

hipError_t launch_restricted(const jet_restricted_problem* p, const jet_restricted_outputs* o,
                             const RestrictedPlan* pl, char* ws, int32_t* flags,
                             hipStream_t stream) {
  const size_t elt = p->w_dtype == JET_BF16 ? 2 : 4;
  const int row_vec = (int)((size_t)p->d * elt / 16);
  // flags: cleared by a one-thread kernel (no memset, so the sequence stays capturable)
  hipError_t e;
  hipLaunchKernelGGL(k_clear_flag, dim3(1), dim3(64), 0, stream, flags);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if (p->n_union > 0) {
    int grid = p->n_union < 4096 ? p->n_union : 4096;
    hipLaunchKernelGGL(k_gather_rows, dim3(grid), dim3(256), 0, stream,
                       static_cast<const uint4*>(p->W), p->V, row_vec, p->union_ids, p->n_union,
                       reinterpret_cast<uint4*>(ws + pl->off_wu), flags);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  float* Z = reinterpret_cast<float*>(ws + pl->off_z);
  if (p->n_union > 0 && p->n_rows > 0) {
    if (p->w_dtype == JET_BF16) {
      const uint16_t* hhi;
      const uint16_t* hlo = nullptr;
      if (pl->hilo) {
        uint16_t* hi = reinterpret_cast<uint16_t*>(ws + pl->off_hhi);
        uint16_t* lo = reinterpret_cast<uint16_t*>(ws + pl->off_hlo);
        if ((e = launch_split(static_cast<const float*>(p->H), (long long)p->n_rows * p->d, hi, lo,
                              stream)) != hipSuccess)
          return e;
        hhi = hi;
        hlo = lo;
      } else {
        hhi = static_cast<const uint16_t*>(p->H);
      }
      e = launch_project_store_bf16(reinterpret_cast<const uint16_t*>(ws + pl->off_wu), p->n_union,
                                    p->d, hhi, hlo, p->n_rows, Z, stream);
    } else {
      e = launch_project_store_f32(reinterpret_cast<const float*>(ws + pl->off_wu), p->n_union,
                                   p->d, static_cast<const float*>(p->H), p->n_rows, Z, stream);
    }
    if (e != hipSuccess) return e;
  }
  if (p->n_fields > 0) {
    hipLaunchKernelGGL(k_field_softmax, dim3((p->n_fields + 3) / 4), dim3(256), 0, stream, Z,
                       p->n_rows, p->n_union, p->field_row, p->field_slot_off, p->slot_uidx,
                       p->n_fields, p->n_slots, p->T, o->slot_logit, o->slot_q, o->field_argmax,
                       flags);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace jet
