// Operand staging and target bucketing, one launch before the projection.
//
//  * fp32 H with a bf16 head: H = hi + lo, hi = bf16_rne(H), lo = bf16_rne(H - hi).  The
//    subtraction is exact in fp32, so hi + lo differs from H by at most one bf16 rounding
//    of the residual (about 2^-17 relative).
//  * Target bucketing: each scored token k belongs to the projection tile that holds
//    (tok_row[k], tok_target[k]).  A counting sort groups tokens by
//    key = (row / row_tile) * n_groups + target / vgroup, so the epilogue of that tile
//    finds its targets without scanning all tokens.  The order of tokens inside a bucket
//    does not matter: every token writes only its own logit slot.
//    Indices are validated here: an out-of-range row or target is never bucketed (its
//    logit stays NaN) and raises a device flag.
#include "jet_internal.h"

namespace jet {
namespace {

constexpr int kPrepThreads = 1024;

__device__ inline void split_range(const float* __restrict__ H, long long n, uint16_t* __restrict__ hi,
                                   uint16_t* __restrict__ lo, long long i0, long long stride) {
  for (long long i = i0; i < n; i += stride) {
    const float x = H[i];
    const uint16_t h = f32_to_bf16_rne(x);
    hi[i] = h;
    lo[i] = f32_to_bf16_rne(x - bf16_to_f32(h));
  }
}

__device__ inline int ld_agent(const int* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__global__ __launch_bounds__(kPrepThreads) void k_prep(
    const float* __restrict__ H, long long n_h, uint16_t* __restrict__ hhi,
    uint16_t* __restrict__ hlo, int n_split_blocks, const int* __restrict__ tok_row,
    const int* __restrict__ tok_target, int n_tok, int n_rows, int V, int row_tile, int vgroup,
    int n_groups, long long n_buckets, int* __restrict__ b_count, int* __restrict__ b_off,
    int* __restrict__ b_tok, int* __restrict__ b_pos, float* __restrict__ z_tgt,
    int32_t* __restrict__ flags) {
  const int tid = threadIdx.x;
  if ((int)blockIdx.x < n_split_blocks) {
    split_range(H, n_h, hhi, hlo, (long long)blockIdx.x * kPrepThreads + tid,
                (long long)n_split_blocks * kPrepThreads);
    return;
  }
  __shared__ int sh[kPrepThreads];
  __shared__ uint32_t sflags;
  if (tid == 0) sflags = 0u;
  for (long long i = tid; i <= n_buckets; i += kPrepThreads) b_count[i] = 0;
  __threadfence();
  __syncthreads();
  uint32_t my_flags = 0u;
  for (int k = tid; k < n_tok; k += kPrepThreads) {
    z_tgt[k] = __builtin_nanf("");
    const int r = tok_row ? tok_row[k] : k;
    const int y = tok_target[k];
    bool ok = true;
    if (r < 0 || r >= n_rows) {
      ok = false;
      my_flags |= JET_FLAG_BAD_ROW;
    }
    if (y < 0 || y >= V) {
      ok = false;
      my_flags |= JET_FLAG_BAD_TARGET;
    }
    int pos = -1;
    if (ok) {
      const long long key = (long long)(r / row_tile) * n_groups + y / vgroup;
      pos = atomicAdd(&b_count[key], 1);
    }
    b_pos[k] = pos;
  }
  if (my_flags) atomicOr(&sflags, my_flags);
  __threadfence();
  __syncthreads();
  // exclusive scan of the counts
  const long long per = (n_buckets + kPrepThreads - 1) / kPrepThreads;
  const long long lo = (long long)tid * per;
  const long long hi = lo + per < n_buckets ? lo + per : n_buckets;
  int sum = 0;
  for (long long i = lo; i < hi; ++i) sum += ld_agent(&b_count[i]);
  sh[tid] = sum;
  __syncthreads();
  for (int off = 1; off < kPrepThreads; off <<= 1) {
    const int v = tid >= off ? sh[tid - off] : 0;
    __syncthreads();
    sh[tid] += v;
    __syncthreads();
  }
  int run = tid ? sh[tid - 1] : 0;
  for (long long i = lo; i < hi; ++i) {
    b_off[i] = run;
    run += ld_agent(&b_count[i]);
  }
  if (tid == kPrepThreads - 1) b_off[n_buckets] = sh[kPrepThreads - 1];
  __threadfence();
  __syncthreads();
  for (int k = tid; k < n_tok; k += kPrepThreads) {
    const int pos = b_pos[k];
    if (pos < 0) continue;
    const int r = tok_row ? tok_row[k] : k;
    const long long key = (long long)(r / row_tile) * n_groups + tok_target[k] / vgroup;
    b_tok[ld_agent(&b_off[key]) + pos] = k;
  }
  if (tid == 0 && flags) flags[0] = (int32_t)sflags;
}

// Counting sort in LDS when the buckets fit (one workgroup): counts, exclusive scan and
// offsets never leave LDS until the final offsets are stored.
constexpr int kLdsBuckets = 12288;

__global__ __launch_bounds__(kPrepThreads) void k_bucket_lds(
    const int* __restrict__ tok_row, const int* __restrict__ tok_target, int n_tok, int n_rows,
    int V, int row_tile, int vgroup, int n_groups, int n_buckets, int* __restrict__ b_off,
    int* __restrict__ b_tok, int* __restrict__ b_pos, float* __restrict__ z_tgt,
    int32_t* __restrict__ flags) {
  __shared__ int cnt[kLdsBuckets + 1];
  __shared__ int sh[kPrepThreads];
  __shared__ uint32_t sflags;
  const int tid = threadIdx.x;
  if (tid == 0) sflags = 0u;
  for (int i = tid; i <= n_buckets; i += kPrepThreads) cnt[i] = 0;
  __syncthreads();
  uint32_t my_flags = 0u;
  for (int k = tid; k < n_tok; k += kPrepThreads) {
    z_tgt[k] = __builtin_nanf("");
    const int r = tok_row ? tok_row[k] : k;
    const int y = tok_target[k];
    bool ok = true;
    if (r < 0 || r >= n_rows) {
      ok = false;
      my_flags |= JET_FLAG_BAD_ROW;
    }
    if (y < 0 || y >= V) {
      ok = false;
      my_flags |= JET_FLAG_BAD_TARGET;
    }
    b_pos[k] = ok ? atomicAdd(&cnt[(r / row_tile) * n_groups + y / vgroup], 1) : -1;
  }
  if (my_flags) atomicOr(&sflags, my_flags);
  __syncthreads();
  const int per = (n_buckets + kPrepThreads - 1) / kPrepThreads;
  const int lo = tid * per, hi = min(lo + per, n_buckets);
  int sum = 0;
  for (int i = lo; i < hi; ++i) sum += cnt[i];
  sh[tid] = sum;
  __syncthreads();
  for (int off = 1; off < kPrepThreads; off <<= 1) {
    const int v = tid >= off ? sh[tid - off] : 0;
    __syncthreads();
    sh[tid] += v;
    __syncthreads();
  }
  int run = tid ? sh[tid - 1] : 0;
  for (int i = lo; i < hi; ++i) {
    const int c = cnt[i];
    cnt[i] = run;
    b_off[i] = run;
    run += c;
  }
  if (tid == kPrepThreads - 1) b_off[n_buckets] = sh[kPrepThreads - 1];
  __syncthreads();
  for (int k = tid; k < n_tok; k += kPrepThreads) {
    const int pos = b_pos[k];
    if (pos < 0) continue;
    const int r = tok_row ? tok_row[k] : k;
    b_tok[cnt[(r / row_tile) * n_groups + tok_target[k] / vgroup] + pos] = k;
  }
  if (tid == 0 && flags) flags[0] = (int32_t)sflags;
}

__global__ __launch_bounds__(256) void k_split(const float* __restrict__ H, long long n,
                                               uint16_t* __restrict__ hi, uint16_t* __restrict__ lo) {
  split_range(H, n, hi, lo, (long long)blockIdx.x * 256 + threadIdx.x, (long long)gridDim.x * 256);
}

int split_blocks(long long n, int threads) {
  long long b = (n + threads - 1) / threads;
  if (b > 2048) b = 2048;
  return (int)b;
}

}  // namespace

hipError_t launch_prep(const ScoreArgs& a) {
  const jet_problem* p = a.p;
  const Plan& pl = *a.plan;
  char* ws = a.ws;
  const long long n_h = (long long)p->n_rows * p->d;
  const bool need_split = pl.hilo && !pl.stream;
  if (!need_split && pl.n_buckets <= kLdsBuckets) {
    hipLaunchKernelGGL(k_bucket_lds, dim3(1), dim3(kPrepThreads), 0, a.stream, p->tok_row,
                       p->tok_target, p->n_tok, p->n_rows, p->V, pl.row_tile, pl.vgroup,
                       pl.n_vgroups, (int)pl.n_buckets, reinterpret_cast<int*>(ws + pl.off_boff),
                       reinterpret_cast<int*>(ws + pl.off_btok),
                       reinterpret_cast<int*>(ws + pl.off_bpos),
                       reinterpret_cast<float*>(ws + pl.off_ztgt), a.flags);
    return hipGetLastError();
  }
  const int nsb = need_split ? split_blocks(n_h, kPrepThreads) : 0;
  hipLaunchKernelGGL(k_prep, dim3(nsb + 1), dim3(kPrepThreads), 0, a.stream,
                     static_cast<const float*>(p->H), n_h,
                     reinterpret_cast<uint16_t*>(ws + pl.off_hhi),
                     reinterpret_cast<uint16_t*>(ws + pl.off_hlo), nsb, p->tok_row, p->tok_target,
                     p->n_tok, p->n_rows, p->V, pl.row_tile, pl.vgroup, pl.n_vgroups, pl.n_buckets,
                     reinterpret_cast<int*>(ws + pl.off_bcount), reinterpret_cast<int*>(ws + pl.off_boff),
                     reinterpret_cast<int*>(ws + pl.off_btok), reinterpret_cast<int*>(ws + pl.off_bpos),
                     reinterpret_cast<float*>(ws + pl.off_ztgt), a.flags);
  return hipGetLastError();
}

hipError_t launch_split(const float* H, long long n_elems, uint16_t* hi, uint16_t* lo,
                        hipStream_t stream) {
  if (n_elems <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_split, dim3(split_blocks(n_elems, 256)), dim3(256), 0, stream, H, n_elems, hi, lo);
  return hipGetLastError();
}

}  // namespace jet
