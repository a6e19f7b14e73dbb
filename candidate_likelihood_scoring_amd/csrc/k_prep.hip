// Operand staging and target bucketing, one launch before the projection.
//
//  * fp32 H with a bf16 head: H = hi + lo, hi = bf16_rne(H), lo = bf16_rne(H - hi).  The
//    subtraction is exact in fp32, so hi + lo differs from H by at most one bf16 rounding
//    of the residual (about 2^-17 relative).
//  * Fewer rows than one tile of the tiled kernel: the kernel runs one whole row tile, so
//    the split planes (fp32 H) or a copy of H (bf16 H) get zero rows appended up to it; the
//    padding rows' partials are never merged.
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

constexpr int kPrepThreads = 1024;  // = kScanThreads: k_bucket_lds uses block_exscan

__device__ inline void split_range(const float* __restrict__ H, long long n, long long n_out,
                                   uint16_t* __restrict__ hi, uint16_t* __restrict__ lo,
                                   long long i0, long long stride) {
  for (long long i = i0; i < n_out; i += stride) {
    const float x = i < n ? H[i] : 0.f;
    const uint16_t h = f32_to_bf16_rne(x);
    hi[i] = h;
    lo[i] = f32_to_bf16_rne(x - bf16_to_f32(h));
  }
}

// Counting sort over many buckets (more than fit in LDS), as a chain of grid-wide launches:
// clear the counts, count (each token takes its slot in its bucket with an atomic add),
// sum the counts per tile of kScanTile buckets, scan the tile sums (one workgroup), scan
// inside each tile from its tile offset, scatter.  Every step is exact integer work, so the
// offsets do not depend on scheduling; only the order of tokens inside a bucket does, which
// nothing depends on.
constexpr int kScanThreads = 1024, kScanPer = 8, kScanTile = kScanThreads * kScanPer;
static_assert(kPrepThreads == kScanThreads, "k_bucket_lds scans with block_exscan");

__global__ __launch_bounds__(256) void k_bk_clear(int* __restrict__ b_count, long long n,
                                                  int32_t* __restrict__ flags) {
  for (long long i = (long long)blockIdx.x * 256 + threadIdx.x; i < n; i += (long long)gridDim.x * 256)
    b_count[i] = 0;
  if (blockIdx.x == 0 && threadIdx.x == 0 && flags) flags[0] = 0;
}

__global__ __launch_bounds__(256) void k_bk_count(
    const int* __restrict__ tok_row, const int* __restrict__ tok_target, int n_tok, int n_rows,
    int V, int row_tile, int vgroup, int n_groups, int* __restrict__ b_count,
    int* __restrict__ b_pos, float* __restrict__ z_tgt, int32_t* __restrict__ flags) {
  const int k = blockIdx.x * 256 + threadIdx.x;
  if (k >= n_tok) return;
  z_tgt[k] = __builtin_nanf("");
  const int r = tok_row ? tok_row[k] : k;
  const int y = tok_target[k];
  uint32_t bad = 0u;
  if (r < 0 || r >= n_rows) bad |= JET_FLAG_BAD_ROW;
  if (y < 0 || y >= V) bad |= JET_FLAG_BAD_TARGET;
  if (bad) {
    flag_or(flags, bad);
    b_pos[k] = -1;
    return;
  }
  b_pos[k] = atomicAdd(&b_count[(long long)(r / row_tile) * n_groups + y / vgroup], 1);
}

// block-wide exclusive scan of one value per thread (1024 threads); returns the exclusive
// prefix and writes the block total to *total
__device__ inline int block_exscan(int v, int* sh, int* total) {
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  int x = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int y = __shfl_up(x, off);
    if (lane >= off) x += y;
  }
  if (lane == 63) sh[w] = x;
  __syncthreads();
  if (tid < 64) {
    int t = tid < kScanThreads / 64 ? sh[tid] : 0;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int y = __shfl_up(t, off);
      if (lane >= off) t += y;
    }
    if (tid < kScanThreads / 64) sh[64 + tid] = t;
  }
  __syncthreads();
  const int before = w ? sh[64 + w - 1] : 0;
  *total = sh[64 + kScanThreads / 64 - 1];
  return before + x - v;
}

__global__ __launch_bounds__(kScanThreads) void k_bk_tile_sums(const int* __restrict__ b_count,
                                                               long long n, int* __restrict__ tile_sum) {
  __shared__ int sh[128];
  const long long base = (long long)blockIdx.x * kScanTile + (long long)threadIdx.x * kScanPer;
  int v = 0;
#pragma unroll
  for (int j = 0; j < kScanPer; ++j)
    if (base + j < n) v += b_count[base + j];
  int total;
  block_exscan(v, sh, &total);
  if (threadIdx.x == 0) tile_sum[blockIdx.x] = total;
}

// exclusive scan of up to kScanTile tile sums, in place (one workgroup)
__global__ __launch_bounds__(kScanThreads) void k_bk_scan_tiles(int* __restrict__ tile_sum,
                                                                int n_tiles) {
  __shared__ int sh[128];
  const int base = threadIdx.x * kScanPer;
  int v[kScanPer], sum = 0;
#pragma unroll
  for (int j = 0; j < kScanPer; ++j) {
    v[j] = base + j < n_tiles ? tile_sum[base + j] : 0;
    sum += v[j];
  }
  int total;
  int run = block_exscan(sum, sh, &total);
#pragma unroll
  for (int j = 0; j < kScanPer; ++j)
    if (base + j < n_tiles) {
      tile_sum[base + j] = run;
      run += v[j];
    }
}

__global__ __launch_bounds__(kScanThreads) void k_bk_offsets(const int* __restrict__ b_count,
                                                             long long n_buckets,
                                                             const int* __restrict__ tile_off,
                                                             int* __restrict__ b_off) {
  __shared__ int sh[128];
  const long long base = (long long)blockIdx.x * kScanTile + (long long)threadIdx.x * kScanPer;
  int v[kScanPer], sum = 0;
#pragma unroll
  for (int j = 0; j < kScanPer; ++j) {
    v[j] = base + j < n_buckets ? b_count[base + j] : 0;
    sum += v[j];
  }
  int total;
  int run = tile_off[blockIdx.x] + block_exscan(sum, sh, &total);
#pragma unroll
  for (int j = 0; j < kScanPer; ++j)
    if (base + j < n_buckets) {
      b_off[base + j] = run;
      run += v[j];
    }
  if (blockIdx.x == gridDim.x - 1 && threadIdx.x == 0) b_off[n_buckets] = tile_off[blockIdx.x] + total;
}

__global__ __launch_bounds__(256) void k_bk_scatter(
    const int* __restrict__ tok_row, const int* __restrict__ tok_target, int n_tok,
    int row_tile, int vgroup, int n_groups, const int* __restrict__ b_off,
    const int* __restrict__ b_pos, int* __restrict__ b_tok) {
  const int k = blockIdx.x * 256 + threadIdx.x;
  if (k >= n_tok) return;
  const int pos = b_pos[k];
  if (pos < 0) return;
  const int r = tok_row ? tok_row[k] : k;
  b_tok[b_off[(long long)(r / row_tile) * n_groups + tok_target[k] / vgroup] + pos] = k;
}

// Counting sort in LDS when the buckets fit (one workgroup, 128 KB of counts): counts,
// exclusive scan and offsets never leave LDS until the final offsets are stored.
constexpr int kLdsBuckets = 32768;

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
  int total;
  int run = block_exscan(sum, sh, &total);  // wave scans and one scan of the wave totals
  for (int i = lo; i < hi; ++i) {  // each thread's contiguous range, in LDS only
    const int c = cnt[i];
    cnt[i] = run;
    run += c;
  }
  if (tid == 0) cnt[n_buckets] = total;
  __syncthreads();
  // offsets stored with consecutive threads on consecutive buckets (a store per bucket
  // from each thread's own range touched a cache line per lane)
  for (int i = tid; i <= n_buckets; i += kPrepThreads) b_off[i] = cnt[i];
  for (int k = tid; k < n_tok; k += kPrepThreads) {
    const int pos = b_pos[k];
    if (pos < 0) continue;
    const int r = tok_row ? tok_row[k] : k;
    b_tok[cnt[(r / row_tile) * n_groups + tok_target[k] / vgroup] + pos] = k;
  }
  if (tid == 0 && flags) flags[0] = (int32_t)sflags;
}

__global__ __launch_bounds__(256) void k_split(const float* __restrict__ H, long long n,
                                               long long n_out, uint16_t* __restrict__ hi,
                                               uint16_t* __restrict__ lo) {
  split_range(H, n, n_out, hi, lo, (long long)blockIdx.x * 256 + threadIdx.x,
              (long long)gridDim.x * 256);
}

// bf16 H with fewer rows than one tile of the tiled kernel: copied whole, then zero rows up
// to the tile (16-byte chunks: n16 copied, n16_out in all).
__global__ __launch_bounds__(256) void k_pad_rows(const u32x4* __restrict__ src, long long n16,
                                                  long long n16_out, u32x4* __restrict__ dst) {
  for (long long i = (long long)blockIdx.x * 256 + threadIdx.x; i < n16_out;
       i += (long long)gridDim.x * 256)
    dst[i] = i < n16 ? src[i] : u32x4{0u, 0u, 0u, 0u};
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
  if (pl.hilo && !pl.stream) {
    const hipError_t e = launch_split(static_cast<const float*>(p->H), (long long)p->n_rows * p->d,
                                      (long long)pl.rows_k * p->d,
                                      reinterpret_cast<uint16_t*>(ws + pl.off_hhi),
                                      reinterpret_cast<uint16_t*>(ws + pl.off_hlo), a.stream);
    if (e != hipSuccess) return e;
  }
  if (pl.pad_h) {  // bf16 H: d is a multiple of 128, so rows are whole 16-byte chunks
    const long long n16 = (long long)p->n_rows * p->d / 8, n16_out = (long long)pl.rows_k * p->d / 8;
    hipLaunchKernelGGL(k_pad_rows, dim3(split_blocks(n16_out, 256)), dim3(256), 0, a.stream,
                       static_cast<const u32x4*>(p->H), n16, n16_out,
                       reinterpret_cast<u32x4*>(ws + pl.off_hpad));
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  int* b_count = reinterpret_cast<int*>(ws + pl.off_bcount);
  int* b_tile = reinterpret_cast<int*>(ws + pl.off_btile);
  int* b_off = reinterpret_cast<int*>(ws + pl.off_boff);
  int* b_tok = reinterpret_cast<int*>(ws + pl.off_btok);
  int* b_pos = reinterpret_cast<int*>(ws + pl.off_bpos);
  float* z_tgt = reinterpret_cast<float*>(ws + pl.off_ztgt);
  if (pl.n_buckets <= kLdsBuckets) {
    hipLaunchKernelGGL(k_bucket_lds, dim3(1), dim3(kPrepThreads), 0, a.stream, p->tok_row,
                       p->tok_target, p->n_tok, p->n_rows, p->V, pl.row_tile, pl.vgroup,
                       pl.n_vgroups, (int)pl.n_buckets, b_off, b_tok, b_pos, z_tgt, a.flags);
    return hipGetLastError();
  }
  static_assert(kScanTile == kBucketScanTile && kScanTile == kBucketMaxTiles, "scan shape");
  const long long nb = pl.n_buckets;
  const int n_tiles = (int)pl.n_btiles;  // <= kBucketMaxTiles, checked by the caller
  const int tok_blocks = (p->n_tok + 255) / 256;
  hipLaunchKernelGGL(k_bk_clear, dim3((unsigned)std::min<long long>((nb + 256) / 256, 4096)),
                     dim3(256), 0, a.stream, b_count, nb + 1, a.flags);
  if (tok_blocks > 0)
    hipLaunchKernelGGL(k_bk_count, dim3(tok_blocks), dim3(256), 0, a.stream, p->tok_row,
                       p->tok_target, p->n_tok, p->n_rows, p->V, pl.row_tile, pl.vgroup,
                       pl.n_vgroups, b_count, b_pos, z_tgt, a.flags);
  hipLaunchKernelGGL(k_bk_tile_sums, dim3(n_tiles), dim3(kScanThreads), 0, a.stream, b_count, nb,
                     b_tile);
  hipLaunchKernelGGL(k_bk_scan_tiles, dim3(1), dim3(kScanThreads), 0, a.stream, b_tile, n_tiles);
  hipLaunchKernelGGL(k_bk_offsets, dim3(n_tiles), dim3(kScanThreads), 0, a.stream, b_count, nb,
                     b_tile, b_off);
  if (tok_blocks > 0)
    hipLaunchKernelGGL(k_bk_scatter, dim3(tok_blocks), dim3(256), 0, a.stream, p->tok_row,
                       p->tok_target, p->n_tok, pl.row_tile, pl.vgroup, pl.n_vgroups, b_off, b_pos,
                       b_tok);
  return hipGetLastError();
}

hipError_t launch_split(const float* H, long long n_elems, long long n_out, uint16_t* hi,
                        uint16_t* lo, hipStream_t stream) {
  if (n_out <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_split, dim3(split_blocks(n_out, 256)), dim3(256), 0, stream, H, n_elems,
                     n_out, hi, lo);
  return hipGetLastError();
}

}  // namespace jet
