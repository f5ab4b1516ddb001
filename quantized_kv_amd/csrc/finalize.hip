// Per-record aggregation and output comparison kernels.
//
// Heatmap: "Catnip Week 10 KV Cache Attention Study", Figure 2 — the 6x16 temporal map, each query
// frame's 16 key-frame masses averaged over its sampled rows (rows sum to 100 %), and the per-layer
// maps of Figure 8. Histograms: the distributions of support and region mass over the rows of a record
// (Figure 5). Comparison: "KV residual window" (relative L2 of the attention output) and the
// MiniCPM5-2B predictor study, section 0 (recall@32).
#include "kvprof_internal.h"

namespace kvp {
namespace {

// One thread per (batch, head, group, frame): mean over the rows of that group, in row order.
// One workgroup per (batch, query head) when n_groups * n_frames <= 256: the head's frame masses and
// the rows' groups pass through LDS in chunks of 128 rows, and thread (group, frame) adds its group's
// rows in row order, the same order as heatmap_kernel (so the same sums).
constexpr int kHmChunk = 128;
__global__ __launch_bounds__(256) void heatmap_block_kernel(const float* __restrict__ fm, const int* __restrict__ row_group,
                                                            int nq, int ng, int nf, float* __restrict__ hm) {
  __shared__ float tile[kHmChunk * KVPROF_MAX_FRAMES];
  __shared__ int tg[kHmChunk];
  const long long bh = blockIdx.x;
  const float* base = fm + bh * (long long)nq * nf;
  const int t = threadIdx.x;
  const bool act = t < ng * nf;
  const int gq = act ? t / nf : 0, f = act ? t - gq * nf : 0;
  float s = 0.f;
  int cnt = 0;
  for (int i0 = 0; i0 < nq; i0 += kHmChunk) {
    const int nr = min(kHmChunk, nq - i0);
    __syncthreads();  // the previous chunk has been read
    for (int e = t; e < nr * nf; e += blockDim.x) tile[e] = base[(long long)i0 * nf + e];
    for (int e = t; e < nr; e += blockDim.x) tg[e] = row_group[i0 + e];
    __syncthreads();
    if (act)
      for (int i = 0; i < nr; ++i)
        if (tg[i] == gq) {
          s += tile[i * nf + f];
          ++cnt;
        }
  }
  if (act) hm[bh * ng * nf + t] = cnt ? s / (float)cnt : 0.f;
}

__global__ void heatmap_kernel(const float* __restrict__ fm, const int* __restrict__ row_group,
                               int n_batch, int hq, int nq, int ng, int nf, float* __restrict__ hm) {
  long long total = (long long)n_batch * hq * ng * nf;
  for (long long t = blockIdx.x * (long long)blockDim.x + threadIdx.x; t < total;
       t += (long long)gridDim.x * blockDim.x) {
    int f = (int)(t % nf);
    int gq = (int)((t / nf) % ng);
    long long bh = t / ((long long)nf * ng);
    const float* base = fm + bh * nq * nf;
    float s = 0.f;
    int cnt = 0;
    for (int i = 0; i < nq; ++i) {
      if (row_group[i] == gq) {
        s += base[(long long)i * nf + f];
        ++cnt;
      }
    }
    hm[t] = cnt ? s / (float)cnt : 0.f;
  }
}

// Mean over the query heads of each (batch, group, frame), in head order.
__global__ void heatmap_mean_kernel(const float* __restrict__ hm, int n_batch, int hq, int ng, int nf,
                                    float* __restrict__ out) {
  long long total = (long long)n_batch * ng * nf;
  for (long long t = blockIdx.x * (long long)blockDim.x + threadIdx.x; t < total;
       t += (long long)gridDim.x * blockDim.x) {
    long long b = t / ((long long)ng * nf);
    long long gf = t % ((long long)ng * nf);
    float s = 0.f;
    for (int h = 0; h < hq; ++h) s += hm[(b * hq + h) * ng * nf + gf];
    out[t] = s / (float)hq;
  }
}

__device__ __forceinline__ int bin100(float x, int bins) {
  int bn = (int)floorf(x * (float)bins);
  return bn < 0 ? 0 : (bn >= bins ? bins - 1 : bn);
}

// Workgroup (record b, chunk c) counts rows [c*kHistRows, (c+1)*kHistRows) of record b into an LDS
// histogram, then adds its nonzero bins to the record's histogram. Integer atomics only, so the
// counts do not depend on the order.
constexpr int kHistRows = 2048;
constexpr int kHistMaxWords = 9 * 1024;  // (1 + KVPROF_MAX_REGIONS) histograms of <= 1024 bins
__global__ __launch_bounds__(256) void hist_kernel(const float* __restrict__ support, const float* __restrict__ region,
                                                   int rows_per_b, int nreg, int bins, unsigned* __restrict__ hist) {
  __shared__ unsigned h[kHistMaxWords];
  const int nw = (1 + nreg) * bins;
  const int chunks = (rows_per_b + kHistRows - 1) / kHistRows;
  const long long b = blockIdx.x / chunks;
  for (int i = threadIdx.x; i < nw; i += blockDim.x) h[i] = 0u;
  __syncthreads();
  const int r0 = (int)(blockIdx.x % chunks) * kHistRows, r1 = min(rows_per_b, r0 + kHistRows);
  for (int r = r0 + threadIdx.x; r < r1; r += blockDim.x) {
    const long long t = b * rows_per_b + r;
    atomicAdd(&h[bin100(support[t], bins)], 1u);
    for (int q = 0; q < nreg; ++q) atomicAdd(&h[(1 + q) * bins + bin100(region[t * nreg + q], bins)], 1u);
  }
  __syncthreads();
  unsigned* hb = hist + b * (long long)nw;
  for (int i = threadIdx.x; i < nw; i += blockDim.x)
    if (h[i]) atomicAdd(&hb[i], h[i]);
}

__global__ void zero_u32_kernel(unsigned* p, long long n) {
  for (long long t = blockIdx.x * (long long)blockDim.x + threadIdx.x; t < n;
       t += (long long)gridDim.x * blockDim.x)
    p[t] = 0u;
}

// One wave per row: squared norms in float64, recall from the two index lists.
__global__ __launch_bounds__(64) void compare_kernel(const float* __restrict__ oq, const float* __restrict__ oref,
                                                     const int* __restrict__ tq, const int* __restrict__ tref,
                                                     long long rows, int d, float* __restrict__ rel,
                                                     float* __restrict__ recall, double* __restrict__ part) {
  const int lane = threadIdx.x;
  for (long long rrow = blockIdx.x; rrow < rows; rrow += gridDim.x) {
    double dd = 0.0, nn = 0.0;
    for (int c = lane; c < d; c += 64) {
      double a = oq[rrow * d + c], bb = oref[rrow * d + c];
      dd += (a - bb) * (a - bb);
      nn += bb * bb;
    }
    for (int o = 32; o >= 1; o >>= 1) {
      dd += __shfl_xor(dd, o);
      nn += __shfl_xor(nn, o);
    }
    int hit = 0;
    if (tq && tref && lane < 32) {
      int x = tq[rrow * 32 + lane];
      if (x >= 0)
        for (int q = 0; q < 32; ++q) hit += (tref[rrow * 32 + q] == x);
    }
    for (int o = 32; o >= 1; o >>= 1) hit += __shfl_xor(hit, o);
    if (lane == 0) {
      rel[rrow] = (float)(nn > 0 ? sqrt(dd / nn) : 0.0);
      if (recall) recall[rrow] = (float)hit / 32.f;
      part[2 * rrow] = dd;
      part[2 * rrow + 1] = nn;
    }
  }
}

// Single block, fixed order: thread t sums rows t, t + 256, ... in turn, then thread 0 adds the 256
// partial sums in order (deterministic).
__global__ __launch_bounds__(256) void compare_sum_kernel(const double* __restrict__ part, long long rows,
                                                          double* __restrict__ sums) {
  __shared__ double sd[256], sn[256];
  const int t = threadIdx.x;
  double a = 0.0, b = 0.0;
#pragma unroll 8  // loads issued ahead; the additions keep their order
  for (long long i = t; i < rows; i += 256) {  // thread t sums rows t, t + 256, ... (coalesced)
    a += part[2 * i];
    b += part[2 * i + 1];
  }
  sd[t] = a;
  sn[t] = b;
  __syncthreads();
  if (t == 0) {
    double x = 0.0, y = 0.0;
    for (int i = 0; i < 256; ++i) {
      x += sd[i];
      y += sn[i];
    }
    sums[0] = x;
    sums[1] = y;
  }
}

inline unsigned grid_for(long long n, int block) {
  long long g = (n + block - 1) / block;
  if (g < 1) g = 1;
  return (unsigned)(g > 65536 ? 65536 : g);
}

}  // namespace

hipError_t launch_heatmap(const float* frame_mass, const int* row_group, int n_batch, int hq, int nq,
                          int n_groups, int n_frames, float* heatmap, float* heatmap_mean,
                          hipStream_t s) {
  long long n = (long long)n_batch * hq * n_groups * n_frames;
  if (n == 0) return hipSuccess;
  if ((long long)n_groups * n_frames <= 256)
    hipLaunchKernelGGL(heatmap_block_kernel, dim3((unsigned)((long long)n_batch * hq)), dim3(256), 0, s, frame_mass,
                       row_group, nq, n_groups, n_frames, heatmap);
  else
    hipLaunchKernelGGL(heatmap_kernel, dim3(grid_for(n, 256)), dim3(256), 0, s, frame_mass, row_group,
                       n_batch, hq, nq, n_groups, n_frames, heatmap);
  if (heatmap_mean) {
    long long m = (long long)n_batch * n_groups * n_frames;
    hipLaunchKernelGGL(heatmap_mean_kernel, dim3(grid_for(m, 256)), dim3(256), 0, s, heatmap, n_batch,
                       hq, n_groups, n_frames, heatmap_mean);
  }
  return hipGetLastError();
}

hipError_t launch_hist(const float* support, const float* region_mass, int n_batch, int rows_per_b,
                       int n_regions, int bins, unsigned* hist, hipStream_t s) {
  long long nh = (long long)n_batch * (1 + n_regions) * bins;
  hipLaunchKernelGGL(zero_u32_kernel, dim3(grid_for(nh, 256)), dim3(256), 0, s, hist, nh);
  if ((long long)n_batch * rows_per_b > 0)
    hipLaunchKernelGGL(hist_kernel, dim3((unsigned)((long long)((rows_per_b + kHistRows - 1) / kHistRows) * n_batch)),
                       dim3(256), 0, s, support, region_mass, rows_per_b, n_regions, bins, hist);
  return hipGetLastError();
}

hipError_t launch_compare(const float* oq, const float* oref, const int* tq, const int* tref,
                          int64_t rows, int d, float* rel_row, float* recall_row, double* sums,
                          hipStream_t s) {
  // the per-row partials live in the sums buffer's tail: sums[2 + 2*rows]
  if (rows == 0) return hipSuccess;
  double* part = sums + 2;
  hipLaunchKernelGGL(compare_kernel, dim3(grid_for(rows, 1)), dim3(64), 0, s, oq, oref, tq, tref,
                     (long long)rows, d, rel_row, recall_row, part);
  hipLaunchKernelGGL(compare_sum_kernel, dim3(1), dim3(256), 0, s, part, (long long)rows, sums);
  return hipGetLastError();
}

}  // namespace kvp
