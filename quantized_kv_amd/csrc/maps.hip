// Probability maps of the KV-cache attention profiler (bf16 scores): the attention mass each key
// receives from a query head, the region-normalised key spatial maps built from it, each head's query x
// key probability matrix average-pooled to a small grid, one row's probabilities copied out, and the
// percentile clip of a map's colour range.
//
// Definitions: "Catnip Week 10 KV Cache Attention Study", section "Temporal & spatial heatmaps" —
// Figure 9 (key spatial preference on the latent grid, normalised inside each region of the KV-cache
// banner) and Figure 10 (one query's maps over all key frames, colour range clipped at the record's
// 99.5th percentile); the run manifest of the fine-grained per-head analysis, config block (heatmap
// pool shape, the 65,536-value sample of a quantile statistic).
//
// The maps kernel runs after the row kernel and takes its log-sum-exp: p_ij = 2^(u_ij - lse_i log2 e)
// with u the score in log2 units. One workgroup = 32 query rows of one (batch, query head) against all
// keys; wave w takes a contiguous range of 32-key tiles. S^T = K Q^T on the 32x32x16 bf16 MFMA leaves
// lane l with query row l%32 and the 16 keys 8(v/4) + 4(l/32) + v%4 (v = 0..15) of the tile, so
//   - key masses (sums over the 32 rows) come from a transposing butterfly over the 32 lanes of a
//     half-wave: each exchange (permlane16 swap, then DPP mirrors) halves the values a lane holds, and
//     every lane ends with the sum of one key;
//   - pooled sums (per row, over key windows) are a contraction over keys: a second MFMA takes the
//     probabilities as its A operand (f16, scaled by 2^15) and 0/1 window membership as B.
// Partial results go to the workspace; small kernels reduce them in a fixed order (deterministic).
#include "kvprof_internal.h"

namespace kvp {
namespace {

constexpr int MW = 8;         // waves per workgroup
constexpr int MROWS = 32;     // query rows per workgroup
constexpr int MAXCB = kMaxPoolW / 32;  // 32-column blocks of the pooled map
constexpr float kLog2eM = 1.44269504088896340736f;
constexpr float kPoolScale = 32768.f;  // probabilities enter the f16 MFMA as p * 2^15
constexpr float kNegBigM = -1.0e37f;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __amdgpu_buffer_rsrc_t rsrc_t;

// Buffer resource over [base, base + bytes): loads past the end return zero.
__device__ __forceinline__ rsrc_t mrsrc(const void* base, size_t bytes) {
  const size_t cap = 0x7fffffff;
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)(bytes < cap ? bytes : cap),
                                           0x00020000);
}

// Adaptive-pooling window of cell c of n cells over a length: [floor(c len / n), ceil((c+1) len / n)).
__host__ __device__ __forceinline__ int win_lo(int c, int len, int n) { return (int)(((long long)c * len) / n); }
__host__ __device__ __forceinline__ int win_hi(int c, int len, int n) {
  return (int)(((long long)(c + 1) * len + n - 1) / n);
}

template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}
constexpr int kRowMirror = 0x140;      // lane i of a 16-lane row reads lane 15 - i
constexpr int kRowHalfMirror = 0x141;  // lane i of an 8-lane half-row reads lane 7 - i
constexpr int kQuadRev = 0x1B;         // quad_perm [3,2,1,0]: lane i of a quad reads lane 3 - i
constexpr int kQuadSwap = 0xB1;        // quad_perm [1,0,3,2]: lane i reads lane i ^ 1

// Consecutive workgroups go to the 8 XCDs round-robin; give each XCD a contiguous range of logical
// blocks so that the row blocks of one head share that XCD's L2.
__device__ __forceinline__ int remap_xcd(int bid, int n) {
  if ((n & 7) == 0) return (bid & 7) * (n >> 3) + (bid >> 3);
  return bid;
}

__global__ __launch_bounds__(MW * 64) void maps_kernel(const MapsParams p) {
  __shared__ float pred[MROWS][kMaxPoolW + 1];
  const int nrb = (p.n_q + MROWS - 1) / MROWS;
  const int nblk = p.n_batch * p.n_heads_q * nrb;
  const int bid = remap_xcd((int)blockIdx.x, nblk);
  const int rb = bid % nrb;
  const int hq = (bid / nrb) % p.n_heads_q;
  const int b = bid / (nrb * p.n_heads_q);
  const int hkv = hq / p.group;
  const int tid = threadIdx.x;
  const int w = tid >> 6;
  const int lane = tid & 63;
  const int rho = lane & 31;  // query row inside the block
  const int h = lane >> 5;    // k half of the MFMA operands

  const int qi = rb * MROWS + rho;
  const bool rok = qi < p.n_q;
  const long long grow0 = ((long long)b * p.n_heads_q + hq) * p.n_q + (long long)rb * MROWS;
  const long long grow = grow0 + rho;
  int nvis = 0;
  float lse2 = 0.f;
  if (rok) {
    nvis = p.n_k;
    if (p.causal) {
      const long long v = p.q_pos0 + qi + 1;
      nvis = v < (long long)p.n_k ? (int)v : p.n_k;
    }
    lse2 = p.row_lse[grow] * kLog2eM;
  }

  // Q fragments (B operand): k-step ks holds dims 16 ks + 8 h .. + 7 of this lane's row
  bf16x8 qf[8];
#pragma unroll
  for (int ks = 0; ks < 8; ++ks) {
    u32x4 v = u32x4{0u, 0u, 0u, 0u};
    if (rok) v = *reinterpret_cast<const u32x4*>(p.q + grow * 128 + 16 * ks + 8 * h);
    qf[ks] = __builtin_bit_cast(bf16x8, v);
  }

  const size_t kvh = (size_t)b * p.n_heads_kv + hkv;
  const rsrc_t rk = mrsrc(p.k + kvh * p.n_k * 128, (size_t)p.n_k * 256);
  const rsrc_t rbias = mrsrc(p.key_bias ? (const void*)p.key_bias : (const void*)p.q,
                             p.key_bias ? (size_t)p.n_k * 4 : 0);

  // pooled-column windows of this lane's columns 32 cb + rho, and each block's key range (uniform)
  const int W = p.pool_w;
  int clo[MAXCB], chi[MAXCB], blo[MAXCB], bhi[MAXCB];
#pragma unroll
  for (int cb = 0; cb < MAXCB; ++cb) {
    const int c = 32 * cb + rho;
    clo[cb] = c < W ? win_lo(c, p.n_k, W) : 0;
    chi[cb] = c < W ? win_hi(c, p.n_k, W) : 0;
    const int c0 = 32 * cb, c1 = min(32 * cb + 31, W - 1);
    blo[cb] = c0 < W ? win_lo(c0, p.n_k, W) : 0x7fffffff;
    bhi[cb] = c0 < W ? win_hi(c1, p.n_k, W) : 0;
  }
  f32x16 pacc[MAXCB];
#pragma unroll
  for (int cb = 0; cb < MAXCB; ++cb)
#pragma unroll
    for (int v = 0; v < 16; ++v) pacc[cb][v] = 0.f;

  const bool mine = p.p_row_out && rok && grow == p.p_row;  // this lane's row is copied out

  const int ntiles = (p.n_k + 31) / 32;
  const int tpw = (ntiles + MW - 1) / MW;
  const int t0 = w * tpw, t1 = min(ntiles, t0 + tpw);
  for (int t = t0; t < t1; ++t) {
    const int j0 = t * 32;
    f32x16 acc;
#pragma unroll
    for (int v = 0; v < 16; ++v) acc[v] = 0.f;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
      const u32x4 kf = __builtin_amdgcn_raw_buffer_load_b128(rk, (unsigned)(((j0 + rho) * 128 + 16 * ks + 8 * h) * 2), 0, 0);
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, kf), qf[ks], acc, 0, 0, 0);
    }
    // probabilities of keys j0 + 8 (v/4) + 4 h + v%4
    float pv[16];
#pragma unroll
    for (int g4 = 0; g4 < 4; ++g4) {
      const int jb = j0 + 8 * g4 + 4 * h;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int j = jb + i;
        // one dword per key: the range check of the buffer then zeroes exactly the keys past n_k
        const float bias = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rbias, (unsigned)j * 4u, 0, 0));
        const float u = fmaf(acc[4 * g4 + i], p.scale_log2, fmaxf(bias * kLog2eM, kNegBigM));
        pv[4 * g4 + i] = j < nvis ? __builtin_amdgcn_exp2f(u - lse2) : 0.f;
      }
    }
    if (mine) {
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int j = j0 + 8 * (v >> 2) + 4 * h + (v & 3);
        if (j < p.n_k) p.p_row_out[j] = pv[v];
      }
    }
    if (p.key_part) {
      // butterfly over the 32 rows of this half-wave; see the file comment
      float y[8];
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(pv[q]), __float_as_uint(pv[q + 8]), false, false);
        y[q] = __uint_as_float(r[0]) + __uint_as_float(r[1]);  // value q + 8 r16 (r16 = bit 4 of the lane)
      }
      const bool b3 = (lane >> 3) & 1, b2 = (lane >> 2) & 1, b1 = (lane >> 1) & 1;
      float z[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const float keep = b3 ? y[q + 4] : y[q], send = b3 ? y[q] : y[q + 4];
        z[q] = keep + dpp<kRowMirror>(send);  // value q + 4 b3 + 8 r16
      }
      float x2[2];
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        const float keep = b2 ? z[q + 2] : z[q], send = b2 ? z[q] : z[q + 2];
        x2[q] = keep + dpp<kRowHalfMirror>(send);  // value q + 2 b2 + 4 b3 + 8 r16
      }
      float s = (b1 ? x2[1] : x2[0]) + dpp<kQuadRev>(b1 ? x2[0] : x2[1]);  // value b1 + 2 b2 + 4 b3 + 8 r16
      s += dpp<kQuadSwap>(s);  // both lanes of a pair hold the same value
      const int vi = (lane >> 1) & 15;
      const int j = j0 + 8 * (vi >> 2) + 4 * h + (vi & 3);
      if (!(lane & 1) && j < p.n_k) p.key_part[(size_t)bid * p.n_k + j] = s;
    }
    if (p.pool_part) {
      // A operand: k slot 8 h + q of k-step s2 = key 16 s2 + 8 (q/4) + 4 h + q%4 of the tile
      f16x8 pa[2];
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
        for (int q = 0; q < 8; ++q) pa[s2][q] = (_Float16)(pv[8 * s2 + q] * kPoolScale);
#pragma unroll
      for (int cb = 0; cb < MAXCB; ++cb) {
        if (blo[cb] < j0 + 32 && bhi[cb] > j0) {  // uniform: the tile meets this block's columns
          const unsigned span = (unsigned)(chi[cb] - clo[cb]);
#pragma unroll
          for (int s2 = 0; s2 < 2; ++s2) {
            f16x8 wb;
#pragma unroll
            for (int q = 0; q < 8; ++q) {
              const int j = j0 + 16 * s2 + 8 * (q >> 2) + 4 * h + (q & 3);
              wb[q] = (unsigned)(j - clo[cb]) < span ? (_Float16)1.f : (_Float16)0.f;
            }
            pacc[cb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(pa[s2], wb, pacc[cb], 0, 0, 0);
          }
        }
      }
    }
  }

  if (p.pool_part) {
    // waves add their partial sums in wave order (fixed), then the block writes its rows
    const int ncb = (W + 31) / 32;
    for (int ww = 0; ww < MW; ++ww) {
      if (w == ww) {
#pragma unroll
        for (int cb = 0; cb < MAXCB; ++cb) {
          if (cb < ncb) {
#pragma unroll
            for (int v = 0; v < 16; ++v) {
              const int m = 8 * (v >> 2) + 4 * h + (v & 3);
              float& dst = pred[m][32 * cb + rho];
              dst = (ww == 0 ? 0.f : dst) + pacc[cb][v];
            }
          }
        }
      }
      __syncthreads();
    }
    const int nr = min(MROWS, p.n_q - rb * MROWS);
    for (int idx = tid; idx < nr * W; idx += MW * 64) {
      const int row = idx / W, c = idx - row * W;
      p.pool_part[(size_t)(grow0 + row) * W + c] = pred[row][c] * (1.f / kPoolScale);
    }
  }
}

// key_mass[bh][j] = sum over the row blocks of head bh of key_part, in block order.
__global__ void key_mass_kernel(const float* __restrict__ part, int n_bh, int nrb, int n_k, float* __restrict__ km) {
  const long long total = (long long)n_bh * n_k;
  for (long long t = blockIdx.x * (long long)blockDim.x + threadIdx.x; t < total;
       t += (long long)gridDim.x * blockDim.x) {
    const long long bh = t / n_k;
    const int j = (int)(t - bh * n_k);
    float s = 0.f;
    for (int r = 0; r < nrb; ++r) s += part[((size_t)bh * nrb + r) * n_k + j];
    km[t] = s;
  }
}

// Workgroup (batch b, head set hs, region q): hs < n_heads is one head, hs == n_heads all of them.
// Cell c sums the key masses of the region's keys j with j mod frame_len = c (heads in order, then
// keys ascending); the cells are then divided by their total (a fixed-order tree over the threads).
__global__ __launch_bounds__(256) void spatial_kernel(const float* __restrict__ km, int n_heads, int n_k,
                                                      const RegionBounds bounds, int n_regions,
                                                      int frame_len, float* __restrict__ spatial,
                                                      float* __restrict__ spatial_mean) {
  __shared__ float part[256];
  const int q = blockIdx.x % n_regions;
  const int hs = (blockIdx.x / n_regions) % (n_heads + 1);
  const int b = blockIdx.x / (n_regions * (n_heads + 1));
  float* out = hs < n_heads ? (spatial ? spatial + (((size_t)b * n_heads + hs) * n_regions + q) * frame_len : nullptr)
                            : (spatial_mean ? spatial_mean + ((size_t)b * n_regions + q) * frame_len : nullptr);
  if (!out) return;  // uniform over the workgroup
  const int a = bounds.b[q], e = bounds.b[q + 1];
  const int h0 = hs < n_heads ? hs : 0, h1 = hs < n_heads ? hs + 1 : n_heads;
  float mine = 0.f;
  for (int c = threadIdx.x; c < frame_len; c += blockDim.x) {
    // first key of the region in cell c
    int j = a + ((c - a % frame_len) % frame_len + frame_len) % frame_len;
    float s = 0.f;
    for (int hh = h0; hh < h1; ++hh) {
      const float* kr = km + ((size_t)b * n_heads + hh) * n_k;
      for (int jj = j; jj < e; jj += frame_len) s += kr[jj];
    }
    out[c] = s;
    mine += s;
  }
  part[threadIdx.x] = mine;
  __syncthreads();
  for (int st = 128; st >= 1; st >>= 1) {
    if ((int)threadIdx.x < st) part[threadIdx.x] += part[threadIdx.x + st];
    __syncthreads();
  }
  const float tot = part[0];
  const float inv = tot > 0.f ? 1.f / tot : 0.f;
  for (int c = threadIdx.x; c < frame_len; c += blockDim.x) out[c] = tot > 0.f ? out[c] * inv : 0.f;
}

// pooled[bh][i][c] = mean of p over query rows [win(i, n_q, H)) x keys [win(c, n_k, W)), from the
// per-row window sums (rows in order).
__global__ void pool_rows_kernel(const float* __restrict__ part, int n_bh, int n_q, int n_k, int H, int W,
                                 float* __restrict__ pooled) {
  const long long total = (long long)n_bh * H * W;
  for (long long t = blockIdx.x * (long long)blockDim.x + threadIdx.x; t < total;
       t += (long long)gridDim.x * blockDim.x) {
    const int c = (int)(t % W);
    const int i = (int)((t / W) % H);
    const long long bh = t / ((long long)W * H);
    const int r0 = win_lo(i, n_q, H), r1 = win_hi(i, n_q, H);
    const int k0 = win_lo(c, n_k, W), k1 = win_hi(c, n_k, W);
    float s = 0.f;
    for (int r = r0; r < r1; ++r) s += part[((size_t)bh * n_q + r) * W + c];
    pooled[t] = s / ((float)(r1 - r0) * (float)(k1 - k0));
  }
}

// Order key of a float: unsigned compare of keys = numeric compare (no NaN).
__device__ __forceinline__ unsigned fkey(float f) {
  const unsigned u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float funkey(unsigned k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7fffffffu) : ~k);
}

// One workgroup: the values of ranks lo and hi (0-based, ascending) of the sample x[0], x[s], x[2s], ...
// (m values) by four 8-bit radix passes each, then the linear interpolation in float64.
constexpr int kPctThreads = 1024;
__global__ __launch_bounds__(kPctThreads) void percentile_kernel(const float* __restrict__ x, long long stride,
                                                                 long long m, long long lo, long long hi,
                                                                 double frac, float* __restrict__ clip) {
  __shared__ unsigned hist[256];
  __shared__ unsigned s_prefix;
  __shared__ long long s_rank;
  double val[2];
  for (int which = 0; which < 2; ++which) {
    if (threadIdx.x == 0) {
      s_prefix = 0u;
      s_rank = which ? hi : lo;
    }
    __syncthreads();
    for (int pass = 0; pass < 4; ++pass) {
      const int sh = 24 - 8 * pass;
      const unsigned himask = pass == 0 ? 0u : ~0u << (32 - 8 * pass);
      const unsigned prefix = s_prefix;
      for (int i = threadIdx.x; i < 256; i += blockDim.x) hist[i] = 0u;
      __syncthreads();
      for (long long i = threadIdx.x; i < m; i += blockDim.x) {
        const unsigned k = fkey(x[i * stride]);
        if ((k & himask) == prefix) atomicAdd(&hist[(k >> sh) & 255u], 1u);
      }
      __syncthreads();
      if (threadIdx.x == 0) {
        long long r = s_rank, cum = 0;
        int bin = 0;
        for (; bin < 255; ++bin) {
          if (r < cum + (long long)hist[bin]) break;
          cum += hist[bin];
        }
        s_prefix = prefix | ((unsigned)bin << sh);
        s_rank = r - cum;
      }
      __syncthreads();
    }
    val[which] = (double)funkey(s_prefix);
    __syncthreads();
  }
  if (threadIdx.x == 0) *clip = (float)(val[0] + frac * (val[1] - val[0]));
}

__global__ void clip_apply_kernel(const float* __restrict__ x, long long n, const float* __restrict__ clip,
                                  float* __restrict__ y) {
  const float c = *clip;
  for (long long t = blockIdx.x * (long long)blockDim.x + threadIdx.x; t < n; t += (long long)gridDim.x * blockDim.x)
    y[t] = fminf(x[t], c);
}

__global__ void zero_f32_kernel(float* __restrict__ x, long long n) {
  for (long long t = blockIdx.x * (long long)blockDim.x + threadIdx.x; t < n; t += (long long)gridDim.x * blockDim.x)
    x[t] = 0.f;
}

unsigned grid_for(long long n, int threads) {
  long long g = (n + threads - 1) / threads;
  return (unsigned)(g < 1 ? 1 : (g > 65536 ? 65536 : g));
}

}  // namespace

hipError_t launch_maps(const MapsParams& p, const RegionBounds& bounds, float* key_mass, float* spatial,
                       float* spatial_mean, int n_regions, int frame_len, float* pooled, int pool_h, hipStream_t s) {
  const int nrb = (p.n_q + MROWS - 1) / MROWS;
  const long long nblk = (long long)p.n_batch * p.n_heads_q * nrb;
  if (nblk == 0) return hipSuccess;
  hipLaunchKernelGGL(maps_kernel, dim3((unsigned)nblk), dim3(MW * 64), 0, s, p);
  const int n_bh = p.n_batch * p.n_heads_q;
  if (p.key_part) {
    hipLaunchKernelGGL(key_mass_kernel, dim3(grid_for((long long)n_bh * p.n_k, 256)), dim3(256), 0, s, p.key_part,
                       n_bh, nrb, p.n_k, key_mass);
    if (spatial || spatial_mean)
      hipLaunchKernelGGL(spatial_kernel, dim3((unsigned)(p.n_batch * (p.n_heads_q + 1) * n_regions)), dim3(256), 0, s,
                         key_mass, p.n_heads_q, p.n_k, bounds, n_regions, frame_len, spatial, spatial_mean);
  }
  if (p.pool_part)
    hipLaunchKernelGGL(pool_rows_kernel, dim3(grid_for((long long)n_bh * pool_h * p.pool_w, 256)), dim3(256), 0, s,
                       p.pool_part, n_bh, p.n_q, p.n_k, pool_h, p.pool_w, pooled);
  return hipGetLastError();
}

hipError_t launch_zero_f32(float* x, long long n, hipStream_t s) {
  if (n > 0) hipLaunchKernelGGL(zero_f32_kernel, dim3(grid_for(n, 256)), dim3(256), 0, s, x, n);
  return hipGetLastError();
}

hipError_t launch_percentile(const float* x, long long n, long long stride, long long m, long long lo, long long hi,
                             double frac, float* clip, float* y, hipStream_t s) {
  hipLaunchKernelGGL(percentile_kernel, dim3(1), dim3(kPctThreads), 0, s, x, stride, m, lo, hi, frac, clip);
  if (y) hipLaunchKernelGGL(clip_apply_kernel, dim3(grid_for(n, 256)), dim3(256), 0, s, x, n, clip, y);
  return hipGetLastError();
}

}  // namespace kvp
