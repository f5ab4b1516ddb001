// Local output ablation ("Catnip Week 10 KV Cache Attention Study", section on the current judgement and
// next steps, recommended sequence, first item): for the same Q/K/V, drop the sink, the recent region
// or all history, renormalise P over what is kept, and compare the attention output before the output
// projection by relative L2 and cosine.
//
// The drop is expressed as a key bias: every key of the dropped range gets -1e4 added to its bias.
// Scores of kept keys are O(10), so a dropped key's exponential exp(s - m) falls below 2^-14000 and
// is exactly zero in the row kernel's float32 exponentials; the row kernel's softmax over all keys is
// then the softmax over the kept keys, i.e. P renormalised, with no change to the row kernel.
#include <hip/hip_runtime.h>

#include <cstdint>

namespace kvp {
namespace {

constexpr float kDropBias = -1.0e4f;

__global__ __launch_bounds__(256) void ablation_bias_kernel(const float* __restrict__ bias, int n, int lo,
                                                            int hi, float* __restrict__ out) {
  for (int j = blockIdx.x * blockDim.x + threadIdx.x; j < n; j += gridDim.x * blockDim.x) {
    const float b = bias ? bias[j] : 0.f;
    out[j] = (j >= lo && j < hi) ? b + kDropBias : b;
  }
}

// One wave per row: a.b, |a|^2, |b|^2 in float64 (lane-strided, then a butterfly), the row's cosine,
// and the three partials for the tensor-level sums.
__global__ __launch_bounds__(64) void cosine_kernel(const float* __restrict__ a, const float* __restrict__ b,
                                                    long long rows, int d, float* __restrict__ cos_row,
                                                    double* __restrict__ part) {
  const int lane = threadIdx.x;
  for (long long r = blockIdx.x; r < rows; r += gridDim.x) {
    double ab = 0.0, aa = 0.0, bb = 0.0;
    for (int c = lane; c < d; c += 64) {
      const double x = a[r * d + c], y = b[r * d + c];
      ab += x * y;
      aa += x * x;
      bb += y * y;
    }
    for (int o = 32; o >= 1; o >>= 1) {
      ab += __shfl_xor(ab, o);
      aa += __shfl_xor(aa, o);
      bb += __shfl_xor(bb, o);
    }
    if (lane == 0) {
      cos_row[r] = (aa > 0.0 && bb > 0.0) ? (float)(ab / sqrt(aa * bb)) : 0.f;
      part[3 * r] = ab;
      part[3 * r + 1] = aa;
      part[3 * r + 2] = bb;
    }
  }
}

// Fixed-order sums of the partials: 256 interleaved subsets, then the subset sums in order.
__global__ __launch_bounds__(256) void cosine_sum_kernel(const double* __restrict__ part, long long rows,
                                                         double* __restrict__ sums) {
  __shared__ double s[3][256];
  const int t = threadIdx.x;
  double x = 0.0, y = 0.0, z = 0.0;
#pragma unroll 8  // loads issued ahead; the additions keep their order
  for (long long i = t; i < rows; i += 256) {  // thread t sums rows t, t + 256, ... (coalesced)
    x += part[3 * i];
    y += part[3 * i + 1];
    z += part[3 * i + 2];
  }
  s[0][t] = x;
  s[1][t] = y;
  s[2][t] = z;
  __syncthreads();
  if (t < 3) {
    double acc = 0.0;
    for (int i = 0; i < 256; ++i) acc += s[t][i];
    sums[t] = acc;
  }
}

unsigned grid_of(long long n, int block) {
  long long g = (n + block - 1) / block;
  if (g < 1) g = 1;
  return (unsigned)(g > 65536 ? 65536 : g);
}

}  // namespace

hipError_t launch_ablation_bias(const float* bias, int n_k, int lo, int hi, float* out, hipStream_t s) {
  if (n_k == 0) return hipSuccess;
  hipLaunchKernelGGL(ablation_bias_kernel, dim3(grid_of(n_k, 256)), dim3(256), 0, s, bias, n_k, lo, hi, out);
  return hipGetLastError();
}

hipError_t launch_cosine(const float* a, const float* b, int64_t rows, int d, float* cos_row, double* sums,
                         hipStream_t s) {
  // the per-row partials live in the sums buffer's tail: sums[3 + 3*rows]
  if (rows == 0) return hipSuccess;
  double* part = sums + 3;
  hipLaunchKernelGGL(cosine_kernel, dim3(grid_of(rows, 1)), dim3(64), 0, s, a, b, (long long)rows, d, cos_row,
                     part);
  hipLaunchKernelGGL(cosine_sum_kernel, dim3(1), dim3(256), 0, s, part, (long long)rows, sums);
  return hipGetLastError();
}

}  // namespace kvp
