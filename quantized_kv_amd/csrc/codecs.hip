// Codec kernels: signed-Hadamard + MXFP8 (E4M3 elements, E8M0 block exponent, 32-element blocks)
// and grouped 4-bit K/V with a float32 recent window.
//
// MXFP8: "Catnip Week 10 KV Cache Attention Study", experiment design step 4 (signed-H128 +
// physical E4M3/E8M0 K32 Q/K) and the section on Q/K and probability quantization.
// Int4 KV: "KV residual window" (huhohoo.com), sections on the fixed budget (group 32, K per channel
// over token groups, V per token over feature groups, R in {0, 16, 64}) and on the payload.
//
// Both codecs are exact specifications: the codes and scale bytes are reproduced bit for bit, so the
// arithmetic below is fixed (float64 sums, float32 IEEE operations, round to nearest even).
#include "kvprof_internal.h"
#include "kvprof_device.h"

namespace kvp {
namespace {

// One 64-lane block per row (grid-stride over rows). The rotation runs as a Walsh-Hadamard
// butterfly on float64 values in LDS; sums of bf16 inputs are exact, so the butterfly order does not
// change the result.
__global__ __launch_bounds__(64) void pack_mxfp8_kernel(const uint16_t* __restrict__ x, int64_t rows,
                                                        int d, const int8_t* __restrict__ signs,
                                                        uint8_t* __restrict__ codes,
                                                        uint8_t* __restrict__ scales) {
  __shared__ double buf[256];
  __shared__ float yv[256];
  __shared__ int bexp[8];
  const int lane = threadIdx.x;
  for (int64_t r = blockIdx.x; r < rows; r += gridDim.x) {
    const uint16_t* xr = x + r * d;
    for (int c = lane; c < d; c += 64) {
      double v = (double)bf16_to_f32(xr[c]);
      buf[c] = signs ? v * (double)signs[c] : v;
    }
    __syncthreads();
    if (signs) {
      for (int h = 1; h < d; h <<= 1) {
        for (int b = lane; b < d / 2; b += 64) {
          int i = (b / h) * 2 * h + (b % h);
          double a0 = buf[i], a1 = buf[i + h];
          buf[i] = a0 + a1;
          buf[i + h] = a0 - a1;
        }
        __syncthreads();
      }
      const double c = (d == 128) ? kInvSqrt128 : 1.0 / sqrt((double)d);
      for (int i = lane; i < d; i += 64) {
        double t = __dmul_rn(buf[i], c);  // rounded to float64, then to float32 below
        yv[i] = (float)t;
      }
    } else {
      for (int i = lane; i < d; i += 64) yv[i] = (float)buf[i];
    }
    __syncthreads();
    const int nb = d / 32;
    if (lane < nb) {
      float amax = 0.f;
      for (int i = 0; i < 32; ++i) amax = fmaxf(amax, fabsf(yv[lane * 32 + i]));
      int e = e8m0_exp(amax);
      bexp[lane] = e;
      scales[r * nb + lane] = (uint8_t)(e + 127);
    }
    __syncthreads();
    for (int i = lane; i < d; i += 64) {
      float sv = ldexpf(yv[i], -bexp[i / 32]);
      codes[r * d + i] = e4m3_rne(sv);
    }
    __syncthreads();
  }
}

// d = 128: eight lanes per row, sixteen consecutive elements per lane, eight rows per wave, so the
// whole transform stays in registers. The butterfly runs in float64 (exact, as above): the four
// stages inside a lane's sixteen elements first, then the three across the row's lanes (lane
// bits 1, 2, 4 = element strides 16, 32, 64) by shuffles. A 32-element block is two lanes.
__global__ __launch_bounds__(256) void pack_mxfp8_d128_kernel(const uint16_t* __restrict__ x, int64_t rows,
                                                              const int8_t* __restrict__ signs,
                                                              uint8_t* __restrict__ codes,
                                                              uint8_t* __restrict__ scales) {
  const int lane = threadIdx.x & 63;
  const int sl = lane & 7;  // lane inside the row: elements 16 sl .. 16 sl + 15
  const int64_t wave0 = ((int64_t)blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6)) * 8;
  const int64_t wstride = (int64_t)gridDim.x * (blockDim.x >> 6) * 8;
  uint32_t sg[4] = {0u, 0u, 0u, 0u};
  if (signs) {
    const uint4 t = *reinterpret_cast<const uint4*>(signs + 16 * sl);
    sg[0] = t.x; sg[1] = t.y; sg[2] = t.z; sg[3] = t.w;
  }
  for (int64_t r0 = wave0; r0 < rows; r0 += wstride) {  // wave-uniform loop: every lane shuffles
    const int64_t r = r0 + (lane >> 3);
    const bool ok = r < rows;
    uint4 raw[2] = {{0u, 0u, 0u, 0u}, {0u, 0u, 0u, 0u}};
    if (ok) {
      const uint4* src = reinterpret_cast<const uint4*>(x + (size_t)r * 128 + 16 * sl);
      raw[0] = src[0];
      raw[1] = src[1];
    }
    double v[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const uint4 q = raw[i >> 3];
      const uint32_t w = (i & 6) == 0 ? q.x : (i & 6) == 2 ? q.y : (i & 6) == 4 ? q.z : q.w;
      const double a = (double)bf16_to_f32((uint16_t)(w >> (16 * (i & 1))));
      const bool neg = signs && ((sg[i >> 2] >> (8 * (i & 3))) & 0x80u);  // int8 -1 has its top bit set
      v[i] = neg ? -a : a;
    }
    float y[16];
    if (signs) {
#pragma unroll
      for (int h = 1; h < 16; h <<= 1)
#pragma unroll
        for (int i = 0; i < 16; ++i)
          if (!(i & h)) {
            const double a0 = v[i], a1 = v[i + h];
            v[i] = a0 + a1;
            v[i + h] = a0 - a1;
          }
#pragma unroll
      for (int b = 1; b < 8; b <<= 1) {
        const bool hi = sl & b;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const double o = __shfl_xor(v[i], b);
          v[i] = hi ? o - v[i] : v[i] + o;
        }
      }
#pragma unroll
      for (int i = 0; i < 16; ++i) y[i] = (float)__dmul_rn(v[i], kInvSqrt128);
    } else {
#pragma unroll
      for (int i = 0; i < 16; ++i) y[i] = (float)v[i];
    }
    float amax = 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i) amax = fmaxf(amax, fabsf(y[i]));
    amax = fmaxf(amax, __shfl_xor(amax, 1));
    const int e = e8m0_exp(amax);
    uint32_t cw[4] = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int i = 0; i < 16; ++i) cw[i >> 2] |= (uint32_t)e4m3_rne(ldexpf(y[i], -e)) << (8 * (i & 3));
    if (ok) {
      *reinterpret_cast<uint4*>(codes + (size_t)r * 128 + 16 * sl) = make_uint4(cw[0], cw[1], cw[2], cw[3]);
      if (!(sl & 1)) scales[(size_t)r * 4 + (sl >> 1)] = (uint8_t)(e + 127);
    }
  }
}

__global__ void unpack_mxfp8_kernel(const uint8_t* __restrict__ codes, const uint8_t* __restrict__ scales,
                                    int64_t n, int d, float* __restrict__ out_f32,
                                    uint16_t* __restrict__ out_bf16) {
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * blockDim.x) {
    int64_t r = i / d;
    int c = (int)(i - r * d);
    int e = (int)scales[r * (d / 32) + c / 32] - 127;
    float v = ldexpf(e4m3_value(codes[i]), e);
    if (out_f32) out_f32[i] = v;
    if (out_bf16) out_bf16[i] = (uint16_t)(__float_as_uint(v) >> 16);  // exact: <= 4 significant bits
  }
}

// ---- grouped 4-bit K/V ---------------------------------------------------------------------------

// Asymmetric 4-bit code of x in a group with min/max lo/hi: every operation is an IEEE float32
// operation with round to nearest even (no contraction: there is no multiply to fuse).
struct Int4Meta {
  _Float16 s, m;
};
__device__ __forceinline__ Int4Meta int4_meta(float lo, float hi) {
  float scale32 = __fdiv_rn(__fsub_rn(hi, lo), 15.0f);
  Int4Meta mt;
  mt.s = (_Float16)scale32;
  mt.m = (_Float16)lo;
  return mt;
}
__device__ __forceinline__ uint32_t int4_code(float x, Int4Meta mt) {
  float s = (float)mt.s;
  if (s == 0.f) return 0;
  float q = __builtin_rintf(__fdiv_rn(__fsub_rn(x, (float)mt.m), s));
  q = fminf(fmaxf(q, 0.f), 15.f);
  return (uint32_t)q;
}

// K: one thread per (head, token group, channel pair).
// The same decode, sixteen consecutive elements per thread (one 16-byte load of codes, one scale
// byte: sixteen elements never straddle a 32-element block), written with 16-byte stores.
__global__ void unpack_mxfp8_vec16_kernel(const uint8_t* __restrict__ codes, const uint8_t* __restrict__ scales,
                                          int64_t n16, float* __restrict__ out_f32, uint16_t* __restrict__ out_bf16) {
  for (int64_t t = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; t < n16; t += (int64_t)gridDim.x * blockDim.x) {
    const uint4 c4 = reinterpret_cast<const uint4*>(codes)[t];
    const int e = (int)scales[t >> 1] - 127;  // element 16 t lies in block (16 t) / 32
    const uint32_t cw[4] = {c4.x, c4.y, c4.z, c4.w};
    float v[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) v[i] = ldexpf(e4m3_value((uint8_t)(cw[i >> 2] >> (8 * (i & 3)))), e);
    if (out_f32) {
      float4* o = reinterpret_cast<float4*>(out_f32) + 4 * t;
#pragma unroll
      for (int q = 0; q < 4; ++q) o[q] = make_float4(v[4 * q], v[4 * q + 1], v[4 * q + 2], v[4 * q + 3]);
    }
    if (out_bf16) {
      uint32_t h[8];
#pragma unroll
      for (int q = 0; q < 8; ++q)
        h[q] = (__float_as_uint(v[2 * q]) >> 16) | (__float_as_uint(v[2 * q + 1]) & 0xFFFF0000u);  // exact
      uint4* o = reinterpret_cast<uint4*>(out_bf16) + 2 * t;
      o[0] = make_uint4(h[0], h[1], h[2], h[3]);
      o[1] = make_uint4(h[4], h[5], h[6], h[7]);
    }
  }
}

__global__ void pack_k_kernel(const uint16_t* __restrict__ k, int heads, int64_t N, int d, int R,
                              uint8_t* __restrict__ out, size_t blob) {
  Int4Layout L = int4_layout(N, d, R);
  int64_t total = (int64_t)heads * L.G * (d / 2);
  for (int64_t t = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; t < total;
       t += (int64_t)gridDim.x * blockDim.x) {
    int cp = (int)(t % (d / 2));
    int64_t g = (t / (d / 2)) % L.G;
    int h = (int)(t / ((d / 2) * L.G));
    const uint16_t* kh = k + (int64_t)h * N * d;
    uint8_t* ob = out + (size_t)h * blob;
    int64_t t0 = g * 32, t1 = min(t0 + 32, L.n);
    Int4Meta mt[2];
    for (int q = 0; q < 2; ++q) {
      int c = 2 * cp + q;
      float lo = INFINITY, hi = -INFINITY;
      for (int64_t tok = t0; tok < t1; ++tok) {
        float xv = bf16_to_f32(kh[tok * d + c]);
        lo = fminf(lo, xv);
        hi = fmaxf(hi, xv);
      }
      mt[q] = int4_meta(lo, hi);
      _Float16* meta = reinterpret_cast<_Float16*>(ob + L.km) + (g * d + c) * 2;
      meta[0] = mt[q].s;
      meta[1] = mt[q].m;
    }
    for (int64_t tok = t0; tok < g * 32 + 32; ++tok) {
      uint32_t byte = 0;
      if (tok < t1) {
        byte = int4_code(bf16_to_f32(kh[tok * d + 2 * cp]), mt[0]) |
               (int4_code(bf16_to_f32(kh[tok * d + 2 * cp + 1]), mt[1]) << 4);
      }
      ob[L.kc + tok * (d / 2) + cp] = (uint8_t)byte;
    }
  }
}

// V: one thread per (head, token, 32-feature group).
__global__ void pack_v_kernel(const uint16_t* __restrict__ v, int heads, int64_t N, int d, int R,
                              uint8_t* __restrict__ out, size_t blob) {
  Int4Layout L = int4_layout(N, d, R);
  const int nfg = d / 32;
  int64_t total = (int64_t)heads * L.n * nfg;
  for (int64_t t = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; t < total;
       t += (int64_t)gridDim.x * blockDim.x) {
    int f = (int)(t % nfg);
    int64_t tok = (t / nfg) % L.n;
    int h = (int)(t / (nfg * L.n));
    const uint16_t* xr = v + ((int64_t)h * N + tok) * d + f * 32;
    uint8_t* ob = out + (size_t)h * blob;
    float lo = INFINITY, hi = -INFINITY;
    for (int c = 0; c < 32; ++c) {
      float xv = bf16_to_f32(xr[c]);
      lo = fminf(lo, xv);
      hi = fmaxf(hi, xv);
    }
    Int4Meta mt = int4_meta(lo, hi);
    _Float16* meta = reinterpret_cast<_Float16*>(ob + L.vm) + (tok * nfg + f) * 2;
    meta[0] = mt.s;
    meta[1] = mt.m;
    for (int c = 0; c < 32; c += 2) {
      uint32_t byte = int4_code(bf16_to_f32(xr[c]), mt) | (int4_code(bf16_to_f32(xr[c + 1]), mt) << 4);
      ob[L.vc + tok * (d / 2) + (f * 32 + c) / 2] = (uint8_t)byte;
    }
  }
}

// One workgroup per (head, 32-token group) for d in {32, 64, 128, 256}: the group's K and V rows come in
// with 16-byte loads (a K group is 32 consecutive token rows, so both tiles are contiguous in memory),
// then K's per-channel (scale, min) over the group's valid tokens, K's codes four bytes (8 channels of
// one token) per store, and V's per-token 32-feature groups. The arithmetic is int4_meta / int4_code,
// as in pack_k_kernel and pack_v_kernel.
template <int D>
__global__ __launch_bounds__(256) void pack_group_kernel(const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
                                                         int64_t N, int R, uint8_t* __restrict__ out, size_t blob) {
  constexpr int CH = D / 8;  // 16-byte chunks per row
  __shared__ uint16_t kt[32][D + 8];
  __shared__ uint16_t vt[32][D + 8];
  __shared__ Int4Meta kmeta[D];
  const Int4Layout L = int4_layout(N, D, R);
  const int64_t g = blockIdx.x % L.G;
  const int h = (int)(blockIdx.x / L.G);
  const int64_t t0 = g * 32;
  const int nt = (int)min((int64_t)32, L.n - t0);  // valid tokens of the group
  const int tid = threadIdx.x;
  const uint16_t* kh = k + ((int64_t)h * N + t0) * D;
  const uint16_t* vh = v + ((int64_t)h * N + t0) * D;
  for (int c = tid; c < 32 * CH; c += 256) {
    const int tok = c / CH, off = (c % CH) * 8;
    uint4 a = make_uint4(0u, 0u, 0u, 0u), b = a;
    if (tok < nt) {
      a = *reinterpret_cast<const uint4*>(kh + (int64_t)tok * D + off);
      b = *reinterpret_cast<const uint4*>(vh + (int64_t)tok * D + off);
    }
    *reinterpret_cast<uint4*>(&kt[tok][off]) = a;
    *reinterpret_cast<uint4*>(&vt[tok][off]) = b;
  }
  __syncthreads();
  uint8_t* ob = out + (size_t)h * blob;
  for (int c = tid; c < D; c += 256) {
    float lo = INFINITY, hi = -INFINITY;
    for (int tok = 0; tok < nt; ++tok) {
      const float xv = bf16_to_f32(kt[tok][c]);
      lo = fminf(lo, xv);
      hi = fmaxf(hi, xv);
    }
    const Int4Meta mt = int4_meta(lo, hi);
    kmeta[c] = mt;
    _Float16* meta = reinterpret_cast<_Float16*>(ob + L.km) + (g * D + c) * 2;
    meta[0] = mt.s;
    meta[1] = mt.m;
  }
  __syncthreads();
  // K codes: token tok, channels 8q .. 8q+7 -> one 32-bit word (pad tokens code 0)
  for (int it = tid; it < 32 * CH; it += 256) {
    const int tok = it / CH, q = it % CH;
    uint32_t wd = 0u;
    if (tok < nt) {
#pragma unroll
      for (int e = 0; e < 8; ++e) wd |= int4_code(bf16_to_f32(kt[tok][8 * q + e]), kmeta[8 * q + e]) << (4 * e);
    }
    *reinterpret_cast<uint32_t*>(ob + L.kc + (t0 + tok) * (D / 2) + 4 * q) = wd;
  }
  // V: token tok, 32-feature group f -> (scale, min) and 16 bytes of codes
  for (int it = tid; it < nt * (D / 32); it += 256) {
    const int tok = it / (D / 32), f = it % (D / 32);
    float lo = INFINITY, hi = -INFINITY;
#pragma unroll 8
    for (int c = 0; c < 32; ++c) {
      const float xv = bf16_to_f32(vt[tok][32 * f + c]);
      lo = fminf(lo, xv);
      hi = fmaxf(hi, xv);
    }
    const Int4Meta mt = int4_meta(lo, hi);
    _Float16* meta = reinterpret_cast<_Float16*>(ob + L.vm) + ((t0 + tok) * (D / 32) + f) * 2;
    meta[0] = mt.s;
    meta[1] = mt.m;
    uint32_t* cw = reinterpret_cast<uint32_t*>(ob + L.vc + (t0 + tok) * (D / 2) + 16 * f);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      uint32_t wd = 0u;
#pragma unroll
      for (int e = 0; e < 8; ++e) wd |= int4_code(bf16_to_f32(vt[tok][32 * f + 8 * q + e]), mt) << (4 * e);
      cw[q] = wd;
    }
  }
}

// Header and the float32 residual window (bf16 -> fp32 is exact).
__global__ void pack_tail_kernel(const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
                                 int heads, int64_t N, int d, int R, uint8_t* __restrict__ out,
                                 size_t blob) {
  Int4Layout L = int4_layout(N, d, R);
  int64_t per = (int64_t)R * d;
  int64_t total = (int64_t)heads * (per + 1);
  for (int64_t t = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; t < total;
       t += (int64_t)gridDim.x * blockDim.x) {
    int h = (int)(t / (per + 1));
    int64_t e = t % (per + 1);
    uint8_t* ob = out + (size_t)h * blob;
    if (e == per) {
      int32_t* hd = reinterpret_cast<int32_t*>(ob);
      hd[0] = (int32_t)N;
      hd[1] = d;
      hd[2] = R;
      hd[3] = 32;
      continue;
    }
    int64_t src = ((int64_t)h * N + L.n) * d + e;
    reinterpret_cast<float*>(ob + L.kr)[e] = bf16_to_f32(k[src]);
    reinterpret_cast<float*>(ob + L.vr)[e] = bf16_to_f32(v[src]);
  }
}

__global__ void unpack_int4_kernel(const uint8_t* __restrict__ packed, int heads, int64_t N, int d,
                                   int R, size_t blob, float* __restrict__ k_out,
                                   float* __restrict__ v_out) {
  Int4Layout L = int4_layout(N, d, R);
  int64_t total = (int64_t)heads * N * d;
  for (int64_t t = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; t < total;
       t += (int64_t)gridDim.x * blockDim.x) {
    int c = (int)(t % d);
    int64_t tok = (t / d) % N;
    int h = (int)(t / (d * N));
    const uint8_t* b = packed + (size_t)h * blob;
    float kv, vv;
    if (tok < L.n) {
      int g = (int)(tok / 32);
      const _Float16* km = reinterpret_cast<const _Float16*>(b + L.km) + ((int64_t)g * d + c) * 2;
      uint32_t kc = (b[L.kc + tok * (d / 2) + c / 2] >> ((c & 1) * 4)) & 0xF;
      kv = fmaf((float)kc, (float)km[0], (float)km[1]);
      const _Float16* vm = reinterpret_cast<const _Float16*>(b + L.vm) + (tok * (d / 32) + c / 32) * 2;
      uint32_t vc = (b[L.vc + tok * (d / 2) + c / 2] >> ((c & 1) * 4)) & 0xF;
      vv = fmaf((float)vc, (float)vm[0], (float)vm[1]);
    } else {
      kv = reinterpret_cast<const float*>(b + L.kr)[(tok - L.n) * d + c];
      vv = reinterpret_cast<const float*>(b + L.vr)[(tok - L.n) * d + c];
    }
    k_out[t] = kv;
    v_out[t] = vv;
  }
}

inline unsigned grid_for(int64_t n, int block, unsigned cap = 65536) {
  int64_t g = (n + block - 1) / block;
  if (g < 1) g = 1;
  return (unsigned)(g > cap ? cap : g);
}

}  // namespace

hipError_t launch_pack_mxfp8(const uint16_t* x, int64_t rows, int d, const int8_t* signs,
                             uint8_t* codes, uint8_t* scales, hipStream_t s) {
  if (rows == 0) return hipSuccess;
  if (d == 128 && ((uintptr_t)x & 15) == 0 && ((uintptr_t)codes & 15) == 0 && ((uintptr_t)signs & 15) == 0) {
    const int64_t blocks = (rows + 31) / 32;  // 32 rows per 256-thread block
    hipLaunchKernelGGL(pack_mxfp8_d128_kernel, dim3((unsigned)(blocks < 8192 ? blocks : 8192)), dim3(256), 0, s,
                       x, rows, signs, codes, scales);
    return hipGetLastError();
  }
  unsigned g = (unsigned)(rows < 65536 * 4 ? rows : 65536 * 4);
  hipLaunchKernelGGL(pack_mxfp8_kernel, dim3(g), dim3(64), 0, s, x, rows, d, signs, codes, scales);
  return hipGetLastError();
}

hipError_t launch_unpack_mxfp8(const uint8_t* codes, const uint8_t* scales, int64_t rows, int d,
                               float* out_f32, uint16_t* out_bf16, hipStream_t s) {
  int64_t n = rows * d;
  if (n == 0) return hipSuccess;
  if (d % 32 == 0 && ((uintptr_t)codes & 15) == 0 && ((uintptr_t)out_f32 & 15) == 0 &&
      ((uintptr_t)out_bf16 & 15) == 0) {
    hipLaunchKernelGGL(unpack_mxfp8_vec16_kernel, dim3(grid_for(n / 16, 256)), dim3(256), 0, s, codes, scales,
                       n / 16, out_f32, out_bf16);
    return hipGetLastError();
  }
  hipLaunchKernelGGL(unpack_mxfp8_kernel, dim3(grid_for(n, 256)), dim3(256), 0, s, codes, scales, n,
                     d, out_f32, out_bf16);
  return hipGetLastError();
}

// ---- rolling window: append tokens, move the oldest float32 tokens to the 4-bit part ----------------
// The combined window of a head is its old float32 tokens followed by the new bf16 tokens; token u of it
// reads the old window for u < R_in and the new tokens after (bf16 -> fp32 is exact, so a moved token
// is quantized from the same value the one-shot pack would see).
struct AppendGeom {
  Int4Layout Lo, Ln;  // old and new blob layouts
  int d, r_in;
  int64_t t;          // new tokens per head
  int64_t moved;      // tokens moved to the 4-bit part (a multiple of 32)
  size_t blob_in, blob_out;
};

__device__ __forceinline__ float win_val(const uint8_t* ib, const uint16_t* xnew, const AppendGeom& g, size_t res_off,
                                         int h, int64_t u, int c) {
  if (u < g.r_in) return reinterpret_cast<const float*>(ib + res_off)[u * g.d + c];
  return bf16_to_f32(xnew[((int64_t)h * g.t + (u - g.r_in)) * g.d + c]);
}

// The old 4-bit sections, copied a word at a time to their new offsets.
__global__ void append_copy_kernel(const uint8_t* __restrict__ in, uint8_t* __restrict__ out, int heads, AppendGeom g) {
  const int64_t wkc = (g.Lo.km - g.Lo.kc) / 4, wkm = (g.Lo.vc - g.Lo.km) / 4, wvc = (g.Lo.vm - g.Lo.vc) / 4,
                wvm = (g.Lo.kr - g.Lo.vm) / 4;
  const int64_t per = wkc + wkm + wvc + wvm;
  const int64_t total = (int64_t)heads * per;
  for (int64_t t = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; t < total; t += (int64_t)gridDim.x * blockDim.x) {
    const int h = (int)(t / per);
    int64_t e = t - (int64_t)h * per;
    size_t so, dst;
    if (e < wkc) {
      so = g.Lo.kc;
      dst = g.Ln.kc;
    } else if ((e -= wkc) < wkm) {
      so = g.Lo.km;
      dst = g.Ln.km;
    } else if ((e -= wkm) < wvc) {
      so = g.Lo.vc;
      dst = g.Ln.vc;
    } else {
      e -= wvc;
      so = g.Lo.vm;
      dst = g.Ln.vm;
    }
    const uint32_t w = reinterpret_cast<const uint32_t*>(in + (size_t)h * g.blob_in + so)[e];
    reinterpret_cast<uint32_t*>(out + (size_t)h * g.blob_out + dst)[e] = w;
  }
}

// New K groups: one thread per (head, moved group, channel pair), as pack_k_kernel.
__global__ void append_k_kernel(const uint8_t* __restrict__ in, const uint16_t* __restrict__ knew, uint8_t* __restrict__ out,
                                int heads, AppendGeom g) {
  const int64_t ng = g.moved / 32, G0 = g.Lo.G;
  const int d = g.d;
  const int64_t total = (int64_t)heads * ng * (d / 2);
  for (int64_t t = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; t < total; t += (int64_t)gridDim.x * blockDim.x) {
    const int cp = (int)(t % (d / 2));
    const int64_t gi = (t / (d / 2)) % ng;
    const int h = (int)(t / ((d / 2) * ng));
    const uint8_t* ib = in + (size_t)h * g.blob_in;
    uint8_t* ob = out + (size_t)h * g.blob_out;
    Int4Meta mt[2];
    for (int q = 0; q < 2; ++q) {
      const int c = 2 * cp + q;
      float lo = INFINITY, hi = -INFINITY;
      for (int64_t u = gi * 32; u < gi * 32 + 32; ++u) {
        const float xv = win_val(ib, knew, g, g.Lo.kr, h, u, c);
        lo = fminf(lo, xv);
        hi = fmaxf(hi, xv);
      }
      mt[q] = int4_meta(lo, hi);
      _Float16* meta = reinterpret_cast<_Float16*>(ob + g.Ln.km) + ((G0 + gi) * d + c) * 2;
      meta[0] = mt[q].s;
      meta[1] = mt[q].m;
    }
    for (int64_t u = gi * 32; u < gi * 32 + 32; ++u) {
      const uint32_t byte = int4_code(win_val(ib, knew, g, g.Lo.kr, h, u, 2 * cp), mt[0]) |
                            (int4_code(win_val(ib, knew, g, g.Lo.kr, h, u, 2 * cp + 1), mt[1]) << 4);
      ob[g.Ln.kc + (G0 * 32 + u) * (d / 2) + cp] = (uint8_t)byte;
    }
  }
}

// New V rows: one thread per (head, moved token, 32-feature group), as pack_v_kernel.
__global__ void append_v_kernel(const uint8_t* __restrict__ in, const uint16_t* __restrict__ vnew, uint8_t* __restrict__ out,
                                int heads, AppendGeom g) {
  const int d = g.d, nfg = d / 32;
  const int64_t n0 = g.Lo.n;
  const int64_t total = (int64_t)heads * g.moved * nfg;
  for (int64_t t = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; t < total; t += (int64_t)gridDim.x * blockDim.x) {
    const int f = (int)(t % nfg);
    const int64_t u = (t / nfg) % g.moved;
    const int h = (int)(t / (nfg * g.moved));
    const uint8_t* ib = in + (size_t)h * g.blob_in;
    uint8_t* ob = out + (size_t)h * g.blob_out;
    float lo = INFINITY, hi = -INFINITY;
    for (int c = 0; c < 32; ++c) {
      const float xv = win_val(ib, vnew, g, g.Lo.vr, h, u, f * 32 + c);
      lo = fminf(lo, xv);
      hi = fmaxf(hi, xv);
    }
    const Int4Meta mt = int4_meta(lo, hi);
    _Float16* meta = reinterpret_cast<_Float16*>(ob + g.Ln.vm) + ((n0 + u) * nfg + f) * 2;
    meta[0] = mt.s;
    meta[1] = mt.m;
    for (int c = 0; c < 32; c += 2) {
      const uint32_t byte = int4_code(win_val(ib, vnew, g, g.Lo.vr, h, u, f * 32 + c), mt) |
                            (int4_code(win_val(ib, vnew, g, g.Lo.vr, h, u, f * 32 + c + 1), mt) << 4);
      ob[g.Ln.vc + (n0 + u) * (d / 2) + (f * 32 + c) / 2] = (uint8_t)byte;
    }
  }
}

// Header and the new float32 window (the combined window's tokens from `moved` on).
__global__ void append_tail_kernel(const uint8_t* __restrict__ in, const uint16_t* __restrict__ knew,
                                   const uint16_t* __restrict__ vnew, uint8_t* __restrict__ out, int heads, AppendGeom g) {
  const int64_t rn = g.r_in + g.t - g.moved;
  const int64_t per = rn * g.d;
  const int64_t total = (int64_t)heads * (per + 1);
  for (int64_t t = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; t < total; t += (int64_t)gridDim.x * blockDim.x) {
    const int h = (int)(t / (per + 1));
    const int64_t e = t % (per + 1);
    const uint8_t* ib = in + (size_t)h * g.blob_in;
    uint8_t* ob = out + (size_t)h * g.blob_out;
    if (e == per) {
      int32_t* hd = reinterpret_cast<int32_t*>(ob);
      hd[0] = (int32_t)(g.Lo.n + g.r_in + g.t);
      hd[1] = g.d;
      hd[2] = (int32_t)rn;
      hd[3] = 32;
      continue;
    }
    const int64_t u = g.moved + e / g.d;
    const int c = (int)(e % g.d);
    reinterpret_cast<float*>(ob + g.Ln.kr)[e] = win_val(ib, knew, g, g.Lo.kr, h, u, c);
    reinterpret_cast<float*>(ob + g.Ln.vr)[e] = win_val(ib, vnew, g, g.Lo.vr, h, u, c);
  }
}

hipError_t launch_int4kv_append(const uint8_t* in, int heads, int64_t N, int d, int r_in, const uint16_t* knew,
                                const uint16_t* vnew, int64_t t, int r_out, uint8_t* out, size_t blob_in,
                                size_t blob_out, hipStream_t s) {
  if (heads == 0) return hipSuccess;
  AppendGeom g;
  g.Lo = int4_layout(N, d, r_in);
  g.Ln = int4_layout(N + t, d, r_out);
  g.d = d;
  g.r_in = r_in;
  g.t = t;
  g.moved = (int64_t)r_in + t - r_out;
  g.blob_in = blob_in;
  g.blob_out = blob_out;
  const int64_t ncopy = (int64_t)heads * (int64_t)((g.Lo.kr - g.Lo.kc) / 4);
  const int64_t nk = (int64_t)heads * (g.moved / 32) * (d / 2);
  const int64_t nv = (int64_t)heads * g.moved * (d / 32);
  const int64_t nt = (int64_t)heads * ((int64_t)r_out * d + 1);
  if (ncopy > 0) hipLaunchKernelGGL(append_copy_kernel, dim3(grid_for(ncopy, 256)), dim3(256), 0, s, in, out, heads, g);
  if (nk > 0) hipLaunchKernelGGL(append_k_kernel, dim3(grid_for(nk, 128)), dim3(128), 0, s, in, knew, out, heads, g);
  if (nv > 0) hipLaunchKernelGGL(append_v_kernel, dim3(grid_for(nv, 128)), dim3(128), 0, s, in, vnew, out, heads, g);
  hipLaunchKernelGGL(append_tail_kernel, dim3(grid_for(nt, 256)), dim3(256), 0, s, in, knew, vnew, out, heads, g);
  return hipGetLastError();
}

hipError_t launch_pack_int4kv(const uint16_t* k, const uint16_t* v, int heads, int64_t N, int d,
                              int R, uint8_t* out, size_t blob, hipStream_t s) {
  if (heads == 0) return hipSuccess;
  Int4Layout L = int4_layout(N, d, R);
  int64_t nk = (int64_t)heads * L.G * (d / 2);
  int64_t nv = (int64_t)heads * L.n * (d / 32);
  int64_t nt = (int64_t)heads * ((int64_t)R * d + 1);
  const int64_t nwg = (int64_t)heads * L.G;
  const bool grouped = (d == 32 || d == 64 || d == 128 || d == 256) && ((uintptr_t)k & 15) == 0 &&
                       ((uintptr_t)v & 15) == 0 && ((uintptr_t)out & 3) == 0 && nwg <= 0x7fffffff;
  if (grouped) {
    if (nwg > 0) {
      if (d == 32) hipLaunchKernelGGL(pack_group_kernel<32>, dim3((unsigned)nwg), dim3(256), 0, s, k, v, N, R, out, blob);
      if (d == 64) hipLaunchKernelGGL(pack_group_kernel<64>, dim3((unsigned)nwg), dim3(256), 0, s, k, v, N, R, out, blob);
      if (d == 128) hipLaunchKernelGGL(pack_group_kernel<128>, dim3((unsigned)nwg), dim3(256), 0, s, k, v, N, R, out, blob);
      if (d == 256) hipLaunchKernelGGL(pack_group_kernel<256>, dim3((unsigned)nwg), dim3(256), 0, s, k, v, N, R, out, blob);
    }
  } else {
    if (nk > 0) hipLaunchKernelGGL(pack_k_kernel, dim3(grid_for(nk, 128)), dim3(128), 0, s, k, heads, N, d, R, out, blob);
    if (nv > 0) hipLaunchKernelGGL(pack_v_kernel, dim3(grid_for(nv, 128)), dim3(128), 0, s, v, heads, N, d, R, out, blob);
  }
  hipLaunchKernelGGL(pack_tail_kernel, dim3(grid_for(nt, 256)), dim3(256), 0, s, k, v, heads, N, d, R, out, blob);
  return hipGetLastError();
}

hipError_t launch_unpack_int4kv(const uint8_t* packed, int heads, int64_t N, int d, int R,
                                size_t blob, float* k_out, float* v_out, hipStream_t s) {
  int64_t n = (int64_t)heads * N * d;
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(unpack_int4_kernel, dim3(grid_for(n, 256)), dim3(256), 0, s, packed, heads, N, d,
                     R, blob, k_out, v_out);
  return hipGetLastError();
}

}  // namespace kvp
