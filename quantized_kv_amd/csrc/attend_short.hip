// Attention over short heads (d = 32 or 64): O = softmax(scale q k^T + b) V together with the row
// max, the log-sum-exp, the entropy support and the region masses, over bf16 K/V or over packed 4-bit
// K/V with the float32 recent window. ("KV residual window": its fixed-budget experiments attend over
// the whole dequantized cache at head dimension 32 — full float32 K/V of 128 tokens is 32,768 bytes —
// and report the relative L2 of the output and the attention mass of the recent window.)
//
// One wave = 16 query rows of one (batch, KV head); four waves per workgroup, each on its own rows.
// Two passes over the keys, 16 per tile. S^T = K Q^T on the 16x16x32 MFMA (bf16, or the f16 hi + lo
// halves of the dequantized 4-bit K with Q in f16) leaves lane l with query row l % 16 and the keys
// 4 (l / 16) + i, i = 0..3, of the tile.
//   pass 1: each lane keeps a running max and sum over its keys (online rescaling); the row's four
//           lanes are combined at the end;
//   pass 2: p = 2^(u - lse) exactly normalised; O += P V on the f16 MFMA (V as f16, or hi + lo halves
//           for dequantized 4-bit V), region masses and sum p (lse - u) for the entropy.
#include "kvprof_internal.h"
#include "kvprof_device.h"

namespace kvp {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __amdgpu_buffer_rsrc_t rsrc_t;

constexpr int SW = 4;  // waves per workgroup
constexpr float kLog2eS = 1.44269504088896340736f;
constexpr float kLn2S = 0.69314718055994530942f;
constexpr float kNegBigS = -1.0e37f;
constexpr float kPScaleS = 32768.f;  // P enters the f16 MFMA as p * 2^15
constexpr unsigned kOORS = 0x7FFF0000u;  // an offset past the end of every buffer read here

__device__ __forceinline__ rsrc_t srsrc(const void* base, size_t bytes) {
  const size_t cap = 0x7fffffff;
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)(bytes < cap ? bytes : cap),
                                           0x00020000);
}
__device__ __forceinline__ float ld_f32(rsrc_t r, unsigned off) {
  return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0));
}
__device__ __forceinline__ float half_lo(uint32_t w) { return (float)__builtin_bit_cast(_Float16, (uint16_t)(w & 0xFFFFu)); }
__device__ __forceinline__ float half_hi(uint32_t w) { return (float)__builtin_bit_cast(_Float16, (uint16_t)(w >> 16)); }

__device__ __forceinline__ float sum4(float x) {
  x += __shfl_xor(x, 16);
  return x + __shfl_xor(x, 32);
}
__device__ __forceinline__ float max4(float x) {
  x = fmaxf(x, __shfl_xor(x, 16));
  return fmaxf(x, __shfl_xor(x, 32));
}

struct RowOf {
  bool ok;
  long long grow;
  int nvis;
};
__device__ __forceinline__ RowOf row_of(const ShortParams& p, int b, int hkv, int rl) {
  RowOf o;
  o.ok = rl < p.rows_per_kv;
  const int hloc = o.ok ? rl / p.n_q : 0;
  const int qi = o.ok ? rl - hloc * p.n_q : 0;
  o.grow = ((long long)b * p.n_heads_q + (long long)hkv * p.group + hloc) * p.n_q + qi;
  int nv = p.n_k;
  if (p.causal) {
    const long long v = p.q_pos0 + qi + 1;
    nv = v < (long long)p.n_k ? (int)v : p.n_k;
  }
  o.nvis = o.ok ? nv : 0;
  return o;
}

// A-operand fragment of K: key j, dims c0 .. c0+7. 4-bit blobs are read a dword at a time (a blob of
// head dimension 32 may start at any 4-byte boundary); the 4-bit and float32-window values are both
// loaded and one is selected, reads outside a section fall past the buffer end and return zero.
template <int D, int KSRC>
__device__ __forceinline__ u32x4 k_frag(rsrc_t rk, const Int4Layout& L, int n_k, int j, int c0, u32x4& lo) {
  if (KSRC == KSRC_BF16) {
    lo = u32x4{0u, 0u, 0u, 0u};
    return __builtin_amdgcn_raw_buffer_load_b128(rk, (unsigned)(j * D + c0) * 2u, 0, 0);
  } else {
    const bool quant = j < (int)L.n;
    const int jq = quant ? j : 0;
    const uint32_t codes = __builtin_amdgcn_raw_buffer_load_b32(rk, (unsigned)(L.kc + (size_t)jq * (D / 2) + c0 / 2), 0, 0);
    const unsigned mo = (unsigned)(L.km + ((size_t)(jq >> 5) * D + c0) * 4);
    const unsigned ro = (quant || j >= n_k) ? kOORS : (unsigned)(L.kr + ((size_t)(j - (int)L.n) * D + c0) * 4);
    f16x8 h, hl;
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      const uint32_t wd = __builtin_amdgcn_raw_buffer_load_b32(rk, mo + 4u * c, 0, 0);
      const float qv = fmaf((float)((codes >> (4 * c)) & 0xFu), half_lo(wd), half_hi(wd));
      const float rv = ld_f32(rk, ro + 4u * c);
      const float x = quant ? qv : rv;
      h[c] = (_Float16)x;
      hl[c] = (_Float16)(x - (float)h[c]);
    }
    lo = __builtin_bit_cast(u32x4, hl);
    return __builtin_bit_cast(u32x4, h);
  }
}

// V value of key j, channel c (keys past n_k read zero), as an f16 hi + lo pair.
template <int D, int KSRC>
__device__ __forceinline__ void v_val(rsrc_t rv, const Int4Layout& L, int n_k, int j, int c, _Float16& hi,
                                      _Float16& lo) {
  float x;
  if (KSRC == KSRC_BF16) {
    x = __uint_as_float((uint32_t)__builtin_amdgcn_raw_buffer_load_b16(rv, (unsigned)(j * D + c) * 2u, 0, 0) << 16);
  } else {
    const bool quant = j < (int)L.n;
    const int jq = quant ? j : 0;
    const uint32_t byte = __builtin_amdgcn_raw_buffer_load_b8(rv, (unsigned)(L.vc + (size_t)jq * (D / 2) + c / 2), 0, 0);
    const uint32_t code = (c & 1) ? (byte >> 4) & 0xFu : byte & 0xFu;
    const uint32_t wd = __builtin_amdgcn_raw_buffer_load_b32(rv, (unsigned)(L.vm + ((size_t)jq * (D / 32) + c / 32) * 4), 0, 0);
    const unsigned ro = (quant || j >= n_k) ? kOORS : (unsigned)(L.vr + ((size_t)(j - (int)L.n) * D + c) * 4);
    const float rvv = ld_f32(rv, ro);
    x = quant ? fmaf((float)code, half_lo(wd), half_hi(wd)) : rvv;
  }
  hi = (_Float16)x;
  lo = (_Float16)(x - (float)hi);
}

template <int D, int KSRC>
__global__ __launch_bounds__(SW * 64) void short_kernel(const ShortParams p) {
  constexpr int KS = D / 32;  // k-steps of the score MFMA
  constexpr int NB = D / 16;  // 16-channel blocks of O
  const int nrb = (p.rows_per_kv + 16 * SW - 1) / (16 * SW);
  const int bid = blockIdx.x;
  const int rb = bid % nrb;
  const int hkv = (bid / nrb) % p.n_heads_kv;
  const int b = bid / (nrb * p.n_heads_kv);
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int r = lane & 15, g = lane >> 4;
  const int rl0 = rb * 16 * SW + w * 16;  // first row (inside the KV head's rows) of this wave
  const RowOf me = row_of(p, b, hkv, rl0 + r);
  int kmax = me.nvis;
  for (int o = 1; o < 16; o <<= 1) kmax = max(kmax, __shfl_xor(kmax, o));
  kmax = __builtin_amdgcn_readfirstlane(kmax);
  if (kmax == 0) return;  // no valid row in this wave (the wave uses no shared memory)

  // Q fragments (B operand): dims 32 ks + 8 g .. + 7 of this lane's row
  u32x4 qf[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    u32x4 v = u32x4{0u, 0u, 0u, 0u};
    if (me.ok) v = *reinterpret_cast<const u32x4*>(p.q + me.grow * D + 32 * ks + 8 * g);
    if (KSRC == KSRC_INT4) {
      f16x8 hq;
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        hq[2 * c] = (_Float16)__uint_as_float(v[c] << 16);
        hq[2 * c + 1] = (_Float16)__uint_as_float(v[c] & 0xFFFF0000u);
      }
      v = __builtin_bit_cast(u32x4, hq);
    }
    qf[ks] = v;
  }
  const size_t kvh = (size_t)b * p.n_heads_kv + hkv;
  rsrc_t rk, rv;
  Int4Layout L{};
  if (KSRC == KSRC_BF16) {
    rk = srsrc(p.k + kvh * p.n_k * D, (size_t)p.n_k * D * 2);
    rv = srsrc(p.v ? p.v + kvh * p.n_k * D : p.k, p.v ? (size_t)p.n_k * D * 2 : 0);
  } else {
    rk = srsrc(p.kv_packed + kvh * p.blob_bytes, p.blob_bytes);
    rv = rk;
    L = int4_layout(p.n_k, D, p.r_window);
  }
  const rsrc_t rbs = srsrc(p.key_bias ? (const void*)p.key_bias : (const void*)p.q, p.key_bias ? (size_t)p.n_k * 4 : 0);

  auto tile_u = [&](int j0, float (&u)[4]) {
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      u32x4 lo;
      const u32x4 hi = k_frag<D, KSRC>(rk, L, p.n_k, j0 + r, 32 * ks + 8 * g, lo);
      if (KSRC == KSRC_BF16) {
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, hi), __builtin_bit_cast(bf16x8, qf[ks]), acc, 0, 0, 0);
      } else {
        acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, hi), __builtin_bit_cast(f16x8, qf[ks]), acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, lo), __builtin_bit_cast(f16x8, qf[ks]), acc, 0, 0, 0);
      }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int j = j0 + 4 * g + i;
      const float bias = ld_f32(rbs, (unsigned)j * 4u);
      u[i] = j < me.nvis ? fmaf(acc[i], p.scale_log2, fmaxf(bias * kLog2eS, kNegBigS)) : -INFINITY;
    }
  };

  // pass 1: running max and sum per lane
  float m = -INFINITY, z = 0.f;
  for (int j0 = 0; j0 < kmax; j0 += 16) {
    float u[4];
    tile_u(j0, u);
    const float tm = fmaxf(fmaxf(u[0], u[1]), fmaxf(u[2], u[3]));
    if (tm > m) {
      z = (m == -INFINITY) ? 0.f : z * __builtin_amdgcn_exp2f(m - tm);
      m = tm;
    }
    if (m != -INFINITY)
#pragma unroll
      for (int i = 0; i < 4; ++i) z += __builtin_amdgcn_exp2f(u[i] - m);
  }
  const float mrow = max4(m);
  const float zrow = sum4(m == -INFINITY ? 0.f : z * __builtin_amdgcn_exp2f(m - mrow));
  const float lse2 = me.nvis > 0 ? mrow + __log2f(zrow) : 0.f;

  // pass 2: exact probabilities, O, region masses, entropy
  f32x4 oacc[NB];
#pragma unroll
  for (int db = 0; db < NB; ++db) oacc[db] = f32x4{0.f, 0.f, 0.f, 0.f};
  float ra[KVPROF_MAX_REGIONS];
#pragma unroll
  for (int q = 0; q < KVPROF_MAX_REGIONS; ++q) ra[q] = 0.f;
  float hs = 0.f;
  for (int j0 = 0; j0 < kmax; j0 += 16) {
    float u[4];
    tile_u(j0, u);
    f16x4 pa;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int j = j0 + 4 * g + i;
      const bool vis = j < me.nvis;
      const float pj = vis ? __builtin_amdgcn_exp2f(u[i] - lse2) : 0.f;
      hs += vis ? pj * (lse2 - u[i]) : 0.f;
#pragma unroll
      for (int q = 0; q < KVPROF_MAX_REGIONS; ++q)
        if (q < p.n_regions) ra[q] += (j >= p.region_bounds[q] && j < p.region_bounds[q + 1]) ? pj : 0.f;
      pa[i] = (_Float16)(pj * kPScaleS);
    }
    if (p.o) {
#pragma unroll
      for (int db = 0; db < NB; ++db) {
        f16x4 vh, vl;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          _Float16 xh, xl;
          v_val<D, KSRC>(rv, L, p.n_k, j0 + 4 * g + i, 16 * db + r, xh, xl);
          vh[i] = xh;
          vl[i] = xl;
        }
        oacc[db] = __builtin_amdgcn_mfma_f32_16x16x16f16(pa, vh, oacc[db], 0, 0, 0);
        if (KSRC == KSRC_INT4) oacc[db] = __builtin_amdgcn_mfma_f32_16x16x16f16(pa, vl, oacc[db], 0, 0, 0);
      }
    }
  }
  hs = sum4(hs);
#pragma unroll
  for (int q = 0; q < KVPROF_MAX_REGIONS; ++q) ra[q] = sum4(ra[q]);
  if (g == 0 && me.ok) {
    if (p.row_max) p.row_max[me.grow] = mrow * kLn2S;
    if (p.row_lse) p.row_lse[me.grow] = lse2 * kLn2S;
    if (p.support) p.support[me.grow] = expf(hs * kLn2S) / (float)me.nvis;
    if (p.region_mass)
      for (int q = 0; q < p.n_regions; ++q) p.region_mass[me.grow * p.n_regions + q] = ra[q];
  }
  if (p.o) {
    // O tile: lane l holds rows 4 (l / 16) + i of the wave, channel 16 db + l % 16
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const RowOf ro = row_of(p, b, hkv, rl0 + 4 * g + i);
      if (ro.ok) {
#pragma unroll
        for (int db = 0; db < NB; ++db) p.o[ro.grow * D + 16 * db + r] = oacc[db][i] * (1.f / kPScaleS);
      }
    }
  }
}

template <int D, int KSRC>
hipError_t launch_d(const ShortParams& p, hipStream_t s) {
  const long long nrb = (p.rows_per_kv + 16 * SW - 1) / (16 * SW);
  const long long nwg = (long long)p.n_batch * p.n_heads_kv * nrb;
  if (nwg == 0) return hipSuccess;
  hipLaunchKernelGGL((short_kernel<D, KSRC>), dim3((unsigned)nwg), dim3(SW * 64), 0, s, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attend_short(const ShortParams& p, int d, int ksrc, hipStream_t s) {
  if (d == 32) return ksrc == KSRC_INT4 ? launch_d<32, KSRC_INT4>(p, s) : launch_d<32, KSRC_BF16>(p, s);
  if (d == 64) return ksrc == KSRC_INT4 ? launch_d<64, KSRC_INT4>(p, s) : launch_d<64, KSRC_BF16>(p, s);
  return hipErrorInvalidValue;
}

}  // namespace kvp
