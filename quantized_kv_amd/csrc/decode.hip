// Split-key attention for decode steps: at most 16 query rows per (batch, KV head) — one GQA group at
// one or a few positions — over a long cache, bf16 or packed 4-bit K/V. Outputs O, the top-32 key
// indices, region masses, row max and log-sum-exp ("KV residual window": attention over the
// dequantized cache and the recent-window mass; the MiniCPM5-2B predictor study, section 0: the GQA
// decode shape and recall@32).
//
// A decode step reads every cached byte once, so the launch must spread one sequence's keys over
// many workgroups. One workgroup = one 1,024-key chunk of one (batch, KV head): 4 waves x 16 tiles of
// 16 keys, S^T = K Q^T on 16x16x32 MFMAs (lane l: row l % 16, keys 4 (l / 16) + i of a tile), with
// every score of the chunk kept in registers. Per chunk and row it records, in the workspace:
//   m   the chunk max of u = s log2(e),          z   sum 2^(u - m),
//   reg the region sums of 2^(u - m),             o   sum 2^(u - m) v (P.V on 16x16x16 f16 MFMAs),
//   the chunk's exact top-32 (u, j), and a flag when the candidate list overflowed.
// Top-32 inside a chunk: a 64-bin LDS histogram of (m - u) (bins of 1/2 in log2 units) locates the bin
// of rank 31; the keys of that bin and above (about 50 on random rows) are gathered and ranked exactly by
// (u descending, j ascending). A merge kernel then combines the chunks by log-sum-exp rescaling and
// ranks the chunks' candidates; rows whose candidates overflowed (ties crowding one bin, or fewer than
// 32 keys within 32 log2 units of the max) are finished by an exact fallback that re-scores the whole
// row in float32 and sorts it in LDS.
#include "kvprof_internal.h"
#include "kvprof_device.h"


namespace kvp {
namespace {

constexpr int DW = 4;                 // waves per workgroup
constexpr int DTPW = kDecChunk / 16 / DW;  // 16-key tiles per wave
constexpr int DBINS = 64;
constexpr int DCAP = 96;              // candidate slots per row and chunk
constexpr float kLog2eD = 1.44269504088896340736f;
constexpr float kLn2D = 0.69314718055994530942f;
constexpr float kNegBigD = -1.0e37f;
constexpr float kPScaleD = 32768.f;
constexpr unsigned kOORD = 0x7FFF0000u;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef __amdgpu_buffer_rsrc_t rsrc_t;

__device__ __forceinline__ rsrc_t drsrc(const void* base, size_t bytes) {
  const size_t cap = 0x7fffffff;
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)(bytes < cap ? bytes : cap),
                                           0x00020000);
}
__device__ __forceinline__ float hlo(uint32_t w) { return (float)__builtin_bit_cast(_Float16, (uint16_t)(w & 0xFFFFu)); }
__device__ __forceinline__ float hhi(uint32_t w) { return (float)__builtin_bit_cast(_Float16, (uint16_t)(w >> 16)); }
__device__ __forceinline__ float max4d(float x) {
  x = fmaxf(x, __shfl_xor(x, 16));
  return fmaxf(x, __shfl_xor(x, 32));
}
__device__ __forceinline__ float sum4d(float x) {
  x += __shfl_xor(x, 16);
  return x + __shfl_xor(x, 32);
}

struct DRow {
  bool ok;
  long long grow;
  int nvis;
};
__device__ __forceinline__ DRow drow(const DecParams& p, int b, int hkv, int slot) {
  DRow o;
  o.ok = slot < p.rows_per_kv;
  const int hloc = o.ok ? slot / p.n_q : 0;
  const int qi = o.ok ? slot - hloc * p.n_q : 0;
  o.grow = ((long long)b * p.n_heads_q + (long long)hkv * p.group + hloc) * p.n_q + qi;
  int nv = p.n_k;
  if (p.causal) {
    const long long v = p.q_pos0 + qi + 1;
    nv = v < (long long)p.n_k ? (int)v : p.n_k;
  }
  o.nvis = o.ok ? nv : 0;
  return o;
}

// A-operand fragment of K (key j, dims c0 .. c0+7): bf16 as is; 4-bit as an f16 hi + lo pair (exact),
// the 4-bit and float32-window words both loaded and one selected (reads outside a section return 0).
template <int KSRC, bool WIN>
__device__ __forceinline__ u32x4 dk_frag(rsrc_t rk, const Int4Layout& L, int n_k, int j, int c0, u32x4& lo) {
  if (KSRC == KSRC_BF16) {
    lo = u32x4{0u, 0u, 0u, 0u};
    return __builtin_amdgcn_raw_buffer_load_b128(rk, (unsigned)(j * 128 + c0) * 2u, 0, 0);
  } else {
    const bool quant = j < (int)L.n;
    const int jq = quant ? j : 0;
    const uint32_t codes = __builtin_amdgcn_raw_buffer_load_b32(rk, (unsigned)(L.kc + (size_t)jq * 64 + c0 / 2), 0, 0);
    const unsigned mo = (unsigned)(L.km + ((size_t)(jq >> 5) * 128 + c0) * 4);
    const u32x4 m0 = __builtin_amdgcn_raw_buffer_load_b128(rk, mo, 0, 0);
    const u32x4 m1 = __builtin_amdgcn_raw_buffer_load_b128(rk, mo + 16u, 0, 0);
    f32x4 a = {0.f, 0.f, 0.f, 0.f}, bb = a;
    if (WIN) {  // the tile reaches the float32 window
      const unsigned ro = (quant || j >= n_k) ? kOORD : (unsigned)(L.kr + ((size_t)(j - (int)L.n) * 128 + c0) * 4);
      a = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(rk, ro, 0, 0));
      bb = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(rk, ro + 16u, 0, 0));
    }
    f16x8 h, hl;
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      const uint32_t wd = c < 4 ? m0[c] : m1[c - 4];
      const float qv = fmaf((float)((codes >> (4 * c)) & 0xFu), hlo(wd), hhi(wd));
      const float x = quant ? qv : (c < 4 ? a[c] : bb[c - 4]);
      h[c] = (_Float16)x;
      hl[c] = (_Float16)(x - (float)h[c]);
    }
    lo = __builtin_bit_cast(u32x4, hl);
    return __builtin_bit_cast(u32x4, h);
  }
}

// V of key j, channels c0 .. c0+15, as f16 (bf16 exactly; dequantized 4-bit rounded once).
template <int KSRC>
__device__ __forceinline__ void dv16(rsrc_t rv, const Int4Layout& L, int n_k, int j, int c0, bool win, _Float16 (&x)[16]) {
  if (KSRC == KSRC_BF16) {
    const u32x4 v0 = __builtin_amdgcn_raw_buffer_load_b128(rv, (unsigned)(j * 128 + c0) * 2u, 0, 0);
    const u32x4 v1 = __builtin_amdgcn_raw_buffer_load_b128(rv, (unsigned)(j * 128 + c0 + 8) * 2u, 0, 0);
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const uint32_t wd = e < 8 ? v0[e >> 1] : v1[(e - 8) >> 1];
      x[e] = (_Float16)__uint_as_float(((wd >> (16 * (e & 1))) & 0xFFFFu) << 16);
    }
  } else {
    const bool quant = j < (int)L.n;
    const int jq = quant ? j : 0;
    const u32x2 codes = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(rv, (unsigned)(L.vc + (size_t)jq * 64 + c0 / 2), 0, 0));
    const uint32_t wd = __builtin_amdgcn_raw_buffer_load_b32(rv, (unsigned)(L.vm + ((size_t)jq * 4 + c0 / 32) * 4), 0, 0);
    f32x4 r4[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) r4[q] = f32x4{0.f, 0.f, 0.f, 0.f};
    if (win) {  // uniform: the tile reaches the float32 window
      const unsigned ro = (quant || j >= n_k) ? kOORD : (unsigned)(L.vr + ((size_t)(j - (int)L.n) * 128 + c0) * 4);
#pragma unroll
      for (int q = 0; q < 4; ++q) r4[q] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(rv, ro + 16u * q, 0, 0));
    }
    const float s_ = hlo(wd), m_ = hhi(wd);
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const float qv = fmaf((float)((codes[e >> 3] >> (4 * (e & 7))) & 0xFu), s_, m_);
      x[e] = (_Float16)(quant ? qv : r4[e >> 2][e & 3]);
    }
  }
}

// S^T tile: key j (this lane's A row) against the 16 rows' Q fragments.
template <int KSRC, bool WIN>
__device__ __forceinline__ f32x4 score_tile(rsrc_t rk, const Int4Layout& L, int n_k, int j, int g, const u32x4 (&qf)[4]) {
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
    u32x4 lo;
    const u32x4 hi = dk_frag<KSRC, WIN>(rk, L, n_k, j, 32 * ks + 8 * g, lo);
    if (KSRC == KSRC_BF16) {
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, hi), __builtin_bit_cast(bf16x8, qf[ks]), acc, 0, 0, 0);
    } else {
      acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, hi), __builtin_bit_cast(f16x8, qf[ks]), acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, lo), __builtin_bit_cast(f16x8, qf[ks]), acc, 0, 0, 0);
    }
  }
  return acc;
}

template <int KSRC>
__global__ __launch_bounds__(DW * 64) void dec_chunk_kernel(const DecParams p) {
  __shared__ float s_m[DW][16];
  __shared__ float s_z[DW][16];
  __shared__ float s_reg[DW][16][KVPROF_MAX_REGIONS];
  __shared__ unsigned s_hist[16][DBINS];
  __shared__ int s_nc[16];
  __shared__ int s_b[16];  // boundary bin of rank need - 1; -1: the row has no candidate to rank
  __shared__ int s_flag[16];
  __shared__ float s_cu[16][DCAP];
  __shared__ int s_cj[16][DCAP];
  __shared__ uint32_t s_v[DW][128][10];  // per wave: 128 channels x 16 keys of V (f16 pairs), padded to keep 8-byte reads aligned
  __shared__ float s_o[16][129];

  const int S = p.n_chunks;
  const int c = blockIdx.x % S;
  const int bkv = blockIdx.x / S;
  const int hkv = bkv % p.n_heads_kv;
  const int b = bkv / p.n_heads_kv;
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
  const int r = lane & 15, g = lane >> 4;
  const int key0 = c * kDecChunk;
  const DRow me = drow(p, b, hkv, r);

  for (int i = tid; i < 16 * DBINS; i += DW * 64) (&s_hist[0][0])[i] = 0u;
  if (tid < 16) {
    s_nc[tid] = 0;
    s_flag[tid] = 0;
  }

  u32x4 qf[4];
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
    u32x4 v = u32x4{0u, 0u, 0u, 0u};
    if (me.ok) v = *reinterpret_cast<const u32x4*>(p.q + me.grow * 128 + 32 * ks + 8 * g);
    if (KSRC == KSRC_INT4) {
      f16x8 hq;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        hq[2 * e] = (_Float16)__uint_as_float(v[e] << 16);
        hq[2 * e + 1] = (_Float16)__uint_as_float(v[e] & 0xFFFF0000u);
      }
      v = __builtin_bit_cast(u32x4, hq);
    }
    qf[ks] = v;
  }
  const size_t kvh = (size_t)b * p.n_heads_kv + hkv;
  rsrc_t rk, rv;
  Int4Layout L{};
  if (KSRC == KSRC_BF16) {
    rk = drsrc(p.k + kvh * p.n_k * 128, (size_t)p.n_k * 256);
    rv = drsrc(p.v ? p.v + kvh * p.n_k * 128 : p.k, p.v ? (size_t)p.n_k * 256 : 0);
  } else {
    rk = drsrc(p.kv_packed + kvh * p.blob_bytes, p.blob_bytes);
    rv = rk;
    L = int4_layout(p.n_k, 128, p.r_window);
  }
  const rsrc_t rbs = drsrc(p.key_bias ? (const void*)p.key_bias : (const void*)p.q, p.key_bias ? (size_t)p.n_k * 4 : 0);

  // ---- scores of this wave's 16 tiles (keys wk0 .. wk0 + 255) --------------------------------------
  const int wk0 = key0 + w * DTPW * 16;
  float u[DTPW][4];
#pragma unroll
  for (int t = 0; t < DTPW; ++t) {
    const int j0 = wk0 + 16 * t;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    if (j0 < p.n_k) {  // uniform
      if (KSRC == KSRC_INT4 && j0 + 16 > (int)L.n)  // uniform: the tile reaches the float32 window
        acc = score_tile<KSRC, true>(rk, L, p.n_k, j0 + r, g, qf);
      else
        acc = score_tile<KSRC, false>(rk, L, p.n_k, j0 + r, g, qf);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int j = j0 + 4 * g + i;
      const float bias = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rbs, (unsigned)j * 4u, 0, 0));
      u[t][i] = j < me.nvis ? fmaf(acc[i], p.scale_log2, fmaxf(bias * kLog2eD, kNegBigD)) : -INFINITY;
    }
  }

  // ---- chunk max per row ----------------------------------------------------------------------------
  float lm = -INFINITY;
#pragma unroll
  for (int t = 0; t < DTPW; ++t)
#pragma unroll
    for (int i = 0; i < 4; ++i) lm = fmaxf(lm, u[t][i]);
  lm = max4d(lm);
  if (g == 0) s_m[w][r] = lm;
  __syncthreads();
  float m = s_m[0][r];
#pragma unroll
  for (int ww = 1; ww < DW; ++ww) m = fmaxf(m, s_m[ww][r]);
  const bool any = m != -INFINITY;

  // ---- exponentials, sum, region sums, O, and the top-32 histogram --------------------------------
  float zl = 0.f;
  float ra[KVPROF_MAX_REGIONS];
#pragma unroll
  for (int q = 0; q < KVPROF_MAX_REGIONS; ++q) ra[q] = 0.f;
  f32x4 oacc[8];
#pragma unroll
  for (int db = 0; db < 8; ++db) oacc[db] = f32x4{0.f, 0.f, 0.f, 0.f};
  const int kp = lane & 7, q16 = lane >> 3;  // V staging: keys 2kp, 2kp + 1, channels 16 q16 .. + 15
#pragma unroll
  for (int t = 0; t < DTPW; ++t) {
    const int j0 = wk0 + 16 * t;
    if (j0 < p.n_k) {  // uniform
    // V tile -> LDS, channel-major, two keys packed per word
    {
      _Float16 x0[16], x1[16];
      const bool win = KSRC == KSRC_INT4 && j0 + 16 > (int)L.n;
      dv16<KSRC>(rv, L, p.n_k, j0 + 2 * kp, 16 * q16, win, x0);
      dv16<KSRC>(rv, L, p.n_k, j0 + 2 * kp + 1, 16 * q16, win, x1);
#pragma unroll
      for (int e = 0; e < 16; ++e)
        s_v[w][16 * q16 + e][kp] = (uint32_t)__builtin_bit_cast(uint16_t, x0[e]) | ((uint32_t)__builtin_bit_cast(uint16_t, x1[e]) << 16);
    }
    f16x4 pa;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int j = j0 + 4 * g + i;
      const float uu = u[t][i];
      const float e = (any && uu != -INFINITY) ? __builtin_amdgcn_exp2f(uu - m) : 0.f;
      zl += e;
#pragma unroll
      for (int q = 0; q < KVPROF_MAX_REGIONS; ++q)
        if (q < p.n_regions) ra[q] += (j >= p.region_bounds[q] && j < p.region_bounds[q + 1]) ? e : 0.f;
      pa[i] = (_Float16)(e * kPScaleD);
      if (any && uu > m - 32.f) {
        const int bin = min(DBINS - 1, (int)((m - uu) * 2.f));
        atomicAdd(&s_hist[r][bin], 1u);
      }
    }
    __atomic_signal_fence(__ATOMIC_SEQ_CST);  // the wave's LDS writes above complete before its reads below
#pragma unroll
    for (int db = 0; db < 8; ++db) {
      const u32x2 vw = *reinterpret_cast<const u32x2*>(&s_v[w][16 * db + r][2 * g]);  // keys 4g .. 4g+3
      oacc[db] = __builtin_amdgcn_mfma_f32_16x16x16f16(pa, __builtin_bit_cast(f16x4, vw), oacc[db], 0, 0, 0);
    }
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    }
  }
  zl = sum4d(zl);
#pragma unroll
  for (int q = 0; q < KVPROF_MAX_REGIONS; ++q) ra[q] = sum4d(ra[q]);
  if (g == 0) {
    s_z[w][r] = zl;
#pragma unroll
    for (int q = 0; q < KVPROF_MAX_REGIONS; ++q) s_reg[w][r][q] = ra[q];
  }
  // O across the waves, in wave order (lane l holds rows 4g + i, channel 16 db + r)
  for (int ww = 0; ww < DW; ++ww) {
    if (w == ww) {
#pragma unroll
      for (int db = 0; db < 8; ++db)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          float& d = s_o[4 * g + i][16 * db + r];
          d = (ww == 0 ? 0.f : d) + oacc[db][i];
        }
    }
    __syncthreads();
  }

  // ---- boundary bin of each row (wave w scans rows w, w + 4, ...) -----------------------------------
  for (int row = w; row < 16; row += DW) {
    const DRow ri = drow(p, b, hkv, row);
    const int nch = max(0, min(ri.nvis - key0, kDecChunk));  // visible keys of the row in this chunk
    const int need = min(32, nch);
    unsigned cnt = s_hist[row][lane];
    unsigned inc = cnt;
    for (int o = 1; o < 64; o <<= 1) {
      const unsigned t2 = __shfl_up(inc, o);
      if (lane >= o) inc += t2;
    }
    const unsigned total = __shfl(inc, 63);
    const unsigned long long hit = __ballot(need > 0 && inc >= (unsigned)need);
    if (lane == 0) {
      int bq = -1;
      if (need > 0) {
        if (total < (unsigned)need) s_flag[row] = 1;  // keys below the histogram window are needed
        else bq = __builtin_ctzll(hit);
      }
      s_b[row] = bq;
    }
  }
  __syncthreads();
  // ---- gather the candidates (bins 0 .. s_b) --------------------------------------------------------
  {
    const int bq = s_b[r];
#pragma unroll
    for (int t = 0; t < DTPW; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float uu = u[t][i];
        if (bq >= 0 && uu > m - 32.f && min(DBINS - 1, (int)((m - uu) * 2.f)) <= bq) {
          const int slot = atomicAdd(&s_nc[r], 1);
          if (slot < DCAP) {
            s_cu[r][slot] = uu;
            s_cj[r][slot] = wk0 + 16 * t + 4 * g + i;
          }
        }
      }
  }
  __syncthreads();
  // ---- rank the candidates, write the chunk record --------------------------------------------------
  for (int row = w; row < 16; row += DW) {
    const DRow ri = drow(p, b, hkv, row);
    if (!ri.ok) continue;  // uniform over the wave
    float* rec = p.part + (((size_t)bkv * S + c) * 16 + row) * kDecRecWords;
    const int nc = s_nc[row];
    const int flag = s_flag[row] | (nc > DCAP ? 1 : 0);
    const int ncl = min(nc, DCAP);
    float mm = s_m[0][row];
    for (int ww = 1; ww < DW; ++ww) mm = fmaxf(mm, s_m[ww][row]);
    if (lane == 0) {
      float z = 0.f;
      for (int ww = 0; ww < DW; ++ww) z += s_z[ww][row];
      rec[kDecM] = mm;
      rec[kDecZ] = z;
      rec[kDecFlag] = flag ? 1.f : 0.f;
    }
    if (lane < KVPROF_MAX_REGIONS) {
      float a = 0.f;
      for (int ww = 0; ww < DW; ++ww) a += s_reg[ww][row][lane];
      rec[kDecReg + lane] = a;
    }
    for (int ch = lane; ch < 128; ch += 64) rec[kDecO + ch] = s_o[row][ch] * (1.f / kPScaleD);
    if (lane < 32) {
      rec[kDecCu + lane] = -INFINITY;
      reinterpret_cast<int*>(rec)[kDecCj + lane] = -1;
    }
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    for (int a = lane; a < ncl; a += 64) {
      const float ua = s_cu[row][a];
      const int ja = s_cj[row][a];
      int rank = 0;
      for (int q = 0; q < ncl; ++q) {
        const float uq = s_cu[row][q];
        rank += (uq > ua) || (uq == ua && s_cj[row][q] < ja);
      }
      if (rank < 32) {
        rec[kDecCu + rank] = ua;
        reinterpret_cast<int*>(rec)[kDecCj + rank] = ja;
      }
    }
  }
}

// One wave per row: combine the chunks (log-sum-exp rescaling), rank the chunks' candidates, and write
// the row's outputs. Rows whose candidates overflowed in some chunk are marked for the fallback.
__global__ __launch_bounds__(64) void dec_merge_kernel(const DecParams p) {
  __shared__ float s_cu[32 * kDecMaxChunks];
  __shared__ int s_cj[32 * kDecMaxChunks];
  const int lane = threadIdx.x;
  const int S = p.n_chunks;
  const long long nslots = (long long)p.n_batch * p.n_heads_kv * 16;
  for (long long sl = blockIdx.x; sl < nslots; sl += gridDim.x) {
    const int slot = (int)(sl % 16);
    const long long bkv = sl / 16;
    const int hkv = (int)(bkv % p.n_heads_kv), b = (int)(bkv / p.n_heads_kv);
    const DRow ri = drow(p, b, hkv, slot);
    if (!ri.ok) continue;
    const float* rec0 = p.part + ((size_t)bkv * S * 16 + slot) * kDecRecWords;
    auto rec = [&](int c) { return rec0 + (size_t)c * 16 * kDecRecWords; };
    float m = -INFINITY;
    int flag = 0;
    for (int c = 0; c < S; ++c) {
      m = fmaxf(m, rec(c)[kDecM]);
      flag |= rec(c)[kDecFlag] != 0.f;
    }
    float z = 0.f, o0 = 0.f, o1 = 0.f, rg = 0.f;
    for (int c = 0; c < S; ++c) {
      const float mc = rec(c)[kDecM];
      const float wgt = mc == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(mc - m);
      z += wgt * rec(c)[kDecZ];
      o0 += wgt * rec(c)[kDecO + lane];
      o1 += wgt * rec(c)[kDecO + 64 + lane];
      if (lane < p.n_regions) rg += wgt * rec(c)[kDecReg + lane];
    }
    const float iz = z > 0.f ? 1.f / z : 0.f;
    if (p.o) {
      p.o[ri.grow * 128 + lane] = o0 * iz;
      p.o[ri.grow * 128 + 64 + lane] = o1 * iz;
    }
    if (p.region_mass && lane < p.n_regions) p.region_mass[ri.grow * p.n_regions + lane] = rg * iz;
    if (lane == 0) {
      if (p.row_max) p.row_max[ri.grow] = m * kLn2D;
      if (p.row_lse) p.row_lse[ri.grow] = (m + log2f(z)) * kLn2D;
      p.flags[ri.grow] = flag;
    }
    if (p.top32) {
      // the chunks' candidates (32 each) ranked by (u descending, j ascending)
      for (int a = lane; a < 32 * S; a += 64) {
        s_cu[a] = rec(a / 32)[kDecCu + a % 32];
        s_cj[a] = reinterpret_cast<const int*>(rec(a / 32))[kDecCj + a % 32];
      }
      __syncthreads();
      for (int a = lane; a < 32 * S; a += 64) {
        const float ua = s_cu[a];
        const int ja = s_cj[a];
        int rank = 0;
        for (int q = 0; q < 32 * S; ++q) {
          const float uq = s_cu[q];
          const int jq = s_cj[q];
          rank += jq >= 0 && ((uq > ua) || (uq == ua && jq < ja));
        }
        if (ja >= 0 && rank < 32) p.top32[ri.grow * 32 + rank] = ja;
      }
      // positions past the row's visible keys
      if (lane < 32 && lane >= ri.nvis) p.top32[ri.grow * 32 + lane] = -1;
      __syncthreads();
    }
  }
}

// Exact fallback for flagged rows: the whole row re-scored in float32 (the dequantized K, the same
// value the MFMA path sees), keys sorted in LDS by (u descending, j ascending), the first 32 written.
constexpr int kFbThreads = 256;
template <int KSRC>
__global__ __launch_bounds__(kFbThreads) void dec_fallback_kernel(const DecParams p) {
  __shared__ unsigned long long keys[kDecMaxKeys];
  const long long rows = (long long)p.n_batch * p.n_heads_q * p.n_q;
  for (long long grow = blockIdx.x; grow < rows; grow += gridDim.x) {
    if (!p.flags[grow]) continue;  // uniform over the workgroup
    const int qi = (int)(grow % p.n_q);
    const long long bh = grow / p.n_q;
    const int hq = (int)(bh % p.n_heads_q), b = (int)(bh / p.n_heads_q);
    const int hkv = hq / p.group;
    int nvis = p.n_k;
    if (p.causal) {
      const long long v = p.q_pos0 + qi + 1;
      nvis = v < (long long)p.n_k ? (int)v : p.n_k;
    }
    const size_t kvh = (size_t)b * p.n_heads_kv + hkv;
    Int4Layout L{};
    if (KSRC == KSRC_INT4) L = int4_layout(p.n_k, 128, p.r_window);
    const uint8_t* blob = KSRC == KSRC_INT4 ? p.kv_packed + kvh * p.blob_bytes : nullptr;
    int npow = 1;
    while (npow < p.n_k) npow <<= 1;
    for (int j = threadIdx.x; j < npow; j += blockDim.x) {
      unsigned long long key = 0ull;  // sorts below every real key
      if (j < nvis) {
        float s = 0.f;
        for (int c = 0; c < 128; ++c) {
          const float qv = bf16_to_f32(p.q[grow * 128 + c]);
          float kv;
          if (KSRC == KSRC_BF16) {
            kv = bf16_to_f32(p.k[(kvh * p.n_k + j) * 128 + c]);
          } else if (j < (int)L.n) {
            const uint8_t byte = blob[L.kc + (size_t)j * 64 + c / 2];
            const uint32_t code = (c & 1) ? (byte >> 4) : (byte & 0xFu);
            const _Float16* mt = reinterpret_cast<const _Float16*>(blob + L.km) + ((size_t)(j >> 5) * 128 + c) * 2;
            kv = fmaf((float)code, (float)mt[0], (float)mt[1]);
          } else {
            kv = reinterpret_cast<const float*>(blob + L.kr)[(size_t)(j - L.n) * 128 + c];
          }
          s = fmaf(qv, kv, s);
        }
        const float bias = p.key_bias ? p.key_bias[j] : 0.f;
        const float uu = fmaf(s, p.scale_log2, fmaxf(bias * kLog2eD, kNegBigD));
        const unsigned bits = __float_as_uint(uu);
        const unsigned ord = (bits & 0x80000000u) ? ~bits : (bits | 0x80000000u);
        key = ((unsigned long long)ord << 32) | (0xFFFFFFFFu - (unsigned)j);  // larger = earlier
      }
      keys[j] = key;
    }
    __syncthreads();
    // bitonic sort, descending
    for (int k2 = 2; k2 <= npow; k2 <<= 1)
      for (int jj = k2 >> 1; jj > 0; jj >>= 1) {
        for (int i = threadIdx.x; i < npow; i += blockDim.x) {
          const int l2 = i ^ jj;
          if (l2 > i) {
            const unsigned long long a = keys[i], bb = keys[l2];
            const bool desc = (i & k2) == 0;
            if (desc ? a < bb : a > bb) {
              keys[i] = bb;
              keys[l2] = a;
            }
          }
        }
        __syncthreads();
      }
    if (threadIdx.x < 32)
      p.top32[grow * 32 + threadIdx.x] =
          (int)threadIdx.x < nvis ? (int)(0xFFFFFFFFu - (unsigned)(keys[threadIdx.x] & 0xFFFFFFFFull)) : -1;
    __syncthreads();
  }
}

template <int KSRC>
hipError_t launch_k(const DecParams& p, hipStream_t s) {
  const long long nbkv = (long long)p.n_batch * p.n_heads_kv;
  if (nbkv == 0) return hipSuccess;
  hipLaunchKernelGGL(dec_chunk_kernel<KSRC>, dim3((unsigned)(nbkv * p.n_chunks)), dim3(DW * 64), 0, s, p);
  const long long slots = nbkv * 16;
  hipLaunchKernelGGL(dec_merge_kernel, dim3((unsigned)(slots < 65536 ? slots : 65536)), dim3(64), 0, s, p);
  if (p.top32) {
    const long long rows = (long long)p.n_batch * p.n_heads_q * p.n_q;
    hipLaunchKernelGGL(dec_fallback_kernel<KSRC>, dim3((unsigned)(rows < 4096 ? rows : 4096)), dim3(kFbThreads), 0, s, p);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_decode(const DecParams& p, int ksrc, hipStream_t s) {
  return ksrc == KSRC_INT4 ? launch_k<KSRC_INT4>(p, s) : launch_k<KSRC_BF16>(p, s);
}

}  // namespace kvp
