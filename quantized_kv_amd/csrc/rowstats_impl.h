// Row kernel of the KV-cache attention row profiler (template; instantiated by rowstats_*.hip).
//
// One workgroup = 8 waves = 16 query rows (the 16 columns of a 16x16 MFMA tile) of one (batch,
// KV head). Wave w owns keys [w*TPW*16, (w+1)*TPW*16). The whole score row of every query stays on
// chip: each lane holds one row's scores for 4 keys of each of its TPW tiles, as produced by the MFMA
// S^T = K Q^T (lane l: query row l%16, keys 4*(l/16)+i of the tile). Every statistic is then a pass
// over registers, with cross-lane / cross-wave reductions in a fixed order (bitwise deterministic):
//
//   A  scores u = (scale q.k + b) log2(e) on bf16 / f16 MFMA; row max, min, mean and deviation
//   B  e' = 2^(u - max + 31); Z', sum e'(u - max + 31) for the entropy; per-segment masses (regions,
//      key frames); and, for the keys above a selection threshold T (mean + 0.8 sd), a 256-bin
//      histogram over [T, max] with counts and fixed-point masses round(e'). The registers keep u:
//      ranks are taken on scores, which never underflow.
//   D  exact selection of four ranks (top-32 boundary, top-1/5/10 %): one gather of the keys ranked
//      above the top-32 boundary bin and of the boundary bins' keys, ranked exactly in LDS; rare
//      overfull bins are refined by further radix levels on (order key, key index)
//   E  outputs; optional O = P.V on f16 MFMA; MXFP8 mode adds the bf16 reference row (TV, argmax)
//      and the per-32-key E4M3/E8M0 probability path.
//
// Definitions ("Catnip Week 10 KV Cache Attention Study"): the Structural / Effective / Numerical
// MXFP8 statistics of the experiment-design section, region masses of the KV-cache banner, frame
// masses of Figure 2, TV and argmax agreement of the quantization section. Recall@32 and the GQA
// layout: the MiniCPM5-2B predictor study, section 0. Int4 K/V source: "KV residual window".
#pragma once

#include "kvprof_internal.h"
#include "kvprof_device.h"

namespace kvp {
namespace {

constexpr int NW = 8;   // waves per workgroup: 2 per SIMD, so each lane may use 256 VGPRs
constexpr int WGT = NW * 64;
constexpr int ROWS = 16;
constexpr int HB = 257;  // padded histogram stride (rows land in different LDS banks)
constexpr int CAP = 256; // candidate slots per row (boundary bins)
constexpr int CAPL = CAP + 32;   // fast-path list: the boundary bins plus the keys ranked above them
constexpr int kRedoGrid = 256;  // workgroups of the redo kernel (they loop over the redo list)
constexpr int kVstStride = 10;  // 32-bit words per staged V channel row: 16 keys (f16) + 2 words of padding
constexpr float kOff = 31.f;    // e' = 2^(u - max + kOff): the largest key weighs 2^31
constexpr int NT = 4;    // selected ranks per row
constexpr float kLog2e = 1.44269504088896340736f;
constexpr float kLn2 = 0.69314718055994530942f;
constexpr float kPScale = 32768.f;  // P is fed to the f16 MFMA as p * 2^15
constexpr int kRing = 2;  // K tiles per wave in the LDS load ring (the load rate does not improve with more)
constexpr unsigned long long kOne = 1ull << 44;            // one key in a packed histogram counter
constexpr unsigned long long kMassMask = (1ull << 44) - 1;
constexpr float kNegBig = -1.0e37f;  // floor of the staged key bias
constexpr float kSelSigma = 0.8f;    // selection threshold: about mean + kSelSigma standard deviations
constexpr float kInterpTol = 4e-4f;  // bound on a top-f mass taken by interpolation inside its bin

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef unsigned long long u64x2 __attribute__((ext_vector_type(2)));

// Keys are ordered by (D, j): D the 32-bit order key of the score, j the key index. The group that
// holds a target's rank is narrowed one 8-bit digit at a time, first over D (phase 0: the group is
// {D >> sh == prefix}), then, if one value of D still holds too many keys, over j (phase 1: the
// group is {D == dfix, j >> sh == prefix}). All of it in 32-bit arithmetic.
struct TState {
  unsigned prefix;        // digits fixed so far
  unsigned dfix;          // phase 1: the order key shared by the group
  int ph, sh;             // phase and shift of the group's digits
  int valid;              // 0 for rows past the end of the problem
  int cnt_before;         // elements ranked before the group
  int cnt_in;             // elements in the group
  int target;             // 0-based rank to locate
  int resolved;
  int interp;             // top-f target whose mass comes from the level-1 bin by interpolation
  unsigned long long mass_in;      // interp: fixed-point mass of the target's bin
  unsigned long long mass_before;  // fixed-point mass (units of 1 / Z') ranked before the group
  float frac;
};

__device__ __forceinline__ bool ts_in(unsigned D, int j, int ph, int sh, unsigned pre, unsigned dfix) {
  return ph ? (D == dfix && ((unsigned)j >> sh) == pre) : ((D >> sh) == pre);
}
__device__ __forceinline__ bool ts_before(unsigned D, int j, int ph, int sh, unsigned pre, unsigned dfix) {
  return ph ? (D < dfix || (D == dfix && ((unsigned)j >> sh) < pre)) : ((D >> sh) < pre);
}

struct Sel {
  // one 64-bit counter per bin: key count in bits 44..63, fixed-point mass (2^31 = 1) in bits 0..43,
  // so a single LDS atomic per key updates both
  unsigned long long hist[ROWS][HB];
  union {
    struct {
      float ce[ROWS][CAPL];  // slow path: candidate scores u
      int cj[ROWS][CAPL];    // slow path: candidate key index
    };
    unsigned long long ck[ROWS][CAPL];  // fast path: rank keys (rank_key)
  };
  union {
    float sorted_e[ROWS][CAP];  // slow path: candidate e' by rank
    int crank[ROWS][CAPL];      // fast path: rank of a candidate inside its level-1 bin
    unsigned gbits[7][NW][64];  // fast-path gather: list membership of each lane's keys, 32 per word
  };
};

// NL: score tiles of each wave kept in LDS instead of registers (the rest of the kernel needs the
// registers they free).
template <int NL>
struct Smem {
  float red_a[NW][ROWS];
  float red_b[NW][ROWS];
  float red_e[NW][ROWS];
  int red_i[NW][ROWS];
  float red_c[NW][ROWS];
  float segpart[NW][ROWS][kSegPerWave];
  float segmass[ROWS][kMaxSeg];
  signed char sreg[kMaxSeg], sfr[kMaxSeg];  // region and frame of each segment
  int cs0[NW];
  float r_z[ROWS], r_e[ROWS], r_m[ROWS], r_mn[ROWS], r_T[ROWS], r_k8[ROWS];
  int rfb[ROWS];  // 1: the row's histogram is redone over every visible key
  int flag;
  TState ts[ROWS][NT];
  float tmass[ROWS][3];
  int ncand[ROWS], nwin[ROWS];
  alignas(16) float win_u[ROWS][32];  // scores of the top-32 keys
  alignas(16) int win_j[ROWS][32];
  int top0[ROWS];
  u32x4 qs[ROWS][17];  // Q rows as 16-byte chunks (B operand of S^T = K Q^T); padded against bank conflicts
  f32x4 stash[NL > 0 ? NL : 1][NW][64];  // score tiles 0 .. NL-1 of every wave, one f32x4 per lane
  union {
    Sel sel;
    float ored[NW / 2][ROWS][64];
    _Float16 vst[NW][64][2 * kVstStride];  // P.V: per wave, 64 channels x 16 keys of V (f16), padded
    struct {
      u32x4 ring[NW][kRing][4][64];  // per wave: kRing K tiles x 4 k-steps x 64 lanes (A fragments)
      float rbias[NW][kRing][16];    // the tiles' raw key bias
    } a;
  } u;
};

struct RowInfo {
  bool ok;
  long long grow;  // global output row
  int qi;          // query index inside its head
  int nvis;        // visible keys
};

__device__ __forceinline__ RowInfo row_info(const RowStatsParams& p, int b, int hkv, int rb, int r) {
  RowInfo ri;
  int rl = rb * ROWS + r;
  ri.ok = rl < p.rows_per_kv;
  int hloc = ri.ok ? rl / p.n_q : 0;
  ri.qi = ri.ok ? rl - hloc * p.n_q : 0;
  int hq = hkv * p.group + hloc;
  ri.grow = ((long long)b * p.n_heads_q + hq) * p.n_q + ri.qi;
  int nv = p.n_k;
  if (p.causal) {
    long long v = p.q_pos0 + ri.qi + 1;
    nv = v < (long long)p.n_k ? (int)v : p.n_k;
  }
  ri.nvis = ri.ok ? nv : 0;
  return ri;
}

// Cross-lane exchanges without LDS round trips. A permlane16 swap of x with itself leaves lane l
// holding x of lane l and x of lane l ^ 16 in its two results (which one is which depends on the
// row), a permlane32 swap the same for lane l ^ 32; DPP moves serve the exchanges inside a row of 16.
// Every step combines two lanes that hold the same partial result, so all lanes end with the same
// bits (fixed order, deterministic).
__device__ __forceinline__ u32x2 swap16(unsigned x) {
  const auto r = __builtin_amdgcn_permlane16_swap(x, x, false, false);
  return u32x2{r[0], r[1]};
}
__device__ __forceinline__ u32x2 swap32(unsigned x) {
  const auto r = __builtin_amdgcn_permlane32_swap(x, x, false, false);
  return u32x2{r[0], r[1]};
}
template <int CTRL>
__device__ __forceinline__ unsigned dpp_mov(unsigned x) {
  return (unsigned)__builtin_amdgcn_update_dpp(0, (int)x, CTRL, 0xF, 0xF, false);
}
constexpr int kDppXor1 = 0xB1;        // quad_perm [1,0,3,2]
constexpr int kDppXor2 = 0x4E;        // quad_perm [2,3,0,1]
constexpr int kDppHalfMirror = 0x141; // lane i of an 8-lane half-row reads lane 7 - i
constexpr int kDppMirror = 0x140;     // lane i of a 16-lane row reads lane 15 - i

// Sum over the 4 lanes that hold one row (lanes r, r+16, r+32, r+48); same result on all four.
__device__ __forceinline__ float row_sum4(float x) {
  u32x2 s = swap16(__float_as_uint(x));
  x = __uint_as_float(s[0]) + __uint_as_float(s[1]);
  s = swap32(__float_as_uint(x));
  return __uint_as_float(s[0]) + __uint_as_float(s[1]);
}
__device__ __forceinline__ float row_max4(float x) {
  u32x2 s = swap16(__float_as_uint(x));
  x = fmaxf(__uint_as_float(s[0]), __uint_as_float(s[1]));
  s = swap32(__float_as_uint(x));
  return fmaxf(__uint_as_float(s[0]), __uint_as_float(s[1]));
}
__device__ __forceinline__ float row_min4(float x) {
  u32x2 s = swap16(__float_as_uint(x));
  x = fminf(__uint_as_float(s[0]), __uint_as_float(s[1]));
  s = swap32(__float_as_uint(x));
  return fminf(__uint_as_float(s[0]), __uint_as_float(s[1]));
}
__device__ __forceinline__ int row_isum4(int x) {
  u32x2 s = swap16((unsigned)x);
  x = (int)(s[0] + s[1]);
  s = swap32((unsigned)x);
  return (int)(s[0] + s[1]);
}
// Sum over a whole wave (every lane must be active).
__device__ __forceinline__ float wave_sum(float x) {
  x += __uint_as_float(dpp_mov<kDppXor1>(__float_as_uint(x)));
  x += __uint_as_float(dpp_mov<kDppXor2>(__float_as_uint(x)));
  x += __uint_as_float(dpp_mov<kDppHalfMirror>(__float_as_uint(x)));
  x += __uint_as_float(dpp_mov<kDppMirror>(__float_as_uint(x)));
  return row_sum4(x);
}
// Max / min over the 16 lanes of a row (every lane must be active).
__device__ __forceinline__ int row16_max(int x) {
  x = max(x, (int)dpp_mov<kDppXor1>((unsigned)x));
  x = max(x, (int)dpp_mov<kDppXor2>((unsigned)x));
  x = max(x, (int)dpp_mov<kDppHalfMirror>((unsigned)x));
  return max(x, (int)dpp_mov<kDppMirror>((unsigned)x));
}
__device__ __forceinline__ int row16_min(int x) {
  x = min(x, (int)dpp_mov<kDppXor1>((unsigned)x));
  x = min(x, (int)dpp_mov<kDppXor2>((unsigned)x));
  x = min(x, (int)dpp_mov<kDppHalfMirror>((unsigned)x));
  return min(x, (int)dpp_mov<kDppMirror>((unsigned)x));
}

// Returns x through an empty asm statement: values derived from the copy are computed where the copy
// is made. Used at the top of each pass over the score registers so that the compiler does not hoist
// per-key work (validity tests, order keys) out of the pass loops and keep it live in registers.
template <typename T>
__device__ __forceinline__ T opaque(T x) {
  asm volatile("" : "+v"(x));
  return x;
}

// Level-1 bin of a score at or above the row's selection threshold T: 256 equal bins over
// [T, max], bin 0 holding the largest scores. Monotone (a larger score never gets a larger bin);
// explicit rounding intrinsics make every pass compute the identical bin.
__device__ __forceinline__ float bin_scale(float m, float T) {
  const float d = m - T;
  return (d > 1e-20f && d < 1e30f) ? 256.f / d : 0.f;  // 0: every key in bin 0 (ranked by index)
}
// x = (max - u) k8 as one rounding: fma(-u, k8, mk8) with mk8 = round(max k8). Monotone in u.
__device__ __forceinline__ int bin1(float u, float k8, float mk8) {
  return (int)fminf(__fmaf_rn(-u, k8, mk8), 255.f);  // (a tiny negative x truncates to bin 0)
}
// 32-bit order key for the refinement levels: the same quantity scaled by 2^24 (k32 = k8 2^24,
// mk32 = mk8 2^24, exact powers of two, so key >> 24 is the level-1 bin).
__device__ __forceinline__ unsigned dkey32(float u, float k32, float mk32) {
  return (unsigned)fminf(fmaxf(__fmaf_rn(-u, k32, mk32), 0.f), 4294967040.f);
}
// Fixed-point mass of a key: trunc(e') <= 2^31 (an error below 2^-31 of the largest key's weight).
__device__ __forceinline__ unsigned fixmass(float e) { return (unsigned)e; }

// Rank key of a gathered key: level-1 bin (bits 48..55), then the score descending (its bits mapped
// to an increasing unsigned order, complemented: bits 16..47), then the key index (bits 0..15). Keys
// of one bin are contiguous and ordered as the ranks are defined (score descending, index
// ascending), so a rank inside the bin is a count of smaller keys minus the keys of earlier bins.
__device__ __forceinline__ unsigned long long rank_key(float u, int j, int bin) {
  const unsigned b = __float_as_uint(u);
  const unsigned ord = (b & 0x80000000u) ? ~b : (b | 0x80000000u);
  return ((unsigned long long)bin << 48) | ((unsigned long long)(~ord) << 16) | (unsigned)j;
}
__device__ __forceinline__ float rank_key_score(unsigned long long k) {
  const unsigned ord = ~(unsigned)(k >> 16);
  return __uint_as_float((ord & 0x80000000u) ? (ord & 0x7FFFFFFFu) : ~ord);
}
constexpr int kSh = 24;  // level-1 bin = key >> 24

__device__ __forceinline__ int remap_block(int bid, int n) {
  // Dispatch places consecutive workgroups on the 8 XCDs round-robin; this mapping gives each XCD a
  // contiguous range of logical blocks, so the row blocks of one KV head share that XCD's L2.
  if ((n & 7) == 0) {
    const int per = n >> 3;
    return (bid & 7) * per + (bid >> 3);
  }
  return bid;
}

// ---- K / Q / V operand loaders ------------------------------------------------------------------

__device__ __forceinline__ u32x4 zero4() { return u32x4{0u, 0u, 0u, 0u}; }

__device__ __forceinline__ u32x4 bf16x8_to_f16x8_bits(u32x4 v) {
  f16x8 h;
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    h[2 * c] = (_Float16)__uint_as_float(v[c] << 16);
    h[2 * c + 1] = (_Float16)__uint_as_float(v[c] & 0xFFFF0000u);
  }
  return __builtin_bit_cast(u32x4, h);
}

typedef __amdgpu_buffer_rsrc_t rsrc_t;

// A byte offset past the end of every buffer this kernel reads (each is far below 1 GiB) that stays
// clear of 32-bit wrap-around when small constants are added to it.
constexpr unsigned kOOR = 0x7FFF0000u;

// Buffer resource over [base, base + bytes): loads take one 32-bit offset register, and loads past
// the end return zero (the hardware range check), which pads ragged key tails.
__device__ __forceinline__ rsrc_t make_rsrc(const void* base, size_t bytes) {
  const size_t cap = 0x7fffffff;
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)(bytes < cap ? bytes : cap),
                                           0x00020000);
}

// A-operand fragment of K for one 32-wide k-step: key ja, dims d0..d0+7 (d0 = ks*32 + 8g).
// Int4 blobs: both the 4-bit and the float32-window paths are loaded and one is selected, so there
// is no divergent branch; offsets outside a section fall outside the buffer and read zeros.
// Dequantized int4 K is fed to the f16 MFMA as hi + lo halves (hi = f16(x), lo = f16(x - hi)): 22
// significant bits, so the scores carry only the float32 accumulation error, like the bf16 path.
template <int KSRC>
__device__ __forceinline__ u32x4 load_k(const RowStatsParams& p, rsrc_t rk, const Int4Layout& L, int ja, int d0,
                                        u32x4* lo_out = nullptr) {
  if (KSRC == KSRC_BF16) {
    return __builtin_amdgcn_raw_buffer_load_b128(rk, (unsigned)(ja * KVPROF_HEAD_DIM + d0) * 2u, 0, 0);
  } else {
    const bool quant = ja < (int)L.n;
    const int jq = quant ? ja : 0;
    const uint32_t codes = __builtin_amdgcn_raw_buffer_load_b32(rk, (unsigned)(L.kc + (size_t)jq * 64 + d0 / 2), 0, 0);
    const unsigned mo = (unsigned)(L.km + ((size_t)(jq >> 5) * 128 + d0) * 4);
    const u32x4 m0 = __builtin_amdgcn_raw_buffer_load_b128(rk, mo, 0, 0);
    const u32x4 m1 = __builtin_amdgcn_raw_buffer_load_b128(rk, mo + 16u, 0, 0);
    // rows of the float32 window; keys before it (or past n_k) read past the buffer end -> zeros
    const unsigned ro = (quant || ja >= p.n_k) ? kOOR
                                               : (unsigned)(L.kr + ((size_t)(ja - (int)L.n) * 128 + d0) * 4);
    const f32x4 a = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(rk, ro, 0, 0));
    const f32x4 bb = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(rk, ro + 16u, 0, 0));
    f16x8 h, hl;
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      const uint32_t wd = c < 4 ? m0[c] : m1[c - 4];
      const float sc_ = (float)__builtin_bit_cast(_Float16, (uint16_t)(wd & 0xFFFF));
      const float mn_ = (float)__builtin_bit_cast(_Float16, (uint16_t)(wd >> 16));
      const float qv = fmaf((float)((codes >> (4 * c)) & 0xF), sc_, mn_);
      const float rv = c < 4 ? a[c] : bb[c - 4];
      const float x = quant ? qv : rv;
      h[c] = (_Float16)x;
      hl[c] = (_Float16)(x - (float)h[c]);
    }
    if (lo_out) *lo_out = __builtin_bit_cast(u32x4, hl);
    return __builtin_bit_cast(u32x4, h);
  }
}

// Int4 K of a key inside the 4-bit section, from its raw words (as load_k decodes them): the code
// word of dims d0 .. d0+7 and their (scale, min) pairs, read from the LDS load ring.
struct K4Raw {
  uint32_t codes;
  u32x4 m0, m1;
};
__device__ __forceinline__ u32x4 decode_k4(const K4Raw& k, u32x4& lo_out) {
  f16x8 h, hl;
#pragma unroll
  for (int c = 0; c < 8; ++c) {
    const uint32_t wd = c < 4 ? k.m0[c] : k.m1[c - 4];
    const float sc_ = (float)__builtin_bit_cast(_Float16, (uint16_t)(wd & 0xFFFF));
    const float mn_ = (float)__builtin_bit_cast(_Float16, (uint16_t)(wd >> 16));
    const float x = fmaf((float)((k.codes >> (4 * c)) & 0xF), sc_, mn_);
    h[c] = (_Float16)x;
    hl[c] = (_Float16)(x - (float)h[c]);
  }
  lo_out = __builtin_bit_cast(u32x4, hl);
  return __builtin_bit_cast(u32x4, h);
}

// V values of key j, channels c0 .. c0+7 (c0 a multiple of 8), as f16 for the P.V product: one
// 16-byte load for bf16; for int4 one word of codes and one of (scale, min), with the float32 window
// selected branchlessly as in load_k. Keys past n_k read zeros.
template <int KSRC>
__device__ __forceinline__ void load_v8(const RowStatsParams& p, rsrc_t rv, const Int4Layout& L, int j, int c0,
                                        _Float16 (&x)[8]) {
  if (KSRC == KSRC_BF16) {
    const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(rv, (unsigned)(j * KVPROF_HEAD_DIM + c0) * 2u, 0, 0);
#pragma unroll
    for (int e = 0; e < 8; ++e) x[e] = (_Float16)__uint_as_float(((v[e >> 1] >> (16 * (e & 1))) & 0xFFFFu) << 16);
  } else {
    const bool quant = j < (int)L.n;
    const int jq = quant ? j : 0;
    const uint32_t codes = __builtin_amdgcn_raw_buffer_load_b32(rv, (unsigned)(L.vc + (size_t)jq * 64 + c0 / 2), 0, 0);
    const uint32_t wd = __builtin_amdgcn_raw_buffer_load_b32(rv, (unsigned)(L.vm + ((size_t)jq * 4 + c0 / 32) * 4), 0, 0);
    const unsigned ro = (quant || j >= p.n_k) ? kOOR : (unsigned)(L.vr + ((size_t)(j - (int)L.n) * 128 + c0) * 4);
    const f32x4 a = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(rv, ro, 0, 0));
    const f32x4 bb = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(rv, ro + 16u, 0, 0));
    const float s_ = (float)__builtin_bit_cast(_Float16, (uint16_t)(wd & 0xFFFF));
    const float m_ = (float)__builtin_bit_cast(_Float16, (uint16_t)(wd >> 16));
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float rv_ = e < 4 ? a[e] : bb[e - 4];
      x[e] = (_Float16)(quant ? fmaf((float)((codes >> (4 * e)) & 0xF), s_, m_) : rv_);
    }
  }
}

// Raw words of eight V values (channels c0 .. c0+7 of key j), for keys in the 4-bit section (INT4KV:
// the code word and the (scale, min) word) or any key (BF16: one 16-byte load), and their decode as
// load_v8 does it. Loaded a few tiles ahead of their use.
template <int KSRC>
struct VRaw;
template <>
struct VRaw<KSRC_BF16> { u32x4 v; };
template <>
struct VRaw<KSRC_INT4> { uint32_t codes, wd; };
template <int KSRC>
__device__ __forceinline__ VRaw<KSRC> load_v_raw(rsrc_t rv, const Int4Layout& L, int j, int c0) {
  VRaw<KSRC> x;
  if constexpr (KSRC == KSRC_BF16) {
    x.v = __builtin_amdgcn_raw_buffer_load_b128(rv, (unsigned)(j * KVPROF_HEAD_DIM + c0) * 2u, 0, 0);
  } else {
    x.codes = __builtin_amdgcn_raw_buffer_load_b32(rv, (unsigned)(L.vc + (size_t)j * 64 + c0 / 2), 0, 0);
    x.wd = __builtin_amdgcn_raw_buffer_load_b32(rv, (unsigned)(L.vm + ((size_t)j * 4 + c0 / 32) * 4), 0, 0);
  }
  return x;
}
template <int KSRC>
__device__ __forceinline__ void decode_v8(const VRaw<KSRC>& r, _Float16 (&x)[8]) {
  if constexpr (KSRC == KSRC_BF16) {
#pragma unroll
    for (int e = 0; e < 8; ++e) x[e] = (_Float16)__uint_as_float(((r.v[e >> 1] >> (16 * (e & 1))) & 0xFFFFu) << 16);
  } else {
    const float s_ = (float)__builtin_bit_cast(_Float16, (uint16_t)(r.wd & 0xFFFF));
    const float m_ = (float)__builtin_bit_cast(_Float16, (uint16_t)(r.wd >> 16));
#pragma unroll
    for (int e = 0; e < 8; ++e) x[e] = (_Float16)fmaf((float)((r.codes >> (4 * e)) & 0xF), s_, m_);
  }
}

template <int KSRC>
__device__ __forceinline__ f32x4 mfma_step(u32x4 a, u32x4 b, f32x4 acc) {
  if (KSRC == KSRC_BF16)
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), acc, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), acc, 0, 0, 0);
}

__device__ __forceinline__ void init_target(TState& ts, int t, int n) {
  ts.prefix = 0;
  ts.dfix = 0;
  ts.ph = 0;
  ts.sh = kSh;
  ts.valid = n > 0;
  ts.cnt_before = 0;
  ts.cnt_in = 0;
  ts.resolved = n > 0 ? 0 : 1;
  ts.interp = 0;
  ts.mass_before = 0;
  if (t == 0) {
    ts.target = min(31, n - 1);
    ts.frac = 0.f;
  } else {
    const int pct = t == 1 ? 1 : (t == 2 ? 5 : 10);
    ts.target = (n * pct) / 100;
    ts.frac = (float)((n * pct) % 100) / 100.f;
  }
}

// Top-f mass of an interpolated target (see scan_row): the mass before its bin plus the share of the
// bin's mass taken by its first rr keys and frac of the next, with the bin's keys evenly spaced in score.
__device__ __forceinline__ float interp_mass(const TState& ts, float k8, float z) {
  const float wbin = k8 > 0.f ? 1.f / k8 : 0.f;  // bin width (log2 units)
  const float cf = (float)ts.cnt_in;
  const float rr = (float)(ts.target - ts.cnt_before);
  float share;
  if (wbin < 1e-3f) {  // (1 - x^k) would lose its relative precision; the bin is flat to 1e-3
    share = (rr + ts.frac) / cf;
  } else {
    const float a = wbin / cf;  // x = 2^-a
    const float xr = __builtin_amdgcn_exp2f(-rr * a);
    const float top = (1.f - xr) + ts.frac * xr * (1.f - __builtin_amdgcn_exp2f(-a));
    share = top / (1.f - __builtin_amdgcn_exp2f(-wbin));
  }
  return ((float)ts.mass_before + share * (float)ts.mass_in) / z;
}

// Inclusive prefix sums over the 64 lanes of a wave (all lanes active): Hillis-Steele steps inside
// each row of 16 lanes on DPP row shifts (lanes without a source add 0), then the totals of the lower
// rows, read from lanes 15, 31 and 47.
__device__ __forceinline__ unsigned dpp_shr(unsigned x, int sh) {
  switch (sh) {
    case 1: return (unsigned)__builtin_amdgcn_update_dpp(0, (int)x, 0x111, 0xf, 0xf, true);
    case 2: return (unsigned)__builtin_amdgcn_update_dpp(0, (int)x, 0x112, 0xf, 0xf, true);
    case 4: return (unsigned)__builtin_amdgcn_update_dpp(0, (int)x, 0x114, 0xf, 0xf, true);
    default: return (unsigned)__builtin_amdgcn_update_dpp(0, (int)x, 0x118, 0xf, 0xf, true);
  }
}
__device__ __forceinline__ unsigned wave_scan_u32(unsigned x, int lane) {
#pragma unroll
  for (int sh = 1; sh < 16; sh <<= 1) x += dpp_shr(x, sh);
  const unsigned t0 = (unsigned)__builtin_amdgcn_readlane((int)x, 15);
  const unsigned t1 = (unsigned)__builtin_amdgcn_readlane((int)x, 31);
  const unsigned t2 = (unsigned)__builtin_amdgcn_readlane((int)x, 47);
  return x + (lane >= 16 ? t0 : 0u) + (lane >= 32 ? t1 : 0u) + (lane >= 48 ? t2 : 0u);
}
__device__ __forceinline__ unsigned long long wave_scan_u64(unsigned long long x, int lane) {
#pragma unroll
  for (int sh = 1; sh < 16; sh <<= 1) {
    const unsigned lo = dpp_shr((unsigned)x, sh), hi = dpp_shr((unsigned)(x >> 32), sh);
    x += ((unsigned long long)hi << 32) | lo;
  }
  auto at = [&](int l) {
    return ((unsigned long long)(unsigned)__builtin_amdgcn_readlane((int)(x >> 32), l) << 32) |
           (unsigned)__builtin_amdgcn_readlane((int)(unsigned)x, l);
  };
  const unsigned long long t0 = at(15), t1 = at(31), t2 = at(47);
  return x + (lane >= 16 ? t0 : 0ull) + (lane >= 32 ? t1 : 0ull) + (lane >= 48 ? t2 : 0ull);
}

// Per-row scan of the level-1 histogram by one wave (lane holds bins 4*lane..4*lane+3): locates, for
// every target of the row, the bin that holds its rank. A row whose histogram holds no more keys than
// its deepest target is marked for a redo over every visible key.
//
// A top-f mass (targets 1..3) is the mass before its bin plus the share of the bin's mass held by the
// bin's first rr keys and frac of the next (rr = rank - keys before the bin). Taking the bin's c keys as
// evenly spaced in score across the bin's width w (log2 units) gives that share in closed form,
// [1 - x^rr + frac x^rr (1 - x)] / (1 - x^c) with x = 2^(-w/c). Whatever the keys' placement inside the
// bin, the true share differs from it by less than about 0.35 w times the bin's mass; when that bound
// is within kInterpTol the target takes no part in the exact rank passes (decided at the start of
// phase D, computed by interp_mass where the outputs are written).
template <typename SM>
__device__ void scan_row(SM& sm, int row, int lane) {
  unsigned c[4];
  unsigned long long m[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const unsigned long long h = sm.u.sel.hist[row][4 * lane + q];
    c[q] = (unsigned)(h >> 44);
    m[q] = h & kMassMask;
  }
  const unsigned lc = c[0] + c[1] + c[2] + c[3];
  const unsigned long long lm = m[0] + m[1] + m[2] + m[3];
  const unsigned ic = wave_scan_u32(lc, lane);
  const unsigned long long im = wave_scan_u64(lm, lane);
  const unsigned total = (unsigned)__builtin_amdgcn_readlane((int)ic, 63);
  const unsigned run = ic - lc;
  const unsigned long long mrun = im - lm;
  int redo = 0;
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    TState& ts = sm.ts[row][t];
    if (!ts.valid) continue;
    const unsigned T = (unsigned)(ts.target - ts.cnt_before);
    redo |= T >= total;
    unsigned r0 = run;
    unsigned long long m0 = mrun;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      if (r0 <= T && T < r0 + c[q]) {
        ts.prefix = (unsigned)(4 * lane + q);
        ts.sh = kSh;
        ts.cnt_before += (int)r0;
        ts.mass_before += m0;
        ts.cnt_in = (int)c[q];
        ts.resolved = c[q] <= (unsigned)CAP;
      }
      r0 += c[q];
      m0 += m[q];
    }
  }
  if (lane == 0) {
    sm.rfb[row] = redo;
    if (redo) atomicOr(&sm.flag, 1);
  }
}

template <int TPW>
constexpr int stash_tiles() { return TPW == 49 ? 5 : (TPW == 50 ? 6 : 0); }

// One workgroup = one row block (16 rows of one (batch, KV head)). SLOW = false: the main kernel, one
// block per workgroup; a block whose exact ranks need the slow path is appended to the redo list
// (p.redo) and finished by the SLOW = true kernel, which loops over that list and compiles the slow
// path (its code would otherwise raise the register peak of the common case).
template <int TPW, int KSRC, bool MX, bool SLOW, bool WO>
__global__ __launch_bounds__(WGT) void row_kernel(const RowStatsParams p) {
  constexpr int NL = stash_tiles<TPW>();
  __shared__ Smem<NL> sm;
  const int nblk = SLOW ? (int)p.redo[0] : 1;
  for (int it = SLOW ? (int)blockIdx.x : 0; it < nblk; it += SLOW ? (int)gridDim.x : 1) {
  const int bid = SLOW ? (int)p.redo[1 + it]
                       : remap_block((int)blockIdx.x, p.n_batch * p.n_heads_kv * ((p.rows_per_kv + ROWS - 1) / ROWS));
  const int tid = threadIdx.x;
  const int w = tid >> 6;
  const int lane = tid & 63;
  const int r = lane & 15;  // query row inside the workgroup
  const int g = lane >> 4;  // key quad inside a 16-key tile

  const int nrb = (p.rows_per_kv + ROWS - 1) / ROWS;
  const int rb = bid % nrb;
  const int hkv = (bid / nrb) % p.n_heads_kv;
  const int b = bid / (nrb * p.n_heads_kv);

  const RowInfo me0 = row_info(p, b, hkv, rb, r);
  const int nvis = me0.nvis;
  // workgroup-uniform extent of visible keys
  int kmax = nvis;
  kmax = row16_max(kmax);
  kmax = __builtin_amdgcn_readfirstlane(kmax);  // identical on every lane: keep it scalar
  // keys below kmin are visible to every row of the workgroup (rows past the end do not count)
  int kmin = me0.ok ? nvis : 0x7fffffff;
  kmin = row16_min(kmin);
  kmin = __builtin_amdgcn_readfirstlane(kmin);

  const size_t kvh = (size_t)b * p.n_heads_kv + hkv;
  const size_t head_bytes = (size_t)p.n_k * KVPROF_HEAD_DIM * 2;
  rsrc_t rk, rv;
  if (KSRC == KSRC_BF16) {
    rk = make_rsrc(p.k + kvh * p.n_k * KVPROF_HEAD_DIM, head_bytes);
    rv = make_rsrc(p.v ? p.v + kvh * p.n_k * KVPROF_HEAD_DIM : p.k, p.v ? head_bytes : 0);
  } else {
    rk = make_rsrc(p.kv_packed + kvh * p.blob_bytes, p.blob_bytes);
    rv = rk;
  }
  Int4Layout L{};
  if (KSRC == KSRC_INT4) L = int4_layout(p.n_k, KVPROF_HEAD_DIM, p.r_window);

  // clear the shared accumulators; the segments' region and frame maps into LDS
  for (int i = tid; i < NW * ROWS * kSegPerWave; i += WGT) (&sm.segpart[0][0][0])[i] = 0.f;
  if (tid < p.n_seg) {
    sm.sreg[tid] = p.seg_region[tid];
    sm.sfr[tid] = p.seg_frame[tid];
  }

  // Q rows of the workgroup into LDS (wave 0): chunk c of row r holds dims 8c .. 8c+7
  if (w == 0) {
#pragma unroll
    for (int c = g; c < 16; c += 4) {
      u32x4 v = zero4();
      if (me0.ok) {
        v = *reinterpret_cast<const u32x4*>(p.q + (size_t)me0.grow * KVPROF_HEAD_DIM + 8 * c);
        if (KSRC == KSRC_INT4) v = bf16x8_to_f16x8_bits(v);
      }
      sm.qs[r][c] = v;
    }
  }
  __syncthreads();

  // ---- A: scores ---------------------------------------------------------------------------------
  const int kbase = __builtin_amdgcn_readfirstlane(w * TPW * 16);  // wave-uniform: keep it scalar
  float sc[TPW - NL][4];  // tiles NL .. TPW-1 (tiles below NL live in sm.stash)
  // score u of key 4g + i of tile t of this lane
  auto scr = [&](int t, int i) -> float { return t < NL ? sm.stash[t][w][lane][i] : sc[t < NL ? 0 : t - NL][i]; };
  float umax = -INFINITY, umin = INFINITY, usum = 0.f;
  // key bias: a buffer resource of 0 bytes when there is none (its loads return zero)
  const rsrc_t rbs = make_rsrc(p.key_bias ? (const void*)p.key_bias : (const void*)p.q,
                               p.key_bias ? (size_t)p.n_k * 4 : 0);
  // Direct global->LDS loads (no VGPRs) of tile t into ring slot t % kRing. Load ks brings keys
  // 4ks .. 4ks+3 of the tile whole (lane l: key 4ks + l/16, 16-byte chunk l%16 of its LDS row), so
  // every load reads complete cache lines; the chunk stored at position q of key k's row is chunk
  // q ^ k, which makes the A-fragment reads below free of bank conflicts. Lanes 0..15 also load the
  // tile's 16 bias values. The compiler does not track these writes, so the wait before reading a
  // slot is explicit: loads retire in issue order, and the 5 (kRing - 1) loads of the later tiles
  // may still be outstanding.
  auto issue_from = [&](rsrc_t src, int t) {
    const int slot = t % kRing;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const int kt = 4 * ks + (lane >> 4);  // key inside the tile
      __builtin_amdgcn_raw_ptr_buffer_load_lds(src, (__attribute__((address_space(3))) void*)&sm.u.a.ring[w][slot][ks][0], 16,
                                               (unsigned)((kbase + t * 16 + kt) * (KVPROF_HEAD_DIM * 2) + (((lane & 15) ^ kt) * 16)),
                                               0, 0, 0);
    }
    if (lane < 16)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rbs, (__attribute__((address_space(3))) void*)&sm.u.a.rbias[w][slot][0], 4,
                                               (unsigned)(kbase + t * 16 + lane) * 4u, 0, 0, 0);
  };
  auto issue = [&](int t) { issue_from(rk, t); };
  if (KSRC == KSRC_BF16) {
#pragma unroll
    for (int t = 0; t < kRing - 1 && t < TPW; ++t) issue(t);
  }
  // Int4 keys of the 4-bit section reach LDS the same way, kRing4 tiles deep, in the same per-wave
  // bytes: a slot holds the tile's 16 code rows (64 B each, key-major), the (scale, min) words of its
  // 32-token group (128 channels x 4 B) and its 16 bias values. Three loads per tile: the codes (all
  // lanes, 16 B each), the group words (lanes 0..31) and the bias (lanes 0..15). A tile goes through
  // the ring when it is visible and inside the 4-bit section (tiles never straddle the window: the
  // section holds whole 32-token groups); float32 window tiles load directly.
  constexpr int kRing4 = 5;
  constexpr int kSlot4 = 16 * 64 + 128 * 4 + 16 * 4;  // 1,600 B
  static_assert(kRing4 * kSlot4 <= (int)sizeof(sm.u.a.ring[0]), "int4 ring slots fit the wave's ring bytes");
  auto ring4 = [&](int slot) { return reinterpret_cast<char*>(&sm.u.a.ring[w][0][0][0]) + slot * kSlot4; };
  auto q4 = [&](int t) {  // wave-uniform, and false from the first tile it is false for
    const int jt = kbase + t * 16;
    return KSRC == KSRC_INT4 && jt < kmax && jt + 16 <= (int)L.n;
  };
  auto issue4 = [&](int t) {
    const int jt = kbase + t * 16;
    char* dst = ring4(t % kRing4);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rk, (__attribute__((address_space(3))) void*)dst, 16,
                                             (unsigned)(L.kc + (size_t)jt * 64 + lane * 16), 0, 0, 0);
    if (lane < 32)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rk, (__attribute__((address_space(3))) void*)(dst + 1024), 16,
                                               (unsigned)(L.km + ((size_t)(jt >> 5) * 128 + 4 * lane) * 4), 0, 0, 0);
    if (lane < 16)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rbs, (__attribute__((address_space(3))) void*)(dst + 1536), 4,
                                               (unsigned)(jt + lane) * 4u, 0, 0, 0);
  };
  if (KSRC == KSRC_INT4) {
#pragma unroll
    for (int t = 0; t < kRing4 - 1 && t < TPW; ++t)
      if (q4(t)) issue4(t);
  }
  // bf16 keys: this lane's Q fragments stay in registers for the score pass (read from LDS once
  // instead of once per tile: a third of the pass's LDS traffic). The int4 path, whose prefetched raw
  // words need those registers, keeps reading them from LDS.
  u32x4 qfr[4];
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) qfr[ks] = KSRC == KSRC_BF16 ? sm.qs[r][ks * 4 + g] : zero4();
  // The scheduling barrier at the end of each tile keeps the compiler from hoisting every tile's
  // loads, which would push the score registers out to scratch.
#pragma unroll
  for (int t = 0; t < TPW; ++t) {
    const int j0 = kbase + t * 16;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    f32x4 bias = {0.f, 0.f, 0.f, 0.f};
    if (KSRC == KSRC_BF16) {
      if (t + kRing - 1 < TPW) issue(t + kRing - 1);
      // s_waitcnt vmcnt(5 * later tiles in flight), expcnt / lgkmcnt left alone (gfx9 encoding)
      if (t + kRing - 1 < TPW)
        __builtin_amdgcn_s_waitcnt(0x0F70 | (5 * (kRing - 1)));
      else
        __builtin_amdgcn_s_waitcnt(0x0F70);
      if (j0 < kmax) {
#pragma unroll
        for (int ks = 0; ks < 4; ++ks)  // chunk 4ks + g of key r (see issue)
          acc = mfma_step<KSRC>(sm.u.a.ring[w][t % kRing][r >> 2][(r & 3) * 16 + ((4 * ks + g) ^ r)], qfr[ks], acc);
      }
      bias = *reinterpret_cast<const f32x4*>(&sm.u.a.rbias[w][t % kRing][4 * g]);
    } else if (q4(t)) {
      // wave-uniform: the tile's codes, group words and bias are in ring slot t % kRing4; the three
      // loads of each later tile in the ring may still be outstanding
      if (t + kRing4 - 1 < TPW && q4(t + kRing4 - 1)) {
        issue4(t + kRing4 - 1);
        __builtin_amdgcn_s_waitcnt(0x0F70 | (3 * (kRing4 - 1)));
      } else {
        __builtin_amdgcn_s_waitcnt(0x0F70);
      }
      const char* src = ring4(t % kRing4);
      u32x4 kf[4], kl[4];
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        K4Raw kr;
        kr.codes = *reinterpret_cast<const uint32_t*>(src + r * 64 + ks * 16 + 4 * g);
        kr.m0 = *reinterpret_cast<const u32x4*>(src + 1024 + (ks * 32 + 8 * g) * 4);
        kr.m1 = *reinterpret_cast<const u32x4*>(src + 1024 + (ks * 32 + 8 * g) * 4 + 16);
        kf[ks] = decode_k4(kr, kl[ks]);
      }
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        acc = mfma_step<KSRC>(kf[ks], sm.qs[r][ks * 4 + g], acc);
        acc = mfma_step<KSRC>(kl[ks], sm.qs[r][ks * 4 + g], acc);
      }
      bias = *reinterpret_cast<const f32x4*>(src + 1536 + 16 * g);
    } else {
      // float32 window tiles (after every ring tile of this wave has been consumed) and tiles past the
      // visible keys
      if (j0 < kmax) {
        u32x4 kf[4], kl[4];
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) kf[ks] = load_k<KSRC>(p, rk, L, j0 + r, ks * 32 + 8 * g, &kl[ks]);
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
          acc = mfma_step<KSRC>(kf[ks], sm.qs[r][ks * 4 + g], acc);
          acc = mfma_step<KSRC>(kl[ks], sm.qs[r][ks * 4 + g], acc);
        }
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)  // one dword each: a key past the end reads zero on its own
        bias[i] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rbs, (unsigned)(j0 + 4 * g + i) * 4u, 0, 0));
    }
    // Invisible keys are -inf, so they never pass a selection threshold; visible keys are finite (a
    // -inf bias is clamped: zero probability). The scores are pinned here: otherwise the compiler
    // sinks this epilogue to the next use and keeps both the MFMA accumulators and the bias values
    // live for every tile.
    f32x4 ut;
    if (j0 + 16 <= kmin) {  // the whole tile is visible to every row (wave-uniform)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float u = fmaf(acc[i], p.scale_log2, fmaxf(bias[i] * kLog2e, kNegBig));
        ut[i] = u;
        umax = fmaxf(umax, u);
        umin = fminf(umin, u);
        usum += u;
      }
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int j = j0 + 4 * g + i;
        const bool valid = j < nvis;
        const float u = valid ? fmaf(acc[i], p.scale_log2, fmaxf(bias[i] * kLog2e, kNegBig)) : -INFINITY;
        ut[i] = u;
        umax = fmaxf(umax, u);
        umin = valid ? fminf(umin, u) : umin;
        usum += valid ? u : 0.f;
      }
    }
    if (t < NL) {
      sm.stash[t][w][lane] = ut;
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) sc[t < NL ? 0 : t - NL][i] = opaque(ut[i]);
    }
    umax = opaque(umax);
    umin = opaque(umin);
    usum = opaque(usum);
    __builtin_amdgcn_sched_barrier(0);
  }
  __builtin_amdgcn_s_waitcnt(0x0F70);  // every ring load has landed
  umax = row_max4(umax);
  umin = row_min4(umin);
  usum = row_sum4(usum);
  if (g == 0) {
    sm.red_a[w][r] = umax;
    sm.red_b[w][r] = umin;
    sm.red_c[w][r] = usum;
  }
  // first segment overlapping this wave's keys
  int cs = 0;
  while (cs < p.n_seg && p.seg_bounds[cs + 1] <= kbase) ++cs;
  const int cs_first = cs;
  if (lane == 0) sm.cs0[w] = cs_first;
  __syncthreads();
  float m = -INFINITY, mn = INFINITY, s1 = 0.f;
#pragma unroll
  for (int ww = 0; ww < NW; ++ww) {
    m = fmaxf(m, sm.red_a[ww][r]);
    mn = fminf(mn, sm.red_b[ww][r]);
    s1 += sm.red_c[ww][r];
  }
  // Selection threshold: only keys at or above T enter the level-1 histogram. The largest of n
  // bell-shaped scores lies about sqrt(2 ln n) standard deviations above the mean, so T = mean +
  // kSelSigma (max - mean) / sqrt(2 ln n) sits near kSelSigma deviations above the mean and keeps a
  // few times more keys than the deepest rank (10 %) needs; a row whose histogram ends up too small
  // is redone with T = min.
  float T = m;
  if (me0.ok) {
    const float mu = s1 / (float)nvis;
    const float c = kSelSigma * rsqrtf(fmaxf(2.f * logf((float)nvis), 1.f));
    T = fmaxf(fminf(m, fmaf(c, m - mu, mu)), mn);
  } else {
    m = 0.f;
    mn = 0.f;
    T = 0.f;
  }
  const float k8 = bin_scale(m, T);
  if (w == 0 && g == 0) {
    sm.r_m[r] = m;
    sm.r_mn[r] = mn;
    sm.r_T[r] = T;
    sm.r_k8[r] = k8;
  }
  // the histogram shares LDS with the phase-A load ring, which every wave has finished reading
  for (int i = tid; i < ROWS * HB; i += WGT) (&sm.u.sel.hist[0][0])[i] = 0ull;
  __syncthreads();

  // ---- B: exponentials, entropy sum, segment masses and the level-1 histogram ---------------------
  // Histogram counters pack a key count (bits 44..63) with a fixed-point mass f = round(e') (bits
  // 0..43): f <= 2^31 per key, so a row of <= 8192 keys cannot carry out of the mass field. One LDS
  // atomic per selected key updates both.
  {
  const float off = kOff - m;
  float esum = 0.f, acc_seg = 0.f;
  int nb = (cs < p.n_seg) ? p.seg_bounds[cs + 1] : 0x7fffffff;
  const int gB = opaque(g);
  const float Tq = opaque(T), k8q = opaque(k8), mk8q = opaque(__fmul_rn(m, k8));
  auto flush = [&](float a, int seg) {
    float v = row_sum4(a);
    if (g == 0 && seg - cs_first < kSegPerWave) sm.segpart[w][r][seg - cs_first] = v;
  };
#pragma unroll
  for (int t = 0; t < TPW; ++t) {
    const int j0 = kbase + t * 16;
    if (j0 < kmax) {
    float e[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float u = scr(t, i);
      const float tp = fmaxf(u + off, -256.f);
      e[i] = __builtin_amdgcn_exp2f(tp);
      esum = fmaf(e[i], tp, esum);
      if (u >= Tq)
        atomicAdd(&sm.u.sel.hist[r][bin1(u, k8q, mk8q)], kOne + (unsigned long long)fixmass(e[i]));
    }
    if (j0 + 16 <= nb) {
      acc_seg += (e[0] + e[1]) + (e[2] + e[3]);
    } else {
      int lo = j0;
      while (lo < j0 + 16) {
        const int hi = min(nb, j0 + 16);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int j = j0 + 4 * gB + i;
          if (j >= lo && j < hi) acc_seg += e[i];
        }
        lo = hi;
        if (hi == nb) {
          flush(acc_seg, cs);
          acc_seg = 0.f;
          ++cs;
          nb = (cs < p.n_seg) ? p.seg_bounds[cs + 1] : 0x7fffffff;
        }
      }
    }
    }
    // running sums pinned per tile (else their add chains are sunk past the loop)
    esum = opaque(esum);
    acc_seg = opaque(acc_seg);
    __builtin_amdgcn_sched_barrier(0);
  }
  if (kbase < kmax && cs < p.n_seg) flush(acc_seg, cs);
  esum = row_sum4(esum);
  if (g == 0) sm.red_e[w][r] = esum;
  }
  __syncthreads();

  // ---- per-row finalisation of B (wave w handles rows w and w + 8) --------------------------------------------
  for (int row = w; row < ROWS; row += NW) {
    const RowInfo ri = row_info(p, b, hkv, rb, row);
    const int span = TPW * 16;
    float zpart = 0.f;
    for (int s = lane; s < p.n_seg; s += 64) {
      float v = 0.f;
      const int s0 = p.seg_bounds[s], s1_ = p.seg_bounds[s + 1];
#pragma unroll
      for (int ww = 0; ww < NW; ++ww) {
        const int w0 = ww * span, w1 = w0 + span;
        const int slot = s - sm.cs0[ww];
        const bool hit = w0 < s1_ && w1 > s0 && slot >= 0 && slot < kSegPerWave;
        const float x = sm.segpart[ww][row][hit ? slot : 0];
        v += hit ? x : 0.f;
      }
      sm.segmass[row][s] = v;
      zpart += v;
    }
    // fixed-order wave reductions: Z' over the segments, the entropy sum over the waves
    float z = wave_sum(zpart);
    const float e_ = wave_sum(lane < NW ? sm.red_e[lane < NW ? lane : 0][row] : 0.f);
    if (lane == 0) {
      if (!ri.ok || !(z > 0.f)) z = 1.f;
      sm.r_z[row] = z;
      sm.r_e[row] = e_;
    }
  }
  __syncthreads();
  // Row constants are read back from LDS where they are used (they would otherwise stay live in
  // registers next to the scores for the rest of the kernel).
  auto rc_m = [&]() { return sm.r_m[r]; };
  auto rc_z = [&]() { return sm.r_z[r]; };
  auto rc_T = [&]() { return sm.r_T[r]; };
  auto rc_k8 = [&]() { return sm.r_k8[r]; };
  // p <= 2^-150 (an fp32 zero) <=> u - max + kOff - log2 Z' <= -150
  auto rc_thr = [&]() { return sm.r_m[r] + log2f(sm.r_z[r]) - (kOff + 150.f); };

  // region / frame / scalar outputs and target setup (wave w handles rows w and w + 8)
  for (int row = w; row < ROWS; row += NW) {
    const RowInfo ri = row_info(p, b, hkv, rb, row);
    if (ri.ok) {
      const float z = sm.r_z[row];
      const float iz = 1.f / z;
      // lane q < n_regions sums region q, lane q < n_frames frame q (segments in key order)
      float ar = 0.f, af = 0.f;
#pragma unroll 8
      for (int s = 0; s < p.n_seg; ++s) {
        const float x = sm.segmass[row][s];
        ar += sm.sreg[s] == lane ? x : 0.f;
        af += sm.sfr[s] == lane ? x : 0.f;
      }
      if (p.region_mass && lane < p.n_regions) p.region_mass[ri.grow * p.n_regions + lane] = ar * iz;
      if (p.frame_mass && lane < p.n_frames) p.frame_mass[ri.grow * p.n_frames + lane] = af * iz;
    }
    if (lane < NT) init_target(sm.ts[row][lane], lane, ri.ok ? ri.nvis : 0);
  }
  if (tid == 0) sm.flag = 0;
  __syncthreads();
  for (int row = w; row < ROWS; row += NW) scan_row(sm, row, lane);
  __syncthreads();

  // Rows whose histogram holds no more keys than their deepest rank: redo it over every visible key.
  if (sm.flag) {
    for (int row = w; row < ROWS; row += NW) {
      if (sm.rfb[row]) {
        for (int i = lane; i < HB; i += 64) sm.u.sel.hist[row][i] = 0ull;
        if (lane == 0) {
          sm.r_T[row] = sm.r_mn[row];
          sm.r_k8[row] = bin_scale(sm.r_m[row], sm.r_mn[row]);
        }
        if (lane < NT) init_target(sm.ts[row][lane], lane, row_info(p, b, hkv, rb, row).nvis);
      }
    }
    __syncthreads();
    if (sm.rfb[r]) {
      const float mq = rc_m(), Tq = rc_T(), k8q = rc_k8(), offq = kOff - mq, mk8q = __fmul_rn(mq, k8q);
#pragma unroll
      for (int t = 0; t < TPW; ++t) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float u = scr(t, i);
          if (u >= Tq) {
            const float e = __builtin_amdgcn_exp2f(fmaxf(u + offq, -256.f));
            atomicAdd(&sm.u.sel.hist[r][bin1(u, k8q, mk8q)], kOne + (unsigned long long)fixmass(e));
          }
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    __syncthreads();
    for (int row = w; row < ROWS; row += NW)
      if (sm.rfb[row]) scan_row(sm, row, lane);
    __syncthreads();
  }

  // ---- D: exact ranks ------------------------------------------------------------------------------
  // Fast path (the common case): every target's boundary bin holds at most CAP keys and the distinct
  // boundary bins of a row hold at most CAP keys together. One pass then gathers, for every row, the
  // keys of its boundary bins (candidates) and the keys ranked above the top-32 boundary (winners);
  // candidates are ranked inside their bin by (score descending, index ascending). Masses are summed
  // as fixed-point integers, whose sum does not depend on the order. Otherwise the slow path narrows
  // each target with further radix levels.
  if (tid == 0) sm.flag = 0;
  __syncthreads();
  // top-f targets (lanes 1..3 of the row's wave) whose bin is narrow enough take the interpolated mass
  // (see interp_mass) and leave the exact rank passes; the test needs no division
  for (int row = w; row < ROWS; row += NW) {
    if (lane >= 1 && lane < NT) {
      TState& ts = sm.ts[row][lane];
      if (ts.valid && ts.ph == 0 && ts.prefix < 256u) {
        const unsigned long long mb = sm.u.sel.hist[row][ts.prefix] & kMassMask;
        const float k8 = sm.r_k8[row];
        const float wbin = k8 > 0.f ? __builtin_amdgcn_rcpf(k8) : 0.f;
        if ((float)mb * (0.35f * wbin) <= kInterpTol * sm.r_z[row]) {
          ts.mass_in = mb;
          ts.interp = 1;
          ts.resolved = 1;
        }
      }
    }
  }
  for (int row = w; row < ROWS; row += NW) {
    // all four states read at once (one LDS round trip), then a wave-uniform test
    unsigned pv[NT];
    int cin[NT], val[NT], res[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      pv[t] = sm.ts[row][t].prefix;
      cin[t] = sm.ts[row][t].cnt_in;
      val[t] = sm.ts[row][t].valid && !sm.ts[row][t].interp;  // interpolated targets need no ranks
      res[t] = sm.ts[row][t].resolved;
    }
    int tot = 0, bad = 0;
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      if (!val[t]) continue;  // row past the end
      bad |= !res[t];
      bool seen = false;
#pragma unroll
      for (int q = 0; q < t; ++q) seen |= val[q] && pv[q] == pv[t];
      tot += seen ? 0 : cin[t];
    }
    if (lane == 0 && (bad || tot > CAP)) atomicOr(&sm.flag, 1);
  }
  if (tid < ROWS) {
    sm.ncand[tid] = 0;
    sm.nwin[tid] = 0;
  }
  __syncthreads();
  const bool slow_path = sm.flag != 0;
  // Only the top-32 list, the top-f masses and the MX argmax depend on the ranks. Without them a
  // slow-path block needs no redo: it skips the gather, and phase E writes none of those outputs.
  const bool need_ranks = p.top32 != nullptr || p.top_mass != nullptr || (MX && p.argmax != nullptr);
  if (!SLOW && slow_path && need_ranks && tid == 0) {  // left to the redo kernel, which rewrites every output
    const unsigned k = atomicAdd(p.redo, 1u);
    p.redo[1 + k] = (unsigned)bid;
  }
  if (!slow_path && need_ranks) {  // (without rank outputs the gather is skipped: phase E reads its
                                    // results only for the top-32 list, the top-f masses and the argmax)
    {
      // boundary bins of this lane's row (level-1 bins; keys below the threshold get bin 256). The
      // list holds every key of a bin <= bq0 (the top-32 boundary bin and the bins above it: at most
      // 31 + CAP keys) and of the other boundary bins.
      int bq[NT];
#pragma unroll
      for (int t = 0; t < NT; ++t) bq[t] = (sm.ts[r][t].valid && !sm.ts[r][t].interp) ? (int)sm.ts[r][t].prefix : -1;
      // When no row of the wave has an exact top-f target left, a key belongs to the list iff its
      // level-1 bin is at most bq0: u >= T and fma(-u, k8, m k8) < bq0 + 1 (the bin before clamping
      // and truncation), one compare pair instead of the bin and four tests.
      const bool only32 = __ballot((bq[1] >= 0) | (bq[2] >= 0) | (bq[3] >= 0)) == 0ull;
      // Two passes without returning atomics in the loop: mark and count this lane's list keys (one
      // bit per key, 8 tiles per word, kept in LDS), reserve slots with one atomic, then write.
      static_assert((TPW + 7) / 8 <= 7, "gather bit words");
      int nc = 0;
      {
        const float Tq = rc_T(), k8q = rc_k8(), mk8q = __fmul_rn(rc_m(), k8q);
        unsigned bits = 0u;
        if (only32) {
          const float lim = bq[0] < 0 ? -INFINITY : (bq[0] >= 255 ? INFINITY : (float)(bq[0] + 1));
          // x = fma(-u, k8, m k8) does not increase with u, so where x(T) >= lim already, a key with
          // x < lim lies above T and the threshold test is implied: one compare per key remains
          // (the same keys as the two-test form, exactly).
          const bool implied = !(__fmaf_rn(-Tq, k8q, mk8q) < lim);
          if (__ballot(!implied) == 0ull) {
            // (fresh copies of the row constants: otherwise the compiler shares values between the
            // two forms of the loop and the score registers spill)
            const float k8f = opaque(k8q), mk8f = opaque(mk8q), limf = opaque(lim);
#pragma unroll
            for (int tt = 0; tt < TPW; ++tt) {
#pragma unroll
              for (int i = 0; i < 4; ++i) {
                const bool in = __fmaf_rn(-scr(tt, i), k8f, mk8f) < limf;
                bits |= in ? 1u << (4 * (tt & 7) + i) : 0u;
              }
              if ((tt & 7) == 7 || tt == TPW - 1) {
                sm.u.sel.gbits[tt >> 3][w][lane] = bits;
                nc += __builtin_popcount(bits);
                bits = 0u;
              }
              bits = opaque(bits);
              __builtin_amdgcn_sched_barrier(0);
            }
          } else {
#pragma unroll
          for (int tt = 0; tt < TPW; ++tt) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const float u = scr(tt, i);
              const bool in = (u >= Tq) & (__fmaf_rn(-u, k8q, mk8q) < lim);
              bits |= in ? 1u << (4 * (tt & 7) + i) : 0u;
            }
            if ((tt & 7) == 7 || tt == TPW - 1) {
              sm.u.sel.gbits[tt >> 3][w][lane] = bits;
              nc += __builtin_popcount(bits);
              bits = 0u;
            }
            bits = opaque(bits);
            __builtin_amdgcn_sched_barrier(0);
          }
          }
        } else {
#pragma unroll
        for (int tt = 0; tt < TPW; ++tt) {
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const float u = scr(tt, i);
            const int dig = u >= Tq ? bin1(u, k8q, mk8q) : 256;
            const bool in = (dig <= bq[0]) | (dig == bq[1]) | (dig == bq[2]) | (dig == bq[3]);
            bits |= in ? 1u << (4 * (tt & 7) + i) : 0u;
          }
          if ((tt & 7) == 7 || tt == TPW - 1) {
            sm.u.sel.gbits[tt >> 3][w][lane] = bits;
            nc += __builtin_popcount(bits);
            bits = 0u;
          }
          bits = opaque(bits);
          __builtin_amdgcn_sched_barrier(0);
        }
        }
      }
      int cpos = nc ? atomicAdd(&sm.ncand[r], nc) : 0;
      if (nc) {
        // the list takes (score bits, key index) pairs here; they become rank keys below, once per
        // listed key instead of in this pass over every key
        const int gq = opaque(g);
        unsigned bits = 0u;
#pragma unroll
        for (int tt = 0; tt < TPW; ++tt) {
          if ((tt & 7) == 0) bits = sm.u.sel.gbits[tt >> 3][w][lane];
          const unsigned jt = (unsigned)(kbase + tt * 16 + 4 * opaque(gq));
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            if ((bits >> (4 * (tt & 7) + i)) & 1u) {  // (the fast path holds <= 31 + CAP < CAPL keys)
              // (the score goes through a copy: stored straight from its register it would tie that
              // register to the index in an aligned pair, and the score registers then spill)
              sm.u.sel.ck[r][cpos] = ((unsigned long long)(jt + i) << 32) | opaque(__float_as_uint(scr(tt, i)));
              ++cpos;
            }
          }
          cpos = opaque(cpos);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
    }
    __syncthreads();
    // (score, index) pairs -> rank keys, by the wave that owns the row
    for (int row = w; row < ROWS; row += NW) {
      const int c = min(sm.ncand[row], CAPL);
      const float k8q = sm.r_k8[row], mk8q = __fmul_rn(sm.r_m[row], k8q);
      for (int a = lane; a < c; a += 64) {
        const unsigned long long e = sm.u.sel.ck[row][a];
        const float u = __uint_as_float((unsigned)e);
        sm.u.sel.ck[row][a] = rank_key(u, (int)(e >> 32), bin1(u, k8q, mk8q));
      }
    }
    __syncthreads();
    // rank every boundary-bin key inside its bin (the other keys of the bins above bq0 need none):
    // lane a takes entry a and counts the smaller rank keys of the list, and those of earlier bins.
    // The wave that owns the row pads the list to a multiple of 4 with the largest key first.
    for (int row = w; row < ROWS; row += NW) {
      const int c = __builtin_amdgcn_readfirstlane(min(sm.ncand[row], CAPL));
      const int c4 = (c + 3) & ~3;
      if (c + lane < c4) sm.u.sel.ck[row][c + lane] = ~0ull;
      const int b0 = sm.ts[row][0].valid ? (int)sm.ts[row][0].prefix : -1;
      const int b1 = sm.ts[row][1].interp ? -1 : (int)sm.ts[row][1].prefix;
      const int b2 = sm.ts[row][2].interp ? -1 : (int)sm.ts[row][2].prefix;
      const int b3 = sm.ts[row][3].interp ? -1 : (int)sm.ts[row][3].prefix;
      for (int a0 = 0; a0 < c; a0 += 64) {
        const int a = a0 + lane;
        const unsigned long long ka = a < c ? sm.u.sel.ck[row][a] : 0ull;
        const unsigned long long k0 = ka & ~((1ull << 48) - 1);  // first key of a's bin
        int below = 0, earlier = 0;
#pragma unroll 4
        for (int q = 0; q < c4; q += 2) {
          const u64x2 k2 = *reinterpret_cast<const u64x2*>(&sm.u.sel.ck[row][q]);
          below += (int)(k2[0] < ka) + (int)(k2[1] < ka);
          earlier += (int)(k2[0] < k0) + (int)(k2[1] < k0);
        }
        const int ba = (int)(ka >> 48);
        const bool need = ba >= b0 || ba == b1 || ba == b2 || ba == b3;
        if (a < c) sm.u.sel.crank[row][a] = need ? below - earlier : 0;
      }
    }
    __syncthreads();
    for (int row = w; row < ROWS; row += NW) {
      const float mr = sm.r_m[row];
      const RowInfo ri = row_info(p, b, hkv, rb, row);
      const int c = min(sm.ncand[row], CAPL);
      // the row's targets (the same on every lane of the wave): those ranked exactly, their bins,
      // ranks inside the bin, keys before the bin and fractions
      bool ex[NT];
      unsigned pre[NT];
      int rrk[NT], cb[NT];
      float fr[NT];
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        const TState& ts = sm.ts[row][t];
        ex[t] = ts.valid && !ts.interp;
        pre[t] = ts.prefix;
        rrk[t] = ts.target - ts.cnt_before;
        cb[t] = ts.cnt_before;
        fr[t] = ts.frac;
      }
      const int b0 = ex[0] ? (int)pre[0] : -1;
      const bool anyf = ex[1] | ex[2] | ex[3];
      unsigned long long acc[NT] = {0ull, 0ull, 0ull, 0ull};
      for (int a = lane; a < c; a += 64) {
        const unsigned long long ka = sm.u.sel.ck[row][a];
        const float ua = rank_key_score(ka);
        const int ja = (int)(ka & 0xFFFFu);
        const unsigned dga = (unsigned)(ka >> 48);
        const int rk = sm.u.sel.crank[row][a];
        if ((int)dga < b0) {  // ranked above the top-32 boundary bin: one of the 32
          const int slot = atomicAdd(&sm.nwin[row], 1);
          sm.win_u[row][slot] = ua;
          sm.win_j[row][slot] = ja;
        }
        if (ex[0] && pre[0] == dga && rk <= rrk[0]) {  // ranks 0..target of the top-32 list
          sm.win_u[row][cb[0] + rk] = ua;
          sm.win_j[row][cb[0] + rk] = ja;
        }
        if (anyf) {
          const float ea = __builtin_amdgcn_exp2f(fmaxf(ua + (kOff - mr), -256.f));
#pragma unroll
          for (int t = 1; t < NT; ++t) {
            if (!ex[t] || pre[t] != dga) continue;
            if (rk < rrk[t]) acc[t] += fixmass(ea);
            if (rk == rrk[t]) acc[t] += fixmass(fr[t] * ea);
          }
        }
      }
#pragma unroll
      for (int t = 1; t < NT; ++t) {
        if (!ex[t]) continue;  // interpolated (phase E) or a row past the end
        unsigned long long x = acc[t];
        for (int o = 32; o >= 1; o >>= 1) x += __shfl_xor(x, o);
        if (lane == 0 && ri.ok) sm.tmass[row][t - 1] = (float)(sm.ts[row][t].mass_before + x) / sm.r_z[row];
      }
    }
    __syncthreads();
  } else if (SLOW && need_ranks) {  // here slow_path holds
  // ---- D: refine and gather, one target at a time --------------------------------------------------
#pragma unroll 1
  for (int t = 0; t < NT; ++t) {
#pragma unroll 1
    for (int level = 1; level <= 8; ++level) {
      if (tid == 0) sm.flag = 0;
      __syncthreads();
      for (int row = w; row < ROWS; row += NW)
        if (lane == 0 && !sm.ts[row][t].resolved && sm.ts[row][t].valid) atomicOr(&sm.flag, 1);
      __syncthreads();
      if (!sm.flag) break;
      for (int i = tid; i < ROWS * HB; i += WGT) (&sm.u.sel.hist[0][0])[i] = 0ull;
      __syncthreads();
      // histogram of the next 8-bit digit over the group of every unresolved target
      if (!sm.ts[r][t].resolved && sm.ts[r][t].valid) {
        const int ph = opaque(sm.ts[r][t].ph), sh = opaque(sm.ts[r][t].sh);
        const unsigned pre = opaque(sm.ts[r][t].prefix), dfix = opaque(sm.ts[r][t].dfix);
        const int gq = opaque(g);
        const float mq = rc_m(), Tq = rc_T(), k32 = rc_k8() * 0x1p24f, offq = kOff - mq;
        const float mk32 = __fmul_rn(mq, rc_k8()) * 0x1p24f;
#pragma unroll
        for (int tt = 0; tt < TPW; ++tt) {
          const int j0 = kbase + tt * 16;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int j = j0 + 4 * gq + i;
            const float u = scr(tt, i);
            if (u >= Tq) {
              const unsigned D = dkey32(u, k32, mk32);
              if (ts_in(D, j, ph, sh, pre, dfix)) {
                const int dig = (int)(((ph ? (unsigned)j : D) >> (sh - 8)) & 255u);
                const float e = __builtin_amdgcn_exp2f(fmaxf(u + offq, -256.f));
                atomicAdd(&sm.u.sel.hist[r][dig], kOne + (unsigned long long)fixmass(e));
              }
            }
          }
          __builtin_amdgcn_sched_barrier(0);
        }
      }
      __syncthreads();
      for (int row = w; row < ROWS; row += NW) {
        const TState ts = sm.ts[row][t];
        const bool act = !ts.resolved && ts.valid;
        unsigned c[4];
        unsigned long long mm[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const unsigned long long h = sm.u.sel.hist[row][4 * lane + q];
          c[q] = (unsigned)(h >> 44);
          mm[q] = h & kMassMask;
        }
        const unsigned lc = c[0] + c[1] + c[2] + c[3];
        const unsigned long long lm = mm[0] + mm[1] + mm[2] + mm[3];
        unsigned ic = lc;
        unsigned long long im = lm;
        for (int o = 1; o < 64; o <<= 1) {
          const unsigned tc = __shfl_up(ic, o);
          const unsigned long long tm = __shfl_up(im, o);
          if (lane >= o) {
            ic += tc;
            im += tm;
          }
        }
        unsigned r0 = ic - lc;
        unsigned long long m0 = im - lm;
        const unsigned T = (unsigned)(ts.target - ts.cnt_before);
        TState nt = ts;
        bool found = false;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          if (r0 <= T && T < r0 + c[q]) {
            found = true;
            nt.prefix = (ts.prefix << 8) | (unsigned)(4 * lane + q);
            nt.sh = ts.sh - 8;
            nt.cnt_before = ts.cnt_before + (int)r0;
            nt.mass_before = ts.mass_before + m0;
            nt.cnt_in = (int)c[q];
            nt.resolved = c[q] <= (unsigned)CAP || (ts.ph == 1 && nt.sh == 0);
            if (!nt.resolved && ts.ph == 0 && nt.sh == 0) {
              // more than CAP keys share one order key: continue on their indices (j < 2^16)
              nt.ph = 1;
              nt.dfix = nt.prefix;
              nt.prefix = 0;
              nt.sh = 16;
            }
          }
          r0 += c[q];
          m0 += mm[q];
        }
        __syncthreads();
        if (act && found) sm.ts[row][t] = nt;
      }
      __syncthreads();
    }

    // gather the candidates of target t (and, for the top-32 boundary, every key ranked before it)
    if (tid < ROWS) {
      sm.ncand[tid] = 0;
      if (t == 0) sm.nwin[tid] = 0;
    }
    __syncthreads();
    if (sm.ts[r][t].valid && !sm.ts[r][t].interp) {
      const int ph = opaque(sm.ts[r][t].ph), sh = opaque(sm.ts[r][t].sh);
      const unsigned pre = opaque(sm.ts[r][t].prefix), dfix = opaque(sm.ts[r][t].dfix);
      const int gq = opaque(g);
      const float Tq = rc_T(), k32 = rc_k8() * 0x1p24f, mk32 = __fmul_rn(rc_m(), rc_k8()) * 0x1p24f;
#pragma unroll
      for (int tt = 0; tt < TPW; ++tt) {
        const int j0 = kbase + tt * 16;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int j = j0 + 4 * gq + i;
          const float u = scr(tt, i);
          if (u >= Tq) {
            const unsigned D = dkey32(u, k32, mk32);
            if (ts_in(D, j, ph, sh, pre, dfix)) {
              const int slot = atomicAdd(&sm.ncand[r], 1);
              if (slot < CAP) {
                sm.u.sel.ce[r][slot] = u;
                sm.u.sel.cj[r][slot] = j;
              }
            } else if (t == 0 && ts_before(D, j, ph, sh, pre, dfix)) {
              const int slot = atomicAdd(&sm.nwin[r], 1);
              if (slot < 32) {
                sm.win_u[r][slot] = u;
                sm.win_j[r][slot] = j;
              }
            }
          }
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    __syncthreads();
    // rank the candidates of row w exactly by (order key, index)
    for (int row = w; row < ROWS; row += NW) {
      const TState ts = sm.ts[row][t];
      const int c = min(sm.ncand[row], CAP);
      const float mr = sm.r_m[row], k32r = sm.r_k8[row] * 0x1p24f, mk32r = __fmul_rn(mr, sm.r_k8[row]) * 0x1p24f;
      if (ts.valid && !ts.interp) {
        for (int a = lane; a < c; a += 64) {
          const float ua = sm.u.sel.ce[row][a];
          const int ja = sm.u.sel.cj[row][a];
          const unsigned Da = dkey32(ua, k32r, mk32r);
          int rank = 0;
          for (int q = 0; q < c; ++q) {
            const unsigned Dq = dkey32(sm.u.sel.ce[row][q], k32r, mk32r);
            const int jq = sm.u.sel.cj[row][q];
            rank += (Dq < Da) || (Dq == Da && jq < ja);
          }
          sm.u.sel.sorted_e[row][rank] = __builtin_amdgcn_exp2f(fmaxf(ua + (kOff - mr), -256.f));
          if (t == 0) {
            const int nsel = ts.target + 1;  // min(32, n)
            const int slot = ts.cnt_before + rank;
            if (slot < nsel) {
              sm.win_u[row][slot] = ua;
              sm.win_j[row][slot] = ja;
            }
          }
        }
      }
    }
    __syncthreads();
    if (t > 0) for (int row = w; row < ROWS; row += NW) {
      const TState ts = sm.ts[row][t];
      const RowInfo ri = row_info(p, b, hkv, rb, row);
      if (ri.ok && ts.valid && !ts.interp) {
        const int rr = ts.target - ts.cnt_before;
        const int c = min(sm.ncand[row], CAP);
        float a = 0.f;
        for (int q = lane; q < c; q += 64)
          if (q < rr) a += sm.u.sel.sorted_e[row][q];
        a = wave_sum(a);
        if (lane == 0) {
          const float iz = 1.f / sm.r_z[row];
          float mass = (float)ts.mass_before * iz + a * iz;
          if (rr < c) mass += ts.frac * sm.u.sel.sorted_e[row][rr] * iz;
          sm.tmass[row][t - 1] = mass;
        }
      }
    }
    __syncthreads();
  }

  }

  // ---- E: outputs ---------------------------------------------------------------------------------
  for (int row = w; row < ROWS; row += NW) {
    const RowInfo ri = row_info(p, b, hkv, rb, row);
    if (ri.ok) {
      const int nsel = min(32, ri.nvis);
      int rank = 0, jl = -1;
      if (lane < nsel) {
        const float ul = sm.win_u[row][lane];
        jl = sm.win_j[row][lane];
#pragma unroll
        for (int q = 0; q < 32; q += 4) {  // four entries per (broadcast) read, branch-free compares
          const f32x4 u4 = *reinterpret_cast<const f32x4*>(&sm.win_u[row][q]);
          const u32x4 j4 = *reinterpret_cast<const u32x4*>(&sm.win_j[row][q]);
#pragma unroll
          for (int e = 0; e < 4; ++e)
            rank += (int)(q + e < nsel) & ((int)(u4[e] > ul) | ((int)(u4[e] == ul) & (int)((int)j4[e] < jl)));
        }
        if (p.top32) p.top32[ri.grow * 32 + rank] = jl;
        if (rank == 0) sm.top0[row] = jl;
      } else if (lane < 32) {
        if (p.top32) p.top32[ri.grow * 32 + lane] = -1;
      }
      if (lane == 0) {
        const float z = sm.r_z[row];
        const float e_ = sm.r_e[row];
        const float H = logf(z) - kLn2 * (e_ / z);
        if (p.support) p.support[ri.grow] = expf(H) / (float)ri.nvis;
      } else if (lane < NT && p.top_mass) {  // top-f mass of target t = lane
        const TState& ts = sm.ts[row][lane];
        const float mass = !ts.valid ? 0.f
                           : (ts.interp ? interp_mass(ts, sm.r_k8[row], sm.r_z[row]) : sm.tmass[row][lane - 1]);
        p.top_mass[ri.grow * 3 + lane - 1] = mass;
      }
    }
  }
  {
    // row max / lse: the lane of row r in wave 0 writes them
    const RowInfo me2 = row_info(p, b, hkv, rb, r);
    if (w == 0 && g == 0 && me2.ok) {
      if (p.row_max) p.row_max[me2.grow] = rc_m() * kLn2;
      if (p.row_lse) p.row_lse[me2.grow] = (rc_m() + log2f(rc_z()) - kOff) * kLn2;
    }
  }

  // strict zeros: only rows whose smallest e' can be at or below Z' 2^-150 need a counting pass
  {
    const float thr_u = rc_thr();
    int need = (nvis > 0 && sm.r_mn[r] <= thr_u) ? 1 : 0;
    if (tid == 0) sm.flag = 0;
    __syncthreads();
    if (need) atomicOr(&sm.flag, 1);
    __syncthreads();
    int cnt = 0;
    if (sm.flag) {
      const int gq = opaque(g), nv = opaque(nvis);
#pragma unroll
      for (int t = 0; t < TPW; ++t) {
        const int j0 = kbase + t * 16;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int j = j0 + 4 * gq + i;
          cnt += (j < nv && scr(t, i) <= thr_u) ? 1 : 0;
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    cnt = row_isum4(cnt);
    if (g == 0) sm.red_i[w][r] = cnt;
    __syncthreads();
    const RowInfo me3 = row_info(p, b, hkv, rb, r);
    if (w == 0 && g == 0 && me3.ok) {
      int tot = 0;
      for (int ww = 0; ww < NW; ++ww) tot += sm.red_i[ww][r];
      if (p.strict_zero) p.strict_zero[me3.grow] = tot;
      if (MX && p.argmax) p.argmax[me3.grow] = sm.top0[r];
    }
  }

  // ---- O = P.V --------------------------------------------------------------------------------------
  // V tiles pass through LDS, transposed: lane (kp, q8) loads keys 2kp and 2kp + 1, channels
  // 8 q8 .. 8 q8 + 7 of the half with wide loads and stores them channel-major (keys contiguous);
  // the B fragment of the MFMA (four consecutive keys of one channel) is then one 8-byte read. The
  // staging area of a wave is written and read by that wave only (LDS operations of a wave complete
  // in order).
  if (WO) {  // (compiled only into the kernels launched with p.o set: its registers stay out of the others)
    __syncthreads();  // the staging area overlays LDS that phase E read
    const float pmul = kPScale / rc_z();
#pragma unroll 1
    for (int half = 0; half < 2; ++half) {
      const float pm = opaque(pmul), offq = opaque(kOff - rc_m());  // recomputed per half, not hoisted per tile
      const int rq = opaque(r), gq = opaque(g);
      const int kp = opaque(lane & 7), q8 = opaque(lane >> 3);
      f32x4 oacc[4];
#pragma unroll
      for (int db = 0; db < 4; ++db) oacc[db] = f32x4{0.f, 0.f, 0.f, 0.f};
      // V words of a tile are loaded kVPf tiles before their use where the tile is visible and (INT4KV)
      // inside the 4-bit section; other tiles (the float32 window) load at their use. Rows of more than
      // 40 tiles per wave have no registers to spare for it.
      constexpr int kVPf = 2;
      constexpr bool kVOn = TPW <= 40;
      auto vpre = [&](int t) {
        const int jt = kbase + t * 16;
        return kVOn && jt < kmax && (KSRC == KSRC_BF16 || jt + 16 <= (int)L.n);
      };
      VRaw<KSRC> vraw[kVPf][2];
#pragma unroll
      for (int t = 0; t < kVPf && t < TPW; ++t)
        if (vpre(t))
#pragma unroll
          for (int kk = 0; kk < 2; ++kk)
            vraw[t][kk] = load_v_raw<KSRC>(rv, L, kbase + t * 16 + 2 * kp + kk, half * 64 + 8 * q8);
#pragma unroll
      for (int t = 0; t < TPW; ++t) {
        const int j0 = kbase + t * 16;
        if (j0 < kmax) {
          const bool pre = vpre(t);
#pragma unroll
          for (int kk = 0; kk < 2; ++kk) {  // one key at a time (the scores are live in registers)
            _Float16 x[8];
            if (pre)
              decode_v8<KSRC>(vraw[t % kVPf][kk], x);
            else
              load_v8<KSRC>(p, rv, L, j0 + 2 * kp + kk, half * 64 + 8 * q8, x);
#pragma unroll
            for (int e = 0; e < 8; ++e) sm.u.vst[w][8 * q8 + e][2 * kp + kk] = x[e];
          }
          if (t + kVPf < TPW && vpre(t + kVPf))
#pragma unroll
            for (int kk = 0; kk < 2; ++kk)
              vraw[t % kVPf][kk] = load_v_raw<KSRC>(rv, L, j0 + kVPf * 16 + 2 * kp + kk, half * 64 + 8 * q8);
          f16x4 pa;
#pragma unroll
          for (int i = 0; i < 4; ++i) pa[i] = (_Float16)(__builtin_amdgcn_exp2f(fmaxf(scr(t, i) + offq, -256.f)) * pm);
          __atomic_signal_fence(__ATOMIC_SEQ_CST);
#pragma unroll
          for (int db = 0; db < 4; ++db) {
            const uint2 vw = *reinterpret_cast<const uint2*>(&sm.u.vst[w][db * 16 + rq][4 * gq]);
            const f16x4 vb = __builtin_bit_cast(f16x4, vw);
            oacc[db] = __builtin_amdgcn_mfma_f32_16x16x16f16(pa, vb, oacc[db], 0, 0, 0);
          }
          __atomic_signal_fence(__ATOMIC_SEQ_CST);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
      __syncthreads();  // every wave is done with its staging area (the reduction below overlays it)
      // fixed-order tree over the waves
      for (int s = NW / 2; s >= 1; s >>= 1) {
        if (w >= s && w < 2 * s) {
#pragma unroll
          for (int db = 0; db < 4; ++db)
#pragma unroll
            for (int i = 0; i < 4; ++i) sm.u.ored[w - s][4 * g + i][db * 16 + r] = oacc[db][i];
        }
        __syncthreads();
        if (w < s) {
#pragma unroll
          for (int db = 0; db < 4; ++db)
#pragma unroll
            for (int i = 0; i < 4; ++i) oacc[db][i] += sm.u.ored[w][4 * g + i][db * 16 + r];
        }
        __syncthreads();
      }
      if (w == 0) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const RowInfo ri = row_info(p, b, hkv, rb, 4 * g + i);
          if (ri.ok) {
#pragma unroll
            for (int db = 0; db < 4; ++db)
              p.o[ri.grow * KVPROF_HEAD_DIM + half * 64 + db * 16 + r] = oacc[db][i] * (1.f / kPScale);
          }
        }
      }
    }
  }

  // ---- MXFP8 mode: bf16 reference row and the probability path ------------------------------------
  // None of these outputs depends on the exact ranks, so the main kernel writes them for every block,
  // the redo blocks included, and the redo kernel (SLOW) leaves them alone.
  if (MX && !SLOW) {
    __syncthreads();
    const RowInfo me = row_info(p, b, hkv, rb, r);
    const rsrc_t rkr = make_rsrc(p.k_ref + kvh * p.n_k * KVPROF_HEAD_DIM, head_bytes);
    // the reference Q fragments replace this lane's (long consumed) MX Q fragments in LDS
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
      sm.qs[r][ks * 4 + g] = me.ok ? *reinterpret_cast<const u32x4*>(p.q_ref + (size_t)me.grow * KVPROF_HEAD_DIM + ks * 32 + 8 * g)
                                   : zero4();
    // Reference scores of tile t through the same LDS load ring as the MX scores (whole keys per
    // load, swizzled rows); the caller has issued tile t, and this issues tile t + 1 first.
    auto ref_tile = [&](int t, float (&u)[4]) {
      const int j0 = kbase + t * 16;
      if (t + 1 < TPW) {
        issue_from(rkr, t + 1);
        __builtin_amdgcn_s_waitcnt(0x0F70 | (5 * (kRing - 1)));
      } else {
        __builtin_amdgcn_s_waitcnt(0x0F70);
      }
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
      if (j0 < kmax) {
#pragma unroll
        for (int ks = 0; ks < 4; ++ks)
          acc = mfma_step<KSRC_BF16>(sm.u.a.ring[w][t % kRing][r >> 2][(r & 3) * 16 + ((4 * ks + g) ^ r)],
                                     sm.qs[r][ks * 4 + g], acc);
      }
      const f32x4 bias = *reinterpret_cast<const f32x4*>(&sm.u.a.rbias[w][t % kRing][4 * g]);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int j = j0 + 4 * g + i;
        u[i] = j < nvis ? fmaf(acc[i], p.scale_log2, fmaxf(bias[i] * kLog2e, kNegBig)) : -INFINITY;
      }
    };
    // R1: reference max, argmax (ties to the lowest index) and normaliser in one pass: the running
    // sum is rescaled whenever the running max grows
    float best = -INFINITY, zr = 0.f;
    int bestj = 0x7fffffff;
    issue_from(rkr, 0);
#pragma unroll 1
    for (int t = 0; t < TPW; ++t) {
      const int j0 = kbase + t * 16;
      float u[4];
      ref_tile(t, u);
      float nb_ = best;  // the running max, updated key by key together with its index
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int j = j0 + 4 * g + i;
        if (u[i] > nb_ || (u[i] == nb_ && j < bestj)) {
          nb_ = u[i];
          bestj = j;
        }
      }
      if (nb_ > -INFINITY) {
        zr *= __builtin_amdgcn_exp2f(best - nb_);  // (0 while best is -inf)
#pragma unroll
        for (int i = 0; i < 4; ++i) zr += __builtin_amdgcn_exp2f(u[i] - nb_);
      }
      best = nb_;
      __builtin_amdgcn_sched_barrier(0);
    }
    // merge (max, argmax, sum) over the row's 4 lanes, then over the waves, in a fixed order
    auto merge = [](float& m1, int& j1, float& z1, float m2, int j2, float z2) {
      const float mm = fmaxf(m1, m2);
      const float za = m1 > -INFINITY ? z1 * __builtin_amdgcn_exp2f(m1 - mm) : 0.f;
      const float zb = m2 > -INFINITY ? z2 * __builtin_amdgcn_exp2f(m2 - mm) : 0.f;
      if (m2 > m1 || (m2 == m1 && j2 < j1)) j1 = j2;
      m1 = mm;
      z1 = za + zb;
    };
#pragma unroll
    for (int o = 16; o <= 32; o <<= 1) {
      const float ob = __shfl_xor(best, o), oz = __shfl_xor(zr, o);
      const int oj = __shfl_xor(bestj, o);
      merge(best, bestj, zr, ob, oj, oz);
    }
    if (g == 0) {
      sm.red_a[w][r] = best;
      sm.red_i[w][r] = bestj;
      sm.red_b[w][r] = zr;
    }
    __syncthreads();
    float mref = -INFINITY, Zr = 0.f;
    int aref = 0x7fffffff;
    for (int ww = 0; ww < NW; ++ww) merge(mref, aref, Zr, sm.red_a[ww][r], sm.red_i[ww][r], sm.red_b[ww][r]);
    if (!me.ok) mref = 0.f;
    const float invZr = me.ok ? 1.f / Zr : 0.f;
    __syncthreads();
    // R3: TV between the MX row and the reference row, and the P path
    float tv = 0.f, pz = 0.f, tvp = 0.f, psum = 0.f;
    const float offm = kOff - rc_m(), invz = 1.f / rc_z();
    // TV: the reference K tiles once more through the load ring
    issue_from(rkr, 0);
#pragma unroll
    for (int t = 0; t < TPW; ++t) {
      const int j0 = kbase + t * 16;
      if (j0 < kmax) {
        float u[4];
        ref_tile(opaque(t), u);  // (a run-time tile index: its load addresses are formed here, not kept live)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float pm = __builtin_amdgcn_exp2f(fmaxf(scr(t, i) + offm, -256.f)) * invz;
          tv += fabsf(pm - __builtin_amdgcn_exp2f(u[i] - mref) * invZr);
        }
      }
      tv = opaque(tv);
      __builtin_amdgcn_sched_barrier(0);
    }
    __builtin_amdgcn_s_waitcnt(0x0F70);  // a tile issued past this wave's last visible key has landed
    // the P path: per 32-key block (tiles t, t+1; TPW is even in MX mode) of the MX row
#pragma unroll
    for (int t = 0; t < TPW; t += 2) {
      const int j0 = kbase + t * 16;
      if (j0 < kmax) {
      float pv[2][4];
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
        for (int i = 0; i < 4; ++i) pv[h2][i] = __builtin_amdgcn_exp2f(fmaxf(scr(t + h2, i) + offm, -256.f)) * invz;
      float amax = 0.f;
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
        for (int i = 0; i < 4; ++i) amax = fmaxf(amax, pv[h2][i]);
      amax = row_max4(amax);
      const int eb = e8m0_exp(amax);
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int j = j0 + 16 * h2 + 4 * g + i;
          if (j < nvis) {
            const float pm = pv[h2][i];
            const float ph = ldexpf(e4m3_grid(ldexpf(pm, -eb)), eb);
            pz += (pm > 0.f && ph == 0.f) ? 1.f : 0.f;
            tvp += fabsf(ph - pm);
            psum += ph;
          }
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    tv = row_sum4(tv);
    pz = row_sum4(pz);
    tvp = row_sum4(tvp);
    psum = row_sum4(psum);
    if (g == 0) {
      sm.red_a[w][r] = tv;
      sm.red_b[w][r] = tvp;
      sm.segpart[w][r][0] = pz;
      sm.segpart[w][r][1] = psum;
    }
    __syncthreads();
    if (w == 0 && g == 0 && me.ok) {
      float a = 0.f, bq = 0.f, c = 0.f, d = 0.f;
      for (int ww = 0; ww < NW; ++ww) {
        a += sm.red_a[ww][r];
        bq += sm.red_b[ww][r];
        c += sm.segpart[ww][r][0];
        d += sm.segpart[ww][r][1];
      }
      if (p.tv_qk) p.tv_qk[me.grow] = 0.5f * a;
      if (p.tv_p) p.tv_p[me.grow] = 0.5f * bq;
      if (p.p_zero_frac) p.p_zero_frac[me.grow] = c / (float)me.nvis;
      if (p.p_rowsum) p.p_rowsum[me.grow] = d;
      if (p.argmax_ref) p.argmax_ref[me.grow] = aref;
    }
  }
  if (SLOW) __syncthreads();  // the next block reuses the shared memory
  }
}

__global__ void redo_reset(unsigned* redo) {
  if (threadIdx.x == 0) redo[0] = 0u;
}

template <int TPW, int KSRC, bool MX, bool WO>
hipError_t launch_wo(const RowStatsParams& p, long long nwg, hipStream_t s) {
  hipLaunchKernelGGL(redo_reset, dim3(1), dim3(64), 0, s, p.redo);
  hipLaunchKernelGGL((row_kernel<TPW, KSRC, MX, false, WO>), dim3((unsigned)nwg), dim3(WGT), 0, s, p);
  hipLaunchKernelGGL((row_kernel<TPW, KSRC, MX, true, WO>), dim3((unsigned)(nwg < kRedoGrid ? nwg : kRedoGrid)),
                     dim3(WGT), 0, s, p);
  return hipGetLastError();
}

template <int TPW, int KSRC, bool MX>
hipError_t launch_t(const RowStatsParams& p, hipStream_t s) {
  const int nrb = (p.rows_per_kv + ROWS - 1) / ROWS;
  const long long nwg = (long long)p.n_batch * p.n_heads_kv * nrb;
  if (nwg == 0) return hipSuccess;
  return p.o ? launch_wo<TPW, KSRC, MX, true>(p, nwg, s) : launch_wo<TPW, KSRC, MX, false>(p, nwg, s);
}

}  // namespace

}  // namespace kvp
