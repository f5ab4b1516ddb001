// Internal declarations shared by the HIP translation units of libkvprof (not installed).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/kvprof.h"

namespace kvp {

// ---- launch wrappers (each returns hipSuccess or the launch error) ------------------------------

hipError_t launch_pack_mxfp8(const uint16_t* x, int64_t rows, int d, const int8_t* signs,
                             uint8_t* codes, uint8_t* scales, hipStream_t s);
hipError_t launch_unpack_mxfp8(const uint8_t* codes, const uint8_t* scales, int64_t rows, int d,
                               float* out_f32, uint16_t* out_bf16, hipStream_t s);
hipError_t launch_pack_int4kv(const uint16_t* k, const uint16_t* v, int heads, int64_t N, int d,
                              int R, uint8_t* out, size_t blob_bytes, hipStream_t s);
hipError_t launch_int4kv_append(const uint8_t* in, int heads, int64_t N, int d, int r_in, const uint16_t* knew,
                                const uint16_t* vnew, int64_t t, int r_out, uint8_t* out, size_t blob_in,
                                size_t blob_out, hipStream_t s);
hipError_t launch_unpack_int4kv(const uint8_t* packed, int heads, int64_t N, int d, int R,
                                size_t blob_bytes, float* k_out, float* v_out, hipStream_t s);

// Segments: the union of region and frame boundaries, clipped to [0, n_k]. Per-row segment masses
// are the primitive the kernel reduces; region and frame masses are sums of segments.
constexpr int kMaxSeg = 80;
constexpr int kSegPerWave = 8;  // segments one wave's key range may overlap

struct RowStatsParams {
  // shapes
  int n_batch, n_heads_q, n_heads_kv, n_q, n_k;
  int group;  // n_heads_q / n_heads_kv
  int rows_per_kv;  // group * n_q
  int causal;
  long long q_pos0;
  float scale_log2;  // scale * log2(e)
  // score source
  const uint16_t* q;  // bf16 [b][hq][nq][128] (MX mode: dequantized MX values as bf16)
  const uint16_t* k;  // bf16 [b][hkv][nk][128]
  const uint16_t* v;
  const uint8_t* kv_packed;  // INT4 mode
  size_t blob_bytes;
  int r_window;
  const float* key_bias;
  // reference stream for MX mode (unrotated bf16)
  const uint16_t* q_ref;
  const uint16_t* k_ref;
  // segments
  int n_seg;
  int seg_bounds[kMaxSeg + 1];
  signed char seg_region[kMaxSeg];  // region of the segment or -1
  signed char seg_frame[kMaxSeg];   // frame of the segment or -1
  int n_regions, n_frames;
  // outputs
  float* support;
  float* top_mass;
  int* top32;
  int* strict_zero;
  float* region_mass;
  float* frame_mass;
  float* row_max;
  float* row_lse;
  float* o;
  float* tv_qk;
  int* argmax;
  int* argmax_ref;
  float* p_zero_frac;
  float* tv_p;
  float* p_rowsum;
  // workspace: [0] = number of row blocks left to the redo kernel, [1 ..] = their logical ids
  unsigned* redo;
};

// Words of the redo list for a problem of n_blocks row blocks.
inline size_t redo_words(long long n_blocks) { return (size_t)n_blocks + 1; }
inline long long row_blocks(int n_batch, int n_heads_kv, int rows_per_kv) {
  return (long long)n_batch * n_heads_kv * ((rows_per_kv + 15) / 16);
}

enum KSrc { KSRC_BF16 = 0, KSRC_INT4 = 1 };

// Main row kernel. tpw = 16-key tiles per wave (8 waves per workgroup, 16 rows per workgroup).
hipError_t launch_row_stats(const RowStatsParams& p, int tpw, int ksrc, bool mx, hipStream_t s);
hipError_t launch_row_stats_bf16(const RowStatsParams& p, int tpw, hipStream_t s);
hipError_t launch_row_stats_int4(const RowStatsParams& p, int tpw, hipStream_t s);
hipError_t launch_row_stats_mx(const RowStatsParams& p, int tpw, hipStream_t s);
int row_stats_tpw_for(int n_k, bool mx);  // tiles per wave the library uses for n_k keys, or -1

hipError_t launch_heatmap(const float* frame_mass, const int* row_group, int n_batch, int hq,
                          int nq, int n_groups, int n_frames, float* heatmap, float* heatmap_mean,
                          hipStream_t s);
hipError_t launch_hist(const float* support, const float* region_mass, int n_batch, int rows_per_b,
                       int n_regions, int bins, unsigned* hist, hipStream_t s);
hipError_t launch_compare(const float* oq, const float* oref, const int* tq, const int* tref,
                          int64_t rows, int d, float* rel_row, float* recall_row, double* sums,
                          hipStream_t s);

// ---- short heads (attend_short.hip) ----------------------------------------------------------------

struct ShortParams {
  int n_batch, n_heads_q, n_heads_kv, n_q, n_k;
  int group, rows_per_kv, causal;
  long long q_pos0;
  float scale_log2;
  const uint16_t* q;  // bf16 [b][hq][nq][d]
  const uint16_t* k;  // bf16 [b][hkv][nk][d]
  const uint16_t* v;
  const uint8_t* kv_packed;  // INT4 mode: one blob per (b, hkv)
  size_t blob_bytes;
  int r_window;
  const float* key_bias;
  int n_regions;
  int region_bounds[KVPROF_MAX_REGIONS + 1];
  float *o, *row_max, *row_lse, *region_mass, *support;
};

// d = 32 or 64; ksrc = KSRC_BF16 or KSRC_INT4.
hipError_t launch_attend_short(const ShortParams& p, int d, int ksrc, hipStream_t s);

// ---- split-key decode (decode.hip) ------------------------------------------------------------------

constexpr int kDecChunk = 1024;      // keys per workgroup
constexpr int kDecMaxChunks = 8;     // so n_k <= 8192
constexpr int kDecMaxKeys = kDecChunk * kDecMaxChunks;
// per (batch, KV head, chunk, row slot) record in the workspace, in 32-bit words
constexpr int kDecM = 0, kDecZ = 1, kDecFlag = 2, kDecReg = 3, kDecO = kDecReg + KVPROF_MAX_REGIONS,
              kDecCu = kDecO + 128, kDecCj = kDecCu + 32, kDecRecWords = 208;
static_assert(kDecCj + 32 <= kDecRecWords, "decode record");

struct DecParams {
  int n_batch, n_heads_q, n_heads_kv, n_q, n_k;
  int group, rows_per_kv, causal;
  long long q_pos0;
  float scale_log2;
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const uint8_t* kv_packed;
  size_t blob_bytes;
  int r_window;
  const float* key_bias;
  int n_regions;
  int region_bounds[KVPROF_MAX_REGIONS + 1];
  int n_chunks;
  float* part;   // workspace: n_batch * n_heads_kv * n_chunks * 16 records
  int* flags;    // workspace: [rows] 1 = the row's top-32 needs the exact fallback
  float *o, *region_mass, *row_max, *row_lse;
  int* top32;
};

hipError_t launch_decode(const DecParams& p, int ksrc, hipStream_t s);

// ---- probability maps (maps.hip) -------------------------------------------------------------------

constexpr int kMaxPoolW = 128;  // widest pooled map (four 32-column MFMA blocks)

struct MapsParams {
  int n_batch, n_heads_q, n_heads_kv, n_q, n_k;
  int group;  // n_heads_q / n_heads_kv
  int causal;
  long long q_pos0;
  float scale_log2;  // scale * log2(e)
  const uint16_t* q;  // bf16 [b][hq][nq][128]
  const uint16_t* k;  // bf16 [b][hkv][nk][128]
  const float* key_bias;
  const float* row_lse;  // [rows] natural-log log-sum-exp of every row (from the row kernel)
  float* key_part;       // [b][hq][ceil(nq/32)][nk] per-block key masses, or null
  float* pool_part;      // [rows][pool_w] per-row sums over the pooled key windows, or null
  int pool_w;
  long long p_row;       // row copied to p_row_out (when that is not null)
  float* p_row_out;
};

struct RegionBounds {
  int b[KVPROF_MAX_REGIONS + 1];
};

inline long long map_blocks(int n_batch, int n_heads_q, int n_q) {
  return (long long)n_batch * n_heads_q * ((n_q + 31) / 32);
}

hipError_t launch_maps(const MapsParams& p, const RegionBounds& bounds, float* key_mass, float* spatial,
                       float* spatial_mean, int n_regions, int frame_len, float* pooled, int pool_h,
                       hipStream_t s);
hipError_t launch_zero_f32(float* x, long long n, hipStream_t s);
hipError_t launch_percentile(const float* x, long long n, long long stride, long long m, long long lo,
                             long long hi, double frac, float* clip, float* y, hipStream_t s);

}  // namespace kvp
