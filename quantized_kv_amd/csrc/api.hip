// C ABI of libkvprof: host-side validation, workspace layout and kernel dispatch.
// Every entry point validates all arguments before enqueueing anything, so a failed call leaves the
// stream untouched. The library keeps no state beyond the thread-local error message.
#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <vector>

#include "kvprof_internal.h"

namespace kvp {  // ablation.hip
hipError_t launch_ablation_bias(const float* bias, int n_k, int lo, int hi, float* out, hipStream_t s);
hipError_t launch_cosine(const float* a, const float* b, int64_t rows, int d, float* cos_row, double* sums,
                         hipStream_t s);
}  // namespace kvp

namespace {

thread_local char g_err[512] = "";

int fail(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return code;
}

int ok() {
  g_err[0] = '\0';
  return KVPROF_OK;
}

int launched(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(KVPROF_ELAUNCH, "%s: %s", what, hipGetErrorString(e));
  return ok();
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

size_t round256(size_t x) { return (x + 255) & ~size_t(255); }

bool is_pow2(int x) { return x > 0 && (x & (x - 1)) == 0; }

int check_mx_shape(const void* x, const void* codes, const void* scales, int64_t rows, int32_t d,
                   bool rotate) {
  if (rows < 0) return fail(KVPROF_EINVAL, "rows must be >= 0 (got %lld)", (long long)rows);
  if (d <= 0 || d % 32 != 0 || d > 256) return fail(KVPROF_ESHAPE, "d must be a multiple of 32 in [32, 256] (got %d)", d);
  if (rotate && !is_pow2(d)) return fail(KVPROF_ESHAPE, "the Hadamard rotation needs a power-of-two d (got %d)", d);
  if (rows > 0 && (!x || !codes || !scales)) return fail(KVPROF_EINVAL, "null input or output pointer");
  return KVPROF_OK;
}

struct Workspace {
  size_t q_mx = 0, k_mx = 0, frame = 0, support = 0, region = 0, redo = 0;
  size_t lse = 0, kpart = 0, kmass = 0, ppart = 0, dec = 0, decflags = 0, total = 0;
};

int64_t total_rows(const kvprof_args* a) { return (int64_t)a->n_batch * a->n_heads_q * a->n_q; }

bool wants_key_mass(const kvprof_args* a) { return a->key_mass || a->spatial || a->spatial_mean; }
bool wants_maps(const kvprof_args* a) { return wants_key_mass(a) || a->pooled || a->p_row_out; }

// Decode-shaped calls (at most 16 query rows per KV head, attention outputs only) whose rows are longer
// than one workgroup holds on chip (KVPROF_MAX_KEYS) take the split-key kernels, which spread a
// sequence's keys over several workgroups; shorter rows stay on the row kernel, which is faster there.
bool decode_path(const kvprof_args* a) {
  if (a->d != KVPROF_HEAD_DIM || a->mode == KVPROF_MODE_MXFP8 || a->n_heads_kv <= 0) return false;
  const int64_t rows_per_kv = (int64_t)(a->n_heads_q / a->n_heads_kv) * a->n_q;
  if (rows_per_kv < 1 || rows_per_kv > 16) return false;
  if (a->n_k <= KVPROF_MAX_KEYS || a->n_k > kvp::kDecMaxKeys) return false;
  if (a->support || a->top_mass || a->strict_zero || a->frame_mass || a->heatmap || a->heatmap_mean || a->hist)
    return false;
  if (a->tv_qk || a->argmax || a->argmax_ref || a->p_zero_frac || a->tv_p || a->p_rowsum || wants_maps(a)) return false;
  return true;
}

Workspace workspace_layout(const kvprof_args* a) {
  Workspace w;
  const int64_t rows = total_rows(a);
  size_t off = 0;
  if (a->mode == KVPROF_MODE_MXFP8) {
    w.q_mx = off;
    off += round256((size_t)rows * a->d * 2);
    w.k_mx = off;
    off += round256((size_t)a->n_batch * a->n_heads_kv * a->n_k * a->d * 2);
  }
  if (a->heatmap && !a->frame_mass) {
    w.frame = off;
    off += round256((size_t)rows * a->n_frames * 4);
  }
  if (a->hist && a->hist_bins > 0) {
    if (!a->support) {
      w.support = off;
      off += round256((size_t)rows * 4);
    }
    if (!a->region_mass && a->n_regions > 0) {
      w.region = off;
      off += round256((size_t)rows * a->n_regions * 4);
    }
  }
  if (rows > 0 && wants_maps(a)) {  // probability maps
    if (!a->row_lse) {
      w.lse = off;
      off += round256((size_t)rows * 4);
    }
    if (wants_key_mass(a)) {
      w.kpart = off;
      off += round256((size_t)kvp::map_blocks(a->n_batch, a->n_heads_q, a->n_q) * a->n_k * 4);
      if (!a->key_mass) {
        w.kmass = off;
        off += round256((size_t)a->n_batch * a->n_heads_q * a->n_k * 4);
      }
    }
    if (a->pooled && a->pool_w > 0) {
      w.ppart = off;
      off += round256((size_t)rows * a->pool_w * 4);
    }
  }
  if (rows > 0 && decode_path(a)) {  // split-key decode: chunk records and per-row fallback flags
    const int64_t nch = (a->n_k + kvp::kDecChunk - 1) / kvp::kDecChunk;
    w.dec = off;
    off += round256((size_t)a->n_batch * a->n_heads_kv * nch * 16 * kvp::kDecRecWords * 4);
    w.decflags = off;
    off += round256((size_t)rows * 4);
    w.total = off;
    return w;
  }
  if (rows > 0 && a->n_heads_kv > 0) {  // redo list of the row kernel
    w.redo = off;
    const long long nb = kvp::row_blocks(a->n_batch, a->n_heads_kv, (a->n_heads_q / a->n_heads_kv) * a->n_q);
    off += round256(kvp::redo_words(nb) * 4);
  }
  w.total = off;
  return w;
}

int validate_args(const kvprof_args* a, bool need_o) {
  if (!a) return fail(KVPROF_EINVAL, "null argument struct");
  if (a->mode != KVPROF_MODE_BF16 && a->mode != KVPROF_MODE_MXFP8 && a->mode != KVPROF_MODE_INT4KV)
    return fail(KVPROF_EINVAL, "unknown mode %d", a->mode);
  if (a->n_batch < 0 || a->n_heads_q < 0 || a->n_heads_kv < 0 || a->n_q < 0 || a->n_k < 0)
    return fail(KVPROF_EINVAL, "negative dimension");
  const bool short_head = a->d == 32 || a->d == 64;
  if (a->d != KVPROF_HEAD_DIM && !short_head)
    return fail(KVPROF_ESHAPE, "head dimension must be 32, 64 or %d (got %d)", KVPROF_HEAD_DIM, a->d);
  if (short_head) {
    if (a->mode == KVPROF_MODE_MXFP8) return fail(KVPROF_EUNSUPPORTED, "MXFP8 mode needs head dimension %d", KVPROF_HEAD_DIM);
    if (a->top_mass || a->top32 || a->strict_zero || a->frame_mass || a->heatmap || a->heatmap_mean || wants_maps(a))
      return fail(KVPROF_EUNSUPPORTED,
                  "head dimension %d computes o, row_max, row_lse, region_mass, support and histograms only", a->d);
  }
  if (a->n_heads_kv == 0 && a->n_heads_q != 0) return fail(KVPROF_ESHAPE, "n_heads_kv is 0");
  if (a->n_heads_kv > 0 && a->n_heads_q % a->n_heads_kv != 0)
    return fail(KVPROF_ESHAPE, "n_heads_q (%d) must be a multiple of n_heads_kv (%d)", a->n_heads_q, a->n_heads_kv);
  if (a->n_k < 1) return fail(KVPROF_ESHAPE, "n_k must be >= 1");
  if (a->n_k >= 65536) return fail(KVPROF_EUNSUPPORTED, "n_k must be < 65536");
  const int maxk = short_head ? 65535
                             : (decode_path(a) ? kvp::kDecMaxKeys
                                               : (a->mode == KVPROF_MODE_MXFP8 ? KVPROF_MAX_KEYS_MX : KVPROF_MAX_KEYS));
  if (a->n_k > maxk) return fail(KVPROF_EUNSUPPORTED, "n_k = %d exceeds the %d keys a row can hold in this mode", a->n_k, maxk);
  if (!std::isfinite(a->scale)) return fail(KVPROF_EINVAL, "scale must be finite");
  if (a->causal != 0 && a->causal != 1) return fail(KVPROF_EINVAL, "causal must be 0 or 1");
  if (a->q_pos0 < 0) return fail(KVPROF_EINVAL, "q_pos0 must be >= 0");
  const int64_t rows = total_rows(a);
  if (rows > 0x7fffffffLL / 32) return fail(KVPROF_EUNSUPPORTED, "too many rows (%lld)", (long long)rows);
  if (rows > 0) {
    if (!a->q) return fail(KVPROF_EINVAL, "q is null");
    if (!aligned(a->q, 16)) return fail(KVPROF_EALIGN, "q must be 16-byte aligned");
    if (a->mode != KVPROF_MODE_INT4KV) {
      if (!a->k) return fail(KVPROF_EINVAL, "k is null");
      if (!aligned(a->k, 16)) return fail(KVPROF_EALIGN, "k must be 16-byte aligned");
    }
    if (a->mode == KVPROF_MODE_MXFP8) {
      if (!a->q_codes || !a->q_scales || !a->k_codes || !a->k_scales)
        return fail(KVPROF_EINVAL, "MXFP8 mode needs q_codes, q_scales, k_codes and k_scales");
    }
    if (a->mode == KVPROF_MODE_INT4KV) {
      if (!a->kv_packed) return fail(KVPROF_EINVAL, "INT4KV mode needs kv_packed");
      if (!aligned(a->kv_packed, 16)) return fail(KVPROF_EALIGN, "kv_packed must be 16-byte aligned");
      if (a->r_window < 0 || a->r_window > a->n_k) return fail(KVPROF_EINVAL, "r_window must lie in [0, n_k]");
    }
    if (a->key_bias && !aligned(a->key_bias, 16)) return fail(KVPROF_EALIGN, "key_bias must be 16-byte aligned");
    if (need_o && !a->o) return fail(KVPROF_EINVAL, "kvprof_attend needs o");
    if (a->o && a->mode != KVPROF_MODE_INT4KV && !a->v) return fail(KVPROF_EINVAL, "o needs v");
    if (a->v && !aligned(a->v, 16)) return fail(KVPROF_EALIGN, "v must be 16-byte aligned");
  }
  if (a->n_regions < 0 || a->n_regions > KVPROF_MAX_REGIONS)
    return fail(KVPROF_EUNSUPPORTED, "n_regions must lie in [0, %d]", KVPROF_MAX_REGIONS);
  if (a->n_regions > 0) {
    if (!a->region_bounds) return fail(KVPROF_EINVAL, "region_bounds is null");
    for (int i = 0; i <= a->n_regions; ++i) {
      if (a->region_bounds[i] < 0 || a->region_bounds[i] > a->n_k)
        return fail(KVPROF_ESHAPE, "region bound %d outside [0, n_k]", a->region_bounds[i]);
      if (i > 0 && a->region_bounds[i] < a->region_bounds[i - 1])
        return fail(KVPROF_ESHAPE, "region bounds must be ascending");
    }
  }
  if (a->n_frames < 0 || a->n_frames > KVPROF_MAX_FRAMES)
    return fail(KVPROF_EUNSUPPORTED, "n_frames must lie in [0, %d]", KVPROF_MAX_FRAMES);
  if (a->n_frames > 0 && a->frame_len <= 0) return fail(KVPROF_EINVAL, "frame_len must be > 0");
  if ((a->frame_mass || a->heatmap || a->heatmap_mean) && a->n_frames == 0)
    return fail(KVPROF_EINVAL, "frame outputs need n_frames > 0");
  if (a->region_mass && a->n_regions == 0) return fail(KVPROF_EINVAL, "region_mass needs n_regions > 0");
  if (a->heatmap_mean && !a->heatmap) return fail(KVPROF_EINVAL, "heatmap_mean needs heatmap");
  if (a->heatmap && (!a->row_group || a->n_groups <= 0)) return fail(KVPROF_EINVAL, "heatmap needs row_group and n_groups > 0");
  if (a->hist_bins < 0 || a->hist_bins > 1024) return fail(KVPROF_EINVAL, "hist_bins must lie in [0, 1024]");
  if (a->hist && a->hist_bins == 0) return fail(KVPROF_EINVAL, "hist needs hist_bins > 0");
  if (wants_maps(a)) {
    if (a->mode != KVPROF_MODE_BF16) return fail(KVPROF_EUNSUPPORTED, "probability maps need BF16 mode");
    if ((a->spatial || a->spatial_mean) && (a->n_regions == 0 || a->frame_len <= 0))
      return fail(KVPROF_EINVAL, "spatial maps need n_regions > 0 and frame_len > 0");
    if (a->pooled && (a->pool_h < 1 || a->pool_w < 1 || a->pool_w > KVPROF_MAX_POOL_W))
      return fail(KVPROF_EINVAL, "pooled needs pool_h >= 1 and 1 <= pool_w <= %d (got %d x %d)", KVPROF_MAX_POOL_W,
                  a->pool_h, a->pool_w);
    if (a->pooled && a->n_q < 1) return fail(KVPROF_EINVAL, "pooled needs n_q >= 1");
    if (a->p_row_out && (a->p_row < 0 || a->p_row >= rows))
      return fail(KVPROF_EINVAL, "p_row %lld outside [0, %lld)", (long long)a->p_row, (long long)rows);
  }
  const bool tvouts = a->tv_qk || a->argmax || a->argmax_ref || a->p_zero_frac || a->tv_p || a->p_rowsum;
  if (tvouts && a->mode != KVPROF_MODE_MXFP8) return fail(KVPROF_EINVAL, "TV / argmax / P-path outputs need MXFP8 mode");
  const void* outs[] = {a->support, a->top_mass, a->top32, a->strict_zero, a->region_mass, a->frame_mass,
                        a->row_max, a->row_lse, a->o, a->tv_qk, a->argmax, a->argmax_ref, a->p_zero_frac,
                        a->tv_p, a->p_rowsum, a->heatmap, a->heatmap_mean, a->hist, a->key_mass,
                        a->spatial, a->spatial_mean, a->pooled, a->p_row_out};
  for (const void* o : outs)
    if (o && !aligned(o, 4)) return fail(KVPROF_EALIGN, "outputs must be 4-byte aligned");
  const Workspace ws = workspace_layout(a);
  if (ws.total > 0) {
    if (!a->workspace || a->workspace_bytes < ws.total)
      return fail(KVPROF_ESIZE, "workspace of %zu bytes needed (got %zu)", ws.total, a->workspace_bytes);
    if (!aligned(a->workspace, 256)) return fail(KVPROF_EALIGN, "workspace must be 256-byte aligned");
  }
  return KVPROF_OK;
}

// Segments = the union of region and frame boundaries inside [0, n_k].
int build_segments(const kvprof_args* a, kvp::RowStatsParams& p, int tpw) {
  std::vector<int> b = {0, a->n_k};
  for (int i = 0; i <= a->n_regions && a->n_regions > 0; ++i) b.push_back(a->region_bounds[i]);
  for (int f = 0; f <= a->n_frames && a->n_frames > 0; ++f) {
    long long x = (long long)f * a->frame_len;
    b.push_back((int)std::min<long long>(x, a->n_k));
  }
  std::sort(b.begin(), b.end());
  b.erase(std::unique(b.begin(), b.end()), b.end());
  const int nseg = (int)b.size() - 1;
  if (nseg > kvp::kMaxSeg) return fail(KVPROF_EUNSUPPORTED, "too many region/frame segments (%d > %d)", nseg, kvp::kMaxSeg);
  p.n_seg = nseg;
  for (int s = 0; s <= nseg; ++s) p.seg_bounds[s] = b[s];
  for (int s = 0; s < nseg; ++s) {
    const int s0 = b[s];
    p.seg_region[s] = -1;
    for (int q = 0; q < a->n_regions; ++q)
      if (a->region_bounds[q] <= s0 && s0 < a->region_bounds[q + 1]) p.seg_region[s] = (signed char)q;
    p.seg_frame[s] = -1;
    if (a->n_frames > 0 && (long long)s0 < (long long)a->n_frames * a->frame_len) p.seg_frame[s] = (signed char)(s0 / a->frame_len);
  }
  // every wave's key range may overlap at most kSegPerWave segments
  const int span = tpw * 16;
  for (int w = 0; w < 16; ++w) {
    const int w0 = w * span, w1 = w0 + span;
    int cnt = 0;
    for (int s = 0; s < nseg; ++s)
      if (b[s] < w1 && b[s + 1] > w0) ++cnt;
    if (cnt > kvp::kSegPerWave)
      return fail(KVPROF_EUNSUPPORTED, "regions/frames too fine: %d segments meet one %d-key slice (max %d)", cnt, span, kvp::kSegPerWave);
  }
  return KVPROF_OK;
}

// Short heads (d = 32, 64): the two-pass attention kernel, then the histograms.
int run_short(const kvprof_args* a, hipStream_t s) {
  const int64_t rows = total_rows(a);
  const Workspace ws = workspace_layout(a);
  char* wsb = reinterpret_cast<char*>(a->workspace);
  kvp::ShortParams p;
  std::memset(&p, 0, sizeof(p));
  p.n_batch = a->n_batch;
  p.n_heads_q = a->n_heads_q;
  p.n_heads_kv = a->n_heads_kv;
  p.n_q = a->n_q;
  p.n_k = a->n_k;
  p.group = a->n_heads_kv > 0 ? a->n_heads_q / a->n_heads_kv : 0;
  p.rows_per_kv = p.group * a->n_q;
  p.causal = a->causal;
  p.q_pos0 = a->q_pos0;
  p.scale_log2 = a->scale * 1.44269504088896340736f;
  p.q = a->q;
  p.k = a->k;
  p.v = a->v;
  p.key_bias = a->key_bias;
  p.n_regions = a->n_regions;
  for (int i = 0; i <= a->n_regions && a->n_regions > 0; ++i) p.region_bounds[i] = a->region_bounds[i];
  p.o = a->o;
  p.row_max = a->row_max;
  p.row_lse = a->row_lse;
  p.region_mass = a->region_mass;
  p.support = a->support;
  if (a->hist) {
    if (!a->support) p.support = reinterpret_cast<float*>(wsb + ws.support);
    if (!a->region_mass && a->n_regions > 0) p.region_mass = reinterpret_cast<float*>(wsb + ws.region);
  }
  int ksrc = kvp::KSRC_BF16;
  if (a->mode == KVPROF_MODE_INT4KV) {
    ksrc = kvp::KSRC_INT4;
    p.kv_packed = reinterpret_cast<const uint8_t*>(a->kv_packed);
    p.blob_bytes = kvprof_int4kv_bytes(a->n_k, a->d, a->r_window);
    p.r_window = a->r_window;
    p.k = nullptr;
    p.v = nullptr;
  }
  hipError_t e = hipSuccess;
  if (rows > 0) e = kvp::launch_attend_short(p, a->d, ksrc, s);
  if (e != hipSuccess) return launched(e, "short-head attention");
  if (a->hist) {
    e = kvp::launch_hist(p.support, p.region_mass, a->n_batch, rows > 0 ? a->n_heads_q * a->n_q : 0, a->n_regions,
                         a->hist_bins, a->hist, s);
    if (e != hipSuccess) return launched(e, "histogram");
  }
  return ok();
}

int run_decode(const kvprof_args* a, hipStream_t s) {
  const Workspace ws = workspace_layout(a);
  char* wsb = reinterpret_cast<char*>(a->workspace);
  kvp::DecParams p;
  std::memset(&p, 0, sizeof(p));
  p.n_batch = a->n_batch;
  p.n_heads_q = a->n_heads_q;
  p.n_heads_kv = a->n_heads_kv;
  p.n_q = a->n_q;
  p.n_k = a->n_k;
  p.group = a->n_heads_q / a->n_heads_kv;
  p.rows_per_kv = p.group * a->n_q;
  p.causal = a->causal;
  p.q_pos0 = a->q_pos0;
  p.scale_log2 = a->scale * 1.44269504088896340736f;
  p.q = a->q;
  p.k = a->k;
  p.v = a->v;
  p.key_bias = a->key_bias;
  p.n_regions = a->n_regions;
  for (int i = 0; i <= a->n_regions && a->n_regions > 0; ++i) p.region_bounds[i] = a->region_bounds[i];
  p.n_chunks = (a->n_k + kvp::kDecChunk - 1) / kvp::kDecChunk;
  p.part = reinterpret_cast<float*>(wsb + ws.dec);
  p.flags = reinterpret_cast<int*>(wsb + ws.decflags);
  p.o = a->o;
  p.region_mass = a->region_mass;
  p.row_max = a->row_max;
  p.row_lse = a->row_lse;
  p.top32 = a->top32;
  int ksrc = kvp::KSRC_BF16;
  if (a->mode == KVPROF_MODE_INT4KV) {
    ksrc = kvp::KSRC_INT4;
    p.kv_packed = reinterpret_cast<const uint8_t*>(a->kv_packed);
    p.blob_bytes = kvprof_int4kv_bytes(a->n_k, a->d, a->r_window);
    p.r_window = a->r_window;
    p.k = nullptr;
    p.v = nullptr;
  }
  return launched(kvp::launch_decode(p, ksrc, s), "split-key decode");
}

int run_rows(const kvprof_args* a, void* stream, bool need_o) {
  int st = validate_args(a, need_o);
  if (st != KVPROF_OK) return st;
  const int64_t rows = total_rows(a);
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  if (a->d != KVPROF_HEAD_DIM) return run_short(a, s);
  if (rows > 0 && decode_path(a)) return run_decode(a, s);
  const bool mx = a->mode == KVPROF_MODE_MXFP8;
  const int tpw = kvp::row_stats_tpw_for(a->n_k, mx);
  if (tpw < 0) return fail(KVPROF_EUNSUPPORTED, "n_k = %d is not supported", a->n_k);
  kvp::RowStatsParams p;
  std::memset(&p, 0, sizeof(p));
  st = build_segments(a, p, tpw);
  if (st != KVPROF_OK) return st;
  if (rows == 0) {
    hipError_t e0 = hipSuccess;
    if (a->hist) e0 = kvp::launch_hist(nullptr, nullptr, a->n_batch, 0, a->n_regions, a->hist_bins, a->hist, s);
    // no queries: every key receives no mass and every spatial map is zero
    const long long nbh = (long long)a->n_batch * a->n_heads_q;
    if (e0 == hipSuccess && a->key_mass) e0 = kvp::launch_zero_f32(a->key_mass, nbh * a->n_k, s);
    if (e0 == hipSuccess && a->spatial) e0 = kvp::launch_zero_f32(a->spatial, nbh * a->n_regions * a->frame_len, s);
    if (e0 == hipSuccess && a->spatial_mean)
      e0 = kvp::launch_zero_f32(a->spatial_mean, (long long)a->n_batch * a->n_regions * a->frame_len, s);
    return launched(e0, "empty problem");
  }
  const Workspace ws = workspace_layout(a);
  char* wsb = reinterpret_cast<char*>(a->workspace);
  p.n_batch = a->n_batch;
  p.n_heads_q = a->n_heads_q;
  p.n_heads_kv = a->n_heads_kv;
  p.n_q = a->n_q;
  p.n_k = a->n_k;
  p.group = a->n_heads_q / a->n_heads_kv;
  p.rows_per_kv = p.group * a->n_q;
  p.causal = a->causal;
  p.q_pos0 = a->q_pos0;
  p.scale_log2 = a->scale * 1.44269504088896340736f;
  p.q = a->q;
  p.k = a->k;
  p.v = a->v;
  p.key_bias = a->key_bias;
  p.n_regions = a->n_regions;
  p.n_frames = a->n_frames;
  p.support = a->support;
  p.top_mass = a->top_mass;
  p.top32 = a->top32;
  p.strict_zero = a->strict_zero;
  p.region_mass = a->region_mass;
  p.frame_mass = a->frame_mass;
  p.row_max = a->row_max;
  p.row_lse = a->row_lse;
  p.o = a->o;
  p.tv_qk = a->tv_qk;
  p.argmax = a->argmax;
  p.argmax_ref = a->argmax_ref;
  p.p_zero_frac = a->p_zero_frac;
  p.tv_p = a->tv_p;
  p.p_rowsum = a->p_rowsum;
  p.redo = reinterpret_cast<unsigned*>(wsb + ws.redo);
  if (a->heatmap && !a->frame_mass) p.frame_mass = reinterpret_cast<float*>(wsb + ws.frame);
  const bool maps = wants_maps(a);
  if (maps && !a->row_lse) p.row_lse = reinterpret_cast<float*>(wsb + ws.lse);
  if (a->hist) {
    if (!a->support) p.support = reinterpret_cast<float*>(wsb + ws.support);
    if (!a->region_mass && a->n_regions > 0) p.region_mass = reinterpret_cast<float*>(wsb + ws.region);
  }
  int ksrc = kvp::KSRC_BF16;
  if (a->mode == KVPROF_MODE_INT4KV) {
    ksrc = kvp::KSRC_INT4;
    p.kv_packed = reinterpret_cast<const uint8_t*>(a->kv_packed);
    p.blob_bytes = kvprof_int4kv_bytes(a->n_k, a->d, a->r_window);
    p.r_window = a->r_window;
    p.k = nullptr;
    p.v = nullptr;
  }
  if (mx) {
    uint16_t* qmx = reinterpret_cast<uint16_t*>(wsb + ws.q_mx);
    uint16_t* kmx = reinterpret_cast<uint16_t*>(wsb + ws.k_mx);
    hipError_t e = kvp::launch_unpack_mxfp8(a->q_codes, a->q_scales, rows, a->d, nullptr, qmx, s);
    if (e == hipSuccess)
      e = kvp::launch_unpack_mxfp8(a->k_codes, a->k_scales, (int64_t)a->n_batch * a->n_heads_kv * a->n_k, a->d, nullptr, kmx, s);
    if (e != hipSuccess) return launched(e, "MXFP8 decode");
    p.q_ref = a->q;
    p.k_ref = a->k;
    p.q = qmx;
    p.k = kmx;
  }
  hipError_t e = kvp::launch_row_stats(p, tpw, ksrc, mx, s);
  if (e != hipSuccess) return launched(e, "row kernel");
  if (a->heatmap) {
    e = kvp::launch_heatmap(p.frame_mass, a->row_group, a->n_batch, a->n_heads_q, a->n_q, a->n_groups,
                            a->n_frames, a->heatmap, a->heatmap_mean, s);
    if (e != hipSuccess) return launched(e, "heatmap");
  }
  if (a->hist) {
    e = kvp::launch_hist(p.support, p.region_mass, a->n_batch, a->n_heads_q * a->n_q, a->n_regions,
                         a->hist_bins, a->hist, s);
    if (e != hipSuccess) return launched(e, "histogram");
  }
  if (maps) {
    kvp::MapsParams mp;
    std::memset(&mp, 0, sizeof(mp));
    mp.n_batch = a->n_batch;
    mp.n_heads_q = a->n_heads_q;
    mp.n_heads_kv = a->n_heads_kv;
    mp.n_q = a->n_q;
    mp.n_k = a->n_k;
    mp.group = a->n_heads_q / a->n_heads_kv;
    mp.causal = a->causal;
    mp.q_pos0 = a->q_pos0;
    mp.scale_log2 = p.scale_log2;
    mp.q = a->q;
    mp.k = a->k;
    mp.key_bias = a->key_bias;
    mp.row_lse = p.row_lse;
    float* key_mass = a->key_mass;
    if (wants_key_mass(a)) {
      mp.key_part = reinterpret_cast<float*>(wsb + ws.kpart);
      if (!key_mass) key_mass = reinterpret_cast<float*>(wsb + ws.kmass);
    }
    if (a->pooled) {
      mp.pool_part = reinterpret_cast<float*>(wsb + ws.ppart);
      mp.pool_w = a->pool_w;
    }
    mp.p_row = a->p_row;
    mp.p_row_out = a->p_row_out;
    kvp::RegionBounds bounds;
    std::memset(&bounds, 0, sizeof(bounds));
    for (int i = 0; i <= a->n_regions && a->n_regions > 0; ++i) bounds.b[i] = a->region_bounds[i];
    e = kvp::launch_maps(mp, bounds, key_mass, a->spatial, a->spatial_mean, a->n_regions, a->frame_len, a->pooled,
                         a->pool_h, s);
    if (e != hipSuccess) return launched(e, "probability maps");
  }
  return ok();
}

// ---- device scratch of the allocation-free entry point -------------------------------------------
// A file-scope device array: each GPU the library runs on holds one copy until the process ends. In host
// code its name is only a stand-in, never a device address; the address comes from hipGetSymbolAddress,
// taken once per device with that device current and kept per device.
constexpr size_t kScratchBytes = size_t(32) << 20;
__device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

int scratch_of_current_device(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(KVPROF_ELAUNCH, "hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices) return fail(KVPROF_EUNSUPPORTED, "device index %d out of range", dev);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !ptr)
      return fail(KVPROF_ELAUNCH, "hipGetSymbolAddress(scratch) on device %d: %s", dev, hipGetErrorString(e));
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return KVPROF_OK;
}

}  // namespace

extern "C" {

int kvprof_abi_version(void) { return KVPROF_ABI_VERSION; }

const char* kvprof_last_error(void) { return g_err; }

int kvprof_pack_mxfp8(const uint16_t* x, int64_t rows, int32_t d, const int8_t* signs, uint8_t* codes,
                      uint8_t* scales, void* stream) {
  int st = check_mx_shape(x, codes, scales, rows, d, signs != nullptr);
  if (st != KVPROF_OK) return st;
  return launched(kvp::launch_pack_mxfp8(x, rows, d, signs, codes, scales, reinterpret_cast<hipStream_t>(stream)),
                  "pack_mxfp8");
}

int kvprof_unpack_mxfp8(const uint8_t* codes, const uint8_t* scales, int64_t rows, int32_t d, float* out,
                        void* stream) {
  int st = check_mx_shape(codes, out, scales, rows, d, false);
  if (st != KVPROF_OK) return st;
  return launched(kvp::launch_unpack_mxfp8(codes, scales, rows, d, out, nullptr, reinterpret_cast<hipStream_t>(stream)),
                  "unpack_mxfp8");
}

size_t kvprof_int4kv_bytes(int64_t n_tokens, int32_t d, int32_t r_window) {
  if (n_tokens < 0 || r_window < 0 || r_window > n_tokens || d <= 0 || d % 32 != 0) return 0;
  const int64_t n = n_tokens - r_window;
  const int64_t G = (n + 31) / 32;
  return (size_t)(16 + G * 32 * d / 2 + G * d * 4 + n * d / 2 + n * (d / 32) * 4 + 8LL * r_window * d);
}

static int check_int4(const void* a, const void* b, int32_t heads, int64_t n_tokens, int32_t d, int32_t r) {
  if (heads < 0 || n_tokens < 0) return fail(KVPROF_EINVAL, "negative size");
  if (r < 0 || r > n_tokens) return fail(KVPROF_EINVAL, "r_window must lie in [0, n_tokens] (got %d)", r);
  if (d <= 0 || d % 32 != 0) return fail(KVPROF_ESHAPE, "d must be a positive multiple of 32 (got %d)", d);
  if (heads > 0 && n_tokens > 0 && (!a || !b)) return fail(KVPROF_EINVAL, "null pointer");
  return KVPROF_OK;
}

int kvprof_pack_int4kv(const uint16_t* k, const uint16_t* v, int32_t n_heads_kv, int64_t n_tokens, int32_t d,
                       int32_t r_window, void* out, size_t out_bytes, void* stream) {
  int st = check_int4(k, v, n_heads_kv, n_tokens, d, r_window);
  if (st != KVPROF_OK) return st;
  const size_t blob = kvprof_int4kv_bytes(n_tokens, d, r_window);
  if (n_heads_kv > 0 && !out) return fail(KVPROF_EINVAL, "out is null");
  if (out_bytes < blob * (size_t)n_heads_kv)
    return fail(KVPROF_ESIZE, "out needs %zu bytes (got %zu)", blob * (size_t)n_heads_kv, out_bytes);
  if (out && !aligned(out, 4)) return fail(KVPROF_EALIGN, "out must be 4-byte aligned");
  return launched(kvp::launch_pack_int4kv(k, v, n_heads_kv, n_tokens, d, r_window, reinterpret_cast<uint8_t*>(out),
                                          blob, reinterpret_cast<hipStream_t>(stream)),
                  "pack_int4kv");
}

int kvprof_unpack_int4kv(const void* packed, int32_t n_heads_kv, int64_t n_tokens, int32_t d, int32_t r_window,
                         float* k_out, float* v_out, void* stream) {
  int st = check_int4(k_out, v_out, n_heads_kv, n_tokens, d, r_window);
  if (st != KVPROF_OK) return st;
  if (n_heads_kv > 0 && !packed) return fail(KVPROF_EINVAL, "packed is null");
  if (packed && !aligned(packed, 4)) return fail(KVPROF_EALIGN, "packed must be 4-byte aligned");
  const size_t blob = kvprof_int4kv_bytes(n_tokens, d, r_window);
  return launched(kvp::launch_unpack_int4kv(reinterpret_cast<const uint8_t*>(packed), n_heads_kv, n_tokens, d,
                                            r_window, blob, k_out, v_out, reinterpret_cast<hipStream_t>(stream)),
                  "unpack_int4kv");
}

int64_t kvprof_int4kv_append_window(int64_t r_in, int64_t n_new, int32_t r_window) {
  if (r_in < 0 || n_new < 0 || r_window < 0) return -1;
  const int64_t r = r_in + n_new;
  if (r < (int64_t)r_window + 32) return r;
  return r - 32 * ((r - r_window) / 32);
}

int kvprof_int4kv_append(const void* packed, int32_t n_heads_kv, int64_t n_tokens, int32_t d, int32_t r_in,
                         const uint16_t* k_new, const uint16_t* v_new, int64_t n_new, int32_t r_window, void* out,
                         size_t out_bytes, void* stream) {
  int st = check_int4(packed, out, n_heads_kv, n_tokens, d, r_in);
  if (st != KVPROF_OK) return st;
  if (n_new < 0 || r_window < 0) return fail(KVPROF_EINVAL, "n_new and r_window must be >= 0");
  if ((n_tokens - r_in) % 32 != 0)
    return fail(KVPROF_EINVAL, "the 4-bit part (%lld tokens) must hold whole 32-token groups", (long long)(n_tokens - r_in));
  if (n_tokens + n_new > 0x7fffffffLL) return fail(KVPROF_EINVAL, "n_tokens + n_new exceeds 2^31 - 1");
  if (n_heads_kv > 0 && n_new > 0 && (!k_new || !v_new)) return fail(KVPROF_EINVAL, "k_new / v_new is null");
  const int64_t r_out = kvprof_int4kv_append_window(r_in, n_new, r_window);
  const size_t bin = kvprof_int4kv_bytes(n_tokens, d, r_in);
  const size_t bout = kvprof_int4kv_bytes(n_tokens + n_new, d, (int32_t)r_out);
  if (out_bytes < bout * (size_t)n_heads_kv)
    return fail(KVPROF_ESIZE, "out needs %zu bytes (got %zu)", bout * (size_t)n_heads_kv, out_bytes);
  if ((packed && !aligned(packed, 4)) || (out && !aligned(out, 4))) return fail(KVPROF_EALIGN, "blobs must be 4-byte aligned");
  if ((k_new && !aligned(k_new, 2)) || (v_new && !aligned(v_new, 2))) return fail(KVPROF_EALIGN, "k_new / v_new must be 2-byte aligned");
  if (n_heads_kv > 0) {
    const uintptr_t a0 = reinterpret_cast<uintptr_t>(packed), a1 = a0 + bin * (size_t)n_heads_kv;
    const uintptr_t b0 = reinterpret_cast<uintptr_t>(out), b1 = b0 + bout * (size_t)n_heads_kv;
    if (a0 < b1 && b0 < a1) return fail(KVPROF_EINVAL, "out overlaps packed");
  }
  return launched(kvp::launch_int4kv_append(reinterpret_cast<const uint8_t*>(packed), n_heads_kv, n_tokens, d, r_in,
                                            k_new, v_new, n_new, (int)r_out, reinterpret_cast<uint8_t*>(out), bin,
                                            bout, reinterpret_cast<hipStream_t>(stream)),
                  "int4kv_append");
}

size_t kvprof_workspace_bytes(const kvprof_args* a) {
  if (!a) return 0;
  return workspace_layout(a).total;
}

int kvprof_row_stats(const kvprof_args* a, void* stream) { return run_rows(a, stream, false); }

int kvprof_attend(const kvprof_args* a, void* stream) { return run_rows(a, stream, true); }

size_t kvprof_noalloc_scratch_bytes(void) { return kScratchBytes; }

int kvprof_row_stats_noalloc(const kvprof_args* a, void* stream) {
  if (!a) return fail(KVPROF_EINVAL, "null argument struct");
  kvprof_args b = *a;
  b.workspace = nullptr;
  b.workspace_bytes = 0;
  const size_t need = workspace_layout(&b).total;
  if (need > kScratchBytes)
    return fail(KVPROF_ESIZE, "these arguments need %zu bytes of scratch; the allocation-free entry point holds %zu",
                need, kScratchBytes);
  int st = validate_args(&b, false);  // every argument check except the workspace, before any device call
  if (st != KVPROF_OK && st != KVPROF_ESIZE) return st;
  void* ptr = nullptr;
  st = scratch_of_current_device(&ptr);
  if (st != KVPROF_OK) return st;
  b.workspace = ptr;
  b.workspace_bytes = kScratchBytes;
  return run_rows(&b, stream, false);
}

int kvprof_percentile_clip(const float* x, int64_t n, double pct, int64_t cap, float* clip, float* y,
                           void* stream) {
  if (n < 1 || cap < 1) return fail(KVPROF_EINVAL, "n and cap must be >= 1 (got %lld, %lld)", (long long)n, (long long)cap);
  if (!std::isfinite(pct) || pct < 0.0 || pct > 100.0) return fail(KVPROF_EINVAL, "pct must lie in [0, 100]");
  if (!x || !clip) return fail(KVPROF_EINVAL, "null pointer");
  if (!aligned(x, 4) || !aligned(clip, 4) || (y && !aligned(y, 4))) return fail(KVPROF_EALIGN, "arrays must be 4-byte aligned");
  const int64_t stride = n <= cap ? 1 : (n + cap - 1) / cap;
  const int64_t m = (n + stride - 1) / stride;
  const double pos = (double)(m - 1) * pct / 100.0;
  const int64_t lo = (int64_t)std::floor(pos);
  const int64_t hi = std::min<int64_t>(lo + 1, m - 1);
  return launched(kvp::launch_percentile(x, n, stride, m, lo, hi, pos - (double)lo, clip, y,
                                         reinterpret_cast<hipStream_t>(stream)),
                  "percentile_clip");
}

int kvprof_compare(const float* o_q, const float* o_ref, const int32_t* top32_q, const int32_t* top32_ref,
                   int64_t rows, int32_t d, float* rel_l2_row, float* recall_row, double* sums, void* stream) {
  if (rows < 0 || d < 1) return fail(KVPROF_EINVAL, "rows must be >= 0 and d >= 1");
  if (rows > 0 && (!o_q || !o_ref || !rel_l2_row || !sums)) return fail(KVPROF_EINVAL, "null pointer");
  if ((top32_q == nullptr) != (top32_ref == nullptr)) return fail(KVPROF_EINVAL, "pass both top32 lists or neither");
  if (recall_row && !top32_q) return fail(KVPROF_EINVAL, "recall_row needs the top32 lists");
  if (sums && !aligned(sums, 8)) return fail(KVPROF_EALIGN, "sums must be 8-byte aligned");
  return launched(kvp::launch_compare(o_q, o_ref, top32_q, top32_ref, rows, d, rel_l2_row, recall_row, sums,
                                      reinterpret_cast<hipStream_t>(stream)),
                  "compare");
}

int kvprof_ablation_bias(const float* key_bias, int32_t n_k, int32_t drop_lo, int32_t drop_hi, float* out,
                         void* stream) {
  if (n_k < 1) return fail(KVPROF_EINVAL, "n_k must be >= 1 (got %d)", n_k);
  if (!out) return fail(KVPROF_EINVAL, "null output");
  if (drop_lo < 0 || drop_hi < drop_lo || drop_hi > n_k)
    return fail(KVPROF_EINVAL, "drop range [%d, %d) must lie in [0, %d]", drop_lo, drop_hi, n_k);
  if (drop_hi - drop_lo == n_k) return fail(KVPROF_EINVAL, "the ablation must keep at least one key");
  if (!aligned(out, 4) || (key_bias && !aligned(key_bias, 4))) return fail(KVPROF_EALIGN, "float arrays must be 4-byte aligned");
  return launched(kvp::launch_ablation_bias(key_bias, n_k, drop_lo, drop_hi, out,
                                            reinterpret_cast<hipStream_t>(stream)),
                  "ablation_bias");
}

int kvprof_cosine(const float* a, const float* b, int64_t rows, int32_t d, float* cos_row, double* sums,
                  void* stream) {
  if (rows < 0 || d < 1) return fail(KVPROF_EINVAL, "rows must be >= 0 and d >= 1");
  if (rows > 0 && (!a || !b || !cos_row || !sums)) return fail(KVPROF_EINVAL, "null pointer");
  if (sums && !aligned(sums, 8)) return fail(KVPROF_EALIGN, "sums must be 8-byte aligned");
  return launched(kvp::launch_cosine(a, b, rows, d, cos_row, sums, reinterpret_cast<hipStream_t>(stream)),
                  "cosine");
}

}  // extern "C"
