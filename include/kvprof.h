/* kvprof.h — C ABI of the KV-cache attention row profiler for MI355X (gfx950).
 *
 * For every (head, query) row the library forms scaled scores against all cached keys, applies a
 * stable softmax and reduces the probability row to statistics: entropy-equivalent support exp(H)/n,
 * top-1/5/10 % mass, exact top-32 key indices, the strict-zero count, region masses and per-key-frame
 * masses; in the quantized modes it adds TV distance and argmax agreement against the bf16 row and
 * can produce O = P.V.
 *
 * Sources of the definitions (page title, section):
 *   "Catnip Week 10 KV Cache Attention Study" (cappuccino.cafe/kv-attn.html) — experiment design
 *     (boundary, sampling, signed-H128 + E4M3/E8M0 K32 Q/K, reduction), the Structural / Effective /
 *     Numerical MXFP8 definitions, the KV-cache region banner, Figure 2 (temporal heatmap) and the
 *     section on Q/K and probability quantization (TV, argmax agreement, P-path).
 *   "KV residual window" (huhohoo.com/zh-TW/docs/llm/kv-residual-window) — grouped 4-bit K/V with a
 *     float32 recent-R window, the payload table and the cut = N - R rule.
 *   The MiniCPM5-2B attention-predictor study (bjdmk.com.cn/news/5855973), section 0 — recall@32 and
 *     the GQA shape (16 query heads, 2 KV heads, head_dim 128).
 *
 * Conventions for every call:
 *   - Tensor pointers are DEVICE pointers owned by the caller. bf16 tensors are passed as uint16_t
 *     bit patterns. Argument structs and region-boundary arrays are HOST memory.
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream). On KVPROF_OK the work has
 *     been enqueued on it; nothing is synchronised.
 *   - All arguments are validated on the host before anything is enqueued: a failed call leaves the
 *     stream untouched and returns a negative status; kvprof_last_error() then describes it.
 *   - The library never allocates device memory. Scratch space comes from the caller's workspace
 *     (kvprof_workspace_bytes). Outputs must not alias inputs.
 *   - Results are bitwise deterministic for identical inputs and launch configuration.
 *   - Element types: the pages take Q/K/V at the bf16 production boundary ("Catnip Week 10 KV Cache
 *     Attention Study", experiment design: BF16 boundary tensors against an FP32 reference), so every
 *     tensor input is bf16 and rows are dense (row stride = d). The codec calls therefore carry no
 *     dtype or leading-dimension argument; a strided or float32 source is copied to dense bf16 by the
 *     caller first.
 *   - Range: the P.V product and the INT4KV scores run on f16 MFMAs. V (every call that writes o) and,
 *     in INT4KV mode, Q must lie within the f16 range (|x| < 65520); larger values overflow to inf.
 *     bf16 values below 2^-14 in magnitude lose mantissa bits there (f16 subnormals).
 */
#ifndef KVPROF_H
#define KVPROF_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define KVPROF_ABI_VERSION 2

/* Status codes. */
#define KVPROF_OK 0
#define KVPROF_EINVAL (-1)      /* null pointer where one is required, negative size, bad flag   */
#define KVPROF_ESHAPE (-2)      /* inconsistent or unsupported dimensions                          */
#define KVPROF_EALIGN (-3)      /* pointer not aligned as the argument requires                    */
#define KVPROF_ESIZE (-4)       /* an output or workspace buffer is too small                      */
#define KVPROF_EUNSUPPORTED (-6)/* valid request outside what the library implements                */
#define KVPROF_ELAUNCH (-7)     /* the HIP runtime rejected a kernel launch                        */

/* Score sources of kvprof_row_stats / kvprof_attend. */
#define KVPROF_MODE_BF16 0   /* bf16 Q and K                                                       */
#define KVPROF_MODE_MXFP8 1  /* MXFP8 Q and K codes (from kvprof_pack_mxfp8); bf16 Q, K = reference  */
#define KVPROF_MODE_INT4KV 2 /* bf16 Q against packed 4-bit K/V blobs (from kvprof_pack_int4kv)     */

/* Limits of the library. */
#define KVPROF_HEAD_DIM 128      /* head dimension of the full statistics (32 and 64: see attend)    */
#define KVPROF_MAX_KEYS 6272     /* keys per row held on chip by one workgroup (8 waves x 49 tiles)  */
#define KVPROF_MAX_KEYS_MX 6400  /* keys per row in MXFP8 mode (8 waves x 50 tiles)                    */
#define KVPROF_MAX_REGIONS 8
#define KVPROF_MAX_FRAMES 64
#define KVPROF_MAX_POOL_W 128    /* widest pooled probability map                                     */

int kvprof_abi_version(void);

/* Message describing the last non-OK status returned on the calling thread ("" if none). */
const char* kvprof_last_error(void);

/* Signed Hadamard rotation + MXFP8 E4M3/E8M0 block quantization ("K32"), per row.
 * ("Catnip Week 10 KV Cache Attention Study": experiment design step 4, and the Q/K quantization
 *  section.)
 *   x       bf16 [rows][d], rows contiguous (row stride d).
 *   signs   device int8 [d] of +1/-1, or NULL for no rotation. With signs, d must be a power of two
 *           in [32, 256]; the rotation is y = (signs * x) H_d / sqrt(d) with exact float64 sums, the
 *           product with the float64 constant 1/sqrt(d) rounded to float64 and then to float32.
 *   d       multiple of 32, at most 256.
 *   codes   uint8 [rows][d] E4M3FN codes (round to nearest even, -0 kept as 0x80).
 *   scales  uint8 [rows][d/32] E8M0 bytes e+127, e = the smallest integer with amax <= 448 * 2^e,
 *           clamped to [-127, 127] (amax = 0 gives -127); no element saturates.
 * Errors: EINVAL (null x/codes/scales, rows < 0), ESHAPE (d not a multiple of 32, or not a power of
 * two in [32, 256] with signs). rows = 0 is a no-op. */
int kvprof_pack_mxfp8(const uint16_t* x, int64_t rows, int32_t d, const int8_t* signs,
                      uint8_t* codes, uint8_t* scales, void* stream);

/* Decode MXFP8 rows: out[r][c] = E4M3(codes[r][c]) * 2^(scales[r][c/32] - 127) as float32.
 * ("Catnip Week 10 KV Cache Attention Study": experiment design step 4, E4M3 elements with E8M0 K32
 *  scales.) d: a multiple of 32 up to 256. Errors as for kvprof_pack_mxfp8. */
int kvprof_unpack_mxfp8(const uint8_t* codes, const uint8_t* scales, int64_t rows, int32_t d,
                        float* out, void* stream);

/* Bytes of one KV head's packed blob ("KV residual window": payload counting group padding, scales
 * and shapes): 16 + G*32*d/2 + G*d*4 + n*d/2 + n*(d/32)*4 + 8*R*d with n = N - R, G = ceil(n/32).
 * Returns 0 for invalid arguments (N < 0, R < 0, R > N, d not a positive multiple of 32). Host only. */
size_t kvprof_int4kv_bytes(int64_t n_tokens, int32_t d, int32_t r_window);

/* Pack grouped 4-bit K/V with a float32 recent-R window ("KV residual window": cache = [first N-R
 * tokens grouped 4-bit | last R tokens float32], group 32; K per channel over 32-token groups, V per
 * token over 32-feature groups; cut = N - R so R = 0 stores no tail).
 *   k, v     bf16 [n_heads_kv][n_tokens][d].
 *   out      n_heads_kv blobs back to back, each kvprof_int4kv_bytes(n_tokens, d, r_window) bytes,
 *            4-byte aligned. Blob layout: int32[4] {N, d, R, 32}; K codes [G*32][d/2] (low nibble =
 *            even channel, pad tokens 0); K meta [G][d] x (fp16 scale, fp16 min); V codes [n][d/2];
 *            V meta [n][d/32] x (fp16 scale, fp16 min); K residual f32 [R][d]; V residual f32 [R][d].
 *            Per group: scale = fp16(fp32(hi - lo) / 15), min = fp16(lo) over the group's valid
 *            values; code = clamp(rint((x - min) / scale), 0, 15) in float32 (0 when scale is 0).
 *            Values must lie within the fp16 range.
 *   out_bytes  capacity of out in bytes.
 * Errors: EINVAL (null pointers, negative sizes, R > N), ESHAPE (d not a multiple of 32), ESIZE
 * (out_bytes too small), EALIGN (out not 4-byte aligned). */
int kvprof_pack_int4kv(const uint16_t* k, const uint16_t* v, int32_t n_heads_kv, int64_t n_tokens,
                       int32_t d, int32_t r_window, void* out, size_t out_bytes, void* stream);

/* Dequantize packed blobs: x_hat = code * scale + min for the first N-R tokens, the float32 residual
 * after. k_out, v_out: float32 [n_heads_kv][n_tokens][d]. Errors as for kvprof_pack_int4kv. */
int kvprof_unpack_int4kv(const void* packed, int32_t n_heads_kv, int64_t n_tokens, int32_t d,
                         int32_t r_window, float* k_out, float* v_out, void* stream);

/* Rolling float32 window ("KV residual window", section on the study's limits: it builds the cache once
 * and names KIVI's residual mechanism — moving the oldest window tokens into the 4-bit part as tokens
 * arrive — as what it leaves out). Window length after appending n_new tokens to a window of r_in with
 * nominal length r_window: r = r_in + n_new if r < r_window + 32, else r - 32 * floor((r - r_window)/32)
 * (the window keeps at least the last r_window tokens and, once full, between r_window and
 * r_window + 31). Returns -1 for negative arguments. Host only. */
int64_t kvprof_int4kv_append_window(int64_t r_in, int64_t n_new, int32_t r_window);

/* Append n_new tokens to packed blobs with the rolling window above: the new tokens join the float32
 * window, whose oldest tokens then move to the 4-bit part in whole 32-token groups (K per channel over
 * the 32 tokens, V per token over 32-feature groups, the arithmetic of kvprof_pack_int4kv). The result
 * equals, byte for byte, kvprof_pack_int4kv of all n_tokens + n_new tokens with the new window length.
 *   packed   n_heads_kv input blobs (n_tokens tokens, window r_in), whose 4-bit part must hold whole
 *            groups: (n_tokens - r_in) % 32 == 0. Not modified.
 *   k_new, v_new  bf16 [n_heads_kv][n_new][d] (may be NULL when n_new == 0).
 *   out      n_heads_kv blobs of kvprof_int4kv_bytes(n_tokens + n_new, d, new window), 4-byte aligned,
 *            not overlapping packed.
 * Errors: EINVAL (null pointers, negative sizes, r_in > n_tokens, partial 4-bit group, overlap,
 * n_tokens + n_new above 2^31 - 1), ESHAPE (d not a positive multiple of 32), ESIZE (out_bytes), EALIGN. */
int kvprof_int4kv_append(const void* packed, int32_t n_heads_kv, int64_t n_tokens, int32_t d, int32_t r_in,
                         const uint16_t* k_new, const uint16_t* v_new, int64_t n_new, int32_t r_window,
                         void* out, size_t out_bytes, void* stream);

/* Arguments of kvprof_row_stats and kvprof_attend. Rows are (batch, query head, query) in that
 * order: row = (b * n_heads_q + h) * n_q + i; query head h reads KV head h / (n_heads_q/n_heads_kv). */
typedef struct kvprof_args {
  int32_t mode;                 /* KVPROF_MODE_*                                                   */
  int32_t n_batch, n_heads_q, n_heads_kv, n_q, n_k, d;
  float scale;                  /* score = scale * q.k + key_bias[j]                               */
  /* inputs (device) */
  const uint16_t* q;            /* bf16 [n_batch][n_heads_q][n_q][d]                               */
  const uint16_t* k;            /* bf16 [n_batch][n_heads_kv][n_k][d]                              */
  const uint16_t* v;            /* bf16, layout of k; needed when o != NULL outside INT4KV mode     */
  const uint8_t* q_codes;       /* MXFP8 mode: codes/scales of q and k from kvprof_pack_mxfp8       */
  const uint8_t* q_scales;
  const uint8_t* k_codes;
  const uint8_t* k_scales;
  const void* kv_packed;        /* INT4KV mode: n_batch*n_heads_kv blobs from kvprof_pack_int4kv    */
  int32_t r_window;             /* INT4KV mode: residual window the blobs were packed with          */
  const float* key_bias;        /* [n_k] additive score bias, or NULL                               */
  int32_t causal;               /* 1: key j visible to query i iff j <= q_pos0 + i                  */
  int64_t q_pos0;               /* absolute position of query 0 (>= 0)                              */
  int32_t n_regions;            /* 0..KVPROF_MAX_REGIONS                                             */
  const int32_t* region_bounds; /* HOST [n_regions+1] ascending key boundaries                       */
  int32_t frame_len, n_frames;  /* key frames [f*frame_len, (f+1)*frame_len); n_frames = 0: off      */
  const int32_t* row_group;     /* device [n_q] group (query frame) of each query, for the heatmap   */
  int32_t n_groups;
  int32_t hist_bins;            /* 0: off; 100: per-batch histograms of support and region masses   */
  /* outputs (device; NULL = not produced) */
  float* support;               /* [rows]           exp(H)/n_visible                                */
  float* top_mass;              /* [rows][3]        top-1/5/10 % mass                               */
  int32_t* top32;               /* [rows][32]       indices, score descending, ties low index; -1 pad*/
  int32_t* strict_zero;         /* [rows]           keys whose fp32 probability is exactly 0        */
  float* region_mass;           /* [rows][n_regions]                                                */
  float* frame_mass;            /* [rows][n_frames]                                                 */
  float* row_max;               /* [rows]           max score                                       */
  float* row_lse;               /* [rows]           log-sum-exp of the scores                       */
  float* o;                     /* [rows][d]        O = P.V (float32)                               */
  float* tv_qk;                 /* MXFP8 mode [rows]: 1/2 sum |p_mx - p_ref|                          */
  int32_t* argmax;              /* MXFP8 mode [rows]: argmax of the MX row (ties low index)           */
  int32_t* argmax_ref;          /* MXFP8 mode [rows]: argmax of the bf16 reference row                */
  float* p_zero_frac;           /* MXFP8 mode [rows]: keys with p > 0 whose P-path value is 0, / n     */
  float* tv_p;                  /* MXFP8 mode [rows]: 1/2 sum |P_hat - p|                              */
  float* p_rowsum;              /* MXFP8 mode [rows]: sum P_hat (not renormalised)                     */
  float* heatmap;               /* [n_batch][n_heads_q][n_groups][n_frames] mean frame mass per group */
  float* heatmap_mean;          /* [n_batch][n_groups][n_frames] heatmap averaged over query heads    */
  uint32_t* hist;               /* [n_batch][1+n_regions][hist_bins]: support, then each region mass; */
                                /*   bin = min(floor(100 x), 99). Accumulated with atomics: the call  */
                                /*   clears it first.                                                  */
  /* Probability maps, BF16 mode only ("Catnip Week 10 KV Cache Attention Study", section "Temporal & */
  /* spatial heatmaps": Figure 9's region-normalised key spatial maps, Figure 10's per-query maps; the */
  /* run manifest of the fine-grained per-head analysis, config block: the heatmap pool shape). A    */
  /* second pass over K after the row statistics, with p_ij = exp(s_ij - lse_i).                      */
  float* key_mass;              /* [n_batch][n_heads_q][n_k] sum over the head's n_q queries of p_j   */
  float* spatial;               /* [n_batch][n_heads_q][n_regions][frame_len] key spatial maps: cell c*/
                                /*   of region q = mass of the region's keys j with j mod frame_len =  */
                                /*   c, over the region's mass (all 0 when the region has none)        */
  float* spatial_mean;          /* [n_batch][n_regions][frame_len] the same over all query heads'     */
                                /*   summed key masses                                                 */
  int32_t pool_h, pool_w;       /* shape of `pooled`: pool_h >= 1, 1 <= pool_w <= KVPROF_MAX_POOL_W    */
  float* pooled;                /* [n_batch][n_heads_q][pool_h][pool_w] adaptive average pooling of   */
                                /*   each head's [n_q][n_k] probability matrix: cell (i, c) = mean of p */
                                /*   over rows [floor(i n_q/pool_h), ceil((i+1) n_q/pool_h)) x keys     */
                                /*   [floor(c n_k/pool_w), ceil((c+1) n_k/pool_w)) (invisible keys 0)   */
  int64_t p_row;                /* row (global index) whose probabilities are copied to p_row_out     */
  float* p_row_out;             /* [n_k] p of row p_row (invisible keys 0), or NULL for none          */
  void* workspace;              /* device scratch of at least kvprof_workspace_bytes(args) bytes,     */
  size_t workspace_bytes;       /*   256-byte aligned (may be NULL when that size is 0)                */
} kvprof_args;

/* Workspace bytes kvprof_row_stats / kvprof_attend need for these arguments (0 for invalid ones).
 * (The pages reduce on the GPU and move only small arrays off it — "Catnip Week 10 KV Cache Attention
 *  Study", experiment design, GPU-side reduction — so intermediate state stays in this device buffer.)
 * Every call with at least one row needs some: a list of the 16-row blocks whose exact ranks take
 * the slow path (4 bytes per block + 4), plus the decoded MXFP8 operands and, for heatmaps or
 * histograms requested without their per-row inputs, those per-row arrays; for the probability maps,
 * per-32-row-block key masses (key_mass, spatial, spatial_mean), per-row pooled window sums (pooled)
 * and row_lse / key_mass when not requested. The contents need no initialisation; concurrent calls
 * must not share a workspace. */
size_t kvprof_workspace_bytes(const kvprof_args* a);

/* Row statistics over bf16 or MXFP8 scores (modes BF16 and MXFP8), optionally with O = P.V.
 * ("Catnip Week 10 KV Cache Attention Study": the Structural / Effective / Numerical MXFP8 definitions
 *  of the experiment design — strict zeros, exp(H)/Sk support, top-1/5/10 % mass, region masses of the
 *  KV-cache banner, Figure 2's key-frame masses, Figure 5's histograms; the section on Q/K and
 *  probability quantization for TV, argmax agreement and the P-path. Top-32 indices: the MiniCPM5-2B
 *  predictor study, section 0.)
 * Requires d == 128 and n_k <= KVPROF_MAX_KEYS (KVPROF_MAX_KEYS_MX in MXFP8 mode).
 * The probability maps (key_mass ... p_row_out) need BF16 mode; spatial and spatial_mean need
 * n_regions > 0 and frame_len > 0.
 * Errors: EINVAL, ESHAPE, EALIGN (q, k, v, codes not 16-byte aligned), ESIZE (workspace),
 * EUNSUPPORTED (n_k or region/frame counts beyond the limits, maps outside BF16 mode), ELAUNCH. */
int kvprof_row_stats(const kvprof_args* a, void* stream);

/* ("KV residual window": the output of attention over the dequantized cache and its relative L2; the
 *  MiniCPM5-2B predictor study, section 0: the GQA decode shape and recall@32.)
 * Attention output O = softmax(scale q k^T + bias, causal) V over bf16 K/V (mode BF16) or over packed
 * 4-bit K/V with the float32 recent window (mode INT4KV), with any of the row statistics (the top-32
 * indices and region masses give recall@32 and the recent-window mass). o is required.
 * Head dimension 128 gives every statistic. Head dimensions 32 and 64 (the residual-window study runs at
 * 32) give o, row_max, row_lse, region_mass, support and the histograms (modes BF16 and INT4KV, any
 * n_k < 65536); other outputs return EUNSUPPORTED. kvprof_row_stats accepts the same short heads.
 * Decode-shaped calls — at most 16 query rows per KV head ((n_heads_q / n_heads_kv) * n_q <= 16), modes
 * BF16 and INT4KV, outputs among o, top32, region_mass, row_max and row_lse only — accept n_k up to
 * 8,192: rows longer than KVPROF_MAX_KEYS are split over several workgroups and merged by log-sum-exp. */
int kvprof_attend(const kvprof_args* a, void* stream);

/* Colour-range clip of a heatmap ("Catnip Week 10 KV Cache Attention Study", Figure 10: maps clipped at
 * the record's 99.5th percentile; the run manifest of the fine-grained per-head analysis, config block:
 * a quantile statistic is taken over at most 65,536 values).
 *   x     device float32 [n], n >= 1, no NaN.
 *   pct   percentile in [0, 100].
 *   cap   sample limit >= 1: all n values when n <= cap, else x[0], x[s], x[2s], ... with
 *         s = ceil(n / cap) (m = ceil(n / s) values).
 *   clip  device float32 [1]: with the m sampled values sorted ascending as v, pos = (m - 1) * pct / 100
 *         in float64, lo = floor(pos), hi = min(lo + 1, m - 1): v[lo] + (pos - lo) * (v[hi] - v[lo])
 *         in float64, rounded to float32 (linear interpolation between order statistics).
 *   y     device float32 [n] = min(x, clip) elementwise, or NULL. y may equal x.
 * Errors: EINVAL (n < 1, cap < 1, pct outside [0, 100] or not finite, null x or clip), EALIGN (arrays not
 * 4-byte aligned). */
int kvprof_percentile_clip(const float* x, int64_t n, double pct, int64_t cap, float* clip, float* y,
                           void* stream);

/* Allocation-free variant of kvprof_row_stats, for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc). It takes the same
 * arguments and produces the same results with the same kernels, but ignores a->workspace and
 * a->workspace_bytes: its scratch space is a fixed device array inside the library, of
 * kvprof_noalloc_scratch_bytes() bytes (32 MiB) on every GPU the library runs on, held until the
 * process ends. The call allocates nothing (no hipMalloc, no library allocation). Calls whose
 * kvprof_workspace_bytes() exceeds that size fail with KVPROF_ESIZE before any device work.
 * Every call on one GPU shares that GPU's array: calls that overlap in time on one GPU (on different
 * streams or host threads) race and must be serialised by the caller. The array keeps the last call's
 * contents; the kernels clear what must start at zero themselves.
 * Errors: those of kvprof_row_stats, ESIZE as above, ELAUNCH if the array's device address cannot be
 * obtained. */
int kvprof_row_stats_noalloc(const kvprof_args* a, void* stream);
size_t kvprof_noalloc_scratch_bytes(void);

/* Compare two attention outputs row by row ("KV residual window": relative L2 of the output; the
 * predictor study, section 0: recall@32).
 *   o_q, o_ref     float32 [rows][d];  top32_q, top32_ref  int32 [rows][32] (or both NULL)
 *   rel_l2_row     float32 [rows]: ||o_q[i] - o_ref[i]|| / ||o_ref[i]||
 *   recall_row     float32 [rows]: |T_q[i] intersect T_ref[i]| / 32 (needs the top32 inputs)
 *   sums           device double [2 + 2*rows]: sums[0] = sum_i ||o_q[i] - o_ref[i]||^2 and
 *                  sums[1] = sum_i ||o_ref[i]||^2 (the square root of their ratio is the tensor-level
 *                  relative L2); the remaining 2*rows entries are scratch.
 * Norms are accumulated in float64. sums[0..1] are formed in a fixed order: 256 interleaved partial
 * sums (partial t adds rows t, t+256, t+512, ... in that order), then the 256 partials in order; the
 * result is deterministic.
 * Errors: EINVAL (null outputs, rows < 0, d < 1). */
int kvprof_compare(const float* o_q, const float* o_ref, const int32_t* top32_q,
                   const int32_t* top32_ref, int64_t rows, int32_t d, float* rel_l2_row,
                   float* recall_row, double* sums, void* stream);

/* Local output ablation ("Catnip Week 10 KV Cache Attention Study", section on the current judgement
 * and next steps, recommended sequence, first item: drop the sink, the recent region or all history,
 * renormalise P, compare the output by relative L2 and cosine).
 *
 * kvprof_ablation_bias writes the key bias that drops keys [drop_lo, drop_hi):
 *   out[j] = key_bias[j] (0 when key_bias is NULL), plus -1e4 for drop_lo <= j < drop_hi.
 * A row_stats/attend call with this bias gives every dropped key an exponential that is exactly 0 in
 * float32, so its O is the output with P renormalised over the kept keys. Rows must see at least one
 * kept key (non-causal rows always do, since the range may not cover every key).
 *   key_bias  device float32 [n_k] or NULL;  out  device float32 [n_k] (may equal key_bias)
 * Errors: EINVAL (n_k < 1, null out, range outside [0, n_k], range covering every key), EALIGN.
 *
 * kvprof_cosine: cos_row[i] = a_i.b_i / (|a_i| |b_i|) (0 if either row is zero), float64 accumulation;
 *   a, b      device float32 [rows][d]; cos_row  device float32 [rows]
 *   sums      device double [3 + 3*rows]: sums[0] = sum_i a_i.b_i, sums[1] = sum_i |a_i|^2,
 *             sums[2] = sum_i |b_i|^2 (tensor-level cosine = sums[0] / sqrt(sums[1] sums[2])); the
 *             remaining 3*rows entries are scratch. The sums use the fixed interleaved order of
 *             kvprof_compare (256 partials over rows t, t+256, ..., then the partials in order).
 * Errors: EINVAL (rows < 0, d < 1, null pointers), EALIGN (sums not 8-byte aligned). */
int kvprof_ablation_bias(const float* key_bias, int32_t n_k, int32_t drop_lo, int32_t drop_hi, float* out,
                         void* stream);
int kvprof_cosine(const float* a, const float* b, int64_t rows, int32_t d, float* cos_row, double* sums,
                  void* stream);

#ifdef __cplusplus
}
#endif

#endif /* KVPROF_H */
