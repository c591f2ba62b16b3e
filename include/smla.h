/*
 * smla.h -- C ABI of libsmla, sparse MLA attention over a paged, quantized
 * latent KV cache for AMD MI355X (gfx950).
 *
 * What is computed (sources: FlashInfer PR #4802 "Refactor Sparse MLA SM120"
 * -- review of decode_dsv3_2_kernel.cuh for the 656-byte row, PR description
 * "Runtime envelopes"/"Dispatch"/"Runner and CUDA graphs" for page block 64,
 * strided index rows, row-strided LSE, topk_length, sinks and the decode
 * split-K scratch; AppMana flash-mla-ampere-dsv4 releases "decode H6" for the
 * log-sum-exp merge and "native int8_ds_mla entry" for the INT8 cache; vLLM
 * PR #57673 "Test Result" for d=512, combined top-k lists, attn_sink and
 * topk_length with non-contiguous q/out head views):
 *
 *   For each query token t and head h, the candidates are the list entries
 *   j < L_t (L_t = clamp(topk_length[t], 0, topk), or topk when no lengths
 *   are given) whose index is a slot of the pool, i.e. in [0, num_blocks*64);
 *   every other entry (-1 padding included) contributes nothing.  With K the
 *   dequantized 576-element latent row (512 "nope" + 64 "rope") and V its
 *   first 512 elements:
 *     s_j  = sm_scale * <q[t,h,:], K_j>
 *     lse  = ln sum_j exp(s_j)                (natural log, sink excluded)
 *     out  = sum_j exp(s_j) V_j / (sum_j exp(s_j) + exp(sink_h))
 *   (the sink term only when a sink array is given; it is one extra logit
 *   per head in scaled-score units and carries no value).  An empty
 *   candidate set gives out = 0 and lse = -inf.  out is BF16 (round to
 *   nearest even), lse FP32.
 *
 * Arithmetic: the scores accumulate in FP32 from the BF16 q and the exactly
 * dequantized K; the probabilities enter the value product as P x scale
 * rounded once to FP16 (11 significant bits) for quantized rows, under a
 * per-tile power-of-two bias that keeps FP16's range for any scale, and as
 * a BF16 pair (16 bits) for BF16 rows.  DSv4 rope values enter the value
 * product as FP16 and must lie within +-65504.
 *
 * Conventions for every entry point:
 *  - All data pointers are DEVICE pointers; `stream` is a hipStream_t (NULL
 *    = the default stream).  Work is enqueued asynchronously on `stream`.
 *  - The caller owns every buffer.  The library allocates and frees nothing,
 *    never synchronizes, and keeps no pointer after returning; calls on
 *    different streams may run concurrently.
 *  - Strides are in ELEMENTS of the pointed-to type; the last dimension of
 *    every tensor is contiguous.
 *  - Arguments are validated on the host before any launch; on a failed
 *    check nothing is launched and a non-zero status is returned, with a
 *    message naming the mismatch in smla_last_error().
 *  - Device-side data (indices, slots, lengths) is not validated on the
 *    host; the kernels treat out-of-range slots as padding, so no access
 *    ever leaves the pool.
 *  - T == 0 (or n == 0) returns SMLA_OK without launching anything.
 */
#ifndef SMLA_H
#define SMLA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  SMLA_OK = 0,
  SMLA_ERR_NULL = 1,        /* a required pointer is NULL */
  SMLA_ERR_SHAPE = 2,       /* a size is out of range (negative T, H < 1, topk < 1, ...) */
  SMLA_ERR_STRIDE = 3,      /* a stride or address is smaller than its row, or misaligned */
  SMLA_ERR_UNSUPPORTED = 4, /* a well-formed request outside what is built (page block != 64, H > 128, ...) */
  SMLA_ERR_HIP = 5          /* the HIP runtime reported an error when launching */
} smla_status;

/* Latent-cache row formats.  Row layout (FlashInfer PR #4802 review of the
 * DSv3.2 decode kernel): FP8 row = 656 bytes: [0,512) e4m3 codes of the 512
 * nope values, [512,528) four FP32 scales (one per 128-element tile),
 * [528,656) 64 BF16 rope values.  DSv3.2 stores power-of-two scales, and
 * the attention entry points require FP8 scales of loaded rows to be
 * positive normal powers of two (smla_quantize_kv writes only those); with
 * H > 16 a loaded row with any other scale makes its token's output NaN.
 * INT8 uses the same layout with int8 codes and any positive FP32 scale.
 * FP8_E4M3_ANY_SCALE is the same row with e4m3 codes and arbitrary positive
 * FP32 scales: the same PR's layout comment says GLM_NSA rows store
 * arbitrary scales where DSv3.2 rows store powers of two; its cache writer
 * takes scale = amax/448, and the attention entry points accept any positive
 * scale for it.  FP8_E4M3_NOPE is the FP8 row of GLM53_NOPE (same comment):
 * bytes [528, 656) are reserved padding, never written, gathered or read;
 * K and V are the 512 nope values, q rows hold 512 values (q_stride_h >=
 * 512) and the writer reads 512 values per row (kv_stride >= 512).  BF16
 * row = 576 BF16 values (1152 bytes).
 * FP8_E4M3_DOTS3 is the DOTS3_SWA row (same PR's description: d_qk 1088,
 * d_v 1024, 1160 bytes per token with the scales in a footer): [0,1024)
 * e4m3 codes of the 1024 nope values, [1024,1152) 64 BF16 rope values,
 * [1152,1160) one scale byte per 128-element tile, read as the power of
 * two 2^(b-127) (b = 255 is NaN); the byte count leaves one byte per scale.
 * K is the 1024 nope + 64 rope values and V the 1024 nope values: q rows
 * hold 1088 values, out and decode partial rows 1024, and the writer reads
 * 1088 values per latent row.  Its writer takes the power-of-two scale of
 * the FP8 rows, raised to at least 2^-126, so it stores b in [1, 254].
 * Lists of any width run on it (the page's lists hold at least 513
 * entries).
 * FP8_E4M3_DSV4 is the DSv4 row, which the same PR gives only as 584 bytes
 * (and d_v = 512 for the V3.2 family); read as [0,448) e4m3 codes of 448
 * nope values, [448,576) 64 BF16 rope values, [576,583) one scale byte per
 * 64-element tile (2^(b-127), as above; 448 = 7 x 64), [583] a pad byte the
 * writer sets to 0 and no reader uses.  K and V are the same 512 values
 * (448 nope + 64 rope): q rows hold 512 values, out rows 512, and the
 * writer reads 512 values per latent row.  Scales as for FP8_E4M3_DOTS3. */
typedef enum {
  SMLA_KV_BF16 = 0,
  SMLA_KV_FP8_E4M3 = 1,
  SMLA_KV_INT8 = 2,
  SMLA_KV_FP8_E4M3_ANY_SCALE = 3,
  SMLA_KV_FP8_E4M3_NOPE = 4,
  SMLA_KV_FP8_E4M3_DOTS3 = 5,
  SMLA_KV_FP8_E4M3_DSV4 = 6
} smla_kv_format;

/* A paged latent pool.  Slot s (a flat pool position) lives in block s/64 at
 * row s%64: byte address base + (s/64)*block_stride_bytes + (s%64)*R, with
 * R = row_stride_bytes, or the format's row bytes when row_stride_bytes is 0
 * (dense rows).  A padded row stride describes caches whose rows carry
 * bytes beyond the format's (PR #4802 review of the binding: rows addressed
 * by a token-axis stride that may exceed bytes_per_token); with one latent
 * head per row the NHD and HND block layouts differ only in these two
 * strides.  base must be 16-byte aligned; R a multiple of 16 (of 8 for
 * FP8_E4M3_DOTS3 and FP8_E4M3_DSV4, whose 1160- and 584-byte rows pack
 * 8-byte aligned) and at least
 * the row bytes; block_stride_bytes a multiple of the same and at least 64*R;
 * page_block must be 64 (PR #4802: the kernels are compiled for page block
 * 64 and launchers reject anything else).  Bytes outside the rows are never
 * read or written. */
typedef struct {
  void* base;
  int64_t num_blocks;
  int64_t block_stride_bytes;
  int32_t page_block;
  int32_t format; /* smla_kv_format */
  int64_t row_stride_bytes; /* 0: dense rows */
} smla_kv_pool;

/* Bytes of one cache row: 1152 (BF16), 656 (FP8, INT8 and the other
 * 656-byte rows), 1160 (FP8_E4M3_DOTS3), 584 (FP8_E4M3_DSV4); -1 for an
 * unknown format. */
int32_t smla_row_bytes(int32_t format);

/* Values per q row that enter a score, which is also the values per latent
 * row that smla_quantize_kv reads: 576, 512 (FP8_E4M3_NOPE and
 * FP8_E4M3_DSV4) or 1088 (FP8_E4M3_DOTS3); -1 for an unknown format. */
int32_t smla_query_dims(int32_t format);

/* Values per output row (d_v): 1024 for FP8_E4M3_DOTS3, else 512; -1 for an
 * unknown format. */
int32_t smla_value_dims(int32_t format);

/* Width of one decode split: 64 * ceil(ceil(topk / num_splits) / 64).  Split
 * s covers list positions [s*w, min((s+1)*w, topk)); trailing splits may be
 * empty.  (PR #4802: decode splits the candidate list into 64-wide chunks.)
 * Returns -1 when topk < 1 or num_splits < 1. */
int32_t smla_split_width(int32_t topk, int32_t num_splits);

/* Scratch smla_decode needs, for callers that carve it from one buffer:
 * *bytes_out = T*num_splits*H*d_v*4 (part_out) + T*num_splits*H*4
 * (part_lse), d_v = smla_value_dims of the pool's format.  part_out may
 * start at the buffer and part_lse at byte offset T*num_splits*H*d_v*4,
 * which keeps both 16-byte aligned.  (PR #4802 makes decode scratch
 * caller-owned and sized by the library so that a graph can hold it.)
 * T >= 0, H in [1, 128], num_splits in [1, 64], d_v 512 or 1024;
 * SMLA_ERR_NULL when bytes_out is NULL, SMLA_ERR_SHAPE otherwise out of
 * range. */
smla_status smla_decode_workspace_size(int64_t T, int32_t H, int32_t num_splits, int32_t d_v, size_t* bytes_out);

/* Write n latent rows into the pool.
 *   kv     BF16 [n, >=D], row i at kv + i*kv_stride (kv_stride >= D =
 *          smla_query_dims(format), multiple of 8, kv 16-byte aligned)
 *   slots  int32 [n]: destination slot of row i; slots outside
 *          [0, num_blocks*64) (-1 included) are skipped.
 * FP8: per 128-element tile of the nope part, amax = max |x|; scale = 1 when
 * amax = 0, else the power of two 2^max(ceil(log2(amax/448)), -126) (DSv3.2
 * stores FP32 power-of-two scales; the floor keeps the scale a normal FP32
 * number, which the attention entry points require); codes = e4m3(x /
 * scale), round to nearest even, sign kept.  FP8_E4M3_ANY_SCALE: scale = amax/448 (FP32, correctly rounded;
 * 1 when amax = 0), codes as for FP8.  INT8: scale = amax/127 (1 when amax = 0), codes =
 * clamp(rne(x/scale), -127, 127).  FP8_E4M3_DOTS3 and FP8_E4M3_DSV4: the
 * FP8 rule over their 128- or 64-element tiles with the scale 2^e raised
 * to at least 2^-126, e + 127 stored as the tile's scale byte.  BF16: a copy.  Rope values are copied bit for
 * bit.  Two slots that are equal race (last writer wins). */
smla_status smla_quantize_kv(const void* kv, int64_t n, int64_t kv_stride, const int32_t* slots,
                             smla_kv_pool pool, void* stream);

/* Prefill form: attention for T query tokens, written straight to out/lse.
 *   q            BF16 [T, H, D] (D = smla_query_dims(format)) with strides (q_stride_t, q_stride_h):
 *                both multiples of 8, q 16-byte aligned (views such as
 *                q[:, :8] of a wider head buffer are allowed)
 *   indices      int32 [T, >=topk], row stride idx_stride_t >= topk: flat
 *                slot ids (a narrowed view of a wider buffer is allowed)
 *   topk_length  int32 [T] or NULL
 *   sink         FP32 [H] or NULL
 *   out          BF16 [T, H, d_v] (d_v = smla_value_dims(format)) with strides (out_stride_t, out_stride_h),
 *                multiples of 8, 16-byte aligned; written in place
 *   lse          FP32 [T, H] with row stride lse_stride_t >= H
 * H in [1, 128]. */
smla_status smla_prefill(const void* q, int64_t T, int32_t H, int64_t q_stride_t, int64_t q_stride_h,
                         smla_kv_pool kv, const int32_t* indices, int32_t topk, int64_t idx_stride_t,
                         const int32_t* topk_length, const float* sink, float sm_scale,
                         void* out, int64_t out_stride_t, int64_t out_stride_h,
                         float* lse, int64_t lse_stride_t, void* stream);

/* The secondary candidate list of a dual-cache call.  FlashInfer #4802
 * gives the DSv4 decode a secondary cache with its own strided index rows
 * (commit message on strided decode indices) and lets DSv3.2-family calls
 * carry one too (PR description, "Plan layer": dual-cache decode calls had
 * ignored it); its dual-cache shapes pair a 1024-wide main list with a
 * 2176-wide secondary list.  Here the two lists form one candidate list:
 * positions [0, topk) are the main list over the main pool and positions
 * [topk, topk + extra.topk) the secondary list over extra.kv, each cut at its
 * own length (extra.topk_length, int32 [T] or NULL), and one softmax runs
 * over all candidates.  extra.kv has the main pool's format; indices are
 * int32 [T, >= extra.topk] with row stride idx_stride_t (a narrowed view is
 * allowed) and index the secondary pool's slots. */
typedef struct {
  smla_kv_pool kv;
  const int32_t* indices;
  int32_t topk;
  int64_t idx_stride_t;
  const int32_t* topk_length;
} smla_kv_extra;

/* smla_prefill over the main list and a secondary list (extra may be NULL:
 * then it is smla_prefill).  With a secondary list the main list width topk
 * must be a multiple of 64 (SMLA_ERR_UNSUPPORTED otherwise), extra.topk >= 1,
 * and extra.kv must pass the pool checks with the main pool's format. */
smla_status smla_prefill_dual(const void* q, int64_t T, int32_t H, int64_t q_stride_t, int64_t q_stride_h,
                              smla_kv_pool kv, const int32_t* indices, int32_t topk, int64_t idx_stride_t,
                              const int32_t* topk_length, const smla_kv_extra* extra, const float* sink,
                              float sm_scale, void* out, int64_t out_stride_t, int64_t out_stride_h, float* lse,
                              int64_t lse_stride_t, void* stream);

/* Decode split form: per split s (smla_split_width) of each token's list,
 * the partial result over that split's candidates, with no sink:
 *   part_lse[t,s,h] = ln sum_{j in split} exp(s_j)   (-inf when empty)
 *   part_out[t,s,h,:] = sum exp(s_j) V_j / sum exp(s_j)  (0 when empty)
 * part_out FP32 [T, num_splits, H, d_v] and part_lse FP32 [T, num_splits, H]
 * are caller-owned, contiguous, 16-byte aligned.  Other arguments as in
 * smla_prefill.  num_splits in [1, 64]. */
smla_status smla_decode(const void* q, int64_t T, int32_t H, int64_t q_stride_t, int64_t q_stride_h,
                        smla_kv_pool kv, const int32_t* indices, int32_t topk, int64_t idx_stride_t,
                        const int32_t* topk_length, float sm_scale, int32_t num_splits,
                        float* part_out, float* part_lse, void* stream);

/* smla_decode over the main list and a secondary list (as smla_prefill_dual):
 * the splits run over the combined positions [0, topk + extra.topk), with
 * split width smla_split_width(topk + extra.topk, num_splits). */
smla_status smla_decode_dual(const void* q, int64_t T, int32_t H, int64_t q_stride_t, int64_t q_stride_h,
                             smla_kv_pool kv, const int32_t* indices, int32_t topk, int64_t idx_stride_t,
                             const int32_t* topk_length, const smla_kv_extra* extra, float sm_scale,
                             int32_t num_splits, float* part_out, float* part_lse, void* stream);

/* Log-sum-exp merge of decode splits (AppMana "decode H6" combine): with
 * M = max_s part_lse, w_s = exp(part_lse_s - M) and W = sum w_s,
 *   lse = M + ln W,  o = sum_s (w_s / W) part_out_s,
 *   and with a sink o *= 1 / (1 + exp(sink_h - lse));  out = bf16(o).
 * All splits empty (M = -inf): out = 0, lse = -inf.  d_v (512 or 1024) is
 * the row width of part_out and out (smla_value_dims of the pool that
 * smla_decode read).  Buffers as in smla_decode / smla_prefill. */
smla_status smla_combine(const float* part_out, const float* part_lse, int64_t T, int32_t num_splits,
                         int32_t H, int32_t d_v, const float* sink, void* out, int64_t out_stride_t,
                         int64_t out_stride_h, float* lse, int64_t lse_stride_t, void* stream);

/* Split-count model (FlashInfer PR #4802, description sections "cpb model"
 * and "Crossover": a closed form over a few per-device constants replaces a
 * per-shape tuning sweep, and small-T prefill is routed to the split form
 * when that is predicted at most 0.95x the prefill time).  Predicted time in
 * microseconds on MI355X of smla_decode + smla_combine with num_splits
 * splits, or of smla_prefill when num_splits == 0, for T tokens of H heads
 * with topk list entries in the given format:
 *   decode  = waves * (a + b * tiles per workgroup + f * splits per workgroup)
 *             + w * MB of partials (T*S*H*(4*d_v + 4) bytes);  combine = c0 + c1 * MB;
 *   prefill = ap0 + waves * (ap + bp * tiles per token),
 * with waves = rounds of workgroups over compute_units and constants fitted
 * per kernel class (format, H > 16) by calibrate_splits.py in the package.
 * compute_units <= 0 means the current device's.  Returns -1 when T < 1,
 * H outside [1, 128], topk < 1, the format is unknown or num_splits is
 * outside [0, 64]. */
double smla_split_model_cost(int64_t T, int32_t H, int32_t topk, int32_t format, int32_t num_splits,
                             int32_t compute_units);

/* The split count in [1, min(64, ceil(topk / 64))] with the least predicted
 * decode + combine time (ties go to the smaller count); -1 on the argument
 * errors of smla_split_model_cost. */
int32_t smla_decode_num_splits(int64_t T, int32_t H, int32_t topk, int32_t format, int32_t compute_units);

/* 1 when the split form at smla_decode_num_splits is predicted to take at
 * most 0.95 of the prefill form's time, 0 when not, -1 on argument errors. */
int32_t smla_use_split_form(int64_t T, int32_t H, int32_t topk, int32_t format, int32_t compute_units);

/* Workspace smla_attention uses on the current device for this shape: the
 * smla_decode_workspace_size of the chosen split count when the split form
 * is chosen, else 0.  T >= 0, H in [1, 128], topk >= 1 (SMLA_ERR_SHAPE),
 * known format (SMLA_ERR_UNSUPPORTED), bytes_out non-NULL (SMLA_ERR_NULL). */
smla_status smla_attention_workspace_size(int64_t T, int32_t H, int32_t topk, int32_t format, size_t* bytes_out);

/* Prefill-form result (out, lse as smla_prefill defines them) by whichever
 * form the split-count model predicts faster on the current device: the
 * prefill form, or smla_decode at smla_decode_num_splits into `workspace`
 * followed by smla_combine with the sink.  The split form runs only when
 * it is chosen and workspace (16-byte aligned, caller-owned, its contents
 * overwritten) holds at least smla_attention_workspace_size bytes; with a
 * NULL or smaller workspace the prefill form runs.  Both forms compute the
 * same values up to rounding order.  Arguments and errors as smla_prefill;
 * a misaligned workspace is SMLA_ERR_STRIDE. */
smla_status smla_attention(const void* q, int64_t T, int32_t H, int64_t q_stride_t, int64_t q_stride_h,
                           smla_kv_pool kv, const int32_t* indices, int32_t topk, int64_t idx_stride_t,
                           const int32_t* topk_length, const float* sink, float sm_scale, void* out,
                           int64_t out_stride_t, int64_t out_stride_h, float* lse, int64_t lse_stride_t,
                           void* workspace, size_t workspace_bytes, void* stream);

/* ---- Measurement aids (not steps of the attention path) ---- */

/* Gather probe: moves every candidate row of each token's list (positions
 * j < L_t whose index is a slot of the pool, as in smla_prefill) into LDS
 * with 16-byte direct-to-LDS pieces, eight lanes per row, one long-lived
 * workgroup per compute unit, the index entries of up to eight tiles
 * loaded before their gathers are issued -- and computes nothing on them;
 * its time is a measured ceiling for gathering those rows.  rows_out
 * (uint32 [T], device) receives the number of rows moved for each token
 * (a kernel on the same stream clears it first).  Pools of 656- or
 * 1152-byte rows only (SMLA_ERR_UNSUPPORTED otherwise); other arguments as
 * in smla_prefill. */
smla_status smla_probe_gather(smla_kv_pool kv, const int32_t* indices, int64_t T, int32_t topk, int64_t idx_stride_t,
                              const int32_t* topk_length, uint32_t* rows_out, void* stream);

/* Clock probe: `blocks` workgroups of 4 waves each run `iters` rounds of
 * four independent BF16 MFMAs and record the shader clock counter and the
 * constant-rate counter around them; out (uint64 [2*blocks], device)
 * receives per workgroup {shader cycles, constant-rate ticks}.  With the
 * constant rate from smla_device_attributes this gives the shader clock
 * under matrix load. */
smla_status smla_probe_clock(uint64_t* out, int32_t blocks, int32_t iters, void* stream);

/* Attributes of the current device: attrs[0] compute units, attrs[1] peak
 * shader clock (kHz), attrs[2] constant-rate counter clock (kHz), attrs[3]
 * memory clock (kHz), attrs[4] memory bus width (bits).  attrs is host
 * memory, int32 [5]. */
smla_status smla_device_attributes(int32_t* attrs);

/* Bytes of the static scratch smla_attention_noalloc uses (64 MiB). */
#define SMLA_NOALLOC_SCRATCH_BYTES (64u << 20)

/* smla_attention without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc).  It computes the same out and lse
 * with the same kernels; when the split form is chosen, the decode partials
 * go to a file-scope device array of SMLA_NOALLOC_SCRATCH_BYTES bytes that
 * each GPU the library runs on holds until the process ends.  The call
 * allocates nothing (no hipMalloc, no allocating library routine); its
 * first call on a device looks up that device's copy of the array.  Every
 * call on one GPU shares the array: calls that overlap on one GPU (e.g. on
 * two streams) race and must be ordered by the caller.  The array keeps the
 * last call's partials; each call overwrites all the partials it reads.
 * Arguments and errors as smla_attention; when the chosen split form needs
 * more than SMLA_NOALLOC_SCRATCH_BYTES of partials (T*S*H*(4*d_v + 4)
 * bytes), it returns SMLA_ERR_UNSUPPORTED and launches nothing. */
smla_status smla_attention_noalloc(const void* q, int64_t T, int32_t H, int64_t q_stride_t, int64_t q_stride_h,
                                   smla_kv_pool kv, const int32_t* indices, int32_t topk, int64_t idx_stride_t,
                                   const int32_t* topk_length, const float* sink, float sm_scale, void* out,
                                   int64_t out_stride_t, int64_t out_stride_h, float* lse, int64_t lse_stride_t,
                                   void* stream);

/* Message describing the last failed call on this thread ("" if none). */
const char* smla_last_error(void);

/* Library version string. */
const char* smla_version(void);

#ifdef __cplusplus
}
#endif

#endif /* SMLA_H */
