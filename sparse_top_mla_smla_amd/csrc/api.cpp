// api.cpp -- the C entry points declared in include/smla.h: argument
// validation (everything is checked on the host before any launch) and
// dispatch to the kernels.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>

#include "smla.h"
#include "launch.h"

namespace {

thread_local char g_err[512] = "";

smla_status fail(smla_status st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof g_err, fmt, ap);
  va_end(ap);
  return st;
}

smla_status ok() {
  g_err[0] = '\0';
  return SMLA_OK;
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// rows with exponent-byte scales are 1160 or 584 bytes: rows and blocks need only 8-byte alignment
bool mx_format(int32_t format) { return format == SMLA_KV_FP8_E4M3_DOTS3 || format == SMLA_KV_FP8_E4M3_DSV4; }
int64_t row_align(int32_t format) { return mx_format(format) ? 8 : 16; }

smla_status check_pool(const smla_kv_pool& kv) {
  if (!kv.base) return fail(SMLA_ERR_NULL, "kv pool base is NULL");
  if (kv.page_block != 64)
    return fail(SMLA_ERR_UNSUPPORTED, "page_block %d is not supported (supported: 64)", kv.page_block);
  int32_t rb = smla_row_bytes(kv.format);
  if (rb < 0)
    return fail(SMLA_ERR_UNSUPPORTED,
                "kv format %d is not supported (supported: 0 = BF16, 1 = FP8_E4M3, 2 = INT8, 3 = FP8_E4M3_ANY_SCALE, "
                "4 = FP8_E4M3_NOPE, 5 = FP8_E4M3_DOTS3, 6 = FP8_E4M3_DSV4)",
                kv.format);
  if (kv.num_blocks < 1) return fail(SMLA_ERR_SHAPE, "num_blocks %lld must be >= 1", (long long)kv.num_blocks);
  if (kv.num_blocks > (int64_t)(INT32_MAX / 64) + 1)
    return fail(SMLA_ERR_SHAPE, "num_blocks %lld exceeds the int32 slot range", (long long)kv.num_blocks);
  const int64_t rs = kv.row_stride_bytes ? kv.row_stride_bytes : rb;
  if (rs < rb) return fail(SMLA_ERR_STRIDE, "row_stride_bytes %lld is smaller than the %d-byte row", (long long)rs, rb);
  const int64_t ra = row_align(kv.format);
  if (rs % ra != 0)
    return fail(SMLA_ERR_STRIDE, "row_stride_bytes %lld is not a multiple of %lld", (long long)rs, (long long)ra);
  if (kv.block_stride_bytes < 64LL * rs)
    return fail(SMLA_ERR_STRIDE, "block_stride_bytes %lld is smaller than 64 rows of %lld bytes",
                (long long)kv.block_stride_bytes, (long long)rs);
  if (kv.block_stride_bytes % ra != 0)
    return fail(SMLA_ERR_STRIDE, "block_stride_bytes %lld is not a multiple of %lld", (long long)kv.block_stride_bytes,
                (long long)ra);
  if (!aligned(kv.base, 16)) return fail(SMLA_ERR_STRIDE, "kv pool base is not 16-byte aligned");
  return SMLA_OK;
}

smla_status check_attn_common(const void* q, int64_t T, int32_t H, int64_t q_st, int64_t q_sh,
                              const smla_kv_pool& kv, const int32_t* indices, int32_t topk,
                              int64_t idx_st) {
  if (T < 0) return fail(SMLA_ERR_SHAPE, "T = %lld must be >= 0", (long long)T);
  if (T > INT32_MAX) return fail(SMLA_ERR_SHAPE, "T = %lld exceeds 2^31-1", (long long)T);
  if (T == 0) return SMLA_OK;  // nothing is read or launched
  if (H < 1) return fail(SMLA_ERR_SHAPE, "H = %d must be >= 1", H);
  if (H > 128) return fail(SMLA_ERR_UNSUPPORTED, "H = %d is not supported (supported: 1..128)", H);
  if (topk < 1) return fail(SMLA_ERR_SHAPE, "topk = %d must be >= 1", topk);
  if (!q) return fail(SMLA_ERR_NULL, "q is NULL");
  if (!indices) return fail(SMLA_ERR_NULL, "indices is NULL");
  smla_status st = check_pool(kv);
  if (st != SMLA_OK) return st;
  if (!aligned(q, 16)) return fail(SMLA_ERR_STRIDE, "q is not 16-byte aligned");
  const int64_t qd = smla_query_dims(kv.format);  // values per q row
  if (q_sh < qd || q_sh % 8 != 0)
    return fail(SMLA_ERR_STRIDE, "q_stride_h = %lld must be >= %lld and a multiple of 8", (long long)q_sh,
                (long long)qd);
  if (q_st % 8 != 0 || q_st < 0)
    return fail(SMLA_ERR_STRIDE, "q_stride_t = %lld must be a non-negative multiple of 8", (long long)q_st);
  if (idx_st < topk) return fail(SMLA_ERR_STRIDE, "idx_stride_t = %lld is smaller than topk = %d", (long long)idx_st, topk);
  if (!aligned(indices, 4)) return fail(SMLA_ERR_STRIDE, "indices is not 4-byte aligned");
  return SMLA_OK;
}

smla_status check_out(const void* out, int64_t out_st, int64_t out_sh, int32_t H, const float* lse,
                      int64_t lse_st, int32_t dv) {
  if (!out) return fail(SMLA_ERR_NULL, "out is NULL");
  if (!lse) return fail(SMLA_ERR_NULL, "lse is NULL");
  if (!aligned(out, 16)) return fail(SMLA_ERR_STRIDE, "out is not 16-byte aligned");
  if (out_sh < dv || out_sh % 8 != 0)
    return fail(SMLA_ERR_STRIDE, "out_stride_h = %lld must be >= %d and a multiple of 8", (long long)out_sh, dv);
  if (out_st % 8 != 0 || out_st < 0)
    return fail(SMLA_ERR_STRIDE, "out_stride_t = %lld must be a non-negative multiple of 8", (long long)out_st);
  if (lse_st < H) return fail(SMLA_ERR_STRIDE, "lse_stride_t = %lld is smaller than H = %d", (long long)lse_st, H);
  if (!aligned(lse, 4)) return fail(SMLA_ERR_STRIDE, "lse is not 4-byte aligned");
  return SMLA_OK;
}

// the secondary list of a dual-cache call (extra != NULL)
smla_status check_extra(const smla_kv_pool& kv, int32_t topk, const smla_kv_extra* extra) {
  if (!extra) return SMLA_OK;
  if (topk % 64 != 0)
    return fail(SMLA_ERR_UNSUPPORTED, "topk = %d: with a secondary list the main list width must be a multiple of 64",
                topk);
  if (extra->topk < 1) return fail(SMLA_ERR_SHAPE, "extra topk = %d must be >= 1", extra->topk);
  if ((int64_t)topk + extra->topk > INT32_MAX) return fail(SMLA_ERR_SHAPE, "topk + extra topk exceeds 2^31-1");
  if (!extra->indices) return fail(SMLA_ERR_NULL, "extra indices is NULL");
  smla_status st = check_pool(extra->kv);
  if (st != SMLA_OK) return st;
  if (extra->kv.format != kv.format)
    return fail(SMLA_ERR_UNSUPPORTED, "extra pool format %d differs from the main pool's %d", extra->kv.format,
                kv.format);
  if (extra->idx_stride_t < extra->topk)
    return fail(SMLA_ERR_STRIDE, "extra idx_stride_t = %lld is smaller than extra topk = %d",
                (long long)extra->idx_stride_t, extra->topk);
  if (!aligned(extra->indices, 4)) return fail(SMLA_ERR_STRIDE, "extra indices is not 4-byte aligned");
  return SMLA_OK;
}

smla_status launched(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(SMLA_ERR_HIP, "%s launch failed: %s", what, hipGetErrorString(e));
  return ok();
}

}  // namespace

extern "C" {

int32_t smla_row_bytes(int32_t format) {
  switch (format) {
    case SMLA_KV_BF16: return 1152;
    case SMLA_KV_FP8_E4M3: return 656;
    case SMLA_KV_INT8: return 656;
    case SMLA_KV_FP8_E4M3_ANY_SCALE: return 656;
    case SMLA_KV_FP8_E4M3_NOPE: return 656;
    case SMLA_KV_FP8_E4M3_DOTS3: return 1160;
    case SMLA_KV_FP8_E4M3_DSV4: return 584;
    default: return -1;
  }
}

int32_t smla_query_dims(int32_t format) {
  switch (format) {
    case SMLA_KV_BF16:
    case SMLA_KV_FP8_E4M3:
    case SMLA_KV_INT8:
    case SMLA_KV_FP8_E4M3_ANY_SCALE: return 576;
    case SMLA_KV_FP8_E4M3_NOPE:
    case SMLA_KV_FP8_E4M3_DSV4: return 512;
    case SMLA_KV_FP8_E4M3_DOTS3: return 1088;
    default: return -1;
  }
}

int32_t smla_value_dims(int32_t format) {
  if (smla_row_bytes(format) < 0) return -1;
  return format == SMLA_KV_FP8_E4M3_DOTS3 ? 1024 : 512;  // (DSv4: V is the whole 512-value row)
}

int32_t smla_split_width(int32_t topk, int32_t num_splits) {
  if (topk < 1 || num_splits < 1) return -1;
  int32_t per = (topk + num_splits - 1) / num_splits;
  return ((per + 63) / 64) * 64;
}

smla_status smla_decode_workspace_size(int64_t T, int32_t H, int32_t num_splits, int32_t d_v, size_t* bytes_out) {
  if (!bytes_out) return fail(SMLA_ERR_NULL, "bytes_out is NULL");
  if (T < 0) return fail(SMLA_ERR_SHAPE, "T = %lld must be >= 0", (long long)T);
  if (H < 1 || H > 128) return fail(SMLA_ERR_SHAPE, "H = %d is outside [1, 128]", H);
  if (num_splits < 1 || num_splits > 64)
    return fail(SMLA_ERR_SHAPE, "num_splits = %d is outside [1, 64]", num_splits);
  if (d_v != 512 && d_v != 1024) return fail(SMLA_ERR_SHAPE, "d_v = %d is not 512 or 1024", d_v);
  const size_t rows = (size_t)T * (size_t)num_splits * (size_t)H;
  *bytes_out = rows * (size_t)d_v * sizeof(float) + rows * sizeof(float);
  return ok();
}

const char* smla_last_error(void) { return g_err; }

const char* smla_version(void) { return "smla 0.2.0 (gfx950)"; }

smla_status smla_quantize_kv(const void* kv, int64_t n, int64_t kv_stride, const int32_t* slots,
                             smla_kv_pool pool, void* stream) {
  if (n < 0) return fail(SMLA_ERR_SHAPE, "n = %lld must be >= 0", (long long)n);
  if (n == 0) return ok();
  if (!kv) return fail(SMLA_ERR_NULL, "kv is NULL");
  if (!slots) return fail(SMLA_ERR_NULL, "slots is NULL");
  smla_status st = check_pool(pool);
  if (st != SMLA_OK) return st;
  const int64_t kd = smla_query_dims(pool.format);  // values read per latent row
  if (kv_stride < kd || kv_stride % 8 != 0)
    return fail(SMLA_ERR_STRIDE, "kv_stride = %lld must be >= %lld and a multiple of 8", (long long)kv_stride,
                (long long)kd);
  if (!aligned(kv, 16)) return fail(SMLA_ERR_STRIDE, "kv is not 16-byte aligned");
  if (!aligned(slots, 4)) return fail(SMLA_ERR_STRIDE, "slots is not 4-byte aligned");
  if ((n + 3) / 4 > (int64_t)UINT32_MAX) return fail(SMLA_ERR_SHAPE, "n = %lld is too large", (long long)n);
  smla::QuantParams p{};
  p.kv = static_cast<const uint16_t*>(kv);
  p.n = n;
  p.kv_stride = kv_stride;
  p.slots = slots;
  p.pool = static_cast<uint8_t*>(pool.base);
  p.nslots = pool.num_blocks * 64;
  p.block_stride = pool.block_stride_bytes;
  p.row_stride = pool.row_stride_bytes ? pool.row_stride_bytes : smla_row_bytes(pool.format);
  return launched(smla::launch_quantize(p, pool.format, static_cast<hipStream_t>(stream)), "quantize");
}

static void fill_attn(smla::AttnParams& p, const void* q, int64_t T, int32_t H, int64_t q_st, int64_t q_sh,
                      const smla_kv_pool& kv, const int32_t* indices, int32_t topk, int64_t idx_st,
                      const int32_t* topk_length, float sm_scale) {
  std::memset(&p, 0, sizeof p);
  p.q = static_cast<const uint16_t*>(q);
  p.q_st = q_st;
  p.q_sh = q_sh;
  p.T = T;
  p.H = H;
  p.pool = static_cast<const uint8_t*>(kv.base);
  p.block_stride = kv.block_stride_bytes;
  p.row_stride = kv.row_stride_bytes ? kv.row_stride_bytes : smla_row_bytes(kv.format);
  p.nslots = kv.num_blocks * 64;
  p.idx = indices;
  p.idx_st = idx_st;
  p.topk = topk;
  p.topk_length = topk_length;
  p.scale_log2 = sm_scale * 1.4426950408889634f;
  p.nope = kv.format == SMLA_KV_FP8_E4M3_NOPE;
}

static void fill_extra(smla::AttnParams& p, const smla_kv_extra* extra) {
  if (!extra) return;
  p.pool2 = static_cast<const uint8_t*>(extra->kv.base);
  p.block_stride2 = extra->kv.block_stride_bytes;
  p.row_stride2 = extra->kv.row_stride_bytes ? extra->kv.row_stride_bytes : smla_row_bytes(extra->kv.format);
  p.nslots2 = extra->kv.num_blocks * 64;
  p.idx2 = extra->indices;
  p.idx_st2 = extra->idx_stride_t;
  p.topk2 = extra->topk;
  p.topk_length2 = extra->topk_length;
}

smla_status smla_prefill(const void* q, int64_t T, int32_t H, int64_t q_stride_t, int64_t q_stride_h,
                         smla_kv_pool kv, const int32_t* indices, int32_t topk, int64_t idx_stride_t,
                         const int32_t* topk_length, const float* sink, float sm_scale, void* out,
                         int64_t out_stride_t, int64_t out_stride_h, float* lse, int64_t lse_stride_t,
                         void* stream) {
  return smla_prefill_dual(q, T, H, q_stride_t, q_stride_h, kv, indices, topk, idx_stride_t, topk_length, nullptr,
                           sink, sm_scale, out, out_stride_t, out_stride_h, lse, lse_stride_t, stream);
}

smla_status smla_prefill_dual(const void* q, int64_t T, int32_t H, int64_t q_stride_t, int64_t q_stride_h,
                              smla_kv_pool kv, const int32_t* indices, int32_t topk, int64_t idx_stride_t,
                              const int32_t* topk_length, const smla_kv_extra* extra, const float* sink,
                              float sm_scale, void* out, int64_t out_stride_t, int64_t out_stride_h, float* lse,
                              int64_t lse_stride_t, void* stream) {
  smla_status st = check_attn_common(q, T, H, q_stride_t, q_stride_h, kv, indices, topk, idx_stride_t);
  if (st != SMLA_OK) return st;
  if (T == 0) return ok();
  st = check_extra(kv, topk, extra);
  if (st != SMLA_OK) return st;
  st = check_out(out, out_stride_t, out_stride_h, H, lse, lse_stride_t, smla_value_dims(kv.format));
  if (st != SMLA_OK) return st;
  if (!std::isfinite(sm_scale)) return fail(SMLA_ERR_SHAPE, "sm_scale must be finite");
  if (T == 0) return ok();
  smla::AttnParams p{};
  fill_attn(p, q, T, H, q_stride_t, q_stride_h, kv, indices, topk, idx_stride_t, topk_length, sm_scale);
  fill_extra(p, extra);
  p.sink = sink;
  p.out = static_cast<uint16_t*>(out);
  p.out_st = out_stride_t;
  p.out_sh = out_stride_h;
  p.lse = lse;
  p.lse_st = lse_stride_t;
  return launched(smla::launch_attention(p, kv.format, false, static_cast<hipStream_t>(stream)), "prefill");
}

smla_status smla_decode(const void* q, int64_t T, int32_t H, int64_t q_stride_t, int64_t q_stride_h,
                        smla_kv_pool kv, const int32_t* indices, int32_t topk, int64_t idx_stride_t,
                        const int32_t* topk_length, float sm_scale, int32_t num_splits, float* part_out,
                        float* part_lse, void* stream) {
  return smla_decode_dual(q, T, H, q_stride_t, q_stride_h, kv, indices, topk, idx_stride_t, topk_length, nullptr,
                          sm_scale, num_splits, part_out, part_lse, stream);
}

smla_status smla_decode_dual(const void* q, int64_t T, int32_t H, int64_t q_stride_t, int64_t q_stride_h,
                             smla_kv_pool kv, const int32_t* indices, int32_t topk, int64_t idx_stride_t,
                             const int32_t* topk_length, const smla_kv_extra* extra, float sm_scale,
                             int32_t num_splits, float* part_out, float* part_lse, void* stream) {
  smla_status st = check_attn_common(q, T, H, q_stride_t, q_stride_h, kv, indices, topk, idx_stride_t);
  if (st != SMLA_OK) return st;
  if (T == 0) return ok();
  st = check_extra(kv, topk, extra);
  if (st != SMLA_OK) return st;
  if (num_splits < 1 || num_splits > 64)
    return fail(SMLA_ERR_UNSUPPORTED, "num_splits = %d is not supported (supported: 1..64)", num_splits);
  if (!part_out) return fail(SMLA_ERR_NULL, "part_out is NULL");
  if (!part_lse) return fail(SMLA_ERR_NULL, "part_lse is NULL");
  if (!aligned(part_out, 16)) return fail(SMLA_ERR_STRIDE, "part_out is not 16-byte aligned");
  if (!aligned(part_lse, 4)) return fail(SMLA_ERR_STRIDE, "part_lse is not 4-byte aligned");
  if (!std::isfinite(sm_scale)) return fail(SMLA_ERR_SHAPE, "sm_scale must be finite");
  if (T == 0) return ok();
  smla::AttnParams p{};
  fill_attn(p, q, T, H, q_stride_t, q_stride_h, kv, indices, topk, idx_stride_t, topk_length, sm_scale);
  fill_extra(p, extra);
  p.part_out = part_out;
  p.part_lse = part_lse;
  p.num_splits = num_splits;
  p.split_w = smla_split_width(topk + p.topk2, num_splits);
  p.splits_per_block = 1;
  return launched(smla::launch_attention(p, kv.format, true, static_cast<hipStream_t>(stream)), "decode");
}

smla_status smla_combine(const float* part_out, const float* part_lse, int64_t T, int32_t num_splits,
                         int32_t H, int32_t d_v, const float* sink, void* out, int64_t out_stride_t,
                         int64_t out_stride_h, float* lse, int64_t lse_stride_t, void* stream) {
  if (T < 0) return fail(SMLA_ERR_SHAPE, "T = %lld must be >= 0", (long long)T);
  if (T == 0) return ok();  // nothing is read or launched
  if (d_v != 512 && d_v != 1024) return fail(SMLA_ERR_SHAPE, "d_v = %d is not 512 or 1024", d_v);
  if (H < 1) return fail(SMLA_ERR_SHAPE, "H = %d must be >= 1", H);
  if (H > 128) return fail(SMLA_ERR_UNSUPPORTED, "H = %d is not supported (supported: 1..128)", H);
  if (num_splits < 1 || num_splits > 64)
    return fail(SMLA_ERR_UNSUPPORTED, "num_splits = %d is not supported (supported: 1..64)", num_splits);
  if (!part_out) return fail(SMLA_ERR_NULL, "part_out is NULL");
  if (!part_lse) return fail(SMLA_ERR_NULL, "part_lse is NULL");
  if (!aligned(part_out, 16)) return fail(SMLA_ERR_STRIDE, "part_out is not 16-byte aligned");
  smla_status st = check_out(out, out_stride_t, out_stride_h, H, lse, lse_stride_t, d_v);
  if (st != SMLA_OK) return st;
  if (T == 0) return ok();
  if ((T * H + 3) / 4 > (int64_t)UINT32_MAX) return fail(SMLA_ERR_SHAPE, "T*H is too large");
  smla::CombineParams p;
  p.dv = d_v;
  p.part_out = part_out;
  p.part_lse = part_lse;
  p.T = T;
  p.S = num_splits;
  p.H = H;
  p.sink = sink;
  p.out = static_cast<uint16_t*>(out);
  p.out_st = out_stride_t;
  p.out_sh = out_stride_h;
  p.lse = lse;
  p.lse_st = lse_stride_t;
  return launched(smla::launch_combine(p, static_cast<hipStream_t>(stream)), "combine");
}

}  // extern "C"

smla_status smla_attention_workspace_size(int64_t T, int32_t H, int32_t topk, int32_t format, size_t* bytes_out) {
  if (!bytes_out) return fail(SMLA_ERR_NULL, "bytes_out is NULL");
  if (T < 0 || T > INT32_MAX) return fail(SMLA_ERR_SHAPE, "T = %lld is outside [0, 2^31-1]", (long long)T);
  if (H < 1 || H > 128) return fail(SMLA_ERR_SHAPE, "H = %d is outside [1, 128]", H);
  if (topk < 1) return fail(SMLA_ERR_SHAPE, "topk = %d must be >= 1", topk);
  if (smla_row_bytes(format) < 0) return fail(SMLA_ERR_UNSUPPORTED, "kv format %d is not supported", format);
  *bytes_out = 0;
  if (T == 0 || smla_use_split_form(T, H, topk, format, 0) != 1) return ok();
  return smla_decode_workspace_size(T, H, smla_decode_num_splits(T, H, topk, format, 0), smla_value_dims(format),
                                    bytes_out);
}

smla_status smla_attention(const void* q, int64_t T, int32_t H, int64_t q_stride_t, int64_t q_stride_h,
                           smla_kv_pool kv, const int32_t* indices, int32_t topk, int64_t idx_stride_t,
                           const int32_t* topk_length, const float* sink, float sm_scale, void* out,
                           int64_t out_stride_t, int64_t out_stride_h, float* lse, int64_t lse_stride_t,
                           void* workspace, size_t workspace_bytes, void* stream) {
  // both forms validate the same way before anything is chosen
  smla_status st = check_attn_common(q, T, H, q_stride_t, q_stride_h, kv, indices, topk, idx_stride_t);
  if (st != SMLA_OK) return st;
  if (T == 0) return ok();
  const int32_t dv = smla_value_dims(kv.format);
  st = check_out(out, out_stride_t, out_stride_h, H, lse, lse_stride_t, dv);
  if (st != SMLA_OK) return st;
  if (!std::isfinite(sm_scale)) return fail(SMLA_ERR_SHAPE, "sm_scale must be finite");
  if (workspace && !aligned(workspace, 16)) return fail(SMLA_ERR_STRIDE, "workspace is not 16-byte aligned");
  int32_t S = 0;
  if (workspace && smla_use_split_form(T, H, topk, kv.format, 0) == 1) {
    S = smla_decode_num_splits(T, H, topk, kv.format, 0);
    size_t need = 0;
    if (smla_decode_workspace_size(T, H, S, dv, &need) != SMLA_OK || need > workspace_bytes) S = 0;
  }
  if (S == 0)
    return smla_prefill(q, T, H, q_stride_t, q_stride_h, kv, indices, topk, idx_stride_t, topk_length, sink,
                        sm_scale, out, out_stride_t, out_stride_h, lse, lse_stride_t, stream);
  float* part_out = static_cast<float*>(workspace);
  float* part_lse = part_out + (size_t)T * (size_t)S * (size_t)H * (size_t)dv;
  st = smla_decode(q, T, H, q_stride_t, q_stride_h, kv, indices, topk, idx_stride_t, topk_length, sm_scale, S,
                   part_out, part_lse, stream);
  if (st != SMLA_OK) return st;
  return smla_combine(part_out, part_lse, T, S, H, dv, sink, out, out_stride_t, out_stride_h, lse, lse_stride_t,
                      stream);
}

// ---------------------------------------------------------------------------
// Measurement aids
// ---------------------------------------------------------------------------
smla_status smla_probe_gather(smla_kv_pool kv, const int32_t* indices, int64_t T, int32_t topk, int64_t idx_stride_t,
                              const int32_t* topk_length, uint32_t* rows_out, void* stream) {
  if (T < 0 || T > INT32_MAX) return fail(SMLA_ERR_SHAPE, "T = %lld must be in [0, 2^31-1]", (long long)T);
  if (T == 0) return ok();
  if (topk < 1) return fail(SMLA_ERR_SHAPE, "topk = %d must be >= 1", topk);
  if (!indices || !rows_out) return fail(SMLA_ERR_NULL, "indices or rows_out is NULL");
  smla_status st = check_pool(kv);
  if (st != SMLA_OK) return st;
  const int32_t rb = smla_row_bytes(kv.format);
  if (rb != 656 && rb != 1152)
    return fail(SMLA_ERR_UNSUPPORTED, "the gather probe takes 656- or 1152-byte rows, not %d-byte ones", rb);
  if (idx_stride_t < topk)
    return fail(SMLA_ERR_STRIDE, "idx_stride_t = %lld is smaller than topk = %d", (long long)idx_stride_t, topk);
  smla::GatherProbeParams p;
  p.pool = static_cast<const uint8_t*>(kv.base);
  p.block_stride = kv.block_stride_bytes;
  p.row_stride = kv.row_stride_bytes ? kv.row_stride_bytes : rb;
  p.nslots = kv.num_blocks * 64;
  p.idx = indices;
  p.idx_st = idx_stride_t;
  p.topk = topk;
  p.topk_length = topk_length;
  p.T = T;
  p.rows_out = rows_out;
  return launched(smla::launch_gather_probe(p, rb / 16, static_cast<hipStream_t>(stream)), "gather probe");
}

smla_status smla_probe_clock(uint64_t* out, int32_t blocks, int32_t iters, void* stream) {
  if (!out) return fail(SMLA_ERR_NULL, "out is NULL");
  if (blocks < 1 || blocks > 65536 || iters < 1)
    return fail(SMLA_ERR_SHAPE, "blocks = %d must be in [1, 65536] and iters = %d >= 1", blocks, iters);
  return launched(smla::launch_clock_probe(out, blocks, iters, static_cast<hipStream_t>(stream)), "clock probe");
}

smla_status smla_device_attributes(int32_t* attrs) {
  if (!attrs) return fail(SMLA_ERR_NULL, "attrs is NULL");
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(SMLA_ERR_HIP, "hipGetDevice failed: %s", hipGetErrorString(e));
  const hipDeviceAttribute_t which[5] = {hipDeviceAttributeMultiprocessorCount, hipDeviceAttributeClockRate,
                                         hipDeviceAttributeWallClockRate, hipDeviceAttributeMemoryClockRate,
                                         hipDeviceAttributeMemoryBusWidth};
  for (int i = 0; i < 5; ++i) {
    int v = 0;
    e = hipDeviceGetAttribute(&v, which[i], dev);
    if (e != hipSuccess) return fail(SMLA_ERR_HIP, "hipDeviceGetAttribute(%d) failed: %s", (int)which[i], hipGetErrorString(e));
    attrs[i] = v;
  }
  return ok();
}

// ---------------------------------------------------------------------------
// smla_attention_noalloc: smla_attention with its decode partials in a
// file-scope device array instead of a caller's workspace, for callers that
// cannot allocate.  One copy of the array per device, held until the process
// ends.  In host code `scratch` names a host-side stand-in, never the device
// array: its device address comes from hipGetSymbolAddress, once per device
// (on that device's first call), and only that address reaches the kernels.
// ---------------------------------------------------------------------------
static __device__ __align__(256) uint8_t scratch[SMLA_NOALLOC_SCRATCH_BYTES];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_dev[kMaxDevices] = {nullptr};

// the device address of the current device's scratch array
smla_status scratch_of_current_device(void** ptr_out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(SMLA_ERR_HIP, "hipGetDevice failed: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices)
    return fail(SMLA_ERR_UNSUPPORTED, "device %d is outside the %d devices the static scratch supports", dev,
                kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_dev[dev]) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !ptr)
      return fail(SMLA_ERR_HIP, "hipGetSymbolAddress(scratch) failed on device %d: %s", dev, hipGetErrorString(e));
    g_scratch_dev[dev] = ptr;
  }
  *ptr_out = g_scratch_dev[dev];
  return SMLA_OK;
}
}  // namespace

smla_status smla_attention_noalloc(const void* q, int64_t T, int32_t H, int64_t q_stride_t, int64_t q_stride_h,
                                   smla_kv_pool kv, const int32_t* indices, int32_t topk, int64_t idx_stride_t,
                                   const int32_t* topk_length, const float* sink, float sm_scale, void* out,
                                   int64_t out_stride_t, int64_t out_stride_h, float* lse, int64_t lse_stride_t,
                                   void* stream) {
  smla_status st = check_attn_common(q, T, H, q_stride_t, q_stride_h, kv, indices, topk, idx_stride_t);
  if (st != SMLA_OK) return st;
  if (T == 0) return ok();
  const int32_t dv = smla_value_dims(kv.format);
  st = check_out(out, out_stride_t, out_stride_h, H, lse, lse_stride_t, dv);
  if (st != SMLA_OK) return st;
  if (!std::isfinite(sm_scale)) return fail(SMLA_ERR_SHAPE, "sm_scale must be finite");
  if (smla_use_split_form(T, H, topk, kv.format, 0) != 1)
    return smla_prefill(q, T, H, q_stride_t, q_stride_h, kv, indices, topk, idx_stride_t, topk_length, sink,
                        sm_scale, out, out_stride_t, out_stride_h, lse, lse_stride_t, stream);
  const int32_t S = smla_decode_num_splits(T, H, topk, kv.format, 0);
  size_t need = 0;
  st = smla_decode_workspace_size(T, H, S, dv, &need);
  if (st != SMLA_OK) return st;
  if (need > (size_t)SMLA_NOALLOC_SCRATCH_BYTES)
    return fail(SMLA_ERR_UNSUPPORTED,
                "the split form chosen for T=%lld, H=%d, topk=%d (%d splits) needs %zu bytes of partials; the static "
                "scratch holds %zu: call smla_attention with a workspace",
                (long long)T, H, topk, S, need, (size_t)SMLA_NOALLOC_SCRATCH_BYTES);
  void* base = nullptr;
  st = scratch_of_current_device(&base);
  if (st != SMLA_OK) return st;
  // every partial and LSE of the T x S x H block is written by the decode
  // launch (empty splits included), so nothing needs clearing first
  float* part_out = static_cast<float*>(base);
  float* part_lse = part_out + (size_t)T * (size_t)S * (size_t)H * (size_t)dv;
  st = smla_decode(q, T, H, q_stride_t, q_stride_h, kv, indices, topk, idx_stride_t, topk_length, sm_scale, S,
                   part_out, part_lse, stream);
  if (st != SMLA_OK) return st;
  return smla_combine(part_out, part_lse, T, S, H, dv, sink, out, out_stride_t, out_stride_h, lse, lse_stride_t,
                      stream);
}
