// split_model.cpp -- the decode split count and the choice between the split
// form (decode + combine) and the prefill form, from a cost model fitted on
// MI355X.
//
// FlashInfer PR #4802 ("cpb model" and "Crossover" in its description)
// replaces a per-shape tuning sweep with a closed form over a few hardware
// constants, fitted once per device from timings over an HBM-sized pool,
// and routes small-T prefill to the split form when that form is predicted
// at most 0.95x the prefill time.  Here the terms follow this library's
// launch geometry:
//   decode  = waves * (a + b * tiles_per_block + f * splits_per_block) + w * MB
//   combine = c0 + c1 * MB + c2 * T * H / 1000
//   prefill = ap0 + waves_p * (ap + bp * tiles_per_token)
// with MB the partial buffers (T * S * H * (4 d_v + 4) bytes), waves the
// rounds of workgroups over the compute units (one workgroup per CU per
// round: the many-head kernels fill a CU's LDS; two for the column-split
// kernel (16 or fewer heads, and BF16 rows at any head count) and the
// exponent-byte kernel's DSv4 instantiation), and a, b, f, ap0, ap, bp per
// kernel class.  The constants were fitted by
// sparse_top_mla_smla_amd/calibrate_splits.py on one MI355X (256 CUs) over
// 324 decode shapes and their prefill counterparts; there the pick is on
// average 0.5% and at most 12% slower than the best measured split count.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdint>

#include "launch.h"
#include "smla.h"

namespace smla {
namespace {

struct KernelClass {
  double a, b, f;  // decode: per block, per tile of the longest block, per split it finishes (us)
  double ap0, ap, bp;  // prefill: per launch, per round of blocks, per tile of a round (us)
  int heads_per_block;
  bool grouped;    // consecutive splits per workgroup (the FP8 many-head kernel)
  int occupancy;   // workgroups per CU in one round
};

// fitted constants (microseconds), MI355X
constexpr KernelClass kFp8Wide{14.09, 2.993, 1.554, 2.596, 10.08, 3.211, 64, true, 1};
constexpr KernelClass kInt8Wide{14.71, 4.805, 0.1746, 2.036, 10.82, 4.751, 64, true, 1};
constexpr KernelClass kBf16Cols{1.982, 3.671, 1.982, 0.0, 10.47, 3.488, 16, false, 2};
constexpr KernelClass kFp8Cols{3.377, 3.673, 3.377, 0.0, 12.60, 3.767, 16, false, 2};
constexpr KernelClass kInt8Cols{3.249, 4.358, 3.249, 0.0, 11.74, 4.483, 16, false, 2};
constexpr KernelClass kDots3Mx{3.851, 6.568, 3.851, 0.0, 14.10, 6.380, 16, false, 1};
constexpr KernelClass kDots3Mx32{2.827, 7.815, 2.827, 1.264, 12.92, 7.461, 32, false, 1};
constexpr KernelClass kDsv4Mx{3.134, 4.672, 3.134, 0, 13.51, 4.609, 16, false, 2};
constexpr KernelClass kDsv4Wide{16.36, 3.857, 0, 9.336, 9.113, 3.969, 64, true, 1};
constexpr double kWriteUsPerMB = 0.186;  // decode's partial stores
constexpr double kComb0 = 10.57, kComb1 = 0.1856, kComb2 = 0.0;
constexpr double kCrossover = 0.95;  // split form only when at most this fraction of prefill

const KernelClass* kernel_class(int32_t format, int32_t H) {
  // the dispatch rule of launch_attention
  switch (format) {
    case SMLA_KV_FP8_E4M3:
    case SMLA_KV_FP8_E4M3_NOPE: return H > 16 ? &kFp8Wide : &kFp8Cols;
    case SMLA_KV_INT8: return H > 16 ? &kInt8Wide : &kInt8Cols;
    // arbitrary-scale FP8 rows convert and scale like INT8 rows (their
    // conversion is cheaper: the INT8 constants bound it)
    case SMLA_KV_FP8_E4M3_ANY_SCALE: return H > 16 ? &kInt8Wide : &kInt8Cols;
    case SMLA_KV_BF16: return &kBf16Cols;
    // DOTS3_SWA rows: the exponent-byte kernels at any H; DSv4 rows: the
    // exponent-byte kernel up to 16 heads, the many-head kernel above
    case SMLA_KV_FP8_E4M3_DOTS3: return H > 16 ? &kDots3Mx32 : &kDots3Mx;
    case SMLA_KV_FP8_E4M3_DSV4: return H > 16 ? &kDsv4Wide : &kDsv4Mx;
    default: return nullptr;
  }
}

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

double split_cost(const KernelClass& c, int64_t T, int32_t H, int32_t topk, int32_t S, int cus, int32_t dv) {
  const int64_t hb = ceil_div(H, c.heads_per_block);
  const int64_t w = smla_split_width(topk, S);
  const int64_t spb = c.grouped ? fp8_splits_per_block(T, H, S, cus) : 1;
  const int64_t blocks = T * hb * ceil_div(S, spb);
  const double waves = (double)ceil_div(blocks, (int64_t)cus * c.occupancy);
  const double tiles = (double)ceil_div(std::min<int64_t>(spb * w, topk), 64);
  const double mb = (double)T * S * H * (4.0 * dv + 4.0) / 1e6;
  const double decode = waves * (c.a + c.b * tiles + c.f * (double)spb) + kWriteUsPerMB * mb;
  const double combine = kComb0 + kComb1 * mb + kComb2 * (double)T * H / 1000.0;
  return decode + combine;
}

double prefill_cost(const KernelClass& c, int64_t T, int32_t H, int32_t topk, int cus) {
  const double waves = (double)ceil_div(T * ceil_div(H, c.heads_per_block), (int64_t)cus * c.occupancy);
  return c.ap0 + waves * (c.ap + c.bp * (double)ceil_div(topk, 64));
}

int max_splits(int32_t topk) { return (int)std::min<int64_t>(64, ceil_div(topk, 64)); }

bool valid(int64_t T, int32_t H, int32_t topk, int32_t format) {
  return T >= 1 && T <= INT32_MAX && H >= 1 && H <= 128 && topk >= 1 && kernel_class(format, H) != nullptr;
}

int resolve_cus(int32_t compute_units) { return compute_units > 0 ? compute_units : device_compute_units(); }

int best_splits(const KernelClass& c, int64_t T, int32_t H, int32_t topk, int cus, int32_t dv, double* cost) {
  int best = 1;
  double best_cost = split_cost(c, T, H, topk, 1, cus, dv);
  for (int S = 2; S <= max_splits(topk); ++S) {
    const double v = split_cost(c, T, H, topk, S, cus, dv);
    if (v < best_cost) {  // ties keep the smaller split count
      best = S;
      best_cost = v;
    }
  }
  if (cost) *cost = best_cost;
  return best;
}

}  // namespace
}  // namespace smla

extern "C" {

double smla_split_model_cost(int64_t T, int32_t H, int32_t topk, int32_t format, int32_t num_splits,
                             int32_t compute_units) {
  if (!smla::valid(T, H, topk, format) || num_splits < 0 || num_splits > 64) return -1.0;
  const smla::KernelClass& c = *smla::kernel_class(format, H);
  const int cus = smla::resolve_cus(compute_units);
  return num_splits == 0 ? smla::prefill_cost(c, T, H, topk, cus)
                         : smla::split_cost(c, T, H, topk, num_splits, cus, smla_value_dims(format));
}

int32_t smla_decode_num_splits(int64_t T, int32_t H, int32_t topk, int32_t format, int32_t compute_units) {
  if (!smla::valid(T, H, topk, format)) return -1;
  return smla::best_splits(*smla::kernel_class(format, H), T, H, topk, smla::resolve_cus(compute_units),
                           smla_value_dims(format), nullptr);
}

int32_t smla_use_split_form(int64_t T, int32_t H, int32_t topk, int32_t format, int32_t compute_units) {
  if (!smla::valid(T, H, topk, format)) return -1;
  const smla::KernelClass& c = *smla::kernel_class(format, H);
  const int cus = smla::resolve_cus(compute_units);
  double split = 0.0;
  smla::best_splits(c, T, H, topk, cus, smla_value_dims(format), &split);
  return split <= smla::kCrossover * smla::prefill_cost(c, T, H, topk, cus) ? 1 : 0;
}

}  // extern "C"
