// launch.h -- kernel parameter blocks and host launchers behind the C ABI.
// Everything here is called only after the C entry points have validated
// their arguments (see api.cpp).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace smla {

struct QuantParams {
  const uint16_t* kv;   // bf16 [n, kv_stride]
  int64_t n;
  int64_t kv_stride;    // elements
  const int32_t* slots; // [n]
  uint8_t* pool;
  int64_t nslots;       // num_blocks * 64
  int64_t block_stride; // bytes
  int64_t row_stride;   // bytes between the rows of a block
};

struct AttnParams {
  const uint16_t* q;    // bf16
  int64_t q_st, q_sh;   // elements
  int64_t T;
  int32_t H;
  const uint8_t* pool;
  int64_t block_stride; // bytes
  int64_t row_stride;   // bytes between the rows of a block
  int64_t nslots;
  const int32_t* idx;
  int64_t idx_st;       // elements
  int32_t topk;
  const int32_t* topk_length;  // may be null
  const float* sink;           // may be null (prefill only)
  float scale_log2;            // sm_scale * log2(e)
  int32_t nope;                // rows have no rope dimensions: q rows hold 512 values and row
                               // bytes [528, 656) are padding, never gathered or read
  // prefill outputs
  uint16_t* out;
  int64_t out_st, out_sh;
  float* lse;
  int64_t lse_st;
  // decode outputs
  float* part_out;      // [T, S, H, d_v]
  float* part_lse;      // [T, S, H]
  int32_t num_splits;
  int32_t split_w;
  int32_t splits_per_block;  // decode: consecutive splits one workgroup runs (FP8 many-head kernel)
  // secondary candidate list (list positions [topk, topk + topk2)) over a
  // second pool of the same format; topk2 = 0: none
  const uint8_t* pool2;
  int64_t block_stride2, row_stride2, nslots2;
  const int32_t* idx2;
  int64_t idx_st2;
  int32_t topk2;
  const int32_t* topk_length2;  // may be null
};

struct CombineParams {
  const float* part_out;
  const float* part_lse;
  int64_t T;
  int32_t S, H;
  int32_t dv;           // values per part_out and out row: 512, or 1024 (DOTS3_SWA)
  const float* sink;
  uint16_t* out;
  int64_t out_st, out_sh;
  float* lse;
  int64_t lse_st;
};

// the gather probe (a measurement aid): rows of a candidate list moved into
// LDS with nothing computed on them
struct GatherProbeParams {
  const uint8_t* pool;
  int64_t block_stride, row_stride, nslots;
  const int32_t* idx;
  int64_t idx_st;
  int32_t topk;
  const int32_t* topk_length;  // may be null
  int64_t T;
  uint32_t* rows_out;          // [T]
};

hipError_t launch_quantize(const QuantParams& p, int fmt, hipStream_t s);
hipError_t launch_gather_probe(const GatherProbeParams& p, int chunks, hipStream_t s);
hipError_t launch_clock_probe(uint64_t* out, int blocks, int iters, hipStream_t s);
hipError_t launch_attention(const AttnParams& p, int fmt, bool decode, hipStream_t s);
hipError_t launch_attention_fp8(const AttnParams& p, int fmt, bool decode, hipStream_t s);
hipError_t launch_attention_mx(const AttnParams& p, int fmt, bool decode, hipStream_t s);
// the kernel whose waves split QK over candidates and PV over value columns
// (two workgroups per CU): BF16 rows at any head count, and the 656-byte
// quantized rows (FP8 with any scales, with or without rope, INT8) with 16
// or fewer heads
hipError_t launch_attention_bf16(const AttnParams& p, int fmt, bool decode, hipStream_t s);
hipError_t launch_combine(const CombineParams& p, hipStream_t s);

// compute units of the current device (256 when it cannot be queried)
int device_compute_units();
// consecutive decode splits one workgroup of the FP8 many-head kernel runs:
// about one workgroup per compute unit when (token, split) pairs outnumber
// the units
int fp8_splits_per_block(int64_t T, int32_t H, int32_t num_splits, int compute_units);
// prefill workgroups per head block of the FP8 many-head kernel: each runs
// tokens blockIdx.x, blockIdx.x + gridDim.x, ... (at most one per compute unit)
int fp8_prefill_blocks(int64_t T, int32_t H, int compute_units);

}  // namespace smla
