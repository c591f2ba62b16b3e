// quantize.hip -- cache writer: BF16 latent rows -> pool rows.
//
// Row layout from the FlashInfer PR #4802 review of the DSv3.2 decode kernel:
// 512 e4m3 codes, four FP32 per-128 scales, 64 BF16 rope values (656 bytes);
// the page states DSv3.2 stores power-of-two scales.  INT8 rows reuse the
// layout with int8 codes and amax/127 scales; BF16 rows are a copy.
//
// One wave per row.  Lane l owns nope elements [8l, 8l+8): the 16 lanes of
// a lane group cover one 128-element scale tile, so the tile amax is a
// 16-lane max.  All scale and code arithmetic is IEEE float32 (correctly
// rounded division), which is what fixes the integer codes.
#include "device_common.h"
#include "launch.h"

namespace smla {

// Nearest E4M3 code to a float32 y with |y| <= 448 (larger magnitudes
// saturate to 448), ties to the even mantissa, sign kept.  Works on the
// float32 bit pattern.
__device__ __forceinline__ uint32_t e4m3_from_f32(float y) {
  uint32_t u = __builtin_bit_cast(uint32_t, y);
  uint32_t sign = (u >> 24) & 0x80u;
  uint32_t a = u & 0x7FFFFFFFu;
  if (a >= 0x43E00000u) return sign | 0x7Eu;          // >= 448 (and inf/nan)
  if (a < 0x3C800000u) {                              // < 2^-6: quantum 2^-9
    float t = __builtin_bit_cast(float, a) * 512.0f;  // exact scaling
    uint32_t m = (uint32_t)__builtin_rintf(t);        // 0..8, ties to even
    return sign | m;                                  // 8 -> 0x08 = 2^-6
  }
  int32_t e = (int32_t)(a >> 23) - 127;               // -6..8
  uint32_t mant = a & 0x7FFFFFu;
  uint32_t keep = mant >> 20, rest = mant & 0xFFFFFu;
  if (rest > 0x80000u || (rest == 0x80000u && (keep & 1u))) keep += 1;
  if (keep == 8u) { keep = 0; e += 1; }
  uint32_t code = (uint32_t)((e + 7) << 3) | keep;
  if (code > 0x7Eu) code = 0x7Eu;
  return sign | code;
}

// e with 2^e = 2^ceil(log2(amax/448)), from the bits of r = amax / 448
// (float32, amax > 0).
__device__ __forceinline__ int fp8_scale_exponent(float amax) {
  float r = __fdiv_rn(amax, 448.0f);
  uint32_t rb = __builtin_bit_cast(uint32_t, r);
  if (rb >= 0x00800000u) return (int)(rb >> 23) - 127 + ((rb & 0x7FFFFFu) != 0u);
  return (32 - __clz((int)(rb - 1u))) - 149;  // subnormal r = rb * 2^-149
}

// 2^max(ceil(log2(amax/448)), -126), a normal float32 power of two; 1 when
// amax = 0.
__device__ __forceinline__ float fp8_tile_scale(float amax) {
  if (amax == 0.0f) return 1.0f;
  int e = fp8_scale_exponent(amax);
  e = e < -126 ? -126 : e;
  return __builtin_bit_cast(float, (uint32_t)(e + 127) << 23);
}

template <int FMT>
__global__ __launch_bounds__(256) void quantize_kernel(QuantParams p) {
  using G = RowGeom<FMT>;
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= p.n) return;
  const int64_t slot = p.slots[row];
  if (slot < 0 || slot >= p.nslots) return;
  const uint16_t* src = p.kv + row * p.kv_stride;
  uint8_t* dst = p.pool + (slot / PAGE) * p.block_stride + (slot % PAGE) * p.row_stride;

  if constexpr (FMT == FMT_BF16) {
    const uint4* s4 = reinterpret_cast<const uint4*>(src);
    uint4* d4 = reinterpret_cast<uint4*>(dst);
    d4[lane] = s4[lane];
    if (lane < G::CHUNKS - 64) d4[64 + lane] = s4[64 + lane];
    return;
  } else {
    const uint4 raw = reinterpret_cast<const uint4*>(src)[lane];  // 8 bf16
    float x[8];
    uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      x[2 * i] = __builtin_bit_cast(float, w[i] << 16);
      x[2 * i + 1] = __builtin_bit_cast(float, w[i] & 0xFFFF0000u);
    }
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(x[i]));
#pragma unroll
    for (int o = 1; o < 16; o <<= 1) amax = fmaxf(amax, __shfl_xor(amax, o));

    uint32_t code[8];
    float scale;
    if constexpr (FMT == FMT_FP8 || FMT == FMT_FP8_ANY || FMT == FMT_FP8_NOPE) {
      scale = FMT != FMT_FP8_ANY ? fp8_tile_scale(amax) : (amax == 0.0f ? 1.0f : __fdiv_rn(amax, 448.0f));
#pragma unroll
      for (int i = 0; i < 8; ++i) code[i] = e4m3_from_f32(__fdiv_rn(x[i], scale));
    } else {
      scale = (amax == 0.0f) ? 1.0f : __fdiv_rn(amax, 127.0f);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        float qv = __builtin_rintf(__fdiv_rn(x[i], scale));
        qv = fminf(fmaxf(qv, -127.0f), 127.0f);
        code[i] = (uint32_t)(int32_t)qv & 0xFFu;
      }
    }
    uint2 packed;
    packed.x = code[0] | (code[1] << 8) | (code[2] << 16) | (code[3] << 24);
    packed.y = code[4] | (code[5] << 8) | (code[6] << 16) | (code[7] << 24);
    reinterpret_cast<uint2*>(dst)[lane] = packed;
    if ((lane & 15) == 0) reinterpret_cast<float*>(dst + G::SCALE_OFF)[lane >> 4] = scale;
    if (FMT != FMT_FP8_NOPE && lane < 16) {  // (NOPE rows: padding, not written)
      const uint2* rs = reinterpret_cast<const uint2*>(src + D_NOPE);
      reinterpret_cast<uint2*>(dst + G::ROPE_OFF)[lane] = rs[lane];
    }
  }
}

// Rows with exponent-byte scales (DOTS3_SWA: 1024 codes in 128-element
// tiles; DSv4: 448 codes in 64-element tiles): the same power-of-two scale
// as the FP8 rows, with its exponent raised to at least -126 and stored as
// one byte (e + 127) in the row's tail; DSv4's pad byte is written as 0.
// One wave per row; lane l owns nope elements [EPL*l, EPL*l + EPL), so the
// 8 lanes of an aligned group cover one tile.  Rows are 8-byte aligned.
template <int NOPE, int EPL, int ROPE_OFF, int SCALE_OFF>
__global__ __launch_bounds__(256) void quantize_mx_kernel(QuantParams p) {
  constexpr int LANES = NOPE / EPL;  // lanes holding nope elements
  constexpr int NG = LANES / 8;      // scale tiles
  static_assert(NOPE % EPL == 0 && LANES % 8 == 0 && LANES <= 64 && EPL % 8 == 0 && NG <= 8, "row geometry");
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= p.n) return;
  const int64_t slot = p.slots[row];
  if (slot < 0 || slot >= p.nslots) return;
  const uint16_t* src = p.kv + row * p.kv_stride;
  uint8_t* dst = p.pool + (slot / PAGE) * p.block_stride + (slot % PAGE) * p.row_stride;
  const bool active = lane < LANES;

  float x[EPL];
#pragma unroll
  for (int c = 0; c < EPL / 8; ++c) {
    const uint4 r = active ? reinterpret_cast<const uint4*>(src + EPL * lane)[c] : make_uint4(0, 0, 0, 0);
    const uint32_t w[4] = {r.x, r.y, r.z, r.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      x[8 * c + 2 * i] = __builtin_bit_cast(float, w[i] << 16);
      x[8 * c + 2 * i + 1] = __builtin_bit_cast(float, w[i] & 0xFFFF0000u);
    }
  }
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < EPL; ++i) amax = fmaxf(amax, fabsf(x[i]));
#pragma unroll
  for (int o = 1; o < 8; o <<= 1) amax = fmaxf(amax, __shfl_xor(amax, o));
  int e = amax == 0.0f ? 0 : fp8_scale_exponent(amax);
  e = e < -126 ? -126 : e;
  const float scale = __builtin_bit_cast(float, (uint32_t)(e + 127) << 23);
  if (active) {
#pragma unroll
    for (int c = 0; c < EPL / 8; ++c) {
      uint32_t code[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) code[i] = e4m3_from_f32(__fdiv_rn(x[8 * c + i], scale));
      const uint2 pk = make_uint2(code[0] | (code[1] << 8) | (code[2] << 16) | (code[3] << 24),
                                  code[4] | (code[5] << 8) | (code[6] << 16) | (code[7] << 24));
      reinterpret_cast<uint2*>(dst + EPL * lane)[c] = pk;
    }
  }
  if (lane < 16) {  // 64 rope values, 4 per lane
    const uint2* rs = reinterpret_cast<const uint2*>(src + NOPE) + lane;
    reinterpret_cast<uint2*>(dst + ROPE_OFF)[lane] = *rs;
  }
  // the scale bytes (and zero padding up to 8 bytes), from the first lane
  // of each tile, in one store
  const uint32_t b = (uint32_t)(e + 127);
  uint32_t lo = 0, hi = 0;
#pragma unroll
  for (int g = 0; g < 4; ++g) {
    const uint32_t b0 = (uint32_t)__shfl((int)b, 8 * g), b1 = (uint32_t)__shfl((int)b, 8 * (g + 4));
    lo |= (g < NG ? b0 : 0u) << (8 * g);
    hi |= (g + 4 < NG ? b1 : 0u) << (8 * g);
  }
  if (lane == 0) *reinterpret_cast<uint2*>(dst + SCALE_OFF) = make_uint2(lo, hi);
}

hipError_t launch_quantize(const QuantParams& p, int fmt, hipStream_t s) {
  dim3 grid((unsigned)((p.n + 3) / 4)), block(256);
  switch (fmt) {
    case FMT_BF16: hipLaunchKernelGGL(quantize_kernel<FMT_BF16>, grid, block, 0, s, p); break;
    case FMT_FP8: hipLaunchKernelGGL(quantize_kernel<FMT_FP8>, grid, block, 0, s, p); break;
    case FMT_INT8: hipLaunchKernelGGL(quantize_kernel<FMT_INT8>, grid, block, 0, s, p); break;
    case FMT_FP8_ANY: hipLaunchKernelGGL(quantize_kernel<FMT_FP8_ANY>, grid, block, 0, s, p); break;
    case FMT_FP8_NOPE: hipLaunchKernelGGL(quantize_kernel<FMT_FP8_NOPE>, grid, block, 0, s, p); break;
    case FMT_FP8_DOTS3:
      hipLaunchKernelGGL((quantize_mx_kernel<dots3::D_NOPE, 16, dots3::ROPE_OFF, dots3::SCALE_OFF>), grid, block, 0, s, p);
      break;
    case FMT_FP8_DSV4:
      hipLaunchKernelGGL((quantize_mx_kernel<dsv4::D_NOPE, 8, dsv4::ROPE_OFF, dsv4::SCALE_OFF>), grid, block, 0, s, p);
      break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace smla
