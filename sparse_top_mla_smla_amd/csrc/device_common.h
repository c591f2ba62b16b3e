// device_common.h -- gfx950 device helpers shared by the smla kernels:
// vector types, MFMA wrappers, FP8/INT8 -> BF16 converters and the cache
// row geometry.  Lane layouts used below were checked on gfx950:
//  * v_mfma_f32_16x16x32_bf16: lane l holds A[m = l%16][k = 8(l/16)+i] and
//    B[k = 8(l/16)+i][n = l%16] (i < 8); D[m = 4(l/16)+i][n = l%16] (i < 4).
//  * v_mfma_f32_16x16x16_bf16: same with k = 4(l/16)+i (i < 4).
//  * ds_read_b64_tr_b16: within each 16-lane group, lane 4r+b supplies the
//    address of row r, columns 4b..4b+3 of a 4x16 block of 16-bit values and
//    receives column (lane%16) of rows 0..3.
//  * ds_read_b64_tr_b8: lane 2r+b supplies row r, byte columns 8b..8b+7 of
//    an 8x16 byte block and receives byte column (lane%16) of rows 0..7.
//  * v_cvt_pk_f32_fp8 decodes OCP E4M3 exactly.
//  * v_permlane32_swap_b32 (vdst, vsrc): vdst's lanes 32..63 and vsrc's
//    lanes 0..31 trade places.  The builtin returns both registers; with
//    this compiler, __builtin_bit_cast applied in place to the second
//    element of that result yields the first, so copy both elements to
//    scalars before any cast.
//  * v_cvt_scalef32_pk_f16_fp8, v_cvt_pk_f16_f32 and the FP16 MFMAs keep
//    FP16 subnormals.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace smla {

constexpr int D_NOPE = 512;
constexpr int D_ROPE = 64;
constexpr int D_QK = 576;
constexpr int D_V = 512;
constexpr int PAGE = 64;
constexpr int QTILE = 128;  // quantization tile along the nope part

// FMT_FP8_ANY: FP8 codes with arbitrary positive per-128 scales (the row of FMT_FP8)
// FMT_FP8_NOPE: the FP8 row whose rope bytes are padding (no rope dimensions)
// FMT_FP8_DOTS3: 1160-byte rows of 1024 e4m3 codes, 64 BF16 rope values and
//   eight power-of-two exponent bytes (its own kernels, attention_mx.hip)
// FMT_FP8_DSV4: 584-byte rows of 448 e4m3 codes, 64 BF16 rope values, seven
//   exponent bytes and a pad byte (attention_mx.hip)
enum : int {
  FMT_BF16 = 0, FMT_FP8 = 1, FMT_INT8 = 2, FMT_FP8_ANY = 3, FMT_FP8_NOPE = 4, FMT_FP8_DOTS3 = 5, FMT_FP8_DSV4 = 6
};

// DOTS3_SWA row geometry: [0,1024) codes, [1024,1152) rope, [1152,1160) scale bytes
namespace dots3 {
constexpr int D_NOPE = 1024;
constexpr int D_QK = 1088;
constexpr int D_V = 1024;
constexpr int ROW_BYTES = 1160;
constexpr int ROPE_OFF = 1024;
constexpr int SCALE_OFF = 1152;
constexpr int NGROUPS = 8;  // 128-element scale tiles
}  // namespace dots3

// DSv4 row geometry: [0,448) codes, [448,576) rope, [576,583) scale bytes, [583] pad
namespace dsv4 {
constexpr int D_NOPE = 448;
constexpr int D_QK = 512;
constexpr int D_V = 512;
constexpr int ROW_BYTES = 584;
constexpr int ROPE_OFF = 448;
constexpr int SCALE_OFF = 576;
constexpr int NGROUPS = 7;  // 64-element scale tiles
}  // namespace dsv4

template <int FMT>
struct RowGeom {
  // bytes of one cache row and its sections
  static constexpr int BYTES = (FMT == FMT_BF16) ? 2 * D_QK : D_NOPE + 16 + 2 * D_ROPE;
  static constexpr int SCALE_OFF = D_NOPE;        // FP8/INT8: 4 x fp32
  static constexpr int ROPE_OFF = (FMT == FMT_BF16) ? 2 * D_NOPE : D_NOPE + 16;
  static constexpr int CHUNKS = BYTES / 16;       // 16-byte pieces per row
};

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef int i32x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));

__device__ __forceinline__ f32x4 mfma_16x16x32(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma_16x16x32_f16(f16x8 a, f16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma_16x16x16(i16x4 a, i16x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
}

// two floats -> packed BF16 pair (round to nearest even)
__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
  bf16x2 v;
  v[0] = (__bf16)lo;
  v[1] = (__bf16)hi;
  return __builtin_bit_cast(uint32_t, v);
}

// two floats -> packed FP16 pair (round to nearest even; subnormals kept)
__device__ __forceinline__ uint32_t pack_f16(float lo, float hi) {
  f16x2 v;
  v[0] = (_Float16)lo;
  v[1] = (_Float16)hi;
  return __builtin_bit_cast(uint32_t, v);
}

// two BF16 values (x's halves) as an FP16 pair: exact for magnitudes in
// [2^-14, 65504], rounded to FP16's subnormal grid below
__device__ __forceinline__ uint32_t bf16x2_to_f16x2(uint32_t x) {
  return pack_f16(__builtin_bit_cast(float, x << 16), __builtin_bit_cast(float, x & 0xFFFF0000u));
}

// four e4m3 codes (one dword) times a power-of-two scale as four FP16
// values: exact, subnormal results included, while 448 x scale stays below
// 65504 and the smallest code (2^-9) times the scale is at least 2^-24
__device__ __forceinline__ uint2 fp8x4_to_f16x4(uint32_t v, float scale) {
  return make_uint2(__builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(v, scale, false)),
                    __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(v, scale, true)));
}

// PV over quantized codes runs in FP16: P' = P x scale rounded once to FP16
// has 11 significant bits against BF16's 8.  FP16's range is held by a
// power-of-two bias per tile: with e the largest biased exponent of the
// tile's scales (so every scale is below 2^(e-126); an exponent byte is the
// scale's biased exponent), P' = P x scale x 2^-B with B = e - 133 (at
// least -15), so P' < 2^8 x 2^7 (P <= 2^8 under a lazy running max that
// moves when exceeded by 2^8), and V^T = codes x 2^b with b = min(B, bmax),
// so the codes times 2^b are exact FP16 values (e4m3 codes, 2^-9 .. 448:
// bmax = 7; int8 codes, whose conversion also needs -1152 x 2^b in FP16:
// bmax = 5).  The rest of 2^-B, 2^-k with k = B - b, is nonzero only for
// scales of 2^14 (int8: 2^11) and above (values beyond 7.3e6): the
// kernels take P relative to 2^(running max + k), which moves P, O and the
// row sum into units of 2^-k together, like a move of the running max
// (exactly: by a power of two), and add k back to the max for the LSE.
// P' = P x scale x 2^-b then stays below 2^15 in every case.
struct F16Bias {
  float v;  // 2^b, for the codes
  float p;  // 2^-b, for P'
  float B;  // b + k
  int k;    // 0 below scales of 2^14 (int8: 2^11)
};
__device__ __forceinline__ float exp2i(int n) {  // 2^n for -126 <= n <= 127
  return __builtin_bit_cast(float, (uint32_t)(127 + n) << 23);
}
__device__ __forceinline__ F16Bias f16_bias(uint32_t e, int bmax = 7) {
  const int B = max((int)e - 133, -15);
  const int b = min(B, bmax);
  return F16Bias{exp2i(b), exp2i(-b), (float)B, B - b};
}

// four int8 codes (one dword) times 2^b as four FP16 values, exactly: the
// biased byte x + 128 placed in the mantissa of 1024 gives 1024 + x + 128,
// and one fused multiply-add per pair gives (1024 + x + 128 - 1152) x 2^b
// (sb: 2^b in both halves, ob: -1152 x 2^b in both halves)
__device__ __forceinline__ uint2 int8x4_to_f16x4(uint32_t v, f16x2 sb, f16x2 ob) {
  const uint32_t u = v ^ 0x80808080u;
  const uint32_t lo = __builtin_amdgcn_perm(0x64646464u, u, 0x04010400u);  // halves 0x64u0, 0x64u1
  const uint32_t hi = __builtin_amdgcn_perm(0x64646464u, u, 0x04030402u);  // halves 0x64u2, 0x64u3
  const f16x2 a = __builtin_elementwise_fma(__builtin_bit_cast(f16x2, lo), sb, ob);
  const f16x2 b = __builtin_elementwise_fma(__builtin_bit_cast(f16x2, hi), sb, ob);
  return make_uint2(__builtin_bit_cast(uint32_t, a), __builtin_bit_cast(uint32_t, b));
}

// the largest value of v over the 64 lanes, in every lane (DPP within each
// 16-lane row, then the four row maxima); every lane of the wave must call it
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0xB1, 0xF, 0xF, false));   // lanes i ^ 1
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x4E, 0xF, 0xF, false));   // lanes i ^ 2
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x141, 0xF, 0xF, false));  // 7 - i within 8
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x140, 0xF, 0xF, false));  // 15 - i within 16
  const uint32_t a = max((uint32_t)__builtin_amdgcn_readlane((int)v, 0), (uint32_t)__builtin_amdgcn_readlane((int)v, 16));
  const uint32_t b = max((uint32_t)__builtin_amdgcn_readlane((int)v, 32), (uint32_t)__builtin_amdgcn_readlane((int)v, 48));
  return max(a, b);
}

// the largest of the low n bytes of the 8-byte word (x, y)
template <int N>
__device__ __forceinline__ uint32_t max_byte(uint32_t x, uint32_t y) {
  uint32_t m = 0;
#pragma unroll
  for (int i = 0; i < N; ++i) m = max(m, ((i < 4 ? x : y) >> (8 * (i & 3))) & 0xFFu);
  return m;
}

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __builtin_bit_cast(float, (uint32_t)b << 16);
}

// four E4M3 codes (one dword) -> four BF16 values (exact)
__device__ __forceinline__ uint2 fp8x4_to_bf16x4(uint32_t v) {
  f32x2 lo = __builtin_amdgcn_cvt_pk_f32_fp8(v, false);
  f32x2 hi = __builtin_amdgcn_cvt_pk_f32_fp8(v, true);
  return make_uint2(pack_bf16(lo[0], lo[1]), pack_bf16(hi[0], hi[1]));
}

// four int8 codes (one dword) -> four BF16 values (exact: |code| <= 127)
__device__ __forceinline__ uint2 int8x4_to_bf16x4(uint32_t v) {
  float a = (float)(int8_t)(v & 0xFF);
  float b = (float)(int8_t)((v >> 8) & 0xFF);
  float c = (float)(int8_t)((v >> 16) & 0xFF);
  float d = (float)(int8_t)(v >> 24);
  return make_uint2(pack_bf16(a, b), pack_bf16(c, d));
}

template <int FMT>
__device__ __forceinline__ uint2 codes4_to_bf16x4(uint32_t v) {
  if constexpr (FMT == FMT_FP8 || FMT == FMT_FP8_NOPE) return fp8x4_to_bf16x4(v);
  else return int8x4_to_bf16x4(v);
}

__device__ __forceinline__ i32x2 lds_read_tr8(const void* p) {
  return __builtin_amdgcn_ds_read_tr8_b64_v2i32((__attribute__((address_space(3))) i32x2*)(p));
}
__device__ __forceinline__ i16x4 lds_read_tr16(const void* p) {
  typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
  bf16x4 r = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((__attribute__((address_space(3))) bf16x4*)(p));
  return __builtin_bit_cast(i16x4, r);
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

constexpr float LOG2E = 1.4426950408889634f;
constexpr float LN2 = 0.6931471805599453f;

}  // namespace smla
