// attention_wide.hip -- sparse MLA attention for many heads (H > 16) over
// the INT8 paged latent cache, and over FP8 rows with arbitrary scales
// (GLM_NSA rows), prefill form and split-KV decode partials.
//
// What is computed is stated in include/smla.h.  These rows carry arbitrary
// FP32 scales (amax/127, amax/448), so code * scale is not exact in BF16:
// the codes are converted exactly and the scales are applied to FP32
// partial scores and folded into P.  (The FP8 cache with power-of-two
// scales has its own kernel that dequantizes while converting.)  One workgroup owns
// one token (and split) for 64 heads, so every selected row is gathered
// from the pool once per token, not once per head group.
//
// All products use v_mfma_f32_32x32x16_bf16 (full matrix rate on gfx950).
// Eight waves (two per SIMD); wave w = g + 4hh works on latent group g and
// head half hh.  Per 64-candidate tile:
//  1. QK^T, split over the latent dimension: wave (g, hh) multiplies the
//     tile's K rows restricted to nope columns [128g, 128g+128) -- exactly
//     one 128-wide scale tile -- by its slice of Q (kept in registers for
//     the whole token).  Result: unscaled partial S^T, 64 candidates x 32
//     heads.
//  2. Reduce-scatter of the partials through LDS: four owner waves (one
//     per SIMD) each own a 32x32 score tile, receive the other three
//     groups' partials for it and form S = sum_g scale[c][g] * N_g + R,
//     where R is the 64-wide rope product of the tile.
//  3. Online softmax on the owned 32x32 tile; the two waves that own the
//     same heads exchange their row maxima, so every head has one running
//     max.  The max moves lazily (only when exceeded by 2^8), so O is
//     rarely rescaled.  P goes to LDS in FP32.
//  4. PV, split over output columns and heads: wave (g, hh) accumulates
//     O^T for columns [128g, 128g+128) of its 32 heads.  V^T comes from the raw FP8/INT8
//     codes with ds_read_b64_tr_b8 and is converted to BF16 exactly; the
//     row scale of column group w is folded into P.
// The raw tiles are double-buffered in LDS, chunk-major: 16-byte piece ck
// (0..40) of tile row r (0..63) sits at byte ck*1024 + r*16.  The four
// non-owner waves fill the next tile straight from global memory with
// global_load_lds_dwordx4: one instruction moves piece ck of all 64 rows
// (lane = row, landing at base + 16*lane), so a lane needs only its own
// row's address.  The same layout makes the 32-row operand reads of QK and
// the transposed V reads contiguous in LDS.  Rows that are never loaded
// (masked entries) keep finite stale data from earlier rows or the initial
// zero fill, and contribute nothing because their probabilities are
// exactly 0.
#include "device_common.h"
#include "launch.h"
#include "lists.h"

namespace smla {

typedef float f32x16 __attribute__((ext_vector_type(16)));

__device__ __forceinline__ f32x16 mfma_32x32x16(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

template <int FMT>
__device__ __forceinline__ bf16x8 codes8_to_bf16x8(uint32_t c0, uint32_t c1) {
  const uint2 lo = codes4_to_bf16x4<FMT>(c0), hi = codes4_to_bf16x4<FMT>(c1);
  return __builtin_bit_cast(bf16x8, make_uint4(lo.x, lo.y, hi.x, hi.y));
}

__device__ __forceinline__ void global_to_lds_16(const void* src, void* lds_wave_base) {
  __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)src,
                                   (__attribute__((address_space(3))) void*)lds_wave_base, 16, 0, 0);
}

namespace wide {
constexpr int NT = 512;                      // 8 waves, 2 per SIMD
constexpr int TC = 64;                       // candidates per tile
constexpr int RB = 656;                      // FP8/INT8 row bytes
constexpr int CHUNKS = RB / 16;              // 41 pieces of 16 bytes per row
constexpr int CS = TC * 16;                  // bytes of one piece column (64 rows)
constexpr int TILE = CHUNKS * CS;            // 41,984 bytes per tile
constexpr int CK_SCALE = D_NOPE / 16;        // piece 32 holds the four scales
constexpr int CK_ROPE = CK_SCALE + 1;        // pieces 33..40 hold the rope
constexpr int GROUNDS = (CHUNKS + 3) / 4;    // pieces per gather wave (11, last one partial)
constexpr int OFF_RAW = 0;                   // [2][TILE]
constexpr int OFF_RECV = 2 * TILE;           // [4 score tiles][3 senders][64 lanes][16] f32
constexpr int OFF_PL = OFF_RECV + 4 * 3 * 64 * 16 * 4;
constexpr int PLS = 68;                      // P row stride (floats): [64 heads][PLS]
constexpr int OFF_MAX = OFF_PL + 64 * PLS * 4;   // [2][64] f32
constexpr int OFF_ALPHA = OFF_MAX + 2 * 64 * 4;  // [64] f32
constexpr int OFF_SCT = OFF_ALPHA + 64 * 4;      // [4 groups][64 rows] f32
constexpr int OFF_VALID = OFF_SCT + 4 * TC * 4;  // [2][64] int32: row was loaded
constexpr int LDS_BYTES = OFF_VALID + 2 * TC * 4;
constexpr float TAU = 8.0f;
}  // namespace wide

// Wave w = g + 4*hh works on latent group g (nope columns [128g, 128g+128),
// output columns likewise) for head half hh (heads [32hh, 32hh+32)).  Score
// tile (c2, hh) -- candidates [32c2, +32) x heads [32hh, +32) -- is owned by
// wave c2 + 6hh (waves 0, 1, 6, 7: one owner per SIMD); waves 2..5 gather.
template <int FMT, bool DECODE, bool DUAL>
__global__ __launch_bounds__(wide::NT, 1) void attn_wide_kernel(AttnParams p) {
  using namespace wide;
  static_assert(FMT == FMT_FP8 || FMT == FMT_INT8, "wide kernel serves quantized caches");
  __shared__ __attribute__((aligned(16))) uint8_t smem[LDS_BYTES];
  float* recv = reinterpret_cast<float*>(smem + OFF_RECV);
  float* pl = reinterpret_cast<float*>(smem + OFF_PL);
  float* maxb = reinterpret_cast<float*>(smem + OFF_MAX);
  float* alpha_l = reinterpret_cast<float*>(smem + OFF_ALPHA);
  float* sct = reinterpret_cast<float*>(smem + OFF_SCT);
  int32_t* valid = reinterpret_cast<int32_t*>(smem + OFF_VALID);

  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform, kept in SGPRs
  const int g = w & 3, hh = w >> 2;
  const int lane = tid & 63;
  const int l32 = lane & 31;
  const int hi = lane >> 5;
  const bool owner = (w == 0 || w == 1 || w == 6 || w == 7);
  const int oc2 = owner ? (w & 1) : 0;  // candidate half of the owned score tile
  const int nw = w - 2;                 // gather wave 0..3 (waves 2..5)

  const int64_t t = blockIdx.x;
  const int h0 = blockIdx.y * 64;
  const int split = DECODE ? (int)blockIdx.z : 0;

  const ListEnds le = list_ends(p, t);
  const Sources src_lists = sources<DUAL>(p);
  const int64_t topk_all = (int64_t)p.topk + p.topk2;
  int64_t j_begin = 0, j_end = topk_all;
  if (DECODE) {
    j_begin = (int64_t)split * p.split_w;
    j_end = j_begin + p.split_w;
    if (j_end > topk_all) j_end = topk_all;
  }
  if (j_end > le.end) j_end = le.end;
  const int n_tiles = j_end > j_begin ? (int)((j_end - j_begin + TC - 1) / TC) : 0;

  // Q as the B operand of S^T = K Q^T for head h0 + 32hh + l32.  A K lane
  // reads one 16-byte piece (8g + 2j + hi) that feeds MFMA steps 2j and
  // 2j+1, so qn[2j + b] holds nope columns 128g + 32j + 16hi + 8b + i; qr
  // holds rope columns 16ks + 8hi + i (owners).
  bf16x8 qn[8], qr[4];
  {
    const int h = h0 + 32 * hh + l32;
    const bool hv = h < p.H;
    const uint16_t* qrow = p.q + t * p.q_st + (int64_t)(hv ? h : 0) * p.q_sh;
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int b = 0; b < 2; ++b) {
        uint4 v = *reinterpret_cast<const uint4*>(qrow + 128 * g + 32 * j + 16 * hi + 8 * b);
        qn[2 * j + b] = __builtin_bit_cast(bf16x8, hv ? v : make_uint4(0, 0, 0, 0));
      }
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      uint4 v = *reinterpret_cast<const uint4*>(qrow + D_NOPE + 16 * ks + 8 * hi);
      qr[ks] = __builtin_bit_cast(bf16x8, hv ? v : make_uint4(0, 0, 0, 0));
    }
  }

  // the row of list position j_begin + k*64 + lane of this workgroup's
  // range, or null when the position holds no candidate
  auto row_offset = [&](int k) -> const uint8_t* {
    const int64_t j = j_begin + (int64_t)k * TC + lane;
    if (j >= j_end || !in_list<DUAL>(p, le, j)) return nullptr;
    return row_of<DUAL>(src_lists, j, *entry_ptr<DUAL>(src_lists, t, j));
  };
  // gather wave nw moves pieces nw, nw + 4, ... of all 64 rows of tile k
  // (lane = row) into raw buffer k&1, and wave 2 records which rows exist
  auto issue_tile = [&](int k, const uint8_t* src) {
    uint8_t* raw = smem + OFF_RAW + (k & 1) * TILE;
    if (src) {
#pragma unroll
      for (int r = 0; r < GROUNDS; ++r) {
        const int ck = nw + 4 * r;
        if (r + 1 < GROUNDS || ck < CHUNKS) global_to_lds_16(src + 16 * ck, raw + ck * CS);
      }
    }
    if (nw == 0) valid[(k & 1) * TC + lane] = src != nullptr;
  };

  // running softmax state of an owned score tile (heads 32hh + l32)
  float m_run = -INFINITY;
  float l_part = 0.0f;
  // O^T accumulators: columns [128g + 32dt, +32) x heads [32hh, +32)
  f32x16 O[4];
#pragma unroll
  for (int dt = 0; dt < 4; ++dt)
#pragma unroll
    for (int i = 0; i < 16; ++i) O[dt][i] = 0.0f;

  if (n_tiles > 0) {
    for (int i = tid; i < 2 * TILE / 16; i += NT) reinterpret_cast<uint4*>(smem + OFF_RAW)[i] = make_uint4(0, 0, 0, 0);
    const uint8_t* off0 = owner ? nullptr : row_offset(0);
    __syncthreads();
    if (!owner) issue_tile(0, off0);
  }

  for (int k = 0; k < n_tiles; ++k) {
    const uint8_t* raw = smem + OFF_RAW + (k & 1) * TILE;
    __builtin_amdgcn_s_waitcnt(0);  // this wave's part of tile k has landed
    __syncthreads();                // B0: all of tile k is in LDS
    const uint8_t* pend = nullptr;
    if (!owner) {
      if (k + 1 < n_tiles) pend = row_offset(k + 1);
      // the gather waves transpose the tile's scales:
      // sct[gg][row] = scale of row `row`, 128-column group gg
      const int e = nw * 64 + lane;
      const int row = e >> 2, gg = e & 3;
      sct[gg * TC + row] = *reinterpret_cast<const float*>(raw + CK_SCALE * CS + row * 16 + 4 * gg);
    }

    // ---- 1./2. unscaled partial S^T over nope columns [128g, 128g+128)
    // for heads 32hh..; the tile (c2, hh) goes to its owner c2 + 6hh ----
    f32x16 own;
#pragma unroll
    for (int c2 = 0; c2 < 2; ++c2) {
      f32x16 acc;
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[i] = 0.0f;
      const uint8_t* kp = raw + (8 * g + hi) * CS + (32 * c2 + l32) * 16;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint4 c16 = *reinterpret_cast<const uint4*>(kp + 2 * j * CS);
        acc = mfma_32x32x16(codes8_to_bf16x8<FMT>(c16.x, c16.y), qn[2 * j], acc);
        acc = mfma_32x32x16(codes8_to_bf16x8<FMT>(c16.z, c16.w), qn[2 * j + 1], acc);
      }
      const int ow = c2 + 6 * hh;
      if (ow == w) {
        own = acc;
      } else {
        const int og = c2 + 2 * hh;             // latent group of the owner
        const int slot = g < og ? g : g - 1;
        f32x4* dst = reinterpret_cast<f32x4*>(recv + (((c2 + 2 * hh) * 3 + slot) * 64 + lane) * 16);
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) dst[q4] = f32x4{acc[4 * q4], acc[4 * q4 + 1], acc[4 * q4 + 2], acc[4 * q4 + 3]};
      }
    }
    // rope product of the owned tile (all 64 rope columns)
    f32x16 s;
#pragma unroll
    for (int i = 0; i < 16; ++i) s[i] = 0.0f;
    if (owner) {
      const uint8_t* rp = raw + (CK_ROPE + hi) * CS + (32 * oc2 + l32) * 16;
#pragma unroll
      for (int ks = 0; ks < 4; ++ks)
        s = mfma_32x32x16(__builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(rp + 2 * ks * CS)), qr[ks], s);
    }
    __syncthreads();  // B1: partials visible; every wave is past PV(k-1)

    if (!owner && k + 1 < n_tiles) issue_tile(k + 1, pend);

    if (owner) {
      // S = sum_g scale[c][g] * N_g + rope over the owned rows
      // c = 32oc2 + 8q4 + 4hi + r; scales come from the transposed table,
      // four rows of one group per read
      const int tile_id = oc2 + 2 * hh;
      const f32x4* rsrc = reinterpret_cast<const f32x4*>(recv + (tile_id * 3 * 64 + lane) * 16);
      const float* srow = sct + 32 * oc2 + 4 * hi;
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const f32x4 so = *reinterpret_cast<const f32x4*>(srow + g * TC + 8 * q4);
#pragma unroll
        for (int r = 0; r < 4; ++r) s[4 * q4 + r] += so[r] * own[4 * q4 + r];
#pragma unroll
        for (int slot = 0; slot < 3; ++slot) {
          const int gs = slot < g ? slot : slot + 1;
          const f32x4 sc = *reinterpret_cast<const f32x4*>(srow + gs * TC + 8 * q4);
          const f32x4 v = rsrc[slot * 64 * 4 + q4];
#pragma unroll
          for (int r = 0; r < 4; ++r) s[4 * q4 + r] += sc[r] * v[r];
        }
      }
      const int32_t* vl = valid + (k & 1) * TC + 32 * oc2 + 4 * hi;
      float mx = -INFINITY;
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int i = 4 * q4 + r;
          s[i] = vl[8 * q4 + r] ? s[i] * p.scale_log2 : -INFINITY;
          mx = fmaxf(mx, s[i]);
        }
      }
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      if (hi == 0) maxb[oc2 * 64 + 32 * hh + l32] = mx;
    }
    __syncthreads();  // B2
    if (owner) {
      const float mx = fmaxf(maxb[32 * hh + l32], maxb[64 + 32 * hh + l32]);
      const bool need = mx > m_run + TAU;
      const float alpha = need ? ((m_run == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(m_run - mx)) : 1.0f;
      m_run = need ? mx : m_run;
      float psum = 0.0f;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        s[i] = (s[i] == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(s[i] - m_run);
        psum += s[i];
      }
      l_part = l_part * alpha + psum;
      float* prow = pl + (32 * hh + l32) * PLS + 32 * oc2 + 4 * hi;
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4)
        *reinterpret_cast<f32x4*>(prow + 8 * q4) = f32x4{s[4 * q4], s[4 * q4 + 1], s[4 * q4 + 2], s[4 * q4 + 3]};
      if (oc2 == 0 && hi == 0) alpha_l[32 * hh + l32] = alpha;
    }
    __syncthreads();  // B3

    // ---- 4. O^T += V^T P'^T over columns [128g, 128g + 128), heads 32hh.. ----
    {
      const float a = alpha_l[32 * hh + l32];
      if (__any(a != 1.0f)) {
#pragma unroll
        for (int dt = 0; dt < 4; ++dt) O[dt] *= a;
      }
    }
    // ds_read_b64_tr_b8: in each 16-lane group, lane 2r + b addresses row r
    // of an 8-row block, bytes 8b..8b+7 of a 16-column piece
    const int g16 = (lane >> 4) & 1;  // which 16 columns of the 32-column tile this lane group reads
    const int jr = (lane & 15) >> 1;
    const int jb = lane & 1;
    const uint8_t* vbase = raw + (8 * g + g16) * CS + (8 * hi + jr) * 16 + 8 * jb;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const f32x4 sa = *reinterpret_cast<const f32x4*>(sct + g * TC + 16 * ks + 8 * hi);
      const f32x4 sb = *reinterpret_cast<const f32x4*>(sct + g * TC + 16 * ks + 8 * hi + 4);
      const float* prow = pl + (32 * hh + l32) * PLS + 16 * ks + 8 * hi;
      const f32x4 x0 = *reinterpret_cast<const f32x4*>(prow);
      const f32x4 x1 = *reinterpret_cast<const f32x4*>(prow + 4);
      const bf16x8 pb = __builtin_bit_cast(
          bf16x8, make_uint4(pack_bf16(x0[0] * sa[0], x0[1] * sa[1]), pack_bf16(x0[2] * sa[2], x0[3] * sa[3]),
                             pack_bf16(x1[0] * sb[0], x1[1] * sb[1]), pack_bf16(x1[2] * sb[2], x1[3] * sb[3])));
#pragma unroll
      for (int dt = 0; dt < 4; ++dt) {
        const i32x2 v8 = lds_read_tr8(vbase + 2 * dt * CS + 16 * ks * 16);
        O[dt] = mfma_32x32x16(codes8_to_bf16x8<FMT>((uint32_t)v8[0], (uint32_t)v8[1]), pb, O[dt]);
      }
    }
  }

  // ---- epilogue: per-head max and sum, normalize, store ----
  float* lsum = maxb;     // [2][64]
  float* mfin = alpha_l;  // [64]
  __syncthreads();
  if (owner) {
    const float lt = l_part + __shfl_xor(l_part, 32);
    if (hi == 0) {
      lsum[oc2 * 64 + 32 * hh + l32] = lt;
      if (oc2 == 0) mfin[32 * hh + l32] = m_run;
    }
  }
  __syncthreads();
  const int hl = 32 * hh + l32;
  const int h = h0 + hl;
  const float Ls = lsum[hl] + lsum[64 + hl];
  const float M = mfin[hl];
  const bool empty = !(Ls > 0.0f);
  const float lse_v = empty ? -INFINITY : (M + __log2f(Ls)) * LN2;
  if (h >= p.H) return;
  if constexpr (DECODE) {
    const float inv = empty ? 0.0f : 1.0f / Ls;
    float* po = p.part_out + ((t * p.num_splits + split) * p.H + h) * (int64_t)D_V + 128 * g + 4 * hi;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4)
        *reinterpret_cast<f32x4*>(po + 32 * dt + 8 * q4) =
            f32x4{O[dt][4 * q4] * inv, O[dt][4 * q4 + 1] * inv, O[dt][4 * q4 + 2] * inv, O[dt][4 * q4 + 3] * inv};
    if (g == 0 && hi == 0) p.part_lse[(t * p.num_splits + split) * p.H + h] = lse_v;
  } else {
    float factor;
    if (empty) {
      factor = 0.0f;
    } else if (p.sink) {
      const float s2 = p.sink[h] * LOG2E;
      const float ms = fmaxf(M, s2);
      const float a = exp2f(M - ms);
      factor = a / (Ls * a + exp2f(s2 - ms));
    } else {
      factor = 1.0f / Ls;
    }
    uint16_t* orow = p.out + t * p.out_st + (int64_t)h * p.out_sh + 128 * g + 4 * hi;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4)
        *reinterpret_cast<uint2*>(orow + 32 * dt + 8 * q4) =
            make_uint2(pack_bf16(O[dt][4 * q4] * factor, O[dt][4 * q4 + 1] * factor),
                       pack_bf16(O[dt][4 * q4 + 2] * factor, O[dt][4 * q4 + 3] * factor));
    if (g == 0 && hi == 0) p.lse[t * p.lse_st + h] = lse_v;
  }
}

hipError_t launch_attention_wide(const AttnParams& p, int fmt, bool decode, hipStream_t s) {
  dim3 block(wide::NT);
  dim3 grid((unsigned)p.T, (unsigned)((p.H + 63) / 64), decode ? (unsigned)p.num_splits : 1u);
  const bool dual = p.topk2 > 0;
  if (fmt == FMT_INT8) {
    if (decode && dual) hipLaunchKernelGGL((attn_wide_kernel<FMT_INT8, true, true>), grid, block, 0, s, p);
    else if (decode) hipLaunchKernelGGL((attn_wide_kernel<FMT_INT8, true, false>), grid, block, 0, s, p);
    else if (dual) hipLaunchKernelGGL((attn_wide_kernel<FMT_INT8, false, true>), grid, block, 0, s, p);
    else hipLaunchKernelGGL((attn_wide_kernel<FMT_INT8, false, false>), grid, block, 0, s, p);
  } else if (fmt == FMT_FP8) {
    if (decode && dual) hipLaunchKernelGGL((attn_wide_kernel<FMT_FP8, true, true>), grid, block, 0, s, p);
    else if (decode) hipLaunchKernelGGL((attn_wide_kernel<FMT_FP8, true, false>), grid, block, 0, s, p);
    else if (dual) hipLaunchKernelGGL((attn_wide_kernel<FMT_FP8, false, true>), grid, block, 0, s, p);
    else hipLaunchKernelGGL((attn_wide_kernel<FMT_FP8, false, false>), grid, block, 0, s, p);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace smla
