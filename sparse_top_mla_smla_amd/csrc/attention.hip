// attention.hip -- sparse MLA attention over a paged latent cache (prefill
// form and split-KV decode partials) for gfx950.
//
// What is computed is stated in include/smla.h (FlashInfer PR #4802 row
// layout, page block, strided indices, topk_length, sinks; vLLM PR #57673
// d=512 and few-head views).  This file is the execution scheme.
//
// Work unit: one workgroup (4 waves) per (token, 16-head group, split).
// Candidates are processed in tiles of 64 list entries.  Per tile:
//  * the 64 rows are gathered from the pool into LDS (16-byte loads,
//    software-pipelined one tile ahead through registers; masked rows are
//    zero-filled so they can never inject NaN into the PV product);
//  * wave w owns candidates [16w, 16w+16) of the tile and computes
//      S^T[c][h] = K[c] . Q[h]          (v_mfma 16x16x32, K rows as A)
//    FP8/INT8 codes are converted to BF16 exactly and the per-(row, 128-
//    tile) scales are applied to the four partial accumulators;
//  * online softmax in the exp2 domain with a lazy max update: the running
//    max only moves (and O is only rescaled) when a score exceeds it by
//    more than 2^8, so probabilities stay <= 256 and the rescale of the
//    128 accumulator registers is rare;
//  * O^T[d][h] += V^T[d][c] P^T[c][h]   (v_mfma 16x16x16): V^T comes from
//    LDS with the gfx950 transpose reads, and the MFMA output layout of
//    S^T is already the B-operand layout P^T needs, so P never touches LDS.
//    For FP8/INT8 the V scale of each row is folded into P per 128-column
//    group.
// Each wave keeps its own (max, sum, O) over its candidates; the four
// states are merged through LDS once at the end (the same log-sum-exp merge
// the decode combine uses).
#include <type_traits>

#include "device_common.h"
#include "launch.h"
#include "lists.h"

namespace smla {

constexpr int TILE_C = 64;     // candidates per tile
constexpr int NTHREADS = 256;  // 4 waves
constexpr float LAZY_TAU = 8.0f;

// DUAL: the call has a secondary list, and the index stage holds row
// addresses (0: no candidate) instead of main-pool slots (-1: none); the
// single-list kernels keep the narrower stage and its registers.
template <int FMT, bool DUAL>
struct Cfg {
  using G = RowGeom<FMT>;
  using IdxT = typename std::conditional<DUAL, uint64_t, int32_t>::type;
  static constexpr IdxT NONE = DUAL ? (IdxT)0 : (IdxT)-1;
  // (a slot stage holds NONE or slots >= 0: testing the sign lets the
  // compiler form row addresses with shifts)
  static __device__ __forceinline__ bool present(IdxT e) {
    if constexpr (DUAL) return e != 0;
    return e >= 0;
  }
  static constexpr int LDS_ROW = G::BYTES + 16;                 // padded row stride
  static constexpr int TILE_BYTES = TILE_C * LDS_ROW;
  static constexpr int IDX_OFF = TILE_BYTES;                    // IdxT [3][64]
  static constexpr int RED_O_BYTES = 2 * 16 * D_V * 4;          // two waves' O
  static constexpr int RED_ML_OFF = RED_O_BYTES;                // [4 waves][16][2] f32
  static constexpr int LDS_BYTES =
      (TILE_BYTES + 3 * TILE_C * (int)sizeof(IdxT)) > (RED_O_BYTES + 4 * 16 * 2 * 4)
          ? (TILE_BYTES + 3 * TILE_C * (int)sizeof(IdxT))
          : (RED_O_BYTES + 4 * 16 * 2 * 4);
  static constexpr int TOTAL_CHUNKS = TILE_C * G::CHUNKS;
  static constexpr int NCH = (TOTAL_CHUNKS + NTHREADS - 1) / NTHREADS;  // staged chunks/thread
};

template <int FMT, bool DECODE, bool DUAL>
__global__ __launch_bounds__(NTHREADS, 1) void attn_kernel(AttnParams p) {
  using C = Cfg<FMT, DUAL>;
  using IdxT = typename C::IdxT;
  using G = RowGeom<FMT>;
  constexpr bool QUANT = FMT != FMT_BF16;
  constexpr bool NOPE = FMT == FMT_FP8_NOPE;  // rows without rope dimensions
  __shared__ __attribute__((aligned(16))) uint8_t smem[C::LDS_BYTES];
  uint8_t* tile = smem;
  IdxT* idx_lds = reinterpret_cast<IdxT*>(smem + C::IDX_OFF);

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int lg = lane >> 4;   // lane group 0..3
  const int lc = lane & 15;   // lane column 0..15

  const int64_t t = blockIdx.x;
  const int h0 = blockIdx.y * 16;
  const int split = DECODE ? (int)blockIdx.z : 0;

  // candidate range of this workgroup over the token's list positions
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
  const int n_tiles = j_end > j_begin ? (int)((j_end - j_begin + TILE_C - 1) / TILE_C) : 0;

  // Q^T as the B operand of S^T = K Q^T: lane holds Q[h0+lc][32ks + 8lg + i]
  bf16x8 qreg[18];
  {
    const int h = h0 + lc;
    const bool hv = h < p.H;
    const uint16_t* qrow = p.q + t * p.q_st + (int64_t)(hv ? h : 0) * p.q_sh;
#pragma unroll
    for (int ks = 0; ks < 18; ++ks) {
      // (rows without rope dimensions: q rows end at 512, the rope slices are 0)
      const bool load = hv && (ks < 16 || !NOPE);
      uint4 v = load ? *reinterpret_cast<const uint4*>(qrow + 32 * ks + 8 * lg) : make_uint4(0, 0, 0, 0);
      qreg[ks] = __builtin_bit_cast(bf16x8, v);
    }
  }

  // index stage entry of list position j_begin + 64k + tid: with a
  // secondary list the address of its row, else its main-pool slot; NONE
  // when the position holds no candidate
  auto load_idx = [&](int k) -> IdxT {
    int64_t j = j_begin + (int64_t)k * TILE_C + tid;
    IdxT v = C::NONE;
    if (j < j_end && in_list<DUAL>(p, le, j)) {
      const int32_t x = *entry_ptr<DUAL>(src_lists, t, j);
      if constexpr (DUAL) {
        v = (uint64_t)row_of<DUAL>(src_lists, j, x);
      } else {
        if (x >= 0 && (int64_t)x < p.nslots) v = x;
      }
    }
    return v;
  };

  uint4 stage[C::NCH];
  auto issue_rows = [&](int k) {
    const IdxT* il = idx_lds + (k % 3) * TILE_C;
#pragma unroll
    for (int r = 0; r < C::NCH; ++r) {
      const int qc = tid + r * NTHREADS;
      uint4 v = make_uint4(0, 0, 0, 0);
      if (qc < C::TOTAL_CHUNKS) {
        const int row = qc / G::CHUNKS, ck = qc % G::CHUNKS;
        const IdxT e = il[row];
        // (rows without rope dimensions: their padding is not gathered)
        if (C::present(e) && !(NOPE && 16 * ck >= G::ROPE_OFF)) {
          const uint8_t* src;
          if constexpr (DUAL) {
            src = (const uint8_t*)e;
          } else {
            src = p.pool + (int64_t)(e / PAGE) * p.block_stride + (int64_t)(e % PAGE) * p.row_stride;
          }
          v = *reinterpret_cast<const uint4*>(src + 16 * ck);
        }
      }
      stage[r] = v;
    }
  };
  auto store_rows = [&]() {
#pragma unroll
    for (int r = 0; r < C::NCH; ++r) {
      const int qc = tid + r * NTHREADS;
      if (qc < C::TOTAL_CHUNKS) {
        const int row = qc / G::CHUNKS, ck = qc % G::CHUNKS;
        *reinterpret_cast<uint4*>(tile + row * C::LDS_ROW + 16 * ck) = stage[r];
      }
    }
  };

  // running state of this wave: max (log2 units) per head lc, per-lane
  // partial sum, O^T accumulators O[dt] (lane: d = 16dt + 4lg + i, head lc)
  float m_run = -INFINITY;
  float l_part = 0.0f;
  f32x4 O[32];
#pragma unroll
  for (int i = 0; i < 32; ++i) O[i] = f32x4{0.f, 0.f, 0.f, 0.f};

  if (n_tiles > 0) {
    if (tid < TILE_C) {
      idx_lds[tid] = load_idx(0);
      if (n_tiles > 1) idx_lds[TILE_C + tid] = load_idx(1);
    }
    __syncthreads();
    issue_rows(0);
    store_rows();
    __syncthreads();
  }

  for (int k = 0; k < n_tiles; ++k) {
    if (k + 1 < n_tiles) issue_rows(k + 1);
    IdxT pend = C::NONE;
    if (k + 2 < n_tiles && tid < TILE_C) pend = load_idx(k + 2);

    // ---- S^T for this wave's 16 candidates x 16 heads ----
    const uint8_t* rowA = tile + (16 * wave + lc) * C::LDS_ROW;
    f32x4 acc[QUANT ? 5 : 1];
#pragma unroll
    for (int i = 0; i < (QUANT ? 5 : 1); ++i) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < 16; ++ks) {
      bf16x8 a;
      if constexpr (QUANT) {
        const uint2 c8 = *reinterpret_cast<const uint2*>(rowA + 32 * ks + 8 * lg);
        const uint2 lo = codes4_to_bf16x4<FMT>(c8.x), hi = codes4_to_bf16x4<FMT>(c8.y);
        a = __builtin_bit_cast(bf16x8, make_uint4(lo.x, lo.y, hi.x, hi.y));
        acc[ks >> 2] = mfma_16x16x32(a, qreg[ks], acc[ks >> 2]);
      } else {
        a = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(rowA + 2 * (32 * ks + 8 * lg)));
        acc[0] = mfma_16x16x32(a, qreg[ks], acc[0]);
      }
    }
    // rope product (rows without rope dimensions have none)
#pragma unroll
    for (int ks = 16; ks < 18 && !NOPE; ++ks) {
      const bf16x8 a = __builtin_bit_cast(
          bf16x8, *reinterpret_cast<const uint4*>(rowA + G::ROPE_OFF + 2 * (32 * (ks - 16) + 8 * lg)));
      acc[QUANT ? 4 : 0] = mfma_16x16x32(a, qreg[ks], acc[QUANT ? 4 : 0]);
    }

    // scores of candidates c = 16*wave + 4lg + i for head lc
    const IdxT* il = idx_lds + (k % 3) * TILE_C + 16 * wave + 4 * lg;
    float s[4];
    f32x4 sc[4];  // sc[i][g]: scale of row (4lg+i), 128-group g
    if constexpr (QUANT) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
        sc[i] = *reinterpret_cast<const f32x4*>(tile + (16 * wave + 4 * lg + i) * C::LDS_ROW + G::SCALE_OFF);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float v;
      if constexpr (QUANT) {
        v = acc[4][i];
#pragma unroll
        for (int g = 0; g < 4; ++g) v += sc[i][g] * acc[g][i];
      } else {
        v = acc[0][i];
      }
      s[i] = C::present(il[i]) ? v * p.scale_log2 : -INFINITY;
    }

    // ---- online softmax (lazy max) ----
    float mx = fmaxf(fmaxf(s[0], s[1]), fmaxf(s[2], s[3]));
    mx = fmaxf(mx, __shfl_xor(mx, 16));
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    // The decision is per head (all lanes of a head agree), so one head's
    // result never depends on the other heads of the group; lanes that do
    // not move their max multiply by exactly 1.
    const bool need = mx > m_run + LAZY_TAU;
    if (__any(need)) {
      const float alpha = need ? ((m_run == -INFINITY) ? 0.0f : exp2f(m_run - mx)) : 1.0f;
      m_run = need ? mx : m_run;
      l_part *= alpha;
#pragma unroll
      for (int dt = 0; dt < 32; ++dt) O[dt] *= alpha;
    }
    float pr[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      pr[i] = (s[i] == -INFINITY) ? 0.0f : exp2f(s[i] - m_run);
      l_part += pr[i];
    }

    // ---- O^T += V^T P^T ----
    i16x4 pb[QUANT ? 4 : 1];
    if constexpr (QUANT) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const uint32_t u0 = pack_bf16(pr[0] * sc[0][g], pr[1] * sc[1][g]);
        const uint32_t u1 = pack_bf16(pr[2] * sc[2][g], pr[3] * sc[3][g]);
        pb[g] = __builtin_bit_cast(i16x4, make_uint2(u0, u1));
      }
    } else {
      pb[0] = __builtin_bit_cast(i16x4, make_uint2(pack_bf16(pr[0], pr[1]), pack_bf16(pr[2], pr[3])));
    }
    if constexpr (QUANT) {
      // tr8: lane lc = 2r + b reads row (4lg + r%4), byte columns 8b..8b+7
      const uint8_t* vbase = tile + (16 * wave + 4 * lg + ((lc >> 1) & 3)) * C::LDS_ROW + 8 * (lc & 1);
#pragma unroll
      for (int dt = 0; dt < 32; ++dt) {
        const i32x2 raw = lds_read_tr8(vbase + 16 * dt);
        const uint2 v4 = codes4_to_bf16x4<FMT>((uint32_t)raw[0]);
        O[dt] = mfma_16x16x16(__builtin_bit_cast(i16x4, v4), pb[dt >> 3], O[dt]);
      }
    } else {
      // tr16: lane lc = 4r + b reads row (4lg + r), columns 4b..4b+3
      const uint8_t* vbase = tile + (16 * wave + 4 * lg + (lc >> 2)) * C::LDS_ROW + 8 * (lc & 3);
#pragma unroll
      for (int dt = 0; dt < 32; ++dt) {
        const i16x4 v4 = lds_read_tr16(vbase + 32 * dt);
        O[dt] = mfma_16x16x16(v4, pb[0], O[dt]);
      }
    }

    if (k + 2 < n_tiles && tid < TILE_C) idx_lds[((k + 2) % 3) * TILE_C + tid] = pend;
    __syncthreads();
    if (k + 1 < n_tiles) store_rows();
    __syncthreads();
  }

  // ---- merge the four waves' states ----
  float l_w = l_part + __shfl_xor(l_part, 16);
  l_w += __shfl_xor(l_w, 32);
  float* red_o = reinterpret_cast<float*>(smem);
  float* red_ml = reinterpret_cast<float*>(smem + C::RED_ML_OFF);
  __syncthreads();  // LDS reuse
  if (lg == 0) {
    red_ml[(wave * 16 + lc) * 2 + 0] = m_run;
    red_ml[(wave * 16 + lc) * 2 + 1] = l_w;
  }
  __syncthreads();
  float M = -INFINITY;
#pragma unroll
  for (int w = 0; w < 4; ++w) M = fmaxf(M, red_ml[(w * 16 + lc) * 2]);
  float Lsum = 0.0f;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    const float mw = red_ml[(w * 16 + lc) * 2];
    const float fw = (mw == -INFINITY) ? 0.0f : exp2f(mw - M);
    Lsum += fw * red_ml[(w * 16 + lc) * 2 + 1];
  }
  {
    const float f_own = (m_run == -INFINITY) ? 0.0f : exp2f(m_run - M);
#pragma unroll
    for (int dt = 0; dt < 32; ++dt) O[dt] *= f_own;
  }
  if (wave >= 2) {
    f32x4* dst = reinterpret_cast<f32x4*>(red_o) + (wave - 2) * 32 * 64;
#pragma unroll
    for (int dt = 0; dt < 32; ++dt) dst[dt * 64 + lane] = O[dt];
  }
  __syncthreads();
  if (wave < 2) {
    const f32x4* srcp = reinterpret_cast<const f32x4*>(red_o) + wave * 32 * 64;
#pragma unroll
    for (int dt = 0; dt < 32; ++dt) O[dt] += srcp[dt * 64 + lane];
  }
  __syncthreads();
  if (wave == 1) {
    f32x4* dst = reinterpret_cast<f32x4*>(red_o);
#pragma unroll
    for (int dt = 0; dt < 32; ++dt) dst[dt * 64 + lane] = O[dt];
  }
  __syncthreads();
  if (wave != 0) return;
  {
    const f32x4* srcp = reinterpret_cast<const f32x4*>(red_o);
#pragma unroll
    for (int dt = 0; dt < 32; ++dt) O[dt] += srcp[dt * 64 + lane];
  }

  const int h = h0 + lc;
  if (h >= p.H) return;
  const bool empty = !(Lsum > 0.0f);
  const float lse_v = empty ? -INFINITY : (M + __log2f(Lsum)) * LN2;
  if constexpr (DECODE) {
    const float inv = empty ? 0.0f : 1.0f / Lsum;
    float* po = p.part_out + ((t * p.num_splits + split) * p.H + h) * (int64_t)D_V + 4 * lg;
#pragma unroll
    for (int dt = 0; dt < 32; ++dt) *reinterpret_cast<f32x4*>(po + 16 * dt) = O[dt] * inv;
    if (lg == 0) p.part_lse[(t * p.num_splits + split) * p.H + h] = lse_v;
  } else {
    float factor;
    if (empty) {
      factor = 0.0f;
    } else if (p.sink) {
      const float s2 = p.sink[h] * LOG2E;
      const float ms = fmaxf(M, s2);
      const float a = exp2f(M - ms);
      factor = a / (Lsum * a + exp2f(s2 - ms));
    } else {
      factor = 1.0f / Lsum;
    }
    uint16_t* orow = p.out + t * p.out_st + (int64_t)h * p.out_sh + 4 * lg;
#pragma unroll
    for (int dt = 0; dt < 32; ++dt) {
      const f32x4 v = O[dt] * factor;
      *reinterpret_cast<uint2*>(orow + 16 * dt) = make_uint2(pack_bf16(v[0], v[1]), pack_bf16(v[2], v[3]));
    }
    if (lg == 0) p.lse[t * p.lse_st + h] = lse_v;
  }
}

template <int FMT>
static hipError_t launch_fmt(const AttnParams& p, bool decode, hipStream_t s) {
  dim3 block(NTHREADS);
  dim3 grid((unsigned)p.T, (unsigned)((p.H + 15) / 16), decode ? (unsigned)p.num_splits : 1u);
  if (p.topk2 > 0) {
    if (decode) hipLaunchKernelGGL((attn_kernel<FMT, true, true>), grid, block, 0, s, p);
    else hipLaunchKernelGGL((attn_kernel<FMT, false, true>), grid, block, 0, s, p);
  } else {
    if (decode) hipLaunchKernelGGL((attn_kernel<FMT, true, false>), grid, block, 0, s, p);
    else hipLaunchKernelGGL((attn_kernel<FMT, false, false>), grid, block, 0, s, p);
  }
  return hipGetLastError();
}

hipError_t launch_attention(const AttnParams& p, int fmt, bool decode, hipStream_t s) {
  // BF16 rows at any head count: the kernel whose waves split PV over columns
  if (fmt == FMT_BF16) return launch_attention_bf16(p, FMT_BF16, decode, s);
  // FP8 rows with power-of-two scales and few heads: the same kernel
  if (fmt == FMT_FP8 && p.H <= 16) return launch_attention_bf16(p, FMT_FP8, decode, s);
  // rows with exponent-byte scales have their own row geometry and widths
  if (fmt == FMT_FP8_DOTS3 || fmt == FMT_FP8_DSV4) return launch_attention_mx(p, fmt, decode, s);
  // many heads over a quantized cache (FP8 with any scales, with or without
  // rope, and INT8): one workgroup per token for 64 heads
  if (p.H > 16) return launch_attention_fp8(p, fmt, decode, s);
  switch (fmt) {
    case FMT_BF16: return launch_fmt<FMT_BF16>(p, decode, s);
    case FMT_FP8:
    case FMT_FP8_ANY: return launch_fmt<FMT_FP8>(p, decode, s);
    case FMT_FP8_NOPE: return launch_fmt<FMT_FP8_NOPE>(p, decode, s);
    case FMT_INT8: return launch_fmt<FMT_INT8>(p, decode, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace smla
