// attention_bf16.hip -- sparse MLA attention over BF16 cache rows (576
// BF16 values: 512 nope + 64 rope) at any head count, and over the 656-byte
// quantized rows (FP8 with power-of-two or arbitrary scales, rope-less FP8,
// INT8) with 16 or fewer heads; prefill form and split-KV decode partials,
// for gfx950.
//
// What is computed is stated in include/smla.h.  The shapes it serves come
// from vLLM PR #57673 (Test Result): few native heads (h_q = 8 per rank),
// d = 512, combined top-k lists of 640 with attn_sink and topk_length, q
// and out read and written as head views of wider buffers.
//
// Work unit: one workgroup (4 waves) per (token, 16-head group, split);
// tiles of 64 list entries.  The work split follows the exponent-byte
// kernel (attention_mx.hip): QK over candidates (wave w owns candidates
// [16w, 16w+16), v_mfma 16x16x32, K rows as A), one running max per head
// shared by the four waves through LDS, and PV over value columns (wave w
// owns columns [128w, +128) for all 64 candidates, V^T read with
// ds_read_b64_tr_b16).  Each wave then holds 32 accumulator registers for
// O instead of 128, Q stays in registers (72), and the 64-row tile plus the
// probabilities fit in 79 KB of LDS, so two workgroups share a CU and
// their per-tile chains overlap.
//
// Quantized rows: PV reads V^T from the codes with ds_read_b64_tr_b8 and
// converts them with scale 1, and P is written in four versions, P times
// each wave's column scale.  With power-of-two scales QK converts each
// lane's codes with the row's scale of their 128 columns (exact in BF16);
// with arbitrary scales (INT8, GLM_NSA FP8) the codes convert exactly with
// scale 1, each 128-column group accumulates apart and is scaled per
// candidate, and each P version is a BF16 pair (the rounded value and the
// rest) so that the scale's rounding does not reach the output.
//
// Rows are gathered one tile ahead through registers (four threads per
// row, 16-byte pieces, one row address per thread and immediate offsets);
// masked rows are zero-filled so they can never inject NaN into PV.
// Block order: the head groups of one (token, split) sit on one XCD (the
// dispatcher deals consecutive workgroups to the 8 XCDs in turn) and meet
// in its L2.
#include <type_traits>

#include "device_common.h"
#include "launch.h"
#include "lists.h"

namespace smla {
namespace {

constexpr int TC = 64;        // candidates per tile
constexpr int NT = 256;       // 4 waves
constexpr float LAZY = 8.0f;  // log2 units
constexpr int NXCD = 8;       // XCDs of the chip
constexpr int KS = D_QK / 32;                 // 18 QK k-steps
constexpr int KS_NOPE = D_NOPE / 32;          // 16 of them over the nope part
constexpr int WCOLS = D_V / 4;                // 128 value columns per wave
constexpr int NDT = WCOLS / 16;               // 8
constexpr int P_HEAD = 144;                   // bytes of one head's P row (64 BF16, padded)

// Row geometry.  BF16 rows: 576 BF16 values.  Quantized rows (656 bytes):
// 512 codes, four FP32 scales (one per 128 columns), 64 BF16 rope values
// (padding in rope-less rows, never gathered).  P is kept in four versions,
// P times the scale of each wave's value columns, in FP16 under a per-tile
// bias (f16_bias).  BF16 rows keep P as a BF16 pair (the rounded value and
// the rest, two slots), so P enters PV with 16 significant bits.
template <int FMT>
struct Cols {
  static constexpr bool QUANT = FMT != FMT_BF16;
  static constexpr bool POW2 = FMT == FMT_FP8 || FMT == FMT_FP8_NOPE;  // scales applied while converting
  static constexpr bool ROPE = FMT != FMT_FP8_NOPE;
  static constexpr int ROW = FMT == FMT_BF16 ? 2 * D_QK : D_NOPE + 16 + 2 * D_ROPE;  // 1152 or 656
  static constexpr int LDS_ROW = ROW + 16;    // bank spread
  static constexpr int PIECES = ROPE ? ROW / 16 : (D_NOPE + 16) / 16;  // gathered: 72, 41 or 33
  static constexpr int NCH = (PIECES + 3) / 4;  // pieces per thread (4 threads per row)
  static constexpr int VERSIONS = !QUANT ? 2 : 4;
  // LDS: tile, P [versions][16 heads][64] BF16, wave maxima / sums [4][16],
  // index stage [3][64] (row addresses)
  static constexpr int TILE_BYTES = TC * LDS_ROW;
  static constexpr int P_OFF = TILE_BYTES;
  static constexpr int RED_OFF = P_OFF + VERSIONS * 16 * P_HEAD;
  static constexpr int IDX_OFF = RED_OFF + 4 * 16 * 4;
  static constexpr int EMAX_OFF = IDX_OFF + 3 * TC * 8;  // [4 waves] largest scale exponent of their rows
  static constexpr int LDS_BYTES = EMAX_OFF + 4 * 4;
  static_assert(LDS_BYTES <= 80 * 1024, "two workgroups per CU");
};

// eight e4m3 codes (bytes of c0 then c1, in order) times a power-of-two
// scale, exactly, as BF16
__device__ __forceinline__ bf16x8 e4m3x8_scaled(uint32_t c0, uint32_t c1, float scale) {
  const bf16x2 a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(c0, scale, false);
  const bf16x2 b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(c0, scale, true);
  const bf16x2 c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(c1, scale, false);
  const bf16x2 d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(c1, scale, true);
  return __builtin_bit_cast(bf16x8, make_uint4(__builtin_bit_cast(uint32_t, a), __builtin_bit_cast(uint32_t, b),
                                               __builtin_bit_cast(uint32_t, c), __builtin_bit_cast(uint32_t, d)));
}

// x - bf16(x) and y - bf16(y) as a BF16 pair, given hi = the BF16 pair of
// (x, y) (x in the low half)
__device__ __forceinline__ uint32_t bf16_pair_rest(float x, float y, uint32_t hi) {
  const float xh = __builtin_bit_cast(float, hi << 16);
  const float yh = __builtin_bit_cast(float, hi & 0xFFFF0000u);
  return pack_bf16(x - xh, y - yh);
}

// eight codes of a quantized row as BF16 (exact): e4m3 times a power-of-two
// scale, or int8 (scale applied later)
template <int FMT>
__device__ __forceinline__ bf16x8 codes8(uint32_t c0, uint32_t c1, float scale) {
  if constexpr (FMT == FMT_INT8) {
    const uint2 lo = int8x4_to_bf16x4(c0), hi = int8x4_to_bf16x4(c1);
    return __builtin_bit_cast(bf16x8, make_uint4(lo.x, lo.y, hi.x, hi.y));
  } else {
    return e4m3x8_scaled(c0, c1, scale);
  }
}

// a positive, finite, normal power of two
__device__ __forceinline__ bool pow2_scale(float s) {
  const uint32_t b = __builtin_bit_cast(uint32_t, s);
  const uint32_t e = b >> 23;
  return (b & 0x007FFFFFu) == 0 && e != 0 && e < 255;
}

template <bool DECODE, bool DUAL, int FMT>
__global__ __launch_bounds__(NT, 2) void attn_bf16_kernel(AttnParams p) {
  using G = Cols<FMT>;
  constexpr int LDS_ROW = G::LDS_ROW, PIECES = G::PIECES, NCH = G::NCH;
  constexpr int P_OFF = G::P_OFF, RED_OFF = G::RED_OFF, IDX_OFF = G::IDX_OFF;
  __shared__ __attribute__((aligned(16))) uint8_t smem[G::LDS_BYTES];
  uint8_t* tile = smem;
  uint8_t* pbuf = smem + P_OFF;
  float* red = reinterpret_cast<float*>(smem + RED_OFF);
  uint64_t* idx_lds = reinterpret_cast<uint64_t*>(smem + IDX_OFF);  // 0: no candidate
  uint32_t* emax = reinterpret_cast<uint32_t*>(smem + G::EMAX_OFF);

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int lg = lane >> 4;
  const int lc = lane & 15;

  // workgroup x -> (pair u = t*S + split, head group): x = ((u / 8)*HG + hg)*8 + u % 8
  const int HG = (p.H + 15) >> 4;
  const int S = DECODE ? p.num_splits : 1;
  const int64_t bx = blockIdx.x;
  const int64_t rest = bx / NXCD;
  const int hg = (int)(rest % HG);
  const int64_t u = (rest / HG) * NXCD + bx % NXCD;
  if (u >= p.T * S) return;  // the last round of pairs may be short (whole workgroup)
  const int64_t t = u / S;
  const int split = DECODE ? (int)(u % S) : 0;
  const int h0 = hg * 16;

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

  // Q^T as the B operand of S^T = K Q^T: lane holds Q[h0+lc][32ks + 8lg + i]
  bf16x8 qreg[KS];
  {
    const int h = h0 + lc;
    const bool hv = h < p.H;
    const uint16_t* qrow = p.q + t * p.q_st + (int64_t)(hv ? h : 0) * p.q_sh + 8 * lg;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      // (rope-less rows: q rows hold 512 values and the rope k-steps are 0)
      if (!G::ROPE && ks >= KS_NOPE) {
        qreg[ks] = __builtin_bit_cast(bf16x8, make_uint4(0, 0, 0, 0));
        continue;
      }
      const uint4 v = *reinterpret_cast<const uint4*>(qrow + 32 * ks);
      qreg[ks] = __builtin_bit_cast(bf16x8, hv ? v : make_uint4(0, 0, 0, 0));
    }
  }

  // row address of list position j_begin + 64k + tid, or 0
  auto load_idx = [&](int k) -> uint64_t {
    const int64_t j = j_begin + (int64_t)k * TC + tid;
    uint64_t v = 0;
    if (j < j_end && in_list<DUAL>(p, le, j)) v = (uint64_t)row_of<DUAL>(src_lists, j, *entry_ptr<DUAL>(src_lists, t, j));
    return v;
  };

  // thread tid gathers 16-byte pieces sub + 4r (r < NCH) of tile row tid / 4
  const int grow = tid >> 2, sub = tid & 3;
  uint4 stage[NCH];
  auto issue_rows = [&](int k) {
    const uint4* row = (const uint4*)idx_lds[(k % 3) * TC + grow];
    if (row) {
#pragma unroll
      for (int r = 0; r < NCH; ++r)
        if (PIECES % 4 == 0 || sub + 4 * r < PIECES) stage[r] = row[sub + 4 * r];
    } else {
#pragma unroll
      for (int r = 0; r < NCH; ++r) stage[r] = make_uint4(0, 0, 0, 0);
    }
  };
  auto store_rows = [&]() {
    uint4* dst = reinterpret_cast<uint4*>(tile + grow * LDS_ROW) + sub;
#pragma unroll
    for (int r = 0; r < NCH; ++r)
      if (PIECES % 4 == 0 || sub + 4 * r < PIECES) dst[4 * r] = stage[r];
    if constexpr (G::QUANT) {
      // the largest scale exponent of this wave's rows (piece 32, the four
      // scales, is stage[8] of the row's thread sub == 0), for the FP16 bias
      static_assert(D_NOPE / 16 == 8 * 4 && NCH > 8, "the scale piece");
      const uint4 sc = stage[8];
      const uint32_t e = sub == 0 ? max(max((sc.x >> 23) & 0xFFu, (sc.y >> 23) & 0xFFu),
                                        max((sc.z >> 23) & 0xFFu, (sc.w >> 23) & 0xFFu))
                                  : 0u;
      const uint32_t m = wave_max_u32(e);
      if (lane == 0) emax[wave] = m;
    }
  };

  // running max (log2 units) of head lc, shared by the four waves; this
  // lane's partial sum over its candidates; O^T for columns
  // 128*wave + 16dt + 4lg + i of head lc
  float m_run = -INFINITY;
  float l_part = 0.0f;
  int o_k = 0;  // FP16 rows: P, l and O are taken relative to 2^(m_run + o_k) (see f16_bias)
  f32x4 O[NDT];
#pragma unroll
  for (int i = 0; i < NDT; ++i) O[i] = f32x4{0.f, 0.f, 0.f, 0.f};

  if (n_tiles > 0) {
    if (tid < TC) {
      idx_lds[tid] = load_idx(0);
      if (n_tiles > 1) idx_lds[TC + tid] = load_idx(1);
    }
    __syncthreads();
    issue_rows(0);
    store_rows();
    __syncthreads();
  }

  for (int k = 0; k < n_tiles; ++k) {
    // power-of-two rows: PV of this tile in FP16 under the bias of its
    // largest scale (the waves' maxima are read before the next tile's rows
    // replace them)
    F16Bias bias{1.0f, 1.0f, 0.0f, 0};
    if constexpr (G::QUANT) bias = f16_bias(max(max(emax[0], emax[1]), max(emax[2], emax[3])), FMT == FMT_INT8 ? 5 : 7);
    if (k + 1 < n_tiles) issue_rows(k + 1);
    uint64_t pend = 0;
    if (k + 2 < n_tiles && tid < TC) pend = load_idx(k + 2);

    // ---- S^T for candidates 16*wave + (0..15) x heads h0 + (0..15) ----
    const uint8_t* rowA = tile + (16 * wave + lc) * LDS_ROW;
    f32x4 acc[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
    if constexpr (FMT == FMT_BF16) {
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {  // two chains
        const bf16x8 a = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(rowA + 16 * lg + 64 * ks));
        acc[ks & 1] = mfma_16x16x32(a, qreg[ks], acc[ks & 1]);
      }
    } else if constexpr (G::POW2) {
      // codes times the row's power-of-two scale of their 128 columns, exact
      // in BF16; a scale that is not a positive power of two makes the row's
      // first operand NaN, so the row's scores are NaN for every head (a row
      // that is not loaded holds zeros and is masked out below)
      const f32x4 sc = *reinterpret_cast<const f32x4*>(rowA + D_NOPE);
      const bool bad = !(pow2_scale(sc[0]) && pow2_scale(sc[1]) && pow2_scale(sc[2]) && pow2_scale(sc[3]));
#pragma unroll
      for (int ks = 0; ks < KS_NOPE; ++ks) {
        const uint2 c8 = *reinterpret_cast<const uint2*>(rowA + 32 * ks + 8 * lg);
        bf16x8 a = e4m3x8_scaled(c8.x, c8.y, sc[ks / 4]);
        if (ks == 0 && bad) a = __builtin_bit_cast(bf16x8, make_uint4(0x7FC07FC0u, 0x7FC07FC0u, 0x7FC07FC0u, 0x7FC07FC0u));
        acc[ks & 1] = mfma_16x16x32(a, qreg[ks], acc[ks & 1]);
      }
      if constexpr (G::ROPE) {
#pragma unroll
        for (int ks = KS_NOPE; ks < KS; ++ks) {
          const uint4 r = *reinterpret_cast<const uint4*>(rowA + D_NOPE + 16 + 64 * (ks - KS_NOPE) + 16 * lg);
          acc[ks & 1] = mfma_16x16x32(__builtin_bit_cast(bf16x8, r), qreg[ks], acc[ks & 1]);
        }
      }
    } else {
      // arbitrary scales: the codes convert exactly with scale 1, each
      // 128-column group accumulates apart, and S = sum_g scale(c, g) N_g +
      // rope; accumulator element i is candidate 16*wave + 4lg + i
      f32x4 accg[4] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f},
                       f32x4{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
      for (int ks = 0; ks < KS_NOPE; ++ks) {
        const uint2 c8 = *reinterpret_cast<const uint2*>(rowA + 32 * ks + 8 * lg);
        accg[ks / 4] = mfma_16x16x32(codes8<FMT>(c8.x, c8.y, 1.0f), qreg[ks], accg[ks / 4]);
      }
#pragma unroll
      for (int ks = KS_NOPE; ks < KS; ++ks) {
        const uint4 r = *reinterpret_cast<const uint4*>(rowA + D_NOPE + 16 + 64 * (ks - KS_NOPE) + 16 * lg);
        acc[1] = mfma_16x16x32(__builtin_bit_cast(bf16x8, r), qreg[ks], acc[1]);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const f32x4 sci = *reinterpret_cast<const f32x4*>(tile + (16 * wave + 4 * lg + i) * LDS_ROW + D_NOPE);
        acc[0][i] = (sci[0] * accg[0][i] + sci[1] * accg[1][i]) + (sci[2] * accg[2][i] + sci[3] * accg[3][i]);
      }
    }
    const uint64_t* il = idx_lds + (k % 3) * TC + 16 * wave + 4 * lg;
    float s[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) s[i] = il[i] != 0 ? (acc[0][i] + acc[1][i]) * p.scale_log2 : -INFINITY;

    // ---- one running max per head across the four waves ----
    float mx = fmaxf(fmaxf(s[0], s[1]), fmaxf(s[2], s[3]));
    mx = fmaxf(mx, __shfl_xor(mx, 16));
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    if (lg == 0) red[wave * 16 + lc] = mx;
    __syncthreads();
    mx = fmaxf(fmaxf(red[lc], red[16 + lc]), fmaxf(red[32 + lc], red[48 + lc]));
    // every wave takes the same decision per head, so the waves' column
    // slices stay under one max; lanes that do not move multiply by 1
    const bool need = mx > m_run + LAZY;
    const bool shift = G::QUANT && bias.k != o_k;  // this tile's k (scales above 2^14): O and l move with P
    if (__any(need) || shift) {
      const float alpha = (need ? ((m_run == -INFINITY) ? 0.0f : exp2f(m_run - mx)) : 1.0f) * exp2i(o_k - bias.k);
      m_run = need ? mx : m_run;
      o_k = bias.k;
      l_part *= alpha;
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) O[dt] *= alpha;
    }
    // (the finite floor keeps -inf scores at probability 0 while every score of a head is -inf)
    const float mb = fmaxf(m_run + (float)o_k, -__FLT_MAX__);
    float pr[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      pr[i] = __builtin_amdgcn_exp2f(s[i] - mb);
      l_part += pr[i];
    }
    if constexpr (FMT == FMT_BF16) {
      // P as a BF16 pair: the rounded value, then the rest
      const uint2 hi = make_uint2(pack_bf16(pr[0], pr[1]), pack_bf16(pr[2], pr[3]));
      *reinterpret_cast<uint2*>(pbuf + lc * P_HEAD + 2 * (16 * wave + 4 * lg)) = hi;
      *reinterpret_cast<uint2*>(pbuf + 16 * P_HEAD + lc * P_HEAD + 2 * (16 * wave + 4 * lg)) =
          make_uint2(bf16_pair_rest(pr[0], pr[1], hi.x), bf16_pair_rest(pr[2], pr[3], hi.y));
    } else {
      // version v: P x 2^-b x the scale of value columns [128v, +128) in
      // FP16, for the wave that owns those columns
      f32x4 scl[4];
#pragma unroll
      for (int i = 0; i < 4; ++i)
        scl[i] = *reinterpret_cast<const f32x4*>(tile + (16 * wave + 4 * lg + i) * LDS_ROW + D_NOPE);
#pragma unroll
      for (int i = 0; i < 4; ++i) pr[i] *= bias.p;
#pragma unroll
      for (int v = 0; v < 4; ++v)
        *reinterpret_cast<uint2*>(pbuf + v * 16 * P_HEAD + lc * P_HEAD + 2 * (16 * wave + 4 * lg)) =
            make_uint2(pack_f16(pr[0] * scl[0][v], pr[1] * scl[1][v]), pack_f16(pr[2] * scl[2][v], pr[3] * scl[3][v]));
    }
    __syncthreads();

    // ---- O^T += V^T P^T over value columns [128*wave, +128) ----
#pragma unroll
    for (int kc = 0; kc < 2; ++kc) {
      const uint8_t* pv = pbuf + (G::QUANT ? wave : 0) * 16 * P_HEAD;
      const uint4 pw = *reinterpret_cast<const uint4*>(pv + lc * P_HEAD + 2 * (32 * kc + 8 * lg));
      const bf16x8 pb = __builtin_bit_cast(bf16x8, pw);
      if constexpr (FMT == FMT_BF16) {
        // tr16: lane lc = 4r + b reads rows (32kc + 8lg + 4half + r), columns 4b..4b+3 of the block
        const bf16x8 pl = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(pbuf + 16 * P_HEAD + lc * P_HEAD +
                                                                                        2 * (32 * kc + 8 * lg)));
        const uint8_t* rb = tile + (32 * kc + 8 * lg + (lc >> 2)) * LDS_ROW + 2 * WCOLS * wave + 8 * (lc & 3);
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) {
          const i16x4 r0 = lds_read_tr16(rb + 32 * dt), r1 = lds_read_tr16(rb + 32 * dt + 4 * LDS_ROW);
          const bf16x8 a = __builtin_bit_cast(bf16x8, make_uint4(__builtin_bit_cast(uint2, r0).x, __builtin_bit_cast(uint2, r0).y,
                                                                 __builtin_bit_cast(uint2, r1).x, __builtin_bit_cast(uint2, r1).y));
          O[dt] = mfma_16x16x32(a, pb, O[dt]);
          O[dt] = mfma_16x16x32(a, pl, O[dt]);
        }
      } else {
        // tr8: lane lc = 2r + b reads row 32kc + 8lg + r (a candidate), bytes
        // 8b..8b+7 of a 16-column piece; lane lc receives column lc of the
        // 8 rows.  The codes convert to FP16 times 2^b (the row scale and
        // 2^-b are in P').
        const uint8_t* rb = tile + (32 * kc + 8 * lg + (lc >> 1)) * LDS_ROW + WCOLS * wave + 8 * (lc & 1);
        const f16x2 sb = {(_Float16)bias.v, (_Float16)bias.v};
        const f16x2 ob = {(_Float16)(-1152.0f * bias.v), (_Float16)(-1152.0f * bias.v)};
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) {
          const i32x2 c = lds_read_tr8(rb + 16 * dt);
          uint2 lo, hi;
          if constexpr (FMT == FMT_INT8) {
            lo = int8x4_to_f16x4((uint32_t)c[0], sb, ob);
            hi = int8x4_to_f16x4((uint32_t)c[1], sb, ob);
          } else {
            lo = fp8x4_to_f16x4((uint32_t)c[0], bias.v);
            hi = fp8x4_to_f16x4((uint32_t)c[1], bias.v);
          }
          O[dt] = mfma_16x16x32_f16(__builtin_bit_cast(f16x8, make_uint4(lo.x, lo.y, hi.x, hi.y)),
                                    __builtin_bit_cast(f16x8, pw), O[dt]);
        }
      }
    }

    if (k + 2 < n_tiles && tid < TC) idx_lds[((k + 2) % 3) * TC + tid] = pend;
    __syncthreads();
    if (k + 1 < n_tiles) store_rows();
    __syncthreads();
  }

  // ---- per-head sums from the four waves ----
  float l_w = l_part + __shfl_xor(l_part, 16);
  l_w += __shfl_xor(l_w, 32);
  if (lg == 0) red[wave * 16 + lc] = l_w;
  __syncthreads();
  const float Lsum = (red[lc] + red[16 + lc]) + (red[32 + lc] + red[48 + lc]);
  const float M = m_run + (float)o_k;

  const int h = h0 + lc;
  if (h >= p.H) return;
  const bool empty = !(Lsum > 0.0f);
  const float lse_v = empty ? -INFINITY : (M + __log2f(Lsum)) * LN2;
  const int col = WCOLS * wave + 4 * lg;
  if constexpr (DECODE) {
    const float inv = empty ? 0.0f : 1.0f / Lsum;
    float* po = p.part_out + ((t * p.num_splits + split) * p.H + h) * (int64_t)D_V + col;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) *reinterpret_cast<f32x4*>(po + 16 * dt) = O[dt] * inv;
    if (wave == 0 && lg == 0) p.part_lse[(t * p.num_splits + split) * p.H + h] = lse_v;
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
    uint16_t* orow = p.out + t * p.out_st + (int64_t)h * p.out_sh + col;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) {
      const f32x4 v = O[dt] * factor;
      *reinterpret_cast<uint2*>(orow + 16 * dt) = make_uint2(pack_bf16(v[0], v[1]), pack_bf16(v[2], v[3]));
    }
    if (wave == 0 && lg == 0) p.lse[t * p.lse_st + h] = lse_v;
  }
}

}  // namespace

hipError_t launch_attention_bf16(const AttnParams& p, int fmt, bool decode, hipStream_t s) {
  const int64_t pairs = p.T * (decode ? p.num_splits : 1);
  const int64_t blocks = (pairs + NXCD - 1) / NXCD * NXCD * ((p.H + 15) / 16);
  if (blocks > (int64_t)UINT32_MAX) return hipErrorInvalidConfiguration;
  dim3 block(NT);
  dim3 grid((unsigned)blocks);
  auto go = [&](auto f) {
    constexpr int F = decltype(f)::value;
    if (p.topk2 > 0) {
      if (decode) hipLaunchKernelGGL((attn_bf16_kernel<true, true, F>), grid, block, 0, s, p);
      else hipLaunchKernelGGL((attn_bf16_kernel<false, true, F>), grid, block, 0, s, p);
    } else {
      if (decode) hipLaunchKernelGGL((attn_bf16_kernel<true, false, F>), grid, block, 0, s, p);
      else hipLaunchKernelGGL((attn_bf16_kernel<false, false, F>), grid, block, 0, s, p);
    }
  };
  switch (fmt) {
    case FMT_FP8: go(std::integral_constant<int, FMT_FP8>{}); break;
    case FMT_FP8_NOPE: go(std::integral_constant<int, FMT_FP8_NOPE>{}); break;
    case FMT_FP8_ANY: go(std::integral_constant<int, FMT_FP8_ANY>{}); break;
    case FMT_INT8: go(std::integral_constant<int, FMT_INT8>{}); break;
    default: go(std::integral_constant<int, FMT_BF16>{}); break;
  }
  return hipGetLastError();
}

}  // namespace smla
