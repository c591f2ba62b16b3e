// attention_mx.hip -- sparse MLA attention over cache rows whose nope part
// carries one power-of-two exponent byte per tile (prefill form and
// split-KV decode partials) for gfx950.  Two row families, from FlashInfer
// PR #4802:
//  * DOTS3_SWA (description: d_qk = 1088, d_v = 1024, 1160 bytes per token
//    with the scales in a footer): 1024 e4m3 codes, 64 BF16 rope values,
//    eight exponent bytes (128-element tiles); V is the 1024 nope values.
//    Its lists hold at least 513 entries (a 512-entry selection plus the
//    sliding window), so tails are ragged.
//  * DSv4 (584 bytes; d_v = 512 for the V3.2 family): 448 e4m3 codes, 64
//    BF16 rope values, seven exponent bytes (64-element tiles) and a pad
//    byte; K and V are the whole 512-value row, so V's last 64 columns are
//    the BF16 rope values.
// What is computed is stated in include/smla.h.
//
// Work unit: one workgroup (4 waves) per (token, 16-head group, split);
// tiles of 64 list entries.  The value width (up to 1024 f32 per head) is
// too wide for one wave to hold the output of all its candidates, so the
// two products split the work differently:
//  * QK: wave w owns candidates [16w, 16w+16) of the tile and forms S^T
//    (v_mfma 16x16x32, K rows as A, Q^T from LDS, where the token's 16 q
//    rows stay for the whole list: in registers they would take up to 136
//    of them, more than the gather stage and O leave free).  Codes convert
//    to BF16 with scale 1 (exact); each scale tile accumulates apart and is
//    scaled afterwards, and the rope columns (BF16 in the row) add on top.
//  * The four waves agree on one running max per head through LDS (lazy:
//    it moves only when exceeded by 2^8, so O is rarely rescaled); each
//    wave writes its candidates' probabilities times each tile's scale
//    and the tile's FP16 bias, P'_g = P * scale(c, g) * 2^-b (and P itself
//    for BF16 value columns), in FP16 to LDS (f16_bias: b follows the
//    tile's largest exponent byte, from the waves' maxima in LDS).
//  * PV: wave w owns value columns [w*DV/4, (w+1)*DV/4) for all 64
//    candidates: O^T[d][h] += V^T[d][c] P'^T[c][h] (v_mfma_f32_16x16x32_f16);
//    V^T comes from the raw codes with ds_read_b64_tr_b8 (converted to FP16
//    times 2^b) or, for BF16 columns, with ds_read_b64_tr_b16 (converted to
//    FP16).
// Because every wave holds a disjoint slice of the value columns under the
// same running max, the end of the list needs only the per-head sums from
// the other waves, not a merge of outputs.
//
// Rows are gathered one tile ahead through registers while the current
// tile is consumed from LDS: four threads per row, each loading every
// fourth 16-byte piece (gfx950 serves 16-byte loads from these 8-byte-
// aligned rows); the 8-byte tail, which holds the exponent bytes, goes to
// the row's first thread, which also decodes it once into a float table
// for the tile.  One row address per thread and immediate offsets serve
// all the loads.  Masked rows are zero-filled so they can never inject NaN
// into PV.
//
// A secondary list (positions [topk, topk + topk2) over a second pool of
// the same format) runs in the DUAL instantiation: the index stage holds
// row addresses in both, so the two lists differ only where an entry is
// read and its row located.
//
// Block order: the head groups of one (token, split) read the same rows,
// so they are placed on the same XCD (the dispatcher deals consecutive
// workgroups to the 8 XCDs in turn) and meet in its L2, while consecutive
// (token, split) pairs go to different XCDs.
#include "device_common.h"
#include "launch.h"
#include "lists.h"

namespace smla {
namespace {

struct Dots3Row {
  static constexpr int NOPE = 1024, QK = 1088, DV = 1024, ROW = 1160;
  static constexpr int ROPE_OFF = 1024, SCALE_OFF = 1152, TILE = 128, NG = 8;
  static constexpr int OCC = 1;  // workgroups per CU the kernel is built for
};
struct Dsv4Row {
  static constexpr int NOPE = 448, QK = 512, DV = 512, ROW = 584;
  static constexpr int ROPE_OFF = 448, SCALE_OFF = 576, TILE = 64, NG = 7;
  static constexpr int OCC = 2;
};

constexpr int TC = 64;        // candidates per tile
constexpr int NT = 256;       // 4 waves
constexpr float LAZY = 8.0f;  // log2 units
constexpr int NXCD = 8;       // XCDs of the chip
constexpr int P_HEAD = 144;   // bytes of one head's P' row (64 BF16, padded)
constexpr int P_SLOT = 16 * P_HEAD;

template <class R>
struct Geo {
  static constexpr int KS_NOPE = R::NOPE / 32;          // QK k-steps over the nope part
  static constexpr int KS = R::QK / 32;                 // all QK k-steps (+2 rope)
  static constexpr int KS_PER_TILE = R::TILE / 32;      // k-steps per scale tile
  static constexpr bool ROPE_V = R::DV > R::NOPE;       // BF16 value columns (the rope part)
  static constexpr int SLOTS = R::NG + (ROPE_V ? 1 : 0);  // P' slots: one per scale tile (+ scale 1)
  static constexpr int WCOLS = R::DV / 4;               // value columns per wave
  static constexpr int NDT = WCOLS / 16;                // 16-column blocks per wave
  static constexpr int LDS_ROW = (R::ROW + 15) / 16 * 16 + 16;  // row stride in LDS (bank spread)
  static constexpr int PIECES = R::ROW / 16;            // whole 16-byte pieces per row (+ 8-byte tail)
  static constexpr int NCH = PIECES / 4;                // staged pieces per thread (4 threads per row)
  static constexpr int Q_ROW = 2 * R::QK + 16;
  // LDS: tile, Q [16][QK] BF16, P' [SLOTS][16 heads][64] BF16, scales [64][8] f32,
  // wave maxima / sums [4][16], index stage [3][64] (row addresses)
  static constexpr int TILE_BYTES = TC * LDS_ROW;
  static constexpr int Q_OFF = TILE_BYTES;
  static constexpr int P_OFF = Q_OFF + 16 * Q_ROW;
  static constexpr int SC_OFF = P_OFF + SLOTS * P_SLOT;
  static constexpr int RED_OFF = SC_OFF + TC * 8 * 4;
  static constexpr int IDX_OFF = RED_OFF + 4 * 16 * 4;
  static constexpr int EMAX_OFF = IDX_OFF + 3 * TC * 8;  // [4 waves] largest exponent byte of their rows
  static constexpr int LDS_BYTES = EMAX_OFF + 4 * 4;
  static_assert(R::ROW - 16 * PIECES == 8 && R::SCALE_OFF == 16 * PIECES, "the tail holds the scale bytes");
  static_assert(PIECES % 4 == 0 && R::NOPE % R::TILE == 0 && R::TILE % 32 == 0 && R::NG <= 8, "row geometry");
  // a wave's value columns are two scale tiles, 2w and 2w+1 (for DSv4's last
  // wave: tile 6 and the rope columns, whose P' slot is 7)
  static_assert(WCOLS == 2 * R::TILE && (!ROPE_V || R::DV - R::NOPE == R::TILE), "value columns per wave");
};

// scale byte -> 2^(b-127) (0 -> 2^-127, 255 -> NaN; the writer stores 1..254)
__device__ __forceinline__ float e8m0_to_f32(uint32_t b) {
  const uint32_t bits = b == 0u ? 0x00400000u : (b == 255u ? 0x7FC00000u : b << 23);
  return __builtin_bit_cast(float, bits);
}

template <class R, bool DECODE, bool DUAL>
__global__ __launch_bounds__(NT, R::OCC) void attn_mx_kernel(AttnParams p) {
  using G = Geo<R>;
  __shared__ __attribute__((aligned(16))) uint8_t smem[G::LDS_BYTES];
  uint8_t* tile = smem;
  uint8_t* qbuf = smem + G::Q_OFF;
  uint8_t* pbuf = smem + G::P_OFF;
  float* sct = reinterpret_cast<float*>(smem + G::SC_OFF);
  float* red = reinterpret_cast<float*>(smem + G::RED_OFF);
  uint64_t* idx_lds = reinterpret_cast<uint64_t*>(smem + G::IDX_OFF);  // 0: no candidate
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

  // the token's q rows of heads h0..h0+15 into LDS (zeros past H); they
  // are visible after the first barrier below
  for (int qc = tid; qc < 16 * (R::QK / 8); qc += NT) {
    const int hl = qc / (R::QK / 8), piece = qc % (R::QK / 8);
    const int h = h0 + hl;
    uint4 v = make_uint4(0, 0, 0, 0);
    if (h < p.H) v = *reinterpret_cast<const uint4*>(p.q + t * p.q_st + (int64_t)h * p.q_sh + 8 * piece);
    *reinterpret_cast<uint4*>(qbuf + hl * G::Q_ROW + 16 * piece) = v;
  }
  // Q^T as the B operand of S^T = K Q^T: lane reads Q[h0+lc][32ks + 8lg + i]
  const uint8_t* qB = qbuf + lc * G::Q_ROW + 16 * lg;

  // row address of list position j_begin + 64k + tid, or 0
  auto load_idx = [&](int k) -> uint64_t {
    const int64_t j = j_begin + (int64_t)k * TC + tid;
    uint64_t v = 0;
    if (j < j_end && in_list<DUAL>(p, le, j)) v = (uint64_t)row_of<DUAL>(src_lists, j, *entry_ptr<DUAL>(src_lists, t, j));
    return v;
  };

  // thread tid gathers 16-byte pieces sub + 4r (r < NCH) of tile row
  // tid / 4, and the row's 8-byte tail when sub == 0
  const int grow = tid >> 2, sub = tid & 3;
  uint4 stage[G::NCH];
  uint2 tail;
  auto issue_rows = [&](int k) {
    const uint8_t* row = (const uint8_t*)idx_lds[(k % 3) * TC + grow];
    if (row) {
#pragma unroll
      for (int r = 0; r < G::NCH; ++r) __builtin_memcpy(&stage[r], row + 16 * (sub + 4 * r), 16);
      tail = make_uint2(0, 0);
      if (sub == 0) __builtin_memcpy(&tail, row + 16 * G::PIECES, 8);
    } else {
#pragma unroll
      for (int r = 0; r < G::NCH; ++r) stage[r] = make_uint4(0, 0, 0, 0);
      tail = make_uint2(0, 0);
    }
  };
  auto store_rows = [&]() {
    uint8_t* dst = tile + grow * G::LDS_ROW;
#pragma unroll
    for (int r = 0; r < G::NCH; ++r) *reinterpret_cast<uint4*>(dst + 16 * (sub + 4 * r)) = stage[r];
    if (sub == 0) {  // the tail holds the row's scale bytes: decode them once for the tile
      *reinterpret_cast<uint2*>(dst + 16 * G::PIECES) = tail;
      f32x4 lo, hi;
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        lo[g] = e8m0_to_f32((tail.x >> (8 * g)) & 0xFFu);
        hi[g] = e8m0_to_f32((tail.y >> (8 * g)) & 0xFFu);
      }
      reinterpret_cast<f32x4*>(sct + grow * 8)[0] = lo;
      reinterpret_cast<f32x4*>(sct + grow * 8)[1] = hi;
    }
    // the largest exponent byte of this wave's rows, for the tile's FP16 bias
    const uint32_t e = wave_max_u32(sub == 0 ? max_byte<R::NG>(tail.x, tail.y) : 0u);
    if (lane == 0) emax[wave] = e;
  };

  // running max (log2 units) of head lc, shared by the four waves; this
  // lane's partial sum over its candidates; O^T for columns
  // WCOLS*wave + 16dt + 4lg + i of head lc
  float m_run = -INFINITY;
  float l_part = 0.0f;
  int o_k = 0;  // P, l and O are taken relative to 2^(m_run + o_k) (see f16_bias)
  f32x4 O[G::NDT];
#pragma unroll
  for (int i = 0; i < G::NDT; ++i) O[i] = f32x4{0.f, 0.f, 0.f, 0.f};

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
    // PV of this tile in FP16 under the bias of its largest scale (the
    // waves' maxima are read here, before the next tile's rows replace them)
    const F16Bias bias = f16_bias(max(max(emax[0], emax[1]), max(emax[2], emax[3])));
    if (k + 1 < n_tiles) issue_rows(k + 1);
    uint64_t pend = 0;
    if (k + 2 < n_tiles && tid < TC) pend = load_idx(k + 2);

    // ---- S^T for candidates 16*wave + (0..15) x heads h0 + (0..15) ----
    const uint8_t* rowA = tile + (16 * wave + lc) * G::LDS_ROW;
    f32x4 acc[R::NG + 1];
#pragma unroll
    for (int g = 0; g <= R::NG; ++g) acc[g] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < G::KS_PER_TILE; ++kk) {
#pragma unroll
      for (int g = 0; g < R::NG; ++g) {  // consecutive products go to different tiles
        const int ks = G::KS_PER_TILE * g + kk;
        const uint2 c8 = *reinterpret_cast<const uint2*>(rowA + 32 * ks + 8 * lg);
        const uint2 lo = fp8x4_to_bf16x4(c8.x), hi = fp8x4_to_bf16x4(c8.y);
        const bf16x8 b = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(qB + 64 * ks));
        acc[g] = mfma_16x16x32(__builtin_bit_cast(bf16x8, make_uint4(lo.x, lo.y, hi.x, hi.y)), b, acc[g]);
      }
    }
#pragma unroll
    for (int ks = G::KS_NOPE; ks < G::KS; ++ks) {
      const bf16x8 a = __builtin_bit_cast(
          bf16x8, *reinterpret_cast<const uint4*>(rowA + R::ROPE_OFF + 2 * (32 * (ks - G::KS_NOPE) + 8 * lg)));
      const bf16x8 b = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(qB + 64 * ks));
      acc[R::NG] = mfma_16x16x32(a, b, acc[R::NG]);
    }

    // scores of candidates c = 16*wave + 4lg + i for head lc
    const uint64_t* il = idx_lds + (k % 3) * TC + 16 * wave + 4 * lg;
    // scales of candidate (4lg+i), tiles 0..3 and 4..7
    auto scales = [&](int i, int half) -> f32x4 {
      return reinterpret_cast<const f32x4*>(sct + (16 * wave + 4 * lg + i) * 8)[half];
    };
    float s[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const f32x4 lo = scales(i, 0), hi = scales(i, 1);
      float v = acc[R::NG][i];
#pragma unroll
      for (int g = 0; g < R::NG; ++g) v += (g < 4 ? lo[g & 3] : hi[g & 3]) * acc[g][i];
      s[i] = il[i] != 0 ? v * p.scale_log2 : -INFINITY;
    }

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
    const bool shift = bias.k != o_k;  // this tile's k (scales above 2^14): O and l move with P
    if (__any(need) || shift) {
      const float alpha = (need ? ((m_run == -INFINITY) ? 0.0f : exp2f(m_run - mx)) : 1.0f) * exp2i(o_k - bias.k);
      m_run = need ? mx : m_run;
      o_k = bias.k;
      l_part *= alpha;
#pragma unroll
      for (int dt = 0; dt < G::NDT; ++dt) O[dt] *= alpha;
    }
    // (the finite floor keeps -inf scores at probability 0 while every score of a head is -inf)
    const float mb = fmaxf(m_run + (float)o_k, -__FLT_MAX__);
    float pr[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      pr[i] = __builtin_amdgcn_exp2f(s[i] - mb);
      l_part += pr[i];
    }
    // P'_g[h][c] = P[c][h] * scale(c, g) * 2^-b in FP16, candidates
    // 16*wave + 4lg + (0..3); slot NG (the BF16 value columns, unbiased)
    // holds P itself
    float prb[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) prb[i] = pr[i] * bias.p;
#pragma unroll
    for (int g = 0; g < G::SLOTS; ++g) {
      uint32_t u0, u1;
      if (g < R::NG) {
        float sg[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) sg[i] = scales(i, g >> 2)[g & 3];
        u0 = pack_f16(prb[0] * sg[0], prb[1] * sg[1]);
        u1 = pack_f16(prb[2] * sg[2], prb[3] * sg[3]);
      } else {
        u0 = pack_f16(pr[0], pr[1]);
        u1 = pack_f16(pr[2], pr[3]);
      }
      *reinterpret_cast<uint2*>(pbuf + g * P_SLOT + lc * P_HEAD + 2 * (16 * wave + 4 * lg)) = make_uint2(u0, u1);
    }
    __syncthreads();

    // ---- O^T += V^T P'^T over value columns [WCOLS*wave, +WCOLS) ----
#pragma unroll
    for (int kc = 0; kc < 2; ++kc) {
      f16x8 pb[2];  // P' of slots 2w and 2w+1 for candidates 32kc + 8lg + (0..7)
#pragma unroll
      for (int gg = 0; gg < 2; ++gg)
        pb[gg] = __builtin_bit_cast(
            f16x8, *reinterpret_cast<const uint4*>(pbuf + (2 * wave + gg) * P_SLOT + lc * P_HEAD + 2 * (32 * kc + 8 * lg)));
#pragma unroll
      for (int dt = 0; dt < G::NDT; ++dt) {
        const int c0 = G::WCOLS * wave + 16 * dt;  // first column of the block (wave-uniform)
        f16x8 a;
        if (!G::ROPE_V || c0 < R::NOPE) {
          // tr8: lane lc = 2r + b reads candidate row (32kc + 8lg + r), byte columns c0 + 8b..
          const i32x2 raw = lds_read_tr8(tile + (32 * kc + 8 * lg + (lc >> 1)) * G::LDS_ROW + c0 + 8 * (lc & 1));
          const uint2 lo = fp8x4_to_f16x4((uint32_t)raw[0], bias.v), hi = fp8x4_to_f16x4((uint32_t)raw[1], bias.v);
          a = __builtin_bit_cast(f16x8, make_uint4(lo.x, lo.y, hi.x, hi.y));
        } else {
          // tr16 (BF16 rope columns): lane lc = 4r + b reads rows (32kc + 8lg + 4half + r), columns 4b..
          const uint8_t* rb = tile + (32 * kc + 8 * lg + (lc >> 2)) * G::LDS_ROW + R::ROPE_OFF + 2 * (c0 - R::NOPE) + 8 * (lc & 3);
          const uint2 r0 = __builtin_bit_cast(uint2, lds_read_tr16(rb));
          const uint2 r1 = __builtin_bit_cast(uint2, lds_read_tr16(rb + 4 * G::LDS_ROW));
          a = __builtin_bit_cast(f16x8, make_uint4(bf16x2_to_f16x2(r0.x), bf16x2_to_f16x2(r0.y), bf16x2_to_f16x2(r1.x),
                                                   bf16x2_to_f16x2(r1.y)));
        }
        O[dt] = mfma_16x16x32_f16(a, pb[dt / (G::NDT / 2)], O[dt]);
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
  const int col = G::WCOLS * wave + 4 * lg;
  if constexpr (DECODE) {
    const float inv = empty ? 0.0f : 1.0f / Lsum;
    float* po = p.part_out + ((t * p.num_splits + split) * p.H + h) * (int64_t)R::DV + col;
#pragma unroll
    for (int dt = 0; dt < G::NDT; ++dt) *reinterpret_cast<f32x4*>(po + 16 * dt) = O[dt] * inv;
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
    for (int dt = 0; dt < G::NDT; ++dt) {
      const f32x4 v = O[dt] * factor;
      *reinterpret_cast<uint2*>(orow + 16 * dt) = make_uint2(pack_bf16(v[0], v[1]), pack_bf16(v[2], v[3]));
    }
    if (wave == 0 && lg == 0) p.lse[t * p.lse_st + h] = lse_v;
  }
}

// ---------------------------------------------------------------------------
// DOTS3_SWA rows with more than 16 heads: 32 heads per workgroup.  With
// 16 heads a workgroup's per-tile chain is paid once per 16 heads, and the
// 16 q rows (1088 values each) fill LDS; here eight waves share each
// gathered tile between two 16-head halves hh, and QK is split over the
// latent instead of over candidates so that Q stays in registers:
//  * QK: wave (wl, hh) forms partial S^T over nope columns [256wl, +256)
//    (two scale tiles, scaled after accumulating) plus, for wl < 2, rope
//    k-step wl, for all 64 candidates of the tile and the 16 heads of hh;
//    the four partials of each 16-candidate block meet in LDS at the wave
//    that owns the block (wl), which then runs the softmax of the 16-head
//    kernel above for its candidates;
//  * PV is the 16-head kernel's: wave (wl, hh) owns value columns
//    [256wl, +256) of its 16 heads.
// LDS: tile 75.8 KB, partial-score exchange 32 KB, P' 36 KB, scales, sums
// and index stage: 146 KB, one workgroup per CU (two waves per SIMD).
constexpr int NT32 = 512;  // 8 waves

template <class R, bool DECODE, bool DUAL>
__global__ __launch_bounds__(NT32, 1) void attn_mx32_kernel(AttnParams p) {
  using G = Geo<R>;
  constexpr int KSW = R::NOPE / 4 / 32;      // nope k-steps per wave (8)
  constexpr int TPW = R::NOPE / 4 / R::TILE;  // scale tiles per wave (2)
  constexpr int NROPE = G::KS - G::KS_NOPE;   // rope k-steps (2), one per wave wl < NROPE
  constexpr int PIECES8 = G::PIECES / 8;      // 16-byte pieces per thread (8 threads per row)
  static_assert(G::ROPE_V == false && TPW == 2 && KSW == 2 * G::KS_PER_TILE && NROPE <= 4 &&
                    G::PIECES % 8 == 0 && G::WCOLS == 2 * R::TILE,
                "the DOTS3_SWA geometry");
  constexpr int XCH_OFF = G::TILE_BYTES;                       // f32x4 [2 hh][4 src][4 blk][64]
  constexpr int P_OFF2 = XCH_OFF + 2 * 4 * 4 * 64 * 16;
  constexpr int SC_OFF2 = P_OFF2 + 2 * G::SLOTS * P_SLOT;
  constexpr int RED_OFF2 = SC_OFF2 + TC * 8 * 4;
  constexpr int IDX_OFF2 = RED_OFF2 + 2 * 4 * 16 * 4;
  constexpr int EMAX_OFF2 = IDX_OFF2 + 3 * TC * 8;  // [8 waves] largest exponent byte of their rows
  constexpr int LDS_BYTES2 = EMAX_OFF2 + 8 * 4;
  static_assert(LDS_BYTES2 <= 160 * 1024, "LDS");
  __shared__ __attribute__((aligned(16))) uint8_t smem[LDS_BYTES2];
  uint8_t* tile = smem;
  f32x4* xch = reinterpret_cast<f32x4*>(smem + XCH_OFF);
  float* sct = reinterpret_cast<float*>(smem + SC_OFF2);
  uint64_t* idx_lds = reinterpret_cast<uint64_t*>(smem + IDX_OFF2);
  uint32_t* emax = reinterpret_cast<uint32_t*>(smem + EMAX_OFF2);

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int wl = wave & 3, hh = wave >> 2;
  const int lane = tid & 63;
  const int lg = lane >> 4;
  const int lc = lane & 15;
  uint8_t* pbuf = smem + P_OFF2 + hh * G::SLOTS * P_SLOT;
  float* red = reinterpret_cast<float*>(smem + RED_OFF2) + hh * 64;

  // workgroup x -> (pair u = t*S + split, 32-head group): x = ((u / 8)*HG + hg)*8 + u % 8
  const int HG = (p.H + 31) >> 5;
  const int S = DECODE ? p.num_splits : 1;
  const int64_t bx = blockIdx.x;
  const int64_t rest = bx / NXCD;
  const int hg = (int)(rest % HG);
  const int64_t u = (rest / HG) * NXCD + bx % NXCD;
  if (u >= p.T * S) return;  // the last round of pairs may be short (whole workgroup)
  const int64_t t = u / S;
  const int split = DECODE ? (int)(u % S) : 0;
  const int h0 = hg * 32 + 16 * hh;  // this wave's 16 heads

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

  // Q^T slices as B operands: lane holds Q[h0+lc][32ks + 8lg + i] for this
  // wave's nope k-steps ks = KSW*wl + j and, for wl < NROPE, rope k-step wl
  bf16x8 qn[KSW], qr;
  {
    const int h = h0 + lc;
    const bool hv = h < p.H;
    const uint16_t* qrow = p.q + t * p.q_st + (int64_t)(hv ? h : 0) * p.q_sh + 8 * lg;
#pragma unroll
    for (int j = 0; j < KSW; ++j) {
      const uint4 v = *reinterpret_cast<const uint4*>(qrow + 32 * (KSW * wl + j));
      qn[j] = __builtin_bit_cast(bf16x8, hv ? v : make_uint4(0, 0, 0, 0));
    }
    const int rk = wl < NROPE ? wl : 0;
    const uint4 v = *reinterpret_cast<const uint4*>(qrow + 32 * (G::KS_NOPE + rk));
    qr = __builtin_bit_cast(bf16x8, (hv && wl < NROPE) ? v : make_uint4(0, 0, 0, 0));
  }

  auto load_idx = [&](int k) -> uint64_t {
    const int64_t j = j_begin + (int64_t)k * TC + tid;
    uint64_t v = 0;
    if (j < j_end && in_list<DUAL>(p, le, j)) v = (uint64_t)row_of<DUAL>(src_lists, j, *entry_ptr<DUAL>(src_lists, t, j));
    return v;
  };

  // thread tid gathers 16-byte pieces sub + 8r (r < PIECES8) of tile row
  // tid / 8, and the row's 8-byte tail (its scale bytes) when sub == 0
  const int grow = tid >> 3, sub = tid & 7;
  uint4 stage[PIECES8];
  uint2 tail;
  auto issue_rows = [&](int k) {
    const uint8_t* row = (const uint8_t*)idx_lds[(k % 3) * TC + grow];
    if (row) {
#pragma unroll
      for (int r = 0; r < PIECES8; ++r) __builtin_memcpy(&stage[r], row + 16 * (sub + 8 * r), 16);
      tail = make_uint2(0, 0);
      if (sub == 0) __builtin_memcpy(&tail, row + 16 * G::PIECES, 8);
    } else {
#pragma unroll
      for (int r = 0; r < PIECES8; ++r) stage[r] = make_uint4(0, 0, 0, 0);
      tail = make_uint2(0, 0);
    }
  };
  auto store_rows = [&]() {
    uint8_t* dst = tile + grow * G::LDS_ROW;
#pragma unroll
    for (int r = 0; r < PIECES8; ++r) *reinterpret_cast<uint4*>(dst + 16 * (sub + 8 * r)) = stage[r];
    if (sub == 0) {
      *reinterpret_cast<uint2*>(dst + 16 * G::PIECES) = tail;
      f32x4 lo, hi;
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        lo[g] = e8m0_to_f32((tail.x >> (8 * g)) & 0xFFu);
        hi[g] = e8m0_to_f32((tail.y >> (8 * g)) & 0xFFu);
      }
      reinterpret_cast<f32x4*>(sct + grow * 8)[0] = lo;
      reinterpret_cast<f32x4*>(sct + grow * 8)[1] = hi;
    }
    // the largest exponent byte of this wave's rows, for the tile's FP16 bias
    const uint32_t e = wave_max_u32(sub == 0 ? max_byte<R::NG>(tail.x, tail.y) : 0u);
    if (lane == 0) emax[wave] = e;
  };

  float m_run = -INFINITY;
  float l_part = 0.0f;
  int o_k = 0;  // P, l and O are taken relative to 2^(m_run + o_k) (see f16_bias)
  f32x4 O[G::NDT];
#pragma unroll
  for (int i = 0; i < G::NDT; ++i) O[i] = f32x4{0.f, 0.f, 0.f, 0.f};

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
    // PV of this tile in FP16 under the bias of its largest scale
    const F16Bias bias = f16_bias(max(max(max(emax[0], emax[1]), max(emax[2], emax[3])),
                                      max(max(emax[4], emax[5]), max(emax[6], emax[7]))));
    if (k + 1 < n_tiles) issue_rows(k + 1);
    uint64_t pend = 0;
    if (k + 2 < n_tiles && tid < TC) pend = load_idx(k + 2);

    // ---- partial S^T over this wave's latent slice, candidate blocks cb ----
    f32x4 own;  // the block this wave owns (cb == wl), kept in registers
#pragma unroll
    for (int cb = 0; cb < 4; ++cb) {
      const uint8_t* rowA = tile + (16 * cb + lc) * G::LDS_ROW;
      f32x4 acc[TPW + 1];
#pragma unroll
      for (int g = 0; g <= TPW; ++g) acc[g] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < G::KS_PER_TILE; ++kk) {
#pragma unroll
        for (int g = 0; g < TPW; ++g) {
          const int j = G::KS_PER_TILE * g + kk;
          const uint2 c8 = *reinterpret_cast<const uint2*>(rowA + 32 * (KSW * wl + j) + 8 * lg);
          const uint2 lo = fp8x4_to_bf16x4(c8.x), hi = fp8x4_to_bf16x4(c8.y);
          acc[g] = mfma_16x16x32(__builtin_bit_cast(bf16x8, make_uint4(lo.x, lo.y, hi.x, hi.y)), qn[j], acc[g]);
        }
      }
      if (wl < NROPE) {
        const bf16x8 a = __builtin_bit_cast(
            bf16x8, *reinterpret_cast<const uint4*>(rowA + R::ROPE_OFF + 2 * (32 * wl + 8 * lg)));
        acc[TPW] = mfma_16x16x32(a, qr, acc[TPW]);
      }
      // scale tiles TPW*wl + g of candidates 16cb + 4lg + i
      f32x4 ps = acc[TPW];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const f32x2 sc = *reinterpret_cast<const f32x2*>(sct + (16 * cb + 4 * lg + i) * 8 + TPW * wl);
        ps[i] += sc[0] * acc[0][i] + sc[1] * acc[1][i];
      }
      if (cb == wl) own = ps;
      else xch[((hh * 4 + wl) * 4 + cb) * 64 + lane] = ps;
    }
    __syncthreads();
    // scores of candidates c = 16wl + 4lg + i for head lc: the four slices
    const uint64_t* il = idx_lds + (k % 3) * TC + 16 * wl + 4 * lg;
    float s[4];
    {
      f32x4 sum = own;
#pragma unroll
      for (int src = 0; src < 4; ++src)
        if (src != wl) sum += xch[((hh * 4 + src) * 4 + wl) * 64 + lane];
#pragma unroll
      for (int i = 0; i < 4; ++i) s[i] = il[i] != 0 ? sum[i] * p.scale_log2 : -INFINITY;
    }

    // ---- one running max per head across the four waves of hh ----
    float mx = fmaxf(fmaxf(s[0], s[1]), fmaxf(s[2], s[3]));
    mx = fmaxf(mx, __shfl_xor(mx, 16));
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    if (lg == 0) red[wl * 16 + lc] = mx;
    __syncthreads();
    mx = fmaxf(fmaxf(red[lc], red[16 + lc]), fmaxf(red[32 + lc], red[48 + lc]));
    const bool need = mx > m_run + LAZY;
    const bool shift = bias.k != o_k;  // this tile's k (scales above 2^14): O and l move with P
    if (__any(need) || shift) {
      const float alpha = (need ? ((m_run == -INFINITY) ? 0.0f : exp2f(m_run - mx)) : 1.0f) * exp2i(o_k - bias.k);
      m_run = need ? mx : m_run;
      o_k = bias.k;
      l_part *= alpha;
#pragma unroll
      for (int dt = 0; dt < G::NDT; ++dt) O[dt] *= alpha;
    }
    // (the finite floor keeps -inf scores at probability 0 while every score of a head is -inf)
    const float mb = fmaxf(m_run + (float)o_k, -__FLT_MAX__);
    float pr[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      pr[i] = __builtin_amdgcn_exp2f(s[i] - mb);
      l_part += pr[i];
    }
    // P'_g[h][c] = P[c][h] * scale(c, g) * 2^-b in FP16, candidates 16wl + 4lg + (0..3)
#pragma unroll
    for (int i = 0; i < 4; ++i) pr[i] *= bias.p;
#pragma unroll
    for (int g = 0; g < R::NG; ++g) {
      float sg[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) sg[i] = sct[(16 * wl + 4 * lg + i) * 8 + g];
      const uint32_t u0 = pack_f16(pr[0] * sg[0], pr[1] * sg[1]);
      const uint32_t u1 = pack_f16(pr[2] * sg[2], pr[3] * sg[3]);
      *reinterpret_cast<uint2*>(pbuf + g * P_SLOT + lc * P_HEAD + 2 * (16 * wl + 4 * lg)) = make_uint2(u0, u1);
    }
    __syncthreads();

    // ---- O^T += V^T P'^T over value columns [WCOLS*wl, +WCOLS) ----
#pragma unroll
    for (int kc = 0; kc < 2; ++kc) {
      f16x8 pb[2];
#pragma unroll
      for (int gg = 0; gg < 2; ++gg)
        pb[gg] = __builtin_bit_cast(
            f16x8, *reinterpret_cast<const uint4*>(pbuf + (2 * wl + gg) * P_SLOT + lc * P_HEAD + 2 * (32 * kc + 8 * lg)));
#pragma unroll
      for (int dt = 0; dt < G::NDT; ++dt) {
        const int c0 = G::WCOLS * wl + 16 * dt;
        const i32x2 raw = lds_read_tr8(tile + (32 * kc + 8 * lg + (lc >> 1)) * G::LDS_ROW + c0 + 8 * (lc & 1));
        const uint2 lo = fp8x4_to_f16x4((uint32_t)raw[0], bias.v), hi = fp8x4_to_f16x4((uint32_t)raw[1], bias.v);
        O[dt] = mfma_16x16x32_f16(__builtin_bit_cast(f16x8, make_uint4(lo.x, lo.y, hi.x, hi.y)), pb[dt / (G::NDT / 2)],
                                  O[dt]);
      }
    }

    if (k + 2 < n_tiles && tid < TC) idx_lds[((k + 2) % 3) * TC + tid] = pend;
    __syncthreads();
    if (k + 1 < n_tiles) store_rows();
    __syncthreads();
  }

  // ---- per-head sums from the four waves of hh ----
  float l_w = l_part + __shfl_xor(l_part, 16);
  l_w += __shfl_xor(l_w, 32);
  if (lg == 0) red[wl * 16 + lc] = l_w;
  __syncthreads();
  const float Lsum = (red[lc] + red[16 + lc]) + (red[32 + lc] + red[48 + lc]);
  const float M = m_run + (float)o_k;

  const int h = h0 + lc;
  if (h >= p.H) return;
  const bool empty = !(Lsum > 0.0f);
  const float lse_v = empty ? -INFINITY : (M + __log2f(Lsum)) * LN2;
  const int col = G::WCOLS * wl + 4 * lg;
  if constexpr (DECODE) {
    const float inv = empty ? 0.0f : 1.0f / Lsum;
    float* po = p.part_out + ((t * p.num_splits + split) * p.H + h) * (int64_t)R::DV + col;
#pragma unroll
    for (int dt = 0; dt < G::NDT; ++dt) *reinterpret_cast<f32x4*>(po + 16 * dt) = O[dt] * inv;
    if (wl == 0 && lg == 0) p.part_lse[(t * p.num_splits + split) * p.H + h] = lse_v;
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
    for (int dt = 0; dt < G::NDT; ++dt) {
      const f32x4 v = O[dt] * factor;
      *reinterpret_cast<uint2*>(orow + 16 * dt) = make_uint2(pack_bf16(v[0], v[1]), pack_bf16(v[2], v[3]));
    }
    if (wl == 0 && lg == 0) p.lse[t * p.lse_st + h] = lse_v;
  }
}

template <class R>
hipError_t launch_rows32(const AttnParams& p, bool decode, hipStream_t s) {
  const int64_t pairs = p.T * (decode ? p.num_splits : 1);
  const int64_t blocks = (pairs + NXCD - 1) / NXCD * NXCD * ((p.H + 31) / 32);
  if (blocks > (int64_t)UINT32_MAX) return hipErrorInvalidConfiguration;
  dim3 block(NT32);
  dim3 grid((unsigned)blocks);
  if (p.topk2 > 0) {
    if (decode) hipLaunchKernelGGL((attn_mx32_kernel<R, true, true>), grid, block, 0, s, p);
    else hipLaunchKernelGGL((attn_mx32_kernel<R, false, true>), grid, block, 0, s, p);
  } else {
    if (decode) hipLaunchKernelGGL((attn_mx32_kernel<R, true, false>), grid, block, 0, s, p);
    else hipLaunchKernelGGL((attn_mx32_kernel<R, false, false>), grid, block, 0, s, p);
  }
  return hipGetLastError();
}

template <class R>
hipError_t launch_rows(const AttnParams& p, bool decode, hipStream_t s) {
  const int64_t pairs = p.T * (decode ? p.num_splits : 1);
  const int64_t blocks = (pairs + NXCD - 1) / NXCD * NXCD * ((p.H + 15) / 16);
  if (blocks > (int64_t)UINT32_MAX) return hipErrorInvalidConfiguration;
  dim3 block(NT);
  dim3 grid((unsigned)blocks);
  if (p.topk2 > 0) {
    if (decode) hipLaunchKernelGGL((attn_mx_kernel<R, true, true>), grid, block, 0, s, p);
    else hipLaunchKernelGGL((attn_mx_kernel<R, false, true>), grid, block, 0, s, p);
  } else {
    if (decode) hipLaunchKernelGGL((attn_mx_kernel<R, true, false>), grid, block, 0, s, p);
    else hipLaunchKernelGGL((attn_mx_kernel<R, false, false>), grid, block, 0, s, p);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attention_mx(const AttnParams& p, int fmt, bool decode, hipStream_t s) {
  if (fmt == FMT_FP8_DOTS3) return p.H > 16 ? launch_rows32<Dots3Row>(p, decode, s) : launch_rows<Dots3Row>(p, decode, s);
  if (fmt == FMT_FP8_DSV4) return launch_rows<Dsv4Row>(p, decode, s);
  return hipErrorInvalidValue;
}

}  // namespace smla
