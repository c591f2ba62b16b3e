// attention_dots3.hip -- sparse MLA attention over DOTS3_SWA cache rows
// (prefill form and split-KV decode partials) for gfx950.
//
// What is computed is stated in include/smla.h.  FlashInfer PR #4802's
// description gives DOTS3_SWA as d_qk = 1088 (1024 nope + 64 rope), d_v =
// 1024 and 1160 bytes per token with the scales in a footer: 1024 e4m3
// codes, 64 BF16 rope values, then one power-of-two exponent byte (bias 127)
// per 128-element tile.  Its lists hold at least 513 entries (a 512-entry
// selection plus the sliding window), so tails are ragged.
//
// Work unit: one workgroup (4 waves) per (token, 16-head group, split);
// tiles of 64 list entries.  The value width (1024 f32 per head) is too
// wide for one wave to hold the output of all its candidates, so the two
// products split the work differently:
//  * QK: wave w owns candidates [16w, 16w+16) of the tile and forms S^T
//    (v_mfma 16x16x32, K rows as A, Q^T from LDS, where the token's 16 q
//    rows stay for the whole list: in registers they would take 136 of
//    them, more than the gather stage and O leave free).
//    Codes convert to BF16 with scale 1 (exact); each 128-column group
//    accumulates apart and is scaled by its exponent byte afterwards, and
//    the rope columns (BF16 in the row) add on top.
//  * The four waves agree on one running max per head through LDS (lazy:
//    it moves only when exceeded by 2^8, so O is rarely rescaled); each
//    wave writes its candidates' probabilities times each group's scale,
//    P'_g = P * scale(c, g), in BF16 to LDS.
//  * PV: wave w owns value columns [256w, 256w+256) for all 64 candidates:
//    O^T[d][h] += V^T[d][c] P'^T[c][h] (v_mfma 16x16x32), V^T read from the
//    raw codes with ds_read_b64_tr_b8 and converted with scale 1.
// Because every wave holds a disjoint slice of the value columns under the
// same running max, the end of the list needs only the per-head sums from
// the other waves, not a merge of outputs.
//
// Rows are gathered one tile ahead through registers while the current
// tile is consumed from LDS: four threads per row, each loading every
// fourth 16-byte piece (gfx950 serves 16-byte loads from the 8-byte-aligned
// rows; the 8-byte tail goes to the row's first thread), so one row address
// per thread and immediate offsets serve all 19 loads.  Masked rows are
// zero-filled so they can never inject NaN into PV.
//
// Block order: the workgroups of one token's head groups (and of one
// split) read the same rows, so they are placed on the same XCD (the
// dispatcher deals consecutive workgroups to the 8 XCDs in turn) and meet
// in its L2.
#include "device_common.h"
#include "launch.h"
#include "lists.h"

namespace smla {
namespace {

constexpr int TC = 64;        // candidates per tile
constexpr int NT = 256;       // 4 waves
constexpr float LAZY = 8.0f;  // log2 units
constexpr int KS = dots3::D_QK / 32;        // 34 k-steps of QK (32 nope + 2 rope)
constexpr int LDS_ROW = 1184;               // 1160 rounded up to 16, + 16 (bank spread)
constexpr int PIECES = dots3::ROW_BYTES / 16;  // 72 whole 16-byte pieces per row (+ an 8-byte tail)
constexpr int NCH = PIECES / 4;                // 18 staged pieces per thread (4 threads per row)
constexpr int NXCD = 8;                        // XCDs of the chip
// LDS: the tile, Q [16 heads][1088] BF16 (rows padded to 2192 B), P' [8
// groups][16 heads][64 candidates] BF16 (head rows padded to 144 B), the
// tile's scales as floats [64][8], wave maxima / sums [4][16], index stage
// [3][64]
constexpr int TILE_BYTES = TC * LDS_ROW;
constexpr int Q_ROW = 2 * dots3::D_QK + 16;
constexpr int Q_OFF = TILE_BYTES;
constexpr int P_HEAD = 144;
constexpr int P_GROUP = 16 * P_HEAD;
constexpr int P_OFF = Q_OFF + 16 * Q_ROW;
constexpr int SC_OFF = P_OFF + dots3::NGROUPS * P_GROUP;
constexpr int RED_OFF = SC_OFF + TC * dots3::NGROUPS * 4;
constexpr int IDX_OFF = RED_OFF + 4 * 16 * 4;
constexpr int LDS_BYTES = IDX_OFF + 3 * TC * 4;

// scale byte -> 2^(b-127) (0 -> 2^-127, 255 -> NaN; the writer stores 1..254)
__device__ __forceinline__ float e8m0_to_f32(uint32_t b) {
  const uint32_t bits = b == 0u ? 0x00400000u : (b == 255u ? 0x7FC00000u : b << 23);
  return __builtin_bit_cast(float, bits);
}

template <bool DECODE>
__global__ __launch_bounds__(NT, 1) void attn_dots3_kernel(AttnParams p) {
  __shared__ __attribute__((aligned(16))) uint8_t smem[LDS_BYTES];
  uint8_t* tile = smem;
  uint8_t* qbuf = smem + Q_OFF;
  uint8_t* pbuf = smem + P_OFF;
  float* sct = reinterpret_cast<float*>(smem + SC_OFF);
  float* red = reinterpret_cast<float*>(smem + RED_OFF);
  int32_t* idx_lds = reinterpret_cast<int32_t*>(smem + IDX_OFF);

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int lg = lane >> 4;
  const int lc = lane & 15;

  // workgroup x -> (token, head group, split): x = ((tq*S + split)*HG + hg)*8 + xcd, t = 8*tq + xcd
  const int HG = (p.H + 15) >> 4;
  const int S = DECODE ? p.num_splits : 1;
  const int64_t bx = blockIdx.x;
  const int64_t rest = bx / NXCD;
  const int hg = (int)(rest % HG);
  const int split = DECODE ? (int)((rest / HG) % S) : 0;
  const int64_t t = (rest / HG / S) * NXCD + bx % NXCD;
  if (t >= p.T) return;  // the last round of tokens may be short (whole workgroup)
  const int h0 = hg * 16;

  const ListEnds le = list_ends(p, t);
  const Sources src_lists = sources<false>(p);
  int64_t j_begin = 0, j_end = p.topk;
  if (DECODE) {
    j_begin = (int64_t)split * p.split_w;
    j_end = j_begin + p.split_w;
    if (j_end > p.topk) j_end = p.topk;
  }
  if (j_end > le.end) j_end = le.end;
  const int n_tiles = j_end > j_begin ? (int)((j_end - j_begin + TC - 1) / TC) : 0;

  // the token's q rows of heads h0..h0+15 into LDS (zeros past H); they
  // are visible after the first barrier below
  for (int qc = tid; qc < 16 * (dots3::D_QK / 8); qc += NT) {
    const int hl = qc / (dots3::D_QK / 8), piece = qc % (dots3::D_QK / 8);
    const int h = h0 + hl;
    uint4 v = make_uint4(0, 0, 0, 0);
    if (h < p.H) v = *reinterpret_cast<const uint4*>(p.q + t * p.q_st + (int64_t)h * p.q_sh + 8 * piece);
    *reinterpret_cast<uint4*>(qbuf + hl * Q_ROW + 16 * piece) = v;
  }
  // Q^T as the B operand of S^T = K Q^T: lane reads Q[h0+lc][32ks + 8lg + i]
  const uint8_t* qB = qbuf + lc * Q_ROW + 16 * lg;

  // slot of list position j_begin + 64k + tid, or -1
  auto load_idx = [&](int k) -> int32_t {
    const int64_t j = j_begin + (int64_t)k * TC + tid;
    int32_t v = -1;
    if (j < j_end && in_list<false>(p, le, j)) {
      const int32_t x = *entry_ptr<false>(src_lists, t, j);
      if (x >= 0 && (int64_t)x < p.nslots) v = x;
    }
    return v;
  };

  // thread tid gathers 16-byte pieces sub + 4r (r < NCH) of tile row
  // tid / 4, and the row's 8-byte tail when sub == 0
  const int grow = tid >> 2, sub = tid & 3;
  uint4 stage[NCH];
  uint2 tail;
  auto issue_rows = [&](int k) {
    const int32_t e = idx_lds[(k % 3) * TC + grow];
    if (e >= 0) {
      const uint8_t* row = p.pool + (int64_t)(e / PAGE) * p.block_stride + (int64_t)(e % PAGE) * p.row_stride;
#pragma unroll
      for (int r = 0; r < NCH; ++r) __builtin_memcpy(&stage[r], row + 16 * (sub + 4 * r), 16);
      tail = make_uint2(0, 0);
      if (sub == 0) __builtin_memcpy(&tail, row + 16 * PIECES, 8);
    } else {
#pragma unroll
      for (int r = 0; r < NCH; ++r) stage[r] = make_uint4(0, 0, 0, 0);
      tail = make_uint2(0, 0);
    }
  };
  auto store_rows = [&]() {
    uint8_t* dst = tile + grow * LDS_ROW;
#pragma unroll
    for (int r = 0; r < NCH; ++r) *reinterpret_cast<uint4*>(dst + 16 * (sub + 4 * r)) = stage[r];
    if (sub == 0) {  // the tail is the row's eight scale bytes: decode them once for the tile
      *reinterpret_cast<uint2*>(dst + 16 * PIECES) = tail;
      f32x4 lo, hi;
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        lo[g] = e8m0_to_f32((tail.x >> (8 * g)) & 0xFFu);
        hi[g] = e8m0_to_f32((tail.y >> (8 * g)) & 0xFFu);
      }
      reinterpret_cast<f32x4*>(sct + grow * dots3::NGROUPS)[0] = lo;
      reinterpret_cast<f32x4*>(sct + grow * dots3::NGROUPS)[1] = hi;
    }
  };

  // running max (log2 units) of head lc, shared by the four waves; this
  // lane's partial sum over its candidates; O^T for columns
  // 256*wave + 16dt + 4lg + i of head lc
  float m_run = -INFINITY;
  float l_part = 0.0f;
  f32x4 O[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) O[i] = f32x4{0.f, 0.f, 0.f, 0.f};

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
    if (k + 1 < n_tiles) issue_rows(k + 1);
    int32_t pend = -1;
    if (k + 2 < n_tiles && tid < TC) pend = load_idx(k + 2);

    // ---- S^T for candidates 16*wave + (0..15) x heads h0 + (0..15) ----
    const uint8_t* rowA = tile + (16 * wave + lc) * LDS_ROW;
    f32x4 acc[dots3::NGROUPS + 1];
#pragma unroll
    for (int g = 0; g <= dots3::NGROUPS; ++g) acc[g] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
#pragma unroll
      for (int g = 0; g < dots3::NGROUPS; ++g) {  // consecutive products go to different groups
        const int ks = 4 * g + kk;
        const uint2 c8 = *reinterpret_cast<const uint2*>(rowA + 32 * ks + 8 * lg);
        const uint2 lo = fp8x4_to_bf16x4(c8.x), hi = fp8x4_to_bf16x4(c8.y);
        const bf16x8 b = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(qB + 64 * ks));
        acc[g] = mfma_16x16x32(__builtin_bit_cast(bf16x8, make_uint4(lo.x, lo.y, hi.x, hi.y)), b, acc[g]);
      }
    }
#pragma unroll
    for (int ks = 32; ks < KS; ++ks) {
      const bf16x8 a = __builtin_bit_cast(
          bf16x8, *reinterpret_cast<const uint4*>(rowA + dots3::ROPE_OFF + 2 * (32 * (ks - 32) + 8 * lg)));
      const bf16x8 b = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(qB + 64 * ks));
      acc[dots3::NGROUPS] = mfma_16x16x32(a, b, acc[dots3::NGROUPS]);
    }

    // scores of candidates c = 16*wave + 4lg + i for head lc
    const int32_t* il = idx_lds + (k % 3) * TC + 16 * wave + 4 * lg;
    // scales of candidate (4lg+i), groups 0..3 and 4..7
    auto scales = [&](int i, int half) -> f32x4 {
      return reinterpret_cast<const f32x4*>(sct + (16 * wave + 4 * lg + i) * dots3::NGROUPS)[half];
    };
    float s[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const f32x4 lo = scales(i, 0), hi = scales(i, 1);
      float v = acc[dots3::NGROUPS][i];
#pragma unroll
      for (int g = 0; g < 4; ++g) v += lo[g] * acc[g][i] + hi[g] * acc[g + 4][i];
      s[i] = il[i] >= 0 ? v * p.scale_log2 : -INFINITY;
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
    if (__any(need)) {
      const float alpha = need ? ((m_run == -INFINITY) ? 0.0f : exp2f(m_run - mx)) : 1.0f;
      m_run = need ? mx : m_run;
      l_part *= alpha;
#pragma unroll
      for (int dt = 0; dt < 16; ++dt) O[dt] *= alpha;
    }
    float pr[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      pr[i] = (s[i] == -INFINITY) ? 0.0f : exp2f(s[i] - m_run);
      l_part += pr[i];
    }
    // P'_g[h][c] = P[c][h] * scale(c, g), candidates 16*wave + 4lg + (0..3)
#pragma unroll
    for (int g = 0; g < dots3::NGROUPS; ++g) {
      const float s0 = scales(0, g >> 2)[g & 3], s1 = scales(1, g >> 2)[g & 3];
      const float s2 = scales(2, g >> 2)[g & 3], s3 = scales(3, g >> 2)[g & 3];
      const uint32_t u0 = pack_bf16(pr[0] * s0, pr[1] * s1);
      const uint32_t u1 = pack_bf16(pr[2] * s2, pr[3] * s3);
      *reinterpret_cast<uint2*>(pbuf + g * P_GROUP + lc * P_HEAD + 2 * (16 * wave + 4 * lg)) = make_uint2(u0, u1);
    }
    __syncthreads();

    // ---- O^T += V^T P'^T over value columns [256*wave, +256) ----
    // tr8: lane lc = 2r + b reads candidate row (32kc + 8lg + r), byte
    // columns 8b..8b+7 of the 16-column block
#pragma unroll
    for (int kc = 0; kc < 2; ++kc) {
      const uint8_t* vbase = tile + (32 * kc + 8 * lg + (lc >> 1)) * LDS_ROW + 256 * wave + 8 * (lc & 1);
      bf16x8 pb[2];
#pragma unroll
      for (int gg = 0; gg < 2; ++gg)
        pb[gg] = __builtin_bit_cast(
            bf16x8, *reinterpret_cast<const uint4*>(pbuf + (2 * wave + gg) * P_GROUP + lc * P_HEAD + 2 * (32 * kc + 8 * lg)));
#pragma unroll
      for (int dt = 0; dt < 16; ++dt) {
        const i32x2 raw = lds_read_tr8(vbase + 16 * dt);
        const uint2 lo = fp8x4_to_bf16x4((uint32_t)raw[0]), hi = fp8x4_to_bf16x4((uint32_t)raw[1]);
        O[dt] = mfma_16x16x32(__builtin_bit_cast(bf16x8, make_uint4(lo.x, lo.y, hi.x, hi.y)), pb[dt >> 3], O[dt]);
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
  const float M = m_run;

  const int h = h0 + lc;
  if (h >= p.H) return;
  const bool empty = !(Lsum > 0.0f);
  const float lse_v = empty ? -INFINITY : (M + __log2f(Lsum)) * LN2;
  const int col = 256 * wave + 4 * lg;
  if constexpr (DECODE) {
    const float inv = empty ? 0.0f : 1.0f / Lsum;
    float* po = p.part_out + ((t * p.num_splits + split) * p.H + h) * (int64_t)dots3::D_V + col;
#pragma unroll
    for (int dt = 0; dt < 16; ++dt) *reinterpret_cast<f32x4*>(po + 16 * dt) = O[dt] * inv;
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
    for (int dt = 0; dt < 16; ++dt) {
      const f32x4 v = O[dt] * factor;
      *reinterpret_cast<uint2*>(orow + 16 * dt) = make_uint2(pack_bf16(v[0], v[1]), pack_bf16(v[2], v[3]));
    }
    if (wave == 0 && lg == 0) p.lse[t * p.lse_st + h] = lse_v;
  }
}

}  // namespace

hipError_t launch_attention_dots3(const AttnParams& p, bool decode, hipStream_t s) {
  const int64_t rounds = (p.T + NXCD - 1) / NXCD;
  const int64_t blocks = rounds * NXCD * ((p.H + 15) / 16) * (decode ? p.num_splits : 1);
  if (blocks > (int64_t)UINT32_MAX) return hipErrorInvalidConfiguration;
  dim3 block(NT);
  dim3 grid((unsigned)blocks);
  if (decode) hipLaunchKernelGGL((attn_dots3_kernel<true>), grid, block, 0, s, p);
  else hipLaunchKernelGGL((attn_dots3_kernel<false>), grid, block, 0, s, p);
  return hipGetLastError();
}

}  // namespace smla
