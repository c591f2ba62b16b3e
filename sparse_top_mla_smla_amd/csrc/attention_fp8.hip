// attention_fp8.hip -- sparse MLA attention for many heads (H > 16) over the
// quantized 656-byte paged latent rows: FP8 with power-of-two per-128 scales
// (DSv3.2, with or without rope dimensions), FP8 with arbitrary scales
// (GLM_NSA) and INT8 -- prefill form and split-KV decode partials.
//
// What is computed is stated in include/smla.h.  This kernel serves the
// shapes of the AppMana release note's fused prefill (T=1024, ctx 16384,
// H=64, widths 512/1024) and the decode batch: one workgroup owns one token
// (and split) for 64 heads, so each selected row is gathered from the pool
// once per token.
//
// DSv3.2 rows (FlashInfer #4802, KV layout of the decode kernel review) hold
// power-of-two FP32 scales.  Then code * scale is exact in BF16, and gfx950
// converts two e4m3 codes to BF16 with a power-of-two scale in a single
// v_cvt_scalef32_pk_bf16_fp8.  K is therefore dequantized exactly while it
// is converted, and the nope and rope parts of a score accumulate in one
// MFMA accumulator.  A valid row whose scale is not a positive power of two
// turns its token's output into NaN instead of a silently wrong result.
// Rows with arbitrary scales (FP8 amax/448, INT8 amax/127) convert their
// codes exactly with scale 1; a latent group's 128 nope columns are exactly
// one scale tile, so its partial score is multiplied by each candidate's
// scale of that tile before the rope product is added.
//
// QK uses v_mfma_f32_32x32x16_bf16, PV v_mfma_f32_32x32x16_f16 (P' in FP16
// keeps 11 significant bits of each weight against BF16's 8, at the same
// rate; the codes convert exactly to FP16 under the tile's bias).  Eight
// waves; wave w = g + 4hh
// works on latent group g (0..3) and head half hh (heads [32hh, 32hh+32)).
// Per 64-candidate tile:
//  1. QK^T, split over the latent dimension: wave (g, hh) forms the partial
//     S^T of all 64 candidates x its 32 heads over nope columns
//     [128g, 128g+128) and rope columns [16g, 16g+16), with its slice of Q
//     in registers for the whole token.
//  2. Reduce-scatter through LDS: wave (g, hh) owns candidates
//     [16g, 16g+16) of its heads and receives the three other groups'
//     partials for them.
//  3. Online softmax on the owned 16 x 32 block in the exp2 domain.  The
//     four waves of a head half exchange their block maxima, so they all
//     hold the same running max per head; it moves lazily (only when
//     exceeded by 2^8), so O is rarely rescaled.  P' goes to LDS in FP16
//     under the tile's exponent bias (f16_bias).
//  4. PV, split over output columns: wave (g, hh) accumulates O^T for
//     columns [128g, 128g+128) of its heads.  V^T is read from the raw codes
//     with ds_read_b64_tr_b8 and converted to FP16 times the tile's bias 2^b;
//     the row scale of column group g (a per-candidate factor) is folded
//     into P'.
// Raw tiles are double-buffered in LDS, chunk-major: 16-byte piece ck
// (0..40) of tile row r (0..63) sits at byte ck*1024 + r*16.  All eight
// waves gather the next tile straight from global memory with
// global_load_lds_dwordx4, one instruction per piece for all 64 rows
// (lane = row, landing at base + 16*lane), issued as soon as the tile
// before it is consumed; the index list runs one tile further ahead.  List
// positions without a candidate gather a zero row instead, so every LDS row
// of a tile belongs to the tile's own list: such a row has probability 0
// and value 0, and no data of another token's list (a non-finite row
// included) can reach this token's result.
#include <type_traits>

#include "device_common.h"
#include "launch.h"
#include "lists.h"

namespace smla {

namespace f8 {
typedef float f32x16 __attribute__((ext_vector_type(16)));

__device__ __forceinline__ f32x16 mfma_32x32x16(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// eight e4m3 codes (bytes of c0 then c1, in order) times a power-of-two scale
__device__ __forceinline__ bf16x8 cvt8(uint32_t c0, uint32_t c1, float scale) {
  const bf16x2 a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(c0, scale, false);
  const bf16x2 b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(c0, scale, true);
  const bf16x2 c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(c1, scale, false);
  const bf16x2 d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(c1, scale, true);
  return __builtin_bit_cast(bf16x8, make_uint4(__builtin_bit_cast(uint32_t, a), __builtin_bit_cast(uint32_t, b),
                                               __builtin_bit_cast(uint32_t, c), __builtin_bit_cast(uint32_t, d)));
}

__device__ __forceinline__ f32x16 mfma_32x32x16_f16(f16x8 a, f16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}

// eight e4m3 codes times a power-of-two scale as FP16 (see fp8x4_to_f16x4)
__device__ __forceinline__ f16x8 cvt8_f16(uint32_t c0, uint32_t c1, float scale) {
  const uint2 lo = fp8x4_to_f16x4(c0, scale), hi = fp8x4_to_f16x4(c1, scale);
  return __builtin_bit_cast(f16x8, make_uint4(lo.x, lo.y, hi.x, hi.y));
}

// eight codes of the given row format as BF16: e4m3 times a power-of-two
// scale (exact), or int8 (exact, |code| <= 127; the scale is applied later)
template <int CODES>
__device__ __forceinline__ bf16x8 codes8(uint32_t c0, uint32_t c1, float scale) {
  if constexpr (CODES == FMT_INT8) {
    const uint2 lo = int8x4_to_bf16x4(c0), hi = int8x4_to_bf16x4(c1);
    return __builtin_bit_cast(bf16x8, make_uint4(lo.x, lo.y, hi.x, hi.y));
  } else {
    return cvt8(c0, c1, scale);
  }
}

__device__ __forceinline__ void global_to_lds_16(const void* src, void* lds_wave_base) {
  __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)src,
                                   (__attribute__((address_space(3))) void*)lds_wave_base, 16, 0, 0);
}

__device__ __forceinline__ void global_to_lds_4(const void* src, void* lds_wave_base) {
  __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)src,
                                   (__attribute__((address_space(3))) void*)lds_wave_base, 4, 0, 0);
}

// Workgroup barrier for LDS traffic only: this wave's LDS reads and writes
// are complete, and no LDS access moves across it.  Unlike __syncthreads it
// does not wait for outstanding global loads, so the direct-to-LDS gather
// of the next tile stays in flight (that buffer is not touched until the
// full barrier at the top of the next tile).
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// 32-bit LDS address of a pointer into __shared__ memory
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

// ds_read_b64_tr_b8 issued through asm.  The builtin's memory operand has
// no alias information, so the compiler would make it wait for every
// outstanding direct-to-LDS gather; here the caller waits explicitly
// (lgkm_wait) before the results are used.  LDS operations complete in
// order, so the compiler's own lgkmcnt waits stay correct around these.
template <int OFF>
__device__ __forceinline__ i32x2 tr8_issue(uint32_t addr) {
  i32x2 r;
  asm volatile("ds_read_b64_tr_b8 %0, %1 offset:%2" : "=v"(r) : "v"(addr), "i"(OFF));
  return r;
}
// ds_read_b64_tr_b16 likewise: in each 16-lane group, lane 4r + b
// addresses row r of a 4-row block, BF16 columns 4b..4b+3 of a 16-column
// block; lane l then holds column l of the 4 rows
template <int OFF>
__device__ __forceinline__ i32x2 tr16_issue(uint32_t addr) {
  i32x2 r;
  asm volatile("ds_read_b64_tr_b16 %0, %1 offset:%2" : "=v"(r) : "v"(addr), "i"(OFF));
  return r;
}
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
// ds_write_b64 through asm, for the same reason; the LDS barrier that
// follows waits for its completion
template <int OFF>
__device__ __forceinline__ void b64_store(uint32_t addr, u32x2 v) {
  asm volatile("ds_write_b64 %0, %1 offset:%2" : : "v"(addr), "v"(v), "i"(OFF));
}
template <int OFF>
__device__ __forceinline__ u32x4 b128_issue(uint32_t addr) {
  u32x4 r;
  asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(r) : "v"(addr), "i"(OFF));
  return r;
}

// a positive, finite, normal power of two
__device__ __forceinline__ bool is_pow2_scale(float s) {
  const uint32_t b = __builtin_bit_cast(uint32_t, s);
  const uint32_t e = b >> 23;
  return (b & 0x007FFFFFu) == 0 && e != 0 && e < 255;
}

constexpr int NT = 512;                      // 8 waves, 2 per SIMD
constexpr int TC = 64;                       // candidates per tile
constexpr int RB = 656;                      // row bytes
constexpr int CHUNKS = RB / 16;              // 41 pieces of 16 bytes per row
constexpr int CS = TC * 16;                  // bytes of one piece column (64 rows)
constexpr int TILE = CHUNKS * CS;            // 41,984 bytes per tile
constexpr int CK_SCALE = D_NOPE / 16;        // piece 32 holds the four scales
constexpr int CK_ROPE = CK_SCALE + 1;        // pieces 33..40 hold the rope
constexpr int GPARTS = 3;                    // the pieces are issued in three parts per tile
// DSv4 rows (584 bytes, 8-byte aligned in the pool): pieces 0..27 hold the
// 448 e4m3 codes (piece p: values 16p..16p+15, scale tile p/4), pieces
// 28..35 the 64 BF16 rope values (piece 28 + q: values 8q..8q+7), and piece
// 36 is row bytes 568..583, whose bytes 8..14 are the seven scale bytes.
namespace v4 {
constexpr int CHUNKS = 37;
constexpr int CK_ROPE = 28;
constexpr int CK_TAIL = 36;
constexpr int TAIL_FROM = 568;               // row byte where piece 36 starts
constexpr int TILE = CHUNKS * CS;            // 37,888 bytes per tile
static_assert(CK_TAIL - CK_ROPE == NT / 64, "one rope piece per wave for the FP16 conversion");
}  // namespace v4
template <int CODES>
constexpr int chunks_of() { return CODES == FMT_FP8_DSV4 ? v4::CHUNKS : CHUNKS; }
constexpr int RECV_FLOATS = 8 * 3 * 2 * 64 * 4;  // [8 owners][3 senders][2][64 lanes][4] f32
constexpr int PS = 72;                       // P' row stride (16-bit): [4 groups][64 heads][PS], aliases recv
static_assert(4 * 64 * PS * 2 <= RECV_FLOATS * 4, "P' must fit in the partial-exchange buffer");
constexpr int GS = 64 * PS * 2;              // bytes of one P' group slot
// DSv4 rows keep eight P' versions (seven scale tiles and the rope columns)
constexpr int RECV_FLOATS_8 = 8 * GS / 4;
static_assert(RECV_FLOATS_8 >= RECV_FLOATS, "the eight-slot buffer holds the partial exchange");
constexpr float TAU = 8.0f;

template <int V>
struct Buf {
  static constexpr int value = V;
};

// the rows that list positions without a candidate gather (one copy per
// device): zero codes and rope values; the 656-byte rows' four scales are
// 2^-126, a positive power of two (so the row's scores are 0, not NaN) and
// no larger than any real row's scale (so it never raises a tile's FP16
// bias).  The DSv4 rows' scale bytes are 0.
struct ZeroRow {
  uint32_t w[RB / 4];
};
constexpr ZeroRow make_zero_row(bool scales) {
  ZeroRow r{};
  if (scales)
    for (int i = 0; i < 4; ++i) r.w[D_NOPE / 4 + i] = 0x00800000u;
  return r;
}
__device__ __attribute__((aligned(16))) ZeroRow zero_row_656 = make_zero_row(true);
__device__ __attribute__((aligned(16))) ZeroRow zero_row_584 = make_zero_row(false);

// an exponent byte as the FP32 number 2^(b-127) (0: 2^-127, 255: NaN)
__device__ __forceinline__ float e8m0_value(uint32_t b) {
  return __builtin_bit_cast(float, b == 0u ? 0x00400000u : (b == 255u ? 0x7FC00000u : b << 23));
}
// the scale v_cvt_scalef32_pk_bf16_fp8 applies for exponent byte b: the
// instruction reads only the scale's exponent, so byte 0 converts as 2^-126
// (the writer stores 1..254; a 0 byte only doubles values below 2^-118)
__device__ __forceinline__ float e8m0_cvt_scale(uint32_t b) {
  return __builtin_bit_cast(float, (b == 0u ? 1u : b) << 23);
}
}  // namespace f8

// NOPE: rows without rope dimensions (q rows of 512 values, row padding never
// gathered or read).  CODES: FMT_FP8 (power-of-two scales, applied while
// converting), FMT_FP8_ANY or FMT_INT8 (arbitrary scales: the codes convert
// exactly with scale 1, each latent group's partial score is multiplied by
// its candidates' scales before the rope part is added, and P' folds the
// scales into PV as for FMT_FP8), or FMT_FP8_DSV4 (the 584-byte rows: 512
// key and value dimensions, 448 of them e4m3 codes with a power-of-two
// scale per 64, then 64 BF16 rope values; latent group 3 holds the last
// 64 codes and the rope, and P' has eight versions, one per scale tile and
// one for the rope columns).
template <bool DECODE, bool DUAL, bool NOPE, int CODES>
__global__ __launch_bounds__(f8::NT, 1) void attn_fp8_kernel(AttnParams p) {
  using namespace f8;
  // Separate LDS objects, and a loop unrolled by two so that every access
  // names its raw buffer at compile time: the compiler then sees that reads
  // of one buffer (and of the other arrays) do not alias the direct-to-LDS
  // gather into the other buffer, and does not wait for that gather.
  constexpr bool DS = CODES == FMT_FP8_DSV4;                          // DSv4 rows
  constexpr bool ARB = CODES == FMT_FP8_ANY || CODES == FMT_INT8;     // arbitrary scales
  constexpr int NCK = chunks_of<CODES>();                             // pieces per row
  constexpr int RAW = NCK * CS;                                       // bytes per raw tile
  __shared__ __attribute__((aligned(16))) uint8_t raw0[RAW];
  __shared__ __attribute__((aligned(16))) uint8_t raw1[RAW];
  __shared__ __attribute__((aligned(16))) float recv[DS ? RECV_FLOATS_8 : RECV_FLOATS];
  __shared__ __attribute__((aligned(16))) float maxb[4 * 64];   // [4 groups][64 heads]
  // DSv4: the tile's scales, [scale tile][row] (2^(b-127))
  __shared__ __attribute__((aligned(16))) float dsc[DS ? 7 * TC : 4];
  // [buffer][row]: 0 for a row that holds a candidate, -inf for a position without one
  __shared__ __attribute__((aligned(16))) float rowbias[2 * TC];
  __shared__ __attribute__((aligned(16))) int32_t idx0[TC];       // index list of even tiles
  __shared__ __attribute__((aligned(16))) int32_t idx1[TC];       // index list of odd tiles
  uint16_t* pq = reinterpret_cast<uint16_t*>(recv);              // P' (FP16), after the reduce

  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform, kept in SGPRs
  const int g = w & 3, hh = w >> 2;
  const int lane = tid & 63;
  const int l32 = lane & 31;
  const int hi = lane >> 5;

  const int h0 = blockIdx.y * 64;
  // decode: this workgroup covers splits [sp0, sp_end) of token blockIdx.x
  // as one list, with a partial result at the end of each split
  const int sp0 = DECODE ? (int)blockIdx.z * p.splits_per_block : 0;
  const int sp_end = DECODE ? min(sp0 + p.splits_per_block, p.num_splits) : 1;
  const int32_t t_stride = gridDim.x;
  const Sources src_lists = sources<DUAL>(p);

  // token tt's list lengths (read through the scalar cache: a vector load
  // would make the wait for it also wait for the gathers in flight)
  auto token_lists = [&](int32_t tt) -> ListEnds {
    int32_t l1 = p.topk, l2 = 0;
    if (p.topk_length) l1 = clamp_len(*(const __attribute__((address_space(4))) int32_t*)(p.topk_length + tt), p.topk);
    if constexpr (DUAL) {
      l2 = p.topk2;
      if (p.topk_length2) l2 = clamp_len(*(const __attribute__((address_space(4))) int32_t*)(p.topk_length2 + tt), p.topk2);
    }
    return list_ends_of(p, l1, l2);
  };
  // A tile is list positions [j0, j0 + 64) of token t, cut at jend, with
  // the main list's length l1 (positions [l1, topk) hold no candidate; t < 0:
  // no tile; T and the list widths fit in 31 bits).  Prefill: the workgroup takes tokens blockIdx.x,
  // blockIdx.x + gridDim.x, ... and its tile pipeline (gather one tile
  // ahead, index list two tiles ahead) runs on across token boundaries, so
  // no token pays for filling it.  Decode: the tiles of one token's split
  // range.
  struct TileRef {
    int32_t t, j0, jend, l1;
  };
  // (values are built field by field, never chosen between two objects, so
  // the references stay in registers)
  auto first_tile = [&](int32_t t0) -> TileRef {
    TileRef r{-1, 0, 0, 0};
    if (DECODE) {
      const ListEnds le = token_lists(t0);
      const int64_t jb = (int64_t)sp0 * p.split_w;
      int64_t je = (int64_t)sp_end * p.split_w;
      const int64_t topk_all = DUAL ? (int64_t)p.topk + p.topk2 : (int64_t)p.topk;
      if (je > topk_all) je = topk_all;
      if (je > le.end) je = le.end;
      if (je > jb) {
        r.t = t0;
        r.j0 = (int32_t)jb;
        r.jend = (int32_t)je;
        r.l1 = le.l1;
      }
      return r;
    }
    for (int32_t tt = t0; tt < p.T; tt += t_stride) {
      const ListEnds le = token_lists(tt);
      if (le.end > 0) {
        r.t = tt;
        r.j0 = (DUAL && le.l1 == 0) ? p.topk : 0;
        r.jend = le.end;
        r.l1 = le.l1;
        break;
      }
    }
    return r;
  };
  // Prefill skips the positions between the main list's length and the
  // secondary list; decode keeps its tiles contiguous, so split ends fall
  // on tile counts (a skipped range holds no candidate either way).
  auto advance = [&](TileRef r) -> TileRef {
    if (r.t < 0) return r;
    int32_t nj = r.j0 + TC;
    if (DUAL && !DECODE && nj >= r.l1 && nj < p.topk) nj = p.topk;
    if (nj < r.jend) {
      r.j0 = nj;
      return r;
    }
    if (DECODE) {
      r.t = -1;
      return r;
    }
    return first_tile(r.t + t_stride);
  };
  // list position j of tile r holds a candidate position
  auto in_tile = [&](TileRef r, int32_t j) -> bool { return j < r.jend && (!DUAL || j < r.l1 || j >= p.topk); };

  // wave 0 moves the index list entries of tile r into index buffer B
  // (positions without a candidate are not loaded; readers check them)
  auto issue_idx = [&](auto buf, const TileRef& r) {
    constexpr int B = decltype(buf)::value;
    const int32_t j = r.j0 + lane;
    if (in_tile(r, j)) global_to_lds_4(entry_ptr<DUAL>(src_lists, r.t, j), B ? idx1 : idx0);
  };
  // wave w moves pieces w, w + 8, ... of all 64 rows of a tile (lane = row)
  // into raw buffer B, in part P (0..2) the pieces of rounds 2P and 2P + 1.
  // Spreading the issue over the tile keeps the address unit's queue short,
  // so no wave stalls long at issue.  A lane without a candidate (src null)
  // moves the zero row.  Wave 0 records which rows hold candidates.
  auto issue_part = [&](auto buf, auto part, const uint8_t* src) {
    constexpr int B = decltype(buf)::value;
    constexpr int P = decltype(part)::value;
    uint8_t* raw = B ? raw1 : raw0;
    const uint8_t* from = src ? src : reinterpret_cast<const uint8_t*>(DS ? zero_row_584.w : zero_row_656.w);
#pragma unroll
    for (int r = 2 * P; r < 2 * P + 2; ++r) {
      const int ck = w + 8 * r;
      // (rows without rope dimensions: their padding is not gathered; the
      // DSv4 row's last piece starts 8 bytes early, inside the row)
      if ((8 * r + 7 < NCK || ck < NCK) && (!NOPE || ck < CK_ROPE))
        global_to_lds_16(from + (DS && ck == v4::CK_TAIL ? v4::TAIL_FROM : 16 * ck), raw + ck * CS);
    }
    if (P == 0 && w == 0) rowbias[B * TC + lane] = src ? 0.0f : -INFINITY;
  };
  static_assert(2 * GPARTS * 8 >= NCK && 2 * (GPARTS - 1) * 8 < NCK, "three parts of two rounds");

  // Q as the B operand of S^T = K Q^T for head h0 + 32hh + l32.  A K lane
  // reads one 16-byte piece (8g + 2j + hi) that feeds MFMA steps 2j and
  // 2j+1, so qn[2j + b] holds nope columns 128g + 32j + 16hi + 8b + i; qr
  // holds rope columns 16g + 8hi + i.
  bf16x8 qn[8], qr;
  auto load_q = [&](int32_t tq) {
    const int h = h0 + 32 * hh + l32;
    const bool hv = h < p.H;
    const uint16_t* qrow = p.q + (int64_t)tq * p.q_st + (int64_t)(hv ? h : 0) * p.q_sh;
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int b = 0; b < 2; ++b) {
        // loaded for every lane (row 0 stands in for heads past H) and
        // zeroed after, so the loads are unconditional
        const uint4 v = *reinterpret_cast<const uint4*>(qrow + 128 * g + 32 * j + 16 * hi + 8 * b);
        qn[2 * j + b] = __builtin_bit_cast(bf16x8, hv ? v : make_uint4(0, 0, 0, 0));
      }
    // (rows without rope dimensions: q rows end at 512 and the rope slice is
    // 0; DSv4 q rows end at 512 too, their rope values are columns 448..511
    // of latent group 3, loaded above)
    if constexpr (NOPE || DS) {
      qr = __builtin_bit_cast(bf16x8, make_uint4(0, 0, 0, 0));
    } else {
      const uint4 v = *reinterpret_cast<const uint4*>(qrow + D_NOPE + 16 * g + 8 * hi);
      qr = __builtin_bit_cast(bf16x8, hv ? v : make_uint4(0, 0, 0, 0));
    }
  };

  TileRef cur = first_tile((int32_t)blockIdx.x);
  TileRef nxt = advance(cur);
  TileRef nn = advance(nxt);
  // the first tile's index entries (an unconditional load of an entry
  // inside the range, selected after), then Q: the compiler barrier keeps
  // the Q loads behind the wait for the entries, so they are in flight
  // during the first gather instead of delaying its issue
  const uint8_t* src0 = nullptr;
  if (cur.t >= 0) {
    const int32_t j = cur.j0 + lane;
    const int32_t x = *entry_ptr<DUAL>(src_lists, cur.t, j < cur.jend ? j : cur.jend - 1);
    src0 = in_tile(cur, j) ? row_of<DUAL>(src_lists, j, x) : nullptr;
  }
  asm volatile("" ::: "memory");
  if (cur.t >= 0) load_q(cur.t);

  // sink of head h0 + 32hh + l32 in exp2 units (prefill), loaded once
  float sink2 = 0.0f;

  // softmax state for heads 32hh + l32 (identical in the four waves of hh)
  float m_run = -INFINITY;
  float l_part = 0.0f;  // this wave's share: candidates 16g.. of every tile
  int o_k = 0;          // P, l and O are taken relative to 2^(m_run + o_k) (see f16_bias)
  // O^T accumulators: columns [128g + 32dt, +32) x heads [32hh, +32)
  f32x16 O[4];
#pragma unroll
  for (int dt = 0; dt < 4; ++dt)
#pragma unroll
    for (int i = 0; i < 16; ++i) O[dt][i] = 0.0f;

  // A finished result (a split's partial, or a token's output) whose O is
  // kept in registers is stored by the next tile, after that tile's gather
  // is issued, so the stores drain during a tile instead of inside its
  // first wait.
  int32_t pend = -1;  // split (decode) or token (prefill) still to be stored
  float pend_factor = 0.0f, pend_lse = 0.0f;
  // Decode, the workgroup's last split (no gather in flight, every wave past
  // its last PV, so the raw tile buffers are free): each wave stages its
  // 32 heads x 128 columns in LDS, 64 columns at a time, and stores whole
  // 256-byte row pieces of 4 heads per instruction instead of 32-byte
  // pieces of 32 heads.
  auto store_partial_staged = [&](int32_t key, float factor) {
    constexpr int SROW = 68;  // floats per staged head row (64 + 4 pad)
    static_assert(4 * 32 * SROW * 4 <= RAW, "four waves' staging fits one raw buffer");
    float* st = reinterpret_cast<float*>(w < 4 ? raw0 : raw1) + (w & 3) * 32 * SROW;
    const int64_t td = blockIdx.x;
    float* pbase = p.part_out + ((td * p.num_splits + key) * p.H + h0 + 32 * hh) * (int64_t)D_V + 128 * g;
    const int rh = lane >> 4;       // head offset of this lane's reads
    const int rc = 4 * (lane & 15); // column of this lane's reads
    // (LDS accesses of one wave complete in order, so each read sees the
    // writes before it, and the next half's writes follow those reads)
    auto put = [&](const f32x16& o, int d) {
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4)
        *reinterpret_cast<f32x4*>(st + l32 * SROW + 32 * d + 8 * q4 + 4 * hi) =
            f32x4{o[4 * q4] * factor, o[4 * q4 + 1] * factor, o[4 * q4 + 2] * factor, o[4 * q4 + 3] * factor};
    };
    auto drain = [&](int half) {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int hl = 4 * i + rh;
        const f32x4 v = *reinterpret_cast<const f32x4*>(st + hl * SROW + rc);
        if (h0 + 32 * hh + hl < p.H) *reinterpret_cast<f32x4*>(pbase + (int64_t)hl * D_V + 64 * half + rc) = v;
      }
    };
    put(O[0], 0);
    put(O[1], 1);
    drain(0);
    put(O[2], 0);
    put(O[3], 1);
    drain(1);
  };
  auto store_result = [&](int32_t key, float factor, float lse_v, bool staged) {
    if constexpr (DECODE) {
      if (staged) {
        store_partial_staged(key, factor);
        const int h = h0 + 32 * hh + l32;
        if (g == 0 && hi == 0 && h < p.H) p.part_lse[((int64_t)blockIdx.x * p.num_splits + key) * p.H + h] = lse_v;
        return;
      }
    }
    const int h = h0 + 32 * hh + l32;
    if (h >= p.H) return;
    if constexpr (DECODE) {
      const int64_t td = blockIdx.x;
      float* po = p.part_out + ((td * p.num_splits + key) * p.H + h) * (int64_t)D_V + 128 * g + 4 * hi;
#pragma unroll
      for (int dt = 0; dt < 4; ++dt)
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4)
          *reinterpret_cast<f32x4*>(po + 32 * dt + 8 * q4) =
              f32x4{O[dt][4 * q4] * factor, O[dt][4 * q4 + 1] * factor, O[dt][4 * q4 + 2] * factor,
                    O[dt][4 * q4 + 3] * factor};
      if (g == 0 && hi == 0) p.part_lse[(td * p.num_splits + key) * p.H + h] = lse_v;
    } else {
      uint16_t* orow = p.out + (int64_t)key * p.out_st + (int64_t)h * p.out_sh + 128 * g + 4 * hi;
#pragma unroll
      for (int dt = 0; dt < 4; ++dt)
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4)
          *reinterpret_cast<uint2*>(orow + 32 * dt + 8 * q4) =
              make_uint2(pack_bf16(O[dt][4 * q4] * factor, O[dt][4 * q4 + 1] * factor),
                         pack_bf16(O[dt][4 * q4 + 2] * factor, O[dt][4 * q4 + 3] * factor));
      if (g == 0 && hi == 0) p.lse[(int64_t)key * p.lse_st + h] = lse_v;
    }
  };

  // prefill: the workgroup's tokens with an empty list (O is still zero)
  if (!DECODE && p.topk_length) {
    for (int32_t tt = blockIdx.x; tt < p.T; tt += t_stride)
      if (token_lists(tt).end == 0) store_result(tt, 0.0f, -INFINITY, false);
  }

  if (cur.t >= 0) {
    issue_part(Buf<0>{}, Buf<0>{}, src0);
    issue_part(Buf<0>{}, Buf<1>{}, src0);
    issue_part(Buf<0>{}, Buf<2>{}, src0);
    if (w == 0 && nxt.t >= 0) issue_idx(Buf<1>{}, nxt);
    // the sink, in flight beside the first gather
    if (!DECODE && p.sink) {
      const int h = h0 + 32 * hh + l32;
      sink2 = (h < p.H ? p.sink[h] : 0.0f) * LOG2E;
    }
  }

  // one tile (cur) in raw buffer B; nxt is gathered into the other buffer
  // meanwhile, and nn's index list is fetched into index buffer B
  auto step = [&](auto buf, const TileRef& cur, const TileRef& nxt, const TileRef& nn) {
    constexpr int B = decltype(buf)::value;
    const uint8_t* raw = B ? raw1 : raw0;
    __builtin_amdgcn_s_waitcnt(0);  // this wave's part of the tile has landed
    __syncthreads();                // B0: all of the tile is in LDS; the one before is consumed
    // gather of the next tile (its index list arrived before B0), then the
    // index list one tile further ahead, read after the next B0
    const bool more = nxt.t >= 0;
    const uint8_t* src_next = nullptr;
    if (more) {
      const int32_t j = nxt.j0 + lane;
      src_next = in_tile(nxt, j) ? row_of<DUAL>(src_lists, j, (B ? idx0 : idx1)[lane]) : nullptr;
      issue_part(Buf<1 - B>{}, Buf<0>{}, src_next);
    }
    if (w == 0 && nn.t >= 0) issue_idx(Buf<B>{}, nn);
    // PV runs in FP16 under the tile's bias (f16_bias), taken after QK: the
    // largest exponent of the 64 rows' scales (DSv4: of their seven exponent
    // bytes; DSv4's BF16 rope values enter PV as FP16 unbiased)
    F16Bias bias;
    if (pend >= 0) {
      store_result(pend, pend_factor, pend_lse, false);
      pend = -1;
#pragma unroll
      for (int dt = 0; dt < 4; ++dt)
#pragma unroll
        for (int i = 0; i < 16; ++i) O[dt][i] = 0.0f;
    }
  // ---- 1. partial S^T (exact dequantized K) for candidates 32c2 + m ----
    f32x16 acc[2];
#pragma unroll
    for (int c2 = 0; c2 < 2; ++c2) {
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[c2][i] = 0.0f;
      const int row = 32 * c2 + l32;
      if constexpr (DS) {
        // DSv4: this wave's 128 key columns are codes of scale tiles 2g and
        // 2g + 1 (group 3: the codes of tile 6, then the 64 BF16 rope
        // values).  The row's scale bytes are bytes 8..14 of piece 36; a
        // byte 255 (NaN) makes the row's scores NaN for every head, as a bad
        // scale does for the 656-byte rows.
        const uint2 tb = *reinterpret_cast<const uint2*>(raw + v4::CK_TAIL * CS + row * 16 + 8);
        const int t0 = 2 * g, t1 = g < 3 ? 2 * g + 1 : 2 * g;
        const uint32_t b0 = ((t0 < 4 ? tb.x : tb.y) >> (8 * (t0 & 3))) & 0xFFu;
        const uint32_t b1 = ((t1 < 4 ? tb.x : tb.y) >> (8 * (t1 & 3))) & 0xFFu;
        const float s0c = e8m0_cvt_scale(b0), s1c = e8m0_cvt_scale(b1);
        const bool bad = b0 == 255u || b1 == 255u;
        // the exact scales, for P' (read after the next barrier): lanes
        // hi = 0 write tile t0, lanes hi = 1 tile t1 (group 3: tile 6 only)
        if (g < 3 || hi == 0) dsc[(hi ? t1 : t0) * TC + row] = e8m0_value(hi ? b1 : b0);
        const uint8_t* kp = raw + (8 * g + hi) * CS + row * 16;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          if (g < 3 || j < 2) {
            // e4m3 codes: key columns 128g + 32j + 16hi + 8b + i, scale tile 2g + j/2
            const uint4 c16 = *reinterpret_cast<const uint4*>(kp + 2 * j * CS);
            const float sc = j < 2 ? s0c : s1c;
            bf16x8 k0 = cvt8(c16.x, c16.y, sc);
            if (j == 0 && bad) k0 = __builtin_bit_cast(bf16x8, make_uint4(0x7FC07FC0u, 0x7FC07FC0u, 0x7FC07FC0u, 0x7FC07FC0u));
            acc[c2] = mfma_32x32x16(k0, qn[2 * j], acc[c2]);
            acc[c2] = mfma_32x32x16(cvt8(c16.z, c16.w, sc), qn[2 * j + 1], acc[c2]);
          } else {
            // group 3, BF16 rope values 32(j - 2) + 16hi + 8b + i (key
            // columns 384 + 32j + 16hi + 8b + i) in piece 28 + 4(j - 2) + 2hi + b
            const uint8_t* rp = raw + (v4::CK_ROPE + 4 * (j - 2) + 2 * hi) * CS + row * 16;
            acc[c2] = mfma_32x32x16(__builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(rp)), qn[2 * j], acc[c2]);
            acc[c2] = mfma_32x32x16(__builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(rp + CS)), qn[2 * j + 1],
                                    acc[c2]);
          }
        }
      } else {
        // power-of-two scales: applied while converting.  A scale that is
        // not a positive power of two makes this row's rope operand NaN: the
        // row's scores become NaN for every head (rows that are not loaded
        // are masked out by selection later)
        const float sc = CODES == FMT_FP8 ? *reinterpret_cast<const float*>(raw + CK_SCALE * CS + row * 16 + 4 * g) : 1.0f;
        const bool bad = CODES == FMT_FP8 && !is_pow2_scale(sc);
        const uint8_t* kp = raw + (8 * g + hi) * CS + row * 16;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const uint4 c16 = *reinterpret_cast<const uint4*>(kp + 2 * j * CS);
          acc[c2] = mfma_32x32x16(codes8<CODES>(c16.x, c16.y, sc), qn[2 * j], acc[c2]);
          acc[c2] = mfma_32x32x16(codes8<CODES>(c16.z, c16.w, sc), qn[2 * j + 1], acc[c2]);
        }
        if constexpr (ARB) {
          // arbitrary scales: accumulator element 4a + b is candidate
          // 32c2 + 8a + 4hi + b, whose scale of group g is read here
          const uint8_t* sp = raw + CK_SCALE * CS + (32 * c2 + 4 * hi) * 16 + 4 * g;
#pragma unroll
          for (int a = 0; a < 4; ++a)
#pragma unroll
            for (int b = 0; b < 4; ++b) acc[c2][4 * a + b] *= *reinterpret_cast<const float*>(sp + (8 * a + b) * 16);
        }
        uint4 r16 = make_uint4(0, 0, 0, 0);  // rows without rope dimensions: 0
        if constexpr (!NOPE) r16 = *reinterpret_cast<const uint4*>(raw + (CK_ROPE + 2 * g + hi) * CS + row * 16);
        if (bad) r16 = make_uint4(0x7FC07FC0u, 0x7FC07FC0u, 0x7FC07FC0u, 0x7FC07FC0u);
        acc[c2] = mfma_32x32x16(__builtin_bit_cast(bf16x8, r16), qr, acc[c2]);
      }
    }
    // the tile's FP16 bias from row lane's scales (DSv4: exponent bytes),
    // formed while the QK MFMAs finish
    {
      const uint4 sc4 = DS ? make_uint4(0, 0, 0, 0) : *reinterpret_cast<const uint4*>(raw + CK_SCALE * CS + lane * 16);
      const uint2 tb = DS ? *reinterpret_cast<const uint2*>(raw + v4::CK_TAIL * CS + lane * 16 + 8) : make_uint2(0, 0);
      bias = f16_bias(wave_max_u32(DS ? max_byte<7>(tb.x, tb.y)
                                      : max(max((sc4.x >> 23) & 0xFFu, (sc4.y >> 23) & 0xFFu),
                                            max((sc4.z >> 23) & 0xFFu, (sc4.w >> 23) & 0xFFu))),
                      CODES == FMT_INT8 ? 5 : 7);
    }
    // prefill: Q of the next token, not read again before that token's QK
    if (!DECODE && more && nxt.t != cur.t) load_q(nxt.t);
    // ---- 2. reduce-scatter: accumulator elements [8hf, 8hf+8) of tile c2
    // are candidates 32c2 + 16hf + 8(i/4) + 4hi + i%4, owned by wave
    // (2c2 + hf, hh) ----
    f32x4 s0, s1;  // own candidates 16g + 4hi + r and 16g + 8 + 4hi + r
#pragma unroll
    for (int c2 = 0; c2 < 2; ++c2)
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
        const int og = 2 * c2 + hf;
        const f32x4 a = f32x4{acc[c2][8 * hf + 0], acc[c2][8 * hf + 1], acc[c2][8 * hf + 2], acc[c2][8 * hf + 3]};
        const f32x4 b = f32x4{acc[c2][8 * hf + 4], acc[c2][8 * hf + 5], acc[c2][8 * hf + 6], acc[c2][8 * hf + 7]};
        if (og == g) {
          s0 = a;
          s1 = b;
        } else {
          const int slot = g < og ? g : g - 1;
          f32x4* dst = reinterpret_cast<f32x4*>(recv) + ((og + 4 * hh) * 3 + slot) * 128 + lane;
          dst[0] = a;
          dst[64] = b;
        }
      }
    lds_barrier();  // B1: partials visible
    if (more) issue_part(Buf<1 - B>{}, Buf<1>{}, src_next);

    {
      // all the reads first, then one wait
      const f32x4* src = reinterpret_cast<const f32x4*>(recv) + w * 3 * 128 + lane;
      f32x4 part[3][2];
#pragma unroll
      for (int slot = 0; slot < 3; ++slot) {
        part[slot][0] = src[slot * 128];
        part[slot][1] = src[slot * 128 + 64];
      }
      const float* vl = rowbias + B * TC + 16 * g + 4 * hi;
      const f32x4 va = *reinterpret_cast<const f32x4*>(vl), vb = *reinterpret_cast<const f32x4*>(vl + 8);
      // DSv4: wave w's piece of the BF16 rope values (piece 28 + w), which QK
      // has read as K by now, goes back as FP16 for PV
      uint8_t* rope = (B ? raw1 : raw0) + (v4::CK_ROPE + w) * CS + lane * 16;
      const uint4 r16 = DS ? *reinterpret_cast<const uint4*>(rope) : make_uint4(0, 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
      if constexpr (DS)
        *reinterpret_cast<uint4*>(rope) = make_uint4(bf16x2_to_f16x2(r16.x), bf16x2_to_f16x2(r16.y),
                                                     bf16x2_to_f16x2(r16.z), bf16x2_to_f16x2(r16.w));
#pragma unroll
      for (int slot = 0; slot < 3; ++slot) {
        s0 += part[slot][0];
        s1 += part[slot][1];
      }
      // positions without a candidate hold the zero row, whose score is 0:
      // adding -inf masks them
      float mx = -INFINITY;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        s0[r] = fmaf(s0[r], p.scale_log2, va[r]);
        s1[r] = fmaf(s1[r], p.scale_log2, vb[r]);
        mx = fmaxf(mx, fmaxf(s0[r], s1[r]));
      }
      {
        // the other half of the wave: v_permlane32_swap gives the low half's
        // values in one result and the high half's in the other, in all lanes
        // (both results are copied out before they are reinterpreted: a bit
        // cast applied to the second element of the builtin's result in place
        // is compiled as a cast of the first)
        const auto sw = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(uint32_t, mx), __builtin_bit_cast(uint32_t, mx), false, false);
        const uint32_t lo = sw[0], hi2 = sw[1];
        mx = fmaxf(__builtin_bit_cast(float, lo), __builtin_bit_cast(float, hi2));
      }
      if (hi == 0) maxb[g * 64 + 32 * hh + l32] = mx;
    }
    lds_barrier();  // B2: block maxima visible; every partial has been read
    if (more) issue_part(Buf<1 - B>{}, Buf<2>{}, src_next);

    float alpha;
    // 656-byte rows: the row scales for P' are read now, behind the block
    // maxima, so that their latency passes under the softmax
    f32x4 sc0[4], sc1[4];
    {
      const int hl = 32 * hh + l32;
      const float m0 = maxb[hl], m1 = maxb[64 + hl], m2 = maxb[128 + hl], m3 = maxb[192 + hl];
      if constexpr (!DS) {
        const uint8_t* scp = raw + CK_SCALE * CS + (16 * g + 4 * hi) * 16;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          sc0[r] = *reinterpret_cast<const f32x4*>(scp + r * 16);
          sc1[r] = *reinterpret_cast<const f32x4*>(scp + (8 + r) * 16);
        }
      }
      __builtin_amdgcn_sched_barrier(0);
      const float mx = fmaxf(fmaxf(m0, m1), fmaxf(m2, m3));
      const bool need = mx > m_run + TAU;
      alpha = need ? ((m_run == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(m_run - mx)) : 1.0f;
      m_run = need ? mx : m_run;
      // this tile's k (scales of 2^14 and above): O and l move with P
      alpha *= exp2i(o_k - bias.k);
      o_k = bias.k;
      // P relative to 2^(m_run + k); P' of the 656-byte rows takes P x 2^-b
      // straight from the exponential
      constexpr bool FOLD = !DS;
      // (a head whose scores are all -inf so far has m_run = -inf; the
      // finite floor keeps -inf - mb at -inf, whose exponential is 0)
      const float mb = fmaxf(m_run + (FOLD ? bias.B : (float)o_k), -__FLT_MAX__);
      float psum = 0.0f;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        s0[r] = __builtin_amdgcn_exp2f(s0[r] - mb);
        s1[r] = __builtin_amdgcn_exp2f(s1[r] - mb);
        psum += s0[r] + s1[r];
      }
      l_part = l_part * alpha + (FOLD ? psum * bias.v : psum);
      const uint32_t pw = lds_addr(pq + hl * PS + 16 * g + 4 * hi);
      if constexpr (DS) {
        // DSv4: P'_t = P x 2^-b x (the row's scale of tile t) in FP16 for
        // the seven scale tiles, in slots 0..6, and P itself in slot 7 for
        // the rope columns (which enter PV unbiased)
        const f32x4 s0b = s0 * bias.p, s1b = s1 * bias.p;  // P x 2^-b
#pragma unroll
        for (int t = 0; t < 8; ++t) {
          u32x2 v0, v1;
          if (t < 7) {
            // scales of tile t of candidates 16g + 4hi + r and 16g + 8 + 4hi + r
            const f32x4 c0 = *reinterpret_cast<const f32x4*>(dsc + t * TC + 16 * g + 4 * hi);
            const f32x4 c1 = *reinterpret_cast<const f32x4*>(dsc + t * TC + 16 * g + 8 + 4 * hi);
            v0 = u32x2{pack_f16(s0b[0] * c0[0], s0b[1] * c0[1]), pack_f16(s0b[2] * c0[2], s0b[3] * c0[3])};
            v1 = u32x2{pack_f16(s1b[0] * c1[0], s1b[1] * c1[1]), pack_f16(s1b[2] * c1[2], s1b[3] * c1[3])};
          } else {
            v0 = u32x2{pack_f16(s0[0], s0[1]), pack_f16(s0[2], s0[3])};
            v1 = u32x2{pack_f16(s1[0], s1[1]), pack_f16(s1[2], s1[3])};
          }
#define SMLA_PST(T)                   \
  if (t == (T)) {                     \
    b64_store<(T) * GS>(pw, v0);      \
    b64_store<(T) * GS + 16>(pw, v1); \
  }
          SMLA_PST(0) SMLA_PST(1) SMLA_PST(2) SMLA_PST(3) SMLA_PST(4) SMLA_PST(5) SMLA_PST(6) SMLA_PST(7)
#undef SMLA_PST
        }
      } else {
        // P'_gg = P x (row scale of column group gg) (x 2^-b in FP16), for the PV of
        // every group; the four scales of a row are one 16-byte piece
        u32x2 w0[4], w1[4];
#pragma unroll
        for (int gg = 0; gg < 4; ++gg) {
          w0[gg] = u32x2{pack_f16(s0[0] * sc0[0][gg], s0[1] * sc0[1][gg]), pack_f16(s0[2] * sc0[2][gg], s0[3] * sc0[3][gg])};
          w1[gg] = u32x2{pack_f16(s1[0] * sc1[0][gg], s1[1] * sc1[1][gg]), pack_f16(s1[2] * sc1[2][gg], s1[3] * sc1[3][gg])};
        }
        b64_store<0>(pw, w0[0]);
        b64_store<16>(pw, w1[0]);
        b64_store<GS>(pw, w0[1]);
        b64_store<GS + 16>(pw, w1[1]);
        b64_store<2 * GS>(pw, w0[2]);
        b64_store<2 * GS + 16>(pw, w1[2]);
        b64_store<3 * GS>(pw, w0[3]);
        b64_store<3 * GS + 16>(pw, w1[3]);
      }
    }
    // ---- 4. O^T += V^T P'^T over columns [128g, 128g + 128), heads 32hh.. ----
    // ds_read_b64_tr_b8: in each 16-lane group, lane 2r + b addresses row r
    // of an 8-row block, bytes 8b..8b+7 of a 16-column piece.  656-byte
    // rows: the V^T operands of candidate blocks 0..2 are read before B3
    // (they need only the tile), and B3's wait completes them; block 3's are
    // read in PV once the first three blocks' MFMAs are issued, so that less
    // LDS traffic falls into the interval every wave waits on at B3.
    const int g16 = (lane >> 4) & 1;
    const int jr = (lane & 15) >> 1;
    const int jb = lane & 1;
    i32x2 v8[4][4];  // [ks][dt]: candidates 16ks.., columns 128g + 32dt..
    const uint32_t vta = lds_addr(raw + (8 * g + g16) * CS + (8 * hi + jr) * 16 + 8 * jb);
#define SMLA_VT8(ks, dt) v8[ks][dt] = tr8_issue<2 * (dt) * CS + 256 * (ks)>(vta)
    if constexpr (!DS) {
      SMLA_VT8(0, 0); SMLA_VT8(0, 1); SMLA_VT8(0, 2); SMLA_VT8(0, 3);
      SMLA_VT8(1, 0); SMLA_VT8(1, 1); SMLA_VT8(1, 2); SMLA_VT8(1, 3);
      SMLA_VT8(2, 0); SMLA_VT8(2, 1); SMLA_VT8(2, 2); SMLA_VT8(2, 3);
    }
    if (__any(alpha != 1.0f)) {
#pragma unroll
      for (int dt = 0; dt < 4; ++dt) O[dt] *= alpha;
    }
    lds_barrier();  // B3: P visible
    if constexpr (DS) {
      // DSv4: columns 128g + 32dt.. take P' of scale tile 2g + dt/2 (slot
      // A for dt 0, 1, slot B for dt 2, 3); group 3's columns 448..511 are
      // the rope values (slot 7, P itself; FP16 since the exchange phase),
      // read with ds_read_b64_tr_b16 from pieces 28 + 4(dt - 2) + 2g16 + (b >> 1)
      const uint32_t va = lds_addr(raw + (8 * g + g16) * CS + (8 * hi + jr) * 16 + 8 * jb);
      // columns 128g + 0..63 (codes of scale tile 2g, slot A) first; the
      // reads of the other 64 columns are issued under their MFMAs.  The
      // transposed reads are inline asm and each batch is waited for right
      // after it is issued, in the same block (the compiler takes an asm
      // result as ready at once); the P' rows are plain loads, whose waits
      // the compiler places itself.
      const u32x4* pA = reinterpret_cast<const u32x4*>(pq + (2 * g * 64 + 32 * hh + l32) * PS + 8 * hi);
      const u32x4* pB = reinterpret_cast<const u32x4*>(pq + ((g < 3 ? 2 * g + 1 : 7) * 64 + 32 * hh + l32) * PS + 8 * hi);
      i32x2 v8[4][2];  // [ks][dt]: candidates 16ks.., columns 128g + 32dt..
#define SMLA_TR8(ks, dt) v8[ks][dt] = tr8_issue<2 * (dt) * CS + 256 * (ks)>(va)
      SMLA_TR8(0, 0); SMLA_TR8(0, 1); SMLA_TR8(1, 0); SMLA_TR8(1, 1);
      SMLA_TR8(2, 0); SMLA_TR8(2, 1); SMLA_TR8(3, 0); SMLA_TR8(3, 1);
#undef SMLA_TR8
      asm volatile("s_waitcnt lgkmcnt(0)"
                   : "+v"(v8[0][0]), "+v"(v8[0][1]), "+v"(v8[1][0]), "+v"(v8[1][1]), "+v"(v8[2][0]), "+v"(v8[2][1]),
                     "+v"(v8[3][0]), "+v"(v8[3][1]));
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const u32x4 pb = pA[2 * ks];  // candidates 16ks + 8hi + i
#pragma unroll
        for (int dt = 0; dt < 2; ++dt) {
          const f16x8 v = cvt8_f16((uint32_t)v8[ks][dt][0], (uint32_t)v8[ks][dt][1], bias.v);
          O[dt] = mfma_32x32x16_f16(v, __builtin_bit_cast(f16x8, pb), O[dt]);
        }
      }
      u32x4 pr[4];
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) pr[ks] = pB[2 * ks];
      if (g < 3) {
        // codes of scale tile 2g + 1, two candidate blocks at a time
#pragma unroll
        for (int kh = 0; kh < 2; ++kh) {
          i32x2 w8[2][2];
#define SMLA_TR8(KH, k, d) w8[k][d] = tr8_issue<2 * (2 + (d)) * CS + 256 * (2 * (KH) + (k))>(va)
          if (kh == 0) {
            SMLA_TR8(0, 0, 0); SMLA_TR8(0, 0, 1); SMLA_TR8(0, 1, 0); SMLA_TR8(0, 1, 1);
          } else {
            SMLA_TR8(1, 0, 0); SMLA_TR8(1, 0, 1); SMLA_TR8(1, 1, 0); SMLA_TR8(1, 1, 1);
          }
#undef SMLA_TR8
          asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(w8[0][0]), "+v"(w8[0][1]), "+v"(w8[1][0]), "+v"(w8[1][1]));
#pragma unroll
          for (int k = 0; k < 2; ++k)
#pragma unroll
            for (int d = 0; d < 2; ++d) {
              const f16x8 v = cvt8_f16((uint32_t)w8[k][d][0], (uint32_t)w8[k][d][1], bias.v);
              O[2 + d] = mfma_32x32x16_f16(v, __builtin_bit_cast(f16x8, pr[2 * kh + k]), O[2 + d]);
            }
        }
      } else {
        // group 3: the rope columns 448 + 32(dt - 2) + 16g16 + lc (FP16 by
        // now), two candidate blocks at a time
        const int lc = lane & 15;
        const uint32_t vb = lds_addr(raw + (v4::CK_ROPE + 2 * g16 + ((lc & 3) >> 1)) * CS + (8 * hi + (lc >> 2)) * 16 +
                                     8 * (lc & 1));
#pragma unroll
        for (int kh = 0; kh < 2; ++kh) {
          i32x2 vr[2][2][2];  // [ks - 2kh][dt - 2][rows 0..3 / 4..7]
#define SMLA_TR16(KH, k, d)                                                    \
  vr[k][d][0] = tr16_issue<4 * (d) * CS + 256 * (2 * (KH) + (k))>(vb);        \
  vr[k][d][1] = tr16_issue<4 * (d) * CS + 256 * (2 * (KH) + (k)) + 64>(vb)
          if (kh == 0) {
            SMLA_TR16(0, 0, 0); SMLA_TR16(0, 0, 1); SMLA_TR16(0, 1, 0); SMLA_TR16(0, 1, 1);
          } else {
            SMLA_TR16(1, 0, 0); SMLA_TR16(1, 0, 1); SMLA_TR16(1, 1, 0); SMLA_TR16(1, 1, 1);
          }
#undef SMLA_TR16
          asm volatile("s_waitcnt lgkmcnt(0)"
                       : "+v"(vr[0][0][0]), "+v"(vr[0][0][1]), "+v"(vr[0][1][0]), "+v"(vr[0][1][1]), "+v"(vr[1][0][0]),
                         "+v"(vr[1][0][1]), "+v"(vr[1][1][0]), "+v"(vr[1][1][1]));
#pragma unroll
          for (int k = 0; k < 2; ++k)
#pragma unroll
            for (int d = 0; d < 2; ++d) {
              const f16x8 v = __builtin_bit_cast(
                  f16x8, make_uint4((uint32_t)vr[k][d][0][0], (uint32_t)vr[k][d][0][1], (uint32_t)vr[k][d][1][0],
                                    (uint32_t)vr[k][d][1][1]));
              O[2 + d] = mfma_32x32x16_f16(v, __builtin_bit_cast(f16x8, pr[2 * kh + k]), O[2 + d]);
            }
        }
      }
    } else {
      // P'_g for heads 32hh + l32, candidates 16ks + 8hi + i: the B operands
      const uint32_t pa = lds_addr(pq + (g * 64 + 32 * hh + l32) * PS + 8 * hi);
      u32x4 pb[4];
      pb[0] = b128_issue<0>(pa);
      pb[1] = b128_issue<32>(pa);
      pb[2] = b128_issue<64>(pa);
      pb[3] = b128_issue<96>(pa);
      // one wait for all the reads so far
      asm volatile("s_waitcnt lgkmcnt(0)"
                   : "+v"(v8[0][0]), "+v"(v8[0][1]), "+v"(v8[0][2]), "+v"(v8[0][3]), "+v"(v8[1][0]), "+v"(v8[1][1]),
                     "+v"(v8[1][2]), "+v"(v8[1][3]), "+v"(v8[2][0]), "+v"(v8[2][1]), "+v"(v8[2][2]), "+v"(v8[2][3]),
                     "+v"(pb[0]), "+v"(pb[1]), "+v"(pb[2]), "+v"(pb[3]));
      // int8 codes: 2^b and -1152 x 2^b for int8x4_to_f16x4
      const f16x2 sb = {(_Float16)bias.v, (_Float16)bias.v};
      const f16x2 ob = {(_Float16)(-1152.0f * bias.v), (_Float16)(-1152.0f * bias.v)};
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        if (ks == 3) {
          // block 3's V^T, read while the MFMAs of blocks 0..2 run (the
          // compiler barrier keeps those MFMAs ahead of the reads and wait)
          __builtin_amdgcn_sched_barrier(0);
          SMLA_VT8(3, 0); SMLA_VT8(3, 1); SMLA_VT8(3, 2); SMLA_VT8(3, 3);
          asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(v8[3][0]), "+v"(v8[3][1]), "+v"(v8[3][2]), "+v"(v8[3][3]));
        }
#pragma unroll
        for (int dt = 0; dt < 4; ++dt) {
          f16x8 v;
          if constexpr (CODES == FMT_INT8) {
            const uint2 lo = int8x4_to_f16x4((uint32_t)v8[ks][dt][0], sb, ob);
            const uint2 hi = int8x4_to_f16x4((uint32_t)v8[ks][dt][1], sb, ob);
            v = __builtin_bit_cast(f16x8, make_uint4(lo.x, lo.y, hi.x, hi.y));
          } else {
            v = cvt8_f16((uint32_t)v8[ks][dt][0], (uint32_t)v8[ks][dt][1], bias.v);
          }
          O[dt] = mfma_32x32x16_f16(v, __builtin_bit_cast(f16x8, pb[ks]), O[dt]);
        }
      }
    }
#undef SMLA_VT8
  };
  // ---- end of a split (decode) or of a token (prefill): per-head sum over
  // the four groups, normalization; the result is stored now, or by the
  // next tile when there is one; then start over with empty state ----
  float* lsum = maxb;  // [4][64]; free once every wave is past the softmax of the tile
  auto finish = [&](int32_t key, bool defer) __attribute__((always_inline)) {
    {
      const float lt = l_part + __shfl_xor(l_part, 32);
      if (hi == 0) lsum[g * 64 + 32 * hh + l32] = lt;
    }
    lds_barrier();
    const int hl = 32 * hh + l32;
    const float Ls = (lsum[hl] + lsum[64 + hl]) + (lsum[128 + hl] + lsum[192 + hl]);
    const float M = m_run + (float)o_k;
    const bool empty = !(Ls > 0.0f);
    const float lse_v = empty ? -INFINITY : (M + __log2f(Ls)) * LN2;
    m_run = -INFINITY;
    l_part = 0.0f;
    float factor;
    if (empty) {
      factor = 0.0f;
    } else if (!DECODE && p.sink) {
      const float ms = fmaxf(M, sink2);
      const float a = exp2f(M - ms);
      factor = a / (Ls * a + exp2f(sink2 - ms));
    } else {
      factor = 1.0f / Ls;
    }
    if (defer) {
      // the next tile's first barrier also orders these lsum reads before
      // the next writes of that buffer
      pend = key;
      pend_factor = factor;
      pend_lse = lse_v;
      return;
    }
    // (decode without a next tile: nothing is gathered any more)
    store_result(key, factor, lse_v, DECODE);
    // every wave has read lsum before anyone writes it again
    lds_barrier();
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
      for (int i = 0; i < 16; ++i) O[dt][i] = 0.0f;
  };
  int sp_next = sp0;  // decode: next split to finish
  const int tiles_per_split = DECODE ? p.split_w / TC : 0;
  int split_tiles_left = tiles_per_split;  // decode: tiles of the current split still to run
  auto after_tile = [&](const TileRef& c, const TileRef& n) {
    if constexpr (DECODE) {
      if (--split_tiles_left == 0 || n.t < 0) {
        finish(sp_next++, n.t >= 0);
        split_tiles_left = tiles_per_split;
      }
    } else {
      if (n.t != c.t) finish(c.t, n.t >= 0);
    }
  };
  while (cur.t >= 0) {
    step(Buf<0>{}, cur, nxt, nn);
    after_tile(cur, nxt);
    cur = nxt;
    nxt = nn;
    nn = advance(nn);
    if (cur.t < 0) break;
    step(Buf<1>{}, cur, nxt, nn);
    after_tile(cur, nxt);
    cur = nxt;
    nxt = nn;
    nn = advance(nn);
  }
  // decode: splits left empty by the list length
  if (DECODE)
    while (sp_next < sp_end) finish(sp_next++, false);
}

// looked up once per device
int device_compute_units() {
  static int cached[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cached[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n < 1) n = 256;
    cached[dev] = n;
  }
  return cached[dev];
}

// One workgroup takes several consecutive splits of a token when there are
// more (token, split) pairs than compute units: the gather pipeline and Q
// carry across the split boundary, and the grid fills the chip about once
// instead of leaving a ragged second round.
int fp8_splits_per_block(int64_t T, int32_t H, int32_t num_splits, int compute_units) {
  const int64_t pairs = T * (int64_t)((H + 63) / 64) * num_splits;
  const int64_t g = pairs / (compute_units > 0 ? compute_units : 1);
  return (int)(g < 1 ? 1 : (g > num_splits ? num_splits : g));
}

// prefill: workgroups per head block; each takes tokens blockIdx.x,
// blockIdx.x + gridDim.x, ... (one workgroup per compute unit in all)
int fp8_prefill_blocks(int64_t T, int32_t H, int compute_units) {
  const int64_t hb = (H + 63) / 64;
  int64_t per = (compute_units > 0 ? compute_units : 1) / hb;
  if (per < 1) per = 1;
  return (int)(T < per ? T : per);
}

hipError_t launch_attention_fp8(const AttnParams& p, int fmt, bool decode, hipStream_t s) {
  AttnParams q = p;
  const int cus = device_compute_units();
  q.splits_per_block = decode ? fp8_splits_per_block(p.T, p.H, p.num_splits, cus) : 1;
  dim3 block(f8::NT);
  dim3 grid(decode ? (unsigned)q.T : (unsigned)fp8_prefill_blocks(q.T, q.H, cus), (unsigned)((q.H + 63) / 64),
            decode ? (unsigned)((q.num_splits + q.splits_per_block - 1) / q.splits_per_block) : 1u);
  const bool dual = q.topk2 > 0;
  // one instantiation per (row format, form, list count)
  auto go = [&](auto nope, auto codes) {
    constexpr bool N = decltype(nope)::value;
    constexpr int C = decltype(codes)::value;
    if (decode && dual) hipLaunchKernelGGL((attn_fp8_kernel<true, true, N, C>), grid, block, 0, s, q);
    else if (decode) hipLaunchKernelGGL((attn_fp8_kernel<true, false, N, C>), grid, block, 0, s, q);
    else if (dual) hipLaunchKernelGGL((attn_fp8_kernel<false, true, N, C>), grid, block, 0, s, q);
    else hipLaunchKernelGGL((attn_fp8_kernel<false, false, N, C>), grid, block, 0, s, q);
  };
  using yes = std::true_type;
  using no = std::false_type;
  if (fmt == FMT_FP8_NOPE) go(yes{}, std::integral_constant<int, FMT_FP8>{});
  else if (fmt == FMT_FP8_DSV4) go(no{}, std::integral_constant<int, FMT_FP8_DSV4>{});
  else if (fmt == FMT_FP8_ANY) go(no{}, std::integral_constant<int, FMT_FP8_ANY>{});
  else if (fmt == FMT_INT8) go(no{}, std::integral_constant<int, FMT_INT8>{});
  else go(no{}, std::integral_constant<int, FMT_FP8>{});
  return hipGetLastError();
}

}  // namespace smla
