// lists.h -- the candidate list of one query token, shared by the attention
// kernels.  List positions [0, topk) are the main list (indices into the
// main pool, cut at the token's length); with a secondary cache, positions
// [topk, topk + topk2) are the secondary list (indices into the second pool,
// cut at its own length).  A position holds a candidate when it is inside
// its list's length and its index is a slot of its pool; any other position
// contributes nothing.
#pragma once
#include "device_common.h"
#include "launch.h"

namespace smla {

struct ListEnds {
  int32_t l1;   // main list length, clamped to [0, topk]
  int32_t end;  // one past the last position that may hold a candidate
};

__device__ __forceinline__ int32_t clamp_len(int32_t v, int32_t cap) { return v < 0 ? 0 : (v > cap ? cap : v); }

// (l1, l2 are the lengths of token t's main and secondary lists)
__device__ __forceinline__ ListEnds list_ends_of(const AttnParams& p, int32_t l1, int32_t l2) {
  return ListEnds{l1, l2 > 0 ? p.topk + l2 : l1};
}

__device__ __forceinline__ ListEnds list_ends(const AttnParams& p, int64_t t) {
  const int32_t l1 = p.topk_length ? clamp_len(p.topk_length[t], p.topk) : p.topk;
  int32_t l2 = 0;
  if (p.topk2 > 0) l2 = p.topk_length2 ? clamp_len(p.topk_length2[t], p.topk2) : p.topk2;
  return list_ends_of(p, l1, l2);
}

// position j lies inside its list's length
template <bool DUAL>
__device__ __forceinline__ bool in_list(const AttnParams& p, const ListEnds& e, int64_t j) {
  if constexpr (!DUAL) return j < e.end;
  return j < e.end && (j < e.l1 || j >= p.topk);
}

__device__ __forceinline__ uint64_t uniform64(uint64_t v) {
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return ((uint64_t)hi << 32) | lo;
}

struct PoolRef {
  const uint8_t* base;
  int64_t block_stride, row_stride, nslots;
};

// The lists' indices and pools.  With a secondary list (DUAL) they are
// read once as wave-uniform values, so that a per-lane choice between the
// two is a choice between computed addresses; a choice between two kernel
// arguments could otherwise become a per-lane load of one of them inside the
// tile loop.  Without one, the single-list kernels use the arguments as they
// are and hold nothing for a second source.
struct Sources {
  PoolRef p1, p2;
  const int32_t* idx1;
  const int32_t* idx2;
  int64_t st1, st2;
  int32_t topk;
};

template <bool DUAL>
__device__ __forceinline__ Sources sources(const AttnParams& p) {
  Sources s;
  if constexpr (!DUAL) {
    s.p1 = PoolRef{p.pool, p.block_stride, p.row_stride, p.nslots};
    s.p2 = s.p1;
    s.idx1 = s.idx2 = p.idx;
    s.st1 = p.idx_st;
    s.st2 = 0;
    s.topk = p.topk;
    return s;
  }
  s.p1 = PoolRef{(const uint8_t*)uniform64((uint64_t)p.pool), (int64_t)uniform64(p.block_stride),
                 (int64_t)uniform64(p.row_stride), (int64_t)uniform64(p.nslots)};
  const bool two = p.topk2 > 0;
  s.p2 = two ? PoolRef{(const uint8_t*)uniform64((uint64_t)p.pool2), (int64_t)uniform64(p.block_stride2),
                       (int64_t)uniform64(p.row_stride2), (int64_t)uniform64(p.nslots2)}
             : PoolRef{s.p1.base, 0, 0, 0};
  s.idx1 = (const int32_t*)uniform64((uint64_t)p.idx);
  s.idx2 = two ? (const int32_t*)uniform64((uint64_t)p.idx2) : s.idx1;
  s.st1 = (int64_t)uniform64(p.idx_st);
  s.st2 = two ? (int64_t)uniform64(p.idx_st2) : 0;
  s.topk = __builtin_amdgcn_readfirstlane(p.topk);
  return s;
}

// the index entry of position j of token t (j inside its list)
template <bool DUAL>
__device__ __forceinline__ const int32_t* entry_ptr(const Sources& s, int64_t t, int64_t j) {
  const int32_t* a = s.idx1 + t * s.st1 + j;
  if constexpr (!DUAL) return a;
  const int32_t* b = s.idx2 + t * s.st2 + (j - s.topk);
  return j < s.topk ? a : b;
}

__device__ __forceinline__ const uint8_t* row_in(const PoolRef& r, int32_t x) {
  return (x >= 0 && (int64_t)x < r.nslots)
             ? r.base + (int64_t)(x / PAGE) * r.block_stride + (int64_t)(x % PAGE) * r.row_stride
             : nullptr;
}

// the row of index value x found at position j, or null when x is not a slot
// of that position's pool
template <bool DUAL>
__device__ __forceinline__ const uint8_t* row_of(const Sources& s, int64_t j, int32_t x) {
  const uint8_t* a = row_in(s.p1, x);
  if constexpr (!DUAL) return a;
  const uint8_t* b = row_in(s.p2, x);
  return j < s.topk ? a : b;
}

}  // namespace smla
