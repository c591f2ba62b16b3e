// combine.hip -- log-sum-exp merge of decode splits.
//
// AppMana flash-mla-ampere-dsv4 "decode H6" describes the merge as a
// warp-wide combine with one split per lane and no branches; on gfx950 a
// wave is 64 lanes, so one wave merges one (token, head) with split s in
// lane s (up to 64 splits): a wave max gives M, a wave sum gives
// W = sum exp(lse_s - M), and each lane then accumulates 8 of the 512
// output columns over the splits (16 of 1024 for DOTS3_SWA's value width).  The sink (FlashInfer PR #4802 / vLLM
// PR #57673 attn_sink) scales the merged output by 1 / (1 + exp(sink - lse)).
#include "device_common.h"
#include "launch.h"

namespace smla {

template <int DV>
__global__ __launch_bounds__(256) void combine_kernel(CombineParams p) {
  constexpr int NV = DV / 256;  // f32x4 per lane
  const int lane = threadIdx.x & 63;
  const int64_t pair = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (pair >= p.T * p.H) return;  // whole waves exit together
  const int64_t t = pair / p.H;
  const int h = (int)(pair % p.H);

  const float v = lane < p.S ? p.part_lse[(t * p.S + lane) * p.H + h] : -INFINITY;
  const float M = wave_max(v);
  const float w = (v == -INFINITY) ? 0.0f : exp2f((v - M) * LOG2E);
  const float W = wave_sum(w);
  const bool empty = (M == -INFINITY);
  const float lse_v = empty ? -INFINITY : M + logf(W);

  f32x4 a[NV];
#pragma unroll
  for (int i = 0; i < NV; ++i) a[i] = f32x4{0.f, 0.f, 0.f, 0.f};
  if (!empty) {
    const float invW = 1.0f / W;
    for (int s = 0; s < p.S; ++s) {
      const float ws = __shfl(w, s) * invW;
      if (ws != 0.0f) {
        const f32x4* src = reinterpret_cast<const f32x4*>(p.part_out + ((t * p.S + s) * p.H + h) * (int64_t)DV) + NV * lane;
#pragma unroll
        for (int i = 0; i < NV; ++i) a[i] += ws * src[i];
      }
    }
    if (p.sink) {
      const float f = 1.0f / (1.0f + expf(p.sink[h] - lse_v));
#pragma unroll
      for (int i = 0; i < NV; ++i) a[i] *= f;
    }
  }
  uint16_t* orow = p.out + t * p.out_st + (int64_t)h * p.out_sh + 4 * NV * lane;
#pragma unroll
  for (int i = 0; i < NV; i += 2)
    *reinterpret_cast<uint4*>(orow + 4 * i) = make_uint4(pack_bf16(a[i][0], a[i][1]), pack_bf16(a[i][2], a[i][3]),
                                                         pack_bf16(a[i + 1][0], a[i + 1][1]),
                                                         pack_bf16(a[i + 1][2], a[i + 1][3]));
  if (lane == 0) p.lse[t * p.lse_st + h] = lse_v;
}

hipError_t launch_combine(const CombineParams& p, hipStream_t s) {
  const int64_t pairs = p.T * p.H;
  dim3 grid((unsigned)((pairs + 3) / 4)), block(256);
  if (p.dv == dots3::D_V) hipLaunchKernelGGL(combine_kernel<dots3::D_V>, grid, block, 0, s, p);
  else hipLaunchKernelGGL(combine_kernel<D_V>, grid, block, 0, s, p);
  return hipGetLastError();
}

}  // namespace smla
