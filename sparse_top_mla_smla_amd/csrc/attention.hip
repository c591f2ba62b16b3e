// attention.hip -- which kernel computes a sparse MLA attention call.
//
// What is computed is stated in include/smla.h.  The rule depends only on
// the row format and the head count:
//  * 16 or fewer heads, and BF16 rows at any head count: the column-split
//    kernel (attention_bf16.hip; one workgroup of 4 waves per (token,
//    16-head group, split), QK over candidates, PV over value columns, two
//    workgroups per CU);
//  * DOTS3_SWA rows at any head count, and DSv4 rows with 16 or fewer
//    heads: the exponent-byte kernel (attention_mx.hip);
//  * more than 16 heads over 656-byte quantized rows (FP8 with any scales,
//    with or without rope, and INT8) and over DSv4 rows: the many-head
//    kernel (attention_fp8.hip; one workgroup per token for 64 heads).
#include "device_common.h"
#include "launch.h"

namespace smla {

hipError_t launch_attention(const AttnParams& p, int fmt, bool decode, hipStream_t s) {
  if (fmt == FMT_FP8_DOTS3 || (fmt == FMT_FP8_DSV4 && p.H <= 16)) return launch_attention_mx(p, fmt, decode, s);
  if (fmt == FMT_FP8_DSV4) return launch_attention_fp8(p, fmt, decode, s);
  if (fmt == FMT_BF16 || p.H <= 16) return launch_attention_bf16(p, fmt, decode, s);
  return launch_attention_fp8(p, fmt, decode, s);
}

}  // namespace smla
