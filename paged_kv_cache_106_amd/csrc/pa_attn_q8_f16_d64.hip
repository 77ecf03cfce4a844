// Attention kernels over INT8 pools instantiated for f16 queries, head_dim 64.
#include "pa_attn.h"

namespace pa {
int launch_attn_q8_f16_d64(int kind, const AttnParams& p, hipStream_t stream, hipEvent_t start,
                          hipEvent_t stop) {
  return launch_attn<PA_F16, 64, true>(kind, p, stream, start, stop);
}
}  // namespace pa
