// Attention kernels instantiated for f16, head_dim 128.
#include "pa_attn.h"

namespace pa {
int launch_attn_f16_d128(int kind, const AttnParams& p, hipStream_t stream, hipEvent_t start,
                         hipEvent_t stop) {
  return launch_attn<PA_F16, 128>(kind, p, stream, start, stop);
}
}  // namespace pa
