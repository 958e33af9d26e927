// kvq_attn_rope.hip -- decode-attention kernels of the low-bit format with pre-RoPE keys (gfx950).
#include "kvq_attn_impl.h"

namespace kvq {

KVQ_LOW_BIT_FAMILIES(KVQ_INSTANTIATE_FAMILY, kFmtRope)

}  // namespace kvq
