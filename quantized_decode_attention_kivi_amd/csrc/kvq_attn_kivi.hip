// kvq_attn_kivi.hip -- decode-attention kernels of the low-bit format (gfx950).
#include "kvq_attn_impl.h"

namespace kvq {

KVQ_LOW_BIT_FAMILIES(KVQ_INSTANTIATE_FAMILY, kFmtKivi)

}  // namespace kvq
