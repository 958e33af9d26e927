// kvq_attn_8bit.hip -- decode-attention kernels of the 8-bit formats (gfx950).
#include "kvq_attn_impl.h"

namespace kvq {

KVQ_8BIT_FAMILIES(KVQ_INSTANTIATE_FAMILY)

}  // namespace kvq
