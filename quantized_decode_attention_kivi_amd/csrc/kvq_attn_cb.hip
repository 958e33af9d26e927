// kvq_attn_cb.hip -- decode-attention kernels of the codebook grid (with and without pre-RoPE keys) (gfx950).
#include "kvq_attn_impl.h"

namespace kvq {

KVQ_LOW_BIT_FAMILIES(KVQ_INSTANTIATE_FAMILY, kFmtKiviCb)
KVQ_LOW_BIT_FAMILIES(KVQ_INSTANTIATE_FAMILY, kFmtRopeCb)

}  // namespace kvq
