// kvq_attn_sparse.hip -- decode-attention kernels with dense-and-sparse keys (gfx950).
#include "kvq_attn_impl.h"

namespace kvq {

KVQ_LOW_BIT_FAMILIES(KVQ_INSTANTIATE_FAMILY, kFmtKiviSp)
KVQ_LOW_BIT_FAMILIES(KVQ_INSTANTIATE_FAMILY, kFmtKiviCbSp)

}  // namespace kvq
