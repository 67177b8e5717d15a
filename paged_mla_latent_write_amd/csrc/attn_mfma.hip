// MFMA split-KV kernel (placeholder until the CDNA4 kernel lands).
#include "mla_internal.h"

namespace mla {

bool mfma_attn_supported(const CacheView&, int32_t) { return false; }

hipError_t launch_attn_mfma(const AttnArgs&, hipStream_t) { return hipErrorNotSupported; }

}  // namespace mla
