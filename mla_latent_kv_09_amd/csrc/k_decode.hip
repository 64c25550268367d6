// MFMA decode path (placeholder until the split/combine kernels land).
#include "common.h"
#include "launch.h"

namespace mla {
bool decode_fast_supported(const mla_dims& d, const CacheView& c) { (void)d; (void)c; return false; }
size_t decode_fast_workspace(const mla_dims& d, int batch, int max_context) { (void)d; (void)batch; (void)max_context; return 0; }
hipError_t decode_fast(const mla_dims&, float, int, int, const void*, const void*, const void*, const void*,
                       const CacheView&, void*, void*, size_t, hipStream_t) { return hipErrorNotSupported; }
}  // namespace mla
