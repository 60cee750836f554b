// AsymSpec kernels with fusion source delta = a, the raw full-context logits (mechanism ablation),
// under both gates (AsymSpec reading notes).
#include "asym_kernels.hpp"

namespace vwl {
template int asym_blocks_per_cu_ds<kDeltaA>(int dt, int nv, int gate);
template hipError_t launch_asym_ds<kDeltaA>(int dt, int gate, const Plan &plan, const AsymParams &p, hipStream_t s,
                                            hipEvent_t after_rows);
} // namespace vwl
