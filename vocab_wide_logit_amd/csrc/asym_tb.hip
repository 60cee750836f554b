// AsymSpec kernels with fusion source delta = t - b, the two-model difference (mechanism ablation),
// under both gates (AsymSpec reading notes).
#include "asym_kernels.hpp"

namespace vwl {
template int asym_blocks_per_cu_ds<kDeltaTMinusB>(int dt, int nv, int gate);
template hipError_t launch_asym_ds<kDeltaTMinusB>(int dt, int gate, const Plan &plan, const AsymParams &p, hipStream_t s,
                                            hipEvent_t after_rows);
} // namespace vwl
