// Dispatch of the launch entry points on the state type; the per-state-type
// instantiations live in the ssu_kernels_inst.hip builds.
#include "ssu_internal.h"

namespace ssu {

#define SSU_DISPATCH_ST(FN, ...)                       \
  switch (state_type) {                                \
    case kF32: return FN<kF32>(__VA_ARGS__);           \
    case kBF16: return FN<kBF16>(__VA_ARGS__);         \
    case kF16: return FN<kF16>(__VA_ARGS__);           \
    case kFP8: return FN<kFP8>(__VA_ARGS__);           \
    case kNVFP4: return FN<kNVFP4>(__VA_ARGS__);       \
    default: return hipErrorInvalidValue;              \
  }

hipError_t launch_replay_monolith(const KCache &c, const KStep &s, int state_type, int out_type,
                                  hipStream_t stream) {
  SSU_DISPATCH_ST(replay_monolith_st, c, s, out_type, stream)
}

hipError_t launch_replay_split(const KCache &c, const KStep &s, int state_type, int out_type,
                               hipStream_t stream) {
  SSU_DISPATCH_ST(replay_split_st, c, s, out_type, stream)
}

hipError_t launch_flush(const KCache &c, const int32_t *slot_idx, const int32_t *num_fold, const float *A,
                        int n, int state_type, hipStream_t stream) {
  SSU_DISPATCH_ST(flush_st, c, slot_idx, num_fold, A, n, stream)
}

hipError_t launch_init(const KCache &c, const float *states, int64_t states_stride, const int32_t *slot_idx,
                       int n, int state_type, hipStream_t stream) {
  SSU_DISPATCH_ST(init_st, c, states, states_stride, slot_idx, n, stream)
}

}  // namespace ssu
