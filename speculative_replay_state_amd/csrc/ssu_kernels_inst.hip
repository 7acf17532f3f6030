// One state type's kernels and launchers (SSU_INST_ST = 0 fp32, 1 bf16,
// 2 fp16, 3 fp8 e4m3, 4 nvfp4): the build compiles this file once per state type.
#include "ssu_kernels.cuh"

#ifndef SSU_INST_ST
#error "SSU_INST_ST must name the state type to instantiate"
#endif

namespace ssu {

template hipError_t replay_monolith_st<SSU_INST_ST>(const KCache &, const KStep &, int, hipStream_t);
template hipError_t replay_split_st<SSU_INST_ST>(const KCache &, const KStep &, int, hipStream_t);
template hipError_t flush_st<SSU_INST_ST>(const KCache &, const int32_t *, const int32_t *, const float *, int,
                                          hipStream_t);
template hipError_t init_st<SSU_INST_ST>(const KCache &, const float *, int64_t, const int32_t *, int, hipStream_t);

}  // namespace ssu
