// Internal interface between the host entry points (ssu_api.cpp) and the
// gfx950 kernels (ssu_kernels.cuh, instantiated per state type by
// ssu_kernels_inst.hip, dispatched in ssu_launch.cpp).  Not part of the
// public ABI.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

namespace ssu {

// Fixed head geometry the kernels implement.
constexpr int kHeadDim = 64;   // P
constexpr int kDState = 128;   // N
constexpr int kMaxRing = 32;   // L <= 32: the combined window fits one 32-deep MFMA K step
constexpr int kMaxTokens = 16; // T <= 16: new tokens are the 16 columns of the readout MFMA
constexpr int kCbStride = 32;  // floats per (entry, group, token) row of the split scratch

enum StateType { kF32 = 0, kBF16 = 1, kF16 = 2, kFP8 = 3, kNVFP4 = 4 };
enum OutType { kOutF32 = 0, kOutBF16 = 1 };

// Cache description as the kernels see it (byte strides between slots).
struct KCache {
  uint8_t *state;
  int64_t state_stride;
  uint8_t *scale;
  int64_t scale_stride;
  uint8_t *xc;
  int64_t x_stride;
  uint8_t *Bc;
  int64_t B_stride;
  uint8_t *dtc;
  int64_t dt_stride;
  int32_t *ring_start;
  int32_t *status;
  int num_slots, H, G, L, hpg;
  uint8_t *recur;        // NULL, or the FP16 recurrence checkpoint (separate checkpoints)
  int64_t recur_stride;
  uint32_t seed_lo, seed_hi;  // this call's stochastic-rounding seed
  uint8_t *gw;           // nvfp4: f32 words per slot: the slot's second-level scale, then the head maxima
  int64_t gw_stride;
};

// One replay step.
struct KStep {
  int batch, T;  // T = max_seqlen
  const int32_t *slot_idx;
  const int32_t *pnat;
  const int32_t *cu;  // NULL unless varlen
  const int32_t *fold;  // NULL, or tokens to fold per entry before the readout (monolith only)
  const uint16_t *x;  // bf16 bits
  const uint16_t *B;
  const uint16_t *C;
  const float *dt;
  const float *A;
  const float *D;
  const float *dt_bias;
  void *out;
  float *cb;  // SPLIT scratch [batch][G][T][kCbStride]
  const uint16_t *z;  // NULL, or the output gate (bf16) [rows][H][64]
  int dt_softplus;    // 1: dt' = softplus(dt + dt_bias); 0: dt' = dt + dt_bias
};

// Per-state-type entry points (definitions in ssu_kernels.cuh, one explicit
// instantiation per state type).
template <int ST>
hipError_t replay_monolith_st(const KCache &c, const KStep &s, int out_type, hipStream_t stream);
template <int ST>
hipError_t replay_split_st(const KCache &c, const KStep &s, int out_type, hipStream_t stream);
template <int ST>
hipError_t flush_st(const KCache &c, const int32_t *slot_idx, const int32_t *num_fold, const float *A, int n,
                    hipStream_t stream);
template <int ST>
hipError_t init_st(const KCache &c, const float *states, int64_t states_stride, const int32_t *slot_idx, int n,
                   hipStream_t stream);

hipError_t launch_replay_monolith(const KCache &c, const KStep &s, int state_type, int out_type,
                                  hipStream_t stream);
hipError_t launch_replay_split(const KCache &c, const KStep &s, int state_type, int out_type,
                               hipStream_t stream);
hipError_t launch_flush(const KCache &c, const int32_t *slot_idx, const int32_t *num_fold,
                        const float *A, int n, int state_type, hipStream_t stream);
hipError_t launch_init(const KCache &c, const float *states, int64_t states_stride,
                       const int32_t *slot_idx, int n, int state_type, hipStream_t stream);

}  // namespace ssu
