// gfx950 (MI355X) kernels of the checkpointing selective state update
// (ReplaySSM / MTP-replay SSU).
//
// Method (FlashInfer PR "mamba checkpointing SSU: two-kernel split +
// ring-buffer cache", Description items 1-2; vLLM "replayssm_cutedsl" API
// page): per (entry, head) the checkpoint h0[64][128] is replayed through the
// live ring tokens and the new tokens of this step.  With dt'_s the step sizes
// (softplus(dt + dt_bias) for new tokens, stored dt' for ring tokens) and
// cumA_s = sum_{u<=s} A dt'_u, every new token t reads out
//
//   y_t = exp(cumA_t) (h0 . C_t) + sum_{s<=t} exp(cumA_t - cumA_s) dt'_s (C_t . B_s) x_s + D x_t.
//
// The decay prefix is recomputed every call (it changes when the ring start
// advances); C . B is formed once per (entry, group) and shared by the heads
// of the group.  The state stream dominates the bytes, so every kernel here
// is built around reading each checkpoint exactly once with 16-byte loads.
//
// MI355X mapping (a wave64 reads out one head, two heads, or a part of a
// head's rows):
//  * readout h0 . C_t is a [64 x 128] x [128 x T] product: 16 MFMA
//    v_mfma_f32_16x16x32 (bf16 / f16 state; fp8 codes decoded to bf16
//    exactly; fp32 state uses v_mfma_f32_16x16x4f32), the state tile feeding
//    the A operand straight from global memory;
//  * the replay term sum_s W[t][s] x_s is a [64 x 32] x [32 x 16] MFMA with
//    W split into bf16 hi + lo (+ lo2 for fp32 state) parts, so W keeps
//    16 (24) mantissa bits while x (bf16) is exact;
//  * the 32-long decay prefix is a wave scan; the dstate row maxima of the
//    fp8 encoder are DPP reductions inside 16-lane rows.
// The monolith forms C . B inside each replay wave, in the kernel its size
// picks: each head's rows in parts (small batches), the persistent kernel,
// two heads per wave (16-bit checkpoints from 1536 pairs) or one head per
// wave (the fused flush-in-step, and some large plain steps); the split
// writes C . B to a caller-provided fp32 scratch from a precompute kernel and
// the persistent kernel replays every (entry, head).  All of them run the
// same device functions on the same operands, so their outputs are
// bit-identical.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>

#include "../../include/ssu.h"
#include "ssu_internal.h"

namespace ssu {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kWaves = 4;        // waves per workgroup of the replay kernels
#ifndef SSU_FUSED_WPE
// Waves per SIMD the fused kernel is compiled for.  The kernel is latency
// bound (each wave streams its tile only between compute phases), so it runs
// as many waves as fit: the fp8 step with bf16 output folds in 96 registers
// (5 waves, no spills); the other forms need more and get 3, 2 or 1.  The
// NVFP4 step (not gated, rings up to 16) runs 3 waves although registers
// spill (12 before its C.B shared the readout's C, 2 since): 344.5 us per
// step with 12 spilled against 351.2 at 2 waves (182 registers, none
// spilled), batch 256 of 128 heads.
#define SSU_FUSED_WPE(ST, OT, KW, HAS_Z, SEP) \
  (ST == kF32 ? 1                                                                 \
   : ((KW == 32 || (SEP && !(ST == kNVFP4 && !HAS_Z))) ? 2                        \
      : ((ST == kFP8 && OT == kOutBF16 && !HAS_Z) ? 5 : 3)))
#endif
constexpr int kHeadWaves = 4;    // waves per workgroup of the one-head-per-wave kernels on large grids (1, 2, 4 measure alike there)
// (entry, head) pairs from which a plain bf16 or fp8 step runs one head per wave
constexpr int64_t kPerHeadPlainUnits = 32768;
constexpr int kXS = 40;          // LDS row stride (bf16) of the transposed x window
constexpr int kCbLds = 36;       // LDS row stride (fp32) of C.B in the monolith
constexpr int kHeadElems = kHeadDim * kDState;

// ---------------------------------------------------------------------------
// small helpers
// ---------------------------------------------------------------------------

__device__ __forceinline__ float bf2f(uint32_t b16) { return __uint_as_float(b16 << 16); }
__device__ __forceinline__ u32x4 ld16(const void *p) { return *reinterpret_cast<const u32x4 *>(p); }
__device__ __forceinline__ void st16(void *p, u32x4 v) { *reinterpret_cast<u32x4 *>(p) = v; }
__device__ __forceinline__ u32x2 ld8(const void *p) { return *reinterpret_cast<const u32x2 *>(p); }
__device__ __forceinline__ void st8(void *p, u32x2 v) { *reinterpret_cast<u32x2 *>(p) = v; }
// Streaming (non-temporal) forms for data touched once per call whose every
// wave instruction covers whole cache lines (the tiled checkpoint, whose
// chunk u of a row block is 1 KiB contiguous over the wave, the x windows and
// the staged output rows).  Measured on the large-batch step (bf16, batch
// 1024 of 128 heads, one head per wave): its output rows written with plain
// stores took 469 us per step against 450 us with streaming stores.
__device__ __forceinline__ u32x4 ld16_nt(const void *p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(p));
}
__device__ __forceinline__ void st16_nt(void *p, u32x4 v) {
  __builtin_nontemporal_store(v, reinterpret_cast<u32x4 *>(p));
}

__device__ __forceinline__ f32x4 mfma_bf16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma_f16(f16x8 a, f16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma_f32(float a, float b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// Orders this wave's LDS writes before its later LDS reads (no s_barrier).
__device__ __forceinline__ void wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

__device__ __forceinline__ float softplus_f(float v) { return v > 20.f ? v : log1pf(expf(v)); }

// One of four values for a lane-varying i in [0, 4), taken by value so that
// no register array is indexed at run time (that would go through scratch).
__device__ __forceinline__ float pick4(float v0, float v1, float v2, float v3, int i) {
  return i < 2 ? (i == 0 ? v0 : v1) : (i == 2 ? v2 : v3);
}

__device__ __forceinline__ int ring_pos(int r, int s, int L) {
  int p = r + s;
  return p >= L ? p - L : p;
}

__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
  bf16x2 v = {(__bf16)a, (__bf16)b};
  return __builtin_bit_cast(uint32_t, v);
}
__device__ __forceinline__ uint32_t pack_f16(float a, float b) {
  _Float16 x = (_Float16)a, y = (_Float16)b;
  return (uint32_t)__builtin_bit_cast(uint16_t, x) | ((uint32_t)__builtin_bit_cast(uint16_t, y) << 16);
}

// 8 bf16 (one 16-byte chunk) -> 8 f16, exact for |v| in the f16 normal range.
__device__ __forceinline__ f16x8 bf16x8_to_f16x8(u32x4 v) {
  f16x8 r;
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    r[2 * t] = (_Float16)bf2f(v[t] & 0xFFFFu);
    r[2 * t + 1] = (_Float16)bf2f(v[t] >> 16);
  }
  return r;
}

// 4 e4m3fn codes -> 4 bf16 (exact), packed in two dwords.
__device__ __forceinline__ u32x2 fp8x4_to_bf16(uint32_t w) {
  bf16x2 a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, false);
  bf16x2 b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, true);
  u32x2 r = {__builtin_bit_cast(uint32_t, a), __builtin_bit_cast(uint32_t, b)};
  return r;
}

// 8 e2m1 codes (one dword, value 2 i in the low nibble of byte i) times the
// block scale s -> 8 bf16, exact: an e2m1 value has at most 2 significant
// bits and an e4m3 value 4.  The conversion's own scale operand applies a
// power of two only, so it gets 1 and s is multiplied in fp32.
__device__ __forceinline__ bf16x8 nvfp4_word_to_bf16(uint32_t w, float s) {
  const f32x2 a = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 0);
  const f32x2 b = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 1);
  const f32x2 c = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 2);
  const f32x2 d = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 3);
  const u32x4 r = {pack_bf16(a[0] * s, a[1] * s), pack_bf16(b[0] * s, b[1] * s), pack_bf16(c[0] * s, c[1] * s),
                   pack_bf16(d[0] * s, d[1] * s)};
  return __builtin_bit_cast(bf16x8, r);
}

// fp8 row scale: max|h| / 448, 1 when that is not positive (zero row).
__device__ __forceinline__ float fp8_row_scale(float m) {
  float sc = m / 448.0f;
  return sc > 0.0f ? sc : 1.0f;
}

// Byte offset, inside one head's checkpoint, of 16-byte chunk u of lane l in
// row block rb.  The checkpoint is stored MFMA-tiled: row p = 16 rb + m is cut
// into four quarters of 32 values (q = n / 32); quarter q of row p belongs to
// lane l = 16 q + m and is stored as 16-byte chunks, chunk u of every lane of
// a row block side by side, so one wave load instruction reads 1 KiB
// contiguous that is directly the lanes' MFMA operand.
__device__ __forceinline__ int tile_chunk(int rb, int u, int lane, int eb) {
  return rb * 2048 * eb + (u * 64 + lane) * 16;
}

// 16-byte chunks per lane per row block (32 values) and bytes per head of a
// state type: fp32 8, bf16 / fp16 4, fp8 2, nvfp4 1 (two e2m1 codes a byte).
constexpr int st_chunks(int ST) { return ST == kF32 ? 8 : (ST == kFP8 ? 2 : (ST == kNVFP4 ? 1 : 4)); }
constexpr int st_head_bytes(int ST) { return st_chunks(ST) * 4096; }
__device__ __forceinline__ int tile_off(int rb, int u, int lane, int chunks) {
  return (rb * chunks + u) * 1024 + lane * 16;
}

// ---------------------------------------------------------------------------
// per-entry metadata and device-side contract checks
// ---------------------------------------------------------------------------

// pnat and r describe the replay window.  With a fused fold of k tokens they
// are the values after the fold (pnat - k live tokens from ring_start + k);
// r0 is the ring start the fold reads from.
struct Entry {
  int slot, pnat, r, Tb, bos;
  int k, r0;
  int mode;  // 0: skip entirely, 1: zero the output rows only, 2: replay
};

// The per-entry words of a step in the one-head-per-wave kernel, loaded
// without branches so that they go out together: a word that does not apply
// (no varlen, no num_fold) is read from another valid address and ignored.
struct EntryIn {
  int bos, eos, pnat, fold, ring_word;
};

// kUniform: b is the same in the whole wave (scalar loads); else one entry per lane.
template <bool kUniform = true>
__device__ __forceinline__ EntryIn load_entry_in(const KCache &c, const KStep &s, int b, int slot, bool slot_ok) {
  const bool varlen = s.cu != nullptr;
  const int32_t *cu0 = varlen ? s.cu + b : s.pnat + b;
  const int32_t *cu1 = varlen ? s.cu + b + 1 : s.pnat + b;
  const int32_t *rs = c.ring_start + (slot_ok ? slot : 0);
  const int32_t *kp = s.fold ? s.fold + b : s.pnat + b;
  int w0 = *cu0, w1 = *cu1, pn = s.pnat[b], kf = *kp, rw = *rs;
  // an empty statement that takes and gives back the five words: the loads
  // cannot be moved into the branches that use them, so they are issued
  // together and waited for once
  if constexpr (kUniform)
    asm volatile("" : "+s"(w0), "+s"(w1), "+s"(pn), "+s"(kf), "+s"(rw));
  else
    asm volatile("" : "+v"(w0), "+v"(w1), "+v"(pn), "+v"(kf), "+v"(rw));
  EntryIn in;
  in.pnat = pn;
  in.fold = s.fold ? kf : 0;
  in.ring_word = rw;
  in.bos = varlen ? w0 : b * s.T;
  in.eos = varlen ? w1 : in.bos + s.T;
  return in;
}

// Validates an entry of a fused step from its words (the same checks as
// load_entry).
__device__ __forceinline__ Entry make_entry(const KCache &c, const KStep &s, int slot, const EntryIn &in,
                                            bool report) {
  Entry e;
  e.bos = in.bos;
  e.Tb = in.eos - in.bos;
  e.slot = slot;
  e.pnat = 0;
  e.r = 0;
  e.k = 0;
  e.r0 = 0;
  e.mode = 2;
  int bit = 0;
  if (e.Tb < 0 || e.Tb > s.T) {
    e.mode = 0;
    bit = SSU_STATUS_BAD_SEQLEN;
  } else if (e.slot <= 0 || e.slot >= c.num_slots) {
    e.mode = 1;  // padding entry
  } else {
    e.pnat = in.pnat;
    if (e.pnat < 0 || e.pnat + e.Tb > c.L) {
      e.mode = 1;
      bit = SSU_STATUS_BAD_PNAT;
    } else {
      e.r = in.ring_word;
      e.r0 = e.r;
      if (e.r < 0 || e.r >= c.L) {
        e.mode = 1;
        bit = SSU_STATUS_BAD_RING;
      } else if (s.fold) {
        const int k = in.fold;
        if (k < 0 || k > e.pnat) {
          e.mode = 1;
          bit = SSU_STATUS_BAD_FOLD;
        } else {
          e.k = k;
          e.r = ring_pos(e.r0, k, c.L);
          e.pnat -= k;
        }
      }
    }
  }
  if (bit && report && c.status && (threadIdx.x & 63) == 0) atomicOr(c.status, bit);
  return e;
}

// The same checks, loading each word only where it is needed (the replay and
// flush kernels, whose waves do not start with a tile load).
__device__ __forceinline__ Entry load_entry(const KCache &c, const KStep &s, int b, bool report) {
  Entry e;
  if (s.cu) {
    e.bos = s.cu[b];
    e.Tb = s.cu[b + 1] - e.bos;
  } else {
    e.bos = b * s.T;
    e.Tb = s.T;
  }
  e.slot = s.slot_idx[b];
  e.pnat = 0;
  e.r = 0;
  e.k = 0;
  e.r0 = 0;
  e.mode = 2;
  int bit = 0;
  if (e.Tb < 0 || e.Tb > s.T) {
    e.mode = 0;
    bit = SSU_STATUS_BAD_SEQLEN;
  } else if (e.slot <= 0 || e.slot >= c.num_slots) {
    e.mode = 1;  // padding entry
  } else {
    e.pnat = s.pnat[b];
    if (e.pnat < 0 || e.pnat + e.Tb > c.L) {
      e.mode = 1;
      bit = SSU_STATUS_BAD_PNAT;
    } else {
      e.r = c.ring_start[e.slot];
      e.r0 = e.r;
      if (e.r < 0 || e.r >= c.L) {
        e.mode = 1;
        bit = SSU_STATUS_BAD_RING;
      } else if (s.fold) {
        const int k = s.fold[b];
        if (k < 0 || k > e.pnat) {
          e.mode = 1;
          bit = SSU_STATUS_BAD_FOLD;
        } else {
          e.k = k;
          e.r = ring_pos(e.r0, k, c.L);
          e.pnat -= k;
        }
      }
    }
  }
  if (bit && report && c.status && (threadIdx.x & 63) == 0) atomicOr(c.status, bit);
  return e;
}

// ---------------------------------------------------------------------------
// Combined-window geometry.  KW is the capacity of the combined window
// (live ring tokens + new tokens, S <= L <= KW): 16 for rings up to 16
// entries, else 32.  It is the K depth of the replay-term MFMA
// (v_mfma_f32_16x16x16_bf16 or ..._16x16x32_bf16), so lane (i, q) holds the
// coefficients of window positions s = kE q .. kE q + kE - 1.
// ---------------------------------------------------------------------------

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));

template <int KW>
struct Win;
template <>
struct Win<16> {
  static constexpr int kE = 4;        // window positions per lane in the MFMA operands
  static constexpr int kRounds = 2;   // 16-byte x loads per lane to cover the window
  static constexpr int kXS = 20;      // LDS row stride (bf16) of the transposed window
  static constexpr int kSigBits = 4;  // lane -> (s = l % 16, chunk = l / 16 + 4 jj)
  typedef bf16x4 V;
};
template <>
struct Win<32> {
  static constexpr int kE = 8;
  static constexpr int kRounds = 4;
  static constexpr int kXS = 40;
  static constexpr int kSigBits = 5;  // lane -> (s = l % 32, chunk = l / 32 + 2 jj)
  typedef bf16x8 V;
};

// Readout window loads: round jj of lane l holds the 16-byte chunk l % 8 of
// window position s = l / 8 + 8 jj, so one wave instruction reads 8 whole
// 128-byte rows (ring rows side by side, new-token rows H * 128 bytes apart).
// The fold's window (its k ring rows) keeps the kSigBits mapping above: its
// LDS transposition then has half the bank conflicts, which matters more
// there than whole-row loads.
__device__ __forceinline__ int xw_pos(int lane, int jj) { return (lane >> 3) + 8 * jj; }
__device__ __forceinline__ int xw_chunk(int lane) { return lane & 7; }

template <int KW>
__device__ __forceinline__ f32x4 mfma_win(typename Win<KW>::V a, typename Win<KW>::V b, f32x4 c) {
  if constexpr (KW == 16)
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s16x4, a), __builtin_bit_cast(s16x4, b),
                                                      c, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// Cross-lane moves.  lane_get: the value of lane src (any lane, one LDS
// permute); lane_get_uniform: the value of lane src for a wave-uniform src
// (a scalar read); lane_xor: the value of lane ^ mask.
__device__ __forceinline__ float lane_get(float v, int src) {
  return __int_as_float(__builtin_amdgcn_ds_bpermute(src << 2, __float_as_int(v)));
}
__device__ __forceinline__ float lane_get_uniform(float v, int src) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), src));
}
__device__ __forceinline__ float lane_xor(float v, int lane, int mask) {
  return lane_get(v, lane ^ mask);
}

// Inclusive prefix sum over lanes 0..KW-1: a Hillis-Steele scan inside each
// row of 16 lanes (row shifts, lanes past the row start add zero), then for
// KW = 32 the second row adds the first row's total.
template <int D>
__device__ __forceinline__ float row_shr(float v) {  // v of lane - D within the row, 0 past its start
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x110 + D, 0xF, 0xF, true));
}

template <int KW>
__device__ __forceinline__ float scan_win(float v, int lane) {
  v += row_shr<1>(v);
  v += row_shr<2>(v);
  v += row_shr<4>(v);
  v += row_shr<8>(v);
  if constexpr (KW == 32) {
    const float r0 = lane_get_uniform(v, 15);
    if (lane >= 16 && lane < 32) v += r0;
  }
  return v;
}

// ---------------------------------------------------------------------------
// C.B of one (entry, group): CB[i][s] = sum_n C_i[n] B_s[n] for new token i
// and combined index s (ring tokens, then new tokens), as KW/16 MFMA tiles of
// 16x16.  Rows i >= T_b and columns s >= S come out zero.  On return lane l
// holds cb[nb][j] = CB[4*(l/16) + j][16*nb + l%16].  Optionally appends this
// step's B rows to the group's ring (one writer per (entry, group)).
// ---------------------------------------------------------------------------

// Operands of the C.B MFMA tiles: C of new token m and B of combined index
// s = 16 nb + m (ring or new token), in k order n = 32 u + 8 q + e (k step u,
// lane quarter q: one load instruction reads 64 contiguous bytes of each
// row), or (qorder) in the order of the readout's C chunks (ItemLoads::craw),
// n = 32 q + 8 u + e, so that a caller holding those can pass them as the A
// operand instead of loading C again (own_c = false).  The k order changes the
// MFMA's summation grouping, so every path of one state type uses the same
// order (cb_qorder): the fp8 and nvfp4 paths q order, the others u order.
template <int KW>
struct CbLoads {
  bf16x8 ca[4];
  u32x4 bw[KW / 16][4];
};

// Element offset, in a row of 128, of k step u's chunk for lane quarter q.
__device__ __forceinline__ int cb_k(bool qorder, int u, int q) { return qorder ? 32 * q + 8 * u : 32 * u + 8 * q; }

// The C.B k order of a state type (the fp8 and nvfp4 fused steps share the
// readout's C: for nvfp4 that takes the fused kernel's spill from 12 registers
// to 2 at 3 waves per SIMD).
constexpr bool cb_qorder(int ST) { return ST == kFP8 || ST == kNVFP4; }

template <int KW>
__device__ __forceinline__ void load_cb(const KCache &c, const KStep &s, const Entry &e, int g, int lane,
                                        CbLoads<KW> &cl, bool own_c, bool qorder) {
  const int m = lane & 15, q = lane >> 4, L = c.L, S = e.pnat + e.Tb;
  const bf16x8 zero8 = {};
  const uint16_t *Crow = s.C + ((int64_t)(e.bos + m) * c.G + g) * kDState;
  if (own_c) {
#pragma unroll
    for (int u = 0; u < 4; ++u)
      cl.ca[u] = m < e.Tb ? __builtin_bit_cast(bf16x8, ld16(Crow + cb_k(qorder, u, q))) : zero8;
  }
  const uint16_t *Bring = reinterpret_cast<const uint16_t *>(c.Bc + (int64_t)e.slot * c.B_stride) +
                          (int64_t)g * L * kDState;
#pragma unroll
  for (int nb = 0; nb < KW / 16; ++nb) {
    const int sig = nb * 16 + m;
#pragma unroll
    for (int u = 0; u < 4; ++u) cl.bw[nb][u] = u32x4{0u, 0u, 0u, 0u};
    if (sig < S) {
      const uint16_t *rp = sig < e.pnat ? Bring + ring_pos(e.r, sig, L) * kDState
                                        : s.B + ((int64_t)(e.bos + sig - e.pnat) * c.G + g) * kDState;
#pragma unroll
      for (int u = 0; u < 4; ++u) cl.bw[nb][u] = ld16(rp + cb_k(qorder, u, q));
    }
  }
}

// This step's B rows -> the group's ring (one writer per (entry, group));
// qorder as for the load_cb that filled cl.
template <int KW>
__device__ __forceinline__ void append_B_rows(const KCache &c, const Entry &e, int g, int lane,
                                              const CbLoads<KW> &cl, bool qorder) {
  const int m = lane & 15, q = lane >> 4, L = c.L, S = e.pnat + e.Tb;
  uint16_t *Bring = reinterpret_cast<uint16_t *>(c.Bc + (int64_t)e.slot * c.B_stride) + (int64_t)g * L * kDState;
#pragma unroll
  for (int nb = 0; nb < KW / 16; ++nb) {
    const int sig = nb * 16 + m;
    if (sig >= e.pnat && sig < S) {
      uint16_t *rp = Bring + ring_pos(e.r, sig, L) * kDState;
#pragma unroll
      for (int u = 0; u < 4; ++u) st16(rp + cb_k(qorder, u, q), cl.bw[nb][u]);
    }
  }
}

// ca_ext: C chunks in the same k order (the readout's), or null for cl.ca.
template <int KW>
__device__ __forceinline__ void cb_tiles(const CbLoads<KW> &cl, f32x4 cb[KW / 16], const u32x4 *ca_ext = nullptr) {
#pragma unroll
  for (int nb = 0; nb < KW / 16; ++nb) {
    f32x4 a = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int u = 0; u < 4; ++u)
      a = mfma_bf16(ca_ext ? __builtin_bit_cast(bf16x8, ca_ext[u]) : cl.ca[u], __builtin_bit_cast(bf16x8, cl.bw[nb][u]),
                    a);
    cb[nb] = a;
  }
}

// ca_ext (C chunks in q order) or null; qorder must be true with ca_ext.
template <int KW>
__device__ __forceinline__ void compute_cb(const KCache &c, const KStep &s, const Entry &e, int g,
                                           bool append_B, int lane, f32x4 cb[KW / 16], bool qorder,
                                           const u32x4 *ca_ext = nullptr) {
  CbLoads<KW> cl;
  load_cb<KW>(c, s, e, g, lane, cl, ca_ext == nullptr, qorder);
  // The MFMAs before the append: after the append's branch the compiler can
  // no longer count which loads are still in flight, so a use of the B rows
  // there waits for every load and store the wave has issued.
  cb_tiles<KW>(cl, cb, ca_ext);
  if (append_B) append_B_rows<KW>(c, e, g, lane, cl, qorder);
}

// ---------------------------------------------------------------------------
// Output rows of one (entry, head): lane (i = l%16, q = l/16) owns token i and
// state rows p = 16 rb + 4 q + j.
// ---------------------------------------------------------------------------

template <int OT>
__device__ __forceinline__ void store_out(const KStep &s, int H, const Entry &e, int h, int lane,
                                          const f32x4 acc[4]) {
  const int m = lane & 15, q = lane >> 4;
  if (m >= e.Tb) return;
  const int64_t row = ((int64_t)(e.bos + m) * H + h) * kHeadDim;
#pragma unroll
  for (int rb = 0; rb < 4; ++rb) {
    const int p = rb * 16 + 4 * q;
    if constexpr (OT == kOutF32) {
      st16(static_cast<float *>(s.out) + row + p, __builtin_bit_cast(u32x4, acc[rb]));
    } else {
      u32x2 v = {pack_bf16(acc[rb][0], acc[rb][1]), pack_bf16(acc[rb][2], acc[rb][3])};
      st8(static_cast<uint16_t *>(s.out) + row + p, v);
    }
  }
}

// The same rows staged through LDS (ot: kOutTile words of this wave) so that
// every global store is 16 contiguous bytes per lane and one instruction
// covers whole 128-byte output rows (bf16: 8 token rows, fp32: 4).
constexpr int kOutRowWords = 68;                       // 64 fp32 + 4 pad (bank spread)
constexpr int kOutTile = kMaxTokens * kOutRowWords;    // 32-bit words per wave

__device__ __forceinline__ float silu_f(float v) { return v / (1.0f + expf(-v)); }

// Gate chunks of the staged store's lane mapping, loaded with the head's
// prefetch: bf16 out, lane (c = l % 8, i0 = l / 8): 8 values of tokens
// i0 + 8 r; fp32 out, lane (c = l % 16, i0 = l / 16): 4 values of tokens
// i0 + 4 r, two tokens per u32x4.
template <int OT>
__device__ __forceinline__ void load_gate(const KStep &s, int H, const Entry &e, int h, int lane, u32x4 zw[2]) {
  const u32x4 zero4 = {0u, 0u, 0u, 0u};
  if constexpr (OT == kOutF32) {
    const int c = lane & 15, i0 = lane >> 4;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int i = i0 + 4 * r;
      const u32x2 v = i < e.Tb ? ld8(s.z + ((int64_t)(e.bos + i) * H + h) * kHeadDim + 4 * c) : u32x2{0u, 0u};
      if (r & 1) {
        zw[r >> 1][2] = v[0];
        zw[r >> 1][3] = v[1];
      } else {
        zw[r >> 1][0] = v[0];
        zw[r >> 1][1] = v[1];
      }
    }
  } else {
    const int c = lane & 7, i0 = lane >> 3;
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      const int i = i0 + 8 * r;
      zw[r] = i < e.Tb ? ld16(s.z + ((int64_t)(e.bos + i) * H + h) * kHeadDim + 8 * c) : zero4;
    }
  }
}

// NRB < 4: acc holds row blocks rb0 .. rb0 + NRB - 1 (values 16 rb0 ..
// 16 (rb0 + NRB) - 1 of each output row), which are all this call writes.
template <int OT, bool HAS_Z, int NRB = 4>
__device__ __forceinline__ void store_out_staged(const KStep &s, int H, const Entry &e, int h, int lane,
                                                 const f32x4 *acc, const u32x4 zw[2], uint32_t *ot, int rb0 = 0) {
  static_assert(NRB == 4 || !HAS_Z, "the gate chunks cover whole rows");
  const int m = lane & 15, q = lane >> 4;
  if constexpr (OT == kOutF32 || HAS_Z) {  // fp32 rows (the gate is applied before rounding)
#pragma unroll
    for (int rb = 0; rb < NRB; ++rb)
      *reinterpret_cast<u32x4 *>(ot + m * kOutRowWords + rb * 16 + 4 * q) = __builtin_bit_cast(u32x4, acc[rb]);
  } else {
    // bf16 rows of 64 values = 32 words, same row pitch
#pragma unroll
    for (int rb = 0; rb < NRB; ++rb)
      *reinterpret_cast<u32x2 *>(ot + m * kOutRowWords + rb * 8 + 2 * q) =
          u32x2{pack_bf16(acc[rb][0], acc[rb][1]), pack_bf16(acc[rb][2], acc[rb][3])};
  }
  wave_sync();
  constexpr int kChunks = (OT == kOutF32 ? 16 : 8) * NRB / 4;  // 16-byte output chunks per token row
  constexpr int kRowsPer = 64 / kChunks;                       // token rows per instruction
  const int c = lane % kChunks, i0 = lane / kChunks;
#pragma unroll
  for (int r = 0; r < (kMaxTokens + kRowsPer - 1) / kRowsPer; ++r) {
    const int i = i0 + kRowsPer * r;
    if (i < e.Tb) {
      u32x4 v;
      if constexpr (!HAS_Z) {
        v = *reinterpret_cast<const u32x4 *>(ot + i * kOutRowWords + 4 * c);
      } else if constexpr (OT == kOutF32) {
        const f32x4 y = *reinterpret_cast<const f32x4 *>(ot + i * kOutRowWords + 4 * c);
        const uint32_t z01 = zw[r >> 1][(r & 1) * 2], z23 = zw[r >> 1][(r & 1) * 2 + 1];
        v = u32x4{__float_as_uint(y[0] * silu_f(bf2f(z01 & 0xFFFFu))), __float_as_uint(y[1] * silu_f(bf2f(z01 >> 16))),
                  __float_as_uint(y[2] * silu_f(bf2f(z23 & 0xFFFFu))), __float_as_uint(y[3] * silu_f(bf2f(z23 >> 16)))};
      } else {
        const f32x4 y0 = *reinterpret_cast<const f32x4 *>(ot + i * kOutRowWords + 8 * c);
        const f32x4 y1 = *reinterpret_cast<const f32x4 *>(ot + i * kOutRowWords + 8 * c + 4);
        const u32x4 zz = zw[r];
        float g[8];
#pragma unroll
        for (int e2 = 0; e2 < 8; ++e2) g[e2] = silu_f(bf2f((e2 & 1) ? (zz[e2 >> 1] >> 16) : (zz[e2 >> 1] & 0xFFFFu)));
        v = u32x4{pack_bf16(y0[0] * g[0], y0[1] * g[1]), pack_bf16(y0[2] * g[2], y0[3] * g[3]),
                  pack_bf16(y1[0] * g[4], y1[1] * g[5]), pack_bf16(y1[2] * g[6], y1[3] * g[7])};
      }
      uint8_t *dst = static_cast<uint8_t *>(s.out) +
                     (((int64_t)(e.bos + i) * H + h) * kHeadDim + 16 * rb0) * (OT == kOutF32 ? 4 : 2) + 16 * c;
      st16_nt(dst, v);
    }
  }
  wave_sync();  // LDS reads done before the tile is reused
}

template <int OT>
__device__ __forceinline__ void zero_out_head(const KStep &s, int H, const Entry &e, int h, int lane) {
  const f32x4 z = {0.f, 0.f, 0.f, 0.f};
  const f32x4 acc[4] = {z, z, z, z};
  store_out<OT>(s, H, e, h, lane, acc);
}

// ---------------------------------------------------------------------------
// FLUSH: fold the first k live ring tokens into the checkpoint and re-encode
// it.  One wave per (entry, head).  With coef_s = exp(cumA_{k-1} - cumA_s) dt'_s
// and D0 = exp(cumA_{k-1}) the new checkpoint is D0 h0 + sum_{s<k} coef_s x_s B_s^T.
// The rank-k update runs on MFMA in transposed form: for row block rb and
// tile nb (0..7),
//   acc_nb[r][c] += sum_s (coef_s B_s[n(r, nb)]) x_s[16 rb + c],
//   n(r, nb) = 32 (r / 4) + 8 (r % 4) + nb,
// so lane l = 16 q + m ends up holding values t = 8 j + nb (j = 0..3,
// nb = 0..7) of quarter q of row 16 rb + m: exactly its own chunks of the
// tiled checkpoint, and decode, update, row max and encode stay in registers.
// coef_s B_s is split into bf16 hi + lo (+ lo2 for fp32 state) parts; x is
// bf16 and exact.  The A operands do not depend on rb and are built once.
// ---------------------------------------------------------------------------

// A lane's quarter row (32 values t of quarter q of row 16 rb + m) is held
// as eight f32x4 MFMA accumulators in the fold's order: value t sits in
// acc[t % 8][t / 8].  Decode, the fold's MFMAs, the row max and the encode
// all work on that layout, so no value is ever moved between registers.
#define QV(acc, t) (acc)[(t) & 7][(t) >> 3]

// fp8 encode of 8 values of a row whose scale is sc = fp32(max|row| / 448),
// fast form: q = v * y with y = fp32(1 / sc).  The product is within one ulp
// of the correctly rounded quotient v / sc, so the code can only differ from
// the quotient's where that quotient lies within an ulp of a rounding
// midpoint of e4m3 (the reciprocal reading of the encoder; such a code is one
// step away).  No clamp is needed: |v| <= max|row| bounds |q| by
// 448 (1 + 2^-22), which the round-to-nearest conversion maps to 448.  Valid
// while y is a normal number: sc in [2^-60, 2^100].
__device__ __forceinline__ u32x2 fp8_encode8_rcp(const float *v, float y) {
  int w0 = __builtin_amdgcn_cvt_pk_fp8_f32(v[0] * y, v[1] * y, 0, false);
  w0 = __builtin_amdgcn_cvt_pk_fp8_f32(v[2] * y, v[3] * y, w0, true);
  int w1 = __builtin_amdgcn_cvt_pk_fp8_f32(v[4] * y, v[5] * y, 0, false);
  w1 = __builtin_amdgcn_cvt_pk_fp8_f32(v[6] * y, v[7] * y, w1, true);
  return u32x2{(uint32_t)w0, (uint32_t)w1};
}

// Same with the plain IEEE division (scales outside that range).
__device__ __forceinline__ u32x2 fp8_encode8_div(const float *v, float sc) {
  float qv[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) qv[e] = __builtin_amdgcn_fmed3f(v[e] / sc, -448.0f, 448.0f);
  int w0 = __builtin_amdgcn_cvt_pk_fp8_f32(qv[0], qv[1], 0, false);
  w0 = __builtin_amdgcn_cvt_pk_fp8_f32(qv[2], qv[3], w0, true);
  int w1 = __builtin_amdgcn_cvt_pk_fp8_f32(qv[4], qv[5], 0, false);
  w1 = __builtin_amdgcn_cvt_pk_fp8_f32(qv[6], qv[7], w1, true);
  return u32x2{(uint32_t)w0, (uint32_t)w1};
}

__device__ __forceinline__ bool scale_fast(float sc) { return sc >= 0x1p-60f && sc <= 0x1p100f; }

// Max |v| over a lane's quarter row, then over the four lanes (q = 0..3) that
// hold the same row.
// max(m, |x|, |y|): the NaN-propagating maximum lowers to gfx950's
// v_maximum3_f32 with the absolute values as source modifiers; fmaxf would
// first quiet each input (one more instruction per value, as the kernels run
// in IEEE mode).  A NaN in a row makes its scale NaN (the row is NaN anyway).
__device__ __forceinline__ float max3_abs(float m, float x, float y) {
  return __builtin_elementwise_maximum(m, __builtin_elementwise_maximum(fabsf(x), fabsf(y)));
}

// max over lanes l, l ^ 16, l ^ 32, l ^ 48 (the four quarters of a row).
// gfx950's lane swaps exchange rows 16 lanes apart (permlane16_swap) and
// halves 32 lanes apart (permlane32_swap) between two registers; given v
// twice, the two results hold v of the lane and of its partner, in some order,
// so their maximum is the pair's maximum.  No LDS and no address registers.
__device__ __forceinline__ float quad_max(float v) {
  const auto r16 = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = fmaxf(__uint_as_float(r16[0]), __uint_as_float(r16[1]));
  const auto r32 = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r32[0]), __uint_as_float(r32[1]));
}

__device__ __forceinline__ float quarter_row_max(const f32x4 *acc) {
  float a = 0.f, b = 0.f;
#pragma unroll
  for (int nb = 0; nb < 8; ++nb) {
    a = max3_abs(a, acc[nb][0], acc[nb][1]);
    b = max3_abs(b, acc[nb][2], acc[nb][3]);
  }
  return quad_max(fmaxf(a, b));
}

// Encodes a quarter row into the lane's 16-byte chunks of a row block
// (2 * element bytes of them; chunk u holds values t = u * (16 / eb) ...).
// fp8 uses the row scale sc and y = fp32(1 / sc) (fast: y normal).
template <int ST>
__device__ __forceinline__ void encode_quarter(const f32x4 *acc, float sc, float y, bool fast, u32x4 *ch) {
  if constexpr (ST == kFP8) {
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      float lo8[8], hi8[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        lo8[i] = QV(acc, 16 * u + i);
        hi8[i] = QV(acc, 16 * u + 8 + i);
      }
      const u32x2 lo = fast ? fp8_encode8_rcp(lo8, y) : fp8_encode8_div(lo8, sc);
      const u32x2 hi = fast ? fp8_encode8_rcp(hi8, y) : fp8_encode8_div(hi8, sc);
      ch[u] = u32x4{lo[0], lo[1], hi[0], hi[1]};
    }
  } else if constexpr (ST == kF32) {
#pragma unroll
    for (int u = 0; u < 8; ++u)
      ch[u] = u32x4{__float_as_uint(QV(acc, 4 * u)), __float_as_uint(QV(acc, 4 * u + 1)),
                    __float_as_uint(QV(acc, 4 * u + 2)), __float_as_uint(QV(acc, 4 * u + 3))};
  } else if constexpr (ST == kBF16) {
#pragma unroll
    for (int u = 0; u < 4; ++u)
      ch[u] = u32x4{pack_bf16(QV(acc, 8 * u), QV(acc, 8 * u + 1)), pack_bf16(QV(acc, 8 * u + 2), QV(acc, 8 * u + 3)),
                    pack_bf16(QV(acc, 8 * u + 4), QV(acc, 8 * u + 5)),
                    pack_bf16(QV(acc, 8 * u + 6), QV(acc, 8 * u + 7))};
  } else {
#pragma unroll
    for (int u = 0; u < 4; ++u)
      ch[u] = u32x4{pack_f16(QV(acc, 8 * u), QV(acc, 8 * u + 1)), pack_f16(QV(acc, 8 * u + 2), QV(acc, 8 * u + 3)),
                    pack_f16(QV(acc, 8 * u + 4), QV(acc, 8 * u + 5)),
                    pack_f16(QV(acc, 8 * u + 6), QV(acc, 8 * u + 7))};
  }
}

template <int ST>
__device__ __forceinline__ void store_chunks(uint8_t *hp, int rb, int lane, const u32x4 *ch) {
  constexpr int kC = st_chunks(ST);
#pragma unroll
  for (int u = 0; u < kC; ++u) st16_nt(hp + tile_off(rb, u, lane, kC), ch[u]);
}

// ---------------------------------------------------------------------------
// Stochastic rounding for the FP16 recurrence checkpoint.  Each value of a
// (slot, head) takes 7 random bits: Philox4x32-10 (Salmon, Moraes, Dror and
// Shaw, SC 2011) with counter (value / 16, head, slot, 0) and the call's
// 64-bit seed as key gives 16 bytes, and value index e uses the low 7 bits of
// byte e % 16 (little-endian within each 32-bit word).
// ---------------------------------------------------------------------------

__device__ __forceinline__ u32x4 philox4x32_10(u32x4 ctr, uint32_t k0, uint32_t k1) {
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    if (r > 0) {
      k0 += 0x9E3779B9u;
      k1 += 0xBB67AE85u;
    }
    const uint64_t p0 = (uint64_t)0xD2511F53u * ctr[0], p1 = (uint64_t)0xCD9E8D57u * ctr[2];
    ctr = u32x4{(uint32_t)(p1 >> 32) ^ ctr[1] ^ k0, (uint32_t)p1, (uint32_t)(p0 >> 32) ^ ctr[3] ^ k1,
                (uint32_t)p0};
  }
  return ctr;
}

// Stochastic rounding fp32 -> fp16 with 7 random bits u: keep the top 7 bits
// of the fraction fp16 discards, add u, round away from zero on a carry.
// gfx950's v_cvt_sr_f16_f32 adds the top 13 bits of its random word to the
// top 13 discarded bits (also in the fp16 subnormal range, and carrying to
// infinity past 65504); the word u << 25 puts 64 u there, and a carry of
// R13 + 64 u out of 13 bits is exactly one of floor(R13 / 64) + u out of 7.
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint32_t sr_f16_pair(float v0, uint32_t r0, float v1, uint32_t r1) {
  f16x2_t o = {0, 0};
  o = __builtin_amdgcn_cvt_sr_f16_f32(o, v0, r0, false);
  o = __builtin_amdgcn_cvt_sr_f16_f32(o, v1, r1, true);
  return __builtin_bit_cast(uint32_t, o);
}

// The recurrence checkpoint chunks (fp16) of a quarter row, stochastically
// rounded: row p of (slot, head), quarter q.  Value n = 32 q + t takes byte
// t % 16 of Philox call t / 16 (counter p * 8 + 2 q + t / 16).
__device__ __forceinline__ void encode_quarter_sr(const f32x4 *acc, const KCache &c, int slot, int head, int p,
                                                  int q, u32x4 *ch) {
#pragma unroll
  for (int w = 0; w < 2; ++w) {
    const u32x4 r = philox4x32_10(u32x4{(uint32_t)(p * 8 + 2 * q + w), (uint32_t)head, (uint32_t)slot, 0u},
                                  c.seed_lo, c.seed_hi);
#pragma unroll
    for (int i = 0; i < 8; ++i) {  // values 16 w + 2 i, 16 w + 2 i + 1: bytes 2 i, 2 i + 1
      const uint32_t word = r[i >> 1], sh = 16 * (i & 1);
      const uint32_t r0 = (word >> sh) << 25, r1 = (word >> (sh + 8)) << 25;
      ch[2 * w + (i >> 2)][i & 3] = sr_f16_pair(QV(acc, 16 * w + 2 * i), r0, QV(acc, 16 * w + 2 * i + 1), r1);
    }
  }
}

// Decodes one lane's chunks of a row block into the quarter-row layout,
// times f.
template <int ST>
__device__ __forceinline__ void decode_quarter(const u32x4 *raw, float f, f32x4 *acc) {
  if constexpr (ST == kFP8) {
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const f32x2 a = __builtin_amdgcn_cvt_pk_f32_fp8(raw[u][w], false);
        const f32x2 b = __builtin_amdgcn_cvt_pk_f32_fp8(raw[u][w], true);
        QV(acc, 16 * u + 4 * w + 0) = f * a[0];
        QV(acc, 16 * u + 4 * w + 1) = f * a[1];
        QV(acc, 16 * u + 4 * w + 2) = f * b[0];
        QV(acc, 16 * u + 4 * w + 3) = f * b[1];
      }
  } else if constexpr (ST == kF32) {
#pragma unroll
    for (int u = 0; u < 8; ++u)
#pragma unroll
      for (int e = 0; e < 4; ++e) QV(acc, 4 * u + e) = f * __uint_as_float(raw[u][e]);
  } else if constexpr (ST == kBF16) {
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int e = 0; e < 8; ++e)
        QV(acc, 8 * u + e) = f * bf2f((e & 1) ? (raw[u][e >> 1] >> 16) : (raw[u][e >> 1] & 0xFFFFu));
  } else {
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const uint32_t bits = (e & 1) ? (raw[u][e >> 1] >> 16) : (raw[u][e >> 1] & 0xFFFFu);
        QV(acc, 8 * u + e) = f * (float)__builtin_bit_cast(_Float16, (uint16_t)bits);
      }
  }
}

// What the fold of one (slot, head) reads besides the checkpoint, in two
// parts.  Per head: dt' of ring token s in lane s < k, the x window of the k
// tokens and, for fp8, the old scales of rows 16 rb + m.  Per group: the B
// values of the lane's A operands (tokens s = kE q + e, values
// n = 32 (m / 4) + 8 (m % 4) + 0..7).
template <int ST, int KW>
struct FoldHeadLoads {
  float dtp;
  u32x4 xw[Win<KW>::kRounds];
  float osc[4];
};

template <int KW>
struct FoldBLoads {
  u32x4 bw[Win<KW>::kE];
};

template <int ST, int KW>
__device__ __forceinline__ void load_fold_head(const KCache &c, int slot, int h, int r, int k, int lane,
                                               FoldHeadLoads<ST, KW> &fl) {
  using WC = Win<KW>;
  const int m = lane & 15, L = c.L;
#pragma unroll
  for (int rb = 0; rb < 4; ++rb) fl.osc[rb] = 1.f;
  if constexpr (ST == kFP8) {
    const float *scp = reinterpret_cast<const float *>(c.scale + (int64_t)slot * c.scale_stride) + h * kHeadDim;
#pragma unroll
    for (int rb = 0; rb < 4; ++rb) fl.osc[rb] = scp[16 * rb + m];
  }
  const float *dtring = reinterpret_cast<const float *>(c.dtc + (int64_t)slot * c.dt_stride) + h * L;
  fl.dtp = lane < k ? dtring[ring_pos(r, lane, L)] : 0.f;
  const uint16_t *xring = reinterpret_cast<const uint16_t *>(c.xc + (int64_t)slot * c.x_stride) +
                          (int64_t)h * L * kHeadDim;
  // Rows past the k folded tokens load row k - 1 again instead of being
  // branched around (a load behind a lane branch is waited for at the branch's
  // end): their fold coefficient is exactly zero, so a finite copy of a live
  // row adds nothing.  The repeated addresses merge inside the instruction.
  const int klast = k > 0 ? k - 1 : 0;
#pragma unroll
  for (int jj = 0; jj < WC::kRounds; ++jj) {
    const int sg = lane & (KW - 1), pc = (lane >> WC::kSigBits) + (64 >> WC::kSigBits) * jj;
    fl.xw[jj] = ld16(xring + ring_pos(r, sg < k ? sg : klast, L) * kHeadDim + pc * 8);
  }
}

template <int KW>
__device__ __forceinline__ void load_fold_B(const KCache &c, int slot, int g, int r, int k, int lane,
                                            FoldBLoads<KW> &fb) {
  using WC = Win<KW>;
  const int m = lane & 15, q = lane >> 4, L = c.L;
  const uint16_t *Bring = reinterpret_cast<const uint16_t *>(c.Bc + (int64_t)slot * c.B_stride) +
                          (int64_t)g * L * kDState;
  const int klast = k > 0 ? k - 1 : 0;  // rows past k: row k - 1 again (see load_fold_head)
#pragma unroll
  for (int e = 0; e < WC::kE; ++e) {
    const int sg = WC::kE * q + e;
    fb.bw[e] = ld16(Bring + ring_pos(r, sg < k ? sg : klast, L) * kDState + 32 * (m >> 2) + 8 * (m & 3));
  }
}

// The fold's operands: A operands of the 8 tiles, ab[nb][e] =
// B_s[32 (m / 4) + 8 (m % 4) + nb] for s = kE q + e (bf16, exact), the
// coefficients cf[e] = coef_s of those positions, and the checkpoint decay D0
// (wave-uniform: a scalar register).
// The coefficients go into the B operand (coef_s x_s[p], split into bf16
// parts per row block), which has half as many values per lane as the A side.
// LEAN (register-lean) form: the A operands, the same for all four row
// blocks, wait in the wave's LDS (abl[nb][lane], 512 contiguous bytes per
// tile) instead of 16 (KW 32: 32) registers, and each row block gathers its
// lane's kE coefficients from coef (kE permutes) instead of holding cf across
// the fold.  The fold's register peak (checkpoint tile + a row block's
// accumulators) sets the occupancy of the folding kernels; the lean form pays
// off where it lifts occupancy, and costs time at low occupancy.
template <int ST, int KW, bool LEAN = false>
struct FoldOps {
  typename Win<KW>::V ab[LEAN ? 1 : 8];
  float cf[LEAN ? 1 : Win<KW>::kE];
  const typename Win<KW>::V *abl;  // LEAN: LDS [8][64]
  float coef;                      // LEAN: coef_s of lane s
  float D0;
};
template <int KW>
constexpr int fold_ab_words() { return 8 * 64 * (int)sizeof(typename Win<KW>::V) / 4; }

// Decay prefix and coefficients coef_s = exp(cumA_{k-1} - cumA_s) dt'_s,
// D0 = exp(cumA_{k-1}); the x window goes to LDS transposed, xT[p][s] (zero
// for s >= k).  The caller orders the LDS writes before the MFMA reads.
template <int ST, int KW, bool LEAN>
__device__ __forceinline__ void fold_setup(float Ah, int k, const FoldHeadLoads<ST, KW> &fl,
                                           const FoldBLoads<KW> &fb, uint16_t *xT, typename Win<KW>::V *abl,
                                           int lane, FoldOps<ST, KW, LEAN> &fo) {
  using WC = Win<KW>;
  constexpr int kE = WC::kE;
  const int q = lane >> 4;
  const float cum = scan_win<KW>(Ah * fl.dtp, lane);
  const float ctot = lane_get_uniform(cum, k - 1);
  const float coef = lane < k ? expf(ctot - cum) * fl.dtp : 0.f;
#pragma unroll
  for (int jj = 0; jj < WC::kRounds; ++jj) {
    const int sg = lane & (KW - 1), pc = (lane >> WC::kSigBits) + (64 >> WC::kSigBits) * jj;
#pragma unroll
    for (int tt = 0; tt < 8; ++tt)
      xT[(pc * 8 + tt) * WC::kXS + sg] =
          (uint16_t)((tt & 1) ? (fl.xw[jj][tt >> 1] >> 16) : (fl.xw[jj][tt >> 1] & 0xFFFFu));
  }
  if constexpr (LEAN) {  // D0 in a scalar register, operands to LDS, coef gathered per row block
    fo.D0 = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(expf(ctot))));
    fo.coef = coef;
    fo.abl = abl;
#pragma unroll
    for (int nb = 0; nb < 8; ++nb) {
      typename WC::V a;
#pragma unroll
      for (int e = 0; e < kE; ++e)
        a[e] = __builtin_bit_cast(__bf16, (uint16_t)((nb & 1) ? (fb.bw[e][nb >> 1] >> 16) : (fb.bw[e][nb >> 1] & 0xFFFFu)));
      abl[nb * 64 + lane] = a;
    }
  } else {
    fo.D0 = expf(ctot);
#pragma unroll
    for (int e = 0; e < kE; ++e) {
      fo.cf[e] = lane_get(coef, kE * q + e);
#pragma unroll
      for (int nb = 0; nb < 8; ++nb)
        fo.ab[nb][e] = __builtin_bit_cast(
            __bf16, (uint16_t)((nb & 1) ? (fb.bw[e][nb >> 1] >> 16) : (fb.bw[e][nb >> 1] & 0xFFFFu)));
    }
  }
}

// The rank-k update of row block rb into the lane's quarter row:
// acc[nb] += sum_s B_s[n] (coef_s x_s[p]) for p = 16 rb + m, with coef_s x_s[p]
// split into bf16 hi + lo (+ lo2 for fp32 and fp8 states).  Two parts keep 16
// bits of each term (relative error 2^-17); an fp8 row's subnormal codes are
// rowmax * 2^-9 / 448 apart, which a value that cancels to near zero can
// straddle with that error, so fp8 folds take the third part (24 bits, the
// precision of the fp32 flush itself) as fp32 states do.
constexpr bool fold_lo2(int ST) { return ST == kF32 || ST == kFP8; }

template <int ST, int KW, bool LEAN>
__device__ __forceinline__ void fold_update(const FoldOps<ST, KW, LEAN> &fo, const uint16_t *xT, int rb, int lane,
                                            f32x4 *acc) {
  using WC = Win<KW>;
  using V = typename WC::V;
  const int m = lane & 15, q = lane >> 4;
  const V xb = *reinterpret_cast<const V *>(xT + (rb * 16 + m) * WC::kXS + WC::kE * q);
  V bhi, blo, blo2;
#pragma unroll
  for (int e = 0; e < WC::kE; ++e) {
    const float w = (LEAN ? lane_get(fo.coef, WC::kE * q + e) : fo.cf[LEAN ? 0 : e]) * (float)xb[e];
    const __bf16 hi = (__bf16)w;
    const float r1 = w - (float)hi;
    const __bf16 lo = (__bf16)r1;
    bhi[e] = hi;
    blo[e] = lo;
    if constexpr (fold_lo2(ST)) blo2[e] = (__bf16)(r1 - (float)lo);
  }
#pragma unroll
  for (int nb = 0; nb < 8; ++nb) {
    const V a = LEAN ? fo.abl[nb * 64 + (lane & 63)] : fo.ab[LEAN ? 0 : nb];
    acc[nb] = mfma_win<KW>(a, bhi, acc[nb]);
    acc[nb] = mfma_win<KW>(a, blo, acc[nb]);
    if constexpr (fold_lo2(ST)) acc[nb] = mfma_win<KW>(a, blo2, acc[nb]);
  }
}

// One row block of the fold: decode and decay the lane's chunks ch (old
// checkpoint), add the rank-k update, re-encode into ch (new checkpoint) and
// return the fp8 row scale of row 16 rb + m (1 for other dtypes).
template <int ST, int KW, bool LEAN>
__device__ __forceinline__ float fold_rowblock(const FoldOps<ST, KW, LEAN> &fo, const uint16_t *xT, int rb, int lane,
                                               float old_scale, u32x4 *ch) {
  f32x4 acc[8];
  decode_quarter<ST>(ch, ST == kFP8 ? fo.D0 * old_scale : fo.D0, acc);
  fold_update<ST, KW>(fo, xT, rb, lane, acc);
  float sc = 1.f, y = 1.f;
  bool fast = true;
  if constexpr (ST == kFP8) {
    sc = fp8_row_scale(quarter_row_max(acc));
    y = 1.0f / sc;
    fast = __all(scale_fast(sc));
  }
  encode_quarter<ST>(acc, sc, y, fast, ch);
  return sc;
}

// The same with separate checkpoints: decode the FP16 recurrence chunks rch,
// fold, write the read checkpoint chunks ch (nearest encoding in ST) and the
// new recurrence chunks into rch (stochastic rounding).
template <int ST, int KW, bool LEAN>
__device__ __forceinline__ float fold_rowblock_sep(const FoldOps<ST, KW, LEAN> &fo, const uint16_t *xT, int rb,
                                                   int lane, const KCache &c, int slot, int head, u32x4 *rch,
                                                   u32x4 *ch) {
  const int m = lane & 15, q = lane >> 4;
  f32x4 acc[8];
  decode_quarter<kF16>(rch, fo.D0, acc);
  fold_update<ST, KW>(fo, xT, rb, lane, acc);
  float sc = 1.f, y = 1.f;
  bool fast = true;
  if constexpr (ST == kFP8) {
    sc = fp8_row_scale(quarter_row_max(acc));
    y = 1.0f / sc;
    fast = __all(scale_fast(sc));
  }
  encode_quarter<ST>(acc, sc, y, fast, ch);
  encode_quarter_sr(acc, c, slot, head, 16 * rb + m, q, rch);
  return sc;
}

// NVFP4 encoding of a quarter row block: the lane's 32 values (two blocks of
// 16) times y0 (block t < 16) or y1 (t >= 16), as e2m1 codes, value 2 i in the
// low nibble of byte i.  The conversion rounds to nearest even and saturates
// at 6; its scale operand (a power of two) gets 1.
__device__ __forceinline__ u32x4 nvfp4_encode_quarter(const f32x4 *acc, float y0, float y1) {
  u32x4 cw;
#pragma unroll
  for (int w = 0; w < 4; ++w) {  // values t = 8 w .. 8 w + 7
    const float y = w < 2 ? y0 : y1;
    uint32_t word = 0;
    word = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(word, QV(acc, 8 * w + 0) * y, QV(acc, 8 * w + 1) * y, 1.0f, 0);
    word = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(word, QV(acc, 8 * w + 2) * y, QV(acc, 8 * w + 3) * y, 1.0f, 1);
    word = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(word, QV(acc, 8 * w + 4) * y, QV(acc, 8 * w + 5) * y, 1.0f, 2);
    word = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(word, QV(acc, 8 * w + 6) * y, QV(acc, 8 * w + 7) * y, 1.0f, 3);
    cw[w] = word;
  }
  return cw;
}

// The lane's maxima |v| of its two blocks of 16 in a row block.
__device__ __forceinline__ f32x2 block_max2(const f32x4 *acc) {
  float a = 0.f, b = 0.f;
#pragma unroll
  for (int nb = 0; nb < 8; ++nb) {
    a = max3_abs(a, acc[nb][0], acc[nb][1]);  // values t < 16
    b = max3_abs(b, acc[nb][2], acc[nb][3]);  // values t >= 16
  }
  return f32x2{a, b};
}

// NVFP4 scales.  A slot has one second-level scale g = fp32(M / 2688) (1 if
// not positive), M the largest |value| over every head of the slot, as the
// vLLM API page's initialize_replayssm_state computes it (2688 = 6 * 448: the
// largest e2m1 value times the largest e4m3 value); word 0 of the slot's
// scale words holds g and word 1 + h head h's largest |value|.  Block i of a
// lane gets the e4m3 code of fp32(bm[i] / fp32(6 g)) (nearest, saturating at
// 448) in byte i of sfw, and y[i] = fp32(1 / (e4m3 value * g)), 0 for a zero
// block scale (its values encode as signed zeros).
__device__ __forceinline__ float wave_max(float v, int lane) {
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) v = fmaxf(v, lane_xor(v, lane, d));
  return v;
}
__device__ __forceinline__ float nvfp4_gscale(float slot_max) {
  const float g = slot_max / 2688.0f;
  return g > 0.0f ? g : 1.0f;
}
__device__ __forceinline__ uint32_t nvfp4_block_scale(float a, float g, float &y) {
  const float t = fminf(a / (6.0f * g), 448.0f);
  const uint32_t code = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(t, 0.0f, 0, false) & 0xFFu;
  const float es = __builtin_amdgcn_cvt_pk_f32_fp8(code, false)[0] * g;
  y = es > 0.0f ? 1.0f / es : 0.0f;
  return code;
}

__device__ __forceinline__ float *nvfp4_words(const KCache &c, int slot) {
  return reinterpret_cast<float *>(c.gw + (int64_t)slot * c.gw_stride);
}

// The slot's head maxima (words 1 .. H), read in two parts so that the loads
// can go out early: head_max_load takes words lane and lane + 64 (clamped to
// the last head: every address is valid and a repeated word changes no
// maximum), slot_scale finishes with any heads past 128 and reduces over the
// wave.
struct HeadMaxLoads {
  float a, b;
};
__device__ __forceinline__ HeadMaxLoads head_max_load(const KCache &c, int slot, int lane) {
  const float *w = nvfp4_words(c, slot) + 1;
  const int last = c.H - 1;
  return HeadMaxLoads{w[lane < last ? lane : last], w[lane + 64 < last ? lane + 64 : last]};
}
__device__ __forceinline__ float slot_scale(const KCache &c, int slot, int lane, const HeadMaxLoads &hm) {
  float m = fmaxf(hm.a, hm.b);
  const float *w = nvfp4_words(c, slot) + 1;
  for (int i = lane + 128; i < c.H; i += 64) m = fmaxf(m, w[i]);
  return nvfp4_gscale(wave_max(m, lane));
}

// The fold of an FP16 recurrence tile rch for an NVFP4 read checkpoint, first
// pass: the largest |value| of the folded head.  The same instructions on the
// same operands as fold_head_nvfp4, hence the same values.
template <int KW, bool LEAN>
__device__ __forceinline__ float fold_head_max(const FoldOps<kNVFP4, KW, LEAN> &fo, const uint16_t *xT, int lane,
                                               const u32x4 (*rch)[4]) {
  float mx = 0.f;
#pragma unroll
  for (int rb = 0; rb < 4; ++rb) {
    f32x4 acc[8];
    decode_quarter<kF16>(rch[rb], fo.D0, acc);
    fold_update<kNVFP4, KW>(fo, xT, rb, lane, acc);
    const f32x2 b2 = block_max2(acc);
    mx = fmaxf(mx, fmaxf(b2[0], b2[1]));
  }
  return wave_max(mx, lane);
}

// Separate checkpoints with an NVFP4 read checkpoint: fold the FP16
// recurrence tile rch with the slot's second-level scale g, one row block at
// a time (a block of 16 values lies inside one lane's quarter row, so its
// scale needs only that row block's values): the new recurrence chunks
// (stochastic rounding) over rch, the e2m1 codes into codes, the block
// scales into sfw.
template <int KW, bool LEAN>
__device__ __forceinline__ void fold_head_nvfp4(const FoldOps<kNVFP4, KW, LEAN> &fo, const uint16_t *xT, int lane,
                                                const KCache &c, int slot, int head, float g, u32x4 (*rch)[4],
                                                u32x4 (*codes)[1], u32x2 &sfw) {
  const int m = lane & 15, q = lane >> 4;
  uint32_t sb[8];
#pragma unroll
  for (int rb = 0; rb < 4; ++rb) {
    f32x4 acc[8];
    decode_quarter<kF16>(rch[rb], fo.D0, acc);
    fold_update<kNVFP4, KW>(fo, xT, rb, lane, acc);
    const f32x2 b2 = block_max2(acc);
    float y0, y1;
    sb[2 * rb] = nvfp4_block_scale(b2[0], g, y0);
    sb[2 * rb + 1] = nvfp4_block_scale(b2[1], g, y1);
    encode_quarter_sr(acc, c, slot, head, 16 * rb + m, q, rch[rb]);
    codes[rb][0] = nvfp4_encode_quarter(acc, y0, y1);
  }
  sfw = u32x2{sb[0] | (sb[1] << 8) | (sb[2] << 16) | (sb[3] << 24), sb[4] | (sb[5] << 8) | (sb[6] << 16) | (sb[7] << 24)};
}

// Stores an NVFP4 tile with its block scales; the wave of head 0 also writes
// the slot's second-level scale (word 0: no wave of a folding slot reads it).
__device__ __forceinline__ void store_nvfp4(const KCache &c, int slot, int h, int lane, const u32x4 (*codes)[1],
                                            u32x2 sfw, float g) {
  uint8_t *hp = c.state + (int64_t)slot * c.state_stride + (int64_t)h * st_head_bytes(kNVFP4);
#pragma unroll
  for (int rb = 0; rb < 4; ++rb) store_chunks<kNVFP4>(hp, rb, lane, codes[rb]);
  st8(c.scale + (int64_t)slot * c.scale_stride + (int64_t)h * (kHeadElems / 16) + lane * 8, sfw);
  if (h == 0 && lane == 0) nvfp4_words(c, slot)[0] = g;
}

// ---------------------------------------------------------------------------
// The replay of one (entry, head) by one wave, in two phases so that a wave
// can have the next head's loads in flight while this one computes:
//   load_head  -- every global load of the head: the checkpoint tile (the
//                 bulk of the bytes), C of the group's new tokens, the C.B row
//                 of token i, the dt / x window and the fp8 row scales;
//   head_compute -- softplus, decay prefix, appends, W, MFMAs, output.
// ---------------------------------------------------------------------------

// Per-head loads, prefetched one head ahead: the checkpoint tile (the bulk of
// the bytes), the dt and x windows, and the fp8 row scales.
template <int ST, int KW>
struct HeadLoads {
  static constexpr int kNLD = st_chunks(ST);  // 16-byte chunks per lane per 16-row block
  u32x4 raw[4][kNLD];                   // lane l = 16 q + m: chunk u of quarter q of row 16 rb + m
  u32x4 xw[Win<KW>::kRounds];                // x window chunks
  f32x4 rscale[4];                           // fp8 row scales of rows 16 rb + 4 q + j
  u32x2 sfw;                                 // nvfp4: the lane's 8 block scales (rb 0..3, 2 each)
  float gs;                                  // nvfp4: the slot's second-level scale
  float dtv;                                 // lane s: stored dt' (s < pnat) or raw dt (new)
  float dtb, Ah, Dh;                         // dt_bias[h], A[h], D[h]
  u32x4 zw[2];                               // output gate chunks (gated variant only)
};

// Per-(entry, group) loads: C of the new tokens and the C.B row of token m.
template <int ST, int KW>
struct ItemLoads {
  u32x4 craw[4];       // C of token m in the tile's k order (bf16 / f16 / fp8 state)
  float cf32[32];      // C of token m for the fp32 tile
  f32x4 cbr[KW / 16];  // C.B[m][kE q .. kE q + kE - 1]
};

// The checkpoint tile of (slot, h): 16-byte chunks, 1 KiB contiguous per wave
// instruction, streamed (non-temporal).  NRB < 4: row blocks rb0 ..
// rb0 + NRB - 1 only, into raw[0 .. NRB - 1].
template <int ST, int KW, int NRB = 4>
__device__ __forceinline__ void load_state(const KCache &c, int slot, int h, int lane, HeadLoads<ST, KW> &ld,
                                           int rb0 = 0) {
  using T = HeadLoads<ST, KW>;
  static_assert(NRB == 4 || ST == kF32 || ST == kBF16 || ST == kF16, "part tiles: 16- and 32-bit checkpoints");
  const uint8_t *hp = c.state + (int64_t)slot * c.state_stride + (int64_t)h * st_head_bytes(ST);
#pragma unroll
  for (int rb = 0; rb < NRB; ++rb)
#pragma unroll
    for (int u = 0; u < T::kNLD; ++u) ld.raw[rb][u] = ld16_nt(hp + tile_off(rb0 + rb, u, lane, T::kNLD));
  if constexpr (ST == kNVFP4) {  // the block scales and the head scale belong to the tile
    ld.sfw = ld8(c.scale + (int64_t)slot * c.scale_stride + (int64_t)h * (kHeadElems / 16) + lane * 8);
    ld.gs = nvfp4_words(c, slot)[0];
  }
}

// The readout window of (entry, h): dt in lane s (ring dt' or raw dt), the
// head's dt_bias, A and D, and the x chunks of the combined window.  Nothing
// loaded here is used before the head's compute phase: one counter tracks a
// wave's loads in issue order, so using a value loaded here right away would
// also wait for every load issued before it, including a prefetched tile.
// FLAT: no load sits behind a lane branch (a load behind one is waited for at
// the branch's end, before the loads after it are issued).  Positions past
// the window (s >= S) then load the window's last token again instead of
// zeros: their replay coefficient is exactly zero, so a finite copy of a
// token adds nothing; an empty window (S = 0) loads ring row 0, which no
// output uses.  Each position picks its ring or new-token address with a
// select, so each position is one load.
template <int ST, int OT, int KW, bool HAS_Z, bool FLAT = false>
__device__ __forceinline__ void load_window(const KCache &c, const KStep &s, const Entry &e, int h, int lane,
                                            HeadLoads<ST, KW> &ld) {
  if constexpr (HAS_Z) load_gate<OT>(s, c.H, e, h, lane, ld.zw);
  using WC = Win<KW>;
  const int H = c.H, L = c.L, S = e.pnat + e.Tb;
  if constexpr (FLAT) {
    const float *dtring = reinterpret_cast<const float *>(c.dtc + (int64_t)e.slot * c.dt_stride) + h * L;
    const uint16_t *xring = reinterpret_cast<const uint16_t *>(c.xc + (int64_t)e.slot * c.x_stride) +
                            (int64_t)h * L * kHeadDim;
    const int slast = S > 0 ? S - 1 : 0;
    {
      const int sg = lane < S ? lane : slast;
      const bool ring = sg < e.pnat || S == 0;
      const float *p = ring ? dtring + ring_pos(e.r, sg, L) : s.dt + (int64_t)(e.bos + sg - e.pnat) * H + h;
      ld.dtv = *p;
    }
    ld.dtb = s.dt_bias[h];
    ld.Ah = s.A[h];
    ld.Dh = s.D[h];
#pragma unroll
    for (int jj = 0; jj < WC::kRounds; ++jj) {
      const int sig = xw_pos(lane, jj), pc = xw_chunk(lane);
      const int sg = sig < S ? sig : slast;
      const bool ring = sg < e.pnat || S == 0;
      const uint16_t *p = ring ? xring + ring_pos(e.r, sg, L) * kHeadDim + pc * 8
                               : s.x + ((int64_t)(e.bos + sg - e.pnat) * H + h) * kHeadDim + pc * 8;
      ld.xw[jj] = ld16_nt(p);
    }
    return;
  }
  const u32x4 zero4 = {0u, 0u, 0u, 0u};
  ld.dtv = 0.f;
  if (lane < S) {
    if (lane < e.pnat) {
      const float *dtring = reinterpret_cast<const float *>(c.dtc + (int64_t)e.slot * c.dt_stride) + h * L;
      ld.dtv = dtring[ring_pos(e.r, lane, L)];
    } else {
      ld.dtv = s.dt[(int64_t)(e.bos + lane - e.pnat) * H + h];
    }
  }
  ld.dtb = s.dt_bias[h];
  ld.Ah = s.A[h];
  ld.Dh = s.D[h];
  const uint16_t *xring = reinterpret_cast<const uint16_t *>(c.xc + (int64_t)e.slot * c.x_stride) +
                          (int64_t)h * L * kHeadDim;
#pragma unroll
  for (int jj = 0; jj < WC::kRounds; ++jj) {
    const int sig = xw_pos(lane, jj), pc = xw_chunk(lane);
    ld.xw[jj] = zero4;
    if (sig < S)
      ld.xw[jj] = sig < e.pnat
                      ? ld16_nt(xring + ring_pos(e.r, sig, L) * kHeadDim + pc * 8)
                      : ld16_nt(s.x + ((int64_t)(e.bos + sig - e.pnat) * H + h) * kHeadDim + pc * 8);
  }
}

// Every per-head load of the replay: checkpoint, fp8 row scales of rows
// 16 rb + 4 q + j, and the window.
template <int ST, int OT, int KW, bool HAS_Z>
__device__ __forceinline__ void load_head(const KCache &c, const KStep &s, const Entry &e, int h, int lane,
                                          HeadLoads<ST, KW> &ld) {
  const int q = lane >> 4;
  load_state<ST, KW>(c, e.slot, h, lane, ld);
  if constexpr (ST == kFP8) {
    const float *sp = reinterpret_cast<const float *>(c.scale + (int64_t)e.slot * c.scale_stride) +
                      h * kHeadDim;
#pragma unroll
    for (int rb = 0; rb < 4; ++rb) ld.rscale[rb] = *reinterpret_cast<const f32x4 *>(sp + rb * 16 + 4 * q);
  }
  load_window<ST, OT, KW, HAS_Z>(c, s, e, h, lane, ld);
}

template <int ST, int KW>
__device__ __forceinline__ void load_item_c(const KCache &c, const KStep &s, const Entry &e, int g, int lane,
                                            ItemLoads<ST, KW> &il) {
  const int m = lane & 15, q = lane >> 4;
  const bool tok_ok = m < e.Tb;
  const u32x4 zero4 = {0u, 0u, 0u, 0u};
  // k step kk of the readout takes values t = 8 kk .. 8 kk + 7 of the lane's
  // quarter q, i.e. n = 32 q + 8 kk + e (fp32 tile: k step t, n = 32 q + t).
  const uint16_t *Crow = s.C + ((int64_t)(e.bos + m) * c.G + g) * kDState + 32 * q;
  if constexpr (ST == kBF16 || ST == kFP8 || ST == kNVFP4) {
#pragma unroll
    for (int u = 0; u < 4; ++u) il.craw[u] = tok_ok ? ld16(Crow + 8 * u) : zero4;
  } else if constexpr (ST == kF16) {
    // C as f16 (exact for |C| in the f16 normal range), converted once per item
#pragma unroll
    for (int u = 0; u < 4; ++u)
      il.craw[u] = __builtin_bit_cast(u32x4, bf16x8_to_f16x8(tok_ok ? ld16(Crow + 8 * u) : zero4));
  } else {
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const u32x2 v = tok_ok ? ld8(Crow + 4 * u) : u32x2{0u, 0u};
      il.cf32[4 * u + 0] = bf2f(v[0] & 0xFFFFu);
      il.cf32[4 * u + 1] = bf2f(v[0] >> 16);
      il.cf32[4 * u + 2] = bf2f(v[1] & 0xFFFFu);
      il.cf32[4 * u + 3] = bf2f(v[1] >> 16);
    }
  }
}

// The C.B row of token m from a [16][cbs] fp32 table (LDS or the scratch).
template <int ST, int KW>
__device__ __forceinline__ void load_cb_row(const Entry &e, const float *cb, int cbs, int lane,
                                            ItemLoads<ST, KW> &il) {
  const int m = lane & 15, q = lane >> 4;
#pragma unroll
  for (int v = 0; v < KW / 16; ++v)
    il.cbr[v] = m < e.Tb ? *reinterpret_cast<const f32x4 *>(cb + m * cbs + Win<KW>::kE * q + 4 * v)
                         : f32x4{0.f, 0.f, 0.f, 0.f};
}

// NRB < 4 (part tiles): ld.raw holds row blocks rb0 .. rb0 + NRB - 1 and only
// those output values are read out and written; append = false leaves the
// dt and x rings to another part's wave.
template <int ST, int OT, int KW, bool HAS_Z, int NRB = 4>
__device__ __forceinline__ void head_compute(const KCache &c, const KStep &s, const Entry &e, int h,
                                             const HeadLoads<ST, KW> &ld, const ItemLoads<ST, KW> &il,
                                             uint16_t *xT, uint32_t *ot, int lane, const float *osc = nullptr,
                                             int rb0 = 0, bool append = true) {
  static_assert(NRB == 4 || ST == kF32 || ST == kBF16 || ST == kF16, "part tiles: 16- and 32-bit checkpoints");
  using WC = Win<KW>;
  using V = typename WC::V;
  const int m = lane & 15, q = lane >> 4;
  const int H = c.H, L = c.L, S = e.pnat + e.Tb;
  const bool tok_ok = m < e.Tb;

  // 1. dt' of the combined window (lane = combined index); new positions are
  //    softplus'd and appended to the dt ring.  Then the inclusive decay prefix.
  float dtp = ld.dtv;
  if (lane >= e.pnat && lane < S) {
    dtp = ld.dtv + ld.dtb;
    if (s.dt_softplus) dtp = softplus_f(dtp);
    float *dtring = reinterpret_cast<float *>(c.dtc + (int64_t)e.slot * c.dt_stride) + h * L;
    if (append) dtring[ring_pos(e.r, lane, L)] = dtp;
  }
  const float cum = scan_win<KW>(ld.Ah * dtp, lane);

  // 2. x window -> LDS, transposed to xT[p][s]; new tokens appended to the x
  //    ring.  Positions s >= S hold zeros.
  uint16_t *xring = reinterpret_cast<uint16_t *>(c.xc + (int64_t)e.slot * c.x_stride) +
                    (int64_t)h * L * kHeadDim;
#pragma unroll
  for (int jj = 0; jj < WC::kRounds; ++jj) {
    const int sig = xw_pos(lane, jj), pc = xw_chunk(lane);
    const u32x4 v = ld.xw[jj];
    if (append && sig >= e.pnat && sig < S) st16(xring + ring_pos(e.r, sig, L) * kHeadDim + pc * 8, v);
#pragma unroll
    for (int tt = 0; tt < 8; ++tt)
      xT[(pc * 8 + tt) * WC::kXS + sig] = (uint16_t)((tt & 1) ? (v[tt >> 1] >> 16) : (v[tt >> 1] & 0xFFFFu));
  }

  // 3. replay coefficients W[i][s] for s = kE q + t (the B operand of the x
  //    MFMA, split into bf16 hi + lo (+ lo2 for fp32 state) parts), and the
  //    checkpoint decay beta_i = exp(cumA_{pnat+i}).
  const int ti = e.pnat + m;
  const float ct = lane_get(cum, ti < KW ? ti : KW - 1);
  const float beta = tok_ok ? expf(ct) : 0.f;
  const float Dh = ld.Dh;
  V whi, wlo, wlo2;
#pragma unroll
  for (int tt = 0; tt < WC::kE; ++tt) {
    const int sig = WC::kE * q + tt;
    const float cs = lane_get(cum, sig);
    const float ds = lane_get(dtp, sig);
    const float cbv = il.cbr[tt >> 2][tt & 3];
    float w = 0.f;
    if (tok_ok && sig <= ti) w = expf(ct - cs) * ds * cbv;
    if (tok_ok && sig == ti) w += Dh;
    const __bf16 hi = (__bf16)w;
    const float r1 = w - (float)hi;
    const __bf16 lo = (__bf16)r1;
    whi[tt] = hi;
    wlo[tt] = lo;
    if constexpr (ST == kF32) wlo2[tt] = (__bf16)(r1 - (float)lo);
  }
  wave_sync();  // xT written by this wave -> read below

  // 4. checkpoint readout: acc[rb][j] = sum_n h0[16 (rb0 + rb) + 4 q + j][n] C_i[n]
  f32x4 acc[NRB];
#pragma unroll
  for (int rb = 0; rb < NRB; ++rb) {
    f32x4 a = {0.f, 0.f, 0.f, 0.f};
    if constexpr (ST == kBF16) {
#pragma unroll
      for (int u = 0; u < 4; ++u)
        a = mfma_bf16(__builtin_bit_cast(bf16x8, ld.raw[rb][u]), __builtin_bit_cast(bf16x8, il.craw[u]), a);
    } else if constexpr (ST == kF16) {
#pragma unroll
      for (int u = 0; u < 4; ++u)
        a = mfma_f16(__builtin_bit_cast(f16x8, ld.raw[rb][u]), __builtin_bit_cast(f16x8, il.craw[u]), a);
    } else if constexpr (ST == kNVFP4) {
      const f32x2 sfv = (rb & 1) ? __builtin_amdgcn_cvt_pk_f32_fp8(ld.sfw[rb >> 1], true)
                                 : __builtin_amdgcn_cvt_pk_f32_fp8(ld.sfw[rb >> 1], false);  // blocks t < 16, t >= 16
#pragma unroll
      for (int w = 0; w < 4; ++w)  // k step w: values t = 8 w .. 8 w + 7
        a = mfma_bf16(nvfp4_word_to_bf16(ld.raw[rb][0][w], w < 2 ? sfv[0] : sfv[1]),
                      __builtin_bit_cast(bf16x8, il.craw[w]), a);
    } else if constexpr (ST == kFP8) {
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const u32x2 d0 = fp8x4_to_bf16(ld.raw[rb][u][0]), d1 = fp8x4_to_bf16(ld.raw[rb][u][1]);
        const u32x2 d2 = fp8x4_to_bf16(ld.raw[rb][u][2]), d3 = fp8x4_to_bf16(ld.raw[rb][u][3]);
        const u32x4 lo = {d0[0], d0[1], d1[0], d1[1]}, hi = {d2[0], d2[1], d3[0], d3[1]};
        a = mfma_bf16(__builtin_bit_cast(bf16x8, lo), __builtin_bit_cast(bf16x8, il.craw[2 * u]), a);
        a = mfma_bf16(__builtin_bit_cast(bf16x8, hi), __builtin_bit_cast(bf16x8, il.craw[2 * u + 1]), a);
      }
    } else {
#pragma unroll
      for (int u = 0; u < 8; ++u)
#pragma unroll
        for (int e4 = 0; e4 < 4; ++e4) a = mfma_f32(__uint_as_float(ld.raw[rb][u][e4]), il.cf32[4 * u + e4], a);
    }
    acc[rb] = a;
  }

  // 5. epilogue: decay to the token (and fp8 row scale), then add the ring /
  //    new-token replay terms through the x MFMA.
#pragma unroll
  for (int rb = 0; rb < NRB; ++rb) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      if constexpr (ST == kFP8)  // row 16 rb + 4 q + j: loaded, or held by lane 4 q + j in osc[rb]
        acc[rb][j] = (acc[rb][j] * (osc ? lane_get(osc[rb], 4 * q + j) : ld.rscale[rb][j])) * beta;
      else if constexpr (ST == kNVFP4)
        acc[rb][j] = (acc[rb][j] * ld.gs) * beta;
      else
        acc[rb][j] = acc[rb][j] * beta;
    }
    const V xa = *reinterpret_cast<const V *>(xT + ((rb0 + rb) * 16 + m) * WC::kXS + WC::kE * q);
    acc[rb] = mfma_win<KW>(xa, whi, acc[rb]);
    acc[rb] = mfma_win<KW>(xa, wlo, acc[rb]);
    if constexpr (ST == kF32) acc[rb] = mfma_win<KW>(xa, wlo2, acc[rb]);
  }
  wave_sync();  // xT reads done before the tile is reused

  // 6. output rows of the new tokens
  store_out_staged<OT, HAS_Z, NRB>(s, H, e, h, lane, acc, ld.zw, ot, rb0);
}

// ---------------------------------------------------------------------------
// The replay kernel.  Persistent; a work item is (entry, group, chunk of nc
// heads) and one wave runs one item at a time: it loads C and the C.B row of
// the group once, then walks the item's heads, the loads of head j + 1 in
// flight while head j computes (two register buffers alternate).
//   SPLIT = false (monolith, one launch): the wave forms C.B itself (and the
//     chunk-0 wave appends the group's B rows);
//   SPLIT = true: C.B comes from the scratch written by precompute_kernel.
// Both run identical arithmetic, so their outputs are bit-identical.
// ---------------------------------------------------------------------------

template <int ST, int OT, int KW, bool SPLIT, bool HAS_Z>
__global__ __launch_bounds__(kWaves * 64) __attribute__((amdgpu_waves_per_eu(2)))
void replay_kernel(KCache c, KStep s, int d) {
  __shared__ uint16_t xT_all[kWaves][kHeadDim * Win<KW>::kXS];
  __shared__ float cbw_all[SPLIT ? 1 : kWaves][SPLIT ? 4 : kMaxTokens * kCbLds];
  __shared__ __align__(16) uint32_t ot_all[kWaves][kOutTile];
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int nc = c.hpg / d;
  const int64_t nitems = (int64_t)s.batch * c.G * d;
  const int64_t nw = (int64_t)gridDim.x * kWaves;
  uint16_t *xT = xT_all[wave];
  uint32_t *ot = ot_all[wave];
  for (int64_t item = (int64_t)blockIdx.x * kWaves + wave; item < nitems; item += nw) {
    const int chunk = (int)(item % d);
    const int64_t bg = item / d;
    const int g = (int)(bg % c.G), b = (int)(bg / c.G);
    const int h0 = g * c.hpg + chunk * nc;
    const Entry e = load_entry(c, s, b, g == 0 && chunk == 0);
    if (e.mode == 0) continue;
    if (e.mode == 1) {
      for (int j = 0; j < nc; ++j) zero_out_head<OT>(s, c.H, e, h0 + j, lane);
      continue;
    }
    HeadLoads<ST, KW> la, lb;
    ItemLoads<ST, KW> il;
    load_head<ST, OT, KW, HAS_Z>(c, s, e, h0, lane, la);
    load_item_c<ST, KW>(c, s, e, g, lane, il);
    if constexpr (SPLIT) {
      load_cb_row<ST, KW>(e, s.cb + ((int64_t)b * c.G + g) * s.T * kCbStride, kCbStride, lane, il);
    } else {
      float *cbw = cbw_all[wave];
      f32x4 cb[KW / 16];
      compute_cb<KW>(c, s, e, g, chunk == 0, lane, cb, cb_qorder(ST), cb_qorder(ST) ? il.craw : nullptr);
#pragma unroll
      for (int nb = 0; nb < KW / 16; ++nb)
#pragma unroll
        for (int j = 0; j < 4; ++j) cbw[(4 * (lane >> 4) + j) * kCbLds + nb * 16 + (lane & 15)] = cb[nb][j];
      wave_sync();
      load_cb_row<ST, KW>(e, cbw, kCbLds, lane, il);
      wave_sync();
    }
    if constexpr (ST == kF32) {  // a 32 KiB fp32 tile per head: no room for a second buffer
      for (int j = 0; j < nc; ++j) {
        if (j > 0) load_head<ST, OT, KW, HAS_Z>(c, s, e, h0 + j, lane, la);
        head_compute<ST, OT, KW, HAS_Z>(c, s, e, h0 + j, la, il, xT, ot, lane);
      }
      continue;
    }
    int j = 0;
    for (; j + 2 < nc; j += 2) {  // heads j + 1 and j + 2 exist: prefetch unconditionally
      load_head<ST, OT, KW, HAS_Z>(c, s, e, h0 + j + 1, lane, lb);
      __builtin_amdgcn_sched_barrier(0);
      head_compute<ST, OT, KW, HAS_Z>(c, s, e, h0 + j, la, il, xT, ot, lane);
      load_head<ST, OT, KW, HAS_Z>(c, s, e, h0 + j + 2, lane, la);
      __builtin_amdgcn_sched_barrier(0);
      head_compute<ST, OT, KW, HAS_Z>(c, s, e, h0 + j + 1, lb, il, xT, ot, lane);
    }
    if (j + 1 < nc) {  // two heads left
      load_head<ST, OT, KW, HAS_Z>(c, s, e, h0 + j + 1, lane, lb);
      __builtin_amdgcn_sched_barrier(0);
      head_compute<ST, OT, KW, HAS_Z>(c, s, e, h0 + j, la, il, xT, ot, lane);
      head_compute<ST, OT, KW, HAS_Z>(c, s, e, h0 + j + 1, lb, il, xT, ot, lane);
    } else {  // one head left
      head_compute<ST, OT, KW, HAS_Z>(c, s, e, h0 + j, la, il, xT, ot, lane);
    }
  }
}

// ---------------------------------------------------------------------------
// SPLIT precompute (one wave per (entry, group)): C.B -> scratch, B append.
// ---------------------------------------------------------------------------

template <int KW, bool QORDER>
__global__ __launch_bounds__(kWaves * 64) void precompute_kernel(KCache c, KStep s) {
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int item = blockIdx.x * kWaves + wave;
  if (item >= s.batch * c.G) return;
  const int b = item / c.G, g = item - b * c.G;
  const Entry e = load_entry(c, s, b, false);
  if (e.mode != 2) return;
  f32x4 cb[KW / 16];
  compute_cb<KW>(c, s, e, g, true, lane, cb, QORDER);
  const int m = lane & 15, q = lane >> 4;
  float *dst = s.cb + ((int64_t)b * c.G + g) * s.T * kCbStride;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int i = 4 * q + j;
    if (i < s.T) {
#pragma unroll
      for (int nb = 0; nb < KW / 16; ++nb) dst[i * kCbStride + nb * 16 + m] = cb[nb][j];
    }
  }
}

// Workgroups of a launch go to the 8 XCDs round-robin by ID, and each XCD
// has its own L2.  The one-head-per-wave kernels take their (entry, head tile)
// from xcd_tile, so XCD x runs the contiguous tiles [x per, (x + 1) per): the
// heads of one group, which read the same B and C rows, read them through
// one L2.  The grid is rounded up to a multiple of 8 (tiles >= ntiles idle).
__device__ __forceinline__ int64_t xcd_tile(int64_t id, int64_t ngrid) { return (id & 7) * (ngrid >> 3) + (id >> 3); }
inline unsigned xcd_grid(int64_t ntiles) { return (unsigned)((ntiles + 7) / 8 * 8); }

// (entry, head) pairs up to which the one-head-per-wave kernels (flush, the
// NVFP4 maxima pass, the fused step) run one wave per workgroup, so that a
// small grid spreads over every CU instead of filling a quarter of them: fp8
// fused step, batch 1 of 128 heads, 9.84 us per step against 11.14 with 4
// waves per workgroup; batch 4, 10.97 against 11.40; from batch 16 up alike.
constexpr int64_t kFusedOneWaveMax = 512;

// WPG waves (heads) per workgroup: 1 up to kFusedOneWaveMax pairs, else 4.
template <int ST, int KW, bool SEP, int WPG>
__global__ __launch_bounds__(WPG * 64) __attribute__((amdgpu_waves_per_eu(ST == kF32 ? 1 : ((KW == 32 || SEP) ? 2 : 3))))
void flush_kernel(KCache c, const int32_t *slot_idx, const int32_t *num_fold, const float *A, int htiles,
                  int64_t ntiles) {
  using WC = Win<KW>;
  constexpr int kNLD = st_chunks(ST);
  static_assert(ST != kNVFP4 || SEP, "an nvfp4 read checkpoint needs the recurrence checkpoint");
  __shared__ uint16_t xT_all[WPG][kHeadDim * WC::kXS];
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int64_t tile = xcd_tile(blockIdx.x, gridDim.x);
  if (tile >= ntiles) return;
  const int j = (int)(tile / htiles);
  const int h = (int)(tile - (int64_t)j * htiles) * WPG + wave;
  if (h >= c.H) return;
  const int slot = slot_idx[j], k = num_fold[j], L = c.L;
  if (slot <= 0 || slot >= c.num_slots) return;
  if (k < 0 || k > L) {
    if (h == 0 && lane == 0 && c.status) atomicOr(c.status, SSU_STATUS_BAD_FOLD);
    return;
  }
  if (k == 0) return;
  const int r = c.ring_start[slot];
  if (r < 0 || r >= L) {
    if (h == 0 && lane == 0 && c.status) atomicOr(c.status, SSU_STATUS_BAD_RING);
    return;
  }
  const int m = lane & 15, q = lane >> 4;
  uint16_t *xT = xT_all[wave];
  uint8_t *hp = c.state + (int64_t)slot * c.state_stride + (int64_t)h * st_head_bytes(ST);

  // 1. loads, issued before any arithmetic (fp32: the checkpoint per row
  //    block, below)
  u32x4 raw[(ST == kF32 || SEP) ? 1 : 4][kNLD];
  u32x4 rraw[SEP ? 4 : 1][4];  // separate checkpoints: the FP16 recurrence tile
  uint8_t *rp = SEP ? c.recur + (int64_t)slot * c.recur_stride + (int64_t)h * (kHeadElems * 2) : nullptr;
  if constexpr (SEP) {
#pragma unroll
    for (int rb = 0; rb < 4; ++rb)
#pragma unroll
      for (int u = 0; u < 4; ++u) rraw[rb][u] = ld16_nt(rp + tile_chunk(rb, u, lane, 2));
  } else if constexpr (ST != kF32) {
#pragma unroll
    for (int rb = 0; rb < 4; ++rb)
#pragma unroll
      for (int u = 0; u < kNLD; ++u) raw[rb][u] = ld16_nt(hp + tile_off(rb, u, lane, kNLD));
  }
  FoldHeadLoads<ST, KW> fl;
  FoldBLoads<KW> fb;
  load_fold_head<ST, KW>(c, slot, h, r, k, lane, fl);
  load_fold_B<KW>(c, slot, h / c.hpg, r, k, lane, fb);
  HeadMaxLoads hm{};
  if constexpr (ST == kNVFP4) hm = head_max_load(c, slot, lane);  // written by fold_max_kernel

  // 2. coefficients, xT, A operands
  FoldOps<ST, KW> fo;
  fold_setup<ST, KW>(A[h], k, fl, fb, xT, nullptr, lane, fo);
  wave_sync();  // xT written by this wave -> read below

  if constexpr (ST == kNVFP4) {  // the whole head at once: its block scales need the slot's scale
    u32x4 codes[4][1];
    u32x2 sfw;
    const float g = slot_scale(c, slot, lane, hm);
    fold_head_nvfp4<KW>(fo, xT, lane, c, slot, h, g, rraw, codes, sfw);
#pragma unroll
    for (int rb = 0; rb < 4; ++rb) store_chunks<kF16>(rp, rb, lane, rraw[rb]);
    store_nvfp4(c, slot, h, lane, codes, sfw, g);
  } else {
  // 3. row block by row block: decode and decay, rank-k update, encode, store
  float scs[4];
#pragma unroll
  for (int rb = 0; rb < 4; ++rb) {
    u32x4 ch[kNLD];
    if constexpr (SEP) {
      scs[rb] = fold_rowblock_sep<ST, KW>(fo, xT, rb, lane, c, slot, h, rraw[rb], ch);
      store_chunks<kF16>(rp, rb, lane, rraw[rb]);
    } else {
#pragma unroll
      for (int u = 0; u < kNLD; ++u) {
        if constexpr (ST == kF32)
          ch[u] = ld16_nt(hp + tile_off(rb, u, lane, kNLD));
        else
          ch[u] = raw[rb][u];
      }
      scs[rb] = fold_rowblock<ST, KW>(fo, xT, rb, lane, fl.osc[rb], ch);
    }
    store_chunks<ST>(hp, rb, lane, ch);
  }
  // new row scales: lane l holds row l's (row 16 q + m is in rb = q)
  if constexpr (ST == kFP8)
    (reinterpret_cast<float *>(c.scale + (int64_t)slot * c.scale_stride) + h * kHeadDim)[lane] = pick4(scs[0], scs[1], scs[2], scs[3], q);
  }
}

// NVFP4 folds, first pass: the largest |value| of every folded head, stored
// as word 1 + h of the slot's scale words; the fold's encode pass (flush or
// fused step, launched next on the same stream) reduces them to the slot's
// second-level scale.  A slot's scale depends on every head of the slot, so
// no head can be encoded before all of them are folded: this pass reads the
// FP16 recurrence tiles once more.  One wave per (entry, head), the same
// loads and fold instructions as the encode pass.  STEP: the entries of a
// fused step (its validity rules; k = num_fold from the ring start at call
// time); else those of a flush (slot_idx, num_fold, A).
template <int KW, bool STEP, int WPG>
__global__ __launch_bounds__(WPG * 64) __attribute__((amdgpu_waves_per_eu(3)))
void fold_max_kernel(KCache c, KStep s, const int32_t *slot_idx, const int32_t *num_fold, const float *A,
                     int htiles, int64_t ntiles) {
  __shared__ uint16_t xT_all[WPG][kHeadDim * Win<KW>::kXS];
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int64_t tile = xcd_tile(blockIdx.x, gridDim.x);
  if (tile >= ntiles) return;
  const int j = (int)(tile / htiles);
  const int h = (int)(tile - (int64_t)j * htiles) * WPG + wave;
  if (h >= c.H) return;
  int slot, k, r;
  float Ah;
  if constexpr (STEP) {
    const Entry e = load_entry(c, s, j, false);
    if (e.mode != 2 || e.k <= 0) return;
    slot = e.slot;
    k = e.k;
    r = e.r0;
    Ah = s.A[h];
  } else {
    slot = slot_idx[j];
    k = num_fold[j];
    if (slot <= 0 || slot >= c.num_slots || k <= 0 || k > c.L) return;
    r = c.ring_start[slot];
    if (r < 0 || r >= c.L) return;
    Ah = A[h];
  }
  uint16_t *xT = xT_all[wave];
  u32x4 rraw[4][4];
  const uint8_t *rp = c.recur + (int64_t)slot * c.recur_stride + (int64_t)h * (kHeadElems * 2);
#pragma unroll
  for (int rb = 0; rb < 4; ++rb)
#pragma unroll
    for (int u = 0; u < 4; ++u) rraw[rb][u] = ld16_nt(rp + tile_chunk(rb, u, lane, 2));
  FoldHeadLoads<kNVFP4, KW> fl;
  FoldBLoads<KW> fb;
  load_fold_head<kNVFP4, KW>(c, slot, h, r, k, lane, fl);
  load_fold_B<KW>(c, slot, h / c.hpg, r, k, lane, fb);
  FoldOps<kNVFP4, KW> fo;
  fold_setup<kNVFP4, KW>(Ah, k, fl, fb, xT, nullptr, lane, fo);
  wave_sync();  // xT written by this wave -> read below
  const float mx = fold_head_max<KW>(fo, xT, lane, rraw);
  if (lane == 0) nvfp4_words(c, slot)[1 + h] = mx;
}

// ---------------------------------------------------------------------------
// FUSED flush-in-step: one wave per (entry, head).  An entry with k = fold[b]
// > 0 first folds its first k live ring tokens into the checkpoint with the
// flush's own device functions and keeps the re-encoded tile in registers;
// the readout then replays the remaining pnat - k live tokens and the new
// tokens from those very codes.  The result is that of a flush followed by
// a step, with one read of the checkpoint instead of two.
// The phases run in sequence (checkpoint loads issued as soon as the slot is
// known, the fold, the readout's loads, the new tile's stores, the readout)
// so that their registers do not add up and the kernel keeps three waves per
// SIMD; those waves, not a prefetch buffer, keep the memory system busy, and
// the tile's writes drain while the readout computes.  Each wave forms its
// group's C.B itself (a few MFMAs); the wave of the group's first head
// appends the group's B rows.
// ---------------------------------------------------------------------------

// WPG waves (heads) per workgroup: 1 for the smallest grids (see fused_zs).
template <int ST, int OT, int KW, bool HAS_Z, bool SEP, int WPG>
__global__ __launch_bounds__(WPG * 64) __attribute__((amdgpu_waves_per_eu(SSU_FUSED_WPE(ST, OT, KW, HAS_Z, SEP))))
void fused_kernel(KCache c, KStep s, int htiles, int64_t ntiles) {
  // LDS per wave: the transposed x window, then the fold's A operands and
  // later (once the fold is done) the C.B table in the same words, and last
  // (once both have been read) the output staging tile.
  constexpr int kXTWords = kHeadDim * Win<KW>::kXS / 2, kCbWords = kMaxTokens * kCbLds;
  constexpr bool kAbLds = SSU_FUSED_WPE(ST, OT, KW, HAS_Z, SEP) >= 5;  // register-lean form
  constexpr int kAbWords = kAbLds ? fold_ab_words<KW>() : 0;
  constexpr int kMid = kCbWords > kAbWords ? kCbWords : kAbWords;
  constexpr int kWords = kXTWords + kMid > kOutTile ? kXTWords + kMid : kOutTile;
  __shared__ __align__(16) uint32_t lds_all[WPG][kWords];
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int64_t tile = xcd_tile(blockIdx.x, gridDim.x);
  if (tile >= ntiles) return;
  const int b = (int)(tile / htiles);
  const int h = (int)(tile - (int64_t)b * htiles) * WPG + wave;
  if (h >= c.H) return;
  const int g = h / c.hpg, m = lane & 15, q = lane >> 4;
  uint16_t *xT = reinterpret_cast<uint16_t *>(lds_all[wave]);
  float *cbw = reinterpret_cast<float *>(lds_all[wave] + kXTWords);

  // 1. the checkpoint as soon as the slot is known (discarded if the entry
  //    turns out to be skipped).  Separate
  //    checkpoints: an entry that asks for a fold reads the FP16 recurrence
  //    tile (the fold writes the read tile from it), any other the read tile.
  //    A replayed entry folds exactly the k it asks for, so the choice holds.
  HeadLoads<ST, KW> ld;
  u32x4 rraw[SEP ? 4 : 1][4];
  // 8- and 4-bit checkpoints: the tile loads go out as soon as the slot is
  // known; the entry's other words (the slot's ring start among them) follow
  // as scalar loads.  One counter tracks a wave's vector loads in issue order,
  // so words loaded as vector loads after the tile could only be used once
  // the tile had arrived; as scalar loads they arrive on their own, and the
  // fold's window loads that need them go out while the tile is in flight.
  // (The 16- and 32-bit tiles hold too many registers for this: it spills.)
  constexpr bool kEarly = ST == kFP8 || ST == kNVFP4;
  const int slot0 = s.slot_idx[b];
  const bool slot_ok = slot0 > 0 && slot0 < c.num_slots;
  if (kEarly || slot_ok) {
    // An entry whose slot is out of range loads slot 0's tile (in bounds,
    // never used), so that the tile loads are not behind a branch.
    const int slot = slot_ok ? slot0 : 0;
    bool recur_tile = false;
    if constexpr (SEP) recur_tile = slot_ok && s.fold && s.fold[b] > 0;
    if (recur_tile) {
      const uint8_t *rp = c.recur + (int64_t)slot * c.recur_stride + (int64_t)h * (kHeadElems * 2);
#pragma unroll
      for (int rb = 0; rb < 4; ++rb)
#pragma unroll
        for (int u = 0; u < 4; ++u) rraw[rb][u] = ld16_nt(rp + tile_chunk(rb, u, lane, 2));
    } else {
      load_state<ST, KW>(c, slot, h, lane, ld);
    }
  }
  Entry e;
  if constexpr (kEarly) {
    __builtin_amdgcn_sched_barrier(0);
    e = make_entry(c, s, slot0, load_entry_in(c, s, b, slot0, slot_ok), h == 0);
  } else {
    e = load_entry(c, s, b, h == 0);
  }
  if (e.mode == 0) return;
  if (e.mode == 1) {
    zero_out_head<OT>(s, c.H, e, h, lane);
    return;
  }

  // 2. fold the first k live tokens: the new tile replaces ld.raw, the new
  //    fp8 row scales of rows 16 rb + m replace fl.osc
  const float Ah = s.A[h];
  FoldHeadLoads<ST, KW> fl;  // fp8: the old scales even when k == 0
  load_fold_head<ST, KW>(c, e.slot, h, e.r0, e.k, lane, fl);
  if (e.k > 0) {
    FoldBLoads<KW> fb;
    load_fold_B<KW>(c, e.slot, g, e.r0, e.k, lane, fb);
    HeadMaxLoads hm{};
    if constexpr (ST == kNVFP4) hm = head_max_load(c, e.slot, lane);  // written by fold_max_kernel
    FoldOps<ST, KW, kAbLds> fo;
    fold_setup<ST, KW>(Ah, e.k, fl, fb, xT,
                       kAbLds ? reinterpret_cast<typename Win<KW>::V *>(lds_all[wave] + kXTWords) : nullptr, lane,
                       fo);
    wave_sync();  // xT written by this wave -> read below
    if constexpr (ST == kNVFP4) {
      ld.gs = slot_scale(c, e.slot, lane, hm);
      fold_head_nvfp4<KW>(fo, xT, lane, c, e.slot, h, ld.gs, rraw, ld.raw, ld.sfw);
    } else {
#pragma unroll
      for (int rb = 0; rb < 4; ++rb) {
        if constexpr (SEP)
          fl.osc[rb] = fold_rowblock_sep<ST, KW>(fo, xT, rb, lane, c, e.slot, h, rraw[rb], ld.raw[rb]);
        else
          fl.osc[rb] = fold_rowblock<ST, KW>(fo, xT, rb, lane, fl.osc[rb], ld.raw[rb]);
        if constexpr (kAbLds) __builtin_amdgcn_sched_barrier(0);  // one row block's values live at a time
      }
    }
    wave_sync();  // the fold's xT reads done before the readout rewrites xT
  }

  // 3. the readout's loads, C.B of the group and the new tile's stores.  One
  //    counter tracks a wave's loads and stores in issue order: loads issued
  //    after the stores would wait for the writes, and once the stores sit
  //    behind a branch (k > 0) the compiler can no longer count which loads
  //    are still in flight, so a use of loaded values after them waits for
  //    the stores too.  For 8- and 4-bit checkpoints the C.B MFMAs (which need
  //    the last of the loads) therefore go before the stores and the window
  //    loads are unbranched; the 16- and 32-bit tiles hold too many registers
  //    for that order (it spills), so they store first.
  constexpr bool kCbFirst = kEarly;
  load_window<ST, OT, KW, HAS_Z, kCbFirst>(c, s, e, h, lane, ld);
  ItemLoads<ST, KW> il;
  load_item_c<ST, KW>(c, s, e, g, lane, il);
  constexpr bool kShareC = cb_qorder(ST);  // C.B takes the readout's C chunks
  CbLoads<KW> cl;
  load_cb<KW>(c, s, e, g, lane, cl, !kShareC, kShareC);
  auto cb_to_lds = [&]() {
    if (h % c.hpg == 0) append_B_rows<KW>(c, e, g, lane, cl, kShareC);
    f32x4 cb[KW / 16];
    cb_tiles<KW>(cl, cb, kShareC ? il.craw : nullptr);
#pragma unroll
    for (int nb = 0; nb < KW / 16; ++nb)
#pragma unroll
      for (int j = 0; j < 4; ++j) cbw[(4 * q + j) * kCbLds + nb * 16 + m] = cb[nb][j];
  };
  if constexpr (kCbFirst) cb_to_lds();
  if (e.k > 0) {
    if constexpr (ST == kNVFP4) {
      store_nvfp4(c, e.slot, h, lane, ld.raw, ld.sfw, ld.gs);
    } else {
      uint8_t *hp = c.state + (int64_t)e.slot * c.state_stride + (int64_t)h * st_head_bytes(ST);
#pragma unroll
      for (int rb = 0; rb < 4; ++rb) store_chunks<ST>(hp, rb, lane, ld.raw[rb]);
    }
    if constexpr (SEP) {
      uint8_t *rp = c.recur + (int64_t)e.slot * c.recur_stride + (int64_t)h * (kHeadElems * 2);
#pragma unroll
      for (int rb = 0; rb < 4; ++rb) store_chunks<kF16>(rp, rb, lane, rraw[rb]);
    }
    if constexpr (ST == kFP8)  // lane l holds row l's new scale (row 16 q + m is in rb = q)
      (reinterpret_cast<float *>(c.scale + (int64_t)e.slot * c.scale_stride) + h * kHeadDim)[lane] = pick4(fl.osc[0], fl.osc[1], fl.osc[2], fl.osc[3], q);
  }
  if constexpr (!kCbFirst) cb_to_lds();

  // 4. the replay of the head from the (new) tile
  wave_sync();  // C.B rows written by this wave -> read below
  load_cb_row<ST, KW>(e, cbw, kCbLds, lane, il);
  if constexpr (ST == kFP8 && !kAbLds) {  // row scales of the (new) tile, rows 16 rb + 4 q + j
#pragma unroll
    for (int rb = 0; rb < 4; ++rb)
#pragma unroll
      for (int j = 0; j < 4; ++j) ld.rscale[rb][j] = lane_get(fl.osc[rb], 4 * q + j);
  }
  // the lean form gathers them where the epilogue uses them
  head_compute<ST, OT, KW, HAS_Z>(c, s, e, h, ld, il, xT, lds_all[wave], lane,
                                  (ST == kFP8 && kAbLds) ? fl.osc : nullptr);
}

// ---------------------------------------------------------------------------
// PAIR: plain steps of 16-bit checkpoints, two heads of one group per wave.
// A wave issues every load of both heads (checkpoint tiles, windows) and of
// their group (C, the B rows of the window) at once, then reads out head A,
// stores it, and reads out head B.  A one-head wave spends much of its life
// on the latency of its loads and, at its end, on the acknowledgements of its
// stores (a wave's memory operations must complete before it ends), with no
// loads in flight meanwhile; two heads per wave pay each of those waits once
// per two heads, keep 32 KiB of checkpoint in flight per wave, and share C
// and C.B.  Workgroup: 4 waves, heads h0 .. h0 + 7 of one entry, wave w runs
// h0 + w and h0 + 4 + w (both in one group: the group size is a multiple of
// 8).  Same arithmetic as the other paths, so the outputs are bit-identical.
// ---------------------------------------------------------------------------

#ifndef SSU_PAIR_MIN_UNITS
// (entry, head) pairs from which plain 16-bit steps run two heads per wave.
// Measured against the persistent kernel (fp16 prod, graph-replayed steps):
// batch 5 (640 pairs) 8.80 against 8.38 us, 8 (1024): 9.66 / 9.50, 12 (1536):
// 11.05 / 11.96, 16: 12.47 / 12.78, 32: 18.95 / 19.18, 64: 33.16 / 32.84, 128:
// 61.00 / 64.71, 192: 89.82 / 96.44; bf16 mtp (64 heads) batch 12 (768):
// 8.56 / 8.02, 24 (1536): 10.52 / 11.37, 64: 18.35 / 18.31.
#define SSU_PAIR_MIN_UNITS 1536
#endif
constexpr int kPairHeads = 2 * kHeadWaves;  // heads per workgroup

// C of the group's new tokens in the readout's k order, without branches: the
// rows of tokens past T_b (>= 1) load token T_b - 1 again; their readout
// column, C.B row and coefficients are never used.
template <int ST, int KW>
__device__ __forceinline__ void load_item_c_flat(const KCache &c, const KStep &s, const Entry &e, int g, int lane,
                                                 ItemLoads<ST, KW> &il) {
  static_assert(ST == kBF16 || ST == kF16, "16-bit checkpoints");
  const int m = lane & 15, q = lane >> 4;
  const int mm = m < e.Tb ? m : e.Tb - 1;
  const uint16_t *Crow = s.C + ((int64_t)(e.bos + mm) * c.G + g) * kDState + 32 * q;
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const u32x4 v = ld16(Crow + 8 * u);
    il.craw[u] = ST == kF16 ? __builtin_bit_cast(u32x4, bf16x8_to_f16x8(v)) : v;
  }
}

// The operands of the group's C.B (load_cb with its own C, u order), without
// branches: window positions past S (>= 1) load position S - 1 again and
// tokens past T_b token T_b - 1; those columns and rows are never used.
template <int KW>
__device__ __forceinline__ void load_cb_flat(const KCache &c, const KStep &s, const Entry &e, int g, int lane,
                                             CbLoads<KW> &cl) {
  const int m = lane & 15, q = lane >> 4, L = c.L, S = e.pnat + e.Tb;
  const int mm = m < e.Tb ? m : e.Tb - 1;
  const uint16_t *Crow = s.C + ((int64_t)(e.bos + mm) * c.G + g) * kDState;
#pragma unroll
  for (int u = 0; u < 4; ++u) cl.ca[u] = __builtin_bit_cast(bf16x8, ld16(Crow + cb_k(false, u, q)));
  const uint16_t *Bring = reinterpret_cast<const uint16_t *>(c.Bc + (int64_t)e.slot * c.B_stride) +
                          (int64_t)g * L * kDState;
#pragma unroll
  for (int nb = 0; nb < KW / 16; ++nb) {
    const int sig = nb * 16 + m, sg = sig < S ? sig : S - 1;
    const uint16_t *rp = sg < e.pnat ? Bring + ring_pos(e.r, sg, L) * kDState
                                     : s.B + ((int64_t)(e.bos + sg - e.pnat) * c.G + g) * kDState;
#pragma unroll
    for (int u = 0; u < 4; ++u) cl.bw[nb][u] = ld16(rp + cb_k(false, u, q));
  }
}

template <int ST, int OT, int KW, bool HAS_Z>
__global__ __launch_bounds__(kHeadWaves * 64) __attribute__((amdgpu_waves_per_eu(2)))
void pair_kernel(KCache c, KStep s, int ptiles, int64_t ntiles) {
  static_assert(ST == kBF16 || ST == kF16, "two 16-bit tiles per wave");
  constexpr int kXTWords = kHeadDim * Win<KW>::kXS / 2, kCbWords = kMaxTokens * kCbLds;
  constexpr int kWords = kXTWords + kCbWords > kOutTile ? kXTWords + kCbWords : kOutTile;
  __shared__ __align__(16) uint32_t lds_all[kHeadWaves][kWords];
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int64_t tile = xcd_tile(blockIdx.x, gridDim.x);
  if (tile >= ntiles) return;
  const int b = (int)(tile / ptiles);
  const int h0 = (int)(tile - (int64_t)b * ptiles) * kPairHeads;
  const int hA = h0 + wave, hB = hA + kHeadWaves, g = h0 / c.hpg, m = lane & 15, q = lane >> 4;
  uint16_t *xT = reinterpret_cast<uint16_t *>(lds_all[wave]);
  float *cbw = reinterpret_cast<float *>(lds_all[wave] + kXTWords);

  // 1. both tiles as soon as the slot is known (an out-of-range slot loads
  //    slot 0's page, in bounds and never used), then the entry's words as
  //    scalar loads, then both windows and the group's C and B rows: every
  //    load of the wave is issued before its first store
  const int slot0 = s.slot_idx[b];
  const bool slot_ok = slot0 > 0 && slot0 < c.num_slots;
  HeadLoads<ST, KW> la, lb;
  load_state<ST, KW>(c, slot_ok ? slot0 : 0, hA, lane, la);
  load_state<ST, KW>(c, slot_ok ? slot0 : 0, hB, lane, lb);
  __builtin_amdgcn_sched_barrier(0);
  const Entry e = make_entry(c, s, slot0, load_entry_in(c, s, b, slot0, slot_ok), h0 == 0 && wave == 0);
  if (e.mode == 0) return;
  if (e.mode == 1) {
    zero_out_head<OT>(s, c.H, e, hA, lane);
    zero_out_head<OT>(s, c.H, e, hB, lane);
    return;
  }
  if (e.Tb == 0) return;  // no new token: nothing to read out or append
  load_window<ST, OT, KW, HAS_Z, true>(c, s, e, hA, lane, la);
  load_window<ST, OT, KW, HAS_Z, true>(c, s, e, hB, lane, lb);
  ItemLoads<ST, KW> il;
  load_item_c_flat<ST, KW>(c, s, e, g, lane, il);
  CbLoads<KW> cl;
  load_cb_flat<KW>(c, s, e, g, lane, cl);

  // 2. C.B of the group (the wave of its first head appends the B rows)
  {
    f32x4 cb[KW / 16];
    cb_tiles<KW>(cl, cb, nullptr);
    if (hA % c.hpg == 0) append_B_rows<KW>(c, e, g, lane, cl, false);
#pragma unroll
    for (int nb = 0; nb < KW / 16; ++nb)
#pragma unroll
      for (int j = 0; j < 4; ++j) cbw[(4 * q + j) * kCbLds + nb * 16 + m] = cb[nb][j];
  }
  wave_sync();  // C.B rows written by this wave -> read below
  load_cb_row<ST, KW>(e, cbw, kCbLds, lane, il);
  wave_sync();  // C.B rows read before the LDS words are reused

  // 3. the two heads, one after the other.  (A wave that loaded a third head
  //    after storing the first, reusing the first head's registers, measured
  //    slower: one counter tracks a wave's loads and stores in issue order,
  //    so using those loads waits for the stores before them.)
  head_compute<ST, OT, KW, HAS_Z>(c, s, e, hA, la, il, xT, lds_all[wave], lane);
  head_compute<ST, OT, KW, HAS_Z>(c, s, e, hB, lb, il, xT, lds_all[wave], lane);
}

// ---------------------------------------------------------------------------
// D-SPLIT: plain steps of few (entry, head) pairs (small batches), and fp32
// plain steps of any size (a 32 KiB tile is too much for one wave's register
// budget).  The head's 64 state rows are cut into DS parts of 64 / DS rows
// and each part is read out by a wave of its own, one wave per (entry, head,
// part), so a small batch still spreads over the chip and each wave's serial
// work (its share of the tile loads, the readout MFMAs and the output stores)
// shrinks DS-fold.
// Every part forms the group's C.B and the head's decay prefix itself (a few
// hundred flops) and loads the whole x window (the other parts' rows come
// from L2); part 0 appends the new tokens' x and dt' to the rings, part 0 of
// the group's first head its B rows.  Each output value is the same
// arithmetic as on the other paths: the outputs are bit-identical.
// ---------------------------------------------------------------------------

// WPG waves per workgroup: 1 for the smallest grids, so that their few waves
// spread over every CU (fp32 tiny, 64 waves: 4.82 us per step against 5.72
// with 4 waves per workgroup; fp16 batch 1, 512 waves: 5.11 against 5.54),
// else kHeadWaves (fp16 batch 4, 1024 waves: 6.15 against 6.25 with 1).
template <int ST, int OT, int KW, int DS, int WPG>
__global__ __launch_bounds__(WPG * 64) void dsplit_kernel(KCache c, KStep s, int64_t nwaves) {
  static_assert(ST == kF32 || ST == kBF16 || ST == kF16, "part tiles: 16- and 32-bit checkpoints");
  static_assert(DS == 2 || DS == 4, "parts of 2 or 1 row blocks");
  constexpr int NRB = 4 / DS;
  constexpr int kXTWords = kHeadDim * Win<KW>::kXS / 2, kCbWords = kMaxTokens * kCbLds;
  constexpr int kWords = kXTWords + kCbWords > kOutTile ? kXTWords + kCbWords : kOutTile;
  __shared__ __align__(16) uint32_t lds_all[WPG][kWords];
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int64_t gw = xcd_tile(blockIdx.x, gridDim.x) * WPG + wave;
  if (gw >= nwaves) return;
  const int part = (int)(gw % DS);
  const int64_t unit = gw / DS;
  const int b = (int)(unit / c.H), h = (int)(unit - (int64_t)b * c.H);
  const int g = h / c.hpg, m = lane & 15, q = lane >> 4, rb0 = part * NRB;
  uint16_t *xT = reinterpret_cast<uint16_t *>(lds_all[wave]);
  float *cbw = reinterpret_cast<float *>(lds_all[wave] + kXTWords);

  // the part's rows of the tile as soon as the slot is known (an out-of-range
  // slot loads slot 0's page, in bounds and never used), then the entry's
  // words, then the window and the group's C and B rows
  const int slot0 = s.slot_idx[b];
  const bool slot_ok = slot0 > 0 && slot0 < c.num_slots;
  HeadLoads<ST, KW> ld;
  load_state<ST, KW, NRB>(c, slot_ok ? slot0 : 0, h, lane, ld, rb0);
  __builtin_amdgcn_sched_barrier(0);
  const Entry e = make_entry(c, s, slot0, load_entry_in(c, s, b, slot0, slot_ok), h == 0 && part == 0);
  if (e.mode == 0) return;
  if (e.mode == 1) {
    if (part == 0) zero_out_head<OT>(s, c.H, e, h, lane);
    return;
  }
  if (e.Tb == 0) return;  // no new token: nothing to read out or append
  load_window<ST, OT, KW, false, true>(c, s, e, h, lane, ld);
  ItemLoads<ST, KW> il;
  if constexpr (ST == kF32)
    load_item_c<ST, KW>(c, s, e, g, lane, il);
  else
    load_item_c_flat<ST, KW>(c, s, e, g, lane, il);
  CbLoads<KW> cl;
  load_cb_flat<KW>(c, s, e, g, lane, cl);
  {
    f32x4 cb[KW / 16];
    cb_tiles<KW>(cl, cb, nullptr);
    if (h % c.hpg == 0 && part == 0) append_B_rows<KW>(c, e, g, lane, cl, false);
#pragma unroll
    for (int nb = 0; nb < KW / 16; ++nb)
#pragma unroll
      for (int j = 0; j < 4; ++j) cbw[(4 * q + j) * kCbLds + nb * 16 + m] = cb[nb][j];
  }
  wave_sync();  // C.B rows written by this wave -> read below
  load_cb_row<ST, KW>(e, cbw, kCbLds, lane, il);
  wave_sync();  // C.B rows read before the LDS words are reused
  head_compute<ST, OT, KW, false, NRB>(c, s, e, h, ld, il, xT, lds_all[wave], lane, nullptr, rb0, part == 0);
}

// Ring bookkeeping after a flush: ring_start <- (ring_start + k) mod L.
template <int ST>
__global__ void ring_advance_kernel(KCache c, const int32_t *slot_idx, const int32_t *num_fold, int n) {
  const int j = blockIdx.x * blockDim.x + threadIdx.x;
  if (j >= n) return;
  const int slot = slot_idx[j], k = num_fold[j];
  if (slot <= 0 || slot >= c.num_slots || k <= 0 || k > c.L) return;
  const int r = c.ring_start[slot];
  if (r < 0 || r >= c.L) return;
  c.ring_start[slot] = ring_pos(r, k, c.L);
}

// ---------------------------------------------------------------------------
// INIT: encode fp32 prefill states (one workgroup per (entry, head), row
// block w per wave: lane 16 q + m encodes quarter q of row 16 w + m) and
// clear the slot's rings.
// ---------------------------------------------------------------------------

// NVFP4 init, first pass: the largest |value| of every head of the prefill
// states (word 1 + h of the slot's scale words), from which init_rows_kernel
// takes the slot's second-level scale.  Same geometry as init_rows_kernel.
template <int ST>
__global__ __launch_bounds__(kWaves * 64) void init_max_kernel(KCache c, const float *states,
                                                               int64_t states_stride, const int32_t *slot_idx) {
  static_assert(ST == kNVFP4, "only an nvfp4 checkpoint has a slot scale");
  const int j = blockIdx.x / c.H, h = blockIdx.x - j * c.H;
  const int slot = slot_idx[j];
  if (slot <= 0 || slot >= c.num_slots) return;
  const int rb = threadIdx.x >> 6, lane = threadIdx.x & 63, m = lane & 15, q = lane >> 4;
  const float *src = states + (int64_t)j * states_stride + (int64_t)h * kHeadElems +
                     (16 * rb + m) * kDState + 32 * q;
  f32x4 acc[8];
#pragma unroll
  for (int u = 0; u < 8; ++u) {
    const f32x4 a = *reinterpret_cast<const f32x4 *>(src + 4 * u);
#pragma unroll
    for (int e = 0; e < 4; ++e) QV(acc, 4 * u + e) = a[e];
  }
  __shared__ float wmax[kWaves];
  const f32x2 b2 = block_max2(acc);
  const float mx = wave_max(fmaxf(b2[0], b2[1]), lane);
  if (lane == 0) wmax[rb] = mx;
  __syncthreads();
  if (threadIdx.x == 0) nvfp4_words(c, slot)[1 + h] = fmaxf(fmaxf(wmax[0], wmax[1]), fmaxf(wmax[2], wmax[3]));
}

template <int ST>
__global__ __launch_bounds__(kWaves * 64) void init_rows_kernel(KCache c, const float *states,
                                                                int64_t states_stride,
                                                                const int32_t *slot_idx) {
  static_assert(kWaves == 4, "one row block per wave");
  const int j = blockIdx.x / c.H, h = blockIdx.x - j * c.H;
  const int slot = slot_idx[j];
  if (slot <= 0 || slot >= c.num_slots) return;
  const int rb = threadIdx.x >> 6, lane = threadIdx.x & 63, m = lane & 15, q = lane >> 4;
  uint8_t *hp = c.state + (int64_t)slot * c.state_stride + (int64_t)h * st_head_bytes(ST);
  const float *src = states + (int64_t)j * states_stride + (int64_t)h * kHeadElems +
                     (16 * rb + m) * kDState + 32 * q;
  f32x4 acc[8];
#pragma unroll
  for (int u = 0; u < 8; ++u) {
    const f32x4 a = *reinterpret_cast<const f32x4 *>(src + 4 * u);
#pragma unroll
    for (int e = 0; e < 4; ++e) QV(acc, 4 * u + e) = a[e];
  }
  if constexpr (ST == kNVFP4) {
    // the slot's scale from every head's maximum (init_max_kernel ran first)
    const float g = slot_scale(c, slot, lane, head_max_load(c, slot, lane));
    const f32x2 b2 = block_max2(acc);
    float y0, y1;
    const uint32_t s0 = nvfp4_block_scale(b2[0], g, y0), s1 = nvfp4_block_scale(b2[1], g, y1);
    u32x4 ch[1] = {nvfp4_encode_quarter(acc, y0, y1)};
    store_chunks<ST>(hp, rb, lane, ch);
    *reinterpret_cast<uint16_t *>(c.scale + (int64_t)slot * c.scale_stride + (int64_t)h * (kHeadElems / 16) +
                                  lane * 8 + rb * 2) = (uint16_t)(s0 | (s1 << 8));
    if (h == 0 && threadIdx.x == 0) nvfp4_words(c, slot)[0] = g;
  } else {
    float sc = 1.f, y = 1.f;
    bool fast = true;
    if constexpr (ST == kFP8) {
      sc = fp8_row_scale(quarter_row_max(acc));
      y = 1.0f / sc;
      fast = __all(scale_fast(sc));
      if (q == 0) reinterpret_cast<float *>(c.scale + (int64_t)slot * c.scale_stride)[h * kHeadDim + 16 * rb + m] = sc;
    }
    u32x4 ch[st_chunks(ST)];
    encode_quarter<ST>(acc, sc, y, fast, ch);
    store_chunks<ST>(hp, rb, lane, ch);
  }
  if constexpr (ST == kFP8 || ST == kNVFP4) {
    if (c.recur) {  // separate checkpoints: the FP16 recurrence one, stochastically rounded
      u32x4 rch[4];
      encode_quarter_sr(acc, c, slot, h, 16 * rb + m, q, rch);
      store_chunks<kF16>(c.recur + (int64_t)slot * c.recur_stride + (int64_t)h * (kHeadElems * 2), rb, lane,
                         rch);
    }
  }
}

__device__ __forceinline__ void zero_bytes(uint8_t *p, int64_t nbytes, int tid, int nthreads) {
  const int64_t n16 = nbytes >> 4;
  const u32x4 z = {0u, 0u, 0u, 0u};
  for (int64_t i = tid; i < n16; i += nthreads) st16(p + 16 * i, z);
  for (int64_t i = (n16 << 4) + 4 * tid; i < nbytes; i += 4 * (int64_t)nthreads)
    *reinterpret_cast<uint32_t *>(p + i) = 0u;
}

template <int ST>
__global__ __launch_bounds__(256) void init_clear_kernel(KCache c, const int32_t *slot_idx) {
  const int slot = slot_idx[blockIdx.x];
  if (slot <= 0 || slot >= c.num_slots) return;
  const int tid = threadIdx.x;
  zero_bytes(c.xc + (int64_t)slot * c.x_stride, (int64_t)c.H * c.L * kHeadDim * 2, tid, 256);
  zero_bytes(c.Bc + (int64_t)slot * c.B_stride, (int64_t)c.G * c.L * kDState * 2, tid, 256);
  zero_bytes(c.dtc + (int64_t)slot * c.dt_stride, (int64_t)c.H * c.L * 4, tid, 256);
  if (tid == 0) c.ring_start[slot] = 0;
}

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------

namespace {

template <typename K>
int resident_blocks(K kernel, int lds_dynamic) {
  int dev = 0, cus = 0, per_cu = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 1024;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) cus = 256;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, kWaves * 64, lds_dynamic) !=
          hipSuccess ||
      per_cu < 1)
    per_cu = 1;
  return cus * per_cu;
}

// Heads per work item: the whole group unless that leaves fewer items than
// the GPU runs waves at once, then the group is split into d chunks.
int chunks_per_group(int64_t batch, int G, int hpg, int64_t resident_waves) {
  for (int d = 1; d <= hpg; ++d)
    if (hpg % d == 0 && batch * G * d >= resident_waves) return d;
  return hpg;
}

// Blocks of a kernel resident on the current device, from the occupancy
// query, remembered per device (devices 0..63; others query every call).  A
// host-side query: no stream operation, so a first call inside a HIP graph
// capture is fine.
template <typename K>
int resident_on_device(K kernel, std::atomic<int> *cache) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) dev = -1;
  if (dev >= 0 && dev < 64) {
    int r = cache[dev].load(std::memory_order_relaxed);
    if (r == 0) {
      r = resident_blocks(kernel, 0);
      cache[dev].store(r, std::memory_order_relaxed);
    }
    return r;
  }
  return resident_blocks(kernel, 0);
}

template <int ST, int OT, int KW, bool SPLIT, bool HAS_Z>
hipError_t replay_kw(const KCache &c, const KStep &s, hipStream_t st) {
  static std::atomic<int> cache[64];  // per template instance, per device
  const int resident = resident_on_device(replay_kernel<ST, OT, KW, SPLIT, HAS_Z>, cache);
  if (SPLIT) {
    const int64_t pre_items = (int64_t)s.batch * c.G;
    precompute_kernel<KW, cb_qorder(ST)><<<dim3((unsigned)((pre_items + kWaves - 1) / kWaves)), dim3(kWaves * 64), 0, st>>>(c, s);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
  }
  const int d = chunks_per_group(s.batch, c.G, c.hpg, (int64_t)resident * kWaves);
  const int64_t items = (int64_t)s.batch * c.G * d;
  const int64_t need = (items + kWaves - 1) / kWaves;
  const int64_t blocks = need < resident ? need : resident;
  replay_kernel<ST, OT, KW, SPLIT, HAS_Z><<<dim3((unsigned)blocks), dim3(kWaves * 64), 0, st>>>(c, s, d);
  return hipGetLastError();
}

// Ring bookkeeping after a fused step: ring_start <- ring_start + k for every
// entry the step folded (same validity rules as the step itself).  A separate
// launch on the same stream: counting the heads of a slot with an atomic
// inside the step (one address per slot, hit by every head at once) measured
// ~15 % slower than this launch inside a captured graph.
template <int ST>
__global__ void step_ring_advance_kernel(KCache c, KStep s) {
  const int b = blockIdx.x * blockDim.x + threadIdx.x;
  if (b >= s.batch) return;
  // the slot, then every other word at once: two memory round trips, not a
  // chain of one per check
  const int slot = s.slot_idx[b];
  const bool slot_ok = slot > 0 && slot < c.num_slots;
  const Entry e = make_entry(c, s, slot, load_entry_in<false>(c, s, b, slot, slot_ok), false);
  if (e.mode == 2 && e.k > 0) c.ring_start[e.slot] = e.r;
}

// The fused kernel at WPG heads per workgroup (with an NVFP4 fold, the maxima
// pass first: the encode needs the slot's scale).
template <int ST, int OT, bool HAS_Z, bool SEP, int WPG>
hipError_t fused_launch(const KCache &c, const KStep &s, hipStream_t st) {
  const int htiles = (c.H + WPG - 1) / WPG;
  const int64_t ntiles = (int64_t)s.batch * htiles;
  if constexpr (ST == kNVFP4) {
    if (s.fold) {
      if (c.L <= 16)
        fold_max_kernel<16, true, WPG><<<dim3(xcd_grid(ntiles)), dim3(WPG * 64), 0, st>>>(c, s, nullptr, nullptr,
                                                                                         nullptr, htiles, ntiles);
      else
        fold_max_kernel<32, true, WPG><<<dim3(xcd_grid(ntiles)), dim3(WPG * 64), 0, st>>>(c, s, nullptr, nullptr,
                                                                                         nullptr, htiles, ntiles);
      const hipError_t err = hipGetLastError();
      if (err != hipSuccess) return err;
    }
  }
  if (c.L <= 16)
    fused_kernel<ST, OT, 16, HAS_Z, SEP, WPG><<<dim3(xcd_grid(ntiles)), dim3(WPG * 64), 0, st>>>(c, s, htiles, ntiles);
  else
    fused_kernel<ST, OT, 32, HAS_Z, SEP, WPG><<<dim3(xcd_grid(ntiles)), dim3(WPG * 64), 0, st>>>(c, s, htiles, ntiles);
  return hipGetLastError();
}

template <int ST, int OT, bool HAS_Z, bool SEP>
hipError_t fused_zs(const KCache &c, const KStep &s, hipStream_t st) {
  const hipError_t err = (int64_t)s.batch * c.H <= kFusedOneWaveMax ? fused_launch<ST, OT, HAS_Z, SEP, 1>(c, s, st)
                                                                     : fused_launch<ST, OT, HAS_Z, SEP, kHeadWaves>(c, s, st);
  if (err != hipSuccess || !s.fold) return err;  // nothing folded: ring_start stays
  step_ring_advance_kernel<ST><<<dim3((unsigned)((s.batch + 255) / 256)), dim3(256), 0, st>>>(c, s);
  return hipGetLastError();
}

// Separate checkpoints exist for the fp8 read checkpoint only (the API
// rejects recur_state with any other state type).
template <int ST, int OT, bool HAS_Z>
hipError_t fused_z(const KCache &c, const KStep &s, hipStream_t st) {
  if constexpr (ST == kNVFP4) {  // an nvfp4 read checkpoint always comes with the recurrence checkpoint
    return fused_zs<ST, OT, HAS_Z, true>(c, s, st);
  } else {
    if constexpr (ST == kFP8) {
      if (c.recur) return fused_zs<ST, OT, HAS_Z, true>(c, s, st);
    }
    return fused_zs<ST, OT, HAS_Z, false>(c, s, st);
  }
}

template <int ST, int OT, bool HAS_Z>
hipError_t pair_z(const KCache &c, const KStep &s, hipStream_t st) {
  if constexpr (ST == kBF16 || ST == kF16) {
    const int ptiles = c.H / kPairHeads;
    const int64_t ntiles = (int64_t)s.batch * ptiles;
    pair_kernel<ST, OT, 16, HAS_Z><<<dim3(xcd_grid(ntiles)), dim3(kHeadWaves * 64), 0, st>>>(c, s, ptiles, ntiles);
    return hipGetLastError();
  } else {
    return hipErrorInvalidValue;
  }
}

// (entry, head) pairs up to which plain 16-bit steps split each head's rows
// over 2 waves, and over 4 (fp32 plain steps split at every size, in 4 parts
// up to SSU_DSPLIT4_MAX_UNITS pairs, else in 2).  Measured (graph-replayed
// steps, one MI355X): fp16 prod, batch 1 (128 pairs): 7.25 us per step on the
// persistent kernel, 5.65 in 2 parts, 5.49 in 4; batch 4 (512): 7.90, 6.17,
// 7.55; batch 16 (2048): 12.85, 13.79, 17.64; fp32 tiny (16 pairs): 9.71,
// 6.58, 5.71; bf16 mtp (4096 pairs): 18.24, 19.58, 24.12.  Between 512 and
// 1024 pairs, in 2 parts against the persistent kernel: fp16 batch 5 (640)
// 8.17 / 8.33, 6 (768) 8.73 / 8.85, 7 (896) 9.16 / 9.06, 8 (1024) 9.81 /
// 9.46; bf16 mtp (64 heads) batch 10 (640) 7.26 / 7.54.
#ifndef SSU_DSPLIT_MAX_UNITS
#define SSU_DSPLIT_MAX_UNITS 768
#endif
#ifndef SSU_DSPLIT4_MAX_UNITS
#define SSU_DSPLIT4_MAX_UNITS 256
#endif

constexpr int64_t kDsplitOneWaveMax = 512;  // waves up to which the split runs one wave per workgroup

template <int ST, int OT, int KW, int DS>
void dsplit_launch(const KCache &c, const KStep &s, int64_t nwaves, hipStream_t st) {
  if (nwaves <= kDsplitOneWaveMax)
    dsplit_kernel<ST, OT, KW, DS, 1><<<dim3(xcd_grid(nwaves)), dim3(64), 0, st>>>(c, s, nwaves);
  else
    dsplit_kernel<ST, OT, KW, DS, kHeadWaves><<<dim3(xcd_grid((nwaves + kHeadWaves - 1) / kHeadWaves)),
                                                dim3(kHeadWaves * 64), 0, st>>>(c, s, nwaves);
}

template <int ST, int OT>
hipError_t dsplit_t(const KCache &c, const KStep &s, int ds, hipStream_t st) {
  if constexpr (ST == kF32 || ST == kBF16 || ST == kF16) {
    const int64_t nwaves = (int64_t)s.batch * c.H * ds;
    if (ds == 4) {
      if (c.L <= 16)
        dsplit_launch<ST, OT, 16, 4>(c, s, nwaves, st);
      else
        dsplit_launch<ST, OT, 32, 4>(c, s, nwaves, st);
    } else {
      if (c.L <= 16)
        dsplit_launch<ST, OT, 16, 2>(c, s, nwaves, st);
      else
        dsplit_launch<ST, OT, 32, 2>(c, s, nwaves, st);
    }
    return hipGetLastError();
  } else {
    return hipErrorInvalidValue;
  }
}

template <int ST, int OT, bool SPLIT, bool HAS_Z>
hipError_t replay_z(const KCache &c, const KStep &s, hipStream_t st) {
  return c.L <= 16 ? replay_kw<ST, OT, 16, SPLIT, HAS_Z>(c, s, st) : replay_kw<ST, OT, 32, SPLIT, HAS_Z>(c, s, st);
}

template <int ST, int OT>
hipError_t mono_t(const KCache &c, const KStep &s, hipStream_t st) {
  if (s.batch <= 0) return hipSuccess;
  if (s.fold) return s.z ? fused_z<ST, OT, true>(c, s, st) : fused_z<ST, OT, false>(c, s, st);
  // Plain steps, by checkpoint type and size (every path is the same
  // arithmetic per output value, bit for bit):
  //  - 16-bit, from SSU_PAIR_MIN_UNITS (entry, head) pairs, groups of a
  //    multiple of 8 heads, rings up to 16: two heads per wave;
  //  - fp8 without the recurrence checkpoint at any size, bf16 (other group
  //    sizes or rings) from kPerHeadPlainUnits pairs, and fp8 with the
  //    recurrence checkpoint and nvfp4 up to kFusedOneWaveMax pairs: the
  //    one-head-per-wave kernel with nothing to fold (one wave per workgroup
  //    up to kFusedOneWaveMax pairs).  fp8, 128 heads, per call against the
  //    persistent kernel: batch 1 / 2 / 4 9.24 / 9.11 / 9.79 us against
  //    10.62 / 10.34 / 10.24, batch 8 / 32 / 128 9.67 / 17.10 / 39.82 against
  //    10.94 / 18.50 / 41.94.  fp8 with the recurrence checkpoint: batch 1
  //    8.75 against 10.09, batch 32 19.91 against 17.85; nvfp4: batch 1 9.53
  //    against 10.33, batch 32 18.18 against 17.72.  Measured against the persistent kernel from
  //    32768 pairs up: bf16 1-3 % faster (batch 256-1024 of 128 heads), fp8
  //    10 % faster; fp16 1.5-5 % slower, fp8 with the recurrence checkpoint
  //    20 % and nvfp4 57 % slower (those forms of it hold more registers);
  //  - not gated: 16-bit up to SSU_DSPLIT_MAX_UNITS pairs and 32-bit at
  //    any size, each head's rows in parts (fp32 tiny at batch 128 / 256 /
  //    512 of 8 heads: 12.31 / 19.39 / 35.11 us per step against 16.06 /
  //    26.02 / 40.57 on the persistent kernel);
  //  - the rest: the persistent kernel.
  if constexpr (ST == kBF16 || ST == kF16) {
    // (rings of up to 16 entries: with a 32-deep window the two register sets spill)
    if ((int64_t)s.batch * c.H >= SSU_PAIR_MIN_UNITS && c.hpg % kPairHeads == 0 && c.L <= 16)
      return s.z ? pair_z<ST, OT, true>(c, s, st) : pair_z<ST, OT, false>(c, s, st);
  }
  if constexpr (ST == kBF16 || ST == kFP8 || ST == kNVFP4) {
    const int64_t units = (int64_t)s.batch * c.H;
    const bool big = (ST == kBF16 && units >= kPerHeadPlainUnits) || (ST == kFP8 && !c.recur);
    const bool small = (ST == kFP8 || ST == kNVFP4) && units <= kFusedOneWaveMax;
    if (big || small) return s.z ? fused_z<ST, OT, true>(c, s, st) : fused_z<ST, OT, false>(c, s, st);
  }
  if constexpr (ST == kF32 || ST == kBF16 || ST == kF16) {
    const int64_t units = (int64_t)s.batch * c.H;
    if (!s.z && (ST == kF32 || units <= SSU_DSPLIT_MAX_UNITS))
      return dsplit_t<ST, OT>(c, s, units <= SSU_DSPLIT4_MAX_UNITS ? 4 : 2, st);
  }
  return s.z ? replay_z<ST, OT, false, true>(c, s, st) : replay_z<ST, OT, false, false>(c, s, st);
}

template <int ST, int OT>
hipError_t split_t(const KCache &c, const KStep &s, hipStream_t st) {
  if (s.batch <= 0) return hipSuccess;
  return s.z ? replay_z<ST, OT, true, true>(c, s, st) : replay_z<ST, OT, true, false>(c, s, st);
}

// The flush's kernels at WPG heads per workgroup (an NVFP4 flush: the maxima
// pass first, the encode needs the slot's scale).
template <int ST, int WPG>
hipError_t flush_launch(const KCache &c, const int32_t *slot_idx, const int32_t *num_fold, const float *A, int n,
                        hipStream_t st) {
  const int htiles = (c.H + WPG - 1) / WPG;
  const int64_t ntiles = (int64_t)n * htiles;
  const dim3 grid(xcd_grid(ntiles)), block(WPG * 64);
  bool sep = ST == kNVFP4;
  if constexpr (ST == kFP8) sep = c.recur != nullptr;
  if constexpr (ST == kNVFP4) {
    const KStep none{};
    if (c.L <= 16)
      fold_max_kernel<16, false, WPG><<<grid, block, 0, st>>>(c, none, slot_idx, num_fold, A, htiles, ntiles);
    else
      fold_max_kernel<32, false, WPG><<<grid, block, 0, st>>>(c, none, slot_idx, num_fold, A, htiles, ntiles);
    const hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
  }
  if (sep) {
    if constexpr (ST == kFP8 || ST == kNVFP4) {
      if (c.L <= 16)
        flush_kernel<ST, 16, true, WPG><<<grid, block, 0, st>>>(c, slot_idx, num_fold, A, htiles, ntiles);
      else
        flush_kernel<ST, 32, true, WPG><<<grid, block, 0, st>>>(c, slot_idx, num_fold, A, htiles, ntiles);
    }
  } else {
    if constexpr (ST != kNVFP4) {
      if (c.L <= 16)
        flush_kernel<ST, 16, false, WPG><<<grid, block, 0, st>>>(c, slot_idx, num_fold, A, htiles, ntiles);
      else
        flush_kernel<ST, 32, false, WPG><<<grid, block, 0, st>>>(c, slot_idx, num_fold, A, htiles, ntiles);
    }
  }
  return hipGetLastError();
}

template <int ST>
hipError_t flush_t(const KCache &c, const int32_t *slot_idx, const int32_t *num_fold, const float *A,
                   int n, hipStream_t st) {
  const hipError_t err = (int64_t)n * c.H <= kFusedOneWaveMax ? flush_launch<ST, 1>(c, slot_idx, num_fold, A, n, st)
                                                               : flush_launch<ST, kHeadWaves>(c, slot_idx, num_fold, A, n, st);
  if (err != hipSuccess) return err;
  ring_advance_kernel<ST><<<dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st>>>(c, slot_idx, num_fold, n);
  return hipGetLastError();
}

template <int ST>
hipError_t init_t(const KCache &c, const float *states, int64_t stride, const int32_t *slot_idx, int n,
                  hipStream_t st) {
  if constexpr (ST == kNVFP4) {
    init_max_kernel<ST><<<dim3((unsigned)((int64_t)n * c.H)), dim3(kWaves * 64), 0, st>>>(c, states, stride, slot_idx);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
  }
  init_rows_kernel<ST><<<dim3((unsigned)((int64_t)n * c.H)), dim3(kWaves * 64), 0, st>>>(c, states, stride,
                                                                                         slot_idx);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  init_clear_kernel<ST><<<dim3((unsigned)n), dim3(256), 0, st>>>(c, slot_idx);
  return hipGetLastError();
}

}  // namespace

// Entry points of one state type, instantiated once per state type (each in
// its own translation unit, so the kernels compile in parallel).
template <int ST>
hipError_t replay_monolith_st(const KCache &c, const KStep &s, int out_type, hipStream_t stream) {
  return out_type == kOutF32 ? mono_t<ST, kOutF32>(c, s, stream) : mono_t<ST, kOutBF16>(c, s, stream);
}

template <int ST>
hipError_t replay_split_st(const KCache &c, const KStep &s, int out_type, hipStream_t stream) {
  return out_type == kOutF32 ? split_t<ST, kOutF32>(c, s, stream) : split_t<ST, kOutBF16>(c, s, stream);
}

template <int ST>
hipError_t flush_st(const KCache &c, const int32_t *slot_idx, const int32_t *num_fold, const float *A, int n,
                    hipStream_t stream) {
  return flush_t<ST>(c, slot_idx, num_fold, A, n, stream);
}

template <int ST>
hipError_t init_st(const KCache &c, const float *states, int64_t states_stride, const int32_t *slot_idx, int n,
                   hipStream_t stream) {
  return init_t<ST>(c, states, states_stride, slot_idx, n, stream);
}

}  // namespace ssu
