// Host entry points of libssu (see include/ssu.h): argument validation,
// monolith / split dispatch and kernel launches.  Nothing here allocates or
// synchronises; every launch goes to the caller's stream.
#include <atomic>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>

#include <hip/hip_runtime.h>

#include "../../include/ssu.h"
#include "ssu_internal.h"

namespace {

thread_local char g_err[512] = "";

// Default AUTO crossover in work units (batch * nheads).  On MI355X the
// monolith is faster than the split at every measured size (128 to 65536
// work units of fp16 with 128 heads: the split reaches 0.55-0.60 of the
// monolith's throughput up to 512 units, 0.74-0.91 from 1024 to 8192, and
// 0.89-0.90 from 16384 up), because forming C.B on MFMA inside each replay
// wave costs less than the split's extra launch and scratch round trip.  AUTO
// therefore never picks the split unless a caller lowers the threshold.
std::atomic<int64_t> g_split_threshold{INT64_MAX};

int fail(int code, const char *fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof g_err, fmt, ap);
  va_end(ap);
  return code;
}

int ok() {
  g_err[0] = '\0';
  return SSU_OK;
}

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool aligned4(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }

// A C caller may store any int in the descriptors' enum fields.  Loading a
// value outside the enumerators' range through the C++ enum type is
// undefined, so every read of such a field goes through its 32 bits.
template <class E>
int32_t raw(const E &e) {
  static_assert(sizeof(E) == sizeof(int32_t), "the ABI's enums are 32-bit");
  int32_t v;
  std::memcpy(&v, &e, sizeof v);
  return v;
}

// Bytes of one head's checkpoint.
int64_t state_head_bytes(int32_t t) {
  const int64_t e = (int64_t)ssu::kHeadDim * ssu::kDState;
  switch (t) {
    case SSU_F32: return 4 * e;
    case SSU_BF16: return 2 * e;
    case SSU_F16: return 2 * e;
    case SSU_FP8_E4M3: return e;
    case SSU_NVFP4: return e / 2;
  }
  return 0;
}

int state_type_of(int32_t t) {
  switch (t) {
    case SSU_F32: return ssu::kF32;
    case SSU_BF16: return ssu::kBF16;
    case SSU_F16: return ssu::kF16;
    case SSU_FP8_E4M3: return ssu::kFP8;
    case SSU_NVFP4: return ssu::kNVFP4;
  }
  return -1;
}

// Checks of the cache description shared by every entry point.
int check_cache(const ssu_cache *c) {
  if (!c) return fail(SSU_ERR_INVALID, "cache descriptor is NULL");
  if (c->num_slots < 1 || c->nheads < 1 || c->ngroups < 1)
    return fail(SSU_ERR_INVALID, "num_slots, nheads and ngroups must be positive (got %d, %d, %d)",
                c->num_slots, c->nheads, c->ngroups);
  if (c->nheads % c->ngroups != 0)
    return fail(SSU_ERR_INVALID, "nheads (%d) must be a multiple of ngroups (%d)", c->nheads, c->ngroups);
  if (c->headdim != ssu::kHeadDim || c->dstate != ssu::kDState)
    return fail(SSU_ERR_UNSUPPORTED, "only headdim 64 and dstate 128 are implemented (got %d, %d)",
                c->headdim, c->dstate);
  if (c->ring_len < 1 || c->ring_len > ssu::kMaxRing)
    return fail(SSU_ERR_UNSUPPORTED, "ring_len must be in [1, %d] (got %d)", ssu::kMaxRing, c->ring_len);
  const int32_t sd = raw(c->state_dtype);
  if (state_type_of(sd) < 0) return fail(SSU_ERR_INVALID, "unknown state_dtype %d", sd);
  if (raw(c->io_dtype) != SSU_BF16)
    return fail(SSU_ERR_UNSUPPORTED, "io_dtype must be SSU_BF16 (x, B, C and the x/B rings)");
  if (!c->state || !c->x_cache || !c->B_cache || !c->dt_cache || !c->ring_start)
    return fail(SSU_ERR_INVALID, "cache tensors must not be NULL");
  const bool nvfp4 = sd == SSU_NVFP4;
  if ((sd == SSU_FP8_E4M3 || nvfp4) && !c->state_scale)
    return fail(SSU_ERR_INVALID, "fp8 and nvfp4 states require state_scale");
  if (nvfp4 && !c->state_gscale)
    return fail(SSU_ERR_INVALID, "nvfp4 state requires state_gscale");
  if (nvfp4 && !c->recur_state)
    return fail(SSU_ERR_UNSUPPORTED, "an nvfp4 read checkpoint requires recur_state (separate checkpoints)");
  if (c->recur_state && sd != SSU_FP8_E4M3 && !nvfp4)
    return fail(SSU_ERR_UNSUPPORTED, "recur_state (separate checkpoints) requires an fp8 or nvfp4 state");
  if (c->state_gscale && !aligned16(c->state_gscale))
    return fail(SSU_ERR_INVALID, "state_gscale must be 16-byte aligned");
  if (c->recur_state && !aligned16(c->recur_state))
    return fail(SSU_ERR_INVALID, "recur_state must be 16-byte aligned");
  if (!aligned16(c->state) || !aligned16(c->x_cache) || !aligned16(c->B_cache) || !aligned16(c->dt_cache) ||
      (c->state_scale && !aligned16(c->state_scale)) || !aligned4(c->ring_start) ||
      (c->status && !aligned4(c->status)))
    return fail(SSU_ERR_INVALID, "cache pointers must be 16-byte aligned (ring_start, status: 4-byte)");
  const int64_t H = c->nheads, G = c->ngroups, L = c->ring_len;
  const int64_t need_state = H * state_head_bytes(sd);
  struct {
    const char *name;
    int64_t stride, need;
    bool used;
  } s[] = {
      {"state", c->state_slot_stride, need_state, true},
      {"state_scale", c->scale_slot_stride, nvfp4 ? H * ssu::kHeadDim * ssu::kDState / 16 : H * ssu::kHeadDim * 4,
       sd == SSU_FP8_E4M3 || nvfp4},
      {"state_gscale", c->gscale_slot_stride, (1 + H) * 4, nvfp4},
      {"x_cache", c->x_slot_stride, H * L * ssu::kHeadDim * 2, true},
      {"B_cache", c->B_slot_stride, G * L * ssu::kDState * 2, true},
      {"dt_cache", c->dt_slot_stride, H * L * 4, true},
      {"recur_state", c->recur_slot_stride, H * ssu::kHeadDim * ssu::kDState * 2, c->recur_state != nullptr},
  };
  for (auto &t : s) {
    if (!t.used) continue;
    if (t.stride < t.need)
      return fail(SSU_ERR_INVALID, "%s slot stride %lld is smaller than one packed slot (%lld bytes)",
                  t.name, (long long)t.stride, (long long)t.need);
    if (t.stride % 16 != 0)
      return fail(SSU_ERR_INVALID, "%s slot stride %lld is not a multiple of 16 bytes", t.name,
                  (long long)t.stride);
  }
  return SSU_OK;
}

ssu::KCache kcache(const ssu_cache *c, uint64_t seed) {
  ssu::KCache k;
  k.state = static_cast<uint8_t *>(c->state);
  k.state_stride = c->state_slot_stride;
  k.scale = reinterpret_cast<uint8_t *>(c->state_scale);
  k.scale_stride = c->scale_slot_stride;
  k.xc = static_cast<uint8_t *>(c->x_cache);
  k.x_stride = c->x_slot_stride;
  k.Bc = static_cast<uint8_t *>(c->B_cache);
  k.B_stride = c->B_slot_stride;
  k.dtc = reinterpret_cast<uint8_t *>(c->dt_cache);
  k.dt_stride = c->dt_slot_stride;
  k.ring_start = c->ring_start;
  k.status = c->status;
  k.num_slots = c->num_slots;
  k.H = c->nheads;
  k.G = c->ngroups;
  k.L = c->ring_len;
  k.hpg = c->nheads / c->ngroups;
  k.recur = static_cast<uint8_t *>(c->recur_state);
  k.recur_stride = c->recur_slot_stride;
  k.seed_lo = (uint32_t)seed;
  k.seed_hi = (uint32_t)(seed >> 32);
  k.gw = reinterpret_cast<uint8_t *>(c->state_gscale);
  k.gw_stride = c->gscale_slot_stride;
  return k;
}

size_t split_bytes(const ssu_cache *c, int64_t batch, int64_t T) {
  return (size_t)(batch * c->ngroups * T * ssu::kCbStride * (int64_t)sizeof(float));
}

int check_step(const ssu_cache *c, const ssu_step *s) {
  if (!s) return fail(SSU_ERR_INVALID, "step descriptor is NULL");
  if (s->batch < 0) return fail(SSU_ERR_INVALID, "batch must be >= 0 (got %d)", s->batch);
  const int tmax = c->ring_len < ssu::kMaxTokens ? c->ring_len : ssu::kMaxTokens;
  if (s->max_seqlen < 1) return fail(SSU_ERR_INVALID, "max_seqlen must be >= 1 (got %d)", s->max_seqlen);
  if (s->max_seqlen > tmax)
    return fail(s->max_seqlen > c->ring_len ? SSU_ERR_INVALID : SSU_ERR_UNSUPPORTED,
                "max_seqlen %d exceeds min(16, ring_len) = %d", s->max_seqlen, tmax);
  if (s->batch == 0) return SSU_OK;
  if ((int64_t)s->batch * c->nheads > SSU_MAX_PAIRS)
    return fail(SSU_ERR_UNSUPPORTED, "batch %d x nheads %d exceeds SSU_MAX_PAIRS (%d) (entry, head) pairs per call",
                s->batch, c->nheads, SSU_MAX_PAIRS);
  if (!s->slot_idx || !s->prev_num_accepted || !s->x || !s->B || !s->C || !s->dt || !s->A || !s->D ||
      !s->dt_bias || !s->out)
    return fail(SSU_ERR_INVALID, "step tensors must not be NULL (cu_seqlens and workspace may be)");
  const int32_t od = raw(s->out_dtype), algo = raw(s->algo);
  if (od != SSU_BF16 && od != SSU_F32) return fail(SSU_ERR_UNSUPPORTED, "out_dtype must be SSU_BF16 or SSU_F32");
  if (!aligned16(s->x) || !aligned16(s->B) || !aligned16(s->C) || !aligned16(s->out))
    return fail(SSU_ERR_INVALID, "x, B, C and out must be 16-byte aligned");
  if (!aligned4(s->dt) || !aligned4(s->A) || !aligned4(s->D) || !aligned4(s->dt_bias) ||
      !aligned4(s->slot_idx) || !aligned4(s->prev_num_accepted) || (s->cu_seqlens && !aligned4(s->cu_seqlens)))
    return fail(SSU_ERR_INVALID, "dt, A, D, dt_bias and the index arrays must be 4-byte aligned");
  if (algo != SSU_ALGO_AUTO && algo != SSU_ALGO_MONOLITH && algo != SSU_ALGO_SPLIT)
    return fail(SSU_ERR_INVALID, "unknown algo %d", algo);
  if (s->num_fold && !aligned4(s->num_fold)) return fail(SSU_ERR_INVALID, "num_fold must be 4-byte aligned");
  if (s->z && !aligned16(s->z)) return fail(SSU_ERR_INVALID, "z must be 16-byte aligned");
  if (s->num_fold && algo == SSU_ALGO_SPLIT)
    return fail(SSU_ERR_UNSUPPORTED, "the fused flush (num_fold) runs in the monolith only; use AUTO or MONOLITH");
  return SSU_OK;
}

// The scratch of ssu_replay_step_noalloc: a file-scope device array (one
// copy per GPU, held until the process ends).  In host code `scratch` names a
// host-side stand-in, not device memory: its device address is looked up per
// device with hipGetSymbolAddress, and only that address is passed on.
constexpr size_t kNoAllocBytes = SSU_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[kNoAllocBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_dev[kMaxDevices] = {};

// The current device's address of `scratch`, looked up on the first call on
// that device.
int scratch_of_current_device(void **out) {
  int dev = -1;
  hipError_t err = hipGetDevice(&dev);
  if (err != hipSuccess) return fail(SSU_ERR_HIP, "hipGetDevice failed: %s", hipGetErrorString(err));
  if (dev < 0 || dev >= kMaxDevices)
    return fail(SSU_ERR_UNSUPPORTED, "device %d: the no-allocation scratch serves devices 0..%d", dev,
                kMaxDevices - 1);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_dev[dev]) {
    void *p = nullptr;
    err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (err != hipSuccess || !p)
      return fail(SSU_ERR_HIP, "hipGetSymbolAddress of the scratch array failed on device %d: %s", dev,
                  hipGetErrorString(err));
    g_scratch_dev[dev] = p;
  }
  *out = g_scratch_dev[dev];
  return SSU_OK;
}

int resolve(const ssu_cache *c, const ssu_step *s) {
  const int32_t algo = raw(s->algo);
  if (algo == SSU_ALGO_MONOLITH || algo == SSU_ALGO_SPLIT) return algo;
  if (s->num_fold) return SSU_ALGO_MONOLITH;
  const int64_t units = (int64_t)s->batch * c->nheads;
  return units >= g_split_threshold.load(std::memory_order_relaxed) ? SSU_ALGO_SPLIT : SSU_ALGO_MONOLITH;
}

}  // namespace

extern "C" {

const char *ssu_last_error(void) { return g_err; }

int64_t ssu_get_split_threshold(void) { return g_split_threshold.load(); }

int64_t ssu_set_split_threshold(int64_t work_units) { return g_split_threshold.exchange(work_units); }

size_t ssu_workspace_size(const ssu_cache *cache, int32_t batch, int32_t max_seqlen) {
  if (check_cache(cache) != SSU_OK) return 0;
  const int tmax = cache->ring_len < ssu::kMaxTokens ? cache->ring_len : ssu::kMaxTokens;
  if (batch < 0 || max_seqlen < 0 || max_seqlen > tmax) {
    fail(SSU_ERR_INVALID, "workspace for batch %d, max_seqlen %d: need batch >= 0 and 0 <= max_seqlen <= %d", batch,
         max_seqlen, tmax);
    return 0;
  }
  if ((int64_t)batch * cache->nheads > SSU_MAX_PAIRS) {
    fail(SSU_ERR_UNSUPPORTED, "batch %d x nheads %d exceeds SSU_MAX_PAIRS (%d)", batch, cache->nheads,
         SSU_MAX_PAIRS);
    return 0;
  }
  ok();
  return split_bytes(cache, batch, max_seqlen);
}

int ssu_resolve_algo(const ssu_cache *cache, const ssu_step *step) {
  int rc = check_cache(cache);
  if (rc != SSU_OK) return rc;
  rc = check_step(cache, step);
  if (rc != SSU_OK) return rc;
  ok();
  return resolve(cache, step);
}

}  // extern "C"

namespace {

// ssu_replay_step after validation, with the SPLIT scratch `ws` of ws_bytes
// bytes (the caller's workspace or the no-allocation array).
int replay_step_checked(const ssu_cache *cache, const ssu_step *step, int algo, void *ws, size_t ws_bytes,
                        hipStream_t stream) {
  ssu::KStep k;
  k.batch = step->batch;
  k.T = step->max_seqlen;
  k.slot_idx = step->slot_idx;
  k.pnat = step->prev_num_accepted;
  k.cu = step->cu_seqlens;
  k.fold = step->num_fold;
  k.z = static_cast<const uint16_t *>(step->z);
  k.dt_softplus = step->no_dt_softplus ? 0 : 1;
  k.x = static_cast<const uint16_t *>(step->x);
  k.B = static_cast<const uint16_t *>(step->B);
  k.C = static_cast<const uint16_t *>(step->C);
  k.dt = step->dt;
  k.A = step->A;
  k.D = step->D;
  k.dt_bias = step->dt_bias;
  k.out = step->out;
  k.cb = nullptr;
  const int st = state_type_of(raw(cache->state_dtype));
  const int ot = raw(step->out_dtype) == SSU_F32 ? ssu::kOutF32 : ssu::kOutBF16;
  hipError_t err;
  if (algo == SSU_ALGO_SPLIT) {
    const size_t need = split_bytes(cache, step->batch, step->max_seqlen);
    if (!ws || ws_bytes < need)
      return fail(SSU_ERR_WORKSPACE, "SPLIT needs a workspace of %zu bytes (got %zu%s)", need, ws_bytes,
                  ws ? "" : ", NULL");
    if (!aligned16(ws)) return fail(SSU_ERR_INVALID, "workspace must be 16-byte aligned");
    k.cb = static_cast<float *>(ws);
    err = ssu::launch_replay_split(kcache(cache, step->sr_seed), k, st, ot, stream);
  } else {
    err = ssu::launch_replay_monolith(kcache(cache, step->sr_seed), k, st, ot, stream);
  }
  if (err != hipSuccess) return fail(SSU_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(err));
  return ok();
}

}  // namespace

extern "C" {

int ssu_replay_step(const ssu_cache *cache, const ssu_step *step, hipStream_t stream) {
  int rc = check_cache(cache);
  if (rc != SSU_OK) return rc;
  rc = check_step(cache, step);
  if (rc != SSU_OK) return rc;
  if (step->batch == 0) return ok();
  return replay_step_checked(cache, step, resolve(cache, step), step->workspace, step->workspace_bytes, stream);
}

int ssu_replay_step_noalloc(const ssu_cache *cache, const ssu_step *step, hipStream_t stream) {
  int rc = check_cache(cache);
  if (rc != SSU_OK) return rc;
  rc = check_step(cache, step);
  if (rc != SSU_OK) return rc;
  if (step->batch == 0) return ok();
  const int algo = resolve(cache, step);
  if (algo != SSU_ALGO_SPLIT) return replay_step_checked(cache, step, algo, nullptr, 0, stream);
  const size_t need = split_bytes(cache, step->batch, step->max_seqlen);
  if (need > kNoAllocBytes)
    return fail(SSU_ERR_WORKSPACE,
                "ssu_replay_step_noalloc: SPLIT needs %zu bytes of scratch for batch %d, max_seqlen %d, %d groups; "
                "the library's array holds %zu (SSU_NOALLOC_SCRATCH_BYTES)",
                need, step->batch, step->max_seqlen, cache->ngroups, kNoAllocBytes);
  void *ws = nullptr;
  rc = scratch_of_current_device(&ws);
  if (rc != SSU_OK) return rc;
  return replay_step_checked(cache, step, algo, ws, kNoAllocBytes, stream);
}

int ssu_flush(const ssu_cache *cache, const int32_t *slot_idx, const int32_t *num_fold, const float *A,
              int32_t n, uint64_t sr_seed, hipStream_t stream) {
  int rc = check_cache(cache);
  if (rc != SSU_OK) return rc;
  if (n < 0) return fail(SSU_ERR_INVALID, "n must be >= 0 (got %d)", n);
  if (n == 0) return ok();
  if ((int64_t)n * cache->nheads > SSU_MAX_PAIRS)
    return fail(SSU_ERR_UNSUPPORTED, "n %d x nheads %d exceeds SSU_MAX_PAIRS (%d) (entry, head) pairs per call", n,
                cache->nheads, SSU_MAX_PAIRS);
  if (!slot_idx || !num_fold || !A) return fail(SSU_ERR_INVALID, "slot_idx, num_fold and A must not be NULL");
  if (!aligned4(slot_idx) || !aligned4(num_fold) || !aligned4(A))
    return fail(SSU_ERR_INVALID, "slot_idx, num_fold and A must be 4-byte aligned");
  hipError_t err = ssu::launch_flush(kcache(cache, sr_seed), slot_idx, num_fold, A, n,
                                     state_type_of(raw(cache->state_dtype)), stream);
  if (err != hipSuccess) return fail(SSU_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(err));
  return ok();
}

int ssu_init_state(const ssu_cache *cache, const float *states, int64_t states_batch_stride,
                   const int32_t *slot_idx, int32_t n, uint64_t sr_seed, hipStream_t stream) {
  int rc = check_cache(cache);
  if (rc != SSU_OK) return rc;
  if (n < 0) return fail(SSU_ERR_INVALID, "n must be >= 0 (got %d)", n);
  if (n == 0) return ok();
  if ((int64_t)n * cache->nheads > SSU_MAX_PAIRS)
    return fail(SSU_ERR_UNSUPPORTED, "n %d x nheads %d exceeds SSU_MAX_PAIRS (%d) (entry, head) pairs per call", n,
                cache->nheads, SSU_MAX_PAIRS);
  if (!states || !slot_idx) return fail(SSU_ERR_INVALID, "states and slot_idx must not be NULL");
  if (states_batch_stride < 0) return fail(SSU_ERR_INVALID, "states_batch_stride must be >= 0");
  if (!aligned16(states) || states_batch_stride % 4 != 0 || !aligned4(slot_idx))
    return fail(SSU_ERR_INVALID, "states must be 16-byte aligned with a stride that is a multiple of 4");
  hipError_t err = ssu::launch_init(kcache(cache, sr_seed), states, states_batch_stride, slot_idx, n,
                                    state_type_of(raw(cache->state_dtype)), stream);
  if (err != hipSuccess) return fail(SSU_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(err));
  return ok();
}

}  // extern "C"
