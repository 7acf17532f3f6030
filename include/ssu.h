/*
 * ssu.h -- C ABI of libssu: the checkpointing selective state update
 * (ReplaySSM / MTP-replay SSU) of Mamba-2 speculative decode, for AMD
 * Instinct MI355X (gfx950).
 *
 * For every cache slot (one request) and head the library keeps a checkpoint
 * state h[headdim=64][dstate=128] and head-major rings holding the inputs of
 * the accepted tokens that are not yet folded into it.  A replay step reads
 * the checkpoint, replays it through the live ring tokens and this step's new
 * (draft) tokens, writes one output row per new token and appends the new
 * tokens to the ring; a flush folds accepted tokens into the checkpoint.
 *
 * Sources, by page and section:
 *  [FI]  FlashInfer PR "mamba checkpointing SSU: two-kernel split +
 *        ring-buffer cache for checkpointing SSU" -- Description item 1 (the
 *        two-kernel split, caller-provided graph-safe scratch, auto-dispatch
 *        on batch x nheads, the algorithm override) and item 2 (the ring
 *        contract table: x_cache, B_cache, dt_cache f32, ring_start i32; the
 *        live / append positions; the host owns ring bookkeeping; the decay
 *        prefix is recomputed, never cached).
 *  [VD]  vLLM API page "replayssm_cutedsl" -- initialize_replayssm_state
 *        (FP32 [batch, heads, 64, 128] prefill states, a stride-0 broadcast
 *        state, nonpositive / out-of-range slots ignored, rings cleared) and
 *        selective_state_update_replayssm (softplus of dt + dt_bias; per-head
 *        dt, A, dt_bias, D; per-group B and C; BF16 x, B, C and output;
 *        unique active slots; slot 0 reserved for padding; padding allowed
 *        between slot pages; invalid arguments raise ValueError).
 *  [VP]  vLLM PR "Add separate CuTeDSL ReplaySSM checkpoints" -- Overview
 *        and Claims (FP32 flush work; the FP8 read checkpoint uses nearest
 *        encoding with an FP32 scale per row; only the accepted prefix may
 *        change the checkpoint).
 *
 * Conventions for every entry point:
 *  - All tensor pointers are DEVICE pointers owned by the caller; the library
 *    never allocates, frees or synchronises, and every kernel is enqueued on
 *    the given stream (NULL = the default stream), so calls can be captured
 *    in a HIP graph.  Calls that touch the same slots must be ordered by the
 *    caller (same stream or events).
 *  - Returns SSU_OK (0) or a negative error code; nothing is launched when an
 *    error is returned.  ssu_last_error() gives the calling thread's last
 *    message.  SSU_ERR_INVALID corresponds to the pages' ValueError,
 *    SSU_ERR_UNSUPPORTED to a shape/type the kernels do not implement.
 *  - Device-side preconditions that the host cannot see (slot ids, token
 *    counts, ring positions) are checked in the kernels: a padding entry
 *    (slot <= 0 or slot >= num_slots, [VD]) writes zero output rows and
 *    touches no cache; an entry that breaks the ring contract is skipped the
 *    same way and ORs a bit into *cache->status when status is not NULL.
 *    What no kernel can check is the size of the caller's buffers: the token
 *    rows an entry addresses (b*T + t, or [cu_seqlens[b], cu_seqlens[b+1]))
 *    must lie inside x, B, C, dt, out and z, and the device index arrays
 *    must hold batch (batch + 1 for cu_seqlens) entries.
 */
#ifndef SSU_H
#define SSU_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum ssu_dtype {
  SSU_F32 = 0,
  SSU_BF16 = 1,
  SSU_F16 = 2,
  SSU_FP8_E4M3 = 3, /* OCP e4m3fn codes (max 448) with an fp32 scale per state row */
  SSU_NVFP4 = 4     /* e2m1 codes, an e4m3 scale per 16 values, one fp32 scale per slot */
} ssu_dtype;

typedef enum ssu_algo {
  SSU_ALGO_AUTO = 0,     /* monolith below the work-unit threshold, split above [FI item 1] */
  SSU_ALGO_MONOLITH = 1, /* one kernel per step (a fused step adds a small ring-advance launch, an NVFP4 fold a maxima pass) */
  SSU_ALGO_SPLIT = 2     /* precompute (C.B per group) + persistent replay kernel */
} ssu_algo;

enum {
  SSU_OK = 0,
  SSU_ERR_INVALID = -1,     /* bad argument: null pointer, shape, alignment, dtype */
  SSU_ERR_UNSUPPORTED = -2, /* valid but not implemented (e.g. headdim != 64) */
  SSU_ERR_HIP = -3,         /* a HIP launch / runtime call failed */
  SSU_ERR_WORKSPACE = -4    /* SPLIT chosen and workspace missing or too small */
};

/* Bits ORed into *ssu_cache.status by the kernels (device-side checks). */
enum {
  SSU_STATUS_BAD_PNAT = 1,   /* replay entry with pnat < 0 or pnat + T_b > ring_len */
  SSU_STATUS_BAD_FOLD = 2,   /* flush entry with k < 0 or k > ring_len */
  SSU_STATUS_BAD_SEQLEN = 4, /* varlen entry with T_b < 0 or T_b > max_seqlen */
  SSU_STATUS_BAD_RING = 8    /* ring_start[slot] outside [0, ring_len) */
};

/*
 * The per-slot cache [FI item 2; VD].  Inside one slot page every tensor is
 * packed; *_slot_stride is the distance in BYTES between slot pages (it may
 * include padding).  Layouts:
 *   state       [slot][nheads][64 * 128]         state_dtype, MFMA-tiled (below)
 *   state_scale [slot][nheads][headdim]          f32, fp8 state only: the row's
 *                                                value is code * scale
 *               [slot][nheads][512]              u8, nvfp4 state: e4m3 block scales
 *   state_gscale [slot][1 + nheads]              f32, nvfp4 state only: word 0
 *                                                the slot's second-level scale,
 *                                                word 1 + h head h's largest
 *                                                |value| at its last encode
 *   x_cache     [slot][nheads][ring_len][headdim] io_dtype
 *   B_cache     [slot][ngroups][ring_len][dstate] io_dtype
 *   dt_cache    [slot][nheads][ring_len]          f32, holds dt' = softplus(dt + dt_bias)
 *   ring_start  [slot]                            i32, in [0, ring_len)
 * Live token j (j < pnat) of a slot is ring entry (ring_start + j) mod L; new
 * token i is appended at (ring_start + pnat + i) mod L.
 * Checkpoint tiling: element h[p][n] of one head (eb bytes per element) sits
 * at byte offset
 *     rb * 2048 * eb + (u * 64 + l) * 16 + (t % (16 / eb)) * eb
 * with p = 16 rb + m, n = 32 q + t, l = 16 q + m, u = t / (16 / eb).  Each
 * row is cut into four quarters of 32 values; quarter q of row 16 rb + m is
 * lane l's share of a 64-lane wave, stored as 16-byte chunks u with chunk u of
 * all 64 lanes side by side, so every 16-byte-per-lane load or store of a
 * row block is 1 KiB contiguous.  ssu_init_state writes this layout from
 * plain row-major fp32 [headdim][dstate] states.
 * Separate checkpoints [VP Overview, Claims]: recur_state [slot][nheads][64 *
 * 128] fp16 in the same tiled layout as state (or NULL for one shared
 * checkpoint).  With it, state is the read checkpoint every step reads, and
 * recur_state the recurrence checkpoint: flushes fold from it, write it back
 * with stochastic rounding (below) and write state with the nearest encoding
 * of the same fp32 result; init writes both.  Stochastic rounding: a value
 * goes to the fp16 neighbour away from zero when floor(128 f) + u >= 128,
 * f = (|v| - lo) / (hi - lo) (lo <= |v| < hi its fp16 neighbours, infinity
 * past 65504), else toward zero; u is the low 7 bits of byte e % 16 of
 * Philox4x32-10 at counter (e / 16, head, slot, 0) keyed by the call's
 * 64-bit sr_seed (e = p * 128 + n); a caller passes a different seed on
 * every call.  recur_state requires state_dtype SSU_FP8_E4M3 or SSU_NVFP4
 * (else SSU_ERR_UNSUPPORTED).
 * NVFP4 read checkpoint [VP Claims; VD initialize_replayssm_state, NVFP4
 * branch] (requires recur_state): value = e2m1(code) * e4m3(block scale) * g,
 * blocks of 16 consecutive n of a row, ONE g per slot: g = fp32(M / 2688)
 * (1 if not positive) with M the largest |value| over every head of the slot
 * (2688 = 6 * 448), as the page's init computes it.  Init and every fold write
 * the whole slot that way, with nearest encoding of the fp32 values: block
 * scale = e4m3(fp32(a / fp32(6 g))) for a block's max |v| (saturating), code
 * = e2m1(v * fp32(1 / fp32(e4m3 * g))) (nearest even, saturating at 6; a zero
 * block scale gives signed zeros).  Because g needs every head's folded
 * values, an NVFP4 fold is two launches: a pass that records each head's
 * maximum in state_gscale, then the encode.  Layout of one head: row block rb, lane
 * l = 16 q + m (row 16 rb + m, values n = 32 q + t): codes of t = 0..31 in
 * the 16 bytes at rb * 1024 + l * 16 (value t in byte t / 2, even t in the
 * low nibble); block scales (t < 16, t >= 16) in state_scale bytes
 * l * 8 + rb * 2 + 0 / 1 of the head's 512.
 * Requirements: headdim == 64, dstate == 128, nheads % ngroups == 0,
 * 1 <= ring_len <= 32, io_dtype == SSU_BF16; every pointer 16-byte aligned
 * (ring_start and status, i32 arrays: 4-byte), even one that the state dtype
 * leaves unused; the slot stride of every tensor in use at least one packed
 * page and a multiple of 16.  status may be NULL.
 */
typedef struct ssu_cache {
  int32_t num_slots, nheads, ngroups, headdim, dstate, ring_len;
  ssu_dtype state_dtype;
  ssu_dtype io_dtype;
  void *state;
  int64_t state_slot_stride;
  void *state_scale;
  int64_t scale_slot_stride;
  void *x_cache;
  int64_t x_slot_stride;
  void *B_cache;
  int64_t B_slot_stride;
  float *dt_cache;
  int64_t dt_slot_stride;
  int32_t *ring_start;
  int32_t *status;
  void *recur_state;
  int64_t recur_slot_stride;
  float *state_gscale; /* nvfp4 only, else NULL */
  int64_t gscale_slot_stride;
} ssu_cache;

/*
 * One decode step over `batch` entries [FI item 1-2; VD].
 *   slot_idx, prev_num_accepted  [batch] i32   (prev_num_accepted = pnat, the
 *                                               live ring tokens ahead of the
 *                                               new ones)
 *   cu_seqlens  [batch+1] i32 or NULL.  NULL: every entry has T = max_seqlen
 *               new tokens and token t of entry b is row b*T + t.  Otherwise
 *               entry b owns rows [cu_seqlens[b], cu_seqlens[b+1]) (varlen).
 *   x   [rows][nheads][64]   io_dtype      B, C [rows][ngroups][128] io_dtype
 *   dt  [rows][nheads] f32 (raw; softplus(dt + dt_bias) is applied here)
 *   A, D, dt_bias  [nheads] f32
 *   out [rows][nheads][64]   out_dtype (SSU_BF16 or SSU_F32)
 *   workspace / workspace_bytes: scratch for SPLIT, at least
 *               ssu_workspace_size(cache, batch, max_seqlen) bytes, 16-byte
 *               aligned; may be NULL for MONOLITH.
 *   num_fold    [batch] i32 or NULL: fused flush-in-step (see ssu_replay_step).
 *               Runs in the monolith: AUTO resolves to MONOLITH, an explicit
 *               SPLIT returns SSU_ERR_UNSUPPORTED.
 *   z           [rows][nheads][64] io_dtype or NULL: output gate; each output
 *               value is y * z * sigmoid(z), computed in fp32 before the
 *               output is rounded [FI, the HAS_Z output flag].  16-byte
 *               aligned.
 *   no_dt_softplus  0: dt' = softplus(dt + dt_bias) (the default of [VD]);
 *               nonzero: dt' = dt + dt_bias [FI, the dt_softplus flag].  The
 *               dt ring stores dt' either way.
 * Requirements: 1 <= max_seqlen <= min(16, ring_len); pointers 16-byte
 * aligned (dt, A, D, dt_bias and the i32 arrays slot_idx, prev_num_accepted,
 * cu_seqlens, num_fold: 4-byte); batch * nheads <= SSU_MAX_PAIRS (else
 * SSU_ERR_UNSUPPORTED).  Active slots must be unique.  batch == 0 is a no-op:
 * past the cache and max_seqlen checks nothing else is looked at.
 */
/* (entry, head) pairs one call may cover: every launch grid, in threads,
 * then fits 32 bits and every token row index 31 bits.  Calls past it
 * return SSU_ERR_UNSUPPORTED; split such a batch over several calls. */
#define SSU_MAX_PAIRS ((1 << 24) - 1)

typedef struct ssu_step {
  int32_t batch, max_seqlen;
  const int32_t *slot_idx;
  const int32_t *prev_num_accepted;
  const int32_t *cu_seqlens;
  const void *x;
  const void *B;
  const void *C;
  const float *dt;
  const float *A;
  const float *D;
  const float *dt_bias;
  void *out;
  ssu_dtype out_dtype;
  void *workspace;
  size_t workspace_bytes;
  ssu_algo algo;
  const int32_t *num_fold;
  const void *z;
  int32_t no_dt_softplus;
  uint64_t sr_seed; /* stochastic-rounding seed of a fused fold (separate checkpoints) */
} ssu_step;

/* Bytes of scratch the SPLIT algorithm needs for (batch, max_seqlen): the
 * fp32 C.B products of every (entry, group) [FI Description item 1: the
 * precompute writes C.B to caller-provided, graph-safe scratch, allocated by
 * the caller like the output].  Returns 0 for an invalid cache description,
 * a negative batch, a max_seqlen outside [0, min(16, ring_len)] or
 * batch * nheads > SSU_MAX_PAIRS (with the reason in ssu_last_error). */
size_t ssu_workspace_size(const ssu_cache *cache, int32_t batch, int32_t max_seqlen);

/*
 * Initialise n slots from FP32 prefill states [VD initialize_replayssm_state].
 * states: device f32, entry j at states + j * states_batch_stride elements,
 * each [nheads][64][128] packed; states_batch_stride == 0 broadcasts entry 0
 * to every slot.  For each slot_idx[j] in [1, num_slots): encode the state
 * (fp32 stored, bf16/fp16 round to nearest even, fp8 per row:
 * scale = max|h| / 448 (1 if zero), code = nearest e4m3fn of h / scale;
 * nvfp4 as described at ssu_cache, g from the slot's largest |value|),
 * write recur_state when present (fp16 with the stochastic rounding above,
 * keyed by sr_seed; sr_seed is unused otherwise), zero its x/B/dt rings and
 * set ring_start to 0.  Other ids are ignored.  slot ids must be unique.
 * n == 0 is a no-op; n < 0 is SSU_ERR_INVALID, n * nheads > SSU_MAX_PAIRS
 * SSU_ERR_UNSUPPORTED.  states 16-byte aligned and states_batch_stride >= 0
 * a multiple of 4; slot_idx 4-byte aligned.
 */
int ssu_init_state(const ssu_cache *cache, const float *states, int64_t states_batch_stride,
                   const int32_t *slot_idx, int32_t n, uint64_t sr_seed, hipStream_t stream);

/*
 * One replay step [FI items 1-2; VD selective_state_update_replayssm].
 * Per entry b and head h, with S = pnat + T_b combined tokens (live ring
 * tokens then new tokens), dt'_s from the ring for s < pnat and
 * softplus(dt + dt_bias[h]) for new ones, cumA_s = sum_{u<=s} A[h] dt'_u:
 *   y_t = exp(cumA_t) C_t.h0 + sum_{s<=t} exp(cumA_t - cumA_s) dt'_s (C_t.B_s) x_s + D[h] x_t
 * for every new token t, written to out.  The new tokens' x, B and dt' are
 * appended to the ring.  The checkpoint and ring_start are not modified, so
 * repeating a step with the same inputs gives the same result.
 * Requires pnat + T_b <= ring_len per entry (else SSU_STATUS_BAD_PNAT).
 *
 * Fused flush-in-step [FI, the checkpoint write path inside the replay
 * kernel; Reviewer Notes]: with step->num_fold non-NULL, an entry with
 * k = num_fold[b] in [1, pnat] first folds its first k live ring tokens into
 * the checkpoint exactly as ssu_flush does (fp32 fold, re-encode, new fp8
 * row scales), then reads out from the new checkpoint with the remaining
 * pnat - k live tokens; after the call ring_start[slot] has advanced by k.
 * The result equals ssu_flush(k) followed by this step with pnat - k, but the
 * checkpoint is read once instead of twice.  k == 0 is a plain step; k < 0 or
 * k > pnat skips the entry like padding (zero output rows, cache untouched)
 * and sets SSU_STATUS_BAD_FOLD.  A fused step is not repeatable (it changes
 * the checkpoint and ring_start).
 */
int ssu_replay_step(const ssu_cache *cache, const ssu_step *step, hipStream_t stream);

/*
 * ssu_replay_step for callers that cannot allocate (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same
 * step, bit for bit, except that the SPLIT algorithm's scratch (the fp32 C.B
 * table of every (entry, group), ssu_workspace_size bytes) is a device array
 * the library holds, SSU_NOALLOC_SCRATCH_BYTES bytes on every GPU it runs on
 * until the process ends, instead of step->workspace, which is ignored.
 *  - A step whose SPLIT scratch would exceed SSU_NOALLOC_SCRATCH_BYTES
 *    (ssu_workspace_size(cache, batch, max_seqlen) > it: at 128 bytes per
 *    (entry, group, token), e.g. batch 2048 with 8 groups and 8 tokens fits,
 *    batch 2049 does not) returns SSU_ERR_WORKSPACE before any launch.
 *  - Allocates and frees nothing.  Its first call on a device looks up the
 *    array's device address there (hipGetSymbolAddress; SSU_ERR_HIP if that
 *    fails); devices 0..63.
 *  - Every call on one GPU shares that GPU's array and it keeps the last
 *    call's contents (a call reads only what it wrote itself): calls that may
 *    overlap on one GPU (streams not ordered with each other) race, and the
 *    caller must order them.
 * A step that AUTO resolves to MONOLITH uses no scratch and runs exactly as
 * ssu_replay_step.
 */
#define SSU_NOALLOC_SCRATCH_BYTES ((size_t)16 << 20)
int ssu_replay_step_noalloc(const ssu_cache *cache, const ssu_step *step, hipStream_t stream);

/*
 * Flush [FI item 2 (host owns the ring); VP (FP32 flush, nearest-encoded FP8
 * with FP32 row scales)].  For each j with slot = slot_idx[j] valid and
 * k = num_fold[j] in [1, ring_len]: fold the first k live ring tokens into
 * the checkpoint in fp32,
 *   h <- exp(cumA_{k-1}) h + sum_{s<k} exp(cumA_{k-1} - cumA_s) dt'_s x_s B_s^T,
 * re-encode it in state_dtype, then advance ring_start[slot] by k (mod L).
 * k == 0 changes nothing.  A: [nheads] f32, the same A the steps use.
 * The caller's next pnat for the slot is pnat + accepted - k.  n == 0 is a
 * no-op, n < 0 SSU_ERR_INVALID, n * nheads > SSU_MAX_PAIRS
 * SSU_ERR_UNSUPPORTED; slot_idx, num_fold and A are 4-byte aligned.
 */
int ssu_flush(const ssu_cache *cache, const int32_t *slot_idx, const int32_t *num_fold,
              const float *A, int32_t n, uint64_t sr_seed, hipStream_t stream);

/* The algorithm this step runs (MONOLITH or SPLIT): step->algo when it names
 * one, else what SSU_ALGO_AUTO resolves to; or the negative error code that
 * ssu_replay_step would return for these descriptors (the workspace aside).
 * Launches nothing. */
int ssu_resolve_algo(const ssu_cache *cache, const ssu_step *step);

/* Work-unit threshold (batch * nheads) at or above which AUTO picks SPLIT.
 * Process-wide; set_ returns the previous value.  The default is INT64_MAX
 * (AUTO = monolith): on MI355X the split never overtook the monolith between
 * 128 and 65536 work units. */
int64_t ssu_get_split_threshold(void);
int64_t ssu_set_split_threshold(int64_t work_units);

/* The message of the calling thread's last call that failed; "" after a
 * call that succeeded (ssu_get/set_split_threshold leave it as it was). */
const char *ssu_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* SSU_H */
