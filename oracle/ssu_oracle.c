/*
 * ssu_oracle.c -- CPU reference ("oracle") for the checkpointing selective
 * state update (ReplaySSM / MTP-replay SSU).  TEST INFRASTRUCTURE ONLY.
 *
 * This file is the plain, slow, obviously-correct definition that the GPU
 * library is checked against.  Only the tests, the smoke check and the CPU
 * baseline leg of the benchmark may load it; the product never does.  It
 * shares no code, header, table or constant with the HIP path.
 *
 * Everything is computed in fp64 with the textbook sequential recurrence,
 * replayed from the checkpoint one token at a time:
 *
 *     dt'  = softplus(dt + dt_bias[h])
 *     h   <- exp(A[h] * dt') * h  +  dt' * x (outer) B
 *     y    = h . C  +  D[h] * x                 (times z sigmoid(z) when gated)
 *
 * Sources (cited by page title and section):
 *  - FlashInfer PR "mamba checkpointing SSU: two-kernel split + ring-buffer
 *    cache", Description item 2 (ring-buffer cache contract table): the
 *    head-major rings x_cache (slot, nheads, L, dim), B_cache (slot, ngroups,
 *    L, dstate), dt_cache (slot, nheads, L) f32, ring_start (slot,) i32; live
 *    token j sits at (ring_start + j) mod L for j < pnat, append i goes to
 *    (ring_start + pnat + i) mod L; the host advances ring_start on flush;
 *    the decay prefix is recomputed, never cached.
 *  - vLLM API page "replayssm_cutedsl", selective_state_update_replayssm:
 *    softplus is applied to dt plus dt_bias; dt, A, dt_bias are one value per
 *    head, D is per head; B and C are per group; x/B/C are BF16; slot zero is
 *    reserved for padding; nonpositive / out-of-range slots are ignored
 *    (initialize_replayssm_state docstring).
 *  - vLLM PR "Add separate CuTeDSL ReplaySSM checkpoints", Overview and
 *    Claims: the flush works in FP32 and the FP8 read checkpoint is written
 *    with nearest encoding and an FP32 scale per row; only the accepted
 *    prefix may change the checkpoint.
 *
 * Readings where the pages are silent (each one is also listed in the design
 * notes of the repository):
 *  - dt_cache holds dt' (after softplus), as fp32.
 *  - softplus(v) = v for v > 20, else log1p(exp(v)).
 *  - A flush folds the first k live ring tokens into the checkpoint and
 *    advances ring_start by k (mod L); k = 0 changes nothing.
 *  - The flush result is an FP32 state; it is then encoded.  fp32: stored;
 *    bf16 / fp16: round to nearest, ties to even (fp16 overflow -> inf);
 *    fp8 e4m3fn (OCP, max 448), per row of dstate: m = max |h|, scale =
 *    fp32(m / 448) (1 when that is 0), code = nearest e4m3fn value of
 *    fp32(h / scale) after clamping to [-448, 448], ties to even code.
 *  - The optional output gate is Mamba-2's: y * z * sigmoid(z) with z bf16
 *    [tok][H][P], applied to the fp64 readout; dt_softplus = 0 makes dt' the
 *    plain dt + dt_bias (FlashInfer PR, the HAS_Z output and dt_softplus
 *    flags named in its commits).
 *  - Separate checkpoints (vLLM PR "Add separate CuTeDSL ReplaySSM
 *    checkpoints", Overview and Claims: an FP16 recurrence checkpoint with
 *    "SR7" and an FP8 read checkpoint with nearest encoding): with a
 *    recurrence checkpoint, the flush folds from it, writes it back with
 *    stochastic rounding to fp16 and writes the read checkpoint with the
 *    nearest encoding of the same fp32 result; steps read only the read
 *    checkpoint; init writes both from the FP32 prefill states.  "SR7" is
 *    read as stochastic rounding with 7 random bits per value (or_sr_f16),
 *    the bits coming from Philox4x32-10 keyed by a per-call 64-bit seed.
 *  - NVFP4 read checkpoint (same PR, Claims: FP8/NVFP4 read checkpoints with
 *    nearest encoding; vLLM API page, initialize_replayssm_state, NVFP4
 *    branch: the largest |value| of each group of heads, then their maximum
 *    over the groups divided by 6 * 448, one second-level scale per slot,
 *    1 where that is not positive): e2m1 elements, an e4m3 scale per block of
 *    16 along dstate, one fp32 second-level scale g per slot.  The page shows
 *    the encode only at init; a fold is read here as re-encoding the whole
 *    slot the same way from its folded fp32 state (encode_slot_nvfp4), so the
 *    read checkpoint is always the init encoding of the current state.
 *  - A padding entry (slot <= 0 or slot >= num_slots) writes zero output rows
 *    and touches no cache.  An entry with pnat < 0 or pnat + T_b > L is
 *    treated the same way and raises status bit 1; a flush entry with k < 0
 *    or k > L is skipped and raises status bit 2; a varlen entry whose token
 *    count is negative or above max_seqlen is skipped (no output written) and
 *    raises status bit 4; a slot whose ring_start lies outside [0, L) is
 *    skipped by the step (zero output rows) and by the flush, and raises
 *    status bit 8.
 *
 * Layouts (all byte strides between slots are arguments; inside a slot the
 * layout is packed):
 *   state     [slot][H][P][N]  element type = state dtype, each head either
 *                              row-major or in the tiled order (elem_offset)
 *   scale     [slot][H][P]     f32 (fp8 state only)
 *   x_cache   [slot][H][L][P]  bf16 bits
 *   B_cache   [slot][G][L][N]  bf16 bits
 *   dt_cache  [slot][H][L]     f32
 *   ring_start[slot]           i32
 *   x   [tok][H][P] bf16 bits,  B, C [tok][G][N] bf16 bits,  dt [tok][H] f32
 *   out [tok][H][P] f64
 * Token rows of entry b are tok = bos + i, with bos = cu_seqlens[b] when
 * cu_seqlens is given (varlen) and bos = b * T otherwise.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <omp.h>

enum { OR_F32 = 0, OR_BF16 = 1, OR_F16 = 2, OR_FP8 = 3, OR_F64 = 4, OR_NVFP4 = 5 };

/* ---------------------------------------------------------------------- */
/* Number formats, written from their definitions.                         */
/* ---------------------------------------------------------------------- */

double or_bf16_value(uint16_t bits) {
  /* bfloat16 is the upper half of an IEEE binary32. */
  uint32_t u = (uint32_t)bits << 16;
  float f;
  memcpy(&f, &u, 4);
  return (double)f;
}

double or_f16_value(uint16_t bits) {
  /* IEEE binary16: 1 sign, 5 exponent (bias 15), 10 mantissa bits. */
  int s = bits >> 15, e = (bits >> 10) & 31, m = bits & 1023;
  double v;
  if (e == 0)
    v = ldexp((double)m, -24);
  else if (e == 31)
    v = m ? NAN : INFINITY;
  else
    v = ldexp((double)(1024 + m), e - 25);
  return s ? -v : v;
}

double or_e4m3_value(uint8_t code) {
  /* OCP FP8 E4M3FN: 1 sign, 4 exponent (bias 7), 3 mantissa bits, no
   * infinities; exponent 15 with mantissa 7 is NaN, so the largest finite
   * magnitude is 1.75 * 2^8 = 448. */
  int s = code >> 7, e = (code >> 3) & 15, m = code & 7;
  double v;
  if (e == 15 && m == 7)
    v = NAN;
  else if (e == 0)
    v = ldexp((double)m, -9);
  else
    v = ldexp((double)(8 + m), e - 10);
  return s ? -v : v;
}

double or_e2m1_value(uint8_t code) {
  /* OCP MX FP4 E2M1: 1 sign, 2 exponent (bias 1), 1 mantissa bit, no
   * infinities or NaN; exponent 0 is subnormal (0 or 0.5), the largest
   * magnitude is 1.5 * 2^2 = 6. */
  int s = (code >> 3) & 1, e = (code >> 1) & 3, m = code & 1;
  double v = e == 0 ? 0.5 * m : ldexp(1.0 + 0.5 * m, e - 1);
  return s ? -v : v;
}

/* Round to nearest, ties to even, by searching the sorted table of the
 * format's non-negative representable values.  `table[i]` is the value of
 * code i (codes 0..n-1 increase with value).  Returns the code of the
 * nearest entry; on a tie the entry whose code is even wins. */
static int nearest_code(const double *table, int n, double a) {
  int lo = 0, hi = n - 1;
  if (a <= table[0]) return 0;
  if (a >= table[n - 1]) return n - 1;
  while (hi - lo > 1) { /* invariant: table[lo] <= a < table[hi] */
    int mid = (lo + hi) / 2;
    if (table[mid] <= a)
      lo = mid;
    else
      hi = mid;
  }
  double dl = a - table[lo], dh = table[hi] - a;
  if (dl < dh) return lo;
  if (dh < dl) return hi;
  return (lo % 2 == 0) ? lo : hi;
}

static double g_e4m3_tab[127];   /* codes 0x00..0x7E */
static double g_e2m1_tab[8];     /* codes 0..7 */
static double g_f16_tab[0x7C01]; /* codes 0x0000..0x7C00, 0x7C00 = 2^16 */
static double *g_bf16_tab;       /* codes 0x0000..0x7F80, 0x7F80 = 2^128 */
static int g_tabs_ready = 0;

static void build_tables(void) {
  if (g_tabs_ready) return;
  for (int c = 0; c < 127; ++c) g_e4m3_tab[c] = or_e4m3_value((uint8_t)c);
  for (int c = 0; c < 8; ++c) g_e2m1_tab[c] = or_e2m1_value((uint8_t)c);
  /* For IEEE rounding the first code past the largest finite value stands
   * for the next power of two: a value at least halfway to it rounds to
   * infinity, and infinity's code is even, as IEEE ties-to-even requires. */
  for (int c = 0; c < 0x7C00; ++c) g_f16_tab[c] = or_f16_value((uint16_t)c);
  g_f16_tab[0x7C00] = 65536.0;
  double *t = (double *)malloc(sizeof(double) * 0x7F81);
  for (int c = 0; c < 0x7F80; ++c) t[c] = or_bf16_value((uint16_t)c);
  t[0x7F80] = ldexp(1.0, 128);
  g_bf16_tab = t;
  g_tabs_ready = 1;
}

void or_init_tables(void) { build_tables(); }

/* Thread control for timing runs: the parallel loops over (entry, head) use
 * at most this many OpenMP threads. */
void or_set_threads(int n) { omp_set_num_threads(n > 0 ? n : 1); }
int or_max_threads(void) { return omp_get_max_threads(); }

uint16_t or_enc_bf16(double v) {
  build_tables();
  if (isnan(v)) return 0x7FC0;
  uint16_t s = signbit(v) ? 0x8000 : 0;
  return s | (uint16_t)nearest_code(g_bf16_tab, 0x7F81, fabs(v));
}

uint16_t or_enc_f16(double v) {
  build_tables();
  if (isnan(v)) return 0x7E00;
  uint16_t s = signbit(v) ? 0x8000 : 0;
  return s | (uint16_t)nearest_code(g_f16_tab, 0x7C01, fabs(v));
}

/* Saturating e4m3fn encoder: clamp to [-448, 448], then nearest. NaN -> 0x7F. */
uint8_t or_enc_e4m3_sat(double v) {
  build_tables();
  if (isnan(v)) return 0x7F;
  uint8_t s = signbit(v) ? 0x80 : 0;
  double a = fabs(v);
  if (a > 448.0) a = 448.0;
  return s | (uint8_t)nearest_code(g_e4m3_tab, 127, a);
}

/* Saturating e2m1 encoder: nearest, ties to the even code, magnitudes past 6
 * give 6; the sign is kept (a negative value that rounds to zero gives the
 * negative zero code 0x8).  NaN -> 0x7. */
uint8_t or_enc_e2m1_sat(double v) {
  build_tables();
  if (isnan(v)) return 0x7;
  uint8_t s = signbit(v) ? 0x8 : 0;
  return s | (uint8_t)nearest_code(g_e2m1_tab, 8, fabs(v));
}

double or_softplus(double v) { return v > 20.0 ? v : log1p(exp(v)); }

/* ---------------------------------------------------------------------- */
/* Counter-based random bits and stochastic rounding.                      */
/* ---------------------------------------------------------------------- */

/*
 * Philox4x32 (Salmon, Moraes, Dror and Shaw, "Parallel random numbers: as
 * easy as 1, 2, 3", SC 2011), written from its definition: a round maps
 * (c0, c1, c2, c3) with key (k0, k1) to
 *   (hi(M1 c2) ^ c1 ^ k0, lo(M1 c2), hi(M0 c0) ^ c3 ^ k1, lo(M0 c0))
 * with M0 = 0xD2511F53, M1 = 0xCD9E8D57 and 64-bit products split into
 * hi / lo words; between rounds the key is bumped by the Weyl constants
 * (0x9E3779B9, 0xBB67AE85).  The standard generator uses 10 rounds.
 */
void or_philox4x32(const uint32_t ctr[4], const uint32_t key[2], int rounds, uint32_t out[4]) {
  uint32_t c0 = ctr[0], c1 = ctr[1], c2 = ctr[2], c3 = ctr[3], k0 = key[0], k1 = key[1];
  for (int r = 0; r < rounds; ++r) {
    if (r > 0) {
      k0 += 0x9E3779B9u;
      k1 += 0xBB67AE85u;
    }
    const uint64_t p0 = (uint64_t)0xD2511F53u * c0, p1 = (uint64_t)0xCD9E8D57u * c2;
    const uint32_t n0 = (uint32_t)(p1 >> 32) ^ c1 ^ k0, n1 = (uint32_t)p1;
    const uint32_t n2 = (uint32_t)(p0 >> 32) ^ c3 ^ k1, n3 = (uint32_t)p0;
    c0 = n0; c1 = n1; c2 = n2; c3 = n3;
  }
  out[0] = c0; out[1] = c1; out[2] = c2; out[3] = c3;
}

/*
 * The 7 random bits of value e (index p * N + n inside its head) of one
 * (slot, head) for a given seed: Philox4x32-10 with counter
 * (e / 16, head, slot, 0) and key (seed low word, seed high word) gives 16
 * bytes; value e takes byte e % 16 (little-endian within each word) and uses
 * its low 7 bits.
 */
static unsigned sr_bits(uint64_t seed, int slot, int head, int e) {
  const uint32_t ctr[4] = {(uint32_t)(e / 16), (uint32_t)head, (uint32_t)slot, 0u};
  const uint32_t key[2] = {(uint32_t)seed, (uint32_t)(seed >> 32)};
  uint32_t out[4];
  or_philox4x32(ctr, key, 10, out);
  const int j = e % 16;
  return (out[j / 4] >> (8 * (j % 4))) & 0x7Fu;
}

/*
 * Stochastic rounding of an fp32 value to fp16 with 7 random bits u in
 * [0, 128), in the usual few-random-bits form: with lo and hi the two fp16
 * values that bracket |v| (lo <= |v| < hi; past the largest finite value hi
 * is infinity, standing at 2^16) and f = (|v| - lo) / (hi - lo), keep the
 * top 7 bits of f, floor(128 f), add u, and round away from zero (to hi)
 * when the sum carries, i.e. floor(128 f) + u >= 128, else to lo.  Values
 * that are exactly representable stay; a value rounds away with probability
 * floor(128 f) / 128.  The sign is kept; NaN gives a quiet NaN (0x7E00 with
 * the sign of v).
 */
uint16_t or_sr_f16(float v, unsigned u) {
  build_tables();
  if (isnan(v)) return signbit(v) ? 0xFE00 : 0x7E00;
  const uint16_t s = signbit(v) ? 0x8000 : 0;
  const double a = fabs((double)v);
  if (a >= 65536.0) return s | 0x7C00;
  int lo = 0, hi = 0x7C00; /* g_f16_tab[0x7C00] = 2^16 stands for infinity */
  while (hi - lo > 1) {    /* invariant: tab[lo] <= a < tab[hi] */
    const int mid = (lo + hi) / 2;
    if (g_f16_tab[mid] <= a)
      lo = mid;
    else
      hi = mid;
  }
  if (g_f16_tab[lo] == a) return s | (uint16_t)lo;
  const double frac = (a - g_f16_tab[lo]) / (g_f16_tab[hi] - g_f16_tab[lo]); /* exact */
  return s | (uint16_t)(floor(128.0 * frac) + (double)u >= 128.0 ? hi : lo);
}

/* ---------------------------------------------------------------------- */
/* Cache description.                                                      */
/* ---------------------------------------------------------------------- */

typedef struct {
  int num_slots, nheads, ngroups, headdim, dstate, ring_len;
  int state_dtype;
  int state_layout; /* 0: row-major [P][N]; 1: tiled (P = 64, N = 128) */
  uint8_t *state;
  int64_t state_stride; /* bytes between slots */
  uint8_t *scale;
  int64_t scale_stride;
  uint8_t *x_cache;
  int64_t x_stride;
  uint8_t *B_cache;
  int64_t B_stride;
  uint8_t *dt_cache;
  int64_t dt_stride;
  int32_t *ring_start;
  /* Separate checkpoints: the FP16 recurrence checkpoint (same layout as the
   * state, element type fp16) or NULL when the state is the only checkpoint. */
  uint8_t *recur;
  int64_t recur_stride;
  /* NVFP4 state only, f32 [slot][1 + H]: word 0 the slot's second-level
   * scale g, word 1 + h the largest |value| of head h when it was encoded. */
  uint8_t *gscale;
  int64_t gscale_stride;
} or_cache;

static int state_elem_bytes(int dt) {
  switch (dt) {
  case OR_F32: return 4;
  case OR_BF16: return 2;
  case OR_F16: return 2;
  case OR_FP8: return 1;
  case OR_NVFP4: return 0; /* two elements per byte: see head_bytes */
  default: return 8;
  }
}

/* Bytes of one head's checkpoint. */
static int64_t head_bytes(const or_cache *c) {
  const int64_t PN = (int64_t)c->headdim * c->dstate;
  return c->state_dtype == OR_NVFP4 ? PN / 2 : PN * state_elem_bytes(c->state_dtype);
}

/*
 * NVFP4 checkpoint (a reading of the pages' NVFP4 read checkpoint; the
 * layout is this library's): element (p, n) is an e2m1 code, blocks of 16
 * consecutive n of a row share an e4m3 block scale, and each slot has one
 * fp32 second-level scale g; the value is e2m1 * e4m3(block) * g.
 * Codes, row-major: element p N + n in byte (p N + n) / 2, the even element
 * in the low nibble.  Tiled (P = 64, N = 128): the 32 values of quarter q of
 * row p (lane l = 16 q + m, rb = p / 16, m = p % 16, t = n % 32) fill the
 * 16 bytes at rb * 1024 + l * 16, value t in byte t / 2 (even t low nibble).
 * Block scales (P N / 16 bytes per head), row-major: p (N / 16) + n / 16.
 * Tiled: the two blocks of lane l's quarter in row block rb are bytes
 * l * 8 + rb * 2 + (t / 16), so each lane's eight scales are contiguous.
 */
static int64_t nvfp4_code_byte(const or_cache *c, int p, int n, int *high) {
  if (c->state_layout == 0) {
    const int64_t i = (int64_t)p * c->dstate + n;
    *high = (int)(i & 1);
    return i >> 1;
  }
  const int rb = p / 16, m = p % 16, q = n / 32, t = n % 32, l = 16 * q + m;
  *high = t & 1;
  return (int64_t)rb * 1024 + (int64_t)l * 16 + t / 2;
}

static int64_t nvfp4_scale_byte(const or_cache *c, int p, int n) {
  if (c->state_layout == 0) return (int64_t)p * (c->dstate / 16) + n / 16;
  const int rb = p / 16, m = p % 16, q = n / 32, t = n % 32, l = 16 * q + m;
  return (int64_t)l * 8 + rb * 2 + t / 16;
}

/* Word w of a slot's NVFP4 scale words (0: g; 1 + h: head h's maximum). */
static float nvfp4_word(const or_cache *c, int slot, int w) {
  float g;
  memcpy(&g, c->gscale + (int64_t)slot * c->gscale_stride + (int64_t)w * 4, 4);
  return g;
}

static void nvfp4_set_word(const or_cache *c, int slot, int w, float v) {
  memcpy(c->gscale + (int64_t)slot * c->gscale_stride + (int64_t)w * 4, &v, 4);
}

/* Byte offset of element (p, n) inside one head's checkpoint.
 * Row-major: (p N + n) eb.
 * Tiled (P = 64, N = 128; the layout the library documents): rows come in
 * blocks of 16 (rb = p / 16, m = p % 16) and each row in four quarters of 32
 * values (q = n / 32, t = n % 32).  Quarter q of row p is owned by lane
 * l = 16 q + m; its 32 values are cut into 16-byte chunks of ce = 16 / eb
 * values, and chunk u = t / ce of lane l is stored at byte
 * rb * 2048 eb + (64 u + l) * 16, value t % ce of it at + (t % ce) eb. */
static int64_t elem_offset(const or_cache *c, int eb, int p, int n) {
  if (c->state_layout == 0) return ((int64_t)p * c->dstate + n) * eb;
  const int rb = p / 16, m = p % 16, q = n / 32, t = n % 32, ce = 16 / eb;
  const int l = 16 * q + m, u = t / ce;
  return (int64_t)rb * 2048 * eb + ((int64_t)u * 64 + l) * 16 + (int64_t)(t % ce) * eb;
}

/* Decode the checkpoint of (slot, head) into h[P*N] (fp64). */
static void decode_state(const or_cache *c, int slot, int head, double *h) {
  const int P = c->headdim, N = c->dstate, eb = state_elem_bytes(c->state_dtype);
  const uint8_t *base = c->state + (int64_t)slot * c->state_stride + (int64_t)head * head_bytes(c);
  if (c->state_dtype == OR_NVFP4) {
    const uint8_t *sf = c->scale + (int64_t)slot * c->scale_stride + (int64_t)head * (P * N / 16);
    const double g = nvfp4_word(c, slot, 0);
    for (int p = 0; p < P; ++p)
      for (int n = 0; n < N; ++n) {
        int hi;
        const uint8_t byte = base[nvfp4_code_byte(c, p, n, &hi)];
        h[p * N + n] = or_e2m1_value(hi ? byte >> 4 : byte & 15) * or_e4m3_value(sf[nvfp4_scale_byte(c, p, n)]) * g;
      }
    return;
  }
  for (int p = 0; p < P; ++p) {
    double sc = 1.0;
    if (c->state_dtype == OR_FP8) {
      float f;
      memcpy(&f, c->scale + (int64_t)slot * c->scale_stride +
                     ((int64_t)head * P + p) * 4, 4);
      sc = (double)f;
    }
    for (int n = 0; n < N; ++n) {
      const uint8_t *e = base + elem_offset(c, eb, p, n);
      double v;
      switch (c->state_dtype) {
      case OR_F32: { float f; memcpy(&f, e, 4); v = f; } break;
      case OR_BF16: { uint16_t u; memcpy(&u, e, 2); v = or_bf16_value(u); } break;
      case OR_F16: { uint16_t u; memcpy(&u, e, 2); v = or_f16_value(u); } break;
      case OR_FP8: v = or_e4m3_value(*e) * sc; break;
      default: memcpy(&v, e, 8); break;
      }
      h[p * N + n] = v;
    }
  }
}

/* Decode the FP16 recurrence checkpoint of (slot, head) into h[P*N]. */
static void decode_recur(const or_cache *c, int slot, int head, double *h) {
  const int P = c->headdim, N = c->dstate;
  const uint8_t *base = c->recur + (int64_t)slot * c->recur_stride + (int64_t)head * P * N * 2;
  for (int p = 0; p < P; ++p)
    for (int n = 0; n < N; ++n) {
      uint16_t u;
      memcpy(&u, base + elem_offset(c, 2, p, n), 2);
      h[p * N + n] = or_f16_value(u);
    }
}

/* Write one row of an fp32 state into the recurrence checkpoint with
 * stochastic rounding (random bits from the seed, slot, head and index). */
static void encode_recur_row(const or_cache *c, int slot, int head, int p, const float *row,
                             uint64_t seed) {
  const int P = c->headdim, N = c->dstate;
  uint8_t *base = c->recur + (int64_t)slot * c->recur_stride + (int64_t)head * P * N * 2;
  for (int n = 0; n < N; ++n) {
    const uint16_t u = or_sr_f16(row[n], sr_bits(seed, slot, head, p * N + n));
    memcpy(base + elem_offset(c, 2, p, n), &u, 2);
  }
}

/* Encode one row of an fp32 state (the flush result) into the checkpoint. */
static void encode_row(const or_cache *c, int slot, int head, int p,
                       const float *row) {
  const int P = c->headdim, N = c->dstate, eb = state_elem_bytes(c->state_dtype);
  uint8_t *base = c->state + (int64_t)slot * c->state_stride + (int64_t)head * P * N * eb;
  if (c->state_dtype == OR_FP8) {
    float m = 0.0f;
    for (int n = 0; n < N; ++n)
      if (fabsf(row[n]) > m) m = fabsf(row[n]);
    float scale = m / 448.0f; /* IEEE single division, correctly rounded */
    if (!(scale > 0.0f)) scale = 1.0f;
    memcpy(c->scale + (int64_t)slot * c->scale_stride + ((int64_t)head * P + p) * 4,
           &scale, 4);
    for (int n = 0; n < N; ++n) {
      float q = row[n] / scale;
      base[elem_offset(c, eb, p, n)] = or_enc_e4m3_sat((double)q);
    }
    return;
  }
  for (int n = 0; n < N; ++n) {
    uint8_t *e = base + elem_offset(c, eb, p, n);
    switch (c->state_dtype) {
    case OR_F32: memcpy(e, &row[n], 4); break;
    case OR_BF16: { uint16_t u = or_enc_bf16((double)row[n]); memcpy(e, &u, 2); } break;
    case OR_F16: { uint16_t u = or_enc_f16((double)row[n]); memcpy(e, &u, 2); } break;
    default: break;
    }
  }
}

/*
 * Encode one head of an fp32 state into the NVFP4 checkpoint with the slot's
 * second-level scale g, nearest encoding: per block of 16 with a = max |v|,
 * block scale = e4m3_sat(fp32(a / fp32(6 g))), element scale
 * es = fp32(e4m3 value * g), code = e2m1_sat(fp32(v / es)) (a zero block
 * scale stores signed zeros).  IEEE single precision throughout.
 */
static void encode_head_nvfp4(const or_cache *c, int slot, int head, const float *hv, float g) {
  const int P = c->headdim, N = c->dstate;
  uint8_t *base = c->state + (int64_t)slot * c->state_stride + (int64_t)head * head_bytes(c);
  uint8_t *sf = c->scale + (int64_t)slot * c->scale_stride + (int64_t)head * (P * N / 16);
  const float ds = 6.0f * g;
  for (int p = 0; p < P; ++p)
    for (int n0 = 0; n0 < N; n0 += 16) {
      float a = 0.0f;
      for (int i = 0; i < 16; ++i)
        if (fabsf(hv[p * N + n0 + i]) > a) a = fabsf(hv[p * N + n0 + i]);
      const float t = a / ds;
      const uint8_t code = or_enc_e4m3_sat((double)t);
      sf[nvfp4_scale_byte(c, p, n0)] = code;
      const float es = (float)or_e4m3_value(code) * g;
      for (int i = 0; i < 16; ++i) {
        const float v = hv[p * N + n0 + i];
        const float q = es > 0.0f ? v / es : 0.0f * v;
        int hi;
        uint8_t *byte = base + nvfp4_code_byte(c, p, n0 + i, &hi);
        const uint8_t e = or_enc_e2m1_sat((double)q);
        *byte = hi ? (uint8_t)((*byte & 0x0F) | (e << 4)) : (uint8_t)((*byte & 0xF0) | e);
      }
    }
}

/*
 * Encode a whole slot of fp32 values hv[H][P][N] into the NVFP4 checkpoint,
 * as initialize_replayssm_state's NVFP4 branch does (vLLM API page): the
 * second-level scale is the largest |value| over every head of the slot
 * divided by 6 * 448 = 2688 (the largest e2m1 value times the largest e4m3
 * value), in IEEE single precision, and 1 where that is not positive.  Word
 * 1 + h of the slot's scale words records head h's largest |value|.
 */
static void encode_slot_nvfp4(const or_cache *c, int slot, const float *hv) {
  const int H = c->nheads, PN = c->headdim * c->dstate;
  float m = 0.0f;
  for (int h = 0; h < H; ++h) {
    float mh = 0.0f;
    for (int i = 0; i < PN; ++i)
      if (fabsf(hv[(int64_t)h * PN + i]) > mh) mh = fabsf(hv[(int64_t)h * PN + i]);
    nvfp4_set_word(c, slot, 1 + h, mh);
    if (mh > m) m = mh;
  }
  float g = m / 2688.0f;
  if (!(g > 0.0f)) g = 1.0f;
  nvfp4_set_word(c, slot, 0, g);
  for (int h = 0; h < H; ++h) encode_head_nvfp4(c, slot, h, hv + (int64_t)h * PN, g);
}

/* fp64 state mode (test only, row-major): store without rounding. */
static void store_state_f64(const or_cache *c, int slot, int head, const double *h) {
  const int PN = c->headdim * c->dstate;
  uint8_t *base = c->state + (int64_t)slot * c->state_stride + (int64_t)head * PN * 8;
  memcpy(base, h, sizeof(double) * PN);
}

static uint16_t rd_u16(const uint8_t *p) { uint16_t u; memcpy(&u, p, 2); return u; }
static float rd_f32(const uint8_t *p) { float f; memcpy(&f, p, 4); return f; }

/* One recurrence step on h[P*N]:  h <- exp(a*d) h + d x B^T.  */
static void ssu_token(double *h, int P, int N, double a, double d,
                      const double *xv, const double *Bv) {
  const double decay = exp(a * d);
  for (int p = 0; p < P; ++p)
    for (int n = 0; n < N; ++n)
      h[p * N + n] = decay * h[p * N + n] + d * xv[p] * Bv[n];
}

/* ---------------------------------------------------------------------- */
/* Replay step.                                                            */
/* ---------------------------------------------------------------------- */

/*
 * For each batch entry: replay the checkpoint through the pnat live ring
 * tokens and then the T_b new tokens, reading out y after every new token;
 * append the new tokens' x, B and dt' to the ring.  The checkpoint and
 * ring_start are not modified.  Returns the status bits.
 */
/*
 * dt' of a new token.  With dt_softplus (the default of the pages) it is
 * softplus(dt + dt_bias); without it (the dt_softplus = false variant named
 * in the FlashInfer PR's commits) it is dt + dt_bias itself.
 */
static double new_dt(float dt, float bias, int dt_softplus) {
  const double v = (double)dt + (double)bias;
  return dt_softplus ? or_softplus(v) : v;
}

/* The output gate z * sigmoid(z) (Mamba-2's SiLU gate on the readout). */
static double silu(double z) { return z / (1.0 + exp(-z)); }

int or_replay_step(const or_cache *c, int batch, int T, const int32_t *cu_seqlens,
                   const int32_t *slot_idx, const int32_t *pnat,
                   const uint16_t *x, const uint16_t *Bm, const uint16_t *Cm,
                   const float *dt, const float *A, const float *D,
                   const float *dt_bias, const uint16_t *z, int dt_softplus, double *out) {
  const int H = c->nheads, G = c->ngroups, P = c->headdim, N = c->dstate,
            L = c->ring_len, HPG = H / G;
  int status = 0;
  build_tables(); /* before any parallel region */
  /* Pass 1: validity of each entry (serial; cheap). */
  int *ok = (int *)calloc(batch > 0 ? batch : 1, sizeof(int));
  for (int b = 0; b < batch; ++b) {
    int bos = cu_seqlens ? cu_seqlens[b] : b * T;
    int Tb = cu_seqlens ? cu_seqlens[b + 1] - cu_seqlens[b] : T;
    int slot = slot_idx[b];
    if (Tb < 0 || Tb > T) { status |= 4; ok[b] = 0; continue; }
    if (slot <= 0 || slot >= c->num_slots) { ok[b] = 1; /* padding */ }
    else if (pnat[b] < 0 || pnat[b] + Tb > L) { status |= 1; ok[b] = 1; }
    else if (c->ring_start[slot] < 0 || c->ring_start[slot] >= L) { status |= 8; ok[b] = 1; }
    else ok[b] = 2;
    if (ok[b] == 1)
      for (int i = 0; i < Tb; ++i)
        for (int hh = 0; hh < H; ++hh)
          for (int p = 0; p < P; ++p)
            out[((int64_t)(bos + i) * H + hh) * P + p] = 0.0;
  }
  /* Pass 2: the recurrence, one (entry, head) at a time. */
#pragma omp parallel for collapse(2) schedule(dynamic)
  for (int b = 0; b < batch; ++b) {
    for (int hh = 0; hh < H; ++hh) {
      if (ok[b] != 2) continue;
      const int bos = cu_seqlens ? cu_seqlens[b] : b * T;
      const int Tb = cu_seqlens ? cu_seqlens[b + 1] - cu_seqlens[b] : T;
      const int slot = slot_idx[b], p0 = pnat[b], r = c->ring_start[slot];
      const int g = hh / HPG;
      double *h = (double *)malloc(sizeof(double) * P * N);
      double *xv = (double *)malloc(sizeof(double) * P);
      double *Bv = (double *)malloc(sizeof(double) * N);
      decode_state(c, slot, hh, h);
      const uint8_t *xs = c->x_cache + (int64_t)slot * c->x_stride;
      const uint8_t *Bs = c->B_cache + (int64_t)slot * c->B_stride;
      const uint8_t *ds = c->dt_cache + (int64_t)slot * c->dt_stride;
      /* live ring tokens: stored dt' is used as is */
      for (int s = 0; s < p0; ++s) {
        int pos = (r + s) % L;
        double d = rd_f32(ds + ((int64_t)hh * L + pos) * 4);
        for (int p = 0; p < P; ++p)
          xv[p] = or_bf16_value(rd_u16(xs + (((int64_t)hh * L + pos) * P + p) * 2));
        for (int n = 0; n < N; ++n)
          Bv[n] = or_bf16_value(rd_u16(Bs + (((int64_t)g * L + pos) * N + n) * 2));
        ssu_token(h, P, N, A[hh], d, xv, Bv);
      }
      /* new tokens: softplus, update, read out */
      for (int i = 0; i < Tb; ++i) {
        int64_t tok = bos + i;
        double d = new_dt(dt[tok * H + hh], dt_bias[hh], dt_softplus);
        for (int p = 0; p < P; ++p) xv[p] = or_bf16_value(x[(tok * H + hh) * P + p]);
        for (int n = 0; n < N; ++n) Bv[n] = or_bf16_value(Bm[(tok * G + g) * N + n]);
        ssu_token(h, P, N, A[hh], d, xv, Bv);
        for (int p = 0; p < P; ++p) {
          double y = 0.0;
          for (int n = 0; n < N; ++n)
            y += h[p * N + n] * or_bf16_value(Cm[(tok * G + g) * N + n]);
          y += (double)D[hh] * xv[p];
          if (z) y *= silu(or_bf16_value(z[(tok * H + hh) * P + p]));
          out[(tok * H + hh) * P + p] = y;
        }
      }
      free(h); free(xv); free(Bv);
    }
  }
  /* Pass 3: ring appends (after every read of this call). */
  for (int b = 0; b < batch; ++b) {
    if (ok[b] != 2) continue;
    const int bos = cu_seqlens ? cu_seqlens[b] : b * T;
    const int Tb = cu_seqlens ? cu_seqlens[b + 1] - cu_seqlens[b] : T;
    const int slot = slot_idx[b], p0 = pnat[b], r = c->ring_start[slot];
    uint8_t *xs = c->x_cache + (int64_t)slot * c->x_stride;
    uint8_t *Bs = c->B_cache + (int64_t)slot * c->B_stride;
    uint8_t *ds = c->dt_cache + (int64_t)slot * c->dt_stride;
    for (int i = 0; i < Tb; ++i) {
      int64_t tok = bos + i;
      int pos = (r + p0 + i) % L;
      for (int hh = 0; hh < H; ++hh) {
        float d = (float)new_dt(dt[tok * H + hh], dt_bias[hh], dt_softplus);
        memcpy(ds + ((int64_t)hh * L + pos) * 4, &d, 4);
        memcpy(xs + ((int64_t)hh * L + pos) * P * 2, x + (tok * H + hh) * P, (size_t)P * 2);
      }
      for (int g = 0; g < G; ++g)
        memcpy(Bs + ((int64_t)g * L + pos) * N * 2, Bm + (tok * G + g) * N, (size_t)N * 2);
    }
  }
  free(ok);
  return status;
}

/* ---------------------------------------------------------------------- */
/* Flush.                                                                  */
/* ---------------------------------------------------------------------- */

/*
 * The fold of the first k live ring tokens of (slot, head) into h[P*N] in
 * fp64, starting from the checkpoint's value (the FP16 recurrence checkpoint
 * when there is one): the same recurrence as the step, over ring tokens
 * (ring_start + s) mod L, s < k, with their stored dt'.
 */
static void fold_head(const or_cache *c, int slot, int hh, int k, float a, double *h) {
  const int G = c->ngroups, P = c->headdim, N = c->dstate, L = c->ring_len, g = hh / (c->nheads / G);
  const int r = c->ring_start[slot];
  double *xv = (double *)malloc(sizeof(double) * P);
  double *Bv = (double *)malloc(sizeof(double) * N);
  if (c->recur)
    decode_recur(c, slot, hh, h);
  else
    decode_state(c, slot, hh, h);
  const uint8_t *xs = c->x_cache + (int64_t)slot * c->x_stride;
  const uint8_t *Bs = c->B_cache + (int64_t)slot * c->B_stride;
  const uint8_t *ds = c->dt_cache + (int64_t)slot * c->dt_stride;
  for (int s = 0; s < k; ++s) {
    int pos = (r + s) % L;
    double d = rd_f32(ds + ((int64_t)hh * L + pos) * 4);
    for (int p = 0; p < P; ++p)
      xv[p] = or_bf16_value(rd_u16(xs + (((int64_t)hh * L + pos) * P + p) * 2));
    for (int q = 0; q < N; ++q)
      Bv[q] = or_bf16_value(rd_u16(Bs + (((int64_t)g * L + pos) * N + q) * 2));
    ssu_token(h, P, N, a, d, xv, Bv);
  }
  free(xv); free(Bv);
}

/*
 * For each entry j with k = num_fold[j] > 0: fold the first k live ring
 * tokens into the checkpoint (fp64 recurrence, result rounded to fp32 as the
 * flush's FP32 state), re-encode it, and advance ring_start by k (mod L).
 * An NVFP4 checkpoint is re-encoded slot by slot (encode_slot_nvfp4).
 */
int or_flush(const or_cache *c, int n, const int32_t *slot_idx,
             const int32_t *num_fold, const float *A, uint64_t seed) {
  const int H = c->nheads, P = c->headdim, N = c->dstate, L = c->ring_len;
  int status = 0;
  build_tables(); /* before any parallel region */
  /* which entries fold: a valid slot, k in [1, L] and a valid ring_start */
  int *go = (int *)calloc(n > 0 ? n : 1, sizeof(int));
  for (int j = 0; j < n; ++j) {
    int slot = slot_idx[j], k = num_fold[j];
    if (slot <= 0 || slot >= c->num_slots) continue;
    if (k < 0 || k > L) { status |= 2; continue; }
    if (k == 0) continue;
    if (c->ring_start[slot] < 0 || c->ring_start[slot] >= L) { status |= 8; continue; }
    go[j] = 1;
  }
  if (c->state_dtype == OR_NVFP4) {
    /* the slot's scale needs every head's folded values: fold all heads of an
     * entry, then encode the slot */
    float *hvs = (float *)malloc(sizeof(float) * (size_t)H * P * N);
    for (int j = 0; j < n; ++j) {
      if (!go[j]) continue;
#pragma omp parallel for schedule(dynamic)
      for (int hh = 0; hh < H; ++hh) {
        double *h = (double *)malloc(sizeof(double) * P * N);
        fold_head(c, slot_idx[j], hh, num_fold[j], A[hh], h);
        for (int e = 0; e < P * N; ++e) hvs[(int64_t)hh * P * N + e] = (float)h[e];
        free(h);
      }
      encode_slot_nvfp4(c, slot_idx[j], hvs);
      if (c->recur)
        for (int hh = 0; hh < H; ++hh)
          for (int p = 0; p < P; ++p)
            encode_recur_row(c, slot_idx[j], hh, p, hvs + ((int64_t)hh * P + p) * N, seed);
    }
    free(hvs);
  } else {
#pragma omp parallel for collapse(2) schedule(dynamic)
    for (int j = 0; j < n; ++j) {
      for (int hh = 0; hh < H; ++hh) {
        if (!go[j]) continue;
        const int slot = slot_idx[j];
        double *h = (double *)malloc(sizeof(double) * P * N);
        float *row = (float *)malloc(sizeof(float) * N);
        fold_head(c, slot, hh, num_fold[j], A[hh], h);
        if (c->state_dtype == OR_F64) {
          store_state_f64(c, slot, hh, h);
        } else {
          for (int p = 0; p < P; ++p) {
            for (int q = 0; q < N; ++q) row[q] = (float)h[p * N + q];
            encode_row(c, slot, hh, p, row);
            if (c->recur) encode_recur_row(c, slot, hh, p, row, seed);
          }
        }
        free(h); free(row);
      }
    }
  }
  for (int j = 0; j < n; ++j)
    if (go[j]) c->ring_start[slot_idx[j]] = (c->ring_start[slot_idx[j]] + num_fold[j]) % L;
  free(go);
  return status;
}

/* ---------------------------------------------------------------------- */
/* Initialisation from FP32 prefill states.                                */
/* ---------------------------------------------------------------------- */

/*
 * states: [n][H][P][N] f32 with `states_stride` elements between entries
 * (0 broadcasts entry 0).  For each valid slot: encode the state, zero the
 * slot's x/B/dt rings and set ring_start to 0.  Invalid slots are ignored.
 */
void or_init_state(const or_cache *c, const float *states, int64_t states_stride,
                   const int32_t *slot_idx, int n, uint64_t seed) {
  const int H = c->nheads, G = c->ngroups, P = c->headdim, N = c->dstate,
            L = c->ring_len;
  build_tables();
  for (int j = 0; j < n; ++j) {
    int slot = slot_idx[j];
    if (slot <= 0 || slot >= c->num_slots) continue;
    const float *src = states + (int64_t)j * states_stride;
    for (int hh = 0; hh < H; ++hh) {
      if (c->state_dtype == OR_F64) {
        double *h = (double *)malloc(sizeof(double) * P * N);
        for (int e = 0; e < P * N; ++e) h[e] = src[(int64_t)hh * P * N + e];
        store_state_f64(c, slot, hh, h);
        free(h);
      } else if (c->state_dtype == OR_NVFP4) {
        if (hh == 0) encode_slot_nvfp4(c, slot, src); /* one scale over every head */
        if (c->recur)
          for (int p = 0; p < P; ++p) encode_recur_row(c, slot, hh, p, src + ((int64_t)hh * P + p) * N, seed);
      } else {
        for (int p = 0; p < P; ++p) {
          encode_row(c, slot, hh, p, src + ((int64_t)hh * P + p) * N);
          if (c->recur) encode_recur_row(c, slot, hh, p, src + ((int64_t)hh * P + p) * N, seed);
        }
      }
    }
    memset(c->x_cache + (int64_t)slot * c->x_stride, 0, (size_t)H * L * P * 2);
    memset(c->B_cache + (int64_t)slot * c->B_stride, 0, (size_t)G * L * N * 2);
    memset(c->dt_cache + (int64_t)slot * c->dt_stride, 0, (size_t)H * L * 4);
    c->ring_start[slot] = 0;
  }
}

/* ---------------------------------------------------------------------- */
/* Array forms of the format helpers (used by the tests' pins).            */
/* ---------------------------------------------------------------------- */

void or_enc_bf16_array(const double *v, uint16_t *out, int64_t n) {
  for (int64_t i = 0; i < n; ++i) out[i] = or_enc_bf16(v[i]);
}
void or_enc_f16_array(const double *v, uint16_t *out, int64_t n) {
  for (int64_t i = 0; i < n; ++i) out[i] = or_enc_f16(v[i]);
}
void or_enc_e4m3_array(const double *v, uint8_t *out, int64_t n) {
  for (int64_t i = 0; i < n; ++i) out[i] = or_enc_e4m3_sat(v[i]);
}
void or_bf16_value_array(const uint16_t *b, double *out, int64_t n) {
  for (int64_t i = 0; i < n; ++i) out[i] = or_bf16_value(b[i]);
}
void or_f16_value_array(const uint16_t *b, double *out, int64_t n) {
  for (int64_t i = 0; i < n; ++i) out[i] = or_f16_value(b[i]);
}
void or_e2m1_value_array(const uint8_t *b, double *out, int64_t n) {
  for (int64_t i = 0; i < n; ++i) out[i] = or_e2m1_value(b[i]);
}
void or_enc_e2m1_array(const double *v, uint8_t *out, int64_t n) {
  for (int64_t i = 0; i < n; ++i) out[i] = or_enc_e2m1_sat(v[i]);
}
/* Decode one (slot, head) checkpoint into out[P*N] (any state dtype). */
void or_decode_head(const or_cache *c, int slot, int head, double *out) { decode_state(c, slot, head, out); }
/* Encode a slot of fp32 values [H][P][N] into an NVFP4 checkpoint. */
void or_encode_slot_nvfp4(const or_cache *c, int slot, const float *hv) {
  build_tables();
  encode_slot_nvfp4(c, slot, hv);
}
void or_e4m3_value_array(const uint8_t *b, double *out, int64_t n) {
  for (int64_t i = 0; i < n; ++i) out[i] = or_e4m3_value(b[i]);
}
void or_sr_f16_array(const float *v, const uint8_t *u, uint16_t *out, int64_t n) {
  for (int64_t i = 0; i < n; ++i) out[i] = or_sr_f16(v[i], u[i]);
}
void or_sr_bits_array(uint64_t seed, int slot, int head, uint8_t *out, int64_t n) {
  for (int64_t i = 0; i < n; ++i) out[i] = (uint8_t)sr_bits(seed, slot, head, (int)i);
}
void or_softplus_array(const double *v, double *out, int64_t n) {
  for (int64_t i = 0; i < n; ++i) out[i] = or_softplus(v[i]);
}
