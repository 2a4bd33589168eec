/*
 * sage_attn.h - C ABI of the MI355X (gfx950) SageAttention2-style quantized
 * exact attention forward: INT8 QK^T with int32 accumulation, online softmax
 * with FP8 (OCP E4M3FN) probabilities, FP8 PV with two-level accumulation and
 * BF16 output.
 *
 * The operation is the numerical contract named in "Experiment Log", Phase 0
 * Import And Verification (stage list: Q/K preparation, K smoothing, INT8
 * quantization, QK traversal, online softmax, FP8 V/P, two-level PV
 * accumulation, final conversion, ragged tails) with the invariants of the
 * Phase 1 State-Ownership Decision (strict KV-tile order, exact FP8 score
 * bytes, per-tile RO rescaling, two-level PV, final conversion).
 *
 * Conventions for every entry point
 *  - All tensor pointers are DEVICE pointers on the current HIP device; the
 *    caller allocates and frees every buffer.  The library never allocates,
 *    never synchronizes and keeps no per-call state: calls are asynchronous on
 *    `stream` (a hipStream_t; NULL = the default stream) and inputs must stay
 *    unchanged until the stream has passed the call.
 *  - Validation is pure host code and runs before any HIP call.  The return
 *    value is SAGE_OK or a negative SAGE_E_* status; nothing is printed and
 *    nothing aborts.  Device faults surface at the caller's next sync.
 *  - Shapes: B, H >= 1; Nq, Nkv >= 1; D in {64, 128}.  Inputs Q [B,H,Nq,D],
 *    K and V [B,H,Nkv,D] and output O [B,H,Nq,D] are bfloat16 with element
 *    strides (b, h, n) given in sage_strides_t; the d dimension is contiguous.
 *    Strides must be multiples of 8 elements and base pointers 16-byte aligned.
 *  - Calls that share buffers on one stream are ordered; calls on different
 *    streams that write the same buffers race.
 */
#ifndef SAGE_ATTN_H
#define SAGE_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* status codes */
#define SAGE_OK 0
#define SAGE_E_NULL (-1)     /* a required pointer is NULL */
#define SAGE_E_SHAPE (-2)    /* B, H, Nq or Nkv out of range */
#define SAGE_E_HEADDIM (-3)  /* D not 64 or 128 */
#define SAGE_E_ALIGN (-4)    /* base pointer or stride misaligned */
#define SAGE_E_ALIAS (-5)    /* the output overlaps itself, an input or a code buffer */
#define SAGE_E_DEVICE (-6)   /* no device, or the device is not gfx950 */
#define SAGE_E_LAUNCH (-7)   /* a kernel launch failed (hipGetLastError) */
#define SAGE_E_ARG (-8)      /* another argument is invalid */
#define SAGE_E_SCRATCH (-9)  /* the allocation-free prep's static scratch is too small for the shape */

/* problem shape */
typedef struct sage_shape {
  int32_t B, H, Nq, Nkv, D;
} sage_shape_t;

/* element strides of dims (b, h, n) for each bf16 tensor; d is contiguous */
typedef struct sage_strides {
  int64_t q[3], k[3], v[3], o[3];
} sage_strides_t;

/*
 * Quantized operands written by sage_quant_prep and read by sage_attn_fwd.
 * Sizes come from sage_buffer_bytes().  Let NQB = ceil(Nq/128),
 * T = ceil(Nkv/64).  Pad rows (queries >= Nq, keys >= Nkv) hold code 0.
 *
 *  q_codes  int8, per (b,h): NQB*128 rows in groups of 32 rows; a group is
 *           stored as [D/32 steps][64 lanes][16 bytes]: lane L, step s holds
 *           row 32g + L%32, channels 32s + 16*(L/32) ... +15.  This is the
 *           operand order of the 32x32x32 INT8 matrix instruction.
 *  q_scale  float [B,H,NQB]: absmax/127 of each 128-row block (0 if all zero).
 *  k_codes  int8, per (b,h): T*64 rows of smoothed K in the same 32-row-group
 *           layout as q_codes (a 64-key tile is two consecutive groups).
 *  k_scale  float [B,H,T]: absmax/127 of each 64-row block of smoothed K.
 *  v_codes  uint8 OCP E4M3FN, per (b,h) and 64-key tile:
 *           [D/32 blocks][2 halves][64 lanes][16 bytes]: block c, half h,
 *           lane L, byte e holds V[key = 32h + 8*(e/4) + 4*(L/32) + e%4]
 *           [channel = 32c + L%32] quantized with the channel scale.
 *  v_scale  float [B,H,D]: per-channel absmax/448 over all Nkv keys.
 *  k_mean   float [B,H,D]: per-channel mean of K over all Nkv keys.
 *  workspace  scratch of the prep (sage_buffer_bytes): column partials of the
 *           K sums and V maxima, V inverses and, for the single pass, per-(b,h)
 *           arrival counters and ready flags and one status word.  Its
 *           contents before a call do not matter (each call initializes what
 *           it reads); two prep calls must not use one workspace at the same
 *           time.
 * sage_quant_prep_kv and sage_attn_fwd_q neither read nor write q_codes and
 * q_scale (they may be NULL there); the forward entries do not use the
 * workspace (it may be NULL there).
 */
typedef struct sage_quant {
  int8_t *q_codes;
  float *q_scale;
  int8_t *k_codes;
  float *k_scale;
  uint8_t *v_codes;
  float *v_scale;
  float *k_mean;
  void *workspace;
} sage_quant_t;

enum sage_buffer {
  SAGE_BUF_Q_CODES = 0,
  SAGE_BUF_Q_SCALE = 1,
  SAGE_BUF_K_CODES = 2,
  SAGE_BUF_K_SCALE = 3,
  SAGE_BUF_V_CODES = 4,
  SAGE_BUF_V_SCALE = 5,
  SAGE_BUF_K_MEAN = 6,
  SAGE_BUF_WORKSPACE = 7,
  SAGE_BUF_COUNT = 8
};

/* Size in bytes of buffer `which` (enum sage_buffer) for `shape`.
 * Returns SAGE_OK, SAGE_E_NULL, SAGE_E_SHAPE, SAGE_E_HEADDIM or SAGE_E_ARG. */
int sage_buffer_bytes(const sage_shape_t *shape, int which, size_t *bytes);

/* Byte offset inside the workspace of the single-pass prep's status word (one
 * uint32).  sage_quant_prep_single_pass sets it to 0 before its work and to a
 * nonzero value if one of its workgroups stopped waiting for the others of its
 * (b,h); the outputs of that call are then invalid.  The three-launch
 * sage_quant_prep does not use it.  Returns SAGE_OK, SAGE_E_NULL,
 * SAGE_E_SHAPE or SAGE_E_HEADDIM. */
int sage_prep_status_offset(const sage_shape_t *shape, size_t *offset);

/*
 * Stages 1-2 of the contract ("Experiment Log", Phase 0 stage list: Q/K
 * preparation, K smoothing, INT8 quantization, FP8 V):
 *   k_mean[c] = fp32(exact sum_t K[t,c] / Nkv)           (FP64 sum, exact)
 *   K smoothed: ks = fp32(K - k_mean)
 *   Q per 128-row block, ks per 64-row block: A = max|x|, scale = fp32(A/127),
 *     code = RNE(fp32(x * fp32(127/A))) in [-127, 127]; A = 0 -> all zero
 *   V per channel: v_scale = fp32(vamax/448), code = E4M3FN_RNE(fp32(v * fp32(448/vamax)))
 * The FP64 column sum is exact, so its order does not matter, whenever
 * sum_t |K[t,c]| < 2^53 * u_c, u_c being the bf16 unit in the last place of the
 * smallest nonzero |K[t,c]| of the column: for instance Nkv * (largest /
 * smallest nonzero magnitude) below 2^45.  Gaussian-like bf16 data meets it up
 * to about a million keys (its smallest magnitude shrinks like 1/Nkv); data on
 * a coarser grid (multiples of 2^-12, say) much further.  Outside that
 * condition the sum rounds: this entry
 * still gives the same bits on every call (fixed order), the single pass
 * below may not (its partial sums meet in atomic order).
 * q, k, v: bf16 device tensors with strides->q/k/v.  Writes every buffer of
 * `quant` (including the workspace).  Launches 3 kernels on `stream`.
 */
int sage_quant_prep(const void *q, const void *k, const void *v, const sage_shape_t *shape,
                    const sage_strides_t *strides, const sage_quant_t *quant, void *stream);

/*
 * The same stages in one pass over K and V (the fused preparation entry of
 * "Experiment Log", Closed Prior Work: P1 entry fusion and P2 direct V
 * preparation, and the matching rows of "Experiment Registry", Complete
 * Registry): every workgroup keeps its K/V rows in registers while the
 * workgroups of a head combine their column statistics, so K and V are read
 * from memory once.  Arguments, layouts, results (bit-identical to
 * sage_quant_prep), ownership and errors as for sage_quant_prep.  Used while a
 * (b,h) needs at most 256 such workgroups (Nkv <= 65536 at D = 128, <= 131072 at
 * D = 64); longer keys take sage_quant_prep's three launches.  Launches 2
 * kernels on `stream`.  Its workgroups wait for each other inside the launch:
 * this relies on a head's workgroups all becoming resident, so do not run it
 * concurrently (other streams) with another single-pass prep or with kernels
 * that hold compute units indefinitely.  The wait is bounded (~0.1 s); one that
 * ran out leaves a nonzero status word in the workspace (at
 * sage_prep_status_offset) and NaN K scales for the tiles of the workgroup
 * that stopped waiting, so a forward on those buffers gives NaN rows instead of
 * silently wrong ones (never observed; the tests and bench.py check the word).
 * About as fast as sage_quant_prep on the shapes measured so far.
 */
int sage_quant_prep_single_pass(const void *q, const void *k, const void *v, const sage_shape_t *shape,
                                const sage_strides_t *strides, const sage_quant_t *quant, void *stream);

/*
 * Allocation-free variant of sage_quant_prep, for callers that cannot allocate
 * device memory (code under stream/graph capture, tight serving loops,
 * harnesses that forbid hipMalloc).  Same kernels, arguments and results as
 * sage_quant_prep, except that the prep's scratch (column partials and V
 * inverses) lives in a static device array of 8 MiB per GPU, created with the
 * library's code object and held until the process ends; quant->workspace is
 * ignored and may be NULL.  The entry allocates nothing.  Shapes whose prep
 * needs more scratch than that (sage_buffer_bytes of SAGE_BUF_WORKSPACE above
 * 8 MiB; the long video workload, 24 heads of 32760 keys at D = 128, needs
 * 4.8 MiB) return SAGE_E_SCRATCH before any HIP call.  Every call on one GPU
 * shares that GPU's array, and each call writes before it reads all it uses:
 * calls ordered on one stream are safe, calls that overlap in time on one GPU
 * (different streams or host threads without ordering) race.
 */
int sage_quant_prep_no_alloc(const void *q, const void *k, const void *v, const sage_shape_t *shape,
                             const sage_strides_t *strides, const sage_quant_t *quant, void *stream);

/*
 * Stages 3-5 ("Experiment Log", Phase 0 stage list and Phase 1 invariants;
 * checkpoint names of Phase 2B Fixed Aligned Numerical Prototype):
 * for each query row, 64-key tiles j = 0..T-1 strictly in order:
 *   S = q_codes . k_codes_j^T                     (INT8 MFMA, int32, exact)
 *   s = S * fp32(fp32(q_scale * k_scale_j) * sm_scale * log2 e); keys >= Nkv masked
 *   m' = max(m, max s); alpha = 2^(m - m'); p = 2^(s - m')
 *   d = d * alpha + sum p                         (from FP32 p)
 *   P8 = E4M3FN(448 p)                            ("exact FP8 score bytes")
 *   partial = P8 . V8_j (FP8 MFMA, FP32); RO = RO * alpha + partial
 * then O = bf16(RO / d * v_scale / 448), rows < Nq stored.
 * sm_scale <= 0 selects 1/sqrt(D).  The exp2 argument is one FMA,
 * fma(S, c, log2(448) - m), which rounds once where the formula above rounds
 * twice; agreement with the formula's own FP32 evaluation to the stated
 * tolerances holds while |m| (scaled scores, log2 units) stays below about
 * 1500.  out: bf16 [B,H,Nq,D] with strides->o; it must not overlap any buffer
 * of `quant`, and its strides must give every element its own address
 * (ordered by stride, each dimension of size > 1 steps past the span of the
 * ones inside it; every packed layout qualifies), else SAGE_E_ALIAS.  One
 * kernel launch on `stream`.
 */
int sage_attn_fwd(const sage_quant_t *quant, const sage_shape_t *shape, float sm_scale, void *out,
                  const sage_strides_t *strides, void *stream);
/* (The forward reads every buffer of `quant` but the workspace, which may be
 * NULL here; this holds for every forward entry below.) */

/*
 * K/V half of sage_quant_prep: the K mean, K smoothing and per-tile INT8 K, and
 * the per-channel FP8 V of stage 1-2 above ("Experiment Log", Phase 0 stage
 * list), bit-identical to what sage_quant_prep writes for them.  q is not an
 * argument: quant->q_codes and quant->q_scale are neither read nor written and
 * may be NULL; shape->Nq is not used (any value >= 1).  The resulting K/V set
 * serves sage_attn_fwd_q for queries of any length.  k, v: bf16 device tensors
 * with strides->k/v (strides->q unused).  Writes k_mean, k_codes, k_scale,
 * v_codes, v_scale and the workspace.  Errors as for sage_quant_prep.
 * Launches 3 kernels on `stream`.
 */
int sage_quant_prep_kv(const void *k, const void *v, const sage_shape_t *shape, const sage_strides_t *strides,
                       const sage_quant_t *quant, void *stream);

/*
 * sage_attn_fwd on bf16 Q: every workgroup first quantizes its own 128-row Q
 * block by stage 2's rule (A = max|x| over the block's real rows and all
 * channels, scale = fp32(A/127), code = RNE(fp32(x * fp32(127/A))), the same
 * arithmetic as sage_quant_prep), then runs stages 3-5 as sage_attn_fwd.  The
 * codes and scales equal the prep's bit for bit, so the output equals
 * sage_quant_prep + sage_attn_fwd bit for bit, while the Q codes never pass
 * through memory.  q: bf16 [B,H,Nq,D] with strides->q (16-byte aligned, strides
 * multiples of 8 elements); shape->Nq is q's length and may differ from the
 * one the K/V set was prepared with.  quant: a K/V set from sage_quant_prep_kv
 * or sage_quant_prep (q_codes, q_scale and the workspace unused, may be NULL).
 * out as for sage_attn_fwd, and it must not overlap q (SAGE_E_ALIAS).  One
 * kernel launch on `stream`.
 */
int sage_attn_fwd_q(const void *q, const sage_quant_t *quant, const sage_shape_t *shape, float sm_scale,
                    void *out, const sage_strides_t *strides, void *stream);

/*
 * sage_attn_fwd with the paired schedule (the analogue of the pages' temporal
 * pairing, "Experiment Log", Closed Prior Work, and "Experiment Registry",
 * Complete Registry): each workgroup takes three consecutive 128-row Q blocks
 * of one (b,h) (twelve wavefronts) and streams every K/V tile through LDS once
 * for all three, instead of once per block.  Same arithmetic per query row,
 * so the output is bit-identical to sage_attn_fwd.  Arguments, layouts,
 * ownership and errors as for sage_attn_fwd.  Slower than sage_attn_fwd on the
 * workloads measured: the K/V re-reads it removes are L2 hits there, and the
 * three wavefronts that share a SIMD then run in step behind one barrier
 * instead of overlapping their matrix and vector phases.
 */
int sage_attn_fwd_paired(const sage_quant_t *quant, const sage_shape_t *shape, float sm_scale, void *out,
                         const sage_strides_t *strides, void *stream);

/*
 * Diagnostic variant of sage_attn_fwd (same kernel source, capture build):
 * runs only the n_units work units listed in `units` (device int32 array;
 * unit = ((b*H + h) * NQB + qblock)) and, besides their O rows, writes all
 * nine checkpoints of the Phase 2B prototype description (QK, m, d, FP8
 * probability, rescale, PV partial, FP32 RO, reciprocal, BF16 output) for them:
 *   s_cap    int32 [n_units][128][T*64]  QK scores (pad keys: the raw score)
 *   p8_cap   uint8 [n_units][128][T*64]  FP8 probability codes (masked: 0)
 *   md_cap   float [n_units][128][T][3]  after tile j: running max m, 448*d and
 *                                        the rescale factor alpha of tile j
 *   part_cap float [n_units][128][T][D]  PV partial of tile j (P8 . V8_j, FP32)
 *   ro_cap   float [n_units][128][T][D]  RO after tile j
 *   r_cap    float [n_units][128]        reciprocal 1/(448*d) of the final d
 * (P is carried as 448 * p, so d carries the factor 448 too.)  Rows >= Nq of a
 * unit hold values for zero pad codes.  Unit ids must be distinct; the kernel
 * skips ids outside [0, B*H*NQB) and their capture slots are left unwritten.
 * Every capture pointer must be 16-byte aligned.
 */
int sage_attn_fwd_capture(const sage_quant_t *quant, const sage_shape_t *shape, float sm_scale,
                          void *out, const sage_strides_t *strides, const int32_t *units,
                          int32_t n_units, int32_t *s_cap, uint8_t *p8_cap, float *md_cap,
                          float *part_cap, float *ro_cap, float *r_cap, void *stream);

/*
 * Race gate (tests only; the analogue of the race checks the pages require of
 * every candidate, "Experiment Log", Phase 2A VEA-B Capability Decision):
 * sage_quant_prep followed by sage_attn_fwd, both built with wave-uniform
 * pseudo-random pauses (0 to 1024 cycles, drawn from `seed`, the workgroup, the
 * wave, the site and the step) before every LDS write and read and every HBM ->
 * LDS tile copy of the three prep launches and the forward.  With correct
 * synchronisation the order in which waves reach those accesses cannot change
 * any result, so every buffer of `quant` and `out` must come out bit-identical
 * to the two normal calls.  Much slower than the normal calls.  Arguments as for
 * sage_quant_prep and sage_attn_fwd; `out` must not overlap q, k or v; seed 0
 * returns SAGE_E_ARG.
 */
int sage_race_gate(const void *q, const void *k, const void *v, const sage_shape_t *shape,
                   const sage_strides_t *strides, const sage_quant_t *quant, float sm_scale, void *out,
                   uint32_t seed, void *stream);

/* Diagnostics: when `stream` reaches the call, SAGE_CLOCK_SAMPLES workgroups
 * each write to dst[4*i .. 4*i+3] (device uint64, 8-byte aligned): the
 * shader-clock counter (s_memtime, kept per compute unit), the constant
 * 100 MHz counter (s_memrealtime), the XCD id and the compute unit's hardware
 * id (HW_REG_HW_ID; bits 8-14 name the unit inside its XCD).  Two
 * samples around a timed region, matched by (XCD, unit), give each unit's
 * average shader clock over it: delta(counter) / delta(100 MHz counter) * 100 MHz. */
#define SAGE_CLOCK_SAMPLES 2048
int sage_clock_sample(uint64_t *dst, void *stream);

/* Diagnostics: a sample of the matrix cores' sustained rate, for comparing the
 * forward with what the hardware reaches rather than only with the nominal
 * peak.  SAGE_PEAK_WORKGROUPS workgroups of four waves (four waves per SIMD of
 * a 256-CU device); every wave issues `iters` rounds of four independent
 * accumulation chains of one matrix instruction on register operands:
 * kind 0 = v_mfma_i32_32x32x32_i8 (32*32*32*2 = 65536 ops each), kind 1 =
 * v_mfma_f32_32x32x64_f8f6f4 with E4M3 operands (131072 ops each).  Operations
 * per call: SAGE_PEAK_WORKGROUPS * 4 * iters * 4 * (ops per instruction); the
 * caller times the call with events on `stream`.  Each thread writes one word
 * of its accumulators to dst[SAGE_PEAK_WORKGROUPS * 256] (device, 4-byte
 * aligned; caller-owned; contents meaningless).  SAGE_E_ARG for a kind other
 * than 0 or 1 or iters outside [1, SAGE_PEAK_MAX_ITERS]. */
#define SAGE_PEAK_WORKGROUPS 1024
#define SAGE_PEAK_MAX_ITERS 65536
int sage_mfma_peak_sample(int kind, int iters, uint32_t *dst, void *stream);

/* Diagnostics: a sample of the vector issue rates that bound the forward's
 * softmax work, alone and beside matrix work, for the per-wave-tile cycle
 * account of the forward.  SAGE_VALU_WORKGROUPS workgroups of sixteen waves
 * (one per compute unit of a 256-CU device; wave w runs on SIMD w % 4); the
 * four waves of each SIMD take the roles of `mix` (role 0 idle, 1 FP32 FMA
 * v_fma_f32 with sixteen independent chains, 2 v_exp_f32, 3 the INT8
 * 32x32x32 matrix instruction in four independent accumulation chains):
 *   mix 0 = {1,0,0,0}  one FMA wave per SIMD
 *   mix 1 = {1,1,1,0}  three FMA waves
 *   mix 2 = {1,1,1,1}  four FMA waves
 *   mix 3 = {2,2,2,0}  three exp waves
 *   mix 4 = {3,1,1,1}  a matrix stream beside three FMA waves
 *   mix 5 = {3,2,2,2}  a matrix stream beside three exp waves
 * Every active wave issues rounds of 64 vector (or 16 matrix) instructions
 * until window_kcycles * 1000 shader-clock cycles have passed, then writes
 * dst[3 * (16 * workgroup + wave) + {0, 1, 2}] = {rounds completed (0 for idle
 * waves), cycles taken (s_memtime), a word of its results}; dst: device uint32
 * of 3 * 16 * SAGE_VALU_WORKGROUPS elements, 4-byte aligned, caller-owned.
 * SAGE_E_ARG for a mix outside [0, SAGE_VALU_MIXES) or window_kcycles outside
 * [1, SAGE_VALU_MAX_KCYCLES]. */
#define SAGE_VALU_WORKGROUPS 256
#define SAGE_VALU_MIXES 6
#define SAGE_VALU_MAX_KCYCLES 10000
int sage_valu_sample(int mix, int window_kcycles, uint32_t *dst, void *stream);

/* SAGE_OK if `device` is a gfx950 GPU, else SAGE_E_DEVICE (one HIP query). */
int sage_device_check(int device);

/* Static description of a status code. */
const char *sage_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* SAGE_ATTN_H */
