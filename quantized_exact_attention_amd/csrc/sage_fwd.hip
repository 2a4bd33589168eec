// Fused quantized attention forward for gfx950 (CDNA4).
//
// Stages 3-5 of the contract imported in "Experiment Log", Phase 0 Import And
// Verification: QK traversal (INT8, int32 accumulation), online softmax, FP8
// probabilities, two-level PV accumulation and final conversion, keeping the
// invariants of the Phase 1 State-Ownership Decision (strict KV-tile order,
// exact FP8 score bytes, per-tile RO rescaling, two-level PV).  The capture
// build (template flag CAP) writes, for listed work units, every checkpoint
// named in Phase 2B Fixed Aligned Numerical Prototype (QK, m, d, FP8
// probability, rescale, PV partial, RO, reciprocal, BF16 output); the race-gate
// build (RACE) adds seeded pauses before every LDS access and tile copy; QPW
// selects one Q block per workgroup (default) or the paired schedule; the
// Q-quantizing build (QIN) takes bf16 Q and quantizes its block in the
// prologue instead of reading the prep's codes.
//
// Work decomposition: one workgroup = 4 wavefronts = one 128-row Q block of one
// (b,h); each wavefront owns 32 query rows and walks all 64-key tiles in order.
// Per tile and wavefront:
//   S^T[64 keys x 32 queries] = K_j . Q^T   2 x (D/32) v_mfma_i32_32x32x32_i8
//   (accumulated on a constant offset so that each score reads back as a
//   float with one subtraction, see kScoreBias)
//   softmax on S^T: every lane holds ONE query and 32 of the 64 keys, so the
//   row max is an in-lane reduction plus one permlane32 swap, m and alpha are
//   per-lane scalars, and each half-wave carries the running row sum of its
//   own 32 keys (the two halves are added once, after the last tile)
//   P8^T stays in registers: the accumulator layout of S^T is already the
//   B-operand layout of O^T = V^T . P^T (no LDS round trip for P)
//   partial^T[D x 32] = V_j^T . P8^T         (D/32) v_mfma_f32_32x32x64_f8f6f4
//   RO = fma(RO, alpha, partial)            (two-level accumulation)
// K and V tiles (operand-ordered by the prep stage) are streamed through two
// LDS buffers by global_load_lds (HBM -> LDS without registers): the copy of
// tile j+1 is issued before tile j's math and waited for at its end.  Each
// wave sets its issue priority by the phase of the tile (see kPrioMatrix).
#include <climits>

#include "sage_common.h"

namespace sage {

// Workgroup id -> work unit, so that the units of one (b,h) (consecutive ids)
// run on the same XCD: hardware dispatches workgroup i to XCD i % 8, and each
// XCD has its own L2, which then serves the K/V re-reads of that head.
__device__ __forceinline__ int xcd_remap(int i, int n) {
  constexpr int NX = 8;
  const int per = (n + NX - 1) / NX;
  int tall = n % NX;
  if (tall == 0) tall = NX;
  const int x = i % NX, loc = i / NX;
  return x < tall ? x * per + loc : tall * per + (x - tall) * (per - 1) + loc;
}

__device__ __forceinline__ int partner_max(int x) {
  auto s = __builtin_amdgcn_permlane32_swap((unsigned)x, (unsigned)x, false, false);
  return max((int)s[0], (int)s[1]);
}
__device__ __forceinline__ float partner_sum(float x) {
  auto s = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(s[0]) + __uint_as_float(s[1]);
}

// Waves per SIMD: 3 at D = 128 (at most 168 VGPRs per lane for the per-wave
// state RO 64, S/p 32, P8 8, Q 16, partials up to 64; the kernel uses 152 with
// no scratch), 5 at D = 64 (at most 96 VGPRs; no scratch in the fast build).
template <int D> struct FwdOccupancy { static constexpr int waves_per_simd = D == 128 ? 3 : 5; };

// Wave priority by phase of the tile.  While one wave's matrix instructions
// run, the SIMD's other waves issue VALU instructions at a reduced rate, and
// the reduction is smallest for the quarter-rate exp and FP8 conversions
// (about 8 -> 11 cycles, against 2 -> 5 for an FMA).  So matrix issue runs at
// priority 3, the exp / row-sum / pack block at 2, the full-rate scale
// arithmetic before it at 1 and the RO update at 0: when several waves are
// ready, the one whose work suffers least beside matrix work issues first,
// and the RO update fills the gaps.
constexpr int kPrioMatrix = 3, kPrioExp = 2, kPrioScale = 1, kPrioUpdate = 0;

// The lane id, computed afresh where it is used (v_mbcnt) so that no register
// carries it through the traversal.  Volatile asm: the compiler would otherwise
// hoist the computation out of the tile loop, or merge it with an earlier one,
// and keep the result live across the loop.
__device__ __forceinline__ int fresh_lane_id() {
  int l;
  asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(l));
  return l;
}

// Masking of the ragged last tile: lane l holds keys kb*32 + 8*(v/4) + 4*(l/32)
// + v%4, so key (kb, v) is past Nkv iff kb*32 + 8*(v/4) + v%4 >= kvalid -
// 4*(l/32).  No register carries the 32 key indices through the traversal.
__device__ __forceinline__ int masked_key_limit(int kvalid) { return kvalid - 4 * (fresh_lane_id() >> 5); }

// Scores accumulate on top of the bit pattern of 1/(2 pi), 0x3E22F983, which
// the matrix instruction takes as an inline constant for its accumulator
// input.  That float lies in the binade [1/8, 1/4), where consecutive floats
// are 2^-26 apart and consecutive bit patterns are consecutive floats; its
// pattern is 0x22F983 = 2292099 steps above the binade's start.  So for
// -2292099 <= s < 6096509 the int32 result read as a float is exactly
// 1/(2 pi) + s * 2^-26, and one full-rate subtraction (exact: both operands
// in one binade) gives s * 2^-26 (v_cvt_f32_i32 issues at half the rate of
// v_sub_f32 on gfx950).  Scaling the per-tile factor by 2^26 is exact too, so
// fma(s * 2^-26, c * 2^26, b) rounds s * c + b exactly once, as from s itself.
// The biased integers keep the order of the scores: the row max is taken on
// them directly.  |s| <= 127 * 127 * D.
constexpr int kScoreBias = 0x3E22F983;
constexpr float kScoreUnit = 67108864.0f;   // 2^26
static_assert(127 * 127 * 128 < 0x22F983, "biased scores must stay in one binade");

// First k-step of S^T with the accumulator input set to kScoreBias.  Written
// out because the compiler materialises a constant shared by several matrix
// instructions in registers instead of using the inline constant.  Its result
// is read only by the next k-step's matrix instruction of the same opcode, as
// that instruction's accumulator input (back-to-back accumulation, which needs
// no wait states); its inputs come from an LDS read (waited for by the
// compiler) and from registers written once before the traversal.
__device__ __forceinline__ v16i mfma_i8_biased(v4i a, v4i b) {
  v16i d;
  asm volatile("v_mfma_i32_32x32x32_i8 %0, %1, %2, 0.15915494" : "=v"(d) : "v"(a), "v"(b));
  return d;
}

// s * 2^-26 from a biased score (exact)
__device__ __forceinline__ float score_scaled(int biased) {
  return __int_as_float(biased) - __int_as_float(kScoreBias);
}

// log2(448): P is produced directly as 448 * 2^(s - m) = 2^(s - m + log2 448).
constexpr float kLog2_448 = 8.80735492205760410744f;

// Read-only scalars through the constant address space: a scalar (SMEM) load,
// tracked by lgkmcnt, so waiting for it never waits for the in-flight K/V DMA.
__device__ __forceinline__ float load_uniform(const float *ptr) {
  return *(const __attribute__((address_space(4))) float *)ptr;
}

typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(1))) void glb_void_t;

// Issue the HBM -> LDS copy of K/V tile t (global_load_lds_dwordx4, no VGPRs):
// wave w copies 1 KiB chunks c = i*4 + w of the [K tile | V tile] image.
template <int D>
__device__ __forceinline__ void issue_tile(uint8_t *dst, const int8_t *kg, const uint8_t *vg, int t, int wave,
                                           int lane) {
  constexpr int TILE = kBK * D;
  constexpr int NLD = 2 * TILE / 4096;
#pragma unroll
  for (int i = 0; i < NLD; ++i) {
    const int c = i * 4 + wave;
    // uniform base per chunk + one unsigned 32-bit offset (the tile and the
    // lane) shared by the chunks: the SGPR-base addressing form.  The tile
    // index is split so that the 32-bit offset stays below 2^29 for any number
    // of tiles; the high part moves the base once every 65536 tiles.
    const uint8_t *base = (i < NLD / 2 ? (const uint8_t *)kg + c * 1024 : vg + (c - TILE / 1024) * 1024) +
                          (size_t)(t >> 16) * ((size_t)TILE << 16);
    const uint32_t off = (uint32_t)(t & 0xffff) * (uint32_t)TILE + (uint32_t)lane * 16u;
    __builtin_amdgcn_global_load_lds((glb_void_t *)(base + off), (lds_void_t *)(dst + c * 1024), 16, 0, 0);
  }
}

template <int D>
struct FwdState {
  float m;      // running row max (scaled, log2 units), the same in both half-waves
  float dsum;   // running row sum over this half-wave's keys (x 448)
  v16f ro[D / 32];
};

// One 64-key tile of the ordered traversal for one wavefront (32 query rows).
// `cur` holds tile j; tile j+1 is copied into `nxt` meanwhile.  Ends with the
// workgroup barrier that publishes `nxt` and retires `cur`.
template <int D, bool CAP, bool RACE, int QPW>
__device__ __forceinline__ void tile_step(const FwdParams &p, FwdState<D> &st, const v4i *qop, float sq, float pinf, int j,
                                          const uint8_t *cur, uint8_t *nxt, const int8_t *kg, const uint8_t *vg,
                                          const float *ksc, int wave, int lane, int row) {
  constexpr int NS = D / 32;
  constexpr int TILE = kBK * D;
  const int T = p.T;
  const int hi = lane >> 5;   // which 4-key group of each 8 this lane holds
  if (RACE) race_pause(p.race_seed, 0, j);
  if (j + 1 < T && (QPW == 1 || wave < 4)) issue_tile<D>(nxt, kg, vg, j + 1, wave, lane);
  const uint8_t *kl = cur + lane * 16;        // this lane's 16 bytes of every 1 KiB operand block
  const uint8_t *vl = kl + TILE;

  // ---- S^T = K_j . Q^T (int32, exact, offset by kScoreBias) ----
  __builtin_amdgcn_s_setprio(kPrioMatrix);
  if (RACE) race_pause(p.race_seed, 1, j);
  v16i sacc[2];
#pragma unroll
  for (int s = 0; s < NS; ++s) {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const v4i a = *(const v4i *)(kl + (kb * NS + s) * 1024);
      if (s == 0) sacc[kb] = mfma_i8_biased(a, qop[0]);
      else sacc[kb] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, qop[s], sacc[kb], 0, 0, 0);
    }
  }
  if (CAP) {
    int32_t *sc = p.s_cap + ((size_t)blockIdx.x * kBQ + row) * ((size_t)T * kBK) + (size_t)j * kBK;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int v = 0; v < 16; ++v) sc[kb * 32 + 8 * (v >> 2) + 4 * hi + (v & 3)] = sacc[kb][v] - kScoreBias;
  }
  __builtin_amdgcn_s_setprio(kPrioScale);
  // ragged tail: keys >= Nkv of the last tile take no part in max, sum or PV
  const int kvalid = p.Nkv - j * kBK;
  const bool masked = kvalid < kBK;
  if (masked) {
    const int klim = masked_key_limit(kvalid);
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int v = 0; v < 16; ++v)
        if (kb * 32 + 8 * (v >> 2) + (v & 3) >= klim) sacc[kb][v] = INT_MIN;
  }

  // ---- online softmax; max in the integer domain (the per-tile factor is >= 0) ----
  // 32 values -> 12 -> 4 -> 1: fifteen three-input maxima and one two-input
  int m12[10];
#pragma unroll
  for (int i = 0; i < 10; ++i) {
    const int x = 3 * i;
    m12[i] = max(max(sacc[x >> 4][x & 15], sacc[(x + 1) >> 4][(x + 1) & 15]), sacc[(x + 2) >> 4][(x + 2) & 15]);
  }
  const int m4a = max(max(m12[0], m12[1]), m12[2]), m4b = max(max(m12[3], m12[4]), m12[5]);
  const int m4c = max(max(m12[6], m12[7]), m12[8]), m4d = max(max(m12[9], sacc[1][14]), sacc[1][15]);
  int mx = max(max(max(m4a, m4b), m4c), m4d);
  mx = partner_max(mx);
  const float c = (sq * load_uniform(ksc + j)) * p.sl2;   // fp32(fp32(sq * sk_j) * sl2)
  const float cu = c * kScoreUnit;                          // exact
  const float mnew = __builtin_amdgcn_fmed3f(st.m, score_scaled(mx) * cu, pinf);   // max; no NaN here
  const float alpha = __builtin_amdgcn_exp2f(st.m - mnew);   // "rescale"; 0 on the first tile
  const float nb = kLog2_448 - mnew;
  // arguments first (full rate), then the exps under the higher priority
  float pv[2][16];
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int v = 0; v < 16; ++v) pv[kb][v] = __builtin_fmaf(score_scaled(sacc[kb][v]), cu, nb);
  __builtin_amdgcn_s_setprio(kPrioExp);
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int v = 0; v < 16; ++v) pv[kb][v] = __builtin_amdgcn_exp2f(pv[kb][v]);
  if (masked) {
    const int klim = masked_key_limit(kvalid);
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int v = 0; v < 16; ++v)
        if (kb * 32 + 8 * (v >> 2) + (v & 3) >= klim) pv[kb][v] = 0.f;
  }
  // row sum as a tree (short dependency chains)
  float s8[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int kb = i >> 2, v0 = 4 * (i & 3);
    s8[i] = (pv[kb][v0] + pv[kb][v0 + 1]) + (pv[kb][v0 + 2] + pv[kb][v0 + 3]);
  }
  const float ls = ((s8[0] + s8[1]) + (s8[2] + s8[3])) + ((s8[4] + s8[5]) + (s8[6] + s8[7]));
  // this half-wave's running sum (d carries the factor 448); the halves meet
  // after the last tile, which only reorders the FP32 additions of the row sum
  st.dsum = __builtin_fmaf(st.dsum, alpha, ls);
  asm volatile("" ::"v"(ls));   // kept live past the FMA, as the partials below
  st.m = mnew;

  // ---- P8 (E4M3FN, RNE) packed straight into the B operand of the PV product ----
  v8i pop;
#pragma unroll
  for (int w = 0; w < 8; ++w) {
    const int kb = w >> 2, v0 = 4 * (w & 3);
    // the high half is written next, so the first conversion's "old" operand
    // can be any dead register (no zeroing move)
    int x = __builtin_amdgcn_cvt_pk_fp8_f32(pv[kb][v0], pv[kb][v0 + 1], __float_as_int(pv[kb][v0 + 1]), false);
    x = __builtin_amdgcn_cvt_pk_fp8_f32(pv[kb][v0 + 2], pv[kb][v0 + 3], x, true);
    pop[w] = x;
  }
  if (CAP) {
    uint8_t *pc = p.p8_cap + ((size_t)blockIdx.x * kBQ + row) * ((size_t)T * kBK) + (size_t)j * kBK;
#pragma unroll
    for (int w = 0; w < 8; ++w)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int v = 4 * (w & 3) + e;
        pc[(w >> 2) * 32 + 8 * (v >> 2) + 4 * hi + (v & 3)] = (uint8_t)((uint32_t)pop[w] >> (8 * e));
      }
    const float dj = partner_sum(st.dsum);   // d after tile j: both halves
    if (hi == 0) {
      float *md = p.md_cap + (((size_t)blockIdx.x * kBQ + row) * T + j) * 3;
      md[0] = st.m;
      md[1] = dj;
      md[2] = alpha;
    }
  }

  // ---- partial^T = V_j^T . P8^T (FP32, fresh), then RO = RO * alpha + partial ----
  __builtin_amdgcn_s_setprio(kPrioMatrix);
  if (RACE) race_pause(p.race_seed, 2, j);
  const v16f zero16 = {};
  v16f part[NS];
#pragma unroll
  for (int cb = 0; cb < NS; ++cb) {
    const v4i a0 = *(const v4i *)(vl + (cb * 2 + 0) * 1024);
    const v4i a1 = *(const v4i *)(vl + (cb * 2 + 1) * 1024);
    const v8i a = {a0[0], a0[1], a0[2], a0[3], a1[0], a1[1], a1[2], a1[3]};
    part[cb] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, pop, zero16, 0, 0, 0, 0, 0, 0);
  }
  __builtin_amdgcn_s_setprio(kPrioUpdate);
#pragma unroll
  for (int cb = 0; cb < NS; ++cb)
#pragma unroll
    for (int v = 0; v < 16; ++v) st.ro[cb][v] = __builtin_fmaf(st.ro[cb][v], alpha, part[cb][v]);
  // The partials stay live past their last FMA: where the addend dies at the
  // FMA, the compiler writes the sum over it (v_fmac) and copies it back into
  // the loop-carried register, one extra move per accumulator tuple and tile.
#pragma unroll
  for (int cb = 0; cb < NS; ++cb)
    asm volatile("" ::"v"(part[cb].lo.lo), "v"(part[cb].lo.hi), "v"(part[cb].hi.lo), "v"(part[cb].hi.hi));
  if (CAP) {
    // lane (hi, row) holds channels 32 cb + 8 (v / 4) + 4 hi + v % 4
    const size_t o = (((size_t)blockIdx.x * kBQ + row) * T + j) * D;
#pragma unroll
    for (int cb = 0; cb < NS; ++cb)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int ch = 32 * cb + 8 * (v >> 2) + 4 * hi + (v & 3);
        p.part_cap[o + ch] = part[cb][v];
        p.ro_cap[o + ch] = st.ro[cb][v];
      }
  }

  // tile j+1 landed (this wave's copies) and every wave is done with `cur`
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
}

// Q-quantizing build: the workgroup's 128-row Q block from bf16 Q, by the rule
// of the prep stage (absmax over the block's real rows and all channels, scale
// = absmax / 127, code = clamp(RNE(fp32(x * fp32(127 / absmax))))), so the
// codes and the scale equal the prep's bit for bit.  Lane l of wave wq holds
// row wq*32 + l%32 and, per k-step s, channels 32 s + 16 (l/32) .. +15: exactly
// the 16 bytes of the B operand it reads from the prep's code buffer.  The
// four wave maxima meet in `red` (16 bytes of LDS not yet used by the tile
// ring).  Returns the block's scale.
template <int D>
__device__ __forceinline__ float quantize_q_operand(const FwdParams &p, int bh, int qb, int wq, int lane, float *red,
                                                    v4i *qop) {
  constexpr int NS = D / 32;
  const int b = bh / p.H, h = bh - b * p.H;
  const int n = qb * kBQ + wq * 32 + (lane & 31);
  uint4 raw[2 * NS];
  if (n < p.Nq) {                               // rows past Nq are zero and do not raise the max
    const uint16_t *row = p.q + b * p.qs[0] + h * p.qs[1] + (int64_t)n * p.qs[2] + 16 * (lane >> 5);
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      raw[2 * s] = *(const uint4 *)(row + 32 * s);
      raw[2 * s + 1] = *(const uint4 *)(row + 32 * s + 8);
    }
  } else {
#pragma unroll
    for (int i = 0; i < 2 * NS; ++i) raw[i] = make_uint4(0, 0, 0, 0);
  }
  float amax = 0.f;
#pragma unroll
  for (int i = 0; i < 2 * NS; ++i) {
    float f[8];
    unpack8(raw[i], f);
#pragma unroll
    for (int e = 0; e < 8; ++e) amax = fmaxf(amax, fabsf(f[e]));
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off));
  if (lane == 0) red[wq] = amax;
  __syncthreads();
  const float A = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  const float inv = A > 0.f ? 127.0f / A : 0.f;
#pragma unroll
  for (int s = 0; s < NS; ++s) {
    float lo[8], hi[8];
    unpack8(raw[2 * s], lo);
    unpack8(raw[2 * s + 1], hi);
    qop[s] = v4i{(int)pack_i8x4(lo, inv), (int)pack_i8x4(lo + 4, inv), (int)pack_i8x4(hi, inv),
                 (int)pack_i8x4(hi + 4, inv)};
  }
  return A > 0.f ? A / 127.0f : 0.f;
}

// QPW: 128-row Q blocks per workgroup.  1 is the default schedule; 3 is the
// paired schedule (the analogue of temporal pairing, "Experiment Log", Closed
// Prior Work, and the split variants of the Phase 1 decision): three Q blocks
// of one (b,h), twelve waves, share one K/V tile stream through LDS, so each
// K/V tile is copied from L2 once per three blocks instead of once per block.
// QIN: the Q-quantizing build (default schedule only).
template <int D, bool CAP, bool RACE, int QPW, bool QIN = false>
__global__ __launch_bounds__(256 * QPW, FwdOccupancy<D>::waves_per_simd) void k_attn_fwd(FwdParams p) {
  static_assert(!QIN || (QPW == 1 && !CAP && !RACE), "Q quantization in the default schedule only");
  constexpr int NS = D / 32;                 // INT8 k-steps per key row == PV row blocks
  constexpr int TILE = kBK * D;              // bytes of one K (or V) tile
  // two LDS buffers of [K tile | V tile], alternating per tile
  __shared__ __attribute__((aligned(16))) uint8_t lds_a[2 * TILE];
  __shared__ __attribute__((aligned(16))) uint8_t lds_b[2 * TILE];

  const int tid = threadIdx.x, lane = tid & 63;
  // wave index as a scalar: tile-copy addresses and LDS bases stay in SGPRs
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  int u, wq = wave;           // work unit of this wave, wave index inside its Q block
  bool live = true;           // false: a wave group past the head's last Q block (paired schedule)
  if (CAP) {
    u = p.units[blockIdx.x];
    if (u < 0 || u >= p.n_units) return;
  } else if (QPW == 1) {
    u = xcd_remap(blockIdx.x, gridDim.x);
  } else {
    const int g = xcd_remap(blockIdx.x, gridDim.x), ngq = (p.nqb + QPW - 1) / QPW;
    const int gbh = g / ngq, qraw = (g - gbh * ngq) * QPW + wave / 4;
    live = qraw < p.nqb;
    u = gbh * p.nqb + (live ? qraw : p.nqb - 1);   // a dead group repeats the last block, stores nothing
    wq = wave & 3;
  }
  const int bh = u / p.nqb, qb = u - bh * p.nqb;
  const int T = p.T;
  const int8_t *kg = p.k_codes + (size_t)bh * T * TILE;
  const uint8_t *vg = p.v_codes + (size_t)bh * T * TILE;
  const float *ksc = p.k_scale + (size_t)bh * T;

  if (RACE) race_pause(p.race_seed, 3, 0);
  if (QPW == 1 || wave < 4) issue_tile<D>(lds_a, kg, vg, 0, wave, lane);

  // Q^T operand (B of the INT8 product) for this wave's 32 rows, kept in registers.
  v4i qop[NS];
  float sq;
  if (QIN) {
    // lds_b is first written by tile 0's step, after the barrier below; the
    // scale is the same in every lane and stays in a VGPR (as below)
    sq = quantize_q_operand<D>(p, bh, qb, wq, lane, (float *)lds_b, qop);
  } else {
    const int8_t *qsrc = p.q_codes + ((size_t)u * 4 + wq) * (NS * 1024) + lane * 16;
#pragma unroll
    for (int s = 0; s < NS; ++s) qop[s] = *(const v4i *)(qsrc + s * 1024);
    // the Q scale in a VGPR: its per-tile product with the K scale (an SGPR)
    // then needs no copy, as one VALU instruction reads at most one SGPR
    asm volatile("v_mov_b32 %0, %1" : "=v"(sq) : "s"(load_uniform(p.q_scale + u)));
  }
  const int row = wq * 32 + (lane & 31);
  // +inf as a value the compiler cannot fold: the running max then stays one
  // v_med3_f32 (folded to a max, it costs one more instruction to canonicalize
  // its loop-carried operand)
  float pinf;
  asm volatile("s_mov_b32 %0, 0x7f800000" : "=s"(pinf));

  FwdState<D> st;
  st.m = -INFINITY;
  st.dsum = 0.f;
#pragma unroll
  for (int cb = 0; cb < NS; ++cb)
#pragma unroll
    for (int v = 0; v < 16; ++v) st.ro[cb][v] = 0.f;

  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
#pragma nounroll
  for (int j = 0; j < T; ++j) {
    uint8_t *cur = (j & 1) ? lds_b : lds_a;
    uint8_t *nxt = (j & 1) ? lds_a : lds_b;
    tile_step<D, CAP, RACE, QPW>(p, st, qop, sq, pinf, j, cur, nxt, kg, vg, ksc, wave, lane, row);
  }

  __builtin_amdgcn_s_setprio(3);                 // finish and free the slot quickly

  // ---- final conversion: reciprocal of d, per-channel V scale, BF16 ----
  // lane and row recomputed (scalar wave index) so that no register holds them
  // through the traversal
  const int elane = fresh_lane_id();
  const int hi = elane >> 5;
  const int n = qb * kBQ + wq * 32 + (elane & 31);
  const float r = 1.0f / partner_sum(st.dsum);    // "reciprocal" of both halves' d (includes the 448)
  if (CAP && hi == 0) p.r_cap[(size_t)blockIdx.x * kBQ + wq * 32 + (elane & 31)] = r;
  if (live && n < p.Nq) {
    const int b = bh / p.H, h = bh - b * p.H;
    uint16_t *orow = p.out + b * p.os[0] + h * p.os[1] + (int64_t)n * p.os[2];
    const float *vs = p.v_scale + (size_t)bh * D;
#pragma unroll
    for (int cb = 0; cb < NS; ++cb)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const int ch = 32 * cb + 8 * q4 + 4 * hi;
        uint32_t w[2];
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          const float o0 = (st.ro[cb][4 * q4 + 2 * e] * r) * vs[ch + 2 * e];
          const float o1 = (st.ro[cb][4 * q4 + 2 * e + 1] * r) * vs[ch + 2 * e + 1];
          const __bf16 b0 = (__bf16)o0, b1 = (__bf16)o1;
          w[e] = (uint32_t)__builtin_bit_cast(uint16_t, b0) | ((uint32_t)__builtin_bit_cast(uint16_t, b1) << 16);
        }
        *(uint2 *)(orow + ch) = make_uint2(w[0], w[1]);
      }
  }
}

template <int D>
static void launch_fwd_d(const FwdParams &p, int grid, FwdVariant variant, hipStream_t st) {
  switch (variant) {
    case FwdVariant::kCapture:
      hipLaunchKernelGGL((k_attn_fwd<D, true, false, 1>), dim3(grid), dim3(256), 0, st, p);
      break;
    case FwdVariant::kRace:
      hipLaunchKernelGGL((k_attn_fwd<D, false, true, 1>), dim3(grid), dim3(256), 0, st, p);
      break;
    case FwdVariant::kPaired: {
      const int groups = (p.n_units / p.nqb) * ((p.nqb + kPairedBlocks - 1) / kPairedBlocks);
      hipLaunchKernelGGL((k_attn_fwd<D, false, false, kPairedBlocks>), dim3(groups), dim3(256 * kPairedBlocks), 0,
                         st, p);
      break;
    }
    case FwdVariant::kQuantizeQ:
      hipLaunchKernelGGL((k_attn_fwd<D, false, false, 1, true>), dim3(grid), dim3(256), 0, st, p);
      break;
    default:
      hipLaunchKernelGGL((k_attn_fwd<D, false, false, 1>), dim3(grid), dim3(256), 0, st, p);
      break;
  }
}

hipError_t launch_fwd(const FwdParams &p, int D, int grid, FwdVariant variant, hipStream_t st) {
  if (D == 128) launch_fwd_d<128>(p, grid, variant, st);
  else launch_fwd_d<64>(p, grid, variant, st);
  return hipGetLastError();
}

}  // namespace sage
