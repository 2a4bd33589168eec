// Fused quantized attention forward for gfx950 (CDNA4).
//
// Stages 3-5 of the contract imported in "Experiment Log", Phase 0 Import And
// Verification: QK traversal (INT8, int32 accumulation), online softmax, FP8
// probabilities, two-level PV accumulation and final conversion, keeping the
// invariants of the Phase 1 State-Ownership Decision (strict KV-tile order,
// exact FP8 score bytes, per-tile RO rescaling, two-level PV) and producing the
// checkpoints named in Phase 2B Fixed Aligned Numerical Prototype (QK, m, d,
// FP8 probability, rescale, PV partial, RO, reciprocal, BF16 output).
//
// Work decomposition: one workgroup = 4 wavefronts = one 128-row Q block of one
// (b,h); each wavefront owns 32 query rows and walks all 64-key tiles in order.
// Per tile and wavefront:
//   S^T[64 keys x 32 queries] = K_j . Q^T   2 x (D/32) v_mfma_i32_32x32x32_i8
//   softmax on S^T: every lane holds ONE query and 32 of the 64 keys, so the
//   row max / row sum are in-lane reductions plus one permlane32 swap, and
//   m, d, alpha are per-lane scalars
//   P8^T stays in registers: the accumulator layout of S^T is already the
//   B-operand layout of O^T = V^T . P^T (no LDS round trip for P)
//   partial^T[D x 32] = V_j^T . P8^T         (D/32) v_mfma_f32_32x32x64_f8f6f4
//   RO = fma(RO, alpha, partial)            (two-level accumulation)
// K and V tiles (operand-ordered by the prep stage) are streamed through a
// double-buffered LDS ring: the next tile's global loads are issued before the
// current tile's math and written to the other buffer after it.
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

// log2(448): P is produced directly as 448 * 2^(s - m) = 2^(s - m + log2 448).
constexpr float kLog2_448 = 8.80735492205760410744f;

template <int D, bool CAP>
__global__ __launch_bounds__(256) void k_attn_fwd(FwdParams p) {
  constexpr int NS = D / 32;                 // INT8 k-steps per key row == PV row blocks
  constexpr int TILE = kBK * D;              // bytes of one K (or V) tile
  constexpr int NLD = 2 * TILE / (256 * 16); // 16-byte loads per thread per K+V tile
  __shared__ __attribute__((aligned(16))) uint8_t lds[2][2 * TILE];

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  int u;
  if (CAP) {
    u = p.units[blockIdx.x];
    if (u < 0 || u >= p.n_units) return;
  } else {
    u = xcd_remap(blockIdx.x, gridDim.x);
  }
  const int bh = u / p.nqb, qb = u - bh * p.nqb;
  const int T = p.T;

  // Q^T operand (B of the INT8 product) for this wave's 32 rows, kept in registers.
  v4i qop[NS];
  {
    const int8_t *qsrc = p.q_codes + ((size_t)u * 4 + wave) * (NS * 1024) + lane * 16;
#pragma unroll
    for (int s = 0; s < NS; ++s) qop[s] = *(const v4i *)(qsrc + s * 1024);
  }
  const float sq = p.q_scale[u];
  const int8_t *kg = p.k_codes + (size_t)bh * T * TILE;
  const uint8_t *vg = p.v_codes + (size_t)bh * T * TILE;
  const float *ksc = p.k_scale + (size_t)bh * T;

  // chunk i of this thread: 16 bytes at offset (i*256 + tid)*16 of [K tile | V tile]
  const uint8_t *gsrc[NLD];
#pragma unroll
  for (int i = 0; i < NLD; ++i) {
    const int idx = i * 256 + tid;
    gsrc[i] = idx < TILE / 16 ? (const uint8_t *)kg + idx * 16 : vg + (idx - TILE / 16) * 16;
  }
  uint4 pre[NLD];
#pragma unroll
  for (int i = 0; i < NLD; ++i) pre[i] = *(const uint4 *)gsrc[i];
#pragma unroll
  for (int i = 0; i < NLD; ++i) *(uint4 *)(&lds[0][(i * 256 + tid) * 16]) = pre[i];
  __syncthreads();

  float m = -INFINITY, dsum = 0.f;
  v16f ro[NS];
#pragma unroll
  for (int c = 0; c < NS; ++c)
#pragma unroll
    for (int v = 0; v < 16; ++v) ro[c][v] = 0.f;
  const v16f zero16 = {};
  const int hi = lane >> 5;            // which 4-key group of each 8 this lane holds
  const int row = wave * 32 + (lane & 31);

  for (int j = 0; j < T; ++j) {
    const int buf = j & 1;
    // next tile's loads are always issued (the last iteration reloads its own
    // tile into the idle buffer), which keeps the ring free of branches
    const size_t jn = (size_t)min(j + 1, T - 1) * TILE;
#pragma unroll
    for (int i = 0; i < NLD; ++i) pre[i] = *(const uint4 *)(gsrc[i] + jn);
    const uint8_t *kl = lds[buf];
    const uint8_t *vl = lds[buf] + TILE;

    // ---- S^T = K_j . Q^T (int32, exact) ----
    v16i sacc[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      sacc[kb] = (v16i){};
#pragma unroll
      for (int s = 0; s < NS; ++s) {
        const v4i a = *(const v4i *)(kl + (kb * NS + s) * 1024 + lane * 16);
        sacc[kb] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, qop[s], sacc[kb], 0, 0, 0);
      }
    }
    if (CAP) {
      int32_t *sc = p.s_cap + ((size_t)blockIdx.x * kBQ + row) * ((size_t)T * kBK) + (size_t)j * kBK;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int v = 0; v < 16; ++v) sc[kb * 32 + 8 * (v >> 2) + 4 * hi + (v & 3)] = sacc[kb][v];
    }
    // ragged tail: keys >= Nkv of the last tile take no part in max, sum or PV
    const int kvalid = p.Nkv - j * kBK;
    const bool masked = kvalid < kBK;
    if (masked) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int v = 0; v < 16; ++v)
          if (kb * 32 + 8 * (v >> 2) + 4 * hi + (v & 3) >= kvalid) sacc[kb][v] = INT_MIN;
    }

    // ---- online softmax: max in the integer domain (the per-tile factor is >= 0) ----
    int mx = sacc[0][0];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int v = 0; v < 16; ++v) mx = max(mx, sacc[kb][v]);
    mx = partner_max(mx);
    const float c = (sq * ksc[j]) * p.sl2;        // fp32(fp32(sq * sk_j) * sl2)
    const float mnew = fmaxf(m, (float)mx * c);
    const float alpha = __builtin_amdgcn_exp2f(m - mnew);   // "rescale"; 0 on the first tile
    const float nb = kLog2_448 - mnew;
    float pv[2][16];
    float ls = 0.f;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        pv[kb][v] = __builtin_amdgcn_exp2f(__builtin_fmaf((float)sacc[kb][v], c, nb));
      }
    if (masked) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int v = 0; v < 16; ++v)
          if (kb * 32 + 8 * (v >> 2) + 4 * hi + (v & 3) >= kvalid) pv[kb][v] = 0.f;
    }
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int v = 0; v < 16; ++v) ls += pv[kb][v];
    ls = partner_sum(ls);
    dsum = __builtin_fmaf(dsum, alpha, ls);        // d carries the factor 448
    m = mnew;

    // ---- P8 (E4M3FN, RNE) packed straight into the B operand of the PV product ----
    v8i pop;
#pragma unroll
    for (int w = 0; w < 8; ++w) {
      const int kb = w >> 2, v0 = 4 * (w & 3);
      int x = __builtin_amdgcn_cvt_pk_fp8_f32(pv[kb][v0], pv[kb][v0 + 1], 0, false);
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
      if (hi == 0) {
        float *md = p.md_cap + (((size_t)blockIdx.x * kBQ + row) * T + j) * 2;
        md[0] = m;
        md[1] = dsum;
      }
    }

    // ---- partial^T = V_j^T . P8^T (FP32), then RO = RO * alpha + partial ----
#pragma unroll
    for (int c = 0; c < NS; ++c) {
      const v4i a0 = *(const v4i *)(vl + (c * 2 + 0) * 1024 + lane * 16);
      const v4i a1 = *(const v4i *)(vl + (c * 2 + 1) * 1024 + lane * 16);
      const v8i a = {a0[0], a0[1], a0[2], a0[3], a1[0], a1[1], a1[2], a1[3]};
      const v16f part = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, pop, zero16, 0, 0, 0, 0, 0, 0);
#pragma unroll
      for (int v = 0; v < 16; ++v) ro[c][v] = __builtin_fmaf(ro[c][v], alpha, part[v]);
    }

#pragma unroll
    for (int i = 0; i < NLD; ++i) *(uint4 *)(&lds[buf ^ 1][(i * 256 + tid) * 16]) = pre[i];
    __syncthreads();
  }

  // ---- final conversion: reciprocal of d, per-channel V scale, BF16 ----
  const int n = qb * kBQ + row;
  if (n < p.Nq) {
    const float r = 1.0f / dsum;                  // "reciprocal" (d includes the 448)
    const int b = bh / p.H, h = bh - b * p.H;
    uint16_t *orow = p.out + b * p.os[0] + h * p.os[1] + (int64_t)n * p.os[2];
    const float *vs = p.v_scale + (size_t)bh * D;
#pragma unroll
    for (int c = 0; c < NS; ++c)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const int ch = 32 * c + 8 * q4 + 4 * hi;
        uint32_t w[2];
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          const float o0 = (ro[c][4 * q4 + 2 * e] * r) * vs[ch + 2 * e];
          const float o1 = (ro[c][4 * q4 + 2 * e + 1] * r) * vs[ch + 2 * e + 1];
          const __bf16 b0 = (__bf16)o0, b1 = (__bf16)o1;
          w[e] = (uint32_t)__builtin_bit_cast(uint16_t, b0) | ((uint32_t)__builtin_bit_cast(uint16_t, b1) << 16);
        }
        *(uint2 *)(orow + ch) = make_uint2(w[0], w[1]);
      }
  }
}

hipError_t launch_fwd(const FwdParams &p, int D, int grid, bool capture, hipStream_t st) {
  if (D == 128) {
    if (capture) hipLaunchKernelGGL((k_attn_fwd<128, true>), dim3(grid), dim3(256), 0, st, p);
    else hipLaunchKernelGGL((k_attn_fwd<128, false>), dim3(grid), dim3(256), 0, st, p);
  } else {
    if (capture) hipLaunchKernelGGL((k_attn_fwd<64, true>), dim3(grid), dim3(256), 0, st, p);
    else hipLaunchKernelGGL((k_attn_fwd<64, false>), dim3(grid), dim3(256), 0, st, p);
  }
  return hipGetLastError();
}

}  // namespace sage
