// Prep stage for gfx950: K/V column statistics, K smoothing, per-block INT8
// Q/K and per-channel FP8 (OCP E4M3FN) V, written in the operand order of the
// attention kernel's matrix instructions.  Stages "Q/K preparation, K
// smoothing, INT8 quantization, FP8 V" of the contract imported in
// "Experiment Log", Phase 0 Import And Verification.
//
// All passes are HBM-bound streaming kernels: 16-byte loads along the
// contiguous channel dimension, 16-byte code stores.
#include "sage_common.h"

namespace sage {

__device__ __forceinline__ float bf16f(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

__device__ __forceinline__ void unpack8(const uint4 &x, float *f) {
  const uint32_t w[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f[2 * i] = __uint_as_float(w[i] << 16);
    f[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
  }
}

// Max of a non-negative float over the 256-thread block (bit order == value order).
__device__ __forceinline__ float block_max_nonneg(float x, float *red) {
  uint32_t u = __float_as_uint(x);
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) u = max(u, (uint32_t)__shfl_xor((int)u, o, 64));
  const int w = threadIdx.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[w] = __uint_as_float(u);
  __syncthreads();
  float r = red[0];
#pragma unroll
  for (int i = 1; i < 4; ++i) r = fmaxf(r, red[i]);
  return r;
}

// Byte offset of the 16-byte unit (row r, 16-channel chunk c16) inside a run of
// 32-row groups in INT8 operand order: group g = r/32 holds [D/32 steps][64
// lanes][16 B]; lane = r%32 + 32*(c16%2), step = c16/2.
template <int D>
__device__ __forceinline__ int i8_operand_offset(int r, int c16) {
  const int g = r >> 5, lane = (r & 31) + 32 * (c16 & 1), s = c16 >> 1;
  return ((g * (D / 32) + s) * 64 + lane) * 16;
}

__device__ __forceinline__ uint32_t pack_i8x4(const float *x, float inv) {
  uint32_t w = 0;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    float q = __builtin_rintf(x[e] * inv);          // fp32 product, round half to even
    q = fminf(fmaxf(q, -127.f), 127.f);
    w |= ((uint32_t)(int32_t)q & 0xffu) << (8 * e);
  }
  return w;
}

// ---- 1. per (b,h, key chunk): FP64 column sums of K (exact for bf16 data) and
//         column max |V|; partials go to the workspace --------------------------
template <int D>
struct StatsSmem {
  static constexpr int CG = D / 8;      // 8-channel groups of one row
  static constexpr int TL = 256 / CG;   // rows handled in parallel
  double sum[TL][D];
  float max[TL][D];
};

template <int D>
__device__ __forceinline__ void prep_stats_block(const PrepParams &p, int chunk, int bh, StatsSmem<D> &sm) {
  constexpr int CG = StatsSmem<D>::CG, TL = StatsSmem<D>::TL;
  auto &s_sum = sm.sum;
  auto &s_max = sm.max;
  const int b = bh / p.H, h = bh - b * p.H;
  const int cg = threadIdx.x % CG, tl = threadIdx.x / CG;
  const int n0 = chunk * kStatChunk, n1 = min(p.Nkv, n0 + kStatChunk);
  const uint16_t *kb = p.k + b * p.ks[0] + h * p.ks[1] + cg * 8;
  const uint16_t *vb = p.v + b * p.vs[0] + h * p.vs[1] + cg * 8;
  double acc[8];
  float vmx[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) { acc[e] = 0.0; vmx[e] = 0.f; }
  for (int n = n0 + tl; n < n1; n += TL) {
    float kf[8], vf[8];
    unpack8(*(const uint4 *)(kb + (int64_t)n * p.ks[2]), kf);
    unpack8(*(const uint4 *)(vb + (int64_t)n * p.vs[2]), vf);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      acc[e] += (double)kf[e];
      vmx[e] = fmaxf(vmx[e], fabsf(vf[e]));
    }
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) { s_sum[tl][cg * 8 + e] = acc[e]; s_max[tl][cg * 8 + e] = vmx[e]; }
  __syncthreads();
  for (int c = threadIdx.x; c < D; c += 256) {
    double s = 0.0;
    float mx = 0.f;
    for (int i = 0; i < TL; ++i) { s += s_sum[i][c]; mx = fmaxf(mx, s_max[i][c]); }
    const size_t o = ((size_t)bh * p.nchunk + chunk) * D + c;
    p.ws_ksum[o] = s;
    p.ws_vmax[o] = mx;
  }
}

// ---- 2. per (b,h): K mean, V channel scale and inverse -------------------------
// 256 threads: channel c = t % D, chunk group t / D; the partial sums are exact,
// so their order does not matter.
template <int D>
__global__ __launch_bounds__(256) void k_prep_finalize(PrepParams p) {
  constexpr int NG = 256 / D;
  __shared__ double s_sum[NG][D];
  __shared__ float s_max[NG][D];
  const int bh = blockIdx.x, c = threadIdx.x % D, g = threadIdx.x / D;
  double s = 0.0;
  float mx = 0.f;
  for (int i = g; i < p.nchunk; i += NG) {
    const size_t o = ((size_t)bh * p.nchunk + i) * D + c;
    s += p.ws_ksum[o];
    mx = fmaxf(mx, p.ws_vmax[o]);
  }
  s_sum[g][c] = s;
  s_max[g][c] = mx;
  __syncthreads();
  if (g == 0) {
#pragma unroll
    for (int i = 1; i < NG; ++i) { s += s_sum[i][c]; mx = fmaxf(mx, s_max[i][c]); }
    p.k_mean[bh * D + c] = (float)(s / (double)p.Nkv);   // FP64 quotient, one FP32 rounding
    p.v_scale[bh * D + c] = mx > 0.f ? mx / 448.0f : 0.f;  // correctly rounded FP32 divides
    p.ws_vinv[bh * D + c] = mx > 0.f ? 448.0f / mx : 0.f;
  }
}

// ---- 3. Q: per 128-row block INT8 --------------------------------------------
template <int D>
__device__ __forceinline__ void quant_q_block(const PrepParams &p, int qb, int bh, float *red) {
  constexpr int UPR = D / 16, UPT = kBQ * UPR / 256;
  const int b = bh / p.H, h = bh - b * p.H;
  const uint16_t *base = p.q + b * p.qs[0] + h * p.qs[1];
  float x[UPT][16];
  float amax = 0.f;
#pragma unroll
  for (int i = 0; i < UPT; ++i) {
    const int u = i * 256 + threadIdx.x, r = u / UPR, c16 = u % UPR, n = qb * kBQ + r;
    if (n < p.Nq) {
      const uint4 *src = (const uint4 *)(base + (int64_t)n * p.qs[2] + c16 * 16);
      unpack8(src[0], x[i]);
      unpack8(src[1], x[i] + 8);
    } else {
#pragma unroll
      for (int e = 0; e < 16; ++e) x[i][e] = 0.f;
    }
#pragma unroll
    for (int e = 0; e < 16; ++e) amax = fmaxf(amax, fabsf(x[i][e]));
  }
  amax = block_max_nonneg(amax, red);
  const float inv = amax > 0.f ? 127.0f / amax : 0.f;
  if (threadIdx.x == 0) p.q_scale[bh * p.nqb + qb] = amax > 0.f ? amax / 127.0f : 0.f;
  int8_t *dst = p.q_codes + ((size_t)bh * p.nqb + qb) * kBQ * D;
#pragma unroll
  for (int i = 0; i < UPT; ++i) {
    const int u = i * 256 + threadIdx.x, r = u / UPR, c16 = u % UPR;
    uint4 w;
    w.x = pack_i8x4(x[i] + 0, inv);
    w.y = pack_i8x4(x[i] + 4, inv);
    w.z = pack_i8x4(x[i] + 8, inv);
    w.w = pack_i8x4(x[i] + 12, inv);
    *(uint4 *)(dst + i8_operand_offset<D>(r, c16)) = w;
  }
}

// ---- 4. K: smoothing, then per 64-row block INT8 -------------------------------
template <int D>
__device__ __forceinline__ void quant_k_block(const PrepParams &p, int j, int bh, float *red) {
  constexpr int UPR = D / 16, UPT = kBK * UPR / 256;
  const int b = bh / p.H, h = bh - b * p.H;
  const uint16_t *base = p.k + b * p.ks[0] + h * p.ks[1];
  const float *mean = p.k_mean + (size_t)bh * D;
  float x[UPT][16];
  float amax = 0.f;
#pragma unroll
  for (int i = 0; i < UPT; ++i) {
    const int u = i * 256 + threadIdx.x, r = u / UPR, c16 = u % UPR, n = j * kBK + r;
    if (n < p.Nkv) {
      const uint4 *src = (const uint4 *)(base + (int64_t)n * p.ks[2] + c16 * 16);
      unpack8(src[0], x[i]);
      unpack8(src[1], x[i] + 8);
#pragma unroll
      for (int e = 0; e < 16; ++e) x[i][e] = x[i][e] - mean[c16 * 16 + e];   // one FP32 rounding
    } else {
#pragma unroll
      for (int e = 0; e < 16; ++e) x[i][e] = 0.f;
    }
#pragma unroll
    for (int e = 0; e < 16; ++e) amax = fmaxf(amax, fabsf(x[i][e]));
  }
  amax = block_max_nonneg(amax, red);
  const float inv = amax > 0.f ? 127.0f / amax : 0.f;
  if (threadIdx.x == 0) p.k_scale[(size_t)bh * p.T + j] = amax > 0.f ? amax / 127.0f : 0.f;
  int8_t *dst = p.k_codes + ((size_t)bh * p.T + j) * kBK * D;
#pragma unroll
  for (int i = 0; i < UPT; ++i) {
    const int u = i * 256 + threadIdx.x, r = u / UPR, c16 = u % UPR;
    uint4 w;
    w.x = pack_i8x4(x[i] + 0, inv);
    w.y = pack_i8x4(x[i] + 4, inv);
    w.z = pack_i8x4(x[i] + 8, inv);
    w.w = pack_i8x4(x[i] + 12, inv);
    *(uint4 *)(dst + i8_operand_offset<D>(r, c16)) = w;
  }
}

// ---- 5. V: per-channel E4M3FN, written as the A operand of the PV product ------
// A 64-key tile is staged in LDS, then each thread gathers the 16 bytes of one
// (channel block, half, lane) unit: byte e holds key 32*half + 8*(e/4) +
// 4*(lane/32) + e%4 of channel 32*block + lane%32.
template <int D>
struct VTileSmem {
  uint16_t tile[kBK][D + 2];                 // +2 shifts rows across banks
};

template <int D>
__device__ __forceinline__ void quant_v_block(const PrepParams &p, int j, int bh, VTileSmem<D> &sm) {
  constexpr int UPR = D / 8;                 // 8-value loads per row
  constexpr int NUNIT = (D / 32) * 2 * 64;   // 16-byte output units per tile
  auto &tile = sm.tile;
  const int b = bh / p.H, h = bh - b * p.H;
  const uint16_t *base = p.v + b * p.vs[0] + h * p.vs[1];
  for (int u = threadIdx.x; u < kBK * UPR; u += 256) {
    const int r = u / UPR, c8 = u % UPR, n = j * kBK + r;
    uint4 w = make_uint4(0, 0, 0, 0);
    if (n < p.Nkv) w = *(const uint4 *)(base + (int64_t)n * p.vs[2] + c8 * 8);
    const uint32_t ww[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      tile[r][c8 * 8 + 2 * e] = (uint16_t)(ww[e] & 0xffffu);
      tile[r][c8 * 8 + 2 * e + 1] = (uint16_t)(ww[e] >> 16);
    }
  }
  __syncthreads();
  const float *vinv = p.ws_vinv + (size_t)bh * D;
  uint8_t *dst = p.v_codes + ((size_t)bh * p.T + j) * kBK * D;
  for (int u = threadIdx.x; u < NUNIT; u += 256) {
    const int blk = u >> 7, half = (u >> 6) & 1, lane = u & 63;
    const int ch = 32 * blk + (lane & 31);
    const float inv = vinv[ch];
    uint32_t w[4];
#pragma unroll
    for (int d4 = 0; d4 < 4; ++d4) {
      float f[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int key = 32 * half + 8 * d4 + 4 * (lane >> 5) + e;
        f[e] = bf16f(tile[key][ch]) * inv;
      }
      int x = __builtin_amdgcn_cvt_pk_fp8_f32(f[0], f[1], 0, false);
      x = __builtin_amdgcn_cvt_pk_fp8_f32(f[2], f[3], x, true);
      w[d4] = (uint32_t)x;
    }
    *(uint4 *)(dst + (size_t)u * 16) = make_uint4(w[0], w[1], w[2], w[3]);
  }
}

// ---- launches: [stats | Q quant] -> finalize -> [K quant | V quant] ------------
// Q quantization does not depend on the statistics, so it shares the first
// launch; K and V quantization share the last one.
template <int D>
__global__ __launch_bounds__(256) void k_prep_pass1(PrepParams p) {
  __shared__ StatsSmem<D> sm;
  const int bh = blockIdx.y;
  if ((int)blockIdx.x < p.nchunk) prep_stats_block<D>(p, blockIdx.x, bh, sm);
  else quant_q_block<D>(p, blockIdx.x - p.nchunk, bh, (float *)&sm);
}

template <int D>
__global__ __launch_bounds__(256) void k_prep_pass2(PrepParams p) {
  __shared__ VTileSmem<D> sm;
  const int bh = blockIdx.y;
  if ((int)blockIdx.x < p.T) quant_k_block<D>(p, blockIdx.x, bh, (float *)&sm);
  else quant_v_block<D>(p, blockIdx.x - p.T, bh, sm);
}

template <int D>
static hipError_t launch_prep_d(const PrepParams &p, hipStream_t st) {
  const int BH = p.B * p.H;
  hipLaunchKernelGGL(k_prep_pass1<D>, dim3(p.nchunk + p.nqb, BH), dim3(256), 0, st, p);
  hipLaunchKernelGGL(k_prep_finalize<D>, dim3(BH), dim3(256), 0, st, p);
  hipLaunchKernelGGL(k_prep_pass2<D>, dim3(2 * p.T, BH), dim3(256), 0, st, p);
  return hipGetLastError();
}

hipError_t launch_prep(const PrepParams &p, hipStream_t stream) {
  return p.D == 128 ? launch_prep_d<128>(p, stream) : launch_prep_d<64>(p, stream);
}

}  // namespace sage
