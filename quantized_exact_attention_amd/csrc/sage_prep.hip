// Prep stage for gfx950: K/V column statistics, K smoothing, per-block INT8
// Q/K and per-channel FP8 (OCP E4M3FN) V, written in the operand order of the
// attention kernel's matrix instructions.  Stages "Q/K preparation, K
// smoothing, INT8 quantization, FP8 V" of the contract imported in
// "Experiment Log", Phase 0 Import And Verification.
//
// Every kernel here is an HBM-bound stream: 16-byte loads along the contiguous
// channel dimension, code stores of 8 (Q, K) or 16 (V) bytes in operand order.
// Two schedules: three launches ([statistics | Q] -> finalize -> [K, V per
// tile]), which read K and V twice, and a single pass that reads them once
// (sections 1-4 and 5 below).
#include "sage_common.h"

namespace sage {

// Max of a non-negative float over the 256-thread block (bit order == value order).
// RACE: the race-gate build (pauses before the LDS write and read).
template <bool RACE = false>
__device__ __forceinline__ float block_max_nonneg(float x, float *red, uint32_t seed = 0) {
  uint32_t u = __float_as_uint(x);
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) u = max(u, (uint32_t)__shfl_xor((int)u, o, 64));
  const int w = threadIdx.x >> 6;
  __syncthreads();
  if (RACE) race_pause(seed, 10, 0);
  if ((threadIdx.x & 63) == 0) red[w] = __uint_as_float(u);
  __syncthreads();
  if (RACE) race_pause(seed, 11, 0);
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

// ---- 1. per (b,h, key chunk): FP64 column sums of K (exact for bf16 data) and
//         column max |V|; partials go to the workspace --------------------------
// Thread (cg, tl) reads the 8-channel group cg of rows n0 + tl + TL*i; the loads
// of kBatch rows are issued before any is used, so each thread keeps 2*kBatch
// 16-byte loads in flight.
template <int D>
struct StatsSmem {
  static constexpr int CG = D / 8;      // 8-channel groups of one row
  static constexpr int TL = 256 / CG;   // rows handled in parallel
  double sum[TL][D];
  float max[TL][D];
};

constexpr int kBatch = 8;

template <int D, bool RACE>
__device__ __forceinline__ void prep_stats_block(const PrepParams &p, int chunk, int bh, StatsSmem<D> &sm) {
  constexpr int CG = StatsSmem<D>::CG, TL = StatsSmem<D>::TL, RPT = kStatChunk / TL;
  static_assert(RPT % kBatch == 0, "rows per thread must be a multiple of the load batch");
  auto &s_sum = sm.sum;
  auto &s_max = sm.max;
  const int b = bh / p.H, h = bh - b * p.H;
  const int cg = threadIdx.x % CG, tl = threadIdx.x / CG;
  const int n0 = chunk * kStatChunk + tl;
  const uint16_t *kb = p.k + b * p.ks[0] + h * p.ks[1] + cg * 8;
  const uint16_t *vb = p.v + b * p.vs[0] + h * p.vs[1] + cg * 8;
  double acc[8];
  float vmx[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) { acc[e] = 0.0; vmx[e] = 0.f; }
#pragma unroll
  for (int i0 = 0; i0 < RPT; i0 += kBatch) {
    uint4 kr[kBatch], vr[kBatch];
#pragma unroll
    for (int i = 0; i < kBatch; ++i) {
      const int n = n0 + (i0 + i) * TL;
      kr[i] = vr[i] = make_uint4(0, 0, 0, 0);    // rows past Nkv add 0 and max 0
      if (n < p.Nkv) {
        kr[i] = *(const uint4 *)(kb + (int64_t)n * p.ks[2]);
        vr[i] = *(const uint4 *)(vb + (int64_t)n * p.vs[2]);
      }
    }
#pragma unroll
    for (int i = 0; i < kBatch; ++i) {
      float kf[8], vf[8];
      unpack8(kr[i], kf);
      unpack8(vr[i], vf);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        acc[e] += (double)kf[e];
        vmx[e] = fmaxf(vmx[e], fabsf(vf[e]));
      }
    }
  }
  if (RACE) race_pause(p.race_seed, 0, chunk);
#pragma unroll
  for (int e = 0; e < 8; ++e) { s_sum[tl][cg * 8 + e] = acc[e]; s_max[tl][cg * 8 + e] = vmx[e]; }
  __syncthreads();
  if (RACE) race_pause(p.race_seed, 1, chunk);
  for (int c = threadIdx.x; c < D; c += 256) {
    double s = 0.0;
    float mx = 0.f;
    for (int i = 0; i < TL; ++i) { s += s_sum[i][c]; mx = fmaxf(mx, s_max[i][c]); }
    const size_t o = ((size_t)bh * p.nchunk + chunk) * D + c;
    p.ws_ksum[o] = s;
    p.ws_vmax[o] = mx;
  }
}

// ---- 2. per (b,h, 16 channels): K mean, V channel scale and inverse ------------
// 256 threads: channel 16*blockIdx.y + t % 16, chunk group t / 16; the partial
// sums are exact, so their order does not matter.
template <int D, bool RACE>
__global__ __launch_bounds__(256) void k_prep_finalize(PrepParams p) {
  constexpr int NG = 16, U = 4;
  __shared__ double s_sum[NG][16];
  __shared__ float s_max[NG][16];
  const int bh = blockIdx.x, cl = threadIdx.x % 16, g = threadIdx.x / 16, c = blockIdx.y * 16 + cl;
  double s = 0.0;
  float mx = 0.f;
  for (int i0 = g; i0 < p.nchunk; i0 += NG * U) {
    double ps[U];
    float pm[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int i = i0 + u * NG;
      ps[u] = 0.0;
      pm[u] = 0.f;
      if (i < p.nchunk) {
        const size_t o = ((size_t)bh * p.nchunk + i) * D + c;
        ps[u] = p.ws_ksum[o];
        pm[u] = p.ws_vmax[o];
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) { s += ps[u]; mx = fmaxf(mx, pm[u]); }
  }
  if (RACE) race_pause(p.race_seed, 2, 0);
  s_sum[g][cl] = s;
  s_max[g][cl] = mx;
  __syncthreads();
  if (RACE) race_pause(p.race_seed, 3, 0);
  if (g == 0) {
#pragma unroll
    for (int i = 1; i < NG; ++i) { s += s_sum[i][cl]; mx = fmaxf(mx, s_max[i][cl]); }
    p.k_mean[bh * D + c] = (float)(s / (double)p.Nkv);   // FP64 quotient, one FP32 rounding
    p.v_scale[bh * D + c] = mx > 0.f ? mx / 448.0f : 0.f;  // correctly rounded FP32 divides
    p.ws_vinv[bh * D + c] = mx > 0.f ? 448.0f / mx : 0.f;
  }
}

// ---- 3. INT8 block quantization of R rows (Q: 128, smoothed K: 64) ------------
// Thread t owns the 8-channel units t + 256 i: row (t + 256 i) / (D/8), channels
// 8 * (t % (D/8)) (the same for every i, since 256 is a multiple of D/8), so a
// wave reads whole rows.  The raw bf16 words stay in registers and are unpacked
// again for the codes; each unit becomes 8 bytes of a 16-byte operand unit.
template <int D, int R, bool SMOOTH, bool RACE = false>
__device__ __forceinline__ void quant_i8_rows(const uint16_t *base, int64_t rs, int nvalid, const float *mean,
                                              int8_t *dst, float *scale_out, float *red, uint32_t seed = 0) {
  constexpr int UPR = D / 8, UPT = R * UPR / 256;
  static_assert(256 % UPR == 0 && UPT >= 1, "unit mapping");
  const int c8 = threadIdx.x % UPR, r0 = threadIdx.x / UPR;
  uint4 raw[UPT];
#pragma unroll
  for (int i = 0; i < UPT; ++i) {
    const int r = r0 + i * (256 / UPR);
    raw[i] = make_uint4(0, 0, 0, 0);             // pad rows are 0 and do not raise the max
    if (r < nvalid) raw[i] = *(const uint4 *)(base + (int64_t)r * rs + c8 * 8);
  }
  float mu[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) mu[e] = SMOOTH ? mean[c8 * 8 + e] : 0.f;
  auto values = [&](int i, float *f) {
    unpack8(raw[i], f);
    if (SMOOTH && r0 + i * (256 / UPR) < nvalid) {
#pragma unroll
      for (int e = 0; e < 8; ++e) f[e] = f[e] - mu[e];   // one FP32 rounding
    }
  };
  float amax = 0.f;
#pragma unroll
  for (int i = 0; i < UPT; ++i) {
    float f[8];
    values(i, f);
#pragma unroll
    for (int e = 0; e < 8; ++e) amax = fmaxf(amax, fabsf(f[e]));
  }
  amax = block_max_nonneg<RACE>(amax, red, seed);
  const float inv = amax > 0.f ? 127.0f / amax : 0.f;
  if (threadIdx.x == 0) *scale_out = amax > 0.f ? amax / 127.0f : 0.f;
#pragma unroll
  for (int i = 0; i < UPT; ++i) {
    float f[8];
    values(i, f);
    const int r = r0 + i * (256 / UPR);
    uint2 w;
    w.x = pack_i8x4(f, inv);
    w.y = pack_i8x4(f + 4, inv);
    *(uint2 *)(dst + i8_operand_offset<D>(r, c8 >> 1) + (c8 & 1) * 8) = w;
  }
}

template <int D, bool RACE = false>
__device__ __forceinline__ void quant_q_block(const PrepParams &p, int qb, int bh, float *red) {
  const int b = bh / p.H, h = bh - b * p.H;
  const uint16_t *base = p.q + b * p.qs[0] + h * p.qs[1] + (int64_t)qb * kBQ * p.qs[2];
  quant_i8_rows<D, kBQ, false, RACE>(base, p.qs[2], min(kBQ, p.Nq - qb * kBQ), nullptr,
                                     p.q_codes + ((size_t)bh * p.nqb + qb) * kBQ * D, p.q_scale + bh * p.nqb + qb,
                                     red, p.race_seed);
}

// ---- 4. one 64-key tile: K smoothing + per-tile INT8, and per-channel E4M3FN V -
// written as the A operands of the two products.  Both tiles' loads are issued
// first.  V is staged in LDS, then each thread gathers the 16 bytes of one
// (channel block, half, lane) unit: byte e holds key 32*half + 8*(e/4) +
// 4*(lane/32) + e%4 of channel 32*block + lane%32.
template <int D>
struct KVTileSmem {
  uint16_t tile[kBK][D + 8];                 // 16-byte aligned rows, +8 shifts rows across banks
  float red[4];
};

template <int D, bool RACE>
__device__ __forceinline__ void quant_kv_tile(const PrepParams &p, int j, int bh, KVTileSmem<D> &sm) {
  constexpr int VU = D / 8, VUPT = kBK * VU / 256;    // V: 8-channel loads per thread
  constexpr int NUNIT = (D / 32) * 2 * 64;            // 16-byte V output units per tile
  const int b = bh / p.H, h = bh - b * p.H;
  const int nvalid = min(kBK, p.Nkv - j * kBK);
  const uint16_t *vbase = p.v + b * p.vs[0] + h * p.vs[1] + (int64_t)j * kBK * p.vs[2];
  uint4 vraw[VUPT];
#pragma unroll
  for (int i = 0; i < VUPT; ++i) {
    const int u = i * 256 + threadIdx.x, r = u / VU, c8 = u % VU;
    vraw[i] = make_uint4(0, 0, 0, 0);
    if (r < nvalid) vraw[i] = *(const uint4 *)(vbase + (int64_t)r * p.vs[2] + c8 * 8);
  }
  if (RACE) race_pause(p.race_seed, 4, j);
#pragma unroll
  for (int i = 0; i < VUPT; ++i) {
    const int u = i * 256 + threadIdx.x, r = u / VU, c8 = u % VU;
    *(uint4 *)&sm.tile[r][c8 * 8] = vraw[i];
  }

  // K: ks = fp32(K - mean), then the tile's INT8 scale and codes; the barriers of
  // its block maximum also publish the V tile in LDS.
  quant_i8_rows<D, kBK, true, RACE>(p.k + b * p.ks[0] + h * p.ks[1] + (int64_t)j * kBK * p.ks[2], p.ks[2],
                                    nvalid, p.k_mean + (size_t)bh * D, p.k_codes + ((size_t)bh * p.T + j) * kBK * D,
                                    p.k_scale + (size_t)bh * p.T + j, sm.red, p.race_seed);
  if (RACE) race_pause(p.race_seed, 5, j);

  // V: code = E4M3FN_RNE(fp32(v * vinv_c)).
  const float *vinv = p.ws_vinv + (size_t)bh * D;
  uint8_t *vdst = p.v_codes + ((size_t)bh * p.T + j) * kBK * D;
#pragma unroll
  for (int u = threadIdx.x; u < NUNIT; u += 256) {
    const int blk = u >> 7, half = (u >> 6) & 1, lane = u & 63;
    const int ch = 32 * blk + (lane & 31);
    const float vi = vinv[ch];
    uint32_t w[4];
#pragma unroll
    for (int d4 = 0; d4 < 4; ++d4) {
      float f[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int key = 32 * half + 8 * d4 + 4 * (lane >> 5) + e;
        f[e] = bf16f(sm.tile[key][ch]) * vi;
      }
      int xw = __builtin_amdgcn_cvt_pk_fp8_f32(f[0], f[1], 0, false);
      xw = __builtin_amdgcn_cvt_pk_fp8_f32(f[2], f[3], xw, true);
      w[d4] = (uint32_t)xw;
    }
    *(uint4 *)(vdst + (size_t)u * 16) = make_uint4(w[0], w[1], w[2], w[3]);
  }
}

// ---- 5. single pass: K and V read from HBM once -------------------------------
// Workgroup (b,h, g) keeps rows [g*R, g*R + R) of K and V in registers, adds
// its column sums and maxima into the head's accumulators (atomics: the sums
// are exact, so their order does not matter) and counts itself in; the last
// workgroup of the head turns the totals into the K mean, V scale and inverse
// and raises the head's flag; every workgroup of the head waits for the flag, then quantizes its
// rows; the head's Q blocks follow its groups in the grid.  Workgroups are
// dispatched in index order and a head needs at most kFusedMaxGroups of them,
// far fewer than fit on the device at once, so the workgroups of a head are
// all resident before any waits for long; the wait is still bounded, and on
// expiry the status word records it and the workgroup goes on.
constexpr unsigned kSpinLimit = 1u << 19;   // x ~0.25 us of s_sleep: ~0.1 s

// Data shared between the workgroups of a head (partials, K mean, V inverse)
// is written and read with agent-scope atomic accesses, which go to the
// device-coherent level instead of an XCD's own L2, so no L2 write-back or
// invalidation is needed.  A store is ordered before the arrival count or the
// ready flag by waiting until every store of the workgroup has completed.
template <typename T>
__device__ __forceinline__ void coherent_store(T *ptr, T v) {
  __hip_atomic_store(ptr, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
template <typename T>
__device__ __forceinline__ T coherent_load(const T *ptr) {
  return __hip_atomic_load(ptr, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void completed_barrier() {
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // this wave's stores have completed
  __syncthreads();
}

template <int D>
struct FusedSmem {
  static constexpr int CG = D / 8, TL = 256 / CG;
  union {
    struct {
      double sum[TL][D];
      float max[TL][D];
    } st;
    uint16_t tile[kBK][D + 8];
  } u;
  float red[kFusedRows(D) / kBK][4];
  int last;
  int expired;                    // this group's wait for the head's statistics ran out
};

template <int D>
__device__ __forceinline__ void fused_kv_group(const PrepParams &p, int bh, int g, FusedSmem<D> &sm) {
  constexpr int CG = D / 8, TL = 256 / CG, RPT = 16, R = TL * RPT, TPW = R / kBK, RPTT = kBK / TL;
  constexpr int NUNIT = (D / 32) * 2 * 64;
  const int tid = threadIdx.x;
  const int b = bh / p.H, h = bh - b * p.H;
  const int cg = tid % CG, tl = tid / CG;
  const int n0 = g * R + tl;
  const uint16_t *kb = p.k + b * p.ks[0] + h * p.ks[1] + cg * 8;
  const uint16_t *vb = p.v + b * p.vs[0] + h * p.vs[1] + cg * 8;
  uint4 kr[RPT], vr[RPT];
#pragma unroll
  for (int i = 0; i < RPT; ++i) {
    const int n = n0 + i * TL;
    kr[i] = vr[i] = make_uint4(0, 0, 0, 0);    // rows past Nkv add 0 and max 0
    if (n < p.Nkv) {
      kr[i] = *(const uint4 *)(kb + (int64_t)n * p.ks[2]);
      vr[i] = *(const uint4 *)(vb + (int64_t)n * p.vs[2]);
    }
  }

  // ---- column partials of this group ----
  {
    double acc[8];
    float vmx[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) { acc[e] = 0.0; vmx[e] = 0.f; }
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
      float kf[8], vf[8];
      unpack8(kr[i], kf);
      unpack8(vr[i], vf);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        acc[e] += (double)kf[e];
        vmx[e] = fmaxf(vmx[e], fabsf(vf[e]));
      }
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) { sm.u.st.sum[tl][cg * 8 + e] = acc[e]; sm.u.st.max[tl][cg * 8 + e] = vmx[e]; }
  }
  __syncthreads();
  for (int c = tid; c < D; c += 256) {
    double s = 0.0;
    float mx = 0.f;
    for (int i = 0; i < TL; ++i) { s += sm.u.st.sum[i][c]; mx = fmaxf(mx, sm.u.st.max[i][c]); }
    // exact partial sums: the atomic additions give the exact total in any order
    __hip_atomic_fetch_add(p.ws_asum + (size_t)bh * D + c, s, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_fetch_max(p.ws_amax + (size_t)bh * D + c, __float_as_uint(mx), __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);   // max |v| >= 0: bit order is value order
  }
  completed_barrier();                           // every update of the group has completed
  uint32_t *arrived = p.ws_sync + bh, *ready = p.ws_sync + p.B * p.H + bh, *status = p.ws_sync + 2 * p.B * p.H;
  if (tid == 0)
    sm.last = __hip_atomic_fetch_add(arrived, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == (unsigned)(p.G - 1);
  __syncthreads();

  // ---- the last group of the head: K mean, V scale and inverse ----
  if (sm.last) {
    for (int c = tid; c < D; c += 256) {
      const double s = coherent_load(p.ws_asum + (size_t)bh * D + c);
      const float mx = __uint_as_float(coherent_load(p.ws_amax + (size_t)bh * D + c));
      coherent_store(p.k_mean + bh * D + c, (float)(s / (double)p.Nkv));   // FP64 quotient, one rounding
      p.v_scale[bh * D + c] = mx > 0.f ? mx / 448.0f : 0.f;
      coherent_store(p.ws_vinv + bh * D + c, mx > 0.f ? 448.0f / mx : 0.f);
    }
    completed_barrier();
    if (tid == 0) __hip_atomic_store(ready, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  // Ordering: the head's statistics were written with agent-scope (coherent)
  // stores that had completed before the flag was stored, and the loads below
  // are coherent too and are issued only after the flag load has returned, so
  // they observe those stores.  (Acquire/release fences would add L2
  // write-back and invalidation on every workgroup, which measured 120 us on
  // the long video workload.)
  if (tid == 0) {
    unsigned it = 0;
    sm.expired = 0;
    while (__hip_atomic_load(ready, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == 0u) {
      if (++it > kSpinLimit) {
        __hip_atomic_store(status, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        sm.expired = 1;
        break;
      }
      __builtin_amdgcn_s_sleep(8);
    }
  }
  __syncthreads();

  // ---- K: smoothing and per-tile INT8 ----
  float mu[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) mu[e] = coherent_load(p.k_mean + bh * D + cg * 8 + e);
  auto kvals = [&](int i, float *f) {
    unpack8(kr[i], f);
    if (n0 + i * TL < p.Nkv) {
#pragma unroll
      for (int e = 0; e < 8; ++e) f[e] = f[e] - mu[e];   // one FP32 rounding
    }
  };
  {
    uint32_t am[TPW];
#pragma unroll
    for (int q = 0; q < TPW; ++q) {
      float a = 0.f;
#pragma unroll
      for (int i = q * RPTT; i < (q + 1) * RPTT; ++i) {
        float f[8];
        kvals(i, f);
#pragma unroll
        for (int e = 0; e < 8; ++e) a = fmaxf(a, fabsf(f[e]));
      }
      am[q] = __float_as_uint(a);
#pragma unroll
      for (int o = 32; o >= 1; o >>= 1) am[q] = max(am[q], (uint32_t)__shfl_xor((int)am[q], o, 64));
    }
    if ((tid & 63) == 0) {
#pragma unroll
      for (int q = 0; q < TPW; ++q) sm.red[q][tid >> 6] = __uint_as_float(am[q]);
    }
  }
  __syncthreads();
#pragma unroll
  for (int q = 0; q < TPW; ++q) {
    const int j = g * TPW + q;                   // tile index in the head
    if (j >= p.T) break;
    const float amax = fmaxf(fmaxf(sm.red[q][0], sm.red[q][1]), fmaxf(sm.red[q][2], sm.red[q][3]));
    const float inv = amax > 0.f ? 127.0f / amax : 0.f;
    // a group whose wait ran out writes NaN scales for its tiles: every output
    // row of the head then comes out NaN instead of silently wrong
    if (tid == 0) p.k_scale[(size_t)bh * p.T + j] = sm.expired ? __builtin_nanf("") : amax > 0.f ? amax / 127.0f : 0.f;
    int8_t *kdst = p.k_codes + ((size_t)bh * p.T + j) * kBK * D;
#pragma unroll
    for (int i = q * RPTT; i < (q + 1) * RPTT; ++i) {
      float f[8];
      kvals(i, f);
      const int r = tl + (i - q * RPTT) * TL;
      uint2 w;
      w.x = pack_i8x4(f, inv);
      w.y = pack_i8x4(f + 4, inv);
      *(uint2 *)(kdst + i8_operand_offset<D>(r, cg >> 1) + (cg & 1) * 8) = w;
    }
  }

  // ---- V: per-channel E4M3FN, one tile at a time through LDS ----
  const float *vinv = p.ws_vinv + (size_t)bh * D;
#pragma unroll
  for (int q = 0; q < TPW; ++q) {
    const int j = g * TPW + q;
    if (j >= p.T) break;
#pragma unroll
    for (int i = q * RPTT; i < (q + 1) * RPTT; ++i) *(uint4 *)&sm.u.tile[tl + (i - q * RPTT) * TL][cg * 8] = vr[i];
    __syncthreads();
    uint8_t *vdst = p.v_codes + ((size_t)bh * p.T + j) * kBK * D;
#pragma unroll
    for (int uu = tid; uu < NUNIT; uu += 256) {
      const int blk = uu >> 7, half = (uu >> 6) & 1, lane = uu & 63;
      const int ch = 32 * blk + (lane & 31);
      const float vi = coherent_load(vinv + ch);
      uint32_t w[4];
#pragma unroll
      for (int d4 = 0; d4 < 4; ++d4) {
        float f[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int key = 32 * half + 8 * d4 + 4 * (lane >> 5) + e;
          f[e] = bf16f(sm.u.tile[key][ch]) * vi;
        }
        int xw = __builtin_amdgcn_cvt_pk_fp8_f32(f[0], f[1], 0, false);
        xw = __builtin_amdgcn_cvt_pk_fp8_f32(f[2], f[3], xw, true);
        w[d4] = (uint32_t)xw;
      }
      *(uint4 *)(vdst + (size_t)uu * 16) = make_uint4(w[0], w[1], w[2], w[3]);
    }
    __syncthreads();
  }
}

// Workgroup order, head by head: the head's G K/V groups, then its Q blocks,
// whose loads keep memory busy while the head's groups wait for each other.
template <int D>
__global__ __launch_bounds__(256) void k_prep_fused(PrepParams p) {
  __shared__ FusedSmem<D> sm;
  const int per = p.G + (p.kv_only ? 0 : p.nqb);
  const int bh = blockIdx.x / per, r = blockIdx.x - bh * per;
  if (r < p.G) fused_kv_group<D>(p, bh, r, sm);
  else quant_q_block<D>(p, r - p.G, bh, &sm.red[0][0]);
}

// Zero the arrival counters, ready flags and status word of the single pass.
__global__ __launch_bounds__(256) void k_prep_clear(uint32_t *w, int n) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i < n) w[i] = 0u;
}

// ---- launches: [stats | Q quant] -> finalize -> [K and V quant per tile] --------
// Q quantization does not depend on the statistics, so it shares the first
// launch; one workgroup of the last launch quantizes the K and V rows of a tile.
template <int D, bool RACE>
__global__ __launch_bounds__(256) void k_prep_pass1(PrepParams p) {
  __shared__ StatsSmem<D> sm;
  const int bh = blockIdx.y;
  if ((int)blockIdx.x < p.nchunk) prep_stats_block<D, RACE>(p, blockIdx.x, bh, sm);
  else quant_q_block<D, RACE>(p, blockIdx.x - p.nchunk, bh, (float *)&sm);
}

template <int D, bool RACE>
__global__ __launch_bounds__(256) void k_prep_pass2(PrepParams p) {
  __shared__ KVTileSmem<D> sm;
  quant_kv_tile<D, RACE>(p, blockIdx.x, blockIdx.y, sm);
}

template <int D>
static hipError_t launch_prep_d(const PrepParams &p, hipStream_t st) {
  const int BH = p.B * p.H;
  if (p.G > 0) {
    const int nsync = (int)ws_sync_words(BH, D);
    hipLaunchKernelGGL(k_prep_clear, dim3((nsync + 255) / 256), dim3(256), 0, st, p.ws_sync, nsync);
    hipLaunchKernelGGL(k_prep_fused<D>, dim3(BH * (p.G + (p.kv_only ? 0 : p.nqb))), dim3(256), 0, st, p);
    return hipGetLastError();
  }
  if (p.race_seed) {
    hipLaunchKernelGGL((k_prep_pass1<D, true>), dim3(p.nchunk + p.nqb, BH), dim3(256), 0, st, p);
    hipLaunchKernelGGL((k_prep_finalize<D, true>), dim3(BH, D / 16), dim3(256), 0, st, p);
    hipLaunchKernelGGL((k_prep_pass2<D, true>), dim3(p.T, BH), dim3(256), 0, st, p);
    return hipGetLastError();
  }
  hipLaunchKernelGGL((k_prep_pass1<D, false>), dim3(p.nchunk + (p.kv_only ? 0 : p.nqb), BH), dim3(256), 0, st,
                     p);
  hipLaunchKernelGGL((k_prep_finalize<D, false>), dim3(BH, D / 16), dim3(256), 0, st, p);
  hipLaunchKernelGGL((k_prep_pass2<D, false>), dim3(p.T, BH), dim3(256), 0, st, p);
  return hipGetLastError();
}

hipError_t launch_prep(const PrepParams &p, hipStream_t stream) {
  return p.D == 128 ? launch_prep_d<128>(p, stream) : launch_prep_d<64>(p, stream);
}

}  // namespace sage
