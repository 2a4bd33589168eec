// Shared definitions of the gfx950 HIP path (kernels and host launchers).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sage {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef float v16f __attribute__((ext_vector_type(16)));

// Block sizes of the contract: Q quantization block / workgroup query tile,
// and the K quantization block == online-softmax KV tile (two 8 KiB K/V slots
// of 64 one-byte rows at D = 128, "Experiment Log", Phase 2A capability decision).
constexpr int kBQ = 128;
constexpr int kBK = 64;
constexpr int kStatChunk = 256;   // keys per block of the K/V statistics pass

struct PrepParams {
  const uint16_t *q, *k, *v;      // bf16 bits
  int64_t qs[3], ks[3], vs[3];    // element strides (b, h, n)
  int B, H, Nq, Nkv, D;
  int nqb, T, nchunk;
  int8_t *q_codes;
  float *q_scale;
  int8_t *k_codes;
  float *k_scale;
  uint8_t *v_codes;
  float *v_scale;
  float *k_mean;
  double *ws_ksum;                // [B*H][nchunk][D]
  float *ws_vmax;                 // [B*H][nchunk][D]
  float *ws_vinv;                 // [B*H][D]
  uint32_t *ws_sync;              // single-pass path: [B*H] arrivals, [B*H] ready flags, 1 status word
  double *ws_asum;                // single-pass path: [B*H][D] K column sums (atomic, exact)
  uint32_t *ws_amax;              // single-pass path: [B*H][D] V column max |v| (float bits, atomic max)
  int G;                          // single-pass path: K/V workgroups per (b,h); 0 selects three launches
  int kv_only;                    // three launches without the Q blocks (q, q_codes, q_scale unused)
  uint32_t race_seed;             // nonzero: the race-gate build of the three launches (tests only)
};

struct FwdParams {
  const int8_t *q_codes;
  const float *q_scale;
  const int8_t *k_codes;
  const float *k_scale;
  const uint8_t *v_codes;
  const float *v_scale;
  uint16_t *out;                  // bf16 bits
  int64_t os[3];
  int H, Nq, Nkv, nqb, T;
  int n_units;                    // B*H*nqb
  float sl2;                      // fp32(sm_scale * fp32(log2 e))
  // capture build only
  const int32_t *units;
  int32_t *s_cap;
  uint8_t *p8_cap;
  float *md_cap;                  // [unit][128][T][3]: m, 448*d, alpha after tile j
  float *part_cap;                // [unit][128][T][D]: fresh PV partial of tile j
  float *ro_cap;                  // [unit][128][T][D]: RO after tile j
  float *r_cap;                   // [unit][128]: reciprocal of 448*d
  uint32_t race_seed;             // race-gate build only
  // Q-quantizing build only: bf16 Q and its element strides (b, h, n); q_codes
  // and q_scale are not read
  const uint16_t *q;
  int64_t qs[3];
};

__device__ __forceinline__ float bf16f(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

// Eight bf16 values (16 bytes, element order) as float32 (exact).
__device__ __forceinline__ void unpack8(const uint4 &x, float *f) {
  const uint32_t w[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f[2 * i] = __uint_as_float(w[i] << 16);
    f[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
  }
}

// Four INT8 codes, byte e = clamp(RNE(fp32(x[e] * inv)), -127, 127): the
// quantization rule of Q and K blocks (inv = fp32(127 / absmax)).
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

// Race gate (test builds only).  A wave-uniform pseudo-random pause of 0, 64,
// 256 or 1024 cycles, drawn from (seed, workgroup, wave, site, step), placed
// before the LDS writes and reads (and the HBM -> LDS copies) of a kernel: with
// correct synchronisation the results cannot depend on the order in which
// waves reach them, so a race-gate run must give the normal build's bits.
__device__ __forceinline__ void race_pause(uint32_t seed, uint32_t site, uint32_t step) {
  uint32_t h = seed ^ (blockIdx.x * 0x9E3779B1u) ^ (blockIdx.y * 0x85EBCA77u) ^ ((threadIdx.x >> 6) * 0xC2B2AE3Du) ^
               (site * 0x27D4EB2Fu) ^ (step * 0x165667B1u);
  h ^= h >> 15;
  h *= 0x2C1B3C6Du;
  h ^= h >> 12;
  h *= 0x297A2D39u;
  h ^= h >> 15;
  switch (__builtin_amdgcn_readfirstlane(h) & 3u) {
    case 1: __builtin_amdgcn_s_sleep(1); break;
    case 2: __builtin_amdgcn_s_sleep(4); break;
    case 3: __builtin_amdgcn_s_sleep(16); break;
    default: break;
  }
}

// Workspace layout of the prep statistics, shared by the size query and the launcher.
inline size_t ws_ksum_bytes(int BH, int nchunk, int D) { return (size_t)BH * nchunk * D * sizeof(double); }
inline size_t ws_vmax_bytes(int BH, int nchunk, int D) { return (size_t)BH * nchunk * D * sizeof(float); }
inline size_t ws_vinv_bytes(int BH, int D) { return (size_t)BH * D * sizeof(float); }
// Single-pass region, cleared as 32-bit words before every single-pass call:
// arrivals, ready flags, status word, then (8-byte aligned) the column sums and
// column maxima.
inline size_t ws_sync_head_words(int BH) { return ((size_t)2 * BH + 2) & ~(size_t)1; }
inline size_t ws_sync_words(int BH, int D) { return ws_sync_head_words(BH) + (size_t)BH * D * 3; }
inline size_t ws_sync_bytes(int BH, int D) { return ws_sync_words(BH, D) * sizeof(uint32_t); }

// Single-pass prep: one workgroup holds kFusedRows(D) K and V rows in registers
// (16 per thread); used while a head needs at most kFusedMaxGroups workgroups.
constexpr int kFusedRows(int D) { return 16 * (256 / (D / 8)); }
constexpr int kFusedMaxGroups = 256;
inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

hipError_t launch_prep(const PrepParams &p, hipStream_t stream);
// Q blocks per workgroup of the paired forward schedule
constexpr int kPairedBlocks = 3;

// Forward builds: the default schedule, the capture build (checkpoints of the
// listed units), the race-gate build (p.race_seed nonzero), the paired schedule,
// and the build that quantizes each Q block itself from bf16 Q (p.q).
enum class FwdVariant { kDefault, kCapture, kRace, kPaired, kQuantizeQ };
hipError_t launch_fwd(const FwdParams &p, int D, int grid, FwdVariant variant, hipStream_t stream);

}  // namespace sage
