// C ABI of the gfx950 quantized attention library: argument validation (pure
// host code, before any HIP call), buffer sizing and kernel launches.
#include <atomic>
#include <climits>
#include <cmath>
#include <cstring>
#include <mutex>
#include <utility>

#include "../../include/sage_attn.h"
#include "sage_common.h"

using namespace sage;

namespace {

constexpr int kMaxDevices = 64;
std::atomic<int> g_device_ok[kMaxDevices];   // 0 unknown, 1 gfx950, -1 other

int ceil_div(int64_t a, int64_t b) { return (int)((a + b - 1) / b); }

// Workspace regions, each 256-byte aligned: K column partials, V column
// partials, V inverses, then the single-pass region (arrival counters [BH],
// ready flags [BH], the status word, then the column sums and maxima).
size_t ws_vmax_offset(int BH, int nchunk, int D) { return align256(ws_ksum_bytes(BH, nchunk, D)); }
size_t ws_vinv_offset(int BH, int nchunk, int D) {
  return ws_vmax_offset(BH, nchunk, D) + align256(ws_vmax_bytes(BH, nchunk, D));
}
size_t ws_sync_offset(int BH, int nchunk, int D) {
  return ws_vinv_offset(BH, nchunk, D) + align256(ws_vinv_bytes(BH, D));
}
size_t ws_total_bytes(int BH, int nchunk, int D) {
  return ws_sync_offset(BH, nchunk, D) + align256(ws_sync_bytes(BH, D));
}

int check_shape(const sage_shape_t *s) {
  if (!s) return SAGE_E_NULL;
  if (s->D != 64 && s->D != 128) return SAGE_E_HEADDIM;
  if (s->B < 1 || s->H < 1 || s->Nq < 1 || s->Nkv < 1) return SAGE_E_SHAPE;
  const int64_t BH = (int64_t)s->B * s->H;
  if (BH > 65535) return SAGE_E_SHAPE;                      // second grid dimension of the prep
  if ((int64_t)s->Nq > (1 << 28) || (int64_t)s->Nkv > (1 << 28)) return SAGE_E_SHAPE;
  if (BH * ceil_div(s->Nq, kBQ) > INT32_MAX / 2) return SAGE_E_SHAPE;
  return SAGE_OK;
}

bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

int check_strides(const int64_t st[3]) {
  for (int i = 0; i < 3; ++i)
    if (st[i] < 0 || (st[i] & 7) != 0) return SAGE_E_ALIGN;
  return SAGE_OK;
}

// bytes spanned by a strided bf16 tensor [B,H,N,D]
size_t span_bytes(const sage_shape_t *s, const int64_t st[3], int N) {
  return (size_t)(((int64_t)(s->B - 1) * st[0] + (int64_t)(s->H - 1) * st[1] +
                   (int64_t)(N - 1) * st[2] + s->D) * 2);
}

// true if no two elements of a strided [B,H,N,D] tensor (d contiguous) share an
// address: ordered by stride, every dimension of size > 1 steps past the span
// of the dimensions inside it.  Sufficient, and it holds for every packed
// layout and permutation of one (BHND, BNHD, ...).
bool rows_disjoint(const sage_shape_t *s, const int64_t st[3], int N) {
  int64_t size[3] = {s->B, s->H, N}, stride[3] = {st[0], st[1], st[2]};
  for (int i = 1; i < 3; ++i)                    // insertion sort by stride
    for (int j = i; j > 0 && stride[j] < stride[j - 1]; --j) {
      std::swap(stride[j], stride[j - 1]);
      std::swap(size[j], size[j - 1]);
    }
  int64_t span = s->D;
  for (int i = 0; i < 3; ++i) {
    if (size[i] == 1) continue;
    if (stride[i] < span) return false;
    span += stride[i] * (size[i] - 1);
  }
  return true;
}

bool overlap(const void *a, size_t na, const void *b, size_t nb) {
  const uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
  return x < y + nb && y < x + na;
}

size_t buffer_bytes(const sage_shape_t *s, int which) {
  const size_t BH = (size_t)s->B * s->H;
  const size_t nqb = ceil_div(s->Nq, kBQ), T = ceil_div(s->Nkv, kBK);
  const int nchunk = ceil_div(s->Nkv, kStatChunk);
  switch (which) {
    case SAGE_BUF_Q_CODES: return BH * nqb * kBQ * s->D;
    case SAGE_BUF_Q_SCALE: return BH * nqb * sizeof(float);
    case SAGE_BUF_K_CODES: return BH * T * kBK * s->D;
    case SAGE_BUF_K_SCALE: return BH * T * sizeof(float);
    case SAGE_BUF_V_CODES: return BH * T * kBK * s->D;
    case SAGE_BUF_V_SCALE: return BH * s->D * sizeof(float);
    case SAGE_BUF_K_MEAN: return BH * s->D * sizeof(float);
    case SAGE_BUF_WORKSPACE: return ws_total_bytes((int)BH, nchunk, s->D);
    default: return 0;
  }
}

// need_ws: the workspace pointer is required (every entry but the
// allocation-free prep, which ignores it); need_q: the Q codes and scale are
// required (every entry but the K/V-only prep and the Q-quantizing forward,
// which neither read nor write them)
int check_quant(const sage_quant_t *q, bool need_ws = true, bool need_q = true) {
  if (!q || (need_q && (!q->q_codes || !q->q_scale)) || !q->k_codes || !q->k_scale || !q->v_codes ||
      !q->v_scale || !q->k_mean || (need_ws && !q->workspace))
    return SAGE_E_NULL;
  if ((need_q && (!aligned16(q->q_codes) || ((uintptr_t)q->q_scale & 3))) || !aligned16(q->k_codes) ||
      !aligned16(q->v_codes) || (need_ws && !aligned16(q->workspace)) || ((uintptr_t)q->k_scale & 3) ||
      ((uintptr_t)q->v_scale & 3) || ((uintptr_t)q->k_mean & 3))
    return SAGE_E_ALIGN;
  return SAGE_OK;
}

// true if [p, p+n) overlaps any buffer of the quant set (a NULL buffer overlaps nothing)
bool overlaps_quant(const void *p, size_t n, const sage_quant_t *q, const sage_shape_t *s) {
  const void *bufs[SAGE_BUF_COUNT] = {q->q_codes, q->q_scale, q->k_codes, q->k_scale,
                                      q->v_codes, q->v_scale, q->k_mean, q->workspace};
  for (int i = 0; i < SAGE_BUF_COUNT; ++i)
    if (bufs[i] && overlap(p, n, bufs[i], buffer_bytes(s, i))) return true;
  return false;
}

// ---- static device scratch of the allocation-free prep entry ----------------
// One copy of the array per GPU, created with the library's code object and
// held until the process ends.  In host code `scratch` names a host-side
// stand-in, not device memory: its device address comes from
// hipGetSymbolAddress, taken once per device with that device current, and only
// that address is ever passed to kernels.
constexpr size_t kScratchBytes = (size_t)8 << 20;
__device__ __align__(256) static uint8_t scratch[kScratchBytes];
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices];

// Device address of the current device's scratch, looked up on the first call
// on that device.
int scratch_address(void **ptr) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return SAGE_E_DEVICE;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void *p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return SAGE_E_DEVICE;
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return SAGE_OK;
}

int device_ok() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return SAGE_E_DEVICE;
  return sage_device_check(dev);
}

float resolve_sl2(float sm_scale, int D) {
  const float sm = sm_scale > 0.f ? sm_scale : (float)(1.0 / std::sqrt((double)D));
  return sm * 1.44269504088896340736f;   // fp32(sm_scale * fp32(log2 e))
}

int fill_fwd(const sage_quant_t *q, const sage_shape_t *s, float sm_scale, void *out, const sage_strides_t *st,
             FwdParams *fp, bool need_q = true) {
  int r = check_shape(s);
  if (r) return r;
  if (!out || !st) return SAGE_E_NULL;
  if ((r = check_quant(q, false, need_q))) return r;      // the forward does not use the workspace
  if (!aligned16(out) || check_strides(st->o)) return SAGE_E_ALIGN;
  if (!std::isfinite(sm_scale)) return SAGE_E_ARG;
  if (!rows_disjoint(s, st->o, s->Nq) || overlaps_quant(out, span_bytes(s, st->o, s->Nq), q, s))
    return SAGE_E_ALIAS;
  std::memset(fp, 0, sizeof(*fp));
  fp->q_codes = q->q_codes;
  fp->q_scale = q->q_scale;
  fp->k_codes = q->k_codes;
  fp->k_scale = q->k_scale;
  fp->v_codes = q->v_codes;
  fp->v_scale = q->v_scale;
  fp->out = (uint16_t *)out;
  for (int i = 0; i < 3; ++i) fp->os[i] = st->o[i];
  fp->H = s->H;
  fp->Nq = s->Nq;
  fp->Nkv = s->Nkv;
  fp->nqb = ceil_div(s->Nq, kBQ);
  fp->T = ceil_div(s->Nkv, kBK);
  fp->n_units = s->B * s->H * fp->nqb;
  fp->sl2 = resolve_sl2(sm_scale, s->D);
  return SAGE_OK;
}

// Every workgroup records, from one lane: the shader-clock counter
// (s_memtime, kept per compute unit), the constant 100 MHz counter
// (s_memrealtime), the XCD id (HW_REG_XCC_ID) and the hardware id of its
// compute unit (HW_REG_HW_ID).  SAGE_CLOCK_SAMPLES workgroups cover every
// compute unit with high probability, so two samples can be matched unit by unit.
__global__ void k_clock_sample(uint64_t *dst) {
  if (threadIdx.x == 0) {
    uint64_t *d = dst + 4 * (size_t)blockIdx.x;
    d[0] = __builtin_amdgcn_s_memtime();
    d[1] = __builtin_amdgcn_s_memrealtime();
    d[2] = __builtin_amdgcn_s_getreg((15 << 11) | 20);   // HW_REG_XCC_ID
    d[3] = __builtin_amdgcn_s_getreg((31 << 11) | 4);    // HW_REG_HW_ID
  }
}

// Matrix-core peak sample: four independent accumulation chains of one
// matrix instruction per wave on register operands, so that each SIMD's matrix
// core is fed back to back (a dependent chain of one instruction would wait for
// its own result).  The operands are fixed non-NaN bit patterns; the values
// are irrelevant, the last lane words keep the work from being removed.
template <int KIND>
__global__ __launch_bounds__(256) void k_mfma_peak(int iters, uint32_t *dst) {
  const int lane = threadIdx.x & 63;
  uint32_t word;
  if (KIND == 0) {
    const v4i a = {lane, lane * 3, lane * 5, lane * 7}, b = {lane * 11, lane * 13, 17, 19};
    v16i c0 = {}, c1 = {}, c2 = {}, c3 = {};
    for (int i = 0; i < iters; ++i) {
      c0 = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b, c0, 0, 0, 0);
      c1 = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b, c1, 0, 0, 0);
      c2 = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b, c2, 0, 0, 0);
      c3 = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b, c3, 0, 0, 0);
    }
    word = (uint32_t)(c0[lane & 15] ^ c1[3] ^ c2[7] ^ c3[15]);
  } else {
    const int e = 0x38302820;   // E4M3 codes of 1.0, 0.5, 0.25, 0.125
    const v8i a = {e, e, e, e, e, e, e, e}, b = {e, e, e, e, e, e, e, e};
    v16f c0 = {}, c1 = {}, c2 = {}, c3 = {};
    for (int i = 0; i < iters; ++i) {
      c0 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c0, 0, 0, 0, 0, 0, 0);
      c1 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c1, 0, 0, 0, 0, 0, 0);
      c2 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c2, 0, 0, 0, 0, 0, 0);
      c3 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c3, 0, 0, 0, 0, 0, 0);
    }
    word = __float_as_uint(c0[lane & 15] + c1[3] + c2[7] + c3[15]);
  }
  dst[(size_t)blockIdx.x * 256 + threadIdx.x] = word;
}


// Vector-issue sample.  One workgroup of sixteen waves per compute unit; wave
// w runs on SIMD w % 4 and takes role kValuMix[mix][w / 4]: 0 idle, 1 FP32 FMA
// (v_fma_f32, sixteen independent chains), 2 v_exp_f32 (sixteen independent),
// 3 v_mfma_i32_32x32x32_i8 (four independent accumulation chains).  Every
// active wave issues its stream for `window` shader-clock cycles (checked once
// per 64 vector or 16 matrix instructions) and records how many such rounds it
// completed and the cycles it took, so the instructions each SIMD retired per
// cycle follow for every role, alone and beside a matrix-instruction stream.
constexpr int kValuMix[SAGE_VALU_MIXES][4] = {
    {1, 0, 0, 0}, {1, 1, 1, 0}, {1, 1, 1, 1}, {2, 2, 2, 0}, {3, 1, 1, 1}, {3, 2, 2, 2},
};

#define SAGE_FMA16                                                                                     \
  _Pragma("unroll") for (int i = 0; i < 16; ++i) asm volatile("v_fma_f32 %0, %1, %2, %0" : "+v"(acc[i]) \
                                                              : "v"(x), "v"(y));
#define SAGE_EXP16 _Pragma("unroll") for (int i = 0; i < 16; ++i) asm volatile("v_exp_f32 %0, %0" : "+v"(acc[i]));

__global__ __launch_bounds__(1024) void k_valu_sample(int mix, uint64_t window, uint32_t *dst) {
  // 96 KiB of LDS: more than half of a compute unit's, so each workgroup gets a unit of its own
  __shared__ uint32_t pin[24 * 1024];
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  if (threadIdx.x == 0) pin[blockIdx.x % (24 * 1024)] = (uint32_t)mix;
  const int role = kValuMix[mix][wave >> 2];
  uint32_t rounds = 0;
  uint32_t word = 0;
  float acc[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) acc[i] = (float)(i + lane) * 0x1p-8f;
  const float x = 1.0f, y = (float)lane * 0x1p-20f;
  __syncthreads();
  const uint64_t t0 = __builtin_amdgcn_s_memtime();
  if (role == 1) {
    for (;;) {
      const uint64_t t = __builtin_amdgcn_s_memtime();
      SAGE_FMA16 SAGE_FMA16 SAGE_FMA16 SAGE_FMA16
      ++rounds;
      if (t - t0 >= window) break;
    }
  } else if (role == 2) {
    // exp2 of exp2 grows to +inf within a few rounds and stays there; the
    // instruction's issue cost does not depend on the value
    for (;;) {
      const uint64_t t = __builtin_amdgcn_s_memtime();
      SAGE_EXP16 SAGE_EXP16 SAGE_EXP16 SAGE_EXP16
      ++rounds;
      if (t - t0 >= window) break;
    }
  } else if (role == 3) {
    const v4i a = {lane, lane * 3, lane * 5, lane * 7}, b = {lane * 11, lane * 13, 17, 19};
    v16i c0 = {}, c1 = {}, c2 = {}, c3 = {};
    for (;;) {
      const uint64_t t = __builtin_amdgcn_s_memtime();
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        c0 = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b, c0, 0, 0, 0);
        c1 = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b, c1, 0, 0, 0);
        c2 = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b, c2, 0, 0, 0);
        c3 = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b, c3, 0, 0, 0);
      }
      ++rounds;
      if (t - t0 >= window) break;
    }
    word = (uint32_t)(c0[lane & 15] ^ c1[3] ^ c2[7] ^ c3[15]);
  }
  const uint64_t cycles = __builtin_amdgcn_s_memtime() - t0;
#pragma unroll
  for (int i = 0; i < 16; ++i) word ^= __float_as_uint(acc[i]);
  if (lane == 0) {
    uint32_t *d = dst + ((size_t)blockIdx.x * 16 + wave) * 3;
    d[0] = role == 0 ? 0u : rounds;
    d[1] = (uint32_t)min(cycles, (uint64_t)0xffffffffu);
    d[2] = word ^ pin[blockIdx.x % (24 * 1024)];   // written by thread 0 before the first barrier
  }
}
#undef SAGE_FMA16
#undef SAGE_EXP16

}  // namespace

extern "C" {

int sage_mfma_peak_sample(int kind, int iters, uint32_t *dst, void *stream) {
  if (!dst) return SAGE_E_NULL;
  if (((uintptr_t)dst & 3u) != 0) return SAGE_E_ALIGN;
  if ((kind != 0 && kind != 1) || iters < 1 || iters > SAGE_PEAK_MAX_ITERS) return SAGE_E_ARG;
  int r = device_ok();
  if (r) return r;
  if (kind == 0)
    hipLaunchKernelGGL(k_mfma_peak<0>, dim3(SAGE_PEAK_WORKGROUPS), dim3(256), 0, (hipStream_t)stream, iters, dst);
  else
    hipLaunchKernelGGL(k_mfma_peak<1>, dim3(SAGE_PEAK_WORKGROUPS), dim3(256), 0, (hipStream_t)stream, iters, dst);
  return hipGetLastError() == hipSuccess ? SAGE_OK : SAGE_E_LAUNCH;
}

int sage_valu_sample(int mix, int window_kcycles, uint32_t *dst, void *stream) {
  if (!dst) return SAGE_E_NULL;
  if (((uintptr_t)dst & 3u) != 0) return SAGE_E_ALIGN;
  if (mix < 0 || mix >= SAGE_VALU_MIXES || window_kcycles < 1 || window_kcycles > SAGE_VALU_MAX_KCYCLES)
    return SAGE_E_ARG;
  int r = device_ok();
  if (r) return r;
  hipLaunchKernelGGL(k_valu_sample, dim3(SAGE_VALU_WORKGROUPS), dim3(1024), 0, (hipStream_t)stream, mix,
                     (uint64_t)window_kcycles * 1000u, dst);
  return hipGetLastError() == hipSuccess ? SAGE_OK : SAGE_E_LAUNCH;
}

int sage_clock_sample(uint64_t *dst, void *stream) {
  if (!dst) return SAGE_E_NULL;
  if (((uintptr_t)dst & 7u) != 0) return SAGE_E_ALIGN;
  int r = device_ok();
  if (r) return r;
  hipLaunchKernelGGL(k_clock_sample, dim3(SAGE_CLOCK_SAMPLES), dim3(64), 0, (hipStream_t)stream, dst);
  return hipGetLastError() == hipSuccess ? SAGE_OK : SAGE_E_LAUNCH;
}

const char *sage_status_string(int status) {
  switch (status) {
    case SAGE_OK: return "ok";
    case SAGE_E_NULL: return "a required pointer is NULL";
    case SAGE_E_SHAPE: return "shape out of range (B, H, Nq, Nkv >= 1; B*H <= 65535)";
    case SAGE_E_HEADDIM: return "head dimension must be 64 or 128";
    case SAGE_E_ALIGN: return "base pointer not 16-byte aligned or stride not a multiple of 8 elements";
    case SAGE_E_ALIAS: return "output overlaps itself, an input or a quantized buffer";
    case SAGE_E_DEVICE: return "no HIP device, or the device is not gfx950";
    case SAGE_E_LAUNCH: return "kernel launch failed";
    case SAGE_E_ARG: return "invalid argument";
    case SAGE_E_SCRATCH: return "the prep needs more scratch than the allocation-free entry's static 8 MiB";
    default: return "unknown status";
  }
}

int sage_device_check(int device) {
  if (device < 0 || device >= kMaxDevices) return SAGE_E_DEVICE;
  int known = g_device_ok[device].load(std::memory_order_relaxed);
  if (known == 0) {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, device) != hipSuccess) return SAGE_E_DEVICE;
    known = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : -1;
    g_device_ok[device].store(known, std::memory_order_relaxed);
  }
  return known == 1 ? SAGE_OK : SAGE_E_DEVICE;
}

int sage_buffer_bytes(const sage_shape_t *shape, int which, size_t *bytes) {
  if (!bytes) return SAGE_E_NULL;
  const int r = check_shape(shape);
  if (r) return r;
  if (which < 0 || which >= SAGE_BUF_COUNT) return SAGE_E_ARG;
  *bytes = buffer_bytes(shape, which);
  return SAGE_OK;
}

int sage_prep_status_offset(const sage_shape_t *shape, size_t *offset) {
  if (!offset) return SAGE_E_NULL;
  const int r = check_shape(shape);
  if (r) return r;
  const int BH = shape->B * shape->H, nchunk = ceil_div(shape->Nkv, kStatChunk);
  // single-pass region: arrival counters [BH], ready flags [BH], status word
  *offset = ws_sync_offset(BH, nchunk, shape->D) + (size_t)2 * BH * sizeof(uint32_t);
  return SAGE_OK;
}

}  // extern "C"

namespace {

// no_alloc: the workspace is the static device scratch instead of quant->workspace;
// race_seed: nonzero runs the race-gate build of the three launches
// kv_only: K and V only (q, the Q codes and the Q scale are not used)
int quant_prep(const void *q, const void *k, const void *v, const sage_shape_t *s, const sage_strides_t *st,
               const sage_quant_t *quant, void *stream, bool single_pass, bool no_alloc = false,
               uint32_t race_seed = 0, bool kv_only = false) {
  int r = check_shape(s);
  if (r) return r;
  if ((!kv_only && !q) || !k || !v || !st) return SAGE_E_NULL;
  if ((r = check_quant(quant, !no_alloc, !kv_only))) return r;
  sage_quant_t qs = *quant;
  if (kv_only) {
    qs.q_codes = nullptr;                        // neither read nor written
    qs.q_scale = nullptr;
  }
  if (no_alloc) {
    qs.workspace = nullptr;                      // ignored; the scratch is checked below
    if (buffer_bytes(s, SAGE_BUF_WORKSPACE) > kScratchBytes) return SAGE_E_SCRATCH;
  }
  quant = &qs;
  if ((!kv_only && (!aligned16(q) || check_strides(st->q))) || !aligned16(k) || !aligned16(v) ||
      check_strides(st->k) || check_strides(st->v))
    return SAGE_E_ALIGN;
  if ((!kv_only && overlaps_quant(q, span_bytes(s, st->q, s->Nq), quant, s)) ||
      overlaps_quant(k, span_bytes(s, st->k, s->Nkv), quant, s) ||
      overlaps_quant(v, span_bytes(s, st->v, s->Nkv), quant, s))
    return SAGE_E_ALIAS;
  if ((r = device_ok())) return r;
  if (no_alloc && (r = scratch_address(&qs.workspace))) return r;

  PrepParams p;
  std::memset(&p, 0, sizeof(p));
  p.q = (const uint16_t *)q;
  p.k = (const uint16_t *)k;
  p.v = (const uint16_t *)v;
  for (int i = 0; i < 3; ++i) {
    p.qs[i] = st->q[i];
    p.ks[i] = st->k[i];
    p.vs[i] = st->v[i];
  }
  p.B = s->B;
  p.H = s->H;
  p.Nq = s->Nq;
  p.Nkv = s->Nkv;
  p.D = s->D;
  p.nqb = ceil_div(s->Nq, kBQ);
  p.T = ceil_div(s->Nkv, kBK);
  p.nchunk = ceil_div(s->Nkv, kStatChunk);
  p.q_codes = quant->q_codes;
  p.q_scale = quant->q_scale;
  p.k_codes = quant->k_codes;
  p.k_scale = quant->k_scale;
  p.v_codes = quant->v_codes;
  p.v_scale = quant->v_scale;
  p.k_mean = quant->k_mean;
  const int BH = s->B * s->H;
  uint8_t *ws = (uint8_t *)quant->workspace;
  p.ws_ksum = (double *)ws;
  p.ws_vmax = (float *)(ws + ws_vmax_offset(BH, p.nchunk, s->D));
  p.ws_vinv = (float *)(ws + ws_vinv_offset(BH, p.nchunk, s->D));
  p.ws_sync = (uint32_t *)(ws + ws_sync_offset(BH, p.nchunk, s->D));
  p.ws_asum = (double *)(p.ws_sync + ws_sync_head_words(BH));
  p.ws_amax = (uint32_t *)(p.ws_asum + (size_t)BH * s->D);
  const int groups = ceil_div(s->Nkv, kFusedRows(s->D));
  // G = 0: statistics, finalize and quantization launches
  p.G = single_pass && groups <= kFusedMaxGroups ? groups : 0;
  p.kv_only = kv_only;
  p.race_seed = race_seed;
  return launch_prep(p, (hipStream_t)stream) == hipSuccess ? SAGE_OK : SAGE_E_LAUNCH;
}

}  // namespace

extern "C" {

int sage_quant_prep(const void *q, const void *k, const void *v, const sage_shape_t *s,
                    const sage_strides_t *st, const sage_quant_t *quant, void *stream) {
  return quant_prep(q, k, v, s, st, quant, stream, false);
}

int sage_quant_prep_single_pass(const void *q, const void *k, const void *v, const sage_shape_t *s,
                                const sage_strides_t *st, const sage_quant_t *quant, void *stream) {
  return quant_prep(q, k, v, s, st, quant, stream, true);
}

int sage_quant_prep_no_alloc(const void *q, const void *k, const void *v, const sage_shape_t *s,
                             const sage_strides_t *st, const sage_quant_t *quant, void *stream) {
  return quant_prep(q, k, v, s, st, quant, stream, false, true);
}

int sage_quant_prep_kv(const void *k, const void *v, const sage_shape_t *s, const sage_strides_t *st,
                       const sage_quant_t *quant, void *stream) {
  return quant_prep(nullptr, k, v, s, st, quant, stream, false, false, 0, true);
}

int sage_attn_fwd_q(const void *q, const sage_quant_t *quant, const sage_shape_t *s, float sm_scale, void *out,
                    const sage_strides_t *st, void *stream) {
  if (!quant) return SAGE_E_NULL;
  sage_quant_t kv = *quant;
  kv.q_codes = nullptr;                          // neither read nor written
  kv.q_scale = nullptr;
  FwdParams fp;
  int r = fill_fwd(&kv, s, sm_scale, out, st, &fp, false);
  if (r) return r;
  if (!q) return SAGE_E_NULL;
  if (!aligned16(q) || check_strides(st->q)) return SAGE_E_ALIGN;
  if (overlap(out, span_bytes(s, st->o, s->Nq), q, span_bytes(s, st->q, s->Nq))) return SAGE_E_ALIAS;
  if ((r = device_ok())) return r;
  fp.q = (const uint16_t *)q;
  for (int i = 0; i < 3; ++i) fp.qs[i] = st->q[i];
  fp.q_codes = nullptr;
  fp.q_scale = nullptr;
  return launch_fwd(fp, s->D, fp.n_units, FwdVariant::kQuantizeQ, (hipStream_t)stream) == hipSuccess
             ? SAGE_OK
             : SAGE_E_LAUNCH;
}

int sage_attn_fwd(const sage_quant_t *quant, const sage_shape_t *s, float sm_scale, void *out,
                  const sage_strides_t *st, void *stream) {
  FwdParams fp;
  int r = fill_fwd(quant, s, sm_scale, out, st, &fp);
  if (r) return r;
  if ((r = device_ok())) return r;
  return launch_fwd(fp, s->D, fp.n_units, FwdVariant::kDefault, (hipStream_t)stream) == hipSuccess ? SAGE_OK
                                                                                                   : SAGE_E_LAUNCH;
}

int sage_attn_fwd_paired(const sage_quant_t *quant, const sage_shape_t *s, float sm_scale, void *out,
                         const sage_strides_t *st, void *stream) {
  FwdParams fp;
  int r = fill_fwd(quant, s, sm_scale, out, st, &fp);
  if (r) return r;
  if ((r = device_ok())) return r;
  return launch_fwd(fp, s->D, fp.n_units, FwdVariant::kPaired, (hipStream_t)stream) == hipSuccess ? SAGE_OK
                                                                                                  : SAGE_E_LAUNCH;
}

int sage_attn_fwd_capture(const sage_quant_t *quant, const sage_shape_t *s, float sm_scale, void *out,
                          const sage_strides_t *st, const int32_t *units, int32_t n_units, int32_t *s_cap,
                          uint8_t *p8_cap, float *md_cap, float *part_cap, float *ro_cap, float *r_cap,
                          void *stream) {
  FwdParams fp;
  int r = fill_fwd(quant, s, sm_scale, out, st, &fp);
  if (r) return r;
  if (!units || !s_cap || !p8_cap || !md_cap || !part_cap || !ro_cap || !r_cap) return SAGE_E_NULL;
  if (n_units < 1 || n_units > fp.n_units) return SAGE_E_ARG;
  if (!aligned16(s_cap) || !aligned16(p8_cap) || !aligned16(md_cap) || !aligned16(part_cap) ||
      !aligned16(ro_cap) || !aligned16(r_cap))
    return SAGE_E_ALIGN;
  if ((r = device_ok())) return r;
  fp.units = units;
  fp.s_cap = s_cap;
  fp.p8_cap = p8_cap;
  fp.md_cap = md_cap;
  fp.part_cap = part_cap;
  fp.ro_cap = ro_cap;
  fp.r_cap = r_cap;
  return launch_fwd(fp, s->D, n_units, FwdVariant::kCapture, (hipStream_t)stream) == hipSuccess ? SAGE_OK
                                                                                               : SAGE_E_LAUNCH;
}

int sage_race_gate(const void *q, const void *k, const void *v, const sage_shape_t *s, const sage_strides_t *st,
                   const sage_quant_t *quant, float sm_scale, void *out, uint32_t seed, void *stream) {
  if (seed == 0) return SAGE_E_ARG;
  FwdParams fp;
  int r = fill_fwd(quant, s, sm_scale, out, st, &fp);
  if (r) return r;
  if (out && (overlap(out, span_bytes(s, st->o, s->Nq), q, span_bytes(s, st->q, s->Nq)) ||
              overlap(out, span_bytes(s, st->o, s->Nq), k, span_bytes(s, st->k, s->Nkv)) ||
              overlap(out, span_bytes(s, st->o, s->Nq), v, span_bytes(s, st->v, s->Nkv))))
    return SAGE_E_ALIAS;
  if ((r = quant_prep(q, k, v, s, st, quant, stream, false, false, seed))) return r;
  fp.race_seed = seed;
  return launch_fwd(fp, s->D, fp.n_units, FwdVariant::kRace, (hipStream_t)stream) == hipSuccess ? SAGE_OK
                                                                                                 : SAGE_E_LAUNCH;
}

}  // extern "C"
