"""Python binding of the gfx950 quantized attention library (ctypes).

Argument marshalling only: every step of the path runs in the HIP kernels of
``libsage_attn.so``.  PyTorch provides device memory (``torch.empty``) and the
stream (``torch.cuda.current_stream()``).  There is no fallback: if the
library is not built, or a call fails, an exception is raised.

Names mirror the C ABI in ``include/sage_attn.h``.
"""

from __future__ import annotations

import ctypes
import functools
import os
from dataclasses import dataclass, field

import torch

from .build import LIB_PATH

SAGE_OK = 0
BQ = 128
BK = 64
BUFFERS = ["q_codes", "q_scale", "k_codes", "k_scale", "v_codes", "v_scale", "k_mean", "workspace"]

_STATUS = {
    0: "SAGE_OK", -1: "SAGE_E_NULL", -2: "SAGE_E_SHAPE", -3: "SAGE_E_HEADDIM", -4: "SAGE_E_ALIGN",
    -5: "SAGE_E_ALIAS", -6: "SAGE_E_DEVICE", -7: "SAGE_E_LAUNCH", -8: "SAGE_E_ARG",
}


class SageError(RuntimeError):
    def __init__(self, status: int, what: str, text: str):
        super().__init__("%s failed: %s (%s)" % (what, _STATUS.get(status, status), text))
        self.status = status


class SageShape(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int32), ("H", ctypes.c_int32), ("Nq", ctypes.c_int32),
                ("Nkv", ctypes.c_int32), ("D", ctypes.c_int32)]


class SageStrides(ctypes.Structure):
    _fields_ = [("q", ctypes.c_int64 * 3), ("k", ctypes.c_int64 * 3),
                ("v", ctypes.c_int64 * 3), ("o", ctypes.c_int64 * 3)]


class SageQuantC(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in BUFFERS]


_lib = None


def lib() -> ctypes.CDLL:
    """Load the HIP library (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError("libsage_attn.so is not built (%s); run __graft_entry__.build()" % LIB_PATH)
        L = ctypes.CDLL(LIB_PATH)
        vp, i32, f32 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_float
        L.sage_buffer_bytes.argtypes = [ctypes.POINTER(SageShape), ctypes.c_int, ctypes.POINTER(ctypes.c_size_t)]
        L.sage_prep_status_offset.argtypes = [ctypes.POINTER(SageShape), ctypes.POINTER(ctypes.c_size_t)]
        for name in ("sage_quant_prep", "sage_quant_prep_single_pass"):
            getattr(L, name).argtypes = [vp, vp, vp, ctypes.POINTER(SageShape), ctypes.POINTER(SageStrides),
                                         ctypes.POINTER(SageQuantC), vp]
        for name in ("sage_attn_fwd", "sage_attn_fwd_paired"):
            getattr(L, name).argtypes = [ctypes.POINTER(SageQuantC), ctypes.POINTER(SageShape), f32, vp,
                                         ctypes.POINTER(SageStrides), vp]
        L.sage_attn_fwd_capture.argtypes = [ctypes.POINTER(SageQuantC), ctypes.POINTER(SageShape), f32, vp,
                                            ctypes.POINTER(SageStrides), vp, i32, vp, vp, vp, vp, vp, vp, vp]
        L.sage_quant_prep_kv.argtypes = [vp, vp, ctypes.POINTER(SageShape), ctypes.POINTER(SageStrides),
                                         ctypes.POINTER(SageQuantC), vp]
        L.sage_attn_fwd_q.argtypes = [vp, ctypes.POINTER(SageQuantC), ctypes.POINTER(SageShape), f32, vp,
                                      ctypes.POINTER(SageStrides), vp]
        L.sage_clock_sample.argtypes = [vp, vp]
        L.sage_mfma_peak_sample.argtypes = [ctypes.c_int, ctypes.c_int, vp, vp]
        L.sage_valu_sample.argtypes = [ctypes.c_int, ctypes.c_int, vp, vp]
        L.sage_device_check.argtypes = [ctypes.c_int]
        L.sage_status_string.argtypes = [ctypes.c_int]
        L.sage_status_string.restype = ctypes.c_char_p
        for name in ("sage_buffer_bytes", "sage_prep_status_offset", "sage_quant_prep",
                     "sage_quant_prep_single_pass", "sage_attn_fwd", "sage_attn_fwd_paired", "sage_attn_fwd_capture",
                     "sage_device_check", "sage_clock_sample", "sage_mfma_peak_sample", "sage_valu_sample",
                     "sage_quant_prep_kv",
                     "sage_attn_fwd_q"):
            getattr(L, name).restype = ctypes.c_int
        _lib = L
    return _lib


def _check(status: int, what: str):
    if status != SAGE_OK:
        raise SageError(status, what, lib().sage_status_string(status).decode())


def status_string(status: int) -> str:
    return lib().sage_status_string(status).decode()


@functools.lru_cache(maxsize=256)
def sage_buffer_bytes(B: int, H: int, Nq: int, Nkv: int, D: int, which: int) -> int:
    n = ctypes.c_size_t(0)
    shape = SageShape(B, H, Nq, Nkv, D)
    _check(lib().sage_buffer_bytes(ctypes.byref(shape), which, ctypes.byref(n)), "sage_buffer_bytes")
    return n.value


def _stream_handle(stream, device) -> ctypes.c_void_p:
    s = torch.cuda.current_stream(device) if stream is None else stream
    if s.device != device:
        raise ValueError("stream is on %s, the tensors on %s" % (s.device, device))
    return ctypes.c_void_p(s.cuda_stream)


def _strides3(t: torch.Tensor):
    if t.dim() != 4 or t.stride(3) != 1:
        raise ValueError("expected a [B,H,N,D] tensor with a contiguous last dimension")
    return (ctypes.c_int64 * 3)(t.stride(0), t.stride(1), t.stride(2))


@dataclass
class SageQuant:
    """Device buffers of the quantized operands (see sage_quant_t in the header).

    A K/V-only set (from sage_quant_prep_kv) has q_codes = q_scale = None and
    serves sage_attn_fwd_q for queries of any length."""
    B: int
    H: int
    Nq: int
    Nkv: int
    D: int
    q_codes: torch.Tensor | None
    q_scale: torch.Tensor | None
    k_codes: torch.Tensor
    k_scale: torch.Tensor
    v_codes: torch.Tensor
    v_scale: torch.Tensor
    k_mean: torch.Tensor
    workspace: torch.Tensor
    # (buffer addresses and sizes, device) last validated, and its C struct
    _checked: tuple = field(default=None, repr=False, compare=False)
    _cstruct: object = field(default=None, repr=False, compare=False)

    @property
    def shape(self) -> SageShape:
        return SageShape(self.B, self.H, self.Nq, self.Nkv, self.D)

    @property
    def nqb(self) -> int:
        return -(-self.Nq // BQ)

    @property
    def T(self) -> int:
        return -(-self.Nkv // BK)

    @property
    def kv_only(self) -> bool:
        return self.q_codes is None and self.q_scale is None

    @property
    def device(self) -> torch.device:
        return self.k_codes.device

    def _key(self, device, need_q):
        bufs = [getattr(self, n) for n in BUFFERS]
        if not all(isinstance(t, torch.Tensor) or t is None for t in bufs):
            return None
        return (device, need_q) + tuple(None if t is None else (t.data_ptr(), t.numel(), t.is_contiguous(),
                                                                 t.device) for t in bufs)

    def check_buffers(self, device: torch.device, need_q: bool = True):
        """Every buffer on `device`, contiguous and at least as large as the C
        ABI's size for this shape (a caller-built or reused set included); the
        Q codes and scale only if need_q.  The outcome is remembered for the
        same buffers, so repeated calls on one set cost one address comparison."""
        key = self._key(device, need_q)
        if key is not None and key == self._checked:
            return
        for i, name in enumerate(BUFFERS):
            t = getattr(self, name)
            if not need_q and name in ("q_codes", "q_scale"):
                continue
            if not isinstance(t, torch.Tensor) or t.device != device or not t.is_contiguous():
                raise ValueError("quant.%s must be a contiguous tensor on %s" % (name, device))
            if t.numel() * t.element_size() < sage_buffer_bytes(self.B, self.H, self.Nq, self.Nkv, self.D, i):
                raise ValueError("quant.%s is smaller than the shape needs" % name)
        self._checked = key

    def single_pass_status(self) -> int:
        """Status word of the last single-pass prep into these buffers (0: every
        wait completed; nonzero: the outputs of that call are invalid).  Reads
        the word after synchronizing the device."""
        off = ctypes.c_size_t(0)
        _check(lib().sage_prep_status_offset(ctypes.byref(self.shape), ctypes.byref(off)), "sage_prep_status_offset")
        torch.cuda.synchronize(self.workspace.device)
        return int(self.workspace[off.value:off.value + 4].cpu().view(torch.int32).item())

    def c_struct(self) -> SageQuantC:
        ptrs = tuple(0 if getattr(self, n) is None else getattr(self, n).data_ptr() for n in BUFFERS)
        if self._cstruct is None or self._cstruct[0] != ptrs:
            self._cstruct = (ptrs, SageQuantC(*ptrs))
        return self._cstruct[1]

    @classmethod
    def allocate(cls, B, H, Nq, Nkv, D, device, kv_only: bool = False) -> "SageQuant":
        dt = {"q_codes": torch.int8, "k_codes": torch.int8, "v_codes": torch.uint8, "workspace": torch.uint8}
        bufs = {}
        for i, name in enumerate(BUFFERS):
            if kv_only and name in ("q_codes", "q_scale"):
                bufs[name] = None
                continue
            nbytes = sage_buffer_bytes(B, H, Nq, Nkv, D, i)
            dtype = dt.get(name, torch.float32)
            count = nbytes // torch.empty(0, dtype=dtype).element_size()
            bufs[name] = torch.empty(count, dtype=dtype, device=device)
        return cls(B, H, Nq, Nkv, D, **bufs)


def sage_quant_prep(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, out: SageQuant | None = None,
                    stream=None, single_pass: bool = False) -> SageQuant:
    """K mean, K smoothing, INT8 Q/K per block and FP8 V per channel on the GPU.

    single_pass selects sage_quant_prep_single_pass (K and V read once; same
    results)."""
    for t in (q, k, v):
        if t.dtype != torch.bfloat16 or not t.is_cuda:
            raise TypeError("q, k, v must be bfloat16 CUDA tensors")
    if q.dim() != 4 or k.dim() != 4:
        raise ValueError("q, k, v must be [B,H,N,D]")
    B, H, Nq, D = q.shape
    Nkv = k.shape[2]
    if k.shape != (B, H, Nkv, D) or v.shape != (B, H, Nkv, D):
        raise ValueError("k and v must be [B,H,Nkv,D] matching q")
    if k.device != q.device or v.device != q.device:
        raise ValueError("q, k, v must be on one device")
    if out is None:
        quant = SageQuant.allocate(B, H, Nq, Nkv, D, q.device)
    else:
        if (out.B, out.H, out.Nq, out.Nkv, out.D) != (B, H, Nq, Nkv, D):
            raise ValueError("out was allocated for another shape")
        out.check_buffers(q.device)
        quant = out
    st = SageStrides()
    st.q, st.k, st.v = _strides3(q), _strides3(k), _strides3(v)
    qc = quant.c_struct()
    name = "sage_quant_prep_single_pass" if single_pass else "sage_quant_prep"
    _check(getattr(lib(), name)(q.data_ptr(), k.data_ptr(), v.data_ptr(), ctypes.byref(quant.shape),
                                ctypes.byref(st), ctypes.byref(qc), _stream_handle(stream, q.device)), name)
    return quant


def sage_quant_prep_kv(k: torch.Tensor, v: torch.Tensor, out: SageQuant | None = None, stream=None) -> SageQuant:
    """K mean, K smoothing, INT8 K per tile and FP8 V per channel only: the
    K/V set that sage_attn_fwd_q uses for queries of any length (Q is
    quantized inside that forward)."""
    for t in (k, v):
        if t.dtype != torch.bfloat16 or not t.is_cuda:
            raise TypeError("k, v must be bfloat16 CUDA tensors")
    if k.dim() != 4 or v.shape != k.shape:
        raise ValueError("k and v must be [B,H,Nkv,D] of one shape")
    if v.device != k.device:
        raise ValueError("k and v must be on one device")
    B, H, Nkv, D = k.shape
    if out is None:
        quant = SageQuant.allocate(B, H, 1, Nkv, D, k.device, kv_only=True)
    else:
        if (out.B, out.H, out.Nkv, out.D) != (B, H, Nkv, D):
            raise ValueError("out was allocated for another shape")
        out.check_buffers(k.device, need_q=False)
        quant = out
    st = SageStrides()
    st.k, st.v = _strides3(k), _strides3(v)
    qc = quant.c_struct()
    _check(lib().sage_quant_prep_kv(k.data_ptr(), v.data_ptr(), ctypes.byref(quant.shape), ctypes.byref(st),
                                    ctypes.byref(qc), _stream_handle(stream, k.device)), "sage_quant_prep_kv")
    return quant


def sage_attn_fwd_q(q: torch.Tensor, quant: SageQuant, sm_scale: float | None = None,
                    out: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """The forward on bf16 Q: each workgroup quantizes its Q block by the prep's
    rule, then runs the default forward on the K/V set `quant` (from
    sage_quant_prep_kv or sage_quant_prep).  Same output as sage_quant_prep +
    sage_attn_fwd, bit for bit.  Returns bf16 [B,H,Nq,D]."""
    if q.dtype != torch.bfloat16 or not q.is_cuda or q.dim() != 4:
        raise TypeError("q must be a bfloat16 CUDA tensor [B,H,Nq,D]")
    B, H, Nq, D = q.shape
    if (B, H, D) != (quant.B, quant.H, quant.D):
        raise ValueError("q does not match the K/V set's B, H, D")
    if q.device != quant.device:
        raise ValueError("q must be on the device of the quantized buffers")
    quant.check_buffers(q.device, need_q=False)
    if out is None:
        out = torch.empty(B, H, Nq, D, dtype=torch.bfloat16, device=q.device)
    if out.dtype != torch.bfloat16 or tuple(out.shape) != (B, H, Nq, D) or out.device != q.device:
        raise ValueError("out must be bfloat16 [B,H,Nq,D] on the device of q")
    shape = SageShape(B, H, Nq, quant.Nkv, D)
    st = SageStrides()
    st.q, st.o = _strides3(q), _strides3(out)
    qc = quant.c_struct()
    _check(lib().sage_attn_fwd_q(q.data_ptr(), ctypes.byref(qc), ctypes.byref(shape),
                                 ctypes.c_float(0.0 if sm_scale is None else sm_scale), out.data_ptr(),
                                 ctypes.byref(st), _stream_handle(stream, q.device)), "sage_attn_fwd_q")
    return out


def _out_tensor(quant: SageQuant, out):
    if out is None:
        out = torch.empty(quant.B, quant.H, quant.Nq, quant.D, dtype=torch.bfloat16, device=quant.device)
    if out.dtype != torch.bfloat16 or tuple(out.shape) != (quant.B, quant.H, quant.Nq, quant.D):
        raise ValueError("out must be bfloat16 [B,H,Nq,D]")
    if out.device != quant.device:
        raise ValueError("out must be on the device of the quantized buffers")
    quant.check_buffers(out.device)
    return out


def sage_attn_fwd(quant: SageQuant, sm_scale: float | None = None, out: torch.Tensor | None = None,
                  stream=None, paired: bool = False) -> torch.Tensor:
    """Fused INT8-QK / FP8-PV online-softmax attention; returns bf16 [B,H,Nq,D].

    paired selects sage_attn_fwd_paired (three Q blocks per workgroup share
    one K/V stream; same results)."""
    out = _out_tensor(quant, out)
    st = SageStrides()
    st.o = _strides3(out)
    qc = quant.c_struct()
    name = "sage_attn_fwd_paired" if paired else "sage_attn_fwd"
    _check(getattr(lib(), name)(ctypes.byref(qc), ctypes.byref(quant.shape),
                                ctypes.c_float(0.0 if sm_scale is None else sm_scale), out.data_ptr(),
                                ctypes.byref(st), _stream_handle(stream, out.device)), name)
    return out


def sage_attn_fwd_capture(quant: SageQuant, units, sm_scale: float | None = None,
                          out: torch.Tensor | None = None, stream=None):
    """Run the listed work units with checkpoint capture.

    Returns (out, caps) where caps holds device tensors: s int32 [n,128,T*64],
    p8 uint8 [n,128,T*64], md float32 [n,128,T,3] (m, 448*d, alpha), part and ro
    float32 [n,128,T,D], r float32 [n,128] (1/(448*d)).
    """
    out = _out_tensor(quant, out)
    dev = quant.device
    units_t = torch.as_tensor(list(units), dtype=torch.int32).to(dev)
    n = units_t.numel()
    T = quant.T
    caps = {
        "s": torch.zeros(n, BQ, T * BK, dtype=torch.int32, device=dev),
        "p8": torch.zeros(n, BQ, T * BK, dtype=torch.uint8, device=dev),
        "md": torch.zeros(n, BQ, T, 3, dtype=torch.float32, device=dev),
        "part": torch.zeros(n, BQ, T, quant.D, dtype=torch.float32, device=dev),
        "ro": torch.zeros(n, BQ, T, quant.D, dtype=torch.float32, device=dev),
        "r": torch.zeros(n, BQ, dtype=torch.float32, device=dev),
    }
    st = SageStrides()
    st.o = _strides3(out)
    qc = quant.c_struct()
    _check(lib().sage_attn_fwd_capture(ctypes.byref(qc), ctypes.byref(quant.shape),
                                       ctypes.c_float(0.0 if sm_scale is None else sm_scale), out.data_ptr(),
                                       ctypes.byref(st), units_t.data_ptr(), n,
                                       *[caps[k].data_ptr() for k in ("s", "p8", "md", "part", "ro", "r")],
                                       _stream_handle(stream, dev)),
           "sage_attn_fwd_capture")
    return out, caps


def sage_attention(q, k, v, sm_scale: float | None = None) -> torch.Tensor:
    """The whole hot path on bf16 q, k, v: the K/V prep, then the forward that
    quantizes its own Q blocks (the same output bits as sage_quant_prep +
    sage_attn_fwd, without the Q codes' round trip through memory)."""
    return sage_attn_fwd_q(q, sage_quant_prep_kv(k, v), sm_scale)


CLOCK_SAMPLES = 2048


def sage_clock_sample(dst: torch.Tensor, stream=None) -> None:
    """Record per-workgroup (shader-clock counter, 100 MHz counter, XCD id,
    unit hardware id) into dst (int64 [CLOCK_SAMPLES, 4] on the GPU) when the
    stream reaches this point."""
    if dst.dtype != torch.int64 or dst.numel() < 4 * CLOCK_SAMPLES or not dst.is_cuda or not dst.is_contiguous():
        raise ValueError("dst must be a contiguous int64 CUDA tensor of %d elements" % (4 * CLOCK_SAMPLES))
    _check(lib().sage_clock_sample(dst.data_ptr(), _stream_handle(stream, dst.device)), "sage_clock_sample")


PEAK_WORKGROUPS = 1024
PEAK_MAX_ITERS = 65536
PEAK_OPS_PER_INSTRUCTION = {0: 32 * 32 * 32 * 2, 1: 32 * 32 * 64 * 2}   # kind 0: INT8, kind 1: FP8


def sage_mfma_peak_sample(kind: int, iters: int, dst: torch.Tensor, stream=None) -> int:
    """Launch the matrix-core peak sample (kind 0: INT8 32x32x32, 1: FP8
    32x32x64) on `stream`; dst: contiguous int32 CUDA tensor of
    PEAK_WORKGROUPS * 256 elements (scratch).  Returns the number of operations
    the launch performs; the caller times it."""
    if dst.dtype != torch.int32 or dst.numel() < PEAK_WORKGROUPS * 256 or not dst.is_cuda or not dst.is_contiguous():
        raise ValueError("dst must be a contiguous int32 CUDA tensor of %d elements" % (PEAK_WORKGROUPS * 256))
    _check(lib().sage_mfma_peak_sample(kind, iters, dst.data_ptr(), _stream_handle(stream, dst.device)),
           "sage_mfma_peak_sample")
    return PEAK_WORKGROUPS * 4 * iters * 4 * PEAK_OPS_PER_INSTRUCTION[kind]


VALU_WORKGROUPS = 256
VALU_MAX_KCYCLES = 10000
# roles of the four waves of each SIMD per mix: 0 idle, 1 FP32 FMA, 2 exp,
# 3 INT8 matrix instruction; instructions per round of each role
VALU_MIXES = {0: (1, 0, 0, 0), 1: (1, 1, 1, 0), 2: (1, 1, 1, 1), 3: (2, 2, 2, 0), 4: (3, 1, 1, 1), 5: (3, 2, 2, 2)}
VALU_ROUND_INSTRUCTIONS = {1: 64, 2: 64, 3: 16}


def sage_valu_sample(mix: int, window_kcycles: int, dst: torch.Tensor, stream=None) -> None:
    """Launch the vector-issue sample `mix` (see VALU_MIXES) for about
    window_kcycles * 1000 shader-clock cycles on `stream`; dst: contiguous
    int32 CUDA tensor of 3 * 16 * VALU_WORKGROUPS elements, per wave (rounds
    completed, cycles taken, a result word)."""
    if dst.dtype != torch.int32 or dst.numel() < 3 * 16 * VALU_WORKGROUPS or not dst.is_cuda or \
            not dst.is_contiguous():
        raise ValueError("dst must be a contiguous int32 CUDA tensor of %d elements" % (3 * 16 * VALU_WORKGROUPS))
    _check(lib().sage_valu_sample(mix, window_kcycles, dst.data_ptr(), _stream_handle(stream, dst.device)),
           "sage_valu_sample")
