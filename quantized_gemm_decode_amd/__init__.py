"""MI355X-native scaled quantized linear for LLM decode.

    Y[M, N] = s_a[m] * s_w[n] * (A_q[M, K] . W_q[N, K]^T)     (bf16 out)

Formats: FP8_Dynamic (OCP E4M3, per-token / per-channel), W8A8_INT8
(per-token / per-channel), Block_FP8 (1x128 activation groups, 128x128
weight blocks), MXFP8 (E4M3 with one E8M0 scale byte per 32 values along
K, applied by the matrix core) and MXFP4 (E2M1 weights two a byte, same
scales, MXFP8 activations).  All arithmetic runs in the hand-written gfx950 HIP kernels
of ``libqlinear.so`` behind the C ABI of ``include/qlinear.h``; this module
only marshals torch tensors (device memory) and streams into that ABI, with
the same function names.  There is no CPU or PyTorch fallback: if the
library is missing, or a tensor is not on the GPU, calls raise.
"""

import ctypes
import math
import os

import torch

from . import _lib
from ._lib import QLConfig, QLPlanFacts

FP8_DYNAMIC, W8A8_INT8, BLOCK_FP8, MXFP8, MXFP4 = 0, 1, 2, 3, 4
FORMATS = (FP8_DYNAMIC, W8A8_INT8, BLOCK_FP8, MXFP8, MXFP4)
FORMAT_NAMES = {FP8_DYNAMIC: "FP8_Dynamic", W8A8_INT8: "W8A8_INT8", BLOCK_FP8: "Block_FP8", MXFP8: "MXFP8",
                MXFP4: "MXFP4"}
MX_FORMATS = (MXFP8, MXFP4)
ALGO_DECODE, ALGO_TILED = 0, 1
SOURCES = {0: "table", 1: "heuristic", 2: "custom"}
DEFAULT_TABLE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "tables", "decode_table.txt")
CONFIG_FIELDS = [f for f, _ in QLConfig._fields_]


class QLinearError(RuntimeError):
    def __init__(self, status, where):
        lib = _lib.load()
        self.status = status
        msg = lib.qlinear_last_error().decode()
        super().__init__("%s failed: %s (%s)" % (where, lib.qlinear_status_string(status).decode(), msg))


def lib():
    return _lib.load()


def _check(status, where):
    if status != 0:
        raise QLinearError(status, where)


def _stream(stream):
    if stream is None:
        return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    if isinstance(stream, torch.cuda.Stream):
        return ctypes.c_void_p(stream.cuda_stream)
    return ctypes.c_void_p(int(stream))


def _ptr(t, name, dtype=None, required=True):
    if t is None:
        if required:
            raise ValueError("%s is required" % name)
        return None
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise ValueError("%s must be a CUDA (HIP) tensor" % name)
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    if dtype is not None and t.dtype not in (dtype if isinstance(dtype, tuple) else (dtype,)):
        raise ValueError("%s has dtype %s, expected %s" % (name, t.dtype, dtype))
    return ctypes.c_void_p(t.data_ptr())


def _need(t, name, nbytes):
    """Refuse an output (or input) tensor smaller than the call will touch."""
    if isinstance(t, torch.Tensor) and t.numel() * t.element_size() < nbytes:
        raise ValueError("%s holds %d bytes; this call needs at least %d"
                         % (name, t.numel() * t.element_size(), nbytes))


CODE_DTYPES = (torch.int8, torch.uint8, torch.float8_e4m3fn)
SCALE_DTYPES = (torch.float32, torch.uint8)      # binary32 scales, or MXFP8's E8M0 bytes


# ----------------------------------------------------------------- shapes

def act_scale_shape(fmt, M, K):
    if fmt in MX_FORMATS:
        return (M, K // 32)
    return (M, K // 128) if fmt == BLOCK_FP8 else (M,)


def weight_scale_shape(fmt, N, K):
    if fmt in MX_FORMATS:
        return (N, K // 32)
    return (-(-N // 128), K // 128) if fmt == BLOCK_FP8 else (N,)


def scale_dtype(fmt):
    return torch.uint8 if fmt in MX_FORMATS else torch.float32


def code_dtype(fmt):
    """Activation code dtype (MXFP4 plans take E4M3 activations)."""
    return torch.int8 if fmt == W8A8_INT8 else torch.float8_e4m3fn


def weight_code_shape(fmt, N, K):
    """Row-major W_q shape: MXFP4 holds two E2M1 values a byte."""
    return (N, K // 2) if fmt == MXFP4 else (N, K)


def weight_code_dtype(fmt):
    return torch.uint8 if fmt == MXFP4 else code_dtype(fmt)


# ----------------------------------------------------------------- quantizers

def qlinear_quantize_act(fmt, x, a_q, a_scale, stream=None):
    M, K = x.shape
    _need(a_q, "a_q", M * K)
    _need(a_scale, "a_scale", math.prod(act_scale_shape(fmt, M, K)) * (1 if fmt in MX_FORMATS else 4))
    _check(lib().qlinear_quantize_act(fmt, _ptr(x, "x", torch.bfloat16), M, K, _ptr(a_q, "a_q", CODE_DTYPES),
                                      _ptr(a_scale, "a_scale", SCALE_DTYPES), _stream(stream)),
           "qlinear_quantize_act")


def qlinear_packed_act_bytes(M, K):
    return int(lib().qlinear_packed_act_bytes(M, K))


def qlinear_quantize_act_packed(fmt, x, a_packed, a_scale, stream=None):
    M, K = x.shape
    _need(a_packed, "a_packed", qlinear_packed_act_bytes(M, K))
    _need(a_scale, "a_scale", qlinear_packed_mx_scale_bytes(M, K) if fmt in MX_FORMATS
          else 4 * math.prod(act_scale_shape(fmt, M, K)))
    _check(lib().qlinear_quantize_act_packed(fmt, _ptr(x, "x", torch.bfloat16), M, K,
                                             _ptr(a_packed, "a_packed", CODE_DTYPES),
                                             _ptr(a_scale, "a_scale", SCALE_DTYPES), _stream(stream)),
           "qlinear_quantize_act_packed")


def qlinear_quantize_weight(fmt, w, w_q, w_scale, stream=None):
    N, K = w.shape
    _need(w_q, "w_q", math.prod(weight_code_shape(fmt, N, K)))
    _need(w_scale, "w_scale", math.prod(weight_scale_shape(fmt, N, K)) * (1 if fmt in MX_FORMATS else 4))
    _check(lib().qlinear_quantize_weight(fmt, _ptr(w, "w", torch.bfloat16), N, K, _ptr(w_q, "w_q", CODE_DTYPES),
                                         _ptr(w_scale, "w_scale", SCALE_DTYPES), _stream(stream)),
           "qlinear_quantize_weight")


def quantize_act(fmt, x, stream=None):
    """Allocate (A_q, s_a) and run the activation quantizer."""
    M, K = x.shape
    a_q = torch.empty(M, K, dtype=code_dtype(fmt), device=x.device)
    a_s = torch.empty(act_scale_shape(fmt, M, K), dtype=scale_dtype(fmt), device=x.device)
    qlinear_quantize_act(fmt, x, a_q, a_s, stream)
    return a_q, a_s


def packed_act_scale_shape(fmt, M, K):
    """Shape of s_a as the packed quantizer writes it (MXFP8: flat lane-order bytes)."""
    return (max(qlinear_packed_mx_scale_bytes(M, K), 16),) if fmt in MX_FORMATS else act_scale_shape(fmt, M, K)


def act_scale_buffer(plan, device="cuda"):
    """s_a buffer for a forward with this plan (packed MXFP8 scales when it reads packed activations)."""
    shape = (packed_act_scale_shape if plan.config["a_mode"] >= 2 else act_scale_shape)(plan.fmt, plan.M, plan.K)
    return torch.empty(shape, dtype=scale_dtype(plan.fmt), device=device)


def quantize_act_packed(fmt, x, stream=None):
    """Allocate (packed A_q as a flat code buffer, s_a) and run the packed-layout quantizer."""
    M, K = x.shape
    a_p = torch.empty(max(qlinear_packed_act_bytes(M, K), 16), dtype=code_dtype(fmt), device=x.device)
    a_s = torch.empty(packed_act_scale_shape(fmt, M, K), dtype=scale_dtype(fmt), device=x.device)
    qlinear_quantize_act_packed(fmt, x, a_p, a_s, stream)
    return a_p, a_s


def act_buffer(plan, device="cuda"):
    """Activation code buffer in the plan's layout (packed when its a_mode is 2, 3 or 4)."""
    n = qlinear_packed_act_bytes(plan.M, plan.K) if plan.config["a_mode"] >= 2 else plan.M * plan.K
    return torch.empty(max(n, 16), dtype=code_dtype(plan.fmt), device=device)


def quantize_weight(fmt, w, stream=None):
    """Allocate (W_q, s_w) and run the weight quantizer."""
    N, K = w.shape
    w_q = torch.empty(weight_code_shape(fmt, N, K), dtype=weight_code_dtype(fmt), device=w.device)
    w_s = torch.empty(weight_scale_shape(fmt, N, K), dtype=scale_dtype(fmt), device=w.device)
    qlinear_quantize_weight(fmt, w, w_q, w_s, stream)
    return w_q, w_s


# ----------------------------------------------------------------- packing

def qlinear_encode_e4m3(x, codes, stream=None):
    """The library's E4M3 encoder: codes = E4M3(clamp(x, -448, 448)), round to nearest even."""
    _need(codes, "codes", x.numel())
    _check(lib().qlinear_encode_e4m3(_ptr(x, "x", torch.float32), x.numel(), _ptr(codes, "codes", CODE_DTYPES),
                                     _stream(stream)), "qlinear_encode_e4m3")


def qlinear_stream_read(src, nbytes, workgroups, sink, loads_in_flight=8, check=False, stream=None):
    """Measurement aid: read nbytes of src once (the streaming-read ceiling of a
    buffer that size); with check, sink gets one wrapping 32-bit word sum per
    workgroup."""
    _need(src, "src", nbytes)
    _need(sink, "sink", 4 * (workgroups or 1024))
    _check(lib().qlinear_stream_read(_ptr(src, "src"), int(nbytes), int(workgroups), int(loads_in_flight),
                                     int(bool(check)), _ptr(sink, "sink"), _stream(stream)), "qlinear_stream_read")


def qlinear_stream_read_bcast(src, nbytes, bcast, bcast_bytes, sink, workgroups=256, threads=1024,
                              loads_in_flight=4, check=False, stream=None):
    """Measurement aid: every workgroup reads its slice of nbytes of src and all
    bcast_bytes of bcast (the bytes each compute unit of an unsplit
    weight-streaming GEMM loads); with check, sink gets one wrapping 32-bit
    word sum per workgroup."""
    _need(src, "src", nbytes)
    if bcast_bytes:
        _need(bcast, "bcast", bcast_bytes)
    _need(sink, "sink", 4 * (workgroups or 256))
    _check(lib().qlinear_stream_read_bcast(_ptr(src, "src"), int(nbytes),
                                           _ptr(bcast, "bcast") if bcast_bytes else None, int(bcast_bytes),
                                           int(workgroups), int(threads), int(loads_in_flight), int(bool(check)),
                                           _ptr(sink, "sink"), _stream(stream)), "qlinear_stream_read_bcast")


def qlinear_packed_weight_bytes(N, K):
    return int(lib().qlinear_packed_weight_bytes(N, K))


def qlinear_pack_weight(w_q, w_packed, stream=None):
    N, K = w_q.shape
    _need(w_packed, "w_packed", qlinear_packed_weight_bytes(N, K))
    _check(lib().qlinear_pack_weight(_ptr(w_q, "w_q", CODE_DTYPES), N, K, _ptr(w_packed, "w_packed", CODE_DTYPES),
                                     _stream(stream)), "qlinear_pack_weight")


def qlinear_packed_mx_scale_bytes(R, K):
    return int(lib().qlinear_packed_mx_scale_bytes(R, K))


def qlinear_pack_mx_scales(s, K, out, stream=None):
    R = s.shape[0]
    _need(s, "scales", R * (K // 32))
    _need(out, "packed", qlinear_packed_mx_scale_bytes(R, K))
    _check(lib().qlinear_pack_mx_scales(_ptr(s, "scales", torch.uint8), R, K, _ptr(out, "packed", torch.uint8),
                                        _stream(stream)), "qlinear_pack_mx_scales")


def pack_mx_scales(s, stream=None):
    """Row-major MXFP8 scales [R, K/32] -> a new flat buffer in lane order."""
    R, KS = s.shape
    out = torch.empty(max(qlinear_packed_mx_scale_bytes(R, KS * 32), 16), dtype=torch.uint8, device=s.device)
    qlinear_pack_mx_scales(s, KS * 32, out, stream)
    return out


def qlinear_packed_weight_bytes_fp4(N, K):
    return int(lib().qlinear_packed_weight_bytes_fp4(N, K))


def pack_weight_fp4(w_q, stream=None):
    """MXFP4 row-major E2M1 pairs [N, K/2] -> a new flat buffer of packed 1 KB tiles."""
    N, K = w_q.shape[0], w_q.shape[1] * 2
    out = torch.empty(max(qlinear_packed_weight_bytes_fp4(N, K), 16), dtype=torch.uint8, device=w_q.device)
    _check(lib().qlinear_pack_weight_fp4(_ptr(w_q, "w_q", torch.uint8), N, K, _ptr(out, "w_packed", torch.uint8),
                                         _stream(stream)), "qlinear_pack_weight_fp4")
    return out


def pack_weight(w_q, stream=None):
    """Allocate the packed buffer (same code dtype, flat) and pack row-major codes into it."""
    N, K = w_q.shape
    out = torch.empty(qlinear_packed_weight_bytes(N, K), dtype=w_q.dtype, device=w_q.device)
    qlinear_pack_weight(w_q, out, stream)
    return out


# ----------------------------------------------------------------- table

def qlinear_table_load(path=DEFAULT_TABLE):
    n = ctypes.c_int64(0)
    _check(lib().qlinear_table_load(path.encode(), ctypes.byref(n)), "qlinear_table_load")
    return n.value


def qlinear_table_clear():
    lib().qlinear_table_clear()


# ----------------------------------------------------------------- plans

class Plan:
    """Owner of a ql_plan handle (host object)."""

    def __init__(self, handle, fmt, M, N, K):
        self.handle = ctypes.c_void_p(handle)
        self.fmt, self.M, self.N, self.K = fmt, M, N, K

    def __del__(self):
        h = getattr(self, "handle", None)
        try:
            if h is not None and h.value and _lib._lib is not None:
                _lib._lib.qlinear_plan_destroy(h)
        except Exception:       # interpreter shutdown: module globals may be gone
            pass
        self.handle = None

    def info(self):
        cfg, facts = QLConfig(), QLPlanFacts()
        _check(lib().qlinear_plan_info(self.handle, ctypes.byref(cfg), ctypes.byref(facts)), "qlinear_plan_info")
        c = {f: getattr(cfg, f) for f in CONFIG_FIELDS}
        f = {n: getattr(facts, n) for n, _ in QLPlanFacts._fields_}
        f["source"] = SOURCES.get(f["source"], f["source"])
        return c, f

    @property
    def config(self):
        return self.info()[0]

    @property
    def facts(self):
        return self.info()[1]

    @property
    def workspace_bytes(self):
        return int(lib().qlinear_workspace_bytes(self.handle))

    def operand_bytes(self):
        """Least bytes each operand of a run / forward with this plan must hold
        (the kernels read and write by the plan's shape, not the tensors')."""
        if getattr(self, "_operand_bytes", None) is None:
            cfg, facts = self.info()
            fmt, M, N, K = self.fmt, self.M, self.N, self.K
            mx = fmt in MX_FORMATS
            packed_a = cfg["a_mode"] >= 2
            sbytes = 1 if mx else 4
            if cfg["w_layout"] == 1:
                w = qlinear_packed_weight_bytes_fp4(N, K) if fmt == MXFP4 else qlinear_packed_weight_bytes(N, K)
            else:
                w = N * K // 2 if fmt == MXFP4 else N * K
            self._operand_bytes = dict(
                x=2 * M * K,
                a_q=qlinear_packed_act_bytes(M, K) if packed_a else M * K,
                a_scale=(qlinear_packed_mx_scale_bytes(M, K) if mx and packed_a
                         else math.prod(act_scale_shape(fmt, M, K)) * sbytes),
                w_q=w,
                w_scale=(qlinear_packed_mx_scale_bytes(N, K) if mx and cfg["w_layout"] == 1
                         else math.prod(weight_scale_shape(fmt, N, K)) * sbytes),
                y=2 * M * (N // 2 if facts["epilogue"] == 1 else N),
                acc_out=4 * M * N,
                workspace=facts["workspace_bytes"])
            if M == 0 or N == 0 or K == 0:     # a no-op, or (K == 0) a run that only zeroes Y
                self._operand_bytes = {k: (v if k == "y" else 0) for k, v in self._operand_bytes.items()}
        return self._operand_bytes

    def check_operands(self, **tensors):
        """Raise ValueError for any operand smaller than the plan needs."""
        need = self.operand_bytes()
        for name, t in tensors.items():
            if not isinstance(t, torch.Tensor):
                continue      # None, or not a tensor (the pointer check reports it)
            have = t.numel() * t.element_size()
            if have < need[name]:
                raise ValueError("%s holds %d bytes; this plan needs at least %d" % (name, have, need[name]))

    def new_workspace(self, device="cuda"):
        """Zero-initialised workspace (zeroed once; runs keep it all-zero)."""
        n = self.workspace_bytes
        return torch.zeros(max(n, 16), dtype=torch.uint8, device=device) if n else None


def qlinear_plan(fmt, M, N, K):
    h = ctypes.c_void_p()
    _check(lib().qlinear_plan(fmt, M, N, K, ctypes.byref(h)), "qlinear_plan")
    return Plan(h.value, fmt, M, N, K)


def qlinear_plan_packed(fmt, M, N, K):
    """Plan for weights packed with qlinear_pack_weight."""
    h = ctypes.c_void_p()
    _check(lib().qlinear_plan_packed(fmt, M, N, K, ctypes.byref(h)), "qlinear_plan_packed")
    return Plan(h.value, fmt, M, N, K)


def qlinear_plan_layouts(fmt, M, N, K, w_layout, a_packed):
    """Plan for the given operand layouts (w_layout: 0 row-major, 1 packed weights;
    a_packed: 0 row-major A_q, 1 packed A_q from qlinear_quantize_act_packed,
    2 a forward plan -- possibly with the quantizer fused into the GEMM --
    that runs only through qlinear_forward)."""
    h = ctypes.c_void_p()
    _check(lib().qlinear_plan_layouts(fmt, M, N, K, w_layout, a_packed, ctypes.byref(h)), "qlinear_plan_layouts")
    return Plan(h.value, fmt, M, N, K)


def qlinear_plan_glu(fmt, M, N, K, a_packed=1):
    """Plan for a merged gate/up weight [N, K] (packed) whose runs write the
    SiLU-and-mul output [M, N/2]; a_packed 1 = packed A_q (qlinear_run),
    2 = a forward plan (qlinear_forward, quantization possibly fused)."""
    h = ctypes.c_void_p()
    _check(lib().qlinear_plan_glu(fmt, M, N, K, a_packed, ctypes.byref(h)), "qlinear_plan_glu")
    return Plan(h.value, fmt, M, N, K)


def qlinear_plan_glu_with_config(fmt, M, N, K, cfg):
    c = QLConfig(**make_config(**cfg))
    h = ctypes.c_void_p()
    _check(lib().qlinear_plan_glu_with_config(fmt, M, N, K, ctypes.byref(c), ctypes.byref(h)),
           "qlinear_plan_glu_with_config")
    return Plan(h.value, fmt, M, N, K)


def qlinear_plan_from_table(fmt, M, N, K):
    h = ctypes.c_void_p()
    _check(lib().qlinear_plan_from_table(fmt, M, N, K, ctypes.byref(h)), "qlinear_plan_from_table")
    return Plan(h.value, fmt, M, N, K)


def make_config(**kw):
    base = dict(algo=ALGO_DECODE, swap_ab=0, split_k=1, waves_n=4, waves_k=1, rows_per_wave=16, prefetch=2,
                a_mode=0, w_lds=0, w_layout=0, tile_m=0, tile_n=0)
    unknown = set(kw) - set(base)
    if unknown:
        raise ValueError("unknown config fields %s" % sorted(unknown))
    base.update(kw)
    return base


def qlinear_plan_with_config(fmt, M, N, K, cfg):
    c = QLConfig(**make_config(**cfg))
    h = ctypes.c_void_p()
    _check(lib().qlinear_plan_with_config(fmt, M, N, K, ctypes.byref(c), ctypes.byref(h)),
           "qlinear_plan_with_config")
    return Plan(h.value, fmt, M, N, K)


# ----------------------------------------------------------------- GEMM

def qlinear_run(plan, a_q, a_scale, w_q, w_scale, y, workspace=None, stream=None):
    plan.check_operands(a_q=a_q, a_scale=a_scale, w_q=w_q, w_scale=w_scale, y=y, workspace=workspace)
    _check(lib().qlinear_run(plan.handle, _ptr(a_q, "a_q", CODE_DTYPES), _ptr(a_scale, "a_scale", SCALE_DTYPES),
                             _ptr(w_q, "w_q", CODE_DTYPES), _ptr(w_scale, "w_scale", SCALE_DTYPES),
                             _ptr(y, "y", torch.bfloat16), _ptr(workspace, "workspace", required=False),
                             _stream(stream)), "qlinear_run")


def qlinear_run_debug_acc(plan, a_q, a_scale, w_q, w_scale, y, acc_out, workspace=None, stream=None):
    plan.check_operands(a_q=a_q, a_scale=a_scale, w_q=w_q, w_scale=w_scale, y=y, acc_out=acc_out,
                        workspace=workspace)
    _check(lib().qlinear_run_debug_acc(plan.handle, _ptr(a_q, "a_q", CODE_DTYPES),
                                       _ptr(a_scale, "a_scale", SCALE_DTYPES), _ptr(w_q, "w_q", CODE_DTYPES),
                                       _ptr(w_scale, "w_scale", SCALE_DTYPES), _ptr(y, "y", torch.bfloat16),
                                       _ptr(workspace, "workspace", required=False),
                                       _ptr(acc_out, "acc_out", (torch.int32, torch.float32)), _stream(stream)),
           "qlinear_run_debug_acc")


def qlinear_forward(plan, x, a_q, a_scale, w_q, w_scale, y, workspace=None, stream=None):
    plan.check_operands(x=x, a_q=a_q, a_scale=a_scale, w_q=w_q, w_scale=w_scale, y=y, workspace=workspace)
    _check(lib().qlinear_forward(plan.handle, _ptr(x, "x", torch.bfloat16), _ptr(a_q, "a_q", CODE_DTYPES),
                                 _ptr(a_scale, "a_scale", SCALE_DTYPES), _ptr(w_q, "w_q", CODE_DTYPES),
                                 _ptr(w_scale, "w_scale", SCALE_DTYPES), _ptr(y, "y", torch.bfloat16),
                                 _ptr(workspace, "workspace", required=False), _stream(stream)),
           "qlinear_forward")


# QL_AMAX_BUFFER_BYTES of qlinear.h: 64 replica lines of 32 words (token m
# of replica r at word 32 r + m), then 17 counter lines
AMAX_BUFFER_BYTES = 10368
AMAX_REPLICAS, AMAX_LINE = 64, 32


def amax_buffer(M=None, device="cuda"):
    """Zeroed per-token amax buffer for qlinear_forward_glu_amax /
    qlinear_forward_amax (any M <= 32); reusable, the consumer leaves it zeroed."""
    return torch.zeros(AMAX_BUFFER_BYTES // 4, dtype=torch.int32, device=device)


def amax_of_buffer(buf, M):
    """The per-token maxima a buffer holds (the maximum over its replicas),
    as binary32 bit patterns (uint32 numpy array of M values)."""
    import numpy as np
    w = buf.cpu().numpy().view(np.uint32)
    return w[:AMAX_REPLICAS * AMAX_LINE].reshape(AMAX_REPLICAS, AMAX_LINE)[:, :M].max(axis=0)


def _need_amax(plan, t, name):
    _need(t, name, AMAX_BUFFER_BYTES)


def qlinear_forward_glu_amax(plan, x, a_q, a_scale, w_q, w_scale, h, h_amax, workspace=None, stream=None):
    """SiLU-and-mul forward that also folds max |h| per token into h_amax."""
    plan.check_operands(x=x, a_q=a_q, a_scale=a_scale, w_q=w_q, w_scale=w_scale, y=h, workspace=workspace)
    _need_amax(plan, h_amax, "h_amax")
    _check(lib().qlinear_forward_glu_amax(plan.handle, _ptr(x, "x", torch.bfloat16), _ptr(a_q, "a_q", CODE_DTYPES),
                                          _ptr(a_scale, "a_scale", SCALE_DTYPES), _ptr(w_q, "w_q", CODE_DTYPES),
                                          _ptr(w_scale, "w_scale", SCALE_DTYPES), _ptr(h, "h", torch.bfloat16),
                                          _ptr(h_amax, "h_amax", torch.int32),
                                          _ptr(workspace, "workspace", required=False), _stream(stream)),
           "qlinear_forward_glu_amax")


def qlinear_forward_amax(plan, x, x_amax, a_q, a_scale, w_q, w_scale, y, workspace=None, stream=None):
    """Forward of X whose per-token amax words are x_amax (left zeroed)."""
    plan.check_operands(x=x, a_q=a_q, a_scale=a_scale, w_q=w_q, w_scale=w_scale, y=y, workspace=workspace)
    _need_amax(plan, x_amax, "x_amax")
    _check(lib().qlinear_forward_amax(plan.handle, _ptr(x, "x", torch.bfloat16), _ptr(x_amax, "x_amax", torch.int32),
                                      _ptr(a_q, "a_q", CODE_DTYPES), _ptr(a_scale, "a_scale", SCALE_DTYPES),
                                      _ptr(w_q, "w_q", CODE_DTYPES), _ptr(w_scale, "w_scale", SCALE_DTYPES),
                                      _ptr(y, "y", torch.bfloat16), _ptr(workspace, "workspace", required=False),
                                      _stream(stream)),
           "qlinear_forward_amax")


def qlinear_forward_noalloc(plan, x, a_q, a_scale, w_q, w_scale, y, stream=None):
    """qlinear_forward with the split-K workspace taken from the library's
    per-GPU scratch (no allocation; calls on one GPU must not overlap)."""
    plan.check_operands(x=x, a_q=a_q, a_scale=a_scale, w_q=w_q, w_scale=w_scale, y=y)
    _check(lib().qlinear_forward_noalloc(plan.handle, _ptr(x, "x", torch.bfloat16), _ptr(a_q, "a_q", CODE_DTYPES),
                                         _ptr(a_scale, "a_scale", SCALE_DTYPES), _ptr(w_q, "w_q", CODE_DTYPES),
                                         _ptr(w_scale, "w_scale", SCALE_DTYPES), _ptr(y, "y", torch.bfloat16),
                                         _stream(stream)),
           "qlinear_forward_noalloc")


# Bytes of the per-GPU scratch behind qlinear_forward_noalloc (stated in include/qlinear.h).
NOALLOC_SCRATCH_BYTES = 16 << 20


# ----------------------------------------------------------------- graphs

class Graph:
    """Owner of a ql_graph (an instantiated hipGraph)."""

    def __init__(self, handle):
        self.handle = ctypes.c_void_p(handle)

    def launch(self, stream=None):
        qlinear_graph_launch(self, stream)

    def __del__(self):
        h = getattr(self, "handle", None)
        try:
            if h is not None and h.value and _lib._lib is not None:
                _lib._lib.qlinear_graph_destroy(h)
        except Exception:       # interpreter shutdown: module globals may be gone
            pass
        self.handle = None


def qlinear_graph_begin(stream):
    _check(lib().qlinear_graph_begin(_stream(stream)), "qlinear_graph_begin")


def qlinear_graph_end(stream):
    h = ctypes.c_void_p()
    _check(lib().qlinear_graph_end(_stream(stream), ctypes.byref(h)), "qlinear_graph_end")
    return Graph(h.value)


def qlinear_graph_launch(graph, stream=None):
    _check(lib().qlinear_graph_launch(graph.handle, _stream(stream)), "qlinear_graph_launch")


def load_default_table():
    """Load the sweep table shipped with the package (returns its entry count, 0 if absent)."""
    if os.path.exists(DEFAULT_TABLE):
        return qlinear_table_load(DEFAULT_TABLE)
    return 0
