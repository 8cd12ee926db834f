"""ctypes binding of libmoe_decode.so (include/moe_decode.h).

Argument marshalling only: every step of the routed-expert path runs in the
library's HIP kernels. PyTorch provides device memory and the stream.
"""

from __future__ import annotations

import ctypes
import glob
import os
import re
from typing import Optional, Sequence

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libmoe_decode.so")
HEADER = os.path.join(os.path.dirname(HERE), "include", "moe_decode.h")

OK = 0
ERR_INVALID_ARG = -1
ERR_UNSUPPORTED = -2
ERR_TOO_MANY_TOKENS = -3
ERR_HIP = -4
ERR_OUT_OF_MEMORY = -5
ERR_SCRATCH_TOO_SMALL = -6

DTYPE_F32 = 0
DTYPE_BF16 = 1
SCALES_F32 = 0
SCALES_UE8M0_PACKED = 1
WEIGHT_FORMATS = {"fp8": 0, "nvfp4": 1}
GEMM_PATHS = {"auto": 0, "valu_splitk": 1, "mfma_splitk": 2, "mfma": 3, "fp4": 4}
LAUNCH_MODES = {"auto": 0, "separate": 1, "combine_in_gemm2": 2, "swiglu_in_gemm1": 3, "route_in_gemm1": 4}

STAGES = {
    "ctrl": 0, "uexp": 1, "uoff": 2, "ucnt": 3, "routes": 4, "x_q": 5, "x_s": 6,
    "part1": 7, "h_q": 8, "h_s": 9, "part2": 10,
    "shared_x_q": 11, "shared_x_s": 12, "shared_part1": 13, "shared_h_q": 14,
    "shared_h_s": 15, "shared_part2": 16, "jobs": 17, "route_jobs": 18,
    "shared_scale13": 19, "shared_scale2": 20,
}
TIMING_SLOTS = ("route_quant", "gemm1", "swiglu_requant", "gemm2", "combine")


class MoeDecodeConfig(ctypes.Structure):
    _fields_ = [
        ("hidden", ctypes.c_int32),
        ("inter", ctypes.c_int32),
        ("experts", ctypes.c_int32),
        ("top_k", ctypes.c_int32),
        ("max_tokens", ctypes.c_int32),
        ("logits_dtype", ctypes.c_int32),
        ("ue8m0_act", ctypes.c_int32),
        ("limit", ctypes.c_float),
        ("routed_scale", ctypes.c_float),
        ("w13", ctypes.c_void_p),
        ("w13_scale", ctypes.c_void_p),
        ("w2", ctypes.c_void_p),
        ("w2_scale", ctypes.c_void_p),
        ("shared_inter", ctypes.c_int32),
        ("shared_scale_format", ctypes.c_int32),
        ("shared_ue8m0_act", ctypes.c_int32),
        ("shared_limit", ctypes.c_float),
        ("sw13", ctypes.c_void_p),
        ("sw13_scale", ctypes.c_void_p),
        ("sw2", ctypes.c_void_p),
        ("sw2_scale", ctypes.c_void_p),
        ("gemm_path", ctypes.c_int32),
        ("splits1", ctypes.c_int32),
        ("splits2", ctypes.c_int32),
        ("weight_format", ctypes.c_int32),
        ("local_begin", ctypes.c_int32),
        ("local_experts", ctypes.c_int32),
        ("launch_mode", ctypes.c_int32),
    ]


class MoeDecodeError(RuntimeError):
    def __init__(self, code: int, what: str = ""):
        self.code = code
        super().__init__(f"{what}: {error_string(code)} ({code})" if what else error_string(code))


_lib = None


def header_functions() -> Sequence[str]:
    """Names of the functions the headers in include/ declare."""
    names = set()
    for h in sorted(glob.glob(os.path.join(os.path.dirname(HEADER), "*.h"))):
        text = open(h).read()
        names |= set(re.findall(r"^\s*(?:const\s+)?[\w\s\*]+?\b(moe_\w+)\s*\(", text, re.M))
    return sorted(names)


def lib() -> ctypes.CDLL:
    """The loaded library. Raises if it has not been built: there is no
    fallback implementation."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(
            f"{LIB_PATH} is missing: build it with `python -m fp8_block_scaled_moe_amd.build` "
            "(the routed-expert path has no implementation outside the HIP library)")
    L = ctypes.CDLL(LIB_PATH)
    vp, i32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
    L.moe_decode_create.argtypes = [ctypes.POINTER(MoeDecodeConfig), ctypes.POINTER(vp)]
    L.moe_decode_create.restype = ctypes.c_int
    L.moe_decode_run.argtypes = [vp, i32, vp, vp, vp, vp, vp, vp, vp, vp, vp]
    L.moe_decode_run.restype = ctypes.c_int
    L.moe_decode_run_noalloc.argtypes = [ctypes.POINTER(MoeDecodeConfig), i32, vp, vp, vp, vp, vp, vp, vp,
                                         vp, vp]
    L.moe_decode_run_noalloc.restype = ctypes.c_int
    L.moe_decode_destroy.argtypes = [vp]
    L.moe_decode_destroy.restype = None
    L.moe_decode_error_string.argtypes = [ctypes.c_int]
    L.moe_decode_error_string.restype = ctypes.c_char_p
    L.moe_decode_plan.argtypes = [vp, i32, ctypes.POINTER(i32), i32]
    L.moe_decode_plan.restype = ctypes.c_int
    L.moe_decode_debug_stage.argtypes = [vp, i32, vp, sz, vp]
    L.moe_decode_debug_stage.restype = ctypes.c_int
    L.moe_decode_set_timing.argtypes = [vp, i32]
    L.moe_decode_set_timing.restype = ctypes.c_int
    L.moe_decode_last_timing.argtypes = [vp, ctypes.POINTER(ctypes.c_float), i32]
    L.moe_decode_last_timing.restype = ctypes.c_int
    L.moe_decode_debug_codec.argtypes = [vp, vp, vp, i32, vp]
    L.moe_decode_debug_codec.restype = ctypes.c_int
    L.moe_decode_debug_codec_fp4.argtypes = [vp, vp, vp, i32, vp]
    L.moe_decode_debug_codec_fp4.restype = ctypes.c_int
    L.moe_mxfp8_quantize.argtypes = [vp, i32, i32, vp, vp, vp]
    L.moe_mxfp8_quantize.restype = ctypes.c_int
    L.moe_reduce_rmsnorm.argtypes = [vp, i32, i32, i32, vp, ctypes.c_float, vp, vp, vp]
    L.moe_reduce_rmsnorm.restype = ctypes.c_int
    _lib = L
    return L


def error_string(code: int) -> str:
    return lib().moe_decode_error_string(code).decode()


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else stream


def _need(t: torch.Tensor, name: str, dtypes, dev, align: int = 16, shape=None,
          min_rows: bool = False) -> None:
    """Device, dtype, contiguity, alignment and shape of one buffer. With
    min_rows the first dimension may exceed shape[0] (a buffer with room for
    more rows than this call uses); the others must match."""
    if not isinstance(t, torch.Tensor):
        raise ValueError(f"{name} must be a tensor, got {type(t).__name__}")
    if shape is not None:
        have = tuple(t.shape)
        ok = (len(have) == len(shape) and have[1:] == tuple(shape[1:]) and
              (have[0] >= shape[0] if min_rows else have[0] == shape[0]))
        if not ok:
            more = " (or more rows)" if min_rows else ""
            raise ValueError(f"{name} has shape {have}, expected {tuple(shape)}{more}")
    if t.device != dev:
        raise ValueError(f"{name} must be on {dev}, got {t.device}")
    if t.dtype not in dtypes:
        raise ValueError(f"{name} has dtype {t.dtype}, expected one of {dtypes}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if t.data_ptr() % align:
        raise ValueError(f"{name} must start on a {align}-byte boundary (a slice can be copied with .clone())")


_FP8 = (torch.uint8, torch.float8_e4m3fn)


class MoeDecode:
    """Handle over moe_decode_create / moe_decode_run / moe_decode_destroy.

    Weight tensors are borrowed: the handle keeps references so they outlive
    it. w13 [E, 2I, H] (up rows, then gate rows) and w2 [E, H, I] are e4m3
    bytes (uint8 or float8_e4m3fn); scales are FP32 [E, N/128, K/128].

    Optional shared expert: sw13 [2Is, H] (gate rows, then up rows) and
    sw2 [H, Is] e4m3, with FP32 block scales [2Is/128, H/128] / [H/128, Is/128]
    or packed UE8M0 int32 scales [2Is, ceil(H/512)] / [H, ceil(Is/512)].

    weight_format "nvfp4": w13 [El, 2I, H/2] and w2 [El, H, I/2] packed E2M1
    (uint8, low nibble first; gate rows first), w13_scale [El, 2I, H/16] and
    w2_scale [El, H, I/16] UE4M3 bytes (uint8 or float8_e4m3fn). With
    local_experts > 0 only experts [local_begin, local_begin + local_experts)
    of `experts` (routing) are computed and the weights cover those alone.
    """

    def __init__(self, w13, w13_scale, w2, w2_scale, *, top_k: int, limit: float,
                 routed_scale: float, max_tokens: int, logits_dtype=torch.float32,
                 ue8m0_act: bool = False, gemm_path: str = "auto", splits1: int = 0,
                 splits2: int = 0, sw13=None, sw13_scale=None, sw2=None, sw2_scale=None,
                 shared_limit: Optional[float] = None, shared_ue8m0_act: bool = True,
                 weight_format: str = "fp8", experts: Optional[int] = None, local_begin: int = 0,
                 launch_mode: str = "auto"):
        self.device = w13.device
        if weight_format not in WEIGHT_FORMATS:
            raise ValueError(f"weight_format must be one of {sorted(WEIGHT_FORMATS)}")
        fp4 = weight_format == "nvfp4"
        if w13.dim() != 3 or w13.shape[1] % 2:
            raise ValueError(f"w13 must be [E, 2I, {'H/2' if fp4 else 'H'}], got {tuple(w13.shape)}")
        El, N1, H = w13.shape
        if fp4:
            H *= 2
        I = N1 // 2
        if fp4:   # packed E2M1 two per byte, a UE4M3 byte per 16 values along K
            shapes = ((El, 2 * I, H // 2), (El, 2 * I, H // 16), (El, H, I // 2), (El, H, I // 16))
        else:     # e4m3 bytes, FP32 per 128 x 128 block
            shapes = ((El, 2 * I, H), (El, 2 * I // 128, H // 128), (El, H, I),
                      (El, H // 128, I // 128))
        sdt = _FP8 if fp4 else (torch.float32,)
        for t, n, d, want in zip((w13, w13_scale, w2, w2_scale), ("w13", "w13_scale", "w2", "w2_scale"),
                                 (_FP8, sdt, _FP8, sdt), shapes):
            _need(t, n, d, self.device, shape=want)
        E = El if experts is None else experts
        if not 0 <= local_begin or local_begin + El > E:
            raise ValueError(f"local experts [{local_begin}, {local_begin + El}) must lie in [0, {E})")
        self.experts, self.hidden, self.inter, self.top_k = E, H, N1 // 2, top_k
        self.local_begin, self.local_experts = local_begin, El
        self.max_tokens = max_tokens
        self.logits_dtype = logits_dtype
        self._keep = (w13, w13_scale, w2, w2_scale)
        cfg = MoeDecodeConfig()
        cfg.hidden, cfg.inter, cfg.experts, cfg.top_k = H, N1 // 2, E, top_k
        cfg.max_tokens = max_tokens
        cfg.logits_dtype = DTYPE_BF16 if logits_dtype == torch.bfloat16 else DTYPE_F32
        cfg.ue8m0_act = int(bool(ue8m0_act))
        cfg.limit, cfg.routed_scale = limit, routed_scale
        cfg.w13, cfg.w13_scale, cfg.w2, cfg.w2_scale = (t.data_ptr() for t in self._keep)
        cfg.gemm_path = GEMM_PATHS[gemm_path]
        cfg.splits1, cfg.splits2 = splits1, splits2
        cfg.weight_format = WEIGHT_FORMATS[weight_format]
        cfg.local_begin = local_begin
        cfg.local_experts = 0 if El == E else El
        cfg.launch_mode = LAUNCH_MODES[launch_mode]
        self.shared_inter = 0
        if sw13 is not None:
            _need(sw13, "sw13", _FP8, self.device)
            _need(sw2, "sw2", _FP8, self.device)
            sdt = (torch.float32, torch.int32)
            _need(sw13_scale, "sw13_scale", sdt, self.device)
            _need(sw2_scale, "sw2_scale", sdt, self.device)
            if sw13_scale.dtype != sw2_scale.dtype:
                raise ValueError("sw13_scale and sw2_scale must have the same format")
            Is = sw13.shape[0] // 2
            if sw13.dim() != 2 or tuple(sw13.shape) != (2 * Is, H) or tuple(sw2.shape) != (H, Is):
                raise ValueError(f"shared weights must be [2Is, {H}] and [{H}, Is]")
            if sw13_scale.dtype == torch.float32:
                want13, want2 = (2 * Is // 128, H // 128), (H // 128, Is // 128)
            else:
                want13, want2 = (2 * Is, -(-H // 512)), (H, -(-Is // 512))
            if tuple(sw13_scale.shape) != want13 or tuple(sw2_scale.shape) != want2:
                raise ValueError(f"shared scales must be {want13} and {want2}")
            self.shared_inter = Is
            self._keep += (sw13, sw13_scale, sw2, sw2_scale)
            cfg.shared_inter = self.shared_inter
            cfg.shared_scale_format = (SCALES_F32 if sw13_scale.dtype == torch.float32
                                       else SCALES_UE8M0_PACKED)
            cfg.shared_ue8m0_act = int(bool(shared_ue8m0_act))
            cfg.shared_limit = limit if shared_limit is None else shared_limit
            cfg.sw13, cfg.sw13_scale, cfg.sw2, cfg.sw2_scale = (
                t.data_ptr() for t in (sw13, sw13_scale, sw2, sw2_scale))
        self.cfg = cfg
        h = ctypes.c_void_p()
        with torch.cuda.device(self.device):
            rc = lib().moe_decode_create(ctypes.byref(cfg), ctypes.byref(h))
        if rc != OK:
            raise MoeDecodeError(rc, "moe_decode_create")
        self._h = h

    # -- calls --------------------------------------------------------------
    def check_run_args(self, x, logits, bias, slots, ids, weights, combined, shared_out=None):
        """Device, dtype, contiguity, alignment and shape of every run buffer
        (the C ABI receives bare pointers and cannot check sizes). Raises
        ValueError; nothing has been launched then."""
        dev, H, k, E = self.device, self.hidden, self.top_k, self.experts
        if not isinstance(x, torch.Tensor) or x.dim() != 2:
            raise ValueError("x must be a [M, H] tensor")
        M = x.shape[0]
        bf16 = (torch.bfloat16,)
        _need(x, "x", bf16, dev, shape=(M, H))
        _need(logits, "logits", (self.logits_dtype,), dev, shape=(M, E), min_rows=True)
        _need(bias, "bias", (torch.float32,), dev, align=4, shape=(E,))
        _need(slots, "slots", bf16, dev, shape=(M * k, H), min_rows=True)
        _need(ids, "ids", (torch.int32,), dev, align=4, shape=(M, k), min_rows=True)
        _need(weights, "weights", (torch.float32,), dev, align=4, shape=(M, k), min_rows=True)
        _need(combined, "combined", bf16, dev, shape=(M, H), min_rows=True)
        if shared_out is not None:
            if not self.shared_inter:
                raise ValueError("shared_out given, but the handle has no shared expert")
            _need(shared_out, "shared_out", bf16, dev, shape=(M, H), min_rows=True)
        return M

    def run_into(self, x, logits, bias, slots, ids, weights, combined, shared_out=None,
                 stream=None) -> None:
        M = self.check_run_args(x, logits, bias, slots, ids, weights, combined, shared_out)
        rc = lib().moe_decode_run(self._h, M, _ptr(x), _ptr(logits), _ptr(bias), _ptr(slots),
                                  _ptr(ids), _ptr(weights), _ptr(combined), _ptr(shared_out),
                                  _stream(stream))
        if rc != OK:
            raise MoeDecodeError(rc, "moe_decode_run")

    def run_noalloc(self, x, logits, bias, slots, ids, weights, combined, shared_out=None,
                    stream=None) -> None:
        """moe_decode_run_noalloc with this handle's configuration: the same
        step, its workspace in the library's fixed per-GPU buffer instead of
        the handle's (nothing allocated; calls overlapping on one GPU race)."""
        M = self.check_run_args(x, logits, bias, slots, ids, weights, combined, shared_out)
        rc = lib().moe_decode_run_noalloc(ctypes.byref(self.cfg), M, _ptr(x), _ptr(logits), _ptr(bias),
                                          _ptr(slots), _ptr(ids), _ptr(weights), _ptr(combined),
                                          _ptr(shared_out), _stream(stream))
        if rc != OK:
            raise MoeDecodeError(rc, "moe_decode_run_noalloc")

    def outputs(self, M: int):
        dev, H, k = self.device, self.hidden, self.top_k
        return (torch.empty((M * k, H), dtype=torch.bfloat16, device=dev),
                torch.empty((M, k), dtype=torch.int32, device=dev),
                torch.empty((M, k), dtype=torch.float32, device=dev),
                torch.empty((M, H), dtype=torch.bfloat16, device=dev))

    def __call__(self, x, logits, bias, stream=None):
        """(slots [M*k, H] bf16, ids [M, k] int32, weights [M, k] f32,
        combined [M, H] bf16), plus shared_out [M, H] bf16 when the handle
        has a shared expert."""
        if not isinstance(x, torch.Tensor) or x.dim() != 2:
            raise ValueError("x must be a [M, H] tensor")
        out = self.outputs(x.shape[0])
        shared = None
        if self.shared_inter:
            shared = torch.empty((x.shape[0], self.hidden), dtype=torch.bfloat16, device=self.device)
        self.run_into(x, logits, bias, *out, shared_out=shared, stream=stream)
        return out + (shared,) if shared is not None else out

    # -- introspection ------------------------------------------------------
    def is_local(self, ids: torch.Tensor) -> torch.Tensor:
        return (ids >= self.local_begin) & (ids < self.local_begin + self.local_experts)

    def plan(self, M: int) -> dict:
        buf = (ctypes.c_int32 * 20)()
        rc = lib().moe_decode_plan(self._h, M, buf, 20)
        if rc != OK:
            raise MoeDecodeError(rc, "moe_decode_plan")
        keys = ("path", "splits1", "splits2", "ks1", "ks2", "grid1", "grid2", "rows1", "rows2",
                "shared_splits1", "shared_splits2", "shared_ks1", "shared_ks2",
                "shared_units1", "shared_units2", "kparts1", "kparts2", "launches",
                "persist1", "persist2")
        return dict(zip(keys, list(buf)))

    def stage(self, name: str, dst: torch.Tensor, stream=None) -> torch.Tensor:
        rc = lib().moe_decode_debug_stage(self._h, STAGES[name], dst.data_ptr(),
                                          dst.numel() * dst.element_size(), _stream(stream))
        if rc != OK:
            raise MoeDecodeError(rc, "moe_decode_debug_stage")
        return dst

    def set_timing(self, enable: bool) -> None:
        rc = lib().moe_decode_set_timing(self._h, int(enable))
        if rc != OK:
            raise MoeDecodeError(rc, "moe_decode_set_timing")

    def last_timing(self):
        """Milliseconds of each launch of the last timed run, in the order of
        TIMING_SLOTS."""
        n = len(TIMING_SLOTS)
        ms = (ctypes.c_float * n)()
        rc = lib().moe_decode_last_timing(self._h, ms, n)
        if rc != OK:
            raise MoeDecodeError(rc, "moe_decode_last_timing")
        return list(ms)

    def close(self) -> None:
        if getattr(self, "_h", None):
            lib().moe_decode_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def debug_codec_fp4(values: torch.Tensor):
    """(codes, decoded) from the library's device E2M1 encoder and its FP4
    reader (decoded[i] is code i & 15 read from nibble position (i >> 4) & 7)."""
    n = values.numel()
    q = torch.empty(n, dtype=torch.uint8, device=values.device)
    dq = torch.empty(n, dtype=torch.float32, device=values.device)
    rc = lib().moe_decode_debug_codec_fp4(values.data_ptr(), q.data_ptr(), dq.data_ptr(), n, _stream(None))
    if rc != OK:
        raise MoeDecodeError(rc, "moe_decode_debug_codec_fp4")
    return q, dq


def debug_codec(values: torch.Tensor):
    """(codes, decoded) from the library's device quantiser and FP8 reader."""
    n = values.numel()
    q = torch.empty(n, dtype=torch.uint8, device=values.device)
    dq = torch.empty(n, dtype=torch.float32, device=values.device)
    rc = lib().moe_decode_debug_codec(values.data_ptr(), q.data_ptr(), dq.data_ptr(), n, _stream(None))
    if rc != OK:
        raise MoeDecodeError(rc, "moe_decode_debug_codec")
    return q, dq


def mxfp8_quantize(x: torch.Tensor, stream=None):
    """MXFP8 of BF16 rows x [T, D] (include/moe_boundary.h): e4m3 codes
    [T, D] uint8 and E8M0 scale bytes [T, D/32] uint8."""
    if x.dtype != torch.bfloat16 or x.dim() != 2 or not x.is_contiguous():
        raise ValueError("x must be a contiguous [T, D] bfloat16 tensor")
    T, D = x.shape
    q = torch.empty((T, D), dtype=torch.uint8, device=x.device)
    sf = torch.empty((T, max(D // 32, 0)), dtype=torch.uint8, device=x.device)
    rc = lib().moe_mxfp8_quantize(x.data_ptr(), T, D, q.data_ptr(), sf.data_ptr(), _stream(stream))
    if rc != OK:
        raise MoeDecodeError(rc, "moe_mxfp8_quantize")
    return q, sf


def reduce_rmsnorm(partials: torch.Tensor, gamma: torch.Tensor, eps: float = 1e-5,
                   want_latent: bool = True, stream=None):
    """Reduce + RMSNorm (include/moe_boundary.h): partials [T, N, D] BF16,
    gamma [D] BF16 -> (latent [T, D] BF16 or None, out [T, D] BF16)."""
    if partials.dtype != torch.bfloat16 or partials.dim() != 3 or not partials.is_contiguous():
        raise ValueError("partials must be a contiguous [T, N, D] bfloat16 tensor")
    T, N, D = partials.shape
    if gamma.dtype != torch.bfloat16 or tuple(gamma.shape) != (D,) or not gamma.is_contiguous():
        raise ValueError(f"gamma must be a contiguous [{D}] bfloat16 tensor")
    out = torch.empty((T, D), dtype=torch.bfloat16, device=partials.device)
    latent = torch.empty_like(out) if want_latent else None
    rc = lib().moe_reduce_rmsnorm(partials.data_ptr(), T, N, D, gamma.data_ptr(), float(eps), _ptr(latent),
                                  out.data_ptr(), _stream(stream))
    if rc != OK:
        raise MoeDecodeError(rc, "moe_reduce_rmsnorm")
    return latent, out
