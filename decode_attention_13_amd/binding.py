"""ctypes binding of ``libfd.so`` (include/fd.h): argument marshalling only.

Every step of the decode runs in the HIP kernels behind the C ABI. This module
turns torch tensors into pointers, sizes and a dtype code, allocates the
workspace with torch when the caller does not pass one, and raises on any
non-zero status. There is no fallback: if the library is not built, the first
call raises.
"""
from __future__ import annotations

import ctypes
import math
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libfd.so")

FD_DTYPE = {torch.float32: 0, torch.float16: 1, torch.bfloat16: 2}
DTYPE_NAMES = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}
# FP8 E4M3 caches: code by query dtype, and by name
FD_DTYPE_KV_E4M3 = {torch.float16: 3, torch.bfloat16: 4}
FP8_CODES = {"f16_kv_e4m3": 3, "bf16_kv_e4m3": 4}
FP8_CACHE_DTYPES = (torch.float8_e4m3fn, torch.uint8)  # uint8 = raw E4M3 codes
KERNELS = {"auto": 0, "valu": 1, "mfma": 2}
MERGES = {"auto": 0, "kernel": 1, "fused": 2}
LAUNCHES = {"auto": 0, "grid": 1, "persistent": 2}
WS_COUNTER_BYTES = 16384  # zeroed head block of every workspace (include/fd.h)
NOALLOC_SCRATCH_BYTES = 64 << 20  # static scratch of fd_paged_decode_noalloc (include/fd.h)
HEAD_DIM = 128
CHUNK_QUANTUM = 64


class FdOptions(ctypes.Structure):
    _fields_ = [("force_num_splits", ctypes.c_int), ("force_chunk", ctypes.c_int), ("force_kernel", ctypes.c_int),
                ("debug_checks", ctypes.c_int), ("split_begin_event", ctypes.c_void_p),
                ("split_end_event", ctypes.c_void_p), ("force_merge", ctypes.c_int),
                ("force_launch", ctypes.c_int)]


class FdPlan(ctypes.Structure):
    _fields_ = [("kernel", ctypes.c_int), ("heads_per_group", ctypes.c_int), ("chunk", ctypes.c_int),
                ("num_splits", ctypes.c_int), ("grid_x", ctypes.c_int), ("grid_y", ctypes.c_int),
                ("grid_z", ctypes.c_int), ("threads", ctypes.c_int), ("merge", ctypes.c_int),
                ("kv_heads_per_group", ctypes.c_int), ("workspace_bytes", ctypes.c_size_t),
                ("ws_lse_offset", ctypes.c_size_t), ("work_list", ctypes.c_int), ("persistent", ctypes.c_int),
                ("ws_err_offset", ctypes.c_size_t), ("ws_o_offset", ctypes.c_size_t), ("head_slices", ctypes.c_int),
                ("reserved3", ctypes.c_int)]

    def as_dict(self) -> dict:
        return {name: getattr(self, name) for name, _ in self._fields_ if name != "reserved3"}


class FdError(RuntimeError):
    def __init__(self, status: int, name: str, message: str):
        super().__init__(f"{name}: {message}")
        self.status = status
        self.name = name


_lib = None

# name -> (restype, argtypes); mirrors include/fd.h
SIGNATURES = {
    "fd_device_num_cus": (ctypes.c_int, []),
    "fd_decode_plan": (ctypes.c_int, [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                      ctypes.c_int, ctypes.POINTER(FdOptions), ctypes.POINTER(FdPlan)]),
    "fd_paged_plan": (ctypes.c_int, [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                     ctypes.c_int, ctypes.c_int, ctypes.c_longlong, ctypes.c_int,
                                     ctypes.POINTER(FdOptions), ctypes.POINTER(FdPlan)]),
    "fd_decode": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                 ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                 ctypes.c_float, ctypes.c_void_p, ctypes.c_size_t, ctypes.POINTER(FdOptions),
                                 ctypes.c_void_p]),
    "fd_paged_decode": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                       ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p, ctypes.c_float,
                                       ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                       ctypes.c_int, ctypes.c_int, ctypes.c_longlong, ctypes.c_int,
                                       ctypes.c_void_p, ctypes.c_size_t, ctypes.POINTER(FdOptions),
                                       ctypes.c_void_p]),
    "fd_paged_decode_noalloc": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                               ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p, ctypes.c_float,
                                               ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                               ctypes.c_int, ctypes.c_int, ctypes.c_longlong, ctypes.c_int,
                                               ctypes.POINTER(FdOptions), ctypes.c_void_p]),
    "fd_decode_fp8kv": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                       ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                       ctypes.c_float, ctypes.c_float, ctypes.c_float, ctypes.c_void_p,
                                       ctypes.c_size_t, ctypes.POINTER(FdOptions), ctypes.c_void_p]),
    "fd_paged_decode_fp8kv": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                             ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p, ctypes.c_float,
                                             ctypes.c_float, ctypes.c_float, ctypes.c_int, ctypes.c_int,
                                             ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                             ctypes.c_longlong, ctypes.c_int, ctypes.c_void_p, ctypes.c_size_t,
                                             ctypes.POINTER(FdOptions), ctypes.c_void_p]),
    "fd_prefill": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int,
                                  ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_float,
                                  ctypes.c_int, ctypes.c_void_p, ctypes.c_size_t, ctypes.POINTER(FdOptions),
                                  ctypes.c_void_p]),
    "fd_prefill_workspace_size": (ctypes.c_size_t, [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                                     ctypes.c_int]),
    "fd_decode_workspace_size": (ctypes.c_int, [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                                ctypes.c_int, ctypes.POINTER(FdOptions),
                                                ctypes.POINTER(ctypes.c_size_t)]),
    "fd_paged_workspace_size": (ctypes.c_int, [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                               ctypes.c_int, ctypes.c_int, ctypes.c_longlong, ctypes.c_int,
                                               ctypes.POINTER(FdOptions), ctypes.POINTER(ctypes.c_size_t)]),
    "fd_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "fd_last_error": (ctypes.c_char_p, []),
}


def lib() -> ctypes.CDLL:
    """The loaded library; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m decode_attention_13_amd.build`")
        handle = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(handle, name)
            fn.restype = res
            fn.argtypes = args
        _lib = handle
    return _lib


def _check(status: int) -> None:
    if status != 0:
        L = lib()
        raise FdError(status, L.fd_status_string(status).decode(), L.fd_last_error().decode())


def options(force_num_splits: int = 0, force_chunk: int = 0, kernel: str | int = "auto",
            split_begin_event=None, split_end_event=None, debug_checks: bool | int = False,
            merge: str | int = "auto", launch: str | int = "auto") -> FdOptions:
    """An ``fd_options`` block; events are ``torch.cuda.Event`` objects (or raw handles).
    ``debug_checks``: paged calls check the block table and lengths on the device and
    raise ``FdError`` (FD_ERR_BAD_DATA) on an out-of-range value (the call synchronises).
    ``merge``: "kernel" (a merge kernel), "fused" (the last workgroups merge) or "auto".
    ``launch`` (paged calls): "grid" (a workgroup per item), "persistent" (a workgroup per
    resident slot claiming items) or "auto"."""
    def handle(ev):
        if ev is None:
            return None
        return ev.cuda_event if hasattr(ev, "cuda_event") else int(ev)
    k = KERNELS[kernel] if isinstance(kernel, str) else int(kernel)
    mg = MERGES[merge] if isinstance(merge, str) else int(merge)
    ln = LAUNCHES[launch] if isinstance(launch, str) else int(launch)
    return FdOptions(int(force_num_splits), int(force_chunk), k, int(debug_checks), handle(split_begin_event),
                     handle(split_end_event), mg, ln)


def _opt_ptr(opt):
    return ctypes.byref(opt) if opt is not None else None


def _dtype_code(dt) -> int:
    """fd_dtype code of a torch dtype, a name ("bf16", "f16_kv_e4m3", ...) or a code."""
    if isinstance(dt, int):
        return dt
    if isinstance(dt, str):
        if dt in FP8_CODES:
            return FP8_CODES[dt]
        dt = DTYPE_NAMES[dt]
    if dt not in FD_DTYPE:
        raise TypeError(f"unsupported dtype {dt}")
    return FD_DTYPE[dt]


def _fp8_code(q_dtype) -> int:
    if q_dtype not in FD_DTYPE_KV_E4M3:
        raise TypeError(f"an FP8 cache needs f16 or bf16 queries, not {q_dtype}")
    return FD_DTYPE_KV_E4M3[q_dtype]


def device_num_cus() -> int:
    return int(lib().fd_device_num_cus())


def decode_plan(H: int, Hkv: int, S: int, dtype, num_cus: int = 0, opt: FdOptions | None = None) -> dict:
    p = FdPlan()
    _check(lib().fd_decode_plan(H, Hkv, S, HEAD_DIM, _dtype_code(dtype), num_cus, _opt_ptr(opt), ctypes.byref(p)))
    return p.as_dict()


def paged_plan(B: int, H: int, Hkv: int, dtype, page_size: int, max_seq_len: int, total_kv: int = 0,
               num_cus: int = 0, opt: FdOptions | None = None) -> dict:
    p = FdPlan()
    _check(lib().fd_paged_plan(B, H, Hkv, HEAD_DIM, _dtype_code(dtype), page_size, max_seq_len, total_kv, num_cus,
                               _opt_ptr(opt), ctypes.byref(p)))
    return p.as_dict()


def decode_workspace_size(H: int, Hkv: int, S: int, dtype, num_cus: int = 0, opt: FdOptions | None = None) -> int:
    n = ctypes.c_size_t(0)
    _check(lib().fd_decode_workspace_size(H, Hkv, S, HEAD_DIM, _dtype_code(dtype), num_cus, _opt_ptr(opt),
                                          ctypes.byref(n)))
    return int(n.value)


def paged_workspace_size(B: int, H: int, Hkv: int, dtype, page_size: int, max_seq_len: int, total_kv: int = 0,
                         num_cus: int = 0, opt: FdOptions | None = None) -> int:
    n = ctypes.c_size_t(0)
    _check(lib().fd_paged_workspace_size(B, H, Hkv, HEAD_DIM, _dtype_code(dtype), page_size, max_seq_len, total_kv,
                                         num_cus, _opt_ptr(opt), ctypes.byref(n)))
    return int(n.value)


def _stream_handle(stream, *owned) -> int | None:
    """The HIP stream handle of ``stream`` (default: the current stream). ``owned`` are
    tensors this call allocated (and the workspace zero-filled) on the current stream:
    when the library runs on another stream, that stream first waits for the current
    one, and the allocator keeps their memory until the other stream's work is done."""
    cur = torch.cuda.current_stream()
    if stream is None:
        return cur.cuda_stream
    s = stream if hasattr(stream, "cuda_stream") else torch.cuda.ExternalStream(int(stream))
    owned = [t for t in owned if t is not None]
    if owned and s.cuda_stream != cur.cuda_stream:
        s.wait_stream(cur)
        for t in owned:
            t.record_stream(s)
    return s.cuda_stream


def _require(t: torch.Tensor, name: str, dtype=None) -> None:
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} has dtype {t.dtype}, expected {dtype}")


def new_workspace(nbytes: int, device) -> torch.Tensor:
    """A workspace of ``nbytes`` (uint8) whose counter block is zero, as every call
    needs it on first use (the rest is never read before it is written)."""
    return torch.zeros(max(int(nbytes), 1), dtype=torch.uint8, device=device)


def _workspace(ws, need: int, device) -> tuple[int, int, torch.Tensor | None]:
    if need == 0:
        return (ws.data_ptr() if ws is not None else 0), (ws.numel() * ws.element_size() if ws is not None else 0), None
    if ws is None:
        ws = new_workspace(need, device)
    return ws.data_ptr(), ws.numel() * ws.element_size(), ws


def _single_args(q, k, v, o, kv_dtype):
    H, D = q.shape
    S, Hkv, Dk = k.shape
    if v.shape != k.shape or Dk != D:
        raise ValueError("k and v must both be [S, Hkv, D] with q's D")
    _require(q, "q", q.dtype)
    for t, n in ((k, "k"), (v, "v")):
        _require(t, n, kv_dtype)
    if o is None:
        o = torch.empty_like(q)
    _require(o, "o", q.dtype)
    if o.shape != q.shape:
        raise ValueError("o must have q's shape")
    return H, Hkv, S, D, o


def fd_decode(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, o: torch.Tensor | None = None,
              scale: float | None = None, ws: torch.Tensor | None = None, opt: FdOptions | None = None,
              stream=None) -> torch.Tensor:
    """Single decode over a contiguous cache: q [H, D], k/v [S, Hkv, D] -> o [H, D]."""
    o_new = o is None
    H, Hkv, S, D, o = _single_args(q, k, v, o, q.dtype)
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    dt = _dtype_code(q.dtype)
    plan = decode_plan(H, Hkv, S, dt, 0, opt)
    wp, wb, _keep = _workspace(ws, plan["workspace_bytes"], q.device)
    st = _stream_handle(stream, o if o_new else None, _keep if ws is None else None)
    _check(lib().fd_decode(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), H, Hkv, S, D, dt, float(scale),
                           wp or None, wb, _opt_ptr(opt), st))
    return o


def _fp8_cache_dtype(t: torch.Tensor, name: str) -> torch.dtype:
    if t.dtype not in FP8_CACHE_DTYPES:
        raise TypeError(f"{name} must hold E4M3 codes (float8_e4m3fn or uint8), not {t.dtype}")
    return t.dtype


def fd_decode_fp8kv(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, k_scale: float, v_scale: float,
                    o: torch.Tensor | None = None, scale: float | None = None, ws: torch.Tensor | None = None,
                    opt: FdOptions | None = None, stream=None) -> torch.Tensor:
    """Single decode over an FP8 E4M3 cache: K = k_scale * E4M3(k), V = v_scale * E4M3(v);
    q [H, D] f16/bf16, k/v [S, Hkv, D] codes -> o [H, D] in q's dtype."""
    o_new = o is None
    H, Hkv, S, D, o = _single_args(q, k, v, o, _fp8_cache_dtype(k, "k"))
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    dt = _fp8_code(q.dtype)
    plan = decode_plan(H, Hkv, S, dt, 0, opt)
    wp, wb, _keep = _workspace(ws, plan["workspace_bytes"], q.device)
    st = _stream_handle(stream, o if o_new else None, _keep if ws is None else None)
    _check(lib().fd_decode_fp8kv(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), H, Hkv, S, D, dt,
                                 float(scale), float(k_scale), float(v_scale), wp or None, wb, _opt_ptr(opt), st))
    return o


def _paged_args(q, k_cache, v_cache, block_table, seq_lens, page_size, o, max_seq_len, kv_dtype):
    B, H, D = q.shape
    num_pages, ps, Hkv, Dk = k_cache.shape
    if page_size is None:
        page_size = ps
    if v_cache.shape != k_cache.shape or Dk != D or ps != page_size:
        raise ValueError("k_cache and v_cache must both be [num_pages, page_size, Hkv, D]")
    _require(q, "q", q.dtype)
    for t, n in ((k_cache, "k_cache"), (v_cache, "v_cache")):
        _require(t, n, kv_dtype)
    _require(block_table, "block_table", torch.int32)
    _require(seq_lens, "seq_lens", torch.int32)
    if block_table.dim() != 2 or block_table.shape[0] != B or seq_lens.shape != (B,):
        raise ValueError("block_table must be [B, max_blocks] and seq_lens [B]")
    if o is None:
        o = torch.empty_like(q)
    _require(o, "o", q.dtype)
    if max_seq_len is None:
        max_seq_len = int(seq_lens.max().item()) if B > 0 else 0
    return B, H, Hkv, D, num_pages, page_size, block_table.shape[1], int(max_seq_len), o


def fd_paged_decode(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor, block_table: torch.Tensor,
                    seq_lens: torch.Tensor, page_size: int | None = None, o: torch.Tensor | None = None,
                    scale: float | None = None, max_seq_len: int | None = None, total_kv: int = 0,
                    ws: torch.Tensor | None = None, opt: FdOptions | None = None, stream=None) -> torch.Tensor:
    """Batched paged GQA decode: q [B, H, D], caches [num_pages, page_size, Hkv, D],
    block_table [B, max_blocks] int32, seq_lens [B] int32 -> o [B, H, D].

    ``max_seq_len`` must bound every entry of ``seq_lens``; if omitted it is read
    from the device (a synchronising copy).
    """
    o_new = o is None
    B, H, Hkv, D, num_pages, page_size, max_blocks, max_seq_len, o = _paged_args(
        q, k_cache, v_cache, block_table, seq_lens, page_size, o, max_seq_len, q.dtype)
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    dt = _dtype_code(q.dtype)
    eff_max = min(max_seq_len, max_blocks * page_size)
    plan = paged_plan(B, H, Hkv, dt, page_size, eff_max, int(total_kv), 0, opt)
    wp, wb, _keep = _workspace(ws, plan["workspace_bytes"], q.device)
    st = _stream_handle(stream, o if o_new else None, _keep if ws is None else None)
    _check(lib().fd_paged_decode(q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(), block_table.data_ptr(),
                                 seq_lens.data_ptr(), page_size, o.data_ptr(), float(scale), B, H, Hkv, D,
                                 num_pages, max_blocks, max_seq_len, int(total_kv), dt, wp or None, wb,
                                 _opt_ptr(opt), st))
    return o


def fd_paged_decode_noalloc(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor, block_table: torch.Tensor,
                            seq_lens: torch.Tensor, page_size: int | None = None, o: torch.Tensor | None = None,
                            scale: float | None = None, max_seq_len: int | None = None, total_kv: int = 0,
                            opt: FdOptions | None = None, stream=None) -> torch.Tensor:
    """``fd_paged_decode`` on the library's static per-GPU scratch (no workspace is
    allocated); calls that overlap on one GPU race on that scratch."""
    o_new = o is None
    B, H, Hkv, D, num_pages, page_size, max_blocks, max_seq_len, o = _paged_args(
        q, k_cache, v_cache, block_table, seq_lens, page_size, o, max_seq_len, q.dtype)
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    st = _stream_handle(stream, o if o_new else None)
    _check(lib().fd_paged_decode_noalloc(q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(), block_table.data_ptr(),
                                         seq_lens.data_ptr(), page_size, o.data_ptr(), float(scale), B, H, Hkv, D,
                                         num_pages, max_blocks, max_seq_len, int(total_kv), _dtype_code(q.dtype),
                                         _opt_ptr(opt), st))
    return o


def fd_paged_decode_fp8kv(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor, block_table: torch.Tensor,
                          seq_lens: torch.Tensor, k_scale: float, v_scale: float, page_size: int | None = None,
                          o: torch.Tensor | None = None, scale: float | None = None, max_seq_len: int | None = None,
                          total_kv: int = 0, ws: torch.Tensor | None = None, opt: FdOptions | None = None,
                          stream=None) -> torch.Tensor:
    """Batched paged GQA decode over FP8 E4M3 caches (codes as float8_e4m3fn or uint8)
    with per-tensor scales; otherwise as ``fd_paged_decode``."""
    o_new = o is None
    B, H, Hkv, D, num_pages, page_size, max_blocks, max_seq_len, o = _paged_args(
        q, k_cache, v_cache, block_table, seq_lens, page_size, o, max_seq_len, _fp8_cache_dtype(k_cache, "k_cache"))
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    dt = _fp8_code(q.dtype)
    eff_max = min(max_seq_len, max_blocks * page_size)
    plan = paged_plan(B, H, Hkv, dt, page_size, eff_max, int(total_kv), 0, opt)
    wp, wb, _keep = _workspace(ws, plan["workspace_bytes"], q.device)
    st = _stream_handle(stream, o if o_new else None, _keep if ws is None else None)
    _check(lib().fd_paged_decode_fp8kv(q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(), block_table.data_ptr(),
                                       seq_lens.data_ptr(), page_size, o.data_ptr(), float(scale), float(k_scale),
                                       float(v_scale), B, H, Hkv, D, num_pages, max_blocks, max_seq_len,
                                       int(total_kv), dt, wp or None, wb, _opt_ptr(opt), st))
    return o


def prefill_workspace_size(B: int, N: int, Hkv: int, dtype) -> int:
    """Bytes fd_prefill's workspace needs (bf16: the f16 copy of V and the flag rows; 0 for f16)."""
    code = dtype if isinstance(dtype, int) else _dtype_code(dtype)
    return int(lib().fd_prefill_workspace_size(B, N, Hkv, HEAD_DIM, code))


def prefill_flags(ws: torch.Tensor, B: int, N: int, Hkv: int) -> torch.Tensor:
    """[B, 1024] uint8 view of a bf16 prefill workspace's flag rows (1: that chunk of the
    sequence's V held a finite value of 65536 or more, so the sequence took the split-P path)."""
    off = B * N * Hkv * HEAD_DIM * 2
    return ws[off: off + B * 1024].view(B, 1024)


def fd_prefill(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, o: torch.Tensor | None = None,
               scale: float | None = None, causal: bool = True, opt: FdOptions | None = None,
               stream=None, ws: torch.Tensor | bool | None = None) -> torch.Tensor:
    """Prefill attention: q [B, N, H, D], k/v [B, N, Hkv, D] (f16/bf16) -> o [B, N, H, D];
    causal: query i sees keys 0..i. bf16: ws None allocates the workspace of the f16-V
    path (uninitialised; the library writes it before reading), a tensor is used as the
    workspace, False passes none (the split-P path)."""
    B, N, H, D = q.shape
    if k.dim() != 4 or k.shape[0] != B or k.shape[1] != N or k.shape[3] != D or v.shape != k.shape:
        raise ValueError("k and v must both be [B, N, Hkv, D] with q's B, N and D")
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        _require(t, n, q.dtype)
    o_new = o is None
    if o_new:
        o = torch.empty_like(q)
    _require(o, "o", q.dtype)
    if o.shape != q.shape:
        raise ValueError("o must have q's shape")
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    Hkv = k.shape[2]
    wp, wb, ws_new = None, 0, None
    if ws is not False:
        need = prefill_workspace_size(B, N, Hkv, q.dtype)
        if need and ws is None:
            ws = ws_new = torch.empty(need, dtype=torch.uint8, device=q.device)
        if isinstance(ws, torch.Tensor):
            _require(ws, "ws", torch.uint8)
            wp, wb = ws.data_ptr(), ws.numel()
    st = _stream_handle(stream, o if o_new else None, ws_new)
    _check(lib().fd_prefill(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), B, N, H, Hkv, D,
                            _dtype_code(q.dtype), float(scale), 1 if causal else 0, wp, wb, _opt_ptr(opt), st))
    return o


def workspace_views(ws: torch.Tensor, plan: dict, B: int, H: int) -> tuple[torch.Tensor, torch.Tensor]:
    """(ws_o [B, H, num_splits, D], ws_lse [B, H, num_splits]) float32 views of a workspace."""
    n = plan["num_splits"]
    rows = B * H * n
    o0 = plan["ws_o_offset"]
    o = ws[o0: o0 + rows * HEAD_DIM * 4].view(torch.float32).view(B, H, n, HEAD_DIM)
    off = plan["ws_lse_offset"]
    lse = ws[off: off + rows * 4].view(torch.float32).view(B, H, n)
    return o, lse
