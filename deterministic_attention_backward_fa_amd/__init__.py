"""Python binding of libdetattn (include/detattn.h): argument marshalling only.

Every step of the attention backward runs in the HIP library's own kernels;
PyTorch only allocates device memory and supplies the current stream. The
functions mirror the C entry points by name. If the library is not built, the
first call raises: there is no fallback path.
"""
import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libdetattn.so")

MASKS = {"full": 0, "causal": 1}
SCHEDULES = {"serial_ascending": 0, "descending_q": 1, "shift": 2, "symmetric_shift": 3, "atomic_nondet": 4,
             "auto": 5}
SCHEDULE_NAMES = {v: k for k, v in SCHEDULES.items()}
DQ_MODES = {"default": 0, "rmw": 1, "atomic": 2, "xcd_local": 3}
DISPATCH = {"default": 0, "ticket": 1, "ring": 2}
STATUS = {0: "OK", 1: "ERR_INVALID_ARG", 2: "ERR_UNSUPPORTED", 3: "ERR_WORKSPACE", 4: "ERR_HIP",
          5: "ERR_DEVICE_TIMEOUT", 6: "ERR_DEVICE_PLACEMENT (not returned any more)", 7: "ERR_SCRATCH_LIMIT"}
NOALLOC_SCRATCH_BYTES = 136 << 20  # DETATTN_NOALLOC_SCRATCH_BYTES


class DetAttnError(RuntimeError):
    def __init__(self, status, what):
        self.status = status
        super().__init__(f"{what}: {STATUS.get(status, status)} ({status_string(status)})")


class Shape(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int32), ("H", ctypes.c_int32), ("S", ctypes.c_int32), ("D", ctypes.c_int32),
                ("softmax_scale", ctypes.c_float)]


class BwdOptions(ctypes.Structure):
    _fields_ = [("block_q", ctypes.c_int32), ("block_kv", ctypes.c_int32), ("grid", ctypes.c_int32),
                ("xcd_remap", ctypes.c_int32), ("dq_mode", ctypes.c_int32), ("debug_delay_seed", ctypes.c_uint32),
                ("timeout_us", ctypes.c_uint32), ("debug_skip_signal", ctypes.c_int32),
                ("main_begin_event", ctypes.c_void_p), ("main_end_event", ctypes.c_void_p),
                ("trace", ctypes.c_void_p), ("trace_records", ctypes.c_int32), ("ring_size", ctypes.c_int32),
                ("dispatch", ctypes.c_int32), ("pair_columns", ctypes.c_int32),
                ("cooperative_launch", ctypes.c_int32), ("debug_misplace", ctypes.c_int32)]


class Plan(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in ("block_q", "block_kv", "n_q", "n_kv", "items", "grid", "ring", "rings",
                                              "dq_mode", "cooperative", "schedule", "pair_columns")]

    def as_dict(self):
        return {n: getattr(self, n) for n, _ in self._fields_}


_lib = None


def lib():
    """The loaded libdetattn (raises if it was never built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m deterministic_attention_backward_fa_amd.build` (no fallback exists)")
        L = ctypes.CDLL(LIB_PATH)
        vp, i32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
        L.detattn_fwd.argtypes = [vp, vp, vp, vp, vp, Shape, ctypes.c_int, vp]
        L.detattn_fwd.restype = ctypes.c_int
        L.detattn_bwd_workspace_bytes.argtypes = [Shape, ctypes.c_int, ctypes.c_int]
        L.detattn_bwd_workspace_bytes.restype = sz
        bwd_args = [vp] * 9 + [vp, sz, Shape, ctypes.c_int, ctypes.c_int]
        L.attn_bwd_deterministic.argtypes = bwd_args + [vp]
        L.attn_bwd_deterministic.restype = ctypes.c_int
        L.attn_bwd_deterministic_ex.argtypes = bwd_args + [ctypes.POINTER(BwdOptions), vp]
        L.attn_bwd_deterministic_ex.restype = ctypes.c_int
        L.attn_bwd_deterministic_noalloc.argtypes = [vp] * 9 + [Shape, ctypes.c_int, ctypes.c_int, vp]
        L.attn_bwd_deterministic_noalloc.restype = ctypes.c_int
        L.detattn_xcd_handoff.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, vp, vp, vp]
        L.detattn_xcd_handoff.restype = ctypes.c_int
        L.detattn_bwd_plan.argtypes = [Shape, ctypes.c_int, ctypes.c_int, ctypes.POINTER(BwdOptions),
                                       ctypes.POINTER(Plan)]
        L.detattn_bwd_plan.restype = ctypes.c_int
        L.detattn_device_status.argtypes = [vp, vp]
        L.detattn_device_status.restype = ctypes.c_int
        L.detattn_status_string.argtypes = [ctypes.c_int]
        L.detattn_status_string.restype = ctypes.c_char_p
        ip = ctypes.POINTER(ctypes.c_int32)
        L.detattn_schedule_item.argtypes = [i32, i32, i32, i32, i32, ip, ip, ip, i32]
        L.detattn_schedule_item.restype = ctypes.c_int
        L.detattn_schedule_item_ring.argtypes = [i32, i32, i32, i32, i32, i32, ip, ip, ip, i32]
        L.detattn_schedule_item_ring.restype = ctypes.c_int
        L.detattn_schedule_items_per_head.argtypes = [i32, i32, i32, i32]
        L.detattn_schedule_items_per_head.restype = ctypes.c_int
        _lib = L
    return _lib


def status_string(status: int) -> str:
    return lib().detattn_status_string(int(status)).decode()


detattn_status_string = status_string


def _shape(q, scale):
    B, H, S, D = q.shape
    return Shape(B, H, S, D, float(scale if scale is not None else D ** -0.5))


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else ctypes.c_void_p(0)


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _check_tensor(name, t, dtype, shape):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be a device tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _options(block_q=0, block_kv=0, grid=0, xcd_remap=None, dq_mode="default", debug_delay_seed=0, timeout_us=0,
             debug_skip_signal=0, main_begin_event=None, main_end_event=None, trace=None, trace_records=0,
             ring_size=0, dispatch="default", pair_columns=False, cooperative_launch=False, debug_misplace=False):
    xr = 0 if xcd_remap is None else (1 if xcd_remap else 2)
    return BwdOptions(int(block_q), int(block_kv), int(grid), xr, DQ_MODES[dq_mode], int(debug_delay_seed),
                      int(timeout_us), int(debug_skip_signal), main_begin_event, main_end_event,
                      trace.data_ptr() if trace is not None else None, int(trace_records), int(ring_size),
                      DISPATCH[dispatch], 1 if pair_columns else 0, 1 if cooperative_launch else 0,
                      1 if debug_misplace else 0)


def detattn_fwd(q, k, v, causal=False, scale=None, out=None, lse=None, stream=None):
    """O (bf16) and LSE (fp32, natural log) for bf16 q, k, v of shape [B,H,S,D]."""
    B, H, S, D = q.shape
    for n, t in (("q", q), ("k", k), ("v", v)):
        _check_tensor(n, t, torch.bfloat16, (B, H, S, D))
    o = out if out is not None else torch.empty_like(q)
    lse = lse if lse is not None else torch.empty((B, H, S), dtype=torch.float32, device=q.device)
    st = lib().detattn_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _shape(q, scale), MASKS[
        "causal" if causal else "full"], _stream(stream))
    if st != 0:
        raise DetAttnError(st, "detattn_fwd")
    return o, lse


def detattn_bwd_workspace_bytes(B, H, S, D, causal=False, schedule="serial_ascending"):
    return int(lib().detattn_bwd_workspace_bytes(Shape(B, H, S, D, 1.0), MASKS["causal" if causal else "full"],
                                                 SCHEDULES[schedule]))


def detattn_bwd_plan(B, H, S, D, causal=False, schedule="serial_ascending", **opts):
    plan = Plan()
    st = lib().detattn_bwd_plan(Shape(B, H, S, D, 1.0), MASKS["causal" if causal else "full"], SCHEDULES[schedule],
                                ctypes.byref(_options(**opts)), ctypes.byref(plan))
    if st != 0:
        raise DetAttnError(st, "detattn_bwd_plan")
    return plan.as_dict()


def alloc_workspace(B, H, S, D, device="cuda"):
    """A workspace tensor of the size the library asks for (256-byte aligned by the caching allocator)."""
    n = detattn_bwd_workspace_bytes(B, H, S, D)
    return torch.empty(n, dtype=torch.uint8, device=device)


def attn_bwd_deterministic(q, k, v, o, dout, lse, causal=False, schedule="serial_ascending", scale=None,
                           workspace=None, out=None, stream=None, check=False, **opts):
    """dQ, dK, dV (bf16) of softmax attention. `opts` are BwdOptions fields
    (block_q, block_kv, grid, xcd_remap, dq_mode, debug_delay_seed, timeout_us, debug_skip_signal, ring_size, dispatch,
    pair_columns, cooperative_launch, debug_misplace).
    check=True synchronises the stream after the call and raises DetAttnError if the
    workspace's device status reports an error (detattn_device_status)."""
    B, H, S, D = q.shape
    for n, t in (("q", q), ("k", k), ("v", v), ("o", o), ("dout", dout)):
        _check_tensor(n, t, torch.bfloat16, (B, H, S, D))
    _check_tensor("lse", lse, torch.float32, (B, H, S))
    if out is None:
        out = (torch.empty_like(q), torch.empty_like(k), torch.empty_like(v))
    dq, dk, dv = out
    for n, t in (("dq", dq), ("dk", dk), ("dv", dv)):
        _check_tensor(n, t, torch.bfloat16, (B, H, S, D))
    if workspace is None:
        workspace = alloc_workspace(B, H, S, D, q.device)
    shape = _shape(q, scale)
    mask = MASKS["causal" if causal else "full"]
    args = [_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(dout), _ptr(lse), _ptr(dq), _ptr(dk), _ptr(dv),
            _ptr(workspace), ctypes.c_size_t(workspace.numel() * workspace.element_size()), shape, mask,
            SCHEDULES[schedule]]
    if opts:
        st = lib().attn_bwd_deterministic_ex(*args, ctypes.byref(_options(**opts)), _stream(stream))
    else:
        st = lib().attn_bwd_deterministic(*args, _stream(stream))
    if st != 0:
        raise DetAttnError(st, f"attn_bwd_deterministic({schedule})")
    if check:
        st = detattn_device_status(workspace, stream)
        if st != 0:
            raise DetAttnError(st, f"attn_bwd_deterministic({schedule}) on the device")
    return dq, dk, dv


def attn_bwd_deterministic_noalloc(q, k, v, o, dout, lse, causal=False, schedule="serial_ascending", scale=None,
                                   out=None, stream=None):
    """attn_bwd_deterministic on the library's fixed per-GPU scratch (no workspace;
    the C entry point allocates nothing). `out` = (dq, dk, dv) is allocated here
    only when not given."""
    B, H, S, D = q.shape
    for n, t in (("q", q), ("k", k), ("v", v), ("o", o), ("dout", dout)):
        _check_tensor(n, t, torch.bfloat16, (B, H, S, D))
    _check_tensor("lse", lse, torch.float32, (B, H, S))
    if out is None:
        out = (torch.empty_like(q), torch.empty_like(k), torch.empty_like(v))
    dq, dk, dv = out
    for n, t in (("dq", dq), ("dk", dk), ("dv", dv)):
        _check_tensor(n, t, torch.bfloat16, (B, H, S, D))
    st = lib().attn_bwd_deterministic_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(dout), _ptr(lse), _ptr(dq),
                                              _ptr(dk), _ptr(dv), _shape(q, scale),
                                              MASKS["causal" if causal else "full"], SCHEDULES[schedule],
                                              _stream(stream))
    if st != 0:
        raise DetAttnError(st, f"attn_bwd_deterministic_noalloc({schedule})")
    return dq, dk, dv


def detattn_device_status(workspace, stream=None) -> int:
    """Status word of `workspace` (None: the no-alloc scratch of the current device)."""
    return int(lib().detattn_device_status(_ptr(workspace), _stream(stream)))


def detattn_schedule_item(schedule, causal, n_q, n_kv, item, ring=0):
    """[(q_tile, kv_tile, rank), ...] of one item, from the library's own schedule
    functions; `ring` = workgroups per ring of the shift schedules (0 = one round)."""
    mask = 1 if causal else 0
    n = lib().detattn_schedule_item_ring(SCHEDULES[schedule], mask, n_q, n_kv, ring, item, None, None, None, 0)
    if n < 0:
        raise DetAttnError(1, "detattn_schedule_item_ring")
    arr = (ctypes.c_int32 * max(n, 1))
    qi, kj, rk = arr(), arr(), arr()
    lib().detattn_schedule_item_ring(SCHEDULES[schedule], mask, n_q, n_kv, ring, item, qi, kj, rk, n)
    return [(qi[t], kj[t], rk[t]) for t in range(n)]


def detattn_schedule_items_per_head(schedule, causal, n_q, n_kv):
    return int(lib().detattn_schedule_items_per_head(SCHEDULES[schedule], 1 if causal else 0, n_q, n_kv))


def detattn_xcd_handoff(wg_a, wg_b, round_trips=4096, device="cuda"):
    """Round-trip latency of a device-scope flag passed between workgroups wg_a
    and wg_b (the ordered dQ hand-off's mechanism): {"ns", "cycles" per round
    trip, "xcd_a", "xcd_b", "timed_out"}. Synchronises the current stream."""
    scratch = torch.empty(256, dtype=torch.uint8, device=device)
    out = torch.zeros(5, dtype=torch.int64, device=device)
    st = lib().detattn_xcd_handoff(int(wg_a), int(wg_b), int(round_trips), _ptr(scratch), _ptr(out), _stream(None))
    if st != 0:
        raise DetAttnError(st, "detattn_xcd_handoff")
    torch.cuda.synchronize()
    r = out.cpu().tolist()
    n = round_trips - 1
    return {"ns": r[0] * 10.0 / n, "cycles": r[1] / n, "xcd_a": r[2], "xcd_b": r[3], "timed_out": bool(r[4])}
