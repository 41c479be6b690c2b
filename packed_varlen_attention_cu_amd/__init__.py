"""Python binding of the libra C ABI (``include/libra.h``).

Argument marshalling only: every step of the planner and of the attention
pass runs in the native library ``_lib/liblibra.so``.  Functions named
``libra_*`` mirror the C entry points one to one; ``Plan``, ``attn_fwd`` and
``attn_bwd`` are conveniences that allocate outputs with torch (which is
used for device memory and streams only).  Importing this package fails
loudly if the library has not been built.
"""
from __future__ import annotations

import ctypes
import math
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
# LIBRA_LIB may name another build of the same library (e.g. one compiled
# with different tuning macros); by default the in-tree build is loaded.
LIB_PATH = os.environ.get("LIBRA_LIB") or os.path.join(_HERE, "_lib", "liblibra.so")

LIBRA_OK, LIBRA_EINVAL, LIBRA_ESIZE, LIBRA_EUNSUPPORTED, LIBRA_EHIP, LIBRA_EHOST = 0, -1, -2, -3, -4, -5
ASSIGN_PLACER, ASSIGN_ROUND_ROBIN, ASSIGN_PLACER_L2 = 0, 1, 2
COST_EXECUTED, COST_PAIRS = 0, 1
QUEUE_FWD, QUEUE_DQ, QUEUE_KV = 0, 1, 2
PLAN_MAGIC, PLAN_VERSION = 0x4152424C, 5
RECORD_PLAN_MISMATCH = 1
RECORD_WAIT_EXPIRED = 2


class LibraError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        detail = f" [{libra_last_hip_error()}]" if status == LIBRA_EHIP else ""
        super().__init__(f"{what}: {libra_status_str(status)} ({status}){detail}")


class PlanParams(ctypes.Structure):
    _fields_ = [("total_tokens", ctypes.c_int32), ("num_samples", ctypes.c_int32),
                ("h_q", ctypes.c_int32), ("h_kv", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("tile_tokens", ctypes.c_int32), ("tile_heads", ctypes.c_int32),
                ("num_cus", ctypes.c_int32), ("tau", ctypes.c_float), ("assign", ctypes.c_int32),
                ("item_overhead", ctypes.c_int64), ("worker_speed", ctypes.c_uint16 * 8),
                ("cost", ctypes.c_int32), ("reserved", ctypes.c_int32)]


class PlanInfo(ctypes.Structure):
    _fields_ = [("magic", ctypes.c_uint32), ("version", ctypes.c_uint32), ("bytes", ctypes.c_uint64),
                ("params", PlanParams), ("num_cus", ctypes.c_int32), ("n_tiles", ctypes.c_int32),
                ("n_items", ctypes.c_int32), ("n_dq_items", ctypes.c_int32), ("n_kv_items", ctypes.c_int32),
                ("reserved", ctypes.c_int32),
                ("total_pairs", ctypes.c_int64), ("load_max", ctypes.c_int64),
                ("load_sum", ctypes.c_int64), ("dq_load_max", ctypes.c_int64),
                ("dq_load_sum", ctypes.c_int64), ("kv_load_max", ctypes.c_int64),
                ("kv_load_sum", ctypes.c_int64), ("off_tiles", ctypes.c_uint64),
                ("off_items", ctypes.c_uint64), ("off_cu_off", ctypes.c_uint64),
                ("off_dq_items", ctypes.c_uint64), ("off_dq_cu_off", ctypes.c_uint64),
                ("off_kv_items", ctypes.c_uint64), ("off_kv_cu_off", ctypes.c_uint64),
                ("checksum", ctypes.c_uint64)]


TILE_DTYPE = np.dtype([("tile_id", "<i4"), ("block", "<i4"), ("shard", "<i4"), ("tok_begin", "<i4"),
                       ("tok_end", "<i4"), ("head_begin", "<i4"), ("head_count", "<i4"),
                       ("sample_first", "<i4"), ("sample_last", "<i4"), ("n_items", "<i4"),
                       ("pairs", "<i8")])
ITEM_DTYPE = np.dtype([("row0", "<i4"), ("nrows", "<i4"), ("kv_head", "<i4"), ("head0", "<i4"),
                       ("nheads", "<i4"), ("tile_id", "<i4"), ("id", "<i4"), ("flags", "<i4"),
                       ("cost", "<i8"), ("pairs", "<i8")])
RECORD_DTYPE = np.dtype([("hw_id", "<u4"), ("xcc_id", "<u4"), ("n_items", "<u4"), ("flags", "<u4"),
                         ("t_start", "<u8"), ("t_end", "<u8")])

assert ctypes.sizeof(PlanParams) == 72 and ctypes.sizeof(PlanInfo) == 232
assert TILE_DTYPE.itemsize == 48 and ITEM_DTYPE.itemsize == 48 and RECORD_DTYPE.itemsize == 32


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with "
                          "`python packed_varlen_attention_cu_amd/build.py`")
    # torch ships its own HIP runtime under the same soname as the system one.
    # Loading torch first makes the dynamic loader resolve this library's HIP
    # dependency to that already-loaded runtime, so the process holds exactly
    # one HIP runtime and torch's device pointers and streams are valid here.
    # (Loaded the other way round, two runtimes coexist and the second one
    # does not see the device.)
    import torch  # noqa: F401
    lib = ctypes.CDLL(LIB_PATH)
    vp, sz = ctypes.c_void_p, ctypes.c_size_t
    lib.libra_plan.argtypes = [vp, ctypes.POINTER(PlanParams), vp, ctypes.POINTER(sz)]
    lib.libra_plan_check.argtypes = [vp, sz, ctypes.POINTER(PlanInfo)]
    lib.libra_attn_bwd_workspace.argtypes = [vp, ctypes.POINTER(sz)]
    lib.libra_attn_fwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, ctypes.c_float, vp, vp]
    lib.libra_attn_bwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, ctypes.c_float,
                                   vp, sz, vp, vp]
    lib.libra_attn_bwd_noalloc.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, ctypes.c_float, vp, vp]
    lib.libra_attn_bwd_prepare.argtypes = [vp, vp, vp, vp, vp, sz, vp]
    lib.libra_attn_bwd_dkdv.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, ctypes.c_float, vp, sz, vp, vp]
    lib.libra_attn_bwd_dq.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, ctypes.c_float, vp, sz, vp, vp]
    lib.libra_device_clock_khz.argtypes = [ctypes.POINTER(ctypes.c_int32)]
    lib.libra_status_str.argtypes = [ctypes.c_int]
    lib.libra_status_str.restype = ctypes.c_char_p
    lib.libra_last_hip_error.argtypes = []
    lib.libra_last_hip_error.restype = ctypes.c_char_p
    lib.libra_pack_workload.argtypes = [vp, ctypes.c_int32, vp]
    lib.libra_vrsp.argtypes = [vp, ctypes.c_int32, ctypes.c_int32, vp, vp, vp]
    lib.libra_worker_speed.argtypes = [vp, ctypes.c_int32, vp, vp]
    for name in ("libra_plan", "libra_plan_check", "libra_attn_bwd_workspace", "libra_attn_fwd",
                 "libra_attn_bwd", "libra_device_clock_khz", "libra_attn_bwd_prepare", "libra_attn_bwd_dkdv",
                 "libra_attn_bwd_dq", "libra_pack_workload", "libra_vrsp", "libra_attn_bwd_noalloc",
                 "libra_worker_speed"):
        getattr(lib, name).restype = ctypes.c_int
    return lib


_lib = _load()


def _check(status: int, what: str):
    if status != LIBRA_OK:
        raise LibraError(status, what)


def _ptr(t):
    """Device/host address of a torch tensor or numpy array (None -> NULL)."""
    if t is None:
        return None
    if isinstance(t, np.ndarray):
        return t.ctypes.data
    return t.data_ptr()


# ----------------------------------------------------------------- C entry points
def libra_status_str(status: int) -> str:
    return _lib.libra_status_str(int(status)).decode()


def libra_last_hip_error() -> str:
    return _lib.libra_last_hip_error().decode()


def libra_plan(cu_seqlens, params: PlanParams) -> np.ndarray:
    """Build a plan; returns the host buffer as an 8-byte aligned uint8 array."""
    cu = np.ascontiguousarray(cu_seqlens, dtype=np.int32)
    need = ctypes.c_size_t(0)
    _check(_lib.libra_plan(cu.ctypes.data, ctypes.byref(params), None, ctypes.byref(need)), "libra_plan")
    words = np.empty((need.value + 7) // 8, dtype=np.uint64)   # the library fills every byte
    buf = words.view(np.uint8)[:need.value]
    cap = ctypes.c_size_t(need.value)
    _check(_lib.libra_plan(cu.ctypes.data, ctypes.byref(params), buf.ctypes.data, ctypes.byref(cap)),
           "libra_plan")
    return buf


def libra_pack_workload(cu_seqlens) -> int:
    """Workload proxy of one packed sequence: sum of squared sample lengths."""
    cu = np.ascontiguousarray(cu_seqlens, dtype=np.int32)
    out = ctypes.c_int64(0)
    _check(_lib.libra_pack_workload(cu.ctypes.data, len(cu) - 1, ctypes.byref(out)), "libra_pack_workload")
    return out.value


def libra_vrsp(workload, pool_size: int):
    """Variance-reduced sequence placement of one window: (pool_of, order, pool_load)."""
    f = np.ascontiguousarray(workload, dtype=np.int64)
    n = len(f)
    pool_of = np.empty(n, dtype=np.int32)
    order = np.empty(n, dtype=np.int32)
    pools = n // pool_size if pool_size > 0 else 0
    pool_load = np.empty(max(pools, 1), dtype=np.int64)
    _check(_lib.libra_vrsp(f.ctypes.data, n, pool_size, pool_of.ctypes.data, order.ctypes.data,
                           pool_load.ctypes.data), "libra_vrsp")
    return pool_of, order, pool_load[:pools]


def libra_worker_speed(plan_host: np.ndarray, queue: int, records) -> np.ndarray:
    """Speed of each worker class (worker mod 8), in thousandths of the mean, from the records of
    one completed launch of ``queue`` (QUEUE_FWD, QUEUE_DQ, QUEUE_KV) of this plan.  ``records``:
    host bytes or array holding the launch's num_cus records."""
    rec = np.ascontiguousarray(np.asarray(records).view(np.uint8))
    out = np.zeros(8, dtype=np.uint16)
    _check(_lib.libra_worker_speed(_ptr(plan_host), int(queue), rec.ctypes.data, out.ctypes.data),
           "libra_worker_speed")
    return out


def libra_plan_check(buf: np.ndarray) -> PlanInfo:
    info = PlanInfo()
    _check(_lib.libra_plan_check(buf.ctypes.data, buf.nbytes, ctypes.byref(info)), "libra_plan_check")
    return info


def libra_attn_bwd_workspace(plan_host: np.ndarray) -> int:
    n = ctypes.c_size_t(0)
    _check(_lib.libra_attn_bwd_workspace(plan_host.ctypes.data, ctypes.byref(n)), "libra_attn_bwd_workspace")
    return n.value


def libra_attn_fwd(plan_host, plan_dev, q, k, v, cu_seqlens_dev, o, lse, softmax_scale, records, stream):
    _check(_lib.libra_attn_fwd(_ptr(plan_host), _ptr(plan_dev), _ptr(q), _ptr(k), _ptr(v),
                               _ptr(cu_seqlens_dev), _ptr(o), _ptr(lse), float(softmax_scale),
                               _ptr(records), stream),
           "libra_attn_fwd")


def libra_attn_bwd(plan_host, plan_dev, q, k, v, o, dout, lse, cu_seqlens_dev, dq, dk, dv,
                   softmax_scale, workspace, workspace_bytes, records, stream):
    _check(_lib.libra_attn_bwd(_ptr(plan_host), _ptr(plan_dev), _ptr(q), _ptr(k), _ptr(v), _ptr(o),
                               _ptr(dout), _ptr(lse), _ptr(cu_seqlens_dev), _ptr(dq), _ptr(dk), _ptr(dv),
                               float(softmax_scale), _ptr(workspace), int(workspace_bytes),
                               _ptr(records), stream),
           "libra_attn_bwd")


NOALLOC_SCRATCH_BYTES = 64 << 20


def libra_attn_bwd_noalloc(plan_host, plan_dev, q, k, v, o, dout, lse, cu_seqlens_dev, dq, dk, dv,
                           softmax_scale, records, stream):
    _check(_lib.libra_attn_bwd_noalloc(_ptr(plan_host), _ptr(plan_dev), _ptr(q), _ptr(k), _ptr(v), _ptr(o),
                                       _ptr(dout), _ptr(lse), _ptr(cu_seqlens_dev), _ptr(dq), _ptr(dk),
                                       _ptr(dv), float(softmax_scale), _ptr(records), stream),
           "libra_attn_bwd_noalloc")


def libra_attn_bwd_prepare(plan_host, o, dout, lse, workspace, workspace_bytes, stream):
    _check(_lib.libra_attn_bwd_prepare(_ptr(plan_host), _ptr(o), _ptr(dout), _ptr(lse),
                                       _ptr(workspace), int(workspace_bytes), stream),
           "libra_attn_bwd_prepare")


def libra_attn_bwd_dkdv(plan_host, plan_dev, q, k, v, dout, lse, cu_seqlens_dev, dk, dv, softmax_scale,
                        workspace, workspace_bytes, records, stream):
    _check(_lib.libra_attn_bwd_dkdv(_ptr(plan_host), _ptr(plan_dev), _ptr(q), _ptr(k), _ptr(v), _ptr(dout),
                                    _ptr(lse), _ptr(cu_seqlens_dev), _ptr(dk), _ptr(dv), float(softmax_scale),
                                    _ptr(workspace), int(workspace_bytes), _ptr(records), stream),
           "libra_attn_bwd_dkdv")


def libra_attn_bwd_dq(plan_host, plan_dev, q, k, v, dout, lse, cu_seqlens_dev, dq, softmax_scale, workspace,
                      workspace_bytes, records, stream):
    _check(_lib.libra_attn_bwd_dq(_ptr(plan_host), _ptr(plan_dev), _ptr(q), _ptr(k), _ptr(v), _ptr(dout), _ptr(lse),
                                  _ptr(cu_seqlens_dev), _ptr(dq), float(softmax_scale), _ptr(workspace),
                                  int(workspace_bytes), _ptr(records), stream),
           "libra_attn_bwd_dq")


def libra_device_clock_khz() -> int:
    khz = ctypes.c_int32(0)
    _check(_lib.libra_device_clock_khz(ctypes.byref(khz)), "libra_device_clock_khz")
    return khz.value


# ----------------------------------------------------------------- conveniences
class Plan:
    """A host plan buffer, typed views of its sections, and (lazily) its device copy."""

    def __init__(self, cu_seqlens, *, total_tokens, h_q, h_kv, head_dim, tile_tokens, tile_heads,
                 num_cus=0, tau=0.03, assign=ASSIGN_PLACER, item_overhead=0, worker_speed=None,
                 cost=COST_EXECUTED):
        cu = np.ascontiguousarray(cu_seqlens, dtype=np.int32)
        speed = (ctypes.c_uint16 * 8)(*([int(x) for x in worker_speed] if worker_speed is not None else [0] * 8))
        self.params = PlanParams(int(total_tokens), int(cu.size - 1), int(h_q), int(h_kv), int(head_dim),
                                 int(tile_tokens), int(tile_heads), int(num_cus), float(tau), int(assign),
                                 int(item_overhead), speed, int(cost), 0)
        self.cu_seqlens = cu
        self.host = libra_plan(cu, self.params)
        # the header of a buffer the library just built (libra_plan_check verifies foreign ones)
        self.info = PlanInfo.from_buffer_copy(self.host[:ctypes.sizeof(PlanInfo)].tobytes())
        self._dev = {}

    def _section(self, off, count, dtype):
        return self.host[off:off + count * dtype.itemsize].view(dtype)

    @property
    def tiles(self):
        return self._section(self.info.off_tiles, self.info.n_tiles, TILE_DTYPE)

    @property
    def items(self):
        return self._section(self.info.off_items, self.info.n_items, ITEM_DTYPE)

    @property
    def cu_off(self):
        return self._section(self.info.off_cu_off, self.info.num_cus + 1, np.dtype("<i4"))

    @property
    def dq_items(self):
        return self._section(self.info.off_dq_items, self.info.n_dq_items, ITEM_DTYPE)

    @property
    def dq_cu_off(self):
        return self._section(self.info.off_dq_cu_off, self.info.num_cus + 1, np.dtype("<i4"))

    @property
    def kv_items(self):
        return self._section(self.info.off_kv_items, self.info.n_kv_items, ITEM_DTYPE)

    @property
    def kv_cu_off(self):
        return self._section(self.info.off_kv_cu_off, self.info.num_cus + 1, np.dtype("<i4"))

    def device(self, device="cuda"):
        """Byte copy of the plan (and cu_seqlens) in device memory, cached per device."""
        import torch
        dev = torch.device(device)
        if dev not in self._dev:
            plan = torch.from_numpy(self.host.copy()).to(dev)
            cu = torch.from_numpy(self.cu_seqlens.copy()).to(dev)
            self._dev[dev] = (plan, cu)
        return self._dev[dev]


def _stream_handle(device):
    import torch
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _check_tensors(plan: Plan, **tensors):
    """Shapes, dtypes, contiguity and device of the tensors of one call, against the plan.  Every
    check runs before any pointer reaches the library (a tensor shorter than the plan's packing
    would let the kernels read or write past its end)."""
    import torch
    p = plan.params
    L, d = p.total_tokens, p.head_dim
    want = {"q": ((L, p.h_q, d), torch.bfloat16), "o": ((L, p.h_q, d), torch.bfloat16),
            "dout": ((L, p.h_q, d), torch.bfloat16), "k": ((L, p.h_kv, d), torch.bfloat16),
            "v": ((L, p.h_kv, d), torch.bfloat16), "lse": ((p.h_q, L), torch.float32)}
    device = None
    for name, t in tensors.items():
        shape, dtype = want[name]
        if tuple(t.shape) != shape:
            raise ValueError(f"{name}: shape {tuple(t.shape)}, the plan needs {shape}")
        if t.dtype != dtype:
            raise ValueError(f"{name}: dtype {t.dtype}, needs {dtype}")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
        if device is None:
            device = t.device
        elif t.device != device:
            raise ValueError(f"{name} is on {t.device}, the other tensors on {device}")
    if device is None or device.type != "cuda":
        raise ValueError(f"the tensors must be on a GPU (got {device})")
    return device


def attn_fwd(plan: Plan, q, k, v, softmax_scale=None, *, out=None, lse=None, records=None):
    """Forward pass on torch tensors (bf16 q [L, h_q, d], k and v [L, h_kv, d], contiguous, on one
    GPU); returns (o, lse)."""
    import torch
    p = plan.params
    scale = 1.0 / math.sqrt(p.head_dim) if softmax_scale is None else softmax_scale
    extra = {n: t for n, t in (("o", out), ("lse", lse)) if t is not None}
    dev = _check_tensors(plan, q=q, k=k, v=v, **extra)
    plan_dev, cu_dev = plan.device(dev)
    o = torch.empty((p.total_tokens, p.h_q, p.head_dim), dtype=torch.bfloat16, device=dev) if out is None else out
    lse = torch.empty((p.h_q, p.total_tokens), dtype=torch.float32, device=dev) if lse is None else lse
    libra_attn_fwd(plan.host, plan_dev, q, k, v, cu_dev, o, lse, scale, records, _stream_handle(dev))
    return o, lse


def attn_bwd(plan: Plan, q, k, v, o, lse, dout, softmax_scale=None, *, workspace=None, records=None):
    """Backward pass; returns (dq, dk, dv) as bf16 tensors."""
    import torch
    p = plan.params
    scale = 1.0 / math.sqrt(p.head_dim) if softmax_scale is None else softmax_scale
    dev = _check_tensors(plan, q=q, k=k, v=v, o=o, lse=lse, dout=dout)
    plan_dev, cu_dev = plan.device(dev)
    dq = torch.empty(tuple(q.shape), dtype=torch.bfloat16, device=dev)
    dk = torch.empty(tuple(k.shape), dtype=torch.bfloat16, device=dev)
    dv = torch.empty(tuple(v.shape), dtype=torch.bfloat16, device=dev)
    ws_bytes = libra_attn_bwd_workspace(plan.host)
    if workspace is None:
        workspace = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=dev)
    elif workspace.device != dev or workspace.numel() * workspace.element_size() < ws_bytes:
        raise ValueError(f"workspace: needs {ws_bytes} bytes on {dev}")
    libra_attn_bwd(plan.host, plan_dev, q, k, v, o, dout, lse, cu_dev, dq, dk, dv, scale, workspace,
                   workspace.numel() * workspace.element_size(), records, _stream_handle(dev))
    return dq, dk, dv
