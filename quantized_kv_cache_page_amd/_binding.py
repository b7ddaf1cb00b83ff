"""ctypes binding of libskvd.so: the C-ABI functions under the same names, and `Plan`, which
marshals torch tensors (device memory and streams only) into those calls.

Nothing here computes any part of the decode: every step runs in the HIP kernels of
libskvd.so. Importing fails loudly when the library has not been built.
"""
from __future__ import annotations

import ctypes
import os

import torch  # imported first: libskvd.so then binds to the HIP runtime torch already loaded

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libskvd.so")

SKVD_KV_F16 = 0
SKVD_KV_I8_F16SCALE32 = 1
SKVD_KV_FP8_E4M3 = 2
SKVD_KV_Q4_0 = 3
REDUCERS = {"auto": 0, "direct": 1, "cooperative": 2, "multipass": 3, "hierarchical": 4,
            "none": 5}
REDUCER_NAMES = {v: k for k, v in REDUCERS.items()}
SCHEDULES = {"auto": 0, "static": 1, "balanced": 2}
SCHEDULE_NAMES = {v: k for k, v in SCHEDULES.items()}
ABI_VERSION = 11
STATUS_KV_LEN_CLAMPED = 0x1
STATUS_PAGE_CLAMPED = 0x2


class SkvdError(RuntimeError):
    def __init__(self, status: int, where: str, msg: str):
        super().__init__(f"{where}: status {status} ({status_string(status)}): {msg}")
        self.status = status


class skvd_plan_params(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "num_qo_heads", "num_kv_heads", "head_dim", "page_size", "max_batch", "max_q_per_seq",
        "max_kv_len", "kv_dtype", "device", "num_cus", "force_blocks_per_split",
        "force_reducer", "debug", "schedule", "wgs_per_cu", "heads_per_wg")]


class skvd_plan_info(ctypes.Structure):
    _fields_ = [("blocks_per_split", ctypes.c_int32), ("splits_cap", ctypes.c_int32),
                ("reducer", ctypes.c_int32), ("hier_groups_cap", ctypes.c_int32),
                ("rows_per_group", ctypes.c_int32), ("num_cus", ctypes.c_int32),
                ("rows_cap", ctypes.c_int64), ("workspace_bytes", ctypes.c_uint64),
                ("status_offset", ctypes.c_uint64), ("schedule", ctypes.c_int32),
                ("part_stride", ctypes.c_int32), ("grid_wgs", ctypes.c_int32),
                ("heads_per_wg", ctypes.c_int32)]


class skvd_decode_args(ctypes.Structure):
    _fields_ = [
        ("q", ctypes.c_void_p), ("q_tok_stride", ctypes.c_int64), ("q_head_stride", ctypes.c_int64),
        ("k_pages", ctypes.c_void_p), ("v_pages", ctypes.c_void_p),
        ("page_stride", ctypes.c_int64), ("tok_stride", ctypes.c_int64),
        ("head_stride", ctypes.c_int64), ("num_k_pages", ctypes.c_int64),
        ("num_v_pages", ctypes.c_int64),
        ("k_scales", ctypes.c_void_p), ("v_scales", ctypes.c_void_p),
        ("scale_page_stride", ctypes.c_int64), ("scale_tok_stride", ctypes.c_int64),
        ("scale_head_stride", ctypes.c_int64),
        ("page_table", ctypes.c_void_p), ("table_stride", ctypes.c_int64),
        ("kv_len", ctypes.c_void_p),
        ("batch", ctypes.c_int32), ("q_per_seq", ctypes.c_int32),
        ("sm_scale", ctypes.c_float), ("reserved", ctypes.c_int32),
        ("o", ctypes.c_void_p), ("lse", ctypes.c_void_p),
    ]


class skvd_append_args(ctypes.Structure):
    _fields_ = [
        ("k_new", ctypes.c_void_p), ("v_new", ctypes.c_void_p),
        ("new_tok_stride", ctypes.c_int64), ("new_head_stride", ctypes.c_int64),
        ("batch_idx", ctypes.c_void_p), ("positions", ctypes.c_void_p),
        ("num_tokens", ctypes.c_int32), ("batch", ctypes.c_int32),
        ("k_pages", ctypes.c_void_p), ("v_pages", ctypes.c_void_p),
        ("page_stride", ctypes.c_int64), ("tok_stride", ctypes.c_int64),
        ("head_stride", ctypes.c_int64), ("num_k_pages", ctypes.c_int64),
        ("num_v_pages", ctypes.c_int64),
        ("k_scales", ctypes.c_void_p), ("v_scales", ctypes.c_void_p),
        ("scale_page_stride", ctypes.c_int64), ("scale_tok_stride", ctypes.c_int64),
        ("scale_head_stride", ctypes.c_int64),
        ("page_table", ctypes.c_void_p), ("table_stride", ctypes.c_int64),
    ]


# Every symbol include/skvd.h declares, with its ctypes signature.
_PLAN_P = ctypes.c_void_p
SIGNATURES = {
    "skvd_plan_create": (ctypes.c_int, [ctypes.POINTER(skvd_plan_params), ctypes.POINTER(ctypes.c_void_p)]),
    "skvd_plan_destroy": (None, [_PLAN_P]),
    "skvd_plan_workspace_bytes": (ctypes.c_size_t, [_PLAN_P]),
    "skvd_plan_get_info": (ctypes.c_int, [_PLAN_P, ctypes.POINTER(skvd_plan_info)]),
    "skvd_plan_describe": (ctypes.c_int, [_PLAN_P, ctypes.c_char_p, ctypes.c_size_t]),
    "skvd_decode_check": (ctypes.c_int, [_PLAN_P, ctypes.POINTER(skvd_decode_args), ctypes.c_size_t]),
    "skvd_decode": (ctypes.c_int, [_PLAN_P, ctypes.POINTER(skvd_decode_args), ctypes.c_void_p,
                                   ctypes.c_size_t, ctypes.c_void_p]),
    "skvd_decode_noalloc": (ctypes.c_int, [_PLAN_P, ctypes.POINTER(skvd_decode_args),
                                           ctypes.c_void_p]),
    "skvd_decode_partial": (ctypes.c_int, [_PLAN_P, ctypes.POINTER(skvd_decode_args),
                                           ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]),
    "skvd_decode_merge": (ctypes.c_int, [_PLAN_P, ctypes.POINTER(skvd_decode_args),
                                         ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]),
    "skvd_decode_partial_timed": (ctypes.c_int, [_PLAN_P, ctypes.POINTER(skvd_decode_args),
                                                 ctypes.c_void_p, ctypes.c_size_t,
                                                 ctypes.c_void_p, ctypes.c_void_p,
                                                 ctypes.c_void_p]),
    "skvd_gather_debug": (ctypes.c_int, [_PLAN_P, ctypes.POINTER(skvd_decode_args), ctypes.c_int32,
                                         ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                         ctypes.c_void_p, ctypes.c_void_p]),
    "skvd_stream_read": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p,
                                        ctypes.c_void_p]),
    "skvd_attention": (ctypes.c_int, [_PLAN_P, ctypes.POINTER(skvd_decode_args), ctypes.c_void_p,
                                      ctypes.c_size_t, ctypes.c_void_p]),
    "skvd_merge_states": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64,
                                         ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32,
                                         ctypes.c_int64, ctypes.c_int32, ctypes.c_void_p,
                                         ctypes.c_void_p, ctypes.c_void_p]),
    "skvd_prefill_check": (ctypes.c_int, [_PLAN_P, ctypes.POINTER(skvd_decode_args)]),
    "skvd_prefill": (ctypes.c_int, [_PLAN_P, ctypes.POINTER(skvd_decode_args), ctypes.c_void_p]),
    "skvd_append_check": (ctypes.c_int, [_PLAN_P, ctypes.POINTER(skvd_append_args)]),
    "skvd_append": (ctypes.c_int, [_PLAN_P, ctypes.POINTER(skvd_append_args), ctypes.c_void_p]),
    "skvd_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "skvd_last_error": (ctypes.c_char_p, []),
    "skvd_abi_version": (ctypes.c_int32, []),
}

_lib = None


def _hip_runtimes_mapped():
    try:
        with open("/proc/self/maps") as f:
            return sorted({ln.split()[-1] for ln in f if "libamdhip64" in ln})
    except OSError:
        return []


def lib():
    """Load libskvd.so once. Raises if it is missing or if two HIP runtimes end up mapped."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built: run `python -m quantized_kv_cache_page_amd.build`")
    L = ctypes.CDLL(LIB_PATH)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(L, name)
        fn.restype = res
        fn.argtypes = args
    rts = _hip_runtimes_mapped()
    if len(rts) > 1:
        raise ImportError(f"two HIP runtimes are mapped ({rts}); import torch before libskvd")
    if L.skvd_abi_version() != ABI_VERSION:
        raise ImportError("libskvd ABI version mismatch")
    _lib = L
    return L


def status_string(st: int) -> str:
    return lib().skvd_status_string(st).decode()


def last_error() -> str:
    return lib().skvd_last_error().decode()


def _check(st: int, where: str):
    if st != 0:
        raise SkvdError(st, where, last_error())


# ---------------------------------------------------------------- thin C-ABI wrappers
def skvd_plan_create(params: skvd_plan_params) -> int:
    h = ctypes.c_void_p()
    _check(lib().skvd_plan_create(ctypes.byref(params), ctypes.byref(h)), "skvd_plan_create")
    return h.value


def skvd_plan_destroy(plan: int) -> None:
    lib().skvd_plan_destroy(plan)


def skvd_plan_workspace_bytes(plan: int) -> int:
    return int(lib().skvd_plan_workspace_bytes(plan))


def skvd_plan_get_info(plan: int) -> skvd_plan_info:
    info = skvd_plan_info()
    _check(lib().skvd_plan_get_info(plan, ctypes.byref(info)), "skvd_plan_get_info")
    return info


def skvd_plan_describe(plan: int) -> str:
    buf = ctypes.create_string_buffer(512)
    _check(lib().skvd_plan_describe(plan, buf, 512), "skvd_plan_describe")
    return buf.value.decode()


def skvd_decode_check(plan: int, args: skvd_decode_args, workspace_bytes: int) -> int:
    return int(lib().skvd_decode_check(plan, ctypes.byref(args), workspace_bytes))


def skvd_decode(plan, args, workspace, workspace_bytes, stream) -> int:
    return int(lib().skvd_decode(plan, ctypes.byref(args), workspace, workspace_bytes, stream))


def skvd_decode_noalloc(plan, args, stream) -> int:
    return int(lib().skvd_decode_noalloc(plan, ctypes.byref(args), stream))


def skvd_decode_partial(plan, args, workspace, workspace_bytes, stream) -> int:
    return int(lib().skvd_decode_partial(plan, ctypes.byref(args), workspace, workspace_bytes,
                                         stream))


def skvd_decode_partial_timed(plan, args, workspace, workspace_bytes, stream, start_event,
                              stop_event) -> int:
    return int(lib().skvd_decode_partial_timed(plan, ctypes.byref(args), workspace,
                                               workspace_bytes, stream, start_event, stop_event))


def skvd_decode_merge(plan, args, workspace, workspace_bytes, stream) -> int:
    return int(lib().skvd_decode_merge(plan, ctypes.byref(args), workspace, workspace_bytes,
                                       stream))


def skvd_gather_debug(plan, args, max_len, dk, dv, dks, dvs, stream) -> int:
    return int(lib().skvd_gather_debug(plan, ctypes.byref(args), max_len, dk, dv, dks, dvs,
                                       stream))


def skvd_attention(plan, args, workspace, workspace_bytes, stream) -> int:
    return int(lib().skvd_attention(plan, ctypes.byref(args), workspace, workspace_bytes, stream))


def skvd_merge_states(o_states, o_state_stride, o_row_stride, lse_states, lse_state_stride,
                      num_states, rows, head_dim, o, lse, stream) -> int:
    return int(lib().skvd_merge_states(o_states, o_state_stride, o_row_stride, lse_states,
                                       lse_state_stride, num_states, rows, head_dim, o, lse,
                                       stream))


def merge_states(o_states, lse_states, out=None, lse=None, stream=None):
    """skvd_merge_states on torch tensors: o_states [S, rows, D] f16 (D dense), lse_states
    [S, rows] f32 (row stride 1). Returns (o [rows, D] f16, lse [rows] f32)."""
    if o_states.dtype != torch.float16 or lse_states.dtype != torch.float32:
        raise TypeError("o_states must be float16 and lse_states float32")
    if o_states.dim() != 3 or lse_states.dim() != 2 or o_states.shape[:2] != lse_states.shape:
        raise SkvdError(2, "merge_states", "o_states [S, rows, D] and lse_states [S, rows]")
    if o_states.stride(2) != 1 or lse_states.stride(1) != 1:
        raise SkvdError(3, "merge_states", "head_dim and rows must be dense")
    S, rows, D = o_states.shape
    if out is None:
        out = torch.empty((rows, D), dtype=torch.float16, device=o_states.device)
    if lse is None:
        lse = torch.empty((rows,), dtype=torch.float32, device=o_states.device)
    if not out.is_contiguous() or not lse.is_contiguous():
        raise SkvdError(3, "merge_states", "outputs are written densely")
    st = (stream if stream is not None else torch.cuda.current_stream(o_states.device)).cuda_stream
    _check(skvd_merge_states(o_states.data_ptr(), o_states.stride(0), o_states.stride(1),
                             lse_states.data_ptr(), lse_states.stride(0), S, rows, D,
                             out.data_ptr(), lse.data_ptr(), st), "skvd_merge_states")
    return out, lse


def skvd_prefill_check(plan, args) -> int:
    return int(lib().skvd_prefill_check(plan, ctypes.byref(args)))


def skvd_prefill(plan, args, stream) -> int:
    return int(lib().skvd_prefill(plan, ctypes.byref(args), stream))


def skvd_append_check(plan, args) -> int:
    return int(lib().skvd_append_check(plan, ctypes.byref(args)))


def skvd_append(plan, args, stream) -> int:
    return int(lib().skvd_append(plan, ctypes.byref(args), stream))


def skvd_stream_read(buf: int, nbytes: int, sink: int, stream) -> int:
    return int(lib().skvd_stream_read(buf, nbytes, sink, stream))


def stream_read(t, sink, stream=None):
    """Read tensor t once (measurement aid; see skvd_stream_read)."""
    s = (stream if stream is not None else torch.cuda.current_stream(t.device)).cuda_stream
    _check(skvd_stream_read(t.data_ptr(), t.numel() * t.element_size(), sink.data_ptr(), s),
           "skvd_stream_read")


# ---------------------------------------------------------------- torch-facing plan
def _ptr(t):
    return None if t is None else t.data_ptr()


def _kv_dtype_code(kv_dtype) -> int:
    if kv_dtype in ("f16", torch.float16):
        return SKVD_KV_F16
    if kv_dtype in ("i8", torch.int8):
        return SKVD_KV_I8_F16SCALE32
    if kv_dtype in ("f8", "fp8", "e4m3", torch.uint8, torch.float8_e4m3fn):
        return SKVD_KV_FP8_E4M3
    if kv_dtype in ("q4", "q4_0"):
        return SKVD_KV_Q4_0
    raise ValueError(f"unknown kv_dtype {kv_dtype!r}")


_POOL_DTYPES = {"f16": (torch.float16,), "i8": (torch.int8,),
                "f8": (torch.uint8, torch.float8_e4m3fn), "q4": (torch.uint8,)}


def _set_scales(a, k_scales, v_scales, kv_dtype, where):
    """Scale pointers (and, for int8 and q4_0, strides) of a decode or append argument struct."""
    if k_scales is None:
        if v_scales is not None:
            raise SkvdError(4, where, "v_scales given without k_scales")
        return
    if v_scales is None:
        raise SkvdError(4, where, "k_scales given without v_scales")
    if kv_dtype == "f8":
        if k_scales.dtype != torch.float32 or v_scales.dtype != torch.float32 or \
                k_scales.numel() != 1 or v_scales.numel() != 1:
            raise SkvdError(4, where, "fp8 k_scales/v_scales must be one-element float32 tensors")
        a.k_scales, a.v_scales = k_scales.data_ptr(), v_scales.data_ptr()
        return
    if k_scales.dtype != torch.float16 or v_scales.stride() != k_scales.stride():
        raise SkvdError(4, where, "k_scales/v_scales must be f16 with equal strides")
    a.k_scales, a.v_scales = k_scales.data_ptr(), v_scales.data_ptr()
    a.scale_page_stride, a.scale_tok_stride, a.scale_head_stride = (
        k_scales.stride(0), k_scales.stride(1), k_scales.stride(2))


class Plan:
    """A decode plan and its workspace.

    Plan(num_qo_heads, num_kv_heads, head_dim, page_size, kv_dtype, max_batch, max_q_per_seq,
         max_kv_len, device) sizes everything once, outside any capture; run() then launches
    the decode on the current stream with no allocation other than the default outputs.
    kv_dtype is "f16", "i8" (int8 with one f16 scale per 32 elements), "f8" (OCP E4M3
    bytes, held in uint8 tensors, with one f32 scale per tensor passed as k_scales / v_scales:
    one-element float32 device tensors) or "q4" (q4_0: uint8 pools [pages, P, Hkv, D/2], two
    4-bit codes per byte, with f16 scale pools [pages, P, Hkv, D/32])."""

    def __init__(self, num_qo_heads, num_kv_heads, head_dim, page_size, kv_dtype="f16",
                 max_batch=1, max_q_per_seq=1, max_kv_len=1, device=0, num_cus=0,
                 force_blocks_per_split=0, force_reducer="auto", debug=False,
                 schedule="auto", wgs_per_cu=0, heads_per_wg=0):
        dev = torch.device("cuda", device) if isinstance(device, int) else torch.device(device)
        self.device = dev
        idx = dev.index if dev.index is not None else torch.cuda.current_device()
        red = REDUCERS[force_reducer] if isinstance(force_reducer, str) else int(force_reducer)
        sch = SCHEDULES[schedule] if isinstance(schedule, str) else int(schedule)
        self.params = skvd_plan_params(
            int(num_qo_heads), int(num_kv_heads), int(head_dim), int(page_size), int(max_batch),
            int(max_q_per_seq), int(max_kv_len),
            _kv_dtype_code(kv_dtype),
            int(idx), int(num_cus), int(force_blocks_per_split), red, int(bool(debug)), sch,
            int(wgs_per_cu), int(heads_per_wg))
        self.kv_dtype = {SKVD_KV_F16: "f16", SKVD_KV_I8_F16SCALE32: "i8",
                         SKVD_KV_FP8_E4M3: "f8", SKVD_KV_Q4_0: "q4"}[self.params.kv_dtype]
        self.handle = skvd_plan_create(self.params)
        self.info = skvd_plan_get_info(self.handle)
        self.workspace_bytes = int(self.info.workspace_bytes)
        self.workspace = None

    def __del__(self):
        h = getattr(self, "handle", None)
        if h:
            try:
                skvd_plan_destroy(h)
            except Exception:
                pass
            self.handle = None

    def describe(self) -> str:
        return skvd_plan_describe(self.handle)

    @property
    def reducer(self) -> str:
        return REDUCER_NAMES[self.info.reducer]

    @property
    def schedule(self) -> str:
        return SCHEDULE_NAMES[self.info.schedule]

    def ensure_workspace(self):
        """Allocate the workspace (once; call it outside graph capture)."""
        if self.workspace is None:
            self.workspace = torch.zeros(self.workspace_bytes + 256, dtype=torch.uint8,
                                         device=self.device)
            off = (-self.workspace.data_ptr()) % 256
            self.workspace = self.workspace[off:off + self.workspace_bytes]
        return self.workspace

    def status_word(self) -> int:
        """Debug status bits recorded by the kernels (reads device memory: synchronizes)."""
        ws = self.ensure_workspace()
        o = int(self.info.status_offset)
        return int(ws[o:o + 4].view(torch.int32).item())

    def clear_status(self):
        ws = self.ensure_workspace()
        o = int(self.info.status_offset)
        ws[o:o + 4].zero_()

    def make_args(self, q, k_pages, v_pages, page_table, kv_len, sm_scale, k_scales=None,
                  v_scales=None, out=None, lse=None, q_per_seq=1) -> skvd_decode_args:
        if q.dtype != torch.float16:
            raise TypeError("q must be float16")
        want = _POOL_DTYPES[self.kv_dtype]
        if k_pages.dtype not in want or v_pages.dtype not in want:
            raise TypeError(f"k_pages and v_pages must be {want[0]}")
        if k_pages.stride() != v_pages.stride() or k_pages.shape[1:] != v_pages.shape[1:]:
            raise SkvdError(3, "Plan.run", "K and V must share page shape and strides")
        if page_table.dtype != torch.int32 or kv_len.dtype != torch.int32:
            raise TypeError("page_table and kv_len must be int32")
        if page_table.dim() != 2 or page_table.stride(1) != 1:
            raise SkvdError(3, "Plan.run", "page_table must be [B, n] with unit inner stride")
        if q.dim() != 3 or k_pages.dim() != 4:
            raise SkvdError(2, "Plan.run", "q must be [B*T, Hq, D] and pools [pages, P, Hkv, D]")
        if q.stride(2) != 1 or k_pages.stride(3) != 1:
            raise SkvdError(3, "Plan.run", "head_dim must be dense in q and the pools")
        if k_pages.shape[3] != self._row_len():
            raise SkvdError(2, "Plan.run", f"pool rows must hold {self._row_len()} elements")
        B = int(kv_len.shape[0])
        a = skvd_decode_args()
        a.q = q.data_ptr()
        a.q_tok_stride, a.q_head_stride = q.stride(0), q.stride(1)
        a.k_pages, a.v_pages = k_pages.data_ptr(), v_pages.data_ptr()
        a.page_stride, a.tok_stride, a.head_stride = k_pages.stride(0), k_pages.stride(1), k_pages.stride(2)
        a.num_k_pages, a.num_v_pages = k_pages.shape[0], v_pages.shape[0]
        _set_scales(a, k_scales, v_scales, self.kv_dtype, "Plan.run")
        a.page_table = page_table.data_ptr()
        a.table_stride = page_table.stride(0)
        a.kv_len = kv_len.data_ptr()
        a.batch, a.q_per_seq = B, int(q_per_seq)
        a.sm_scale = float(sm_scale)
        a.reserved = 0
        a.o = _ptr(out)
        a.lse = _ptr(lse)
        return a

    def _row_len(self) -> int:
        """Elements of a pool row: head_dim, or head_dim / 2 bytes for q4_0."""
        D = int(self.params.head_dim)
        return D // 2 if self.kv_dtype == "q4" else D

    def _outputs(self, q, out, lse):
        if out is None:
            out = torch.empty(q.shape, dtype=torch.float16, device=q.device)  # dense
        if lse is None:
            lse = torch.empty(q.shape[:2], dtype=torch.float32, device=q.device)
        if not out.is_contiguous() or (lse is not None and not lse.is_contiguous()):
            raise SkvdError(3, "Plan.run", "o and lse are written densely: pass contiguous tensors")
        return out, lse

    def _stream(self, stream):
        s = stream if stream is not None else torch.cuda.current_stream(self.device)
        return s.cuda_stream

    def run(self, q, k_pages, v_pages, page_table, kv_len, sm_scale, k_scales=None,
            v_scales=None, out=None, lse=None, q_per_seq=1, stream=None, stage="all",
            events=None):
        """Decode. q [B*T, Hq, D] f16 (token and head strides free, D dense); pools
        [pages, P, Hkv, D]; page_table [B, n] int32; kv_len [B] int32 on the device.
        Returns (o [B*T, Hq, D] f16 dense, lse [B*T, Hq] f32). stage: "all", "partial" or
        "merge" (the two halves of one decode, for timing). events: with stage "partial", a
        (start, stop) pair of already recorded torch.cuda.Event(enable_timing=True) that the
        partial kernel's dispatch stamps with its own begin and end (skvd_decode_partial_timed)."""
        out, lse = self._outputs(q, out, lse)
        ws = self.ensure_workspace()
        a = self.make_args(q, k_pages, v_pages, page_table, kv_len, sm_scale, k_scales, v_scales,
                           out, lse, q_per_seq)
        if events is not None:
            if stage != "partial":
                raise ValueError("events time the partial stage only")
            e0, e1 = (ctypes.c_void_p(e.cuda_event) for e in events)
            if not e0.value or not e1.value:
                raise ValueError("record each event once before passing it (HIP creates it then)")
            _check(skvd_decode_partial_timed(self.handle, a, ws.data_ptr(), self.workspace_bytes,
                                             self._stream(stream), e0, e1),
                   "skvd_decode_partial_timed")
            return out, lse
        fn = {"all": skvd_decode, "partial": skvd_decode_partial, "merge": skvd_decode_merge}[stage]
        _check(fn(self.handle, a, ws.data_ptr(), self.workspace_bytes, self._stream(stream)),
               f"skvd_decode[{stage}]")
        return out, lse

    def run_noalloc(self, q, k_pages, v_pages, page_table, kv_len, sm_scale, k_scales=None,
                    v_scales=None, out=None, lse=None, q_per_seq=1, stream=None):
        """skvd_decode_noalloc: the decode with the library's own device workspace (no plan
        workspace is allocated). out and lse must be passed by callers that cannot allocate
        (the defaults allocate them). Returns (o, lse) as run()."""
        out, lse = self._outputs(q, out, lse)
        a = self.make_args(q, k_pages, v_pages, page_table, kv_len, sm_scale, k_scales, v_scales,
                           out, lse, q_per_seq)
        _check(skvd_decode_noalloc(self.handle, a, self._stream(stream)), "skvd_decode_noalloc")
        return out, lse

    def check(self, q, k_pages, v_pages, page_table, kv_len, sm_scale, k_scales=None,
              v_scales=None, out=None, lse=None, q_per_seq=1, workspace_bytes=None) -> int:
        """skvd_decode_check: the validation alone, no HIP call. Returns the status."""
        a = self.make_args(q, k_pages, v_pages, page_table, kv_len, sm_scale, k_scales, v_scales,
                           out, lse, q_per_seq)
        return skvd_decode_check(self.handle, a, self.workspace_bytes if workspace_bytes is None
                                 else workspace_bytes)

    def attend(self, q, k_pages, v_pages, page_table, kv_len, sm_scale, k_scales=None,
               v_scales=None, out=None, lse=None, q_per_seq=1, stream=None):
        """skvd_attention: the decode for q_per_seq <= max_q_per_seq, the tiled route beyond
        (the pages' batch-aware routing). Returns (o, lse) as run()."""
        out, lse = self._outputs(q, out, lse)
        ws = self.ensure_workspace()
        a = self.make_args(q, k_pages, v_pages, page_table, kv_len, sm_scale, k_scales, v_scales,
                           out, lse, q_per_seq)
        _check(skvd_attention(self.handle, a, ws.data_ptr(), self.workspace_bytes,
                              self._stream(stream)), "skvd_attention")
        return out, lse

    def prefill(self, q, k_pages, v_pages, page_table, kv_len, sm_scale, k_scales=None,
                v_scales=None, out=None, lse=None, q_per_seq=1, stream=None):
        """skvd_prefill: the multi-token route (any q_per_seq = T >= 1; same arguments, causal
        reading and outputs as run()). Returns (o [B*T, Hq, D] f16, lse [B*T, Hq] f32)."""
        out, lse = self._outputs(q, out, lse)
        a = self.make_args(q, k_pages, v_pages, page_table, kv_len, sm_scale, k_scales, v_scales,
                           out, lse, q_per_seq)
        _check(skvd_prefill(self.handle, a, self._stream(stream)), "skvd_prefill")
        return out, lse

    def prefill_check(self, q, k_pages, v_pages, page_table, kv_len, sm_scale, k_scales=None,
                      v_scales=None, out=None, lse=None, q_per_seq=1) -> int:
        """skvd_prefill_check: the validation alone, no HIP call. Returns the status."""
        a = self.make_args(q, k_pages, v_pages, page_table, kv_len, sm_scale, k_scales, v_scales,
                           out, lse, q_per_seq)
        return skvd_prefill_check(self.handle, a)

    def make_append_args(self, k_new, v_new, batch_idx, positions, k_pages, v_pages, page_table,
                         k_scales=None, v_scales=None, batch=None) -> skvd_append_args:
        if k_new.dtype != torch.float16 or v_new.dtype != torch.float16:
            raise TypeError("k_new and v_new must be float16")
        if k_new.shape != v_new.shape or k_new.stride() != v_new.stride() or k_new.dim() != 3:
            raise SkvdError(3, "Plan.append", "k_new and v_new must be [N, Hkv, D] with equal strides")
        empty = k_new.shape[0] == 0  # torch may give an empty tensor any strides
        if (not empty and k_new.stride(2) != 1) or k_pages.stride(3) != 1:
            raise SkvdError(3, "Plan.append", "head_dim must be dense in the new rows and the pools")
        want = _POOL_DTYPES[self.kv_dtype]
        if k_pages.dtype not in want or v_pages.dtype not in want:
            raise TypeError(f"k_pages and v_pages must be {want[0]}")
        if k_pages.stride() != v_pages.stride() or k_pages.shape[1:] != v_pages.shape[1:]:
            raise SkvdError(3, "Plan.append", "K and V must share page shape and strides")
        if k_pages.dim() != 4 or k_pages.shape[3] != self._row_len():
            raise SkvdError(2, "Plan.append", f"pool rows must hold {self._row_len()} elements")
        if batch_idx.dtype != torch.int32 or positions.dtype != torch.int32 or \
                page_table.dtype != torch.int32:
            raise TypeError("batch_idx, positions and page_table must be int32")
        if batch_idx.shape != (k_new.shape[0],) or positions.shape != (k_new.shape[0],) or \
                (not empty and (not batch_idx.is_contiguous() or not positions.is_contiguous())):
            raise SkvdError(2, "Plan.append", "batch_idx and positions must be dense [N]")
        if page_table.dim() != 2 or page_table.stride(1) != 1:
            raise SkvdError(3, "Plan.append", "page_table must be [B, n] with unit inner stride")
        if k_new.shape[1] != self.params.num_kv_heads or k_new.shape[2] != self.params.head_dim:
            raise SkvdError(2, "Plan.append", "new rows must be [N, Hkv, D] of the plan")
        a = skvd_append_args()
        a.k_new, a.v_new = k_new.data_ptr(), v_new.data_ptr()
        a.new_tok_stride, a.new_head_stride = ((k_new.shape[1] * k_new.shape[2], k_new.shape[2])
                                               if empty else (k_new.stride(0), k_new.stride(1)))
        a.batch_idx, a.positions = batch_idx.data_ptr(), positions.data_ptr()
        a.num_tokens = int(k_new.shape[0])
        a.batch = int(page_table.shape[0] if batch is None else batch)
        a.k_pages, a.v_pages = k_pages.data_ptr(), v_pages.data_ptr()
        a.page_stride, a.tok_stride, a.head_stride = k_pages.stride(0), k_pages.stride(1), k_pages.stride(2)
        a.num_k_pages, a.num_v_pages = k_pages.shape[0], v_pages.shape[0]
        _set_scales(a, k_scales, v_scales, self.kv_dtype, "Plan.append")
        a.page_table = page_table.data_ptr()
        a.table_stride = page_table.stride(0)
        return a

    def append(self, k_new, v_new, batch_idx, positions, k_pages, v_pages, page_table,
               k_scales=None, v_scales=None, batch=None, stream=None):
        """skvd_append: write new rows k_new, v_new [N, Hkv, D] f16 of tokens (batch_idx[i],
        positions[i]) into the pools in place (int8 and q4_0 pools: quantized, scales written;
        fp8 pools: quantized with the given tensor scales, which are only read). Only the
        named slots are written; nothing is allocated."""
        a = self.make_append_args(k_new, v_new, batch_idx, positions, k_pages, v_pages,
                                  page_table, k_scales, v_scales, batch)
        _check(skvd_append(self.handle, a, self._stream(stream)), "skvd_append")

    def append_check(self, *args, **kw) -> int:
        """skvd_append_check: the validation alone, no HIP call. Returns the status."""
        return skvd_append_check(self.handle, self.make_append_args(*args, **kw))

    def gather_debug(self, q, k_pages, v_pages, page_table, kv_len, max_len, k_scales=None,
                     v_scales=None, q_per_seq=1, stream=None):
        """skvd_gather_debug: dense raw copies of the visible K/V rows (zeros elsewhere; q4_0
        rows are their D/2 code bytes)."""
        B = int(kv_len.shape[0])
        Hkv, row, D = k_pages.shape[2], k_pages.shape[3], int(self.params.head_dim)
        dk = torch.zeros((B, max_len, Hkv, row), dtype=k_pages.dtype, device=k_pages.device)
        dv = torch.zeros_like(dk)
        dks = dvs = None
        if k_scales is not None and self.kv_dtype in ("i8", "q4"):
            dks = torch.zeros((B, max_len, Hkv, D // 32), dtype=torch.float16, device=k_pages.device)
            dvs = torch.zeros_like(dks)
        o = torch.empty(q.shape, dtype=torch.float16, device=q.device)
        a = self.make_args(q, k_pages, v_pages, page_table, kv_len, 1.0, k_scales, v_scales, o,
                           None, q_per_seq)
        _check(skvd_gather_debug(self.handle, a, int(max_len), dk.data_ptr(), dv.data_ptr(),
                                 _ptr(dks), _ptr(dvs), self._stream(stream)), "skvd_gather_debug")
        return dk, dv, dks, dvs


def skvd_abi_version_py() -> int:
    return int(lib().skvd_abi_version())
