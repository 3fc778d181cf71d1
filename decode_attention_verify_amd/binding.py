"""ctypes binding of librattn (the C ABI in include/rattn.h).

Argument marshalling only: every step of the attention runs in the HIP library. The
functions keep the C names (``rattn_plan``, ``rattn_decode``, ``rattn_free``, ...) and
take torch tensors, of which only the device pointer and torch's current HIP stream
are passed on. If the library is missing, loading raises: there is no fallback.
"""

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "librattn.so")
ABI_VERSION = 4

RATTN_OK, RATTN_E_INVALID, RATTN_E_UNSUPPORTED, RATTN_E_HIP, RATTN_E_NOMEM = range(5)
RATTN_KV_BF16, RATTN_KV_FP8_E4M3 = 0, 1
RATTN_FLAG_SEQ_LEN_CLAMPED, RATTN_FLAG_PAGE_CLAMPED, RATTN_FLAG_ROWS_INVALID = 1, 2, 4
RATTN_KERNEL_SPLIT_KV, RATTN_KERNEL_PREFILL = 0, 1


class Problem(ctypes.Structure):
    _fields_ = [(name, ctypes.c_int32) for name in (
        "batch", "num_q_heads", "num_kv_heads", "head_dim", "n_query_rows", "page_size",
        "num_pages", "max_pages_per_seq", "max_seq_len", "window", "dmax")] + [
        ("softmax_scale", ctypes.c_float), ("kv_dtype", ctypes.c_int32),
        ("num_splits", ctypes.c_int32)]


class PlanInfo(ctypes.Structure):
    _fields_ = [(name, ctypes.c_int32) for name in (
        "num_splits", "keys_per_split", "tile_keys", "row_tiles", "grid_x", "grid_y",
        "grid_z", "combine_blocks", "num_cus", "blocks_per_cu", "kernel", "pieces_per_group")] + [
        ("workspace_bytes", ctypes.c_int64), ("tiles_per_wave", ctypes.c_int32)]

    def as_dict(self):
        return {name: getattr(self, name) for name, _ in self._fields_}


class RattnError(RuntimeError):
    def __init__(self, status, what):
        self.status = status
        super().__init__("%s failed: %s (status %d)" % (what, _status_string(status), status))


_lib = None


def _status_string(status):
    try:
        return load().rattn_status_string(status).decode()
    except Exception:                                   # library not loadable
        return "status %d" % status


def load(path=None):
    """Load librattn.so (once) and declare the C signatures."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    path = path or LIB_PATH
    if not os.path.exists(path):
        raise ImportError("librattn.so not found at %s: build it with "
                          "`python -m decode_attention_verify_amd.build`" % path)
    lib = ctypes.CDLL(path)
    vp, i32, f32p, i32p = ctypes.c_void_p, ctypes.c_int32, ctypes.POINTER(ctypes.c_float), \
        ctypes.POINTER(ctypes.c_int32)
    lib.rattn_plan.argtypes = [ctypes.POINTER(Problem), ctypes.POINTER(vp)]
    lib.rattn_plan_describe.argtypes = [ctypes.POINTER(Problem), i32, ctypes.POINTER(PlanInfo)]
    lib.rattn_plan_get_info.argtypes = [vp, ctypes.POINTER(PlanInfo)]
    lib.rattn_decode.argtypes = [vp] * 12
    lib.rattn_decode_varlen.argtypes = [vp] * 9 + [i32] + [vp] * 4
    lib.rattn_decode_static.argtypes = [ctypes.POINTER(Problem)] + [vp] * 12
    lib.rattn_free.argtypes = [vp]
    lib.rattn_debug_flags.argtypes = [vp, i32p, vp]
    lib.rattn_profile_begin.argtypes = [vp, i32, i32]
    lib.rattn_profile_end.argtypes = [vp, f32p, f32p, i32p]
    lib.rattn_append_kv.argtypes = [ctypes.POINTER(Problem)] + [vp] * 10
    lib.rattn_read_probe.argtypes = [vp, ctypes.c_int64, i32, vp, i32, vp, vp]
    lib.rattn_status_string.argtypes = [ctypes.c_int]
    lib.rattn_status_string.restype = ctypes.c_char_p
    lib.rattn_abi_version.argtypes = []
    for fn in ("rattn_plan", "rattn_plan_describe", "rattn_plan_get_info", "rattn_decode",
               "rattn_free", "rattn_debug_flags", "rattn_profile_begin", "rattn_profile_end",
               "rattn_abi_version", "rattn_append_kv", "rattn_decode_varlen",
               "rattn_read_probe", "rattn_decode_static"):
        getattr(lib, fn).restype = ctypes.c_int32
    if lib.rattn_abi_version() != ABI_VERSION:
        raise ImportError("librattn ABI %d, binding expects %d" % (lib.rattn_abi_version(),
                                                                   ABI_VERSION))
    if path == LIB_PATH:
        _lib = lib
    return lib


def make_problem(*, batch, num_q_heads, num_kv_heads, n_query_rows, page_size, num_pages,
                 max_pages_per_seq, max_seq_len, window, dmax, softmax_scale,
                 kv_dtype=RATTN_KV_BF16, num_splits=0, head_dim=128):
    return Problem(batch=batch, num_q_heads=num_q_heads, num_kv_heads=num_kv_heads,
                   head_dim=head_dim, n_query_rows=n_query_rows, page_size=page_size,
                   num_pages=num_pages, max_pages_per_seq=max_pages_per_seq,
                   max_seq_len=max_seq_len, window=window, dmax=dmax,
                   softmax_scale=softmax_scale, kv_dtype=kv_dtype, num_splits=num_splits)


def rattn_plan(problem):
    """Plan on the current HIP device; returns an opaque handle (free with rattn_free)."""
    handle = ctypes.c_void_p()
    st = load().rattn_plan(ctypes.byref(problem), ctypes.byref(handle))
    if st != RATTN_OK:
        raise RattnError(st, "rattn_plan")
    return handle


def rattn_plan_describe(problem, num_cus):
    """Planner decisions for a device with ``num_cus`` CUs; host only, no HIP call."""
    info = PlanInfo()
    st = load().rattn_plan_describe(ctypes.byref(problem), int(num_cus), ctypes.byref(info))
    if st != RATTN_OK:
        raise RattnError(st, "rattn_plan_describe")
    return info


def rattn_plan_get_info(plan):
    info = PlanInfo()
    st = load().rattn_plan_get_info(plan, ctypes.byref(info))
    if st != RATTN_OK:
        raise RattnError(st, "rattn_plan_get_info")
    return info


def rattn_free(plan):
    st = load().rattn_free(plan)
    if st != RATTN_OK:
        raise RattnError(st, "rattn_free")


def _ptr(t, what, dtype=None, device=None):
    import torch
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError("%s must be a torch.Tensor" % what)
    if t.device.type != "cuda":
        raise ValueError("%s must be on the GPU, got %s" % (what, t.device))
    if device is not None and t.device != device:
        raise ValueError("%s is on %s, expected %s" % (what, t.device, device))
    if dtype is not None and t.dtype not in dtype:
        raise TypeError("%s has dtype %s, expected one of %s" % (what, t.dtype, dtype))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % what)
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def check_shapes(problem, q, k_cache, v_cache, k_scale, v_scale, page_table, seq_lens, bias,
                 out, lse=None, only=None):
    """Raise ValueError unless every tensor has the shape ``problem`` implies (all of them,
    or the names in ``only``)."""
    p = problem
    want = {
        "q": (q, (p.batch, p.n_query_rows, p.num_q_heads, p.head_dim)),
        "k_cache": (k_cache, (p.num_pages, p.num_kv_heads, p.page_size, p.head_dim)),
        "v_cache": (v_cache, (p.num_pages, p.num_kv_heads, p.page_size, p.head_dim)),
        "page_table": (page_table, (p.batch, p.max_pages_per_seq)),
        "seq_lens": (seq_lens, (p.batch,)),
        "bias": (bias, (p.num_q_heads, p.dmax + 1)),
        "out": (out, (p.batch, p.n_query_rows, p.num_q_heads, p.head_dim)),
        "lse": (lse, (p.batch, p.n_query_rows, p.num_q_heads)),
    }
    if p.kv_dtype == RATTN_KV_FP8_E4M3:
        want["k_scale"] = (k_scale, (p.num_pages, p.num_kv_heads, p.page_size))
        want["v_scale"] = (v_scale, (p.num_pages, p.num_kv_heads, p.page_size))
    elif k_scale is not None or v_scale is not None:
        raise ValueError("k_scale / v_scale are only for the E4M3 cache")
    for name, (t, shape) in want.items():
        if only is not None and name not in only:
            continue
        if t is None:
            if name == "lse":
                continue
            raise ValueError("%s is required" % name)
        if tuple(t.shape) != tuple(shape):
            raise ValueError("%s has shape %s, the problem needs %s" % (name, tuple(t.shape),
                                                                        tuple(shape)))
    elem = 1 if p.kv_dtype == RATTN_KV_FP8_E4M3 else 2
    for name, t in (("k_cache", k_cache), ("v_cache", v_cache)):
        if t.element_size() != elem:
            raise ValueError("%s element size %d does not match the problem's KV dtype" % (
                name, t.element_size()))


def rattn_decode(plan, q, k_cache, v_cache, k_scale, v_scale, page_table, seq_lens, bias,
                 out, lse=None, stream=None, problem=None):
    """Enqueue one decode/verify attention call on ``stream`` (default: torch's current).

    With ``problem`` (the plan's rattn_problem) every tensor's shape is checked first.
    """
    import torch
    if problem is not None:
        check_shapes(problem, q, k_cache, v_cache, k_scale, v_scale, page_table, seq_lens, bias,
                     out, lse)
    dev = q.device
    args = [
        plan,
        _ptr(q, "q", (torch.bfloat16,)),
        _ptr(k_cache, "k_cache", (torch.bfloat16, torch.uint8, torch.float8_e4m3fn), dev),
        _ptr(v_cache, "v_cache", (torch.bfloat16, torch.uint8, torch.float8_e4m3fn), dev),
        _ptr(k_scale, "k_scale", (torch.float32,), dev),
        _ptr(v_scale, "v_scale", (torch.float32,), dev),
        _ptr(page_table, "page_table", (torch.int32,), dev),
        _ptr(seq_lens, "seq_lens", (torch.int32,), dev),
        _ptr(bias, "bias", (torch.float32,), dev),
        _ptr(out, "out", (torch.bfloat16,), dev),
        _ptr(lse, "lse", (torch.float32,), dev),
        _stream(stream),
    ]
    st = load().rattn_decode(*args)
    if st != RATTN_OK:
        raise RattnError(st, "rattn_decode")


def rattn_decode_static(problem, q, k_cache, v_cache, k_scale, v_scale, page_table, seq_lens,
                        bias, out, lse=None, flags=None, stream=None):
    """Enqueue one call without a plan, whose partials live in the library's static
    device array (no allocation); shapes are checked against ``problem`` first."""
    import torch
    check_shapes(problem, q, k_cache, v_cache, k_scale, v_scale, page_table, seq_lens, bias,
                 out, lse)
    dev = q.device
    args = [
        ctypes.byref(problem),
        _ptr(q, "q", (torch.bfloat16,)),
        _ptr(k_cache, "k_cache", (torch.bfloat16, torch.uint8, torch.float8_e4m3fn), dev),
        _ptr(v_cache, "v_cache", (torch.bfloat16, torch.uint8, torch.float8_e4m3fn), dev),
        _ptr(k_scale, "k_scale", (torch.float32,), dev),
        _ptr(v_scale, "v_scale", (torch.float32,), dev),
        _ptr(page_table, "page_table", (torch.int32,), dev),
        _ptr(seq_lens, "seq_lens", (torch.int32,), dev),
        _ptr(bias, "bias", (torch.float32,), dev),
        _ptr(out, "out", (torch.bfloat16,), dev),
        _ptr(lse, "lse", (torch.float32,), dev),
        _ptr(flags, "flags", (torch.int32,), dev),
        _stream(stream),
    ]
    st = load().rattn_decode_static(*args)
    if st != RATTN_OK:
        raise RattnError(st, "rattn_decode_static")


def rattn_decode_varlen(plan, q, k_cache, v_cache, k_scale, v_scale, page_table, seq_lens,
                        cu_rows, bias, out, lse=None, stream=None, problem=None):
    """Enqueue an attention call where sequence b brings cu_rows[b+1] - cu_rows[b] query
    rows, packed in q [rows][Hq][D]; out (and lse) hold as many rows as q."""
    import torch
    rows = int(q.shape[0])
    if problem is not None:
        p = problem
        if q.dim() != 3 or tuple(q.shape[1:]) != (p.num_q_heads, p.head_dim):
            raise ValueError("q must be [rows][%d][%d], got %s" % (p.num_q_heads, p.head_dim,
                                                                   tuple(q.shape)))
        if tuple(out.shape) != tuple(q.shape):
            raise ValueError("out has shape %s, q %s" % (tuple(out.shape), tuple(q.shape)))
        if lse is not None and tuple(lse.shape) != (rows, p.num_q_heads):
            raise ValueError("lse has shape %s, needs %s" % (tuple(lse.shape),
                                                            (rows, p.num_q_heads)))
        if tuple(cu_rows.shape) != (p.batch + 1,):
            raise ValueError("cu_rows has shape %s, needs (%d,)" % (tuple(cu_rows.shape),
                                                                   p.batch + 1))
        check_shapes(p, None, k_cache, v_cache, k_scale, v_scale, page_table, seq_lens, bias,
                     None, None, only=("k_cache", "v_cache", "k_scale", "v_scale",
                                       "page_table", "seq_lens", "bias"))
    dev = q.device
    args = [
        plan,
        _ptr(q, "q", (torch.bfloat16,)),
        _ptr(k_cache, "k_cache", (torch.bfloat16, torch.uint8, torch.float8_e4m3fn), dev),
        _ptr(v_cache, "v_cache", (torch.bfloat16, torch.uint8, torch.float8_e4m3fn), dev),
        _ptr(k_scale, "k_scale", (torch.float32,), dev),
        _ptr(v_scale, "v_scale", (torch.float32,), dev),
        _ptr(page_table, "page_table", (torch.int32,), dev),
        _ptr(seq_lens, "seq_lens", (torch.int32,), dev),
        _ptr(cu_rows, "cu_rows", (torch.int32,), dev),
        ctypes.c_int32(rows),
        _ptr(bias, "bias", (torch.float32,), dev),
        _ptr(out, "out", (torch.bfloat16,), dev),
        _ptr(lse, "lse", (torch.float32,), dev),
        _stream(stream),
    ]
    st = load().rattn_decode_varlen(*args)
    if st != RATTN_OK:
        raise RattnError(st, "rattn_decode_varlen")


def rattn_append_kv(problem, k_new, v_new, page_table, seq_lens, k_cache, v_cache,
                    k_scale=None, v_scale=None, flags=None, stream=None):
    """Enqueue the write of each sequence's n newest tokens into the paged cache."""
    import torch
    p = problem
    shape = (p.batch, p.n_query_rows, p.num_kv_heads, p.head_dim)
    for name, t in (("k_new", k_new), ("v_new", v_new)):
        if tuple(t.shape) != shape:
            raise ValueError("%s has shape %s, the problem needs %s" % (name, tuple(t.shape), shape))
    check_shapes(p, torch.empty(0), k_cache, v_cache, k_scale, v_scale, page_table, seq_lens,
                 None, None, None, only=("k_cache", "v_cache", "k_scale", "v_scale",
                                         "page_table", "seq_lens"))
    dev = k_new.device
    args = [
        ctypes.byref(problem),
        _ptr(k_new, "k_new", (torch.bfloat16,)),
        _ptr(v_new, "v_new", (torch.bfloat16,), dev),
        _ptr(page_table, "page_table", (torch.int32,), dev),
        _ptr(seq_lens, "seq_lens", (torch.int32,), dev),
        _ptr(k_cache, "k_cache", (torch.bfloat16, torch.uint8, torch.float8_e4m3fn), dev),
        _ptr(v_cache, "v_cache", (torch.bfloat16, torch.uint8, torch.float8_e4m3fn), dev),
        _ptr(k_scale, "k_scale", (torch.float32,), dev),
        _ptr(v_scale, "v_scale", (torch.float32,), dev),
        _ptr(flags, "flags", (torch.int32,), dev),
        _stream(stream),
    ]
    st = load().rattn_append_kv(*args)
    if st != RATTN_OK:
        raise RattnError(st, "rattn_append_kv")


def rattn_debug_flags(plan, stream=None):
    flags = ctypes.c_int32()
    st = load().rattn_debug_flags(plan, ctypes.byref(flags), _stream(stream))
    if st != RATTN_OK:
        raise RattnError(st, "rattn_debug_flags")
    return flags.value


def rattn_profile_begin(plan, max_calls, stride=1):
    st = load().rattn_profile_begin(plan, int(max_calls), int(stride))
    if st != RATTN_OK:
        raise RattnError(st, "rattn_profile_begin")


def rattn_profile_end(plan, max_calls):
    split = (ctypes.c_float * max_calls)()
    comb = (ctypes.c_float * max_calls)()
    n = ctypes.c_int32()
    st = load().rattn_profile_end(plan, split, comb, ctypes.byref(n))
    if st != RATTN_OK:
        raise RattnError(st, "rattn_profile_end")
    return list(split[:n.value]), list(comb[:n.value])


class Plan:
    """An owned plan: ``with Plan(problem) as p: p.decode(...)``."""

    def __init__(self, problem):
        self.problem = problem
        self.handle = rattn_plan(problem)

    @property
    def info(self):
        return rattn_plan_get_info(self.handle)

    def decode(self, q, k_cache, v_cache, k_scale, v_scale, page_table, seq_lens, bias, out,
               lse=None, stream=None):
        rattn_decode(self.handle, q, k_cache, v_cache, k_scale, v_scale, page_table, seq_lens,
                     bias, out, lse, stream, problem=self.problem)

    def decode_varlen(self, q, k_cache, v_cache, k_scale, v_scale, page_table, seq_lens,
                      cu_rows, bias, out, lse=None, stream=None):
        rattn_decode_varlen(self.handle, q, k_cache, v_cache, k_scale, v_scale, page_table,
                            seq_lens, cu_rows, bias, out, lse, stream, problem=self.problem)

    def debug_flags(self, stream=None):
        return rattn_debug_flags(self.handle, stream)

    def close(self):
        if self.handle is not None:
            rattn_free(self.handle)
            self.handle = None

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        self.close()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def problem_from_case(case, num_splits=0):
    """The rattn_problem of an input drawn by ``synth.make_case``."""
    sp = case.spec
    fp8 = case.k_cache.dtype != __import__("torch").bfloat16
    return make_problem(batch=sp.batch, num_q_heads=sp.num_q_heads, num_kv_heads=sp.num_kv_heads,
                        n_query_rows=sp.n_rows, page_size=sp.page_size,
                        num_pages=int(case.k_cache.shape[0]),
                        max_pages_per_seq=int(case.page_table.shape[1]),
                        max_seq_len=int(case.max_seq_len), window=sp.window, dmax=sp.dmax,
                        softmax_scale=float(case.softmax_scale),
                        kv_dtype=RATTN_KV_FP8_E4M3 if fp8 else RATTN_KV_BF16,
                        num_splits=num_splits, head_dim=sp.head_dim)
