"""ctypes binding of libhtgemm.so: the same entry points as include/htgemm.h and
include/htlayout.h, with argument marshalling only.  Every step of the GEMM runs in the HIP
library; nothing here computes.  If the library has not been built, every call raises.
"""
from __future__ import annotations

import ctypes
import os

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libhtgemm.so")

# status codes (htgemm.h)
GEMM_OK = 0
GEMM_ERR_INVALID_ARG, GEMM_ERR_LAYOUT, GEMM_ERR_MISALIGNED, GEMM_ERR_NO_CONFIG = 1, 3, 4, 8
STATUS_NAMES = {0: "GEMM_OK", 1: "GEMM_ERR_INVALID_ARG", 2: "GEMM_ERR_DTYPE_COMBO",
                3: "GEMM_ERR_LAYOUT", 4: "GEMM_ERR_MISALIGNED", 5: "GEMM_ERR_ARCH",
                6: "GEMM_ERR_LAUNCH", 7: "GEMM_ERR_BAD_HANDLE", 8: "GEMM_ERR_NO_CONFIG",
                9: "GEMM_ERR_HIP", 10: "GEMM_ERR_LANE_MAP", 11: "GEMM_ERR_SCRATCH_LIMIT"}
GEMM_ERR_SCRATCH_LIMIT = 11
GEMM_NOALLOC_SCRATCH_BYTES = 32 << 20
GEMM_PROBE_INTS = 8192
DTYPES = {"f32": 0, "f16": 1, "bf16": 2, "e4m3": 3}
ACTS = {"none": 0, "relu": 1, "gelu": 2, "gelu_erf": 2, "silu": 3}
# layout status codes (htlayout.h)
HT_STATUS_NAMES = {0: "HT_OK", 1: "HT_ERR_PARSE", 2: "HT_ERR_RANGE", 3: "HT_ERR_NOT_COMPOSABLE",
                   4: "HT_ERR_CAPACITY", 5: "HT_ERR_NO_COMPLEMENT"}


class GemmError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {STATUS_NAMES.get(status, status)}")


class LayoutError(ValueError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {HT_STATUS_NAMES.get(status, status)}")


class gemm_desc(ctypes.Structure):
    _fields_ = [("M", ctypes.c_int64), ("N", ctypes.c_int64), ("K", ctypes.c_int64),
                ("a_type", ctypes.c_int32), ("b_type", ctypes.c_int32),
                ("c_type", ctypes.c_int32), ("d_type", ctypes.c_int32),
                ("bias_type", ctypes.c_int32), ("has_c", ctypes.c_int32),
                ("has_bias", ctypes.c_int32), ("act", ctypes.c_int32),
                ("a_stride_m", ctypes.c_int64), ("a_stride_k", ctypes.c_int64),
                ("b_stride_k", ctypes.c_int64), ("b_stride_n", ctypes.c_int64),
                ("c_stride_m", ctypes.c_int64), ("c_stride_n", ctypes.c_int64),
                ("d_stride_m", ctypes.c_int64), ("d_stride_n", ctypes.c_int64),
                ("force_config", ctypes.c_int32), ("split_k", ctypes.c_int32),
                ("has_row_scale", ctypes.c_int32), ("has_col_scale", ctypes.c_int32),
                ("batch", ctypes.c_int64),
                ("a_stride_l", ctypes.c_int64), ("b_stride_l", ctypes.c_int64),
                ("c_stride_l", ctypes.c_int64), ("d_stride_l", ctypes.c_int64),
                ("ragged_m", ctypes.c_int32), ("has_row_sumsq", ctypes.c_int32),
                ("has_col_sum", ctypes.c_int32), ("grouped", ctypes.c_int32),
                ("decomposition", ctypes.c_int32)]


class gemm_problem(ctypes.Structure):
    _fields_ = [("M", ctypes.c_int64), ("N", ctypes.c_int64), ("K", ctypes.c_int64),
                ("A", ctypes.c_void_p), ("B", ctypes.c_void_p), ("C", ctypes.c_void_p),
                ("D", ctypes.c_void_p), ("bias", ctypes.c_void_p),
                ("lda", ctypes.c_int64), ("ldb", ctypes.c_int64), ("ldc", ctypes.c_int64),
                ("ldd", ctypes.c_int64)]


class gemm_args(ctypes.Structure):
    _fields_ = [("A", ctypes.c_void_p), ("B", ctypes.c_void_p), ("C", ctypes.c_void_p),
                ("D", ctypes.c_void_p), ("bias", ctypes.c_void_p),
                ("row_scale", ctypes.c_void_p), ("col_scale", ctypes.c_void_p),
                ("alpha", ctypes.c_float), ("beta", ctypes.c_float),
                ("scale_a", ctypes.c_float), ("scale_b", ctypes.c_float),
                ("workspace", ctypes.c_void_p), ("row_sumsq", ctypes.c_void_p),
                ("col_sum", ctypes.c_void_p)]


class gemm_info(ctypes.Structure):
    _fields_ = [("config", ctypes.c_int32), ("fallback", ctypes.c_int32),
                ("bm", ctypes.c_int32), ("bn", ctypes.c_int32), ("bk", ctypes.c_int32),
                ("waves", ctypes.c_int32), ("stages", ctypes.c_int32),
                ("lds_bytes", ctypes.c_int32), ("split_k", ctypes.c_int32),
                ("grid", ctypes.c_int64), ("name", ctypes.c_char * 96),
                ("tail_tiles", ctypes.c_int32), ("tail_split", ctypes.c_int32),
                ("repack", ctypes.c_int32), ("sk_tiles", ctypes.c_int32),
                ("sk_wgs", ctypes.c_int32), ("predicted_us", ctypes.c_double)]


class ht_tile_stats(ctypes.Structure):
    _fields_ = [("flops", ctypes.c_int64), ("bytes", ctypes.c_int64),
                ("intensity", ctypes.c_double), ("double_buffer_bytes", ctypes.c_int64),
                ("fits", ctypes.c_int32)]


_lib = None


def lib():
    """The loaded library; raises if it has not been built (no fallback path exists)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m hierarchical_tiling_amd.build`"
                           " (or __graft_entry__.build()); there is no CPU fallback")
    L = ctypes.CDLL(LIB_PATH)
    vp, i64, i32, sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_size_t
    cp = ctypes.c_char_p
    sig = {
        "gemm_create": ([ctypes.POINTER(gemm_desc), ctypes.POINTER(vp)], i32),
        "gemm_workspace_size": ([vp, ctypes.POINTER(sz)], i32),
        "gemm_run": ([vp, vp, vp, vp, vp, vp, ctypes.c_float, ctypes.c_float, ctypes.c_float,
                      ctypes.c_float, vp, vp], i32),
        "gemm_run_ex": ([vp, ctypes.POINTER(gemm_args), vp], i32),
        "gemm_run_grouped": ([vp, ctypes.POINTER(gemm_args), vp, vp], i32),
        "gemm_run_noalloc": ([vp, ctypes.POINTER(gemm_args), vp], i32),
        "gemm_run_problems": ([vp, ctypes.POINTER(gemm_problem), i64, ctypes.POINTER(gemm_args), vp],
                              i32),
        "gemm_destroy": ([vp], i32),
        "gemm_status_string": ([i32], cp),
        "gemm_get_info": ([vp, ctypes.POINTER(gemm_info)], i32),
        "gemm_num_configs": ([], i32),
        "gemm_config_name": ([i32, ctypes.c_char_p, sz], i32),
        "gemm_atom_layouts": ([i32, i32, ctypes.c_char_p, ctypes.c_char_p, sz], i32),
        "gemm_probe_atom": ([i32, i32, vp, vp], i32),
        "gemm_set_clock_record": ([vp, vp, i64], i32),
        "ht_layout_eval": ([cp, ctypes.POINTER(i64), i32, ctypes.POINTER(i64)], i32),
        "ht_layout_eval_str": ([cp, cp, ctypes.POINTER(i64)], i32),
        "ht_layout_size": ([cp, ctypes.POINTER(i64)], i32),
        "ht_layout_table": ([cp, ctypes.POINTER(i64), i64], i32),
        "ht_layout_coalesce": ([cp, ctypes.c_char_p, sz], i32),
        "ht_layout_compose": ([cp, cp, ctypes.c_char_p, sz], i32),
        "ht_layout_complement": ([cp, i64, ctypes.c_char_p, sz], i32),
        "ht_layout_logical_divide": ([cp, cp, ctypes.c_char_p, sz], i32),
        "ht_layout_zipped_divide": ([cp, cp, cp, ctypes.c_char_p, sz], i32),
        "ht_layout_local_tile": ([cp, cp, cp, cp, ctypes.POINTER(i64), ctypes.c_char_p, sz], i32),
        "ht_layout_local_partition": ([cp, cp, i64, ctypes.POINTER(i64), ctypes.c_char_p, sz], i32),
        "ht_swizzle": ([i64, i32, i32, i32], i64),
        "ht_tile_plan": ([i64, i64, i64, i32, i64, ctypes.POINTER(ht_tile_stats)], i32),
        "ht_pipeline_time": ([i64, ctypes.c_double, ctypes.c_double], ctypes.c_double),
    }
    for name, (args, res) in sig.items():
        f = getattr(L, name)
        f.argtypes = args
        f.restype = res
    _lib = L
    return L


EXPORTED = ["gemm_create", "gemm_workspace_size", "gemm_run", "gemm_run_ex", "gemm_run_grouped",
            "gemm_run_noalloc", "gemm_run_problems",
            "gemm_destroy",
            "gemm_status_string",
            "gemm_get_info", "gemm_num_configs", "gemm_config_name", "gemm_atom_layouts",
            "gemm_probe_atom", "gemm_set_clock_record", "ht_layout_eval",
            "ht_layout_eval_str",
            "ht_layout_size", "ht_layout_table", "ht_layout_coalesce", "ht_layout_compose",
            "ht_layout_complement", "ht_layout_logical_divide", "ht_layout_zipped_divide",
            "ht_layout_local_tile", "ht_layout_local_partition", "ht_swizzle", "ht_tile_plan", "ht_pipeline_time"]


def _check(rc, where):
    if rc != GEMM_OK:
        raise GemmError(rc, where)


# ---- GEMM entry points --------------------------------------------------------------------

def gemm_create(desc: gemm_desc) -> int:
    h = ctypes.c_void_p()
    _check(lib().gemm_create(ctypes.byref(desc), ctypes.byref(h)), "gemm_create")
    return h.value


def gemm_workspace_size(h) -> int:
    n = ctypes.c_size_t()
    _check(lib().gemm_workspace_size(h, ctypes.byref(n)), "gemm_workspace_size")
    return n.value


def gemm_run(h, A, B, C, D, bias, alpha, beta, scale_a=1.0, scale_b=1.0, workspace=None,
             stream=None):
    """Pointers are integers (device addresses) or None; stream is a hipStream_t as an integer."""
    _check(lib().gemm_run(h, A, B, C, D, bias, alpha, beta, scale_a, scale_b, workspace, stream),
           "gemm_run")


def gemm_run_ex(h, A, B, C, D, bias, row_scale, col_scale, alpha, beta, scale_a=1.0, scale_b=1.0,
                workspace=None, stream=None, row_sumsq=None, col_sum=None):
    """gemm_run with the scale vectors and the row reduction (device addresses or None),
    through the argument struct."""
    a = gemm_args(A, B, C, D, bias, row_scale, col_scale, alpha, beta, scale_a, scale_b, workspace,
                  row_sumsq, col_sum)
    _check(lib().gemm_run_ex(h, ctypes.byref(a), stream), "gemm_run_ex")


def gemm_run_grouped(h, A, B, C, D, bias, row_scale, col_scale, offsets, alpha, beta,
                     scale_a=1.0, scale_b=1.0, stream=None, workspace=None):
    """Grouped ragged-M run: `offsets` is the device address of batch + 1 int32 row offsets;
    `workspace` the device address of gemm_workspace_size bytes (the groups' tile table)."""
    a = gemm_args(A, B, C, D, bias, row_scale, col_scale, alpha, beta, scale_a, scale_b, workspace)
    _check(lib().gemm_run_grouped(h, ctypes.byref(a), offsets, stream), "gemm_run_grouped")


def gemm_run_noalloc(h, A, B, C, D, bias, row_scale, col_scale, alpha, beta, scale_a=1.0,
                     scale_b=1.0, stream=None, row_sumsq=None, col_sum=None):
    """gemm_run_ex with the library's static scratch as the workspace (no allocation)."""
    a = gemm_args(A, B, C, D, bias, row_scale, col_scale, alpha, beta, scale_a, scale_b, None,
                  row_sumsq, col_sum)
    _check(lib().gemm_run_noalloc(h, ctypes.byref(a), stream), "gemm_run_noalloc")


def gemm_run_problems(h, problems, alpha, beta, scale_a=1.0, scale_b=1.0, stream=None,
                      workspace=None):
    """Grouped run of independent problems: `problems` is a sequence of dicts (or gemm_problem)
    with M, N, K, A, B, C, D, bias (device addresses or None) and lda, ldb, ldc, ldd."""
    n = len(problems)
    arr = (gemm_problem * max(n, 1))()
    for i, q in enumerate(problems):
        if isinstance(q, gemm_problem):
            arr[i] = q
        else:
            arr[i] = gemm_problem(q["M"], q["N"], q["K"], q.get("A"), q.get("B"), q.get("C"),
                                  q.get("D"), q.get("bias"), q.get("lda", 0), q.get("ldb", 0),
                                  q.get("ldc", 0), q.get("ldd", 0))
    a = gemm_args(None, None, None, None, None, None, None, alpha, beta, scale_a, scale_b,
                  workspace, None, None)
    _check(lib().gemm_run_problems(h, arr, n, ctypes.byref(a), stream), "gemm_run_problems")


def gemm_destroy(h):
    _check(lib().gemm_destroy(h), "gemm_destroy")


def gemm_status_string(status: int) -> str:
    return lib().gemm_status_string(status).decode()


def gemm_get_info(h) -> gemm_info:
    info = gemm_info()
    _check(lib().gemm_get_info(h, ctypes.byref(info)), "gemm_get_info")
    return info


def gemm_num_configs() -> int:
    return lib().gemm_num_configs()


def gemm_config_name(i: int) -> str:
    buf = ctypes.create_string_buffer(128)
    _check(lib().gemm_config_name(i, buf, 128), "gemm_config_name")
    return buf.value.decode()


def gemm_atom_layouts(dtype: str, mi: int):
    """(operand layout, accumulator layout) of the MFMA atom the kernels use, as text."""
    a = ctypes.create_string_buffer(256)
    c = ctypes.create_string_buffer(256)
    _check(lib().gemm_atom_layouts(DTYPES[dtype], mi, a, c, 256), "gemm_atom_layouts")
    return a.value.decode(), c.value.decode()


def gemm_set_clock_record(h, records, max_workgroups: int):
    """records: a device tensor of at least 4 * max_workgroups int64 values, or None (off)."""
    _check(lib().gemm_set_clock_record(h, _addr(records), max_workgroups if records is not None else 0),
           "gemm_set_clock_record")


def gemm_probe_atom(dtype: str, mi: int, out, stream=None):
    """Enqueue the index probe of atom (dtype, mi); `out` is a device buffer of GEMM_PROBE_INTS
    int32 values (a device address or a tensor)."""
    _check(lib().gemm_probe_atom(DTYPES[dtype], mi, _addr(out), _stream(stream)), "gemm_probe_atom")


def make_desc(M, N, K, dtype, a_strides, b_strides, d_strides, c_strides=None, has_bias=False,
              act="none", force_config=-1, split_k=0, row_scale=False, col_scale=False, batch=1,
              batch_strides=(0, 0, 0, 0), ragged_m=False, row_sumsq=False,
              col_sum=False, grouped=False, decomposition=0) -> gemm_desc:
    """a_strides = (stride_m, stride_k); b_strides = (stride_k, stride_n); c/d = (m, n);
    batch_strides = element offsets between consecutive problems of A, B, C, D."""
    out_t = "bf16" if dtype == "e4m3" else dtype
    d = gemm_desc()
    d.M, d.N, d.K = M, N, K
    d.a_type = d.b_type = DTYPES[dtype]
    d.c_type = d.d_type = d.bias_type = DTYPES[out_t]
    d.has_c = 1 if c_strides is not None else 0
    d.has_bias = 1 if has_bias else 0
    d.act = ACTS[act]
    d.a_stride_m, d.a_stride_k = a_strides
    d.b_stride_k, d.b_stride_n = b_strides
    d.c_stride_m, d.c_stride_n = c_strides if c_strides is not None else (0, 0)
    d.d_stride_m, d.d_stride_n = d_strides
    d.force_config = force_config
    d.split_k = split_k
    d.has_row_scale = 1 if row_scale else 0
    d.has_col_scale = 1 if col_scale else 0
    d.batch = batch
    d.a_stride_l, d.b_stride_l, d.c_stride_l, d.d_stride_l = batch_strides
    d.ragged_m = 1 if ragged_m else 0
    d.has_row_sumsq = 1 if row_sumsq else 0
    d.has_col_sum = 1 if col_sum else 0
    d.grouped = 1 if grouped else 0
    d.decomposition = decomposition
    return d


class Gemm:
    """RAII wrapper: a handle for one problem description."""

    def __init__(self, desc: gemm_desc):
        self.desc = desc
        self.handle = gemm_create(desc)

    @property
    def info(self) -> gemm_info:
        return gemm_get_info(self.handle)

    @property
    def workspace_bytes(self) -> int:
        return gemm_workspace_size(self.handle)

    def run(self, A, B, C, D, bias=None, alpha=1.0, beta=0.0, scale_a=1.0, scale_b=1.0,
            stream=None, workspace=None, row_scale=None, col_scale=None, row_sumsq=None,
            col_sum=None):
        """gemm_run, or gemm_run_ex when a scale vector or a reduction output is given."""
        if row_scale is None and col_scale is None and row_sumsq is None and col_sum is None:
            gemm_run(self.handle, _addr(A), _addr(B), _addr(C), _addr(D), _addr(bias), alpha,
                     beta, scale_a, scale_b, _addr(workspace), _stream(stream))
        else:
            gemm_run_ex(self.handle, _addr(A), _addr(B), _addr(C), _addr(D), _addr(bias),
                        _addr(row_scale), _addr(col_scale), alpha, beta, scale_a, scale_b,
                        _addr(workspace), _stream(stream), _addr(row_sumsq), _addr(col_sum))

    def close(self):
        if self.handle:
            gemm_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def _addr(x):
    if x is None:
        return None
    if isinstance(x, int):
        return x
    return x.data_ptr()


def _stream(s):
    if s is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(s, int):
        return s
    return s.cuda_stream


# ---- layout helper ------------------------------------------------------------------------

def _lcheck(rc, where):
    if rc != 0:
        raise LayoutError(rc, where)


def _out_str(fn, *args):
    buf = ctypes.create_string_buffer(4096)
    _lcheck(fn(*args, buf, 4096), fn.__name__)
    return buf.value.decode()


def ht_layout_eval(layout: str, coord) -> int:
    """Offset of `coord`: an int (a 1-D coordinate), a flat tuple of ints (one per top-level
    mode), or text / a nested tuple (passed to ht_layout_eval_str)."""
    out = ctypes.c_int64()
    if isinstance(coord, str) or (isinstance(coord, (tuple, list))
                                  and any(isinstance(x, (tuple, list)) for x in coord)):
        text = coord if isinstance(coord, str) else _coord_str(coord)
        _lcheck(lib().ht_layout_eval_str(layout.encode(), text.encode(), ctypes.byref(out)),
                "ht_layout_eval_str")
        return out.value
    vals = [int(coord)] if not isinstance(coord, (tuple, list)) else [int(x) for x in coord]
    arr = (ctypes.c_int64 * max(len(vals), 1))(*vals)
    _lcheck(lib().ht_layout_eval(layout.encode(), arr, len(vals), ctypes.byref(out)), "ht_layout_eval")
    return out.value


def _coord_str(c):
    if isinstance(c, (tuple, list)):
        return "(" + ",".join(_coord_str(x) for x in c) + ")"
    return str(int(c))


def ht_layout_size(layout: str) -> int:
    out = ctypes.c_int64()
    _lcheck(lib().ht_layout_size(layout.encode(), ctypes.byref(out)), "ht_layout_size")
    return out.value


def ht_layout_table(layout: str):
    n = ht_layout_size(layout)
    arr = (ctypes.c_int64 * max(n, 1))()
    _lcheck(lib().ht_layout_table(layout.encode(), arr, n), "ht_layout_table")
    return list(arr[:n])


def ht_layout_coalesce(layout: str) -> str:
    return _out_str(lib().ht_layout_coalesce, layout.encode())


def ht_layout_compose(a: str, b: str) -> str:
    return _out_str(lib().ht_layout_compose, a.encode(), b.encode())


def ht_layout_complement(a: str, m: int) -> str:
    return _out_str(lib().ht_layout_complement, a.encode(), int(m))


def ht_layout_logical_divide(a: str, b: str) -> str:
    return _out_str(lib().ht_layout_logical_divide, a.encode(), b.encode())


def ht_layout_zipped_divide(a: str, t0: str, t1: str) -> str:
    return _out_str(lib().ht_layout_zipped_divide, a.encode(), t0.encode(), t1.encode())


def _slots(x):
    if isinstance(x, str):
        return x
    return "(" + ",".join("_" if v is None else str(v) for v in x) + ")"


def ht_layout_local_tile(a: str, tiler, coord, proj=None):
    """(offset, layout): the view of `a`'s tile at `coord` (None or "_" keeps a mode)."""
    buf = ctypes.create_string_buffer(4096)
    off = ctypes.c_int64()
    _lcheck(lib().ht_layout_local_tile(a.encode(), _slots(tiler).encode(), _slots(coord).encode(),
                                       None if proj is None else _slots(proj).encode(),
                                       ctypes.byref(off), buf, 4096), "ht_layout_local_tile")
    return off.value, buf.value.decode()


def ht_layout_local_partition(a: str, thr_shape, idx: int):
    """(offset, layout): thread `idx`'s elements of `a` under a thread layout of `thr_shape`."""
    buf = ctypes.create_string_buffer(4096)
    off = ctypes.c_int64()
    _lcheck(lib().ht_layout_local_partition(a.encode(), _slots(thr_shape).encode(), int(idx),
                                            ctypes.byref(off), buf, 4096),
            "ht_layout_local_partition")
    return off.value, buf.value.decode()


def ht_swizzle(offset: int, bbits: int, mbase: int, sshift: int) -> int:
    return lib().ht_swizzle(offset, bbits, mbase, sshift)


def ht_tile_plan(m, n, k, bytes_per_elem, budget_bytes) -> ht_tile_stats:
    st = ht_tile_stats()
    _lcheck(lib().ht_tile_plan(m, n, k, bytes_per_elem, budget_bytes, ctypes.byref(st)), "ht_tile_plan")
    return st


def ht_pipeline_time(n, load, compute) -> float:
    return lib().ht_pipeline_time(n, load, compute)
