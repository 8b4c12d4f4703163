"""ctypes view of the C ABI in include/fmha_bwd.h (argument marshalling only)."""

import ctypes
import os

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libfmha_bwd.so")

ABI_VERSION = 8

MASK_NONE = 0
MASK_CAUSAL_TOP_LEFT = 1
MASK_CAUSAL_BOTTOM_RIGHT = 2
MASK_WINDOW = 3

DQ_ACC_FP32 = 0
DQ_ACC_BF16 = 1

KERNEL_AUTO = 0
KERNEL_FOUR_WAVE = 1
KERNEL_WIDE = 2

OK = 0
ERR_INVALID_ARG = -1
ERR_UNSUPPORTED = -2
ERR_WORKSPACE_TOO_SMALL = -3
ERR_PLAN_MISMATCH = -4
ERR_HIP = -5

STAGE_DOT = 1
STAGE_MAIN = 2
STAGE_REDUCE = 4
STAGE_ALL = STAGE_DOT | STAGE_MAIN | STAGE_REDUCE

EXPORTS = (
    "fmha_bwd_workspace_size",
    "fmha_bwd_prepare_workspace",
    "fmha_bwd_run",
    "fmha_bwd_status_string",
    "fmha_bwd_plan_query",
    "fmha_bwd_run_stages",
    "fmha_fwd_run",
    "fmha_bwd_run_noalloc",
)

NOALLOC_MAX_BYTES = 256 << 20  # FMHA_BWD_NOALLOC_MAX_BYTES

_i64x3 = ctypes.c_int64 * 3


class Args(ctypes.Structure):
    _fields_ = [
        ("struct_size", ctypes.c_uint32),
        ("abi_version", ctypes.c_uint32),
        ("B", ctypes.c_int32),
        ("Hq", ctypes.c_int32),
        ("Hkv", ctypes.c_int32),
        ("Sq", ctypes.c_int32),
        ("Sk", ctypes.c_int32),
        ("d_qk", ctypes.c_int32),
        ("d_v", ctypes.c_int32),
        ("scale", ctypes.c_float),
        ("mask_type", ctypes.c_int32),
        ("window_left", ctypes.c_int32),
        ("window_right", ctypes.c_int32),
        ("deterministic", ctypes.c_int32),
        ("seqstart_q_host", ctypes.c_void_p),
        ("seqstart_k_host", ctypes.c_void_p),
        ("seqstart_q_dev", ctypes.c_void_p),
        ("seqstart_k_dev", ctypes.c_void_p),
        ("q", ctypes.c_void_p),
        ("k", ctypes.c_void_p),
        ("v", ctypes.c_void_p),
        ("o", ctypes.c_void_p),
        ("dout", ctypes.c_void_p),
        ("lse", ctypes.c_void_p),
        ("dq", ctypes.c_void_p),
        ("dk", ctypes.c_void_p),
        ("dv", ctypes.c_void_p),
        ("q_stride", _i64x3),
        ("k_stride", _i64x3),
        ("v_stride", _i64x3),
        ("o_stride", _i64x3),
        ("do_stride", _i64x3),
        ("dq_stride", _i64x3),
        ("dk_stride", _i64x3),
        ("dv_stride", _i64x3),
        ("lse_stride", ctypes.c_int64 * 2),
        ("seqstart_q_padded_host", ctypes.c_void_p),
        ("seqstart_k_padded_host", ctypes.c_void_p),
        ("seqstart_q_padded_dev", ctypes.c_void_p),
        ("seqstart_k_padded_dev", ctypes.c_void_p),
        ("dq_acc_dtype", ctypes.c_int32),
        ("reserved", ctypes.c_int32),
        ("bias", ctypes.c_void_p),
        ("dbias", ctypes.c_void_p),
        ("bias_stride", _i64x3),
        ("dbias_stride", _i64x3),
        ("bias_b", ctypes.c_int32),
        ("bias_h", ctypes.c_int32),
        ("p_drop", ctypes.c_float),
        ("reserved2", ctypes.c_int32),
        ("philox_seed", ctypes.c_uint64),
        ("philox_offset", ctypes.c_uint64),
        ("tune_kernel", ctypes.c_int32),
        ("tune_tile_m", ctypes.c_int32),
        ("tune_tiles_per_item", ctypes.c_int32),
        ("tune_kv_parts", ctypes.c_int32),
    ]

    def __init__(self, **kw):
        super().__init__()
        self.struct_size = ctypes.sizeof(Args)
        self.abi_version = ABI_VERSION
        self.window_left = -1
        self.window_right = -1
        self.deterministic = 1
        for k, v in kw.items():
            setattr(self, k, v)


class PlanInfo(ctypes.Structure):
    _fields_ = [
        ("group_mode", ctypes.c_int32),
        ("tile_m", ctypes.c_int32),
        ("tile_n", ctypes.c_int32),
        ("n_kv_tiles", ctypes.c_int32),
        ("n_q_blocks", ctypes.c_int32),
        ("nsplits", ctypes.c_int32),
        ("needs_zero", ctypes.c_int32),
        ("tiles_per_item", ctypes.c_int32),
        ("rows_q", ctypes.c_int64),
        ("d_offset", ctypes.c_int64),
        ("dq_acc_offset", ctypes.c_int64),
        ("dq_acc_bytes", ctypes.c_int64),
        ("workspace_bytes", ctypes.c_int64),
        ("pairs", ctypes.c_int64),
        ("flops", ctypes.c_double),
        ("acc_rows", ctypes.c_int64),
        ("dq_acc_elem_bytes", ctypes.c_int32),
        ("kv_parts", ctypes.c_int32),
        ("dbias_acc_offset", ctypes.c_int64),
        ("dbias_acc_bytes", ctypes.c_int64),
        ("reduce_read_bytes", ctypes.c_int64),
        ("dkv_acc_offset", ctypes.c_int64),
        ("dkv_acc_bytes", ctypes.c_int64),
        ("kernel", ctypes.c_int32),
        ("ordered_groups", ctypes.c_int32),
    ]

    def as_dict(self):
        return {name: getattr(self, name) for name, _ in self._fields_}


class FmhaError(RuntimeError):
    def __init__(self, status, where):
        self.status = status
        super().__init__("%s failed: %s (%d)" % (where, status_string(status), status))


_lib = None


def lib():
    """Load the built library; raise if it is missing (there is no fallback path)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(
                "libfmha_bwd.so is not built (%s); run python -m attention_backward_fmha_amd.build"
                % LIB_PATH)
        L = ctypes.CDLL(LIB_PATH)
        ap = ctypes.POINTER(Args)
        L.fmha_bwd_workspace_size.argtypes = [ap, ctypes.POINTER(ctypes.c_size_t)]
        L.fmha_bwd_prepare_workspace.argtypes = [ap, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]
        L.fmha_bwd_run.argtypes = [ap, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]
        L.fmha_bwd_run_stages.argtypes = [ap, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int,
                                          ctypes.c_void_p]
        L.fmha_bwd_plan_query.argtypes = [ap, ctypes.POINTER(PlanInfo)]
        L.fmha_fwd_run.argtypes = [ap, ctypes.c_void_p]
        L.fmha_bwd_run_noalloc.argtypes = [ap, ctypes.c_void_p]
        L.fmha_bwd_status_string.argtypes = [ctypes.c_int]
        L.fmha_bwd_status_string.restype = ctypes.c_char_p
        for name in EXPORTS:
            if name != "fmha_bwd_status_string":
                getattr(L, name).restype = ctypes.c_int
        _lib = L
    return _lib


def status_string(status):
    return lib().fmha_bwd_status_string(int(status)).decode()


def workspace_size(args):
    n = ctypes.c_size_t(0)
    st = lib().fmha_bwd_workspace_size(ctypes.byref(args), ctypes.byref(n))
    if st != OK:
        raise FmhaError(st, "fmha_bwd_workspace_size")
    return n.value


def plan_query(args):
    info = PlanInfo()
    st = lib().fmha_bwd_plan_query(ctypes.byref(args), ctypes.byref(info))
    if st != OK:
        raise FmhaError(st, "fmha_bwd_plan_query")
    return info


def prepare_workspace(args, ws_ptr, ws_bytes, stream):
    st = lib().fmha_bwd_prepare_workspace(ctypes.byref(args), ctypes.c_void_p(ws_ptr), ws_bytes,
                                          ctypes.c_void_p(stream))
    if st != OK:
        raise FmhaError(st, "fmha_bwd_prepare_workspace")


def run(args, ws_ptr, ws_bytes, stream, stages=STAGE_ALL):
    if stages == STAGE_ALL:
        st = lib().fmha_bwd_run(ctypes.byref(args), ctypes.c_void_p(ws_ptr), ws_bytes,
                                ctypes.c_void_p(stream))
    else:
        st = lib().fmha_bwd_run_stages(ctypes.byref(args), ctypes.c_void_p(ws_ptr), ws_bytes,
                                       int(stages), ctypes.c_void_p(stream))
    if st != OK:
        raise FmhaError(st, "fmha_bwd_run")


def run_noalloc(args, stream):
    st = lib().fmha_bwd_run_noalloc(ctypes.byref(args), ctypes.c_void_p(stream))
    if st != OK:
        raise FmhaError(st, "fmha_bwd_run_noalloc")


def fwd_run(args, stream):
    st = lib().fmha_fwd_run(ctypes.byref(args), ctypes.c_void_p(stream))
    if st != OK:
        raise FmhaError(st, "fmha_fwd_run")
