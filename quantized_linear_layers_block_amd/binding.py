"""ctypes binding of libqlinear (include/qlinear.h).

Argument marshalling only: every function here passes tensor data pointers, sizes and
the current HIP stream to the C entry point of the same name and turns a non-zero
status into QlinearError.  PyTorch supplies device memory and streams; no step of
the layer runs in Python.  The library must have been built
(quantized_linear_layers_block_amd.build); importing this module fails loudly if it
is missing.
"""
import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
# QLINEAR_LIB names another build of this same library (the host-sanitizer build of the ABI
# checks loads that way); by default the in-tree one.
LIB_PATH = os.environ.get("QLINEAR_LIB") or os.path.join(HERE, "libqlinear.so")

QL_OK, QL_ERR_NULL, QL_ERR_SHAPE, QL_ERR_ALIGN, QL_ERR_FORMAT, QL_ERR_WORKSPACE, QL_ERR_HIP, QL_ERR_ARG = range(8)
QL_NVFP4, QL_FP8_BLOCK128, QL_FP8_POW2 = 1, 2, 3
QL_OUT_BF16, QL_OUT_F32 = 1, 2

# every symbol include/qlinear.h declares
EXPORTS = [
    "qlinear_status_string",
    "qlinear_quantize_nvfp4",
    "qlinear_quantize_fp8_block",
    "qlinear_quantize_act_fp8",
    "qlinear_quantize_workspace",
    "qlinear_forward",
    "qlinear_forward_fp8_prequant",
    "qlinear_forward_workspace",
    "qlinear_forward_prequant_workspace",
    "qlinear_requant_workspace",
    "qlinear_requantize_all",
    "qlinear_status_word",
    "qlinear_forward_noalloc",
    "qlinear_quantize_fp8_pow2",
    "qlinear_quantize_act_fp8_pow2",
    "qlinear_update_requantize_all",
    "qlinear_kv_store_fp8",
    "qlinear_kv_load_fp8",
    "qlinear_backward",
    "qlinear_backward_workspace",
    "qlinear_forward_group",
    "qlinear_forward_group_workspace",
]

QLINEAR_STATUS_NONFINITE, QLINEAR_STATUS_TIMEOUT, QLINEAR_STATUS_BAD_ITEM = 1, 2, 4
QLINEAR_WS_RESERVED_BYTES = 131072
QLINEAR_NOALLOC_MAX_BYTES = 32 << 20


class QlinearError(RuntimeError):
    def __init__(self, status, where):
        self.status = status
        super().__init__(f"{where}: {status_string(status)} (status {status})")


class QWeight(ctypes.Structure):
    _fields_ = [("format", ctypes.c_int32), ("reserved", ctypes.c_int32),
                ("n", ctypes.c_int64), ("k", ctypes.c_int64),
                ("codes", ctypes.c_void_p), ("scales", ctypes.c_void_p),
                ("tensor_scale", ctypes.c_void_p)]


class RequantItem(ctypes.Structure):
    _fields_ = [("w", ctypes.c_void_p), ("q", QWeight)]


class GroupLayer(ctypes.Structure):
    _fields_ = [("w", QWeight), ("lora_a", ctypes.c_void_p), ("lora_b", ctypes.c_void_p), ("y", ctypes.c_void_p)]


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with "
                          "`python -m quantized_linear_layers_block_amd.build`")
    # One HIP runtime per process.  PyTorch ships its own libamdhip64 (same soname); loaded
    # after this library it is mapped beside the system one, and device memory and streams
    # of the one are unknown to the other (launches then fail).  Loaded first, it is the
    # runtime this library binds to.  QLINEAR_NO_TORCH=1 skips it (the host-sanitizer run
    # of the ABI checks, which launches nothing).
    if not os.environ.get("QLINEAR_NO_TORCH"):
        try:
            import torch  # noqa: F401
        except ImportError:
            pass
    lib = ctypes.CDLL(LIB_PATH)
    vp, i32, i64, sz, f32 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t, ctypes.c_float
    sig = {
        "qlinear_status_string": ([i32], ctypes.c_char_p),
        "qlinear_quantize_nvfp4": ([vp, i64, i64, vp, vp, vp, vp, vp, sz, vp], i32),
        "qlinear_quantize_fp8_block": ([vp, i64, i64, vp, vp, vp, vp], i32),
        "qlinear_quantize_act_fp8": ([vp, i64, i64, vp, vp, vp], i32),
        "qlinear_quantize_workspace": ([i32, i64, i64], sz),
        "qlinear_forward": ([ctypes.POINTER(QWeight), vp, i64, vp, vp, i32, f32, vp, i32, vp, sz, vp], i32),
        "qlinear_forward_fp8_prequant": ([ctypes.POINTER(QWeight), vp, vp, i64, vp, vp, vp, i32, f32, vp,
                                          i32, vp, sz, vp], i32),
        "qlinear_forward_workspace": ([i32, i64, i64, i64, i32], sz),
        "qlinear_forward_prequant_workspace": ([i64, i64, i64, i32], sz),
        "qlinear_requant_workspace": ([i32], sz),
        "qlinear_requantize_all": ([vp, i32, i32, vp, sz, vp], i32),
        "qlinear_status_word": ([vp], vp),
        "qlinear_forward_noalloc": ([ctypes.POINTER(QWeight), vp, i64, vp, vp, i32, f32, vp, i32, vp], i32),
        "qlinear_quantize_fp8_pow2": ([vp, i64, i64, vp, vp, vp, vp], i32),
        "qlinear_quantize_act_fp8_pow2": ([vp, i64, i64, vp, vp, vp], i32),
        "qlinear_update_requantize_all": ([vp, vp, i32, i32, vp, sz, vp], i32),
        "qlinear_kv_store_fp8": ([vp, i64, i32, i32, vp, vp, vp, i64, vp, vp], i32),
        "qlinear_kv_load_fp8": ([vp, vp, i64, vp, i64, i32, i32, vp, vp, vp], i32),
        "qlinear_backward": ([ctypes.POINTER(QWeight), vp, vp, i64, vp, vp, i32, f32, vp, i32, vp, vp, vp, sz, vp],
                             i32),
        "qlinear_backward_workspace": ([i32, i64, i64, i64, i32], sz),
        "qlinear_forward_group": ([vp, i32, vp, i64, i32, f32, i32, vp, sz, vp], i32),
        "qlinear_forward_group_workspace": ([i64, i64, vp, i32, i32], sz),
    }
    for name, (args, res) in sig.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = res
    return lib


LIB = _load()


def status_string(status):
    return LIB.qlinear_status_string(status).decode()


def _check(status, where):
    if status != QL_OK:
        raise QlinearError(status, where)


def _ptr(t):
    return None if t is None else t.data_ptr()


def _stream(stream):
    if stream is not None:
        return stream
    import torch
    return torch.cuda.current_stream().cuda_stream


# ------------------------------------------------------------------ quantizers

def qlinear_quantize_workspace(fmt, n, k):
    return LIB.qlinear_quantize_workspace(fmt, n, k)


def qlinear_quantize_nvfp4(w, codes, scales, tensor_scale, ws, status_word=None, stream=None):
    """w bf16 [n,k] -> codes u8 [n,k/2], scales u8 [n,k/16], tensor_scale f32 [1]."""
    n, k = w.shape
    _check(LIB.qlinear_quantize_nvfp4(_ptr(w), n, k, _ptr(codes), _ptr(scales), _ptr(tensor_scale),
                                      _ptr(status_word), _ptr(ws), ws.numel() * ws.element_size(),
                                      _stream(stream)), "qlinear_quantize_nvfp4")


def qlinear_quantize_fp8_block(w, codes, scales, status_word=None, stream=None):
    """w bf16 [n,k] -> codes u8 [n,k], scales f32 [n/128, k/128]."""
    n, k = w.shape
    _check(LIB.qlinear_quantize_fp8_block(_ptr(w), n, k, _ptr(codes), _ptr(scales), _ptr(status_word),
                                          _stream(stream)), "qlinear_quantize_fp8_block")


def qlinear_quantize_fp8_pow2(w, codes, scales, status_word=None, stream=None):
    """w bf16 [n,k] -> codes u8 [n,k], E8M0 scale bytes u8 [n/128, k/128]."""
    n, k = w.shape
    _check(LIB.qlinear_quantize_fp8_pow2(_ptr(w), n, k, _ptr(codes), _ptr(scales), _ptr(status_word),
                                         _stream(stream)), "qlinear_quantize_fp8_pow2")


def qlinear_quantize_act_fp8_pow2(x, xq, sx, stream=None):
    """x bf16 [m,k] -> xq u8 [m,k], E8M0 scale bytes u8 [m, k/128]."""
    m, k = x.shape
    _check(LIB.qlinear_quantize_act_fp8_pow2(_ptr(x), m, k, _ptr(xq), _ptr(sx), _stream(stream)),
           "qlinear_quantize_act_fp8_pow2")


def qlinear_quantize_act_fp8(x, xq, sx, stream=None):
    """x bf16 [m,k] -> xq u8 [m,k], sx f32 [m, k/128]."""
    m, k = x.shape
    _check(LIB.qlinear_quantize_act_fp8(_ptr(x), m, k, _ptr(xq), _ptr(sx), _stream(stream)),
           "qlinear_quantize_act_fp8")


# --------------------------------------------------------------------- forward

def make_qweight(fmt, n, k, codes, scales, tensor_scale=None):
    return QWeight(fmt, 0, n, k, _ptr(codes), _ptr(scales), _ptr(tensor_scale))


def qlinear_forward_workspace(fmt, m, n, k, rank):
    return LIB.qlinear_forward_workspace(fmt, m, n, k, rank)


def qlinear_forward_prequant_workspace(m, n, k, rank):
    return LIB.qlinear_forward_prequant_workspace(m, n, k, rank)


def qlinear_forward(qw, x, y, out_dtype, ws=None, lora_a=None, lora_b=None, rank=0, lora_scale=0.0,
                    stream=None):
    """y [m,n] = x [m,k] . dequant(qw)^T + lora_scale (x A^T) B^T."""
    m = x.shape[0]
    wsb = 0 if ws is None else ws.numel() * ws.element_size()
    _check(LIB.qlinear_forward(ctypes.byref(qw), _ptr(x), m, _ptr(lora_a), _ptr(lora_b), rank,
                               float(lora_scale), _ptr(y), out_dtype, _ptr(ws), wsb, _stream(stream)),
           "qlinear_forward")


def qlinear_forward_group_workspace(m, k, ns, rank):
    arr = (ctypes.c_int64 * len(ns))(*ns)
    return LIB.qlinear_forward_group_workspace(m, k, ctypes.cast(arr, ctypes.c_void_p), len(ns), rank)


def qlinear_forward_group(layers, x, out_dtype, ws=None, rank=0, lora_scale=0.0, stream=None):
    """Layers reading the same x [m,k]: layers is a list of (qweight, lora_a, lora_b, y)."""
    m = x.shape[0]
    wsb = 0 if ws is None else ws.numel() * ws.element_size()
    arr = (GroupLayer * len(layers))(*[GroupLayer(qw, _ptr(a), _ptr(b), _ptr(y)) for qw, a, b, y in layers])
    _check(LIB.qlinear_forward_group(ctypes.cast(arr, ctypes.c_void_p), len(layers), _ptr(x), m, rank,
                                     float(lora_scale), out_dtype, _ptr(ws), wsb, _stream(stream)),
           "qlinear_forward_group")


def qlinear_backward_workspace(fmt, m, n, k, rank):
    return LIB.qlinear_backward_workspace(fmt, m, n, k, rank)


def qlinear_backward(qw, x, dy, dx, dx_dtype, da=None, db=None, ws=None, lora_a=None, lora_b=None, rank=0,
                     lora_scale=0.0, stream=None):
    """dx [m,k] = dy . dequant(qw) + du . A; da [r,k] = du^T x; db [n,r] = dy^T t (du, t: bf16)."""
    m = dy.shape[0]
    wsb = 0 if ws is None else ws.numel() * ws.element_size()
    _check(LIB.qlinear_backward(ctypes.byref(qw), _ptr(x), _ptr(dy), m, _ptr(lora_a), _ptr(lora_b), rank,
                                float(lora_scale), _ptr(dx), dx_dtype, _ptr(da), _ptr(db), _ptr(ws), wsb,
                                _stream(stream)),
           "qlinear_backward")


def qlinear_forward_noalloc(qw, x, y, out_dtype, lora_a=None, lora_b=None, rank=0, lora_scale=0.0,
                            stream=None):
    """qlinear_forward on the library's own device array instead of a workspace."""
    m = x.shape[0]
    _check(LIB.qlinear_forward_noalloc(ctypes.byref(qw), _ptr(x), m, _ptr(lora_a), _ptr(lora_b), rank,
                                       float(lora_scale), _ptr(y), out_dtype, _stream(stream)),
           "qlinear_forward_noalloc")


def qlinear_forward_fp8_prequant(qw, xq, sx, y, out_dtype, ws=None, x=None, lora_a=None, lora_b=None,
                                 rank=0, lora_scale=0.0, stream=None):
    m = xq.shape[0]
    wsb = 0 if ws is None else ws.numel() * ws.element_size()
    _check(LIB.qlinear_forward_fp8_prequant(ctypes.byref(qw), _ptr(xq), _ptr(sx), m, _ptr(x), _ptr(lora_a),
                                            _ptr(lora_b), rank, float(lora_scale), _ptr(y), out_dtype,
                                            _ptr(ws), wsb, _stream(stream)),
           "qlinear_forward_fp8_prequant")


# --------------------------------------------------------------------- requant

def qlinear_requant_workspace(count):
    return LIB.qlinear_requant_workspace(count)


def requant_items_bytes(items):
    """items: list of (w bf16 tensor, QWeight) -> the host image of the device item array."""
    arr = (RequantItem * len(items))()
    for i, (w, qw) in enumerate(items):
        arr[i].w = _ptr(w)
        arr[i].q = qw
    return bytes(arr)


def qlinear_requantize_all(items_dev, count, fmt, ws, stream=None):
    """items_dev: device tensor holding `count` qlinear_requant_item entries."""
    _check(LIB.qlinear_requantize_all(_ptr(items_dev), count, fmt, _ptr(ws), ws.numel() * ws.element_size(),
                                      _stream(stream)), "qlinear_requantize_all")


def qlinear_update_requantize_all(items_dev, deltas_dev, count, fmt, ws, stream=None):
    """deltas_dev: device tensor holding `count` pointers (int64) to the bf16 updates."""
    _check(LIB.qlinear_update_requantize_all(_ptr(items_dev), _ptr(deltas_dev), count, fmt, _ptr(ws),
                                             ws.numel() * ws.element_size(), _stream(stream)),
           "qlinear_update_requantize_all")


# -------------------------------------------------------------------- KV cache

def qlinear_kv_store_fp8(kv, slots, cache_codes, cache_scales, status_word=None, stream=None):
    """kv bf16 [T, H, D] -> cache rows slots[t] of codes u8 [S, H, D] and scales f32 [S, H]."""
    t, h, d = kv.shape
    _check(LIB.qlinear_kv_store_fp8(_ptr(kv), t, h, d, _ptr(slots), _ptr(cache_codes), _ptr(cache_scales),
                                    cache_codes.shape[0], _ptr(status_word), _stream(stream)),
           "qlinear_kv_store_fp8")


def qlinear_kv_load_fp8(cache_codes, cache_scales, slots, out, status_word=None, stream=None):
    """cache rows slots[t] -> out bf16 [T, H, D]."""
    t, h, d = out.shape
    _check(LIB.qlinear_kv_load_fp8(_ptr(cache_codes), _ptr(cache_scales), cache_codes.shape[0], _ptr(slots), t,
                                   h, d, _ptr(out), _ptr(status_word), _stream(stream)),
           "qlinear_kv_load_fp8")


def qlinear_status_word(ws):
    """Device address of the workspace's status word (the first int32)."""
    return LIB.qlinear_status_word(_ptr(ws))
