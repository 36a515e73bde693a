"""The C ABI on the host (no GPU needed): the library loads, exports every entry point
include/qlinear.h declares, and rejects invalid arguments with the documented status
before touching the device.  The binding is loaded by file path, without the package (and
so without PyTorch), which lets test_host_sanitizers.py run this file against a build of
the ABI under the host AddressSanitizer and UndefinedBehaviorSanitizer."""
import ctypes
import importlib.util
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _binding():
    spec = importlib.util.spec_from_file_location(
        "qlinear_abi_binding", os.path.join(ROOT, "quantized_linear_layers_block_amd", "binding.py"))
    mod = importlib.util.module_from_spec(spec)
    try:
        spec.loader.exec_module(mod)
    except (ImportError, OSError) as e:
        pytest.skip(f"libqlinear is not built: {e}", allow_module_level=True)
    return mod


b = _binding()


def test_one_hip_runtime_in_process():
    # PyTorch's bundled HIP runtime and the system one must not both be mapped: the binding
    # loads PyTorch (when present) before the library, whatever imported first
    if os.environ.get("QLINEAR_NO_TORCH"):
        pytest.skip("PyTorch deliberately not loaded")
    pytest.importorskip("torch")
    with open("/proc/self/maps") as f:
        paths = {line.split()[-1] for line in f if "libamdhip64" in line}
    assert len(paths) == 1, sorted(paths)


def _declared():
    src = open(os.path.join(ROOT, "include", "qlinear.h")).read()
    return sorted(set(re.findall(r"\b(qlinear_[a-z0-9_]+)\s*\(", src)))


def test_exports_every_declared_symbol():
    declared = _declared()
    assert set(declared) == set(b.EXPORTS)
    for name in declared:
        assert hasattr(b.LIB, name), name


def test_status_strings():
    for s in range(8):
        assert b.status_string(s)
    assert b.status_string(b.QL_ERR_ALIGN) == "pointer not 16-byte aligned"


RES = b.QLINEAR_WS_RESERVED_BYTES


def test_workspace_queries():
    assert b.qlinear_quantize_workspace(b.QL_NVFP4, 256, 512) == 4096
    assert b.qlinear_quantize_workspace(b.QL_FP8_BLOCK128, 256, 512) == 0
    # every forward workspace starts with the reserved region (status word + counters)
    assert b.qlinear_forward_workspace(b.QL_NVFP4, 1, 3584, 3584, 32) > RES
    assert b.qlinear_forward_workspace(b.QL_NVFP4, 1, 3584, 3584, 0) >= RES
    # NVFP4 prefill (k % 64 == 0) holds f16 activations (m*k*2 bytes), m row factors, the
    # LoRA intermediate (m * rank rounded up to 32, bf16) and the pre-pass partials:
    # per K split, m row maxima and m * rank_pad float32 LoRA sums (16 splits here)
    m, k = 4096, 5120
    assert b.qlinear_forward_workspace(b.QL_NVFP4, m, 27648, k, 0) == RES + m * k * 2 + m * 4 + 16 * m * 4
    assert b.qlinear_forward_workspace(b.QL_NVFP4, m, 27648, k, 40) == RES + (
        m * k * 2 + m * 4 + m * 64 * 2 + 16 * m * 4 + 16 * m * 64 * 4)
    # other k take the kernel that reads bf16 activations directly: only the reserved region
    # without LoRA, plus the LoRA down-projection's t and split partials with it
    assert b.qlinear_forward_workspace(b.QL_NVFP4, 4096, 256, 5136, 0) == RES
    assert b.qlinear_forward_workspace(b.QL_NVFP4, 4096, 256, 5136, 32) > RES + 4096 * 32 * 2
    # FP8 forward holds the quantized activations (m*k bytes + scales)
    assert b.qlinear_forward_workspace(b.QL_FP8_BLOCK128, 8192, 4096, 14336, 0) >= RES + 8192 * 14336
    assert b.qlinear_forward_prequant_workspace(8192, 4096, 14336, 0) == RES
    assert b.qlinear_forward_workspace(b.QL_NVFP4, 0, 16, 16, 0) == 0
    # shapes the kernels cannot run have no workspace: FP8 k >= 2^24
    assert b.qlinear_forward_workspace(b.QL_FP8_BLOCK128, 8, 128, 1 << 24, 0) == 0
    assert b.qlinear_requant_workspace(448) >= 448 * (64 + 4)
    assert b.qlinear_requant_workspace(0) == 0
    assert b.qlinear_requant_workspace(65537) == 0


def test_status_word_is_first_int32():
    assert b.LIB.qlinear_status_word(0x20000) == 0x20000


FAKE = 0x10000  # an aligned, never-dereferenced address


def test_quantize_argument_errors():
    L = b.LIB
    assert L.qlinear_quantize_nvfp4(None, 4, 16, FAKE, FAKE, FAKE, None, FAKE, 4096, None) == b.QL_ERR_NULL
    assert L.qlinear_quantize_nvfp4(FAKE, 4, 24, FAKE, FAKE, FAKE, None, FAKE, 4096, None) == b.QL_ERR_SHAPE
    assert L.qlinear_quantize_nvfp4(FAKE, 0, 16, FAKE, FAKE, FAKE, None, FAKE, 4096, None) == b.QL_ERR_SHAPE
    assert L.qlinear_quantize_nvfp4(FAKE + 2, 4, 16, FAKE, FAKE, FAKE, None, FAKE, 4096, None) == b.QL_ERR_ALIGN
    assert L.qlinear_quantize_nvfp4(FAKE, 4, 16, FAKE, FAKE, FAKE, None, FAKE, 100, None) == b.QL_ERR_WORKSPACE
    assert L.qlinear_quantize_nvfp4(FAKE, 1 << 21, 1 << 20, FAKE, FAKE, FAKE, None, FAKE, 4096, None) == b.QL_ERR_SHAPE
    assert L.qlinear_quantize_fp8_block(FAKE, 100, 128, FAKE, FAKE, None, None) == b.QL_ERR_SHAPE
    assert L.qlinear_quantize_fp8_block(FAKE, 128, 128, None, FAKE, None, None) == b.QL_ERR_NULL
    assert L.qlinear_quantize_act_fp8(FAKE, 3, 100, FAKE, FAKE, None) == b.QL_ERR_SHAPE


def test_forward_argument_errors():
    L = b.LIB
    qw = b.QWeight(b.QL_NVFP4, 0, 256, 512, FAKE, FAKE, FAKE)
    f = lambda qw_, x=FAKE, m=4, la=None, lb=None, r=0, s=0.0, y=FAKE, od=b.QL_OUT_BF16, ws=FAKE, wsb=1 << 30: \
        L.qlinear_forward(ctypes.byref(qw_), x, m, la, lb, r, s, y, od, ws, wsb, None)
    assert f(qw, x=None) == b.QL_ERR_NULL
    assert f(qw, y=None) == b.QL_ERR_NULL
    assert f(qw, m=0) == b.QL_ERR_SHAPE
    assert f(qw, od=3) == b.QL_ERR_FORMAT
    assert f(qw, r=-1) == b.QL_ERR_ARG
    assert f(qw, r=129) == b.QL_ERR_ARG
    assert f(qw, la=FAKE, lb=FAKE, r=8, s=2.0, ws=None) == b.QL_ERR_WORKSPACE
    assert f(qw, la=FAKE, lb=FAKE, r=8, s=2.0, wsb=16) == b.QL_ERR_WORKSPACE
    assert f(qw, x=FAKE + 8) == b.QL_ERR_ALIGN
    assert f(b.QWeight(9, 0, 256, 512, FAKE, FAKE, FAKE)) == b.QL_ERR_FORMAT
    assert f(b.QWeight(b.QL_NVFP4, 0, 256, 500, FAKE, FAKE, FAKE)) == b.QL_ERR_SHAPE
    assert f(b.QWeight(b.QL_NVFP4, 0, 256, 512, FAKE, FAKE, None)) == b.QL_ERR_NULL
    assert f(b.QWeight(b.QL_FP8_BLOCK128, 0, 200, 512, FAKE, FAKE, None)) == b.QL_ERR_SHAPE
    pq = L.qlinear_forward_fp8_prequant(ctypes.byref(qw), FAKE, FAKE, 4, None, None, None, 0, 0.0, FAKE,
                                        b.QL_OUT_BF16, None, 0, None)
    assert pq == b.QL_ERR_FORMAT


def test_forward_shape_limits_before_launch():
    """Limits of the kernels are argument errors reported before anything is enqueued."""
    L = b.LIB
    qf = b.QWeight(b.QL_FP8_BLOCK128, 0, 128, 1 << 24, FAKE, FAKE, None)
    assert L.qlinear_forward(ctypes.byref(qf), FAKE, 8, None, None, 0, 0.0, FAKE, b.QL_OUT_BF16,
                             FAKE, 1 << 40, None) == b.QL_ERR_SHAPE
    pq = L.qlinear_forward_fp8_prequant(ctypes.byref(qf), FAKE, FAKE, 8, None, None, None, 0, 0.0, FAKE,
                                        b.QL_OUT_BF16, FAKE, 1 << 40, None)
    assert pq == b.QL_ERR_SHAPE
    # a few-token NVFP4 call whose counters cannot fit the reserved region
    qn = b.QWeight(b.QL_NVFP4, 0, 1 << 24, 16, FAKE, FAKE, FAKE)
    assert L.qlinear_forward(ctypes.byref(qn), FAKE, 1, None, None, 0, 0.0, FAKE, b.QL_OUT_BF16,
                             FAKE, 1 << 40, None) == b.QL_ERR_SHAPE
    assert b.qlinear_forward_workspace(b.QL_NVFP4, 1, 1 << 24, 16, 0) == 0


def test_requant_argument_errors():
    L = b.LIB
    nb = b.qlinear_requant_workspace(2)
    ra = lambda items=FAKE, count=2, fmt=b.QL_NVFP4, ws=FAKE, wsb=nb: L.qlinear_requantize_all(
        items, count, fmt, ws, wsb, None)
    assert ra(items=None) == b.QL_ERR_NULL
    assert ra(count=0) == b.QL_ERR_ARG
    assert ra(count=65537) == b.QL_ERR_ARG
    assert ra(fmt=9) == b.QL_ERR_FORMAT
    assert ra(ws=None) == b.QL_ERR_WORKSPACE
    assert ra(wsb=nb - 1) == b.QL_ERR_WORKSPACE
    assert ra(items=FAKE + 8) == b.QL_ERR_ALIGN
    assert ra(ws=FAKE + 8) == b.QL_ERR_ALIGN


def test_requant_item_layout():
    """The item array is read on the device: its layout is the header's struct."""
    assert ctypes.sizeof(b.RequantItem) == 56
    assert b.RequantItem.q.offset == 8
    assert b.QWeight.tensor_scale.offset == 40


def test_new_entry_argument_errors():
    L = b.LIB
    # power-of-two FP8 quantizers share the FP8 shape rules
    assert L.qlinear_quantize_fp8_pow2(FAKE, 100, 128, FAKE, FAKE, None, None) == b.QL_ERR_SHAPE
    assert L.qlinear_quantize_fp8_pow2(FAKE, 128, 128, None, FAKE, None, None) == b.QL_ERR_NULL
    assert L.qlinear_quantize_act_fp8_pow2(FAKE, 3, 100, FAKE, FAKE, None) == b.QL_ERR_SHAPE
    # the FP8 prequant GEMM takes both FP8 kinds but no NVFP4 weight
    qn = b.QWeight(b.QL_NVFP4, 0, 128, 128, FAKE, FAKE, FAKE)
    assert L.qlinear_forward_fp8_prequant(ctypes.byref(qn), FAKE, FAKE, 4, None, None, None, 0, 0.0, FAKE,
                                          b.QL_OUT_BF16, FAKE, 1 << 30, None) == b.QL_ERR_FORMAT
    qp = b.QWeight(b.QL_FP8_POW2, 0, 200, 128, FAKE, FAKE, None)
    assert L.qlinear_forward(ctypes.byref(qp), FAKE, 4, None, None, 0, 0.0, FAKE, b.QL_OUT_BF16,
                             FAKE, 1 << 30, None) == b.QL_ERR_SHAPE
    # fused update: the update array is required
    nb = b.qlinear_requant_workspace(1)
    assert L.qlinear_update_requantize_all(FAKE, None, 1, b.QL_NVFP4, FAKE, nb, None) == b.QL_ERR_NULL
    assert L.qlinear_update_requantize_all(FAKE, FAKE + 4, 1, b.QL_NVFP4, FAKE, nb, None) == b.QL_ERR_ALIGN
    assert L.qlinear_update_requantize_all(FAKE, FAKE, 0, b.QL_NVFP4, FAKE, nb, None) == b.QL_ERR_ARG
    # KV cache: head_dim a power of two in [16, 512], positive heads and slots
    st = lambda t=4, h=8, d=128, s=16, kv=FAKE, slots=FAKE: L.qlinear_kv_store_fp8(kv, t, h, d, slots, FAKE, FAKE, s,
                                                                                   None, None)
    assert st(d=96) == b.QL_ERR_SHAPE
    assert st(d=1024) == b.QL_ERR_SHAPE
    assert st(h=0) == b.QL_ERR_SHAPE
    assert st(s=0) == b.QL_ERR_SHAPE
    assert st(t=-1) == b.QL_ERR_SHAPE
    assert st(kv=None) == b.QL_ERR_NULL
    assert st(slots=FAKE + 4) == b.QL_ERR_ALIGN
    assert st(t=0) == b.QL_OK          # nothing to store: nothing launched
    ld = L.qlinear_kv_load_fp8(FAKE, FAKE, 16, FAKE, 4, 8, 100, FAKE, None, None)
    assert ld == b.QL_ERR_SHAPE


def test_backward_argument_errors():
    L = b.LIB
    qn = b.QWeight(b.QL_NVFP4, 0, 256, 512, FAKE, FAKE, FAKE)

    def bw(q=qn, x=FAKE, dy=FAKE, m=8, a=FAKE, bb=FAKE, r=8, s=2.0, dx=FAKE, dt=b.QL_OUT_BF16, da=FAKE, db=FAKE,
           ws=FAKE, wsb=1 << 30):
        return L.qlinear_backward(ctypes.byref(q), x, dy, m, a, bb, r, s, dx, dt, da, db, ws, wsb, None)

    assert bw(q=b.QWeight(b.QL_FP8_BLOCK128, 0, 256, 512, FAKE, FAKE, None)) == b.QL_ERR_FORMAT
    assert bw(q=b.QWeight(b.QL_NVFP4, 0, 200, 512, FAKE, FAKE, FAKE)) == b.QL_ERR_SHAPE   # n % 64
    assert bw(q=b.QWeight(b.QL_NVFP4, 0, 256, 528, FAKE, FAKE, FAKE)) == b.QL_ERR_SHAPE   # k % 128
    assert bw(m=0) == b.QL_ERR_SHAPE
    assert bw(dy=None) == b.QL_ERR_NULL
    assert bw(dx=None) == b.QL_ERR_NULL
    assert bw(x=None) == b.QL_ERR_NULL       # an adapter needs x, da and db
    assert bw(da=None) == b.QL_ERR_NULL
    assert bw(r=129) == b.QL_ERR_ARG
    assert bw(dt=7) == b.QL_ERR_FORMAT
    assert bw(dx=FAKE + 8) == b.QL_ERR_ALIGN
    assert bw(ws=None) == b.QL_ERR_WORKSPACE
    need = b.qlinear_backward_workspace(b.QL_NVFP4, 8, 256, 512, 8)
    assert need > 0 and bw(wsb=need - 1) == b.QL_ERR_WORKSPACE
    # no adapter: still a workspace (dY as f16 rows), but no x / da / db
    need0 = b.qlinear_backward_workspace(b.QL_NVFP4, 8, 256, 512, 0)
    assert 0 < need0 < need
    assert bw(x=None, a=None, bb=None, r=0, da=None, db=None, ws=None) == b.QL_ERR_WORKSPACE
    assert b.qlinear_backward_workspace(b.QL_FP8_BLOCK128, 8, 256, 512, 0) == 0
    assert b.qlinear_backward_workspace(b.QL_NVFP4, 8, 200, 512, 8) == 0


def test_forward_group_workspace_and_argument_errors():
    L = b.LIB
    m, k = 256, 5120
    # fused (m > 64, k % 64 == 0, rank % 32 == 0, count * rank <= 128): one pre-pass over x
    # with the adapters stacked (f16 x, row factors, t of 3 x 32 ranks) and one GEMM
    fused = b.qlinear_forward_group_workspace(m, k, [8192, 1024, 1024], 32)
    assert fused >= RES + m * k * 2 + m * 4 + m * 96 * 2
    # layer by layer otherwise: the largest single-layer workspace
    few = b.qlinear_forward_group_workspace(8, k, [8192, 1024], 32)
    assert few == max(b.qlinear_forward_workspace(b.QL_NVFP4, 8, n, k, 32) for n in (8192, 1024))
    odd = b.qlinear_forward_group_workspace(m, k, [512, 256], 12)  # rank not a multiple of 32
    assert odd == max(b.qlinear_forward_workspace(b.QL_NVFP4, m, n, k, 12) for n in (512, 256))
    assert b.qlinear_forward_group_workspace(m, k, [], 32) == 0
    assert b.qlinear_forward_group_workspace(m, k, [256] * 5, 32) == 0
    assert b.qlinear_forward_group_workspace(m, k, [256, 0], 32) == 0
    assert b.qlinear_forward_group_workspace(m, k, [256], 129) == 0

    def call(layers, count=None, x=FAKE, rank=0, s=0.0, ws=FAKE, wsb=1 << 40):
        arr = (b.GroupLayer * len(layers))(*layers) if layers else None
        ptr = ctypes.cast(arr, ctypes.c_void_p) if arr is not None else None
        return L.qlinear_forward_group(ptr, len(layers) if count is None else count, x, 4, rank, s,
                                       b.QL_OUT_BF16, ws, wsb, None)

    def layer(n=256, kk=512, fmt=b.QL_NVFP4, a=None, bb=None):
        return b.GroupLayer(b.QWeight(fmt, 0, n, kk, FAKE, FAKE, FAKE), a, bb, FAKE)

    assert call([]) == b.QL_ERR_NULL
    assert call([layer()], count=0) == b.QL_ERR_ARG
    assert call([layer()] * 5) == b.QL_ERR_ARG
    assert call([layer()], x=None) == b.QL_ERR_NULL
    assert call([layer(), layer(kk=1024)]) == b.QL_ERR_SHAPE
    assert call([layer(), layer(fmt=b.QL_FP8_BLOCK128)]) == b.QL_ERR_FORMAT
    assert call([layer(a=FAKE, bb=FAKE), layer()], rank=8, s=2.0) == b.QL_ERR_NULL
    assert call([layer(a=FAKE, bb=FAKE), layer(a=FAKE, bb=FAKE)], rank=8, s=2.0, wsb=64) == b.QL_ERR_WORKSPACE
    assert call([layer(), layer()], ws=None) == b.QL_ERR_WORKSPACE
