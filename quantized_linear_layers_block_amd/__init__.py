"""MI355X (gfx950) quantized rollout linear layer: NVFP4 and blockwise-FP8 weights with a bf16
LoRA adapter, behind the C ABI of include/qlinear.h.

    y = x . dequant(Wq)^T + s . (x A^T) B^T

``binding`` is the one-to-one ctypes binding of the C entry points (same names).  The
helpers below only allocate the output and workspace tensors with PyTorch (device memory
and the current stream are all PyTorch is used for) and call the binding; every step of
the layer runs in the HIP kernels of libqlinear.so.  Importing the package fails if the
library has not been built -- there is no fallback.
"""
from dataclasses import dataclass

import torch

from . import binding
from .binding import (QL_FP8_BLOCK128, QL_FP8_POW2, QL_NVFP4, QL_OUT_BF16, QL_OUT_F32,  # noqa: F401
                      QlinearError, make_qweight)

__all__ = ["NVFP4Weight", "FP8Weight", "quantize_nvfp4", "quantize_fp8_block", "quantize_act_fp8",
           "forward", "forward_fp8_prequant", "RequantTable", "QlinearError", "binding", "workspace_status",
           "quantize_fp8_pow2", "kv_store_fp8", "kv_load_fp8"]


def _dev(t):
    if not t.is_cuda:
        raise ValueError("tensors must live on the GPU")
    return t


@dataclass
class NVFP4Weight:
    codes: torch.Tensor         # uint8 [n, k/2]
    scales: torch.Tensor        # uint8 [n, k/16] (E4M3)
    tensor_scale: torch.Tensor  # float32 [1]
    n: int
    k: int

    def qweight(self):
        return make_qweight(QL_NVFP4, self.n, self.k, self.codes, self.scales, self.tensor_scale)

    @staticmethod
    def empty(n, k, device="cuda"):
        return NVFP4Weight(torch.empty((n, k // 2), dtype=torch.uint8, device=device),
                           torch.empty((n, k // 16), dtype=torch.uint8, device=device),
                           torch.empty((1,), dtype=torch.float32, device=device), n, k)


@dataclass
class FP8Weight:
    codes: torch.Tensor   # uint8 [n, k] (E4M3)
    scales: torch.Tensor  # float32 [n/128, k/128], or uint8 E8M0 bytes with pow2
    n: int
    k: int
    pow2: bool = False    # power-of-two block scales (QL_FP8_POW2)

    def qweight(self):
        return make_qweight(QL_FP8_POW2 if self.pow2 else QL_FP8_BLOCK128, self.n, self.k, self.codes,
                            self.scales, None)

    @staticmethod
    def empty(n, k, device="cuda", pow2=False):
        return FP8Weight(torch.empty((n, k), dtype=torch.uint8, device=device),
                         torch.empty((n // 128, k // 128), dtype=torch.uint8 if pow2 else torch.float32,
                                     device=device), n, k, pow2)


def _u16(t):
    if t.dtype != torch.bfloat16:
        raise TypeError("bf16 tensors expected")
    return t


def _ws(nbytes, device):
    # zero-filled: a workspace starts with the status word and the workgroup counters
    return torch.zeros((max(int(nbytes), 1),), dtype=torch.uint8, device=device)


def workspace_status(ws):
    """Status word (QLINEAR_STATUS_* bits) of a forward or requantization workspace."""
    return int(ws[:4].view(torch.int32).item())


def quantize_nvfp4(w, out=None, status_word=None):
    _dev(_u16(w))
    n, k = w.shape
    q = out if out is not None else NVFP4Weight.empty(n, k, w.device)
    ws = _ws(binding.qlinear_quantize_workspace(QL_NVFP4, n, k), w.device)
    binding.qlinear_quantize_nvfp4(w, q.codes, q.scales, q.tensor_scale, ws, status_word)
    return q


def quantize_fp8_block(w, out=None, status_word=None):
    _dev(_u16(w))
    n, k = w.shape
    q = out if out is not None else FP8Weight.empty(n, k, w.device)
    binding.qlinear_quantize_fp8_block(w, q.codes, q.scales, status_word)
    return q


def quantize_fp8_pow2(w, out=None, status_word=None):
    _dev(_u16(w))
    n, k = w.shape
    q = out if out is not None else FP8Weight.empty(n, k, w.device, pow2=True)
    binding.qlinear_quantize_fp8_pow2(w, q.codes, q.scales, status_word)
    return q


def quantize_act_fp8(x, pow2=False):
    _dev(_u16(x))
    m, k = x.shape
    xq = torch.empty((m, k), dtype=torch.uint8, device=x.device)
    sx = torch.empty((m, k // 128), dtype=torch.uint8 if pow2 else torch.float32, device=x.device)
    (binding.qlinear_quantize_act_fp8_pow2 if pow2 else binding.qlinear_quantize_act_fp8)(x, xq, sx)
    return xq, sx


def _fmt(qw):
    if isinstance(qw, NVFP4Weight):
        return QL_NVFP4
    return QL_FP8_POW2 if qw.pow2 else QL_FP8_BLOCK128


def forward(qw, x, lora_a=None, lora_b=None, lora_scale=0.0, out_dtype=torch.bfloat16, out=None, ws=None):
    """y = x . dequant(qw)^T + lora_scale (x A^T) B^T  (bf16 or float32 output)."""
    _dev(_u16(x))
    m = x.shape[0]
    rank = 0 if lora_a is None else lora_a.shape[0]
    if out is None:
        out = torch.empty((m, qw.n), dtype=out_dtype, device=x.device)
    od = QL_OUT_F32 if out.dtype == torch.float32 else QL_OUT_BF16
    eff_rank = rank if (lora_a is not None and lora_b is not None and lora_scale != 0) else 0
    if ws is None:
        ws = _ws(binding.qlinear_forward_workspace(_fmt(qw), m, qw.n, qw.k, eff_rank), x.device)
    binding.qlinear_forward(qw.qweight(), x, out, od, ws, lora_a, lora_b, rank, lora_scale)
    return out


def forward_group(qws, x, loras=None, lora_scale=0.0, out_dtype=torch.bfloat16, outs=None, ws=None):
    """Several NVFP4 layers on the same x (a fused q/k/v or gate/up projection): returns
    [x . dequant(qw)^T + lora_scale (x A^T) B^T for each qw]; loras is a list of (A, B)."""
    _dev(_u16(x))
    m = x.shape[0]
    if loras is None:
        loras = [(None, None)] * len(qws)
    rank = 0 if loras[0][0] is None else loras[0][0].shape[0]
    if outs is None:
        outs = [torch.empty((m, qw.n), dtype=out_dtype, device=x.device) for qw in qws]
    od = QL_OUT_F32 if outs[0].dtype == torch.float32 else QL_OUT_BF16
    with_lora = all(a is not None and b is not None for a, b in loras)
    eff_rank = rank if (with_lora and lora_scale != 0) else 0
    if ws is None:
        ws = _ws(binding.qlinear_forward_group_workspace(m, qws[0].k, [qw.n for qw in qws], eff_rank), x.device)
    layers = [(qw.qweight(), a, b, y) for qw, (a, b), y in zip(qws, loras, outs)]
    binding.qlinear_forward_group(layers, x, od, ws, rank, lora_scale)
    return outs


def forward_fp8_prequant(qw, xq, sx, x=None, lora_a=None, lora_b=None, lora_scale=0.0,
                         out_dtype=torch.bfloat16, out=None, ws=None):
    m = xq.shape[0]
    rank = 0 if lora_a is None else lora_a.shape[0]
    if out is None:
        out = torch.empty((m, qw.n), dtype=out_dtype, device=xq.device)
    od = QL_OUT_F32 if out.dtype == torch.float32 else QL_OUT_BF16
    eff_rank = rank if (lora_a is not None and lora_b is not None and lora_scale != 0) else 0
    if ws is None:
        ws = _ws(binding.qlinear_forward_prequant_workspace(m, qw.n, qw.k, eff_rank), xq.device)
    binding.qlinear_forward_fp8_prequant(qw.qweight(), xq, sx, out, od, ws, x, lora_a, lora_b, rank, lora_scale)
    return out


def backward(qw, dy, x=None, lora_a=None, lora_b=None, lora_scale=0.0, dx_dtype=torch.bfloat16, ws=None):
    """Gradients of the NVFP4 layer with LoRA: (dx, da, db); da, db are float32 (None
    without an adapter)."""
    _dev(_u16(dy))
    if not isinstance(qw, NVFP4Weight):
        raise TypeError("the backward pass is defined for NVFP4 weights")
    m = dy.shape[0]
    rank = 0 if lora_a is None else lora_a.shape[0]
    eff_rank = rank if (lora_a is not None and lora_b is not None and lora_scale != 0) else 0
    dx = torch.empty((m, qw.k), dtype=dx_dtype, device=dy.device)
    da = torch.empty((rank, qw.k), dtype=torch.float32, device=dy.device) if eff_rank else None
    db = torch.empty((qw.n, rank), dtype=torch.float32, device=dy.device) if eff_rank else None
    if ws is None:
        nb = binding.qlinear_backward_workspace(QL_NVFP4, m, qw.n, qw.k, eff_rank)
        ws = _ws(nb, dy.device) if nb else None
    od = QL_OUT_F32 if dx_dtype == torch.float32 else QL_OUT_BF16
    binding.qlinear_backward(qw.qweight(), x, dy, dx, od, da, db, ws, lora_a, lora_b, rank, lora_scale)
    return dx, da, db


class RequantTable:
    """A whole policy to requantize after every training step: a list of (bf16 weight,
    quantized weight) pairs, whose item array is copied to the device once."""

    def __init__(self, pairs, fmt=QL_NVFP4, device="cuda"):
        self.pairs = list(pairs)   # keep the tensors alive
        self.fmt = fmt
        img = binding.requant_items_bytes([(w, q.qweight()) for w, q in self.pairs])
        self.items = torch.frombuffer(bytearray(img), dtype=torch.uint8).to(device)
        self.ws = _ws(binding.qlinear_requant_workspace(len(self.pairs)), device)

    def requantize_all(self):
        binding.qlinear_requantize_all(self.items, len(self.pairs), self.fmt, self.ws)

    def set_updates(self, deltas):
        """Device pointer array of one dense bf16 update per tensor (kept alive here)."""
        self.deltas = list(deltas)
        ptrs = torch.tensor([d.data_ptr() for d in self.deltas], dtype=torch.int64)
        self.delta_ptrs = ptrs.to(self.ws.device)

    def update_requantize_all(self):
        """W <- bf16(W + delta) for every tensor, fused with the requantization."""
        binding.qlinear_update_requantize_all(self.items, self.delta_ptrs, len(self.pairs), self.fmt, self.ws)

    def status(self):
        """The workspace's status word (QLINEAR_STATUS_* bits); synchronises."""
        return int(self.ws[:4].view(torch.int32).item())


def kv_store_fp8(kv, slots, cache_codes, cache_scales, status_word=None):
    """Store bf16 kv [T, H, D] into FP8 cache rows slots[t] (codes u8 [S, H, D], scales f32 [S, H])."""
    binding.qlinear_kv_store_fp8(_dev(_u16(kv)), slots, cache_codes, cache_scales, status_word)


def kv_load_fp8(cache_codes, cache_scales, slots, heads=None, status_word=None):
    """Load cache rows `slots` back to bf16 [T, H, D]."""
    t = slots.shape[0]
    out = torch.empty((t, cache_codes.shape[1], cache_codes.shape[2]), dtype=torch.bfloat16,
                      device=cache_codes.device)
    binding.qlinear_kv_load_fp8(cache_codes, cache_scales, slots, out, status_word)
    return out
