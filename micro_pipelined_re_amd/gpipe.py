"""ctypes binding of libgpipe_cell.so (declared in include/gpipe.h).

The functions carry the C names and only marshal arguments: tensors become
device pointers, return codes become GpipeError.  Every step of the cell runs
in the library's HIP kernels; torch supplies device memory and the stream.
There is no fallback: if the library is not built, lib() raises.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libgpipe_cell.so")

GPIPE_FP32, GPIPE_BF16 = 0, 1
TENSORS = ("ln1_g", "ln1_b", "w_qkv", "b_qkv", "w_o", "b_o",
           "ln2_g", "ln2_b", "w_1", "b_1", "w_2", "b_2")
SAVED = ("x", "h1", "st1", "qkv", "p", "ctx", "x1", "h2", "st2", "u", "g")
CONV_TENSORS = ("w1", "bn1_g", "bn1_b", "w2", "bn2_g", "bn2_b")
CONV_SAVED = ("x", "a", "st1", "r", "z", "st2")

EXPORTS = ("gpipe_cell_create", "gpipe_cell_destroy", "gpipe_cell_param_count",
           "gpipe_cell_param_offset", "gpipe_cell_bind", "gpipe_cell_sync_lowp",
           "gpipe_cell_workspace_bytes", "gpipe_cell_saved_offset", "gpipe_cell_step",
           "gpipe_apply_update", "gpipe_partition", "gpipe_status_string",
           "gpipe_cell_profile", "gpipe_cell_profile_sampled", "gpipe_cell_profile_read",
           "gpipe_cell_gemm_plan",
           "gpipe_conv_cell_create", "gpipe_cell_bind_running", "gpipe_cell_forward_plan",
           "gpipe_cell_forward", "gpipe_cell_backward", "gpipe_cell_step_noalloc",
           "gpipe_cell_step_update",
           "gpipe_cell_set_logit_clip", "gpipe_cell_scale_ffn_init")

ROLES = ("ln1_fwd", "qkv_fwd", "scores_fwd", "softmax_fwd", "pv_fwd", "out_fwd", "ln2_fwd",
         "ffn1_fwd", "ffn2_fwd", "mse", "ffn2_dgrad", "ffn2_wgrad", "ffn1_dgrad", "ffn1_wgrad",
         "ln2_bwd", "out_dgrad", "out_wgrad", "dp", "dv", "softmax_bwd", "dq", "dk", "qkv_dgrad",
         "qkv_wgrad", "ln1_bwd", "bias_grad", "norm_grad", "loss_reduce", "rmsprop",
         "conv_fwd", "conv_dgrad", "conv_wgrad", "im2col", "col2im", "bn_stats", "bn_apply",
         "bn_bwd", "bn_running", "attn_fwd", "attn_delta", "attn_dkdv", "attn_dq",
         "conv_fwd_implicit", "conv_dgrad_implicit", "conv_wgrad_implicit")


class GpipeError(RuntimeError):
    def __init__(self, func: str, code: int):
        self.code = code
        super().__init__(f"{func}: {_status_string(code)} (status {code})")


_LIB = None
_sz = ctypes.c_size_t
_vp = ctypes.c_void_p
_i = ctypes.c_int


def lib() -> ctypes.CDLL:
    global _LIB
    if _LIB is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built: run `python -m micro_pipelined_re_amd.csrc.build`")
        L = ctypes.CDLL(LIB_PATH)
        sig = {
            "gpipe_cell_create": [_i, _i, _i, _i, _i, _i, _i, ctypes.POINTER(_vp)],
            "gpipe_cell_destroy": [_vp],
            "gpipe_cell_param_count": [_vp, ctypes.POINTER(_sz)],
            "gpipe_cell_param_offset": [_vp, _i, _i, ctypes.POINTER(_sz), ctypes.POINTER(_sz)],
            "gpipe_cell_bind": [_vp, _vp, _vp, _vp, _vp],
            "gpipe_cell_sync_lowp": [_vp, _vp],
            "gpipe_cell_workspace_bytes": [_vp, _i, _i, _i, ctypes.POINTER(_sz)],
            "gpipe_cell_saved_offset": [_vp, _i, _i, _i, _i, _i, _i, ctypes.POINTER(_sz),
                                        ctypes.POINTER(_sz)],
            "gpipe_cell_step": [_vp, _vp, _vp, _vp, _vp, _i, _i, _i, _vp, _sz, _vp, _vp],
            "gpipe_cell_forward": [_vp, _vp, _vp, _i, _i, _i, _vp, _sz, _vp],
            "gpipe_cell_set_logit_clip": [_vp, ctypes.c_float],
            "gpipe_cell_scale_ffn_init": [_vp, _i, _vp],
            "gpipe_cell_step_noalloc": [_vp, _vp, _vp, _vp, _vp, _i, _i, _i, _vp, _vp],
            "gpipe_cell_step_update": [_vp, _vp, _vp, _vp, _vp, _i, _i, _i, _vp, _sz, _vp, _vp,
                                       ctypes.c_float, ctypes.c_float, ctypes.c_float],
            "gpipe_cell_backward": [_vp, _vp, _vp, _vp, _i, _i, _i, _vp, _sz, _vp],
            "gpipe_apply_update": [_vp, ctypes.c_float, ctypes.c_float, ctypes.c_float, _vp],
            "gpipe_partition": [ctypes.POINTER(ctypes.c_double), _i, _i, ctypes.POINTER(_i),
                                ctypes.POINTER(ctypes.c_double)],
            "gpipe_cell_profile": [_vp, ctypes.c_ulonglong],
            "gpipe_cell_profile_sampled": [_vp, ctypes.c_ulonglong, _i],
            "gpipe_cell_gemm_plan": [_vp, _i, _i, _i, ctypes.POINTER(_i), ctypes.POINTER(_i),
                                     ctypes.POINTER(_i)],
            "gpipe_cell_profile_read": [_vp, _i, ctypes.POINTER(ctypes.c_double),
                                        ctypes.POINTER(ctypes.c_longlong)],
            "gpipe_conv_cell_create": [_i, _i, _i, _i, ctypes.c_float, _i, ctypes.POINTER(_vp)],
            "gpipe_cell_bind_running": [_vp, _vp],
            "gpipe_cell_forward_plan": [_vp, _i, _i, _i, ctypes.POINTER(_i), ctypes.POINTER(_i),
                                        ctypes.POINTER(_sz)],
        }
        for name, argtypes in sig.items():
            f = getattr(L, name)
            f.argtypes = argtypes
            f.restype = _i
        L.gpipe_status_string.argtypes = [_i]
        L.gpipe_status_string.restype = ctypes.c_char_p
        _LIB = L
    return _LIB


def _status_string(code: int) -> str:
    return lib().gpipe_status_string(code).decode()


def _check(func: str, code: int) -> None:
    if code != 0:
        raise GpipeError(func, code)


def _ptr(t):
    """Device pointer of a torch tensor, an int address, or None."""
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream):
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


# ---------------------------------------------------------------- the C entry points
def gpipe_status_string(code: int) -> str:
    return _status_string(code)


def gpipe_cell_create(layers, d_model, heads, d_ff, seq, causal, precision) -> int:
    h = _vp()
    _check("gpipe_cell_create",
           lib().gpipe_cell_create(layers, d_model, heads, d_ff, seq, int(bool(causal)),
                                   int(precision), ctypes.byref(h)))
    return h.value


def gpipe_conv_cell_create(blocks, channels, height, width, bn_momentum, precision) -> int:
    h = _vp()
    _check("gpipe_conv_cell_create",
           lib().gpipe_conv_cell_create(blocks, channels, height, width, float(bn_momentum),
                                        int(precision), ctypes.byref(h)))
    return h.value


def gpipe_cell_bind_running(cell, running) -> None:
    _check("gpipe_cell_bind_running", lib().gpipe_cell_bind_running(cell, _ptr(running)))


def gpipe_cell_destroy(cell) -> None:
    _check("gpipe_cell_destroy", lib().gpipe_cell_destroy(cell))


def gpipe_cell_param_count(cell) -> int:
    n = _sz()
    _check("gpipe_cell_param_count", lib().gpipe_cell_param_count(cell, ctypes.byref(n)))
    return n.value


def gpipe_cell_param_offset(cell, layer: int, tensor: int):
    off, cnt = _sz(), _sz()
    _check("gpipe_cell_param_offset",
           lib().gpipe_cell_param_offset(cell, layer, tensor, ctypes.byref(off), ctypes.byref(cnt)))
    return off.value, cnt.value


def gpipe_cell_bind(cell, master, w_lowp, grad, ms) -> None:
    _check("gpipe_cell_bind",
           lib().gpipe_cell_bind(cell, _ptr(master), _ptr(w_lowp), _ptr(grad), _ptr(ms)))


def gpipe_cell_sync_lowp(cell, stream=None) -> None:
    _check("gpipe_cell_sync_lowp", lib().gpipe_cell_sync_lowp(cell, _stream(stream)))


def gpipe_cell_workspace_bytes(cell, N: int, M: int, remat: bool) -> int:
    b = _sz()
    _check("gpipe_cell_workspace_bytes",
           lib().gpipe_cell_workspace_bytes(cell, N, M, int(bool(remat)), ctypes.byref(b)))
    return b.value


def gpipe_cell_workspace_fit(cell, N: int, M: int, remat: bool):
    """(plan bytes, fits): gpipe_cell_workspace_bytes with GPIPE_ERR_OOM as fits=False."""
    b = _sz()
    code = lib().gpipe_cell_workspace_bytes(cell, N, M, int(bool(remat)), ctypes.byref(b))
    if code == 2:
        return b.value, False
    _check("gpipe_cell_workspace_bytes", code)
    return b.value, True


def gpipe_cell_saved_offset(cell, N, M, remat, micro, layer, which):
    off, nb = _sz(), _sz()
    _check("gpipe_cell_saved_offset",
           lib().gpipe_cell_saved_offset(cell, N, M, int(bool(remat)), micro, layer, which,
                                         ctypes.byref(off), ctypes.byref(nb)))
    return off.value, nb.value


def gpipe_cell_step(cell, x, target, y, dx, N, M, remat, workspace, ws_bytes, stream, loss) -> None:
    _check("gpipe_cell_step",
           lib().gpipe_cell_step(cell, _ptr(x), _ptr(target), _ptr(y), _ptr(dx), N, M,
                                 int(bool(remat)), _ptr(workspace), ws_bytes, _stream(stream),
                                 _ptr(loss)))


def gpipe_cell_step_update(cell, x, target, y, dx, N, M, remat, workspace, ws_bytes, stream, loss,
                           lr, decay, eps) -> None:
    _check("gpipe_cell_step_update",
           lib().gpipe_cell_step_update(cell, _ptr(x), _ptr(target), _ptr(y), _ptr(dx), N, M,
                                        int(bool(remat)), _ptr(workspace), ws_bytes,
                                        _stream(stream), _ptr(loss), lr, decay, eps))


GPIPE_SCRATCH_BYTES = 64 << 20


def gpipe_cell_step_noalloc(cell, x, target, y, dx, N, M, remat, stream, loss) -> None:
    _check("gpipe_cell_step_noalloc",
           lib().gpipe_cell_step_noalloc(cell, _ptr(x), _ptr(target), _ptr(y), _ptr(dx), N, M,
                                         int(bool(remat)), _stream(stream), _ptr(loss)))


def gpipe_cell_forward(cell, x, y, N, M, remat, workspace, ws_bytes, stream) -> None:
    _check("gpipe_cell_forward",
           lib().gpipe_cell_forward(cell, _ptr(x), _ptr(y), N, M, int(bool(remat)),
                                    _ptr(workspace), ws_bytes, _stream(stream)))


def gpipe_cell_backward(cell, x, dy, dx, N, M, remat, workspace, ws_bytes, stream) -> None:
    _check("gpipe_cell_backward",
           lib().gpipe_cell_backward(cell, _ptr(x), _ptr(dy), _ptr(dx), N, M, int(bool(remat)),
                                     _ptr(workspace), ws_bytes, _stream(stream)))


def gpipe_cell_set_logit_clip(cell, threshold: float) -> None:
    _check("gpipe_cell_set_logit_clip", lib().gpipe_cell_set_logit_clip(cell, float(threshold)))


def gpipe_cell_scale_ffn_init(cell, total_layers: int, stream=None) -> None:
    _check("gpipe_cell_scale_ffn_init",
           lib().gpipe_cell_scale_ffn_init(cell, int(total_layers), _stream(stream)))


def gpipe_apply_update(cell, lr, decay, eps, stream=None) -> None:
    _check("gpipe_apply_update", lib().gpipe_apply_update(cell, lr, decay, eps, _stream(stream)))


def gpipe_partition(costs, K: int):
    c = np.ascontiguousarray(costs, dtype=np.float64)
    bounds = (_i * (K + 1))()
    var = ctypes.c_double()
    _check("gpipe_partition",
           lib().gpipe_partition(c.ctypes.data_as(ctypes.POINTER(ctypes.c_double)), int(c.size), K,
                                 bounds, ctypes.byref(var)))
    return list(bounds), var.value


def gpipe_cell_profile(cell, role_mask: int) -> None:
    _check("gpipe_cell_profile", lib().gpipe_cell_profile(cell, role_mask))


def gpipe_cell_profile_sampled(cell, role_mask: int, every: int) -> None:
    _check("gpipe_cell_profile_sampled", lib().gpipe_cell_profile_sampled(cell, role_mask, every))


def gpipe_cell_profile_read(cell, role: int):
    ms, n = ctypes.c_double(), ctypes.c_longlong()
    _check("gpipe_cell_profile_read",
           lib().gpipe_cell_profile_read(cell, role, ctypes.byref(ms), ctypes.byref(n)))
    return ms.value, n.value


def gpipe_cell_gemm_plan(cell, N: int, M: int, role: int):
    tm, tn, sp = _i(), _i(), _i()
    _check("gpipe_cell_gemm_plan",
           lib().gpipe_cell_gemm_plan(cell, N, M, role, ctypes.byref(tm), ctypes.byref(tn),
                                      ctypes.byref(sp)))
    return tm.value, tn.value, sp.value


def gpipe_cell_forward_plan(cell, N: int, M: int, remat: bool):
    lanes, group, nb = _i(), _i(), _sz()
    _check("gpipe_cell_forward_plan",
           lib().gpipe_cell_forward_plan(cell, N, M, int(bool(remat)), ctypes.byref(lanes),
                                         ctypes.byref(group), ctypes.byref(nb)))
    return lanes.value, group.value, nb.value


# ---------------------------------------------------------------- convenience
class Cell:
    """A cell plus the device buffers the caller owns (torch tensors).

    Allocation and host<->device copies only; compute is the library's.
    """

    def __init__(self, layers, d_model, heads, d_ff, seq, causal, precision, device="cuda"):
        import torch
        self.torch = torch
        self.layers, self.d_model, self.heads, self.d_ff, self.seq = layers, d_model, heads, d_ff, seq
        self.causal = bool(causal)
        self.precision = precision
        self.bf16 = precision in ("bf16", GPIPE_BF16)
        self.device = device
        self.handle = gpipe_cell_create(layers, d_model, heads, d_ff, seq, causal,
                                        GPIPE_BF16 if self.bf16 else GPIPE_FP32)
        self.n_params = gpipe_cell_param_count(self.handle)
        self.act_dtype = torch.bfloat16 if self.bf16 else torch.float32
        n = self.n_params
        self.master = torch.zeros(n, dtype=torch.float32, device=device)
        self.w_lowp = torch.zeros(n, dtype=torch.bfloat16, device=device) if self.bf16 else None
        self.grad = torch.zeros(n, dtype=torch.float32, device=device)
        self.ms = torch.zeros(n, dtype=torch.float32, device=device)
        gpipe_cell_bind(self.handle, self.master, self.w_lowp, self.grad, self.ms)
        self.loss = torch.zeros(1, dtype=torch.float32, device=device)
        self._ws = None
        self._plans = {}

    @classmethod
    def from_config(cls, cfg, device="cuda"):
        return cls(cfg.layers, cfg.d_model, cfg.heads, cfg.d_ff, cfg.seq, cfg.causal,
                   cfg.precision, device)

    def __del__(self):
        try:
            if getattr(self, "handle", None):
                gpipe_cell_destroy(self.handle)
                self.handle = None
        except Exception:
            pass

    # -- parameters ---------------------------------------------------------
    def offsets(self):
        return [[gpipe_cell_param_offset(self.handle, l, t) for t in range(len(TENSORS))]
                for l in range(self.layers)]

    def load_params(self, flat: np.ndarray) -> None:
        """Copies float32 master weights (flat layout) and makes the bf16 copy."""
        assert flat.size == self.n_params
        self.master.copy_(self.torch.from_numpy(np.ascontiguousarray(flat, np.float32)))
        gpipe_cell_sync_lowp(self.handle)

    def unflatten(self, flat):
        """Flat host vector -> list of per-layer dicts keyed by tensor name."""
        from .inputs import param_shapes
        shapes = param_shapes(self.d_model, self.d_ff)
        out = []
        for l, offs in enumerate(self.offsets()):
            out.append({name: np.asarray(flat[o:o + c]).reshape(shapes[name])
                        for name, (o, c) in zip(TENSORS, offs)})
        return out

    # -- activations --------------------------------------------------------
    def to_device(self, a: np.ndarray):
        """Host float32 array -> device tensor of the cell's activation type.

        bf16 cells take bf16-representable values; their bit patterns are
        copied as they are (no conversion arithmetic)."""
        torch = self.torch
        if self.bf16:
            from .inputs import bf16_bits
            bits = torch.from_numpy(bf16_bits(a).view(np.int16))
            return bits.to(self.device).view(torch.bfloat16)
        return torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(self.device)

    def workspace(self, N, M, remat=True):
        """The workspace for (N, M, remat).  Each plan is queried once, before
        anything is allocated for it (the query's fit check counts a workspace
        already held as used memory); a refused plan that the held workspace
        cannot cover releases it and is asked again, raising GpipeError (OOM)
        if it still does not fit."""
        key = (N, M, bool(remat))
        nb = self._plans.get(key)
        if nb is None:
            nb, fits = gpipe_cell_workspace_fit(self.handle, N, M, remat)
            held = 0 if self._ws is None else self._ws.numel()
            if not fits and nb > held:
                self._ws = None
                self.torch.cuda.empty_cache()
                nb = gpipe_cell_workspace_bytes(self.handle, N, M, remat)
            self._plans[key] = nb
        if self._ws is None or self._ws.numel() < nb:
            self._ws = None
            self._ws = self.torch.empty(max(nb, 1), dtype=self.torch.uint8, device=self.device)
        return self._ws, nb

    def step(self, x, t, N, M, remat=True, want_dx=True, y=None, dx=None, stream=None):
        torch = self.torch
        if y is None:
            y = torch.empty_like(x)
        if want_dx and dx is None:
            dx = torch.empty_like(x)
        ws, nb = self.workspace(N, M, remat)
        gpipe_cell_step(self.handle, x, t, y, dx if want_dx else None, N, M, remat, ws, nb,
                        stream, self.loss)
        return y, (dx if want_dx else None)

    def step_update(self, x, t, N, M, lr, decay, eps, remat=True, want_dx=True, y=None, dx=None,
                    stream=None):
        """step() and update() in one call (each layer updated once its gradients are complete)."""
        torch = self.torch
        if y is None:
            y = torch.empty_like(x)
        if want_dx and dx is None:
            dx = torch.empty_like(x)
        ws, nb = self.workspace(N, M, remat)
        gpipe_cell_step_update(self.handle, x, t, y, dx if want_dx else None, N, M, remat, ws, nb,
                               stream, self.loss, lr, decay, eps)
        return y, (dx if want_dx else None)

    def forward(self, x, N, M, remat=True, y=None, stream=None):
        """Phase 1 only: y of every micro-batch (for a cell below others)."""
        if y is None:
            y = self.torch.empty_like(x)
        ws, nb = self.workspace(N, M, remat)
        gpipe_cell_forward(self.handle, x, y, N, M, remat, ws, nb, stream)
        return y

    def backward(self, x, dy, N, M, remat=True, want_dx=True, dx=None, stream=None):
        """Phase 2 with the output gradient dy handed down by the cell above."""
        if want_dx and dx is None:
            dx = self.torch.empty_like(x)
        ws, nb = self.workspace(N, M, remat)
        gpipe_cell_backward(self.handle, x, dy, dx if want_dx else None, N, M, remat, ws, nb,
                            stream)
        return dx if want_dx else None

    def update(self, lr, decay, eps, stream=None):
        gpipe_apply_update(self.handle, lr, decay, eps, stream)


class ConvCell(Cell):
    """A conv cell (residual blocks with micro-batch BatchNorm) plus its buffers.

    running: float32 [blocks][2][mean[C], var[C]], initialised to mean 0, var 1."""

    def __init__(self, blocks, channels, height, width, bn_momentum, precision, device="cuda"):
        import torch
        self.torch = torch
        self.layers, self.channels, self.height, self.width = blocks, channels, height, width
        self.precision = precision
        self.bf16 = precision in ("bf16", GPIPE_BF16)
        self.device = device
        self.handle = gpipe_conv_cell_create(blocks, channels, height, width, bn_momentum,
                                             GPIPE_BF16 if self.bf16 else GPIPE_FP32)
        self.n_params = gpipe_cell_param_count(self.handle)
        self.act_dtype = torch.bfloat16 if self.bf16 else torch.float32
        n = self.n_params
        self.master = torch.zeros(n, dtype=torch.float32, device=device)
        self.w_lowp = torch.zeros(n, dtype=torch.bfloat16, device=device) if self.bf16 else None
        self.grad = torch.zeros(n, dtype=torch.float32, device=device)
        self.ms = torch.zeros(n, dtype=torch.float32, device=device)
        gpipe_cell_bind(self.handle, self.master, self.w_lowp, self.grad, self.ms)
        self.running = torch.zeros(blocks, 2, 2, channels, dtype=torch.float32, device=device)
        self.running[:, :, 1, :] = 1.0
        gpipe_cell_bind_running(self.handle, self.running)
        self.loss = torch.zeros(1, dtype=torch.float32, device=device)
        self._ws = None
        self._plans = {}

    @classmethod
    def from_config(cls, cfg, device="cuda"):
        return cls(cfg.blocks, cfg.channels, cfg.height, cfg.width, cfg.bn_momentum,
                   cfg.precision, device)

    def offsets(self):
        return [[gpipe_cell_param_offset(self.handle, l, t) for t in range(len(CONV_TENSORS))]
                for l in range(self.layers)]

    def unflatten(self, flat):
        from .inputs import conv_param_shapes
        shapes = conv_param_shapes(self.channels)
        return [{name: np.asarray(flat[o:o + c]).reshape(shapes[name])
                 for name, (o, c) in zip(CONV_TENSORS, offs)} for offs in self.offsets()]
