"""MI355X (gfx950) training-step library: Python binding over the C ABI.

The functions below only marshal arguments: torch tensors provide device
memory and the current HIP stream, and every step of the computation runs in
the HIP kernels of ``libnc.so`` (see include/nc.h).  Nothing here computes on
the host, and nothing falls back to PyTorch: a missing library raises.
"""

import ctypes

from . import _nc
from ._nc import NC_BF16, NC_FP32, NcConfig, NcError, NcTensorDesc, check, lib

__all__ = ["Model", "NC_BF16", "NC_FP32", "NcError", "lib", "ops"]


def _dtype_code(dtype):
    if dtype in ("bf16", NC_BF16):
        return NC_BF16
    if dtype in ("fp32", "f32", NC_FP32):
        return NC_FP32
    raise ValueError(f"dtype must be 'bf16' or 'fp32', got {dtype!r}")


def _stream(stream=None):
    """A HIP stream handle: a torch stream, a raw handle, or (None) torch's current stream."""
    if stream is not None:
        return ctypes.c_void_p(stream.cuda_stream) if hasattr(stream, "cuda_stream") else stream
    import torch
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else None


class Model:
    """One nc context: configuration, parameter layout and workspace.

    depth drives d_model = 64*depth, n_heads = d_model/128, head_dim = 128 and
    d_ff = 4*d_model unless overridden; n_kv_heads < n_heads gives grouped-query
    attention.
    """

    def __init__(self, depth, vocab=65536, seq_len=2048, max_batch=1, dtype="bf16", d_model=0,
                 n_heads=0, head_dim=0, d_ff=0, rope_base=10000.0, eps=1e-6, stream=None, n_kv_heads=0):
        cfg = NcConfig(depth, d_model, n_heads, head_dim, d_ff, vocab, seq_len, max_batch,
                       rope_base, eps, _dtype_code(dtype), n_kv_heads)
        h = ctypes.c_void_p()
        s = stream if stream is not None else None
        check(lib().nc_init(ctypes.byref(cfg), s, ctypes.byref(h)), "nc_init")
        self._h = h
        self._ws = None
        out = NcConfig()
        check(lib().nc_get_config(h, ctypes.byref(out)), "nc_get_config")
        self.config = {f: getattr(out, f) for f, _ in NcConfig._fields_}
        self.dtype = out.dtype

    def __del__(self):
        h = getattr(self, "_h", None)
        if h:
            try:
                lib().nc_destroy(h)
            except Exception:
                pass
            self._h = None

    @property
    def param_count(self):
        return int(lib().nc_param_count(self._h))

    def layout(self):
        n = lib().nc_param_layout(self._h, None, 0)
        arr = (NcTensorDesc * n)()
        lib().nc_param_layout(self._h, arr, n)
        return [(a.name.decode(), int(a.offset), int(a.rows), int(a.cols)) for a in arr]

    def workspace_bytes(self, batch):
        return int(lib().nc_workspace_bytes(self._h, batch))

    def set_stream(self, stream=None):
        check(lib().nc_set_stream(self._h, _stream(stream)), "nc_set_stream")

    def ensure_workspace(self, batch):
        """Allocate (with torch) a workspace large enough for `batch` sequences."""
        import torch
        need = self.workspace_bytes(batch)
        if need == 0:
            raise ValueError(f"invalid batch {batch}")
        if self._ws is None or self._ws.numel() < need:
            self._ws = None
            self._ws = torch.empty(need, dtype=torch.uint8, device="cuda")
            self.set_stream()
            check(lib().nc_set_workspace(self._h, _ptr(self._ws), need), "nc_set_workspace")
        return self._ws

    def forward_backward(self, params, tokens, targets, loss, grads, accumulate=False):
        batch = tokens.shape[0]
        self.ensure_workspace(batch)
        self.set_stream()
        check(lib().nc_forward_backward(self._h, _ptr(params), _ptr(tokens), _ptr(targets), batch,
                                        _ptr(loss), _ptr(grads), int(bool(accumulate))),
              "nc_forward_backward")

    def forward_backward_accum(self, params, tokens, targets, n_micro, loss, grads):
        """One step over tokens [n_micro * micro_batch, T] as n_micro microbatches (gradient accumulation)."""
        rows = tokens.shape[0]
        if n_micro < 1 or rows % n_micro:
            raise ValueError(f"{rows} sequences do not split into {n_micro} microbatches")
        micro = rows // n_micro
        self.ensure_workspace(micro)
        self.set_stream()
        check(lib().nc_forward_backward_accum(self._h, _ptr(params), _ptr(tokens), _ptr(targets), int(n_micro),
                                              micro, _ptr(loss), _ptr(grads)),
              "nc_forward_backward_accum")

    def forward_logits(self, params, tokens, logits):
        batch = tokens.shape[0]
        self.ensure_workspace(batch)
        self.set_stream()
        check(lib().nc_forward_logits(self._h, _ptr(params), _ptr(tokens), batch, _ptr(logits)),
              "nc_forward_logits")

    # ---- inference with a KV cache (nc_prefill, nc_decode)
    def kv_cache_bytes(self, cache_batch, max_len):
        return int(lib().nc_kv_cache_bytes(self._h, cache_batch, max_len))

    def decode_workspace_bytes(self, batch, max_len):
        return int(lib().nc_decode_workspace_bytes(self._h, batch, max_len))

    def prefill(self, params, tokens, cache, cache_batch, max_len, logits, slot0=0):
        """tokens [batch, len] into cache slots slot0..; logits [batch, V] of the last positions."""
        batch, length = tokens.shape
        self.ensure_workspace(batch)
        self.set_stream()
        check(lib().nc_prefill(self._h, _ptr(params), _ptr(tokens), batch, length, _ptr(cache), int(cache_batch),
                               int(max_len), int(slot0), _ptr(logits)),
              "nc_prefill")

    def decode(self, params, tokens, pos, cache, max_len, workspace, logits):
        """One token per sequence (tokens [B], pos [B] int32 on the device); logits [B, V]."""
        self.set_stream()
        check(lib().nc_decode(self._h, _ptr(params), _ptr(tokens), _ptr(pos), tokens.shape[0], _ptr(cache),
                              int(max_len), _ptr(workspace), workspace.numel() * workspace.element_size(),
                              _ptr(logits)),
              "nc_decode")

    def profile(self, on=True):
        """Enable (and clear) or disable per-kernel-class event timing."""
        check(lib().nc_profile_enable(self._h, int(bool(on))), "nc_profile_enable")

    def profile_read(self):
        """Dict class -> (launches, ms, flops, bytes) accumulated since enabling."""
        n = lib().nc_profile_read(self._h, None, 0)
        if n < 0:
            raise NcError(-n, "nc_profile_read")
        arr = (_nc.NcProfEntry * n)()
        lib().nc_profile_read(self._h, arr, n)
        return {a.name.decode(): (int(a.launches), a.ms, a.flops, a.bytes) for a in arr}

    def check(self):
        """Synchronise and return the device status code (0 = ok)."""
        return int(lib().nc_check(self._h))

    def set_residual_fp32(self, on=True):
        """bf16 path: add the attention / MLP outputs to the residual stream in
        fp32 in the projection epilogue instead of as bf16 (nc_set_residual_fp32)."""
        check(lib().nc_set_residual_fp32(self._h, int(bool(on))), "nc_set_residual_fp32")

    def poison_workspace(self, on=True):
        """Debug: NaN-fill the workspace before each call (nc_debug_poison_workspace)."""
        check(lib().nc_debug_poison_workspace(self._h, int(bool(on))), "nc_debug_poison_workspace")

    # ---- optimizer step (nc_optim_*)
    OPTIM_DEFAULTS = dict(lr_adamw=3e-3, lr_muon=0.02, beta1=0.9, beta2=0.95, eps=1e-8, momentum=0.95,
                          weight_decay=0.1, clip=1.0, final_frac=0.0, warmup_steps=1, total_steps=1, ns_steps=5)

    def optim_state_bytes(self):
        return int(lib().nc_optim_state_bytes(self._h))

    def optim_workspace_bytes(self):
        return int(lib().nc_optim_workspace_bytes(self._h))

    def optim_init(self, params, state):
        """Masters = params, moments = 0 (state: device buffer of optim_state_bytes())."""
        self.set_stream()
        check(lib().nc_optim_init(self._h, _ptr(params), _ptr(state)), "nc_optim_init")

    def optim_step(self, step, grads, params, state, workspace, grad_norm=None, **hp):
        """One optimizer step; hp overrides OPTIM_DEFAULTS (nc_optim_config fields)."""
        vals = dict(self.OPTIM_DEFAULTS)
        unknown = set(hp) - set(vals)
        if unknown:
            raise TypeError(f"unknown optimizer settings {sorted(unknown)}")
        vals.update(hp)
        cfg = _nc.NcOptimConfig(**vals)
        self.set_stream()
        check(lib().nc_optim_step(self._h, ctypes.byref(cfg), int(step), _ptr(grads), _ptr(params), _ptr(state),
                                  _ptr(workspace), workspace.numel() * workspace.element_size(),
                                  _ptr(grad_norm) if grad_norm is not None else None),
              "nc_optim_step")


from . import ops  # noqa: E402,F401
