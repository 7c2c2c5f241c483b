"""ctypes binding of libsmolexp.so: the C ABI of include/smolexp.h, same names.

Argument marshalling only.  Tensors are torch tensors on the handle's GPU
(torch supplies device memory and the current stream); every step of the
denoising loop runs in the library's HIP kernels.  There is no fallback: if
the library is missing the import fails.
"""
import ctypes
import os

# torch ships its own HIP runtime under the soname libamdhip64.so.7.  Loading
# torch first makes the dynamic loader bind this library to that same runtime
# instead of bringing in a second copy from /opt/rocm (two HIP runtimes in one
# process leave torch without a device).
import torch  # noqa: F401  (load order matters)

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libsmolexp.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(
        f"{LIB_PATH} is missing: build it with `python flow_matching_action_step_amd/build.py` "
        "(hipcc, gfx950). There is no fallback implementation.")
_lib = ctypes.CDLL(LIB_PATH)

SMOLEXP_OK, SMOLEXP_E_INVAL, SMOLEXP_E_STATE, SMOLEXP_E_SIZE, SMOLEXP_E_NOMEM, SMOLEXP_E_HIP = 0, -1, -2, -3, -4, -5

# kernel ids of smolexp_time_kernel
(K_QKV, K_ATTN_SELF, K_ATTN_CROSS, K_O, K_GATE_UP, K_DOWN, K_ACTION_OUT, K_WHOLE_LOOP, K_Q_CROSS, K_TIME_IN,
 K_TIME_OUT) = range(11)


class smolexp_config(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int) for n in ("n_layers", "d_model", "n_q_heads", "n_kv_heads", "head_dim", "ffn",
                                             "chunk", "action_dim", "n_steps", "max_batch", "max_prefix")] + \
               [(n, ctypes.c_float) for n in ("rope_theta", "rms_eps", "t_min_period", "t_max_period")] + \
               [("use_graphs", ctypes.c_int), ("batch_groups", ctypes.c_int), ("weight_format", ctypes.c_int)]


class smolexp_denoise_opts(ctypes.Structure):
    _fields_ = [("prev_actions", ctypes.c_void_p), ("overwrite_rows", ctypes.c_int),
                ("out_velocities", ctypes.c_void_p), ("out_states", ctypes.c_void_p),
                ("out_status", ctypes.c_void_p)]


SMOLEXP_RANGE_RESIDUAL, SMOLEXP_RANGE_FFN, SMOLEXP_RANGE_ATTENTION, SMOLEXP_RANGE_TIME = 1, 2, 4, 8
SMOLEXP_WEIGHTS_FP16, SMOLEXP_WEIGHTS_E4M3 = 0, 1


_H = ctypes.c_void_p
_P = ctypes.c_void_p
_sig = {
    "smolexp_default_config": (None, [ctypes.POINTER(smolexp_config)]),
    "smolexp_weight_count": (ctypes.c_size_t, [ctypes.POINTER(smolexp_config)]),
    "smolexp_schedule": (ctypes.c_int, [ctypes.POINTER(smolexp_config), ctypes.POINTER(ctypes.c_float),
                                        ctypes.POINTER(ctypes.c_float)]),
    "smolexp_batch_groups": (ctypes.c_int, [ctypes.POINTER(smolexp_config), ctypes.c_int,
                                            ctypes.POINTER(ctypes.c_int)]),
    "smolexp_quantize_e4m3_rows": (ctypes.c_int, [_P, ctypes.c_int, ctypes.c_int, _P, _P]),
    "smolexp_create": (ctypes.c_int, [ctypes.POINTER(smolexp_config), ctypes.c_int, ctypes.POINTER(_H)]),
    "smolexp_load_weights": (ctypes.c_int, [_H, _P, ctypes.c_size_t]),
    "smolexp_denoise": (ctypes.c_int, [_H, _P, _P, ctypes.c_int, _P, _P, ctypes.c_int, _P]),
    "smolexp_denoise_ex": (ctypes.c_int, [_H, _P, _P, ctypes.c_int, _P, _P, ctypes.c_int, _P,
                                          ctypes.POINTER(smolexp_denoise_opts)]),
    "smolexp_denoise_noalloc": (ctypes.c_int, [_H, _P, _P, ctypes.c_int, _P, _P, ctypes.c_int, _P]),
    "smolexp_velocity": (ctypes.c_int, [_H, _P, _P, ctypes.c_int, _P, ctypes.c_float, _P, ctypes.c_int, _P]),
    "smolexp_time_kernel": (ctypes.c_int, [_H, ctypes.c_int, ctypes.c_int, _P, ctypes.POINTER(ctypes.c_float)]),
    "smolexp_lm_weight_count": (ctypes.c_size_t, [ctypes.POINTER(smolexp_config)]),
    "smolexp_load_lm_weights": (ctypes.c_int, [_H, _P, ctypes.c_size_t]),
    "smolexp_prefill": (ctypes.c_int, [_H, _P, _P, ctypes.c_int, _P, ctypes.c_int, _P]),
    "smolexp_train_step": (ctypes.c_int, [_H, _P, _P, ctypes.c_int, _P, _P, _P, _P, _P, ctypes.c_int, _P]),
    "smolexp_strerror": (ctypes.c_char_p, [ctypes.c_int]),
    "smolexp_last_error": (ctypes.c_char_p, [_H]),
    "smolexp_destroy": (None, [_H]),
}
for _name, (_res, _args) in _sig.items():
    _f = getattr(_lib, _name)
    _f.restype = _res
    _f.argtypes = _args

EXPORTED = tuple(_sig)


class SmolexpError(RuntimeError):
    def __init__(self, code, message):
        super().__init__(f"{message} (code {code}: {_lib.smolexp_strerror(code).decode()})")
        self.code = code


def _check(rc, h=None, what="smolexp"):
    if rc != SMOLEXP_OK:
        msg = _lib.smolexp_last_error(h).decode() if h else ""
        raise SmolexpError(rc, f"{what}: {msg}" if msg else what)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is not None:
        return ctypes.c_void_p(int(stream))
    import torch
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _need(t, name, dtype, shape=None):
    if t is None:
        raise ValueError(f"{name} is required")
    if not t.is_cuda or not t.is_contiguous() or t.dtype != dtype:
        raise ValueError(f"{name} must be a contiguous CUDA tensor of dtype {dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")


def smolexp_default_config(**overrides):
    c = smolexp_config()
    _lib.smolexp_default_config(ctypes.byref(c))
    for k, v in overrides.items():
        setattr(c, k, v)
    return c


def smolexp_weight_count(cfg):
    return int(_lib.smolexp_weight_count(ctypes.byref(cfg)))


def smolexp_schedule(cfg):
    t = (ctypes.c_float * max(cfg.n_steps, 1))()
    dt = ctypes.c_float()
    _check(_lib.smolexp_schedule(ctypes.byref(cfg), t, ctypes.byref(dt)), what="smolexp_schedule")
    return [t[i] for i in range(cfg.n_steps)], dt.value


def smolexp_batch_groups(cfg, batch):
    """Queries per concurrent group of a call with `batch` queries (host only)."""
    sizes = (ctypes.c_int * 8)()
    n = _lib.smolexp_batch_groups(ctypes.byref(cfg), int(batch), sizes)
    _check(min(n, 0), what="smolexp_batch_groups")
    return [sizes[i] for i in range(n)]


def smolexp_quantize_e4m3_rows(w):
    """E4M3 codes (uint8 [rows, cols]) and row scales (float32 [rows]) of a float64 numpy
    matrix, as the library stores 8-bit weights (host only)."""
    import numpy as np
    w = np.ascontiguousarray(w, dtype=np.float64)
    if w.ndim != 2:
        raise ValueError("w must be a 2-d matrix")
    rows, cols = w.shape
    codes = np.zeros((rows, cols), np.uint8)
    scales = np.zeros(rows, np.float32)
    _check(_lib.smolexp_quantize_e4m3_rows(w.ctypes.data_as(ctypes.c_void_p), rows, cols,
                                           codes.ctypes.data_as(ctypes.c_void_p),
                                           scales.ctypes.data_as(ctypes.c_void_p)), what="smolexp_quantize_e4m3_rows")
    return codes, scales


def smolexp_create(cfg, hip_device=0):
    h = _H()
    _check(_lib.smolexp_create(ctypes.byref(cfg), int(hip_device), ctypes.byref(h)), what="smolexp_create")
    return h


def smolexp_load_weights(h, bf16_flat):
    """bf16_flat: numpy uint16 array (bf16 bit patterns) in manifest order."""
    import numpy as np
    a = np.ascontiguousarray(bf16_flat, dtype=np.uint16)
    _check(_lib.smolexp_load_weights(h, a.ctypes.data_as(ctypes.c_void_p), a.size), h, "smolexp_load_weights")


def _kv_shape(cfg, B, P):
    return (cfg.n_layers, 2, B, cfg.n_kv_heads, P, cfg.head_dim)


def smolexp_denoise(h, cfg, prefix_kv, prefix_mask, noise, out_actions, stream=None):
    return smolexp_denoise_ex(h, cfg, prefix_kv, prefix_mask, noise, out_actions, stream=stream)


def smolexp_denoise_ex(h, cfg, prefix_kv, prefix_mask, noise, out_actions, prev_actions=None,
                       overwrite_rows=0, out_velocities=None, out_states=None, out_status=None, stream=None):
    """prefix_kv: uint16/bfloat16 [L,2,B,5,P,64]; prefix_mask uint8 [B,P]; noise, out fp32 [B,50,32]."""
    import torch
    B, P = prefix_mask.shape
    _need(prefix_mask, "prefix_mask", torch.uint8)
    if prefix_kv.dtype not in (torch.bfloat16, torch.uint16, torch.int16):
        raise ValueError("prefix_kv must hold bf16 values")
    _need(prefix_kv, "prefix_kv", prefix_kv.dtype, _kv_shape(cfg, B, P))
    _need(noise, "noise", torch.float32, (B, cfg.chunk, cfg.action_dim))
    _need(out_actions, "out_actions", torch.float32, (B, cfg.chunk, cfg.action_dim))
    opts = smolexp_denoise_opts()
    opts.overwrite_rows = int(overwrite_rows)
    if prev_actions is not None:
        _need(prev_actions, "prev_actions", torch.float32, (B, int(overwrite_rows), cfg.action_dim))
        opts.prev_actions = prev_actions.data_ptr()
    for name, t in (("out_velocities", out_velocities), ("out_states", out_states)):
        if t is not None:
            _need(t, name, torch.float32, (cfg.n_steps, B, cfg.chunk, cfg.action_dim))
            setattr(opts, name, t.data_ptr())
    if out_status is not None:
        _need(out_status, "out_status", torch.int32, (1,))
        opts.out_status = out_status.data_ptr()
    rc = _lib.smolexp_denoise_ex(h, _ptr(prefix_kv), _ptr(prefix_mask), P, _ptr(noise), _ptr(out_actions), B,
                                 _stream(stream), ctypes.byref(opts))
    _check(rc, h, "smolexp_denoise_ex")


def smolexp_denoise_noalloc(h, cfg, prefix_kv, prefix_mask, noise, out_actions, stream=None):
    """As smolexp_denoise, on the library's fixed workspace (batch <= 16; allocates nothing)."""
    import torch
    B, P = prefix_mask.shape
    _need(prefix_mask, "prefix_mask", torch.uint8)
    if prefix_kv.dtype not in (torch.bfloat16, torch.uint16, torch.int16):
        raise ValueError("prefix_kv must hold bf16 values")
    _need(prefix_kv, "prefix_kv", prefix_kv.dtype, _kv_shape(cfg, B, P))
    _need(noise, "noise", torch.float32, (B, cfg.chunk, cfg.action_dim))
    _need(out_actions, "out_actions", torch.float32, (B, cfg.chunk, cfg.action_dim))
    rc = _lib.smolexp_denoise_noalloc(h, _ptr(prefix_kv), _ptr(prefix_mask), P, _ptr(noise), _ptr(out_actions), B,
                                      _stream(stream))
    _check(rc, h, "smolexp_denoise_noalloc")


def smolexp_velocity(h, cfg, prefix_kv, prefix_mask, x, t, out_v, stream=None):
    import torch
    B, P = prefix_mask.shape
    _need(prefix_mask, "prefix_mask", torch.uint8)
    _need(prefix_kv, "prefix_kv", prefix_kv.dtype, _kv_shape(cfg, B, P))
    _need(x, "x", torch.float32, (B, cfg.chunk, cfg.action_dim))
    _need(out_v, "out_v", torch.float32, (B, cfg.chunk, cfg.action_dim))
    rc = _lib.smolexp_velocity(h, _ptr(prefix_kv), _ptr(prefix_mask), P, _ptr(x), float(t), _ptr(out_v), B,
                               _stream(stream))
    _check(rc, h, "smolexp_velocity")


def smolexp_lm_weight_count(cfg):
    return int(_lib.smolexp_lm_weight_count(ctypes.byref(cfg)))


def smolexp_load_lm_weights(h, bf16_flat):
    """bf16_flat: numpy uint16 array (bf16 bit patterns) in the language model's manifest order."""
    import numpy as np
    a = np.ascontiguousarray(bf16_flat, dtype=np.uint16)
    _check(_lib.smolexp_load_lm_weights(h, a.ctypes.data_as(ctypes.c_void_p), a.size), h,
           "smolexp_load_lm_weights")


def smolexp_prefill(h, cfg, prefix_emb, prefix_mask, out_kv, stream=None):
    """prefix_emb: bf16 (or its uint16/int16 bits) [B,P,960]; prefix_mask uint8 [B,P];
    out_kv: bf16 bits [L,2,B,5,P,64], written."""
    import torch
    B, P = prefix_mask.shape
    _need(prefix_mask, "prefix_mask", torch.uint8)
    for name, t in (("prefix_emb", prefix_emb), ("out_kv", out_kv)):
        if t.dtype not in (torch.bfloat16, torch.uint16, torch.int16):
            raise ValueError(f"{name} must hold bf16 values")
    _need(prefix_emb, "prefix_emb", prefix_emb.dtype, (B, P, 960))
    _need(out_kv, "out_kv", out_kv.dtype, _kv_shape(cfg, B, P))
    rc = _lib.smolexp_prefill(h, _ptr(prefix_emb), _ptr(prefix_mask), P, _ptr(out_kv), B, _stream(stream))
    _check(rc, h, "smolexp_prefill")


def smolexp_train_step(h, cfg, prefix_kv, prefix_mask, actions, noise, t, out_grads, out_loss, stream=None):
    """prefix_kv bf16 bits [L,2,B,5,P,64]; prefix_mask uint8 [B,P]; actions, noise fp32 [B,50,32];
    t fp32 [B]; out_grads fp32 [weight_count] and out_loss fp32 [1], written."""
    import torch
    B, P = prefix_mask.shape
    _need(prefix_mask, "prefix_mask", torch.uint8)
    if prefix_kv.dtype not in (torch.bfloat16, torch.uint16, torch.int16):
        raise ValueError("prefix_kv must hold bf16 values")
    _need(prefix_kv, "prefix_kv", prefix_kv.dtype, _kv_shape(cfg, B, P))
    for name, x in (("actions", actions), ("noise", noise)):
        _need(x, name, torch.float32, (B, 50, 32))
    _need(t, "t", torch.float32, (B,))
    _need(out_grads, "out_grads", torch.float32, (smolexp_weight_count(cfg),))
    _need(out_loss, "out_loss", torch.float32, (1,))
    rc = _lib.smolexp_train_step(h, _ptr(prefix_kv), _ptr(prefix_mask), P, _ptr(actions), _ptr(noise), _ptr(t),
                                 _ptr(out_grads), _ptr(out_loss), B, _stream(stream))
    _check(rc, h, "smolexp_train_step")


def smolexp_time_kernel(h, kernel, reps, stream=None):
    us = ctypes.c_float()
    _check(_lib.smolexp_time_kernel(h, int(kernel), int(reps), _stream(stream), ctypes.byref(us)), h,
           "smolexp_time_kernel")
    return us.value


def smolexp_strerror(code):
    return _lib.smolexp_strerror(int(code)).decode()


def smolexp_last_error(h):
    return _lib.smolexp_last_error(h).decode()


def smolexp_destroy(h):
    _lib.smolexp_destroy(h)


def raw():
    """The loaded ctypes library (for tests that call the C ABI directly)."""
    return _lib
