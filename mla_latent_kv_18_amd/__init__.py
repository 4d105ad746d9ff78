"""libmla Python binding: argument marshalling for the C ABI in include/mla.h.

Every computation runs in the HIP kernels of libmla.so; this module only
turns torch tensors into device pointers, picks the current HIP stream and
allocates caller-owned workspaces with torch.  There is no fallback: if the
library is missing or a call fails, an exception is raised.
"""

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmla.so")

F32, BF16, FP8_E4M3 = 0, 1, 2
_DTYPE_CODE = {"f32": F32, "bf16": BF16, "fp8": FP8_E4M3}

STATUS = {0: "MLA_OK", 1: "MLA_ERR_INVALID_ARGUMENT", 2: "MLA_ERR_UNSUPPORTED",
          3: "MLA_ERR_WORKSPACE_TOO_SMALL", 4: "MLA_ERR_HIP"}

# every entry point declared in include/mla.h
EXPORTS = ("mla_cache_row_bytes", "mla_q_lat_row_bytes", "mla_append_workspace_size", "mla_append_latent",
           "mla_absorb_workspace_size", "mla_absorb_q", "mla_decode_workspace_size",
           "mla_decode", "mla_decode_default_split", "mla_out_proj", "mla_linear_workspace_size",
           "mla_linear", "mla_prefill_attention", "mla_status_string", "mla_last_error_message",
           "mla_version")


class MlaError(RuntimeError):
    def __init__(self, status, message):
        super().__init__(f"{STATUS.get(status, status)}: {message}")
        self.status = status


class Dims(ctypes.Structure):
    _fields_ = [("num_heads", ctypes.c_int32), ("kv_lora_rank", ctypes.c_int32),
                ("qk_nope_head_dim", ctypes.c_int32), ("qk_rope_head_dim", ctypes.c_int32),
                ("v_head_dim", ctypes.c_int32), ("hidden_size", ctypes.c_int32),
                ("block_size", ctypes.c_int32), ("cache_dtype", ctypes.c_int32),
                ("act_dtype", ctypes.c_int32), ("softmax_scale", ctypes.c_float),
                ("rope_theta", ctypes.c_float), ("rms_eps", ctypes.c_float)]


def make_dims(n_h, d_c, d_h, d_r, d_v, d_model, block_size, cache_dtype, act_dtype,
              softmax_scale=0.0, rope_theta=10000.0, rms_eps=1e-6):
    return Dims(n_h, d_c, d_h, d_r, d_v, d_model, block_size, _DTYPE_CODE[cache_dtype],
                _DTYPE_CODE[act_dtype], softmax_scale, rope_theta, rms_eps)


_lib = None


def lib():
    """Load libmla.so (built by mla_latent_kv_18_amd.build); raises if absent."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"libmla.so not found at {LIB_PATH}; run python -m mla_latent_kv_18_amd.build")
    L = ctypes.CDLL(LIB_PATH)
    P, I32, I64, SZ, DP = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t, ctypes.POINTER(Dims)
    sig = {
        "mla_cache_row_bytes": (SZ, [DP]),
        "mla_q_lat_row_bytes": (SZ, [DP]),
        "mla_append_workspace_size": (SZ, [DP, I32]),
        "mla_append_latent": (I32, [DP, P, P, P, P, P, I32, I64, P, P, P, SZ, P]),
        "mla_absorb_workspace_size": (SZ, [DP, I32]),
        "mla_absorb_q": (I32, [DP, P, P, P, P, I32, P, P, P, SZ, P]),
        "mla_decode_workspace_size": (SZ, [DP, I32, I32, I32, I32]),
        "mla_decode": (I32, [DP, P, P, P, P, P, I32, I32, P, I32, I32, I32, I32, P, SZ, P, P, P]),
        "mla_decode_default_split": (I32, [DP, I32, I32, I32]),
        "mla_out_proj": (I32, [DP, P, P, I32, P, P]),
        "mla_linear_workspace_size": (SZ, [I32, I32, I32]),
        "mla_prefill_attention": (I32, [DP, P, P, P, P, I32, P, I32, P, P, P]),
        "mla_linear": (I32, [P, I32, P, I32, I32, I32, P, P, SZ, P]),
        "mla_status_string": (ctypes.c_char_p, [I32]),
        "mla_last_error_message": (ctypes.c_char_p, []),
        "mla_version": (I32, []),
    }
    for name, (res, args) in sig.items():
        fn = getattr(L, name)
        fn.restype = res
        fn.argtypes = args
    _lib = L
    return L


def _check(status):
    if status != 0:
        raise MlaError(status, lib().mla_last_error_message().decode())


def _ptr(t):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("libmla needs device tensors")
    if not t.is_contiguous():
        raise ValueError("libmla needs contiguous tensors")
    return t.data_ptr()


def _stream(device):
    return torch.cuda.current_stream(device).cuda_stream


def _workspace(nbytes, device):
    if nbytes == 0:
        return None, 0
    return torch.empty(nbytes, dtype=torch.uint8, device=device), nbytes


# ------------------------------------------------------------------- calls
def append_latent(dims, hidden, w_dkv_kr, gamma, positions, slot_mapping, cache, cache_scale=None,
                  workspace=None):
    """mla_append_latent.  hidden [N, d_model] (or [N, d_c+d_R] fp32 when
    w_dkv_kr is None); cache [blocks, block_size, d_c+d_R]."""
    n = positions.numel()
    need = lib().mla_append_workspace_size(ctypes.byref(dims), n)
    if workspace is None:
        workspace, _ = _workspace(need, cache.device)
    nbytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    slots = cache.shape[0] * cache.shape[1]
    _check(lib().mla_append_latent(ctypes.byref(dims), _ptr(hidden), _ptr(w_dkv_kr), _ptr(gamma),
                                   _ptr(positions), _ptr(slot_mapping), n, slots, _ptr(cache),
                                   _ptr(cache_scale), _ptr(workspace), nbytes, _stream(cache.device)))


def absorb_q(dims, q_nope, q_pe, w_uk, positions, q_lat, q_scale=None, workspace=None):
    """mla_absorb_q: q_lat [N, n_h, row] with row = mla_q_lat_row_bytes (and q_scale
    [N, n_h] for fp8: two e4m3 planes per row)."""
    n = q_nope.shape[0]
    need = lib().mla_absorb_workspace_size(ctypes.byref(dims), n)
    if workspace is None:
        workspace, _ = _workspace(need, q_lat.device)
    nbytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(lib().mla_absorb_q(ctypes.byref(dims), _ptr(q_nope), _ptr(q_pe), _ptr(w_uk),
                              _ptr(positions), n, _ptr(q_lat), _ptr(q_scale), _ptr(workspace),
                              nbytes, _stream(q_lat.device)))


def decode_workspace_size(dims, batch, q_len, max_seq_len, split_tokens=0):
    return lib().mla_decode_workspace_size(ctypes.byref(dims), batch, q_len, max_seq_len, split_tokens)


def default_split(dims, batch, q_len, max_seq_len):
    return lib().mla_decode_default_split(ctypes.byref(dims), batch, q_len, max_seq_len)


def decode(dims, q_lat, cache, block_table, seq_lens, max_seq_len, o_lat, lse=None, q_scale=None,
           cache_scale=None, q_len=1, split_tokens=0, workspace=None):
    """mla_decode over the paged latent cache; writes o_lat [B*q_len, n_h, d_c]."""
    batch = block_table.shape[0]
    need = decode_workspace_size(dims, batch, q_len, max_seq_len, split_tokens)
    if workspace is None:
        workspace, _ = _workspace(need, q_lat.device)
    nbytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(lib().mla_decode(ctypes.byref(dims), _ptr(q_lat), _ptr(q_scale), _ptr(cache),
                            _ptr(cache_scale), _ptr(block_table), block_table.shape[1],
                            cache.shape[0], _ptr(seq_lens), batch, q_len, max_seq_len, split_tokens,
                            _ptr(workspace), nbytes, _ptr(o_lat), _ptr(lse), _stream(q_lat.device)))


def out_proj(dims, o_lat, w_uv, out):
    """mla_out_proj: out [N, n_h, d_v] = W^UV_i o_lat."""
    _check(lib().mla_out_proj(ctypes.byref(dims), _ptr(o_lat), _ptr(w_uv), o_lat.shape[0],
                              _ptr(out), _stream(o_lat.device)))


def linear_workspace_size(m, n, k):
    return lib().mla_linear_workspace_size(m, n, k)


def linear(x, w, y, workspace=None, ldx=None):
    """mla_linear: y [m, n] = x [m, k] w [n, k]^T (bf16).  x and y may be any
    contiguous tensors whose leading dimension is m; with ldx, x is a 2-D
    view whose rows are ldx elements apart (e.g. the latent part of cache
    rows, x = rows[:, :d_c], ldx = d_c + d_R)."""
    m = x.shape[0]
    n, k = w.shape[0], w.numel() // w.shape[0]
    if ldx is None:
        if not x.is_contiguous() or x.numel() != m * k:
            raise ValueError(f"linear: x {tuple(x.shape)} does not match w {tuple(w.shape)}")
        ldx, xp = k, _ptr(x)
    else:
        if x.dim() != 2 or x.shape[1] != k or x.stride() != (ldx, 1) or not x.is_cuda:
            raise ValueError(f"linear: x must be a [{m}, {k}] view with row stride {ldx}")
        xp = x.data_ptr()
    if y.numel() != m * n or y.shape[0] != m:
        raise ValueError(f"linear: y {tuple(y.shape)} does not match [{m}, {n}]")
    if not (x.dtype == w.dtype == y.dtype == torch.bfloat16):
        raise ValueError("linear: x, w and y must be bfloat16")
    need = linear_workspace_size(m, n, k)
    if workspace is None:
        workspace, _ = _workspace(need, y.device)
    nbytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(lib().mla_linear(xp, ldx, _ptr(w), m, n, k, _ptr(y), _ptr(workspace), nbytes, _stream(y.device)))


def prefill_attention(dims, q_nope, q_pe, k_nope, k_rope, v, out, lse=None):
    """mla_prefill_attention over one prompt of q_nope.shape[0] tokens.
    k_rope is a [T, d_R] view whose rows may be strided (e.g. the RoPE part
    of contiguous cache rows)."""
    T = q_nope.shape[0]
    n_h, d_h, d_r, d_v = dims.num_heads, dims.qk_nope_head_dim, dims.qk_rope_head_dim, dims.v_head_dim
    if (k_rope.dim() != 2 or k_rope.stride(1) != 1 or k_rope.shape[0] != T or k_rope.shape[1] != d_r
            or not k_rope.is_cuda):
        raise ValueError("prefill_attention: k_rope must be a [T, d_R] device view with unit column stride")
    for name, t, width in (("q_nope", q_nope, d_h), ("q_pe", q_pe, d_r), ("k_nope", k_nope, d_h), ("v", v, d_v),
                           ("out", out, d_v)):
        if t.shape[0] != T or t.numel() != T * n_h * width or t.dtype != torch.bfloat16:
            raise ValueError(f"prefill_attention: {name} must be bf16 [{T}, {n_h}, {width}], got "
                             f"{t.dtype} {tuple(t.shape)}")
    if lse is not None and (lse.numel() != T * n_h or lse.dtype != torch.float32):
        raise ValueError("prefill_attention: lse must be float32 [T, n_h]")
    _check(lib().mla_prefill_attention(ctypes.byref(dims), _ptr(q_nope), _ptr(q_pe), _ptr(k_nope),
                                       k_rope.data_ptr(), k_rope.stride(0), _ptr(v), T, _ptr(out), _ptr(lse),
                                       _stream(out.device)))


def version():
    return lib().mla_version()
