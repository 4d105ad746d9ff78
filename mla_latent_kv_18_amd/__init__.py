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

F32, BF16, FP8_E4M3, FP4_E2M1, FP8_E4M3_KR_BF16 = 0, 1, 2, 3, 4
_DTYPE_CODE = {"f32": F32, "bf16": BF16, "fp8": FP8_E4M3, "fp4": FP4_E2M1, "fp8kr": FP8_E4M3_KR_BF16}

STATUS = {0: "MLA_OK", 1: "MLA_ERR_INVALID_ARGUMENT", 2: "MLA_ERR_UNSUPPORTED",
          3: "MLA_ERR_WORKSPACE_TOO_SMALL", 4: "MLA_ERR_PLAN_MISMATCH", 5: "MLA_ERR_HIP"}

# every entry point declared in include/mla.h
EXPORTS = ("mla_cache_row_bytes", "mla_cache_bytes_per_token", "mla_q_lat_row_bytes",
           "mla_append_workspace_size", "mla_append_latent", "mla_absorb_workspace_size", "mla_absorb_q",
           "mla_append_absorb_workspace_size", "mla_append_absorb",
           "mla_decode_plan_workspace_size", "mla_decode_plan", "mla_decode_plan_host", "mla_decode",
           "mla_decode_uniform_workspace_size", "mla_decode_uniform", "mla_decode_uniform_noalloc",
           "mla_decode_default_split",
           "mla_out_proj", "mla_linear_workspace_size", "mla_linear", "mla_linear_pair", "mla_prefill_attention", "mla_prefill_attention_varlen",
           "mla_absorb_output_weights", "mla_absorb_query_weights", "mla_hbm_read_probe",
           "mla_status_string", "mla_last_error_message", "mla_version")


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


class Plan(ctypes.Structure):
    """mla_plan_t: filled by decode_plan, read by decode."""
    _fields_ = [("batch", ctypes.c_int32), ("q_len", ctypes.c_int32), ("num_items", ctypes.c_int32),
                ("max_splits", ctypes.c_int32), ("hash", ctypes.c_uint64), ("workspace_bytes", ctypes.c_size_t),
                ("image_bytes", ctypes.c_size_t),
                ("split_tokens", ctypes.c_int32), ("max_seq_len", ctypes.c_int32),
                ("num_slots", ctypes.c_int32), ("num_partials", ctypes.c_int32),
                ("seq_digest", ctypes.c_uint64), ("workspace", ctypes.c_uint64)]


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
    PP = ctypes.POINTER(Plan)
    sig = {
        "mla_cache_row_bytes": (SZ, [DP]),
        "mla_cache_bytes_per_token": (SZ, [DP]),
        "mla_q_lat_row_bytes": (SZ, [DP]),
        "mla_append_workspace_size": (SZ, [DP, I32]),
        "mla_append_latent": (I32, [DP, P, P, P, P, P, I32, I64, P, P, P, SZ, P]),
        "mla_absorb_workspace_size": (SZ, [DP, I32]),
        "mla_append_absorb_workspace_size": (SZ, [DP, I32, I32]),
        "mla_append_absorb": (I32, [DP, P, P, P, P, P, I32, I64, P, P, P, P, P, P, I32, P, P, P, SZ, P]),
        "mla_absorb_q": (I32, [DP, P, P, P, P, I32, P, P, P, SZ, P]),
        "mla_decode_plan_workspace_size": (SZ, [DP, P, I32, I32, I32]),
        "mla_decode_plan": (I32, [DP, P, I32, I32, I32, PP, P, SZ, P]),
        "mla_decode_plan_host": (I32, [DP, P, I32, I32, I32, P, PP, P, SZ]),
        "mla_decode": (I32, [DP, PP, P, P, P, P, P, I32, I32, P, P, SZ, P, P, P]),
        "mla_decode_uniform_workspace_size": (SZ, [DP, I32, I32, I32, I32]),
        "mla_decode_uniform": (I32, [DP, P, P, P, P, P, I32, I32, P, I32, I32, I32, I32, P, SZ, P, P, P]),
        "mla_decode_uniform_noalloc": (I32, [DP, P, P, P, P, P, I32, I32, P, I32, I32, I32, I32, P, P, P]),
        "mla_absorb_output_weights": (I32, [DP, P, P, P, P]),
        "mla_absorb_query_weights": (I32, [DP, I32, P, P, P, P]),
        "mla_decode_default_split": (I32, [DP, I32, I32, I32]),
        "mla_out_proj": (I32, [DP, P, P, I32, P, P]),
        "mla_linear_workspace_size": (SZ, [I32, I32, I32]),
        "mla_linear_pair": (I32, [P, I32, I32, I32, P, I32, P, P, I32, P, P, SZ, P]),
        "mla_prefill_attention": (I32, [DP, P, P, P, P, I32, P, I32, P, P, P]),
        "mla_prefill_attention_varlen": (I32, [DP, P, P, P, P, I32, P, P, P, I32, I32, I32, P, P, P]),
        "mla_linear": (I32, [P, I32, P, I32, I32, I32, P, P, SZ, P]),
        "mla_hbm_read_probe": (I32, [P, SZ, I32, P, SZ, P]),
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


def _host_lens(seq_lens):
    import numpy as np
    if isinstance(seq_lens, torch.Tensor):
        seq_lens = seq_lens.detach().cpu().numpy()
    return np.ascontiguousarray(np.asarray(seq_lens, dtype=np.int32))


def append_absorb(dims, hidden, w_dkv_kr, gamma, positions, slot_mapping, cache, cache_scale, q_nope, q_pe, w_uk,
                  q_positions, q_lat, q_scale=None, workspace=None):
    """mla_append_absorb: append_latent and absorb_q in one call."""
    n, nq = positions.numel(), q_nope.shape[0]
    need = lib().mla_append_absorb_workspace_size(ctypes.byref(dims), n, nq)
    if workspace is None:
        workspace, _ = _workspace(need, cache.device)
    nbytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    slots = cache.shape[0] * cache.shape[1]
    _check(lib().mla_append_absorb(ctypes.byref(dims), _ptr(hidden), _ptr(w_dkv_kr), _ptr(gamma), _ptr(positions),
                                   _ptr(slot_mapping), n, slots, _ptr(cache), _ptr(cache_scale), _ptr(q_nope),
                                   _ptr(q_pe), _ptr(w_uk), _ptr(q_positions), nq, _ptr(q_lat), _ptr(q_scale),
                                   _ptr(workspace), nbytes, _stream(cache.device)))


def decode_plan_workspace_size(dims, seq_lens_host, q_len, split_tokens=0):
    lens = _host_lens(seq_lens_host)
    return lib().mla_decode_plan_workspace_size(ctypes.byref(dims), lens.ctypes.data, len(lens), q_len,
                                                split_tokens)


def decode_plan(dims, seq_lens_host, q_len, device, split_tokens=0, workspace=None):
    """mla_decode_plan: plans a decode over requests of the given host
    lengths.  Returns (plan, workspace); pass both to decode()."""
    lens = _host_lens(seq_lens_host)
    need = lib().mla_decode_plan_workspace_size(ctypes.byref(dims), lens.ctypes.data, len(lens), q_len,
                                                split_tokens)
    if need == 0:
        raise MlaError(1, lib().mla_last_error_message().decode())
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=device)
    plan = Plan()
    nbytes = workspace.numel() * workspace.element_size()
    _check(lib().mla_decode_plan(ctypes.byref(dims), lens.ctypes.data, len(lens), q_len, split_tokens,
                                 ctypes.byref(plan), _ptr(workspace), nbytes, _stream(workspace.device)))
    return plan, workspace


def decode(dims, plan, workspace, q_lat, cache, block_table, seq_lens, o_lat, lse=None, q_scale=None,
           cache_scale=None):
    """mla_decode: runs a plan made by decode_plan over the paged latent
    cache; writes o_lat [B*q_len, n_h, d_c] (and lse)."""
    nbytes = workspace.numel() * workspace.element_size()
    _check(lib().mla_decode(ctypes.byref(dims), ctypes.byref(plan), _ptr(q_lat), _ptr(q_scale), _ptr(cache),
                            _ptr(cache_scale), _ptr(block_table), block_table.shape[1], cache.shape[0],
                            _ptr(seq_lens), _ptr(workspace), nbytes, _ptr(o_lat), _ptr(lse),
                            _stream(q_lat.device)))


def decode_uniform_workspace_size(dims, batch, q_len, max_seq_len, split_tokens=0):
    return lib().mla_decode_uniform_workspace_size(ctypes.byref(dims), batch, q_len, max_seq_len, split_tokens)


def default_split(dims, batch, q_len, max_seq_len):
    return lib().mla_decode_default_split(ctypes.byref(dims), batch, q_len, max_seq_len)


def decode_uniform(dims, q_lat, cache, block_table, seq_lens, max_seq_len, o_lat, lse=None, q_scale=None,
                   cache_scale=None, q_len=1, split_tokens=0, workspace=None):
    """mla_decode_uniform: one chunk length for every request, sized from
    max_seq_len; writes o_lat [B*q_len, n_h, d_c]."""
    batch = block_table.shape[0]
    need = decode_uniform_workspace_size(dims, batch, q_len, max_seq_len, split_tokens)
    if workspace is None:
        workspace, _ = _workspace(need, q_lat.device)
    nbytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(lib().mla_decode_uniform(ctypes.byref(dims), _ptr(q_lat), _ptr(q_scale), _ptr(cache),
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


def linear_pair(x, w1, y1, w2, y2, workspace=None):
    """mla_linear_pair: y1 [m, n1] = x w1^T and y2 [m, n2] = x w2^T in one
    launch (x contiguous [m, k]; y1, y2 any contiguous tensors with m rows)."""
    m, k = x.shape[0], x.numel() // x.shape[0]
    n1, n2 = w1.shape[0], w2.shape[0]
    if not x.is_contiguous() or w1.numel() != n1 * k or w2.numel() != n2 * k:
        raise ValueError(f"linear_pair: x {tuple(x.shape)} does not match w1 {tuple(w1.shape)}, w2 {tuple(w2.shape)}")
    if y1.numel() != m * n1 or y2.numel() != m * n2:
        raise ValueError("linear_pair: outputs do not match [m, n1] and [m, n2]")
    if not all(t.dtype == torch.bfloat16 for t in (x, w1, y1, w2, y2)):
        raise ValueError("linear_pair: all tensors must be bfloat16")
    need = linear_workspace_size(m, n1 + n2, k)
    if workspace is None:
        workspace, _ = _workspace(need, y1.device)
    nbytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(lib().mla_linear_pair(_ptr(x), k, m, k, _ptr(w1), n1, _ptr(y1), _ptr(w2), n2, _ptr(y2), _ptr(workspace),
                                 nbytes, _stream(y1.device)))


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


NOALLOC_SCRATCH_BYTES = 48 << 20


def decode_uniform_noalloc(dims, q_lat, cache, block_table, seq_lens, max_seq_len, o_lat, lse=None,
                           q_scale=None, cache_scale=None, q_len=1, split_tokens=0):
    """mla_decode_uniform_noalloc: decode_uniform with the split partials in
    the library's static scratch (no workspace, no allocation)."""
    batch = block_table.shape[0]
    _check(lib().mla_decode_uniform_noalloc(ctypes.byref(dims), _ptr(q_lat), _ptr(q_scale), _ptr(cache),
                                            _ptr(cache_scale), _ptr(block_table), block_table.shape[1],
                                            cache.shape[0], _ptr(seq_lens), batch, q_len, max_seq_len,
                                            split_tokens, _ptr(o_lat), _ptr(lse), _stream(q_lat.device)))


def absorb_output_weights(dims, w_o, w_uv, b):
    """mla_absorb_output_weights: b [d_model, n_h*d_c] with B_i = W^O_i W^UV_i."""
    _check(lib().mla_absorb_output_weights(ctypes.byref(dims), _ptr(w_o), _ptr(w_uv), _ptr(b), _stream(b.device)))


def absorb_query_weights(dims, w_uq, w_uk, a):
    """mla_absorb_query_weights: a [n_h*d_c, d_cq] with A_i = W^UK_i^T W^UQ_i."""
    d_cq = w_uq.shape[-1]
    _check(lib().mla_absorb_query_weights(ctypes.byref(dims), d_cq, _ptr(w_uq), _ptr(w_uk), _ptr(a),
                                          _stream(a.device)))


def cache_bytes_per_token(dims):
    return lib().mla_cache_bytes_per_token(ctypes.byref(dims))


def prefill_attention_varlen(dims, q_nope, q_pe, k_nope, k_rope, v, cu_q, cu_k, max_q, out, lse=None):
    """mla_prefill_attention_varlen: sequences whose new tokens (queries,
    rows cu_q[s]..cu_q[s+1]-1) follow their cached context (keys, rows
    cu_k[s]..cu_k[s+1]-1).  cu_q, cu_k: int32 device tensors [num_seqs + 1];
    max_q: the most queries of one sequence (host int)."""
    n_h, d_h, d_r, d_v = dims.num_heads, dims.qk_nope_head_dim, dims.qk_rope_head_dim, dims.v_head_dim
    S = cu_q.numel() - 1
    Tq, Tk = q_nope.shape[0], k_nope.shape[0]
    if cu_k.numel() != S + 1 or cu_q.dtype != torch.int32 or cu_k.dtype != torch.int32:
        raise ValueError("prefill_attention_varlen: cu_q and cu_k must be int32 [num_seqs + 1]")
    if k_rope.dim() != 2 or k_rope.stride(1) != 1 or k_rope.shape[0] != Tk or k_rope.shape[1] != d_r:
        raise ValueError("prefill_attention_varlen: k_rope must be a [total keys, d_R] view with unit column stride")
    for name, t, rows, width in (("q_nope", q_nope, Tq, d_h), ("q_pe", q_pe, Tq, d_r), ("k_nope", k_nope, Tk, d_h),
                                 ("v", v, Tk, d_v), ("out", out, Tq, d_v)):
        if t.shape[0] != rows or t.numel() != rows * n_h * width or t.dtype != torch.bfloat16:
            raise ValueError(f"prefill_attention_varlen: {name} must be bf16 [{rows}, {n_h}, {width}]")
    if lse is not None and (lse.numel() != Tq * n_h or lse.dtype != torch.float32):
        raise ValueError("prefill_attention_varlen: lse must be float32 [total queries, n_h]")
    _check(lib().mla_prefill_attention_varlen(ctypes.byref(dims), _ptr(q_nope), _ptr(q_pe), _ptr(k_nope),
                                              k_rope.data_ptr(), k_rope.stride(0), _ptr(v), _ptr(cu_q), _ptr(cu_k),
                                              S, max_q, Tq, _ptr(out), _ptr(lse), _stream(out.device)))


PROBE_SINK_WORDS = 2048


def hbm_read_probe(buf, mode, sink=None):
    """mla_hbm_read_probe: read the bytes of device tensor `buf` once (mode 0:
    loads into registers, XOR words into sink, an int32 device tensor of at
    least PROBE_SINK_WORDS; mode 1: the decode kernels' direct global->LDS
    tile copies, no sink)."""
    nbytes = buf.numel() * buf.element_size()
    if mode == 0 and (sink is None or sink.numel() < PROBE_SINK_WORDS or sink.element_size() != 4):
        raise ValueError(f"hbm_read_probe: mode 0 needs a 4-byte sink of at least {PROBE_SINK_WORDS} words")
    _check(lib().mla_hbm_read_probe(_ptr(buf), nbytes, mode, _ptr(sink), 0 if sink is None else sink.numel(),
                                    _stream(buf.device)))


def version():
    return lib().mla_version()
