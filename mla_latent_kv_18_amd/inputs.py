"""Seeded synthetic inputs for MLA latent-cache decode.

Shared by the GPU tests, the benchmark and the smoke check; holds only
random draws, storage-format conversion and integer indexing (block tables,
slots, positions) -- none of the method's arithmetic.  Both the HIP path and
the CPU oracle consume the arrays produced here.

Workloads (dims from the attention-variants page's DeepSeek-V3 / Kimi-K2
hyper-parameters; shapes and lengths as the workload list states):

  tiny_f32          fp32, 1 layer: B=1, n_h=4, d_model=64, d_c=32, d_h=16,
                    d_R=8, d_v=16, 64 cached tokens (all built by the append
                    call from hidden states), 1 query token
  v3_bs64_ctx4k     DeepSeek-V3 attention dims, bf16: B=64, 4096 tokens each
  v3_paged_bs16_ctx32k  same dims, B=16, 32768 tokens each, 64-token blocks
                    with a seed-shuffled block table (split context + combine)
  kimi_k2_ragged_bs32   n_h=64, B=32, lengths uniform in [1024, 131072]
  v3_fp8_bs4_ctx128k_q2 fp8 e4m3 cache with one fp32 scale per token, B=4,
                    131072 tokens each, 2 causal queries per request
  Cache variants (same V3 dims and batch as v3_bs64_ctx4k):
  v3_fp4_bs64_ctx4k     MX FP4 rows: 576 E2M1 codes, one E8M0 scale per 32
  v3_fp8kr_bs64_ctx4k   e4m3 latent (one fp32 scale per token) beside a
                        bf16 RoPE key
  nope_bs64_ctx4k       no decoupled RoPE part (d_R = 0): 512-wide bf16 rows

Value recipe: weights N(0,1)/sqrt(fan_in) (fan_in = d_model for the
down-projection, d_c for W^UK and W^UV); RMSNorm gain U[0.5, 1.5]; hidden
states, q_nope, q_pe and pre-filled latent rows N(0,1).  Rows T-q_len..T-1
of each request are left empty in the pool: the append call writes them.

Draw order for numpy.random.default_rng(seed): sequence lengths (ragged
workload only), W_dkv_kr, W_UK, W_UV, gamma, pre-filled rows (request by
request), hidden states, q_nope, q_pe, block permutation (shuffled tables).
"""

from dataclasses import dataclass, replace

import numpy as np
import torch


@dataclass(frozen=True)
class Workload:
    name: str
    n_h: int
    d_c: int
    d_h: int
    d_r: int
    d_v: int
    d_model: int
    batch: int
    seq_len: int            # tokens per request (upper bound when ragged)
    q_len: int
    dtype: str              # cache: "f32" | "bf16" | "fp8" | "fp4" | "fp8kr"; activations f32 or bf16
    block_size: int = 64
    shuffle: bool = False
    ragged_min: int = 0     # >0: lengths uniform in [ragged_min, seq_len]
    seed: int = 0
    all_rows_appended: bool = False
    lens: tuple = ()        # explicit per-request lengths (overrides seq_len / ragged)

    @property
    def act_dtype(self):
        return "f32" if self.dtype == "f32" else "bf16"

    @property
    def row_dim(self):
        return self.d_c + self.d_r

    @property
    def row_bytes(self):
        """Bytes of one stored cache row."""
        D = self.row_dim
        return {"f32": 4 * D, "bf16": 2 * D, "fp8": D, "fp4": (D // 2 + D // 32 + 15) // 16 * 16,
                "fp8kr": self.d_c + 2 * self.d_r}[self.dtype]

    @property
    def softmax_scale(self):
        return 1.0 / float(np.sqrt(self.d_h + self.d_r))

    def scaled(self, **kw):
        return replace(self, **kw)


WORKLOADS = {
    "tiny_f32": Workload("tiny_f32", n_h=4, d_c=32, d_h=16, d_r=8, d_v=16, d_model=64,
                         batch=1, seq_len=64, q_len=1, dtype="f32", seed=1, all_rows_appended=True),
    "v3_bs64_ctx4k": Workload("v3_bs64_ctx4k", n_h=128, d_c=512, d_h=128, d_r=64, d_v=128,
                              d_model=7168, batch=64, seq_len=4096, q_len=1, dtype="bf16", seed=2),
    "v3_paged_bs16_ctx32k": Workload("v3_paged_bs16_ctx32k", n_h=128, d_c=512, d_h=128, d_r=64,
                                     d_v=128, d_model=7168, batch=16, seq_len=32768, q_len=1,
                                     dtype="bf16", shuffle=True, seed=3),
    "kimi_k2_ragged_bs32": Workload("kimi_k2_ragged_bs32", n_h=64, d_c=512, d_h=128, d_r=64,
                                    d_v=128, d_model=7168, batch=32, seq_len=131072, q_len=1,
                                    dtype="bf16", shuffle=True, ragged_min=1024, seed=4),
    "v3_fp8_bs4_ctx128k_q2": Workload("v3_fp8_bs4_ctx128k_q2", n_h=128, d_c=512, d_h=128, d_r=64,
                                      d_v=128, d_model=7168, batch=4, seq_len=131072, q_len=2,
                                      dtype="fp8", seed=5),
    "v3_fp4_bs64_ctx4k": Workload("v3_fp4_bs64_ctx4k", n_h=128, d_c=512, d_h=128, d_r=64, d_v=128,
                                  d_model=7168, batch=64, seq_len=4096, q_len=1, dtype="fp4", seed=6),
    "v3_fp8kr_bs64_ctx4k": Workload("v3_fp8kr_bs64_ctx4k", n_h=128, d_c=512, d_h=128, d_r=64, d_v=128,
                                    d_model=7168, batch=64, seq_len=4096, q_len=1, dtype="fp8kr", seed=7),
    "nope_bs64_ctx4k": Workload("nope_bs64_ctx4k", n_h=128, d_c=512, d_h=128, d_r=0, d_v=128,
                                d_model=7168, batch=64, seq_len=4096, q_len=1, dtype="bf16", seed=8),
}


# ------------------------------------------------------------ storage formats
def to_bf16_bits(x):
    """float32 array -> uint16 bfloat16 bit patterns (round to nearest even)."""
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def to_fp8_rows(x):
    """float32 rows -> (uint8 e4m3 codes, float32 scale per row), one scale
    per row = max|row|/448 (1 for a zero row)."""
    x = np.asarray(x, dtype=np.float32)
    amax = np.max(np.abs(x), axis=-1)
    scale = np.where(amax > 0, amax / np.float32(448.0), np.float32(1.0)).astype(np.float32)
    q = torch.from_numpy(x / scale[..., None]).to(torch.float8_e4m3fn)
    return q.view(torch.uint8).numpy(), scale


def to_fp4_rows(x):
    """float32 rows [n, d] -> stored MX FP4 rows [n, row bytes] uint8: per
    32-element block one E8M0 scale 2^(floor(log2 max|x|) - 2) (127 for an
    all-zero block) and E2M1 codes of x / scale, nearest value, ties to the
    even code, saturating at 6; two codes per byte (element 2i in the low
    nibble); then the d/32 scale bytes; then zero padding to 16 bytes."""
    x = np.asarray(x, dtype=np.float64)
    n, d = x.shape
    blk = x.reshape(n, d // 32, 32)
    amax = np.abs(blk).max(axis=-1)
    _, e = np.frexp(np.where(amax > 0, amax, 1.0))
    shared = np.clip(np.where(amax > 0, e - 3, 0), -127, 127)
    y = blk / np.ldexp(1.0, shared)[..., None]
    grid = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])
    dist = np.abs(np.minimum(np.abs(y), 6.0)[..., None] - grid) + 1e-12 * (np.arange(8) & 1)
    codes = (np.argmin(dist, axis=-1) | np.where(np.signbit(y), 8, 0)).astype(np.uint8).reshape(n, d)
    row_bytes = (d // 2 + d // 32 + 15) // 16 * 16
    out = np.zeros((n, row_bytes), dtype=np.uint8)
    out[:, :d // 2] = codes[:, 0::2] | (codes[:, 1::2] << 4)
    out[:, d // 2:d // 2 + d // 32] = (shared + 127).astype(np.uint8)
    return out


def to_fp8kr_rows(x, d_c):
    """float32 rows [n, d_c + d_R] -> (uint8 rows [n, d_c + 2 d_R], float32
    scale per row): the latent as e4m3 codes of latent / s, s the smallest
    power of two with max|latent| / s <= 448 (1 for an all-zero latent), the
    RoPE key as bf16 (little-endian bytes)."""
    lat = np.asarray(x, dtype=np.float32)[:, :d_c]
    amax = np.abs(lat).max(axis=-1)
    f, e = np.frexp(np.where(amax > 0, amax, 1.0).astype(np.float64))
    scale = np.where(amax > 0, np.ldexp(1.0, np.where(f <= 0.875, e - 9, e - 8)), 1.0).astype(np.float32)
    codes = torch.from_numpy(lat / scale[:, None]).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    kr = to_bf16_bits(np.asarray(x, dtype=np.float32)[:, d_c:])
    return np.concatenate([codes, np.ascontiguousarray(kr).view(np.uint8)], axis=1), scale


def _store(x, fmt):
    if fmt == "f32":
        return np.ascontiguousarray(x, dtype=np.float32)
    if fmt == "bf16":
        return to_bf16_bits(x)
    raise ValueError(fmt)


# ------------------------------------------------------------------ generate
def seq_lens_of(w, rng=None):
    if w.lens:
        assert len(w.lens) == w.batch
        return np.asarray(w.lens, dtype=np.int32)
    if w.ragged_min > 0:
        rng = np.random.default_rng(w.seed) if rng is None else rng
        return rng.integers(w.ragged_min, w.seq_len, size=w.batch, endpoint=True).astype(np.int32)
    return np.full(w.batch, w.seq_len, dtype=np.int32)


def generate(w: Workload):
    """All inputs of one decode step of `w`, as numpy arrays in storage form.

    Returns a dict with:
      seq_lens [B] int32, block_table [B, max_blocks] int32, pool
      [num_blocks, block_size, d_c+d_R] (f32 / uint16 bf16 bits / uint8 e4m3
      codes), pool_scale [num_blocks, block_size] float32 (fp8 only),
      w_dkv_kr [d_c+d_R, d_model], w_uk [n_h, d_h, d_c], w_uv [n_h, d_v, d_c]
      (f32 or bf16 bits), gamma [d_c] float32, h [N_new, d_model],
      new_positions [N_new] int32, slot_mapping [N_new] int64,
      q_nope [N, n_h, d_h], q_pe [N, n_h, d_R], q_positions [N] int32
      (N = B*q_len), with N_new = N (or every row for all_rows_appended)."""
    rng = np.random.default_rng(w.seed)
    B, D, bs = w.batch, w.row_dim, w.block_size
    seq = seq_lens_of(w, rng)
    act = w.act_dtype
    out = {"workload": w, "seq_lens": seq}
    out["w_dkv_kr"] = _store(rng.standard_normal((D, w.d_model)) / np.sqrt(w.d_model), act)
    out["w_uk"] = _store(rng.standard_normal((w.n_h, w.d_h, w.d_c)) / np.sqrt(w.d_c), act)
    out["w_uv"] = _store(rng.standard_normal((w.n_h, w.d_v, w.d_c)) / np.sqrt(w.d_c), act)
    out["gamma"] = rng.uniform(0.5, 1.5, size=w.d_c).astype(np.float32)

    nblk = (seq + bs - 1) // bs
    total_blocks = int(nblk.sum())
    max_blocks = int(nblk.max())
    # logical block i of request b -> physical block (identity before shuffling)
    offsets = np.concatenate([[0], np.cumsum(nblk)[:-1]]).astype(np.int64)
    pool_shape = (total_blocks, bs, D)
    if w.dtype == "f32":
        pool = np.zeros(pool_shape, dtype=np.float32)
    elif w.dtype == "bf16":
        pool = np.zeros(pool_shape, dtype=np.uint16)
    else:
        pool = np.zeros((total_blocks, bs, w.row_bytes), dtype=np.uint8)
    pool_scale = np.ones((total_blocks, bs), dtype=np.float32) if w.dtype in ("fp8", "fp8kr") else None

    # pre-filled rows, request by request, written in logical order; the
    # physical placement is applied after the permutation is drawn
    prefill = []
    for b in range(B):
        n_pre = 0 if w.all_rows_appended else max(0, int(seq[b]) - w.q_len)
        rows = rng.standard_normal((n_pre, D), dtype=np.float32)
        prefill.append(rows)

    n_new = int(seq[0]) if w.all_rows_appended else B * w.q_len
    out["h"] = _store(rng.standard_normal((n_new, w.d_model)), act)
    N = B * w.q_len
    out["q_nope"] = _store(rng.standard_normal((N, w.n_h, w.d_h)), act)
    out["q_pe"] = _store(rng.standard_normal((N, w.n_h, w.d_r)), act)

    phys = np.arange(total_blocks, dtype=np.int64)
    if w.shuffle:
        phys = rng.permutation(total_blocks).astype(np.int64)
    table = np.zeros((B, max_blocks), dtype=np.int32)
    for b in range(B):
        table[b, :nblk[b]] = phys[offsets[b]:offsets[b] + nblk[b]]
    out["block_table"] = table

    for b in range(B):
        rows = prefill[b]
        n_pre = rows.shape[0]
        if n_pre == 0:
            continue
        idx = np.arange(n_pre)
        blk = table[b, idx // bs]
        if w.dtype == "f32":
            pool[blk, idx % bs] = rows
        elif w.dtype == "bf16":
            pool[blk, idx % bs] = to_bf16_bits(rows)
        elif w.dtype == "fp4":
            pool[blk, idx % bs] = to_fp4_rows(rows)
        elif w.dtype == "fp8kr":
            codes, scale = to_fp8kr_rows(rows, w.d_c)
            pool[blk, idx % bs] = codes
            pool_scale[blk, idx % bs] = scale
        else:
            codes, scale = to_fp8_rows(rows)
            pool[blk, idx % bs] = codes
            pool_scale[blk, idx % bs] = scale
        prefill[b] = None
    out["pool"] = pool
    out["pool_scale"] = pool_scale

    if w.all_rows_appended:
        pos = np.arange(n_new, dtype=np.int32)
        req = np.zeros(n_new, dtype=np.int64)
    else:
        pos = np.concatenate([np.arange(w.q_len) + seq[b] - w.q_len for b in range(B)]).astype(np.int32)
        req = np.repeat(np.arange(B), w.q_len)
    valid = pos >= 0                       # a request shorter than q_len has nothing to append there
    posc = np.where(valid, pos, 0)
    out["new_positions"] = posc.astype(np.int32)
    out["slot_mapping"] = np.where(valid, table[req, posc // bs].astype(np.int64) * bs + posc % bs, -1).astype(np.int64)
    out["q_positions"] = np.concatenate(
        [np.arange(w.q_len) + seq[b] - w.q_len for b in range(B)]).astype(np.int32)
    return out


def generate_block_weights(w: Workload, d_cq: int = 1536):
    """Seeded weights of the projections around the attention block, in
    storage form (N(0,1)/sqrt(fan_in), like the others):
      w_dq [d_cq, d_model], w_uq [n_h*d_h, d_cq], w_qr [n_h*d_r, d_cq],
      w_o [d_model, n_h*d_v].
    d_cq = 1536 is the V3 query-latent width.  Drawn from their own stream
    (seed + 1000), so generate() is unchanged."""
    rng = np.random.default_rng(w.seed + 1000)
    act = w.act_dtype
    return {
        "d_cq": d_cq,
        "w_dq": _store(rng.standard_normal((d_cq, w.d_model), dtype=np.float32) / np.sqrt(w.d_model), act),
        "w_uq": _store(rng.standard_normal((w.n_h * w.d_h, d_cq), dtype=np.float32) / np.sqrt(d_cq), act),
        "w_qr": _store(rng.standard_normal((w.n_h * w.d_r, d_cq), dtype=np.float32) / np.sqrt(d_cq), act),
        "w_o": _store(rng.standard_normal((w.d_model, w.n_h * w.d_v), dtype=np.float32) / np.sqrt(w.n_h * w.d_v),
                      act),
    }
