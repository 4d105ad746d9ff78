"""The C-ABI library on the host: it loads, exports every entry point that
include/mla.h declares, and rejects bad arguments before any launch (these
calls never reach the GPU).  CPU only."""

import ctypes
import os
import re

import pytest

import mla_latent_kv_18_amd as mla

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "mla.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(mla_[a-z0-9_]+)\s*\(", text)))


def test_library_exports_every_declared_entry_point():
    lib = mla.lib()
    names = declared_functions()
    assert len(names) >= 10
    for n in names:
        assert hasattr(lib, n), n
    assert sorted(mla.EXPORTS) == names


def v3_dims(**kw):
    a = dict(n_h=128, d_c=512, d_h=128, d_r=64, d_v=128, d_model=7168, block_size=64,
             cache_dtype="bf16", act_dtype="bf16")
    a.update(kw)
    return mla.make_dims(**a)


def test_sizes_and_status_strings():
    lib = mla.lib()
    d = v3_dims()
    assert lib.mla_cache_row_bytes(ctypes.byref(d)) == 576 * 2
    assert lib.mla_cache_row_bytes(ctypes.byref(v3_dims(cache_dtype="fp8"))) == 576
    assert lib.mla_q_lat_row_bytes(ctypes.byref(d)) == 576 * 2
    assert lib.mla_q_lat_row_bytes(ctypes.byref(v3_dims(cache_dtype="fp8"))) == 2 * 576   # hi + lo planes
    f32 = mla.make_dims(4, 32, 16, 8, 16, 64, 64, "f32", "f32")
    assert lib.mla_cache_row_bytes(ctypes.byref(f32)) == 40 * 4
    assert lib.mla_status_string(0) == b"MLA_OK"
    assert lib.mla_status_string(4) == b"MLA_ERR_PLAN_MISMATCH"
    assert lib.mla_status_string(5) == b"MLA_ERR_HIP"
    assert lib.mla_version() >= 300
    # bytes per cached token and layer: the row, plus the fp32 scale for fp8
    assert mla.cache_bytes_per_token(d) == 1152
    assert mla.cache_bytes_per_token(v3_dims(cache_dtype="fp8")) == 576 + 4
    assert mla.cache_bytes_per_token(f32) == 160
    # x 61 layers: the V3 per-token cache of 35,136 elements (2 B each in bf16)
    assert 61 * mla.cache_bytes_per_token(d) == 35136 * 2
    # default split: one resident wave of workgroups for the 64 x 4096 decode
    assert mla.default_split(d, 64, 1, 4096) == 1024
    assert mla.decode_uniform_workspace_size(d, 64, 1, 4096) == 64 * 4 * 128 * (512 * 2 + 4)   # bf16 partials + lse
    assert mla.decode_uniform_workspace_size(d, 64, 1, 256) == 0          # one chunk: no partials


def call_decode(d, **over):
    lib = mla.lib()
    a = dict(q_lat=1, q_scale=None, cache=1, cache_scale=None, block_table=1, max_blocks=64,
             num_blocks=64, seq_lens=1, batch=64, q_len=1, max_seq_len=4096, split=0, ws=1,
             ws_bytes=1 << 30, o_lat=1, lse=None, stream=None)
    a.update(over)
    return lib.mla_decode_uniform(ctypes.byref(d), a["q_lat"], a["q_scale"], a["cache"], a["cache_scale"],
                                  a["block_table"], a["max_blocks"], a["num_blocks"], a["seq_lens"], a["batch"],
                                  a["q_len"], a["max_seq_len"], a["split"], a["ws"], a["ws_bytes"], a["o_lat"],
                                  a["lse"], a["stream"])


@pytest.mark.parametrize("over,status", [
    (dict(q_lat=None), 1),
    (dict(q_len=3), 2),
    (dict(max_seq_len=4097), 1),
    (dict(split=100), 1),
    (dict(ws_bytes=10), 3),
    (dict(num_blocks=0), 1),
])
def test_decode_rejects_bad_arguments_on_host(over, status):
    assert call_decode(v3_dims(), **over) == status
    assert mla.lib().mla_last_error_message()


def test_unsupported_dims_and_dtypes():
    lib = mla.lib()
    bad = v3_dims(d_c=256)
    assert lib.mla_cache_row_bytes(ctypes.byref(bad)) == (256 + 64) * 2   # defined for any dims
    assert call_decode(bad) == 2
    assert call_decode(v3_dims(n_h=96)) == 2
    assert call_decode(v3_dims(block_size=32)) == 2
    mixed = v3_dims(cache_dtype="bf16", act_dtype="f32")
    assert call_decode(mixed) == 2
    odd = v3_dims(d_r=63)
    assert call_decode(odd) == 1


def test_zero_work_calls_succeed_without_launch():
    lib = mla.lib()
    d = v3_dims()
    assert lib.mla_append_latent(ctypes.byref(d), None, None, None, None, None, 0, 64, None, None,
                                 None, 0, None) == 0
    assert lib.mla_absorb_q(ctypes.byref(d), None, None, None, None, 0, None, None, None, 0, None) == 0
    assert lib.mla_out_proj(ctypes.byref(d), None, None, 0, None, None) == 0
    assert call_decode(d, batch=0) == 0


def test_missing_workspace_and_scales_are_reported():
    lib = mla.lib()
    d = v3_dims()
    assert lib.mla_append_latent(ctypes.byref(d), 1, 1, 1, 1, 1, 64, 4096, 1, None, None, 0, None) == 3
    d8 = v3_dims(cache_dtype="fp8")
    assert lib.mla_append_latent(ctypes.byref(d8), 1, 1, 1, 1, 1, 64, 4096, 1, None, 1, 1 << 30, None) == 1
    assert lib.mla_absorb_q(ctypes.byref(d8), 1, 1, 1, 1, 64, 1, None, 1, 1 << 30, None) == 1
    assert call_decode(d8) == 1


def test_linear_sizes_and_host_checks():
    lib = mla.lib()
    # slices of k: W^O (7168 x 16384) at 64 tokens, 56 row groups x 8 slices
    assert mla.linear_workspace_size(64, 7168, 16384) == 8 * 64 * 7168 * 4
    # W^UQ (16384 x 1536): 128 row groups x 4 slices
    assert mla.linear_workspace_size(64, 16384, 1536) == 4 * 64 * 16384 * 4
    # W^DQ (1536 x 7168): 12 row groups x 16 slices, partials at most half the weight bytes
    assert mla.linear_workspace_size(64, 1536, 7168) == 16 * 64 * 1536 * 4
    assert mla.linear_workspace_size(64, 1536, 7168) <= 1536 * 7168
    # W^QR (8192 x 1536): 64 row groups x 4 slices
    assert mla.linear_workspace_size(64, 8192, 1536) == 4 * 64 * 8192 * 4
    # many tokens, few columns: the cap leaves one slice
    assert mla.linear_workspace_size(4096, 128, 4096) == 0
    # many tokens over k = 512 (prefill up-projections): the weight-stationary form, no workspace
    assert mla.linear_workspace_size(4096, 16384, 512) == 0
    # a large row count needs no slices
    assert mla.linear_workspace_size(64, 65536, 128) == 0
    assert mla.linear_workspace_size(64, 100, 128) == 0              # unsupported: 0
    P = ctypes.c_void_p
    assert lib.mla_linear(P(1), 128, P(1), 4, 100, 128, P(1), None, 0, None) == 2          # n % 128
    assert lib.mla_linear(P(1), 128, P(1), 4, 128, 100, P(1), None, 0, None) == 2          # k % 16
    assert lib.mla_linear(P(1), 128, P(1), -1, 128, 128, P(1), None, 0, None) == 1
    assert lib.mla_linear(None, 128, P(1), 4, 128, 128, P(1), None, 0, None) == 1
    assert lib.mla_linear(P(1), 128, P(1), 0, 128, 128, P(1), None, 0, None) == 0     # nothing to do
    assert lib.mla_linear(P(1), 100, P(1), 4, 128, 128, P(1), None, 0, None) == 1   # ldx < k
    assert lib.mla_linear(P(1), 16384, P(1), 64, 7168, 16384, P(1), P(1), 16, None) == 3     # workspace too small


def test_prefill_host_checks():
    lib = mla.lib()
    P = ctypes.c_void_p
    d = v3_dims()

    def call(dims=d, T=128, stride=576, q=P(1)):
        return lib.mla_prefill_attention(ctypes.byref(dims), q, P(1), P(1), P(1), stride, P(1), T, P(1), None,
                                         None)
    assert call(T=0) == 0                                   # nothing to do
    assert call(T=-1) == 1
    assert call(q=None) == 1
    assert call(stride=60) == 1                             # shorter than d_R
    assert call(stride=100) == 1                            # rows not 16-byte aligned
    assert call(dims=v3_dims(cache_dtype="fp8")) == 2       # bf16 cache and activations only
    assert call(dims=mla.make_dims(4, 32, 16, 8, 16, 64, 64, "f32", "f32")) == 2


def test_missing_library_fails_loudly(tmp_path, monkeypatch):
    """No fallback: without libmla.so every call raises instead of computing
    something else."""
    monkeypatch.setattr(mla, "LIB_PATH", str(tmp_path / "absent" / "libmla.so"))
    monkeypatch.setattr(mla, "_lib", None)
    with pytest.raises(ImportError):
        mla.lib()
    with pytest.raises(ImportError):
        mla.linear_workspace_size(64, 128, 128)


# ---------------------------------------------------------------------------
# The split-KV planner (host half): coverage, no overlap, placement, balance,
# and the plan checks mla_decode makes before any launch.
# ---------------------------------------------------------------------------
def plan_host(d, lens, q_len=1, hint=0, ws=0x7f0000000000):
    import numpy as np
    lib = mla.lib()
    lens = np.ascontiguousarray(np.asarray(lens, dtype=np.int32))
    plan = mla.Plan()
    st = lib.mla_decode_plan_host(ctypes.byref(d), lens.ctypes.data, len(lens), q_len, hint, ctypes.c_void_p(ws),
                                  ctypes.byref(plan), None, 0)
    assert st == 0, lib.mla_last_error_message()
    img = np.zeros(plan.image_bytes, dtype=np.uint8)
    assert lib.mla_decode_plan_host(ctypes.byref(d), lens.ctypes.data, len(lens), q_len, hint, ctypes.c_void_p(ws),
                                    ctypes.byref(plan), img.ctypes.data, img.nbytes) == 0
    assert bytes(img[:8]) == b"MLAPLAN1"
    assert int(img[8:16].view(np.uint64)[0]) == plan.hash
    words = img.view(np.int32)
    entries = words[64:64 + 4 * plan.num_slots].reshape(-1, 4)
    pp_off = (256 + ((plan.num_slots * 16 + 255) // 256) * 256) // 4
    part_ptr = words[pp_off:pp_off + len(lens) + 1]
    return plan, entries, part_ptr


def check_plan(d, lens, q_len, plan, entries, part_ptr, row_groups):
    import numpy as np
    lens = np.asarray(lens)
    B = len(lens)
    assert plan.batch == B and plan.q_len == q_len
    assert plan.split_tokens % 64 == 0 and plan.split_tokens > 0
    assert plan.num_slots % 8 == 0 and plan.num_slots == len(entries)
    live = entries[entries[:, 0] >= 0]
    b = live[:, 0] & 0xFFFFFF
    rg = live[:, 0] >> 24
    slot_xcd = (np.nonzero(entries[:, 0] >= 0)[0]) % 8
    # every (item, row group) exactly once; the row groups of an item on one XCD
    seen = {}
    for (bb, r, j0, j1, part), x in zip(zip(b, rg, live[:, 1], live[:, 2], live[:, 3]), slot_xcd):
        key = (int(bb), int(j0), int(j1), int(part))
        assert 0 <= r < row_groups
        seen.setdefault(key, {})
        assert r not in seen[key], "row group launched twice"
        seen[key][int(r)] = int(x)
    for key, groups in seen.items():
        assert sorted(groups) == list(range(row_groups))
        assert len(set(groups.values())) == 1, "row groups of one chunk on different XCDs"
    # per request: the chunks tile [0, T) without gaps or overlap (one empty chunk for T = 0)
    assert plan.num_items == len(seen)
    parts = []
    for r_ in range(B):
        chunks = sorted((j0, j1, part) for (bb, j0, j1, part) in seen if bb == r_)
        T = int(lens[r_])
        if T == 0:
            assert chunks == [(0, 0, -1)]
        else:
            assert chunks[0][0] == 0 and chunks[-1][1] == T
            for (a0, a1, _), (c0, c1, _) in zip(chunks, chunks[1:]):
                assert a1 == c0
            assert all(j1 - j0 <= plan.split_tokens and j1 > j0 for j0, j1, _ in chunks)
        # partial blocks: none for a one-chunk request, else exactly part_ptr[b] .. part_ptr[b+1]-1
        ps = sorted(p for _, _, p in chunks)
        if len(chunks) == 1:
            assert ps == [-1] and part_ptr[r_ + 1] == part_ptr[r_]
        else:
            assert ps == list(range(part_ptr[r_], part_ptr[r_ + 1]))
        parts += [p for p in ps if p >= 0]
        assert plan.max_splits >= len(chunks)
    assert sorted(parts) == list(range(plan.num_partials))
    assert part_ptr[0] == 0 and part_ptr[B] == plan.num_partials
    # balance: per-XCD rows (plus a fixed per-chunk cost) within one chunk of the mean
    load = np.zeros(8)
    for (bb, j0, j1, part), groups in seen.items():
        load[next(iter(groups.values()))] += (j1 - j0 + 256) * row_groups
    assert load.max() - load.mean() <= (plan.split_tokens + 256) * row_groups + 1e-9
    return seen


def test_plan_v3_bs64_matches_uniform_and_groups_requests():
    d = v3_dims()
    lens = [4096] * 64
    plan, entries, part_ptr = plan_host(d, lens)
    seen = check_plan(d, lens, 1, plan, entries, part_ptr, 1)
    assert plan.split_tokens == 1024 and plan.num_items == 256 and plan.num_slots == 256
    # each request's four chunks run on one XCD (its queries and partials share that L2)
    by_req = {}
    for (bb, _, _, _), groups in seen.items():
        by_req.setdefault(bb, set()).update(groups.values())
    assert all(len(x) == 1 for x in by_req.values())
    ws = plan.workspace_bytes
    assert ws >= 256 * 128 * (512 * 2 + 4)


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_plan_ragged_kimi_like(seed):
    import numpy as np
    d = v3_dims(n_h=64)
    rng = np.random.default_rng(seed)
    lens = rng.integers(1024, 131072, size=32, endpoint=True)
    plan, entries, part_ptr = plan_host(d, lens)
    check_plan(d, lens, 1, plan, entries, part_ptr, 1)
    # about one resident wave (two 64-head workgroups per CU): no launch of mostly idle workgroups
    assert plan.num_slots <= 2 * 512
    assert (entries[:, 0] >= 0).sum() == plan.num_items


def test_plan_fp8_two_queries_pairs_row_groups():
    d = v3_dims(cache_dtype="fp8")
    lens = [131072] * 4
    plan, entries, part_ptr = plan_host(d, lens, q_len=2)
    check_plan(d, lens, 2, plan, entries, part_ptr, 2)
    assert plan.split_tokens == 4096 and plan.num_slots == 256


@pytest.mark.parametrize("lens", [[0], [0, 50, 0, 1, 100, 0, 64, 65], [1, 2, 63, 64, 65, 500, 1000, 2048],
                                  [5000] + [10] * 40, [131072], list(range(0, 3000, 97))])
@pytest.mark.parametrize("hint", [0, 64, 256])
def test_plan_edge_lengths(lens, hint):
    d = v3_dims()
    plan, entries, part_ptr = plan_host(d, lens, hint=hint)
    check_plan(d, lens, 1, plan, entries, part_ptr, 1)
    if hint:
        assert plan.split_tokens == hint


def test_plan_is_checked_before_any_launch():
    import numpy as np
    lib = mla.lib()
    d = v3_dims()
    ws = 0x7f0000000000
    plan, _, _ = plan_host(d, [300, 5000], ws=ws)
    P = ctypes.c_void_p

    def call(dims=d, p=plan, w=ws, nbytes=None):
        return lib.mla_decode(ctypes.byref(dims), ctypes.byref(p), P(1), None, P(1), None, P(1), 128, 256, P(1),
                              P(w), plan.workspace_bytes if nbytes is None else nbytes, P(1), None, None)
    assert call(dims=v3_dims(n_h=64)) == 4                     # planned for other dims
    assert call(w=ws + 256) == 4                               # another workspace
    assert call(nbytes=plan.workspace_bytes - 1) == 3
    tampered = mla.Plan.from_buffer_copy(plan)
    tampered.num_slots += 8
    assert call(p=tampered) == 4                               # modified plan
    assert call(dims=v3_dims(cache_dtype="fp8")) == 4
    assert lib.mla_last_error_message()
    # bad planning arguments
    lens = np.array([10, -1], dtype=np.int32)
    p2 = mla.Plan()
    assert lib.mla_decode_plan_host(ctypes.byref(d), lens.ctypes.data, 2, 1, 0, None, ctypes.byref(p2), None, 0) == 1
    ok = np.array([10, 20], dtype=np.int32)
    assert lib.mla_decode_plan_host(ctypes.byref(d), ok.ctypes.data, 2, 1, 100, None, ctypes.byref(p2), None, 0) == 1
    assert lib.mla_decode_plan_host(ctypes.byref(d), ok.ctypes.data, 2, 3, 0, None, ctypes.byref(p2), None, 0) == 2
    small = np.zeros(16, dtype=np.uint8)
    assert lib.mla_decode_plan_host(ctypes.byref(d), ok.ctypes.data, 2, 1, 0, None, ctypes.byref(p2),
                                    small.ctypes.data, 16) == 3
    assert lib.mla_decode_plan(ctypes.byref(d), ok.ctypes.data, 2, 1, 0, ctypes.byref(p2), None, 0, None) == 3
    assert mla.decode_plan_workspace_size(d, [4096] * 64, 1) >= 256 * 128 * 1028


def test_fold_weights_host_checks():
    lib = mla.lib()
    P = ctypes.c_void_p
    d = v3_dims()
    assert lib.mla_absorb_output_weights(ctypes.byref(d), None, P(1), P(1), None) == 1
    assert lib.mla_absorb_query_weights(ctypes.byref(d), 0, P(1), P(1), P(1), None) == 1
    assert lib.mla_absorb_query_weights(ctypes.byref(d), 1536, P(1), None, P(1), None) == 1


def test_hbm_read_probe_host_checks():
    """mla_hbm_read_probe rejects a bad mode, a misaligned size and a short
    sink before any launch; zero bytes launch nothing."""
    lib = mla.lib()
    assert lib.mla_hbm_read_probe(None, 16, 0, 1, 4096, None) == 1          # NULL buffer
    assert lib.mla_hbm_read_probe(1, 17, 0, 1, 4096, None) == 1             # not a multiple of 16
    assert lib.mla_hbm_read_probe(1, 16, 0, 1, 2047, None) == 1             # sink too short
    assert lib.mla_hbm_read_probe(1, 16, 0, None, 4096, None) == 1          # no sink
    assert lib.mla_hbm_read_probe(1, 36864 + 16, 1, None, 0, None) == 1     # not whole 36 KB tiles
    assert lib.mla_hbm_read_probe(1, 36864, 2, None, 0, None) == 1          # no such mode
    assert b"mode" in lib.mla_last_error_message()
    assert lib.mla_hbm_read_probe(1, 0, 1, None, 0, None) == 0
