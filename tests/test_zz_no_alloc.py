"""mla_decode_uniform_noalloc, the decode for callers that cannot allocate
(split partials in the library's static scratch), against
mla_decode_uniform (partials in a caller workspace), through the C ABI:
several calls in a row, each smaller than the one before, each bitwise
equal to the workspace form and within the bf16 / fp8 bar of the oracle;
and an oversized call rejected before anything is launched."""

import ctypes

import numpy as np
import pytest
import torch

from tests import oracle_views as ov

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import mla_latent_kv_18_amd as mla
    from mla_latent_kv_18_amd.inputs import WORKLOADS, generate
    from mla_latent_kv_18_amd.step import DeviceStep
    from tests.test_gpu_parity import check_decode_call

CALLS = [   # largest first: later calls leave earlier contents in the scratch
    ("v3_bs64_ctx4k", dict(batch=8, lens=(4096, 4096, 3000, 4096, 17, 4096, 2500, 4096)), 0),
    ("v3_fp8_bs4_ctx128k_q2", dict(batch=2, lens=(1500, 700)), 128),
    ("v3_bs64_ctx4k", dict(batch=3, lens=(900, 1, 300), shuffle=True), 64),
    ("v3_bs64_ctx4k", dict(n_h=64, batch=2, lens=(520, 65)), 64),
]


def _call_noalloc(step, st):
    w = step.w
    mla.decode_uniform_noalloc(step.dims, step.q_lat, step.cache, step.block_table, step.seq_lens,
                               step.max_seq_len, step.o_lat, step.lse, q_scale=step.q_scale,
                               cache_scale=step.cache_scale, q_len=w.q_len, split_tokens=st)


def test_noalloc_equals_workspace_form_on_calls_in_a_row():
    steps = []
    for base, over, st in CALLS:
        w = WORKLOADS[base].scaled(name="noalloc", seed=31, **over)
        gen = generate(w)
        step = DeviceStep(gen, split_tokens=st, mode="uniform")
        step.append()
        step.absorb()
        steps.append((gen, step, st))
    torch.cuda.synchronize()
    sizes = [mla.decode_uniform_workspace_size(s.dims, s.w.batch, s.w.q_len, s.max_seq_len, st)
             for _, s, st in steps]
    assert sizes[0] > 0 and all(a >= b for a, b in zip(sizes, sizes[1:])), sizes
    assert sizes[0] <= mla.NOALLOC_SCRATCH_BYTES
    for gen, step, st in steps:
        step.decode(mode="uniform", split_tokens=st)
        torch.cuda.synchronize()
        want_o, want_l = step.o_lat.clone(), step.lse.clone()
        step.o_lat.fill_(float("nan"))
        step.lse.fill_(float("nan"))
        torch.cuda.synchronize()
        _call_noalloc(step, st)
        torch.cuda.synchronize()
        assert torch.equal(step.o_lat, want_o), step.w
        assert torch.equal(step.lse, want_l), step.w
        for b in range(step.w.batch):
            if int(gen["seq_lens"][b]) > 0:
                check_decode_call(step, gen, b, ov.TOL[step.w.dtype])


def test_noalloc_rejects_a_decode_larger_than_its_scratch():
    lib = mla.lib()
    d = mla.make_dims(128, 512, 128, 64, 128, 7168, 64, "bf16", "bf16")
    need = mla.decode_uniform_workspace_size(d, 64, 1, 4096, 64)       # 64 chunks per request
    assert need > mla.NOALLOC_SCRATCH_BYTES
    P = ctypes.c_void_p
    st = lib.mla_decode_uniform_noalloc(ctypes.byref(d), P(1), None, P(1), None, P(1), 64, 4096, P(1), 64, 1, 4096,
                                        64, P(1), None, None)
    assert st == 3
    assert b"static scratch" in lib.mla_last_error_message()
