"""One MLA decode step on the GPU: upload a generated workload and run the
four libmla calls (append -> absorb q -> decode -> out proj).  Plumbing
only: torch allocates device memory and streams, libmla does every
computation.  The decode is planned once from the host copy of the
lengths (mla_decode_plan) and run with mla_decode; mode="uniform" runs
mla_decode_uniform instead.  capture() records a whole step (or the decode
call alone) into a HIP graph for callers that replay steps from a graph."""

import ctypes

import numpy as np
import torch

from . import (absorb_output_weights, absorb_q, absorb_query_weights, append_absorb, append_latent, decode, decode_plan,
               decode_uniform, decode_uniform_workspace_size, lib, linear, linear_pair, linear_workspace_size,
               make_dims, out_proj)


def _dev(a, device, fmt):
    a = np.ascontiguousarray(a)
    if fmt == "bf16":
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(device)
    return torch.from_numpy(a).to(device)


class DeviceStep:
    """fused: run() appends and absorbs with one mla_append_absorb call
    (else mla_append_latent then mla_absorb_q)."""

    def __init__(self, gen, device="cuda:0", split_tokens=0, mode="planned", fused=True):
        w = gen["workload"]
        self.w = w
        self.device = device
        act = w.act_dtype
        self.dims = make_dims(w.n_h, w.d_c, w.d_h, w.d_r, w.d_v, w.d_model, w.block_size,
                              w.dtype, act)
        self.w_dkv_kr = _dev(gen["w_dkv_kr"], device, act)
        self.w_uk = _dev(gen["w_uk"], device, act)
        self.w_uv = _dev(gen["w_uv"], device, act)
        self.gamma = _dev(gen["gamma"], device, "f32")
        self.h = _dev(gen["h"], device, act)
        self.q_nope = _dev(gen["q_nope"], device, act)
        self.q_pe = _dev(gen["q_pe"], device, act)
        self.cache = _dev(gen["pool"], device, w.dtype if w.dtype in ("f32", "bf16") else "u8")
        self.cache_scale = _dev(gen["pool_scale"], device, "f32") if gen["pool_scale"] is not None else None
        self.block_table = _dev(gen["block_table"], device, "i32")
        self.seq_lens = _dev(gen["seq_lens"], device, "i32")
        self.max_seq_len = int(gen["seq_lens"].max())
        self.new_pos = _dev(gen["new_positions"], device, "i32")
        self.slots = _dev(gen["slot_mapping"], device, "i64")
        self.q_pos = _dev(gen["q_positions"], device, "i32")
        N = w.batch * w.q_len
        D = w.d_c + w.d_r
        lat_dtype = {"f32": torch.float32, "bf16": torch.bfloat16, "fp8": torch.uint8, "fp4": torch.bfloat16,
                     "fp8kr": torch.bfloat16}[w.dtype]
        out_dtype = torch.float32 if act == "f32" else torch.bfloat16
        self.q_lat = torch.empty(N, w.n_h, 2 * D if w.dtype == "fp8" else D, dtype=lat_dtype, device=device)
        self.q_scale = torch.empty(N, w.n_h, dtype=torch.float32, device=device) if w.dtype == "fp8" else None
        self.o_lat = torch.empty(N, w.n_h, w.d_c, dtype=out_dtype, device=device)
        self.lse = torch.empty(N, w.n_h, dtype=torch.float32, device=device)
        self.out = torch.empty(N, w.n_h, w.d_v, dtype=out_dtype, device=device)
        self.split_tokens = split_tokens
        self.mode = mode
        self.seq_lens_host = np.asarray(gen["seq_lens"], dtype=np.int32)
        self.plan, self.plan_ws = decode_plan(self.dims, self.seq_lens_host, w.q_len, device, split_tokens)
        nws = decode_uniform_workspace_size(self.dims, w.batch, w.q_len, self.max_seq_len, split_tokens)
        self.decode_ws = torch.empty(max(nws, 1), dtype=torch.uint8, device=device)
        n_new = len(gen["new_positions"])
        self.append_ws = torch.empty(max(lib().mla_append_workspace_size(ctypes.byref(self.dims), n_new), 1),
                                     dtype=torch.uint8, device=device)
        self.absorb_ws = torch.empty(max(lib().mla_absorb_workspace_size(ctypes.byref(self.dims), N), 1),
                                     dtype=torch.uint8, device=device)
        self.fused = fused
        self.fused_ws = torch.empty(max(lib().mla_append_absorb_workspace_size(ctypes.byref(self.dims), n_new, N), 1),
                                    dtype=torch.uint8, device=device)

    def append(self):
        append_latent(self.dims, self.h, self.w_dkv_kr, self.gamma, self.new_pos, self.slots,
                      self.cache, self.cache_scale, workspace=self.append_ws)

    def absorb(self):
        absorb_q(self.dims, self.q_nope, self.q_pe, self.w_uk, self.q_pos, self.q_lat, self.q_scale,
                 workspace=self.absorb_ws)

    def decode(self, split_tokens=None, mode=None):
        mode = self.mode if mode is None else mode
        st = self.split_tokens if split_tokens is None else split_tokens
        if mode == "planned":
            plan, ws = self.plan, self.plan_ws
            if st != self.split_tokens:
                plan, ws = decode_plan(self.dims, self.seq_lens_host, self.w.q_len, self.device, st)
            decode(self.dims, plan, ws, self.q_lat, self.cache, self.block_table, self.seq_lens, self.o_lat,
                   self.lse, q_scale=self.q_scale, cache_scale=self.cache_scale)
            return
        ws = self.decode_ws
        need = decode_uniform_workspace_size(self.dims, self.w.batch, self.w.q_len, self.max_seq_len, st)
        if need > ws.numel():
            ws = torch.empty(need, dtype=torch.uint8, device=self.device)
        decode_uniform(self.dims, self.q_lat, self.cache, self.block_table, self.seq_lens, self.max_seq_len,
                       self.o_lat, self.lse, q_scale=self.q_scale, cache_scale=self.cache_scale,
                       q_len=self.w.q_len, split_tokens=st, workspace=ws)

    def out_proj(self):
        out_proj(self.dims, self.o_lat, self.w_uv, self.out)

    def append_and_absorb(self):
        append_absorb(self.dims, self.h, self.w_dkv_kr, self.gamma, self.new_pos, self.slots, self.cache,
                      self.cache_scale, self.q_nope, self.q_pe, self.w_uk, self.q_pos, self.q_lat, self.q_scale,
                      workspace=self.fused_ws)

    def run(self):
        if self.fused:
            self.append_and_absorb()
        else:
            self.append()
            self.absorb()
        self.decode()
        self.out_proj()

    def capture(self, decode_only=False):
        """HIP graph of one step (or of the decode call).  Every buffer the
        kernels touch is allocated beforehand; the step is run eagerly once
        first so that all kernels are loaded before capture."""
        fn = self.decode if decode_only else self.run
        fn()
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            fn()
        torch.cuda.synchronize()
        return g


class BlockStep(DeviceStep):
    """The whole attention block of one decode step: the query path from the
    new tokens' hidden states (c^Q = W^DQ h, q^C = W^UQ c^Q, W^QR c^Q), the
    four calls, and the output projection u = sum_i W^O_i o_i, all through
    libmla (mla_linear for the dense projections).  The new tokens' hidden
    states are the ones the append writes into the cache."""

    def __init__(self, gen, block, device="cuda:0", split_tokens=0):
        super().__init__(gen, device, split_tokens)
        w = self.w
        act = w.act_dtype
        N = w.batch * w.q_len
        if self.h.shape[0] != N:
            raise ValueError("the block needs every request to append its q_len query tokens")
        self.d_cq = block["d_cq"]
        self.w_dq = _dev(block["w_dq"], device, act)
        self.w_uq = _dev(block["w_uq"], device, act)
        self.w_qr = _dev(block["w_qr"], device, act)
        self.w_o = _dev(block["w_o"], device, act)
        self.c_q = torch.empty(N, self.d_cq, dtype=torch.bfloat16, device=device)
        self.u = torch.empty(N, w.d_model, dtype=torch.bfloat16, device=device)
        shapes = [(self.d_cq, w.d_model), (w.n_h * w.d_h, self.d_cq), (w.n_h * (w.d_h + w.d_r), self.d_cq),
                  (w.d_model, w.n_h * w.d_v), (w.d_model, w.n_h * w.d_c)]
        nws = max(linear_workspace_size(N, n, k) for n, k in shapes)
        self.linear_ws = torch.empty(max(nws, 1), dtype=torch.uint8, device=device)
        self.b = None

    def query(self):
        """c^Q = W^DQ h, then W^UQ c^Q and W^QR c^Q in one mla_linear_pair call
        (a model without the RoPE part runs W^UQ alone)."""
        linear(self.h, self.w_dq, self.c_q, workspace=self.linear_ws)
        if self.w.d_r > 0:
            linear_pair(self.c_q, self.w_uq, self.q_nope, self.w_qr, self.q_pe, workspace=self.linear_ws)
        else:
            linear(self.c_q, self.w_uq, self.q_nope, workspace=self.linear_ws)

    def o_proj(self):
        linear(self.out, self.w_o, self.u, workspace=self.linear_ws)

    def run(self):
        self.query()
        super().run()
        self.o_proj()

    def absorbed_output_weights(self):
        """B_i = W^O_i W^UV_i side by side [d_model, n_h * d_c], formed once (as
        at model load) by mla_absorb_output_weights."""
        w = self.w
        self.b = torch.empty(w.d_model, w.n_h * w.d_c, dtype=torch.bfloat16, device=self.device)
        absorb_output_weights(self.dims, self.w_o, self.w_uv, self.b)
        return self.b

    def o_proj_absorbed(self):
        """u = sum_i B_i o_lat_i straight from the latent output."""
        linear(self.o_lat, self.b, self.u, workspace=self.linear_ws)

    def absorbed_query_weights(self):
        """A_i = W^UK_i^T W^UQ_i stacked [n_h * d_c, d'_c], formed once by
        mla_absorb_query_weights; q_lat_absorbed() then gives the latent
        queries from c^Q in one projection."""
        w = self.w
        self.a = torch.empty(w.n_h * w.d_c, self.d_cq, dtype=torch.bfloat16, device=self.device)
        absorb_query_weights(self.dims, self.w_uq, self.w_uk, self.a)
        N = w.batch * w.q_len
        self.q_lat_a = torch.empty(N, w.n_h * w.d_c, dtype=torch.bfloat16, device=self.device)
        need = linear_workspace_size(N, w.n_h * w.d_c, self.d_cq)
        if need > self.linear_ws.numel():
            self.linear_ws = torch.empty(need, dtype=torch.uint8, device=self.device)
        return self.a

    def q_lat_absorbed(self):
        """q~ [N, n_h * d_c] = A c^Q (the RoPE part still comes from W^QR)."""
        linear(self.c_q, self.a, self.q_lat_a, workspace=self.linear_ws)
