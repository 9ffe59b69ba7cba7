"""One MLA decode step on the GPU: inputs uploaded once, the four library calls.

Used by the tests, the smoke check and bench.py. Holds device tensors for the
weights, the new tokens, the latent cache and every output, plus the
workspace the library asks for.
"""
from __future__ import annotations

from typing import Optional

import numpy as np
import torch

from . import mla
from .inputs import MLAInputs, make_topk_indices as gen_topk


def to_device(a: Optional[np.ndarray], dtype: str, device="cuda") -> Optional[torch.Tensor]:
    """Stored numpy array (uint16 bf16 bits or float32) -> device tensor."""
    if a is None:
        return None
    if dtype == "bf16":
        t = torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16)
    else:
        t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return t.to(device)


class DeviceStep:
    def __init__(self, inp: MLAInputs, num_splits: int = 0, device="cuda", ws_splits=(), precomposed=False,
                 poison=False):
        """ws_splits: further split counts the workspace must also cover.
        precomposed: form W_QK and W_OV once here and run the query and output
        sides as one product each (no per-head outputs then).
        poison: before every library call, fill the workspace with 0xFF bytes
        (NaN as float32) and the call's outputs with NaN, so that an output
        element or a partial result the call fails to write cannot pass on a
        value left by an earlier call (the tests use this; timing does not)."""
        cfg = inp.cfg
        self.cfg, self.inp, self.device = cfg, inp, device
        self.num_splits = num_splits
        dt = cfg.dtype
        self.W = {k: to_device(v, dt, device) for k, v in inp.weights.items()}
        self.h_t = to_device(inp.h_t, dt, device)
        self.cache = to_device(inp.cache, dt, device)
        self.block_table = (None if inp.block_table is None
                            else torch.from_numpy(inp.block_table).to(device))
        self.pos = torch.from_numpy(inp.ctx.astype(np.int32)).to(device)
        self.seq_lens = torch.from_numpy(inp.seq_lens.astype(np.int32)).to(device)
        self.max_seq_len = int(inp.seq_lens.max())
        self.dims = mla.make_dims(cfg.d, cfg.H, cfg.d_h, cfg.d_v, cfg.d_c, cfg.d_R, cfg.d_cq, dt,
                                  softmax_scale=cfg.scale, rope_theta=cfg.theta)
        self.cdesc = mla.make_cache(self.cache, self.block_table)
        B, H, D = cfg.B, cfg.H, cfg.D
        tdt = self.dims.torch_dtype
        if cfg.topk:
            # sparse attention over a seeded top-k list per sequence
            idx, counts = gen_topk(cfg, inp.seq_lens, cfg.topk)
            self.topk_idx_host, self.topk_counts_host = idx, counts
            self.topk_idx = torch.from_numpy(idx).to(device)
            self.topk_counts = torch.from_numpy(counts).to(device)
        ws_bytes = max(mla.workspace_bytes(self.dims, B, max(self.max_seq_len, cfg.topk), s)
                       for s in (num_splits, *ws_splits))
        self.ws = torch.empty(ws_bytes, dtype=torch.uint8, device=device)
        # query rows [q_lat ; q_R ; low term of q_R]
        self.q = torch.empty(B, H, D + cfg.d_R, dtype=tdt, device=device)
        self.o_lat = torch.empty(B, H, cfg.d_c, dtype=torch.float32, device=device)
        self.lse = torch.empty(B, H, dtype=torch.float32, device=device)
        self.o_heads = torch.empty(B, H, cfg.d_v, dtype=tdt, device=device)
        self.out = torch.empty(B, cfg.d, dtype=tdt, device=device)
        self.precomposed = precomposed
        self.poison = poison
        if precomposed:
            qin = cfg.d_cq if cfg.d_cq else cfg.d
            self.W_QK = torch.empty(H, cfg.d_c, qin, dtype=tdt, device=device)
            self.W_OV = torch.empty(cfg.d, H * cfg.d_c, dtype=tdt, device=device)
            mla.mla_precompose(self.dims, self.W["W_UQ"], self.W["W_UK"], self.W_QK, self.W["W_UV"],
                               self.W["W_O"], self.W_OV)

    @property
    def splits(self) -> int:
        n = self.cfg.topk if self.cfg.topk else self.max_seq_len
        return mla.decode_num_splits(self.dims, self.cfg.B, n, self.num_splits)

    def _poison(self, *outs):
        if self.poison:
            self.ws.fill_(0xFF)
            for t in outs:
                if t is not None:
                    t.fill_(float("nan"))

    def compress_append(self):
        self._poison()
        mla.mla_compress_append(self.dims, self.h_t, self.W["W_DKV"], self.W["W_KR"],
                                self.W.get("gamma_kv"), self.pos, self.cdesc, self.ws)

    def absorb_q(self):
        self._poison(self.q)
        if self.precomposed:
            mla.mla_absorb_q_precomposed(self.dims, self.h_t, self.W["W_DQ"], self.W_QK, self.W["W_QR"],
                                         self.pos, self.q, self.ws)
            return
        mla.mla_absorb_q(self.dims, self.h_t, self.W["W_DQ"], self.W["W_UQ"], self.W["W_QR"],
                         self.W["W_UK"], self.pos, self.q, self.ws)

    def decode_attn(self, num_splits: Optional[int] = None):
        s = self.num_splits if num_splits is None else num_splits
        self._poison(self.o_lat, self.lse)
        if self.cfg.topk:
            mla.mla_decode_attn_sparse(self.dims, self.q, self.cdesc, self.topk_idx, self.topk_counts,
                                       self.o_lat, self.lse, self.ws, s)
        else:
            mla.mla_decode_attn(self.dims, self.q, self.cdesc, self.seq_lens, self.max_seq_len,
                                self.o_lat, self.lse, self.ws, s)

    def out_proj(self):
        self._poison(self.o_heads, self.out)
        if self.precomposed:
            mla.mla_out_proj_precomposed(self.dims, self.o_lat, self.W_OV, self.out, self.ws)
            return
        mla.mla_out_proj(self.dims, self.o_lat, self.W["W_UV"], self.W["W_O"], self.o_heads,
                         self.out, self.ws)

    def run(self):
        self.compress_append()
        self.absorb_q()
        self.decode_attn()
        self.out_proj()

    # host copies as float64 numpy
    @staticmethod
    def host(t: torch.Tensor) -> np.ndarray:
        return t.detach().to(torch.float64).cpu().numpy()

    def cache_row(self, b: int, u: int) -> np.ndarray:
        if self.block_table is None:
            return self.host(self.cache[b, u])
        bs = self.cfg.block_size
        blk = int(self.inp.block_table[b, u // bs])
        return self.host(self.cache[blk, u % bs])


class DevicePrefill:
    """Causal prefill of the newest T tokens of every sequence: the cache holds
    ctx_b rows per sequence (the T tokens' own rows among them), q is the
    seeded per-head query [B][T][H][d_h + d_R]."""

    def __init__(self, inp: MLAInputs, T: int, device="cuda", q_std: float = 1.0, poison=False):
        """poison: fill the workspace (0xFF bytes) and the outputs (NaN) before
        every call, as DeviceStep does."""
        from .inputs import make_prefill_query
        cfg = inp.cfg
        self.cfg, self.inp, self.T = cfg, inp, T
        dt = cfg.dtype
        self.W_UK = to_device(inp.weights["W_UK"], dt, device)
        self.W_UV = to_device(inp.weights["W_UV"], dt, device)
        self.cache = to_device(inp.cache, dt, device)
        self.block_table = (None if inp.block_table is None
                            else torch.from_numpy(inp.block_table).to(device))
        self.seq_lens_host = inp.ctx.astype(np.int32)
        self.seq_lens = torch.from_numpy(self.seq_lens_host).to(device)
        self.max_seq_len = int(self.seq_lens_host.max())
        self.dims = mla.make_dims(cfg.d, cfg.H, cfg.d_h, cfg.d_v, cfg.d_c, cfg.d_R, cfg.d_cq, dt,
                                  softmax_scale=cfg.scale, rope_theta=cfg.theta)
        self.cdesc = mla.make_cache(self.cache, self.block_table)
        self.q_host = make_prefill_query(cfg, T, q_std)
        self.q = to_device(self.q_host, dt, device)
        tdt = self.dims.torch_dtype
        self.o = torch.empty(cfg.B, T, cfg.H, cfg.d_v, dtype=tdt, device=device)
        self.lse = torch.empty(cfg.B, T, cfg.H, dtype=torch.float32, device=device)
        ws = max(mla.prefill_workspace_bytes(self.dims, cfg.B, T, self.max_seq_len, self.cdesc, a)
                 for a in (mla.PREFILL_MATERIALIZED, mla.PREFILL_ABSORBED))
        self.ws = torch.empty(ws, dtype=torch.uint8, device=device)
        self.poison = poison

    def run(self, algo: int):
        if self.poison:
            self.ws.fill_(0xFF)
            self.o.fill_(float("nan"))
            self.lse.fill_(float("nan"))
        mla.mla_prefill_attn(self.dims, self.q, self.cdesc, self.seq_lens, self.max_seq_len, self.W_UK, self.W_UV,
                             algo, self.o, self.lse, self.ws)
