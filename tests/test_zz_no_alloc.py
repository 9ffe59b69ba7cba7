"""The allocation-free decode attention (mla_decode_attn_noalloc) against
mla_decode_attn on the same inputs, through the C ABI: identical kernels and
chunk plan, so the outputs must agree bit for bit. Two calls in a row share
the library's static scratch, the second with a smaller batch (the first
call's contents are left behind in the scratch and must not matter)."""
import numpy as np
import pytest
import torch

from kv_cache_compression_mla_amd import inputs as gen
from kv_cache_compression_mla_amd import mla
from kv_cache_compression_mla_amd.step import DeviceStep
from _common import make_inputs

pytestmark = pytest.mark.gpu

V3 = gen.CONFIGS["v3_b1_ctx4k"]


def _case(cfg, splits):
    inp = make_inputs(cfg)
    st = DeviceStep(inp, poison=True, num_splits=splits)
    st.compress_append()        # the new token's row, which the attention reads last
    st.absorb_q()
    q = st.q
    # the workspace path
    st._poison(st.o_lat, st.lse)
    mla.mla_decode_attn(st.dims, q, st.cdesc, st.seq_lens, st.max_seq_len, st.o_lat, st.lse, st.ws, splits)
    torch.cuda.synchronize()
    ref_o, ref_l = st.o_lat.clone(), st.lse.clone()
    # the static-scratch path, outputs poisoned first
    st._poison(st.o_lat, st.lse)
    mla.mla_decode_attn_noalloc(st.dims, q, st.cdesc, st.seq_lens, st.max_seq_len, st.o_lat, st.lse, splits)
    torch.cuda.synchronize()
    assert torch.isfinite(ref_o).all(), cfg.name
    print(f"[gpu-case] noalloc {cfg.name} B={cfg.B} splits={splits}: "
          f"max |o_lat diff| {(st.o_lat - ref_o).abs().max().item():.3e}", flush=True)
    assert torch.equal(st.o_lat, ref_o), cfg.name
    assert torch.equal(st.lse, ref_l), cfg.name


def test_noalloc_matches_workspace_call_twice_second_smaller():
    first = V3.with_(name="noalloc_big", B=12, ctx=None, ctx_range=(200, 3000), seed=41)
    second = V3.with_(name="noalloc_small", B=3, ctx=(5, 90, 700), paged=True, block_size=16, seed=42)
    _case(first, 0)
    _case(second, 0)
    _case(second, 3)
