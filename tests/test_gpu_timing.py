"""GPU: the kernel-timing hook (mla_time_next_attn).

The next attention call stamps the caller's events from its own launches: the
attention kernel's start and end, and the end of the call's last kernel. The
hook must leave the call's results unchanged (bit for bit against an untimed
call on the same inputs), give ordered, positive spans, hold for one call
only, and be cleared by a call that fails validation.
"""
import os
import sys

import numpy as np
import pytest
import torch

from kv_cache_compression_mla_amd import inputs as gen
from kv_cache_compression_mla_amd import mla
from kv_cache_compression_mla_amd.step import DeviceStep
from _common import make_inputs

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
from bench import DeviceEvents  # noqa: E402

pytestmark = pytest.mark.gpu

V3 = gen.CONFIGS["v3_b1_ctx4k"]


def say(msg):
    print(f"[gpu-case] {msg}", flush=True)


@pytest.fixture(scope="module")
def events():
    ev = DeviceEvents(torch)
    yield ev
    ev.close()


def _timed_call(st, ev, num_splits=None):
    e = [ev.create() for _ in range(3)]
    mla.mla_time_next_attn(e[0].value, e[1].value, e[2].value)
    st.decode_attn(num_splits=num_splits)
    torch.cuda.synchronize()
    return ev.elapsed_ms(e[0], e[1]), ev.elapsed_ms(e[0], e[2])


@pytest.mark.parametrize("num_splits,label", [(0, "balanced plan, merged"), (1, "one chunk per sequence")])
def test_hook_stamps_the_mfma_call_and_changes_nothing(events, num_splits, label):
    cfg = V3.with_(name="v3_timed", B=3, ctx=(700, 1500, 64), seed=41)
    inp = make_inputs(cfg)
    st = DeviceStep(inp, poison=True, num_splits=num_splits)
    say(f"{label}: B={cfg.B} splits={st.splits} kernel={mla.decode_kernel(st.dims)}")
    assert mla.decode_kernel(st.dims) == 1
    st.compress_append()
    st.absorb_q()
    st.decode_attn()
    torch.cuda.synchronize()
    ref = (st.host(st.o_lat), st.host(st.lse))
    k_ms, c_ms = _timed_call(st, events)
    say(f"{label}: kernel {k_ms * 1e3:.1f} us, call {c_ms * 1e3:.1f} us")
    assert 0.0 < k_ms <= c_ms < 1000.0
    assert np.array_equal(ref[0], st.host(st.o_lat)) and np.array_equal(ref[1], st.host(st.lse))
    # one call only: the next, untimed call leaves fresh events unrecorded
    e = [events.create() for _ in range(2)]
    st.decode_attn()
    torch.cuda.synchronize()
    with pytest.raises(RuntimeError):
        events.elapsed_ms(e[0], e[1])


def test_hook_on_the_general_kernel_and_the_sparse_call(events):
    cfg = V3.with_(name="v3_h16_timed", H=16, d=1024, d_cq=256, B=2, ctx=(5, 150), seed=42)
    st = DeviceStep(make_inputs(cfg), poison=True)
    assert mla.decode_kernel(st.dims) == 2
    st.compress_append()
    st.absorb_q()
    k_ms, c_ms = _timed_call(st, events)
    say(f"general kernel: kernel {k_ms * 1e3:.1f} us, call {c_ms * 1e3:.1f} us")
    assert 0.0 <= k_ms <= c_ms < 1000.0

    cfg = V3.with_(name="v3_topk_timed", B=2, ctx=(900, 300), topk=64, seed=43)
    st = DeviceStep(make_inputs(cfg), poison=True)
    st.compress_append()
    st.absorb_q()
    st.decode_attn()
    torch.cuda.synchronize()
    ref = st.host(st.o_lat)
    k_ms, c_ms = _timed_call(st, events)
    say(f"sparse: kernel {k_ms * 1e3:.1f} us, call {c_ms * 1e3:.1f} us")
    assert 0.0 < k_ms <= c_ms < 1000.0
    assert np.array_equal(ref, st.host(st.o_lat))


def test_failed_call_clears_the_hook(events):
    cfg = V3.with_(name="v3_timed_fail", B=2, ctx=(100, 200), seed=44)
    st = DeviceStep(make_inputs(cfg), poison=True)
    st.compress_append()
    st.absorb_q()
    e = [events.create() for _ in range(3)]
    mla.mla_time_next_attn(e[0].value, e[1].value, e[2].value)
    with pytest.raises(RuntimeError):
        # max_seq_len beyond the cache's capacity: rejected on the host
        mla.mla_decode_attn(st.dims, st.q, st.cdesc, st.seq_lens, st.cdesc.capacity + 1, st.o_lat, st.lse, st.ws)
    st.decode_attn()
    torch.cuda.synchronize()
    with pytest.raises(RuntimeError):
        events.elapsed_ms(e[0], e[2])
