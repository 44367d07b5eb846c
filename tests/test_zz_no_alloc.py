"""stream_attend_scratch, the allocation-free attention entry point, against stream_attend.

The variant keeps the split-KV partials in the library's static per-GPU
scratch instead of the pool's workspace; with the same split count it runs the
same kernels, so its output and log-sum-exp equal stream_attend's bit for bit.
Two calls in a row, the second smaller, then a call whose partials would not
fit in the scratch (refused, nothing consumed).  The outputs are also checked
against the fp64 oracle at the bf16 tolerance.
"""

import numpy as np
import pytest

from bounded_kv_cache_stream_amd import kvstream as kv
from bounded_kv_cache_stream_amd import synth
from oracle import attention, window
from tests.gpu_common import LSE_ABS_BF16, assert_close, max_abs, say, to64, torch_cuda

pytestmark = pytest.mark.gpu


def test_scratch_entry_point_matches_stream_attend():
    torch = torch_cuda()
    T, H, S, W = 1004, 16, 1, 8
    cfg = kv.make_config(num_layers=1, num_heads=H, page_tokens=T, scale_frames=S, sliding_window=W,
                         keyframe_interval=1, pages_per_layer=S + W + 1, max_queries=T, max_splits=64)
    c = kv.KVCache(cfg, device="cuda")
    host = {}
    for t in range(10):  # frames 0..9: the window holds 1..8 after frame 9's eviction
        _, k, v = synth.iid_frame(130, 0, t, (T, H, 64), device="cuda", dtype=torch.bfloat16)
        c.append(0, t, k, v)
        c.evict(0)
        host[t] = (to64(k), to64(v))
    att = window.attended_frames(9, S, W, 1)
    K = np.concatenate([host[f][0] for f in att])
    V = np.concatenate([host[f][1] for f in att])
    # two calls in a row (1004 queries: 8 splits; then 300 queries: 16 splits, smaller partials)
    for n_q, wid in ((T, 131), (300, 132)):
        q = synth.iid_frame(wid, 0, 0, (n_q, H, 64), device="cuda", dtype=torch.bfloat16)[0]
        want = torch.empty_like(q)
        got = torch.full_like(q, float("nan"))
        lse_want = torch.empty(n_q * H, dtype=torch.float32, device="cuda")
        lse_got = torch.full((n_q * H,), float("nan"), dtype=torch.float32, device="cuda")
        c.attend(0, q, 0.125, out=want, lse=lse_want)
        c.attend(0, q, 0.125, out=got, lse=lse_got, static_scratch=True)
        torch.cuda.synchronize()
        assert torch.equal(got.view(torch.int16), want.view(torch.int16)), n_q
        assert torch.equal(lse_got.view(torch.int32), lse_want.view(torch.int32)), n_q
        ref, ref_lse = attention.attend(to64(q), K, V, 0.125)
        ma, rl = assert_close(to64(got), ref, bf16=True, what=f"scratch entry point, {n_q} queries")
        assert max_abs(to64(lse_got).reshape(n_q, H), ref_lse) <= LSE_ABS_BF16
        say(f"stream_attend_scratch, {n_q} queries: equal to stream_attend bit for bit; max_abs {ma:.2e} "
            f"rel_l2 {rl:.2e}")
    # 64 splits of 1004 queries x 16 heads need 271 MB of partials: refused before anything is enqueued
    q = synth.iid_frame(133, 0, 0, (T, H, 64), device="cuda", dtype=torch.bfloat16)[0]
    out = torch.zeros_like(q)
    c.set_splits(64)
    with pytest.raises(kv.KVError) as e:
        c.attend(0, q, 0.125, out=out, static_scratch=True)
    assert e.value.status == kv.KV_ERR_SHAPE and "static scratch" in str(e.value)
    torch.cuda.synchronize()
    assert not out.view(torch.int16).any()
    c.set_splits(0)
    # a transient frame is consumed by the scratch call exactly as by stream_attend
    _, k, v = synth.iid_frame(130, 0, 10, (T, H, 64), device="cuda", dtype=torch.bfloat16)
    c.append(0, 10, k, v, transient=True)
    assert c.info(0)["transient_pending"] == 1
    c.attend(0, q, 0.125, out=out, static_scratch=True)
    assert c.info(0)["transient_pending"] == 0
