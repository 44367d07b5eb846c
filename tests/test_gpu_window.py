"""GPU parity of the window-mode path (page write, eviction, attention) with the oracle.

Workloads (bounded_kv_cache_stream_amd.synth.WORKLOADS): the tiny fp32 stream
(every frame checked), the 1004-token / 16-head stream with a 64-frame window
(200 frames; page tables every frame; attention fully at the scale phase, at
the last frame before and the first after eviction starts and at the end, and
on sampled query rows every 10th frame), and the 10,000-frame stream with
keyframe interval 4 (page tables and occupancy every frame, attention at the
checkpoints).  Inputs come from the seeded generators; the oracle sees the
exact bf16/fp32 values the GPU got, widened to float64.
"""

import numpy as np
import pytest

from bounded_kv_cache_stream_amd import kvstream as kv
from bounded_kv_cache_stream_amd import synth
from oracle import attention, window
from tests.gpu_common import LSE_ABS_BF16, LSE_ABS_FP32, assert_close, max_abs, say, to32, to64, torch_cuda

pytestmark = pytest.mark.gpu


def _cfg(w, pages=None, max_queries=None, max_splits=16):
    return kv.make_config(num_layers=1, num_heads=w["heads"], head_dim=w["head_dim"], page_tokens=w["tokens"],
                          dtype=kv.KV_BF16 if w["dtype"] == "bf16" else kv.KV_FP32,
                          scale_frames=w["scale_frames"], sliding_window=w["window"],
                          keyframe_interval=w["keyframe_interval"],
                          pages_per_layer=pages or (w["scale_frames"] + w["window"] + 1),
                          max_queries=max_queries or max(1, w["scale_frames"]) * w["tokens"], max_splits=max_splits)


class _Stream:
    """Drives one window-mode layer through append -> evict -> attend and the oracle's policy."""

    def __init__(self, wid, device="cuda", keep=None):
        self.torch = torch_cuda()
        self.w = synth.WORKLOADS[wid]
        self.wid = wid
        self.cache = kv.KVCache(_cfg(self.w), device=device)
        self.sim = window.WindowCache(self.w["scale_frames"], self.w["window"], self.w["keyframe_interval"],
                                      self.w["scale_frames"] + self.w["window"] + 1)
        shape = (self.w["tokens"], self.w["heads"], self.w["head_dim"])
        self.shape = shape
        self.ar1 = synth.AR1Stream(wid, 0, shape, device=device) if self.w["ar1"] else None
        self.host = {}  # frame -> (k, v) float32 numpy, only frames the checks need
        self.keep = keep  # None = keep every retained frame
        self.pending_q = []

    def frame(self, t):
        if self.ar1 is not None:
            q, k, v = self.ar1.next()
        else:
            q, k, v = synth.iid_frame(self.wid, 0, t, self.shape, device="cuda")
        return q, k, v

    def step(self, t):
        """Append + evict frame t; returns (q of this call or None, attended frames or None)."""
        q, k, v = self.frame(t)
        S = self.w["scale_frames"]
        transient = not window.is_keyframe(t, S, self.w["keyframe_interval"])
        self.cache.append(0, t, k, v)
        self.cache.evict(0)
        self.sim.append(t)
        self.sim.evict()
        if self.keep is None or t in self.keep:
            self.host[t] = (to32(k), to32(v))
        ids, lens, frames = self.cache.page_table(0)
        assert ids == self.sim.page_ids() and frames == self.sim.persisted(), f"page table at frame {t}"
        assert lens == [self.w["tokens"]] * len(ids)
        assert self.cache.info(0)["transient_pending"] == int(transient)
        if self.w["window"]:
            assert len(ids) <= S + self.w["window"]
        if t < S - 1:
            self.pending_q.append(q)
            return None, None
        if t == S - 1:
            self.pending_q.append(q)
            q = self.torch.cat(self.pending_q)
            self.pending_q = []
        att = self.sim.attended()
        if self.keep is None:
            for f in list(self.host):
                if f not in att:
                    del self.host[f]
        return q, att

    def kv_of(self, att):
        K = np.concatenate([self.host[f][0] for f in att]).astype(np.float64)
        V = np.concatenate([self.host[f][1] for f in att]).astype(np.float64)
        return K, V


def test_tiny_fp32_stream_every_frame():
    s = _Stream(0)
    torch = s.torch
    tau = s.w["sm_scale"]
    for t in range(s.w["frames"]):
        q, att = s.step(t)
        if q is None:
            continue
        lse = torch.empty(q.shape[0] * q.shape[1], dtype=torch.float32, device="cuda")
        out = s.cache.attend(0, q, tau, lse=lse)
        K, V = s.kv_of(att)
        ref, ref_lse = attention.attend(to64(q), K, V, tau)
        assert_close(to64(out), ref, bf16=False, what=f"tiny frame {t}")
        assert max_abs(to64(lse).reshape(ref_lse.shape), ref_lse) <= LSE_ABS_FP32
    say("tiny fp32 stream: 12 frames match")


def _check_rows(s, q, out, att, rows, tau, what, lse=None):
    K, V = s.kv_of(att)
    q64 = to64(q)[rows]
    ref, ref_lse = attention.attend(q64, K, V, tau)
    ma, rl = assert_close(to64(out)[rows], ref, bf16=True, what=what)
    if lse is not None:
        l = to64(lse).reshape(-1, q.shape[1])[rows]
        assert max_abs(l, ref_lse) <= LSE_ABS_BF16, what
    return ma, rl


def test_frame1004_window64_stream():
    s = _Stream(1)
    torch = s.torch
    tau = s.w["sm_scale"]
    full = {7, 71, 72, 199}
    rng = np.random.default_rng(1)
    for t in range(s.w["frames"]):
        q, att = s.step(t)
        if q is None:
            continue
        lse = torch.empty(q.shape[0] * q.shape[1], dtype=torch.float32, device="cuda")
        out = s.cache.attend(0, q, tau, lse=lse)
        n_tok = sum(1 for _ in att) * s.w["tokens"]
        if t in full:
            ma, rl = _check_rows(s, q, out, att, slice(None), tau, f"frame {t} (all rows)", lse)
            say(f"frame {t}: {q.shape[0]} queries x {n_tok} keys, max_abs {ma:.2e} rel_l2 {rl:.2e}")
        elif t % 10 == 0:
            rows = np.sort(rng.choice(q.shape[0], 48, replace=False))
            _check_rows(s, q, out, att, rows, tau, f"frame {t} (48 rows)", lse)
    torch.cuda.synchronize()


def test_split_count_does_not_change_results():
    # split-KV is an internal partition; any count gives the same attention up to fp32 reassociation
    s = _Stream(1)
    torch = s.torch
    for t in range(12):
        q, att = s.step(t)
    outs = []
    for splits in (1, 3, 8, 16):
        s.cache.set_splits(splits)
        # re-run the same attention: the transient page is not involved (every frame is a keyframe)
        outs.append(to64(s.cache.attend(0, q, 1.0)))
    K, V = s.kv_of(att)
    ref, _ = attention.attend(to64(q), K, V, 1.0)
    for o in outs:
        assert_close(o, ref, bf16=True, what="split variant")
        assert max_abs(o, outs[0]) <= 8e-3


def test_attention_kernel_timing_events():
    # kv_attend_timing records the kernel's own duration on the call's stream for the next max_calls calls
    # and leaves the results unchanged; calls beyond max_calls are not timed
    s = _Stream(1)
    torch = s.torch
    for t in range(12):
        q, att = s.step(t)
    plain = s.cache.attend(0, q, 1.0).clone()
    kv.kv_attend_timing(s.cache.handle, 3)
    outs = [s.cache.attend(0, q, 1.0).clone() for _ in range(5)]
    ms, n = kv.kv_attend_timing_read(s.cache.handle)
    assert n == 3 and 0.0 < ms < 1000.0
    for o in outs:
        assert torch.equal(o, plain)
    kv.kv_attend_timing(s.cache.handle, 0)
    s.cache.attend(0, q, 1.0)
    assert kv.kv_attend_timing_read(s.cache.handle) == (0.0, 0)


def test_long_stream_keyframe4_10000_frames():
    w = synth.WORKLOADS[2]
    S, W, k = w["scale_frames"], w["window"], w["keyframe_interval"]
    checks = [99, 999, 9999]
    rng = np.random.default_rng(2)
    checks += sorted(int(x) for x in rng.choice(np.arange(300, 9999), 3, replace=False))
    need = set()
    for t in checks:
        need.update(window.attended_frames(t, S, W, k))
    s = _Stream(2, keep=need)
    torch = s.torch
    tau = w["sm_scale"]
    q_saved = {}
    for t in range(w["frames"]):
        q, att = s.step(t)
        if t in (99, 999, 9999):
            assert s.cache.page_table(0)[2] == window.persisted_frames(t, S, W, k)
        if q is None:
            continue
        lse = torch.empty(q.shape[0] * q.shape[1], dtype=torch.float32, device="cuda")
        out = s.cache.attend(0, q, tau, lse=lse)
        if t in checks:
            q_saved[t] = (to32(q), to32(out), to32(lse), att)
        if t % 1000 == 0:
            say(f"long stream: frame {t}")
    torch.cuda.synchronize()
    for t in checks:
        qn, on, ln, att = q_saved[t]
        K, V = s.kv_of(att)
        ref, ref_lse = attention.attend(qn.astype(np.float64), K, V, tau)
        ma, rl = assert_close(on.astype(np.float64), ref, bf16=True, what=f"long stream frame {t}")
        assert max_abs(ln.astype(np.float64).reshape(ref_lse.shape), ref_lse) <= LSE_ABS_BF16
        say(f"long stream frame {t}: {len(att)} frames attended, max_abs {ma:.2e} rel_l2 {rl:.2e}")


def test_multi_layer_append_matches_single_layer_append():
    torch = torch_cuda()
    T, H, L = 100, 4, 3
    cfg = kv.make_config(num_layers=L, num_heads=H, page_tokens=T, scale_frames=0, sliding_window=2,
                         keyframe_interval=1, pages_per_layer=3, max_queries=T, max_splits=4)
    a = kv.KVCache(cfg, device="cuda")
    b = kv.KVCache(cfg, device="cuda")
    for t in range(5):
        k = torch.randn(L, T, H, 64, device="cuda").bfloat16()
        v = torch.randn(L, T, H, 64, device="cuda").bfloat16()
        a.append_layers(0, t, k, v)
        for l in range(L):
            b.append(l, t, k[l].contiguous(), v[l].contiguous())
            a.evict(l)
            b.evict(l)
    torch.cuda.synchronize()
    for l in range(L):
        ids, lens, fr = a.page_table(l)
        assert (ids, lens, fr) == b.page_table(l)
        for pid, n in zip(ids, lens):
            for x, y in zip(a.page_view(l, pid), b.page_view(l, pid)):
                assert torch.equal(x.cpu().view(torch.uint8) if x.dtype != torch.int32 else x.cpu(),
                                   y.cpu().view(torch.uint8) if y.dtype != torch.int32 else y.cpu())


def test_batched_page_write_full_shape_bytes():
    # the 24-layer batched write the append benchmark times (24 layers x 1004 tokens x 16 heads x 64, bf16,
    # 197 MB per frame): every layer's page holds the caller's K and V as [H][Ts][D] bit for bit, zero pad
    # slots and the token ids, for two persisted frames and then a transient one
    torch = torch_cuda()
    T, H, L = 1004, 16, 24
    cfg = kv.make_config(num_layers=L, num_heads=H, page_tokens=T, scale_frames=1, sliding_window=1,
                         keyframe_interval=2, pages_per_layer=3, max_queries=T, max_splits=4)
    c = kv.KVCache(cfg, device="cuda")
    Ts = c.layout["token_stride"]
    g = torch.Generator(device="cuda")
    g.manual_seed(11)
    for t in range(3):  # frames 0 (scale) and 1 (keyframe) persist; frame 2 is not a keyframe: transient
        k = torch.randn(L, T, H, 64, device="cuda", generator=g).bfloat16()
        v = torch.randn(L, T, H, 64, device="cuda", generator=g).bfloat16()
        c.append_layers(0, t, k, v)
        torch.cuda.synchronize()
        for l in range(L):
            c.evict(l)
            pid = c.page_table(l)[0][-1] if t < 2 else cfg.pages_per_layer
            pk, pv, ids = c.page_view(l, pid)
            assert torch.equal(pk[:, :T].view(torch.int16), k[l].permute(1, 0, 2).view(torch.int16)), (t, l)
            assert torch.equal(pv[:, :T].view(torch.int16), v[l].permute(1, 0, 2).view(torch.int16)), (t, l)
            assert not pk[:, T:].view(torch.int16).any() and not pv[:, T:].view(torch.int16).any(), (t, l)
            assert ids.cpu().numpy().tolist() == [t * T + i for i in range(T)] + [-1] * (Ts - T), (t, l)
    say(f"batched page write: {L} layers x {T} tokens x {H} heads bit for bit")


@pytest.mark.parametrize("dtype,T,H", [("bf16", 1004, 16), ("fp32", 100, 2)])
def test_page_write_bytes(dtype, T, H):
    # a page holds the frame's K and V as [H][Ts][D] bit for bit, zero pad slots
    # and the global token ids frame*T + slot (-1 in pad slots); a non-keyframe
    # goes to the layer's transient page (id pages_per_layer)
    torch = torch_cuda()
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    cfg = kv.make_config(num_layers=2, num_heads=H, page_tokens=T, dtype=kv.KV_BF16 if dtype == "bf16" else kv.KV_FP32,
                         scale_frames=1, sliding_window=2, keyframe_interval=2, pages_per_layer=4, max_queries=T,
                         max_splits=4)
    c = kv.KVCache(cfg, device="cuda")
    Ts = c.layout["token_stride"]
    assert Ts == (T + 63) // 64 * 64
    g = torch.Generator(device="cuda")
    g.manual_seed(5)
    for t in range(3):  # frames 0 (scale), 1 (keyframe), 2 (transient)
        k = torch.randn(T, H, 64, device="cuda", generator=g).to(tdt)
        v = torch.randn(T, H, 64, device="cuda", generator=g).to(tdt)
        c.append(1, t, k, v)
        c.evict(1)
        pid = c.page_table(1)[0][-1] if t < 2 else cfg.pages_per_layer
        pk, pv, ids = c.page_view(1, pid)
        torch.cuda.synchronize()
        iv = torch.int16 if dtype == "bf16" else torch.int32
        assert torch.equal(pk[:, :T].cpu().view(iv), k.permute(1, 0, 2).cpu().view(iv)), f"K of frame {t}"
        assert torch.equal(pv[:, :T].cpu().view(iv), v.permute(1, 0, 2).cpu().view(iv)), f"V of frame {t}"
        assert not pk[:, T:].cpu().view(iv).any() and not pv[:, T:].cpu().view(iv).any(), f"pad of frame {t}"
        expect = [t * T + i for i in range(T)] + [-1] * (Ts - T)
        assert ids.cpu().numpy().tolist() == expect, f"ids of frame {t}"


def test_two_head_shard_many_splits():
    # one GPU's share when the heads are split across 8 GPUs: 2 heads of the
    # 1004-token, 72-frame cache; the library fills the chip with many KV splits
    torch = torch_cuda()
    T, H, S, Wf = 1004, 2, 8, 64
    cfg = kv.make_config(num_layers=1, num_heads=H, page_tokens=T, scale_frames=S, sliding_window=Wf,
                         keyframe_interval=1, pages_per_layer=S + Wf + 1, max_queries=S * T, max_splits=64)
    cache = kv.KVCache(cfg, device="cuda")
    ar = synth.AR1Stream(1, 0, (T, H, 64), device="cuda")
    host = {}
    for t in range(S + Wf + 1):
        q, k, v = ar.next()
        cache.append(0, t, k, v)
        cache.evict(0)
        host[t] = (to32(k), to32(v))
    att = list(range(S)) + list(range(S + 1, S + Wf + 1))
    assert cache.page_table(0)[2] == att
    K = np.concatenate([host[f][0] for f in att]).astype(np.float64)
    V = np.concatenate([host[f][1] for f in att]).astype(np.float64)
    ref, ref_lse = attention.attend(to64(q), K, V, 1.0)
    for splits in (0, 64):
        cache.set_splits(splits)
        lse = torch.empty(T * H, dtype=torch.float32, device="cuda")
        out = cache.attend(0, q, 1.0, lse=lse)
        ma, rl = assert_close(to64(out), ref, bf16=True, what=f"2-head shard, splits {splits or 'auto'}")
        assert max_abs(to64(lse).reshape(ref_lse.shape), ref_lse) <= LSE_ABS_BF16
        say(f"2-head shard (splits {splits or 'auto'}): max_abs {ma:.2e} rel_l2 {rl:.2e}")


@pytest.mark.parametrize("dname,T,sp,k", [("bf16", 40, 5, 2), ("fp32", 20, 3, 1)])
def test_special_tokens_stream_every_frame(dname, T, sp, k):
    # window eviction with cross-frame special-token persistence: every frame
    # the page table matches the oracle, attention covers scale frames +
    # special tokens of every evicted frame + window + transient, and the
    # special pages hold the evicted frames' first rows bit-exactly
    torch = torch_cuda()
    S, W, H, F = 2, 4, 4, 40
    per_page = (T // sp) * sp
    pages = S + W + 1 + (F * sp) // per_page + 2
    dt = torch.bfloat16 if dname == "bf16" else torch.float32
    cfg = kv.make_config(num_layers=1, num_heads=H, page_tokens=T, dtype=kv.KV_BF16 if dname == "bf16" else kv.KV_FP32,
                         scale_frames=S, sliding_window=W, keyframe_interval=k, pages_per_layer=pages,
                         max_queries=S * T, max_splits=8, special_tokens=sp)
    cache = kv.KVCache(cfg, device="cuda")
    sim = window.SpecialWindowCache(S, W, k, pages, special=sp, tokens_per_frame=T)
    host = {}
    pending = []
    for t in range(F):
        q, kk, v = synth.iid_frame(103, 0, t, (T, H, 64), device="cuda", dtype=dt)
        host[t] = (kk.cpu(), v.cpu())
        cache.append(0, t, kk, v)
        sim.append(t)
        assert cache.evict(0) == sim.evict()
        ids, lens, fr = cache.page_table(0)
        assert list(zip(ids, fr, lens)) == sim.page_table(), t
        if t < S - 1:
            pending.append(q)
            continue
        if t == S - 1:
            q = torch.cat(pending + [q])
            pending = []
        toks = np.array(sim.attended_tokens())
        out = cache.attend(0, q.contiguous(), 0.125)
        K = attention.gather_tokens(lambda f: host[f][0].double().numpy(), toks, T)
        V = attention.gather_tokens(lambda f: host[f][1].double().numpy(), toks, T)
        ref, _ = attention.attend(to64(q), K, V, 0.125)
        assert_close(to64(out), ref, bf16=dname == "bf16", what=f"{dname} frame {t}")
    assert len(sim.special_pages) >= 2
    bits = torch.int16 if dname == "bf16" else torch.int32
    for pid, toks in sim.special_pages:
        k_pg, v_pg, id_pg = cache.page_view(0, pid)
        n = len(toks)
        fr, sl = np.array(toks) // T, np.array(toks) % T
        ek = torch.stack([host[int(a)][0][int(b)] for a, b in zip(fr, sl)]).permute(1, 0, 2).contiguous()
        ev = torch.stack([host[int(a)][1][int(b)] for a, b in zip(fr, sl)]).permute(1, 0, 2).contiguous()
        assert torch.equal(k_pg[:, :n].cpu().view(bits), ek.view(bits)), f"K of special page {pid}"
        assert torch.equal(v_pg[:, :n].cpu().view(bits), ev.view(bits)), f"V of special page {pid}"
        assert id_pg[:n].cpu().numpy().tolist() == list(toks)
    info = cache.info(0)
    assert info["special_tokens"] == sum(len(x) for _, x in sim.special_pages)
    say(f"{dname}: {len(sim.special_pages)} special pages, {info['special_tokens']} special tokens attended")
