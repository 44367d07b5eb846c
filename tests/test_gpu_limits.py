"""The path at the edges of its sizes, against the oracle.

- The largest page the library takes (8192 tokens, also the ceiling of the CLCES and diversity kernels):
  a window stream, a CLCES step and a diversity prune.
- One-token pages: a window stream with transient frames, and a token-budget stream whose compaction
  empties pages.
- A single query row, and a query count one past a 256-row workgroup tile.
- An fp32 pool with pages of several tiles and a ragged tail.
"""

import numpy as np
import pytest

from bounded_kv_cache_stream_amd import kvstream as kv
from bounded_kv_cache_stream_amd import synth
from oracle import attention, budget, window
from tests.gpu_common import LSE_ABS_BF16, LSE_ABS_FP32, assert_close, max_abs, say, to64, torch_cuda
from tests.test_gpu_clces import _page_bytes_equal
from tests.test_gpu_diversity import Stream as DivStream

pytestmark = pytest.mark.gpu


def _window_cfg(T, H, S, W, k, pages, max_queries, max_splits=16, dtype=kv.KV_BF16):
    return kv.make_config(num_layers=1, num_heads=H, page_tokens=T, scale_frames=S, sliding_window=W, dtype=dtype,
                          keyframe_interval=k, pages_per_layer=pages, max_queries=max_queries, max_splits=max_splits)


def _window_stream(T, H, S, W, k, frames, rows, wid, tau=0.125, fp32=False):
    """append -> evict -> attend for `frames` frames; every frame's output rows `rows` (or all) against the
    oracle over the frames the policy attends."""
    torch = torch_cuda()
    dt = kv.KV_FP32 if fp32 else kv.KV_BF16
    c = kv.KVCache(_window_cfg(T, H, S, W, k, S + W + 1, max(S, 1) * T, dtype=dt), device="cuda")
    host = {}
    pending = []
    rng = np.random.default_rng(wid)
    for t in range(frames):
        q, kk, vv = synth.iid_frame(wid, 0, t, (T, H, 64), device="cuda",
                                    dtype=torch.float32 if fp32 else torch.bfloat16)
        host[t] = (kk.double().cpu().numpy(), vv.double().cpu().numpy())
        c.append(0, t, kk, vv)
        c.evict(0)
        if t < S - 1:
            pending.append(q)
            continue
        if t == S - 1 and pending:
            q = torch.cat(pending + [q])
        lse = torch.empty(q.shape[0] * H, dtype=torch.float32, device="cuda")
        out = c.attend(0, q, tau, lse=lse)
        att = window.attended_frames(t, S, W, k)
        assert c.page_table(0)[2] == window.persisted_frames(t, S, W, k), t
        sel = slice(None) if rows is None else np.sort(rng.choice(q.shape[0], min(rows, q.shape[0]), replace=False))
        K = np.concatenate([host[f][0] for f in att])
        V = np.concatenate([host[f][1] for f in att])
        ref, ref_lse = attention.attend(to64(q)[sel], K, V, tau)
        ma, rl = assert_close(to64(out)[sel], ref, bf16=not fp32, what=f"T={T} frame {t}")
        assert max_abs(to64(lse).reshape(-1, H)[sel], ref_lse) <= (LSE_ABS_FP32 if fp32 else LSE_ABS_BF16), t
    return c, host


def test_largest_page_window_stream():
    torch = torch_cuda()
    T, H = 8192, 2
    c, host = _window_stream(T, H, 1, 2, 1, 5, 64, wid=70)
    # the newest page holds the frame as [H][T][D], bit for bit
    ids, lens, frames = c.page_table(0)
    assert lens == [T] * len(ids)
    k, v, pid = c.page_view(0, ids[-1])
    f = frames[-1]
    assert np.array_equal(k.float().cpu().numpy(), host[f][0].transpose(1, 0, 2))
    assert np.array_equal(v.float().cpu().numpy(), host[f][1].transpose(1, 0, 2))
    assert pid.cpu().numpy().tolist() == [f * T + i for i in range(T)]
    say("8192-token pages: window stream matches the oracle")


def test_largest_page_clces_step():
    torch = torch_cuda()
    T, H, L, F, K = 8192, 2, 2, 3, 10000
    cfg = kv.make_config(num_layers=L, num_heads=H, page_tokens=T, scale_frames=0, sliding_window=0,
                         keyframe_interval=1, pages_per_layer=F + 1, max_queries=T, max_splits=8, max_window=5)
    c = kv.KVCache(cfg, device="cuda")
    host = {}
    for t in range(F):
        _, kk, vv = synth.iid_frame(71, 1, t, (T, H, 64), device="cuda", dtype=torch.bfloat16)
        c.append(1, t, kk, vv)
        host[t] = (kk.cpu(), vv.cpu())
    scores = synth.raw_scores(71, F * T, L)
    keep = torch.empty(K, dtype=torch.int32, device="cuda")
    ranks = torch.empty((2, F * T), dtype=torch.int32, device="cuda")
    assert c.score_and_compact(1, torch.from_numpy(scores).cuda(), 5, 0.5, K, keep_ids=keep, ranks=ranks) == K
    b = budget.BudgetCache(1, T, K, F + 1)
    for t in range(F):
        b.append(t)
    assert b.score_and_compact(scores)
    assert ranks.cpu().numpy().tolist() == b.last["ranks"].tolist()
    assert keep.cpu().numpy().tolist() == b.last["keep_ids"].tolist()
    ids, lens, frames = c.page_table(1)
    assert list(zip(ids, frames, lens)) == b.page_table()
    for pid, f, tok in b.table:
        fr, sl = tok // T, tok % T
        k_rows = torch.stack([host[int(a)][0][int(s)] for a, s in zip(fr, sl)])
        v_rows = torch.stack([host[int(a)][1][int(s)] for a, s in zip(fr, sl)])
        _page_bytes_equal(c, 1, pid, len(tok), k_rows, v_rows, tok.tolist())
    say("8192-token pages: CLCES ranks, keep set and compacted bytes match the oracle")


def test_largest_page_diversity_prune():
    torch = torch_cuda()
    T, H, F = 8192, 2, 4
    cfg = kv.make_config(num_layers=1, num_heads=H, page_tokens=T, scale_frames=1, sliding_window=0,
                         keyframe_interval=1, pages_per_layer=F + 1, max_queries=T, max_splits=8, max_window=5)
    c = kv.KVCache(cfg, device="cuda")
    s = DivStream(c, T, H, F + 1, wid=72)
    for t in range(F):
        s.append(t)
    assert c.diversity_prune(0, 9000) == [9000] * H
    s.prune(9000)
    s.check_pages("8192-token pages, prune")
    q = synth.iid_frame(73, 0, 0, (32, H, 64), device="cuda", dtype=torch.bfloat16)[0]
    s.check_attention(q, 0.125, "8192-token pages, attention after the prune")
    say("8192-token pages: diversity prune matches the oracle")


def test_fp32_multi_tile_pages_window_stream():
    # fp32 pool, 200-token pages (several 64-token tiles and a ragged tail), 3 heads, two scale frames attended
    # jointly, keyframe interval 2 (every other frame transient): every row of every frame
    _window_stream(200, 3, 2, 3, 2, 12, None, wid=78, fp32=True)
    say("fp32 200-token pages: window stream matches the oracle")


def test_one_token_pages_window_stream():
    # every frame is one token: each tile holds one valid key; keyframe interval 2 makes every other frame
    # transient
    _window_stream(1, 2, 1, 3, 2, 14, None, wid=74)


def test_shared_table_past_the_inline_limit():
    # a shared bf16 table rides in the attention kernel's arguments up to 192 entries and is uploaded beyond:
    # 4-token frames under a 200-frame window grow the table from 1 to 201 entries, crossing 192 at frame 192;
    # every row of every frame against the oracle
    _window_stream(4, 2, 1, 200, 1, 205, None, wid=79)
    say("shared table of up to 201 entries: window stream matches the oracle on both sides of 192")


def test_one_token_pages_budget_stream():
    # one-token pages under a 5-token budget: each step empties a page (its id is released) and the cache
    # stays at 5 pages
    torch = torch_cuda()
    T, H, F, B = 1, 2, 12, 5
    cfg = kv.make_config(num_layers=1, num_heads=H, page_tokens=T, scale_frames=0, sliding_window=0,
                         keyframe_interval=1, pages_per_layer=B + 2, max_queries=T, max_splits=4, max_window=5)
    c = kv.KVCache(cfg, device="cuda")
    b = budget.BudgetCache(0, T, B, B + 2)
    scores = synth.raw_scores(75, F * T, 1)
    table = torch.from_numpy(scores).cuda()
    host = {}
    for t in range(F):
        q, kk, vv = synth.iid_frame(75, 0, t, (T, H, 64), device="cuda", dtype=torch.bfloat16)
        host[t] = (kk.double().cpu().numpy(), vv.double().cpu().numpy())
        c.append(0, t, kk, vv)
        b.append(t)
        out = c.attend(0, q, 0.125)
        ids = b.all_ids()
        K = np.concatenate([host[int(i)][0] for i in ids])
        V = np.concatenate([host[int(i)][1] for i in ids])
        ref, _ = attention.attend(to64(q), K, V, 0.125)
        assert_close(to64(out), ref, bf16=True, what=f"one-token budget frame {t}")
        n = c.score_and_compact(0, table, 5, 0.5, B)
        b.score_and_compact(scores)
        assert n == min(B, t + 1)
        ids_, lens, frames = c.page_table(0)
        assert list(zip(ids_, frames, lens)) == b.page_table(), t
    assert c.info(0)["pages_used"] == B


def test_single_query_row_and_ragged_query_tiles():
    torch = torch_cuda()
    T, H, F = 1004, 16, 10
    c = kv.KVCache(_window_cfg(T, H, 1, 64, 1, 66, 512), device="cuda")
    host = {}
    for t in range(F):
        _, kk, vv = synth.iid_frame(76, 0, t, (T, H, 64), device="cuda", dtype=torch.bfloat16)
        c.append(0, t, kk, vv)
        c.evict(0)
        host[t] = (kk.double().cpu().numpy(), vv.double().cpu().numpy())
    K = np.concatenate([host[f][0] for f in range(F)])
    V = np.concatenate([host[f][1] for f in range(F)])
    q = synth.iid_frame(77, 0, 0, (512, H, 64), device="cuda", dtype=torch.bfloat16)[0] * 0.125
    for n_q in (1, 257):
        qq = q[:n_q].contiguous()
        for splits in (0, 1, 7):
            c.set_splits(splits)
            out = c.attend(0, qq, 1.0)
            ref, _ = attention.attend(to64(qq), K, V, 1.0)
            assert_close(to64(out), ref, bf16=True, what=f"n_q {n_q}, splits {splits}")
