"""The C-ABI library on the CPU: it loads, exports every declared symbol, and
its host-side policy (metadata-only pools) matches the oracle bit for bit.

No kernel runs here: a metadata-only pool (NULL device buffers) executes the
page allocation / eviction bookkeeping and refuses every device call.
"""

import ctypes
import os
import re

import numpy as np
import pytest

from bounded_kv_cache_stream_amd import kvstream as kv
from oracle import window

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kvstream.h")


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[a-z_]+\s*\*?\s*([a-z_]+)\s*\(", text, flags=re.M)))


def test_library_exports_every_declared_symbol():
    names = _declared_functions()
    assert set(names) == set(kv.EXPORTED), names
    L = kv.lib()
    for n in names:
        assert hasattr(L, n), n
        assert ctypes.cast(getattr(L, n), ctypes.c_void_p).value


def _meta_pool(S, W, k, pages, T=16, layers=1):
    cfg = kv.make_config(num_layers=layers, num_heads=2, page_tokens=T, dtype=kv.KV_FP32, scale_frames=S,
                         sliding_window=W, keyframe_interval=k, pages_per_layer=pages, max_queries=64)
    return kv.KVCache(cfg, device=None)


def test_tiny_page_tables_through_the_c_abi():
    gold = {}
    for line in open(os.path.join(ROOT, "tests", "golden", "config0_page_tables.txt")):
        line = line.strip()
        if line and not line.startswith("#"):
            t, rest = line.split(":", 1)
            gold[int(t)] = [tuple(int(x) for x in e.split(":")) for e in rest.split()]
    c = _meta_pool(1, 4, 1, 6)
    for t in range(12):
        c.append(0, t)
        c.evict(0)
        ids, lens, frames = c.page_table(0)
        assert list(zip(ids, frames)) == gold[t], t
        assert lens == [16] * len(ids)


@pytest.mark.parametrize("S,W,k,frames", [(8, 64, 4, 10000), (8, 64, 1, 200), (0, 3, 2, 300), (3, 0, 5, 120)])
def test_long_stream_metadata_matches_oracle_every_frame(S, W, k, frames):
    # Non-keyframes go to the transient page, which only an attention call
    # consumes; a metadata-only pool therefore gets the keyframes only.  The
    # persisted table must equal the oracle's after every keyframe.
    pages = S + (W if W else frames) + 1
    c = _meta_pool(S, W, k, pages, T=1004)
    sim = window.WindowCache(S, W, k, pages)
    for t in range(frames):
        if not window.is_keyframe(t, S, k):
            continue
        c.append(0, t)
        c.evict(0)
        sim.append(t)
        sim.evict()
        ids, lens, fr = c.page_table(0)
        assert ids == sim.page_ids() and fr == sim.persisted(), t
        assert fr == window.persisted_frames(t, S, W, k)
        info = c.info(0)
        assert info["persisted_frames"] == len(sim.table) and info["transient_pending"] == 0
        if W:
            assert len(ids) <= S + W


def test_pending_transient_blocks_the_next_append():
    c = _meta_pool(0, 4, 2, 6)
    c.append(0, 0)
    c.append(0, 1)  # not a keyframe -> transient
    assert c.info(0)["transient_pending"] == 1
    with pytest.raises(kv.KVError) as e:
        c.append(0, 2)
    assert e.value.status == kv.KV_ERR_STATE
    assert c.page_table(0)[2] == [0]


def test_keyframe_only_stream_long():
    # keyframe_interval 4 with every non-keyframe forced transient would need attention;
    # exercise the long-stream checkpoints with keyframes only instead.
    S, W, k = 8, 64, 4
    c = _meta_pool(S, W, 1, S + W + 1, T=1004)
    sim = window.WindowCache(S, W, 1, S + W + 1)
    for t in range(10000):
        if not window.is_keyframe(t, S, k):
            continue
        c.append(0, t)
        c.evict(0)
        sim.append(t)
        sim.evict()
    ids, _, fr = c.page_table(0)
    assert fr == window.persisted_frames(9999, S, W, k)
    assert ids == sim.page_ids()


def test_error_paths_leave_state_unchanged():
    c = _meta_pool(1, 4, 1, 5)  # needs 6 pages for the window to work
    for t in range(5):
        c.append(0, t)
    before = c.page_table(0)
    with pytest.raises(kv.KVError) as e:
        c.append(0, 5)
    assert e.value.status == kv.KV_ERR_NO_PAGES
    assert c.page_table(0) == before
    with pytest.raises(kv.KVError) as e:
        c.append(0, 3)  # frame order
    assert e.value.status == kv.KV_ERR_STATE
    with pytest.raises(kv.KVError) as e:
        kv.kv_append_frame(c.handle, 0, 6, None, None, 15, 0, None)  # wrong token count
    assert e.value.status == kv.KV_ERR_SHAPE
    with pytest.raises(kv.KVError) as e:
        c.append(1, 6)  # bad layer
    assert e.value.status == kv.KV_ERR_ARG
    with pytest.raises(kv.KVError) as e:
        kv.stream_attend(c.handle, 0, None, 16, 0.125, None, None, None)  # no device memory
    assert e.value.status == kv.KV_ERR_STATE
    assert "device memory" in kv.kv_last_error()
    assert c.page_table(0) == before
    assert kv.kv_last_error() == ""  # a successful call clears the message


def test_bad_configs_rejected():
    for bad in (dict(head_dim=32), dict(page_tokens=0), dict(keyframe_interval=0), dict(max_splits=0),
                dict(max_window=9), dict(pages_per_layer=0), dict(dtype=7)):
        cfg = kv.make_config(**bad)
        with pytest.raises(kv.KVError) as e:
            kv.kv_pool_required_bytes(cfg)
        assert e.value.status == kv.KV_ERR_ARG


def test_reset_replay_identical_and_sizes():
    c = _meta_pool(8, 64, 1, 73, T=1004)
    def run():
        out = []
        for t in range(300):
            c.append(0, t)
            c.evict(0)
            out.append(c.page_table(0))
        return out
    a = run()
    c.reset()
    assert c.page_table(0) == ([], [], [])
    assert run() == a
    info = c.info(0)
    assert info["persisted_frames"] == 72 and info["evictions"] == 300 - 72
    cfg = kv.make_config()
    lay = kv.kv_pool_get_layout(cfg)
    assert lay["token_stride"] == 1024 and lay["elem_bytes"] == 2
    assert lay["page_bytes"] == 2 * 16 * 1024 * 64 * 2 + 1024 * 4
    pool, ws = kv.kv_pool_required_bytes(cfg)
    assert pool == 74 * lay["page_bytes"]


def test_multi_layer_append_is_all_or_nothing():
    c = _meta_pool(1, 4, 1, 6, layers=3)
    for t in range(3):
        c.append_layers(0, t, n_layers=3)
    assert [c.page_table(l)[2] for l in range(3)] == [[0, 1, 2]] * 3
    c.append(2, 3)  # layer 2 is one frame ahead
    with pytest.raises(kv.KVError) as e:
        c.append_layers(0, 3, n_layers=3)
    assert e.value.status == kv.KV_ERR_STATE
    assert [c.page_table(l)[2] for l in range(2)] == [[0, 1, 2]] * 2  # no layer changed
    c.append_layers(0, 3, n_layers=2)
    assert [c.page_table(l)[2] for l in range(3)] == [[0, 1, 2, 3]] * 3
    with pytest.raises(kv.KVError) as e:
        c.append_layers(1, 4, n_layers=3)  # layers 1..3 of a 3-layer pool
    assert e.value.status == kv.KV_ERR_ARG


def test_page_merge_host_rules():
    # window pools refuse it (their pages are whole frames the window evicts);
    # in a budget pool, full pages never fit together, so nothing merges
    c = _meta_pool(1, 4, 1, 6)
    c.append(0, 0, None, None)
    with pytest.raises(kv.KVError) as e:
        c.merge_pages(0)
    assert e.value.status == kv.KV_ERR_STATE
    b = _meta_pool(0, 0, 1, 5)
    for t in range(4):
        b.append(0, t, None, None)
    assert b.merge_pages(0) == 0
    assert b.page_table(0)[1] == [16] * 4
    assert b.info(0)["merges"] == 0
    # the batched call: same rules for every layer, and a bad range changes nothing
    m = _meta_pool(0, 0, 1, 5, layers=3)
    for l in range(3):
        m.append(l, 0, None, None)
    assert m.merge_pages_layers(0, 3) == [0, 0, 0]
    with pytest.raises(kv.KVError) as e:
        m.merge_pages_layers(1, 3)
    assert e.value.status == kv.KV_ERR_ARG
    w = _meta_pool(1, 4, 1, 6, layers=2)
    with pytest.raises(kv.KVError) as e:
        w.merge_pages_layers(0, 2)
    assert e.value.status == kv.KV_ERR_STATE


def test_layer_budgets_match_oracle():
    # host arithmetic of the library against the oracle's softmax budgets; the
    # two evaluate exp with different libraries, so a floor may differ only
    # where its argument sits within rounding of an integer
    import numpy as np
    from oracle import diversity
    rng = np.random.default_rng(11)
    for _ in range(400):
        L = int(rng.integers(1, 40))
        heads = int(rng.integers(1, 33))
        tau = float(rng.uniform(0.005, 2.0))
        total = int(rng.integers(0, 10 ** 9))
        md = rng.uniform(-1.0, 0.0, L)
        got = np.array(kv.kv_layer_budgets(md, tau, total, heads))
        want = diversity.layer_budgets(md, tau, total, heads)
        d = md / tau
        p = np.exp(d - d.max())
        p = p / p.sum()
        for g, w, share in zip(got, want, p * total):
            if g != w:
                assert abs(g - w) == 1
                edge = min(abs(share - round(share)), abs(np.floor(share) / heads - round(np.floor(share) / heads)))
                assert edge < 1e-6 * max(1.0, share)
    # the explainer's worked numbers: 12 layers of equal diversity share a
    # total of 98,304 head-tokens as 512 per head of 16 heads
    gold = {}
    for ln in open(os.path.join(ROOT, "tests", "golden", "diversity_budget_example.txt")):
        if ln.strip() and not ln.startswith("#"):
            k, v = ln.split(":")
            gold[k.strip()] = int(v)
    got = kv.kv_layer_budgets([-0.25] * gold["layers"], 0.7, gold["total"], gold["heads"])
    assert got == [gold["per_head_budget"]] * gold["layers"]
    for bad in [dict(tau=0.0), dict(tau=float("nan")), dict(heads=0), dict(total=-1)]:
        a = dict(md=[-0.1, -0.2], tau=1.0, total=100, heads=2)
        a.update(bad)
        with pytest.raises(kv.KVError) as e:
            kv.kv_layer_budgets(a["md"], a["tau"], a["total"], a["heads"])
        assert e.value.status == kv.KV_ERR_ARG
    with pytest.raises(kv.KVError):
        kv.kv_layer_budgets([1.0, 0.0], 1e-310, 100, 2)  # mean / tau overflows


def test_diversity_host_rules():
    # no candidate: mean 0 without device work; every head within its budget:
    # nothing to do; otherwise a metadata-only pool refuses the device step
    c = _meta_pool(1, 0, 1, 6)
    c.append(0, 0, None, None)
    assert c.diversity_score(0) == 0.0
    assert c.diversity_prune(0, 0) == [0, 0]
    for t in range(1, 4):
        c.append(0, t, None, None)
    assert c.diversity_prune(0, 48) == [48, 48]
    assert c.diversity_prune(0, 100) == [48, 48]
    for call in (lambda: c.diversity_prune(0, 47), lambda: c.diversity_score(0)):
        with pytest.raises(kv.KVError) as e:
            call()
        assert e.value.status == kv.KV_ERR_STATE
    with pytest.raises(kv.KVError) as e:
        c.diversity_prune(0, -1)
    assert e.value.status == kv.KV_ERR_ARG
    assert c.head_lengths(0) == [[16, 16]] * 4
    assert c.info(0)["prunes"] == 0
    # batched forms: range checks, and the same host rules per layer
    m = _meta_pool(1, 0, 1, 6, layers=3)
    assert m.diversity_score_layers(0, 3) == [0.0, 0.0, 0.0]
    m.append(1, 0, None, None)
    m.append(1, 1, None, None)
    assert m.diversity_prune_layers(0, [5, 16, 0]) == [[0, 0], [16, 16], [0, 0]]
    out = np.full((3, 2), -1, dtype=np.int64)
    assert m.diversity_prune_layers(0, [5, 16, 0], out=out) is out and out.tolist() == [[0, 0], [16, 16], [0, 0]]
    with pytest.raises(ValueError):
        m.diversity_prune_layers(0, [5, 16, 0], out=np.zeros((3, 2), dtype=np.int32))
    for call in (lambda: m.diversity_prune_layers(1, [5, 5]), lambda: m.diversity_score_layers(0, 3)):
        with pytest.raises(kv.KVError) as e:
            call()
        assert e.value.status == kv.KV_ERR_STATE
    for call in (lambda: m.diversity_score_layers(1, 3), lambda: m.diversity_prune_layers(2, [1, 1]),
                 lambda: m.diversity_score_layers(0, 0), lambda: m.diversity_prune_layers(0, [1, -1])):
        with pytest.raises(kv.KVError) as e:
            call()
        assert e.value.status == kv.KV_ERR_ARG


@pytest.mark.parametrize("S,W,k,T,sp,frames", [(1, 2, 1, 4, 1, 8), (8, 64, 4, 1004, 5, 3000), (0, 3, 2, 16, 5, 200),
                                             (2, 5, 1, 12, 12, 60), (1, 4, 3, 10, 3, 400)])
def test_special_tokens_page_tables_match_oracle(S, W, k, T, sp, frames):
    # window eviction with special-token persistence through the C ABI, frame
    # by frame: page ids, frame ids (-1 - f for a special page), lengths,
    # free count and the special counters equal the oracle's
    n_special = (frames * sp + (T // sp) * sp - 1) // ((T // sp) * sp) + 1
    pages = S + W + 1 + n_special
    cfg = kv.make_config(num_layers=1, num_heads=2, page_tokens=T, dtype=kv.KV_FP32, scale_frames=S,
                         sliding_window=W, keyframe_interval=k, pages_per_layer=pages, max_queries=64,
                         special_tokens=sp)
    c = kv.KVCache(cfg, device=None)
    sim = window.SpecialWindowCache(S, W, k, pages, special=sp, tokens_per_frame=T)
    for t in range(frames):
        if not window.is_keyframe(t, S, k):
            continue  # a metadata-only pool cannot consume a transient frame (no attention)
        c.append(0, t)
        sim.append(t)
        assert c.evict(0) == sim.evict()
        ids, lens, fr = c.page_table(0)
        assert list(zip(ids, fr, lens)) == sim.page_table(), t
        info = c.info(0)
        assert info["special_pages"] == len(sim.special_pages)
        assert info["special_tokens"] == sum(len(x) for _, x in sim.special_pages)
        assert info["pages_free"] == len(sim.free)
        assert info["persisted_frames"] == len(sim.table)
    assert len(sim.special_pages) > 0


def test_special_tokens_need_a_free_page():
    # no id left for a special page: the eviction fails and nothing changes
    cfg = kv.make_config(num_layers=1, num_heads=2, page_tokens=4, dtype=kv.KV_FP32, scale_frames=1,
                         sliding_window=2, keyframe_interval=1, pages_per_layer=4, max_queries=8, special_tokens=1)
    c = kv.KVCache(cfg, device=None)
    for t in range(3):
        c.append(0, t)
        c.evict(0)
    c.append(0, 3)
    before = c.page_table(0)
    with pytest.raises(kv.KVError) as e:
        c.evict(0)
    assert e.value.status == kv.KV_ERR_NO_PAGES
    assert c.page_table(0) == before
    for bad in (-1, 5):
        with pytest.raises(kv.KVError):
            kv.KVCache(kv.make_config(page_tokens=4, special_tokens=bad), device=None)
    # compaction and pruning would move the special tokens out of the first
    # slots: a pool with special tokens refuses both
    for call in (lambda: kv.score_and_compact(c.handle, 0, None, 1, 5, 0.5, 1), lambda: c.diversity_prune(0, 1)):
        with pytest.raises(kv.KVError) as e:
            call()
        assert e.value.status == kv.KV_ERR_STATE


def test_append_attend_checks_before_changing_anything():
    # kv_append_attend validates every argument first: a metadata-only pool has
    # no device memory to attend with, and a frame of the wrong size is refused;
    # either way the layer is left as it was
    c = _meta_pool(1, 4, 1, 6)
    c.append(0, 0)
    c.evict(0)
    before = (c.page_table(0), c.info(0))
    with pytest.raises(kv.KVError) as e:
        kv.kv_append_attend(c.handle, 0, 1, None, None, 16, 0, None, 16, 1.0, None)
    assert e.value.status == kv.KV_ERR_STATE
    with pytest.raises(kv.KVError) as e:
        kv.kv_append_attend(c.handle, 0, 1, None, None, 15, 0, None, 16, 1.0, None)
    assert e.value.status == kv.KV_ERR_SHAPE
    with pytest.raises(kv.KVError) as e:
        kv.kv_append_attend(c.handle, 0, 1, None, None, 16, 0, None, 65, 1.0, None)
    assert e.value.status == kv.KV_ERR_SHAPE
    assert (c.page_table(0), c.info(0)) == before


def test_clces_flags_and_sync_on_a_metadata_pool():
    # unknown flag bits are refused before anything else; kv_sync is a no-op where nothing is pending
    c = _meta_pool(0, 0, 1, 5)
    for t in range(3):
        c.append(0, t, None, None)
    prm = kv.kv_clces_params(5, 8, 0.5, 10)
    n = ctypes.c_int64()
    st = kv.lib().score_and_compact(c.handle, 0, None, 0, ctypes.byref(prm), None, None, ctypes.byref(n), None)
    assert st == kv.KV_ERR_ARG and "flags" in kv.kv_last_error()
    kv.kv_sync(c.handle, -1)
    kv.kv_sync(c.handle, 0)
    with pytest.raises(kv.KVError):
        kv.kv_sync(c.handle, 1)
    assert c.page_table(0)[1] == [16] * 3


def test_attend_tiling_values():
    # the three tilings are accepted, anything else refused
    c = _meta_pool(0, 0, 1, 5)
    for tiling in (kv.KV_TILING_AUTO, kv.KV_TILING_PAGE, kv.KV_TILING_PACKED):
        kv.kv_set_attend_tiling(c.handle, tiling)
    for bad in (-1, 3):
        with pytest.raises(kv.KVError) as e:
            kv.kv_set_attend_tiling(c.handle, bad)
        assert e.value.status == kv.KV_ERR_ARG


def test_attend_timing_arguments_on_a_metadata_pool():
    # timing off (0 calls) needs no device; bad counts and NULL pools are refused
    c = _meta_pool(0, 0, 1, 5)
    kv.kv_attend_timing(c.handle, 0)
    assert kv.kv_attend_timing_read(c.handle) == (0.0, 0)
    for bad in (-1, (1 << 20) + 1):
        with pytest.raises(kv.KVError) as e:
            kv.kv_attend_timing(c.handle, bad)
        assert e.value.status == kv.KV_ERR_ARG
    assert kv.lib().kv_attend_timing(None, 1) == kv.KV_ERR_ARG
    assert kv.lib().kv_attend_timing_read(c.handle, None, None) == kv.KV_ERR_ARG
