"""ctypes binding of ``libkvstream.so`` (C ABI declared in include/kvstream.h).

Argument marshalling only: every step of the path runs in the library's HIP
kernels.  The functions below carry the C names; ``KVCache`` adds PyTorch
plumbing (device buffers, the current stream, tensor checks).  Loading fails
loudly when the library has not been built -- there is no fallback.
"""

from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
# KVSTREAM_LIB: another build of the same library (the host-sanitized one of build.py)
LIB_PATH = os.environ.get("KVSTREAM_LIB") or os.path.join(_HERE, "libkvstream.so")

KV_OK, KV_ERR_ARG, KV_ERR_SHAPE, KV_ERR_NO_PAGES, KV_ERR_STATE, KV_ERR_HIP, KV_ERR_NAN = 0, -1, -2, -3, -4, -5, -6
KV_CLCES_DEFER = 1
KV_CLCES_REUSE_RANKS = 2
KV_CLCES_RANK_RADIX = 4
KV_BF16, KV_FP32 = 0, 1
KV_TRANSIENT = 1

EXPORTED = (
    "kv_pool_required_bytes", "kv_pool_get_layout", "kv_pool_create", "kv_pool_destroy", "kv_reset",
    "kv_append_frame", "kv_append_frame_layers", "kv_evict", "stream_attend", "stream_attend_scratch",
    "kv_append_attend", "score_and_compact",
    "kv_get_info", "kv_get_page_table", "kv_set_attend_splits", "kv_set_attend_tiling", "kv_merge_pages", "kv_merge_pages_layers",
    "kv_diversity_score",
    "kv_diversity_score_layers", "kv_layer_budgets", "kv_diversity_prune", "kv_diversity_prune_layers",
    "kv_get_head_lengths", "kv_sync", "kv_attend_timing", "kv_attend_timing_read", "kv_last_error",
)


class kv_pool_config(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "num_layers", "num_heads", "head_dim", "page_tokens", "dtype", "scale_frames", "sliding_window",
        "keyframe_interval", "pages_per_layer", "max_queries", "max_splits", "max_window", "special_tokens")]


class kv_clces_params(ctypes.Structure):
    _fields_ = [("window", ctypes.c_int32), ("flags", ctypes.c_uint32), ("lambda_", ctypes.c_double),
                ("keep_count", ctypes.c_int64), ("s_hat_out", ctypes.c_void_p)]


class kv_cache_info(ctypes.Structure):
    _fields_ = [("persisted_frames", ctypes.c_int32), ("pages_used", ctypes.c_int32),
                ("pages_free", ctypes.c_int32), ("transient_pending", ctypes.c_int32),
                ("tokens", ctypes.c_int64), ("bytes", ctypes.c_int64), ("evictions", ctypes.c_int64),
                ("compactions", ctypes.c_int64), ("last_keep_count", ctypes.c_int64), ("merges", ctypes.c_int64),
                ("prunes", ctypes.c_int64), ("special_pages", ctypes.c_int64), ("special_tokens", ctypes.c_int64)]


class kv_pool_layout(ctypes.Structure):
    _fields_ = [("page_bytes", ctypes.c_int64), ("k_offset", ctypes.c_int64), ("v_offset", ctypes.c_int64),
                ("id_offset", ctypes.c_int64), ("token_stride", ctypes.c_int32), ("elem_bytes", ctypes.c_int32)]


class KVError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"kvstream status {status}: {message}")
        self.status = status


_lib = None


def lib() -> ctypes.CDLL:
    """The loaded library; raises if it is not built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m bounded_kv_cache_stream_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        P, I32, I64, SZ, U32, F32 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t, ctypes.c_uint32, ctypes.c_float
        cfgp = ctypes.POINTER(kv_pool_config)
        sig = {
            "kv_pool_required_bytes": [cfgp, ctypes.POINTER(SZ), ctypes.POINTER(SZ)],
            "kv_pool_get_layout": [cfgp, ctypes.POINTER(kv_pool_layout)],
            "kv_pool_create": [cfgp, P, SZ, P, SZ, ctypes.POINTER(P)],
            "kv_pool_destroy": [P],
            "kv_reset": [P],
            "kv_append_frame": [P, I32, I64, P, P, I32, U32, P],
            "kv_append_frame_layers": [P, I32, I32, I64, P, P, I32, U32, P],
            "kv_evict": [P, I32, ctypes.POINTER(I32), P],
            "stream_attend": [P, I32, P, I32, F32, P, P, P],
            "stream_attend_scratch": [P, I32, P, I32, F32, P, P, P],
            "kv_append_attend": [P, I32, I64, P, P, I32, U32, P, I32, F32, P, P, ctypes.POINTER(I32), P],
            "score_and_compact": [P, I32, P, I64, ctypes.POINTER(kv_clces_params), P, P, ctypes.POINTER(I64), P],
            "kv_get_info": [P, I32, ctypes.POINTER(kv_cache_info)],
            "kv_get_page_table": [P, I32, P, P, P, I32, ctypes.POINTER(I32)],
            "kv_set_attend_splits": [P, I32],
            "kv_set_attend_tiling": [P, I32],
            "kv_merge_pages": [P, I32, ctypes.POINTER(I32), P],
            "kv_merge_pages_layers": [P, I32, I32, ctypes.POINTER(I32), P],
            "kv_diversity_score": [P, I32, P, I64, ctypes.POINTER(ctypes.c_double), P],
            "kv_layer_budgets": [ctypes.POINTER(ctypes.c_double), I32, ctypes.c_double, I64, I32,
                                 ctypes.POINTER(I64)],
            "kv_diversity_prune": [P, I32, I64, P, I64, ctypes.POINTER(I64), P],
            "kv_diversity_score_layers": [P, I32, I32, ctypes.POINTER(ctypes.c_double), P],
            "kv_diversity_prune_layers": [P, I32, I32, ctypes.POINTER(I64), ctypes.POINTER(I64), P],
            "kv_get_head_lengths": [P, I32, P, I32, ctypes.POINTER(I32)],
            "kv_sync": [P, I32],
            "kv_attend_timing": [P, I32],
            "kv_attend_timing_read": [P, ctypes.POINTER(ctypes.c_double), ctypes.POINTER(I32)],
        }
        for name, args in sig.items():
            fn = getattr(L, name)
            fn.argtypes = args
            fn.restype = ctypes.c_int
        L.kv_last_error.argtypes = []
        L.kv_last_error.restype = ctypes.c_char_p
        _lib = L
    return _lib


def kv_last_error() -> str:
    return lib().kv_last_error().decode()


def _check(status: int) -> None:
    if status != KV_OK:
        raise KVError(status, kv_last_error())


def make_config(num_layers=1, num_heads=16, head_dim=64, page_tokens=1004, dtype=KV_BF16, scale_frames=8,
                sliding_window=64, keyframe_interval=1, pages_per_layer=73, max_queries=8032, max_splits=16,
                max_window=5, special_tokens=0) -> kv_pool_config:
    return kv_pool_config(num_layers, num_heads, head_dim, page_tokens, dtype, scale_frames, sliding_window,
                          keyframe_interval, pages_per_layer, max_queries, max_splits, max_window, special_tokens)


def kv_pool_required_bytes(cfg: kv_pool_config) -> tuple[int, int]:
    a, b = ctypes.c_size_t(), ctypes.c_size_t()
    _check(lib().kv_pool_required_bytes(ctypes.byref(cfg), ctypes.byref(a), ctypes.byref(b)))
    return a.value, b.value


def kv_pool_get_layout(cfg: kv_pool_config) -> dict:
    out = kv_pool_layout()
    _check(lib().kv_pool_get_layout(ctypes.byref(cfg), ctypes.byref(out)))
    return {f: getattr(out, f) for f, _ in out._fields_}


def kv_pool_create(cfg, pool_ptr, pool_bytes, ws_ptr, ws_bytes) -> ctypes.c_void_p:
    h = ctypes.c_void_p()
    _check(lib().kv_pool_create(ctypes.byref(cfg), pool_ptr, pool_bytes, ws_ptr, ws_bytes, ctypes.byref(h)))
    return h


def kv_pool_destroy(pool) -> None:
    _check(lib().kv_pool_destroy(pool))


def kv_reset(pool) -> None:
    _check(lib().kv_reset(pool))


def kv_append_frame(pool, layer, frame_idx, k_ptr, v_ptr, n_tokens, flags=0, stream=None) -> None:
    _check(lib().kv_append_frame(pool, layer, frame_idx, k_ptr, v_ptr, n_tokens, flags, stream))


def kv_append_frame_layers(pool, first_layer, n_layers, frame_idx, k_ptr, v_ptr, n_tokens, flags=0,
                           stream=None) -> None:
    _check(lib().kv_append_frame_layers(pool, first_layer, n_layers, frame_idx, k_ptr, v_ptr, n_tokens, flags,
                                        stream))


def kv_evict(pool, layer, stream=None) -> int:
    n = ctypes.c_int32()
    _check(lib().kv_evict(pool, layer, ctypes.byref(n), stream))
    return n.value


def stream_attend(pool, layer, q_ptr, n_q, sm_scale, out_ptr, lse_ptr=None, stream=None) -> None:
    _check(lib().stream_attend(pool, layer, q_ptr, n_q, sm_scale, out_ptr, lse_ptr, stream))


def stream_attend_scratch(pool, layer, q_ptr, n_q, sm_scale, out_ptr, lse_ptr=None, stream=None) -> None:
    _check(lib().stream_attend_scratch(pool, layer, q_ptr, n_q, sm_scale, out_ptr, lse_ptr, stream))


def kv_append_attend(pool, layer, frame_idx, k_ptr, v_ptr, n_tokens, flags, q_ptr, n_q, sm_scale, out_ptr,
                     lse_ptr=None, stream=None) -> int:
    n = ctypes.c_int32()
    _check(lib().kv_append_attend(pool, layer, frame_idx, k_ptr, v_ptr, n_tokens, flags, q_ptr, n_q, sm_scale,
                                  out_ptr, lse_ptr, ctypes.byref(n), stream))
    return n.value


def score_and_compact(pool, layer, table_ptr, score_rows, window, lam, keep_count, keep_ids_ptr=None,
                      ranks_ptr=None, stream=None, defer=False, reuse_ranks=False, s_hat_ptr=None,
                      rank_radix=False) -> int:
    flags = (KV_CLCES_DEFER if defer else 0) | (KV_CLCES_REUSE_RANKS if reuse_ranks else 0) \
        | (KV_CLCES_RANK_RADIX if rank_radix else 0)
    prm = kv_clces_params(window, flags, lam, keep_count, s_hat_ptr)
    n = ctypes.c_int64()
    _check(lib().score_and_compact(pool, layer, table_ptr, score_rows, ctypes.byref(prm), keep_ids_ptr, ranks_ptr,
                                   ctypes.byref(n), stream))
    return n.value


def kv_attend_timing(pool, max_calls) -> None:
    _check(lib().kv_attend_timing(pool, max_calls))


def kv_attend_timing_read(pool) -> tuple:
    """(sum of the timed attention kernels in ms, number of calls timed)."""
    ms = ctypes.c_double()
    n = ctypes.c_int32()
    _check(lib().kv_attend_timing_read(pool, ctypes.byref(ms), ctypes.byref(n)))
    return ms.value, n.value


def kv_sync(pool, layer=-1) -> None:
    _check(lib().kv_sync(pool, layer))


def kv_merge_pages(pool, layer, stream=None) -> int:
    n = ctypes.c_int32()
    _check(lib().kv_merge_pages(pool, layer, ctypes.byref(n), stream))
    return n.value


def kv_merge_pages_layers(pool, first_layer, n_layers, stream=None) -> list:
    n = (ctypes.c_int32 * n_layers)()
    _check(lib().kv_merge_pages_layers(pool, first_layer, n_layers, n, stream))
    return list(n)


def kv_diversity_score(pool, layer, scores_ptr=None, score_stride=0, stream=None) -> float:
    m = ctypes.c_double()
    _check(lib().kv_diversity_score(pool, layer, scores_ptr, score_stride, ctypes.byref(m), stream))
    return m.value


def kv_layer_budgets(mean_diversity, tau, total_tokens, heads) -> list:
    n = len(mean_diversity)
    md = (ctypes.c_double * max(n, 1))(*[float(x) for x in mean_diversity])
    out = (ctypes.c_int64 * max(n, 1))()
    _check(lib().kv_layer_budgets(md, n, float(tau), int(total_tokens), int(heads), out))
    return list(out[:n])


def kv_diversity_prune(pool, layer, keep_per_head, heads, scores_ptr=None, score_stride=0, stream=None) -> list:
    kept = (ctypes.c_int64 * heads)()
    _check(lib().kv_diversity_prune(pool, layer, keep_per_head, scores_ptr, score_stride, kept, stream))
    return list(kept)


def kv_diversity_score_layers(pool, first_layer, n_layers, stream=None) -> list:
    out = (ctypes.c_double * n_layers)()
    _check(lib().kv_diversity_score_layers(pool, first_layer, n_layers, out, stream))
    return list(out)


def kv_diversity_prune_layers(pool, first_layer, keep_per_head, heads, stream=None, out=None):
    """Kept candidates per layer and head: a list of lists, or written into `out` (a C-contiguous int64 numpy
    array of n x heads, returned) without building Python lists."""
    n = len(keep_per_head)
    keep = (ctypes.c_int64 * max(n, 1))(*[int(k) for k in keep_per_head])
    if out is not None:
        if out.dtype.name != "int64" or out.size != n * heads or not out.flags["C_CONTIGUOUS"]:
            raise ValueError("out must be a C-contiguous int64 array of len(keep_per_head) x heads")
        _check(lib().kv_diversity_prune_layers(pool, first_layer, n, keep,
                                               out.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)), stream))
        return out
    kept = (ctypes.c_int64 * max(n * heads, 1))()
    _check(lib().kv_diversity_prune_layers(pool, first_layer, n, keep, kept, stream))
    return [list(kept[i * heads:(i + 1) * heads]) for i in range(n)]


def kv_get_head_lengths(pool, layer, heads) -> list:
    n = ctypes.c_int32()
    _check(lib().kv_get_head_lengths(pool, layer, None, 0, ctypes.byref(n)))
    cap = n.value
    buf = (ctypes.c_int32 * max(cap * heads, 1))()
    _check(lib().kv_get_head_lengths(pool, layer, buf, cap, ctypes.byref(n)))
    return [list(buf[i * heads:(i + 1) * heads]) for i in range(cap)]


def kv_get_info(pool, layer) -> dict:
    out = kv_cache_info()
    _check(lib().kv_get_info(pool, layer, ctypes.byref(out)))
    return {f: getattr(out, f) for f, _ in out._fields_}


def kv_get_page_table(pool, layer) -> tuple[list, list, list]:
    n = ctypes.c_int32()
    _check(lib().kv_get_page_table(pool, layer, None, None, None, 0, ctypes.byref(n)))
    cap = n.value
    ids = (ctypes.c_int32 * max(cap, 1))()
    lens = (ctypes.c_int32 * max(cap, 1))()
    frames = (ctypes.c_int64 * max(cap, 1))()
    _check(lib().kv_get_page_table(pool, layer, ids, lens, frames, cap, ctypes.byref(n)))
    return list(ids[:cap]), list(lens[:cap]), list(frames[:cap])


def kv_set_attend_splits(pool, splits: int) -> None:
    _check(lib().kv_set_attend_splits(pool, splits))


KV_TILING_AUTO, KV_TILING_PAGE, KV_TILING_PACKED = 0, 1, 2


def kv_set_attend_tiling(pool, tiling: int) -> None:
    _check(lib().kv_set_attend_tiling(pool, tiling))


class KVCache:
    """A pool with its device buffers allocated by PyTorch (``device=None``: metadata only)."""

    def __init__(self, cfg: kv_pool_config, device=None):
        self.cfg = cfg
        self.layout = kv_pool_get_layout(cfg)
        self.pool_bytes, self.ws_bytes = kv_pool_required_bytes(cfg)
        self.device = device
        self.pool_buf = self.ws_buf = None
        if device is None:
            self.handle = kv_pool_create(cfg, None, 0, None, 0)
        else:
            import torch
            self.torch = torch
            self.pool_buf = torch.empty(self.pool_bytes + 256, dtype=torch.uint8, device=device)
            self.ws_buf = torch.empty(self.ws_bytes + 256, dtype=torch.uint8, device=device)
            self.pool_ptr = (self.pool_buf.data_ptr() + 255) // 256 * 256
            self.ws_ptr = (self.ws_buf.data_ptr() + 255) // 256 * 256
            self.handle = kv_pool_create(cfg, self.pool_ptr, self.pool_bytes, self.ws_ptr, self.ws_bytes)
        self.dtype_name = "bf16" if cfg.dtype == KV_BF16 else "fp32"

    def close(self):
        if getattr(self, "handle", None) is not None:
            kv_pool_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    # -- marshalling helpers -------------------------------------------------
    def _stream(self):
        if self.device is None:
            return None
        return ctypes.c_void_p(self.torch.cuda.current_stream(self.device).cuda_stream)

    def _tensor(self, t, rows=None):
        torch = self.torch
        want = torch.bfloat16 if self.cfg.dtype == KV_BF16 else torch.float32
        if t.dtype != want or not t.is_contiguous() or t.device.type != "cuda":
            raise ValueError(f"expected a contiguous {want} CUDA tensor, got {t.dtype} on {t.device}")
        if t.dim() != 3 or t.shape[1] != self.cfg.num_heads or t.shape[2] != self.cfg.head_dim:
            raise ValueError(f"expected [n, {self.cfg.num_heads}, {self.cfg.head_dim}], got {tuple(t.shape)}")
        if rows is not None and t.shape[0] != rows:
            raise ValueError(f"expected {rows} rows, got {t.shape[0]}")
        return ctypes.c_void_p(t.data_ptr())

    # -- the C calls -----------------------------------------------------------
    def append(self, layer, frame_idx, k=None, v=None, transient=False):
        flags = KV_TRANSIENT if transient else 0
        if self.device is None:
            kv_append_frame(self.handle, layer, frame_idx, None, None, self.cfg.page_tokens, flags, None)
            return
        kv_append_frame(self.handle, layer, frame_idx, self._tensor(k), self._tensor(v, k.shape[0]), k.shape[0],
                        flags, self._stream())

    def append_layers(self, first_layer, frame_idx, k=None, v=None, n_layers=None, transient=False):
        """k, v: [n_layers, T, H, D] contiguous (one frame of several layers)."""
        flags = KV_TRANSIENT if transient else 0
        if self.device is None:
            kv_append_frame_layers(self.handle, first_layer, n_layers, frame_idx, None, None, self.cfg.page_tokens,
                                   flags, None)
            return
        if k.dim() != 4 or k.shape != v.shape:
            raise ValueError("k and v must be [n_layers, T, H, D] tensors of the same shape")
        self._tensor(k[0])
        if not (k.is_contiguous() and v.is_contiguous()):
            raise ValueError("k and v must be contiguous")
        kv_append_frame_layers(self.handle, first_layer, k.shape[0], frame_idx, ctypes.c_void_p(k.data_ptr()),
                               ctypes.c_void_p(v.data_ptr()), k.shape[1], flags, self._stream())

    def evict(self, layer) -> int:
        # device work (and so a stream) only when special tokens persist
        return kv_evict(self.handle, layer, self._stream() if self.cfg.special_tokens else None)

    def attend(self, layer, q, sm_scale, out=None, lse=None, static_scratch=False):
        """stream_attend (static_scratch: stream_attend_scratch, the allocation-free variant; out must then
        be given for the call to allocate nothing)."""
        torch = self.torch
        if out is None:
            out = torch.empty_like(q)
        qp = self._tensor(q)
        op = self._tensor(out, q.shape[0])
        lp = None
        if lse is not None:
            if lse.dtype != torch.float32 or not lse.is_contiguous() or lse.numel() != q.shape[0] * q.shape[1]:
                raise ValueError("lse must be a contiguous fp32 tensor of n_q * H elements")
            lp = ctypes.c_void_p(lse.data_ptr())
        fn = stream_attend_scratch if static_scratch else stream_attend
        fn(self.handle, layer, qp, q.shape[0], float(sm_scale), op, lp, self._stream())
        return out

    def append_attend(self, layer, frame_idx, k, v, q, sm_scale, transient=False, out=None, lse=None):
        """append + evict + attend of one frame in one call; returns (out, frames evicted)."""
        torch = self.torch
        if out is None:
            out = torch.empty_like(q)
        kp, vp = self._tensor(k), self._tensor(v, k.shape[0])
        qp = self._tensor(q)
        op = self._tensor(out, q.shape[0])
        lp = None
        if lse is not None:
            if lse.dtype != torch.float32 or not lse.is_contiguous() or lse.numel() != q.shape[0] * q.shape[1]:
                raise ValueError("lse must be a contiguous fp32 tensor of n_q * H elements")
            lp = ctypes.c_void_p(lse.data_ptr())
        n = kv_append_attend(self.handle, layer, frame_idx, kp, vp, k.shape[0], KV_TRANSIENT if transient else 0,
                             qp, q.shape[0], float(sm_scale), op, lp, self._stream())
        return out, n

    def score_and_compact(self, layer, score_table, window, lam, keep_count, keep_ids=None, ranks=None,
                          defer=False, reuse_ranks=False, s_hat=None, rank_radix=False) -> int:
        torch = self.torch
        if score_table.dtype != torch.float32 or not score_table.is_contiguous() or score_table.dim() != 2 \
                or score_table.shape[1] != self.cfg.num_layers:
            raise ValueError("score table must be a contiguous fp32 [rows, num_layers] tensor")
        for t in (keep_ids, ranks):
            if t is not None and (t.dtype != torch.int32 or not t.is_contiguous()):
                raise ValueError("keep_ids / ranks must be contiguous int32 tensors")
        if s_hat is not None and (s_hat.dtype != torch.float64 or not s_hat.is_contiguous()):
            raise ValueError("s_hat must be a contiguous float64 tensor")
        # the library writes up to keep_count ids, n_window x N ranks and N fused scores (N = the candidate
        # tokens, pages of the scale frames excluded); it cannot see the buffers' sizes
        if keep_ids is not None and keep_ids.numel() < keep_count:
            raise ValueError(f"keep_ids holds {keep_ids.numel()} ids, the step may write {keep_count}")
        if ranks is not None or s_hat is not None:
            _, lens, frames = self.page_table(layer)
            n_cand = sum(n for n, f in zip(lens, frames) if f >= self.cfg.scale_frames)
            if ranks is not None and ranks.numel() < min(window, layer + 1) * n_cand:
                raise ValueError(f"ranks holds {ranks.numel()} entries, the step writes "
                                 f"{min(window, layer + 1) * n_cand}")
            if s_hat is not None and s_hat.numel() < n_cand:
                raise ValueError(f"s_hat holds {s_hat.numel()} entries, the step writes {n_cand}")
        return score_and_compact(self.handle, layer, ctypes.c_void_p(score_table.data_ptr()), score_table.shape[0],
                                 window, lam, keep_count,
                                 None if keep_ids is None else ctypes.c_void_p(keep_ids.data_ptr()),
                                 None if ranks is None else ctypes.c_void_p(ranks.data_ptr()), self._stream(),
                                 defer, reuse_ranks,
                                 None if s_hat is None else ctypes.c_void_p(s_hat.data_ptr()), rank_radix)

    def sync(self, layer=-1) -> None:
        """Complete deferred score_and_compact steps (layer -1: every layer); raises their error, if any."""
        kv_sync(self.handle, layer)

    def merge_pages(self, layer) -> int:
        return kv_merge_pages(self.handle, layer, self._stream())

    def merge_pages_layers(self, first_layer, n_layers) -> list:
        """Page merges of n_layers layers in one call; pages released per layer."""
        return kv_merge_pages_layers(self.handle, first_layer, n_layers, self._stream())

    def _scores_arg(self, scores):
        if scores is None:
            return None, 0
        torch = self.torch
        if scores.dtype != torch.float64 or not scores.is_contiguous() or scores.dim() != 2 \
                or scores.shape[0] != self.cfg.num_heads:
            raise ValueError("scores must be a contiguous float64 [num_heads, stride] tensor")
        return ctypes.c_void_p(scores.data_ptr()), scores.shape[1]

    def diversity_score(self, layer, scores=None) -> float:
        """Mean diversity of the layer's candidates; scores: optional float64 [H, stride] output."""
        sp, stride = self._scores_arg(scores)
        return kv_diversity_score(self.handle, layer, sp, stride, self._stream())

    def diversity_prune(self, layer, keep_per_head, scores=None) -> list:
        """Per-head top-K prune; returns the candidates kept per head."""
        sp, stride = self._scores_arg(scores)
        return kv_diversity_prune(self.handle, layer, keep_per_head, self.cfg.num_heads, sp, stride, self._stream())

    def diversity_score_layers(self, first_layer, n_layers) -> list:
        """Mean diversity of each of n_layers layers, one wait."""
        return kv_diversity_score_layers(self.handle, first_layer, n_layers, self._stream())

    def diversity_prune_layers(self, first_layer, keep_per_head, out=None):
        """Per-head top-K prune of len(keep_per_head) layers, one wait; kept per layer and head (into `out`,
        an int64 numpy array, when given)."""
        return kv_diversity_prune_layers(self.handle, first_layer, keep_per_head, self.cfg.num_heads,
                                         self._stream(), out=out)

    def head_lengths(self, layer) -> list:
        return kv_get_head_lengths(self.handle, layer, self.cfg.num_heads)

    def page_table(self, layer):
        return kv_get_page_table(self.handle, layer)

    def info(self, layer) -> dict:
        return kv_get_info(self.handle, layer)

    def reset(self):
        kv_reset(self.handle)

    def set_splits(self, splits):
        kv_set_attend_splits(self.handle, splits)

    def set_tiling(self, tiling):
        """KV_TILING_AUTO, KV_TILING_PAGE or KV_TILING_PACKED (the bf16 attention's KV tiles)."""
        kv_set_attend_tiling(self.handle, tiling)

    # -- reading pages back (tests) -------------------------------------------
    def page_view(self, layer, page_id):
        """(K [H, Ts, D], V [H, Ts, D], ids [Ts]) views of one page in the pool."""
        torch = self.torch
        L = self.layout
        base = self.pool_ptr - self.pool_buf.data_ptr() + \
            (layer * (self.cfg.pages_per_layer + 1) + page_id) * L["page_bytes"]
        raw = self.pool_buf[base: base + L["page_bytes"]]
        dt = torch.bfloat16 if self.cfg.dtype == KV_BF16 else torch.float32
        H, D, Ts, E = self.cfg.num_heads, self.cfg.head_dim, L["token_stride"], L["elem_bytes"]
        k = raw[L["k_offset"]: L["k_offset"] + H * Ts * D * E].view(dt).view(H, Ts, D)
        v = raw[L["v_offset"]: L["v_offset"] + H * Ts * D * E].view(dt).view(H, Ts, D)
        ids = raw[L["id_offset"]: L["id_offset"] + Ts * 4].view(torch.int32)
        return k, v, ids
