"""Torch-tensor front end of liboasis.so: argument marshalling only.

Every function checks shapes, dtypes and devices of its tensors, hands their
device pointers to the matching ``oasis_*`` entry point of the C ABI together
with torch's current HIP stream, and returns.  No step of the path is computed
here; workspaces are plain torch allocations.  Layouts and semantics are the
ones documented in include/oasis.h.
"""
from __future__ import annotations

import ctypes

import torch

from . import _lib
from ._lib import IMPL_AUTO, IMPL_MFMA, IMPL_VALU, OasisShape, OasisStepOpts, check  # noqa: F401

_DTYPES = {torch.float32: _lib.OASIS_F32, torch.bfloat16: _lib.OASIS_BF16}


def _dt(t: torch.Tensor) -> int:
    if t.dtype not in _DTYPES:
        raise TypeError(f"unsupported dtype {t.dtype}; use float32 or bfloat16")
    return _DTYPES[t.dtype]


def _ptr(t):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("tensor must live on the GPU")
    if not t.is_contiguous():
        raise ValueError("tensor must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _i32(t: torch.Tensor, name: str) -> torch.Tensor:
    if t.dtype != torch.int32:
        raise TypeError(f"{name} must be int32")
    return t


def _stream(stream) -> ctypes.c_void_p:
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _shape(R, n_q, Hq, H, D, B, dtype, tile_stride=0) -> OasisShape:
    return OasisShape(int(R), int(n_q), int(Hq), int(H), int(D), int(B), int(dtype),
                      int(tile_stride))


def _tile_store(t: torch.Tensor, name: str, tile: int) -> tuple[int, int]:
    """Pointer and tile stride (elements) of a store of ``tile``-element tiles: the
    trailing dims that make up one tile must be dense, and the leading dims must
    step by one uniform tile stride (a dense store such as [..][L][D] or
    [..][n][B][D], or the K or V half of an interleaved store)."""
    dims = list(zip(t.shape, t.stride()))
    inner = 1
    while dims and inner < tile:
        n, st = dims.pop()
        if n > 1 and st != inner:
            raise ValueError(f"{name}: tiles must be dense")
        if inner * n > tile:
            # this dim spans several tiles (e.g. L of [..][L][D]): split it
            part = tile // inner
            if tile % inner or n % part:
                break
            dims.append((n // part, st * part))
            n = part
        inner *= n
    if inner != tile:
        raise ValueError(f"{name}: trailing dims do not split into {tile}-element tiles")
    step, span = None, 1
    for n, st in reversed(dims):
        if n > 1:
            if step is None:
                step = st
            elif st != step * span:
                raise ValueError(f"{name}: leading dims must step by one tile stride")
        span *= n
    step = tile if step is None else step
    if step < tile:
        raise ValueError(f"{name}: tiles overlap")
    return t.data_ptr(), int(step)


def interleaved_kv(kv: torch.Tensor) -> tuple[torch.Tensor, torch.Tensor]:
    """K and V tile views of an interleaved store kv [..][n][2][B][D]: block-head
    (.., n) keeps its K tile ([B][D], token-major) and V tile ([D][B], dim-major)
    side by side as one contiguous 2*B*D record.  The views are [..][n][B][D]
    and [..][n][D][B]."""
    if kv.dim() < 3 or kv.shape[-3] != 2:
        raise ValueError("interleaved store must be [..][n][2][B][D]")
    if not kv.is_contiguous():
        raise ValueError("interleaved store must be contiguous")
    B, D = kv.shape[-2:]
    flat = kv.view(*kv.shape[:-3], 2, B * D)
    return kv[..., 0, :, :], flat[..., 1, :].unflatten(-1, (D, B))


def build_summaries(keys: torch.Tensor, block_size: int, seq_len: torch.Tensor | None = None,
                    blk_begin: int = 0, blk_end: int | None = None,
                    out: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """keys [R][H][L_max][D], or a K tile store [R][H][n][B][D] (dense or the K half
    of an interleaved store) -> summaries [R][H][n][2][D] (0 = min, 1 = max)."""
    lib = _lib.load()
    B = int(block_size)
    if keys.dim() == 4:
        R, H, Lmax, D = keys.shape
        if Lmax % B:
            raise ValueError("L_max must be a multiple of block_size")
        nb = Lmax // B
    elif keys.dim() == 5:
        R, H, nb, B2, D = keys.shape
        if B2 != B:
            raise ValueError("key tiles do not match block_size")
    else:
        raise ValueError("keys must be [R][H][L_max][D] or [R][H][n][B][D]")
    kptr, ts = _tile_store(keys, "keys", B * D)
    if out is None:
        out = torch.zeros((R, H, nb, 2, D), dtype=keys.dtype, device=keys.device)
    if out.shape != (R, H, nb, 2, D) or out.dtype != keys.dtype:
        raise ValueError("summaries buffer has the wrong shape or dtype")
    if seq_len is not None:
        _i32(seq_len, "seq_len")
    shp = _shape(R, 1, H, H, D, B, _dt(keys), ts)
    end = nb if blk_end is None else int(blk_end)
    if not keys.is_cuda:
        raise ValueError("keys must live on the GPU")
    check("oasis_build_summaries",
          lib.oasis_build_summaries(ctypes.byref(shp), ctypes.c_void_p(kptr), nb, _ptr(seq_len),
                                    int(blk_begin), end, _ptr(out), _stream(stream)))
    return out


class PreparedAppend:
    """A validated oasis_append_kv call; calling it appends the tokens held in
    the prepared k_new / v_new / pos buffers (rewrite them in place between
    calls)."""

    def __init__(self, args, keep, lib):
        self.args = args
        self._keep = keep
        self._fn = lib.oasis_append_kv

    def __call__(self, stream=None) -> None:
        a = self.args
        if stream is not None:
            a = a[:-1] + [_stream(stream)]
        st = self._fn(*a)
        if st != 0:
            check("oasis_append_kv", st)


def prepare_append_kv(k_new: torch.Tensor, v_new: torch.Tensor, pos: torch.Tensor,
                      k_tiles: torch.Tensor, v_tiles: torch.Tensor, block_size: int,
                      summaries: torch.Tensor | None = None, stream=None) -> PreparedAppend:
    """``append_kv`` with the argument checks done once."""
    lib = _lib.load()
    R, H, D = k_new.shape
    B = int(block_size)
    if v_new.shape != k_new.shape or k_new.dtype != v_new.dtype:
        raise ValueError("k_new and v_new must match")
    _i32(pos, "pos")
    if pos.shape != (R,):
        raise ValueError("pos must be [R]")
    if k_tiles.dim() < 4 or k_tiles.shape[:2] != (R, H):
        raise ValueError("tile stores must be [R][H][n_blk_max][..tile..]")
    nb = k_tiles.shape[2]
    if v_tiles.shape[:3] != k_tiles.shape[:3] or k_tiles.dtype != k_new.dtype or \
            v_tiles.dtype != k_new.dtype:
        raise ValueError("k_tiles / v_tiles do not match the new tokens")
    kptr, ks = _tile_store(k_tiles, "k_tiles", B * D)
    vptr, vs = _tile_store(v_tiles, "v_tiles", B * D)
    if ks != vs:
        raise ValueError("k_tiles and v_tiles must share one tile stride")
    if summaries is not None and (summaries.shape != (R, H, nb, 2, D) or
                                  summaries.dtype != k_new.dtype):
        raise ValueError("summaries must be [R][H][n_blk_max][2][D] in the tiles' dtype")
    shp = _shape(R, 1, H, H, D, B, _dt(k_new), ks)
    args = [ctypes.byref(shp), _ptr(k_new), _ptr(v_new), _ptr(pos), ctypes.c_void_p(kptr),
            ctypes.c_void_p(vptr), nb, _ptr(summaries), _stream(stream)]
    return PreparedAppend(args, (shp, k_new, v_new, pos, k_tiles, v_tiles, summaries), lib)


def append_kv(k_new: torch.Tensor, v_new: torch.Tensor, pos: torch.Tensor, k_tiles: torch.Tensor,
              v_tiles: torch.Tensor, block_size: int, summaries: torch.Tensor | None = None,
              stream=None) -> None:
    """Write each request's new token (k_new / v_new [R][H][D], position pos [R],
    -1 = skip) into the tile stores; a token completing its block rebuilds that
    block's summary rows when ``summaries`` is given."""
    prepare_append_kv(k_new, v_new, pos, k_tiles, v_tiles, block_size, summaries, stream)()


def _opts_ref(opts):
    return ctypes.byref(opts) if opts is not None else None


def scored_rows(n_q: int, opts: OasisStepOpts | None) -> int:
    """Rows of the top-K and score outputs: n_q, or 2 when the drafts are averaged."""
    return 2 if (opts is not None and opts.draft_avg) else int(n_q)


class PreparedCall:
    """A validated entry-point call whose ctypes arguments are built once;
    calling it re-issues the call, with named slots optionally replaced: a
    tensor of the same shape (its pointer) or an integer.  For decode loops and
    timing, where marshalling would cost as much as the kernel."""

    def __init__(self, name: str, args: list, keep, lib, slots: dict, result=None):
        self.args = args
        self.result = result
        self._keep = keep
        self._slots = slots
        self._name = name
        self._fn = getattr(lib, name)

    def __call__(self, **updates):
        a = self.args
        for k, v in updates.items():
            a[self._slots[k]] = ctypes.c_void_p(v.data_ptr()) if isinstance(v, torch.Tensor) \
                else int(v)
        st = self._fn(*a)
        if st != 0:
            check(self._name, st)
        return self.result


def score_topk(q: torch.Tensor, summaries: torch.Tensor, top_k: int,
               n_blk: torch.Tensor | None = None, want_scores: bool = False,
               stream=None, out=None, opts: OasisStepOpts | None = None, prepare: bool = False):
    """q [R][n_q][Hq][D], summaries [R][H][n_blk_max][2][D].

    Returns (topk_idx int32, topk_score fp32, scores fp32 or None), top-K tensors
    shaped [R][n_s][H][top_k], scores [R][n_s][H][n_blk_max], n_s the scored rows
    (``scored_rows``).  ``opts`` selects the scoring variant (``step_opts``).
    ``out`` may pass preallocated (topk_idx, topk_score, scores, workspace).
    ``prepare``: return a PreparedCall (slot ``q``) instead of running.
    """
    lib = _lib.load()
    R, n_q, Hq, D = q.shape
    R2, H, nb, two, D2 = summaries.shape
    if R2 != R or two != 2 or D2 != D or summaries.dtype != q.dtype:
        raise ValueError("summaries do not match q")
    shp = _shape(R, n_q, Hq, H, D, 1, _dt(q))
    ns = scored_rows(n_q, opts)
    dev = q.device
    if out is not None:
        idx, val, sc, ws = out
    else:
        idx = torch.empty((R, ns, H, top_k), dtype=torch.int32, device=dev)
        val = torch.empty((R, ns, H, top_k), dtype=torch.float32, device=dev)
        sc = torch.empty((R, ns, H, nb), dtype=torch.float32, device=dev) if want_scores else None
        wsb = lib.oasis_score_topk_workspace(ctypes.byref(shp), nb, int(top_k), _opts_ref(opts))
        ws = torch.zeros(max(int(wsb), 1), dtype=torch.uint8, device=dev)
    if n_blk is not None:
        _i32(n_blk, "n_blk")
    args = [ctypes.byref(shp), _ptr(q), _ptr(summaries), nb, _ptr(n_blk), int(top_k), _ptr(idx),
            _ptr(val), _ptr(sc), _opts_ref(opts), _ptr(ws), ws.numel(), _stream(stream)]
    if prepare:
        return PreparedCall("oasis_score_topk", args, (shp, opts, q, summaries, n_blk, ws), lib,
                            {"q": 1}, (idx, val, sc))
    check("oasis_score_topk", lib.oasis_score_topk(*args))
    return idx, val, sc


def select_plan(topk_idx: torch.Tensor, slot_block: torch.Tensor, slot_stamp: torch.Tensor,
                step: int, cap: int, pred_row: int = 1, slot_block_out=None,
                slot_stamp_out=None, plan=None, want_evicted: bool = True,
                ins_blk: torch.Tensor | None = None, stream=None, prepare: bool = False):
    """Capped least-recently-selected plan, plus the insertion of each request's
    newly completed block (``ins_blk`` [R] int32, -1 = none).  Slot tables are
    updated in place unless *_out tensors are given.  Returns dict of plan tensors
    (``prepare``: a PreparedCall with slot ``step`` instead)."""
    lib = _lib.load()
    R, n_q, H, K = topk_idx.shape
    for t, n in ((topk_idx, "topk_idx"), (slot_block, "slot_block"), (slot_stamp, "slot_stamp")):
        _i32(t, n)
    if ins_blk is not None:
        _i32(ins_blk, "ins_blk")
        if ins_blk.shape != (R,):
            raise ValueError("ins_blk must be [R]")
    if slot_block.shape != (R, H, K) or slot_stamp.shape != (R, H, K):
        raise ValueError("slot tables must be [R][H][K]")
    bo = slot_block if slot_block_out is None else slot_block_out
    so = slot_stamp if slot_stamp_out is None else slot_stamp_out
    dev = topk_idx.device
    if plan is None:
        plan = {
            "plan_count": torch.empty((R, H), dtype=torch.int32, device=dev),
            "plan_src": torch.empty((R, H, K), dtype=torch.int32, device=dev),
            "plan_dst": torch.empty((R, H, K), dtype=torch.int32, device=dev),
            "plan_evicted": (torch.empty((R, H, K), dtype=torch.int32, device=dev)
                             if want_evicted else None),
        }
    args = [R, H, n_q, int(pred_row), K, _ptr(topk_idx), _ptr(slot_block), _ptr(slot_stamp),
            _ptr(bo), _ptr(so), int(step), int(cap), _ptr(ins_blk), _ptr(plan["plan_count"]),
            _ptr(plan["plan_src"]), _ptr(plan["plan_dst"]), _ptr(plan.get("plan_evicted")),
            _stream(stream)]
    if prepare:
        return PreparedCall("oasis_select_plan", args,
                            (topk_idx, slot_block, slot_stamp, bo, so, ins_blk), lib,
                            {"step": 10}, plan)
    check("oasis_select_plan", lib.oasis_select_plan(*args))
    return plan


def copy_blocks(src_k: torch.Tensor, src_v: torch.Tensor, res_k: torch.Tensor,
                res_v: torch.Tensor, plan: dict, block_size: int, stream=None) -> None:
    """src_* [R][H][n_blk_max][..tile..] (device or pinned host), res_* [R][H][K][..tile..]
    (device); K tiles [B][D], V tiles [D][B]; dense or interleaved, one shared tile stride."""
    prepare_copy_blocks(src_k, src_v, res_k, res_v, plan, block_size, stream)()


class PreparedCopy:
    """A validated oasis_copy_blocks call with its ctypes arguments built once;
    calling it enqueues the copy again (on the stream given at preparation, or
    on ``stream``)."""

    def __init__(self, args, keep, lib, name: str = "oasis_copy_blocks"):
        self.args = args
        self._keep = keep
        self._name = name
        self._fn = getattr(lib, name)

    def __call__(self, stream=None) -> None:
        a = self.args
        if stream is not None:
            a = a[:-1] + [_stream(stream)]
        st = self._fn(*a)
        if st != 0:
            check(self._name, st)


def prepare_copy_blocks(src_k: torch.Tensor, src_v: torch.Tensor, res_k: torch.Tensor,
                        res_v: torch.Tensor, plan: dict, block_size: int,
                        stream=None) -> PreparedCopy:
    """``copy_blocks`` with the argument checks done once (see ``PreparedCopy``)."""
    lib = _lib.load()
    if any(t.dim() < 4 for t in (src_k, src_v, res_k, res_v)):
        raise ValueError("tile stores must be [R][H][n][..tile..]")
    R, H, nb = src_k.shape[:3]
    K = res_k.shape[2]
    B = int(block_size)
    tile = src_k[0, 0, 0].numel()
    D = tile // B
    if D * B != tile:
        raise ValueError("tile size is not a multiple of block_size")
    if src_v.shape[:3] != src_k.shape[:3] or res_v.shape[:3] != res_k.shape[:3] or \
            res_k.shape[:2] != (R, H):
        raise ValueError("store shapes do not match")
    for t in (src_v, res_k, res_v):
        if t[0, 0, 0].numel() != tile or t.dtype != src_k.dtype:
            raise ValueError("tile size or dtype mismatch")
    for t in (src_k, src_v):
        if not t.is_cuda and not t.is_pinned():
            raise ValueError("source store must be device memory or pinned host memory")
    for t in (res_k, res_v):
        if not t.is_cuda:
            raise ValueError("resident store must live on the GPU")
    ptrs, strides = zip(*(_tile_store(t, n, tile) for t, n in
                          ((src_k, "src_k"), (src_v, "src_v"), (res_k, "res_k"), (res_v, "res_v"))))
    if len(set(strides)) != 1:
        raise ValueError("all four stores must share one tile stride")
    shp = _shape(R, 1, H, H, D, B, _dt(src_k), strides[0])
    cp = [ctypes.c_void_p(x) for x in ptrs]
    for k in ("plan_count", "plan_src", "plan_dst"):
        _i32(plan[k], k)
    if plan["plan_count"].shape != (R, H) or plan["plan_src"].shape != (R, H, K) or \
            plan["plan_dst"].shape != (R, H, K):
        raise ValueError("plan tensors must be [R][H] and [R][H][K]")
    args = [ctypes.byref(shp), cp[0], cp[1], nb, cp[2], cp[3], K, _ptr(plan["plan_count"]),
            _ptr(plan["plan_src"]), _ptr(plan["plan_dst"]), _stream(stream)]
    keep = (shp, src_k, src_v, res_k, res_v, plan["plan_count"], plan["plan_src"],
            plan["plan_dst"])
    return PreparedCopy(args, keep, lib)


# ------------------------------------------------------------ decode-host tier
def _np_or_tensor_ptr(a):
    """Host pointer of a numpy array or a CPU (pinned or not) tensor; None stays None."""
    if a is None:
        return None
    if isinstance(a, torch.Tensor):
        if a.is_cuda:
            raise ValueError("expected host memory")
        if not a.is_contiguous():
            raise ValueError("host array must be contiguous")
        return ctypes.c_void_p(a.data_ptr())
    import numpy as np
    if not (isinstance(a, np.ndarray) and a.flags["C_CONTIGUOUS"]):
        raise ValueError("host array must be a contiguous numpy array or tensor")
    return ctypes.c_void_p(a.ctypes.data)


class HostTier:
    """The decode-host block cache of one layer (oasis_host_tier_*): whole
    blocks of ``remote`` [R][n_blk][block] cached in ``cache`` [R][cap_max][block]
    (pinned, as the GPU gather reads it), with the union map ``map`` [R][n_blk]
    int32 (pinned).  The arrays must outlive the tier."""

    def __init__(self, batch: int, n_kv_heads: int, top_k: int, n_blk: int, capacity,
                 remote, cache, map_, block_bytes: int, workers: int = 1):
        import numpy as np
        self._lib = _lib.load()
        self.R, self.H, self.K, self.n_blk = int(batch), int(n_kv_heads), int(top_k), int(n_blk)
        self.capacity = np.ascontiguousarray(np.asarray(capacity, np.int32))
        self.cap_max = int(self.capacity.max()) if cache is None else int(cache.shape[1])
        self._keep = (remote, cache, map_, self.capacity)
        h = self._lib.oasis_host_tier_create(
            self.R, self.H, self.K, self.n_blk, _np_or_tensor_ptr(self.capacity), self.cap_max,
            int(block_bytes), _np_or_tensor_ptr(remote), _np_or_tensor_ptr(cache),
            _np_or_tensor_ptr(map_))
        if not h:
            raise ValueError("oasis_host_tier_create rejected its arguments")
        self._h = ctypes.c_void_p(h)
        if workers != 1:
            self.set_workers(workers)

    def set_workers(self, n: int) -> None:
        """Host threads per fetch (no fetch may be in flight)."""
        check("oasis_host_tier_set_workers", self._lib.oasis_host_tier_set_workers(self._h, int(n)))

    def fetch(self, step: int, plan_count, plan_src, slot_block=None) -> int:
        return int(self._lib.oasis_host_tier_fetch(self._h, int(step), _np_or_tensor_ptr(plan_count),
                                                   _np_or_tensor_ptr(plan_src),
                                                   _np_or_tensor_ptr(slot_block)))

    def prepare_submit(self, cache: torch.Tensor, res_k: torch.Tensor, res_v: torch.Tensor,
                       plan: dict, block_size: int):
        """Prepared oasis_host_tier_submit for one layer: returns
        ``submit(slot_block, after, copy_stream, done)`` (after / done: recorded
        torch events).  cache: pinned [R][cap_max][H][2][B][D]; res_*: the
        interleaved resident store; plan: the layer's plan buffers."""
        if cache.dim() != 6 or cache.shape[3] != 2 or not cache.is_pinned():
            raise ValueError("cache must be pinned [R][cap_max][H][2][B][D]")
        R, cap_max, H, _, B, D = cache.shape
        if int(block_size) != B or R != self.R or H != self.H:
            raise ValueError("cache does not match the tier or block_size")
        rptr_k, rs = _tile_store(res_k, "res_k", B * D)
        rptr_v, rs2 = _tile_store(res_v, "res_v", B * D)
        if rs != 2 * B * D or rs2 != rs:
            raise ValueError("the resident store must be interleaved (tile stride 2*B*D)")
        ck, cv = interleaved_kv(cache.view(R, cap_max * H, 2, B, D))
        shp = _shape(R, 1, H, H, D, B, _dt(cache), rs)
        for k in ("plan_count", "plan_src", "plan_dst"):
            _i32(plan[k], k)
        head = [self._h, ctypes.byref(shp), ctypes.c_void_p(ck.data_ptr()),
                ctypes.c_void_p(cv.data_ptr()), ctypes.c_void_p(rptr_k), ctypes.c_void_p(rptr_v),
                _ptr(plan["plan_count"]), _ptr(plan["plan_src"]), _ptr(plan["plan_dst"])]
        keep = (shp, cache, res_k, res_v, plan)
        fn = self._lib.oasis_host_tier_submit

        def submit(slot_block: torch.Tensor, after, copy_stream, done) -> None:
            if not after.cuda_event or not done.cuda_event:
                raise ValueError("record both events once before submitting")
            _ = keep
            check("oasis_host_tier_submit",
                  fn(*head, _ptr(_i32(slot_block, "slot_block")), ctypes.c_void_p(after.cuda_event),
                     _stream(copy_stream), ctypes.c_void_p(done.cuda_event)))

        return submit

    def wait_issued(self) -> None:
        """Host wait until every submitted job has been issued."""
        check("oasis_host_tier_wait_issued", self._lib.oasis_host_tier_wait_issued(self._h))

    def add_generated(self, req: int, block: int, step: int, slot_block=None) -> int:
        return int(self._lib.oasis_host_tier_add_generated(self._h, int(req), int(block), int(step),
                                                           _np_or_tensor_ptr(slot_block)))

    def trim(self, target, slot_block=None) -> None:
        import numpy as np
        t = np.ascontiguousarray(np.asarray(target, np.int32))
        check("oasis_host_tier_trim",
              self._lib.oasis_host_tier_trim(self._h, _np_or_tensor_ptr(t),
                                             _np_or_tensor_ptr(slot_block)))

    def state(self):
        """(slot_block [R][cap_max], last [R][cap_max], stats dict)."""
        import numpy as np
        sb = np.empty((self.R, self.cap_max), np.int32)
        last = np.empty((self.R, self.cap_max), np.int64)
        st = np.empty(5, np.int64)
        check("oasis_host_tier_state",
              self._lib.oasis_host_tier_state(self._h, _np_or_tensor_ptr(sb),
                                              _np_or_tensor_ptr(last), _np_or_tensor_ptr(st)))
        return sb, last, {"fetched": int(st[0]), "evicted": int(st[1]), "failed": int(st[2]),
                          "steps": int(st[3]), "fetch_ns": int(st[4])}

    def close(self) -> None:
        if getattr(self, "_h", None):
            self._lib.oasis_host_tier_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:  # interpreter shutdown
            pass


def prepare_copy_blocks_mapped(cache: torch.Tensor, map_: torch.Tensor, res_k: torch.Tensor,
                               res_v: torch.Tensor, plan: dict, block_size: int,
                               stream=None) -> PreparedCopy:
    """The gather of planned blocks from the decode-host cache (pinned,
    [R][cap_max][H][2][B][D]) through the union map (pinned [R][n_blk] int32)
    into the resident slots (res_* as ``copy_blocks``)."""
    lib = _lib.load()
    if cache.dim() != 6 or cache.shape[3] != 2 or not cache.is_pinned():
        raise ValueError("cache must be pinned [R][cap_max][H][2][B][D]")
    R, cap_max, H, _, B, D = cache.shape
    if int(block_size) != B:
        raise ValueError("block_size does not match the cache")
    if map_.dtype != torch.int32 or map_.dim() != 2 or map_.shape[0] != R or not map_.is_pinned():
        raise ValueError("map must be pinned int32 [R][n_blk]")
    K = res_k.shape[2]
    rptr_k, rs = _tile_store(res_k, "res_k", B * D)
    rptr_v, rs2 = _tile_store(res_v, "res_v", B * D)
    if rs != 2 * B * D or rs2 != rs:
        raise ValueError("the resident store must be interleaved (tile stride 2*B*D)")
    ck, cv = interleaved_kv(cache.view(R, cap_max * H, 2, B, D))
    shp = _shape(R, 1, H, H, D, B, _dt(cache), rs)
    for k in ("plan_count", "plan_src", "plan_dst"):
        _i32(plan[k], k)
    args = [ctypes.byref(shp), ctypes.c_void_p(ck.data_ptr()), ctypes.c_void_p(cv.data_ptr()),
            cap_max, ctypes.c_void_p(map_.data_ptr()), map_.shape[1], ctypes.c_void_p(rptr_k),
            ctypes.c_void_p(rptr_v), K, _ptr(plan["plan_count"]), _ptr(plan["plan_src"]),
            _ptr(plan["plan_dst"]), _stream(stream)]
    return PreparedCopy(args, (shp, cache, map_, res_k, res_v, plan), lib,
                        "oasis_copy_blocks_mapped")


def sparse_attn_workspace_bytes(q_shape, n_kv_heads: int, block_size: int, n_sel: int,
                                dtype: torch.dtype) -> int:
    R, n_q, Hq, D = q_shape
    shp = _shape(R, n_q, Hq, n_kv_heads, D, block_size, _DTYPES[dtype])
    return int(_lib.load().oasis_sparse_attn_workspace(ctypes.byref(shp), int(n_sel)))


def sparse_attn(q: torch.Tensor, k_tiles: torch.Tensor, v_tiles: torch.Tensor,
                tile_table: torch.Tensor, unit_stride: int, block_size: int,
                tail_tile: torch.Tensor | None = None, tail_len: torch.Tensor | None = None,
                scale: float = 0.0, want_lse: bool = True, impl: int = IMPL_AUTO,
                out=None, lse=None, workspace=None, stream=None, prepare: bool = False):
    """q [R][n_q][Hq][D]; k_tiles [..][B][D]; v_tiles [..][D][B] (dim-major);
    tile_table [R][H][n_sel] unit-local indices (-1 = skip).  Returns (out, lse)
    (``prepare``: a PreparedCall with slot ``q`` instead)."""
    lib = _lib.load()
    R, n_q, Hq, D = q.shape
    R2, H, n_sel = tile_table.shape
    _i32(tile_table, "tile_table")
    if R2 != R:
        raise ValueError("tile_table batch mismatch")
    if k_tiles.dtype != q.dtype or v_tiles.dtype != q.dtype:
        raise ValueError("q, k_tiles and v_tiles must share a dtype")
    B = int(block_size)
    kptr, ks = _tile_store(k_tiles, "k_tiles", B * D)
    vptr, vs = _tile_store(v_tiles, "v_tiles", B * D)
    if ks != vs:
        raise ValueError("k_tiles and v_tiles must share one tile stride")
    if not (k_tiles.is_cuda and v_tiles.is_cuda):
        raise ValueError("tile stores must live on the GPU")
    shp = _shape(R, n_q, Hq, H, D, B, _dt(q), ks)
    dev = q.device
    if out is None:
        out = torch.empty_like(q)
    if want_lse and lse is None:
        lse = torch.empty((R, n_q, Hq), dtype=torch.float32, device=dev)
    if workspace is None:
        wsb = lib.oasis_sparse_attn_workspace(ctypes.byref(shp), n_sel)
        workspace = torch.zeros(max(int(wsb), 1), dtype=torch.uint8, device=dev)
    for t, n in ((tail_tile, "tail_tile"), (tail_len, "tail_len")):
        if t is not None:
            _i32(t, n)
    args = [ctypes.byref(shp), _ptr(q), ctypes.c_void_p(kptr), ctypes.c_void_p(vptr),
            _ptr(tile_table), n_sel, int(unit_stride), _ptr(tail_tile), _ptr(tail_len),
            float(scale), _ptr(out), _ptr(lse if want_lse else None), _ptr(workspace),
            workspace.numel(), int(impl), _stream(stream)]
    res = (out, (lse if want_lse else None))
    if prepare:
        return PreparedCall("oasis_sparse_attn_impl", args,
                            (shp, q, k_tiles, v_tiles, tile_table, tail_tile, tail_len,
                             workspace), lib, {"q": 1}, res)
    check("oasis_sparse_attn_impl", lib.oasis_sparse_attn_impl(*args))
    return res


def step_opts(scan_chunks: int = 0, attn_splits: int = 0, impl: int = IMPL_AUTO,
              alpha: float | None = None, draft_avg: bool = False) -> OasisStepOpts:
    """Tuning (0 = automatic) and scoring variants: ``alpha`` scores s_b(alpha)
    (None = the exact bound), ``draft_avg`` takes three query rows and averages
    the two drafts before scoring."""
    return OasisStepOpts(int(scan_chunks), int(attn_splits), int(impl),
                         0 if alpha is None else 1, 1.0 if alpha is None else float(alpha),
                         1 if draft_avg else 0)


def lookahead_step_workspace_bytes(q_shape, n_kv_heads: int, block_size: int, n_blk_max: int,
                                   top_k: int, n_sel: int, dtype: torch.dtype,
                                   opts: OasisStepOpts | None = None) -> int:
    R, n_q, Hq, D = q_shape
    shp = _shape(R, n_q, Hq, n_kv_heads, D, block_size, _DTYPES[dtype])
    return int(_lib.load().oasis_lookahead_step_workspace(
        ctypes.byref(shp), int(n_blk_max), int(top_k), int(n_sel),
        ctypes.byref(opts) if opts is not None else None))


class PreparedStep:
    """A validated oasis_lookahead_step call whose ctypes arguments are built
    once; calling it re-issues the step with a new step index (and,
    optionally, new query and tile-table pointers of the same shape).  Meant
    for decode loops where Python marshalling would otherwise cost as much as
    the kernel."""

    _Q, _STEP, _BI, _SI, _BO, _SO, _INS, _TBL = 1, 13, 9, 10, 11, 12, 16, 23
    _NBLK = 4
    _KNEW, _VNEW, _POS = 26, 27, 28  # oasis_lookahead_step_append only
    _TT, _TL = 26, 27                # tail_tile, tail_len of oasis_lookahead_step

    def __init__(self, args, res, lib, append=False, no_alloc=False):
        self.args = args
        self.res = res
        self.append = append
        self._name = ("oasis_lookahead_step_append" if append else
                      "oasis_lookahead_step_noalloc" if no_alloc else "oasis_lookahead_step")
        self._fn = getattr(lib, self._name)

    def __call__(self, step: int, q: torch.Tensor | None = None, token=None,
                 n_blk: torch.Tensor | None = None, ins_blk: torch.Tensor | None = None,
                 tail=None) -> dict:
        """token: (k_new, v_new, pos) of this step (append form only).  n_blk,
        ins_blk and tail = (tail_tile, tail_len) replace the prepared tensors
        of those arguments (same shapes and dtypes; each was given at
        preparation, so its pointer slot exists)."""
        a = self.args
        a[self._STEP] = int(step)
        if q is not None:
            a[self._Q] = ctypes.c_void_p(q.data_ptr())
        if token is not None:
            if not self.append:
                raise ValueError("this step was prepared without a new token")
            for i, t in zip((self._KNEW, self._VNEW, self._POS), token):
                a[i] = ctypes.c_void_p(t.data_ptr())
        for i, t in ((self._NBLK, n_blk), (self._INS, ins_blk)):
            if t is not None:
                if a[i] is None or t.dtype != torch.int32 or not t.is_contiguous():
                    raise ValueError("prepare the step with this argument first (int32, contiguous)")
                a[i] = ctypes.c_void_p(t.data_ptr())
        if tail is not None:
            if self.append or a[self._TT] is None:
                raise ValueError("this step was prepared without tail_tile / tail_len")
            a[self._TT] = ctypes.c_void_p(tail[0].data_ptr())
            a[self._TL] = ctypes.c_void_p(tail[1].data_ptr())
        st = self._fn(*a)
        if st != 0:
            check(self._name, st)
        return self.res


def lookahead_step(*args, **kwargs) -> dict:
    """One fused layer-step; see ``prepare_lookahead_step`` for the arguments."""
    call = prepare_lookahead_step(*args, **kwargs)
    return call(call.args[PreparedStep._STEP])


def prepare_lookahead_step(q: torch.Tensor, summaries: torch.Tensor, top_k: int,
                   slot_block: torch.Tensor, slot_stamp: torch.Tensor,
                   slot_block_out: torch.Tensor, slot_stamp_out: torch.Tensor,
                   step: int, cap: int, k_tiles: torch.Tensor, v_tiles: torch.Tensor,
                   tile_table: torch.Tensor, unit_stride: int, block_size: int,
                   pred_row: int = 1, n_blk: torch.Tensor | None = None,
                   ins_blk: torch.Tensor | None = None,
                   tail_tile: torch.Tensor | None = None, tail_len: torch.Tensor | None = None,
                   scale: float = 0.0, want_scores: bool = False, want_lse: bool = True,
                   want_evicted: bool = True, opts: OasisStepOpts | None = None,
                   bufs: dict | None = None, stream=None, new_token=None,
                   no_alloc: bool = False) -> PreparedStep:
    """One fused layer-step (attention over ``tile_table`` + scan, top-K and plan).

    no_alloc: call oasis_lookahead_step_noalloc (the library's per-GPU scratch
    array instead of a workspace tensor; no ``workspace`` is allocated).

    new_token: (k_new [R][H][D], v_new [R][H][D], pos [R] int32) appends one
    token per request in the same launch (oasis_lookahead_step_append): the
    full cache is the store (unit_stride = n_blk_max), the active block comes
    from pos, so tail_tile / tail_len must be None.

    q [R][n_q][Hq][D]; summaries [R][H][n_blk_max][2][D]; slot tables [R][H][top_k]
    (the ``*_out`` pair must not overlap ``tile_table``); tiles and table as in
    ``sparse_attn``.  ``bufs`` may hold preallocated outputs under the keys of the
    result dict plus ``workspace`` (zero-filled); missing ones are allocated and
    added to it.  Returns the prepared call; its result is a dict with out, lse,
    topk_idx, topk_score, scores, plan_count, plan_src, plan_dst, plan_evicted.
    """
    lib = _lib.load()
    R, n_q, Hq, D = q.shape
    R2, H, nb, two, D2 = summaries.shape
    if R2 != R or two != 2 or D2 != D or summaries.dtype != q.dtype:
        raise ValueError("summaries do not match q")
    if k_tiles.dtype != q.dtype or v_tiles.dtype != q.dtype:
        raise ValueError("q, k_tiles and v_tiles must share a dtype")
    K = int(top_k)
    for t, n in ((slot_block, "slot_block"), (slot_stamp, "slot_stamp"),
                 (slot_block_out, "slot_block_out"), (slot_stamp_out, "slot_stamp_out")):
        _i32(t, n)
        if t.shape != (R, H, K):
            raise ValueError(f"{n} must be [R][H][top_k]")
    _i32(tile_table, "tile_table")
    if tile_table.shape[:2] != (R, H):
        raise ValueError("tile_table must be [R][H][n_sel]")
    n_sel = tile_table.shape[2]
    B = int(block_size)
    kptr, ks = _tile_store(k_tiles, "k_tiles", B * D)
    vptr, vs = _tile_store(v_tiles, "v_tiles", B * D)
    if ks != vs:
        raise ValueError("k_tiles and v_tiles must share one tile stride")
    if not (k_tiles.is_cuda and v_tiles.is_cuda):
        raise ValueError("tile stores must live on the GPU")
    shp = _shape(R, n_q, Hq, H, D, B, _dt(q), ks)
    dev = q.device
    b = {} if bufs is None else bufs

    def get(key, shape, dtype, zero=False):
        t = b.get(key)
        if t is None:
            t = (torch.zeros if zero else torch.empty)(shape, dtype=dtype, device=dev)
            b[key] = t
        return t

    ns = scored_rows(n_q, opts)
    res = {
        "out": get("out", q.shape, q.dtype),
        "lse": get("lse", (R, n_q, Hq), torch.float32) if want_lse else None,
        "topk_idx": get("topk_idx", (R, ns, H, K), torch.int32),
        "topk_score": get("topk_score", (R, ns, H, K), torch.float32),
        "scores": get("scores", (R, ns, H, nb), torch.float32) if want_scores else None,
        "plan_count": get("plan_count", (R, H), torch.int32),
        "plan_src": get("plan_src", (R, H, K), torch.int32),
        "plan_dst": get("plan_dst", (R, H, K), torch.int32),
        "plan_evicted": get("plan_evicted", (R, H, K), torch.int32) if want_evicted else None,
    }
    if no_alloc and new_token is not None:
        raise ValueError("the no-allocation form has no appended token")
    if no_alloc:
        ws = None
    else:
        if b.get("workspace") is None:
            wsb = lib.oasis_lookahead_step_workspace(
                ctypes.byref(shp), nb, K, n_sel, ctypes.byref(opts) if opts is not None else None)
            b["workspace"] = torch.zeros(max(int(wsb), 1), dtype=torch.uint8, device=dev)
        ws = b["workspace"]
    for t, n in ((n_blk, "n_blk"), (tail_tile, "tail_tile"), (tail_len, "tail_len"),
                 (ins_blk, "ins_blk")):
        if t is not None:
            _i32(t, n)
    if ins_blk is not None and ins_blk.shape != (R,):
        raise ValueError("ins_blk must be [R]")
    if new_token is not None:
        if tail_tile is not None or tail_len is not None:
            raise ValueError("with new_token the active block comes from pos")
        k_new, v_new, pos = new_token
        for t, n in ((k_new, "k_new"), (v_new, "v_new")):
            if t.shape != (R, H, D) or t.dtype != q.dtype:
                raise ValueError(f"{n} must be [R][H][D] of q's dtype")
        _i32(pos, "pos")
        if pos.shape != (R,):
            raise ValueError("pos must be [R]")
        tail = [_ptr(k_new), _ptr(v_new), _ptr(pos)]
    else:
        tail = [_ptr(tail_tile), _ptr(tail_len)]
    args = [ctypes.byref(shp), _ptr(q), _ptr(summaries), nb, _ptr(n_blk), K,
            _ptr(res["topk_idx"]), _ptr(res["topk_score"]), _ptr(res["scores"]),
            _ptr(slot_block), _ptr(slot_stamp), _ptr(slot_block_out), _ptr(slot_stamp_out),
            int(step), int(cap), int(pred_row), _ptr(ins_blk), _ptr(res["plan_count"]),
            _ptr(res["plan_src"]),
            _ptr(res["plan_dst"]), _ptr(res["plan_evicted"]), ctypes.c_void_p(kptr),
            ctypes.c_void_p(vptr),
            _ptr(tile_table), n_sel, int(unit_stride), *tail,
            float(scale), _ptr(res["out"]), _ptr(res["lse"]),
            ctypes.byref(opts) if opts is not None else None,
            *([] if no_alloc else [_ptr(ws), ws.numel()]), _stream(stream)]
    call = PreparedStep(args, res, lib, append=new_token is not None, no_alloc=no_alloc)
    call._keep = (shp, opts, q, summaries, slot_block, slot_stamp, slot_block_out,
                  slot_stamp_out, k_tiles, v_tiles, tile_table, n_blk, tail_tile, tail_len, ins_blk,
                  ws, new_token)
    return call
