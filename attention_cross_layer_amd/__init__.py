"""Python binding of libkvshare.so, the gfx950 cross-layer shared-KV attention
library.  Argument marshalling only: every step of the path runs in the HIP
library; PyTorch supplies device memory and the stream.

The functions carry the C ABI's names (include/kvshare.h).  Tensors are
passed by device pointer; shapes and dtypes are checked here only to build
the call, the library re-validates everything it is given.

There is no fallback: if the library is missing or cannot be loaded, the
first call raises.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch  # must be loaded before the library so both share one HIP runtime

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libkvshare.so")

KVS_OK, KVS_ERR_ARG, KVS_ERR_MAP, KVS_ERR_NOT_SOURCE, KVS_ERR_RANGE = 0, 1, 2, 3, 4
KVS_ERR_UNSUPPORTED, KVS_ERR_ALIGN, KVS_ERR_HIP = 5, 6, 7
STATUS_NAMES = {0: "KVS_OK", 1: "KVS_ERR_ARG", 2: "KVS_ERR_MAP", 3: "KVS_ERR_NOT_SOURCE",
                4: "KVS_ERR_RANGE", 5: "KVS_ERR_UNSUPPORTED", 6: "KVS_ERR_ALIGN",
                7: "KVS_ERR_HIP"}
KVS_F32, KVS_BF16 = 0, 1
KVS_DENSE, KVS_FACTORIZED = 0, 1
PAGE = 64

# Every symbol include/kvshare.h declares.
EXPORTS = ("kvs_share_plan", "kvs_plan_free", "kvs_plan_layer", "kvs_plan_summary",
           "kvs_cache_layout", "kvs_decode_splits", "kvs_decode_workspace_size", "kvs_append",
           "kvs_append_factorized", "kvs_encode_workspace_size", "kvs_encode_factorized",
           "kvs_basis_workspace_size", "kvs_pair_basis", "kvs_pair_bases", "kvs_residual_basis",
           "kvs_residual_bases",
           "kvs_attn_decode", "kvs_attn_decode_noalloc", "kvs_attn_decode_stats", "kvs_route_ranks",
           "kvs_attn_prefill_chunk", "kvs_time_next_launch", "kvs_last_error")


class KvsError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {message}")
        self.status = status


class kvs_config(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "n_layers", "n_q_heads", "n_kv_heads", "head_dim", "dtype", "kind", "basis_rank",
        "resid_rank_max", "max_batch", "max_ctx")]


class kvs_layer_info(ctypes.Structure):
    _fields_ = [("owns_kv", ctypes.c_int32), ("n_src", ctypes.c_int32),
                ("src_layer", ctypes.c_int32 * 2), ("src_slot", ctypes.c_int32 * 2),
                ("weight", ctypes.c_float * 2), ("masks_current", ctypes.c_int32)]


class kvs_plan_info(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in ("n_layers", "n_slots", "last_owner_layer",
                                              "n_mixed_layers")]


class kvs_cache_sizes(ctypes.Structure):
    _fields_ = ([(n, ctypes.c_int32) for n in ("page_tokens", "pages_per_seq", "n_phys_pages",
                                                "n_slots")]
                + [(n, ctypes.c_size_t) for n in (
                    "k_pool_bytes", "v_pool_bytes", "page_table_bytes", "coef_pool_bytes",
                    "resid_pool_bytes", "scale_pool_bytes", "rank_pool_bytes", "basis_bytes",
                    "resid_basis_bytes")])


class kvs_cache(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in (
        "k_pool", "v_pool", "page_table", "ck_pool", "cv_pool", "dk_pool", "dv_pool", "sk_pool",
        "sv_pool", "rank_pool", "basis_k", "basis_v", "ubasis_k", "ubasis_v")]


class kvs_router(ctypes.Structure):
    _fields_ = [("entropy_focused", ctypes.c_float), ("entropy_diffuse", ctypes.c_float),
                ("peak_focused", ctypes.c_float), ("rank_focused", ctypes.c_int32),
                ("rank_mid", ctypes.c_int32), ("rank_diffuse", ctypes.c_int32)]


_lib = None


def _hip_runtimes_mapped():
    paths = set()
    with open("/proc/self/maps") as f:
        for line in f:
            if "libamdhip64" in line:
                paths.add(line.split()[-1])
    return paths


def lib():
    """Load libkvshare.so (once).  Raises if it is missing or would bring a
    second HIP runtime into the process."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run __graft_entry__.build() or "
                          "python -m attention_cross_layer_amd.build")
    L = ctypes.CDLL(LIB_PATH)
    rts = _hip_runtimes_mapped()
    if len(rts) > 1:
        raise ImportError(f"two HIP runtimes mapped: {sorted(rts)}")
    P = ctypes.POINTER
    vp, i32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
    sig = {
        "kvs_share_plan": (i32, [P(kvs_config), vp, vp, P(vp)]),
        "kvs_plan_free": (None, [vp]),
        "kvs_plan_layer": (i32, [vp, i32, P(kvs_layer_info)]),
        "kvs_plan_summary": (i32, [vp, P(kvs_plan_info)]),
        "kvs_cache_layout": (i32, [vp, P(kvs_cache_sizes)]),
        "kvs_decode_splits": (i32, [vp, i32, i32, P(i32)]),
        "kvs_decode_workspace_size": (i32, [vp, i32, i32, P(sz)]),
        "kvs_append": (i32, [vp, P(kvs_cache), i32, vp, vp, i32, vp, i32, vp]),
        "kvs_append_factorized": (i32, [vp, P(kvs_cache), i32, vp, vp, vp, vp, vp, vp, vp, i32,
                                        vp, i32, vp]),
        "kvs_attn_decode": (i32, [vp, P(kvs_cache), i32, vp, vp, i32, i32, i32, vp, i32, vp, sz,
                                  vp]),
        "kvs_attn_decode_noalloc": (i32, [vp, P(kvs_cache), i32, vp, vp, i32, i32, i32, vp, i32,
                                          vp]),
        "kvs_attn_prefill_chunk": (i32, [vp, P(kvs_cache), i32, vp, i32, vp, i32, i32, vp, i32,
                                         vp]),
        "kvs_encode_workspace_size": (i32, [vp, i32, i32, P(sz)]),
        "kvs_encode_factorized": (i32, [vp, P(kvs_cache), i32, vp, vp, vp, vp, vp, i32, vp, i32,
                                        vp, sz, vp]),
        "kvs_basis_workspace_size": (i32, [vp, i32, i32, P(sz)]),
        "kvs_pair_basis": (i32, [vp, vp, vp, vp, vp, vp, i32, i32, vp, vp, vp, sz, vp]),
        "kvs_residual_basis": (i32, [vp, vp, vp, vp, vp, vp, vp, vp, i32, i32, vp, vp, vp, sz,
                                     vp]),
        "kvs_attn_decode_stats": (i32, [vp, P(kvs_cache), i32, vp, vp, i32, i32, i32, vp, i32, vp,
                                        vp, sz, vp]),
        "kvs_route_ranks": (i32, [vp, vp, i32, vp, i32, P(kvs_router), vp, vp]),
        "kvs_pair_bases": (i32, [vp, i32, vp, vp, vp, vp, vp, i32, i32, vp, vp, vp, sz, vp]),
        "kvs_residual_bases": (i32, [vp, i32, vp, vp, vp, vp, vp, vp, vp, i32, i32, vp, vp, vp, sz,
                                     vp]),
        "kvs_time_next_launch": (i32, [vp, vp]),
        "kvs_last_error": (ctypes.c_char_p, []),
    }
    for name, (res, args) in sig.items():
        fn = getattr(L, name)
        fn.restype = res
        fn.argtypes = args
    _lib = L
    return L


def _check(status: int):
    if status != KVS_OK:
        raise KvsError(status, lib().kvs_last_error().decode())


def _ptr(t: Optional[torch.Tensor]):
    if t is None:
        return None
    if not t.is_contiguous():
        raise ValueError("tensors passed to the library must be contiguous (dense row-major)")
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    if isinstance(stream, torch.cuda.Stream):
        return ctypes.c_void_p(stream.cuda_stream)
    return ctypes.c_void_p(int(stream))


def _dtype_code(dt) -> int:
    if dt == torch.float32:
        return KVS_F32
    if dt == torch.bfloat16:
        return KVS_BF16
    raise ValueError(f"unsupported dtype {dt}")


def _torch_dtype(code: int):
    return torch.float32 if code == KVS_F32 else torch.bfloat16


# ---------------------------------------------------------------------------
# planning
# ---------------------------------------------------------------------------

class Plan:
    """Owner of a kvs_plan handle."""

    def __init__(self, handle: ctypes.c_void_p, cfg: kvs_config):
        self.handle = handle
        self.cfg = cfg

    def __del__(self):
        if getattr(self, "handle", None) and _lib is not None:
            _lib.kvs_plan_free(self.handle)
            self.handle = None

    @property
    def _as_arg(self):
        return self.handle


def kvs_share_plan(cfg: kvs_config, src, w=None) -> Plan:
    """Build a plan; ``src`` [L,2] int32 and ``w`` [L,2] float32 (host tensors
    or sequences)."""
    src_t = torch.as_tensor(src, dtype=torch.int32).contiguous().cpu()
    w_t = None if w is None else torch.as_tensor(w, dtype=torch.float32).contiguous().cpu()
    h = ctypes.c_void_p()
    _check(lib().kvs_share_plan(ctypes.byref(cfg), ctypes.c_void_p(src_t.data_ptr()),
                                None if w_t is None else ctypes.c_void_p(w_t.data_ptr()),
                                ctypes.byref(h)))
    return Plan(h, cfg)


def kvs_plan_layer(plan: Plan, layer: int) -> kvs_layer_info:
    out = kvs_layer_info()
    _check(lib().kvs_plan_layer(plan.handle, layer, ctypes.byref(out)))
    return out


def kvs_plan_summary(plan: Plan) -> kvs_plan_info:
    out = kvs_plan_info()
    _check(lib().kvs_plan_summary(plan.handle, ctypes.byref(out)))
    return out


def kvs_cache_layout(plan: Plan) -> kvs_cache_sizes:
    out = kvs_cache_sizes()
    _check(lib().kvs_cache_layout(plan.handle, ctypes.byref(out)))
    return out


def kvs_decode_splits(plan: Plan, batch: int, max_seq_len: int) -> int:
    out = ctypes.c_int32()
    _check(lib().kvs_decode_splits(plan.handle, batch, max_seq_len, ctypes.byref(out)))
    return out.value


def kvs_decode_workspace_size(plan: Plan, batch: int, n_splits: int) -> int:
    out = ctypes.c_size_t()
    _check(lib().kvs_decode_workspace_size(plan.handle, batch, n_splits, ctypes.byref(out)))
    return out.value


# ---------------------------------------------------------------------------
# device buffers (torch allocations sized by the library)
# ---------------------------------------------------------------------------

class Cache:
    """Caller-owned device buffers of one cache instance, allocated with torch
    in the sizes kvs_cache_layout() reports, plus the kvs_cache struct that
    points at them.  ``page_perm`` optionally permutes physical pages."""

    def __init__(self, plan: Plan, device="cuda", page_perm: Optional[torch.Tensor] = None):
        sz = kvs_cache_layout(plan)
        self.sizes = sz
        self.plan = plan
        dev = torch.device(device)
        B = plan.cfg.max_batch
        n_pages = sz.n_phys_pages
        if page_perm is None:
            pt = torch.arange(n_pages, dtype=torch.int32)
        else:
            pt = torch.as_tensor(page_perm, dtype=torch.int32)
        self.page_table = pt.view(B, sz.pages_per_seq).to(dev).contiguous()
        u8 = torch.uint8

        def buf(nbytes):
            return torch.empty(max(nbytes, 16), dtype=u8, device=dev) if nbytes else None

        self.k_pool = buf(sz.k_pool_bytes)
        self.v_pool = buf(sz.v_pool_bytes)
        self.ck_pool = buf(sz.coef_pool_bytes)
        self.cv_pool = buf(sz.coef_pool_bytes)
        self.dk_pool = buf(sz.resid_pool_bytes)
        self.dv_pool = buf(sz.resid_pool_bytes)
        self.sk_pool = buf(sz.scale_pool_bytes)
        self.sv_pool = buf(sz.scale_pool_bytes)
        self.rank_pool = buf(sz.rank_pool_bytes)
        self.basis_k = buf(sz.basis_bytes)
        self.basis_v = buf(sz.basis_bytes)
        self.ubasis_k = buf(sz.resid_basis_bytes)
        self.ubasis_v = buf(sz.resid_basis_bytes)
        self.struct = kvs_cache()
        for name in ("k_pool", "v_pool", "page_table", "ck_pool", "cv_pool", "dk_pool",
                     "dv_pool", "sk_pool", "sv_pool", "rank_pool", "basis_k", "basis_v",
                     "ubasis_k", "ubasis_v"):
            t = getattr(self, name)
            setattr(self.struct, name, None if t is None else t.data_ptr())


# ---------------------------------------------------------------------------
# compute calls
# ---------------------------------------------------------------------------

def kvs_append(plan: Plan, cache: Cache, layer: int, k: torch.Tensor, v: torch.Tensor,
               start_pos: torch.Tensor, stream=None):
    """Append k, v [B, n, Hkv, hd] of an owner layer at start_pos[b] (device int32)."""
    B, n = k.shape[0], k.shape[1]
    _check(lib().kvs_append(plan.handle, ctypes.byref(cache.struct), layer, _ptr(k), _ptr(v), n,
                            _ptr(start_pos), B, _stream(stream)))


def kvs_append_factorized(plan: Plan, cache: Cache, layer: int, ck, cv, dk, dv, sk, sv, rank,
                          start_pos: torch.Tensor, stream=None):
    B, n = dk.shape[0], dk.shape[1]
    _check(lib().kvs_append_factorized(plan.handle, ctypes.byref(cache.struct), layer, _ptr(ck),
                                       _ptr(cv), _ptr(dk), _ptr(dv), _ptr(sk), _ptr(sv),
                                       _ptr(rank), n, _ptr(start_pos), B, _stream(stream)))


def kvs_encode_workspace_size(plan: Plan, batch: int, n: int) -> int:
    out = ctypes.c_size_t()
    _check(lib().kvs_encode_workspace_size(plan.handle, batch, n, ctypes.byref(out)))
    return out.value


def kvs_encode_factorized(plan: Plan, cache: Cache, layer: int, k: torch.Tensor, v: torch.Tensor,
                          rank: torch.Tensor, start_pos: torch.Tensor, k_owner=None, v_owner=None,
                          workspace: Optional[torch.Tensor] = None, stream=None):
    """Encode k, v [B, n, Hkv, hd] (bf16) of ``layer`` into the factorized
    cache at start_pos; k_owner / v_owner: rows of the pair's coefficient-
    writing layer (None when ``layer`` is that layer)."""
    B, n = k.shape[0], k.shape[1]
    if workspace is None:
        workspace = torch.empty(kvs_encode_workspace_size(plan, B, n), dtype=torch.uint8,
                                device=k.device)
    _check(lib().kvs_encode_factorized(plan.handle, ctypes.byref(cache.struct), layer, _ptr(k),
                                       _ptr(v), _ptr(k_owner), _ptr(v_owner), _ptr(rank), n,
                                       _ptr(start_pos), B, _ptr(workspace), workspace.numel(),
                                       _stream(stream)))


def kvs_basis_workspace_size(plan: Plan, batch: int, n: int) -> int:
    out = ctypes.c_size_t()
    _check(lib().kvs_basis_workspace_size(plan.handle, batch, n, ctypes.byref(out)))
    return out.value


def kvs_pair_basis(plan: Plan, k_a, v_a, k_b, v_b, n_tokens: torch.Tensor, basis_k: torch.Tensor,
                   basis_v: torch.Tensor, workspace: Optional[torch.Tensor] = None, stream=None):
    """Pair basis [Hkv, R, hd] (bf16, written into basis_k / basis_v) from the
    rows [B, n, Hkv, hd] of the pair's two layers (k_b, v_b may be None)."""
    B, n = k_a.shape[0], k_a.shape[1]
    if workspace is None:
        workspace = torch.empty(kvs_basis_workspace_size(plan, B, n), dtype=torch.uint8,
                                device=k_a.device)
    _check(lib().kvs_pair_basis(plan.handle, _ptr(k_a), _ptr(v_a), _ptr(k_b), _ptr(v_b),
                                _ptr(n_tokens), n, B, _ptr(basis_k), _ptr(basis_v),
                                _ptr(workspace), workspace.numel(), _stream(stream)))


def kvs_residual_basis(plan: Plan, k, v, basis_k, basis_v, n_tokens: torch.Tensor,
                       ubasis_k: torch.Tensor, ubasis_v: torch.Tensor, k_owner=None,
                       v_owner=None, workspace: Optional[torch.Tensor] = None, stream=None):
    """Residual directions [Hkv, Rmax, hd] (bf16, written into ubasis_k /
    ubasis_v) of a layer from its rows, the owner's rows and the pair basis."""
    B, n = k.shape[0], k.shape[1]
    if workspace is None:
        workspace = torch.empty(kvs_basis_workspace_size(plan, B, n), dtype=torch.uint8,
                                device=k.device)
    _check(lib().kvs_residual_basis(plan.handle, _ptr(k), _ptr(v), _ptr(k_owner), _ptr(v_owner),
                                    _ptr(basis_k), _ptr(basis_v), _ptr(n_tokens), n, B,
                                    _ptr(ubasis_k), _ptr(ubasis_v), _ptr(workspace),
                                    workspace.numel(), _stream(stream)))


def _ptr_array(ts):
    """Host array of device pointers (None entries -> NULL), or None."""
    if ts is None:
        return None
    arr = (ctypes.c_void_p * len(ts))()
    for i, t in enumerate(ts):
        p = _ptr(t)
        arr[i] = None if p is None else p.value
    return arr


def kvs_pair_bases(plan: Plan, k_a, v_a, k_b, v_b, n_tokens: torch.Tensor, basis_k, basis_v,
                   workspace: Optional[torch.Tensor] = None, stream=None):
    """kvs_pair_basis over lists of pairs (k_b / v_b: None or lists with None
    entries); the workspace default holds every item at once (at most 32)."""
    n_items = len(k_a)
    B, n = k_a[0].shape[0], k_a[0].shape[1]
    if workspace is None:
        workspace = torch.empty(kvs_basis_workspace_size(plan, B, n) * min(n_items, 32),
                                dtype=torch.uint8, device=k_a[0].device)
    _check(lib().kvs_pair_bases(plan.handle, n_items, _ptr_array(k_a), _ptr_array(v_a),
                                _ptr_array(k_b), _ptr_array(v_b), _ptr(n_tokens), n, B,
                                _ptr_array(basis_k), _ptr_array(basis_v), _ptr(workspace),
                                workspace.numel(), _stream(stream)))


def kvs_residual_bases(plan: Plan, k, v, basis_k, basis_v, n_tokens: torch.Tensor, ubasis_k,
                       ubasis_v, k_owner=None, v_owner=None,
                       workspace: Optional[torch.Tensor] = None, stream=None):
    """kvs_residual_basis over lists of layers (k_owner / v_owner: None or
    lists with None entries for owner layers)."""
    n_items = len(k)
    B, n = k[0].shape[0], k[0].shape[1]
    if workspace is None:
        workspace = torch.empty(kvs_basis_workspace_size(plan, B, n) * min(n_items, 32),
                                dtype=torch.uint8, device=k[0].device)
    _check(lib().kvs_residual_bases(plan.handle, n_items, _ptr_array(k), _ptr_array(v),
                                    _ptr_array(k_owner), _ptr_array(v_owner), _ptr_array(basis_k),
                                    _ptr_array(basis_v), _ptr(n_tokens), n, B, _ptr_array(ubasis_k),
                                    _ptr_array(ubasis_v), _ptr(workspace), workspace.numel(),
                                    _stream(stream)))


def kvs_attn_decode(plan: Plan, cache: Cache, layer: int, q: torch.Tensor,
                    seq_len: torch.Tensor, max_seq_len: int, out: Optional[torch.Tensor] = None,
                    out_dtype=torch.float32, n_splits: int = 0,
                    workspace: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """Decode attention of ``layer``: q [B, Hq, hd] -> out [B, Hq, hd]."""
    B = q.shape[0]
    if n_splits == 0:
        n_splits = kvs_decode_splits(plan, B, max_seq_len)
    if workspace is None:
        # partial results: every partition writes its whole row, so no clearing is
        # needed; zero-filled only so that a failed launch leaves no stale data
        workspace = torch.zeros(kvs_decode_workspace_size(plan, B, n_splits), dtype=torch.uint8,
                                device=q.device)
    if out is None:
        out = torch.empty(q.shape, dtype=out_dtype, device=q.device)
    _check(lib().kvs_attn_decode(plan.handle, ctypes.byref(cache.struct), layer, _ptr(q),
                                 _ptr(seq_len), B, max_seq_len, n_splits, _ptr(out),
                                 _dtype_code(out.dtype), _ptr(workspace), workspace.numel(),
                                 _stream(stream)))
    return out


def kvs_attn_decode_noalloc(plan: Plan, cache: Cache, layer: int, q: torch.Tensor,
                            seq_len: torch.Tensor, max_seq_len: int, out: torch.Tensor,
                            n_splits: int = 0, stream=None) -> torch.Tensor:
    """kvs_attn_decode with the partials in the library's device scratch:
    the caller passes the output buffer; nothing is allocated."""
    _check(lib().kvs_attn_decode_noalloc(plan.handle, ctypes.byref(cache.struct), layer, _ptr(q),
                                         _ptr(seq_len), q.shape[0], max_seq_len, n_splits,
                                         _ptr(out), _dtype_code(out.dtype), _stream(stream)))
    return out


def kvs_attn_decode_stats(plan: Plan, cache: Cache, layer: int, q: torch.Tensor,
                          seq_len: torch.Tensor, max_seq_len: int,
                          out: Optional[torch.Tensor] = None, stats: Optional[torch.Tensor] = None,
                          out_dtype=torch.float32, n_splits: int = 0,
                          workspace: Optional[torch.Tensor] = None, stream=None):
    """Factorized decode attention of ``layer`` plus per (sequence, query
    head) attention statistics: returns (out [B, Hq, hd], stats [B, Hq, 2] =
    entropy in nats, peak probability)."""
    B, Hq = q.shape[0], q.shape[1]
    if n_splits == 0:
        n_splits = kvs_decode_splits(plan, B, max_seq_len)
    if workspace is None:
        workspace = torch.zeros(kvs_decode_workspace_size(plan, B, n_splits), dtype=torch.uint8,
                                device=q.device)
    if out is None:
        out = torch.empty(q.shape, dtype=out_dtype, device=q.device)
    if stats is None:
        stats = torch.empty((B, Hq, 2), dtype=torch.float32, device=q.device)
    _check(lib().kvs_attn_decode_stats(plan.handle, ctypes.byref(cache.struct), layer, _ptr(q),
                                       _ptr(seq_len), B, max_seq_len, n_splits, _ptr(out),
                                       _dtype_code(out.dtype), _ptr(stats), _ptr(workspace),
                                       workspace.numel(), _stream(stream)))
    return out, stats


def kvs_route_ranks(plan: Plan, stats: torch.Tensor, n_keys: torch.Tensor, router: kvs_router,
                    rank_out: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """Residual rank [B] (uint8) of each sequence's current token from
    statistics [n_sets, B, Hq, 2] (or [B, Hq, 2]) and the keys each query saw."""
    st = stats if stats.dim() == 4 else stats.unsqueeze(0)
    n_sets, B = st.shape[0], st.shape[1]
    if rank_out is None:
        rank_out = torch.empty(B, dtype=torch.uint8, device=stats.device)
    _check(lib().kvs_route_ranks(plan.handle, _ptr(st), n_sets, _ptr(n_keys), B,
                                 ctypes.byref(router), _ptr(rank_out), _stream(stream)))
    return rank_out


def _event_handle(ev, stream) -> Optional[int]:
    if ev is None:
        return None
    if not ev.cuda_event:            # torch creates the event on its first record
        ev.record(stream)
    return ev.cuda_event


def kvs_time_next_launch(start, stop, stream=None) -> None:
    """Time the main kernel of this thread's next attention call with two
    torch.cuda.Event objects (created with enable_timing=True): start.elapsed_time(stop)
    is then that kernel's duration.  None, None disarms."""
    s = stream if stream is not None else torch.cuda.current_stream()
    _check(lib().kvs_time_next_launch(_event_handle(start, s), _event_handle(stop, s)))


def kvs_attn_prefill_chunk(plan: Plan, cache: Cache, layer: int, q: torch.Tensor,
                           seq_len: torch.Tensor, causal: bool = True,
                           out: Optional[torch.Tensor] = None, out_dtype=torch.float32,
                           stream=None) -> torch.Tensor:
    """Prefill-chunk attention of ``layer``: q [B, n, Hq, hd] -> out [B, n, Hq, hd]."""
    B, n = q.shape[0], q.shape[1]
    if out is None:
        out = torch.empty(q.shape, dtype=out_dtype, device=q.device)
    _check(lib().kvs_attn_prefill_chunk(plan.handle, ctypes.byref(cache.struct), layer, _ptr(q),
                                        n, _ptr(seq_len), B, int(bool(causal)), _ptr(out),
                                        _dtype_code(out.dtype), _stream(stream)))
    return out


def make_config(n_layers, n_q_heads, n_kv_heads, head_dim, dtype, max_batch, max_ctx,
                kind=KVS_DENSE, basis_rank=0, resid_rank_max=0) -> kvs_config:
    code = dtype if isinstance(dtype, int) else (KVS_F32 if dtype in ("f32", torch.float32)
                                                 else KVS_BF16)
    return kvs_config(n_layers, n_q_heads, n_kv_heads, head_dim, code, kind, basis_rank,
                      resid_rank_max, max_batch, max_ctx)
