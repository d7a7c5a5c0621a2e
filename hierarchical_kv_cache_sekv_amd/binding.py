"""ctypes binding of libsekv (include/sekv.h).

Argument marshalling only: every step of the decode path runs in the HIP
kernels of ``libsekv.so``.  torch is used for device memory and streams.  If
the library is not built, importing this module raises; there is no fallback.
"""
from __future__ import annotations

import ctypes
import dataclasses
import os
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.environ.get("SEKV_LIB") or os.path.join(_HERE, "libsekv.so")  # SEKV_LIB: load another build

SEKV_OK, SEKV_EINVAL, SEKV_ESHAPE, SEKV_ECAPACITY, SEKV_EHIP, SEKV_ENOMEM = range(6)
SEKV_F32, SEKV_BF16 = 0, 1
STATUS_NAMES = {0: "SEKV_OK", 1: "SEKV_EINVAL", 2: "SEKV_ESHAPE", 3: "SEKV_ECAPACITY", 4: "SEKV_EHIP", 5: "SEKV_ENOMEM"}

EXPORTS = [
    "sekv_ctx_create", "sekv_ctx_destroy", "sekv_last_error", "sekv_capacities", "sekv_plan_spans",
    "sekv_build_spans", "sekv_route_workspace_bytes", "sekv_route", "sekv_reconstruct",
    "sekv_decode_workspace_bytes", "sekv_decode_host_workspace_bytes", "sekv_mixed_attention_decode",
    "sekv_profile_enable", "sekv_profile_read", "sekv_ctx_set_split", "sekv_ctx_set_fetch_mode",
    "sekv_ctx_inject_fault", "sekv_profile_read_host", "sekv_route_noalloc", "sekv_dense_workspace_bytes",
    "sekv_dense_attention_decode", "sekv_decode_step", "sekv_profile_read_overlap", "sekv_append_workspace_bytes",
    "sekv_append_token", "sekv_ctx_set_build_mode", "sekv_factor_cache_create", "sekv_factor_cache_destroy",
    "sekv_factor_cache_invalidate", "sekv_factor_cache_stats", "sekv_factor_cache_lookup",
    "sekv_cached_decode_workspace_bytes", "sekv_cached_decode_host_workspace_bytes", "sekv_cached_attention_decode",
    "sekv_profile_read_fill",
]
CACHE_HIT, CACHE_FILL, CACHE_BYPASS = 0, 1, 2
CACHE_PAGE_BYTES = 2 << 20
SEKV_FETCH_STAGED, SEKV_FETCH_DIRECT = 0, 1
SEKV_FAULT_NONE, SEKV_FAULT_GATHER = 0, 1
SEKV_BUILD_DEVICE, SEKV_BUILD_HOST = 0, 1


class SekvError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {msg}")
        self.status = status


class Config(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "batch", "n_ctx", "n_q_heads", "n_kv_heads", "head_dim", "n_sink", "n_recent", "min_span",
        "max_span", "dtype", "factors_on_host", "rank_cap", "basis", "route_keys", "sealed", "n_ctx_max")]


_p = ctypes.c_void_p


class CacheStats(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int64) for n in (
        "lookups", "hits", "fills", "bypasses", "evictions", "bytes_hit", "bytes_filled", "bytes_bypassed",
        "resident_blocks", "resident_bytes", "pages_used", "pages_total")]

    def as_dict(self) -> dict:
        return {n: int(getattr(self, n)) for n, _ in self._fields_}


class Spans(ctypes.Structure):
    _fields_ = [
        ("seg_cap", ctypes.c_int32), ("full_cap", ctypes.c_int32),
        ("n_seg_host", _p), ("n_full_host", _p), ("seg_off", _p), ("rank", _p),
        ("full_k", _p), ("full_v", _p), ("sum_k", _p), ("sum_v", _p), ("rho", _p),
        ("fac_off", _p), ("sg_off", _p), ("fac", _p), ("sg", _p),
        ("fac_elems", ctypes.c_int64), ("sg_elems", ctypes.c_int64),
        ("seg_off_host", _p), ("rank_host", _p), ("fac_off_host", _p), ("sg_off_host", _p),
        ("key_scale", _p), ("fold", _p),
    ]


def _load():
    # torch ships its own HIP runtime; load it first so libsekv binds to that one
    # instance (its DT_NEEDED libamdhip64.so.7 then resolves to the loaded copy)
    # instead of bringing a second runtime into the process.
    import torch  # noqa: F401
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run `python -m hierarchical_kv_cache_sekv_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    S, C = ctypes.POINTER(Spans), ctypes.POINTER(Config)
    i32, i64, sz = ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
    sig = {
        "sekv_ctx_create": (i32, [ctypes.c_int, ctypes.POINTER(_p)]),
        "sekv_ctx_destroy": (None, [_p]),
        "sekv_last_error": (ctypes.c_char_p, []),
        "sekv_capacities": (i32, [C, ctypes.POINTER(i32), ctypes.POINTER(i32)]),
        "sekv_plan_spans": (i32, [C, _p, _p, _p, _p, _p, _p, _p, _p, _p, ctypes.POINTER(i64), ctypes.POINTER(i64)]),
        "sekv_build_spans": (i32, [_p, C, _p, _p, _p, _p, _p, i32, S, _p]),
        "sekv_route_workspace_bytes": (sz, [C, S]),
        "sekv_route": (i32, [_p, C, S, _p, _p, _p, _p, _p, _p, sz, _p]),
        "sekv_route_noalloc": (i32, [_p, C, S, _p, _p, _p, _p, _p, _p]),
        "sekv_dense_workspace_bytes": (sz, [_p, C]),
        "sekv_dense_attention_decode": (i32, [_p, C, _p, _p, _p, _p, _p, sz, _p]),
        "sekv_reconstruct": (i32, [_p, C, S, _p, _p, _p, _p, _p, _p]),
        "sekv_decode_workspace_bytes": (sz, [_p, C, S]),
        "sekv_decode_host_workspace_bytes": (sz, [_p, C, S]),
        "sekv_ctx_set_split": (i32, [_p, i32]),
        "sekv_ctx_set_fetch_mode": (i32, [_p, i32]),
        "sekv_ctx_inject_fault": (i32, [_p, i32]),
        "sekv_ctx_set_build_mode": (i32, [_p, i32]),
        "sekv_profile_read_host": (i32, [_p] + [ctypes.POINTER(ctypes.c_double)] * 3 + [ctypes.POINTER(i64)]),
        "sekv_mixed_attention_decode": (i32, [_p, C, S, _p, _p, _p, _p, _p, _p, sz, _p, sz, _p, _p]),
        "sekv_profile_enable": (i32, [_p, i32]),
        "sekv_profile_read": (i32, [_p] + [ctypes.POINTER(ctypes.c_double), ctypes.POINTER(i64)] * 3),
        "sekv_profile_read_overlap": (i32, [_p, ctypes.POINTER(ctypes.c_double), ctypes.POINTER(i64)]),
        "sekv_profile_read_fill": (i32, [_p, ctypes.POINTER(ctypes.c_double), ctypes.POINTER(i64)]),
        "sekv_factor_cache_create": (i32, [_p, sz, i32, ctypes.POINTER(_p)]),
        "sekv_factor_cache_destroy": (None, [_p]),
        "sekv_factor_cache_invalidate": (i32, [_p, i32]),
        "sekv_factor_cache_stats": (i32, [_p, ctypes.POINTER(CacheStats), i32]),
        "sekv_factor_cache_lookup": (i32, [_p, i32, C, S, _p, _p, _p, _p]),
        "sekv_cached_decode_workspace_bytes": (sz, [_p, C, S]),
        "sekv_cached_decode_host_workspace_bytes": (sz, [_p, C, S]),
        "sekv_cached_attention_decode": (i32, [_p, _p, i32, C, S, _p, _p, _p, _p, _p, _p, sz, _p, sz, _p, _p]),
        "sekv_decode_step": (i32, [_p, C, S, _p, _p, _p, _p, _p, _p, _p, sz, _p, sz, _p]),
        "sekv_append_workspace_bytes": (sz, [C, S]),
        "sekv_append_token": (i32, [_p, C, S, _p, _p, _p, i32, _p, _p, _p, i32, _p, ctypes.POINTER(i64),
                                    ctypes.POINTER(i64), _p, _p, sz, _p]),
    }
    for name, (res, args) in sig.items():
        f = getattr(lib, name)
        f.restype = res
        f.argtypes = args
    return lib


LIB = _load()


def last_error() -> str:
    return LIB.sekv_last_error().decode()


def _check(status: int):
    if status != SEKV_OK:
        raise SekvError(status, last_error())


def _ptr(x) -> Optional[int]:
    """Address of a torch tensor or numpy array (None for None)."""
    if x is None:
        return None
    if isinstance(x, np.ndarray):
        assert x.flags["C_CONTIGUOUS"]
        return x.ctypes.data
    assert x.is_contiguous()
    return x.data_ptr()


def make_config(w, factors_on_host: Optional[bool] = None) -> Config:
    """Config from a workload description (any object with the workload fields;
    the reading-variant fields rank_cap, basis and route_keys default to the
    default readings)."""
    return Config(w.batch, w.n_ctx, w.n_q_heads, w.n_kv_heads, w.head_dim, w.n_sink, w.n_recent,
                  w.min_span, w.max_span, SEKV_BF16 if w.dtype == "bf16" else SEKV_F32,
                  int(w.factors_on_host if factors_on_host is None else factors_on_host),
                  int(getattr(w, "rank_cap", "full") == "half"), int(getattr(w, "basis", "joint") == "separate"),
                  int(getattr(w, "route_keys", "rho") == "folded"), int(getattr(w, "sealed", False)),
                  int(getattr(w, "n_ctx_max", 0)))


def capacities(cfg: Config):
    a, b = ctypes.c_int32(), ctypes.c_int32()
    _check(LIB.sekv_capacities(ctypes.byref(cfg), ctypes.byref(a), ctypes.byref(b)))
    return a.value, b.value


@dataclasses.dataclass
class Plan:
    n_seg: np.ndarray
    n_full: np.ndarray
    seg_off: np.ndarray
    rank: np.ndarray
    fac_off: np.ndarray
    sg_off: np.ndarray
    fac_elems: int
    sg_elems: int


def plan_spans(cfg: Config, surprisal: np.ndarray, thr: np.ndarray, rank_req: np.ndarray) -> Plan:
    """Host-only segmentation and pool layout (sekv_plan_spans)."""
    B, Hkv = cfg.batch, cfg.n_kv_heads
    cap, _ = capacities(cfg)
    s = np.ascontiguousarray(surprisal, np.float32)
    t = np.ascontiguousarray(thr, np.float32)
    rr = np.ascontiguousarray(rank_req, np.int32)
    assert s.shape == (B, cfg.n_ctx) and t.shape == (B,) and rr.shape == (B, cap)
    n_seg = np.zeros(B, np.int32)
    n_full = np.zeros(B, np.int32)
    seg_off = np.zeros((B, cap + 1), np.int32)
    rank = np.zeros((B, cap), np.int32)
    fac_off = np.zeros((B, Hkv, cap), np.int64)
    sg_off = np.zeros((B, Hkv, cap), np.int64)
    fe, ge = ctypes.c_int64(), ctypes.c_int64()
    _check(LIB.sekv_plan_spans(ctypes.byref(cfg), _ptr(s), _ptr(t), _ptr(rr), _ptr(n_seg), _ptr(n_full),
                               _ptr(seg_off), _ptr(rank), _ptr(fac_off), _ptr(sg_off), ctypes.byref(fe),
                               ctypes.byref(ge)))
    return Plan(n_seg, n_full, seg_off, rank, fac_off, sg_off, fe.value, ge.value)


class Context:
    def __init__(self, device: int = 0):
        h = _p()
        _check(LIB.sekv_ctx_create(device, ctypes.byref(h)))
        self.handle = h
        self.device = device

    def profile(self, enable: bool):
        _check(LIB.sekv_profile_enable(self.handle, int(enable)))

    def profile_read(self):
        """{kernel: (total_ms, launches)} for "route", "full", "expand" and
        "overlap" (decode_step's full-resolution pass) since the last read."""
        ms = [ctypes.c_double() for _ in range(3)]
        n = [ctypes.c_int64() for _ in range(3)]
        _check(LIB.sekv_profile_read(self.handle, ctypes.byref(ms[0]), ctypes.byref(n[0]), ctypes.byref(ms[1]),
                                     ctypes.byref(n[1]), ctypes.byref(ms[2]), ctypes.byref(n[2])))
        res = {k: (ms[i].value, n[i].value) for i, k in enumerate(("route", "full", "expand"))}
        m1, n1 = ctypes.c_double(), ctypes.c_int64()
        _check(LIB.sekv_profile_read_overlap(self.handle, ctypes.byref(m1), ctypes.byref(n1)))
        res["overlap"] = (m1.value, n1.value)
        _check(LIB.sekv_profile_read_fill(self.handle, ctypes.byref(m1), ctypes.byref(n1)))
        res["fill"] = (m1.value, n1.value)
        return res

    def set_split(self, entries: int):
        """Full-resolution entries per split-K chunk (0: the library chooses)."""
        _check(LIB.sekv_ctx_set_split(self.handle, int(entries)))

    def set_fetch_mode(self, mode: int):
        _check(LIB.sekv_ctx_set_fetch_mode(self.handle, int(mode)))

    def set_build_mode(self, mode: int):
        """Where sekv_build_spans works: SEKV_BUILD_DEVICE (default) or SEKV_BUILD_HOST."""
        _check(LIB.sekv_ctx_set_build_mode(self.handle, int(mode)))

    def inject_fault(self, fault: int):
        _check(LIB.sekv_ctx_inject_fault(self.handle, int(fault)))

    def host_timing(self):
        """Per-call microseconds of the staged host-resident decode's host
        phases since the last read: wait for the list, gather, whole call."""
        ms = [ctypes.c_double() for _ in range(3)]
        n = ctypes.c_int64()
        _check(LIB.sekv_profile_read_host(self.handle, ctypes.byref(ms[0]), ctypes.byref(ms[1]), ctypes.byref(ms[2]),
                                          ctypes.byref(n)))
        k = max(n.value, 1)
        return {"calls": n.value, "wait_us": ms[0].value * 1e3 / k, "gather_us": ms[1].value * 1e3 / k,
                "call_us": ms[2].value * 1e3 / k}

    def close(self):
        if self.handle:
            LIB.sekv_ctx_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def _torch():
    import torch
    return torch


class SpanCache:
    """Caller-owned span cache: torch device tensors plus the host plan arrays.

    Element arrays use torch.bfloat16 (bit-identical to the raw bf16 the
    kernels read) or torch.float32.  With factors_on_host the two factor pools
    are pinned host tensors.
    """

    def __init__(self, cfg: Config, plan: Plan, device="cuda", fac_capacity: int = 0, sg_capacity: int = 0):
        """fac_capacity / sg_capacity: pool elements to allocate (at least the
        plan's; more leaves room for spans sealed during decode)."""
        torch = _torch()
        self.cfg = cfg
        self.plan = plan
        self.seg_cap, self.full_cap = capacities(cfg)
        B, Hkv, D = cfg.batch, cfg.n_kv_heads, cfg.head_dim
        et = torch.bfloat16 if cfg.dtype == SEKV_BF16 else torch.float32
        self.elem = et
        dev = torch.device(device)
        self.seg_off = torch.from_numpy(plan.seg_off).to(dev)
        self.rank = torch.from_numpy(plan.rank).to(dev)
        self.fac_off = torch.from_numpy(plan.fac_off).to(dev)
        self.sg_off = torch.from_numpy(plan.sg_off).to(dev)
        self.full_k = torch.zeros((B, Hkv, self.full_cap, D), dtype=et, device=dev)
        self.full_v = torch.zeros((B, Hkv, -(-self.full_cap // 32), D, 32), dtype=et, device=dev)
        self.sum_k = torch.zeros((B, Hkv, self.seg_cap, D), dtype=et, device=dev)
        self.sum_v = torch.zeros((B, Hkv, -(-self.seg_cap // 32), D, 32), dtype=et, device=dev)
        self.rho = torch.zeros_like(self.sum_k)
        self.key_scale = torch.zeros((B, Hkv, self.seg_cap), dtype=torch.float32, device=dev)
        self.fold = torch.zeros((Hkv, D, D), dtype=torch.float64, device=dev)
        nf = max(plan.fac_elems, fac_capacity, 8)
        ng = max(plan.sg_elems, sg_capacity, 8)
        self.fac_used, self.sg_used = plan.fac_elems, plan.sg_elems
        if cfg.factors_on_host:
            self.fac = torch.zeros(nf, dtype=et, pin_memory=True)
            self.sg = torch.zeros(ng, dtype=torch.float32, pin_memory=True)
        else:
            self.fac = torch.zeros(nf, dtype=et, device=dev)
            self.sg = torch.zeros(ng, dtype=torch.float32, device=dev)
        self._host = [np.ascontiguousarray(a) for a in (plan.n_seg, plan.n_full, plan.seg_off, plan.rank,
                                                          plan.fac_off, plan.sg_off)]

    def struct(self) -> Spans:
        n_seg, n_full, seg_off, rank, fac_off, sg_off = self._host
        return Spans(self.seg_cap, self.full_cap, _ptr(n_seg), _ptr(n_full), _ptr(self.seg_off), _ptr(self.rank),
                     _ptr(self.full_k), _ptr(self.full_v), _ptr(self.sum_k), _ptr(self.sum_v), _ptr(self.rho),
                     _ptr(self.fac_off), _ptr(self.sg_off), _ptr(self.fac), _ptr(self.sg),
                     self.fac.numel(), self.sg.numel(), _ptr(seg_off), _ptr(rank), _ptr(fac_off), _ptr(sg_off),
                     _ptr(self.key_scale), _ptr(self.fold))

    def clone(self) -> "SpanCache":
        """Independent copy at new addresses (same contents)."""
        new = object.__new__(SpanCache)
        new.__dict__.update(self.__dict__)
        for name in ("seg_off", "rank", "fac_off", "sg_off", "full_k", "full_v", "sum_k", "sum_v", "rho",
                     "key_scale", "fold"):
            setattr(new, name, getattr(self, name).clone())
        if self.cfg.factors_on_host:
            new.fac = self.fac.clone().pin_memory()
            new.sg = self.sg.clone().pin_memory()
        else:
            new.fac = self.fac.clone()
            new.sg = self.sg.clone()
        return new

    def device_bytes(self) -> int:
        n = 0
        names = ["seg_off", "rank", "fac_off", "sg_off", "full_k", "full_v", "sum_k", "sum_v"]
        names += ["key_scale", "fold"] if self.cfg.route_keys else ["rho"]
        for name in names:
            t = getattr(self, name)
            n += t.numel() * t.element_size()
        if not self.cfg.factors_on_host:
            n += self.fac.numel() * self.fac.element_size() + self.sg.numel() * 4
        return n


def _stream_handle(stream) -> Optional[int]:
    torch = _torch()
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream


def build_spans(ctx: Context, cache: SpanCache, k, v, surprisal: np.ndarray, route_proj: np.ndarray,
                gate: np.ndarray, stream=None):
    """sekv_build_spans: fill ``cache`` from device K/V [B][Hkv][T][d]."""
    cfg = cache.cfg
    s = np.ascontiguousarray(surprisal, np.float32)
    P = np.ascontiguousarray(route_proj, np.float32)
    g = np.ascontiguousarray(gate, np.float32)
    assert g.shape[:3] == (cfg.batch, cfg.n_kv_heads, cache.seg_cap)
    st = cache.struct()
    _check(LIB.sekv_build_spans(ctx.handle, ctypes.byref(cfg), _ptr(k), _ptr(v), _ptr(s), _ptr(P), _ptr(g),
                                g.shape[3], ctypes.byref(st), _stream_handle(stream)))


def append_workspace(cache: SpanCache, device="cuda"):
    torch = _torch()
    n = LIB.sekv_append_workspace_bytes(ctypes.byref(cache.cfg), ctypes.byref(cache.struct()))
    return torch.zeros(max(n, 256), dtype=torch.uint8, device=device)


def append_token(ctx: Context, cache: SpanCache, k_new, v_new, surprisal: np.ndarray, thr: np.ndarray,
                 route_proj_dev, gate: np.ndarray, rank_req: np.ndarray, ws, stream=None) -> np.ndarray:
    """sekv_append_token: the cache (sealed layout of cache.cfg.n_ctx tokens)
    grows by one token; k_new, v_new [B][Hkv][d] device; surprisal [B][>= n_ctx
    + 1] host; route_proj_dev [Hkv][d][d] f32 device.  Advances cache.cfg.n_ctx
    and the pools' use; returns the per-sequence sealed flags."""
    cfg = cache.cfg
    s = np.ascontiguousarray(surprisal, np.float32)
    t = np.ascontiguousarray(thr, np.float32)
    g = np.ascontiguousarray(gate, np.float32)
    rr = np.ascontiguousarray(rank_req, np.int32)
    assert g.shape[:3] == (cfg.batch, cfg.n_kv_heads, cache.seg_cap) and rr.shape == (cfg.batch, cache.seg_cap)
    fu, gu = ctypes.c_int64(cache.fac_used), ctypes.c_int64(cache.sg_used)
    sealed = np.zeros(cfg.batch, np.int32)
    st = cache.struct()
    _check(LIB.sekv_append_token(ctx.handle, ctypes.byref(cfg), ctypes.byref(st), _ptr(k_new), _ptr(v_new), _ptr(s),
                                 s.shape[1], _ptr(t), _ptr(route_proj_dev), _ptr(g), g.shape[3], _ptr(rr),
                                 ctypes.byref(fu), ctypes.byref(gu), _ptr(sealed), _ptr(ws), ws.numel(),
                                 _stream_handle(stream)))
    cache.fac_used, cache.sg_used = fu.value, gu.value
    cfg.n_ctx += 1
    return sealed


class RouteOut:
    def __init__(self, cfg: Config, seg_cap: int, device="cuda"):
        torch = _torch()
        B, Hkv = cfg.batch, cfg.n_kv_heads
        self.exp_list = torch.zeros((B, Hkv, seg_cap), dtype=torch.int32, device=device)
        self.exp_mask = torch.zeros((B, Hkv, seg_cap), dtype=torch.uint8, device=device)
        self.exp_count = torch.zeros((B, Hkv), dtype=torch.int32, device=device)


def route_workspace(cache: SpanCache, device="cuda"):
    """Zero-filled route workspace (sekv_route leaves it zero after each call)."""
    torch = _torch()
    n = LIB.sekv_route_workspace_bytes(ctypes.byref(cache.cfg), ctypes.byref(cache.struct()))
    return torch.zeros(max(n, 256), dtype=torch.uint8, device=device)


def route(ctx: Context, cache: SpanCache, q, theta, out: RouteOut, ws, stream=None, spans: Optional[Spans] = None):
    """sekv_route: q [B][Hq][d] (cache dtype), theta [B][Hq] f32, all device."""
    st = spans if spans is not None else cache.struct()
    _check(LIB.sekv_route(ctx.handle, ctypes.byref(cache.cfg), ctypes.byref(st), _ptr(q), _ptr(theta),
                          _ptr(out.exp_list), _ptr(out.exp_mask), _ptr(out.exp_count), _ptr(ws),
                          ws.numel(), _stream_handle(stream)))


def route_noalloc(ctx: Context, cache: SpanCache, q, theta, out: RouteOut, stream=None,
                  spans: Optional[Spans] = None):
    """sekv_route_noalloc: like route(), with the library's static route state
    instead of a workspace (nothing is allocated by the call)."""
    st = spans if spans is not None else cache.struct()
    _check(LIB.sekv_route_noalloc(ctx.handle, ctypes.byref(cache.cfg), ctypes.byref(st), _ptr(q), _ptr(theta),
                                  _ptr(out.exp_list), _ptr(out.exp_mask), _ptr(out.exp_count),
                                  _stream_handle(stream)))


def reconstruct(ctx: Context, cache: SpanCache, out: RouteOut, stream=None):
    """sekv_reconstruct: returns (tok_off, k_out, v_out) device tensors."""
    torch = _torch()
    cfg = cache.cfg
    B, Hkv, T, D = cfg.batch, cfg.n_kv_heads, cfg.n_ctx, cfg.head_dim
    dev = out.exp_list.device
    tok_off = torch.zeros((B, Hkv, cache.seg_cap + 1), dtype=torch.int32, device=dev)
    k_out = torch.zeros((B, Hkv, T, D), dtype=torch.float32, device=dev)
    v_out = torch.zeros_like(k_out)
    _check(LIB.sekv_reconstruct(ctx.handle, ctypes.byref(cfg), ctypes.byref(cache.struct()), _ptr(out.exp_list),
                                _ptr(out.exp_count), _ptr(tok_off), _ptr(k_out), _ptr(v_out), _stream_handle(stream)))
    return tok_off, k_out, v_out


class DecodeWorkspace:
    """Device (and, for the staged host-resident fetch, pinned host) workspace
    sized for ``ctx``'s split and fetch mode (ctx None: the defaults)."""

    def __init__(self, cache: SpanCache, device="cuda", ctx: Optional["Context"] = None):
        torch = _torch()
        st = cache.struct()
        h = ctx.handle if ctx is not None else None
        nd = LIB.sekv_decode_workspace_bytes(h, ctypes.byref(cache.cfg), ctypes.byref(st))
        nh = LIB.sekv_decode_host_workspace_bytes(h, ctypes.byref(cache.cfg), ctypes.byref(st))
        self.dev = torch.empty(max(nd, 256), dtype=torch.uint8, device=device)
        self.host = torch.empty(nh, dtype=torch.uint8, pin_memory=True) if nh > 0 else None


def decode(ctx: Context, cache: SpanCache, q, route_out: RouteOut, out, ws: DecodeWorkspace, stream=None,
           copy_stream=None, spans: Optional[Spans] = None):
    """sekv_mixed_attention_decode: out [B][Hq][d] f32 device."""
    st = spans if spans is not None else cache.struct()
    host_ptr = _ptr(ws.host) if ws.host is not None else None
    host_n = ws.host.numel() if ws.host is not None else 0
    cs = copy_stream.cuda_stream if copy_stream is not None else None
    _check(LIB.sekv_mixed_attention_decode(ctx.handle, ctypes.byref(cache.cfg), ctypes.byref(st), _ptr(q),
                                           _ptr(route_out.exp_list), _ptr(route_out.exp_mask),
                                           _ptr(route_out.exp_count), _ptr(out), _ptr(ws.dev), ws.dev.numel(),
                                           host_ptr, host_n, _stream_handle(stream), cs))


def decode_step(ctx: Context, cache: SpanCache, q, theta, route_out: RouteOut, out, route_ws, ws: DecodeWorkspace,
                stream=None, spans: Optional[Spans] = None):
    """sekv_decode_step: route + attention of one step, the full-resolution
    pass on the context's second stream beside the route."""
    st = spans if spans is not None else cache.struct()
    _check(LIB.sekv_decode_step(ctx.handle, ctypes.byref(cache.cfg), ctypes.byref(st), _ptr(q), _ptr(theta),
                                _ptr(route_out.exp_list), _ptr(route_out.exp_mask), _ptr(route_out.exp_count),
                                _ptr(out), _ptr(route_ws), route_ws.numel(), _ptr(ws.dev), ws.dev.numel(),
                                _stream_handle(stream)))


class FactorCache:
    """sekv_factor_cache: an HBM arena of ``nbytes`` (whole 2 MiB pages, split
    evenly among ``partitions``; 0: the library's default) for host-resident
    factor blocks, shared by the layers of a model.  ctx None: bookkeeping
    only (``lookup`` works, the cached decode does not)."""

    def __init__(self, ctx: Optional[Context], nbytes: int, partitions: int = 0):
        h = _p()
        _check(LIB.sekv_factor_cache_create(ctx.handle if ctx is not None else None, int(nbytes), int(partitions),
                                            ctypes.byref(h)))
        self.handle = h

    def stats(self, reset: bool = False) -> dict:
        st = CacheStats()
        _check(LIB.sekv_factor_cache_stats(self.handle, ctypes.byref(st), int(reset)))
        return st.as_dict()

    def invalidate(self, layer: int = -1):
        _check(LIB.sekv_factor_cache_invalidate(self.handle, int(layer)))

    def lookup(self, layer: int, cfg: Config, spans: Spans, exp_list: np.ndarray, exp_count: np.ndarray):
        """Host bookkeeping of one call: (status, offset), shaped like exp_list."""
        exp_list = np.ascontiguousarray(exp_list, dtype=np.int32)
        exp_count = np.ascontiguousarray(exp_count, dtype=np.int32)
        status = np.full(exp_list.shape, -1, np.int32)
        offset = np.full(exp_list.shape, -1, np.int64)
        _check(LIB.sekv_factor_cache_lookup(self.handle, int(layer), ctypes.byref(cfg), ctypes.byref(spans),
                                            _ptr(exp_list), _ptr(exp_count), _ptr(status), _ptr(offset)))
        return status, offset

    def close(self):
        if self.handle:
            LIB.sekv_factor_cache_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


class CachedDecodeWorkspace:
    """Device and pinned host workspaces of sekv_cached_attention_decode."""

    def __init__(self, cache: SpanCache, device="cuda", ctx: Optional[Context] = None):
        torch = _torch()
        st = cache.struct()
        h = ctx.handle if ctx is not None else None
        nd = LIB.sekv_cached_decode_workspace_bytes(h, ctypes.byref(cache.cfg), ctypes.byref(st))
        nh = LIB.sekv_cached_decode_host_workspace_bytes(h, ctypes.byref(cache.cfg), ctypes.byref(st))
        self.dev = torch.empty(max(nd, 256), dtype=torch.uint8, device=device)
        self.host = torch.empty(max(nh, 256), dtype=torch.uint8, pin_memory=True)


def cached_decode(ctx: Context, fcache: FactorCache, layer: int, cache: SpanCache, q, route_out: RouteOut, out,
                  ws: CachedDecodeWorkspace, stream=None, copy_stream=None, spans: Optional[Spans] = None):
    """sekv_cached_attention_decode: one layer's decode through the factor cache."""
    st = spans if spans is not None else cache.struct()
    cs = copy_stream.cuda_stream if copy_stream is not None else None
    _check(LIB.sekv_cached_attention_decode(ctx.handle, fcache.handle, int(layer), ctypes.byref(cache.cfg),
                                            ctypes.byref(st), _ptr(q), _ptr(route_out.exp_list),
                                            _ptr(route_out.exp_mask), _ptr(route_out.exp_count), _ptr(out),
                                            _ptr(ws.dev), ws.dev.numel(), _ptr(ws.host), ws.host.numel(),
                                            _stream_handle(stream), cs))


def tile_values_device(v):
    """Device value rows [..., T, d] -> [..., ceil(T/32), d, 32] transposed
    32-token tiles (zero padding): the layout of full_v / sum_v and of the
    dense baseline's values (layout marshalling only)."""
    torch = _torch()
    *lead, T, d = v.shape
    nt = -(-T // 32)
    pad = torch.zeros((*lead, nt * 32, d), dtype=v.dtype, device=v.device)
    pad[..., :T, :] = v
    return pad.view(*lead, nt, 32, d).transpose(-1, -2).contiguous()


def dense_workspace(ctx: Context, cfg: Config, device="cuda"):
    torch = _torch()
    n = LIB.sekv_dense_workspace_bytes(ctx.handle, ctypes.byref(cfg))
    return torch.empty(max(n, 256), dtype=torch.uint8, device=device)


def dense_decode(ctx: Context, cfg: Config, k, v_tiles, q, out, ws, stream=None):
    """sekv_dense_attention_decode: k [B][Hkv][T][d], v_tiles [B][Hkv][ceil(T/32)][d][32]
    (cache dtype), q [B][Hq][d], out [B][Hq][d] f32, all device."""
    _check(LIB.sekv_dense_attention_decode(ctx.handle, ctypes.byref(cfg), _ptr(k), _ptr(v_tiles), _ptr(q), _ptr(out),
                                           _ptr(ws), ws.numel(), _stream_handle(stream)))


# ----------------------------------------------------------------- marshalling
def fac_block_elems(L: int, r: int, d: int, sep: bool = False) -> int:
    """Elements of one span's factor block: Vh_K [r][d] (groups of 8 rotated by
    the row) | U [L][rp] | (separate bases: U_V [L][rp]) | W_V in 16-rank
    column blocks [d][min(16, rp - 16 g)]."""
    rp = (r + 7) // 8 * 8
    return r * d + L * rp * (2 if sep else 1) + d * rp


def sg_entry_elems(r: int, sep: bool = False) -> int:
    """Floats of one span's sigma|gate entry: sigma [rq] | gate [rq], rq = ceil(r/4)*4
    (separate bases: sigma_K | gate | sigma_V | gate)."""
    return (4 if sep else 2) * ((r + 3) // 4 * 4)


def _vk_rotate(vk: np.ndarray) -> np.ndarray:
    """[r][d] key part -> ABI order: row k's groups of 8 rotated by k."""
    r, d = vk.shape
    ng = d // 8
    out = np.empty_like(vk)
    for k in range(r):
        g = vk[k].reshape(ng, 8)
        out[k] = g[(np.arange(ng) - k) % ng].reshape(-1)   # position p holds group (p - k) mod ng
    return out


def _vk_unrotate(rot: np.ndarray) -> np.ndarray:
    r, d = rot.shape
    ng = d // 8
    out = np.empty_like(rot)
    for k in range(r):
        g = rot[k].reshape(ng, 8)
        out[k] = g[(np.arange(ng) + k) % ng].reshape(-1)   # group u sits at position (u + k) mod ng
    return out


def _wv_blocks(wv: np.ndarray) -> np.ndarray:
    """[d][rp] value part -> flat 16-rank column blocks [d][wk] (ABI order)."""
    d, rp = wv.shape
    return np.concatenate([wv[:, k0:min(k0 + 16, rp)].reshape(-1) for k0 in range(0, rp, 16)])


def _wv_unblock(flat: np.ndarray, d: int, rp: int) -> np.ndarray:
    out = np.zeros((d, rp), flat.dtype)
    o = 0
    for k0 in range(0, rp, 16):
        wk = min(16, rp - k0)
        out[:, k0:k0 + wk] = flat[o:o + d * wk].reshape(d, wk)
        o += d * wk
    return out


def read_factors(cache: "SpanCache", b: int, kv: int, i: int):
    """Factors of span i from a cache's pools (host copies, float64): one basis
    (U [L][r], sigma [r], gate [r], Vh [r][2d]); separate bases ((U_K, sigma_K,
    gate, Vh_K [r][d]), (U_V, sigma_V, gate, Vh_V [r][d]))."""
    plan, D = cache.plan, cache.cfg.head_dim
    sep = bool(cache.cfg.basis)
    so = plan.seg_off[b]
    L = int(so[i + 1] - so[i] - 1)
    r = int(plan.rank[b, i])
    rp = (r + 7) // 8 * 8
    o = int(plan.fac_off[b, kv, i])
    fac = cache.fac[o:o + fac_block_elems(L, r, D, sep)].float().cpu().numpy().astype(np.float64)
    vk = _vk_unrotate(fac[:r * D].reshape(r, D))
    U = fac[r * D:r * D + L * rp].reshape(L, rp)[:, :r]
    w0 = r * D + L * rp * (2 if sep else 1)
    wv = _wv_unblock(fac[w0:], D, rp)[:, :r]
    go = int(plan.sg_off[b, kv, i])
    rq = (r + 3) // 4 * 4
    sg = cache.sg[go:go + sg_entry_elems(r, sep)].float().cpu().numpy().astype(np.float64)
    if not sep:
        return U, sg[:r], sg[rq:rq + r], np.concatenate([vk, wv.T], axis=1)
    Uv = fac[r * D + L * rp:r * D + 2 * L * rp].reshape(L, rp)[:, :r]
    return (U, sg[:r], sg[rq:rq + r], vk), (Uv, sg[2 * rq:2 * rq + r], sg[3 * rq:3 * rq + r], wv.T)


def tile_values(rows: np.ndarray) -> np.ndarray:
    """[..., n, d] value rows -> [..., ceil(n/32), d, 32] transposed 32-entry
    tiles (zero padding), the layout of full_v / sum_v."""
    *lead, n, d = rows.shape
    nt = -(-n // 32)
    pad = np.zeros((*lead, nt * 32, d), rows.dtype)
    pad[..., :n, :] = rows
    return np.ascontiguousarray(np.swapaxes(pad.reshape(*lead, nt, 32, d), -1, -2))


def untile_values(tiles: np.ndarray, n: int) -> np.ndarray:
    """Inverse of tile_values: [..., nt, d, 32] -> [..., n, d]."""
    *lead, nt, d, _ = tiles.shape
    return np.swapaxes(tiles, -1, -2).reshape(*lead, nt * 32, d)[..., :n, :]


def fill_cache(cache: SpanCache, parts) -> None:
    """Copy span-cache contents given as plain per-sequence numpy arrays into
    the ABI layout (layout marshalling only).

    ``parts`` provides, for each sequence b and KV head kv: ``full_k[b][kv]``,
    ``full_v``, ``sum_k``, ``sum_v``, ``rho`` ([n][d] arrays of values that are
    exact in the cache dtype), ``key_scale[b][kv]`` [n] and ``fold[kv]`` [d][d]
    and, for each span i, ``U[b][kv][i]`` [L][r], ``sigma[b][kv][i]`` [r],
    ``gate[b][kv][i]`` [r], ``Vh[b][kv][i]`` ([r][2d] for one basis; [r][d]
    key part for separate bases, with ``U_V``, ``sigma_V``, ``Vh_V`` [r][d]).
    Spans whose U is None are left zero.  The plan of ``cache`` must describe
    the same spans and ranks.
    """
    torch = _torch()
    cfg, plan = cache.cfg, cache.plan
    B, Hkv, D = cfg.batch, cfg.n_kv_heads, cfg.head_dim
    et = cache.elem
    fk = np.zeros((B, Hkv, cache.full_cap, D), np.float32)
    fv = np.zeros_like(fk)
    sk = np.zeros((B, Hkv, cache.seg_cap, D), np.float32)
    sv = np.zeros_like(sk)
    rh = np.zeros_like(sk)
    ks = np.zeros((B, Hkv, cache.seg_cap), np.float32)
    sep = bool(cfg.basis)
    fac = np.zeros(cache.fac.numel(), np.float32)
    sg = np.zeros(cache.sg.numel(), np.float32)
    for b in range(B):
        n = int(plan.n_seg[b])
        so = plan.seg_off[b]
        for kv in range(Hkv):
            nf = parts.full_k[b][kv].shape[0]
            fk[b, kv, :nf] = parts.full_k[b][kv]
            fv[b, kv, :nf] = parts.full_v[b][kv]
            sk[b, kv, :n] = parts.sum_k[b][kv]
            sv[b, kv, :n] = parts.sum_v[b][kv]
            rh[b, kv, :n] = parts.rho[b][kv]
            if getattr(parts, "key_scale", None) is not None:
                ks[b, kv, :n] = parts.key_scale[b][kv]
            for i in range(n):
                if parts.U[b][kv][i] is None:
                    continue
                U = np.asarray(parts.U[b][kv][i], np.float32)
                Vh = np.asarray(parts.Vh[b][kv][i], np.float32)
                L, r = U.shape
                assert L == so[i + 1] - so[i] - 1 and r == plan.rank[b, i]
                rp = (r + 7) // 8 * 8
                o = int(plan.fac_off[b, kv, i])
                fac[o:o + r * D] = _vk_rotate(Vh[:, :D]).reshape(-1)  # key part [r][d], rotated groups
                o += r * D
                for Ub in ([U, np.asarray(parts.U_V[b][kv][i], np.float32)] if sep else [U]):
                    blk = np.zeros((L, rp), np.float32)
                    blk[:, :r] = Ub
                    fac[o:o + L * rp] = blk.reshape(-1)
                    o += L * rp
                wv = np.zeros((D, rp), np.float32)
                wv[:, :r] = np.asarray(parts.Vh_V[b][kv][i], np.float32).T if sep else Vh[:, D:].T
                fac[o:o + D * rp] = _wv_blocks(wv)                  # value part transposed, column blocks
                go = int(plan.sg_off[b, kv, i])
                rq = (r + 3) // 4 * 4
                sg[go:go + r] = parts.sigma[b][kv][i]
                sg[go + rq:go + rq + r] = parts.gate[b][kv][i]
                if sep:
                    sg[go + 2 * rq:go + 2 * rq + r] = parts.sigma_V[b][kv][i]
                    sg[go + 3 * rq:go + 3 * rq + r] = parts.gate[b][kv][i]

    def put(dst, src):
        dst.copy_(torch.from_numpy(src).to(et))

    put(cache.full_k, fk)
    put(cache.full_v, tile_values(fv))
    put(cache.sum_k, sk)
    put(cache.sum_v, tile_values(sv))
    put(cache.rho, rh)
    cache.key_scale.copy_(torch.from_numpy(ks))
    if getattr(parts, "fold", None) is not None:
        cache.fold.copy_(torch.from_numpy(np.ascontiguousarray(np.stack(parts.fold), np.float64)))
    cache.fac.copy_(torch.from_numpy(fac).to(et))
    cache.sg.copy_(torch.from_numpy(sg))


def layout_from_segments(cfg: Config, seg_offs, ranks) -> Plan:
    """Plan (pool layout) for spans given by per-sequence offsets and ranks,
    laid out in (b, kv, span) order like sekv_plan_spans.  Marshalling only."""
    B, Hkv, D, T = cfg.batch, cfg.n_kv_heads, cfg.head_dim, cfg.n_ctx
    cap, _ = capacities(cfg)
    n_seg = np.zeros(B, np.int32)
    n_full = np.zeros(B, np.int32)
    seg_off = np.zeros((B, cap + 1), np.int32)
    rank = np.zeros((B, cap), np.int32)
    fac_off = np.zeros((B, Hkv, cap), np.int64)
    sg_off = np.zeros((B, Hkv, cap), np.int64)
    fo = go = 0
    for b in range(B):
        so = np.asarray(seg_offs[b], np.int64)
        n = len(so) - 1
        n_seg[b] = n
        seg_off[b, :n + 1] = so
        seg_off[b, n + 1:] = so[-1]
        n_full[b] = cfg.n_sink + n + (T - int(so[-1]))
        rank[b, :n] = np.asarray(ranks[b], np.int32)[:n]
        L = so[1:] - so[:-1] - 1
        for kv in range(Hkv):
            for i in range(n):
                r = int(rank[b, i])
                fac_off[b, kv, i] = fo
                sg_off[b, kv, i] = go
                fo += fac_block_elems(int(L[i]), r, D, bool(cfg.basis))
                go += sg_entry_elems(r, bool(cfg.basis))
    return Plan(n_seg, n_full, seg_off, rank, fac_off, sg_off, fo, go)
