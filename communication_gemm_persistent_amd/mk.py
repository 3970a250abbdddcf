"""ctypes binding of libmk (include/mk.h): argument marshalling only.

Every operation runs in the HIP library; this module checks dtypes, shapes and
contiguity of torch tensors, passes their data pointers and the current HIP
stream, and turns status codes into exceptions.  It never computes anything
itself and has no fallback: if libmk.so is missing, load() raises.

bf16 tensors may be torch.bfloat16 or int16 / uint16 bit patterns.  Peer
buffers may live on the GPU or in pinned host memory (pin_memory=True).
"""
from __future__ import annotations

import ctypes
import os
from typing import List, Optional, Sequence, Tuple

import torch

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libmk.so")

MK_OK = 0
MK_ERR_INVALID = 1
MK_ERR_UNSUPPORTED = 2
MK_ERR_OOM = 3
MK_ERR_HIP = 4
MK_ERR_TIMEOUT = 5

OP_AG_GEMM = 0
OP_GEMM_RS = 1
OP_GEMM_AR = 2
OP_MOE = 3
OP_RING_ATTN = 4

F_PRELANDED = 0x1
F_NO_GATE = 0x2
F_STATIC_ROLES = 0x4
F_NO_PEERS = 0x8

MAX_WORLD = 16

# Names declared in include/mk.h (the CPU tests check the library exports them).
EXPORTS = ("mk_create", "mk_destroy", "mk_set_roles", "mk_get_roles", "mk_last_launch",
           "mk_sync", "mk_status_string", "mk_last_error", "mk_ag_gemm", "mk_gemm_rs",
           "mk_gemm_ar", "mk_moe_dispatch_gemm", "mk_moe_dispatch_gemm_combine",
           "mk_ring_attention", "mk_mfma_ceiling", "mk_ag_gemm_noalloc")


class MkError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(msg)
        self.status = status


class _Config(ctypes.Structure):
    _fields_ = [("device", ctypes.c_int), ("spin_timeout_ms", ctypes.c_int),
                ("flags", ctypes.c_uint), ("workspace_bytes", ctypes.c_size_t)]


class Roles(ctypes.Structure):
    _fields_ = [("n_land", ctypes.c_int), ("n_compute", ctypes.c_int), ("n_reduce", ctypes.c_int)]

    def as_tuple(self) -> Tuple[int, int, int]:
        return (self.n_land, self.n_compute, self.n_reduce)


_lib: Optional[ctypes.CDLL] = None
_vp = ctypes.c_void_p
_i = ctypes.c_int
_u = ctypes.c_uint
_pp = ctypes.POINTER(ctypes.c_void_p)


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libmk.so (once).  Raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with "
                           "`python -m communication_gemm_persistent_amd.build`")
    lib = ctypes.CDLL(path)
    lib.mk_create.argtypes = [ctypes.POINTER(_vp), ctypes.POINTER(_Config)]
    lib.mk_destroy.argtypes = [_vp]
    lib.mk_set_roles.argtypes = [_vp, _i, ctypes.POINTER(Roles)]
    lib.mk_get_roles.argtypes = [_vp, _i, ctypes.POINTER(Roles)]
    lib.mk_last_launch.argtypes = [_vp, _i, ctypes.POINTER(Roles), ctypes.POINTER(_i)]
    lib.mk_sync.argtypes = [_vp, _vp]
    lib.mk_status_string.argtypes = [_i]
    lib.mk_status_string.restype = ctypes.c_char_p
    lib.mk_last_error.argtypes = [_vp]
    lib.mk_last_error.restype = ctypes.c_char_p
    lib.mk_ag_gemm.argtypes = [_vp, _vp, _i, _i, _pp, _vp, _vp, _vp, _i, _i, _i, _u]
    lib.mk_gemm_rs.argtypes = [_vp, _vp, _i, _i, _vp, _vp, _pp, _vp, _pp, _i, _i, _i, _u]
    lib.mk_gemm_ar.argtypes = [_vp, _vp, _i, _i, _vp, _vp, _pp, _vp, _pp, _i, _i, _i, _i, _u]
    lib.mk_moe_dispatch_gemm.argtypes = [_vp, _vp, _i, _i, _pp, _pp, _vp, _i, _i, _i, _i, _i, _i,
                                         _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i, _u]
    lib.mk_mfma_ceiling.argtypes = [_vp, _vp, _i, _vp]
    lib.mk_ring_attention.argtypes = [_vp, _vp, _i, _i, _vp, _pp, _pp, _i, _i, _i, _i,
                                      ctypes.c_float, _vp, _vp, _vp, _vp, _u]
    lib.mk_ag_gemm_noalloc.argtypes = [_vp, _i, _i, _pp, _vp, _vp, _vp, _i, _i, _i, _u, _vp]
    lib.mk_moe_dispatch_gemm_combine.argtypes = [
        _vp, _vp, _i, _i, _pp, _pp, _vp, _i, _i, _i, _i, _i, _i, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
        _i, _vp, _pp, _vp, _u]
    for name in EXPORTS:
        if name not in ("mk_status_string", "mk_last_error"):
            getattr(lib, name).restype = _i
    _lib = lib
    return lib


# ---------------------------------------------------------------- marshalling

_BF16 = (torch.bfloat16, torch.int16, torch.uint16)


def _ptr(t: Optional[torch.Tensor], name: str, dtypes, shape=None) -> int:
    if t is None:
        return 0
    if t.dtype not in dtypes:
        raise TypeError(f"{name}: dtype {t.dtype} not in {dtypes}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: shape {tuple(t.shape)} != {tuple(shape)}")
    if not t.is_cuda and not t.is_pinned():
        raise ValueError(f"{name} must be a GPU tensor or pinned host memory")
    return t.data_ptr()


def _ptr_array(ptrs: Sequence[int]):
    arr = (ctypes.c_void_p * max(1, len(ptrs)))()
    for i, p in enumerate(ptrs):
        arr[i] = p or None
    return arr


def _stream(stream, device: int) -> int:
    if stream is None:
        stream = torch.cuda.current_stream(device)
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def ag_gemm_noalloc(shards: Sequence[torch.Tensor], bt: torch.Tensor, c: torch.Tensor,
                    a_gathered: torch.Tensor, rank: int = 0, flags: int = 0, stream=None,
                    status: Optional[torch.Tensor] = None) -> None:
    """mk_ag_gemm_noalloc: AllGather+GEMM on the current device with no handle
    and no allocation (control memory in the library's per-device array).
    status: optional int32 device tensor of >= 2 elements that receives the
    launch's result code and detail.  Calls overlapping on one GPU race."""
    lib = load()
    W = len(shards)
    m_s, k = shards[rank].shape
    n = bt.shape[0]
    sp = [0 if (s is None and q != rank and flags & F_PRELANDED)
          else _ptr(s, f"shards[{q}]", _BF16, (m_s, k)) for q, s in enumerate(shards)]
    if status is not None and (status.dtype != torch.int32 or status.numel() < 2):
        raise ValueError("status must be an int32 tensor of at least 2 elements")
    st = lib.mk_ag_gemm_noalloc(_vp(_stream(stream, torch.cuda.current_device())), W, rank,
                                _ptr_array(sp), _ptr(bt, "bt", _BF16, (n, k)),
                                _ptr(c, "c", _BF16, (W * m_s, n)),
                                _ptr(a_gathered, "a_gathered", _BF16, (W * m_s, k)), m_s, n, k, flags,
                                _ptr(status, "status", (torch.int32,)) if status is not None else None)
    if st != MK_OK:
        raise MkError(st, "mk_ag_gemm_noalloc: " + lib.mk_status_string(st).decode())


class Handle:
    """One libmk handle bound to a device; calls on it must be stream-ordered."""

    def __init__(self, device: int = 0, spin_timeout_ms: int = 0, workspace_bytes: int = 0):
        self.lib = load()
        self.device = device
        h = _vp()
        cfg = _Config(device, spin_timeout_ms, 0, workspace_bytes)
        self._check(self.lib.mk_create(ctypes.byref(h), ctypes.byref(cfg)), "mk_create", None)
        self.h = h

    # -- housekeeping
    def close(self) -> None:
        if getattr(self, "h", None):
            self.lib.mk_destroy(self.h)
            self.h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        self.close()

    def _check(self, st: int, what: str, h) -> None:
        if st != MK_OK:
            detail = self.lib.mk_last_error(h).decode() if h else ""
            msg = self.lib.mk_status_string(st).decode()
            raise MkError(st, f"{what}: {msg}" + (f" ({detail})" if detail else ""))

    def set_roles(self, op: int, n_land: int = -1, n_compute: int = -1, n_reduce: int = -1) -> None:
        r = Roles(n_land, n_compute, n_reduce)
        self._check(self.lib.mk_set_roles(self.h, op, ctypes.byref(r)), "mk_set_roles", self.h)

    def get_roles(self, op: int) -> Tuple[int, int, int]:
        r = Roles()
        self._check(self.lib.mk_get_roles(self.h, op, ctypes.byref(r)), "mk_get_roles", self.h)
        return r.as_tuple()

    def last_launch(self, op: int) -> Tuple[Tuple[int, int, int], int]:
        r = Roles()
        g = _i()
        self._check(self.lib.mk_last_launch(self.h, op, ctypes.byref(r), ctypes.byref(g)),
                    "mk_last_launch", self.h)
        return r.as_tuple(), g.value

    def sync(self, stream=None) -> None:
        self._check(self.lib.mk_sync(self.h, _vp(_stream(stream, self.device))), "mk_sync", self.h)

    # -- operations
    def ag_gemm(self, shards: Sequence[torch.Tensor], bt: torch.Tensor, c: torch.Tensor,
                a_gathered: torch.Tensor, rank: int = 0, flags: int = 0, stream=None) -> None:
        W = len(shards)
        m_s, k = shards[rank].shape
        n = bt.shape[0]
        sp = [0 if (s is None and q != rank and flags & F_PRELANDED)
              else _ptr(s, f"shards[{q}]", _BF16, (m_s, k)) for q, s in enumerate(shards)]
        st = self.lib.mk_ag_gemm(self.h, _vp(_stream(stream, self.device)), W, rank, _ptr_array(sp),
                                 _ptr(bt, "bt", _BF16, (n, k)), _ptr(c, "c", _BF16, (W * m_s, n)),
                                 _ptr(a_gathered, "a_gathered", _BF16, (W * m_s, k)),
                                 m_s, n, k, flags)
        self._check(st, "mk_ag_gemm", self.h)

    def gemm_rs(self, a: torch.Tensor, bt: torch.Tensor, peer_part: Sequence[Optional[torch.Tensor]],
                c_own: torch.Tensor, outbox: Sequence[Optional[torch.Tensor]], rank: int = 0,
                flags: int = 0, stream=None) -> None:
        W = len(peer_part)
        m, k = a.shape
        n = bt.shape[0]
        ms = m // W
        pp = [0 if q == rank or (peer_part[q] is None and flags & F_NO_PEERS)
              else _ptr(peer_part[q], f"peer_part[{q}]", (torch.float32,), (ms, n)) for q in range(W)]
        ob = [0 if q == rank else _ptr(outbox[q], f"outbox[{q}]", _BF16, (ms, n)) for q in range(W)]
        st = self.lib.mk_gemm_rs(self.h, _vp(_stream(stream, self.device)), W, rank,
                                 _ptr(a, "a", _BF16), _ptr(bt, "bt", _BF16, (n, k)), _ptr_array(pp),
                                 _ptr(c_own, "c_own", _BF16, (ms, n)), _ptr_array(ob), m, n, k, flags)
        self._check(st, "mk_gemm_rs", self.h)

    def gemm_ar(self, a: torch.Tensor, bt: torch.Tensor, peer_part: Sequence[Optional[torch.Tensor]],
                c: torch.Tensor, bcast: Sequence[torch.Tensor], rank: int = 0, flags: int = 0,
                stream=None) -> None:
        W = len(peer_part)
        m, k = a.shape
        n = bt.shape[0]
        pp = [0 if q == rank or (peer_part[q] is None and flags & F_NO_PEERS)
              else _ptr(peer_part[q], f"peer_part[{q}]", (torch.float32,), (m, n)) for q in range(W)]
        bc = [_ptr(b, f"bcast[{i}]", _BF16, (m, n)) for i, b in enumerate(bcast)]
        st = self.lib.mk_gemm_ar(self.h, _vp(_stream(stream, self.device)), W, rank,
                                 _ptr(a, "a", _BF16), _ptr(bt, "bt", _BF16, (n, k)), _ptr_array(pp),
                                 _ptr(c, "c", _BF16, (m, n)), _ptr_array(bc), len(bcast), m, n, k,
                                 flags)
        self._check(st, "mk_gemm_ar", self.h)

    def moe_dispatch_gemm(self, x: Sequence[torch.Tensor], logits: Sequence[torch.Tensor],
                          wt: torch.Tensor, E: int, top_k: int, y: torch.Tensor,
                          topk_idx: torch.Tensor, topk_gate: torch.Tensor,
                          slot_token: torch.Tensor, expert_offsets: torch.Tensor,
                          chunk_offsets: torch.Tensor, x_slots: torch.Tensor, rank: int = 0,
                          flags: int = 0, stream=None) -> None:
        S = len(x)
        T, H = x[0].shape
        E_loc, N, _ = wt.shape
        cap = y.shape[0]
        xp = [_ptr(xx, f"x[{s}]", _BF16, (T, H)) for s, xx in enumerate(x)]
        lp = [_ptr(ll, f"logits[{s}]", (torch.float32,), (T, E)) for s, ll in enumerate(logits)]
        i32 = (torch.int32,)
        st = self.lib.mk_moe_dispatch_gemm(
            self.h, _vp(_stream(stream, self.device)), S, rank, _ptr_array(xp), _ptr_array(lp),
            _ptr(wt, "wt", _BF16, (E_loc, N, H)), T, H, N, E, E_loc, top_k,
            _ptr(y, "y", _BF16, (cap, N)), _ptr(topk_idx, "topk_idx", i32, (S * T, top_k)),
            _ptr(topk_gate, "topk_gate", (torch.float32,), (S * T, top_k)),
            _ptr(slot_token, "slot_token", i32, (cap,)),
            _ptr(expert_offsets, "expert_offsets", i32, (E_loc + 1,)),
            _ptr(chunk_offsets, "chunk_offsets", i32, (E_loc, S + 1)),
            _ptr(x_slots, "x_slots", _BF16, (cap, H)), cap, flags)
        self._check(st, "mk_moe_dispatch_gemm", self.h)

    def moe_dispatch_gemm_combine(self, x: Sequence[torch.Tensor], logits: Sequence[torch.Tensor],
                                  wt: torch.Tensor, E: int, top_k: int, y: torch.Tensor,
                                  topk_idx: torch.Tensor, topk_gate: torch.Tensor,
                                  slot_token: torch.Tensor, expert_offsets: torch.Tensor,
                                  chunk_offsets: torch.Tensor, x_slots: torch.Tensor,
                                  y_peer: torch.Tensor, ret: Sequence[Optional[torch.Tensor]],
                                  out: torch.Tensor, rank: int = 0, flags: int = 0,
                                  stream=None) -> None:
        """Dispatch + grouped GEMM as moe_dispatch_gemm, plus the return of
        every remote token's rows into ret[s] ([T * top_k, N]) and the combine
        of this rank's tokens into out ([T, N])."""
        S = len(x)
        T, H = x[0].shape
        E_loc, N, _ = wt.shape
        cap = y.shape[0]
        if len(ret) != S:
            raise ValueError(f"ret has {len(ret)} entries, expected {S}")
        xp = [_ptr(xx, f"x[{s}]", _BF16, (T, H)) for s, xx in enumerate(x)]
        lp = [_ptr(ll, f"logits[{s}]", (torch.float32,), (T, E)) for s, ll in enumerate(logits)]
        rp = [0 if s == rank else _ptr(r, f"ret[{s}]", _BF16, (T * top_k, N))
              for s, r in enumerate(ret)]
        i32 = (torch.int32,)
        st = self.lib.mk_moe_dispatch_gemm_combine(
            self.h, _vp(_stream(stream, self.device)), S, rank, _ptr_array(xp), _ptr_array(lp),
            _ptr(wt, "wt", _BF16, (E_loc, N, H)), T, H, N, E, E_loc, top_k,
            _ptr(y, "y", _BF16, (cap, N)), _ptr(topk_idx, "topk_idx", i32, (S * T, top_k)),
            _ptr(topk_gate, "topk_gate", (torch.float32,), (S * T, top_k)),
            _ptr(slot_token, "slot_token", i32, (cap,)),
            _ptr(expert_offsets, "expert_offsets", i32, (E_loc + 1,)),
            _ptr(chunk_offsets, "chunk_offsets", i32, (E_loc, S + 1)),
            _ptr(x_slots, "x_slots", _BF16, (cap, H)), cap,
            _ptr(y_peer, "y_peer", _BF16, (T * top_k, N)), _ptr_array(rp),
            _ptr(out, "out", _BF16, (T, N)), flags)
        self._check(st, "mk_moe_dispatch_gemm_combine", self.h)

    def mfma_ceiling(self, iters: int, sink: torch.Tensor, stream=None) -> float:
        """Launch the MFMA-only loop; returns its FLOP count (time it with events)."""
        st = self.lib.mk_mfma_ceiling(self.h, _vp(_stream(stream, self.device)), iters,
                                      _ptr(sink, "sink", (torch.float32,)))
        self._check(st, "mk_mfma_ceiling", self.h)
        props = torch.cuda.get_device_properties(self.device)
        return 2.0 * props.multi_processor_count * 4 * iters * 8 * 32768

    def ring_attention(self, q: torch.Tensor, k_src: Sequence[torch.Tensor],
                       v_src: Sequence[torch.Tensor], o: torch.Tensor, lse: torch.Tensor,
                       k_recv: torch.Tensor, vt_recv: torch.Tensor, scale: Optional[float] = None,
                       rank: int = 0, flags: int = 0, stream=None) -> None:
        """Ring attention of this rank's queries q [BH, S_q, D] over every rank's
        keys / values k_src[r], v_src[r] [BH, S_kv, D]: o [BH, S_q, D] bf16,
        lse [BH, S_q] fp32, k_recv [W, BH, S_kv, D] and vt_recv [W, BH, D, S_kv]
        (the landed blocks, values transposed).  scale defaults to 1/sqrt(D).
        With F_PRELANDED the receive buffers are inputs and k_src / v_src may
        hold None."""
        W = k_recv.shape[0]
        BH, S_q, D = q.shape
        S_kv = k_recv.shape[2]
        if len(k_src) != W or len(v_src) != W:
            raise ValueError(f"k_src / v_src need {W} entries (one per rank)")
        if scale is None:
            scale = 1.0 / float(D) ** 0.5
        kp = [_ptr(k, f"k_src[{r}]", _BF16, (BH, S_kv, D)) for r, k in enumerate(k_src)]
        vp = [_ptr(v, f"v_src[{r}]", _BF16, (BH, S_kv, D)) for r, v in enumerate(v_src)]
        st = self.lib.mk_ring_attention(
            self.h, _vp(_stream(stream, self.device)), W, rank, _ptr(q, "q", _BF16),
            _ptr_array(kp), _ptr_array(vp), BH, S_q, S_kv, D, ctypes.c_float(scale),
            _ptr(o, "o", _BF16, (BH, S_q, D)), _ptr(lse, "lse", (torch.float32,), (BH, S_q)),
            _ptr(k_recv, "k_recv", _BF16, (W, BH, S_kv, D)),
            _ptr(vt_recv, "vt_recv", _BF16, (W, BH, D, S_kv)), flags)
        self._check(st, "mk_ring_attention", self.h)
