"""Thin ctypes binding of the CRISP HIP library (include/crisp.h).

Argument marshalling only: every step runs in the HIP kernels of
``_lib/libcrisp.so``.  Tensors are torch tensors used as device memory; the
stream is torch's current HIP stream unless one is given.  There is no CPU
fallback: if the library is missing the import-time loader raises.
"""
from __future__ import annotations

import ctypes as C
import os
import re

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "_lib", "libcrisp.so")
HEADER = os.path.join(os.path.dirname(PKG), "include", "crisp.h")

CRISP_OK = 0
CRISP_ERR_INVALID_ARG = 1
CRISP_ERR_SHAPE = 2
CRISP_ERR_UNSUPPORTED = 3
CRISP_ERR_WORKSPACE = 4
CRISP_ERR_HIP = 5


class CrispError(RuntimeError):
    def __init__(self, code: int, where: str):
        self.code = code
        super().__init__(f"{where}: {status_string(code)} (code {code})")


class crisp_opts(C.Structure):
    _fields_ = [("tau_proxy", C.c_float), ("gamma", C.c_float), ("k_min_tokens", C.c_int),
                ("w_sink", C.c_int), ("w_local", C.c_int), ("router", C.c_int),
                ("tau_jsd", C.c_float), ("vs_rule", C.c_int), ("gamma_vs", C.c_float),
                ("dense_below_tokens", C.c_int)]


class crisp_seq(C.Structure):
    _fields_ = [("q", C.c_void_p), ("k", C.c_void_p), ("v", C.c_void_p), ("out", C.c_void_p),
                ("seq_len", C.c_int)]


class crisp_strides(C.Structure):
    _fields_ = [(n, C.c_int64) for n in ("q_head", "q_token", "k_head", "k_token", "v_head",
                                         "v_token", "out_head", "out_token")]


# crisp_prefill_noalloc's static scratch (CRISP_NOALLOC_SCRATCH_BYTES)
NOALLOC_SCRATCH_BYTES = 64 << 20

ROUTER_CSTRUCT, ROUTER_JSD = 0, 1
VS_NOISE_MEAN, VS_NOISE_MEDIAN, VS_GAMMA = 0, 1, 2


def default_opts(**overrides) -> crisp_opts:
    """The library's defaults (crisp_default_opts), with fields overridden."""
    o = crisp_opts()
    lib().crisp_default_opts(C.byref(o))
    for k, v in overrides.items():
        setattr(o, k, v)
    return o


def flexprefill_opts(**overrides) -> crisp_opts:
    """The FlexPrefill baseline of Appendix A: JSD routing (Alg. 5) and the
    cumulative gamma rule for VS heads (Alg. 6), k_min as configured."""
    return default_opts(router=ROUTER_JSD, vs_rule=VS_GAMMA, **overrides)


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"CRISP HIP library not built: {LIB_PATH} "
                              "(run python -m dynamic_sparse_attention_map_amd.build)")
        L = C.CDLL(LIB_PATH)
        P, i, f, sz, i64 = C.c_void_p, C.c_int, C.c_float, C.c_size_t, C.c_int64
        L.crisp_status_string.argtypes = [i]
        L.crisp_status_string.restype = C.c_char_p
        L.crisp_workspace_size.argtypes = [i, i, i, i, i, C.POINTER(sz), C.POINTER(i64)]
        L.crisp_workspace_size_batch.argtypes = [P, i, i, i, i, i, C.POINTER(sz)]
        L.crisp_route.argtypes = [P, P, i, i, i, i, i, P, P, sz, P, P, P, P, P]
        L.crisp_select.argtypes = [P, P, P, P, P, i, i, i, i, i, f, P, P, sz, P, P, P, P, P, i64, P]
        L.crisp_attend.argtypes = [P, P, P, P, P, i, i, i, i, i, P, sz, P, P]
        L.crisp_attend_dense.argtypes = [P, P, P, i, i, i, i, i, P, sz, P, P]
        L.crisp_prefill.argtypes = [P, P, P, i, i, i, i, i, f, P, P, sz, P, P]
        L.crisp_prefill_batch.argtypes = [P, i, P, i, i, i, i, f, P, P, sz, P]
        L.crisp_prefill_noalloc.argtypes = [P, P, P, i, i, i, i, i, f, P, P, P]
        L.crisp_set_stage_events.argtypes = [P, i]
        L.crisp_default_opts.argtypes = [P]
        L.crisp_default_opts.restype = None
        for name in ("crisp_workspace_size", "crisp_workspace_size_batch", "crisp_route", "crisp_select", "crisp_attend",
                     "crisp_attend_dense", "crisp_prefill", "crisp_prefill_batch",
                     "crisp_prefill_noalloc", "crisp_set_stage_events"):
            getattr(L, name).restype = i
        _lib = L
    return _lib


def header_symbols() -> list:
    """Function names declared in include/crisp.h."""
    text = open(HEADER).read()
    return sorted(set(re.findall(r"\b(crisp_[a-z_]+)\s*\(", text)))


def status_string(code: int) -> str:
    return lib().crisp_status_string(code).decode()


def _check(rc: int, where: str):
    if rc != CRISP_OK:
        raise CrispError(rc, where)


def _ptr(t):
    return None if t is None else C.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        import torch
        return C.c_void_p(torch.cuda.current_stream().cuda_stream)
    if isinstance(stream, int):
        return C.c_void_p(stream)
    return C.c_void_p(stream.cuda_stream)


def _opts(opts):
    return None if opts is None else C.byref(opts)


def _tensor(t, name, dtype=None, ndim=None, numel=None, min_numel=None):
    """A contiguous device tensor of the given dtype (bfloat16 by default)."""
    import torch
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    want = torch.bfloat16 if dtype is None else dtype
    if t.dtype != want:
        raise ValueError(f"{name} must be {want}, got {t.dtype}")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dimensions, got shape {tuple(t.shape)}")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if numel is not None and t.numel() != numel:
        raise ValueError(f"{name} must have {numel} elements, got {t.numel()}")
    if min_numel is not None and t.numel() < min_numel:
        raise ValueError(f"{name} must have at least {min_numel} elements, got {t.numel()}")
    return t


def _shape(q, k, v=None, out=None):
    """(seq_len, n_heads, n_kv_heads, head_dim) of q [H, n, d], k [H_kv, n, d],
    after checking that v / out match k / q, then dtypes, devices and
    contiguity.  head_dim and the block size are checked by the library."""
    import torch
    for t, name in ((q, "q"), (k, "k"), (v, "v"), (out, "out")):
        if t is None:
            continue
        if not isinstance(t, torch.Tensor):
            raise TypeError(f"{name} must be a torch.Tensor")
        if t.dim() != 3:
            raise ValueError(f"{name} must have 3 dimensions, got shape {tuple(t.shape)}")
    hq, n, d = q.shape
    hkv = k.shape[0]
    if k.shape[1] != n or k.shape[2] != d:
        raise ValueError(f"k {tuple(k.shape)} does not match q {tuple(q.shape)} in length or head_dim")
    if v is not None and v.shape != k.shape:
        raise ValueError(f"v {tuple(v.shape)} must have k's shape {tuple(k.shape)}")
    if out is not None and out.shape != q.shape:
        raise ValueError(f"out {tuple(out.shape)} must have q's shape {tuple(q.shape)}")
    for t, name in ((q, "q"), (k, "k"), (v, "v"), (out, "out")):
        if t is not None:
            _tensor(t, name)
            if t.device != q.device:
                raise ValueError(f"{name} must be on q's device")
    return n, hq, hkv, d


def _workspace(ws):
    import torch
    return _tensor(ws, "ws", dtype=torch.uint8)


def _nblocks(n, block_size):
    return -(-n // block_size) if block_size > 0 else 0


def crisp_workspace_size(seq_len, n_heads, n_kv_heads, head_dim=128, block_size=128):
    ws = C.c_size_t(0)
    cap = C.c_int64(0)
    _check(lib().crisp_workspace_size(seq_len, n_heads, n_kv_heads, head_dim, block_size,
                                      C.byref(ws), C.byref(cap)), "crisp_workspace_size")
    return int(ws.value), int(cap.value)


def crisp_workspace_size_batch(seq_lens, n_heads, n_kv_heads, head_dim=128, block_size=128):
    """Workspace with which crisp_prefill_batch attends the whole batch in one launch."""
    lens = (C.c_int * max(len(seq_lens), 1))(*[int(x) for x in seq_lens])
    ws = C.c_size_t(0)
    _check(lib().crisp_workspace_size_batch(lens, len(seq_lens), n_heads, n_kv_heads, head_dim,
                                            block_size, C.byref(ws)), "crisp_workspace_size_batch")
    return int(ws.value)


def alloc_batch_workspace(seq_lens, n_heads, n_kv_heads, device="cuda"):
    """A caller-owned workspace for the single-launch batch path."""
    import torch
    return torch.empty(crisp_workspace_size_batch(seq_lens, n_heads, n_kv_heads), dtype=torch.uint8,
                       device=device)


def alloc_workspace(seq_len, n_heads, n_kv_heads, device="cuda"):
    """A caller-owned workspace (torch allocates it; the library never does)."""
    import torch
    ws_bytes, _ = crisp_workspace_size(seq_len, n_heads, n_kv_heads)
    return torch.empty(ws_bytes, dtype=torch.uint8, device=device)


def crisp_route(q, k, ws, pattern, c_struct, p_v, p_s, opts=None, block_size=128, stream=None):
    import torch
    n, hq, hkv, d = _shape(q, k)
    _workspace(ws)
    nb = _nblocks(n, block_size)
    _tensor(pattern, "pattern", dtype=torch.uint8, numel=hq)
    _tensor(c_struct, "c_struct", dtype=torch.float32, numel=hq)
    _tensor(p_v, "p_v", dtype=torch.float32, numel=hq * nb)
    _tensor(p_s, "p_s", dtype=torch.float32, numel=hq * nb)
    _check(lib().crisp_route(_ptr(q), _ptr(k), n, hq, hkv, d, block_size, _opts(opts), _ptr(ws),
                             ws.numel(), _ptr(pattern), _ptr(c_struct), _ptr(p_v), _ptr(p_s),
                             _stream(stream)), "crisp_route")


def crisp_select(q, k, pattern, p_v, p_s, alpha, ws, sel_v, sel_s, sel_counts, row_ptr, col_idx,
                 opts=None, block_size=128, stream=None):
    import torch
    n, hq, hkv, d = _shape(q, k)
    _workspace(ws)
    nb = _nblocks(n, block_size)
    _tensor(pattern, "pattern", dtype=torch.uint8, numel=hq)
    _tensor(p_v, "p_v", dtype=torch.float32, numel=hq * nb)
    _tensor(p_s, "p_s", dtype=torch.float32, numel=hq * nb)
    _tensor(sel_v, "sel_v", dtype=torch.int32, numel=hq * nb)
    _tensor(sel_s, "sel_s", dtype=torch.int32, numel=hq * nb)
    _tensor(sel_counts, "sel_counts", dtype=torch.int32, numel=hq * 3)
    _tensor(row_ptr, "row_ptr", dtype=torch.int32, numel=hq * (nb + 1))
    _tensor(col_idx, "col_idx", dtype=torch.int32)
    _check(lib().crisp_select(_ptr(q), _ptr(k), _ptr(pattern), _ptr(p_v), _ptr(p_s), n, hq, hkv, d,
                              block_size, float(alpha), _opts(opts), _ptr(ws), ws.numel(),
                              _ptr(sel_v), _ptr(sel_s), _ptr(sel_counts), _ptr(row_ptr),
                              _ptr(col_idx), col_idx.numel(), _stream(stream)), "crisp_select")


def crisp_attend(q, k, v, row_ptr, col_idx, ws, out, block_size=128, stream=None,
                 check_lists=True):
    """Eq. 1 on given lists.  row_ptr int32 [hq, N_b + 1] of absolute offsets
    into col_idx (int32); every offset must lie inside col_idx.  With
    check_lists (and outside graph capture) that is checked on a host copy of
    row_ptr, which synchronises with the device; timing loops pass False."""
    import torch
    n, hq, hkv, d = _shape(q, k, v, out)
    _workspace(ws)
    nb = _nblocks(n, block_size)
    _tensor(row_ptr, "row_ptr", dtype=torch.int32, numel=hq * (nb + 1))
    _tensor(col_idx, "col_idx", dtype=torch.int32)
    if n > 0 and check_lists and not torch.cuda.is_current_stream_capturing():
        rp = row_ptr.detach().to("cpu").view(hq, nb + 1)
        lo, hi = int(rp.min()), int(rp.max())
        if lo < 0 or hi > col_idx.numel() or bool((rp[:, 1:] < rp[:, :-1]).any()):
            raise ValueError("row_ptr must be non-decreasing per head and stay inside col_idx")
    _check(lib().crisp_attend(_ptr(q), _ptr(k), _ptr(v), _ptr(row_ptr), _ptr(col_idx), n, hq, hkv, d,
                              block_size, _ptr(ws), ws.numel(), _ptr(out), _stream(stream)),
           "crisp_attend")


def crisp_attend_dense(q, k, v, ws, out, block_size=128, stream=None):
    n, hq, hkv, d = _shape(q, k, v, out)
    _workspace(ws)
    _check(lib().crisp_attend_dense(_ptr(q), _ptr(k), _ptr(v), n, hq, hkv, d, block_size, _ptr(ws),
                                    ws.numel(), _ptr(out), _stream(stream)), "crisp_attend_dense")


def crisp_prefill(q, k, v, alpha, ws, out, opts=None, block_size=128, stream=None):
    n, hq, hkv, d = _shape(q, k, v, out)
    _workspace(ws)
    _check(lib().crisp_prefill(_ptr(q), _ptr(k), _ptr(v), n, hq, hkv, d, block_size, float(alpha),
                               _opts(opts), _ptr(ws), ws.numel(), _ptr(out), _stream(stream)),
           "crisp_prefill")


def crisp_prefill_noalloc(q, k, v, alpha, out, opts=None, block_size=128, stream=None):
    """crisp_prefill on the library's static per-device scratch (no
    workspace argument; layers needing more than NOALLOC_SCRATCH_BYTES are
    refused with CRISP_ERR_WORKSPACE).  Calls overlapping on one device race."""
    n, hq, hkv, d = _shape(q, k, v, out)
    _check(lib().crisp_prefill_noalloc(_ptr(q), _ptr(k), _ptr(v), n, hq, hkv, d, block_size,
                                       float(alpha), _opts(opts), _ptr(out), _stream(stream)),
           "crisp_prefill_noalloc")


def crisp_prefill_batch(qs, ks, vs, outs, alpha, ws, opts=None, block_size=128, stream=None):
    """Several sequences in one call.  qs, ks, vs, outs: lists of
    [heads, seq_len, head_dim] tensors.  Either every tensor is contiguous
    (strides NULL: each sequence [heads][seq_len][head_dim]) or all share one
    head and token stride per operand (head_dim contiguous).  The workspace
    must fit the longest sequence."""
    batch = len(qs)
    if not (len(ks) == len(vs) == len(outs) == batch):
        raise ValueError("qs, ks, vs, outs must have the same length")
    if batch == 0:
        _check(lib().crisp_prefill_batch(None, 0, None, 1, 1, 128, block_size, float(alpha),
                                         _opts(opts), _ptr(ws), ws.numel(), _stream(stream)),
               "crisp_prefill_batch")
        return
    hq, hkv, d = qs[0].shape[0], ks[0].shape[0], qs[0].shape[2]
    if all(t.dim() == 3 and t.is_contiguous() for t in (*qs, *ks, *vs, *outs)):
        arr = (crisp_seq * batch)()
        for b in range(batch):
            n = qs[b].shape[1]
            if ks[b].shape[1] != n or vs[b].shape[1] != n or outs[b].shape[1] != n:
                raise ValueError("q, k, v, out of a sequence must have the same length")
            arr[b] = crisp_seq(qs[b].data_ptr(), ks[b].data_ptr(), vs[b].data_ptr(),
                               outs[b].data_ptr(), n)
        _check(lib().crisp_prefill_batch(arr, batch, None, hq, hkv, d, block_size, float(alpha),
                                         _opts(opts), _ptr(ws), ws.numel(), _stream(stream)),
               "crisp_prefill_batch")
        return
    st = crisp_strides(qs[0].stride(0), qs[0].stride(1), ks[0].stride(0), ks[0].stride(1),
                       vs[0].stride(0), vs[0].stride(1), outs[0].stride(0), outs[0].stride(1))
    arr = (crisp_seq * batch)()
    for b in range(batch):
        views = (qs[b], ks[b], vs[b], outs[b])
        for t, (sh, stk) in zip(views, ((st.q_head, st.q_token), (st.k_head, st.k_token),
                                        (st.v_head, st.v_token), (st.out_head, st.out_token))):
            if t.dim() != 3 or t.shape[2] != d or t.stride(2) != 1:
                raise ValueError("each tensor must be a [heads, seq_len, head_dim] view with "
                                 "contiguous head_dim")
            if t.shape[1] > 1 and t.stride(1) != stk or t.shape[0] > 1 and t.stride(0) != sh:
                raise ValueError("all sequences must share the same strides")
        n = qs[b].shape[1]
        if ks[b].shape[1] != n or vs[b].shape[1] != n or outs[b].shape[1] != n:
            raise ValueError("q, k, v, out of a sequence must have the same length")
        if qs[b].shape[0] != hq or ks[b].shape[0] != hkv or outs[b].shape[0] != hq:
            raise ValueError("head counts must match across the batch")
        arr[b] = crisp_seq(qs[b].data_ptr(), ks[b].data_ptr(), vs[b].data_ptr(),
                           outs[b].data_ptr(), n)
    _check(lib().crisp_prefill_batch(arr, batch, C.byref(st), hq, hkv, d, block_size, float(alpha),
                                     _opts(opts), _ptr(ws), ws.numel(), _stream(stream)),
           "crisp_prefill_batch")


def prefill_varlen(q, k, v, cu_seqlens, out, alpha, ws, opts=None, stream=None):
    """Packed variable-length batch: q, out [total, heads, head_dim] and k, v
    [total, kv_heads, head_dim]; sequence b holds tokens
    cu_seqlens[b] .. cu_seqlens[b+1] (a host sequence of ints)."""
    cu = [int(x) for x in cu_seqlens]
    sl = [slice(cu[b], cu[b + 1]) for b in range(len(cu) - 1)]
    crisp_prefill_batch([q[s].transpose(0, 1) for s in sl], [k[s].transpose(0, 1) for s in sl],
                        [v[s].transpose(0, 1) for s in sl], [out[s].transpose(0, 1) for s in sl],
                        alpha, ws, opts=opts, stream=stream)


def crisp_set_stage_events(events):
    """events: five torch.cuda.Event (created with enable_timing) or None."""
    if events is None:
        _check(lib().crisp_set_stage_events(None, 0), "crisp_set_stage_events")
        return
    arr = (C.c_void_p * len(events))(*[C.c_void_p(e.cuda_event) for e in events])
    _check(lib().crisp_set_stage_events(arr, len(events)), "crisp_set_stage_events")
