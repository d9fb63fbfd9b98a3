"""Speculative-decoding verify step on AMD MI355X (gfx950): Python binding.

Three calls, each a thin marshalling layer over the C ABI of libspecverify.so
(include/spec_verify.h); every step of the computation runs in the library's HIP kernels, and
torch only provides device memory and the current stream:

    verify_attn(q, k_pool, v_pool, page_table, ctx_lens, window, ...)   -> out [B, K1, Hq, D]
    lm_head(hidden, weight, temperature, ...)                            -> (logits | None, p)
    lm_head_noalloc(hidden, weight, temperature, ...)  (no workspace)    -> (logits | None, p)
    accept(draft, q, p, uniforms, ...)                                   -> (n_accepted, tokens)
    accept_philox(draft, q, p, seed, offset, ...)                        -> (n_accepted, tokens, u)
    lm_head_accept(hidden, weight, temperature, draft, q, uniforms | seed/offset)
                                                                          -> (n_accepted, tokens, u)

Workspaces are allocated once per device and kind and reused (calls on one stream are ordered,
so reuse is safe; concurrent streams should pass their own `workspace`).
"""
from __future__ import annotations

import math

from . import _lib
from ._lib import SpecError  # noqa: F401

SPEC_F32, SPEC_BF16 = 0, 1

_workspaces: dict = {}


def _torch():
    import torch
    return torch


def _dtype_code(t) -> int:
    torch = _torch()
    if t.dtype == torch.float32:
        return SPEC_F32
    if t.dtype == torch.bfloat16:
        return SPEC_BF16
    raise TypeError(f"unsupported dtype {t.dtype}; float32 or bfloat16 expected")


def _need(t, name, dtype=None, device=None):
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on a GPU, got {t.device}")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")


def _stream_ptr(device, stream):
    torch = _torch()
    s = stream if stream is not None else torch.cuda.current_stream(device)
    return ctypes_void(s.cuda_stream)


def ctypes_void(x):
    import ctypes
    return ctypes.c_void_p(int(x)) if x else None


def _run(device, name: str, *args) -> None:
    """Call `name` of the C ABI with `device` current (the library launches on the current
    device, whose stream `args` carries) and raise on a negative status."""
    torch = _torch()
    with torch.cuda.device(device):
        rc = getattr(_lib.load(), name)(*args)
    _lib.check(name, rc)


def _nbytes(t) -> int:
    return t.numel() * t.element_size()


def _workspace(kind: str, device, nbytes: int, given=None):
    torch = _torch()
    if given is not None:
        _need(given, "workspace", device=device)
        if _nbytes(given) < nbytes:
            raise ValueError(f"workspace of {nbytes} bytes needed, got {_nbytes(given)}")
        return given
    key = (kind, str(device))
    ws = _workspaces.get(key)
    if ws is None or ws.numel() < nbytes:
        ws = torch.zeros(max(nbytes, 256), dtype=torch.uint8, device=device)
        _workspaces[key] = ws
    return ws


def verify_attn_workspace_bytes(B, K1, Hq, Hkv, D, max_pages, window, page_size=16) -> int:
    n = _lib.load().spec_verify_attn_workspace(B, K1, Hq, Hkv, D, page_size, max_pages, window)
    if n == 0:
        raise SpecError("spec_verify_attn_workspace", -1, _lib.last_error())
    return int(n)


def verify_attn(q, k_pool, v_pool, page_table, ctx_lens, window: int = 0, scale=None, out=None,
                workspace=None, stream=None):
    """(k+1)-query causal GQA attention over the paged cache; returns out [B, K1, Hq, D] fp32."""
    torch = _torch()
    dev = q.device
    _need(q, "q", device=dev)
    _need(k_pool, "k_pool", q.dtype, dev)
    _need(v_pool, "v_pool", q.dtype, dev)
    _need(page_table, "page_table", torch.int32, dev)
    _need(ctx_lens, "ctx_lens", torch.int32, dev)
    B, K1, Hq, D = q.shape
    P, Hkv, ps, D2 = k_pool.shape
    if D2 != D or tuple(v_pool.shape) != tuple(k_pool.shape):
        raise ValueError("k_pool / v_pool must be [P, Hkv, page_size, D] with q's D")
    if page_table.dim() != 2 or page_table.shape[0] != B or ctx_lens.shape != (B,):
        raise ValueError("page_table must be [B, max_pages] and ctx_lens [B]")
    max_pages = page_table.shape[1]
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    if out is None:
        out = torch.empty((B, K1, Hq, D), dtype=torch.float32, device=dev)
    _need(out, "out", torch.float32, dev)
    with torch.cuda.device(dev):   # the split depends on the device's compute units
        nbytes = verify_attn_workspace_bytes(B, K1, Hq, Hkv, D, max_pages, window, ps)
    ws = _workspace("attn", dev, nbytes, workspace)
    _run(dev, "spec_verify_attn",
        q.data_ptr(), k_pool.data_ptr(), v_pool.data_ptr(), page_table.data_ptr(),
        ctx_lens.data_ptr(), out.data_ptr(), B, K1, Hq, Hkv, D, ps, P, max_pages, int(window),
        float(scale), _dtype_code(q), ws.data_ptr(), _nbytes(ws), _stream_ptr(dev, stream))
    return out


def lm_head_workspace_bytes(R, H, V) -> int:
    n = _lib.load().spec_lm_head_workspace(R, H, V)
    if n == 0:
        raise SpecError("spec_lm_head_workspace", -1, _lib.last_error())
    return int(n)


def lm_head(hidden, weight, temperature, probs=None, logits=None, want_logits: bool = False,
            workspace=None, stream=None):
    """logits = hidden weight^T and p = softmax(logits / T) per row; returns (logits, probs).

    logits is None unless `want_logits` or a `logits` buffer is given.
    """
    torch = _torch()
    dev = hidden.device
    _need(hidden, "hidden", device=dev)
    _need(weight, "weight", hidden.dtype, dev)
    _need(temperature, "temperature", torch.float32, dev)
    R, H = hidden.shape
    V, H2 = weight.shape
    if H2 != H or temperature.shape != (R,):
        raise ValueError("weight must be [V, H] and temperature [R]")
    if probs is None:
        probs = torch.empty((R, V), dtype=torch.float32, device=dev)
    _need(probs, "probs", torch.float32, dev)
    if logits is None and want_logits:
        logits = torch.empty((R, V), dtype=torch.float32, device=dev)
    if logits is not None:
        _need(logits, "logits", torch.float32, dev)
    ws = _workspace("lm_head", dev, lm_head_workspace_bytes(R, H, V), workspace)
    _run(dev, "spec_lm_head",
        hidden.data_ptr(), weight.data_ptr(), temperature.data_ptr(),
        logits.data_ptr() if logits is not None else None, probs.data_ptr(), R, H, V,
        _dtype_code(hidden), ws.data_ptr(), _nbytes(ws), _stream_ptr(dev, stream))
    return logits, probs


def lm_head_noalloc(hidden, weight, temperature, probs=None, logits=None,
                    want_logits: bool = False, stream=None):
    """lm_head() through the entry point that allocates nothing: its scratch is the library's
    static device array (spec_lm_head_noalloc).  Outputs are allocated here unless given."""
    torch = _torch()
    dev = hidden.device
    _need(hidden, "hidden", device=dev)
    _need(weight, "weight", hidden.dtype, dev)
    _need(temperature, "temperature", torch.float32, dev)
    R, H = hidden.shape
    V, H2 = weight.shape
    if H2 != H or temperature.shape != (R,):
        raise ValueError("weight must be [V, H] and temperature [R]")
    if probs is None:
        probs = torch.empty((R, V), dtype=torch.float32, device=dev)
    _need(probs, "probs", torch.float32, dev)
    if logits is None and want_logits:
        logits = torch.empty((R, V), dtype=torch.float32, device=dev)
    if logits is not None:
        _need(logits, "logits", torch.float32, dev)
    _run(dev, "spec_lm_head_noalloc",
        hidden.data_ptr(), weight.data_ptr(), temperature.data_ptr(),
        logits.data_ptr() if logits is not None else None, probs.data_ptr(), R, H, V,
        _dtype_code(hidden), _stream_ptr(dev, stream))
    return logits, probs


def accept_workspace_bytes(B, k, V) -> int:
    n = _lib.load().spec_accept_workspace(B, k, V)
    if n == 0:
        raise SpecError("spec_accept_workspace", -1, _lib.last_error())
    return int(n)


def accept(draft, q, p, uniforms, n_accepted=None, tokens=None, workspace=None, stream=None):
    """Leviathan acceptance with correction / bonus draw; returns (n_accepted [B], tokens [B, K1])."""
    torch = _torch()
    dev = p.device
    _need(p, "p", torch.float32, dev)
    _need(uniforms, "uniforms", torch.float32, dev)
    B, K1, V = p.shape
    k = K1 - 1
    if k > 0:
        _need(draft, "draft", torch.int32, dev)
        _need(q, "q", torch.float32, dev)
        if tuple(draft.shape) != (B, k) or tuple(q.shape) != (B, k, V):
            raise ValueError("draft must be [B, k] and q [B, k, V] with p [B, k+1, V]")
    if tuple(uniforms.shape) != (B, K1):
        raise ValueError("uniforms must be [B, k+1]")
    if n_accepted is None:
        n_accepted = torch.empty((B,), dtype=torch.int32, device=dev)
    if tokens is None:
        tokens = torch.empty((B, K1), dtype=torch.int32, device=dev)
    _need(n_accepted, "n_accepted", torch.int32, dev)
    _need(tokens, "tokens", torch.int32, dev)
    ws = _workspace("accept", dev, accept_workspace_bytes(B, k, V), workspace)
    _run(dev, "spec_accept",
        draft.data_ptr() if k > 0 else None, q.data_ptr() if k > 0 else None, p.data_ptr(),
        uniforms.data_ptr(), n_accepted.data_ptr(), tokens.data_ptr(), B, k, V,
        ws.data_ptr(), _nbytes(ws), _stream_ptr(dev, stream))
    return n_accepted, tokens


def accept_philox(draft, q, p, seed: int, offset: int, return_uniforms: bool = False,
                  n_accepted=None, tokens=None, workspace=None, stream=None):
    """accept() with the uniforms drawn on the GPU by Philox4x32-10 (seed, offset); returns
    (n_accepted [B], tokens [B, k+1], uniforms [B, k+1] or None)."""
    torch = _torch()
    dev = p.device
    _need(p, "p", torch.float32, dev)
    B, K1, V = p.shape
    k = K1 - 1
    if k > 0:
        _need(draft, "draft", torch.int32, dev)
        _need(q, "q", torch.float32, dev)
        if tuple(draft.shape) != (B, k) or tuple(q.shape) != (B, k, V):
            raise ValueError("draft must be [B, k] and q [B, k, V] with p [B, k+1, V]")
    if not (0 <= seed < 2 ** 64 and 0 <= offset < 2 ** 64):
        raise ValueError("seed and offset are unsigned 64-bit integers")
    if n_accepted is None:
        n_accepted = torch.empty((B,), dtype=torch.int32, device=dev)
    if tokens is None:
        tokens = torch.empty((B, K1), dtype=torch.int32, device=dev)
    _need(n_accepted, "n_accepted", torch.int32, dev)
    _need(tokens, "tokens", torch.int32, dev)
    u = torch.empty((B, K1), dtype=torch.float32, device=dev) if return_uniforms else None
    ws = _workspace("accept", dev, accept_workspace_bytes(B, k, V), workspace)
    _run(dev, "spec_accept_philox",
        draft.data_ptr() if k > 0 else None, q.data_ptr() if k > 0 else None, p.data_ptr(),
        int(seed), int(offset), u.data_ptr() if u is not None else None, n_accepted.data_ptr(),
        tokens.data_ptr(), B, k, V, ws.data_ptr(), _nbytes(ws), _stream_ptr(dev, stream))
    return n_accepted, tokens, u


def lm_head_accept_workspace_bytes(B, k, H, V) -> int:
    n = _lib.load().spec_lm_head_accept_workspace(B, k, H, V)
    if n == 0:
        raise SpecError("spec_lm_head_accept_workspace", -1, _lib.last_error())
    return int(n)


def lm_head_accept(hidden, weight, temperature, draft, q, uniforms=None, seed: int = 0,
                   offset: int = 0, return_uniforms: bool = False, n_accepted=None, tokens=None,
                   workspace=None, stream=None):
    """lm-head of the B * (k + 1) verify rows and accept / reject in one call (no finalize pass
    over p); n_accepted and tokens equal lm_head() then accept() bit for bit.  uniforms [B, k+1]
    fp32, or None for Philox4x32-10 at (seed, offset).  Returns (n_accepted, tokens, u or None)."""
    torch = _torch()
    dev = hidden.device
    _need(hidden, "hidden", device=dev)
    _need(weight, "weight", hidden.dtype, dev)
    _need(temperature, "temperature", torch.float32, dev)
    R, H = hidden.shape
    V, H2 = weight.shape
    if k_of(draft) is None:
        raise ValueError("draft must be [B, k] int32")
    B, k = draft.shape
    if H2 != H or R != B * (k + 1) or temperature.shape != (R,):
        raise ValueError("hidden must be [B*(k+1), H], weight [V, H], temperature [B*(k+1)]")
    if k > 0:
        _need(draft, "draft", torch.int32, dev)
        _need(q, "q", torch.float32, dev)
        if tuple(q.shape) != (B, k, V):
            raise ValueError("q must be [B, k, V]")
    if uniforms is not None:
        _need(uniforms, "uniforms", torch.float32, dev)
        if tuple(uniforms.shape) != (B, k + 1):
            raise ValueError("uniforms must be [B, k+1]")
    if not (0 <= seed < 2 ** 64 and 0 <= offset < 2 ** 64):
        raise ValueError("seed and offset are unsigned 64-bit integers")
    if n_accepted is None:
        n_accepted = torch.empty((B,), dtype=torch.int32, device=dev)
    if tokens is None:
        tokens = torch.empty((B, k + 1), dtype=torch.int32, device=dev)
    _need(n_accepted, "n_accepted", torch.int32, dev)
    _need(tokens, "tokens", torch.int32, dev)
    u = torch.empty((B, k + 1), dtype=torch.float32, device=dev) if return_uniforms else None
    ws = _workspace("lm_head_accept", dev, lm_head_accept_workspace_bytes(B, k, H, V), workspace)
    _run(dev, "spec_lm_head_accept",
        hidden.data_ptr(), weight.data_ptr(), temperature.data_ptr(),
        draft.data_ptr() if k > 0 else None, q.data_ptr() if k > 0 else None,
        uniforms.data_ptr() if uniforms is not None else None, int(seed), int(offset),
        u.data_ptr() if u is not None else None, n_accepted.data_ptr(), tokens.data_ptr(),
        B, k, H, V, _dtype_code(hidden), ws.data_ptr(), _nbytes(ws), _stream_ptr(dev, stream))
    return n_accepted, tokens, u


def k_of(draft):
    """k of a [B, k] draft tensor, or None if it is not one."""
    torch = _torch()
    if not isinstance(draft, torch.Tensor) or draft.dim() != 2:
        return None
    return int(draft.shape[1])


def kv_append(k_new, v_new, k_pool, v_pool, page_table, ctx_lens, stream=None):
    """Write the K/V of the K1 verified positions, [B, K1, Hkv, D], into their cache pages
    (positions ctx_lens[b] - K1 + i; ctx_lens already counts them)."""
    torch = _torch()
    dev = k_pool.device
    _need(k_pool, "k_pool", device=dev)
    _need(v_pool, "v_pool", k_pool.dtype, dev)
    _need(k_new, "k_new", k_pool.dtype, dev)
    _need(v_new, "v_new", k_pool.dtype, dev)
    _need(page_table, "page_table", torch.int32, dev)
    _need(ctx_lens, "ctx_lens", torch.int32, dev)
    B, K1, Hkv, D = k_new.shape
    P, Hkv2, ps, D2 = k_pool.shape
    if (Hkv2, D2) != (Hkv, D) or tuple(v_new.shape) != tuple(k_new.shape):
        raise ValueError("k_new / v_new must be [B, K1, Hkv, D] matching the pools")
    _run(dev, "spec_kv_append",
        k_new.data_ptr(), v_new.data_ptr(), k_pool.data_ptr(), v_pool.data_ptr(),
        page_table.data_ptr(), ctx_lens.data_ptr(), B, K1, Hkv, D, ps, P, page_table.shape[1],
        _dtype_code(k_pool), _stream_ptr(dev, stream))


def kv_commit(ctx_lens, n_accepted, K1: int, stream=None):
    """Keep the last committed token and the accepted drafts: ctx -= K1 - 1 - n (in place)."""
    torch = _torch()
    dev = ctx_lens.device
    _need(ctx_lens, "ctx_lens", torch.int32, dev)
    _need(n_accepted, "n_accepted", torch.int32, dev)
    _run(dev, "spec_kv_commit", ctx_lens.data_ptr(), n_accepted.data_ptr(), ctx_lens.shape[0],
         int(K1), _stream_ptr(dev, stream))


def version() -> int:
    return int(_lib.load().spec_version())
