"""Python binding of the verify step: torch tensors in, torch tensors out.

Marshalling only -- shapes and dtypes are checked, outputs and the workspace
are allocated with torch on the tensors' device, and the C ABI is called on
torch's current stream.  Every step of the computation runs in the HIP
kernels of libspecverify.so.
"""

from __future__ import annotations

from typing import Optional

import torch

from ._lib import SV_BF16, SV_F32, SV_OK, SamplingParamsC, load_library, status_string

FLAG_BAD_ID = 1
FLAG_Q_ZERO = 2
FLAG_Z_DEGENERATE = 4
FLAG_NONFINITE = 8
FLAG_EOS = 16
FLAG_BAD_SPAN = 32

_DT = {torch.float32: SV_F32, torch.bfloat16: SV_BF16}


def _params(temperature: float, top_k: int, top_p: float) -> SamplingParamsC:
    return SamplingParamsC(float(temperature), int(top_k), float(top_p))


def _check(t: torch.Tensor, name: str, dtype, shape) -> None:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be on a GPU")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _raise(code: int, what: str) -> None:
    if code != SV_OK:
        raise RuntimeError(f"{what}: {status_string(code)} (status {code})")


def workspace_size(B: int, gamma: int, V: int, dtype=torch.bfloat16, temperature=1.0, top_k=0, top_p=1.0) -> int:
    n = load_library().spec_verify_workspace_size(B, gamma, V, _DT[dtype], _params(temperature, top_k, top_p))
    if n == 0:
        raise ValueError("invalid sizes or sampling parameters")
    return int(n)


def _workspace(ws: Optional[torch.Tensor], need: int, device) -> torch.Tensor:
    if ws is None:
        return torch.empty(need, dtype=torch.uint8, device=device)
    if ws.numel() * ws.element_size() < need:
        raise ValueError(f"workspace holds {ws.numel() * ws.element_size()} bytes, {need} needed")
    return ws


def _stream(device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


def verify_sample(logits, q, ids, u_accept, u_resample, temperature=1.0, top_k=0, top_p=1.0,
                  workspace: Optional[torch.Tensor] = None, out=None):
    """Sampling verify step; returns (tokens [B, gamma+1] int32, n_accepted [B] int32, flags [B] int32)."""
    if logits.dim() != 3:
        raise ValueError("logits must be [B, gamma+1, V]")
    B, G1, V = logits.shape
    G = G1 - 1
    _check(logits, "logits", None, (B, G1, V))
    if logits.dtype not in _DT:
        raise ValueError("logits must be float32 or bfloat16")
    dev = logits.device
    if G > 0:
        _check(q, "q", torch.float32, (B, G, V))
        _check(ids, "ids", torch.int32, (B, G))
        _check(u_accept, "u_accept", torch.float32, (B, G))
    _check(u_resample, "u_resample", torch.float32, (B, G1))
    if out is None:
        out = (torch.empty((B, G1), dtype=torch.int32, device=dev),
               torch.empty((B,), dtype=torch.int32, device=dev),
               torch.empty((B,), dtype=torch.int32, device=dev))
    tokens, nacc, flags = out
    need = workspace_size(B, G, V, logits.dtype, temperature, top_k, top_p)
    ws = _workspace(workspace, need, dev)
    lib = load_library()
    code = lib.spec_verify_sample(
        logits.data_ptr(), _DT[logits.dtype],
        q.data_ptr() if G > 0 else None, ids.data_ptr() if G > 0 else None,
        u_accept.data_ptr() if G > 0 else None, u_resample.data_ptr(),
        B, G, V, _params(temperature, top_k, top_p),
        tokens.data_ptr(), nacc.data_ptr(), flags.data_ptr(),
        ws.data_ptr(), ws.numel() * ws.element_size(), _stream(dev))
    _raise(code, "spec_verify_sample")
    return tokens, nacc, flags


def verify_sample_lenient(logits, q, ids, u_accept, u_resample, temperature=1.0, top_k=0, top_p=1.0,
                          lenience=1.0, workspace: Optional[torch.Tensor] = None, out=None):
    """Sampling verify step with lenient acceptance u < p / (lenience * q),
    0 < lenience <= 1 (1: exactly verify_sample); returns (tokens, n_accepted, flags)."""
    if logits.dim() != 3:
        raise ValueError("logits must be [B, gamma+1, V]")
    B, G1, V = logits.shape
    G = G1 - 1
    _check(logits, "logits", None, (B, G1, V))
    if logits.dtype not in _DT:
        raise ValueError("logits must be float32 or bfloat16")
    dev = logits.device
    if G > 0:
        _check(q, "q", torch.float32, (B, G, V))
        _check(ids, "ids", torch.int32, (B, G))
        _check(u_accept, "u_accept", torch.float32, (B, G))
    _check(u_resample, "u_resample", torch.float32, (B, G1))
    if out is None:
        out = (torch.empty((B, G1), dtype=torch.int32, device=dev),
               torch.empty((B,), dtype=torch.int32, device=dev),
               torch.empty((B,), dtype=torch.int32, device=dev))
    tokens, nacc, flags = out
    need = workspace_size(B, G, V, logits.dtype, temperature, top_k, top_p)
    ws = _workspace(workspace, need, dev)
    code = load_library().spec_verify_sample_lenient(
        logits.data_ptr(), _DT[logits.dtype],
        q.data_ptr() if G > 0 else None, ids.data_ptr() if G > 0 else None,
        u_accept.data_ptr() if G > 0 else None, u_resample.data_ptr(),
        B, G, V, _params(temperature, top_k, top_p), float(lenience),
        tokens.data_ptr(), nacc.data_ptr(), flags.data_ptr(),
        ws.data_ptr(), ws.numel() * ws.element_size(), _stream(dev))
    _raise(code, "spec_verify_sample_lenient")
    return tokens, nacc, flags


def verify_greedy(logits, ids, workspace: Optional[torch.Tensor] = None, out=None):
    """Greedy verify step; returns (tokens, n_accepted, flags)."""
    if logits.dim() != 3:
        raise ValueError("logits must be [B, gamma+1, V]")
    B, G1, V = logits.shape
    G = G1 - 1
    _check(logits, "logits", None, (B, G1, V))
    if logits.dtype not in _DT:
        raise ValueError("logits must be float32 or bfloat16")
    dev = logits.device
    if G > 0:
        _check(ids, "ids", torch.int32, (B, G))
    if out is None:
        out = (torch.empty((B, G1), dtype=torch.int32, device=dev),
               torch.empty((B,), dtype=torch.int32, device=dev),
               torch.empty((B,), dtype=torch.int32, device=dev))
    tokens, nacc, flags = out
    need = workspace_size(B, G, V, logits.dtype)
    ws = _workspace(workspace, need, dev)
    code = load_library().spec_verify_greedy(
        logits.data_ptr(), _DT[logits.dtype], ids.data_ptr() if G > 0 else None, B, G, V,
        tokens.data_ptr(), nacc.data_ptr(), flags.data_ptr(),
        ws.data_ptr(), ws.numel() * ws.element_size(), _stream(dev))
    _raise(code, "spec_verify_greedy")
    return tokens, nacc, flags


def _stats_outs(stats_out, B, G, dev, z_qp):
    """(alpha, Z, Z', accept_prob) buffers; an entry may be None (not
    computed).  Without Z' (z_qp=False) a position whose p is truncated to a
    kept set reads q only at that set's ids."""
    if stats_out is None:
        stats_out = tuple(None if (k == 2 and not z_qp) else torch.empty((B, G), dtype=torch.float32, device=dev)
                          for k in range(4))
    return stats_out


def _ptr(t):
    return None if t is None else t.data_ptr()


def accept_stats(logits, q, ids, temperature=1.0, top_k=0, top_p=1.0,
                 workspace: Optional[torch.Tensor] = None, out=None, z_qp: bool = True):
    """Per-position (alpha, Z, Z', accept_prob), each [B, gamma] float32 (Z'
    None when z_qp is False)."""
    if logits.dim() != 3:
        raise ValueError("logits must be [B, gamma+1, V]")
    B, G1, V = logits.shape
    G = G1 - 1
    _check(logits, "logits", None, (B, G1, V))
    if logits.dtype not in _DT:
        raise ValueError("logits must be float32 or bfloat16")
    dev = logits.device
    _check(q, "q", torch.float32, (B, G, V))
    _check(ids, "ids", torch.int32, (B, G))
    alpha, zpq, zqp, acc = _stats_outs(out, B, G, dev, z_qp)
    need = workspace_size(B, G, V, logits.dtype, temperature, top_k, top_p)
    ws = _workspace(workspace, need, dev)
    code = load_library().spec_accept_stats(
        logits.data_ptr(), _DT[logits.dtype], q.data_ptr(), ids.data_ptr(), B, G, V,
        _params(temperature, top_k, top_p), _ptr(alpha), _ptr(zpq), _ptr(zqp), _ptr(acc),
        ws.data_ptr(), ws.numel() * ws.element_size(), _stream(dev))
    _raise(code, "spec_accept_stats")
    return alpha, zpq, zqp, acc


def draft_logits_workspace_size(B: int, gamma: int, V: int, dtype=torch.bfloat16, draft_dtype=torch.bfloat16,
                                temperature=1.0, top_k=0, top_p=1.0) -> int:
    n = load_library().spec_verify_draft_logits_workspace_size(
        B, gamma, V, _DT[dtype], _DT[draft_dtype], _params(temperature, top_k, top_p))
    if n == 0:
        raise ValueError("invalid sizes or sampling parameters")
    return int(n)


def verify_sample_draft_logits(logits, draft_logits, ids, u_accept, u_resample, temperature=1.0, top_k=0,
                               top_p=1.0, workspace: Optional[torch.Tensor] = None, out=None):
    """Sampling verify step with q formed from the draft's logits [B, gamma, V]
    by the same rules as p; returns (tokens, n_accepted, flags)."""
    if logits.dim() != 3:
        raise ValueError("logits must be [B, gamma+1, V]")
    B, G1, V = logits.shape
    G = G1 - 1
    _check(logits, "logits", None, (B, G1, V))
    if logits.dtype not in _DT:
        raise ValueError("logits must be float32 or bfloat16")
    dev = logits.device
    ddt = logits.dtype
    if G > 0:
        _check(draft_logits, "draft_logits", None, (B, G, V))
        if draft_logits.dtype not in _DT:
            raise ValueError("draft_logits must be float32 or bfloat16")
        ddt = draft_logits.dtype
        _check(ids, "ids", torch.int32, (B, G))
        _check(u_accept, "u_accept", torch.float32, (B, G))
    _check(u_resample, "u_resample", torch.float32, (B, G1))
    if out is None:
        out = (torch.empty((B, G1), dtype=torch.int32, device=dev),
               torch.empty((B,), dtype=torch.int32, device=dev),
               torch.empty((B,), dtype=torch.int32, device=dev))
    tokens, nacc, flags = out
    need = draft_logits_workspace_size(B, G, V, logits.dtype, ddt, temperature, top_k, top_p)
    ws = _workspace(workspace, need, dev)
    code = load_library().spec_verify_sample_draft_logits(
        logits.data_ptr(), _DT[logits.dtype],
        draft_logits.data_ptr() if G > 0 else None, _DT[ddt], ids.data_ptr() if G > 0 else None,
        u_accept.data_ptr() if G > 0 else None, u_resample.data_ptr(),
        B, G, V, _params(temperature, top_k, top_p),
        tokens.data_ptr(), nacc.data_ptr(), flags.data_ptr(),
        ws.data_ptr(), ws.numel() * ws.element_size(), _stream(dev))
    _raise(code, "spec_verify_sample_draft_logits")
    return tokens, nacc, flags


def accept_stats_draft_logits(logits, draft_logits, ids, temperature=1.0, top_k=0, top_p=1.0,
                              workspace: Optional[torch.Tensor] = None, out=None, z_qp: bool = True):
    """Per-position (alpha, Z, Z', accept_prob) with q formed from the draft's
    logits (Z' None when z_qp is False)."""
    if logits.dim() != 3:
        raise ValueError("logits must be [B, gamma+1, V]")
    B, G1, V = logits.shape
    G = G1 - 1
    _check(logits, "logits", None, (B, G1, V))
    if logits.dtype not in _DT:
        raise ValueError("logits must be float32 or bfloat16")
    dev = logits.device
    _check(draft_logits, "draft_logits", None, (B, G, V))
    if draft_logits.dtype not in _DT:
        raise ValueError("draft_logits must be float32 or bfloat16")
    _check(ids, "ids", torch.int32, (B, G))
    alpha, zpq, zqp, acc = _stats_outs(out, B, G, dev, z_qp)
    need = draft_logits_workspace_size(B, G, V, logits.dtype, draft_logits.dtype, temperature, top_k, top_p)
    ws = _workspace(workspace, need, dev)
    code = load_library().spec_accept_stats_draft_logits(
        logits.data_ptr(), _DT[logits.dtype], draft_logits.data_ptr(), _DT[draft_logits.dtype], ids.data_ptr(),
        B, G, V, _params(temperature, top_k, top_p), _ptr(alpha), _ptr(zpq), _ptr(zqp),
        _ptr(acc), ws.data_ptr(), ws.numel() * ws.element_size(), _stream(dev))
    _raise(code, "spec_accept_stats_draft_logits")
    return alpha, zpq, zqp, acc


def _ragged_shapes(logits, ids, cu):
    if logits.dim() != 2:
        raise ValueError("ragged logits must be packed [n_draft + B, V]")
    _check(cu, "cu_draft", torch.int32, (cu.shape[0],))
    B = cu.shape[0] - 1
    if B < 0:
        raise ValueError("cu_draft must hold B + 1 offsets")
    N = ids.shape[0] if ids is not None else 0
    V = logits.shape[1]
    _check(logits, "logits", None, (N + B, V))
    if logits.dtype not in _DT:
        raise ValueError("logits must be float32 or bfloat16")
    if N > 0:
        _check(ids, "ids", torch.int32, (N,))
    return B, N, V


def _ragged_out(out, B, gamma_max, dev):
    if out is None:
        out = (torch.empty((B, gamma_max + 1), dtype=torch.int32, device=dev),
               torch.empty((B,), dtype=torch.int32, device=dev),
               torch.empty((B,), dtype=torch.int32, device=dev))
    return out


def verify_sample_ragged(logits, q, ids, cu_draft, u_accept, u_resample, gamma_max: int, temperature=1.0, top_k=0,
                         top_p=1.0, eos_id: int = -1, workspace: Optional[torch.Tensor] = None, out=None):
    """Sampling verify of a ragged batch (request b has cu_draft[b+1] - cu_draft[b]
    drafts); packed inputs: logits [n_draft + B, V], q [n_draft, V], ids and
    u_accept [n_draft], u_resample [n_draft + B], cu_draft [B + 1] int32 on the
    device.  Returns (tokens [B, gamma_max + 1], n_accepted [B], flags [B])."""
    B, N, V = _ragged_shapes(logits, ids, cu_draft)
    dev = logits.device
    if N > 0:
        _check(q, "q", torch.float32, (N, V))
        _check(u_accept, "u_accept", torch.float32, (N,))
    _check(u_resample, "u_resample", torch.float32, (N + B,))
    tokens, nacc, flags = _ragged_out(out, B, gamma_max, dev)
    need = workspace_size(B, gamma_max, V, logits.dtype, temperature, top_k, top_p)
    ws = _workspace(workspace, need, dev)
    code = load_library().spec_verify_sample_ragged(
        logits.data_ptr(), _DT[logits.dtype], q.data_ptr() if N > 0 else None, ids.data_ptr() if N > 0 else None,
        cu_draft.data_ptr(), N, u_accept.data_ptr() if N > 0 else None, u_resample.data_ptr(),
        B, gamma_max, V, _params(temperature, top_k, top_p), int(eos_id),
        tokens.data_ptr(), nacc.data_ptr(), flags.data_ptr(),
        ws.data_ptr(), ws.numel() * ws.element_size(), _stream(dev))
    _raise(code, "spec_verify_sample_ragged")
    return tokens, nacc, flags


def verify_greedy_ragged(logits, ids, cu_draft, gamma_max: int, eos_id: int = -1,
                         workspace: Optional[torch.Tensor] = None, out=None):
    """Greedy verify of a ragged batch (layout as in verify_sample_ragged)."""
    B, N, V = _ragged_shapes(logits, ids, cu_draft)
    dev = logits.device
    tokens, nacc, flags = _ragged_out(out, B, gamma_max, dev)
    need = workspace_size(B, gamma_max, V, logits.dtype)
    ws = _workspace(workspace, need, dev)
    code = load_library().spec_verify_greedy_ragged(
        logits.data_ptr(), _DT[logits.dtype], ids.data_ptr() if N > 0 else None, cu_draft.data_ptr(), N,
        B, gamma_max, V, int(eos_id), tokens.data_ptr(), nacc.data_ptr(), flags.data_ptr(),
        ws.data_ptr(), ws.numel() * ws.element_size(), _stream(dev))
    _raise(code, "spec_verify_greedy_ragged")
    return tokens, nacc, flags


def _sample_stats_outs(out, stats_out, B, G, dev, z_qp):
    if out is None:
        out = (torch.empty((B, G + 1), dtype=torch.int32, device=dev),
               torch.empty((B,), dtype=torch.int32, device=dev),
               torch.empty((B,), dtype=torch.int32, device=dev))
    return out, _stats_outs(stats_out, B, G, dev, z_qp)


def verify_sample_stats(logits, q, ids, u_accept, u_resample, temperature=1.0, top_k=0, top_p=1.0,
                        workspace: Optional[torch.Tensor] = None, out=None, stats_out=None, z_qp: bool = True):
    """verify_sample and accept_stats of the same inputs from one pass over the
    logits; returns (tokens, n_accepted, flags, alpha, z_pq, z_qp, accept_prob)
    (z_qp None when not asked for)."""
    if logits.dim() != 3:
        raise ValueError("logits must be [B, gamma+1, V]")
    B, G1, V = logits.shape
    G = G1 - 1
    _check(logits, "logits", None, (B, G1, V))
    if logits.dtype not in _DT:
        raise ValueError("logits must be float32 or bfloat16")
    dev = logits.device
    if G > 0:
        _check(q, "q", torch.float32, (B, G, V))
        _check(ids, "ids", torch.int32, (B, G))
        _check(u_accept, "u_accept", torch.float32, (B, G))
    _check(u_resample, "u_resample", torch.float32, (B, G1))
    (tokens, nacc, flags), (alpha, zpq, zqp, acc) = _sample_stats_outs(out, stats_out, B, G, dev, z_qp)
    need = workspace_size(B, G, V, logits.dtype, temperature, top_k, top_p)
    ws = _workspace(workspace, need, dev)
    code = load_library().spec_verify_sample_stats(
        logits.data_ptr(), _DT[logits.dtype],
        q.data_ptr() if G > 0 else None, ids.data_ptr() if G > 0 else None,
        u_accept.data_ptr() if G > 0 else None, u_resample.data_ptr(),
        B, G, V, _params(temperature, top_k, top_p),
        tokens.data_ptr(), nacc.data_ptr(), flags.data_ptr(),
        _ptr(alpha), _ptr(zpq), _ptr(zqp), _ptr(acc),
        ws.data_ptr(), ws.numel() * ws.element_size(), _stream(dev))
    _raise(code, "spec_verify_sample_stats")
    return tokens, nacc, flags, alpha, zpq, zqp, acc


def verify_sample_stats_draft_logits(logits, draft_logits, ids, u_accept, u_resample, temperature=1.0, top_k=0,
                                     top_p=1.0, workspace: Optional[torch.Tensor] = None, out=None, stats_out=None,
                                     z_qp: bool = True):
    """verify_sample_draft_logits and accept_stats_draft_logits of the same
    inputs from one pass over each logits tensor."""
    if logits.dim() != 3:
        raise ValueError("logits must be [B, gamma+1, V]")
    B, G1, V = logits.shape
    G = G1 - 1
    _check(logits, "logits", None, (B, G1, V))
    if logits.dtype not in _DT:
        raise ValueError("logits must be float32 or bfloat16")
    dev = logits.device
    ddt = logits.dtype
    if G > 0:
        _check(draft_logits, "draft_logits", None, (B, G, V))
        if draft_logits.dtype not in _DT:
            raise ValueError("draft_logits must be float32 or bfloat16")
        ddt = draft_logits.dtype
        _check(ids, "ids", torch.int32, (B, G))
        _check(u_accept, "u_accept", torch.float32, (B, G))
    _check(u_resample, "u_resample", torch.float32, (B, G1))
    (tokens, nacc, flags), (alpha, zpq, zqp, acc) = _sample_stats_outs(out, stats_out, B, G, dev, z_qp)
    need = draft_logits_workspace_size(B, G, V, logits.dtype, ddt, temperature, top_k, top_p)
    ws = _workspace(workspace, need, dev)
    code = load_library().spec_verify_sample_stats_draft_logits(
        logits.data_ptr(), _DT[logits.dtype],
        draft_logits.data_ptr() if G > 0 else None, _DT[ddt], ids.data_ptr() if G > 0 else None,
        u_accept.data_ptr() if G > 0 else None, u_resample.data_ptr(),
        B, G, V, _params(temperature, top_k, top_p),
        tokens.data_ptr(), nacc.data_ptr(), flags.data_ptr(),
        _ptr(alpha), _ptr(zpq), _ptr(zqp), _ptr(acc),
        ws.data_ptr(), ws.numel() * ws.element_size(), _stream(dev))
    _raise(code, "spec_verify_sample_stats_draft_logits")
    return tokens, nacc, flags, alpha, zpq, zqp, acc


def verify_sample_ragged_draft_logits(logits, draft_logits, ids, cu_draft, u_accept, u_resample, gamma_max: int,
                                      temperature=1.0, top_k=0, top_p=1.0, eos_id: int = -1,
                                      workspace: Optional[torch.Tensor] = None, out=None):
    """verify_sample_ragged with q formed from the draft's logits, packed
    [n_draft, V] like ids."""
    B, N, V = _ragged_shapes(logits, ids, cu_draft)
    dev = logits.device
    ddt = logits.dtype
    if N > 0:
        _check(draft_logits, "draft_logits", None, (N, V))
        if draft_logits.dtype not in _DT:
            raise ValueError("draft_logits must be float32 or bfloat16")
        ddt = draft_logits.dtype
        _check(u_accept, "u_accept", torch.float32, (N,))
    _check(u_resample, "u_resample", torch.float32, (N + B,))
    tokens, nacc, flags = _ragged_out(out, B, gamma_max, dev)
    need = draft_logits_workspace_size(B, gamma_max, V, logits.dtype, ddt, temperature, top_k, top_p)
    ws = _workspace(workspace, need, dev)
    code = load_library().spec_verify_sample_ragged_draft_logits(
        logits.data_ptr(), _DT[logits.dtype], draft_logits.data_ptr() if N > 0 else None, _DT[ddt],
        ids.data_ptr() if N > 0 else None, cu_draft.data_ptr(), N, u_accept.data_ptr() if N > 0 else None,
        u_resample.data_ptr(), B, gamma_max, V, _params(temperature, top_k, top_p), int(eos_id),
        tokens.data_ptr(), nacc.data_ptr(), flags.data_ptr(),
        ws.data_ptr(), ws.numel() * ws.element_size(), _stream(dev))
    _raise(code, "spec_verify_sample_ragged_draft_logits")
    return tokens, nacc, flags
