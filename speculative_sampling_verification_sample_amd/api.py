"""Python binding of the verify step: torch tensors in, torch tensors out.

Marshalling only -- shapes, dtypes, devices and layouts of every tensor
handed over (inputs, caller-supplied outputs and the workspace) are checked,
missing outputs and workspace are allocated with torch on the logits'
device, and the C ABI is called on torch's current stream.  Every step of
the computation runs in the HIP kernels of libspecverify.so.
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


def _check(t: torch.Tensor, name: str, dtype, shape, device=None) -> None:
    """t is a contiguous GPU tensor of this shape (and dtype: one dtype, a
    tuple of allowed dtypes, or None for any), on `device` when given."""
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be on a GPU")
    if device is not None and t.device != device:
        raise ValueError(f"{name} must be on {device}, got {t.device}")
    if isinstance(dtype, tuple):
        if t.dtype not in dtype:
            raise ValueError(f"{name} must be one of {dtype}, got {t.dtype}")
    elif dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


_LOGIT_DT = (torch.float32, torch.bfloat16)


def _raise(code: int, what: str) -> None:
    if code != SV_OK:
        raise RuntimeError(f"{what}: {status_string(code)} (status {code})")


def _nbytes(t: torch.Tensor) -> int:
    return t.numel() * t.element_size()


def _logits3(logits):
    """(B, gamma + 1, V) of uniform-batch logits [B, gamma+1, V], checked."""
    if not isinstance(logits, torch.Tensor) or logits.dim() != 3:
        raise ValueError("logits must be a [B, gamma+1, V] tensor")
    B, G1, V = logits.shape
    _check(logits, "logits", _LOGIT_DT, (B, G1, V))
    return B, G1, V


def _sample_inputs(logits, q_name, q, ids, u_accept, u_resample, B, G, V, q_dtype):
    """The sampling calls' per-position inputs (unused, and may be None, when
    gamma = 0).  Returns q's dtype (the logits' when gamma = 0)."""
    dev = logits.device
    qdt = logits.dtype
    if G > 0:
        _check(q, q_name, q_dtype, (B, G, V), dev)
        qdt = q.dtype
        _check(ids, "ids", torch.int32, (B, G), dev)
        _check(u_accept, "u_accept", torch.float32, (B, G), dev)
    _check(u_resample, "u_resample", torch.float32, (B, G + 1), dev)
    return qdt


def _outs(out, B, P1, dev):
    """(tokens [B, P1], n_accepted [B], flags [B]) int32 on dev: allocated,
    or the caller's, checked."""
    if out is None:
        return (torch.empty((B, P1), dtype=torch.int32, device=dev),
                torch.empty((B,), dtype=torch.int32, device=dev),
                torch.empty((B,), dtype=torch.int32, device=dev))
    tokens, nacc, flags = out
    _check(tokens, "out tokens", torch.int32, (B, P1), dev)
    _check(nacc, "out n_accepted", torch.int32, (B,), dev)
    _check(flags, "out flags", torch.int32, (B,), dev)
    return tokens, nacc, flags


def _stats_outs(stats_out, B, G, dev, z_qp):
    """(alpha, Z, Z', accept_prob) buffers, each [B, gamma] float32 on dev or
    None (not computed).  Without Z' (z_qp=False) a position whose p is
    truncated to a kept set reads q only at that set's ids."""
    if stats_out is None:
        return tuple(None if (k == 2 and not z_qp) else torch.empty((B, G), dtype=torch.float32, device=dev)
                     for k in range(4))
    if len(stats_out) != 4:
        raise ValueError("stats_out must hold (alpha, z_pq, z_qp, accept_prob)")
    for name, t in zip(("alpha", "z_pq", "z_qp", "accept_prob"), stats_out):
        if t is not None:
            _check(t, f"stats_out {name}", torch.float32, (B, G), dev)
    return tuple(stats_out)


def _workspace(ws: Optional[torch.Tensor], need: int, device) -> torch.Tensor:
    """The caller's workspace (a contiguous uint8 tensor on the logits'
    device, 16-byte aligned, at least `need` bytes), or a new one."""
    if ws is None:
        return torch.empty(need, dtype=torch.uint8, device=device)
    _check(ws, "workspace", torch.uint8, (ws.numel(),), device)
    if _nbytes(ws) < need:
        raise ValueError(f"workspace holds {_nbytes(ws)} bytes, {need} needed")
    if ws.data_ptr() % 16 != 0:
        raise ValueError("workspace must be 16-byte aligned")
    return ws


def _stream(device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


def _ptr(t):
    return None if t is None else t.data_ptr()


def _if(cond, t):
    return t.data_ptr() if cond else None


def workspace_size(B: int, gamma: int, V: int, dtype=torch.bfloat16, temperature=1.0, top_k=0, top_p=1.0) -> int:
    n = load_library().spec_verify_workspace_size(B, gamma, V, _DT[dtype], _params(temperature, top_k, top_p))
    if n == 0:
        raise ValueError("invalid sizes or sampling parameters")
    return int(n)


def draft_logits_workspace_size(B: int, gamma: int, V: int, dtype=torch.bfloat16, draft_dtype=torch.bfloat16,
                                temperature=1.0, top_k=0, top_p=1.0) -> int:
    n = load_library().spec_verify_draft_logits_workspace_size(
        B, gamma, V, _DT[dtype], _DT[draft_dtype], _params(temperature, top_k, top_p))
    if n == 0:
        raise ValueError("invalid sizes or sampling parameters")
    return int(n)


def verify_sample(logits, q, ids, u_accept, u_resample, temperature=1.0, top_k=0, top_p=1.0,
                  workspace: Optional[torch.Tensor] = None, out=None):
    """Sampling verify step; returns (tokens [B, gamma+1] int32, n_accepted [B] int32, flags [B] int32)."""
    B, G1, V = _logits3(logits)
    G, dev = G1 - 1, logits.device
    _sample_inputs(logits, "q", q, ids, u_accept, u_resample, B, G, V, torch.float32)
    tokens, nacc, flags = _outs(out, B, G1, dev)
    ws = _workspace(workspace, workspace_size(B, G, V, logits.dtype, temperature, top_k, top_p), dev)
    code = load_library().spec_verify_sample(
        logits.data_ptr(), _DT[logits.dtype], _if(G > 0, q), _if(G > 0, ids), _if(G > 0, u_accept),
        u_resample.data_ptr(), B, G, V, _params(temperature, top_k, top_p),
        tokens.data_ptr(), nacc.data_ptr(), flags.data_ptr(), ws.data_ptr(), _nbytes(ws), _stream(dev))
    _raise(code, "spec_verify_sample")
    return tokens, nacc, flags


def verify_sample_noalloc(logits, q, ids, u_accept, u_resample, temperature=1.0, top_k=0, top_p=1.0, out=None):
    """verify_sample through the allocation-free entry point: the library's
    static per-GPU scratch replaces the workspace (sizes whose workspace
    exceeds it are refused), and calls on one GPU must not overlap.  Pass
    `out` to allocate nothing here either."""
    B, G1, V = _logits3(logits)
    G, dev = G1 - 1, logits.device
    _sample_inputs(logits, "q", q, ids, u_accept, u_resample, B, G, V, torch.float32)
    tokens, nacc, flags = _outs(out, B, G1, dev)
    code = load_library().spec_verify_sample_noalloc(
        logits.data_ptr(), _DT[logits.dtype], _if(G > 0, q), _if(G > 0, ids), _if(G > 0, u_accept),
        u_resample.data_ptr(), B, G, V, _params(temperature, top_k, top_p),
        tokens.data_ptr(), nacc.data_ptr(), flags.data_ptr(), _stream(dev))
    _raise(code, "spec_verify_sample_noalloc")
    return tokens, nacc, flags


def verify_sample_lenient(logits, q, ids, u_accept, u_resample, temperature=1.0, top_k=0, top_p=1.0,
                          lenience=1.0, workspace: Optional[torch.Tensor] = None, out=None):
    """Sampling verify step with lenient acceptance u < p / (lenience * q),
    0 < lenience <= 1 (1: exactly verify_sample); returns (tokens, n_accepted, flags)."""
    B, G1, V = _logits3(logits)
    G, dev = G1 - 1, logits.device
    _sample_inputs(logits, "q", q, ids, u_accept, u_resample, B, G, V, torch.float32)
    tokens, nacc, flags = _outs(out, B, G1, dev)
    ws = _workspace(workspace, workspace_size(B, G, V, logits.dtype, temperature, top_k, top_p), dev)
    code = load_library().spec_verify_sample_lenient(
        logits.data_ptr(), _DT[logits.dtype], _if(G > 0, q), _if(G > 0, ids), _if(G > 0, u_accept),
        u_resample.data_ptr(), B, G, V, _params(temperature, top_k, top_p), float(lenience),
        tokens.data_ptr(), nacc.data_ptr(), flags.data_ptr(), ws.data_ptr(), _nbytes(ws), _stream(dev))
    _raise(code, "spec_verify_sample_lenient")
    return tokens, nacc, flags


def verify_greedy(logits, ids, workspace: Optional[torch.Tensor] = None, out=None):
    """Greedy verify step; returns (tokens, n_accepted, flags)."""
    B, G1, V = _logits3(logits)
    G, dev = G1 - 1, logits.device
    if G > 0:
        _check(ids, "ids", torch.int32, (B, G), dev)
    tokens, nacc, flags = _outs(out, B, G1, dev)
    ws = _workspace(workspace, workspace_size(B, G, V, logits.dtype), dev)
    code = load_library().spec_verify_greedy(
        logits.data_ptr(), _DT[logits.dtype], _if(G > 0, ids), B, G, V,
        tokens.data_ptr(), nacc.data_ptr(), flags.data_ptr(), ws.data_ptr(), _nbytes(ws), _stream(dev))
    _raise(code, "spec_verify_greedy")
    return tokens, nacc, flags


def accept_stats(logits, q, ids, temperature=1.0, top_k=0, top_p=1.0,
                 workspace: Optional[torch.Tensor] = None, out=None, z_qp: bool = True):
    """Per-position (alpha, Z, Z', accept_prob), each [B, gamma] float32 (Z'
    None when z_qp is False)."""
    B, G1, V = _logits3(logits)
    G, dev = G1 - 1, logits.device
    _check(q, "q", torch.float32, (B, G, V), dev)
    _check(ids, "ids", torch.int32, (B, G), dev)
    alpha, zpq, zqp, acc = _stats_outs(out, B, G, dev, z_qp)
    ws = _workspace(workspace, workspace_size(B, G, V, logits.dtype, temperature, top_k, top_p), dev)
    code = load_library().spec_accept_stats(
        logits.data_ptr(), _DT[logits.dtype], q.data_ptr(), ids.data_ptr(), B, G, V,
        _params(temperature, top_k, top_p), _ptr(alpha), _ptr(zpq), _ptr(zqp), _ptr(acc),
        ws.data_ptr(), _nbytes(ws), _stream(dev))
    _raise(code, "spec_accept_stats")
    return alpha, zpq, zqp, acc


def verify_sample_draft_logits(logits, draft_logits, ids, u_accept, u_resample, temperature=1.0, top_k=0,
                               top_p=1.0, workspace: Optional[torch.Tensor] = None, out=None):
    """Sampling verify step with q formed from the draft's logits [B, gamma, V]
    by the same rules as p; returns (tokens, n_accepted, flags)."""
    B, G1, V = _logits3(logits)
    G, dev = G1 - 1, logits.device
    ddt = _sample_inputs(logits, "draft_logits", draft_logits, ids, u_accept, u_resample, B, G, V, _LOGIT_DT)
    tokens, nacc, flags = _outs(out, B, G1, dev)
    need = draft_logits_workspace_size(B, G, V, logits.dtype, ddt, temperature, top_k, top_p)
    ws = _workspace(workspace, need, dev)
    code = load_library().spec_verify_sample_draft_logits(
        logits.data_ptr(), _DT[logits.dtype], _if(G > 0, draft_logits), _DT[ddt], _if(G > 0, ids),
        _if(G > 0, u_accept), u_resample.data_ptr(), B, G, V, _params(temperature, top_k, top_p),
        tokens.data_ptr(), nacc.data_ptr(), flags.data_ptr(), ws.data_ptr(), _nbytes(ws), _stream(dev))
    _raise(code, "spec_verify_sample_draft_logits")
    return tokens, nacc, flags


def accept_stats_draft_logits(logits, draft_logits, ids, temperature=1.0, top_k=0, top_p=1.0,
                              workspace: Optional[torch.Tensor] = None, out=None, z_qp: bool = True):
    """Per-position (alpha, Z, Z', accept_prob) with q formed from the draft's
    logits (Z' None when z_qp is False)."""
    B, G1, V = _logits3(logits)
    G, dev = G1 - 1, logits.device
    _check(draft_logits, "draft_logits", _LOGIT_DT, (B, G, V), dev)
    _check(ids, "ids", torch.int32, (B, G), dev)
    alpha, zpq, zqp, acc = _stats_outs(out, B, G, dev, z_qp)
    need = draft_logits_workspace_size(B, G, V, logits.dtype, draft_logits.dtype, temperature, top_k, top_p)
    ws = _workspace(workspace, need, dev)
    code = load_library().spec_accept_stats_draft_logits(
        logits.data_ptr(), _DT[logits.dtype], draft_logits.data_ptr(), _DT[draft_logits.dtype], ids.data_ptr(),
        B, G, V, _params(temperature, top_k, top_p), _ptr(alpha), _ptr(zpq), _ptr(zqp),
        _ptr(acc), ws.data_ptr(), _nbytes(ws), _stream(dev))
    _raise(code, "spec_accept_stats_draft_logits")
    return alpha, zpq, zqp, acc


def verify_sample_stats(logits, q, ids, u_accept, u_resample, temperature=1.0, top_k=0, top_p=1.0,
                        workspace: Optional[torch.Tensor] = None, out=None, stats_out=None, z_qp: bool = True):
    """verify_sample and accept_stats of the same inputs from one pass over the
    logits; returns (tokens, n_accepted, flags, alpha, z_pq, z_qp, accept_prob)
    (z_qp None when not asked for)."""
    B, G1, V = _logits3(logits)
    G, dev = G1 - 1, logits.device
    _sample_inputs(logits, "q", q, ids, u_accept, u_resample, B, G, V, torch.float32)
    tokens, nacc, flags = _outs(out, B, G1, dev)
    alpha, zpq, zqp, acc = _stats_outs(stats_out, B, G, dev, z_qp)
    ws = _workspace(workspace, workspace_size(B, G, V, logits.dtype, temperature, top_k, top_p), dev)
    code = load_library().spec_verify_sample_stats(
        logits.data_ptr(), _DT[logits.dtype], _if(G > 0, q), _if(G > 0, ids), _if(G > 0, u_accept),
        u_resample.data_ptr(), B, G, V, _params(temperature, top_k, top_p),
        tokens.data_ptr(), nacc.data_ptr(), flags.data_ptr(), _ptr(alpha), _ptr(zpq), _ptr(zqp), _ptr(acc),
        ws.data_ptr(), _nbytes(ws), _stream(dev))
    _raise(code, "spec_verify_sample_stats")
    return tokens, nacc, flags, alpha, zpq, zqp, acc


def verify_sample_stats_draft_logits(logits, draft_logits, ids, u_accept, u_resample, temperature=1.0, top_k=0,
                                     top_p=1.0, workspace: Optional[torch.Tensor] = None, out=None, stats_out=None,
                                     z_qp: bool = True):
    """verify_sample_draft_logits and accept_stats_draft_logits of the same
    inputs from one pass over each logits tensor."""
    B, G1, V = _logits3(logits)
    G, dev = G1 - 1, logits.device
    ddt = _sample_inputs(logits, "draft_logits", draft_logits, ids, u_accept, u_resample, B, G, V, _LOGIT_DT)
    tokens, nacc, flags = _outs(out, B, G1, dev)
    alpha, zpq, zqp, acc = _stats_outs(stats_out, B, G, dev, z_qp)
    need = draft_logits_workspace_size(B, G, V, logits.dtype, ddt, temperature, top_k, top_p)
    ws = _workspace(workspace, need, dev)
    code = load_library().spec_verify_sample_stats_draft_logits(
        logits.data_ptr(), _DT[logits.dtype], _if(G > 0, draft_logits), _DT[ddt], _if(G > 0, ids),
        _if(G > 0, u_accept), u_resample.data_ptr(), B, G, V, _params(temperature, top_k, top_p),
        tokens.data_ptr(), nacc.data_ptr(), flags.data_ptr(), _ptr(alpha), _ptr(zpq), _ptr(zqp), _ptr(acc),
        ws.data_ptr(), _nbytes(ws), _stream(dev))
    _raise(code, "spec_verify_sample_stats_draft_logits")
    return tokens, nacc, flags, alpha, zpq, zqp, acc


# ---- ragged batches ------------------------------------------------------------

def _ragged_shapes(logits, ids, cu):
    """(B, n_draft, V) of a ragged call's packed logits [n_draft + B, V],
    ids [n_draft] and offsets cu [B + 1], checked."""
    if not isinstance(logits, torch.Tensor) or logits.dim() != 2:
        raise ValueError("ragged logits must be packed [n_draft + B, V]")
    dev = logits.device
    if not isinstance(cu, torch.Tensor) or cu.dim() != 1:
        raise ValueError("cu_draft must be a [B + 1] tensor")
    _check(cu, "cu_draft", torch.int32, (cu.shape[0],), dev)
    B = cu.shape[0] - 1
    if B < 0:
        raise ValueError("cu_draft must hold B + 1 offsets")
    N = ids.shape[0] if ids is not None else 0
    V = logits.shape[1]
    _check(logits, "logits", _LOGIT_DT, (N + B, V))
    if N > 0:
        _check(ids, "ids", torch.int32, (N,), dev)
    return B, N, V


def _ragged_inputs(logits, q_name, q, u_accept, u_resample, B, N, V, q_dtype):
    dev = logits.device
    qdt = logits.dtype
    if N > 0:
        _check(q, q_name, q_dtype, (N, V), dev)
        qdt = q.dtype
        _check(u_accept, "u_accept", torch.float32, (N,), dev)
    _check(u_resample, "u_resample", torch.float32, (N + B,), dev)
    return qdt


def verify_sample_ragged(logits, q, ids, cu_draft, u_accept, u_resample, gamma_max: int, temperature=1.0, top_k=0,
                         top_p=1.0, eos_id: int = -1, workspace: Optional[torch.Tensor] = None, out=None):
    """Sampling verify of a ragged batch (request b has cu_draft[b+1] - cu_draft[b]
    drafts); packed inputs: logits [n_draft + B, V], q [n_draft, V], ids and
    u_accept [n_draft], u_resample [n_draft + B], cu_draft [B + 1] int32 on the
    device.  Returns (tokens [B, gamma_max + 1], n_accepted [B], flags [B])."""
    B, N, V = _ragged_shapes(logits, ids, cu_draft)
    dev = logits.device
    _ragged_inputs(logits, "q", q, u_accept, u_resample, B, N, V, torch.float32)
    tokens, nacc, flags = _outs(out, B, gamma_max + 1, dev)
    ws = _workspace(workspace, workspace_size(B, gamma_max, V, logits.dtype, temperature, top_k, top_p), dev)
    code = load_library().spec_verify_sample_ragged(
        logits.data_ptr(), _DT[logits.dtype], _if(N > 0, q), _if(N > 0, ids), cu_draft.data_ptr(), N,
        _if(N > 0, u_accept), u_resample.data_ptr(), B, gamma_max, V, _params(temperature, top_k, top_p),
        int(eos_id), tokens.data_ptr(), nacc.data_ptr(), flags.data_ptr(), ws.data_ptr(), _nbytes(ws), _stream(dev))
    _raise(code, "spec_verify_sample_ragged")
    return tokens, nacc, flags


def verify_greedy_ragged(logits, ids, cu_draft, gamma_max: int, eos_id: int = -1,
                         workspace: Optional[torch.Tensor] = None, out=None):
    """Greedy verify of a ragged batch (layout as in verify_sample_ragged)."""
    B, N, V = _ragged_shapes(logits, ids, cu_draft)
    dev = logits.device
    tokens, nacc, flags = _outs(out, B, gamma_max + 1, dev)
    ws = _workspace(workspace, workspace_size(B, gamma_max, V, logits.dtype), dev)
    code = load_library().spec_verify_greedy_ragged(
        logits.data_ptr(), _DT[logits.dtype], _if(N > 0, ids), cu_draft.data_ptr(), N,
        B, gamma_max, V, int(eos_id), tokens.data_ptr(), nacc.data_ptr(), flags.data_ptr(),
        ws.data_ptr(), _nbytes(ws), _stream(dev))
    _raise(code, "spec_verify_greedy_ragged")
    return tokens, nacc, flags


def verify_sample_ragged_draft_logits(logits, draft_logits, ids, cu_draft, u_accept, u_resample, gamma_max: int,
                                      temperature=1.0, top_k=0, top_p=1.0, eos_id: int = -1,
                                      workspace: Optional[torch.Tensor] = None, out=None):
    """verify_sample_ragged with q formed from the draft's logits, packed
    [n_draft, V] like ids."""
    B, N, V = _ragged_shapes(logits, ids, cu_draft)
    dev = logits.device
    ddt = _ragged_inputs(logits, "draft_logits", draft_logits, u_accept, u_resample, B, N, V, _LOGIT_DT)
    tokens, nacc, flags = _outs(out, B, gamma_max + 1, dev)
    need = draft_logits_workspace_size(B, gamma_max, V, logits.dtype, ddt, temperature, top_k, top_p)
    ws = _workspace(workspace, need, dev)
    code = load_library().spec_verify_sample_ragged_draft_logits(
        logits.data_ptr(), _DT[logits.dtype], _if(N > 0, draft_logits), _DT[ddt], _if(N > 0, ids),
        cu_draft.data_ptr(), N, _if(N > 0, u_accept), u_resample.data_ptr(), B, gamma_max, V,
        _params(temperature, top_k, top_p), int(eos_id), tokens.data_ptr(), nacc.data_ptr(), flags.data_ptr(),
        ws.data_ptr(), _nbytes(ws), _stream(dev))
    _raise(code, "spec_verify_sample_ragged_draft_logits")
    return tokens, nacc, flags
