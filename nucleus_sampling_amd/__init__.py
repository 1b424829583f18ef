"""Python binding of libnucleus: batched top-p (nucleus) sampling on MI355X.

Argument marshalling only.  Every step of the sampler runs in the HIP
kernels of ``libnucleus.so`` (built in-tree by ``nucleus_sampling_amd.build``);
PyTorch supplies device memory and the stream.  There is no CPU fallback:
if the library is missing or the device is not a gfx950, calls raise.

    tok, cnt = nucleus_sampling_amd.sample(logits, temperature, top_p,
                                           top_k=None, min_p=None,
                                           seed=0, step=0)[:2]

The C ABI, with the semantics of every argument, is ``include/nucleus.h``.
"""
from __future__ import annotations

import ctypes
import os
from typing import NamedTuple, Optional

import torch

__all__ = ["sample", "sample_rejection", "RejectionResult", "spec_verify", "SpecResult", "workspace_bytes", "strerror", "version", "stream_read", "NucleusError", "lib", "LIB_PATH"]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libnucleus.so")

NUCLEUS_F32 = 0
NUCLEUS_BF16 = 1
NUCLEUS_FLAG_SINGLE_WORKGROUP = 1
NUCLEUS_FLAG_SPLIT_ROWS = 2
NUCLEUS_FLAG_ROW_RACE = 4


class NucleusError(RuntimeError):
    pass


class _Options(ctypes.Structure):
    _fields_ = [
        ("dtype", ctypes.c_int32),
        ("flags", ctypes.c_int32),
        ("stream", ctypes.c_void_p),
        ("row_stride", ctypes.c_int64),
        ("workspace", ctypes.c_void_p),
        ("workspace_bytes", ctypes.c_size_t),
        ("out_min_kept_logit", ctypes.c_void_p),
        ("seeds", ctypes.c_void_p),
        ("out_logprobs", ctypes.c_void_p),
        ("history", ctypes.c_void_p),
        ("history_len", ctypes.c_int64),
        ("repetition_penalty", ctypes.c_void_p),
        ("frequency_penalty", ctypes.c_void_p),
        ("presence_penalty", ctypes.c_void_p),
        ("allowed_mask", ctypes.c_void_p),
        ("split_give_up_row", ctypes.c_int64),
    ]


_lib = None


def lib():
    """Load libnucleus.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise NucleusError(f"{LIB_PATH} is missing: build it with `python -m nucleus_sampling_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        vp, i64, u64 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_uint64
        L.nucleus_sample.argtypes = [vp, i64, i64, vp, vp, vp, vp, u64, u64, vp, vp, vp, ctypes.POINTER(_Options)]
        L.nucleus_sample.restype = ctypes.c_int
        L.nucleus_sample_noalloc.argtypes = L.nucleus_sample.argtypes
        L.nucleus_sample_noalloc.restype = ctypes.c_int
        L.nucleus_noalloc_scratch_bytes.argtypes = []
        L.nucleus_noalloc_scratch_bytes.restype = ctypes.c_size_t
        L.nucleus_sample_rejection.argtypes = [vp, i64, i64, vp, vp, vp, u64, u64, vp, vp, ctypes.POINTER(_Options)]
        L.nucleus_sample_rejection.restype = ctypes.c_int
        L.nucleus_spec_verify.argtypes = [vp, vp, vp, i64, i64, u64, u64, vp, vp, ctypes.POINTER(_Options)]
        L.nucleus_spec_verify.restype = ctypes.c_int
        L.nucleus_spec_workspace_bytes.argtypes = [i64, i64]
        L.nucleus_spec_workspace_bytes.restype = ctypes.c_size_t
        L.nucleus_workspace_bytes.argtypes = [i64, i64, ctypes.c_int32]
        L.nucleus_workspace_bytes.restype = ctypes.c_size_t
        L.nucleus_workspace_bytes_for.argtypes = [i64, i64, ctypes.c_int32, ctypes.c_int32]
        L.nucleus_workspace_bytes_for.restype = ctypes.c_size_t
        L.nucleus_strerror.argtypes = [ctypes.c_int]
        L.nucleus_strerror.restype = ctypes.c_char_p
        L.nucleus_version.argtypes = []
        L.nucleus_version.restype = ctypes.c_int
        L.nucleus_stream_read.argtypes = [vp, ctypes.c_size_t, vp, vp]
        L.nucleus_stream_read.restype = ctypes.c_int
        L.nucleus_phase_stamps.argtypes = [vp, i64]
        L.nucleus_phase_stamps.restype = ctypes.c_int
        _lib = L
    return _lib


def strerror(code: int) -> str:
    return lib().nucleus_strerror(int(code)).decode()


def version() -> int:
    return int(lib().nucleus_version())


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return NUCLEUS_F32
    if t.dtype == torch.bfloat16:
        return NUCLEUS_BF16
    raise TypeError(f"logits must be float32 or bfloat16, got {t.dtype}")


def workspace_bytes(B: int, V: int, dtype: torch.dtype = torch.float32, flags: int = 0) -> int:
    code = NUCLEUS_BF16 if dtype == torch.bfloat16 else NUCLEUS_F32
    return int(lib().nucleus_workspace_bytes_for(int(B), int(V), code, int(flags)))


_workspaces = {}


def workspace_for(device: torch.device, stream: torch.cuda.Stream, nbytes: int) -> torch.Tensor:
    """A workspace of at least ``nbytes``, cached per (device, stream): calls
    on one stream are ordered, so they may share it (its contents need no
    initial value)."""
    key = (device.index, stream.cuda_stream)
    ws = _workspaces.get(key)
    if ws is None or ws.numel() < nbytes:
        ws = torch.empty(nbytes, dtype=torch.uint8, device=device)
        _workspaces[key] = ws
    return ws


def _check(code: int, what: str):
    if code != 0:
        raise NucleusError(f"{what}: {strerror(code)} ({code})")


def _vec(t, B, dtype, name, dev):
    if t is None:
        return None
    if not torch.is_tensor(t):
        t = torch.as_tensor(t, dtype=dtype)
    if t.device != dev:
        t = t.to(dev)
    t = t.to(dtype).contiguous()
    if t.numel() != B:
        raise ValueError(f"{name} must have {B} elements")
    return t


class SampleResult(NamedTuple):
    token: torch.Tensor          # int32 [B]; -1 on a row error
    keep_count: torch.Tensor     # int32 [B]
    probs: Optional[torch.Tensor]     # float32 [B, V] or None
    min_kept_logit: Optional[torch.Tensor]  # float32 [B] or None
    logprobs: Optional[torch.Tensor] = None  # float32 [B, V] or None


def sample(logits: torch.Tensor, temperature, top_p, top_k=None, min_p=None, seed: int = 0, step: int = 0, *,
           want_probs: bool = False, want_min_kept: bool = False, out: Optional[SampleResult] = None,
           workspace: Optional[torch.Tensor] = None, stream: Optional[torch.cuda.Stream] = None,
           single_workgroup: bool = False, split_rows: bool = False, row_race: bool = False,
           seeds=None, want_logprobs: bool = False, history=None, repetition_penalty=None,
           frequency_penalty=None, presence_penalty=None, allowed_mask=None, noalloc: bool = False,
           split_give_up_row: Optional[int] = None) -> SampleResult:
    """Sample one token per row of ``logits`` [B, V] (float32 or bfloat16 on a
    gfx950 device; rows may be strided, the last dimension must be dense).

    Launches on ``stream`` (default: the current stream) and returns without
    synchronising.  ``out`` may supply preallocated outputs; ``workspace`` a
    byte tensor of at least ``workspace_bytes(B, V, dtype)`` (by default one
    is cached per device and stream).  ``seeds`` (optional [B] integers)
    gives every row its own Philox key; ``want_logprobs`` also returns the
    log-probabilities of the processed distribution.  ``single_workgroup`` runs every row
    on one workgroup that re-reads the row; ``split_rows`` splits every row
    over workgroups whatever the batch size; ``row_race`` takes the
    large-batch path (a workgroup per row, the race spread over chunks)
    whatever the batch size.  All give the same results, bit for bit; they
    exist for verification.

    The pre-chain (``include/nucleus.h``): ``history`` [B, H] token ids
    (-1 padded, H <= 1024) with ``repetition_penalty`` / ``frequency_penalty``
    / ``presence_penalty`` [B], and ``allowed_mask`` [B, ceil(V/32)] 32-bit
    words (bit i % 32 of word i // 32 allows token i), applied to the raw
    logits before the chain.

    ``noalloc`` calls nucleus_sample_noalloc instead: the library's static
    per-GPU scratch replaces the workspace (nothing is allocated for it).

    ``split_give_up_row`` (tests of the failure path only): on the split-row
    path, that row's workgroups give up their waits at once and the row
    reports token -2.
    """
    if logits.dim() != 2:
        raise ValueError("logits must be [B, V]")
    if not logits.is_cuda:
        raise NucleusError("logits must be on the GPU: this library has no CPU path")
    B, V = logits.shape
    if V > 1 and logits.stride(1) != 1:
        raise ValueError("the vocabulary dimension of logits must be contiguous")
    dev = logits.device
    code = _dtype_code(logits)
    T = _vec(temperature, B, torch.float32, "temperature", dev)
    P = _vec(top_p, B, torch.float32, "top_p", dev)
    K = _vec(top_k, B, torch.int32, "top_k", dev)
    MP = _vec(min_p, B, torch.float32, "min_p", dev)
    S = _seeds(seeds, B, dev)
    Hs = None
    if history is not None:
        Hs = torch.as_tensor(history).to(dev).to(torch.int32).reshape(B, -1).contiguous()
    RP = _vec(repetition_penalty, B, torch.float32, "repetition_penalty", dev)
    FP = _vec(frequency_penalty, B, torch.float32, "frequency_penalty", dev)
    PP = _vec(presence_penalty, B, torch.float32, "presence_penalty", dev)
    AM = None
    if allowed_mask is not None:
        am = torch.as_tensor(allowed_mask)
        if am.dtype == torch.uint32:
            am = am.view(torch.int32)
        AM = am.to(dev).to(torch.int32).reshape(B, (V + 31) // 32).contiguous()
    if out is None:
        out = SampleResult(
            torch.empty(B, dtype=torch.int32, device=dev),
            torch.empty(B, dtype=torch.int32, device=dev),
            torch.empty((B, V), dtype=torch.float32, device=dev) if want_probs else None,
            torch.empty(B, dtype=torch.float32, device=dev) if want_min_kept else None,
            torch.empty((B, V), dtype=torch.float32, device=dev) if want_logprobs else None,
        )
    s = stream if stream is not None else torch.cuda.current_stream(dev)
    flags = ((NUCLEUS_FLAG_SINGLE_WORKGROUP if single_workgroup else 0) | (NUCLEUS_FLAG_SPLIT_ROWS if split_rows else 0)
             | (NUCLEUS_FLAG_ROW_RACE if row_race else 0))
    need = 0 if noalloc else workspace_bytes(B, V, logits.dtype, flags)
    if need and (workspace is None or workspace.numel() * workspace.element_size() < need):
        workspace = workspace_for(dev, s, need)
    opt = _Options()
    opt.dtype = code
    opt.flags = flags
    opt.stream = s.cuda_stream
    opt.row_stride = logits.stride(0) if B > 1 else V
    opt.workspace = workspace.data_ptr() if (workspace is not None and need) else None
    opt.workspace_bytes = (workspace.numel() * workspace.element_size()) if (workspace is not None and need) else 0
    opt.out_min_kept_logit = out.min_kept_logit.data_ptr() if out.min_kept_logit is not None else None
    opt.seeds = S.data_ptr() if S is not None else None
    opt.out_logprobs = out.logprobs.data_ptr() if out.logprobs is not None else None
    if Hs is not None and Hs.shape[1] > 0:
        opt.history = Hs.data_ptr()
        opt.history_len = Hs.shape[1]
    opt.repetition_penalty = RP.data_ptr() if RP is not None else None
    opt.frequency_penalty = FP.data_ptr() if FP is not None else None
    opt.presence_penalty = PP.data_ptr() if PP is not None else None
    opt.allowed_mask = AM.data_ptr() if AM is not None else None
    opt.split_give_up_row = 0 if split_give_up_row is None else int(split_give_up_row) + 1

    def ptr(t):
        return None if t is None else t.data_ptr()

    entry = lib().nucleus_sample_noalloc if noalloc else lib().nucleus_sample
    rc = entry(ptr(logits), B, V, ptr(T), ptr(P), ptr(K), ptr(MP), ctypes.c_uint64(seed),
               ctypes.c_uint64(step), ptr(out.token), ptr(out.keep_count), ptr(out.probs),
               ctypes.byref(opt))
    _check(rc, "nucleus_sample_noalloc" if noalloc else "nucleus_sample")
    return out


def _seeds(seeds, B, dev):
    if seeds is None:
        return None
    # uint64 keys travel as their int64 bit patterns
    S = torch.as_tensor([int(v) & (2**64 - 1) for v in torch.as_tensor(seeds).reshape(-1).tolist()],
                        dtype=torch.uint64).view(torch.int64).to(dev).contiguous()
    if S.numel() != B:
        raise ValueError(f"seeds must have {B} elements")
    return S


class RejectionResult(NamedTuple):
    token: torch.Tensor   # int32 [B]; -1 on a row error or without acceptance
    rounds: torch.Tensor  # int32 [B]: proposal rounds (0 for greedy and error rows)


def sample_rejection(logits: torch.Tensor, temperature, top_p, min_p=None, seed: int = 0, step: int = 0, *,
                     seeds=None, out: Optional[RejectionResult] = None,
                     stream: Optional[torch.cuda.Stream] = None) -> RejectionResult:
    """Sort-free top-p by rejection (``nucleus_sample_rejection``): one token
    per row of ``logits`` [B, V] for the chain temperature -> min-p -> top-p,
    and the number of proposal rounds each row took.  With the same seed,
    step and parameters it draws the token ``sample`` draws (top_k None), up
    to rows within rounding of a boundary.  Asynchronous on ``stream``."""
    if logits.dim() != 2:
        raise ValueError("logits must be [B, V]")
    if not logits.is_cuda:
        raise NucleusError("logits must be on the GPU: this library has no CPU path")
    B, V = logits.shape
    if V > 1 and logits.stride(1) != 1:
        raise ValueError("the vocabulary dimension of logits must be contiguous")
    dev = logits.device
    code = _dtype_code(logits)
    T = _vec(temperature, B, torch.float32, "temperature", dev)
    P = _vec(top_p, B, torch.float32, "top_p", dev)
    MP = _vec(min_p, B, torch.float32, "min_p", dev)
    S = _seeds(seeds, B, dev)
    if out is None:
        out = RejectionResult(torch.empty(B, dtype=torch.int32, device=dev),
                              torch.empty(B, dtype=torch.int32, device=dev))
    s = stream if stream is not None else torch.cuda.current_stream(dev)
    opt = _Options()
    opt.dtype = code
    opt.stream = s.cuda_stream
    opt.row_stride = logits.stride(0) if B > 1 else V
    opt.seeds = S.data_ptr() if S is not None else None

    def ptr(t):
        return None if t is None else t.data_ptr()

    rc = lib().nucleus_sample_rejection(ptr(logits), B, V, ptr(T), ptr(P), ptr(MP), ctypes.c_uint64(seed),
                                        ctypes.c_uint64(step), ptr(out.token), ptr(out.rounds), ctypes.byref(opt))
    _check(rc, "nucleus_sample_rejection")
    return out


class SpecResult(NamedTuple):
    token: torch.Tensor     # int32 [B]: the draft token if accepted, else the residual draw; -1 on errors
    accepted: torch.Tensor  # int32 [B]: 1 if the draft token was accepted


def spec_verify(target_probs: torch.Tensor, draft_probs: torch.Tensor, draft_token, seed: int = 0, step: int = 0, *,
                seeds=None, out: Optional[SpecResult] = None, workspace: Optional[torch.Tensor] = None,
                stream: Optional[torch.cuda.Stream] = None) -> SpecResult:
    """Speculative acceptance (``nucleus_spec_verify``): accept each row's
    draft token with probability min(1, p/q), else draw from the normalised
    positive part of p - q.  ``target_probs`` must be the target's truncated
    distribution (``sample(..., want_probs=True).probs``); ``draft_probs`` the
    draft's sampling distribution; both float32 [B, V] on the GPU."""
    for name, t in (("target_probs", target_probs), ("draft_probs", draft_probs)):
        if t.dim() != 2 or t.dtype != torch.float32 or not t.is_cuda:
            raise ValueError(f"{name} must be a float32 [B, V] tensor on the GPU")
    if target_probs.shape != draft_probs.shape:
        raise ValueError("target_probs and draft_probs must have the same shape")
    B, V = target_probs.shape
    dev = target_probs.device
    Pt = target_probs.contiguous()
    Qt = draft_probs.contiguous()
    D = _vec(draft_token, B, torch.int32, "draft_token", dev)
    S = _seeds(seeds, B, dev)
    if out is None:
        out = SpecResult(torch.empty(B, dtype=torch.int32, device=dev), torch.empty(B, dtype=torch.int32, device=dev))
    s = stream if stream is not None else torch.cuda.current_stream(dev)
    need = lib().nucleus_spec_workspace_bytes(B, V)
    if need and (workspace is None or workspace.numel() * workspace.element_size() < need):
        workspace = workspace_for(dev, s, need)
    opt = _Options()
    opt.stream = s.cuda_stream
    opt.seeds = S.data_ptr() if S is not None else None
    opt.workspace = workspace.data_ptr() if (workspace is not None and need) else None
    opt.workspace_bytes = (workspace.numel() * workspace.element_size()) if (workspace is not None and need) else 0
    rc = lib().nucleus_spec_verify(Pt.data_ptr() if B else None, Qt.data_ptr() if B else None,
                                   D.data_ptr() if B else None, B, V, ctypes.c_uint64(seed), ctypes.c_uint64(step),
                                   out.token.data_ptr() if B else None, out.accepted.data_ptr() if B else None,
                                   ctypes.byref(opt))
    _check(rc, "nucleus_spec_verify")
    return out


def stream_read(buf: torch.Tensor, sink: torch.Tensor, stream: Optional[torch.cuda.Stream] = None):
    """Read every byte of ``buf`` once (the HBM read ceiling); ``sink`` is a
    device tensor of 256 int64 words that receives an XOR checksum."""
    if sink.numel() * sink.element_size() < 256 * 8:
        raise ValueError("sink must hold 256 uint64 words")
    s = stream if stream is not None else torch.cuda.current_stream(buf.device)
    rc = lib().nucleus_stream_read(buf.data_ptr(), buf.numel() * buf.element_size(), sink.data_ptr(), s.cuda_stream)
    _check(rc, "nucleus_stream_read")
