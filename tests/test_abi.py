"""The C ABI library: it loads, exports every function include/nucleus.h
declares, and rejects bad arguments on the host without touching a GPU."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "nucleus.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(nucleus_\w+)\s*\(", text)))


@pytest.fixture(scope="module")
def L():
    import nucleus_sampling_amd as ns

    return ns.lib()


def test_header_declares_the_abi():
    names = declared_functions()
    for n in ("nucleus_sample", "nucleus_sample_rejection", "nucleus_spec_verify", "nucleus_workspace_bytes",
              "nucleus_strerror", "nucleus_version", "nucleus_stream_read"):
        assert n in names


def test_library_exports_every_declared_symbol(L):
    missing = [n for n in declared_functions() if not hasattr(L, n)]
    assert not missing, missing


def test_strerror_and_version(L):
    import nucleus_sampling_amd as ns

    assert ns.strerror(0) == "ok"
    for code in (-1, -2, -3, -4):
        assert ns.strerror(code) not in ("ok", "unknown error")
    assert ns.version() >= 100


def test_workspace_query(L):
    import nucleus_sampling_amd as ns

    assert L.nucleus_workspace_bytes(-1, 10, 0) == 0
    assert L.nucleus_workspace_bytes(4, 0, 0) == 0
    assert L.nucleus_workspace_bytes(4, 1 << 31, 0) == 0
    assert L.nucleus_workspace_bytes(4, 10, 7) == 0
    # Small batches of long rows split rows (per-chunk slots); others run a
    # workgroup per row and need nothing; the chunked-race flag needs per-row
    # state and a candidate list.
    assert L.nucleus_workspace_bytes(2, 40000, 0) > 0
    assert L.nucleus_workspace_bytes(2, 32768, 0) == 0 and L.nucleus_workspace_bytes(2, 8, 0) == 0
    assert L.nucleus_workspace_bytes(96, 128256, 0) > 0 and L.nucleus_workspace_bytes(97, 128256, 0) == 0
    assert L.nucleus_workspace_bytes(127, 40000, 0) > 0 and L.nucleus_workspace_bytes(128, 40000, 0) == 0
    assert L.nucleus_workspace_bytes(256, 128256, 0) == 0
    assert L.nucleus_workspace_bytes_for(256, 128256, 0, 1) == 0
    assert L.nucleus_workspace_bytes_for(256, 128256, 0, 4) >= 256 * (256 + 8192 * 8)
    assert L.nucleus_workspace_bytes_for(256, 128256, 0, 2) > L.nucleus_workspace_bytes_for(256, 128256, 0, 4)
    small, large = L.nucleus_workspace_bytes_for(2, 8, 0, 4), L.nucleus_workspace_bytes_for(256, 8, 0, 4)
    assert 0 < small < large and large >= 256 * 8192 * 8  # grows with the rows: per-row state and list
    assert L.nucleus_workspace_bytes_for(4, 64 * 8192 + 1, 0, 2) == 0  # too long to split
    assert L.nucleus_workspace_bytes_for(4, 100, 0, 3) == 0            # two flags
    assert L.nucleus_workspace_bytes_for(4, 100, 0, 8) == 0            # unknown flag
    assert ns.workspace_bytes(256, 128256) == L.nucleus_workspace_bytes(256, 128256, 0)


def _call(L, logits=1 << 20, B=2, V=8, T=1 << 21, P=1 << 22, tok=1 << 23, cnt=1 << 24, opt=None):
    # Fake, never-dereferenced device addresses: every case below must be
    # rejected on the host before any launch.
    return L.nucleus_sample(logits, B, V, T, P, None, None, ctypes.c_uint64(0), ctypes.c_uint64(0), tok, cnt, None,
                            opt)


def test_host_side_argument_errors(L):
    import nucleus_sampling_amd as ns

    EINVAL = -1
    assert _call(L, logits=None) == EINVAL
    assert _call(L, T=None) == EINVAL
    assert _call(L, P=None) == EINVAL
    assert _call(L, tok=None) == EINVAL
    assert _call(L, cnt=None) == EINVAL
    assert _call(L, B=-1) == EINVAL
    assert _call(L, V=0) == EINVAL
    assert _call(L, V=1 << 31) == EINVAL
    assert _call(L, logits=(1 << 20) + 2) == EINVAL  # fp32 logits not 4-byte aligned
    assert _call(L, T=(1 << 21) + 1) == EINVAL
    opt = ns._Options()
    opt.dtype = 5
    assert _call(L, opt=ctypes.byref(opt)) == EINVAL
    opt = ns._Options()
    opt.row_stride = 4  # < V
    assert _call(L, opt=ctypes.byref(opt)) == EINVAL
    for flags in (8, 3, 5, 6, 7):  # an undefined bit, or more than one flag
        opt = ns._Options()
        opt.flags = flags
        assert _call(L, opt=ctypes.byref(opt)) == EINVAL
    opt = ns._Options()
    opt.flags = 2
    assert _call(L, V=64 * 8192 + 1, opt=ctypes.byref(opt)) == EINVAL  # too long to split
    # The default path needs a workspace for these shapes.
    opt = ns._Options()
    assert _call(L, V=40000, opt=ctypes.byref(opt)) == -2


def test_empty_batch_launches_nothing(L):
    assert _call(L, B=0) == 0
    assert _call(L, B=0, logits=None, T=None, P=None, tok=None, cnt=None) == 0


def _call_rej(L, logits=1 << 20, B=2, V=8, T=1 << 21, P=1 << 22, MP=None, tok=1 << 23, rounds=1 << 24, opt=None):
    # Fake, never-dereferenced device addresses, as above.
    return L.nucleus_sample_rejection(logits, B, V, T, P, MP, ctypes.c_uint64(0), ctypes.c_uint64(0), tok, rounds,
                                      opt)


def test_rejection_host_side_argument_errors(L):
    import nucleus_sampling_amd as ns

    EINVAL = -1
    assert _call_rej(L, logits=None) == EINVAL
    assert _call_rej(L, T=None) == EINVAL
    assert _call_rej(L, P=None) == EINVAL
    assert _call_rej(L, tok=None) == EINVAL
    assert _call_rej(L, B=-1) == EINVAL
    assert _call_rej(L, V=0) == EINVAL
    assert _call_rej(L, V=1 << 31) == EINVAL
    assert _call_rej(L, logits=(1 << 20) + 2) == EINVAL
    assert _call_rej(L, MP=(1 << 25) + 2) == EINVAL
    assert _call_rej(L, rounds=(1 << 24) + 1) == EINVAL
    for field, value in (("dtype", 5), ("row_stride", 4), ("flags", 1), ("out_min_kept_logit", 1 << 26),
                         ("out_logprobs", 1 << 26)):
        opt = ns._Options()
        setattr(opt, field, value)
        assert _call_rej(L, opt=ctypes.byref(opt)) == EINVAL, field
    assert _call_rej(L, B=0) == 0
    assert _call_rej(L, B=0, logits=None, T=None, P=None, tok=None) == 0


def _call_spec(L, P=1 << 20, Q=1 << 21, D=1 << 22, B=2, V=8, tok=1 << 23, acc=1 << 24, opt=None):
    # Fake, never-dereferenced device addresses, as above.
    return L.nucleus_spec_verify(P, Q, D, B, V, ctypes.c_uint64(0), ctypes.c_uint64(0), tok, acc, opt)


def test_spec_host_side_argument_errors(L):
    import nucleus_sampling_amd as ns

    EINVAL = -1
    for kw in (dict(P=None), dict(Q=None), dict(D=None), dict(tok=None), dict(B=-1), dict(V=0), dict(V=1 << 31),
               dict(P=(1 << 20) + 2), dict(Q=(1 << 21) + 1), dict(D=(1 << 22) + 2), dict(acc=(1 << 24) + 1)):
        assert _call_spec(L, **kw) == EINVAL, kw
    for field, value in (("dtype", 1), ("row_stride", 9), ("flags", 4), ("out_min_kept_logit", 1 << 26),
                         ("out_logprobs", 1 << 26)):
        opt = ns._Options()
        setattr(opt, field, value)
        assert _call_spec(L, opt=ctypes.byref(opt)) == EINVAL, field
    assert _call_spec(L, B=0) == 0
    assert _call_spec(L, B=0, P=None, Q=None, D=None, tok=None) == 0
    assert _call_spec(L) == -2  # no workspace
    opt = ns._Options()
    opt.workspace, opt.workspace_bytes = 1 << 27, 8  # too small
    assert _call_spec(L, opt=ctypes.byref(opt)) == -2
    assert L.nucleus_spec_workspace_bytes(256, 128256) == 256 * 16 * 8
    assert L.nucleus_spec_workspace_bytes(3, 1) == 256
    assert L.nucleus_spec_workspace_bytes(-1, 8) == 0 and L.nucleus_spec_workspace_bytes(2, 0) == 0


def test_prechain_host_side_argument_errors(L):
    import nucleus_sampling_amd as ns

    EINVAL = -1

    def opt(**kw):
        o = ns._Options()
        for k, v in kw.items():
            setattr(o, k, v)
        return ctypes.byref(o)

    assert _call(L, opt=opt(history=1 << 26, history_len=1025)) == EINVAL       # history too long
    assert _call(L, opt=opt(history_len=4)) == EINVAL                           # length without ids
    assert _call(L, opt=opt(history=(1 << 26) + 2, history_len=4)) == EINVAL    # misaligned ids
    assert _call(L, opt=opt(allowed_mask=1 << 26, flags=2)) == EINVAL           # not on the split path
    assert _call(L, opt=opt(allowed_mask=1 << 26, flags=4)) == EINVAL           # nor the chunked race
    assert _call(L, V=166913, opt=opt(allowed_mask=1 << 26)) == EINVAL          # bits too long to stage
    assert _call(L, V=166913, opt=opt(presence_penalty=1 << 26)) == EINVAL
    assert _call_rej(L, opt=opt(allowed_mask=1 << 26)) == EINVAL                # other entry points refuse it
    assert _call_spec(L, opt=opt(repetition_penalty=1 << 26, workspace=1 << 27, workspace_bytes=1 << 20)) == EINVAL


def _call_na(L, logits=1 << 20, B=2, V=8, T=1 << 21, P=1 << 22, tok=1 << 23, cnt=1 << 24, opt=None):
    # Fake, never-dereferenced device addresses, as above.
    return L.nucleus_sample_noalloc(logits, B, V, T, P, None, None, ctypes.c_uint64(0), ctypes.c_uint64(0), tok, cnt,
                                    None, opt)


def test_noalloc_host_side_checks(L):
    """nucleus_sample_noalloc: its static scratch is 32 MiB per GPU; a call
    whose path needs more is refused on the host before any launch, as are
    bad arguments."""
    import nucleus_sampling_amd as ns

    assert L.nucleus_noalloc_scratch_bytes() == 32 << 20
    opt = ns._Options()
    opt.flags = 2  # split rows: 127 rows of 64 chunks need ~100 MB of per-chunk slots and lists
    assert L.nucleus_workspace_bytes_for(127, 64 * 8192, 0, 2) > L.nucleus_noalloc_scratch_bytes()
    assert _call_na(L, B=127, V=64 * 8192, opt=ctypes.byref(opt)) == -2
    assert _call_na(L, B=-1) == -1
    assert _call_na(L, V=0) == -1
    opt = ns._Options()
    opt.flags = 3  # two flags
    assert _call_na(L, opt=ctypes.byref(opt)) == -1
    assert _call_na(L, B=0) in (0, -4)  # no batch: nothing to launch (or no usable device here)


def test_phase_stamps_are_off_in_the_product_build(L):
    """The product library has no phase clocks compiled in: registering a
    buffer is refused and nothing is recorded."""
    assert L.nucleus_phase_stamps(1 << 20, 4) == -1
    assert L.nucleus_phase_stamps(None, 0) == -1
