"""C-ABI tests that need no GPU: the library loads, exports every function
include/linrec.h declares, sizes its buffers as documented, and rejects bad
arguments with the documented status before touching any device state.

The pointers below are fake addresses: a rejected call must never
dereference them, and the valid-looking calls all stop at the NULL context
check, which comes after every argument check."""
import ctypes
import os
import re

import pytest

from state_passing_amd import linrec

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "linrec.h")

FAKE = 0x10000000  # 16-byte aligned, never dereferenced


def header_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(linrec_\w+)\s*\(", src)))


def test_library_exports_every_declared_function():
    declared = header_functions()
    assert declared, "no declarations parsed"
    lib = linrec._lib()
    missing = [n for n in declared if not hasattr(lib, n)]
    assert not missing, missing
    assert sorted(linrec.EXPORTS) == declared


def test_version_and_status_strings():
    lib = linrec._lib()
    assert lib.linrec_version() >= 100
    for code in range(10):
        assert lib.linrec_status_str(code)
    assert lib.linrec_status_str(99) == b"unknown status"


def d(**kw):
    base = dict(B=1, H=16, T=4096, dk=128, dv=128, dtype=linrec.BF16, decay=linrec.DECAY_HEAD)
    base.update(kw)
    return linrec.Desc(base["B"], base["H"], base["T"], base["dk"], base["dv"], 64,
                       base["dtype"], base["decay"], base.get("out", base["dtype"]))


def test_sizes():
    # one fp32 record (state + 64 floats) per segment of 4 chunks (256 tokens)
    rec = (128 * 128 + 64) * 4
    assert linrec.states_bytes(d()) == 16 * 16 * rec
    assert linrec.states_bytes(d(dtype=linrec.F32, dk=64, dv=64)) == 16 * 16 * (64 * 64 + 64) * 4
    assert linrec.states_bytes(d(out=linrec.F32)) == linrec.states_bytes(d())
    assert linrec.states_bytes(d(T=320)) == 16 * 2 * rec     # a short last segment
    assert linrec.bwd_workspace_bytes(d()) == linrec.states_bytes(d())
    # the per-piece store is linear in the piece length only
    assert linrec.states_bytes(d(T=8192)) == 2 * linrec.states_bytes(d())
    # sequence store: the sum of the pieces' stores
    assert linrec.seq_states_bytes(d(T=8192), [2048, 4096, 2048]) == linrec.states_bytes(d(T=8192))
    assert linrec.seq_states_bytes(d(T=384), [64, 320]) == 16 * 3 * rec
    assert linrec.seq_states_bytes(d(T=384), [64, 300]) == 0            # sums to 364
    # ragged lengths: a partial last chunk counts as a chunk
    assert linrec.seq_states_bytes(d(T=364), [64, 300]) == 16 * (1 + 2) * rec
    assert linrec.states_bytes(d(T=100)) == 16 * 1 * rec
    assert linrec.states_bytes(d(T=1)) == 16 * 1 * rec
    assert linrec.states_bytes(d(T=257)) == 16 * 2 * rec
    # three slots of one piece's records, sized for the longest piece
    assert linrec.bwd_seq_workspace_bytes(d(T=8192), [2048, 4096, 2048]) == \
        3 * linrec.states_bytes(d(T=4096))
    assert linrec.bwd_seq_workspace_bytes(d(T=4096), [4096]) == 3 * linrec.states_bytes(d())
    for bad in (d(T=-64), d(dk=96), d(dtype=linrec.F32), d(B=0), d(decay=7)):
        assert linrec.states_bytes(bad) == 0
    # an empty piece is valid and needs no records
    assert linrec.states_bytes(d(T=0)) == 0 and linrec.bwd_workspace_bytes(d(T=0)) == 0
    assert linrec.seq_states_bytes(d(T=0), [0]) == 0
    assert linrec.bwd_seq_workspace_bytes(d(T=8192), [4096, 4000]) == 0


def act(ptr=FAKE, sb=16 * 4096 * 128, sh=4096 * 128, st=128):
    return linrec.Tensor(ptr, sb, sh, st)


def call_fwd(desc, q=None, k=None, v=None, decay=None, S_in=None, o=None, S_out=FAKE,
             states=FAKE, ctx=None):
    lib = linrec._lib()
    return lib.linrec_fwd(ctx, ctypes.byref(desc), q or act(), k or act(), v or act(),
                          decay or linrec.Tensor(FAKE, 0, 1, 0), S_in, o or act(), S_out,
                          states, None)


def call_bwd(desc, dq=None, workspace=FAKE, dS_in=FAKE, states=FAKE, ctx=None):
    lib = linrec._lib()
    return lib.linrec_bwd(ctx, ctypes.byref(desc), act(), act(), act(),
                          linrec.Tensor(FAKE, 0, 1, 0), states, act(), None,
                          dq or act(), act(), act(), dS_in, workspace, None)


def call_bwd_recompute(desc, S_in=None, workspace=FAKE, dS_in=FAKE, ctx=None):
    lib = linrec._lib()
    return lib.linrec_bwd_recompute(ctx, ctypes.byref(desc), act(), act(), act(),
                                    linrec.Tensor(FAKE, 0, 1, 0), S_in, act(), None,
                                    act(), act(), act(), dS_in, workspace, None)


def call_bwd_da(desc, da=None, carry_in=None, carry_out=FAKE, workspace=FAKE, ctx=None):
    lib = linrec._lib()
    return lib.linrec_bwd_da(ctx, ctypes.byref(desc), act(), act(), act(),
                             linrec.Tensor(FAKE, 0, 1, 0), FAKE, act(), None, act(), act(), act(),
                             FAKE, da or linrec.Tensor(FAKE, 16 * 4096, 4096, 1), carry_in,
                             carry_out, workspace, None)


E = {v: k for k, v in linrec.STATUS.items()}


@pytest.mark.parametrize("desc,code", [
    (d(T=-64), "LINREC_E_SHAPE"),
    (d(T=0), "LINREC_E_NULL"),             # an empty piece is valid; no context
    (d(T=2147479552), "LINREC_E_NULL"),    # LINREC_MAX_T
    (d(T=2147479553), "LINREC_E_SHAPE"),
    (d(T=2147483647), "LINREC_E_SHAPE"),
    (d(T=100), "LINREC_E_NULL"),           # a ragged length is valid; no context
    (d(dk=96), "LINREC_E_SHAPE"),
    (d(B=0), "LINREC_E_SHAPE"),
    (d(B=32767), "LINREC_E_NULL"),         # the largest batch; no context
    (d(B=32768), "LINREC_E_SHAPE"),
    (d(H=65535), "LINREC_E_NULL"),
    (d(H=65536), "LINREC_E_SHAPE"),
    (d(H=0), "LINREC_E_SHAPE"),
    (d(dtype=5), "LINREC_E_DTYPE"),
    (d(dtype=linrec.F32), "LINREC_E_DTYPE"),
    (d(dtype=linrec.F32, dk=64, dv=64, out=linrec.BF16), "LINREC_E_DTYPE"),
    (d(out=3), "LINREC_E_DTYPE"),
    (d(decay=3), "LINREC_E_LAYOUT"),
])
def test_bad_desc(desc, code):
    assert call_fwd(desc) == E[code]
    assert call_bwd(desc) == E[code]


def test_bad_tensors():
    good = d()
    assert call_fwd(good, q=act(ptr=0)) == E["LINREC_E_NULL"]
    assert call_fwd(good, k=act(ptr=FAKE + 2)) == E["LINREC_E_ALIGN"]
    assert call_fwd(good, v=act(st=100)) == E["LINREC_E_LAYOUT"]    # rows overlap
    assert call_fwd(good, o=act(st=132)) == E["LINREC_E_ALIGN"]     # 264-byte rows
    # the output's alignment is judged in the output dtype: 132 fp32 = 528-byte rows
    assert call_fwd(d(out=linrec.F32), o=act(st=132)) == E["LINREC_E_NULL"]
    assert call_fwd(good, q=act(sh=-1)) == E["LINREC_E_LAYOUT"]
    assert call_fwd(good, decay=linrec.Tensor(None, 0, 1, 0)) == E["LINREC_E_NULL"]
    assert call_fwd(good, decay=linrec.Tensor(FAKE + 2, 0, 1, 0)) == E["LINREC_E_ALIGN"]
    assert call_fwd(good, S_out=None) == E["LINREC_E_NULL"]
    assert call_fwd(good, S_in=FAKE + 2) == E["LINREC_E_ALIGN"]
    assert call_fwd(good, states=None) == E["LINREC_E_WORKSPACE"]
    assert call_fwd(good, states=FAKE + 8) == E["LINREC_E_WORKSPACE"]
    assert call_bwd(good, workspace=None) == E["LINREC_E_WORKSPACE"]
    assert call_bwd(good, dS_in=None) == E["LINREC_E_NULL"]
    assert call_bwd(good, dq=act(ptr=0)) == E["LINREC_E_NULL"]
    # no decay tensor needed when there is no decay
    assert call_fwd(d(decay=linrec.DECAY_NONE), decay=linrec.Tensor(None, 0, 0, 0)) == E["LINREC_E_NULL"]


def test_valid_arguments_stop_at_missing_context():
    # every argument check passes; the NULL context is the first thing rejected
    assert call_fwd(d()) == E["LINREC_E_NULL"]
    assert call_bwd(d()) == E["LINREC_E_NULL"]
    assert call_bwd_recompute(d()) == E["LINREC_E_NULL"]
    assert call_bwd_recompute(d(), S_in=FAKE) == E["LINREC_E_NULL"]


def test_decay_gradient_arguments():
    good = d(decay=linrec.DECAY_TOKEN)
    rec = (128 * 128 + 64) * 4
    # the gradient records plus one fp32 total per segment (padded to 256 bytes)
    assert linrec.bwd_da_workspace_bytes(good) == 16 * 16 * rec + 1024
    assert linrec.bwd_da_workspace_bytes(d(T=0)) == 0
    assert linrec.bwd_da_workspace_bytes(d(T=100, decay=linrec.DECAY_TOKEN)) > 0
    assert call_bwd_da(good) == E["LINREC_E_NULL"]            # all checks pass, no context
    assert call_bwd_da(d(decay=linrec.DECAY_HEAD)) == E["LINREC_E_NULL"]
    assert call_bwd_da(d(decay=linrec.DECAY_NONE)) == E["LINREC_E_LAYOUT"]
    assert call_bwd_da(good, da=linrec.Tensor(None, 0, 0, 1)) == E["LINREC_E_NULL"]
    assert call_bwd_da(good, da=linrec.Tensor(FAKE + 2, 0, 0, 1)) == E["LINREC_E_ALIGN"]
    assert call_bwd_da(good, da=linrec.Tensor(FAKE, 0, 0, 0)) == E["LINREC_E_LAYOUT"]
    assert call_bwd_da(good, carry_out=None) == E["LINREC_E_NULL"]
    assert call_bwd_da(good, carry_in=FAKE + 2) == E["LINREC_E_ALIGN"]
    assert call_bwd_da(good, workspace=None) == E["LINREC_E_WORKSPACE"]


def test_recompute_arguments():
    good = d()
    rec = (128 * 128 + 64) * 4
    # two record sets of the piece plus one fp32 state of scratch
    assert linrec.bwd_recompute_workspace_bytes(good) == 2 * 16 * 16 * rec + 16 * 128 * 128 * 4
    assert linrec.bwd_recompute_workspace_bytes(d(T=8192)) == \
        2 * linrec.states_bytes(d(T=8192)) + 16 * 128 * 128 * 4
    assert linrec.bwd_recompute_workspace_bytes(d(T=0)) == 0
    assert call_bwd_recompute(d(T=0)) == E["LINREC_E_NULL"]
    assert call_bwd_recompute(d(T=100)) == E["LINREC_E_NULL"]
    assert call_bwd_recompute(good, workspace=None) == E["LINREC_E_WORKSPACE"]
    assert call_bwd_recompute(good, workspace=FAKE + 8) == E["LINREC_E_WORKSPACE"]
    assert call_bwd_recompute(good, S_in=FAKE + 2) == E["LINREC_E_ALIGN"]
    assert call_bwd_recompute(good, dS_in=None) == E["LINREC_E_NULL"]


def test_bad_piece_lists():
    lib = linrec._lib()
    desc = d(T=8192)
    for lengths in ([4096, 4000], [4096], [4096, 4096, 64], [0, 8192]):
        arr = (ctypes.c_int32 * len(lengths))(*lengths)
        rc = lib.linrec_fwd_seq(None, ctypes.byref(desc), len(lengths), arr, act(), act(), act(),
                                linrec.Tensor(FAKE, 0, 1, 0), None, act(), FAKE, FAKE, None)
        # the piece list is checked before the context
        assert rc == E["LINREC_E_SHAPE"], lengths
    for lengths in ([4096, 4096], [4000, 4192], [1, 8191]):   # ragged pieces are valid
        arr = (ctypes.c_int32 * 2)(*lengths)
        assert lib.linrec_fwd_seq(None, ctypes.byref(desc), 2, arr, act(), act(), act(),
                                  linrec.Tensor(FAKE, 0, 1, 0), None, act(), FAKE, FAKE,
                                  None) == E["LINREC_E_NULL"], lengths
    assert lib.linrec_fwd_seq(None, ctypes.byref(desc), 0, arr, act(), act(), act(),
                              linrec.Tensor(FAKE, 0, 1, 0), None, act(), FAKE, FAKE,
                              None) == E["LINREC_E_SHAPE"]


def test_null_desc_and_ctx_destroy_null():
    lib = linrec._lib()
    assert lib.linrec_fwd(None, None, act(), act(), act(), linrec.Tensor(FAKE, 0, 1, 0), None,
                          act(), FAKE, FAKE, None) == E["LINREC_E_NULL"]
    assert lib.linrec_ctx_destroy(None) == 0
    assert lib.linrec_ctx_create(None, 0) == E["LINREC_E_NULL"]


def test_noalloc_arguments():
    """The no-allocation backward checks its arguments like linrec_bwd and
    rejects a piece whose gradient records exceed the fixed scratch before
    looking at the context."""
    lib = linrec._lib()

    def call(desc, states=FAKE, dS_in=FAKE):
        return lib.linrec_bwd_noalloc(None, ctypes.byref(desc), act(), act(), act(),
                                      linrec.Tensor(FAKE, 0, 1, 0), states, act(), None, act(),
                                      act(), act(), dS_in, None)
    assert call(d()) == E["LINREC_E_NULL"]                 # checks pass, no context
    assert call(d(T=7936)) == E["LINREC_E_NULL"]           # 31 segments: fits 32 MiB
    assert linrec.bwd_workspace_bytes(d(T=7936)) <= linrec.NOALLOC_SCRATCH_BYTES
    assert call(d(T=8192)) == E["LINREC_E_SCRATCH"]        # 32 segments: does not
    assert call(d(T=0)) == E["LINREC_E_NULL"]
    assert call(d(T=100)) == E["LINREC_E_NULL"]
    assert call(d(), states=None) == E["LINREC_E_WORKSPACE"]
    assert call(d(), dS_in=None) == E["LINREC_E_NULL"]


def test_delta_arguments():
    lib = linrec._lib()
    # W_k and W_v per token, then P (64 x 64) and the decay tables (256) per chunk
    assert linrec.delta_workspace_bytes(d()) == 16 * 4096 * (256 + 64 + 4) * 4
    assert linrec.delta_workspace_bytes(d(dk=64)) == 0        # d_k != d_v
    # a partial last chunk counts whole
    assert linrec.delta_workspace_bytes(d(T=100)) == 16 * 128 * (256 + 64 + 4) * 4
    assert linrec.delta_saved_bytes(d(T=100)) == linrec.delta_saved_bytes(d(T=128))
    assert linrec.delta_bwd_workspace_bytes(d(T=100)) == linrec.delta_bwd_workspace_bytes(d(T=128))

    def call(desc, beta=linrec.Tensor(FAKE, 16 * 4096, 4096, 1), ws=FAKE, saved=None):
        return lib.linrec_delta_fwd(None, ctypes.byref(desc), act(), act(), act(), beta,
                                    linrec.Tensor(FAKE, 0, 1, 0), None, act(), FAKE, saved, ws, None)
    assert call(d()) == E["LINREC_E_NULL"]                   # checks pass, no context
    assert call(d(dk=64)) == E["LINREC_E_SHAPE"]
    assert call(d(), beta=linrec.Tensor(None, 0, 0, 1)) == E["LINREC_E_NULL"]
    assert call(d(), beta=linrec.Tensor(FAKE + 2, 0, 0, 1)) == E["LINREC_E_ALIGN"]
    assert call(d(), beta=linrec.Tensor(FAKE, -1, 0, 1)) == E["LINREC_E_LAYOUT"]
    assert call(d(), ws=None) == E["LINREC_E_WORKSPACE"]
    assert call(d(), saved=FAKE + 8) == E["LINREC_E_WORKSPACE"]
    assert call(d(), saved=FAKE) == E["LINREC_E_NULL"]
    # saved: one state per chunk and U per token; backward workspace: W_k, W_v,
    # T per chunk, dU per token, one gradient state per chunk, P and the decay
    # tables per chunk
    N = 4096 // 64
    assert linrec.delta_saved_bytes(d()) == 16 * (N * 128 * 128 + 4096 * 128) * 4
    assert linrec.delta_bwd_workspace_bytes(d()) == \
        16 * (4096 * 384 + 2 * N * 64 * 64 + N * 256 + N * 128 * 128) * 4

    def bcall(desc, dbeta=linrec.Tensor(FAKE, 16 * 4096, 4096, 1), saved=FAKE):
        return lib.linrec_delta_bwd(None, ctypes.byref(desc), act(), act(), act(),
                                    linrec.Tensor(FAKE, 16 * 4096, 4096, 1),
                                    linrec.Tensor(FAKE, 0, 1, 0), saved, act(), None, act(), act(),
                                    act(), dbeta, FAKE, FAKE, None)
    assert bcall(d()) == E["LINREC_E_NULL"]
    assert bcall(d(), dbeta=linrec.Tensor(None, 0, 0, 1)) == E["LINREC_E_NULL"]
    assert bcall(d(), saved=None) == E["LINREC_E_WORKSPACE"]
    assert bcall(d(dk=64)) == E["LINREC_E_SHAPE"]


def test_delta_sequence_arguments():
    """The delta-rule sequence drivers: saved buffers of the pieces one after
    another, the workspace of the longest piece (the backward: two slots, one
    for a single piece), the piece list checked as for the linear sequence
    drivers."""
    lib = linrec._lib()
    seq = d(T=8192)
    lens = [4096, 4000, 96]
    per = [linrec.delta_saved_bytes(d(T=n)) for n in lens]
    assert linrec.delta_seq_saved_bytes(seq, lens) == sum(per)
    assert linrec.delta_fwd_seq_workspace_bytes(seq, lens) == linrec.delta_workspace_bytes(d())
    assert linrec.delta_bwd_seq_workspace_bytes(seq, lens) == \
        2 * linrec.delta_bwd_workspace_bytes(d())
    assert linrec.delta_fwd_seq_workspace_bytes(seq, [8192]) == \
        linrec.delta_workspace_bytes(d(T=8192))
    assert linrec.delta_seq_saved_bytes(seq, [8192]) == linrec.delta_saved_bytes(d(T=8192))
    assert linrec.delta_seq_saved_bytes(seq, [4096, 4000]) == 0      # does not sum to T
    assert linrec.delta_seq_saved_bytes(d(T=8192, dk=64), [8192]) == 0
    assert linrec.delta_bwd_seq_workspace_bytes(seq, [8192, 0]) == 0

    beta = linrec.Tensor(FAKE, 16 * 8192, 8192, 1)

    def fcall(lengths, desc=seq, beta=beta, ws=FAKE, saved=None):
        arr = (ctypes.c_int32 * max(len(lengths), 1))(*lengths)
        return lib.linrec_delta_fwd_seq(None, ctypes.byref(desc), len(lengths), arr, act(), act(),
                                        act(), beta, linrec.Tensor(FAKE, 0, 1, 0), None, act(), FAKE,
                                        saved, ws, None)

    def bcall(lengths, desc=seq, dbeta=beta, saved=FAKE):
        arr = (ctypes.c_int32 * max(len(lengths), 1))(*lengths)
        return lib.linrec_delta_bwd_seq(None, ctypes.byref(desc), len(lengths), arr, act(), act(),
                                        act(), beta, linrec.Tensor(FAKE, 0, 1, 0), saved, act(), None,
                                        act(), act(), act(), dbeta, FAKE, FAKE, None)
    for call in (fcall, bcall):
        assert call(lens) == E["LINREC_E_NULL"]                  # checks pass, no context
        assert call([8192]) == E["LINREC_E_NULL"]
        assert call([4096, 4000]) == E["LINREC_E_SHAPE"]
        assert call([8192, 0]) == E["LINREC_E_SHAPE"]
        assert call([]) == E["LINREC_E_SHAPE"]
        assert call(lens, desc=d(T=8192, dk=64)) == E["LINREC_E_SHAPE"]
    assert fcall(lens, beta=linrec.Tensor(None, 0, 0, 1)) == E["LINREC_E_NULL"]
    assert fcall(lens, ws=None) == E["LINREC_E_WORKSPACE"]
    assert fcall(lens, saved=FAKE + 8) == E["LINREC_E_WORKSPACE"]
    assert bcall(lens, dbeta=linrec.Tensor(FAKE + 2, 0, 0, 1)) == E["LINREC_E_ALIGN"]
    assert bcall(lens, saved=None) == E["LINREC_E_WORKSPACE"]


def test_empty_piece_arguments():
    """T = 0: only the carried state and gradient pointers are checked;
    activations, decay, beta, states, saved and workspace may all be NULL.
    The sequence calls still want every piece to hold a token."""
    lib = linrec._lib()
    e = d(T=0, decay=linrec.DECAY_TOKEN)
    none = linrec.Tensor(None, 0, 0, 0)
    assert lib.linrec_fwd(None, ctypes.byref(e), none, none, none, none, None, none, FAKE, None,
                          None) == E["LINREC_E_NULL"]
    assert lib.linrec_fwd(None, ctypes.byref(e), none, none, none, none, FAKE + 2, none, FAKE,
                          None, None) == E["LINREC_E_ALIGN"]      # S_in still checked
    assert lib.linrec_bwd(None, ctypes.byref(e), none, none, none, none, None, none, FAKE + 2,
                          none, none, none, FAKE, None, None) == E["LINREC_E_ALIGN"]
    assert lib.linrec_bwd(None, ctypes.byref(e), none, none, none, none, None, none, None,
                          none, none, none, FAKE, None, None) == E["LINREC_E_NULL"]
    assert lib.linrec_bwd_noalloc(None, ctypes.byref(e), none, none, none, none, None, none,
                                  FAKE + 2, none, none, none, FAKE, None) == E["LINREC_E_ALIGN"]
    assert lib.linrec_bwd_recompute(None, ctypes.byref(e), none, none, none, none, FAKE + 2, none,
                                    None, none, none, none, FAKE, None, None) == E["LINREC_E_ALIGN"]
    assert lib.linrec_bwd_da(None, ctypes.byref(e), none, none, none, none, None, none, None,
                             none, none, none, FAKE, none, None, FAKE, None,
                             None) == E["LINREC_E_NULL"]
    assert lib.linrec_bwd_da(None, ctypes.byref(e), none, none, none, none, None, none, None,
                             none, none, none, FAKE, none, FAKE + 2, FAKE, None,
                             None) == E["LINREC_E_ALIGN"]          # the carry still checked
    assert lib.linrec_bwd_da(None, ctypes.byref(d(T=0, decay=linrec.DECAY_NONE)), none, none, none,
                             none, None, none, None, none, none, none, FAKE, none, None, FAKE,
                             None, None) == E["LINREC_E_LAYOUT"]   # no decay, no gradient
    assert lib.linrec_delta_fwd(None, ctypes.byref(e), none, none, none, none, none, FAKE + 2, none,
                                FAKE, None, None, None) == E["LINREC_E_ALIGN"]
    assert lib.linrec_delta_bwd(None, ctypes.byref(e), none, none, none, none, none, None, none,
                                FAKE + 2, none, none, none, none, FAKE, None,
                                None) == E["LINREC_E_ALIGN"]
    assert linrec.delta_workspace_bytes(e) == 0 and linrec.delta_saved_bytes(e) == 0
    arr = (ctypes.c_int32 * 1)(0)
    assert lib.linrec_fwd_seq(None, ctypes.byref(e), 1, arr, none, none, none, none, None, none,
                              FAKE, None, None) == E["LINREC_E_SHAPE"]
    assert lib.linrec_bwd_seq(None, ctypes.byref(e), 1, arr, none, none, none, none, None, none,
                              None, none, none, none, FAKE, None, None) == E["LINREC_E_SHAPE"]
