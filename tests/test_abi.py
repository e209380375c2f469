"""The C-ABI library loads without a GPU, exports every symbol kda.h declares,
and rejects every invalid argument before any HIP call (so these run on the
CPU with fake, never-dereferenced device addresses)."""
import ctypes
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kda.h")
# a host-only build of the argument checks may stand in (tests/test_sanitize.py)
STAND_IN = os.environ.get("KDA_ABI_TEST_LIBRARY")
LIB = STAND_IN or os.path.join(ROOT, "gated_delta_rule_38_amd", "libkda.so")

SUCCESS, INVALID, NOT_SUPPORTED, MISALIGNED, WORKSPACE, HIP = range(6)


@pytest.fixture(scope="module")
def lib():
    import gated_delta_rule_38_amd as kda
    if STAND_IN:
        return kda._bind_signatures(ctypes.CDLL(STAND_IN))
    if not os.path.exists(LIB):
        import __graft_entry__
        __graft_entry__.build()
    return kda.load_library()


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(kda_\w+)\s*\(", text, re.M)))


def test_header_declares_the_entry_points():
    names = declared_functions()
    for n in ["kda_chunk_fwd", "kda_chunk_fwd_gated", "kda_chunk_fwd_fused", "kda_recurrent_step",
              "kda_recurrent_step_gated", "kda_recurrent_step_fused", "kda_backward",
              "kda_backward_workspace_size", "kda_chunk_fwd_workspace_size", "kda_status_string",
              "kda_version"]:
        assert n in names, names


def test_library_exports_every_declared_symbol(lib):
    out = subprocess.run(["nm", "-D", "--defined-only", LIB], capture_output=True, text=True,
                         check=True).stdout
    exported = set(re.findall(r" T (\w+)$", out, re.M))
    for n in declared_functions():
        assert n in exported, n
        assert getattr(lib, n) is not None


def test_status_strings_cover_every_code(lib):
    names = [lib.kda_status_string(i).decode() for i in range(6)]
    assert names == ["KDA_SUCCESS", "KDA_ERROR_INVALID_VALUE", "KDA_ERROR_NOT_SUPPORTED",
                     "KDA_ERROR_MISALIGNED", "KDA_ERROR_INSUFFICIENT_WORKSPACE", "KDA_ERROR_HIP"]
    assert lib.kda_status_string(99).decode() == "unknown status"
    assert lib.kda_version() >= 100


# fake device addresses, far apart and 256-byte aligned; never dereferenced
BASE = 0x7F0000000000
GAP = 1 << 36


def fake(i, off=0):
    return ctypes.c_void_p(BASE + i * GAP + off)


def chunk_call(lib, **kw):
    a = dict(q=fake(0), k=fake(1), v=fake(2), alpha=fake(3), beta=fake(4), s0=fake(5), o=fake(6),
             sT=fake(7), B=2, T=100, H=4, dk=128, dv=128, dt=1, cu_dev=None, cu_host=None,
             num_seqs=0, scale=0.0, chunk=64, ws=None, ws_bytes=0, stream=None)
    a.update(kw)
    return lib.kda_chunk_fwd(a["q"], a["k"], a["v"], a["alpha"], a["beta"], a["s0"], a["o"],
                             a["sT"], a["B"], a["T"], a["H"], a["dk"], a["dv"], a["dt"],
                             a["cu_dev"], a["cu_host"], a["num_seqs"], a["scale"], a["chunk"],
                             a["ws"], a["ws_bytes"], a["stream"])


GATE_CHANNEL, GATE_HEAD, GATE_NONE = range(3)


def chunk_gated_call(lib, gate, **kw):
    a = dict(q=fake(0), k=fake(1), v=fake(2), alpha=fake(3), beta=fake(4), s0=fake(5), o=fake(6),
             sT=fake(7), B=2, T=100, H=4, dk=128, dv=128, dt=1, cu_dev=None, cu_host=None,
             num_seqs=0, scale=0.0, chunk=64, ws=None, ws_bytes=0, stream=None)
    a.update(kw)
    return lib.kda_chunk_fwd_gated(a["q"], a["k"], a["v"], a["alpha"], a["beta"], a["s0"],
                                   a["o"], a["sT"], a["B"], a["T"], a["H"], a["dk"], a["dv"],
                                   a["dt"], gate, a["cu_dev"], a["cu_host"], a["num_seqs"],
                                   a["scale"], a["chunk"], a["ws"], a["ws_bytes"], a["stream"])


def step_call(lib, **kw):
    a = dict(q=fake(0), k=fake(1), v=fake(2), alpha=fake(3), beta=fake(4), state=fake(5),
             o=fake(6), N=8, H=4, dk=128, dv=128, dt=1, scale=0.0, stream=None)
    a.update(kw)
    return lib.kda_recurrent_step(a["q"], a["k"], a["v"], a["alpha"], a["beta"], a["state"],
                                  a["o"], a["N"], a["H"], a["dk"], a["dv"], a["dt"], a["scale"],
                                  a["stream"])


def host_cu(vals):
    return (ctypes.c_int * len(vals))(*vals)


@pytest.mark.parametrize("kw,code", [
    (dict(dt=7), INVALID),
    (dict(B=-1), INVALID),
    (dict(T=-3), INVALID),
    (dict(H=-1), INVALID),
    (dict(dk=96), NOT_SUPPORTED),
    (dict(dv=256), NOT_SUPPORTED),
    (dict(chunk=128), NOT_SUPPORTED),
    (dict(q=None), INVALID),
    (dict(alpha=None), INVALID),
    (dict(o=None), INVALID),
    (dict(k=fake(1, 4)), MISALIGNED),
    (dict(alpha=fake(3, 4)), MISALIGNED),
    (dict(v=fake(2, 1)), MISALIGNED),
    (dict(beta=fake(4, 2)), MISALIGNED),
    (dict(sT=fake(7, 2)), MISALIGNED),
    (dict(o=fake(0, 64)), INVALID),          # output inside q
    (dict(sT=fake(3, 256)), INVALID),        # final state inside alpha
    (dict(sT=fake(6, 512)), INVALID),        # final state inside o
    (dict(sT=fake(5, 256)), INVALID),        # partial overlap with the initial state
    (dict(cu_dev=fake(8)), INVALID),         # cu_seqlens without num_seqs
])
def test_chunk_rejects_before_any_hip_call(lib, kw, code):
    assert chunk_call(lib, **kw) == code


def test_chunk_varlen_validation(lib):
    cu = host_cu([0, 10, 10, 40])
    good = dict(B=1, T=40, num_seqs=3, cu_dev=fake(8), cu_host=cu, ws=fake(9), ws_bytes=256)
    ws = lib.kda_chunk_fwd_workspace_size(1, 40, 4, 128, 128, 3, 1)
    assert ws == 256
    assert chunk_call(lib, **dict(good, ws=None, ws_bytes=0)) == WORKSPACE
    assert chunk_call(lib, **dict(good, ws_bytes=128)) == WORKSPACE
    assert chunk_call(lib, **dict(good, B=2)) == INVALID
    assert chunk_call(lib, **dict(good, T=41)) == INVALID
    assert chunk_call(lib, **dict(good, cu_host=host_cu([0, 10, 5, 40]))) == INVALID
    assert chunk_call(lib, **dict(good, cu_host=host_cu([1, 10, 10, 40]))) == INVALID
    assert chunk_call(lib, **dict(good, cu_host=None)) == INVALID
    assert chunk_call(lib, **dict(good, cu_dev=None)) == INVALID
    assert chunk_call(lib, **dict(good, cu_dev=fake(8, 2))) == MISALIGNED
    assert chunk_call(lib, **dict(good, ws=fake(0, 256))) == INVALID  # workspace inside q
    assert chunk_call(lib, **dict(good, ws=fake(9, 2))) == MISALIGNED


def test_noalloc_validation(lib):
    """kda_chunk_fwd_noalloc validates like kda_chunk_fwd (no workspace) and
    rejects more packed sequences than its fixed scratch holds."""
    a = dict(q=fake(0), k=fake(1), v=fake(2), alpha=fake(3), beta=fake(4), s0=fake(5), o=fake(6),
             sT=fake(7), B=2, T=100, H=4, dk=128, dv=128, dt=1, cu_dev=None, cu_host=None,
             num_seqs=0, scale=0.0, chunk=64, stream=None)

    def call(**kw):
        x = dict(a, **kw)
        return lib.kda_chunk_fwd_noalloc(x["q"], x["k"], x["v"], x["alpha"], x["beta"], x["s0"],
                                         x["o"], x["sT"], x["B"], x["T"], x["H"], x["dk"],
                                         x["dv"], x["dt"], x["cu_dev"], x["cu_host"],
                                         x["num_seqs"], x["scale"], x["chunk"], x["stream"])
    n = 65537
    assert call(B=1, T=0, num_seqs=n, cu_dev=fake(8), cu_host=host_cu([0] * (n + 1))) == \
        NOT_SUPPORTED
    assert call(dk=96) == NOT_SUPPORTED
    assert call(q=None) == INVALID
    assert call(o=fake(0, 64)) == INVALID
    assert call(k=fake(1, 4)) == MISALIGNED
    cu = host_cu([0, 10, 5, 40])
    assert call(B=1, T=40, num_seqs=3, cu_dev=fake(8), cu_host=cu) == INVALID
    assert call(B=0) == SUCCESS


def test_workspace_size(lib):
    assert lib.kda_chunk_fwd_workspace_size(2, 100, 4, 128, 128, 0, 1) == 0
    assert lib.kda_chunk_fwd_workspace_size(1, 100, 4, 128, 128, 64, 1) == 256
    assert lib.kda_chunk_fwd_workspace_size(1, 100, 4, 128, 128, 65, 1) == 512
    assert lib.kda_chunk_fwd_workspace_size(1, 100, 4, 96, 128, 65, 1) == 0


def test_chunk_empty_is_a_noop(lib):
    # no units: returns before any HIP call
    assert chunk_call(lib, B=0) == SUCCESS
    assert chunk_call(lib, H=0) == SUCCESS


@pytest.mark.parametrize("kw,code", [
    (dict(dt=3), INVALID),
    (dict(N=-1), INVALID),
    (dict(dk=32), NOT_SUPPORTED),
    (dict(dv=100), NOT_SUPPORTED),
    (dict(state=None), INVALID),
    (dict(o=None), INVALID),
    (dict(q=fake(0, 1)), MISALIGNED),
    (dict(alpha=fake(3, 2)), MISALIGNED),
    (dict(state=fake(5, 8)), MISALIGNED),
    (dict(o=fake(5, 1024)), INVALID),        # output inside the state
    (dict(state=fake(3, 0)), INVALID),       # state aliasing alpha
])
def test_step_rejects_before_any_hip_call(lib, kw, code):
    assert step_call(lib, **kw) == code


def test_step_empty_is_a_noop(lib):
    assert step_call(lib, N=0) == SUCCESS


def step_gated_call(lib, gate, **kw):
    a = dict(q=fake(0), k=fake(1), v=fake(2), alpha=fake(3), beta=fake(4), state=fake(5),
             o=fake(6), N=8, H=4, dk=128, dv=128, dt=1, scale=0.0, stream=None)
    a.update(kw)
    return lib.kda_recurrent_step_gated(a["q"], a["k"], a["v"], a["alpha"], a["beta"],
                                        a["state"], a["o"], a["N"], a["H"], a["dk"], a["dv"],
                                        a["dt"], gate, a["scale"], a["stream"])


@pytest.mark.parametrize("gate,kw,code", [
    (3, {}, INVALID),                                   # not a gate
    (-1, {}, INVALID),
    (GATE_NONE, {}, INVALID),                           # alpha given without a gate
    (GATE_HEAD, dict(alpha=None), INVALID),             # gate without alpha
    (GATE_CHANNEL, dict(alpha=None), INVALID),
    (GATE_HEAD, dict(alpha=fake(3, 2)), MISALIGNED),    # per-head alpha: 4-byte words
    (GATE_CHANNEL, dict(alpha=fake(3, 4)), MISALIGNED),  # per-channel alpha: pairs
    # a 4-byte aligned per-head alpha passes the alignment checks and the call
    # then fails on the overlap below it
    (GATE_HEAD, dict(alpha=fake(3, 4), sT=fake(6, 512)), INVALID),
    (GATE_HEAD, dict(sT=fake(3, 256)), INVALID),        # final state inside alpha
    (GATE_NONE, dict(alpha=None, dk=96), NOT_SUPPORTED),
    (GATE_NONE, dict(alpha=None, o=None), INVALID),
])
def test_chunk_gated_rejects_before_any_hip_call(lib, gate, kw, code):
    assert chunk_gated_call(lib, gate, **kw) == code


def test_gated_empty_is_a_noop(lib):
    for gate in (GATE_CHANNEL, GATE_HEAD):
        assert chunk_gated_call(lib, gate, B=0) == SUCCESS
        assert step_gated_call(lib, gate, N=0) == SUCCESS
    assert chunk_gated_call(lib, GATE_NONE, alpha=None, H=0) == SUCCESS
    assert step_gated_call(lib, GATE_NONE, alpha=None, N=0) == SUCCESS


@pytest.mark.parametrize("gate,kw,code", [
    (3, {}, INVALID),
    (GATE_NONE, {}, INVALID),
    (GATE_HEAD, dict(alpha=None), INVALID),
    (GATE_HEAD, dict(alpha=fake(3, 2)), MISALIGNED),
    (GATE_HEAD, dict(state=fake(3, 0)), INVALID),       # state aliasing alpha
    (GATE_NONE, dict(alpha=None, state=fake(5, 8)), MISALIGNED),
])
def test_step_gated_rejects_before_any_hip_call(lib, gate, kw, code):
    assert step_gated_call(lib, gate, **kw) == code


GL, BL, QN = 1, 2, 4


def chunk_fused_call(lib, gate, flags, **kw):
    a = dict(q=fake(0), k=fake(1), v=fake(2), alpha=fake(3), beta=fake(4), s0=fake(5), o=fake(6),
             sT=fake(7), B=2, T=100, H=4, dk=128, dv=128, dt=1, cu_dev=None, cu_host=None,
             num_seqs=0, scale=0.0, chunk=64, ws=None, ws_bytes=0, stream=None)
    a.update(kw)
    return lib.kda_chunk_fwd_fused(a["q"], a["k"], a["v"], a["alpha"], a["beta"], a["s0"],
                                   a["o"], a["sT"], a["B"], a["T"], a["H"], a["dk"], a["dv"],
                                   a["dt"], gate, flags, a["cu_dev"], a["cu_host"],
                                   a["num_seqs"], a["scale"], a["chunk"], a["ws"], a["ws_bytes"],
                                   a["stream"])


def step_fused_call(lib, gate, flags, **kw):
    a = dict(q=fake(0), k=fake(1), v=fake(2), alpha=fake(3), beta=fake(4), state=fake(5),
             o=fake(6), N=8, H=4, dk=128, dv=128, dt=1, scale=0.0, stream=None)
    a.update(kw)
    return lib.kda_recurrent_step_fused(a["q"], a["k"], a["v"], a["alpha"], a["beta"],
                                        a["state"], a["o"], a["N"], a["H"], a["dk"], a["dv"],
                                        a["dt"], gate, flags, a["scale"], a["stream"])


@pytest.mark.parametrize("gate,flags,kw,code", [
    (GATE_CHANNEL, 8, {}, INVALID),                                  # unknown flag bit
    (GATE_CHANNEL, 0x80000000, {}, INVALID),
    (GATE_NONE, GL, dict(alpha=None), INVALID),                      # logits without a gate
    (GATE_HEAD, GL | QN, dict(alpha=None), INVALID),
    (GATE_CHANNEL, GL, dict(alpha=fake(3, 4)), MISALIGNED),          # per-channel: 8 bytes
    (GATE_HEAD, GL, dict(alpha=fake(3, 1)), MISALIGNED),             # bf16 per head: 2 bytes
    (GATE_HEAD, 0, dict(alpha=fake(3, 2)), MISALIGNED),              # float32 per head: 4 bytes
    # a 2-byte aligned bf16 per-head logit passes and the call fails on the overlap
    (GATE_HEAD, GL, dict(alpha=fake(3, 2), sT=fake(6, 512)), INVALID),
    # bf16 per-channel logits span B*T*H*dk*2 bytes: a final state 4 KB past
    # their start overlaps them
    (GATE_CHANNEL, GL | BL | QN, dict(sT=fake(3, 4096)), INVALID),
    (GATE_CHANNEL, GL | BL | QN, dict(dk=96), NOT_SUPPORTED),
    (GATE_NONE, QN | BL, dict(alpha=None, o=None), INVALID),
])
def test_chunk_fused_rejects_before_any_hip_call(lib, gate, flags, kw, code):
    assert chunk_fused_call(lib, gate, flags, **kw) == code


def test_fused_empty_is_a_noop(lib):
    assert chunk_fused_call(lib, GATE_CHANNEL, GL | BL | QN, B=0) == SUCCESS
    assert step_fused_call(lib, GATE_HEAD, GL | BL | QN, N=0) == SUCCESS


@pytest.mark.parametrize("gate,flags,kw,code", [
    (GATE_CHANNEL, 16, {}, INVALID),
    (GATE_NONE, GL, dict(alpha=None), INVALID),
    (GATE_HEAD, GL, dict(alpha=fake(3, 1)), MISALIGNED),
    (GATE_CHANNEL, GL | QN, dict(state=fake(3, 0)), INVALID),        # state aliasing the logits
])
def test_step_fused_rejects_before_any_hip_call(lib, gate, flags, kw, code):
    assert step_fused_call(lib, gate, flags, **kw) == code


def bwd_call(lib, **kw):
    B, T, H, dk, dv = kw.get("B", 2), kw.get("T", 100), kw.get("H", 4), 128, 128
    ws_need = lib.kda_backward_workspace_size(B, T, H, dk, dv, 0, 1)
    a = dict(q=fake(0), k=fake(1), v=fake(2), alpha=fake(3), beta=fake(4), s0=fake(5), do=fake(6),
             dsT=fake(7), dq=fake(8), dk=fake(9), dv=fake(10), da=fake(11), db=fake(12),
             ds0=fake(13), B=B, T=T, H=H, dkd=dk, dvd=dv, dt=1, cu_dev=None, cu_host=None,
             num_seqs=0, scale=0.0, ws=fake(14), ws_bytes=ws_need, stream=None)
    a.update(kw)
    return lib.kda_backward(a["q"], a["k"], a["v"], a["alpha"], a["beta"], a["s0"], a["do"],
                            a["dsT"], a["dq"], a["dk"], a["dv"], a["da"], a["db"], a["ds0"],
                            a["B"], a["T"], a["H"], a["dkd"], a["dvd"], a["dt"], a["cu_dev"],
                            a["cu_host"], a["num_seqs"], a["scale"], a["ws"], a["ws_bytes"],
                            a["stream"])


def test_backward_workspace_size(lib):
    B, T, H, d = 2, 100, 4, 128
    r = lambda x: (x + 255) // 256 * 256
    # bf16 (chunk form): the state at every chunk start and end, two spare slots per
    # sequence; then, for each value-column slice but the first (dv / 32 of them),
    # its partial dq, dk, dalpha (tokens * H * dk each) and dbeta (tokens * H,
    # padded to 64) in float32
    slots = (B * T) // 64 + 2 * B + 1
    nk, nb = B * T * H * d, (B * T * H + 63) // 64 * 64
    for dv in (64, 128):
        assert lib.kda_backward_workspace_size(B, T, H, d, dv, 0, 1) == (
            r(slots * H * d * dv * 4) + (dv // 32 - 1) * (3 * nk + nb) * 4)
    # float32 (token recurrence): checkpoints every 8 tokens (+ one slot per sequence and a spare)
    slots = (B * T + 7) // 8 + B + 1
    assert lib.kda_backward_workspace_size(B, T, H, d, d, 0, 0) == r(slots * H * d * d * 4)
    assert lib.kda_backward_workspace_size(B, T, H, 96, d, 0, 1) == 0
    assert lib.kda_backward_workspace_size(0, T, H, d, d, 0, 1) == 0


@pytest.mark.parametrize("kw,code", [
    (dict(dt=5), INVALID),
    (dict(T=-1), INVALID),
    (dict(dkd=32), NOT_SUPPORTED),
    (dict(q=None), INVALID),
    (dict(do=None), INVALID),
    (dict(ds0=None), INVALID),                 # the initial-state gradient is always written
    (dict(s0=fake(5, 8)), MISALIGNED),         # states: 16 bytes
    (dict(ds0=fake(13, 4)), MISALIGNED),
    (dict(ws=fake(14, 16)), MISALIGNED),       # workspace: 256 bytes
    (dict(ws=None, ws_bytes=0), WORKSPACE),
    (dict(ws_bytes=1024), WORKSPACE),
    (dict(dq=fake(0, 256)), INVALID),          # gradient inside q
    (dict(dk=fake(8, 1024)), INVALID),         # two gradients overlapping
    (dict(ws=fake(12, 256)), INVALID),         # workspace inside dbeta
    (dict(cu_dev=fake(15)), INVALID),          # cu_seqlens without num_seqs
    (dict(v=fake(2, 2)), MISALIGNED),          # v and dout: runs of four elements
    (dict(do=fake(6, 4)), MISALIGNED),
    (dict(dt=0, v=fake(2, 8)), MISALIGNED),    # 16 bytes for float32
    (dict(q=fake(0, 4)), MISALIGNED),          # bf16: q, k and alpha in pairs (8 bytes)
    (dict(alpha=fake(3, 4)), MISALIGNED),
])
def test_backward_rejects_before_any_hip_call(lib, kw, code):
    assert bwd_call(lib, **kw) == code


def test_python_binding_checks_arguments():
    import torch
    import gated_delta_rule_38_amd as kda
    q = torch.zeros(1, 4, 1, 64)
    with pytest.raises(TypeError):
        kda.kda_chunk_fwd(q.to(torch.float16), q, q, q, q[..., 0])
    with pytest.raises(ValueError):
        kda.kda_chunk_fwd(q, q[:, :2], q, q, q[..., 0])
    b = q[..., 0].contiguous()
    with pytest.raises(ValueError):  # a per-head alpha has no channel axis
        kda.kda_chunk_fwd_gated(q, q, q, q, b, gate="head")
    with pytest.raises(ValueError):  # no alpha without a gate
        kda.kda_chunk_fwd_gated(q, q, q, b, b, gate="none")
    with pytest.raises(ValueError):
        kda.kda_chunk_fwd_gated(q, q, q, b, b, gate="scalar")
    s = torch.zeros(1, 1, 64, 64)
    with pytest.raises(ValueError):
        kda.kda_recurrent_step_gated(q[0], q[0], q[0], q[0], b[0], s, gate="head")
    with pytest.raises(TypeError):  # gate logits come in the dtype of q (bf16 here)
        qb = q.to(torch.bfloat16)
        kda.kda_chunk_fwd_fused(qb, qb, qb, q, b)


# ------------------------------------------------------- Gated DeltaNet-2

def gdn2_chunk_call(lib, **kw):
    a = dict(q=fake(0), k=fake(1), v=fake(2), alpha=fake(3), erase=fake(4), write=fake(9),
             s0=fake(5), o=fake(6), sT=fake(7), B=2, T=100, H=4, dk=128, dv=128, dt=1,
             cu_dev=None, cu_host=None, num_seqs=0, scale=0.0, chunk=64, ws=None, ws_bytes=0,
             stream=None)
    a.update(kw)
    return lib.kda_gdn2_chunk_fwd(a["q"], a["k"], a["v"], a["alpha"], a["erase"], a["write"],
                                  a["s0"], a["o"], a["sT"], a["B"], a["T"], a["H"], a["dk"],
                                  a["dv"], a["dt"], a["cu_dev"], a["cu_host"], a["num_seqs"],
                                  a["scale"], a["chunk"], a["ws"], a["ws_bytes"], a["stream"])


def gdn2_step_call(lib, **kw):
    a = dict(q=fake(0), k=fake(1), v=fake(2), alpha=fake(3), erase=fake(4), write=fake(9),
             state=fake(5), o=fake(6), N=8, H=4, dk=128, dv=128, dt=1, scale=0.0, stream=None)
    a.update(kw)
    return lib.kda_gdn2_recurrent_step(a["q"], a["k"], a["v"], a["alpha"], a["erase"],
                                       a["write"], a["state"], a["o"], a["N"], a["H"], a["dk"],
                                       a["dv"], a["dt"], a["scale"], a["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(dt=7), INVALID),
    (dict(B=-1), INVALID),
    (dict(dt=0), NOT_SUPPORTED),             # the chunk kernel takes bf16 q, k, v only
    (dict(dk=96), NOT_SUPPORTED),
    (dict(chunk=32), NOT_SUPPORTED),
    (dict(erase=None), INVALID),
    (dict(write=None), INVALID),
    (dict(o=None), INVALID),
    (dict(erase=fake(4, 4)), MISALIGNED),    # the gates are read in pairs of channels
    (dict(write=fake(9, 4)), MISALIGNED),
    (dict(alpha=fake(3, 4)), MISALIGNED),
    (dict(q=fake(0, 4)), MISALIGNED),
    (dict(o=fake(4, 64)), INVALID),          # output inside the erase gate
    (dict(sT=fake(9, 256)), INVALID),        # final state inside the write gate
    (dict(sT=fake(5, 256)), INVALID),        # partial overlap with the initial state
    (dict(cu_dev=fake(8)), INVALID),         # cu_seqlens without num_seqs
    (dict(B=1, T=10, num_seqs=2, cu_dev=fake(8), cu_host=host_cu([0, 4, 9])), INVALID),
    (dict(B=1, T=10, num_seqs=2, cu_dev=fake(8), cu_host=host_cu([0, 6, 5])), INVALID),
])
def test_gdn2_chunk_rejects_before_any_hip_call(lib, kw, code):
    assert gdn2_chunk_call(lib, **kw) == code


def test_gdn2_chunk_workspace_and_empty(lib):
    # packed sequences need the workspace of kda_chunk_fwd
    cu = host_cu([0, 4, 10])
    assert gdn2_chunk_call(lib, B=1, T=10, num_seqs=2, cu_dev=fake(8), cu_host=cu) == WORKSPACE
    # no forget gate is allowed; no units is a no-op
    assert gdn2_chunk_call(lib, alpha=None, H=0) == SUCCESS
    assert gdn2_chunk_call(lib, B=0) == SUCCESS


@pytest.mark.parametrize("kw,code", [
    (dict(dt=7), INVALID),
    (dict(N=-1), INVALID),
    (dict(dv=32), NOT_SUPPORTED),
    (dict(erase=None), INVALID),
    (dict(write=None), INVALID),
    (dict(state=None), INVALID),
    (dict(state=fake(5, 8)), MISALIGNED),    # the state is read as float4
    (dict(erase=fake(4, 2)), MISALIGNED),
    (dict(write=fake(9, 2)), MISALIGNED),
    (dict(dt=0, q=fake(0, 2)), MISALIGNED),  # float32 q: 4-byte elements
    (dict(o=fake(5, 1024)), INVALID),        # output inside the state
    (dict(state=fake(4, 0)), INVALID),       # state aliasing the erase gate
])
def test_gdn2_step_rejects_before_any_hip_call(lib, kw, code):
    assert gdn2_step_call(lib, **kw) == code


def test_gdn2_step_empty_is_a_noop(lib):
    assert gdn2_step_call(lib, N=0) == SUCCESS
    assert gdn2_step_call(lib, H=0, alpha=None) == SUCCESS


def test_chunk_split_workspace_is_range_checked(lib):
    """A dense call whose workspace holds the two-segment path's buffers takes
    that path, so the workspace must then not overlap an input or an output
    (every case here is refused before any HIP call)."""
    big = dict(B=1, T=65536, H=32, s0=None, sT=fake(7))
    n = lib.kda_chunk_fwd_split_workspace_size(1, 65536, 32, 128, 128, 1)
    assert n > 0
    assert chunk_call(lib, **big, ws=fake(0), ws_bytes=n) == INVALID            # inside q
    assert chunk_call(lib, **big, ws=fake(6, 1 << 20), ws_bytes=n) == INVALID  # inside o
    assert chunk_call(lib, **big, ws=fake(7), ws_bytes=n) == INVALID           # is the final state
