"""C-ABI checks that need no GPU: the library loads, exports every function
include/kda.h declares, sizes its workspace, and rejects every bad argument on
the host before making any HIP call (failure injection from the host)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kda.h")

kda = pytest.importorskip("gated_delta_rule_prep_amd.kda")


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(kda_[a-z_]+)\s*\(", src)))


def test_every_declared_symbol_is_exported():
    names = declared_functions()
    assert "kda_fwd" in names and len(names) >= 6
    for n in names:
        assert hasattr(kda.lib(), n), n
    assert set(names) == set(kda.EXPORTS)


def test_header_codes_match_binding():
    src = open(HEADER).read()
    for name, val in [("KDA_OK", 0), ("KDA_EINVAL", 1), ("KDA_EDTYPE", 2), ("KDA_EWORKSPACE", 3),
                      ("KDA_EUNSUPPORTED", 4), ("KDA_EHIP", 5), ("KDA_DTYPE_NONE", 0), ("KDA_DTYPE_BF16", 1),
                      ("KDA_DTYPE_FP32", 2), ("KDA_STATUS_BAD_CU_SEQLENS", 1), ("KDA_STATUS_OVERFLOW", 2), ("KDA_STATUS_SYNC_TIMEOUT", 4), ("KDA_CHUNK", 16),
                      ("KDA_PATH_AUTO", 0), ("KDA_PATH_SPLIT", 1), ("KDA_PATH_FUSED", 2)]:
        m = re.search(r"#define\s+%s\s+(\d+)" % name, src)
        assert m and int(m.group(1)) == val, name
        if hasattr(kda, name):
            assert getattr(kda, name) == val


def test_version():
    assert kda.version() >= 100


def test_workspace_sizes_and_layout():
    lay = kda.workspace_layout(1, 8192, 96)
    assert lay["max_chunks"] == 8192 // 16 + 1
    assert lay["rec_bytes"] == 13824
    assert lay["records"] % 256 == 0 and lay["total"] % 256 == 0
    assert lay["total"] >= lay["records"] + 96 * lay["max_chunks"] * lay["rec_bytes"]
    assert kda.workspace_bytes(1, 8192, 96) >= lay["total"]
    # varlen capacity: floor(T/16) + N chunks covers every split into N sequences
    lay2 = kda.workspace_layout(1, 8192, 96, 12, True)
    assert lay2["max_chunks"] == 512 + 12
    assert kda.workspace_bytes(1, 0, 4) > 0
    assert kda.workspace_bytes(1, 10, 4, 0, True) == 0      # no sequences with cu_seqlens
    assert kda.workspace_bytes(0, 10, 4) == 0


def test_chunk_capacity_bound_is_tight():
    """sum ceil(l_n / 16) <= floor(T / 16) + N for every split of T into N parts."""
    import itertools
    for T in range(0, 40):
        for N in range(1, 4):
            for cuts in itertools.combinations_with_replacement(range(T + 1), N - 1):
                b = [0, *cuts, T]
                lens = [b[i + 1] - b[i] for i in range(N)]
                assert sum((l + 15) // 16 for l in lens) <= T // 16 + N


FAKE = ctypes.c_void_p(0x1000)        # never dereferenced: validation fails first
WS = ctypes.c_void_p(0x100000)        # 256-byte aligned fake workspace


def call(**over):
    a = dict(q=FAKE, k=FAKE, v=FAKE, g=FAKE, beta=FAKE, scale=0.088, out=FAKE, A_log=FAKE, dt_bias=FAKE,
             lb=-5.0, s0=None, s0_dt=0, s1=None, s1_dt=0, cu=None, N=0, B=1, T=64, H=2, K=128, V=128,
             ws=WS, ws_bytes=1 << 40, stream=None)
    a.update(over)
    return kda.lib().kda_fwd(a["q"], a["k"], a["v"], a["g"], a["beta"], a["scale"], a["out"], a["A_log"],
                             a["dt_bias"], a["lb"], a["s0"], a["s0_dt"], a["s1"], a["s1_dt"], a["cu"], a["N"],
                             a["B"], a["T"], a["H"], a["K"], a["V"], a["ws"], a["ws_bytes"], a["stream"])


@pytest.mark.parametrize("over,code", [
    (dict(q=None), kda.KDA_EINVAL),
    (dict(k=None), kda.KDA_EINVAL),
    (dict(v=None), kda.KDA_EINVAL),
    (dict(g=None), kda.KDA_EINVAL),
    (dict(beta=None), kda.KDA_EINVAL),
    (dict(out=None), kda.KDA_EINVAL),
    (dict(A_log=None), kda.KDA_EINVAL),
    (dict(dt_bias=None), kda.KDA_EINVAL),
    (dict(ws=None), kda.KDA_EINVAL),
    (dict(ws=ctypes.c_void_p(0x100010)), kda.KDA_EINVAL),     # misaligned workspace
    (dict(q=ctypes.c_void_p(0x1002)), kda.KDA_EINVAL),        # misaligned tensor
    (dict(out=ctypes.c_void_p(0x1008)), kda.KDA_EINVAL),
    (dict(dt_bias=ctypes.c_void_p(0x1004)), kda.KDA_EINVAL),  # dt_bias is read in 16-byte vectors
    (dict(K=64), kda.KDA_EINVAL),
    (dict(V=256), kda.KDA_EINVAL),
    (dict(B=0), kda.KDA_EINVAL),
    (dict(T=-1), kda.KDA_EINVAL),
    (dict(H=0), kda.KDA_EINVAL),
    (dict(H=70000), kda.KDA_EINVAL),
    (dict(cu=FAKE, N=2, B=2), kda.KDA_EINVAL),                # B != 1 with cu_seqlens
    (dict(cu=FAKE, N=0), kda.KDA_EINVAL),
    (dict(lb=-5.5), kda.KDA_EINVAL),
    (dict(lb=0.25), kda.KDA_EINVAL),
    (dict(lb=float("nan")), kda.KDA_EINVAL),
    (dict(scale=float("inf")), kda.KDA_EINVAL),
    (dict(B=1 << 20, T=1 << 12), kda.KDA_EINVAL),            # token rows overflow int32
    (dict(s0=FAKE, s0_dt=3), kda.KDA_EDTYPE),
    (dict(s0=FAKE, s0_dt=0), kda.KDA_EDTYPE),                 # pointer without dtype
    (dict(s0=None, s0_dt=1), kda.KDA_EDTYPE),                 # dtype without pointer
    (dict(s0=FAKE, s0_dt=1, s1=FAKE, s1_dt=2), kda.KDA_EDTYPE),  # dtypes differ
    (dict(ws_bytes=700), kda.KDA_EWORKSPACE),
])
def test_host_validation_rejects(over, code):
    rc = call(**over)
    assert rc == code, (rc, kda.last_error())
    assert kda.last_error()


def test_debug_prep_validation():
    rc = kda.lib().kda_debug_prep(FAKE, FAKE, FAKE, FAKE, 0.1, FAKE, FAKE, -6.0, None, 0, 1, 64, 2, 128, WS,
                                  1 << 40, None, 16)
    assert rc == kda.KDA_EINVAL
    rc = kda.lib().kda_debug_prep(FAKE, FAKE, FAKE, FAKE, 0.1, FAKE, FAKE, -5.0, None, 0, 1, 64, 2, 128, WS,
                                  1 << 40, None, 24)
    assert rc == kda.KDA_EINVAL and "chunk" in kda.last_error()


def test_python_binding_rejects_bad_tensors():
    import torch
    q = torch.zeros(1, 4, 2, 128, dtype=torch.bfloat16)
    v = torch.zeros(1, 4, 2, 128, dtype=torch.bfloat16)
    b = torch.zeros(1, 4, 2, dtype=torch.bfloat16)
    A = torch.zeros(2)
    dt = torch.zeros(2, 128)
    with pytest.raises(ValueError):
        kda.fwd(q.float(), q, v, q, b, 0.1, v.clone(), A, dt, -5.0)        # q not bf16
    with pytest.raises(ValueError):
        kda.fwd(q, q, v, q, b, 0.1, v.clone(), A, dt[:, :64].contiguous(), -5.0)
    with pytest.raises(ValueError):
        kda.fwd(q, q, v, q, b, 0.1, v.clone(), A, dt, -5.0,
                initial_state=torch.zeros(1, 2, 128, 128, dtype=torch.float16))
    with pytest.raises(ValueError):                                          # CPU tensors
        kda.fwd(q, q, v, q, b, 0.1, v.clone(), A, dt, -5.0)


def call_ex(parts, events, n_events, chunk=0, path=0, **over):
    a = dict(q=FAKE, k=FAKE, v=FAKE, g=FAKE, beta=FAKE, scale=0.088, out=FAKE, A_log=FAKE, dt_bias=FAKE,
             lb=-5.0, s0=None, s0_dt=0, s1=None, s1_dt=0, cu=None, N=0, B=1, T=64, H=2, K=128, V=128,
             ws=WS, ws_bytes=1 << 40, stream=None)
    a.update(over)
    return kda.lib().kda_fwd_ex(a["q"], a["k"], a["v"], a["g"], a["beta"], a["scale"], a["out"], a["A_log"],
                                a["dt_bias"], a["lb"], a["s0"], a["s0_dt"], a["s1"], a["s1_dt"], a["cu"],
                                a["N"], a["B"], a["T"], a["H"], a["K"], a["V"], a["ws"], a["ws_bytes"],
                                a["stream"], chunk, parts, path, events, n_events)


def test_parts_choice():
    assert kda.parts(1, 0) == 1 and kda.parts(1, 0, 5) == 1      # nothing to overlap
    assert kda.parts(1, 8192) == 1 and kda.parts(4, 8192) == 1    # the library's own choice
    assert kda.parts(1, 64, 3) == 3 and kda.parts(1, 64, 100) == 8
    assert kda.lib().kda_fwd_parts(1, 64, -1) == 0 and kda.lib().kda_fwd_parts(-1, 64, 0) == 0


def test_fwd_ex_rejects_bad_parts_and_event_counts():
    assert call_ex(-1, None, 0) == kda.KDA_EINVAL
    ev = (ctypes.c_void_p * 10)(*([FAKE.value] * 10))
    # parts = 2 needs 2 + 4 * 2 = 10 events; 9 or 14 are rejected before any HIP call
    assert call_ex(2, ev, 9) == kda.KDA_EINVAL and "events" in kda.last_error()
    assert call_ex(3, ev, 10) == kda.KDA_EINVAL
    null_ev = (ctypes.c_void_p * 10)()
    assert call_ex(2, null_ev, 10) == kda.KDA_EINVAL and "NULL" in kda.last_error()
    assert call_ex(2, None, 0, q=None) == kda.KDA_EINVAL
    for bad in (8, 17, 48, 128, -16):
        assert call_ex(1, None, 0, chunk=bad) == kda.KDA_EINVAL and "chunk" in kda.last_error()


def test_path_choice_events_and_workspace():
    """Which path a kda_fwd_ex request takes, how many events it records and
    how much workspace it needs, and the requests it rejects on the host."""
    assert kda.path_used() == "auto"                # both enqueued, the scheduler kernel picks
    assert kda.path_used(chunk=16) == "auto" and kda.path_used(parts=1) == "auto"
    assert kda.path_used(chunk=32) == "split" and kda.path_used(parts=2) == "split"
    assert kda.path_used(chunk=64) == "split"
    assert kda.path_used(path="split") == "split" and kda.path_used(path="fused", chunk=16) == "fused"
    assert kda.path_used(path="fused", parts=1) == "fused"
    for bad in (dict(path="fused", chunk=32), dict(path="fused", chunk=64), dict(path="fused", parts=3),
                dict(path=7), dict(chunk=24), dict(chunk=128)):
        with pytest.raises(ValueError):
            kda.path_used(**bad)
    assert kda.num_events(1, 8192, path="fused") == 4 and kda.num_events(1, 8192, path="split") == 6
    assert kda.num_events(1, 8192) == 8                  # scheduler, prep, recurrence, fused
    assert kda.num_events(1, 8192, parts=3) == 2 + 4 * 3
    assert kda.lib().kda_fwd_num_events(1, 64, 32, 0, 2) == 0         # fused cannot take 32-token chunks
    # the fused path keeps only the per-sequence tables; the split path its records
    fused = kda.workspace_bytes(1, 8192, 96, path="fused")
    split = kda.workspace_bytes(1, 8192, 96, path="split")
    assert 0 < fused <= 4096 and fused % 256 == 0
    assert split == kda.workspace_layout(1, 8192, 96, chunk=16)["total"]
    assert kda.workspace_bytes(1, 8192, 96, chunk=32) == kda.workspace_layout(1, 8192, 96, chunk=32)["total"]
    assert kda.workspace_bytes(1, 8192, 96, chunk=64) == kda.workspace_layout(1, 8192, 96, chunk=64)["total"]
    assert kda.workspace_bytes(1, 8192, 96) >= max(fused, split)
    assert kda.workspace_bytes(1, 8192, 96, path="auto") == split      # both paths enqueued
    assert kda.workspace_bytes(1, 8192, 96, 100000, True, path="fused") >= 100000 * 20
    assert kda.lib().kda_fwd_workspace_bytes_ex(1, 64, 2, 0, 0, 32, 0, 2) == 0
    # a fused call is rejected when its workspace is smaller than that, and the
    # fused path refuses what it cannot run; all on the host
    assert call_ex(0, None, 0, path=2, ws_bytes=fused - 1, T=8192, H=96) == kda.KDA_EWORKSPACE
    assert call_ex(0, None, 0, chunk=32, path=2) == kda.KDA_EINVAL and "fused" in kda.last_error()
    assert call_ex(2, None, 0, path=2) == kda.KDA_EINVAL
    assert call_ex(0, None, 0, path=3) == kda.KDA_EINVAL
    ev = (ctypes.c_void_p * 6)(*([FAKE.value] * 6))
    assert call_ex(0, ev, 6, path=2) == kda.KDA_EINVAL and "events" in kda.last_error()   # fused takes 4


def test_layout_for_every_chunk_size():
    l16 = kda.workspace_layout(1, 8192, 96, chunk=16)
    l32 = kda.workspace_layout(1, 8192, 96, chunk=32)
    l64 = kda.workspace_layout(1, 8192, 96, chunk=64)
    assert l32["max_chunks"] == 8192 // 32 + 1 and l32["rec_bytes"] == 29184
    assert l32["records"] % 256 == 0 and l32["total"] >= l32["records"] + 96 * l32["max_chunks"] * 29184
    assert l64["max_chunks"] == 8192 // 64 + 1 and l64["rec_bytes"] == 66048
    assert l64["records"] % 256 == 0 and l64["total"] >= l64["records"] + 96 * l64["max_chunks"] * 66048
    # the plain workspace query covers kda_fwd's 16- and 32-token forms; the
    # 64-token chunk (kda_fwd_ex only) takes kda_fwd_workspace_bytes_ex
    assert kda.workspace_bytes(1, 8192, 96) == max(l16["total"], l32["total"])
    with pytest.raises(ValueError):
        kda.workspace_layout(1, 64, 2, chunk=24)


def call_decode(**over):
    a = dict(q=FAKE, k=FAKE, v=FAKE, g=FAKE, beta=FAKE, scale=0.088, out=FAKE, A_log=FAKE, dt_bias=FAKE,
             lb=-5.0, s0=None, s0_dt=0, s1=None, s1_dt=0, N=4, H=2, K=128, V=128, stream=None)
    a.update(over)
    return kda.lib().kda_decode(a["q"], a["k"], a["v"], a["g"], a["beta"], a["scale"], a["out"], a["A_log"],
                                a["dt_bias"], a["lb"], a["s0"], a["s0_dt"], a["s1"], a["s1_dt"], a["N"], a["H"],
                                a["K"], a["V"], a["stream"])


@pytest.mark.parametrize("over,code", [
    (dict(q=None), kda.KDA_EINVAL),
    (dict(v=None), kda.KDA_EINVAL),
    (dict(out=None), kda.KDA_EINVAL),
    (dict(beta=None), kda.KDA_EINVAL),
    (dict(A_log=None), kda.KDA_EINVAL),
    (dict(dt_bias=ctypes.c_void_p(0x1004)), kda.KDA_EINVAL),   # misaligned
    (dict(k=ctypes.c_void_p(0x1008)), kda.KDA_EINVAL),
    (dict(K=64), kda.KDA_EINVAL),
    (dict(V=64), kda.KDA_EINVAL),
    (dict(N=-1), kda.KDA_EINVAL),
    (dict(H=0), kda.KDA_EINVAL),
    (dict(N=1 << 30, H=4), kda.KDA_EINVAL),
    (dict(lb=-6.0), kda.KDA_EINVAL),
    (dict(scale=float("nan")), kda.KDA_EINVAL),
    (dict(s0=FAKE, s0_dt=0), kda.KDA_EDTYPE),
    (dict(s1=None, s1_dt=2), kda.KDA_EDTYPE),
    (dict(s0=FAKE, s0_dt=2, s1=FAKE, s1_dt=1), kda.KDA_EDTYPE),
    (dict(s0=FAKE, s0_dt=7), kda.KDA_EDTYPE),
])
def test_decode_host_validation_rejects(over, code):
    rc = call_decode(**over)
    assert rc == code, (rc, kda.last_error())
    assert kda.last_error()


def call_seg(segments, **over):
    a = dict(q=FAKE, k=FAKE, v=FAKE, g=FAKE, beta=FAKE, scale=0.088, out=FAKE, A_log=FAKE, dt_bias=FAKE,
             lb=-5.0, s0=None, s0_dt=0, s1=None, s1_dt=0, cu=None, N=0, B=1, T=64, H=2, K=128, V=128,
             ws=WS, ws_bytes=1 << 40, stream=None)
    a.update(over)
    return kda.lib().kda_fwd_segmented(a["q"], a["k"], a["v"], a["g"], a["beta"], a["scale"], a["out"],
                                       a["A_log"], a["dt_bias"], a["lb"], a["s0"], a["s0_dt"], a["s1"], a["s1_dt"],
                                       a["cu"], a["N"], a["B"], a["T"], a["H"], a["K"], a["V"], segments, a["ws"],
                                       a["ws_bytes"], a["stream"])


@pytest.mark.parametrize("segments", [1, 4])
@pytest.mark.parametrize("over,code", [
    (dict(q=None), kda.KDA_EINVAL),
    (dict(v=None), kda.KDA_EINVAL),
    (dict(out=None), kda.KDA_EINVAL),
    (dict(dt_bias=None), kda.KDA_EINVAL),
    (dict(ws=None), kda.KDA_EINVAL),
    (dict(ws=ctypes.c_void_p(0x100010)), kda.KDA_EINVAL),
    (dict(v=ctypes.c_void_p(0x1004)), kda.KDA_EINVAL),
    (dict(K=64), kda.KDA_EINVAL),
    (dict(cu=FAKE, N=2, B=2), kda.KDA_EINVAL),
    (dict(lb=0.5), kda.KDA_EINVAL),
    (dict(s0=FAKE, s0_dt=1, s1=FAKE, s1_dt=2), kda.KDA_EDTYPE),
    (dict(s0=None, s0_dt=2), kda.KDA_EDTYPE),
    (dict(ws_bytes=700), kda.KDA_EWORKSPACE),
])
def test_segmented_host_validation_rejects(segments, over, code):
    rc = call_seg(segments, **over)
    assert rc == code, (rc, kda.last_error())


def test_segmented_segments_and_workspace():
    """kda_fwd_segmented: the segment count it takes and its workspace, which
    starts with the plain forward's workspace for the segments (so the status
    word sits where kda_fwd_check_status reads it)."""
    for bad in (-1, 4097):
        assert call_seg(bad) == kda.KDA_EINVAL and "segments" in kda.last_error()
        assert kda.segmented_workspace_bytes(1, 64, 2, 0, False, bad) == 0
    # the library's count: the largest power of two with at most 128
    # (segment, head) chains and segments of at least 512 tokens, 1 below 4
    for (B, T, H, N, cu), want in (((1, 8192, 4, 0, False), 16), ((1, 8192, 16, 0, False), 8),
                                   ((1, 8192, 32, 0, False), 4), ((1, 8192, 64, 0, False), 1),
                                   ((1, 8192, 96, 0, False), 1), ((1, 65536, 4, 0, False), 32),
                                   ((1, 32768, 8, 0, False), 16), ((1, 1024, 4, 0, False), 1),
                                   ((2, 8192, 4, 0, False), 16), ((1, 16384, 4, 2, True), 16),
                                   ((1, 8192, 1, 8, True), 1)):
        assert kda.segments_for(B, T, H, N, cu) == want, (B, T, H, N, cu)
        assert (kda.segmented_workspace_bytes(B, T, H, N, cu, 0)
                == kda.segmented_workspace_bytes(B, T, H, N, cu, want))
    assert kda.segments_for(1, 64, 0) == 0
    assert kda.segmented_workspace_bytes(1, 8192, 96, 0, False, 1) == kda.workspace_bytes(1, 8192, 96, path="auto")
    al = lambda x: (x + 255) // 256 * 256
    for B, T, H, N, has_cu, S in ((1, 8192, 8, 0, False, 4), (2, 1000, 3, 0, False, 3), (1, 5000, 4, 3, True, 8)):
        NS = (N if has_cu else B) * S
        inner = kda.workspace_bytes(1, B * T, H, NS, True, path="auto")
        mat = NS * H * 128 * 128 * 4
        want = al(inner) + al((NS + 1) * 8) + al(mat // 2) + 2 * al(mat)   # A in fp16, two fp32 states
        assert kda.segmented_workspace_bytes(B, T, H, N, has_cu, S) == want
    # a workspace one byte short is refused on the host
    need = kda.segmented_workspace_bytes(1, 64, 2, 0, False, 4)
    assert call_seg(4, ws_bytes=need - 1) == kda.KDA_EWORKSPACE


def test_precision_study_rejects_bad_variants():
    a = [FAKE, FAKE, FAKE, FAKE, FAKE, 0.088, FAKE, FAKE, FAKE, -5.0, None, 0, None, 0, None, 0, 1, 64, 2, 128,
         128, WS, 1 << 40, None]
    for bad in (-1, 16, 17, 32):
        assert kda.lib().kda_fwd_precision(*a, bad) == kda.KDA_EINVAL and "precision" in kda.last_error()
    # the remaining checks are kda_fwd's, made before any HIP call
    a[0] = None
    assert kda.lib().kda_fwd_precision(*a, 1) == kda.KDA_EINVAL
    a[0] = FAKE
    a[22] = 700
    assert kda.lib().kda_fwd_precision(*a, 7) == kda.KDA_EWORKSPACE
    assert kda.lib().kda_fwd_precision(*a, kda.KDA_PREC_NEUMANN_FP16 | 1) == kda.KDA_EWORKSPACE


def test_kda_fwd_workspace_covers_its_segmented_form():
    """kda_fwd cuts B sequences of T tokens into kda_fwd_segments' count of
    segments when that is above 1 and the workspace allows; its all-paths size
    covers that layout, and stays the plain one when the count is 1."""
    for B, T, H in ((1, 8192, 4), (2, 4096, 8), (1, 65536, 2)):
        S = kda.segments_for(B, T, H)
        assert S > 1
        seg = kda.segmented_workspace_bytes(B, T, H, 0, False, S)
        assert kda.workspace_bytes(B, T, H) == max(seg, kda.workspace_layout(B, T, H, chunk=16)["total"],
                                                   kda.workspace_layout(B, T, H, chunk=32)["total"])
    for B, T, H in ((1, 8192, 96), (1, 1024, 4)):
        assert kda.segments_for(B, T, H) == 1
        assert kda.workspace_bytes(B, T, H) == max(kda.workspace_layout(B, T, H, chunk=16)["total"],
                                                   kda.workspace_layout(B, T, H, chunk=32)["total"])
    # with cu_seqlens the lengths are the device's: no cut, plain sizes
    assert kda.workspace_bytes(1, 8192, 4, 1, True) == max(kda.workspace_layout(1, 8192, 4, 1, True, chunk=16)["total"],
                                                            kda.workspace_layout(1, 8192, 4, 1, True, chunk=32)["total"])


def test_bench_refuses_more_than_one_gpu():
    """bench.py measures one GPU; asked for more it exits with status 2 and a
    message, before touching a device."""
    import subprocess
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    r = subprocess.run([sys.executable, os.path.join(root, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "--gpus 1" in r.stderr and r.stdout == ""
