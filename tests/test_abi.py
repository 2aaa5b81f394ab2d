"""The C ABI library loads, exports every function include/spectree.h declares,
and rejects bad arguments on the host before anything reaches the GPU.  No
compute call is made here (these tests run without a GPU)."""
import ctypes

import pytest

import tree_verify_attention_masked_amd as stv
from tree_verify_attention_masked_amd import binding


@pytest.fixture(scope="module")
def lib():
    return stv.load_library()


def test_every_declared_symbol_is_exported(lib):
    names = stv.header_functions()
    assert {"spec_tree_attn", "spec_tree_reject", "spec_kv_compact"} <= set(names)
    for n in names:
        assert hasattr(lib, n), n
    assert set(binding._SIGNATURES) == set(names)


def test_status_strings_and_version(lib):
    assert stv.spec_version() >= 100
    for code in (0, -1, -2, -3, -4):
        assert stv.spec_status_string(code).startswith("SPEC_")
    assert stv.spec_status_string(7) == "unknown spec_status"


def test_workspace_sizes(lib):
    # fp32 and single-split bf16 need none; split-KV needs room for every partial
    assert lib.spec_tree_attn_workspace_size(1, 8, 2, 2, 64, 9, 0) == 0
    ws = lib.spec_tree_attn_workspace_size(1, 5, 40, 40, 128, 129, 1)
    assert ws > 0 and ws % 4 == 0
    assert lib.spec_tree_attn_workspace_size(1, 5, 40, 40, 100, 129, 1) == 0  # unsupported head dim
    ws = lib.spec_tree_reject_workspace_size(2, 5, 32000)
    assert ws >= 2 * 64 and ws % 16 == 0  # per-sequence header + exchange slots
    assert lib.spec_tree_reject_workspace_size(4, 5, 32000) > ws
    assert lib.spec_tree_reject_workspace_size(0, 5, 32000) == 0


FAKE = ctypes.c_void_p(0x1000)  # never dereferenced: every call below fails validation first


def _attn(lib, **kw):
    a = dict(B=1, T=5, Hq=4, Hkv=4, D=128, bs=16, mb=8, nb=8, scale=0.1, dtype=1, ws=None, wsz=0)
    a.update(kw)
    ptrs = [FAKE] * 7
    if kw.get("null_q"):
        ptrs[0] = None
    if kw.get("misaligned"):
        ptrs[0] = ctypes.c_void_p(0x1008)
    return lib.spec_tree_attn(*ptrs, a["B"], a["T"], a["Hq"], a["Hkv"], a["D"], a["bs"], a["mb"], a["nb"],
                              a["scale"], a["dtype"], None, a["ws"], a["wsz"], None)


def test_attn_host_validation(lib):
    assert _attn(lib, null_q=True) == -1
    assert _attn(lib, T=0) == -1
    assert _attn(lib, Hq=6, Hkv=4) == -1
    assert _attn(lib, D=64) == -2  # bf16 needs D = 128
    assert _attn(lib, dtype=0, D=96) == -2
    assert _attn(lib, bs=8) == -2
    assert _attn(lib, T=513, mb=40) == -2
    assert _attn(lib, mb=0) == -1
    assert _attn(lib, T=200, mb=8) == -1  # the table cannot even hold the tree
    assert _attn(lib, scale=float("nan")) == -1
    assert _attn(lib, scale=0.0) == -1
    assert _attn(lib, scale=-0.1) == -1
    assert _attn(lib, dtype=5) == -1
    assert _attn(lib, B=0) == 0  # empty batch: nothing to do
    assert _attn(lib, misaligned=True) == -1  # rows move with 16-byte accesses
    # a split-KV plan without workspace
    assert _attn(lib, T=5, Hq=40, Hkv=40, mb=129, nb=129) == -3


def _reject(lib, **kw):
    a = dict(B=1, T=4, V=100, tau=1.0, ws=FAKE, wsz=1 << 20, null_logits=False)
    a.update(kw)
    logits = None if a["null_logits"] else FAKE
    return lib.spec_tree_reject(logits, FAKE, FAKE, FAKE, a["B"], a["T"], a["V"], a["tau"], 0, 0, 0,
                                FAKE, FAKE, FAKE, None, a["ws"], a["wsz"], None)


def test_reject_host_validation(lib):
    assert _reject(lib, null_logits=True) == -1
    assert _reject(lib, tau=-1.0) == -1
    assert _reject(lib, tau=float("inf")) == -1
    assert _reject(lib, T=0) == -1
    assert _reject(lib, T=513) == -2
    assert _reject(lib, V=300000) == -2
    assert _reject(lib, ws=None) == -3
    assert _reject(lib, wsz=10) == -3
    assert _reject(lib, B=0) == 0


def test_compact_host_validation(lib):
    def call(**kw):
        a = dict(B=1, T=5, Hkv=2, D=128, bs=16, mb=4, nb=4, dtype=1)
        a.update(kw)
        return lib.spec_kv_compact(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, a["B"], a["T"], a["Hkv"], a["D"],
                                   a["bs"], a["mb"], a["nb"], a["dtype"], None, None)
    assert call(D=32) == -2
    assert call(bs=32) == -2
    assert call(Hkv=0) == -1
    assert call(B=0) == 0
    assert lib.spec_kv_compact(None, FAKE, FAKE, FAKE, FAKE, FAKE, None, 1, 5, 2, 128, 16, 4, 4, 1, None,
                               None) == -1


def test_reject_compact_host_validation(lib):
    def call(**kw):
        a = dict(B=1, T=5, V=100, tau=1.0, ws=FAKE, wsz=1 << 20, k=FAKE, Hkv=2, D=128, bs=16, mb=4, nb=4, dtype=1)
        a.update(kw)
        return lib.spec_tree_reject_compact(FAKE, FAKE, FAKE, FAKE, a["B"], a["T"], a["V"], a["tau"], 0, 0, 0,
                                            FAKE, FAKE, FAKE, None, a["ws"], a["wsz"], a["k"], FAKE, FAKE, FAKE,
                                            None, a["Hkv"], a["D"], a["bs"], a["mb"], a["nb"], a["dtype"], None)
    assert call(tau=-1.0) == -1     # the sampler's checks
    assert call(T=513) == -2
    assert call(wsz=10) == -3
    assert call(k=None) == -1       # the compaction's checks
    assert call(D=32) == -2
    assert call(bs=32) == -2
    assert call(Hkv=0) == -1
    assert call(B=0) == 0



def test_kv_write_host_validation(lib):
    def call(**kw):
        a = dict(B=1, T=5, Hq=4, Hkv=2, D=128, bs=16, mb=4, nb=4, theta=10000.0, dtype=1, q=FAKE, k=FAKE)
        a.update(kw)
        return lib.spec_tree_kv_write(a["k"], FAKE, a["q"], FAKE, FAKE, FAKE, FAKE, FAKE, None, a["B"], a["T"],
                                      a["Hq"], a["Hkv"], a["D"], a["bs"], a["mb"], a["nb"], a["theta"], a["dtype"],
                                      None)
    assert call(k=None) == -1
    assert call(Hq=3) == -1            # query heads must be a multiple of kv heads
    assert call(Hq=0) == -1
    assert call(theta=-1.0) == -1
    assert call(theta=float("nan")) == -1
    assert call(theta=float("inf")) == -1
    assert call(D=64) == -2            # bf16 needs D = 128
    assert call(bs=8) == -2
    assert call(T=513, mb=40) == -2
    assert call(T=100, mb=4) == -1     # the table cannot hold the tree
    assert call(B=0) == 0
    assert call(B=0, q=None, Hq=0) == 0  # no queries to rotate
    assert call(k=ctypes.c_void_p(0x1002)) == -1  # rows move with 16-byte accesses
    assert call(q=ctypes.c_void_p(0x1008)) == -1

def test_binding_refuses_cpu_tensors():
    import torch
    q = torch.zeros(1, 2, 2, 128, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        stv.spec_tree_attn(q, q, q, torch.zeros(1, 1, dtype=torch.int32), torch.zeros(1, dtype=torch.int32),
                           torch.zeros(1, 2, dtype=torch.int32))


def test_truncate_host_validation(lib):
    def call(**kw):
        a = dict(B=1, T=5, V=100, tau=1.0, k=10, p=0.9, i=FAKE, o=FAKE)
        a.update(kw)
        return lib.spec_tree_truncate(a["i"], a["o"], a["B"], a["T"], a["V"], a["tau"], a["k"], a["p"], None, None)
    assert call(i=None) == -1
    assert call(o=None) == -1
    assert call(B=-1) == -1
    assert call(T=0) == -1
    assert call(V=0) == -1
    assert call(V=(1 << 24) + 1) == -2
    assert call(tau=-0.5) == -1
    assert call(tau=float("inf")) == -1
    assert call(tau=float("nan")) == -1
    assert call(p=0.0) == -1
    assert call(p=float("nan")) == -1
    assert call(B=0) == 0
    assert call(B=0, i=None) == 0    # nothing to do before the pointers matter



def test_reject_team_plan_fits_the_resident_grid(lib):
    # The sampler's team members wait for each other, so a team of more than one
    # member needs the whole grid resident: B * team <= what the device holds.
    full = 256  # one workgroup per CU on a 256-CU device
    assert stv.spec_tree_reject_plan(1, 5, 32000, full) == (63, 508)       # chain: 63 members
    assert stv.spec_tree_reject_plan(64, 16, 32000, full) == (4, 8000)     # batched serving
    assert stv.spec_tree_reject_plan(1, 256, 32000, full) == (32, 1000)    # deep trees: at most 32
    assert stv.spec_tree_reject_plan(1, 5, 1000, full) == (2, 500)         # at least 512 entries a member
    for B in (1, 3, 8, 64, 100, 255, 256, 300, 1000):
        for T in (1, 5, 16, 64, 256):
            for V in (3, 1000, 32000, 128256, 262144):
                for cap in (1, 2, 7, 64, 100, 255, 256, 1024):
                    team, sl = stv.spec_tree_reject_plan(B, T, V, cap)
                    assert team >= 1 and team * sl >= V and (team - 1) * sl < V
                    assert team == 1 or B * team <= cap, (B, T, V, cap, team)
                    assert team <= (32 if T > 16 else 64)
                    # the workspace size query covers the largest team any device gets
                    big, _ = stv.spec_tree_reject_plan(B, T, V, 1 << 40)
                    assert team <= big
    # a device holding fewer workgroups gets smaller teams, down to one per sequence
    assert stv.spec_tree_reject_plan(64, 16, 32000, 128) == (2, 16000)
    assert stv.spec_tree_reject_plan(64, 16, 32000, 127) == (1, 32000)
    assert stv.spec_tree_reject_plan(300, 5, 32000, 256) == (1, 32000)
    with pytest.raises(stv.SpecError):
        stv.spec_tree_reject_plan(1, 5, 32000, 0)
    with pytest.raises(stv.SpecError):
        stv.spec_tree_reject_plan(1, 513, 32000, 256)


def test_truncated_sampler_plan_and_validation(lib):
    full = 256
    # first lists of a later row: each member's slice cut into 4 parts from 2048 logits on (2 from 1024) while a
    # row keeps at most 64 lists, a list of about twice a part's share of the top-k plus 6 (chain: 63 parts,
    # 2 * 50 / 63 -> 2 + 6; batched serving: 4 members x 4 parts of 2000, 100 / 16 -> 7 + 6; EAGLE-style:
    # 32 members x 2 parts of 2004, 80 / 64 -> 2 + 6)
    assert stv.spec_tree_reject_truncated_plan(1, 5, 32000, 50, full) == (63, 8)
    assert stv.spec_tree_reject_truncated_plan(64, 16, 32000, 50, full) == (4, 13)
    assert stv.spec_tree_reject_truncated_plan(8, 64, 128256, 40, full) == (32, 8)
    assert stv.spec_tree_reject_truncated_plan(1, 256, 32000, 50, full) == (32, 10)
    for B in (1, 3, 64, 300):
        for T in (1, 5, 16, 300, 512):
            for V in (3, 1000, 32000, 128256):
                for k in (1, 7, 50, 64):
                    team, kc = stv.spec_tree_reject_truncated_plan(B, T, V, k, full)
                    assert team == stv.spec_tree_reject_plan(B, T, V, full)[0]
                    assert 1 <= kc <= k
                    # every list of one row fits the buffer that merges them (at most 4 parts a member)
                    assert team * (k + 2) <= 7680 and 4 * team * (kc + 2) <= 7680
    ws = lib.spec_tree_reject_truncated_workspace_size(2, 5, 32000, 50)
    assert ws > lib.spec_tree_reject_workspace_size(2, 5, 32000)
    assert lib.spec_tree_reject_truncated_workspace_size(2, 5, 32000, 64) > ws
    assert lib.spec_tree_reject_truncated_workspace_size(2, 5, 32000, 0) == 0
    assert lib.spec_tree_reject_truncated_workspace_size(2, 5, 32000, 65) == 0
    for k in (0, 65):
        with pytest.raises(stv.SpecError, match="UNSUPPORTED"):
            stv.spec_tree_reject_truncated_plan(1, 5, 32000, k, full)

    def call(**kw):  # every call below fails validation (or has nothing to do) before any launch
        a = dict(B=1, T=5, V=100, tau=1.0, k=10, p=0.9, ws=FAKE, wsz=1 << 30, kc=None, Hkv=2, D=128, bs=16, mb=4,
                 nb=4, dtype=1)
        a.update(kw)
        return lib.spec_tree_reject_truncated(FAKE, FAKE, FAKE, FAKE, a["B"], a["T"], a["V"], a["tau"], a["k"],
                                              a["p"], 0, 0, 0, FAKE, FAKE, FAKE, None, a["ws"], a["wsz"], a["kc"],
                                              FAKE, FAKE, FAKE, None, a["Hkv"], a["D"], a["bs"], a["mb"], a["nb"],
                                              a["dtype"], None)
    assert call(k=0) == -2
    assert call(k=65) == -2
    assert call(p=0.0) == -1
    assert call(p=float("nan")) == -1
    assert call(tau=-1.0) == -1
    assert call(T=513) == -2
    assert call(wsz=10) == -3
    assert call(ws=FAKE, wsz=lib.spec_tree_reject_workspace_size(1, 5, 100)) == -3  # the plain sampler's is short
    assert call(kc=FAKE, D=32) == -2    # the compaction's checks apply when a cache is given
    assert call(kc=FAKE, Hkv=0) == -1
    assert call(B=0) == 0
