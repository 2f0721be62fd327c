"""The C ABI on the CPU: the library loads, exports what include/rtp.h declares,
sizes workspaces and rejects bad arguments before any launch (no GPU calls)."""
import ctypes
import os
import re

import pytest

import long_context_sparse_retrieval_amd as rtp

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "rtp.h")

needs_lib = pytest.mark.skipif(not os.path.exists(rtp.library_path()),
                               reason="librtp.so not built (run __graft_entry__.build())")


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(rtp_[a-z_0-9]+)\s*\(", src)))


def test_header_declares_the_boundary():
    names = declared_functions()
    for required in ("rtp_index_score", "rtp_topp_select", "rtp_sparse_attn", "rtp_swa_attn", "rtp_decode_step",
                     "rtp_index_keys", "rtp_rope_keys", "rtp_workspace_bytes", "rtp_workspace_init",
                     "rtp_status_str", "rtp_num_retrieval"):
        assert required in names
    assert set(names) == set(rtp.SYMBOLS)


@needs_lib
def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(rtp.library_path())
    for name in declared_functions():
        assert hasattr(lib, name), name


def _layer(**kw):
    d = dict(B=2, Hq=8, Hkv=2, N=5000, head_mode=[1, 1, 1, 1, 0, 0, 0, 0])
    d.update(kw)
    return rtp.Layer(**d)


@needs_lib
def test_status_strings_and_retrieval_count():
    lib = rtp.load()
    assert lib.rtp_status_str(0) == b"ok"
    assert lib.rtp_status_str(-3) == b"workspace too small"
    assert rtp.num_retrieval(_layer()) == 4
    assert rtp.num_retrieval(_layer(head_mode=[0] * 8)) == 0


@needs_lib
def test_workspace_sizing_monotone():
    small = rtp.workspace_bytes(_layer(N=1000))
    big = rtp.workspace_bytes(_layer(N=100000))
    assert 0 < small < big
    assert rtp.workspace_bytes(_layer(N=5000, Ncap=9000)) == rtp.workspace_bytes(_layer(N=5000))


@needs_lib
@pytest.mark.parametrize("kw,code", [
    (dict(D=64), -2), (dict(R=8), -2), (dict(Hkv=3), -2), (dict(N=0), -2), (dict(N=10, Ncap=5), -2),
    (dict(nq=0), -2), (dict(N=1 << 31, Ncap=1 << 31), -2), (dict(p=0.0), -1), (dict(p=float("nan")), -1),
    (dict(window=0), -1), (dict(n_sink=-1), -1), (dict(head_mode=[2, 0, 0, 0, 0, 0, 0, 0]), -1),
    (dict(rope_theta=0.0), -1), (dict(top_k=-1), -1), (dict(idx_group=3), -1), (dict(idx_group=-1), -1),
    (dict(local_ring=2), -1), (dict(local_ring=-1), -1), (dict(scan_tile=3000), -1), (dict(scan_tile=512), -1),
    (dict(swa_chunk=100), -1), (dict(swa_chunk=-64), -1), (dict(pf_qch=24), -1), (dict(pf_qch=-16), -1),
    (dict(Hq=512, Hkv=2, head_mode=[0] * 512), -2),
])
def test_layer_validation(kw, code):
    lay = _layer(**kw)
    assert rtp.load().rtp_num_retrieval(ctypes.byref(lay.c())) == code
    assert rtp.load().rtp_workspace_bytes(ctypes.byref(lay.c())) == 0


@needs_lib
def test_tuning_fields_change_the_split_not_the_validity():
    base = rtp.workspace_bytes(_layer(N=40000))
    for kw in (dict(scan_tile=1024), dict(scan_tile=8192), dict(swa_chunk=64), dict(swa_chunk=1024)):
        assert rtp.workspace_bytes(_layer(N=40000, **kw)) > 0
    # smaller scan tiles need more tile summaries
    assert rtp.workspace_bytes(_layer(N=40000, scan_tile=1024)) > rtp.workspace_bytes(_layer(N=40000, scan_tile=8192))
    assert base > 0


def test_p_crosses_the_abi_as_double():
    """p is not narrowed: the struct field is a C double."""
    fields = dict(rtp._CLayer._fields_)
    assert fields["p"] is ctypes.c_double
    lay = _layer(p=0.1)
    assert lay.c().p == 0.1


@needs_lib
def test_calls_reject_before_launch():
    lib = rtp.load()
    lay = _layer()
    L = ctypes.byref(lay.c())
    need = rtp.workspace_bytes(lay)
    fake = 1 << 40     # never dereferenced: every call below fails validation first
    # workspace too small
    assert lib.rtp_topp_select(L, fake, fake, fake, 16, fake, need - 1, None) == -3
    assert lib.rtp_decode_step(L, fake, fake, fake, fake, fake, fake, None, None, 0, fake, need - 1, None, None) == -3
    # null pointers / bad ranges
    assert lib.rtp_index_score(L, None, fake, fake, fake, None) == -1
    assert lib.rtp_rope_keys(L, fake, fake, 10, 5, None) == -1
    assert lib.rtp_index_keys(L, fake, fake, fake, 0, lay.N + 1, None) == -1
    assert lib.rtp_swa_attn(L, None, fake, fake, fake, fake, need, None) == -1
    assert lib.rtp_sparse_attn(L, fake, fake, fake, fake, fake, -1, fake, fake, need, None) == -1
    assert lib.rtp_workspace_init(None, 16, None) == -1
    cap = lay.cap_rows
    assert lib.rtp_append_kv(L, fake, fake, fake, fake, fake, fake, cap - 1, 2, None) == -1     # past Ncap
    assert lib.rtp_append_kv(L, fake, fake, fake, fake, fake, fake, -1, 1, None) == -1
    assert lib.rtp_append_kv(L, fake, fake, fake, fake, fake, fake, 0, -1, None) == -1
    assert lib.rtp_append_kv(L, None, fake, fake, fake, fake, fake, 0, 1, None) == -1
    assert lib.rtp_append_kv(L, fake, fake, None, fake, fake, fake, 0, 1, None) == -1           # retrieval layer needs W_k
    assert lib.rtp_append_kv(L, None, None, None, None, None, None, 5, 0, None) == 0            # nothing to do
    # misaligned workspace or arrays (the kernels use 16-byte vector accesses)
    assert lib.rtp_swa_attn(L, fake, fake, fake, fake, fake + 8, need, None) == -1
    assert lib.rtp_swa_attn(L, fake + 2, fake, fake, fake, fake, need, None) == -1
    assert lib.rtp_decode_step(L, fake, fake, fake, fake + 8, fake, fake, None, None, 0, fake, need, None, None) == -1
    assert lib.rtp_index_keys(L, fake, fake, fake + 4, 0, 10, None) == -1
    assert lib.rtp_append_kv(L, fake, fake, fake, fake, fake + 16 + 8, fake, 0, 1, None) == -1
    # chunked prefill (nq > 1) is validated the same way before any launch
    lay2 = _layer(nq=4)
    L2 = ctypes.byref(lay2.c())
    need2 = rtp.workspace_bytes(lay2)
    assert lib.rtp_decode_step(L2, fake, fake, fake, fake, fake, fake, None, None, 0, fake, need2 - 1, None, None) == -3
    assert lib.rtp_decode_step(L2, fake, None, fake, fake, fake, fake, None, None, 0, fake, need2, None, None) == -1


@needs_lib
def test_ring_layout_rows_and_limits():
    """K/V rows per sequence with local_ring (closed form), and the calls that
    need positions a ring no longer holds refuse it before any launch."""
    lib = rtp.load()
    fake = 1 << 40
    N, W, S = 5000, 4096, 4
    # KV group 0 retrieval, group 1 all local
    assert rtp.kv_rows(_layer()) == 2 * N
    assert rtp.kv_rows(_layer(local_ring=1)) == N + (S + W)
    assert rtp.kv_rows(_layer(local_ring=1, head_mode=[1, 0, 0, 0] + [0] * 4)) == N + (S + W)   # mixed group: full
    assert rtp.kv_rows(_layer(local_ring=1, head_mode=[0] * 8, window=100, n_sink=0)) == 2 * 100
    assert rtp.kv_rows(_layer(local_ring=1, head_mode=[1] * 8)) == 2 * N
    assert rtp.kv_rows(_layer(local_ring=1, Ncap=9000)) == 9000 + (S + W)
    assert lib.rtp_kv_rows(ctypes.byref(_layer(local_ring=3).c())) == -1
    ring = _layer(local_ring=1)
    L = ctypes.byref(ring.c())
    need = rtp.workspace_bytes(ring)
    assert lib.rtp_prefill_attn(L, fake, fake, fake, fake, 0, None) == -4
    assert lib.rtp_dense_attn(L, fake, fake, fake, fake, fake, need, None) == -4
    r4 = _layer(local_ring=1, nq=4)
    L4 = ctypes.byref(r4.c())
    n4 = rtp.workspace_bytes(r4)
    assert lib.rtp_decode_step(L4, fake, fake, fake, fake, fake, fake, None, None, 0, fake, n4, None, None) == -4
    assert lib.rtp_swa_attn(L4, fake, fake, fake, fake, fake, n4, None) == -4
    # no ring group (every KV group has a retrieval head): local_ring changes nothing
    nr = _layer(local_ring=1, head_mode=[1, 0, 0, 0, 0, 0, 0, 1])
    assert rtp.kv_rows(nr) == 2 * N
    assert lib.rtp_prefill_attn(ctypes.byref(nr.c()), None, fake, fake, fake, 0, None) == -1    # reaches the checks


@needs_lib
def test_cluster_calls_validate_before_launch():
    lib = rtp.load()
    fake = 1 << 40
    lay = _layer()
    L = ctypes.byref(lay.c())
    need = lib.rtp_cluster_workspace_bytes(L, 16)
    assert need > rtp.workspace_bytes(lay)
    assert lib.rtp_cluster_workspace_bytes(L, 0) == 0 and lib.rtp_cluster_workspace_bytes(L, 257) == 0
    assert lib.rtp_cluster_workspace_bytes(ctypes.byref(_layer(N=10).c()), 11) == 0      # K > N
    assert lib.rtp_cluster_build(L, fake, 16, -1, fake, fake, fake, fake, fake, need, None) == -1
    assert lib.rtp_cluster_build(L, fake, 16, 2, fake, fake, fake, fake, fake, need - 1, None) == -3
    assert lib.rtp_cluster_build(L, None, 16, 2, fake, fake, fake, fake, fake, need, None) == -1
    for kw in (dict(top_k=5), dict(nq=4)):
        lk = _layer(**kw)
        nk = lib.rtp_cluster_workspace_bytes(ctypes.byref(lk.c()), 16)
        assert lib.rtp_cluster_step(ctypes.byref(lk.c()), fake, fake, 16, fake, fake, fake, fake, fake, fake, fake,
                                    None, None, 0, fake, nk, None) == -4
    assert lib.rtp_cluster_step(L, fake, fake, 16, fake, fake, fake, fake, fake, fake, fake, None, None, 0, fake,
                                need - 1, None) == -3


def test_layer_struct_follows_field_changes():
    """The binding memoises the C struct of a layer: a changed field rebuilds
    it, and a dataclasses.replace copy owns its own struct and head_mode array."""
    import dataclasses
    lay = _layer()
    c1 = lay.c()
    assert lay.c() is c1                                   # unchanged fields: the same struct
    lay.N = 4000
    c2 = lay.c()
    assert c2 is not c1 and c2.N == 4000 and c2.Ncap == 4000
    ring = dataclasses.replace(lay, local_ring=1)
    assert ring._memo is not lay._memo
    assert ring.c().local_ring == 1 and lay.c().local_ring == 0
    lay.head_mode = [0] * 8
    assert [lay.c().head_mode[h] for h in range(8)] == [0] * 8
    assert [ring.c().head_mode[h] for h in range(8)] == [1, 1, 1, 1, 0, 0, 0, 0]


def test_binding_checks_tensors_without_gpu():
    import torch
    lay = _layer()
    with pytest.raises((TypeError, ValueError, rtp.RtpError)):
        rtp.index_score(lay, torch.zeros(2, 8, 1, 128), torch.zeros(4, 128, 16), torch.zeros(2, 4, 5000, 16))


def test_package_does_not_touch_the_oracle():
    pkg = os.path.dirname(rtp.__file__)
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".h", ".cpp")):
                txt = open(os.path.join(dirpath, f)).read()
                assert not re.search(r"^\s*(import|from)\s+oracle", txt, re.M), f
                assert "rtp_oracle" not in txt, f


@needs_lib
def test_static_step_checks_before_any_device_work():
    """rtp_decode_step_static validates the layer and the scratch bound on the
    host and returns without touching a device (dummy pointers are never used)."""
    lib = rtp.load()
    big = _layer(B=64, Hq=64, Hkv=8, N=1 << 20, head_mode=[1] * 64)
    assert rtp.workspace_bytes(big) > rtp.STATIC_SCRATCH_BYTES
    p = 16
    assert lib.rtp_decode_step_static(ctypes.byref(big.c()), p, p, p, p, p, p, None, None, 0, None) == -3
    assert lib.rtp_decode_step_static(ctypes.byref(_layer(D=64).c()), p, p, p, p, p, p, None, None, 0, None) == -2
