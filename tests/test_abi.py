"""C ABI checks that need no GPU: the library loads, exports every symbol the
header declares, and rejects invalid arguments before launching anything."""

import ctypes
import os
import re

import pytest

import causal_attention_attn_amd as attn
from causal_attention_attn_amd import _lib

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                      "include", "attn.h")

# a fake, 16-byte aligned, non-null address; every call below fails validation
# before any launch, so it is never dereferenced
FAKE = 0x100000
MIS = FAKE + 4


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(_lib.LIB_PATH):
        import __graft_entry__
        __graft_entry__.build()
    return attn.load()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[\w\*]+\s+\**\s*(attn_\w+)\s*\(", text, re.M)))


def test_header_declares_the_entry_points():
    names = declared_functions()
    for n in ("attn_fwd", "attn_fwd_rotated", "attn_rotate_qk", "attn_saved_bytes", "attn_bwd",
              "attn_bwd_prep", "attn_bwd_grads", "attn_rope_tables", "attn_bwd_workspace_bytes",
              "attn_fwd_packed", "attn_bwd_packed", "attn_kv_cache_bytes", "attn_kv_append",
              "attn_decode_workspace_bytes", "attn_decode", "attn_decode_step", "attn_rmsnorm_fwd",
              "attn_rmsnorm_bwd_workspace_bytes", "attn_rmsnorm_bwd", "attn_swiglu_fwd",
              "attn_swiglu_bwd", "attn_status_string", "attn_last_hip_error"):
        assert n in names


def test_library_exports_every_declared_symbol(lib):
    raw = ctypes.CDLL(_lib.LIB_PATH)
    for n in declared_functions():
        assert hasattr(raw, n), n
    assert set(declared_functions()) == set(_lib._SIGS)


def test_status_strings(lib):
    for code in range(10):
        assert attn.attn_status_string(code) != "unknown status"
    assert attn.attn_status_string(99) == "unknown status"
    assert attn.attn_last_hip_error() == 0


def test_workspace_size(lib):
    assert attn.attn_bwd_workspace_bytes(8, 12, 1024, 64, 0) == 8 * 8 * 12 * 1024
    assert attn.attn_bwd_workspace_bytes(8, 12, 1024, 64, 1) == 4 * 8 * 12 * 1024
    assert attn.attn_bwd_workspace_bytes(1, 1, 3, 64, 0) == 256
    assert attn.attn_saved_bytes(8, 12, 1024, 64, 0) == 4 * 8 * 12 * 1024 * 64
    assert attn.attn_saved_bytes(8, 12, 1024, 64, 1) == 0
    assert attn.attn_saved_bytes(1, 1, 3, 96, 0) == 0
    assert attn.attn_bwd_workspace_bytes(1, 1, 3, 96, 0) == 0
    assert attn.attn_bwd_workspace_bytes(1, 1, 0, 64, 0) == 0
    assert attn.attn_bwd_workspace_bytes(1, 1, 3, 64, 7) == 0


def status_of(fn, *args):
    with pytest.raises(attn.AttnError) as e:
        fn(*args)
    return e.value.status


def fwd_args(**over):
    a = dict(q=FAKE, k=FAKE + 16, v=FAKE + 32, cos_tab=FAKE + 48, sin_tab=FAKE + 64,
             o=FAKE + 80, lse=FAKE + 96, saved=FAKE + 112, saved_bytes=4 * 8 * 64,
             B=1, H=1, T=8, D=64, dtype=0, stream=0)
    a.update(over)
    return a


def test_fwd_rejects_bad_arguments(lib):
    f = lambda **o: status_of(lambda: attn.attn_fwd(**fwd_args(**o)))
    assert f(q=0) == 1
    assert f(lse=0) == 1
    assert f(D=96) == 2
    assert f(D=32) == 2
    assert f(T=0) == 2
    assert f(B=0) == 2
    assert f(B=1 << 16, H=1 << 10, T=1 << 10) == 2      # 2^42 elements
    assert f(dtype=3) == 3
    assert f(k=MIS) == 4
    assert f(o=FAKE) == 7                                 # o aliases q
    assert f(lse=FAKE + 32) == 7                          # lse aliases v
    assert f(saved=0) == 1                                # bf16 needs the saved buffer
    assert f(saved=MIS) == 4
    assert f(saved_bytes=4 * 8 * 64 - 1) == 9
    assert f(saved=FAKE + 16) == 7                        # saved aliases k


def test_fwd_rotated_and_rotate_reject_bad_arguments(lib):
    f = lambda **o: status_of(lambda: attn.attn_fwd_rotated(
        **{**dict(saved=FAKE, saved_bytes=4 * 8 * 64, v=FAKE + 16, o=FAKE + 32, lse=FAKE + 48,
                  B=1, H=1, T=8, D=64, dtype=0, stream=0), **o}))
    assert f(dtype=1) == 3                                # fp32 has no rotated path
    assert f(saved=0) == 1
    assert f(saved_bytes=100) == 9
    assert f(o=FAKE) == 7
    g = lambda **o: status_of(lambda: attn.attn_rotate_qk(
        **{**dict(q=FAKE, k=FAKE + 16, cos_tab=FAKE + 32, sin_tab=FAKE + 48, saved=FAKE + 64,
                  saved_bytes=4 * 8 * 64, B=1, H=1, T=8, D=64, dtype=0, stream=0), **o}))
    assert g(q=0) == 1
    assert g(saved_bytes=0) == 9
    assert g(saved=FAKE) == 7
    assert g(D=48) == 2


def test_bwd_rejects_bad_arguments(lib):
    base = dict(q=FAKE, k=FAKE + 16, v=FAKE + 32, o=FAKE + 48, dO=FAKE + 64, lse=FAKE + 80,
                cos_tab=FAKE + 96, sin_tab=FAKE + 112, saved=FAKE + 192, saved_bytes=4 * 8 * 64,
                dq=FAKE + 128, dk=FAKE + 144, dv=FAKE + 160, workspace=FAKE + 176,
                workspace_bytes=256, B=1, H=1, T=8, D=64, dtype=0, stream=0)
    f = lambda **o: status_of(lambda: attn.attn_bwd(**{**base, **o}))
    assert f(dO=0) == 1
    assert f(D=100) == 2
    assert f(dtype=-1) == 3
    assert f(dq=MIS) == 4
    assert f(workspace=0) == 5
    assert f(workspace_bytes=255) == 5
    assert f(dk=FAKE) == 7
    assert f(dv=FAKE + 144) == 7                          # dv aliases dk
    assert f(workspace=FAKE + 80) == 7                    # workspace aliases lse
    assert f(saved=0) == 1
    assert f(saved_bytes=8) == 9
    assert f(dq=FAKE + 192) == 7                          # dq aliases saved


def test_bwd_stages_reject_bad_arguments(lib):
    f = lambda **o: status_of(lambda: attn.attn_bwd_prep(
        **{**dict(o=FAKE, dO=FAKE + 16, lse=FAKE + 32, workspace=FAKE + 48, workspace_bytes=256,
                  B=1, H=1, T=8, D=64, dtype=0, stream=0), **o}))
    assert f(o=0) == 1
    assert f(lse=0) == 1
    assert f(D=32) == 2
    assert f(dtype=5) == 3
    assert f(dO=MIS) == 4
    assert f(workspace=0) == 5
    assert f(workspace_bytes=255) == 5
    assert f(workspace=MIS) == 4
    assert f(workspace=FAKE + 16) == 7                   # workspace aliases dO
    base = dict(q=FAKE, k=FAKE + 16, v=FAKE + 32, dO=FAKE + 64, lse=FAKE + 80,
                cos_tab=FAKE + 96, sin_tab=FAKE + 112, saved=FAKE + 192, saved_bytes=4 * 8 * 64,
                dq=FAKE + 128, dk=FAKE + 144, dv=FAKE + 160, workspace=FAKE + 176,
                workspace_bytes=256, B=1, H=1, T=8, D=64, dtype=0, stream=0)
    g = lambda **o: status_of(lambda: attn.attn_bwd_grads(**{**base, **o}))
    assert g(dq=0) == 1
    assert g(saved=0) == 1
    assert g(saved_bytes=8) == 9
    assert g(workspace=0) == 5
    assert g(dv=FAKE + 32) == 7                           # dv aliases v
    assert g(dk=FAKE + 128) == 7                          # dk aliases dq
    assert g(dq=FAKE + 176) == 7                          # dq aliases the workspace


def test_packed_entry_points_reject_bad_arguments(lib):
    fb = dict(qkv=FAKE, cos_tab=FAKE + 16, sin_tab=FAKE + 32, o=FAKE + 48, lse=FAKE + 64,
              saved=FAKE + 80, saved_bytes=4 * 8 * 64, B=1, H=1, T=8, D=64, dtype=0, stream=0)
    f = lambda **o: status_of(lambda: attn.attn_fwd_packed(**{**fb, **o}))
    assert f(qkv=0) == 1
    assert f(saved=0) == 1
    assert f(D=96) == 2
    assert f(dtype=1) == 3                                # fp32 has no packed path
    assert f(dtype=7) == 3
    assert f(o=MIS) == 4
    assert f(saved_bytes=16) == 9
    assert f(o=FAKE) == 7                                 # o aliases qkv
    assert f(saved=FAKE + 32) == 7                        # saved aliases a table
    # the packed tensor (3*B*H*T*D elements) must stay below 2^31 elements
    assert f(B=1, H=16, T=1 << 19, D=128, saved_bytes=1 << 40) == 2   # 3 * 2^30 elements
    assert f(B=1, H=1 << 16, T=1, D=64, saved_bytes=1 << 40) == 2     # a token row of 3 * 2^22
    bb = dict(qkv=FAKE, o=FAKE + 16, dO=FAKE + 32, lse=FAKE + 48, cos_tab=FAKE + 64,
              sin_tab=FAKE + 80, saved=FAKE + 96, saved_bytes=4 * 8 * 64, dqkv=FAKE + 112,
              workspace=FAKE + 128, workspace_bytes=256, B=1, H=1, T=8, D=64, dtype=0, stream=0)
    g = lambda **o: status_of(lambda: attn.attn_bwd_packed(**{**bb, **o}))
    assert g(dqkv=0) == 1
    assert g(dO=0) == 1
    assert g(dtype=1) == 3
    assert g(T=0) == 2
    assert g(dqkv=MIS) == 4
    assert g(workspace=0) == 5
    assert g(workspace_bytes=255) == 5
    assert g(saved_bytes=8) == 9
    assert g(dqkv=FAKE) == 7                              # dqkv aliases qkv
    assert g(workspace=FAKE + 112) == 7                   # workspace aliases dqkv
    assert g(dqkv=FAKE + 96) == 7                         # dqkv aliases saved


def test_decode_sizes(lib):
    assert attn.attn_kv_cache_bytes(8, 12, 1024, 64, 0) == 4 * 8 * 12 * 1024 * 64
    assert attn.attn_kv_cache_bytes(8, 12, 1024, 64, 1) == 0             # fp32: no cache path
    assert attn.attn_kv_cache_bytes(1, 1, 1, 96, 0) == 0                 # unsupported D
    # one partial (D + 4 floats) per 64-key slice of Tmax, per head
    assert attn.attn_decode_workspace_bytes(8, 12, 1024, 64, 0) == 8 * 12 * 16 * 68 * 4
    assert attn.attn_decode_workspace_bytes(1, 2, 65, 128, 2) == ((2 * 2 * 132 * 4 + 255) // 256) * 256


def test_decode_entry_points_reject_bad_arguments(lib):
    cb = 4 * 1 * 1 * 8 * 64
    ab = dict(k=FAKE, v=FAKE + 16, cos_tab=FAKE + 32, sin_tab=FAKE + 48, cache=FAKE + 64,
              cache_bytes=cb, pos0=0, n=1, B=1, H=1, Tmax=8, D=64, dtype=0, stream=0)
    f = lambda **o: status_of(lambda: attn.attn_kv_append(**{**ab, **o}))
    assert f(k=0) == 1
    assert f(D=32) == 2
    assert f(n=0) == 2
    assert f(pos0=-1) == 2
    assert f(pos0=7, n=2) == 2                            # past Tmax
    assert f(dtype=1) == 3
    assert f(cache=MIS) == 4
    assert f(cache_bytes=cb - 1) == 5
    assert f(cache=FAKE) == 7                             # cache aliases k
    db = dict(q=FAKE, cache=FAKE + 16, cache_bytes=cb, cos_tab=FAKE + 32, sin_tab=FAKE + 48,
              o=FAKE + 64, lse=FAKE + 80, workspace=FAKE + 96, workspace_bytes=512, pos=3, B=1,
              H=1, Tmax=8, D=64, dtype=0, stream=0)
    g = lambda **o: status_of(lambda: attn.attn_decode(**{**db, **o}))
    assert g(q=0) == 1
    assert g(lse=0) == 1
    assert g(pos=8) == 2
    assert g(pos=-1) == 2
    assert g(Tmax=0) == 2
    assert g(dtype=1) == 3
    assert g(o=MIS) == 4
    assert g(cache_bytes=8) == 5
    assert g(workspace=0) == 5
    assert g(workspace_bytes=255) == 5
    assert g(workspace=MIS) == 4
    assert g(o=FAKE) == 7                                 # o aliases q
    assert g(workspace=FAKE + 16) == 7                    # workspace aliases the cache
    sb = dict(q=FAKE, k_new=FAKE + 112, v_new=FAKE + 128, cache=FAKE + 16, cache_bytes=cb,
              cos_tab=FAKE + 32, sin_tab=FAKE + 48, o=FAKE + 64, lse=FAKE + 80,
              workspace=FAKE + 96, workspace_bytes=512, pos=3, B=1, H=1, Tmax=8, D=64, dtype=0,
              stream=0)
    h = lambda **o: status_of(lambda: attn.attn_decode_step(**{**sb, **o}))
    assert h(k_new=0) == 1
    assert h(pos=8) == 2
    assert h(dtype=1) == 3
    assert h(v_new=MIS) == 4
    assert h(workspace_bytes=16) == 5
    assert h(cache=FAKE + 112) == 7                       # the cache aliases k_new
    assert h(o=FAKE + 16) == 7                            # o aliases the cache


def test_layer_entry_points_reject_bad_arguments(lib):
    assert attn.attn_rmsnorm_bwd_workspace_bytes(8192, 768, 0) == 1024 * 768 * 4
    assert attn.attn_rmsnorm_bwd_workspace_bytes(5, 256, 2) == 2 * 256 * 4
    assert attn.attn_rmsnorm_bwd_workspace_bytes(5, 300, 0) == 0
    fb = dict(x=FAKE, res=FAKE + 16, g=FAKE + 32, eps=1e-5, h=FAKE + 48, y=FAKE + 64,
              rstd=FAKE + 80, N=4, C=256, dtype=0, stream=0)
    f = lambda **o: status_of(lambda: attn.attn_rmsnorm_fwd(**{**fb, **o}))
    assert f(x=0) == 1
    assert f(y=0) == 1
    assert f(C=300) == 2
    assert f(C=4352) == 2
    assert f(N=0) == 2
    assert f(dtype=1) == 3
    assert f(eps=0.0) == 8
    assert f(eps=float("nan")) == 8
    assert f(res=MIS) == 4
    assert f(h=MIS) == 4
    assert f(y=FAKE) == 7                                 # y aliases x
    assert f(h=FAKE + 16) == 7                            # h aliases res
    bb = dict(h=FAKE, g=FAKE + 16, rstd=FAKE + 32, dy=FAKE + 48, dres=FAKE + 64, dh=FAKE + 80,
              dg=FAKE + 96, workspace=FAKE + 112, workspace_bytes=1024, N=4, C=256, dtype=0,
              stream=0)
    g = lambda **o: status_of(lambda: attn.attn_rmsnorm_bwd(**{**bb, **o}))
    assert g(dy=0) == 1
    assert g(C=128) == 2
    assert g(dtype=1) == 3
    assert g(dres=MIS) == 4
    assert g(workspace=0) == 5
    assert g(workspace_bytes=1023) == 5
    assert g(dh=FAKE) == 7                                # dh aliases h
    assert g(dg=FAKE + 64) == 7                           # dg aliases dres
    sf = lambda **o: status_of(lambda: attn.attn_swiglu_fwd(
        **{**dict(u=FAKE, out=FAKE + 16, N=2, F=8, dtype=0, stream=0), **o}))
    assert sf(u=0) == 1
    assert sf(F=12) == 2
    assert sf(F=0) == 2
    assert sf(dtype=1) == 3
    assert sf(out=MIS) == 4
    assert sf(out=FAKE) == 7
    sb = lambda **o: status_of(lambda: attn.attn_swiglu_bwd(
        **{**dict(u=FAKE, dout=FAKE + 16, du=FAKE + 32, N=2, F=8, dtype=0, stream=0), **o}))
    assert sb(dout=0) == 1
    assert sb(N=0) == 2
    assert sb(dtype=7) == 3
    assert sb(du=FAKE + 16) == 7


def test_rope_tables_reject_bad_arguments(lib):
    f = lambda **o: status_of(lambda: attn.attn_rope_tables(
        **{**dict(cos_tab=FAKE, sin_tab=FAKE + 16, T=4, D=64, base=10000.0, stream=0), **o}))
    assert f(cos_tab=0) == 1
    assert f(D=63) == 2
    assert f(T=0) == 2
    assert f(base=1.0) == 8
    assert f(base=float("nan")) == 8
    assert f(sin_tab=FAKE) == 7


def test_missing_library_fails_loudly(tmp_path):
    with pytest.raises(RuntimeError, match="missing"):
        _lib.load(str(tmp_path / "libattn.so"))
