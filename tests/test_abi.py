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

# fake, 16-byte aligned, non-null addresses 1 MiB apart (far more than any
# buffer below needs, so they overlap only where a test plants an overlap);
# every call below fails validation before any launch, so none is dereferenced
FAKE = 0x10000000
MIS = FAKE + 4


def A(i, off=0):
    return FAKE + (i << 20) + off

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
    for n in ("attn_fwd", "attn_fwd_save", "attn_fwd_rotated", "attn_rotate_qk",
              "attn_saved_bytes", "attn_bwd", "attn_bwd_saved",
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
    for code in range(11):
        assert attn.attn_status_string(code) != "unknown status"
    assert attn.attn_status_string(99) == "unknown status"
    assert attn.attn_last_hip_error() == 0


def test_workspace_size(lib):
    # per-row entries (two fp32 per row, rounded up to 256), then room for the
    # rotated q and k on the 16-bit path
    assert attn.attn_bwd_workspace_bytes(8, 12, 1024, 64, 0) == 8 * 8 * 12 * 1024 + 4 * 8 * 12 * 1024 * 64
    assert attn.attn_bwd_workspace_bytes(8, 12, 1024, 64, 1) == 4 * 8 * 12 * 1024
    assert attn.attn_bwd_workspace_bytes(1, 1, 3, 64, 0) == 256 + 768
    assert attn.attn_bwd_workspace_bytes(1, 1, 3, 64, 2) == 256 + 768
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


# B=1, H=1, T=8, D=64 bf16: 1 KiB per [B,H,T,D] tensor, 32 B of lse, 1 KiB per
# table, a 2 KiB saved buffer, 256 B of per-row workspace entries
X, ROW, TAB, SAVED, WROWS = 1024, 32, 1024, 2048, 256


def fwd_args(**over):
    a = dict(q=A(0), k=A(1), v=A(2), cos_tab=A(3), sin_tab=A(4), o=A(5), lse=A(6),
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
    assert f(B=1, H=2048, T=8192, D=128) == 2           # exactly 2^31 elements per tensor
    assert f(dtype=3) == 3
    assert f(k=MIS) == 4
    assert f(o=A(0)) == 7                                 # o is q
    assert f(o=A(0, X - 16)) == 7                         # o's first row overlaps q's last bytes
    assert f(lse=A(2, 512)) == 7                          # lse inside v
    assert f(o=A(3, -X + 16)) == 7                        # o's tail runs into the cos table


def test_adjacent_buffers_are_not_aliases(lib):
    # o ends exactly where lse starts and q ends exactly where o starts: no byte is
    # shared, so validation passes the alias check and fails on the next argument
    f = lambda **o: status_of(lambda: attn.attn_fwd_save(**{**fwd_args(), **o}))
    assert f(o=A(0, X), lse=A(0, 2 * X), saved=A(7), saved_bytes=SAVED - 256) == 9


def test_fwd_save_rejects_bad_arguments(lib):
    base = fwd_args(saved=A(7), saved_bytes=SAVED)
    f = lambda **o: status_of(lambda: attn.attn_fwd_save(**{**base, **o}))
    assert f(saved=0) == 1                                # bf16 needs the saved buffer
    assert f(saved=MIS) == 4
    assert f(saved_bytes=SAVED - 1) == 9
    assert f(saved=A(1, 256)) == 7                        # saved overlaps k
    assert f(saved=A(6, -SAVED + 16)) == 7                # saved runs into lse
    assert f(o=A(7, 1008)) == 7                           # o inside saved
    assert f(v=0) == 1


def test_fwd_rotated_and_rotate_reject_bad_arguments(lib):
    f = lambda **o: status_of(lambda: attn.attn_fwd_rotated(
        **{**dict(saved=A(0), saved_bytes=SAVED, v=A(1), o=A(2), lse=A(3),
                  B=1, H=1, T=8, D=64, dtype=0, stream=0), **o}))
    assert f(dtype=1) == 3                                # fp32 has no rotated path
    assert f(saved=0) == 1
    assert f(saved_bytes=100) == 9
    assert f(o=A(0, 1024)) == 7                           # o inside saved
    g = lambda **o: status_of(lambda: attn.attn_rotate_qk(
        **{**dict(q=A(0), k=A(1), cos_tab=A(2), sin_tab=A(3), saved=A(4),
                  saved_bytes=SAVED, B=1, H=1, T=8, D=64, dtype=0, stream=0), **o}))
    assert g(q=0) == 1
    assert g(saved_bytes=0) == 9
    assert g(saved=A(0, 16)) == 7                         # saved overlaps q
    assert g(D=48) == 2


def bwd_base(**over):
    a = dict(q=A(0), k=A(1), v=A(2), o=A(3), dO=A(4), lse=A(5), cos_tab=A(6), sin_tab=A(7),
             dq=A(8), dk=A(9), dv=A(10), workspace=A(11), workspace_bytes=WROWS + SAVED,
             B=1, H=1, T=8, D=64, dtype=0, stream=0)
    a.update(over)
    return a


def test_bwd_rejects_bad_arguments(lib):
    f = lambda **o: status_of(lambda: attn.attn_bwd(**bwd_base(**o)))
    assert f(dO=0) == 1
    assert f(q=0) == 1                                    # attn_bwd reads q and k itself
    assert f(D=100) == 2
    assert f(dtype=-1) == 3
    assert f(dq=MIS) == 4
    assert f(workspace=0) == 5
    assert f(workspace_bytes=WROWS + SAVED - 1) == 5      # room for the rotated q, k too
    assert f(dk=A(0)) == 7
    assert f(dv=A(9, 512)) == 7                           # dv overlaps dk
    assert f(workspace=A(5, 16)) == 7                     # workspace overlaps lse
    assert f(workspace=A(10, X - 256)) == 7               # workspace starts in dv's last row
    assert f(dq=A(11, WROWS + 1024)) == 7                 # dq inside the workspace's q, k part


def test_bwd_saved_rejects_bad_arguments(lib):
    base = bwd_base(saved=A(12), saved_bytes=SAVED, workspace_bytes=WROWS)
    f = lambda **o: status_of(lambda: attn.attn_bwd_saved(**{**base, **o}))
    assert f(saved=0) == 1
    assert f(saved_bytes=8) == 9
    assert f(workspace_bytes=WROWS - 1) == 5              # the per-row part suffices
    assert f(dq=A(12, 64)) == 7                           # dq overlaps saved
    assert f(workspace=A(12, SAVED - 16)) == 7            # workspace overlaps saved's end
    assert f(v=0) == 1
    # the 16-bit path takes the rotated q, k from saved: q and k may be NULL there,
    # and are then required for fp32 (which rotates on load)
    assert f(q=0, k=0, dq=A(8, 1)) == 4                   # got past q, k to dq's alignment
    assert f(q=0, dtype=1, workspace_bytes=256) == 1


def test_bwd_stages_reject_bad_arguments(lib):
    f = lambda **o: status_of(lambda: attn.attn_bwd_prep(
        **{**dict(q=0, k=0, o=A(0), dO=A(1), lse=A(2), cos_tab=0, sin_tab=0, workspace=A(3),
                  workspace_bytes=WROWS, B=1, H=1, T=8, D=64, dtype=0, stream=0), **o}))
    assert f(o=0) == 1
    assert f(lse=0) == 1
    assert f(D=32) == 2
    assert f(dtype=5) == 3
    assert f(dO=MIS) == 4
    assert f(workspace=0) == 5
    assert f(workspace_bytes=WROWS - 1) == 5
    assert f(workspace=MIS) == 4
    assert f(workspace=A(1, 1008)) == 7                   # workspace overlaps dO's last row
    # with q and k the pass also rotates them: the tables are needed, and room for q', k'
    assert f(q=A(4), k=A(5)) == 1                         # no tables
    assert f(q=A(4), k=A(5), cos_tab=A(6), sin_tab=A(7)) == 5
    assert f(q=A(4), k=A(5), cos_tab=A(6), sin_tab=A(7), workspace_bytes=WROWS + SAVED,
             workspace=A(4, 512)) == 7                    # the workspace overlaps q
    assert f(q=A(4), k=0, cos_tab=A(6), sin_tab=A(7), workspace_bytes=WROWS + SAVED) == 1
    base = dict(q=A(0), k=A(1), v=A(2), dO=A(4), lse=A(5), cos_tab=A(6), sin_tab=A(7),
                saved=A(12), saved_bytes=SAVED, dq=A(8), dk=A(9), dv=A(10), workspace=A(11),
                workspace_bytes=WROWS, B=1, H=1, T=8, D=64, dtype=0, stream=0)
    g = lambda **o: status_of(lambda: attn.attn_bwd_grads(**{**base, **o}))
    assert g(dq=0) == 1
    assert g(saved=0) == 5                                # then q', k' come from the workspace
    assert g(saved=0, workspace_bytes=WROWS + SAVED, dq=A(11, WROWS + 64)) == 7
    assert g(saved_bytes=8) == 9
    assert g(workspace=0) == 5
    assert g(dv=A(2)) == 7                                # dv is v
    assert g(dk=A(8, 512)) == 7                           # dk overlaps dq
    assert g(dq=A(11, 128)) == 7                          # dq overlaps the workspace


def test_packed_entry_points_reject_bad_arguments(lib):
    # the packed tensor is 3 KiB here
    fb = dict(qkv=A(0), cos_tab=A(1), sin_tab=A(2), o=A(3), lse=A(4), saved=A(5),
              saved_bytes=SAVED, B=1, H=1, T=8, D=64, dtype=0, stream=0)
    f = lambda **o: status_of(lambda: attn.attn_fwd_packed(**{**fb, **o}))
    assert f(qkv=0) == 1
    assert f(D=96) == 2
    assert f(dtype=1) == 3                                # fp32 has no packed path
    assert f(dtype=7) == 3
    assert f(o=MIS) == 4
    assert f(saved_bytes=16) == 9
    assert f(o=A(0, 2048)) == 7                           # o inside qkv's third kilobyte
    assert f(saved=A(1, 512)) == 7                        # saved overlaps a table
    # the packed tensor (3*B*H*T*D elements) must stay below 2^31 elements
    assert f(B=1, H=16, T=1 << 19, D=128, saved_bytes=1 << 40) == 2   # 3 * 2^30 elements
    assert f(B=1, H=1 << 16, T=1, D=64, saved_bytes=1 << 40) == 2     # a token row of 3 * 2^22
    bb = dict(qkv=A(0), o=A(1), dO=A(2), lse=A(3), cos_tab=A(4), sin_tab=A(5), saved=A(6),
              saved_bytes=SAVED, dqkv=A(7), workspace=A(8), workspace_bytes=WROWS, B=1, H=1,
              T=8, D=64, dtype=0, stream=0)
    g = lambda **o: status_of(lambda: attn.attn_bwd_packed(**{**bb, **o}))
    assert g(dqkv=0) == 1
    assert g(dO=0) == 1
    assert g(dtype=1) == 3
    assert g(T=0) == 2
    assert g(dqkv=MIS) == 4
    assert g(workspace=0) == 5
    assert g(workspace_bytes=WROWS - 1) == 5
    assert g(saved=0) == 5                                # without saved: room for q, k needed
    assert g(saved_bytes=8) == 9
    assert g(dqkv=A(0, 1024)) == 7                        # dqkv overlaps qkv
    assert g(workspace=A(7, 3008)) == 7                   # workspace overlaps dqkv's end
    assert g(dqkv=A(6, 16)) == 7                          # dqkv overlaps saved


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
    assert attn.attn_rmsnorm_bwd_workspace_bytes(8192, 768, 0) == 256 * 768 * 4
    assert attn.attn_rmsnorm_bwd_workspace_bytes(8192, 1024, 0) == 1024 * 1024 * 4
    assert attn.attn_rmsnorm_bwd_workspace_bytes(5, 256, 2) == 1 * 256 * 4
    assert attn.attn_rmsnorm_bwd_workspace_bytes(33, 512, 0) == 3 * 512 * 4
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


def _readme_blocks(lang):
    readme = os.path.join(os.path.dirname(HEADER), os.pardir, "README.md")
    return re.findall(r"```" + lang + r"\n(.*?)```", open(readme).read(), re.S)


def test_readme_examples_compile(tmp_path):
    """The usage examples stay in step with the header and the binding: the C one
    compiles against include/attn.h with warnings as errors, and the Python one
    parses and names only functions the binding has."""
    import ast
    import shutil
    import subprocess
    (c_src,) = _readme_blocks("c")
    (py_src,) = _readme_blocks("python")
    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        pytest.skip("no C compiler")
    src = tmp_path / "example.c"
    src.write_text(c_src)
    r = subprocess.run([cc, "-std=c99", "-Wall", "-Wextra", "-Werror", "-c",
                        "-I", os.path.dirname(HEADER), str(src), "-o", str(tmp_path / "e.o")],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    tree = ast.parse(py_src)
    used = {n.attr for n in ast.walk(tree)
            if isinstance(n, ast.Attribute) and isinstance(n.value, ast.Name)
            and n.value.id == "attn"}
    assert used and all(hasattr(attn, a) for a in used), used
