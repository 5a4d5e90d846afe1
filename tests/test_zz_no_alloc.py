"""attn_bwd_saved_noalloc, the backward that allocates nothing (its per-row
entries live in the library's static device array), against attn_bwd_saved with
a caller workspace: bitwise the same gradients, on two calls in a row (the
second on a smaller problem, over the array the first one left behind); and the
training pair built on it captured into a HIP graph and replayed."""

import pytest

import workloads

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import causal_attention_attn_amd as attn
    from tests.gpu_util import assert_close, oracle_run


@pytest.fixture(scope="module", autouse=True)
def need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    attn.load()


def both(x, dtype_code):
    """(gradients from attn_bwd_saved with a workspace, from attn_bwd_saved_noalloc)"""
    dev = torch.device("cuda", 0)
    g = {n: t.to(dev) for n, t in x.items()}
    q, k, v, do = g["q"], g["k"], g["v"], g["do"]
    B, H, T, D = q.shape
    cs, sn = attn.rope_tables(T, D, 10000.0, dev)
    o, lse, saved = attn.forward(q, k, v)
    ns = saved.numel() if saved is not None else 0
    nw = attn.attn_bwd_workspace_bytes(B, H, T, D, dtype_code)
    ws = torch.empty(nw, dtype=torch.uint8, device=dev)
    ref = [torch.empty_like(q) for _ in range(3)]
    got = [torch.full_like(q, float("nan")) for _ in range(3)]
    attn.attn_bwd_saved(q, k, v, o, do, lse, cs, sn, saved, ns, *ref, ws, nw, B, H, T, D,
                        dtype_code)
    attn.attn_bwd_saved_noalloc(q, k, v, o, do, lse, cs, sn, saved, ns, *got, B, H, T, D,
                                dtype_code)
    torch.cuda.synchronize()
    return ref, got, dict(o=o.cpu(), lse=lse.cpu())


@pytest.mark.parametrize("dtype,code", [("bf16", 0), ("f16", 2)])
def test_noalloc_backward_matches_workspace_backward(dtype, code):
    w = workloads.WORKLOADS[workloads.HEADLINE if dtype == "bf16" else "gpt2s_f16_b8h12t1024d64"]
    for shape in ((2, 3, 700, 64), (1, 2, 130, 64), (1, 1, 257, 128)):  # the later calls smaller
        x = workloads.make(w, seed=sum(shape), shape=shape)
        ref, got, fo = both(x, code)
        for a, b, n in zip(ref, got, ("dq", "dk", "dv")):
            assert torch.equal(a, b), (shape, n)
        out = dict(fo, dq=got[0].cpu(), dk=got[1].cpu(), dv=got[2].cpu())
        assert_close(out, oracle_run(x), dtype, f"noalloc {dtype} {shape}")


def test_noalloc_backward_fp32():
    x = workloads.make(workloads.WORKLOADS[workloads.TINY], seed=4)
    ref, got, _ = both(x, 1)
    for a, b in zip(ref, got):
        assert torch.equal(a, b)


def test_noalloc_rejects_problems_beyond_its_scratch():
    assert attn.attn_noalloc_scratch_bytes() == 4 << 20
    dev = torch.device("cuda", 0)
    t = torch.zeros(16, dtype=torch.uint8, device=dev)
    # 8 bytes per row on the 16-bit path: 524288 rows fit, 524289 do not; the
    # size is checked before anything is launched or touched
    B, H, T, D = 1, 1, 524289, 64
    ns = attn.attn_saved_bytes(B, H, T, D, 0)
    with pytest.raises(attn.AttnError) as e:
        attn.attn_bwd_saved_noalloc(t, t, t, t, t, t, t, t, t, ns, t, t, t, B, H, T, D, 0)
    assert e.value.status == 10


def test_noalloc_training_pair_in_a_hip_graph():
    """The training pair with nothing allocated inside it (attn_fwd_save into caller
    buffers, then attn_bwd_saved_noalloc) captured into a HIP graph, the use these
    entry points serve. Every replay, with eager launches and synchronisations
    between the replays, gives bitwise the eager outputs; after an input changes in
    place, a replay gives bitwise the new eager outputs (the graph reads its inputs
    when it runs). Only the library's kernel launches are captured."""
    w = workloads.WORKLOADS[workloads.HEADLINE]
    B, H, T, D = 2, 3, 700, 64
    x = workloads.make(w, seed=11, shape=(B, H, T, D))
    dev = torch.device("cuda", 0)
    g = {n: t.to(dev) for n, t in x.items()}
    q, k, v, do = g["q"], g["k"], g["v"], g["do"]
    cs, sn = attn.rope_tables(T, D, 10000.0, dev)
    ns = attn.attn_saved_bytes(B, H, T, D, 0)
    saved = torch.empty(ns, dtype=torch.uint8, device=dev)
    o = torch.empty_like(q)
    lse = torch.empty((B, H, T), dtype=torch.float32, device=dev)
    dq, dk, dv = (torch.empty_like(q) for _ in range(3))
    outs = (o, lse, dq, dk, dv)
    names = ("o", "lse", "dq", "dk", "dv")

    def step():
        attn.attn_fwd_save(q, k, v, cs, sn, o, lse, saved, ns, B, H, T, D, 0)
        attn.attn_bwd_saved_noalloc(q, k, v, o, do, lse, cs, sn, saved, ns, dq, dk, dv,
                                    B, H, T, D, 0)

    def spoil():
        # eager work between replays: a fill kernel over every output
        for t in outs:
            t.fill_(float("nan"))
        torch.cuda.synchronize()

    step()  # eager warm-up: the scratch address and the CU count are looked up here
    torch.cuda.synchronize()
    ref = [t.clone() for t in outs]
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    torch.cuda.synchronize()
    for r in range(4):
        spoil()
        graph.replay()
        torch.cuda.synchronize()
        for a, b, n in zip(outs, ref, names):
            assert torch.equal(a, b), (r, n)
    v.mul_(0.5)
    step()
    torch.cuda.synchronize()
    ref2 = [t.clone() for t in outs]
    assert not torch.equal(ref2[0], ref[0])
    for r in range(2):
        spoil()
        graph.replay()
        torch.cuda.synchronize()
        for a, b, n in zip(outs, ref2, names):
            assert torch.equal(a, b), ("after the input changed", r, n)
