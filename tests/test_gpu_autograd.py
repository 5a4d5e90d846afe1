"""The autograd wrappers (attention, attention_packed): the library's forward and
backward as one differentiable torch op. Their outputs and gradients are bitwise
those of forward()/backward() (forward_packed()/backward_packed()) on the same
values, and within the parity bar of the oracle inside a larger torch graph."""

import pytest

import workloads

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import causal_attention_attn_amd as attn
    from tests.gpu_util import assert_close, oracle_run, to_packed


@pytest.fixture(scope="module", autouse=True)
def need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    attn.load()


DEV = torch.device("cuda", 0)
NAMES = {"bf16": workloads.HEADLINE, "f16": "gpt2s_f16_b8h12t1024d64", "f32": workloads.TINY}


@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
@pytest.mark.parametrize("B,H,T,D", [(1, 2, 1, 64), (2, 3, 200, 64), (1, 2, 130, 128)])
def test_attention_matches_the_paired_calls(B, H, T, D, dtype):
    x = workloads.make(workloads.WORKLOADS[NAMES[dtype]], seed=B + H + T + D, shape=(B, H, T, D))
    g = {n: t.to(DEV) for n, t in x.items()}
    q, k, v = (g[n].clone().requires_grad_() for n in ("q", "k", "v"))
    o = attn.attention(q, k, v)
    o.backward(g["do"])
    o2, lse2, saved2 = attn.forward(g["q"], g["k"], g["v"])
    dq2, dk2, dv2 = attn.backward(g["q"], g["k"], g["v"], o2, g["do"], lse2, saved2)
    assert torch.equal(o.detach(), o2)
    for got, ref, n in ((q.grad, dq2, "dq"), (k.grad, dk2, "dk"), (v.grad, dv2, "dv")):
        assert torch.equal(got, ref), n


def test_attention_packed_matches_the_paired_calls():
    x = workloads.make(workloads.WORKLOADS[workloads.HEADLINE], seed=9, shape=(2, 3, 150, 64))
    qkv, do = to_packed(x, DEV)
    qkv_g = qkv.clone().requires_grad_()
    o = attn.attention_packed(qkv_g)
    o.backward(do)
    o2, lse2, saved2 = attn.forward_packed(qkv)
    dqkv2 = attn.backward_packed(qkv, o2, do, lse2, saved2)
    assert torch.equal(o.detach(), o2)
    assert torch.equal(qkv_g.grad, dqkv2)


def test_attention_inside_a_torch_graph():
    """loss = sum(attention(2a, k, 4c) * w), with the scalings done by torch:
    autograd chains through the op, and a.grad / 2, k.grad and c.grad / 4 meet the
    parity bar against the oracle's dq, dk and dv for dO = w (the scalings are
    exact in bf16, so q = 2a and v = 4c are the workload's own values)."""
    x = workloads.make(workloads.WORKLOADS[workloads.HEADLINE], seed=21, shape=(1, 2, 96, 64))
    g = {n: t.to(DEV) for n, t in x.items()}
    a = (g["q"] / 2).requires_grad_()
    k = g["k"].clone().requires_grad_()
    c = (g["v"] / 4).requires_grad_()
    q, v = a * 2, c * 4
    assert torch.equal(q, g["q"]) and torch.equal(v, g["v"])
    o = attn.attention(q, k, v)
    loss = (o.float() * g["do"].float()).sum()
    loss.backward()
    _, lse, _ = attn.forward(g["q"], g["k"], g["v"], save=False)
    got = dict(o=o.detach().cpu(), lse=lse.cpu(), dq=(a.grad / 2).cpu(), dk=k.grad.cpu(),
               dv=(c.grad / 4).cpu())
    assert_close(got, oracle_run(x), "bf16", "attention inside a torch graph")
