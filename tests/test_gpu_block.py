"""The Llama MLP block and the q/k/v projections around the layer on the GPU, through the
C ABI: the fused SiLU(gate) * up + quantization kernel, the block's four launches, the
three projections packed as one layer, and their HIP-graph replays.

Each step is compared with the oracle applied to the GPU's own input of that step (the
steps round to fp16 in between, so this is how a pipeline's parity is checked):
* mixllm_silu_mul_quant: h within 1 fp16 ulp of the fp64 definition (the GPU evaluates
  SiLU in fp32 with the library exp), and the int8 codes, scales, code sums and row
  operands bit-exact to quantizing that h;
* the gate/up GEMM and the down GEMM: within the layer tolerance;
* graph replays: bit-identical to the eager forward pass, with other work between replays.
"""
import numpy as np
import pytest

from tests import gpu_util as U
from weight_activation_quantized_amd import workloads as WL

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def L():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a GPU")
    from weight_activation_quantized_amd import mixllm
    return mixllm


def _check_h_and_codes(h_gpu, ref_h, aq, sa, asum, ro):
    import oracle as O
    d = np.abs(h_gpu.astype(np.float64) - ref_h.astype(np.float64))
    assert np.all(d <= O.ulp_fp16(ref_h)), "h off by more than one fp16 ulp"
    assert (d == 0).mean() >= 0.999, "h differs from the definition too often"
    oq, osa, osum = O.quant_act(h_gpu)
    assert np.array_equal(aq, oq)
    assert np.array_equal(sa.T.view(np.uint32), osa.view(np.uint32))
    assert np.array_equal(asum.T, osum)
    assert np.array_equal(ro, U.rowop_records(osa.T, osum.T.astype(np.float32) * osa.T))


@pytest.mark.parametrize("m,inter,ld_extra", [(16, 512, 0), (33, 1408, 8), (130, 384, 384), (1, 128, 0)])
def test_silu_mul_quant(L, m, inter, ld_extra):
    import oracle as O
    g16 = WL.make_acts(m, inter, (21, m, inter))
    u16 = WL.make_acts(m, inter, (22, m, inter))
    U.say("silu_mul_quant", m, inter, ld_extra)
    buf = torch.zeros((m, 2 * inter + ld_extra), dtype=torch.float16, device="cuda")
    buf[:, :inter] = torch.from_numpy(g16).cuda()
    buf[:, inter:2 * inter] = torch.from_numpy(u16).cuda()
    gi = inter // 128
    aq = torch.empty((m, inter), dtype=torch.int8, device="cuda")
    sa = torch.empty((gi, m), dtype=torch.float32, device="cuda")
    asum = torch.empty((gi, m), dtype=torch.int32, device="cuda")
    ro = L.rowop_buffer(m, inter)
    h = torch.empty((m, inter), dtype=torch.float16, device="cuda")
    L.mixllm_silu_mul_quant(buf[:, :inter], buf[:, inter:2 * inter], aq, sa, asum, ro, h)
    torch.cuda.synchronize()
    _check_h_and_codes(h.cpu().numpy(), O.silu_mul_fp16(g16, u16), aq.cpu().numpy(), sa.cpu().numpy(),
                       asum.cpu().numpy(), ro.cpu().numpy().view(np.uint32))


def _block(L, m, hidden, inter, n8, seed):
    x16, wg, wu, wd, ig, iu, idn = WL.mlp_block_inputs(m, hidden, inter, n8, seed)
    blk = L.MLPBlock(wg, wu, wd, ig, iu, idn)
    return (x16, wg, wu, wd, ig, iu, idn), blk


@pytest.mark.parametrize("m,hidden,inter,n8,rows", [
    (65, 256, 384, dict(gate=3, up=40, down=130), None),
    (130, 512, 1408, dict(gate=10, up=141, down=276), None),
    (512, 4096, 14336, WL.llama8b_n8(), 12),
    # decode and small batches at the full block size: the gemv and strip kernels for the
    # gate/up layer (28672 channels), the skinny kernel for the down projection
    (1, 4096, 14336, WL.llama8b_n8(), None),
    (4, 4096, 14336, WL.llama8b_n8(), None),
])
def test_mlp_block_chain(L, m, hidden, inter, n8, rows):
    import oracle as O
    (x16, wg, wu, wd, ig, iu, idn), blk = _block(L, m, hidden, inter, n8, (31,))
    U.say("mlp block", m, hidden, inter)
    x = torch.from_numpy(x16).cuda()
    bufs = blk.buffers(m)
    y = blk.forward(x, bufs, keep_h=True)
    torch.cuda.synchronize()
    rs = np.arange(m) if rows is None else U.sample_rows(m, np.random.default_rng(5), rows)
    gu = bufs["x"]["y"].cpu().numpy()[rs]
    h = bufs["h16"].cpu().numpy()[rs]
    yg = y.cpu().numpy()[rs]
    w_gu = np.concatenate([wg, wu])
    idx_gu = np.concatenate([ig, iu + inter])
    ref_gu = U.oracle_at(x16[rs], w_gu, idx_gu)
    U.assert_y_close(gu, ref_gu["y16"], "gate/up")
    bh = bufs["h"]
    _check_h_and_codes(h, O.silu_mul_fp16(gu[:, :inter], gu[:, inter:]), bh["aq"].cpu().numpy()[rs],
                       bh["sa"].cpu().numpy()[:, rs], bh["asum"].cpu().numpy()[:, rs],
                       bh["rowop"].cpu().numpy().view(np.uint32)[:, rs])
    ref_dn = U.oracle_at(h, wd, idn)
    U.assert_y_close(yg, ref_dn["y16"], "down")


@pytest.mark.parametrize("m", [130, 1])
def test_mlp_block_graph_replays(L, m):
    (x16, *_), blk = _block(L, m, 512, 1408, dict(gate=10, up=141, down=276), (32,))
    x = torch.from_numpy(x16).cuda()
    U.say("mlp block graph", m)
    eager_bufs = blk.buffers(m)
    want = blk.forward(x, eager_bufs).clone()
    torch.cuda.synchronize()
    bufs = blk.buffers(m)
    graph = blk.capture(x, bufs)
    other = torch.randn(1 << 20, device="cuda")
    for i in range(4):
        bufs["h"]["y"].fill_(float("nan"))
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(bufs["h"]["y"], want), f"replay {i}"
        other.mul_(1.0001).add_(1.0)              # eager work between replays
        blk.forward(x, eager_bufs)                # and an eager pass on other buffers
        torch.cuda.synchronize()
        assert torch.equal(eager_bufs["h"]["y"], want)


@pytest.mark.parametrize("m,rows", [(1, None), (16, None), (130, None), (512, 12)])
def test_qkv_projection(L, m, rows):
    """Llama-3.1-8B q, k, v over one hidden state: one quant_act, one GEMM over the packed
    6144 channels; each projection within the layer tolerance of the oracle applied to it
    alone."""
    n8 = WL.llama8b_n8()
    x16, wq, wk, wv, iq, ik, iv = WL.qkv_inputs(m, WL.QKV8B["hidden"], WL.QKV8B["q"], WL.QKV8B["kv"], n8)
    U.say("qkv projection", m)
    proj = L.QKVProjection(wq, wk, wv, iq, ik, iv)
    bufs = proj.buffers(m)
    q, k, v = proj.forward(torch.from_numpy(x16).cuda(), bufs)
    torch.cuda.synchronize()
    assert q.shape == (m, 4096) and k.shape == (m, 1024) and v.shape == (m, 1024)
    rs = np.arange(m) if rows is None else U.sample_rows(m, np.random.default_rng(7), rows)
    for name, out, w, idx in (("q", q, wq, iq), ("k", k, wk, ik), ("v", v, wv, iv)):
        ref = U.oracle_at(x16[rs], w, idx)
        U.assert_y_close(out.cpu().numpy()[rs], ref["y16"], name)


def test_qkv_graph_replays(L):
    n8 = dict(q=22, k=5, v=73)
    m = 40
    x16, wq, wk, wv, iq, ik, iv = WL.qkv_inputs(m, 512, 512, 128, n8, (33,))
    proj = L.QKVProjection(wq, wk, wv, iq, ik, iv)
    x = torch.from_numpy(x16).cuda()
    U.say("qkv graph", m)
    eager_bufs = proj.buffers(m)
    want = torch.cat(proj.forward(x, eager_bufs), dim=1).clone()
    torch.cuda.synchronize()
    bufs = proj.buffers(m)
    graph = proj.capture(x, bufs)
    other = torch.randn(1 << 20, device="cuda")
    for i in range(4):
        bufs["y"].fill_(float("nan"))
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(bufs["y"], want), f"replay {i}"
        other.mul_(1.0001).add_(1.0)
        proj.forward(x, eager_bufs)
        torch.cuda.synchronize()
        assert torch.equal(eager_bufs["y"], want)


def test_graph_of_chained_steps(L):
    """Several steps (each on its own buffers) captured in sequence as one graph: every
    step's output equals its eager forward pass, on every replay."""
    n8 = dict(q=22, k=5, v=73)
    m = 24
    x16, wq, wk, wv, iq, ik, iv = WL.qkv_inputs(m, 512, 512, 128, n8, (34,))
    projs = [L.QKVProjection(wq, wk, wv, iq, ik, iv) for _ in range(3)]
    xs = [torch.from_numpy(x16).cuda() * (1 + j) for j in range(3)]
    U.say("graph chain", m)
    want = []
    for pj, x in zip(projs, xs):
        want.append(torch.cat(pj.forward(x, pj.buffers(m)), dim=1).clone())
    torch.cuda.synchronize()
    bufs = [pj.buffers(m) for pj in projs]
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        for pj, x, b in zip(projs, xs, bufs):
            pj.forward(x, b, s)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        for pj, x, b in zip(projs, xs, bufs):
            pj.forward(x, b, s)
    for r in range(3):
        for b in bufs:
            b["y"].fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        for j, b in enumerate(bufs):
            assert torch.equal(b["y"], want[j]), f"replay {r} step {j}"
