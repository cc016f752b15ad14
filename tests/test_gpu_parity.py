"""GPU parity of the HIP path against the CPU oracle, through the C ABI.

Bit-exact: int8 activation codes, fp32 activation scales, code sums, the bf16 row
operands of the scale products, int32 group partials.  Within tolerance (2 fp16 ulp of the oracle value + 1e-3 max|Y|): the fp16
layer output.  Small shapes compare every element; the five workloads at their full
sizes compare sampled rows x columns (the oracle computes exactly those) and a window
of group partials.
"""
import zlib

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


def _dev(x):
    return torch.from_numpy(np.ascontiguousarray(x)).cuda()


def _quant(L, a16, lda_pad=0, with_sum=True):
    m, k = a16.shape
    if lda_pad:
        big = np.zeros((m, k + lda_pad), np.float16)
        big[:, :k] = a16
        a = _dev(big)[:, :k]
    else:
        a = _dev(a16)
    aq = torch.empty((m, k), dtype=torch.int8, device="cuda")
    sa = torch.empty((k // 128, m), dtype=torch.float32, device="cuda")
    asum = torch.empty((k // 128, m), dtype=torch.int32, device="cuda") if with_sum else None
    rowop = L.rowop_buffer(m, k)
    L.mixllm_quant_act(a, aq, sa, asum, rowop)
    return aq, sa, asum, rowop


# --------------------------------------------------------------------------- quant_act

QA_SHAPES = [(16, 1024, "normal"), (1, 128, "normal"), (17, 384, "normal"), (512, 4096, "normal"),
             (1, 4096, "normal"), (100, 14336, "normal"), (33, 28672, "t3"), (2048, 8192, "t3")]


@pytest.mark.parametrize("m,k,dist", QA_SHAPES)
def test_quant_act_bitexact(L, m, k, dist):
    import oracle as O
    a16 = WL.make_acts(m, k, (7, m, k), dist)
    if m > 2:
        a16[1, :128] = 0  # an all-zero group
    U.say("quant_act", m, k, dist)
    aq, sa, asum, rowop = _quant(L, a16, lda_pad=8 if m % 2 else 0)
    torch.cuda.synchronize()
    oq, osa, osum = O.quant_act(a16)
    assert np.array_equal(aq.cpu().numpy(), oq)
    assert np.array_equal(sa.cpu().numpy().T.view(np.uint32), osa.view(np.uint32))
    assert np.array_equal(asum.cpu().numpy().T, osum)
    # row operand records of s_a and fp32(S_A * s_a)
    ro = rowop.cpu().numpy().view(np.uint32)
    assert np.array_equal(ro, U.rowop_records(osa.T, osum.T.astype(np.float32) * osa.T))


def test_quant_act_golden_ties(L):
    """The hand-derived tie examples of tests/golden/quant_examples.json on the GPU."""
    from tests import pins
    gold = pins.load_golden("quant_examples.json")
    rows = [pins._group_vec(ex) for ex in gold["activation"]]
    a16 = np.stack(rows).astype(np.float16)
    U.say("quant_act golden")
    aq, sa, asum, _ = _quant(L, a16)
    torch.cuda.synchronize()
    for i, ex in enumerate(gold["activation"]):
        assert float(sa[0, i].item()) == ex["scale"]
        assert np.array_equal(aq[i].cpu().numpy().astype(np.int64), pins._codes(ex))
        assert int(asum[0, i].item()) == ex["code_sum"]


# --------------------------------------------------------------------------- GEMM, full compare

SMALL = [
    # (M, N, K, n8) -- config 0 and edge shapes: ragged M and N, empty subsets, K = 128,
    # n4 a multiple of 32 (no shared block), a single channel
    (16, 512, 1024, 52), (1, 512, 1024, 52), (4, 100, 256, 7), (17, 96, 384, 0), (31, 96, 384, 96),
    (33, 160, 256, 64), (64, 64, 128, 1), (65, 200, 512, 31), (100, 72, 256, 8), (130, 300, 384, 30),
    (1, 1, 128, 0), (3, 1, 128, 1), (256, 520, 640, 52), (200, 33, 256, 32),
    # tile kernel: slices with an odd step count, the LDS stage ring wrapping several times
    # (these narrow layers take two-block tiles); four-block tiles need a grid as large as
    # the device: a ragged last M tile
    (160, 288, 1920, 40), (96, 130, 2688, 13), (4150, 1024, 128, 100),
    # more 8-bit blocks than N tiles: consecutive blocks per tile, tiles of both kinds
    # (two-block and four-block tiles; the cases above interleave the blocks over the tiles)
    (160, 640, 512, 400), (4150, 1024, 128, 700),
    # M <= 64 on layers wide enough (on a 256-CU part) for the tile kernel's cost rule
    (48, 12800, 256, 1280), (20, 16448, 128, 100), (1, 29000, 128, 290),
    # M = 1 .. 3 on layers wide enough for the one-lane-per-channel kernel, and 4 .. 16 for
    # the strip kernel: an odd or even number of 4-bit blocks, promoted 4-bit channels,
    # several groups per wave and a ragged tail, or only the tail; ragged M
    (1, 16448, 8960, 1608), (2, 16448, 8960, 1608), (3, 16448, 2688, 1640), (4, 16448, 8960, 1608),
    (9, 16448, 4480, 1608), (16, 16448, 1152, 1640),
    # the strip kernel with one 4-bit block per strip (layers with 3/4 as many blocks as CUs),
    # and with two 16-row blocks (17 <= M <= 32)
    (8, 8192, 2688, 820), (13, 6400, 1152, 640), (24, 16448, 2688, 1608), (32, 8192, 1152, 820),
    # M = 1 .. 3 on a layer with fewer 4-bit block pairs than CUs (on 256 CUs): one 4-bit
    # block per strip, the group's inputs split over the half-waves; an odd block count
    (1, 8192, 2688, 820), (2, 8192, 1152, 820), (3, 8192, 896, 820),
    # the one-lane-per-channel kernel with one-block strips on the headline's width and a
    # ragged last block (4100); the strip kernel with one-block strips whose 8-bit blocks
    # go in 16-channel halves (every strip fits a CU), one and two row blocks, and a last
    # 8-bit block whose second half holds no channel (6150 = 192 * 32 + 6)
    (1, 4096, 640, 410), (2, 4096, 256, 410), (3, 4100, 384, 411),
    (8, 6150, 1280, 615), (13, 6400, 1152, 640), (24, 6400, 640, 650),
]


def _run_gemm(L, a16, w16, idx8, ldy_pad=0):
    m, k = a16.shape
    n = w16.shape[0]
    blob = L.DeviceBlob(L.mixllm_pack_weights(w16, idx8))
    aq, sa, asum, rowop = _quant(L, a16)
    y = torch.full((m, n + ldy_pad), float("nan"), dtype=torch.float16, device="cuda")
    assert L.mixllm_gemm_workspace_bytes(m, n, k, len(idx8)) == 0
    L.mixllm_gemm_w4w8a8(aq, sa, asum, rowop, m, n, k, len(idx8), blob, y)
    return blob, (aq, sa, asum, rowop), y


@pytest.mark.parametrize("m,n,k,n8", SMALL)
def test_gemm_full_compare(L, m, n, k, n8):
    sh = WL.Shape(0, "edge", m, n, k, n8)
    a16, w16, idx8 = WL.make_layer_inputs(sh)
    U.say("gemm full", sh.name)
    blob, qa, y = _run_gemm(L, a16, w16, idx8, ldy_pad=5)
    torch.cuda.synchronize()
    ref = U.oracle_at(a16, w16, idx8)
    yg = y.cpu().numpy()
    assert np.all(np.isnan(yg[:, n:].astype(np.float32))), "wrote outside [0, N)"
    U.assert_y_close(yg[:, :n], ref["y16"], sh.name)
    # int32 group partials over every channel, bit-exact
    g = k // 128
    part = torch.zeros((m, n, g), dtype=torch.int32, device="cuda")
    U.say("gemm partials", sh.name)
    L.mixllm_gemm_w4w8a8_partials(*qa, m, n, k, n8, blob, 0, n, part)
    torch.cuda.synchronize()
    assert np.array_equal(part.cpu().numpy().astype(np.int64), U.partials_at(ref))


@pytest.mark.parametrize("m,n,k,n8,ldy_pad", [(130, 96, 256, 0, 0), (100, 200, 384, 200, 0), (65, 4100, 256, 0, 4),
                                              (129, 136, 512, 136, 8), (70, 100, 128, 0, 4), (80, 64, 256, 64, 3),
                                              (1, 4096, 1024, 0, 0), (2, 4096, 512, 4096, 0), (3, 8192, 384, 0, 8)])
def test_gemm_pure_paths(L, m, n, k, n8, ldy_pad):
    """All channels 4-bit (p0) or all 8-bit (p100): no scatter, 16-byte output stores when
    the output rows allow them (row stride a multiple of 8), including a partial last run
    of channels; a row stride that does not allow them takes the scatter path.  The M <= 3
    cases run the one-lane-per-channel kernel (on 256 CUs: one-block 4-bit strips, 8-bit
    blocks only)."""
    sh = WL.Shape(0, "edge", m, n, k, n8)
    a16, w16, idx8 = WL.make_layer_inputs(sh)
    U.say("gemm pure", sh.name, "ldy", n + ldy_pad)
    blob, qa, y = _run_gemm(L, a16, w16, idx8, ldy_pad=ldy_pad)
    torch.cuda.synchronize()
    ref = U.oracle_at(a16, w16, idx8)
    yg = y.cpu().numpy()
    assert np.all(np.isnan(yg[:, n:].astype(np.float32))), "wrote outside [0, N)"
    U.assert_y_close(yg[:, :n], ref["y16"], sh.name)


@pytest.mark.parametrize("m,n,k,n8", [(128, 256, 1024, 26), (512, 4096, 4096, 410), (65, 4100, 256, 500),
                                    (192, 384, 128, 40)])
def test_gemm_repeat_deterministic(L, m, n, k, n8):
    """Repeated calls give bit-identical outputs (the group slices of a tile are summed in a
    fixed order); one group per channel (K = 128) leaves some slices empty."""
    sh = WL.Shape(0, "edge", m, n, k, n8)
    a16, w16, idx8 = WL.make_layer_inputs(sh)
    U.say("gemm repeat", sh.name)
    blob = L.DeviceBlob(L.mixllm_pack_weights(w16, idx8))
    qa = _quant(L, a16)
    ys = []
    for _ in range(3):
        y = torch.empty((m, n), dtype=torch.float16, device="cuda")
        L.mixllm_gemm_w4w8a8(*qa, m, n, k, n8, blob, y)
        torch.cuda.synchronize()
        ys.append(y.cpu().numpy())
    assert all(np.array_equal(ys[0].view(np.uint16), y.view(np.uint16)) for y in ys[1:])
    if m * n * k <= 2 ** 24:
        U.assert_y_close(ys[0], U.oracle_at(a16, w16, idx8)["y16"], sh.name)


def test_gemm_golden_tiny(L):
    """The hand-derived M=1, N=2 example of tests/golden/quant_examples.json."""
    from tests import pins
    gold = pins.load_golden("quant_examples.json")
    t = gold["tiny_gemm"]
    a16 = np.zeros((1, 128), np.float16)
    a16[0, 0] = 127.0
    w8 = next(e for e in gold["weight8"] if e["name"] == "ties_scale_2^-8")
    w4 = next(e for e in gold["weight4"] if e["name"] == "mixed_sign_ties")
    w16 = np.stack([pins._group_vec(w8), pins._group_vec(w4)]).astype(np.float16)
    U.say("gemm golden tiny")
    blob, qa, y = _run_gemm(L, a16, w16, np.array(t["idx8"], np.int32))
    part = torch.zeros((1, 2, 1), dtype=torch.int32, device="cuda")
    L.mixllm_gemm_w4w8a8_partials(*qa, 1, 2, 128, 1, blob, 0, 2, part)
    torch.cuda.synchronize()
    assert [float(v) for v in y[0].cpu().numpy()] == t["y16"]
    assert [int(v) for v in part[0, :, 0].cpu().numpy()] == t["partials"]


def test_gemm_m_zero_and_errors(L):
    sh = WL.Shape(0, "edge", 4, 64, 256, 3)
    a16, w16, idx8 = WL.make_layer_inputs(sh)
    blob_host = L.mixllm_pack_weights(w16, idx8)
    blob = L.DeviceBlob(blob_host)
    aq, sa, asum, rowop = _quant(L, a16)
    y = torch.zeros((4, 64), dtype=torch.float16, device="cuda")
    L.mixllm_gemm_w4w8a8(aq, sa, asum, rowop, 0, 64, 256, 3, blob, y)
    short = L.DeviceBlob(blob_host)
    short.nbytes -= 1
    with pytest.raises(L.MixLLMError) as e:
        L.mixllm_gemm_w4w8a8(aq, sa, asum, rowop, 4, 64, 256, 3, short, y)
    assert e.value.status == -5
    # a blob packed for another 8-bit count: refused by its header, nothing launched
    w_o, i_o = WL.make_layer_weights(WL.Shape(0, "edge", 4, 64, 256, 0))
    other = L.DeviceBlob(L.mixllm_pack_weights(w_o, i_o))
    with pytest.raises(L.MixLLMError) as e:
        L.mixllm_gemm_w4w8a8(aq, sa, asum, rowop, 4, 64, 256, 3, other, y)
    assert e.value.status == -6
    with pytest.raises(ValueError):
        L.mixllm_gemm_w4w8a8(aq, sa, None, rowop, 4, 64, 256, 3, blob, y)
    with pytest.raises(ValueError):
        L.mixllm_gemm_w4w8a8(aq, sa, asum, None, 4, 64, 256, 3, blob, y)
    with pytest.raises(ValueError):
        L.mixllm_gemm_w4w8a8(aq, sa, asum, rowop, 4, 64, 256, 3, blob, y[:, :32])   # too few columns
    with pytest.raises(ValueError):
        L.mixllm_gemm_w4w8a8(aq, sa, asum, rowop, 4, 64, 256, 3, blob, y.cpu())    # not on the GPU
    with pytest.raises(ValueError):
        L.mixllm_gemm_w4w8a8(aq, sa, asum, rowop, 4, 64, 256, 3, blob.dev, y)      # no host header
    torch.cuda.synchronize()
    assert float(y.abs().max()) == 0.0


# --------------------------------------------------------------------------- the five workloads at full size

def _layers():
    seen = {}
    for cfg in range(5):
        for sh in WL.config_shapes(cfg):
            seen.setdefault((cfg, sh.layer, sh.n, sh.k, sh.n8, sh.dist), []).append(sh.m)
    return sorted(seen.items())


@pytest.mark.parametrize("key,ms", _layers(), ids=lambda v: "-".join(map(str, v)) if isinstance(v, tuple) else None)
def test_gemm_workloads_sampled(L, key, ms):
    cfg, layer, n, k, n8, dist = key
    rng = np.random.default_rng(zlib.crc32(repr(key).encode()))
    sh0 = WL.Shape(cfg, layer, ms[0], n, k, n8, dist)
    w16, idx8 = WL.make_layer_weights(sh0)
    U.say("pack", sh0.name)
    blob_host = L.mixllm_pack_weights(w16, idx8)
    blob = L.DeviceBlob(blob_host)
    cols = U.sample_cols(n, idx8, rng)
    # packed codes of the sampled channels against the oracle quantizers
    q, z, s16, is8 = L.mixllm_unpack_weights(blob_host)
    for m in ms:
        sh = WL.Shape(cfg, layer, m, n, k, n8, dist)
        a16 = WL.make_acts(m, k, sh.seed, dist)
        rows = U.sample_rows(m, rng)
        U.say("gemm sampled", sh.name)
        qa = _quant(L, a16)
        aq = qa[0]
        y = torch.empty((m, n), dtype=torch.float16, device="cuda")
        L.mixllm_gemm_w4w8a8(*qa, m, n, k, n8, blob, y)
        win = int(rng.integers(0, n - 48)) if n > 48 else 0
        cnt = min(48, n - win)
        part = torch.zeros((m, cnt, k // 128), dtype=torch.int32, device="cuda")
        L.mixllm_gemm_w4w8a8_partials(*qa, m, n, k, n8, blob, win, cnt, part)
        torch.cuda.synchronize()
        ref = U.oracle_at(a16, w16, idx8, rows, cols)
        if m == ms[0]:
            assert np.array_equal(q[cols], (ref["q"].astype(np.int16) & 0xFF).astype(np.uint8))
            assert np.array_equal(z[cols], ref["z"])
            assert np.array_equal(s16[cols].view(np.uint16), ref["s16"].view(np.uint16))
        assert np.array_equal(aq.cpu().numpy()[rows], ref["aq"])
        U.assert_y_close(y.cpu().numpy()[np.ix_(rows, cols)], ref["y16"], sh.name)
        wref = U.oracle_at(a16, w16, idx8, rows, np.arange(win, win + cnt))
        assert np.array_equal(part.cpu().numpy()[rows].astype(np.int64), U.partials_at(wref)), sh.name
