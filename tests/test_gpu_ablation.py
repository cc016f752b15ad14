"""The measured variants of the tile GEMM (libmixllm_<name>.so, same C ABI) against the
CPU oracle.

* zero_pre: 4-bit zero points subtracted from the codes before the matrix cores (the
  pages' vsub4 design, talk notes 二段階逆量子化) instead of the matrix-core correction.
* fold_bias: the float-bits int-to-float conversion (talk notes 高速 I2F 変換): the MFMA
  chain of a partial starts from the integer 0x4B400000, so its bits read as a float are
  B + P exactly (B = 1.5 * 2^23, |P| < 2^22), and one exact subtraction of B gives P.
Both compute the same partials and scale products as the library, so both meet the same
parity bar.
"""
import numpy as np
import pytest

from tests import gpu_util as U
from weight_activation_quantized_amd import workloads as WL

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

SHAPES = [(65, 200, 512, 31), (128, 256, 1024, 26), (96, 130, 2688, 13), (192, 384, 128, 40)]


@pytest.fixture(scope="module")
def L():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a GPU")
    from weight_activation_quantized_amd import mixllm
    return mixllm


def _run(L, lib, a16, w16, idx8):
    m, k = a16.shape
    n = w16.shape[0]
    g = k // 128
    blob = L.DeviceBlob(L.mixllm_pack_weights(w16, idx8))
    a = torch.from_numpy(np.ascontiguousarray(a16)).cuda()
    aq = torch.empty((m, k), dtype=torch.int8, device="cuda")
    sa = torch.empty((g, m), dtype=torch.float32, device="cuda")
    asum = torch.empty((g, m), dtype=torch.int32, device="cuda")
    ro = L.rowop_buffer(m, k)
    L.mixllm_quant_act(a, aq, sa, asum, ro, lib=lib)
    y = torch.full((m, n), float("nan"), dtype=torch.float16, device="cuda")
    L.mixllm_gemm_w4w8a8(aq, sa, asum, ro, m, n, k, len(idx8), blob, y, lib=lib)
    torch.cuda.synchronize()
    return y.cpu().numpy().astype(np.float64)


@pytest.mark.parametrize("variant", ["zero_pre", "fold_bias"])
@pytest.mark.parametrize("m,n,k,n8", SHAPES)
def test_variant_parity(L, variant, m, n, k, n8):
    lib = L.load_variant(variant)
    sh = WL.Shape(0, "edge", m, n, k, n8)
    a16, w16, idx8 = WL.make_layer_inputs(sh)
    U.say(variant, sh.name)
    yg = _run(L, lib, a16, w16, idx8)
    ref = U.oracle_at(a16, w16, idx8)
    U.assert_y_close(yg.astype(np.float16), ref["y16"], variant + " " + sh.name)
