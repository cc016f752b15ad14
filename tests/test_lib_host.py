"""Host side of libmixllm.so, no GPU needed: the library loads and exports every symbol
declared in include/mixllm.h; the C++ packer is bit-exact against the oracle's
quantizers; blob sizes follow the layout; every argument check returns its status
before any HIP call."""
import ctypes

import numpy as np
import pytest

import oracle as O
from weight_activation_quantized_amd import workloads as WL

L = pytest.importorskip("weight_activation_quantized_amd.mixllm")


def test_exports_every_declared_symbol():
    names = L.exported_symbols()
    assert len(names) >= 9
    lib = L.library_handle()
    for name in names:
        assert hasattr(lib, name), name


def test_single_hip_runtime():
    assert len(L.hip_runtimes_loaded()) <= 1


def test_status_strings():
    for code, name in L.STATUS.items():
        assert L.mixllm_status_str(code).startswith(name)
    assert "unknown" in L.mixllm_status_str(-99)


def _check_pack(w, idx8):
    blob = L.mixllm_pack_weights(w, idx8)
    q, z, s16, is8 = L.mixllm_unpack_weights(blob)
    oq, oz, os_, ois8 = O.quant_weights_mixed(w, idx8)
    assert np.array_equal(is8, ois8)
    assert np.array_equal(q, (oq.astype(np.int16) & 0xFF).astype(np.uint8)), "codes"
    assert np.array_equal(z, oz), "zero points"
    assert np.array_equal(s16.view(np.uint16), os_.view(np.uint16)), "scales"
    return blob


@pytest.mark.parametrize("n,k,n8", [(512, 1024, 52), (96, 256, 0), (96, 256, 96), (100, 384, 7),
                                    (64, 128, 32), (33, 256, 1), (1, 128, 0), (1, 128, 1),
                                    (200, 512, 169)])
def test_pack_matches_oracle(n, k, n8):
    sh = WL.Shape(0, "edge", 1, n, k, n8)
    w, idx8 = WL.make_layer_weights(sh)
    blob = _check_pack(w, idx8)
    info = L.mixllm_blob_get_info(blob)
    assert info["N"] == n and info["K"] == k and info["n8"] == n8 and info["n4"] == n - n8
    assert info["nb"] == (n + 31) // 32
    assert info["nb4"] == (n - n8) // 32 and info["nb8"] == info["nb"] - info["nb4"]
    assert info["n4_promoted"] == (n - n8) % 32
    assert info["total_bytes"] == blob.size == L.mixllm_packed_bytes(n, k, 128, n8)


def test_concat_layers_packs_each_projection_as_alone():
    """q, k, v packed as one layer: each slice of the unpacked blob equals that projection
    quantized on its own (the concatenation shifts only the 8-bit indices)."""
    n8 = dict(q=22, k=5, v=73)
    x, wq, wk, wv, iq, ik, iv = WL.qkv_inputs(1, 256, 128, 96, n8)
    w, idx, bounds = L.concat_layers((wq, wk, wv), (iq, ik, iv))
    assert bounds == [(0, 128), (128, 224), (224, 320)]
    assert idx.size == 22 + 5 + 73 and np.all(np.diff(idx) > 0)
    q, z, s16, is8 = L.mixllm_unpack_weights(L.mixllm_pack_weights(w, idx))
    for (a, b), wp, ip in zip(bounds, (wq, wk, wv), (iq, ik, iv)):
        oq, oz, os_, ois8 = O.quant_weights_mixed(wp, ip)
        assert np.array_equal(is8[a:b], ois8)
        assert np.array_equal(q[a:b], (oq.astype(np.int16) & 0xFF).astype(np.uint8))
        assert np.array_equal(z[a:b], oz)
        assert np.array_equal(s16[a:b].view(np.uint16), os_.view(np.uint16))
    with pytest.raises(ValueError):
        L.concat_layers((wq, wk[:, :128]), (iq, ik))


def _split_bf16_pair(x32):
    """The tile kernel's operand split, restated: the leading 8 significant bits of the
    fp32 value (its bf16 truncation) and the remainder, as float64 values."""
    x32 = np.asarray(x32, np.float32)
    b0 = x32.view(np.uint32) & np.uint32(0xFFFF0000)
    hi = b0.view(np.float32)
    lo = (x32 - hi).astype(np.float32)
    return hi.astype(np.float64), lo


def test_column_operands_split_exactly_into_bf16_pairs():
    """The GEMM's scale-product operands s_w and z * s_w (z in 0..15) are formed on the
    device as two bf16 values each: exhaustively over every finite fp16 s_w, both
    products are exact in fp32 and the remainder after the bf16 truncation is itself a
    bf16 value (its low 16 bits are zero), so the pair sums to the value exactly."""
    s16 = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16).view(np.float16)
    s16 = s16[np.isfinite(s16)]
    for z in range(16):
        v64 = z * s16.astype(np.float64)
        v32 = v64.astype(np.float32)
        assert np.array_equal(v32.astype(np.float64), v64), z     # z * s_w exact in fp32
        hi, lo = _split_bf16_pair(v32)
        assert not (lo.view(np.uint32) & np.uint32(0xFFFF)).any(), z  # a bf16 value
        assert np.array_equal(hi + lo.astype(np.float64), v64), z


def test_blob_has_no_column_word_section():
    """Every byte after the channel indices is alignment padding: the tile kernel reads
    the column scales and zero points from s4, s8 and z4."""
    for n, k, n8 in [(200, 512, 169), (100, 384, 7), (64, 256, 0)]:
        w, idx8 = WL.make_layer_weights(WL.Shape(0, "edge", 1, n, k, n8))
        blob = L.mixllm_pack_weights(w, idx8)
        info = L.mixllm_blob_get_info(blob)
        nb = info["nb"]
        end_idx = info["off_idx"] + nb * 32 * 4
        assert info["total_bytes"] == (end_idx + 255) // 256 * 256
        assert not blob[end_idx:].any()


def test_pack_special_groups():
    """All-zero groups, one-signed groups, subnormal-range groups and the golden ties."""
    rng = np.random.default_rng(7)
    w = rng.normal(0, 0.02, size=(40, 512))
    w[0] = 0
    w[1, :128] = 0
    w[2] = np.abs(w[2])
    w[3] = -np.abs(w[3])
    w[4] *= 1e-5
    w[5] *= 1e-7
    w[6, :128] = 6e-8
    w = w.astype(np.float16)
    for idx8 in ([], [0, 1, 2, 3, 4, 5, 6], [0, 2, 4, 6, 39], list(range(40))):
        _check_pack(w, np.array(idx8, dtype=np.int32))


def test_pack_idx8_order_irrelevant():
    sh = WL.Shape(0, "edge", 1, 70, 256, 9)
    w, idx8 = WL.make_layer_weights(sh)
    a = L.mixllm_pack_weights(w, idx8)
    b = L.mixllm_pack_weights(w, idx8[::-1].copy())
    assert np.array_equal(a, b)


def test_packed_bytes_formula():
    """Blob bytes = the pages' footprints (0.5 + 2.5/G per 4-bit element, 1 + 2/G per
    8-bit element) over the padded blocks, plus the channel index and alignment."""
    for n, k, n8 in [(4096, 4096, 410), (14336, 4096, 105), (1024, 4096, 729), (8192, 28672, 820)]:
        nb = (n + 31) // 32
        nb4 = (n - n8) // 32
        nb8 = nb - nb4
        g = k // 128
        w_bytes = 32 * k * (nb4 * O.weight_footprint(4) + nb8 * O.weight_footprint(8))
        side = 32 * g  # zero points of the <= 31 promoted 4-bit channels (unpacking only)
        size = L.mixllm_packed_bytes(n, k, 128, n8)
        assert w_bytes + 4 * 32 * nb + side <= size <= w_bytes + 4 * 32 * nb + side + 8 * 256 + 256
        # the padding to 32-channel blocks and the <= 31 4-bit channels stored as int8
        # cost at most one 8-bit block more than the algorithmic byte count
        alg = O.algorithmic_bytes(0, n, k, n8)
        assert alg <= size <= alg + 32 * k * O.weight_footprint(8) + side + 4096


def test_pack_errors():
    w = np.zeros((64, 256), np.float16)
    ok = np.array([1, 2], np.int32)
    pack = L.library_handle().mixllm_pack_weights
    blob = np.zeros(L.mixllm_packed_bytes(64, 256, 128, 2), np.uint8)
    wp, bp, ip = w.ctypes.data, blob.ctypes.data, ok.ctypes.data
    assert pack(None, 64, 256, 128, ip, 2, bp, blob.size) == -1
    assert pack(wp, 64, 256, 128, None, 2, bp, blob.size) == -1
    assert pack(wp, 64, 256, 128, ip, 2, None, blob.size) == -1
    assert pack(wp, 64, 256, 64, ip, 2, bp, blob.size) == -3
    assert pack(wp, 64, 200, 128, ip, 2, bp, blob.size) == -2
    assert pack(wp, 0, 256, 128, ip, 2, bp, blob.size) == -2
    assert pack(wp, 64, 256, 128, ip, 65, bp, blob.size) == -4
    assert pack(wp, 64, 256, 128, ip, -1, bp, blob.size) == -4
    dup = np.array([3, 3], np.int32)
    assert pack(wp, 64, 256, 128, dup.ctypes.data, 2, bp, blob.size) == -4
    bad = np.array([3, 64], np.int32)
    assert pack(wp, 64, 256, 128, bad.ctypes.data, 2, bp, blob.size) == -4
    neg = np.array([-1, 3], np.int32)
    assert pack(wp, 64, 256, 128, neg.ctypes.data, 2, bp, blob.size) == -4
    assert pack(wp, 64, 256, 128, ip, 2, bp, blob.size - 1) == -5
    assert pack(wp, 64, 256, 128, ip, 2, bp, blob.size) == 0
    assert L.mixllm_packed_bytes(64, 200, 128, 2) == 0
    assert L.mixllm_packed_bytes(64, 256, 64, 2) == 0
    assert L.mixllm_packed_bytes(64, 256, 128, 65) == 0


def test_blob_format_errors():
    w = np.zeros((64, 256), np.float16)
    blob = L.mixllm_pack_weights(w, [5])
    with pytest.raises(L.MixLLMError) as e:
        L.mixllm_blob_get_info(blob[:100])
    assert e.value.status == -5
    for off, val in [(0, 0x11), (4, 9), (8, 7)]:
        bad = blob.copy()
        bad[off] ^= val
        with pytest.raises(L.MixLLMError) as e:
            L.mixllm_blob_get_info(bad)
        assert e.value.status == -6
    with pytest.raises(L.MixLLMError) as e:
        L.mixllm_unpack_weights(blob[:-1])
    assert e.value.status == -5


def test_device_entry_points_validate_on_host():
    """Argument errors come back before any HIP call, so these run without a GPU."""
    lib = L.library_handle()
    fake = ctypes.c_void_p(0x10000)       # never dereferenced: every call below fails validation
    odd = ctypes.c_void_p(0x10004)
    s = ctypes.c_void_p(0)
    qa = lib.mixllm_quant_act
    assert qa(fake, 256, 4, 256, 64, fake, fake, None, None, s) == -3
    assert qa(fake, 256, 4, 200, 128, fake, fake, None, None, s) == -2
    assert qa(fake, 128, 4, 256, 128, fake, fake, None, None, s) == -2      # lda < K
    assert qa(fake, 260, 4, 256, 128, fake, fake, None, None, s) == -2      # lda % 8
    assert qa(fake, 256, -1, 256, 128, fake, fake, None, None, s) == -2
    assert qa(None, 256, 4, 256, 128, fake, fake, None, None, s) == -1
    assert qa(fake, 256, 4, 256, 128, None, fake, None, None, s) == -1
    assert qa(odd, 256, 4, 256, 128, fake, fake, None, None, s) == -2
    assert qa(fake, 256, 4, 256, 128, fake, fake, odd, None, s) == -2
    assert qa(fake, 256, 4, 256, 128, fake, fake, None, odd, s) == -2
    assert qa(None, 256, 0, 256, 128, None, None, None, None, s) == 0       # M = 0: no-op

    nbytes = L.mixllm_packed_bytes(64, 256, 128, 2)
    gm = lib.mixllm_gemm_w4w8a8
    f4 = (fake, fake, fake, fake)
    # the host header of a blob packed for (N, K, n8) = (64, 256, 2)
    wl, il = WL.make_layer_weights(WL.Shape(0, "edge", 1, 64, 256, 2))
    hdr = L.blob_header(L.mixllm_pack_weights(wl, il))
    hp = ctypes.byref(hdr)
    assert gm(*f4, 4, 64, 200, 2, hp, fake, nbytes, fake, 64, None, 0, s) == -2
    assert gm(*f4, 4, 64, 256, 65, hp, fake, nbytes, fake, 64, None, 0, s) == -4
    assert gm(*f4, -1, 64, 256, 2, hp, fake, nbytes, fake, 64, None, 0, s) == -2
    for i in range(4):
        args = list(f4)
        args[i] = None
        assert gm(*args, 4, 64, 256, 2, hp, fake, nbytes, fake, 64, None, 0, s) == -1
        args[i] = odd
        assert gm(*args, 4, 64, 256, 2, hp, fake, nbytes, fake, 64, None, 0, s) == -2
    assert gm(*f4, 4, 64, 256, 2, hp, None, nbytes, fake, 64, None, 0, s) == -1
    assert gm(*f4, 4, 64, 256, 2, None, fake, nbytes, fake, 64, None, 0, s) == -1
    assert gm(*f4, 4, 64, 256, 2, hp, fake, nbytes, None, 64, None, 0, s) == -1
    assert gm(*f4, 4, 64, 256, 2, hp, fake, nbytes - 1, fake, 64, None, 0, s) == -5
    assert gm(*f4, 4, 64, 256, 2, hp, fake, nbytes, fake, 63, None, 0, s) == -2
    assert gm(*f4, 4, 64, 256, 2, hp, odd, nbytes, fake, 64, None, 0, s) == -2
    assert gm(None, None, None, None, 0, 64, 256, 2, hp, None, 0, None, 64, None, 0, s) == 0  # M = 0
    # a blob packed for another layer is refused before any launch (E_FORMAT): another
    # 8-bit count (which needs fewer bytes than the caller's buffer), another shape, an
    # older format version, a damaged section offset
    for other in [(64, 256, 0), (64, 256, 3), (96, 256, 2), (64, 384, 2)]:
        wo, io = WL.make_layer_weights(WL.Shape(0, "edge", 1, *other))
        ho = L.blob_header(L.mixllm_pack_weights(wo, io))
        assert gm(*f4, 4, 64, 256, 2, ctypes.byref(ho), fake, 1 << 20, fake, 64, None, 0, s) == -6, other
    for field, delta in [("version", -1), ("magic", 1), ("off_idx", 256), ("total_bytes", -256), ("nb4", 1)]:
        h2 = L.blob_header(L.mixllm_pack_weights(wl, il))
        setattr(h2, field, getattr(h2, field) + delta)
        assert gm(*f4, 4, 64, 256, 2, ctypes.byref(h2), fake, 1 << 20, fake, 64, None, 0, s) == -6, field
    # with no whole 4-bit block (all channels 8-bit) the code sums are not needed
    w8, i8 = WL.make_layer_weights(WL.Shape(0, "edge", 1, 64, 256, 64))
    h8 = L.blob_header(L.mixllm_pack_weights(w8, i8))
    assert h8.nb4 == 0
    nb8 = L.mixllm_packed_bytes(64, 256, 128, 64)
    assert gm(fake, fake, None, fake, 4, 64, 256, 64, ctypes.byref(h8), fake, nb8, fake, 63, None, 0, s) == -2  # ldy < N: past the null checks
    assert gm(fake, fake, None, fake, 4, 64, 256, 2, hp, fake, nbytes, fake, 64, None, 0, s) == -1
    # the tile kernel's 32-bit operand offsets: G * M * 32 must stay below 2^31
    big = L.mixllm_packed_bytes(64, 1 << 17, 128, 2)
    wb = np.zeros((64, 1 << 17), np.float16)
    hb = L.blob_header(L.mixllm_pack_weights(wb, np.array([0, 1], np.int32)))
    assert gm(*f4, 1 << 16, 64, 1 << 17, 2, ctypes.byref(hb), fake, big, fake, 64, None, 0, s) == -2
    assert L.mixllm_gemm_workspace_bytes(512, 4096, 4096, 410) == 0
    gp = lib.mixllm_gemm_w4w8a8_partials
    assert gp(*f4, 4, 64, 256, 2, hp, fake, nbytes, 60, 5, fake, s) == -2
    assert gp(*f4, 4, 64, 256, 2, hp, fake, nbytes, -1, 5, fake, s) == -2
    for other in [(64, 256, 0), (64, 256, 3)]:
        wo, io = WL.make_layer_weights(WL.Shape(0, "edge", 1, *other))
        ho = L.blob_header(L.mixllm_pack_weights(wo, io))
        assert gp(*f4, 4, 64, 256, 2, ctypes.byref(ho), fake, 1 << 20, 0, 5, fake, s) == -6
    assert gp(*f4, 4, 64, 256, 2, hp, fake, nbytes, 0, 5, None, s) == -1
    assert gp(*f4, 4, 64, 256, 2, hp, fake, nbytes, 0, 0, None, s) == 0
