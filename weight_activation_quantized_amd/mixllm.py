"""Thin Python binding of libmixllm.so (C ABI in include/mixllm.h).

Argument marshalling only: every step of the layer runs in the library (host packer in
C++, activation quantization and the mixed GEMM in HIP kernels).  PyTorch supplies
device memory and the HIP stream.  The functions carry the C names; a non-zero status
raises ``MixLLMError``.  Importing this module fails loudly when the library is missing.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

try:  # torch first: its HIP runtime must be the one the library binds to
    import torch
except ImportError:  # pragma: no cover - host-only use of the packer
    torch = None

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.environ.get("MIXLLM_LIB") or os.path.join(HERE, "libmixllm.so")
HEADER = os.path.join(os.path.dirname(HERE), "include", "mixllm.h")
GROUP = 128

if not os.path.exists(LIB_PATH):
    raise ImportError(
        f"{LIB_PATH} is missing: build it with `python -m weight_activation_quantized_amd.build` "
        "(there is no fallback implementation)")

_lib = ctypes.CDLL(LIB_PATH, mode=ctypes.RTLD_GLOBAL)
_variants = {}


def hip_runtimes_loaded():
    """Distinct libamdhip64 files mapped into this process."""
    paths = set()
    with open("/proc/self/maps") as f:
        for line in f:
            parts = line.split()
            if len(parts) >= 6 and "libamdhip64" in parts[-1]:
                paths.add(os.path.realpath(parts[-1]))
    return paths


_runtimes = hip_runtimes_loaded()
if len(_runtimes) > 1:
    raise ImportError(f"two HIP runtimes are loaded into one process: {sorted(_runtimes)}")


class BlobInfo(ctypes.Structure):
    _fields_ = [("magic", ctypes.c_uint32), ("version", ctypes.c_uint32),
                ("N", ctypes.c_int32), ("K", ctypes.c_int32), ("group", ctypes.c_int32),
                ("n8", ctypes.c_int32), ("n4", ctypes.c_int32), ("G", ctypes.c_int32),
                ("nb", ctypes.c_int32), ("nb4", ctypes.c_int32), ("nb8", ctypes.c_int32),
                ("n4_promoted", ctypes.c_int32),
                ("off_w4", ctypes.c_uint64), ("off_s4", ctypes.c_uint64), ("off_z4", ctypes.c_uint64),
                ("off_w8", ctypes.c_uint64), ("off_s8", ctypes.c_uint64), ("off_zp", ctypes.c_uint64),
                ("off_idx", ctypes.c_uint64), ("total_bytes", ctypes.c_uint64)]

    def as_dict(self):
        return {name: getattr(self, name) for name, _ in self._fields_}


_vp, _i32, _i64, _sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
_SIGS = {
    "mixllm_status_str": ([ctypes.c_int], ctypes.c_char_p),
    "mixllm_packed_bytes": ([_i32, _i32, _i32, _i32], _sz),
    "mixllm_pack_weights": ([_vp, _i32, _i32, _i32, _vp, _i32, _vp, _sz], ctypes.c_int),
    "mixllm_blob_get_info": ([_vp, _sz, ctypes.POINTER(BlobInfo)], ctypes.c_int),
    "mixllm_unpack_weights": ([_vp, _sz, _vp, _vp, _vp, _vp], ctypes.c_int),
    "mixllm_channel_salience": ([_vp, _vp, _i32, _i32, _i32, _i32, _vp], ctypes.c_int),
    "mixllm_assign_channels": ([_vp, _vp, _i32, _i64, _vp, _vp], ctypes.c_int),
    "mixllm_quant_act": ([_vp, _i64, _i32, _i32, _i32, _vp, _vp, _vp, _vp, _vp], ctypes.c_int),
    "mixllm_silu_mul_quant": ([_vp, _vp, _i64, _i32, _i32, _i32, _vp, _vp, _vp, _vp, _vp, _vp], ctypes.c_int),
    "mixllm_gemm_workspace_bytes": ([_i32, _i32, _i32, _i32], _sz),
    "mixllm_gemm_w4w8a8": ([_vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _vp, _vp, _sz, _vp, _i64, _vp, _sz,
                            _vp], ctypes.c_int),
    "mixllm_gemm_w4w8a8_partials": ([_vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _vp, _vp, _sz, _i32, _i32,
                                     _vp, _vp], ctypes.c_int),
}
def _bind(lib):
    for name, (args, res) in _SIGS.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = res
    return lib


_bind(_lib)


def load_variant(name: str):
    """A measured variant of the library (libmixllm_<name>.so, built by
    ``python -m weight_activation_quantized_amd.build --variants``), loaded beside the
    main one with its symbols kept local.  Pass it as ``lib=`` to the device calls."""
    if name not in _variants:
        path = os.path.join(HERE, f"libmixllm_{name}.so")
        if not os.path.exists(path):
            raise ImportError(f"{path} is missing: build it with "
                              "`python -m weight_activation_quantized_amd.build --variants`")
        _variants[name] = _bind(ctypes.CDLL(path, mode=ctypes.RTLD_LOCAL))
    return _variants[name]

STATUS = {0: "MIXLLM_OK", -1: "MIXLLM_E_NULL", -2: "MIXLLM_E_SHAPE", -3: "MIXLLM_E_GROUP",
          -4: "MIXLLM_E_INDEX", -5: "MIXLLM_E_SPACE", -6: "MIXLLM_E_FORMAT", -7: "MIXLLM_E_HIP"}


class MixLLMError(RuntimeError):
    def __init__(self, status: int):
        self.status = status
        self.name = STATUS.get(status, str(status))
        super().__init__(mixllm_status_str(status))


def _check(status: int) -> None:
    if status != 0:
        raise MixLLMError(status)


def exported_symbols():
    """Function names declared in include/mixllm.h."""
    import re
    with open(HEADER) as f:
        text = f.read()
    return sorted(set(re.findall(r"\b(mixllm_[a-z0-9_]+)\s*\(", text)))


def library_handle():
    return _lib


# ---------------------------------------------------------------------------- host calls

def mixllm_status_str(status: int) -> str:
    return _lib.mixllm_status_str(int(status)).decode()


def mixllm_packed_bytes(n: int, k: int, group: int = GROUP, n8: int = 0) -> int:
    return int(_lib.mixllm_packed_bytes(n, k, group, n8))


def mixllm_pack_weights(w_fp16: np.ndarray, idx8, group: int = GROUP) -> np.ndarray:
    """Packs an fp16 [N, K] weight matrix; returns the blob as a uint8 numpy array."""
    w = np.ascontiguousarray(w_fp16, dtype=np.float16)
    n, k = w.shape
    idx = np.ascontiguousarray(np.asarray(idx8, dtype=np.int32).reshape(-1))
    size = mixllm_packed_bytes(n, k, group, int(idx.size))
    blob = np.zeros(max(size, 1), dtype=np.uint8)
    _check(_lib.mixllm_pack_weights(w.ctypes.data, n, k, group,
                                    idx.ctypes.data if idx.size else None, int(idx.size),
                                    blob.ctypes.data, blob.size if size else 0))
    return blob


def blob_header(blob: np.ndarray) -> BlobInfo:
    """The checked header of a host blob (mixllm_blob_get_info), as the C struct the GEMM
    calls take."""
    b = np.ascontiguousarray(blob, dtype=np.uint8)
    info = BlobInfo()
    _check(_lib.mixllm_blob_get_info(b.ctypes.data, b.size, ctypes.byref(info)))
    return info


def mixllm_blob_get_info(blob: np.ndarray) -> dict:
    return blob_header(blob).as_dict()


def mixllm_unpack_weights(blob: np.ndarray):
    """Returns (q uint8 [N, K], z uint8 [N, G], s fp16 [N, G], is8 bool [N])."""
    info = mixllm_blob_get_info(blob)
    n, k, g = info["N"], info["K"], info["G"]
    b = np.ascontiguousarray(blob, dtype=np.uint8)
    q = np.zeros((n, k), np.uint8)
    z = np.zeros((n, g), np.uint8)
    s = np.zeros((n, g), np.uint16)
    is8 = np.zeros(n, np.uint8)
    _check(_lib.mixllm_unpack_weights(b.ctypes.data, b.size, q.ctypes.data, z.ctypes.data,
                                      s.ctypes.data, is8.ctypes.data))
    return q, z, s.view(np.float16), is8.astype(bool)


def mixllm_channel_salience(w_fp16: np.ndarray, grads: np.ndarray, group: int = GROUP) -> np.ndarray:
    """w_fp16: [N, K] fp16; grads: [D, N, K] fp32.  Returns the fp64 salience of each channel."""
    w = np.ascontiguousarray(w_fp16, dtype=np.float16)
    g = np.ascontiguousarray(grads, dtype=np.float32)
    n, k = w.shape
    if g.ndim != 3 or g.shape[1:] != (n, k):
        raise ValueError("grads must be [D, N, K]")
    out = np.zeros(n, np.float64)
    _check(_lib.mixllm_channel_salience(w.ctypes.data, g.ctypes.data, n, k, group, g.shape[0], out.ctypes.data))
    return out


def mixllm_assign_channels(scores, total_8bit: int):
    """scores: list of per-layer fp64 arrays.  Returns the per-layer idx8 arrays (int32,
    ascending) of the global top-``total_8bit`` channels."""
    per = [np.ascontiguousarray(s, dtype=np.float64).reshape(-1) for s in scores]
    flat = np.ascontiguousarray(np.concatenate(per)) if per else np.zeros(0)
    sizes = np.array([len(s) for s in per], np.int32)
    idx = np.zeros(max(int(total_8bit), 1), np.int32)
    n8 = np.zeros(max(len(per), 1), np.int32)
    _check(_lib.mixllm_assign_channels(flat.ctypes.data, sizes.ctypes.data, len(per), int(total_8bit),
                                       idx.ctypes.data, n8.ctypes.data))
    out, o = [], 0
    for c in n8[:len(per)]:
        out.append(idx[o:o + c].copy())
        o += int(c)
    return out


# ---------------------------------------------------------------------------- device calls

def _stream(stream):
    if stream is None:
        return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    if isinstance(stream, int):
        return ctypes.c_void_p(stream)
    return ctypes.c_void_p(stream.cuda_stream)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def mixllm_quant_act(a, aq, sa, asum=None, rowop=None, stream=None, lib=None):
    """a: fp16 [M, K] CUDA tensor (rows may be strided); aq: int8 [M, K];
    sa: fp32 [G, M]; asum: int32 [G, M] or None; rowop: 32-bit [G, M, 8] or None."""
    m, k = a.shape
    if a.dtype != torch.float16 or a.stride(1) != 1 or not a.is_cuda:
        raise ValueError("a must be an fp16 CUDA tensor with unit column stride")
    if m:
        g = k // GROUP
        _need(aq, "aq", torch.int8, (m, k))
        _need(sa, "sa", torch.float32, (g, m))
        if asum is not None:
            _need(asum, "asum", torch.int32, (g, m))
        if rowop is not None:
            _need(rowop, "rowop", torch.int32, (g, m, 8))
    lda = a.stride(0) if m > 1 else k
    _check((lib or _lib).mixllm_quant_act(_ptr(a), lda, m, k, GROUP, _ptr(aq), _ptr(sa), _ptr(asum),
                                          _ptr(rowop), _stream(stream)))


def mixllm_silu_mul_quant(gate, up, aq, sa, asum=None, rowop=None, h=None, stream=None, lib=None):
    """gate, up: fp16 [M, I] CUDA views with the same row stride (e.g. the two halves of a
    [M, 2I] GEMM output); outputs as mixllm_quant_act with K = I; h: fp16 [M, I] or None."""
    m, inter = gate.shape
    if gate.dtype != torch.float16 or up.dtype != torch.float16 or gate.stride(1) != 1 or up.stride(1) != 1:
        raise ValueError("gate and up must be fp16 with unit column stride")
    if up.shape != gate.shape or (m > 1 and up.stride(0) != gate.stride(0)):
        raise ValueError("gate and up must have the same shape and row stride")
    if m:
        g = inter // GROUP
        _need(aq, "aq", torch.int8, (m, inter))
        _need(sa, "sa", torch.float32, (g, m))
        if asum is not None:
            _need(asum, "asum", torch.int32, (g, m))
        if rowop is not None:
            _need(rowop, "rowop", torch.int32, (g, m, 8))
        if h is not None:
            _need(h, "h", torch.float16, (m, inter))
    ld = gate.stride(0) if m > 1 else inter
    _check((lib or _lib).mixllm_silu_mul_quant(_ptr(gate), _ptr(up), ld, m, inter, GROUP, _ptr(aq), _ptr(sa),
                                               _ptr(asum), _ptr(rowop), _ptr(h), _stream(stream)))


def mixllm_gemm_workspace_bytes(m: int, n: int, k: int, n8: int) -> int:
    return int(_lib.mixllm_gemm_workspace_bytes(m, n, k, n8))


class DeviceBlob:
    """A packed blob on the GPU with the host copy of its header (the GEMM calls check
    the header against the layer they are asked to compute)."""

    def __init__(self, blob_host: np.ndarray, device="cuda"):
        self.info = blob_header(blob_host)
        self.dev = torch.from_numpy(np.ascontiguousarray(blob_host, dtype=np.uint8)).to(device)
        self.nbytes = int(self.dev.numel())


def _need(t, name, dtype, shape=None, what=""):
    """Argument checks before a device call: a CUDA tensor of this dtype whose shape
    covers `shape` and whose innermost stride is 1."""
    if t is None:
        raise ValueError(f"{name} is required{what}")
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise ValueError(f"{name} must be a CUDA tensor")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if t.dim() and t.stride(-1) != 1:
        raise ValueError(f"{name} must have unit innermost stride")
    if shape is not None:
        if t.dim() != len(shape) or any(a < b for a, b in zip(t.shape, shape)):
            raise ValueError(f"{name} has shape {tuple(t.shape)}, needs at least {tuple(shape)}")
        if not t.is_contiguous() and name != "y":
            raise ValueError(f"{name} must be contiguous")


def _gemm_inputs(aq, sa, asum, rowop, m, k, nb4):
    g = k // GROUP
    _need(aq, "aq", torch.int8, (m, k))
    _need(sa, "sa", torch.float32, (g, m))
    if asum is not None or nb4 > 0:
        _need(asum, "asum", torch.int32, (g, m), " for layers with 4-bit blocks")
    _need(rowop, "rowop", torch.int32, (g, m, 8))
    for t, name, shape in ((aq, "aq", (m, k)), (sa, "sa", (g, m)), (asum, "asum", (g, m)),
                           (rowop, "rowop", (g, m, 8))):
        if t is not None and m and tuple(t.shape) != shape:
            raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {shape}")


def _blob(blob):
    if not isinstance(blob, DeviceBlob):
        raise ValueError("blob must be a DeviceBlob (the device copy plus its host header)")
    return blob


def mixllm_gemm_w4w8a8(aq, sa, asum, rowop, m: int, n: int, k: int, n8: int, blob, y, workspace=None,
                       stream=None, lib=None):
    """aq, sa, asum, rowop: outputs of mixllm_quant_act; y: fp16 [M, ldy] CUDA tensor (ldy >= N);
    blob: DeviceBlob of the packed layer."""
    b = _blob(blob)
    if m:
        _gemm_inputs(aq, sa, asum, rowop, m, k, b.info.nb4)
        _need(y, "y", torch.float16, (m, n))
        if y.dim() != 2:
            raise ValueError("y must be 2-D")
    ldy = y.stride(0) if y is not None and y.dim() == 2 and m > 1 else n
    ws = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check((lib or _lib).mixllm_gemm_w4w8a8(_ptr(aq), _ptr(sa), _ptr(asum), _ptr(rowop), m, n, k, n8,
                                            ctypes.byref(b.info), _ptr(b.dev), b.nbytes, _ptr(y), ldy,
                                            _ptr(workspace), ws, _stream(stream)))


def mixllm_gemm_w4w8a8_partials(aq, sa, asum, rowop, m: int, n: int, k: int, n8: int, blob, n_begin: int,
                                n_count: int, part, stream=None, lib=None):
    """part: int32 [M, n_count, G] CUDA tensor."""
    b = _blob(blob)
    if m and n_count:
        _gemm_inputs(aq, sa, asum, rowop, m, k, b.info.nb4)
        _need(part, "part", torch.int32, (m, n_count, k // GROUP))
        if not part.is_contiguous():
            raise ValueError("part must be contiguous")
    _check((lib or _lib).mixllm_gemm_w4w8a8_partials(_ptr(aq), _ptr(sa), _ptr(asum), _ptr(rowop), m, n, k, n8,
                                                     ctypes.byref(b.info), _ptr(b.dev), b.nbytes, n_begin,
                                                     n_count, _ptr(part), _stream(stream)))


def rowop_buffer(m: int, k: int, device="cuda"):
    """Storage for mixllm_quant_act's row operands: 32-bit words [G, M, 8]."""
    return torch.empty((k // GROUP, m, 8), dtype=torch.int32, device=device)


# ---------------------------------------------------------------------------- convenience

class PackedLinear:
    """A packed layer resident on the GPU plus the buffers one forward pass needs.

    ``forward(a)`` runs the hot path: mixllm_quant_act then mixllm_gemm_w4w8a8.
    """

    def __init__(self, w_fp16: np.ndarray, idx8, device="cuda"):
        self.n, self.k = w_fp16.shape
        self.n8 = int(np.asarray(idx8).size)
        self.g = self.k // GROUP
        self.blob_host = mixllm_pack_weights(w_fp16, idx8)
        self.blob = DeviceBlob(self.blob_host, device)
        self.device = device

    def buffers(self, m: int):
        dev = self.device
        return dict(aq=torch.empty((m, self.k), dtype=torch.int8, device=dev),
                    sa=torch.empty((self.g, m), dtype=torch.float32, device=dev),
                    asum=torch.empty((self.g, m), dtype=torch.int32, device=dev),
                    rowop=rowop_buffer(m, self.k, dev),
                    y=torch.empty((m, self.n), dtype=torch.float16, device=dev),
                    ws=self._workspace(m))

    def _workspace(self, m):
        nbytes = mixllm_gemm_workspace_bytes(m, self.n, self.k, self.n8)
        return torch.zeros(nbytes, dtype=torch.uint8, device=self.device) if nbytes else None

    def forward(self, a, bufs=None, stream=None):
        m = a.shape[0]
        bufs = bufs or self.buffers(m)
        mixllm_quant_act(a, bufs["aq"], bufs["sa"], bufs["asum"], bufs["rowop"], stream)
        mixllm_gemm_w4w8a8(bufs["aq"], bufs["sa"], bufs["asum"], bufs["rowop"], m, self.n, self.k, self.n8,
                           self.blob, bufs["y"], bufs["ws"], stream)
        return bufs["y"]


def concat_layers(weights, idx8s):
    """Several layers over the same input as one: their fp16 weights stacked along the output
    channels, each layer's 8-bit channel indices shifted to its rows.  Returns (w, idx8,
    bounds), bounds[i] = the output columns (begin, end) of layer i."""
    ws = [np.asarray(w, np.float16) for w in weights]
    if len({w.shape[1] for w in ws}) != 1:
        raise ValueError("the layers must share the input width")
    offs = np.cumsum([0] + [w.shape[0] for w in ws])
    idx = np.concatenate([np.asarray(i, np.int32).reshape(-1) + np.int32(o) for i, o in zip(idx8s, offs[:-1])])
    return np.concatenate(ws), idx, [(int(offs[i]), int(offs[i + 1])) for i in range(len(ws))]


class QKVProjection:
    """The attention input projections of one hidden state: q, k and v packed together as
    one layer (their output channels concatenated, each keeping its own 8-bit channels),
    so one activation quantization and one GEMM launch produce all three.  ``forward``
    returns views of the one output.  Argument marshalling only."""

    def __init__(self, w_q, w_k, w_v, idx8_q, idx8_k, idx8_v, device="cuda"):
        w, idx, self.bounds = concat_layers((w_q, w_k, w_v), (idx8_q, idx8_k, idx8_v))
        self.layer = PackedLinear(w, idx, device)
        self.device = device

    def buffers(self, m: int):
        return self.layer.buffers(m)

    def split(self, y):
        return tuple(y[:, a:b] for a, b in self.bounds)

    def forward(self, x, bufs, stream=None):
        return self.split(self.layer.forward(x, bufs, stream))

    def capture(self, x, bufs):
        """A HIP graph of one forward pass on these buffers (torch.cuda.CUDAGraph)."""
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            self.forward(x, bufs, s)  # warm-up outside the capture
        torch.cuda.current_stream().wait_stream(s)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=s):
            self.forward(x, bufs, s)
        return g


class MLPBlock:
    """The Llama MLP block on the packed layers: one activation quantization feeds one GEMM
    over the gate and up channels (packed together as one layer of 2I channels), the fused
    SiLU(gate) * up + quantization feeds the down projection.  Four launches on one stream;
    ``capture`` records them in a HIP graph.  Argument marshalling only."""

    def __init__(self, w_gate, w_up, w_down, idx8_gate, idx8_up, idx8_down, device="cuda"):
        self.inter, self.hidden = np.asarray(w_gate).shape
        w_gu, idx_gu, _ = concat_layers((w_gate, w_up), (idx8_gate, idx8_up))
        self.gu = PackedLinear(w_gu, idx_gu, device)
        self.down = PackedLinear(np.asarray(w_down, np.float16), idx8_down, device)
        self.device = device

    def buffers(self, m: int):
        dev = self.device
        return dict(x=self.gu.buffers(m), h=self.down.buffers(m),
                    h16=torch.empty((m, self.inter), dtype=torch.float16, device=dev))

    def forward(self, x, bufs, stream=None, keep_h=False):
        m = x.shape[0]
        bx, bh = bufs["x"], bufs["h"]
        self.gu.forward(x, bx, stream)
        gu = bx["y"]
        mixllm_silu_mul_quant(gu[:, :self.inter], gu[:, self.inter:], bh["aq"], bh["sa"], bh["asum"], bh["rowop"],
                              bufs["h16"] if keep_h else None, stream)
        mixllm_gemm_w4w8a8(bh["aq"], bh["sa"], bh["asum"], bh["rowop"], m, self.down.n, self.down.k,
                           self.down.n8, self.down.blob, bh["y"], bh["ws"], stream)
        return bh["y"]

    def capture(self, x, bufs, keep_h=False):
        """A HIP graph of one forward pass on these buffers (torch.cuda.CUDAGraph)."""
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            self.forward(x, bufs, s, keep_h)  # warm-up outside the capture
        torch.cuda.current_stream().wait_stream(s)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=s):
            self.forward(x, bufs, s, keep_h)
        return g
