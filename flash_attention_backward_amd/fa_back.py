"""ctypes binding of libfa_back.so (include/fa_back.h): argument marshalling only.

Every step of the backward runs in the HIP library; this module builds descriptors, passes
device pointers and unpacks the packed output. It raises if the library is missing.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libfa_back.so")

NONE, F32, F16, BF16, Q8_0, Q4_0, Q4_1, Q5_0, Q5_1 = -1, 0, 1, 2, 8, 9, 10, 11, 12
CAUSAL_TAIL = 16   # mask type only: query i sees keys j <= M - N + i, nothing stored
# descriptor flags (include/fa_back.h)
FLAG_CENTER_V = 1    # centre V before its fp16 rounding
FLAG_WALK1_KEYS = 2  # LSE/delta walk owned by key tiles
FLAG_WALK1_ROWS = 4  # LSE/delta walk owned by row tiles
FLAG_CENTER_K = 8    # centre K before its fp16 rounding
FLAG_KV_IMAGE = 16   # decode the cache once into the workspace for the query-side walks
FLAG_KV_INLINE = 32  # every query-side workgroup decodes the cache tiles it reads
FLAG_DS_STORE = 64   # the key side stores dS; dQ is formed from it (no second query-side walk)
FLAG_DS_RECOMPUTE = 128  # walk 2 recomputes S and dP for dQ
TYPE_IDS = {"none": NONE, "f32": F32, "f16": F16, "bf16": BF16, "q8_0": Q8_0, "q4_0": Q4_0,
            "q4_1": Q4_1, "q5_0": Q5_0, "q5_1": Q5_1, "causal_tail": CAUSAL_TAIL}
# bytes of one element (one 32-value block for the ggml block types)
ELEM_BYTES = {F32: 4, F16: 2, BF16: 2, Q8_0: 34, Q4_0: 18, Q4_1: 20, Q5_0: 22, Q5_1: 24}
BLOCK_TYPES = ("q8_0", "q4_0", "q4_1", "q5_0", "q5_1")

OK, EINVAL, ESHAPE, ESTRIDE, EUNSUPPORTED, EHIP, EALIGN, ESCRATCH = 0, -1, -2, -3, -4, -5, -6, -7
NOALLOC_MAX_WORKSPACE = 64 << 20   # bytes of the library's static scratch (fa_back_run_noalloc)


class FaBackError(RuntimeError):
    def __init__(self, status: int, what: str = ""):
        self.status = status
        super().__init__(f"{what}: status {status} ({status_string(status)})" if what else
                         f"status {status} ({status_string(status)})")


class Tensor(ctypes.Structure):
    _fields_ = [("type", ctypes.c_int32), ("ne", ctypes.c_int64 * 3), ("nb", ctypes.c_int64 * 3)]


class Desc(ctypes.Structure):
    _fields_ = [("q", Tensor), ("k", Tensor), ("v", Tensor), ("d", Tensor), ("mask", Tensor),
                ("scale", ctypes.c_float), ("flags", ctypes.c_uint32)]


class Layout(ctypes.Structure):
    _fields_ = [("off_dq", ctypes.c_uint64), ("off_dk", ctypes.c_uint64), ("off_dv", ctypes.c_uint64),
                ("off_lse", ctypes.c_uint64), ("off_delta", ctypes.c_uint64),
                ("out_bytes", ctypes.c_uint64), ("workspace_bytes", ctypes.c_uint64),
                ("plan_flags", ctypes.c_uint32)]


_lib = None


def load_library():
    """Load libfa_back.so from the package directory (build it with
    `python -m flash_attention_backward_amd.build`)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: the HIP library has not been built")
    lib = ctypes.CDLL(LIB_PATH)
    lib.fa_back_layout_query.argtypes = [ctypes.POINTER(Desc), ctypes.POINTER(Layout)]
    lib.fa_back_layout_query.restype = ctypes.c_int
    lib.fa_back_create.argtypes = [ctypes.POINTER(Desc), ctypes.c_int, ctypes.POINTER(ctypes.c_void_p),
                                   ctypes.POINTER(Layout)]
    lib.fa_back_create.restype = ctypes.c_int
    lib.fa_back_run.argtypes = [ctypes.c_void_p] + [ctypes.c_void_p] * 8
    lib.fa_back_run.restype = ctypes.c_int
    lib.fa_back_run_timed.argtypes = [ctypes.c_void_p] + [ctypes.c_void_p] * 8 + [ctypes.POINTER(ctypes.c_float)]
    lib.fa_back_run_timed.restype = ctypes.c_int
    lib.fa_back_run_saved.argtypes = [ctypes.c_void_p] + [ctypes.c_void_p] * 10
    lib.fa_back_run_saved.restype = ctypes.c_int
    lib.fa_back_run_saved_timed.argtypes = ([ctypes.c_void_p] + [ctypes.c_void_p] * 10 +
                                            [ctypes.POINTER(ctypes.c_float)])
    lib.fa_back_run_saved_timed.restype = ctypes.c_int
    lib.fa_back_run_noalloc.argtypes = [ctypes.c_void_p] + [ctypes.c_void_p] * 7
    lib.fa_back_run_noalloc.restype = ctypes.c_int
    lib.fa_back_destroy.argtypes = [ctypes.c_void_p]
    lib.fa_back_destroy.restype = None
    lib.fa_back_status_string.argtypes = [ctypes.c_int]
    lib.fa_back_status_string.restype = ctypes.c_char_p
    _lib = lib
    return lib


def status_string(status: int) -> str:
    try:
        return load_library().fa_back_status_string(status).decode()
    except ImportError:
        return "library not loaded"


# ----------------------------------------------------------------------------- C entry points

def fa_back_layout_query(desc: Desc) -> Layout:
    lay = Layout()
    rc = load_library().fa_back_layout_query(ctypes.byref(desc), ctypes.byref(lay))
    if rc != OK:
        raise FaBackError(rc, "fa_back_layout_query")
    return lay


def fa_back_create(desc: Desc, device: int = 0):
    """Returns (plan handle, Layout)."""
    plan = ctypes.c_void_p()
    lay = Layout()
    rc = load_library().fa_back_create(ctypes.byref(desc), device, ctypes.byref(plan), ctypes.byref(lay))
    if rc != OK:
        raise FaBackError(rc, "fa_back_create")
    return plan, lay


def fa_back_run(plan, q: int, k: int, v: int, d: int, mask: Optional[int], out: int, workspace: int,
                stream: int = 0) -> None:
    rc = load_library().fa_back_run(plan, q, k, v, d, mask or None, out, workspace, stream or None)
    if rc != OK:
        raise FaBackError(rc, "fa_back_run")


def fa_back_run_noalloc(plan, q: int, k: int, v: int, d: int, mask: Optional[int], out: int,
                        stream: int = 0) -> None:
    """fa_back_run with the library's static scratch as the workspace (no device allocation)."""
    rc = load_library().fa_back_run_noalloc(plan, q, k, v, d, mask or None, out, stream or None)
    if rc != OK:
        raise FaBackError(rc, "fa_back_run_noalloc")


NUM_PHASES = 7
PHASES = ("absmax", "prep", "walk1", "merge", "walk2", "dqreduce", "kvpass")


def fa_back_run_timed(plan, q: int, k: int, v: int, d: int, mask: Optional[int], out: int,
                      workspace: int, stream: int = 0) -> list:
    """Run once, blocking, and return the elapsed milliseconds of each kernel phase."""
    ms = (ctypes.c_float * NUM_PHASES)()
    rc = load_library().fa_back_run_timed(plan, q, k, v, d, mask or None, out, workspace,
                                          stream or None, ms)
    if rc != OK:
        raise FaBackError(rc, "fa_back_run_timed")
    return list(ms)


def fa_back_run_saved(plan, q: int, k: int, v: int, d: int, mask: Optional[int], lse: int, o: int,
                      out: int, workspace: int, stream: int = 0, timed: bool = False):
    """fa_back_run with the forward's LSE (F32, row h*N + i) and O (F32 [Dv, N, H]); with
    timed=True it blocks and returns the phase times like fa_back_run_timed."""
    lib = load_library()
    if timed:
        ms = (ctypes.c_float * NUM_PHASES)()
        rc = lib.fa_back_run_saved_timed(plan, q, k, v, d, mask or None, lse or None, o or None, out,
                                         workspace, stream or None, ms)
    else:
        rc = lib.fa_back_run_saved(plan, q, k, v, d, mask or None, lse or None, o or None, out,
                                   workspace, stream or None)
    if rc != OK:
        raise FaBackError(rc, "fa_back_run_saved")
    return list(ms) if timed else None


def fa_back_destroy(plan) -> None:
    load_library().fa_back_destroy(plan)


# ----------------------------------------------------------------------------- descriptors

def make_tensor(typ, ne, nb) -> Tensor:
    t = Tensor()
    t.type = TYPE_IDS[typ] if isinstance(typ, str) else int(typ)
    for a in range(3):
        t.ne[a] = int(ne[a])
        t.nb[a] = int(nb[a])
    return t


def _storage(x: np.ndarray):
    """(contiguous storage array, byte offset of x[0,...]) for a permuted view x."""
    if x.flags.c_contiguous or x.size == 0:
        return x, 0
    perm = np.argsort([-s for s in x.strides], kind="stable")
    st = np.transpose(x, perm)
    if not st.flags.c_contiguous:
        raise ValueError("only permuted views of contiguous storage are supported")
    return st, 0


def _ggml(x: np.ndarray, typ: str, ne0: int):
    """ggml (ne, nb) of a logical numpy array (outer, mid, inner[bytes or values])."""
    a, b, c = x.shape
    s0, s1, s2 = x.strides
    nb0 = ELEM_BYTES[TYPE_IDS[typ]]
    if x.size == 0:   # numpy strides of an empty array are arbitrary: use contiguous ones
        s2 = x.itemsize
        s1 = max(c, 1) * s2
        s0 = max(b, 1) * s1
    if typ in BLOCK_TYPES:
        assert s2 == 1
    else:
        assert s2 == x.itemsize == nb0
    return (ne0, b, a), (nb0, s1, s0)


def describe(p) -> Desc:
    """Descriptor for a fa_inputs.Problem (numpy arrays in the ABI memory order)."""
    ds = Desc()
    ne, nb = _ggml(p.q, p.q_type, p.D)
    ds.q = make_tensor(p.q_type, ne, nb)
    ne, nb = _ggml(p.k, p.k_type, p.D)
    ds.k = make_tensor(p.k_type, ne, nb)
    ne, nb = _ggml(p.v, p.v_type, p.Dv)
    ds.v = make_tensor(p.v_type, ne, nb)
    ne, nb = _ggml(p.d, p.d_type, p.Dv)
    ds.d = make_tensor(p.d_type, ne, nb)
    if p.mask is None:
        ds.mask = make_tensor(NONE, (0, 0, 0), (0, 0, 0))
    elif p.mask_type == "causal_tail":
        # the array (kept for the CPU oracle) is not passed: the library forms the mask itself
        ds.mask = make_tensor(CAUSAL_TAIL, (p.M, p.N, 1), (0, 0, 0))
    else:
        ne, nb = _ggml(p.mask, p.mask_type, p.M)
        ds.mask = make_tensor(p.mask_type, ne, nb)
    ds.scale = float(p.scale)
    ds.flags = int(getattr(p, "flags", 0))
    return ds


# ----------------------------------------------------------------------------- torch helpers

def _to_device(x: np.ndarray, device):
    import torch
    st, _ = _storage(x)
    buf = torch.from_numpy(np.frombuffer(np.ascontiguousarray(st).tobytes(), dtype=np.uint8).copy())
    return buf.to(device)


class DeviceProblem:
    """A Problem's inputs resident in device memory (torch uint8 buffers), a plan, and
    the output/workspace buffers."""

    def __init__(self, p, device="cuda:0", poison: bool = True):
        import torch
        self.p = p
        self.device = torch.device(device)
        self.desc = describe(p)
        self.plan, self.layout = fa_back_create(self.desc, self.device.index or 0)
        self.bufs = {n: _to_device(getattr(p, n), self.device) for n in ("q", "k", "v", "d")}
        self.bufs["mask"] = (None if p.mask is None or p.mask_type == "causal_tail"
                             else _to_device(p.mask, self.device))
        self.out = torch.empty(int(self.layout.out_bytes), dtype=torch.uint8, device=self.device)
        self.ws = torch.empty(int(self.layout.workspace_bytes), dtype=torch.uint8, device=self.device)
        if poison:
            self.out.fill_(0xFF)   # NaN bytes: any defined byte left unwritten shows up
            self.ws.fill_(0xFF)

    def run(self, stream=None):
        import torch
        s = stream if stream is not None else torch.cuda.current_stream(self.device)
        m = self.bufs["mask"]
        fa_back_run(self.plan, self.bufs["q"].data_ptr(), self.bufs["k"].data_ptr(),
                    self.bufs["v"].data_ptr(), self.bufs["d"].data_ptr(),
                    None if m is None else m.data_ptr(), self.out.data_ptr(), self.ws.data_ptr(),
                    s.cuda_stream)

    def run_noalloc(self, stream=None):
        import torch
        s = stream if stream is not None else torch.cuda.current_stream(self.device)
        m = self.bufs["mask"]
        fa_back_run_noalloc(self.plan, self.bufs["q"].data_ptr(), self.bufs["k"].data_ptr(),
                            self.bufs["v"].data_ptr(), self.bufs["d"].data_ptr(),
                            None if m is None else m.data_ptr(), self.out.data_ptr(), s.cuda_stream)

    def run_timed(self, stream=None) -> list:
        import torch
        s = stream if stream is not None else torch.cuda.current_stream(self.device)
        m = self.bufs["mask"]
        return fa_back_run_timed(self.plan, self.bufs["q"].data_ptr(), self.bufs["k"].data_ptr(),
                                 self.bufs["v"].data_ptr(), self.bufs["d"].data_ptr(),
                                 None if m is None else m.data_ptr(), self.out.data_ptr(),
                                 self.ws.data_ptr(), s.cuda_stream)

    def run_saved(self, lse, o, stream=None, timed=False):
        """Run with saved statistics: lse and o are device tensors (float32, lse (H, N) and
        o (H, N, Dv), contiguous)."""
        import torch
        s = stream if stream is not None else torch.cuda.current_stream(self.device)
        m = self.bufs["mask"]
        return fa_back_run_saved(self.plan, self.bufs["q"].data_ptr(), self.bufs["k"].data_ptr(),
                                 self.bufs["v"].data_ptr(), self.bufs["d"].data_ptr(),
                                 None if m is None else m.data_ptr(), lse.data_ptr(), o.data_ptr(),
                                 self.out.data_ptr(), self.ws.data_ptr(), s.cuda_stream, timed)

    def outputs(self) -> dict:
        return unpack(self.out.cpu().numpy(), self.layout, self.p)

    def close(self):
        if self.plan:
            fa_back_destroy(self.plan)
            self.plan = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def unpack(raw: np.ndarray, lay: Layout, p) -> dict:
    """Split a packed output (bytes) into dq (H,N,D), dk (Hkv,M,D), dv (Hkv,M,Dv),
    lse (H,N), delta (H,N) float32 arrays."""
    def f32(off, n):
        return np.frombuffer(raw[off:off + 4 * n].tobytes(), dtype=np.float32)
    H, N, D, Dv, Hkv, M = p.H, p.N, p.D, p.Dv, p.Hkv, p.M
    return {
        "dq": f32(lay.off_dq, H * N * D).reshape(H, N, D),
        "dk": f32(lay.off_dk, Hkv * M * D).reshape(Hkv, M, D),
        "dv": f32(lay.off_dv, Hkv * M * Dv).reshape(Hkv, M, Dv),
        "lse": f32(lay.off_lse, H * N).reshape(H, N),
        "delta": f32(lay.off_delta, H * N).reshape(H, N),
    }


def defined_bytes(raw: np.ndarray, lay: Layout, p) -> np.ndarray:
    """The bytes of a packed output that the layout defines (for bitwise comparisons)."""
    H, N, D, Dv, Hkv, M = p.H, p.N, p.D, p.Dv, p.Hkv, p.M
    parts = [raw[lay.off_dq:lay.off_dq + 4 * H * N * D], raw[lay.off_dk:lay.off_dk + 4 * Hkv * M * D],
             raw[lay.off_dv:lay.off_dv + 4 * Hkv * M * Dv], raw[lay.off_lse:lay.off_lse + 8 * H * N]]
    return np.concatenate(parts)
