"""ctypes binding of libsubmconv.so: argument marshalling only.

Every function here has the name of the C entry point it calls.  Tensors are
device tensors; PyTorch supplies their memory (data_ptr) and the current HIP
stream.  No arithmetic of the method happens in Python, and there is no
fallback: when the shared library is missing, every call raises.
"""
from __future__ import annotations

import ctypes
import os
import threading

import torch

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "lib", "libsubmconv.so")

SUBM_F32, SUBM_F16, SUBM_BF16 = 0, 1, 2
SUBM_MAP_AUTO, SUBM_MAP_HASH, SUBM_MAP_GRID, SUBM_MAP_SUBDIVIDED = 0, 1, 2, 3
SUBM_POOL_MAX, SUBM_POOL_MEAN = 1, 2
SUBM_COARSE, SUBM_FINE, SUBM_PARENT = 0, 1, 2
SUBM_SUBDIVIDE, SUBM_DOWNSAMPLE, SUBM_UPSAMPLE_MASKED = 0, 1, 2
SUBM_ACT_NONE, SUBM_ACT_SILU, SUBM_ACT_RELU = 0, 1, 2
_DTYPE_CODES = {torch.float32: SUBM_F32, torch.float16: SUBM_F16, torch.bfloat16: SUBM_BF16}
TAPS = 27

# Exported C symbols (kept equal to the declarations in include/*.h).  Every one but the last
# two returns an int status.
C_FUNCTIONS = (
    "sparse_indice_map_build",
    "sparse_indice_map_build_ex",
    "sparse_indice_map_build_async",
    "sparse_indice_map_status",
    "sparse_indice_map_mode",
    "sparse_indice_map_free",
    "sparse_indice_map_info",
    "sparse_indice_map_offset_counts",
    "sparse_indice_map_copy_nbr",
    "sparse_indice_map_plan_state",
    "sparse_indice_map_row_order_state",
    "subm_release_cached_memory",
    "subm_timing_events",
    "subm_mfma_rate",
    "subm_conv3d_forward",
    "subm_conv3d_forward_noalloc",
    "subm_conv3d_forward_per_offset",
    "sparse_subdivide",
    "sparse_downsample_build",
    "sparse_upsample_masked_build",
    "sparse_subdivision_info",
    "sparse_subdivision_kind",
    "sparse_subdivision_coords",
    "sparse_subdivision_parent",
    "sparse_subdivision_copy",
    "sparse_subdivision_free",
    "sparse_downsample_forward",
    "sparse_upsample_forward",
    "sparse_indice_map_subdivide",
    "sparse_group_norm_act",
    "subm_conv3d_forward_group_norm_act",
    "subm_status_string",
    "subm_last_error",
)

_lib = None
_lib_lock = threading.Lock()


class SubmError(RuntimeError):
    """A non-zero status returned by the library."""

    def __init__(self, func: str, status: int, name: str, detail: str):
        super().__init__(f"{func} failed: {name} ({status}): {detail}")
        self.status = status
        self.name = name
        self.detail = detail


def load_library(path: str | None = None) -> ctypes.CDLL:
    """Load (once) and return the shared library.  Raises if it has not been built."""
    global _lib
    with _lib_lock:
        if _lib is not None and path is None:
            return _lib
        p = path or LIB_PATH
        if not os.path.exists(p):
            raise RuntimeError(
                f"HIP library not found at {p}; build it with "
                "`python -m submanifold_sparse_convolution_amd.build` (there is no CPU fallback)")
        lib = ctypes.CDLL(p)
        vp, i64, ci = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
        lib.sparse_indice_map_build.argtypes = [vp, i64, vp, ctypes.POINTER(vp)]
        lib.sparse_indice_map_build_ex.argtypes = [vp, i64, ci, vp, ctypes.POINTER(vp)]
        lib.sparse_indice_map_build_async.argtypes = [vp, i64, ci, vp, ctypes.POINTER(vp)]
        lib.sparse_indice_map_status.argtypes = [vp]
        lib.sparse_indice_map_mode.argtypes = [vp, ctypes.POINTER(ci)]
        lib.sparse_indice_map_free.argtypes = [vp]
        lib.sparse_indice_map_info.argtypes = [vp, ctypes.POINTER(i64), ctypes.POINTER(i64)]
        lib.sparse_indice_map_offset_counts.argtypes = [vp, ctypes.POINTER(i64)]
        lib.sparse_indice_map_copy_nbr.argtypes = [vp, vp, vp]
        lib.sparse_indice_map_plan_state.argtypes = [vp, ctypes.POINTER(ci)]
        lib.sparse_indice_map_row_order_state.argtypes = [vp, ctypes.POINTER(ci)]
        lib.subm_release_cached_memory.argtypes = []
        lib.subm_timing_events.argtypes = [vp, vp]
        lib.subm_mfma_rate.argtypes = [i64, ci, vp, vp, vp]
        lib.subm_conv3d_forward.argtypes = [vp, i64, ci, ci, ci, ci, vp, vp, vp, vp, vp]
        lib.subm_conv3d_forward_noalloc.argtypes = [vp, i64, ci, ci, ci, ci, vp, vp, vp, vp, vp]
        lib.subm_conv3d_forward_per_offset.argtypes = [vp, i64, ci, ci, ci, vp, vp, vp, vp, vp]
        lib.sparse_subdivide.argtypes = [vp, i64, vp, ctypes.POINTER(vp)]
        lib.sparse_downsample_build.argtypes = [vp, i64, vp, ctypes.POINTER(vp)]
        lib.sparse_upsample_masked_build.argtypes = [vp, vp, i64, vp, ctypes.POINTER(vp)]
        lib.sparse_subdivision_info.argtypes = [vp, ctypes.POINTER(i64), ctypes.POINTER(i64)]
        lib.sparse_subdivision_kind.argtypes = [vp, ctypes.POINTER(ci)]
        lib.sparse_subdivision_coords.argtypes = [vp, ci, ctypes.POINTER(vp)]
        lib.sparse_subdivision_parent.argtypes = [vp, ctypes.POINTER(vp)]
        lib.sparse_subdivision_copy.argtypes = [vp, ci, vp, vp]
        lib.sparse_subdivision_free.argtypes = [vp]
        lib.sparse_downsample_forward.argtypes = [vp, ci, ci, ci, vp, vp, vp]
        lib.sparse_upsample_forward.argtypes = [vp, ci, ci, vp, vp, vp]
        lib.sparse_indice_map_subdivide.argtypes = [vp, vp, vp, ctypes.POINTER(vp)]
        lib.sparse_group_norm_act.argtypes = [vp, i64, ci, ci, vp, ci, ci, vp, vp, ctypes.c_float, ci, vp, vp]
        lib.subm_conv3d_forward_group_norm_act.argtypes = [vp, i64, ci, ci, ci, ci, vp, vp, vp, vp, ci, ci, vp, vp,
                                                           ctypes.c_float, ci, vp, vp]
        for name in C_FUNCTIONS[:-2]:
            getattr(lib, name).restype = ci
        lib.subm_status_string.argtypes = [ci]
        lib.subm_status_string.restype = ctypes.c_char_p
        lib.subm_last_error.argtypes = []
        lib.subm_last_error.restype = ctypes.c_char_p
        if path is None:
            _lib = lib
        return lib


def _check(lib, func: str, status: int) -> None:
    if status != 0:
        name = lib.subm_status_string(status).decode()
        detail = lib.subm_last_error().decode()
        raise SubmError(func, status, name, detail)


_raw_stream = getattr(torch._C, "_cuda_getCurrentRawStream", None)


def _stream_ptr(stream, device) -> int:
    if stream is None:
        if _raw_stream is not None:  # the current stream's handle without building a Stream object
            return _raw_stream(device.index if device.index is not None else torch.cuda.current_device())
        return torch.cuda.current_stream(device).cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


class _Current:
    def __enter__(self):
        return None

    def __exit__(self, *exc):
        return False


_CURRENT = _Current()


def _on_device(device):
    """Make `device` current for a call, skipping the switch when it already is."""
    if device.index is None or device.index == torch.cuda.current_device():
        return _CURRENT
    return torch.cuda.device(device)


def _device_tensor(t: torch.Tensor, what: str) -> None:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{what} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{what} must be a device tensor (got {t.device})")
    if not t.is_contiguous():
        raise ValueError(f"{what} must be contiguous")


class IndiceMap:
    """Owner of one built indice map (submconv_map_t) for one coordinate set."""

    def __init__(self, handle: int, device: torch.device, n: int):
        self._handle = handle
        self.device = device
        self.n = n
        self._pairs = None

    @property
    def pairs(self) -> int:
        """Total pair count (rulebook entries >= 0, centre included)."""
        if self._pairs is None:
            self._pairs = sparse_indice_map_info(self)[1]
        return self._pairs

    @property
    def mode(self) -> int:
        """SUBM_MAP_HASH or SUBM_MAP_GRID: the structure the build used."""
        return sparse_indice_map_mode(self)

    @property
    def handle(self) -> int:
        if self._handle is None:
            raise ValueError("indice map already freed")
        return self._handle

    def check(self) -> None:
        """Raise the build's coordinate error, if any (waits for an asynchronous build's insert)."""
        sparse_indice_map_status(self)

    def free(self) -> None:
        """Release the map.  No work using it may still be in flight."""
        if self._handle is not None:
            lib = load_library()
            h, self._handle = self._handle, None
            _check(lib, "sparse_indice_map_free", lib.sparse_indice_map_free(h))

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        self.free()

    def __del__(self):
        try:
            self.free()
        except Exception:
            pass


def sparse_indice_map_build(coords: torch.Tensor, stream=None, sync: bool = True) -> IndiceMap:
    """Build the indice map of int32 device coordinates [N, 4] = (b, z, y, x).

    sync=False enqueues the build without any host wait (sparse_indice_map_build_async):
    coordinate errors are then raised by IndiceMap.check() or by the first call that reads the
    map on the host."""
    if not sync:
        return sparse_indice_map_build_async(coords, SUBM_MAP_AUTO, stream)
    return sparse_indice_map_build_ex(coords, SUBM_MAP_AUTO, stream)


def sparse_indice_map_build_async(coords: torch.Tensor, mode: int = SUBM_MAP_AUTO, stream=None) -> IndiceMap:
    """Enqueue the build with no host wait; see IndiceMap.check for its coordinate status."""
    return _build(coords, mode, stream, "sparse_indice_map_build_async")


def sparse_indice_map_status(m: IndiceMap) -> None:
    """Raise SubmError with the build's coordinate error, if any."""
    lib = load_library()
    _check(lib, "sparse_indice_map_status", lib.sparse_indice_map_status(m.handle))


def sparse_indice_map_build_ex(coords: torch.Tensor, mode: int, stream=None) -> IndiceMap:
    """Build the indice map with an explicit structure request (SUBM_MAP_AUTO / _HASH / _GRID)."""
    return _build(coords, mode, stream, "sparse_indice_map_build_ex")


def _build(coords: torch.Tensor, mode: int, stream, func: str) -> IndiceMap:
    _device_tensor(coords, "coords")
    if coords.dtype != torch.int32 or coords.dim() != 2 or coords.shape[1] != 4:
        raise ValueError("coords must be int32 [N, 4]")
    lib = load_library()
    out = ctypes.c_void_p()
    with _on_device(coords.device):
        st = getattr(lib, func)(coords.data_ptr(), coords.shape[0], int(mode), _stream_ptr(stream, coords.device),
                                ctypes.byref(out))
    _check(lib, func, st)
    return IndiceMap(out.value, coords.device, coords.shape[0])


def sparse_indice_map_mode(m: IndiceMap) -> int:
    lib = load_library()
    mode = ctypes.c_int()
    _check(lib, "sparse_indice_map_mode", lib.sparse_indice_map_mode(m.handle, ctypes.byref(mode)))
    return mode.value


SUBM_PLAN_NONE, SUBM_PLAN_PENDING, SUBM_PLAN_READY, SUBM_PLAN_OVERFLOW = 0, 1, 2, 3
SUBM_ORDER_NONE, SUBM_ORDER_ON, SUBM_ORDER_OFF = 0, 1, 2


def subm_release_cached_memory(device=None) -> None:
    """Free the library's cached device memory on `device` (default: torch's current device),
    after waiting for that device; see subm_release_cached_memory in include/submconv.h."""
    lib = load_library()
    dev = torch.device("cuda", torch.cuda.current_device()) if device is None else torch.device(device)
    with _on_device(dev):
        _check(lib, "subm_release_cached_memory", lib.subm_release_cached_memory())


def subm_timing_events(start, stop) -> None:
    """Bind two timing events (torch.cuda.Event, already recorded once so that they exist) to the
    next convolution kernel this thread launches: start.elapsed_time(stop) is then that kernel's
    own duration.  None, None cancels.  See subm_timing_events in include/submconv.h."""
    lib = load_library()
    h = lambda e: None if e is None else ctypes.c_void_p(e.cuda_event)
    _check(lib, "subm_timing_events", lib.subm_timing_events(h(start), h(stop)))


def subm_mfma_rate(iters: int, blocks: int, device=None, stream=None):
    """Launch the matrix-core rate loop (see subm_mfma_rate in include/submconv.h) on `stream`
    (default: torch's current stream).  Returns (sink, clocks) device tensors; the caller times
    the launch.  FLOP = blocks * 4 waves * iters * 8 * 32768."""
    lib = load_library()
    dev = torch.device("cuda", torch.cuda.current_device()) if device is None else torch.device(device)
    sink = torch.empty(blocks * 256, dtype=torch.float32, device=dev)
    clocks = torch.empty(2 * blocks, dtype=torch.int64, device=dev)
    s = torch.cuda.current_stream(dev) if stream is None else stream
    with _on_device(dev):
        _check(lib, "subm_mfma_rate", lib.subm_mfma_rate(int(iters), int(blocks), ctypes.c_void_p(sink.data_ptr()),
                                                           ctypes.c_void_p(clocks.data_ptr()),
                                                           ctypes.c_void_p(s.cuda_stream)))
    return sink, clocks


def sparse_indice_map_row_order_state(m: IndiceMap) -> int:
    """State of the map's sparse-row order: SUBM_ORDER_NONE / _ON / _OFF (waits for its kernels)."""
    lib = load_library()
    state = ctypes.c_int()
    _check(lib, "sparse_indice_map_row_order_state",
           lib.sparse_indice_map_row_order_state(m.handle, ctypes.byref(state)))
    return state.value


def sparse_indice_map_plan_state(m: IndiceMap) -> int:
    """State of the map's neighbour-pool plan: SUBM_PLAN_NONE / _PENDING / _READY / _OVERFLOW."""
    lib = load_library()
    state = ctypes.c_int()
    _check(lib, "sparse_indice_map_plan_state", lib.sparse_indice_map_plan_state(m.handle, ctypes.byref(state)))
    return state.value


def sparse_indice_map_free(m: IndiceMap) -> None:
    m.free()


def sparse_indice_map_info(m: IndiceMap) -> tuple[int, int]:
    """(voxel count, pair count) of a built map."""
    lib = load_library()
    n = ctypes.c_int64()
    pairs = ctypes.c_int64()
    _check(lib, "sparse_indice_map_info", lib.sparse_indice_map_info(m.handle, ctypes.byref(n), ctypes.byref(pairs)))
    return n.value, pairs.value


def sparse_indice_map_offset_counts(m: IndiceMap) -> list[int]:
    """Pairs per tap k (27 values)."""
    lib = load_library()
    arr = (ctypes.c_int64 * TAPS)()
    _check(lib, "sparse_indice_map_offset_counts", lib.sparse_indice_map_offset_counts(m.handle, arr))
    return list(arr)


def sparse_indice_map_copy_nbr(m: IndiceMap, out: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """The rulebook nbr [N, 27] int32 (input row of the neighbour, or -1) as a device tensor."""
    if out is None:
        out = torch.empty((m.n, TAPS), dtype=torch.int32, device=m.device)
    _device_tensor(out, "out")
    if out.dtype != torch.int32 or tuple(out.shape) != (m.n, TAPS):
        raise ValueError("out must be int32 [N, 27]")
    lib = load_library()
    with _on_device(out.device):
        st = lib.sparse_indice_map_copy_nbr(m.handle, out.data_ptr(), _stream_ptr(stream, out.device))
    _check(lib, "sparse_indice_map_copy_nbr", st)
    return out


def _conv_args(feats, weight, bias, out, need_out=False):
    _device_tensor(feats, "feats")
    _device_tensor(weight, "weight")
    if feats.dim() != 2 or weight.dim() != 5:
        raise ValueError("feats must be [N, Cin] and weight KRSC [Cout, k, k, k, Cin]")
    k = weight.shape[1]
    if weight.shape[2] != k or weight.shape[3] != k:
        raise ValueError("weight spatial dims must be equal (KRSC [Cout, k, k, k, Cin])")
    if weight.shape[4] != feats.shape[1]:
        raise ValueError("weight Cin does not match feats")
    if feats.dtype not in _DTYPE_CODES or weight.dtype != feats.dtype:
        raise ValueError("feats and weight must share one of float32 / float16 / bfloat16")
    n, cout = feats.shape[0], weight.shape[0]
    bias_ptr = None
    if bias is not None:
        _device_tensor(bias, "bias")
        if bias.dtype != feats.dtype or tuple(bias.shape) != (cout,):
            raise ValueError("bias must be [Cout] in the feats dtype")
        bias_ptr = bias.data_ptr()
    if out is None:
        if need_out:
            raise ValueError("out must be given (this call allocates nothing)")
        out = torch.empty((n, cout), dtype=feats.dtype, device=feats.device)
    _device_tensor(out, "out")
    if out.dtype != feats.dtype or tuple(out.shape) != (n, cout):
        raise ValueError("out must be [N, Cout] in the feats dtype")
    return k, bias_ptr, out


def subm_conv3d_forward_per_offset(m: IndiceMap, feats: torch.Tensor, weight: torch.Tensor,
                                   bias: torch.Tensor | None = None, out: torch.Tensor | None = None,
                                   stream=None) -> torch.Tensor:
    """SubMConv3d (k = 3) computed as a per-offset gather -> GEMM -> scatter-add loop."""
    k, bias_ptr, out = _conv_args(feats, weight, bias, out)
    if k != 3:
        raise ValueError("the per-offset path is the k = 3 convolution")
    lib = load_library()
    with _on_device(feats.device):
        st = lib.subm_conv3d_forward_per_offset(m.handle, feats.shape[0], feats.shape[1], weight.shape[0],
                                                _DTYPE_CODES[feats.dtype], feats.data_ptr(), weight.data_ptr(),
                                                bias_ptr, out.data_ptr(), _stream_ptr(stream, feats.device))
    _check(lib, "subm_conv3d_forward_per_offset", st)
    return out


def subm_conv3d_forward(m: IndiceMap | None, feats: torch.Tensor, weight: torch.Tensor,
                        bias: torch.Tensor | None = None, out: torch.Tensor | None = None,
                        stream=None) -> torch.Tensor:
    """SubMConv3d forward: feats [N, Cin], KRSC weight [Cout, k, k, k, Cin] (k = 3 or 1), bias [Cout]."""
    k, bias_ptr, out = _conv_args(feats, weight, bias, out)
    n, cin, cout = feats.shape[0], feats.shape[1], weight.shape[0]
    lib = load_library()
    handle = None if m is None else m.handle
    with _on_device(feats.device):
        st = lib.subm_conv3d_forward(handle, n, k, cin, cout, _DTYPE_CODES[feats.dtype], feats.data_ptr(),
                                     weight.data_ptr(), bias_ptr, out.data_ptr(), _stream_ptr(stream, feats.device))
    _check(lib, "subm_conv3d_forward", st)
    return out


def subm_conv3d_forward_noalloc(m: IndiceMap | None, feats: torch.Tensor, weight: torch.Tensor,
                                bias: torch.Tensor | None, out: torch.Tensor, stream=None) -> torch.Tensor:
    """subm_conv3d_forward with no device allocation (out must be given); see subm_conv3d_forward_noalloc
    in include/submconv.h."""
    k, bias_ptr, out = _conv_args(feats, weight, bias, out, need_out=True)
    n, cin, cout = feats.shape[0], feats.shape[1], weight.shape[0]
    lib = load_library()
    handle = None if m is None else m.handle
    with _on_device(feats.device):
        st = lib.subm_conv3d_forward_noalloc(handle, n, k, cin, cout, _DTYPE_CODES[feats.dtype], feats.data_ptr(),
                                             weight.data_ptr(), bias_ptr, out.data_ptr(),
                                             _stream_ptr(stream, feats.device))
    _check(lib, "subm_conv3d_forward_noalloc", st)
    return out


# --------------------------------------------------------------------------- structure ops

class Subdivision:
    """Owner of one coarse / fine relation (sparse_subdivision_t): subdivide, downsample or masked
    upsample structure."""

    def __init__(self, handle: int, device: torch.device):
        self._handle = handle
        self.device = device
        self.n_coarse, self.n_fine = sparse_subdivision_info(self)
        self.kind = sparse_subdivision_kind(self)

    @property
    def handle(self) -> int:
        if self._handle is None:
            raise ValueError("subdivision already freed")
        return self._handle

    def coarse_coords(self, stream=None) -> torch.Tensor:
        return sparse_subdivision_copy(self, SUBM_COARSE, stream=stream)

    def fine_coords(self, stream=None) -> torch.Tensor:
        return sparse_subdivision_copy(self, SUBM_FINE, stream=stream)

    def parent(self, stream=None) -> torch.Tensor:
        return sparse_subdivision_copy(self, SUBM_PARENT, stream=stream)

    def free(self) -> None:
        if self._handle is not None:
            lib = load_library()
            h, self._handle = self._handle, None
            _check(lib, "sparse_subdivision_free", lib.sparse_subdivision_free(h))

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        self.free()

    def __del__(self):
        try:
            self.free()
        except Exception:
            pass


def _coords_arg(coords: torch.Tensor) -> None:
    _device_tensor(coords, "coords")
    if coords.dtype != torch.int32 or coords.dim() != 2 or coords.shape[1] != 4:
        raise ValueError("coords must be int32 [N, 4]")


def _build_subdivision(func: str, coords: torch.Tensor, args: tuple, stream) -> Subdivision:
    lib = load_library()
    out = ctypes.c_void_p()
    with _on_device(coords.device):
        st = getattr(lib, func)(*args, _stream_ptr(stream, coords.device), ctypes.byref(out))
    _check(lib, func, st)
    return Subdivision(out.value, coords.device)


def sparse_subdivide(coords: torch.Tensor, stream=None) -> Subdivision:
    """The 8 children of every voxel of int32 [N, 4] (b, z, y, x), C order, parent-major."""
    _coords_arg(coords)
    return _build_subdivision("sparse_subdivide", coords, (coords.data_ptr(), coords.shape[0]), stream)


def sparse_downsample_build(coords: torch.Tensor, stream=None) -> Subdivision:
    """The 2x coarse cells of int32 [N, 4] coordinates and the fine-to-coarse relation."""
    _coords_arg(coords)
    return _build_subdivision("sparse_downsample_build", coords, (coords.data_ptr(), coords.shape[0]), stream)


def sparse_upsample_masked_build(coords: torch.Tensor, mask: torch.Tensor, stream=None) -> Subdivision:
    """Masked 2x expansion of int32 [N, 4] coordinates by a uint8 [N, 8] child mask."""
    _coords_arg(coords)
    _device_tensor(mask, "mask")
    if mask.dtype != torch.uint8 or tuple(mask.shape) != (coords.shape[0], 8):
        raise ValueError("mask must be uint8 [N, 8]")
    return _build_subdivision("sparse_upsample_masked_build", coords,
                              (coords.data_ptr(), mask.data_ptr(), coords.shape[0]), stream)


def sparse_subdivision_info(s: Subdivision) -> tuple[int, int]:
    """(n_coarse, n_fine)."""
    lib = load_library()
    a, b = ctypes.c_int64(), ctypes.c_int64()
    _check(lib, "sparse_subdivision_info", lib.sparse_subdivision_info(s.handle, ctypes.byref(a), ctypes.byref(b)))
    return a.value, b.value


def sparse_subdivision_kind(s: Subdivision) -> int:
    lib = load_library()
    k = ctypes.c_int()
    _check(lib, "sparse_subdivision_kind", lib.sparse_subdivision_kind(s.handle, ctypes.byref(k)))
    return k.value


def sparse_subdivision_coords(s: Subdivision, level: int) -> int:
    """Raw device address of the handle-owned coarse / fine coordinates (0 when empty)."""
    lib = load_library()
    p = ctypes.c_void_p()
    _check(lib, "sparse_subdivision_coords", lib.sparse_subdivision_coords(s.handle, int(level), ctypes.byref(p)))
    return p.value or 0


def sparse_subdivision_parent(s: Subdivision) -> int:
    """Raw device address of the handle-owned parent index (0 when empty)."""
    lib = load_library()
    p = ctypes.c_void_p()
    _check(lib, "sparse_subdivision_parent", lib.sparse_subdivision_parent(s.handle, ctypes.byref(p)))
    return p.value or 0


def sparse_subdivision_copy(s: Subdivision, what: int, out: torch.Tensor | None = None,
                            stream=None) -> torch.Tensor:
    """Copy of the coarse coords (SUBM_COARSE), fine coords (SUBM_FINE) or parent index (SUBM_PARENT)."""
    shape = {SUBM_COARSE: (s.n_coarse, 4), SUBM_FINE: (s.n_fine, 4), SUBM_PARENT: (s.n_fine,)}
    if what not in shape:
        raise ValueError("what must be SUBM_COARSE, SUBM_FINE or SUBM_PARENT")
    if out is None:
        out = torch.empty(shape[what], dtype=torch.int32, device=s.device)
    _device_tensor(out, "out")
    if out.dtype != torch.int32 or tuple(out.shape) != shape[what]:
        raise ValueError(f"out must be int32 {shape[what]}")
    lib = load_library()
    with _on_device(out.device):
        st = lib.sparse_subdivision_copy(s.handle, int(what), out.data_ptr(), _stream_ptr(stream, out.device))
    _check(lib, "sparse_subdivision_copy", st)
    return out


def sparse_subdivision_free(s: Subdivision) -> None:
    s.free()


def _feature_pair(inp: torch.Tensor, rows_in: int, out: torch.Tensor | None, rows_out: int, what: str):
    _device_tensor(inp, what)
    if inp.dim() != 2 or inp.shape[0] != rows_in or inp.dtype not in _DTYPE_CODES:
        raise ValueError(f"{what} must be [{rows_in}, C] float32 / float16 / bfloat16")
    if out is None:
        out = torch.empty((rows_out, inp.shape[1]), dtype=inp.dtype, device=inp.device)
    _device_tensor(out, "out")
    if out.dtype != inp.dtype or tuple(out.shape) != (rows_out, inp.shape[1]):
        raise ValueError(f"out must be [{rows_out}, {inp.shape[1]}] in the input dtype")
    return out


def sparse_downsample_forward(s: Subdivision, fine: torch.Tensor, mode: int, out: torch.Tensor | None = None,
                              stream=None) -> torch.Tensor:
    """Pool fine features [n_fine, C] onto the coarse rows: mode SUBM_POOL_MAX or SUBM_POOL_MEAN."""
    out = _feature_pair(fine, s.n_fine, out, s.n_coarse, "fine")
    lib = load_library()
    with _on_device(fine.device):
        st = lib.sparse_downsample_forward(s.handle, fine.shape[1], _DTYPE_CODES[fine.dtype], int(mode),
                                           fine.data_ptr(), out.data_ptr(), _stream_ptr(stream, fine.device))
    _check(lib, "sparse_downsample_forward", st)
    return out


def sparse_upsample_forward(s: Subdivision, coarse: torch.Tensor, out: torch.Tensor | None = None,
                            stream=None) -> torch.Tensor:
    """Fine features [n_fine, C]: every fine row a copy of its parent's coarse row."""
    out = _feature_pair(coarse, s.n_coarse, out, s.n_fine, "coarse")
    lib = load_library()
    with _on_device(coarse.device):
        st = lib.sparse_upsample_forward(s.handle, coarse.shape[1], _DTYPE_CODES[coarse.dtype], coarse.data_ptr(),
                                         out.data_ptr(), _stream_ptr(stream, coarse.device))
    _check(lib, "sparse_upsample_forward", st)
    return out


def sparse_indice_map_subdivide(parent: IndiceMap, s: Subdivision, stream=None) -> IndiceMap:
    """Indice map of a subdivide's fine set, derived from the map of its coarse set."""
    lib = load_library()
    out = ctypes.c_void_p()
    with _on_device(s.device):
        st = lib.sparse_indice_map_subdivide(parent.handle, s.handle, _stream_ptr(stream, s.device),
                                             ctypes.byref(out))
    _check(lib, "sparse_indice_map_subdivide", st)
    return IndiceMap(out.value, s.device, s.n_fine)


# --------------------------------------------------------------------------- normalisation

def _norm_affine(c, dtype, gamma, beta):
    ptrs = []
    for t, name in ((gamma, "gamma"), (beta, "beta")):
        if t is None:
            ptrs.append(None)
            continue
        _device_tensor(t, name)
        if t.dtype != dtype or tuple(t.shape) != (c,):
            raise ValueError(f"{name} must be [C] in the activation dtype")
        ptrs.append(t.data_ptr())
    return ptrs


def _offsets_arg(item_offsets):
    _device_tensor(item_offsets, "item_offsets")
    if item_offsets.dtype != torch.int64 or item_offsets.dim() != 1 or item_offsets.shape[0] < 2:
        raise ValueError("item_offsets must be int64 [num_items + 1]")


def subm_conv3d_forward_group_norm_act(m: IndiceMap | None, feats: torch.Tensor, weight: torch.Tensor,
                                       bias: torch.Tensor | None, item_offsets: torch.Tensor, groups: int,
                                       gamma: torch.Tensor | None = None, beta: torch.Tensor | None = None,
                                       eps: float = 1e-5, act: int = SUBM_ACT_NONE,
                                       out: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """act(group_norm(SubMConv3d(feats))) with the group statistics taken in the conv epilogue."""
    k, bias_ptr, out = _conv_args(feats, weight, bias, out)
    _offsets_arg(item_offsets)
    ptrs = _norm_affine(weight.shape[0], feats.dtype, gamma, beta)
    lib = load_library()
    handle = None if m is None else m.handle
    with _on_device(feats.device):
        st = lib.subm_conv3d_forward_group_norm_act(
            handle, feats.shape[0], k, feats.shape[1], weight.shape[0], _DTYPE_CODES[feats.dtype], feats.data_ptr(),
            weight.data_ptr(), bias_ptr, item_offsets.data_ptr(), item_offsets.shape[0] - 1, int(groups), ptrs[0],
            ptrs[1], float(eps), int(act), out.data_ptr(), _stream_ptr(stream, feats.device))
    _check(lib, "subm_conv3d_forward_group_norm_act", st)
    return out


def sparse_group_norm_act(x: torch.Tensor, item_offsets: torch.Tensor, groups: int,
                          gamma: torch.Tensor | None = None, beta: torch.Tensor | None = None,
                          eps: float = 1e-5, act: int = SUBM_ACT_NONE, out: torch.Tensor | None = None,
                          stream=None) -> torch.Tensor:
    """Group normalisation per batch item (rows item_offsets[b] .. item_offsets[b+1] - 1, int64
    device tensor) then an activation (SUBM_ACT_NONE / _SILU / _RELU).  out may be x (in place)."""
    _device_tensor(x, "x")
    if x.dim() != 2 or x.dtype not in _DTYPE_CODES:
        raise ValueError("x must be [N, C] float32 / float16 / bfloat16")
    _offsets_arg(item_offsets)
    c = x.shape[1]
    ptrs = _norm_affine(c, x.dtype, gamma, beta)
    if out is None:
        out = torch.empty_like(x)
    _device_tensor(out, "out")
    if out.dtype != x.dtype or out.shape != x.shape:
        raise ValueError("out must match x")
    lib = load_library()
    with _on_device(x.device):
        st = lib.sparse_group_norm_act(x.data_ptr(), x.shape[0], c, _DTYPE_CODES[x.dtype], item_offsets.data_ptr(),
                                       item_offsets.shape[0] - 1, int(groups), ptrs[0], ptrs[1], float(eps), int(act),
                                       out.data_ptr(), _stream_ptr(stream, x.device))
    _check(lib, "sparse_group_norm_act", st)
    return out
