"""The benchmark's clock probe (libtsd_probe.so, built beside the attention library; not part of it or of
its C ABI): the shader clock and the bf16 matrix rate the GPU sustains when every SIMD issues nothing but
32x32x16 MFMAs on pseudo-random operands. The published peak assumes 2.4 GHz; under a data-carrying matrix
load the chip's power management holds the clock well below that, and this measures where."""
from __future__ import annotations

import ctypes
import os

_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libtsd_probe.so")
_lib = None


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_PATH):
            raise RuntimeError("libtsd_probe.so is not built; run `python -m transformer_scaled_dot_amd.build`")
        lib = ctypes.CDLL(_PATH)
        lib.tsd_probe_clock.argtypes = [ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p]
        lib.tsd_probe_clock.restype = ctypes.c_int
        _lib = lib
    return _lib


def clock_probe(device=None, spin_us: int = 2000) -> dict:
    """One workgroup of four waves per compute unit for ``spin_us`` of wall time (synchronises the device).
    Returns {"clock_mhz": mean shader clock, "tflops": bf16 32x32x16 flops issued / wall time}."""
    import torch

    device = torch.device("cuda", 0) if device is None else torch.device(device)
    blocks = torch.cuda.get_device_properties(device).multi_processor_count
    out = torch.zeros(3 * blocks, dtype=torch.int64, device=device)
    stream = torch.cuda.current_stream(device).cuda_stream
    st = _load().tsd_probe_clock(ctypes.c_void_p(out.data_ptr()), blocks, int(spin_us), ctypes.c_void_p(stream))
    if st != 0:
        raise RuntimeError("tsd_probe_clock failed with status %d" % st)
    v = out.view(blocks, 3).double().cpu()
    wall_s = float(v[:, 1].max()) / 100e6
    return {"clock_mhz": 100.0 * float(v[:, 0].sum()) / max(float(v[:, 1].sum()), 1.0),
            "tflops": 4 * 32 * 32 * 16 * 2 * float(v[:, 2].sum()) / max(wall_s, 1e-9) / 1e12}
