"""ctypes binding of the benchmark's probe library (bench_probes/libmsa_probe.so):
a streaming read and the dense f16 MFMA issue rate, the two ceilings bench.py sets
the MSA kernels against.  Not part of libmsa."""
import ctypes
import os

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libmsa_probe.so")
SINK_WORDS = 4096          # MSA_PROBE_SINK_WORDS
_LIB = None


def _lib():
    global _LIB
    if _LIB is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built; run __graft_entry__.build()")
        import torch  # noqa: F401  (its HIP runtime first, as for libmsa)
        lib = ctypes.CDLL(LIB_PATH)
        vp = ctypes.c_void_p
        lib.msa_probe_stream_read.argtypes = [vp, ctypes.c_size_t, vp, vp]
        lib.msa_probe_mfma_f16.argtypes = [vp, ctypes.c_int32, ctypes.c_int32, vp]
        lib.msa_probe_stream_read.restype = lib.msa_probe_mfma_f16.restype = ctypes.c_int
        _LIB = lib
    return _LIB


def _stream(stream):
    if stream is not None:
        return stream
    import torch
    return torch.cuda.current_stream().cuda_stream


def stream_read(buf, sink, stream=None):
    """One streaming read of the device tensor `buf` (16-byte aligned, a multiple of 16 bytes)."""
    if sink.numel() * sink.element_size() < 4 * SINK_WORDS:
        raise ValueError("sink must hold 4096 uint32")
    st = _lib().msa_probe_stream_read(buf.data_ptr(), buf.numel() * buf.element_size(), sink.data_ptr(),
                                      _stream(stream))
    if st != 0:
        raise RuntimeError(f"msa_probe_stream_read: status {st}")


def mfma_f16(out, workgroups, iters, stream=None):
    """`iters` rounds of 16 independent 16x16x32 f16 MFMAs in every wave of `workgroups`
    4-wave workgroups; `out` holds workgroups * 256 floats."""
    if out.numel() < workgroups * 256:
        raise ValueError("out must hold workgroups * 256 floats")
    st = _lib().msa_probe_mfma_f16(out.data_ptr(), int(workgroups), int(iters), _stream(stream))
    if st != 0:
        raise RuntimeError(f"msa_probe_mfma_f16: status {st}")
