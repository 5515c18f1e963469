"""The streaming-read probe (measurement support for the bench) reads every word of its buffer
exactly once: the XOR of its per-thread sink words equals the XOR of the buffer's words, for each
depth of loads in flight, grid sizes below and above the block count, and a ragged tail."""
import ctypes

import numpy as np
import pytest

pytestmark = pytest.mark.gpu


def _lib():
    from compressed_kv_attention_kvexec_amd import build as hipbuild
    lib = ctypes.CDLL(hipbuild.PROBE_LIB)
    lib.tq4_probe_sink_words.argtypes = [ctypes.c_int32]
    lib.tq4_probe_sink_words.restype = ctypes.c_size_t
    lib.tq4_probe_stream_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_int32,
                                          ctypes.c_int32, ctypes.c_void_p]
    lib.tq4_probe_stream_read.restype = ctypes.c_int
    return lib


@pytest.mark.parametrize("loads", [4, 8, 16])
@pytest.mark.parametrize("workgroups", [1, 3, 64])
def test_probe_reads_every_word_once(loads, workgroups):
    import torch
    lib = _lib()
    rng = np.random.default_rng(1000 * loads + workgroups)
    # 37 blocks of the deepest probe plus 5 16-byte words of tail
    n_words = 4 * (512 * 16 * 37 + 5)
    host = rng.integers(0, 2**32, size=n_words, dtype=np.uint64).astype(np.uint32)
    x = torch.from_numpy(host.view(np.int32)).cuda()
    sink = torch.full((lib.tq4_probe_sink_words(workgroups),), -1, dtype=torch.int32, device="cuda")
    rc = lib.tq4_probe_stream_read(ctypes.c_void_p(x.data_ptr()), n_words * 4, ctypes.c_void_p(sink.data_ptr()),
                                   workgroups, loads, None)
    assert rc == 0
    torch.cuda.synchronize()
    got = np.bitwise_xor.reduce(sink.cpu().numpy().view(np.uint32))
    assert int(got) == int(np.bitwise_xor.reduce(host))


def test_probe_rejects_bad_arguments():
    lib = _lib()
    assert lib.tq4_probe_stream_read(None, 64, None, 1, 8, None) == -1
    assert lib.tq4_probe_sink_words(0) == 0
