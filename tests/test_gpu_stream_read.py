"""GPU check of pa_stream_read, the measurement's achievable-read line: the
XOR of its per-workgroup partials equals the XOR of every 32-bit word of the
buffer (computed on the host), for sizes from one 16-byte chunk (one
workgroup reads, the rest write a zero partial) to ranges that end inside a
workgroup's unrolled step, and it writes nothing else."""

import numpy as np
import pytest
import torch

import paged_kv_cache_313_amd as P
from paged_kv_cache_313_amd import _lib

pytestmark = pytest.mark.gpu

STEP_BYTES = _lib.PA_STREAM_READ_PARTIALS * 256 * 8 * 16   # every workgroup one full unrolled step


@pytest.mark.parametrize("nbytes", [16, 4096, 16 * 1000 + 16, 64 << 20, STEP_BYTES - 16,
                                    STEP_BYTES + 48])
def test_stream_read_xor(nbytes):
    print(f"stream_read {nbytes} B", flush=True)
    rng = np.random.default_rng(nbytes)
    host = rng.integers(0, 2**32, size=nbytes // 4, dtype=np.uint32)
    buf = torch.from_numpy(host.view(np.int32)).cuda()
    partials = torch.full((_lib.PA_STREAM_READ_PARTIALS + 8,), -1, dtype=torch.int32, device="cuda")
    P.stream_read(buf, partials)
    torch.cuda.synchronize()
    got = partials.cpu().numpy().view(np.uint32)
    assert np.bitwise_xor.reduce(got[:_lib.PA_STREAM_READ_PARTIALS]) == np.bitwise_xor.reduce(host)
    assert (got[_lib.PA_STREAM_READ_PARTIALS:] == np.uint32(0xFFFFFFFF)).all()   # nothing past the partials
