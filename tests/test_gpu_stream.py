"""The read-ceiling hook: it reads every byte once (the XOR of its sink words
is the XOR of the buffer's 32-bit words, computed on the host) for sizes that
take one partial workgroup, several, and more vectors than the 8192-workgroup
grid covers in one pass, in both of its shapes (1 and 8 loads a thread)."""
import numpy as np
import pytest
import torch

import synth

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def m():
    import nvfp4_moe_skinny_amd as m
    return m


@pytest.mark.parametrize("nbytes", [16, 48, 4096, 4096 + 16, 9216 * 7, 1 << 20,
                                    8192 * 4096 * 2 + 4096 * 16 + 16,  # one vector a thread
                                    (512 << 20) + 4096 * 16 + 16])     # eight a thread
def test_stream_read_xor(m, gpu, nbytes):
    host = synth.uniform_bytes(synth.key(0, 400, nbytes), nbytes)
    src = torch.from_numpy(host).to(gpu)
    sink = m.nvfp4moe_stream_read(src)
    torch.cuda.synchronize()
    assert sink.numel() == m.nvfp4moe_stream_blocks(nbytes)
    got = np.bitwise_xor.reduce(sink.cpu().numpy().view(np.uint32))
    want = np.bitwise_xor.reduce(host.view(np.uint32))
    assert int(got) == int(want)
