"""The read-bandwidth probe streams every byte it is given: the XOR of its
per-workgroup words equals the XOR of the buffer's 32-bit words (numpy on
the host), for empty, tiny, ragged and multi-pass sizes."""
import sys

import numpy as np
import pytest
import torch

import decode_attention_kvc_amd as kvc

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.mark.parametrize("nbytes", [0, 16, 48, 16 * 1000, (64 << 20) + 48])
def test_read_probe_reads_every_word(nbytes):
    print("read probe", nbytes, file=sys.stderr, flush=True)
    g = torch.Generator(device="cpu").manual_seed(nbytes)
    host = torch.randint(-2**31, 2**31 - 1, (nbytes // 4,), dtype=torch.int32, generator=g)
    buf = host.to(DEV)
    out = torch.full((kvc.PROBE_BLOCKS,), 7, dtype=torch.int32, device=DEV)
    kvc.kvc_read_probe(buf, out)
    torch.cuda.synchronize()
    got = np.bitwise_xor.reduce(out.cpu().numpy().view(np.uint32))
    want = np.bitwise_xor.reduce(host.numpy().view(np.uint32)) if nbytes else np.uint32(0)
    assert got == want
