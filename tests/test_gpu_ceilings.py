"""GPU checks of the ceiling kernels the benchmark times (sv_ceilings.h).

sv_ceiling_read must read every 16-byte vector of its source exactly once: its
workgroups fold the words they read with XOR, so the XOR of all workgroups'
results equals the XOR of every word of the buffer (numpy), for whole 16 KB
chunks and a remainder, and for grids smaller and larger than the chunk count.
The MFMA and exp2 loops only have to produce finite values in their ranges.
"""
import numpy as np
import pytest
import torch

import speculative_decoding_verification_15_amd as sv

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("nbytes", [16384 * 40, 16384 * 40 + 16 * 37, 16 * 5])
@pytest.mark.parametrize("wgs", [1, 7, 64, 4096])
def test_read_ceiling_reads_every_vector_once(nbytes, wgs):
    rng = np.random.default_rng(nbytes + wgs)
    words = rng.integers(0, 2 ** 32, nbytes // 4, dtype=np.uint64).astype(np.uint32)
    src = torch.from_numpy(words.view(np.int32).copy()).cuda()
    sink = torch.full((wgs,), np.nan, dtype=torch.float32, device="cuda")
    sv.sv_ceiling_read(src, nbytes, wgs, sink)
    torch.cuda.synchronize()
    got = np.bitwise_xor.reduce(sink.cpu().numpy().view(np.uint32))
    assert got == np.bitwise_xor.reduce(words)


def test_mfma_and_exp2_ceilings_run():
    sink = torch.full((64 * 1024,), np.nan, dtype=torch.float32, device="cuda")
    sv.sv_ceiling_mfma_bf16(16, 8, sink)
    torch.cuda.synchronize()
    m = sink[:64].cpu().numpy()
    assert np.isfinite(m).all() and (m > 0).all()
    sv.sv_ceiling_exp2(16, 8, sink)
    torch.cuda.synchronize()
    e = sink[:16 * 256].cpu().numpy()          # each: the sum of 8 chains in [0.47, 1]
    assert np.isfinite(e).all() and ((e >= 8 * 0.47) & (e <= 8.0)).all()
