"""GPU checks of the benchmark's unit-rate probes (the matrix product and
LDS read kernels the floor record reports): they run, read what they claim to
read, and report cycle counts."""
import numpy as np
import pytest

from tests.gpu_helpers import log

pytestmark = pytest.mark.gpu


def _need_gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def test_lds_read_probe_reads_the_filled_words():
    _need_gpu()
    import torch
    import split_kv_amd as sk
    wgs, iters = 4, 3
    sink = torch.zeros(8 * wgs, dtype=torch.int32, device="cuda")
    log("calib lds read, 4 workgroups, 3 rounds")
    sk.splitkv_calib_lds_read(wgs, iters, 0, sink.data_ptr())
    torch.cuda.synchronize()
    got = sink.view(-1, 2).cpu().numpy().astype(np.uint32)
    # word i of the 64 KiB holds (i, 3i, 5i, 7i); wave w reads, in round it
    # and read j, lane l: word ((16 it + j + 4 w) * 64 + l) mod 4096
    i = np.arange(4096, dtype=np.uint64)
    word = ((i ^ (3 * i) ^ (5 * i) ^ (7 * i)) & 0xffffffff).astype(np.uint32)
    for w in range(4):
        idx = [((16 * it + j + 4 * w) * 64 + lane) % 4096 for it in range(iters) for j in range(16)
               for lane in range(64)]
        want = np.bitwise_xor.reduce(word[idx])
        for g in range(wgs):
            assert got[4 * g + w, 0] == want, (g, w)
            assert got[4 * g + w, 1] > 0


def test_mfma_and_transposing_probes_are_deterministic():
    _need_gpu()
    import torch
    import split_kv_amd as sk
    wgs = 8
    outs = []
    for _ in range(2):
        a = torch.zeros(8 * wgs, dtype=torch.int32, device="cuda")
        b = torch.zeros(8 * wgs, dtype=torch.int32, device="cuda")
        log("calib mfma and transposing lds read, 8 workgroups")
        sk.splitkv_calib_mfma(wgs, 64, a.data_ptr())
        sk.splitkv_calib_lds_read(wgs, 5, 1, b.data_ptr())
        torch.cuda.synchronize()
        outs.append((a.view(-1, 2).cpu().numpy(), b.view(-1, 2).cpu().numpy()))
    for k in range(2):
        assert np.array_equal(outs[0][k][:, 0], outs[1][k][:, 0])
        assert (outs[0][k][:, 1] != 0).all()
    # every wave of the matrix probe runs the same products
    assert (outs[0][0][:, 0] == outs[0][0][0, 0]).all()
