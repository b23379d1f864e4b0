"""The roofline calibration probes (measurement only): the read-only stream
reads every byte once (its per-chunk XOR checksums equal numpy's), and the
MFMA-only loops run every data type to finite results."""

import numpy as np
import pytest
import torch

import quantized_gemm_group_amd as qg
from tests.gpu_util import device, host

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("chunks", [1, 7, 300])
def test_stream_read_checksums(chunks):
    dev = device()
    rng = np.random.default_rng(chunks)
    data = rng.integers(0, 2 ** 32, size=chunks * 16384, dtype=np.uint32)
    print(f"calib stream read {chunks} chunks", flush=True)
    got = host(qg.calib_stream_read(torch.from_numpy(data.view(np.int32)).to(dev)))
    want = np.bitwise_xor.reduce(data.reshape(chunks, 16384), axis=1)
    assert (got.view(np.uint32) == want).all()


@pytest.mark.parametrize("kind", ["bf16", "fp8", "fp4", "int8"])
def test_mfma_loop_runs(kind):
    dev = device()
    waves = 64
    out = torch.full((waves * 64,), float("nan"), dtype=torch.float32, device=dev)
    print(f"calib mfma {kind}", flush=True)
    got = host(qg.calib_mfma(kind, waves, 16, out))
    assert np.isfinite(got).all()
    assert (got != 0).mean() > 0.9
