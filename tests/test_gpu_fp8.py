"""FP8 projection on the GPU: E4M3 codes and scales bit-exact against the
oracle's quantization (the same fp32 scale and quotient, round to nearest
even)."""
import numpy as np
import pytest

import synth
from tests import harness as H

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def torch():
    import torch
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible")
    return torch


def _quantize(torch, x):
    import hashed_gram_embedding_canon_amd as eg
    rows, cols = x.shape
    codes = torch.empty(rows, cols, dtype=torch.uint8, device="cuda")
    scales = torch.empty(rows, dtype=torch.float32, device="cuda")
    dt = eg.ENGRAM_BF16 if x.dtype == np.uint16 else eg.ENGRAM_F32
    eg.engram_quantize_fp8(H.to_dev(x), dt, rows, cols, codes, scales)
    torch.cuda.synchronize()
    return codes.cpu().numpy(), scales.cpu().numpy()


def test_quantize_matches_oracle(torch, oracle_lib):
    w = synth.normal_stream(11, 512 * 256, 0.05, "bf16").reshape(512, 256)
    # fp32 rows spanning many binades, so that many quotients are E4M3 subnormals
    u = synth.unit_stream(12, 64 * 1024).reshape(64, 1024)
    x = ((u * 2 - 1) * np.exp2(np.floor(synth.unit_stream(13, 64 * 1024) * 40) - 30).reshape(64, 1024)).astype(np.float32)
    x[5] = 0.0
    x[6] = 1e-3
    x[6, 17] = 3e4
    for arr in (w, x):
        codes, scales = _quantize(torch, arr)
        rc, rs, _ = oracle_lib.quantize_rows(arr)
        assert np.array_equal(scales, rs)
        mism = np.argwhere(codes != rc)
        assert mism.size == 0, (mism[:5], codes[tuple(mism[0])], rc[tuple(mism[0])])
