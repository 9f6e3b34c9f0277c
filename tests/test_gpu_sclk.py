"""Shader-clock probe (the measurement aid behind the bench's peak at the
measured clock): the clock under a sustained MFMA stream is a plausible
value, below the 2.4 GHz the published peak is quoted at plus a margin, and
a NULL output is rejected before anything runs."""

import pytest

pytestmark = pytest.mark.gpu


def test_sclk_probe():
    import torch
    from dynamic_block_sparse_macro_amd import binding as B
    lib = B.load_library()
    assert lib.prism_sclk_probe(None, None) == B.PRISM_EINVAL
    s = torch.cuda.current_stream()
    ghz = [B.prism_sclk_probe(s) for _ in range(3)]
    print("[sclk] GHz under MFMA load:", [round(x, 3) for x in ghz], flush=True)
    assert all(0.5 < x < 2.6 for x in ghz)
