"""GPU parity of the audio-to-video norm producer (prism_a2v_norms, the
per-token a_n = |h-hat_n|_2 of Prism guide (pt), Método 1) against the
oracle's float64 norms, through the C ABI: the float32 result must be the
oracle's value rounded to nearest (either neighbour within 1e-12 of a
rounding midpoint)."""

import numpy as np
import pytest

import oracle as O
from workload import CONFIGS, a2v_output, bf16_bits_to_f32, bf16_round, generate

from parity_utils import check_f32_rounding, log

pytestmark = pytest.mark.gpu


def _run(bits: np.ndarray, channels: int, n: int | None = None):
    import torch
    from dynamic_block_sparse_macro_amd import binding as B
    N, stride = bits.shape
    n = N if n is None else n
    h = torch.from_numpy(bits.view(np.int16)).cuda()
    a = torch.full((N,), -1.0, dtype=torch.float32, device="cuda")
    B.prism_a2v_norms(h, n, channels, stride, a, stream=torch.cuda.current_stream())
    torch.cuda.synchronize()
    return a.cpu().numpy()


def _ref(bits: np.ndarray, channels: int):
    return O.a2v_norms(bf16_bits_to_f32(bits[:, :channels]))


# (workload, channels, row stride): every lane-group width, a ragged chunk
# tail, padded rows, and the tiny workload's own h-hat
CASES = [("tiny", 64, 64), ("tiny", 8, 8), ("tiny", 24, 32), ("par_d64", 40, 48), ("par_small", 256, 264),
         ("par_cap", 512, 512), ("par_d64", 1544, 1552), ("one_zone", 3072, 3072)]


@pytest.mark.parametrize("name,channels,stride", CASES)
def test_a2v_norms(name, channels, stride):
    wl = generate(name)
    bits = a2v_output(wl, channels, stride)
    got = _run(bits, channels)
    ties = check_f32_rounding(got, _ref(bits, channels))
    log(f"{name}: {wl.cfg.N} rows x {channels} channels (stride {stride}): rounding ties taken the other way {ties}")


def test_a2v_norms_tiny_h_hat():
    """The tiny workload's own h-hat (whose norms are its audio map)."""
    wl = generate("tiny")
    bits = bf16_round(wl.h_hat)
    got = _run(bits, bits.shape[1])
    check_f32_rounding(got, _ref(bits, bits.shape[1]))
    np.testing.assert_allclose(got, wl.a, rtol=1e-2)


def test_a2v_norms_partial_rows():
    """n_tokens below the buffer's rows: later rows are not written; ragged
    row counts against the rows each workgroup covers."""
    wl = generate("par_small")
    bits = a2v_output(wl, 256)
    for n in (1, 7, 129, 1000):
        got = _run(bits, 256, n)
        check_f32_rounding(got[:n], _ref(bits[:n], 256))
        assert (got[n:] == -1.0).all()


@pytest.mark.slow
def test_a2v_norms_fullsize():
    """The 2K clip's 450,560 tokens at 256 channels (one GPU's two heads of
    128), every row, in the benchmark's launch configuration."""
    wl = generate(CONFIGS["2k"])
    bits = a2v_output(wl, 256)
    got = _run(bits, 256)
    ties = check_f32_rounding(got, _ref(bits, 256))
    log(f"2k: ties taken the other way {ties}")
