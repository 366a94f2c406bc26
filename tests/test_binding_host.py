"""Host-side tests of the Python binding's argument checks and of the GPU
tests' tolerance rule (no GPU needed; no kernel is launched).

The C ABI takes plain pointers and cannot see buffer sizes, so the binding
must reject every caller-supplied output or workspace that is short,
mistyped, on another device or not contiguous before it reaches the library.
Tensors on torch's "meta" device stand in for device tensors here: they carry
shape, dtype, device and strides without memory.
"""
import numpy as np
import pytest
import torch

import datagen
import invariant_token_log_fp32_amd as rlk
from gpu_util import ORDINARY_MAX_Z, TOL, row_tolerance

META = torch.device("meta")


def test_output_check_accepts_exact_outputs():
    a = torch.empty(7, dtype=torch.float32, device=META)
    assert rlk._out(a, (7,), torch.float32, META, "out") is a
    s = torch.empty((7, 4), dtype=torch.int32, device=META)
    assert rlk._out(s, (7, 4), torch.int32, META, "state_out") is s
    new = rlk._out(None, (5,), torch.float32, META, "out")
    assert new.shape == (5,) and new.dtype == torch.float32


@pytest.mark.parametrize("bad", [
    torch.empty(6, dtype=torch.float32, device=META),                 # short
    torch.empty(8, dtype=torch.float32, device=META),                 # long
    torch.empty(7, dtype=torch.float64, device=META),                 # wrong dtype
    torch.empty(7, dtype=torch.float32),                              # other device
    torch.empty(14, dtype=torch.float32, device=META)[::2],           # not contiguous
    torch.empty((7, 1), dtype=torch.float32, device=META),            # wrong rank
])
def test_output_check_rejects(bad):
    with pytest.raises(ValueError):
        rlk._out(bad, (7,), torch.float32, META, "out")


def test_workspace_size_is_counted_in_bytes():
    ws = torch.empty(100, dtype=torch.int64, device=META)             # 800 bytes
    t, nbytes = rlk._workspace(ws, 800, META)
    assert t is ws and nbytes == 800
    with pytest.raises(ValueError):
        rlk._workspace(ws, 801, META)
    with pytest.raises(ValueError):
        rlk._workspace(torch.empty(1000, dtype=torch.uint8), 10, META)   # other device
    with pytest.raises(ValueError):
        rlk._workspace(torch.empty(2000, dtype=torch.uint8, device=META)[::2], 10, META)
    assert rlk._workspace(None, 0, META) == (None, 0)
    t, nbytes = rlk._workspace(None, 64, META)
    assert nbytes == 64 and t.dtype == torch.uint8


def test_accumulator_check():
    good = torch.empty(rlk.NORM_BIN_WORDS, dtype=torch.int64, device=META)
    assert rlk._bins_tensor(good, META) is good
    for bad in (torch.empty(rlk.NORM_BIN_WORDS - 1, dtype=torch.int64, device=META),
                torch.empty(rlk.NORM_BIN_WORDS, dtype=torch.int32, device=META),
                torch.empty(rlk.NORM_BIN_WORDS, dtype=torch.int64)):
        with pytest.raises(ValueError):
            rlk._bins_tensor(bad, META)


def test_ordinary_rows_get_the_flat_tolerance():
    """Benchmark-shaped rows (sigma 2.5 with a +8 spike) at every temperature
    the workloads use (and 0.25) are compared at exactly 2e-5; only rows whose scaled
    logits exceed ORDINARY_MAX_Z are widened, by 2^-22 * max|x/T|."""
    w = datagen.full(n_rows=6)
    logits, _ = w.generate()
    for t in (0.25, 0.5, 0.7, 1.0, 1.3, 2.0):
        tol = row_tolerance(logits, w.vocab_real, np.full(6, t, np.float32))
        assert np.all(tol == TOL), (t, tol)
    tol = row_tolerance(logits, w.vocab_real, np.full(6, 0.1, np.float32))
    zmax = np.array([np.abs(datagen.bf16_bits_to_f32(r[:w.vocab_real])).max() / np.float32(0.1) for r in logits])
    want = np.where(zmax > ORDINARY_MAX_Z, TOL + 2.0 ** -22 * zmax, TOL)
    assert np.all(zmax > ORDINARY_MAX_Z)
    assert np.allclose(tol, want, rtol=1e-6, atol=0)
