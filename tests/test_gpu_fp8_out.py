"""GPU parity of fp8 (E4M3FN) output with a per-tensor scale: O is stored as
the saturating round-to-nearest conversion of O * o_scale. The stored bytes are
decoded exactly and compared with the oracle's O within the input path's
tolerance plus half an fp8 step of the stored value."""

import numpy as np
import pytest
import torch

import oracle
import synth
from tests import _cases as C

pytestmark = pytest.mark.gpu
DEV = "cuda"
FP8_MAX = 448.0


def _check_fp8_out(out, lse, O, LSE, o_scale, base_tol, what):
    assert out.dtype == torch.float8_e4m3fn
    dec = oracle.e4m3fn_bits_to_f64(out.detach().cpu().view(torch.uint8).numpy(), 1.0)
    valid = ~np.isnan(LSE)
    ref = np.clip(O[valid] * o_scale, -FP8_MAX, FP8_MAX)      # saturated reference, in stored units
    got = dec[valid]
    assert np.isfinite(got).all(), f"{what}: NaN byte on a valid row"
    # input-path error (scaled) + half an E4M3 step: 2^-4 relative, 2^-10 absolute near zero
    bound = base_tol * o_scale + np.abs(ref) * 2.0 ** -4 + 2.0 ** -10
    err = np.abs(got - ref) - bound
    assert err.max() <= 0, f"{what}: fp8 O off by {float(err.max()):.3e} beyond the bound"
    l_gpu = C.to_np(lse)[valid]
    fin = np.isfinite(LSE[valid])
    assert float(np.abs(l_gpu[fin] - LSE[valid][fin]).max()) <= 1e-3


@pytest.mark.parametrize("o_scale", [1.0, 16.0, 3000.0])     # 3000: most |O * s| saturate at 448
def test_prefill_bf16_in_fp8_out(o_scale):
    case = synth.dense_case(2, 8, 2, 300, 300, 128, "bf16", seed=17, causal=True, device=DEV)
    out, lse = C.run_dense(case, out_dtype=torch.float8_e4m3fn, o_scale=o_scale)
    O, LSE = C.oracle_dense(case)
    _check_fp8_out(out, lse, O, LSE, o_scale, 2e-2, f"bf16->fp8 o_scale={o_scale}")


def test_prefill_fp8_in_fp8_out_softcap():
    case = synth.dense_case(1, 8, 8, 500, 500, 128, "fp8", seed=18, causal=True, softcap=30.0, device=DEV)
    out, lse = C.run_dense(case, out_dtype=torch.float8_e4m3fn, o_scale=8.0)
    O, LSE = C.oracle_dense(case)
    _check_fp8_out(out, lse, O, LSE, 8.0, 6e-2, "fp8->fp8")


def test_varlen_fp8_out():
    case = synth.varlen_case([200, 513], [200, 513], 8, 2, 128, "bf16", seed=19, device=DEV)
    out, lse = C.run_varlen(case, out_dtype=torch.float8_e4m3fn, o_scale=4.0)
    O, LSE = C.oracle_varlen(case)
    _check_fp8_out(out, lse.T, O, LSE.T, 4.0, 2e-2, "varlen fp8 out")


@pytest.mark.parametrize("d", [128, 64])
def test_paged_decode_fp8_out(d):
    case = synth.paged_case([1200, 90], 1, 32, 8, d, 64, "bf16", seed=20 + d, device=DEV)
    out, lse = C.run_paged(case, out_dtype=torch.float8_e4m3fn, o_scale=32.0)
    O, LSE = C.oracle_paged(case)
    _check_fp8_out(out, lse, O, LSE, 32.0, 2e-2, f"paged decode fp8 out d={d}")
