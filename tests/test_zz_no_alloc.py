"""The allocation-free ctx_features entry point against the workspace one.

dflash_ctx_features_noalloc runs the same kernels as dflash_ctx_features,
with their scratch in the library's static device array instead of a
caller workspace, so its output must be bitwise equal.  Two calls in a row,
the second with fewer rows, check that the shared array's leftovers from
one call do not leak into the next.  Every call goes through the C ABI.
"""
import numpy as np
import pytest
import torch

import synth
from tests.gpu_util import dev, host

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("cfg", [synth.ROUND8_BF16, synth.TINY_F32, synth.ROUND8_FP8_D2],
                         ids=["bf16", "f32", "fp8"])
def test_noalloc_matches_workspace_entry_point(cfg):
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    from block_diffusion_drafter_round_amd import dflash as D
    sw = synth.make_weights(cfg.replace(n_layers=1))
    dr = D.Drafter(sw, max_rows=64)
    for t, stream in ((48, 7), (5, 8)):           # a second, smaller call on the same scratch
        taps = dev(synth.make_taps(cfg, t, stream=stream))
        ref = torch.empty((t, cfg.hidden), dtype=torch.float32, device="cuda")
        out = torch.full((t, cfg.hidden), float("nan"), dtype=torch.float32, device="cuda")
        D.dflash_ctx_features(dr.model, taps, t, ref, dr.ws, dr.ws_bytes)
        D.dflash_ctx_features_noalloc(dr.model, taps, t, out)
        torch.cuda.synchronize()
        print(f"[noalloc] {cfg.name} t={t}: max |diff| {np.abs(host(out) - host(ref)).max():.3e}", flush=True)
        assert np.array_equal(host(out), host(ref)), f"t={t}: allocation-free result differs"


def test_noalloc_rejects_too_many_rows():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    from block_diffusion_drafter_round_amd import dflash as D
    cfg = synth.TINY_F32
    dr = D.Drafter(synth.make_weights(cfg.replace(n_layers=1)), max_rows=16)
    t = 65537
    with pytest.raises(D.DflashError) as ei:
        D.dflash_ctx_features_noalloc(dr.model, 16, t, 16)
    assert ei.value.code == D.DFLASH_E_INVAL and "maximum" in str(ei.value)
