"""quads_rac_quantize_noalloc (the RAC entry point that allocates nothing and
works in the library's static per-GPU scratch) against quads_rac_quantize
(caller workspace) on the same inputs: every output bit-exact, on two calls
in a row, the second on a smaller input, so the second call runs on scratch
that still holds the first call's partial sums."""

import numpy as np
import pytest
import torch

import synth

pytestmark = pytest.mark.gpu

# (tokens, channels, k): the MoE down-projection input (32768 packed rows x
# 768, k = 64), then the MoE gate/up input (4096 x 2048, k = 64)
CASES = ((32768, 768, 64), (4096, 2048, 64))


def _input(m, kd, seed):
    ra, ro, _, _ = synth.streams(seed)
    x, _ = synth.activations(ra, ro, m, kd, "normal", 3.0, max(1, kd // 100), 20.0)
    return torch.from_numpy(x.view(np.int16)).to("cuda:0")


def test_noalloc_matches_workspace_entry_point():
    import nvfp4_w4a4_quantized_act_amd as Q
    Q.lib()
    for i, (m, kd, k) in enumerate(CASES):
        print(f"no-alloc RAC: call {i}, x [{m}, {kd}], k = {k}", flush=True)
        x = _input(m, kd, 900 + i)
        got = Q.quads_rac_quantize_noalloc(x, k, want_score=True)
        exp = Q.quads_rac_quantize(x, k, want_score=True)
        torch.cuda.synchronize()
        for name in ("nib", "scale", "sel", "r_nib", "r_scale"):
            assert torch.equal(got[name], exp[name]), (i, name)
        for name in ("ts", "r_ts"):
            assert got[name].item() == exp[name].item(), (i, name)
        g, e = got["score"].cpu().numpy(), exp["score"].cpu().numpy()
        assert np.array_equal(g.view(np.uint64), e.view(np.uint64)), i
