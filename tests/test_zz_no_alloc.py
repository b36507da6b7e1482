"""The allocation-free layer decode (gdn_layer_decode_noalloc, intermediates in the
library's device scratch array) against gdn_layer_decode with a caller's workspace, through
the C ABI: two calls in a row, the second with fewer rows and a smaller layer (the scratch
keeps the first call's contents), each bit-identical to the workspace path on its own copy of
the caches; then a size beyond the scratch is refused before anything runs."""
import numpy as np
import pytest
import torch

from helpers import announce
from hybrid_linear_attention_gated_amd import inputs

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


@pytest.fixture(scope="module")
def gdn():
    import hybrid_linear_attention_gated_amd as m
    m.lib()
    return m


def _case(gdn, B, E, Hk, Hv, d, seed):
    wts = inputs.layer_weights(seed, E, Hk, Hv, d, d)
    w = [t.to(DEV) for t in (wts.w_in, wts.conv_w, wts.gamma, wts.w_out)]
    h = inputs.layer_hidden(seed + 1, B, E).to(DEV)
    cs, st = inputs.layer_caches(seed + 2, B, Hk, Hv, d, d)
    cs1, st1, cs2, st2 = cs.to(DEV), st.to(DEV), cs.to(DEV), st.to(DEV)
    ref = gdn.layer_decode(h, *w, cs1, st1, Hk, Hv, d, d, scale=0.5, order=1)
    out = torch.full((B, E), float("nan"), dtype=torch.bfloat16, device=DEV)
    gdn.layer_decode_noalloc(h, *w, cs2, st2, Hk, Hv, d, d, out, scale=0.5, order=1)
    torch.cuda.synchronize()
    assert torch.equal(out, ref), "out differs from the workspace path"
    assert torch.equal(st2, st1), "state differs from the workspace path"
    assert torch.equal(cs2, cs1), "conv cache differs from the workspace path"


def test_layer_decode_noalloc_matches_workspace_path(gdn):
    announce("layer decode without allocation: B=256 E=1024 16/16 heads d=128, then B=33 E=192 2/4 heads d=64")
    _case(gdn, 256, 1024, 16, 16, 128, 700)
    _case(gdn, 33, 192, 2, 4, 64, 710)
    # intermediates beyond the 64 MiB scratch: refused with GDN_ERR_WORKSPACE, nothing written
    B, E, Hk, Hv, d = 1024, 1024, 16, 16, 128
    wts = inputs.layer_weights(720, E, Hk, Hv, d, d)
    w = [t.to(DEV) for t in (wts.w_in, wts.conv_w, wts.gamma, wts.w_out)]
    C = 2 * Hk * d + Hv * d
    h = torch.zeros((B, E), dtype=torch.bfloat16, device=DEV)
    cs = torch.zeros((B, 3, C), dtype=torch.float32, device=DEV)
    st = torch.zeros((B, Hv, d, d), dtype=torch.float32, device=DEV)
    out = torch.full((B, E), 7.0, dtype=torch.bfloat16, device=DEV)
    with pytest.raises(gdn.GdnError) as ei:
        gdn.layer_decode_noalloc(h, *w, cs, st, Hk, Hv, d, d, out)
    assert ei.value.status == 4
    torch.cuda.synchronize()
    assert bool((out == 7.0).all())
