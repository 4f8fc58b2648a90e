"""The allocation-free entry point (moe_layer_forward_noalloc, the library's static device
scratch in place of a workspace) against moe_layer_forward with a workspace, through the
C ABI: the same output and routing bitwise, on two calls in a row, the second smaller."""
import numpy as np
import pytest
import torch

from synth import configs
from tests import gpu_common as G

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    import speculative_verify_moe_amd  # noqa: F401  (fails loudly if the library is missing)
    yield
    torch.cuda.synchronize()


def _call(fn, x, D, T, E, k, **kw):
    logits = torch.empty((T, E), dtype=torch.float32, device="cuda")
    ids = torch.empty((T, k), dtype=torch.int32, device="cuda")
    w = torch.empty((T, k), dtype=torch.float32, device="cuda")
    out = torch.empty((T, D.hidden), dtype=torch.bfloat16, device="cuda")
    fn(x, D, out=out, logits_out=logits, ids_out=ids, w_out=w, **kw)
    torch.cuda.synchronize()
    return G.bf16_bits(out), logits.cpu().numpy(), ids.cpu().numpy(), w.cpu().numpy()


@pytest.mark.parametrize("recipe,T1,T2", [("qwen36_a3b", 8, 5), ("flash_next_fp8", 6, 1), ("qwen36_a3b", 32, 16),
                                          ("qwen36_a3b_mxfp4", 8, 2), ("tiny", 100, 70), ("tiny", 64, 3)])
def test_noalloc_equals_the_workspace_entry_point(recipe, T1, T2):
    import speculative_verify_moe_amd as moe
    print(f"[noalloc] {recipe} T={T1} then T={T2}", flush=True)
    cfg = configs.CONFIGS[recipe]
    D = G.device_layer(G.host_layer(cfg))
    for T in (T1, T2):
        x = G.to_dev_bf16(configs.make_tokens(cfg, T, replica=T))
        ws = torch.zeros((moe.moe_layer_workspace_size(T, D),), dtype=torch.uint8, device="cuda")
        ref = _call(moe.moe_layer_forward, x, D, T, cfg.E, cfg.k, ws=ws)
        got = _call(moe.moe_layer_forward_noalloc, x, D, T, cfg.E, cfg.k)
        for r, g, what in zip(ref, got, ("out", "logits", "ids", "w")):
            assert np.array_equal(r.view(np.uint8), g.view(np.uint8)), f"{recipe} T={T}: {what} differs"
        assert np.all(np.isfinite(G.bf16_values(got[0])))


def test_noalloc_refuses_calls_beyond_its_scratch():
    import speculative_verify_moe_amd as moe
    cfg = configs.CONFIGS["prefill"]
    D = G.device_layer(G.host_layer(cfg))
    x = G.to_dev_bf16(configs.make_tokens(cfg, 4096))
    with pytest.raises(moe.MoeError, match="static scratch"):
        moe.moe_layer_forward_noalloc(x, D)
