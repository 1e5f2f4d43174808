"""The allocation-free layer forward (colibri_moe_layer_forward_noalloc)
against the workspace forward (colibri_moe_layer_forward) through the C ABI:
two calls in a row on the library's static scratch, the second with a
smaller batch, each bit-identical to the workspace call; and a batch whose
workspace exceeds the scratch is refused before anything runs."""

import pytest
import torch

import synth
from tests.gpu_common import say, to_device

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def qre():
    import quantized_routed_expert_sigmoid_amd as m
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a GPU")
    m.lib()
    return m


def _layer(name, **kw):
    w = synth.scaled(synth.WORKLOADS["tiny"], name=name, layer=name, **kw)
    L = synth.make_layer(w)
    return w, to_device(L), L


# (workload changes, first batch, second smaller batch): a small batch then
# one token (the fused one-token kernels), and a prefill-sized batch on the
# matrix cores then a small batch
CASES = {
    "int4_shared_8_then_1": (dict(bits=4, hidden=512, inter=256, n_experts=32, top_k=4, has_shared=True,
                                  rsf=2.5, var_router=1.0 / 512), 8, 1),
    "int8_mfma_96_then_5": (dict(bits=8, n_experts=8, top_k=2, has_shared=True), 96, 5),
}


@pytest.mark.parametrize("case", sorted(CASES))
def test_noalloc_matches_workspace_forward(qre, case):
    kw, s1, s2 = CASES[case]
    w, dev, L = _layer("na_" + case.split("_")[0], **kw)
    for i, S in enumerate((s1, s2)):
        say(f"noalloc {case}: call {i} S={S}")
        assert dev.workspace_bytes(S) <= qre.NOALLOC_SCRATCH_BYTES
        x = synth.activations(w, S, tag=f"na{i}").cuda().contiguous()
        out_na = torch.full_like(x, float("nan"))
        qre.moe_layer_forward_noalloc(dev, x, out_na)
        ref = qre.moe_layer_forward(dev, x)
        torch.cuda.synchronize()
        assert torch.equal(out_na, ref), f"{case} call {i}: max|diff| {(out_na - ref).abs().max().item():.3e}"


def test_noalloc_refuses_batches_beyond_the_scratch(qre):
    w, dev, L = _layer("na_big", bits=8)
    S = 1
    while dev.workspace_bytes(S) <= qre.NOALLOC_SCRATCH_BYTES:
        S *= 2
    say(f"noalloc refusal at S={S} ({dev.workspace_bytes(S)} workspace bytes)")
    x = torch.zeros((S, w.hidden), dtype=torch.float32, device="cuda")
    out = torch.full_like(x, 7.0)
    with pytest.raises(qre.ColibriError) as e:
        qre.moe_layer_forward_noalloc(dev, x, out)
    assert e.value.status == qre.COLI_E_SCRATCH
    torch.cuda.synchronize()
    assert bool((out == 7.0).all())  # nothing was enqueued
    # the largest batch that fits still runs, and matches the workspace call
    S_fit = S // 2
    x = synth.activations(w, S_fit, tag="nafit").cuda().contiguous()
    out = torch.empty_like(x)
    qre.moe_layer_forward_noalloc(dev, x, out)
    ref = qre.moe_layer_forward(dev, x)
    torch.cuda.synchronize()
    assert torch.equal(out, ref)
