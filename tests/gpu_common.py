"""Shared helpers of the GPU parity tests: moving generated layers to the
device, gap-checked activations, and the output tolerance."""

import math
import sys

import numpy as np
import torch

import oracle
import synth

# Routing-score gap below which a token's draw is replaced (the oracle's k-th
# minus (k+1)-th selection score must exceed it; GPU and oracle logits differ
# by fp32 summation order only, orders of magnitude less).
GAP = 1e-5
# Final outputs: max |gpu - oracle| <= REL_TOL * RMS(oracle output).
REL_TOL = 1e-4


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def to_device(L: synth.Layer):
    import quantized_routed_expert_sigmoid_amd as qre

    def qb(b):
        return qre.QBank(b.storage.cuda().contiguous(), b.scale_storage.cuda().contiguous(), b.bits, b.group)
    w = L.w
    shared = [qb(L.sh_gate), qb(L.sh_up), qb(L.sh_down)] if w.has_shared else None
    return qre.MoELayer(w.hidden, w.inter, w.n_experts, w.top_k, w.rsf,
                        L.router_w.cuda().contiguous(), L.bias.cuda().contiguous(),
                        qb(L.gate), qb(L.up), qb(L.down), shared,
                        w.n_group, w.topk_group, w.top_p)


def gapped_activations(w: synth.Workload, router_w, bias, S=None, tag=""):
    """Activations whose oracle routing gaps all exceed GAP (redrawing a
    token's row with the next attempt number until they do)."""
    S = w.S if S is None else S
    attempts = {}
    x = synth.activations(w, S, tag=tag).numpy()
    W, b = router_w.cpu().numpy(), bias.cpu().numpy()
    opts = oracle.route_opts(w.n_group, w.topk_group, w.top_p)
    for t in range(S):
        a = 0
        while True:
            r = oracle.route_token(x[t], W, b, w.top_k, w.rsf, opts)
            if r["gap"] > GAP:
                break
            a += 1
            x[t] = synth.token_activation(w, t, a, tag).numpy()
        if a:
            attempts[t] = a
    return torch.from_numpy(x), attempts


def assert_close_rms(gpu_out, ref_out, what=""):
    ref = np.asarray(ref_out, dtype=np.float64)
    got = np.asarray(gpu_out, dtype=np.float64)
    rms = math.sqrt(float(np.mean(ref ** 2)))
    err = float(np.max(np.abs(got - ref))) if ref.size else 0.0
    assert err <= REL_TOL * rms, f"{what}: max|diff| {err:.3e} > {REL_TOL} * rms {rms:.3e}"
    return err / rms if rms > 0 else 0.0


def pinned_copy(t: torch.Tensor) -> torch.Tensor:
    """A copy of t in newly allocated pinned host memory."""
    p = torch.empty(t.shape, dtype=t.dtype, pin_memory=True)
    p.copy_(t)
    return p


def to_slow_tier(L: synth.Layer, dev, where="host"):
    """The layer with its routed banks in pinned host memory (where="host")
    or in device memory (where="device"); router and shared expert are dev's
    device tensors."""
    import quantized_routed_expert_sigmoid_amd as qre

    def qb(b):
        if where == "device":
            return qre.QBank(b.storage.cuda().contiguous(), b.scale_storage.cuda().contiguous(), b.bits,
                             b.group)
        return qre.QBank(pinned_copy(b.storage.contiguous()), pinned_copy(b.scale_storage.contiguous()),
                         b.bits, b.group)
    w = L.w
    return qre.MoELayer(w.hidden, w.inter, w.n_experts, w.top_k, w.rsf, dev.router_w, dev.router_bias,
                        qb(L.gate), qb(L.up), qb(L.down), dev.shared, w.n_group, w.topk_group, w.top_p)
