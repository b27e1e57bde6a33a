"""The serving harness's KV caching, on the CPU in float64 (no GPU, no library):
a prefill of the prompt with the R2L sidecar hooks active over it, followed by
one step over the generation block, equals one causal pass over prompt + block
in which each hooked layer runs the sidecar over the prompt and over the block
separately (the R2L stream covers the prompt at prefill and the generation
tokens during denoising, "Bifocal Diffusion Language Models", section 2,
inference). The hooks here are the oracle's fp64 sidecar block on tiny widths,
so what is checked is the harness: cache positions, the causal mask across the
prefill / step boundary, and that the cache holds keys and values of post-hook
hidden states.
"""
import numpy as np
import pytest
import torch

import bench
import oracle
import synth

B, P, L = 2, 12, 5
DM, DI, R = 32, 64, 8
LAYERS, EVERY = 4, 2


def backbone():
    return bench.StubBackbone(torch, layers=LAYERS, dm=DM, hq=4, hkv=2, hd=8, ff=64, batch=B,
                              max_tokens=P + L, device="cpu", dtype=torch.float64, seed=11)


def sidecar_hooks(segments):
    """One hook per hooked layer: h <- h + s * sidecar(h) over each of the
    token ranges in `segments` separately (each an R2L stream of its own)."""
    hooks = {}
    for j, l in enumerate(x for x in range(LAYERS) if (x + 1) % EVERY == 0):
        w = synth.sidecar_weights(900 + j, DM, DI, R)
        s = 0.5 + 0.25 * j

        def run(h, w=w, s=s):
            for a, b in segments:
                seg = h[:, a:b].contiguous()
                r = oracle.sidecar_forward(seg.reshape(-1, DM).numpy(), w["W_in"], w["conv_w"],
                                           w["conv_b"], w["W_x"], w["W_dt"], w["dt_bias"],
                                           w["A"], w["Dskip"], w["W_out"], s=s, batch=B,
                                           seqlen=b - a)
                h[:, a:b] = torch.from_numpy(r["out"]).reshape(B, b - a, DM)
        hooks[l] = run
    return hooks


def inputs():
    g = torch.Generator().manual_seed(12)
    return (torch.randn((B, P, DM), generator=g, dtype=torch.float64),
            torch.randn((B, L, DM), generator=g, dtype=torch.float64))


def test_prefill_then_block_step_equals_one_causal_pass():
    prompt, block = inputs()
    # the harness: prefill (hooks over the prompt), then the step (hooks over the block)
    cached = backbone()
    hp = prompt.clone()
    cached.forward(hp, 0, hooks=sidecar_hooks([(0, P)]), q_chunk=5)
    hb = block.clone()
    cached.forward(hb, P, hooks=sidecar_hooks([(0, L)]))
    # one pass over prompt + block
    full = backbone()
    hf = torch.cat([prompt, block], dim=1)
    full.forward(hf, 0, hooks=sidecar_hooks([(0, P), (P, P + L)]))
    assert torch.allclose(hb, hf[:, P:], rtol=0, atol=1e-12), \
        float((hb - hf[:, P:]).abs().max())
    assert torch.allclose(hp, hf[:, :P], rtol=0, atol=1e-12)
    for l in range(LAYERS):
        assert torch.allclose(cached.Kt[l], full.Kt[l], rtol=0, atol=1e-12), l
        assert torch.allclose(cached.V[l], full.V[l], rtol=0, atol=1e-12), l


def test_prefill_cache_holds_post_hook_states():
    """A prefill without its hooks leaves keys / values that differ after the
    first hooked layer, and the block step then differs too: the hooks at
    prefill are part of what the cache holds."""
    prompt, block = inputs()
    with_hooks, without = backbone(), backbone()
    with_hooks.forward(prompt.clone(), 0, hooks=sidecar_hooks([(0, P)]))
    without.forward(prompt.clone(), 0)
    first = EVERY - 1
    for l in range(LAYERS):
        same = torch.allclose(with_hooks.Kt[l][..., :P], without.Kt[l][..., :P], rtol=0,
                              atol=1e-12)
        assert same == (l <= first), l     # layers up to the first hook see no hook yet
    h1, h2 = block.clone(), block.clone()
    with_hooks.forward(h1, P, hooks=sidecar_hooks([(0, L)]))
    without.forward(h2, P, hooks=sidecar_hooks([(0, L)]))
    assert float((h1 - h2).abs().max()) > 1e-6


@pytest.mark.parametrize("q_chunk", [None, 1, 4, 7])
def test_query_chunks_do_not_change_the_prefill(q_chunk):
    prompt, _ = inputs()
    a, b = backbone(), backbone()
    ha, hb = prompt.clone(), prompt.clone()
    a.forward(ha, 0, q_chunk=q_chunk)
    b.forward(hb, 0)
    assert torch.allclose(ha, hb, rtol=0, atol=1e-12)


def test_causal_mask_against_a_masked_softmax():
    """One layer's attention output from the cache path equals a plain masked
    softmax attention written out here (grouped-query heads, causal)."""
    torch.manual_seed(0)
    bb = backbone()
    h = torch.randn((B, P, DM), dtype=torch.float64)
    h0 = h.clone()
    bb.layer(0, h, 0, q_chunk=5)
    W = bb.W[0]
    a = h0 * torch.rsqrt(h0.pow(2).mean(-1, keepdim=True) + 1e-6) * W["ln1"]
    qkv = a @ W["qkv"]
    q = qkv[..., :32].reshape(B, P, 4, 8)
    k = qkv[..., 32:48].reshape(B, P, 2, 8)
    v = qkv[..., 48:].reshape(B, P, 2, 8)
    o = torch.empty((B, P, 4, 8), dtype=torch.float64)
    for hq in range(4):
        kv = hq // 2
        sc = torch.einsum("btd,bsd->bts", q[:, :, hq], k[:, :, kv]) / np.sqrt(8)
        sc = sc.masked_fill(torch.triu(torch.ones(P, P, dtype=torch.bool), 1), float("-inf"))
        o[:, :, hq] = torch.softmax(sc, -1) @ v[:, :, kv]
    ref = h0 + o.reshape(B, P, 32) @ W["o"]
    m = ref * torch.rsqrt(ref.pow(2).mean(-1, keepdim=True) + 1e-6) * W["ln2"]
    ref = ref + (torch.nn.functional.silu(m @ W["gate"]) * (m @ W["up"])) @ W["down"]
    assert torch.allclose(h, ref, rtol=0, atol=1e-12), float((h - ref).abs().max())
