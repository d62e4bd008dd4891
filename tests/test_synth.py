"""The seeded input generators: the in-place forms used for the full
single-GPU share draw exactly the values of the allocating forms."""

import torch

from tenant_serving_amd import synth


def test_laplace_delta_into_matches_laplace_delta():
    a = synth.laplace_delta(synth.generator(11), 37, 48, 1.7e-3)
    out = torch.empty(37, 48)
    tmp = torch.empty(4096)
    b = synth.laplace_delta_into(synth.generator(11), out, tmp, 1.7e-3)
    assert torch.equal(a, b)
    assert torch.equal(torch.signbit(a), torch.signbit(b))


def test_base_weight_into_matches_base_weight():
    a = synth.base_weight(synth.generator(12), 19, 64)
    out = torch.empty(19, 64, dtype=torch.bfloat16)
    b = synth.base_weight_into(synth.generator(12), out, torch.empty(19 * 64 + 5))
    assert torch.equal(a, b)


def test_generators_continue_the_same_stream():
    # drawing into buffers consumes the generator exactly as the allocating
    # form does, so later draws agree too
    g1, g2 = synth.generator(13), synth.generator(13)
    synth.laplace_delta(g1, 8, 16)
    synth.laplace_delta_into(g2, torch.empty(8, 16), torch.empty(128))
    assert torch.equal(synth.activations(g1, 3, 16), synth.activations(g2, 3, 16))


def test_request_mix_range():
    ids = synth.request_mix(synth.generator(5), 16, 14)
    assert ids.dtype == torch.int32 and ids.shape == (16,)
    assert int(ids.min()) >= 0 and int(ids.max()) < 14
