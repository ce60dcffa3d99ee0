"""The seeded input generator: determinism, shapes and planted structure."""

import numpy as np
import torch

from synth import CONFIGS, VideoSpec, config_spec, gen_qkv, micro_heads, rotation_offset
from synth.video_qkv import spike_codes


def test_deterministic_bits_and_head_slices():
    spec = VideoSpec(1, 3, 64, (2, 5, 7), key=99)
    Q1, K1, V1 = gen_qkv(spec)
    Q2, K2, V2 = gen_qkv(spec)
    for a, b in ((Q1, Q2), (K1, K2), (V1, V2)):
        assert a.dtype == torch.bfloat16 and a.shape == (1, 3, 70, 64)
        assert torch.equal(a.view(torch.int16), b.view(torch.int16))
    Qh, _, _ = gen_qkv(spec, heads=[2])
    assert torch.equal(Qh[:, 0].view(torch.int16), Q1[:, 2].view(torch.int16))
    assert not torch.equal(Q1, K1)


def test_config_token_counts():
    assert config_spec(0).N == 1024
    assert config_spec(1).N == 32760
    assert config_spec(2).N == 75600
    assert config_spec(3).N == 118800
    assert config_spec(4).N == 196560
    assert config_spec(1).frame_tokens == 30 * 52


def test_positional_structure_gives_locality():
    # neighbouring tokens must score higher than distant ones on average
    spec = config_spec(0)
    Q, K, _ = gen_qkv(spec, heads=[0])
    q, k = Q[0, 0].double(), K[0, 0].double()
    z = (q @ k.T) / 8.0
    near = torch.diagonal(z, 1).mean()
    far = z[:128, -128:].mean()
    assert near > far + 1.0


def test_spike_codes_match_two_percent_of_tile_pairs():
    spec = config_spec(3)
    qc, kc = spike_codes(spec)
    assert len(qc) == len(kc) == -(-spec.N // 16)
    # fraction of (query tile, key tile) pairs sharing a code
    hq = np.bincount(qc, minlength=50) / len(qc)
    hk = np.bincount(kc, minlength=50) / len(kc)
    assert abs(float(hq @ hk) - 0.02) < 0.002


def test_spikes_raise_matched_pair_logits():
    spec = VideoSpec(1, 1, 128, (3, 16, 16), key=3, spikes=True)
    Q, K, _ = gen_qkv(spec)
    qc, kc = spike_codes(spec)
    q = Q[0, 0].double().reshape(-1, 16, 128).mean(1)
    k = K[0, 0].double().reshape(-1, 16, 128).mean(1)
    z = (q @ k.T).numpy() / np.sqrt(128)
    match = qc[:, None] == kc[None, :]
    assert z[match].mean() > z[~match].mean() + 2.0


def test_micro_heads_and_rotation():
    assert micro_heads(0) == [0, 1]
    h3 = micro_heads(3)
    assert len(h3) == 7 and len(set(h3)) == 7 and all(0 <= h < 24 for h in h3)
    assert micro_heads(3) == h3
    offs = {rotation_offset(4, c, 3072) for c in range(5)}
    assert len(offs) > 1 and all(0 <= o < 3072 for o in offs)
    assert CONFIGS[4]["mode"] == "static"
