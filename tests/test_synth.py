"""The seeded input generator: deterministic, and its bf16 rounding is round-to-nearest-even."""
import numpy as np
import torch

from sequence_long_context_amd import synth


def test_bf16_rounding_matches_torch():
    g = np.random.default_rng(0)
    x = np.concatenate([g.standard_normal(100000).astype(np.float32),
                        np.array([0.0, -0.0, 1.0, np.inf, -np.inf, 1e-40, 3.0e38], np.float32),
                        # exact ties between two bf16 neighbours
                        (np.arange(1, 1000, dtype=np.uint32) << 16 | 0x8000).view(np.float32)])
    want = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(synth.f32_to_bf16_bits(x), want)
    np.testing.assert_array_equal(synth.bf16_bits_to_f32(want),
                                  torch.from_numpy(want.view(np.int16)).view(torch.bfloat16).float().numpy())


def test_nan_stays_nan():
    x = np.array([np.nan, -np.nan], np.float32)
    assert np.isnan(synth.bf16_bits_to_f32(synth.f32_to_bf16_bits(x))).all()


def test_seeded_and_chunk_independent():
    a = synth.normal(synth.seed_for(3, "q"), (3, 5, 7), "bf16")
    b = synth.normal(synth.seed_for(3, "q"), (3, 5, 7), "bf16")
    assert a.tobytes() == b.tobytes()
    assert synth.seed_for(3, "k") == 3002
    f = synth.normal(11, (1000,), "f32")
    assert abs(float(f.mean())) < 0.2 and 0.8 < float(f.std()) < 1.2
