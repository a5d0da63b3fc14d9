"""Checks of the seeded input generators (encoders and workload statistics)."""
import numpy as np
import torch

from oracle import formats, route
from synth import CONFIGS, bf16_bits_from_f32, e4m3_bits_rne, expert_blob, routing_trace, activations
from synth.configs import rows_at_step


def test_e4m3_encoder_round_trips_every_finite_code():
    vals = np.array([formats.e4m3_value(b) for b in range(256) if (b & 0x7F) != 0x7F])
    codes = [b for b in range(256) if (b & 0x7F) != 0x7F]
    enc = e4m3_bits_rne(vals)
    # -0.0 encodes with the sign bit; both zeros decode to zero
    assert [int(c) for c in enc] == codes


def test_e4m3_encoder_rounds_to_nearest_even():
    torch_ref = lambda v: torch.tensor(v, dtype=torch.float64).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    rng = np.random.default_rng(0)
    v = np.concatenate([np.abs(rng.standard_normal(20000)) * 0.02, rng.uniform(0, 440, 2000),
                        [2.0 ** -10, 3 * 2.0 ** -10, 1.0625, 1.1875, 2.0 ** -7 * 1.5]])
    assert np.array_equal(e4m3_bits_rne(v), torch_ref(v))


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(1)
    x = (rng.standard_normal(100000) * np.exp(rng.uniform(-20, 20, 100000))).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(bf16_bits_from_f32(x), ref)


def test_blobs_are_seeded_and_scales_finite():
    cfg = CONFIGS["tiny"]
    a, b, c = expert_blob(cfg, 0, 5), expert_blob(cfg, 0, 5), expert_blob(cfg, 0, 6)
    assert np.array_equal(a, b) and not np.array_equal(a, c)
    sc = a[cfg.hidden * cfg.inter: cfg.hidden * cfg.inter + cfg.hidden * cfg.inter // 8]
    assert not np.any((sc & 0x7F) == 0x7F)
    assert np.array_equal(activations(cfg, 0, 3, 1), activations(cfg, 0, 3, 1))


def test_glm_routing_statistics():
    cfg = CONFIGS["glm"]
    logits, rows = routing_trace(cfg, 0)
    prev, overlaps = None, []
    for t in range(cfg.steps):
        ids, _ = route(logits[t, :1], cfg.top_k)
        cur = set(ids[0].tolist())
        if prev is not None:
            overlaps.append(len(cur & prev) / cfg.top_k)
        prev = cur
    ov = float(np.mean(overlaps))
    assert 0.2 < ov < 0.35, ov      # step-to-step overlap about 0.27 on the pages


def test_drafted_rows_share_picks():
    cfg = CONFIGS["glm_draft"]
    assert [rows_at_step(cfg, t) for t in (0, 9, 49, 50)] == [4, 16, 64, 4]
    logits, rows = routing_trace(cfg, 0, steps=20)
    shares = []
    for t in range(20):
        if rows[t] != 4:
            continue
        ids, _ = route(logits[t, :4], 8)
        r0 = set(ids[0].tolist())
        shares += [len(set(ids[m].tolist()) & r0) / 8 for m in range(1, 4)]
    assert 0.4 < np.mean(shares) < 0.7
