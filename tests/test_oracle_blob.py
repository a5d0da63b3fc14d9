"""Pins of the blob layout and the fp64 dequantisation."""
import json
import os

import numpy as np
import torch

from oracle import blob, formats
from synth import CONFIGS, WorkloadConfig, expert_blob, blob_bytes

GOLD = os.path.join(os.path.dirname(__file__), "golden", "page_sizes.json")


def _close(v, ref, digits):
    return round(v, digits) == ref


def test_sizes_match_the_pages():
    g = json.load(open(GOLD))
    H, I = 6144, 2048
    lay = blob.part_layout(H, I)
    weights = lay["w13_codes"][1] + lay["w2_codes"][1]
    scales = lay["w13_scales"][1] + lay["w2_scales"][1]
    total = blob.blob_size(H, I)
    assert total == 21_233_664
    assert _close(weights / 1e6, g["glm_expert_weights_MB"]["value"], 3)
    assert _close(scales / 1e6, g["glm_expert_scales_MB"]["value"], 3)
    assert _close(total / 1e6, g["glm_expert_total_MB"]["value"], 3)
    assert scales / weights == g["glm_scale_fraction_of_weights"]["value"]
    assert _close(256 * lay["w13_codes"][1] / 1e9, g["glm_w13_slab_GB"]["value"], 2)
    assert _close(256 * lay["w2_codes"][1] / 1e9, g["glm_w2_slab_GB"]["value"], 2)
    assert total / 2 ** 20 == g["glm_expert_MiB"]["value"]
    assert _close(256 * total / 2 ** 30, g["glm_layer_GiB"]["value"], 2)
    flash = blob.blob_size(4096, 2048)
    assert flash / 2 ** 20 == g["flash_expert_MiB"]["value"]
    assert _close(42 * 8 * flash / 2 ** 30, g["flash_token_GiB"]["value"], 2)
    assert blob.blob_size(256, 128) == 55_296
    # the generator's layout agrees with the oracle's
    assert blob_bytes(6144, 2048) == total


def _independent_element(b, H, I, which, r, c, gs13, gs2):
    """Decode one weight by reading bytes directly, through torch's E4M3 decoder
    and the OCP E2M1 magnitude table (no oracle code)."""
    mags = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
    if which in ("G", "U"):
        row = r if which == "G" else I + r
        K, code_off, sc_off, gs = H, 0, 2 * I * H // 2, gs13
    else:
        row, K, gs = r, I, gs2
        code_off = 2 * I * H // 2 + 2 * I * H // 16
        sc_off = code_off + H * I // 2
    byte = int(b[code_off + row * (K // 2) + c // 2])
    nib = byte & 0xF if c % 2 == 0 else byte >> 4
    v = mags[nib & 7] * (-1.0 if nib & 8 else 1.0)
    sb = int(b[sc_off + row * (K // 16) + c // 16])
    s = torch.tensor([sb], dtype=torch.uint8).view(torch.float8_e4m3fn).double().item()
    return v * s * float(np.float32(gs))


def test_one_hot_columns_are_the_decoded_weights():
    cfg = CONFIGS["tiny"]
    H, I = cfg.hidden, cfg.inter
    b = expert_blob(cfg, 0, 3)
    gs13, gs2 = np.float32(1.375), np.float32(0.625)
    G, U, D = blob.dequant_expert(b, H, I, gs13, gs2)
    rng = np.random.default_rng(0)
    for _ in range(40):
        c = int(rng.integers(H))
        x = np.zeros(H)
        x[c] = 1.0
        col_g, col_u = G @ x, U @ x          # a one-hot product selects column c
        for r in rng.integers(I, size=4):
            assert col_g[r] == _independent_element(b, H, I, "G", int(r), c, gs13, gs2)
            assert col_u[r] == _independent_element(b, H, I, "U", int(r), c, gs13, gs2)
        cd = int(rng.integers(I))
        xd = np.zeros(I)
        xd[cd] = 1.0
        col_d = D @ xd
        for r in rng.integers(H, size=4):
            assert col_d[r] == _independent_element(b, H, I, "D", int(r), cd, gs13, gs2)


def test_global_scale_is_a_plain_factor():
    cfg = CONFIGS["tiny"]
    b = expert_blob(cfg, 0, 1)
    G1, U1, D1 = blob.dequant_expert(b, cfg.hidden, cfg.inter, 1.0, 1.0)
    G2, U2, D2 = blob.dequant_expert(b, cfg.hidden, cfg.inter, 2.0, 0.5)
    assert np.array_equal(G2, 2 * G1) and np.array_equal(U2, 2 * U1) and np.array_equal(D2, 0.5 * D1)
