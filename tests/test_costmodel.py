"""Pins the byte/flop accounting used for roofline fractions against the
read-versus-compute numbers printed on 'Muse Spark Open を段階的に分解する'
(sections ⑧-⑭); constants and citations in tests/golden/costmodel_muse.json."""
import json
import os

import pytest

from mixture_experts_gemm_amd import roofline as R

with open(os.path.join(os.path.dirname(__file__), "golden", "costmodel_muse.json")) as f:
    G = json.load(f)

BW = G["h200_hbm_bytes_per_s"]
RATE = G["h200_bf16_flops_per_s"]
D, FF, E, K, NL = G["expert_width"], G["expert_ffn"], G["experts_per_layer"], G["top_k"], G["layers"]
BITS = G["nvfp4_bits_per_value"]


def _derived():
    per_tok = R.compute_time(R.flops_per_slot(D, FF), RATE) * 1e6
    e_bytes = R.expert_bytes(D, FF, BITS)
    return {
        "params_per_expert": R.expert_params(D, FF),
        "expert_params_total": R.expert_params(D, FF) * E * NL,
        "bf16_expert_bytes_total": R.expert_bytes(D, FF, 16) * E * NL,
        "nvfp4_expert_bytes_total": e_bytes * E * NL,
        "nvfp4_bytes_per_expert": e_bytes,
        "read_us_per_expert": R.read_time(e_bytes, BW) * 1e6,
        "compute_us_per_token": per_tok,
        "crossover_tokens": R.crossover_tokens(D, FF, BITS, BW, RATE),
        "compute_us_at_24": 24 * per_tok,
        "compute_us_at_94": 94 * per_tok,
        "bf16_read_us_per_expert": R.read_time(R.expert_bytes(D, FF, 16), BW) * 1e6,
        "slots_753": 753 * K,
        "tokens_per_expert_753": 753 * K / E,
        "read_floor_us_32_experts": (E // G["gpus"]) * R.read_time(e_bytes, BW) * 1e6,
        # 3,012 tokens x 8 slots over 8 GPUs: each GPU computes 3,012 slots
        "compute_floor_us_3012": 3012 * K / G["gpus"] * per_tok,
        "combinations_256_choose_8": R.combinations(E, K),
    }


@pytest.mark.parametrize("key", sorted(G["expect"]))
def test_page_numbers(key):
    want, rel = G["expect"][key]
    got = _derived()[key]
    assert abs(got - want) <= rel * abs(want) + 1e-12, (key, got, want)


def test_nvfp4_bits_from_block_structure():
    # 16 values share one 8-bit scale: about 4.5 bits per value (section ⑪)
    assert R.block_scaled_bits(4, 16) == 4.5
    assert R.block_scaled_bits(4, 32) == 4.25


def test_mxfp4_expert_bytes_at_build_shape():
    assert R.mxfp4_expert_bytes(8192, 2048) == 26_738_688
    assert R.mxfp4_w1_bytes(8192, 2048) + R.mxfp4_w2_bytes(8192, 2048) == 26_738_688
    assert R.layer_bytes(1, 8192, 256, 2048, 8) == 8 * 26_738_688 + 8_388_608 + 65_536 + 32_768
    assert R.layer_flops(4096, 8192, 8, 2048) == 3_298_534_883_328
