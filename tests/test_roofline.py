"""Pins for the roofline calculator: it must reproduce the figures the pages
print (tests/golden/pages_figures.json, each with its citation) from shapes
and peak rates, and count algorithmic work consistently."""
import json
import os

import pytest

from latent_kv_decode_amd import roofline as rf

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "pages_figures.json")))
R = GOLD["reconstruction"]


def _close(name, got):
    g = GOLD[name]
    assert abs(got - g["value"]) <= g["tol"], (name, got, g)


def test_ridges():
    h100 = rf.ridge(R["h100_bf16_tflops"] * 1e12, R["h100_tbps"] * 1e12)
    h20 = rf.ridge(R["h20_bf16_tflops"] * 1e12, R["h20_tbps"] * 1e12)
    _close("ridge_h100", h100)
    _close("ridge_h20", h20)
    _close("h20_compute_cut", R["h100_bf16_tflops"] / R["h20_bf16_tflops"])


def test_intensities():
    _close("absorbed_ai_sq1", rf.absorbed_intensity(R["h_q"], R["d_c"], R["d_rope"], s_q=1))
    assert abs(rf.absorbed_intensity(128, 512, 64) - 241.78) < 0.01
    _close("grouped_ai_g8_sq2", rf.grouped_intensity(128, 8, 128, 64, s_q=2))
    _close("grouped_ai_g4_sq1", rf.grouped_intensity(128, 4, 128, 64, s_q=1))


def test_kv_ratio_exact():
    assert rf.kv_ratio(R["d_c"], R["d_rope"], R["baseline_kv_heads"], R["baseline_head_dim"]) == \
        GOLD["kv_ratio"]["value"]


def test_modelled_throughputs():
    L = R["cache_tokens"]
    lat_bytes = (R["d_c"] + R["d_rope"]) * 2
    lat_flops = R["h_q"] * (2 * (R["d_c"] + R["d_rope"]) + 2 * R["d_c"])
    grp_bytes = (2 * R["g"] * R["d_h"] + R["d_rope"]) * 2
    grp_flops = R["h_q"] * (2 * (R["d_h"] + R["d_rope"]) + 2 * R["d_h"])
    h100 = rf.decode_tokens_per_s(R["h100_bf16_tflops"] * 1e12, R["h100_tbps"] * 1e12, L,
                                  bytes_per_cache_token=lat_bytes,
                                  flops_per_cache_token_per_query=lat_flops)
    h20_mla = rf.decode_tokens_per_s(R["h20_bf16_tflops"] * 1e12, R["h20_tbps"] * 1e12, L,
                                     bytes_per_cache_token=lat_bytes,
                                     flops_per_cache_token_per_query=lat_flops)
    h20_gqa = rf.decode_tokens_per_s(R["h20_bf16_tflops"] * 1e12, R["h20_tbps"] * 1e12, L,
                                     bytes_per_cache_token=grp_bytes,
                                     flops_per_cache_token_per_query=grp_flops, s_q=2)
    _close("h100_absorbed_tok_s", h100)
    _close("h20_absorbed_tok_s", h20_mla)
    _close("h20_grouped_tok_s", h20_gqa)
    _close("h20_speedup", h20_gqa / h20_mla)
    assert round(h100) == 354979 and round(h20_mla) == 64864 and round(h20_gqa) == 220537


def test_work_counts_headline_workload():
    w = rf.mla_work([4096] * 64, s_q=1, h_q=128, n_lat=1, d_c=512, d_rope=64, page_size=64)
    assert w.cache_bytes == 64 * 4096 * 1152
    assert w.flops == 64 * 4096 * 128 * 2176
    assert abs(w.bytes / 1e6 - 319.8) < 0.5
    assert abs(w.intensity - 228.3) < 0.5


def test_work_counts_8bit_cache():
    """An E4M3 cache is one byte per element; query, output, LSE and metadata
    keep their sizes, and the FLOPs do not change."""
    w2 = rf.mla_work([4096] * 64, s_q=1, h_q=128, n_lat=1, d_c=512, d_rope=64, page_size=64)
    w1 = rf.mla_work([4096] * 64, s_q=1, h_q=128, n_lat=1, d_c=512, d_rope=64, page_size=64,
                     cache_elem=1)
    assert w1.cache_bytes == 64 * 4096 * 576
    assert w2.bytes - w1.bytes == w1.cache_bytes and w1.flops == w2.flops
    g = rf.gqa_work([8192] * 128, s_q=1, h_q=32, n_kv=8, d_h=128, d_rope=0, page_size=64,
                    cache_elem=1)
    assert g.cache_bytes == 128 * 8192 * 2 * 8 * 128


def test_work_counts_causal_sq2():
    w1 = rf.mla_work([10], s_q=2, h_q=1, n_lat=1, d_c=4, d_rope=0, page_size=4)
    assert w1.flops == (9 + 10) * (2 * 4 + 2 * 4)
    w2 = rf.gqa_work([10], s_q=2, h_q=2, n_kv=1, d_h=4, d_rope=0, page_size=4, causal=False)
    assert w2.flops == 2 * 10 * 2 * 16


def test_mi355x_ridge():
    assert abs(rf.ridge(rf.MI355X_BF16_TFLOPS * 1e12, rf.MI355X_HBM_GBPS * 1e9) - 312.5) < 1e-9
