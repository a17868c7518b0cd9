"""The seeded input generators: determinism, bf16 rounding, id laws."""
import numpy as np
import torch

import workloads as W


def test_normal_is_deterministic_and_chunked():
    a = W.normal(7, "x", (3, 1 << 21), 0.5)   # spans two chunks
    b = W.normal(7, "x", (3, 1 << 21), 0.5)
    c = W.normal(7, "y", (3, 1 << 21), 0.5)
    assert np.array_equal(a, b) and not np.array_equal(a, c)
    assert abs(float(a.std()) - 0.5) < 0.01


def test_round_bf16_matches_torch_rne():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(10000).astype(np.float32) * 10,
                        np.array([1.00390625, 1.01171875, -1.00390625, 3.0e-40, 0.0, -0.0], np.float32)])
    ours = W.round_bf16(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)
    assert np.array_equal(W.bf16_to_f32(ours), torch.from_numpy(x).to(torch.bfloat16).float().numpy())


def test_zipf_ids_in_range_and_skewed():
    w = W.workload("ctr")
    ids = W.candidate_ids(w)
    assert ids.shape == (w.B * w.M,) and ids.min() >= 0 and ids.max() < w.n_items
    u, cnt = np.unique(ids, return_counts=True)
    assert 0.1 < len(u) / len(ids) < 0.6          # heavy reuse
    assert cnt.max() > 50 * np.median(cnt)
    assert np.array_equal(ids, W.candidate_ids(w))


def test_uniform_ids_tiny():
    w = W.workload("tiny")
    ids = W.candidate_ids(w)
    assert ids.min() >= 0 and ids.max() < 1000 and len(np.unique(ids)) > 50


def test_ragged_lengths_lifelong():
    w = W.workload("lifelong")
    lens = W.lengths(w)
    off = W.offsets_from_lengths(lens)
    assert lens.min() >= 8192 and lens.max() <= 16384 and len(set(lens.tolist())) > 1
    assert off[0] == 0 and np.array_equal(np.diff(off), lens)


def test_user_inputs_shapes():
    w = W.workload("tiny")
    u = W.user_inputs(w)
    assert u["links_ctx"].shape == (4, 8, 32) and u["links_ctx"].dtype == np.float32
    assert u["hist"].shape == (256, 32) and len(u["weights"]) == 1
    assert u["weights"][0]["w_qkv"].shape == (96, 32)
    w2 = W.workload("ctr")
    assert W.user_inputs(w2)["hist"].dtype == np.uint16
