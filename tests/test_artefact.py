"""The folded-weight artefact on the CPU: .npy round trip of packed codes and
scales is byte-exact, and malformed pairs are rejected without pickling."""

import numpy as np
import pytest
import torch

from rotation_bit_quantization_amd import artefact


def test_round_trip_is_byte_exact(tmp_path):
    rng = np.random.default_rng(0)
    codes = rng.integers(0, 256, size=(37, 640), dtype=np.uint8)
    scales = (rng.random(37) * 1e-2).astype(np.float32)
    scales[3] = 0.0
    scales[5] = np.float32(1e-38)
    stem = str(tmp_path / "down_proj")
    artefact.save_folded(stem, torch.from_numpy(codes), scales)
    Wq, ws = artefact.load_folded(stem)
    assert Wq.dtype == torch.uint8 and ws.dtype == torch.float32
    assert np.array_equal(Wq.numpy(), codes)
    assert np.array_equal(ws.numpy().view(np.uint32), scales.view(np.uint32))


def test_rejects_malformed_pairs(tmp_path):
    stem = str(tmp_path / "w")
    with pytest.raises(ValueError):
        artefact.save_folded(stem, np.zeros((4, 8), np.uint8), np.zeros(5, np.float32))
    with pytest.raises(ValueError):
        artefact.save_folded(stem, np.zeros((4, 8), np.int8), np.zeros(4, np.float32))
    with pytest.raises(ValueError):
        artefact.save_folded(stem, np.zeros((4, 8), np.uint8), np.zeros(4, np.float64))
    pc, ps = artefact.folded_paths(stem)
    np.save(pc, np.zeros((4, 8), np.uint8))
    np.save(ps, np.zeros(3, np.float32))
    with pytest.raises(ValueError):
        artefact.load_folded(stem)
    np.save(ps, np.array([{"a": 1}] * 4, dtype=object), allow_pickle=True)
    with pytest.raises(ValueError):          # an object array needs unpickling: refused
        artefact.load_folded(stem)
