"""HIP-graph replay of the prefill hot path, through the C ABI.

One graph holds a layer's prefill work at full size: the down projection's
online Hadamard H_12288 + INT4 (4096 tokens, fp16) and its W4A4 GEMM against
4096 output channels (the FP6-matrix-core tiles), the one-launch KV step (Q, K
rotated by H_128, K and V quantized), and the same down projection with both
operands in the FP6 operand layout.  Serving loops replay such graphs, so every
replay, with eager work and synchronisations between replays, must equal the
eager results bit for bit (page "SpinQuant, Reproduced", Q5: R3 and R4 run
online on every forward pass).  The eager results are checked against the
oracle by the parity tests; here the two down projections must also agree with
each other, bit for bit, as the library promises.
"""

import numpy as np
import pytest
import torch

from rotation_bit_quantization_amd import spin, synth

pytestmark = pytest.mark.gpu

DEV = "cuda"


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    spin.load()


def _dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def _host(t):
    torch.cuda.synchronize()
    return t.cpu().numpy()


def test_prefill_step_kv_step_and_f6_pair_replay_in_a_graph():
    rng = np.random.default_rng(29)
    M, N, K = 4096, 4096, 12288
    x = _dev(rng.standard_normal((M, K)).astype(np.float16))
    q = rng.integers(-7, 8, size=(N, K)).astype(np.int64)
    wq = _dev(((q[:, 0::2] & 15) | ((q[:, 1::2] & 15) << 4)).astype(np.uint8))
    ws = _dev((rng.random(N) * 0.01 + 1e-3).astype(np.float32))
    wf6, wsum = spin.spin_codes_f6(wq)                        # offline packing, outside the graph
    kv = synth.kv_config(seed=5, T=512, H=32)
    Kt, Vt, Qt = _dev(kv["k"]), _dev(kv["v"]), _dev(kv["q"])

    bufs = {
        "xq": torch.empty((M, K // 2), dtype=torch.uint8, device=DEV),
        "xs": torch.empty((M,), dtype=torch.float32, device=DEV),
        "y": torch.empty((M, N), dtype=torch.float32, device=DEV),
        "xf6": torch.empty((spin.f6_bytes(M, K),), dtype=torch.uint8, device=DEV),
        "xsum": torch.empty((M,), dtype=torch.int32, device=DEV),
        "xs6": torch.empty((M,), dtype=torch.float32, device=DEV),
        "y6": torch.empty((M, N), dtype=torch.float32, device=DEV),
    }
    kv_out = spin.spin_kv_qkv(Kt, Vt, Qt)                     # allocates the KV outputs once
    kv_bufs = {k: v for k, v in kv_out.items() if v is not None}

    def step():
        spin.spin_fwht_quant(x, 12288, Xq=bufs["xq"], x_scale=bufs["xs"])
        spin.spin_w4a4_gemm(bufs["xq"], bufs["xs"], wq, ws, Y=bufs["y"])
        spin.spin_kv_qkv(Kt, Vt, Qt, out=kv_bufs)
        spin.spin_fwht_quant_f6(x, Xf6=bufs["xf6"], x_sum=bufs["xsum"], x_scale=bufs["xs6"])
        spin.spin_w4a4_gemm_f6f6(bufs["xf6"], bufs["xsum"], bufs["xs6"], wf6, wsum, ws, K, Y=bufs["y6"])

    step()
    everything = dict(bufs, **{"kv_" + k: v for k, v in kv_bufs.items()})
    eager = {k: _host(v).copy() for k, v in everything.items()}
    # the two down projections write the same bits
    assert np.array_equal(eager["xs"], eager["xs6"])
    assert np.array_equal(eager["y"].view(np.uint32), eager["y6"].view(np.uint32))

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=torch.cuda.Stream()):
        step()
    for rep in range(3):
        for v in everything.values():   # eager work between replays
            if v.dtype in (torch.uint8, torch.int8):
                v.fill_(0x5A)
            elif v.dtype == torch.int32:
                v.fill_(-1)
            else:
                v.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        for k, v in everything.items():
            got = _host(v)
            assert np.array_equal(got.view(np.uint8), eager[k].view(np.uint8)), f"replay {rep}: {k} differs"
