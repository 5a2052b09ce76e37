"""The bandwidth probe (include/flashopt_probe.h) reads and writes every byte
of the AdamW step's state and gradients: its documented XOR of the values it
read, checked on every element of a ragged list (full tiles and partial
tails), through the interleaved code records."""
import numpy as np
import pytest
import torch

from compressed_adamw_state_amd import flashopt as F

from parity import state_fields

pytestmark = pytest.mark.gpu


def test_stream_probe_touches_every_byte():
    gen = torch.Generator().manual_seed(7)
    sizes = [2048 * 5, 2048 + 7, 33, 8192 + 2047]
    states, grads, before = [], [], []
    for n in sizes:
        st = F.TensorState(n, "adamw", "cuda")
        st.theta.view(torch.int16).copy_(torch.randint(-2 ** 15, 2 ** 15, (n,), generator=gen,
                                                       dtype=torch.int16))
        st.codes.copy_(torch.randint(0, 256, st.codes.shape, generator=gen, dtype=torch.uint8))
        st.scales.copy_(torch.randint(-2 ** 15, 2 ** 15, st.scales.shape, generator=gen,
                                      dtype=torch.int16))
        gr = torch.randint(-2 ** 15, 2 ** 15, (n,), generator=gen, dtype=torch.int16)
        grads.append(gr.cuda().view(torch.bfloat16))
        states.append(st)
        before.append(state_fields(st))
    lst = F.FlashoptList(states, grads)
    F.flashopt_stream_probe(lst)
    torch.cuda.synchronize()
    for st, gr, b in zip(states, grads, before):
        f = state_fields(st)
        g = gr.view(torch.int16).cpu().numpy().view(np.uint16)
        np.testing.assert_array_equal(f["theta"], b["theta"] ^ g)
        np.testing.assert_array_equal(f["rho"], b["rho"] ^ b["m_code"])
        np.testing.assert_array_equal(f["m_code"], b["m_code"] ^ b["v_code"].view(np.int8))
        np.testing.assert_array_equal(f["v_code"], b["v_code"] ^ b["rho"].view(np.uint8))
        np.testing.assert_array_equal(f["m_scale"], b["m_scale"] ^ 1)
        np.testing.assert_array_equal(f["v_scale"], b["v_scale"] ^ 1)
