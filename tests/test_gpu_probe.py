"""The bandwidth probe (include/flashopt_probe.h) reads and writes every byte
of the AdamW step's state and gradients: its documented XOR of the values it
read, checked word for word on a ragged list (full tiles and partial tails)."""
import numpy as np
import pytest
import torch

from compressed_adamw_state_amd import flashopt as F

pytestmark = pytest.mark.gpu


def _rand_bytes(n, dtype, gen):
    b = torch.randint(0, 256, (n * torch.empty(0, dtype=dtype).element_size(),),
                      generator=gen, dtype=torch.uint8)
    return b.view(dtype).cuda()


def test_stream_probe_touches_every_byte():
    gen = torch.Generator().manual_seed(7)
    sizes = [2048 * 5, 2048 + 7, 33, 8192 + 2047]
    states, grads, before = [], [], []
    for n in sizes:
        st = F.TensorState(n, "adamw", "cuda")
        st.theta.copy_(_rand_bytes(n, torch.int16, gen).view(torch.bfloat16))
        st.rho.copy_(_rand_bytes(n, torch.int8, gen))
        st.m_code.copy_(_rand_bytes(n, torch.int8, gen))
        st.v_code.copy_(_rand_bytes(n, torch.uint8, gen))
        g = (n + 31) // 32
        st.m_scale.copy_(_rand_bytes(g, torch.int16, gen).view(torch.float16))
        st.v_scale.copy_(_rand_bytes(g, torch.int16, gen).view(torch.float16))
        gr = _rand_bytes(n, torch.int16, gen).view(torch.bfloat16)
        states.append(st)
        grads.append(gr)
        before.append({k: v.clone() for k, v in st.arrays().items()})
    lst = F.FlashoptList(states, grads)
    F.flashopt_stream_probe(lst)
    torch.cuda.synchronize()
    for st, gr, b in zip(states, grads, before):
        h = lambda t: t.view(torch.int16).cpu().numpy() if t.element_size() == 2 else \
            t.cpu().numpy().view(np.uint8)
        np.testing.assert_array_equal(h(st.theta), h(b["theta"]) ^ h(gr))
        np.testing.assert_array_equal(h(st.rho), h(b["rho"]) ^ h(b["m_code"]))
        np.testing.assert_array_equal(h(st.m_code), h(b["m_code"]) ^ h(b["v_code"]))
        np.testing.assert_array_equal(h(st.v_code), h(b["v_code"]) ^ h(b["rho"]))
        np.testing.assert_array_equal(h(st.m_scale), h(b["m_scale"]) ^ 1)
        np.testing.assert_array_equal(h(st.v_scale), h(b["v_scale"]) ^ 1)
