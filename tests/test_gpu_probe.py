"""The bandwidth probe (include/flashopt_probe.h) reads and writes every byte
of the AdamW, SGD and Lion steps' state and gradients: its documented XOR of
the values it read, checked on every element of a ragged list (full tiles and
partial tails), through the code planes and records."""
import numpy as np
import pytest
import torch

from compressed_adamw_state_amd import flashopt as F

from parity import state_fields

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("kind", ["adamw", "sgd", "lion"])
def test_stream_probe_touches_every_byte(kind):
    gen = torch.Generator().manual_seed(7)
    sizes = [2048 * 5, 2048 + 7, 33, 8192 + 2047]
    states, grads, before = [], [], []
    for n in sizes:
        st = F.TensorState(n, kind, "cuda")
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
        np.testing.assert_array_equal(f["m_scale"], b["m_scale"] ^ 1)
        if kind == "adamw":
            np.testing.assert_array_equal(f["m_code"], b["m_code"] ^ b["v_code"].view(np.int8))
            np.testing.assert_array_equal(f["v_code"], b["v_code"] ^ b["rho"].view(np.uint8))
            np.testing.assert_array_equal(f["v_scale"], b["v_scale"] ^ 1)
        else:
            np.testing.assert_array_equal(f["m_code"], ~b["m_code"])


def test_stream_probe_refuses_the_fp32_kinds():
    st = F.TensorState(2048, "adamw_fp32", "cuda")
    lst = F.FlashoptList([st], [torch.zeros(2048, dtype=torch.bfloat16, device="cuda")])
    with pytest.raises(F.FlashoptError):
        F.flashopt_stream_probe(lst)


def test_mix_ceiling_touches_every_byte():
    """flashopt_mix_ceiling: theta ^= grad, every code byte ^= 0x5A, every
    scale word ^= 1, over 5 tiles of 2048 parameters (and nothing beyond)."""
    gen = torch.Generator().manual_seed(8)
    n = 2048 * 5
    pad = 64
    theta = torch.randint(-2 ** 15, 2 ** 15, (n + pad,), generator=gen, dtype=torch.int16)
    grad = torch.randint(-2 ** 15, 2 ** 15, (n + pad,), generator=gen, dtype=torch.int16)
    codes = torch.randint(0, 256, (3 * n + pad,), generator=gen, dtype=torch.uint8)
    scales = torch.randint(-2 ** 15, 2 ** 15, (n // 16 + pad,), generator=gen, dtype=torch.int16)
    d = [t.cuda() for t in (theta, grad, codes, scales)]
    F.flashopt_mix_ceiling(d[0], d[1], d[2], d[3], n)
    torch.cuda.synchronize()
    th, gr, cd, sc = (t.cpu() for t in d)
    assert torch.equal(th[:n], theta[:n] ^ grad[:n]) and torch.equal(th[n:], theta[n:])
    assert torch.equal(gr, grad)
    assert torch.equal(cd[:3 * n], codes[:3 * n] ^ 0x5A) and torch.equal(cd[3 * n:], codes[3 * n:])
    assert torch.equal(sc[:n // 16], scales[:n // 16] ^ 1)
    assert torch.equal(sc[n // 16:], scales[n // 16:])


@pytest.mark.parametrize("rw", [(1, 0), (0, 1), (1, 1), (2, 1), (1, 2), (2, 2), (3, 2), (4, 3),
                                (7, 5), (4, 0), (0, 4)])
@pytest.mark.parametrize("in_place", [False, True])
def test_stream_sweep_values(rw, in_place):
    """flashopt_stream_sweep writes the XOR of the buffers read into every
    written buffer, with the written buffer's index in every fourth word."""
    r, w = rw
    if in_place and w > r:
        pytest.skip("in place needs nwrite <= nread")
    gen = torch.Generator().manual_seed(9)
    words = 4 * 1000 + 4            # 1001 units of 16 bytes: a partial block
    reads = [torch.randint(-2 ** 31, 2 ** 31 - 1, (words,), generator=gen, dtype=torch.int32)
             for _ in range(r)]
    writes = [] if in_place else [torch.zeros(words, dtype=torch.int32) for _ in range(w)]
    dr = [t.cuda() for t in reads]
    dw = dr[:w] if in_place else [t.cuda() for t in writes]
    F.flashopt_stream_sweep(dr, dw, 4 * words, in_place=in_place)
    torch.cuda.synchronize()
    acc = torch.zeros(words, dtype=torch.int32)
    for t in reads:
        acc ^= t
    outs = dr[:w] if in_place else dw
    for k, o in enumerate(outs):
        exp = acc.clone()
        exp[0::4] ^= k
        assert torch.equal(o.cpu(), exp), (rw, in_place, k)
    for k in range(w if in_place else 0, r):
        assert torch.equal(dr[k].cpu(), reads[k])


@pytest.mark.parametrize("variant", [0, 1, 2, 3, 4, 5])
def test_pattern_probe_variants(variant):
    """flashopt_pattern_probe: theta ^= grad; each lane's three 8-byte code
    words (a, b, c) -> (a^b, b^c, c^a), the words one per 512-byte plane of a
    1536-byte sub-tile block for variants 0, 3 and 4 and one 24-byte record
    for 5; every byte ^= 0x5A for 1 and 2; every scale word ^= 0x00010001;
    over 7 tiles and nothing beyond (variant 4: every tile once, in its
    hashed order)."""
    gen = torch.Generator().manual_seed(10 + variant)
    n = 2048 * 7
    pad = 64
    theta = torch.randint(-2 ** 15, 2 ** 15, (n + pad,), generator=gen, dtype=torch.int16)
    grad = torch.randint(-2 ** 15, 2 ** 15, (n + pad,), generator=gen, dtype=torch.int16)
    codes = torch.randint(0, 256, (3 * n + pad,), generator=gen, dtype=torch.uint8)
    scales = torch.randint(-2 ** 15, 2 ** 15, (n // 16 + pad,), generator=gen, dtype=torch.int16)
    d = [t.cuda() for t in (theta, grad, codes, scales)]
    F.flashopt_pattern_probe(variant, d[0], d[1], d[2], d[3], n)
    torch.cuda.synchronize()
    th, gr, cd, sc = (t.cpu() for t in d)
    assert torch.equal(th[:n], theta[:n] ^ grad[:n]) and torch.equal(th[n:], theta[n:])
    assert torch.equal(gr, grad)
    if variant in (0, 3, 4, 5):
        # words of one lane: [block][plane][lane] for the planes, [record][word] for 5
        shape = (-1, 3, 64) if variant != 5 else (-1, 3)
        w = codes[:3 * n].view(torch.int64).view(shape)
        exp = torch.stack([w[:, 0] ^ w[:, 1], w[:, 1] ^ w[:, 2], w[:, 2] ^ w[:, 0]], 1)
        assert torch.equal(cd[:3 * n].view(torch.int64).view(shape), exp)
    else:
        assert torch.equal(cd[:3 * n], codes[:3 * n] ^ 0x5A)
    assert torch.equal(cd[3 * n:], codes[3 * n:])
    s32 = scales[:n // 16].view(torch.int32)
    assert torch.equal(sc[:n // 16].view(torch.int32), s32 ^ 0x00010001)
    assert torch.equal(sc[n // 16:], scales[n // 16:])
