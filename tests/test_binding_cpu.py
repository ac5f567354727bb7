"""The Python binding rejects tensors whose dtype, size, layout or device do
not match include/moe_verify.h before anything reaches the C ABI (the C side
sees only pointers, so a short or mistyped buffer would make the kernels read
or write outside it).  CPU only: every case raises before a launch."""
import numpy as np
import pytest
import torch

import moe_speculative_decoding_router_amd as m

CPU = torch.device("cpu")


def bf16_layer(H=128, I=64, E=8, k=2, shared=False, **over):
    d = dict(H=H, I=I, E=E, k=k, wdtype="bf16", Wr=torch.zeros(E, H),
             W_gu=torch.zeros(E, 2 * I, H, dtype=torch.int16), W_d=torch.zeros(E, H, I, dtype=torch.int16))
    if shared:
        d.update(Wsh_gu=torch.zeros(2 * I, H, dtype=torch.int16), Wsh_d=torch.zeros(H, I, dtype=torch.int16))
    d.update(over)
    return m.LayerWeights(**d)


def fp8_layer(H=256, I=128, E=4, k=2, shared=True, **over):
    d = dict(H=H, I=I, E=E, k=k, wdtype="fp8", Wr=torch.zeros(E, H),
             W_gu=torch.zeros(E, 2 * I, H, dtype=torch.uint8), W_d=torch.zeros(E, H, I, dtype=torch.uint8),
             s_gu=torch.ones(E, 2 * I // 128, H // 128), s_d=torch.ones(E, H // 128, I // 128))
    if shared:
        d.update(Wsh_gu=torch.zeros(2 * I, H, dtype=torch.uint8), Wsh_d=torch.zeros(H, I, dtype=torch.uint8),
                 ssh_gu=torch.ones(2 * I // 128, H // 128), ssh_d=torch.ones(H // 128, I // 128))
    d.update(over)
    return m.LayerWeights(**d)


def test_well_formed_layers_pass():
    bf16_layer().validate(CPU)
    bf16_layer(shared=True).validate(CPU)
    fp8_layer().validate(CPU)
    fp8_layer(shared=False).validate(CPU)
    bf16_layer(W_gu=torch.zeros(8, 128, 128, dtype=torch.bfloat16)).validate(CPU)


@pytest.mark.parametrize("over,msg", [
    (dict(Wr=torch.zeros(8, 128, dtype=torch.float64)), "Wr"),
    (dict(Wr=torch.zeros(7, 128)), "Wr"),
    (dict(W_gu=torch.zeros(8, 2 * 32, 128, dtype=torch.int16)), "W_gu"),         # I of another layer
    (dict(W_gu=torch.zeros(8, 128, 128, dtype=torch.uint8)), "W_gu"),            # fp8 codes in a bf16 layer
    (dict(W_d=torch.zeros(8, 64, 128, dtype=torch.int16).transpose(1, 2)), "W_d"),  # not contiguous
    (dict(W_d=torch.zeros(8, 128, 64, dtype=torch.float32)), "W_d"),
    (dict(Wsh_gu=torch.zeros(128, 128, dtype=torch.int16)), "shared"),          # half a shared expert
    (dict(s_gu=torch.ones(8, 1, 1)), "s_gu"),                                    # scales in a bf16 layer
    (dict(Wr=torch.zeros(8, 128, device="meta")), "Wr"),                        # another device
])
def test_bad_bf16_layer_rejected(over, msg):
    with pytest.raises(ValueError, match=msg):
        bf16_layer(**over).validate(CPU)


@pytest.mark.parametrize("over,msg", [
    (dict(s_gu=None), "s_gu"),
    (dict(s_d=torch.ones(4, 1, 1)), "s_d"),
    (dict(ssh_gu=None), "ssh_gu"),
    (dict(ssh_d=torch.ones(2, 1, dtype=torch.float16)), "ssh_d"),
    (dict(W_gu=torch.zeros(4, 256, 256, dtype=torch.int16)), "W_gu"),
    (dict(H=192, Wr=torch.zeros(4, 192)), "multiples of 128"),
])
def test_bad_fp8_layer_rejected(over, msg):
    with pytest.raises(ValueError, match=msg):
        fp8_layer(**over).validate(CPU)


def test_verify_layer_rejects_host_and_mistyped_inputs():
    L = bf16_layer()
    with pytest.raises(ValueError, match="device"):
        m.verify_layer(torch.zeros(5, 128), L)
    with pytest.raises(ValueError, match="x"):
        m.verify_layer(torch.zeros(5, 128, dtype=torch.float64), L)
    with pytest.raises(ValueError, match="x"):
        m.verify_layer(torch.zeros(5, 64), L)
    with pytest.raises(ValueError, match="x"):
        m.verify_layer(torch.zeros(5), L)


def test_workspace_checks():
    L = bf16_layer()
    T = 5
    need = m.workspace_bytes(L, T)
    aux = m.alloc_aux(L, T, CPU)
    good = m.Workspace(ws=torch.zeros(need, dtype=torch.uint8), nbytes=need, aux=aux)
    m._check_workspace(good, L, T, None, CPU)
    with pytest.raises(ValueError, match="needs"):
        m._check_workspace(m.Workspace(ws=torch.zeros(need, dtype=torch.uint8), nbytes=need - 256, aux=aux),
                           L, T, None, CPU)
    with pytest.raises(ValueError, match="workspace.ws"):
        m._check_workspace(m.Workspace(ws=torch.zeros(need - 1, dtype=torch.uint8), nbytes=need, aux=aux),
                           L, T, None, CPU)
    # aux sized for fewer tokens or fewer experts
    small = m.alloc_aux(L, 2, CPU)
    with pytest.raises(ValueError, match="aux"):
        m._check_workspace(m.Workspace(ws=good.ws, nbytes=need, aux=small), L, T, None, CPU)
    other = m.alloc_aux(bf16_layer(E=4, Wr=torch.zeros(4, 128), W_gu=torch.zeros(4, 128, 128, dtype=torch.int16),
                                   W_d=torch.zeros(4, 128, 64, dtype=torch.int16)), T, CPU)
    with pytest.raises(ValueError, match="aux"):
        m._check_workspace(m.Workspace(ws=good.ws, nbytes=need, aux=other), L, T, None, CPU)
    bad = m.alloc_aux(L, T, CPU)
    bad.topk_idx = torch.zeros(T, 2, dtype=torch.int64)
    with pytest.raises(ValueError, match="topk_idx"):
        m._check_workspace(m.Workspace(ws=good.ws, nbytes=need, aux=bad), L, T, None, CPU)


def test_output_buffers_of_statistics_and_selection():
    idx = torch.zeros(3, 5, 2, dtype=torch.int32)
    with pytest.raises(ValueError, match="counts"):
        m.union_stats(idx, 8, counts=torch.zeros(2, dtype=torch.int32), reuse=torch.zeros(3))
    with pytest.raises(ValueError, match="reuse"):
        m.union_stats(idx, 8, counts=torch.zeros(3, dtype=torch.int32), reuse=torch.zeros(3, dtype=torch.float64))
    P = torch.zeros(2, 6)
    F = torch.zeros(2, 6, 4, dtype=torch.int32)
    with pytest.raises(ValueError, match="out"):
        m.select_drafts(np.full(6, -1), P, F, 3, out=torch.zeros(2, 2, dtype=torch.int32))
    with pytest.raises(ValueError, match="out"):
        m.select_drafts(np.full(6, -1), P, F, 3, out=torch.zeros(2, 3, dtype=torch.int64))
    with pytest.raises(ValueError, match="same device"):
        m.select_drafts(np.full(6, -1), P, F.to("meta"), 3)
