"""The binding rejects tensors of the wrong dtype, shape or layout before any library
call: the C ABI takes bare pointers and cannot check these itself, and a wrong one
would make the kernels read or write past a buffer.  CPU tensors suffice, since the
checks run before any pointer is taken (the messages are matched, so the later
"tensors must be on the GPU" error cannot stand in for them)."""
import pytest
import torch

import gated_deltanet_causal_amd as gdn

HK, HV, D = 16, 48, 128
CC = 2 * HK * D + HV * D


def _f32(*s):
    return torch.zeros(*s, dtype=torch.float32)


def _bf16(*s):
    return torch.zeros(*s, dtype=torch.bfloat16)


def _cu(*vals):
    return torch.tensor(vals, dtype=torch.int32)


def _decode_args(B=2, state=None, g=None, z=None, conv_state=None):
    return dict(x=_bf16(B, CC), conv_w=_f32(CC, 4),
                conv_state=_bf16(B, 3, CC) if conv_state is None else conv_state,
                g=_f32(B, HV) if g is None else g, beta=_f32(B, HV),
                z=_bf16(B, HV, D) if z is None else z, norm_w=_f32(D),
                state=_f32(B, HV, D, D) if state is None else state)


def test_decode_rejects_bf16_state():
    with pytest.raises(ValueError, match="state must be"):
        gdn.decode_step(**_decode_args(state=_bf16(2, HV, D, D)))


def test_decode_rejects_state_of_another_batch():
    with pytest.raises(ValueError, match=r"state must have shape \(2, 48, 128, 128\)"):
        gdn.decode_step(**_decode_args(state=_f32(3, HV, D, D)))


def test_decode_rejects_conv_state_of_another_dtype():
    with pytest.raises(ValueError, match="conv_state must be torch.bfloat16"):
        gdn.decode_step(**_decode_args(conv_state=_f32(2, 3, CC)))


def test_decode_rejects_per_channel_g_with_scalar_decay():
    with pytest.raises(ValueError, match=r"g must have shape \(2, 48\)"):
        gdn.decode_step(**_decode_args(g=_f32(2, HV, D)))


def test_decode_rejects_z_of_another_dtype():
    with pytest.raises(ValueError, match="z must be torch.bfloat16"):
        gdn.decode_step(**_decode_args(z=_f32(2, HV, D)))


def _chunk_args(T=70, **over):
    a = dict(q=_bf16(T, HK * D), k=_bf16(T, HK * D), v=_bf16(T, HV * D), g=_f32(T, HV), beta=_f32(T, HV),
             cu=_cu(0, T))
    a.update(over)
    return a


def test_chunk_rejects_bf16_gates():
    with pytest.raises(ValueError, match="g must be torch.float32"):
        gdn.chunk_prefill(**_chunk_args(g=_bf16(70, HV)))
    with pytest.raises(ValueError, match="beta must be torch.float32"):
        gdn.chunk_prefill(**_chunk_args(beta=_bf16(70, HV)))


def test_chunk_rejects_non_contiguous_states():
    s = _f32(1, HV, D, D).transpose(2, 3)
    with pytest.raises(ValueError, match="initial_state must be contiguous"):
        gdn.chunk_prefill(**_chunk_args(), initial_state=s)
    with pytest.raises(ValueError, match="final_state must be contiguous"):
        gdn.chunk_prefill(**_chunk_args(), final_state=s)


def test_chunk_rejects_wrong_widths_and_lengths():
    with pytest.raises(ValueError, match="k must be"):
        gdn.chunk_prefill(**_chunk_args(k=_bf16(70, HK * D - 8)))
    with pytest.raises(ValueError, match="v must be"):
        gdn.chunk_prefill(**_chunk_args(v=_bf16(69, HV * D)))
    with pytest.raises(ValueError, match="k must be torch.bfloat16"):
        gdn.chunk_prefill(**_chunk_args(k=_f32(70, HK * D)))
    with pytest.raises(ValueError, match="cu_seqlens must be"):
        gdn.chunk_prefill(**_chunk_args(cu=torch.tensor([0, 70], dtype=torch.int64)))


def test_chunk_rejects_scalar_g_with_per_channel_decay():
    cfg = gdn.config(decay_per_key_channel=1)
    with pytest.raises(ValueError, match=r"g must have shape \(70, 48, 128\)"):
        gdn.chunk_prefill(**_chunk_args(), cfg=cfg)


def test_conv_rejects_state_dtype_and_width():
    x = _bf16(10, CC)
    with pytest.raises(ValueError, match="conv_state_in must be torch.bfloat16"):
        gdn.conv1d_prefill(x, _f32(CC, 4), _cu(0, 10), conv_state_in=_f32(1, 3, CC))
    with pytest.raises(ValueError, match="x must be"):
        gdn.conv1d_prefill(_bf16(10, CC - 128), _f32(CC, 4), _cu(0, 10))
    with pytest.raises(ValueError, match="conv weight must be"):
        gdn.conv1d_prefill(x, _bf16(CC, 4), _cu(0, 10))
    with pytest.raises(ValueError, match="conv_state must have shape"):
        gdn.conv1d_step(_bf16(2, CC), _f32(CC, 4), _bf16(2, 2, CC))


def test_prefill_rejects_wrong_final_state_and_z():
    T = 20
    args = (_bf16(T, CC), _f32(CC, 4), _cu(0, T), _f32(T, HV), _f32(T, HV))
    with pytest.raises(ValueError, match="final_state must have shape"):
        gdn.prefill(*args, _bf16(T, HV, D), _f32(D), final_state=_f32(2, HV, D, D))
    with pytest.raises(ValueError, match="z must be torch.bfloat16"):
        gdn.prefill(*args, _f32(T, HV, D), _f32(D))
    with pytest.raises(ValueError, match="norm weight must"):
        gdn.prefill(*args, _bf16(T, HV, D), _f32(D + 1))


def test_norm_and_verify_reject_wrong_shapes():
    with pytest.raises(ValueError, match="z must have shape"):
        gdn.gated_rmsnorm(_f32(4, HV, D), _f32(4, HV, D - 1), _f32(D))
    B, K = 2, 3
    with pytest.raises(ValueError, match="state must be torch.float32"):
        gdn.verify(_bf16(B, K, CC), _f32(CC, 4), _bf16(B, 3, CC), _f32(B, K, HV), _f32(B, K, HV),
                   _bf16(B, K, HV, D), _f32(D), _bf16(B, HV, D, D))
    with pytest.raises(ValueError, match="beta must have shape"):
        gdn.verify(_bf16(B, K, CC), _f32(CC, 4), _bf16(B, 3, CC), _f32(B, K, HV), _f32(B, HV),
                   _bf16(B, K, HV, D), _f32(D), _f32(B, HV, D, D))


def test_state_convert_rejects_other_dtypes():
    with pytest.raises(ValueError, match="state must be"):
        gdn.state_convert(_bf16(1, HV, D, D), torch.float32)
    with pytest.raises(ValueError, match="converts between"):
        gdn.state_convert(_f32(1, HV, D, D), torch.float32)


def test_row_stride_of_empty_and_strided_rows():
    """Row strides the binding passes on: an empty tensor counts as packed rows whatever
    strides it reports (numpy-made empties report zeros), a row-strided view its own stride,
    and a view whose inner dimensions are not contiguous is refused."""
    import numpy as np
    empty = torch.from_numpy(np.zeros((0, CC), dtype=np.float32)).to(torch.bfloat16)
    assert gdn._row_stride(empty) == CC
    assert gdn._row_stride(torch.zeros(0, HV, D)) == HV * D
    wide = torch.zeros(4, CC + 64)
    assert gdn._row_stride(wide[:, :CC]) == CC + 64
    with pytest.raises(ValueError, match="inner dimensions must be contiguous"):
        gdn._row_stride(torch.zeros(4, 2 * CC)[:, ::2])
