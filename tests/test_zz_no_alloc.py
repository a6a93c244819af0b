"""gdn_chunk_prefill_noalloc (the chunk prefill with the library's fixed device scratch
as its workspace) against gdn_chunk_prefill with a caller workspace: the same kernels,
so outputs and final states must be bit-identical.  Two calls in a row, the second
smaller, so the second runs over scratch the first left behind."""
import ctypes

import numpy as np
import pytest
import torch

import gated_deltanet_causal_amd as gdn
import gdn_inputs as gi
from gpu_common import dev, dev_i32

pytestmark = pytest.mark.gpu

HK, HV, D = gi.HK, gi.HV, gi.DK


def _both(d, out_dtype):
    q, k, v = dev(d["q"], True), dev(d["k"], True), dev(d["v"], True)
    g, beta, cu = dev(d["g"]), dev(d["beta"]), dev_i32(d["cu"])
    s0 = dev(d["state_in"])
    T, N = q.shape[0], len(d["cu"]) - 1
    ref_o, ref_s = gdn.chunk_prefill(q, k, v, g, beta, cu, cu_host=d["cu"], initial_state=s0,
                                     out_dtype=out_dtype)
    out = torch.full((T, HV, D), float("nan"), dtype=out_dtype, device=q.device)
    fs = torch.full((N, HV, D, D), float("nan"), dtype=torch.float32, device=q.device)
    cfg = gdn.config()
    hc = (ctypes.c_int32 * (N + 1))(*[int(x) for x in d["cu"]])
    qk_stride = q.stride(0)
    status = gdn.load_library().gdn_chunk_prefill_noalloc(
        ctypes.byref(cfg), gdn.GDN_BF16, gdn._dtype(out), ctypes.c_void_p(q.data_ptr()),
        ctypes.c_void_p(k.data_ptr()), qk_stride, ctypes.c_void_p(v.data_ptr()), v.stride(0),
        ctypes.c_void_p(g.data_ptr()), ctypes.c_void_p(beta.data_ptr()), ctypes.c_void_p(s0.data_ptr()),
        ctypes.c_void_p(cu.data_ptr()), hc, N, T, ctypes.c_void_p(out.data_ptr()),
        ctypes.c_void_p(fs.data_ptr()), ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert status == gdn.GDN_OK, gdn.load_library().gdn_status_string(status)
    torch.cuda.synchronize()
    return ref_o, ref_s, out, fs


def test_noalloc_chunk_prefill_matches_workspace_call_twice():
    for seed, lengths, odt in ((3100, [700, 65, 129], torch.float32), (3101, [70, 0, 1, 64], torch.bfloat16)):
        print(f"[no-alloc] lengths {lengths} out {odt}", flush=True)
        d = gi.gen_qkv(seed, lengths)
        ref_o, ref_s, out, fs = _both(d, odt)
        assert torch.equal(out, ref_o), f"out differs for {lengths}"
        assert torch.equal(fs, ref_s), f"final state differs for {lengths}"


def test_noalloc_binding_full_4096_tokens():
    """The binding's no-alloc call at the 4096-token single-sequence size (105 MB of the
    128 MiB scratch), bit-identical to the workspace call."""
    d = gi.gen_qkv(3102, [4096])
    q, k, v = dev(d["q"], True), dev(d["k"], True), dev(d["v"], True)
    g, beta, cu = dev(d["g"]), dev(d["beta"]), dev_i32(d["cu"])
    s0 = dev(d["state_in"])
    ref_o, ref_s = gdn.chunk_prefill(q, k, v, g, beta, cu, cu_host=d["cu"], initial_state=s0,
                                     out_dtype=torch.bfloat16)
    out = torch.empty_like(ref_o)
    fs = torch.empty_like(ref_s)
    gdn.chunk_prefill_noalloc(q, k, v, g, beta, cu, cu_host=d["cu"], initial_state=s0, out=out, final_state=fs)
    torch.cuda.synchronize()
    assert torch.equal(out, ref_o) and torch.equal(fs, ref_s)
