"""The entry point that allocates nothing (sa_select_attend_noalloc, for callers that cannot
allocate device memory): through the C ABI, its outputs equal sa_select_attend's bit for
bit on consecutive calls of decreasing size -- later calls find the library's scratch
holding the earlier calls' data -- and a caller-supplied status word reports non-finite
index inputs."""
import numpy as np
import pytest
import torch

import sa_synth
import token_selector_gather_amd as sa
from tests import gpu_common as gc
from tests.device_inputs import empty_outputs
from token_selector_gather_amd.inputs import device_workload

pytestmark = pytest.mark.gpu

# a decode batch (sliced top-k, split latent attention), a bf16 multi-head prefill (tile
# attention, register top-k), then a smaller decode batch
CASES = [
    ("decode_b16_kv20000_k1024", dict(cid=3, B=16, n_kv=20000, k=1024)),
    ("prefill_bf16_n512", dict(cid=1, n=512)),
    ("decode_b4_kv3000_k256", dict(cid=3, B=4, n_kv=3000, k=256)),
]


def _run(W, P, d, noalloc, status=None):
    O, lse, idx = empty_outputs(W, gc.out_dtype(W))
    if noalloc:
        sa.sa_select_attend_noalloc(P, d["q_idx"], d["k_idx"], d["w"], d["Q"], d["K"], d["V"], idx, O, lse, status)
        st = sa.sa_device_status(status) if status is not None else sa.SA_OK
    else:
        ws = sa.workspace(P, sa.SA_OP_SELECT_ATTEND)
        sa.sa_select_attend(P, d["q_idx"], d["k_idx"], d["w"], d["Q"], d["K"], d["V"], idx, O, lse, ws)
        st = sa.sa_device_status(ws)
    torch.cuda.synchronize()
    return idx, O, lse, st


def _bits(t):
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t.view(torch.int32)


def test_no_alloc_equals_the_workspace_call_on_consecutive_calls():
    status = torch.zeros(256, dtype=torch.uint8, device="cuda")
    for name, kw in CASES:
        print("no-alloc %s" % name, flush=True)
        W = sa_synth.make_config(**kw)
        P, d = device_workload(W)
        assert sa.sa_workspace_bytes(P, sa.SA_OP_SELECT_ATTEND) <= 64 << 20
        a = _run(W, P, d, False)
        b = _run(W, P, d, True, status)
        assert a[3] == sa.SA_OK and b[3] == sa.SA_OK
        assert torch.equal(a[0], b[0]), name
        assert torch.equal(_bits(a[1]), _bits(b[1])), name
        assert torch.equal(_bits(a[2]), _bits(b[2])), name


def test_no_alloc_reports_nonfinite_inputs_in_the_callers_status_word():
    W = sa_synth.make_config(3, B=4, n_kv=3000, k=256)
    P, d = device_workload(W)
    status = torch.zeros(256, dtype=torch.uint8, device="cuda")
    d["q_idx"][2, 0, 5, 7] = float("nan")
    assert _run(W, P, d, True, status)[3] == sa.SA_ERR_NONFINITE
    d["q_idx"][2, 0, 5, 7] = 0.5
    assert _run(W, P, d, True, status)[3] == sa.SA_OK  # cleared by the read


def test_no_alloc_rejects_problems_beyond_its_scratch():
    W = sa_synth.custom(B=1, n_q=4096, n_kv=4096, Hq=2, Hkv=2, d_qk=64, d_v=64, Hidx=8, d_idx=64, k=64)
    P, d = device_workload(W)
    assert sa.sa_workspace_bytes(P, sa.SA_OP_SELECT_ATTEND) > 64 << 20
    O, lse, idx = empty_outputs(W, torch.bfloat16)
    with pytest.raises(sa.SaError) as e:
        sa.sa_select_attend_noalloc(P, d["q_idx"], d["k_idx"], d["w"], d["Q"], d["K"], d["V"], idx, O, lse)
    assert e.value.status == sa.SA_ERR_WORKSPACE
