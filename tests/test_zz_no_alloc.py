"""The prefill entry point that allocates nothing (gdn_prefill_noalloc, its workspace in the
library's static device array) against gdn_prefill with a caller workspace, through the C
ABI: outputs and states bit-identical, on two calls in a row, the second with a smaller
input, after the static array has been left holding the first call's packages."""

import numpy as np
import pytest
import torch

import gated_deltanet_speculative_amd as gdn
from gpu_util import dev, log
from workloads import synth_case

pytestmark = pytest.mark.gpu


def _case(C, T, P, Hk, Hv, d, seed):
    case = synth_case(C, T, P, Hk, Hv, d, d, seed=seed, tree=False)
    rng = np.random.default_rng(seed)
    case["qkv"] = rng.standard_normal(case["x"].shape).astype(np.float32)
    case["z"] = rng.standard_normal((C, T, Hv, d)).astype(np.float32)
    return case


def _run(case, Hk, noalloc, gate_mode):
    C, T, Ch = case["qkv"].shape
    P, Hv, dk, dv = case["state"].shape
    sh = gdn.Shape(C, T, P, Hk, Hv, dk, dv)
    state = dev(case["state"])
    ba = dev(case["ba"])
    out = torch.full((C, T, Hv, dv), float("nan"), device="cuda")
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    args = (sh, dev(case["qkv"]), ba[..., :Hv], ba[..., Hv:], dev(case["dt_bias"]), dev(case["A"]), state,
            dev(case["slot_ids"]), status)
    z = dev(case["z"]) if gate_mode is not None else None
    if noalloc:
        gdn.prefill_noalloc(*args, out=out, gate_z=z, gate_mode=gate_mode or 0)
    else:
        ws = torch.full((gdn.prefill_workspace_size(sh) // 4,), float("nan"), device="cuda")
        gdn.prefill(*args, gate_z=z, gate_mode=gate_mode or 0, out=out, workspace=ws)
    return state, out, status


def test_noalloc_prefill_matches_caller_workspace():
    calls = [
        # C, T, P, Hk, Hv, d, gate: the prefill bench shape (19 MB of packages), then a smaller one
        (4, 1024, 8, 16, 32, 128, None),
        (2, 53, 3, 2, 4, 64, 1),
    ]
    for k, (C, T, P, Hk, Hv, d, gate) in enumerate(calls):
        log(f"[noalloc] call {k}: C={C} T={T} Hk={Hk} Hv={Hv} d={d} gate={gate}")
        case = _case(C, T, P, Hk, Hv, d, seed=500 + k)
        st_n, out_n, status_n = _run(case, Hk, True, gate)
        st_w, out_w, status_w = _run(case, Hk, False, gate)
        torch.cuda.synchronize()
        assert int(status_n.item()) == 0 and int(status_w.item()) == 0
        assert torch.equal(out_n, out_w), f"call {k}: outputs differ"
        assert torch.equal(st_n, st_w), f"call {k}: states differ"
        assert not torch.isnan(out_n).any()


def test_noalloc_prefill_rejects_an_oversized_shape():
    sh = gdn.Shape(4, 4096, 8, 16, 32, 128, 128)  # 49 MB of packages against 32 MiB
    t = torch.zeros(1, device="cuda")
    with pytest.raises(gdn.GdnError) as ei:
        gdn.prefill_noalloc(sh, torch.zeros((4, 4096, sh.channels), device="cuda"),
                            torch.zeros((4, 4096, 32), device="cuda"), torch.zeros((4, 4096, 32), device="cuda"),
                            torch.zeros(32, device="cuda"), torch.zeros(32, device="cuda"),
                            torch.zeros((8, 32, 128, 128), device="cuda"), torch.arange(4, dtype=torch.int32,
                                                                                        device="cuda"),
                            torch.zeros(1, dtype=torch.int32, device="cuda"),
                            torch.zeros((4, 4096, 32, 128), device="cuda"))
    assert ei.value.code == gdn._lib.GDN_ERR_SCRATCH
    del t
