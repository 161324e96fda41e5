"""The allocation-free entry point grpo_loss_fwd_bwd_static against grpo_loss_fwd_bwd: two
calls in a row on the device's static scratch (the second smaller, with the first call's bytes
still in the scratch), every output bitwise equal to the workspace entry point's."""
import gc

import numpy as np
import pytest
import torch

from rl_fine_tuning_amd import grpo_loss_fwd_bwd, grpo_loss_fwd_bwd_static, grpo_workspace_bytes
from rl_fine_tuning_amd.grpo import GRPO_STATIC_SCRATCH_BYTES

from gpu_cases import case, say, to_device

pytestmark = pytest.mark.gpu


def _outputs(k, d):
    T, D = k["T"], k["D"]
    dev = d["H"].device
    return dict(loss=torch.empty(1, dtype=torch.float64, device=dev),
                logp=torch.empty(T, dtype=torch.float32, device=dev),
                token_loss=torch.empty(T, dtype=torch.float32, device=dev),
                dH=torch.empty(T, D, dtype=d["H"].dtype, device=dev))


@pytest.mark.parametrize("dW", [False, True])
def test_static_entry_matches_workspace_entry(dW):
    runs = [dict(seed=201, D=512, V=20000, lengths=[900, 1100, 700, 300], chunk=1024),
            dict(seed=202, D=512, V=20000, lengths=[400, 250], chunk=256)]  # second call smaller
    for r in runs:
        k = case(r["seed"], D=r["D"], V=r["V"], lengths=r["lengths"], G=2, chunk=r["chunk"], old_std=0.3,
                 ref_std=0.3, beta=0.05, mask_frac=0.1, bad_targets=(3,))
        need = grpo_workspace_bytes(k["T"], r["D"], r["V"], r["chunk"], num_seqs=len(r["lengths"]), with_dW=dW)
        assert need <= GRPO_STATIC_SCRATCH_BYTES
        say(f"static entry: T={k['T']} D={r['D']} V={r['V']} chunk={r['chunk']} dW={dW}; workspace {need} bytes")
        d = to_device(k)
        kw = dict(temperature=k["tau"], mask=d["mask"], **k["prm"])
        out = _outputs(k, d)
        if dW:
            out["dW"] = torch.empty(r["V"], r["D"], dtype=torch.float32, device=d["H"].device)
        gc.collect()
        torch.cuda.synchronize()
        before = torch.cuda.memory_stats()["allocation.all.allocated"]  # cumulative allocation requests
        got = grpo_loss_fwd_bwd_static(d["H"], d["W"], d["targets"], k["c"].cu, d["old"], d["ref"], d["adv"],
                                       r["chunk"], **out, **kw)
        torch.cuda.synchronize()
        assert torch.cuda.memory_stats()["allocation.all.allocated"] == before  # outputs passed in: no allocation
        ref = grpo_loss_fwd_bwd(d["H"], d["W"], d["targets"], k["c"].cu, d["old"], d["ref"], d["adv"], r["chunk"],
                                dW=True if dW else None, **kw)
        torch.cuda.synchronize()
        keys = ["loss", "logp", "token_loss", "dH"] + (["dW"] if dW else [])
        for key in keys:
            a, b = got[key], ref[key]
            bits = {torch.float64: torch.int64, torch.float32: torch.int32, torch.bfloat16: torch.int16}[a.dtype]
            assert torch.equal(a.view(bits), b.view(bits)), key  # bit patterns (NaN at the invalid target)
        assert np.isnan(got["logp"][3].item())
