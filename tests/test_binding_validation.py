"""The Python binding rejects what the C ABI cannot see -- tensor shapes,
dtypes, devices, strides of the feature dimension and caller buffer sizes --
before any library call touches a device.  CPU tensors stand in for device
memory: every rejection below happens before the device check, and a CPU
tensor that passes every structural check is rejected as not on a GPU."""
import pytest
import torch

from state_passing_amd import linrec

B, H, T, DK, DV = 1, 2, 128, 64, 64


def acts(dtype=torch.bfloat16):
    g = torch.Generator().manual_seed(0)
    mk = lambda d: torch.randn(B, H, T, d, generator=g).to(dtype)  # noqa: E731
    return mk(DK), mk(DK), mk(DV), mk(DV)


def decay():
    return torch.full((H,), 0.99)


def test_fwd_rejects_mismatches():
    q, k, v, _ = acts()
    a = decay()
    with pytest.raises(ValueError, match="k: shape"):
        linrec.fwd(q, k[:, :, :64], v, a)
    with pytest.raises(TypeError, match="k: dtype"):
        linrec.fwd(q, k.float(), v, a)
    with pytest.raises(ValueError, match="v: shape"):
        linrec.fwd(q, k, v[:, :1], a)
    with pytest.raises(ValueError, match="contiguous"):
        linrec.fwd(q, k, v.transpose(2, 3), a) if DV == T else linrec.fwd(q, k, v[..., ::2], a)
    with pytest.raises(TypeError, match="decay must be float32"):
        linrec.fwd(q, k, v, a.double())
    with pytest.raises(ValueError, match="decay must be"):
        linrec.fwd(q, k, v, torch.full((H + 1,), 0.9))
    with pytest.raises(ValueError, match="decay must be"):
        linrec.fwd(q, k, v, torch.full((B, H, T - 64), 0.9))
    with pytest.raises(TypeError, match="S_in: must be float32"):
        linrec.fwd(q, k, v, a, torch.zeros(B, H, DK, DV, dtype=torch.bfloat16))
    with pytest.raises(ValueError, match="S_in: shape"):
        linrec.fwd(q, k, v, a, torch.zeros(B, H, DV, DK + 64))
    with pytest.raises(ValueError, match="S_out: must be contiguous"):
        linrec.fwd(q, k, v, a, S_out=torch.zeros(B, H, DV, DK).transpose(2, 3))
    with pytest.raises(ValueError, match="o: shape"):
        linrec.fwd(q, k, v, a, o=torch.empty(B, H, T, DV + 64, dtype=torch.bfloat16))
    with pytest.raises(ValueError, match="states: .* bytes, the call needs"):
        linrec.fwd(q, k, v, a, states=torch.empty(100, dtype=torch.uint8))
    with pytest.raises(TypeError, match="unsupported activation dtype"):
        linrec.fwd(q.half(), k.half(), v.half(), a)


def test_bwd_rejects_mismatches():
    q, k, v, dO = acts()
    a = decay()
    d = linrec.desc(B, H, T, DK, DV, linrec.BF16, linrec.DECAY_HEAD)
    states = torch.empty(linrec.states_bytes(d), dtype=torch.uint8)
    with pytest.raises(ValueError, match="dO: shape"):
        linrec.bwd(q, k, v, a, states, dO[:, :, :64])
    with pytest.raises(TypeError, match="dO: dtype"):
        linrec.bwd(q, k, v, a, states, dO.float())
    with pytest.raises(ValueError, match="states: .* bytes"):
        linrec.bwd(q, k, v, a, states[:-1], dO)
    with pytest.raises(ValueError, match="workspace: .* bytes"):
        linrec.bwd(q, k, v, a, states, dO, workspace=torch.empty(16, dtype=torch.uint8))
    with pytest.raises(TypeError, match="dS_out: must be float32"):
        linrec.bwd(q, k, v, a, states, dO, torch.zeros(B, H, DK, DV, dtype=torch.float64))
    with pytest.raises(ValueError, match="dS_in: shape"):
        linrec.bwd(q, k, v, a, states, dO, dS_in=torch.zeros(B, H + 1, DK, DV))
    with pytest.raises(TypeError, match="outputs must share one dtype"):
        linrec.bwd(q, k, v, a, states, dO, dq=torch.empty(B, H, T, DK),
                   dk=torch.empty(B, H, T, DK, dtype=torch.bfloat16))
    with pytest.raises(ValueError, match="dv: shape"):
        linrec.bwd(q, k, v, a, states, dO, dv=torch.empty(B, H, T, DK + 64, dtype=torch.bfloat16))


def test_decay_gradient_and_sequence_rejects():
    q, k, v, dO = acts()
    a = torch.full((B, H, T), 0.95)
    d = linrec.desc(B, H, T, DK, DV, linrec.BF16, linrec.DECAY_TOKEN)
    states = torch.empty(linrec.states_bytes(d), dtype=torch.uint8)
    with pytest.raises(ValueError, match="da: must be float32"):
        linrec.bwd_da(q, k, v, a, states, dO, da=torch.empty(B, H, T - 1))
    with pytest.raises(ValueError, match="da_carry: must be"):
        linrec.bwd_da(q, k, v, a, states, dO, None, torch.zeros(B, H + 1))
    with pytest.raises(ValueError, match="needs a decay"):
        linrec.bwd_da(q, k, v, None, states, dO)
    with pytest.raises(ValueError, match="lengths sum"):
        linrec.fwd_seq(q, k, v, a, [64, 128])
    with pytest.raises(ValueError, match="states: .* bytes"):
        linrec.bwd_seq(q, k, v, a, [64, 64], states[:100], dO)
    with pytest.raises(ValueError, match="workspace: .* bytes"):
        linrec.bwd_recompute(q, k, v, a, None, dO, workspace=torch.empty(64, dtype=torch.uint8))


def test_host_tensors_rejected_before_any_device_call():
    q, k, v, dO = acts()
    with pytest.raises(ValueError, match="must be on a GPU"):
        linrec.fwd(q, k, v, decay())
    with pytest.raises(ValueError, match="must be on a GPU"):
        linrec.fwd_seq(q, k, v, decay(), [64, 64])
