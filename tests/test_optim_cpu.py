"""Host-side checks of the torch.optim front end (no GPU needed)."""
import pytest
import torch

import muon_newton_schulz_06_amd as mns


def _params():
    return [torch.nn.Parameter(torch.zeros(8, 16, dtype=torch.bfloat16)),
            torch.nn.Parameter(torch.zeros(16, 4))]


def test_accepts_matrices_and_defaults():
    opt = mns.Muon(_params())
    g = opt.param_groups[0]
    assert g["lr"] == 0.02 and g["momentum"] == 0.95 and g["ns_steps"] == 5
    assert g["ns_coefficients"] == mns.QUINTIC and g["nesterov"] is False


@pytest.mark.parametrize("kw", [
    dict(lr=-1.0), dict(lr=float("nan")), dict(momentum=float("inf")),
    dict(weight_decay=-0.1), dict(eps=-1.0), dict(ns_steps=65), dict(ns_steps=2.5),
    dict(ns_coefficients=(1.0, 2.0)), dict(ns_coefficients=(1.0, float("nan"), 0.0)),
    dict(nesterov=1),
])
def test_rejects_bad_hyperparameters(kw):
    with pytest.raises(ValueError):
        mns.Muon(_params(), **kw)


def test_rejects_non_matrix_and_bad_dtype():
    with pytest.raises(ValueError):
        mns.Muon([torch.nn.Parameter(torch.zeros(8))])
    with pytest.raises(TypeError):
        mns.Muon([torch.nn.Parameter(torch.zeros(4, 4, dtype=torch.float16))])
    opt = mns.Muon(_params())
    with pytest.raises(ValueError):
        opt.add_param_group({"params": [torch.nn.Parameter(torch.zeros(3, 3))], "lr": -2.0})


def test_step_without_gradients_is_a_noop():
    ps = _params()
    opt = mns.Muon(ps)
    opt.step()
    assert all(p.abs().sum() == 0 for p in ps) and len(opt.state) == 0


def test_cpu_tensors_fail_loudly():
    """There is no CPU fallback: CPU tensors are refused by the binding."""
    ps = _params()
    for p in ps:
        p.grad = torch.ones_like(p)
    opt = mns.Muon(ps)
    with pytest.raises((ValueError, ImportError)):
        opt.step()


def test_state_dict_round_trip_keeps_fp32_momentum():
    """torch casts floating state to the parameter dtype on load; the
    momentum of a bf16 matrix must come back as the saved fp32 values."""
    ps = _params()
    opt = mns.Muon(ps, lr=0.01, nesterov=True, weight_decay=0.1)
    vals = []
    for p in ps:
        buf = torch.randn(p.shape, dtype=torch.float32) * 1e-3 + 1e-4
        opt.state[p]["momentum_buffer"] = buf
        vals.append(buf.clone())
    sd = opt.state_dict()
    ps2 = _params()
    opt2 = mns.Muon(ps2)
    opt2.load_state_dict(sd)
    for p, v in zip(ps2, vals):
        b = opt2.state[p]["momentum_buffer"]
        assert b.dtype == torch.float32 and torch.equal(b, v)
    g = opt2.param_groups[0]
    assert g["lr"] == 0.01 and g["nesterov"] is True and g["weight_decay"] == 0.1


@pytest.mark.parametrize("kw", [
    dict(selected_fraction=0.0), dict(selected_fraction=1.5), dict(selected_fraction=float("nan")),
    dict(selected_fraction=0.5, nesterov=True), dict(selected_fraction=0.5, weight_decay=0.1),
])
def test_rejects_bad_selected_fraction(kw):
    with pytest.raises(ValueError):
        mns.Muon(_params(), **kw)


def test_selected_fraction_default_and_accepted():
    assert mns.Muon(_params()).param_groups[0]["selected_fraction"] is None
    assert mns.Muon(_params(), selected_fraction=0.25).param_groups[0]["selected_fraction"] == 0.25
