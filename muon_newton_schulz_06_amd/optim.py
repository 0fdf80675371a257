"""`torch.optim` front end of the library: Muon for 2-D weight matrices.

The optimiser step is the owner-side update of the DMuon technical summary
(gist.science, Korean), §1 and §2.2 — momentum, Frobenius normalisation,
Newton–Schulz in the Gram formulation, shape-scaled update — used as a
drop-in optimiser module (§3 of the same page: the module replaces the
optimiser and changes nothing else in the training framework).  Every step
runs in the library's HIP kernels through `muon_step` / `muon_step_ex`;
this class only groups tensors and keeps the momentum state.  A group with
`selected_fraction` set runs the row/column-selected step with error
feedback instead (`muon_step_selected`; Dion3 review, blog.secrett2633.cloud,
§3 "Method & Key Results" and §1 "Error Feedback").

Only 2-D parameters are accepted (Muon orthogonalises matrices; biases,
norms and embeddings belong in another optimiser).  Parameters may be bf16
or fp32, gradients fp32 or bf16; the momentum is always kept in fp32.
"""
from __future__ import annotations

import itertools
import math

import torch

from . import QUINTIC, SCALE_EXP_UNKNOWN, muon_step, muon_step_selected


class Muon(torch.optim.Optimizer):
    """Muon with Gram Newton–Schulz orthogonalisation on the GPU.

    Arguments (per parameter group):
      lr:              learning rate; the update of a rows × cols matrix is
                       scaled by lr·√max(1, rows/cols)
      momentum:        β of M ← β·M + g
      nesterov:        orthogonalise g + β·M (after the update) instead of M
      weight_decay:    decoupled, W ← (1 − lr·weight_decay)·W − lr·sc·O
      ns_steps:        Newton–Schulz steps (0–64)
      ns_coefficients: (a, b, c) of X ← a·X + (b·A + c·A²)·X, A = X·Xᵀ
      eps:             added to ‖M‖_F before normalising
      selected_fraction: None for the plain step; ρ in (0, 1] for the
                       row/column-selected step: only the ⌈ρ·m⌉ highest-norm
                       rows of B = M + g along the short side are
                       orthogonalised and applied, the buffer keeps β·B there
                       and B elsewhere (not combinable with nesterov or
                       weight_decay; bf16 gradients are widened to fp32)
    carry_exponents (optimiser-wide, default True): keep each matrix's
                       power-of-two operand exponent between steps (state
                       "operand_exp", an int32 scalar) and pass them as
                       muon_step_ex's scale_exp, so the momentum pass writes
                       the half-precision operand itself (no separate cast
                       pass over the fp32 momentum after the first step)
    """

    def __init__(self, params, lr: float = 0.02, momentum: float = 0.95, nesterov: bool = False,
                 weight_decay: float = 0.0, ns_steps: int = 5, ns_coefficients=QUINTIC,
                 eps: float = 1e-7, selected_fraction=None, carry_exponents: bool = True):
        self._carry = bool(carry_exponents)
        self._exp_bufs: dict = {}
        defaults = dict(lr=lr, momentum=momentum, nesterov=nesterov, weight_decay=weight_decay,
                        ns_steps=ns_steps, ns_coefficients=tuple(ns_coefficients), eps=eps,
                        selected_fraction=selected_fraction)
        _check_hyper(defaults)
        super().__init__(params, defaults)
        for group in self.param_groups:
            _check_hyper(group)
            for p in group["params"]:
                if p.dim() != 2:
                    raise ValueError(f"Muon takes 2-D parameters only, got shape {tuple(p.shape)}")
                if p.dtype not in (torch.float32, torch.bfloat16):
                    raise TypeError(f"parameter dtype {p.dtype} (use float32 or bfloat16)")

    def add_param_group(self, param_group):
        super().add_param_group(param_group)
        _check_hyper(self.param_groups[-1])

    @torch.no_grad()
    def step(self, closure=None):
        loss = None
        if closure is not None:
            with torch.enable_grad():
                loss = closure()
        for group in self.param_groups:
            # one batched library call per (device, param dtype, grad dtype)
            parts: dict = {}
            for p in group["params"]:
                if p.grad is None:
                    continue
                g = p.grad
                if g.is_sparse:
                    raise RuntimeError("Muon does not support sparse gradients")
                if g.dtype not in (torch.float32, torch.bfloat16):
                    raise TypeError(f"gradient dtype {g.dtype} (use float32 or bfloat16)")
                if not p.is_contiguous():
                    raise ValueError("Muon updates parameters in place and needs them contiguous")
                st = self.state[p]
                buf = st.get("momentum_buffer")
                if buf is None:
                    buf = torch.zeros(p.shape, dtype=torch.float32, device=p.device)
                    st["momentum_buffer"] = buf
                elif buf.dtype != torch.float32 or not buf.is_contiguous():
                    buf = buf.to(torch.float32).contiguous()
                    st["momentum_buffer"] = buf
                key = (p.device, p.dtype, g.dtype)
                ps, gs, ms = parts.setdefault(key, ([], [], []))
                ps.append(p)
                gs.append(g.contiguous())
                ms.append(buf)
            for (dev, _, _), (ps, gs, ms) in parts.items():
                stream = torch.cuda.current_stream(dev) if dev.type == "cuda" else None
                if group["selected_fraction"] is not None:
                    muon_step_selected(ps, [g.float() for g in gs], ms,
                                       fraction=group["selected_fraction"], beta=group["momentum"],
                                       lr=group["lr"], steps=group["ns_steps"],
                                       coeffs=group["ns_coefficients"], eps=group["eps"],
                                       stream=stream)
                    continue
                sx = self._exponents(ps, dev) if self._carry and dev.type == "cuda" else None
                muon_step(ps, gs, ms, beta=group["momentum"], lr=group["lr"],
                          steps=group["ns_steps"], coeffs=group["ns_coefficients"],
                          eps=group["eps"], nesterov=group["nesterov"],
                          weight_decay=group["weight_decay"],
                          stream=stream, scale_exp=sx)
        return loss

    def _exponents(self, ps, dev):
        """The carried exponents of one batched call as one int32 tensor whose
        entries the parameters' states hold as views (so the library's
        rewrite is the state).  Rebuilt from the states when the call's
        parameters change or a state was loaded."""
        key = tuple(id(p) for p in ps)
        buf = self._exp_bufs.get(key)
        if buf is not None:
            ok = True
            for k, p in enumerate(ps):
                e = self.state[p].get("operand_exp")
                if e is None or e.data_ptr() != buf[k].data_ptr():
                    ok = False
                    break
            if ok:
                return buf
        held = [self.state[p].get("operand_exp") for p in ps]
        if all(e is not None for e in held):
            buf = torch.stack([e.to(device=dev, dtype=torch.int32).reshape(()) for e in held])
        else:
            buf = torch.full((len(ps),), SCALE_EXP_UNKNOWN, dtype=torch.int32, device=dev)
            for k, e in enumerate(held):
                if e is not None:
                    buf[k] = e.to(device=dev, dtype=torch.int32).reshape(())
        for k, p in enumerate(ps):
            self.state[p]["operand_exp"] = buf[k]
        self._exp_bufs[key] = buf
        return buf

    def load_state_dict(self, state_dict):
        """torch's loader casts state to the parameter dtype; the momentum is
        fp32 state and the carried operand exponent int32 whatever the
        parameter dtype, so the saved tensors are put back after the base
        class has loaded."""
        saved = {pid: s["momentum_buffer"] for pid, s in state_dict["state"].items()
                 if isinstance(s, dict) and "momentum_buffer" in s}
        exps = {pid: s["operand_exp"] for pid, s in state_dict["state"].items()
                if isinstance(s, dict) and "operand_exp" in s}
        super().load_state_dict(state_dict)
        ids = itertools.chain.from_iterable(g["params"] for g in state_dict["param_groups"])
        params = itertools.chain.from_iterable(g["params"] for g in self.param_groups)
        for pid, p in zip(ids, params):
            if pid in saved:
                self.state[p]["momentum_buffer"] = saved[pid].to(
                    device=p.device, dtype=torch.float32).contiguous()
            if pid in exps:
                self.state[p]["operand_exp"] = torch.as_tensor(exps[pid]).to(
                    device=p.device, dtype=torch.int32).reshape(())


def _check_hyper(h):
    def finite(x):
        return isinstance(x, (int, float)) and math.isfinite(float(x))
    if not finite(h["lr"]) or h["lr"] < 0:
        raise ValueError(f"invalid lr {h['lr']}")
    if not finite(h["momentum"]):
        raise ValueError(f"invalid momentum {h['momentum']}")
    if not finite(h["weight_decay"]) or h["weight_decay"] < 0:
        raise ValueError(f"invalid weight_decay {h['weight_decay']}")
    if not finite(h["eps"]) or h["eps"] < 0:
        raise ValueError(f"invalid eps {h['eps']}")
    if not isinstance(h["ns_steps"], int) or not 0 <= h["ns_steps"] <= 64:
        raise ValueError(f"invalid ns_steps {h['ns_steps']}")
    c = tuple(h["ns_coefficients"])
    if len(c) != 3 or not all(finite(v) for v in c):
        raise ValueError(f"invalid ns_coefficients {c}")
    if not isinstance(h["nesterov"], bool):
        raise ValueError(f"nesterov must be a bool, got {h['nesterov']!r}")
    f = h.get("selected_fraction")
    if f is not None:
        if not finite(f) or not 0.0 < float(f) <= 1.0:
            raise ValueError(f"invalid selected_fraction {f} (use a value in (0, 1])")
        if h["nesterov"] or h["weight_decay"] != 0:
            raise ValueError("selected_fraction does not combine with nesterov or weight_decay")
