"""Seeded synthetic workloads for the KDA layer.

This module only draws random numbers; it holds none of the layer's arithmetic.
Both the GPU path and the fp64 CPU oracle take their inputs from here.

Draw order (fixed, one generator per workload -- the CPU's unless the workload
says otherwise -- seed 0 unless given):
lengths, q_raw, k_raw, v_raw, g_raw, beta_logit, z, conv_w, norm_w, state0,
conv_state0.  Values are drawn in float32, then rounded to bfloat16 (round to
nearest even, torch's conversion) where the workload is bf16.  The oracle
widens exactly those rounded values to float64.

Workloads (sizes as in the pages' serving context: 128-wide KDA heads):
  tiny      N=1, H=1, T=256, d=64, fp32, softplus gate, zero carries
  prefill   N=1, T=4096, H=16, d=128, bf16, safe gate lb=-5, zero carries
  varlen    N=8, lengths ~ U{512..8192}, H=32, d=128, bf16, softplus gate,
            state0 ~ N(0, 0.02^2), conv_state0 ~ N(0,1)
  decode    B=256, 64 steps, H=32, d=128, bf16, safe gate lb=-5,
            state0 ~ N(0, 0.02^2), conv_state0 ~ N(0,1)
  verify    B=64, window 4 on top of a carried state, H=32, d=128, bf16,
            safe gate lb=-5, accept length j ~ U{0..3}
  verify_prefilled  the same window on the state a 2048-row prompt per
            sequence leaves (zero initial carries)
Common: q/k/v/gate/beta-logit/z ~ N(0,1); conv_w ~ U(-1/2, 1/2) (bound
1/sqrt(W) for W=4 taps); norm_w ~ U(0.5, 1.5).
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np
import torch

GATE_SOFTPLUS = 0
GATE_SAFE = 1
CONV_W = 4


@dataclass
class Workload:
    name: str
    H: int
    dk: int
    dv: int
    cu_seqlens: torch.Tensor  # int32 [N+1]
    q: torch.Tensor  # [T,H,dk] raw projected rows
    k: torch.Tensor  # [T,H,dk]
    v: torch.Tensor  # [T,H,dv]
    g: torch.Tensor  # [T,H,dk] raw gate
    beta: torch.Tensor  # [T,H] beta logit
    z: torch.Tensor  # [T,H,dv] output-gate rows
    conv_w: torch.Tensor  # [C,4] float32
    norm_w: torch.Tensor  # [dv] float32
    state0: torch.Tensor  # [N,H,dk,dv] float32
    conv_state0: torch.Tensor  # [N,3,C] raw dtype
    gate_mode: int
    lower_bound: float
    meta: dict = field(default_factory=dict)

    @property
    def N(self) -> int:
        return self.cu_seqlens.numel() - 1

    @property
    def T(self) -> int:
        return self.q.shape[0]

    @property
    def C(self) -> int:
        return self.H * (2 * self.dk + self.dv)

    @property
    def dtype(self) -> torch.dtype:
        return self.q.dtype

    def to(self, device) -> "Workload":
        kw = {f: (getattr(self, f).to(device) if isinstance(getattr(self, f), torch.Tensor) else getattr(self, f))
              for f in self.__dataclass_fields__}
        return Workload(**kw)

    def head_channels(self, heads) -> torch.Tensor:
        """Conv-channel indices of a subset of heads, in conv channel order (q, then k, then v)."""
        H, dk, dv = self.H, self.dk, self.dv
        return torch.tensor([h * dk + i for h in heads for i in range(dk)] +
                            [H * dk + h * dk + i for h in heads for i in range(dk)] +
                            [2 * H * dk + h * dv + i for h in heads for i in range(dv)])

    def select_heads(self, heads) -> "Workload":
        """The same workload restricted to a subset of heads (conv channels picked per stream)."""
        heads = list(heads)
        dk, dv = self.dk, self.dv
        ch = self.head_channels(heads)
        hs = torch.tensor(heads)
        pick = (lambda t: t[:, hs].contiguous())
        return Workload(self.name, len(heads), dk, dv, self.cu_seqlens, pick(self.q), pick(self.k), pick(self.v),
                        pick(self.g), pick(self.beta), pick(self.z), self.conv_w[ch].contiguous(), self.norm_w,
                        pick(self.state0), self.conv_state0[:, :, ch].contiguous(), self.gate_mode, self.lower_bound,
                        dict(self.meta))

    def f64(self, name: str) -> np.ndarray:
        """The tensor widened exactly to float64 (what the oracle consumes)."""
        return getattr(self, name).detach().cpu().to(torch.float64).numpy()


def _normal(gen, shape, std=1.0):
    x = torch.randn(shape, generator=gen, dtype=torch.float32, device=gen.device)
    return x if std == 1.0 else x * std


def generate(name: str, *, lengths, H, dk, dv, dtype, gate_mode, lower_bound=-5.0, state_std=0.0,
             conv_state_std=0.0, seed=0, meta=None, device="cpu") -> Workload:
    """device: where the generator draws and the tensors live (cu_seqlens always on the host).  The CPU
    generator is the default; a workload too large to draw on the host in reasonable time draws on the
    GPU's generator instead (other values for the same seed, used by both sides alike)."""
    gen = torch.Generator(device).manual_seed(seed)
    if callable(lengths):
        lengths = lengths(gen)
    lengths = [int(x) for x in lengths]
    N = len(lengths)
    cu = torch.zeros(N + 1, dtype=torch.int32)
    cu[1:] = torch.cumsum(torch.tensor(lengths, dtype=torch.int64), 0).to(torch.int32)
    T = int(cu[-1])
    C = H * (2 * dk + dv)
    q = _normal(gen, (T, H, dk))
    k = _normal(gen, (T, H, dk))
    v = _normal(gen, (T, H, dv))
    g = _normal(gen, (T, H, dk))
    beta = _normal(gen, (T, H))
    z = _normal(gen, (T, H, dv))
    conv_w = torch.rand((C, CONV_W), generator=gen, dtype=torch.float32, device=device) - 0.5
    norm_w = torch.rand((dv,), generator=gen, dtype=torch.float32, device=device) + 0.5
    state0 = (_normal(gen, (N, H, dk, dv), state_std) if state_std > 0
              else torch.zeros((N, H, dk, dv), device=device))
    conv_state0 = (_normal(gen, (N, CONV_W - 1, C), conv_state_std) if conv_state_std > 0
                   else torch.zeros((N, CONV_W - 1, C), device=device))
    cast = (lambda t: t.to(dtype))
    return Workload(name, H, dk, dv, cu, cast(q), cast(k), cast(v), cast(g), cast(beta), cast(z), conv_w, norm_w,
                    state0, cast(conv_state0), gate_mode, float(lower_bound), dict(meta or {}))


def tiny(seed=0, T=256) -> Workload:
    return generate("tiny", lengths=[T], H=1, dk=64, dv=64, dtype=torch.float32, gate_mode=GATE_SOFTPLUS,
                    seed=seed)


def prefill(seed=0, T=4096, H=16, d=128) -> Workload:
    return generate("prefill", lengths=[T], H=H, dk=d, dv=d, dtype=torch.bfloat16, gate_mode=GATE_SAFE,
                    lower_bound=-5.0, seed=seed)


def varlen(seed=0, N=8, lo=512, hi=8192, H=32, d=128) -> Workload:
    lens = (lambda gen: torch.randint(lo, hi + 1, (N,), generator=gen, device=gen.device).tolist())
    return generate("varlen", lengths=lens, H=H, dk=d, dv=d, dtype=torch.bfloat16, gate_mode=GATE_SOFTPLUS,
                    state_std=0.02, conv_state_std=1.0, seed=seed)


def decode(seed=0, B=256, steps=64, H=32, d=128) -> Workload:
    """B sequences of `steps` rows each; step s of a batched decode takes row s of every sequence."""
    return generate("decode", lengths=[steps] * B, H=H, dk=d, dv=d, dtype=torch.bfloat16, gate_mode=GATE_SAFE,
                    lower_bound=-5.0, state_std=0.02, conv_state_std=1.0, seed=seed, meta={"steps": steps})


def verify(seed=0, B=64, window=4, H=32, d=128) -> Workload:
    """B sequences of `window` draft rows each on a carried state; meta['accept'] = j ~ U{0..3}
    (rows 0..j of each window are kept)."""
    w = generate("verify", lengths=[window] * B, H=H, dk=d, dv=d, dtype=torch.bfloat16, gate_mode=GATE_SAFE,
                 lower_bound=-5.0, state_std=0.02, conv_state_std=1.0, seed=seed, meta={"window": window})
    gen = torch.Generator("cpu").manual_seed(seed + 1)
    w.meta["accept"] = torch.randint(0, window, (B,), generator=gen, dtype=torch.int32)
    return w


def verify_prefilled(seed=0, B=64, prompt=2048, window=4, H=32, d=128, device="cuda") -> Workload:
    """B sequences of prompt + window rows each: the first `prompt` rows of a sequence build its state through
    the chunked prompt path, the last `window` rows are its draft window.  Zero initial carries; safe gate
    lb=-5; meta['accept'] = j ~ U{0..window-1} (rows 0..j of each window are kept).  At the full size (2.7 G
    values) it draws on the GPU's generator by default."""
    w = generate("verify_prefilled", lengths=[prompt + window] * B, H=H, dk=d, dv=d, dtype=torch.bfloat16,
                 gate_mode=GATE_SAFE, lower_bound=-5.0, seed=seed, meta={"prompt": prompt, "window": window},
                 device=device)
    gen = torch.Generator("cpu").manual_seed(seed + 1)
    w.meta["accept"] = torch.randint(0, window, (B,), generator=gen, dtype=torch.int32)
    return w


def step_rows(w: Workload, name: str, steps: int) -> torch.Tensor:
    """Rows of equal-length sequences regrouped step-major: [steps, N, ...]."""
    t = getattr(w, name)
    return t.view(w.N, steps, *t.shape[1:]).transpose(0, 1).contiguous()
