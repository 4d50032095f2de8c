"""Named workloads and the seeded synthetic input generator.

This module holds no SSD arithmetic: it only draws random inputs.  Both the HIP path's
callers and the oracle's callers take their inputs from here, so both see exactly the
same values (the oracle gets them upcast to fp64, which is exact for fp32 and bf16).

Distributions (per workload unless a stress case overrides them), all drawn in fp32 on
the CPU from one torch.Generator seeded with `seed`, in the fixed order
x, dt, A, B, C, D, init_state, then cast:
  x    ~ N(0, 1)
  dt   = softplus(N(0, 1) - 2)                      (positive step sizes)
  A_h  = -exp(U(lo, hi))   with (lo, hi) = (ln 1, ln 16) by default
  B, C ~ N(0, 1/N)   (variance 1/N, std N**-0.5)
  D    ~ N(0, 1)
  init ~ N(0, 0.1)   (variance 0.1), only where the workload asks for an init state
x, B and C take the workload dtype (fp32 or bf16, round to nearest even); dt, A, D and
the states stay fp32.

The model-shaped workloads follow the layer shapes of the Mamba-2 130M and 2.7B models
(heads of dimension P=64, state N=128, chunk 256); no dataset is involved.
"""
import math
from dataclasses import dataclass, field, replace

import torch


@dataclass(frozen=True)
class Workload:
    name: str
    batch: int
    seqlen: int
    nheads: int
    headdim: int
    dstate: int
    ngroups: int
    chunk_len: int
    dtype: str = "bf16"              # "fp32" or "bf16": dtype of x, B, C and y
    init_state: bool = False
    seed: int = 0
    log_neg_a_range: tuple = (0.0, math.log(16.0))   # A_h = -exp(U(lo, hi))
    a_zero: bool = False             # stress: A = 0 exactly (no decay)
    dt_zero: bool = False            # stress: dt = 0 exactly
    note: str = field(default="", compare=False)

    @property
    def nchunks(self):
        return (self.seqlen + self.chunk_len - 1) // self.chunk_len

    @property
    def tokens(self):
        return self.batch * self.seqlen

    def dims(self):
        return dict(batch=self.batch, seqlen=self.seqlen, nheads=self.nheads,
                    headdim=self.headdim, dstate=self.dstate, ngroups=self.ngroups)

    def describe(self):
        return (f"{self.name}: B={self.batch} T={self.seqlen} H={self.nheads} P={self.headdim} "
                f"N={self.dstate} G={self.ngroups} Q={self.chunk_len} {self.dtype}"
                f"{' +init' if self.init_state else ''}")


LN = math.log

# The five workloads the performance and parity claims are made on.
TINY_FP32 = Workload("tiny_fp32", 1, 256, 2, 16, 16, 1, 64, dtype="fp32")
MAMBA2_130M = Workload("mamba2_130m", 8, 2048, 24, 64, 128, 1, 256)
MAMBA2_2P7B = Workload("mamba2_2p7b", 4, 4096, 80, 64, 128, 1, 256)
NSWEEP = tuple(Workload(f"nsweep_n{n}", 2, 8192, 32, 64, n, 1, 256) for n in (64, 128, 256))
LONG_CTX = Workload("long_ctx_65k", 1, 65536, 80, 64, 128, 8, 256, init_state=True)

WORKLOADS = {w.name: w for w in (TINY_FP32, MAMBA2_130M, MAMBA2_2P7B, *NSWEEP, LONG_CTX)}

# Decode workloads: one token per sequence per step, continuing a state (seqlen 1, with
# init_state the state the step starts from).  Shapes of the model layers above.
DECODE = {w.name: w for w in (
    Workload("decode_2p7b", 64, 1, 80, 64, 128, 1, 256, init_state=True),
    Workload("decode_130m", 256, 1, 24, 64, 128, 1, 256, init_state=True),
)}

# Stress cases: the model-shaped distributions decay by about e^-254 per 256-step chunk,
# which hides mistakes in the carried state; these make the carry visible.
STRESS = {
    "slow_decay": Workload("slow_decay", 2, 1024, 4, 64, 128, 1, 256, init_state=True,
                           log_neg_a_range=(LN(0.005), LN(0.05))),
    "slow_decay_fp32": Workload("slow_decay_fp32", 1, 512, 2, 32, 32, 1, 64, dtype="fp32",
                                init_state=True, log_neg_a_range=(LN(0.005), LN(0.05))),
    "a_zero": Workload("a_zero", 1, 512, 4, 64, 64, 1, 128, init_state=True, a_zero=True),
    "dt_zero": Workload("dt_zero", 1, 300, 4, 64, 64, 2, 64, init_state=True, dt_zero=True),
    "ragged_1000": Workload("ragged_1000", 1, 1000, 4, 64, 128, 1, 256, init_state=True,
                            log_neg_a_range=(LN(0.005), LN(0.05))),
    "ragged_250_q64": Workload("ragged_250_q64", 2, 250, 3, 32, 64, 3, 64, init_state=True,
                               log_neg_a_range=(LN(0.01), LN(0.1))),
    "groups_eq_heads": Workload("groups_eq_heads", 1, 512, 4, 64, 128, 4, 128, init_state=True,
                                log_neg_a_range=(LN(0.005), LN(0.05))),
    "groups_half": Workload("groups_half", 2, 512, 8, 64, 64, 4, 256, init_state=True,
                            log_neg_a_range=(LN(0.005), LN(0.05))),
    "short_t1": Workload("short_t1", 2, 1, 2, 64, 128, 1, 256, init_state=True),
    "short_t17": Workload("short_t17", 1, 17, 2, 32, 32, 1, 64, init_state=True,
                          log_neg_a_range=(LN(0.01), LN(0.1))),
}


def variants(base, **kw):
    return replace(base, **kw)


def _torch_dtype(name):
    return {"fp32": torch.float32, "bf16": torch.bfloat16}[name]


def generate(w, device="cpu"):
    """Draw the inputs of workload `w`.

    Returns a dict of tensors on `device`: x [B,T,H,P], dt [B,T,H], A [H], B and C
    [B,T,G,N], D [H] and init_state [B,H,N,P] or None.
    """
    g = torch.Generator(device="cpu")
    g.manual_seed(int(w.seed))
    Bz, T, H, P, N, G = w.batch, w.seqlen, w.nheads, w.headdim, w.dstate, w.ngroups
    x = torch.randn((Bz, T, H, P), generator=g, dtype=torch.float32)
    dt = torch.nn.functional.softplus(torch.randn((Bz, T, H), generator=g, dtype=torch.float32) - 2.0)
    lo, hi = w.log_neg_a_range
    A = -torch.exp(torch.rand((H,), generator=g, dtype=torch.float32) * (hi - lo) + lo)
    scale = 1.0 / math.sqrt(N)
    Bm = torch.randn((Bz, T, G, N), generator=g, dtype=torch.float32) * scale
    Cm = torch.randn((Bz, T, G, N), generator=g, dtype=torch.float32) * scale
    D = torch.randn((H,), generator=g, dtype=torch.float32)
    init = None
    if w.init_state:
        init = torch.randn((Bz, H, N, P), generator=g, dtype=torch.float32) * math.sqrt(0.1)
    if w.a_zero:
        A = torch.zeros_like(A)
    if w.dt_zero:
        dt = torch.zeros_like(dt)
    dty = _torch_dtype(w.dtype)
    out = dict(x=x.to(dty), dt=dt, A=A, B=Bm.to(dty), C=Cm.to(dty), D=D, init_state=init)
    if device != "cpu":
        out = {k: (None if v is None else v.to(device)) for k, v in out.items()}
    return out


def generate_grads(w, device="cpu", with_final=True):
    """Upstream gradients for the backward of workload `w`, from their own generator
    (seeded with seed + 1, drawn in fp32 in the order dy, d_final):
      dy      ~ N(0, 1), [B,T,H,P], cast to the workload dtype
      d_final ~ N(0, 1), [B,H,N,P] fp32, or None when with_final is False."""
    g = torch.Generator(device="cpu")
    g.manual_seed(int(w.seed) + 1)
    Bz, T, H, P, N = w.batch, w.seqlen, w.nheads, w.headdim, w.dstate
    dy = torch.randn((Bz, T, H, P), generator=g, dtype=torch.float32).to(_torch_dtype(w.dtype))
    d_final = None
    if with_final:
        d_final = torch.randn((Bz, H, N, P), generator=g, dtype=torch.float32)
    out = dict(dy=dy, d_final=d_final)
    if device != "cpu":
        out = {k: (None if v is None else v.to(device)) for k, v in out.items()}
    return out


def head_slice(inputs, w, b, h):
    """The inputs of the single sequence (batch b, head h) as a B=1, H=1, G=1 problem.
    Every (batch, head) pair is independent, so the full outputs for that pair can be
    checked on their own."""
    g = h // (w.nheads // w.ngroups)
    x = inputs["x"][b:b + 1, :, h:h + 1, :]
    out = dict(x=x, dt=inputs["dt"][b:b + 1, :, h:h + 1], A=inputs["A"][h:h + 1],
               B=inputs["B"][b:b + 1, :, g:g + 1, :], C=inputs["C"][b:b + 1, :, g:g + 1, :],
               D=inputs["D"][h:h + 1], init_state=None)
    if inputs["init_state"] is not None:
        out["init_state"] = inputs["init_state"][b:b + 1, h:h + 1]
    return out


# ---------------------------------------------------------------- the block around the layer
@dataclass(frozen=True)
class BlockCfg:
    """The block's own sizes: conv width, normalisation groups (contiguous channel groups
    of the H*P gated channels, per token), RMS instead of mean/variance, epsilon."""
    conv_k: int = 4
    norm_groups: int = 1
    rms: bool = False
    eps: float = 1e-5


# Model-shaped blocks: the layer shapes above with a width-4 convolution and one
# normalisation group over the H*P channels of a token; and the 2.7B shape with one group
# per head (the group inside a head: the gate and the norm run in the chunk scan's store).
BLOCKS = {
    "block_2p7b": (MAMBA2_2P7B, BlockCfg()),
    "block_130m": (MAMBA2_130M, BlockCfg()),
    "block_2p7b_headnorm": (MAMBA2_2P7B, BlockCfg(norm_groups=80)),
}


def proj_width(w):
    """Channels per token of the projection output [z | x | B | C | dt_raw]."""
    d = w.nheads * w.headdim
    return 2 * d + 2 * w.ngroups * w.dstate + w.nheads


def generate_block(w, cfg, device="cpu"):
    """Inputs of the block between the projections, from their own generator (seeded with
    seed + 2, drawn in fp32 in this order):
      zxbcdt  ~ N(0, 1), [B, T, proj_width], cast to the workload dtype
      conv_w  ~ U(-1/sqrt(K), 1/sqrt(K)), [H*P + 2*G*N, K] fp32
      conv_b  ~ U(-1/sqrt(K), 1/sqrt(K)), [H*P + 2*G*N] fp32
      dt_bias ~ U(-3, -1), [H] fp32
      A_h     = -exp(U(lo, hi)) as for the layer;  D ~ N(0, 1);  init ~ N(0, 0.1) if asked
      norm_w  ~ 1 + N(0, 0.01), [H*P] fp32 (variance 0.01)
      norm_b  ~ N(0, 0.01), [H*P] fp32."""
    g = torch.Generator(device="cpu")
    g.manual_seed(int(w.seed) + 2)
    Bz, T, H, P, N, G = w.batch, w.seqlen, w.nheads, w.headdim, w.dstate, w.ngroups
    d = H * P
    cdim = d + 2 * G * N
    K = cfg.conv_k
    bound = 1.0 / math.sqrt(K)
    zxbcdt = torch.randn((Bz, T, proj_width(w)), generator=g, dtype=torch.float32)
    conv_w = (torch.rand((cdim, K), generator=g, dtype=torch.float32) * 2 - 1) * bound
    conv_b = (torch.rand((cdim,), generator=g, dtype=torch.float32) * 2 - 1) * bound
    dt_bias = torch.rand((H,), generator=g, dtype=torch.float32) * 2 - 3
    lo, hi = w.log_neg_a_range
    A = -torch.exp(torch.rand((H,), generator=g, dtype=torch.float32) * (hi - lo) + lo)
    D = torch.randn((H,), generator=g, dtype=torch.float32)
    init = None
    if w.init_state:
        init = torch.randn((Bz, H, N, P), generator=g, dtype=torch.float32) * math.sqrt(0.1)
    norm_w = 1 + torch.randn((d,), generator=g, dtype=torch.float32) * 0.1
    norm_b = torch.randn((d,), generator=g, dtype=torch.float32) * 0.1
    if w.a_zero:
        A = torch.zeros_like(A)
    out = dict(zxbcdt=zxbcdt.to(_torch_dtype(w.dtype)), conv_w=conv_w, conv_b=conv_b,
               dt_bias=dt_bias, A=A, D=D, init_state=init, norm_w=norm_w, norm_b=norm_b)
    if device != "cpu":
        out = {k: (None if v is None else v.to(device)) for k, v in out.items()}
    return out
