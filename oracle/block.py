"""fp64 CPU oracle for the Mamba-2 block around the SSD layer: the prologue (causal
depthwise conv1d + SiLU on x, B, C; positive step sizes) and the epilogue (output gate and
group normalisation).  Plain numpy, every step written out.

TEST INFRASTRUCTURE ONLY: the test suite, the smoke check and the benchmark's CPU-baseline
leg are the only code allowed to import this module.  It shares no code with the HIP
library and never imports it.

Sources
  "Mamba-2: Attention's Distant Cousin" (docsaid.org), section "The Mamba-2 Block" and its
  Figure 6: one projection at the start of the block yields x, B, C and the step size
  together (and the gate branch z); after the SSM the output is multiplied by the gate and
  passed through an extra normalisation layer before the output projection.
  Structured summary of arXiv 2405.21060 (paper-graph-ui):
    section "The Mamba-2 Architecture": the gate y * phi(z) with phi = Swish by default, and
      GroupNorm as the default extra normalisation, after the gate;
    its "Kernel feature maps (Section 7.3)" paragraph: a pointwise map psi on B and C, Swish
      (SiLU) by default;
    section 6.4: the block's convolution is depthwise and one-dimensional, of width 3-4.

Readings (where the pages leave a step open):
  - the convolution is causal along time (the layer is causal), zero-padded before the
    first step, one filter of width K per channel plus a bias; w[c][K-1] weights the
    current step and w[c][K-1-s] the step s back;
  - it runs on the concatenated x, B, C channels of the projection and is followed by SiLU
    on all of them (the activation after the convolution in Figure 6, and psi on B and C);
  - the step size is dt = softplus(dt_raw + dt_bias[h]) (a positive map of the projected
    value, so that exp(dt A) with A < 0 is a decay); softplus is this oracle's choice of
    that map;
  - the normalisation is per token (so it stays causal): the channels of the gated output
    are split into `groups` contiguous groups, each normalised to zero mean and unit
    variance with eps added to the variance, then scaled and shifted per channel
    (GroupNorm); rms=True is the variant without the mean (scale only, no shift);
  - the projection output is laid out per token as [z | x | B | C | dt_raw], widths
    H*P, H*P, G*N, G*N, H.

Functions
  softplus, silu           the two pointwise maps
  causal_conv1d            the depthwise causal convolution
  block_prologue           conv + SiLU on x, B, C (split) and the step sizes
  gate_norm                y * silu(z) then the per-token group normalisation
  split_projection         the [z | x B C | dt_raw] split of the projection output
  block_fwd                prologue -> SSD recurrence (ssd_ref) -> epilogue
"""
import numpy as np


def softplus(v):
    """log(1 + exp(v)), computed as max(v, 0) + log(1 + exp(-|v|)) (no overflow)."""
    v = np.asarray(v, dtype=np.float64)
    return np.maximum(v, 0.0) + np.log1p(np.exp(-np.abs(v)))


def silu(v):
    """Swish / SiLU: v * sigmoid(v), with sigmoid(v) = 1 / (1 + exp(-v))."""
    v = np.asarray(v, dtype=np.float64)
    with np.errstate(over="ignore"):
        return v / (1.0 + np.exp(-v))


def causal_conv1d(u, w, b=None):
    """Depthwise causal convolution along time.

    u [B, T, Cc], w [Cc, K], b [Cc] or None.
    out[:, t, c] = b[c] + sum_{k=0}^{K-1} w[c, k] * u[:, t - (K - 1) + k, c], with u = 0
    before t = 0."""
    u = np.asarray(u, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64)
    Bz, T, Cc = u.shape
    K = w.shape[1]
    out = np.zeros((Bz, T, Cc))
    if b is not None:
        out += np.asarray(b, dtype=np.float64)
    for k in range(K):
        back = K - 1 - k  # the tap k reads the step `back` positions earlier
        if back < T:
            out[:, back:, :] += w[:, k] * u[:, :T - back, :]
    return out


def block_prologue(xbc, conv_w, conv_b, dt_raw, dt_bias, nheads, headdim, dstate, ngroups):
    """x, B, C and dt for the SSD layer from the projection's x|B|C channels and dt_raw.

    xbc [B, T, H*P + 2*G*N], conv_w [H*P + 2*G*N, K], conv_b [...] or None,
    dt_raw [B, T, H], dt_bias [H] or None.
    Returns dict x [B,T,H,P], B [B,T,G,N], C [B,T,G,N], dt [B,T,H]."""
    Bz, T, _ = np.shape(xbc)
    d = nheads * headdim
    gn = ngroups * dstate
    v = silu(causal_conv1d(xbc, conv_w, conv_b))
    dtr = np.asarray(dt_raw, dtype=np.float64)
    if dt_bias is not None:
        dtr = dtr + np.asarray(dt_bias, dtype=np.float64)
    return dict(x=v[:, :, :d].reshape(Bz, T, nheads, headdim),
                B=v[:, :, d:d + gn].reshape(Bz, T, ngroups, dstate),
                C=v[:, :, d + gn:d + 2 * gn].reshape(Bz, T, ngroups, dstate),
                dt=softplus(dtr))


def gate_norm(y, z, weight, bias, groups, rms=False, eps=1e-5):
    """out = norm(y * silu(z)) per token, over `groups` contiguous channel groups.

    y, z [B, T, Dc] (or [B, T, H, P], flattened over the last two), weight [Dc],
    bias [Dc] or None (ignored when rms)."""
    y = np.asarray(y, dtype=np.float64)
    z = np.asarray(z, dtype=np.float64)
    Bz, T = y.shape[:2]
    v = (y.reshape(Bz, T, -1) * silu(z.reshape(Bz, T, -1)))
    Dc = v.shape[2]
    gs = Dc // groups
    vg = v.reshape(Bz, T, groups, gs)
    if rms:
        ms = np.mean(vg * vg, axis=3, keepdims=True)
        n = vg / np.sqrt(ms + eps)
    else:
        mu = np.mean(vg, axis=3, keepdims=True)
        var = np.mean((vg - mu) ** 2, axis=3, keepdims=True)
        n = (vg - mu) / np.sqrt(var + eps)
    out = n.reshape(Bz, T, Dc) * np.asarray(weight, dtype=np.float64)
    if bias is not None and not rms:
        out = out + np.asarray(bias, dtype=np.float64)
    return out


def split_projection(zxbcdt, nheads, headdim, dstate, ngroups):
    """z [B,T,H*P], xbc [B,T,H*P+2GN], dt_raw [B,T,H] from the rows [z | x B C | dt_raw]."""
    d = nheads * headdim
    gn = ngroups * dstate
    zx = np.asarray(zxbcdt, dtype=np.float64)
    return zx[:, :, :d], zx[:, :, d:2 * d + 2 * gn], zx[:, :, 2 * d + 2 * gn:2 * d + 2 * gn + nheads]


def block_fwd(zxbcdt, conv_w, conv_b, dt_bias, A, D, norm_w, norm_b, nheads, headdim,
              dstate, ngroups, norm_groups, rms=False, eps=1e-5, init_state=None, nthreads=0):
    """The block between the projections: prologue, the SSD layer (the oracle's token
    recurrence, ssd_ref), epilogue.  Returns (out [B,T,H*P], final_state [B,H,N,P])."""
    from . import ssd_ref
    z, xbc, dt_raw = split_projection(zxbcdt, nheads, headdim, dstate, ngroups)
    p = block_prologue(xbc, conv_w, conv_b, dt_raw, dt_bias, nheads, headdim, dstate, ngroups)
    y, final, _ = ssd_ref(p["x"], p["dt"], A, p["B"], p["C"], D, init_state=init_state,
                          nthreads=nthreads)
    return gate_norm(y, z, norm_w, norm_b, norm_groups, rms=rms, eps=eps), final
