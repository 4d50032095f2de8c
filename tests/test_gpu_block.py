"""Parity of the block prologue, epilogue and whole block (through the C ABI) with the
fp64 block oracle (oracle/block.py), on the GPU.

Outputs are compared whole-tensor by rel-L2 at the layer's bounds: 1e-4 for fp32, 2e-2 for
bf16 (fp32 arithmetic, outputs rounded once).  The cases cover:
- conv widths 1..8;
- ragged step counts across the 64-step tiles, and T = 1;
- rows inside the wider projection output (strided) and contiguous rows;
- head counts whose rows are not a multiple of 16 bytes (the element-wise path);
- every register-residency variant of the normalisation, and the streaming one;
- GroupNorm and RMS;
- the whole block at small sizes and at the full model-shaped sizes.
"""
import numpy as np
import pytest
import torch

from mamba_ssd_chunked_03_amd import binding
from mamba_ssd_chunked_03_amd.workloads import (BLOCKS, STRESS, TINY_FP32, BlockCfg, Workload,
                                                generate_block, variants)
from oracle import block as ob
from parity import TOL, np64, per_seq_rel_l2, rel_l2, say, seq_errors

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    assert torch.cuda.is_available(), "GPU tests need a visible GPU"
    binding.library()
    torch.cuda.init()
    return torch.device("cuda:0")


def _split(w, zx):
    d = w.nheads * w.headdim
    gn = w.ngroups * w.dstate
    return zx[:, :, :d], zx[:, :, d:2 * d + 2 * gn], zx[:, :, 2 * d + 2 * gn:]


def _check(name, got, ref, dtype):
    e = rel_l2(np64(got), ref)
    say(f"    {name}: rel_l2 {e:.2e}")
    assert e <= TOL[dtype], f"{name}: rel_l2 {e:.3e} > {TOL[dtype]}"


def _check_per_head(w, out, ref_out, fin, ref_fin):
    """Next to the whole tensors: every (b, h) slice on its own, the output's channels of
    head h over all steps and head h's final state."""
    tol = TOL[w.dtype]
    shape = (w.batch, w.seqlen, w.nheads, w.headdim)
    so = per_seq_rel_l2(*seq_errors(np64(out).reshape(shape), np.asarray(ref_out).reshape(shape),
                                    (1, 3)))
    sf = per_seq_rel_l2(*seq_errors(np64(fin), ref_fin, (2, 3)))
    io = np.unravel_index(np.argmax(so), so.shape)
    jf = np.unravel_index(np.argmax(sf), sf.shape)
    say(f"    worst (b,h): out {so[io]:.2e} at {io}, final_state {sf[jf]:.2e} at {jf}")
    assert so[io] <= tol and sf[jf] <= tol


PRO_CASES = [
    (variants(TINY_FP32, name="pro_fp32_k4", seqlen=130), 4, True),
    (variants(TINY_FP32, name="pro_fp32_k1", seqlen=17), 1, False),
    (Workload("pro_bf16_k3", 2, 200, 4, 64, 64, 2, 64), 3, True),
    (Workload("pro_bf16_k8_h3", 1, 70, 3, 32, 32, 1, 64), 8, True),    # rows not 16-byte
    (Workload("pro_bf16_t1", 3, 1, 8, 64, 128, 1, 64), 4, True),
    (Workload("pro_bf16_k2", 1, 129, 8, 16, 16, 4, 64), 2, False),
]


@pytest.mark.parametrize("w,k,strided", PRO_CASES, ids=[c[0].name for c in PRO_CASES])
def test_prologue_matches_oracle(w, k, strided):
    say(f"[prologue] {w.describe()} K={k} strided={strided}")
    cpu = generate_block(w, BlockCfg(conv_k=k))
    z, xbc, dtr = _split(w, cpu["zxbcdt"])
    dev = "cuda"
    if strided:  # column ranges of the projection output, as the block passes them
        zxd = cpu["zxbcdt"].to(dev)
        _, xbc_d, dtr_d = _split(w, zxd)
    else:
        xbc_d, dtr_d = xbc.contiguous().to(dev), dtr.contiguous().to(dev)
    g = binding.ssd_block_prologue(xbc_d, cpu["conv_w"].to(dev), cpu["conv_b"].to(dev), dtr_d,
                                   cpu["dt_bias"].to(dev), w.nheads, w.headdim, w.dstate,
                                   w.ngroups)
    torch.cuda.synchronize()
    ref = ob.block_prologue(np64(xbc), np64(cpu["conv_w"]), np64(cpu["conv_b"]), np64(dtr),
                            np64(cpu["dt_bias"]), w.nheads, w.headdim, w.dstate, w.ngroups)
    for n in ("x", "B", "C", "dt"):
        _check(n, g[n], ref[n], w.dtype)


def test_prologue_without_biases():
    w = Workload("pro_nobias", 2, 100, 4, 32, 16, 2, 64)
    cpu = generate_block(w, BlockCfg(conv_k=4))
    _, xbc, dtr = _split(w, cpu["zxbcdt"])
    dev = "cuda"
    g = binding.ssd_block_prologue(xbc.contiguous().to(dev), cpu["conv_w"].to(dev), None,
                                   dtr.contiguous().to(dev), None, w.nheads, w.headdim,
                                   w.dstate, w.ngroups)
    torch.cuda.synchronize()
    ref = ob.block_prologue(np64(xbc), np64(cpu["conv_w"]), None, np64(dtr), None, w.nheads,
                            w.headdim, w.dstate, w.ngroups)
    for n in ("x", "B", "C", "dt"):
        _check(n, g[n], ref[n], w.dtype)


# (name, dtype, B, T, H, P, groups, rms, z row padding): group sizes reach every residency
# variant (nv = 1, 2, 4, 8, 16 and streaming) and the element-wise path
EPI_CASES = [
    ("epi_bf16_g1", "bf16", 2, 37, 8, 64, 1, False, 0),       # gs 512: lpg 64, nv 1
    ("epi_bf16_g1_rms", "bf16", 2, 37, 8, 64, 1, True, 0),
    ("epi_bf16_h80", "bf16", 1, 9, 80, 64, 1, False, 0),      # gs 5120: nv 10 (16)
    ("epi_bf16_stream", "bf16", 1, 5, 136, 64, 1, False, 0),  # gs 8704: nv 17, streaming
    ("epi_bf16_g8", "bf16", 2, 33, 8, 64, 8, False, 0),       # gs 64: lpg 8
    ("epi_bf16_g4_rms", "bf16", 1, 20, 12, 32, 4, True, 0),   # gs 96: lpg 4, nv 3 (4)
    ("epi_bf16_hp_g2", "bf16", 1, 11, 16, 64, 2, False, 0),   # gs 512
    ("epi_bf16_pad", "bf16", 2, 21, 4, 32, 2, False, 3),      # z rows not 16-byte
    ("epi_fp32_g1", "fp32", 2, 19, 4, 64, 1, False, 0),       # gs 256: V 4, nv 1
    ("epi_fp32_g2_rms", "fp32", 1, 40, 8, 64, 2, True, 0),
    ("epi_fp32_pad", "fp32", 1, 13, 2, 16, 1, False, 1),      # element-wise path
    ("epi_fp32_big", "fp32", 1, 4, 80, 64, 1, False, 0),      # gs 5120, V 4: nv 20, streaming
]


@pytest.mark.parametrize("case", EPI_CASES, ids=[c[0] for c in EPI_CASES])
def test_epilogue_matches_oracle(case):
    name, dtype, bz, T, H, P, groups, rms, pad = case
    say(f"[epilogue] {case}")
    d = H * P
    g = torch.Generator().manual_seed(7)
    td = torch.float32 if dtype == "fp32" else torch.bfloat16
    y = torch.randn((bz, T, H, P), generator=g).to(td)
    zw = torch.randn((bz, T, d + pad), generator=g).to(td)
    z = zw[:, :, :d]
    nw = 1 + 0.1 * torch.randn(d, generator=g)
    nb = 0.1 * torch.randn(d, generator=g)
    dev = "cuda"
    out = binding.ssd_block_epilogue(y.to(dev), zw.to(dev)[:, :, :d], nw.to(dev), nb.to(dev),
                                     groups, rms=rms, eps=1e-5)
    torch.cuda.synchronize()
    ref = ob.gate_norm(np64(y), np64(z), np64(nw), np64(nb), groups, rms=rms, eps=1e-5)
    _check("out", out, ref, dtype)


BLOCK_CASES = [
    (variants(TINY_FP32, name="blk_fp32", seqlen=200), BlockCfg(conv_k=4, norm_groups=2)),
    (variants(STRESS["slow_decay"], name="blk_bf16_slow"), BlockCfg(conv_k=4, norm_groups=1)),
    (Workload("blk_bf16_g2_rms", 2, 300, 8, 64, 64, 2, 128, init_state=True),
     BlockCfg(conv_k=3, norm_groups=4, rms=True)),
    (Workload("blk_bf16_h2", 1, 77, 2, 64, 128, 1, 64), BlockCfg(conv_k=4)),  # rows not 16B
]


def _run_block(w, cfg, cpu):
    dev = "cuda"
    d = {k: (None if v is None else v.to(dev)) for k, v in cpu.items()}
    out, fin = binding.ssd_block_fwd(d["zxbcdt"], d["conv_w"], d["conv_b"], d["dt_bias"],
                                     d["A"], d["D"], w.chunk_len, d["norm_w"], d["norm_b"],
                                     cfg.norm_groups, w.headdim, w.dstate, w.ngroups,
                                     rms=cfg.rms, eps=cfg.eps, init_state=d["init_state"])
    torch.cuda.synchronize()
    return out, fin


def _oracle_block(w, cfg, cpu):
    return ob.block_fwd(np64(cpu["zxbcdt"]), np64(cpu["conv_w"]), np64(cpu["conv_b"]),
                        np64(cpu["dt_bias"]), np64(cpu["A"]), np64(cpu["D"]),
                        np64(cpu["norm_w"]), np64(cpu["norm_b"]), w.nheads, w.headdim,
                        w.dstate, w.ngroups, cfg.norm_groups, rms=cfg.rms, eps=cfg.eps,
                        init_state=np64(cpu["init_state"]))


@pytest.mark.parametrize("w,cfg", BLOCK_CASES, ids=[c[0].name for c in BLOCK_CASES])
def test_block_matches_oracle(w, cfg):
    say(f"[block] {w.describe()} {cfg}")
    cpu = generate_block(w, cfg)
    out, fin = _run_block(w, cfg, cpu)
    ref_out, ref_fin = _oracle_block(w, cfg, cpu)
    _check("out", out, ref_out, w.dtype)
    _check("final_state", fin, ref_fin, w.dtype)
    _check_per_head(w, out, ref_out, fin, ref_fin)


@pytest.mark.parametrize("name", list(BLOCKS))
def test_block_full_size(name):
    """The model-shaped blocks at full size, in the launch configuration that
    bench.py --block times, compared whole-tensor and per (b, h)."""
    w, cfg = BLOCKS[name]
    say(f"[block full] {w.describe()} {cfg}")
    cpu = generate_block(w, cfg)
    out, fin = _run_block(w, cfg, cpu)
    ref_out, ref_fin = _oracle_block(w, cfg, cpu)
    _check("out", out, ref_out, w.dtype)
    _check("final_state", fin, ref_fin, w.dtype)
    _check_per_head(w, out, ref_out, fin, ref_fin)


@pytest.mark.parametrize("w,cfg", [BLOCK_CASES[1], BLOCK_CASES[2], BLOCK_CASES[0]],
                         ids=["bf16_slow", "bf16_g2_rms", "fp32"])
def test_block_fwd_equals_its_three_calls(w, cfg):
    """ssd_block_fwd makes the step sizes inside the forward's cumsum pass (softplus fused,
    dt never stored); it must give exactly what the prologue, ssd_fwd and the epilogue give
    as three calls."""
    say(f"[block = 3 calls] {w.describe()} {cfg}")
    cpu = generate_block(w, cfg)
    out, fin = _run_block(w, cfg, cpu)
    d = {k: (None if v is None else v.to("cuda")) for k, v in cpu.items()}
    H, P, N, G = w.nheads, w.headdim, w.dstate, w.ngroups
    hp, gn = H * P, G * N
    zx = d["zxbcdt"]
    pro = binding.ssd_block_prologue(zx[:, :, hp:2 * hp + 2 * gn], d["conv_w"], d["conv_b"],
                                     zx[:, :, 2 * hp + 2 * gn:], d["dt_bias"], H, P, N, G)
    y, f2 = binding.ssd_fwd(pro["x"], pro["dt"], d["A"], pro["B"], pro["C"], d["D"],
                            w.chunk_len, init_state=d["init_state"])
    o2 = binding.ssd_block_epilogue(y, zx[:, :, :hp], d["norm_w"], d["norm_b"], cfg.norm_groups,
                                    rms=cfg.rms, eps=cfg.eps, dstate=N, ngroups=G)
    torch.cuda.synchronize()
    assert torch.equal(out, o2) and torch.equal(fin, f2)


# Norm groups inside one head (S = H P / norm_groups a multiple of 16 dividing P): the gate
# and the norm run in the chunk scan's store, which writes the block output (y is never
# stored).  One, two and four groups per head, GroupNorm and RMS, head sizes 64 and 32,
# ragged lengths, init on and off.
LN_ = np.log
FUSED_CASES = [
    (Workload("blk_fused_g1", 2, 300 + 77, 8, 64, 128, 2, 128, init_state=True,
              log_neg_a_range=(LN_(0.005), LN_(0.05))), BlockCfg(conv_k=4, norm_groups=8)),
    (Workload("blk_fused_g2_rms", 1, 500, 4, 64, 64, 1, 256),
     BlockCfg(conv_k=4, norm_groups=8, rms=True)),
    (Workload("blk_fused_g4", 1, 256 + 31, 4, 64, 128, 1, 256, init_state=True),
     BlockCfg(conv_k=3, norm_groups=16)),
    (Workload("blk_fused_p32_g2", 2, 200, 4, 32, 128, 1, 64, init_state=True,
              log_neg_a_range=(LN_(0.01), LN_(0.1))), BlockCfg(conv_k=2, norm_groups=8)),
]


@pytest.mark.parametrize("w,cfg", FUSED_CASES, ids=[c[0].name for c in FUSED_CASES])
def test_block_with_norm_groups_inside_a_head(w, cfg):
    """The fused gate and norm against the oracle's block (the bf16 bar, whole tensor and per
    (b, h)), and against the same block made by the three unfused calls (prologue, ssd_fwd,
    epilogue), which differ only by the rounding of y to bf16 before the norm."""
    say(f"[block fused norm] {w.describe()} {cfg}")
    cpu = generate_block(w, cfg)
    out, fin = _run_block(w, cfg, cpu)
    ref_out, ref_fin = _oracle_block(w, cfg, cpu)
    _check("out", out, ref_out, w.dtype)
    _check("final_state", fin, ref_fin, w.dtype)
    _check_per_head(w, out, ref_out, fin, ref_fin)
    d = {k: (None if v is None else v.to("cuda")) for k, v in cpu.items()}
    H, P, N, G = w.nheads, w.headdim, w.dstate, w.ngroups
    hp, gn = H * P, G * N
    zx = d["zxbcdt"]
    pro = binding.ssd_block_prologue(zx[:, :, hp:2 * hp + 2 * gn], d["conv_w"], d["conv_b"],
                                     zx[:, :, 2 * hp + 2 * gn:], d["dt_bias"], H, P, N, G)
    y, f2 = binding.ssd_fwd(pro["x"], pro["dt"], d["A"], pro["B"], pro["C"], d["D"],
                            w.chunk_len, init_state=d["init_state"])
    o2 = binding.ssd_block_epilogue(y, zx[:, :, :hp], d["norm_w"], d["norm_b"], cfg.norm_groups,
                                    rms=cfg.rms, eps=cfg.eps, dstate=N, ngroups=G)
    torch.cuda.synchronize()
    assert torch.equal(fin, f2)
    e = rel_l2(np64(out), np64(o2))
    say(f"    fused against three calls: rel_l2 {e:.3e}")
    assert e <= 1e-2


def test_block_with_unaligned_norm_params():
    """Norm parameters 4 bytes past a 16-byte boundary (the ABI asks only for 4-byte
    alignment): the fused store and the epilogue's vector path both need 16-byte runs, so
    ssd_block_fwd takes the epilogue pass, and the epilogue its element-wise variant.  The
    block must equal the three calls bit for bit and the three calls with aligned
    parameters within the bf16 bar, on sizes that would otherwise take the fused path."""
    w, cfg = FUSED_CASES[0]
    say(f"[block unaligned norm params] {w.describe()} {cfg}")
    d_ = binding.SsdDims(w.batch, w.seqlen, w.nheads, w.headdim, w.dstate, w.ngroups)
    assert binding.ssd_block_fwd_norm_in_scan(d_, binding.SSD_BF16, w.chunk_len, cfg.norm_groups)
    cpu = generate_block(w, cfg)
    d = {k: (None if v is None else v.to("cuda")) for k, v in cpu.items()}
    H, P, N, G = w.nheads, w.headdim, w.dstate, w.ngroups
    hp, gn = H * P, G * N
    wbuf = torch.zeros(hp + 1, device="cuda")
    bbuf = torch.zeros(hp + 1, device="cuda")
    wbuf[1:].copy_(d["norm_w"])
    bbuf[1:].copy_(d["norm_b"])
    nw, nb = wbuf[1:], bbuf[1:]
    assert nw.data_ptr() % 16 == 4 and nb.data_ptr() % 16 == 4
    out, fin = binding.ssd_block_fwd(d["zxbcdt"], d["conv_w"], d["conv_b"], d["dt_bias"],
                                     d["A"], d["D"], w.chunk_len, nw, nb, cfg.norm_groups,
                                     P, N, G, rms=cfg.rms, eps=cfg.eps,
                                     init_state=d["init_state"])
    zx = d["zxbcdt"]
    pro = binding.ssd_block_prologue(zx[:, :, hp:2 * hp + 2 * gn], d["conv_w"], d["conv_b"],
                                     zx[:, :, 2 * hp + 2 * gn:], d["dt_bias"], H, P, N, G)
    y, f2 = binding.ssd_fwd(pro["x"], pro["dt"], d["A"], pro["B"], pro["C"], d["D"],
                            w.chunk_len, init_state=d["init_state"])
    o2 = binding.ssd_block_epilogue(y, zx[:, :, :hp], nw, nb, cfg.norm_groups, rms=cfg.rms,
                                    eps=cfg.eps, dstate=N, ngroups=G)
    o3 = binding.ssd_block_epilogue(y, zx[:, :, :hp], d["norm_w"], d["norm_b"], cfg.norm_groups,
                                    rms=cfg.rms, eps=cfg.eps, dstate=N, ngroups=G)
    torch.cuda.synchronize()
    assert torch.equal(out, o2) and torch.equal(fin, f2)
    e = rel_l2(np64(o2), np64(o3))
    say(f"    element-wise against vector epilogue: rel_l2 {e:.3e}")
    assert e <= TOL["bf16"]


def test_block_empty_sequence():
    """T = 0: nothing to compute; final_state = init_state."""
    w = Workload("blk_empty", 2, 0, 4, 32, 16, 1, 64, init_state=True)
    cfg = BlockCfg()
    cpu = generate_block(w, cfg)
    out, fin = _run_block(w, cfg, cpu)
    assert out.shape == (2, 0, 128)
    assert torch.equal(fin.cpu(), cpu["init_state"])


def test_block_is_deterministic():
    w, cfg = BLOCK_CASES[2]
    cpu = generate_block(w, cfg)
    a, fa = _run_block(w, cfg, cpu)
    b, fb = _run_block(w, cfg, cpu)
    assert torch.equal(a, b) and torch.equal(fa, fb)
