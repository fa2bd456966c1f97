"""GPU parity of the MoE-layer forward entry points against the CPU oracle,
through the C ABI: routing and the permuted cast bit-exact, the SwiGLU cast
against the fp64 definition (the kernel's fp32 exp may move a value across a
rounding boundary: every code must be a correct rounding of a value within
1e-6 of the exact one, and almost all codes equal the oracle's), the weighted
combine within its fp32 bound, then the whole layer composed from the library
against the oracle's composition, and the full-size layer's steps."""
import numpy as np
import pytest
import torch

import workloads
from helpers import SENTINEL, assert_codes_equal, assert_f32_bits_equal, check_full, dev_bf16, say

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


@pytest.fixture(scope="module")
def fp8():
    import fp8_scaled_gemm_amax_amd as m
    return m


def gpu_route(fp8, idx, E):
    T, k = idx.shape
    off = torch.full((E + 1,), -7, dtype=torch.int64, device=DEV)
    dest = torch.full((T, k), -7, dtype=torch.int32, device=DEV)
    fp8.fp8_moe_route(torch.from_numpy(np.ascontiguousarray(idx, np.int32)).to(DEV), E, off, dest)
    torch.cuda.synchronize()
    return off.cpu().numpy(), dest.cpu().numpy()


ROUTES = [(2048, 8, 32, 0), (1, 1, 1, 1), (3000, 4, 1024, 2), (5000, 2, 3, 3), (700, 6, 64, 4), (9000, 4, 16, 5)]


@pytest.mark.parametrize("T,k,E,seed", ROUTES)
def test_route_parity(fp8, orc, T, k, E, seed):
    """Zipf top-k routing (distinct experts per token), one expert, 1024
    experts, more entries than one chunk per expert, -1 / E indices that drop
    their entries, and more entries than one register batch (36000)."""
    rng = np.random.default_rng(seed)
    if k <= E:
        idx, _ = workloads.topk_routing(rng, T, E, k)
    else:
        idx = rng.integers(0, E, (T, k)).astype(np.int32)
    if seed == 3:
        idx[::7, 0] = -1
        idx[::11, 1] = E
    say("route", T, k, E)
    off, dest = gpu_route(fp8, idx, E)
    ooff, odest = orc.moe_route(idx, E)
    assert np.array_equal(off, ooff), "offsets"
    assert np.array_equal(dest, odest), "dest"


def test_route_no_tokens(fp8):
    say("route empty")
    off = torch.full((9,), -7, dtype=torch.int64, device=DEV)
    fp8.fp8_moe_route(torch.empty((0, 4), dtype=torch.int32, device=DEV), 8, off,
                      torch.empty((0, 4), dtype=torch.int32, device=DEV))
    torch.cuda.synchronize()
    assert (off.cpu() == 0).all()


@pytest.mark.parametrize("fmt", [0, 1, 2])
@pytest.mark.parametrize("H", [64, 520, 7168])
def test_permute_quantize_parity(fp8, orc, fmt, H):
    """Tokens with a NaN row, a zero row and an Inf; each token to k rows; a
    spare output row nobody writes keeps its sentinel; a dropped slot (-1)."""
    rng = np.random.default_rng(H + fmt)
    T, k, E = 300, 4, 16
    idx, _ = workloads.topk_routing(rng, T, E, k)
    idx[5, 2] = -1
    x = workloads.bf16_bits(rng.standard_normal((T, H)).astype(np.float32) *
                            np.exp2(rng.integers(-8, 9, (T, 1))).astype(np.float32))
    x[3, 7] = 0x7FC0
    x[4] = 0
    x[6, 1] = 0xFF80
    _, dest = orc.moe_route(idx, E)
    rows_out = T * k + 1                                  # one spare row
    say("permute quantize", H, fmt)
    q = torch.full((rows_out, H), SENTINEL, dtype=torch.uint8, device=DEV)
    si = torch.full((rows_out,), -1.0, device=DEV)
    fp8.fp8_moe_permute_quantize_row(dev_bf16(x), torch.from_numpy(dest).to(DEV), fmt, 0, q, si)
    torch.cuda.synchronize()
    oq, osi = orc.moe_permute_quantize_row(x, dest, fmt)      # [T*k] rows
    used = np.zeros(rows_out, bool)
    used[dest[dest >= 0]] = True
    qh, sih = q.cpu().numpy(), si.cpu().numpy()
    u = used[:T * k]
    assert_codes_equal(qh[:T * k][u], oq[u], "codes")
    assert_f32_bits_equal(sih[:T * k][u], osi[u], "scale_inv")
    assert np.all(qh[~used] == SENTINEL) and np.all(sih[~used] == -1.0), "write to an unrouted row"


def check_swiglu(orc, fmt, h, q, si, min_equal=0.999):
    """Every GPU code a correct rounding of a value within 1e-6 (relative) of
    the exact a * s_gpu (NaN where a is NaN); scale_inv within 1e-6 of the
    oracle's; nearly all codes equal to the oracle's."""
    oq, osi, a32 = orc.swiglu_quantize_row(h, fmt)
    hv = workloads.bf16_to_f32(h).astype(np.float64)
    inter = hv.shape[1] // 2
    with np.errstate(invalid="ignore", over="ignore"):
        a = orc.silu(hv[:, :inter]) * hv[:, inter:]
    assert np.allclose(si, osi, rtol=1e-6, atol=0), "scale_inv"
    fmax, _, mbits, bias = orc.fmt_info(fmt)
    table = orc.decode_table(fmt)
    dec = table[q]
    nan = np.isnan(a)
    assert np.all(np.isnan(dec[nan])), "NaN inputs must give NaN codes"
    scaled = np.where(nan, 0.0, a) / si[:, None].astype(np.float64)     # a * s_gpu
    mag = np.minimum(np.abs(scaled), fmax)
    e = np.maximum(np.floor(np.log2(np.maximum(mag, 1e-300))), 1 - bias)
    half = 0.5 * np.exp2(e - mbits)
    err = np.abs(dec - np.clip(scaled, -fmax, fmax))
    ok = nan | (err <= half * (1 + 1e-5) + 1e-6 * np.abs(scaled))
    assert ok.all(), f"{int((~ok).sum())} codes are not a rounding of a * s"
    frac = float((q == oq).mean())
    assert frac >= min_equal, f"only {frac:.5f} of the codes equal the oracle's"


@pytest.mark.parametrize("fmt", [0, 1])
@pytest.mark.parametrize("rows,inter", [(1, 8), (37, 256), (300, 2048), (64, 4096), (5, 520)])
def test_swiglu_quantize_parity(fp8, orc, fmt, rows, inter):
    rng = np.random.default_rng(rows + inter + fmt)
    hf = (rng.standard_normal((rows, 2 * inter)) * np.exp2(rng.integers(-6, 7, (rows, 1)))).astype(np.float32)
    h = workloads.bf16_bits(hf)
    say("swiglu quantize", rows, inter, fmt)
    q = torch.full((rows, inter + 8), SENTINEL, dtype=torch.uint8, device=DEV)[:, :inter]
    si = torch.empty(rows, device=DEV)
    fp8.fp8_swiglu_quantize_row(dev_bf16(h), fmt, 0, q, si)
    torch.cuda.synchronize()
    qb = q.cpu().numpy()
    check_swiglu(orc, fmt, h, qb, si.cpu().numpy())


def test_swiglu_special_rows(fp8, orc):
    """A NaN in gate (its row's scale is 1 and the NaN is kept), a zero row,
    -Inf gate (silu -> NaN), a large gate (silu = gate)."""
    inter = 64
    hf = np.random.default_rng(9).standard_normal((4, 2 * inter)).astype(np.float32)
    hf[1] = 0
    hf[2, 3] = -np.inf
    hf[3, 0] = 80.0
    h = workloads.bf16_bits(hf)
    h[0, 5] = 0x7FC0
    say("swiglu special")
    q = torch.empty((4, inter), dtype=torch.uint8, device=DEV)
    si = torch.empty(4, device=DEV)
    fp8.fp8_swiglu_quantize_row(dev_bf16(h), 0, 0, q, si)
    torch.cuda.synchronize()
    qh, sih = q.cpu().numpy(), si.cpu().numpy()
    assert sih[0] == 1.0 and sih[2] == 1.0 and sih[1] == 1.0      # NaN rows and the zero row: scale 1
    assert not qh[1].any()
    check_swiglu(orc, 0, h, qh, sih, min_equal=0.95)


@pytest.mark.parametrize("T,k,H", [(300, 4, 520), (64, 8, 7168), (1, 1, 8)])
def test_unpermute_combine_parity(fp8, orc, T, k, H):
    rng = np.random.default_rng(T + H)
    E = 16
    idx = rng.integers(0, E, (T, k)).astype(np.int32) if k > E else workloads.topk_routing(rng, T, E, k)[0]
    _, dest = orc.moe_route(idx, E)
    dest = dest.copy()
    if T > 1:
        dest[1, 0] = -1                                   # a dropped slot adds nothing
    w = rng.uniform(0, 1, (T, k)).astype(np.float32)
    y = workloads.bf16_bits(rng.standard_normal((T * k, H)).astype(np.float32))
    say("combine", T, k, H)
    out = torch.full((T, H + 8), float("nan"), dtype=torch.bfloat16, device=DEV)[:, :H]
    fp8.fp8_moe_unpermute_combine(dev_bf16(y), torch.from_numpy(dest).to(DEV), torch.from_numpy(w).to(DEV), out)
    torch.cuda.synchronize()
    got = out.float().cpu().numpy().astype(np.float64)
    o, mag = orc.moe_unpermute_combine(y, dest, w)
    tol = 2.0 ** -8 * np.abs(o) + (k + 1) * 2.0 ** -24 * mag
    bad = np.abs(got - o) > tol
    assert not bad.any(), f"{int(bad.sum())} outputs outside the bound"


def layer_gpu(fp8, d, fmt_act=0, fmt_w=0):
    """The layer forward through the library only; returns (out, intermediates)."""
    x, idx, wts, w1, w2 = d["x"], d["idx"], d["weights"], d["w1"], d["w2"]
    T, H = x.shape
    k = idx.shape[1]
    E, I2, _ = w1.shape
    inter = I2 // 2
    P = T * k
    off = torch.empty(E + 1, dtype=torch.int64, device=DEV)
    dest = torch.empty((T, k), dtype=torch.int32, device=DEV)
    fp8.fp8_moe_route(torch.from_numpy(idx).to(DEV), E, off, dest)
    xq = torch.empty((P, H), dtype=torch.uint8, device=DEV)
    xs = torch.empty(P, device=DEV)
    fp8.fp8_moe_permute_quantize_row(dev_bf16(x), dest, fmt_act, 0, xq, xs)
    w1q = torch.empty((E * I2, H), dtype=torch.uint8, device=DEV)
    w1s = torch.empty(E * I2, device=DEV)
    fp8.fp8_quantize_row(dev_bf16(w1.reshape(E * I2, H)), fmt_w, 0, w1q, w1s)
    h = torch.empty((P, I2), dtype=torch.bfloat16, device=DEV)
    fp8.fp8_grouped_gemm_scaled(xq, fmt_act, w1q.view(E, I2, H), fmt_w, off, xs, w1s.view(E, I2), h)
    aq = torch.empty((P, inter), dtype=torch.uint8, device=DEV)
    asi = torch.empty(P, device=DEV)
    fp8.fp8_swiglu_quantize_row(h, fmt_act, 0, aq, asi)
    w2q = torch.empty((E * H, inter), dtype=torch.uint8, device=DEV)
    w2s = torch.empty(E * H, device=DEV)
    fp8.fp8_quantize_row(dev_bf16(w2.reshape(E * H, inter)), fmt_w, 0, w2q, w2s)
    y = torch.empty((P, H), dtype=torch.bfloat16, device=DEV)
    fp8.fp8_grouped_gemm_scaled(aq, fmt_act, w2q.view(E, H, inter), fmt_w, off, asi, w2s.view(E, H), y)
    out = torch.empty((T, H), dtype=torch.bfloat16, device=DEV)
    fp8.fp8_moe_unpermute_combine(y, dest, torch.from_numpy(wts).to(DEV), out)
    torch.cuda.synchronize()
    return out, {"off": off, "dest": dest, "xq": xq, "xs": xs, "h": h, "aq": aq, "asi": asi, "y": y}


def layer_oracle(orc, d):
    """The oracle's composition of the same steps (GEMM outputs rounded to bf16
    as the library stores them). Returns (out fp64, bound base)."""
    x, idx, wts, w1, w2 = d["x"], d["idx"], d["weights"], d["w1"], d["w2"]
    T, H = x.shape
    E, I2, _ = w1.shape
    off, dest = orc.moe_route(idx, E)
    xq, xs = orc.moe_permute_quantize_row(x, dest, 0)
    w1q, w1s, _ = orc.quantize_row(w1.reshape(E * I2, H), 0)
    h, _ = orc.grouped_gemm(xq, 0, w1q.reshape(E, I2, H), 0, off, xs, w1s.reshape(E, I2))
    aq, asi, _ = orc.swiglu_quantize_row(orc.bf16_round(h), 0)
    w2q, w2s, _ = orc.quantize_row(w2.reshape(E * H, -1), 0)
    y, ybound = orc.grouped_gemm(aq, 0, w2q.reshape(E, H, -1), 0, off, asi, w2s.reshape(E, H))
    out, _ = orc.moe_unpermute_combine(orc.bf16_round(y), dest, wts)
    base, _ = orc.moe_unpermute_combine(orc.bf16_round(ybound), dest, wts)
    return out, base, (off, dest, xq, xs)


def test_moe_layer_composed(fp8, orc):
    """A small layer (300 tokens, top-4 of 8 experts, hidden 512, expert FFN
    256): routing and permuted codes bit-exact; the output within
    2^-7 |out| + 2% of the weighted sum of the down product's magnitudes (a
    bf16 step of h can move a SwiGLU code by one quantum)."""
    d = workloads.c6(tokens=300, experts=8, topk=4, hidden=512, inter=256, seed=3)
    say("moe layer composed")
    out, mid = layer_gpu(fp8, d)
    o, base, (off, dest, xq, xs) = layer_oracle(orc, d)
    assert np.array_equal(mid["off"].cpu().numpy(), off)
    assert np.array_equal(mid["dest"].cpu().numpy(), dest)
    assert_codes_equal(mid["xq"].cpu().numpy(), xq, "permuted token codes")
    got = out.float().cpu().numpy().astype(np.float64)
    bad = np.abs(got - o) > 2.0 ** -7 * np.abs(o) + 0.02 * base
    assert not bad.any(), f"{int(bad.sum())} of {bad.size} layer outputs off"


def test_c6_layer_full_size_steps(fp8, orc):
    """The full-size layer (2048 tokens, top-8 of 32, hidden 7168, FFN 2048) in
    the bench's launch configuration: routing and permuted codes bit-exact on
    the whole tensors, every output of the gate|up product within the GEMM
    bound; the SwiGLU cast and the combine at the same shapes on generated
    inputs (the oracle never takes the GPU's intermediates)."""
    say("c6 generate")
    d = workloads.c6()
    T, H = d["x"].shape
    E, I2, _ = d["w1"].shape
    k = d["idx"].shape[1]
    P, inter = T * k, I2 // 2
    say("c6 layer")
    out, mid = layer_gpu(fp8, d)
    off, dest = orc.moe_route(d["idx"], E)
    assert np.array_equal(mid["off"].cpu().numpy(), off)
    assert np.array_equal(mid["dest"].cpu().numpy(), dest)
    xq, xs = orc.moe_permute_quantize_row(d["x"], dest, 0)
    assert_codes_equal(mid["xq"].cpu().numpy(), xq, "permuted token codes")
    assert_f32_bits_equal(mid["xs"].cpu().numpy(), xs, "permuted token scale_inv")
    w1q, w1s, _ = orc.quantize_row(d["w1"].reshape(E * I2, H), 0)
    h_gpu = mid["h"].float().cpu().numpy()
    rows = 0
    for e in range(E):
        lo, hi = int(off[e]), int(off[e + 1])
        if hi > lo:
            rows += check_full(orc, h_gpu, orc.gemm_by_rows(xq[lo:hi], 0, w1q[e * I2:(e + 1) * I2], 0, xs[lo:hi],
                                                            w1s[e * I2:(e + 1) * I2]), f"c6 gate|up expert {e}",
                               row_offset=lo)
    assert rows == P
    say("c6 swiglu at full shape")
    h = workloads.bf16_bits((np.random.default_rng(22).standard_normal((P, I2)) * 3).astype(np.float32))
    q = torch.empty((P, inter), dtype=torch.uint8, device=DEV)
    si = torch.empty(P, device=DEV)
    fp8.fp8_swiglu_quantize_row(dev_bf16(h), 0, 0, q, si)
    torch.cuda.synchronize()
    rows = np.random.default_rng(23).choice(P, 512, replace=False)
    check_swiglu(orc, 0, h[rows], q.cpu().numpy()[rows], si.cpu().numpy()[rows])
    say("c6 combine at full shape")
    yb = workloads.bf16_bits(np.random.default_rng(24).standard_normal((P, H)).astype(np.float32))
    o = torch.empty((T, H), dtype=torch.bfloat16, device=DEV)
    fp8.fp8_moe_unpermute_combine(dev_bf16(yb), torch.from_numpy(dest).to(DEV),
                                  torch.from_numpy(d["weights"]).to(DEV), o)
    torch.cuda.synchronize()
    ref, mag = orc.moe_unpermute_combine(yb, dest, d["weights"])
    got = o.float().cpu().numpy().astype(np.float64)
    assert not (np.abs(got - ref) > 2.0 ** -8 * np.abs(ref) + (k + 1) * 2.0 ** -24 * mag).any()
