"""Shared helpers of the GPU parity tests: moving the generators' bit patterns
to the device, allocating outputs with guard bands, and printing the case
before each GPU step."""
import sys

import numpy as np
import torch

SENTINEL = 0x5A


def say(*args):
    """Name the case (flushed) before a GPU step, so a failure can be located."""
    print("[case]", *args, flush=True)
    sys.stdout.flush()


def dev_bf16(bits):
    """uint16 bf16 bit patterns (numpy) -> torch.bfloat16 tensor on cuda:0."""
    bits = np.ascontiguousarray(bits, np.uint16)
    return torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to("cuda:0")


def host_bits(t):
    """torch.bfloat16 tensor -> uint16 numpy bit patterns."""
    return t.detach().view(torch.int16).cpu().numpy().view(np.uint16)


def dev_u8(a):
    return torch.from_numpy(np.ascontiguousarray(a, np.uint8)).to("cuda:0")


def dev_f32(a):
    return torch.from_numpy(np.ascontiguousarray(a, np.float32)).to("cuda:0")


def guarded(rows, cols, dtype, ld=None, pad_rows=2, fill=SENTINEL):
    """A [rows x cols] view with row stride ld (default cols + 32) inside a
    buffer with pad_rows extra rows above and below; everything outside the
    view holds a sentinel, so check_guard() afterwards detects any write outside
    the view. Returns (view, buffer, (r0, c0))."""
    ld = ld if ld is not None else cols + 32
    assert ld >= cols
    r0, c0 = pad_rows, 0
    buf = torch.empty((rows + 2 * pad_rows, max(ld, 1)), dtype=dtype, device="cuda:0")
    ints = {1: torch.uint8, 2: torch.int16, 4: torch.int32}[buf.element_size()]
    buf.view(ints).fill_(fill)
    view = buf[r0:r0 + rows, c0:c0 + cols]
    return view, buf, (r0, c0)


def check_guard(buf, origin, rows, cols, fill=SENTINEL):
    """Every element of buf outside the [rows x cols] view at origin still holds the sentinel."""
    r0, c0 = origin
    host = buf.detach().cpu()
    if host.element_size() == 1:
        raw = host.view(torch.uint8).numpy()
        expect = fill
    elif host.element_size() == 2:
        raw = host.view(torch.int16).numpy().view(np.uint16)
        expect = np.array(fill, np.int16).view(np.uint16)
    else:
        raw = host.view(torch.int32).numpy().view(np.uint32)
        expect = np.array(fill, np.int32).view(np.uint32)
    mask = np.ones(raw.shape, bool)
    mask[r0:r0 + rows, c0:c0 + cols] = False
    bad = np.nonzero(raw[mask] != expect)[0]
    assert bad.size == 0, f"{bad.size} writes outside the output view"


def assert_codes_equal(got, want, what):
    got = np.asarray(got)
    want = np.asarray(want)
    assert got.shape == want.shape, (what, got.shape, want.shape)
    bad = np.argwhere(got != want)
    if bad.size:
        i = tuple(bad[0])
        raise AssertionError(f"{what}: {len(bad)} mismatches, first at {i}: gpu {got[i]!r} oracle {want[i]!r}")


def assert_f32_bits_equal(got, want, what):
    """Bitwise equality of fp32 arrays, treating any NaN as equal to any NaN."""
    g = np.asarray(got, np.float32)
    w = np.asarray(want, np.float32)
    assert g.shape == w.shape, (what, g.shape, w.shape)
    same = (g.view(np.uint32) == w.view(np.uint32)) | (np.isnan(g) & np.isnan(w))
    bad = np.argwhere(~same)
    if bad.size:
        i = tuple(bad[0])
        raise AssertionError(f"{what}: {len(bad)} mismatches, first at {i}: gpu {g[i]!r} oracle {w[i]!r}")


def check_full(orc, d, blocks, what, row_offset=0, out_bf16=True):
    """Every output of d (a torch tensor [rows x n], or its values already on
    the host as a numpy array) against the oracle's row blocks (r0, r1, y,
    bound), r0/r1 counted from row_offset of d. Reports the largest
    |gpu - oracle| as a fraction of the allowed error."""
    host = d if isinstance(d, np.ndarray) else d.float().cpu().numpy()
    worst, rows = 0.0, 0
    for r0, r1, y, bound in blocks:
        got = host[row_offset + r0:row_offset + r1].astype(np.float64)
        ok = orc.gemm_within_bound(got, y, bound, out_bf16=out_bf16)
        if not ok.all():
            i, j = np.argwhere(~ok)[0]
            raise AssertionError(f"{what}: {int((~ok).sum())} outputs outside the bound in rows {r0}..{r1}; first "
                                 f"({row_offset + r0 + i}, {j}): gpu {got[i, j]!r} oracle {y[i, j]!r} "
                                 f"bound {bound[i, j]!r}")
        tol = 1e-3 * bound + (2.0 ** -8 * np.abs(y) if out_bf16 else 0.0)
        fin = np.isfinite(y) & (tol > 0)
        if fin.any():
            worst = max(worst, float((np.abs(got - y)[fin] / tol[fin]).max()))
        rows += r1 - r0
    say(what, "every output of", rows, "rows within the bound; max |err| / allowed =", round(worst, 4))
    return rows
