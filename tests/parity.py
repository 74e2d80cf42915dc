"""Parity rules between the HIP path and the oracle (test helper).

The rules (codes and sign bits bit-exact except coordinates within 1e-4 of a
decision boundary or of zero, at most 1e-6 of them; norms and dequantized
values to 1e-3 relative; scores to 1e-3 of the L1 size of the summed terms and
to 1e-3 relative wherever the score is not small against that size) are
applied here.  The oracle takes every decision in float64; the kernels decide
in fp32, so a coordinate within the fp32 error of a boundary may take the other
side -- such flips are counted, reported as a rate and capped.  Where floating point legitimately decides an integer on
either side of a boundary, the oracle supplies the other candidate itself
(``codec.boundary_distance``) and the GPU result must be one of the oracle's
candidates; dependent results (residual bits) are then compared with the
oracle's computation for that candidate.  No expected value is read from the
GPU.
"""

import math

import numpy as np
import torch

import oracle
from oracle import codec, qjl, numerics

BAND = 1e-4          # N(0,1) units for codes, units of ||r|| for sign bits
RATE_CAP = 1e-6      # largest fraction of band mismatches
NORM_SLOP = 4e-6     # relative fp32 error of a block norm the fp16 rounding may see


def mismatch_cap(n):
    """Allowed count of band mismatches among n decisions: 1e-6 of them, and one
    when fewer than 1e6 decisions are compared (the rate cannot be resolved there)."""
    return max(1, int(math.floor(RATE_CAP * n)))


# ------------------------------------------------------------------------------ conversions

def bf16_tensor(u16, device="cuda"):
    return torch.from_numpy(np.ascontiguousarray(u16).view(np.int16)).view(torch.bfloat16).to(device)


def u16_of(t):
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def f16_values(t):
    return t.cpu().numpy().astype(np.float64)


def u8_tensor(a, device="cuda"):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.uint8)).to(device)


# ------------------------------------------------------------------------------ checks

def fp16_candidates(v):
    """fp16 values a float64 quantity may round to once computed in fp32."""
    return (numerics.round_fp16(v * (1 - NORM_SLOP)), numerics.round_fp16(v), numerics.round_fp16(v * (1 + NORM_SLOP)))


def pick_candidate(gpu, cands, what):
    lo, mid, hi = cands
    ok = (gpu == lo) | (gpu == mid) | (gpu == hi) | (np.isnan(gpu) & np.isnan(mid))
    bad = np.flatnonzero(~ok)
    assert bad.size == 0, "%s: %d fp16 values outside the rounding candidates, first at %d: gpu %r oracle %r" % (
        what, bad.size, bad[0], gpu[bad[0]], mid[bad[0]])
    return np.where(gpu == lo, lo, np.where(gpu == hi, hi, mid))


def check_quantize(x, bits, D, gpu_codes, gpu_n16, G=None, gpu_qbits=None, gpu_rn16=None, label="", cap=True):
    """x (n, d) float64 exact inputs; D +-1 vector; G (m, d) float64 or None.

    Returns a dict of mismatch statistics.  ``cap=False`` leaves the rate cap to the caller
    (a ``Tally`` over the chunks of a whole output); the band rule is always enforced."""
    n, d = x.shape
    ref = codec.quantize(x, bits, D)
    dist, other = codec.boundary_distance(ref["y"], bits)
    diff = gpu_codes != ref["codes"]
    allowed = (dist < BAND) & (gpu_codes == other)
    bad = diff & ~allowed
    nb = int(bad.sum())
    if nb:
        i = np.argwhere(bad)[0]
        raise AssertionError("%s: %d codes differ outside the boundary band; first block %d coord %d gpu %d "
                             "oracle %d y %.9g dist %.3g" % (label, nb, i[0], i[1], gpu_codes[tuple(i)],
                                                              ref["codes"][tuple(i)], ref["y"][tuple(i)],
                                                              dist[tuple(i)]))
    nflip = int(diff.sum())
    assert not cap or nflip <= mismatch_cap(diff.size), "%s: %d band flips among %d codes (rate %.3g)" % (
        label, nflip, diff.size, nflip / max(diff.size, 1))
    n16 = pick_candidate(gpu_n16, fp16_candidates(ref["norm"]), label + " norms")
    stats = {"codes": diff.size, "code_flips": nflip,
             "norm_ulp_diffs": int(np.sum(n16 != ref["n16"]))}
    if G is None:
        return stats
    m = G.shape[0]
    alt_codes = np.where(diff, other, ref["codes"])          # the oracle's candidate on the far side
    res = codec.qjl_residual(x, alt_codes, n16, bits, D, G)
    gb = numerics.unpack_bits_lsb(gpu_qbits, m)
    eb = numerics.unpack_bits_lsb(res["bits"], m)
    bdiff = gb != eb
    near = np.abs(res["p"]) < BAND * res["rnorm"][:, None]
    bbad = bdiff & ~near
    nbb = int(bbad.sum())
    if nbb:
        i = np.argwhere(bbad)[0]
        raise AssertionError("%s: %d sign bits differ away from zero; first block %d bit %d p/||r|| %.3g" % (
            label, nbb, i[0], i[1], res["p"][tuple(i)] / max(res["rnorm"][i[0]], 1e-300)))
    nbf = int(bdiff.sum())
    assert not cap or nbf <= mismatch_cap(bdiff.size), "%s: %d band sign flips among %d bits (rate %.3g)" % (
        label, nbf, bdiff.size, nbf / max(bdiff.size, 1))
    pick_candidate(gpu_rn16, fp16_candidates(res["rnorm"]), label + " residual norms")
    stats.update({"bits": bdiff.size, "bit_flips": nbf})
    return stats


def report(label, stats):
    """Print the measured flip rates of a comparison (visible with pytest -s or on failure)."""
    parts = []
    for k, f in (("codes", "code_flips"), ("bits", "bit_flips")):
        if k in stats:
            parts.append("%s %d flips / %d = %.3g" % (k, stats[f], stats[k], stats[f] / max(stats[k], 1)))
    print("[parity] %s: %s" % (label, "; ".join(parts)), flush=True)
    return stats


def check_dequantize(codes, n16, bits, D, gpu_out, out_bf16, label=""):
    """gpu_out float64 values of the GPU output; checks against the oracle's reconstruction."""
    ref = codec.dequantize(codes, n16, bits, D)
    d = codes.shape[1]
    floor = 0.01 * n16[:, None] / math.sqrt(d)
    if out_bf16:
        r = numerics.round_bf16(ref)
        ulp = np.ldexp(1.0, np.frexp(np.abs(r))[1] - 8)          # bf16 ulp at |r| (8 significant bits)
        err = np.abs(gpu_out - r)
        ok = (err <= ulp) | (err <= 1e-3 * np.maximum(np.abs(ref), floor))
    else:
        ok = np.abs(gpu_out - ref) <= 1e-3 * np.maximum(np.abs(ref), floor)
    bad = np.argwhere(~ok)
    assert bad.size == 0, "%s: %d dequantized values off; first %s gpu %r oracle %r" % (
        label, len(bad), tuple(bad[0]), gpu_out[tuple(bad[0])], ref[tuple(bad[0])])
    den = np.maximum(np.abs(ref), floor)
    use = np.isfinite(ref) & (den > 0)           # zero blocks reconstruct exactly to zero
    rel = np.abs(gpu_out - ref)[use] / den[use]
    return float(np.max(rel, initial=0.0))


def check_sketch(k, G, gpu_bits, gpu_n16, label="", cap=True):
    m = G.shape[0]
    ref = qjl.sketch(k, G)
    pick_candidate(gpu_n16, fp16_candidates(ref["norm"]), label + " key norms")
    gb = numerics.unpack_bits_lsb(gpu_bits, m)
    eb = numerics.unpack_bits_lsb(ref["bits"], m)
    bdiff = gb != eb
    near = np.abs(ref["p"]) < BAND * ref["norm"][:, None] * np.sqrt(np.mean(G * G))
    bbad = bdiff & ~near
    assert not bbad.any(), "%s: %d sign bits differ away from zero" % (label, int(bbad.sum()))
    nbf = int(bdiff.sum())
    assert not cap or nbf <= mismatch_cap(bdiff.size), "%s: %d band sign flips among %d (rate %.3g)" % (
        label, nbf, bdiff.size, nbf / max(bdiff.size, 1))
    return {"bits": bdiff.size, "bit_flips": nbf}


class Tally:
    """Flip counts summed over the chunks of one whole output; ``finish`` applies the rate cap
    to the totals and prints the measured rates."""

    def __init__(self):
        self.t = {"codes": 0, "code_flips": 0, "bits": 0, "bit_flips": 0, "norm_ulp_diffs": 0}

    def add(self, stats):
        for k, v in stats.items():
            self.t[k] = self.t.get(k, 0) + v
        return stats

    def finish(self, label):
        t = self.t
        assert t["code_flips"] <= mismatch_cap(t["codes"]), "%s: %d band flips among %d codes (rate %.3g)" % (
            label, t["code_flips"], t["codes"], t["code_flips"] / max(t["codes"], 1))
        assert t["bit_flips"] <= mismatch_cap(t["bits"]), "%s: %d band sign flips among %d bits (rate %.3g)" % (
            label, t["bit_flips"], t["bits"], t["bit_flips"] / max(t["bits"], 1))
        stats = {k: v for k, v in t.items() if v or k in ("codes", "code_flips", "bits", "bit_flips")}
        if not t["bits"]:
            stats.pop("bits", None), stats.pop("bit_flips", None)
        return report(label, stats)


REL_FLOOR = 0.01     # scores this small against their L1 size are held to the L1 rule only


def check_scores(gpu, ref, scale, label="", tol=1e-3):
    """|gpu - ref| <= tol * L1 size of the summed terms everywhere, and <= tol * |ref| wherever
    |ref| >= REL_FLOOR * L1 size (a relative error of a score near zero is undefined).  Returns
    the worst error relative to the L1 size."""
    gpu = np.asarray(gpu, dtype=np.float64)
    err = np.abs(gpu - ref)
    bad = err > tol * scale
    assert not bad.any(), "%s: %d scores off; worst rel-to-L1 %.3g" % (label, int(bad.sum()),
                                                                        float(np.max(err / scale)))
    big = np.abs(ref) >= REL_FLOOR * scale
    if big.any():
        rel = err[big] / np.abs(ref[big])
        assert float(rel.max()) <= tol, "%s: %d scores off by more than %.0e relative (worst %.3g)" % (
            label, int(np.sum(rel > tol)), tol, float(rel.max()))
    return float(np.max(err / scale, initial=0.0))
