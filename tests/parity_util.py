"""Helpers for GPU-vs-oracle parity tests."""
import sys

import numpy as np

E2M1_MAG = np.array([0, .5, 1, 1.5, 2, 3, 4, 6])

# Tolerances for the rotated path: rotated values agree to 1e-5 relative
# (fp32 butterfly vs dense double product); at most 1e-4 of codes differ, each
# by one grid step with the oracle's value within 1e-5 * amax_b of the midpoint
# that separates the two codes; a scale byte may differ only when the block's
# oracle amax lies within 1e-5 relative of a scale boundary 6 * 2^e.
ROT_REL = 1e-5
ROT_CODE_FRAC = 1e-4


def note(msg):
    """Name the case on stdout before a GPU step (flushed)."""
    print(msg, flush=True)
    sys.stdout.flush()


def to_dev(x_u16, dev="cuda"):
    import torch
    return torch.from_numpy(np.ascontiguousarray(x_u16).view(np.int16)).to(dev).view(torch.bfloat16)


def bf16_bits(t):
    import torch
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def unpack(codes):
    out = np.empty((codes.shape[0], codes.shape[1] * 2), np.uint8)
    out[:, 0::2] = codes & 15
    out[:, 1::2] = codes >> 4
    return out


def same_bf16(a, b):
    """Bitwise equal, except that any NaN matches any NaN."""
    a = np.asarray(a, np.uint16)
    b = np.asarray(b, np.uint16)
    na = ((a & 0x7F80) == 0x7F80) & ((a & 0x7F) != 0)
    nb = ((b & 0x7F80) == 0x7F80) & ((b & 0x7F) != 0)
    return bool(np.all((a == b) | (na & nb)))


def check_rotated(y_gpu, y_orc, codes_gpu, scales_gpu, codes_orc, scales_orc):
    """Apply the rotated-path tolerance; returns a dict of counts."""
    r = rotated_counts(y_gpu, y_orc, codes_gpu, scales_gpu, codes_orc, scales_orc)
    n_bad = r["codes_differ"] + 32 * r["scales_differ"]
    assert n_bad <= ROT_CODE_FRAC * r["total"], f"{n_bad} of {r['total']} codes differ"
    return r


def check_rotated_rows(y_gpu_dev, y_orc, codes_gpu, scales_gpu, codes_orc, scales_orc,
                       chunk=1024):
    """check_rotated over a whole tensor in chunks of rows (bounded host
    memory): every element and block condition on every chunk, the fraction
    of differing codes over the whole tensor. y_gpu_dev: device fp32."""
    rows = y_orc.shape[0]
    tot = {"codes_differ": 0, "scales_differ": 0, "total": 0}
    for r0 in range(0, rows, chunk):
        r1 = min(rows, r0 + chunk)
        r = rotated_counts(y_gpu_dev[r0:r1].cpu().numpy(), y_orc[r0:r1], codes_gpu[r0:r1],
                           scales_gpu[r0:r1], codes_orc[r0:r1], scales_orc[r0:r1])
        for k in tot:
            tot[k] += r[k]
    n_bad = tot["codes_differ"] + 32 * tot["scales_differ"]
    assert n_bad <= ROT_CODE_FRAC * tot["total"], f"{n_bad} of {tot['total']} codes differ"
    return tot


def rotated_counts(y_gpu, y_orc, codes_gpu, scales_gpu, codes_orc, scales_orc):
    """The per-element and per-block conditions of the rotated-path tolerance
    (asserted); returns the counts of differing codes and scale bytes."""
    rows, cols = y_orc.shape
    yo = y_orc.astype(np.float64).reshape(rows, cols // 32, 32)
    yg = y_gpu.astype(np.float64).reshape(rows, cols // 32, 32)
    amax = np.abs(yo).max(-1)
    d = yg - yo
    blk_norm = np.sqrt((yo * yo).sum(-1))
    assert np.all(np.sqrt((d * d).sum(-1)) <= ROT_REL * np.maximum(blk_norm, 1e-30)), \
        "rotated values: block relative error above tolerance"
    assert np.all(np.abs(d) <= ROT_REL * np.maximum(amax, 1e-30)[..., None]), \
        "rotated values: element error above tolerance"

    sg, so = scales_gpu.astype(np.int64), scales_orc.astype(np.int64)
    bad_scale = sg != so
    if bad_scale.any():
        e = so[bad_scale] - 127
        near = np.minimum(np.abs(amax[bad_scale] - 6 * np.ldexp(1.0, e)),
                          np.abs(amax[bad_scale] - 6 * np.ldexp(1.0, e - 1)))
        assert np.all(near <= ROT_REL * amax[bad_scale]), "scale byte differs away from a boundary"

    ug = unpack(codes_gpu).reshape(rows, cols // 32, 32).astype(np.int64)
    uo = unpack(codes_orc).reshape(rows, cols // 32, 32).astype(np.int64)
    # +0 and -0 are the same value
    vg = np.where((ug & 7) == 0, 0, ug)
    vo = np.where((uo & 7) == 0, 0, uo)
    diff = (vg != vo) & ~bad_scale[..., None]
    n_diff = int(diff.sum())
    if n_diff:
        sgn_g, sgn_o = (ug >> 3) & 1, (uo >> 3) & 1
        mg, mo = ug & 7, uo & 7
        sel = diff
        one_step = (np.abs(mg[sel] - mo[sel]) == 1) & ((sgn_g[sel] == sgn_o[sel]) |
                                                       (mg[sel] == 0) | (mo[sel] == 0))
        assert np.all(one_step), "a code differs by more than one grid step"
        e = (so - 127)[..., None] * np.ones_like(mg)
        scale = np.ldexp(1.0, e[sel])
        mid = (E2M1_MAG[mg[sel]] + E2M1_MAG[mo[sel]]) / 2 * scale
        amax_e = (amax[..., None] * np.ones_like(mg))[sel]
        assert np.all(np.abs(np.abs(yo[sel]) - mid) <= ROT_REL * amax_e), \
            "a code differs away from a rounding midpoint"
    return {"codes_differ": n_diff, "scales_differ": int(bad_scale.sum()), "total": rows * cols}
