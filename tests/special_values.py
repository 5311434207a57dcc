"""IEEE special-value inputs and the comparison rule for them (test helpers).

Inputs are bit patterns built from the seeded generator in `gen`; nothing
here computes the sync method's arithmetic. Used by the GPU parity tests and
by the oracle's CPU pins on the same scenarios.
"""
import numpy as np
import torch

import gen
from tests.helpers import to_np

# bit patterns of special values
F32 = dict(pz=0x00000000, nz=0x80000000, pinf=0x7F800000, ninf=0xFF800000, qnan=0x7FC00000,
           snan=0x7F800001, max=0x7F7FFFFF, min_normal=0x00800000, one=0x3F800000,
           one_ulp=0x3F800001, tie=0x33800000)              # tie = 2^-24: 1 + 2^-24 is a tie
BF16 = dict(pz=0x0000, nz=0x8000, pinf=0x7F80, ninf=0xFF80, qnan=0x7FC0, snan=0x7F81,
            max=0x7F7F, min_normal=0x0080, one=0x3F80, one_ulp=0x3F81,
            tie=0x3B80,                                     # 2^-8: 1 + 2^-8 rounds to even
            over_tie=0x7B00, under_tie=0x7A80)              # 2^119, 2^118 beside max


def _is_nan(bits, dtype):
    if dtype == np.uint16:
        return ((bits & 0x7F80) == 0x7F80) & ((bits & 0x007F) != 0)
    b = bits.view(np.uint32)
    return ((b & 0x7F800000) == 0x7F800000) & ((b & 0x007FFFFF) != 0)


def _as_bits(a):
    return a if a.dtype == np.uint16 else a.view(np.uint32)


def special_equal(got, want):
    """Bit-exact, except that a NaN of the oracle only needs a NaN."""
    if got.shape != want.shape:
        return False
    g, w = _as_bits(got), _as_bits(want)
    wn = _is_nan(w, w.dtype)
    gn = _is_nan(g, g.dtype)
    return bool(np.array_equal(g[~wn], w[~wn]) and np.all(gn[wn]))


def special_inputs(dtype, k, n, seed):
    """K rank vectors (numpy bit patterns: uint32 for fp32, uint16 for bf16)
    in which every position follows one of 16 scenarios drawn from the seeded
    generator: ordinary values, all -0.0, mixed signed zeros, one or two
    infinities, one or two NaNs (quiet and signalling, both signs, varied
    payloads), all subnormal, a free mix of specials, a sum at or just below
    the bf16 overflow point, an exact rounding tie, a cancelling +-2^30 pair."""
    bf = dtype == torch.bfloat16
    S = BF16 if bf else F32
    ut = np.uint16 if bf else np.uint32
    sign = ut(0x8000) if bf else ut(0x80000000)
    scen = (gen.raw_u64(seed, 90, 0, 0, n).numpy().view(np.uint64) >> np.uint64(60)).astype(np.int64)
    rnd = [gen.raw_u64(seed, 91, r, 0, n).numpy().view(np.uint64) for r in range(k)]
    pick = gen.raw_u64(seed, 92, 0, 0, n).numpy().view(np.uint64)
    a_rank = (pick % np.uint64(k)).astype(np.int64)
    b_rank = (a_rank + 1 + ((pick >> np.uint64(8)) % np.uint64(max(1, k - 1))).astype(np.int64)) % k
    ordinary = []
    for r in range(k):
        u = gen.uniform_pm1(seed, 93, r, n)
        ordinary.append(to_np(u.to(torch.bfloat16)) if bf else u.numpy().view(np.uint32))
    x = [o.copy() for o in ordinary]

    def put(mask, rank_of, bits):
        """x[rank_of[i]][i] = bits[i] for i in mask (rank_of: array or int)."""
        ro = np.broadcast_to(np.asarray(rank_of), (n,))
        bb = np.broadcast_to(np.asarray(bits, dtype=ut), (n,))
        for r in range(k):
            m = mask & (ro == r)
            x[r][m] = bb[m]

    def rsign(r, shift):
        return np.where((rnd[r] >> np.uint64(shift)) & np.uint64(1), sign, ut(0)).astype(ut)

    def nan_bits(r, signalling):
        mbits = 7 if bf else 23
        pay = ((rnd[r] >> np.uint64(20)) & np.uint64((1 << (mbits - 1)) - 1)).astype(ut)
        if signalling:
            pay = np.maximum(pay, ut(1))                    # quiet bit clear, payload non-zero
            base = ut(S["pinf"])
        else:
            base = ut(S["qnan"])
        return (base | pay | rsign(r, 3)).astype(ut)

    zeros_mixed = lambda r: rsign(r, 5)
    for r in range(k):
        # 4: every rank -0.0; 5: mixed signed zeros
        x[r][scen == 4] = ut(S["nz"])
        x[r][scen == 5] = zeros_mixed(r)[scen == 5]
        # 10: every rank subnormal (random sign and fraction)
        mbits = 7 if bf else 23
        frac = ((rnd[r] >> np.uint64(30)) & np.uint64((1 << mbits) - 1)).astype(ut)
        frac = np.maximum(frac, ut(1))
        x[r][scen == 10] = (frac | rsign(r, 7))[scen == 10]
        # 11: a free mix of specials per rank
        pool = np.array([S["pz"], S["nz"], S["pinf"], S["ninf"], S["qnan"], S["snan"], S["max"],
                         S["min_normal"]], dtype=ut)
        choice = ((rnd[r] >> np.uint64(40)) % np.uint64(len(pool) + 2)).astype(np.int64)
        mix = np.where(choice < len(pool), pool[np.minimum(choice, len(pool) - 1)] | rsign(r, 9),
                       ordinary[r]).astype(ut)
        mix = np.where(choice == 4, nan_bits(r, False), mix)
        mix = np.where(choice == 5, nan_bits(r, True), mix)
        x[r][scen == 11] = mix[scen == 11]
        # 12-14: zeros everywhere except the two ranks set below
        x[r][(scen >= 12) & (scen <= 14)] = zeros_mixed(r)[(scen >= 12) & (scen <= 14)]
    # 6: one infinity; 7: +Inf and -Inf
    put(scen == 6, a_rank, np.where(rsign(0, 11) != 0, ut(S["ninf"]), ut(S["pinf"])))
    put(scen == 7, a_rank, ut(S["pinf"]))
    put(scen == 7, b_rank, ut(S["ninf"]))
    # 8: one NaN (quiet or signalling); 9: two NaNs with different payloads
    for r in range(k):
        q = nan_bits(r, bool(r & 1))
        put((scen == 8) & (a_rank == r), r, q)
        put((scen == 9) & (a_rank == r), r, q)
        put((scen == 9) & (b_rank == r), r, nan_bits(r, False) ^ ut(1 << 1))
    # 12: the largest finite value twice (fp32: overflows to Inf in the sum);
    #     bf16: max + 2^119 is exactly the rounding tie above max -> Inf
    # 13: bf16: max + 2^118 stays below the tie -> max; fp32: max + max again
    s_ab = rsign(1 % k, 13)
    if bf:
        put(scen == 12, a_rank, ut(S["max"]) | s_ab)
        put(scen == 12, b_rank, ut(S["over_tie"]) | s_ab)
        put(scen == 13, a_rank, ut(S["max"]) | s_ab)
        put(scen == 13, b_rank, ut(S["under_tie"]) | s_ab)
    else:
        put((scen == 12) | (scen == 13), a_rank, ut(S["max"]) | s_ab)
        put((scen == 12) | (scen == 13), b_rank, ut(S["max"]) | s_ab)
    # 14: an exact rounding tie: 1 (or 1 + ulp) plus half an ulp, same sign
    odd = ((rnd[0] >> np.uint64(17)) & np.uint64(1)).astype(bool)
    put(scen == 14, a_rank, np.where(odd, ut(S["one_ulp"]), ut(S["one"])) | s_ab)
    put(scen == 14, b_rank, ut(S["tie"]) | s_ab)
    # 15: +-2^30 pair cancelling over ordinary values
    big = ut(0x4E80) if bf else ut(0x4E800000)
    put(scen == 15, a_rank, big)
    put(scen == 15, b_rank, big | sign)
    return x


def scenarios(n, seed):
    """Scenario id (0..15) of every position, as special_inputs draws it."""
    return (gen.raw_u64(seed, 90, 0, 0, n).numpy().view(np.uint64) >> np.uint64(60)).astype(np.int64)
