"""The split calls' selection rules, restated from include/rlca.h for the
tests (no GPU needed): which form a split window call takes."""
import torch

import reverse_linear_recurrence_amd as rl


def residency(algo, k, waves, tiles, bf16):
    """Workgroups of a chained instance one compute unit holds at once,
    counted up to 2: 1 for the 16-wavefront two-tile segments of returns,
    GAE and TD(lambda) at K = 8, of V-trace, and of Retrace at K = 8 or on
    bf16 inputs; 2 otherwise."""
    if waves != 16 or tiles != 2:
        return 2
    if algo in ("returns", "gae", "td_lambda"):
        return 1 if k == 8 else 2
    if algo == "vtrace":
        return 1
    if algo == "retrace":
        return 1 if k == 8 or bf16 else 2
    return 2


def chain_segments(N, T, dtype, algo):
    """The chained split's segments per row (0: none), by its stated rule:
    N rows of T >= 8192 steps with N <= 224 and N <= T / 128; segments of L
    steps, one or two whole tiles of a tiling with whole wavefronts per row,
    2 to 256 per row; of those, the one with the least
    ceil(N * S / 256) * L + ceil(N * S / (256 * r)) * 4096 + 32 * S (r:
    residency),
    ties going to the longer segment; on bf16 inputs (but for V-trace) the
    tilings with K = 8 first, the others only where none of those fits.
    algo: a key of rl.ALGO_CODES (the affine scan: "affine", either
    direction)."""
    if N < 1 or N > 224 or T < 8192 or 128 * N > T:
        return 0
    bf16 = torch_dtype(dtype) == torch.bfloat16

    def best_of(wide_only):
        best = None
        for v in range(rl.rlca_num_variants()):
            k, lanes, waves = rl.rlca_variant_info(v, dtype, algo)
            if waves == 1 or (wide_only and k != 8):
                continue
            for tiles in (1, 2):
                length = tiles * k * lanes
                if T % length:
                    continue
                S = T // length
                if S < 2 or S > 256:
                    continue
                r = residency(algo, k, waves, tiles, bf16)
                cost = -(-N * S // 256) * length + -(-N * S // (256 * r)) * 4096 + 32 * S
                key = (cost, -length)
                if best is None or key < best[0]:
                    best = (key, S)
        return None if best is None else best[1]

    S = best_of(True) if bf16 and algo != "vtrace" else None
    if S is None:
        S = best_of(False)
    return S or 0


def torch_dtype(dtype):
    return torch.bfloat16 if dtype in ("bf16", torch.bfloat16) else torch.float32


def takes_chained(N, T, dtype, algo):
    """Whether a split window call (workspace large enough, 8-byte aligned,
    rows sharing one stride, chaining on) takes the chained form: whenever a
    chained plan exists."""
    return chain_segments(N, T, torch_dtype(dtype), algo) > 0
