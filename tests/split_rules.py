"""The split calls' selection rules, restated from include/rlca.h for the
tests (no GPU needed): which form a split window call takes."""
import torch

import reverse_linear_recurrence_amd as rl


def chain_segments(N, T, dtype, algo):
    """The chained split's segments per row (0: none), by its stated rule:
    tilings with whole wavefronts per row from the longest tile down, two
    tiles per segment before one, at most 256 segments per row; the first
    choice with N * S >= 256, else the one with the most segments."""
    if N < 1 or N > 64 or T < 32768:
        return 0
    best = 0
    for v in reversed(range(rl.rlca_num_variants())):
        k, lanes, waves = rl.rlca_variant_info(v, dtype, algo)
        if waves == 1:
            continue
        for tiles in (2, 1):
            length = tiles * k * lanes
            if T % length:
                continue
            S = T // length
            if S < 2 or S > 256:
                continue
            best = max(best, S)
            if N * S >= 256:
                return best
    return best


def torch_dtype(dtype):
    return torch.bfloat16 if dtype in ("bf16", torch.bfloat16) else torch.float32


def takes_chained(N, T, dtype, algo):
    """Whether a split window call (workspace large enough, 8-byte aligned,
    rows sharing one stride, chaining on) takes the chained form: whenever a
    chained plan exists."""
    return chain_segments(N, T, torch_dtype(dtype), algo) > 0
