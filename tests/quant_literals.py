"""Hand-worked cases of the one-byte caches' write rule, as literals.

The rule (fp8 E4M3 and int8 caches, one fp32 scale per (layer, block, KV
head) for K and one for V; the pages name FP8/E4M3 and INT8 KV but fix no
scheme -- "大模型推理加速核心KV Cache 复用机制与内存布局优化" §四, "LLM推理优化实战…" §6.1):
for each run of new rows that lands in one block already holding n0 rows with
scale s, s_old = (n0 > 0 ? s : 0), s_new = max(s_old, amax(run) / C) with C =
448 (E4M3) or 127 (int8); if s_new > s_old and n0 > 0 the held codes become
enc(dec(c) * s_old / s_new); the new rows become enc(x / s_new) (enc(x) when
s_new = 0).  E4M3 enc rounds to nearest, ties to the even mantissa; int8 enc
rounds to nearest integer, ties to even, clamped to +-127, and has no signed
zero.

Every expected code below was worked out by hand from that text and the two
formats' definitions (E4M3: value 2^(e-7) (1 + m/8), code (e << 3) | m, code 0
.. 7 subnormal m/8 * 2^-6, sign bit 0x80).  No code computed them.  Inputs are
chosen so that every x / s is exact in float32; ties are planted on purpose.

Scenario (one sequence, 1 layer, 1 KV head, head dim 64 with only dims 0 and 1
non-zero, 16-token blocks, blocks popped in the order 0, 1, 2, ...):
  step 1: 10 rows  -> block 0 slots 0..9                    (fresh block)
  step 2: 20 rows  -> block 0 slots 10..15 (run 1, 6 rows)  (held rows 10)
                      block 1 slots 0..13 (run 2, 14 rows)  (fresh block)
  step 3: 2 rows   -> block 1 slots 14..15                  (held rows 14)
The 20-row write is two runs with separate amax and scale updates: a rule that
took one amax over the whole write, or carried block 0's scale into block 1,
gives other codes and scales.
"""
from __future__ import annotations

# Per case: inputs[step] = (K rows, V rows), each row [dim0, dim1];
# expected codes after the last step: blocks[(block, "k" | "v")] = 16 rows of
# [dim0 code, dim1 code] (None = slot never written), and scales per step.

FP8 = dict(
    dtype="fp8",
    inputs=[
        # step 1: K amax 448 -> s = 1; V amax 7 -> s = 7/448 = 1/64
        ([[448, -1]] + [[r, -r] for r in range(1, 10)],
         [[-(r + 1) / 16, 7.0 if r == 9 else 0.0] for r in range(10)]),
        # step 2: K run 1 amax 896 -> s 1 -> 2 (held codes re-encoded at 1/2);
        #         K run 2 amax 28 -> fresh s = 28/448 = 1/16;
        #         V run 1 amax 3.5 (3.5/448 < 1/64: no growth); V run 2 all zero -> s = 0
        ([[896, 1], [2, -2], [3, -3], [5, -5], [7, -7], [9, -9],
          [28, -28], [1.0, -1.0], [1.0625, -1.0625], [1.1875, -1.1875], [2.0 ** -11, -(2.0 ** -11)],
          [0.0, -0.0], [1.125, 0.5]] + [[0.25 * (r - 12), 0.0625] for r in range(13, 20)],
         [[3.5, -0.5], [0.25, 0.125], [0.0, 0.0], [-1.0, 1.0], [0.0078125, 0.0], [2.0, -2.0]] +
         [[0.0, -0.0] for _ in range(14)]),
        # step 3: K amax 3 (no growth at 1/16); V held zeros at scale 0, amax 7 -> s = 1/64
        ([[0.5, -0.5], [3.0, 1.0]],
         [[7.0, 0.0], [-3.5, 0.25]]),
    ],
    scales={  # (block, pool): scale after step 1, 2, 3 (None = block not in use yet)
        (0, "k"): [1.0, 2.0, 2.0],
        (0, "v"): [1 / 64, 1 / 64, 1 / 64],
        (1, "k"): [None, 0.0625, 0.0625],
        (1, "v"): [None, 0.0, 1 / 64],
    },
    blocks={
        # block 0 K: rows 0..9 re-encoded at s 1 -> 2 (value / 2): 448 -> 224 (0x76),
        # -1 -> -0.5 (0xB0); r -> r/2: 0.5 0x30, 1 0x38, 1.5 0x3C, 2 0x40, 2.5 0x42,
        # 3 0x44, 3.5 0x46, 4 0x48, 4.5 0x49.  Rows 10..15 = step 2 run 1 / 2:
        # [448, .5] [1, -1] [1.5, -1.5] [2.5, -2.5] [3.5, -3.5] [4.5, -4.5]
        (0, "k"): [[0x76, 0xB0], [0x30, 0xB0], [0x38, 0xB8], [0x3C, 0xBC], [0x40, 0xC0], [0x42, 0xC2],
                   [0x44, 0xC4], [0x46, 0xC6], [0x48, 0xC8], [0x49, 0xC9],
                   [0x7E, 0x30], [0x38, 0xB8], [0x3C, 0xBC], [0x42, 0xC2], [0x46, 0xC6], [0x49, 0xC9]],
        # block 1 K (s = 1/16, values x 16): 448 0x7E; 16 0x58; 17 ties 16/18 -> 16 (even
        # mantissa) 0x58; 19 ties 18/20 -> 20 0x5A; 2^-7 subnormal m = 4 0x04; +-0 0x00 / 0x80;
        # [18, 8] [0x59, 0x50]; 4 8 12 16 20 24 28 -> 0x48 0x50 0x54 0x58 0x5A 0x5C 0x5E
        # with dim 1 = 1 (0x38); step 3: [8, -8] [48, 16] -> [0x50, 0xD0] [0x64, 0x58]
        (1, "k"): [[0x7E, 0xFE], [0x58, 0xD8], [0x58, 0xD8], [0x5A, 0xDA], [0x04, 0x84], [0x00, 0x80],
                   [0x59, 0x50], [0x48, 0x38], [0x50, 0x38], [0x54, 0x38], [0x58, 0x38], [0x5A, 0x38],
                   [0x5C, 0x38], [0x5E, 0x38], [0x50, 0xD0], [0x64, 0x58]],
        # block 0 V (s = 1/64, values x 64): rows 0..9: -4 -8 -12 -16 -20 -24 -28 -32 -36 -40
        # -> 0xC8 0xD0 0xD4 0xD8 0xDA 0xDC 0xDE 0xE0 0xE1 0xE2, dim 1 zero except 448 (0x7E)
        # in row 9; rows 10..15 (no growth): [224, -32] [16, 8] [0, 0] [-64, 64] [0.5, 0]
        # [128, -128]
        (0, "v"): [[0xC8, 0x00], [0xD0, 0x00], [0xD4, 0x00], [0xD8, 0x00], [0xDA, 0x00], [0xDC, 0x00],
                   [0xDE, 0x00], [0xE0, 0x00], [0xE1, 0x00], [0xE2, 0x7E],
                   [0x76, 0xE0], [0x58, 0x50], [0x00, 0x00], [0xE8, 0x68], [0x30, 0x00], [0x70, 0xF0]],
        # block 1 V: 14 zero rows at s = 0 keep their signed zeros (enc(x)); step 3 grows the
        # scale 0 -> 1/64 and re-encodes them as enc(+-0 * 0 / s) = the same codes; new rows
        # x 64: [448, 0] [-224, 16]
        (1, "v"): [[0x00, 0x80]] * 14 + [[0x7E, 0x00], [0xF6, 0x58]],
    },
)

INT8 = dict(
    dtype="int8",
    inputs=[
        # step 1: K amax 127 -> s = 1, ties 0.5 -> 0, 1.5 -> 2, 2.5 -> 2, 3.5 -> 4 (signs alike);
        #         V amax 31.75 -> s = 0.25, x / s = r + 0.5 and -r / 2 (ties)
        ([[127, -0.5], [0.5, 1.5], [2.5, -1.5], [-2.5, 3.5]] + [[r, -r] for r in range(4, 10)],
         [[31.75, 0.0]] + [[0.25 * r + 0.125, -0.125 * r] for r in range(1, 10)]),
        # step 2: K run 1 amax 254 -> s 1 -> 2 (held codes halved, ties to even);
        #         K run 2 amax 7.9375 = 127/16 -> fresh s = 1/16;
        #         V run 1 amax 10 (10/127 < 0.25: no growth); V run 2 all zero -> s = 0
        ([[254, 1], [3, -3], [5, 7], [-1, 0], [9, -11], [0.5, 2],
          [7.9375, -7.9375], [0.03125, -0.03125], [0.09375, -0.09375], [0.15625, -0.15625],
          [1.0, -1.0], [0.0, -0.0]] + [[(r - 11) * 0.5, 0.0625] for r in range(12, 20)],
         [[10.0, -10.0], [0.375, 0.625], [0.0, 0.0], [1.0, 2.0], [-0.125, 0.125], [3.0, -3.0]] +
         [[0.0, -0.0] for _ in range(14)]),
        # step 3: K amax 1 (no growth at 1/16); V held zeros at scale 0, amax 63.5 -> s = 0.5
        ([[1.0, -0.5], [0.5, 0.25]],
         [[63.5, -1.25], [0.75, -0.25]]),
    ],
    scales={
        (0, "k"): [1.0, 2.0, 2.0],
        (0, "v"): [0.25, 0.25, 0.25],
        (1, "k"): [None, 0.0625, 0.0625],
        (1, "v"): [None, 0.0, 0.5],
    },
    blocks={
        # block 0 K: step 1 codes [127, 0] [0, 2] [2, -2] [-2, 4] [4, -4] .. [9, -9], halved by
        # step 2: 63.5 -> 64, 0, [0, 1], [1, -1], [-1, 2], [2, -2], 2.5 -> 2 / -2.5 -> -2,
        # [3, -3], 3.5 -> 4 / -4, [4, -4], 4.5 -> 4 / -4.5 -> -4; rows 10..15 = run 1 / 2:
        # [127, 0.5 -> 0] [1.5 -> 2, -2] [2.5 -> 2, 3.5 -> 4] [-0.5 -> 0, 0] [4.5 -> 4, -5.5 -> -6]
        # [0.25 -> 0, 1]
        (0, "k"): [[0x40, 0x00], [0x00, 0x01], [0x01, 0xFF], [0xFF, 0x02], [0x02, 0xFE], [0x02, 0xFE],
                   [0x03, 0xFD], [0x04, 0xFC], [0x04, 0xFC], [0x04, 0xFC],
                   [0x7F, 0x00], [0x02, 0xFE], [0x02, 0x04], [0x00, 0x00], [0x04, 0xFA], [0x00, 0x01]],
        # block 1 K (s = 1/16, x 16): [127, -127]; 0.5 -> 0; 1.5 -> 2; 2.5 -> 2; [16, -16];
        # zeros (no signed zero); 8 16 .. 64 with dim 1 = 1; step 3: [16, -8] [8, 4]
        (1, "k"): [[0x7F, 0x81], [0x00, 0x00], [0x02, 0xFE], [0x02, 0xFE], [0x10, 0xF0], [0x00, 0x00],
                   [0x08, 0x01], [0x10, 0x01], [0x18, 0x01], [0x20, 0x01], [0x28, 0x01], [0x30, 0x01],
                   [0x38, 0x01], [0x40, 0x01], [0x10, 0xF8], [0x08, 0x04]],
        # block 0 V (s = 0.25, x 4): [127, 0]; r + 0.5 -> 2 2 4 4 6 6 8 8 10; -r/2 -> 0 -1 -2 -2
        # -2 -3 -4 -4 -4; rows 10..15: [40, -40] [1.5 -> 2, 2.5 -> 2] [0, 0] [4, 8]
        # [-0.5 -> 0, 0.5 -> 0] [12, -12]
        (0, "v"): [[0x7F, 0x00], [0x02, 0x00], [0x02, 0xFF], [0x04, 0xFE], [0x04, 0xFE], [0x06, 0xFE],
                   [0x06, 0xFD], [0x08, 0xFC], [0x08, 0xFC], [0x0A, 0xFC],
                   [0x28, 0xD8], [0x02, 0x02], [0x00, 0x00], [0x04, 0x08], [0x00, 0x00], [0x0C, 0xF4]],
        # block 1 V: zeros at s = 0, unchanged by the growth to 0.5; step 3 (/0.5):
        # [127, -2.5 -> -2] [1.5 -> 2, -0.5 -> 0]
        (1, "v"): [[0x00, 0x00]] * 14 + [[0x7F, 0xFE], [0x02, 0x00]],
    },
)

CASES = {"fp8": FP8, "int8": INT8}
STEP_ROWS = [10, 20, 2]
HEAD_DIM = 64
NUM_BLOCKS = 4
# free list whose pops give blocks 0, 1, 2, 3 in that order (taken from the end)
FREE_ORDER = [3, 2, 1, 0]


def step_rows(case, step):
    """(K, V) rows of one step as float lists [rows][HEAD_DIM] (dims 2.. zero)."""
    k, v = case["inputs"][step]
    assert len(k) == len(v) == STEP_ROWS[step]
    pad = lambda rows: [[float(a), float(b)] + [0.0] * (HEAD_DIM - 2) for a, b in rows]
    return pad(k), pad(v)
