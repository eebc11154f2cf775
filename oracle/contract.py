"""Constants of the attention contract the oracle checks against.

P modes (where the softmax weights are rounded before they multiply V):
  P_FP32    no rounding (decode: "fp32 accumulate", partials per 256-key chunk)
  P_BF16    P = bf16(p)                      (sliding-layer prompt tiles)
  P_BF16X2  P = bf16(p) + bf16(p - bf16(p))  (PR #1183 commit bodies,
            the window_rows note keeps P to 16 significant bits in two bf16
            halves)

Key block KB: in prompt tiles the softmax keeps a running row maximum that is
updated once per block of KB keys, blocks aligned to absolute key positions
(key j is in block j // KB), and P is rounded against the running maximum of
its own block.  Which maximum P is rounded against changes the rounded value,
so KB is part of the contract: the pages fix the online softmax per block
(PR #975: row maxima and probabilities are exchanged once per key
block) but not its size.
This library's kernels use the sizes below; its C-ABI reports them through
attn_prefill_key_block(), and the tests check that both agree.

Error radius (the range fp32 allows, after PR #1183's attention_range note):
  EPS_P bounds the relative error of a kernel's p before its rounding point.
  The fp32 score of a D-term bf16 dot product accumulated in fp32 blocks is
  off by a few 2^-24 of sum |q k| * scale (about 2^-18 of p at D=512 with
  N(0,1) data), the scale product and exp2 add about 2^-23 each, and a
  decode kernel that carries p as two bf16 halves (16 significant bits, the
  pages' 16-bit P) adds up to 2^-16.  EPS_P = 2^-16 covers all of these.
  EPS_ACC bounds the fp32 accumulation of P*V and of the row sum, relative to
  the sum of absolute terms: sequential fp32 sums over up to 2^10 key blocks
  grow like sqrt(blocks) * 2^-24, about 2^-19; EPS_ACC = 2^-18.
  Both stay far below a bf16 step (2^-8), so every planted control of the
  tests is still refused.
"""

P_FP32, P_BF16, P_BF16X2 = 0, 1, 2

DECODE_CHUNK = 256                 # slots per decode partial (window_rows note)

PREFILL_KEY_BLOCK = {              # (head_dim, p_mode) -> KB
    (256, P_BF16): 64,
    (256, P_BF16X2): 64,
    (512, P_BF16): 32,
    (512, P_BF16X2): 32,
}

EPS_P = 2.0 ** -16
EPS_ACC = 2.0 ** -18
ULP_SLACK = 1                      # ordered-bits steps allowed past the range
MEAN_REL_ERR_MAX = 1e-3


def key_block(head_dim: int, p_mode: int) -> int:
    return PREFILL_KEY_BLOCK[(head_dim, p_mode)]
