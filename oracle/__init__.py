"""fp64 CPU oracle of the fused multi-head attention forward and backward passes.

TEST INFRASTRUCTURE, NOT PART OF THE PRODUCT.  Only ``tests/``,
``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` may
import or run anything in this package.  It shares no code with the HIP path
(no kernels, headers, helpers, tables or constants); both take their inputs
from the separate ``workloads`` generator, which holds none of the attention
arithmetic.

Pins (tests/test_oracle.py, run with ``-m "not gpu"``):

* format decoders: every code of bf16, fp16 and e4m3fn against torch/numpy casts,
  plus values fixed by the format definitions;
* brute force: pure-Python loops over tiny problems, written as the direct
  softmax quotient without the max shift, every mask, GQA and packed batches;
* library routine: torch's CPU ``scaled_dot_product_attention`` in fp64 for the
  no-mask, top-left causal and explicit-mask cases;
* closed forms: one key gives O = V[0]; constant V rows give that row; causal
  row 0 gives V[0]; Q = 0 or Q = K = ones give uniform weights with known LSE;
* invariants: rows of P sum to 1, sum_j exp(S_ij - LSE_i) = 1, K/V at masked
  positions do not change O (bit-identical), key permutation invariance,
  packed batch == per-sequence runs, GQA == MHA with repeated K/V heads,
  causal-qend == causal-qbegin when Sq == Sk;
* planted mistakes in a copy of the oracle (off-by-one diagonal, flipped qend
  offset, wrong GQA head, missing scale, transposed operand) fail the pins;
* the FLOP convention reproduces the TFLOP/s column printed by the sm120 article.

Backward pins (tests/test_oracle_backward.py): torch autograd through a materialised fp64
attention and through torch's scaled_dot_product_attention (GQA batches, every mask); central
finite differences of the forward oracle; closed forms (one key: dQ = dK = 0 and dV = sum of
dO; Q = 0: uniform weights); invariants (sum of dK over the keys is 0, sum of dV equals the
sum of dO over rows with a key, unseen keys get no gradient, linearity in dO, sum_d O dO =
sum_j P dP, GQA == MHA on repeated heads summed, packed == per-sequence); planted mistakes
(dropped or sign-flipped softmax term, untransposed operands, missing or doubled scale, dP
from K, GQA overwrite or wrong head, varlen key offset) fail the pins.  The row-block form
for sequences too long to hold S (attention_head_backward_rows) is pinned against autograd
directly at several block sizes and on rows that see no key; its planted mistakes (dropped
softmax term, dV from dS, dQ row off by one, block mask taken from row 0, dK without the
scale) fail the pins too.  delta taken from a given O (the ``o`` argument, for an O stored in a
coarse type such as e4m3) is pinned against autograd with the exact O and against the closed
form of a perturbed O (dQ and dK shift by the changed delta times P K and P^T Q, dV does not),
through the single-head, dense GQA and packed forms; planted mistakes (the given O ignored,
delta without dO, the K/V head's O, O at the key rows) fail the pins.

Paged-cache pins (tests/test_oracle_paged.py): brute force with per-key page arithmetic and
the plain softmax quotient; the dense forward oracle on a cache laid out in order; invariance
under relabelling the physical pages; NaN in memory no sequence owns changes nothing; the empty
sequence; planted mistakes (page index off by one, whole last page kept, table order ignored,
wrong GQA head) fail the pins.

No function is "parity unpinned" except the two choices the pages leave open:
rows with no visible key (O = 0, LSE = -inf) and fp8 saturation at +-448, which
are pinned only by those stated choices.
"""
from .attention import (  # noqa: F401
    MASKS,
    attention_dense,
    attention_head,
    attention_rows,
    attention_varlen,
    visible_keys,
)
from .formats import decode, decode_minifloat  # noqa: F401
from .backward import (  # noqa: F401
    attention_backward_dense,
    attention_backward_varlen,
    attention_head_backward,
    attention_head_backward_rows,
    sum_o_do,
)
from .paged import append_paged, attention_paged, gather_pages  # noqa: F401
