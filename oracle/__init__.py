"""fp64 CPU oracle for Lightning Attention prefill and decode.

TEST INFRASTRUCTURE ONLY.  This package is the slow, obviously-correct
reference that the HIP kernels are checked against.  Only the test suite,
the smoke check in ``__graft_entry__`` and the ``cpu_baseline`` leg of
``bench.py`` may import it.  The product path (``linear_attention_la_amd``)
never imports, calls or links anything here, and nothing here imports the
product path: the two share no code.  The only module both sides use is
``la_inputs``, which draws seeded inputs and holds none of the method's
arithmetic.

Sources (web pages on MiniMax-01; cited by title and section):

* [EMZ]  emonzhong.com, "MiniMax-01: Scaling Foundation Models with
  Lightning Attention" -- section 方法要点 (method).
* [CSDN] CSDN, "【AI论文】MiniMax-01:利用闪电注意力机制扩展基础模型" --
  §2.1 (MiniMax-Text-01 architecture), §3.2 (computation optimisation).
* [JVY]  jvyan.cn news article on MiniMax-01 -- 一、模型架构 (architecture),
  二、计算优化 (computation optimisation).
* [MZK]  mizuki blog, "MiniMax-01：4M 上下文破局" -- 三 (why 7 linear + 1
  softmax), 附/关键概念清单 (glossary).

Every function states which passage it follows.  Where the pages leave a
step open the reading taken is stated in the function's docstring.

Pins: every function here is pinned by ``tests/test_oracle_pins.py`` to
facts that do not come from this package (brute force on tiny inputs,
exact rational arithmetic, closed forms, ``scipy.signal.lfilter`` and plain
matrix products for the no-decay special case, hand-worked golden values).
"""

from .lightning import (  # noqa: F401
    decay_mask,
    quadratic,
    quadratic_loops,
    recurrent,
    blockwise,
    decode_step,
    prefill_varlen,
    prefill_pool,
    decode_batch,
    decode_pool,
    backward_quadratic,
    backward_recurrent,
    backward_varlen,
    norm_gate,
)
