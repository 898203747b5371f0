"""fp64 CPU oracle for exact tiled attention.

TEST INFRASTRUCTURE: only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s
``cpu_baseline`` leg may import this package. The HIP library and its binding
(``exact_attention_27_amd``) never import it and share no code with it.

``oracle.attention`` is the plain definition (materialises S and P in float64);
``oracle.online`` is the blocked online-softmax recurrence, used only to pin the
oracle through the pages' block-invariance claims and worked examples.
"""
from . import attention, online  # noqa: F401
