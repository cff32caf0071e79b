"""CPU oracle for the InfLLM v2 hot path (test infrastructure only).

Only tests/, the smoke check and the bench's CPU-baseline leg may import this
package.  ``infv2_ref`` is the step-by-step float64 oracle; ``dense_ref`` is an
independent dense / sink-plus-window attention; ``brute`` re-derives every
definition with pure-Python loops on tiny inputs.  ``dense_ref`` and ``brute``
do not import ``infv2_ref``.
"""
