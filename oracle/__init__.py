"""CPU oracle of the fused int8 convolution path -- test infrastructure only.

Only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg may
import this package.  The GPU library never imports, links or calls it.
"""
