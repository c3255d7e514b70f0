"""CPU oracle for exact tiled attention -- TEST INFRASTRUCTURE ONLY.

Plain, slow, float64 numpy implementations of what the GPU library computes.  It
shares no code with the HIP path and the HIP path never imports it: only the
tests, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py``
may import or run anything in this package.

Sources (page titles of the reference text):
  [IO]   "M4.3 - IO-Aware Attention and FlashAttention-1: Online Softmax, Tiling,
          and Exactness"
  [FA2]  "M4.4 - FlashAttention-2 Work Partitioning and the Decode Boundary"
  [HW]   "M4.6 - FlashAttention-3/4 Hardware Pipelines: Hopper, Blackwell, and
          the Moving Bottleneck"

Modules:
  dense   -- the dense definition (forward, LSE, backward, decode), its
             packed variable-length form and the paged-cache decode       [pinned]
  state   -- the online (m, l, u, n) state algebra and its merges     [pinned]
  fp8     -- the E4M3FN codebook, the quantised forward steps and the
             backward on E4M3 operands                               [pinned: the
             codebook, hand-derived cases of each rounding step, the reduction to
             the dense definition without the rounding, the backward's reduction to
             the dense exact gradient]
  tiles   -- causal tile classes, visit counts, packed-launch census  [pinned]
  dropout -- Philox4x32-10 keep decisions by element coordinates, the dropout
             forward and its backward                              [pinned]
  exp2soft -- the software exp2 (range reduction, degree-3 relative minimax
             polynomial fitted by the Remez exchange), float32 emulation [pinned]
"""
