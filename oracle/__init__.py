"""CPU oracle for packed attention over a rollout DAG.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute anything in this package; only the test-suite, the smoke check and the
benchmark's CPU-baseline leg use it.  It shares no code, tables or helpers with
the HIP library: it rebuilds positions and visibility from the raw node and
mount tables itself, in plain Python/NumPy, in float64 unless a caller asks for
float32.

What it computes (the plain definition that the packed method reaches up to
rounding order):

* ``dag``       -- node validation, start positions (Octopus Eq. 2), active
                   mounts with their transitive closure, visible sets, the
                   root-to-leaf trajectories with mounted spans spliced in, and
                   each node's owning leaf (Octopus Eq. 6).
* ``rope``      -- the rotary phase of Octopus Eq. 1.
* ``attention`` -- four independent evaluations of attention over the DAG:
                   brute force (explicit loops), flat per-trajectory dense causal
                   attention (the reference), a dense packed mask, and per-row /
                   per-key evaluations for sampling large inputs.
* ``gdn``       -- the gated delta rule over the same tree as a plain token
                   recurrence per root-to-leaf trajectory (mounted spans
                   skipped), with back-propagation through time.
* ``gdn_plan``  -- HARTS's minimum-call planning of chunked linear-attention
                   execution: segment tree, T_pre / T_in, the recovery of
                   rounds, mandatory replay, and a brute-force minimum.
* ``logprob``   -- compact-to-semantic log-probabilities (HARTS Eq. 17) on
                   expanded per-position rows, the semantic position map of
                   the original batch, and the reused-row gradient (Eq. 19-20).
* ``harts_plan`` -- HARTS's prefix-aware microbatch planning over raw
                   trajectories: compact work (Eq. 5-6), natural partition,
                   K range, exact DP, sampled-K evolution, trie-aware greedy
                   with Eq. 10, repair and refinement, replica/slot assignment.
* ``conv``      -- the short causal convolution of a linear-attention block
                   along each trajectory's own tokens (mounted spans skipped),
                   one output per compact token, gradients summed over readers.

Parity unpinned: the RoPE pairing convention (first half / second half of the
head dimension) and the frequency base (10000) are a textbook choice the pages
do not fix; both sides take them as parameters.  Likewise the gated delta
rule's parameterisation and its output scale (default 1): the pages name the
layer but print no recurrence for it.  And the short convolution's activation
(identity or SiLU, a parameter) and tap order.
"""
