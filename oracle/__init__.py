"""CPU oracle for tree-verification attention -- TEST INFRASTRUCTURE ONLY.

This package is the plain, slow, obviously-correct statement of what the tree-verify
path computes.  It exists so that tests, the smoke check and the benchmark's CPU
baseline can check the HIP library against it.  Nothing on the product path may import,
call or link anything under ``oracle/``; the product path has no CPU fallback.

It shares no code, tables, headers or helpers with the HIP path
(``tree_attention_draft_amd``) and imports nothing from it.

Modules
-------
``meta``   pure-Python integer metadata: rank paths -> parent, depth, ancestor mask,
           bitmask, position ids; and the same from a parent array.
``attn``   fp64 numpy tree attention: masked softmax over the full step mask
           (whole prefix plus the node's ancestors and itself), natural-log LSE.
``brute``  per-node brute force: ordinary causal attention over the node's exact
           root path, through ``torch.nn.functional.scaled_dot_product_attention``
           in float64 on the CPU (an independent library routine).
``accept`` after the pass: the target's greedy token per node (argmax), the greedy walk
           down the tree, and the compaction of the accepted path's KV rows.

Sources (the pages the method is described on):
  [TAM]  "Tree attention mask for draft-tree verification" (inferenceinterviews.com),
         sections "TL;DR", "A strong answer", "Common mistakes".
  [TV]   "Tree Verification" (stable-lab specdec notes), section "Tree Attention".
  [EBH]  "Encode branch histories in masks and positions"
         (study.greatitself.com, speculative tree verification layouts).
  [TV] also "Accepting on a Tree" and "The Cost Side"; [TAM] also "What it costs".

Pinning status: every function here is pinned by tests under ``tests/`` (printed mask
rows and expected-token sums of the worked example, the empty tree, the missing-parent
rejection, exhaustive brute force on all trees of up to 6 nodes with repeated token
labels and rotary positions, closed forms and invariants; for ``accept``: the worked
example's walks, its expected tokens per step by exact enumeration, an independent
per-node rule, and the compacted cache reproducing the tree output).  The only unpinned items are
conventions the pages do not fix: natural-log LSE, LSB-first bit order of the bitmask,
the GQA head map h -> h // (Hq/Hkv), softmax scale 1/sqrt(D), round-to-nearest-even
for bf16 outputs.  Those are "parity unpinned" conventions shared with the HIP path
as written specification only.
"""
