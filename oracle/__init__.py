"""Oracle: a plain, slow CPU implementation of one GPipe pipeline cell's training step.

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the bench's
CPU-baseline leg may import or call anything here; the library's product
path never does, and shares no code, header, table or helper with it.

Sources: the GPipe technical review page (zzz0906.github.io, "GPipe：微批次流水线并行
的大规模模型训练 — 深度技术评审"), sections "GPipe algorithm in detail" (interface,
pipeline execution flow phases 1-3, BatchNorm handling) and preliminaries 2
(memory wall: RMSProp state) and 5 (re-materialization).

Modules
  transformer_cell  pre-LN Transformer cell: forward, backward, MSE loss,
                    micro-batched step with and without re-materialization,
                    RMSProp update
  partition         exhaustive minimum-variance contiguous partition
  conv_cell         conv + micro-batch BatchNorm cell

Pins (tests/test_oracle_*.py) tie every function to something other than
itself: torch's own TransformerEncoderLayer and RMSprop, finite differences,
closed forms and the pages' invariants.
"""
