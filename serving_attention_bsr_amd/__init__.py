"""MI355X-native attention over a block-sparse-row (paged) KV cache.

The compute path is the HIP library ``libbsr_attn.so`` built from ``csrc/``;
``serving_attention_bsr_amd.lib`` is its thin ctypes binding.  Importing this
package loads nothing; ``workloads`` builds seeded synthetic inputs.
"""

__all__ = ["lib", "workloads"]
