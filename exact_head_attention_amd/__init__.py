"""MI355X-native exact per-head attention for MiniMax-H3's Ulysses ranks.

The compute path is the HIP library ``libh3attn.so`` (built for gfx950) behind
a C ABI; ``binding`` marshals PyTorch device tensors into it.  ``inputs`` holds
the seeded synthetic workloads.
"""
