"""Quantized gated delta-rule decode step for AMD MI355X (gfx950).

The compute path is the in-tree HIP library ``libstq.so`` (C ABI declared in
``include/stq.h``); ``linear_attention_recurrent_rule_amd.stq`` is its thin
ctypes binding.  ``workloads`` holds the seeded synthetic inputs."""
