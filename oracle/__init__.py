"""CPU oracle for one rank's share of context-parallel diffusion attention.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import anything from this package.  The
library under ``context_attention_diffusion_amd`` never imports it and shares no
code with it; the two meet only through the seeded inputs of ``workloads.py``.

Plain numpy, float64 for floating point, bf16 carried as uint16 bit patterns:

* ``oracle.bf16``      -- exact bf16 <-> float64 widening (and RNE narrowing for reports);
* ``oracle.layout``    -- Ulysses pack / chunk exchange / unpack / output reverse,
                          each as a reshape-transpose definition and as explicit loops;
* ``oracle.attention`` -- softmax(scale * Q K^T) V with an optional key-validity mask;
* ``oracle.cp_share``  -- the AllGather-KV and 2D (Ulysses x AllGather-KV) rank layouts
                          composed from the above, for end-to-end invariants.
* ``oracle.varlen``    -- packed variable-length attention: the per-rank remap of the
                          packed query boundaries and per-document attention.

Sources, cited by page title and section:

* [sglang#33667] prhub summary of sglang PR #33667, "pack the Ulysses QKV
  all-to-all into one collective and reuse staging buffers": sections
  "Implementation breakdown" and "Key source snippets" (usp.py and
  test_usp_packed_qkv_a2a.py excerpts).
* [vllm-omni#7641] vllm-omni PR #7641, "[Feature] Compose Ulysses with
  AllGather-KV as a 2D diffusion SP": commit message and review-fix commits.
* [chitu-fastcp] ChituDiffusion docs, "Install and enable Fast CP", section
  "Support scope".

Every function is pinned by a test under ``tests/`` marked ``not gpu``; there is
no function here with "parity unpinned".
"""
