"""CPU oracle for one GPU's share of the deterministic fused MoE layer.

TEST INFRASTRUCTURE ONLY. Nothing in the product path imports, calls or links this package:
only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` use
it. It shares no code with the HIP path (no kernels, headers, helpers, tables or constants);
the two meet only in the seeded arrays that ``datagen`` returns.

The oracle is written from three pages about the "Mixture-of-Kittens (MoK)" MoE training
megakernel:

* "Mixture-of-Kittens (MoK)" (wiki summary page);
* "Cursor Open-Sources Mixture-of-Kittens (MoK): A Deterministic MoE Training Megakernel for
  GB300 NVL72 Racks" (digest page);
* "把 MoE 通信延迟从 103μs 压到 18μs：Cursor 开源 GPU 内核 MoK" (explainer page).

Citations in the modules name the page by (a prefix of) its title and the section.

Modules:

* ``moe_oracle``  forward and backward of the layer in fp64 (numpy), step by step in the
  order the pages describe: router top-k, schedule table, pull dispatch, grouped SwiGLU
  expert FFN, push combine and final weighted merge; backward with the router-weight
  gradient taken inside SwiGLU backward.
* ``mx``          the MXFP8 (E4M3 + UE8M0, 32-element blocks) quantiser, from the OCP
  Microscaling Formats v1.0 definition.
* ``brute``       pure-Python loops over the same definitions, for tiny shapes only; it
  pins ``moe_oracle``.
"""
