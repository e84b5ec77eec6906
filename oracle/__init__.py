"""CPU oracle for the DeepSeekMoE forward layer with FP8 block scaling.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute anything in this package: only ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code, table
or constant generator with the HIP library in ``fp8_block_scaled_sigmoid_amd``
and never takes an input produced by that library.

Everything here is plain NumPy in float64 (float32 only where the method fixes
a float32 rounding point).  It follows these pages, cited by title and section:

  [VE]  "DeepSeek-V3, explained." (vibeengines.com) -- the numbered recipe
        (step 3: MoE shape, step 4: sigmoid routing and bias, step 7: FP8) and
        the symbol glossary below it.
  [TP]  "DeepSeek-V3: Auxiliary-Loss-Free MoE Load Balancing, Multi-Token
        Prediction, and FP8 Training at 671B Scale" (trishampatil.com) --
        section II (DeepSeekMoE shape), section III (affinity, gate and
        selection equations, the bias thermostat and its flowchart) and
        section V (FP8 mixed precision, Figure 6 and details 1-4).
  [DF]  "DeepSeek-V3 Technical Report" (deepforge.srivtx.xyz) -- part 1
        ("FP8 training, from first principles", "Per-tile FP8 scaling",
        "Balancing without a balance loss") and part 4 "Build it yourself"
        (success criteria).

Modules:
  e4m3     OCP E4M3 codec, written twice (table search and arithmetic).
  quant    1x128 activation and 128x128 weight quantisers.
  route    sigmoid router, biased top-k (plain and group-limited), unbiased gates.
  permute  per-expert counts, offsets and the stable token permutation.
  ffn      block-scaled FP8 GEMM, SwiGLU expert, combine (two precisions).
  bias     sign-based bias update.
  balance  sequence-wise balance statistic (f_i P_i per sequence).
  layer    the whole layer chained from the pieces above.
  backward FP8 input-gradient and weight-gradient GEMMs (token-tile quantiser).

Parity status: every function above is pinned by ``tests/test_oracle_*.py``
against closed forms, brute force, invariants or library special cases; none
is "parity unpinned".
"""
