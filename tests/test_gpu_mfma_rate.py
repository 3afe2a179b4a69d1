"""Sustained rates of the matrix instructions the GEMMs use, and the shader
clock while they run (test instrument in tests/mfma_probe/rate_probe.hip).

These facts bound the per-tile FP8 GEMM.  A per-tile scale product changes
every 32-wide K block ("Why grind FP8 GEMM on CDNA4", section 3.3), so each
block's partial sum must be kept apart and promoted in FP32 (section 3.2).
Only the K = 16 FP8 instruction (two per block) and the 16 x 16 x 32 one (one
per block) keep a block's sum apart; the K = 64 block-scaled instruction sums
two blocks whose scale products are unrelated FP32 numbers.  The tests check
the relations the design rests on and print the measured figures:

* the K = 16 FP8 instruction sustains about half the FLOP rate of the K = 64
  block-scaled one on the same data;
* the per-block promotion pattern (two K = 16 instructions and 16 FP32 FMAs
  per lane per 32 x 32 tile) runs no faster than the bare K = 16 rate;
* the shader clock under sustained matrix load, from each wave's s_memtime /
  s_memrealtime, lies in a plausible range (it is below the 2.4 GHz that the
  peak figures assume on random data).
"""
import pytest

from gpu_common import say

pytestmark = pytest.mark.gpu


def _rate(instr, pattern, data, wps=2, seconds=0.03):
    import mfma_probe as mp
    cyc = {mp.R_FP8_K16: 32, mp.R_SCALE_FP8_K64: 64, mp.R_SCALE_FP4_K64: 32,
           mp.R_BF16_K16: 32, mp.R_FP8_16X16X32: 16}[instr]
    per_iter = cyc * (4 if pattern == mp.P_CHAINS else
                      {mp.R_FP8_K16: 8, mp.R_BF16_K16: 8, mp.R_FP8_16X16X32: 16}.get(instr, 4))
    iters = int(seconds * 2.4e9 / (per_iter * wps))
    say(f"rate probe: {mp.RATE_NAMES[instr]}, {mp.PATTERN_NAMES[pattern]}, {data}, "
        f"{wps} waves/SIMD, {iters} iterations")
    r = mp.rate(instr, pattern, data, waves_per_simd=wps, iters=iters)
    say(f"  -> {r['tflops']} TFLOP/s, sclk {r['sclk_ghz']} GHz, "
        f"{r['shader_cycles_per_instr_per_simd']} shader cycles per instruction per SIMD")
    return r


def test_k16_fp8_is_half_rate_of_k64_block_scaled():
    import mfma_probe as mp
    k16 = _rate(mp.R_FP8_K16, mp.P_CHAINS, "random")
    k64 = _rate(mp.R_SCALE_FP8_K64, mp.P_CHAINS, "random")
    assert k16["tflops"] > 0 and k64["tflops"] > 0
    # cycles per instruction: K = 16 takes at least half the time of K = 64
    # while doing a quarter of the work
    assert k16["tflops"] < 0.75 * k64["tflops"], (k16, k64)


def test_promotion_pattern_no_faster_than_k16():
    import mfma_probe as mp
    bare = _rate(mp.R_FP8_K16, mp.P_CHAINS, "random")
    prom = _rate(mp.R_FP8_K16, mp.P_PROMOTE, "random")
    assert prom["tflops"] <= 1.05 * bare["tflops"], (bare, prom)


def test_shader_clock_plausible_under_load():
    import mfma_probe as mp
    r = _rate(mp.R_SCALE_FP8_K64, mp.P_CHAINS, "random", seconds=0.1)
    assert 0.3 < r["sclk_ghz"] < 3.0, r
    z = _rate(mp.R_SCALE_FP8_K64, mp.P_CHAINS, "zero", seconds=0.1)
    assert 0.3 < z["sclk_ghz"] < 3.0, z
