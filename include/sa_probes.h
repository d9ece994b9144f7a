/*
 * sa_probes.h -- calibration micro-benchmarks for MI355X (gfx950), used by
 * the benchmark to state the measured ceilings its roofline figures are read
 * against.  Not part of the attention path.  Each call launches its kernels
 * on the null stream, waits for them and returns the measured rates; it
 * allocates and frees its own device buffers.  Returns 0, or a negative
 * HIP-related status (-4) when a HIP call fails.
 */
#ifndef SA_PROBES_H
#define SA_PROBES_H

#ifdef __cplusplus
extern "C" {
#endif

typedef struct {
  double mfma_bf16_tflops;     /* back-to-back v_mfma_f32_32x32x16_bf16, 4 waves per SIMD */
  double shader_clock_ghz;     /* shader clock during that loop (cycle counter vs real-time clock) */
  double mfma_cycles;          /* cycles one 32x32x16 bf16 MFMA occupies its SIMD (from the above) */
  double fma_cycles;           /* cycles per wave64 v_fma_f32 per SIMD, independent chains */
  double exp_cycles;           /* cycles per wave64 v_exp_f32 per SIMD, independent chains */
  double lds_b128_cycles;      /* cycles per ds_read_b128 instruction per CU (all waves of the CU) */
  double lds_tr_b64_cycles;    /* cycles per ds_read_b64_tr_b16 instruction per CU */
  double atomic_f32_tbs;       /* fp32 global atomic adds (no return) into 50 MB, TB/s of updates */
  double store_f32_tbs;        /* plain stores of the same pattern, TB/s */
} sa_probe_results;

int sa_probe_run(sa_probe_results* out);

#ifdef __cplusplus
}
#endif

#endif /* SA_PROBES_H */
