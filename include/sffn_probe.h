/* Device-rate probes (libsffn_probe.so): the measured ceilings that bound
 * the bf16 MFMA GEMMs of libsffn.so on gfx950. Not part of the layer's
 * boundary (include/sffn.h); bench.py reports the rates beside the GEMM
 * rooflines.
 */
#ifndef SFFN_PROBE_H
#define SFFN_PROBE_H

#ifdef __cplusplus
extern "C" {
#endif

/* Measure, on the current HIP device with `num_cu` compute units, in bytes
 * per second per compute unit:
 *   out[0]  LDS: 16-byte fragment reads (ds_read_b128) alone;
 *   out[1]  LDS: 16-byte direct-to-LDS copies (global_load_lds_dwordx4)
 *           from an L2-resident source, alone;
 *   out[2]  both kinds issued together, the two summed;
 *   out[3]  16-byte L2-to-register loads, four lanes per 64-byte row piece;
 *   out[4]  the same bytes loaded in the 32 x 32 MFMA operand layout
 *           (lane l: row l % 32, 16-byte piece l / 32).
 * Two workgroups of 4 waves per CU for the LDS probes, eight for the loads;
 * each rate is one launch timed with HIP events after two warm-up launches.
 * `out` is host memory of at least 5 doubles (n_out >= 5); the probe
 * allocates and frees 32 MiB of device memory and synchronises the device.
 * Returns 0, hipErrorInvalidValue for bad arguments, or the HIP error of
 * the first failing call (out is then unspecified). */
int sffn_probe_rates(int num_cu, double* out, int n_out);

#ifdef __cplusplus
}
#endif

#endif /* SFFN_PROBE_H */
