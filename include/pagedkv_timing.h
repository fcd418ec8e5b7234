/* Per-wave timing of the shared-prefix decode's stage 1, for measurement.
 *
 * Exported only by libpagedkv_timing.so, a second build of the library whose
 * shared-prefix stage-1 kernel ("PagedAttention and vLLM Architecture",
 * section 3: forked sequences reading their common prompt blocks) also
 * records, per wave, the device real-time counter (100 MHz) at entry, when
 * its stream of chunks starts and when its last piece is queued, plus its
 * share of chunks and its workgroup id.  libpagedkv.so has no such code: the
 * recording is compiled in only with PKV_WAVE_TIMING.  Every other entry point
 * of the timing build behaves as declared in pagedkv.h.
 */
#ifndef PAGEDKV_TIMING_H
#define PAGEDKV_TIMING_H

#ifdef __cplusplus
extern "C" {
#endif

/* Copies the records of waves 0 .. n_waves - 1 of the most recent stage-1
 * launches into host memory and clears them on the device.
 *   host     host buffer of n_waves * 4 unsigned 64-bit words, owned by the
 *            caller; record w is words 4w .. 4w + 3: entry, stream start,
 *            end, (share chunks << 32) | workgroup id.  A wave that got no
 *            share (or a wave id the launch did not have) reads as zeros.
 *   n_waves  0 .. 8192.
 * Returns 0; -2 for a null buffer or n_waves out of range; -6 when a HIP copy
 * fails.  Synchronous with respect to the host; call it after the stage-1
 * launch has completed. */
int pkv_wave_timing_read(unsigned long long* host, int n_waves);

#ifdef __cplusplus
}
#endif

#endif /* PAGEDKV_TIMING_H */
