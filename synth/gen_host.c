/* gen_host.c -- host build of the synthetic expert-blob generator
 * (synth_common.h).  Built with gcc -ffp-contract=off so that every fp32
 * operation is rounded on its own, as on the device. */
#include <stddef.h>
#include <stdint.h>

#include "synth_common.h"

/* Number of 32-bit words in one blob. */
uint64_t synth_blob_words(int32_t H, int32_t I, int32_t bits) {
  uint64_t off[7];
  return synth_layout(H, I, bits, off);
}

/* Writes the blob of (layer, expert) to out (host memory, blob_words words). */
void synth_gen_blob_host(const synth_params *p, uint32_t layer, uint32_t expert,
                         uint32_t *out) {
  uint64_t off[7];
  uint64_t n = synth_layout(p->H, p->I, p->bits, off);
  uint64_t key = synth_key(p->seed, layer, expert);
  for (uint64_t i = 0; i < n; ++i) out[i] = synth_blob_word(p, key, off, i);
}

/* Writes words [w0, w0 + n) of the blob of (layer, expert) to out. */
void synth_gen_words_host(const synth_params *p, uint32_t layer, uint32_t expert,
                          uint64_t w0, uint64_t n, uint32_t *out) {
  uint64_t off[7];
  synth_layout(p->H, p->I, p->bits, off);
  uint64_t key = synth_key(p->seed, layer, expert);
  for (uint64_t i = 0; i < n; ++i) out[i] = synth_blob_word(p, key, off, w0 + i);
}
