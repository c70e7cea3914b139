/* Oracle for NF12, the fixed-rate lossless BF16 format (nf12_oracle.c).
 * TEST INFRASTRUCTURE ONLY: the product library never includes it. */
#ifndef NF12_ORACLE_H
#define NF12_ORACLE_H
#include <stdint.h>

#define NF12_ORACLE_OK 0
#define NF12_ORACLE_E_ARG 1
#define NF12_ORACLE_E_FORMAT 2

int oracle_nf12_fits(uint16_t w);
uint32_t oracle_nf12_code(uint16_t w);
uint16_t oracle_nf12_word(uint32_t code);
uint64_t oracle_nf12_bound(uint64_t n);
int oracle_nf12_encode(const uint16_t *w, uint64_t n, uint8_t *out, uint64_t cap, uint64_t *out_bytes);
int oracle_nf12_check(const uint8_t *c, uint64_t bytes);
int oracle_nf12_decode(const uint8_t *c, uint64_t bytes, uint16_t *out, uint64_t n);

#endif
