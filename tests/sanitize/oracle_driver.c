/* Sanitizer driver for the C oracles (df11_oracle.c, nf12_oracle.c), built
 * with gcc -fsanitize=address,undefined on the CPU.  Manifest lines
 * "<kind> <path>":
 *   words <16-bit words>  encode, check and decode both formats; the decoded
 *                         words must equal the input
 *   df11  <container>     oracle_check on the file and on prefixes (status only)
 *   nf12  <container>     oracle_nf12_check on the file and on prefixes
 * Memory errors and undefined behaviour abort with the sanitizer's report; a
 * wrong round trip exits 3. */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "df11_oracle.h"
#include "nf12_oracle.h"

static uint8_t *read_file(const char *path, size_t *n) {
    FILE *f = fopen(path, "rb");
    if (!f) exit(2);
    fseek(f, 0, SEEK_END);
    long sz = ftell(f);
    fseek(f, 0, SEEK_SET);
    uint8_t *b = (uint8_t *)malloc(sz > 0 ? (size_t)sz : 1);
    if (!b || (sz > 0 && fread(b, 1, (size_t)sz, f) != (size_t)sz)) exit(2);
    fclose(f);
    *n = (size_t)sz;
    return b;
}

static void prefixes(const uint8_t *c, size_t n, int nf12) {
    size_t cuts[] = {0, 1, 16, 255, 256, 511, 512, 1024, n / 3, n / 2, n ? n - 1 : 0, n};
    for (size_t k = 0; k < sizeof cuts / sizeof cuts[0]; ++k) {
        size_t m = cuts[k];
        if (m > n) continue;
        uint8_t *p = (uint8_t *)malloc(m ? m : 1);
        if (m) memcpy(p, c, m);
        if (nf12)
            (void)oracle_nf12_check(p, m);
        else
            (void)oracle_check(p, m);
        free(p);
    }
}

static int check_words(const char *path) {
    size_t bytes;
    uint8_t *raw = read_file(path, &bytes);
    uint64_t n = bytes / 2;
    uint16_t *w = (uint16_t *)malloc(n ? 2 * n : 2);
    if (n) memcpy(w, raw, 2 * n);
    uint64_t dims[1] = {n};
    uint64_t cap = oracle_container_bound(n), got = 0;
    uint8_t *c = (uint8_t *)malloc(cap);
    uint16_t *d = (uint16_t *)malloc(n ? 2 * n : 2);
    int r = 0;
    if (oracle_encode_flags(w, n, 1, dims, ORACLE_FLAG_SHA256, c, cap, &got) != ORACLE_OK) r = 3;
    if (!r && oracle_check(c, got) != ORACLE_OK) r = 3;
    if (!r && oracle_decode(c, got, d, n) != ORACLE_OK) r = 3;
    if (!r && n && memcmp(d, w, 2 * n) != 0) r = 3;
    free(c);
    uint64_t ncap = oracle_nf12_bound(n);
    uint8_t *f = (uint8_t *)malloc(ncap ? ncap : 1);
    if (!r && oracle_nf12_encode(w, n, f, ncap, &got) != NF12_ORACLE_OK) r = 3;
    if (!r && oracle_nf12_check(f, got) != NF12_ORACLE_OK) r = 3;
    memset(d, 0, n ? 2 * n : 2);
    if (!r && oracle_nf12_decode(f, got, d, n) != NF12_ORACLE_OK) r = 3;
    if (!r && n && memcmp(d, w, 2 * n) != 0) r = 3;
    free(f);
    free(d);
    free(w);
    free(raw);
    return r;
}

int main(int argc, char **argv) {
    if (argc != 2) return 2;
    FILE *m = fopen(argv[1], "r");
    if (!m) return 2;
    char kind[16], path[4096];
    long counts[3] = {0, 0, 0};
    while (fscanf(m, "%15s %4095s", kind, path) == 2) {
        if (!strcmp(kind, "words")) {
            int r = check_words(path);
            if (r) {
                fprintf(stderr, "words %s: status %d\n", path, r);
                return r;
            }
            ++counts[0];
        } else if (!strcmp(kind, "df11") || !strcmp(kind, "nf12")) {
            size_t n;
            uint8_t *c = read_file(path, &n);
            prefixes(c, n, kind[0] == 'n');
            free(c);
            ++counts[kind[0] == 'n' ? 2 : 1];
        } else if (strcmp(kind, "slots") != 0 && strcmp(kind, "luts") != 0) {   /* (the host driver's own checks) */
            return 2;
        }
    }
    fclose(m);
    printf("ok: %ld word files, %ld df11, %ld nf12\n", counts[0], counts[1], counts[2]);
    return 0;
}
