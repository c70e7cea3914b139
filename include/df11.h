/*
 * df11 -- lossless BF16 weight decompression on AMD Instinct MI355X (gfx950).
 *
 * C ABI of libdf11.so.  No C++ or torch types cross it: plain pointers
 * (host or device, as each argument says), sizes, and a hipStream_t.
 *
 * The method (mlx-dfloat project page, introduction and its 16-bit weight
 * diagram; df11pack project page, introduction): every BF16 weight keeps its
 * sign and 7-bit fraction as one raw byte, and its 8-bit exponent is replaced
 * by a variable-length prefix code; decoding gives back each weight bit for
 * bit.  The weights stay compressed in GPU memory and are decoded on the GPU
 * when they are needed (mlx-dfloat project page, introduction).
 *
 * Container version 4 (one tensor = one container = one code table; all
 * integers little-endian; every section starts on a 256-byte boundary):
 *
 *   header (512 bytes)
 *      0 char[8] magic "DF11HIPC"    8 u32 version = 4      12 u32 flags
 *     16 u64 n_elems                24 u32 ndim            28 u32 chunk_elems = 32768
 *     32 u64 dims[8]                96 u8 max_code_len = 24 97 u8 0
 *     98 u16 windows = 512         100 u32 n_chunks       104 u64 total_bits
 *    112 u64 off_chunk_index       120 u64 off_windows    128 u64 0
 *    136 u64 off_stream            144 u64 stream_bytes   152 u64 off_raw
 *    160 u64 raw_bytes             168 u64 total_bytes    176 u8 sha256[32]
 *    208 u8 code_len[256]          464 u8[48] 0
 *   chunk index  (n_chunks + 1) x { u64 start_bit, u64 out_elem }; the last
 *                entry is { total_bits, n_elems }
 *   windows      n_chunks x 512 x u16: cnt | (gap << 11)
 *   stream       the exponent codes, concatenated, most significant bit first
 *                (bit 7 of byte 0 is the first bit); ceil(total_bits/8) bytes
 *                rounded up to 16, plus 16 zero bytes
 *   raw          one byte per element: (sign << 7) | fraction; n_elems bytes
 *                rounded up to 16
 *   flags: bit 0 (DF11_FLAG_SHA256) set = sha256 is the SHA-256 (FIPS 180-4)
 *   of the source tensor's bytes, each word least significant byte first
 *   (df11pack page, "Beyond the official format": a per-tensor SHA-256 in the
 *   header lets a verify find corruption without the source; the other
 *   sections are the same with or without it); clear = sha256 is zero.
 *   Bytes not named above are zero.
 *
 * Code: code_len[e] is the length of the code of exponent byte e (0 = absent),
 * at most 24 bits.  Code values are canonical: symbols sorted by (length,
 * symbol) get consecutive values, the first is 0 (the deflate construction).
 *
 * Chunks: element j of the tensor is in chunk j / 32768.  Chunk c owns the
 * stream bits [b0, b1) = [start_bit[c], start_bit[c+1]), N = b1 - b0 bits.
 * They are cut into 512 windows as evenly as integers allow: window i is
 * [b0 + floor(i*N/512), b0 + floor((i+1)*N/512)), so every window has
 * floor(N/512) or ceil(N/512) bits.  cnt[c][i] counts the codes that START in
 * window i (at most 1536, a window's largest bit count, so 11 bits); gap[c][i]
 * is the offset of the first of them from the window start (always < 24, 5
 * bits), and 0 when cnt is 0.  One 16-bit entry per window holds both, 1024
 * bytes per chunk.  (The df11pack page's experimental 8-bit block index,
 * "Beyond the official format", halves that with windows of equal code
 * counts; such windows decode slower on this kernel, whose lanes run
 * windows side by side and wait for the one with the most look-ups, so the
 * windows here have equal bit counts instead.)  The first code of window i is
 * element out_elem[c] + (cnt[c][0] + ... + cnt[c][i-1]) -- a prefix sum over
 * the windows.  The decoder gives one 256-lane workgroup to a chunk and two
 * neighbouring windows to each lane, and forms the prefix sum with one
 * wavefront scan per wave plus the totals of the waves below.
 */
#ifndef DF11_H
#define DF11_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define DF11_ABI_VERSION 2
#define DF11_HEADER_BYTES 512
#define DF11_CHUNK_ELEMS 32768
#define DF11_WINDOWS 512
#define DF11_MAX_CODE_LEN 24
/* Header flag and encode option: the header holds the SHA-256 of the
 * source words. */
#define DF11_FLAG_SHA256 1u
/* Tensors decoded by one kernel launch; larger batches are split. */
#define DF11_MAX_BATCH 64

typedef enum {
    DF11_OK = 0,
    DF11_E_ARG = 1,          /* a NULL / misaligned / out-of-range argument */
    DF11_E_FORMAT = 2,       /* the container fails structural validation */
    DF11_E_UNSUPPORTED = 3,  /* a valid header this build does not decode */
    DF11_E_HIP = 4,          /* a HIP runtime call failed */
    DF11_E_CORRUPT = 5,      /* a decode found a stream inconsistent with its index */
    DF11_E_NOMEM = 6         /* host allocation failed */
} df11_status;

typedef struct df11_plan_s *df11_plan_t;

typedef struct {
    uint64_t n_elems;
    uint32_t ndim;
    uint32_t n_chunks;
    uint64_t dims[8];
    uint64_t total_bits;
    uint64_t container_bytes;     /* whole container */
    uint64_t meta_bytes;          /* header + chunk index + window index (what df11_plan needs) */
    uint64_t bytes_read_per_decode;  /* what a decode reads: the plan's 64-byte record per chunk,
                                        the window index, the code bits and the raw bytes */
    uint8_t code_len[256];
    uint32_t flags;               /* header flags (DF11_FLAG_SHA256) */
    uint8_t sha256[32];           /* the source hash when flags has DF11_FLAG_SHA256, else zero */
} df11_tensor_info;

/* ---------------------------------------------------------------- host-only */

/* Validate a container prefix held in HOST memory and describe it.
 * `host_meta` must hold at least the metadata prefix (header, chunk index,
 * window index: info->meta_bytes).  When `bytes` covers the whole container
 * the stream padding is checked too.  Checks: magic, version, chunk size,
 * window count, code lengths <= 24, Kraft sum (exactly 1, or 1/2 for a single
 * symbol), section offsets and sizes, start bits monotone with out_elem =
 * 32768*c, per chunk: sum of cnt = chunk size, gap < 24 when cnt > 0, gap =
 * 0 when cnt = 0, and a window's codes fit its share of the stream.
 * `info` may be NULL.  Reads only; allocates nothing on the device.
 * Returns DF11_OK, DF11_E_ARG, DF11_E_FORMAT or DF11_E_UNSUPPORTED. */
df11_status df11_validate(const void *host_meta, size_t bytes, df11_tensor_info *info);

/* Size bound of the container for n elements (any data). */
uint64_t df11_container_bound(uint64_t n_elems);

/* Encode n BF16 words (HOST memory, uint16 bit patterns) into a version-4
 * container in HOST memory `out` (capacity `out_cap`, at least
 * df11_container_bound(n)).  dims[ndim] is the shape (ndim <= 8, product =
 * n; ndim = 0 means a scalar, n = 1).  `threads` = 0 uses every hardware
 * thread.  The result is deterministic (independent of `threads`).
 * On success *out_bytes is the container size. */
df11_status df11_encode(const uint16_t *host_words, uint64_t n_elems, int ndim,
                        const uint64_t *dims, void *out, uint64_t out_cap,
                        uint64_t *out_bytes, int threads);

/* df11_encode with options: flags = 0 or DF11_FLAG_SHA256 (the header then
 * holds the SHA-256 of the source words, computed on one more thread while
 * the others encode; the other bytes are those df11_encode writes).  Any
 * other flag bit: DF11_E_ARG. */
df11_status df11_encode_ex(const uint16_t *host_words, uint64_t n_elems, int ndim,
                           const uint64_t *dims, uint32_t flags, void *out, uint64_t out_cap,
                           uint64_t *out_bytes, int threads);

/* Encode n BF16 words held in DEVICE memory (16-byte aligned) into a
 * version-4 container in DEVICE memory `d_out` (16-byte aligned, capacity
 * out_cap, at least df11_container_bound(n)), on `stream` of device
 * `hip_device`: the bytes df11_encode writes for the same words and shape.
 * The exponent histogram, the chunk bit counts, the chunk index, the packed
 * code stream, the window index and the raw bytes are computed by kernels;
 * the 256-symbol code and the layout are built on the host once the
 * histogram is back, so the call waits for the stream once and returns with
 * the rest enqueued on it (*out_bytes is the container size; the bytes are
 * there once the stream reaches that point).  Allocates 2 KiB of device
 * memory on the stream for the histogram.  No source hash (df11_encode_ex
 * adds it on the host). */
df11_status df11_encode_device(const void *d_words, uint64_t n_elems, int ndim, const uint64_t *dims,
                               void *d_out, uint64_t out_cap, uint64_t *out_bytes, int hip_device,
                               hipStream_t stream);

/* df11_encode_device for n_tensors tensors at once, sharing the one wait:
 * d_words[t], n_elems[t], ndims[t], dims[8 t .. 8 t + ndims[t]), d_outs[t],
 * out_caps[t] and out_bytes[t] describe tensor t.  Allocates 2 KiB of device
 * memory per tensor on the stream. */
df11_status df11_encode_device_batch(int n_tensors, const void *const *d_words, const uint64_t *n_elems,
                                     const int *ndims, const uint64_t *dims, void *const *d_outs,
                                     const uint64_t *out_caps, uint64_t *out_bytes, int hip_device,
                                     hipStream_t stream);

/* df11_encode_device_batch for callers that cannot allocate memory (tight
 * serving loops, harnesses that forbid hipMalloc): the same arguments, the
 * same kernels and the same bytes, but no device or host memory is allocated
 * and nothing is freed.  The histograms live in a fixed 128 KiB array of
 * device memory that each GPU the library runs on holds until the process
 * ends; its address on a device is looked up on the first call there.
 * At most 64 tensors per call (more: DF11_E_UNSUPPORTED, nothing enqueued);
 * hip_device below 64.  Every call on a GPU shares that GPU's array, which
 * keeps the last call's counts and is cleared at the start of each call:
 * the library holds a process-wide lock from that clearing until the codes
 * are built, so calls from several host threads take their turns instead of
 * racing on it (calls from different processes each have their own array).
 * Like df11_encode_device_batch it waits for the stream once, so it cannot
 * be captured into a graph.  The caller still allocates the outputs. */
df11_status df11_encode_device_batch_noalloc(int n_tensors, const void *const *d_words,
                                             const uint64_t *n_elems, const int *ndims,
                                             const uint64_t *dims, void *const *d_outs,
                                             const uint64_t *out_caps, uint64_t *out_bytes,
                                             int hip_device, hipStream_t stream);

/* SHA-256 (FIPS 180-4) of `bytes` bytes of HOST memory into digest[32]. */
void df11_sha256(const void *host_data, uint64_t bytes, uint8_t *digest);

/* Verify decoded words against the source hash in a container's header:
 * host_meta holds at least the container's metadata prefix (HOST memory),
 * host_words the n decoded words (HOST memory).  Returns DF11_OK when the
 * SHA-256 of the words equals the header's, DF11_E_CORRUPT when it differs,
 * DF11_E_UNSUPPORTED when the header holds no hash, DF11_E_ARG when n is not
 * the container's element count, DF11_E_FORMAT for an invalid container (the
 * df11pack page's verify exit codes: pass, a check failed, could not check). */
df11_status df11_verify_words(const void *host_meta, size_t bytes, const uint16_t *host_words,
                              uint64_t n_elems);

/* -------------------------------------------------------------------- plan */

/* Build a decode plan for n_tensors containers (the set of weights a caller
 * keeps compressed in GPU memory and decodes as it needs them: mlx-dfloat
 * project page, introduction).  Validation is the structural check the
 * df11pack page's verify runs with no source ("Use"); the decode tables are
 * built from the code lengths alone, every entry no valid stream reaches set
 * to zero (df11pack page, "Beyond the official format", the correct-LUTs
 * option).  host_meta[t] points to HOST
 * memory holding (at least) the metadata prefix of container t, of
 * host_meta_bytes[t] bytes.  Every prefix is validated (df11_validate).  The
 * plan builds each tensor's decode tables (a 1024-entry first-level table
 * that resolves up to three codes per look-up, a second-level table for codes
 * of 11 to 16 bits, canonical limits for longer codes) and uploads them, with
 * one 64-byte record per chunk (where its stream, window index and raw bytes
 * lie, from the validated chunk index), to device `hip_device` in one
 * allocation.  The caller may free host_meta once this returns.
 * flags: reserved, pass 0. */
df11_status df11_plan(const void *const *host_meta, const size_t *host_meta_bytes,
                      int n_tensors, int hip_device, uint32_t flags, df11_plan_t *out);

/* Release a plan.  The caller must first synchronize every stream that has
 * a decode of this plan in flight. */
void df11_plan_destroy(df11_plan_t plan);

df11_status df11_plan_info(df11_plan_t plan, int tensor, df11_tensor_info *info);

/* How many decode workgroups the plan's later launches may place on one
 * compute unit: 0 (the default) for as many as fit (three on gfx950), or 1
 * to that number.  For a decode that runs next to the model's own kernels
 * (the mlx-dfloat page, introduction: each block is decoded as the model
 * runs; "Measured numbers": the overhead that adds to a step), a smaller
 * number leaves LDS and wave slots on every compute unit for the other
 * kernel, so that the two can run at once; a decode alone is fastest with
 * the default.  Returns DF11_E_ARG for a NULL plan or a negative number;
 * numbers above the limit act as 0.  Set it before the plan's decodes are
 * issued from other threads: it is read, not locked, at each launch. */
df11_status df11_plan_set_wgs_per_cu(df11_plan_t plan, int wgs_per_cu);

/* ------------------------------------------------------------------ decode */

/* Decode tensor `tensor` of the plan: rebuild every BF16 word from its raw
 * byte (sign, 7-bit fraction) and its exponent byte, read as a prefix code
 * from the stream, bit for bit the original (mlx-dfloat project page,
 * introduction and its 16-bit weight diagram; df11pack project page,
 * introduction).  d_container: DEVICE pointer to the
 * whole container (16-byte aligned, at least container_bytes long, same
 * bytes as the prefix given to df11_plan).  d_out: DEVICE pointer to
 * n_elems * 2 bytes (16-byte aligned), not overlapping the container.
 * Enqueues on `stream` and returns; never allocates and never waits on a
 * stream.  Launches of one plan may run at the same time on any streams:
 * each takes one of the plan's 256 ticket counters that no unfinished launch
 * holds (a launch's last workgroup reports it finished through host memory);
 * when all 256 are held, the call waits on the host for one to come free (at
 * most 60 s, then DF11_E_HIP).  A launch made while `stream` is being
 * captured keeps its counter for good, so that the graph may be replayed any
 * number of times, one replay at a time; a plan gives at most 128 captured
 * launches a counter (then DF11_E_UNSUPPORTED).  The chunk start bits come from the plan;
 * the window index, the stream and the raw bytes from d_container.  Memory
 * safety does not depend on the device bytes: a container that differs from
 * the planned one gives wrong words and sets the plan's corruption flag (see
 * df11_check), never an out-of-bounds access. */
df11_status df11_decode(df11_plan_t plan, int tensor, const void *d_container,
                        void *d_out, hipStream_t stream);

/* Decode every tensor of the plan in one launch: a block's weights decoded
 * together, just before they are used (mlx-dfloat project page,
 * introduction: each block decoded on the GPU as it runs); one launch per
 * DF11_MAX_BATCH tensors.  d_containers[t] / d_outs[t] are HOST arrays of
 * DEVICE pointers, with the rules of df11_decode for each t. */
df11_status df11_decode_batch(df11_plan_t plan, const void *const *d_containers,
                              void *const *d_outs, hipStream_t stream);

/* The decode-side analogue of the df11pack page's verify ("Use": a check
 * passes or fails; exit codes 0, 1, 2): synchronize `stream`, then read and
 * clear the plan's corruption flag:
 * DF11_OK, or DF11_E_CORRUPT if some decode since the last check found a
 * window whose codes did not end where the index says the next window's
 * first code starts (or that starts past the chunk's bytes).  The flag is
 * one per plan: a decode of the plan on another stream that is still running
 * may set it after the read, and its finding then waits for the next check;
 * one that sets it between the read and the clear is lost, so check after the
 * decodes of interest have finished. */
df11_status df11_check(df11_plan_t plan, hipStream_t stream);

/* ------------------------------------------------------------ measurement */

/* Bandwidth control: enqueue on `stream` a kernel that reads src_bytes from
 * DEVICE memory d_src and writes dst_bytes to DEVICE memory d_dst with the
 * access pattern of a decode (16-byte non-temporal loads and stores,
 * contiguous ranges per workgroup) and no decoding; every source byte is read
 * and every output byte written.  Called with a decode's read and write
 * sizes, its rate is the HBM ceiling for that decode -- the analogue of the
 * control condition in the mlx-dfloat project page's overhead benchmark (the
 * same path without the decoding).  Sizes: multiples of 16, at least 16,
 * below 2^40 bytes, src_bytes <= dst_bytes (as in every decode: 2 bytes
 * written per element, fewer read; output unit i reads source unit
 * floor(i * src_bytes / dst_bytes)); pointers 16-byte aligned, regions not
 * overlapping.  The output bytes are unspecified.  Never allocates or synchronizes.
 * Returns DF11_OK, DF11_E_ARG or DF11_E_HIP. */
df11_status df11_bw_control(const void *d_src, uint64_t src_bytes, void *d_dst, uint64_t dst_bytes,
                            int hip_device, hipStream_t stream);

/* ------------------------------------------------------------------- NF12 */

/* NF12: a second, fixed-rate lossless format (nf12 news page, "Developer
 * open-sources nf12: lossless 12-bit compression for BF16 models", "How it
 * works" and "Implementation details").  Weights go in groups of 8.  When the
 * top four exponent bits of all 8 are 0111, the group is stored in 12 bytes:
 * code i = (sign << 11) | (low four exponent bits << 7) | fraction occupies
 * bits 12i .. 12i+11 (bit b = bit b % 8 of byte b / 8).  Any other group is
 * an outlier: its 12-byte slot is zero, a bitmap flags it, and its 8 words
 * are kept whole in an escape buffer (28 bytes per outlier group in all).
 * A partial last group is completed with the word 0x3800, which fits.
 *
 * Container (little-endian; sections start on 256-byte boundaries):
 *   header (256 bytes)
 *      0 char[8] magic "NF12HIPC"   8 u32 version = 1     12 u32 flags = 0
 *     16 u64 n_elems               24 u64 n_groups        32 u64 n_escaped
 *     40 u64 off_slots             48 u64 off_flags       56 u64 off_prefix
 *     64 u64 off_escape            72 u64 total_bytes     80 u8[176] 0
 *   slots   n_groups x 12 bytes
 *   flags   ceil(n_groups / 64) x u64: bit g % 64 of word g / 64 = group g
 *           is an outlier
 *   prefix  ceil(n_groups / 64) x u32: outlier groups before each flag word
 *   escape  n_escaped x 16 bytes: the outlier groups' words, in group order
 *   Bytes not named above are zero. */

/* Bytes an NF12 container of n elements can take at most. */
uint64_t df11_nf12_bound(uint64_t n_elems);

/* Encode n BF16 words (HOST, uint16 bit patterns) into an NF12 container in
 * HOST memory out (out_cap bytes, df11_nf12_bound(n) always suffices).
 * threads <= 0: all hardware threads.  The bytes do not depend on threads.
 * Returns DF11_OK or DF11_E_ARG. */
df11_status df11_nf12_encode(const uint16_t *words, uint64_t n, void *out, uint64_t out_cap,
                             uint64_t *out_bytes, int threads);

/* Validate an NF12 container in HOST memory.  With bytes >= its total size
 * every section is checked (flags, prefix counts, zero outlier slots and
 * padding); with fewer (at least the 256-byte header) only the header and
 * the layout.  *n_elems (if not NULL) receives the element count.
 * Returns DF11_OK, DF11_E_ARG, DF11_E_FORMAT or DF11_E_UNSUPPORTED. */
df11_status df11_nf12_validate(const void *container, size_t bytes, uint64_t *n_elems);

/* Decode an NF12 container: host_header = HOST copy of its first 256 bytes
 * (validated here); d_container = DEVICE pointer to the whole container;
 * d_out = DEVICE pointer to n_elems * 2 bytes.  Both 16-byte aligned, not
 * overlapping.  Enqueues on `stream`; never allocates or synchronizes.
 * Memory safety does not depend on the device bytes (an outlier's escape
 * entry is clamped into the escape buffer).
 * Returns DF11_OK, DF11_E_ARG, DF11_E_FORMAT, DF11_E_UNSUPPORTED or DF11_E_HIP. */
df11_status df11_nf12_decode(const void *host_header, const void *d_container, void *d_out,
                             int hip_device, hipStream_t stream);

/* Decode n_tensors NF12 containers in as few launches as possible (up to 24
 * tensors per launch): host_headers[t], d_containers[t] and d_outs[t] as in
 * df11_nf12_decode (the three arrays are HOST arrays).  Every header is
 * validated before anything is enqueued. */
df11_status df11_nf12_decode_batch(const void *const *host_headers, const void *const *d_containers,
                                   void *const *d_outs, int n_tensors, int hip_device, hipStream_t stream);

/* ------------------------------------------------------------------- misc */

/* Text of the last non-OK status on this thread (never NULL). */
const char *df11_last_error(void);
const char *df11_status_str(df11_status s);
int df11_abi_version(void);

#ifdef __cplusplus
}
#endif
#endif /* DF11_H */
