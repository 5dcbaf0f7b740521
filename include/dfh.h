/*
 * dfh.h -- C ABI of the lossless Huffman weight codec for AMD MI355X (gfx950).
 *
 * What the library does.  The DFloat11 digest ("DFloat11: compressao sem
 * perda para inferencia em GPU que reduz LLMs para 70% do tamanho",
 * pt.news.hada.io) and its paper's abstract ("70% Size, 100% Accuracy:
 * Lossless LLM Compression for Efficient GPU Inference via Dynamic-Length
 * Float") describe BF16 weights whose 8-bit exponent is Huffman coded while
 * sign and mantissa are stored raw, decompressed losslessly on the GPU just
 * before each transformer block runs.  The EntroLLM summary ("EntroLLM:
 * Entropy Encoded Weight Compression for Efficient Large Language Model
 * Inference on Edge Devices", section "Metodologia") Huffman codes whole
 * uint8 quantised weights and decodes them in parallel, and names 4-bit
 * codes as well.  This library covers all three: DF_KIND_BF16 codes the
 * exponent byte, DF_KIND_U8 codes the byte, DF_KIND_U4 codes the nibble
 * (16-symbol alphabet; elements packed two per byte, element 2j in the low
 * nibble of byte j, in the input and in the decoded output).
 *
 * Host calls build a codebook and encode into a library-owned container;
 * device calls decompress a container whose sections the caller has copied
 * to device memory.
 *
 * Conventions for every call:
 *   - Returns df_status; nothing throws across the ABI.
 *   - Pointers are borrowed for the duration of the call unless stated.
 *   - Host calls are reentrant; containers are immutable after df_encode or
 *     df_container_load and may be read from several threads.
 *   - Device calls enqueue work on the given HIP stream and return without
 *     synchronising, allocating, or copying between host and device.
 *
 * Container format (little-endian).  Element i has symbol e_i (the BF16
 * exponent byte (u >> 7) & 0xFF, the uint8 value, or the uint4 nibble).  Codes are canonical
 * (RFC 1951 section 3.2.2) from lengths[256] (0 = unused, 1..32).  Sections:
 *   BITSTREAM      codes of e_0, e_1, ... concatenated, packed least
 *                  significant bit first inside each byte, each code emitted
 *                  from its most significant bit; n_tiles*2048 + 16 bytes,
 *                  zero padded.  (Digest, "O formato DFloat11":
 *                  EncodedExponent.)
 *   GAPS           5-bit field per decoding thread t (8 stream bytes each),
 *                  at stream bits [5t, 5t+5), least significant bit first:
 *                  the offset of the first code that starts at or after bit
 *                  64t, always 0..31; 0 for t >= n_threads.
 *                  n_tiles*160 + 16 bytes.  (Digest, "Kernel de GPU em 2
 *                  etapas e metadados auxiliares": Gaps array.)
 *   TILE_OUT       uint64[n_tiles + 1]: number of codes starting before bit
 *                  16384*b (the output index of the first element of thread
 *                  block b); the last entry is n.  (Same section: one output
 *                  position per thread block.)
 *   SIGN_MANTISSA  BF16 only: byte i = (sign << 7) | mantissa7 of element i;
 *                  round_up(n, 64) bytes, zero padded; 0 bytes for uint8
 *                  and uint4.
 *                  (Digest, "O formato DFloat11": PackedSignMantissa.)
 *   LUT            uint16[n_luts * 256]: the code tree cut into height-8
 *                  subtrees, one 256-entry table each, indexed by the next 8
 *                  stream bits (first bit = index bit 0).  Entry: leaf =
 *                  (code length << 8) | symbol; pointer = 0x8000 | table;
 *                  0xFFFF = no code.  Tables numbered breadth first.
 *                  (Digest, "Decodificacao com LUT hierarquica".)
 *   DTAB           derived from lengths, not stored in files: a
 *                  decoder-side table indexed by the next stream bits that
 *                  gives several whole codes at once.
 *                  BF16 and uint4: uint64[4096], indexed by 12 bits, up to
 *                  five codes.  Layout: bits 0..31 symbol bytes of codes
 *                  0..3 (BF16: exponent rotated right by one bit), 32..36
 *                  bits consumed, 37..47 flags for codes starting at window
 *                  bits 1..11, 48..55 symbol byte of code 4, 56..63 number
 *                  of codes; 0 = first code longer than 12 bits.  uint4
 *                  holds its symbols as nibbles instead: bits 0..19 the
 *                  low nibbles of codes 0..4, bits 20..31 and 48..55 zero.
 *                  uint8: uint32[8192] indexed by 13 bits, up to two codes
 *                  (6.6-bit codes rarely leave room for a third): bits 0..3
 *                  bits consumed, 4..7 zero, 8..15 symbol of code 0,
 *                  16..23 symbol of code 1 (0 when one code), 24..31
 *                  number of codes; 0 = first code longer than 13 bits.
 *                  Then uint8[256]: the code length of each symbol.
 *                  DF_DTAB_BYTES_U8 bytes.
 * n_threads = floor(start of last code / 64) + 1 (0 when n == 0) and
 * n_tiles = ceil(n_threads / 256).
 */
#ifndef DFH_H
#define DFH_H

#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  DF_OK = 0,
  DF_ERR_ARG = -1,      /* bad argument: null pointer, bad kind, misaligned dst, ... */
  DF_ERR_ALLOC = -2,    /* host allocation failed */
  DF_ERR_CODEBOOK = -3, /* no code fits max_len, or an input symbol has no code */
  DF_ERR_FORMAT = -4,   /* container header or sections inconsistent */
  DF_ERR_HIP = -5,      /* a HIP runtime call or kernel launch failed */
  DF_ERR_CORRUPT = -6,  /* container contents fail validation */
  DF_ERR_IO = -7        /* file could not be read or written */
} df_status;

typedef enum { DF_KIND_BF16 = 0, DF_KIND_U8 = 1, DF_KIND_U4 = 2 } df_kind;

typedef enum {
  DF_SEC_BITSTREAM = 0,
  DF_SEC_GAPS = 1,
  DF_SEC_TILE_OUT = 2,
  DF_SEC_SIGN_MANTISSA = 3,
  DF_SEC_LUT = 4,
  DF_SEC_DTAB = 5,
  DF_SEC_COUNT = 6
} df_section;

#define DF_MAX_LEN 32           /* longest code; a gap then fits 5 bits        */
#define DF_BYTES_PER_THREAD 8   /* stream bytes per decoding thread           */
#define DF_THREADS_PER_TILE 256 /* decoding threads per tile (thread block)   */
#define DF_TILE_BITS 16384      /* stream bits per tile                       */
#define DF_MAX_LUTS 64          /* cap on hierarchical tables (32 KiB)        */
#define DF_DTAB_BITS 12         /* index width of the multi-code table        */
#define DF_DTAB_BITS_U8 13      /* index width of the uint8 pair table        */
#define DF_DTAB_BYTES_U8 (4 * 8192 + 256) /* uint8 DTAB: pair table + lengths */
#define DF_MAX_BATCH 16         /* containers per df_decompress_batch launch  */
#define DF_ENCODE_SCRATCH_BYTES (16u << 20) /* df_encode_device_noalloc's workspace */

/* Device error bits written by df_decompress_checked. */
#define DF_DEVERR_COUNT 1u  /* a tile (uint8: a pair of tiles) decodes to a different count than tile_out says */
#define DF_DEVERR_CODE 2u   /* a stream prefix matches no code, or a decode table
                              entry claims codes but consumes no bits            */

typedef struct {
  df_kind kind;
  uint32_t max_len;
  uint64_t n;              /* elements                                  */
  uint64_t total_bits;     /* sum of code lengths                       */
  uint64_t n_threads;      /* decoding threads that own a code start    */
  uint64_t n_tiles;        /* ceil(n_threads / 256)                     */
  uint32_t n_luts;         /* hierarchical tables                       */
  uint32_t max_tile_elems; /* largest tile_out[b+1] - tile_out[b]       */
  uint32_t bytes_per_thread;
  uint32_t threads_per_tile;
  uint64_t section_bytes[DF_SEC_COUNT];
  uint8_t lengths[256];
} df_info;

typedef struct df_container df_container; /* opaque, library-owned */

/* Histogram of the coded symbol (digest, "O formato DFloat11": the tree
 * follows the distribution of exponent values).  src holds n uint16 BF16
 * bit patterns (DF_KIND_BF16), n bytes (DF_KIND_U8) or (n + 1) / 2 bytes of
 * packed nibbles (DF_KIND_U4; a final odd element's high nibble is
 * ignored); hist receives 256 counts.  Multi-threaded on the host.  DF_ERR_ARG on a null pointer (src
 * may be null when n == 0) or a bad kind. */
df_status df_histogram(df_kind kind, const void *src, uint64_t n, uint64_t hist[256]);

/* Code lengths from a histogram (digest, "O formato DFloat11": frequent
 * exponents get short codes; "Kernel de GPU em 2 etapas e metadados
 * auxiliares": codes are at most 32 bits).  Huffman's construction merging
 * the two smallest (weight, key) nodes, leaves keyed by symbol and merged
 * nodes by 256 + creation order; when its longest code exceeds max_len, the
 * optimal max_len-limited lengths by package-merge.  One used symbol gets
 * length 1; none gives all zeros.  lengths[s] = 0 for unused symbols.
 * DF_ERR_ARG for max_len outside 1..32; DF_ERR_CODEBOOK when 2^max_len is
 * below the number of used symbols, or when the codes would need more than
 * DF_MAX_LUTS hierarchical tables (a histogram with one dominant symbol and
 * very many rare ones, whose long codes spread over many 8-bit prefixes). */
df_status df_build_codebook(const uint64_t hist[256], uint32_t max_len, uint8_t lengths[256]);

/* Encode n elements with the given lengths into a new container (*out,
 * freed with df_container_free).  Builds every section described above.
 * DF_ERR_CODEBOOK when an element's symbol has length 0, lengths violate
 * Kraft's inequality or exceed 32, or the codes need more than DF_MAX_LUTS
 * hierarchical tables; DF_ERR_ALLOC on allocation failure. */
df_status df_encode(df_kind kind, const void *src, uint64_t n, const uint8_t lengths[256],
                    df_container **out);

/* Header scalars, section sizes and lengths of a container. */
df_status df_container_info(const df_container *c, df_info *out);

/* Pointer to a section's bytes inside the container (valid until
 * df_container_free) and its size in *nbytes; NULL for a bad argument. */
const void *df_container_section(const df_container *c, df_section s, uint64_t *nbytes);

/* Write / read a container file (header, then every section except DTAB,
 * each 64-byte aligned; DTAB is rebuilt on load).  Load validates the
 * result and returns DF_ERR_FORMAT or DF_ERR_CORRUPT on a bad file. */
df_status df_container_save(const df_container *c, const char *path);
df_status df_container_load(const char *path, df_container **out);

/* Structural check of a container: header scalars against each other,
 * section sizes, lengths (Kraft), tile_out monotone from 0 to n with
 * max_tile_elems its largest step, gaps in range and zero past n_threads,
 * LUT and DTAB equal to the tables rebuilt from lengths.  It does not
 * decode the stream.  DF_ERR_FORMAT or DF_ERR_CORRUPT on failure. */
df_status df_container_validate(const df_container *c);

void df_container_free(df_container *c);
const char *df_status_string(df_status s);

/* ------------------------------------------------------------------ device */

/* Borrowed device pointers to a container's sections (caller-owned, e.g.
 * torch tensors) plus its header scalars.  sign_mantissa is NULL unless the
 * kind is DF_KIND_BF16.  Every section must have the size df_info reports.
 * max_workgroups: 0 lets a launch take every workgroup slot the device has
 * (the fastest decode on an otherwise idle GPU); a positive value caps the
 * launch's workgroups (of up to 1024 lanes; at most two share a CU), so a
 * decode on a side stream leaves most CUs to the kernels running beside it
 * (the digest's "Descompressao por bloco de transformer": the next block is
 * decompressed while the current one computes).  A batched launch takes the
 * smallest positive cap of its views. */
typedef struct {
  df_kind kind;
  uint32_t n_luts;
  uint32_t max_tile_elems;
  uint32_t max_workgroups;
  uint64_t n;
  uint64_t total_bits;
  uint64_t n_threads;
  uint64_t n_tiles;
  const uint8_t *bitstream;
  const uint8_t *gaps;
  const uint64_t *tile_out;
  const uint8_t *sign_mantissa;
  const uint16_t *lut;
  const uint64_t *dtab;
} df_device_view;

/* Decompress one container into dst (n * 2 bytes of BF16 bit patterns, n
 * bytes of uint8, or (n + 1) / 2 bytes of packed uint4 with a final odd
 * element's high nibble zero; 16-byte aligned, not aliasing any section).  The
 * digest's "Kernel de GPU em 2 etapas e metadados auxiliares": each thread
 * owns 8 stream bytes and decodes the codes that start in them, first only
 * counting, then (after a prefix sum of the counts over the thread block)
 * decoding again into an on-chip buffer that is written to memory in one
 * coalesced pass; "Decodificacao com LUT hierarquica": code tables sit in
 * on-chip memory.  One launch covers the whole container (the digest's
 * "Descompressao por bloco de transformer": one batch per block).
 * n == 0 enqueues nothing.  DF_ERR_ARG on bad pointers, kind, alignment,
 * or sizes (including containers of 2^31 tiles or more, a 4 TiB stream: the
 * kernels index tiles in 32 bits); DF_ERR_HIP when the launch fails.
 * Scheduling: a BF16 container of more than three steps of tiles (three
 * times the launch's tile groups) is decoded with tiles handed out by
 * device-side counters that the library keeps in its code object (no
 * allocation).  Each running dispatch claims its own counter slot on the
 * device, keyed by its dispatch packet, and frees it clean when its last
 * tile has been handed out, so no state carries from one launch to the
 * next and launches running at once (several streams, several instances of
 * one captured graph) never share counters.  The
 * decoded bytes do not depend on the schedule. */
df_status df_decompress(const df_device_view *v, void *dst, hipStream_t stream);

/* As df_decompress, and also checks every tile on the device: d_err (one
 * device uint32, zeroed by the caller beforehand) receives the OR of
 * DF_DEVERR_* bits; read it after synchronising the stream.  Output of a
 * tile that fails a check is unspecified; writes stay inside dst.  A uint8
 * launch decodes tiles in pairs (2p, 2p + 1) and checks each pair against
 * tile_out[2p] and tile_out[min(2p + 2, n_tiles)]. */
df_status df_decompress_checked(const df_device_view *v, void *dst, uint32_t *d_err,
                                hipStream_t stream);

/* Decompress count containers of one kind in a single launch (the EntroLLM
 * summary, "Metodologia": separate tensors decoded at the same time).  views
 * is an array of count views, dsts an array of count destinations.  count
 * may exceed DF_MAX_BATCH; the library then issues several launches.  Same
 * errors as df_decompress; containers of different kinds give DF_ERR_ARG. */
df_status df_decompress_batch(const df_device_view *views, void *const *dsts, uint32_t count,
                              hipStream_t stream);

/* ------------------------------------------------------- device encoding */

/* Encoding on the GPU, for weights already in device memory (fast
 * conversion of a checkpoint; the pages encode offline and describe no
 * encoder kernel, so this part is this library's own).  The sections it
 * writes are byte-identical to df_encode's.  Steps:
 *   1. df_histogram_device and df_symbol_device (the last element's
 *      symbol), then copy the 256 counts and the symbol to the host;
 *   2. df_build_codebook on the host;
 *   3. df_encode_layout for the sizes, df_build_tables for LUT and DTAB;
 *   4. allocate the device sections and df_encode_workspace_bytes(n) bytes
 *      of device workspace, copy LUT and DTAB, then df_encode_device.
 * Device calls enqueue on the stream and return, as for decompression. */

/* Histogram of the coded symbols of n device elements (layout as for
 * df_histogram; d_src 16-byte aligned) into d_hist, 256 device uint64
 * counts; the call clears them first.  DF_ERR_ARG on a null or misaligned
 * pointer or a bad kind. */
df_status df_histogram_device(df_kind kind, const void *d_src, uint64_t n, uint64_t *d_hist,
                              hipStream_t stream);

/* The coded symbol of device element i (the BF16 exponent byte
 * (u >> 7) & 0xFF, the uint8 value, or the uint4 nibble; layout as for
 * df_histogram), written to *d_sym as one device uint64 (8-byte aligned).
 * With i = n - 1 it is the last_symbol df_encode_layout takes.  i must lie
 * inside the source; DF_ERR_ARG on a null or misaligned pointer or a bad
 * kind. */
df_status df_symbol_device(df_kind kind, const void *d_src, uint64_t i, uint64_t *d_sym, hipStream_t stream);

/* Header scalars and section sizes of the container df_encode would build
 * for n elements with this histogram and these lengths, whose last element
 * has symbol last_symbol (max_tile_elems is left 0: df_encode_device
 * reports it).  DF_ERR_CODEBOOK when a counted symbol has no code or the
 * lengths break Kraft's inequality; DF_ERR_ARG on a bad argument. */
df_status df_encode_layout(df_kind kind, uint64_t n, const uint64_t hist[256], uint8_t last_symbol,
                           const uint8_t lengths[256], df_info *out);

/* The derived decode tables for these lengths: lut (room for lut_cap
 * 256-entry levels) with *n_luts levels used, and dtab (4096 words; uint8:
 * DF_DTAB_BYTES_U8 bytes), as in the container sections LUT and DTAB.
 * DF_ERR_CODEBOOK when more than lut_cap levels are needed. */
df_status df_build_tables(df_kind kind, const uint8_t lengths[256], uint16_t *lut, uint32_t lut_cap,
                          uint32_t *n_luts, uint64_t *dtab);

/* Device workspace bytes df_encode_device needs for n elements. */
uint64_t df_encode_workspace_bytes(uint64_t n);

/* Encode n device elements (d_src 16-byte aligned) into device sections
 * sized by df_encode_layout (layout is its result): bitstream, gaps, tile_out and, for BF16,
 * sign_mantissa (NULL otherwise).  d_workspace: df_encode_workspace_bytes(n)
 * bytes, 16-byte aligned.  d_max_tile (one device uint32) receives
 * max_tile_elems.  Each element's code goes at the sum of the lengths of
 * the codes before it (a scan of code lengths over the elements). */
df_status df_encode_device(df_kind kind, const void *d_src, uint64_t n, const uint8_t lengths[256],
                           const df_info *layout, uint8_t *d_bitstream, uint8_t *d_gaps,
                           uint64_t *d_tile_out, uint8_t *d_sign_mantissa, void *d_workspace,
                           uint32_t *d_max_tile, hipStream_t stream);

/* df_encode_device for callers that cannot allocate device memory: code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc.  Same arguments, results and errors as df_encode_device
 * without d_workspace: the workspace is a DF_ENCODE_SCRATCH_BYTES array in
 * the library's code object (one per device, held until the process ends;
 * its address is taken once per device on the first call there).  The call
 * allocates nothing.  n is limited to df_encode_workspace_bytes(n) <=
 * DF_ENCODE_SCRATCH_BYTES (about 4.29e9 elements); a larger n gives
 * DF_ERR_ARG before anything is enqueued.  Every call on one device uses
 * the same array, and the encode writes every workspace word it reads, so
 * nothing carries over from the previous call; calls that overlap on one
 * device (different streams, or graph instances in flight together) race
 * on it and must be ordered by the caller. */
df_status df_encode_device_noalloc(df_kind kind, const void *d_src, uint64_t n, const uint8_t lengths[256],
                                   const df_info *layout, uint8_t *d_bitstream, uint8_t *d_gaps,
                                   uint64_t *d_tile_out, uint8_t *d_sign_mantissa, uint32_t *d_max_tile,
                                   hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* DFH_H */
