/*
 * oracle.c -- TEST INFRASTRUCTURE ONLY.
 *
 * A plain, slow, scalar CPU oracle for lossless Huffman coding of LLM weights:
 *   - the DFloat11 scheme (BF16 exponent byte Huffman-coded, sign and mantissa
 *     kept raw), and
 *   - the EntroLLM scheme (whole uint8 quantised codes Huffman-coded, and
 *     uint4 codes as a 16-symbol alphabet).
 *
 * Only the test suite, the smoke check and the CPU-baseline leg of the
 * benchmark may load this library.  It shares no code, header, table or
 * constant with the product library: every constant below is restated here
 * from the container format specification.
 *
 * Sources (cited by page title and section heading):
 *   [DF11]  "DFloat11: compressao sem perda para inferencia em GPU que reduz
 *            LLMs para 70% do tamanho" (pt.news.hada.io digest of the DFloat11
 *            paper).
 *   [DF11A] "70% Size, 100% Accuracy: Lossless LLM Compression for Efficient
 *            GPU Inference via Dynamic-Length Float" (abstract page).
 *   [ENTRO] "EntroLLM: Entropy Encoded Weight Compression for Efficient Large
 *            Language Model Inference on Edge Devices" (gist.science summary).
 *   [RFC1951] DEFLATE specification, section 3.2.2 (canonical Huffman codes)
 *            and section 3.1.1 (packing bits into bytes), used where the pages
 *            are silent about which prefix code and which bit order.
 *
 * Readings of the pages that this file follows (each also listed in the
 * design notes of the repository):
 *   - codes are canonical (RFC 1951 3.2.2) and derived from code lengths;
 *   - Huffman ties: merge the two smallest (weight, key) nodes, leaves keyed by
 *     symbol, internal nodes by 256 + creation index;
 *   - lengths are limited to 32 bits; when plain Huffman exceeds 32 the
 *     optimal 32-limited lengths are found by package-merge;
 *   - a single used symbol gets length 1 (code "0");
 *   - bit order: the stream is packed least-significant bit first inside each
 *     byte (RFC 1951 3.1.1), and each code is emitted starting with its most
 *     significant bit;
 *   - 8 bytes of stream per decoding thread, 256 threads per tile;
 *   - gap of chunk t = (first code start >= 64 t) - 64 t, packed in 5-bit
 *     fields, least significant bit first;
 *   - tile_out[b] = number of codes that start before bit 16384 b, with one
 *     extra final entry equal to n;
 *   - uint4 codes are packed two per byte, element 2j in the low nibble of
 *     byte j (a final odd element leaves the high nibble zero), both in the
 *     input and in the decoded output.
 */
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <pthread.h>

#define O_KIND_BF16 0
#define O_KIND_U8 1
#define O_KIND_U4 2
#define O_MAX_LEN 32
#define O_CHUNK_BITS 64             /* 8 bytes of stream per thread            */
#define O_THREADS_PER_TILE 256
#define O_TILE_BITS (O_CHUNK_BITS * O_THREADS_PER_TILE)   /* 16384 bits */
#define O_GAP_BITS 5

/* ------------------------------------------------------------------------ */
/* Field split and merge.  [DF11, "O espaco de compressao ainda disponivel no
 * expoente do BFloat16"]: BF16 = 1 sign bit, 8 exponent bits, 7 mantissa
 * bits.  [DF11, "O formato DFloat11"]: only the exponent is entropy coded;
 * sign and mantissa are kept as they are, one byte per weight
 * (sign << 7 | mantissa).                                                    */
/* ------------------------------------------------------------------------ */
int oracle_split_bf16(const uint16_t *w, uint64_t n, uint8_t *exp_out,
                      uint8_t *sm_out) {
  for (uint64_t i = 0; i < n; i++) {
    uint16_t u = w[i];
    uint8_t sign = (uint8_t)(u >> 15);
    uint8_t expo = (uint8_t)((u >> 7) & 0xFF);
    uint8_t mant = (uint8_t)(u & 0x7F);
    if (exp_out) exp_out[i] = expo;
    if (sm_out) sm_out[i] = (uint8_t)((sign << 7) | mant);
  }
  return 0;
}

int oracle_merge_bf16(const uint8_t *expo, const uint8_t *sm, uint64_t n,
                      uint16_t *w_out) {
  for (uint64_t i = 0; i < n; i++) {
    uint16_t sign = (uint16_t)(sm[i] >> 7);
    uint16_t mant = (uint16_t)(sm[i] & 0x7F);
    w_out[i] = (uint16_t)((sign << 15) | ((uint16_t)expo[i] << 7) | mant);
  }
  return 0;
}

/* The coded symbol of element i: the exponent byte for BF16, the byte itself
 * for uint8, the nibble for uint4 ([ENTRO, "Metodologia"], Huffman coding of
 * the quantised codes, 8-bit or 4-bit). */
static uint8_t symbol_of(int kind, const void *src, uint64_t i) {
  if (kind == O_KIND_BF16) {
    uint16_t u = ((const uint16_t *)src)[i];
    return (uint8_t)((u >> 7) & 0xFF);
  }
  if (kind == O_KIND_U4) {
    uint8_t b = ((const uint8_t *)src)[i / 2];
    return (uint8_t)((i % 2 == 0) ? (b & 0x0F) : (b >> 4));
  }
  return ((const uint8_t *)src)[i];
}

/* uint4 output: pack n symbols (one per byte, values 0..15) two per byte,
 * element 2j in the low nibble of byte j; writes (n + 1) / 2 bytes. */
int oracle_pack_u4(const uint8_t *syms, uint64_t n, uint8_t *out) {
  for (uint64_t j = 0; j < (n + 1) / 2; j++) {
    uint8_t lo = syms[2 * j];
    uint8_t hi = (2 * j + 1 < n) ? syms[2 * j + 1] : 0;
    if (lo > 15 || hi > 15) return -1;
    out[j] = (uint8_t)(lo | (hi << 4));
  }
  return 0;
}

/* Histogram of the coded symbol.  [DF11, "O formato DFloat11"]: the tree is
 * built from the distribution of the exponent values.                       */
int oracle_histogram(int kind, const void *src, uint64_t n, uint64_t *hist) {
  if (kind != O_KIND_BF16 && kind != O_KIND_U8 && kind != O_KIND_U4) return -1;
  for (int s = 0; s < 256; s++) hist[s] = 0;
  for (uint64_t i = 0; i < n; i++) hist[symbol_of(kind, src, i)]++;
  return 0;
}

/* ------------------------------------------------------------------------ */
/* Plain Huffman code lengths.  [DF11, "O formato DFloat11"]: frequent
 * exponents get short codes and rare ones long codes, from a Huffman tree of
 * the histogram.  Textbook construction: repeatedly merge the two lightest
 * nodes.  Ties are broken on (weight, key) where a leaf's key is its symbol
 * and an internal node's key is 256 + its creation index.  The two lightest
 * nodes are found by a linear scan (at most 511 nodes).
 * Writes lengths into len_out (int, may exceed 32).  Returns the number of
 * used symbols.                                                              */
/* ------------------------------------------------------------------------ */
int oracle_huffman_lengths(const uint64_t *hist, int *len_out) {
  uint64_t weight[511];
  int key[511], parent[511], alive[511];
  int nodes = 0, used = 0;
  int leaf_of_sym[256];
  for (int s = 0; s < 256; s++) {
    len_out[s] = 0;
    leaf_of_sym[s] = -1;
    if (hist[s] > 0) {
      weight[nodes] = hist[s];
      key[nodes] = s;
      parent[nodes] = -1;
      alive[nodes] = 1;
      leaf_of_sym[s] = nodes;
      nodes++;
      used++;
    }
  }
  if (used == 0) return 0;
  if (used == 1) {
    /* one symbol: a one-bit code "0" */
    for (int s = 0; s < 256; s++)
      if (hist[s] > 0) len_out[s] = 1;
    return 1;
  }
  int created = 0;
  for (int step = 0; step < used - 1; step++) {
    int a = -1, b = -1;
    for (int i = 0; i < nodes; i++) {
      if (!alive[i]) continue;
      if (a < 0 || weight[i] < weight[a] ||
          (weight[i] == weight[a] && key[i] < key[a])) {
        b = a;
        a = i;
      } else if (b < 0 || weight[i] < weight[b] ||
                 (weight[i] == weight[b] && key[i] < key[b])) {
        b = i;
      }
    }
    alive[a] = 0;
    alive[b] = 0;
    weight[nodes] = weight[a] + weight[b];
    key[nodes] = 256 + created;
    created++;
    parent[nodes] = -1;
    alive[nodes] = 1;
    parent[a] = nodes;
    parent[b] = nodes;
    nodes++;
  }
  for (int s = 0; s < 256; s++) {
    if (leaf_of_sym[s] < 0) continue;
    int depth = 0;
    for (int v = leaf_of_sym[s]; parent[v] >= 0; v = parent[v]) depth++;
    len_out[s] = depth;
  }
  return used;
}

/* ------------------------------------------------------------------------ */
/* Length-limited code lengths by package-merge (Larmore and Hirschberg,
 * "A fast algorithm for optimal length-limited Huffman codes", J. ACM 1990).
 * Needed because [DF11, "Kernel de GPU em 2 etapas e metadados auxiliares"]
 * relies on the maximum code length being 32 (a gap fits 5 bits), while
 * [DF11, "Decodificacao com LUT hierarquica"] reports lengths of 24 to 32 on
 * real models, so a skewed histogram must be limited.
 *
 * Each used symbol owns one coin per level 1..L of face value 2^-level and
 * numismatic value = its count.  Starting from the deepest level, adjacent
 * items are paired into packages and merged with the symbol list of the next
 * level up.  At level 1 the first 2m-2 items are selected, and a symbol's
 * length is the number of its coins inside the selection.  Ordering inside a
 * list: by weight, leaves before packages on equal weight, leaves by symbol,
 * packages by creation order.  Each item carries its per-symbol coin counts
 * explicitly.                                                                */
/* ------------------------------------------------------------------------ */
typedef struct {
  uint64_t w;
  int is_pkg;
  int order;           /* symbol for a leaf, creation index for a package */
  uint8_t cnt[256];    /* coins of each symbol contained */
} pm_item;

int oracle_limited_lengths(const uint64_t *hist, int max_len, int *len_out) {
  int syms[256], m = 0;
  for (int s = 0; s < 256; s++) {
    len_out[s] = 0;
    if (hist[s] > 0) syms[m++] = s;
  }
  if (m == 0) return 0;
  if (m == 1) {
    len_out[syms[0]] = 1;
    return 1;
  }
  if (max_len < 1 || max_len > 63) return -1;
  if (((uint64_t)1 << max_len) < (uint64_t)m) return -1;
  /* leaves sorted by (weight, symbol): insertion sort, m <= 256 */
  for (int i = 1; i < m; i++) {
    int s = syms[i], j = i - 1;
    while (j >= 0 && (hist[syms[j]] > hist[s] ||
                      (hist[syms[j]] == hist[s] && syms[j] > s))) {
      syms[j + 1] = syms[j];
      j--;
    }
    syms[j + 1] = s;
  }
  size_t cap = (size_t)3 * m + 4;
  pm_item *cur = (pm_item *)calloc(cap, sizeof(pm_item));
  pm_item *nxt = (pm_item *)calloc(cap, sizeof(pm_item));
  pm_item *pk = (pm_item *)calloc(cap, sizeof(pm_item));
  if (!cur || !nxt || !pk) {
    free(cur); free(nxt); free(pk);
    return -1;
  }
  int ncur = 0;
  for (int i = 0; i < m; i++) {
    memset(&cur[ncur], 0, sizeof(pm_item));
    cur[ncur].w = hist[syms[i]];
    cur[ncur].is_pkg = 0;
    cur[ncur].order = syms[i];
    cur[ncur].cnt[syms[i]] = 1;
    ncur++;
  }
  int created = 0;
  for (int level = max_len; level >= 2; level--) {
    /* package adjacent pairs of the current list */
    int npk = 0;
    for (int i = 0; i + 1 < ncur; i += 2) {
      pk[npk].w = cur[i].w + cur[i + 1].w;
      pk[npk].is_pkg = 1;
      pk[npk].order = created++;
      for (int s = 0; s < 256; s++)
        pk[npk].cnt[s] = (uint8_t)(cur[i].cnt[s] + cur[i + 1].cnt[s]);
      npk++;
    }
    /* merge the leaves of the next level up with the packages */
    int li = 0, pi = 0, nn = 0;
    while (li < m || pi < npk) {
      int take_leaf;
      if (li >= m) take_leaf = 0;
      else if (pi >= npk) take_leaf = 1;
      else take_leaf = hist[syms[li]] <= pk[pi].w; /* leaf first on ties */
      if (take_leaf) {
        memset(&nxt[nn], 0, sizeof(pm_item));
        nxt[nn].w = hist[syms[li]];
        nxt[nn].is_pkg = 0;
        nxt[nn].order = syms[li];
        nxt[nn].cnt[syms[li]] = 1;
        li++;
      } else {
        nxt[nn] = pk[pi];
        pi++;
      }
      nn++;
    }
    pm_item *t = cur;
    cur = nxt;
    nxt = t;
    ncur = nn;
  }
  /* at level 1: select the first 2m-2 items */
  for (int i = 0; i < 2 * m - 2; i++)
    for (int s = 0; s < 256; s++) len_out[s] += cur[i].cnt[s];
  free(cur);
  free(nxt);
  free(pk);
  return m;
}

/* The codebook policy: plain Huffman when its longest code fits max_len,
 * otherwise the optimal max_len-limited lengths.  Writes u8 lengths.
 * Returns the number of used symbols, or -1 when max_len cannot hold them. */
int oracle_code_lengths(const uint64_t *hist, int max_len, uint8_t *lengths) {
  int lens[256];
  int used = oracle_huffman_lengths(hist, lens);
  int longest = 0;
  for (int s = 0; s < 256; s++)
    if (lens[s] > longest) longest = lens[s];
  if (longest > max_len) {
    used = oracle_limited_lengths(hist, max_len, lens);
    if (used < 0) return -1;
  }
  for (int s = 0; s < 256; s++) lengths[s] = (uint8_t)lens[s];
  return used;
}

/* Canonical codes from lengths, RFC 1951 section 3.2.2: count codes per
 * length, the first code of each length is (first code of the previous
 * length + its count) shifted left by one, then codes are handed out in
 * increasing symbol order within a length.                                   */
int oracle_canonical_codes(const uint8_t *lengths, uint32_t *codes) {
  uint64_t bl_count[O_MAX_LEN + 2];
  uint64_t next_code[O_MAX_LEN + 2];
  for (int i = 0; i < O_MAX_LEN + 2; i++) bl_count[i] = next_code[i] = 0;
  for (int s = 0; s < 256; s++) {
    if (lengths[s] > O_MAX_LEN) return -1;
    if (lengths[s]) bl_count[lengths[s]]++;
  }
  uint64_t code = 0;
  for (int bits = 1; bits <= O_MAX_LEN; bits++) {
    code = (code + bl_count[bits - 1]) << 1;
    next_code[bits] = code;
  }
  for (int s = 0; s < 256; s++) {
    codes[s] = 0;
    if (lengths[s]) codes[s] = (uint32_t)(next_code[lengths[s]]++);
  }
  return 0;
}

/* ------------------------------------------------------------------------ */
/* Layout.  [DF11, "Kernel de GPU em 2 etapas e metadados auxiliares"]: each
 * thread owns a contiguous run of 8 bytes of the encoded exponents and
 * decodes the codes that start inside it; only the output position of the
 * first element of each thread block is stored.                             */
/* ------------------------------------------------------------------------ */
typedef struct {
  uint64_t n;
  uint64_t total_bits;
  uint64_t n_threads;
  uint64_t n_tiles;
  uint64_t bitstream_bytes;
  uint64_t gaps_bytes;
  uint64_t tile_out_entries;
  uint64_t sm_bytes;
  uint64_t max_tile_elems;
} oracle_layout_t;

static uint64_t round_up(uint64_t x, uint64_t a) { return (x + a - 1) / a * a; }

int oracle_layout(int kind, const void *src, uint64_t n, const uint8_t *lengths,
                  oracle_layout_t *out) {
  uint64_t bits = 0, last_start = 0;
  for (uint64_t i = 0; i < n; i++) {
    uint8_t s = symbol_of(kind, src, i);
    if (lengths[s] == 0) return -1; /* symbol without a code */
    last_start = bits;
    bits += lengths[s];
  }
  memset(out, 0, sizeof(*out));
  out->n = n;
  out->total_bits = bits;
  out->n_threads = n ? last_start / O_CHUNK_BITS + 1 : 0;
  out->n_tiles = (out->n_threads + O_THREADS_PER_TILE - 1) / O_THREADS_PER_TILE;
  out->bitstream_bytes = out->n_tiles * (O_TILE_BITS / 8) + 16;
  out->gaps_bytes = out->n_tiles * (O_THREADS_PER_TILE * O_GAP_BITS / 8) + 16;
  out->tile_out_entries = out->n_tiles + 1;
  out->sm_bytes = kind == O_KIND_BF16 ? round_up(n, 64) : 0;
  out->max_tile_elems = 0; /* filled by oracle_encode */
  return 0;
}

static void put_bit(uint8_t *buf, uint64_t pos, int bit) {
  if (bit) buf[pos >> 3] |= (uint8_t)(1u << (pos & 7));
}

static int get_bit(const uint8_t *buf, uint64_t pos) {
  return (buf[pos >> 3] >> (pos & 7)) & 1;
}

/* Encoder: bit-serial, one element at a time.  Writes
 *   bitstream (lay->bitstream_bytes, zero padded): the codes concatenated
 *             ([DF11, "O formato DFloat11"], EncodedExponent);
 *   gaps      (lay->gaps_bytes): 5-bit gap per thread, the offset of the first
 *             code that starts in the thread's 8 bytes ([DF11, "Kernel de GPU
 *             em 2 etapas e metadados auxiliares"], Gaps array);
 *   tile_out  (n_tiles + 1 entries): output index of the first element of
 *             each thread block, plus n at the end;
 *   sm        (BF16 only, lay->sm_bytes, zero padded): sign|mantissa bytes
 *             ([DF11, "O formato DFloat11"], PackedSignMantissa).
 * Sets lay->max_tile_elems.                                                  */
int oracle_encode(int kind, const void *src, uint64_t n, const uint8_t *lengths,
                  oracle_layout_t *lay, uint8_t *bitstream, uint8_t *gaps,
                  uint64_t *tile_out, uint8_t *sm) {
  uint32_t codes[256];
  if (oracle_canonical_codes(lengths, codes) != 0) return -1;
  memset(bitstream, 0, lay->bitstream_bytes);
  memset(gaps, 0, lay->gaps_bytes);
  if (kind == O_KIND_BF16 && lay->sm_bytes) memset(sm, 0, lay->sm_bytes);
  /* starts of every code, by definition: S_i = sum of earlier lengths */
  uint64_t pos = 0;
  uint64_t *first_start = (uint64_t *)malloc(sizeof(uint64_t) *
                                             (lay->n_threads ? lay->n_threads : 1));
  if (!first_start) return -1;
  for (uint64_t t = 0; t < lay->n_threads; t++) first_start[t] = UINT64_MAX;
  for (uint64_t b = 0; b <= lay->n_tiles; b++) tile_out[b] = 0;
  for (uint64_t i = 0; i < n; i++) {
    uint8_t s = symbol_of(kind, src, i);
    int len = lengths[s];
    uint64_t start = pos;
    uint64_t t = start / O_CHUNK_BITS;
    if (t < lay->n_threads && first_start[t] == UINT64_MAX) first_start[t] = start;
    /* emit the code most significant bit first */
    for (int k = len - 1; k >= 0; k--) put_bit(bitstream, pos++, (codes[s] >> k) & 1);
    if (kind == O_KIND_BF16) {
      uint16_t u = ((const uint16_t *)src)[i];
      sm[i] = (uint8_t)(((u >> 8) & 0x80) | (u & 0x7F));
    }
  }
  if (pos != lay->total_bits) {
    free(first_start);
    return -1;
  }
  for (uint64_t t = 0; t < lay->n_threads; t++) {
    uint64_t gap = first_start[t] - t * O_CHUNK_BITS;
    if (first_start[t] == UINT64_MAX || gap > 31) {
      free(first_start);
      return -2; /* cannot happen when every length is <= 32 */
    }
    for (int k = 0; k < O_GAP_BITS; k++)
      put_bit(gaps, t * O_GAP_BITS + k, (int)((gap >> k) & 1));
  }
  free(first_start);
  /* tile_out[b] = number of codes starting before bit 16384 b, by a second
   * pass over the starts */
  pos = 0;
  for (uint64_t i = 0; i < n; i++) {
    uint8_t s = symbol_of(kind, src, i);
    uint64_t first_b = pos / O_TILE_BITS + 1; /* smallest b with pos < 16384 b */
    if (first_b <= lay->n_tiles) tile_out[first_b]++;
    pos += lengths[s];
  }
  /* turn "codes starting in [16384 (b-1), 16384 b)" into a running count */
  for (uint64_t b = 1; b <= lay->n_tiles; b++) tile_out[b] += tile_out[b - 1];
  tile_out[lay->n_tiles] = n;
  lay->max_tile_elems = 0;
  for (uint64_t b = 0; b < lay->n_tiles; b++) {
    uint64_t d = tile_out[b + 1] - tile_out[b];
    if (d > lay->max_tile_elems) lay->max_tile_elems = d;
  }
  return 0;
}

/* ------------------------------------------------------------------------ */
/* Hierarchical lookup tables.  [DF11, "Decodificacao com LUT hierarquica"]:
 * the code tree is cut into disjoint subtrees of height 8, each a 256-entry
 * table; some entries point to a lower table.  Entry format of this repo
 * (u16): leaf = (total code length << 8) | symbol, bit 15 clear; pointer =
 * 0x8000 | child table index; 0xFFFF = no code has this prefix.  A table at
 * depth d is indexed by stream bits [8d, 8d+8) (first stream bit = index bit
 * 0).  Tables are numbered breadth first: table 0 is the root, and children
 * are numbered in the order their pointer entries are met when the tables are
 * scanned in number order, entries in increasing index.  Built here by a
 * plain scan: for each entry, search all symbols.                           */
/* ------------------------------------------------------------------------ */
static uint64_t stream_order(uint32_t code, int len) {
  /* the code's bits as they appear in the stream: first bit = bit 0 */
  uint64_t r = 0;
  for (int k = 0; k < len; k++) r |= (uint64_t)((code >> (len - 1 - k)) & 1) << k;
  return r;
}

int oracle_build_lut(const uint8_t *lengths, uint16_t *lut, int cap, int *n_luts) {
  uint32_t codes[256];
  if (oracle_canonical_codes(lengths, codes) != 0) return -1;
  uint64_t rev[256];
  for (int s = 0; s < 256; s++) rev[s] = lengths[s] ? stream_order(codes[s], lengths[s]) : 0;
  int depth_of[4096];
  uint64_t prefix_of[4096];
  int count = 1;
  depth_of[0] = 0;
  prefix_of[0] = 0;
  for (int tbl = 0; tbl < count; tbl++) {
    if (tbl >= cap) return -1;
    int d = depth_of[tbl];
    for (int j = 0; j < 256; j++) {
      uint64_t full = prefix_of[tbl] | ((uint64_t)j << (8 * d)); /* 8(d+1) bits */
      int hi = 8 * (d + 1);
      uint16_t entry = 0xFFFF;
      int need_child = 0;
      for (int s = 0; s < 256; s++) {
        int len = lengths[s];
        if (len == 0 || len <= 8 * d) continue;
        if (len <= hi) {
          uint64_t mask = ((uint64_t)1 << len) - 1;
          if ((full & mask) == rev[s]) entry = (uint16_t)((len << 8) | s);
        } else {
          uint64_t mask = ((uint64_t)1 << hi) - 1;
          if ((full & mask) == (rev[s] & mask)) need_child = 1;
        }
      }
      if (entry == 0xFFFF && need_child) {
        if (count >= 4096 || count >= cap) return -1;
        depth_of[count] = d + 1;
        prefix_of[count] = full;
        entry = (uint16_t)(0x8000 | count);
        count++;
      }
      lut[tbl * 256 + j] = entry;
    }
  }
  *n_luts = count;
  return 0;
}

/* ------------------------------------------------------------------------ */
/* Decoding.  The textbook bit-serial canonical decoder: read one bit at a
 * time and compare the running code against the first code of each length.
 * This is the sequential kind of decoding that [DF11, "Descompressao adaptada
 * para inferencia em GPU"] describes as a poor fit for a GPU; here it is the
 * reference.  It does not use the lookup tables.                             */
/* ------------------------------------------------------------------------ */
typedef struct {
  uint64_t first[O_MAX_LEN + 2];
  uint64_t count[O_MAX_LEN + 2];
  uint64_t offset[O_MAX_LEN + 2];
  uint8_t sorted[256];
} canon_t;

static int canon_init(const uint8_t *lengths, canon_t *c) {
  uint32_t codes[256];
  if (oracle_canonical_codes(lengths, codes) != 0) return -1;
  memset(c, 0, sizeof(*c));
  int k = 0;
  for (int len = 1; len <= O_MAX_LEN; len++) {
    c->offset[len] = (uint64_t)k;
    for (int s = 0; s < 256; s++) {
      if (lengths[s] != len) continue;
      if (c->count[len] == 0) c->first[len] = codes[s];
      c->count[len]++;
      c->sorted[k++] = (uint8_t)s;
    }
  }
  return 0;
}

/* Decode one code at bit position *pos.  Returns the symbol or -1. */
static int decode_one(const canon_t *c, const uint8_t *stream, uint64_t *pos,
                      uint64_t limit_bits) {
  uint64_t code = 0;
  for (int len = 1; len <= O_MAX_LEN; len++) {
    if (*pos >= limit_bits) return -1;
    code = (code << 1) | (uint64_t)get_bit(stream, *pos);
    (*pos)++;
    if (c->count[len] && code >= c->first[len] && code - c->first[len] < c->count[len])
      return c->sorted[c->offset[len] + (code - c->first[len])];
  }
  return -1;
}

/* Output element i.  BF16: the weight from exponent and sign|mantissa.
 * uint8 and uint4: the symbol, one byte per element (oracle_pack_u4 packs
 * the uint4 result; writing single bytes keeps the tile-range workers of
 * different threads off each other's bytes). */
static void emit(int kind, void *dst, uint64_t i, uint8_t sym, const uint8_t *sm) {
  if (kind == O_KIND_BF16) {
    uint16_t sign = (uint16_t)(sm[i] >> 7), mant = (uint16_t)(sm[i] & 0x7F);
    ((uint16_t *)dst)[i] = (uint16_t)((sign << 15) | ((uint16_t)sym << 7) | mant);
  } else {
    ((uint8_t *)dst)[i] = sym;
  }
}

/* Sequential decode of n codes from the start of the stream.  stream_bytes
 * bounds every read.  Returns 0, or -1 on a code that cannot be decoded. */
int oracle_decode_serial(int kind, const uint8_t *lengths, const uint8_t *stream,
                         uint64_t stream_bytes, uint64_t n, const uint8_t *sm,
                         void *dst) {
  canon_t c;
  if (canon_init(lengths, &c) != 0) return -1;
  uint64_t pos = 0, limit = stream_bytes * 8;
  for (uint64_t i = 0; i < n; i++) {
    int s = decode_one(&c, stream, &pos, limit);
    if (s < 0) return -1;
    emit(kind, dst, i, (uint8_t)s, sm);
  }
  return 0;
}

/* Parallel decode over contiguous tile ranges, one CPU thread per range,
 * using the container's gaps and tile_out to find where each range starts:
 * [ENTRO, "Metodologia"] decodes independent segments on several CPU
 * threads; the segment boundaries here are the DFloat11 thread-block
 * boundaries.  A range starting at tile b0 starts decoding at bit
 * 16384 b0 + gap[256 b0] and output index tile_out[b0], and stops after
 * tile_out[b1] - tile_out[b0] codes.                                        */
typedef struct {
  int kind;
  const canon_t *c;
  const uint8_t *stream;
  uint64_t stream_bytes;
  const uint8_t *gaps;
  const uint64_t *tile_out;
  uint64_t n_threads;
  const uint8_t *sm;
  void *dst;
  uint64_t b0, b1;
  int status;
} range_job;

static uint64_t read_gap(const uint8_t *gaps, uint64_t t) {
  uint64_t g = 0;
  for (int k = 0; k < O_GAP_BITS; k++)
    g |= (uint64_t)get_bit(gaps, t * O_GAP_BITS + k) << k;
  return g;
}

static void *range_worker(void *arg) {
  range_job *j = (range_job *)arg;
  j->status = 0;
  if (j->b0 >= j->b1) return NULL;
  uint64_t t0 = j->b0 * O_THREADS_PER_TILE;
  if (t0 >= j->n_threads) return NULL;
  uint64_t pos = t0 * O_CHUNK_BITS + read_gap(j->gaps, t0);
  uint64_t limit = j->stream_bytes * 8;
  for (uint64_t i = j->tile_out[j->b0]; i < j->tile_out[j->b1]; i++) {
    int s = decode_one(j->c, j->stream, &pos, limit);
    if (s < 0) {
      j->status = -1;
      return NULL;
    }
    emit(j->kind, j->dst, i, (uint8_t)s, j->sm);
  }
  return NULL;
}

int oracle_decode_tiles(int kind, const uint8_t *lengths, const uint8_t *stream,
                        uint64_t stream_bytes, const uint8_t *gaps,
                        const uint64_t *tile_out, uint64_t n_tiles,
                        uint64_t n_threads, const uint8_t *sm, void *dst,
                        int cpu_threads) {
  canon_t c;
  if (canon_init(lengths, &c) != 0) return -1;
  if (cpu_threads < 1) cpu_threads = 1;
  if ((uint64_t)cpu_threads > n_tiles) cpu_threads = n_tiles ? (int)n_tiles : 1;
  range_job *jobs = (range_job *)calloc((size_t)cpu_threads, sizeof(range_job));
  pthread_t *tids = (pthread_t *)calloc((size_t)cpu_threads, sizeof(pthread_t));
  if (!jobs || !tids) {
    free(jobs); free(tids);
    return -1;
  }
  for (int k = 0; k < cpu_threads; k++) {
    jobs[k].kind = kind;
    jobs[k].c = &c;
    jobs[k].stream = stream;
    jobs[k].stream_bytes = stream_bytes;
    jobs[k].gaps = gaps;
    jobs[k].tile_out = tile_out;
    jobs[k].n_threads = n_threads;
    jobs[k].sm = sm;
    jobs[k].dst = dst;
    jobs[k].b0 = n_tiles * (uint64_t)k / (uint64_t)cpu_threads;
    jobs[k].b1 = n_tiles * (uint64_t)(k + 1) / (uint64_t)cpu_threads;
  }
  int status = 0;
  if (cpu_threads == 1) {
    range_worker(&jobs[0]);
    status = jobs[0].status;
  } else {
    int started = 0;
    for (int k = 0; k < cpu_threads; k++) {
      if (pthread_create(&tids[k], NULL, range_worker, &jobs[k]) != 0) break;
      started++;
    }
    for (int k = 0; k < started; k++) pthread_join(tids[k], NULL);
    if (started != cpu_threads) status = -1;
    for (int k = 0; k < cpu_threads; k++)
      if (jobs[k].status) status = jobs[k].status;
  }
  free(jobs);
  free(tids);
  return status;
}

/* Decode tiles [b0, b1) only, single-threaded, into dst (which receives
 * elements tile_out[b0] .. tile_out[b1] - 1 at those same indices).  The
 * same range walk as oracle_decode_tiles, for sampled checks of very large
 * containers. */
int oracle_decode_tile_range(int kind, const uint8_t *lengths, const uint8_t *stream,
                             uint64_t stream_bytes, const uint8_t *gaps,
                             const uint64_t *tile_out, uint64_t b0, uint64_t b1,
                             uint64_t n_threads, const uint8_t *sm, void *dst) {
  canon_t c;
  if (canon_init(lengths, &c) != 0) return -1;
  range_job j;
  j.kind = kind;
  j.c = &c;
  j.stream = stream;
  j.stream_bytes = stream_bytes;
  j.gaps = gaps;
  j.tile_out = tile_out;
  j.n_threads = n_threads;
  j.sm = sm;
  j.dst = dst;
  j.b0 = b0;
  j.b1 = b1;
  range_worker(&j);
  return j.status;
}
