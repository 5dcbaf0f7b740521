// dfh_host.cpp -- host half of the codec: histogram, codebook, canonical
// codes, parallel encoder, hierarchical tables, multi-code decode table,
// container files and validation.  The C ABI is declared in include/dfh.h.
//
// Sources by page title and section heading:
//   DFloat11 digest ("DFloat11: compressao sem perda para inferencia em GPU
//   que reduz LLMs para 70% do tamanho"): "O formato DFloat11" (exponent
//   Huffman coded, sign|mantissa raw), "Decodificacao com LUT hierarquica"
//   (height-8 subtrees as 256-entry tables), "Kernel de GPU em 2 etapas e
//   metadados auxiliares" (8 bytes per thread, 5-bit gaps, one output
//   position per thread block).
//   EntroLLM summary ("EntroLLM: Entropy Encoded Weight Compression for
//   Efficient Large Language Model Inference on Edge Devices"),
//   "Metodologia": Huffman coding of uint8 quantised weights.

#include "dfh.h"

#include <algorithm>
#include <atomic>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <new>
#include <thread>
#include <vector>

namespace {

constexpr uint32_t kMagic = 0x31484644u;  // "DFH1"
constexpr uint32_t kVersion = 1;
constexpr uint64_t kChunkBits = 8ull * DF_BYTES_PER_THREAD;  // 64
constexpr uint64_t kGapBytesPerTile = DF_THREADS_PER_TILE * 5 / 8;  // 160
constexpr int kDtabSize = 1 << DF_DTAB_BITS;

uint64_t round_up(uint64_t x, uint64_t a) { return (x + a - 1) / a * a; }

unsigned host_threads() {
  unsigned n = std::thread::hardware_concurrency();
  if (n == 0) n = 1;
  const char *names[] = {"DF_HOST_THREADS", "OMP_NUM_THREADS"};
  for (const char *name : names) {
    const char *v = getenv(name);
    if (v && atoi(v) > 0) {
      n = std::min<unsigned>(n, (unsigned)atoi(v));
      break;
    }
  }
  return std::max(1u, std::min(n, 64u));
}

// Run f(worker, begin, end) over [0, n) split into contiguous parts.
template <class F>
void parallel_ranges(uint64_t n, unsigned parts, F f) {
  if (parts <= 1 || n < 2) {
    f(0u, (uint64_t)0, n);
    return;
  }
  std::vector<std::thread> pool;
  pool.reserve(parts);
  for (unsigned k = 0; k < parts; k++) {
    uint64_t b = n * k / parts, e = n * (k + 1) / parts;
    pool.emplace_back([=, &f] { f(k, b, e); });
  }
  for (auto &t : pool) t.join();
}

inline bool valid_kind(int kind) {
  return kind == DF_KIND_BF16 || kind == DF_KIND_U8 || kind == DF_KIND_U4;
}

// The coded symbol of element i: BF16 exponent byte, uint8 byte, or uint4
// nibble (element 2j in the low nibble of byte j).
inline uint8_t sym_at(df_kind kind, const void *src, uint64_t i) {
  if (kind == DF_KIND_BF16) return (uint8_t)((((const uint16_t *)src)[i] >> 7) & 0xFF);
  if (kind == DF_KIND_U4) return (uint8_t)((((const uint8_t *)src)[i >> 1] >> (4 * (i & 1))) & 0xF);
  return ((const uint8_t *)src)[i];
}

// ------------------------------------------------------------- codebook
// Huffman code lengths by the two-queue method: leaves sorted by
// (count, symbol) in one queue, merged nodes in creation order in the other
// (their weights never decrease).  Taking the lighter front, leaves first on
// equal weight, always merges the two smallest (weight, key) nodes where a
// leaf's key is its symbol and a merged node's key is 256 + creation order.
int two_queue_huffman(const uint64_t *hist, int *len) {
  std::vector<int> leaf;
  for (int s = 0; s < 256; s++) {
    len[s] = 0;
    if (hist[s]) leaf.push_back(s);
  }
  const int m = (int)leaf.size();
  if (m == 0) return 0;
  if (m == 1) {
    len[leaf[0]] = 1;
    return 1;
  }
  std::stable_sort(leaf.begin(), leaf.end(), [&](int a, int b) { return hist[a] < hist[b]; });
  std::vector<uint64_t> w(2 * m - 1);
  std::vector<int> up(2 * m - 1, -1);
  for (int i = 0; i < m; i++) w[i] = hist[leaf[i]];
  int lf = 0, nf = m, made = m;
  auto take = [&]() {
    if (lf < m && (nf >= made || w[lf] <= w[nf])) return lf++;
    return nf++;
  };
  for (int k = 0; k < m - 1; k++) {
    int a = take();
    int b = take();
    w[made] = w[a] + w[b];
    up[a] = up[b] = made;
    made++;
  }
  std::vector<int> depth(2 * m - 1, 0);
  for (int v = 2 * m - 3; v >= 0; v--) depth[v] = depth[up[v]] + 1;
  for (int i = 0; i < m; i++) len[leaf[i]] = depth[i];
  return m;
}

// Optimal length-limited lengths by package-merge (Larmore and Hirschberg,
// J. ACM 1990).  Lists are kept per level with packages pointing at the pair
// of items below them; the selection at the top level is a prefix of that
// list, and the packages in a selected prefix expand to a prefix of the level
// below, so lengths are counted walking down prefix lengths.  Order inside a
// list: weight, then leaves before packages, leaves by symbol, packages by
// creation.
int package_merge(const uint64_t *hist, int limit, int *len) {
  std::vector<int> leaf;
  for (int s = 0; s < 256; s++) {
    len[s] = 0;
    if (hist[s]) leaf.push_back(s);
  }
  const int m = (int)leaf.size();
  if (m <= 1) {
    if (m == 1) len[leaf[0]] = 1;
    return m;
  }
  if (limit < 1 || limit > 32 || (1ull << limit) < (uint64_t)m) return -1;
  std::stable_sort(leaf.begin(), leaf.end(), [&](int a, int b) { return hist[a] < hist[b]; });
  struct Item {
    uint64_t w;
    int sym;  // >= 0 for a leaf, -1 for a package
  };
  // level[l] for l = limit (deepest) .. 1
  std::vector<std::vector<Item>> level(limit + 1);
  for (int i = 0; i < m; i++) level[limit].push_back({hist[leaf[i]], leaf[i]});
  for (int l = limit - 1; l >= 1; l--) {
    const std::vector<Item> &below = level[l + 1];
    std::vector<Item> &cur = level[l];
    size_t npk = below.size() / 2, li = 0, pi = 0;
    cur.reserve(m + npk);
    while (li < (size_t)m || pi < npk) {
      uint64_t pw = pi < npk ? below[2 * pi].w + below[2 * pi + 1].w : 0;
      if (li < (size_t)m && (pi >= npk || hist[leaf[li]] <= pw)) {
        cur.push_back({hist[leaf[li]], leaf[li]});
        li++;
      } else {
        cur.push_back({pw, -1});
        pi++;
      }
    }
  }
  size_t take = 2 * (size_t)m - 2;
  for (int l = 1; l <= limit; l++) {
    size_t packages = 0;
    for (size_t i = 0; i < take; i++) {
      if (level[l][i].sym >= 0) len[level[l][i].sym]++;
      else packages++;
    }
    take = 2 * packages;
  }
  return m;
}

// Canonical codes: symbols ordered by (length, symbol); the first gets 0 and
// each next code is (previous + 1) shifted left by the growth in length.
void canonical_codes(const uint8_t *len, uint32_t *code) {
  int order[256], k = 0;
  for (int l = 1; l <= 32; l++)
    for (int s = 0; s < 256; s++)
      if (len[s] == l) order[k++] = s;
  uint64_t c = 0;
  for (int i = 0; i < 256; i++) code[i] = 0;
  for (int i = 0; i < k; i++) {
    if (i > 0) c = (c + 1) << (len[order[i]] - len[order[i - 1]]);
    code[order[i]] = (uint32_t)c;
  }
}

// A code's bits in stream order: its first (most significant) bit at bit 0.
uint32_t stream_bits(uint32_t code, int l) {
  uint32_t r = 0;
  for (int k = 0; k < l; k++) r = (r << 1) | ((code >> k) & 1);
  return r;
}

// Kraft sum times 2^32 (exact), or UINT64_MAX for a length above 32.
uint64_t kraft_scaled(const uint8_t *len) {
  uint64_t k = 0;
  for (int s = 0; s < 256; s++) {
    if (len[s] > 32) return UINT64_MAX;
    if (len[s]) k += 1ull << (32 - len[s]);
  }
  return k;
}

int used_symbols(const uint8_t *len) {
  int m = 0;
  for (int s = 0; s < 256; s++) m += len[s] != 0;
  return m;
}

// Hierarchical tables, built level by level: the tables of depth d + 1 are
// the distinct 8(d+1)-bit stream prefixes of codes longer than 8(d+1) bits,
// numbered after all shallower tables in order of (parent table, entry).
// Leaves of length l in a depth-d table fill every entry whose low l - 8d
// bits match the code's bits [8d, l).  Returns the table count or -1 (also
// for lengths above 32 or beyond Kraft's inequality, as a damaged file may
// hold: the tables are built before the container is validated).
int build_tables(const uint8_t *len, std::vector<uint16_t> &lut) {
  if (kraft_scaled(len) > (1ull << 32)) return -1;
  uint32_t code[256], rev[256];
  canonical_codes(len, code);
  for (int s = 0; s < 256; s++) rev[s] = len[s] ? stream_bits(code[s], len[s]) : 0;
  struct Tab {
    int depth;
    uint32_t prefix;  // 8*depth stream bits
    int parent, entry;
  };
  std::vector<Tab> tabs{{0, 0u, -1, -1}};
  auto find = [&](int depth, uint32_t prefix) {
    for (size_t i = 0; i < tabs.size(); i++)
      if (tabs[i].depth == depth && tabs[i].prefix == prefix) return (int)i;
    return -1;
  };
  for (int d = 0; d < 3; d++) {
    std::vector<std::pair<int, int>> kids;  // (parent table, entry)
    for (int s = 0; s < 256; s++) {
      if (len[s] <= 8 * (d + 1)) continue;
      uint32_t pmask = d ? (uint32_t)((1ull << (8 * d)) - 1) : 0u;
      int parent = find(d, rev[s] & pmask);
      if (parent < 0) return -1;
      kids.push_back({parent, (int)((rev[s] >> (8 * d)) & 255)});
    }
    std::sort(kids.begin(), kids.end());
    kids.erase(std::unique(kids.begin(), kids.end()), kids.end());
    for (auto &kd : kids) {
      uint32_t prefix = tabs[kd.first].prefix | ((uint32_t)kd.second << (8 * d));
      tabs.push_back({d + 1, prefix, kd.first, kd.second});
    }
  }
  if ((int)tabs.size() > DF_MAX_LUTS) return -1;
  lut.assign(tabs.size() * 256, 0xFFFF);
  for (size_t t = 1; t < tabs.size(); t++)
    lut[(size_t)tabs[t].parent * 256 + tabs[t].entry] = (uint16_t)(0x8000 | t);
  for (int s = 0; s < 256; s++) {
    int l = len[s];
    if (!l) continue;
    int d = (l - 1) / 8;
    uint32_t pmask = d ? (uint32_t)((1ull << (8 * d)) - 1) : 0u;
    int t = find(d, rev[s] & pmask);
    if (t < 0) return -1;
    int rest = l - 8 * d;
    for (uint32_t j = rev[s] >> (8 * d); j < 256; j += 1u << rest)
      lut[(size_t)t * 256 + j] = (uint16_t)((l << 8) | s);
  }
  return (int)tabs.size();
}

// One code through the hierarchical tables from the low bits of look:
// (length << 8) | symbol, or 0 when no code ends within 16 bits.
uint32_t lut_code(const std::vector<uint16_t> &lut, uint32_t look) {
  uint16_t e = lut[look & 255];
  if (e != 0xFFFF && (e & 0x8000)) e = lut[(size_t)(e & 0x7FFF) * 256 + ((look >> 8) & 255)];
  return (e == 0xFFFF || (e & 0x8000)) ? 0u : e;
}

// uint8 pair table: entry w holds the whole codes inside the 13-bit window
// w, at most two, then the code length of every symbol.  Layout in
// include/dfh.h (section DTAB).
void build_pair_table(const uint8_t lengths[256], const std::vector<uint16_t> &lut, std::vector<uint8_t> &out) {
  out.assign(DF_DTAB_BYTES_U8, 0);
  for (uint32_t w = 0; w < (1u << DF_DTAB_BITS_U8); w++) {
    uint32_t pos = 0, count = 0, syms = 0;
    while (count < 2 && pos < (uint32_t)DF_DTAB_BITS_U8) {
      const uint32_t e = lut_code(lut, w >> pos);
      if (!e || pos + (e >> 8) > (uint32_t)DF_DTAB_BITS_U8) break;
      syms |= (e & 0xFF) << (8 * count);
      pos += e >> 8;
      count++;
    }
    const uint32_t v = count ? pos | (syms << 8) | (count << 24) : 0u;
    memcpy(&out[4 * (size_t)w], &v, 4);
  }
  memcpy(&out[(size_t)4 << DF_DTAB_BITS_U8], lengths, 256);
}

// Multi-code decode table: entry w lists the whole codes inside the 12-bit
// window w (first stream bit = bit 0), at most five, found by walking the
// hierarchical tables.  Layout in include/dfh.h (section DTAB): symbol bytes
// (BF16, the exponent rotated right by one bit), or for uint4 the symbols'
// nibbles in bits 0..19, as the uint4 kernel stages them.
void build_multi_table(df_kind kind, const std::vector<uint16_t> &lut, std::vector<uint64_t> &dtab) {
  dtab.assign(kDtabSize, 0);
  for (uint32_t w = 0; w < (uint32_t)kDtabSize; w++) {
    uint64_t syms = 0, starts = 0;
    uint32_t pos = 0, count = 0;
    while (count < 5 && pos < (uint32_t)DF_DTAB_BITS) {
      uint32_t look = w >> pos;
      uint16_t e = lut[look & 255];
      if (e != 0xFFFF && (e & 0x8000)) e = lut[(size_t)(e & 0x7FFF) * 256 + ((look >> 8) & 255)];
      if (e == 0xFFFF || (e & 0x8000)) break;
      uint32_t l = e >> 8;
      if (pos + l > (uint32_t)DF_DTAB_BITS) break;
      uint32_t s = e & 0xFF;
      if (kind == DF_KIND_BF16) s = ((s >> 1) | (s << 7)) & 0xFF;
      syms |= (uint64_t)s << (8 * count);
      starts |= 1ull << pos;
      pos += l;
      count++;
    }
    if (kind == DF_KIND_U4) {  // nibbles of codes 0..4 | consumed bits | start flags | count
      uint64_t nib = 0;
      for (uint32_t i = 0; i < count; i++) nib |= ((syms >> (8 * i)) & 0xF) << (4 * i);
      if (count) dtab[w] = nib | ((uint64_t)pos << 32) | ((starts >> 1) << 37) | ((uint64_t)count << 56);
      continue;
    }
    // symbols 0..3 | consumed bits | start flags for bits 1..11 | symbol 4 | count
    if (count)
      dtab[w] = (syms & 0xFFFFFFFFull) | ((uint64_t)pos << 32) | ((starts >> 1) << 37) | ((syms >> 32) << 48) |
                ((uint64_t)count << 56);
  }
}

uint64_t dtab_bytes(df_kind kind) {
  return kind == DF_KIND_U8 ? DF_DTAB_BYTES_U8 : (uint64_t)kDtabSize * 8;
}

// The DTAB section of a kind (bytes).
void build_dtab(df_kind kind, const uint8_t lengths[256], const std::vector<uint16_t> &lut,
                std::vector<uint8_t> &out) {
  if (kind == DF_KIND_U8) {
    build_pair_table(lengths, lut, out);
    return;
  }
  std::vector<uint64_t> t;
  build_multi_table(kind, lut, t);
  out.resize(t.size() * 8);
  memcpy(out.data(), t.data(), out.size());
}

}  // namespace

// ------------------------------------------------------------- container
struct df_container {
  df_info info;
  uint8_t *sec[DF_SEC_COUNT];
  df_container() {
    memset(&info, 0, sizeof(info));
    for (auto &p : sec) p = nullptr;
  }
  ~df_container() {
    for (auto &p : sec) free(p);
  }
  bool alloc(df_section s, uint64_t bytes) {
    info.section_bytes[s] = bytes;
    sec[s] = (uint8_t *)aligned_alloc(64, round_up(std::max<uint64_t>(bytes, 1), 64));
    if (!sec[s]) return false;
    memset(sec[s], 0, round_up(std::max<uint64_t>(bytes, 1), 64));
    return true;
  }
};

namespace {

df_status finish_tables(df_container *c) {
  std::vector<uint16_t> lut;
  int nl = build_tables(c->info.lengths, lut);
  if (nl < 0) return DF_ERR_CODEBOOK;
  c->info.n_luts = (uint32_t)nl;
  if (!c->alloc(DF_SEC_LUT, lut.size() * 2)) return DF_ERR_ALLOC;
  memcpy(c->sec[DF_SEC_LUT], lut.data(), lut.size() * 2);
  std::vector<uint8_t> dtab;
  build_dtab(c->info.kind, c->info.lengths, lut, dtab);
  if (!c->alloc(DF_SEC_DTAB, dtab.size())) return DF_ERR_ALLOC;
  memcpy(c->sec[DF_SEC_DTAB], dtab.data(), dtab.size());
  return DF_OK;
}

void set_layout(df_container *c, uint64_t n, uint64_t total_bits, uint64_t last_start) {
  df_info &in = c->info;
  in.max_len = DF_MAX_LEN;
  in.n = n;
  in.total_bits = total_bits;
  in.n_threads = n ? last_start / kChunkBits + 1 : 0;
  in.n_tiles = (in.n_threads + DF_THREADS_PER_TILE - 1) / DF_THREADS_PER_TILE;
  in.bytes_per_thread = DF_BYTES_PER_THREAD;
  in.threads_per_tile = DF_THREADS_PER_TILE;
}

}  // namespace

extern "C" {

const char *df_status_string(df_status s) {
  switch (s) {
    case DF_OK: return "ok";
    case DF_ERR_ARG: return "invalid argument";
    case DF_ERR_ALLOC: return "host allocation failed";
    case DF_ERR_CODEBOOK: return "codebook cannot code the input within the limits";
    case DF_ERR_FORMAT: return "container format error";
    case DF_ERR_HIP: return "HIP runtime error";
    case DF_ERR_CORRUPT: return "container contents are corrupt";
    case DF_ERR_IO: return "file input/output error";
  }
  return "unknown status";
}

df_status df_histogram(df_kind kind, const void *src, uint64_t n, uint64_t hist[256]) {
  if (!hist || (n && !src) || !valid_kind(kind)) return DF_ERR_ARG;
  unsigned parts = n < (1u << 20) ? 1 : host_threads();
  std::vector<uint64_t> local((size_t)parts * 256, 0);
  parallel_ranges(n, parts, [&](unsigned k, uint64_t b, uint64_t e) {
    uint64_t *h = &local[(size_t)k * 256];
    for (uint64_t i = b; i < e; i++) h[sym_at(kind, src, i)]++;
  });
  for (int s = 0; s < 256; s++) {
    uint64_t t = 0;
    for (unsigned k = 0; k < parts; k++) t += local[(size_t)k * 256 + s];
    hist[s] = t;
  }
  return DF_OK;
}

df_status df_build_codebook(const uint64_t hist[256], uint32_t max_len, uint8_t lengths[256]) {
  if (!hist || !lengths || max_len < 1 || max_len > DF_MAX_LEN) return DF_ERR_ARG;
  int len[256];
  int m = two_queue_huffman(hist, len);
  int longest = 0;
  for (int s = 0; s < 256; s++) longest = std::max(longest, len[s]);
  if (longest > (int)max_len && package_merge(hist, (int)max_len, len) < 0) return DF_ERR_CODEBOOK;
  uint8_t out[256];
  for (int s = 0; s < 256; s++) out[s] = (uint8_t)len[s];
  if (m > 0) {
    std::vector<uint16_t> lut;
    if (build_tables(out, lut) < 0) return DF_ERR_CODEBOOK;  // over the table cap
  }
  memcpy(lengths, out, 256);
  return DF_OK;
}

df_status df_encode(df_kind kind, const void *src, uint64_t n, const uint8_t lengths[256],
                    df_container **out) {
  if (!out || !lengths || (n && !src) || !valid_kind(kind))
    return DF_ERR_ARG;
  *out = nullptr;
  uint64_t kr = kraft_scaled(lengths);
  if (kr == UINT64_MAX || kr > (1ull << 32)) return DF_ERR_CODEBOOK;
  uint32_t code[256], rev[256];
  canonical_codes(lengths, code);
  for (int s = 0; s < 256; s++) rev[s] = lengths[s] ? stream_bits(code[s], lengths[s]) : 0;

  df_container *c = new (std::nothrow) df_container();
  if (!c) return DF_ERR_ALLOC;
  c->info.kind = kind;
  memcpy(c->info.lengths, lengths, 256);

  // pass 1: bits per segment, and every symbol must have a code
  unsigned parts = n < (1u << 16) ? 1 : host_threads();
  std::vector<uint64_t> seg_bits(parts + 1, 0);
  std::atomic<bool> missing{false};
  parallel_ranges(n, parts, [&](unsigned k, uint64_t b, uint64_t e) {
    uint64_t bits = 0;
    bool miss = false;
    for (uint64_t i = b; i < e; i++) {
      uint8_t l = lengths[sym_at(kind, src, i)];
      miss |= l == 0;
      bits += l;
    }
    seg_bits[k + 1] = bits;
    if (miss) missing = true;
  });
  if (missing) {
    delete c;
    return DF_ERR_CODEBOOK;
  }
  for (unsigned k = 0; k < parts; k++) seg_bits[k + 1] += seg_bits[k];
  const uint64_t total_bits = seg_bits[parts];
  const uint64_t last_start = n ? total_bits - lengths[sym_at(kind, src, n - 1)] : 0;
  set_layout(c, n, total_bits, last_start);
  const uint64_t n_tiles = c->info.n_tiles;
  if (!c->alloc(DF_SEC_BITSTREAM, n_tiles * (DF_TILE_BITS / 8) + 16) ||
      !c->alloc(DF_SEC_GAPS, n_tiles * kGapBytesPerTile + 16) ||
      !c->alloc(DF_SEC_TILE_OUT, (n_tiles + 1) * 8) ||
      !c->alloc(DF_SEC_SIGN_MANTISSA, kind == DF_KIND_BF16 ? round_up(n, 64) : 0)) {
    delete c;
    return DF_ERR_ALLOC;
  }
  std::vector<uint8_t> gap(n_tiles * DF_THREADS_PER_TILE, 0);
  uint64_t *words = (uint64_t *)c->sec[DF_SEC_BITSTREAM];
  uint64_t *tile_out = (uint64_t *)c->sec[DF_SEC_TILE_OUT];
  uint8_t *sm = c->sec[DF_SEC_SIGN_MANTISSA];

  // pass 2: each segment writes its codes from its known start bit; the
  // words it shares with its neighbours are OR-ed in atomically
  parallel_ranges(n, parts, [&](unsigned k, uint64_t b, uint64_t e) {
    if (b >= e) return;
    uint64_t pos = seg_bits[k];
    uint64_t prev = b ? pos - lengths[sym_at(kind, src, b - 1)] : 0;
    uint64_t wi = pos >> 6;
    uint32_t fill = (uint32_t)(pos & 63);
    uint64_t acc = 0;
    bool first_word = true;
    auto flush = [&](bool partial) {
      if (first_word || partial) __atomic_fetch_or(&words[wi], acc, __ATOMIC_RELAXED);
      else words[wi] = acc;
      first_word = false;
    };
    for (uint64_t i = b; i < e; i++) {
      uint8_t s = sym_at(kind, src, i);
      uint32_t l = lengths[s];
      if (i == 0) {
        tile_out[0] = 0;
        gap[0] = 0;
      } else {
        if ((prev >> 6) != (pos >> 6)) gap[pos >> 6] = (uint8_t)(pos & 63);
        if ((prev >> 14) != (pos >> 14)) tile_out[pos >> 14] = i;
      }
      acc |= (uint64_t)rev[s] << fill;
      fill += l;
      if (fill >= 64) {
        flush(false);
        wi++;
        fill -= 64;
        acc = fill ? (uint64_t)rev[s] >> (l - fill) : 0;
      }
      prev = pos;
      pos += l;
      if (kind == DF_KIND_BF16) {
        uint16_t u = ((const uint16_t *)src)[i];
        sm[i] = (uint8_t)(((u >> 8) & 0x80) | (u & 0x7F));
      }
    }
    if (fill) flush(true);
  });
  tile_out[n_tiles] = n;

  // pack the gaps, 5 bits each, least significant bit first: 8 gaps = 5 bytes
  uint8_t *gp = c->sec[DF_SEC_GAPS];
  uint64_t groups = n_tiles * DF_THREADS_PER_TILE / 8;
  parallel_ranges(groups, groups < 4096 ? 1 : parts, [&](unsigned, uint64_t b, uint64_t e) {
    for (uint64_t g = b; g < e; g++) {
      uint64_t v = 0;
      for (int j = 0; j < 8; j++) v |= (uint64_t)(gap[g * 8 + j] & 31) << (5 * j);
      for (int j = 0; j < 5; j++) gp[g * 5 + j] = (uint8_t)(v >> (8 * j));
    }
  });
  uint64_t mx = 0;
  for (uint64_t t = 0; t < n_tiles; t++) mx = std::max(mx, tile_out[t + 1] - tile_out[t]);
  c->info.max_tile_elems = (uint32_t)mx;

  df_status st = finish_tables(c);
  if (st != DF_OK) {
    delete c;
    return st;
  }
  *out = c;
  return DF_OK;
}

df_status df_encode_layout(df_kind kind, uint64_t n, const uint64_t hist[256], uint8_t last_symbol,
                           const uint8_t lengths[256], df_info *out) {
  if (!hist || !lengths || !out || !valid_kind(kind)) return DF_ERR_ARG;
  uint64_t kr = kraft_scaled(lengths);
  if (kr == UINT64_MAX || kr > (1ull << 32)) return DF_ERR_CODEBOOK;
  uint64_t total_bits = 0, counted = 0;
  for (int s = 0; s < 256; s++) {
    if (!hist[s]) continue;
    if (!lengths[s]) return DF_ERR_CODEBOOK;
    total_bits += hist[s] * lengths[s];
    counted += hist[s];
  }
  if (counted != n || (n && (!hist[last_symbol] || !lengths[last_symbol]))) return DF_ERR_ARG;
  df_container c;  // header arithmetic only: no section is allocated
  c.info.kind = kind;
  memcpy(c.info.lengths, lengths, 256);
  set_layout(&c, n, total_bits, n ? total_bits - lengths[last_symbol] : 0);
  std::vector<uint16_t> lut;
  const int nl = build_tables(lengths, lut);
  if (nl < 0) return DF_ERR_CODEBOOK;
  df_info &in = c.info;
  in.n_luts = (uint32_t)nl;
  in.max_tile_elems = 0;
  in.section_bytes[DF_SEC_BITSTREAM] = in.n_tiles * (DF_TILE_BITS / 8) + 16;
  in.section_bytes[DF_SEC_GAPS] = in.n_tiles * kGapBytesPerTile + 16;
  in.section_bytes[DF_SEC_TILE_OUT] = (in.n_tiles + 1) * 8;
  in.section_bytes[DF_SEC_SIGN_MANTISSA] = kind == DF_KIND_BF16 ? round_up(n, 64) : 0;
  in.section_bytes[DF_SEC_LUT] = lut.size() * 2;
  in.section_bytes[DF_SEC_DTAB] = dtab_bytes(kind);
  *out = in;
  return DF_OK;
}

df_status df_build_tables(df_kind kind, const uint8_t lengths[256], uint16_t *lut, uint32_t lut_cap,
                          uint32_t *n_luts, uint64_t *dtab) {
  if (!lengths || !lut || !n_luts || !dtab || !valid_kind(kind)) return DF_ERR_ARG;
  std::vector<uint16_t> l;
  const int nl = build_tables(lengths, l);
  if (nl < 0 || (uint32_t)nl > lut_cap) return DF_ERR_CODEBOOK;
  memcpy(lut, l.data(), l.size() * 2);
  *n_luts = (uint32_t)nl;
  std::vector<uint8_t> d;
  build_dtab(kind, lengths, l, d);
  memcpy(dtab, d.data(), d.size());
  return DF_OK;
}

df_status df_container_info(const df_container *c, df_info *out) {
  if (!c || !out) return DF_ERR_ARG;
  *out = c->info;
  return DF_OK;
}

const void *df_container_section(const df_container *c, df_section s, uint64_t *nbytes) {
  if (!c || s < 0 || s >= DF_SEC_COUNT) return nullptr;
  if (nbytes) *nbytes = c->info.section_bytes[s];
  return c->sec[s];
}

void df_container_free(df_container *c) { delete c; }

df_status df_container_validate(const df_container *c) {
  if (!c) return DF_ERR_ARG;
  const df_info &in = c->info;
  if (!valid_kind(in.kind)) return DF_ERR_FORMAT;
  if (in.bytes_per_thread != DF_BYTES_PER_THREAD || in.threads_per_tile != DF_THREADS_PER_TILE ||
      in.max_len != DF_MAX_LEN)
    return DF_ERR_FORMAT;
  uint64_t kr = kraft_scaled(in.lengths);
  if (kr == UINT64_MAX || kr > (1ull << 32)) return DF_ERR_CORRUPT;
  int m = used_symbols(in.lengths);
  if (m >= 2 && kr != (1ull << 32)) return DF_ERR_CORRUPT;
  if (in.n > 0 && m == 0) return DF_ERR_CORRUPT;
  if (in.n == 0 && (in.n_threads || in.n_tiles || in.total_bits)) return DF_ERR_FORMAT;
  if (in.n > 0 && in.n_threads == 0) return DF_ERR_FORMAT;
  if (in.n_tiles != (in.n_threads + DF_THREADS_PER_TILE - 1) / DF_THREADS_PER_TILE) return DF_ERR_FORMAT;
  if (in.n_threads && (in.total_bits <= (in.n_threads - 1) * kChunkBits ||
                       in.total_bits > in.n_threads * kChunkBits + DF_MAX_LEN))
    return DF_ERR_FORMAT;
  if (in.total_bits < in.n || in.total_bits > in.n * DF_MAX_LEN) return DF_ERR_FORMAT;
  const uint64_t want[DF_SEC_COUNT] = {
      in.n_tiles * (DF_TILE_BITS / 8) + 16, in.n_tiles * kGapBytesPerTile + 16, (in.n_tiles + 1) * 8,
      in.kind == DF_KIND_BF16 ? round_up(in.n, 64) : 0, (uint64_t)in.n_luts * 512, dtab_bytes(in.kind)};
  for (int s = 0; s < DF_SEC_COUNT; s++)
    if (in.section_bytes[s] != want[s] || !c->sec[s]) return DF_ERR_FORMAT;
  const uint64_t *to = (const uint64_t *)c->sec[DF_SEC_TILE_OUT];
  if (to[0] != 0 || to[in.n_tiles] != in.n) return DF_ERR_CORRUPT;
  uint64_t mx = 0;
  for (uint64_t b = 0; b < in.n_tiles; b++) {
    if (to[b + 1] < to[b] || to[b + 1] - to[b] > DF_TILE_BITS) return DF_ERR_CORRUPT;
    mx = std::max(mx, to[b + 1] - to[b]);
  }
  if (mx != in.max_tile_elems) return DF_ERR_CORRUPT;
  // gaps past n_threads are zero (gaps below are 5-bit fields, so in range)
  const uint8_t *gp = c->sec[DF_SEC_GAPS];
  for (uint64_t t = in.n_threads; t < in.n_tiles * DF_THREADS_PER_TILE; t++) {
    uint64_t bit = 5 * t, v = 0;
    for (int k = 0; k < 5; k++) v |= (uint64_t)((gp[(bit + k) >> 3] >> ((bit + k) & 7)) & 1) << k;
    if (v) return DF_ERR_CORRUPT;
  }
  std::vector<uint16_t> lut;
  int nl = build_tables(in.lengths, lut);
  if (nl < 0 || (uint32_t)nl != in.n_luts || memcmp(lut.data(), c->sec[DF_SEC_LUT], lut.size() * 2))
    return DF_ERR_CORRUPT;
  std::vector<uint8_t> dtab;
  build_dtab(in.kind, in.lengths, lut, dtab);
  if (memcmp(dtab.data(), c->sec[DF_SEC_DTAB], dtab.size())) return DF_ERR_CORRUPT;
  return DF_OK;
}

// File: 64-byte header block, lengths (256 B), then the five stored
// sections, each starting on a 64-byte boundary.
namespace {
struct FileHeader {
  uint32_t magic, version, kind, max_len;
  uint64_t n, total_bits, n_threads, n_tiles;
  uint32_t n_luts, max_tile_elems, bytes_per_thread, threads_per_tile;
};
static_assert(sizeof(FileHeader) == 64, "header is 64 bytes");
constexpr int kStored = 5;  // every section but DTAB
}  // namespace

df_status df_container_save(const df_container *c, const char *path) {
  if (!c || !path) return DF_ERR_ARG;
  FILE *f = fopen(path, "wb");
  if (!f) return DF_ERR_IO;
  const df_info &in = c->info;
  FileHeader h{kMagic, kVersion, (uint32_t)in.kind, in.max_len, in.n, in.total_bits, in.n_threads,
               in.n_tiles, in.n_luts, in.max_tile_elems, in.bytes_per_thread, in.threads_per_tile};
  bool ok = fwrite(&h, sizeof h, 1, f) == 1 && fwrite(in.lengths, 256, 1, f) == 1;
  static const uint8_t zeros[64] = {0};
  for (int s = 0; ok && s < kStored; s++) {
    uint64_t b = in.section_bytes[s];
    ok = fwrite(&b, 8, 1, f) == 1 && fwrite(zeros, 56, 1, f) == 1;
    if (ok && b) ok = fwrite(c->sec[s], 1, b, f) == b;
    uint64_t pad = round_up(b, 64) - b;
    if (ok && pad) ok = fwrite(zeros, 1, pad, f) == pad;
  }
  ok = (fclose(f) == 0) && ok;
  return ok ? DF_OK : DF_ERR_IO;
}

df_status df_container_load(const char *path, df_container **out) {
  if (!path || !out) return DF_ERR_ARG;
  *out = nullptr;
  FILE *f = fopen(path, "rb");
  if (!f) return DF_ERR_IO;
  // the file's size bounds every section size it may claim (a damaged size
  // field must not turn into a huge allocation)
  uint64_t file_bytes = 0;
  if (fseek(f, 0, SEEK_END) == 0) {
    const long e = ftell(f);
    file_bytes = e > 0 ? (uint64_t)e : 0;
  }
  if (fseek(f, 0, SEEK_SET) != 0) {
    fclose(f);
    return DF_ERR_IO;
  }
  FileHeader h;
  df_container *c = new (std::nothrow) df_container();
  df_status st = DF_OK;
  if (!c) st = DF_ERR_ALLOC;
  else if (fread(&h, sizeof h, 1, f) != 1 || fread(c->info.lengths, 256, 1, f) != 1) st = DF_ERR_FORMAT;
  else if (h.magic != kMagic || h.version != kVersion || h.kind > 2 || h.n_luts > DF_MAX_LUTS)
    st = DF_ERR_FORMAT;
  if (st == DF_OK) {
    df_info &in = c->info;
    in.kind = (df_kind)h.kind;
    in.max_len = h.max_len;
    in.n = h.n;
    in.total_bits = h.total_bits;
    in.n_threads = h.n_threads;
    in.n_tiles = h.n_tiles;
    in.n_luts = h.n_luts;
    in.max_tile_elems = h.max_tile_elems;
    in.bytes_per_thread = h.bytes_per_thread;
    in.threads_per_tile = h.threads_per_tile;
    for (int s = 0; st == DF_OK && s < kStored; s++) {
      uint64_t b;
      uint8_t skip[56];
      const long at = ftell(f);
      if (fread(&b, 8, 1, f) != 1 || fread(skip, 56, 1, f) != 1 || at < 0 || b > file_bytes - (uint64_t)at) {
        st = DF_ERR_FORMAT;
        break;
      }
      if (!c->alloc((df_section)s, b)) {
        st = DF_ERR_ALLOC;
        break;
      }
      if (b && fread(c->sec[s], 1, b, f) != b) st = DF_ERR_FORMAT;
      uint64_t pad = round_up(b, 64) - b;
      uint8_t z[64];
      if (st == DF_OK && pad && fread(z, 1, pad, f) != pad) st = DF_ERR_FORMAT;
    }
  }
  fclose(f);
  if (st == DF_OK) {
    std::vector<uint16_t> lut;
    if (build_tables(c->info.lengths, lut) < 0) st = DF_ERR_CORRUPT;
    else {
      std::vector<uint8_t> dtab;
      build_dtab(c->info.kind, c->info.lengths, lut, dtab);
      if (!c->alloc(DF_SEC_DTAB, dtab.size())) st = DF_ERR_ALLOC;
      else memcpy(c->sec[DF_SEC_DTAB], dtab.data(), dtab.size());
    }
  }
  if (st == DF_OK) st = df_container_validate(c);
  if (st != DF_OK) {
    delete c;
    return st;
  }
  *out = c;
  return DF_OK;
}

}  // extern "C"
